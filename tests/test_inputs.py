"""The seeded workload generators produce the shapes and routing structure
the workloads promise (host logic, no GPU)."""

import numpy as np

from mxfp8_block_scaled_06_amd import inputs as inp


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 1e3
    x[:10] = [0.0, -0.0, np.inf, -np.inf, 1.0, 3.0000002, 1e-40, -1e-40, 65504.0, 3e38]
    ours = inp.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_routing_counts():
    rng = np.random.default_rng(1)
    c = inp.uniform_counts(rng, 16384, 16)
    assert c.sum() == 16384 and len(c) == 16
    z = inp.zipf_counts(np.random.default_rng(5), 32768, 32)
    assert z.sum() == 32768 and (z == 0).sum() >= 2
    assert z.max() > 5000 and np.sort(z)[2] > 0


def test_offsets_and_padding():
    counts = [5, 0, 33, 64]
    offs = inp.offsets_from_counts(counts)
    assert offs.dtype == np.int32 and offs.tolist() == [5, 5, 38, 102]
    assert inp.pad_counts(counts).tolist() == [32, 0, 64, 64]


def test_tiny_workload_shapes():
    x = inp.make_inputs("tiny")
    assert x.A.shape == (256, 256) and x.W.shape == (2, 512, 256)
    assert x.offs.tolist() == [96, 256]


def test_padded_workload_zero_rows():
    w = inp.WORKLOADS["llama4_bwd"]
    small = inp.Workload("small_bwd", 3, E=4, M=200, K=64, N=32, routing="uniform", outliers=True, pad32=True)
    x = inp.make_inputs(small, with_grad=True)
    assert (x.offs % 32 == 0).all() and x.M_rows == int(x.offs[-1])
    starts = np.concatenate([[0], x.offs[:-1]])
    for e in range(4):
        pad = slice(int(starts[e] + x.counts[e]), int(x.offs[e]))
        assert (x.A[pad] == 0).all() and (x.dOut[pad] == 0).all()
    assert w.pad32
