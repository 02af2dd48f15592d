"""GPU parity of the one-pass weight quantizer (both orientations of expert
weights, scales in the GEMM layout) and of the forward / dgrad entry points
that take those prequantized weights.

The quantizer is compared bit for bit with the CPU oracle's rowwise (1x32
along K) and colwise (32x1 along N) quantization of the same weights; the
oracle's row-major scales are permuted into the GEMM layout here, in the test.
The prequantized GEMM entry points must return exactly what the bf16 entry
points return (same codes feed the same GEMM) and stay within the GEMM
criterion of the oracle."""

import numpy as np
import pytest

import oracle
from oracle.compare import r1_check
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, u8_host, bf16_host_bits, log

pytestmark = pytest.mark.gpu


def _gemm_layout(s_rowmajor: np.ndarray) -> np.ndarray:
    """[B, R, KB] -> [B, KB/4, R, 4] (the GEMM scale layout)."""
    B, R, KB = s_rowmajor.shape
    return np.ascontiguousarray(s_rowmajor.reshape(B, R, KB // 4, 4).transpose(0, 2, 1, 3))


def _check_weights(W_bits: np.ndarray, tag: str):
    import mxfp8_block_scaled_06_amd as mx
    q, s, qt, st = mx.mx_quantize_weights(to_dev_bf16(W_bits))
    q, s, qt, st = u8_host(q), u8_host(s), u8_host(qt), u8_host(st)
    rq, rs = oracle.quantize_rowwise(W_bits)            # [E, N, K], [E, N, K/32]
    cq, cs = oracle.quantize_colwise(W_bits)            # [E, K, N], [E, K, N/32]
    for name, got, ref in (("q", q, rq), ("s", s, _gemm_layout(rs)), ("q_t", qt, cq), ("s_t", st, _gemm_layout(cs))):
        assert got.shape == ref.shape, (tag, name, got.shape, ref.shape)
        bad = np.flatnonzero(got.ravel() != ref.ravel())
        assert bad.size == 0, f"{tag} {name}: {bad.size} mismatches, first {bad[:5]}"


@pytest.mark.parametrize("shape,seed,std", [
    ((2, 128, 128), 31, 0.02),      # one tile per expert
    ((3, 256, 384), 32, 0.02),      # several tiles, rectangular
    ((1, 384, 256), 33, 300.0),     # saturation path
    ((2, 512, 512), 34, 0.02),      # 256 x 256 tiles, two per expert and orientation
])
def test_quantize_weights_matches_oracle(shape, seed, std):
    require_gpu()
    W = inp.random_bf16(shape, seed=seed, std=std, outliers=True)
    log(f"quantize_weights {shape} seed={seed}")
    _check_weights(W, f"{shape}")


def test_quantize_weights_all_bf16_patterns():
    """Every bf16 bit pattern (NaN, Inf, zeros, subnormals) in one [1, 256, 256]
    weight, in pattern order and shuffled."""
    require_gpu()
    pats = inp.all_bf16_patterns()
    rng = np.random.default_rng(34)
    for tag, arr in (("ordered", pats), ("shuffled", rng.permutation(pats))):
        log(f"quantize_weights all bf16 patterns {tag}")
        _check_weights(arr.reshape(1, 256, 256), tag)


def test_quantize_weights_rejects_bad_shapes():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    with pytest.raises(mx.MXError, match="multiples of 128"):
        mx.mx_quantize_weights(torch.zeros((1, 128, 96), dtype=torch.bfloat16, device="cuda:0"))


@pytest.mark.slow
def test_quantize_weights_full_size_matches_both_quantizers():
    """Llama4-shaped stacked weights [16, 8192, 5120]: the one-pass outputs equal
    the rowwise and colwise quantizers' outputs (themselves oracle-checked),
    and sampled rows / columns equal the oracle directly."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(inp.WORKLOADS["llama4_fwd"].seed)
    W = inp.make_weights(rng, 16, 8192, 5120)
    log(f"quantize_weights full size {W.shape}")
    Wd = to_dev_bf16(W)
    q, s, qt, st = mx.mx_quantize_weights(Wd)
    rq, rs = mx.mx_quantize_rowwise(Wd)
    assert torch.equal(q, rq)
    assert torch.equal(s, mx.mx_scales_to_gemm_layout(rs))
    del rq, rs
    cq, cs = mx.mx_quantize_colwise(Wd)
    assert torch.equal(qt, cq)
    assert torch.equal(st, mx.mx_scales_to_gemm_layout(cs))
    del cq, cs
    srng = np.random.default_rng(35)
    qh, sh = u8_host(q), u8_host(s)
    for _ in range(8):
        e, r = int(srng.integers(16)), srng.integers(8192, size=4)
        oq, os_ = oracle.quantize_rowwise(W[e, r])
        assert np.array_equal(qh[e, r], oq)
        assert np.array_equal(sh[e, :, r, :].reshape(4, -1), os_)
    del qh, sh
    qth, sth = u8_host(qt), u8_host(st)
    for _ in range(8):
        e, c = int(srng.integers(16)), srng.integers(5120, size=2)
        oq, os_ = oracle.quantize_colwise(np.ascontiguousarray(W[e][:, c]))
        assert np.array_equal(qth[e, c], oq)
        assert np.array_equal(sth[e, :, c, :].reshape(2, -1), os_)


CASES = {
    "ragged": ([1, 31, 32, 33, 255, 256, 257, 100], 384, 512),
    "empty_first_last": ([0, 300, 0, 200, 0], 256, 384),
    "single_expert": ([777], 512, 256),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_prequantized_entry_points_equal_bf16_ones(case):
    """fwd_q / dgrad_q on mx_quantize_weights' output are bit-identical to the
    bf16 entry points and within the GEMM criterion of the oracle."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    counts, N, K = CASES[case]
    E, M = len(counts), sum(counts)
    offs = inp.offsets_from_counts(counts)
    A = inp.random_bf16((M, K), seed=700 + E, outliers=True)
    G = inp.random_bf16((M, N), seed=800 + E, std=1e-3)
    W = inp.random_bf16((E, N, K), seed=900 + E, std=0.02)
    log(f"prequantized fwd/dgrad case={case} counts={counts} N={N} K={K}")
    Ad, Gd, Wd, od = to_dev_bf16(A), to_dev_bf16(G), to_dev_bf16(W), to_dev_i32(offs)
    qW, sW, qWt, sWt = mx.mx_quantize_weights(Wd)
    out_q = mx.mx_grouped_mm_fwd_q(Ad, qW, sW, od)
    out = mx.mx_grouped_mm_fwd(Ad, Wd, od)
    assert torch.equal(out_q.view(torch.int16), out.view(torch.int16))
    r = r1_check(bf16_host_bits(out_q), oracle.grouped_mm_fwd(A, W, offs),
                 abs_terms=oracle.grouped_mm_fwd(A, W, offs, absolute=True))
    assert r["ok"], r
    dA_q = mx.mx_grouped_mm_dgrad_q(Gd, qWt, sWt, od)
    dA = mx.mx_grouped_mm_dgrad(Gd, Wd, od)
    assert torch.equal(dA_q.view(torch.int16), dA.view(torch.int16))
    r = r1_check(bf16_host_bits(dA_q), oracle.grouped_mm_dgrad(G, W, offs),
                 abs_terms=oracle.grouped_mm_dgrad(G, W, offs, absolute=True))
    assert r["ok"], r
