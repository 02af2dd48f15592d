"""mx_grouped_mm_fwd_q_noalloc, the allocation-free forward on prequantized
weights, against mx_grouped_mm_fwd_q with a workspace: bit-identical on two
calls in a row, the second with a smaller input (the static scratch keeps the
first call's contents), and a clear error past the scratch size."""

import numpy as np
import pytest

from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, log

pytestmark = pytest.mark.gpu


def _case(counts, N, K, seed):
    A = inp.random_bf16((sum(counts), K), seed=seed, outliers=True)
    W = inp.random_bf16((len(counts), N, K), seed=seed + 1, std=0.02)
    return A, W, inp.offsets_from_counts(counts)


def test_noalloc_forward_matches_workspace_entry_point_twice():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    for counts, N, K, seed in (([700, 0, 1300, 96], 1024, 2048, 71), ([40, 260, 0], 256, 512, 72)):
        A, W, offs = _case(counts, N, K, seed)
        Ad, od = to_dev_bf16(A), to_dev_i32(offs)
        qW, sW, _, _ = mx.mx_quantize_weights(to_dev_bf16(W))
        want = mx.mx_grouped_mm_fwd_q(Ad, qW, sW, od)
        out = torch.full((sum(counts), N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        got = mx.mx_grouped_mm_fwd_q_noalloc(Ad, qW, sW, od, out)
        torch.cuda.synchronize()
        log(f"noalloc counts={counts} N={N} K={K}")
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_noalloc_rejects_inputs_past_the_scratch():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    K, N = 1024, 128
    M = mx.NOALLOC_SCRATCH_BYTES // K + 128           # codes alone overflow the scratch
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
    qW, sW, _, _ = mx.mx_quantize_weights(torch.zeros((1, N, K), dtype=torch.bfloat16, device="cuda:0"))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mx.MXError, match="static scratch"):
        mx.mx_grouped_mm_fwd_q_noalloc(A, qW, sW, to_dev_i32(np.array([M], dtype=np.int32)), out)
