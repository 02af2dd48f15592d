"""GPU parity of the rowwise quantizer with the token gather fused in: bit-exact
against the oracle's rowwise quantization of the gathered (and zero-padded)
rows, and the GEMM it feeds equals the forward on the gathered bf16 rows."""

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, u8_host, log

pytestmark = pytest.mark.gpu


def _dispatch(T, counts, rng):
    """Top-1 routing of T tokens into groups padded to 32: the gather index
    (-1 for pad rows), the grouped bf16 rows it selects, the padded counts."""
    perm = rng.permutation(T)
    rows, st = [], 0
    padded = []
    for c in counts:
        rows.extend(perm[st:st + c].tolist())
        pad = (-c) % 32
        rows.extend([-1] * pad)
        padded.append(c + pad)
        st += c
    return np.array(rows, dtype=np.int32), padded


def _gathered(x, rows):
    out = np.zeros((rows.shape[0], x.shape[1]), dtype=np.uint16)
    ok = (rows >= 0) & (rows < x.shape[0])
    out[ok] = x[rows[ok]]
    return out


def _gemm_layout(s):
    R, KB = s.shape
    return np.ascontiguousarray(s.reshape(R, KB // 4, 4).transpose(1, 0, 2))


@pytest.mark.parametrize("T,counts,K,seed", [
    (300, [50, 0, 130, 120], 256, 41),
    (1000, [1000], 384, 42),
    (77, [3, 30, 44], 128, 43),
])
def test_gather_quantize_matches_oracle(T, counts, K, seed):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(seed)
    x = inp.random_bf16((T, K), seed=seed, outliers=True)
    rows, _ = _dispatch(T, counts, rng)
    rows[::17] = np.where(rows[::17] >= 0, T + 5, rows[::17])   # out-of-range indices give zero rows too
    log(f"gather-quantize T={T} counts={counts} K={K} M={rows.shape[0]}")
    q, s = mx.mx_quantize_rowwise_gather(to_dev_bf16(x), to_dev_i32(rows))
    rq, rs = oracle.quantize_rowwise(_gathered(x, rows))
    assert np.array_equal(u8_host(q), rq)
    assert np.array_equal(u8_host(s), _gemm_layout(rs))


def test_gather_quantize_feeds_the_grouped_gemm():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(44)
    T, counts, K, N = 400, [120, 0, 200, 80], 256, 384
    x = inp.random_bf16((T, K), seed=45, outliers=True)
    W = inp.random_bf16((len(counts), N, K), seed=46, std=0.02)
    rows, padded = _dispatch(T, counts, rng)
    offs = to_dev_i32(inp.offsets_from_counts(padded))
    log(f"gather-quantize -> grouped GEMM counts={counts} padded={padded}")
    Wd = to_dev_bf16(W)
    qX, sX = mx.mx_quantize_rowwise_gather(to_dev_bf16(x), to_dev_i32(rows))
    qW, sW, _, _ = mx.mx_quantize_weights(Wd)
    out = mx.mx_grouped_gemm_mx(qX, sX, qW, sW, offs, 0)
    ref = mx.mx_grouped_mm_fwd(to_dev_bf16(_gathered(x, rows)), Wd, offs)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
