"""GPU parity of the one-pass activation quantizer (mx_quantize_dual: the
forward's A or the backward's dOut in both orientations from one read) and of
the training step composed from it.

The quantizer is compared bit for bit with the CPU oracle's rowwise (1x32
along the columns) and colwise (32x1 along the rows) quantization; the
oracle's row-major scales are permuted into the GEMM layout here, in the test,
and the padding columns of the transposed output (rows .. ldq-1) must be zero
codes with zero scale bytes.  The GEMMs fed by its outputs must return exactly
what the bf16 entry points return for forward, dgrad and wgrad."""

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, u8_host, bf16_host_bits, log

pytestmark = pytest.mark.gpu


def _gemm_layout(s_rowmajor: np.ndarray) -> np.ndarray:
    """[R, KB] -> [KB/4, R, 4] (the GEMM scale layout)."""
    R, KB = s_rowmajor.shape
    return np.ascontiguousarray(s_rowmajor.reshape(R, KB // 4, 4).transpose(1, 0, 2))


def _check_dual(x_bits: np.ndarray, ldq, tag: str):
    import mxfp8_block_scaled_06_amd as mx
    rows, cols = x_bits.shape
    q, s, qt, st = mx.mx_quantize_dual(to_dev_bf16(x_bits), ldq=ldq)
    q, s, qt, st = u8_host(q), u8_host(s), u8_host(qt), u8_host(st)
    ldq = qt.shape[1]
    assert ldq % 128 == 0 and ldq >= rows
    rq, rs = oracle.quantize_rowwise(x_bits)               # [rows, cols], [rows, cols/32]
    cq, cs = oracle.quantize_colwise(x_bits)               # [cols, rows], [cols, rows/32]
    # the transposed orientation over ldq columns: the rows past `rows` are zero rows
    cq_pad = np.zeros((cols, ldq), dtype=np.uint8)
    cq_pad[:, :rows] = cq
    cs_pad = np.zeros((cols, ldq // 32), dtype=np.uint8)
    cs_pad[:, :rows // 32] = cs
    for name, got, ref in (("q", q, rq), ("s", s, _gemm_layout(rs)), ("q_t", qt, cq_pad),
                           ("s_t", st, _gemm_layout(cs_pad))):
        assert got.shape == ref.shape, (tag, name, got.shape, ref.shape)
        bad = np.flatnonzero(got.ravel() != ref.ravel())
        assert bad.size == 0, f"{tag} {name}: {bad.size} mismatches, first {bad[:5]}"


@pytest.mark.parametrize("shape,ldq,seed,std", [
    ((128, 128), None, 41, 1.0),     # one tile
    ((96, 256), None, 42, 1.0),      # rows < 128: a padded tile, ldq 128
    ((416, 384), None, 43, 1.0),     # several tiles, ragged last row tile
    ((256, 128), 512, 44, 1.0),      # explicit wider ldq: two all-padding row tiles
    ((160, 128), None, 45, 300.0),   # saturation path
    ((288, 512), None, 47, 1.0),     # 256 x 256 tiles: a partial row tile, ldq 384 ends inside a tile
    ((256, 768), 512, 48, 1.0),      # 256 x 256 tiles: the second row tile is all padding
    ((160, 256), None, 49, 300.0),   # 256 x 256 tiles, saturation path
])
def test_quantize_dual_matches_oracle(shape, ldq, seed, std):
    require_gpu()
    x = inp.random_bf16(shape, seed=seed, std=std, outliers=True)
    log(f"quantize_dual {shape} ldq={ldq} seed={seed}")
    _check_dual(x, ldq, f"{shape}/{ldq}")


def test_quantize_dual_all_bf16_patterns():
    """Every bf16 bit pattern (NaN, Inf, zeros, subnormals) in one [512, 128]
    and one [256, 256] input (the two tile kernels) with a padded transposed
    output, in pattern order and shuffled."""
    require_gpu()
    pats = inp.all_bf16_patterns()
    rng = np.random.default_rng(46)
    for tag, arr in (("ordered", pats), ("shuffled", rng.permutation(pats))):
        log(f"quantize_dual all bf16 patterns {tag}")
        _check_dual(arr.reshape(512, 128), 640, tag)
        _check_dual(arr.reshape(256, 256), 384, tag + " 256-column tiles")


def test_quantize_dual_rejects_bad_shapes():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    with pytest.raises(mx.MXError, match="multiple of 32"):
        mx.mx_quantize_dual(torch.zeros((48, 128), dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises(mx.MXError, match=">= rows"):
        mx.mx_quantize_dual(torch.zeros((256, 128), dtype=torch.bfloat16, device="cuda:0"), ldq=128)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama4_bwd", "deepseek_share_pad32"])
def test_step_from_dual_quantized_activations_is_bit_identical(name):
    """The step composed from one-pass quantizations (weights both ways, A both
    ways in the forward, dOut both ways in the backward) gives bit for bit the
    outputs of the bf16 entry points, at full size, and the dual outputs over
    the valid rows equal the rowwise / colwise quantizers' own outputs."""
    import dataclasses
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    if name.endswith("_pad32"):
        w = dataclasses.replace(inp.WORKLOADS[name[:-6]], pad32=True)
    else:
        w = inp.WORKLOADS[name]
    x = inp.make_inputs(w, with_grad=True)
    M = x.A.shape[0]
    log(f"dual-quantized step {name} M={M}")
    A, W, dO, offs = to_dev_bf16(x.A), to_dev_bf16(x.W), to_dev_bf16(x.dOut), to_dev_i32(x.offs)
    qW, sW, qWt, sWt = mx.mx_quantize_weights(W)
    qA, sA, qAt, sAt = mx.mx_quantize_dual(A)
    qG, sG, qGt, sGt = mx.mx_quantize_dual(dO)
    # the dual outputs are the single-orientation quantizers' outputs
    rq, rs = mx.mx_quantize_rowwise(A)
    assert torch.equal(qA, rq) and torch.equal(sA, mx.mx_scales_to_gemm_layout(rs))
    cq, cs = mx.mx_quantize_colwise(dO)
    assert torch.equal(qGt[:, :M], cq)
    assert torch.equal(sGt.permute(1, 0, 2).reshape(qGt.shape[0], -1)[:, :M // 32], cs)
    assert not qGt[:, M:].any() and not sGt.permute(1, 0, 2).reshape(qGt.shape[0], -1)[:, M // 32:].any()
    # the three GEMMs on these operands equal the bf16 entry points
    out = mx.mx_grouped_gemm_mx(qA, sA, qW, sW, offs, 0)
    assert torch.equal(out, mx.mx_grouped_mm_fwd(A, W, offs)), "fwd"
    dA = mx.mx_grouped_gemm_mx(qG, sG, qWt, sWt, offs, 0)
    assert torch.equal(dA, mx.mx_grouped_mm_dgrad(dO, W, offs)), "dgrad"
    dW = mx.mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, offs, 1)
    assert torch.equal(dW, mx.mx_grouped_mm_wgrad(dO, A, offs)), "wgrad"
