"""GPU parity of the block-scaled grouped GEMM (forward, dgrad, wgrad and the
GEMM on prequantized operands) against the fp64 oracle, through the C ABI.

Tolerance (oracle/compare.py), all three required:
  (a) every element: |g - r| <= 0.5 ulp_bf16 + 2e-3 * max(|r|, sigma/16)
      + 2^-11 * sum_k |x_k y_k| (the 2e-3 relative bound on top of the final
      bf16 rounding, floored at sigma/16, plus the dot-product error bound of
      the MFMA's internal summation);
  (b) at most 0.2% of the elements need that last term;
  (c) normwise relative error ||g - r|| / ||r|| <= 2e-3.
The bf16 output must also equal the round-to-nearest-even of the fp32 output
bit for bit."""

import dataclasses

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_u8, to_dev_i32, bf16_host_bits, log

pytestmark = pytest.mark.gpu


def _r1(g_bits, ref, tag, abs_terms, sigma=None, f32=False):
    rep = oracle.r1_check(g_bits, ref, sigma=sigma, abs_terms=abs_terms, f32=f32)
    log(f"{tag}: n={rep['n']} bad={rep['n_bad']} max_err/tol={rep['max_err_over_tol']:.3f} "
        f"normwise={rep['normwise_rel']:.2e} exact_rne={rep['exact_rne_rate']:.3f} "
        f"plain_r1_viol={rep['plain_r1_violations']} ({100 * rep['plain_r1_frac']:.3f}%) "
        f"err/abs_terms={rep['max_err_over_abs_terms']:.2e}")
    assert rep["ok"], f"{tag}: {rep}"
    return rep


def _fwd(A, W, offs):
    import mxfp8_block_scaled_06_amd as mx
    return bf16_host_bits(mx.mx_grouped_mm_fwd(to_dev_bf16(A), to_dev_bf16(W), to_dev_i32(offs)))


def _dgrad(G, W, offs):
    import mxfp8_block_scaled_06_amd as mx
    return bf16_host_bits(mx.mx_grouped_mm_dgrad(to_dev_bf16(G), to_dev_bf16(W), to_dev_i32(offs)))


def _wgrad(G, A, offs):
    import mxfp8_block_scaled_06_amd as mx
    return bf16_host_bits(mx.mx_grouped_mm_wgrad(to_dev_bf16(G), to_dev_bf16(A), to_dev_i32(offs)))


def test_fwd_tiny_workload():
    require_gpu()
    x = inp.make_inputs("tiny")
    log(f"fwd tiny counts={x.counts.tolist()}")
    _r1(_fwd(x.A, x.W, x.offs), oracle.grouped_mm_fwd(x.A, x.W, x.offs), "fwd tiny",
        oracle.grouped_mm_fwd(x.A, x.W, x.offs, absolute=True))


ROW_CASES = {
    "ragged": [1, 31, 32, 33, 255, 256, 257, 100],
    "empty_first_last": [0, 300, 0, 200, 0],
    "consecutive_empty": [70, 0, 0, 0, 190],
    "all_in_one": [0, 0, 513, 0],
    "single_expert": [777],
    "zipf_like": [600, 150, 40, 9, 3, 1, 0, 0],
}


@pytest.mark.parametrize("case", sorted(ROW_CASES))
def test_fwd_group_edge_cases(case):
    require_gpu()
    counts = ROW_CASES[case]
    offs = inp.offsets_from_counts(counts)
    M, K, N, E = sum(counts), 384, 520, len(counts)
    A = inp.random_bf16((M, K), seed=100 + len(case), outliers=True)
    W = inp.random_bf16((E, N, K), seed=200 + len(case), std=0.02)
    log(f"fwd case={case} counts={counts} K={K} N={N}")
    _r1(_fwd(A, W, offs), oracle.grouped_mm_fwd(A, W, offs), f"fwd {case}",
        oracle.grouped_mm_fwd(A, W, offs, absolute=True))


@pytest.mark.parametrize("case", ["ragged", "empty_first_last", "single_expert"])
def test_dgrad_group_edge_cases(case):
    require_gpu()
    counts = ROW_CASES[case]
    offs = inp.offsets_from_counts(counts)
    M, K, N, E = sum(counts), 264, 384, len(counts)
    G = inp.random_bf16((M, N), seed=300 + len(case), std=1e-3)
    W = inp.random_bf16((E, N, K), seed=400 + len(case), std=0.02)
    log(f"dgrad case={case} counts={counts} N={N} K={K}")
    _r1(_dgrad(G, W, offs), oracle.grouped_mm_dgrad(G, W, offs), f"dgrad {case}",
        oracle.grouped_mm_dgrad(G, W, offs, absolute=True))


WG_CASES = {
    "padded_mixed": [64, 0, 96, 32, 0, 160],
    "unaligned_starts": [32, 96, 224, 32],      # group starts not multiples of 128
    "all_empty_but_one": [0, 0, 288, 0],
    "single": [416],
}


@pytest.mark.parametrize("case", sorted(WG_CASES))
def test_wgrad_group_edge_cases(case):
    require_gpu()
    counts = WG_CASES[case]
    offs = inp.offsets_from_counts(counts)
    M, K, N, E = sum(counts), 264, 200, len(counts)
    A = inp.random_bf16((M, K), seed=500 + len(case), outliers=True)
    G = inp.random_bf16((M, N), seed=600 + len(case), std=1e-3)
    log(f"wgrad case={case} counts={counts} N={N} K={K}")
    got = _wgrad(G, A, offs)
    ref = oracle.grouped_mm_wgrad(G, A, offs)
    for e, c in enumerate(counts):
        if c == 0:
            assert (got[e] == 0).all(), f"empty expert {e} must get exact zeros"
    _r1(got, ref, f"wgrad {case}", oracle.grouped_mm_wgrad(G, A, offs, absolute=True))


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, c ^ 1, c)      # no NaN codes
    return c.astype(np.uint8)


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_mx_random_operands(mode):
    """The GEMM alone, on seeded random E4M3 codes and E8M0 scales."""
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(700 + mode)
    if mode == 0:
        counts = [130, 0, 257, 61]
        I, J, Kc, E = sum(counts), 296, 384, len(counts)
        X, Y = _random_codes(rng, (I, Kc)), _random_codes(rng, (E, J, Kc))
        sX = rng.integers(112, 142, size=(I, Kc // 32)).astype(np.uint8)
        sY = rng.integers(112, 142, size=(E, J, Kc // 32)).astype(np.uint8)
    else:
        counts = [96, 32, 0, 160, 64]
        I, J, E = 264, 200, len(counts)
        Kc = 384                      # >= sum(counts), multiple of 128
        X, Y = _random_codes(rng, (I, Kc)), _random_codes(rng, (J, Kc))
        sX = rng.integers(112, 142, size=(I, Kc // 32)).astype(np.uint8)
        sY = rng.integers(112, 142, size=(J, Kc // 32)).astype(np.uint8)
    offs = inp.offsets_from_counts(counts)
    log(f"gemm_mx mode={mode} counts={counts}")
    gX = mx.mx_scales_to_gemm_layout(to_dev_u8(sX))
    gY = mx.mx_scales_to_gemm_layout(to_dev_u8(sY))
    args = (to_dev_u8(X), gX, to_dev_u8(Y), gY, to_dev_i32(offs), mode)
    C = bf16_host_bits(mx.mx_grouped_gemm_mx(*args))
    C32 = mx.mx_grouped_gemm_mx_f32(*args).cpu().numpy()
    ref = oracle.grouped_gemm_mx(X, sX, Y, sY, offs, mode)
    absd = oracle.grouped_gemm_mx(X, sX, Y, sY, offs, mode, absolute=True)
    _r1(C, ref, f"gemm_mx mode {mode}", absd)
    _r1(C32, ref, f"gemm_mx_f32 mode {mode}", absd, f32=True)
    # the bf16 epilogue is exactly round-to-nearest-even of the fp32 accumulators
    np.testing.assert_array_equal(C, inp.f32_to_bf16_bits(C32.astype(np.float32)))


@pytest.mark.parametrize("shape", [(1, 64, 8), (3, 100, 12), (2, 256, 160)])
def test_scales_to_gemm_layout_is_the_blocked_permutation(shape):
    """Integer permutation, bit-exact: (b, r, kb) -> [b][kb/4][r][kb%4]."""
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    s = np.random.default_rng(shape[1]).integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    B, R, KB = shape
    want = s.reshape(B, R, KB // 4, 4).transpose(0, 2, 1, 3)
    got = mx.mx_scales_to_gemm_layout(to_dev_u8(s)).cpu().numpy().reshape(B, KB // 4, R, 4)
    np.testing.assert_array_equal(got, want)


def test_gemm_deterministic_and_errors():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = inp.make_inputs("tiny")
    A, W, offs = to_dev_bf16(x.A), to_dev_bf16(x.W), to_dev_i32(x.offs)
    a = mx.mx_grouped_mm_fwd(A, W, offs)
    b = mx.mx_grouped_mm_fwd(A, W, offs)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    with pytest.raises(mx.MXError, match="MX_ERR_SHAPE"):
        mx.mx_grouped_mm_fwd(A[:, :224].contiguous(), W[:, :, :224].contiguous(), offs)
    with pytest.raises(mx.MXError, match="MX_ERR_WORKSPACE"):
        mx.mx_grouped_mm_fwd(A, W, offs, ws=torch.empty(1024, dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(mx.MXError, match="MX_ERR_SHAPE"):
        mx.mx_grouped_mm_wgrad(to_dev_bf16(x.A[:250]), to_dev_bf16(x.A[:250]), offs)


@pytest.mark.parametrize("mode", [0, 1])
def test_tile_order_does_not_change_results(mode):
    """Race check: workgroups dealt to tiles in seeded pseudo-random orders
    (so different tiles share the chip, in a different sequence) give
    bit-identical outputs, ragged and empty groups included, and the same as
    the repeated default order."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(720 + mode)
    if mode == 0:
        counts = [300, 0, 1, 511, 45, 0, 900, 32]
        I, J, Kc, E = sum(counts), 520, 640, len(counts)
        X, Y = _random_codes(rng, (I, Kc)), _random_codes(rng, (E, J, Kc))
        sX = rng.integers(112, 142, size=(I, Kc // 32)).astype(np.uint8)
        sY = rng.integers(112, 142, size=(E, J, Kc // 32)).astype(np.uint8)
    else:
        counts = [96, 32, 0, 480, 64, 0, 320]
        I, J, E = 520, 392, len(counts)
        Kc = 1024
        X, Y = _random_codes(rng, (I, Kc)), _random_codes(rng, (J, Kc))
        sX = rng.integers(112, 142, size=(I, Kc // 32)).astype(np.uint8)
        sY = rng.integers(112, 142, size=(J, Kc // 32)).astype(np.uint8)
    offs = inp.offsets_from_counts(counts)
    log(f"tile order mode={mode} counts={counts}")
    args = (to_dev_u8(X), mx.mx_scales_to_gemm_layout(to_dev_u8(sX)), to_dev_u8(Y),
            mx.mx_scales_to_gemm_layout(to_dev_u8(sY)), to_dev_i32(offs), mode)
    ref = mx.mx_grouped_gemm_mx(*args)
    for seed in [0, 1, 2, 3, 4, 5, 6, 7, 12345, 2 ** 40 + 3]:
        got = mx.mx_grouped_gemm_mx_ordered(*args, seed)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), seed
    # and the default order is reproducible launch after launch
    for _ in range(3):
        assert torch.equal(mx.mx_grouped_gemm_mx(*args).view(torch.int16), ref.view(torch.int16))


def test_gemm_refuses_row_major_scales():
    """The scale layout travels with the data (its shape) and through the C
    ABI (the layout argument): row-major scales raise a clear error."""
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = inp.make_inputs("tiny")
    qA, sA = mx.mx_quantize_rowwise(to_dev_bf16(x.A))           # sA row-major [M, K/32]
    qW, sW = mx.mx_quantize_rowwise(to_dev_bf16(x.W))
    offs = to_dev_i32(x.offs)
    with pytest.raises(ValueError, match="mx_scales_to_gemm_layout"):
        mx.mx_grouped_gemm_mx(qA, sA, qW, sW, offs, 0)
    with pytest.raises(mx.MXError, match="MX_ERR_LAYOUT"):
        mx.mx_grouped_gemm_mx(qA, sA, qW, sW, offs, 0, scale_layout="rowmajor")
    g = mx.mx_scales_to_gemm_layout
    ok = mx.mx_grouped_gemm_mx(qA, g(sA), qW, g(sW), offs, 0)
    ref = mx.mx_grouped_mm_fwd(to_dev_bf16(x.A), to_dev_bf16(x.W), offs)
    import torch
    assert torch.equal(ok.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("offs,M,align,want", [
    ([96, 256], 256, 32, 0),
    ([96, 250], 256, 1, 4),              # last offset != M
    ([100, 256], 256, 32, 8),            # group start 100 not a multiple of 32
    ([160, 96, 256], 256, 1, 1),         # decreasing
    ([-4, 256], 256, 1, 1 | 2),          # below zero: decreasing and out of range
    ([96, 300], 256, 1, 2 | 4),          # past M
    ([0, 0, 256, 256], 256, 32, 0),      # empty groups are fine
])
def test_check_offsets_bitmask(offs, M, align, want):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    got = int(mx.mx_check_offsets(to_dev_i32(np.array(offs, dtype=np.int32)), M, align).item())
    assert got == want, (offs, got, want)


# ---------------------------------------------------------------------------
# Full-size workloads, sampled outputs (the bench's launch configuration).
# ---------------------------------------------------------------------------
_CACHE = {}


def _workload(name):
    # "<name>_pad32": the workload with every group padded to a multiple of 32
    # (the wgrad contract), e.g. the skewed DeepSeek-style routing
    if name.endswith("_pad32"):
        return dataclasses.replace(inp.WORKLOADS[name[:-6]], pad32=True)
    return inp.WORKLOADS[name]


def _inputs(name, with_grad=False):
    key = (name, with_grad)
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = inp.make_inputs(_workload(name), with_grad=with_grad)
    return _CACHE[key]


def _span_corners(lo, hi, rng, span=128, extra=4):
    """First and last index of every `span`-wide block of [lo, hi) (every
    tile's edges, a group's partial last tile included) plus a few random
    indices, sorted and unique."""
    if hi <= lo:
        return np.zeros(0, dtype=np.int64)
    idx = set()
    for s in range(lo, hi, span):
        idx.add(s)
        idx.add(min(s + span, hi) - 1)
    idx.update(int(v) for v in rng.integers(lo, hi, size=extra))
    return np.array(sorted(idx), dtype=np.int64)


def _live_bounds(x):
    return [(e, a, b) for e, (a, b) in enumerate(oracle.group_bounds(x.offs, x.M_rows)) if b > a]


def _pick(t, rows, cols):
    """Device tensor t[rows][:, cols] as host bf16 bits."""
    import torch
    r = torch.as_tensor(rows, device=t.device)
    c = torch.as_tensor(cols, device=t.device)
    return bf16_host_bits(t.index_select(0, r).index_select(1, c))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama4_fwd", "debug_shard", "deepseek_share"])
def test_fwd_full_size_every_expert(name):
    """Every expert, the edges of every 128-row span of its group (each
    M-tile's first and last row, the partial last tile included) against the
    edges of every 128-column span of N, in the bench's launch shape."""
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = _inputs(name)
    rng = np.random.default_rng(800)
    log(f"fwd full {name} M={x.M_rows} counts min/max={int(x.counts.min())}/{int(x.counts.max())}")
    out = mx.mx_grouped_mm_fwd(to_dev_bf16(x.A), to_dev_bf16(x.W), to_dev_i32(x.offs))
    N = x.W.shape[1]
    cols = _span_corners(0, N, rng, extra=16)
    refs, gots, abss = [], [], []
    for e, a, b in _live_bounds(x):
        rows = _span_corners(a, b, rng)
        qW, sW = oracle.quantize_rowwise(np.ascontiguousarray(x.W[e][cols]))   # W rows are blocks along K
        qA, sA = oracle.quantize_rowwise(x.A[rows])
        dA_, dW_ = oracle.dequant_rowwise(qA, sA), oracle.dequant_rowwise(qW, sW)
        refs.append(dA_ @ dW_.T)
        abss.append(np.abs(dA_) @ np.abs(dW_).T)
        gots.append(_pick(out, rows, cols))
    log(f"fwd full {name}: {len(refs)} experts, {sum(r.shape[0] for r in refs)} rows x {len(cols)} cols")
    _r1(np.concatenate(gots), np.concatenate(refs), f"fwd full {name}", np.concatenate(abss))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama4_bwd", "debug_shard", "deepseek_share"])
def test_dgrad_full_size_every_expert(name):
    """dgrad on every expert: tile-edge rows of every group against tile-edge
    columns of K; W is blocked along N (its columns are the blocks)."""
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = _inputs(name, with_grad=True)
    rng = np.random.default_rng(801)
    log(f"dgrad full {name} M={x.M_rows}")
    out = mx.mx_grouped_mm_dgrad(to_dev_bf16(x.dOut), to_dev_bf16(x.W), to_dev_i32(x.offs))
    K = x.W.shape[2]
    cols = _span_corners(0, K, rng, extra=16)
    refs, gots, abss = [], [], []
    for e, a, b in _live_bounds(x):
        rows = _span_corners(a, b, rng)
        qWt, sWt = oracle.quantize_colwise(np.ascontiguousarray(x.W[e][:, cols]))     # [|cols|, N]
        qG, sG = oracle.quantize_rowwise(x.dOut[rows])
        dG_, dWt_ = oracle.dequant_rowwise(qG, sG), oracle.dequant_rowwise(qWt, sWt)
        refs.append(dG_ @ dWt_.T)
        abss.append(np.abs(dG_) @ np.abs(dWt_).T)
        gots.append(_pick(out, rows, cols))
    log(f"dgrad full {name}: {len(refs)} experts, {sum(r.shape[0] for r in refs)} rows x {len(cols)} cols")
    _r1(np.concatenate(gots), np.concatenate(refs), f"dgrad full {name}", np.concatenate(abss))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama4_bwd", "debug_shard", "deepseek_share_pad32"])
def test_wgrad_full_size_every_expert(name):
    """wgrad on every live expert: the edges of every 128-row span of N
    against the edges of every 128-column span of K (every output tile's
    corners); empty experts must be exact zeros."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = _inputs(name, with_grad=True)
    rng = np.random.default_rng(802)
    log(f"wgrad full {name} M={x.M_rows}")
    dW = mx.mx_grouped_mm_wgrad(to_dev_bf16(x.dOut), to_dev_bf16(x.A), to_dev_i32(x.offs))
    E, N, K = x.W.shape
    refs, gots, abss = [], [], []
    live = _live_bounds(x)
    for e, (a, b) in enumerate(oracle.group_bounds(x.offs, x.M_rows)):
        if b == a:
            assert not bool(dW[e].view(torch.int16).any()), f"empty expert {e} must get exact zeros"
    for e, a, b in live:
        ns = _span_corners(0, N, rng, extra=4)
        ks = _span_corners(0, K, rng, extra=4)
        qGt, sGt = oracle.quantize_colwise(np.ascontiguousarray(x.dOut[a:b][:, ns]))   # [|ns|, m_e]
        qAt, sAt = oracle.quantize_colwise(np.ascontiguousarray(x.A[a:b][:, ks]))      # [|ks|, m_e]
        dGt_, dAt_ = oracle.dequant_rowwise(qGt, sGt), oracle.dequant_rowwise(qAt, sAt)
        refs.append((dGt_ @ dAt_.T).ravel())
        abss.append((np.abs(dGt_) @ np.abs(dAt_).T).ravel())
        gots.append(_pick(dW[e], ns, ks).ravel())
    log(f"wgrad full {name}: {len(live)} live experts, {sum(r.size for r in refs)} outputs")
    _r1(np.concatenate(gots), np.concatenate(refs), f"wgrad full {name}", np.concatenate(abss))
