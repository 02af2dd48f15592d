"""Seeded random shapes through every entry point, against the oracle.

The other GPU tests pick their shapes by hand, one per code path.  Here each
case draws its sizes from a seed, within the entry point's shape contract, so
the kernels meet tile remainders, batch counts, padded strides and group
layouts that no hand-picked case covers: the quantizers' two colwise kernels
and both tile orders of the 256-column one, and the grouped GEMM's partial
M-tiles, empty groups and odd N and K extents.  The bar is the usual one:
quantizer bytes equal the oracle's, GEMM outputs pass oracle.r1_check.
"""

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, bf16_host_bits, u8_host, log

pytestmark = pytest.mark.gpu

N_QUANT = 32
N_GEMM = 12


def _quant_shape(rng, mode):
    batch = int(rng.integers(1, 4))
    if mode == "rowwise":
        rows, cols = int(rng.integers(1, 700)), 32 * int(rng.integers(1, 40))
    elif mode == "colwise":
        # half the cases on 256-column multiples (the 256 x 256 tile kernel)
        rows = 32 * int(rng.integers(1, 30))
        cols = 256 * int(rng.integers(1, 5)) if rng.random() < 0.5 else 8 * int(rng.integers(1, 120))
    else:
        rows, cols = 32 * int(rng.integers(1, 25)), 32 * int(rng.integers(1, 30))
    return (batch, rows, cols) if batch > 1 else (rows, cols)


def _oracle_quant(mode, x3):
    fn = {"rowwise": oracle.quantize_rowwise, "colwise": oracle.quantize_colwise,
          "32x32": oracle.quantize_32x32}[mode]
    qs, ss = zip(*(fn(np.ascontiguousarray(x3[b])) for b in range(x3.shape[0])))
    return np.stack(qs), np.stack(ss)


@pytest.mark.parametrize("mode", ["rowwise", "colwise", "32x32"])
@pytest.mark.parametrize("case", range(N_QUANT))
def test_quantizer_random_shapes(mode, case):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(9000 + 100 * ["rowwise", "colwise", "32x32"].index(mode) + case)
    shape = _quant_shape(rng, mode)
    std = float(rng.choice([1e-3, 0.02, 1.0, 300.0]))
    x = inp.random_bf16(shape, seed=int(rng.integers(1 << 30)), std=std, outliers=True)
    log(f"fuzz quant {mode} case={case} shape={shape} std={std}")
    fn = {"rowwise": mx.mx_quantize_rowwise, "colwise": mx.mx_quantize_colwise, "32x32": mx.mx_quantize_32x32}[mode]
    q, s = fn(to_dev_bf16(x))
    x3 = x if x.ndim == 3 else x[None]
    rq, rs = _oracle_quant(mode, x3)
    gq, gs = u8_host(q).reshape(rq.shape), u8_host(s).reshape(rs.shape)
    assert np.array_equal(gq, rq), f"{mode} {shape}: {np.count_nonzero(gq != rq)} code mismatches"
    assert np.array_equal(gs, rs), f"{mode} {shape}: {np.count_nonzero(gs != rs)} scale mismatches"


def _gemm_layout(s_rowmajor):
    R, KB = s_rowmajor.shape
    return np.ascontiguousarray(s_rowmajor.reshape(R, KB // 4, 4).transpose(1, 0, 2))


@pytest.mark.parametrize("case", range(N_QUANT))
def test_dual_random_shapes(case):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(9500 + case)
    rows = 32 * int(rng.integers(1, 30))
    cols = 128 * int(rng.integers(1, 7))
    ldq = (rows + 127) // 128 * 128 + 128 * int(rng.integers(0, 3))
    x = inp.random_bf16((rows, cols), seed=int(rng.integers(1 << 30)), std=1.0, outliers=True)
    log(f"fuzz dual case={case} shape={(rows, cols)} ldq={ldq}")
    q, s, qt, st = (u8_host(t) for t in mx.mx_quantize_dual(to_dev_bf16(x), ldq=ldq))
    rq, rs = oracle.quantize_rowwise(x)
    cq, cs = oracle.quantize_colwise(x)
    cq_pad = np.zeros((cols, ldq), dtype=np.uint8)
    cq_pad[:, :rows] = cq
    cs_pad = np.zeros((cols, ldq // 32), dtype=np.uint8)
    cs_pad[:, :rows // 32] = cs
    for name, got, ref in (("q", q, rq), ("s", s, _gemm_layout(rs)), ("q_t", qt, cq_pad),
                           ("s_t", st, _gemm_layout(cs_pad))):
        assert np.array_equal(got.reshape(ref.shape), ref), f"dual {name} {(rows, cols, ldq)}"


def _counts(rng, E, total_max, mult):
    c = rng.integers(0, total_max // E + 1, size=E) // mult * mult
    c[rng.random(E) < 0.25] = 0
    if c.sum() == 0:
        c[int(rng.integers(E))] = mult * int(rng.integers(1, 8))
    return [int(v) for v in c]


def _check(got, ref, absolute, tag, sigma=None):
    rep = oracle.r1_check(got, ref, sigma=sigma, abs_terms=absolute)
    log(f"{tag}: n={rep['n']} bad={rep['n_bad']} normwise={rep['normwise_rel']:.2e} "
        f"plain_r1={100 * rep['plain_r1_frac']:.3f}%")
    assert rep["ok"], f"{tag}: {rep}"


@pytest.mark.parametrize("case", range(N_GEMM))
def test_fwd_random_groups(case):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(9700 + case)
    E = int(rng.integers(1, 10))
    counts = _counts(rng, E, 1400, 1)
    K, N = 128 * int(rng.integers(1, 7)), 8 * int(rng.integers(1, 100))
    offs = inp.offsets_from_counts(counts)
    M = sum(counts)
    A = inp.random_bf16((M, K), seed=int(rng.integers(1 << 30)), outliers=True)
    W = inp.random_bf16((E, N, K), seed=int(rng.integers(1 << 30)), std=0.02)
    log(f"fuzz fwd case={case} counts={counts} K={K} N={N}")
    got = bf16_host_bits(mx.mx_grouped_mm_fwd(to_dev_bf16(A), to_dev_bf16(W), to_dev_i32(offs)))
    _check(got, oracle.grouped_mm_fwd(A, W, offs), oracle.grouped_mm_fwd(A, W, offs, absolute=True),
           f"fwd case {case}")


@pytest.mark.parametrize("case", range(N_GEMM))
def test_dgrad_random_groups(case):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(9800 + case)
    E = int(rng.integers(1, 10))
    counts = _counts(rng, E, 1400, 1)
    N, K = 128 * int(rng.integers(1, 7)), 8 * int(rng.integers(1, 100))
    offs = inp.offsets_from_counts(counts)
    M = sum(counts)
    G = inp.random_bf16((M, N), seed=int(rng.integers(1 << 30)), std=1e-3)
    W = inp.random_bf16((E, N, K), seed=int(rng.integers(1 << 30)), std=0.02)
    log(f"fuzz dgrad case={case} counts={counts} N={N} K={K}")
    got = bf16_host_bits(mx.mx_grouped_mm_dgrad(to_dev_bf16(G), to_dev_bf16(W), to_dev_i32(offs)))
    _check(got, oracle.grouped_mm_dgrad(G, W, offs), oracle.grouped_mm_dgrad(G, W, offs, absolute=True),
           f"dgrad case {case}")


@pytest.mark.parametrize("case", range(N_GEMM))
def test_wgrad_random_groups(case):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(9900 + case)
    E = int(rng.integers(1, 10))
    counts = _counts(rng, E, 1400, 32)
    N, K = 8 * int(rng.integers(1, 60)), 8 * int(rng.integers(1, 60))
    offs = inp.offsets_from_counts(counts)
    M = sum(counts)
    A = inp.random_bf16((M, K), seed=int(rng.integers(1 << 30)), outliers=True)
    G = inp.random_bf16((M, N), seed=int(rng.integers(1 << 30)), std=1e-3)
    log(f"fuzz wgrad case={case} counts={counts} N={N} K={K}")
    got = bf16_host_bits(mx.mx_grouped_mm_wgrad(to_dev_bf16(G), to_dev_bf16(A), to_dev_i32(offs)))
    for e, c in enumerate(counts):
        if c == 0:
            assert (got[e] == 0).all(), f"empty expert {e} must get exact zeros"
    _check(got, oracle.grouped_mm_wgrad(G, A, offs), oracle.grouped_mm_wgrad(G, A, offs, absolute=True),
           f"wgrad case {case}")


@pytest.mark.parametrize("case", range(N_GEMM))
def test_routed_experts_random_routings(case):
    """mx_routed_experts forward and backward over random routings: top-1 to
    top-3, skewed expert loads with empty experts, and (with check=False)
    some ids outside [0, E), whose items must come out as zero rows."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    from mxfp8_block_scaled_06_amd.autograd import WeightCache
    rng = np.random.default_rng(9950 + case)
    T, E, k = int(rng.integers(1, 500)), int(rng.integers(1, 12)), int(rng.integers(1, 4))
    K, N = 128 * int(rng.integers(1, 4)), 128 * int(rng.integers(1, 4))
    p = rng.dirichlet(np.full(E, 0.5))
    ids = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    drop = case % 3 == 2
    if drop:
        ids[rng.random((T, k)) < 0.05] = E
    x = inp.random_bf16((T, K), seed=int(rng.integers(1 << 30)), outliers=True)
    W = inp.random_bf16((E, N, K), seed=int(rng.integers(1 << 30)), std=0.02)
    G = inp.random_bf16((T * k, N), seed=int(rng.integers(1 << 30)), std=1e-3)
    log(f"fuzz routed case={case} T={T} E={E} k={k} K={K} N={N} drop={drop} "
        f"loads={np.bincount(ids.ravel(), minlength=E + 1).tolist()}")
    xd = to_dev_bf16(x).requires_grad_(True)
    Wd = to_dev_bf16(W).requires_grad_(True)
    ids_d = to_dev_i32(ids if k > 1 else ids[:, 0])
    out = mx.mx_routed_experts(xd, ids_d, Wd, cache=WeightCache(), check=not drop)
    out.backward(to_dev_bf16(G).view(out.shape))
    torch.cuda.synchronize()
    flat = ids.reshape(-1)
    cap = mx.route_capacity(T * k, E)
    got_out = bf16_host_bits(out).reshape(T * k, N)
    if drop:
        assert (got_out[flat == E] == 0).all()
    for name, got, ref, absr in (
            ("out", got_out, oracle.routed_fwd(x, flat, W, cap, topk=k),
             oracle.routed_fwd(x, flat, W, cap, absolute=True, topk=k)),
            ("dx", bf16_host_bits(xd.grad), oracle.routed_dgrad(G, flat, W, cap, topk=k),
             oracle.routed_dgrad(G, flat, W, cap, absolute=True, topk=k)),
            ("dW", bf16_host_bits(Wd.grad), oracle.routed_wgrad(G, x, flat, E, cap, topk=k),
             oracle.routed_wgrad(G, x, flat, E, cap, absolute=True, topk=k))):
        _check(got, ref, absr, f"routed case {case} {name}")
    for e in range(E):
        if not (flat == e).any():
            assert (bf16_host_bits(Wd.grad)[e] == 0).all(), f"expert {e} has no items: dW must be zeros"
