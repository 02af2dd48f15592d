"""GPU parity of the routed-expert path: grouping (mx_route), the token gather
inside the dual quantizer (mx_quantize_dual_gather), the row-mapped GEMM
epilogue (mx_grouped_gemm_mx_rows) and the differentiable composition
(mx_routed_experts).

  - mx_route: offs, rows, pos and status bit-exact against the oracle's
    grouping (stable order, groups padded to 32), on the Llama4-shaped and
    DeepSeek-shaped routings, empty / skewed / single-expert cases, no tokens,
    out-of-range ids and the largest expert count;
  - the gathered dual quantizer: bit-exact against the oracle's rowwise and
    colwise quantization of the gathered, zero-padded rows (top-1 and top-2);
  - the row-mapped GEMM: bit-identical to the plain GEMM followed by a
    scatter, dropped rows and untouched rows included;
  - mx_routed_experts: forward, dx and dW bit-identical to the grouped
    primitive on explicitly grouped bf16 tensors, within the GEMM criterion of
    the routed oracle, and close to an fp64 autograd reference.
"""

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, u8_host, bf16_host_bits, log
from mxfp8_block_scaled_06_amd.autograd import WeightCache

pytestmark = pytest.mark.gpu


def _gemm_layout(s_rowmajor: np.ndarray) -> np.ndarray:
    R, KB = s_rowmajor.shape
    return np.ascontiguousarray(s_rowmajor.reshape(R, KB // 4, 4).transpose(1, 0, 2))


def _ids(case):
    if case == "hand":
        return np.array([1, 0, 1, 2], dtype=np.int32), 3
    if case == "llama4_uniform":
        rng = np.random.default_rng(2)
        return inp.expert_ids(rng, inp.uniform_counts(rng, 16384, 16)), 16
    if case == "deepseek_zipf":
        rng = np.random.default_rng(5)
        return inp.expert_ids(rng, inp.zipf_counts(rng, 32768, 32)), 32
    if case == "all_in_last":
        return np.full(5000, 7, dtype=np.int32), 8
    if case == "empty_first_and_consecutive":
        rng = np.random.default_rng(7)
        return inp.expert_ids(rng, [0, 0, 700, 0, 0, 333]), 6
    if case == "no_tokens":
        return np.zeros(0, dtype=np.int32), 4
    if case == "out_of_range":
        rng = np.random.default_rng(9)
        ids = inp.expert_ids(rng, [1000, 900, 0, 1100, 1])
        ids[::13] = 5
        ids[5::17] = -3
        return ids, 5
    if case == "max_experts":
        rng = np.random.default_rng(11)
        return rng.integers(0, 1024, size=2049).astype(np.int32), 1024
    raise KeyError(case)


ROUTE_CASES = ["hand", "llama4_uniform", "deepseek_zipf", "all_in_last", "empty_first_and_consecutive",
               "no_tokens", "out_of_range", "max_experts"]


@pytest.mark.parametrize("case", ROUTE_CASES)
def test_route_matches_oracle(case):
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    ids, E = _ids(case)
    cap = mx.route_capacity(ids.shape[0], E)
    log(f"route case={case} n={ids.shape[0]} E={E} cap={cap}")
    offs, rows, pos, status = mx.mx_route(to_dev_i32(ids), E)
    torch.cuda.synchronize()
    r_offs, r_rows, r_pos, bad = oracle.route_groups(ids, E, cap)
    assert np.array_equal(offs.cpu().numpy(), r_offs)
    assert np.array_equal(rows.cpu().numpy(), r_rows)
    assert np.array_equal(pos.cpu().numpy(), r_pos)
    assert int(status.item()) == int(bad)


def test_route_is_deterministic_and_rejects_small_capacity():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    ids, E = _ids("deepseek_zipf")
    d = to_dev_i32(ids)
    first = [t.clone() for t in mx.mx_route(d, E)]
    for _ in range(3):
        again = mx.mx_route(d, E)
        assert all(torch.equal(a, b) for a, b in zip(first, again))
    with pytest.raises(mx.MXError, match="cap"):
        mx.mx_route(d, E, cap=ids.shape[0] + 31 * E - 1)


@pytest.mark.parametrize("T,E,K,topk,seed", [
    (300, 4, 256, 1, 21),
    (1000, 3, 128, 2, 22),       # items of a top-2 router: token = item // 2
    (77, 5, 384, 1, 23),         # most groups a single partial block
])
def test_dual_gather_matches_oracle(T, E, K, topk, seed):
    require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=T * topk).astype(np.int32)
    x = inp.random_bf16((T, K), seed=seed, outliers=True)
    offs, rows, _, _ = mx.mx_route(to_dev_i32(ids), E)
    rows_h = rows.cpu().numpy()
    M = rows_h.shape[0]
    log(f"dual gather T={T} E={E} K={K} topk={topk} M={M}")
    q, s, qt, st = mx.mx_quantize_dual_gather(to_dev_bf16(x), rows, topk=topk)
    g = oracle.gather_rows(x, rows_h, topk=topk)
    rq, rs = oracle.quantize_rowwise(g)
    cq, cs = oracle.quantize_colwise(g)
    ldq = qt.shape[1]
    cq_pad = np.zeros((K, ldq), dtype=np.uint8)
    cq_pad[:, :M] = cq
    cs_pad = np.zeros((K, ldq // 32), dtype=np.uint8)
    cs_pad[:, :M // 32] = cs
    for name, got, ref in (("q", u8_host(q), rq), ("s", u8_host(s), _gemm_layout(rs)),
                           ("q_t", u8_host(qt), cq_pad), ("s_t", u8_host(st), _gemm_layout(cs_pad))):
        assert got.shape == ref.shape, name
        assert np.array_equal(got, ref), name


def test_rows_gemm_equals_gemm_then_scatter():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(31)
    T, E, K, N = 700, 4, 256, 384
    ids = inp.expert_ids(rng, [200, 0, 320, 180])
    ids[::11] = 9                                           # dropped tokens: their rows stay untouched
    x = inp.random_bf16((T, K), seed=32, outliers=True)
    W = inp.random_bf16((E, N, K), seed=33, std=0.02)
    log(f"rows GEMM T={T} E={E} K={K} N={N}")
    offs, rows, _, _ = mx.mx_route(to_dev_i32(ids), E)
    qX, sX, _, _ = mx.mx_quantize_dual_gather(to_dev_bf16(x), rows)
    qW, sW, _, _ = mx.mx_quantize_weights(to_dev_bf16(W))
    plain = mx.mx_grouped_gemm_mx(qX, sX, qW, sW, offs, 0)
    sentinel = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda:0")
    got = mx.mx_grouped_gemm_mx_rows(qX, sX, qW, sW, offs, rows, out=sentinel.clone())
    torch.cuda.synchronize()
    rows_h = rows.cpu().numpy()
    want = sentinel.clone()
    live = np.flatnonzero((rows_h >= 0) & (np.arange(rows_h.shape[0]) < int(offs[-1].item())))
    want[torch.from_numpy(rows_h[live]).long().cuda()] = plain[torch.from_numpy(live).long().cuda()]
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    # a map entry past c_rows is dropped: store only the first 100 tokens
    part = mx.mx_grouped_gemm_mx_rows(qX, sX, qW, sW, offs, rows, c_rows=100)
    want_part = want[:100].clone()
    want_part[torch.from_numpy(ids[:100] == 9).cuda()] = 0          # a new output starts at zero
    assert torch.equal(part.view(torch.int16), want_part.view(torch.int16))


def _fp64_reference(x, ids, W, G):
    import torch
    x64 = torch.from_numpy(oracle.bf16_to_f64(x)).requires_grad_(True)
    W64 = torch.from_numpy(oracle.bf16_to_f64(W)).requires_grad_(True)
    out = torch.zeros((x.shape[0], W.shape[1]), dtype=torch.float64)
    for e in range(W.shape[0]):
        sel = torch.from_numpy(np.flatnonzero(ids == e))
        if sel.numel():
            out = out.index_put((sel,), x64[sel] @ W64[e].T)
    out.backward(torch.from_numpy(oracle.bf16_to_f64(G)))
    return out.detach().numpy(), x64.grad.numpy(), W64.grad.numpy()


def _normwise(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


ROUTED_CASES = {
    "skewed": ([300, 0, 41, 555, 1], 256, 384),
    "single_expert": ([640], 384, 256),
    "empty_last": ([130, 70, 0], 256, 256),
}


@pytest.mark.parametrize("case", sorted(ROUTED_CASES))
def test_routed_experts_autograd(case):
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    counts, N, K = ROUTED_CASES[case]
    E, T = len(counts), sum(counts)
    rng = np.random.default_rng(40 + E)
    ids = inp.expert_ids(rng, counts)
    x = inp.random_bf16((T, K), seed=41 + E, outliers=True)
    W = inp.random_bf16((E, N, K), seed=42 + E, std=0.02)
    G = inp.random_bf16((T, N), seed=43 + E, std=1e-3)
    log(f"routed autograd case={case} counts={counts} N={N} K={K}")
    xd = to_dev_bf16(x).requires_grad_(True)
    Wd = to_dev_bf16(W).requires_grad_(True)
    out = mx.mx_routed_experts(xd, to_dev_i32(ids), Wd)
    out.backward(to_dev_bf16(G))
    torch.cuda.synchronize()
    # the grouped primitive on explicitly grouped (host-gathered) bf16 tensors
    cap = mx.route_capacity(T, E)
    offs, rows, _, _ = oracle.route_groups(ids, E, cap)
    used = rows[:int(offs[-1])]
    xg = to_dev_bf16(oracle.gather_rows(x, used)).requires_grad_(True)
    Wg = to_dev_bf16(W).requires_grad_(True)
    og = mx.mx_grouped_mm(xg, Wg, to_dev_i32(offs), cache=WeightCache())
    og.backward(to_dev_bf16(oracle.gather_rows(G, used)))
    live = np.flatnonzero(used >= 0)
    tok = used[live]
    got_out, got_dx = bf16_host_bits(out), bf16_host_bits(xd.grad)
    assert np.array_equal(got_out[tok], bf16_host_bits(og)[live])
    assert np.array_equal(got_dx[tok], bf16_host_bits(xg.grad)[live])
    assert np.array_equal(bf16_host_bits(Wd.grad), bf16_host_bits(Wg.grad))
    # the routed oracle
    for name, got, ref, absr in (
            ("out", got_out, oracle.routed_fwd(x, ids, W, cap), oracle.routed_fwd(x, ids, W, cap, absolute=True)),
            ("dx", got_dx, oracle.routed_dgrad(G, ids, W, cap), oracle.routed_dgrad(G, ids, W, cap, absolute=True)),
            ("dW", bf16_host_bits(Wd.grad), oracle.routed_wgrad(G, x, ids, E, cap),
             oracle.routed_wgrad(G, x, ids, E, cap, absolute=True))):
        rep = oracle.r1_check(got, ref, abs_terms=absr)
        log(f"  {name}: normwise={rep['normwise_rel']:.2e} plain_frac={rep['plain_r1_frac']:.2e}")
        assert rep["ok"], (name, rep)
    # fp64 autograd of the unquantized routed layer
    f_out, f_dx, f_dW = _fp64_reference(x, ids, W, G)
    for name, got, ref, mxref in (("out", got_out, f_out, oracle.routed_fwd(x, ids, W, cap)),
                                  ("dx", got_dx, f_dx, oracle.routed_dgrad(G, ids, W, cap)),
                                  ("dW", bf16_host_bits(Wd.grad), f_dW, oracle.routed_wgrad(G, x, ids, E, cap))):
        g = oracle.bf16_to_f64(got)
        assert _normwise(g, ref) <= 2 * _normwise(mxref, ref) + 4e-3, name


def test_routed_experts_checks_and_drops_out_of_range_ids():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    T, E, K, N = 200, 3, 128, 128
    rng = np.random.default_rng(51)
    ids = rng.integers(0, E, size=T).astype(np.int32)
    ids[::9] = 3
    x = inp.random_bf16((T, K), seed=52)
    W = inp.random_bf16((E, N, K), seed=53, std=0.02)
    G = inp.random_bf16((T, N), seed=54, std=1e-3)
    log("routed experts: out-of-range ids")
    with pytest.raises(ValueError, match="outside"):
        mx.mx_routed_experts(to_dev_bf16(x), to_dev_i32(ids), to_dev_bf16(W))
    xd = to_dev_bf16(x).requires_grad_(True)
    Wd = to_dev_bf16(W).requires_grad_(True)
    out = mx.mx_routed_experts(xd, to_dev_i32(ids), Wd, check=False)
    out.backward(to_dev_bf16(G))
    torch.cuda.synchronize()
    dropped = torch.from_numpy(ids == 3).cuda()
    assert (out[dropped] == 0).all() and (xd.grad[dropped] == 0).all()
    cap = mx.route_capacity(T, E)
    for name, got, ref, absr in (
            ("out", bf16_host_bits(out), oracle.routed_fwd(x, ids, W, cap),
             oracle.routed_fwd(x, ids, W, cap, absolute=True)),
            ("dW", bf16_host_bits(Wd.grad), oracle.routed_wgrad(G, x, ids, E, cap),
             oracle.routed_wgrad(G, x, ids, E, cap, absolute=True))):
        assert oracle.r1_check(got, ref, abs_terms=absr)["ok"], name


def test_routed_experts_full_size_llama4_sampled():
    """T=16384 tokens over 16 experts, K=5120, N=8192 (the Llama4-shaped
    forward): every expert's first and last token and a random sample checked
    row by row against the oracle's per-token definition; the output is
    bit-identical to the grouped primitive on the host-grouped tokens."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    T, E, K, N = 16384, 16, 5120, 8192
    rng = np.random.default_rng(2)
    ids = inp.expert_ids(rng, inp.uniform_counts(rng, T, E))
    x = inp.random_bf16((T, K), seed=61, outliers=True)
    W = inp.random_bf16((E, N, K), seed=62, std=0.02)
    log("routed experts full size T=16384 E=16 K=5120 N=8192")
    Wd = to_dev_bf16(W)
    cache = WeightCache()
    out = mx.mx_routed_experts(to_dev_bf16(x), to_dev_i32(ids), Wd, cache=cache)
    cap = mx.route_capacity(T, E)
    offs, rows, _, _ = oracle.route_groups(ids, E, cap)
    used = rows[:int(offs[-1])]
    ref = mx.mx_grouped_mm(to_dev_bf16(oracle.gather_rows(x, used)), Wd, to_dev_i32(offs), cache=cache)
    torch.cuda.synchronize()
    live = np.flatnonzero(used >= 0)
    got = bf16_host_bits(out)
    assert np.array_equal(got[used[live]], bf16_host_bits(ref)[live])
    picks = set(rng.choice(T, size=24, replace=False).tolist())
    for e in range(E):
        mine = np.flatnonzero(ids == e)
        picks.update([int(mine[0]), int(mine[-1])])
    picks = sorted(picks)
    qx, sx = oracle.quantize_rowwise(x[picks])
    dx = oracle.dequant_rowwise(qx, sx)
    r = np.zeros((len(picks), N))
    a = np.zeros((len(picks), N))
    for e in range(E):
        sel = [i for i, t in enumerate(picks) if ids[t] == e]
        if sel:
            qw, sw = oracle.quantize_rowwise(W[e])
            dw = oracle.dequant_rowwise(qw, sw)
            r[sel] = dx[sel] @ dw.T
            a[sel] = np.abs(dx[sel]) @ np.abs(dw).T
    rep = oracle.r1_check(got[picks], r, abs_terms=a)
    log(f"  sampled rows: normwise={rep['normwise_rel']:.2e}")
    assert rep["ok"], rep


# --------------------------------------------------------------------------
# Top-k routers
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,cols", [(300, 3, 264), (64, 1, 128), (1000, 8, 512), (300, 2, 264), (120, 4, 512),
                                      (200, 5, 128), (150, 6, 136), (100, 7, 256)])
def test_topk_sum_rows_matches_oracle(T, k, cols):
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(70 + k)
    x = (rng.standard_normal((T * k, cols)) * np.exp2(rng.integers(-20, 20, size=(T * k, 1)))).astype(np.float32)
    log(f"topk sum T={T} k={k} cols={cols}")
    got = mx.mx_topk_sum_rows(torch.from_numpy(x).cuda(), k)
    assert np.array_equal(bf16_host_bits(got), oracle.topk_sum_rows(x, k))


def test_rows_gemm_f32_equals_gemm_f32_then_scatter():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    rng = np.random.default_rng(71)
    T, k, E, K, N = 200, 2, 3, 256, 128
    ids = rng.integers(0, E, size=T * k).astype(np.int32)
    x = inp.random_bf16((T, K), seed=72, outliers=True)
    W = inp.random_bf16((E, N, K), seed=73, std=0.02)
    log("rows GEMM fp32 output")
    offs, rows, _, _ = mx.mx_route(to_dev_i32(ids), E)
    qX, sX, _, _ = mx.mx_quantize_dual_gather(to_dev_bf16(x), rows, topk=k)
    qW, sW, _, _ = mx.mx_quantize_weights(to_dev_bf16(W))
    plain = mx.mx_grouped_gemm_mx_f32(qX, sX, qW, sW, offs, 0)
    got = mx.mx_grouped_gemm_mx_rows(qX, sX, qW, sW, offs, rows, c_rows=T * k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows_h = rows.cpu().numpy()
    live = np.flatnonzero(rows_h >= 0)
    want = np.zeros((T * k, N), dtype=np.float32)
    want[rows_h[live]] = plain.cpu().numpy()[live]
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("k,counts_seed", [(2, 80), (4, 81)])
def test_routed_experts_topk_autograd(k, counts_seed):
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    T, E, K, N = 160, 5, 256, 256
    rng = np.random.default_rng(counts_seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[ids == 3] = 1                                   # expert 3 gets no items
    x = inp.random_bf16((T, K), seed=counts_seed + 1, outliers=True)
    W = inp.random_bf16((E, N, K), seed=counts_seed + 2, std=0.02)
    G = inp.random_bf16((T * k, N), seed=counts_seed + 3, std=1e-3)
    log(f"routed experts top-{k} autograd T={T} E={E}")
    xd = to_dev_bf16(x).requires_grad_(True)
    Wd = to_dev_bf16(W).requires_grad_(True)
    out = mx.mx_routed_experts(xd, to_dev_i32(ids), Wd, cache=WeightCache())
    assert tuple(out.shape) == (T, k, N)
    out.backward(to_dev_bf16(G).view(T, k, N))
    torch.cuda.synchronize()
    flat = ids.reshape(-1)
    cap = mx.route_capacity(T * k, E)
    for name, got, ref, absr in (
            ("out", bf16_host_bits(out).reshape(T * k, N), oracle.routed_fwd(x, flat, W, cap, topk=k),
             oracle.routed_fwd(x, flat, W, cap, absolute=True, topk=k)),
            ("dx", bf16_host_bits(xd.grad), oracle.routed_dgrad(G, flat, W, cap, topk=k),
             oracle.routed_dgrad(G, flat, W, cap, absolute=True, topk=k)),
            ("dW", bf16_host_bits(Wd.grad), oracle.routed_wgrad(G, x, flat, E, cap, topk=k),
             oracle.routed_wgrad(G, x, flat, E, cap, absolute=True, topk=k))):
        rep = oracle.r1_check(got, ref, abs_terms=absr)
        log(f"  {name}: normwise={rep['normwise_rel']:.2e} plain_frac={rep['plain_r1_frac']:.2e}")
        assert rep["ok"], (name, rep)
    assert (bf16_host_bits(Wd.grad)[3] == 0).all()
    # fp64 autograd of the unquantized top-k layer
    x64 = torch.from_numpy(oracle.bf16_to_f64(x)).requires_grad_(True)
    W64 = torch.from_numpy(oracle.bf16_to_f64(W)).requires_grad_(True)
    ref = torch.stack([x64[t // k] @ W64[int(flat[t])].T for t in range(T * k)])
    ref.backward(torch.from_numpy(oracle.bf16_to_f64(G)))
    for name, got, r64, mxref in (
            ("out", bf16_host_bits(out).reshape(T * k, N), ref.detach().numpy(),
             oracle.routed_fwd(x, flat, W, cap, topk=k)),
            ("dx", bf16_host_bits(xd.grad), x64.grad.numpy(), oracle.routed_dgrad(G, flat, W, cap, topk=k)),
            ("dW", bf16_host_bits(Wd.grad), W64.grad.numpy(), oracle.routed_wgrad(G, x, flat, E, cap, topk=k))):
        assert _normwise(oracle.bf16_to_f64(got), r64) <= 2 * _normwise(mxref, r64) + 4e-3, name
