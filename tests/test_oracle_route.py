"""Pins of the routing oracle (oracle/route.py) against what the readings and
plain arithmetic fix, independent of the oracle's own code path:

  - a grouping worked out by hand;
  - the invariants a stable, 32-padded grouping must satisfy, on random ids
    with empty, skewed and out-of-range experts;
  - routed forward / dgrad equal the per-token definition (each token's row
    quantized on its own, times its expert's weight);
  - on inputs that quantize losslessly, the routed wgrad is exactly
    sum_t dOut[t]^T x[t] over each expert's tokens (Fractions), so a wrong
    gather, scatter or grouping index cannot pass;
  - already-grouped, 32-aligned input reduces to the grouped wgrad.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp


def _bf16_exact(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    bits = v.view(np.uint32)
    assert (bits & 0xFFFF == 0).all(), "value not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def _pow2(shape, seed):
    """Entries 0 or +-2^j, j in [-2, 2]: every 32-block quantizes losslessly."""
    rng = np.random.default_rng(seed)
    v = rng.choice([-1.0, 1.0], size=shape) * np.exp2(rng.integers(-2, 3, size=shape))
    v[rng.random(shape) < 0.1] = 0.0
    return _bf16_exact(v.astype(np.float32))


def test_route_hand_case():
    # ids [1, 0, 1, 2] over 3 experts: expert 0 holds item 1, expert 1 items
    # 0 and 2 (in that order), expert 2 item 3; each group padded to 32 rows
    offs, rows, pos, bad = oracle.route_groups([1, 0, 1, 2], 3, 128)
    assert offs.tolist() == [32, 64, 96]
    want = np.full(128, -1)
    want[0], want[32], want[33], want[64] = 1, 0, 2, 3
    assert rows.tolist() == want.tolist()
    assert pos.tolist() == [32, 0, 33, 64]
    assert not bad


def test_route_hand_case_with_empty_and_invalid():
    # 33 tokens of expert 2 take two 32-row blocks; experts 0, 1, 3 are empty;
    # ids 4 and -1 are outside [0, 4)
    ids = [2] * 33 + [4, -1]
    offs, rows, pos, bad = oracle.route_groups(ids, 4, 200)
    assert offs.tolist() == [0, 0, 64, 64]
    assert rows[:33].tolist() == list(range(33)) and (rows[33:] == -1).all()
    assert pos.tolist() == list(range(33)) + [-1, -1]
    assert bad


def _check_invariants(ids, E, cap):
    offs, rows, pos, bad = oracle.route_groups(ids, E, cap)
    ids = np.asarray(ids)
    valid = (ids >= 0) & (ids < E)
    assert bad == (not valid.all())
    start = 0
    for e in range(E):
        mine = np.flatnonzero(ids == e)
        c = mine.size
        assert offs[e] - start == -(-c // 32) * 32
        assert rows[start:start + c].tolist() == mine.tolist()      # stable order
        assert (rows[start + c:offs[e]] == -1).all()
        start = offs[e]
    assert (rows[start:] == -1).all()
    r = np.flatnonzero(rows >= 0)
    assert (pos[rows[r]] == r).all()
    assert sorted(rows[r].tolist()) == np.flatnonzero(valid).tolist()
    assert (pos[~valid] == -1).all()
    return offs, rows, pos


@pytest.mark.parametrize("seed", range(6))
def test_route_invariants_random(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    n = int(rng.integers(0, 3000))
    p = rng.random(E) ** 3
    p[rng.random(E) < 0.3] = 0.0
    if p.sum() == 0:
        p[0] = 1.0
    ids = rng.choice(E, size=n, p=p / p.sum())
    if seed % 2:
        ids[rng.random(n) < 0.01] = E + 3
    _check_invariants(ids, E, n + 31 * E)


@pytest.mark.parametrize("ids,E", [([], 5), ([0] * 70, 4), ([3] * 64, 4), ([1, 1, 2, 2, 1], 6)],
                         ids=["no_tokens", "all_first", "all_last", "empty_first_and_last"])
def test_route_edge_cases(ids, E):
    _check_invariants(ids, E, len(ids) + 31 * E)


def test_route_rejects_too_small_capacity():
    with pytest.raises(ValueError):
        oracle.route_groups([0] * 33, 1, 63)


def _routed_case(T, E, K, N, seed, invalid=False):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=T)
    ids[: T // 5] = E - 1                       # a skewed expert
    if invalid:
        ids[::7] = -1
    x = inp.random_bf16((T, K), seed=seed + 1, outliers=True)
    W = inp.random_bf16((E, N, K), seed=seed + 2, std=0.02)
    G = inp.random_bf16((T, N), seed=seed + 3, std=1e-3)
    return ids, x, W, G, T + 31 * E


@pytest.mark.parametrize("invalid", [False, True])
def test_routed_fwd_and_dgrad_equal_the_per_token_definition(invalid):
    ids, x, W, G, cap = _routed_case(70, 3, 64, 32, seed=5, invalid=invalid)
    out = oracle.routed_fwd(x, ids, W, cap)
    dx = oracle.routed_dgrad(G, ids, W, cap)
    for t in range(x.shape[0]):
        e = ids[t]
        if not 0 <= e < W.shape[0]:
            assert (out[t] == 0).all() and (dx[t] == 0).all()
            continue
        qx, sx = oracle.quantize_rowwise(x[t:t + 1])
        qw, sw = oracle.quantize_rowwise(W[e])
        np.testing.assert_allclose(out[t], (oracle.dequant_rowwise(qx, sx) @ oracle.dequant_rowwise(qw, sw).T)[0],
                                   rtol=1e-13, atol=1e-300)
        qg, sg = oracle.quantize_rowwise(G[t:t + 1])
        qwt, swt = oracle.quantize_colwise(W[e])              # [K, N] blocked along N
        np.testing.assert_allclose(dx[t], (oracle.dequant_rowwise(qg, sg) @ oracle.dequant_rowwise(qwt, swt).T)[0],
                                   rtol=1e-13, atol=1e-300)


def test_routed_wgrad_lossless_equals_exact_token_sum():
    T, E, K, N = 90, 4, 8, 5
    rng = np.random.default_rng(11)
    ids = rng.integers(0, E, size=T)
    ids[ids == 2] = 1                           # expert 2 gets no tokens
    ids[5] = 9                                  # dropped
    x, G = _pow2((T, K), 12), _pow2((T, N), 13)
    got = oracle.routed_wgrad(G, x, ids, E, T + 31 * E)
    fx = oracle.bf16_to_f64(x)
    fg = oracle.bf16_to_f64(G)
    for e in range(E):
        toks = [t for t in range(T) if ids[t] == e]
        for n in range(N):
            for k in range(K):
                exact = sum((Fraction(float(fg[t, n])) * Fraction(float(fx[t, k])) for t in toks), Fraction(0))
                assert Fraction(float(got[e, n, k])) == exact, (e, n, k)


def test_routed_wgrad_on_grouped_input_is_the_grouped_wgrad():
    counts = [64, 0, 32]
    T, K, N = sum(counts), 64, 32
    ids = np.repeat(np.arange(3), counts)
    x = inp.random_bf16((T, K), seed=14, outliers=True)
    G = inp.random_bf16((T, N), seed=15, std=1e-3)
    got = oracle.routed_wgrad(G, x, ids, 3, T + 93)
    ref = oracle.grouped_mm_wgrad(G, x, inp.offsets_from_counts(counts))
    assert np.array_equal(got, ref)


def test_gather_rows_topk_takes_the_token_of_each_item():
    x = np.arange(12, dtype=np.uint16).reshape(4, 3)
    rows = np.array([5, -1, 0, 7, 8], dtype=np.int32)     # items of a top-2 router
    g = oracle.gather_rows(x, rows, topk=2)
    assert g.tolist() == [x[2].tolist(), [0, 0, 0], x[0].tolist(), x[3].tolist(), [0, 0, 0]]


# --------------------------------------------------------------------------
# Top-k routers: item a = token * k + slot
# --------------------------------------------------------------------------
def test_topk_sum_rows_rounds_once_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties go to the even 1.0;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    x = np.array([[1.0, 1.0], [2.0 ** -8, 3 * 2.0 ** -8], [3.0, -0.0], [1.0, 2.0]], dtype=np.float32)
    got = oracle.topk_sum_rows(x, 2)
    assert got.tolist() == [[0x3F80, 0x3F82], [0x4080, 0x4000]]
    # one slot: a plain fp32 -> bf16 rounding, +0 for -0 (the sum starts at +0)
    assert oracle.topk_sum_rows(np.array([[-0.0, 1.0 + 2.0 ** -7]], np.float32), 1).tolist() == [[0x0000, 0x3F81]]


def _topk_case(T, k, E, K, N, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=T * k)
    x = inp.random_bf16((T, K), seed=seed + 1, outliers=True)
    W = inp.random_bf16((E, N, K), seed=seed + 2, std=0.02)
    G = inp.random_bf16((T * k, N), seed=seed + 3, std=1e-3)
    return ids, x, W, G, T * k + 31 * E


def test_topk_routed_fwd_and_dgrad_equal_the_per_item_definition():
    T, k, E = 40, 3, 4
    ids, x, W, G, cap = _topk_case(T, k, E, 64, 32, seed=61)
    out = oracle.routed_fwd(x, ids, W, cap, topk=k)
    dx = oracle.routed_dgrad(G, ids, W, cap, topk=k)
    assert out.shape == (T * k, 32) and dx.shape == (T, 64)
    for t in range(T):
        qx, sx = oracle.quantize_rowwise(x[t:t + 1])
        want_dx = np.zeros(64)
        for j in range(k):
            a = t * k + j
            qw, sw = oracle.quantize_rowwise(W[ids[a]])
            np.testing.assert_allclose(out[a], (oracle.dequant_rowwise(qx, sx) @ oracle.dequant_rowwise(qw, sw).T)[0],
                                       rtol=1e-13, atol=1e-300)
            qg, sg = oracle.quantize_rowwise(G[a:a + 1])
            qwt, swt = oracle.quantize_colwise(W[ids[a]])
            want_dx += (oracle.dequant_rowwise(qg, sg) @ oracle.dequant_rowwise(qwt, swt).T)[0]
        np.testing.assert_allclose(dx[t], want_dx, rtol=1e-12, atol=1e-300)


def test_topk_routed_wgrad_lossless_equals_exact_item_sum():
    T, k, E, K, N = 30, 2, 3, 8, 4
    rng = np.random.default_rng(62)
    ids = rng.integers(0, E, size=T * k)
    x, G = _pow2((T, K), 63), _pow2((T * k, N), 64)
    got = oracle.routed_wgrad(G, x, ids, E, T * k + 31 * E, topk=k)
    fx, fg = oracle.bf16_to_f64(x), oracle.bf16_to_f64(G)
    for e in range(E):
        items = [a for a in range(T * k) if ids[a] == e]
        for n in range(N):
            for kk in range(K):
                exact = sum((Fraction(float(fg[a, n])) * Fraction(float(fx[a // k, kk])) for a in items), Fraction(0))
                assert Fraction(float(got[e, n, kk])) == exact, (e, n, kk)
