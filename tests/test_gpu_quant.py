"""GPU parity of the three MXFP8 quantizers: bit-exact E4M3 bytes and E8M0
scales against the CPU oracle, through the C ABI (Python binding)."""

import json
import os

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, u8_host, log

pytestmark = pytest.mark.gpu


def _gpu_quant(mode, x_bits):
    import mxfp8_block_scaled_06_amd as mx
    x = to_dev_bf16(x_bits)
    fn = {"rowwise": mx.mx_quantize_rowwise, "colwise": mx.mx_quantize_colwise, "32x32": mx.mx_quantize_32x32}[mode]
    q, s = fn(x)
    return u8_host(q), u8_host(s)


def _oracle(mode, x_bits):
    return {"rowwise": oracle.quantize_rowwise, "colwise": oracle.quantize_colwise,
            "32x32": oracle.quantize_32x32}[mode](x_bits)


def _assert_same(mode, x_bits, tag):
    q, s = _gpu_quant(mode, x_bits)
    rq, rs = _oracle(mode, x_bits)
    assert q.shape == rq.shape and s.shape == rs.shape, (q.shape, rq.shape, s.shape, rs.shape)
    bad_s = np.flatnonzero(s.ravel() != rs.ravel())
    bad_q = np.flatnonzero(q.ravel() != rq.ravel())
    assert bad_s.size == 0, f"{tag}: {bad_s.size} scale mismatches, first {bad_s[:5]} gpu {s.ravel()[bad_s[:5]]} ref {rs.ravel()[bad_s[:5]]}"
    assert bad_q.size == 0, f"{tag}: {bad_q.size} code mismatches, first {bad_q[:5]} gpu {q.ravel()[bad_q[:5]]} ref {rq.ravel()[bad_q[:5]]}"


MODES = ["rowwise", "colwise", "32x32"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape,seed,std", [
    ((96, 256), 1, 1.0),            # tiny workload's activation shape band
    ((3, 128, 96), 2, 0.02),        # batched (3D) like stacked expert weights
    ((256, 512), 3, 1e-3),          # gradient-like magnitudes
    ((160, 384), 4, 300.0),         # large magnitudes, saturation path
    ((32, 32), 5, 1.0),             # a single block / tile
    ((224, 200), 6, 1.0),           # ragged column count (not a tile multiple)
    ((2, 288, 512), 7, 0.02),       # batched, 256-column tiles with a partial last row tile
    ((3, 992, 768), 8, 1.0),        # 36 tiles of 256 x 256: tile chunks crossing batches and slot groups
    ((2, 512, 2048), 9, 1.0),       # 32 tiles, aligned rows: the plain tile order over batches
])
def test_quant_seeded(mode, shape, seed, std):
    require_gpu()
    if mode == "rowwise" and shape[-1] % 32:
        pytest.skip("rowwise needs cols % 32 == 0")
    if mode == "32x32" and shape[-1] % 32:
        pytest.skip("32x32 needs cols % 32 == 0")
    x = inp.random_bf16(shape, seed=seed, std=std, outliers=True)
    log(f"quant {mode} shape={shape} seed={seed}")
    _assert_same(mode, x, f"{mode} {shape}")


@pytest.mark.parametrize("mode", MODES)
def test_quant_all_bf16_patterns(mode):
    """Every bf16 bit pattern (NaN and Inf included) laid out as blocks, once in
    pattern order and once shuffled so blocks mix magnitudes."""
    require_gpu()
    pats = inp.all_bf16_patterns()
    rng = np.random.default_rng(9)
    for tag, arr in (("ordered", pats), ("shuffled", rng.permutation(pats))):
        x = arr.reshape(256, 256)
        log(f"quant {mode} all patterns {tag}")
        _assert_same(mode, x, f"{mode} all-patterns {tag}")
        # finite-only variant, so NaN blocks do not mask neighbours in 32x32 tiles
        fin = arr[(arr & 0x7FFF) < 0x7F80]
        fin = fin[: (fin.size // 8192) * 8192].reshape(-1, 256)
        _assert_same(mode, np.ascontiguousarray(fin), f"{mode} finite {tag}")


def _hand_blocks():
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")) as f:
        return json.load(f)["blocks"]


def _parse(s):
    s = s.strip()
    if s in ("nan", "inf", "-inf"):
        return float(s)
    if "^" in s:
        sign = -1.0 if s.startswith("-") else 1.0
        s = s.lstrip("-")
        mult = 1.0
        if "*" in s:
            m, s = s.split("*")
            mult = float(m)
        b, e = s.split("^")
        return sign * mult * float(b) ** int(e)
    return float(s)


@pytest.mark.parametrize("mode", MODES)
def test_quant_hand_worked_blocks(mode):
    """The hand-worked blocks of tests/golden, checked against their stated
    bytes directly (rowwise), as columns (colwise) and as 32x32 tiles whose
    other rows are zero (the tile amax is then the block's amax)."""
    require_gpu()
    for blk in _hand_blocks():
        vals = [_parse(v) for v in blk["values"]] + [_parse(blk["fill"])] * (32 - len(blk["values"]))
        bits = inp.f32_to_bf16_bits(np.array(vals, dtype=np.float32))
        codes = [int(c, 16) for c in blk["codes"]] + [int(blk["fill_code"], 16)] * (32 - len(blk["codes"]))
        scale = int(blk["scale"], 16)
        if mode == "rowwise":
            q, s = _gpu_quant(mode, bits.reshape(1, 32))
            assert int(s[0, 0]) == scale, blk["id"]
            assert [int(c) for c in q[0]] == codes, blk["id"]
        elif mode == "colwise":
            x = np.zeros((32, 8), dtype=np.uint16)
            x[:, 3] = bits
            q, s = _gpu_quant(mode, x)
            assert int(s[3, 0]) == scale, blk["id"]
            assert [int(c) for c in q[3]] == codes, blk["id"]
        else:
            x = np.zeros((32, 32), dtype=np.uint16)
            x[5] = bits
            q, s = _gpu_quant(mode, x)
            assert int(s[0, 0]) == scale, blk["id"]
            assert [int(c) for c in q[5]] == codes, blk["id"]


@pytest.mark.parametrize("mode", MODES)
def test_quant_special_blocks(mode):
    """Zeros, negative zeros, subnormal-only blocks, 448/464/465/480/510,
    +-Inf and NaN in otherwise ordinary tiles."""
    require_gpu()
    rng = np.random.default_rng(10)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    x[0:32, 0:32] = 0.0
    x[32:64, 0:32] = -0.0
    x[64:96, 0:32] = np.float32(2.0 ** -130) * rng.integers(-7, 8, (32, 32))
    x[96, 0:8] = [448, 464, 465, 480, 510, -464, -480, 1.0]
    x[0, 64] = np.inf
    x[40, 96] = -np.inf
    x[100, 100] = np.nan
    bits = inp.f32_to_bf16_bits(x)
    _assert_same(mode, bits, f"{mode} special")


def test_quant_empty_and_errors():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    q, s = mx.mx_quantize_rowwise(x)
    assert q.shape == (0, 64) and s.shape == (0, 2)
    with pytest.raises(mx.MXError, match="MX_ERR_SHAPE"):
        mx.mx_quantize_rowwise(torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises(mx.MXError, match="MX_ERR_SHAPE"):
        mx.mx_quantize_colwise(torch.zeros((48, 64), dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises(mx.MXError, match="MX_ERR_SHAPE"):
        mx.mx_quantize_32x32(torch.zeros((64, 48), dtype=torch.bfloat16, device="cuda:0"))


def test_quant_deterministic():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    x = to_dev_bf16(inp.random_bf16((512, 1024), seed=12, outliers=True))
    for fn in (mx.mx_quantize_rowwise, mx.mx_quantize_colwise, mx.mx_quantize_32x32):
        a = fn(x)
        b = fn(x)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Full sizes (the standalone quantize sweep [65600, 5120] and the stacked
# Llama4-shaped expert weights [16, 8192, 5120]) in the launch configuration
# the bench times, compared on sampled rows / columns / tiles.
# ---------------------------------------------------------------------------
def _sampled_compare(mode, x_bits, rng, n=48):
    import mxfp8_block_scaled_06_amd as mx
    squeeze = x_bits.ndim == 2
    x3 = x_bits[None] if squeeze else x_bits
    B, R, C = x3.shape
    xd = to_dev_bf16(x_bits)
    fn = {"rowwise": mx.mx_quantize_rowwise, "colwise": mx.mx_quantize_colwise, "32x32": mx.mx_quantize_32x32}[mode]
    q, s = fn(xd)
    q = u8_host(q).reshape((B,) + tuple(q.shape[-2:]))
    s = u8_host(s).reshape((B,) + tuple(s.shape[-2:]))
    del xd
    for _ in range(n):
        b = int(rng.integers(B))
        if mode == "rowwise":
            r = rng.integers(R, size=8)
            rq, rs = oracle.quantize_rowwise(x3[b, r])
            assert np.array_equal(q[b, r], rq)
            assert np.array_equal(s[b, r], rs)
        elif mode == "colwise":
            c = rng.integers(C, size=4)
            rq, rs = oracle.quantize_colwise(np.ascontiguousarray(x3[b][:, c]))
            assert np.array_equal(q[b, c], rq)
            assert np.array_equal(s[b, c], rs)
        else:
            rb = int(rng.integers(R // 32))
            cb = rng.integers(C // 32, size=4)
            for c1 in cb:
                tile = np.ascontiguousarray(x3[b, rb * 32:(rb + 1) * 32, c1 * 32:(c1 + 1) * 32])
                rq, rs = oracle.quantize_32x32(tile)
                assert np.array_equal(q[b, rb * 32:(rb + 1) * 32, c1 * 32:(c1 + 1) * 32], rq)
                assert int(s[b, rb, c1]) == int(rs[0, 0])


@pytest.mark.slow
@pytest.mark.parametrize("mode", MODES)
def test_quant_full_size_sweep(mode):
    require_gpu()
    x = inp.make_sweep()
    log(f"quant {mode} full-size sweep {x.shape}")
    _sampled_compare(mode, x, np.random.default_rng(20))


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["rowwise", "colwise"])
def test_quant_full_size_expert_weights(mode):
    require_gpu()
    rng = np.random.default_rng(inp.WORKLOADS["llama4_fwd"].seed)
    W = inp.make_weights(rng, 16, 8192, 5120)
    log(f"quant {mode} full-size stacked weights {W.shape}")
    _sampled_compare(mode, W, np.random.default_rng(21), n=24)
