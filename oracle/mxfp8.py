"""CPU oracle for MXFP8 quantization and the block-scaled grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
bench's CPU-baseline leg may import this module.  The HIP library never calls
it, and it shares no code, table or constant generator with the HIP path.

What is computed, and where it is defined:

* MXFP8 format -- "MXFP8 (Micro-scaling FP8)" page, section "Definition":
  a shared power-of-two scale is applied to a small block of values.  Blocks
  are 32 elements along the contraction dimension, the shared scale is an
  E8M0 byte and the elements are FP8 E4M3 (OCP conventions: bias 7, largest
  finite 448, code 0x7F is NaN, subnormals on a 2^-9 grid).
* Scales are generated along each GEMM's K dimension -- same page, section
  "Low-precision Flash Attention (MXFP8 on FA4)"; 32x32 square blocks with one
  scale per tile make the quantization transpose-invariant (item 3 there).
* Dynamic quantization of activations and weights followed by a scaled grouped
  GEMM with original-precision output, forward and backward ("Backprop
  mirrors it") -- "MXFP8 training for MoEs" article, sections "Is MXFP8
  Training for MoEs Actually Stable?" and "Why Does MXFP8 Speed Up MoE
  Training So Much?".
* The backward consumes a transposed weight quantization (weight_t_fp8,
  weight_t_scale beside weight_fp8, weight_scale) -- "feat(moe): add MoK MXFP8
  expert support" PR, review comment on the mxfp8_weights argument; the 3D
  colwise quantize kernel in the pytorch/ao PR timeline.

Readings where the pages are silent (each listed in the design notes):
  R-scale   scale exponent = floor(log2 amax) - 8 (8 = E4M3's largest
            exponent), clamped to [-127, 127], byte = exponent + 127;
  R-zero    an all-zero block gets byte 0x00;
  R-nan     a block holding NaN or Inf gets byte 0xFF and elements 0x7F;
  R-sat     |scaled value| > 448 saturates to +-448 (0x7E / 0xFE);
  R-sign    the sign bit is kept for -0.0 and for negative values that round
            to zero (0x80);
  R-sub     E4M3 subnormals are kept (round-to-nearest-even on 2^-9 grid);
  R-offs    group offsets are int32 cumulative END offsets;
  R-layout  W is [E, N, K]; forward contracts over K (out = A @ W[e]^T);
            dgrad uses W quantized in 32-blocks along N, stored [E, K, N];
            wgrad quantizes dOut and A in 32-blocks along tokens, groups
            padded to multiples of 32;
  R-empty   an expert with no tokens gets an all-zero weight gradient.

Everything here is fp64 / integer numpy; matmul is numpy's.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0          # largest finite E4M3 value, 1.75 * 2^8
E4M3_EMAX = 8             # exponent of E4M3's largest binade
E4M3_NAN = 0x7F
E8M0_NAN = 0xFF
BLOCK = 32


# --------------------------------------------------------------------------
# Element codecs
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (sign, 8-bit exponent, 7-bit fraction)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of E4M3 codes: sign | 4-bit exponent (bias 7) | 3-bit mantissa.

    Exponent field 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ef - 7.0))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even cast of finite values to E4M3 codes.

    Steps: sign from the sign bit; |y| > 448 saturates to 448; below 2^-6 the
    value is rounded on the subnormal grid 2^-9; otherwise the exponent is
    floor(log2 |y|) and the 3-bit mantissa is rounded to nearest even, a carry
    into the next binade bumping the exponent.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    code = np.zeros(a.shape, dtype=np.int64)

    sat = a > E4M3_MAX
    code[sat] = 0x7E

    sub = (~sat) & (a < 2.0 ** -6)
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)      # 0..8; 8 == 2^-6

    nrm = (~sat) & (~sub)
    if nrm.any():
        an = a[nrm]
        _, p = np.frexp(an)                   # an = f * 2^p, f in [0.5, 1)
        x = p.astype(np.int64) - 1            # floor(log2 an)
        m = np.rint((an / np.exp2(x.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
        carry = m == 8
        x = np.where(carry, x + 1, x)
        m = np.where(carry, 0, m)
        code[nrm] = ((x + 7) << 3) | m
    return (code | sign).astype(np.uint8)


def e8m0_from_amax(amax: np.ndarray, nonfinite: np.ndarray) -> np.ndarray:
    """Shared-scale byte of a block from its largest magnitude (reading R-scale).

    byte = clamp(floor(log2 amax) - 8, -127, 127) + 127; 0x00 for amax == 0;
    0xFF when the block holds a NaN or an Inf.
    """
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape, dtype=np.int64)
    pos = (amax > 0) & ~nonfinite
    if pos.any():
        _, p = np.frexp(amax[pos])
        e = p.astype(np.int64) - 1
        out[pos] = np.clip(e - E4M3_EMAX, -127, 127) + 127
    out[nonfinite] = E8M0_NAN
    return out.astype(np.uint8)


def e8m0_value(byte: np.ndarray) -> np.ndarray:
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == E8M0_NAN, np.nan, np.exp2(b.astype(np.float64) - 127.0))


# --------------------------------------------------------------------------
# Block quantizer on values already grouped into blocks
# --------------------------------------------------------------------------
def quantize_blocks(v: np.ndarray):
    """Quantize fp64 values shaped [..., nblocks, blocksize] (one scale per row
    of the last axis).  Returns (codes uint8 same shape, scale bytes [..., nblocks]).
    """
    nonfinite = ~np.isfinite(v).all(axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(v), v, 0.0)), axis=-1)
    s = e8m0_from_amax(amax, nonfinite)
    mult = np.exp2(127.0 - np.where(nonfinite, 127, s).astype(np.float64))
    y = v * mult[..., None]
    q = e4m3_encode(np.where(np.isfinite(y), y, 0.0))
    q[np.broadcast_to(nonfinite[..., None], q.shape)] = E4M3_NAN
    return q, s


# --------------------------------------------------------------------------
# The three quantization modes (inputs are bf16 bit patterns)
# --------------------------------------------------------------------------
def _as3d(x):
    x = np.asarray(x)
    return x if x.ndim == 3 else x[None]


def quantize_rowwise(x_bits: np.ndarray):
    """1x32 blocks along the last (contraction) axis.

    x [B,R,C] or [R,C] -> q same shape, s [..., R, C/32].
    """
    squeeze = np.asarray(x_bits).ndim == 2
    v = bf16_to_f64(_as3d(x_bits))
    B, R, C = v.shape
    assert C % BLOCK == 0
    q, s = quantize_blocks(v.reshape(B, R, C // BLOCK, BLOCK))
    q = q.reshape(B, R, C)
    return (q[0], s[0]) if squeeze else (q, s)


def quantize_colwise(x_bits: np.ndarray):
    """32x1 blocks along rows; output stored transposed so the block axis is
    contiguous.  x [B,R,C] -> q_t [B,C,R], s_t [B,C,R/32].
    """
    squeeze = np.asarray(x_bits).ndim == 2
    v = bf16_to_f64(_as3d(x_bits))
    B, R, C = v.shape
    assert R % BLOCK == 0
    blocks = v.reshape(B, R // BLOCK, BLOCK, C)                 # [B, rb, 32, C]
    blocks = np.moveaxis(blocks, 2, 3)                          # [B, rb, C, 32]
    q, s = quantize_blocks(blocks)                              # q [B,rb,C,32], s [B,rb,C]
    q_t = np.moveaxis(q, 2, 1).reshape(B, C, R)                 # [B, C, rb*32]
    s_t = np.moveaxis(s, 2, 1)                                  # [B, C, rb]
    s_t = np.ascontiguousarray(s_t)
    return (q_t[0], s_t[0]) if squeeze else (q_t, s_t)


def quantize_32x32(x_bits: np.ndarray):
    """One scale per 32x32 tile; elements stay in place.
    x [B,R,C] -> q [B,R,C], s [B,R/32,C/32].
    """
    squeeze = np.asarray(x_bits).ndim == 2
    v = bf16_to_f64(_as3d(x_bits))
    B, R, C = v.shape
    assert R % BLOCK == 0 and C % BLOCK == 0
    t = v.reshape(B, R // BLOCK, BLOCK, C // BLOCK, BLOCK)      # b, rb, i, cb, j
    t = t.transpose(0, 1, 3, 2, 4).reshape(B, R // BLOCK, C // BLOCK, BLOCK * BLOCK)
    q, s = quantize_blocks(t)
    q = q.reshape(B, R // BLOCK, C // BLOCK, BLOCK, BLOCK).transpose(0, 1, 3, 2, 4).reshape(B, R, C)
    return (q[0], s[0]) if squeeze else (q, s)


# --------------------------------------------------------------------------
# Dequantization
# --------------------------------------------------------------------------
def dequant_rowwise(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Value of rowwise-quantized data: decode(q) * 2^(s-127), block along last axis."""
    val = e4m3_decode(q)
    scale = e8m0_value(s)
    return val * np.repeat(scale, BLOCK, axis=-1)


def dequant_32x32(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    val = e4m3_decode(q)
    scale = e8m0_value(s)
    return val * np.repeat(np.repeat(scale, BLOCK, axis=-1), BLOCK, axis=-2)


# --------------------------------------------------------------------------
# Grouped GEMMs (fp64 on dequantized operands)
# --------------------------------------------------------------------------
def group_bounds(offs: np.ndarray, M: int):
    """[(start, end)] per expert from cumulative END offsets (reading R-offs)."""
    offs = np.asarray(offs, dtype=np.int64)
    starts = np.concatenate([[0], offs[:-1]])
    return [(int(a), int(b)) for a, b in zip(starts, offs)]


def grouped_gemm_mx(X, sX, Y, sY, offs, mode: int, absolute: bool = False) -> np.ndarray:
    """The GEMM on prequantized operands, in fp64.

    C[i, j] = sum_k deq(X)[i, k] * deq(Y)[j, k], blocks of 32 along k.
    mode 0: groups over the rows i of X; Y is [E, J, Kc]; C is [I, J].
    mode 1: groups over the contraction k; X is [I, Kc], Y is [J, Kc]; C is [E, I, J].
    absolute=True sums |deq(X)| |deq(Y)| instead (the error-bound companion).
    """
    f = np.abs if absolute else (lambda v: v)
    dX = f(dequant_rowwise(X, sX))
    if mode == 0:
        I = dX.shape[0]
        J = Y.shape[1]
        C = np.zeros((I, J), dtype=np.float64)
        for e, (a, b) in enumerate(group_bounds(offs, I)):
            if b > a:
                C[a:b] = dX[a:b] @ f(dequant_rowwise(Y[e], sY[e])).T
        return C
    if mode == 1:
        dY = f(dequant_rowwise(Y, sY))
        E = len(offs)
        C = np.zeros((E, dX.shape[0], dY.shape[0]), dtype=np.float64)
        for e, (a, b) in enumerate(group_bounds(offs, dX.shape[1])):
            if b > a:
                C[e] = dX[:, a:b] @ dY[:, a:b].T
        return C
    raise ValueError(mode)


def grouped_mm_fwd(A_bits, W_bits, offs, absolute: bool = False) -> np.ndarray:
    """out[g_e] = MX(A)[g_e] @ MX(W[e])^T; A rowwise along K, W rowwise along K.
    absolute=True gives sum_k |a_k w_k| instead (error-bound companion)."""
    f = np.abs if absolute else (lambda v: v)
    qA, sA = quantize_rowwise(A_bits)
    M = qA.shape[0]
    N = W_bits.shape[1]
    out = np.zeros((M, N), dtype=np.float64)
    dA = f(dequant_rowwise(qA, sA))
    for e, (a, b) in enumerate(group_bounds(offs, M)):
        if b > a:
            qW, sW = quantize_rowwise(W_bits[e])
            out[a:b] = dA[a:b] @ f(dequant_rowwise(qW, sW)).T
    return out


def grouped_mm_dgrad(dOut_bits, W_bits, offs, absolute: bool = False) -> np.ndarray:
    """dA[g_e] = MX(dOut)[g_e] @ MX_t(W[e]); dOut rowwise along N, W blocked
    along N (stored [K, N]), contraction over N."""
    f = np.abs if absolute else (lambda v: v)
    qG, sG = quantize_rowwise(dOut_bits)
    M = qG.shape[0]
    K = W_bits.shape[2]
    dG = f(dequant_rowwise(qG, sG))
    out = np.zeros((M, K), dtype=np.float64)
    for e, (a, b) in enumerate(group_bounds(offs, M)):
        if b > a:
            qWt, sWt = quantize_colwise(W_bits[e])              # [K, N], [K, N/32]
            out[a:b] = dG[a:b] @ f(dequant_rowwise(qWt, sWt)).T
    return out


def grouped_mm_wgrad(dOut_bits, A_bits, offs, absolute: bool = False) -> np.ndarray:
    """dW[e] = MX_t(dOut)[:, g_e] @ MX_t(A)[:, g_e]^T with both operands blocked
    along tokens; an expert with no tokens gets zeros (reading R-empty)."""
    f = np.abs if absolute else (lambda v: v)
    qGt, sGt = quantize_colwise(dOut_bits)                      # [N, M]
    qAt, sAt = quantize_colwise(A_bits)                         # [K, M]
    dGt = f(dequant_rowwise(qGt, sGt))
    dAt = f(dequant_rowwise(qAt, sAt))
    E = len(offs)
    out = np.zeros((E, dGt.shape[0], dAt.shape[0]), dtype=np.float64)
    for e, (a, b) in enumerate(group_bounds(offs, dGt.shape[1])):
        if b > a:
            out[e] = dGt[:, a:b] @ dAt[:, a:b].T
    return out
