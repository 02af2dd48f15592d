"""MXFP8 quantization + block-scaled grouped GEMM for MoE routed experts (gfx950).

Thin Python binding of the C ABI in include/mxmoe.h.  Every function
marshals torch tensors (device memory and the current stream) into the C
call; all arithmetic runs in the HIP kernels of libmxmoe.so.  If the library
has not been built, every entry point raises: there is no CPU fallback.

Build:  python -m mxfp8_block_scaled_06_amd.build
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "MXError", "library_path", "load_library", "version",
    "mx_quantize_rowwise", "mx_quantize_colwise", "mx_quantize_32x32",
    "mx_grouped_gemm_mx", "mx_grouped_gemm_mx_f32", "mx_grouped_mm_workspace_bytes", "mx_scales_to_gemm_layout",
    "mx_grouped_mm_fwd", "mx_grouped_mm_dgrad", "mx_grouped_mm_wgrad",
    "mx_quantize_weights", "mx_quantize_dual", "mx_quantize_rowwise_gather",
    "mx_grouped_mm_fwd_q", "mx_grouped_mm_dgrad_q", "mx_grouped_mm", "mx_linear",
    "OP_FWD", "OP_DGRAD", "OP_WGRAD", "OP_FWD_Q", "OP_DGRAD_Q", "SCALES_ROWMAJOR", "SCALES_GEMM",
    "mx_check_offsets", "check_offsets", "mx_grouped_mm_fwd_q_noalloc", "NOALLOC_SCRATCH_BYTES",
    "mx_route", "route_capacity", "mx_quantize_dual_gather", "mx_grouped_gemm_mx_rows", "mx_routed_experts",
    "mx_topk_sum_rows", "mx_route_workspace_bytes",
]

OP_FWD, OP_DGRAD, OP_WGRAD, OP_FWD_Q, OP_DGRAD_Q = 0, 1, 2, 3, 4
SCALES_ROWMAJOR, SCALES_GEMM = 0, 1
OFFS_DECREASING, OFFS_RANGE, OFFS_LAST, OFFS_ALIGN = 1, 2, 4, 8
NOALLOC_SCRATCH_BYTES = 128 << 20     # MX_NOALLOC_SCRATCH_BYTES of include/mxmoe.h
_STATUS = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN", 4: "MX_ERR_WORKSPACE",
           5: "MX_ERR_HIP", 6: "MX_ERR_LAYOUT"}

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


class MXError(RuntimeError):
    """A C-ABI call returned a status other than MX_OK."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {text}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libmxmoe.so")


def load_library():
    """Load libmxmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mxfp8_block_scaled_06_amd.build`")
    lib = ctypes.CDLL(path)
    c_i64, c_vp, c_int, c_sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mx_last_error.restype = ctypes.c_char_p
    lib.mx_version.restype = ctypes.c_char_p
    for name in ("mx_quantize_rowwise", "mx_quantize_colwise", "mx_quantize_32x32"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]
    for name in ("mx_grouped_gemm_mx", "mx_grouped_gemm_mx_f32"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_vp, c_int, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp]
    lib.mx_grouped_gemm_mx_ordered.restype = c_int
    lib.mx_grouped_gemm_mx_ordered.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_vp, c_int, c_i64, c_i64, c_i64, c_i64,
                                               c_vp, ctypes.c_uint64, c_vp]
    lib.mx_grouped_gemm_mx_rows.restype = c_int
    lib.mx_grouped_gemm_mx_rows.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp,
                                            c_vp, c_i64, c_vp]
    lib.mx_grouped_gemm_mx_rows_f32.restype = c_int
    lib.mx_grouped_gemm_mx_rows_f32.argtypes = lib.mx_grouped_gemm_mx_rows.argtypes
    lib.mx_topk_sum_rows.restype = c_int
    lib.mx_topk_sum_rows.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]
    lib.mx_route.restype = c_int
    lib.mx_route.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.mx_route_workspace_bytes.restype = c_sz
    lib.mx_route_workspace_bytes.argtypes = [c_i64, c_i64]
    lib.mx_quantize_dual_gather.restype = c_int
    lib.mx_quantize_dual_gather.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                            c_vp]
    lib.mx_check_offsets.restype = c_int
    lib.mx_check_offsets.argtypes = [c_vp, c_i64, c_i64, ctypes.c_int32, c_vp, c_vp]
    lib.mx_scales_to_gemm_layout.restype = c_int
    lib.mx_scales_to_gemm_layout.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]
    lib.mx_grouped_mm_workspace_bytes.restype = c_sz
    lib.mx_grouped_mm_workspace_bytes.argtypes = [c_int, c_i64, c_i64, c_i64, c_i64]
    for name in ("mx_grouped_mm_fwd", "mx_grouped_mm_dgrad", "mx_grouped_mm_wgrad"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]
    lib.mx_quantize_rowwise_gather.restype = c_int
    lib.mx_quantize_rowwise_gather.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]
    lib.mx_quantize_weights.restype = c_int
    lib.mx_quantize_weights.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.mx_quantize_dual.restype = c_int
    lib.mx_quantize_dual.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]
    for name in ("mx_grouped_mm_fwd_q", "mx_grouped_mm_dgrad_q"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]
    lib.mx_grouped_mm_fwd_q_noalloc.restype = c_int
    lib.mx_grouped_mm_fwd_q_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp]
    _lib = lib
    return lib


def version() -> str:
    return load_library().mx_version().decode()


def _check(fn: str, status: int):
    if status != 0:
        raise MXError(fn, status, load_library().mx_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _require(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, shape, dtype, device, name):
    """An output buffer: allocated when None, else checked to be exactly what
    the kernel writes (the C ABI sees only a pointer and cannot)."""
    import torch
    shape = tuple(int(d) for d in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if isinstance(t, torch.Tensor) and tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    _require(t, dtype, name)
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _as3d(x):
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x.shape[0], x.shape[1], x.shape[2]
    raise ValueError("expected a 2-D or 3-D tensor")


# ---------------------------------------------------------------------------
# Quantizers
# ---------------------------------------------------------------------------
def mx_quantize_rowwise(x, q=None, s=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """1x32 blocks along the last axis.  x bf16 [..., R, C] -> (q uint8 same shape, s uint8 [..., R, C/32])."""
    import torch
    lib = load_library()
    _require(x, torch.bfloat16, "x")
    B, R, C = _as3d(x)
    lead = x.shape[:-1]
    q = _out(q, x.shape, torch.uint8, x.device, "q")
    s = _out(s, (*lead, C // 32 if C % 32 == 0 else 0), torch.uint8, x.device, "s")
    _check("mx_quantize_rowwise", lib.mx_quantize_rowwise(_ptr(x), B, R, C, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def mx_quantize_colwise(x, q_t=None, s_t=None):
    """32x1 blocks along rows, output transposed.  x bf16 [B?, R, C] ->
    (q_t uint8 [B?, C, R], s_t uint8 [B?, C, R/32])."""
    import torch
    lib = load_library()
    _require(x, torch.bfloat16, "x")
    B, R, C = _as3d(x)
    lead = x.shape[:-2]
    q_t = _out(q_t, (*lead, C, R), torch.uint8, x.device, "q_t")
    s_t = _out(s_t, (*lead, C, R // 32 if R % 32 == 0 else 0), torch.uint8, x.device, "s_t")
    _check("mx_quantize_colwise",
           lib.mx_quantize_colwise(_ptr(x), B, R, C, _ptr(q_t), _ptr(s_t), _stream(x.device)))
    return q_t, s_t


def mx_quantize_32x32(x, q=None, s=None):
    """32x32 blocks.  x bf16 [B?, R, C] -> (q uint8 same shape, s uint8 [B?, R/32, C/32])."""
    import torch
    lib = load_library()
    _require(x, torch.bfloat16, "x")
    B, R, C = _as3d(x)
    lead = x.shape[:-2]
    q = _out(q, x.shape, torch.uint8, x.device, "q")
    s = _out(s, (*lead, R // 32, C // 32), torch.uint8, x.device, "s")
    _check("mx_quantize_32x32", lib.mx_quantize_32x32(_ptr(x), B, R, C, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def mx_scales_to_gemm_layout(s, out=None):
    """Row-major scales [B?, R, KB] -> the GEMM's blocked layout [B?, KB/4, R, 4]."""
    import torch
    lib = load_library()
    _require(s, torch.uint8, "s")
    B, R, KB = _as3d(s)
    out = _out(out, (*s.shape[:-2], KB // 4, R, 4), torch.uint8, s.device, "out")
    _check("mx_scales_to_gemm_layout",
           lib.mx_scales_to_gemm_layout(_ptr(s), B, R, KB, _ptr(out), _stream(s.device)))
    return out


# ---------------------------------------------------------------------------
# Grouped GEMM on prequantized operands
# ---------------------------------------------------------------------------
def mx_grouped_gemm_mx(X, sX, Y, sY, offs, mode: int, out=None, out_dtype=None, scale_layout: str = "gemm"):
    """C[i,j] = sum_k X[i,k] Y[j,k] 2^(sX+sY-254).  mode 0: Y [E,J,Kc], C [I,J];
    mode 1 (groups over k): Y [J,Kc], C [E,I,J].  The scales must be in the
    GEMM's blocked layout (what mx_quantize_weights / mx_quantize_dual write,
    or mx_scales_to_gemm_layout of a quantizer's row-major scales):
    sX [Kc/128, I, 4]; sY [E, Kc/128, J, 4] in mode 0, [Kc/128, J, 4] in mode 1.
    Row-major scales raise (their shapes differ).  Returns C (bf16, or fp32
    with out_dtype=torch.float32)."""
    import torch
    lib = load_library()
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    I, J, Kc, E, layout = _gemm_operands(X, sX, Y, sY, offs, mode, scale_layout)
    out = _out(out, (I, J) if mode == 0 else (E, I, J), out_dtype, X.device, "out")
    name = "mx_grouped_gemm_mx" if out_dtype == torch.bfloat16 else "mx_grouped_gemm_mx_f32"
    _check(name, getattr(lib, name)(_ptr(X), _ptr(sX), _ptr(Y), _ptr(sY), layout, _ptr(offs), mode, I, J, Kc, E,
                                    _ptr(out), _stream(X.device)))
    return out


def _gemm_operands(X, sX, Y, sY, offs, mode, scale_layout):
    """Shape checks of the GEMM operands; returns (I, J, Kc, E, layout code)."""
    import torch
    if scale_layout not in ("gemm", "rowmajor"):
        raise ValueError("scale_layout must be 'gemm' or 'rowmajor'")
    for t, n in ((X, "X"), (sX, "sX"), (Y, "Y"), (sY, "sY")):
        _require(t, torch.uint8, n)
    _require(offs, torch.int32, "offs")
    E = offs.shape[0]
    if X.dim() != 2:
        raise ValueError("X must be [I, Kc]")
    I, Kc = X.shape
    if mode == 0:
        if Y.dim() != 3 or Y.shape[0] != E or Y.shape[2] != Kc:
            raise ValueError(f"mode 0: Y must be [E={E}, J, Kc={Kc}], got {tuple(Y.shape)}")
        J = Y.shape[1]
    else:
        if Y.dim() != 2 or Y.shape[1] != Kc:
            raise ValueError(f"mode 1: Y must be [J, Kc={Kc}], got {tuple(Y.shape)}")
        J = Y.shape[0]
    if scale_layout == "gemm":
        want_x = (Kc // 128, I, 4)
        want_y = (E, Kc // 128, J, 4) if mode == 0 else (Kc // 128, J, 4)
        for t, want, n in ((sX, want_x, "sX"), (sY, want_y, "sY")):
            if tuple(t.shape) != want:
                hint = (" (these are row-major scales: convert them with mx_scales_to_gemm_layout)"
                        if t.dim() == len(want) - 1 and t.shape[-1] == Kc // 32 else "")
                raise ValueError(f"{n} must be in the GEMM scale layout {want}, got {tuple(t.shape)}{hint}")
    return I, J, Kc, E, SCALES_GEMM if scale_layout == "gemm" else SCALES_ROWMAJOR


def mx_grouped_gemm_mx_rows(X, sX, Y, sY, offs, row_map, c_rows: Optional[int] = None, out=None,
                            out_dtype=None):
    """mx_grouped_gemm_mx (mode 0) storing grouped row i to out row
    row_map[i] (rows whose entry lies outside [0, c_rows) are dropped; out
    rows no entry names are left as they were).  row_map int32 [I] on the GPU
    (the `rows` of mx_route); out bf16 (or fp32 with out_dtype=torch.float32)
    [c_rows, J] (default c_rows: out's rows, else I; a new out starts at
    zero)."""
    import torch
    lib = load_library()
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    I, J, Kc, E, layout = _gemm_operands(X, sX, Y, sY, offs, 0, "gemm")
    _require(row_map, torch.int32, "row_map")
    if tuple(row_map.shape) != (I,):
        raise ValueError(f"row_map must be int32 [{I}] (one entry per row of X), got {tuple(row_map.shape)}")
    if c_rows is None:
        c_rows = out.shape[0] if out is not None else I
    if out is None:
        out = torch.zeros((c_rows, J), dtype=out_dtype, device=X.device)
    out = _out(out, (c_rows, J), out_dtype, X.device, "out")
    name = "mx_grouped_gemm_mx_rows" if out_dtype == torch.bfloat16 else "mx_grouped_gemm_mx_rows_f32"
    _check(name, getattr(lib, name)(_ptr(X), _ptr(sX), _ptr(Y), _ptr(sY), layout, _ptr(offs), I, J, Kc, E,
                                    _ptr(row_map), _ptr(out), int(c_rows), _stream(X.device)))
    return out


def mx_topk_sum_rows(x, k: int, out=None):
    """x fp32 [T*k, cols] -> bf16 [T, cols]: each token's k rows summed in fp32
    in slot order, rounded to nearest even once (the top-k gather's gradient)."""
    import torch
    lib = load_library()
    _require(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[0] % k:
        raise ValueError(f"x must be [T*k, cols] with k={k}, got {tuple(x.shape)}")
    T, cols = x.shape[0] // k, x.shape[1]
    out = _out(out, (T, cols), torch.bfloat16, x.device, "out")
    _check("mx_topk_sum_rows", lib.mx_topk_sum_rows(_ptr(x), T, int(k), cols, _ptr(out), _stream(x.device)))
    return out


def mx_grouped_gemm_mx_ordered(X, sX, Y, sY, offs, mode: int, order_seed: int, out=None):
    """mx_grouped_gemm_mx (bf16) with workgroups dealt to tiles in a seeded
    pseudo-random order (race checks: the result must not depend on it)."""
    import torch
    lib = load_library()
    I, J, Kc, E, layout = _gemm_operands(X, sX, Y, sY, offs, mode, "gemm")
    out = _out(out, (I, J) if mode == 0 else (E, I, J), torch.bfloat16, X.device, "out")
    _check("mx_grouped_gemm_mx_ordered",
           lib.mx_grouped_gemm_mx_ordered(_ptr(X), _ptr(sX), _ptr(Y), _ptr(sY), layout, _ptr(offs), mode, I, J, Kc, E,
                                          _ptr(out), int(order_seed), _stream(X.device)))
    return out


def mx_grouped_gemm_mx_f32(X, sX, Y, sY, offs, mode: int, out=None):
    """mx_grouped_gemm_mx with fp32 output (accumulators stored unrounded)."""
    import torch
    return mx_grouped_gemm_mx(X, sX, Y, sY, offs, mode, out=out, out_dtype=torch.float32)


def mx_grouped_mm_workspace_bytes(op: int, M: int, N: int, K: int, E: int) -> int:
    return int(load_library().mx_grouped_mm_workspace_bytes(op, M, N, K, E))


def _offs(offs, E):
    """offs: int32 [E] group END offsets on the GPU (the kernels read E entries)."""
    import torch
    if isinstance(offs, torch.Tensor) and (offs.dim() != 1 or offs.shape[0] != E):
        raise ValueError(f"offs must be int32 [{E}] (one END offset per expert), got {tuple(offs.shape)}")
    _require(offs, torch.int32, "offs")


def _ws(op, M, N, K, E, device, ws):
    import torch
    need = mx_grouped_mm_workspace_bytes(op, M, N, K, E)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws


# ---------------------------------------------------------------------------
# Grouped GEMMs on bf16 inputs (quantize both operands, then GEMM)
# ---------------------------------------------------------------------------
def mx_grouped_mm_fwd(A, W, offs, out=None, ws=None):
    """out [M, N] = A [M, K] @ W[e] [N, K]^T per expert group (offs: int32 END offsets)."""
    import torch
    lib = load_library()
    _require(A, torch.bfloat16, "A")
    _require(W, torch.bfloat16, "W")
    _require(offs, torch.int32, "offs")
    M, K = A.shape
    E, N, K2 = W.shape
    if K2 != K:
        raise ValueError(f"A has K={K} but W has K={K2}")
    _offs(offs, E)
    out = _out(out, (M, N), torch.bfloat16, A.device, "out")
    ws = _ws(OP_FWD, M, N, K, E, A.device, ws)
    _check("mx_grouped_mm_fwd",
           lib.mx_grouped_mm_fwd(_ptr(A), _ptr(W), _ptr(offs), M, N, K, E, _ptr(out), _ptr(ws), ws.numel(),
                                 _stream(A.device)))
    return out


def mx_grouped_mm_dgrad(dOut, W, offs, out=None, ws=None):
    """dA [M, K] = dOut [M, N] @ W[e] [N, K] per expert group."""
    import torch
    lib = load_library()
    _require(dOut, torch.bfloat16, "dOut")
    _require(W, torch.bfloat16, "W")
    _require(offs, torch.int32, "offs")
    M, N = dOut.shape
    E, N2, K = W.shape
    if N2 != N:
        raise ValueError(f"dOut has N={N} but W has N={N2}")
    _offs(offs, E)
    out = _out(out, (M, K), torch.bfloat16, dOut.device, "out")
    ws = _ws(OP_DGRAD, M, N, K, E, dOut.device, ws)
    _check("mx_grouped_mm_dgrad",
           lib.mx_grouped_mm_dgrad(_ptr(dOut), _ptr(W), _ptr(offs), M, N, K, E, _ptr(out), _ptr(ws), ws.numel(),
                                   _stream(dOut.device)))
    return out


def mx_grouped_mm_wgrad(dOut, A, offs, out=None, ws=None):
    """dW [E, N, K], dW[e] = dOut[g_e]^T @ A[g_e] (groups padded to multiples of 32)."""
    import torch
    lib = load_library()
    _require(dOut, torch.bfloat16, "dOut")
    _require(A, torch.bfloat16, "A")
    _require(offs, torch.int32, "offs")
    M, N = dOut.shape
    M2, K = A.shape
    if M2 != M:
        raise ValueError(f"dOut has M={M} but A has M={M2}")
    E = offs.shape[0]
    out = _out(out, (E, N, K), torch.bfloat16, A.device, "out")
    ws = _ws(OP_WGRAD, M, N, K, E, A.device, ws)
    _check("mx_grouped_mm_wgrad",
           lib.mx_grouped_mm_wgrad(_ptr(dOut), _ptr(A), _ptr(offs), M, N, K, E, _ptr(out), _ptr(ws), ws.numel(),
                                   _stream(A.device)))
    return out


# ---------------------------------------------------------------------------
# Prequantized expert weights (both orientations in one pass)
# ---------------------------------------------------------------------------
def mx_quantize_weights(W, q=None, s=None, q_t=None, s_t=None):
    """W bf16 [E, N, K] -> (q [E, N, K], s [E, K/128, N, 4], q_t [E, K, N], s_t [E, N/128, K, 4]):
    rowwise codes along K and colwise codes along N (stored transposed), scales
    in the GEMM layout.  N and K must be multiples of 128."""
    import torch
    lib = load_library()
    _require(W, torch.bfloat16, "W")
    if W.dim() != 3:
        raise ValueError("W must be [E, N, K]")
    E, N, K = W.shape
    dev = W.device
    q = _out(q, (E, N, K), torch.uint8, dev, "q")
    s = _out(s, (E, K // 128, N, 4), torch.uint8, dev, "s")
    q_t = _out(q_t, (E, K, N), torch.uint8, dev, "q_t")
    s_t = _out(s_t, (E, N // 128, K, 4), torch.uint8, dev, "s_t")
    _check("mx_quantize_weights", lib.mx_quantize_weights(_ptr(W), E, N, K, _ptr(q), _ptr(s), _ptr(q_t), _ptr(s_t),
                                                          _stream(dev)))
    return q, s, q_t, s_t


def mx_quantize_dual(x, ldq: Optional[int] = None, q=None, s=None, q_t=None, s_t=None):
    """Activations x bf16 [rows, cols] in both orientations from one read:
    (q [rows, cols], s [cols/128, rows, 4]) = X of the rows-grouped GEMM, and
    (q_t [cols, ldq], s_t [ldq/128, cols, 4]) = a wgrad operand with Kc = ldq
    (default: rows rounded up to 128; the padding columns are zero codes)."""
    import torch
    lib = load_library()
    _require(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = x.shape
    if ldq is None:
        ldq = (rows + 127) // 128 * 128
    dev = x.device
    q = _out(q, (rows, cols), torch.uint8, dev, "q")
    s = _out(s, (cols // 128, rows, 4), torch.uint8, dev, "s")
    q_t = _out(q_t, (cols, ldq), torch.uint8, dev, "q_t")
    s_t = _out(s_t, (ldq // 128, cols, 4), torch.uint8, dev, "s_t")
    _check("mx_quantize_dual", lib.mx_quantize_dual(_ptr(x), rows, cols, ldq, _ptr(q), _ptr(s), _ptr(q_t), _ptr(s_t),
                                                    _stream(dev)))
    return q, s, q_t, s_t


def mx_grouped_mm_fwd_q(A, qW, sW, offs, out=None, ws=None):
    """mx_grouped_mm_fwd with W given as (q, s) of mx_quantize_weights."""
    import torch
    lib = load_library()
    _require(A, torch.bfloat16, "A")
    _require(qW, torch.uint8, "qW")
    _require(sW, torch.uint8, "sW")
    _require(offs, torch.int32, "offs")
    M, K = A.shape
    E, N, K2 = qW.shape
    if K2 != K:
        raise ValueError(f"A has K={K} but qW has K={K2}")
    _offs(offs, E)
    if sW.numel() != E * N * (K // 32):
        raise ValueError(f"sW must hold E*N*K/32 = {E * N * (K // 32)} bytes, got {sW.numel()}")
    out = _out(out, (M, N), torch.bfloat16, A.device, "out")
    ws = _ws(OP_FWD_Q, M, N, K, E, A.device, ws)
    _check("mx_grouped_mm_fwd_q",
           lib.mx_grouped_mm_fwd_q(_ptr(A), _ptr(qW), _ptr(sW), _ptr(offs), M, N, K, E, _ptr(out), _ptr(ws),
                                   ws.numel(), _stream(A.device)))
    return out


def mx_grouped_mm_dgrad_q(dOut, qWt, sWt, offs, out=None, ws=None):
    """mx_grouped_mm_dgrad with W given as (q_t, s_t) of mx_quantize_weights."""
    import torch
    lib = load_library()
    _require(dOut, torch.bfloat16, "dOut")
    _require(qWt, torch.uint8, "qWt")
    _require(sWt, torch.uint8, "sWt")
    _require(offs, torch.int32, "offs")
    M, N = dOut.shape
    E, K, N2 = qWt.shape
    if N2 != N:
        raise ValueError(f"dOut has N={N} but qWt has N={N2}")
    _offs(offs, E)
    if sWt.numel() != E * K * (N // 32):
        raise ValueError(f"sWt must hold E*K*N/32 = {E * K * (N // 32)} bytes, got {sWt.numel()}")
    out = _out(out, (M, K), torch.bfloat16, dOut.device, "out")
    ws = _ws(OP_DGRAD_Q, M, N, K, E, dOut.device, ws)
    _check("mx_grouped_mm_dgrad_q",
           lib.mx_grouped_mm_dgrad_q(_ptr(dOut), _ptr(qWt), _ptr(sWt), _ptr(offs), M, N, K, E, _ptr(out), _ptr(ws),
                                     ws.numel(), _stream(dOut.device)))
    return out


def mx_check_offsets(offs, M: int, align: int = 1, status=None):
    """Validity bitmask of the group offsets, computed on the device into
    `status` (int32 [1] on the GPU; returned without synchronizing).  0 = valid;
    OFFS_DECREASING / OFFS_RANGE / OFFS_LAST / OFFS_ALIGN otherwise."""
    import torch
    lib = load_library()
    _require(offs, torch.int32, "offs")
    if offs.dim() != 1:
        raise ValueError("offs must be int32 [E]")
    status = _out(status, (1,), torch.int32, offs.device, "status")
    _check("mx_check_offsets", lib.mx_check_offsets(_ptr(offs), offs.shape[0], int(M), int(align), _ptr(status),
                                                    _stream(offs.device)))
    return status


def check_offsets(offs, M: int, align: int = 1):
    """Raise ValueError, naming every violated rule, unless the group offsets
    are valid (reads the device status word: one synchronization)."""
    bits = int(mx_check_offsets(offs, M, align).item())
    if bits:
        why = [text for bit, text in ((OFFS_DECREASING, "an offset is below its predecessor"),
                                      (OFFS_RANGE, f"an offset lies outside [0, {M}]"),
                                      (OFFS_LAST, f"the last offset is not M={M}"),
                                      (OFFS_ALIGN, f"a group starts off a multiple of {align} (pad every group "
                                                   f"with zero rows to a multiple of {align})")) if bits & bit]
        raise ValueError("invalid group offsets: " + "; ".join(why))


def mx_grouped_mm_fwd_q_noalloc(A, qW, sW, offs, out):
    """mx_grouped_mm_fwd_q without a workspace: the library quantizes A into a
    static device array (NOALLOC_SCRATCH_BYTES) instead, so nothing is
    allocated (for graph capture or loops that cannot allocate).  `out` bf16
    [M, N] is the caller's.  Calls overlapping on one GPU share the array and
    race."""
    import torch
    lib = load_library()
    _require(A, torch.bfloat16, "A")
    _require(qW, torch.uint8, "qW")
    _require(sW, torch.uint8, "sW")
    _require(offs, torch.int32, "offs")
    M, K = A.shape
    E, N, K2 = qW.shape
    if K2 != K:
        raise ValueError(f"A has K={K} but qW has K={K2}")
    _offs(offs, E)
    if tuple(sW.shape) != (E, K // 128, N, 4):
        raise ValueError(f"sW must be in the GEMM scale layout {(E, K // 128, N, 4)}, got {tuple(sW.shape)}")
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    out = _out(out, (M, N), torch.bfloat16, A.device, "out")
    _check("mx_grouped_mm_fwd_q_noalloc",
           lib.mx_grouped_mm_fwd_q_noalloc(_ptr(A), _ptr(qW), _ptr(sW), _ptr(offs), M, N, K, E, _ptr(out),
                                           _stream(A.device)))
    return out


def mx_grouped_mm(A, W, offs, check_offsets: bool = True, weights=None, cache=None):
    """Differentiable MXFP8 grouped GEMM (forward, dgrad, wgrad in the library's kernels);
    expert weights quantized once and cached across micro-batches until they change."""
    from .autograd import mx_grouped_mm as _f
    return _f(A, W, offs, check_offsets, weights, cache)


def mx_linear(x, weight):
    """Differentiable dense MXFP8 linear y = x @ weight^T (one expert of mx_grouped_mm)."""
    from .autograd import mx_linear as _f
    return _f(x, weight)


def mx_quantize_rowwise_gather(x, rows, q=None, s=None):
    """Rowwise MX quantization of x[rows[r]] (rows int32 [M]; a negative index gives a zero row).
    Returns (q uint8 [M, cols], s uint8 [cols/128, M, 4] in the GEMM scale layout)."""
    import torch
    lib = load_library()
    _require(x, torch.bfloat16, "x")
    _require(rows, torch.int32, "rows")
    src_rows, cols = x.shape
    M = rows.shape[0]
    q = _out(q, (M, cols), torch.uint8, x.device, "q")
    s = _out(s, (cols // 128, M, 4), torch.uint8, x.device, "s")
    _check("mx_quantize_rowwise_gather",
           lib.mx_quantize_rowwise_gather(_ptr(x), src_rows, _ptr(rows), M, cols, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


# ---------------------------------------------------------------------------
# Routed experts: grouping, gather and scatter on the device
# ---------------------------------------------------------------------------
def route_capacity(n: int, E: int) -> int:
    """Rows of the grouped operands for n routed items over E experts: the
    most the groups can take once each is padded to 32 rows (n + 31 E),
    rounded up to 128 so the rows also serve as the wgrad contraction."""
    return (int(n) + 31 * int(E) + 127) // 128 * 128


def mx_route(expert_idx, E: int, cap: Optional[int] = None, offs=None, rows=None, pos=None, status=None, ws=None):
    """Group routed items by expert on the device.  expert_idx int32 [n] (a
    top-k router's [T, k] ids flattened token-major).  Returns (offs int32 [E]
    padded END offsets, rows int32 [cap] grouped row -> item or -1, pos int32
    [n] item -> grouped row, status int32 [1]: 1 if an id lies outside
    [0, E)).  `ws`: uint8 scratch of mx_route_workspace_bytes(n, E) bytes
    (allocated when None).  Nothing is synchronized."""
    import torch
    lib = load_library()
    _require(expert_idx, torch.int32, "expert_idx")
    if expert_idx.dim() != 1:
        raise ValueError("expert_idx must be int32 [n] (flatten a [T, k] router output)")
    n = expert_idx.shape[0]
    if cap is None:
        cap = route_capacity(n, E)
    dev = expert_idx.device
    offs = _out(offs, (E,), torch.int32, dev, "offs")
    rows = _out(rows, (cap,), torch.int32, dev, "rows")
    pos = _out(pos, (n,), torch.int32, dev, "pos")
    status = _out(status, (1,), torch.int32, dev, "status")
    need = mx_route_workspace_bytes(n, E)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _require(ws, torch.uint8, "ws")
    _check("mx_route", lib.mx_route(_ptr(expert_idx), n, int(E), int(cap), _ptr(offs), _ptr(rows), _ptr(pos),
                                    _ptr(status), _ptr(ws), ws.numel(), _stream(dev)))
    return offs, rows, pos, status


def mx_route_workspace_bytes(n: int, E: int) -> int:
    return int(load_library().mx_route_workspace_bytes(int(n), int(E)))


def mx_quantize_dual_gather(x, rows, topk: int = 1, ldq: Optional[int] = None, q=None, s=None, q_t=None, s_t=None):
    """mx_quantize_dual of the gathered rows x[rows[r] // topk] (zero rows
    where rows[r] < 0 or >= x.shape[0] * topk).  rows int32 [M] (M % 32 == 0).
    Returns (q [M, cols], s [cols/128, M, 4], q_t [cols, ldq], s_t
    [ldq/128, cols, 4]); ldq defaults to M rounded up to 128."""
    import torch
    lib = load_library()
    _require(x, torch.bfloat16, "x")
    _require(rows, torch.int32, "rows")
    if x.dim() != 2 or rows.dim() != 1:
        raise ValueError("x must be [src_rows, cols] and rows int32 [M]")
    src_rows, cols = x.shape
    M = rows.shape[0]
    if ldq is None:
        ldq = (M + 127) // 128 * 128
    dev = x.device
    q = _out(q, (M, cols), torch.uint8, dev, "q")
    s = _out(s, (cols // 128, M, 4), torch.uint8, dev, "s")
    q_t = _out(q_t, (cols, ldq), torch.uint8, dev, "q_t")
    s_t = _out(s_t, (ldq // 128, cols, 4), torch.uint8, dev, "s_t")
    _check("mx_quantize_dual_gather",
           lib.mx_quantize_dual_gather(_ptr(x), src_rows, _ptr(rows), int(topk), M, cols, int(ldq), _ptr(q), _ptr(s),
                                       _ptr(q_t), _ptr(s_t), _stream(dev)))
    return q, s, q_t, s_t


def mx_routed_experts(x, expert_idx, W, check: bool = True, weights=None, cache=None):
    """Differentiable routed experts: out[t] = x[t] @ W[expert_idx[t]]^T for a
    top-1 router (expert_idx [T]), out[t, j] = x[t] @ W[expert_idx[t, j]]^T for
    a top-k router (expert_idx [T, k]), with the grouping, the token gather
    (inside the quantizer) and the scatter back to item order (inside the GEMM
    epilogue) on the device."""
    from .autograd import mx_routed_experts as _f
    return _f(x, expert_idx, W, check, weights, cache)
