"""Differentiable MXFP8 grouped GEMM for MoE routed experts.

    out = mx_grouped_mm(A, W, offs)      # out[g_e] = A[g_e] @ W[e]^T

is the primitive of the "MXFP8 training for MoEs" article (section "Is MXFP8
Training for MoEs Actually Stable?": dynamic MXFP8 quantization, scaled
grouped GEMM, result in the original precision, differentiable; section "Why
Does MXFP8 Speed Up MoE Training So Much?": the backward mirrors the forward).
The forward quantizes the expert weights once in both orientations and keeps
the one the backward needs: the weight 4-tuple of the MoK expert PR review.
Activations get the same treatment: the forward quantizes A in both
orientations from one read (1x32 along K for its own GEMM, 32x1 along the
tokens for the wgrad GEMM) and keeps the fp8 transpose instead of the bf16 A;
the backward quantizes dOut in both orientations (dgrad and wgrad) from one
read.  Every step runs in the library's kernels; this module only wires them
into torch.autograd.

Contract (checked here, with a clear error otherwise; the group offsets are
checked on the device, one synchronization per call, unless
check_offsets=False):
  A    bf16 [M, K] tokens grouped by expert (offs: int32 [E] END offsets on
       the device), every group start a multiple of 32 (pad groups with zero
       rows) and M % 32 == 0 -- the weight gradient sums 32-token blocks that
       never straddle two experts;
  W    bf16 [E, N, K] with N % 128 == 0 and K % 128 == 0;
  out  bf16 [M, N];  dA = dOut @ W[e] per group;  dW[e] = dOut[g_e]^T @ A[g_e].
"""

from __future__ import annotations

from . import (mx_grouped_gemm_mx, mx_grouped_mm_dgrad_q, mx_grouped_mm_fwd_q, mx_quantize_dual,
               mx_quantize_weights)


def _check(A, W, offs, check_offsets=True):
    import torch
    if A.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("mx_grouped_mm: A and W must be bfloat16")
    if offs.dtype != torch.int32:
        raise TypeError("mx_grouped_mm: offs must be int32 cumulative END offsets")
    if A.dim() != 2 or W.dim() != 3:
        raise ValueError("mx_grouped_mm: A must be [M, K] and W [E, N, K]")
    M, K = A.shape
    E, N, K2 = W.shape
    if K2 != K:
        raise ValueError(f"mx_grouped_mm: A has K={K} but W has K={K2}")
    if offs.shape != (E,):
        raise ValueError(f"mx_grouped_mm: offs must have one entry per expert ({E}), got {tuple(offs.shape)}")
    if K % 128 or N % 128:
        raise ValueError(f"mx_grouped_mm: N={N} and K={K} must be multiples of 128")
    if M % 32:
        raise ValueError(f"mx_grouped_mm: M={M} must be a multiple of 32 (pad every group to 32 rows)")
    if check_offsets and A.is_cuda:
        # the weight gradient's 32-token blocks must not straddle two experts
        from . import check_offsets as _chk
        _chk(offs, M, 32)


class _MXGroupedMM:
    """torch.autograd.Function (built lazily so importing the package needs no torch)."""
    fn = None

    @classmethod
    def get(cls):
        if cls.fn is None:
            import torch

            class Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, A, W, offs):
                    qW, sW, qWt, sWt = mx_quantize_weights(W)
                    if ctx.needs_input_grad[1]:
                        # A in both orientations: the 32x1-along-tokens codes
                        # are the wgrad operand, kept instead of the bf16 A
                        qA, sA, qAt, sAt = mx_quantize_dual(A)
                        out = mx_grouped_gemm_mx(qA, sA, qW, sW, offs, 0)
                        del qA, sA
                    else:
                        out = mx_grouped_mm_fwd_q(A, qW, sW, offs)
                        qAt = sAt = None
                    # the forward orientation of W is not needed again; the backward
                    # keeps the 32x1-along-N codes (weight_t_fp8 / weight_t_scale)
                    del qW, sW
                    ctx.save_for_backward(offs, qWt, sWt, qAt, sAt)
                    return out

                @staticmethod
                def backward(ctx, dOut):
                    offs, qWt, sWt, qAt, sAt = ctx.saved_tensors
                    dOut = dOut.contiguous()
                    dA = dW = None
                    if ctx.needs_input_grad[1]:
                        # dOut in both orientations from one read: 1x32 along N
                        # for dgrad, 32x1 along the tokens for wgrad
                        qG, sG, qGt, sGt = mx_quantize_dual(dOut, ldq=qAt.shape[1])
                        if ctx.needs_input_grad[0]:
                            dA = mx_grouped_gemm_mx(qG, sG, qWt, sWt, offs, 0)
                        dW = mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, offs, 1)
                    elif ctx.needs_input_grad[0]:
                        dA = mx_grouped_mm_dgrad_q(dOut, qWt, sWt, offs)
                    return dA, dW, None

            cls.fn = Fn
        return cls.fn


def mx_grouped_mm(A, W, offs, check_offsets: bool = True):
    """Differentiable out[g_e] = A[g_e] @ W[e]^T with MXFP8 operands (see the module docstring)."""
    _check(A, W, offs, check_offsets)
    return _MXGroupedMM.get().apply(A.contiguous(), W.contiguous(), offs)


def mx_linear(x, weight):
    """Differentiable dense MXFP8 linear y = x @ weight^T (x bf16 [M, K], weight bf16 [N, K]):
    the one-expert case of mx_grouped_mm (the dense half of "MoE + dense" in the
    pytorch/ao PR benchmarks).  Same contract with E = 1: M % 32 == 0,
    N % 128 == 0, K % 128 == 0."""
    import torch
    if weight.dim() != 2:
        raise ValueError("mx_linear: weight must be [N, K]")
    if x.dim() != 2:
        raise ValueError("mx_linear: x must be [M, K]")
    offs = torch.tensor([x.shape[0]], dtype=torch.int32, device=x.device)
    return mx_grouped_mm(x, weight.unsqueeze(0), offs)
