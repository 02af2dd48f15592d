"""Differentiable MXFP8 grouped GEMM for MoE routed experts.

    out = mx_grouped_mm(A, W, offs)      # out[g_e] = A[g_e] @ W[e]^T

is the primitive of the "MXFP8 training for MoEs" article (section "Is MXFP8
Training for MoEs Actually Stable?": dynamic MXFP8 quantization, scaled
grouped GEMM, result in the original precision, differentiable; section "Why
Does MXFP8 Speed Up MoE Training So Much?": the backward mirrors the forward).
The expert weights are quantized once in both orientations (the weight
4-tuple of the MoK expert PR review) and cached until they change, so the
micro-batches of one optimizer step share one weight quantization; the
forward keeps the orientation the backward needs.
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

import weakref

from . import (mx_grouped_gemm_mx, mx_grouped_gemm_mx_rows, mx_grouped_mm_dgrad_q, mx_grouped_mm_fwd_q,
               mx_quantize_dual, mx_quantize_dual_gather, mx_quantize_rowwise_gather, mx_quantize_weights,
               mx_route, mx_topk_sum_rows)


class WeightCache:
    """Prequantized expert weights kept across micro-batches until the weights
    change: the weight cache of the "feat(moe): add MoK MXFP8 expert support"
    PR review (keyed by storage identity, reused until optimizer.step()).

    An entry holds the MX 4-tuple (q, s, q_t, s_t) of mx_quantize_weights for
    one weight tensor and is valid while that same tensor object is alive, at
    the same storage and shape, with the same in-place version counter: an
    optimizer step updates the weights in place, which bumps the counter, so
    the next forward quantizes them again.  `quantizations` counts the
    quantization passes run (tests use it)."""

    def __init__(self):
        self._entries = {}
        self.quantizations = 0

    @staticmethod
    def _key(W):
        return (W.data_ptr(), tuple(W.shape), tuple(W.stride()), W.device, W._version)

    def get(self, W, as_experts=None):
        """The 4-tuple of W (or of `as_experts`, a 3-D view of W such as a
        dense weight's unsqueeze(0), while the entry stays keyed on W)."""
        ent = self._entries.get(id(W))
        if ent is not None and ent[0]() is W and ent[1] == self._key(W):
            return ent[2]
        # quantized from a detached view: the 4-tuple is not part of the autograd graph
        mx4 = mx_quantize_weights((W if as_experts is None else as_experts).detach())
        self.quantizations += 1
        self._entries[id(W)] = (weakref.ref(W, lambda _, k=id(W): self._entries.pop(k, None)), self._key(W), mx4)
        return mx4

    def clear(self):
        self._entries.clear()


_DEFAULT_CACHE = WeightCache()


def weight_cache() -> WeightCache:
    """The cache mx_grouped_mm uses unless told otherwise."""
    return _DEFAULT_CACHE


def _check_mx4(W, mx4):
    """The prequantized 4-tuple must match W's shape; a mismatch raises (the
    MoK contract: the FP8 weights are given exactly when they are used)."""
    import torch
    E, N, K = W.shape
    want = ((E, N, K), (E, K // 128, N, 4), (E, K, N), (E, N // 128, K, 4))
    if len(mx4) != 4:
        raise ValueError("mx_grouped_mm: weights must be the 4-tuple (q, s, q_t, s_t) of mx_quantize_weights")
    for t, sh, name in zip(mx4, want, ("q", "s", "q_t", "s_t")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or tuple(t.shape) != sh:
            raise ValueError(f"mx_grouped_mm: prequantized weights {name} must be uint8 {sh}, got "
                             f"{getattr(t, 'dtype', type(t))} {tuple(getattr(t, 'shape', ()))}")


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
                def forward(ctx, A, W, offs, mx4):
                    qW, sW, qWt, sWt = mx4
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
                    return dA, dW, None, None

            cls.fn = Fn
        return cls.fn


def mx_grouped_mm(A, W, offs, check_offsets: bool = True, weights=None, cache: WeightCache | None = None):
    """Differentiable out[g_e] = A[g_e] @ W[e]^T with MXFP8 operands (see the module docstring).

    The expert weights' MX 4-tuple comes from `weights` when given (the
    caller's own prequantized copy, checked against W's shape), else from
    `cache` (default: the module's WeightCache), which quantizes W once and
    reuses the result across micro-batches until W changes."""
    _check(A, W, offs, check_offsets)
    W = W.contiguous()
    if weights is not None:
        _check_mx4(W, weights)
        mx4 = tuple(weights)
    else:
        mx4 = (cache if cache is not None else _DEFAULT_CACHE).get(W)
    return _MXGroupedMM.get().apply(A.contiguous(), W, offs, mx4)


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
    w3 = weight.unsqueeze(0)
    return mx_grouped_mm(x, w3, offs, weights=_DEFAULT_CACHE.get(weight, as_experts=w3))


class _MXRouted:
    """torch.autograd.Function of mx_routed_experts (built lazily)."""
    fn = None

    @classmethod
    def get(cls):
        if cls.fn is None:
            import torch

            class Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, x, W, offs, rows, mx4, zero_fill, topk):
                    qW, sW, qWt, sWt = mx4
                    n_items = x.shape[0] * topk
                    cap = rows.shape[0]
                    alloc = torch.zeros if zero_fill else torch.empty
                    out = alloc((n_items, W.shape[1]), dtype=torch.bfloat16, device=x.device)
                    if ctx.needs_input_grad[1] or topk > 1:
                        # items gathered into their expert groups inside the
                        # quantizer (item a reads token a // topk), in both
                        # orientations (wgrad keeps the 32x1-along-items codes)
                        qA, sA, qAt, sAt = mx_quantize_dual_gather(x, rows, topk=topk, ldq=cap)
                        if not ctx.needs_input_grad[1]:
                            qAt = sAt = None
                    else:
                        qA, sA = mx_quantize_rowwise_gather(x, rows)
                        qAt = sAt = None
                    # the epilogue stores each grouped row at its item's row
                    mx_grouped_gemm_mx_rows(qA, sA, qW, sW, offs, rows, out=out)
                    del qA, sA, qW, sW
                    ctx.zero_fill = zero_fill
                    ctx.topk = topk
                    ctx.save_for_backward(offs, rows, qWt, sWt, qAt, sAt)
                    return out

                @staticmethod
                def backward(ctx, dOut):
                    offs, rows, qWt, sWt, qAt, sAt = ctx.saved_tensors
                    dOut = dOut.contiguous()
                    topk = ctx.topk
                    dx = dW = None
                    alloc = torch.zeros if ctx.zero_fill else torch.empty
                    if ctx.needs_input_grad[1]:
                        qG, sG, qGt, sGt = mx_quantize_dual_gather(dOut, rows, ldq=rows.shape[0])
                        dW = mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, offs, 1)
                    elif ctx.needs_input_grad[0]:
                        qG, sG = mx_quantize_rowwise_gather(dOut, rows)
                    if ctx.needs_input_grad[0]:
                        K = qWt.shape[1]
                        if topk == 1:
                            dx = alloc((dOut.shape[0], K), dtype=torch.bfloat16, device=dOut.device)
                            mx_grouped_gemm_mx_rows(qG, sG, qWt, sWt, offs, rows, out=dx)
                        else:
                            # per-item gradients in fp32, then each token's
                            # topk of them summed and rounded once (the adjoint
                            # of the gather that fed the items)
                            items = torch.zeros((dOut.shape[0], K), dtype=torch.float32, device=dOut.device)
                            mx_grouped_gemm_mx_rows(qG, sG, qWt, sWt, offs, rows, out=items)
                            dx = mx_topk_sum_rows(items, topk)
                    return dx, dW, None, None, None, None, None

            cls.fn = Fn
        return cls.fn


def mx_routed_experts(x, expert_idx, W, check: bool = True, weights=None, cache: WeightCache | None = None):
    """Differentiable routed experts: out[t, j] = x[t] @ W[expert_idx[t, j]]^T.

    x bf16 [T, K] in token order; expert_idx int32 on the device, [T] for a
    top-1 router (out bf16 [T, N]) or [T, k] for a top-k router (out bf16
    [T, k, N], one row per token-expert pair; the caller's combine weights and
    sums them); W bf16 [E, N, K] with N % 128 == 0 and K % 128 == 0.
    mx_route groups the items (token-expert pairs, token-major) by expert on
    the device (each expert's items in their original order, padded with zero
    rows to a multiple of 32), the quantizer gathers the tokens into that
    grouping, and the GEMM epilogue stores every row back at its item, so
    neither a permuted copy of the tokens nor an unpermute pass exists; the
    backward gathers dOut the same way.  For k > 1 the input gradient of a
    token sums its k items' fp32 gradients and rounds once.  Weights as for
    mx_grouped_mm (`weights`, else the cache).

    check=True reads the routing status (one synchronization) and raises on
    an expert id outside [0, E).  With check=False such items are dropped:
    their output rows are zero and they add nothing to the gradients."""
    import torch
    if x.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("mx_routed_experts: x and W must be bfloat16")
    if x.dim() != 2 or W.dim() != 3 or W.shape[2] != x.shape[1]:
        raise ValueError("mx_routed_experts: x must be [T, K] and W [E, N, K]")
    T = x.shape[0]
    if expert_idx.dtype != torch.int32 or expert_idx.dim() not in (1, 2) or expert_idx.shape[0] != T:
        raise ValueError(f"mx_routed_experts: expert_idx must be int32 [T={T}] or [T={T}, k]")
    topk = 1 if expert_idx.dim() == 1 else expert_idx.shape[1]
    if topk < 1:
        raise ValueError("mx_routed_experts: k must be at least 1")
    E, N, K = W.shape
    if K % 128 or N % 128:
        raise ValueError(f"mx_routed_experts: N={N} and K={K} must be multiples of 128")
    offs, rows, _pos, status = mx_route(expert_idx.contiguous().reshape(-1), E)
    if check:
        if int(status.item()):
            raise ValueError(f"mx_routed_experts: an expert id lies outside [0, {E})")
    W = W.contiguous()
    if weights is not None:
        _check_mx4(W, weights)
        mx4 = tuple(weights)
    else:
        mx4 = (cache if cache is not None else _DEFAULT_CACHE).get(W)
    out = _MXRouted.get().apply(x.contiguous(), W, offs, rows, mx4, not check, topk)
    return out if expert_idx.dim() == 1 else out.view(T, topk, N)
