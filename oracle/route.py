"""CPU oracle for the routed-expert grouping and the routed grouped GEMMs.

TEST INFRASTRUCTURE ONLY (same rules as oracle.mxfp8: only the test suite,
the smoke check and the bench's CPU-baseline leg may use it).

What is computed, and where it is defined:

* The scaled grouped GEMM runs over each expert's routed tokens -- "MXFP8
  training for MoEs" article, section "Is MXFP8 Training for MoEs Actually
  Stable?"; the MoK expert PR adds the MXFP8 routed-expert path.  The pages
  leave the grouping itself open.  Readings (listed in the design notes):
    R-route  each expert's items keep their original order (a stable
             grouping by expert id), experts in increasing id order;
    R-pad    every group is followed by zero rows up to a multiple of 32, so
             the weight gradient's 32-token blocks never straddle two experts
             (the wgrad blocks run along the tokens, reading R-layout);
    R-drop   an item whose expert id lies outside [0, E) joins no group: its
             output row and its input gradient are zero.
* The routed GEMMs are the grouped GEMMs of oracle.mxfp8 on the grouped,
  zero-padded operands, with each result row taken back to its item.

Plain numpy and Python loops over experts.
"""

from __future__ import annotations

import numpy as np

from .mxfp8 import grouped_mm_dgrad, grouped_mm_fwd, grouped_mm_wgrad

GROUP_ALIGN = 32


def route_groups(expert_idx, E: int, cap: int):
    """Grouping of routed items (readings R-route, R-pad, R-drop).

    expert_idx: int [n].  Returns (offs int32 [E] cumulative END offsets of the
    padded groups, rows int32 [cap] grouped row -> item or -1, pos int32 [n]
    item -> grouped row or -1, bad: whether some id lies outside [0, E))."""
    idx = np.asarray(expert_idx, dtype=np.int64)
    n = idx.shape[0]
    rows = np.full(cap, -1, dtype=np.int32)
    pos = np.full(n, -1, dtype=np.int32)
    offs = np.zeros(E, dtype=np.int32)
    end = 0
    for e in range(E):
        items = [a for a in range(n) if idx[a] == e]      # original order
        for r, a in enumerate(items):
            rows[end + r] = a
            pos[a] = end + r
        end += -(-len(items) // GROUP_ALIGN) * GROUP_ALIGN
        offs[e] = end
    if end > cap:
        raise ValueError(f"cap={cap} is below the {end} rows the padded groups take")
    bad = bool(((idx < 0) | (idx >= E)).any())
    return offs, rows, pos, bad


def gather_rows(x_bits, rows, topk: int = 1):
    """Grouped operand: row r is x[rows[r] // topk], or zeros where rows[r]
    is negative or past the items (bf16 bit patterns in and out)."""
    x = np.asarray(x_bits)
    out = np.zeros((rows.shape[0],) + x.shape[1:], dtype=x.dtype)
    for r, a in enumerate(rows):
        if 0 <= a < x.shape[0] * topk:
            out[r] = x[a // topk]
    return out


def scatter_rows(g, rows, n: int):
    """Item-order result: item rows[r] gets grouped row r; items no row names
    stay zero (reading R-drop)."""
    out = np.zeros((n,) + g.shape[1:], dtype=g.dtype)
    for r, a in enumerate(rows):
        if 0 <= a < n:
            out[a] = g[r]
    return out


def routed_fwd(x_bits, expert_idx, W_bits, cap: int, absolute: bool = False, topk: int = 1):
    """out[a] = MX(x)[a // topk] @ MX(W[e_a])^T for every routed item a (a
    token of a top-1 router, or item a = token * topk + slot), in item order."""
    E = W_bits.shape[0]
    offs, rows, _, _ = route_groups(expert_idx, E, cap)
    g = grouped_mm_fwd(gather_rows(x_bits, rows, topk), W_bits, offs, absolute=absolute)
    return scatter_rows(g, rows, len(expert_idx))


def routed_dgrad(dOut_bits, expert_idx, W_bits, cap: int, absolute: bool = False, topk: int = 1):
    """dx[t] = sum over the token's items a of MX(dOut)[a] @ MX_t(W[e_a])
    (W blocked along N), in token order; dOut is in item order.  The sum of a
    token's items is the adjoint of the gather that fed them (reading R-topk),
    taken here exactly in fp64."""
    E = W_bits.shape[0]
    offs, rows, _, _ = route_groups(expert_idx, E, cap)
    g = grouped_mm_dgrad(gather_rows(dOut_bits, rows), W_bits, offs, absolute=absolute)
    items = scatter_rows(g, rows, dOut_bits.shape[0])
    return items.reshape(-1, topk, items.shape[1]).sum(axis=1)


def routed_wgrad(dOut_bits, x_bits, expert_idx, E: int, cap: int, absolute: bool = False, topk: int = 1):
    """dW[e] = sum over expert e's items a of dOut[a]^T x[a // topk], both
    operands quantized in 32-row blocks along the padded grouping (R-pad)."""
    offs, rows, _, _ = route_groups(expert_idx, E, cap)
    used = rows[:int(offs[-1])]               # the groups; rows past them are zeros in no group
    return grouped_mm_wgrad(gather_rows(dOut_bits, used), gather_rows(x_bits, used, topk), offs, absolute=absolute)


def topk_sum_rows(x_f32, topk: int):
    """bf16 bits of each token's sum of its topk fp32 rows: fp32 additions in
    slot order starting from +0, then one round to nearest even (the reading
    of the gradient sum for a kernel that keeps fp32 accumulators)."""
    x = np.asarray(x_f32, dtype=np.float32)
    acc = np.zeros((x.shape[0] // topk,) + x.shape[1:], dtype=np.float32)
    for j in range(topk):
        acc = acc + x[j::topk]
    # round to nearest even on the 16 dropped bits (finite values): add half an
    # ulp less one, plus the kept lsb, and truncate
    u = acc.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
