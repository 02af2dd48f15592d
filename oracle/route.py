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


def routed_fwd(x_bits, expert_idx, W_bits, cap: int, absolute: bool = False):
    """out[t] = MX(x)[t] @ MX(W[e_t])^T for top-1 routed tokens, in token order."""
    E = W_bits.shape[0]
    offs, rows, _, _ = route_groups(expert_idx, E, cap)
    g = grouped_mm_fwd(gather_rows(x_bits, rows), W_bits, offs, absolute=absolute)
    return scatter_rows(g, rows, x_bits.shape[0])


def routed_dgrad(dOut_bits, expert_idx, W_bits, cap: int, absolute: bool = False):
    """dx[t] = MX(dOut)[t] @ MX_t(W[e_t]) in token order (W blocked along N)."""
    E = W_bits.shape[0]
    offs, rows, _, _ = route_groups(expert_idx, E, cap)
    g = grouped_mm_dgrad(gather_rows(dOut_bits, rows), W_bits, offs, absolute=absolute)
    return scatter_rows(g, rows, dOut_bits.shape[0])


def routed_wgrad(dOut_bits, x_bits, expert_idx, E: int, cap: int, absolute: bool = False):
    """dW[e] = sum over expert e's tokens of dOut[t]^T x[t], both operands
    quantized in 32-row blocks along the padded grouping (reading R-pad)."""
    offs, rows, _, _ = route_groups(expert_idx, E, cap)
    used = rows[:int(offs[-1])]               # the groups; rows past them are zeros in no group
    return grouped_mm_wgrad(gather_rows(dOut_bits, used), gather_rows(x_bits, used), offs, absolute=absolute)
