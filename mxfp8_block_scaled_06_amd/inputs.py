"""Seeded synthetic inputs shared by the HIP path, the oracle and the bench.

This module only draws random tensors and routing counts.  It holds none of
the MXFP8 arithmetic (no amax, no scale, no cast, no matmul): both the oracle
and the HIP library receive the bf16 bit patterns produced here and compute
everything else on their own.

Workloads follow the shapes of the MoE routed-expert GEMMs on the pages:
  * "MXFP8 training for MoEs" article, sections "Is MXFP8 Training for MoEs
    Actually Stable?" (Llama4 Scout routed experts, EP=16) and "Why Does MXFP8
    Speed Up MoE Training So Much?" (grouped GEMMs over routed experts);
  * pytorch/ao PR "[mxfp8 moe training] wrap 3d quantize tensor in custom ops
    and integrate it", benchmark "seq_len=8192, experts per device = 2"
    (dim 5120, two experts per device, total_M=65600).
The expert hidden size N=8192 and the DeepSeek-style share (E=32, K=7168,
N=2048, Zipf routing) are workload choices of this library, not page facts.

Generation recipe (all host side, numpy PCG64 via ``default_rng(seed)``):
  draw order counts -> A -> outlier mask -> W -> dOut;
  fp32 normal draws, converted to bf16 by round-to-nearest-even on the bits.
Tokens are generated already grouped by expert (the permutation/gather that
routes tokens is outside the path).
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# fp32 -> bf16 bit patterns (round to nearest even), input plumbing only.
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return the uint16 bit patterns.

    NaNs stay NaN (quiet bit forced).  Used only to materialise inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint32, copy=True)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact).  Input plumbing only."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------
# Routing: per-expert token counts and cumulative END offsets.
# --------------------------------------------------------------------------
def offsets_from_counts(counts) -> np.ndarray:
    """int32[E] cumulative end offsets: group e is rows [offs[e-1], offs[e])."""
    return np.cumsum(np.asarray(counts, dtype=np.int64)).astype(np.int32)


def pad_counts(counts, multiple: int = 32) -> np.ndarray:
    c = np.asarray(counts, dtype=np.int64)
    return ((c + multiple - 1) // multiple) * multiple


def expert_ids(rng, counts) -> np.ndarray:
    """Router output in token order: int32 [sum(counts)] holding counts[e]
    copies of each expert id e, in a seeded random order."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), np.asarray(counts, dtype=np.int64))
    return rng.permutation(ids).astype(np.int32)


def uniform_counts(rng, total: int, experts: int) -> np.ndarray:
    """Top-1 routing drawn from a multinomial over uniform expert probabilities."""
    return rng.multinomial(total, np.full(experts, 1.0 / experts)).astype(np.int64)


def zipf_counts(rng, total: int, experts: int, s: float = 1.2, n_empty: int = 2) -> np.ndarray:
    """Zipf-skewed routing with ``n_empty`` experts forced empty.

    A seeded permutation picks which expert ids are empty and which get which
    Zipf rank; the other experts draw tokens from Multinomial(total, p) with
    p proportional to rank**-s.
    """
    perm = rng.permutation(experts)
    live = perm[n_empty:]
    ranks = np.arange(1, len(live) + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    live_counts = rng.multinomial(total, p)
    counts = np.zeros(experts, dtype=np.int64)
    counts[live] = live_counts
    return counts


# --------------------------------------------------------------------------
# Workload registry
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    E: int
    M: int          # total routed tokens (before padding)
    K: int          # model dim (fwd contraction)
    N: int          # expert hidden dim
    routing: str    # "fixed" | "uniform" | "zipf"
    fixed_counts: Optional[tuple] = None
    outliers: bool = False
    pad32: bool = False       # groups padded to multiples of 32 (backward)
    description: str = ""


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, E=2, M=256, K=256, N=512, routing="fixed", fixed_counts=(96, 160),
        description="E=2, M=256 split 96/160, K=256, N=512; forward only"),
    "llama4_fwd": Workload(
        "llama4_fwd", 2, E=16, M=16384, K=5120, N=8192, routing="uniform", outliers=True,
        description="Llama4-Scout-shaped routed experts, forward: E=16, M=16384, K=5120, N=8192"),
    "llama4_bwd": Workload(
        "llama4_bwd", 3, E=16, M=16384, K=5120, N=8192, routing="uniform", outliers=True,
        pad32=True,
        description="Llama4-Scout-shaped routed experts, dgrad + wgrad, groups padded to 32"),
    "debug_shard": Workload(
        "debug_shard", 4, E=2, M=65600, K=5120, N=8192, routing="fixed",
        fixed_counts=(26240, 39360), outliers=True, pad32=True,
        description="Llama4 debug-model shard: E=2, M=65600 split 40/60, K=5120, N=8192"),
    "deepseek_share": Workload(
        "deepseek_share", 5, E=32, M=32768, K=7168, N=2048, routing="zipf",
        description="DeepSeek-style fine-grained experts: E=32, M=32768, K=7168, N=2048, Zipf 1.2, 2 empty"),
}


@dataclasses.dataclass
class Inputs:
    workload: Workload
    counts: np.ndarray            # int64[E], real tokens per expert
    padded_counts: np.ndarray     # int64[E], rows per expert as laid out
    offs: np.ndarray              # int32[E], cumulative END offsets over padded_counts
    A: np.ndarray                 # uint16 bf16 bits [M_rows, K]
    W: Optional[np.ndarray]       # uint16 bf16 bits [E, N, K]
    dOut: Optional[np.ndarray]    # uint16 bf16 bits [M_rows, N]

    @property
    def M_rows(self) -> int:
        return int(self.A.shape[0])


def draw_counts(w: Workload, rng) -> np.ndarray:
    if w.routing == "fixed":
        return np.asarray(w.fixed_counts, dtype=np.int64)
    if w.routing == "uniform":
        return uniform_counts(rng, w.M, w.E)
    if w.routing == "zipf":
        return zipf_counts(rng, w.M, w.E)
    raise ValueError(w.routing)


def make_activations(rng, rows: int, K: int, outliers: bool) -> np.ndarray:
    """A ~ N(0,1); with ``outliers`` a Bernoulli(0.001) mask multiplies by 50."""
    x = rng.standard_normal(size=(rows, K), dtype=np.float32)
    if outliers:
        mask = rng.random(size=(rows, K), dtype=np.float32) < np.float32(0.001)
        x[mask] *= np.float32(50.0)
    return f32_to_bf16_bits(x)


def make_weights(rng, E: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    W = np.empty((E, N, K), dtype=np.uint16)
    for e in range(E):
        W[e] = _normal_bf16(rng, (N, K), std)
    return W


def make_inputs(w: Workload | str, with_weights: bool = True, with_grad: bool = False,
                counts=None) -> Inputs:
    """Materialise the seeded inputs of a workload.

    ``counts`` overrides the routing draw (unit tests of ragged/empty groups).
    With ``pad32`` each group is padded by zero rows to a multiple of 32.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    drawn = draw_counts(w, rng)
    counts = drawn if counts is None else np.asarray(counts, dtype=np.int64)
    padded = pad_counts(counts) if w.pad32 else counts.copy()
    offs = offsets_from_counts(padded)
    rows = int(padded.sum())
    A = make_activations(rng, rows, w.K, w.outliers)
    W = make_weights(rng, w.E, w.N, w.K) if with_weights else None
    dOut = _normal_bf16(rng, (rows, w.N), 1e-3) if with_grad else None
    if w.pad32:
        starts = np.concatenate([[0], offs[:-1]]).astype(np.int64)
        for e in range(w.E):
            lo, hi = int(starts[e] + counts[e]), int(offs[e])
            A[lo:hi] = 0
            if dOut is not None:
                dOut[lo:hi] = 0
    return Inputs(w, counts, padded, offs, A, W, dOut)


def make_sweep(rows: int = 65600, cols: int = 5120, seed: int = 4) -> np.ndarray:
    """Standalone quantize sweep tensor: bf16 [rows, cols], N(0,1) + 0.1% x50 outliers."""
    rng = np.random.default_rng(seed + 1000)
    return make_activations(rng, rows, cols, outliers=True)


def random_bf16(shape, seed: int, std: float = 1.0, outliers: bool = False) -> np.ndarray:
    """Generic seeded bf16 tensor for unit tests."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    if outliers:
        mask = rng.random(size=shape, dtype=np.float32) < np.float32(0.001)
        x[mask] *= np.float32(50.0)
    return f32_to_bf16_bits(x)


def all_bf16_patterns() -> np.ndarray:
    """All 65,536 bf16 bit patterns (for exhaustive codec checks)."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)
