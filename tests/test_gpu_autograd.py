"""GPU checks of the differentiable primitive mx_grouped_mm (forward, dgrad and
wgrad through torch.autograd, all in the library's kernels):
  - bit-identical to the three entry points it composes;
  - within the GEMM criterion of the oracle for out, dA and dW;
  - close to an fp64 autograd reference of the unquantized grouped GEMM: its
    normwise error is no larger than twice the oracle's own MXFP8 error
    against that reference (the quantization is the only approximation).
"""

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_06_amd import inputs as inp
from gpu_util import require_gpu, to_dev_bf16, to_dev_i32, bf16_host_bits, log

pytestmark = pytest.mark.gpu


def _fp64_reference(A, W, G, counts):
    """Unquantized grouped GEMM and its gradients by torch autograd in fp64 (CPU)."""
    import torch
    A64 = torch.from_numpy(oracle.bf16_to_f64(A)).requires_grad_(True)
    W64 = torch.from_numpy(oracle.bf16_to_f64(W)).requires_grad_(True)
    G64 = torch.from_numpy(oracle.bf16_to_f64(G))
    outs, st = [], 0
    for e, c in enumerate(counts):
        outs.append(A64[st:st + c] @ W64[e].T)
        st += c
    out = torch.cat(outs, 0)
    out.backward(G64)
    return out.detach().numpy(), A64.grad.numpy(), W64.grad.numpy()


def _normwise(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


CASES = {
    "three_groups": ([64, 0, 96], 256, 256),
    "single": ([128], 384, 256),
    "empty_last": ([32, 160, 0], 256, 384),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_autograd_matches_entry_points_oracle_and_fp64(case):
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    counts, N, K = CASES[case]
    E, M = len(counts), sum(counts)
    offs = inp.offsets_from_counts(counts)
    A = inp.random_bf16((M, K), seed=1000 + E, outliers=True)
    W = inp.random_bf16((E, N, K), seed=1100 + E, std=0.02)
    G = inp.random_bf16((M, N), seed=1200 + E, std=1e-3)
    log(f"autograd case={case} counts={counts} N={N} K={K}")
    Ad = to_dev_bf16(A).requires_grad_(True)
    Wd = to_dev_bf16(W).requires_grad_(True)
    Gd, od = to_dev_bf16(G), to_dev_i32(offs)
    out = mx.mx_grouped_mm(Ad, Wd, od)
    out.backward(Gd)
    torch.cuda.synchronize()
    # the composed entry points
    with torch.no_grad():
        ref_out = mx.mx_grouped_mm_fwd(Ad.detach(), Wd.detach(), od)
        ref_dA = mx.mx_grouped_mm_dgrad(Gd, Wd.detach(), od)
        ref_dW = mx.mx_grouped_mm_wgrad(Gd, Ad.detach(), od)
    for name, got, ref in (("out", out, ref_out), ("dA", Ad.grad, ref_dA), ("dW", Wd.grad, ref_dW)):
        assert torch.equal(got.detach().view(torch.int16), ref.view(torch.int16)), name
    # the oracle
    o_out = oracle.grouped_mm_fwd(A, W, offs)
    o_dA = oracle.grouped_mm_dgrad(G, W, offs)
    o_dW = oracle.grouped_mm_wgrad(G, A, offs)
    for name, got, ref, absr in (
            ("out", out, o_out, oracle.grouped_mm_fwd(A, W, offs, absolute=True)),
            ("dA", Ad.grad, o_dA, oracle.grouped_mm_dgrad(G, W, offs, absolute=True)),
            ("dW", Wd.grad, o_dW, oracle.grouped_mm_wgrad(G, A, offs, absolute=True))):
        rep = oracle.r1_check(bf16_host_bits(got.detach()), ref, abs_terms=absr)
        assert rep["ok"], (name, rep)
    # fp64 autograd of the unquantized GEMM
    f_out, f_dA, f_dW = _fp64_reference(A, W, G, counts)
    for name, got, orc, ref in (("out", out, o_out, f_out), ("dA", Ad.grad, o_dA, f_dA), ("dW", Wd.grad, o_dW, f_dW)):
        g = oracle.bf16_to_f64(bf16_host_bits(got.detach()))
        err, err_oracle = _normwise(g, ref), _normwise(orc, ref)
        log(f"  {name}: normwise vs fp64 autograd {err:.3e} (oracle {err_oracle:.3e})")
        assert err <= 2 * err_oracle + 1e-3, (name, err, err_oracle)
    # empty experts get exactly zero weight gradient
    for e, c in enumerate(counts):
        if c == 0:
            assert (Wd.grad[e] == 0).all()


def test_autograd_only_requested_gradients():
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    counts = [64, 64]
    offs = to_dev_i32(inp.offsets_from_counts(counts))
    A = to_dev_bf16(inp.random_bf16((128, 256), seed=1300)).requires_grad_(True)
    W = to_dev_bf16(inp.random_bf16((2, 256, 256), seed=1301, std=0.02))
    out = mx.mx_grouped_mm(A, W, offs)
    out.sum().backward()
    assert A.grad is not None and W.grad is None


def test_dense_linear_is_one_expert():
    """mx_linear: E = 1 of the grouped primitive; gradients within the GEMM
    criterion of the oracle (dense matmuls of the dequantized operands)."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    M, N, K = 160, 256, 384
    A = inp.random_bf16((M, K), seed=1400, outliers=True)
    W = inp.random_bf16((N, K), seed=1401, std=0.02)
    G = inp.random_bf16((M, N), seed=1402, std=1e-3)
    log(f"dense linear M={M} N={N} K={K}")
    x = to_dev_bf16(A).requires_grad_(True)
    w = to_dev_bf16(W).requires_grad_(True)
    y = mx.mx_linear(x, w)
    y.backward(to_dev_bf16(G))
    offs = np.array([M], dtype=np.int32)
    for name, got, ref, absr in (
            ("y", y, oracle.grouped_mm_fwd(A, W[None], offs), oracle.grouped_mm_fwd(A, W[None], offs, absolute=True)),
            ("dx", x.grad, oracle.grouped_mm_dgrad(G, W[None], offs),
             oracle.grouped_mm_dgrad(G, W[None], offs, absolute=True)),
            ("dw", w.grad, oracle.grouped_mm_wgrad(G, A, offs)[0],
             oracle.grouped_mm_wgrad(G, A, offs, absolute=True)[0])):
        rep = oracle.r1_check(bf16_host_bits(got.detach()), ref, abs_terms=absr)
        assert rep["ok"], (name, rep)
    assert w.grad.shape == (N, K)


def test_autograd_rejects_unaligned_group_starts():
    """A group starting off a multiple of 32 would make the weight gradient's
    32-token blocks straddle two experts: the primitive refuses it before any
    GEMM, with a message naming the rule."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    A = to_dev_bf16(inp.random_bf16((128, 128), seed=1300))
    W = to_dev_bf16(inp.random_bf16((2, 128, 128), seed=1301, std=0.02))
    with pytest.raises(ValueError, match="multiple of 32"):
        mx.mx_grouped_mm(A, W, to_dev_i32(np.array([40, 128], dtype=np.int32)))
    with pytest.raises(ValueError, match="last offset"):
        mx.mx_grouped_mm(A, W, to_dev_i32(np.array([64, 96], dtype=np.int32)))
    out = mx.mx_grouped_mm(A, W, to_dev_i32(np.array([64, 128], dtype=np.int32)))
    assert out.shape == (128, 128)


def test_weight_cache_spans_micro_batches_until_the_weights_change():
    """Two micro-batches with the same expert weights run one weight
    quantization (the prequantized-weight cache of the MoK expert PR review)
    and give the results of quantizing every time; an in-place update of the
    weights (what an optimizer step does) makes the next forward requantize."""
    torch = require_gpu()
    import mxfp8_block_scaled_06_amd as mx
    from mxfp8_block_scaled_06_amd.autograd import WeightCache
    counts = [64, 0, 96, 32]
    offs = to_dev_i32(inp.offsets_from_counts(counts))
    W = to_dev_bf16(inp.random_bf16((4, 256, 384), seed=1400, std=0.02)).requires_grad_(True)
    cache = WeightCache()
    outs = []
    for mb in range(2):
        A = to_dev_bf16(inp.random_bf16((192, 384), seed=1410 + mb, outliers=True)).requires_grad_(True)
        out = mx.mx_grouped_mm(A, W, offs, cache=cache)
        G = to_dev_bf16(inp.random_bf16((192, 256), seed=1420 + mb, std=1e-3))
        out.backward(G)
        ref = mx.mx_grouped_mm(A.detach(), W.detach(), offs, weights=mx.mx_quantize_weights(W.detach()))
        assert torch.equal(out.detach().view(torch.int16), ref.view(torch.int16))
        outs.append(out.detach())
    assert cache.quantizations == 1
    grad_after_two = W.grad.clone()
    assert grad_after_two.abs().sum() > 0
    with torch.no_grad():
        W.mul_(2.0)                       # an in-place update, as an optimizer step makes
    A = to_dev_bf16(inp.random_bf16((192, 384), seed=1410, outliers=True))
    out = mx.mx_grouped_mm(A, W, offs, cache=cache)
    assert cache.quantizations == 2
    # doubling every weight doubles every scale: the result is exactly twice the first
    assert torch.equal(out.view(torch.int16), (outs[0] * 2).view(torch.int16))
    with pytest.raises(ValueError, match="prequantized weights"):
        mx.mx_grouped_mm(A, W, offs, weights=mx.mx_quantize_weights(W.detach()[:, :128].contiguous()))
