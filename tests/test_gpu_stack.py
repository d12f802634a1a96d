"""The stacked-blocks workload on the GPU (the drop-h report's 4-layer
stack): parity of the whole stack with the oracle's chain rule, the autograd
stack bitwise equal to the same blocks chained by hand through the C ABI, the
drop-h and save-h stacks bitwise equal, and the after-forward memory of each
exactly its saved tensors, so that dropping h saves L * M * I * 2 bytes.

Tolerance.  One block meets max|gpu - oracle| <= 1e-2 * max|oracle| per
output.  In a stack each block reads the previous block's bf16 output, so
the roundings compound: a tensor that depends on a chain of k block
evaluations (forward or backward) is held to k * 1e-2.  The stack output y
follows L forward evaluations; dW of layer l follows L forward and L - l
backward ones (dy reaches layer l through the backward of layers L-1..l);
dx follows 2L.  A chaining mistake (a wrong dy or saved input) is an O(1)
error and fails these bounds."""
import numpy as np
import pytest
import torch

import bwd_gemm_epilogue_amd as sw
import oracle
from gpu_util import assert_close, bits, to_dev, to_f64
from workload import bf16_bits_to_f64, make_custom

pytestmark = pytest.mark.gpu


def _stack_inputs(L, M, D, I, seed):
    x, _, _, dy = make_custom(M, D, I, D, seed=seed)
    ws = [make_custom(M, D, I, D, seed=seed + 101 * (l + 1))[1:3] for l in range(L)]
    return x, dy, ws


def _leaf(t):
    return t.clone().requires_grad_(True)


@pytest.mark.parametrize("shape", [(4, 256, 512, 768), (4, 333, 256, 512)])
def test_stack_vs_oracle(shape):
    L, M, D, I = shape
    print("case: stack vs oracle", shape, flush=True)
    xb, dyb, wb = _stack_inputs(L, M, D, I, seed=41)
    x = _leaf(to_dev(xb))
    layers = [(_leaf(to_dev(a)), _leaf(to_dev(b))) for a, b in wb]
    y = sw.swiglu_mlp_stack(x, layers)
    y.backward(to_dev(dyb))
    torch.cuda.synchronize()
    ref = oracle.stack_backward(bf16_bits_to_f64(xb), [(bf16_bits_to_f64(a), bf16_bits_to_f64(b)) for a, b in wb],
                                bf16_bits_to_f64(dyb))
    errs = {"y": assert_close("y", to_f64(y), ref["y"], tol=L * 1e-2),
            "dx": assert_close("dx", to_f64(x.grad), ref["dx"], tol=2 * L * 1e-2)}
    for l in range(L):
        errs[f"dW1[{l}]"] = assert_close(f"dW1[{l}]", to_f64(layers[l][0].grad), ref["dW1"][l], tol=(2 * L - l) * 1e-2)
        errs[f"dW_down[{l}]"] = assert_close(f"dW_down[{l}]", to_f64(layers[l][1].grad), ref["dW_down"][l],
                                             tol=(2 * L - l) * 1e-2)
    print(" ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    # the same blocks chained by hand through the C ABI: bitwise equal
    xs, pres = [x.detach()], []
    for W1, Wd in layers:
        pre, yl = sw.swiglu_mlp_fwd(xs[-1], W1.detach(), Wd.detach())
        pres.append(pre)
        xs.append(yl)
    assert np.array_equal(bits(xs[-1]), bits(y))
    g = to_dev(dyb)
    for l in range(L - 1, -1, -1):
        g, dW1, dWd = sw.swiglu_mlp_bwd(xs[l], layers[l][0].detach(), layers[l][1].detach(), pres[l], g)
        assert np.array_equal(bits(dW1), bits(layers[l][0].grad))
        assert np.array_equal(bits(dWd), bits(layers[l][1].grad))
    assert np.array_equal(bits(g), bits(x.grad))


def test_stack_memory_and_save_h_equivalence():
    L, M, D, I = 4, 512, 256, 768
    print("case: stack memory", (L, M, D, I), flush=True)
    xb, dyb, wb = _stack_inputs(L, M, D, I, seed=43)
    dy = to_dev(dyb)
    after, outs = {}, {}
    for save_h in (False, True):
        x = _leaf(to_dev(xb))
        layers = [(_leaf(to_dev(a)), _leaf(to_dev(b))) for a, b in wb]
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        y = sw.swiglu_mlp_stack(x, layers, save_h=save_h)
        torch.cuda.synchronize()
        after[save_h] = torch.cuda.memory_allocated() - base
        y.backward(dy)
        torch.cuda.synchronize()
        outs[save_h] = [bits(y), bits(x.grad)] + [bits(w.grad) for pair in layers for w in pair]
        del y, x, layers
    # after the forward each block holds preact [M,2I] and its output [M,D]
    # (the next block's saved input); the save-h stack also holds h [M,I]
    assert after[False] == L * (M * 2 * I * 2 + M * D * 2)
    assert after[True] - after[False] == L * M * I * 2
    for a, b in zip(outs[False], outs[True]):
        assert np.array_equal(a, b)


def test_stack_rejects_mismatched_widths():
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros((256, 1024), dtype=torch.bfloat16, device="cuda")
    Wd = torch.zeros((512, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sw.swiglu_mlp_stack(x, [(W1, Wd)])
