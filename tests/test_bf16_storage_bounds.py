"""Where the stack and per-expert tolerances of the GPU tests come from: an
emulation of bf16 storage on the CPU.

The GPU path stores preact, h, y, grad_preact and every gradient in bf16
(round to nearest even) and keeps dout in fp32 on chip.  The emulation below
uses exact (fp64) products and sums and rounds each tensor to bf16 exactly
where the GPU path stores it:

  forward:  preact = rn(x W1), h = rn(left * silu(gate)) from the rounded
            preact, y = rn(h W_down);
  backward: dout = dy W_down^T (not rounded), grad_preact = rn([dout silu(gate)
            | dout left silu'(gate)]), h = rn(left silu(gate)),
            dW_down = rn(h^T dy), dx = rn(grad_preact W1^T),
            dW1 = rn(x^T grad_preact);

and a stack of blocks feeds each block the previous block's rounded output
(and, backward, the next block's rounded dx).  It is not the GPU path (no
fp32 accumulation order, no kernels): it isolates the error that bf16
storage alone causes, which any correct implementation that stores these
tensors in bf16 carries.  Against the fp64 oracle it shows:

  * one block: every tensor within the per-tensor bound 1e-2 (the bound is
    attainable by a bf16-storing implementation);
  * the 4-block stacks of the GPU stack test: the roundings compound, some
    gradients pass 1e-2, and every tensor stays within the chain bound that
    test applies (k * 1e-2 for a tensor behind k block evaluations: y after
    L forward ones, dW of layer l after L forward and L - l backward ones,
    dx after 2L);
  * experts: an expert's own weight gradient is a sum over its rows only.
    Over the 64 experts of 0 to 11 rows in the GPU expert test, the worst
    (a 10-row expert) reaches 1.02e-2, past 1e-2; the experts of 32 rows
    and more in the tested cases stay within it.  That test holds experts of
    fewer than 32 rows to the stacked per-tensor bound only (which holds
    here too), and every expert bitwise to the dense kernels.
"""
import numpy as np
import pytest

import oracle
from workload import MoEWorkload, bf16_bits_to_f64, make_custom, make_moe_inputs, round_to_bf16_bits


def rn(a):
    """Round to bf16 (via fp32, as the GPU rounds its fp32 values) and back."""
    return bf16_bits_to_f64(round_to_bf16_bits(np.asarray(a, dtype=np.float64).astype(np.float32)))


def rel(got, ref):
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def emu_forward(x, W1, Wd):
    pre = rn(x @ W1)
    h = rn(oracle.swiglu_fwd_elementwise(pre))
    return pre, h, rn(h @ Wd)


def emu_backward(x, W1, Wd, pre, dy):
    gp, h = oracle.swiglu_bwd_elementwise(pre, dy @ Wd.T)
    gp, h = rn(gp), rn(h)
    return rn(gp @ W1.T), rn(x.T @ gp), rn(h.T @ dy)


def _block(M, D, I, Dout, seed):
    return [bf16_bits_to_f64(a) for a in make_custom(M, D, I, Dout, seed=seed)]


@pytest.mark.parametrize("shape", [(128, 256, 512, 256), (300, 512, 768, 512), (2048, 1024, 2816, 1024)])
def test_one_block_meets_the_per_tensor_bound(shape):
    x, W1, Wd, dy = _block(*shape, seed=7)
    ref = oracle.backward(x, W1, Wd, dy)
    pre, h, y = emu_forward(x, W1, Wd)
    dx, dW1, dWd = emu_backward(x, W1, Wd, pre, dy)
    errs = {"preact": rel(pre, ref["preact"]), "y": rel(y, ref["y"]), "dx": rel(dx, ref["dx"]),
            "dW1": rel(dW1, ref["dW1"]), "dW_down": rel(dWd, ref["dW_down"])}
    print(shape, {k: f"{v:.2e}" for k, v in errs.items()})
    assert max(errs.values()) <= 1e-2


# the GPU stack test's shapes and inputs: (L, M, D, I), seed 41, layer l's
# weights drawn with seed 41 + 101 * (l + 1)
@pytest.mark.parametrize("shape", [(4, 256, 512, 768), (4, 333, 256, 512)])
def test_stack_errors_compound_within_the_chain_bound(shape):
    L, M, D, I = shape
    xb, _, _, dyb = make_custom(M, D, I, D, seed=41)
    layers = [[bf16_bits_to_f64(a) for a in make_custom(M, D, I, D, seed=41 + 101 * (l + 1))[1:3]] for l in range(L)]
    x, dy = bf16_bits_to_f64(xb), bf16_bits_to_f64(dyb)
    ref = oracle.stack_backward(x, layers, dy)
    xs, pres = [x], []
    for W1, Wd in layers:
        pre, _, y = emu_forward(xs[-1], W1, Wd)
        pres.append(pre)
        xs.append(y)
    g = dy
    dW1s, dWds = [None] * L, [None] * L
    for l in range(L - 1, -1, -1):
        g, dW1s[l], dWds[l] = emu_backward(xs[l], *layers[l], pres[l], g)
    errs = {"y": (rel(xs[-1], ref["y"]), L), "dx": (rel(g, ref["dx"]), 2 * L)}
    for l in range(L):
        errs[f"dW1[{l}]"] = (rel(dW1s[l], ref["dW1"][l]), 2 * L - l)
        errs[f"dW_down[{l}]"] = (rel(dWds[l], ref["dW_down"][l]), 2 * L - l)
    print(shape, {k: f"{e:.2e} (bound {k_ * 1e-2:g})" for k, (e, k_) in errs.items()})
    for k, (e, chain) in errs.items():
        assert e <= chain * 1e-2, (k, e, chain)
    # the single-block bound does not survive the chain
    assert max(e for e, _ in errs.values()) > 1e-2


def _expert_errors(counts, dims, seed):
    D, I, Dout = dims
    w = MoEWorkload("custom", 1, 1, len(counts), D, I, Dout, 1.0, 1 / np.sqrt(D), 1 / np.sqrt(I), 1.0, skew=1.0)
    xb, W1b, Wdb, dyb, off = make_moe_inputs(w, seed=seed, counts=list(counts))
    x, dy = bf16_bits_to_f64(xb), bf16_bits_to_f64(dyb)
    E = len(counts)
    W1s = [bf16_bits_to_f64(W1b[e]) for e in range(E)]
    Wds = [bf16_bits_to_f64(Wdb[e]) for e in range(E)]
    ref = oracle.moe_backward(x, W1s, Wds, off, dy)
    dW1 = np.zeros_like(ref["dW1"])
    dWd = np.zeros_like(ref["dW_down"])
    per = {}
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        pre, _, _ = emu_forward(x[a:b], W1s[e], Wds[e])
        _, dW1[e], dWd[e] = emu_backward(x[a:b], W1s[e], Wds[e], pre, dy[a:b])
        per[e] = (b - a, max(rel(dW1[e], ref["dW1"][e]), rel(dWd[e], ref["dW_down"][e])))
    stacked = max(rel(dW1, ref["dW1"]), rel(dWd, ref["dW_down"]))
    return per, stacked


def test_expert_gradients_many_small_experts():
    """The 64-expert case of the GPU expert test (0 to 11 rows per expert,
    128 x 128 x 128, seed 59): bf16 storage alone takes a 10-row expert's
    own weight gradient to 1.02e-2, past 1e-2, while the stacked per-tensor
    bound over [E, D, 2I] and [E, I, Dout] holds.  That test therefore holds
    experts of fewer than 32 rows to the stacked bound only."""
    E = 64
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 12, E) * (rng.random(E) < 0.6)
    counts[-1] = max(int(counts[-1]), 3)
    per, stacked = _expert_errors(counts, (128, 128, 128), seed=59)
    worst_e = max(per, key=lambda e: per[e][1])
    print(f"stacked {stacked:.2e}; worst expert {worst_e}: {per[worst_e][0]} rows, {per[worst_e][1]:.2e}")
    assert stacked <= 1e-2
    assert per[worst_e][1] > 1e-2 and per[worst_e][0] < 32


@pytest.mark.parametrize("counts,dims", [([0, 37, 300, 1, 0, 129], (192, 384, 128)), ([211], (256, 256, 256)),
                                         ([32, 40, 64, 100, 500], (256, 512, 256))])
def test_expert_gradients_of_32_rows_and_more(counts, dims):
    """Experts of 32 rows and more meet 1e-2 on their own weight gradients
    (the GPU expert test's cases with such experts, and more)."""
    per, stacked = _expert_errors(counts, dims, seed=53)
    print({f"{n} rows": f"{v:.2e}" for n, v in per.values()}, f"stacked {stacked:.2e}")
    assert stacked <= 1e-2
    assert all(v <= 1e-2 for n, v in per.values() if n >= 32)
