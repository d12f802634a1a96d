"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests retypes an oracle formula to compare it with itself:
each one checks the oracle against an independent fact (a library routine,
a closed form, an identity, brute force, finite differences or a number
printed on the pages).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import optimize, special

import oracle
from workload import WORKLOADS, bf16_bits_to_f64, make_custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def _grid():
    return np.concatenate([np.linspace(-60.0, 60.0, 4801), [0.0, 1e-3, -1e-3, 700.0, -700.0]])


# --------------------------------------------------------------- activations

def test_sigmoid_matches_library_expit():
    g = _grid()
    np.testing.assert_allclose(oracle.sigmoid(g), special.expit(g), rtol=1e-14, atol=0)


def test_silu_matches_library():
    g = _grid()
    np.testing.assert_allclose(oracle.silu(g), g * special.expit(g), rtol=1e-14, atol=1e-300)


def test_three_dsilu_forms_agree():
    # First page, section 2: the three forms of silu' are equal.
    g = _grid()
    f1, f2, f3 = oracle.dsilu_form1(g), oracle.dsilu_form2(g), oracle.dsilu_form3(g)
    scale = np.maximum(np.abs(f1), 1e-3)
    assert np.max(np.abs(f1 - f2) / scale) < 1e-13
    assert np.max(np.abs(f1 - f3) / scale) < 1e-13


def test_dsilu_is_derivative_of_silu():
    g = np.linspace(-20, 20, 2001)
    eps = 1e-5
    fd = (oracle.silu(g + eps) - oracle.silu(g - eps)) / (2 * eps)
    for f in (oracle.dsilu_form1, oracle.dsilu_form2, oracle.dsilu_form3):
        np.testing.assert_allclose(f(g), fd, atol=1e-9)


def test_closed_forms_at_zero():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    assert oracle.dsilu(0.0) == 0.5


def test_symmetries():
    # sigma(-g) = 1 - sigma(g) gives silu(g) - silu(-g) = g and
    # silu'(g) + silu'(-g) = 1 for every g.
    g = np.linspace(-30, 30, 3001)
    np.testing.assert_allclose(oracle.silu(g) - oracle.silu(-g), g, atol=1e-13)
    np.testing.assert_allclose(oracle.dsilu(g) + oracle.dsilu(-g), 1.0, atol=1e-14)


def test_dsilu_root_lambert_w():
    # silu'(g) = 0  <=>  1 + g + e^g = 0  <=>  g = -1 - W(1/e)
    u = special.lambertw(1.0 / math.e).real
    g_star = -1.0 - u
    assert abs(g_star - (-1.2784645427610738)) < 1e-12
    for f in (oracle.dsilu_form1, oracle.dsilu_form2, oracle.dsilu_form3):
        assert abs(f(g_star)) < 1e-15
    assert abs(oracle.silu(g_star) - (g_star + 1.0)) < 1e-15


def test_dsilu_extrema():
    # silu''(g) = 0  <=>  g * tanh(g / 2) = 2; the roots are the extrema of silu'.
    g_e = optimize.brentq(lambda g: g * math.tanh(g / 2) - 2.0, 1.0, 4.0, xtol=1e-15)
    grid = np.linspace(-6, 6, 1_200_001)
    d = oracle.dsilu(grid)
    assert abs(grid[np.argmin(d)] - (-g_e)) < 2e-5
    assert abs(grid[np.argmax(d)] - g_e) < 2e-5
    eps = 1e-5
    for g0 in (g_e, -g_e):
        slope = (oracle.dsilu(g0 + eps) - oracle.dsilu(g0 - eps)) / (2 * eps)
        assert abs(slope) < 1e-9
    assert -0.1 < oracle.dsilu(-g_e) < -0.099


def test_tails():
    # g -> -inf: sigma ~ e^g, silu' ~ (1 + g) e^g ; g -> +inf: silu' -> 1 + (g - 1) e^-g
    for g in (-30.0, -40.0):
        np.testing.assert_allclose(oracle.dsilu(g), (1 + g) * math.exp(g), rtol=1e-10)
        np.testing.assert_allclose(oracle.silu(g), g * math.exp(g), rtol=1e-10)
    for g in (20.0, 30.0):
        np.testing.assert_allclose(oracle.dsilu(g) - 1.0, (g - 1) * math.exp(-g), rtol=1e-2,
                                   atol=1e-16)
    # fp64 overflow of e^-g gives the exact limits
    assert oracle.sigmoid(-1000.0) == 0.0
    assert oracle.silu(1000.0) == 1000.0
    assert oracle.dsilu(1000.0) == 1.0


# --------------------------------------------------------------- whole MLP

def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _loss(x, W1, Wd, dy):
    _, _, y = oracle.forward(x, W1, Wd)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(seed)
    M, D, I, Dout = 5, 6, 7, 4
    x, W1, Wd, dy = (_rand((M, D), rng), _rand((D, 2 * I), rng, 0.7),
                     _rand((I, Dout), rng, 0.5), _rand((M, Dout), rng))
    g = oracle.backward(x, W1, Wd, dy)
    eps = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("W1", W1, g["dW1"]), ("Wd", Wd, g["dW_down"])):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            orig = arr[idx]
            arr[idx] = orig + eps
            lp = _loss(x, W1, Wd, dy)
            arr[idx] = orig - eps
            lm = _loss(x, W1, Wd, dy)
            arr[idx] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def _loss_residual(x, W1, Wd, dy):
    _, _, y = oracle.forward_residual(x, W1, Wd)
    return float(np.sum(y * dy))


def test_residual_block_matches_finite_differences():
    """Y = X + MLP(X) (Lesson 24, section 24): its gradients against central
    differences of <dy, Y>, and Y - X equal to the plain block's output."""
    rng = np.random.default_rng(3)
    M, D, I = 4, 6, 5
    x, W1, Wd, dy = (_rand((M, D), rng), _rand((D, 2 * I), rng, 0.7),
                     _rand((I, D), rng, 0.5), _rand((M, D), rng))
    g = oracle.backward_residual(x, W1, Wd, dy)
    _, _, y_plain = oracle.forward(x, W1, Wd)
    _, _, y_res = oracle.forward_residual(x, W1, Wd)
    assert np.allclose(y_res - x, y_plain, rtol=0, atol=1e-14)
    eps = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("W1", W1, g["dW1"]), ("Wd", Wd, g["dW_down"])):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            orig = arr[idx]
            arr[idx] = orig + eps
            lp = _loss_residual(x, W1, Wd, dy)
            arr[idx] = orig - eps
            lm = _loss_residual(x, W1, Wd, dy)
            arr[idx] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    with pytest.raises(ValueError):
        oracle.forward_residual(x, W1, _rand((I, D + 1), rng))


def test_stack_gradients_match_finite_differences():
    """The stacked blocks' chain rule (the drop-h report's 4-layer stack):
    every layer's weight gradients and the input gradient against central
    differences of <dy, Y> through three blocks."""
    rng = np.random.default_rng(5)
    M, D, I, L = 3, 5, 4, 3
    x = _rand((M, D), rng)
    layers = [(_rand((D, 2 * I), rng, 0.8), _rand((I, D), rng, 0.6)) for _ in range(L)]
    dy = _rand((M, D), rng)
    g = oracle.stack_backward(x, layers, dy)

    def loss():
        return float(np.sum(oracle.stack_forward(x, layers)[2][-1] * dy))

    assert np.array_equal(g["y"], oracle.stack_forward(x, layers)[2][-1])
    eps = 1e-6
    targets = [("x", x, g["dx"])]
    for l in range(L):
        targets += [(f"W1[{l}]", layers[l][0], g["dW1"][l]), (f"Wd[{l}]", layers[l][1], g["dW_down"][l])]
    for name, arr, grad in targets:
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            orig = arr[idx]
            arr[idx] = orig + eps
            lp = loss()
            arr[idx] = orig - eps
            lm = loss()
            arr[idx] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    with pytest.raises(ValueError):
        oracle.stack_forward(x, [(layers[0][0], _rand((I, D + 1), rng))])


def test_moe_gradients_match_finite_differences():
    """The mixture-of-experts block (Lesson 24, sections 41-42): every
    expert's weight gradients and the routed rows' dx against central
    differences of <dy, Y>, with an expert that receives no rows (zero
    gradients) and one that receives a single row."""
    rng = np.random.default_rng(11)
    D, I, Dout = 4, 3, 5
    counts = [2, 0, 3, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    M, E = int(off[-1]), len(counts)
    x, dy = _rand((M, D), rng), _rand((M, Dout), rng)
    W1s = [_rand((D, 2 * I), rng, 0.8) for _ in range(E)]
    Wds = [_rand((I, Dout), rng, 0.6) for _ in range(E)]
    g = oracle.moe_backward(x, W1s, Wds, off, dy)
    assert np.all(g["dW1"][1] == 0) and np.all(g["dW_down"][1] == 0)

    def loss():
        return float(np.sum(oracle.moe_forward(x, W1s, Wds, off)[2] * dy))

    eps = 1e-6
    targets = [("x", x, g["dx"])]
    for e in range(E):
        targets += [(f"W1[{e}]", W1s[e], g["dW1"][e]), (f"Wd[{e}]", Wds[e], g["dW_down"][e])]
    for name, arr, grad in targets:
        for _ in range(8):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            orig = arr[idx]
            arr[idx] = orig + eps
            lp = loss()
            arr[idx] = orig - eps
            lm = loss()
            arr[idx] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    for bad in ([0, 2, 2, 5, 5], [0, 3, 2, 5, 6], [1, 2, 2, 5, 6]):
        with pytest.raises(ValueError):
            oracle.moe_forward(x, W1s, Wds, bad)


def test_moe_with_one_expert_is_the_dense_block():
    rng = np.random.default_rng(13)
    M, D, I, Dout = 5, 4, 3, 2
    x, W1, Wd, dy = _rand((M, D), rng), _rand((D, 2 * I), rng), _rand((I, Dout), rng), _rand((M, Dout), rng)
    g = oracle.moe_backward(x, [W1], [Wd], [0, M], dy)
    r = oracle.backward(x, W1, Wd, dy)
    for k in ("y", "dx", "grad_preact"):
        assert np.array_equal(g[k], r[k])
    assert np.array_equal(g["dW1"][0], r["dW1"]) and np.array_equal(g["dW_down"][0], r["dW_down"])


def test_grad_preact_matches_finite_differences():
    rng = np.random.default_rng(7)
    M, I, Dout = 4, 6, 3
    P = _rand((M, 2 * I), rng, 2.0)
    Wd = _rand((I, Dout), rng)
    dy = _rand((M, Dout), rng)
    dout = dy @ Wd.T
    gp, h = oracle.swiglu_bwd_elementwise(P, dout)

    def loss(P):
        return float(np.sum((oracle.swiglu_fwd_elementwise(P) @ Wd) * dy))

    eps = 1e-6
    for m in range(M):
        for j in range(2 * I):
            Pp, Pm = P.copy(), P.copy()
            Pp[m, j] += eps
            Pm[m, j] -= eps
            fd = (loss(Pp) - loss(Pm)) / (2 * eps)
            assert abs(fd - gp[m, j]) < 1e-7 * max(1.0, abs(fd))


def _brute_force(x, W1, Wd, dy):
    """Pure-Python loops over tiny shapes, with math.exp for the sigmoid."""
    M, D = len(x), len(x[0])
    I = len(W1[0]) // 2
    Dout = len(Wd[0])
    P = [[sum(x[m][d] * W1[d][j] for d in range(D)) for j in range(2 * I)] for m in range(M)]
    sig = [[1.0 / (1.0 + math.exp(-P[m][I + i])) for i in range(I)] for m in range(M)]
    h = [[P[m][i] * P[m][I + i] * sig[m][i] for i in range(I)] for m in range(M)]
    y = [[sum(h[m][i] * Wd[i][o] for i in range(I)) for o in range(Dout)] for m in range(M)]
    dout = [[sum(dy[m][o] * Wd[i][o] for o in range(Dout)) for i in range(I)] for m in range(M)]
    gp = [[0.0] * (2 * I) for _ in range(M)]
    for m in range(M):
        for i in range(I):
            g, s = P[m][I + i], sig[m][i]
            gp[m][i] = dout[m][i] * g * s
            gp[m][I + i] = dout[m][i] * P[m][i] * (s + g * s * (1 - s))
    dx = [[sum(gp[m][j] * W1[d][j] for j in range(2 * I)) for d in range(D)] for m in range(M)]
    dW1 = [[sum(x[m][d] * gp[m][j] for m in range(M)) for j in range(2 * I)] for d in range(D)]
    dWd = [[sum(h[m][i] * dy[m][o] for m in range(M)) for o in range(Dout)] for i in range(I)]
    return dict(preact=P, h=h, y=y, dout=dout, grad_preact=gp, dx=dx, dW1=dW1, dW_down=dWd)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    M, D, I, Dout = 3, 4, 5, 2
    x, W1, Wd, dy = (_rand((M, D), rng), _rand((D, 2 * I), rng),
                     _rand((I, Dout), rng), _rand((M, Dout), rng))
    ref = _brute_force(x.tolist(), W1.tolist(), Wd.tolist(), dy.tolist())
    got = oracle.backward(x, W1, Wd, dy)
    for k, v in ref.items():
        np.testing.assert_allclose(got[k], np.array(v), rtol=1e-12, atol=1e-12, err_msg=k)


def test_brute_force_on_bf16_workload_rows():
    # the tiny workload's exact bf16 inputs, restricted to 2 tokens and 6 channels
    x, W1, Wd, dy = (bf16_bits_to_f64(a) for a in make_custom(2, 8, 6, 4, seed=99))
    ref = _brute_force(x.tolist(), W1.tolist(), Wd.tolist(), dy.tolist())
    got = oracle.backward(x, W1, Wd, dy)
    for k, v in ref.items():
        np.testing.assert_allclose(got[k], np.array(v), rtol=1e-12, atol=1e-12, err_msg=k)


def test_gate_zero_closed_form():
    rng = np.random.default_rng(11)
    M, D, I, Dout = 6, 5, 4, 3
    x, W1, Wd, dy = (_rand((M, D), rng), _rand((D, 2 * I), rng),
                     _rand((I, Dout), rng), _rand((M, Dout), rng))
    W1[:, I:] = 0.0
    g = oracle.backward(x, W1, Wd, dy)
    left = x @ W1[:, :I]
    dout = dy @ Wd.T
    assert np.all(g["h"] == 0) and np.all(g["y"] == 0) and np.all(g["dW_down"] == 0)
    assert np.all(g["grad_preact"][:, :I] == 0)
    np.testing.assert_allclose(g["grad_preact"][:, I:], 0.5 * dout * left, rtol=1e-14)
    assert np.all(g["dx"] == 0)
    assert np.all(g["dW1"][:, :I] == 0)
    np.testing.assert_allclose(g["dW1"][:, I:], 0.5 * x.T @ (dout * left), rtol=1e-13)


def test_large_gate_is_bilinear():
    # gate >= 40 everywhere: sigma = 1 to 4e-18, so h = left * gate,
    # dleft = dout * gate and dgate = dout * left.
    rng = np.random.default_rng(5)
    M, D, I, Dout = 4, 3, 5, 2
    x = np.abs(_rand((M, D), rng)) + 1.0
    W1 = _rand((D, 2 * I), rng)
    W1[:, I:] = np.abs(W1[:, I:]) + 20.0
    Wd, dy = _rand((I, Dout), rng), _rand((M, Dout), rng)
    g = oracle.backward(x, W1, Wd, dy)
    left, gate = x @ W1[:, :I], x @ W1[:, I:]
    assert gate.min() > 40
    dout = dy @ Wd.T
    np.testing.assert_allclose(g["h"], left * gate, rtol=1e-15)
    np.testing.assert_allclose(g["grad_preact"][:, :I], dout * gate, rtol=1e-15)
    np.testing.assert_allclose(g["grad_preact"][:, I:], dout * left, rtol=1e-14)


def test_frobenius_invariants():
    # <dW_down, W_down> = <dy, y> and <dx, x> = <dW1, W1> = <grad_preact, preact>
    rng = np.random.default_rng(2)
    M, D, I, Dout = 9, 7, 6, 5
    x, W1, Wd, dy = (_rand((M, D), rng), _rand((D, 2 * I), rng),
                     _rand((I, Dout), rng), _rand((M, Dout), rng))
    g = oracle.backward(x, W1, Wd, dy)
    a = np.sum(g["dW_down"] * Wd)
    np.testing.assert_allclose(a, np.sum(dy * g["y"]), rtol=1e-12)
    b = np.sum(g["grad_preact"] * g["preact"])
    np.testing.assert_allclose(np.sum(g["dx"] * x), b, rtol=1e-12)
    np.testing.assert_allclose(np.sum(g["dW1"] * W1), b, rtol=1e-12)


def test_sampled_oracle_equals_full():
    x, W1, Wd, dy = (bf16_bits_to_f64(a) for a in make_custom(40, 32, 24, 16, seed=5))
    full = oracle.backward(x, W1, Wd, dy)
    rows = np.array([0, 3, 17, 39])
    chans = np.array([1, 5, 23])
    s = oracle.sampled_forward_backward(x, W1, Wd, dy, rows, chans)
    I = 24
    cols2 = np.concatenate([chans, I + chans])
    np.testing.assert_allclose(s["y_rows"], full["y"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["dx_rows"], full["dx"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["preact_rows"], full["preact"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["grad_preact_rows"], full["grad_preact"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["preact_cols"], full["preact"][:, cols2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["h_cols"], full["h"][:, chans], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["grad_preact_cols"], full["grad_preact"][:, cols2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["dW1_cols"], full["dW1"][:, cols2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["dW_down_rows"], full["dW_down"][chans], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- ledgers

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_flop_ledger_matches_pages():
    gold = _golden()["flop_ledger_GF"]
    # the page's own ledger is consistent: 116+116+232+232 = 696 = 2 x 348
    assert gold["dout"] + gold["dW_down"] + gold["dx"] + gold["dW"] == gold["backward_total"]
    assert gold["backward_total"] == 2 * gold["forward_total"]
    for shape in [(128, 256, 512, 256), (11136, 3584, 14336, 3584), (17, 64, 192, 128)]:
        f = oracle.gemm_flops(*shape)
        assert f["backward"] == 2 * f["forward"]
        assert f["dout"] == f["dW_down"] and f["dx"] == f["dW1"]
        M, D, I, Dout = shape
        assert f["forward"] == 4 * M * D * I + 2 * M * I * Dout
    # with Dout = D the page's 1:1:2:2 split holds
    f = oracle.gemm_flops(11136, 3584, 14336, 3584)
    assert f["dx"] == 2 * f["dout"]
    assert gold["dx"] == 2 * gold["dout"]
    assert f["forward"] == 6 * 11136 * 3584 * 14336


def test_byte_ledger_matches_pages():
    gold = _golden()["byte_ledger_MB"]
    # preact is twice dout's size, grad_preact too, and fusion removes the
    # dout round trip (write + read)
    assert gold["de_read"] == 2 * gold["dout_write"] == gold["grad_de_write"]
    assert gold["round_trip_removed"] == gold["dout_write"] + gold["dout_read"]
    M, D, I, Dout = 1000, 256, 768, 256
    b = oracle.algorithmic_bytes(M, D, I, Dout)
    assert b["saved"] == 2 * (2 * M * I)
    assert b["unfused_dgrad"] - b["fused_dgrad"] == b["saved"]


def test_drop_h_memory_saving_is_one_h():
    gold = _golden()["drop_h_memory_MiB"]
    M, D, H, Dout = gold["shape_M_D_H_Dout"]
    w = WORKLOADS["target"]
    assert (w.M, w.D, w.I, w.Dout) == (M, D, H, Dout)
    assert M * H * 2 / 2**20 == gold["saving"]
    assert abs(gold["after_forward_normal"] - gold["after_forward_drop_h"] - gold["saving"]) < 1e-9
    stack = _golden()["drop_h_stack_MiB"]
    assert abs(stack["after_forward_normal"] - stack["after_forward_drop_h"]
               - stack["layers"] * gold["saving"]) < 1e-9


def _ledger_arrays(M, D, I, Dout, seed=3):
    """The arrays each step reads and writes, as the oracle's own step
    functions take and return them (every dimension distinct, so that a
    term with a wrong or swapped dimension changes the count)."""
    rng = np.random.default_rng(seed)
    x, W1, Wd, dy = (rng.standard_normal(s) for s in ((M, D), (D, 2 * I), (I, Dout), (M, Dout)))
    pre, h, y = oracle.forward(x, W1, Wd)
    dout = dy @ Wd.T
    gp, h_bwd = oracle.swiglu_bwd_elementwise(pre, dout)
    fused = [dy, Wd, pre, gp, h_bwd]                # reads dy, W_down, preact; writes grad_preact, h
    forward = [x, W1, Wd, pre, y, h, h]             # h written once and read once
    return fused, forward, dout


def test_byte_ledger_totals_count_the_tensors_each_step_moves():
    """algorithmic_bytes totals against an independent count: the bf16 sizes
    of the arrays the oracle's own step functions read and write."""
    M, D, I, Dout = 97, 64, 160, 48
    fused, forward, dout = _ledger_arrays(M, D, I, Dout)
    b = oracle.algorithmic_bytes(M, D, I, Dout)
    assert b["fused_dgrad"] == 2 * sum(a.size for a in fused)
    assert b["forward"] == 2 * sum(a.size for a in forward)
    assert b["unfused_dgrad"] == b["fused_dgrad"] + 2 * 2 * dout.size   # dout written and read back
    assert b["saved"] == 2 * 2 * dout.size
