"""Grouped GEMMs for mixture-of-experts blocks on the GPU (Lesson 24,
sections 41-43): every expert's MLP over its packed rows in one launch per
GEMM, the expert found on the device from the offsets table.

Checked against the fp64 oracle per tensor at max|gpu - oracle| <= 1e-2 *
max|oracle| (the stacked dW1 [E, D, 2I] and dW_down [E, I, Dout] are one
tensor each), each expert's weight gradients also on their own when it has
at least 32 rows, and bitwise against the dense kernels run expert by
expert: the tile size does not change any element's accumulation order, so
the grouped launch must reproduce the per-expert launches exactly.  Experts
with no rows get zero weight gradients.

Why not every expert on its own: an expert's weight gradient is a sum over
its rows only, and with a handful of rows the bf16 rounding of the stored
preact and h does not average out.  An emulation of bf16 storage on the CPU
(exact products, RNE at each stored tensor) reaches 1.02e-2 against the fp64
oracle on a 10-row expert, so the per-tensor bound is the one that holds for
any correct bf16-storing implementation."""
import numpy as np
import pytest
import torch

import bwd_gemm_epilogue_amd as sw
import oracle
from gpu_util import assert_close, bits, to_dev, to_f64
from workload import MOE_WORKLOADS, MoEWorkload, bf16_bits_to_f64, make_moe_inputs

pytestmark = pytest.mark.gpu


def _custom(counts, D, I, Dout, seed):
    w = MoEWorkload("custom", 1, 1, len(counts), D, I, Dout, 1.0, 1 / np.sqrt(D), 1 / np.sqrt(I), 1.0, skew=1.0)
    return make_moe_inputs(w, seed=seed, counts=counts)


def _dev_inputs(xb, W1b, Wdb, dyb, off):
    return (to_dev(xb), to_dev(W1b), to_dev(Wdb), to_dev(dyb),
            torch.from_numpy(off.astype(np.int32)).cuda())


def _check_vs_oracle(xb, W1b, Wdb, dyb, off, pre, y, dx, dW1, dWd):
    E = W1b.shape[0]
    ref = oracle.moe_backward(bf16_bits_to_f64(xb), [bf16_bits_to_f64(W1b[e]) for e in range(E)],
                              [bf16_bits_to_f64(Wdb[e]) for e in range(E)], off, bf16_bits_to_f64(dyb))
    if xb.shape[0] > 0:
        assert_close("preact", to_f64(pre), ref["preact"])
        assert_close("y", to_f64(y), ref["y"])
        assert_close("dx", to_f64(dx), ref["dx"])
    g1, gd = to_f64(dW1), to_f64(dWd)
    assert_close("dW1", g1, ref["dW1"])
    assert_close("dW_down", gd, ref["dW_down"])
    for e in range(E):
        if off[e + 1] == off[e]:
            assert np.all(g1[e] == 0) and np.all(gd[e] == 0), e
        elif off[e + 1] - off[e] >= 32:
            assert_close(f"dW1[{e}]", g1[e], ref["dW1"][e])
            assert_close(f"dW_down[{e}]", gd[e], ref["dW_down"][e])


def _dense_per_expert(x, W1, Wd, dy, off):
    """The dense tiled kernels on each expert's rows, for the bitwise
    comparison (the forward by its two step kernels: at 16 rows or fewer the
    whole-forward call would take the split-K decode path instead)."""
    E = W1.shape[0]
    M, I, D, Dout = x.shape[0], Wd.shape[1], x.shape[1], Wd.shape[2]
    pre = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, Dout), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    dW1 = torch.empty((E, D, 2 * I), dtype=torch.bfloat16, device="cuda")
    dWd = torch.empty((E, I, Dout), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        p_e, h_e = sw.swiglu_fwd_gemm1(x[a:b], W1[e])
        y_e = sw.swiglu_fwd_down(h_e, Wd[e])
        dx_e, dW1[e], dWd[e] = sw.swiglu_mlp_bwd(x[a:b], W1[e], Wd[e], p_e, dy[a:b])
        pre[a:b], y[a:b], dx[a:b] = p_e, y_e, dx_e
    return pre, y, dx, dW1, dWd


CASES = [
    ("moe_tiny", None, None),
    ("ragged, empty and 1-row experts, 128-wide tiles", [0, 37, 300, 1, 0, 129], (192, 384, 128)),
    ("one expert", [211], (256, 256, 256)),
    ("64-wide tiles", [70, 0, 5, 190], (128, 320, 64)),
]


@pytest.mark.parametrize("name,counts,dims", CASES, ids=[c[0] for c in CASES])
def test_moe_vs_oracle_and_dense(name, counts, dims):
    print("case: moe", name, counts, dims, flush=True)
    if counts is None:
        xb, W1b, Wdb, dyb, off = make_moe_inputs(MOE_WORKLOADS[name], seed=51)
    else:
        xb, W1b, Wdb, dyb, off = _custom(counts, *dims, seed=53)
    x, W1, Wd, dy, offd = _dev_inputs(xb, W1b, Wdb, dyb, off)
    pre, y = sw.swiglu_moe_fwd(x, W1, Wd, offd)
    dx, dW1, dWd = sw.swiglu_moe_bwd(x, W1, Wd, offd, pre, dy)
    torch.cuda.synchronize()
    _check_vs_oracle(xb, W1b, Wdb, dyb, off, pre, y, dx, dW1, dWd)
    ref = _dense_per_expert(x, W1, Wd, dy, off)
    torch.cuda.synchronize()
    for a, b, n in zip((pre, y, dx, dW1, dWd), ref, ("preact", "y", "dx", "dW1", "dW_down")):
        assert np.array_equal(bits(a), bits(b)), n


@pytest.mark.parametrize("E", [64, 65, 150])
def test_moe_many_experts(E):
    """More experts than one wave scans at once (64 per pass): the device-side
    lookup walks several 64-expert chunks, with runs of empty experts."""
    print("case: moe experts", E, flush=True)
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 12, E) * (rng.random(E) < 0.6)
    counts[-1] = max(int(counts[-1]), 3)          # rows in the last chunk
    xb, W1b, Wdb, dyb, off = _custom(list(counts), 128, 128, 128, seed=59)
    x, W1, Wd, dy, offd = _dev_inputs(xb, W1b, Wdb, dyb, off)
    pre, y = sw.swiglu_moe_fwd(x, W1, Wd, offd)
    dx, dW1, dWd = sw.swiglu_moe_bwd(x, W1, Wd, offd, pre, dy)
    torch.cuda.synchronize()
    _check_vs_oracle(xb, W1b, Wdb, dyb, off, pre, y, dx, dW1, dWd)
    ref = _dense_per_expert(x, W1, Wd, dy, off)
    torch.cuda.synchronize()
    for a, b, n in zip((pre, y, dx, dW1, dWd), ref, ("preact", "y", "dx", "dW1", "dW_down")):
        assert np.array_equal(bits(a), bits(b)), n


def test_moe_dgrad_step_and_degenerate_tables():
    print("case: moe dgrad step, empty batch, everything in the last expert", flush=True)
    xb, W1b, Wdb, dyb, off = _custom([40, 0, 97], 256, 512, 256, seed=55)
    x, W1, Wd, dy, offd = _dev_inputs(xb, W1b, Wdb, dyb, off)
    pre, _ = sw.swiglu_moe_fwd(x, W1, Wd, offd)
    gp, h = sw.swiglu_moe_bwd_dgrad_fused(dy, Wd, offd, pre)
    for e in range(3):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        gp_e, h_e = sw.swiglu_bwd_dgrad_fused(dy[a:b], Wd[e], pre[a:b])
        assert np.array_equal(bits(gp[a:b]), bits(gp_e)) and np.array_equal(bits(h[a:b]), bits(h_e))
    # no rows at all: outputs of zero rows, zero weight gradients
    x0, dy0 = x[:0].contiguous(), dy[:0].contiguous()
    off0 = torch.zeros(4, dtype=torch.int32, device="cuda")
    pre0, y0 = sw.swiglu_moe_fwd(x0, W1, Wd, off0)
    dW1 = torch.full(W1.shape, 3.0, dtype=torch.bfloat16, device="cuda")
    dWd = torch.full(Wd.shape, 3.0, dtype=torch.bfloat16, device="cuda")
    sw.swiglu_moe_bwd(x0, W1, Wd, off0, pre0, dy0, dW1=dW1, dW_down=dWd)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW1).item() == 0 and torch.count_nonzero(dWd).item() == 0
    # all rows in the last expert: equal to the dense block with that expert's weights
    M = x.shape[0]
    offl = torch.tensor([0, 0, 0, M], dtype=torch.int32, device="cuda")
    pre_l, y_l = sw.swiglu_moe_fwd(x, W1, Wd, offl)
    pre_d, y_d = sw.swiglu_mlp_fwd(x, W1[2], Wd[2])
    torch.cuda.synchronize()
    assert np.array_equal(bits(pre_l), bits(pre_d)) and np.array_equal(bits(y_l), bits(y_d))


def test_moe_autograd_function():
    print("case: moe autograd", flush=True)
    xb, W1b, Wdb, dyb, off = _custom([33, 150, 0, 77], 256, 256, 256, seed=57)
    x, W1, Wd, dy, offd = _dev_inputs(xb, W1b, Wdb, dyb, off)
    xr, W1r, Wdr = (t.clone().requires_grad_(True) for t in (x, W1, Wd))
    y = sw.swiglu_moe(xr, W1r, Wdr, offd)
    assert len(y.grad_fn.saved_tensors) == 5
    y.backward(dy)
    pre, y2 = sw.swiglu_moe_fwd(x, W1, Wd, offd)
    dx, dW1, dWd = sw.swiglu_moe_bwd(x, W1, Wd, offd, pre, dy)
    for a, b in ((y, y2), (xr.grad, dx), (W1r.grad, dW1), (Wdr.grad, dWd)):
        assert np.array_equal(bits(a), bits(b))


def test_moe_workload_full_size_matches_dense_per_expert():
    """The MoE workload at its full size (16 experts, 16384 routed rows,
    D = 3584, I = 2048) in the grouped launches the benchmark times, bitwise
    against the per-expert dense launches, and against the fp64 oracle on
    sampled rows and channels of three experts."""
    w = MOE_WORKLOADS["moe"]
    print("case: moe full size", w, flush=True)
    xb, W1b, Wdb, dyb, off = make_moe_inputs(w, weight_sets=2)
    x, W1, Wd, dy, offd = _dev_inputs(xb, W1b, Wdb, dyb, off)
    pre, y = sw.swiglu_moe_fwd(x, W1, Wd, offd)
    dx, dW1, dWd = sw.swiglu_moe_bwd(x, W1, Wd, offd, pre, dy)
    ref = _dense_per_expert(x, W1, Wd, dy, off)
    torch.cuda.synchronize()
    for a, b, n in zip((pre, y, dx, dW1, dWd), ref, ("preact", "y", "dx", "dW1", "dW_down")):
        assert np.array_equal(bits(a), bits(b)), n
    assert torch.isfinite(y.float()).all() and torch.isfinite(dx.float()).all()
    # the fp64 oracle's exact sampled form on three experts (the smallest,
    # the median and the largest): 32 of their rows and 32 intermediate
    # channels, every output on them computed exactly; the per-tensor bound
    # over the sample
    counts = np.diff(off)
    order = np.argsort(counts)
    I = Wdb.shape[1]
    for e in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        a, b = int(off[e]), int(off[e + 1])
        rng = np.random.default_rng(100 + e)
        rows = np.sort(rng.choice(b - a, size=min(32, b - a), replace=False))
        chans = np.sort(rng.choice(I, size=32, replace=False))
        s = oracle.sampled_forward_backward(bf16_bits_to_f64(xb[a:b]), bf16_bits_to_f64(W1b[e]),
                                            bf16_bits_to_f64(Wdb[e]), bf16_bits_to_f64(dyb[a:b]), rows, chans)
        rt = torch.from_numpy(a + rows).cuda()
        c2 = torch.from_numpy(np.concatenate([chans, I + chans])).cuda()
        ct = torch.from_numpy(chans).cuda()
        print(f"expert {e}: {b - a} rows", flush=True)
        assert_close("preact rows", to_f64(pre.index_select(0, rt)), s["preact_rows"])
        assert_close("preact cols", to_f64(pre[a:b].index_select(1, c2)), s["preact_cols"])
        assert_close("y rows", to_f64(y.index_select(0, rt)), s["y_rows"])
        assert_close("dx rows", to_f64(dx.index_select(0, rt)), s["dx_rows"])
        assert_close("dW1 cols", to_f64(dW1[e].index_select(1, c2)), s["dW1_cols"])
        assert_close("dW_down rows", to_f64(dWd[e].index_select(0, ct)), s["dW_down_rows"])
