"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Shapes here are ones the full oracle finishes in seconds; they span several
tiles of every kernel configuration and ragged token counts.  Tolerance: the
per-tensor bound max|gpu - oracle| <= 1e-2 * max|oracle|; the elementwise
activation values within 2 bf16 ulp of the oracle.
"""
import numpy as np
import pytest
import torch

import bwd_gemm_epilogue_amd as sw
import oracle
from gpu_util import assert_close, assert_ulp, bits, to_dev, to_f64, ulp_bf16
from workload import WORKLOADS, bf16_bits_to_f64, make_custom, make_inputs, round_to_bf16_bits

pytestmark = pytest.mark.gpu

# (M, D, I, Dout): tiny workload, ragged token counts, and shapes that select
# the 128- and 64-wide tile configurations (I % 128 != 0, Dout = 64)
SHAPES = [
    (128, 256, 512, 256),
    (200, 256, 512, 256),
    (1, 256, 512, 256),
    (300, 512, 768, 512),
    (96, 192, 320, 64),
    (333, 320, 192, 128),
]


def _case(*a):
    print("case:", *a, flush=True)


def _inputs(M, D, I, Dout, seed=7, **kw):
    x, W1, Wd, dy = make_custom(M, D, I, Dout, seed=seed, **kw)
    return (x, W1, Wd, dy), tuple(to_dev(a) for a in (x, W1, Wd, dy)), \
        tuple(bf16_bits_to_f64(a) for a in (x, W1, Wd, dy))


def test_act_eval_all_finite_bf16():
    _case("act_eval exhaustive")
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f64(allbits)
    g_bits = allbits[np.isfinite(f)]
    g = bf16_bits_to_f64(g_bits)
    s, si, ds = sw.swiglu_act_eval(to_dev(g_bits))
    torch.cuda.synchronize()
    s, si, ds = (t.cpu().numpy().astype(np.float64) for t in (s, si, ds))
    u1 = assert_ulp("sigma", s, oracle.sigmoid(g))
    u2 = assert_ulp("silu", si, oracle.silu(g))
    u3 = assert_ulp("silu'", ds, oracle.dsilu(g))
    print(f"max bf16 ulps: sigma {u1:.4f} silu {u2:.4f} dsilu {u3:.4f}")


def test_elementwise_kernel_2ulp():
    _case("elementwise 2ulp")
    rng = np.random.default_rng(3)
    M, I = 96, 512
    pre = rng.standard_normal((M, 2 * I)).astype(np.float32) * 4
    pre[0, I:I + 64] = np.linspace(-100, 100, 64)            # saturation of sigma
    pre[1, I:I + 8] = [-1.28125, -1.2734375, 0.0, -0.0, 88.0, -88.0, 1e-30, -1e-30]
    d = rng.standard_normal((M, I)).astype(np.float32)
    pb, db = round_to_bf16_bits(pre), round_to_bf16_bits(d)
    gp, h = sw.swiglu_bwd_elementwise(to_dev(pb), to_dev(db))
    ref_gp, ref_h = oracle.swiglu_bwd_elementwise(bf16_bits_to_f64(pb), bf16_bits_to_f64(db))
    assert_ulp("grad_preact", to_f64(gp), ref_gp)
    assert_ulp("h", to_f64(h), ref_h)


@pytest.mark.parametrize("shape", SHAPES)
def test_step_kernels(shape):
    M, D, I, Dout = shape
    _case("steps", shape)
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout)
    # forward GEMM-1 + SwiGLU epilogue
    pre, h = sw.swiglu_fwd_gemm1(x, W1)
    P = xf @ W1f
    assert_close("preact", to_f64(pre), P)
    # h is computed from the stored bf16 preact: within 2 ulp of the oracle on those bits
    assert_ulp("h(fwd)", to_f64(h), oracle.swiglu_fwd_elementwise(to_f64(pre)))
    # down GEMM on the GPU's h
    y = sw.swiglu_fwd_down(h, Wd)
    assert_close("y", to_f64(y), to_f64(h) @ Wdf)
    # fused dgrad epilogue on the GPU's preact
    gp, h2 = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    dout = dyf @ Wdf.T
    ref_gp, ref_h = oracle.swiglu_bwd_elementwise(to_f64(pre), dout)
    assert_close("grad_preact(fused)", to_f64(gp), ref_gp)
    assert_ulp("h(bwd)", to_f64(h2), ref_h)
    # forward h and backward-recomputed h are bitwise identical
    assert np.array_equal(bits(h), bits(h2)), "h_fwd != h_bwd"
    # plain dgrad GEMM
    dgp = sw.swiglu_bwd_dgrad_plain(dy, Wd)
    assert_close("dout(plain)", to_f64(dgp), dout)
    # remaining GEMMs on the GPU's own intermediate tensors
    dWd = sw.swiglu_bwd_dw_down(h2, dy)
    assert_close("dW_down", to_f64(dWd), to_f64(h2).T @ dyf)
    dx = sw.swiglu_bwd_dx(gp, W1)
    assert_close("dx", to_f64(dx), to_f64(gp) @ W1f.T)
    dW1 = sw.swiglu_bwd_dw1(x, gp)
    assert_close("dW1", to_f64(dW1), xf.T @ to_f64(gp))


@pytest.mark.parametrize("shape", SHAPES[:4] + [(2048, 1024, 2816, 1024)])
@pytest.mark.parametrize("fused", [True, False])
def test_whole_step_vs_oracle(shape, fused):
    M, D, I, Dout = shape
    _case("whole step", shape, "fused" if fused else "unfused")
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout, seed=11)
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    fn = sw.swiglu_mlp_bwd if fused else sw.swiglu_mlp_bwd_unfused
    dx, dW1, dWd = fn(x, W1, Wd, pre, dy)
    ref = oracle.backward(xf, W1f, Wdf, dyf)
    assert_close("preact", to_f64(pre), ref["preact"])
    assert_close("y", to_f64(y), ref["y"])
    assert_close("dx", to_f64(dx), ref["dx"])
    assert_close("dW1", to_f64(dW1), ref["dW1"])
    assert_close("dW_down", to_f64(dWd), ref["dW_down"])


@pytest.mark.parametrize("shape", [(1, 256, 512, 256), (7, 512, 768, 512), (13, 320, 192, 128),
                                   (16, 1024, 2816, 1024), (16, 192, 320, 64)])
def test_decode_forward_vs_oracle(shape):
    """At most 16 token rows the forward runs the split-K weight-streaming
    path (the last shape, Dout = 64, falls back to the tiled one): preact and
    y against the full oracle, and preact against the tiled GEMM-1."""
    M, D, I, Dout = shape
    _case("decode forward", shape)
    _, (x, W1, Wd, _), (xf, W1f, Wdf, _) = _inputs(M, D, I, Dout, seed=17)
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    pre_t, _ = sw.swiglu_fwd_gemm1(x, W1)
    torch.cuda.synchronize()
    P, _, Y = oracle.forward(xf, W1f, Wdf)
    assert_close("preact", to_f64(pre), P)
    assert_close("y", to_f64(y), Y)
    assert_close("preact skinny vs tiled", to_f64(pre), to_f64(pre_t))


def test_small_workload_full_oracle():
    w = WORKLOADS["small"]
    _case("small workload", w)
    xb, W1b, Wdb, dyb = make_inputs(w)
    x, W1, Wd, dy = (to_dev(a) for a in (xb, W1b, Wdb, dyb))
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)
    ref = oracle.backward(*(bf16_bits_to_f64(a) for a in (xb, W1b, Wdb, dyb)))
    for name, got in (("preact", pre), ("y", y), ("dx", dx), ("dW1", dW1), ("dW_down", dWd)):
        e = assert_close(name, to_f64(got), ref[name])
        print(f"{name}: rel err {e:.2e}")


def test_fused_matches_unfused_closely():
    M, D, I, Dout = 256, 256, 512, 256
    _case("fused vs unfused", (M, D, I, Dout))
    _, (x, W1, Wd, dy), _ = _inputs(M, D, I, Dout, seed=5)
    pre, _ = sw.swiglu_mlp_fwd(x, W1, Wd)
    gp_f, h_f = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    dout = sw.swiglu_bwd_dgrad_plain(dy, Wd)
    gp_u, h_u = sw.swiglu_bwd_elementwise(pre, dout)
    # h does not depend on dout: identical bits
    assert np.array_equal(bits(h_f), bits(h_u))
    # grad_preact differs only by the bf16 rounding of dout in the baseline
    assert_close("grad_preact fused vs unfused", to_f64(gp_f), to_f64(gp_u), tol=1e-2)


@pytest.mark.parametrize("shape", [(300, 512, 768, 512), (2048, 1024, 2816, 1024)])
def test_save_h_variant(shape):
    """The drop-h report's fallback (h saved from the forward): bitwise the
    same outputs as the drop-h path, h equal to the backward's recompute,
    and the oracle's gradients."""
    M, D, I, Dout = shape
    _case("save-h variant", shape)
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout, seed=23)
    pre, h, y = sw.swiglu_mlp_fwd_save_h(x, W1, Wd)
    pre0, y0 = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd_saved_h(x, W1, Wd, pre, h, dy)
    dx0, dW10, dWd0 = sw.swiglu_mlp_bwd(x, W1, Wd, pre0, dy)
    gp_only = sw.swiglu_bwd_dgrad_fused_gp(dy, Wd, pre)
    gp_full, h_bwd = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    torch.cuda.synchronize()
    for a, b in ((pre, pre0), (y, y0), (h, h_bwd), (gp_only, gp_full), (dx, dx0), (dW1, dW10), (dWd, dWd0)):
        assert np.array_equal(bits(a), bits(b))
    ref = oracle.backward(xf, W1f, Wdf, dyf)
    assert_close("h", to_f64(h), ref["h"])
    assert_close("dx", to_f64(dx), ref["dx"])
    assert_close("dW1", to_f64(dW1), ref["dW1"])
    assert_close("dW_down", to_f64(dWd), ref["dW_down"])


def test_save_h_autograd_saves_five_tensors():
    B, S, D, I, Dout = 2, 64, 256, 512, 256
    _case("save-h autograd")
    _, (x, W1, Wd, dy), _ = _inputs(B * S, D, I, Dout, seed=29)
    grads = []
    for fn, nsaved in ((sw.swiglu_mlp_save_h, 5), (sw.swiglu_mlp, 4)):
        x3 = x.view(B, S, D).clone().requires_grad_(True)
        W1r, Wdr = W1.clone().requires_grad_(True), Wd.clone().requires_grad_(True)
        y = fn(x3, W1r, Wdr)
        assert len(y.grad_fn.saved_tensors) == nsaved
        y.backward(dy.view(B, S, Dout))
        grads.append([bits(t) for t in (y.reshape(-1, Dout), x3.grad.reshape(-1, D), W1r.grad, Wdr.grad)])
    for a, b in zip(*grads):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("shape", [(200, 256, 512, 256), (300, 512, 768, 512), (96, 192, 320, 192),
                                   (2048, 1024, 2816, 1024), (1, 256, 512, 256), (13, 384, 192, 384),
                                   (16, 1024, 2816, 1024)])
def test_residual_block_vs_oracle(shape):
    """Y = X + MLP(X) with the add in the down GEMM's epilogue (the last
    three shapes take the decode path, whose reduce kernel adds x), and
    dX = dy + grad_preact.W1^T with dy added in the dx GEMM's epilogue.
    Checked against the oracle's residual block, the bare MLP part (y - x,
    dx - dy) against the oracle's MLP, and the gradients that the identity
    branch does not touch bitwise against the plain MLP's."""
    M, D, I, Dout = shape
    _case("residual block", shape)
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout, seed=31)
    pre, y = sw.swiglu_mlp_fwd_residual(x, W1, Wd)
    pre0, y0 = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd_residual(x, W1, Wd, pre, dy)
    dx0, dW10, dWd0 = sw.swiglu_mlp_bwd(x, W1, Wd, pre0, dy)
    torch.cuda.synchronize()
    for a, b in ((pre, pre0), (dW1, dW10), (dWd, dWd0)):
        assert np.array_equal(bits(a), bits(b))
    ref = oracle.backward_residual(xf, W1f, Wdf, dyf)
    plain = oracle.backward(xf, W1f, Wdf, dyf)
    assert_close("y", to_f64(y), ref["y"])
    assert_close("dx", to_f64(dx), ref["dx"])
    assert_close("y - x", to_f64(y) - xf, plain["y"])
    assert_close("dx - dy", to_f64(dx) - dyf, plain["dx"])
    # one rounding of (acc + x): within one bf16 ulp of y on each side of
    # the separately rounded MLP output plus x
    yr, y0f = to_f64(y), to_f64(y0)
    assert np.all(np.abs(yr - (y0f + xf)) <= ulp_bf16(yr) + ulp_bf16(y0f))
    dxr, dx0f = to_f64(dx), to_f64(dx0)
    assert np.all(np.abs(dxr - (dx0f + dyf)) <= ulp_bf16(dxr) + ulp_bf16(dx0f))


def test_residual_step_kernels_and_autograd():
    B, S, D, I = 2, 96, 256, 512
    M = B * S
    _case("residual steps + autograd")
    _, (x, W1, Wd, dy), _ = _inputs(M, D, I, D, seed=37)
    pre, y = sw.swiglu_mlp_fwd_residual(x, W1, Wd)
    _, h = sw.swiglu_fwd_gemm1(x, W1)
    assert np.array_equal(bits(sw.swiglu_fwd_down_residual(h, Wd, x)), bits(y))
    gp, _ = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    dx, _, _ = sw.swiglu_mlp_bwd_residual(x, W1, Wd, pre, dy)
    assert np.array_equal(bits(sw.swiglu_bwd_dx_residual(gp, W1, dy)), bits(dx))
    x3 = x.view(B, S, D).clone().requires_grad_(True)
    W1r, Wdr = W1.clone().requires_grad_(True), Wd.clone().requires_grad_(True)
    out = sw.swiglu_mlp_residual(x3, W1r, Wdr)
    assert len(out.grad_fn.saved_tensors) == 4
    out.backward(dy.view(B, S, D))
    assert np.array_equal(bits(out.reshape(-1, D)), bits(y))
    assert np.array_equal(bits(x3.grad.reshape(-1, D)), bits(dx))


def within_reorder_bound(name, a, b):
    """Two GEMM results that differ only in the order of their fp32 sums (the
    split tail adds K-parts of a tile separately): elementwise
    |a - b| <= 1 bf16 ulp of the larger magnitude (a rounding flip) plus
    2^-16 * max|b| (near-zero outputs, where the order changes the fp32 sum by
    about eps32 times the partial sums' size: ~1e-6 of max|b| measured at the
    target shape).  A missing or misplaced K-part is an O(1) error over whole
    tiles."""
    fa, fb = to_f64(a), to_f64(b)
    bound = ulp_bf16(np.maximum(np.abs(fa), np.abs(fb))) + 2.0 ** -16 * np.abs(fb).max()
    bad = np.abs(fa - fb) > bound
    assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond the reordering bound"


@pytest.mark.parametrize("shape", [(5000, 3584, 1024, 3584), (4700, 3584, 768, 3584)])
def test_split_tail_vs_oracle(shape):
    """Shapes whose dx GEMM runs its last, partly filled round of tiles as a
    split tail (K cut into parts, fp32 partial tiles, ordered reduce): the
    whole-step calls against the full oracle, and dx within one bf16 ulp of
    the single-launch dx kernel."""
    M, D, I, Dout = shape
    _case("split tail", shape)
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout, seed=61)
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)
    gp, _ = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    dx1 = sw.swiglu_bwd_dx(gp, W1)
    torch.cuda.synchronize()
    within_reorder_bound("dx split vs single launch", dx, dx1)
    ref = oracle.backward(xf, W1f, Wdf, dyf)
    assert_close("y", to_f64(y), ref["y"])
    assert_close("dx", to_f64(dx), ref["dx"])
    assert_close("dW1", to_f64(dW1), ref["dW1"])
    assert_close("dW_down", to_f64(dWd), ref["dW_down"])


def _fuzz_shapes(n=24, seed=71):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 700))]))
        D, I, Dout = (64 * int(rng.integers(1, 17)) for _ in range(3))
        out.append((M, D, I, Dout))
    return out


@pytest.mark.parametrize("shape", _fuzz_shapes())
def test_random_shapes_vs_oracle(shape):
    """Seeded random shapes: ragged token counts from 1 to 700 (the decode
    path at 16 rows or fewer when 2I and Dout are multiples of 128), and D, I,
    Dout any multiples of 64 up to 1024 (every tile configuration, N tails
    of 64)."""
    M, D, I, Dout = shape
    _case("fuzz", shape)
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout, seed=73)
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)
    torch.cuda.synchronize()
    ref = oracle.backward(xf, W1f, Wdf, dyf)
    for name, got in (("preact", pre), ("y", y), ("dx", dx), ("dW1", dW1), ("dW_down", dWd)):
        assert_close(name, to_f64(got), ref[name])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 9, 10, 14, 15, 16, 17, 20])
def test_k_loop_stage_counts(n):
    """The GEMM core's K loop runs 64-deep stages: stage 0 (its A operand
    came with the prologue), six-stage unrolled trips from stage 1 while at
    least seven more stages follow, single steady stages, then two stages
    that load nothing.  n stages for F1 (K = D), B1 (K = Dout) and B4 (K = M,
    ragged) while their N stays a multiple of 256 (the 256x256 tiles); F2,
    B2 and B3 then see N = 64n or K = 8 and 16 stages on the other tile
    configurations.  n walks across every boundary of that schedule."""
    M, D, I, Dout = 64 * n - 5, 64 * n, 512, 64 * n
    _case("k-loop stages", n, (M, D, I, Dout))
    _, (x, W1, Wd, dy), (xf, W1f, Wdf, dyf) = _inputs(M, D, I, Dout, seed=100 + n)
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)
    torch.cuda.synchronize()
    ref = oracle.backward(xf, W1f, Wdf, dyf)
    for name, got in (("preact", pre), ("y", y), ("dx", dx), ("dW1", dW1), ("dW_down", dWd)):
        assert_close(name, to_f64(got), ref[name])


def test_empty_batch():
    D, I, Dout = 256, 512, 256
    _case("M=0")
    _, (x, W1, Wd, dy), _ = _inputs(4, D, I, Dout)
    x0, dy0 = x[:0].contiguous(), dy[:0].contiguous()
    pre, y = sw.swiglu_mlp_fwd(x0, W1, Wd)
    assert pre.shape == (0, 2 * I) and y.shape == (0, Dout)
    dW1 = torch.full((D, 2 * I), 7.0, dtype=torch.bfloat16, device="cuda")
    dWd = torch.full((I, Dout), 7.0, dtype=torch.bfloat16, device="cuda")
    dx, dW1, dWd = sw.swiglu_mlp_bwd(x0, W1, Wd, pre, dy0, dW1=dW1, dW_down=dWd)
    torch.cuda.synchronize()
    assert dx.shape == (0, D)
    assert torch.count_nonzero(dW1).item() == 0 and torch.count_nonzero(dWd).item() == 0


def test_deterministic_bitwise():
    M, D, I, Dout = 300, 512, 768, 512
    _case("determinism", (M, D, I, Dout))
    _, (x, W1, Wd, dy), _ = _inputs(M, D, I, Dout, seed=9)
    outs = []
    for _ in range(2):
        pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
        dx, dW1, dWd = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)
        outs.append([bits(t) for t in (pre, y, dx, dW1, dWd)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_autograd_function_saves_four_tensors():
    B, S, D, I, Dout = 2, 64, 256, 512, 256
    _case("autograd")
    _, (x, W1, Wd, dy), _ = _inputs(B * S, D, I, Dout, seed=13)
    x3 = x.view(B, S, D).clone().requires_grad_(True)
    W1r, Wdr = W1.clone().requires_grad_(True), Wd.clone().requires_grad_(True)
    y = sw.swiglu_mlp(x3, W1r, Wdr)
    assert y.shape == (B, S, Dout)
    assert len(y.grad_fn.saved_tensors) == 4
    y.backward(dy.view(B, S, Dout))
    pre, y2 = sw.swiglu_mlp_fwd(x, W1, Wd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)
    assert np.array_equal(bits(y.reshape(-1, Dout)), bits(y2))
    assert np.array_equal(bits(x3.grad.reshape(-1, D)), bits(dx))
    assert np.array_equal(bits(W1r.grad), bits(dW1))
    assert np.array_equal(bits(Wdr.grad), bits(dWd))


def test_side_stream_and_workspace_checks():
    """A call on a stream that is not the current one (torch stream or raw
    handle): its outputs and temporary workspace belong to that stream, so
    allocations made meanwhile on the current stream cannot take them over;
    results equal the current-stream call bit for bit.  A workspace that is
    a stride-0 view (its numel overstates its storage) is refused."""
    M, D, I, Dout = 300, 512, 768, 512
    _case("side stream", (M, D, I, Dout))
    _, (x, W1, Wd, dy), _ = _inputs(M, D, I, Dout, seed=21)
    pre, y = sw.swiglu_mlp_fwd(x, W1, Wd)
    ref = [bits(t) for t in sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for handle in (side, side.cuda_stream):
        side.wait_stream(torch.cuda.current_stream())
        got = sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy, stream=handle)
        # allocations on the current stream while the side stream may still run
        junk = [torch.full((1 << 22,), 7, dtype=torch.uint8, device="cuda") for _ in range(8)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert np.array_equal(a, bits(b))
        del junk
    ws = torch.zeros(1, dtype=torch.uint8, device="cuda").expand(1 << 30)
    with pytest.raises(ValueError):
        sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy, ws=ws)
