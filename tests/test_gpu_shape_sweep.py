"""Seeded sweep of GEMM shapes through the C ABI against the fp64 oracle.

Sixteen (M, D, I, Dout) drawn once from a fixed seed: token counts from 1 to
2600 (ragged against every tile height), inner dimensions multiples of 64
from 64 to 1024, so that the dout GEMMs' tile planner, the 64-, 128- and
256-wide tile configurations, the paired GEMM-1 tiles and the decode path
(M <= 16) all come up.  Per shape: every single-step GEMM against the oracle
applied to the GPU's own intermediates, h from the forward and from the
fused backward bitwise equal, and the whole-step calls against the oracle's
backward.  Tolerance: the per-tensor bound max|gpu - oracle| <= 1e-2 *
max|oracle|, h within 2 bf16 ulp.
"""
import numpy as np
import pytest

import bwd_gemm_epilogue_amd as sw
import oracle
from gpu_util import assert_close, assert_ulp, bits, to_dev, to_f64
from workload import bf16_bits_to_f64, make_custom

pytestmark = pytest.mark.gpu


def _shapes(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        # a few decode-sized batches, the rest up to ~10 tiles of 256 rows
        M = int(rng.integers(1, 17)) if k % 5 == 0 else int(rng.integers(17, 2601))
        D, I, Dout = (int(64 * rng.integers(1, 17)) for _ in range(3))
        out.append((M, D, I, Dout))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{d}x{i}x{o}" for m, d, i, o in SHAPES])
def test_shape_sweep(shape):
    M, D, I, Dout = shape
    print("case: sweep", shape, flush=True)
    x, W1, Wd, dy = make_custom(M, D, I, Dout, seed=M + 7 * D + 11 * I + 13 * Dout)
    xd, W1d, Wdd, dyd = (to_dev(a) for a in (x, W1, Wd, dy))
    xf, W1f, Wdf, dyf = (bf16_bits_to_f64(a) for a in (x, W1, Wd, dy))

    # single-step calls, each against the oracle on the GPU's own inputs
    pre, h = sw.swiglu_fwd_gemm1(xd, W1d)
    assert_close("preact", to_f64(pre), xf @ W1f)
    assert_ulp("h(fwd)", to_f64(h), oracle.swiglu_fwd_elementwise(to_f64(pre)))
    y = sw.swiglu_fwd_down(h, Wdd)
    assert_close("y", to_f64(y), to_f64(h) @ Wdf)
    gp, h2 = sw.swiglu_bwd_dgrad_fused(dyd, Wdd, pre)
    ref_gp, ref_h = oracle.swiglu_bwd_elementwise(to_f64(pre), dyf @ Wdf.T)
    assert_close("grad_preact", to_f64(gp), ref_gp)
    assert_ulp("h(bwd)", to_f64(h2), ref_h)
    assert np.array_equal(bits(h), bits(h2)), "h_fwd != h_bwd"
    gp2 = sw.swiglu_bwd_dgrad_fused_gp(dyd, Wdd, pre)
    assert np.array_equal(bits(gp), bits(gp2)), "save-h grad_preact != drop-h grad_preact"
    assert_close("dW_down", to_f64(sw.swiglu_bwd_dw_down(h2, dyd)), to_f64(h2).T @ dyf)
    assert_close("dx", to_f64(sw.swiglu_bwd_dx(gp, W1d)), to_f64(gp) @ W1f.T)
    assert_close("dW1", to_f64(sw.swiglu_bwd_dw1(xd, gp)), xf.T @ to_f64(gp))

    # whole-step calls (split tails, decode path) against the oracle's backward
    pre_w, y_w = sw.swiglu_mlp_fwd(xd, W1d, Wdd)
    dx, dW1, dWd = sw.swiglu_mlp_bwd(xd, W1d, Wdd, pre_w, dyd)
    ref = oracle.backward(xf, W1f, Wdf, dyf)
    assert_close("preact(whole)", to_f64(pre_w), ref["preact"])
    assert_close("y(whole)", to_f64(y_w), ref["y"])
    assert_close("dx(whole)", to_f64(dx), ref["dx"])
    assert_close("dW1(whole)", to_f64(dW1), ref["dW1"])
    assert_close("dW_down(whole)", to_f64(dWd), ref["dW_down"])
