"""The no-allocation forward (swiglu_mlp_fwd_noalloc, for callers that cannot
allocate) through the C ABI, against the workspace forward swiglu_mlp_fwd.

It runs the same kernels on the library's static device workspace, so its
outputs must equal swiglu_mlp_fwd's bit for bit; they are also checked
against the fp64 oracle at the per-tensor bound.  Three calls in a row: the
decode-shaped forward, then a smaller decode-shaped one (the static
workspace still holds the first call's h and partial sums, which the second
must not read), then a tiled shape."""
import numpy as np
import pytest
import torch

import bwd_gemm_epilogue_amd as sw
import oracle
from gpu_util import assert_close, bits, to_dev, to_f64
from workload import WORKLOADS, bf16_bits_to_f64, make_custom, make_inputs

pytestmark = pytest.mark.gpu


def _noalloc(x, W1, Wd, pre, y):
    M, D = x.shape
    I, Dout = Wd.shape
    st = torch.cuda.current_stream().cuda_stream
    return sw.lib().swiglu_mlp_fwd_noalloc(x.data_ptr(), W1.data_ptr(), Wd.data_ptr(), pre.data_ptr(),
                                           y.data_ptr(), M, D, I, Dout, st)


def test_noalloc_forward_matches_the_workspace_forward():
    w = WORKLOADS["decode"]
    cases = [("decode 16x4096x14336", make_inputs(w)[:3]),
             ("decode 7 rows, smaller", make_custom(7, 512, 768, 512, seed=3)[:3]),
             ("tiled 300 rows", make_custom(300, 512, 768, 512, seed=5)[:3])]
    for name, (xb, W1b, Wdb) in cases:
        print("case:", name, xb.shape, Wdb.shape, flush=True)
        x, W1, Wd = (to_dev(a) for a in (xb, W1b, Wdb))
        M, I, Dout = x.shape[0], Wd.shape[0], Wd.shape[1]
        pre_ref, y_ref = sw.swiglu_mlp_fwd(x, W1, Wd)
        pre = torch.full((M, 2 * I), 3.0, dtype=torch.bfloat16, device="cuda")
        y = torch.full((M, Dout), 3.0, dtype=torch.bfloat16, device="cuda")
        assert _noalloc(x, W1, Wd, pre, y) == 0
        torch.cuda.synchronize()
        assert np.array_equal(bits(pre), bits(pre_ref)), name
        assert np.array_equal(bits(y), bits(y_ref)), name
        p64, _, y64 = oracle.forward(*(bf16_bits_to_f64(a) for a in (xb, W1b, Wdb)))
        assert_close("preact", to_f64(pre), p64)
        assert_close("y", to_f64(y), y64)


def test_noalloc_forward_refuses_a_shape_beyond_its_limit():
    x = torch.zeros((4096, 256), dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros((256, 2 * 8192), dtype=torch.bfloat16, device="cuda")
    Wd = torch.zeros((8192, 256), dtype=torch.bfloat16, device="cuda")
    pre = torch.empty((4096, 2 * 8192), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((4096, 256), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(x, W1, Wd, pre, y) == -4   # SWIGLU_ERR_WORKSPACE
