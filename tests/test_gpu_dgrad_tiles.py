"""The dout GEMMs in every tile shape the library picks for them.

The fused dgrad (dout = dy . W_down^T with the SwiGLU backward in its
epilogue; the note "SwiGLU MLP forward principle, backward chain and
optimisation", sections 2-4), its save-h twin and its plain-store twin take
256x256, 256x128, 128x256 or 128x128 tiles by the launch's estimated rounds
on the GPU, or 256x256 tiles over the first columns and another shape over
the rest in a second launch when that fills the rounds better.  These shapes
select each of them (and ragged token counts):
the outputs are checked against the fp64 oracle (per-tensor bound; h within
2 bf16 ulp) and bit for bit against the grouped launch with one expert,
which keeps its own tile rule: the tile shape does not change any element's
accumulation order (the same k-chunks, the same MFMA instruction, in the
same order), so the bits may not change with it.
"""
import numpy as np
import pytest
import torch

import bwd_gemm_epilogue_amd as sw
import oracle
from gpu_util import assert_close, assert_ulp, bits, to_dev, to_f64
from workload import bf16_bits_to_f64, normal_bf16

pytestmark = pytest.mark.gpu

# (M, I, Dout) and the tile shape the library picks for it on 256 compute units
SHAPES = [
    ((640, 7680, 512), "128x256"),
    ((2048, 2816, 1024), "256x128"),
    # 14 x 24 tiles of 256 x 256 would fill 1.3 rounds: 256 x 256 over the
    # first 4608 columns and 256 x 128 over the last 1408, two launches
    ((3333, 6016, 512), "256x256 + 256x128 split, ragged M"),
    ((2148, 5120, 768), "256x256"),
    ((700, 1024, 1024), "128x128"),
]


@pytest.mark.parametrize("shape,tile", SHAPES, ids=[t for _, t in SHAPES])
def test_dout_gemms_in_each_tile_shape(shape, tile):
    M, I, Dout = shape
    print("case: dout GEMMs", shape, tile, flush=True)
    dyb = normal_bf16((M, Dout), 1.0, 31)
    Wdb = normal_bf16((I, Dout), 1.0 / np.sqrt(Dout), 32)
    preb = normal_bf16((M, 2 * I), 2.0, 33)
    dy, Wd, pre = (to_dev(a) for a in (dyb, Wdb, preb))
    gp, h = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    gp_only = sw.swiglu_bwd_dgrad_fused_gp(dy, Wd, pre)
    dout = sw.swiglu_bwd_dgrad_plain(dy, Wd)
    off = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    gp_g, h_g = sw.swiglu_moe_bwd_dgrad_fused(dy, Wd.unsqueeze(0).contiguous(), off, pre)
    torch.cuda.synchronize()

    d64 = bf16_bits_to_f64(dyb) @ bf16_bits_to_f64(Wdb).T
    gp_ref, h_ref = oracle.swiglu_bwd_elementwise(bf16_bits_to_f64(preb), d64)
    assert_close("grad_preact", to_f64(gp), gp_ref)
    assert_close("h", to_f64(h), h_ref)
    assert_ulp("h", to_f64(h), h_ref)
    assert_close("dout", to_f64(dout), d64)
    assert np.array_equal(bits(gp), bits(gp_g)) and np.array_equal(bits(h), bits(h_g))
    assert np.array_equal(bits(gp_only), bits(gp))
