"""Every entry point writes only inside its outputs and its workspace.

The GEMM epilogues bound their global accesses by buffer descriptors that
end at the row bound: stores to rows past it are dropped by the hardware
range check rather than skipped by a branch.  Here each output is the
leading view of a larger buffer, and the workspace the leading bytes of a
larger byte buffer; the tails hold a fill pattern that must survive the
call.  The results must also equal, bit for bit, those of the same call on
buffers of exactly the output's size.  The shapes cover ragged token
counts, weight-gradient row counts (D, I) that are not whole 256-row
tiles, 128- and 64-wide tiles, the split tails, the decode path and ragged
expert groups with empty and one-row experts."""
import numpy as np
import pytest
import torch

import bwd_gemm_epilogue_amd as sw
from gpu_util import bits, to_dev
from workload import MoEWorkload, make_moe_inputs

pytestmark = pytest.mark.gpu

FILL16 = 0x5A5A      # int16 pattern in the output tails
FILL8 = 0x5A         # byte pattern in the workspace tail
GUARD_ROWS = 3
GUARD_BYTES = 4096


class Guarded:
    """Output views whose buffers extend GUARD_ROWS rows past the view."""

    def __init__(self):
        self.bufs = []

    def out(self, name, shape):
        rows = int(np.prod(shape[:-1]))
        buf = torch.full((rows + GUARD_ROWS, shape[-1]), FILL16, dtype=torch.int16, device="cuda")
        self.bufs.append((name, buf, rows))
        return buf[:rows].view(torch.bfloat16).view(shape)

    def ws(self, name, nbytes):
        buf = torch.full((nbytes + GUARD_BYTES,), FILL8, dtype=torch.uint8, device="cuda")
        self.bufs.append((name, buf, nbytes))
        return buf[:nbytes]

    def check(self):
        torch.cuda.synchronize()
        for name, buf, n in self.bufs:
            fill = FILL16 if buf.dtype == torch.int16 else FILL8
            tail = buf[n:]
            bad = int((tail != fill).sum().item())
            assert bad == 0, f"{name}: {bad} elements written past its end"


def _rand(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16).cuda()


def _inputs(M, D, I, Dout, seed):
    g = torch.Generator().manual_seed(seed)
    return (_rand((M, D), g), _rand((D, 2 * I), g, D ** -0.5), _rand((I, Dout), g, I ** -0.5),
            _rand((M, Dout), g))


def _same(name, got, ref):
    assert np.array_equal(bits(got), bits(ref)), f"{name}: differs from the exactly sized call"


DENSE = [
    (300, 320, 576, 192),     # D and I not whole 256-row tiles; 128- and 64-wide tiles
    (1037, 512, 768, 512),    # ragged M on 256x256 tiles
    (4700, 3584, 768, 3584),  # split tails with a ragged last tile row
    (7, 256, 512, 256),       # decode path
    (16, 512, 768, 512),      # decode path, 16 rows
]


@pytest.mark.parametrize("shape", DENSE)
def test_whole_step_writes_stay_in_bounds(shape):
    M, D, I, Dout = shape
    print(f"bounds: whole step {shape}", flush=True)
    x, W1, Wd, dy = _inputs(M, D, I, Dout, seed=11)
    gd = Guarded()
    pre, y = gd.out("preact", (M, 2 * I)), gd.out("y", (M, Dout))
    sw.swiglu_mlp_fwd(x, W1, Wd, preact=pre, y=y, ws=gd.ws("fwd ws", sw.swiglu_mlp_fwd_workspace(M, D, I, Dout)))
    dx, dW1, dWd = gd.out("dx", (M, D)), gd.out("dW1", (D, 2 * I)), gd.out("dW_down", (I, Dout))
    sw.swiglu_mlp_bwd(x, W1, Wd, pre, dy, dx=dx, dW1=dW1, dW_down=dWd,
                      ws=gd.ws("bwd ws", sw.swiglu_mlp_bwd_workspace(M, D, I, Dout)))
    gd.check()
    rpre, ry = sw.swiglu_mlp_fwd(x, W1, Wd)
    rdx, rdW1, rdWd = sw.swiglu_mlp_bwd(x, W1, Wd, rpre, dy)
    for n, a, b in (("preact", pre, rpre), ("y", y, ry), ("dx", dx, rdx), ("dW1", dW1, rdW1),
                    ("dW_down", dWd, rdWd)):
        _same(n, a, b)


@pytest.mark.parametrize("shape", [DENSE[0], DENSE[1]])
def test_single_steps_and_variants_write_stay_in_bounds(shape):
    M, D, I, Dout = shape
    print(f"bounds: single steps, save-h, residual {shape}", flush=True)
    x, W1, Wd, dy = _inputs(M, D, I, Dout, seed=12)
    pre, _ = sw.swiglu_mlp_fwd(x, W1, Wd)
    gd = Guarded()
    # forward GEMM-1 with its SwiGLU epilogue, and the fused dgrad step
    p1, h1 = gd.out("gemm1 preact", (M, 2 * I)), gd.out("gemm1 h", (M, I))
    sw.swiglu_fwd_gemm1(x, W1, preact=p1, h=h1)
    gp, h = gd.out("grad_preact", (M, 2 * I)), gd.out("h", (M, I))
    sw.swiglu_bwd_dgrad_fused(dy, Wd, pre, grad_preact=gp, h=h)
    gp2 = gd.out("grad_preact (save-h)", (M, 2 * I))
    sw.swiglu_bwd_dgrad_fused_gp(dy, Wd, pre, grad_preact=gp2)
    # save-h forward and backward
    sp, sh, sy = gd.out("save-h preact", (M, 2 * I)), gd.out("save-h h", (M, I)), gd.out("save-h y", (M, Dout))
    sw.swiglu_mlp_fwd_save_h(x, W1, Wd, preact=sp, h=sh, y=sy)
    sdx, sdW1, sdWd = gd.out("save-h dx", (M, D)), gd.out("save-h dW1", (D, 2 * I)), gd.out("save-h dW_down", (I, Dout))
    sw.swiglu_mlp_bwd_saved_h(x, W1, Wd, sp, sh, dy, dx=sdx, dW1=sdW1, dW_down=sdWd,
                              ws=gd.ws("save-h bwd ws", sw.swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout)))
    gd.check()
    rp1, rh1 = sw.swiglu_fwd_gemm1(x, W1)
    rgp, rh = sw.swiglu_bwd_dgrad_fused(dy, Wd, pre)
    rsp, rsh, rsy = sw.swiglu_mlp_fwd_save_h(x, W1, Wd)
    rsdx, rsdW1, rsdWd = sw.swiglu_mlp_bwd_saved_h(x, W1, Wd, rsp, rsh, dy)
    for n, a, b in (("gemm1 preact", p1, rp1), ("gemm1 h", h1, rh1), ("grad_preact", gp, rgp), ("h", h, rh),
                    ("grad_preact (save-h)", gp2, rgp), ("save-h y", sy, rsy), ("save-h dx", sdx, rsdx),
                    ("save-h dW1", sdW1, rsdW1), ("save-h dW_down", sdWd, rsdWd)):
        _same(n, a, b)


@pytest.mark.parametrize("shape", [(300, 320, 576, 320), (1037, 512, 768, 512), (7, 256, 512, 256)])
def test_residual_block_writes_stay_in_bounds(shape):
    M, D, I, Dout = shape
    print(f"bounds: residual block {shape}", flush=True)
    x, W1, Wd, dy = _inputs(M, D, I, Dout, seed=13)
    gd = Guarded()
    pre, y = gd.out("preact", (M, 2 * I)), gd.out("y", (M, Dout))
    sw.swiglu_mlp_fwd_residual(x, W1, Wd, preact=pre, y=y,
                               ws=gd.ws("fwd ws", sw.swiglu_mlp_fwd_workspace(M, D, I, Dout)))
    dx, dW1, dWd = gd.out("dx", (M, D)), gd.out("dW1", (D, 2 * I)), gd.out("dW_down", (I, Dout))
    sw.swiglu_mlp_bwd_residual(x, W1, Wd, pre, dy, dx=dx, dW1=dW1, dW_down=dWd,
                               ws=gd.ws("bwd ws", sw.swiglu_mlp_bwd_workspace(M, D, I, Dout)))
    gd.check()
    rpre, ry = sw.swiglu_mlp_fwd_residual(x, W1, Wd)
    rdx, rdW1, rdWd = sw.swiglu_mlp_bwd_residual(x, W1, Wd, rpre, dy)
    for n, a, b in (("y", y, ry), ("dx", dx, rdx), ("dW1", dW1, rdW1), ("dW_down", dWd, rdWd)):
        _same(n, a, b)


@pytest.mark.parametrize("counts,dims", [([0, 37, 300, 1, 0, 129], (192, 384, 128)), ([70, 0, 5, 190], (128, 320, 64))])
def test_moe_writes_stay_in_bounds(counts, dims):
    D, I, Dout = dims
    print(f"bounds: moe {counts} {dims}", flush=True)
    w = MoEWorkload("bounds", 1, 1, len(counts), D, I, Dout, 1.0, 1 / np.sqrt(D), 1 / np.sqrt(I), 1.0, skew=1.0)
    xb, W1b, Wdb, dyb, off = make_moe_inputs(w, seed=14, counts=counts)
    x, W1, Wd, dy = to_dev(xb), to_dev(W1b), to_dev(Wdb), to_dev(dyb)
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    M, E = x.shape[0], len(counts)
    gd = Guarded()
    pre, y = gd.out("preact", (M, 2 * I)), gd.out("y", (M, Dout))
    sw.swiglu_moe_fwd(x, W1, Wd, offs, preact=pre, y=y,
                      ws=gd.ws("fwd ws", sw.swiglu_moe_fwd_workspace(M, D, I, Dout, E)))
    gp, h = gd.out("grad_preact", (M, 2 * I)), gd.out("h", (M, I))
    sw.swiglu_moe_bwd_dgrad_fused(dy, Wd, offs, pre, grad_preact=gp, h=h)
    dx, dW1, dWd = gd.out("dx", (M, D)), gd.out("dW1", (E, D, 2 * I)), gd.out("dW_down", (E, I, Dout))
    sw.swiglu_moe_bwd(x, W1, Wd, offs, pre, dy, dx=dx, dW1=dW1, dW_down=dWd,
                      ws=gd.ws("bwd ws", sw.swiglu_moe_bwd_workspace(M, D, I, Dout, E)))
    gd.check()
    rpre, ry = sw.swiglu_moe_fwd(x, W1, Wd, offs)
    rgp, rh = sw.swiglu_moe_bwd_dgrad_fused(dy, Wd, offs, rpre)
    rdx, rdW1, rdWd = sw.swiglu_moe_bwd(x, W1, Wd, offs, rpre, dy)
    for n, a, b in (("preact", pre, rpre), ("y", y, ry), ("grad_preact", gp, rgp), ("h", h, rh), ("dx", dx, rdx),
                    ("dW1", dW1, rdW1), ("dW_down", dWd, rdWd)):
        _same(n, a, b)
