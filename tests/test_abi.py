"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call.  CPU only: every call below is
one the library must refuse, so nothing is ever launched."""
import ctypes
import subprocess

import pytest

import bwd_gemm_epilogue_amd as sw

OK, NULL, SHAPE, UNSUP, WS, ALIAS, HIP, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7
P = 0x10000000   # fake, 16-byte aligned "device" addresses: never dereferenced
MB = 1 << 20


def addr(i):
    return P + i * (1 << 32)   # far-apart ranges: no accidental overlap


def test_library_loads_and_exports_every_declared_symbol():
    L = sw.lib()
    names = sw.exported_names()
    assert "swiglu_mlp_fwd" in names and "swiglu_mlp_bwd" in names
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sw.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert f" T {n}\n" in out or out.endswith(f" T {n}"), n


def test_status_strings():
    L = sw.lib()
    for s in (OK, NULL, SHAPE, UNSUP, WS, ALIAS, HIP, ALIGN):
        assert L.swiglu_status_string(s).decode().startswith("SWIGLU_")
    assert b"unknown" in L.swiglu_status_string(-99)
    assert L.swiglu_abi_version() >> 16 == 1


def test_workspace_sizes():
    L = sw.lib()
    M, D, I, Dout = 11136, 3584, 14336, 3584
    tile = 256 * 256 * 4                       # one fp32 partial tile of the split tail
    # 616 tiles of the down GEMM (y = h.W_down) = 2 rounds of 256 + a tail of
    # 104, split 2 ways; the backward's splits: dx 104 tiles x 2 parts, dW_down
    # 16 x 13, dW1 32 x 8 (the largest: 256 partial tiles)
    assert L.swiglu_mlp_fwd_workspace(M, D, I, Dout) == M * I * 2 + 104 * 2 * tile
    assert L.swiglu_mlp_bwd_workspace(M, D, I, Dout) == M * 2 * I * 2 + M * I * 2 + 32 * 8 * tile
    assert L.swiglu_mlp_bwd_unfused_workspace(M, D, I, Dout) == M * 2 * I * 2 + 2 * M * I * 2 + 32 * 8 * tile
    assert L.swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout) == M * 2 * I * 2 + 32 * 8 * tile
    # whole rounds of tiles (the Llama-like shape): no split tail, no extra bytes
    assert L.swiglu_mlp_fwd_workspace(8192, 4096, 11008, 4096) == 8192 * 11008 * 2
    assert L.swiglu_mlp_bwd_workspace(8192, 4096, 11008, 4096) == 8192 * 2 * 11008 * 2 + 8192 * 11008 * 2
    assert L.swiglu_mlp_fwd_workspace(-1, D, I, Dout) == 0
    assert L.swiglu_mlp_fwd_workspace(M, 100, I, Dout) == 0
    assert L.swiglu_mlp_bwd_workspace(0, D, I, Dout) == 0


def _fwd(L, x=addr(0), W1=addr(1), Wd=addr(2), pre=addr(3), y=addr(4), ws=addr(5), wsb=1 << 40,
         M=128, D=256, I=512, Dout=256):
    return L.swiglu_mlp_fwd(x, W1, Wd, pre, y, ws, wsb, M, D, I, Dout, None)


def _bwd(L, fn="swiglu_mlp_bwd", ptrs=None, wsb=1 << 40, M=128, D=256, I=512, Dout=256):
    p = [addr(i) for i in range(9)] if ptrs is None else ptrs
    return getattr(L, fn)(*p[:8], p[8], wsb, M, D, I, Dout, None)


def test_fwd_rejects_bad_arguments():
    L = sw.lib()
    assert _fwd(L, x=None) == NULL
    assert _fwd(L, y=None) == NULL
    assert _fwd(L, M=-1) == SHAPE
    assert _fwd(L, D=0) == SHAPE
    assert _fwd(L, I=-64) == SHAPE
    assert _fwd(L, D=100) == UNSUP
    assert _fwd(L, I=96) == UNSUP
    assert _fwd(L, Dout=32) == UNSUP
    assert _fwd(L, I=1 << 21) == UNSUP
    assert _fwd(L, x=addr(0) + 8) == ALIGN
    assert _fwd(L, ws=addr(5) + 2) == ALIGN
    assert _fwd(L, ws=None) == WS
    assert _fwd(L, wsb=128 * 512 * 2 - 1) == WS
    assert _fwd(L, y=addr(0)) == ALIAS                       # output on an input
    assert _fwd(L, y=addr(3) + 64 * 1024) == ALIAS          # inside preact
    assert _fwd(L, ws=addr(4)) == ALIAS                      # workspace on y


def test_bwd_rejects_bad_arguments():
    L = sw.lib()
    for fn in ("swiglu_mlp_bwd", "swiglu_mlp_bwd_unfused"):
        p = [addr(i) for i in range(9)]
        for k in range(8):
            q = list(p)
            q[k] = None
            assert _bwd(L, fn, q) == NULL, (fn, k)
        assert _bwd(L, fn, M=-5) == SHAPE
        assert _bwd(L, fn, Dout=200) == UNSUP
        q = list(p)
        q[5] = addr(5) + 4
        assert _bwd(L, fn, q) == ALIGN
        assert _bwd(L, fn, wsb=10) == WS
        q = list(p)
        q[8] = None
        assert _bwd(L, fn, q) == WS
        q = list(p)
        q[5] = addr(3)     # dx onto preact
        assert _bwd(L, fn, q) == ALIAS
        q = list(p)
        q[6] = addr(7)     # dW1 onto dW_down
        assert _bwd(L, fn, q) == ALIAS
        q = list(p)
        q[8] = addr(0)     # workspace onto x
        assert _bwd(L, fn, q) == ALIAS
    # the unfused path needs the extra dout buffer
    need = L.swiglu_mlp_bwd_workspace(128, 256, 512, 256)
    assert _bwd(L, "swiglu_mlp_bwd_unfused", wsb=need) == WS


def test_step_entry_points_reject_bad_arguments():
    L = sw.lib()
    a = [addr(i) for i in range(6)]
    assert L.swiglu_fwd_gemm1(None, a[1], a[2], a[3], 128, 256, 512, None) == NULL
    assert L.swiglu_fwd_gemm1(a[0], a[1], a[2], a[3], 128, 250, 512, None) == UNSUP
    assert L.swiglu_fwd_gemm1(a[0], a[1], a[0], a[3], 128, 256, 512, None) == ALIAS
    assert L.swiglu_fwd_down(a[0], a[1], a[2], -1, 512, 256, None) == SHAPE
    assert L.swiglu_bwd_dgrad_fused(a[0], a[1], a[2], a[3], a[3], 128, 512, 256, None) == ALIAS
    assert L.swiglu_bwd_dgrad_fused(a[0], a[1], a[2], a[3], a[4] + 1, 128, 512, 256, None) == ALIGN
    assert L.swiglu_bwd_dgrad_plain(a[0], None, a[2], 128, 512, 256, None) == NULL
    assert L.swiglu_bwd_elementwise(a[0], a[1], a[2], a[3], 128, 100, None) == UNSUP
    assert L.swiglu_bwd_dw_down(a[0], a[1], a[1], 128, 512, 256, None) == ALIAS
    assert L.swiglu_bwd_dx(a[0], a[1], a[2], 128, 0, 512, None) == SHAPE
    assert L.swiglu_bwd_dw1(a[0], a[1], None, 128, 256, 512, None) == NULL
    assert L.swiglu_act_eval(a[0], a[1], a[2], a[3], -1, None) == SHAPE
    assert L.swiglu_act_eval(a[0] + 1, a[1], a[2], a[3], 16, None) == ALIGN
    assert L.swiglu_act_eval(a[0], a[1], a[1], a[3], 16, None) == ALIAS


def test_save_h_entry_points_reject_bad_arguments():
    L = sw.lib()
    a = [addr(i) for i in range(11)]
    M, D, I, Dout = 128, 256, 512, 256
    fwd = lambda *p: L.swiglu_mlp_fwd_save_h(*p, M, D, I, Dout, None)
    assert fwd(None, *a[1:6]) == NULL
    assert fwd(*a[:4], None, a[5]) == NULL                  # h is required
    assert fwd(*a[:4], a[4] + 8, a[5]) == ALIGN
    assert fwd(*a[:4], a[3] + 64, a[5]) == ALIAS            # h inside preact
    assert L.swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout) == M * 2 * I * 2   # no split tail at this size
    assert L.swiglu_mlp_bwd_saved_h_workspace(M, 100, I, Dout) == 0
    bwd = lambda p, wsb=1 << 40: L.swiglu_mlp_bwd_saved_h(*p[:9], p[9], wsb, M, D, I, Dout, None)
    p = [addr(i) for i in range(10)]
    for k in range(9):
        q = list(p)
        q[k] = None
        assert bwd(q) == NULL, k
    assert bwd(p, wsb=10) == WS
    q = list(p); q[9] = None
    assert bwd(q) == WS
    q = list(p); q[6] = addr(4)                             # dx onto the saved h
    assert bwd(q) == ALIAS
    q = list(p); q[9] = addr(4)                             # workspace onto the saved h
    assert bwd(q) == ALIAS
    assert L.swiglu_bwd_dgrad_fused_gp(a[0], a[1], a[2], a[2], M, I, Dout, None) == ALIAS
    assert L.swiglu_bwd_dgrad_fused_gp(a[0], None, a[2], a[3], M, I, Dout, None) == NULL
    assert L.swiglu_bwd_dgrad_fused_gp(a[0], a[1], a[2], a[3], M, 100, Dout, None) == UNSUP


def test_residual_entry_points_reject_bad_arguments():
    L = sw.lib()
    M, D, I = 128, 256, 512
    fwd = lambda p, Dout=D, wsb=1 << 40: L.swiglu_mlp_fwd_residual(*p[:5], p[5], wsb, M, D, I, Dout, None)
    p = [addr(i) for i in range(6)]
    assert fwd(p, Dout=D + 64) == SHAPE                       # the identity branch needs Dout == D
    for k in range(5):
        q = list(p); q[k] = None
        assert fwd(q) == NULL, k
    assert fwd(p, wsb=10) == WS
    q = list(p); q[4] = addr(0)                               # y onto x
    assert fwd(q) == ALIAS
    q = list(p); q[4] = p[4] + 8
    assert fwd(q) == ALIGN
    bwd = lambda p, Dout=D, wsb=1 << 40: L.swiglu_mlp_bwd_residual(*p[:8], p[8], wsb, M, D, I, Dout, None)
    p = [addr(i) for i in range(9)]
    assert bwd(p, Dout=D - 64) == SHAPE
    for k in range(8):
        q = list(p); q[k] = None
        assert bwd(q) == NULL, k
    assert bwd(p, wsb=10) == WS
    q = list(p); q[5] = addr(4)                               # dx onto dy
    assert bwd(q) == ALIAS
    a = [addr(i) for i in range(4)]
    assert L.swiglu_fwd_down_residual(a[0], a[1], a[2], a[2], M, I, D, None) == ALIAS
    assert L.swiglu_fwd_down_residual(a[0], a[1], None, a[3], M, I, D, None) == NULL
    assert L.swiglu_fwd_down_residual(a[0], a[1], a[2], a[3], M, I, 100, None) == UNSUP
    assert L.swiglu_bwd_dx_residual(a[0], a[1], a[2], a[2], M, D, I, None) == ALIAS
    assert L.swiglu_bwd_dx_residual(a[0], a[1], None, a[3], M, D, I, None) == NULL
    assert L.swiglu_bwd_dx_residual(a[0], a[1], a[2], a[3], -1, D, I, None) == SHAPE


def test_moe_entry_points_reject_bad_arguments():
    L = sw.lib()
    M, D, I, Dout, E = 300, 256, 512, 256, 8
    assert L.swiglu_moe_fwd_workspace(M, D, I, Dout, E) == M * I * 2
    assert L.swiglu_moe_bwd_workspace(M, D, I, Dout, E) == L.swiglu_mlp_bwd_workspace(M, D, I, Dout)
    assert L.swiglu_moe_fwd_workspace(M, D, I, Dout, 0) == 0
    assert L.swiglu_moe_bwd_workspace(M, 100, I, Dout, E) == 0
    fwd = lambda p, E=E, wsb=1 << 40: L.swiglu_moe_fwd(*p[:6], p[6], wsb, M, D, I, Dout, E, None)
    p = [addr(i) for i in range(7)]
    assert fwd(p, E=0) == SHAPE
    assert fwd(p, E=65537) == UNSUP
    for k in range(6):
        q = list(p); q[k] = None
        assert fwd(q) == NULL, k
    q = list(p); q[3] = p[3] + 2                              # offsets need 4-byte alignment
    assert fwd(q) == ALIGN
    q = list(p); q[3] = p[3] + 4                              # 4 bytes suffice: the next check refuses
    assert fwd(q, wsb=10) == WS
    assert fwd(p, wsb=10) == WS
    q = list(p); q[4] = addr(3)                               # preact onto the offsets
    assert fwd(q) == ALIAS
    q = list(p); q[5] = p[1] + 2 * (D * 2 * I * 2)            # y inside expert 2's W1
    assert fwd(q) == ALIAS
    bwd = lambda p, E=E, wsb=1 << 40: L.swiglu_moe_bwd(*p[:9], p[9], wsb, M, D, I, Dout, E, None)
    p = [addr(i) for i in range(10)]
    for k in range(9):
        q = list(p); q[k] = None
        assert bwd(q) == NULL, k
    assert bwd(p, wsb=10) == WS
    q = list(p); q[7] = p[2] + 16                             # dW1 overlapping W_down
    assert bwd(q) == ALIAS
    assert bwd(p, E=-1) == SHAPE
    g = lambda *a: L.swiglu_moe_bwd_dgrad_fused(*a)
    a = [addr(i) for i in range(6)]
    assert g(a[0], a[1], a[2], a[3], a[3], a[5], M, I, Dout, E, None) == ALIAS
    assert g(a[0], a[1], None, a[3], a[4], a[5], M, I, Dout, E, None) == NULL
    assert g(a[0], a[1], a[2], a[3], a[4], a[5], M, 100, Dout, E, None) == UNSUP


def test_moe_binding_checks_offsets_on_the_host():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sw.swiglu_moe_fwd(x, torch.zeros(2, 64, 128, dtype=torch.bfloat16), torch.zeros(2, 64, 64, dtype=torch.bfloat16),
                          torch.zeros(3, dtype=torch.int32))


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sw.swiglu_fwd_down(x, torch.zeros(64, 64, dtype=torch.bfloat16))


def test_python_binding_refuses_a_workspace_that_is_not_a_gpu_tensor():
    """A caller's workspace goes through the same checks as every other
    tensor: a host tensor (or anything else) is refused before any launch."""
    import torch
    like = torch.zeros(4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sw._ws(16, like, torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(TypeError):
        sw._ws(16, like, bytearray(64))


def test_every_launching_binding_runs_inside_a_launch_context():
    """Every binding that launches kernels takes `stream` and is wrapped so
    that its allocations belong to the launch stream; each refuses a host
    tensor as its first argument with ValueError."""
    import inspect
    import torch
    launching = [n for n in sw.__all__ if n.startswith("swiglu_") and callable(getattr(sw, n))
                 and "stream" in inspect.signature(getattr(sw, n)).parameters]
    assert len(launching) >= 20
    for n in launching:
        f = getattr(sw, n)
        assert getattr(f, "__wrapped__", None) is not None, f"{n} is not wrapped by _launches"
        with pytest.raises(ValueError):
            f(torch.zeros(4, 64, dtype=torch.bfloat16), *([None] * 3))


def test_noalloc_forward_refuses_shapes_beyond_its_static_workspace():
    """The no-allocation forward: the limit is its stated 32 MiB; a shape
    whose workspace fits is checked like swiglu_mlp_fwd (bad arguments are
    refused on the host), and one whose workspace exceeds the limit is
    refused with SWIGLU_ERR_WORKSPACE before any HIP call."""
    L = sw.lib()
    limit = L.swiglu_mlp_fwd_noalloc_limit()
    assert limit == 32 * MB
    f = L.swiglu_mlp_fwd_noalloc
    # decode shape fits
    assert L.swiglu_mlp_fwd_workspace(16, 4096, 14336, 4096) <= limit
    # h alone past the limit: M * I * 2 > 32 MiB
    M, D, I, Dout = 4096, 256, 8192, 256
    assert L.swiglu_mlp_fwd_workspace(M, D, I, Dout) > limit
    assert f(addr(0), addr(1), addr(2), addr(3), addr(4), M, D, I, Dout, None) == WS
    # the forward's other checks, before the workspace one
    assert f(addr(0), addr(1), addr(2), addr(3), addr(4), 16, 100, 512, 256, None) == UNSUP
    assert f(addr(0), None, addr(2), addr(3), addr(4), 16, 256, 512, 256, None) == NULL
    assert f(addr(0) + 8, addr(1), addr(2), addr(3), addr(4), 16, 256, 512, 256, None) == ALIGN
    assert f(addr(0), addr(1), addr(2), addr(0), addr(4), 16, 256, 512, 256, None) == ALIAS
