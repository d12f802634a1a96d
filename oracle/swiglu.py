"""fp64 oracle of the SwiGLU MLP forward and backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's ``cpu_baseline`` leg, never by the product path.

Every function is the plain definition written out in float64, with numpy's
matrix product (a library primitive) for each GEMM and no blocking, fusion
or reordering.  Inputs arrive as exact float64 values of bf16 numbers.  The
oracle does not mimic any bf16 rounding of stored intermediates: where the
GPU stores ``preact`` or ``h`` in bf16, the difference is absorbed by the
test tolerance.

Sources (the three pages this method is described on):
  * "SwiGLU MLP forward principle, backward chain and optimisation"
    (section 1 forward, section 2 backward steps 1-3 and the three silu'
    forms, section 3 FLOP ledger, section 4 byte ledger);
  * "SwiGLU MLP Drop-H technical report" (forward formulas, backward
    formulas, fused h / grad_preact pseudocode);
  * "Lesson 24: MLP, GEMM and operator fusion in Transformers"
    (section 11 sigmoid and SiLU definitions; section 4 the 2-FLOPs-per-MAC
    count; section 28 the GEMM cost 2*M*N*K).

Layouts (the first page's section 1): x [M,D]; W1 [D,2I] with columns
[0,I) the un-gated "left" branch and [I,2I) the gate; W_down [I,Dout];
preact = x @ W1 = [left | gate] [M,2I]; h [M,I]; y [M,Dout].
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Scalar activation functions (Lesson 24, section 11: sigma and SiLU)
# --------------------------------------------------------------------------

def sigmoid(g):
    """sigma(g) = 1 / (1 + e^(-g)).  For g below about -709 e^(-g) overflows
    to inf and sigma is 0, its correctly rounded fp64 value."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def silu(g):
    """SiLU(g) = g * sigma(g)."""
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g)


# The first page (section 2, the SwiGLU step) gives three equal forms of the
# derivative of SiLU; all three are kept so that a test can hold them
# against each other.

def dsilu_form1(g):
    """silu'(g) = sigma + g * sigma * (1 - sigma)."""
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid(g)
    return s + g * s * (1.0 - s)


def dsilu_form2(g):
    """silu'(g) = sigma * (1 + g * (1 - sigma))."""
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def dsilu_form3(g):
    """silu'(g) = sigma + silu(g) * (1 - sigma)."""
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid(g)
    return s + (g * s) * (1.0 - s)


dsilu = dsilu_form2


# --------------------------------------------------------------------------
# Elementwise SwiGLU forward / backward
# --------------------------------------------------------------------------

def swiglu_fwd_elementwise(preact):
    """h = left * silu(gate) with [left | gate] = preact (first page,
    section 1; drop-h report, forward formulas)."""
    P = np.asarray(preact, dtype=np.float64)
    I = P.shape[1] // 2
    left, gate = P[:, :I], P[:, I:]
    return left * silu(gate)


def swiglu_bwd_elementwise(preact, dout):
    """Given preact = [left | gate] and the gradient dout of h, return
    (grad_preact, h):

      dleft = dout * silu(gate)           (first page, section 2, step 2)
      dgate = dout * left * silu'(gate)
      grad_preact = [dleft | dgate]       (drop-h report, backward formulas)
      h = left * silu(gate)               (recomputed; drop-h report, fused
                                           h / grad_preact kernel)
    """
    P = np.asarray(preact, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    I = P.shape[1] // 2
    left, gate = P[:, :I], P[:, I:]
    s = silu(gate)
    dleft = dout * s
    dgate = dout * left * dsilu(gate)
    return np.concatenate([dleft, dgate], axis=1), left * s


# --------------------------------------------------------------------------
# Whole MLP
# --------------------------------------------------------------------------

def forward(x, W1, Wd):
    """preact = x @ W1, h = left * silu(gate), y = h @ W_down.

    First page, section 1 (the three forward lines); drop-h report, forward
    formulas.  Returns (preact, h, y) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    preact = x @ W1
    h = swiglu_fwd_elementwise(preact)
    y = h @ Wd
    return preact, h, y


def backward(x, W1, Wd, dy):
    """Full backward from the saved set {x, W1, W_down, preact}; preact is
    recomputed here in fp64 from x and W1.

      dout     = dy @ W_down^T        (first page, section 2, step 1)
      dW_down  = h^T @ dy
      [dleft | dgate] as in swiglu_bwd_elementwise     (step 2)
      dx       = grad_preact @ W1^T   (step 3)
      dW1      = x^T @ grad_preact    (step 3; one merged [D,M]x[M,2I]
                                       product, first page section 3)

    Returns a dict of fp64 arrays: preact, h, y, dout, grad_preact, dx,
    dW1, dW_down."""
    x = np.asarray(x, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    preact, h, y = forward(x, W1, Wd)
    dout = dy @ Wd.T
    grad_preact, h_re = swiglu_bwd_elementwise(preact, dout)
    dW_down = h_re.T @ dy
    dx = grad_preact @ W1.T
    dW1 = x.T @ grad_preact
    return dict(preact=preact, h=h, y=y, dout=dout, grad_preact=grad_preact,
                dx=dx, dW1=dW1, dW_down=dW_down)


def forward_residual(x, W1, Wd):
    """The residual MLP block Y = X + MLP(X) (Lesson 24, section 24, the
    residual-add epilogue of the down projection); needs Dout = D.
    Returns (preact, h, y) in fp64 with y = x + h @ W_down."""
    x = np.asarray(x, dtype=np.float64)
    preact, h, m = forward(x, W1, Wd)
    if m.shape != x.shape:
        raise ValueError("the residual block needs Dout == D")
    return preact, h, x + m


def backward_residual(x, W1, Wd, dy):
    """Backward of Y = X + MLP(X): the MLP's gradients, with the identity
    path's dy added to dx (dX = dy + grad_preact @ W1^T); dW1 and dW_down are
    the MLP's.  Returns the same dict as backward, with y and dx of the
    residual block."""
    g = backward(x, W1, Wd, dy)
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    if g["y"].shape != x.shape:
        raise ValueError("the residual block needs Dout == D")
    g["y"] = x + g["y"]
    g["dx"] = g["dx"] + dy
    return g


def stack_forward(x, layers):
    """A stack of MLP blocks applied one after another (the drop-h report's
    4-layer stack benchmark): x_0 = x, x_{l+1} = MLP_l(x_l), each block with
    its own (W1, W_down) and Dout = D.  Returns (preacts, hs, ys), one entry
    per layer, with ys[-1] the stack's output."""
    cur = np.asarray(x, dtype=np.float64)
    preacts, hs, ys = [], [], []
    for W1, Wd in layers:
        p, h, y = forward(cur, W1, Wd)
        if y.shape != cur.shape:
            raise ValueError("a stack of blocks needs Dout == D")
        preacts.append(p)
        hs.append(h)
        ys.append(y)
        cur = y
    return preacts, hs, ys


def stack_backward(x, layers, dy):
    """Backward of stack_forward by the chain rule: the last block gets dy,
    and each block's dx is the dy of the block before it.  Returns
    {"y": the stack's output, "dx": the gradient of x, "dW1": [...],
    "dW_down": [...]} with one weight gradient per layer."""
    cur = np.asarray(x, dtype=np.float64)
    inputs = []
    for W1, Wd in layers:
        inputs.append(cur)
        _, _, cur = forward(cur, W1, Wd)
    g = np.asarray(dy, dtype=np.float64)
    dW1s, dWds = [None] * len(layers), [None] * len(layers)
    for l in range(len(layers) - 1, -1, -1):
        W1, Wd = layers[l]
        r = backward(inputs[l], W1, Wd, g)
        dW1s[l], dWds[l] = r["dW1"], r["dW_down"]
        g = r["dx"]
    return {"y": cur, "dx": g, "dW1": dW1s, "dW_down": dWds}


def moe_forward(x, W1s, Wds, offsets):
    """Mixture-of-experts MLP (Lesson 24, section 41: every expert is its own
    MLP block; section 42: the tokens of each expert form one GEMM of their
    own size).  Routed rows arrive packed by expert: expert e owns rows
    [offsets[e], offsets[e+1]) and applies its block (W1s[e], Wds[e]) to
    them.  Returns (preact, h, y) over all rows."""
    x = np.asarray(x, dtype=np.float64)
    off = [int(v) for v in offsets]
    E = len(W1s)
    if len(off) != E + 1 or off[0] != 0 or off[-1] != x.shape[0] or any(b < a for a, b in zip(off, off[1:])):
        raise ValueError("offsets must run from 0 to the row count without decreasing, one more than the experts")
    I = np.asarray(Wds[0]).shape[0]
    Dout = np.asarray(Wds[0]).shape[1]
    M = x.shape[0]
    preact, h, y = np.zeros((M, 2 * I)), np.zeros((M, I)), np.zeros((M, Dout))
    for e in range(E):
        a, b = off[e], off[e + 1]
        preact[a:b], h[a:b], y[a:b] = forward(x[a:b], W1s[e], Wds[e])
    return preact, h, y


def moe_backward(x, W1s, Wds, offsets, dy):
    """Backward of moe_forward: each expert's rows take its block's backward;
    an expert with no rows has zero weight gradients.  Returns the dict of
    ``backward`` over all rows, with dW1 [E, D, 2I] and dW_down [E, I, Dout]
    stacked per expert."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    preact, h, y = moe_forward(x, W1s, Wds, offsets)
    off = [int(v) for v in offsets]
    E = len(W1s)
    M, D = x.shape
    I = np.asarray(Wds[0]).shape[0]
    out = {"preact": preact, "h": h, "y": y, "dout": np.zeros((M, I)), "grad_preact": np.zeros((M, 2 * I)),
           "dx": np.zeros((M, D)), "dW1": np.zeros((E, D, 2 * I)), "dW_down": np.zeros((E, I, dy.shape[1]))}
    for e in range(E):
        a, b = off[e], off[e + 1]
        r = backward(x[a:b], W1s[e], Wds[e], dy[a:b])
        for k in ("dout", "grad_preact", "dx"):
            out[k][a:b] = r[k]
        out["dW1"][e] = r["dW1"]
        out["dW_down"][e] = r["dW_down"]
    return out


def sampled_forward_backward(x, W1, Wd, dy, rows, chans):
    """Exact fp64 values of the outputs at a sample of positions, for shapes
    where the full oracle is too slow.  Same definitions as ``backward``,
    restricted by linearity:

      * for the token rows ``rows``: preact, h, y, dout, grad_preact and dx
        on those rows (each row needs only that row of x and dy);
      * for the intermediate channels ``chans`` (indices into [0, I)):
        preact, h, dout and grad_preact on those columns for every token,
        the columns ``chans`` and ``I + chans`` of dW1, and the rows
        ``chans`` of dW_down.

    Returns a dict; keys ending in ``_rows`` are [len(rows), ...] and keys
    ending in ``_cols`` are [..., len(chans)] (dW_down_rows is
    [len(chans), Dout]).  ``dy`` may be None for a forward-only sample."""
    x = np.asarray(x, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    rows = np.asarray(rows)
    chans = np.asarray(chans)
    I = W1.shape[1] // 2
    out = {}
    # --- rows ---
    pr = x[rows] @ W1
    hr = swiglu_fwd_elementwise(pr)
    out["preact_rows"] = pr
    out["h_rows"] = hr
    out["y_rows"] = hr @ Wd
    # --- channels ---
    cols2 = np.concatenate([chans, I + chans])
    pc = x @ W1[:, cols2]                     # [M, 2c]: [left cols | gate cols]
    out["preact_cols"] = pc
    out["h_cols"] = swiglu_fwd_elementwise(pc)
    if dy is None:
        return out
    dy = np.asarray(dy, dtype=np.float64)
    dr = dy[rows] @ Wd.T
    gpr, _ = swiglu_bwd_elementwise(pr, dr)
    out["dout_rows"] = dr
    out["grad_preact_rows"] = gpr
    out["dx_rows"] = gpr @ W1.T
    dc = dy @ Wd[chans].T                     # [M, c]
    gpc, hc = swiglu_bwd_elementwise(pc, dc)  # [M, 2c], [M, c]
    out["dout_cols"] = dc
    out["grad_preact_cols"] = gpc
    out["dW1_cols"] = x.T @ gpc               # columns chans and I + chans
    out["dW_down_rows"] = hc.T @ dy           # rows chans
    return out


# --------------------------------------------------------------------------
# Algorithmic work
# --------------------------------------------------------------------------

def gemm_flops(M, D, I, Dout):
    """FLOPs of each GEMM at 2 FLOPs per multiply-add (Lesson 24, sections 4
    and 28: a GEMM of [M,K]x[K,N] costs 2*M*N*K).

    forward:  preact [M,D]x[D,2I], y [M,I]x[I,Dout]
    backward: dout [M,Dout]x[Dout,I], dW_down [I,M]x[M,Dout],
              dx [M,2I]x[2I,D], dW1 [D,M]x[M,2I]   (first page, section 3)
    """
    f = dict(
        preact=2 * M * D * (2 * I),
        y=2 * M * I * Dout,
        dout=2 * M * Dout * I,
        dW_down=2 * I * M * Dout,
        dx=2 * M * (2 * I) * D,
        dW1=2 * D * M * (2 * I),
    )
    f["forward"] = f["preact"] + f["y"]
    f["backward"] = f["dout"] + f["dW_down"] + f["dx"] + f["dW1"]
    return f


def algorithmic_bytes(M, D, I, Dout, elem=2):
    """HBM bytes each step must move at least once, every tensor counted
    once at ``elem`` bytes (bf16 = 2).  The fused dgrad step reads dy,
    W_down and preact and writes grad_preact and h; the unfused baseline
    additionally writes dout and reads it back (first page, section 4: the
    dout round trip is what fusion removes)."""
    fused = elem * (M * Dout + I * Dout + M * 2 * I + M * 2 * I + M * I)
    dout_round_trip = 2 * elem * M * I
    fwd = elem * (M * D + D * 2 * I + M * 2 * I + 2 * M * I + I * Dout + M * Dout)
    return dict(fused_dgrad=fused, unfused_dgrad=fused + dout_round_trip,
                saved=dout_round_trip, forward=fwd)
