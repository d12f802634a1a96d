/*
 * swiglu_mlp.h -- C ABI of the MI355X (gfx950) SwiGLU MLP training step.
 *
 * The step (one MLP block, no bias):
 *   forward   preact = x . W1 = [left | gate]        [M,2I]
 *             h      = left * silu(gate)             [M,I]   (transient)
 *             y      = h . W_down                    [M,Dout]
 *   backward  dout   = dy . W_down^T                 [M,I]   (never stored by
 *                                                             the fused path)
 *             grad_preact = [dout*silu(gate) | dout*left*silu'(gate)]
 *             dW_down = h^T . dy,  dx = grad_preact . W1^T,  dW1 = x^T . grad_preact
 *
 * Sources: the note "SwiGLU MLP forward principle, backward chain and
 * optimisation" (section 1 forward; section 2 backward steps 1-3 and the
 * silu' forms; sections 3-4 the fused dout-GEMM epilogue), the "SwiGLU MLP
 * Drop-H technical report" (forward/backward formulas, the saved set
 * {x, W1, W2, preact}, h dropped after the down projection, non-inplace
 * backward that allocates h and grad_preact; its save-h fallback), and
 * "Lesson 24" (section 11 sigma and SiLU; section 24 the residual-add
 * epilogue; sections 41-43 mixture-of-experts MLPs and the grouped GEMM).
 *
 * Conventions for every entry point below:
 *   - Tensor arguments are DEVICE pointers to bf16 values (raw 16-bit
 *     patterns), row-major and densely packed (leading dimension = number
 *     of columns), owned by the caller.  Each must be 16-byte aligned.  The
 *     one exception is the int32 expert-offset table of the mixture-of-
 *     experts calls (4-byte aligned).
 *   - W1 is [D, 2I]: columns [0, I) are the un-gated "left" (up) branch and
 *     columns [I, 2I) the gate branch.  W_down is [I, Dout].
 *   - Inputs are never written.  Outputs are overwritten (not accumulated).
 *     No output may overlap an input or another output.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream).  The library never allocates
 *     device memory (its one static device array, the workspace of
 *     swiglu_mlp_fwd_noalloc, is placed by the HIP runtime when the library
 *     is loaded on a device), never synchronises and never prints.  Device
 *     faults surface at the caller's next synchronisation.
 *   - Shapes: M (tokens) >= 0; D, I and Dout are positive multiples of 64.
 *     With M == 0 the forward outputs are empty and dW1 and dW_down are
 *     written as zeros (a sum over no tokens).
 *   - Arithmetic: bf16 operands, fp32 accumulation and fp32 elementwise
 *     math, bf16 round-to-nearest-even stores.
 *   - A pointer may be NULL only when its tensor holds no elements (M == 0
 *     for the token-indexed tensors); weights and weight gradients never.
 *   - All argument checks run on the host before any HIP call, in this
 *     order: shapes, null pointers, alignment, workspace size, overlap.
 *     On any error nothing is launched and the status is returned.
 *   - Return value: SWIGLU_OK (0) or a negative swiglu_status.  No C++
 *     exception crosses this interface.
 */
#ifndef SWIGLU_MLP_H
#define SWIGLU_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWIGLU_OK = 0,
  SWIGLU_ERR_NULL = -1,        /* a required pointer is NULL                    */
  SWIGLU_ERR_SHAPE = -2,       /* a dimension is negative or zero where > 0 needed */
  SWIGLU_ERR_UNSUPPORTED = -3, /* D, I or Dout not a multiple of 64, or too large */
  SWIGLU_ERR_WORKSPACE = -4,   /* ws is NULL or ws_bytes below the query result  */
  SWIGLU_ERR_ALIAS = -5,       /* an output overlaps an input or another output  */
  SWIGLU_ERR_HIP = -6,         /* the HIP runtime reported an error at launch    */
  SWIGLU_ERR_ALIGN = -7        /* a tensor pointer is not 16-byte aligned        */
} swiglu_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* swiglu_status_string(int status);

/* ABI version of this header, (major << 16) | minor: 1.4. */
int swiglu_abi_version(void);

/* ---------------------------------------------------------------------------
 * Whole step
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace swiglu_mlp_fwd needs: the transient h [M,I], then
 * fp32 partial sums: those of the down GEMM's split tail when its last round of
 * 256x256 tiles is split over K (at 11136x3584x14336: 104 tiles x 2 parts, 54.5
 * MB), or, at 1 <= M <= 16, those of the decode path's split-K GEMMs (a few MB).
 * Size the workspace with this call; returns 0 for invalid shapes. */
size_t swiglu_mlp_fwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout);

/* Bytes of device workspace swiglu_mlp_bwd needs: grad_preact [M,2I] and the
 * recomputed h [M,I] (the drop-h report's extra backward buffers), then the fp32
 * partial tiles of the largest split tail among dW_down, dx and dW1 (at
 * 11136x3584x14336: dW1's 32 tiles x 8 parts, 67.1 MB).  Size the workspace
 * with this call; returns 0 for invalid shapes. */
size_t swiglu_mlp_bwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout);

/* Bytes of device workspace swiglu_mlp_bwd_unfused needs: as
 * swiglu_mlp_bwd plus the materialised dout [M,I]. */
size_t swiglu_mlp_bwd_unfused_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout);

/* Forward of the drop-h report.  Reads x [M,D], W1 [D,2I], W_down [I,Dout];
 * writes preact [M,2I] (the tensor the backward needs; the caller keeps it)
 * and y [M,Dout].  h is written to `ws` and is dead once the call's work has
 * run: the caller may reuse or free ws after the stream reaches that point.
 * The saved set for the backward is exactly {x, W1, W_down, preact}. */
int swiglu_mlp_fwd(const void* x, const void* W1, const void* W_down,
                   void* preact, void* y,
                   void* ws, size_t ws_bytes,
                   int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* Backward with the fused dgrad epilogue (the first note, section 4): the
 * dout GEMM keeps each dout tile on chip, and its epilogue reads the saved
 * [left | gate], recomputes sigma, silu and silu', and writes grad_preact and
 * h into `ws`; then dW_down = h^T.dy, dx = grad_preact.W1^T and
 * dW1 = x^T.grad_preact.  Reads the saved set and dy [M,Dout]; writes
 * dx [M,D], dW1 [D,2I], dW_down [I,Dout]. */
int swiglu_mlp_bwd(const void* x, const void* W1, const void* W_down, const void* preact,
                   const void* dy,
                   void* dx, void* dW1, void* dW_down,
                   void* ws, size_t ws_bytes,
                   int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* The unfused baseline the first note compares against (section 4): the
 * dout GEMM stores dout [M,I] in bf16 to `ws`, a separate elementwise kernel
 * reads it back with preact; the rest as swiglu_mlp_bwd.  Same outputs. */
int swiglu_mlp_bwd_unfused(const void* x, const void* W1, const void* W_down,
                           const void* preact, const void* dy,
                           void* dx, void* dW1, void* dW_down,
                           void* ws, size_t ws_bytes,
                           int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* ---------------------------------------------------------------------------
 * Save-h fallback (the drop-h report's "fallback path": the normal MLPBlock
 * that keeps h; its saved-tensor table lists h as saved by the baseline).
 * Same arithmetic as the drop-h calls; the saved set is {x, W1, W_down,
 * preact, h}, so the backward's dgrad epilogue writes grad_preact only.
 * ------------------------------------------------------------------------- */

/* No-allocation forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as swiglu_mlp_fwd without
 * ws / ws_bytes: the workspace (h and the split-K partial sums) is a
 * library-owned static device array of swiglu_mlp_fwd_noalloc_limit() bytes
 * (32 MiB) on each GPU, placed when the library is loaded on that GPU and
 * kept until the process ends; the first call on a device looks up its
 * address there.  Shapes whose swiglu_mlp_fwd_workspace exceeds the limit
 * (e.g. M * I * 2 > 32 MiB) are refused with SWIGLU_ERR_WORKSPACE before any
 * HIP call; the decode-shaped forward (M <= 16) needs about 4 MB at
 * D = 4096, I = 14336.  Nothing is read from the array before this call
 * writes it, so no clearing is needed.  Every call on one GPU uses that
 * GPU's one array: calls that may overlap on one GPU (on different streams
 * without ordering between them) race and must not be made.  Errors as
 * swiglu_mlp_fwd, plus SWIGLU_ERR_HIP if the array's address cannot be
 * obtained. */
size_t swiglu_mlp_fwd_noalloc_limit(void);
int swiglu_mlp_fwd_noalloc(const void* x, const void* W1, const void* W_down,
                           void* preact, void* y,
                           int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* Forward that keeps h: as swiglu_mlp_fwd, but h [M,I] is written to the
 * caller's `h` (part of the saved set) and no workspace is used (any M takes
 * the tiled path). */
int swiglu_mlp_fwd_save_h(const void* x, const void* W1, const void* W_down,
                          void* preact, void* h, void* y,
                          int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* Bytes of device workspace swiglu_mlp_bwd_saved_h needs: grad_preact [M,2I],
 * then the split tails' fp32 partial tiles as for swiglu_mlp_bwd.  Returns 0 for
 * invalid shapes. */
size_t swiglu_mlp_bwd_saved_h_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout);

/* Backward from the saved h: the fused dgrad GEMM writes grad_preact only
 * (swiglu_bwd_dgrad_fused_gp), dW_down = h^T.dy reads the saved h, then dx
 * and dW1 as in swiglu_mlp_bwd.  Reads x, W1, W_down, preact, h [M,I],
 * dy; writes dx, dW1, dW_down; grad_preact goes to `ws`. */
int swiglu_mlp_bwd_saved_h(const void* x, const void* W1, const void* W_down, const void* preact,
                           const void* h, const void* dy,
                           void* dx, void* dW1, void* dW_down,
                           void* ws, size_t ws_bytes,
                           int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* ---------------------------------------------------------------------------
 * Residual block Y = X + MLP(X) (Lesson 24, section 24, the residual-add
 * epilogue).  Requires Dout == D (else SWIGLU_ERR_SHAPE).  The add happens in
 * the epilogue of the GEMM that produces the MLP output, in fp32 before the
 * single bf16 rounding, so the bare MLP output never reaches HBM.  Same saved
 * set and workspaces as the drop-h calls.
 * ------------------------------------------------------------------------- */

/* As swiglu_mlp_fwd, with y = rn(x + h.W_down) [M,D].  Workspace: the
 * swiglu_mlp_fwd_workspace query. */
int swiglu_mlp_fwd_residual(const void* x, const void* W1, const void* W_down,
                            void* preact, void* y,
                            void* ws, size_t ws_bytes,
                            int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* As swiglu_mlp_bwd, with dx = rn(grad_preact.W1^T + dy): the identity
 * branch's gradient joins in the dx GEMM's epilogue.  dW1 and dW_down are the
 * plain MLP's.  Workspace: the swiglu_mlp_bwd_workspace query. */
int swiglu_mlp_bwd_residual(const void* x, const void* W1, const void* W_down, const void* preact,
                            const void* dy,
                            void* dx, void* dW1, void* dW_down,
                            void* ws, size_t ws_bytes,
                            int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream);

/* ---------------------------------------------------------------------------
 * Mixture-of-experts MLP blocks (Lesson 24, section 41: each expert is its
 * own SwiGLU MLP; sections 42-43: one grouped GEMM launch serves all experts
 * whatever their token counts).  The routed token rows arrive sorted and
 * packed by expert: expert e owns rows [group_offsets[e], group_offsets[e+1])
 * of x, preact, dy and dx.  Routing, sorting and All-to-All are the caller's.
 *
 * group_offsets: int32 [E + 1] in DEVICE memory (4-byte aligned), read by the
 * kernels, so the host never waits for the router.  It must run from 0 to M
 * without decreasing.  The host cannot check its contents: offsets outside
 * [0, M] are clamped and a decreasing pair makes that expert empty, so a bad
 * table gives unspecified results but no access outside the tensors.
 * Weights: W1 [E, D, 2I] and W_down [E, I, Dout], one block per expert, each
 * laid out as the dense block's.  1 <= E <= 65536 (else SWIGLU_ERR_SHAPE /
 * SWIGLU_ERR_UNSUPPORTED).  An expert with no rows gets zero weight
 * gradients.  The saved set for the backward is {x, W1, W_down,
 * group_offsets, preact}; h is recomputed as in swiglu_mlp_bwd.
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace swiglu_moe_fwd needs: the transient h [M,I].
 * Returns 0 for invalid arguments. */
size_t swiglu_moe_fwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E);

/* Bytes of device workspace swiglu_moe_bwd needs: grad_preact [M,2I] and h
 * [M,I].  Returns 0 for invalid arguments. */
size_t swiglu_moe_bwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E);

/* Forward of all experts: two grouped launches (GEMM-1 with the SwiGLU
 * epilogue, then the down GEMM).  x [M,D] -> preact [M,2I], y [M,Dout]. */
int swiglu_moe_fwd(const void* x, const void* W1, const void* W_down, const int32_t* group_offsets,
                   void* preact, void* y,
                   void* ws, size_t ws_bytes,
                   int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E, void* stream);

/* Backward of all experts: the grouped fused dgrad (dout per expert stays on
 * chip; the epilogue writes grad_preact and h to ws), then dW_down [E,I,Dout]
 * and dW1 [E,D,2I] as GEMMs grouped over the token (reduction) dimension, and
 * dx [M,D] grouped over rows.  Four launches. */
int swiglu_moe_bwd(const void* x, const void* W1, const void* W_down, const int32_t* group_offsets,
                   const void* preact, const void* dy,
                   void* dx, void* dW1, void* dW_down,
                   void* ws, size_t ws_bytes,
                   int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E, void* stream);

/* The grouped fused dgrad step alone (one launch): per expert e,
 * dout = dy_e . W_down[e]^T kept in fp32, and the epilogue of
 * swiglu_bwd_dgrad_fused.  dy [M,Dout], W_down [E,I,Dout], preact [M,2I] ->
 * grad_preact [M,2I], h [M,I]. */
int swiglu_moe_bwd_dgrad_fused(const void* dy, const void* W_down, const int32_t* group_offsets,
                               const void* preact, void* grad_preact, void* h,
                               int64_t M, int64_t I, int64_t Dout, int64_t E, void* stream);

/* ---------------------------------------------------------------------------
 * Single steps (each is one kernel launch; used by the whole-step calls
 * above, exported for timing and for step-level parity tests)
 * ------------------------------------------------------------------------- */

/* Forward GEMM-1 with the SwiGLU epilogue (the merged gate/up GEMM of
 * Lesson 24, sections 20-21): preact = x.W1 stored in bf16, and
 * h = rn(left * silu(gate)) computed from the bf16-rounded left and gate.
 * x [M,D], W1 [D,2I] -> preact [M,2I], h [M,I]. */
int swiglu_fwd_gemm1(const void* x, const void* W1, void* preact, void* h,
                     int64_t M, int64_t D, int64_t I, void* stream);

/* Forward down GEMM: y = h . W_down.  h [M,I], W_down [I,Dout] -> y [M,Dout]. */
int swiglu_fwd_down(const void* h, const void* W_down, void* y,
                    int64_t M, int64_t I, int64_t Dout, void* stream);

/* Fused dgrad + SwiGLU backward (the first note, sections 3-4; the drop-h
 * report's fused h / grad_preact kernel): dout = dy . W_down^T is
 * accumulated in fp32 and never leaves the chip; the epilogue writes
 * grad_preact = [dout*silu(gate) | dout*left*silu'(gate)] and
 * h = rn(left*silu(gate)).
 * dy [M,Dout], W_down [I,Dout], preact [M,2I] -> grad_preact [M,2I], h [M,I]. */
int swiglu_bwd_dgrad_fused(const void* dy, const void* W_down, const void* preact,
                           void* grad_preact, void* h,
                           int64_t M, int64_t I, int64_t Dout, void* stream);

/* The fused dgrad GEMM of the save-h fallback: as swiglu_bwd_dgrad_fused
 * without the h store.  dy [M,Dout], W_down [I,Dout], preact [M,2I] ->
 * grad_preact [M,2I]. */
int swiglu_bwd_dgrad_fused_gp(const void* dy, const void* W_down, const void* preact,
                              void* grad_preact, int64_t M, int64_t I, int64_t Dout, void* stream);

/* Down GEMM with the residual-add epilogue: y = rn(h.W_down + x).
 * h [M,I], W_down [I,D], x [M,D] -> y [M,D]. */
int swiglu_fwd_down_residual(const void* h, const void* W_down, const void* x, void* y,
                             int64_t M, int64_t I, int64_t D, void* stream);

/* dx GEMM with the residual-add epilogue: dx = rn(grad_preact.W1^T + dy).
 * grad_preact [M,2I], W1 [D,2I], dy [M,D] -> dx [M,D]. */
int swiglu_bwd_dx_residual(const void* grad_preact, const void* W1, const void* dy, void* dx,
                           int64_t M, int64_t D, int64_t I, void* stream);

/* Baseline dgrad GEMM: dout = dy . W_down^T rounded to bf16 and stored.
 * dy [M,Dout], W_down [I,Dout] -> dout [M,I]. */
int swiglu_bwd_dgrad_plain(const void* dy, const void* W_down, void* dout,
                           int64_t M, int64_t I, int64_t Dout, void* stream);

/* Baseline SwiGLU-backward elementwise kernel (the drop-h report's fused
 * h / grad_preact kernel, as a separate pass over HBM):
 * preact [M,2I], dout [M,I] -> grad_preact [M,2I], h [M,I]. */
int swiglu_bwd_elementwise(const void* preact, const void* dout,
                           void* grad_preact, void* h,
                           int64_t M, int64_t I, void* stream);

/* dW_down = h^T . dy.  h [M,I], dy [M,Dout] -> dW_down [I,Dout]. */
int swiglu_bwd_dw_down(const void* h, const void* dy, void* dW_down,
                       int64_t M, int64_t I, int64_t Dout, void* stream);

/* dx = grad_preact . W1^T.  grad_preact [M,2I], W1 [D,2I] -> dx [M,D]. */
int swiglu_bwd_dx(const void* grad_preact, const void* W1, void* dx,
                  int64_t M, int64_t D, int64_t I, void* stream);

/* dW1 = x^T . grad_preact, one merged [D,M].[M,2I] product (the first note,
 * section 3).  x [M,D], grad_preact [M,2I] -> dW1 [D,2I]. */
int swiglu_bwd_dw1(const void* x, const void* grad_preact, void* dW1,
                   int64_t M, int64_t D, int64_t I, void* stream);

/* The device activation functions on n bf16 inputs g (Lesson 24,
 * section 11; the first note, section 2, silu' forms), written as fp32:
 * sigma(g), silu(g) = g*sigma(g), silu'(g).  Same device code as the
 * epilogues.  n >= 0; outputs are float32 arrays of n elements; g needs
 * only 2-byte alignment, outputs 4-byte alignment. */
int swiglu_act_eval(const void* g, void* sigma, void* silu, void* dsilu,
                    int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_MLP_H */
