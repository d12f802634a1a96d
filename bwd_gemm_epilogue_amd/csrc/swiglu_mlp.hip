// swiglu_mlp.hip -- the SwiGLU MLP training step on gfx950, behind the C ABI
// declared in include/swiglu_mlp.h.
//
// Forward (the drop-h report, forward skeleton): GEMM-1 with a SwiGLU
// epilogue writes preact and a transient h; the down GEMM writes y.
// Backward (the note "SwiGLU MLP forward principle, backward chain and
// optimisation", sections 2-4): the dout GEMM runs with the SwiGLU-backward
// epilogue so dout never reaches HBM, then dW_down, dx and dW1.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "gemm_core.hpp"
#include "skinny.hpp"
#include "swiglu_math.hpp"
#include "swiglu_mlp.h"

#define SW_TRY(expr)                  \
  do {                                \
    int _s = (expr);                  \
    if (_s != SWIGLU_OK) return _s;   \
  } while (0)

namespace swg {

// ---------------------------------------------------------------------------
// Forward GEMM-1 epilogue.  The tile's B columns are paired (left block then
// the matching gate block), so slab columns [0, BN/2) hold left and
// [BN/2, BN) the gate of the same intermediate channels.  Stores the bf16
// preact halves and h = rn(left * silu(gate)) from the rounded values.
// ---------------------------------------------------------------------------
struct EpiSwigluFwd {
  static constexpr int kPrefetchDepth = 1, kLoadsPerItem = 0;
  struct Params {
    uint16_t* preact;  // [M, 2I]
    uint16_t* h;       // [M, I]
    int64_t I;
  };
  template <class T>
  struct Prefetch {};
  template <class T>
  __device__ static void prefetch_item(const Params&, const SlabCtx<T>&, Prefetch<T>&, int, int) {}
  template <class T, class Hook>
  __device__ static void apply(const Params& p, const SlabCtx<T>& c, Prefetch<T>&, int tid, Hook&& hook) {
    constexpr int HALF = T::BN / 2;
    constexpr int CPR = HALF / 8;
    constexpr int ITEMS = T::SLAB_ROWS * CPR;
    static_assert(ITEMS % T::THREADS == 0, "slab items must split evenly");
    const int I = (int)p.I;
    const int64_t rows = c.M - c.r0;
    const brsrc_t pdst = rows_rsrc(p.preact + (int64_t)c.r0 * 2 * p.I, rows * 4 * p.I);
    const brsrc_t hdst = rows_rsrc(p.h + (int64_t)c.r0 * p.I, rows * 2 * p.I);
#pragma unroll
    for (int k = 0; k < ITEMS / T::THREADS; ++k) {
      hook(k);  // this item's share of a later slab's reads, ahead of its stores
      const int it = tid + k * T::THREADS;
      const int sr = it / CPR, ch = it % CPR;
      const int rl = c.row(sr) - c.r0;
      const int i0 = c.tn * HALF + ch * 8;
      const u32x4 lp = pack8(c.read8(sr, ch * 8));
      const u32x4 gp = pack8(c.read8(sr, HALF + ch * 8));
      const f32x8 left = unpack8(lp), gate = unpack8(gp);
      f32x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = swiglu_h(left[e], gate[e]);
      // streaming stores: nothing in this kernel reads them back
      const uint32_t off = (uint32_t)(rl * 2 * I + i0) * 2u;
      bstore16(pdst, off, lp);
      bstore16(pdst, off + (uint32_t)I * 2u, gp);
      bstore16(hdst, (uint32_t)(rl * I + i0) * 2u, pack8(h));
    }
  }
};

// ---------------------------------------------------------------------------
// Fused dgrad epilogue (the centre of the method).  The slab holds fp32 dout
// for intermediate channels [tn*BN, tn*BN + BN).  For each 8-channel chunk it
// reads left = preact[:, i] and gate = preact[:, I + i] (issued before the
// slab is staged so the loads overlap the LDS traffic), recomputes sigma,
// silu and silu', and writes
//   grad_preact[:, i]     = dout * silu(gate)
//   grad_preact[:, I + i] = dout * left * silu'(gate)
//   h[:, i]               = rn(left * silu(gate))     (STORE_H: the drop-h
//                           path recomputes h here; the save-h fallback of
//                           the drop-h report kept h from the forward)
// ---------------------------------------------------------------------------
template <bool STORE_H>
struct EpiSwigluBwdT {
  // three slabs of preact reads in flight: the epilogue waits on their
  // latency otherwise
  static constexpr int kPrefetchDepth = 3, kLoadsPerItem = 2;
  struct Params {
    const uint16_t* preact;  // [M, 2I]
    uint16_t* grad_preact;   // [M, 2I]
    uint16_t* h;             // [M, I]
    int64_t I;
  };
  // the same epilogue for output columns n.. (left, gate and h move by n)
  static Params cols_from(const Params& p, int64_t n) {
    return {p.preact + n, p.grad_preact + n, p.h != nullptr ? p.h + n : nullptr, p.I};
  }
  template <class T>
  struct Prefetch {
    static constexpr int N = T::SLAB_ROWS * (T::BN / 8) / T::THREADS;
    u32x4 left[N], gate[N];
  };
  // Addresses are 32-bit byte offsets from the tile's first row: a tile
  // spans BM rows of at most 2^21 elements, well inside 2^31 bytes.  Item
  // k's row is q + item_row(k) (SlabCtx), so its offset is a per-thread base
  // plus item_row(k) times the row pitch, a scalar product.
  template <class T>
  __device__ static void prefetch_item(const Params& p, const SlabCtx<T>& c, Prefetch<T>& pf, int tid, int k) {
    constexpr int CPR = SlabCtx<T>::CPR;
    const uint32_t pitch = (uint32_t)p.I * 4u;  // bytes per preact row
    const brsrc_t src = rows_rsrc(p.preact + (int64_t)c.r0 * 2 * p.I, (int64_t)(c.M - c.r0) * 4 * p.I);
    const int q = tid / CPR, ch = tid % CPR;
    const uint32_t off = (uint32_t)q * pitch + (uint32_t)(c.tn * T::BN + ch * 8) * 2u + (uint32_t)c.item_row(k) * pitch;
    pf.left[k] = bload16(src, off);
    pf.gate[k] = bload16(src, off + pitch / 2u);
  }
  template <class T, class Hook>
  __device__ static void apply(const Params& p, const SlabCtx<T>& c, Prefetch<T>& pf, int tid, Hook&& hook) {
    constexpr int CPR = SlabCtx<T>::CPR, P = SlabCtx<T>::P;
    const uint32_t gpitch = (uint32_t)p.I * 4u, hpitch = (uint32_t)p.I * 2u;  // bytes per row
    const int64_t rows = c.M - c.r0;
    const brsrc_t gdst = rows_rsrc(p.grad_preact + (int64_t)c.r0 * 2 * p.I, rows * 4 * p.I);
    const brsrc_t hdst = rows_rsrc(STORE_H ? p.h + (int64_t)c.r0 * p.I : nullptr, STORE_H ? rows * 2 * p.I : 0);
    const int q = tid / CPR, ch = tid % CPR;
    const uint32_t col2 = (uint32_t)(c.tn * T::BN + ch * 8) * 2u;
    const uint32_t gbase = (uint32_t)q * gpitch + col2, hbase = (uint32_t)q * hpitch + col2;
#pragma unroll
    for (int k = 0; k < Prefetch<T>::N; ++k) {
      hook(k);  // this item's share of a later slab's reads, ahead of its stores
      const uint32_t r = (uint32_t)c.item_row(k);
      const f32x8 dout = c.read8(q + k * P, ch * 8);
      const f32x8 left = unpack8(pf.left[k]), gate = unpack8(pf.gate[k]);
      f32x8 dl, dg, h;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const Act a = sw_act(gate[e]);
        dl[e] = dout[e] * a.silu;
        dg[e] = (dout[e] * left[e]) * a.dsilu;
        h[e] = left[e] * a.silu;
      }
      const uint32_t off = gbase + r * gpitch;
      // streaming stores: nothing in this kernel reads them back
      bstore16(gdst, off, pack8(dl));
      bstore16(gdst, off + hpitch, pack8(dg));
      if constexpr (STORE_H) bstore16(hdst, hbase + r * hpitch, pack8(h));
    }
  }
};
typedef EpiSwigluBwdT<true> EpiSwigluBwd;     // drop-h backward: grad_preact and h
typedef EpiSwigluBwdT<false> EpiSwigluBwdGp;  // save-h backward: grad_preact only

// ---------------------------------------------------------------------------
// Baseline elementwise SwiGLU backward (the drop-h report's fused
// h / grad_preact kernel as its own pass): one 8-channel chunk per thread.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) swiglu_bwd_elementwise_kernel(const uint16_t* __restrict__ preact,
                                                                     const uint16_t* __restrict__ dout,
                                                                     uint16_t* __restrict__ grad_preact,
                                                                     uint16_t* __restrict__ h, int64_t M,
                                                                     int64_t I) {
  const int64_t chunks_per_row = I / 8;
  const int64_t total = M * chunks_per_row;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / chunks_per_row, i0 = (t % chunks_per_row) * 8;
    const uint16_t* pr = preact + row * 2 * I;
    const f32x8 left = unpack8(*(const u32x4*)(pr + i0));
    const f32x8 gate = unpack8(*(const u32x4*)(pr + I + i0));
    const f32x8 d = unpack8(*(const u32x4*)(dout + row * I + i0));
    f32x8 dl, dg, hh;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const Act a = sw_act(gate[e]);
      dl[e] = d[e] * a.silu;
      dg[e] = (d[e] * left[e]) * a.dsilu;
      hh[e] = left[e] * a.silu;
    }
    uint16_t* gpr = grad_preact + row * 2 * I;
    *(u32x4*)(gpr + i0) = pack8(dl);
    *(u32x4*)(gpr + I + i0) = pack8(dg);
    *(u32x4*)(h + row * I + i0) = pack8(hh);
  }
}

__global__ void __launch_bounds__(256) swiglu_act_eval_kernel(const uint16_t* __restrict__ g,
                                                              float* __restrict__ sigma,
                                                              float* __restrict__ silu,
                                                              float* __restrict__ dsilu, int64_t n) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    const float x = __builtin_bit_cast(float, (uint32_t)g[t] << 16);
    const Act a = sw_act(x);
    sigma[t] = a.sigma;
    silu[t] = a.silu;
    dsilu[t] = a.dsilu;
  }
}

// Zero fill (dW outputs of an empty batch).
__global__ void __launch_bounds__(256) zero_kernel(u32x4* __restrict__ p, int64_t n16) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n16; t += (int64_t)gridDim.x * blockDim.x)
    p[t] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace swg

// ===========================================================================
// Host side
// ===========================================================================

// Workspace of the no-allocation forward (swiglu_mlp_fwd_noalloc): the HIP
// runtime places one copy on each GPU that loads this library, kept until
// the process ends.  32 MiB holds h and the split-K partial sums of the
// decode-shaped forward (about 4.2 MB at 16 x 4096 x 14336) with room.
constexpr size_t kStaticWsBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

namespace {

using namespace swg;

// tile configurations: BM, BN, waves along M and N, BK
typedef TileCfg<256, 256, 2, 2, 64> TBig;  // 4 waves, 128x128 per wave, 160 KB LDS ring
typedef TileCfg<128, 128, 2, 2, 64> TMid;    // 4 waves, 64x64 per wave
typedef TileCfg<64, 64, 2, 2, 64> TSmall;      // 4 waves, 32x32 per wave (N % 128 != 0)
typedef TileCfg<256, 128, 2, 2, 64> TWide;   // 4 waves, 128x64 per wave
typedef TileCfg<128, 256, 2, 2, 64> TTall;   // 4 waves, 64x128 per wave

// D, I, Dout limit: keeps every in-tile byte offset of a 256-row tile below 2^31
constexpr int64_t kMaxDim = (int64_t)1 << 20;

struct Range {
  uintptr_t lo, hi;
};

Range rng(const void* p, int64_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// every output range must be disjoint from every input and from the other outputs
int check_alias(const Range* ins, int n_in, const Range* outs, int n_out) {
  for (int o = 0; o < n_out; ++o) {
    for (int i = 0; i < n_in; ++i)
      if (overlap(outs[o], ins[i])) return SWIGLU_ERR_ALIAS;
    for (int j = o + 1; j < n_out; ++j)
      if (overlap(outs[o], outs[j])) return SWIGLU_ERR_ALIAS;
  }
  return SWIGLU_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// a pointer may be NULL only when its tensor holds no bytes
bool missing(const void* p, int64_t bytes) { return p == nullptr && bytes > 0; }

int check_inner(int64_t d) {
  if (d <= 0) return SWIGLU_ERR_SHAPE;
  if (d % 64 != 0 || d > kMaxDim) return SWIGLU_ERR_UNSUPPORTED;
  return SWIGLU_OK;
}

int check_tokens(int64_t M) {
  if (M < 0) return SWIGLU_ERR_SHAPE;
  if (M > ((int64_t)1 << 31) - 1) return SWIGLU_ERR_UNSUPPORTED;
  return SWIGLU_OK;
}

int check_dims(int64_t M, int64_t D, int64_t I, int64_t Dout) {
  int s;
  if ((s = check_tokens(M))) return s;
  if ((s = check_inner(D))) return s;
  if ((s = check_inner(I))) return s;
  if ((s = check_inner(Dout))) return s;
  return SWIGLU_OK;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int launch_status() { return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_HIP; }

template <class T, bool A_K, bool B_K, class Epi>
int run_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
             int pair_off, const typename Epi::Params& ep, hipStream_t st) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.tiles_m = (int)((M + T::BM - 1) / T::BM);
  g.tiles_n = pair_off > 0 ? (int)(N / T::BN) : (int)((N + T::BN - 1) / T::BN);
  g.pair_off = pair_off;
  const int64_t tiles = (int64_t)g.tiles_m * g.tiles_n;
  g.tile_count = (int)tiles;
  if (tiles == 0) return SWIGLU_OK;
  hipLaunchKernelGGL((gemm_kernel<T, A_K, B_K, Epi>), dim3((unsigned)tiles), dim3(T::THREADS), 0, st, g, ep);
  return launch_status();
}

// Pick the largest tile whose N extent divides the GEMM's N (for the paired
// forward GEMM-1, whose half tile must divide I).
template <bool A_K, bool B_K, class Epi>
int run_gemm_auto(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                  int pair_off, const typename Epi::Params& ep, hipStream_t st) {
  const int64_t n_unit = pair_off > 0 ? N / 2 : N;  // channels per half for paired tiles
  const int64_t div = pair_off > 0 ? 2 : 1;
  if (n_unit % (TBig::BN / div) == 0 && M > 256)
    return run_gemm<TBig, A_K, B_K, Epi>(A, lda, B, ldb, M, N, K, pair_off, ep, st);
  if (n_unit % (TMid::BN / div) == 0)
    return run_gemm<TMid, A_K, B_K, Epi>(A, lda, B, ldb, M, N, K, pair_off, ep, st);
  return run_gemm<TSmall, A_K, B_K, Epi>(A, lda, B, ldb, M, N, K, pair_off, ep, st);
}

// --- split tail: the last, partly filled round of 256x256 tiles ------------
// A GEMM of T tiles on C compute units runs floor(T / C) full rounds and a
// last round of R = T mod C tiles in which most units idle.  When it pays,
// the R tail tiles have their K range cut into S parts: R * S workgroups
// write fp32 partial tiles to workspace and a small kernel adds each tile's
// parts in order.  Plain bf16-store GEMMs only (the sum must be linear);
// used by the whole-step calls, which own a workspace.

constexpr int kComputeUnits = 256;  // MI355X

// Compute units of the current device, queried once per device (0 on a HIP
// error).  The split-tail and decode plans are worked out for kComputeUnits
// (the workspace queries stay free of HIP calls); a launch on a device with
// another count runs unsplit instead (plans_hold()).
int device_compute_units() {
  static int cached[64];  // 0 = not yet queried; racing writers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

bool plans_hold() { return device_compute_units() == kComputeUnits; }

// --- tile shape of the dout GEMMs (K-major dy and W_down) ------------------
// A launch of T tiles on C compute units runs floor(T / C) full rounds and
// a last round of T mod C tiles, whose cost is taken as 0.5 + 0.5 * (T mod
// C) / C of a round (the split-tail model below).  Each tile shape works at
// its own rate per compute unit, measured on the fused dgrad with the same
// k-loop relative to 256 x 256 tiles: 256 x 128 0.945, 128 x 256 0.903,
// 128 x 128 0.723.  The shape of least (rounds x tile area / rate) is used:
// at 11136 x 14336 (K 3584) and 8192 x 11008 (K 4096) that is 256 x 256
// (measured best or tied); at 2048 x 2816, 4096 x 5632 and 11136 x 1792 a
// 256- or 128-row half-size tile (measured 1.53x, 1.12x and 1.13x faster).
enum KkTile { kTileBig, kTileWide, kTileTall, kTileMid, kTileSmall };

KkTile pick_kk_tile(int64_t M, int64_t N, int cus) {
  if (N % 128 != 0) return kTileSmall;
  struct Cand {
    KkTile k;
    int bm, bn;
    double rate;
  };
  const Cand cands[] = {{kTileBig, 256, 256, 1.0},
                        {kTileWide, 256, 128, 0.945},
                        {kTileTall, 128, 256, 0.903},
                        {kTileMid, 128, 128, 0.723}};
  const int64_t C = cus > 0 ? cus : 256;
  KkTile best = kTileMid;
  double best_cost = 0.0;
  bool any = false;
  for (const Cand& c : cands) {
    if (N % c.bn != 0) continue;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * (N / c.bn);
    const int64_t full = tiles / C, rem = tiles % C;
    const double rounds = (double)full + (rem > 0 ? 0.5 + 0.5 * (double)rem / (double)C : 0.0);
    const double cost = rounds * c.bm * c.bn / c.rate;
    if (!any || cost < best_cost - 1e-9) {
      best = c.k;
      best_cost = cost;
      any = true;
    }
  }
  return best;
}

// The cost of one launch in the model above, in units of one round of
// 256 x 256 tiles; -1 when the shape does not divide N.
double kk_cost(int64_t M, int64_t N, KkTile k, int64_t C) {
  static const int bm[] = {256, 256, 128, 128}, bn[] = {256, 128, 256, 128};
  static const double rate[] = {1.0, 0.945, 0.903, 0.723};
  if (k > kTileMid || N <= 0 || N % bn[k] != 0) return -1.0;
  const int64_t tiles = ((M + bm[k] - 1) / bm[k]) * (N / bn[k]);
  const int64_t full = tiles / C, rem = tiles % C;
  const double rounds = (double)full + (rem > 0 ? 0.5 + 0.5 * (double)rem / (double)C : 0.0);
  return rounds * bm[k] * bn[k] / rate[k] / 65536.0;
}

// A launch plan for the dout GEMM: one launch in the shape pick_kk_tile
// chooses, or 256 x 256 tiles over the first n1 columns and another shape
// over the rest, when that fills the rounds better by the same model (a
// second launch counted as 0.02 of a round).  At 8192 x 11008 the 1376 tiles
// of 256 x 256 run 5.4 rounds; 1280 of them (40 tile columns) fill 5 and the
// last 768 columns run as 192 tiles of 256 x 128.
struct KkPlan {
  KkTile first;
  int64_t n1;  // columns of the first launch (N: one launch)
  KkTile second;
};
KkPlan plan_kk(int64_t M, int64_t N, int cus) {
  const KkTile one = pick_kk_tile(M, N, cus);
  KkPlan best{one, N, one};
  if (one == kTileSmall || cus <= 0) return best;
  double best_cost = kk_cost(M, N, one, cus);
  for (int64_t n1 = 256; n1 < N; n1 += 256) {
    const double c1 = kk_cost(M, n1, kTileBig, cus);
    for (int k = kTileBig; k <= kTileMid; ++k) {
      const double c2 = kk_cost(M, N - n1, (KkTile)k, cus);
      if (c1 < 0 || c2 < 0) continue;
      if (c1 + c2 + 0.02 < best_cost - 1e-9) {
        best = {kTileBig, n1, (KkTile)k};
        best_cost = c1 + c2 + 0.02;
      }
    }
  }
  return best;
}

template <class Epi>
int run_gemm_kk_one(KkTile k, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N,
                    int64_t K, const typename Epi::Params& ep, hipStream_t st) {
  switch (k) {
    case kTileBig: return run_gemm<TBig, true, true, Epi>(A, lda, B, ldb, M, N, K, 0, ep, st);
    case kTileWide: return run_gemm<TWide, true, true, Epi>(A, lda, B, ldb, M, N, K, 0, ep, st);
    case kTileTall: return run_gemm<TTall, true, true, Epi>(A, lda, B, ldb, M, N, K, 0, ep, st);
    case kTileMid: return run_gemm<TMid, true, true, Epi>(A, lda, B, ldb, M, N, K, 0, ep, st);
    default: return run_gemm<TSmall, true, true, Epi>(A, lda, B, ldb, M, N, K, 0, ep, st);
  }
}

// A K-major x K-major GEMM (the dout GEMM and its plain-store twin) by
// plan_kk: the second launch covers columns [n1, N), B's rows and the
// epilogue's column base moved by n1 (Epi::cols_from).
template <class Epi>
int run_gemm_kk(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                const typename Epi::Params& ep, hipStream_t st) {
  const KkPlan pl = plan_kk(M, N, device_compute_units());
  int s = run_gemm_kk_one<Epi>(pl.first, A, lda, B, ldb, M, pl.n1, K, ep, st);
  if (s != SWIGLU_OK || pl.n1 == N) return s;
  return run_gemm_kk_one<Epi>(pl.second, A, lda, B + pl.n1 * ldb, ldb, M, N - pl.n1, K, Epi::cols_from(ep, pl.n1), st);
}

struct Scratch {
  float* p = nullptr;
  size_t bytes = 0;
};

struct SplitPlan {
  int full = 0, rem = 0, S = 1;  // full rounds x units, tail tiles, parts per tail tile
  size_t bytes = 0;              // partial tiles: rem * S * 256 * 256 * 4
};

// The plan for a TBig GEMM (N a multiple of 256, M > 256).  The tail's cost
// in units of one round of tile work, for S parts per tile:
//   ceil(rem * S / C) / S                     rounds of 1/S-long workgroups
//   + 2 * rem * S * 256 KB / (5 TB/s)          partial tiles written and read
//     / (256 * 256 * K * 2 FLOP / 5.5 TFLOP/s)  one tile's main loop on one CU
// (the two rates are round figures measured on MI355X; a dx round of
// 256x256x28672 tiles takes ~670 us, 5.6 TFLOP/s per CU).  Unsplit, a last
// round with few busy units runs faster than a full one: its cost is taken
// as 0.5 + 0.5 * rem / C (measured: 0.72 with 41% of the units busy).  The S
// in 2..16 (at most the k-stages) of least cost is kept when it saves at
// least 15% of that.  At the 11136 x 3584 x 14336 block this picks S = 2
// for dx (7 with the 4.5 TFLOP/s figure of a slower core: the whole-step
// backward measured 40-70 us faster with 2) and keeps the down GEMM's S = 2.
SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  SplitPlan pl;
  if (M <= 256 || N % TBig::BN != 0 || K <= 0) return pl;
  const int64_t tiles = ((M + TBig::BM - 1) / TBig::BM) * (N / TBig::BN);
  const int64_t full = tiles / kComputeUnits, rem = tiles % kComputeUnits;
  const int64_t nst = (K + TBig::BK - 1) / TBig::BK;
  if (full < 1 || rem == 0) return pl;
  const double tile_bytes = (double)TBig::BM * TBig::BN * 4;
  const double round_us = 2.0 * TBig::BM * TBig::BN * (double)K / 5.5e6;
  double best = 1.0;
  int bestS = 1;
  for (int S = 2; S <= 16 && S <= nst; ++S) {
    const double rounds = (double)((rem * S + kComputeUnits - 1) / kComputeUnits) / S;
    const double traffic_us = 2.0 * rem * S * tile_bytes / 5e6;
    const double cost = rounds + traffic_us / round_us;
    if (cost < best - 1e-9) {
      best = cost;
      bestS = S;
    }
  }
  const double unsplit = 0.5 + 0.5 * (double)rem / kComputeUnits;
  if (bestS < 2 || best > 0.85 * unsplit) return pl;
  pl.full = (int)(full * kComputeUnits);
  pl.rem = (int)rem;
  pl.S = bestS;
  pl.bytes = (size_t)rem * bestS * TBig::BM * TBig::BN * 4;
  return pl;
}

// A plain bf16-store GEMM, with the split tail when the plan has one and
// the scratch holds it; else one dense launch.
template <bool A_K, bool B_K>
int run_store_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                   const EpiStore::Params& ep, Scratch sc, hipStream_t st) {
  const SplitPlan pl = split_plan(M, N, K);
  if (pl.S < 2 || !sc.p || sc.bytes < pl.bytes || !plans_hold())
    return run_gemm_auto<A_K, B_K, EpiStore>(A, lda, B, ldb, M, N, K, 0, ep, st);
  typedef TBig T;
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.tiles_m = (int)((M + T::BM - 1) / T::BM);
  g.tiles_n = (int)(N / T::BN);
  g.tile_count = pl.full;
  hipLaunchKernelGGL((gemm_kernel<T, A_K, B_K, EpiStore>), dim3((unsigned)pl.full), dim3(T::THREADS), 0, st, g, ep);
  SW_TRY(launch_status());
  g.tile_base = pl.full;
  g.splits = pl.S;
  EpiPartial::Params pp{sc.p};
  hipLaunchKernelGGL((gemm_kernel<T, A_K, B_K, EpiPartial, kSplitTail>), dim3((unsigned)(pl.rem * pl.S)),
                     dim3(T::THREADS), 0, st, g, pp);
  SW_TRY(launch_status());
  constexpr int PER_TILE = T::BM * T::BN / 8 / 256;
  hipLaunchKernelGGL((split_reduce_kernel<T, group_rows<A_K>()>), dim3((unsigned)(pl.rem * PER_TILE)), dim3(256), 0, st, (const float*)sc.p,
                     pl.S, pl.full, g.tiles_m, g.tiles_n, (int)M, (int)N, ep.C, ep.ldc);
  return launch_status();
}

// --- decode-shaped forward (at most 16 token rows) -------------------------

// The skinny path: 1..16 rows and column counts that are whole 128-column
// workgroups (K is a multiple of 64 for every GEMM here).
bool skinny_fits(int64_t M, int64_t N) { return M >= 1 && M <= 16 && N % SK_BN == 0; }

// Split-K factor for BN-wide column blocks: at most one workgroup per CU,
// with every split non-empty.  At 16 x 4096 x 14336 one workgroup per CU
// (GEMM-1: 2 splits of 112 blocks, the down GEMM: 8 of 32) measured 66 us
// per forward against 71 us at two per CU and 72-79 us at three or four:
// longer streams per workgroup and fewer partial sums to add.
// stages_per_split is returned through *spp.
int skinny_splits(int64_t N, int64_t K, int bn, int* spp) {
  const int64_t nblk = N / bn, nk = K / SK_BK;
  int64_t S = kComputeUnits / nblk;
  if (S < 1) S = 1;
  if (S > nk) S = nk;
  const int64_t per = (nk + S - 1) / S;
  *spp = (int)per;
  return (int)((nk + per - 1) / per);
}

// Column-block width: 256 (512-byte runs of each W row) for GEMM-1's wide
// [D, 2I] when it divides; 128 otherwise (the down GEMM's narrower W would
// get too few, too short streams at 256).
int skinny_bn_gemm1(int64_t I) { return (2 * I) % 256 == 0 ? 256 : SK_BN; }

bool fwd_is_skinny(int64_t M, int64_t I, int64_t Dout) { return skinny_fits(M, 2 * I) && skinny_fits(M, Dout); }

size_t skinny_partial_bytes(int64_t D, int64_t I, int64_t Dout) {
  int spp;
  const size_t a = (size_t)skinny_splits(2 * I, D, skinny_bn_gemm1(I), &spp) * 16 * (size_t)(2 * I) * 4;
  const size_t b = (size_t)skinny_splits(Dout, I, SK_BN, &spp) * 16 * (size_t)Dout * 4;
  return a > b ? a : b;
}

int run_skinny(const void* X, int64_t ldx, const void* W, int64_t M, int64_t N, int64_t K, int bn, float* partial,
               hipStream_t st, int* S_out) {
  SkinnyArgs a;
  a.X = (const uint16_t*)X;
  a.W = (const uint16_t*)W;
  a.partial = partial;
  a.ldx = ldx;
  a.ldw = N;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  const int S = skinny_splits(N, K, bn, &a.stages_per_split);
  *S_out = S;
  if (bn == 256)
    hipLaunchKernelGGL(skinny_gemm_kernel<256>, dim3((unsigned)(N / 256), (unsigned)S), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(skinny_gemm_kernel<SK_BN>, dim3((unsigned)(N / SK_BN), (unsigned)S), dim3(256), 0, st, a);
  return launch_status();
}

// residual: nullptr, or x itself for the residual block (Dout == D)
int fwd_skinny(const void* x, const void* W1, const void* Wd, void* preact, void* y, void* h, float* partial,
               int64_t M, int64_t D, int64_t I, int64_t Dout, hipStream_t st, const void* residual = nullptr) {
  int S;
  SW_TRY(run_skinny(x, D, W1, M, 2 * I, D, skinny_bn_gemm1(I), partial, st, &S));
  const int64_t t1 = M * (I / 8);
  // 64-thread workgroups: these short, latency-bound reductions then spread
  // over more CUs (measured 1.3 us less per forward than 256-thread ones)
  hipLaunchKernelGGL(skinny_swiglu_reduce_kernel, dim3((unsigned)((t1 + 63) / 64)), dim3(64), 0, st, partial, S,
                     (int)M, I, (uint16_t*)preact, (uint16_t*)h);
  SW_TRY(launch_status());
  SW_TRY(run_skinny(h, I, Wd, M, Dout, I, SK_BN, partial, st, &S));
  const int64_t t2 = M * (Dout / 8);
  hipLaunchKernelGGL(skinny_store_reduce_kernel, dim3((unsigned)((t2 + 63) / 64)), dim3(64), 0, st, partial, S,
                     (int)M, Dout, (uint16_t*)y, (const uint16_t*)residual);
  return launch_status();
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

const uint16_t* cu16(const void* p) { return (const uint16_t*)p; }
uint16_t* u16(void* p) { return (uint16_t*)p; }

// --- steps (no argument checks: callers have validated) --------------------

int step_gemm1(const void* x, const void* W1, void* preact, void* h, int64_t M, int64_t D, int64_t I,
               hipStream_t st) {
  EpiSwigluFwd::Params ep{u16(preact), u16(h), I};
  return run_gemm_auto<true, false, EpiSwigluFwd>(cu16(x), D, cu16(W1), 2 * I, M, 2 * I, D, (int)I, ep, st);
}

int step_down(const void* h, const void* Wd, void* y, int64_t M, int64_t I, int64_t Dout, hipStream_t st,
              Scratch sc = {}) {
  EpiStore::Params ep{u16(y), Dout};
  return run_store_gemm<true, false>(cu16(h), I, cu16(Wd), Dout, M, Dout, I, ep, sc, st);
}

int step_dgrad_fused(const void* dy, const void* Wd, const void* preact, void* gp, void* h, int64_t M, int64_t I,
                     int64_t Dout, hipStream_t st) {
  EpiSwigluBwd::Params ep{cu16(preact), u16(gp), u16(h), I};
  return run_gemm_kk<EpiSwigluBwd>(cu16(dy), Dout, cu16(Wd), Dout, M, I, Dout, ep, st);
}

// residual-add epilogues (Lesson 24, section 24): y = x + h.W_down and, in
// the backward of the residual block, dx = grad_preact.W1^T + dy
int step_down_residual(const void* h, const void* Wd, const void* x, void* y, int64_t M, int64_t I, int64_t D,
                       hipStream_t st) {
  EpiStoreResidual::Params ep{u16(y), D, cu16(x), D};
  return run_gemm_auto<true, false, EpiStoreResidual>(cu16(h), I, cu16(Wd), D, M, D, I, 0, ep, st);
}

int step_dx_residual(const void* gp, const void* W1, const void* dy, void* dx, int64_t M, int64_t D, int64_t I,
                     hipStream_t st) {
  EpiStoreResidual::Params ep{u16(dx), D, cu16(dy), D};
  return run_gemm_auto<true, true, EpiStoreResidual>(cu16(gp), 2 * I, cu16(W1), 2 * I, M, D, 2 * I, 0, ep, st);
}

int step_dgrad_fused_gp(const void* dy, const void* Wd, const void* preact, void* gp, int64_t M, int64_t I,
                        int64_t Dout, hipStream_t st) {
  EpiSwigluBwdGp::Params ep{cu16(preact), u16(gp), nullptr, I};
  return run_gemm_kk<EpiSwigluBwdGp>(cu16(dy), Dout, cu16(Wd), Dout, M, I, Dout, ep, st);
}

int step_dgrad_plain(const void* dy, const void* Wd, void* dout, int64_t M, int64_t I, int64_t Dout,
                     hipStream_t st) {
  EpiStore::Params ep{u16(dout), I};
  return run_gemm_kk<EpiStore>(cu16(dy), Dout, cu16(Wd), Dout, M, I, Dout, ep, st);
}

int step_elementwise(const void* preact, const void* dout, void* gp, void* h, int64_t M, int64_t I, hipStream_t st) {
  const int64_t total = M * (I / 8);
  if (total == 0) return SWIGLU_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(swiglu_bwd_elementwise_kernel, dim3((unsigned)blocks), dim3(256), 0, st, cu16(preact),
                     cu16(dout), u16(gp), u16(h), M, I);
  return launch_status();
}

int step_zero(void* p, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return SWIGLU_OK;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (u32x4*)p, n16);
  return launch_status();
}

int step_dw_down(const void* h, const void* dy, void* dWd, int64_t M, int64_t I, int64_t Dout, hipStream_t st,
                 Scratch sc = {}) {
  if (M == 0) return step_zero(dWd, I * Dout * 2, st);
  EpiStore::Params ep{u16(dWd), Dout};
  return run_store_gemm<false, false>(cu16(h), I, cu16(dy), Dout, I, Dout, M, ep, sc, st);
}

int step_dx(const void* gp, const void* W1, void* dx, int64_t M, int64_t D, int64_t I, hipStream_t st,
            Scratch sc = {}) {
  EpiStore::Params ep{u16(dx), D};
  return run_store_gemm<true, true>(cu16(gp), 2 * I, cu16(W1), 2 * I, M, D, 2 * I, ep, sc, st);
}

int step_dw1(const void* x, const void* gp, void* dW1, int64_t M, int64_t D, int64_t I, hipStream_t st,
             Scratch sc = {}) {
  if (M == 0) return step_zero(dW1, D * 2 * I * 2, st);
  EpiStore::Params ep{u16(dW1), 2 * I};
  return run_store_gemm<false, false>(cu16(x), D, cu16(gp), 2 * I, D, 2 * I, M, ep, sc, st);
}

// split-tail scratch of the forward (the down GEMM) and of the backward's
// plain-store GEMMs (dW_down, dx, dW1 run one after another and share it)
size_t fwd_split_bytes(int64_t M, int64_t I, int64_t Dout) { return split_plan(M, Dout, I).bytes; }
size_t bwd_split_bytes(int64_t M, int64_t D, int64_t I, int64_t Dout) {
  size_t b = split_plan(I, Dout, M).bytes;
  const size_t c = split_plan(M, D, 2 * I).bytes, d = split_plan(D, 2 * I, M).bytes;
  if (c > b) b = c;
  if (d > b) b = d;
  return b;
}

// --- grouped GEMMs: the experts of a mixture-of-experts layer (Lesson 24,
// sections 41-43).  Token rows are packed by expert; offsets [E + 1] live in
// device memory, so routing needs no host round trip: every workgroup finds
// its expert on the device. ----------------------------------------------

template <class T, bool A_K, bool B_K, class Epi, int GRP>
int run_gemm_grouped(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N,
                     int64_t K, int pair_off, const int* off, int64_t E, int64_t stride_b, int64_t stride_c,
                     const typename Epi::Params& ep, hipStream_t st) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.tiles_n = pair_off > 0 ? (int)(N / T::BN) : (int)((N + T::BN - 1) / T::BN);
  g.pair_off = pair_off;
  g.group_off = off;
  g.groups = (int)E;
  g.group_stride_b = stride_b;
  g.group_stride_c = stride_c;
  int64_t tiles;
  if (GRP == kGroupM) {
    // each group adds at most one partly filled tile row
    const int64_t rows = (M + T::BM - 1) / T::BM + E;
    g.tiles_m = (int)rows;
    tiles = rows * g.tiles_n;
  } else {
    g.tiles_m = (int)((M + T::BM - 1) / T::BM);
    tiles = E * g.tiles_m * g.tiles_n;
  }
  if (tiles == 0) return SWIGLU_OK;
  if (tiles > 0x7FFFFFFFll) return SWIGLU_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_kernel<T, A_K, B_K, Epi, GRP>), dim3((unsigned)tiles), dim3(T::THREADS), 0, st, g, ep);
  return launch_status();
}

// Tile choice as for one GEMM, with the rows per expert (grouped over M) or
// the output rows (grouped over K) in the role of M.
template <bool A_K, bool B_K, class Epi, int GRP>
int run_grouped_auto(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                     int pair_off, const int* off, int64_t E, int64_t stride_b, int64_t stride_c,
                     const typename Epi::Params& ep, hipStream_t st) {
  const int64_t n_unit = pair_off > 0 ? N / 2 : N;
  const int64_t div = pair_off > 0 ? 2 : 1;
  const int64_t rows = GRP == kGroupM ? M / E : M;
  if (n_unit % (TBig::BN / div) == 0 && rows > 256)
    return run_gemm_grouped<TBig, A_K, B_K, Epi, GRP>(A, lda, B, ldb, M, N, K, pair_off, off, E, stride_b, stride_c,
                                                      ep, st);
  if (n_unit % (TMid::BN / div) == 0)
    return run_gemm_grouped<TMid, A_K, B_K, Epi, GRP>(A, lda, B, ldb, M, N, K, pair_off, off, E, stride_b, stride_c,
                                                      ep, st);
  return run_gemm_grouped<TSmall, A_K, B_K, Epi, GRP>(A, lda, B, ldb, M, N, K, pair_off, off, E, stride_b, stride_c,
                                                      ep, st);
}

// The six GEMMs of the expert MLP block, each one launch over all experts.
// M is the routed row count; W1 [E, D, 2I], W_down [E, I, Dout].
int moe_gemm1(const void* x, const void* W1, const int* off, void* preact, void* h, int64_t M, int64_t D, int64_t I,
              int64_t E, hipStream_t st) {
  EpiSwigluFwd::Params ep{u16(preact), u16(h), I};
  return run_grouped_auto<true, false, EpiSwigluFwd, kGroupM>(cu16(x), D, cu16(W1), 2 * I, M, 2 * I, D, (int)I, off, E,
                                                               D * 2 * I, 0, ep, st);
}

int moe_down(const void* h, const void* Wd, const int* off, void* y, int64_t M, int64_t I, int64_t Dout, int64_t E,
             hipStream_t st) {
  EpiStore::Params ep{u16(y), Dout};
  return run_grouped_auto<true, false, EpiStore, kGroupM>(cu16(h), I, cu16(Wd), Dout, M, Dout, I, 0, off, E, I * Dout,
                                                           0, ep, st);
}

int moe_dgrad_fused(const void* dy, const void* Wd, const int* off, const void* preact, void* gp, void* h, int64_t M,
                    int64_t I, int64_t Dout, int64_t E, hipStream_t st) {
  EpiSwigluBwd::Params ep{cu16(preact), u16(gp), u16(h), I};
  return run_grouped_auto<true, true, EpiSwigluBwd, kGroupM>(cu16(dy), Dout, cu16(Wd), Dout, M, I, Dout, 0, off, E,
                                                              I * Dout, 0, ep, st);
}

int moe_dw_down(const void* h, const void* dy, const int* off, void* dWd, int64_t M, int64_t I, int64_t Dout,
                int64_t E, hipStream_t st) {
  EpiStore::Params ep{u16(dWd), Dout};
  return run_grouped_auto<false, false, EpiStore, kGroupK>(cu16(h), I, cu16(dy), Dout, I, Dout, M, 0, off, E, 0,
                                                            I * Dout, ep, st);
}

int moe_dx(const void* gp, const void* W1, const int* off, void* dx, int64_t M, int64_t D, int64_t I, int64_t E,
           hipStream_t st) {
  EpiStore::Params ep{u16(dx), D};
  return run_grouped_auto<true, true, EpiStore, kGroupM>(cu16(gp), 2 * I, cu16(W1), 2 * I, M, D, 2 * I, 0, off, E,
                                                          D * 2 * I, 0, ep, st);
}

int moe_dw1(const void* x, const void* gp, const int* off, void* dW1, int64_t M, int64_t D, int64_t I, int64_t E,
            hipStream_t st) {
  EpiStore::Params ep{u16(dW1), 2 * I};
  return run_grouped_auto<false, false, EpiStore, kGroupK>(cu16(x), D, cu16(gp), 2 * I, D, 2 * I, M, 0, off, E, 0,
                                                            D * 2 * I, ep, st);
}

int check_experts(int64_t E) { return E < 1 ? SWIGLU_ERR_SHAPE : (E > 65536 ? SWIGLU_ERR_UNSUPPORTED : SWIGLU_OK); }

// --- the no-allocation forward's workspace --------------------------------
// `scratch` (file scope, above) is a library-owned device array per GPU.
// Its name is a host-side stand-in: host code uses only the device address
// hipGetSymbolAddress returns for the current device, taken once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (first call on a device: with
// that device current, hipGetSymbolAddress, checked).
int static_workspace(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SWIGLU_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SWIGLU_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SWIGLU_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* swiglu_status_string(int status) {
  switch (status) {
    case SWIGLU_OK: return "SWIGLU_OK";
    case SWIGLU_ERR_NULL: return "SWIGLU_ERR_NULL: a required pointer is NULL";
    case SWIGLU_ERR_SHAPE: return "SWIGLU_ERR_SHAPE: a dimension is negative or zero";
    case SWIGLU_ERR_UNSUPPORTED: return "SWIGLU_ERR_UNSUPPORTED: D, I and Dout must be multiples of 64 (and sizes in range)";
    case SWIGLU_ERR_WORKSPACE: return "SWIGLU_ERR_WORKSPACE: workspace missing or too small";
    case SWIGLU_ERR_ALIAS: return "SWIGLU_ERR_ALIAS: an output overlaps an input or another output";
    case SWIGLU_ERR_HIP: return "SWIGLU_ERR_HIP: the HIP runtime reported an error";
    case SWIGLU_ERR_ALIGN: return "SWIGLU_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    default: return "unknown swiglu status";
  }
}

int swiglu_abi_version(void) { return (1 << 16) | 4; }

// Workspace layouts (each part 256-byte aligned):
//   forward          h [M,I] | skinny partial sums or the down GEMM's split tail
//   backward         grad_preact [M,2I] | h [M,I] | split tail of dW_down, dx, dW1
//   unfused backward grad_preact | h | dout [M,I] | split tail
size_t swiglu_mlp_fwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout) {
  if (check_dims(M, D, I, Dout) != SWIGLU_OK) return 0;
  const size_t h = align256((size_t)(M * I * 2));
  return fwd_is_skinny(M, I, Dout) ? h + skinny_partial_bytes(D, I, Dout) : h + fwd_split_bytes(M, I, Dout);
}

size_t swiglu_mlp_bwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout) {
  if (check_dims(M, D, I, Dout) != SWIGLU_OK) return 0;
  return align256((size_t)(M * 2 * I * 2)) + align256((size_t)(M * I * 2)) + bwd_split_bytes(M, D, I, Dout);
}

size_t swiglu_mlp_bwd_unfused_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout) {
  if (check_dims(M, D, I, Dout) != SWIGLU_OK) return 0;
  return swiglu_mlp_bwd_workspace(M, D, I, Dout) + align256((size_t)(M * I * 2));
}

// The forward after its checks: ws holds at least need bytes.
static int fwd_launch(const void* x, const void* W1, const void* W_down, void* preact, void* y, void* ws,
                      size_t need, int64_t M, int64_t D, int64_t I, int64_t Dout, hipStream_t st) {
  if (fwd_is_skinny(M, I, Dout))
    return fwd_skinny(x, W1, W_down, preact, y, ws, (float*)((char*)ws + align256((size_t)(M * I * 2))), M, D, I,
                      Dout, st);
  SW_TRY(step_gemm1(x, W1, preact, ws, M, D, I, st));
  const size_t h_bytes = align256((size_t)(M * I * 2));
  // the split tail's scratch lies inside the checked [ws, ws + need)
  const Scratch sc{(float*)((char*)ws + h_bytes), need - h_bytes};
  return step_down(ws, W_down, y, M, I, Dout, st, sc);
}

// shapes, null pointers and alignment of the forward's tensors
static int fwd_check(const void* x, const void* W1, const void* W_down, const void* preact, const void* y, int64_t M,
                     int64_t D, int64_t I, int64_t Dout) {
  SW_TRY(check_dims(M, D, I, Dout));
  if (missing(x, M * D) || !W1 || !W_down || missing(preact, M * I) || missing(y, M * Dout))
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned16(preact) || !aligned16(y))
    return SWIGLU_ERR_ALIGN;
  return SWIGLU_OK;
}

int swiglu_mlp_fwd(const void* x, const void* W1, const void* W_down, void* preact, void* y, void* ws,
                   size_t ws_bytes, int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(fwd_check(x, W1, W_down, preact, y, M, D, I, Dout));
  if (ws && !aligned16(ws)) return SWIGLU_ERR_ALIGN;
  const size_t need = swiglu_mlp_fwd_workspace(M, D, I, Dout);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2)};
  const Range outs[] = {rng(preact, M * 2 * I * 2), rng(y, M * Dout * 2), rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 3, outs, 3));
  return fwd_launch(x, W1, W_down, preact, y, ws, need, M, D, I, Dout, as_stream(stream));
}

size_t swiglu_mlp_fwd_noalloc_limit(void) { return kStaticWsBytes; }

int swiglu_mlp_fwd_noalloc(const void* x, const void* W1, const void* W_down, void* preact, void* y, int64_t M,
                           int64_t D, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(fwd_check(x, W1, W_down, preact, y, M, D, I, Dout));
  const size_t need = swiglu_mlp_fwd_workspace(M, D, I, Dout);
  if (need > kStaticWsBytes) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2)};
  const Range outs[] = {rng(preact, M * 2 * I * 2), rng(y, M * Dout * 2)};
  SW_TRY(check_alias(ins, 3, outs, 2));
  void* ws = nullptr;
  SW_TRY(static_workspace(&ws));
  return fwd_launch(x, W1, W_down, preact, y, ws, need, M, D, I, Dout, as_stream(stream));
}

static int bwd_common(bool fused, const void* x, const void* W1, const void* W_down, const void* preact,
                      const void* dy, void* dx, void* dW1, void* dW_down, void* ws, size_t ws_bytes, int64_t M,
                      int64_t D, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  if (missing(x, M * D) || !W1 || !W_down || missing(preact, M * I) || missing(dy, M * Dout) ||
      missing(dx, M * D) || !dW1 || !dW_down)
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned16(preact) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(dW1) || !aligned16(dW_down) || (ws && !aligned16(ws)))
    return SWIGLU_ERR_ALIGN;
  const size_t need = fused ? swiglu_mlp_bwd_workspace(M, D, I, Dout) : swiglu_mlp_bwd_unfused_workspace(M, D, I, Dout);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2),
                       rng(preact, M * 2 * I * 2), rng(dy, M * Dout * 2)};
  const Range outs[] = {rng(dx, M * D * 2), rng(dW1, D * 2 * I * 2), rng(dW_down, I * Dout * 2),
                        rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 5, outs, 4));
  hipStream_t st = as_stream(stream);
  char* w = (char*)ws;
  void* gp = w;
  void* h = w + align256((size_t)(M * 2 * I * 2));
  size_t used = align256((size_t)(M * 2 * I * 2)) + align256((size_t)(M * I * 2));
  if (fused) {
    SW_TRY(step_dgrad_fused(dy, W_down, preact, gp, h, M, I, Dout, st));
  } else {
    void* dout = (char*)h + align256((size_t)(M * I * 2));
    used += align256((size_t)(M * I * 2));
    SW_TRY(step_dgrad_plain(dy, W_down, dout, M, I, Dout, st));
    SW_TRY(step_elementwise(preact, dout, gp, h, M, I, st));
  }
  const Scratch sc{(float*)(w + used), need - used};
  SW_TRY(step_dw_down(h, dy, dW_down, M, I, Dout, st, sc));
  SW_TRY(step_dx(gp, W1, dx, M, D, I, st, sc));
  return step_dw1(x, gp, dW1, M, D, I, st, sc);
}

int swiglu_mlp_bwd(const void* x, const void* W1, const void* W_down, const void* preact, const void* dy, void* dx,
                   void* dW1, void* dW_down, void* ws, size_t ws_bytes, int64_t M, int64_t D, int64_t I,
                   int64_t Dout, void* stream) {
  return bwd_common(true, x, W1, W_down, preact, dy, dx, dW1, dW_down, ws, ws_bytes, M, D, I, Dout, stream);
}

int swiglu_mlp_bwd_unfused(const void* x, const void* W1, const void* W_down, const void* preact, const void* dy,
                           void* dx, void* dW1, void* dW_down, void* ws, size_t ws_bytes, int64_t M, int64_t D,
                           int64_t I, int64_t Dout, void* stream) {
  return bwd_common(false, x, W1, W_down, preact, dy, dx, dW1, dW_down, ws, ws_bytes, M, D, I, Dout, stream);
}

// --- residual block Y = X + MLP(X) (Lesson 24, section 24) ------------------

int swiglu_mlp_fwd_residual(const void* x, const void* W1, const void* W_down, void* preact, void* y, void* ws,
                            size_t ws_bytes, int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  if (Dout != D) return SWIGLU_ERR_SHAPE;
  if (missing(x, M * D) || !W1 || !W_down || missing(preact, M * I) || missing(y, M * Dout))
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned16(preact) || !aligned16(y) ||
      (ws && !aligned16(ws)))
    return SWIGLU_ERR_ALIGN;
  const size_t need = swiglu_mlp_fwd_workspace(M, D, I, Dout);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2)};
  const Range outs[] = {rng(preact, M * 2 * I * 2), rng(y, M * Dout * 2), rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 3, outs, 3));
  hipStream_t st = as_stream(stream);
  if (fwd_is_skinny(M, I, Dout))
    return fwd_skinny(x, W1, W_down, preact, y, ws, (float*)((char*)ws + align256((size_t)(M * I * 2))), M, D, I,
                      Dout, st, x);
  SW_TRY(step_gemm1(x, W1, preact, ws, M, D, I, st));
  return step_down_residual(ws, W_down, x, y, M, I, D, st);
}

int swiglu_mlp_bwd_residual(const void* x, const void* W1, const void* W_down, const void* preact, const void* dy,
                            void* dx, void* dW1, void* dW_down, void* ws, size_t ws_bytes, int64_t M, int64_t D,
                            int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  if (Dout != D) return SWIGLU_ERR_SHAPE;
  if (missing(x, M * D) || !W1 || !W_down || missing(preact, M * I) || missing(dy, M * Dout) ||
      missing(dx, M * D) || !dW1 || !dW_down)
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned16(preact) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(dW1) || !aligned16(dW_down) || (ws && !aligned16(ws)))
    return SWIGLU_ERR_ALIGN;
  const size_t need = swiglu_mlp_bwd_workspace(M, D, I, Dout);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2),
                       rng(preact, M * 2 * I * 2), rng(dy, M * Dout * 2)};
  const Range outs[] = {rng(dx, M * D * 2), rng(dW1, D * 2 * I * 2), rng(dW_down, I * Dout * 2),
                        rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 5, outs, 4));
  hipStream_t st = as_stream(stream);
  char* w = (char*)ws;
  void* gp = w;
  void* h = w + align256((size_t)(M * 2 * I * 2));
  SW_TRY(step_dgrad_fused(dy, W_down, preact, gp, h, M, I, Dout, st));
  const size_t used = align256((size_t)(M * 2 * I * 2)) + align256((size_t)(M * I * 2));
  const Scratch sc{(float*)(w + used), need - used};
  SW_TRY(step_dw_down(h, dy, dW_down, M, I, Dout, st, sc));
  SW_TRY(step_dx_residual(gp, W1, dy, dx, M, D, I, st));
  return step_dw1(x, gp, dW1, M, D, I, st, sc);
}

int swiglu_fwd_down_residual(const void* h, const void* W_down, const void* x, void* y, int64_t M, int64_t I,
                             int64_t D, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(D));
  if (missing(h, M * I) || !W_down || missing(x, M * D) || missing(y, M * D)) return SWIGLU_ERR_NULL;
  if (!aligned16(h) || !aligned16(W_down) || !aligned16(x) || !aligned16(y)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(h, M * I * 2), rng(W_down, I * D * 2), rng(x, M * D * 2)};
  const Range outs[] = {rng(y, M * D * 2)};
  SW_TRY(check_alias(ins, 3, outs, 1));
  return step_down_residual(h, W_down, x, y, M, I, D, as_stream(stream));
}

int swiglu_bwd_dx_residual(const void* grad_preact, const void* W1, const void* dy, void* dx, int64_t M, int64_t D,
                           int64_t I, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(D));
  SW_TRY(check_inner(I));
  if (missing(grad_preact, M * I) || !W1 || missing(dy, M * D) || missing(dx, M * D)) return SWIGLU_ERR_NULL;
  if (!aligned16(grad_preact) || !aligned16(W1) || !aligned16(dy) || !aligned16(dx)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(grad_preact, M * 2 * I * 2), rng(W1, D * 2 * I * 2), rng(dy, M * D * 2)};
  const Range outs[] = {rng(dx, M * D * 2)};
  SW_TRY(check_alias(ins, 3, outs, 1));
  return step_dx_residual(grad_preact, W1, dy, dx, M, D, I, as_stream(stream));
}

// --- mixture-of-experts MLP blocks (Lesson 24, sections 41-43) -------------

size_t swiglu_moe_fwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E) {
  if (check_dims(M, D, I, Dout) != SWIGLU_OK || check_experts(E) != SWIGLU_OK) return 0;
  return (size_t)(M * I * 2);
}

size_t swiglu_moe_bwd_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E) {
  if (check_dims(M, D, I, Dout) != SWIGLU_OK || check_experts(E) != SWIGLU_OK) return 0;
  return align256((size_t)(M * 2 * I * 2)) + align256((size_t)(M * I * 2));
}

int swiglu_moe_fwd(const void* x, const void* W1, const void* W_down, const int32_t* group_offsets, void* preact,
                   void* y, void* ws, size_t ws_bytes, int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E,
                   void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  SW_TRY(check_experts(E));
  if (missing(x, M * D) || !W1 || !W_down || !group_offsets || missing(preact, M * I) || missing(y, M * Dout))
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned4(group_offsets) || !aligned16(preact) ||
      !aligned16(y) || (ws && !aligned16(ws)))
    return SWIGLU_ERR_ALIGN;
  const size_t need = swiglu_moe_fwd_workspace(M, D, I, Dout, E);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, E * D * 2 * I * 2), rng(W_down, E * I * Dout * 2),
                       rng(group_offsets, (E + 1) * 4)};
  const Range outs[] = {rng(preact, M * 2 * I * 2), rng(y, M * Dout * 2), rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 4, outs, 3));
  hipStream_t st = as_stream(stream);
  SW_TRY(moe_gemm1(x, W1, group_offsets, preact, ws, M, D, I, E, st));
  return moe_down(ws, W_down, group_offsets, y, M, I, Dout, E, st);
}

int swiglu_moe_bwd(const void* x, const void* W1, const void* W_down, const int32_t* group_offsets,
                   const void* preact, const void* dy, void* dx, void* dW1, void* dW_down, void* ws, size_t ws_bytes,
                   int64_t M, int64_t D, int64_t I, int64_t Dout, int64_t E, void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  SW_TRY(check_experts(E));
  if (missing(x, M * D) || !W1 || !W_down || !group_offsets || missing(preact, M * I) || missing(dy, M * Dout) ||
      missing(dx, M * D) || !dW1 || !dW_down)
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned4(group_offsets) || !aligned16(preact) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(dW1) || !aligned16(dW_down) || (ws && !aligned16(ws)))
    return SWIGLU_ERR_ALIGN;
  const size_t need = swiglu_moe_bwd_workspace(M, D, I, Dout, E);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, E * D * 2 * I * 2), rng(W_down, E * I * Dout * 2),
                       rng(group_offsets, (E + 1) * 4), rng(preact, M * 2 * I * 2), rng(dy, M * Dout * 2)};
  const Range outs[] = {rng(dx, M * D * 2), rng(dW1, E * D * 2 * I * 2), rng(dW_down, E * I * Dout * 2),
                        rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 6, outs, 4));
  hipStream_t st = as_stream(stream);
  char* w = (char*)ws;
  void* gp = w;
  void* h = w + align256((size_t)(M * 2 * I * 2));
  SW_TRY(moe_dgrad_fused(dy, W_down, group_offsets, preact, gp, h, M, I, Dout, E, st));
  SW_TRY(moe_dw_down(h, dy, group_offsets, dW_down, M, I, Dout, E, st));
  SW_TRY(moe_dx(gp, W1, group_offsets, dx, M, D, I, E, st));
  return moe_dw1(x, gp, group_offsets, dW1, M, D, I, E, st);
}

int swiglu_moe_bwd_dgrad_fused(const void* dy, const void* W_down, const int32_t* group_offsets, const void* preact,
                               void* grad_preact, void* h, int64_t M, int64_t I, int64_t Dout, int64_t E,
                               void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(Dout));
  SW_TRY(check_experts(E));
  if (missing(dy, M * Dout) || !W_down || !group_offsets || missing(preact, M * I) || missing(grad_preact, M * I) ||
      missing(h, M * I))
    return SWIGLU_ERR_NULL;
  if (!aligned16(dy) || !aligned16(W_down) || !aligned4(group_offsets) || !aligned16(preact) ||
      !aligned16(grad_preact) || !aligned16(h))
    return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(dy, M * Dout * 2), rng(W_down, E * I * Dout * 2), rng(group_offsets, (E + 1) * 4),
                       rng(preact, M * 2 * I * 2)};
  const Range outs[] = {rng(grad_preact, M * 2 * I * 2), rng(h, M * I * 2)};
  SW_TRY(check_alias(ins, 4, outs, 2));
  return moe_dgrad_fused(dy, W_down, group_offsets, preact, grad_preact, h, M, I, Dout, E, as_stream(stream));
}

// --- save-h fallback (the drop-h report's normal MLPBlock) ------------------

// grad_preact [M,2I] | split tail of dW_down, dx, dW1
size_t swiglu_mlp_bwd_saved_h_workspace(int64_t M, int64_t D, int64_t I, int64_t Dout) {
  if (check_dims(M, D, I, Dout) != SWIGLU_OK) return 0;
  return align256((size_t)(M * 2 * I * 2)) + bwd_split_bytes(M, D, I, Dout);
}

int swiglu_mlp_fwd_save_h(const void* x, const void* W1, const void* W_down, void* preact, void* h, void* y,
                          int64_t M, int64_t D, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  if (missing(x, M * D) || !W1 || !W_down || missing(preact, M * I) || missing(h, M * I) || missing(y, M * Dout))
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned16(preact) || !aligned16(h) || !aligned16(y))
    return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2)};
  const Range outs[] = {rng(preact, M * 2 * I * 2), rng(h, M * I * 2), rng(y, M * Dout * 2)};
  SW_TRY(check_alias(ins, 3, outs, 3));
  hipStream_t st = as_stream(stream);
  SW_TRY(step_gemm1(x, W1, preact, h, M, D, I, st));
  return step_down(h, W_down, y, M, I, Dout, st);
}

int swiglu_mlp_bwd_saved_h(const void* x, const void* W1, const void* W_down, const void* preact, const void* h,
                           const void* dy, void* dx, void* dW1, void* dW_down, void* ws, size_t ws_bytes, int64_t M,
                           int64_t D, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_dims(M, D, I, Dout));
  if (missing(x, M * D) || !W1 || !W_down || missing(preact, M * I) || missing(h, M * I) || missing(dy, M * Dout) ||
      missing(dx, M * D) || !dW1 || !dW_down)
    return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W_down) || !aligned16(preact) || !aligned16(h) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(dW1) || !aligned16(dW_down) || (ws && !aligned16(ws)))
    return SWIGLU_ERR_ALIGN;
  const size_t need = swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout);
  if (need > 0 && (!ws || ws_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  const Range ins[] = {rng(x, M * D * 2),          rng(W1, D * 2 * I * 2), rng(W_down, I * Dout * 2),
                       rng(preact, M * 2 * I * 2), rng(h, M * I * 2),      rng(dy, M * Dout * 2)};
  const Range outs[] = {rng(dx, M * D * 2), rng(dW1, D * 2 * I * 2), rng(dW_down, I * Dout * 2),
                        rng(ws, (int64_t)need)};
  SW_TRY(check_alias(ins, 6, outs, 4));
  hipStream_t st = as_stream(stream);
  SW_TRY(step_dgrad_fused_gp(dy, W_down, preact, ws, M, I, Dout, st));
  const size_t used = align256((size_t)(M * 2 * I * 2));
  const Scratch sc{(float*)((char*)ws + used), need - used};
  SW_TRY(step_dw_down(h, dy, dW_down, M, I, Dout, st, sc));
  SW_TRY(step_dx(ws, W1, dx, M, D, I, st, sc));
  return step_dw1(x, ws, dW1, M, D, I, st, sc);
}

int swiglu_bwd_dgrad_fused_gp(const void* dy, const void* W_down, const void* preact, void* grad_preact, int64_t M,
                              int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(Dout));
  if (missing(dy, M * Dout) || !W_down || missing(preact, M * I) || missing(grad_preact, M * I))
    return SWIGLU_ERR_NULL;
  if (!aligned16(dy) || !aligned16(W_down) || !aligned16(preact) || !aligned16(grad_preact)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(dy, M * Dout * 2), rng(W_down, I * Dout * 2), rng(preact, M * 2 * I * 2)};
  const Range outs[] = {rng(grad_preact, M * 2 * I * 2)};
  SW_TRY(check_alias(ins, 3, outs, 1));
  return step_dgrad_fused_gp(dy, W_down, preact, grad_preact, M, I, Dout, as_stream(stream));
}

int swiglu_fwd_gemm1(const void* x, const void* W1, void* preact, void* h, int64_t M, int64_t D, int64_t I,
                     void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(D));
  SW_TRY(check_inner(I));
  if (missing(x, M * D) || !W1 || missing(preact, M * I) || missing(h, M * I)) return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(preact) || !aligned16(h)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(x, M * D * 2), rng(W1, D * 2 * I * 2)};
  const Range outs[] = {rng(preact, M * 2 * I * 2), rng(h, M * I * 2)};
  SW_TRY(check_alias(ins, 2, outs, 2));
  return step_gemm1(x, W1, preact, h, M, D, I, as_stream(stream));
}

int swiglu_fwd_down(const void* h, const void* W_down, void* y, int64_t M, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(Dout));
  if (missing(h, M * I) || !W_down || missing(y, M * Dout)) return SWIGLU_ERR_NULL;
  if (!aligned16(h) || !aligned16(W_down) || !aligned16(y)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(h, M * I * 2), rng(W_down, I * Dout * 2)};
  const Range outs[] = {rng(y, M * Dout * 2)};
  SW_TRY(check_alias(ins, 2, outs, 1));
  return step_down(h, W_down, y, M, I, Dout, as_stream(stream));
}

int swiglu_bwd_dgrad_fused(const void* dy, const void* W_down, const void* preact, void* grad_preact, void* h,
                           int64_t M, int64_t I, int64_t Dout, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(Dout));
  if (missing(dy, M * Dout) || !W_down || missing(preact, M * I) || missing(grad_preact, M * I) || missing(h, M * I))
    return SWIGLU_ERR_NULL;
  if (!aligned16(dy) || !aligned16(W_down) || !aligned16(preact) || !aligned16(grad_preact) || !aligned16(h))
    return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(dy, M * Dout * 2), rng(W_down, I * Dout * 2), rng(preact, M * 2 * I * 2)};
  const Range outs[] = {rng(grad_preact, M * 2 * I * 2), rng(h, M * I * 2)};
  SW_TRY(check_alias(ins, 3, outs, 2));
  return step_dgrad_fused(dy, W_down, preact, grad_preact, h, M, I, Dout, as_stream(stream));
}

int swiglu_bwd_dgrad_plain(const void* dy, const void* W_down, void* dout, int64_t M, int64_t I, int64_t Dout,
                           void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(Dout));
  if (missing(dy, M * Dout) || !W_down || missing(dout, M * I)) return SWIGLU_ERR_NULL;
  if (!aligned16(dy) || !aligned16(W_down) || !aligned16(dout)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(dy, M * Dout * 2), rng(W_down, I * Dout * 2)};
  const Range outs[] = {rng(dout, M * I * 2)};
  SW_TRY(check_alias(ins, 2, outs, 1));
  return step_dgrad_plain(dy, W_down, dout, M, I, Dout, as_stream(stream));
}

int swiglu_bwd_elementwise(const void* preact, const void* dout, void* grad_preact, void* h, int64_t M, int64_t I,
                           void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  if (missing(preact, M * I) || missing(dout, M * I) || missing(grad_preact, M * I) || missing(h, M * I))
    return SWIGLU_ERR_NULL;
  if (!aligned16(preact) || !aligned16(dout) || !aligned16(grad_preact) || !aligned16(h)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(preact, M * 2 * I * 2), rng(dout, M * I * 2)};
  const Range outs[] = {rng(grad_preact, M * 2 * I * 2), rng(h, M * I * 2)};
  SW_TRY(check_alias(ins, 2, outs, 2));
  return step_elementwise(preact, dout, grad_preact, h, M, I, as_stream(stream));
}

int swiglu_bwd_dw_down(const void* h, const void* dy, void* dW_down, int64_t M, int64_t I, int64_t Dout,
                       void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(I));
  SW_TRY(check_inner(Dout));
  if (missing(h, M * I) || missing(dy, M * Dout) || !dW_down) return SWIGLU_ERR_NULL;
  if (!aligned16(h) || !aligned16(dy) || !aligned16(dW_down)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(h, M * I * 2), rng(dy, M * Dout * 2)};
  const Range outs[] = {rng(dW_down, I * Dout * 2)};
  SW_TRY(check_alias(ins, 2, outs, 1));
  return step_dw_down(h, dy, dW_down, M, I, Dout, as_stream(stream));
}

int swiglu_bwd_dx(const void* grad_preact, const void* W1, void* dx, int64_t M, int64_t D, int64_t I, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(D));
  SW_TRY(check_inner(I));
  if (missing(grad_preact, M * I) || !W1 || missing(dx, M * D)) return SWIGLU_ERR_NULL;
  if (!aligned16(grad_preact) || !aligned16(W1) || !aligned16(dx)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(grad_preact, M * 2 * I * 2), rng(W1, D * 2 * I * 2)};
  const Range outs[] = {rng(dx, M * D * 2)};
  SW_TRY(check_alias(ins, 2, outs, 1));
  return step_dx(grad_preact, W1, dx, M, D, I, as_stream(stream));
}

int swiglu_bwd_dw1(const void* x, const void* grad_preact, void* dW1, int64_t M, int64_t D, int64_t I, void* stream) {
  SW_TRY(check_tokens(M));
  SW_TRY(check_inner(D));
  SW_TRY(check_inner(I));
  if (missing(x, M * D) || missing(grad_preact, M * I) || !dW1) return SWIGLU_ERR_NULL;
  if (!aligned16(x) || !aligned16(grad_preact) || !aligned16(dW1)) return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(x, M * D * 2), rng(grad_preact, M * 2 * I * 2)};
  const Range outs[] = {rng(dW1, D * 2 * I * 2)};
  SW_TRY(check_alias(ins, 2, outs, 1));
  return step_dw1(x, grad_preact, dW1, M, D, I, as_stream(stream));
}

int swiglu_act_eval(const void* g, void* sigma, void* silu, void* dsilu, int64_t n, void* stream) {
  if (n < 0) return SWIGLU_ERR_SHAPE;
  if (missing(g, n) || missing(sigma, n) || missing(silu, n) || missing(dsilu, n)) return SWIGLU_ERR_NULL;
  if (((uintptr_t)g & 1u) || ((uintptr_t)sigma & 3u) || ((uintptr_t)silu & 3u) || ((uintptr_t)dsilu & 3u))
    return SWIGLU_ERR_ALIGN;
  const Range ins[] = {rng(g, n * 2)};
  const Range outs[] = {rng(sigma, n * 4), rng(silu, n * 4), rng(dsilu, n * 4)};
  SW_TRY(check_alias(ins, 1, outs, 3));
  if (n == 0) return SWIGLU_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(swg::swiglu_act_eval_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     (const uint16_t*)g, (float*)sigma, (float*)silu, (float*)dsilu, n);
  return launch_status();
}

}  // extern "C"
