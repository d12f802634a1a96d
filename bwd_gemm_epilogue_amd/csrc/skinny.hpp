// skinny.hpp -- GEMMs with at most 16 token rows (decode-shaped batches) on
// gfx950.
//
// With M <= 16 the forward GEMMs of the SwiGLU MLP (the merged gate/up GEMM
// and the down GEMM of the drop-h report's forward) are weight streams: every
// byte of W is used for only M multiply-adds, so the bound is HBM, not the
// matrix cores ("Lesson 24", sections 29-30: at decode the MLP GEMMs turn
// into GEMV-like, weight-bandwidth-bound products).  The tiled kernel would spend 8-16x the MFMA work on padding
// rows and launch too few workgroups to keep HBM busy.  Here:
//   * a workgroup owns 128 columns of W and one of S contiguous k-ranges
//     (split-K), about 512 workgroups in all;
//   * W streams in 64-row stages through registers into a double-buffered
//     LDS tile (plain vector loads stream HBM faster than direct-to-LDS
//     loads); X fragments come straight from memory;
//   * one v_mfma_f32_16x16x32_bf16 covers all 16 rows; W fragments are read
//     with ds_read_b64_tr_b16 (W is [K, N] row-major: N contiguous);
//   * fp32 partial sums go to a workspace [S][16][N] (rows >= M hold
//     don't-care values); a second kernel adds
//     them in a fixed order (so results do not depend on timing) and applies
//     the epilogue: SwiGLU for GEMM-1, a bf16 store for the down GEMM.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.hpp"
#include "swiglu_math.hpp"

namespace swg {

constexpr int SK_BN = 128;                       // columns per workgroup (the smaller width)
constexpr int SK_BK = 64;                        // k rows per stage

struct SkinnyArgs {
  const uint16_t* X;  // [M, K] row-major
  const uint16_t* W;  // [K, N] row-major
  float* partial;     // [S][16][N] fp32
  int64_t ldx, ldw;
  int M, N, K;
  int stages_per_split;
};

// grid: (N / 128, S).  Workgroup (nb, s) multiplies X[:, k-range s] by
// W[k-range s, nb*128 .. +128) and writes its partial sum to partial[s].
//
// W is streamed with plain 16-byte vector loads into registers, one stage
// (64 rows) ahead, and written to a double-buffered LDS tile in the GEMM
// core's MN-major layout, from which the transposing LDS read builds the
// k-contiguous B fragments.  (For a pure stream the vector-load path reaches
// about 7.3 TB/s on MI355X against about 6.2 TB/s for direct-to-LDS loads.)
// The X fragments are already k-contiguous and come straight from memory.
// BN (128 or 256) columns per workgroup: a wider block reads longer runs of
// each W row (256 or 512 bytes), which HBM serves faster, at the cost of
// fewer, longer streams.
template <int BN>
__global__ void __launch_bounds__(256) skinny_gemm_kernel(const SkinnyArgs a) {
  constexpr int W_BYTES = SK_BK * BN * 2;   // one stage of W
  constexpr int CPR = BN / 8;               // 16-byte chunks per W row
  constexpr int RPP = 256 / CPR;            // W rows per load pass of the workgroup
  constexpr int PASSES = SK_BK / RPP;       // loads per thread per stage
  constexpr int NT = BN / 64;               // 16-column MFMA tiles per wave
  __shared__ __attribute__((aligned(1024))) char smem[2 * W_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = blockIdx.x, s = blockIdx.y;
  const int nk_all = a.K / SK_BK;
  const int kt0 = s * a.stages_per_split;
  const int nk = min(a.stages_per_split, nk_all - kt0);  // >= 1 by the host's choice of S

  // W: thread t moves chunk c = t%CPR (8 columns) of k-rows t/CPR + RPP*i;
  // one wave instruction covers BN*2-byte segments of 64/CPR rows
  const int wc = tid % CPR, wr = tid / CPR;
  const uint16_t* wsrc = a.W + ((int64_t)kt0 * SK_BK + wr) * a.ldw + (int64_t)nb * BN + wc * 8;
  int woff[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) woff[i] = lds_off_mn<BN>(wr + RPP * i, wc);
  // X: lane l holds row l%16, k-octet (kk*4 + l/16) of the stage.  Rows
  // >= M repeat row M-1: they only feed partial-sum rows >= M, which the
  // reduction never reads.
  const int xr = lane & 15, xo = lane >> 4;
  const uint16_t* xsrc = a.X + (int64_t)min(xr, a.M - 1) * a.ldx + (int64_t)kt0 * SK_BK + xo * 8;

  auto load_w = [&](int j, u32x4 (&r)[PASSES]) {
    const uint16_t* p = wsrc + (int64_t)j * SK_BK * a.ldw;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) r[i] = __builtin_nontemporal_load((const u32x4*)(p + (int64_t)RPP * i * a.ldw));
  };
  auto load_x = [&](int j, bf16x8 (&r)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      r[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xsrc + j * SK_BK + kk * 32));
    }
  };

  typedef float f32x4v __attribute__((ext_vector_type(4)));
  f32x4v acc[NT];  // this wave's 16-column tiles
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = f32x4v{};
  u32x4 wreg[2][PASSES];
  bf16x8 xreg[2][2];

  auto stage = [&](int kt, int b, bool refill) {
    // stage kt's W registers -> LDS buffer b; refill them with stage kt+2.
    // Stage kt+2's X is loaded after this stage's MFMAs have used stage kt's,
    // so no register holding a pending load is ever copied.
    SWG_LDS char* t = (SWG_LDS char*)smem + b * W_BYTES;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) *(SWG_LDS u32x4*)(t + woff[i]) = wreg[b][i];
    if (refill) load_w(kt + 2, wreg[b]);
    // every wave's part of stage kt is in LDS; buffer b's previous readers
    // (stage kt-2) finished before the barrier of stage kt-1
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // B (W) fragments: column c0 + lane%16, k = kk*32 + 8*(lane/16) .. +7.
      // Within each group of 16 lanes, lane 4e+q reads k-row kbase+e,
      // columns c0+4q..+3, and the transposing read hands lane j column
      // c0 + j, k-rows kbase..+3.
      const int g = lane >> 4, j = lane & 15, e = j >> 2, q = j & 3;
      const int kbase = kk * 32 + g * 8 + e;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int col = (wave * NT + u) * 16 + q * 4;
        const int o1 = lds_off_mn<BN>(kbase, col >> 3) + (col & 7) * 2;
        const int o2 = lds_off_mn<BN>(kbase + 4, col >> 3) + (col & 7) * 2;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(t + o1));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(t + o2));
        const bf16x8 wb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xreg[b][kk], wb, acc[u], 0, 0, 0);
      }
    }
    if (refill) load_x(kt + 2, xreg[b]);
  };

  // Both prologue stages are loaded unconditionally and in stage order
  // (stage 0 twice when the split has a single stage), so that the loop is
  // entered with the same loads pending as on every later trip.  Under an
  // `if (nk > 1)` the compiler had issued stage 1 first, and the wait-count
  // pass, which merges the entry and back-edge states, then made every trip
  // wait for the stage loaded one stage earlier instead of two.
  load_w(0, wreg[0]);
  load_x(0, xreg[0]);
  load_w(nk > 1 ? 1 : 0, wreg[1]);
  load_x(nk > 1 ? 1 : 0, xreg[1]);
  // Steady state with unconditional refills, so that the compiler's
  // wait-count tracking sees the same loads pending on every trip (stage
  // kt+1's) and waits only for stage kt's; then the last one to three stages.
  int kt = 0;
  for (; kt + 3 < nk; kt += 2) {
    stage(kt, 0, true);
    stage(kt + 1, 1, true);
  }
  const int rest = nk - kt;  // 1..3
  if (rest >= 1) stage(kt, 0, rest >= 3);
  if (rest >= 2) stage(kt + 1, 1, false);
  if (rest >= 3) stage(kt + 2, 0, false);
  // D of 16x16x32: lane l holds column l%16, rows 4*(l/16) .. +3
  float* out = a.partial + (int64_t)s * 16 * a.N + (int64_t)nb * BN;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int col = (wave * NT + u) * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(int64_t)(4 * (lane >> 4) + i) * a.N + col] = acc[u][i];
  }
}

// preact[m, c] = rn(sum_s partial[s][m][c]) for both halves, and
// h[m, c] = rn(left * silu(gate)) from the rounded halves (as the tiled
// GEMM-1 epilogue).  One thread per (m, 8 channels).
__global__ void __launch_bounds__(256) skinny_swiglu_reduce_kernel(const float* __restrict__ partial, int S, int M,
                                                                   int64_t I, uint16_t* __restrict__ preact,
                                                                   uint16_t* __restrict__ h) {
  const int64_t cpr = I / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * cpr) return;
  const int m = (int)(t / cpr);
  const int64_t i0 = (t % cpr) * 8;
  const int64_t N = 2 * I;
  f32x8 left = {}, gate = {};
  // blocks of 8 splits: all loads first (clamped to a real split), then the
  // adds in split order, keeping only splits < S
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, S - 1);
      const float* p = partial + ((int64_t)s * 16 + m) * N;
      v[u][0] = ((const f32x4*)(p + i0))[0];
      v[u][1] = ((const f32x4*)(p + i0))[1];
      v[u][2] = ((const f32x4*)(p + I + i0))[0];
      v[u][3] = ((const f32x4*)(p + I + i0))[1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < S) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          left[e] += v[u][0][e];
          left[4 + e] += v[u][1][e];
          gate[e] += v[u][2][e];
          gate[4 + e] += v[u][3][e];
        }
      }
    }
  }
  const u32x4 lp = pack8(left), gp = pack8(gate);
  const f32x8 lr = unpack8(lp), gr = unpack8(gp);
  f32x8 hv;
#pragma unroll
  for (int e = 0; e < 8; ++e) hv[e] = swiglu_h(lr[e], gr[e]);
  *(u32x4*)(preact + (int64_t)m * N + i0) = lp;
  *(u32x4*)(preact + (int64_t)m * N + I + i0) = gp;
  *(u32x4*)(h + (int64_t)m * I + i0) = pack8(hv);
}

// y[m, n] = rn(sum_s partial[s][m][n] (+ res[m, n] when res is given: the
// residual-add epilogue, added in fp32 before the one rounding)).  One thread
// per (m, 8 columns).
__global__ void __launch_bounds__(256) skinny_store_reduce_kernel(const float* __restrict__ partial, int S, int M,
                                                                  int64_t N, uint16_t* __restrict__ y,
                                                                  const uint16_t* __restrict__ res) {
  const int64_t cpr = N / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * cpr) return;
  const int m = (int)(t / cpr);
  const int64_t n0 = (t % cpr) * 8;
  f32x8 v = {};
  // blocks of 8 splits: all loads first (clamped to a real split), then the
  // adds in split order, keeping only splits < S
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 w[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, S - 1);
      const f32x4* p = (const f32x4*)(partial + ((int64_t)s * 16 + m) * N + n0);
      w[u][0] = p[0];
      w[u][1] = p[1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < S) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] += w[u][0][e];
          v[4 + e] += w[u][1][e];
        }
      }
    }
  }
  if (res != nullptr) {
    const f32x8 r = unpack8(*(const u32x4*)(res + (int64_t)m * N + n0));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += r[e];
  }
  *(u32x4*)(y + (int64_t)m * N + n0) = pack8(v);
}

}  // namespace swg
