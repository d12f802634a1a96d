// skinny.hpp -- GEMMs with at most 16 token rows (decode-shaped batches) on
// gfx950.
//
// With M <= 16 the forward GEMMs of the SwiGLU MLP (the merged gate/up GEMM
// and the down GEMM of the drop-h report's forward) are weight streams: every
// byte of W is used for only M multiply-adds, so the bound is HBM, not the
// matrix cores.  The tiled kernel would spend 8-16x the MFMA work on padding
// rows and launch too few workgroups to keep HBM busy.  Here:
//   * a workgroup owns 128 columns of W and one of S contiguous k-ranges
//     (split-K), so that there are about two workgroups per CU;
//   * W streams through an LDS ring of 64-row stages with direct-to-LDS loads
//     (no VGPR staging), three stages in flight; the matching 16 x 64 slice
//     of X rides in the same stage, so every wave issues the same loads and
//     the in-order vmcnt accounting stays uniform;
//   * one v_mfma_f32_16x16x32_bf16 covers all 16 rows; W fragments are read
//     with ds_read_b64_tr_b16 (W is [K, N] row-major: N contiguous);
//   * fp32 partial sums go to a workspace [S][16][N]; a second kernel adds
//     them in a fixed order (so results do not depend on timing) and applies
//     the epilogue: SwiGLU for GEMM-1, a bf16 store for the down GEMM.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.hpp"
#include "swiglu_math.hpp"

namespace swg {

constexpr int SK_BN = 128;                       // columns per workgroup
constexpr int SK_BK = 64;                        // k rows per stage
constexpr int SK_R = 4;                          // ring depth (stages)
constexpr int SK_W_BYTES = SK_BK * SK_BN * 2;    // 16 KB of W per stage
constexpr int SK_X_BYTES = 16 * SK_BK * 2;       // 2 KB of X per stage
constexpr int SK_STAGE = SK_W_BYTES + SK_X_BYTES;
constexpr int SK_LDS = SK_R * SK_STAGE;          // 72 KB: two workgroups per CU
constexpr int SK_LW = SK_W_BYTES / 1024 / 4;     // W blocks per wave per stage (4)

struct SkinnyArgs {
  const uint16_t* X;  // [M, K] row-major
  const uint16_t* W;  // [K, N] row-major
  float* partial;     // [S][16][N] fp32
  int64_t ldx, ldw;
  int M, N, K;
  int stages_per_split;
};

// s_waitcnt vmcnt(n) for a wave-uniform runtime n in [0, 3*(SK_LW+1)]
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1 * (SK_LW + 1): wait_vmcnt<1 * (SK_LW + 1)>(); break;
    case 2 * (SK_LW + 1): wait_vmcnt<2 * (SK_LW + 1)>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// LDS image of a stage's X slice: 16 rows of 64 k (8 chunks of 16 B); chunk
// c of row r sits at position c ^ (r % 8) so that the 16 rows one fragment
// read touches spread over the banks.
__device__ __forceinline__ int sk_x_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// grid: (N / 128, S).  Workgroup (nb, s) multiplies X[:, k-range s] by
// W[k-range s, nb*128 .. +128) and writes its partial sum to partial[s].
__global__ void __launch_bounds__(256) skinny_gemm_kernel(const SkinnyArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[SK_LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = blockIdx.x, s = blockIdx.y;
  const int nk_all = a.K / SK_BK;
  const int kt0 = s * a.stages_per_split;
  const int nk = min(a.stages_per_split, nk_all - kt0);  // stages of this split (>= 1 by the host's choice of S)

  auto w_lds = [&](int j) { return (SWG_LDS char*)smem + (j % SK_R) * SK_STAGE; };
  auto x_lds = [&](int j) { return (SWG_LDS char*)smem + (j % SK_R) * SK_STAGE + SK_W_BYTES; };

  // W stage j: rows (kt0 + j)*64 .. +64 of columns nb*128 .. +128, as the
  // GEMM core's MN-major tile (blocks wave + 4i, two swizzle classes).
  const uint32_t wb0 = dma_lane_base<SK_BN, false>(a.ldw, nb, 0, wave, lane);
  const uint32_t wb1 = dma_lane_base<SK_BN, false>(a.ldw, nb, 0, wave + 4, lane);
  // X stage j: rows 0..15 (rows >= M read as zeros), k (kt0 + j)*64 .. +64;
  // wave w fills 512 B of it with lanes 0..31: row 4w + lane/8, position lane%8
  const int xr = wave * 4 + (lane >> 3);
  const int xc = (lane & 7) ^ (xr & 7);
  const uint32_t xoff = (uint32_t)(xr * a.ldx * 2) + (uint32_t)(xc * 16);
  const i32x4 rx = make_rsrc(a.X, (int64_t)a.M * a.ldx * 2);

  auto issue = [&](int j) {
    const int64_t k0 = (int64_t)(kt0 + j) * SK_BK;
    const i32x4 rw = make_rsrc(a.W + k0 * a.ldw, ((int64_t)a.K - k0) * a.ldw * 2);
#pragma unroll
    for (int i = 0; i < SK_LW; ++i) {
      const int b = wave + 4 * i;
      dma16(rw, w_lds(j) + b * 1024, (i & 1) ? wb1 : wb0, dma_block_add<SK_BN, false>(a.ldw, b, 0));
    }
    // half a wave: lanes 32..63 are masked off and write nothing
    if (lane < 32) dma16(rx, x_lds(j) + wave * 512, xoff, (uint32_t)(k0 * 2));
  };
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  typedef float f32x4v __attribute__((ext_vector_type(4)));
  f32x4v acc[2] = {f32x4v{}, f32x4v{}};  // this wave's two 16-column tiles

  // prologue: stages 0 .. R-2
#pragma unroll
  for (int j = 0; j < SK_R - 1; ++j)
    if (j < nk) issue(j);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed: the ones issued after it may stay in flight
    const int ahead = min(nk - 1, kt + SK_R - 2) - kt;
    wait_vmcnt_upto(ahead * (SK_LW + 1));
    barrier();  // every wave's stage kt is visible; nobody reads stage kt-1 any more
    if (kt + SK_R - 1 < nk) issue(kt + SK_R - 1);
    const SWG_LDS char* wt = w_lds(kt);
    const SWG_LDS char* xt = x_lds(kt);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // A (X) fragment: row lane%16, k = kk*32 + 8*(lane/16) .. +7
      const int r = lane & 15, oct = kk * 4 + (lane >> 4);
      const bf16x8 xa = *(const SWG_LDS bf16x8*)(xt + sk_x_off(r, oct));
      // B (W) fragments: column c0 + lane%16, the same 8 k.  Within each
      // group of 16 lanes, lane 4e+q reads k-row kbase+e, columns c0+4q..+3,
      // and the transposing read hands lane j column c0 + j, k-rows kbase..+3.
      const int g = lane >> 4, j = lane & 15, e = j >> 2, q = j & 3;
      const int kbase = kk * 32 + g * 8 + e;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int col = (wave * 2 + t) * 16 + q * 4;
        const int o1 = lds_off_mn<SK_BN>(kbase, col >> 3) + (col & 7) * 2;
        const int o2 = lds_off_mn<SK_BN>(kbase + 4, col >> 3) + (col & 7) * 2;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(wt + o1));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(wt + o2));
        const bf16x8 wb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, acc[t], 0, 0, 0);
      }
    }
  }
  // D of 16x16x32: lane l holds column l%16, rows 4*(l/16) .. +3
  float* out = a.partial + (int64_t)s * 16 * a.N + (int64_t)nb * SK_BN;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int col = (wave * 2 + t) * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(int64_t)(4 * (lane >> 4) + i) * a.N + col] = acc[t][i];
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
  for (int s = 0; s < S; ++s) {
    const float* p = partial + ((int64_t)s * 16 + m) * N;
    const f32x4* pl = (const f32x4*)(p + i0);
    const f32x4* pg = (const f32x4*)(p + I + i0);
    const f32x4 l0 = pl[0], l1 = pl[1], g0 = pg[0], g1 = pg[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      left[e] += l0[e];
      left[4 + e] += l1[e];
      gate[e] += g0[e];
      gate[4 + e] += g1[e];
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

// y[m, n] = rn(sum_s partial[s][m][n]).  One thread per (m, 8 columns).
__global__ void __launch_bounds__(256) skinny_store_reduce_kernel(const float* __restrict__ partial, int S, int M,
                                                                  int64_t N, uint16_t* __restrict__ y) {
  const int64_t cpr = N / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * cpr) return;
  const int m = (int)(t / cpr);
  const int64_t n0 = (t % cpr) * 8;
  f32x8 v = {};
  for (int s = 0; s < S; ++s) {
    const f32x4* p = (const f32x4*)(partial + ((int64_t)s * 16 + m) * N + n0);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] += a[e];
      v[4 + e] += b[e];
    }
  }
  *(u32x4*)(y + (int64_t)m * N + n0) = pack8(v);
}

}  // namespace swg
