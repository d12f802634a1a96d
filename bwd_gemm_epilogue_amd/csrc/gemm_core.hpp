// gemm_core.hpp -- bf16 MFMA GEMM core for gfx950 (CDNA4) with pluggable
// epilogues.
//
// C[M,N] = A[M,K] . B[K,N], bf16 operands, fp32 accumulation.  Every GEMM of
// the SwiGLU MLP step (the forward merged gate/up GEMM and the down GEMM; the
// backward dout, dW_down, dx and dW1 GEMMs -- the note "SwiGLU MLP forward
// principle, backward chain and optimisation", sections 1-3) is one
// instantiation of this kernel with a layout pair and an epilogue.
//
// Operand layouts (row-major storage, "K-major" = the contraction index is
// the contiguous one):
//   A_KMAJ:  A(m,k) = A[m*lda + k]      else  A(m,k) = A[k*lda + m]
//   B_KMAJ:  B(k,n) = B[n*ldb + k]      else  B(k,n) = B[k*ldb + n]
//
// Design (one workgroup per output tile, BK = 64, two LDS stages):
//   * global -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging); the
//     buffer descriptor's range check returns zeros past the end of a
//     tensor, which masks the token tail of every GEMM;
//   * K-major tiles are stored [rows][64] in LDS and MN-major tiles [64][rows],
//     both with an XOR swizzle of 16-byte chunks; K-major fragments are read
//     with ds_read_b128, MN-major ones with two ds_read_b64_tr_b16 (the gfx950
//     transposing LDS read), so both layouts feed the same MFMA;
//   * v_mfma_f32_32x32x16_bf16 with the operands swapped (the B fragment in
//     the instruction's A slot), so each lane's accumulator holds runs of
//     four consecutive output columns of one output row;
//   * the epilogue stages the fp32 accumulators through LDS one 32-row slab
//     per wave at a time, so that every global access of the epilogue is a
//     coalesced 16-byte-per-lane access of a row.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swiglu_math.hpp"

#define SWG_LDS __attribute__((address_space(3)))

namespace swg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // one wave's output tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int SLAB_ROWS = 32 * WM;           // epilogue slab: 32 rows per wave row
  static constexpr int SLAB_LD = BN + 4;              // fp32 row pitch (+16 B breaks bank aliasing)
  static constexpr int SLAB_BYTES = SLAB_ROWS * SLAB_LD * 4;
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > SLAB_BYTES) ? 2 * STAGE_BYTES : SLAB_BYTES;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert((BM / 8) % WAVES == 0 && (BN / 8) % WAVES == 0, "1 KB load blocks must split over waves");
  static_assert(BM >= 64 && BN >= 64, "MN-major LDS rows need at least 8 chunks");
};

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int64_t lda, ldb;  // leading dimensions in elements
  int M, N, K;       // GEMM dimensions
  int tiles_m, tiles_n;
  // pair_off > 0: tile tn's B columns are [tn*BN/2, tn*BN/2 + BN/2) followed by
  // [pair_off + tn*BN/2, ...): the left and gate halves of W1 side by side.
  int pair_off;
};

// ---------------------------------------------------------------------------
// LDS layouts
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_k(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz_mn(int k) { return (k & 3) << 1; }

// K-major tile [rows][64 bf16]: byte offset of 16-byte chunk c of row r
__device__ __forceinline__ int lds_off_k(int r, int c) { return r * 128 + ((c ^ swz_k(r)) << 4); }

// MN-major tile [64][ROWS bf16]: byte offset of 16-byte chunk c of k-row k
template <int ROWS>
__device__ __forceinline__ int lds_off_mn(int k, int c) {
  return k * (ROWS * 2) + ((c ^ swz_mn(k)) << 4);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // dword 3 = 0x00020000: raw (untyped) buffer, 32-bit data format field as
  // gfx9 expects; the range check then zero-fills any 16 B load at or past
  // `bytes` (all offsets and ranges here are multiples of 16 B).
  int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0ll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Element column of local MN index c (a multiple of 8) of a tile whose MN
// origin is `origin`; paired tiles split into two halves pair_off apart.
template <int ROWS>
__device__ __forceinline__ int mn_col(int c, int tile, int pair_off) {
  if (pair_off > 0) {
    const int half = ROWS / 2;
    return (c < half) ? tile * half + c : pair_off + tile * half + (c - half);
  }
  return tile * ROWS + c;
}

// Issue the direct-to-LDS loads of one operand tile (ROWS x 64).  One wave
// instruction fills 1 KB of LDS, 16 B per lane in lane order; each lane picks
// the global chunk that belongs at its LDS slot under the swizzle.
//   K-major: rsrc is based at row `tile*ROWS` of the operand; k0 is the
//            first k of this stage.
//   MN-major: rsrc is based at k-row k0 of the operand.
template <int ROWS, bool KMAJ, int WAVES>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rsrc, SWG_LDS char* dst, int64_t ld,
                                          int k0, int tile, int pair_off, int wave, int lane) {
  constexpr int BLOCKS = ROWS / 8;  // ROWS * 64 * 2 B / 1 KB
#pragma unroll
  for (int i = 0; i < BLOCKS / WAVES; ++i) {
    const int b = wave + i * WAVES;
    uint32_t voff;
    if constexpr (KMAJ) {
      const int r = b * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz_k(r);
      voff = (uint32_t)((int64_t)r * ld * 2) + (uint32_t)(k0 + c * 8) * 2u;
    } else {
      constexpr int CPR = ROWS / 8;     // 16 B chunks per k-row
      constexpr int KROWS = 64 / CPR;   // k-rows per 1 KB block
      const int k = b * KROWS + lane / CPR;
      const int c = (lane % CPR) ^ swz_mn(k);
      const int col = mn_col<ROWS>(c * 8, tile, pair_off);
      voff = (uint32_t)((int64_t)k * ld * 2) + (uint32_t)col * 2u;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SWG_LDS void*)(dst + b * 1024), 16, voff, 0, 0, 0);
  }
}

// 32x16 MFMA operand fragment: lane l gets row r0 + l%32 and the 8 k values
// kk*16 + 8*(l/32) + 0..7.
__device__ __forceinline__ bf16x8 frag_k(const SWG_LDS char* t, int r0, int kk, int lane) {
  const int r = r0 + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *(const SWG_LDS bf16x8*)(t + lds_off_k(r, c));
}

// Same fragment from an MN-major tile.  ds_read_b64_tr_b16 transposes within
// each group of 16 lanes: lane j receives, in slot e, element j%4 of the 8 B
// read by lane 4e + j/4.  So lane 4e+q of group g reads k-row (base + e),
// columns col0 + 4q .. +3, and lane j ends up with column col0 + j, k-rows
// base .. base+3.  Two reads give the 8 k values.
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_mn(const SWG_LDS char* t, int r0, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int e = j >> 2, q = j & 3;
  const int k = kk * 16 + (g >> 1) * 8 + e;
  const int col = r0 + (g & 1) * 16 + q * 4;
  const int o1 = lds_off_mn<ROWS>(k, col >> 3) + (col & 7) * 2;
  const int o2 = lds_off_mn<ROWS>(k + 4, col >> 3) + (col & 7) * 2;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(t + o1));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(t + o2));
  i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <class T>
struct Frags {
  bf16x8 a[T::FM], b[T::FN];
};

template <class T, bool A_K, bool B_K>
__device__ __forceinline__ void load_frags(const SWG_LDS char* As, const SWG_LDS char* Bs, Frags<T>& f, int kk,
                                           int wm, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
    f.a[i] = A_K ? frag_k(As, wm * T::WTM + i * 32, kk, lane) : frag_mn<T::BM>(As, wm * T::WTM + i * 32, kk, lane);
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
    f.b[j] = B_K ? frag_k(Bs, wn * T::WTN + j * 32, kk, lane) : frag_mn<T::BN>(Bs, wn * T::WTN + j * 32, kk, lane);
}

// LDS read instructions per fragment set (transposing reads take two)
template <class T, bool A_K, bool B_K>
constexpr int frag_reads() {
  return T::FM * (A_K ? 1 : 2) + T::FN * (B_K ? 1 : 2);
}

// One LDS stage (BK = 64): four k16 steps.  Fragments of step kk+1 are read
// while the MFMAs of step kk run; sched_group_barrier pins the interleave
// (mask 0x008 = MFMA, 0x100 = LDS read) so each LDS read is covered by MFMAs.
template <class T, bool A_K, bool B_K>
__device__ __forceinline__ void compute_stage(const SWG_LDS char* As, const SWG_LDS char* Bs,
                                              f32x16 (&acc)[T::FM][T::FN], int wm, int wn, int lane) {
  constexpr int KSTEPS = T::BK / 16;
  constexpr int MFMAS = T::FM * T::FN;
  constexpr int READS = frag_reads<T, A_K, B_K>();
  Frags<T> f[2];
  load_frags<T, A_K, B_K>(As, Bs, f[0], 0, wm, wn, lane);
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    Frags<T>& cur = f[kk & 1];
    if (kk + 1 < KSTEPS) load_frags<T, A_K, B_K>(As, Bs, f[(kk + 1) & 1], kk + 1, wm, wn, lane);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
    if (kk + 1 < KSTEPS) {
      // spread the next step's READS LDS reads over this step's MFMAS MFMAs
      constexpr int PER = (MFMAS + READS - 1) / READS;
#pragma unroll
      for (int r = 0; r < READS; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
      }
    }
    // nothing crosses a k16 step boundary: the reads issued above stay in
    // flight under this step's MFMAs and are waited for by the next step
    __builtin_amdgcn_sched_barrier(0);
  }
}

// blockIdx -> (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs, so each XCD is first given a contiguous run of tile ids (its own
// L2 then sees neighbouring tiles), and tile ids are walked in groups of
// GROUP_M tile rows so that concurrently running tiles share A and B panels.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int per = total / 8, rem = total % 8;
  const int xcd = pid % 8, local = pid / 8;
  const int id = xcd * per + (xcd < rem ? xcd : rem) + local;
  constexpr int GROUP_M = 8;
  const int group = id / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int in_group = id - group * GROUP_M * tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Epilogue context handed to the epilogue functors for one slab.
template <class T>
struct SlabCtx {
  const SWG_LDS float* slab;  // [SLAB_ROWS][SLAB_LD] fp32
  int tm, tn, s;              // tile coordinates and slab index
  int M, N;
  // global row of slab row sr (rows past M are not stored)
  __device__ __forceinline__ int row(int sr) const {
    return tm * T::BM + (sr >> 5) * T::WTM + s * 32 + (sr & 31);
  }
  __device__ __forceinline__ f32x8 read8(int sr, int c) const {
    const SWG_LDS f32x4* p = (const SWG_LDS f32x4*)(slab + sr * T::SLAB_LD + c);
    f32x4 lo = p[0], hi = p[1];
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

template <class T, bool A_K, bool B_K, class Epi>
__global__ void __launch_bounds__(T::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) gemm_kernel(const GemmArgs g, const typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x16{};

  // K-major operands: descriptors based at the tile's first row, fixed for
  // the whole K loop.  MN-major: rebased at every stage's first k-row.
  const int nk = (g.K + T::BK - 1) / T::BK;
  __amdgpu_buffer_rsrc_t ra =
      A_K ? make_rsrc(g.A + (int64_t)tm * T::BM * g.lda, ((int64_t)g.M - (int64_t)tm * T::BM) * g.lda * 2)
          : make_rsrc(g.A, 0);
  __amdgpu_buffer_rsrc_t rb =
      B_K ? make_rsrc(g.B + (int64_t)tn * T::BN * g.ldb, ((int64_t)g.N - (int64_t)tn * T::BN) * g.ldb * 2)
          : make_rsrc(g.B, 0);

  auto issue = [&](int kt) {
    SWG_LDS char* st = (SWG_LDS char*)smem + (kt & 1) * T::STAGE_BYTES;
    const int k0 = kt * T::BK;
    if constexpr (!A_K) ra = make_rsrc(g.A + (int64_t)k0 * g.lda, ((int64_t)g.K - k0) * g.lda * 2);
    if constexpr (!B_K) rb = make_rsrc(g.B + (int64_t)k0 * g.ldb, ((int64_t)g.K - k0) * g.ldb * 2);
    load_tile<T::BM, A_K, T::WAVES>(ra, st, g.lda, A_K ? k0 : 0, tm, 0, wave, lane);
    load_tile<T::BN, B_K, T::WAVES>(rb, st + T::A_BYTES, g.ldb, B_K ? k0 : 0, tn, g.pair_off, wave, lane);
  };

  if (nk > 0) issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    // this stage's loads (issued one iteration ago) have landed for this
    // wave; the barrier makes every wave's loads visible and guarantees the
    // other stage is no longer being read
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1);
    const SWG_LDS char* st = (const SWG_LDS char*)smem + (kt & 1) * T::STAGE_BYTES;
    compute_stage<T, A_K, B_K>(st, st + T::A_BYTES, acc, wm, wn, lane);
  }
  __syncthreads();

  // ---- epilogue: one 32-row slab per wave row at a time through LDS ----
  SWG_LDS float* slab = (SWG_LDS float*)smem;
  typename Epi::template Prefetch<T> pf;
  SlabCtx<T> ctx{slab, tm, tn, 0, g.M, g.N};
#pragma unroll
  for (int s = 0; s < T::FM; ++s) {
    ctx.s = s;
    Epi::template prefetch<T>(ep, ctx, pf, tid);
    if (s > 0) __syncthreads();
    const int sr = wm * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * T::WTN + j * 32 + q * 8 + (lane >> 5) * 4;
        f32x4 v = {acc[s][j][4 * q + 0], acc[s][j][4 * q + 1], acc[s][j][4 * q + 2], acc[s][j][4 * q + 3]};
        *(SWG_LDS f32x4*)(slab + sr * T::SLAB_LD + c) = v;
      }
    __syncthreads();
    Epi::template apply<T>(ep, ctx, pf, tid);
  }
}

// ---------------------------------------------------------------------------
// Plain epilogue: C = bf16(acc), row-major with leading dimension ldc.
// ---------------------------------------------------------------------------
struct EpiStore {
  struct Params {
    uint16_t* C;
    int64_t ldc;
  };
  template <class T>
  struct Prefetch {};
  template <class T>
  __device__ static void prefetch(const Params&, const SlabCtx<T>&, Prefetch<T>&, int) {}
  template <class T>
  __device__ static void apply(const Params& p, const SlabCtx<T>& c, Prefetch<T>&, int tid) {
    constexpr int CPR = T::BN / 8;  // 8-column chunks per slab row
    constexpr int ITEMS = T::SLAB_ROWS * CPR;
    static_assert(ITEMS % T::THREADS == 0, "slab items must split evenly");
#pragma unroll
    for (int k = 0; k < ITEMS / T::THREADS; ++k) {
      const int it = tid + k * T::THREADS;
      const int sr = it / CPR, ch = it % CPR;
      const int row = c.row(sr), col = c.tn * T::BN + ch * 8;
      if (row < c.M && col < c.N) {
        u32x4 v = pack8(c.read8(sr, ch * 8));
        *(u32x4*)(p.C + (int64_t)row * p.ldc + col) = v;
      }
    }
  }
};

}  // namespace swg
