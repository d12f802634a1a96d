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
// Design (one workgroup per output tile; BK-deep k-tiles in LDS rings of
// three A buffers and two B buffers):
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

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int SA = 3, SB = 2;  // LDS ring depths of the A and B tiles
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // one wave's output tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int SLAB_ROWS = 32 * WM;           // epilogue slab: 32 rows per wave row
  static constexpr int SLAB_LD = BN + 4;              // fp32 row pitch (+16 B breaks bank aliasing)
  static constexpr int SLAB_BYTES = SLAB_ROWS * SLAB_LD * 4;
  static constexpr int RING_BYTES = SA * A_BYTES + SB * B_BYTES;
  static constexpr int LDS_BYTES = (RING_BYTES > SLAB_BYTES) ? RING_BYTES : SLAB_BYTES;
  // direct-to-LDS load instructions (1 KB each) each wave issues per stage
  static constexpr int LA = A_BYTES / 1024 / WAVES, LB = B_BYTES / 1024 / WAVES;
  static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
  static_assert(BM % (512 / BK) == 0 && BN % (512 / BK) == 0, "whole 1 KB blocks per tile");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per workgroup");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert((A_BYTES / 1024) % WAVES == 0 && (B_BYTES / 1024) % WAVES == 0, "1 KB load blocks must split over waves");
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
  // Grouped GEMMs ("Lesson 24", sections 42-43: one launch for the experts'
  // GEMMs of different sizes).  group_off [groups + 1] holds token offsets
  // in device memory: group e owns token rows [group_off[e], group_off[e+1]).
  // Grouped over M, the tokens are the rows of A and C and each group has its
  // own B, group_stride_b elements apart; tiles_m is then an upper bound on
  // the tile rows of all groups together.  Grouped over K, the tokens are
  // the k-rows of both (MN-major) operands and each group writes its own C,
  // group_stride_c elements apart; tiles_m x tiles_n is one group's output.
  const int* group_off;
  int groups;
  int64_t group_stride_b, group_stride_c;
  // Split tail (kSplitTail): the launch covers tile ids [tile_base,
  // tile_base + grid / splits) of the tiles_m x tiles_n order, each tile's
  // K range cut into `splits` parts, one workgroup each.  Dense launches
  // cover ids [0, tile_count) (tile_count <= tiles_m * tiles_n).
  int tile_base, tile_count, splits;
};

// How the kernel maps work to tiles.
enum GroupMode { kDense = 0, kGroupM = 1, kGroupK = 2, kSplitTail = 3 };

// ---------------------------------------------------------------------------
// LDS layouts
// ---------------------------------------------------------------------------
// LDS layouts.  Every global -> LDS copy is one wave instruction that
// fills 1 KB of LDS, 16 B per lane in lane order, so a layout is fixed by
// which (row, chunk) each lane loads.  With BK = 64 each instruction covers
// whole 128 B lines (one L2 request per line; BK = 32 needed twice the
// requests), and the MFMA fragment reads must not collide in LDS banks.
//
// K-major tile [rows][BK]: rows of BK/8 16-byte chunks, the chunk index
// XOR-ed with a function of the row so that the rows one ds_read_b128 phase
// touches land in distinct banks.  The XOR stays inside a row's 128 B line
// (BK = 64), which the vector memory path still fetches as one request.
template <int BK>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
  else return ((r >> 1) ^ (r >> 3)) & 3;
}
template <int BK>
__device__ __forceinline__ int lds_off_k(int r, int c) { return r * (BK * 2) + ((c ^ swz_k<BK>(r)) << 4); }

// MN-major tile [BK][ROWS]: k-rows of ROWS/8 chunks.  One
// ds_read_b64_tr_b16 reads a 64 B run (4 chunks) from each of four
// consecutive k-rows (and again from the four 8 rows further on).  The
// chunk index is XOR-ed with a function of k%4 so that those four runs fall
// in four different 64 B quarters of the 64 banks (256 B):
//   ROWS >= 128 (k-rows of 256 or 512 B, all starting at bank 0): XOR
//     4*(k%4), which moves the run to quarter (q ^ k%4) of its 256 B;
//   ROWS = 64 (k-rows of 128 B: odd rows start at bank 32): XOR 2*(k%4),
//     which moves rows k%4 >= 2 to the other 64 B of their half.
// (2*(k%4) for the wider rows left rows k and k+1 in the same quarter: a
// two-way bank conflict, measured at 12-15% of all cycles of the GEMMs with
// two MN-major operands.)  The XOR stays below ROWS/8: it permutes the
// chunks of one k-row.
template <int ROWS>
__device__ __forceinline__ int swz_mn(int k) {
  if constexpr (ROWS >= 128) return (k & 3) << 2;
  else return (k & 3) << 1;
}
template <int ROWS>
__device__ __forceinline__ int lds_off_mn(int k, int c) {
  return k * (ROWS * 2) + ((c ^ swz_mn<ROWS>(k)) << 4);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// compile-time bool carried by a type (selects a variant of a generic lambda)
template <bool V>
struct integral_c {
  static constexpr bool value = V;
};
// compile-time int carried by a type; converts to int
template <int V>
struct int_c {
  static constexpr int value = V;
  __device__ constexpr operator int() const { return V; }
};

// Buffer descriptor (V#) of a raw byte range: 48-bit base, stride 0,
// num_records = bytes, dword 3 = 0x00020000 (32-bit data format, as gfx9
// expects for untyped access).  The range check zero-fills any 16 B load at
// or past `bytes` (all offsets and ranges here are multiples of 16 B).
// The byte count is clamped into [0, 0x7FFFFFF0] with 32-bit compares, which
// stay scalar for a uniform count (a 64-bit compare is a vector instruction
// that holds its constant in a VGPR pair).
__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
  const uint32_t hi = (uint32_t)((uint64_t)bytes >> 32), lo = (uint32_t)bytes;
  return (int32_t)hi < 0 ? 0u : ((hi != 0u || lo > 0x7FFFFFF0u) ? 0x7FFFFFF0u : lo);
}
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = clamp_records(bytes);
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = (int)n;
  r[3] = 0x00020000;
  return r;
}

// Epilogue accesses are buffer instructions on a descriptor that starts at
// the tile's first row and ends at the row bound: rows at or past it fall
// outside num_records, so their loads return zeros and their stores are
// dropped by the hardware range check.  The epilogue then has no branch
// around a global access.  (Under `if (row < M)` branches the compiler's
// wait-count pass lost count of the prefetched loads and waited for every
// outstanding access, vmcnt(0), before each 8-column chunk, which undid the
// prefetch.)  Offsets are 32-bit bytes from the tile's first row: a tile
// spans at most 256 rows of at most 2^21 elements.
typedef __amdgpu_buffer_rsrc_t brsrc_t;
__device__ __forceinline__ brsrc_t rows_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)clamp_records(bytes), 0x00020000);
}
// an offset past every num_records above: the access is dropped
constexpr uint32_t kOffOutOfRange = 0x80000000u;
// cache policy of the epilogue's accesses: nontemporal (streamed once)
constexpr int kPolicyNT = 2;
__device__ __forceinline__ u32x4 bload16(brsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyNT);
}
__device__ __forceinline__ void bstore16(brsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kPolicyNT);
}

// One wave-wide direct-to-LDS load: lane i's 16 B at byte offset
// voff + soff of the buffer land at LDS address m0 + 16*i.  Issued as
// inline asm so that the compiler's wait-count pass does not track these LDS
// writes: it cannot tell the ring stages apart and would otherwise wait for
// every in-flight stage before each LDS read.  Ordering is explicit instead
// (wait_vmcnt + barrier in the main loop).  voff: a per-lane offset held in a
// VGPR for the whole K loop (one per 1 KB block), which alone decides the
// range check; soff: a scalar added after it (the hardware leaves the scalar
// offset out of the range check), here a K-major stage's k offset.  Summing
// the two with a v_add before each load had cost a VALU issue slot per load
// between the MFMAs (~1% on every GEMM).  M0 holds the LDS base; the s_nop
// is the one wait state the hardware needs between writing M0 and the LDS
// DMA that reads it.  M0 is a reserved register, which clang does not
// accept in a clobber list (it warns that it may not be preserved), so it is
// written here without one.  That is safe because nothing else in these
// kernels reads M0: in the compiled library every M0 write is one of these
// blocks, and no compiler-generated instruction (v_movrel, s_sendmsg, LDS
// direct, indexed readlane) reads it.  A kernel that added such an
// instruction would have to set M0 after these loads.
// m0: the LDS byte address of the 1 KB destination, a scalar (computed from
// a hoisted LDS base with scalar arithmetic: a pointer-derived value had been
// built in VGPRs and moved back with v_readfirstlane for every load).
__device__ __forceinline__ void dma16(const i32x4& rsrc, int m0, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %3, %1 offen lds"
      :
      : "v"(voff), "s"(soff), "s"(m0), "s"(rsrc)
      : "memory");
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

// Direct-to-LDS loads of one operand tile (ROWS x BK, BK = 64).  One wave
// instruction fills 1 KB block b of the tile's LDS image, 16 B per lane in
// lane order; each lane picks the global chunk that belongs at its LDS slot
// under the swizzle.  The byte offset of lane `lane` in block b splits into
// a per-lane part that depends on b only through its swizzle class and a
// wave-uniform part:
//   K-major: rsrc is based at row tile*ROWS of the operand; block b holds
//            rows 8b .. 8b+7, row 8b + lane/8 gets chunk (lane%8) ^ swz, and
//            swz = (lane/8) ^ (b%8): class b%8, uniform part 16*b*ld + 2*k0.
//   MN-major: rsrc is based at k-row k0 of the operand; block b holds k-rows
//            KROWS*b .. with KROWS = 512/ROWS, and the swizzle of k-row k
//            depends on k%4 only: class b%2 when KROWS = 2, none otherwise;
//            uniform part 2*KROWS*b*ld.
template <int ROWS, bool KMAJ>
__device__ __forceinline__ uint32_t dma_lane_base(int64_t ld, int tile, int pair_off, int b, int lane) {
  if constexpr (KMAJ) {
    const int rr = lane >> 3;
    const int c = (lane & 7) ^ rr ^ (b & 7);
    return (uint32_t)(rr * ld * 2) + (uint32_t)(c * 16);
  } else {
    constexpr int CPR = ROWS / 8, KROWS = 64 / CPR;
    const int kr = lane / CPR;
    const int k = KROWS * b + kr;
    const int c = (lane % CPR) ^ swz_mn<ROWS>(k);
    const int col = mn_col<ROWS>(c * 8, tile, pair_off);
    return (uint32_t)(kr * ld * 2) + (uint32_t)col * 2u;
  }
}
template <int ROWS, bool KMAJ>
__device__ __forceinline__ uint32_t dma_block_add(int64_t ld, int b, int k0) {
  if constexpr (KMAJ) return (uint32_t)(16 * b * ld) + (uint32_t)(2 * k0);
  else return (uint32_t)(2 * (64 / (ROWS / 8)) * b * ld);
}

// 32x16 MFMA operand fragment: lane l gets row r0 + l%32 and the 8 k values
// kk*16 + 8*(l/32) + 0..7.
template <int BK>
__device__ __forceinline__ bf16x8 frag_k(const SWG_LDS char* t, int r0, int kk, int lane) {
  const int r = r0 + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *(const SWG_LDS bf16x8*)(t + lds_off_k<BK>(r, c));
}

// Same fragment from an MN-major tile.  ds_read_b64_tr_b16 transposes within
// each group of 16 lanes: lane j receives, in slot e, element j%4 of the 8 B
// read by lane 4e + j/4.  So lane 4e+q of group g reads k-row (base + e),
// columns col0 + 4q .. +3, and lane j ends up with column col0 + j, k-rows
// base .. base+3.  Two reads, 4 k-rows apart, give the 8 k values.
//
// The MN-major swizzle depends on k % 4 only and a k16 step moves k by 16,
// so the byte offset of a lane's read is a per-lane part, which depends on
// the fragment's column (the XOR mixes the column's 64 B quarter with the
// lane's k-row), plus kk*16*ROWS*2.  frag_mn_lane_off gives the per-lane
// part (kk = 0); the kernel computes it once per fragment, and every read in
// the K loop is then one register plus an immediate offset.
template <int ROWS>
__device__ __forceinline__ int frag_mn_lane_off(int r0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int e = j >> 2, q = j & 3;
  const int k = (g >> 1) * 8 + e;
  const int col = r0 + (g & 1) * 16 + q * 4;
  return lds_off_mn<ROWS>(k, col >> 3) + (col & 7) * 2;
}
// the MN-major fragment of step kk from its per-lane offset
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_mn_at(const SWG_LDS char* t, int off, int kk) {
  const SWG_LDS char* p = t + off + kk * 16 * ROWS * 2;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)p);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWG_LDS i16x4*)(p + 4 * ROWS * 2));
  i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// per-lane offsets of the MN-major fragments (unused for K-major operands)
template <class T>
struct MnOff {
  int a[T::FM], b[T::FN];
};

template <class T>
struct Frags {
  bf16x8 a[T::FM], b[T::FN];
};

template <class T, bool A_K, bool B_K>
__device__ __forceinline__ void load_frags(const SWG_LDS char* As, const SWG_LDS char* Bs, Frags<T>& f, int kk,
                                           int wm, int wn, int lane, const MnOff<T>& mo) {
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
    f.a[i] = A_K ? frag_k<T::BK>(As, wm * T::WTM + i * 32, kk, lane) : frag_mn_at<T::BM>(As, mo.a[i], kk);
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
    f.b[j] = B_K ? frag_k<T::BK>(Bs, wn * T::WTN + j * 32, kk, lane) : frag_mn_at<T::BN>(Bs, mo.b[j], kk);
}

// LDS read instructions per fragment set (transposing reads take two)
template <class T, bool A_K, bool B_K>
constexpr int frag_reads() {
  return T::FM * (A_K ? 1 : 2) + T::FN * (B_K ? 1 : 2);
}

// Read fragment i of the next step: A fragments 0..FM-1, then B fragments.
template <class T, bool A_K, bool B_K>
__device__ __forceinline__ void read_frag(const SWG_LDS char* As, const SWG_LDS char* Bs, Frags<T>& f, int i,
                                          int kk, int wm, int wn, int lane, const MnOff<T>& mo) {
  if (i < T::FM)
    f.a[i] = A_K ? frag_k<T::BK>(As, wm * T::WTM + i * 32, kk, lane) : frag_mn_at<T::BM>(As, mo.a[i], kk);
  else
    f.b[i - T::FM] = B_K ? frag_k<T::BK>(Bs, wn * T::WTN + (i - T::FM) * 32, kk, lane)
                         : frag_mn_at<T::BN>(Bs, mo.b[i - T::FM], kk);
}

// One k16 step with an explicit issue order, slot by slot: the LDS read of
// next-step fragment i, then global->LDS load i (NLOAD of them, issued only
// in a stage's last step), then MFMA i, each slot fenced by sched_barrier(0)
// so the compiler keeps the interleave.  Spreading the loads one per MFMA
// keeps the vector memory queue from backing up into the wave's in-order
// instruction stream, which would stall the MFMAs behind a burst of loads.
template <class T, bool A_K, bool B_K, int NLOAD, class LoadFn>
__device__ __forceinline__ void step(const SWG_LDS char* As, const SWG_LDS char* Bs, const Frags<T>& cur,
                                     Frags<T>& nxt, int kk_next,
                                     f32x16 (&acc)[T::FM][T::FN], int wm, int wn, int lane, const MnOff<T>& mo,
                                     LoadFn&& ld) {
  constexpr int NF = T::FM + T::FN, NM = T::FM * T::FN;
  constexpr int NS = (NM > NF ? NM : NF) > NLOAD ? (NM > NF ? NM : NF) : NLOAD;
  // load j goes into slot j*NS/NLOAD: evenly spread over the step
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i < NF) read_frag<T, A_K, B_K>(As, Bs, nxt, i, kk_next, wm, wn, lane, mo);
    if constexpr (NLOAD > 0) {
      if ((i * NLOAD) % NS < NLOAD) ld(i * NLOAD / NS);
    }
    if (i < NM) {
      const int fi = i / T::FN, fj = i % T::FN;
      acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[fj], cur.a[fi], acc[fi][fj], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// blockIdx -> (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs, so each XCD is first given a contiguous run of tile ids (its own
// L2 then sees neighbouring tiles), and tile ids are walked in groups of GM
// tile rows so that concurrently running tiles share A and B panels.  32
// tiles of an XCD as 4 rows x 8 columns or 8 x 4 share the same 12 panels;
// the wider form puts 8 neighbouring column tiles side by side, whose slices
// of an MN-major B are one contiguous run per k-row.  Measured in randomly
// interleaved rounds: GEMM-1 (MN-major B) 2.5% faster at the target shape
// and 4.6% at the Llama-like one with GM = 4 than with 8, the dout GEMMs
// ~1%, the dx GEMM 1.5%; dW1, whose A is MN-major along m, 0.8% slower.
// group_rows<A_K>() is the rule: 4 unless A is MN-major.
__device__ __forceinline__ int xcd_linear(int pid, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = pid % 8, local = pid / 8;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}
template <bool A_K>
constexpr int group_rows() {
  return A_K ? 4 : 8;
}
template <int GM>
__device__ __forceinline__ void tile_order(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = id / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in_group = id - group * GM * tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}
template <int GM>
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  tile_order<GM>(xcd_linear(pid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// Token range [lo, hi) of group e, clamped into [0, M] and made non-empty
// only when increasing: offsets that are not a valid partition give
// unspecified results but never an access outside the token range.
__device__ __forceinline__ void group_range(const int* off, int e, int M, int& lo, int& hi) {
  int a = off[e], b = off[e + 1];
  a = a < 0 ? 0 : (a > M ? M : a);
  b = b < a ? a : (b > M ? M : b);
  lo = a;
  hi = b;
}

// Grouped over M: tile row r of all groups together (group e contributes
// ceil(size_e / BM) tile rows, in group order) -> its group's first token row
// r0 and end row m_end.  Each wave scans 64 groups at a time: an inclusive
// prefix sum of the tile-row counts across the lanes, then a ballot for the
// lane whose range holds r.  False when r is past the last tile row.
template <int BM>
__device__ __forceinline__ bool find_group_row(const int* off, int groups, int M, int r, int& grp, int& r0,
                                               int& m_end) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c0 = 0; c0 < groups; c0 += 64) {
    const int e = c0 + lane;
    int lo = 0, hi = 0;
    if (e < groups) group_range(off, e, M, lo, hi);
    const int cnt = (hi - lo + BM - 1) / BM;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    const int excl = incl - cnt;
    const unsigned long long hit = __ballot(r >= base + excl && r < base + incl);
    if (hit != 0ull) {
      const int l = __ffsll((long long)hit) - 1;
      const int lo_l = __shfl(lo, l, 64), hi_l = __shfl(hi, l, 64), ex_l = __shfl(excl, l, 64);
      grp = __builtin_amdgcn_readfirstlane(c0 + l);
      r0 = __builtin_amdgcn_readfirstlane(lo_l + (r - base - ex_l) * BM);
      m_end = __builtin_amdgcn_readfirstlane(hi_l);
      return true;
    }
    base += __shfl(incl, 63, 64);
  }
  return false;
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Epilogue context handed to the epilogue functors for one slab.
template <class T>
struct SlabCtx {
  const SWG_LDS float* slab;  // [SLAB_ROWS][SLAB_LD] fp32
  int r0, tn, s;              // the tile's first row, its column tile, the slab index
  int M, N;                   // rows at or past M and columns at or past N are not stored
  int64_t goff;               // element offset of this group's C (grouped over K), else 0
  // global row of slab row sr
  __device__ __forceinline__ int row(int sr) const {
    return r0 + (sr >> 5) * T::WTM + s * 32 + (sr & 31);
  }
  // The epilogues walk a slab in 8-column chunks: a thread's item k is slab
  // row q + k * P, chunk ch, with q = tid / CPR and ch = tid % CPR (CPR
  // chunks per row, P rows per pass of the workgroup).  Since P divides 32,
  // that row lies item_row(k) + q rows below the tile's first row, and
  // item_row(k) is a constant once k and s are (unrolled loops): each item's
  // address is then a per-thread base plus a scalar product.
  static constexpr int CPR = T::BN / 8, P = T::THREADS / CPR;
  static_assert(T::THREADS % CPR == 0 && 32 % P == 0, "item rows must split into q + item_row(k)");
  __device__ __forceinline__ int item_row(int k) const {
    return ((k * P) >> 5) * T::WTM + s * 32 + ((k * P) & 31);
  }
  __device__ __forceinline__ f32x8 read8(int sr, int c) const {
    const SWG_LDS f32x4* p = (const SWG_LDS f32x4*)(slab + sr * T::SLAB_LD + c);
    f32x4 lo = p[0], hi = p[1];
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// The epilogue reads issued while slabs are processed: read e (item e % NI of
// slab PRE + e / NI) goes out during apply(a), a the smallest with
// e < ceil(E (a + 1) / A).  It must be issued before its slab is processed
// (a < slab) and into registers whose previous slab, slab - PD, is done
// (a > slab - PD).
template <int E, int A, int NI, int PRE, int PD>
constexpr bool epi_schedule_ok() {
  for (int e = 0; e < E; ++e) {
    int a = 0;
    while (!(e < (E * (a + 1) + A - 1) / A)) ++a;
    const int slab = PRE + e / NI;
    if (a >= slab || a <= slab - PD) return false;
  }
  return true;
}

template <class T, bool A_K, bool B_K, class Epi, int GRP = kDense>
__global__ void __launch_bounds__(T::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) gemm_kernel(const GemmArgs g, const typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  constexpr int GM = group_rows<A_K>();
  // tile coordinates; r0 / m_end: the tile's first row and the row bound;
  // Ag, Bg, Kg: this tile's operands and reduction length
  int tm, tn, r0, m_end, Kg = g.K;
  const uint16_t* Ag = g.A;
  const uint16_t* Bg = g.B;
  int64_t goff = 0;
  if constexpr (GRP == kDense) {
    tile_order<GM>(xcd_linear(blockIdx.x, g.tile_count), g.tiles_m, g.tiles_n, tm, tn);
    r0 = tm * T::BM;
    m_end = g.M;
  } else if constexpr (GRP == kSplitTail) {
    // workgroup -> (tail tile t, part s); part s takes k-stages
    // [s * nst / splits, (s + 1) * nst / splits) and writes its fp32 partial
    // tile to slot t * splits + s of the epilogue's buffer
    const int t = blockIdx.x / g.splits, sp = blockIdx.x - t * g.splits;
    tile_order<GM>(g.tile_base + t, g.tiles_m, g.tiles_n, tm, tn);
    const int nst = (g.K + T::BK - 1) / T::BK;
    const int k0 = sp * nst / g.splits * T::BK;
    const int k1 = (sp + 1) * nst / g.splits * T::BK;
    Ag += A_K ? (int64_t)k0 : (int64_t)k0 * g.lda;
    Bg += B_K ? (int64_t)k0 : (int64_t)k0 * g.ldb;
    Kg = (k1 < g.K ? k1 : g.K) - k0;
    goff = (int64_t)blockIdx.x * T::BM * T::BN;
    r0 = tm * T::BM;
    m_end = g.M;
  } else if constexpr (GRP == kGroupM) {
    static_assert(A_K, "grouped over M: A is the K-major token operand");
    int r, grp;
    tile_coords<GM>(blockIdx.x, g.tiles_m, g.tiles_n, r, tn);
    // past the last tile row of the last group: the whole workgroup leaves
    // (the condition is uniform across it, before any barrier)
    if (!find_group_row<T::BM>(g.group_off, g.groups, g.M, r, grp, r0, m_end)) return;
    tm = 0;  // K-major A is addressed from r0
    Bg += (int64_t)grp * g.group_stride_b;
  } else {
    static_assert(!A_K && !B_K, "grouped over K: both operands are MN-major token operands");
    // Groups' K loops differ in length.  Workgroup ids go to the XCDs round
    // robin, so taking the ids in plain order gives every XCD an equal share
    // of every group; contiguous runs per XCD (as for one GEMM) had left
    // whole large groups on one XCD (measured: the expert block's backward
    // 2.03 ms against 1.65 ms in plain order; largest-group-first order on
    // top of it gained nothing).
    const int per = g.tiles_m * g.tiles_n;
    const int id = blockIdx.x;
    const int grp = id / per;
    tile_order<GM>(id - grp * per, g.tiles_m, g.tiles_n, tm, tn);
    int lo, hi;
    group_range(g.group_off, grp, g.K, lo, hi);
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    Ag += (int64_t)lo * g.lda;
    Bg += (int64_t)lo * g.ldb;
    Kg = hi - lo;
    goff = (int64_t)grp * g.group_stride_c;
    r0 = tm * T::BM;
    m_end = g.M;
  }

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x16{};

  // K-major operands: descriptors based at the tile's first row, fixed for
  // the whole K loop.  MN-major: rebased at every stage's first k-row.
  const int nk = (Kg + T::BK - 1) / T::BK;
  i32x4 ra = A_K ? make_rsrc(Ag + (int64_t)r0 * g.lda, ((int64_t)m_end - (int64_t)r0) * g.lda * 2)
                 : make_rsrc(Ag, 0);
  i32x4 rb =
      B_K ? make_rsrc(Bg + (int64_t)tn * T::BN * g.ldb, ((int64_t)g.N - (int64_t)tn * T::BN) * g.ldb * 2)
          : make_rsrc(Bg, 0);

  // Software pipeline.
  //  * Global -> LDS: ring of SA = 3 A buffers and SB = 2 B buffers (160 KB
  //    for 256x256 tiles).  A(j) is loaded during the first two k16 steps of
  //    stage j-2, B(j) during the last step of stage j-2 (after its barrier).
  //    The direct-to-LDS path drains about 64 B per clock per CU: a whole
  //    64 KB stage issued within one step fills the address FIFO, and a
  //    blocked load stalls the MFMAs queued behind it in the wave's in-order
  //    stream.  Split this way, no step issues more than 32 KB per CU and
  //    every load has at least three steps to land.
  //  * LDS -> registers: fragments of k16 step s+1 are read while the MFMAs
  //    of step s run, across the stage boundary too.  In the last step of
  //    stage kt each wave waits for its own loads of stage kt+1 (vmcnt) and
  //    its own outstanding LDS reads (lgkmcnt: this step's fragments, read
  //    one step earlier) and joins the barrier.  After it every wave's loads
  //    of stage kt+1 are visible and nobody reads stage kt any more, so B(kt)'s
  //    buffer takes B(kt+2); A(kt)'s buffer takes A(kt+3) one stage later.
  static_assert(T::SA == 3 && T::SB == 2, "schedule written for a 3 + 2 ring");
  constexpr int KS = T::BK / 16;
  static_assert(KS == 4, "A loads use steps 0 and 1, B loads step 3");
  constexpr int LA = T::LA, LB = T::LB;
  static_assert(LA % 2 == 0, "A loads split over two steps");
  // ring slots: A(j) in A buffer j % 3, B(j) in B buffer j % 2
  auto a_buf = [&](int s) { return (SWG_LDS char*)smem + s * T::A_BYTES; };
  auto b_buf = [&](int s) { return (SWG_LDS char*)smem + 3 * T::A_BYTES + s * T::B_BYTES; };
  auto a_ptr = [&](int j) { return a_buf(j % 3); };
  auto b_ptr = [&](int j) { return b_buf(j & 1); };
  // descriptors: K-major fixed, MN-major rebased at the stage's first k-row
  // and ending after its k-rows: BK of them except in the last stage.  That
  // range, rows * ld * 2 bytes, is below 2^28 (ld <= 2^21), so it needs none
  // of make_rsrc's 64-bit clamps, which in the unrolled loop had cost 64-bit
  // compares and SGPR spills every stage; the full and last-stage ranges are
  // computed once and selected per stage with scalar ops (readfirstlane
  // keeps them in SGPRs: the descriptor operand of the DMA asm is scalar).
  const int tail_rows = Kg - (nk - 1) * T::BK;  // 1..BK when nk > 0
  const int mn_full_a = __builtin_amdgcn_readfirstlane(A_K ? 0 : T::BK * (int)g.lda * 2);
  const int mn_tail_a = __builtin_amdgcn_readfirstlane(A_K ? 0 : tail_rows * (int)g.lda * 2);
  const int mn_full_b = __builtin_amdgcn_readfirstlane(B_K ? 0 : T::BK * (int)g.ldb * 2);
  const int mn_tail_b = __builtin_amdgcn_readfirstlane(B_K ? 0 : tail_rows * (int)g.ldb * 2);
  auto rs_mn = [&](const uint16_t* base, int64_t ld, int full, int tail, int j) -> i32x4 {
    const uint64_t a = (uint64_t)(base + (int64_t)j * T::BK * ld);
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
    r[2] = j < nk - 1 ? full : (j == nk - 1 ? tail : 0);
    r[3] = 0x00020000;
    return r;
  };
  auto rs_a = [&](int j) -> i32x4 {
    if constexpr (A_K) return ra;
    else return rs_mn(Ag, g.lda, mn_full_a, mn_tail_a, j);
  };
  auto rs_b = [&](int j) -> i32x4 {
    if constexpr (B_K) return rb;
    else return rs_mn(Bg, g.ldb, mn_full_b, mn_tail_b, j);
  };
  // this wave loads blocks wave + 4i; their swizzle classes alternate
  // between those of blocks wave and wave + 4 (K-major) or are all equal
  // (MN-major), so two per-lane bases per operand cover every block
  static_assert(T::WAVES == 4 && T::BK == 64, "load classes worked out for 4 waves and BK = 64");
  const uint32_t va0 = dma_lane_base<T::BM, A_K>(g.lda, tm, 0, wave, lane);
  const uint32_t va1 = dma_lane_base<T::BM, A_K>(g.lda, tm, 0, wave + T::WAVES, lane);
  const uint32_t vb0 = dma_lane_base<T::BN, B_K>(g.ldb, tn, g.pair_off, wave, lane);
  const uint32_t vb1 = dma_lane_base<T::BN, B_K>(g.ldb, tn, g.pair_off, wave + T::WAVES, lane);
  // load block idx of stage j into ring slot s (s = j % 3 for A, j % 2 for B)
  // LDS byte address of this wave's first 1 KB block in the ring, a scalar
  const int lds_wave = __builtin_amdgcn_readfirstlane((int)(uintptr_t)smem) + wave * 1024;
  // Each 1 KB block's offset within the operand's rows is folded into a
  // per-block lane offset held in a VGPR for the whole K loop (an MN-major
  // operand's descriptor moves from stage to stage instead; a K-major one's
  // k offset goes in the DMA's scalar offset).  As 2 x 8 loop-invariant
  // SGPRs they had pushed the unrolled loop into SGPR spills (v_readlane
  // reloads every stage).
  uint32_t vma[LA], vmb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    vma[i] = ((i & 1) ? va1 : va0) + dma_block_add<T::BM, A_K>(g.lda, wave + i * T::WAVES, 0);
    asm volatile("" : "+v"(vma[i]));
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    vmb[i] = ((i & 1) ? vb1 : vb0) + dma_block_add<T::BN, B_K>(g.ldb, wave + i * T::WAVES, 0);
    asm volatile("" : "+v"(vmb[i]));
  }
  // a K-major stage's k offset, 2 * j * BK bytes (within every row, K being
  // a multiple of BK), goes in the scalar offset; the row range check is
  // decided by the per-lane offsets
  auto load_a_to = [&](const i32x4& r, int j, int s, int idx) {
    const int m0 = lds_wave + s * T::A_BYTES + idx * T::WAVES * 1024;
    dma16(r, m0, vma[idx], A_K ? (uint32_t)(2 * j * T::BK) : 0u);
  };
  auto load_b_to = [&](const i32x4& r, int j, int s, int idx) {
    const int m0 = lds_wave + 3 * T::A_BYTES + s * T::B_BYTES + idx * T::WAVES * 1024;
    dma16(r, m0, vmb[idx], B_K ? (uint32_t)(2 * j * T::BK) : 0u);
  };
  auto load_a = [&](const i32x4& r, int j, int idx) { load_a_to(r, j, j % 3, idx); };
  auto load_b = [&](const i32x4& r, int j, int idx) { load_b_to(r, j, j & 1, idx); };
  // A bare s_barrier after an explicit lgkmcnt(0): __syncthreads() would add
  // a release fence that drains every outstanding LDS DMA (vmcnt(0)) and
  // serialises the ring.  The clobber keeps the compiler from moving LDS
  // accesses across it.
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  auto no_load = [](int) {};

  // prologue, in this issue order: A0 B0 A1 B1 A2
  // Epilogue reads (an epilogue's per-slab global inputs, PD slabs in
  // registers): slabs 0 .. PRE-1 are requested during the last two k-stages,
  // one item per MFMA slot, and slab s + PRE one item at a time while slab s
  // is processed.  Issued in bursts instead (all of a slab's loads at once),
  // they had stalled each wave at the issue point with no other work beside
  // it (~1 us per 16 loads); between the MFMAs of the last stages they are
  // largely hidden.
  constexpr int PD = Epi::kPrefetchDepth < T::FM ? Epi::kPrefetchDepth : T::FM;
  static_assert(PD >= 1, "prefetch depth");
  constexpr int PRE = PD > 1 ? PD - 1 : 1;
  constexpr int NI = T::SLAB_ROWS * (T::BN / 8) / T::THREADS;  // items per thread and slab
  // PRE_PER_STEP items in each of the 2 * KS steps of the last two stages;
  // the stage before the last issues items [0, PRE_HALF)
  constexpr int PRE_LOADS = PRE * NI, PRE_PER_STEP = (PRE_LOADS + 2 * KS - 1) / (2 * KS);
  constexpr int PRE_HALF = KS * PRE_PER_STEP;
  // epilogue loads the stage before the last issues ahead of its wait (steps
  // 1-3; items past PRE_LOADS are skipped)
  constexpr int TAIL1_LOADS = (3 * PRE_PER_STEP < PRE_LOADS ? 3 * PRE_PER_STEP : PRE_LOADS) * Epi::kLoadsPerItem;
  typename Epi::template Prefetch<T> pf[PD];
  Frags<T> f[2];
  MnOff<T> mo;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    mo.a[i] = A_K ? 0 : frag_mn_lane_off<T::BM>(wm * T::WTM + i * 32, lane);
    if constexpr (!A_K) asm volatile("" : "+v"(mo.a[i]));  // kept in a register, not rebuilt per read
  }
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    mo.b[j] = B_K ? 0 : frag_mn_lane_off<T::BN>(wn * T::WTN + j * 32, lane);
    if constexpr (!B_K) asm volatile("" : "+v"(mo.b[j]));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < nk) {
      const i32x4 r1 = rs_a(j), r2 = rs_b(j);
#pragma unroll
      for (int i = 0; i < LA; ++i) load_a(r1, j, i);
#pragma unroll
      for (int i = 0; i < LB; ++i) load_b(r2, j, i);
    }
  }
  if (2 < nk) {
    const i32x4 r1 = rs_a(2);
#pragma unroll
    for (int i = 0; i < LA; ++i) load_a(r1, 2, i);
  }
  if (nk > 0) {
    // stage 0 landed: A1 B1 A2 (when they exist) may stay in flight
    if (nk > 2) wait_vmcnt<2 * LA + LB>();
    else if (nk > 1) wait_vmcnt<LA + LB>();
    else wait_vmcnt<0>();
    barrier();
    load_frags<T, A_K, B_K>(a_ptr(0), b_ptr(0), f[0], 0, wm, wn, lane, mo);
  }
  // One stage of the K loop.  LDA / LDB: whether it issues A(kt+2) /
  // B(kt+2).  The three variants are chosen once per stage, so the loads
  // themselves sit in straight-line code between the MFMAs (a branch around
  // each of them had cost issue slots the MFMA pipe waited on).  sa, sb: the
  // ring slots of A(kt) and B(kt), kt % 3 and kt % 2, compile-time constants
  // in the unrolled steady state (so no slot arithmetic runs between the
  // MFMAs) and plain ints elsewhere.  TAIL: 1 for the stage before the last,
  // 2 for the last; their MFMA slots carry the epilogue's first reads
  // (pre_item below; read idx is item idx % NI of slab idx / NI).
  auto pre_item = [&](int idx) {
    if (idx < PRE_LOADS)
      Epi::template prefetch_item<T>(ep, SlabCtx<T>{nullptr, r0, tn, idx / NI, m_end, g.N, goff}, pf[idx / NI], tid,
                                     idx % NI);
  };
  auto stage = [&](int kt, auto lda, auto ldb, auto sa, auto sb, auto tail) {
    constexpr bool LDA = decltype(lda)::value, LDB = decltype(ldb)::value;
    constexpr int TAIL = decltype(tail)::value;
    static_assert(!(TAIL && (LDA || LDB)), "the last two stages load no operands");
    const int a0 = sa, b0 = sb;
    const int a1 = a0 == 2 ? 0 : a0 + 1, a2 = a0 == 0 ? 2 : a0 - 1;  // slots of A(kt+1), A(kt+2)
    const int b1 = b0 ^ 1;                                            // slot of B(kt+1); B(kt+2) reuses b0
    const SWG_LDS char* as = a_buf(a0);
    const SWG_LDS char* bs = b_buf(b0);
    // LDB holds exactly when kt + 2 < nk: then this is not one of the last
    // two stages
    const bool next = LDB ? true : kt + 1 < nk;
    constexpr int PL = TAIL ? PRE_PER_STEP : 0;
    constexpr int P0 = TAIL == 2 ? PRE_HALF : 0;  // this stage's first epilogue read
    // steps 0 and 1: A(kt+2), half in each (A(2) came with the prologue)
    const i32x4 rA = rs_a(kt + 2);
    step<T, A_K, B_K, LDA ? LA / 2 : PL>(as, bs, f[0], f[1], 1, acc, wm, wn, lane, mo, [&](int i) {
      if constexpr (LDA) load_a_to(rA, kt + 2, a2, i);
      if constexpr (TAIL) pre_item(P0 + i);
    });
    step<T, A_K, B_K, LDA ? LA / 2 : PL>(as, bs, f[1], f[0], 2, acc, wm, wn, lane, mo, [&](int i) {
      if constexpr (LDA) load_a_to(rA, kt + 2, a2, LA / 2 + i);
      if constexpr (TAIL) pre_item(P0 + PL + i);
    });
    step<T, A_K, B_K, PL>(as, bs, f[0], f[1], 3, acc, wm, wn, lane, mo, [&](int i) {
      if constexpr (TAIL) pre_item(P0 + 2 * PL + i);
    });
    // step 3: barrier, then the next stage's first fragments and B(kt+2)
    const SWG_LDS char* nas = as;
    const SWG_LDS char* nbs = bs;
    if (next) {
      // A(kt+1) and B(kt+1) must have landed; A(kt+2), issued after them,
      // may stay in flight, and so may the epilogue reads of the stage before
      // the last (issued after every operand load)
      if (LDB) wait_vmcnt<LA>();
      else wait_vmcnt<TAIL == 1 ? TAIL1_LOADS : 0>();
      barrier();
      nas = a_buf(a1);
      nbs = b_buf(b1);
    }
    const i32x4 rB = rs_b(kt + 2);
    step<T, A_K, B_K, LDB ? LB : PL>(nas, nbs, f[1], f[0], 0, acc, wm, wn, lane, mo, [&](int i) {
      if constexpr (LDB) load_b_to(rB, kt + 2, b0, i);
      if constexpr (TAIL) pre_item(P0 + 3 * PL + i);
    });
  };
  typedef integral_c<true> yes;
  typedef integral_c<false> no;
  int kt = 0;
  if (nk > 2) stage(kt++, no{}, yes{}, int_c<0>{}, int_c<0>{}, int_c<0>{});  // stage 0: A(2) came with the prologue
  // from kt = 1 on, six stages per trip: kt % 3 and kt % 2 run through
  // (1,1) (2,0) (0,1) (1,0) (2,1) (0,0)
  for (; kt + 7 < nk; kt += 6) {
    stage(kt, yes{}, yes{}, int_c<1>{}, int_c<1>{}, int_c<0>{});
    stage(kt + 1, yes{}, yes{}, int_c<2>{}, int_c<0>{}, int_c<0>{});
    stage(kt + 2, yes{}, yes{}, int_c<0>{}, int_c<1>{}, int_c<0>{});
    stage(kt + 3, yes{}, yes{}, int_c<1>{}, int_c<0>{}, int_c<0>{});
    stage(kt + 4, yes{}, yes{}, int_c<2>{}, int_c<1>{}, int_c<0>{});
    stage(kt + 5, yes{}, yes{}, int_c<0>{}, int_c<0>{}, int_c<0>{});
  }
  for (; kt + 2 < nk; ++kt) stage(kt, yes{}, yes{}, kt % 3, kt & 1, int_c<0>{});
  // The last two stages load no operands and request slabs 0 .. PRE-1 (with
  // fewer than two stages, the missing stages' reads are issued at once).
  if (kt + 1 < nk) {
    stage(kt, no{}, no{}, kt % 3, kt & 1, int_c<1>{});
    ++kt;
  } else {
#pragma unroll
    for (int i = 0; i < PRE_HALF; ++i) pre_item(i);
  }
  if (kt < nk) {
    stage(kt, no{}, no{}, kt % 3, kt & 1, int_c<2>{});
    ++kt;
  } else {
#pragma unroll
    for (int i = PRE_HALF; i < 2 * PRE_HALF; ++i) pre_item(i);
  }
  // Every stage load has been waited for.  The only vector memory reads in
  // flight now are the epilogue prefetches, which must stay in flight: the
  // barriers below are bare s_barriers, not __syncthreads() (whose fence
  // would wait for them).
  barrier();

  // ---- epilogue: one 32-row slab per wave row at a time through LDS; the
  // global reads of slabs PRE .. FM-1 are spread evenly over the processing
  // of slabs 0 .. FM-2, one or so per item ----
  constexpr int EPI_READS = PD > 1 ? (T::FM - PRE) * NI : 0;
  constexpr int APPLIES = T::FM > 1 ? T::FM - 1 : 1;
  auto epi_lo = [](int s) { return (EPI_READS * s + APPLIES - 1) / APPLIES; };
  static_assert(epi_schedule_ok<EPI_READS, APPLIES, NI, PRE, PD>(),
                "every slab's reads are issued before it is processed, into registers already consumed");
  SWG_LDS float* slab = (SWG_LDS float*)smem;
  SlabCtx<T> ctx{slab, r0, tn, 0, m_end, g.N, goff};
#pragma unroll
  for (int s = 0; s < T::FM; ++s) {
    ctx.s = s;
    if (s > 0) barrier();
    const int sr = wm * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * T::WTN + j * 32 + q * 8 + (lane >> 5) * 4;
        f32x4 v = {acc[s][j][4 * q + 0], acc[s][j][4 * q + 1], acc[s][j][4 * q + 2], acc[s][j][4 * q + 3]};
        *(SWG_LDS f32x4*)(slab + sr * T::SLAB_LD + c) = v;
      }
    barrier();
    Epi::template apply<T>(ep, ctx, pf[s % PD], tid, [&](int k) {
      // apply(s) issues epilogue reads [epi_lo(s), epi_lo(s + 1)), item k
      // its share; read e is item e % NI of slab PRE + e / NI
      const int a = epi_lo(s), cnt = epi_lo(s + 1) - a;
#pragma unroll
      for (int u = 0; u < (EPI_READS + APPLIES * NI - 1) / (APPLIES * NI) + 1; ++u) {
        const int e = a + (k * cnt + NI - 1) / NI + u;
        if (e < EPI_READS && e < a + ((k + 1) * cnt + NI - 1) / NI)
          Epi::template prefetch_item<T>(ep, SlabCtx<T>{slab, r0, tn, PRE + e / NI, m_end, g.N, goff},
                                         pf[(PRE + e / NI) % PD], tid, e % NI);
      }
    });
  }
}

// ---------------------------------------------------------------------------
// Plain epilogue: C = bf16(acc), row-major with leading dimension ldc.
// ---------------------------------------------------------------------------
struct EpiStore {
  static constexpr int kPrefetchDepth = 1, kLoadsPerItem = 0;
  struct Params {
    uint16_t* C;
    int64_t ldc;
  };
  // the same store for output columns n..
  static Params cols_from(const Params& p, int64_t n) { return {p.C + n, p.ldc}; }
  template <class T>
  struct Prefetch {};
  template <class T>
  __device__ static void prefetch_item(const Params&, const SlabCtx<T>&, Prefetch<T>&, int, int) {}
  template <class T, class Hook>
  __device__ static void apply(const Params& p, const SlabCtx<T>& c, Prefetch<T>&, int tid, Hook&& hook) {
    constexpr int CPR = T::BN / 8;  // 8-column chunks per slab row
    constexpr int ITEMS = T::SLAB_ROWS * CPR;
    static_assert(ITEMS % T::THREADS == 0, "slab items must split evenly");
    const brsrc_t dst = rows_rsrc(p.C + c.goff + (int64_t)c.r0 * p.ldc, (int64_t)(c.M - c.r0) * p.ldc * 2);
    const int ldc = (int)p.ldc;
#pragma unroll
    for (int k = 0; k < ITEMS / T::THREADS; ++k) {
      hook(k);  // this item's share of a later slab's reads, ahead of its stores
      const int it = tid + k * T::THREADS;
      const int sr = it / CPR, ch = it % CPR;
      const int col = c.tn * T::BN + ch * 8;
      const uint32_t off = col < c.N ? (uint32_t)((c.row(sr) - c.r0) * ldc + col) * 2u : kOffOutOfRange;
      bstore16(dst, off, pack8(c.read8(sr, ch * 8)));
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 partial tile of a split tail: the whole BM x BN tile (rows past M
// hold zeros from the zero-filled loads) at slot goff of P, row-major with
// pitch BN.  The split-tail reduce kernel adds a tile's parts in order.
// ---------------------------------------------------------------------------
struct EpiPartial {
  static constexpr int kPrefetchDepth = 1, kLoadsPerItem = 0;
  struct Params {
    float* P;
  };
  template <class T>
  struct Prefetch {};
  template <class T>
  __device__ static void prefetch_item(const Params&, const SlabCtx<T>&, Prefetch<T>&, int, int) {}
  template <class T, class Hook>
  __device__ static void apply(const Params& p, const SlabCtx<T>& c, Prefetch<T>&, int tid, Hook&& hook) {
    constexpr int CPR = T::BN / 8;
    constexpr int ITEMS = T::SLAB_ROWS * CPR;
    static_assert(ITEMS % T::THREADS == 0, "slab items must split evenly");
#pragma unroll
    for (int k = 0; k < ITEMS / T::THREADS; ++k) {
      hook(k);  // this item's share of a later slab's reads, ahead of its stores
      const int it = tid + k * T::THREADS;
      const int sr = it / CPR, ch = it % CPR;
      const f32x8 v = c.read8(sr, ch * 8);
      f32x4* q = (f32x4*)(p.P + c.goff + (int64_t)(c.row(sr) - c.r0) * T::BN + ch * 8);
      __builtin_nontemporal_store(__builtin_shufflevector(v, v, 0, 1, 2, 3), q);
      __builtin_nontemporal_store(__builtin_shufflevector(v, v, 4, 5, 6, 7), q + 1);
    }
  }
};

// C = bf16(sum over s < S of the parts of each tail tile), for tile ids
// [tile_base, tile_base + tiles) of the tiles_m x tiles_n order (GM: the
// group rows of the GEMM that wrote the parts); one thread per 8 columns of a
// tile row, BM * BN / 8 / 256 workgroups per tile.
template <class T, int GM>
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* __restrict__ P, int S, int tile_base,
                                                           int tiles_m, int tiles_n, int M, int N,
                                                           uint16_t* __restrict__ C, int64_t ldc) {
  constexpr int PER_TILE = T::BM * T::BN / 8 / 256;
  static_assert(PER_TILE * 256 * 8 == T::BM * T::BN, "whole workgroups per tile");
  const int t = blockIdx.x / PER_TILE;
  const int it = (blockIdx.x - t * PER_TILE) * 256 + threadIdx.x;
  const int r = it / (T::BN / 8), c = (it % (T::BN / 8)) * 8;
  int tm, tn;
  tile_order<GM>(tile_base + t, tiles_m, tiles_n, tm, tn);
  const int row = tm * T::BM + r, col = tn * T::BN + c;
  if (row >= M || col >= N) return;
  f32x8 v = {};
  for (int s = 0; s < S; ++s) {
    const f32x4* q = (const f32x4*)(P + ((int64_t)t * S + s) * T::BM * T::BN + r * T::BN + c);
    const f32x4 lo = __builtin_nontemporal_load(q), hi = __builtin_nontemporal_load(q + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] += lo[e];
      v[4 + e] += hi[e];
    }
  }
  *(u32x4*)(C + (int64_t)row * ldc + col) = pack8(v);
}

// ---------------------------------------------------------------------------
// Residual-add epilogue ("Lesson 24", section 24): C = bf16(acc + R), the
// residual R read in the epilogue and added in fp32 before the one rounding,
// so no intermediate GEMM output reaches HBM.  R has C's shape.
// ---------------------------------------------------------------------------
struct EpiStoreResidual {
  // every slab's residual is requested before the first slab is stored:
  // measured 0.04 ms over both residual GEMMs of the 11136x3584x14336 block
  // against 0.11 ms at two slabs ahead
  static constexpr int kPrefetchDepth = 4, kLoadsPerItem = 1;
  struct Params {
    uint16_t* C;
    int64_t ldc;
    const uint16_t* R;
    int64_t ldr;
  };
  template <class T>
  struct Prefetch {
    static constexpr int N = T::SLAB_ROWS * (T::BN / 8) / T::THREADS;
    u32x4 r[N];
  };
  template <class T>
  __device__ static void prefetch_item(const Params& p, const SlabCtx<T>& c, Prefetch<T>& pf, int tid, int k) {
    constexpr int CPR = T::BN / 8;
    const brsrc_t src = rows_rsrc(p.R + (int64_t)c.r0 * p.ldr, (int64_t)(c.M - c.r0) * p.ldr * 2);
    const int ldr = (int)p.ldr;
    const int it = tid + k * T::THREADS;
    const int sr = it / CPR, ch = it % CPR;
    const int col = c.tn * T::BN + ch * 8;
    const uint32_t off = col < c.N ? (uint32_t)((c.row(sr) - c.r0) * ldr + col) * 2u : kOffOutOfRange;
    pf.r[k] = bload16(src, off);
  }
  template <class T, class Hook>
  __device__ static void apply(const Params& p, const SlabCtx<T>& c, Prefetch<T>& pf, int tid, Hook&& hook) {
    constexpr int CPR = T::BN / 8;
    const brsrc_t dst = rows_rsrc(p.C + (int64_t)c.r0 * p.ldc, (int64_t)(c.M - c.r0) * p.ldc * 2);
    const int ldc = (int)p.ldc;
#pragma unroll
    for (int k = 0; k < Prefetch<T>::N; ++k) {
      hook(k);  // this item's share of a later slab's reads, ahead of its stores
      const int it = tid + k * T::THREADS;
      const int sr = it / CPR, ch = it % CPR;
      const int col = c.tn * T::BN + ch * 8;
      const uint32_t off = col < c.N ? (uint32_t)((c.row(sr) - c.r0) * ldc + col) * 2u : kOffOutOfRange;
      f32x8 v = c.read8(sr, ch * 8);
      const f32x8 r = unpack8(pf.r[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += r[e];
      bstore16(dst, off, pack8(v));
    }
  }
};

}  // namespace swg
