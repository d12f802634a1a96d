// swiglu_math.hpp -- fp32 device math of the SwiGLU activation and bf16 packing.
//
// sigma(g) = 1 / (1 + e^-g) and SiLU(g) = g * sigma(g) are the definitions of
// "Lesson 24: MLP, GEMM and operator fusion in Transformers", section 11.
// silu'(g) uses the third of the three equal forms on the note "SwiGLU MLP
// forward principle, backward chain and optimisation", section 2:
//   silu'(g) = sigma(g) + silu(g) * (1 - sigma(g)).
//
// e^-g is evaluated as 2^(-g * log2 e) with the hardware base-2 exponential
// (v_exp_f32) and the reciprocal with v_rcp_f32.  For g below about -88,
// 2^(...) overflows to +inf and sigma is exactly 0; for large positive g the
// exponential underflows and sigma is exactly 1.  Non-finite g propagates NaN.
//
// Every kernel that computes h (the forward GEMM-1 epilogue, the fused dgrad
// epilogue and the elementwise baseline) calls swiglu_h() on the same bf16
// inputs, so forward and backward h are bitwise identical.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swg {

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sw_sigmoid(float g) {
  const float kLog2e = 1.4426950408889634f;
  float e = __builtin_amdgcn_exp2f(-g * kLog2e);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

struct Act {
  float sigma, silu, dsilu;
};

__device__ __forceinline__ Act sw_act(float g) {
  Act a;
  a.sigma = sw_sigmoid(g);
  a.silu = g * a.sigma;
  a.dsilu = __builtin_fmaf(a.silu, 1.0f - a.sigma, a.sigma);
  return a;
}

// h = left * silu(gate), rounded once to bf16 by the caller.
__device__ __forceinline__ float swiglu_h(float left, float gate) {
  return left * (gate * sw_sigmoid(gate));
}

// ---- bf16 <-> fp32 (round to nearest even on the way down) -----------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// 8 bf16 values (one 16-byte chunk) -> 8 floats
__device__ __forceinline__ f32x8 unpack8(u32x4 v) {
  f32x8 f;
  f[0] = bf16_lo(v[0]); f[1] = bf16_hi(v[0]);
  f[2] = bf16_lo(v[1]); f[3] = bf16_hi(v[1]);
  f[4] = bf16_lo(v[2]); f[5] = bf16_hi(v[2]);
  f[6] = bf16_lo(v[3]); f[7] = bf16_hi(v[3]);
  return f;
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 pack8(f32x8 f) {
  u32x4 v;
  v[0] = pack2(f[0], f[1]);
  v[1] = pack2(f[2], f[3]);
  v[2] = pack2(f[4], f[5]);
  v[3] = pack2(f[6], f[7]);
  return v;
}

// bf16-round each lane value and return it as float (what a bf16 store then
// reload would give)
__device__ __forceinline__ f32x8 round8(f32x8 f) { return unpack8(pack8(f)); }

}  // namespace swg
