// Internal helpers shared by the HIP kernels of libvc (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vc.h"

#define VC_DEVICE __device__ __forceinline__

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace vc {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Bit reinterpretation through a by-value scalar: __builtin_bit_cast applied
// directly to an ext_vector element (w[e]) reads element 0 with this clang.
VC_DEVICE float u32_as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }

// bf16 <-> fp32 (exact widening; RNE narrowing via the hardware convert).
VC_DEVICE float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
VC_DEVICE float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
VC_DEVICE float bf16_to_f32(uint16_t h) { return __builtin_bit_cast(float, uint32_t(h) << 16); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two floats -> one packed bf16 pair (RNE) in a single v_cvt_pk_bf16_f32.
VC_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}
// acc + lo + hi of a packed bf16 pair, in one v_dot2 against (1, 1).
VC_DEVICE float sum_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), bf16x2{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}
VC_DEVICE uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
VC_DEVICE float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// IEEE maximum (NaN-propagating): lowers to v_maximum3_f32 without the
// canonicalising v_max that fmaxf needs on MFMA results.
VC_DEVICE float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

VC_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
VC_DEVICE float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wave-wide (64 lanes) reductions through ds_swizzle/bpermute-free DPP where possible.
VC_DEVICE float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
VC_DEVICE float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// The hardware hands workgroups to the eight XCDs round-robin by linear
// index (x fastest).  xcd_order remaps a 2-D grid so that each XCD runs a
// contiguous range of (x, y) in row-major order: neighbouring blocks of x,
// which share cache lines at their boundaries, then go through one L2.
VC_DEVICE void xcd_order(int &x, int &y) {
  const int64_t nx = gridDim.x, total = nx * gridDim.y;
  const int64_t L = (int64_t)blockIdx.y * nx + blockIdx.x;
  const int64_t xcd = L % 8, q = L / 8;
  const int64_t base_n = total / 8, extra = total % 8;   // XCD xcd runs base_n + (xcd < extra) workgroups
  const int64_t v = xcd * base_n + (xcd < extra ? xcd : extra) + q;
  y = (int)(v / nx);
  x = (int)(v % nx);
}

VC_DEVICE f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

VC_DEVICE bf16x8 as_bf16x8(const u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }

}  // namespace vc
