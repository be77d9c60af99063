// Device-side helpers shared by the libtq kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "tq_internal.h"

namespace tq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

__device__ __forceinline__ float load_elem(const void* p, int dtype, int64_t i) {
  return dtype == 1 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// --------------------------------------------------------------------------
// OCP FP8 E4M3 (bias 7, max 448, subnormal step 2^-9), round to nearest even.
// Used to split query-side operands into limbs; decode is exact so each
// residual is exact in float.
// --------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e == 0 ? ldexpf(static_cast<float>(m), -9) : ldexpf(static_cast<float>(8u + m), static_cast<int>(e) - 10);
  return (b & 0x80u) ? -v : v;
}

__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t sign = x < 0.f ? 0x80u : 0u;
  float a = fabsf(x);
  if (!(a > 0.f)) return 0u;
  if (a >= 448.f) return sign | 0x7Eu;
  int ex;
  frexpf(a, &ex);              // a = f * 2^ex, f in [0.5, 1)
  int e = ex - 1 + 7;           // biased exponent of a
  uint32_t code;
  if (e <= 0) {                 // subnormal: step 2^-9
    float q = rintf(ldexpf(a, 9));   // round half to even
    code = static_cast<uint32_t>(q); // 0..8 (8 == min normal 2^-6)
  } else {
    float q = rintf(ldexpf(a, 3 - (ex - 1)));   // mantissa with 3 fraction bits, in [8, 16]
    uint32_t mq = static_cast<uint32_t>(q);
    if (mq == 16u) { mq = 8u; ++e; }
    code = (static_cast<uint32_t>(e) << 3) | (mq - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Limb k (k = 0..3) of x: x ~ sum_k 2^(-4k) limb_k with limb values fp8.
__device__ __forceinline__ uint32_t e4m3_limb(float x, int k) {
  float r = x;
  uint32_t b = e4m3_encode(r);
  for (int i = 0; i < k; ++i) {
    r = (r - e4m3_value(b)) * 16.f;
    b = e4m3_encode(r);
  }
  return b;
}

// --------------------------------------------------------------------------
// A 32-bit word of bits (one bit per coordinate or per token) as the fp4
// (E2M1) B operand of the 16x16x128 f8f6f4 MFMA: 4 dwords of 8 nibbles.
// Dword s holds bit 4i+s of w in nibble i (value 0.5 / 1 / 2 / 2 for
// s = 0 / 1 / 2 / 3).  B lane-group g holds K = 32g .. 32g+31 with element
// e = 8s+i in dword s, nibble i, so element e <-> bit 4*(e%8) + e/8.
// --------------------------------------------------------------------------
__device__ __forceinline__ v8i bits_to_fp4(uint32_t w) {
  v8i b = {static_cast<int>(w & 0x11111111u), static_cast<int>(w & 0x22222222u), static_cast<int>(w & 0x44444444u),
           static_cast<int>((w >> 1) & 0x44444444u), 0, 0, 0, 0};
  return b;
}

// The codebook of b' index bits is symmetric, so its centroids expand over
// the odd Walsh functions of the bits: c[idx] = sum_t coef_t (2 x_t - 1) with
// x_t the XOR of the index bits in mask t.  Word t of a packed group is that
// XOR taken over 32 coordinates at once (masks in the host's coefficient
// order).
template <int BP>
__device__ __forceinline__ uint32_t walsh_word(const uint32_t (&w)[5], int t) {
  constexpr int masks[4][8] = {{1}, {1, 2}, {1, 2, 4, 7}, {1, 2, 4, 8, 7, 11, 13, 14}};
  const int mk = masks[BP - 1][t];
  uint32_t r = 0u;
#pragma unroll
  for (int p = 0; p < BP; ++p)
    if (mk & (1 << p)) r ^= w[p];
  return r;
}

// value of a set bit at element slot s = (K % 32) / 8
__host__ __device__ __forceinline__ float fp4_slot_value(int s) { return s == 0 ? 0.5f : (s == 1 ? 1.f : 2.f); }

// bit position inside the 32-bit word for MFMA K index within a 128 chunk
__host__ __device__ __forceinline__ int k_to_bit(int k) { return 4 * (k & 7) + ((k & 31) >> 3); }

// K index of fp8 A operand element e held by lane-group g (16x16x128)
__host__ __device__ __forceinline__ int a_elem_to_k(int g, int e) { return 16 * g + (e & 15) + 64 * (e >> 4); }

__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, 127);
}

// An MFMA reads the operand registers of all 64 lanes.  Code whose result is
// only consumed under a lane-divergent condition may be moved by the compiler
// into that condition, where inactive lanes would feed stale operands.  This
// empty asm marks the value as used in converged control flow.
__device__ __forceinline__ void pin(v4f& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ v4f mfma_f32(float a, float b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace tq
