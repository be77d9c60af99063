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

// The same for key bits (logits, top-k and attention logits), one
// instruction cheaper: dword 3 keeps bit 4i+3 where it is, as the sign of
// 1.0 (nibble 0x2 or 0xA), so that slot's value is 1 - 2 bit.  The query
// side takes the slot's A operand negated and halved and leaves those
// coordinates out of its constant term (key_slot_value).
__device__ __forceinline__ v8i key_bits_to_fp4(uint32_t w) {
  // the 1.0 pattern lives in a vector register (an empty asm hides its
  // value), so that mask-and-or is one v_and_or_b32: with both constants
  // scalar it would break the one-scalar-operand limit and split in two
  uint32_t one = 0x22222222u;
  asm("" : "+v"(one));
  v8i b = {static_cast<int>(w & 0x11111111u), static_cast<int>(w & 0x22222222u), static_cast<int>(w & 0x44444444u),
           static_cast<int>((w & 0x88888888u) | one), 0, 0, 0, 0};
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

// Wave-wide reductions over all 64 lanes without the LDS permute path: DPP
// within rows of 16 (quad swaps, then row rotations by 4 and 8), then the
// four row results through scalar reads.  Every lane must be active; the
// result is uniform.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);   // row_ror:4
  v += dpp_f<0x128>(v);   // row_ror:8
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  return v;
}
__device__ __forceinline__ float row_min16(float v) {
  v = fminf(v, dpp_f<0xB1>(v));
  v = fminf(v, dpp_f<0x4E>(v));
  v = fminf(v, dpp_f<0x124>(v));
  v = fminf(v, dpp_f<0x128>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// s_waitcnt immediate that waits for vmcnt <= N only (gfx9 encoding; the
// counter retires vector-memory operations in issue order)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ __forceinline__ void wait_vm_upto(int n) {   // runtime n in [0, N]
  if constexpr (N > 0) {
    if (n >= N) { wait_vm<N>(); return; }
    wait_vm_upto<N - 1>(n);
  } else {
    wait_vm<0>();
  }
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// LDS destination of the global -> LDS DMA loads
typedef __attribute__((address_space(3))) void lds_ptr_t;
__device__ __forceinline__ lds_ptr_t* as_lds(const void* p) {
  return reinterpret_cast<lds_ptr_t*>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}

// floor(log2 x) for finite x > 0 (normal or subnormal), from the exponent
// field the hardware extracts (x = m 2^e with m in [0.5, 1))
__device__ __forceinline__ int ilogb_pos(float x) { return __builtin_amdgcn_frexp_expf(x) - 1; }

// value of a set bit at element slot s = (K % 32) / 8
__host__ __device__ __forceinline__ float fp4_slot_value(int s) { return s == 0 ? 0.5f : (s == 1 ? 1.f : 2.f); }
// The divisor of a key-side A operand element at slot s: a set bit gives
// 0.5 / 1 / 2 at slots 0-2; slot 3 gives 1 - 2 bit, so with the element
// divided by -2 its product is (value) bit - (value) / 2, the constant half
// of the Walsh term's 2 bit - 1 included.
__host__ __device__ __forceinline__ float key_slot_value(int s) { return s == 3 ? -2.f : fp4_slot_value(s); }
// coordinate j of a 32-coordinate word sits in slot j % 4 (bit 4i + s)
__host__ __device__ __forceinline__ bool key_slot3_coord(int j) { return (j & 3) == 3; }

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
