// Shared device helpers of libbitdelta (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kWave = 64;

// Four dwords reinterpreted as eight bf16 MFMA operands.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// bf16 bit pattern of a float, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats to packed bf16 (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (lo in bits 0..15), round to nearest even, one
// instruction.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Eight weights of one row: bf16(W_base + alpha*s), s from the sign byte
// (bit j = element j, 1 = +1).  The sign of alpha is flipped by xor for -1:
// bitop3 table 0x78 is a ^ (b & c).
__device__ __forceinline__ u32x4 rebuild8(u32x4 w, uint32_t byte, uint32_t ab) {
  const uint32_t nb = ~byte;
  u32x4 out;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = __uint_as_float(w[d] << 16);
    const float hi = __uint_as_float(w[d] & 0xFFFF0000u);
    const float slo =
        __uint_as_float(__builtin_amdgcn_bitop3_b32(ab, nb << (31 - 2 * d), 0x80000000u, 0x78));
    const float shi =
        __uint_as_float(__builtin_amdgcn_bitop3_b32(ab, nb << (30 - 2 * d), 0x80000000u, 0x78));
    out[d] = cvt_pk_bf16(lo + slo, hi + shi);
  }
  return out;
}

// Global loads that bypass nothing special but keep the 128-bit width explicit.
__device__ __forceinline__ u32x4 ld128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ uint32_t ld32(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

// Buffer loads through a resource spanning [base, base + nbytes): offsets
// past the end read as zero.
__device__ __forceinline__ u32x4 bload128(const void* base, int nbytes, int voff, int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ uint32_t bload32(const void* base, int nbytes, int voff, int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

__device__ __forceinline__ uint32_t bload8(const void* base, int nbytes, int voff, int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// 16 bytes per lane through a buffer resource straight into LDS: lane i's
// bytes land at lds + 16*i (lds must be the same for the whole wave).  A
// buffer load rather than a global one: the compiler then counts these loads
// in order with the weight loads and can wait for exactly the ones a step
// needs (with global-to-LDS loads pending it falls back to waiting for all).
__device__ __forceinline__ void lds_bload16(const void* base, int nbytes, int voff, int soff,
                                            void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

}  // namespace bd
