// Shared device helpers of the MoE HIP library (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Raw buffer resource over [base, base + bytes): 32-bit offsets, reads past
// the extent return zero. Dword 3 selects the 32-bit data format used for
// untyped buffer access on this architecture.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(Rsrc r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (lo, hi) with the hardware converter (round to
// nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2_t));
}

// Unpack 8 bf16 (one 16-byte vector) to fp32.
__device__ __forceinline__ void unpack_bf16x8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, eight values
// of K each; lanes 0-31 and 32-63 cover the two halves of K. Any fixed
// mapping of actual k to (lane half, element) gives the same product as
// long as A and B use the same one.
// Result: lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4) for
// element i = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(const u32x4& a, const u32x4& b,
                                                const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies row (l % 16) of A / column (l % 16) of B with eight K
// values for lane group l / 16. Result: lane l holds column (l % 16), rows
// 4*(l/16) + i for element i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b,
                                               const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// SiLU(x) = x·sigmoid(x) with the hardware exp and reciprocal (bf16 path).
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ float silu_precise(float x) {
  return x / (1.0f + expf(-x));
}

// Wave-wide sum with a fixed reduction tree (same order every call).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace moe
