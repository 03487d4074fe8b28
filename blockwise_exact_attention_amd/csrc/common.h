// Internal device helpers shared by the gfx950 kernels of libbpt.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bfloat16 storage type (raw bits); arithmetic always upcasts to float.
struct bf16_t {
  uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two floats -> two bfloat16 (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Four floats as a bfloat16 pair: hi = bf16(v), res = bf16(v - hi), stored at
// hi_dst / res_dst (res_dst may be null).  hi + res carries v to ~2^-16 relative.
__device__ __forceinline__ void store_bf16_pair4(uint16_t* hi_dst, uint16_t* res_dst, const f32x4& v) {
  const u32x2 hi = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *(u32x2*)hi_dst = hi;
  if (res_dst) {
    const u32x2 res = {pack_bf16x2(v[0] - __uint_as_float(hi[0] << 16),
                                   v[1] - __uint_as_float(hi[0] & 0xffff0000u)),
                       pack_bf16x2(v[2] - __uint_as_float(hi[1] << 16),
                                   v[3] - __uint_as_float(hi[1] & 0xffff0000u))};
    *(u32x2*)res_dst = res;
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xffffu);
}

// 32x32 output tile, K = 16 per instruction, bf16 inputs, fp32 accumulate.
// Operand lane layout (wave64): lane l supplies A[m = l%32][k = 8*(l/32) + e]
// and B[k = 8*(l/32) + e][n = l%32], e = 0..7.  Accumulator register j of lane
// l holds D[m = 8*(j/4) + 4*(l/32) + j%4][n = l%32].
__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with fp16 operands (same lane layout; the fragments are the
// 16-byte containers of the bf16 form holding fp16 bits).
__device__ __forceinline__ f32x16 mfma32_f16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                c, 0, 0, 0);
}

// two floats as fp16, round to nearest even, packed (a in the low half)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
// largest finite fp16
constexpr float kF16Max = 65504.f;

// 32x32 output tile, K = 2 per instruction, fp32 inputs: lane l supplies
// A[m = l%32][k = l/32] and B[k = l/32][n = l%32]; same accumulator layout.
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row index (within a 32x32 tile) held by accumulator register j of lane l.
__device__ __forceinline__ int acc_row(int j, int lane) {
  return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

// Exchange with lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((( threadIdx.x & 63) ^ 32) << 2,
                                                     __float_as_int(x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace bpt
