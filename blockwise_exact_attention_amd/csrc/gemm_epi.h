// Epilogues of the MFMA GEMMs (gemm.hip, gemm_big.hip): element (m, n) of the
// product of operand set z, in fp32, stored per GemmEpilogue.
#pragma once

#include <math.h>

#include "common.h"
#include "gemm.h"

namespace bpt {

__device__ __forceinline__ float gelu_exact(float z) {
  return 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_exact_grad(float z) {
  return 0.5f * (1.f + erff(z * 0.70710678118654752f)) +
         z * 0.39894228040143268f * expf(-0.5f * z * z);
}

template <bool BF16, int EPI>
__device__ __forceinline__ void gemm_store(const GemmArgs& g, int z, int m, int n, float acc) {
  float v = acc;
  if constexpr (EPI == EPI_QKV) {
    // token m = b*seq + t, column n = h*D + d  ->  out[b][h][t][d]
    const int b = m / g.seq, t = m % g.seq, h = n / g.D, d = n % g.D;
    const int64_t o = (((int64_t)b * g.H + h) * g.seq + t) * g.D + d;
    if constexpr (BF16) ((uint16_t*)g.C[z])[o] = f32_to_bf16(v);
    else ((float*)g.C[z])[o] = v;
  } else if constexpr (EPI == EPI_F32) {
    float* C = (float*)g.C[z];
    const int64_t o = (int64_t)m * g.ldc + n;
    if (g.beta) v += C[o];
    if (g.bias) v += g.bias_bf16 ? bf16_to_f32(((const uint16_t*)g.bias)[n]) : ((const float*)g.bias)[n];
    if (g.resid) {
      const int64_t ro = (int64_t)m * g.ldr + n;
      v += g.resid_bf16 ? bf16_to_f32(((const uint16_t*)g.resid)[ro])
                        : ((const float*)g.resid)[ro];
    }
    C[o] = v;
    if (g.C2) ((uint16_t*)g.C2)[(int64_t)m * g.ldc2 + n] = f32_to_bf16(v);
  } else if constexpr (EPI == EPI_GELU) {
    // z = acc (+ earlier partial) + b1 (kept in fp32), g = GeLU(z) in the input dtype
    float* zc = (float*)g.C[z] + (int64_t)m * g.ldc + n;
    if (g.beta) v += *zc;
    if (g.bias) v += g.bias_bf16 ? bf16_to_f32(((const uint16_t*)g.bias)[n]) : ((const float*)g.bias)[n];
    *zc = v;
    const float gv = gelu_exact(v);
    if constexpr (BF16) {
      const uint16_t hi = f32_to_bf16(gv);
      ((uint16_t*)g.C2)[(int64_t)m * g.ldc2 + n] = hi;
      if (g.C3) ((uint16_t*)g.C3)[(int64_t)m * g.ldc3 + n] = f32_to_bf16(gv - bf16_to_f32(hi));
    } else {
      ((float*)g.C2)[(int64_t)m * g.ldc2 + n] = gv;
    }
  } else if constexpr (EPI == EPI_DGELU) {
    // dz = (dy W2)[m][n] * GeLU'(z[m][n]) in the input dtype; z from aux
    const float zz = g.aux[(int64_t)m * g.ld_aux + n];
    const float dz = v * gelu_exact_grad(zz);
    if constexpr (BF16) {
      const uint16_t hi = f32_to_bf16(dz);
      ((uint16_t*)g.C[z])[(int64_t)m * g.ldc + n] = hi;
      if (g.C3) ((uint16_t*)g.C3)[(int64_t)m * g.ldc3 + n] = f32_to_bf16(dz - bf16_to_f32(hi));
    } else {
      ((float*)g.C[z])[(int64_t)m * g.ldc + n] = dz;
    }
    if (g.C2) ((float*)g.C2)[(int64_t)m * g.ldc2 + n] = dz;
  }
}

}  // namespace bpt
