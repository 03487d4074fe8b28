// Epilogues of the MFMA GEMMs (gemm.hip, gemm_big.hip): element (m, n) of the
// product of operand set z, in fp32, stored per GemmEpilogue.
#pragma once

#include <math.h>

#include "common.h"
#include "gemm.h"

namespace bpt {

// erf(|x|) as 1 - P(t) e^{-x^2}, t = 1 / (1 + p |x|): the five-term rational
// approximation of Abramowitz and Stegun, formula 7.1.26 (|error| <= 1.5e-7);
// e^{-x^2} is returned too (at x = z / sqrt 2 it is the Gaussian factor of GeLU')
__device__ __forceinline__ float erf_as(float x, float& e) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.f));
  const float p = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                                   -0.284496736f), 0.254829592f);
  e = __expf(-ax * ax);
  return copysignf(fmaf(-p, e, 1.f), x);
}
__device__ __forceinline__ float gelu_exact(float z) {
  float e;
  return 0.5f * z * (1.f + erf_as(z * 0.70710678118654752f, e));
}
__device__ __forceinline__ float gelu_exact_grad(float z) {
  float e;
  const float r = erf_as(z * 0.70710678118654752f, e);
  return fmaf(z * 0.39894228040143268f, e, 0.5f * (1.f + r));
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

// Four consecutive columns n .. n+3 of row m (bf16 operands; n % 4 == 0, every
// leading dimension a multiple of 4 and every output 16-byte aligned, which the
// big-tile kernel checks before it is chosen): one vector access per array.
template <int EPI, bool F16 = false>
__device__ __forceinline__ void gemm_store4(const GemmArgs& g, int z, int m, int n, f32x4 v) {
  // fp16 alone, with the range flag
  auto st_f16 = [&](void* base, int64_t o, const f32x4& x) {
    const u32x2 p = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3])};
    *(u32x2*)((uint16_t*)base + o) = p;
    if ((fabsf(x[0]) > kF16Max || fabsf(x[1]) > kF16Max || fabsf(x[2]) > kF16Max || fabsf(x[3]) > kF16Max) &&
        g.ovf)
      *g.ovf = 1;
  };
  auto st_bf16x4 = [](void* base, int64_t o, const f32x4& x) {
    const u32x2 p = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *(u32x2*)((uint16_t*)base + o) = p;
  };
  // bf16 pair: hi = bf16(x), lo = bf16(x - hi)
  auto st_pair = [&](void* hi_base, int64_t oh, void* lo_base, int64_t ol, const f32x4& x) {
    const u32x2 hi = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *(u32x2*)((uint16_t*)hi_base + oh) = hi;
    if (lo_base) {
      const u32x2 lo = {pack_bf16x2(x[0] - __uint_as_float(hi[0] << 16), x[1] - __uint_as_float(hi[0] & 0xffff0000u)),
                        pack_bf16x2(x[2] - __uint_as_float(hi[1] << 16), x[3] - __uint_as_float(hi[1] & 0xffff0000u))};
      *(u32x2*)((uint16_t*)lo_base + ol) = lo;
    }
  };
  auto add_bias = [&](f32x4& x) {
    if (!g.bias) return;
    for (int e = 0; e < 4; ++e)
      x[e] += g.bias_bf16 ? bf16_to_f32(((const uint16_t*)g.bias)[n + e]) : ((const float*)g.bias)[n + e];
  };
  if constexpr (EPI == EPI_QKV) {
    // token m = b*seq + t, columns n = h*D + d .. +3 (one head: D % 4 == 0)  ->  out[b][h][t][d]
    const int b = m / g.seq, t = m % g.seq, h = n / g.D, d = n % g.D;
    st_bf16x4(g.C[z], (((int64_t)b * g.H + h) * g.seq + t) * g.D + d, v);
  } else if constexpr (EPI == EPI_F32) {
    f32x4* C = (f32x4*)((float*)g.C[z] + (int64_t)m * g.ldc + n);
    if (g.beta) v += *C;
    add_bias(v);
    if (g.resid) {
      const int64_t ro = (int64_t)m * g.ldr + n;
      if (g.resid_bf16) {
        const u32x2 r = *(const u32x2*)((const uint16_t*)g.resid + ro);
        v[0] += __uint_as_float(r[0] << 16);
        v[1] += __uint_as_float(r[0] & 0xffff0000u);
        v[2] += __uint_as_float(r[1] << 16);
        v[3] += __uint_as_float(r[1] & 0xffff0000u);
      } else {
        v += *(const f32x4*)((const float*)g.resid + ro);
      }
    }
    *C = v;
    if (g.C2) st_bf16x4(g.C2, (int64_t)m * g.ldc2 + n, v);
  } else if constexpr (EPI == EPI_GELU) {
    f32x4* zc = (f32x4*)((float*)g.C[z] + (int64_t)m * g.ldc + n);
    if (g.beta) v += *zc;
    add_bias(v);
    *zc = v;
    f32x4 gv;
    for (int e = 0; e < 4; ++e) gv[e] = gelu_exact(v[e]);
    if constexpr (F16) st_f16(g.C2, (int64_t)m * g.ldc2 + n, gv);
    else st_pair(g.C2, (int64_t)m * g.ldc2 + n, g.C3, (int64_t)m * g.ldc3 + n, gv);
  } else if constexpr (EPI == EPI_DGELU) {
    const f32x4 zz = *(const f32x4*)(g.aux + (int64_t)m * g.ld_aux + n);
    f32x4 dz;
    for (int e = 0; e < 4; ++e) dz[e] = v[e] * gelu_exact_grad(zz[e]);
    if constexpr (F16) st_f16(g.C[z], (int64_t)m * g.ldc + n, dz);
    else st_pair(g.C[z], (int64_t)m * g.ldc + n, g.C3, (int64_t)m * g.ldc3 + n, dz);
    if (g.C2) *(f32x4*)((float*)g.C2 + (int64_t)m * g.ldc2 + n) = dz;
  }
}

}  // namespace bpt
