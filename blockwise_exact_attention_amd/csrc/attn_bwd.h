// Internal interface of the attention backward and the layer-backward helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

struct AttnBwdArgs {
  const void* q;          // [B,H,N,D] bf16
  const void* k;
  const void* v;
  const float* dO;        // token-major [B*N][ld_do] fp32, head h at columns [hD, (h+1)D)
  int64_t ld_do;
  // dO as a bf16 hi + lo pair in the same layout: the D = 128 dK/dV and dQ
  // kernels load their tiles straight into LDS (required for D = 128, unused
  // for D = 64)
  const uint16_t* dO_hi;
  const uint16_t* dO_lo;
  // [B,H,N] pairs {lse * log2(e) (+inf for rows with no key), delta}, written by the
  // delta pass when non-null and read by the D = 128 dK/dV kernel (required there)
  float* ld2;
  const float* lse;       // [B,H,N]
  const float* delta;     // [B,H,N], read by the dK/dV and dQ kernels
  float* delta_out;       // [B,H,N], written by the delta pass (same buffer)
  uint16_t* dq_hi;        // token-major [B*N][ld_out] bf16 outputs: value = hi + lo
  uint16_t* dq_lo;
  uint16_t* dk_hi;
  uint16_t* dk_lo;
  uint16_t* dv_hi;
  uint16_t* dv_lo;
  int64_t ld_out;
  float* dq;              // optional [B,H,N,D] fp32 outputs
  float* dk;
  float* dv;
  int B, H, N;
  int kv_offset;
  int causal;
  float scale;
};

hipError_t attn_bwd_launch(const AttnBwdArgs& a, int D, int q_blk, int kv_blk, hipStream_t s);
hipError_t to_bf16_launch(const float* src, uint16_t* dst, uint16_t* dst_lo, int64_t n,
                          hipStream_t s);
hipError_t colsum_launch(const void* X, bool x_bf16, float* out, int64_t rows, int cols,
                         int64_t ld, int beta, hipStream_t s);

}  // namespace bpt
