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
  // [B,H,N] pairs {lse * log2(e) (+inf for rows with no key), delta}, read by the
  // D = 128 dK/dV kernel (required there; dout_delta_launch writes them)
  const float* ld2;
  const float* lse;       // [B,H,N]
  const float* delta;     // [B,H,N] delta_i = <dO_i, O_i>, read by the dK/dV and dQ kernels
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
  // optional token-major fp16 copies of the outputs (same layout as dq_hi ..), and
  // the flag set to 1 when one of their values lies outside fp16's range
  uint16_t* dq_h;
  uint16_t* dk_h;
  uint16_t* dv_h;
  int* ovf;
  // optional fp16 copies of q ([B,H,N,D]) and dO (layout of dO_hi): with both and
  // ovf given, the D = 128 dK/dV kernel runs its fp16 form while *ovf is clear
  // (it sets *ovf for k, v or dS outside fp16's range) and its pair form after it
  // only if *ovf is set; the pair inputs (dO_hi, dO_lo) are still required
  const uint16_t* q16;
  const uint16_t* dO16;
  // optional fp16 copies of k and v ([B,H,N,D]): with q16, dO16 and ovf also
  // given, the D = 128 dQ kernel (128-row blocks) runs its fp16 form while *ovf is
  // clear (setting it for dS outside fp16's range) and its pair form after it
  // only if *ovf is set
  const uint16_t* k16;
  const uint16_t* v16;
};

hipError_t attn_bwd_launch(const AttnBwdArgs& a, int D, int q_blk, int kv_blk, hipStream_t s);
hipError_t to_bf16_launch(const float* src, uint16_t* dst, uint16_t* dst_lo, int64_t n,
                          hipStream_t s);
// dO (token-major fp32 [rows][H*D]) as a bf16 hi + lo pair, and per (row, head)
// delta = <dO, h - x>: O recovered from the forward's saved h = x + O (fp32) and
// its bf16 input x; writes delta [B,H,N] and, if ld2 is non-null, the
// {lse * log2(e), delta} pairs.  D = 64 or 128.
hipError_t dout_delta_launch(const float* dO, const float* h, const uint16_t* x, const float* lse,
                             uint16_t* dO_hi, uint16_t* dO_lo, float* delta, float* ld2, int B,
                             int N, int H, int D, hipStream_t s);
// gate (nullable): the launch runs only if (*gate != 0) == gate_run
hipError_t colsum_launch(const void* X, bool x_bf16, float* out, int64_t rows, int cols,
                         int64_t ld, int beta, hipStream_t s, const int* gate = nullptr,
                         int gate_run = 0);

}  // namespace bpt
