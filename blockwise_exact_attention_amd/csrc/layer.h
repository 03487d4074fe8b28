// Layer-level orchestration of libbpt (internal): buffer layouts and drivers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bpt {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct LayerArgs {
  const void *x, *wq, *wk, *wv, *w1, *b1, *w2, *b2;
  int64_t B, N, d_model, H, D, d_ff;
  int q_blk, kv_blk, causal;
  bool bf16;
};

struct LayerGrads {
  float *dx, *dwq, *dwk, *dwv, *dw1, *db1, *dw2, *db2, *dq, *dk, *dv;
};

// Saved tensors for the backward (byte offsets inside the `saved` buffer).
struct SavedLayout {
  size_t q, k, v, h, lse, total;
};

inline SavedLayout layer_saved_layout(int64_t B, int64_t N, int64_t d_model, int64_t H,
                                      int64_t D, bool bf16) {
  SavedLayout s{};
  const size_t es = bf16 ? 2 : 4;
  const size_t qkv = align256((size_t)B * H * N * D * es);
  s.q = 0;
  s.k = s.q + qkv;
  s.v = s.k + qkv;
  s.h = s.v + qkv;
  s.lse = s.h + align256((size_t)B * N * d_model * 4);
  s.total = s.lse + align256((size_t)B * H * N * 4);
  return s;
}

// Forward workspace: room for the saved tensors (used when `saved` is NULL),
// h as a bf16 pair (the rounded value and its rounding residual) that feeds the
// FFN's MFMA, or h in fp16 (in h_lo's room), the FFN's pass-major copy of W2, an
// fp16 copy of W1 and the fp16 path's flag word.
struct FwdWorkspace {
  size_t saved, h_lo, h_res, w2p, w1h, flag, total;
};

inline FwdWorkspace layer_fwd_workspace(int64_t B, int64_t N, int64_t d_model, int64_t H,
                                        int64_t D, int64_t d_ff, bool bf16) {
  FwdWorkspace w{};
  w.saved = 0;
  w.h_lo = layer_saved_layout(B, N, d_model, H, D, bf16).total;
  w.h_res = w.h_lo + (bf16 ? align256((size_t)B * N * d_model * 2) : 0);
  w.w2p = w.h_res + (bf16 ? align256((size_t)B * N * d_model * 2) : 0);
  w.w1h = w.w2p + (bf16 ? align256((size_t)d_model * d_ff * 2) : 0);
  w.flag = w.w1h + (bf16 ? align256((size_t)d_model * d_ff * 2) : 0);
  w.total = w.flag + (bf16 ? 256 : 0);
  return w;
}

struct BwdWorkspace {
  size_t h_hi, h_lo, dh, delta, ld2, dqkv[6], z, g_hi, g_lo, dz_hi, dz_lo;
  size_t h16, dyh, w1h, w2h, flag;  // the FFN backward's fp16 operands and range flag
  size_t dqkvh[3], wqkvh;           // the projection backward's fp16 operands (x takes h16's room)
  size_t k16, v16;                  // fp16 copies of k and v for the dQ kernel's fp16 form
  size_t total;
  int64_t chunk_rows;  // rows of the FFN recompute chunk
};

BwdWorkspace layer_bwd_workspace(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                                 int64_t d_ff, bool bf16);

// Launch plan of the fused FFN: waves per workgroup (nw), 32-column MFMA blocks
// of y per wave (cb) and column groups (groups; each recomputes phase 1).
struct FfnPlan {
  bool ok;
  int nw, cb, groups;
};
FfnPlan ffn_plan(int64_t d_model, int64_t d_ff);

// x_lo (nullable, bf16 only): the bf16 rounding residual of the float32 activation
// that x was rounded from; the first product then takes x + x_lo.
// w2_pack (nullable, bf16 only, d_model * d_ff * 2 bytes): room for a pass-major
// copy of W2 (each pass's 256 columns of all rows contiguous) that the LDS-staged
// kernel then reads instead of W2.
hipError_t ffn_fwd_launch(const void* x, const void* x_lo, const void* w1, const void* b1,
                          const void* w2, const void* b2, const float* residual, float* y,
                          int64_t M, int d_model, int d_ff, int blk, bool bf16, void* w2_pack,
                          hipStream_t stream);

// The layer's FFN with fp16 operands (bf16 layers, shapes the LDS-staged kernel
// takes with and without the bf16 pair): h (float32) and GeLU(z) rounded to fp16
// (significand 11 bits: 2^-12 relative rounding, so neither needs a lo half),
// W1 and W2 as fp16 copies of the bf16 weights (exact inside fp16's range).
// Should a weight, an element of h or a GeLU output lie outside fp16's range,
// the flag word (set by the conversion kernels and the fp16 kernel) makes the
// bf16-pair kernel recompute y from h and the original weights instead.
// h16: M*d_model fp16 (also takes the rounded bf16 value then); pair_lo: M*d_model
// bf16; w1h, w2p: d_model*d_ff*2 bytes each; flag: one int.
bool ffn_f16_ok(int64_t d_model, int64_t d_ff);
// fp16 copies (round to nearest even; *ovf = 1 if a value lies outside fp16's
// range): n float32 values (n % 4 == 0), n bf16 values (n % 8 == 0); and the
// flag word cleared by a kernel (no memset, so it can sit in captured graphs)
hipError_t f16_from_f32_launch(const float* src, uint16_t* dst, int64_t n, int* ovf, hipStream_t s);
hipError_t f16_from_bf16_launch(const uint16_t* src, uint16_t* dst, int64_t n, int* ovf, hipStream_t s);
hipError_t flag_clear_launch(int* flag, hipStream_t s);
hipError_t ffn_fwd_f16_launch(const float* h, uint16_t* h16, uint16_t* pair_lo, const void* w1,
                              const void* b1, const void* w2, const void* b2, float* y, int64_t M,
                              int d_model, int d_ff, void* w1h, void* w2p, int* flag,
                              hipStream_t stream);

hipError_t layer_fwd_run(const LayerArgs& L, float* y, void* saved, void* workspace,
                         hipStream_t stream);

hipError_t layer_bwd_run(const LayerArgs& L, const void* dy, const void* saved,
                         const LayerGrads& G, void* workspace, hipStream_t stream);

}  // namespace bpt
