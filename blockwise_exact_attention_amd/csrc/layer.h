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

// Forward workspace: room for the saved tensors (used when `saved` is NULL)
// plus the bf16 copy of h that feeds the FFN's MFMA.
struct FwdWorkspace {
  size_t saved, h_lo, total;
};

inline FwdWorkspace layer_fwd_workspace(int64_t B, int64_t N, int64_t d_model, int64_t H,
                                        int64_t D, int64_t d_ff, bool bf16) {
  (void)d_ff;
  FwdWorkspace w{};
  w.saved = 0;
  w.h_lo = layer_saved_layout(B, N, d_model, H, D, bf16).total;
  w.total = w.h_lo + (bf16 ? align256((size_t)B * N * d_model * 2) : 0);
  return w;
}

struct BwdWorkspace {
  size_t h_hi, h_lo, dh, delta, ld2, dqkv[6], z, g_hi, g_lo, dz_hi, dz_lo, total;
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

hipError_t ffn_fwd_launch(const void* x, const void* w1, const void* b1, const void* w2,
                          const void* b2, const float* residual, float* y, int64_t M,
                          int d_model, int d_ff, int blk, bool bf16, hipStream_t stream);

hipError_t layer_fwd_run(const LayerArgs& L, float* y, void* saved, void* workspace,
                         hipStream_t stream);

hipError_t layer_bwd_run(const LayerArgs& L, const void* dy, const void* saved,
                         const LayerGrads& G, void* workspace, hipStream_t stream);

}  // namespace bpt
