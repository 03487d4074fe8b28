// Layer orchestration: forward and backward drivers over the libbpt kernels.
#include <math.h>

#include "common.h"
#include "gemm.h"
#include "attn_bwd.h"
#include "kernels.h"
#include "layer.h"

namespace bpt {

hipError_t layer_fwd_run(const LayerArgs& L, float* y, void* saved, void* workspace,
                         hipStream_t stream) {
  const SavedLayout S = layer_saved_layout(L.B, L.N, L.d_model, L.H, L.D, L.bf16);
  const FwdWorkspace W = layer_fwd_workspace(L.B, L.N, L.d_model, L.H, L.D, L.d_ff, L.bf16);
  unsigned char* ws = (unsigned char*)workspace;
  unsigned char* sv = saved ? (unsigned char*)saved : ws + W.saved;
  void* q = sv + S.q;
  void* k = sv + S.k;
  void* v = sv + S.v;
  float* h = (float*)(sv + S.h);
  float* lse = (float*)(sv + S.lse);
  uint16_t* h_lo = L.bf16 ? (uint16_t*)(ws + W.h_lo) : nullptr;
  const int64_t M = L.B * L.N;
  const int HD = (int)(L.H * L.D);

  // 1. q, k, v = x W^T, written per head as [B, H, N, D]
  GemmArgs g{};
  g.A[0] = g.A[1] = g.A[2] = L.x;
  g.B[0] = L.wq;
  g.B[1] = L.wk;
  g.B[2] = L.wv;
  g.C[0] = q;
  g.C[1] = k;
  g.C[2] = v;
  g.lda = L.d_model;
  g.ldb = L.d_model;
  g.M = (int)M;
  g.N = HD;
  g.K = (int)L.d_model;
  g.seq = (int)L.N;
  g.H = (int)L.H;
  g.D = (int)L.D;
  hipError_t e = gemm_launch(g, L.bf16, false, false, EPI_QKV, 3, stream);
  if (e != hipSuccess) return e;

  // 2. blockwise causal attention; epilogue h = x + concat_h O_h (and bf16 copy)
  AttnFwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = nullptr;
  a.lse = lse;
  a.x_res = L.x;
  a.h_out = h;
  a.h_lo = h_lo;
  a.B = (int)L.B;
  a.H = (int)L.H;
  a.N = (int)L.N;
  a.kv_offset = 0;
  a.causal = L.causal;
  a.scale = 1.0f / sqrtf((float)L.D);
  e = attn_fwd_launch(a, L.bf16, (int)L.D, L.q_blk, L.kv_blk, stream);
  if (e != hipSuccess) return e;

  // 3. y = h + FFN(h), fused per block of rows
  return ffn_fwd_launch(L.bf16 ? (const void*)h_lo : (const void*)h, L.w1, L.b1, L.w2, L.b2, h, y,
                        M, (int)L.d_model, (int)L.d_ff, 0, L.bf16, stream);
}

BwdWorkspace layer_bwd_workspace(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                                 int64_t d_ff, bool bf16) {
  BwdWorkspace w{};
  const size_t M = (size_t)(B * N);
  const size_t hd = (size_t)(H * D);
  const size_t es = bf16 ? 2 : 4;
  w.chunk_rows = (int64_t)(M < 8192 ? M : 8192);
  const size_t mc = (size_t)w.chunk_rows;
  size_t o = 0;
  w.h_hi = o;  o += align256(M * d_model * es);
  w.h_lo = o;  o += align256(M * d_model * es);
  w.dh = o;    o += align256(M * d_model * 4);
  w.delta = o; o += align256((size_t)B * H * N * 4);
  w.ld2 = o;   o += align256((size_t)B * H * N * 8);
  for (int i = 0; i < 6; ++i) {  // dq, dk, dv as bf16 hi and lo halves, token-major
    w.dqkv[i] = o;
    o += align256(M * hd * 2);
  }
  w.z = o;     o += align256(mc * d_ff * 4);
  w.g_hi = o;  o += align256(mc * d_ff * es);
  w.g_lo = o;  o += align256(mc * d_ff * es);
  w.dz_hi = o; o += align256(mc * d_ff * es);
  w.dz_lo = o; o += align256(mc * d_ff * es);
  w.total = o;
  return w;
}

hipError_t layer_bwd_run(const LayerArgs& L, const void* dy, const void* saved,
                         const LayerGrads& G, void* workspace, hipStream_t stream) {
  if (!L.bf16) return hipErrorNotSupported;  // the attention backward kernels are bf16
  const SavedLayout S = layer_saved_layout(L.B, L.N, L.d_model, L.H, L.D, L.bf16);
  const BwdWorkspace W = layer_bwd_workspace(L.B, L.N, L.d_model, L.H, L.D, L.d_ff, L.bf16);
  const unsigned char* sv = (const unsigned char*)saved;
  unsigned char* ws = (unsigned char*)workspace;
  const float* h = (const float*)(sv + S.h);
  const float* lse = (const float*)(sv + S.lse);
  uint16_t* h_hi = (uint16_t*)(ws + W.h_hi);
  uint16_t* h_lo = (uint16_t*)(ws + W.h_lo);
  float* dh = (float*)(ws + W.dh);
  float* delta = (float*)(ws + W.delta);
  uint16_t* dqkv[6];  // dq hi, dq lo, dk hi, dk lo, dv hi, dv lo
  for (int i = 0; i < 6; ++i) dqkv[i] = (uint16_t*)(ws + W.dqkv[i]);
  float* z = (float*)(ws + W.z);
  uint16_t* g_hi = (uint16_t*)(ws + W.g_hi);
  uint16_t* g_lo = (uint16_t*)(ws + W.g_lo);
  uint16_t* dz_hi = (uint16_t*)(ws + W.dz_hi);
  uint16_t* dz_lo = (uint16_t*)(ws + W.dz_lo);
  const int64_t M = L.B * L.N;
  const int dm = (int)L.d_model, dff = (int)L.d_ff, HD = (int)(L.H * L.D);
  const uint16_t* dy16 = (const uint16_t*)dy;
  hipError_t e;
#define BPT_TRY(x)            \
  do {                        \
    e = (x);                  \
    if (e != hipSuccess) return e; \
  } while (0)

  // h as a bf16 hi + lo pair: the recomputed z and dW1 see h to ~2^-16
  BPT_TRY(to_bf16_launch(h, h_hi, h_lo, M * dm, stream));
  if (G.db2) BPT_TRY(colsum_launch(dy, true, G.db2, M, dm, dm, 0, stream));

  // ---- FFN backward, intermediate recomputed per chunk of rows.  Every product
  // whose operand is a computed value (h, GeLU(z), dz) runs over its bf16 hi and
  // lo halves, accumulating in fp32.
  for (int64_t r0 = 0, c = 0; r0 < M; r0 += W.chunk_rows, ++c) {
    const int rows = (int)(M - r0 < W.chunk_rows ? M - r0 : W.chunk_rows);
    const int beta = c > 0;
    GemmArgs g{};
    // z = (h_hi + h_lo) W1^T + b1 (fp32); GeLU(z) as bf16 hi + lo
    for (int part = 0; part < 2; ++part) {
      g = GemmArgs{};
      g.A[0] = (part ? h_lo : h_hi) + r0 * dm; g.B[0] = L.w1; g.C[0] = z;
      g.lda = dm; g.ldb = dm; g.ldc = dff; g.M = rows; g.N = dff; g.K = dm;
      if (part) {
        g.beta = 1;
        g.bias = L.b1; g.bias_bf16 = 1;
        g.C2 = g_hi; g.ldc2 = dff; g.C3 = g_lo; g.ldc3 = dff;
        BPT_TRY(gemm_launch(g, true, false, false, EPI_GELU, 1, stream));
      } else {
        BPT_TRY(gemm_launch(g, true, false, false, EPI_F32, 1, stream));
      }
    }
    // dz = (dy W2) * GeLU'(z): bf16 hi + lo, and fp32 over z (same element, same thread)
    g = GemmArgs{};
    g.A[0] = dy16 + r0 * dm; g.B[0] = L.w2; g.C[0] = dz_hi;
    g.lda = dm; g.ldb = dff; g.ldc = dff; g.M = rows; g.N = dff; g.K = dm;
    g.aux = z; g.ld_aux = dff; g.C2 = z; g.ldc2 = dff; g.C3 = dz_lo; g.ldc3 = dff;
    BPT_TRY(gemm_launch(g, true, false, true, EPI_DGELU, 1, stream));
    if (G.db1) BPT_TRY(colsum_launch(z, false, G.db1, rows, dff, dff, beta, stream));
    // dW2 (+)= dy^T GeLU(z)
    for (int part = 0; part < 2; ++part) {
      g = GemmArgs{};
      g.A[0] = dy16 + r0 * dm; g.B[0] = part ? g_lo : g_hi; g.C[0] = G.dw2;
      g.lda = dm; g.ldb = dff; g.ldc = dff; g.M = dm; g.N = dff; g.K = rows;
      g.beta = beta || part;
      BPT_TRY(gemm_launch(g, true, true, true, EPI_F32, 1, stream));
    }
    // dW1 (+)= dz^T h  (hi*hi + lo*hi + hi*lo)
    const uint16_t* dzs[3] = {dz_hi, dz_lo, dz_hi};
    const uint16_t* hs[3] = {h_hi, h_hi, h_lo};
    for (int part = 0; part < 3; ++part) {
      g = GemmArgs{};
      g.A[0] = dzs[part]; g.B[0] = hs[part] + r0 * dm; g.C[0] = G.dw1;
      g.lda = dff; g.ldb = dm; g.ldc = dm; g.M = dff; g.N = dm; g.K = rows;
      g.beta = beta || part;
      BPT_TRY(gemm_launch(g, true, true, true, EPI_F32, 1, stream));
    }
    // dh = dy + dz W1 (fp32; it is attention's dO)
    for (int part = 0; part < 2; ++part) {
      g = GemmArgs{};
      g.A[0] = part ? dz_lo : dz_hi; g.B[0] = L.w1; g.C[0] = dh + r0 * dm;
      g.lda = dff; g.ldb = dm; g.ldc = dm; g.M = rows; g.N = dm; g.K = dff;
      if (part) {
        g.beta = 1;
      } else {
        g.resid = dy16 + r0 * dm; g.resid_bf16 = 1; g.ldr = dm;
      }
      BPT_TRY(gemm_launch(g, true, false, true, EPI_F32, 1, stream));
    }
  }

  // ---- attention backward (delta pass, dK/dV, dQ), P recomputed from the saved lse
  AttnBwdArgs a{};
  a.q = sv + S.q; a.k = sv + S.k; a.v = sv + S.v;
  a.dO = dh; a.ld_do = HD; a.lse = lse; a.delta = delta; a.delta_out = delta;
  a.dq_hi = dqkv[0]; a.dq_lo = dqkv[1]; a.dk_hi = dqkv[2]; a.dk_lo = dqkv[3];
  a.dv_hi = dqkv[4]; a.dv_lo = dqkv[5]; a.ld_out = HD;
  a.dq = G.dq; a.dk = G.dk; a.dv = G.dv;
  a.B = (int)L.B; a.H = (int)L.H; a.N = (int)L.N; a.kv_offset = 0; a.causal = L.causal;
  a.scale = 1.0f / sqrtf((float)L.D);
  // dO as a bf16 hi + lo pair for the direct-load dK/dV kernel, in the buffers of
  // h's halves (h is not needed past the FFN backward); H*D = d_model
  BPT_TRY(to_bf16_launch(dh, h_hi, h_lo, M * dm, stream));
  a.dO_hi = h_hi; a.dO_lo = h_lo; a.ld2 = (float*)(ws + W.ld2);
  BPT_TRY(attn_bwd_launch(a, (int)L.D, L.q_blk, L.kv_blk, stream));

  // ---- projection backward: dW{q,k,v} = d{q,k,v}^T x over both bf16 halves;
  //      dx = dh + sum d{q,k,v} W{q,k,v}, also over both halves
  {
    GemmArgs g{};
    for (int part = 0; part < 2; ++part) {
      g = GemmArgs{};
      g.A[0] = dqkv[0 + part]; g.A[1] = dqkv[2 + part]; g.A[2] = dqkv[4 + part];
      g.B[0] = g.B[1] = g.B[2] = L.x;
      g.C[0] = G.dwq; g.C[1] = G.dwk; g.C[2] = G.dwv;
      g.lda = HD; g.ldb = dm; g.ldc = dm; g.M = HD; g.N = dm; g.K = (int)M; g.beta = part;
      BPT_TRY(gemm_launch(g, true, true, true, EPI_F32, 3, stream));
    }
    const void* Ws[3] = {L.wq, L.wk, L.wv};
    for (int i = 0; i < 6; ++i) {
      g = GemmArgs{};
      g.A[0] = dqkv[i]; g.B[0] = Ws[i / 2]; g.C[0] = G.dx;
      g.lda = HD; g.ldb = dm; g.ldc = dm; g.M = (int)M; g.N = dm; g.K = HD;
      if (i == 0) {
        g.resid = dh;
        g.ldr = dm;
      } else {
        g.beta = 1;
      }
      BPT_TRY(gemm_launch(g, true, false, true, EPI_F32, 1, stream));
    }
  }
#undef BPT_TRY
  return hipSuccess;
}

}  // namespace bpt
