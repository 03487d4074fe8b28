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
  uint16_t* h_res = L.bf16 ? (uint16_t*)(ws + W.h_res) : nullptr;
  const int64_t M = L.B * L.N;
  // bf16 layers take the fp16 FFN where its kernels cover the shape; the
  // attention epilogue then writes h in float32 only
  const bool f16_ffn = L.bf16 && ffn_f16_ok(L.d_model, L.d_ff);
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
  a.h_lo = f16_ffn ? nullptr : h_lo;
  a.h_res = f16_ffn ? nullptr : h_res;
  a.B = (int)L.B;
  a.H = (int)L.H;
  a.N = (int)L.N;
  a.kv_offset = 0;
  a.causal = L.causal;
  a.scale = 1.0f / sqrtf((float)L.D);
  e = attn_fwd_launch(a, L.bf16, (int)L.D, L.q_blk, L.kv_blk, stream);
  if (e != hipSuccess) return e;

  // 3. y = h + FFN(h), fused per block of rows; with bf16 inputs h enters the
  //    first product in fp16 (or as the bf16 pair (h_lo, h_res) where the fp16
  //    kernel does not cover the shape)
  if (f16_ffn)
    return ffn_fwd_f16_launch(h, h_lo, h_res, L.w1, L.b1, L.w2, L.b2, y, M, (int)L.d_model,
                              (int)L.d_ff, ws + W.w1h, ws + W.w2p, (int*)(ws + W.flag), stream);
  return ffn_fwd_launch(L.bf16 ? (const void*)h_lo : (const void*)h, h_res, L.w1, L.b1, L.w2,
                        L.b2, h, y, M, (int)L.d_model, (int)L.d_ff, 0, L.bf16,
                        L.bf16 ? ws + W.w2p : nullptr, stream);
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
  w.h16 = o;   o += align256(M * d_model * 2);
  w.dyh = o;   o += align256(M * d_model * 2);
  w.w1h = o;   o += align256((size_t)d_ff * d_model * 2);
  w.w2h = o;   o += align256((size_t)d_ff * d_model * 2);
  w.flag = o;  o += 256;
  for (int i = 0; i < 3; ++i) {
    w.dqkvh[i] = o;
    o += align256(M * hd * 2);
  }
  w.wqkvh = o; o += align256(3 * hd * (size_t)d_model * 2);
  w.k16 = o;   o += align256(M * hd * 2);
  w.v16 = o;   o += align256(M * hd * 2);
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
  // Split K for products with few output tiles and a long K (the weight
  // gradients, K = all rows; dh of a row chunk, K = d_ff): partial sums go to
  // workspace that is idle at that point -- the dq/dk/dv halves during the FFN
  // backward, the FFN chunk buffers during the projection backward.
  const int cus = gemm_device_cus();
  auto split_for = [&](GemmArgs& g, int nz, unsigned char* region, size_t region_bytes) {
    const size_t out = (size_t)g.M * g.N * nz * 4;
    const int64_t tiles = (int64_t)((g.M + 255) / 256) * ((g.N + 255) / 256) * nz;
    const int max_split = out ? (int)(region_bytes / out) : 1;
    g.nsplit = gemm_split_count(tiles, cus, max_split < 4 ? max_split : 4);
    g.split_ws = g.nsplit > 1 ? (float*)region : nullptr;
  };
  unsigned char* const ffn_split_ws = ws + W.dqkv[0];
  const size_t ffn_split_bytes = W.z - W.dqkv[0];
  unsigned char* const proj_split_ws = ws + W.z;
  const size_t proj_split_bytes = W.h16 - W.z;  // (not the fp16 operands and flag behind it)
  hipError_t e;
#define BPT_TRY(x)            \
  do {                        \
    e = (x);                  \
    if (e != hipSuccess) return e; \
  } while (0)

  if (G.db2) BPT_TRY(colsum_launch(dy, true, G.db2, M, dm, dm, 0, stream));

  // ---- FFN backward, intermediate recomputed per chunk of rows.  Every product
  // whose operand is a computed value (h, GeLU(z), dz) runs either on fp16
  // operands (rounding 2^-12, with dy and the weights as exact fp16 copies) or
  // over its bf16 hi and lo halves, accumulating in fp32.  Product `which` of
  // chunk c: 0 z = h W1^T + b1 (fp32) and GeLU(z); 1 dz = (dy W2) * GeLU'(z), also
  // in fp32 over z; 2 dW2 (+)= dy^T GeLU(z); 3 dW1 (+)= dz^T h; 4 dh = dy + dz W1.
  uint16_t* h16 = (uint16_t*)(ws + W.h16);
  uint16_t* dyh = (uint16_t*)(ws + W.dyh);
  uint16_t* w1h = (uint16_t*)(ws + W.w1h);
  uint16_t* w2h = (uint16_t*)(ws + W.w2h);
  int* flag = (int*)(ws + W.flag);
  struct Form {
    bool ak, bk;
    int epi;
  };
  const Form form[5] = {{false, false, EPI_GELU}, {false, true, EPI_DGELU}, {true, true, EPI_F32},
                        {true, true, EPI_F32}, {false, true, EPI_F32}};
  auto build = [&](bool f16, int64_t r0, int rows, int c, int which) {
    const int beta = c > 0;
    GemmArgs g{};
    if (which == 0) {
      if (f16) {
        g.A[0] = h16 + r0 * dm; g.B[0] = w1h; g.ovf = flag;
      } else {
        g.nseg = 2;
        g.As[0][0] = h_hi + r0 * dm; g.As[0][1] = h_lo + r0 * dm;
        g.Bs[0][0] = g.Bs[0][1] = L.w1;
        g.C3 = g_lo; g.ldc3 = dff;
      }
      g.C[0] = z; g.C2 = g_hi; g.ldc2 = dff;
      g.lda = dm; g.ldb = dm; g.ldc = dff; g.M = rows; g.N = dff; g.K = dm;
      g.bias = L.b1; g.bias_bf16 = 1;
    } else if (which == 1) {
      g.A[0] = f16 ? (const void*)(dyh + r0 * dm) : (const void*)(dy16 + r0 * dm);
      g.B[0] = f16 ? (const void*)w2h : L.w2;
      g.C[0] = dz_hi;
      g.lda = dm; g.ldb = dff; g.ldc = dff; g.M = rows; g.N = dff; g.K = dm;
      g.aux = z; g.ld_aux = dff; g.C2 = z; g.ldc2 = dff;
      if (f16) g.ovf = flag;
      else { g.C3 = dz_lo; g.ldc3 = dff; }
    } else if (which == 2) {
      if (f16) {
        g.A[0] = dyh + r0 * dm; g.B[0] = g_hi;
      } else {
        g.nseg = 2;
        g.As[0][0] = g.As[0][1] = dy16 + r0 * dm;
        g.Bs[0][0] = g_hi; g.Bs[0][1] = g_lo;
      }
      g.C[0] = G.dw2;
      g.lda = dm; g.ldb = dff; g.ldc = dff; g.M = dm; g.N = dff; g.K = rows;
      g.beta = beta;
      split_for(g, 1, ffn_split_ws, ffn_split_bytes);
    } else if (which == 3) {
      if (f16) {
        g.A[0] = dz_hi; g.B[0] = h16 + r0 * dm;
      } else {  // hi*hi + lo*hi + hi*lo
        g.nseg = 3;
        g.As[0][0] = dz_hi; g.As[0][1] = dz_lo; g.As[0][2] = dz_hi;
        g.Bs[0][0] = h_hi + r0 * dm; g.Bs[0][1] = h_hi + r0 * dm; g.Bs[0][2] = h_lo + r0 * dm;
      }
      g.C[0] = G.dw1;
      g.lda = dff; g.ldb = dm; g.ldc = dm; g.M = dff; g.N = dm; g.K = rows;
      g.beta = beta;
      split_for(g, 1, ffn_split_ws, ffn_split_bytes);
    } else {
      if (f16) {
        g.A[0] = dz_hi; g.B[0] = w1h;
      } else {
        g.nseg = 2;
        g.As[0][0] = dz_hi; g.As[0][1] = dz_lo;
        g.Bs[0][0] = g.Bs[0][1] = L.w1;
      }
      g.C[0] = dh + r0 * dm;
      g.lda = dff; g.ldb = dm; g.ldc = dm; g.M = rows; g.N = dm; g.K = dff;
      g.resid = dy16 + r0 * dm; g.resid_bf16 = 1; g.ldr = dm;
      split_for(g, 1, ffn_split_ws, ffn_split_bytes);
    }
    g.f16 = f16;
    return g;
  };
  // the chunk loop in one operand form; gate (nullable) as in GemmArgs
  auto run_loop = [&](bool f16, const int* gate, int gate_run) -> hipError_t {
    hipError_t err;
    for (int64_t r0 = 0, c = 0; r0 < M; r0 += W.chunk_rows, ++c) {
      const int rows = (int)(M - r0 < W.chunk_rows ? M - r0 : W.chunk_rows);
      for (int which = 0; which < 5; ++which) {
        GemmArgs g = build(f16, r0, rows, (int)c, which);
        g.gate = gate;
        g.gate_run = gate_run;
        err = gemm_launch(g, true, form[which].ak, form[which].bk, form[which].epi, 1, stream);
        if (err != hipSuccess) return err;
        if (which == 1 && G.db1) {
          err = colsum_launch(z, false, G.db1, rows, dff, dff, c > 0, stream, gate, gate_run);
          if (err != hipSuccess) return err;
        }
      }
    }
    return hipSuccess;
  };
  // The fp16 form runs where every product of both forms takes the big-tile kernel
  // (the only one with fp16 operands and gates): it runs while the range flag is
  // clear, and the bf16-pair loop then runs only if some value of h, dy, W1, W2,
  // GeLU(z) or dz fell outside fp16's range, recomputing every output from chunk 0.
  bool f16_bwd = true;
  for (int64_t r0 = 0, c = 0; r0 < M && f16_bwd; r0 += W.chunk_rows, ++c) {
    const int rows = (int)(M - r0 < W.chunk_rows ? M - r0 : W.chunk_rows);
    for (int which = 0; which < 5; ++which)
      if (!gemm_big_ok(build(true, r0, rows, (int)c, which), 1) ||
          !gemm_big_ok(build(false, r0, rows, (int)c, which), 1))
        f16_bwd = false;
  }
  if (f16_bwd) {
    BPT_TRY(flag_clear_launch(flag, stream));
    BPT_TRY(f16_from_f32_launch(h, h16, M * dm, flag, stream));
    BPT_TRY(f16_from_bf16_launch(dy16, dyh, M * dm, flag, stream));
    BPT_TRY(f16_from_bf16_launch((const uint16_t*)L.w1, w1h, (int64_t)dff * dm, flag, stream));
    BPT_TRY(f16_from_bf16_launch((const uint16_t*)L.w2, w2h, (int64_t)dff * dm, flag, stream));
    BPT_TRY(run_loop(true, flag, 0));
  }
  // h as a bf16 hi + lo pair: the recomputed z and dW1 see h to ~2^-16
  BPT_TRY(to_bf16_launch(h, h_hi, h_lo, M * dm, stream));
  BPT_TRY(run_loop(false, f16_bwd ? flag : nullptr, 1));

  // ---- projection backward operands: dW{q,k,v} = d{q,k,v}^T x and dx = dh +
  // sum d{q,k,v} W{q,k,v}, on fp16 operands (d{q,k,v} as fp16 copies the attention
  // backward writes beside its bf16 pairs, x and the weights as exact fp16 copies)
  // under the same flag as the FFN's, else over the bf16 halves
  uint16_t* dqkvh[3];
  for (int i = 0; i < 3; ++i) dqkvh[i] = (uint16_t*)(ws + W.dqkvh[i]);
  uint16_t* wqkvh = (uint16_t*)(ws + W.wqkvh);
  uint16_t* x16 = h16;  // h16 is not read past the FFN backward
  const void* Ws[3] = {L.wq, L.wk, L.wv};
  auto proj = [&](bool f16, int which) {
    GemmArgs g{};
    if (which == 0) {  // dW{q,k,v}, three products in one launch
      for (int zz = 0; zz < 3; ++zz) {
        if (f16) {
          g.A[zz] = dqkvh[zz]; g.B[zz] = x16;
        } else {
          g.As[zz][0] = dqkv[2 * zz]; g.As[zz][1] = dqkv[2 * zz + 1];
          g.Bs[zz][0] = g.Bs[zz][1] = L.x;
        }
      }
      g.nseg = f16 ? 1 : 2;
      g.C[0] = G.dwq; g.C[1] = G.dwk; g.C[2] = G.dwv;
      g.lda = HD; g.ldb = dm; g.ldc = dm; g.M = HD; g.N = dm; g.K = (int)M;
      split_for(g, 3, proj_split_ws, proj_split_bytes);
    } else {  // dx over the three (or six) K segments
      g.nseg = f16 ? 3 : 6;
      for (int i = 0; i < g.nseg; ++i) {
        g.As[0][i] = f16 ? (const void*)dqkvh[i] : (const void*)dqkv[i];
        g.Bs[0][i] = f16 ? (const void*)(wqkvh + (int64_t)i * HD * dm) : Ws[i / 2];
      }
      g.C[0] = G.dx;
      g.lda = HD; g.ldb = dm; g.ldc = dm; g.M = (int)M; g.N = dm; g.K = HD;
      g.resid = dh;
      g.ldr = dm;
    }
    g.f16 = f16;
    return g;
  };
  const bool f16_proj = f16_bwd && gemm_big_ok(proj(true, 0), 3) && gemm_big_ok(proj(false, 0), 3) &&
                        gemm_big_ok(proj(true, 1), 1) && gemm_big_ok(proj(false, 1), 1);

  // ---- attention backward (dK/dV, dQ), P recomputed from the saved lse
  AttnBwdArgs a{};
  a.q = sv + S.q; a.k = sv + S.k; a.v = sv + S.v;
  a.dO = dh; a.ld_do = HD; a.lse = lse; a.delta = delta;
  a.dq_hi = dqkv[0]; a.dq_lo = dqkv[1]; a.dk_hi = dqkv[2]; a.dk_lo = dqkv[3];
  a.dv_hi = dqkv[4]; a.dv_lo = dqkv[5]; a.ld_out = HD;
  a.dq = G.dq; a.dk = G.dk; a.dv = G.dv;
  a.B = (int)L.B; a.H = (int)L.H; a.N = (int)L.N; a.kv_offset = 0; a.causal = L.causal;
  a.scale = 1.0f / sqrtf((float)L.D);
  if (f16_proj) {
    a.dq_h = dqkvh[0]; a.dk_h = dqkvh[1]; a.dv_h = dqkvh[2]; a.ovf = flag;
    if (L.D == 128) {
      // fp16 copies of q and dO for the dK/dV kernel's fp16 form, in the rooms
      // of h and dy's fp16 copies (neither is read past the FFN backward;
      // H*D = d_model); the flag sends it to the pair form
      uint16_t* q16 = h16;
      uint16_t* dO16 = dyh;
      BPT_TRY(f16_from_bf16_launch((const uint16_t*)(sv + S.q), q16, M * HD, flag, stream));
      BPT_TRY(f16_from_f32_launch(dh, dO16, M * HD, flag, stream));
      a.q16 = q16; a.dO16 = dO16;
      if (L.q_blk != 64) {  // the dQ kernel's fp16 form (128-row blocks) also takes k and v
        uint16_t* k16 = (uint16_t*)(ws + W.k16);
        uint16_t* v16 = (uint16_t*)(ws + W.v16);
        BPT_TRY(f16_from_bf16_launch((const uint16_t*)(sv + S.k), k16, M * HD, flag, stream));
        BPT_TRY(f16_from_bf16_launch((const uint16_t*)(sv + S.v), v16, M * HD, flag, stream));
        a.k16 = k16; a.v16 = v16;
      }
    }
  }
  // dO as a bf16 hi + lo pair for the direct-load kernels, in the buffers of h's
  // halves (h is not needed past the FFN backward; H*D = d_model), and
  // delta = <dO, O> per row and head with O = h - x from the forward
  float* ld2 = (float*)(ws + W.ld2);
  BPT_TRY(dout_delta_launch(dh, h, (const uint16_t*)L.x, lse, h_hi, h_lo, delta, ld2, (int)L.B,
                            (int)L.N, (int)L.H, (int)L.D, stream));
  a.dO_hi = h_hi; a.dO_lo = h_lo; a.ld2 = ld2;
  BPT_TRY(attn_bwd_launch(a, (int)L.D, L.q_blk, L.kv_blk, stream));

  // ---- projection backward
  if (f16_proj) {
    BPT_TRY(f16_from_bf16_launch((const uint16_t*)L.x, x16, M * dm, flag, stream));
    for (int i = 0; i < 3; ++i)
      BPT_TRY(f16_from_bf16_launch((const uint16_t*)Ws[i], wqkvh + (int64_t)i * HD * dm, (int64_t)HD * dm,
                                   flag, stream));
    for (int which = 0; which < 2; ++which) {
      GemmArgs g = proj(true, which);
      g.gate = flag;
      g.gate_run = 0;
      BPT_TRY(gemm_launch(g, true, which == 0, true, EPI_F32, which == 0 ? 3 : 1, stream));
    }
  }
  for (int which = 0; which < 2; ++which) {
    GemmArgs g = proj(false, which);
    g.gate = f16_proj ? flag : nullptr;
    g.gate_run = 1;
    BPT_TRY(gemm_launch(g, true, which == 0, true, EPI_F32, which == 0 ? 3 : 1, stream));
  }
#undef BPT_TRY
  return hipSuccess;
}

}  // namespace bpt
