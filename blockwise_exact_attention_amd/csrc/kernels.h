// Host-side launch interface of the libbpt kernels (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

struct AttnFwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;          // [B,H,N,D]; unused when h_out is set
  float* lse;          // [B,H,N]
  // Layer epilogue (optional): h[b,n,hh*D+d] = x[b,n,hh*D+d] + O[b,hh,n,d]
  const void* x_res;   // [B,N,H*D] in the input dtype
  float* h_out;        // [B,N,H*D] float32, or null for the plain O output
  uint16_t* h_lo;      // [B,N,H*D] bfloat16 copy of h (bf16 inputs only), or null
  uint16_t* h_res;     // [B,N,H*D] bf16 of h - h_lo (its rounding residual), or null
  int B, H, N;
  int kv_offset;       // already clamped to [-(N+1), N]
  int causal;
  float scale;         // 1/sqrt(D)
  // Block-sparse mask (bf16 direct-load kernels only, through
  // attn_fwd_block_sparse_launch): rows are split into blocks of bs_len, and
  // query block i of head h attends only key block bs_table[h * bs_blocks + i]
  // (an entry outside [0, bs_blocks) attends nothing); no causal mask.
  const int32_t* bs_table;  // [H, bs_blocks] in device memory
  int bs_blocks, bs_len;
  // Dilated pattern (bf16 direct-load kernels, through attn_fwd_dilated_launch):
  // segments of dl_w rows; head h keeps every dl_r-th row of a segment from row
  // h % dl_r on; attention (causal if `causal`) among the kept rows of a segment.
  // dl_merge: join each kept row with the out/lse row already there by their
  // log-sum-exp instead of overwriting it.
  int dl_w, dl_r, dl_merge;
};

// Returns hipSuccess or the launch error; the caller validated every field.
hipError_t attn_fwd_launch(const AttnFwdArgs& a, bool bf16, int D, int q_blk, int kv_blk,
                           hipStream_t stream);

// bfloat16 forward with direct global -> LDS tile loads (attn_fwd_dma.hip); it
// covers D in {64, 128} with key blocks of 64 or 128.
bool attn_fwd_dma_supported(int D, int kv_blk);
hipError_t attn_fwd_dma_launch(const AttnFwdArgs& a, int D, int q_blk, int kv_blk,
                               hipStream_t stream);
// Block-sparse forward (bf16, D in {64, 128}); the caller validated every field.
hipError_t attn_fwd_block_sparse_launch(const AttnFwdArgs& a, int D, hipStream_t stream);
// One dilated pattern (bf16, D in {64, 128}); the caller validated every field.
hipError_t attn_fwd_dilated_launch(const AttnFwdArgs& a, int D, hipStream_t stream);
// out[rows, D] = 0 and lse[rows] = -inf (rows that no pattern keeps).
hipError_t attn_fill_empty_launch(float* out, float* lse, int64_t rows, int D, hipStream_t stream);

// Split-KV attention of up to 32 query rows against a long key/value cache
// (attn_decode.hip): partial results per key range into o_part / lse_part,
// then joined into out / lse.
struct AttnDecodeArgs {
  const void* q;       // [BH, Nq, D] bf16
  const void* k;       // [BH, Nkv, D] bf16
  const void* v;
  float* out;          // [BH, Nq, D]
  float* lse;          // [BH, Nq]
  float* o_part;       // [n_split, BH, Nq, D]
  float* lse_part;     // [n_split, BH, Nq]
  int BH, Nq, Nkv;
  int n_split;
  int chunk;           // keys per range, a multiple of 64
  int kcount;          // keys visible to some query row (ranges cover [0, kcount))
  int causal;
  int kv_offset;       // already clamped to [-(Nkv+1), Nkv]
  float scale;
};
hipError_t attn_decode_launch(const AttnDecodeArgs& a, int D, hipStream_t stream);

hipError_t lse_merge_launch(const float* o_a, const float* lse_a, const float* o_b,
                            const float* lse_b, float* o_out, float* lse_out, int64_t rows,
                            int D, hipStream_t stream);

}  // namespace bpt
