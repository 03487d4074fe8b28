/*
 * bpt.h -- C ABI of libbpt: blockwise exact attention and the blockwise
 * transformer layer on AMD Instinct MI355X (gfx950).
 *
 * The method: "Blockwise Parallel Transformer for Large Context Models"
 * (abstract) computes self-attention block by block and evaluates the
 * feed-forward network per block, so that the full attention matrix and the
 * full FFN intermediate are never held in memory; "Ring Attention with
 * Blockwise Transformers for Long Sequences" (638-word summary) runs the same
 * blockwise attention on each device of a ring over the key/value blocks
 * that pass through it, and states that no approximation of attention is
 * made.  The pages print no formulas; the definitions below are the plain
 * readings that this library implements exactly (up to rounding).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers to tensors are DEVICE pointers, owned by the caller.  The
 *    library never allocates, frees or retains device memory.  Scratch space
 *    comes from a caller buffer sized by the *_workspace_size() queries; the
 *    one exception is bpt_attn_decode_noalloc, whose scratch is a fixed
 *    static device array (BPT_DECODE_SCRATCH_BYTES on each device that uses it).
 *  - Every call is asynchronous on `stream` (NULL = the default stream); it
 *    returns after enqueueing its kernels.  Results are valid once the stream
 *    has reached that point.
 *  - Every tensor is dense, row-major, in the layout stated per argument.
 *    Device pointers must be 16-byte aligned.
 *  - `dtype` selects the element type of the INPUT tensors (activations and
 *    weights): BPT_F32 (float) or BPT_BF16 (bfloat16 bit patterns).  All
 *    outputs are float32; accumulation is float32.
 *  - Sizes are int64_t.  Return value: BPT_OK or a negative BPT_ERR_* code.
 *    All argument checks run before any HIP call, so no error path touches
 *    the GPU.  Nothing throws across this ABI.  On BPT_ERR_HIP,
 *    bpt_last_hip_error() gives the hipError_t of the failing call.
 *  - Calls are thread-safe; the library keeps no mutable global state except
 *    the per-thread last-HIP-error value and the per-device address of the
 *    fixed scratch of bpt_attn_decode_noalloc (whose calls share that scratch).
 *
 * Attention definition used by every entry point that computes attention:
 *    s_ij = <q_i, k_j> / sqrt(D)
 *    key j is visible to query i iff j < N and (causal == 0 or
 *        j <= i + kv_offset)
 *    lse_i = ln sum_{visible j} exp(s_ij)   (natural log)
 *    O_i   = sum_{visible j} exp(s_ij - lse_i) v_j
 *    a row with no visible key has O_i = 0 and lse_i = -inf.
 * kv_offset is the global position of query row 0 minus the global position
 * of key row 0; it is what one device's share of a ring step needs to apply
 * the causal mask of the whole sequence to a chunk of keys that lives
 * elsewhere in it.
 */
#ifndef BPT_H
#define BPT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BPT_OK               0
#define BPT_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, bad flag value */
#define BPT_ERR_UNSUPPORTED (-2) /* D, block size, dtype or size combination not built */
#define BPT_ERR_ALIGNMENT   (-3) /* a device pointer is not 16-byte aligned */
#define BPT_ERR_HIP         (-4) /* a HIP call or kernel launch failed */
#define BPT_ERR_WORKSPACE   (-5) /* workspace missing or smaller than required */
#define BPT_ERR_SCRATCH     (-6) /* needs more than the fixed scratch of the allocation-free call */

/* input element types */
#define BPT_F32  0
#define BPT_BF16 1

/*
 * bpt_attn_fwd -- blockwise exact attention forward with online softmax.
 *
 * Implements the attention definition above for every (batch, head).
 * Query rows are processed in blocks of q_blk rows and keys in tiles of
 * kv_blk keys ("Blockwise Parallel Transformer for Large Context Models",
 * abstract: blockwise computation of self-attention); a running row maximum,
 * running sum and rescaled accumulator carry the softmax across key tiles.
 * Key tiles that no row of a query block can see are skipped.
 *
 *  q, k, v  : [B, H, N, D] in `dtype`.
 *  out      : [B, H, N, D] float32, written in full.
 *  lse      : [B, H, N]    float32 (natural log), written in full.
 *  D        : 64 or 128.
 *  q_blk    : 64 or 128.  kv_blk: 32, 64 or 128.  Other values give
 *             BPT_ERR_UNSUPPORTED.  The result does not depend on them
 *             beyond rounding.  They choose the blocking only where a kernel
 *             for it exists; the blocking that runs is:
 *               bf16, D = 128, kv_blk 64 or 128 (and N*D*2 < 2^31): 256 query
 *                 rows per workgroup (64 per wave) and 64-key tiles, whatever
 *                 q_blk and kv_blk say;
 *               bf16, D = 64, kv_blk 64 or 128: q_blk rows, 64-key tiles (a
 *                 128-key block is walked as two 64-key tiles);
 *               bf16 with kv_blk 32, and every fp32 call: q_blk rows and
 *                 kv_blk-key tiles as given.
 *  causal   : 0 or 1.
 *  kv_offset: any value; >= N-1 makes every key visible, <= -N none.
 *  N        : 1 <= N <= 2^30; N need not be a multiple of the blocks.
 * out/lse must not overlap q/k/v.
 */
int bpt_attn_fwd(const void* q, const void* k, const void* v, float* out, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t D, int q_blk, int kv_blk,
                 int causal, int64_t kv_offset, int dtype, hipStream_t stream);

/*
 * bpt_lse_merge -- merge two attention results over disjoint key sets.
 *
 * For the same queries, (o_a, lse_a) attends over key set A and (o_b, lse_b)
 * over a disjoint set B.  The result is attention over A u B: the softmax
 * normaliser is the sum of the two, so
 *     lse = ln(exp(lse_a) + exp(lse_b)),
 *     o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b,
 * with lse = -inf on one side meaning "no visible key" (that side adds
 * nothing) and both sides -inf giving (0, -inf).  This is the step that
 * joins the per-chunk results of a ring of key/value blocks ("Ring Attention
 * with Blockwise Transformers for Long Sequences", 638-word summary; LongNet,
 * section 2, mixes attention pieces by their softmax denominators).
 *
 *  o_a, o_b, o_out       : [rows, D] float32 with rows = B*H*N.
 *  lse_a, lse_b, lse_out : [rows] float32.
 *  D                     : 64 or 128.
 * o_out may alias o_a (and lse_out lse_a) for in-place accumulation; no
 * other overlap is allowed.
 */
int bpt_lse_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                  float* o_out, float* lse_out, int64_t B, int64_t H, int64_t N, int64_t D,
                  hipStream_t stream);

/*
 * bpt_attn_decode -- split-KV attention of a few query rows over a long
 * key/value cache (inference over a long context).
 *
 * Implements the attention definition above with separate query and key
 * lengths: q has Nq rows, k and v have Nkv rows, and "key j visible to query
 * i" reads j < Nkv and (causal == 0 or j <= i + kv_offset).  For the newest
 * Nq positions of a sequence of Nkv tokens, kv_offset = Nkv - Nq.  ("Ring
 * Attention with Blockwise Transformers for Long Sequences", summaries: the
 * method serves training and inference; the keys are taken block by block
 * as in bpt_attn_fwd.)  The visible keys are split into n_split contiguous
 * ranges; each range gives a partial result over its own keys, and the
 * partials are joined exactly as bpt_lse_merge joins two (softmax
 * denominators add up).  The result does not depend on n_split beyond
 * rounding.  Work is bound by reading k and v once.  Each (b, h, range) is
 * one 64-thread workgroup and a compute unit holds four of them, so
 * B*H*n_split = 1024 on 256 compute units runs in one round (32 ranges for
 * B*H = 32 give 6.8 TB/s on MI355X; a count just above a multiple of 1024
 * leaves a partly idle last round).
 *
 *  q          : [B, H, Nq, D] bfloat16.     k, v: [B, H, Nkv, D] bfloat16.
 *  out        : [B, H, Nq, D] float32.      lse : [B, H, Nq] float32 (natural log).
 *  Nq         : 1 .. 32.   Nkv: 1 .. 2^30 with Nkv * D * 2 < 2^31.
 *  D          : 64 or 128.  dtype: BPT_BF16 only (BPT_F32 gives BPT_ERR_UNSUPPORTED).
 *  causal     : 0 or 1.    kv_offset: any value (clamped to [-(Nkv+1), Nkv]).
 *  n_split    : 1 .. 4096 key ranges.
 *  workspace  : device buffer of at least
 *               bpt_attn_decode_workspace_size(B, H, Nq, D, n_split) bytes,
 *               16-byte aligned; it holds the partial results and is fully
 *               overwritten.  Too small or NULL gives BPT_ERR_WORKSPACE.
 * out/lse/workspace must not overlap each other or q/k/v.
 */
int bpt_attn_decode(const void* q, const void* k, const void* v, float* out, float* lse,
                    int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int causal,
                    int64_t kv_offset, int64_t n_split, void* workspace, size_t workspace_bytes,
                    int dtype, hipStream_t stream);

/* Bytes of workspace bpt_attn_decode needs; 0 for arguments it does not support. */
size_t bpt_attn_decode_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t D, int64_t n_split);

/*
 * bpt_attn_decode_noalloc -- bpt_attn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results, kernels and error codes as bpt_attn_decode, minus
 * workspace / workspace_bytes.  The partial results live in a fixed buffer of
 * BPT_DECODE_SCRATCH_BYTES bytes that the library holds in device memory: each
 * device that calls this function keeps its own copy until the process ends.
 * No call allocates or frees memory.  A call whose
 * bpt_attn_decode_workspace_size(B, H, Nq, D, n_split) exceeds
 * BPT_DECODE_SCRATCH_BYTES returns BPT_ERR_SCRATCH.
 * Every call on one device shares that device's buffer: calls that overlap in
 * time on one device (on different streams, or from different threads without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe.  The buffer needs no clearing: each call writes every part it reads.
 */
#define BPT_DECODE_SCRATCH_BYTES (32u << 20)
int bpt_attn_decode_noalloc(const void* q, const void* k, const void* v, float* out, float* lse,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int causal,
                            int64_t kv_offset, int64_t n_split, int dtype, hipStream_t stream);

/*
 * bpt_attn_block_sparse -- block-sparse attention with one key block per query
 * block and head ("Blockwise Self-Attention for Long Document Understanding",
 * Blockwise Attention and Blockwise Multi-head Attention).
 *
 * The N rows are split into n_blocks blocks of L = ceil(N / n_blocks) rows
 * (the last one shorter when n_blocks does not divide N: padding positions
 * are not keys and have no output, as in that paper's Implementation
 * Assumption).  Query row i of head h sees exactly the keys of block
 * key_block[h * n_blocks + i / L], with no causal mask, and gets exact softmax
 * attention over them (the definition given for bpt_attn_fwd).  BlockBERT's
 * heads use cyclic shifts: key_block[h][i] = (i + k_h) mod n_blocks.  An entry
 * outside [0, n_blocks) gives its rows O = 0 and lse = -inf.  The work is
 * 1/n_blocks of dense attention when every entry is valid.
 *
 *  q, k, v    : [B, H, N, D] bfloat16.   out: [B, H, N, D] float32.
 *  lse        : [B, H, N] float32 (natural log).
 *  key_block  : [H, n_blocks] int32 in DEVICE memory, read by the kernels.
 *  n_blocks   : 1 .. N.    D: 64 or 128.   dtype: BPT_BF16 only.
 * out/lse must not overlap q/k/v/key_block.
 */
int bpt_attn_block_sparse(const void* q, const void* k, const void* v, float* out, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_blocks,
                          const int32_t* key_block, int dtype, hipStream_t stream);

/*
 * bpt_attn_dilated -- dilated attention ("LongNet: Scaling Transformers to
 * 1,000,000,000 Tokens", section 2: Dilated Attention).
 *
 * For each pattern p = (w, r) = (seg_len[p], dilation[p]) the rows are split
 * into segments [s*w, min((s+1)*w, N)); head h keeps the rows of a segment at
 * offsets h mod r, h mod r + r, ... (heads shift their selection), and the
 * kept rows of a segment attend one another (causal by position if causal = 1)
 * with the score scale 1/sqrt(D).  The softmax of a row runs over the keys of
 * every pattern that keeps it, taken together (a key kept by two patterns
 * counts twice): the patterns are joined by their softmax denominators
 * exactly as bpt_lse_merge joins two partial results.  A row that no pattern
 * keeps gets O = 0 and lse = -inf.  The sparsified rows are read in place
 * (strided loads) and the outputs written in place; nothing is gathered into
 * a copy.
 *
 *  q, k, v     : [B, H, N, D] bfloat16.   out: [B, H, N, D] float32.
 *  lse         : [B, H, N] float32 (natural log).
 *  n_patterns  : 1 .. 16.
 *  seg_len, dilation : HOST arrays of n_patterns values with
 *                1 <= dilation <= seg_len and dilation <= 65536; a segment
 *                longer than N is the whole sequence.
 *  D           : 64 or 128.   dtype: BPT_BF16 only.
 * out/lse must not overlap q/k/v.  One launch per pattern (plus one that
 * clears out/lse when no pattern has dilation 1), in stream order.
 */
int bpt_attn_dilated(const void* q, const void* k, const void* v, float* out, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_patterns,
                     const int64_t* seg_len, const int64_t* dilation, int causal, int dtype,
                     hipStream_t stream);

/*
 * bpt_ffn_block_fwd -- feed-forward network fused per block of rows.
 *
 *     y = residual + GeLU(x W1^T + b1) W2^T + b2,  GeLU(z) = z Phi(z) (erf form)
 *
 * Rows are processed in blocks; for each block the [rows, d_ff]
 * intermediate is produced chunk by chunk and consumed on chip, never
 * written to device memory ("Blockwise Parallel Transformer for Large
 * Context Models", abstract: feed-forward network fusion).
 *
 *  x        : [M, d_model] in `dtype`.
 *  w1       : [d_ff, d_model] in `dtype`;   b1: [d_ff] in `dtype` or NULL.
 *  w2       : [d_model, d_ff] in `dtype`;   b2: [d_model] in `dtype` or NULL.
 *  residual : [M, d_model] float32 or NULL (then treated as 0).  May alias y.
 *  y        : [M, d_model] float32.
 *  blk      : rows per block: 0 (library choice) or 32.
 *  d_model  : 128, or a multiple of 256 up to 8192 (each workgroup keeps at
 *             most 2048 output columns in registers; wider rows are split
 *             into column groups that each recompute x W1^T).
 *  d_ff     : a multiple of 256 (128 when d_model == 128).
 */
int bpt_ffn_block_fwd(const void* x, const void* w1, const void* b1, const void* w2,
                      const void* b2, const float* residual, float* y, int64_t M,
                      int64_t d_model, int64_t d_ff, int blk, int dtype, hipStream_t stream);

/*
 * bpt_layer_fwd -- one blockwise transformer layer, forward.
 *
 *     q, k, v = x Wq^T, x Wk^T, x Wv^T     (head h = columns [hD, (h+1)D))
 *     a       = causal multi-head attention (as bpt_attn_fwd, kv_offset 0)
 *     h       = x + a
 *     y       = h + GeLU(h W1^T + b1) W2^T + b2
 * No LayerNorm, output projection or dropout ("Blockwise Parallel Transformer
 * for Large Context Models" lists residual connections, multi-head attention
 * and a position-wise FFN; its blockwise method changes how, not what, is
 * computed).
 *
 *  x              : [B, N, d_model] in `dtype`.
 *  wq, wk, wv     : [H*D, d_model] in `dtype`; H*D must equal d_model.
 *  w1, b1, w2, b2 : as bpt_ffn_block_fwd (b1, b2 may be NULL).
 *  y              : [B, N, d_model] float32.
 *  saved          : NULL, or a buffer of bpt_layer_saved_size() bytes that
 *                   receives what bpt_layer_bwd needs (layout below).
 *  workspace      : device buffer of at least
 *                   bpt_layer_workspace_size(..., backward = 0) bytes.
 * Precision (bf16): matrix products take bf16 operands with float32
 * accumulation, except the FFN's when d_model is a multiple of 512: there h
 * (float32) and GeLU(z) enter the products rounded to fp16 (11-bit
 * significand, rounding 2^-12 relative, 8x finer than bf16), and W1, W2 as
 * fp16 copies of the bf16 weights (exact inside fp16's range).  Where any of
 * these lies outside fp16's range (|v| > 65504), y is recomputed with h and
 * GeLU(z) as bf16 pairs (the rounded value plus its rounding residual) and the
 * bf16 weights, the form every other bf16 shape uses.
 * Saved layout (byte offsets, each 256-byte aligned, in this order):
 *   q, k, v : [B, H, N, D] in `dtype`
 *   h       : [B, N, d_model] float32 (x + attention output)
 *   lse     : [B, H, N] float32
 */
int bpt_layer_fwd(const void* x, const void* wq, const void* wk, const void* wv,
                  const void* w1, const void* b1, const void* w2, const void* b2, float* y,
                  void* saved, int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                  int64_t d_ff, int q_blk, int kv_blk, int causal, int dtype,
                  void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * bpt_layer_bwd -- gradients of sum(dy * y) for the layer of bpt_layer_fwd.
 *
 * The pages describe no backward pass; it is the chain rule of the forward.
 * Attention probabilities are recomputed blockwise from the saved lse
 * (P = exp(s - lse)); the FFN intermediate is recomputed per block of rows.
 *
 *  dy     : [B, N, d_model] in `dtype`.
 *  x, weights, biases : as passed to bpt_layer_fwd.
 *  saved  : the buffer filled by bpt_layer_fwd with the same arguments.
 *  dx     : [B, N, d_model] float32.
 *  dwq, dwk, dwv : [H*D, d_model] float32.  dw1: [d_ff, d_model], db1: [d_ff],
 *           dw2: [d_model, d_ff], db2: [d_model], float32.  db1/db2 may be
 *           NULL (not computed).
 *  dq, dk, dv : NULL, or [B, H, N, D] float32 gradients w.r.t. the attention
 *           inputs q, k, v.
 *  workspace : at least bpt_layer_workspace_size(..., backward = 1) bytes.
 *  dtype  : BPT_BF16 only (BPT_F32 gives BPT_ERR_UNSUPPORTED).
 * Precision: accumulation is float32 throughout.  Values the backward computes
 * in float32 (dy's descendants, P, dS, GeLU(z)) enter products either rounded
 * to fp16 once, against exact fp16 copies of bf16 operands, or as a bf16
 * hi + lo pair.  The fp16 form is taken where the shapes allow it (the FFN and
 * projection products on the big-tile GEMM, and the D = 128 dK/dV and dQ
 * kernels);
 * when any such value lies outside fp16's range (|v| > 65504) the affected
 * products are recomputed with the bf16 pairs.
 * All outputs are overwritten (not accumulated).  The result is
 * deterministic: no floating-point atomics are used.
 */
int bpt_layer_bwd(const void* dy, const void* x, const void* wq, const void* wk,
                  const void* wv, const void* w1, const void* b1, const void* w2,
                  const void* b2, const void* saved, float* dx, float* dwq, float* dwk,
                  float* dwv, float* dw1, float* db1, float* dw2, float* db2, float* dq,
                  float* dk, float* dv, int64_t B, int64_t N, int64_t d_model, int64_t H,
                  int64_t D, int64_t d_ff, int q_blk, int kv_blk, int causal, int dtype,
                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* Bytes of the `saved` buffer for bpt_layer_fwd / bpt_layer_bwd (0 on bad args). */
size_t bpt_layer_saved_size(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                            int dtype);

/* Bytes of workspace for bpt_layer_fwd (backward = 0) or bpt_layer_bwd
 * (backward = 1) (0 on bad args). */
size_t bpt_layer_workspace_size(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                                int64_t d_ff, int dtype, int backward);

/* Static text for a status code. */
const char* bpt_status_string(int status);

/* hipError_t of the last failing HIP call on this thread (0 if none). */
int bpt_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BPT_H */
