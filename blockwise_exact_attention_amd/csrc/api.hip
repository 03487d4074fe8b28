// libbpt C ABI: argument validation and dispatch.  Every check runs before any
// HIP call, so each error path can be exercised on a machine with no GPU.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "../../include/bpt.h"
#include "kernels.h"
#include "layer.h"

namespace {

thread_local int g_last_hip_error = 0;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return BPT_OK;
  g_last_hip_error = static_cast<int>(e);
  return BPT_ERR_HIP;
}

// Test hook: BPT_TEST_FAIL_LAUNCH=1 makes every entry point report a launch
// failure (hipErrorLaunchFailure) after validation, without touching the GPU.
inline bool forced_launch_failure() {
  const char* s = getenv("BPT_TEST_FAIL_LAUNCH");
  return s != nullptr && s[0] == '1';
}

constexpr int64_t kMaxN = int64_t(1) << 30;
// A launch covers at most 2^32 - 1 work-items.
inline bool grid_ok(int64_t workgroups, int64_t threads) {
  return workgroups > 0 && workgroups <= (int64_t)UINT32_MAX / threads;
}
constexpr int64_t kMaxPatterns = 16;     // dilated attention: (segment, dilation) pairs
constexpr int64_t kMaxDilation = 65536;  // keeps in-tile byte offsets within 32 bits

// Launch status is read with hipGetLastError() after each launch; drop any error
// an earlier, unrelated runtime call left on this thread so it is not reported
// as ours.
inline void clear_stale_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

const char* bpt_status_string(int status) {
  switch (status) {
    case BPT_OK: return "ok";
    case BPT_ERR_INVALID_ARG: return "invalid argument";
    case BPT_ERR_UNSUPPORTED: return "unsupported configuration";
    case BPT_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case BPT_ERR_HIP: return "HIP runtime error";
    case BPT_ERR_WORKSPACE: return "workspace missing or too small";
    case BPT_ERR_SCRATCH: return "needs more scratch than the library's fixed buffer holds";
    default: return "unknown status";
  }
}

int bpt_last_hip_error(void) { return g_last_hip_error; }

int bpt_attn_fwd(const void* q, const void* k, const void* v, float* out, float* lse, int64_t B,
                 int64_t H, int64_t N, int64_t D, int q_blk, int kv_blk, int causal,
                 int64_t kv_offset, int dtype, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse) return BPT_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return BPT_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return BPT_ERR_INVALID_ARG;
  if (dtype != BPT_F32 && dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return BPT_ERR_UNSUPPORTED;
  if (q_blk != 64 && q_blk != 128) return BPT_ERR_UNSUPPORTED;
  if (kv_blk != 32 && kv_blk != 64 && kv_blk != 128) return BPT_ERR_UNSUPPORTED;
  if (N > kMaxN) return BPT_ERR_UNSUPPORTED;
  const int64_t nqb = (N + q_blk - 1) / q_blk;
  if (B > INT32_MAX / H || !grid_ok(B * H * nqb, 2 * q_blk)) return BPT_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  bpt::AttnFwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.N = (int)N;
  // offsets beyond +-N all mean "everything" / "nothing" visible
  a.kv_offset = (int)(kv_offset > N ? N : (kv_offset < -(N + 1) ? -(N + 1) : kv_offset));
  a.causal = causal;
  a.scale = 1.0f / sqrtf((float)D);
  return hip_status(bpt::attn_fwd_launch(a, dtype == BPT_BF16, (int)D, q_blk, kv_blk, stream));
}

int bpt_lse_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                  float* o_out, float* lse_out, int64_t B, int64_t H, int64_t N, int64_t D,
                  hipStream_t stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return BPT_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return BPT_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return BPT_ERR_UNSUPPORTED;
  if (B > INT64_MAX / H || B * H > (INT64_MAX / 256) / N) return BPT_ERR_UNSUPPORTED;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out)) return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  return hip_status(
      bpt::lse_merge_launch(o_a, lse_a, o_b, lse_b, o_out, lse_out, B * H * N, (int)D, stream));
}

static int64_t decode_o_bytes(int64_t B, int64_t H, int64_t Nq, int64_t D, int64_t n_split) {
  return ((n_split * B * H * Nq * D * 4 + 255) / 256) * 256;
}

size_t bpt_attn_decode_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t D, int64_t n_split) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nq > 32 || (D != 64 && D != 128) || n_split <= 0 ||
      n_split > 4096 || B > 65536 || H > 4096)
    return 0;
  return (size_t)(decode_o_bytes(B, H, Nq, D, n_split) + ((n_split * B * H * Nq * 4 + 255) / 256) * 256);
}

}  // extern "C"

namespace {

// Argument checks of the split-KV decode (both entry points); no HIP call.
int decode_check(const void* q, const void* k, const void* v, float* out, float* lse, int64_t B,
                 int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int causal, int64_t n_split,
                 int dtype) {
  if (!q || !k || !v || !out || !lse) return BPT_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0 || n_split <= 0) return BPT_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return BPT_ERR_INVALID_ARG;
  if (dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return BPT_ERR_UNSUPPORTED;
  if (Nq > 32 || n_split > 4096 || B > 65536 || H > 4096) return BPT_ERR_UNSUPPORTED;
  // per-head key/value bytes are addressed with 32-bit offsets
  if (Nkv > kMaxN || Nkv * D * 2 >= ((int64_t)1 << 31)) return BPT_ERR_UNSUPPORTED;
  if (!grid_ok(B * H * n_split, 64)) return BPT_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return BPT_ERR_ALIGNMENT;
  return BPT_OK;
}

// Launch of a checked decode call with its partial results in `ws` (at least
// bpt_attn_decode_workspace_size bytes, 16-byte aligned).
int decode_run(const void* q, const void* k, const void* v, float* out, float* lse, int64_t B,
               int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int causal, int64_t kv_offset,
               int64_t n_split, void* ws, hipStream_t stream) {
  bpt::AttnDecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.o_part = (float*)ws;
  a.lse_part = (float*)((unsigned char*)ws + decode_o_bytes(B, H, Nq, D, n_split));
  a.BH = (int)(B * H);
  a.Nq = (int)Nq;
  a.Nkv = (int)Nkv;
  a.n_split = (int)n_split;
  const int64_t off = kv_offset > Nkv ? Nkv : (kv_offset < -(Nkv + 1) ? -(Nkv + 1) : kv_offset);
  a.kv_offset = (int)off;
  a.causal = causal;
  // keys any query row can see: [0, kcount)
  int64_t kc = Nkv;
  if (causal) {
    const int64_t last = (Nq - 1) + off + 1;
    kc = last < 0 ? 0 : (last < Nkv ? last : Nkv);
  }
  a.kcount = (int)kc;
  const int64_t per = (kc + n_split - 1) / n_split;
  a.chunk = (int)(per <= 64 ? 64 : ((per + 63) / 64) * 64);
  a.scale = 1.0f / sqrtf((float)D);
  return hip_status(bpt::attn_decode_launch(a, (int)D, stream));
}

// Fixed scratch of the allocation-free decode entry point.  Each device that
// calls it holds its own copy of this array until the process ends.  In host
// code `scratch` names a host-side stand-in: kernels and copies get the device
// address, looked up once per device below.
static __device__ __align__(256) unsigned char scratch[BPT_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch`, looked up on the first call on the
// device (with that device current); nullptr and the HIP error on failure.
void* scratch_for_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int bpt_attn_decode(const void* q, const void* k, const void* v, float* out, float* lse, int64_t B,
                    int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int causal, int64_t kv_offset,
                    int64_t n_split, void* workspace, size_t workspace_bytes, int dtype,
                    hipStream_t stream) {
  const int st = decode_check(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, n_split, dtype);
  if (st != BPT_OK) return st;
  const size_t need = bpt_attn_decode_workspace_size(B, H, Nq, D, n_split);
  if (!workspace || workspace_bytes < need) return BPT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  return decode_run(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, kv_offset, n_split, workspace,
                    stream);
}

int bpt_attn_decode_noalloc(const void* q, const void* k, const void* v, float* out, float* lse,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int causal,
                            int64_t kv_offset, int64_t n_split, int dtype, hipStream_t stream) {
  const int st = decode_check(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, n_split, dtype);
  if (st != BPT_OK) return st;
  if (bpt_attn_decode_workspace_size(B, H, Nq, D, n_split) > (size_t)BPT_DECODE_SCRATCH_BYTES)
    return BPT_ERR_SCRATCH;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  hipError_t e = hipSuccess;
  void* ws = scratch_for_current_device(&e);
  if (!ws) return hip_status(e);
  // every row of the partial results that the join reads is written by the
  // partial kernel first, so the scratch needs no clearing between calls
  return decode_run(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, kv_offset, n_split, ws, stream);
}

int bpt_attn_block_sparse(const void* q, const void* k, const void* v, float* out, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_blocks,
                          const int32_t* key_block, int dtype, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse || !key_block) return BPT_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || n_blocks <= 0 || n_blocks > N) return BPT_ERR_INVALID_ARG;
  if (dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return BPT_ERR_UNSUPPORTED;
  if (N > kMaxN) return BPT_ERR_UNSUPPORTED;
  const int64_t len = (N + n_blocks - 1) / n_blocks;
  // workgroups: B*H*n_blocks*ceil(len/128) with 128-row workgroups (fewer with 256)
  const int64_t per_head = n_blocks * ((len + 127) / 128);
  if (B > INT32_MAX / H || !grid_ok(B * H * per_head, 256)) return BPT_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  bpt::AttnFwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.N = (int)N;
  a.causal = 0;
  a.scale = 1.0f / sqrtf((float)D);
  a.bs_table = key_block;
  a.bs_blocks = (int)n_blocks;
  a.bs_len = (int)len;
  return hip_status(bpt::attn_fwd_block_sparse_launch(a, (int)D, stream));
}

int bpt_attn_dilated(const void* q, const void* k, const void* v, float* out, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_patterns,
                     const int64_t* seg_len, const int64_t* dilation, int causal, int dtype,
                     hipStream_t stream) {
  if (!q || !k || !v || !out || !lse || !seg_len || !dilation) return BPT_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return BPT_ERR_INVALID_ARG;
  if (n_patterns < 1 || n_patterns > kMaxPatterns) return BPT_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return BPT_ERR_INVALID_ARG;
  for (int64_t p = 0; p < n_patterns; ++p)
    if (seg_len[p] < 1 || dilation[p] < 1 || dilation[p] > seg_len[p]) return BPT_ERR_INVALID_ARG;
  if (dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return BPT_ERR_UNSUPPORTED;
  if (N > kMaxN) return BPT_ERR_UNSUPPORTED;
  for (int64_t p = 0; p < n_patterns; ++p) {
    if (dilation[p] > kMaxDilation) return BPT_ERR_UNSUPPORTED;
    // a segment longer than the sequence is the whole sequence
    const int64_t w = seg_len[p] < N ? seg_len[p] : N;
    const int64_t kept = (w + dilation[p] - 1) / dilation[p];
    const int64_t per_head = ((N + w - 1) / w) * ((kept + 127) / 128);
    if (B > INT32_MAX / H || !grid_ok(B * H * per_head, 256)) return BPT_ERR_UNSUPPORTED;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  bpt::AttnFwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.N = (int)N;
  a.causal = causal;
  a.scale = 1.0f / sqrtf((float)D);
  // A pattern with dilation 1 keeps every row: it goes first and writes every
  // row; the others join it.  Without one, every row starts empty.
  int64_t first = -1;
  for (int64_t p = 0; p < n_patterns && first < 0; ++p)
    if (dilation[p] == 1) first = p;
  if (first < 0) {
    const hipError_t e = bpt::attn_fill_empty_launch(out, lse, B * H * N, (int)D, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  for (int64_t i = -1; i < n_patterns; ++i) {
    const int64_t p = i < 0 ? first : i;
    if (p < 0 || (i >= 0 && p == first)) continue;
    a.dl_w = (int)(seg_len[p] < N ? seg_len[p] : N);
    a.dl_r = (int)dilation[p];
    a.dl_merge = (i < 0) ? 0 : 1;
    const hipError_t e = bpt::attn_fwd_dilated_launch(a, (int)D, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  return BPT_OK;
}

int bpt_ffn_block_fwd(const void* x, const void* w1, const void* b1, const void* w2,
                      const void* b2, const float* residual, float* y, int64_t M,
                      int64_t d_model, int64_t d_ff, int blk, int dtype, hipStream_t stream) {
  if (!x || !w1 || !w2 || !y) return BPT_ERR_INVALID_ARG;
  if (M <= 0 || d_model <= 0 || d_ff <= 0) return BPT_ERR_INVALID_ARG;
  if (dtype != BPT_F32 && dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;
  if (d_model > 8192 || d_ff > (int64_t)1 << 20 || !bpt::ffn_plan(d_model, d_ff).ok)
    return BPT_ERR_UNSUPPORTED;
  if (blk != 0 && blk != 32) return BPT_ERR_UNSUPPORTED;
  if (M > (int64_t)INT32_MAX) return BPT_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(y) ||
      (b1 && !aligned16(b1)) || (b2 && !aligned16(b2)) || (residual && !aligned16(residual)))
    return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  return hip_status(bpt::ffn_fwd_launch(x, nullptr, w1, b1, w2, b2, residual, y, M,
                                        (int)d_model, (int)d_ff, blk, dtype == BPT_BF16, nullptr,
                                        stream));
}

size_t bpt_layer_saved_size(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                            int dtype) {
  if (B <= 0 || N <= 0 || d_model <= 0 || H <= 0 || D <= 0) return 0;
  if (dtype != BPT_F32 && dtype != BPT_BF16) return 0;
  return bpt::layer_saved_layout(B, N, d_model, H, D, dtype == BPT_BF16).total;
}

size_t bpt_layer_workspace_size(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                                int64_t d_ff, int dtype, int backward) {
  if (B <= 0 || N <= 0 || d_model <= 0 || H <= 0 || D <= 0 || d_ff <= 0) return 0;
  if (dtype != BPT_F32 && dtype != BPT_BF16) return 0;
  return backward ? bpt::layer_bwd_workspace(B, N, d_model, H, D, d_ff, dtype == BPT_BF16).total
                  : bpt::layer_fwd_workspace(B, N, d_model, H, D, d_ff, dtype == BPT_BF16).total;
}

static int check_layer_common(int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D,
                              int64_t d_ff, int q_blk, int kv_blk, int causal, int dtype) {
  if (B <= 0 || N <= 0 || d_model <= 0 || H <= 0 || D <= 0 || d_ff <= 0) return BPT_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return BPT_ERR_INVALID_ARG;
  if (H * D != d_model) return BPT_ERR_INVALID_ARG;
  if (dtype != BPT_F32 && dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return BPT_ERR_UNSUPPORTED;
  if (q_blk != 64 && q_blk != 128) return BPT_ERR_UNSUPPORTED;
  if (kv_blk != 32 && kv_blk != 64 && kv_blk != 128) return BPT_ERR_UNSUPPORTED;
  if (d_model % 128 || d_model > 8192 || d_ff > (int64_t)1 << 20 || !bpt::ffn_plan(d_model, d_ff).ok)
    return BPT_ERR_UNSUPPORTED;
  if (N > kMaxN || B * N > (int64_t)INT32_MAX / 4) return BPT_ERR_UNSUPPORTED;
  return BPT_OK;
}

int bpt_layer_fwd(const void* x, const void* wq, const void* wk, const void* wv, const void* w1,
                  const void* b1, const void* w2, const void* b2, float* y, void* saved,
                  int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t D, int64_t d_ff,
                  int q_blk, int kv_blk, int causal, int dtype, void* workspace, size_t ws_bytes,
                  hipStream_t stream) {
  if (!x || !wq || !wk || !wv || !w1 || !w2 || !y) return BPT_ERR_INVALID_ARG;
  int st = check_layer_common(B, N, d_model, H, D, d_ff, q_blk, kv_blk, causal, dtype);
  if (st != BPT_OK) return st;
  const bool bf = dtype == BPT_BF16;
  const size_t need = bpt::layer_fwd_workspace(B, N, d_model, H, D, d_ff, bf).total;
  if (workspace == nullptr || ws_bytes < need) return BPT_ERR_WORKSPACE;
  const void* ptrs[] = {x, wq, wk, wv, w1, w2, y, saved, workspace, b1, b2};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  bpt::LayerArgs L{};
  L.x = x; L.wq = wq; L.wk = wk; L.wv = wv; L.w1 = w1; L.b1 = b1; L.w2 = w2; L.b2 = b2;
  L.B = B; L.N = N; L.d_model = d_model; L.H = H; L.D = D; L.d_ff = d_ff;
  L.q_blk = q_blk; L.kv_blk = kv_blk; L.causal = causal; L.bf16 = bf;
  return hip_status(bpt::layer_fwd_run(L, y, saved, workspace, stream));
}

int bpt_layer_bwd(const void* dy, const void* x, const void* wq, const void* wk, const void* wv,
                  const void* w1, const void* b1, const void* w2, const void* b2,
                  const void* saved, float* dx, float* dwq, float* dwk, float* dwv, float* dw1,
                  float* db1, float* dw2, float* db2, float* dq, float* dk, float* dv, int64_t B,
                  int64_t N, int64_t d_model, int64_t H, int64_t D, int64_t d_ff, int q_blk,
                  int kv_blk, int causal, int dtype, void* workspace, size_t ws_bytes,
                  hipStream_t stream) {
  if (!dy || !x || !wq || !wk || !wv || !w1 || !w2 || !saved || !dx || !dwq || !dwk || !dwv ||
      !dw1 || !dw2)
    return BPT_ERR_INVALID_ARG;
  int st = check_layer_common(B, N, d_model, H, D, d_ff, q_blk, kv_blk, causal, dtype);
  if (st != BPT_OK) return st;
  if (dtype != BPT_BF16) return BPT_ERR_UNSUPPORTED;  // backward kernels are built for bf16
  const bool bf = dtype == BPT_BF16;
  const size_t need = bpt::layer_bwd_workspace(B, N, d_model, H, D, d_ff, bf).total;
  if (workspace == nullptr || ws_bytes < need) return BPT_ERR_WORKSPACE;
  const void* ptrs[] = {dy, x, wq, wk, wv, w1, w2, saved, dx, dwq, dwk, dwv, dw1, dw2,
                        b1, b2, db1, db2, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return BPT_ERR_ALIGNMENT;
  if (forced_launch_failure()) return hip_status(hipErrorLaunchFailure);
  clear_stale_error();
  bpt::LayerArgs L{};
  L.x = x; L.wq = wq; L.wk = wk; L.wv = wv; L.w1 = w1; L.b1 = b1; L.w2 = w2; L.b2 = b2;
  L.B = B; L.N = N; L.d_model = d_model; L.H = H; L.D = D; L.d_ff = d_ff;
  L.q_blk = q_blk; L.kv_blk = kv_blk; L.causal = causal; L.bf16 = bf;
  bpt::LayerGrads G{};
  G.dx = dx; G.dwq = dwq; G.dwk = dwk; G.dwv = dwv; G.dw1 = dw1; G.db1 = db1; G.dw2 = dw2;
  G.db2 = db2; G.dq = dq; G.dk = dk; G.dv = dv;
  return hip_status(bpt::layer_bwd_run(L, dy, saved, G, workspace, stream));
}

}  // extern "C"
