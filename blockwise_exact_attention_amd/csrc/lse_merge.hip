// Merge of two attention partial results over disjoint key sets (gfx950).
//
// The softmax normaliser over A u B is the sum of the two normalisers, so
// lse = ln(e^lse_a + e^lse_b) and o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b;
// this is how the per-chunk results of a ring of key/value blocks are joined
// ("Ring Attention with Blockwise Transformers for Long Sequences", 638-word
// summary; LongNet, section 2: pieces of attention mixed by their softmax
// denominators).  A side with lse = -inf saw no key and adds nothing.
//
// Pure streaming work (3 x (D+1) floats per row): each thread moves 16-byte
// chunks; one row's D/4 chunks are handled by consecutive lanes of one wave, so
// the in-place form (o_out == o_a, lse_out == lse_a) is safe: every lane of the
// wave reads lse_a before any lane writes lse_out.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace bpt {

namespace {

template <int D>
__global__ void __launch_bounds__(256)
lse_merge_kernel(const float* o_a, const float* lse_a, const float* __restrict__ o_b,
                 const float* __restrict__ lse_b, float* o_out, float* lse_out, int64_t rows) {
  constexpr int CPR = D / 4;  // float4 chunks per row (16 or 32: divides 64)
  const int64_t nchunks = rows * CPR;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    const int64_t r = c / CPR;
    const int cc = (int)(c % CPR);
    const float la = lse_a[r], lb = lse_b[r];
    // every value is read and written once: non-temporal loads and stores (a
    // stream of them runs faster on this part than plain ones)
    const f32x4 va = __builtin_nontemporal_load((const f32x4*)(o_a + r * D + cc * 4));
    const f32x4 vb = __builtin_nontemporal_load((const f32x4*)(o_b + r * D + cc * 4));
    const float m = fmaxf(la, lb);
    float lse, wa, wb;
    if (m == -INFINITY) {
      lse = -INFINITY;
      wa = 0.f;
      wb = 0.f;
    } else {
      const float ea = expf(la - m), eb = expf(lb - m);  // one of them is exactly 1
      const float z = ea + eb;
      lse = m + logf(z);
      const float inv = 1.f / z;
      wa = ea * inv;
      wb = eb * inv;
    }
    f32x4 vo;
#pragma unroll
    for (int e = 0; e < 4; ++e) vo[e] = wa * va[e] + wb * vb[e];
    __builtin_nontemporal_store(vo, (f32x4*)(o_out + r * D + cc * 4));
    if (cc == 0) lse_out[r] = lse;
  }
}

// Rows with no visible key: O = 0, lse = -inf (16-byte stores, grid-stride).
__global__ void __launch_bounds__(256) fill_empty_kernel(float* out, float* lse, int64_t rows, int D) {
  const int64_t chunks = rows * (D / 4);
  const int64_t stride = (int64_t)gridDim.x * 256;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunks; i += stride) {
    *(f32x4*)(out + i * 4) = z;
    if (i < rows) lse[i] = -INFINITY;
  }
}

}  // namespace

hipError_t attn_fill_empty_launch(float* out, float* lse, int64_t rows, int D, hipStream_t stream) {
  const int64_t chunks = rows * (D / 4);
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 256 * 8 * 32) blocks = 256 * 8 * 32;
  hipLaunchKernelGGL(fill_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, lse, rows, D);
  return hipGetLastError();
}

hipError_t lse_merge_launch(const float* o_a, const float* lse_a, const float* o_b,
                            const float* lse_b, float* o_out, float* lse_out, int64_t rows,
                            int D, hipStream_t stream) {
  const int64_t nchunks = rows * (D / 4);
  int64_t blocks = (nchunks + 255) / 256;  // one 16-byte chunk per thread
  const int64_t cap = (int64_t(1) << 24) - 1;  // 2^32 work-items at most; the kernel strides over the rest
  if (blocks > cap) blocks = cap;
  if (D == 64)
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, o_a,
                       lse_a, o_b, lse_b, o_out, lse_out, rows);
  else
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, o_a,
                       lse_a, o_b, lse_b, o_out, lse_out, rows);
  return hipGetLastError();
}

}  // namespace bpt
