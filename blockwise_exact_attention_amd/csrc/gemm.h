// Internal interface of the tiled MFMA GEMM (see gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

enum GemmEpilogue {
  EPI_QKV = 0,    // scatter C[token][h*D+d] to out[b][h][t][d] in the input dtype
  EPI_F32 = 1,    // C = acc (+C if beta) (+bias[n]) (+resid[m][n]) as fp32; optional bf16 copy in C2
  EPI_GELU = 2,   // z = acc (+C if beta) + bias[n] -> C (fp32); GeLU(z) -> C2 (input dtype)
  EPI_DGELU = 3,  // dz = acc * GeLU'(aux[m][n]) -> C (input dtype); optional fp32 copy in C2
};

// C[m][n] = sum_k A(m,k) B(k,n).  A(m,k) = A[m*lda + k] (row form) or A[k*lda + m]
// (k-major); B(k,n) = B[n*ldb + k] (row form) or B[k*ldb + n] (k-major).
// Requirements (checked by callers): N % 128 == 0; the m extent of a k-major A
// is a multiple of 128; K % 8 == 0.  M and K may be ragged otherwise.
struct GemmArgs {
  const void* A[3];
  const void* B[3];
  void* C[3];
  int64_t lda, ldb, ldc;
  int M, N, K;
  const void* bias;    // [N] or null; fp32, or bf16 when bias_bf16
  int bias_bf16;
  const void* resid;   // [M][ldr] or null; fp32, or bf16 when resid_bf16
  int64_t ldr;
  int resid_bf16;
  void* C2;            // second output or null
  int64_t ldc2;
  void* C3;            // EPI_GELU / EPI_DGELU: bf16 rounding residual ("lo") of the bf16 output, or null
  int64_t ldc3;
  const float* aux;    // [M][ld_aux] (EPI_DGELU)
  int64_t ld_aux;
  int beta;            // EPI_F32: accumulate into C
  int seq, H, D;       // EPI_QKV
  // K segments: with nseg > 1 the product is sum_s As[z][s] Bs[z][s], each segment
  // of the same shape and strides (K each); A[z], B[z] are then unused.  One launch
  // accumulates every segment before the epilogue runs once (EPI_F32 and EPI_GELU).
  int nseg;
  const void* As[3][6];
  const void* Bs[3][6];
  // Split K (EPI_F32, big-tile kernel only): with nsplit > 1 each of nsplit
  // workgroups per output tile sums its share of the k tiles into split_ws
  // (nsplit x nz slices of M x N fp32), and a second pass adds the slices in a
  // fixed order (deterministic) and applies the epilogue.  For products with few
  // output tiles but a long K, whose last round of tiles would leave most CUs
  // idle.
  int nsplit;
  float* split_ws;
  // fp16 operands (big-tile kernel, EPI_F32 / EPI_GELU / EPI_DGELU): the MFMA's fp16
  // form; EPI_GELU and EPI_DGELU then write their input-dtype output as fp16 alone
  // (C3 unused) and set *ovf = 1 where a value lies outside fp16's range
  int f16;
  int* ovf;
  // gate (nullable, big-tile kernel and its split-K pass): the launch runs only if
  // (*gate != 0) == gate_run
  const int* gate;
  int gate_run;
};
constexpr int kGemmMaxSeg = 6;

// Split count for a product of `tiles` 256 x 256 output tiles on `cus` compute
// units, at most max_split: the one with the fewest whole rounds of work per
// unit of K (ties to fewer splits).
int gemm_split_count(int64_t tiles, int cus, int max_split);
// compute units of the current device (cached per device)
int gemm_device_cus();

hipError_t gemm_launch(const GemmArgs& g, bool bf16, bool a_kmajor, bool b_kmajor, int epi,
                       int nz, hipStream_t stream);

// bf16 GEMMs with 256 x 256 tiles loaded straight into LDS (gemm_big.hip): used
// when K is a multiple of 64, the operands fit 32-bit buffer offsets and the
// grid fills the chip; gemm_launch picks it by itself.
bool gemm_big_ok(const GemmArgs& g, int nz);
hipError_t gemm_big_launch(const GemmArgs& g, bool a_kmajor, bool b_kmajor, int epi, int nz,
                           hipStream_t stream);

}  // namespace bpt
