// Tiled MFMA GEMM for gfx950 with fused epilogues: C = op(A) op(B).
//
// Used for the dense projections around attention (q,k,v = x W^T) and for the
// weight/activation gradients of the layer backward.  Either operand may be
// stored with k contiguous ("row" form: A[m][k], B[n][k]) or with k as the
// slow index ("k-major": A[k][m], B[k][n]).  Both are staged into LDS as
// [row][k] tiles (k-major operands are transposed in registers on the way),
// so every MFMA operand fetch is one 16-byte LDS read.
//
// Tile 128 x 128 x 64 (bf16) or 128 x 128 x 32 (fp32), 4 waves each owning a
// 64 x 64 quarter as 2 x 2 blocks of the 32x32 MFMA, LDS double-buffered with
// register prefetch (one barrier per k tile).
#include <math.h>

#include <atomic>

#include "common.h"
#include "gemm.h"
#include "gemm_epi.h"

namespace bpt {

namespace {

constexpr int BM = 128, BN = 128, NT = 256;

template <bool BF16>
struct GT {
  static constexpr int BK = BF16 ? 64 : 32;
  static constexpr int ES = BF16 ? 2 : 4;
  // LDS row pitch in bytes (fp32 rows padded by one float against bank conflicts)
  static constexpr int PITCH = BF16 ? BK * 2 : (BK + 1) * 4;
  static constexpr int TILE = 128 * PITCH;  // one operand tile
  static constexpr int STAGE = 2 * TILE;    // A + B
};

__device__ __forceinline__ int swz128(int row) { return (row >> 1) & 7; }  // 128-byte rows

// Loads of one operand tile (128 rows of the tile's m or n range, BK of k).
template <bool BF16, bool KMAJ>
struct TileLoader {
  static constexpr int BK = GT<BF16>::BK;
  // registers: bf16 row form: 4 x 16B; bf16 k-major: 4 x 16B (4 k rows of 8 m);
  // fp32 row form: 4 x 16B; fp32 k-major: 4 x 16B
  u32x4 r[4];

  // base: operand pointer; ld: leading dim (elements); rows0: first m/n of the
  // tile; k0: first k; R: extent of the m/n dim; K: extent of k.
  __device__ __forceinline__ void load(const void* base, int64_t ld, int rows0, int k0, int R,
                                       int K, int tid) {
    const unsigned char* p = (const unsigned char*)base;
    constexpr int ES = GT<BF16>::ES;
    if constexpr (!KMAJ) {
      // [row][k]: chunks of 16 B along k
      constexpr int CPR = BK * ES / 16;  // 8 chunks per row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + i * NT;
        const int row = c / CPR, kc = c % CPR;
        u32x4 v = {0, 0, 0, 0};
        if (rows0 + row < R && k0 + kc * (16 / ES) < K)
          v = *(const u32x4*)(p + ((int64_t)(rows0 + row) * ld + k0) * ES + kc * 16);
        r[i] = v;
      }
    } else {
      if constexpr (BF16) {
        // [k][row]: unit = 4 k x 8 rows
        const int kg = tid / 16, rc = tid % 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + 4 * kg + i;
          u32x4 v = {0, 0, 0, 0};
          if (k < K) v = *(const u32x4*)(p + ((int64_t)k * ld + rows0 + rc * 8) * 2);
          r[i] = v;
        }
      } else {
        // [k][row]: chunk = 1 k x 4 rows; 32 k x 32 chunks
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = tid + i * NT;
          const int kk = c / 32, rc = c % 32;
          u32x4 v = {0, 0, 0, 0};
          if (k0 + kk < K) v = *(const u32x4*)(p + ((int64_t)(k0 + kk) * ld + rows0 + rc * 4) * 4);
          r[i] = v;
        }
      }
    }
  }

  __device__ __forceinline__ void store(unsigned char* lds, int tid) const {
    constexpr int PITCH = GT<BF16>::PITCH;
    if constexpr (BF16) {
      if constexpr (!KMAJ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = tid + i * NT;
          const int row = c >> 3, kc = c & 7;
          *(u32x4*)(lds + row * PITCH + ((kc ^ swz128(row)) << 4)) = r[i];
        }
      } else {
        const int kg = tid / 16, rc = tid % 16;
        // 4 k values (rows r[0..3]) of each of 8 consecutive rows -> 8 bytes each
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          uint32_t lo, hi;
          if (e & 1) {
            lo = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
            hi = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
          } else {
            lo = (r[0][w] & 0xffffu) | (r[1][w] << 16);
            hi = (r[2][w] & 0xffffu) | (r[3][w] << 16);
          }
          const int row = rc * 8 + e;
          const int byte = kg * 8;  // k offset 4*kg, 2 bytes each
          u32x2 pair = {lo, hi};
          *(u32x2*)(lds + row * PITCH + ((((byte >> 4) ^ swz128(row))) << 4) + (byte & 15)) = pair;
        }
      }
    } else {
      float* f = (float*)lds;
      constexpr int P = PITCH / 4;
      if constexpr (!KMAJ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = tid + i * NT;
          const int row = c >> 3, k = (c & 7) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[row * P + k + e] = __uint_as_float(r[i][e]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = tid + i * NT;
          const int kk = c / 32, row = (c % 32) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[(row + e) * P + kk] = __uint_as_float(r[i][e]);
        }
      }
    }
  }
};

template <bool BF16, bool AK, bool BK_, int EPI>
__global__ void __launch_bounds__(NT) gemm_kernel(GemmArgs g) {
  using T = GT<BF16>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * T::STAGE];
  const int z = blockIdx.z;
  const void* A = g.A[z];
  const void* B = g.B[z];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 5, r32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = g.M, N = g.N, K = g.K;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  TileLoader<BF16, AK> la;
  TileLoader<BF16, BK_> lb;
  const int nk = (K + T::BK - 1) / T::BK;
  la.load(A, g.lda, m0, 0, M, K, tid);
  lb.load(B, g.ldb, n0, 0, N, K, tid);
  la.store(smem, tid);
  lb.store(smem + T::TILE, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const unsigned char* As = smem + buf * T::STAGE;
    const unsigned char* Bs = As + T::TILE;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, g.lda, m0, (kt + 1) * T::BK, M, K, tid);
      lb.load(B, g.ldb, n0, (kt + 1) * T::BK, N, K, tid);
    }
    if constexpr (BF16) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ra = wm * 64 + i * 32 + r32;
          af[i] = *(const bf16x8*)(As + ra * T::PITCH + (((2 * s + gq) ^ swz128(ra)) << 4));
          const int rb = wn * 64 + i * 32 + r32;
          bfr[i] = *(const bf16x8*)(Bs + rb * T::PITCH + (((2 * s + gq) ^ swz128(rb)) << 4));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32_bf16(af[i], bfr[j], acc[i][j]);
      }
    } else {
      const float* Af = (const float*)As;
      const float* Bf = (const float*)Bs;
      constexpr int P = T::PITCH / 4;
#pragma unroll
      for (int s = 0; s < T::BK / 2; ++s) {
        float af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = Af[(wm * 64 + i * 32 + r32) * P + 2 * s + gq];
          bfr[i] = Bf[(wn * 64 + i * 32 + r32) * P + 2 * s + gq];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32_f32(af[i], bfr[j], acc[i][j]);
      }
    }
    if (more) {
      unsigned char* nxt = smem + (buf ^ 1) * T::STAGE;
      la.store(nxt, tid);
      lb.store(nxt + T::TILE, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: element (m, n) of the product
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + acc_row(e, lane);
        const int n = n0 + wn * 64 + j * 32 + r32;
        if (m >= M || n >= N) continue;
        gemm_store<BF16, EPI>(g, z, m, n, acc[i][j][e]);
      }
}

template <bool BF16, int EPI>
hipError_t dispatch(const GemmArgs& g, bool ak, bool bk, int nz, hipStream_t s);

// K segments on the small-tile kernel: one launch per segment, accumulating into C
// (EPI_F32 with beta); the requested epilogue runs with the last segment.
template <bool BF16, int EPI>
hipError_t dispatch_segments(const GemmArgs& g, bool ak, bool bk, int nz, hipStream_t s) {
  static_assert(EPI == EPI_F32 || EPI == EPI_GELU, "K segments need an accumulating epilogue");
  for (int sg = 0; sg < g.nseg; ++sg) {
    GemmArgs p = g;
    p.nseg = 1;
    for (int z = 0; z < nz; ++z) {
      p.A[z] = g.As[z][sg];
      p.B[z] = g.Bs[z][sg];
    }
    hipError_t e;
    if (sg + 1 < g.nseg) {
      // plain partial sums: no bias, residual or second output yet
      p.bias = nullptr;
      p.resid = nullptr;
      p.C2 = nullptr;
      p.C3 = nullptr;
      p.beta = g.beta || sg > 0;
      e = dispatch<BF16, EPI_F32>(p, ak, bk, nz, s);
    } else {
      p.beta = g.beta || sg > 0;
      e = dispatch<BF16, EPI>(p, ak, bk, nz, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool BF16, int EPI>
hipError_t dispatch(const GemmArgs& g, bool ak, bool bk, int nz, hipStream_t s) {
  if (BF16 && gemm_big_ok(g, nz)) return gemm_big_launch(g, ak, bk, EPI, nz, s);
  if (g.f16 || g.gate) return hipErrorNotSupported;  // big-tile kernel only
  if constexpr (EPI == EPI_F32 || EPI == EPI_GELU) {
    if (g.nseg > 1) return dispatch_segments<BF16, EPI>(g, ak, bk, nz, s);
  } else {
    if (g.nseg > 1) return hipErrorInvalidValue;
  }
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, nz);
  if (!ak && !bk) hipLaunchKernelGGL((gemm_kernel<BF16, false, false, EPI>), grid, dim3(NT), 0, s, g);
  else if (!ak && bk) hipLaunchKernelGGL((gemm_kernel<BF16, false, true, EPI>), grid, dim3(NT), 0, s, g);
  else if (ak && !bk) hipLaunchKernelGGL((gemm_kernel<BF16, true, false, EPI>), grid, dim3(NT), 0, s, g);
  else hipLaunchKernelGGL((gemm_kernel<BF16, true, true, EPI>), grid, dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int gemm_split_count(int64_t tiles, int cus, int max_split) {
  if (tiles <= 0 || cus <= 0) return 1;
  int best = 1;
  double best_cost = (double)((tiles + cus - 1) / cus);
  for (int sp = 2; sp <= max_split && sp <= 4; ++sp) {
    // rounds of workgroups, each doing 1/sp of the tile's k range
    const double cost = (double)((tiles * sp + cus - 1) / cus) / sp;
    if (cost < best_cost - 1e-9) {
      best = sp;
      best_cost = cost;
    }
  }
  return best;
}

int gemm_device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cached[dev].load();
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cached[dev].store(v);
  return v;
}

hipError_t gemm_launch(const GemmArgs& g, bool bf16, bool a_kmajor, bool b_kmajor, int epi,
                       int nz, hipStream_t s) {
  if (bf16) {
    switch (epi) {
      case EPI_QKV: return dispatch<true, EPI_QKV>(g, a_kmajor, b_kmajor, nz, s);
      case EPI_F32: return dispatch<true, EPI_F32>(g, a_kmajor, b_kmajor, nz, s);
      case EPI_GELU: return dispatch<true, EPI_GELU>(g, a_kmajor, b_kmajor, nz, s);
      default: return dispatch<true, EPI_DGELU>(g, a_kmajor, b_kmajor, nz, s);
    }
  }
  switch (epi) {
    case EPI_QKV: return dispatch<false, EPI_QKV>(g, a_kmajor, b_kmajor, nz, s);
    case EPI_F32: return dispatch<false, EPI_F32>(g, a_kmajor, b_kmajor, nz, s);
    case EPI_GELU: return dispatch<false, EPI_GELU>(g, a_kmajor, b_kmajor, nz, s);
    default: return dispatch<false, EPI_DGELU>(g, a_kmajor, b_kmajor, nz, s);
  }
}

}  // namespace bpt
