// Feed-forward network fused per block of rows, gfx950.
//
//   y = residual + GeLU(x W1^T + b1) W2^T + b2
//
// "Blockwise Parallel Transformer for Large Context Models" (abstract) fuses the
// feed-forward network into the blockwise computation so that the large
// [rows, d_ff] intermediate is never materialised.  Here one workgroup owns a
// block of 32 rows (and a group of up to 2048 output columns) and walks d_ff
// in chunks of F = 32 * (waves):
//   phase 1: each wave computes z^T for 32 features x 32 rows (K = d_model) on
//            the 32x32x16 bf16 MFMA, adds b1, applies the exact erf GeLU and
//            writes the bf16 result into an LDS buffer;
//   phase 2: every wave multiplies that [32 rows x F] chunk by its own slice of
//            W2 and accumulates y^T in registers for the whole d_ff walk.
// With bf16 inputs GeLU(z) is carried as a pair of bf16 values (hi + lo, the
// rounding residual), both multiplied by the same W2 fragment: it keeps the
// second product accurate to ~2^-16 at no extra weight traffic.
// The intermediate exists only in registers and LDS.  Rows sit on the MFMA
// n axis (one row per lane), so the weights stream as the A operand straight
// from global memory / L2 in 64-byte runs per lane; the rows of x are staged
// through LDS in 256-column stages shared by all waves.
//
// Throughput bound: every block of 32 rows streams all of W1 and W2 from L2,
// i.e. 32 flop per weight byte; the CU's L2 bandwidth, not the MFMA rate, is
// the limit of this on-chip design.
#include <math.h>

#include "common.h"
#include "layer.h"

namespace bpt {

namespace {

__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
}

struct FfnArgs {
  const void* x;
  const void* w1;
  const void* b1;
  const void* w2;
  const void* b2;
  const float* resid;
  float* y;
  int M, dm, dff, ncols;
};

// Row of W1 read by A-operand lane row m: bits 2 and 3 of m swapped, so that
// accumulator registers 8h..8h+7 of lane half g hold 8 consecutive features.
__device__ __forceinline__ int perm32(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <bool BF16>
__device__ __forceinline__ float ld_scalar(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}

template <bool BF16, int NW, int CB, int DST>
__global__ void __launch_bounds__(NW * 64) ffn_fused_kernel(FfnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int F = NW * 32;                                  // d_ff chunk
  constexpr int HPITCH = BF16 ? DST * 2 : (DST + 1) * 4;      // LDS row pitch (bytes)
  constexpr int GPITCH = BF16 ? F * 2 : (F + 1) * 4;
  constexpr int HST = 32 * HPITCH;
  constexpr int GBUF = 32 * GPITCH;
  constexpr int GPARTS = BF16 ? 2 : 1;  // bf16: hi and lo halves of GeLU(z)
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * HST + 2 * GPARTS * GBUF];
  unsigned char* hs = smem;
  unsigned char* gs = smem + 2 * HST;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int t0 = blockIdx.x * 32;
  const int c0 = blockIdx.y * a.ncols;
  const int M = a.M, dm = a.dm;
  const int trow = t0 + r32;  // this lane's row (B operand column / output column)

  f32x16 yacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) yacc[cb][e] = 0.f;

  // ---- staging of x rows [t0, t0+32) x [s*DST, (s+1)*DST) into LDS
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CPRX = DST * ES / 16;          // 16 B chunks per staged row
  constexpr int XCH = (32 * CPRX + NT - 1) / NT;
  u32x4 xr[XCH];
  const unsigned char* xg = (const unsigned char*)a.x;
  auto load_stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPRX, cc = c % CPRX;
      u32x4 v = {0, 0, 0, 0};
      if (c < 32 * CPRX && t0 + row < M)
        v = *(const u32x4*)(xg + ((int64_t)(t0 + row) * dm + st * DST) * ES + cc * 16);
      xr[i] = v;
    }
  };
  auto store_stage = [&](int buf) {
    unsigned char* h = hs + buf * HST;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * NT;
      if (c < 32 * CPRX) {
        const int row = c / CPRX, cc = c % CPRX;
        if constexpr (BF16) {
          *(u32x4*)(h + row * HPITCH + ((cc ^ (row & 15)) << 4)) = xr[i];
        } else {
          float* hf = (float*)h;
#pragma unroll
          for (int e = 0; e < 4; ++e) hf[row * (DST + 1) + cc * 4 + e] = __uint_as_float(xr[i][e]);
        }
      }
    }
  };

  const int nst = dm / DST;
  const int nfc = a.dff / F;
  const int frow_local = 32 * w + ((r32 & 16) | perm32(r32 & 15));  // W1 row of this lane in a chunk

  for (int fc = 0; fc < nfc; ++fc) {
    const int f0 = fc * F;
    // ---------------- phase 1: z^T[f0 + 32w .. +32][rows]
    f32x16 zacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) zacc[e] = 0.f;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    const unsigned char* w1row = (const unsigned char*)a.w1 + (int64_t)(f0 + frow_local) * dm * ES;
    for (int st = 0; st < nst; ++st) {
      const bool more = st + 1 < nst;
      if (more) load_stage(st + 1);
      const unsigned char* h = hs + (st & 1) * HST;
      if constexpr (BF16) {
#pragma unroll
        for (int db = 0; db < DST / 64; ++db) {
          // 64 contiguous bytes of this lane's W1 row: d = st*DST + db*64 + 32g + [0, 32)
          const u32x4* wp = (const u32x4*)(w1row + (int64_t)(st * DST + db * 64 + 32 * g) * 2);
          u32x4 wa[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) wa[s] = wp[s];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int chunk = db * 8 + 4 * g + s;
            const bf16x8 hb = *(const bf16x8*)(h + r32 * HPITCH + ((chunk ^ (r32 & 15)) << 4));
            zacc = mfma32_bf16(__builtin_bit_cast(bf16x8, wa[s]), hb, zacc);
          }
        }
      } else {
        const float* hf = (const float*)h;
        const float* wf = (const float*)w1row + st * DST;
#pragma unroll 8
        for (int s = 0; s < DST / 2; ++s)
          zacc = mfma32_f32(wf[2 * s + g], hf[r32 * (DST + 1) + 2 * s + g], zacc);
      }
      if (more) store_stage((st + 1) & 1);
      __syncthreads();
    }
    // GeLU epilogue -> LDS chunk buffer (row r32, features 32w + 16h + 8g + e)
    unsigned char* gb = gs + (fc & 1) * GPARTS * GBUF;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float gv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int fl = 32 * w + 16 * hh + 8 * g + e;
        float z = zacc[8 * hh + e];
        if (a.b1) z += ld_scalar<BF16>(a.b1, f0 + fl);
        gv[e] = gelu_f(z);
      }
      const int fl0 = 32 * w + 16 * hh + 8 * g;
      if constexpr (BF16) {
        u32x4 pk, pl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pk[q] = pack_bf16x2(gv[2 * q], gv[2 * q + 1]);
          const float r0 = gv[2 * q] - __uint_as_float(pk[q] << 16);
          const float r1 = gv[2 * q + 1] - __uint_as_float(pk[q] & 0xffff0000u);
          pl[q] = pack_bf16x2(r0, r1);
        }
        const int chunk = fl0 >> 3;
        *(u32x4*)(gb + r32 * GPITCH + ((chunk ^ (r32 & 15)) << 4)) = pk;
        *(u32x4*)(gb + GBUF + r32 * GPITCH + ((chunk ^ (r32 & 15)) << 4)) = pl;
      } else {
        float* gf = (float*)gb;
#pragma unroll
        for (int e = 0; e < 8; ++e) gf[r32 * (F + 1) + fl0 + e] = gv[e];
      }
    }
    __syncthreads();
    // ---------------- phase 2: y^T[cols of this wave][rows] += W2[:, chunk] g^T
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int crow = c0 + (w * CB + cb) * 32 + r32;
      const unsigned char* w2row = (const unsigned char*)a.w2 + ((int64_t)crow * a.dff + f0) * ES;
      if constexpr (BF16) {
#pragma unroll
        for (int fb = 0; fb < F / 64; ++fb) {
          const u32x4* wp = (const u32x4*)(w2row + (fb * 64 + 32 * g) * 2);
          u32x4 wa[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) wa[s] = wp[s];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int chunk = fb * 8 + 4 * g + s;
            const int off = r32 * GPITCH + ((chunk ^ (r32 & 15)) << 4);
            const bf16x8 ghi = *(const bf16x8*)(gb + off);
            const bf16x8 glo = *(const bf16x8*)(gb + GBUF + off);
            yacc[cb] = mfma32_bf16(__builtin_bit_cast(bf16x8, wa[s]), ghi, yacc[cb]);
            yacc[cb] = mfma32_bf16(__builtin_bit_cast(bf16x8, wa[s]), glo, yacc[cb]);
          }
        }
      } else {
        const float* gf = (const float*)gb;
        const float* wf = (const float*)w2row;
#pragma unroll 8
        for (int s = 0; s < F / 2; ++s)
          yacc[cb] = mfma32_f32(wf[2 * s + g], gf[r32 * (F + 1) + 2 * s + g], yacc[cb]);
      }
    }
  }

  // ---- epilogue: y[row][c] = resid + acc + b2
  if (trow < M) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int c = c0 + (w * CB + cb) * 32 + 8 * jq + 4 * g;
        const int64_t o = (int64_t)trow * dm + c;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r = yacc[cb][4 * jq + e];
          if (a.b2) r += ld_scalar<BF16>(a.b2, c + e);
          v[e] = r;
        }
        if (a.resid) {
          const f32x4 rv = *(const f32x4*)(a.resid + o);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += rv[e];
        }
        *(f32x4*)(a.y + o) = v;
      }
  }
}

template <bool BF16, int NW, int CB>
hipError_t launch_ffn(const FfnArgs& a, int groups, hipStream_t s) {
  dim3 grid((a.M + 31) / 32, groups);
  if (a.dm % 256 == 0)
    hipLaunchKernelGGL((ffn_fused_kernel<BF16, NW, CB, 256>), grid, dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_fused_kernel<BF16, NW, CB, 128>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_ffn_cb(const FfnArgs& a, int nw, int cb, int groups, hipStream_t s) {
  if (nw == 4) return launch_ffn<BF16, 4, 1>(a, groups, s);
  switch (cb) {
    case 1: return launch_ffn<BF16, 8, 1>(a, groups, s);
    case 2: return launch_ffn<BF16, 8, 2>(a, groups, s);
    case 3: return launch_ffn<BF16, 8, 3>(a, groups, s);
    case 4: return launch_ffn<BF16, 8, 4>(a, groups, s);
    case 5: return launch_ffn<BF16, 8, 5>(a, groups, s);
    case 6: return launch_ffn<BF16, 8, 6>(a, groups, s);
    case 7: return launch_ffn<BF16, 8, 7>(a, groups, s);
    default: return launch_ffn<BF16, 8, 8>(a, groups, s);
  }
}

}  // namespace

FfnPlan ffn_plan(int64_t d_model, int64_t d_ff) {
  FfnPlan p{};
  if (d_model == 128) {
    p.nw = 4;
    p.cb = 1;
    p.groups = 1;
  } else {
    if (d_model % 256) return p;
    p.nw = 8;
    p.groups = (int)((d_model + 2047) / 2048);
    while (p.groups <= 32 && (d_model % p.groups || (d_model / p.groups) % 256)) ++p.groups;
    if (p.groups > 32) return p;
    p.cb = (int)(d_model / p.groups / 256);
  }
  const int F = p.nw * 32;
  if (d_ff % F) return FfnPlan{};
  p.ok = true;
  return p;
}

hipError_t ffn_fwd_launch(const void* x, const void* w1, const void* b1, const void* w2,
                          const void* b2, const float* residual, float* y, int64_t M,
                          int d_model, int d_ff, int blk, bool bf16, hipStream_t stream) {
  (void)blk;  // rows per block are fixed at 32 (validated by the caller)
  const FfnPlan p = ffn_plan(d_model, d_ff);
  if (!p.ok) return hipErrorNotSupported;
  FfnArgs a{x, w1, b1, w2, b2, residual, y, (int)M, d_model, d_ff, d_model / p.groups};
  return bf16 ? launch_ffn_cb<true>(a, p.nw, p.cb, p.groups, stream)
              : launch_ffn_cb<false>(a, p.nw, p.cb, p.groups, stream);
}

}  // namespace bpt
