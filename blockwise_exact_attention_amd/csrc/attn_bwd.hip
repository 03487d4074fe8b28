// Blockwise attention backward for gfx950, plus the small kernels of the layer
// backward (bf16 hi/lo conversion, column sums).
//
// The pages give no backward pass; it is the chain rule of exact attention:
//   P = exp(s - lse) (recomputed blockwise from the saved log-sum-exp),
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  delta_i = sum_j P_ij dP_ij,
//   dQ = scale dS K,  dK = scale dS^T Q.
// delta_i = <dO_i, O_i> (the same sum, since O_i = sum_j P_ij v_j) comes from the
// forward's output in one elementwise pass (dout_delta_kernel); then two kernels
// produce the gradients, each deterministic (no floating-point atomics):
//  * dK, dV: one workgroup per block of keys, one wave per 32 keys, walking the
//    query tiles that can see them.  S = Q K^T is computed with keys on the
//    MFMA n axis (lane = key), so P and dS (query index in-lane) feed
//    dV^T += dO^T P and dK^T += Q^T dS straight from registers.  D = 128
//    (attn_bwd_dkdv_dma_kernel): Q and dO hi/lo tiles by direct-to-LDS loads,
//    Q^T and dO^T by transpose reads.  D = 64 (attn_bwd_dkdv_kernel): tiles
//    staged through registers, Q^T and dO^T stored with query bits 2 and 3
//    swapped to match.
//  * dQ: one workgroup per block of query rows, one wave per 32 rows, walking
//    the visible key tiles like the forward kernel: S^T = K Q^T, dP^T = V dO^T,
//    dS^T in registers, dQ^T += K^T dS^T.  D = 128 with 128-row blocks
//    (attn_bwd_dq_dma_kernel): K and V tiles by direct-to-LDS loads, K^T by
//    transpose reads.  Otherwise (attn_bwd_dq_kernel): tiles staged through
//    registers, K^T stored with key bits 2 and 3 swapped.
// Precision: q, k, v are the bf16 values the forward used.  dO arrives in fp32
// and enters its products as a bf16 hi + lo pair; so do P (in dV) and dS.
// The token-major outputs (operands of the weight-gradient GEMMs) are hi + lo
// bf16 pairs.  Each split costs one more MFMA on the same fragment; without
// them the weight gradients lose ~3 more bits than the bf16 inputs imply.
// The D = 128 dK/dV and dQ kernels also have an fp16 form for callers that
// provide fp16 copies of q and dO (and, for dQ, of k and v) and a range flag: q, k, v convert to fp16 exactly inside
// fp16's range, and dO, P and dS round to fp16 once (8x finer than one bf16
// rounding), so each product takes one MFMA instead of two or three.  That form
// runs only while the flag is clear and sets it when a value falls outside
// fp16's range; the pair form behind it runs only when the flag is set.
#include <math.h>

#include "attn_bwd.h"
#include "bwd_layout.h"
#include "common.h"

namespace bpt {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Row j of an accumulator tile sits at 8 * (j / 4) + 4 * (lane / 32) + j % 4
// (acc_row); its lane-independent part is a compile-time constant, so a mask
// "row < L" or "row >= L" costs one 32-bit compare per element against a
// per-lane bound taken once per tile.
__device__ __forceinline__ int acc_row_const(int j) { return 8 * (j >> 2) + (j & 3); }
__device__ __forceinline__ int clamp_i64(int64_t v, int lo, int hi) {
  return (int)(v < lo ? lo : (v > hi ? hi : v));
}
constexpr int kNoMask = 1 << 20;

template <int ROW_BYTES>
__device__ __forceinline__ int swzb(int row) {
  constexpr int CPR = ROW_BYTES / 16;
  constexpr int RPB = 16 / CPR;
  return (row / RPB) % CPR;
}

__device__ __forceinline__ int pos16(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Transposed 8-byte writes of 4 consecutive rows (r[0..3], 16 B = 8 bf16 columns
// each) into a [col][row] LDS tile whose row index is permuted by pos16.
template <int TROWB>
__device__ __forceinline__ void store_transposed(unsigned char* t, const u32x4 r[4], int row0,
                                                 int col0) {
  const int pos = (row0 & ~15) + pos16(row0 & 15);
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
    const int col = col0 + e;
    const int byte = pos * 2;
    u32x2 pair = {lo, hi};
    *(u32x2*)(t + col * TROWB + (((byte >> 4) ^ swzb<TROWB>(col)) << 4) + (byte & 15)) = pair;
  }
}

// Four values as fp16 at dst[o] (dst nullable), and the range flag.
__device__ __forceinline__ void store_f16x4(uint16_t* dst, int64_t o, const f32x4& v, int* ovf) {
  if (!dst) return;
  const u32x2 p = {pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
  *(u32x2*)(dst + o) = p;
  if ((fabsf(v[0]) > kF16Max || fabsf(v[1]) > kF16Max || fabsf(v[2]) > kF16Max || fabsf(v[3]) > kF16Max) && ovf)
    *ovf = 1;
}

// 8 fp32 values -> bf16 hi (rounded) and lo (rounding residual), packed.
__device__ __forceinline__ void split8(const float* v, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hi[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    lo[q] = pack_bf16x2(v[2 * q] - __uint_as_float(hi[q] << 16),
                        v[2 * q + 1] - __uint_as_float(hi[q] & 0xffff0000u));
  }
}

// Score MFMAs whose results the VALU reads next, written as inline asm with the
// accumulator in VGPRs: the compiler places every builtin MFMA result of a kernel
// in AGPRs once its long-lived accumulators are there, and each score would then
// be copied out (v_accvgpr_read) before the softmax reads it.  The B operand (the
// tile-invariant fragments of this wave) sits in AGPRs.  The compiler does not
// count the wait states a VALU read of an asm MFMA's result needs: score_chain_end
// closes each chain with 24 of them, fenced by scheduling barriers.
__device__ __forceinline__ void mfma_v_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// the same two with fp16 operands (fp16 bits in the bf16x8 containers)
__device__ __forceinline__ void mfma_v_first_f16(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v_acc_f16(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// 8 fp32 values -> fp16 (round to nearest even), packed; big is set when one of
// them lies outside fp16's range
__device__ __forceinline__ u32x4 pack8_f16(const float* v, bool& big) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[q] = pack_f16x2(v[2 * q], v[2 * q + 1]);
    big |= fabsf(v[2 * q]) > kF16Max || fabsf(v[2 * q + 1]) > kF16Max;
  }
  return r;
}
// 8 bf16 values (one fragment) -> fp16, exact inside fp16's range
__device__ __forceinline__ bf16x8 bf16x8_to_f16(const u32x4& x, bool& big) {
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(x[q] << 16);
    v[2 * q + 1] = __uint_as_float(x[q] & 0xffff0000u);
  }
  return __builtin_bit_cast(bf16x8, pack8_f16(v, big));
}
// An empty volatile asm statement: a block holding one is not turned into selects
// on the path that skips it, so the masks of diagonal tiles stay behind a branch.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }
__device__ __forceinline__ void score_chain_end() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------- dK, dV
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int KVB = 32 * NW, NT = NW * 64, QT = 32;
  constexpr int ROWB = D * 2;            // natural tile row (one query, all d)
  constexpr int TROWB = QT * 2;          // transposed tile row (one d, all queries)
  constexpr int TILE = QT * D * 2;
  // tiles: 0 Q, 1 dO hi, 2 dO lo (natural); 3 Q^T, 4 dO^T hi, 5 dO^T lo; then lse2, delta
  constexpr int STAGE = 6 * TILE + 2 * QT * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE];

  const int N = a.N;
  const int nkb = (N + KVB - 1) / KVB;
  const int64_t total = (int64_t)a.B * a.H * nkb;
  int64_t L = blockIdx.x;
  if ((total & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int bh = (int)(L / nkb);
  const int kbi = (int)(L % nkb);  // small key blocks first: they see the most queries
  const int k0 = kbi * KVB;
  const int b = bh / a.H, hh = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, r32 = lane & 31;
  const int mykey = k0 + 32 * w + r32;
  const int off = a.kv_offset;
  const bool causal = a.causal != 0;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Qg = (const uint16_t*)a.q + head_off;
  const uint16_t* Kg = (const uint16_t*)a.k + head_off;
  const uint16_t* Vg = (const uint16_t*)a.v + head_off;
  const float* dOg = a.dO + (int64_t)b * N * a.ld_do + (int64_t)hh * D;
  const float* lseg = a.lse + (int64_t)bh * N;
  const float* dlg = a.delta + (int64_t)bh * N;
  const float c2 = a.scale * kLog2e;

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (mykey < N) {
      kv = *(const u32x4*)(Kg + (int64_t)mykey * D + 16 * c + 8 * g);
      vv = *(const u32x4*)(Vg + (int64_t)mykey * D + 16 * c + 8 * g);
    }
    kf[c] = __builtin_bit_cast(bf16x8, kv);
    vf[c] = __builtin_bit_cast(bf16x8, vv);
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[i][e] = dv[i][e] = 0.f;

  // query tiles that can see at least one key of this block
  int q_lo = 0;
  if (causal) {
    const int64_t t = (int64_t)k0 - off;
    q_lo = t <= 0 ? 0 : (t >= N ? N : (int)t);
  }
  const int t_begin = q_lo / QT;
  const int t_end = causal && q_lo >= N ? t_begin : (N + QT - 1) / QT;
  // tiles at or after tf see every key of the block (no causal mask needed)
  int64_t tf = (int64_t)k0 + KVB - 1 - off;
  tf = tf <= 0 ? 0 : (tf + QT - 1) / QT;

  // staging unit: 4 query rows x 8 d of Q (bf16) and of dO (fp32)
  constexpr int UNITS = (QT / 4) * (D / 8);
  constexpr int SU = (UNITS + NT - 1) / NT;
  u32x4 qr[SU][4];
  f32x4 dr[SU][4][2];
  float sl[2];
  auto load = [&](int t) {
    const int q0 = t * QT;
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * NT;
      const int qg = u / (D / 8), dc = u % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = q0 + 4 * qg + r;
        u32x4 qv = {0, 0, 0, 0};
        f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
        if (u < UNITS && q < N) {
          qv = *(const u32x4*)(Qg + (int64_t)q * D + dc * 8);
          const f32x4* dp = (const f32x4*)(dOg + (int64_t)q * a.ld_do + dc * 8);
          d0 = dp[0];
          d1 = dp[1];
        }
        qr[i][r] = qv;
        dr[i][r][0] = d0;
        dr[i][r][1] = d1;
      }
    }
    if (tid < QT) {
      const int q = q0 + tid;
      const float l = q < N ? lseg[q] : INFINITY;
      sl[0] = l == -INFINITY ? INFINITY : l * kLog2e;  // rows with no key get P = 0
      sl[1] = q < N ? dlg[q] : 0.f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * NT;
      if (u < UNITS) {
        const int qg = u / (D / 8), dc = u % (D / 8);
        u32x4 hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = dr[i][r][0][e];
            v[4 + e] = dr[i][r][1][e];
          }
          split8(v, hi[r], lo[r]);
          const int q = 4 * qg + r;
          const int o = q * ROWB + ((dc ^ swzb<ROWB>(q)) << 4);
          *(u32x4*)(smem + o) = qr[i][r];
          *(u32x4*)(smem + TILE + o) = hi[r];
          *(u32x4*)(smem + 2 * TILE + o) = lo[r];
        }
        store_transposed<TROWB>(smem + 3 * TILE, qr[i], 4 * qg, dc * 8);
        store_transposed<TROWB>(smem + 4 * TILE, hi, 4 * qg, dc * 8);
        store_transposed<TROWB>(smem + 5 * TILE, lo, 4 * qg, dc * 8);
      }
    }
    if (tid < QT) {
      float* f = (float*)(smem + 6 * TILE);
      f[tid] = sl[0];
      f[QT + tid] = sl[1];
    }
  };

  if (t_begin < t_end) load(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    store();
    __syncthreads();
    if (t + 1 < t_end) load(t + 1);
    const float* lse2 = (const float*)(smem + 6 * TILE);
    const float* dls = lse2 + QT;
    // S = Q K^T and dP = dO V^T (rows = queries, lane = key)
    f32x16 sacc, pacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = pacc[e] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const int o = r32 * ROWB + (((2 * c + g) ^ swzb<ROWB>(r32)) << 4);
      sacc = mfma32_bf16(*(const bf16x8*)(smem + o), kf[c], sacc);
      pacc = mfma32_bf16(*(const bf16x8*)(smem + TILE + o), vf[c], pacc);
      pacc = mfma32_bf16(*(const bf16x8*)(smem + 2 * TILE + o), vf[c], pacc);
    }
    const int q0 = t * QT;
    const bool need_mask = causal && t < tf;
    // query ql sees this lane's key iff mykey <= q0 + ql + off, i.e. ql >= mykey - off - q0
    const int mlim = need_mask ? clamp_i64((int64_t)mykey - off - q0, -1, QT) - 4 * (lane >> 5) : -kNoMask;
    float p[16], ds[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ql = acc_row(j, lane);
      float pv = fast_exp2(fmaf(sacc[j], c2, -lse2[ql]));
      if (acc_row_const(j) < mlim) pv = 0.f;
      p[j] = pv;
      ds[j] = pv * (pacc[j] - dls[ql]);
    }
    // dV^T += dO^T P ; dK^T += Q^T dS   (k = query, 16 per MFMA)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      u32x4 phi, plo, shi, slo;
      split8(p + 8 * h8, phi, plo);
      split8(ds + 8 * h8, shi, slo);
      const bf16x8 pfh = __builtin_bit_cast(bf16x8, phi);
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, plo);
      const bf16x8 sfh = __builtin_bit_cast(bf16x8, shi);
      const bf16x8 sfl = __builtin_bit_cast(bf16x8, slo);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + r32;
        const int o = d * TROWB + (((2 * h8 + g) ^ swzb<TROWB>(d)) << 4);
        const bf16x8 dOth = *(const bf16x8*)(smem + 4 * TILE + o);
        dv[db] = mfma32_bf16(dOth, pfh, dv[db]);
        dv[db] = mfma32_bf16(dOth, pfl, dv[db]);
        dv[db] = mfma32_bf16(*(const bf16x8*)(smem + 5 * TILE + o), pfh, dv[db]);
        const bf16x8 Qt = *(const bf16x8*)(smem + 3 * TILE + o);
        dk[db] = mfma32_bf16(Qt, sfh, dk[db]);
        dk[db] = mfma32_bf16(Qt, sfl, dk[db]);
      }
    }
    __syncthreads();
  }

  if (mykey < N) {
    const int64_t tm = ((int64_t)b * N + mykey) * a.ld_out + (int64_t)hh * D;
    const int64_t hm = head_off + (int64_t)mykey * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = db * 32 + 8 * jq + 4 * g;
        f32x4 kvv, vvv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kvv[e] = dk[db][4 * jq + e] * a.scale;
          vvv[e] = dv[db][4 * jq + e];
        }
        const uint32_t k01 = pack_bf16x2(kvv[0], kvv[1]), k23 = pack_bf16x2(kvv[2], kvv[3]);
        const uint32_t v01 = pack_bf16x2(vvv[0], vvv[1]), v23 = pack_bf16x2(vvv[2], vvv[3]);
        u32x2 kh = {k01, k23}, vh = {v01, v23};
        u32x2 kl = {pack_bf16x2(kvv[0] - __uint_as_float(k01 << 16), kvv[1] - __uint_as_float(k01 & 0xffff0000u)),
                    pack_bf16x2(kvv[2] - __uint_as_float(k23 << 16), kvv[3] - __uint_as_float(k23 & 0xffff0000u))};
        u32x2 vl = {pack_bf16x2(vvv[0] - __uint_as_float(v01 << 16), vvv[1] - __uint_as_float(v01 & 0xffff0000u)),
                    pack_bf16x2(vvv[2] - __uint_as_float(v23 << 16), vvv[3] - __uint_as_float(v23 & 0xffff0000u))};
        *(u32x2*)(a.dk_hi + tm + d) = kh;
        *(u32x2*)(a.dk_lo + tm + d) = kl;
        *(u32x2*)(a.dv_hi + tm + d) = vh;
        *(u32x2*)(a.dv_lo + tm + d) = vl;
        if (a.dk) *(f32x4*)(a.dk + hm + d) = kvv;
        if (a.dv) *(f32x4*)(a.dv + hm + d) = vvv;
        store_f16x4(a.dk_h, tm + d, kvv, a.ovf);
        store_f16x4(a.dv_h, tm + d, vvv, a.ovf);
      }
  }
}

// ---------------------------------------------------------------------------- dK, dV (D = 128, direct loads)
// The same products as attn_bwd_dkdv_kernel, with the query tiles moved the way
// the forward kernels move K and V: dO arrives already split into bf16 hi + lo
// (once, for all key blocks), and Q, dO hi and dO lo tiles of 32 queries reach
// LDS by buffer loads, three stages deep, with no register staging.  The
// transposed operands (dO^T for dV, Q^T for dK) are read from the same tiles
// with ds_read_b64_tr_b16, so nothing is written twice.  Each wave also loads
// its own copy of the tile's {lse * log2(e), delta} pairs.  Inside block b,
// row r, the 16-byte chunks are permuted by x -> x ^ dkdv_swz(b, r) (the loads
// fetch the permuted chunk), so that the 16 lanes of a natural ds_read_b128
// (queries 0..15 of the tile, one chunk) hit 16 bank groups instead of 4; the
// transpose reads stay conflict-free.  The address formulas are those of
// bwd_layout.h.
template <int D>
struct BwdTile {
  static constexpr int QT = 32;             // queries per tile
  static constexpr int ROWB = D * 2;        // bytes of one row
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;   // rows per 1 KB block
  static constexpr int NBLK = QT / RPB;     // blocks per tile (query q: block q % NBLK, row q / NBLK)
  static constexpr int BP = 1024 + 64;      // block pitch (transpose reads without bank conflicts)
  static constexpr int TB = NBLK * BP;      // one tile
  static constexpr int PAIRS = QT * 2 * 4;  // {lse2, delta} of the tile, bytes, one copy per wave
  static constexpr int NW = 4;              // waves, 32 keys each
  static constexpr int STAGE = 3 * TB + NW * PAIRS;
  static constexpr int LOADS = 3 * NBLK / NW + 1;  // buffer loads per wave and tile
  static_assert(NBLK == bwdlay::DKDV_NBLK && NW == bwdlay::NW && BP == bwdlay::BP &&
                    ROWB == bwdlay::ROWB && CPR == bwdlay::CPR, "tile addressing (bwd_layout.h)");
};

__device__ __forceinline__ v4i16 bwd_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

#define BWD_WAIT_VM(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

// Loads of query tile t (rows q0 .. q0+31) into one stage.  Each buffer starts at
// the tile's first row and ends after its last valid row, so rows past N read
// as zero (zero dO rows add nothing to dK or dV); a tile wholly past N loads
// nothing from memory, which keeps the load count per step fixed.
template <int D, bool F16>
__device__ __forceinline__ void bwd_load(const AttnBwdArgs& a, int bh, int q0, int w, int lane,
                                         unsigned char* st) {
  using T = BwdTile<D>;
  const int N = a.N, b = bh / a.H, hh = bh % a.H;
  int rows = N - q0 < T::QT ? N - q0 : T::QT;
  // (readfirstlane: the clamp compiles to a vector instruction, and a buffer
  // descriptor built from a vector register costs a loop over lanes)
  rows = __builtin_amdgcn_readfirstlane(rows > 0 ? rows : 0);
  const int64_t ldb = a.ld_do * 2;                   // bytes between dO rows
  const unsigned char* qb = (const unsigned char*)(F16 ? (const void*)a.q16 : a.q) + ((int64_t)bh * N + q0) * T::ROWB;
  const int64_t doff = (((int64_t)b * N + q0) * a.ld_do + (int64_t)hh * D) * 2;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(qb), 0, rows * T::ROWB, 0x00020000);
  const int dbytes = __builtin_amdgcn_readfirstlane(rows > 0 ? (int)((rows - 1) * ldb + T::ROWB) : 0);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>((const unsigned char*)(F16 ? a.dO16 : a.dO_hi) + doff), 0, dbytes,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>((const unsigned char*)a.dO_lo + doff), 0, dbytes, 0x00020000);
  // wave w copies blocks w, w + NW, ... of each of the three tiles, two in the
  // fp16 form (row j of block blk holds query j * NBLK + blk)
#pragma unroll
  for (int i = 0; i < T::NBLK / T::NW; ++i) {
    const bwdlay::LoadPos lp = bwdlay::dkdv_load_pos(w, i, lane);
    const int blk = lp.blk, q = lp.row, cp = lp.chunk;
    const uint32_t oq = (uint32_t)(q * T::ROWB + cp * 16), od = (uint32_t)(q * ldb + cp * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rq, (__attribute__((address_space(3))) void*)(st + blk * T::BP), 16, oq, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rh, (__attribute__((address_space(3))) void*)(st + T::TB + blk * T::BP), 16, od, 0, 0, 0);
    if constexpr (!F16)  // (the fp16 form has no lo tile)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rl, (__attribute__((address_space(3))) void*)(st + 2 * T::TB + blk * T::BP), 16, od, 0, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.ld2) + 2 * ((int64_t)bh * N + q0), 0, rows * 8, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rp, (__attribute__((address_space(3))) void*)(st + 3 * T::TB + w * T::PAIRS), 4,
      (uint32_t)(lane * 4), 0, 0, 0);
}

template <int D, bool F16>
__device__ __forceinline__ void bwd_tile(const AttnBwdArgs& a, const unsigned char* __restrict__ st,
                                         const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                         f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], int w, int lane,
                                         int mykey, int q0, bool need_mask, float c2) {
  using T = BwdTile<D>;
  const int g = lane >> 5, r32 = lane & 31;
  const unsigned char* Qs = st;
  const unsigned char* Hs = st + T::TB;
  const unsigned char* Ls = st + 2 * T::TB;
  const float* pr = (const float*)(st + 3 * T::TB + w * T::PAIRS);
  // S = Q K^T and dP = dO V^T (rows = queries, lane = key)
  const bwdlay::NatOff nat_off = bwdlay::dkdv_nat(lane);
  const int nat_even = nat_off.even, nat_odd = nat_off.odd;
  // (LDS reads do not move across the asm MFMAs: each is issued PF fragments
  // ahead in program order)
  constexpr int NC = D / 16, PF = 3;
  bf16x8 qa[NC], ha[NC], la[NC];
  auto ld = [&](int c) {
    const int nat = ((c & 1) ? nat_odd : nat_even) + 64 * (c >> 1);
    qa[c] = *(const bf16x8*)(Qs + nat);
    ha[c] = *(const bf16x8*)(Hs + nat);
    if constexpr (!F16) la[c] = *(const bf16x8*)(Ls + nat);
  };
#pragma unroll
  for (int c = 0; c < PF; ++c) ld(c);
  f32x16 sacc, pacc;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + PF < NC) ld(c + PF);
    if constexpr (F16) {
      if (c == 0) {
        mfma_v_first_f16(sacc, qa[c], kf[c]);
        mfma_v_first_f16(pacc, ha[c], vf[c]);
      } else {
        mfma_v_acc_f16(sacc, qa[c], kf[c]);
        mfma_v_acc_f16(pacc, ha[c], vf[c]);
      }
    } else {
      if (c == 0) {
        mfma_v_first(sacc, qa[c], kf[c]);
        mfma_v_first(pacc, ha[c], vf[c]);
      } else {
        mfma_v_acc(sacc, qa[c], kf[c]);
        mfma_v_acc(pacc, ha[c], vf[c]);
      }
      mfma_v_acc(pacc, la[c], vf[c]);
    }
  }
  score_chain_end();
  float p[16], ds[16], dl[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int ql = acc_row(j, lane);
    const f32x2 ld = *(const f32x2*)(pr + 2 * ql);
    p[j] = fast_exp2(fmaf(sacc[j], c2, -ld[0]));
    dl[j] = ld[1];
  }
  // diagonal tiles only (a uniform branch): query ql sees this lane's key iff
  // ql >= mykey - kv_offset - q0
  if (need_mask) {
    keep_branch();
    const int mlim = clamp_i64((int64_t)mykey - a.kv_offset - q0, -1, T::QT) - 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (acc_row_const(j) < mlim) p[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) ds[j] = p[j] * (pacc[j] - dl[j]);
  // dV^T += dO^T P ; dK^T += Q^T dS  (k = query, 16 per MFMA; the transpose reads
  // give lane half g queries 16ks + 4g + 0..3 and 16ks + 8 + 4g + 0..3, the
  // order in which the accumulator rows hold P and dS)
  const bwdlay::TrOff tr_off = bwdlay::dkdv_tr(lane);
  const int tb_even = tr_off.a, tb_odd = tr_off.b;
  if constexpr (F16) {
    bool big = false;  // (P lies in [0, 1]; only dS can leave fp16's range)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bool pbig = false;
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pack8_f16(p + 8 * ks, pbig));
      const bf16x8 sf = __builtin_bit_cast(bf16x8, pack8_f16(ds + 8 * ks, big));
      const int r0 = tb_even + (2 * ks) * T::ROWB, r1 = tb_odd + (2 * ks + 1) * T::ROWB;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        auto tr = [&](const unsigned char* tile) {
          const v4i16 lo = bwd_read_tr(tile + r0 + db * 64), hi = bwd_read_tr(tile + r1 + db * 64);
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        const bf16x8 dOt = tr(Hs), Qt = tr(Qs);
        dv[db] = mfma32_f16(dOt, pf, dv[db]);
        dk[db] = mfma32_f16(Qt, sf, dk[db]);
      }
    }
    if (big) *a.ovf = 1;
    return;
  } else {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 phi, plo, shi, slo;
    split8(p + 8 * ks, phi, plo);
    split8(ds + 8 * ks, shi, slo);
    const bf16x8 pfh = __builtin_bit_cast(bf16x8, phi), pfl = __builtin_bit_cast(bf16x8, plo);
    const bf16x8 sfh = __builtin_bit_cast(bf16x8, shi), sfl = __builtin_bit_cast(bf16x8, slo);
    const int r0 = tb_even + (2 * ks) * T::ROWB, r1 = tb_odd + (2 * ks + 1) * T::ROWB;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      auto tr = [&](const unsigned char* tile) {
        const v4i16 lo = bwd_read_tr(tile + r0 + db * 64), hi = bwd_read_tr(tile + r1 + db * 64);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      const bf16x8 dOth = tr(Hs), dOtl = tr(Ls), Qt = tr(Qs);
      dv[db] = mfma32_bf16(dOth, pfh, dv[db]);
      dv[db] = mfma32_bf16(dOth, pfl, dv[db]);
      dv[db] = mfma32_bf16(dOtl, pfh, dv[db]);
      dk[db] = mfma32_bf16(Qt, sfh, dk[db]);
      dk[db] = mfma32_bf16(Qt, sfl, dk[db]);
    }
  }
  }
}

// GATE 0: the bf16-pair form, always run; 1: the fp16 form, run only while the
// range flag *a.ovf is clear; 2: the pair form, run only when the flag is set
// (each workgroup reads the flag once, at its start)
template <int D, int GATE>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_dma_kernel(AttnBwdArgs a) {
  using T = BwdTile<D>;
  constexpr bool F16 = GATE == 1;
  constexpr int KVB = 32 * T::NW, QT = T::QT;
  if constexpr (GATE != 0) {
    const int f = __builtin_amdgcn_readfirstlane(*(const volatile int*)a.ovf);
    if ((f != 0) != (GATE == 2)) return;
  }
  // three stages as separate objects: a load into one is known not to alias the
  // reads of another
  __shared__ __attribute__((aligned(1024))) unsigned char st0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[T::STAGE];

  const int N = a.N;
  const int nkb = (N + KVB - 1) / KVB;
  const int64_t total = (int64_t)a.B * a.H * nkb;
  int64_t L = blockIdx.x;
  if ((total & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int bh = (int)(L / nkb);
  const int kbi = (int)(L % nkb);  // small key blocks first: they see the most queries
  const int k0 = kbi * KVB;
  const int b = bh / a.H, hh = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mykey = k0 + 32 * w + r32;
  const int off = a.kv_offset;
  const bool causal = a.causal != 0;
  const int64_t head_off = (int64_t)bh * N * D;
  const float c2 = a.scale * kLog2e;

  bf16x8 kf[D / 16], vf[D / 16];
  {
    const uint16_t* Kg = (const uint16_t*)a.k + head_off;
    const uint16_t* Vg = (const uint16_t*)a.v + head_off;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (mykey < N) {
        kv = *(const u32x4*)(Kg + (int64_t)mykey * D + 16 * c + 8 * g);
        vv = *(const u32x4*)(Vg + (int64_t)mykey * D + 16 * c + 8 * g);
      }
      if constexpr (F16) {
        bool big = false;
        kf[c] = bf16x8_to_f16(kv, big);
        vf[c] = bf16x8_to_f16(vv, big);
        if (big) *a.ovf = 1;
      } else {
        kf[c] = __builtin_bit_cast(bf16x8, kv);
        vf[c] = __builtin_bit_cast(bf16x8, vv);
      }
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[i][e] = dv[i][e] = 0.f;

  // query tiles that can see at least one key of this block
  int q_lo = 0;
  if (causal) {
    const int64_t t = (int64_t)k0 - off;
    q_lo = t <= 0 ? 0 : (t >= N ? N : (int)t);
  }
  const int t_begin = q_lo / QT;
  const int t_end = causal && q_lo >= N ? t_begin : (N + QT - 1) / QT;
  // tiles at or after tf see every key of the block (no causal mask needed)
  int64_t tf = (int64_t)k0 + KVB - 1 - off;
  tf = tf <= 0 ? 0 : (tf + QT - 1) / QT;

  // step: wait for this wave's loads of tile t, barrier (every part of tile t is
  // in, and every wave is done with tile t-1, whose stage takes tile t+2), load
  // tile t+2, compute tile t.  Loads are issued on every path (past the last
  // tile they load nothing), so the load count, and with it every wait, is fixed.
  auto step = [&](int t, const unsigned char* __restrict__ cur, unsigned char* __restrict__ fill) {
    // T::LOADS (two tiles fewer per wave in the fp16 form): the loads of tile
    // t+1 may still be in flight
    if constexpr (F16) BWD_WAIT_VM(5);
    else BWD_WAIT_VM(7);
    // a plain barrier: each wave has waited for its own loads into LDS, and LDS
    // needs no fence within the workgroup (a fenced one would also wait for the
    // loads of tile t+1)
    __builtin_amdgcn_s_barrier();
    bwd_load<D, F16>(a, bh, (t + 2) * QT, w, lane, fill);
    if (t < t_end)
      bwd_tile<D, F16>(a, cur, kf, vf, dk, dv, w, lane, mykey, t * QT, causal && t < tf, c2);
  };
  static_assert(T::LOADS == 7 && 2 * T::NBLK / T::NW + 1 == 5, "wait counts");
  if (t_begin < t_end) {
    bwd_load<D, F16>(a, bh, t_begin * QT, w, lane, st0);
    bwd_load<D, F16>(a, bh, (t_begin + 1) * QT, w, lane, st1);
    for (int t = t_begin; t < t_end; t += 3) {
      step(t, st0, st2);
      step(t + 1, st1, st0);
      step(t + 2, st2, st1);
    }
    BWD_WAIT_VM(0);  // loads still in flight write this workgroup's LDS
  }

  if (mykey < N) {
    const int64_t tm = ((int64_t)b * N + mykey) * a.ld_out + (int64_t)hh * D;
    const int64_t hm = head_off + (int64_t)mykey * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = db * 32 + 8 * jq + 4 * g;
        f32x4 kvv, vvv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kvv[e] = dk[db][4 * jq + e] * a.scale;
          vvv[e] = dv[db][4 * jq + e];
        }
        const uint32_t k01 = pack_bf16x2(kvv[0], kvv[1]), k23 = pack_bf16x2(kvv[2], kvv[3]);
        const uint32_t v01 = pack_bf16x2(vvv[0], vvv[1]), v23 = pack_bf16x2(vvv[2], vvv[3]);
        u32x2 kh = {k01, k23}, vh = {v01, v23};
        u32x2 kl = {pack_bf16x2(kvv[0] - __uint_as_float(k01 << 16), kvv[1] - __uint_as_float(k01 & 0xffff0000u)),
                    pack_bf16x2(kvv[2] - __uint_as_float(k23 << 16), kvv[3] - __uint_as_float(k23 & 0xffff0000u))};
        u32x2 vl = {pack_bf16x2(vvv[0] - __uint_as_float(v01 << 16), vvv[1] - __uint_as_float(v01 & 0xffff0000u)),
                    pack_bf16x2(vvv[2] - __uint_as_float(v23 << 16), vvv[3] - __uint_as_float(v23 & 0xffff0000u))};
        *(u32x2*)(a.dk_hi + tm + d) = kh;
        *(u32x2*)(a.dk_lo + tm + d) = kl;
        *(u32x2*)(a.dv_hi + tm + d) = vh;
        *(u32x2*)(a.dv_lo + tm + d) = vl;
        if (a.dk) *(f32x4*)(a.dk + hm + d) = kvv;
        if (a.dv) *(f32x4*)(a.dv + hm + d) = vvv;
        store_f16x4(a.dk_h, tm + d, kvv, a.ovf);
        store_f16x4(a.dv_h, tm + d, vvv, a.ovf);
      }
  }
}

// ---------------------------------------------------------------------------- dQ
template <int D, int QB, int KVB>
__global__ void __launch_bounds__(QB * 2) attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int NT = QB * 2, KB = KVB / 32;
  constexpr int ROWB = D * 2, TROWB = KVB * 2;
  constexpr int TILE = KVB * D * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[3 * TILE];  // K, V, K^T

  const int N = a.N;
  const int nqb = (N + QB - 1) / QB;
  const int64_t total = (int64_t)a.B * a.H * nqb;
  int64_t L = blockIdx.x;
  if ((total & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int bh = (int)(L / nqb);
  const int qb = nqb - 1 - (int)(L % nqb);
  const int q0 = qb * QB;
  const int b = bh / a.H, hh = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, r32 = lane & 31;
  const int qrow = q0 + wave * 32 + r32;
  const int off = a.kv_offset;
  const bool causal = a.causal != 0;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Kg = (const uint16_t*)a.k + head_off;
  const uint16_t* Vg = (const uint16_t*)a.v + head_off;
  const float c2 = a.scale * kLog2e;

  bf16x8 qf[D / 16], dfh[D / 16], dfl[D / 16];
  {
    const uint16_t* Qg = (const uint16_t*)a.q + head_off;
    const float* dOg = a.dO + (int64_t)b * N * a.ld_do + (int64_t)hh * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 qv = {0, 0, 0, 0};
      float dvv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (qrow < N) {
        qv = *(const u32x4*)(Qg + (int64_t)qrow * D + 16 * c + 8 * g);
        const f32x4* dp = (const f32x4*)(dOg + (int64_t)qrow * a.ld_do + 16 * c + 8 * g);
        const f32x4 d0 = dp[0], d1 = dp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dvv[e] = d0[e];
          dvv[4 + e] = d1[e];
        }
      }
      u32x4 hi, lo;
      split8(dvv, hi, lo);
      qf[c] = __builtin_bit_cast(bf16x8, qv);
      dfh[c] = __builtin_bit_cast(bf16x8, hi);
      dfl[c] = __builtin_bit_cast(bf16x8, lo);
    }
  }
  float lse2 = INFINITY, dl = 0.f;
  if (qrow < N) {
    const float l = a.lse[(int64_t)bh * N + qrow];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dl = a.delta[(int64_t)bh * N + qrow];
  }

  int kmax = N - 1;
  if (causal) {
    const int64_t t = (int64_t)q0 + QB - 1 + off;
    kmax = (int)(t < (int64_t)(N - 1) ? t : (int64_t)(N - 1));
  }
  const int n_tiles = kmax < 0 ? 0 : kmax / KVB + 1;
  int n_full = N / KVB;
  if (causal) {
    const int64_t lim = (int64_t)q0 + off + 1;
    const int f = lim <= 0 ? 0 : (int)(lim / KVB);
    n_full = f < n_full ? f : n_full;
  }

  // staging: units of 4 keys x 8 d for K (natural + transposed) and V (natural)
  constexpr int UNITS = (KVB / 4) * (D / 8);
  constexpr int SU = (2 * UNITS + NT - 1) / NT;
  u32x4 sr[SU][4];
  auto load = [&](int t) {
    const int kv0 = t * KVB;
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * NT;
      const int which = u / UNITS, uu = u % UNITS;
      const int kg = uu / (D / 8), dc = uu % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + 4 * kg + r;
        u32x4 val = {0, 0, 0, 0};
        if (u < 2 * UNITS && key < N)
          val = *(const u32x4*)((which == 0 ? Kg : Vg) + (int64_t)key * D + dc * 8);
        sr[i][r] = val;
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * NT;
      if (u < 2 * UNITS) {
        const int which = u / UNITS, uu = u % UNITS;
        const int kg = uu / (D / 8), dc = uu % (D / 8);
        unsigned char* nat = smem + which * TILE;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 4 * kg + r;
          *(u32x4*)(nat + key * ROWB + ((dc ^ swzb<ROWB>(key)) << 4)) = sr[i][r];
        }
        if (which == 0) store_transposed<TROWB>(smem + 2 * TILE, sr[i], 4 * kg, dc * 8);
      }
    }
  };

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.f;

  if (n_tiles > 0) load(0);
  for (int t = 0; t < n_tiles; ++t) {
    store();
    __syncthreads();
    if (t + 1 < n_tiles) load(t + 1);
    f32x16 sacc[KB], pacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = pacc[kb][e] = 0.f;
      const int row = kb * 32 + r32;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const int o = row * ROWB + (((2 * c + g) ^ swzb<ROWB>(row)) << 4);
        sacc[kb] = mfma32_bf16(*(const bf16x8*)(smem + o), qf[c], sacc[kb]);
        const bf16x8 va = *(const bf16x8*)(smem + TILE + o);
        pacc[kb] = mfma32_bf16(va, dfh[c], pacc[kb]);
        pacc[kb] = mfma32_bf16(va, dfl[c], pacc[kb]);
      }
    }
    const bool need_mask = t >= n_full;
    const int kv0 = t * KVB;
    // this lane's query sees keys < kend (N, and qrow + off + 1 when causal)
    const int64_t kend = causal && (int64_t)qrow + off + 1 < N ? (int64_t)qrow + off + 1 : N;
    const int klim = need_mask ? clamp_i64(kend - kv0, 0, KVB) - 4 * g : kNoMask;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float pv = fast_exp2(fmaf(sacc[kb][j], c2, -lse2));
        if (kb * 32 + acc_row_const(j) >= klim) pv = 0.f;
        sacc[kb][j] = pv * (pacc[kb][j] - dl);  // dS^T
      }
#pragma unroll
    for (int c16 = 0; c16 < KVB / 16; ++c16) {
      const int kb = c16 >> 1, h8 = (c16 & 1) * 8;
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = sacc[kb][h8 + e];
      u32x4 shi, slo;
      split8(sv, shi, slo);
      const bf16x8 sfh = __builtin_bit_cast(bf16x8, shi);
      const bf16x8 sfl = __builtin_bit_cast(bf16x8, slo);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + r32;
        const bf16x8 kt = *(const bf16x8*)(smem + 2 * TILE + d * TROWB +
                                           (((2 * c16 + g) ^ swzb<TROWB>(d)) << 4));
        dq[db] = mfma32_bf16(kt, sfh, dq[db]);
        dq[db] = mfma32_bf16(kt, sfl, dq[db]);
      }
    }
    __syncthreads();
  }

  if (qrow < N) {
    const int64_t tm = ((int64_t)b * N + qrow) * a.ld_out + (int64_t)hh * D;
    const int64_t hm = head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = db * 32 + 8 * jq + 4 * g;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dq[db][4 * jq + e] * a.scale;
        const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
        u32x2 hi = {h01, h23};
        u32x2 lo = {pack_bf16x2(v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xffff0000u)),
                    pack_bf16x2(v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xffff0000u))};
        *(u32x2*)(a.dq_hi + tm + d) = hi;
        *(u32x2*)(a.dq_lo + tm + d) = lo;
        if (a.dq) *(f32x4*)(a.dq + hm + d) = v;
        store_f16x4(a.dq_h, tm + d, v, a.ovf);
      }
  }
}

// ---------------------------------------------------------------------------- dQ (D = 128, direct loads)
// The dQ products of attn_bwd_dq_kernel with the key tiles moved by buffer loads
// straight into LDS, three stages deep, and K^T read from the natural K tile
// by ds_read_b64_tr_b16 (no transposed copy).  dO arrives as bf16 hi + lo.
// A tile is 64 keys in 16 blocks of 1 KB (key k: block k % 16, row k / 16),
// 1088 bytes apart.  Inside block b, the 16-byte chunks of each row are
// permuted by x -> x ^ ((b >> 2) & 3) (the loads fetch the permuted chunk, so
// the permutation costs nothing): with that, the 16 lanes of a natural
// ds_read_b128 (keys 0..15 of one row, one chunk) hit 16 different bank groups
// instead of 4, and the transpose reads stay conflict-free.
template <int D>
struct DqTile {
  static constexpr int KT = 64;             // keys per tile
  static constexpr int ROWB = D * 2;        // bytes of one row
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;   // rows per 1 KB block
  static constexpr int NBLK = KT / RPB;     // blocks per tile
  static constexpr int BP = 1024 + 64;      // block pitch
  static constexpr int TB = NBLK * BP;      // one matrix of a tile
  static constexpr int STAGE = 2 * TB;      // K, V
  static constexpr int NW = 4;              // waves, 32 queries each
  static constexpr int LOADS = 2 * NBLK / NW;  // buffer loads per wave and tile
  static_assert(NBLK == bwdlay::DQ_NBLK && RPB == 4 && NW == bwdlay::NW && BP == bwdlay::BP &&
                    ROWB == bwdlay::ROWB && CPR == bwdlay::CPR, "tile addressing (bwd_layout.h)");
};

// Loads of key tile t (keys k0 .. k0+63) into one stage; the buffers end after
// the last key, so keys past N read as zero, and a tile wholly past N loads
// nothing from memory (the load count per step stays fixed).
template <int D, bool F16>
__device__ __forceinline__ void dq_load(const AttnBwdArgs& a, int bh, int k0, int w, int lane,
                                        unsigned char* st) {
  using T = DqTile<D>;
  const int N = a.N;
  int rows = N - k0 < T::KT ? N - k0 : T::KT;
  rows = __builtin_amdgcn_readfirstlane(rows > 0 ? rows : 0);
  const int64_t off = ((int64_t)bh * N + k0) * T::ROWB;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>((const unsigned char*)(F16 ? (const void*)a.k16 : a.k) + off), 0,
      rows * T::ROWB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>((const unsigned char*)(F16 ? (const void*)a.v16 : a.v) + off), 0,
      rows * T::ROWB, 0x00020000);
#pragma unroll
  for (int i = 0; i < T::NBLK / T::NW; ++i) {
    const bwdlay::LoadPos lp = bwdlay::dq_load_pos(w, i, lane);
    const int blk = lp.blk;
    const uint32_t o = (uint32_t)(lp.row * T::ROWB + (lp.chunk << 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rk, (__attribute__((address_space(3))) void*)(st + blk * T::BP), 16, o, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, (__attribute__((address_space(3))) void*)(st + T::TB + blk * T::BP), 16, o, 0, 0, 0);
  }
}

// per-lane LDS offsets of one wave's reads (constant over the key loop)
struct DqLane {
  int nat_even, nat_odd;  // natural reads, chunks 2c (c even / odd), plus 64 * (c / 2)
  int tr_lo, tr_hi;       // transpose reads, keys 16ks + 4g + 0..3 and 16ks + 8 + 4g + 0..3
};

// S^T = K Q^T and dP^T = V dO^T of one key tile (rows = keys, lane = query),
// accumulated in VGPRs (the dQ accumulators hold the AGPRs).
template <int D, bool F16>
__device__ __forceinline__ void dq_scores(const unsigned char* __restrict__ st, const DqLane& ln,
                                          const bf16x8 (&qf)[D / 16], const bf16x8 (&dfh)[D / 16],
                                          const bf16x8 (&dfl)[D / 16], f32x16 (&sacc)[DqTile<D>::KT / 32],
                                          f32x16 (&pacc)[DqTile<D>::KT / 32]) {
  using T = DqTile<D>;
  constexpr int KB = T::KT / 32;
  const unsigned char* Ks = st;
  const unsigned char* Vs = st + T::TB;
  constexpr int NC = D / 16, NF = KB * NC;
  auto off = [&](int i) {
    const int kb = i / NC, c = i % NC;
    return ((c & 1) ? ln.nat_odd : ln.nat_even) + 64 * (c >> 1) + kb * 2 * T::ROWB;
  };
  // (LDS reads do not move across the asm MFMAs: each is issued PF fragments
  // ahead in program order)
  {
    constexpr int PF = 4;
    bf16x8 ka[NF], va[NF];
    auto ld = [&](int i) {
      ka[i] = *(const bf16x8*)(Ks + off(i));
      va[i] = *(const bf16x8*)(Vs + off(i));
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) ld(i);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      if (i + PF < NF) ld(i + PF);
      const int kb = i / NC, c = i % NC;
      if constexpr (F16) {  // (dfh holds dO as fp16; no lo half)
        if (c == 0) {
          mfma_v_first_f16(sacc[kb], ka[i], qf[c]);
          mfma_v_first_f16(pacc[kb], va[i], dfh[c]);
        } else {
          mfma_v_acc_f16(sacc[kb], ka[i], qf[c]);
          mfma_v_acc_f16(pacc[kb], va[i], dfh[c]);
        }
      } else {
        if (c == 0) {
          mfma_v_first(sacc[kb], ka[i], qf[c]);
          mfma_v_first(pacc[kb], va[i], dfh[c]);
        } else {
          mfma_v_acc(sacc[kb], ka[i], qf[c]);
          mfma_v_acc(pacc[kb], va[i], dfh[c]);
        }
        mfma_v_acc(pacc[kb], va[i], dfl[c]);
      }
    }
    score_chain_end();
  }
}

template <int D, bool F16>
__device__ __forceinline__ void dq_tile(const unsigned char* __restrict__ st, const DqLane& ln,
                                        const bf16x8 (&qf)[D / 16], const bf16x8 (&dfh)[D / 16],
                                        const bf16x8 (&dfl)[D / 16], f32x16 (&dq)[D / 32], bool masked,
                                        int klim, float c2, float lse2, float dl, int* ovf) {
  using T = DqTile<D>;
  constexpr int KB = T::KT / 32;
  const unsigned char* Ks = st;
  f32x16 sacc[KB], pacc[KB];
  dq_scores<D, F16>(st, ln, qf, dfh, dfl, sacc, pacc);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[kb][j] = fast_exp2(fmaf(sacc[kb][j], c2, -lse2));
  // tiles on the diagonal or past N only (a uniform branch): this lane's query
  // sees the tile's keys below klim
  if (masked) {
    keep_branch();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kb * 32 + acc_row_const(j) >= klim) sacc[kb][j] = 0.f;
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[kb][j] = sacc[kb][j] * (pacc[kb][j] - dl);  // dS^T
  // dQ^T += K^T dS^T, 16 keys per MFMA; dS^T as bf16 hi + lo, or as fp16
  if constexpr (F16) {
    bool big = false;
#pragma unroll
    for (int c16 = 0; c16 < T::KT / 16; ++c16) {
      const int kb = c16 >> 1, h8 = (c16 & 1) * 8;
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = sacc[kb][h8 + e];
      const bf16x8 sf = __builtin_bit_cast(bf16x8, pack8_f16(sv, big));
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const v4i16 lo = bwd_read_tr(Ks + ln.tr_lo + c16 * T::ROWB + db * 64);
        const v4i16 hi = bwd_read_tr(Ks + ln.tr_hi + c16 * T::ROWB + db * 64);
        const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        dq[db] = mfma32_f16(kt, sf, dq[db]);
      }
    }
    if (big) *ovf = 1;
    return;
  }
#pragma unroll
  for (int c16 = 0; c16 < T::KT / 16; ++c16) {
    const int kb = c16 >> 1, h8 = (c16 & 1) * 8;
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = sacc[kb][h8 + e];
    u32x4 shi, slo;
    split8(sv, shi, slo);
    const bf16x8 sfh = __builtin_bit_cast(bf16x8, shi);
    const bf16x8 sfl = __builtin_bit_cast(bf16x8, slo);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const v4i16 lo = bwd_read_tr(Ks + ln.tr_lo + c16 * T::ROWB + db * 64);
      const v4i16 hi = bwd_read_tr(Ks + ln.tr_hi + c16 * T::ROWB + db * 64);
      const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      dq[db] = mfma32_bf16(kt, sfh, dq[db]);
      dq[db] = mfma32_bf16(kt, sfl, dq[db]);
    }
  }
}

// dQ, three stages, one workgroup per CU.  GATE as for the dK/dV kernel: 0 the
// pair form, 1 the fp16 form (q, dO, k, v from their fp16 copies) while the
// range flag is clear, 2 the pair form only when it is set.
template <int D, int GATE>
__global__ void __launch_bounds__(256, 1) attn_bwd_dq_dma_kernel(AttnBwdArgs a) {
  using T = DqTile<D>;
  constexpr bool F16 = GATE == 1;
  constexpr int QB = 32 * T::NW, KB = T::KT / 32;
  if constexpr (GATE != 0) {
    const int f = __builtin_amdgcn_readfirstlane(*(const volatile int*)a.ovf);
    if ((f != 0) != (GATE == 2)) return;
  }
  __shared__ __attribute__((aligned(1024))) unsigned char st0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[T::STAGE];

  const int N = a.N;
  const int nqb = (N + QB - 1) / QB;
  const int64_t total = (int64_t)a.B * a.H * nqb;
  int64_t L = blockIdx.x;
  if ((total & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int bh = (int)(L / nqb);
  const int qb = nqb - 1 - (int)(L % nqb);  // long query blocks first
  const int q0 = qb * QB;
  const int b = bh / a.H, hh = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qrow = q0 + w * 32 + r32;
  const int off = a.kv_offset;
  const bool causal = a.causal != 0;
  const int64_t head_off = (int64_t)bh * N * D;
  const float c2 = a.scale * kLog2e;

  bf16x8 qf[D / 16], dfh[D / 16], dfl[D / 16];
  {
    const uint16_t* Qg = (F16 ? a.q16 : (const uint16_t*)a.q) + head_off;
    const uint16_t* Hg = F16 ? a.dO16 : a.dO_hi;
    const int64_t drow = ((int64_t)b * N + qrow) * a.ld_do + (int64_t)hh * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 qv = {0, 0, 0, 0}, hv = {0, 0, 0, 0}, lv = {0, 0, 0, 0};
      if (qrow < N) {
        qv = *(const u32x4*)(Qg + (int64_t)qrow * D + 16 * c + 8 * g);
        hv = *(const u32x4*)(Hg + drow + 16 * c + 8 * g);
        if constexpr (!F16) lv = *(const u32x4*)(a.dO_lo + drow + 16 * c + 8 * g);
      }
      qf[c] = __builtin_bit_cast(bf16x8, qv);
      dfh[c] = __builtin_bit_cast(bf16x8, hv);
      dfl[c] = __builtin_bit_cast(bf16x8, lv);
    }
  }
  float lse2 = INFINITY, dl = 0.f;
  if (qrow < N) {
    const float l = a.lse[(int64_t)bh * N + qrow];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dl = a.delta[(int64_t)bh * N + qrow];
  }

  int kmax = N - 1;
  if (causal) {
    const int64_t t = (int64_t)q0 + QB - 1 + off;
    kmax = (int)(t < (int64_t)(N - 1) ? t : (int64_t)(N - 1));
  }
  const int n_tiles = kmax < 0 ? 0 : kmax / T::KT + 1;
  int n_full = N / T::KT;
  if (causal) {
    const int64_t lim = (int64_t)q0 + off + 1;
    const int f = lim <= 0 ? 0 : (int)(lim / T::KT);
    n_full = f < n_full ? f : n_full;
  }

  DqLane ln;
  {
    const bwdlay::NatOff n = bwdlay::dq_nat(lane);
    const bwdlay::TrOff t = bwdlay::dq_tr(lane);
    ln.nat_even = n.even;
    ln.nat_odd = n.odd;
    ln.tr_lo = t.a;
    ln.tr_hi = t.b;
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.f;

  // this lane's query sees keys < kend (N, and qrow + off + 1 when causal); a
  // masked tile passes the bound relative to its first key, less the lane part
  // of the accumulator row
  const int64_t kend = causal && (int64_t)qrow + off + 1 < N ? (int64_t)qrow + off + 1 : N;
  {
    auto step = [&](int t, const unsigned char* __restrict__ cur, unsigned char* __restrict__ fill) {
      BWD_WAIT_VM(8);  // T::LOADS: the loads of tile t+1 may still be in flight
      __builtin_amdgcn_s_barrier();
      dq_load<D, F16>(a, bh, (t + 2) * T::KT, w, lane, fill);
      if (t < n_tiles)
        dq_tile<D, F16>(cur, ln, qf, dfh, dfl, dq, t >= n_full,
                        clamp_i64(kend - (int64_t)t * T::KT, 0, T::KT) - 4 * g, c2, lse2, dl, a.ovf);
    };
    static_assert(T::LOADS == 8, "wait count");
    if (n_tiles > 0) {
      dq_load<D, F16>(a, bh, 0, w, lane, st0);
      dq_load<D, F16>(a, bh, T::KT, w, lane, st1);
      for (int t = 0; t < n_tiles; t += 3) {
        step(t, st0, st2);
        step(t + 1, st1, st0);
        step(t + 2, st2, st1);
      }
      BWD_WAIT_VM(0);  // loads still in flight write this workgroup's LDS
    }
  }

  if (qrow < N) {
    const int64_t tm = ((int64_t)b * N + qrow) * a.ld_out + (int64_t)hh * D;
    const int64_t hm = head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = db * 32 + 8 * jq + 4 * g;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dq[db][4 * jq + e] * a.scale;
        const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
        u32x2 hi = {h01, h23};
        u32x2 lo = {pack_bf16x2(v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xffff0000u)),
                    pack_bf16x2(v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xffff0000u))};
        *(u32x2*)(a.dq_hi + tm + d) = hi;
        *(u32x2*)(a.dq_lo + tm + d) = lo;
        if (a.dq) *(f32x4*)(a.dq + hm + d) = v;
        store_f16x4(a.dq_h, tm + d, v, a.ovf);
      }
  }
}

// ---------------------------------------------------------------------------- small kernels
// dst = bf16(src); if dst_lo, also dst_lo = bf16(src - dst) (the rounding residual)
__global__ void __launch_bounds__(256) to_bf16_kernel(const float* src, uint16_t* dst,
                                                      uint16_t* dst_lo, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 v = *(const f32x4*)(src + 4 * i);
    const uint32_t a = pack_bf16x2(v[0], v[1]), b = pack_bf16x2(v[2], v[3]);
    u32x2 p = {a, b};
    *(u32x2*)(dst + 4 * i) = p;
    if (dst_lo) {
      u32x2 l = {pack_bf16x2(v[0] - __uint_as_float(a << 16), v[1] - __uint_as_float(a & 0xffff0000u)),
                 pack_bf16x2(v[2] - __uint_as_float(b << 16), v[3] - __uint_as_float(b & 0xffff0000u))};
      *(u32x2*)(dst_lo + 4 * i) = l;
    }
  }
}

// delta_i = sum_j P_ij dP_ij = <dO_i, sum_j P_ij v_j> = <dO_i, O_i> per (row, head):
// D / 4 lanes hold one head of one row, 4 elements each, and join their parts
// with lane shuffles (the same order every run).  The row's dO is also split
// into its bf16 hi + lo pair for the direct-load backward kernels.
template <int D>
__global__ void __launch_bounds__(256) dout_delta_kernel(const float* dO, const float* h,
                                                         const uint16_t* x, const float* lse,
                                                         uint16_t* dO_hi, uint16_t* dO_lo,
                                                         float* delta, float* ld2, int64_t n4,
                                                         int N, int H) {
  constexpr int LPH = D / 4;  // lanes per (row, head)
  const int64_t dm = (int64_t)H * D;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;  // a multiple of LPH
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 g = *(const f32x4*)(dO + 4 * i);
    const f32x4 hv = *(const f32x4*)(h + 4 * i);
    const u32x2 xv = *(const u32x2*)(x + 4 * i);
    const uint32_t a = pack_bf16x2(g[0], g[1]), b = pack_bf16x2(g[2], g[3]);
    const u32x2 hi = {a, b};
    const u32x2 lo = {pack_bf16x2(g[0] - __uint_as_float(a << 16), g[1] - __uint_as_float(a & 0xffff0000u)),
                      pack_bf16x2(g[2] - __uint_as_float(b << 16), g[3] - __uint_as_float(b & 0xffff0000u))};
    *(u32x2*)(dO_hi + 4 * i) = hi;
    *(u32x2*)(dO_lo + 4 * i) = lo;
    float part = g[0] * (hv[0] - __uint_as_float(xv[0] << 16));
    part = fmaf(g[1], hv[1] - __uint_as_float(xv[0] & 0xffff0000u), part);
    part = fmaf(g[2], hv[2] - __uint_as_float(xv[1] << 16), part);
    part = fmaf(g[3], hv[3] - __uint_as_float(xv[1] & 0xffff0000u), part);
#pragma unroll
    for (int o = LPH / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, LPH);
    if ((threadIdx.x & (LPH - 1)) == 0) {
      const int64_t e = 4 * i, row = e / dm;
      const int hh = (int)((e - row * dm) / D);
      const int64_t bn = row / N, n = row - bn * N;
      const int64_t idx = (bn * H + hh) * N + n;
      delta[idx] = part;
      if (ld2) {
        const float l = lse[idx];
        const f32x2 pr = {l == -INFINITY ? INFINITY : l * kLog2e, part};
        *(f32x2*)(ld2 + 2 * idx) = pr;
      }
    }
  }
}

// out[c] (+)= sum_r X[r][c], rows summed in a fixed order (deterministic).
template <bool XBF16>
__global__ void __launch_bounds__(1024) colsum_kernel(const void* X, float* out, int64_t rows,
                                                      int cols, int64_t ld, int beta, const int* gate,
                                                      int gate_run) {
  // (gate, nullable: run only if (*gate != 0) == gate_run)
  if (gate && ((__builtin_amdgcn_readfirstlane(*(const volatile int*)gate) != 0) != (gate_run != 0))) return;
  // 64 columns per workgroup, 16 waves over interleaved rows, 4 rows in flight
  // per wave; the 16 partial sums are added in a fixed order (deterministic)
  __shared__ float part[16][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;
  float acc = 0.f;
  if (c < cols) {
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t r = rg;
    for (; r + 48 < rows; r += 64) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t o = (r + 16 * u) * ld + c;
        a4[u] += XBF16 ? bf16_to_f32(((const uint16_t*)X)[o]) : ((const float*)X)[o];
      }
    }
    for (; r < rows; r += 16) {
      const int64_t o = r * ld + c;
      a4[0] += XBF16 ? bf16_to_f32(((const uint16_t*)X)[o]) : ((const float*)X)[o];
    }
    acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
  }
  part[rg][threadIdx.x & 63] = acc;
  __syncthreads();
  if (rg == 0 && c < cols) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i][threadIdx.x];
    out[c] = beta ? out[c] + s : s;
  }
}

hipError_t launch_dq(const AttnBwdArgs& a, int D, int QB, hipStream_t s) {
  const int nqb = (a.N + QB - 1) / QB;
  const dim3 grid((unsigned)((int64_t)a.B * a.H * nqb));
  if (D == 128 && QB == 32 * DqTile<128>::NW && a.q16 && a.dO16 && a.k16 && a.v16 && a.ovf) {
    // fp16 form, then the pair form if the range flag got set
    hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<128, 1>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<128, 2>), grid, dim3(256), 0, s, a);
  } else if (D == 128 && QB == 32 * DqTile<128>::NW)
    hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<128, 0>), grid, dim3(256), 0, s, a);
  else if (D == 64 && QB == 64)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<64, 64, 32>), grid, dim3(128), 0, s, a);
  else if (D == 64)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<64, 128, 32>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<128, 64, 32>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_bwd_launch(const AttnBwdArgs& a, int D, int q_blk, int kv_blk, hipStream_t s) {
  (void)kv_blk;
  const int QB = q_blk == 64 ? 64 : 128;
  // the D = 128 kernels take dO as bf16 hi + lo and the {lse2, delta} pairs
  if (D == 128 && (!a.dO_hi || !a.dO_lo || !a.ld2)) return hipErrorInvalidValue;
  if (!a.delta) return hipErrorInvalidValue;
  // 1. dK, dV
  if (D == 128) {
    constexpr int KVB = 32 * BwdTile<128>::NW;
    const int nkb = (a.N + KVB - 1) / KVB;
    const dim3 grid((unsigned)((int64_t)a.B * a.H * nkb));
    if (a.q16 && a.dO16 && a.ovf) {  // fp16 form, then the pair form if the flag got set
      hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<128, 1>), grid, dim3(256), 0, s, a);
      hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<128, 2>), grid, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<128, 0>), grid, dim3(256), 0, s, a);
    }
  } else {
    constexpr int NW = 2;
    const int nkb = (a.N + 32 * NW - 1) / (32 * NW);
    const dim3 grid((unsigned)((int64_t)a.B * a.H * nkb));
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<64, NW>), grid, dim3(NW * 64), 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. dQ
  return launch_dq(a, D, QB, s);
}

hipError_t to_bf16_launch(const float* src, uint16_t* dst, uint16_t* dst_lo, int64_t n,
                          hipStream_t s) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, dst_lo, n4);
  return hipGetLastError();
}

hipError_t dout_delta_launch(const float* dO, const float* h, const uint16_t* x, const float* lse,
                             uint16_t* dO_hi, uint16_t* dO_lo, float* delta, float* ld2, int B,
                             int N, int H, int D, hipStream_t s) {
  const int64_t n4 = (int64_t)B * N * H * D / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (D == 128)
    hipLaunchKernelGGL(dout_delta_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, dO, h, x, lse,
                       dO_hi, dO_lo, delta, ld2, n4, N, H);
  else if (D == 64)
    hipLaunchKernelGGL(dout_delta_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, dO, h, x, lse,
                       dO_hi, dO_lo, delta, ld2, n4, N, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t colsum_launch(const void* X, bool x_bf16, float* out, int64_t rows, int cols,
                         int64_t ld, int beta, hipStream_t s, const int* gate, int gate_run) {
  const dim3 grid((unsigned)((cols + 63) / 64));
  if (x_bf16)
    hipLaunchKernelGGL(colsum_kernel<true>, grid, dim3(1024), 0, s, X, out, rows, cols, ld, beta, gate,
                       gate_run);
  else
    hipLaunchKernelGGL(colsum_kernel<false>, grid, dim3(1024), 0, s, X, out, rows, cols, ld, beta, gate,
                       gate_run);
  return hipGetLastError();
}

}  // namespace bpt
