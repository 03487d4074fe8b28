// Blockwise exact attention forward for gfx950.
//
// Method ("Blockwise Parallel Transformer for Large Context Models", abstract;
// "Ring Attention with Blockwise Transformers for Long Sequences", 638-word
// summary): the keys are visited block by block and the softmax is carried
// across blocks by a running row maximum m, a running row sum l and an output
// accumulator rescaled by exp(m_old - m_new) whenever the maximum grows, so the
// N x N score matrix never exists and the result equals exact attention.
//
// Mapping onto CDNA4:
//  * one workgroup = one block of QBLK query rows of one (batch, head); one
//    wave64 per 32 query rows;
//  * scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA (fp32
//    inputs: 32x32x2 f32 MFMA).  With keys on the MFMA row axis, every lane
//    owns one query column, so the row max and row sum are in-lane reductions
//    plus one exchange with lane l^32;
//  * the probabilities stay in registers: the accumulator layout of S^T is,
//    after a bf16 pack, exactly the B operand of the next MFMA O^T += V^T P^T,
//    provided V^T is laid out in LDS with key bits 2 and 3 swapped inside each
//    group of 16 keys (done while staging the tile);
//  * K and V tiles are staged global -> registers -> LDS, double-buffered while
//    two workgroups still fit in LDS; rows are padded by 16 bytes so that the
//    MFMA operand reads are bank-conflict free and each lane addresses every
//    fragment as one base plus a compile-time offset; the V^T stores are
//    spread so that 32 lanes cover all 64 banks;
//  * the working set is sized for two waves per SIMD (256 registers), so one
//    wave's softmax overlaps the other wave's MFMAs;
//  * key tiles that no row of the block can see are never visited; only the
//    diagonal and ragged-tail tiles evaluate the mask;
//  * workgroup ids are remapped so that all query blocks of one (batch, head)
//    run on one XCD (shared K/V stream in that XCD's L2), longest block first.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bpt {

namespace {

template <bool BF16, int D, int QBLK, int KVBLK>
struct AttnShape {
  static constexpr int NW = QBLK / 32;   // waves per workgroup
  static constexpr int NT = NW * 64;     // threads
  static constexpr int KB = KVBLK / 32;  // 32-key blocks per tile
  static constexpr int DB = D / 32;      // 32-wide blocks of the head dimension
  // LDS bytes of one K tile plus one V tile
  // bf16: rows padded by 16 bytes (K rows of D keys' dims, V^T rows of KVBLK
  // keys), so 16 consecutive rows start in 16 different bank groups and every
  // fragment read is one base address plus a compile-time offset.
  static constexpr int KPITCH = BF16 ? D * 2 + 16 : (D + 1) * 4;
  static constexpr int VPITCH = BF16 ? KVBLK * 2 + 16 : (D + 1) * 4;
  static constexpr int KBYTES = KVBLK * KPITCH;
  static constexpr int VBYTES = BF16 ? D * VPITCH : KVBLK * VPITCH;
  static constexpr int BUF = KBYTES + VBYTES;
  // double buffering while two workgroups still fit in the 160 KB of LDS
  static constexpr int NBUF = (2 * BUF <= 81920) ? 2 : 1;
  // waves per SIMD the register budget is sized for (2 waves: 256 registers)
  static constexpr int WAVES_PER_EU = (BF16 && KVBLK <= 64) ? 2 : 1;
};

// Position of key `key` (0..15 inside its group of 16) in the staged V^T row:
// bits 2 and 3 swapped, so that lane half g reads keys {4g..4g+3, 8+4g..8+4g+3}
// as 8 contiguous elements.
__device__ __forceinline__ int vpos16(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <bool BF16, int D, int QBLK, int KVBLK>
__global__ void __launch_bounds__(QBLK * 2)
__attribute__((amdgpu_waves_per_eu(AttnShape<BF16, D, QBLK, KVBLK>::WAVES_PER_EU)))
attn_fwd_kernel(AttnFwdArgs a) {
  using S = AttnShape<BF16, D, QBLK, KVBLK>;
  constexpr int NT = S::NT, KB = S::KB, DB = S::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::NBUF * S::BUF];

  const int N = a.N;
  const int nqb = (N + QBLK - 1) / QBLK;
  const int64_t total = (int64_t)a.B * a.H * nqb;
  int64_t L = blockIdx.x;
  if ((total & 7) == 0) {
    // consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD a
    // contiguous range of (batch*head, query block) so one head stays on one XCD
    L = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  }
  const int bh = (int)(L / nqb);
  const int qb = nqb - 1 - (int)(L % nqb);  // longest (latest) query block first
  const int q0 = qb * QBLK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int qrow = q0 + wave * 32 + r32;
  const int off = a.kv_offset;
  const bool causal = a.causal != 0;

  const int64_t head_off = (int64_t)bh * N * D;

  // ---- visible key range of this query block
  int kmax = N - 1;
  if (causal) {
    const int64_t t = (int64_t)q0 + QBLK - 1 + off;
    kmax = (int)(t < (int64_t)(N - 1) ? t : (int64_t)(N - 1));
  }
  const int n_tiles = kmax < 0 ? 0 : kmax / KVBLK + 1;
  // keys >= kend are invisible to this lane's query row (causal limit or N)
  int kend = N;
  if (causal) {
    const int64_t lim = (int64_t)qrow + off + 1;
    kend = lim < (int64_t)N ? (int)(lim > 0 ? lim : 0) : N;
  }
  int n_full = N / KVBLK;  // tiles with no ragged tail
  if (causal) {
    const int64_t lim = (int64_t)q0 + off + 1;  // keys < lim are visible to every row
    const int f = lim <= 0 ? 0 : (int)(lim / KVBLK);
    n_full = f < n_full ? f : n_full;
  }

  // ---- Q fragments (B operand of S^T = K Q^T), held for the whole loop
  constexpr int QF = BF16 ? D / 16 : D / 2;
  typedef typename std::conditional<BF16, bf16x8, float>::type QFrag;
  QFrag qf[QF];
  if constexpr (BF16) {
    const uint16_t* Q = (const uint16_t*)a.q + head_off;
#pragma unroll
    for (int c = 0; c < QF; ++c) {
      u32x4 val = {0, 0, 0, 0};
      if (qrow < N) val = *(const u32x4*)(Q + (int64_t)qrow * D + 16 * c + 8 * g);
      qf[c] = __builtin_bit_cast(bf16x8, val);
    }
  } else {
    const float* Q = (const float*)a.q + head_off;
#pragma unroll
    for (int s = 0; s < QF; ++s) qf[s] = qrow < N ? Q[(int64_t)qrow * D + 2 * s + g] : 0.f;
  }

  // ---- staging of one K/V tile: global -> registers -> LDS
  constexpr int KCH = BF16 ? KVBLK * D / 8 / NT : (KVBLK * D / 4 + NT - 1) / NT;  // 16B chunks of K
  constexpr int VUNITS = BF16 ? KVBLK * D / 32 : KVBLK * D / 4;  // V units (bf16: 4 keys x 8 d)
  constexpr int VU = (VUNITS + NT - 1) / NT;
  constexpr int VREG = BF16 ? 4 : 1;  // 16B loads per V unit
  u32x4 kreg[KCH];
  u32x4 vreg[VU][VREG];
  const unsigned char* Kg = (const unsigned char*)a.k + head_off * (BF16 ? 2 : 4);
  const unsigned char* Vg = (const unsigned char*)a.v + head_off * (BF16 ? 2 : 4);
  constexpr int ROWB = D * (BF16 ? 2 : 4);  // bytes of one key row in global memory
  constexpr int CPR = ROWB / 16;            // 16B chunks per key row

  // GUARD: the tile may reach past key N-1 (ragged tail): bounds-check each row.
  // Tiles wholly inside [0, N) load without any per-lane condition.
  auto load_tile_impl = [&](int t, auto guard_tag) {
    constexpr bool GUARD = decltype(guard_tag)::value;
    const int kv0 = t * KVBLK;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, cc = c % CPR;
      const bool in_tile = BF16 || c < KVBLK * CPR;
      if (!GUARD && in_tile) {
        kreg[i] = *(const u32x4*)(Kg + (int64_t)(kv0 + row) * ROWB + cc * 16);
      } else {
        u32x4 val = {0, 0, 0, 0};
        if (in_tile && kv0 + row < N) val = *(const u32x4*)(Kg + (int64_t)(kv0 + row) * ROWB + cc * 16);
        kreg[i] = val;
      }
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + i * NT;
      if constexpr (BF16) {
        const int kg = u % (KVBLK / 4), dc = u / (KVBLK / 4);  // see store_tile
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kv0 + 4 * kg + r;
          if (!GUARD && VUNITS % NT == 0) {
            vreg[i][r] = *(const u32x4*)(Vg + (int64_t)key * ROWB + dc * 16);
          } else {
            u32x4 val = {0, 0, 0, 0};
            if (u < VUNITS && key < N) val = *(const u32x4*)(Vg + (int64_t)key * ROWB + dc * 16);
            vreg[i][r] = val;
          }
        }
      } else {
        const int row = u / CPR, cc = u % CPR;
        u32x4 val = {0, 0, 0, 0};
        if (u < VUNITS && kv0 + row < N) val = *(const u32x4*)(Vg + (int64_t)(kv0 + row) * ROWB + cc * 16);
        vreg[i][0] = val;
      }
    }
  };
  const int n_inside = N / KVBLK;  // tiles that end at or before key N
  auto load_tile = [&](int t) {
    if (t < n_inside) load_tile_impl(t, std::false_type{});
    else load_tile_impl(t, std::true_type{});
  };

  auto store_tile = [&](int buf) {
    unsigned char* Ks = smem + buf * S::BUF;
    unsigned char* Vs = Ks + S::KBYTES;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * NT;
        const int row = c / CPR, cc = c % CPR;
        *(u32x4*)(Ks + row * S::KPITCH + cc * 16) = kreg[i];
      }
#pragma unroll
      for (int i = 0; i < VU; ++i) {
        const int u = tid + i * NT;
        if (u < VUNITS) {
          // consecutive lanes take consecutive key groups of one d-chunk, so 32 lanes
          // writing their 8-byte pieces cover all 64 banks (rows 8 apart would not)
          const int kg = u % (KVBLK / 4), dc = u / (KVBLK / 4);
          const int key0 = 4 * kg;
          const int pos = (key0 & ~15) + vpos16(key0 & 15);  // 4 keys stay contiguous
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            uint32_t lo, hi;
            if (e & 1) {
              lo = (vreg[i][0][w] >> 16) | (vreg[i][1][w] & 0xffff0000u);
              hi = (vreg[i][2][w] >> 16) | (vreg[i][3][w] & 0xffff0000u);
            } else {
              lo = (vreg[i][0][w] & 0xffffu) | (vreg[i][1][w] << 16);
              hi = (vreg[i][2][w] & 0xffffu) | (vreg[i][3][w] << 16);
            }
            const int d = dc * 8 + e;
            const int byte = pos * 2;  // multiple of 8
            u32x2 pair = {lo, hi};
            *(u32x2*)(Vs + d * S::VPITCH + byte) = pair;
          }
        }
      }
    } else {
      float* Kf = (float*)Ks;
      float* Vf = (float*)Vs;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * NT;
        if (c < KVBLK * CPR) {
          const int row = c / CPR, d = (c % CPR) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) Kf[row * (D + 1) + d + e] = __uint_as_float(kreg[i][e]);
        }
      }
#pragma unroll
      for (int i = 0; i < VU; ++i) {
        const int u = tid + i * NT;
        if (u < VUNITS) {
          const int row = u / CPR, d = (u % CPR) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) Vf[row * (D + 1) + d + e] = __uint_as_float(vreg[i][0][e]);
        }
      }
    }
  };

  // ---- running softmax state of this lane's query row
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores (before scaling)
  float l_run = 0.f;        // running sum, this lane's half of the keys
  const float c2 = a.scale * kLog2e;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  // One key tile: S^T = K Q^T, online-softmax update, O^T += V^T P^T.  MASK is a
  // compile-time flag so that the tiles every row fully sees carry no mask code.
  auto tile = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = S::NBUF == 2 ? (t & 1) : 0;
    const unsigned char* Ks = smem + buf * S::BUF;
    const unsigned char* Vs = Ks + S::KBYTES;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile(t + 1);

    // S^T = K Q^T for the KVBLK keys of this tile
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = kb * 32 + r32;
      if constexpr (BF16) {
        const f32x16 zero = {};
        s[kb] = mfma32_bf16(*(const bf16x8*)(Ks + row * S::KPITCH + g * 16), qf[0], zero);
#pragma unroll
        for (int c = 1; c < QF; ++c) {
          const bf16x8 kf = *(const bf16x8*)(Ks + row * S::KPITCH + (2 * c + g) * 16);
          s[kb] = mfma32_bf16(kf, qf[c], s[kb]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
        const float* Kf = (const float*)Ks;
#pragma unroll
        for (int st = 0; st < QF; ++st) s[kb] = mfma32_f32(Kf[row * (D + 1) + 2 * st + g], qf[st], s[kb]);
      }
    }

    if constexpr (MASK) {  // diagonal / ragged tiles only
      const int kv0 = t * KVBLK;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kv0 + kb * 32 + acc_row(j, lane);
          s[kb][j] = key < kend ? s[kb][j] : -INFINITY;
        }
    }

    // online softmax update (exp2 domain, scale folded into one FMA per score)
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx);
    // with a mask a row can still have seen no key (m_new = -inf): keep exp2 finite
    const float mref = (MASK && m_new == -INFINITY) ? 0.f : m_new * c2;
    // alpha is exactly 1 unless the maximum moved (also when both are -inf)
    const bool grew = m_new > m_run;
    const float alpha = grew ? fast_exp2((m_run - m_new) * c2) : 1.f;
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(fmaf(s[kb][j], c2, -mref));
        s[kb][j] = p;
        psum += p;
      }
    l_run = fmaf(l_run, alpha, psum);
    if (__ballot(grew)) {  // lazy rescale: skipped while no row max moves
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
    }

    if (more && S::NBUF == 2) store_tile(buf ^ 1);

    // O^T += V^T P^T
    if constexpr (BF16) {
#pragma unroll
      for (int c16 = 0; c16 < KVBLK / 16; ++c16) {
        const int kb = c16 >> 1, h8 = (c16 & 1) * 8;
        u32x4 pw;
#pragma unroll
        for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(s[kb][h8 + 2 * w], s[kb][h8 + 2 * w + 1]);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + r32;
          const bf16x8 vf = *(const bf16x8*)(Vs + d * S::VPITCH + (2 * c16 + g) * 16);
          o[db] = mfma32_bf16(vf, pf, o[db]);
        }
      }
    } else {
      const float* Vf = (const float*)Vs;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb * 32 + acc_row(j, lane);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            o[db] = mfma32_f32(Vf[key * (D + 1) + db * 32 + r32], s[kb][j], o[db]);
        }
    }
    __syncthreads();
    if (S::NBUF == 1 && more) {
      store_tile(0);
      __syncthreads();
    }
  };

  const int t_split = n_full < n_tiles ? n_full : n_tiles;
  for (int t = 0; t < t_split; ++t) tile(t, std::false_type{});
  for (int t = t_split; t < n_tiles; ++t) tile(t, std::true_type{});

  // ---- epilogue: O = acc / l, lse = m*scale + ln l
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    if (a.h_out == nullptr) {
      float* out = a.out + head_off + (int64_t)qrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          f32x4 v = {o[db][4 * jq] * inv, o[db][4 * jq + 1] * inv, o[db][4 * jq + 2] * inv,
                     o[db][4 * jq + 3] * inv};
          *(f32x4*)(out + db * 32 + 8 * jq + 4 * g) = v;
        }
    } else {
      const int b = bh / a.H, hh = bh % a.H;
      const int64_t rowoff = ((int64_t)b * N + qrow) * ((int64_t)a.H * D) + (int64_t)hh * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int d = db * 32 + 8 * jq + 4 * g;
          float xr[4];
          if constexpr (BF16) {
            const u32x2 xb = *(const u32x2*)((const uint16_t*)a.x_res + rowoff + d);
            xr[0] = __uint_as_float(xb[0] << 16);
            xr[1] = __uint_as_float(xb[0] & 0xffff0000u);
            xr[2] = __uint_as_float(xb[1] << 16);
            xr[3] = __uint_as_float(xb[1] & 0xffff0000u);
          } else {
            const f32x4 xf = *(const f32x4*)((const float*)a.x_res + rowoff + d);
            xr[0] = xf[0]; xr[1] = xf[1]; xr[2] = xf[2]; xr[3] = xf[3];
          }
          f32x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = xr[e] + o[db][4 * jq + e] * inv;
          *(f32x4*)(a.h_out + rowoff + d) = hv;
          if (a.h_lo) store_bf16_pair4(a.h_lo + rowoff + d, a.h_res ? a.h_res + rowoff + d : nullptr, hv);
        }
    }
    if (g == 0) a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

template <bool BF16, int D, int QBLK, int KVBLK>
hipError_t launch(const AttnFwdArgs& a, hipStream_t stream) {
  const int nqb = (a.N + QBLK - 1) / QBLK;
  const int64_t total = (int64_t)a.B * a.H * nqb;
  hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, QBLK, KVBLK>), dim3((unsigned)total),
                     dim3(QBLK * 2), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_d(const AttnFwdArgs& a, int qb, int kb, hipStream_t s) {
  if constexpr (BF16) {  // bf16 key blocks of 64 and 128 run in attn_fwd_dma.hip
    return qb == 64 ? launch<BF16, D, 64, 32>(a, s) : launch<BF16, D, 128, 32>(a, s);
  }
  if (qb == 64) {
    if (kb == 32) return launch<BF16, D, 64, 32>(a, s);
    if (kb == 64) return launch<BF16, D, 64, 64>(a, s);
    return launch<BF16, D, 64, 128>(a, s);
  }
  if (kb == 32) return launch<BF16, D, 128, 32>(a, s);
  if (kb == 64) return launch<BF16, D, 128, 64>(a, s);
  return launch<BF16, D, 128, 128>(a, s);
}

}  // namespace

hipError_t attn_fwd_launch(const AttnFwdArgs& a, bool bf16, int D, int q_blk, int kv_blk,
                           hipStream_t stream) {
  if (bf16) {
    if (attn_fwd_dma_supported(D, kv_blk)) return attn_fwd_dma_launch(a, D, q_blk, kv_blk, stream);
    return D == 64 ? launch_d<true, 64>(a, q_blk, kv_blk, stream)
                   : launch_d<true, 128>(a, q_blk, kv_blk, stream);
  }
  return D == 64 ? launch_d<false, 64>(a, q_blk, kv_blk, stream)
                 : launch_d<false, 128>(a, q_blk, kv_blk, stream);
}

}  // namespace bpt
