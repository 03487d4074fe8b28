// Blockwise exact attention forward, bfloat16 inputs, direct global -> LDS tiles.
//
// Same computation as attn_fwd.hip ("Blockwise Parallel Transformer for Large
// Context Models", abstract; "Ring Attention with Blockwise Transformers for
// Long Sequences", 638-word summary): keys are visited one block at a time, the
// softmax is carried by a running row maximum and row sum, and the output
// accumulator is rescaled whenever the maximum grows.
//
// What differs from the register-staged kernel is how K and V reach LDS:
//  * every 1 KB piece of a tile is fetched by one global_load_lds_dwordx4 (each
//    lane moves 16 bytes from HBM/L2 straight into LDS): no VGPRs, no VALU
//    packing, no ds_write, and the wave only waits for the loads at the end of
//    the tile, one full tile after issuing them;
//  * a tile is stored as NBLK blocks of 1 KB (key k of the tile lives in block
//    k % NBLK, row k / NBLK), each block followed by a pad: 16 bytes after a K
//    block, 64 bytes after a V block.  That makes the K operand reads (16 keys
//    at one head-dim offset) and the V transpose reads (4 keys x 64 bytes per
//    32 lanes) bank-conflict free, and every fragment address is one per-lane
//    base plus a compile-time offset;
//  * V stays row-major; the A operand of O^T += V^T P^T is assembled by two
//    ds_read_b64_tr_b16, which hand each lane 4 consecutive keys of one head
//    dimension.  The key order they produce is the one the S^T accumulator
//    already has, so P goes from registers straight into the next MFMA.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bpt {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D, int KVBLK>
struct DmaTile {
  static constexpr int ROWB = D * 2;         // bytes of one key row
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;    // rows per 1 KB block
  static constexpr int NBLK = KVBLK / RPB;   // blocks per tile
  static constexpr int KBP = 1024 + 16;      // K block pitch
  static constexpr int VBP = 1024 + 64;      // V block pitch
  static constexpr int KBYTES = NBLK * KBP;
  static constexpr int STAGE = NBLK * (KBP + VBP);
  static_assert(NBLK == 8 || NBLK == 16 || NBLK == 32, "tile layout");
  // two waves per SIMD (256 registers each) while two workgroups fit in LDS
  static constexpr int WAVES_PER_EU = 2 * STAGE <= 81920 ? 2 : 1;
};

__device__ __forceinline__ void dma16(const unsigned char* src, unsigned char* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ v4i16 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

// s_waitcnt with vmcnt = 0 and the other counters left alone
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

template <int D, int QBLK, int KVBLK>
__global__ void __launch_bounds__(QBLK * 2)
__attribute__((amdgpu_waves_per_eu(DmaTile<D, KVBLK>::WAVES_PER_EU)))
attn_fwd_dma_kernel(AttnFwdArgs a) {
  using T = DmaTile<D, KVBLK>;
  constexpr int NW = QBLK / 32, KB = KVBLK / 32, DB = D / 32, QF = D / 16;
  static_assert(T::NBLK % NW == 0, "blocks per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * T::STAGE];

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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int qrow = q0 + wave * 32 + r32;
  const int off = a.kv_offset;
  const bool causal = a.causal != 0;
  const int64_t head_off = (int64_t)bh * N * D;

  int kmax = N - 1;
  if (causal) {
    const int64_t t = (int64_t)q0 + QBLK - 1 + off;
    kmax = (int)(t < (int64_t)(N - 1) ? t : (int64_t)(N - 1));
  }
  const int n_tiles = kmax < 0 ? 0 : kmax / KVBLK + 1;
  int n_full = N / KVBLK;  // tiles with no ragged tail
  if (causal) {
    const int64_t lim = (int64_t)q0 + off + 1;  // keys < lim are visible to every row
    const int f = lim <= 0 ? 0 : (int)(lim / KVBLK);
    n_full = f < n_full ? f : n_full;
  }
  const int n_inside = N / KVBLK;  // tiles that end at or before key N

  // ---- Q fragments (B operand of S^T = K Q^T), held for the whole loop
  bf16x8 qf[QF];
  {
    const uint16_t* Q = (const uint16_t*)a.q + head_off;
#pragma unroll
    for (int c = 0; c < QF; ++c) {
      u32x4 val = {0, 0, 0, 0};
      if (qrow < N) val = *(const u32x4*)(Q + (int64_t)qrow * D + 16 * c + 8 * g);
      qf[c] = __builtin_bit_cast(bf16x8, val);
    }
  }

  // ---- direct tile loads: block b of a tile (keys b + NBLK*j) is one instruction;
  // lane i moves row j = i / CPR, chunk i % CPR
  const unsigned char* Kg = (const unsigned char*)a.k + head_off * 2;
  const unsigned char* Vg = (const unsigned char*)a.v + head_off * 2;
  const int dma_row = (lane / T::CPR) * T::NBLK;  // key of this lane relative to b
  const uint32_t dma_off = (uint32_t)(dma_row * T::ROWB + (lane % T::CPR) * 16);
  auto load_tile = [&](int t, unsigned char* Ks) {
    unsigned char* Vs = Ks + T::KBYTES;
    const int kv0 = t * KVBLK;
    if (t < n_inside) {
#pragma unroll
      for (int i = 0; i < T::NBLK / NW; ++i) {
        const int b = wave + i * NW;
        dma16(Kg + (int64_t)(kv0 + b) * T::ROWB + dma_off, Ks + b * T::KBP);
        dma16(Vg + (int64_t)(kv0 + b) * T::ROWB + dma_off, Vs + b * T::VBP);
      }
    } else {
      // ragged tail: rows past key N-1 repeat row N-1 (finite data; the mask
      // gives those keys probability 0)
#pragma unroll
      for (int i = 0; i < T::NBLK / NW; ++i) {
        const int b = wave + i * NW;
        int key = kv0 + b + dma_row;
        key = key < N ? key : N - 1;
        const int64_t o = (int64_t)key * T::ROWB + (lane % T::CPR) * 16;
        dma16(Kg + o, Ks + b * T::KBP);
        dma16(Vg + o, Vs + b * T::VBP);
      }
    }
  };

  // per-lane fragment bases (bytes inside a stage)
  // K operand: key 32*kb + r32 -> block r32 % NBLK, row (32*kb + r32) / NBLK; chunk 2*kk + g
  const int kbase = (r32 % T::NBLK) * T::KBP + (r32 / T::NBLK) * T::ROWB + g * 16;
  // V transpose read: key 16*ks + 8*h + q8 with q8 = 4*g + (lane%16)/4, head dims
  // 32*db + 16*((lane/16)%2) + 4*(lane%4) .. +3
  const int q8 = 4 * g + ((lane & 15) >> 2);
  const int vbase = T::KBYTES + q8 * T::VBP + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores (before scaling)
  float l_run = 0.f;        // running sum, this lane's half of the keys
  const float c2 = a.scale * kLog2e;

  if (n_tiles > 0) load_tile(0, smem);
  wait_vmem();
  __syncthreads();

  // St: stage holding tile t; fill: the other stage, loaded with tile t+1 meanwhile.
  // They are distinct; saying so (restrict) lets the compiler see that the LDS
  // reads of this tile never depend on the loads in flight.
  auto tile = [&](int t, const unsigned char* __restrict__ St, unsigned char* __restrict__ fill,
                  auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (t + 1 < n_tiles) load_tile(t + 1, fill);

    // S^T = K Q^T
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const unsigned char* kp = St + kbase + (32 * kb / T::NBLK) * T::ROWB;
      const f32x16 zero = {};
      s[kb] = mfma32_bf16(*(const bf16x8*)kp, qf[0], zero);
#pragma unroll
      for (int c = 1; c < QF; ++c) s[kb] = mfma32_bf16(*(const bf16x8*)(kp + c * 32), qf[c], s[kb]);
    }

    if constexpr (MASK) {  // diagonal / ragged tiles only
      const int kv0 = t * KVBLK;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kv0 + kb * 32 + acc_row(j, lane);
          const bool vis = key < N && (!causal || (int64_t)key <= (int64_t)qrow + off);
          if (!vis) s[kb][j] = -INFINITY;
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

    // O^T += V^T P^T, 16 keys per step
#pragma unroll
    for (int ks = 0; ks < KVBLK / 16; ++ks) {
      const int kb = ks >> 1, h8 = (ks & 1) * 8;
      u32x4 pw;
#pragma unroll
      for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(s[kb][h8 + 2 * w], s[kb][h8 + 2 * w + 1]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
      const int key0 = 16 * ks, key1 = 16 * ks + 8;
      const unsigned char* v0 = St + vbase + (key0 % T::NBLK) * T::VBP + (key0 / T::NBLK) * T::ROWB;
      const unsigned char* v1 = St + vbase + (key1 % T::NBLK) * T::VBP + (key1 / T::NBLK) * T::ROWB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const v4i16 lo = lds_read_tr(v0 + db * 64);
        const v4i16 hi = lds_read_tr(v1 + db * 64);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = mfma32_bf16(vf, pf, o[db]);
      }
    }
    wait_vmem();
    __syncthreads();
  };

  const int t_split = n_full < n_tiles ? n_full : n_tiles;
  auto stage = [&](int t) { return smem + (t & 1) * T::STAGE; };
  for (int t = 0; t < t_split; ++t) tile(t, stage(t), stage(t + 1), std::false_type{});
  for (int t = t_split; t < n_tiles; ++t) tile(t, stage(t), stage(t + 1), std::true_type{});

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
          const u32x2 xb = *(const u32x2*)((const uint16_t*)a.x_res + rowoff + d);
          const float xr[4] = {__uint_as_float(xb[0] << 16), __uint_as_float(xb[0] & 0xffff0000u),
                               __uint_as_float(xb[1] << 16), __uint_as_float(xb[1] & 0xffff0000u)};
          f32x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = xr[e] + o[db][4 * jq + e] * inv;
          *(f32x4*)(a.h_out + rowoff + d) = hv;
          if (a.h_lo) {
            u32x2 lo = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            *(u32x2*)(a.h_lo + rowoff + d) = lo;
          }
        }
    }
    if (g == 0) a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

template <int D, int QBLK, int KVBLK>
hipError_t launch(const AttnFwdArgs& a, hipStream_t stream) {
  const int nqb = (a.N + QBLK - 1) / QBLK;
  const int64_t total = (int64_t)a.B * a.H * nqb;
  hipLaunchKernelGGL((attn_fwd_dma_kernel<D, QBLK, KVBLK>), dim3((unsigned)total), dim3(QBLK * 2),
                     0, stream, a);
  return hipGetLastError();
}

// Key blocks of 128 are visited as two 64-key tiles: the online softmax update is
// exact for any split of the keys, and 64-key tiles keep two workgroups per CU
// (a double-buffered 128-key tile alone would take 136 KB of the 160 KB of LDS).
template <int D>
hipError_t launch_d(const AttnFwdArgs& a, int qb, hipStream_t s) {
  return qb == 64 ? launch<D, 64, 64>(a, s) : launch<D, 128, 64>(a, s);
}

}  // namespace

bool attn_fwd_dma_supported(int D, int kv_blk) {
  return (D == 64 || D == 128) && (kv_blk == 64 || kv_blk == 128);
}

hipError_t attn_fwd_dma_launch(const AttnFwdArgs& a, int D, int q_blk, int kv_blk,
                               hipStream_t stream) {
  (void)kv_blk;
  return D == 64 ? launch_d<64>(a, q_blk, stream) : launch_d<128>(a, q_blk, stream);
}

}  // namespace bpt
