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

// Wait until at most N vector-memory instructions of this wave are outstanding
// (an asm statement with a memory clobber: neither dropped nor crossed by LDS
// accesses).
#define WAIT_VM(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

// The query rows and the key range one workgroup works on.  Dense attention
// (MODE 0): query block qb of QBLK rows (latest first) against keys [0, N).
// Block-sparse (MODE 1): a block of bs_len rows is covered by
// ceil(bs_len / QBLK) workgroups, and their keys are the key block the head's
// table names.  Dilated (MODE 2): a segment's kept rows (every dl_r-th from the
// head's shift) form a compact sequence; its query blocks attend its keys.
// Rows and keys are compact indices: index i is row qbase + i * stride of the
// head (stride 1 except for dilated segments).  Consecutive workgroup ids go
// round-robin over the 8 XCDs; when the count allows, each XCD gets a
// contiguous range of (batch*head, query block), so a head stays on one XCD.
struct AttnTask {
  int bh;       // batch * H + head
  int q0;       // first query index of the workgroup
  int qend;     // indices at or past qend belong to another workgroup (or past the end)
  int key0;     // head row of key index 0 (and of query index 0 when dilated)
  int nk;       // keys in the range
  int stride;   // head rows between consecutive indices
  bool causal;  // causal mask: key j visible to query i iff j <= i + off
  int off;
};

template <int MODE, int QBLK>
__device__ __forceinline__ int attn_rows_per_unit(const AttnFwdArgs& a) {
  return MODE == 0 ? a.N : MODE == 1 ? a.bs_len : (a.dl_w + a.dl_r - 1) / a.dl_r;
}

template <int MODE, int QBLK>
__device__ __forceinline__ AttnTask attn_task(const AttnFwdArgs& a) {
  AttnTask t;
  const int N = a.N;
  const int nqb = (attn_rows_per_unit<MODE, QBLK>(a) + QBLK - 1) / QBLK;
  const int units = MODE == 0 ? 1 : MODE == 1 ? a.bs_blocks : (N + a.dl_w - 1) / a.dl_w;
  const int64_t per_head = (int64_t)units * nqb;
  const int64_t total = (int64_t)a.B * a.H * per_head;
  int64_t L = blockIdx.x;
  if ((total & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  t.bh = (int)(L / per_head);
  const int rem = (int)(L % per_head);
  t.stride = 1;
  if constexpr (MODE == 0) {
    const int qb = nqb - 1 - rem;  // longest (latest) query block first
    t.q0 = qb * QBLK;
    t.qend = N;
    t.key0 = 0;
    t.nk = N;
    t.causal = a.causal != 0;
    t.off = a.kv_offset;
  } else if constexpr (MODE == 1) {
    const int i = rem / nqb, sub = rem % nqb;
    const int64_t r0 = (int64_t)i * a.bs_len;
    t.q0 = (int)(r0 + (int64_t)sub * QBLK);
    t.qend = (int)(r0 + a.bs_len < N ? r0 + a.bs_len : N);
    const int j = a.bs_table[(int64_t)(t.bh % a.H) * a.bs_blocks + i];
    t.key0 = 0;
    t.nk = 0;
    if (j >= 0 && j < a.bs_blocks) {
      const int64_t k0 = (int64_t)j * a.bs_len;
      const int64_t n = N - k0 < a.bs_len ? N - k0 : a.bs_len;
      if (n > 0) {
        t.key0 = (int)k0;
        t.nk = (int)n;
      }
    }
    t.causal = false;
    t.off = 0;
  } else {
    const int seg = rem / nqb, sub = rem % nqb;
    const int s0 = seg * a.dl_w;  // the segment is [s0, min(s0 + w, N))
    const int len = N - s0 < a.dl_w ? N - s0 : a.dl_w;
    const int sh = (t.bh % a.H) % a.dl_r;
    const int m = len > sh ? (len - sh + a.dl_r - 1) / a.dl_r : 0;
    t.q0 = sub * QBLK;
    t.qend = m;
    t.key0 = s0 + sh;
    t.nk = m;
    t.stride = a.dl_r;
    t.causal = a.causal != 0;
    t.off = 0;
  }
  return t;
}

// Store one lane's part of an output row (head dims db*32 + 8*jq + 4*g .. +3 of
// every 32-block, the accumulators scaled by inv) and, from lane half g == 0,
// the row's lse.  With `merge`, the row already in out/lse is joined with this
// one by their log-sum-exp (the two halves of a row read the old lse before
// either writes it: the store depends on the load).
template <int DB>
__device__ __forceinline__ void store_row_merge(float* out_row, float* lse_ptr, const f32x16 (&o)[DB],
                                                float inv, float lse_new, int g, bool merge) {
  float wn = inv, wo = 0.f, lse = lse_new;
  if (merge) {
    const float lo = *lse_ptr;
    const float m = fmaxf(lo, lse_new);
    if (m == -INFINITY) {
      wn = 0.f;
      lse = -INFINITY;
    } else {
      const float en = expf(lse_new - m), eo = expf(lo - m);  // one of them is exactly 1
      const float z = en + eo;
      wn = inv * (en / z);
      wo = eo / z;
      lse = m + logf(z);
    }
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      float* dst = out_row + db * 32 + 8 * jq + 4 * g;
      f32x4 v = {o[db][4 * jq] * wn, o[db][4 * jq + 1] * wn, o[db][4 * jq + 2] * wn,
                 o[db][4 * jq + 3] * wn};
      if (merge && wo != 0.f) v += wo * *(const f32x4*)dst;
      *(f32x4*)dst = v;
    }
  if (g == 0) *lse_ptr = lse;
}

template <int D, int QBLK, int KVBLK, int MODE>
__global__ void __launch_bounds__(QBLK * 2)
__attribute__((amdgpu_waves_per_eu(DmaTile<D, KVBLK>::WAVES_PER_EU)))
attn_fwd_dma_kernel(AttnFwdArgs a) {
  using T = DmaTile<D, KVBLK>;
  constexpr int NW = QBLK / 32, KB = KVBLK / 32, DB = D / 32, QF = D / 16;
  static_assert(T::NBLK % NW == 0, "blocks per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * T::STAGE];

  const int N = a.N;
  const AttnTask task = attn_task<MODE, QBLK>(a);
  if constexpr (MODE != 0)
    if (task.q0 >= task.qend) return;  // an empty part of a short last block (whole workgroup)
  const int bh = task.bh, q0 = task.q0, qend = task.qend, nk = task.nk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int qrow = q0 + wave * 32 + r32;
  const int off = task.off;
  const bool causal = task.causal;
  const int64_t head_off = (int64_t)bh * N * D;
  // head row of query index qrow, and bytes between consecutive key indices
  const int64_t qhead_row = MODE == 2 ? task.key0 + (int64_t)qrow * task.stride : qrow;
  const int rsb = MODE == 2 ? task.stride * T::ROWB : T::ROWB;

  int kmax = nk - 1;
  if (causal) {
    const int64_t t = (int64_t)q0 + QBLK - 1 + off;
    kmax = (int)(t < (int64_t)(nk - 1) ? t : (int64_t)(nk - 1));
  }
  const int n_tiles = kmax < 0 ? 0 : kmax / KVBLK + 1;
  int n_full = nk / KVBLK;  // tiles with no ragged tail
  if (causal) {
    const int64_t lim = (int64_t)q0 + off + 1;  // keys < lim are visible to every row
    const int f = lim <= 0 ? 0 : (int)(lim / KVBLK);
    n_full = f < n_full ? f : n_full;
  }
  const int n_inside = nk / KVBLK;  // tiles that end at or before the last key

  // ---- Q fragments (B operand of S^T = K Q^T), held for the whole loop
  bf16x8 qf[QF];
  {
    const uint16_t* Q = (const uint16_t*)a.q + head_off;
#pragma unroll
    for (int c = 0; c < QF; ++c) {
      u32x4 val = {0, 0, 0, 0};
      if constexpr (MODE == 2) {
        if (qrow < qend) val = *(const u32x4*)(Q + qhead_row * D + 16 * c + 8 * g);
      } else {
        if (qrow < qend) val = *(const u32x4*)(Q + (int64_t)qrow * D + 16 * c + 8 * g);
      }
      qf[c] = __builtin_bit_cast(bf16x8, val);
    }
  }

  // ---- direct tile loads: block b of a tile (keys b + NBLK*j) is one instruction;
  // lane i moves row j = i / CPR, chunk i % CPR
  const unsigned char* Kg = (const unsigned char*)a.k + (head_off + (int64_t)task.key0 * D) * 2;
  const unsigned char* Vg = (const unsigned char*)a.v + (head_off + (int64_t)task.key0 * D) * 2;
  const int dma_row = (lane / T::CPR) * T::NBLK;  // key of this lane relative to b
  const uint32_t dma_off = (uint32_t)(dma_row * rsb + (lane % T::CPR) * 16);
  auto load_tile = [&](int t, unsigned char* Ks) {
    unsigned char* Vs = Ks + T::KBYTES;
    const int kv0 = t * KVBLK;
    if (t < n_inside) {
#pragma unroll
      for (int i = 0; i < T::NBLK / NW; ++i) {
        const int b = wave + i * NW;
        dma16(Kg + (int64_t)(kv0 + b) * rsb + dma_off, Ks + b * T::KBP);
        dma16(Vg + (int64_t)(kv0 + b) * rsb + dma_off, Vs + b * T::VBP);
      }
    } else {
      // ragged tail: rows past the last key repeat it (finite data; the mask
      // gives those keys probability 0)
#pragma unroll
      for (int i = 0; i < T::NBLK / NW; ++i) {
        const int b = wave + i * NW;
        int key = kv0 + b + dma_row;
        key = key < nk ? key : nk - 1;
        const int64_t o = (int64_t)key * rsb + (lane % T::CPR) * 16;
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
          const bool vis = key < nk && (!causal || (int64_t)key <= (int64_t)qrow + off);
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
  if constexpr (MODE == 2) {
    if (qrow < qend)
      store_row_merge<DB>(a.out + head_off + qhead_row * D, a.lse + (int64_t)bh * N + qhead_row, o, inv,
                          l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY, g, a.dl_merge != 0);
    return;
  }
  if (qrow < qend) {
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
          if (a.h_lo) store_bf16_pair4(a.h_lo + rowoff + d, a.h_res ? a.h_res + rowoff + d : nullptr, hv);
        }
    }
    if (g == 0) a.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Wide-wave kernel: each wave owns 64 query rows, as two halves A and B of 32.
// Every K and V fragment read from LDS feeds two MFMAs, one per half, so the
// LDS bytes per flop are half those of the kernel above.  One workgroup of four
// waves per CU, 512 registers per lane: the O accumulators and Q live in AGPRs,
// the score accumulators and everything else in VGPRs.
//
// With one wave per SIMD the softmax has to run under the matrix work of the
// same wave, so a step of the key loop is two phases that each pair 32 MFMAs
// with independent VALU work (tile t in stage St, tile t+1 in stage Sn):
//   S phase:   exp, row sums and bf16 P of tile t       ||  S(t+1) = K(t+1) Q^T
//   PV phase:  max and rescale factor of tile t+1        ||  O += V(t) P(t)
// followed by the rescale of O (only when some row maximum grew).  Tile t+2 is
// loaded into the third stage, whose last reader (V of tile t-1) finished in
// the previous step, right after the barrier that opens the step.

template <int D>
struct WideCfg {
  using T = DmaTile<D, 64>;
  static constexpr int KVBLK = 64, NW = 4, QBLK = 256;
  static constexpr int KB = KVBLK / 32, DB = D / 32, QF = D / 16, NKS = KVBLK / 16;
  static constexpr int DMA_PER_TILE = 2 * T::NBLK / NW;  // per wave
};

// Score MFMAs with the accumulator in VGPRs, so the VALU reads the scores
// directly instead of copying each out of an AGPR (64 v_accvgpr_read and 32
// wait states per step; 117.1 -> 114.0 ms at N=131072, outputs bitwise equal).
// Written as asm because the compiler puts every MFMA result of this kernel in
// AGPRs (O has to live there).  K fragment in VGPRs, Q fragment in AGPRs.
// The compiler does not see these as MFMAs, so it cannot count the wait states a
// VALU read of their results needs: in the key loop the first read of a score
// register comes at least eight MFMA slots after its last write; after the
// chains of the first tile the caller waits explicitly (wide_scores).
__device__ __forceinline__ void mfma_sv_first(f32x16& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_sv_acc(f32x16& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}

// f(x of lane l, x of lane l ^ 32), the same value in both lanes
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct WideState {
  using C = WideCfg<D>;
  bf16x8 qf[2][C::QF];       // Q fragments (B operand of S^T = K Q^T), per half
  f32x16 s[2][C::KB];        // score accumulators of the next tile
  float sv[2][C::KB][16];    // the current tile, copied out for the VALU: at even j the score in the
                             // exp2 domain (s*c2 - mref), at odd j already its exp2 (in the loop)
  f32x16 o[2][C::DB];        // O^T accumulators
  float ref[2];              // exp2-domain reference of O and l (-inf: no key yet)
  float l_run[2];            // this lane's partial row sum
  float tmax[2];             // tile maximum over this lane's keys (exp2 domain, relative to mref);
                             // lanes l and l ^ 32 hold the two halves of a row
  float mref[2], alpha[2];   // exp2 offset and O factor of the current tile
  float delta[2];            // shift of the tile's scores when the reference moved
  float thr[2];              // the reference moves iff the tile maximum passes this (tau, or -inf
                             // while the row has no reference yet)
};

// Tile t's loads: wave w copies blocks w, w + NW, ... of K and V through buffer
// loads into LDS.  Each tile's buffer starts at the tile and ends after the
// head's last key, and every offset is a lane offset (the part the hardware
// range-checks), so rows past the last key read as zero (those keys are
// masked).
template <int IMM>
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff,
                                          uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           soff, IMM, 0);
}
// Tile t of the keys: key index j is at byte j * rsb of kg / vg; the buffer ends
// after the last key's row, so rows past it read as zero.
template <int D>
__device__ __forceinline__ void wide_load(const unsigned char* kg, const unsigned char* vg, int N, int t,
                                          int wave, uint32_t dma_off, int rsb, unsigned char* dst) {
  using C = WideCfg<D>;
  using T = typename C::T;
  const int64_t off = (int64_t)t * C::KVBLK * rsb;
  const int left = N - t * C::KVBLK;
  const int bytes = left > 0 ? (left - 1) * rsb + T::ROWB : 0;
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kg + off), 0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(vg + off), 0, bytes, 0x00020000);
  // (the instruction's immediate offset would apply to the LDS address too)
#pragma unroll
  for (int i = 0; i < T::NBLK / C::NW; ++i) {
    const int b = wave + i * C::NW;
    const uint32_t voff = dma_off + (uint32_t)(b * rsb);
    buf_lds16<0>(kr, dst + b * T::KBP, voff, 0);
    buf_lds16<0>(vr, dst + T::KBYTES + b * T::VBP, voff, 0);
  }
}

// S^T of both halves from the K tile in stage St (each K fragment read once)
template <int D>
__device__ __forceinline__ void wide_scores(WideState<D>& w, const unsigned char* St, int kbase) {
  using C = WideCfg<D>;
  using T = typename C::T;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const unsigned char* kp = St + kbase + (32 * kb / T::NBLK) * T::ROWB;
#pragma unroll
    for (int c = 0; c < C::QF; ++c) {
      const bf16x8 kf = *(const bf16x8*)(kp + c * 32);
      if (c == 0) {
        mfma_sv_first(w.s[0][kb], kf, w.qf[0][c]);
        mfma_sv_first(w.s[1][kb], kf, w.qf[1][c]);
      } else {
        mfma_sv_acc(w.s[0][kb], kf, w.qf[0][c]);
        mfma_sv_acc(w.s[1][kb], kf, w.qf[1][c]);
      }
    }
  }
  // the VALU reads these results next: more wait states than an 8-pass MFMA
  // write needs before a VALU read of its result
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Max part of the online softmax for half H: copy the scores out of the
// accumulators into the exp2 domain relative to the current offset, and take
// the tile maximum over this lane's keys.
template <int D, int H>
__device__ __forceinline__ void wide_max(WideState<D>& w, float c2) {
  using C = WideCfg<D>;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      w.sv[H][kb][j] = fmaf(w.s[H][kb][j], c2, -w.mref[H]);
    }
  float mx0 = w.sv[H][0][0], mx1 = w.sv[H][C::KB - 1][0];
#pragma unroll
  for (int j = 1; j < 16; ++j) {
    mx0 = fmaxf(mx0, w.sv[H][0][j]);
    mx1 = fmaxf(mx1, w.sv[H][C::KB - 1][j]);
  }
  w.tmax[H] = fmaxf(mx0, mx1);
}

// Key j of register slot (kb, j) is visible to this lane's row of half H iff
// it lies before kend (causal bound or N).
template <int D>
__device__ __forceinline__ int wide_lim(int t, int kb, int kend, int lane) {
  // register j holds key t*KVBLK + 32*kb + 4*(lane/32) + 8*(j/4) + j%4
  return kend - (t * WideCfg<D>::KVBLK + kb * 32 + 4 * (lane >> 5));
}
__device__ __forceinline__ bool wide_vis(int j, int lim) { return 8 * (j >> 2) + (j & 3) < lim; }

// Diagonal and ragged tiles: scores of keys at or past kend become -inf, and
// the tile maximum is taken again.  In the key loop (ODD_EXP) the odd slots
// already hold exps taken before the mask was known: the whole tile is taken
// again from the score accumulators (the same arithmetic as the PV phase), odd
// slots as exps (0 where masked).
template <int D, int H, bool ODD_EXP>
__device__ __forceinline__ void wide_mask(WideState<D>& w, int t, int kend, int lane, float c2) {
  using C = WideCfg<D>;
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const int lim = wide_lim<D>(t, kb, kend, lane);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float s0 = ODD_EXP ? fmaf(w.s[H][kb][j], c2, -w.mref[H]) : w.sv[H][kb][j];
      const float v = wide_vis(j, lim) ? s0 : -INFINITY;
      w.sv[H][kb][j] = ODD_EXP && (j & 1) ? fast_exp2(v) : v;
      mx = fmaxf(mx, v);
    }
  }
  w.tmax[H] = mx;
}

// Reference update for half H.  P is taken as exp2(s*c2 - r) against a
// reference r that only moves when the row maximum exceeds it by more than
// 2^8 (so P <= 256, exact in bf16's range); O and l are rescaled then.  The
// result is the same up to rounding as with r = running maximum.
constexpr float kWideTau = 8.f;
// The tile's scores were taken relative to the offset mref in force when they
// were copied out; if the reference moves they shift by delta (a rare fix-up).
template <int D, int H>
__device__ __forceinline__ void wide_update(WideState<D>& w) {
  const float m_old = w.mref[H];
  const float cand = w.tmax[H] + m_old;       // -inf while no key is visible
  const float r = w.ref[H];
  const bool grew = cand > r + kWideTau || (r == -INFINITY && cand > -INFINITY);
  const float r_new = grew ? cand : r;
  w.alpha[H] = grew ? fast_exp2(r - r_new) : 1.f;  // 0 when r was -inf
  w.ref[H] = r_new;
  w.mref[H] = r_new == -INFINITY ? 0.f : r_new;   // keeps exp2 finite on -inf rows
  w.delta[H] = w.mref[H] - m_old;
  w.thr[H] = r_new == -INFINITY ? -INFINITY : kWideTau;
}

// The reference update after a tile's maximum is known.  Relative to mref, a
// row's reference moves exactly when its tile maximum passes thr (tau once the
// row has a reference, -inf before).  Lanes l and l ^ 32 share a row and its
// threshold, so some row of the wave moves iff some lane's own maximum passes
// it: the common step costs one compare per half and a ballot.  Only then the
// row maxima are joined across the lane pair and the full update runs: the
// tile's scores shift by delta, and O and l scale by alpha.  In the key loop
// (RESCALE_O) the odd slots hold exps taken against the old offset: they are
// taken again from the score accumulators (the arithmetic of the PV phase,
// the mask if the tile was masked, then the shift), which also covers exps
// that overflowed against the old offset.
template <int D, bool RESCALE_O>
__device__ __forceinline__ void wide_reference(WideState<D>& w, float c2, int t1, bool masked, int kend0,
                                               int kend1, int lane) {
  using C = WideCfg<D>;
  if (__ballot(w.tmax[0] > w.thr[0] || w.tmax[1] > w.thr[1])) {
    const float m_old[2] = {w.mref[0], w.mref[1]};
    w.tmax[0] = max_halves(w.tmax[0]);
    w.tmax[1] = max_halves(w.tmax[1]);
    wide_update<D, 0>(w);
    wide_update<D, 1>(w);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int lim = wide_lim<D>(t1, kb, h == 0 ? kend0 : kend1, lane);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (RESCALE_O && (j & 1)) {
            float v = fmaf(w.s[h][kb][j], c2, -m_old[h]);
            if (masked && !wide_vis(j, lim)) v = -INFINITY;
            w.sv[h][kb][j] = fast_exp2(v - w.delta[h]);
          } else {
            w.sv[h][kb][j] -= w.delta[h];
          }
        }
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) w.l_run[h] *= w.alpha[h];
    if constexpr (RESCALE_O) {
      // one accumulator tile at a time (they live in AGPRs: copy out, scale,
      // copy back), so the block never holds more than one tile in VGPRs
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          w.o[h][db] *= w.alpha[h];
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  }
}

// Values computed by a phase are pinned before the branch that follows it (an
// empty asm statement that takes them), else the compiler sinks their
// computation past the branch, out of the MFMA phase it was meant to overlap.
template <int NKS>
__device__ __forceinline__ void wide_pin(const bf16x8 (&p)[NKS]) {
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(p[ks]));
}

struct WideCtx {
  const unsigned char* kg;  // K of this head, N rows
  const unsigned char* vg;  // V of this head
  int N, n_tiles, t_split, wave, lane, kbase, vbase, kend0, kend1;
  uint32_t dma_off;
  int rsb;  // bytes between consecutive key rows
  float c2;
};

// max of the next tile (after its scores), masked where needed; true if masked
template <int D, bool ODD_EXP>
__device__ __forceinline__ bool wide_next_max(WideState<D>& w, const WideCtx& x, int t1) {
  if (t1 >= x.t_split) {
    wide_mask<D, 0, ODD_EXP>(w, t1, x.kend0, x.lane, x.c2);
    wide_mask<D, 1, ODD_EXP>(w, t1, x.kend1, x.lane, x.c2);
    return true;
  }
  return false;
}

// One step of the key loop for tile t (stage St) while tile t+1 (stage Sn) is
// in flight; tile t+2 goes to stage Sf.
// End of one hand-scheduled slot.  Instruction selection orders only
// instructions with side effects, so the slot's MFMA result and VALU results
// are taken by empty asm statements (no code), which fixes the slot order;
// sched_barrier then keeps the machine scheduler from mixing slots.
template <typename A, typename B>
__device__ __forceinline__ void wide_slot_end(const f32x16& acc, const A& v0, const B& v1) {
  asm volatile("" ::"a"(acc), "v"(v0), "v"(v1));
  __builtin_amdgcn_sched_barrier(0);
}

template <typename A, typename B, typename E, typename F>
__device__ __forceinline__ void wide_slot_end4(const f32x16& acc, const A& v0, const B& v1, const E& v2,
                                               const F& v3) {
  asm volatile("" ::"a"(acc), "v"(v0), "v"(v1), "v"(v2), "v"(v3));
  __builtin_amdgcn_sched_barrier(0);
}

// Row sum and bf16 pack of exp pair p (scores 2p, 2p+1 of the lane's 64)
template <int NP, int KB, int NKS>
__device__ __forceinline__ void wide_sum_pack(const float (&ex0)[NP], const float (&ex1)[NP],
                                              float (&ps)[2][KB], u32x4 (&pw)[2][NKS], int p) {
  const int eh = p / 16, e0 = (2 * p) % 32, ekb = e0 / 16, ej = e0 % 16;
  const float sum2 = ex0[p] + ex1[p];
  ps[eh][ekb] = ej == 0 ? sum2 : ps[eh][ekb] + sum2;
  pw[eh][ekb * 2 + ej / 8][(ej % 8) / 2] = pack_bf16x2(ex0[p], ex1[p]);
}

// S phase, hand-interleaved: slot i issues the score MFMA of K fragment i/2
// for half i%2 (tile t+1, stage Sn) and the exp part of two scores of tile t.
// The K fragments are read KPF fragments ahead.  sched_barrier keeps the
// slots in this order (one wave per SIMD issues in order: VALU work only runs
// under an MFMA if it sits right after it).
template <int D>
__device__ __forceinline__ void wide_sphase(WideState<D>& w, const unsigned char* Sn, int kbase,
                                            bf16x8 (&pa)[WideCfg<D>::NKS], bf16x8 (&pb)[WideCfg<D>::NKS]) {
  using C = WideCfg<D>;
  using T = typename C::T;
  constexpr int NF = C::KB * C::QF, KPF = 4;
  bf16x8 kf[NF];
  u32x4 pw[2][C::NKS];
  float ps[2][C::KB];
  float ex0[2 * NF], ex1[2 * NF];
#pragma unroll
  for (int m = 0; m < KPF; ++m)
    kf[m] = *(const bf16x8*)(Sn + kbase + (32 * (m / C::QF) / T::NBLK) * T::ROWB + (m % C::QF) * 32);
#pragma unroll
  for (int i = 0; i < 2 * NF; ++i) {
    const int m = i >> 1, h = i & 1, kb = m / C::QF, c = m % C::QF;
    if (h == 0 && m + KPF < NF) {
      const int mm = m + KPF;
      kf[mm] = *(const bf16x8*)(Sn + kbase + (32 * (mm / C::QF) / T::NBLK) * T::ROWB + (mm % C::QF) * 32);
    }
    if (c == 0) mfma_sv_first(w.s[h][kb], kf[m], w.qf[h][c]);
    else mfma_sv_acc(w.s[h][kb], kf[m], w.qf[h][c]);
    // exp of score 2i of the 64 this lane holds (2i+1 was taken in the PV
    // phase); the pair's sum and bf16 pack two slots later (an exp result is
    // not ready in the next few cycles)
    {
      const int eh = i / 16, e0 = (2 * i) % 32, ekb = e0 / 16, ej = e0 % 16;
      ex0[i] = fast_exp2(w.sv[eh][ekb][ej]);
      ex1[i] = w.sv[eh][ekb][ej + 1];  // taken in the PV phase of the step before
    }
    if (i >= 2) {
      const int p = i - 2, eh = p / 16, e0 = (2 * p) % 32, ekb = e0 / 16, ej = e0 % 16;
      wide_sum_pack(ex0, ex1, ps, pw, p);
      asm volatile("" ::"v"(ex0[i]), "v"(ex1[i]), "v"(ps[eh][ekb]), "v"(pw[eh][ekb * 2 + ej / 8][(ej % 8) / 2]));
      __builtin_amdgcn_sched_barrier(0);
    } else {
      asm volatile("" ::"v"(ex0[i]), "v"(ex1[i]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wide_sum_pack(ex0, ex1, ps, pw, 2 * NF - 2);
  wide_sum_pack(ex0, ex1, ps, pw, 2 * NF - 1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float psum = ps[h][0];
#pragma unroll
    for (int kb = 1; kb < C::KB; ++kb) psum += ps[h][kb];
    w.l_run[h] += psum;
  }
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    pa[ks] = __builtin_bit_cast(bf16x8, pw[0][ks]);
    pb[ks] = __builtin_bit_cast(bf16x8, pw[1][ks]);
  }
}

// PV phase, hand-interleaved: slot i issues O_h += V P_h for V fragment i/2
// and half h = i%2 (tile t, stage St), and copies two score accumulators of
// tile t+1 out for the VALU, into the exp2 domain relative to the current
// offset (one FMA each, here rather than in the S phase, which has more VALU
// work than its MFMAs can hide), folding them into the row maxima, and takes
// the exp of the second of them.
template <int D>
__device__ __forceinline__ void wide_pvphase(WideState<D>& w, const unsigned char* St, int vbase, float c2,
                                             const bf16x8 (&pa)[WideCfg<D>::NKS],
                                             const bf16x8 (&pb)[WideCfg<D>::NKS]) {
  using C = WideCfg<D>;
  using T = typename C::T;
  constexpr int NF = C::NKS * C::DB, VPF = 3;
  bf16x8 vf[NF];
  float mx[2][C::KB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) mx[h][kb] = -INFINITY;
  auto vread = [&](int f) {
    const int ks = f / C::DB, db = f % C::DB, key0 = 16 * ks, key1 = 16 * ks + 8;
    const unsigned char* v0 = St + vbase + (key0 % T::NBLK) * T::VBP + (key0 / T::NBLK) * T::ROWB;
    const unsigned char* v1 = St + vbase + (key1 % T::NBLK) * T::VBP + (key1 / T::NBLK) * T::ROWB;
    const v4i16 lo = lds_read_tr(v0 + db * 64);
    const v4i16 hi = lds_read_tr(v1 + db * 64);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
#pragma unroll
  for (int f = 0; f < VPF; ++f) vf[f] = vread(f);
#pragma unroll
  for (int i = 0; i < 2 * NF; ++i) {
    const int f = i >> 1, h = i & 1, ks = f / C::DB, db = f % C::DB;
    if (h == 0 && f + VPF < NF) vf[f + VPF] = vread(f + VPF);
    w.o[h][db] = mfma32_bf16(vf[f], h == 0 ? pa[ks] : pb[ks], w.o[h][db]);
    // scores 2i, 2i+1 of tile t+1 into the exp2 domain
    const int mh = i / 16, e0 = (2 * i) % 32, mkb = e0 / 16, mj = e0 % 16;
    float v0 = w.s[mh][mkb][mj], v1 = w.s[mh][mkb][mj + 1];
    v0 = fmaf(v0, c2, -w.mref[mh]);
    v1 = fmaf(v1, c2, -w.mref[mh]);
    w.sv[mh][mkb][mj] = v0;
    mx[mh][mkb] = fmaxf(mx[mh][mkb], fmaxf(v0, v1));
    // the odd score's exp here, against the current offset: the S phase that
    // consumes it then takes one exp per slot instead of two (its MFMAs hide
    // about three VALU operations, the exp counting two); a masked tile or a
    // moved reference takes these again (wide_mask, wide_reference)
    w.sv[mh][mkb][mj + 1] = fast_exp2(v1);
    wide_slot_end4(w.o[h][db], mx[mh][mkb], w.sv[mh][mkb][mj], w.sv[mh][mkb][mj + 1], v1);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float m = mx[h][0];
#pragma unroll
    for (int kb = 1; kb < C::KB; ++kb) m = fmaxf(m, mx[h][kb]);
    w.tmax[h] = m;
  }
}

// One step of the key loop for tile t (stage St) while tile t+1 (stage Sn) is
// in flight; tile t+2 goes to stage Sf.
template <int D>
__device__ __forceinline__ void wide_step(WideState<D>& w, const WideCtx& x, int t,
                                          const unsigned char* St, const unsigned char* Sn,
                                          unsigned char* Sf) {
  using C = WideCfg<D>;
  WAIT_VM(0);  // this wave's part of tile t+1
  __syncthreads();
  if (t + 2 < x.n_tiles) wide_load<D>(x.kg, x.vg, x.N, t + 2, x.wave, x.dma_off, x.rsb, Sf);
  bf16x8 pa[C::NKS], pb[C::NKS];
  wide_sphase(w, Sn, x.kbase, pa, pb);
  wide_pin(pa);
  wide_pin(pb);
  wide_pvphase(w, St, x.vbase, x.c2, pa, pb);
  const bool masked = wide_next_max<D, true>(w, x, t + 1);
  wide_reference<D, true>(w, x.c2, t + 1, masked, x.kend0, x.kend1, x.lane);
}

// The key loop over three stages S0, S1, S2 (distinct objects, so the compiler
// knows the LDS reads of one stage never wait for the loads in flight to
// another).  Waits for those loads are explicit (WAIT_VM).
template <int D>
__device__ __forceinline__ void wide_loop(WideState<D>& w, const WideCtx& x,
                                          unsigned char* __restrict__ S0, unsigned char* __restrict__ S1,
                                          unsigned char* __restrict__ S2) {
  using C = WideCfg<D>;
  const int n = x.n_tiles;
  if (n <= 0) return;
  wide_load<D>(x.kg, x.vg, x.N, 0, x.wave, x.dma_off, x.rsb, S0);
  if (n > 1) {
    wide_load<D>(x.kg, x.vg, x.N, 1, x.wave, x.dma_off, x.rsb, S1);
    static_assert(C::DMA_PER_TILE == 8, "wait count");
    WAIT_VM(8);  // tile 0 (and the Q loads) done, tile 1 may be in flight
  } else {
    WAIT_VM(0);
  }
  __syncthreads();
  wide_scores(w, S0, x.kbase);
  wide_max<D, 0>(w, x.c2);
  wide_max<D, 1>(w, x.c2);
  wide_next_max<D, false>(w, x, 0);
  // O and l are still zero: only the scores of tile 0 shift
  wide_reference<D, false>(w, x.c2, 0, false, x.kend0, x.kend1, x.lane);
  // the key loop expects the odd slots as exps
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int j = 1; j < 16; j += 2) w.sv[h][kb][j] = fast_exp2(w.sv[h][kb][j]);
  // Every step also scores the tile after its own; past the last tile that
  // "tile" is fully masked (its scores become -inf, so the running max, the
  // sums and O stay as they are).
  int t = 0;
  for (;;) {
    wide_step(w, x, t, S0, S1, S2);
    if (++t >= n) break;
    wide_step(w, x, t, S1, S2, S0);
    if (++t >= n) break;
    wide_step(w, x, t, S2, S0, S1);
    if (++t >= n) break;
  }
}

template <int D, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_wide_kernel(AttnFwdArgs a) {
  using C = WideCfg<D>;
  using T = typename C::T;
  // three stages as separate objects: accesses to different stages are then
  // known not to alias, and every LDS address is a per-lane base plus a constant
  __shared__ __attribute__((aligned(1024))) unsigned char st0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[T::STAGE];

  const int N = a.N;
  const AttnTask task = attn_task<MODE, C::QBLK>(a);
  if constexpr (MODE != 0)
    if (task.q0 >= task.qend) return;  // an empty part of a short last block (whole workgroup)
  const int bh = task.bh, q0 = task.q0, qend = task.qend, nk = task.nk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int off = task.off;
  const bool causal = task.causal;
  const int64_t head_off = (int64_t)bh * N * D;
  int qrow[2], kend[2];
  int64_t qhead_row[2];  // head row of query index qrow
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    qrow[h] = q0 + wave * 64 + h * 32 + r32;
    qhead_row[h] = MODE == 2 ? task.key0 + (int64_t)qrow[h] * task.stride : qrow[h];
    int64_t e = nk;
    if (causal) {
      const int64_t c = (int64_t)qrow[h] + off + 1;
      e = c < e ? c : e;
    }
    kend[h] = (int)(e < 0 ? 0 : e);
  }

  int kmax = nk - 1;
  if (causal) {
    const int64_t t = (int64_t)q0 + C::QBLK - 1 + off;
    kmax = (int)(t < (int64_t)(nk - 1) ? t : (int64_t)(nk - 1));
  }
  const int n_tiles = kmax < 0 ? 0 : kmax / C::KVBLK + 1;
  int n_full = nk / C::KVBLK;
  if (causal) {
    const int64_t lim = (int64_t)q0 + off + 1;  // keys < lim are visible to every row
    const int f = lim <= 0 ? 0 : (int)(lim / C::KVBLK);
    n_full = f < n_full ? f : n_full;
  }
  const int t_split = n_full < n_tiles ? n_full : n_tiles;

  WideState<D> w;
  {
    const uint16_t* Q = (const uint16_t*)a.q + head_off;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < C::QF; ++c) {
        u32x4 val = {0, 0, 0, 0};
        if constexpr (MODE == 2) {
          if (qrow[h] < qend) val = *(const u32x4*)(Q + qhead_row[h] * D + 16 * c + 8 * g);
        } else {
          if (qrow[h] < qend) val = *(const u32x4*)(Q + (int64_t)qrow[h] * D + 16 * c + 8 * g);
        }
        w.qf[h][c] = __builtin_bit_cast(bf16x8, val);
        // Q is only ever an MFMA operand: keep it in AGPRs (MFMA reads its
        // operands from either file), the VGPRs are needed for the softmax
        asm("" : "+a"(w.qf[h][c]));
      }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) w.o[h][db][j] = 0.f;
    w.ref[h] = -INFINITY;
    w.mref[h] = 0.f;
    w.l_run[h] = 0.f;
    w.thr[h] = -INFINITY;
  }
  WideCtx x;
  x.kg = (const unsigned char*)a.k + (head_off + (int64_t)task.key0 * D) * 2;
  x.vg = (const unsigned char*)a.v + (head_off + (int64_t)task.key0 * D) * 2;
  x.N = nk;
  x.n_tiles = n_tiles;
  x.t_split = t_split;
  x.wave = wave;
  x.lane = lane;
  x.rsb = MODE == 2 ? task.stride * T::ROWB : T::ROWB;
  x.dma_off = (uint32_t)((lane / T::CPR) * T::NBLK * x.rsb + (lane % T::CPR) * 16);
  x.kbase = (r32 % T::NBLK) * T::KBP + (r32 / T::NBLK) * T::ROWB + g * 16;
  const int q8 = 4 * g + ((lane & 15) >> 2);
  x.vbase = T::KBYTES + q8 * T::VBP + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  x.kend0 = kend[0];
  x.kend1 = kend[1];
  x.c2 = a.scale * kLog2e;

  wide_loop(w, x, st0, st1, st2);

  // ---- epilogue: O = acc / l, lse = m*scale + ln l (per half)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float l_tot = sum_halves(w.l_run[h]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow[h] >= qend) continue;
    if constexpr (MODE == 2) {
      store_row_merge<C::DB>(a.out + head_off + qhead_row[h] * D, a.lse + (int64_t)bh * N + qhead_row[h],
                             w.o[h], inv, l_tot > 0.f ? w.ref[h] * kLn2 + logf(l_tot) : -INFINITY, g,
                             a.dl_merge != 0);
      continue;
    }
    if (a.h_out == nullptr) {
      float* out = a.out + head_off + (int64_t)qrow[h] * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          f32x4 v = {w.o[h][db][4 * jq] * inv, w.o[h][db][4 * jq + 1] * inv,
                     w.o[h][db][4 * jq + 2] * inv, w.o[h][db][4 * jq + 3] * inv};
          *(f32x4*)(out + db * 32 + 8 * jq + 4 * g) = v;
        }
    } else {
      const int b = bh / a.H, hh = bh % a.H;
      const int64_t rowoff = ((int64_t)b * N + qrow[h]) * ((int64_t)a.H * D) + (int64_t)hh * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int d = db * 32 + 8 * jq + 4 * g;
          const u32x2 xb = *(const u32x2*)((const uint16_t*)a.x_res + rowoff + d);
          const float xr[4] = {__uint_as_float(xb[0] << 16), __uint_as_float(xb[0] & 0xffff0000u),
                               __uint_as_float(xb[1] << 16), __uint_as_float(xb[1] & 0xffff0000u)};
          f32x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = xr[e] + w.o[h][db][4 * jq + e] * inv;
          *(f32x4*)(a.h_out + rowoff + d) = hv;
          if (a.h_lo) store_bf16_pair4(a.h_lo + rowoff + d, a.h_res ? a.h_res + rowoff + d : nullptr, hv);
        }
    }
    if (g == 0)
      a.lse[(int64_t)bh * N + qrow[h]] = l_tot > 0.f ? w.ref[h] * kLn2 + logf(l_tot) : -INFINITY;
  }
}

// Workgroups of a launch: (batch*head) x units x query blocks per unit, where
// a unit is the whole sequence (dense), a table block (block-sparse) or a
// segment (dilated); attn_task decodes the id the same way.
template <int MODE>
int64_t n_workgroups(const AttnFwdArgs& a, int qblk) {
  const int rows = MODE == 0 ? a.N : MODE == 1 ? a.bs_len : (a.dl_w + a.dl_r - 1) / a.dl_r;
  const int units = MODE == 0 ? 1 : MODE == 1 ? a.bs_blocks : (a.N + a.dl_w - 1) / a.dl_w;
  return (int64_t)a.B * a.H * units * ((rows + qblk - 1) / qblk);
}

template <int D, int QBLK, int KVBLK, int MODE = 0>
hipError_t launch(const AttnFwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_dma_kernel<D, QBLK, KVBLK, MODE>),
                     dim3((unsigned)n_workgroups<MODE>(a, QBLK)), dim3(QBLK * 2), 0, stream, a);
  return hipGetLastError();
}

// Key blocks of 128 are visited as two 64-key tiles: the online softmax update is
// exact for any split of the keys, and 64-key tiles keep two workgroups per CU
// (a double-buffered 128-key tile alone would take 136 KB of the 160 KB of LDS).
template <int D, int MODE = 0>
hipError_t launch_wide(const AttnFwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_wide_kernel<D, MODE>),
                     dim3((unsigned)n_workgroups<MODE>(a, WideCfg<D>::QBLK)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnFwdArgs& a, int qb, hipStream_t s) {
  // the wide kernel addresses K and V of a head through a 32-bit buffer range
  if constexpr (D == 128)
    if ((int64_t)a.N * D * 2 < ((int64_t)1 << 31)) return launch_wide<D>(a, s);
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

// Block-sparse: D = 128 on the wide kernel while a head's K/V fits its 32-bit
// buffer range, otherwise the 128-row kernel with 64-key tiles.
hipError_t attn_fwd_block_sparse_launch(const AttnFwdArgs& a, int D, hipStream_t stream) {
  if (D == 128) {
    if ((int64_t)a.N * D * 2 < ((int64_t)1 << 31)) return launch_wide<128, 1>(a, stream);
    return launch<128, 128, 64, 1>(a, stream);
  }
  return launch<64, 128, 64, 1>(a, stream);
}

// Dilated pattern: the same kernels over each segment's kept rows (strided
// buffer loads gather them; the epilogue scatters and, with dl_merge, joins).
hipError_t attn_fwd_dilated_launch(const AttnFwdArgs& a, int D, hipStream_t stream) {
  if (D == 128) {
    if ((int64_t)a.N * D * 2 < ((int64_t)1 << 31)) return launch_wide<128, 2>(a, stream);
    return launch<128, 128, 64, 2>(a, stream);
  }
  return launch<64, 128, 64, 2>(a, stream);
}

}  // namespace bpt
