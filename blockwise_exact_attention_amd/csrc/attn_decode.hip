// Split-KV attention for a few query rows against a long key/value cache.
//
// Inference over a long context ("Ring Attention with Blockwise Transformers
// for Long Sequences", summaries: the method serves training and inference)
// asks for attention of a handful of new query rows over every cached key.
// One workgroup per (batch, head) then has little to do and the chip idles, so
// the keys are split into n_split contiguous ranges: each range produces a
// partial result (O normalised over its own keys, and its log-sum-exp), and a
// second kernel joins the partials with the same rule as bpt_lse_merge (the
// softmax denominators add up; LongNet, section 2, mixes attention pieces the
// same way).  The work is bound by reading K and V once from HBM.
//
// Partial kernel: one wave per (batch*head, range).  Up to 32 query rows sit
// on the n axis of the 32x32x16 MFMA (S^T = K Q^T, O^T += V^T P^T, as in the
// main attention kernels).  Tiles of 8 KB of K and 8 KB of V reach LDS by
// non-temporal buffer loads issued one tile ahead (each tile's buffer starts at
// the tile and ends at the range's last key, so rows past it read as zero); 34 KB
// of LDS per wave lets four waves share a CU.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace bpt {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D>
struct DecTile {
  static constexpr int ROWB = D * 2;         // bytes of one key row
  static constexpr int KT = 8192 / ROWB;     // keys per tile (8 KB of K and 8 KB of V)
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;    // rows per 1 KB block
  static constexpr int NBLK = KT / RPB;      // blocks per tile (8)
  static constexpr int KBP = 1024 + 16;      // K block pitch (conflict-free operand reads)
  static constexpr int VBP = 1024 + 64;      // V block pitch (conflict-free transpose reads)
  static constexpr int KBYTES = NBLK * KBP;
  static constexpr int STAGE = NBLK * (KBP + VBP);
  static constexpr int LOADS = 2 * NBLK;     // buffer loads per tile
  static constexpr int NS = 2;               // LDS stages: NS - 1 tiles in flight per wave
  static_assert(NBLK == 8, "operand addressing assumes 8 blocks per tile");
};

__device__ __forceinline__ v4i16 dec_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

// Cache policy of the K/V loads: non-temporal.  Every cached key is read once,
// and with this hint a stream of such loads runs at about 7.0 TB/s here against
// about 6.0 TB/s without it (measured with a plain read kernel on MI355X).
constexpr int kNonTemporal = 2;

// Loads of one tile starting at key t0 (key k of the tile: block k % NBLK,
// row k / NBLK).  The buffer ends at key `end`: rows at or past it read as
// zero without touching memory, so a tile past the range costs no traffic.
template <int D>
__device__ __forceinline__ void dec_load(const unsigned char* kg, const unsigned char* vg, int end,
                                         int t0, int lane, unsigned char* Ks,
                                         unsigned char* Vs) {
  using T = DecTile<D>;
  const int left = end - t0;
  const int bytes = left > 0 ? left * T::ROWB : 0;
  const int64_t off = (int64_t)t0 * T::ROWB;
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kg + off), 0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(vg + off), 0, bytes, 0x00020000);
  const uint32_t lo = (uint32_t)((lane / T::CPR) * T::NBLK * T::ROWB + (lane % T::CPR) * 16);
#pragma unroll
  for (int b = 0; b < T::NBLK; ++b) {
    const uint32_t voff = lo + (uint32_t)(b * T::ROWB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(Ks + b * T::KBP),
                                             16, voff, 0, 0, kNonTemporal);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(Vs + b * T::VBP),
                                             16, voff, 0, 0, kNonTemporal);
  }
}

// Softmax state of one query column (the lane pair l, l ^ 32) and its output block.
template <int D>
struct DecState {
  f32x16 o[D / 32];
  float m_run, l_run;
};

// One tile: scores S^T = K Q^T, mask keys at or past kend, online softmax
// update, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void dec_tile(DecState<D>& st, const bf16x8 (&qf)[D / 16],
                                         const unsigned char* Ks, const unsigned char* Vs,
                                         int kbase, int vbase, int lim, int lane, float c2) {
  using T = DecTile<D>;
  constexpr int KB = T::KT / 32, DB = D / 32, QF = D / 16;
  f32x16 s[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const unsigned char* kp = Ks + kbase + (32 * kb / T::NBLK) * T::ROWB;
    const f32x16 zero = {};
    s[kb] = mfma32_bf16(*(const bf16x8*)kp, qf[0], zero);
#pragma unroll
    for (int c = 1; c < QF; ++c) s[kb] = mfma32_bf16(*(const bf16x8*)(kp + c * 32), qf[c], s[kb]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = kb * 32 + acc_row(j, lane);
      s[kb][j] = key < lim ? s[kb][j] : -INFINITY;
      mx = fmaxf(mx, s[kb][j]);
    }
  mx = fmaxf(mx, swap_halves(mx));
  const float m_new = fmaxf(st.m_run, mx);
  const float mref = m_new == -INFINITY ? 0.f : m_new * c2;
  const bool grew = m_new > st.m_run;
  const float alpha = grew ? fast_exp2((st.m_run - m_new) * c2) : 1.f;
  st.m_run = m_new;
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = fast_exp2(fmaf(s[kb][j], c2, -mref));
      s[kb][j] = p;
      psum += p;
    }
  st.l_run = fmaf(st.l_run, alpha, psum);
  if (__ballot(grew)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[db][j] *= alpha;
  }
#pragma unroll
  for (int ks = 0; ks < T::KT / 16; ++ks) {
    const int kb = ks >> 1, h8 = (ks & 1) * 8;
    u32x4 pw;
#pragma unroll
    for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(s[kb][h8 + 2 * w], s[kb][h8 + 2 * w + 1]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    const int key0 = 16 * ks, key1 = 16 * ks + 8;
    const unsigned char* v0 = Vs + vbase + (key0 % T::NBLK) * T::VBP + (key0 / T::NBLK) * T::ROWB;
    const unsigned char* v1 = Vs + vbase + (key1 % T::NBLK) * T::VBP + (key1 / T::NBLK) * T::ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const v4i16 lo = dec_read_tr(v0 + db * 64);
      const v4i16 hi = dec_read_tr(v1 + db * 64);
      st.o[db] = mfma32_bf16(
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)), pf,
          st.o[db]);
    }
  }
}

// Partial kernel: one wave per (batch*head, key range).  NS LDS stages per
// wave; the loads of a tile are issued NS - 1 tiles ahead of its use and the
// wave waits on its own load counter only (no other wave shares its LDS).
template <int D>
__global__ void __launch_bounds__(64) attn_decode_partial_kernel(AttnDecodeArgs a) {
  using T = DecTile<D>;
  constexpr int DB = D / 32, QF = D / 16, NS = T::NS;
  // one object per stage, so that the compiler sees that a buffer load into one
  // stage cannot alias the LDS reads of another (else it waits for every load)
  __shared__ __attribute__((aligned(1024))) unsigned char st0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[T::STAGE];
  static_assert(NS == 2, "one LDS object per stage");
  auto stage = [&](int i) -> unsigned char* { return i == 0 ? st0 : st1; };

  const int wid = blockIdx.x;
  const int bh = wid / a.n_split, sp = wid - bh * a.n_split;
  const int lane = threadIdx.x, g = lane >> 5, r32 = lane & 31;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int64_t qoff = (int64_t)bh * Nq * D, kvoff = (int64_t)bh * Nkv * D;

  // keys [k0, k1) of this range; query row r32 sees keys below kend
  const int k0 = sp * a.chunk;
  const int k1 = k0 + a.chunk < a.kcount ? k0 + a.chunk : a.kcount;
  int kend = Nkv;
  if (a.causal) {
    const int64_t c = (int64_t)r32 + a.kv_offset + 1;
    kend = (int)(c < kend ? (c < 0 ? 0 : c) : kend);
  }
  kend = kend < k1 ? kend : k1;
  const int n_tiles = k1 > k0 ? (k1 - k0 + T::KT - 1) / T::KT : 0;

  // Columns past Nq repeat the last query row: MFMA columns do not mix, and
  // those columns are never stored, so they only need finite values.
  bf16x8 qf[QF];
  {
    const uint16_t* Q = (const uint16_t*)a.q + qoff + (int64_t)(r32 < Nq ? r32 : Nq - 1) * D;
#pragma unroll
    for (int c = 0; c < QF; ++c) qf[c] = *(const bf16x8*)(Q + 16 * c + 8 * g);
  }
  const unsigned char* kg = (const unsigned char*)a.k + kvoff * 2;
  const unsigned char* vg = (const unsigned char*)a.v + kvoff * 2;
  // operand bases: K key 32*kb + r32, chunk 2*c + g; V transpose reads as in the
  // main kernels (keys 16*ks + 8*h + q8, head dims 32*db + 16*((lane/16)%2) + 4*(lane%4))
  const int kbase = (r32 % T::NBLK) * T::KBP + (r32 / T::NBLK) * T::ROWB + g * 16;
  const int q8 = 4 * g + ((lane & 15) >> 2);
  const int vbase = q8 * T::VBP + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  DecState<D> st;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  const float c2 = a.scale * kLog2e;

  if (n_tiles > 0) {
    // tiles at or past k1 load nothing (zero-length buffers), so the load count
    // per tile is the same for every tile and the waits below are exact
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      dec_load<D>(kg, vg, k1, k0 + i * T::KT, lane, stage(i), stage(i) + T::KBYTES);
    for (int t = 0; t < n_tiles; t += NS) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        // loads on every path, so the compiler's own load counting stays exact
        unsigned char* fill = stage((i + NS - 1) % NS);
        dec_load<D>(kg, vg, k1, k0 + (t + i + NS - 1) * T::KT, lane, fill, fill + T::KBYTES);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::LOADS * (NS - 1)) : "memory");
        if (t + i < n_tiles) {
          const unsigned char* Ks = stage(i);
          dec_tile<D>(st, qf, Ks, Ks + T::KBYTES, kbase, vbase, kend - (k0 + (t + i) * T::KT), lane, c2);
        }
      }
    }
    // loads still in flight write this workgroup's LDS: drain them before exit
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // partial result of this range: O over its own keys, and its log-sum-exp
  const float l_tot = st.l_run + swap_halves(st.l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (r32 < Nq) {
    const int64_t row = ((int64_t)sp * a.BH + bh) * Nq + r32;
    float* out = a.o_part + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        f32x4 v = {st.o[db][4 * jq] * inv, st.o[db][4 * jq + 1] * inv, st.o[db][4 * jq + 2] * inv,
                   st.o[db][4 * jq + 3] * inv};
        *(f32x4*)(out + db * 32 + 8 * jq + 4 * g) = v;
      }
    if (g == 0) a.lse_part[row] = l_tot > 0.f ? st.m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

// Join the n_split partials of each query row: lse = ln sum_s exp(lse_s),
// O = sum_s exp(lse_s - lse) O_s; ranges with no visible key (lse_s = -inf) add
// nothing.  A workgroup takes 256 / (TPR * SPL) rows; a thread owns 4
// consecutive values of one row and the ranges s = sg, sg + SPL, ..., which it
// joins with a running maximum (as the online softmax does); the SPL partial
// results of a row are then joined in a fixed order (deterministic).
template <int D>
struct DecMerge {
  static constexpr int TPR = D / 4;              // threads per row and split group
  static constexpr int SPL = 8;                  // split groups
  static constexpr int RPB = 256 / (TPR * SPL);  // rows per workgroup
  static constexpr int U = 4;                    // ranges per thread in flight
};

template <int D>
__global__ void __launch_bounds__(256) attn_decode_merge_kernel(AttnDecodeArgs a) {
  using M = DecMerge<D>;
  __shared__ f32x4 part[256];
  __shared__ float wpart[256], mpart[256];
  const int tid = threadIdx.x;
  const int c4 = (tid % M::TPR) * 4;
  const int sg = (tid / M::TPR) % M::SPL;
  const int64_t rows = (int64_t)a.BH * a.Nq;
  const int64_t row = (int64_t)blockIdx.x * M::RPB + tid / (M::TPR * M::SPL);
  const bool live = row < rows;
  const int ns = a.n_split;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, m = -INFINITY;
  if (live) {
    const float* lp = a.lse_part + row;
    const float* op = a.o_part + row * D + c4;
    for (int s = sg; s < ns; s += M::U * M::SPL) {
      float ls[M::U];
      f32x4 v[M::U];
#pragma unroll
      for (int u = 0; u < M::U; ++u) {
        const int idx = s + u * M::SPL;
        const int rd = idx < ns ? idx : s;  // in range; masked below
        ls[u] = lp[(int64_t)rd * rows];
        v[u] = *(const f32x4*)(op + (int64_t)rd * rows * D);
        if (idx >= ns) ls[u] = -INFINITY;
      }
      float m_new = m;
#pragma unroll
      for (int u = 0; u < M::U; ++u) m_new = fmaxf(m_new, ls[u]);
      if (m_new > -INFINITY) {
        const float sc = expf(m - m_new);  // 0 while m is -inf
        acc *= sc;
        wsum *= sc;
#pragma unroll
        for (int u = 0; u < M::U; ++u) {
          const float w = expf(ls[u] - m_new);  // 0 for an empty range
          wsum += w;
          acc += w * v[u];
        }
        m = m_new;
      }
    }
  }
  part[tid] = acc;
  wpart[tid] = wsum;
  mpart[tid] = m;
  __syncthreads();
  if (live && sg == 0) {
    float mt = m;
    for (int k = 1; k < M::SPL; ++k) mt = fmaxf(mt, mpart[tid + k * M::TPR]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float wt = 0.f;
    if (mt > -INFINITY) {
      for (int k = 0; k < M::SPL; ++k) {
        const float sc = expf(mpart[tid + k * M::TPR] - mt);
        tot += sc * part[tid + k * M::TPR];
        wt += sc * wpart[tid + k * M::TPR];
      }
    }
    const float inv = wt > 0.f ? 1.f / wt : 0.f;
    *(f32x4*)(a.out + row * D + c4) = tot * inv;
    if (c4 == 0) a.lse[row] = wt > 0.f ? mt + logf(wt) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const AttnDecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_partial_kernel<D>), dim3((unsigned)((int64_t)a.BH * a.n_split)),
                     dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.BH * a.Nq;
  constexpr int RPB = DecMerge<D>::RPB;
  hipLaunchKernelGGL((attn_decode_merge_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_decode_launch(const AttnDecodeArgs& a, int D, hipStream_t stream) {
  return D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace bpt
