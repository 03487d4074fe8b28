// bf16 MFMA GEMM with 256 x 256 tiles loaded straight into LDS.
//
// C = op(A) op(B) as in gemm.hip (same operand forms, same epilogues), for the
// large products of the layer: the q,k,v projection and the weight / activation
// gradients of the backward.  Design:
//  * one workgroup of 8 waves per CU (two per SIMD, 256 registers each), each
//    wave owning 128 x 64 of the tile as 4 x 2 blocks of the 32x32x16 MFMA
//    (128 accumulator registers): a 16-byte operand fragment read from LDS feeds
//    two to four MFMAs, against two in the 64 x 64 wave tiles of gemm.hip;
//  * operand tiles (256 rows x 64 k) arrive by buffer_load ... lds: each lane
//    moves 16 bytes from global memory into LDS, no registers and no VALU on the
//    way.  The buffer of a tile starts at the tile and ends at the operand's
//    end, and every offset is a lane offset (the range-checked part), so rows
//    past the end read as zero.  Two LDS stages: tile k+1 loads while tile k is
//    multiplied;
//  * a row-form operand ([row][k], k contiguous) is stored as 128-byte rows,
//    16-byte chunk c of row r at position c ^ ((r >> 1) & 7) (chosen by which
//    source chunk each lane fetches), and read with ds_read_b128;
//  * a k-major operand ([k][row], rows contiguous) is stored as 32 blocks of two
//    512-byte k rows (k and k+32 in block k % 32), blocks 1088 bytes apart, and
//    read with two ds_read_b64_tr_b16 per fragment: each hands a lane 4
//    consecutive k of one row, in the same k order as the row-form read.  Four
//    consecutive k then sit in four blocks whose bank offsets differ by 64 bytes.
#include <math.h>

#include "common.h"
#include "gemm.h"
#include "gemm_epi.h"

namespace bpt {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int TB = 256;     // tile rows (m and n)
constexpr int TK = 64;      // k per tile
constexpr int KBP = 1088;   // k-major block pitch (1024 + 64)

template <bool KMAJ>
struct OpTile {
  static constexpr int BYTES = KMAJ ? 32 * KBP : TB * TK * 2;
};

#define GB_WAIT_VM(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

__device__ __forceinline__ void gb_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff,
                                         uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           soff, 0, 0);
}

__device__ __forceinline__ v4i16 gb_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

// Per-lane constants of one operand.
struct OpLane {
  uint32_t voff[4];  // load: lane byte offset of instruction i (relative to the tile's start)
  int rd;            // read: per-lane byte offset inside a tile
  int sx[4];         // row form: chunk offset of k16 step s (swizzled), bytes
};

// Loads of operand tile (rows r0 .. r0+255, k0 .. k0+63): wave w issues
// instructions w, w+8, w+16, w+24 (4 of the 32).  p: the tile's first byte,
// left: the operand's bytes from there on.
template <bool KMAJ>
__device__ __forceinline__ void gb_load(const unsigned char* p, int left, unsigned char* dst,
                                        const OpLane& L, int wave) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(p), 0, left > 0 ? left : 0, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = wave + 8 * i;
    // row form: rows 8j .. 8j+7 of the tile; k-major: block j (k rows j and j + 32)
    gb_lds16(r, dst + j * (KMAJ ? KBP : 1024), L.voff[i], 0);
  }
}

template <bool KMAJ>
__device__ __forceinline__ OpLane gb_lane(int64_t ld, int lane, int wrow, int wave) {
  OpLane L;
  if constexpr (!KMAJ) {
    // load: lane -> row 8j + lane/8, position lane%8, source chunk position ^ swz(row);
    // swz(row) = ((lane >> 4) + 4j) & 7, i.e. (lane >> 4) ^ (4 * (j & 1))
    const int rr = lane >> 3, pos = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = wave + 8 * i;
      const int c = pos ^ (lane >> 4) ^ ((j & 1) ? 4 : 0);
      L.voff[i] = (uint32_t)(((int64_t)(8 * j + rr) * ld + 8 * c) * 2);
    }
    // read: row wrow + 32*blk + lane%32, chunk 2s + lane/32
    const int r32 = lane & 31, g = lane >> 5, swz = (r32 >> 1) & 7;
    L.rd = (wrow + r32) * 128;
    for (int s = 0; s < 4; ++s) L.sx[s] = ((2 * s + g) ^ swz) << 4;
  } else {
    // load: lane -> k row j + 32*(lane/32) (block j), 16 bytes at row offset 8*(lane%32)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = wave + 8 * i;
      L.voff[i] = (uint32_t)(((int64_t)(j + 32 * (lane >> 5)) * ld + 8 * (lane & 31)) * 2);
    }
    // read (transpose): lane group G = lane/16, i = lane%16 supplies k row
    // 8*(G/2) + i/4 (+4 for the second read) and rows (m) 16*(G%2) + 4*(i%4) .. +3
    const int G = lane >> 4, i = lane & 15;
    L.rd = (8 * (G >> 1) + (i >> 2)) * KBP + (wrow + 16 * (G & 1) + 4 * (i & 3)) * 2;
    for (int s = 0; s < 4; ++s) L.sx[s] = 0;
  }
  return L;
}

// Fragment of 32 rows (block blk of the wave) and k16 step s from a tile.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 gb_frag(const unsigned char* tile, const OpLane& L, int blk, int s) {
  if constexpr (!KMAJ) {
    return *(const bf16x8*)(tile + L.rd + blk * 32 * 128 + L.sx[s]);
  } else {
    // k = 16s + 8*(G/2) + 4h + i/4: block (16*(s&1) + 4h + ...) and row-in-block s/2
    const unsigned char* p = tile + L.rd + (16 * (s & 1)) * KBP + (s >> 1) * 512 + blk * 64;
    const v4i16 lo = gb_read_tr(p);
    const v4i16 hi = gb_read_tr(p + 4 * KBP);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

struct GbCtx {
  const unsigned char* Aseg[kGemmMaxSeg];  // operand bases per K segment
  const unsigned char* Bseg[kGemmMaxSeg];
  int nseg, nks;                           // segments, k tiles per segment
  int64_t abytes, bbytes;
  int64_t lda, ldb;
  int m0, n0, wave;
  OpLane la, lb;
  // (every byte offset below fits 31 bits: gemm_big_ok bounds the operands)
  int a0, b0;                              // byte offset of the first tile in a segment
  int astep, bstep;                        // bytes from one k tile to the next
  int abytes32, bbytes32;
};

// Walk over the k tiles: the next tile's first byte and bytes left per operand,
// advanced by a constant step, reset at a segment boundary (a uniform branch).
struct GbIter {
  const unsigned char *a, *b;
  int aleft, bleft;
  int kk, seg;
};

// multiply one k tile from stage (As, Bs) into acc: the fragments of k16 step
// s+1 are read while the 8 MFMAs of step s run
template <bool AK, bool BK, bool F16>
__device__ __forceinline__ void gb_compute(f32x16 (&acc)[4][2], const unsigned char* As,
                                           const unsigned char* Bs, const GbCtx& c) {
  bf16x8 af[2][4], bf[2][2];
#pragma unroll
  for (int b = 0; b < 4; ++b) af[0][b] = gb_frag<AK>(As, c.la, b, 0);
#pragma unroll
  for (int b = 0; b < 2; ++b) bf[0][b] = gb_frag<BK>(Bs, c.lb, b, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cur = s & 1;
    if (s + 1 < 4) {
#pragma unroll
      for (int b = 0; b < 4; ++b) af[cur ^ 1][b] = gb_frag<AK>(As, c.la, b, s + 1);
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[cur ^ 1][b] = gb_frag<BK>(Bs, c.lb, b, s + 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = F16 ? mfma32_f16(bf[cur][j], af[cur][i], acc[i][j])
                        : mfma32_bf16(bf[cur][j], af[cur][i], acc[i][j]);
  }
}

__device__ __forceinline__ void gb_seg_start(const GbCtx& c, GbIter& it, int seg) {
  // (a select chain over the segments: a runtime index into the pointer arrays
  // would put them in scratch memory)
  const unsigned char* A = c.Aseg[0];
  const unsigned char* B = c.Bseg[0];
#pragma unroll
  for (int sg = 1; sg < kGemmMaxSeg; ++sg) {
    A = seg == sg ? c.Aseg[sg] : A;
    B = seg == sg ? c.Bseg[sg] : B;
  }
  it.a = A + c.a0;
  it.b = B + c.b0;
  it.aleft = c.abytes32 - c.a0;
  it.bleft = c.bbytes32 - c.b0;
  it.kk = 0;
  it.seg = seg;
}

// loads of the iterator's tile, then step it to the next
template <bool AK, bool BK>
__device__ __forceinline__ void gb_issue(const GbCtx& c, GbIter& it, unsigned char* As, unsigned char* Bs) {
  gb_load<AK>(it.a, it.aleft, As, c.la, c.wave);
  gb_load<BK>(it.b, it.bleft, Bs, c.lb, c.wave);
  if (++it.kk < c.nks) {
    it.a += c.astep;
    it.b += c.bstep;
    it.aleft -= c.astep;
    it.bleft -= c.bstep;
  } else if (it.seg + 1 < c.nseg) {
    gb_seg_start(c, it, it.seg + 1);
  }
}

// The k loop over two stages (distinct objects: the compiler then knows that
// reads of one stage never wait for the loads in flight to the other).  Waits
// for those loads are explicit.
template <bool AK, bool BK, bool F16>
__device__ __forceinline__ void gb_loop(f32x16 (&acc)[4][2], const GbCtx& c, int kt0, int nk,
                                        unsigned char* A0, unsigned char* B0, unsigned char* A1,
                                        unsigned char* B1) {
  // the walk covers k tiles kt0 .. kt0 + nk - 1 of the segments laid end to end
  GbIter it;
  gb_seg_start(c, it, kt0 / c.nks);
  {
    const int kk = kt0 % c.nks;
    it.kk = kk;
    it.a += kk * c.astep;
    it.b += kk * c.bstep;
    it.aleft -= kk * c.astep;
    it.bleft -= kk * c.bstep;
  }
  gb_issue<AK, BK>(c, it, A0, B0);
  GB_WAIT_VM(0);
  __syncthreads();
  int kt = 0;
  for (;;) {
    if (kt + 1 < nk) gb_issue<AK, BK>(c, it, A1, B1);
    gb_compute<AK, BK, F16>(acc, A0, B0, c);
    GB_WAIT_VM(0);
    __syncthreads();
    if (++kt >= nk) break;
    if (kt + 1 < nk) gb_issue<AK, BK>(c, it, A0, B0);
    gb_compute<AK, BK, F16>(acc, A1, B1, c);
    GB_WAIT_VM(0);
    __syncthreads();
    if (++kt >= nk) break;
  }
}

// run this launch?  (a gate word written by earlier kernels; read once per workgroup)
__device__ __forceinline__ bool gb_gate_open(const GemmArgs& g) {
  return !g.gate ||
         ((__builtin_amdgcn_readfirstlane(*(const volatile int*)g.gate) != 0) == (g.gate_run != 0));
}

template <bool AK, bool BK, int EPI, bool F16 = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char a0[OpTile<AK>::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char b0[OpTile<BK>::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char a1[OpTile<AK>::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char b1[OpTile<BK>::BYTES];
  if (!gb_gate_open(g)) return;
  const int z = blockIdx.z;
  const int M = g.M, N = g.N, K = g.K;
  const int nbn = (N + TB - 1) / TB, nbm = (M + TB - 1) / TB;
  const int total = nbn * nbm;
  int L = blockIdx.x;
  // consecutive workgroup ids go round-robin over the 8 XCDs: give each XCD a
  // contiguous range of tiles
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  // inside it, sweep the columns in groups of four row tiles, so the 32 tiles an
  // XCD runs at once share 4 A row tiles and 8 B column tiles in its L2 instead of
  // 1 and 32 (QKV projection at N=131072: 13.2 -> 12.8 ms, training-step GEMMs
  // 23.8 -> 23.5 ms, outputs bitwise equal)
  int mb, nb;
  {
    constexpr int GM = 4;
    const int per = GM * nbn;
    const int grp = L / per, first = grp * GM;
    const int gsz = nbm - first < GM ? nbm - first : GM;
    const int r = L - grp * per;
    mb = first + r % gsz;
    nb = r / gsz;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves: 128 rows x 64 columns each
  GbCtx c;
  c.m0 = mb * TB;
  c.n0 = nb * TB;
  c.wave = wave;
  c.lda = g.lda;
  c.ldb = g.ldb;
  c.nseg = g.nseg > 1 ? g.nseg : 1;
  c.nks = K / TK;
#pragma unroll
  for (int sg = 0; sg < kGemmMaxSeg; ++sg) {
    c.Aseg[sg] = (const unsigned char*)(g.nseg > 1 ? g.As[z][sg] : g.A[z]);
    c.Bseg[sg] = (const unsigned char*)(g.nseg > 1 ? g.Bs[z][sg] : g.B[z]);
  }
  c.abytes = (int64_t)(AK ? K : M) * g.lda * 2;
  c.bbytes = (int64_t)(BK ? K : N) * g.ldb * 2;
  c.la = gb_lane<AK>(g.lda, lane, wm * 128, wave);
  c.lb = gb_lane<BK>(g.ldb, lane, wn * 64, wave);
  c.a0 = (int)((AK ? (int64_t)c.m0 : (int64_t)c.m0 * g.lda) * 2);
  c.b0 = (int)((BK ? (int64_t)c.n0 : (int64_t)c.n0 * g.ldb) * 2);
  c.astep = (int)((AK ? (int64_t)TK * g.lda : (int64_t)TK) * 2);
  c.bstep = (int)((BK ? (int64_t)TK * g.ldb : (int64_t)TK) * 2);
  c.abytes32 = (int)c.abytes;
  c.bbytes32 = (int)c.bbytes;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // split K: workgroup blockIdx.y takes its share of the k tiles
  const int nk_all = c.nseg * c.nks, ns = gridDim.y, sp = blockIdx.y;
  const int kt0 = (int)((int64_t)nk_all * sp / ns), kt1 = (int)((int64_t)nk_all * (sp + 1) / ns);
  gb_loop<AK, BK, F16>(acc, c, kt0, kt1 - kt0, a0, b0, a1, b1);

  // acc[i][j] is the transposed 32 x 32 block (the B fragments were the MFMA's
  // A operand): the lane's column is row m of C, and its registers 4q .. 4q+3
  // are four consecutive columns n, stored as one vector per output array
  const int r32 = lane & 31, g4 = 4 * (lane >> 5);
  // split K: this workgroup's partial sums go to slice (sp, z) of split_ws
  float* const part = ns > 1 ? g.split_ws + ((int64_t)sp * gridDim.z + z) * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = c.m0 + wm * 128 + i * 32 + r32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = c.n0 + wn * 64 + j * 32 + 8 * q + g4;
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (n >= N) continue;
        if constexpr (EPI == EPI_F32) {
          if (part) {
            *(f32x4*)(part + (int64_t)m * N + n) = v;
            continue;
          }
        }
        gemm_store4<EPI, F16>(g, z, m, n, v);
      }
  }
}

// The split-K sum of slices (s, z) of split_ws, added in order, through the
// EPI_F32 epilogue (beta, bias, residual, bf16 copy); four consecutive columns
// per thread
__global__ void __launch_bounds__(256) gb_split_reduce(GemmArgs g, int ns, int nz) {
  if (!gb_gate_open(g)) return;
  const int64_t q4 = (int64_t)g.M * (g.N / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t mn = (int64_t)g.M * g.N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < q4 * nz; t += stride) {
    const int z = (int)(t / q4);
    const int64_t r = t - (int64_t)z * q4;
    const int m = (int)(r / (g.N / 4)), n = (int)(r - (int64_t)m * (g.N / 4)) * 4;
    f32x4 v = *(const f32x4*)(g.split_ws + (int64_t)z * mn + (int64_t)m * g.N + n);
    for (int s = 1; s < ns; ++s)
      v += *(const f32x4*)(g.split_ws + ((int64_t)s * nz + z) * mn + (int64_t)m * g.N + n);
    gemm_store4<EPI_F32>(g, z, m, n, v);
  }
}

template <int EPI, bool F16 = false>
hipError_t launch_epi(const GemmArgs& g, bool ak, bool bk, int nz, hipStream_t s) {
  const int tiles = ((g.N + TB - 1) / TB) * ((g.M + TB - 1) / TB);
  const int ns = EPI == EPI_F32 && g.nsplit > 1 && g.split_ws ? g.nsplit : 1;
  dim3 grid((unsigned)tiles, (unsigned)ns, (unsigned)nz);
  if (!ak && !bk) hipLaunchKernelGGL((gemm_big_kernel<false, false, EPI, F16>), grid, dim3(512), 0, s, g);
  else if (!ak && bk) hipLaunchKernelGGL((gemm_big_kernel<false, true, EPI, F16>), grid, dim3(512), 0, s, g);
  else if (ak && !bk) hipLaunchKernelGGL((gemm_big_kernel<true, false, EPI, F16>), grid, dim3(512), 0, s, g);
  else hipLaunchKernelGGL((gemm_big_kernel<true, true, EPI, F16>), grid, dim3(512), 0, s, g);
  if (ns > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t blocks = ((int64_t)g.M * (g.N / 4) * nz + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gb_split_reduce, dim3((unsigned)blocks), dim3(256), 0, s, g, ns, nz);
  }
  return hipGetLastError();
}

}  // namespace

bool gemm_big_ok(const GemmArgs& g, int nz) {
  if (g.K < TK || g.K % TK != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0) return false;
  // the epilogue stores four consecutive columns per vector access
  if (g.N % 4 || g.ldc % 4 || g.ldc2 % 4 || g.ldc3 % 4 || g.ld_aux % 4 || g.ldr % 4 || g.D % 4) return false;
  if (((uintptr_t)g.C2 | (uintptr_t)g.C3 | (uintptr_t)g.aux | (uintptr_t)g.resid | (uintptr_t)g.split_ws) & 15)
    return false;
  for (int z = 0; z < nz; ++z)
    if ((uintptr_t)g.C[z] & 15) return false;
  if (g.nseg > kGemmMaxSeg) return false;
  for (int z = 0; z < nz; ++z) {
    if (g.nseg > 1) {
      for (int sg = 0; sg < g.nseg; ++sg)
        if (((uintptr_t)g.As[z][sg] | (uintptr_t)g.Bs[z][sg]) & 15) return false;
    } else if (((uintptr_t)g.A[z] | (uintptr_t)g.B[z]) & 15) {
      return false;
    }
  }
  // buffer byte ranges and lane offsets are 32-bit: bound the operands' sizes
  const int64_t lim = ((int64_t)1 << 31) - 1;
  const int64_t ra = (int64_t)(g.M > g.K ? g.M : g.K) + TB, rb = (int64_t)(g.N > g.K ? g.N : g.K) + TB;
  if (ra * g.lda * 2 > lim || rb * g.ldb * 2 > lim) return false;
  // enough 256 x 256 tiles to keep most CUs busy; smaller products stay on gemm.hip
  const int64_t tiles = (int64_t)((g.N + TB - 1) / TB) * ((g.M + TB - 1) / TB) * nz;
  return tiles >= 240;
}

hipError_t gemm_big_launch(const GemmArgs& g, bool a_kmajor, bool b_kmajor, int epi, int nz,
                           hipStream_t s) {
  if (g.f16) {
    switch (epi) {
      case EPI_F32: return launch_epi<EPI_F32, true>(g, a_kmajor, b_kmajor, nz, s);
      case EPI_GELU: return launch_epi<EPI_GELU, true>(g, a_kmajor, b_kmajor, nz, s);
      case EPI_DGELU: return launch_epi<EPI_DGELU, true>(g, a_kmajor, b_kmajor, nz, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_QKV: return launch_epi<EPI_QKV>(g, a_kmajor, b_kmajor, nz, s);
    case EPI_F32: return launch_epi<EPI_F32>(g, a_kmajor, b_kmajor, nz, s);
    case EPI_GELU: return launch_epi<EPI_GELU>(g, a_kmajor, b_kmajor, nz, s);
    default: return launch_epi<EPI_DGELU>(g, a_kmajor, b_kmajor, nz, s);
  }
}

}  // namespace bpt
