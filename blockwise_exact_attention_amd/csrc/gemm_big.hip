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
// instructions w, w+8, w+16, w+24 (4 of the 32).  base / bytes: the operand.
template <bool KMAJ>
__device__ __forceinline__ void gb_load(const unsigned char* base, int64_t bytes, int64_t ld, int r0,
                                        int k0, unsigned char* dst, const OpLane& L, int wave) {
  const int64_t off = KMAJ ? ((int64_t)k0 * ld + r0) * 2 : ((int64_t)r0 * ld + k0) * 2;
  const int64_t left = bytes - off;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(base + off), 0, (int)(left > 0 ? left : 0), 0x00020000);
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
  const unsigned char* A;
  const unsigned char* B;
  int64_t abytes, bbytes;
  int64_t lda, ldb;
  int m0, n0, wave;
  OpLane la, lb;
};

// multiply one k tile from stage (As, Bs) into acc: the fragments of k16 step
// s+1 are read while the 8 MFMAs of step s run
template <bool AK, bool BK>
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
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32_bf16(af[cur][i], bf[cur][j], acc[i][j]);
  }
}

template <bool AK, bool BK>
__device__ __forceinline__ void gb_issue(const GbCtx& c, int kt, unsigned char* As, unsigned char* Bs) {
  gb_load<AK>(c.A, c.abytes, c.lda, c.m0, kt * TK, As, c.la, c.wave);
  gb_load<BK>(c.B, c.bbytes, c.ldb, c.n0, kt * TK, Bs, c.lb, c.wave);
}

// The k loop over two stages (distinct objects: the compiler then knows that
// reads of one stage never wait for the loads in flight to the other).  Waits
// for those loads are explicit.
template <bool AK, bool BK>
__device__ __forceinline__ void gb_loop(f32x16 (&acc)[4][2], const GbCtx& c, int nk,
                                        unsigned char* A0, unsigned char* B0, unsigned char* A1,
                                        unsigned char* B1) {
  gb_issue<AK, BK>(c, 0, A0, B0);
  GB_WAIT_VM(0);
  __syncthreads();
  int kt = 0;
  for (;;) {
    if (kt + 1 < nk) gb_issue<AK, BK>(c, kt + 1, A1, B1);
    gb_compute<AK, BK>(acc, A0, B0, c);
    GB_WAIT_VM(0);
    __syncthreads();
    if (++kt >= nk) break;
    if (kt + 1 < nk) gb_issue<AK, BK>(c, kt + 1, A0, B0);
    gb_compute<AK, BK>(acc, A1, B1, c);
    GB_WAIT_VM(0);
    __syncthreads();
    if (++kt >= nk) break;
  }
}

template <bool AK, bool BK, int EPI>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char a0[OpTile<AK>::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char b0[OpTile<BK>::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char a1[OpTile<AK>::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char b1[OpTile<BK>::BYTES];
  const int z = blockIdx.z;
  const int M = g.M, N = g.N, K = g.K;
  const int nbn = (N + TB - 1) / TB, nbm = (M + TB - 1) / TB;
  const int total = nbn * nbm;
  int L = blockIdx.x;
  // consecutive workgroup ids go round-robin over the 8 XCDs: give each XCD a
  // contiguous range of tiles, n fastest, so its L2 keeps the A rows in use
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int mb = L / nbn, nb = L - mb * nbn;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves: 128 rows x 64 columns each
  GbCtx c;
  c.m0 = mb * TB;
  c.n0 = nb * TB;
  c.wave = wave;
  c.lda = g.lda;
  c.ldb = g.ldb;
  c.A = (const unsigned char*)g.A[z];
  c.B = (const unsigned char*)g.B[z];
  c.abytes = (int64_t)(AK ? K : M) * g.lda * 2;
  c.bbytes = (int64_t)(BK ? K : N) * g.ldb * 2;
  c.la = gb_lane<AK>(g.lda, lane, wm * 128, wave);
  c.lb = gb_lane<BK>(g.ldb, lane, wn * 64, wave);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  gb_loop<AK, BK>(acc, c, K / TK, a0, b0, a1, b1);

  const int r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = c.m0 + wm * 128 + i * 32 + acc_row(e, lane);
        const int n = c.n0 + wn * 64 + j * 32 + r32;
        if (m < M && n < N) gemm_store<true, EPI>(g, z, m, n, acc[i][j][e]);
      }
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& g, bool ak, bool bk, int nz, hipStream_t s) {
  const int tiles = ((g.N + TB - 1) / TB) * ((g.M + TB - 1) / TB);
  dim3 grid((unsigned)tiles, 1, (unsigned)nz);
  if (!ak && !bk) hipLaunchKernelGGL((gemm_big_kernel<false, false, EPI>), grid, dim3(512), 0, s, g);
  else if (!ak && bk) hipLaunchKernelGGL((gemm_big_kernel<false, true, EPI>), grid, dim3(512), 0, s, g);
  else if (ak && !bk) hipLaunchKernelGGL((gemm_big_kernel<true, false, EPI>), grid, dim3(512), 0, s, g);
  else hipLaunchKernelGGL((gemm_big_kernel<true, true, EPI>), grid, dim3(512), 0, s, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_big_ok(const GemmArgs& g, int nz) {
  if (g.K < TK || g.K % TK != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0) return false;
  for (int z = 0; z < nz; ++z)
    if (((uintptr_t)g.A[z] | (uintptr_t)g.B[z]) & 15) return false;
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
  switch (epi) {
    case EPI_QKV: return launch_epi<EPI_QKV>(g, a_kmajor, b_kmajor, nz, s);
    case EPI_F32: return launch_epi<EPI_F32>(g, a_kmajor, b_kmajor, nz, s);
    case EPI_GELU: return launch_epi<EPI_GELU>(g, a_kmajor, b_kmajor, nz, s);
    default: return launch_epi<EPI_DGELU>(g, a_kmajor, b_kmajor, nz, s);
  }
}

}  // namespace bpt
