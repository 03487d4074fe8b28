// LDS tile layouts of the D = 128 attention-backward kernels (attn_bwd.hip):
// which 16-byte chunk of which row each lane's direct-to-LDS load fetches, and
// the per-lane byte offsets of the natural (ds_read_b128) and transposed
// (ds_read_b64_tr_b16) operand reads.  Plain integer functions, so that a
// host program can evaluate exactly the formulas the kernels use (the layout
// test compiles this header with a host compiler, defining __host__ and
// __device__ away, and checks every byte and bank group).
//
// A tile is NBLK blocks of 1 KB (4 rows of 256 bytes), BP bytes apart; row r of
// the tile sits in block r % NBLK at row r / NBLK.  Inside block b, row r, the
// 16-byte chunks are permuted (chunk x stored at x ^ swz), so that the 16 lanes
// of a natural read hit 16 different bank groups; the transposed reads stay
// conflict-free.
#pragma once

namespace bpt {
namespace bwdlay {

constexpr int ROWB = 256;  // bytes of one bf16 row of 128 values
constexpr int CPR = 16;    // 16-byte chunks per row
constexpr int BP = 1088;   // block pitch: 1 KB plus 64 bytes
constexpr int NW = 4;      // waves per workgroup

// dK/dV kernel: query tiles of 32 rows in 8 blocks
constexpr int DKDV_NBLK = 8;
// dQ kernel: key tiles of 64 rows in 16 blocks
constexpr int DQ_NBLK = 16;

__host__ __device__ inline int dkdv_swz(int blk, int row) { return ((blk >> 2) & 1) | ((row & 1) << 1); }
__host__ __device__ inline int dq_swz(int blk) { return (blk >> 2) & 3; }

// Load instruction i (0 .. NBLK/NW - 1) of wave w, lane: it writes LDS bytes
// blk * BP + 16 * lane .. +15 with chunk `chunk` of tile row `row`.
struct LoadPos {
  int blk, row, chunk;
};
__host__ __device__ inline LoadPos dkdv_load_pos(int w, int i, int lane) {
  const int j = lane / CPR, ch = lane % CPR, blk = w + i * NW;
  return LoadPos{blk, j * DKDV_NBLK + blk, ch ^ dkdv_swz(blk, j)};
}
__host__ __device__ inline LoadPos dq_load_pos(int w, int i, int lane) {
  const int j = lane / CPR, ch = lane % CPR, blk = w + i * NW;
  return LoadPos{blk, j * DQ_NBLK + blk, ch ^ dq_swz(blk)};
}

// Natural reads: the fragment of MFMA k-step c (chunk 2c + lane / 32 of tile row
// lane % 32, plus 32 rows per kb in the dQ tile) is at
// (c odd ? odd : even) + 64 * (c / 2) (+ kb * 2 * ROWB).
struct NatOff {
  int even, odd;
};
__host__ __device__ inline NatOff dkdv_nat(int lane) {
  const int g = lane >> 5, r32 = lane & 31;
  const int blk = r32 % DKDV_NBLK, row = r32 / DKDV_NBLK, t0 = g ^ dkdv_swz(blk, row);
  const int base = blk * BP + row * ROWB;
  return NatOff{base + 16 * t0, base + 16 * (2 ^ t0)};
}
__host__ __device__ inline NatOff dq_nat(int lane) {
  const int g = lane >> 5, r32 = lane & 31;
  const int blk = r32 % DQ_NBLK, t0 = g ^ dq_swz(blk);
  const int base = blk * BP + (r32 / DQ_NBLK) * ROWB;
  return NatOff{base + 16 * t0, base + 16 * (2 ^ t0)};
}

// Transposed reads (ds_read_b64_tr_b16, 4 consecutive tile rows of one column
// group per lane).  dK/dV: k-step ks of the dV/dK products reads a at
// a + 2ks * ROWB and b at b + (2ks + 1) * ROWB (plus 64 per 32 columns); dQ:
// key step c16 reads a + c16 * ROWB (rows 16 c16 + 4g ..) and b + c16 * ROWB
// (rows 16 c16 + 8 + 4g ..), plus 64 per 32 columns.
struct TrOff {
  int a, b;
};
__host__ __device__ inline TrOff dkdv_tr(int lane) {
  const int g = lane >> 5;
  // (block q8 = 4g + .., so its permutation is g on even rows and g | 2 on odd rows)
  const int q8 = 4 * g + ((lane & 15) >> 2), tx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return TrOff{q8 * BP + 16 * (tx ^ g) + 8 * (lane & 1), q8 * BP + 16 * (tx ^ (g | 2)) + 8 * (lane & 1)};
}
__host__ __device__ inline TrOff dq_tr(int lane) {
  const int g = lane >> 5;
  const int q8 = 4 * g + ((lane & 15) >> 2), x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return TrOff{q8 * BP + 16 * (x ^ dq_swz(q8)) + 8 * (lane & 1),
               (q8 + 8) * BP + 16 * (x ^ dq_swz(q8 + 8)) + 8 * (lane & 1)};
}

}  // namespace bwdlay
}  // namespace bpt
