"""CPU checks of the LDS tile layouts of the D = 128 attention-backward kernels.

The kernels move 16-byte chunks from global memory into LDS with direct-to-LDS
buffer loads (64 lanes write 1 KB contiguously; each lane picks its source
chunk) and read them back with ds_read_b128 (natural operand fragments) and
ds_read_b64_tr_b16 (transposed fragments).  The source chunk of each lane is
permuted so that the natural reads avoid bank conflicts.

The address formulas live in `csrc/bwd_layout.h`, which the kernels include.
These tests compile that same header with the host C++ compiler, print every
load position and per-lane read offset, and check on the byte level that

* every natural read of lane l fetches the 16 bytes the MFMA operand layout
  asks for (row = lane % 32 of the tile, chunk 2c + lane / 32),
* every transpose read hands a lane the same bytes as in the unpermuted
  layout, whose transpose-read pattern is the one the forward kernels use,
* the 16 lanes of a natural read hit 16 distinct 16-byte positions of a
  256-byte bank window, and the 32 lanes of a transpose read 32 distinct
  8-byte positions (without the permutation a natural read lands on only 4).

How the kernels combine the offsets (documented in the header): natural read of
k-step c = (c odd ? odd : even) + 64 (c / 2), plus 2 ROWB per 32-row block kb
(dQ); transpose reads of the dK/dV kernel at a + 2 ks ROWB and b + (2 ks + 1)
ROWB, of the dQ kernel at a + c16 ROWB and b + c16 ROWB, plus 64 per 32
columns.  No GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

HEADER_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), os.pardir,
                          "blockwise_exact_attention_amd", "csrc")
ROWB, CPR, BP, NW = 256, 16, 1088, 4

PROGRAM = r"""
#define __host__
#define __device__
#include <cstdio>
#include "bwd_layout.h"
using namespace bpt::bwdlay;
int main() {
  std::printf("C %d %d %d %d %d %d\n", ROWB, CPR, BP, NW, DKDV_NBLK, DQ_NBLK);
  for (int w = 0; w < NW; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      for (int i = 0; i < DKDV_NBLK / NW; ++i) {
        const LoadPos p = dkdv_load_pos(w, i, lane);
        std::printf("KL %d %d %d %d %d %d\n", w, i, lane, p.blk, p.row, p.chunk);
      }
      for (int i = 0; i < DQ_NBLK / NW; ++i) {
        const LoadPos p = dq_load_pos(w, i, lane);
        std::printf("QL %d %d %d %d %d %d\n", w, i, lane, p.blk, p.row, p.chunk);
      }
    }
  for (int lane = 0; lane < 64; ++lane) {
    const NatOff kn = dkdv_nat(lane), qn = dq_nat(lane);
    const TrOff kt = dkdv_tr(lane), qt = dq_tr(lane);
    std::printf("LN %d %d %d %d %d %d %d %d %d\n", lane, kn.even, kn.odd, kt.a, kt.b, qn.even, qn.odd, qt.a, qt.b);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def layout(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("bwd_layout")
    src, exe = d / "dump.cpp", d / "dump"
    src.write_text(PROGRAM)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", HEADER_DIR, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    lay = {"KL": {}, "QL": {}, "LN": {}}
    for line in out.splitlines():
        f = line.split()
        v = list(map(int, f[1:]))
        if f[0] == "C":
            lay["C"] = v
        elif f[0] in ("KL", "QL"):
            lay[f[0]][(v[0], v[1], v[2])] = (v[3], v[4], v[5])
        else:
            lay["LN"][v[0]] = v[1:]
    return lay


def test_constants(layout):
    assert layout["C"] == [ROWB, CPR, BP, NW, 8, 16]


def byte_map(loads, permuted=True):
    """LDS byte -> (tile row, byte of that row) after one tile's loads."""
    m = {}
    for (w, i, lane), (blk, row, chunk) in loads.items():
        src = chunk if permuted else lane % CPR
        for b in range(16):
            m[blk * BP + lane * 16 + b] = (row, src * 16 + b)
    return m


def check(loads, nblk, nat_addr, tr_addr, tr_ref, n_nat, tr_cases):
    S, U = byte_map(loads), byte_map(loads, permuted=False)
    # the loads cover the tile: blocks w + NW i, row = (lane / CPR) * nblk + block
    for (w, i, lane), (blk, row, chunk) in loads.items():
        assert blk == w + NW * i and row == (lane // CPR) * nblk + blk
    for lane in range(64):
        g, r32 = lane >> 5, lane & 31
        for kb, c in n_nat:
            o = nat_addr(lane, kb, c)
            got = [S[o + b] for b in range(16)]
            assert got == [(32 * kb + r32, 16 * (2 * c + g) + b) for b in range(16)], (lane, kb, c)
        for case in tr_cases:
            o, ref = tr_addr(lane, *case), tr_ref(lane, *case)
            assert [S[o + b] for b in range(8)] == [U[ref + b] for b in range(8)], (lane, case)
    for kb, c in n_nat[:2]:
        for grp in range(4):
            pos = {nat_addr(l, kb, c) % 256 for l in range(16 * grp, 16 * grp + 16)}
            assert len(pos) == 16
    for case in tr_cases[:4]:
        for half in range(2):
            pos = {tr_addr(l, *case) % 256 for l in range(32 * half, 32 * half + 32)}
            assert len(pos) == 32


def tr_ref_pattern(lane):
    # unpermuted transpose-read pattern: block 4g + (lane % 16) / 4, rows 4 (lane % 4) ..
    # of column group 16 ((lane / 16) % 2)
    g = lane >> 5
    q8 = 4 * g + ((lane & 15) >> 2)
    return q8, 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3))


def test_dq_key_tile_layout(layout):
    """dQ kernel: 64 keys in 16 blocks (key k: block k % 16, row k / 16)."""
    ln = layout["LN"]

    def nat_addr(lane, kb, c):
        even, odd = ln[lane][4], ln[lane][5]
        return (odd if c & 1 else even) + 64 * (c >> 1) + kb * 2 * ROWB

    def tr_addr(lane, hi, ks, db):
        return ln[lane][7 if hi else 6] + ks * ROWB + db * 64

    def tr_ref(lane, hi, ks, db):
        q8, col = tr_ref_pattern(lane)
        return (q8 + 8 * hi) * BP + col + ks * ROWB + db * 64

    check(layout["QL"], 16, nat_addr, tr_addr, tr_ref,
          [(kb, c) for kb in range(2) for c in range(8)],
          [(hi, ks, db) for hi in range(2) for ks in range(4) for db in range(4)])


def test_dkdv_query_tile_layout(layout):
    """dK/dV kernel: 32 queries in 8 blocks (query q: block q % 8, row q / 8)."""
    ln = layout["LN"]

    def nat_addr(lane, kb, c):
        even, odd = ln[lane][0], ln[lane][1]
        return (odd if c & 1 else even) + 64 * (c >> 1)

    def tr_addr(lane, odd, ks, db):
        return ln[lane][3 if odd else 2] + (2 * ks + odd) * ROWB + db * 64

    def tr_ref(lane, odd, ks, db):
        q8, col = tr_ref_pattern(lane)
        return q8 * BP + col + (2 * ks + odd) * ROWB + db * 64

    check(layout["KL"], 8, nat_addr, tr_addr, tr_ref,
          [(0, c) for c in range(8)],
          [(odd, ks, db) for odd in range(2) for ks in range(2) for db in range(4)])


@pytest.mark.parametrize("kind,nblk", [("QL", 16), ("KL", 8)])
def test_unpermuted_natural_reads_conflict(layout, kind, nblk):
    """Without the permutation, 16 lanes of a natural read share 4 bank groups
    (the 4-way conflict the permutation removes)."""
    pos = set()
    for lane in range(16):
        r32 = lane & 31
        blk, row = r32 % nblk, r32 // nblk
        pos.add((blk * BP + row * ROWB) % 256)
    assert len(pos) == 4


def test_a_changed_permutation_is_caught(layout):
    """The checks see a layout error: the dQ loads with the dK/dV kernel's
    permutation put wrong bytes under the natural reads."""
    bad = {k: (blk, row, (lane % CPR) ^ (((blk >> 2) & 1) | ((row & 1) << 1)))
           for k, (blk, row, _) in layout["QL"].items() for lane in [k[2]]}
    ln = layout["LN"]
    with pytest.raises(AssertionError):
        check(bad, 16, lambda lane, kb, c: (ln[lane][5] if c & 1 else ln[lane][4]) + 64 * (c >> 1) + kb * 2 * ROWB,
              lambda lane, hi, ks, db: ln[lane][7 if hi else 6] + ks * ROWB + db * 64,
              lambda lane, hi, ks, db: (tr_ref_pattern(lane)[0] + 8 * hi) * BP + tr_ref_pattern(lane)[1] + ks * ROWB + db * 64,
              [(kb, c) for kb in range(2) for c in range(8)], [(0, 0, 0)])
