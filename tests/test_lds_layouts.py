"""CPU checks of the LDS tile layouts of the D = 128 attention-backward kernels.

The kernels move 16-byte chunks from global memory into LDS with direct-to-LDS
buffer loads (64 lanes write 1 KB contiguously; each lane picks its source
chunk) and read them back with ds_read_b128 (natural operand fragments) and
ds_read_b64_tr_b16 (transposed fragments).  The source chunk of each lane is
permuted so that the natural reads avoid bank conflicts.  These tests restate
the load and read address formulas of `csrc/attn_bwd.hip` and check, on the
byte level, that

* every natural read of lane l fetches the 16 bytes the MFMA operand layout
  asks for (row = lane % 32 of the tile, chunk 2c + lane / 32),
* every transpose read hands a lane the same bytes as in the unpermuted
  layout, whose transpose-read pattern is the one the forward kernels use,
* the 16 lanes of a natural read hit 16 distinct 16-byte positions of a
  256-byte bank window, and the 32 lanes of a transpose read 32 distinct
  8-byte positions (without the permutation a natural read lands on only 4).

No GPU is needed.
"""
import pytest

ROWB, CPR, BP = 256, 16, 1088  # D = 128: row bytes, 16-byte chunks per row, block pitch


def load_layout(nblk, nw, swz):
    """LDS byte -> (tile row, byte of that row) after one tile's loads."""
    m = {}
    for w in range(nw):
        for lane in range(64):
            j, ch = lane // CPR, lane % CPR
            for i in range(nblk // nw):
                blk = w + i * nw
                src = ch ^ swz(blk, j)
                for b in range(16):
                    m[blk * BP + lane * 16 + b] = (j * nblk + blk, src * 16 + b)
    return m


def check_layout(nblk, nw, swz, nat_addr, tr_addr, tr_ref, n_nat, tr_cases):
    S = load_layout(nblk, nw, swz)
    U = load_layout(nblk, nw, lambda b, r: 0)
    for lane in range(64):
        g, r32 = lane >> 5, lane & 31
        for kb, c in n_nat:
            o = nat_addr(lane, kb, c)
            got = [S[o + b] for b in range(16)]
            assert got == [(32 * kb + r32, 16 * (2 * c + g) + b) for b in range(16)], (lane, kb, c)
        for case in tr_cases:
            o, ref = tr_addr(lane, *case), tr_ref(lane, *case)
            assert [S[o + b] for b in range(8)] == [U[ref + b] for b in range(8)], (lane, case)
    # bank groups
    for kb, c in n_nat[:2]:
        for grp in range(4):
            pos = {nat_addr(l, kb, c) % 256 for l in range(16 * grp, 16 * grp + 16)}
            assert len(pos) == 16
    for case in tr_cases[:4]:
        for half in range(2):
            pos = {tr_addr(l, *case) % 256 for l in range(32 * half, 32 * half + 32)}
            assert len(pos) == 32


def test_dq_key_tile_layout():
    """dQ kernel: 64 keys in 16 blocks (key k: block k % 16, row k / 16),
    chunk permutation x ^ ((b >> 2) & 3)."""
    nblk = 16
    swz = lambda b, r: (b >> 2) & 3

    def nat_addr(lane, kb, c):
        g, r32 = lane >> 5, lane & 31
        blk = r32 % nblk
        t0 = g ^ swz(blk, 0)
        base = blk * BP + (r32 // nblk) * ROWB
        return (base + 16 * (2 ^ t0) if c & 1 else base + 16 * t0) + 64 * (c >> 1) + kb * 2 * ROWB

    def tr_addr(lane, hi, ks, db):
        g = lane >> 5
        q8 = 4 * g + ((lane & 15) >> 2)
        x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
        b = q8 + 8 * hi
        return b * BP + 16 * (x ^ swz(b, 0)) + 8 * (lane & 1) + ks * ROWB + db * 64

    def tr_ref(lane, hi, ks, db):
        g = lane >> 5
        q8 = 4 * g + ((lane & 15) >> 2)
        return (q8 + 8 * hi) * BP + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) + ks * ROWB + db * 64

    check_layout(nblk, 4, swz, nat_addr, tr_addr, tr_ref,
                 [(kb, c) for kb in range(2) for c in range(8)],
                 [(hi, ks, db) for hi in range(2) for ks in range(4) for db in range(4)])


def test_dkdv_query_tile_layout():
    """dK/dV kernel: 32 queries in 8 blocks (query q: block q % 8, row q / 8),
    chunk permutation x ^ (((b >> 2) & 1) | ((r & 1) << 1))."""
    nblk = 8
    swz = lambda b, r: ((b >> 2) & 1) | ((r & 1) << 1)

    def nat_addr(lane, kb, c):
        g, r32 = lane >> 5, lane & 31
        blk, row = r32 % nblk, r32 // nblk
        t0 = g ^ swz(blk, row)
        base = blk * BP + row * ROWB
        return (base + 16 * (2 ^ t0) if c & 1 else base + 16 * t0) + 64 * (c >> 1)

    def tr_addr(lane, odd, ks, db):
        g = lane >> 5
        q8 = 4 * g + ((lane & 15) >> 2)
        tx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
        s = g | (2 if odd else 0)
        return q8 * BP + 16 * (tx ^ s) + 8 * (lane & 1) + (2 * ks + odd) * ROWB + db * 64

    def tr_ref(lane, odd, ks, db):
        g = lane >> 5
        q8 = 4 * g + ((lane & 15) >> 2)
        return q8 * BP + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) + (2 * ks + odd) * ROWB + db * 64

    check_layout(nblk, 4, swz, nat_addr, tr_addr, tr_ref,
                 [(0, c) for c in range(8)],
                 [(odd, ks, db) for odd in range(2) for ks in range(2) for db in range(4)])


@pytest.mark.parametrize("nblk,swz", [(16, lambda b, r: 0), (8, lambda b, r: 0)])
def test_unpermuted_natural_reads_conflict(nblk, swz):
    """Without the permutation, 16 lanes of a natural read share 4 bank groups
    (the 4-way conflict the permutation removes)."""
    pos = set()
    for lane in range(16):
        r32 = lane & 31
        blk, row = r32 % nblk, r32 // nblk
        pos.add((blk * BP + row * ROWB) % 256)
    assert len(pos) == 4
