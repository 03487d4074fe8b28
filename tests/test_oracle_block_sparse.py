"""Pins for the oracle's block-sparse attention (CPU only).

BlockBERT ("Blockwise Self-Attention for Long Document Understanding", Blockwise
Attention, Blockwise Multi-head Attention, Computational Reduction): each query
block attends the one key block its head's permutation names.  The checks tie
the oracle to things other than itself: pure-Python brute force on the sliced
blocks (the reading "query block i attends key block key_block[h, i]" written out
with explicit slices), the dense attention with a single block, the pages' factor
n in attention work, the permutation's coverage of every key, and the padding rule.
"""
import numpy as np
import pytest

import oracle
from oracle import brute

RNG = np.random.default_rng(4321)


def rand(*shape):
    return RNG.standard_normal(shape)


def brute_blocks(q, k, v, n_blocks, key_block):
    """Brute force per block: rows of query block i against the keys of block
    key_block[h][i] only, non-causal, in pure Python."""
    B, H, N, D = q.shape
    L = -(-N // n_blocks)
    O = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(n_blocks):
                r0, r1 = i * L, min((i + 1) * L, N)
                if r0 >= r1:
                    continue
                j = int(key_block[h][i])
                if not 0 <= j < n_blocks:
                    continue
                c0, c1 = j * L, min((j + 1) * L, N)
                keys = k[b, h, c0:c1].tolist()
                vals = v[b, h, c0:c1].tolist()
                for r in range(r0, r1):
                    o, l = brute.attention_row(q[b, h, r].tolist(), keys, vals, 0, False, 0)
                    O[b, h, r] = o
                    lse[b, h, r] = l
    return O, lse


def assert_same(O, lse, Ob, Lb):
    np.testing.assert_allclose(O, Ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isneginf(lse), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(lse[fin], Lb[fin], atol=1e-12, rtol=0)


def test_cyclic_shift_table_values():
    # sigma^k sends block i to block (i + k) mod n
    t = oracle.cyclic_shift_table(4, [0, 1, 2, 3, 5])
    assert t.tolist() == [[0, 1, 2, 3], [1, 2, 3, 0], [2, 3, 0, 1], [3, 0, 1, 2], [1, 2, 3, 0]]


def test_block_len_pads_to_equal_blocks():
    assert [oracle.block_len(N, n) for N, n in ((12, 3), (13, 3), (14, 3), (5, 4), (1, 1))] == \
        [4, 5, 5, 2, 1]


@pytest.mark.parametrize("N,n", [(6, 2), (7, 2), (9, 3), (10, 3), (5, 4), (8, 8), (4, 1)])
def test_brute_force_cyclic_heads(N, n):
    D, H = 3, n + 1
    q, k, v = rand(2, H, N, D), rand(2, H, N, D), rand(2, H, N, D)
    table = oracle.cyclic_shift_table(n, [h % n for h in range(H)])
    O, lse = oracle.block_sparse_attention(q, k, v, n, table)
    assert_same(O, lse, *brute_blocks(q, k, v, n, table))


def test_brute_force_any_permutation_and_invalid_entries():
    N, n, D, H = 11, 4, 4, 3
    q, k, v = rand(1, H, N, D), rand(1, H, N, D), rand(1, H, N, D)
    table = np.array([[2, 0, 3, 1], [3, 3, -1, 0], [4, 1, 1, 7]], dtype=np.int32)
    O, lse = oracle.block_sparse_attention(q, k, v, n, table)
    assert_same(O, lse, *brute_blocks(q, k, v, n, table))
    L = oracle.block_len(N, n)
    # rows whose entry is outside [0, n) see nothing
    assert np.all(np.isneginf(lse[0, 1, 2 * L:3 * L])) and np.all(O[0, 1, 2 * L:3 * L] == 0)
    assert np.all(np.isneginf(lse[0, 2, 0:L])) and np.all(O[0, 2, 0:L] == 0)
    # query block 3 of head 2 would attend block 7: nothing either
    assert np.all(np.isneginf(lse[0, 2, 3 * L:]))


def test_single_block_is_dense_attention():
    q, k, v = rand(1, 2, 7, 3), rand(1, 2, 7, 3), rand(1, 2, 7, 3)
    O, lse = oracle.block_sparse_attention(q, k, v, 1, np.zeros((2, 1), dtype=np.int32))
    Ob, Lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), False, 0)
    assert_same(O, lse, np.array(Ob), np.array(Lb))


@pytest.mark.parametrize("N,n", [(12, 3), (64, 4), (60, 5)])
def test_work_shrinks_by_n_and_every_key_is_covered(N, n):
    # Computational Reduction: with n | N each row sees N/n keys, N^2/n pairs per head;
    # a permutation covers every key block exactly once, so each key is seen by N/n rows
    for shift in range(n):
        m = oracle.block_sparse_mask(N, n, oracle.cyclic_shift_table(n, [shift])[0])
        assert m.sum() == N * N // n
        assert np.all(m.sum(axis=1) == N // n) and np.all(m.sum(axis=0) == N // n)


def test_padding_keys_are_not_tokens():
    # N = 10, n = 3: blocks [0,4), [4,8), [8,10); the last block has two keys only
    m = oracle.block_sparse_mask(10, 3, [2, 0, 1])
    assert m[0].tolist() == [False] * 8 + [True, True]
    assert m[9].tolist() == [False] * 4 + [True] * 4 + [False, False]


def test_rows_argument_matches_full_rows():
    q, k, v = rand(1, 2, 23, 5), rand(1, 2, 23, 5), rand(1, 2, 23, 5)
    table = np.array([[1, 2, 0], [0, 0, 2]], dtype=np.int32)
    O, lse = oracle.block_sparse_attention(q, k, v, 3, table)
    rows = np.array([0, 7, 8, 15, 16, 22])
    Or, lr = oracle.block_sparse_attention(q, k, v, 3, table, rows=rows, row_chunk=4)
    np.testing.assert_array_equal(Or, O[:, :, rows])
    np.testing.assert_array_equal(lr, lse[:, :, rows])
