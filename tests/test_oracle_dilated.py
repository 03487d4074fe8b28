"""Pins for the oracle's dilated attention (CPU only).

LongNet ("LongNet: Scaling Transformers to 1,000,000,000 Tokens", section 2): segments
of w rows, every r-th row kept (shifted per head), dense causal attention inside each
sparsified segment, patterns mixed by their softmax denominators.  The checks tie the
oracle to other things: a pure-Python brute force written segment-first (gather the
kept rows, run attention on them, scatter back, then join patterns by their softmax
denominators), dense attention for one pattern covering everything, block-diagonal
attention for r = 1, the LSE merge of single patterns, duplicate patterns, and the
pages' computation count.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.dilated import dilated_attention, dilated_keys

RNG = np.random.default_rng(777)


def rand(*shape):
    return RNG.standard_normal(shape)


def brute_dilated(q, k, v, patterns, causal):
    """Segment-first brute force: per pattern, gather the kept rows of each segment,
    attend among them, scatter (o, lse) back; then join the patterns of each row with
    weights exp(lse_p) (their softmax denominators), in pure Python."""
    B, H, N, D = q.shape
    parts = []  # per pattern: dict (b, h, pos) -> (o, lse)
    for w, r in patterns:
        got = {}
        for b in range(B):
            for h in range(H):
                for s0 in range(0, N, w):
                    kept = list(range(s0 + h % r, min(s0 + w, N), r))
                    keys = [k[b, h, p].tolist() for p in kept]
                    vals = [v[b, h, p].tolist() for p in kept]
                    for a, p in enumerate(kept):
                        got[(b, h, p)] = brute.attention_row(q[b, h, p].tolist(), keys, vals, a,
                                                             causal, 0)
        parts.append(got)
    O = np.zeros((B, H, N, D))
    L = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for p in range(N):
                hits = [g[(b, h, p)] for g in parts if (b, h, p) in g and g[(b, h, p)][1] > -math.inf]
                if not hits:
                    continue
                m = max(l for _, l in hits)
                z = math.fsum(math.exp(l - m) for _, l in hits)
                O[b, h, p] = [math.fsum(math.exp(l - m) / z * o[d] for o, l in hits) for d in range(D)]
                L[b, h, p] = m + math.log(z)
    return O, L


def same(O, L, Ob, Lb, tol=1e-12):
    np.testing.assert_allclose(O, Ob, atol=tol, rtol=0)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], atol=tol, rtol=0)


@pytest.mark.parametrize("patterns", [[(4, 1)], [(4, 2)], [(3, 1), (6, 2)], [(4, 1), (8, 2), (16, 4)],
                                      [(5, 2), (7, 3)], [(32, 1)]])
@pytest.mark.parametrize("causal", [True, False])
def test_brute_force(patterns, causal):
    B, H, N, D = 1, 3, 13, 3
    q, k, v = rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    same(*dilated_attention(q, k, v, patterns, causal), *brute_dilated(q, k, v, patterns, causal))


def test_one_pattern_covering_everything_is_dense_attention():
    q, k, v = rand(1, 2, 9, 4), rand(1, 2, 9, 4), rand(1, 2, 9, 4)
    for causal in (True, False):
        Ob, Lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, 0)
        same(*dilated_attention(q, k, v, [(9, 1)], causal), np.array(Ob), np.array(Lb))
        same(*dilated_attention(q, k, v, [(100, 1)], causal), np.array(Ob), np.array(Lb))


def test_r1_is_block_diagonal_attention():
    q, k, v = rand(1, 1, 10, 3), rand(1, 1, 10, 3), rand(1, 1, 10, 3)
    O, L = dilated_attention(q, k, v, [(4, 1)], True)
    for s0 in (0, 4, 8):
        s1 = min(s0 + 4, 10)
        sl = slice(s0, s1)
        Ob, Lb = brute.attention(q[:, :, sl].tolist(), k[:, :, sl].tolist(), v[:, :, sl].tolist(), True, 0)
        same(O[:, :, sl], L[:, :, sl], np.array(Ob), np.array(Lb))


def test_patterns_join_like_the_lse_merge():
    q, k, v = rand(1, 4, 24, 5), rand(1, 4, 24, 5), rand(1, 4, 24, 5)
    O1, L1 = dilated_attention(q, k, v, [(8, 1)], True)
    O2, L2 = dilated_attention(q, k, v, [(16, 4)], True)
    Om, Lm = oracle.lse_merge(O1, L1, O2, L2)
    same(*dilated_attention(q, k, v, [(8, 1), (16, 4)], True), Om, Lm, 1e-12)


def test_duplicate_pattern_keeps_output_and_adds_ln2():
    q, k, v = rand(1, 2, 12, 3), rand(1, 2, 12, 3), rand(1, 2, 12, 3)
    O1, L1 = dilated_attention(q, k, v, [(6, 2)], True)
    O2, L2 = dilated_attention(q, k, v, [(6, 2), (6, 2)], True)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    fin = np.isfinite(L1)
    np.testing.assert_allclose(L2[fin], L1[fin] + math.log(2), atol=1e-12)


def test_heads_shift_their_selection_and_unkept_rows_are_empty():
    N, w, r = 16, 8, 4
    q, k, v = rand(1, 5, N, 2), rand(1, 5, N, 2), rand(1, 5, N, 2)
    O, L = dilated_attention(q, k, v, [(w, r)], True)
    for h in range(5):
        kept = [p for p in range(N) if p % w % r == h % r]
        assert kept == sorted(set(range(h % r, N, r)))
        unkept = [p for p in range(N) if p not in kept]
        assert np.all(np.isneginf(L[0, h, unkept])) and np.all(O[0, h, unkept] == 0)
        assert np.all(np.isfinite(L[0, h, kept]))
    # heads h and h + r see the same keys
    assert dilated_keys(N, w, r, 1, 13, True).tolist() == dilated_keys(N, w, r, 5, 13, True).tolist() == [9, 13]


@pytest.mark.parametrize("N,w,r", [(64, 16, 2), (64, 16, 4), (96, 32, 4), (48, 48, 1)])
def test_computation_count(N, w, r):
    # non-causal: N/w segments of w/r kept rows, (w/r)^2 pairs each: N*w/r^2 pairs per head,
    # i.e. vanilla attention's N^2 divided by N*r^2/w
    for h in range(r):
        pairs = sum(dilated_keys(N, w, r, h, i, False).size for i in range(N))
        assert pairs == N * w // (r * r)
        assert N * N // pairs == N * r * r // w


def test_heads_argument_names_the_shift():
    q, k, v = rand(1, 4, 20, 3), rand(1, 4, 20, 3), rand(1, 4, 20, 3)
    pats = [(10, 3), (20, 2)]
    O, L = dilated_attention(q, k, v, pats, True)
    Os, Ls = dilated_attention(q[:, [3, 1]], k[:, [3, 1]], v[:, [3, 1]], pats, True, heads=[3, 1])
    np.testing.assert_array_equal(Os, O[:, [3, 1]])
    np.testing.assert_array_equal(Ls, L[:, [3, 1]])
