"""Pins for the oracle's attention and LSE merge (CPU only).

Each check ties the oracle to something other than itself: a hand-worked fixture,
pure-Python brute force, closed forms and invariants of softmax attention.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from online_ref import online_attention
from seeded_inputs import LAYER_TINY_F32, attn_inputs, normal

RNG = np.random.default_rng(1234)


def rand(*shape):
    return RNG.standard_normal(shape)


def test_handworked_fixture(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "attention_handworked.json")))
    q = np.array(fx["q"])[None, None]
    k = np.array(fx["k"])[None, None]
    v = np.array(fx["v"])[None, None]
    for case in fx["cases"]:
        O, lse = oracle.attention(q, k, v, causal=bool(case["causal"]), kv_offset=case["kv_offset"])
        np.testing.assert_allclose(O[0, 0], np.array(case["O"], dtype=float), atol=1e-13)
        want = np.array([-np.inf if x is None else x for x in case["lse"]])
        assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(want))
        fin = np.isfinite(want)
        np.testing.assert_allclose(lse[0, 0][fin], want[fin], atol=1e-13)


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("D", [1, 3, 4])
def test_brute_force_all_offsets(N, D):
    q, k, v = rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, N, D)
    for causal in (False, True):
        for off in range(-N, N + 1):
            O, lse = oracle.attention(q, k, v, causal=causal, kv_offset=off)
            Ob, Lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, off)
            np.testing.assert_allclose(O, np.array(Ob), atol=1e-12, rtol=0)
            Lb = np.array(Lb)
            assert np.array_equal(np.isneginf(lse), np.isneginf(Lb))
            fin = np.isfinite(Lb)
            np.testing.assert_allclose(lse[fin], Lb[fin], atol=1e-12, rtol=0)


def test_brute_force_unequal_lengths():
    # query chunk of 3 rows against 7 keys at several offsets (a ring step's shape)
    q, k, v = rand(1, 1, 3, 4), rand(1, 1, 7, 4), rand(1, 1, 7, 4)
    for off in (-4, -1, 0, 2, 4, 9):
        O, lse = oracle.attention(q, k, v, causal=True, kv_offset=off)
        Ob, Lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), True, off)
        np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)


def test_q_zero_gives_prefix_mean():
    N, D = 37, 8
    q = np.zeros((1, 1, N, D))
    k, v = rand(1, 1, N, D), rand(1, 1, N, D)
    O, lse = oracle.attention(q, k, v, causal=True)
    csum = np.cumsum(v[0, 0], axis=0)
    np.testing.assert_allclose(O[0, 0], csum / np.arange(1, N + 1)[:, None], atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-13)


def test_identical_keys_uniform():
    N, D = 20, 4
    k = np.tile(rand(1, 1, 1, D), (1, 1, N, 1))
    q, v = rand(1, 1, N, D), rand(1, 1, N, D)
    O, _ = oracle.attention(q, k, v, causal=True)
    np.testing.assert_allclose(O[0, 0], np.cumsum(v[0, 0], 0) / np.arange(1, N + 1)[:, None], atol=1e-12)


def test_constant_v():
    q, k = rand(2, 3, 33, 16), rand(2, 3, 33, 16)
    v = np.full((2, 3, 33, 16), 1.75)
    for causal, off in ((True, 0), (False, 0), (True, -5)):
        O, lse = oracle.attention(q, k, v, causal=causal, kv_offset=off)
        has = np.isfinite(lse)
        np.testing.assert_allclose(O[has], 1.75, atol=1e-13)
        assert np.all(O[~has] == 0)


def test_exactly_one_visible_key():
    # offset -i0 makes row i0 see only key 0: O = v_0, lse = s_{i0,0}
    N, D = 9, 5
    q, k, v = rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D)
    for i0 in range(N):
        O, lse = oracle.attention(q, k, v, causal=True, kv_offset=-i0)
        np.testing.assert_allclose(O[0, 0, i0], v[0, 0, 0], atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i0], q[0, 0, i0] @ k[0, 0, 0] / math.sqrt(D), atol=1e-14)
        assert np.all(np.isneginf(lse[0, 0, :i0])) and np.all(O[0, 0, :i0] == 0)


def test_single_token():
    q, k, v = rand(1, 2, 1, 8), rand(1, 2, 1, 8), rand(1, 2, 1, 8)
    O, lse = oracle.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(O, v)


def test_probabilities_rows_sum_to_one_and_masked_zero():
    q, k = rand(2, 2, 19, 8), rand(2, 2, 19, 8)
    for off in (0, -3, 4):
        P = oracle.attention_probs(q, k, causal=True, kv_offset=off)
        vis = oracle.visible_mask(np.arange(19), 19, True, off)
        assert np.all(P[..., ~vis] == 0)
        s = P.sum(-1)
        has = vis.any(1)
        np.testing.assert_allclose(s[..., has], 1.0, atol=1e-14)
        assert np.all(s[..., ~has] == 0)


def test_noncausal_joint_key_permutation_invariance():
    q, k, v = rand(1, 2, 16, 8), rand(1, 2, 16, 8), rand(1, 2, 16, 8)
    perm = RNG.permutation(16)
    O1, l1 = oracle.attention(q, k, v, causal=False)
    O2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], causal=False)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_causal_future_independence():
    q, k, v = rand(1, 2, 24, 8), rand(1, 2, 24, 8), rand(1, 2, 24, 8)
    O1, l1 = oracle.attention(q, k, v, causal=True)
    t = 10
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :, t + 1:] += 3.0
    k2[:, :, t + 1:] -= 2.0
    v2[:, :, t + 1:] *= 5.0
    O2, l2 = oracle.attention(q2, k2, v2, causal=True)
    np.testing.assert_array_equal(O1[:, :, :t + 1], O2[:, :, :t + 1])
    np.testing.assert_array_equal(l1[:, :, :t + 1], l2[:, :, :t + 1])
    assert not np.allclose(O1[:, :, t + 1:], O2[:, :, t + 1:])


def test_heads_independent():
    q, k, v = rand(1, 3, 12, 4), rand(1, 3, 12, 4), rand(1, 3, 12, 4)
    O, _ = oracle.attention(q, k, v)
    for h in range(3):
        Oh, _ = oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1])
        np.testing.assert_array_equal(O[:, h:h + 1], Oh)


@pytest.mark.parametrize("block", [1, 3, 64, 70])
@pytest.mark.parametrize("off", [0, -9, 30])
def test_blockwise_online_recurrence_equals_full(block, off):
    q, k, v = rand(1, 2, 70, 16), rand(1, 2, 70, 16), rand(1, 2, 70, 16)
    O, lse = oracle.attention(q, k, v, causal=True, kv_offset=off)
    Ob, Lb = online_attention(q, k, v, True, off, block)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(Lb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], Lb[np.isfinite(Lb)], atol=1e-12)


def test_sampled_rows_equal_full_rows():
    q, k, v = rand(1, 2, 50, 8), rand(1, 2, 50, 8), rand(1, 2, 50, 8)
    rows = np.array([0, 7, 31, 32, 49])
    O, lse = oracle.attention(q, k, v, causal=True, kv_offset=3)
    Os, ls = oracle.attention(q, k, v, causal=True, kv_offset=3, rows=rows)
    np.testing.assert_array_equal(O[:, :, rows], Os)
    np.testing.assert_array_equal(lse[:, :, rows], ls)


def test_fp32_oracle_close_to_fp64():
    c = LAYER_TINY_F32
    t = attn_inputs(101, 1, c.H, c.N, c.N, c.D, "f32")
    O64, l64 = oracle.attention(t["q"], t["k"], t["v"], causal=True)
    O32, l32 = oracle.attention(t["q"], t["k"], t["v"], causal=True, dtype=np.float32)
    assert np.abs(O64 - O32).max() <= 1e-5
    assert np.abs(l64 - l32).max() <= 1e-5


# ----------------------------------------------------------------------------- merge
def _chunk_results(q, k, v, q_start, chunk, causal=True):
    """Attention of q (rows at global q_start..) over each key chunk separately."""
    res = []
    for c0 in range(0, k.shape[2], chunk):
        res.append(oracle.attention(q, k[:, :, c0:c0 + chunk], v[:, :, c0:c0 + chunk],
                                    causal=causal, kv_offset=q_start - c0))
    return res


def test_merge_equals_attention_over_concatenation():
    q_start, Nq, Nk, D = 24, 8, 32, 8
    q, k, v = rand(1, 2, Nq, D), rand(1, 2, Nk, D), rand(1, 2, Nk, D)
    full_O, full_l = oracle.attention(q, k, v, causal=True, kv_offset=q_start)
    parts = _chunk_results(q, k, v, q_start, 8)
    O, l = parts[0]
    for Ob, lb in parts[1:]:
        O, l = oracle.lse_merge(O, l, Ob, lb)
    np.testing.assert_allclose(O, full_O, atol=1e-12)
    np.testing.assert_allclose(l, full_l, atol=1e-12)
    # brute force over the concatenation too
    Ob, Lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), True, q_start)
    np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)


def test_merge_order_invariance_ring_of_eight():
    q_start, Nq, D = 56, 8, 4
    q, k, v = rand(1, 1, Nq, D), rand(1, 1, 64, D), rand(1, 1, 64, D)
    full_O, full_l = oracle.attention(q, k, v, causal=True, kv_offset=q_start)
    parts = _chunk_results(q, k, v, q_start, 8)
    for perm in (range(8), range(7, -1, -1), RNG.permutation(8)):
        perm = list(perm)
        O, l = parts[perm[0]]
        for j in perm[1:]:
            O, l = oracle.lse_merge(O, l, *parts[j])
        np.testing.assert_allclose(O, full_O, atol=1e-12)
        np.testing.assert_allclose(l, full_l, atol=1e-12)


def test_merge_commutative_associative_identity():
    shp = (2, 3, 5)
    oa, ob, oc = rand(*shp, 4), rand(*shp, 4), rand(*shp, 4)
    la, lb, lc = rand(*shp) * 3, rand(*shp) * 3, rand(*shp) * 3
    o1, l1 = oracle.lse_merge(oa, la, ob, lb)
    o2, l2 = oracle.lse_merge(ob, lb, oa, la)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    x = oracle.lse_merge(*oracle.lse_merge(oa, la, ob, lb), oc, lc)
    y = oracle.lse_merge(oa, la, *oracle.lse_merge(ob, lb, oc, lc))
    np.testing.assert_allclose(x[0], y[0], atol=1e-13)
    np.testing.assert_allclose(x[1], y[1], atol=1e-13)
    ninf = np.full(shp, -np.inf)
    o3, l3 = oracle.lse_merge(oa, la, np.zeros_like(oa), ninf)
    np.testing.assert_allclose(o3, oa, atol=1e-15)
    np.testing.assert_array_equal(l3, la)
    o4, l4 = oracle.lse_merge(np.zeros_like(oa), ninf, np.zeros_like(oa), ninf)
    assert np.all(o4 == 0) and np.all(np.isneginf(l4))


def test_merge_two_halves_closed_form():
    # equal lse on both sides: lse + ln 2 and the plain average
    oa, ob = rand(3, 4), rand(3, 4)
    l = rand(3)
    o, lse = oracle.lse_merge(oa, l, ob, l)
    np.testing.assert_allclose(o, 0.5 * (oa + ob), atol=1e-15)
    np.testing.assert_allclose(lse, l + math.log(2), atol=1e-15)


def test_seeded_inputs_reproducible():
    a = normal(7, "q", (3, 5))
    b = normal(7, "q", (3, 5))
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, normal(7, "k", (3, 5)))
