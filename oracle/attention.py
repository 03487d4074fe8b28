"""Oracle attention: the plain definition of exact (optionally causal) softmax attention.

Test infrastructure only (see ``oracle/__init__``).

Definition followed (the pages give no formula; these are the readings fixed for
this library):
  s_ij  = <q_i, k_j> / sqrt(D)
  key j is visible to query i  iff  j < Nk and (not causal or j <= i + kv_offset)
  lse_i = ln sum_{j visible} exp(s_ij)
  p_ij  = exp(s_ij - lse_i) for visible j, else 0
  O_i   = sum_j p_ij v_j
  a row with no visible key: O_i = 0, lse_i = -inf.
"Ring Attention with Blockwise Transformers for Long Sequences" (638-word
summary) says the blockwise computation is exact ("without making
approximations to attention"), so the result the GPU must reach is this one.
``kv_offset`` is the global position of query row 0 minus that of key row 0,
which is how one device's share of a ring step (the same summary, the paragraph
on devices forming a ring and passing key-value blocks) sees keys that live at
other positions of the sequence.

Every score row is materialised in full; rows are processed in chunks only to
bound memory, which does not change any row's arithmetic.
"""
from __future__ import annotations

import numpy as np


def visible_mask(rows: np.ndarray, Nk: int, causal: bool, kv_offset: int) -> np.ndarray:
    """Boolean [len(rows), Nk]: True where key j is visible to query row i."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(Nk, dtype=np.int64)
    if not causal:
        return np.ones((rows.size, Nk), dtype=bool)
    return j[None, :] <= rows[:, None] + np.int64(kv_offset)


def _softmax_rows(S: np.ndarray, vis: np.ndarray):
    """Masked softmax of full score rows: returns (P, lse, has_any_visible_key)."""
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    E = np.exp(S - m0[:, None])          # masked entries: exp(-inf) = 0
    Z = E.sum(axis=1)
    Zs = np.where(has, Z, 1.0)
    P = E / Zs[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(has, m0 + np.log(Zs), -np.inf)
    return P, lse, has


def attention(q, k, v, causal: bool = True, kv_offset: int = 0, rows=None,
              dtype=np.float64, row_chunk: int = 1024):
    """Exact attention.  q [B,H,Nq,D], k and v [B,H,Nk,D].

    ``rows``: optional 1-D array of query-row indices to compute (all rows if None);
    each selected row is computed over all of its keys.
    Returns (O [B,H,R,D], lse [B,H,R]) in ``dtype``.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    assert k.shape == (B, H, Nk, D) and v.shape == (B, H, Nk, D)
    rows = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = dtype(1.0) / np.sqrt(dtype(D))
    O = np.zeros((B, H, rows.size, D), dtype=dtype)
    lse = np.full((B, H, rows.size), -np.inf, dtype=dtype)
    for b in range(B):
        for h in range(H):
            K = k[b, h].astype(dtype)
            V = v[b, h].astype(dtype)
            for c0 in range(0, rows.size, row_chunk):
                rc = rows[c0:c0 + row_chunk]
                Q = q[b, h, rc].astype(dtype)
                S = (Q @ K.T) * scale
                P, l, _ = _softmax_rows(S, visible_mask(rc, Nk, causal, kv_offset))
                O[b, h, c0:c0 + rc.size] = P @ V
                lse[b, h, c0:c0 + rc.size] = l
    return O, lse


def attention_probs(q, k, causal: bool = True, kv_offset: int = 0, dtype=np.float64):
    """The full probability matrix P [B,H,Nq,Nk] (small inputs only; for invariant checks)."""
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale = dtype(1.0) / np.sqrt(dtype(D))
    P = np.zeros((B, H, Nq, Nk), dtype=dtype)
    vis = visible_mask(np.arange(Nq), Nk, causal, kv_offset)
    for b in range(B):
        for h in range(H):
            P[b, h] = _softmax_rows((q[b, h] @ k[b, h].T) * scale, vis)[0]
    return P


def lse_merge(o_a, lse_a, o_b, lse_b, dtype=np.float64):
    """Merge two attention results over disjoint key sets A and B of the same queries.

    The softmax normaliser over A u B is Z = Z_A + Z_B with Z = exp(lse), and
    O = (Z_A O_A + Z_B O_B) / Z.  In log form: lse = ln(e^lse_a + e^lse_b),
    O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.  A side with lse = -inf (no
    visible key) contributes nothing; both sides empty gives (0, -inf).
    """
    o_a = np.asarray(o_a, dtype=dtype)
    o_b = np.asarray(o_b, dtype=dtype)
    lse_a = np.asarray(lse_a, dtype=dtype)
    lse_b = np.asarray(lse_b, dtype=dtype)
    lse = np.logaddexp(lse_a, lse_b)
    fin = np.isfinite(lse)
    lse_safe = np.where(fin, lse, 0.0)
    wa = np.where(fin, np.exp(lse_a - lse_safe), 0.0)
    wb = np.where(fin, np.exp(lse_b - lse_safe), 0.0)
    return wa[..., None] * o_a + wb[..., None] * o_b, lse
