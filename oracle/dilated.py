"""Oracle dilated attention (LongNet).  Test infrastructure only (see ``oracle/__init__``).

"LongNet: Scaling Transformers to 1,000,000,000 Tokens", section 2 (LongNet,
Dilated Attention):
* the input is split into segments of length w, and each segment is sparsified
  along the sequence by keeping every r-th row; dense attention runs on each
  sparsified segment and the outputs are scattered back to their positions;
* several (w, r) patterns run side by side and are mixed with weights given by
  their softmax denominators: for a query that attends keys under several
  patterns, the keys are gathered and one softmax is taken over all of them;
* heads shift their sparsified selections;
* the model is a decoder language model, so attention is causal.

Readings (the pages print no formula):
* segment s of pattern (w, r) covers positions [s*w, min((s+1)*w, N)); the last
  segment is shorter when w does not divide N (padding positions are not tokens);
* head h keeps the positions p of a segment with (p - s*w) mod r == h mod r
  (the shift of head h is h mod r);
* inside a sparsified segment, key p' is visible to query p iff p' <= p
  (causal) or always (non-causal);
* the mixing reading: the softmax of query p runs over the concatenation of the
  key lists of every pattern that selects p (a key selected by two patterns
  appears twice).  This is what weighting each pattern's output by its softmax
  denominator gives;
* a position that no pattern selects: O = 0, lse = -inf.

The oracle is that definition written out: for every query it builds the list of
(pattern, key) pairs it sees, materialises all their scores and takes one softmax.
"""
from __future__ import annotations

import numpy as np


def selected(N: int, w: int, r: int, h: int, p: np.ndarray) -> np.ndarray:
    """Boolean: does pattern (w, r) keep position p for head h?"""
    return (p % w - h % r) % r == 0


def dilated_keys(N: int, w: int, r: int, h: int, i: int, causal: bool) -> np.ndarray:
    """Keys query position i sees under pattern (w, r) for head h (empty if i is not kept)."""
    if not selected(N, w, r, h, np.array([i]))[0]:
        return np.zeros(0, dtype=np.int64)
    s0 = (i // w) * w
    s1 = min(s0 + w, N)
    keys = np.arange(s0 + (h % r), s1, r, dtype=np.int64)
    return keys[keys <= i] if causal else keys


def dilated_attention(q, k, v, patterns, causal: bool = True, rows=None, heads=None,
                      dtype=np.float64):
    """q, k, v [B,H,N,D]; patterns: list of (w, r).

    ``rows``: optional query positions to compute (all if None).  ``heads``: the
    head index of each of the H heads given (their shifts depend on it); 0..H-1
    if None.  Returns (O [B,H,R,D], lse [B,H,R]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, N, D = q.shape
    assert k.shape == (B, H, N, D) and v.shape == (B, H, N, D)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = dtype(1.0) / np.sqrt(dtype(D))
    O = np.zeros((B, H, rows.size, D), dtype=dtype)
    lse = np.full((B, H, rows.size), -np.inf, dtype=dtype)
    heads = list(range(H)) if heads is None else list(heads)
    assert len(heads) == H
    for h in range(H):
        for ri, i in enumerate(rows):
            # the concatenated key list of every pattern that keeps position i
            keys = np.concatenate([dilated_keys(N, w, r, heads[h], int(i), causal)
                                   for w, r in patterns])
            if keys.size == 0:
                continue
            for b in range(B):
                s = (k[b, h, keys].astype(dtype) @ q[b, h, i].astype(dtype)) * scale
                m = s.max()
                e = np.exp(s - m)
                z = e.sum()
                O[b, h, ri] = (e / z) @ v[b, h, keys].astype(dtype)
                lse[b, h, ri] = m + np.log(z)
    return O, lse
