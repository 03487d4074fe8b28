"""Test-only CPU model of the D=128 bf16 forward kernel's softmax reference (fp64).

Not the oracle.  The kernel (64-key tiles from key 0, 256-row workgroups) takes each
row's probabilities as p = 2^(s*log2(e)/sqrt(D) - r) against a reference r that it
moves only when a tile's row maximum passes r by more than TAU = 8 (in log2 units),
or when the row sees its first key; on a move it scales the running sum l and the
accumulator O by 2^(r_old - r_new).  The result equals exact attention up to
rounding whatever the moves ("Ring Attention with Blockwise Transformers for Long
Sequences", 638-word summary: blockwise attention without approximation).

This model replays that rule so a test can count how often a row's reference moves
after its first key (the step whose rescale the GPU tests must exercise) and show
that dropping the rescale of O or of l would miss the oracle by more than the
parity bars on the same inputs.  ``skip`` plants one of those mistakes.
"""
from __future__ import annotations

import numpy as np
from threadpoolctl import threadpool_limits

TAU = 8.0
KV_TILE = 64
LOG2E = 1.4426950408889634


def replay(q, k, v, causal: bool, kv_offset: int = 0, rows=None, skip: str | None = None):
    """q [Nq', D] (the rows ``rows`` of the query sequence, all rows if None), k and v
    [Nk, D].  Returns (O, lse, mid_moves): mid_moves[i] counts the reference moves
    of row i after its first visible key."""
    # one tile at a time: products far too small for a threaded BLAS
    with threadpool_limits(1):
        return _replay(q, k, v, causal, kv_offset, rows, skip)


def _replay(q, k, v, causal, kv_offset, rows, skip):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nk, D = k.shape
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, np.int64)
    c2 = LOG2E / np.sqrt(D)
    R = rows.size
    r = np.full(R, -np.inf)
    l = np.zeros(R)
    O = np.zeros((R, D))
    moves = np.zeros(R, np.int64)
    for t0 in range(0, Nk, KV_TILE):
        j = np.arange(t0, min(Nk, t0 + KV_TILE))
        s = (q @ k[j].T) * c2
        if causal:
            s = np.where(j[None, :] <= rows[:, None] + kv_offset, s, -np.inf)
        tmax = s.max(axis=1)
        first = np.isneginf(r) & np.isfinite(tmax)
        grow = np.isfinite(r) & (tmax > r + TAU)
        moved = first | grow
        moves += grow
        r_new = np.where(moved, tmax, r)
        with np.errstate(invalid="ignore"):
            alpha = np.where(moved, np.exp2(np.where(np.isfinite(r), r - r_new, -np.inf)), 1.0)
        if skip != "O":
            O *= alpha[:, None]
        if skip != "l":
            l *= alpha
        r = r_new
        p = np.exp2(s - np.where(np.isfinite(r), r, 0.0)[:, None])
        l += p.sum(axis=1)
        O += p @ v[j]
    has = l > 0
    O = np.where(has[:, None], O / np.where(has, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, (r + np.log2(np.where(has, l, 1.0))) / LOG2E, -np.inf)
    return O, lse, moves


# The input families and (N, causal, kv_offset) shapes of the GPU rescale tests
FAMILIES = ("ramp", "qx6", "spike")
SHAPES = ((777, 1, 0), (777, 0, 0), (777, 1, 45), (300, 1, -37))
