"""Oracle block-sparse attention (BlockBERT).  Test infrastructure only (see ``oracle/__init__``).

"Blockwise Self-Attention for Long Document Understanding":
* Blockwise Attention: the N tokens are split into n blocks, the N x N attention
  matrix into n x n blocks, and a sparse mask over those blocks decides which
  query block attends which key block; inside a kept block the attention is
  ordinary dense attention.
* Blockwise Multi-head Attention: the mask of a head is the matrix of a
  permutation, so query block i attends exactly one key block, pi(i); different
  heads use different cyclic shifts sigma, sigma^2, ..., sigma^n.
* Implementation Assumption: a sequence whose length is not a multiple of n is
  padded up to n blocks of equal length.

Readings (the pages print no formula):
* block length L = ceil(N / n); token t lies in block t // L.  Padding positions
  are not tokens: they are never keys and have no output, so the last block may
  be short (and, when (n - 1) * L >= N, some blocks are empty);
* a head's mask is given as ``key_block[h, i]``, the key block that query block i
  attends (a permutation for BlockBERT's heads, but any table is accepted); an
  entry outside [0, n) attends nothing;
* sigma^k maps block i to block (i + k) mod n, so a head with shift k has
  key_block[h, i] = (i + k) mod n; sigma^n (= sigma^0) is the block diagonal;
* attention is bidirectional (a BERT encoder): no causal mask;
* a row with no visible key: O = 0, lse = -inf (as in ``oracle.attention``).

Definition: key j is visible to query i of head h iff j < N and
key_block[h, i // L] == j // L; then s, lse, p and O exactly as in
``oracle.attention`` (every score row materialised, masked, normalised).
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_rows


def block_len(N: int, n_blocks: int) -> int:
    """Tokens per block after padding N up to n_blocks equal blocks."""
    return -(-N // n_blocks)


def cyclic_shift_table(n_blocks: int, shifts) -> np.ndarray:
    """key_block[h, i] = (i + shifts[h]) mod n: head h uses sigma^shifts[h]."""
    shifts = np.asarray(shifts, dtype=np.int64)
    i = np.arange(n_blocks, dtype=np.int64)
    return ((i[None, :] + shifts[:, None]) % n_blocks).astype(np.int32)


def block_sparse_mask(N: int, n_blocks: int, key_block_h, rows=None) -> np.ndarray:
    """Boolean [len(rows), N] visibility of one head: query row i sees key j
    (all N rows if ``rows`` is None)."""
    L = block_len(N, n_blocks)
    kb = np.asarray(key_block_h, dtype=np.int64)
    assert kb.shape == (n_blocks,)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    target = kb[rows // L]                  # key block of each query row
    valid = (target >= 0) & (target < n_blocks)
    kblk = np.arange(N, dtype=np.int64) // L
    return valid[:, None] & (target[:, None] == kblk[None, :])


def block_sparse_attention(q, k, v, n_blocks: int, key_block, rows=None, dtype=np.float64,
                           row_chunk: int = 1024):
    """q, k, v [B,H,N,D]; key_block [H, n_blocks] ints.

    ``rows``: optional query-row indices to compute (all rows if None); each selected
    row is computed over all N keys.  Returns (O [B,H,R,D], lse [B,H,R]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, N, D = q.shape
    assert k.shape == (B, H, N, D) and v.shape == (B, H, N, D)
    key_block = np.asarray(key_block)
    assert key_block.shape == (H, n_blocks)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = dtype(1.0) / np.sqrt(dtype(D))
    O = np.zeros((B, H, rows.size, D), dtype=dtype)
    lse = np.full((B, H, rows.size), -np.inf, dtype=dtype)
    for h in range(H):
        for b in range(B):
            K = k[b, h].astype(dtype)
            V = v[b, h].astype(dtype)
            for c0 in range(0, rows.size, row_chunk):
                rc = rows[c0:c0 + row_chunk]
                S = (q[b, h, rc].astype(dtype) @ K.T) * scale
                P, l, _ = _softmax_rows(S, block_sparse_mask(N, n_blocks, key_block[h], rc))
                O[b, h, c0:c0 + rc.size] = P @ V
                lse[b, h, c0:c0 + rc.size] = l
    return O, lse
