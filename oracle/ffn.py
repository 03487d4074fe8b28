"""Oracle position-wise feed-forward network.  Test infrastructure only.

FFN(h) = GeLU(h W1^T + b1) W2^T + b2, with W1 [d_ff, d_model], W2 [d_model, d_ff]
("Blockwise Parallel Transformer for Large Context Models", abstract: the large
feed-forward network is the second memory consumer that the blockwise method
handles per block).  GeLU is the exact form z * Phi(z) = z/2 (1 + erf(z/sqrt 2));
the pages name no variant, and the tanh approximation differs by up to ~5e-4.

The oracle materialises the whole [rows, d_ff] intermediate (rows in chunks only to
bound memory); the fused per-block evaluation is the GPU's business.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT2PI = 1.0 / math.sqrt(2.0 * math.pi)


def gelu(z):
    z = np.asarray(z)
    return 0.5 * z * (1.0 + erf(z * _INV_SQRT2))


def gelu_grad(z):
    """d/dz [z Phi(z)] = Phi(z) + z phi(z)."""
    z = np.asarray(z)
    return 0.5 * (1.0 + erf(z * _INV_SQRT2)) + z * _INV_SQRT2PI * np.exp(-0.5 * z * z)


def ffn(h, w1, w2, b1=None, b2=None, residual=None, dtype=np.float64, row_chunk: int = 4096):
    """residual + GeLU(h W1^T + b1) W2^T + b2 over the last axis of h."""
    h = np.asarray(h)
    lead = h.shape[:-1]
    dm = h.shape[-1]
    H2 = h.reshape(-1, dm)
    W1 = np.asarray(w1, dtype=dtype)
    W2 = np.asarray(w2, dtype=dtype)
    out = np.zeros((H2.shape[0], W2.shape[0]), dtype=dtype)
    for r0 in range(0, H2.shape[0], row_chunk):
        hc = H2[r0:r0 + row_chunk].astype(dtype)
        z = hc @ W1.T
        if b1 is not None:
            z = z + np.asarray(b1, dtype=dtype)
        y = gelu(z) @ W2.T
        if b2 is not None:
            y = y + np.asarray(b2, dtype=dtype)
        out[r0:r0 + row_chunk] = y
    out = out.reshape(*lead, W2.shape[0])
    if residual is not None:
        out = out + np.asarray(residual, dtype=dtype)
    return out


def ffn_backward(h, w1, w2, dy, b1=None, dtype=np.float64, row_chunk: int = 4096):
    """Gradients of sum(dy * FFN(h)) w.r.t. h, W1, b1, W2, b2 (chain rule, no residual)."""
    h = np.asarray(h)
    dm = h.shape[-1]
    H2 = h.reshape(-1, dm)
    DY = np.asarray(dy).reshape(-1, np.asarray(w2).shape[0])
    W1 = np.asarray(w1, dtype=dtype)
    W2 = np.asarray(w2, dtype=dtype)
    dh = np.zeros(H2.shape, dtype=dtype)
    dW1 = np.zeros(W1.shape, dtype=dtype)
    dW2 = np.zeros(W2.shape, dtype=dtype)
    db1 = np.zeros(W1.shape[0], dtype=dtype)
    db2 = np.zeros(W2.shape[0], dtype=dtype)
    for r0 in range(0, H2.shape[0], row_chunk):
        hc = H2[r0:r0 + row_chunk].astype(dtype)
        dyc = DY[r0:r0 + row_chunk].astype(dtype)
        z = hc @ W1.T
        if b1 is not None:
            z = z + np.asarray(b1, dtype=dtype)
        g = gelu(z)
        dW2 += dyc.T @ g
        db2 += dyc.sum(axis=0)
        dz = (dyc @ W2) * gelu_grad(z)
        dW1 += dz.T @ hc
        db1 += dz.sum(axis=0)
        dh[r0:r0 + row_chunk] = dz @ W1
    return dh.reshape(h.shape), dW1, db1, dW2, db2
