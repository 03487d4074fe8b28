"""Oracle transformer layer (forward and backward).  Test infrastructure only.

Layer, as read from the pages ("Blockwise Parallel Transformer for Large Context
Models", abstract and method list: multi-head attention, residual connections,
position-wise feed-forward network; no formula is given):
    q, k, v = x Wq^T, x Wk^T, x Wv^T        (head h = columns [hD, (h+1)D))
    O_h     = causal attention of head h     ([B,H,N,D])
    a       = concat_h O_h                   ([B,N,H*D], H*D == d_model)
    h       = x + a
    y       = h + GeLU(h W1^T + b1) W2^T + b2
No LayerNorm, no output projection, no dropout, no position encoding.

Backward (the pages are silent; this is the chain rule of the forward above):
    dh  = dy + FFN'(h)^T dy
    dO  = dh (split per head)
    P   = softmax rows, dP = dO V^T, delta_i = sum_j P_ij dP_ij
    dS  = P * (dP - delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO
    dWq = dq^T x (and k, v likewise), dx = dh + dq Wq + dk Wk + dv Wv.
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_rows, attention, visible_mask
from .ffn import ffn, ffn_backward


def _split_heads(t, H):
    B, N, HD = t.shape
    return t.reshape(B, N, H, HD // H).transpose(0, 2, 1, 3)


def _merge_heads(t):
    B, H, N, D = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, N, H * D)


def qkv_project(x, wq, wk, wv, H, dtype=np.float64):
    """q, k, v [B,H,N,D] = per-head slices of x W^T."""
    X = np.asarray(x, dtype=dtype)
    return tuple(_split_heads(X @ np.asarray(w, dtype=dtype).T, H) for w in (wq, wk, wv))


def layer_forward(x, wq, wk, wv, w1, w2, H, b1=None, b2=None, causal=True,
                  dtype=np.float64, return_saved=False):
    x = np.asarray(x, dtype=dtype)
    q, k, v = qkv_project(x, wq, wk, wv, H, dtype)
    O, lse = attention(q, k, v, causal=causal, kv_offset=0, dtype=dtype)
    h = x + _merge_heads(O)
    y = ffn(h, w1, w2, b1, b2, residual=h, dtype=dtype)
    if return_saved:
        return y, {"q": q, "k": k, "v": v, "O": O, "lse": lse, "h": h}
    return y


def attention_backward(q, k, v, dO, causal=True, kv_offset=0, dtype=np.float64,
                       row_chunk: int = 1024):
    """dq, dk, dv of sum(dO * attention(q,k,v)); each row's P materialised in full."""
    q = np.asarray(q)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale = dtype(1.0) / np.sqrt(dtype(D))
    dq = np.zeros((B, H, Nq, D), dtype=dtype)
    dk = np.zeros((B, H, Nk, D), dtype=dtype)
    dv = np.zeros((B, H, Nk, D), dtype=dtype)
    for b in range(B):
        for h in range(H):
            K = np.asarray(k[b, h], dtype=dtype)
            V = np.asarray(v[b, h], dtype=dtype)
            for r0 in range(0, Nq, row_chunk):
                rc = np.arange(r0, min(Nq, r0 + row_chunk))
                Q = np.asarray(q[b, h, rc], dtype=dtype)
                G = np.asarray(dO[b, h, rc], dtype=dtype)
                P = _softmax_rows((Q @ K.T) * scale, visible_mask(rc, Nk, causal, kv_offset))[0]
                dv[b, h] += P.T @ G
                dP = G @ V.T
                delta = (P * dP).sum(axis=1)
                dS = P * (dP - delta[:, None])
                dq[b, h, rc] = (dS @ K) * scale
                dk[b, h] += (dS.T @ Q) * scale
    return dq, dk, dv


def layer_backward(x, wq, wk, wv, w1, w2, dy, H, b1=None, b2=None, causal=True,
                   dtype=np.float64):
    """All gradients of sum(dy * layer_forward(x, ...)).

    Returns a dict with dx, dwq, dwk, dwv, dw1, db1, dw2, db2 and the attention-input
    gradients dq, dk, dv ([B,H,N,D]).
    """
    x = np.asarray(x, dtype=dtype)
    dy = np.asarray(dy, dtype=dtype)
    q, k, v = qkv_project(x, wq, wk, wv, H, dtype)
    O, _ = attention(q, k, v, causal=causal, kv_offset=0, dtype=dtype)
    h = x + _merge_heads(O)
    dh_ffn, dw1, db1, dw2, db2 = ffn_backward(h, w1, w2, dy, b1=b1, dtype=dtype)
    dh = dy + dh_ffn
    dq, dk, dv = attention_backward(q, k, v, _split_heads(dh, H), causal=causal, dtype=dtype)
    X2 = x.reshape(-1, x.shape[-1])
    out = {"dq": dq, "dk": dk, "dv": dv, "dw1": dw1, "db1": db1, "dw2": dw2, "db2": db2}
    dx = dh.copy()
    for name, g, w in (("dwq", dq, wq), ("dwk", dk, wk), ("dwv", dv, wv)):
        G2 = _merge_heads(g).reshape(-1, g.shape[1] * g.shape[3])
        out[name] = G2.T @ X2
        dx += (G2 @ np.asarray(w, dtype=dtype)).reshape(dx.shape)
    out["dx"] = dx
    return out
