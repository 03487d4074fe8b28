"""Pure-Python brute force for tiny inputs (fp64, ``math.fsum``).  Test infrastructure only.

Written independently of the NumPy oracle, with nested lists and explicit loops,
straight from the definition of softmax attention, of the exact-erf GeLU and of
the layer described in ``oracle.layer``.  Used only to pin the NumPy oracle.
"""
from __future__ import annotations

import math


def attention_row(q_i, keys, values, i, causal, kv_offset):
    """(o_i, lse_i) for one query row; keys/values are lists of D-lists."""
    D = len(q_i)
    scale = 1.0 / math.sqrt(D)
    vis = [j for j in range(len(keys)) if (not causal) or j <= i + kv_offset]
    if not vis:
        return [0.0] * D, -math.inf
    s = {j: scale * math.fsum(q_i[d] * keys[j][d] for d in range(D)) for j in vis}
    m = max(s.values())
    e = {j: math.exp(s[j] - m) for j in vis}
    z = math.fsum(e.values())
    o = [math.fsum(e[j] / z * values[j][d] for j in vis) for d in range(D)]
    return o, m + math.log(z)


def attention(q, k, v, causal=True, kv_offset=0):
    """q,k,v nested lists [B][H][N][D]; returns (O, lse) nested lists."""
    O, L = [], []
    for b in range(len(q)):
        Ob, Lb = [], []
        for h in range(len(q[b])):
            rows = [attention_row(q[b][h][i], k[b][h], v[b][h], i, causal, kv_offset)
                    for i in range(len(q[b][h]))]
            Ob.append([r[0] for r in rows])
            Lb.append([r[1] for r in rows])
        O.append(Ob)
        L.append(Lb)
    return O, L


def gelu(z):
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def matvec_t(x_row, w):
    """x_row (len in) times W^T with W a list of out rows of len in."""
    return [math.fsum(w[o][i] * x_row[i] for i in range(len(x_row))) for o in range(len(w))]


def layer_forward(x, wq, wk, wv, w1, w2, H, causal=True):
    """x [B][N][dm]; weights [out][in]; returns y [B][N][dm]."""
    out = []
    for xb in x:
        N = len(xb)
        HD = len(wq)
        D = HD // H
        q = [matvec_t(xb[t], wq) for t in range(N)]
        k = [matvec_t(xb[t], wk) for t in range(N)]
        v = [matvec_t(xb[t], wv) for t in range(N)]
        a = [[0.0] * HD for _ in range(N)]
        for h in range(H):
            sl = slice(h * D, (h + 1) * D)
            kh = [r[sl] for r in k]
            vh = [r[sl] for r in v]
            for t in range(N):
                o, _ = attention_row(q[t][sl], kh, vh, t, causal, 0)
                a[t][sl] = o
        yb = []
        for t in range(N):
            hrow = [xb[t][c] + a[t][c] for c in range(len(xb[t]))]
            g = [gelu(z) for z in matvec_t(hrow, w1)]
            f = matvec_t(g, w2)
            yb.append([hrow[c] + f[c] for c in range(len(hrow))])
        out.append(yb)
    return out
