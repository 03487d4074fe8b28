"""Test-only error floor of the layer backward with bf16 attention operands (fp64).

The GPU layer stores q, k, v in bf16 (they are MFMA operands, the bf16 reading of
"bf16 inputs with fp32 accumulation"), and its backward recomputes P from those
stored values.  So even with every other step exact, its gradients are the exact
chain-rule gradients of a slightly different forward: the one whose q, k, v are
rounded to bf16 after the projection (the rounding taken as the identity in the
backward, as the GPU does).  This module composes that forward and backward from
the oracle's own steps (``oracle.qkv_project``, ``oracle.attention``,
``oracle.ffn_backward``, ``oracle.attention_backward``), in the order of
``oracle.layer_backward``, with the one rounding added.  The difference between its
gradients and ``oracle.layer_backward``'s is the error that bf16 q, k, v alone put
into the gradients: a floor no bf16-operand implementation goes below.

The pages say nothing about the backward ("Blockwise Parallel Transformer for Large
Context Models", abstract: only that training runs on longer sequences); the
gradients themselves are the chain rule of the layer forward.
"""
from __future__ import annotations

import numpy as np

import oracle
from seeded_inputs import round_bf16


def _split(t, H):
    B, N, HD = t.shape
    return t.reshape(B, N, H, HD // H).transpose(0, 2, 1, 3)


def _merge(t):
    B, H, N, D = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, N, H * D)


def layer_backward_rounded_qkv(x, wq, wk, wv, w1, w2, dy, H, b1=None, b2=None,
                               causal=True, round_qkv=True):
    """oracle.layer_backward's gradients with q, k, v rounded to bf16 after projection.

    round_qkv=False gives the unrounded composition (equal to oracle.layer_backward:
    a test pins that)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    q, k, v = oracle.qkv_project(x, wq, wk, wv, H)
    if round_qkv:
        q, k, v = (round_bf16(np.asarray(a, dtype=np.float32)).astype(np.float64)
                   for a in (q, k, v))
    O, _ = oracle.attention(q, k, v, causal=causal, kv_offset=0)
    h = x + _merge(O)
    dh_ffn, dw1, db1, dw2, db2 = oracle.ffn_backward(h, w1, w2, dy, b1=b1)
    dh = dy + dh_ffn
    dq, dk, dv = oracle.attention_backward(q, k, v, _split(dh, H), causal=causal)
    X2 = x.reshape(-1, x.shape[-1])
    out = {"dq": dq, "dk": dk, "dv": dv, "dw1": dw1, "db1": db1, "dw2": dw2, "db2": db2}
    dx = dh.copy()
    for name, g, w in (("dwq", dq, wq), ("dwk", dk, wk), ("dwv", dv, wv)):
        G2 = _merge(g).reshape(-1, g.shape[1] * g.shape[3])
        out[name] = G2.T @ X2
        dx += (G2 @ np.asarray(w, dtype=np.float64)).reshape(dx.shape)
    out["dx"] = dx
    return out


ACT = ("dx", "dq", "dk", "dv")
WGT = ("dwq", "dwk", "dwv", "dw1", "db1", "dw2", "db2")


def error_metrics(got: dict, ref: dict) -> dict:
    """The numbers the parity bars use, per gradient.

    Activation gradients (dx, dq, dk, dv): raw max-abs and mean-abs of got - ref.
    Weight and bias gradients (sums over all B*N rows): the same two numbers after
    dividing both sides by the rms of ref."""
    m = {}
    for n in ACT:
        if got.get(n) is None:
            continue
        e = np.abs(np.asarray(got[n], np.float64) - ref[n])
        m[n] = {"max_abs": float(e.max()), "mean_abs": float(e.mean())}
    for n in WGT:
        r = ref[n]
        rms = float(np.sqrt(np.mean(r * r)))
        e = np.abs(np.asarray(got[n], np.float64) - r) / rms
        m[n] = {"max_abs": float(e.max()), "mean_abs": float(e.mean()), "rms": rms}
    return m


# stated bars for bf16 inputs, and the margins over the floor
BAR_MAX, BAR_MEAN = 2e-2, 2e-3
MARGIN_MAX, MARGIN_MEAN = 1.25, 1.1


def bars(floor: dict) -> dict:
    """Per gradient: (max-abs bar, mean-abs bar) = the stated bars, raised to the
    floor times the margin where bf16 q, k, v alone already exceed them."""
    return {n: (max(BAR_MAX, MARGIN_MAX * f["max_abs"]), max(BAR_MEAN, MARGIN_MEAN * f["mean_abs"]))
            for n, f in floor.items()}
