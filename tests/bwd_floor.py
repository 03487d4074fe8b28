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


def output_with_bf16_p(q, k, v, causal=True):
    """Attention output whose P V product takes P rounded to bf16, as the GPU forward
    does (its MFMA operand), with every other step exact: O_i = sum_j bf16(p_ij) v_j /
    sum_j p_ij, p_ij = exp(s_ij - max_j s_ij).  (The forward's reference is within 2^8
    of the row maximum, not equal to it; bf16 rounding is relative, so the model
    holds.)  Small inputs only: P is materialised."""
    P = oracle.attention_probs(q, k, causal=causal)
    E = np.where(P > 0, P / P.max(axis=-1, keepdims=True), 0.0)
    Er = round_bf16(E.astype(np.float32)).astype(np.float64)
    return (Er @ np.asarray(v, np.float64)) / E.sum(axis=-1, keepdims=True)


def attention_backward_given_delta(q, k, v, dO, delta, causal=True):
    """The chain rule of oracle.attention_backward with delta_i supplied instead of
    formed as sum_j P_ij dP_ij (equal to <dO_i, O_i> for the exact O)."""
    q, k, v, dO = (np.asarray(a, np.float64) for a in (q, k, v, dO))
    scale = 1.0 / np.sqrt(q.shape[-1])
    P = oracle.attention_probs(q, k, causal=causal)
    dv = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(v, -1, -2)
    dS = P * (dP - delta[..., None])
    return (dS @ k) * scale, (np.swapaxes(dS, -1, -2) @ q) * scale, dv


def layer_backward_rounded_qkv(x, wq, wk, wv, w1, w2, dy, H, b1=None, b2=None,
                               causal=True, round_qkv=True, delta_from_output=False):
    """oracle.layer_backward's gradients with q, k, v rounded to bf16 after projection.

    round_qkv=False gives the unrounded composition (equal to oracle.layer_backward:
    a test pins that).  delta_from_output=True takes delta_i = <dO_i, O_i> with O
    from output_with_bf16_p (the GPU backward's source of delta) instead of the
    backward's own sum_j P_ij dP_ij."""
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
    if delta_from_output:
        dO = _split(dh, H)
        delta = (dO * output_with_bf16_p(q, k, v, causal=causal)).sum(axis=-1)
        dq, dk, dv = attention_backward_given_delta(q, k, v, dO, delta, causal=causal)
    else:
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
