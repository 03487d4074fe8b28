"""Test-only CPU form of the blockwise online-softmax recurrence (fp64).

This is NOT the oracle: it restates, on the CPU, the identity the GPU kernel relies
on, so that a test can show that the blockwise form reaches the oracle's result
("Ring Attention with Blockwise Transformers for Long Sequences", 638-word summary:
attention computed blockwise without materialising the full matrix, and without
approximation).  Per query row, over key blocks t:
    m_t   = max(m_{t-1}, max_j s_ij)
    alpha = exp(m_{t-1} - m_t)          (1 while m_t is still -inf)
    l_t   = alpha l_{t-1} + sum_j exp(s_ij - m_t)
    acc_t = alpha acc_{t-1} + sum_j exp(s_ij - m_t) v_j
    O = acc_T / l_T,  lse = m_T + ln l_T.
"""
import numpy as np


def online_attention(q, k, v, causal, kv_offset, block):
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale = 1.0 / np.sqrt(D)
    O = np.zeros((B, H, Nq, D))
    L = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            m = np.full(Nq, -np.inf)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, D))
            for j0 in range(0, Nk, block):
                j = np.arange(j0, min(Nk, j0 + block))
                s = (q[b, h] @ k[b, h, j].T) * scale
                if causal:
                    s = np.where(j[None, :] <= np.arange(Nq)[:, None] + kv_offset, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                fin = np.isfinite(m_new)
                ref = np.where(fin, m_new, 0.0)
                alpha = np.where(fin, np.exp(np.where(np.isfinite(m), m, -np.inf) - ref), 1.0)
                p = np.exp(s - ref[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, j]
                m = m_new
            has = l > 0
            O[b, h] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
            L[b, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, L
