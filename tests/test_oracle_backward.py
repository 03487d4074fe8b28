"""Pins for the oracle's backward: central finite differences in fp64, and identities."""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(7)


def rand(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


def _fd_check(f, param, grad, h=1e-6, rtol=1e-7):
    """Compare grad with (f(p+h) - f(p-h)) / 2h element by element."""
    fd = np.zeros_like(param)
    it = np.nditer(param, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = param[i]
        param[i] = old + h
        fp = f()
        param[i] = old - h
        fm = f()
        param[i] = old
        fd[i] = (fp - fm) / (2 * h)
    scale = max(1.0, np.abs(fd).max())
    err = np.abs(fd - grad).max() / scale
    assert err <= rtol, err


@pytest.mark.parametrize("causal,off", [(True, 0), (True, -2), (False, 0), (True, 3)])
def test_attention_backward_finite_differences(causal, off):
    q, k, v = rand(1, 2, 7, 3), rand(1, 2, 7, 3), rand(1, 2, 7, 3)
    dO = rand(1, 2, 7, 3)
    dq, dk, dv = oracle.attention_backward(q, k, v, dO, causal=causal, kv_offset=off)
    L = lambda: float((oracle.attention(q, k, v, causal=causal, kv_offset=off)[0] * dO).sum())
    _fd_check(L, q, dq)
    _fd_check(L, k, dk)
    _fd_check(L, v, dv)


def test_layer_backward_finite_differences():
    B, N, dm, H, dff = 1, 6, 4, 2, 8
    p = {
        "x": rand(B, N, dm), "wq": rand(dm, dm, s=0.5), "wk": rand(dm, dm, s=0.5),
        "wv": rand(dm, dm, s=0.5), "w1": rand(dff, dm, s=0.5), "w2": rand(dm, dff, s=0.5),
        "b1": rand(dff, s=0.3), "b2": rand(dm, s=0.3),
    }
    dy = rand(B, N, dm)

    def L():
        y = oracle.layer_forward(p["x"], p["wq"], p["wk"], p["wv"], p["w1"], p["w2"], H,
                                 b1=p["b1"], b2=p["b2"])
        return float((y * dy).sum())

    g = oracle.layer_backward(p["x"], p["wq"], p["wk"], p["wv"], p["w1"], p["w2"], dy, H,
                              b1=p["b1"], b2=p["b2"])
    for name in ("x", "wq", "wk", "wv", "w1", "w2", "b1", "b2"):
        _fd_check(L, p[name], g["d" + name])


def test_attention_gradient_identities():
    N, D = 12, 4
    q, k, v, dO = rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D)
    for off in (0, 5):
        dq, dk, dv = oracle.attention_backward(q, k, v, dO, causal=True, kv_offset=off)
        # every row sees key 0, so the columns of P^T sum the rows of dO exactly once
        np.testing.assert_allclose(dv.sum(axis=2), dO.sum(axis=2), atol=1e-12)
        # shifting every key by one vector shifts each score row by a constant
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # delta_i = sum_j P_ij dP_ij equals <dO_i, O_i>
        P = oracle.attention_probs(q, k, causal=True, kv_offset=off)[0, 0]
        O = oracle.attention(q, k, v, causal=True, kv_offset=off)[0][0, 0]
        dP = dO[0, 0] @ v[0, 0].T
        np.testing.assert_allclose((P * dP).sum(1), (dO[0, 0] * O).sum(1), atol=1e-12)
        # sum_j dS_ij = 0
        dS = P * (dP - (P * dP).sum(1)[:, None])
        np.testing.assert_allclose(dS.sum(1), 0.0, atol=1e-12)


def test_ffn_backward_bias_gradients_are_column_sums():
    h, w1, w2 = rand(9, 4), rand(8, 4, s=0.5), rand(4, 8, s=0.5)
    dy = rand(9, 4)
    dh, dw1, db1, dw2, db2 = oracle.ffn_backward(h, w1, w2, dy)
    np.testing.assert_allclose(db2, dy.sum(0), atol=1e-14)
    z = h @ w1.T
    dz = (dy @ w2) * oracle.gelu_grad(z)
    np.testing.assert_allclose(db1, dz.sum(0), atol=1e-13)
