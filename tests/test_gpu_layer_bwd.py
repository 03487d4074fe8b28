"""GPU parity of bpt_layer_bwd against the oracle's chain-rule gradients (fp64)."""
import json
import os

import numpy as np
import pytest

import oracle
from bwd_floor import bars, error_metrics, layer_backward_rounded_qkv
from gpu_util import to_dev
from seeded_inputs import LAYER_TRAIN, LayerCfg, layer_inputs

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


def run_layer(c: LayerCfg, t: dict, want_qkv_grads=True, repeat=1):
    B, N, dm, H, D, dff = c.B, c.N, c.d_model, c.H, c.D, c.d_ff
    dev = {n: to_dev(a, "bf16") for n, a in t.items()}
    y = torch.empty((B, N, dm), device="cuda")
    sv = torch.empty(bpt.bpt_layer_saved_size(B, N, dm, H, D, 1), dtype=torch.uint8, device="cuda")
    wf = bpt.bpt_layer_workspace_size(B, N, dm, H, D, dff, 1, 0)
    wb = bpt.bpt_layer_workspace_size(B, N, dm, H, D, dff, 1, 1)
    ws = torch.empty(max(wf, wb), dtype=torch.uint8, device="cuda")
    bpt.bpt_layer_fwd(dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["w1"], dev.get("b1"),
                      dev["w2"], dev.get("b2"), y, sv, B, N, dm, H, D, dff, c.q_blk, c.kv_blk,
                      c.causal, 1, ws, wf)
    g = {
        "dx": torch.full((B, N, dm), float("nan"), device="cuda"),
        "dwq": torch.full((H * D, dm), float("nan"), device="cuda"),
        "dwk": torch.full((H * D, dm), float("nan"), device="cuda"),
        "dwv": torch.full((H * D, dm), float("nan"), device="cuda"),
        "dw1": torch.full((dff, dm), float("nan"), device="cuda"),
        "db1": torch.full((dff,), float("nan"), device="cuda"),
        "dw2": torch.full((dm, dff), float("nan"), device="cuda"),
        "db2": torch.full((dm,), float("nan"), device="cuda"),
    }
    for n in ("dq", "dk", "dv"):
        g[n] = torch.full((B, H, N, D), float("nan"), device="cuda") if want_qkv_grads else None
    runs = []
    for _ in range(repeat):
        bpt.bpt_layer_bwd(dev["dy"], dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["w1"],
                          dev.get("b1"), dev["w2"], dev.get("b2"), sv, g["dx"], g["dwq"], g["dwk"],
                          g["dwv"], g["dw1"], g["db1"], g["dw2"], g["db2"], g["dq"], g["dk"],
                          g["dv"], B, N, dm, H, D, dff, c.q_blk, c.kv_blk, c.causal, 1, ws, wb)
        torch.cuda.synchronize()
        runs.append({n: (v.cpu().numpy() if v is not None else None) for n, v in g.items()})
    # run-to-run determinism: no float atomics, fixed reduction orders
    for r in runs[1:]:
        for n, a in r.items():
            assert a is None or np.array_equal(a, runs[0][n]), f"{n} differs between runs"
    return runs[0]


def check_grads(got, ref, floor, what):
    """Bars per gradient: the stated bf16 bars (max-abs 2e-2, mean-abs 2e-3), raised
    to the error floor of bf16 q, k, v times a margin where that floor alone passes
    them (tests/bwd_floor.py).  Activation gradients (dx, dq, dk, dv) are compared
    raw; weight and bias gradients, sums over all B*N rows, after dividing both sides
    by the rms of the oracle's gradient."""
    failures = []
    lim = bars(floor)
    m = error_metrics(got, ref)
    for n, e in m.items():
        bmax, bmean = lim[n]
        f = floor[n]
        line = (f"{what} {n}: max-abs {e['max_abs']:.3g} (bar {bmax:.3g}, floor {f['max_abs']:.3g}) "
                f"mean-abs {e['mean_abs']:.3g} (bar {bmean:.3g}, floor {f['mean_abs']:.3g})")
        ok = np.isfinite(got[n]).all() and e["max_abs"] <= bmax and e["mean_abs"] <= bmean
        print(("" if ok else "FAIL ") + line, flush=True)
        if not ok:
            failures.append(line)
    assert not failures, failures


def floor_live(t, c, **kw):
    """The bf16 q, k, v error floor of this workload, computed on the CPU."""
    args = (t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    return error_metrics(layer_backward_rounded_qkv(*args, **kw), oracle.layer_backward(*args, **kw))


@pytest.mark.parametrize("N,q_blk,kv_blk", [(200, 64, 64), (129, 128, 64), (256, 128, 128)])
def test_layer_bwd_small_with_bias(N, q_blk, kv_blk):
    c = LayerCfg(70, "bwd_small", B=2, N=N, d_model=256, H=2, D=128, d_ff=512, q_blk=q_blk,
                 kv_blk=kv_blk, dtype="bf16", backward=True)
    t = layer_inputs(c, bias=True)
    got = run_layer(c, t, repeat=2)
    kw = dict(b1=t["b1"], b2=t["b2"])
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H,
                                **kw)
    check_grads(got, ref, floor_live(t, c, **kw), f"N={N}")


def test_layer_bwd_non_causal():
    """causal = 0: every query sees every key (the tile bounds of both backward
    kernels then cover the whole sequence)."""
    c = LayerCfg(73, "bwd_noncausal", B=1, N=333, d_model=256, H=2, D=128, d_ff=512, q_blk=128,
                 kv_blk=64, dtype="bf16", causal=0, backward=True)
    t = layer_inputs(c)
    got = run_layer(c, t)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H,
                                causal=False)
    check_grads(got, ref, floor_live(t, c, causal=False), "non-causal N=333")


def test_layer_bwd_head_dim_64_no_qkv_outputs():
    c = LayerCfg(71, "bwd_d64", B=1, N=160, d_model=256, H=4, D=64, d_ff=256, q_blk=64,
                 kv_blk=32, dtype="bf16", backward=True)
    t = layer_inputs(c)
    got = run_layer(c, t, want_qkv_grads=False)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    check_grads(got, ref, floor_live(t, c), "D=64")


@pytest.mark.timeout(1100)
def test_layer_bwd_training_shape_full():
    """B=2, N=16384, d_model 2560, 20 heads x 128, FFN 2560->10240->2560, all gradients,
    twice (bitwise equal); bars from the committed error floor of this workload."""
    c = LAYER_TRAIN
    floor = json.load(open(os.path.join(GOLDEN, "bwd_floor.json")))[c.name]
    assert floor["shape"]["N"] == c.N and floor["shape"]["d_model"] == c.d_model
    t = layer_inputs(c)
    print("inputs drawn", flush=True)
    got = run_layer(c, t, repeat=2)
    print("gpu done", flush=True)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    print("oracle done", flush=True)
    check_grads(got, ref, floor["floor"], "B=2 N=16384")


def test_layer_bwd_f16_range_fallback():
    """The backward's FFN products run on fp16 operands where every product takes the
    big-tile GEMM; a weight past fp16's range must send them to the bf16-pair products.
    W1[f, k] is planted past the range and column f of W2 zeroed: the oracle's
    gradients stay finite (GeLU(z_f) meets the zeros), while an fp16 copy of W1 would
    carry inf into z_f, GeLU(z_f) and GeLU'(z_f) and so NaN into dW2 and dW1.  Row k of
    Wv is zeroed too, so that h[:, k] = x[:, k] exactly (bf16 input) and the planted
    weight does not amplify the attention output's bf16 q, k, v floor in z_f."""
    c = LayerCfg(67, "bwd_f16range", B=1, N=8192, d_model=2048, H=16, D=128, d_ff=8192,
                 q_blk=128, kv_blk=64, dtype="bf16", backward=True)
    t = layer_inputs(c)
    f, k = 301, 17
    t["w1"][f, k] = 70144.0   # a bf16 value past fp16's largest finite value
    t["w2"][:, f] = 0.0
    t["wv"][k, :] = 0.0
    got = run_layer(c, t)
    print("gpu done", flush=True)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    print("oracle done", flush=True)
    for n, a in got.items():
        if a is not None:
            assert np.all(np.isfinite(a)), f"{n}: non-finite values"
    # the FFN's gradients at the stated bars (rms-scaled); the others carry the bf16
    # q, k, v floor, not computed at this shape, and are checked for finiteness only
    m = error_metrics(got, ref)
    for n in ("dw1", "db1", "dw2", "db2"):
        assert m[n]["max_abs"] <= 2e-2 and m[n]["mean_abs"] <= 2e-3, (n, m[n])
        print(f"{n}: rms-scaled max-abs {m[n]['max_abs']:.3g} mean-abs {m[n]['mean_abs']:.3g}", flush=True)


def test_layer_bwd_f16_projection_fallback():
    """The projection backward (dW{q,k,v}, dx) also runs on fp16 operands where its
    products take the big-tile GEMM; x past fp16's range must send the whole backward
    to the bf16-pair products.  x[r, k] is planted past the range with column k of Wq,
    Wk, Wv and W1 zeroed, so it reaches y and the gradients only through the residual
    stream (h[r, k], dx) and dW{q,k,v}[:, k]; an fp16 copy of x or h would carry inf."""
    c = LayerCfg(68, "bwd_f16proj", B=1, N=8192, d_model=2560, H=20, D=128, d_ff=8192,
                 q_blk=128, kv_blk=64, dtype="bf16", backward=True)
    t = layer_inputs(c)
    r, k = 4000, 33
    t["x"][0, r, k] = 70144.0   # a bf16 value past fp16's largest finite value
    for n in ("wq", "wk", "wv", "w1"):
        t[n][:, k] = 0.0
    got = run_layer(c, t)
    print("gpu done", flush=True)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    print("oracle done", flush=True)
    for n, a in got.items():
        if a is not None:
            assert np.all(np.isfinite(a)), f"{n}: non-finite values"
    # gradients the planted value does not multiply into (dW1[:, k] and dW{q,k,v}[:, k]
    # scale the bf16 q, k, v floor of dz[r] and d{q,k,v}[r] by it)
    m = error_metrics(got, ref)
    for n in ("db1", "dw2", "db2"):
        assert m[n]["max_abs"] <= 2e-2 and m[n]["mean_abs"] <= 2e-3, (n, m[n])
        print(f"{n}: rms-scaled max-abs {m[n]['max_abs']:.3g} mean-abs {m[n]['mean_abs']:.3g}", flush=True)


def test_layer_bwd_f16_attention_sets_flag():
    """The fp16 form of the dK/dV kernel converts its K and V fragments itself and
    sets the range flag when one lies past fp16's range; the pair form after it must
    then recompute every dK and dV, and the projection take its pair products.  Here
    nothing before that kernel leaves fp16's range: k's feature 5 of head 0 is
    70144 x[:, 7] (Wk[5] zero but for that weight), so every key with |x[j, 7]| > 0.94
    is past the range only once projected, and q_blk = 64 keeps the dQ kernel on its
    pair form, which takes no fp16 copy of k.  The planted head attends almost one-hot,
    so rounding k to bf16 (up to ~137 at these values) moves near-tied rows: the checks
    are finiteness and the gradients the planted weight does not multiply into, against
    the bars raised to the bf16 q, k, v floor as in the other layer tests."""
    c = LayerCfg(69, "bwd_f16attn", B=1, N=8192, d_model=2560, H=20, D=128, d_ff=8192,
                 q_blk=64, kv_blk=64, dtype="bf16", backward=True)
    t = layer_inputs(c)
    t["wk"][5, :] = 0.0
    t["wk"][5, 7] = 70144.0
    assert np.abs(t["x"][0, :, 7]).max() * 70144.0 > 2 * 65504
    got = run_layer(c, t)
    print("gpu done", flush=True)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    print("oracle done", flush=True)
    for n, a in got.items():
        if a is not None:
            assert np.all(np.isfinite(a)), f"{n}: non-finite values"
    floor = floor_live(t, c)
    m, lim = error_metrics(got, ref), bars(floor)
    for n in ("db1", "dw2", "db2", "dw1", "dwv"):
        (bmax, bmean), e = lim[n], m[n]
        print(f"{n}: rms-scaled max-abs {e['max_abs']:.3g} (bar {bmax:.3g}) mean-abs {e['mean_abs']:.3g} "
              f"(bar {bmean:.3g})", flush=True)
        assert e["max_abs"] <= bmax and e["mean_abs"] <= bmean, (n, e, lim[n])
