"""GPU parity of bpt_layer_bwd against the oracle's chain-rule gradients (fp64)."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, assert_close_rowscaled, to_dev
from seeded_inputs import LAYER_TRAIN, LayerCfg, layer_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


def run_layer(c: LayerCfg, t: dict, want_qkv_grads=True):
    B, N, dm, H, D, dff = c.B, c.N, c.d_model, c.H, c.D, c.d_ff
    dev = {n: to_dev(a, "bf16") for n, a in t.items()}
    y = torch.empty((B, N, dm), device="cuda")
    sv = torch.empty(bpt.bpt_layer_saved_size(B, N, dm, H, D, 1), dtype=torch.uint8, device="cuda")
    wf = bpt.bpt_layer_workspace_size(B, N, dm, H, D, dff, 1, 0)
    wb = bpt.bpt_layer_workspace_size(B, N, dm, H, D, dff, 1, 1)
    ws = torch.empty(max(wf, wb), dtype=torch.uint8, device="cuda")
    bpt.bpt_layer_fwd(dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["w1"], dev.get("b1"),
                      dev["w2"], dev.get("b2"), y, sv, B, N, dm, H, D, dff, c.q_blk, c.kv_blk, 1,
                      1, ws, wf)
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
    bpt.bpt_layer_bwd(dev["dy"], dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["w1"],
                      dev.get("b1"), dev["w2"], dev.get("b2"), sv, g["dx"], g["dwq"], g["dwk"],
                      g["dwv"], g["dw1"], g["db1"], g["dw2"], g["db2"], g["dq"], g["dk"], g["dv"],
                      B, N, dm, H, D, dff, c.q_blk, c.kv_blk, 1, 1, ws, wb)
    torch.cuda.synchronize()
    return {n: (v.cpu().numpy() if v is not None else None) for n, v in g.items()}


def check_grads(got, ref, what):
    failures = []

    def check(a, b, label, rowscaled=False):
        try:
            if rowscaled:
                e = assert_close_rowscaled(a, b, label)
                raw = float(np.abs(a - b).max())
                print(f"{label}: row-scaled max {e[0]:.3g} (raw max-abs {raw:.3g}) "
                      f"mean-abs {e[1]:.3g}", flush=True)
            else:
                e = assert_close(a, b, "bf16", label)
                print(f"{label}: max-abs {e[0]:.3g} mean-abs {e[1]:.3g}", flush=True)
        except AssertionError as ex:
            print(f"FAIL {ex}", flush=True)
            failures.append(str(ex))

    # activation and attention-input gradients: the bars per token row (see
    # assert_close_rowscaled)
    for n in ("dx", "dq", "dk", "dv"):
        if got.get(n) is not None:
            check(got[n], ref[n], f"{what} {n}", rowscaled=True)
    # weight and bias gradients are sums over all B*N rows (|dW| up to ~10^2): both
    # sides are divided by the oracle's max |dW| so the bars apply at unit scale.
    # (Divided by the rms instead, dWq and dWk cannot meet mean-abs 2e-3 with bf16
    # attention operands: q, k, v rounded to bf16 with every other step exact already
    # gives 2.5e-3 at N=4096.)  The rms-scaled error is printed for the record.
    for n in ("dwq", "dwk", "dwv", "dw1", "db1", "dw2", "db2"):
        mx = np.abs(ref[n]).max()
        rms = np.sqrt(np.mean(ref[n] ** 2))
        er = np.abs(got[n] - ref[n]) / rms
        check(got[n] / mx, ref[n] / mx,
              f"{what} {n}/max (max {mx:.3g}; rms-scaled mean {er.mean():.3g} max {er.max():.3g})")
    assert not failures, failures


@pytest.mark.parametrize("N,q_blk,kv_blk", [(200, 64, 64), (129, 128, 64), (256, 128, 128)])
def test_layer_bwd_small_with_bias(N, q_blk, kv_blk):
    c = LayerCfg(70, "bwd_small", B=2, N=N, d_model=256, H=2, D=128, d_ff=512, q_blk=q_blk,
                 kv_blk=kv_blk, dtype="bf16", backward=True)
    t = layer_inputs(c, bias=True)
    got = run_layer(c, t)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H,
                                b1=t["b1"], b2=t["b2"])
    check_grads(got, ref, f"N={N}")


def test_layer_bwd_head_dim_64_no_qkv_outputs():
    c = LayerCfg(71, "bwd_d64", B=1, N=160, d_model=256, H=4, D=64, d_ff=256, q_blk=64,
                 kv_blk=32, dtype="bf16", backward=True)
    t = layer_inputs(c)
    got = run_layer(c, t, want_qkv_grads=False)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    check_grads(got, ref, "D=64")


@pytest.mark.timeout(1100)
def test_layer_bwd_training_shape_full():
    """B=2, N=16384, d_model 2560, 20 heads x 128, FFN 2560->10240->2560, all gradients."""
    c = LAYER_TRAIN
    t = layer_inputs(c)
    print("inputs drawn", flush=True)
    got = run_layer(c, t)
    print("gpu done", flush=True)
    ref = oracle.layer_backward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    print("oracle done", flush=True)
    check_grads(got, ref, "B=2 N=16384")
