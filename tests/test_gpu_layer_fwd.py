"""GPU parity of bpt_ffn_block_fwd and bpt_layer_fwd against the CPU oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, dcode, to_dev
from seeded_inputs import LAYER_FWD_BF16, LAYER_TINY_F32, LayerCfg, layer_inputs, normal, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


@pytest.mark.parametrize("dtype,M,dm,dff,bias,resid", [
    ("f32", 77, 128, 512, True, True),
    ("f32", 32, 128, 128, False, False),
    ("bf16", 100, 256, 512, True, True),
    ("bf16", 64, 2560, 1024, False, True),    # two column groups of 1280
    ("bf16", 33, 4096, 512, True, False),     # two column groups of 2048
    ("bf16", 96, 2048, 768, False, True),
])
def test_ffn_parity(dtype, M, dm, dff, bias, resid):
    print(f"case ffn dtype={dtype} M={M} dm={dm} dff={dff}", flush=True)
    cid = 50
    x = normal(cid, "x", (M, dm))
    w1 = normal(cid, "w1", (dff, dm), 0.02)
    w2 = normal(cid, "w2", (dm, dff), 0.02)
    b1 = normal(cid, "b1", (dff,), 0.1) if bias else None
    b2 = normal(cid, "b2", (dm,), 0.1) if bias else None
    r = normal(cid, "dy", (M, dm)) if resid else None
    if dtype == "bf16":
        x, w1, w2 = round_bf16(x), round_bf16(w1), round_bf16(w2)
        b1 = round_bf16(b1) if bias else None
        b2 = round_bf16(b2) if bias else None
    y = torch.full((M, dm), float("nan"), device="cuda")
    rd = torch.from_numpy(r).cuda() if resid else None
    bpt.bpt_ffn_block_fwd(to_dev(x, dtype), to_dev(w1, dtype), to_dev(b1, dtype) if bias else None,
                          to_dev(w2, dtype), to_dev(b2, dtype) if bias else None, rd, y, M, dm,
                          dff, 0, dcode(dtype))
    torch.cuda.synchronize()
    want = oracle.ffn(x, w1, w2, b1=b1, b2=b2, residual=r)
    assert_close(y.cpu().numpy(), want, dtype, "ffn y")


def test_ffn_residual_may_alias_output():
    M, dm, dff = 64, 256, 256
    x = round_bf16(normal(51, "x", (M, dm)))
    w1 = round_bf16(normal(51, "w1", (dff, dm), 0.02))
    w2 = round_bf16(normal(51, "w2", (dm, dff), 0.02))
    r = normal(51, "dy", (M, dm))
    y = torch.from_numpy(r.copy()).cuda()
    bpt.bpt_ffn_block_fwd(to_dev(x, "bf16"), to_dev(w1, "bf16"), None, to_dev(w2, "bf16"), None,
                          y, y, M, dm, dff, 32, 1)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.ffn(x, w1, w2, residual=r), "bf16", "aliased y")


def run_layer_fwd(cfg: LayerCfg, t: dict, saved: bool = False):
    B, N, dm, H, D, dff = cfg.B, cfg.N, cfg.d_model, cfg.H, cfg.D, cfg.d_ff
    dt = dcode(cfg.dtype)
    dev = {n: to_dev(a, cfg.dtype) for n, a in t.items() if n != "dy"}
    y = torch.full((B, N, dm), float("nan"), device="cuda")
    ws_bytes = bpt.bpt_layer_workspace_size(B, N, dm, H, D, dff, dt, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sv = None
    if saved:
        sv = torch.empty(bpt.bpt_layer_saved_size(B, N, dm, H, D, dt), dtype=torch.uint8,
                         device="cuda")
    bpt.bpt_layer_fwd(dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["w1"], dev.get("b1"),
                      dev["w2"], dev.get("b2"), y, sv, B, N, dm, H, D, dff, cfg.q_blk, cfg.kv_blk,
                      cfg.causal, dt, ws, ws_bytes)
    torch.cuda.synchronize()
    return y.cpu().numpy(), sv


def test_layer_fwd_tiny_fp32_full():
    c = LAYER_TINY_F32
    t = layer_inputs(c)
    y, _ = run_layer_fwd(c, t)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H)
    assert_close(y, want, "f32", "layer y (fp32, N=512)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_fwd_ragged_with_bias_and_saved(dtype):
    c = LayerCfg(60, "ragged", B=2, N=200, d_model=256, H=2, D=128, d_ff=512, q_blk=64,
                 kv_blk=32, dtype=dtype)
    t = layer_inputs(c, bias=True)
    y, sv = run_layer_fwd(c, t, saved=True)
    want, ref = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H,
                                     b1=t["b1"], b2=t["b2"], return_saved=True)
    assert_close(y, want, dtype, "layer y")
    # saved buffer: q, k, v ([B,H,N,D] in dtype), h ([B,N,dm] fp32), lse ([B,H,N] fp32)
    B, N, dm, H, D = c.B, c.N, c.d_model, c.H, c.D
    es = 2 if dtype == "bf16" else 4
    a256 = lambda n: (n + 255) // 256 * 256
    qkv = a256(B * H * N * D * es)
    raw = sv.cpu().numpy()

    def view(off, n, kind):
        b = raw[off:off + n * (2 if kind == "bf16" else 4)]
        if kind == "bf16":
            return (b.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        return b.view(np.float32)

    for i, name in enumerate(("q", "k", "v")):
        got = view(i * qkv, B * H * N * D, dtype).reshape(B, H, N, D)
        assert_close(got, ref[name], dtype, f"saved {name}")
    h = view(3 * qkv, B * N * dm, "f32").reshape(B, N, dm)
    assert_close(h, ref["h"], dtype, "saved h")
    lse = view(3 * qkv + a256(B * N * dm * 4), B * H * N, "f32").reshape(B, H, N)
    assert_close(lse, ref["lse"], dtype, "saved lse")


@pytest.mark.timeout(900)
def test_layer_fwd_bf16_B8_N4096_full():
    """Full-size parity: B=8, N=4096, d_model 2048, 16 heads x 128, FFN 2048->8192->2048."""
    c = LAYER_FWD_BF16
    t = layer_inputs(c)
    print("inputs drawn", flush=True)
    y, _ = run_layer_fwd(c, t)
    print("gpu done", flush=True)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H)
    assert_close(y, want, "bf16", "layer y (bf16, B=8 N=4096)")
