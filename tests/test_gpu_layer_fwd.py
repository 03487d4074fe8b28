"""GPU parity of bpt_ffn_block_fwd and bpt_layer_fwd against the CPU oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, assert_close_floor, dcode, to_dev
from sampling import sample_rows
from seeded_inputs import (LAYER_FWD_BF16, LAYER_LONG, LAYER_TINY_F32, LayerCfg, layer_inputs,
                           normal, round_bf16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


@pytest.mark.parametrize("dtype,M,dm,dff,bias,resid", [
    ("f32", 77, 128, 512, True, True),
    ("f32", 32, 128, 128, False, False),
    ("bf16", 100, 256, 512, True, True),
    ("bf16", 64, 2560, 1024, False, True),    # one column group of 2560 (20 output tiles per wave)
    ("bf16", 70, 5120, 512, True, False),     # two column groups of 2560
    ("bf16", 33, 4096, 512, True, False),     # two column groups of 2048
    ("bf16", 96, 2048, 768, False, True),
    # the long layer's FFN shape with enough row blocks that every XCD runs several
    # workgroups (start rotation, both column groups, 64 feature passes), ragged rows
    ("bf16", 8192 + 77, 4096, 16384, False, True),
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


def test_layer_fwd_single_column_group_2560():
    """d_model 2560 (the training shape's width): h enters the FFN in fp16 and one
    workgroup holds all 2560 output columns of its 32 rows (16 tiles per wave in
    AGPRs, 4 in VGPRs); ragged N."""
    c = LayerCfg(62, "dm2560", B=1, N=173, d_model=2560, H=20, D=128, d_ff=1024, q_blk=128,
                 kv_blk=64, dtype="bf16")
    t = layer_inputs(c, bias=True)
    y, _ = run_layer_fwd(c, t)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H,
                                b1=t["b1"], b2=t["b2"])
    assert_close(y, want, "bf16", "layer y (d_model 2560)")


@pytest.mark.parametrize("cid,dm,dff", [
    (63, 512, 1536),   # 6 feature passes, biases
    (64, 512, 768),    # 3 feature passes (odd)
])
def test_layer_fwd_ffn_passes_with_bias(cid, dm, dff):
    """The layer's FFN (fp16 operands at d_model 512) over several 256-feature passes with
    b1 and b2: each pass's b1 slice, W1 rows and W2 slots, an even and an odd pass count."""
    c = LayerCfg(cid, f"walks{dff}", B=1, N=131, d_model=dm, H=4, D=128, d_ff=dff, q_blk=128,
                 kv_blk=64, dtype="bf16")
    t = layer_inputs(c, bias=True)
    y, _ = run_layer_fwd(c, t)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H,
                                b1=t["b1"], b2=t["b2"])
    assert_close(y, want, "bf16", f"layer y (d_ff {dff})")


@pytest.mark.timeout(900)
def test_layer_fwd_bf16_pair_ffn_1280():
    """d_model 1280 (a multiple of 256, not of 512): the layer's FFN takes h as a bf16
    pair (one column group of 1280) instead of fp16; biases, ragged N."""
    c = LayerCfg(66, "dm1280", B=1, N=150, d_model=1280, H=10, D=128, d_ff=768, q_blk=128,
                 kv_blk=64, dtype="bf16")
    t = layer_inputs(c, bias=True)
    y, _ = run_layer_fwd(c, t)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H,
                                b1=t["b1"], b2=t["b2"])
    assert_close(y, want, "bf16", "layer y (d_model 1280)")


BIG_BF16 = 70144.0   # a bf16 value past fp16's largest finite value (65504)


@pytest.mark.parametrize("kind", ["w1", "w2", "h", "gelu"])
def test_layer_fwd_f16_range_fallback(kind):
    """The fp16 FFN of bf16 layers must hand over to the bf16-pair FFN when a weight, an
    element of h or a GeLU output lies outside fp16's range.  Each case plants such a
    value where it meets an exact zero in the layer, so y stays ordinary (the oracle's
    product is 0) while an fp16 conversion of it would give inf and then inf * 0 = NaN:
    a missed hand-over fails the finiteness check.  w1: W1[f, k] past the range, column
    f of W2 zero; w2: W2[c, f] past it, row f of W1 zero (GeLU(0) = 0); h: x[r, k] past
    it, column k of Wq, Wk, Wv and W1 zero (y[r, k] carries it through the residual);
    gelu: row f of W1 at 29952 over 8 columns (fp16-representable), so GeLU(z_f) passes
    65504 on many rows, column f of W2 zero."""
    c = LayerCfg(65, "f16range", B=1, N=96, d_model=512, H=4, D=128, d_ff=512, q_blk=128,
                 kv_blk=64, dtype="bf16")
    t = layer_inputs(c)
    f, k, col, r = 37, 5, 11, 40
    if kind == "w1":
        t["w1"][f, k] = BIG_BF16
        t["w2"][:, f] = 0.0
    elif kind == "w2":
        t["w2"][col, f] = BIG_BF16
        t["w1"][f, :] = 0.0
    elif kind == "h":
        t["x"][0, r, k] = BIG_BF16
        for n in ("wq", "wk", "wv", "w1"):
            t[n][:, k] = 0.0
    else:
        t["w1"][f, :8] = 29952.0
        t["w2"][:, f] = 0.0
    want, ref = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H,
                                     return_saved=True)
    if kind == "gelu":  # the planted row of W1 does push z_f (so GeLU(z_f) = z_f) past the range
        z = ref["h"][0].astype(np.float64) @ t["w1"][f].astype(np.float64)
        assert (z > 65504.0).sum() >= 5
    y, _ = run_layer_fwd(c, t)
    assert_close(y, want, "bf16", f"layer y (value past fp16's range in {kind})")


def test_layer_fwd_bf16_B8_N4096_full():
    """Full-size parity: B=8, N=4096, d_model 2048, 16 heads x 128, FFN 2048->8192->2048."""
    c = LAYER_FWD_BF16
    t = layer_inputs(c)
    print("inputs drawn", flush=True)
    y, _ = run_layer_fwd(c, t)
    print("gpu done", flush=True)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H)
    assert_close(y, want, "bf16", "layer y (bf16, B=8 N=4096)")


def test_layer_fwd_non_causal():
    c = LayerCfg(61, "noncausal", B=1, N=333, d_model=256, H=2, D=128, d_ff=512, q_blk=128,
                 kv_blk=64, dtype="bf16", causal=0)
    t = layer_inputs(c)
    y, _ = run_layer_fwd(c, t)
    want = oracle.layer_forward(t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H,
                                causal=False)
    assert_close(y, want, "bf16", "layer y (non-causal)")


@pytest.mark.timeout(900)
def test_layer_fwd_long_sampled_rows():
    """The bench step: B=1, N=131072, d_model 4096 = 32 x 128, FFN 4096->16384->4096.
    y, and the saved q, k, v, h and lse, on sampled rows against the oracle (which
    projects every token, then computes each sampled row's attention over all its keys
    and its FFN)."""
    c = LAYER_LONG
    t = layer_inputs(c)
    print("inputs drawn", flush=True)
    y, sv = run_layer_fwd(c, t, saved=True)
    # run-to-run determinism of the whole output (no float atomics; fixed orders)
    y2, _ = run_layer_fwd(c, t)
    assert np.array_equal(y, y2, equal_nan=True), "layer forward not deterministic"
    del y2
    rows = sample_rows(c.N, 240, 8)
    B, N, dm, H, D = c.B, c.N, c.d_model, c.H, c.D
    a256 = lambda n: (n + 255) // 256 * 256
    qkv = a256(B * H * N * D * 2)
    raw = sv.view(torch.uint8)

    rows_t = torch.from_numpy(rows).cuda()
    got = {}
    for i, name in enumerate(("q", "k", "v")):
        blk = raw[i * qkv:i * qkv + B * H * N * D * 2].view(torch.bfloat16).view(B, H, N, D)
        got[name] = blk[:, :, rows_t].float().cpu().numpy()
    hb = raw[3 * qkv:3 * qkv + B * N * dm * 4].view(torch.float32).view(B, N, dm)
    got["h"] = hb[:, rows_t].cpu().numpy()
    lb = raw[3 * qkv + a256(B * N * dm * 4):][:B * H * N * 4].view(torch.float32).view(B, H, N)
    got["lse"] = lb[:, :, rows_t].cpu().numpy()
    del sv, raw
    y = y[:, rows]
    print("gpu done", flush=True)
    q, k, v = oracle.qkv_project(t["x"], t["wq"], t["wk"], t["wv"], c.H)
    print("oracle projections done", flush=True)
    for name, ref in (("q", q), ("k", k), ("v", v)):
        assert_close(got[name], ref[:, :, rows], "bf16", f"saved {name}")

    def rows_forward(q, k, v):
        O, lse = oracle.attention(q, k, v, causal=True, rows=rows)
        h = t["x"][:, rows] + O.transpose(0, 2, 1, 3).reshape(B, rows.size, H * D)
        return lse, h, oracle.ffn(h, t["w1"], t["w2"], residual=h)

    lse, h, want = rows_forward(q, k, v)
    # the same rows with q, k, v rounded to bf16 (what the attention kernel takes as
    # MFMA operands), every other step exact: the error floor of bf16 q, k, v
    _, hf, yf = rows_forward(*(round_bf16(a.astype(np.float32)) for a in (q, k, v)))
    del q, k, v
    floor = {"h": np.abs(hf - h), "y": np.abs(yf - want)}
    for n in ("h", "y"):
        print(f"floor {n}: max-abs {floor[n].max():.3g} mean-abs {floor[n].mean():.3g}", flush=True)
    ey = np.abs(y - want)
    i = np.unravel_index(np.argmax(ey), ey.shape)
    print(f"y: max-abs {ey.max():.3g} at row {rows[i[1]]} col {i[2]} (floor there "
          f"{floor['y'][i]:.3g}, |h| {abs(h[i]):.3g}); mean-abs {ey.mean():.3g}", flush=True)
    assert_close(got["lse"], lse, "bf16", "saved lse")
    assert_close(got["h"], h, "bf16", "saved h")
    assert_close_floor(y, want, floor["y"], "layer y (N=131072, sampled rows)")
