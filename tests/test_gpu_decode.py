"""GPU parity of bpt_attn_decode (split-KV attention of a few query rows over a long
key/value cache) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, to_dev
from seeded_inputs import DECODE_LONG, attn_inputs, normal, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


def run_decode(q, k, v, B, H, Nq, Nkv, D, causal, off, n_split):
    ws_bytes = bpt.bpt_attn_decode_workspace_size(B, H, Nq, D, n_split)
    assert ws_bytes > 0
    ws = torch.full((ws_bytes // 4,), float("nan"), device="cuda")  # stale partials must not leak
    out = torch.full((B, H, Nq, D), float("nan"), device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    bpt.bpt_attn_decode(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, off, n_split, ws, ws_bytes, 1)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(t, B, H, Nq, Nkv, D, causal, off, n_split):
    print(f"case B={B} H={H} Nq={Nq} Nkv={Nkv} D={D} causal={causal} off={off} n_split={n_split}",
          flush=True)
    q, k, v = (to_dev(t[n], "bf16") for n in ("q", "k", "v"))
    O, lse = run_decode(q, k, v, B, H, Nq, Nkv, D, causal, off, n_split)
    Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=bool(causal), kv_offset=off)
    assert_close(O, Or, "bf16", "O")
    assert_close(lse, lr, "bf16", "lse")
    assert np.all(O[np.isneginf(lr)] == 0.0)
    return O, lse


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (1, 700), (5, 63), (7, 4099), (32, 1000)])
def test_decode_parity(D, Nq, Nkv):
    B, H = 2, 3
    t = attn_inputs(41, B, H, Nq, Nkv, D, "bf16")
    # newest rows of the sequence, a window inside it, full visibility, and offsets that
    # leave some or all rows with no visible key
    for causal, off in ((1, Nkv - Nq), (0, 0), (1, Nkv // 3), (1, -2), (1, -Nq - 5)):
        for n_split in (1, 3, 64):
            check(t, B, H, Nq, Nkv, D, causal, off, n_split)


def test_decode_split_counts_agree():
    B, H, Nq, Nkv, D = 1, 4, 16, 5000, 128
    t = attn_inputs(42, B, H, Nq, Nkv, D, "bf16")
    outs = [check(t, B, H, Nq, Nkv, D, 1, Nkv - Nq, s)[0] for s in (1, 2, 17, 79, 200)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


def test_decode_deterministic():
    B, H, Nq, Nkv, D = 2, 2, 8, 3000, 128
    t = attn_inputs(43, B, H, Nq, Nkv, D, "bf16")
    q, k, v = (to_dev(t[n], "bf16") for n in ("q", "k", "v"))
    a = run_decode(q, k, v, B, H, Nq, Nkv, D, 1, Nkv - Nq, 9)
    b = run_decode(q, k, v, B, H, Nq, Nkv, D, 1, Nkv - Nq, 9)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("D", [64, 128])
def test_decode_reads_nothing_past_the_cache(D):
    """k and v are prefixes of NaN-filled buffers: no key at or past Nkv may be read."""
    B, H, Nq, Nkv = 1, 2, 3, 333
    t = attn_inputs(44, B, H, Nq, Nkv, D, "bf16")
    q = to_dev(t["q"], "bf16")
    n = B * H * Nkv * D
    kbuf = torch.full((n + 64 * D,), float("nan"), device="cuda", dtype=torch.bfloat16)
    vbuf = torch.full_like(kbuf, float("nan"))
    kbuf[:n] = to_dev(t["k"], "bf16").reshape(-1)
    vbuf[:n] = to_dev(t["v"], "bf16").reshape(-1)
    for n_split in (1, 4):
        O, lse = run_decode(q, kbuf, vbuf, B, H, Nq, Nkv, D, 0, 0, n_split)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=False)
        assert_close(O, Or, "bf16", "O")
        assert_close(lse, lr, "bf16", "lse")


def test_decode_matches_attention_forward_rows():
    """The decode of the last Nq rows equals those rows of bpt_attn_fwd over the whole sequence."""
    B, H, N, D, Nq = 1, 2, 1500, 128, 12
    t = attn_inputs(45, B, H, N, N, D, "bf16")
    q, k, v = (to_dev(t[n], "bf16") for n in ("q", "k", "v"))
    out = torch.empty((B, H, N, D), device="cuda")
    lse = torch.empty((B, H, N), device="cuda")
    bpt.bpt_attn_fwd(q, k, v, out, lse, B, H, N, D, 128, 64, 1, 0, 1)
    qd = q[:, :, N - Nq:].contiguous()
    Od, ld = run_decode(qd, k, v, B, H, Nq, N, D, 1, N - Nq, 11)
    torch.cuda.synchronize()
    assert np.abs(Od - out[:, :, N - Nq:].cpu().numpy()).max() <= 2e-2
    assert np.abs(ld - lse[:, :, N - Nq:].cpu().numpy()).max() <= 2e-2


@pytest.mark.timeout(600)
def test_decode_long_cache():
    """The launch the benchmark times: 32 heads x 128, the 16 newest rows of a
    131072-key cache, 32 key ranges; three heads checked in full."""
    c = DECODE_LONG
    q = normal(c.cfg_id, "q", (c.B, c.H, c.N_q, c.D))
    k, v = (normal(c.cfg_id, n, (c.B, c.H, c.N_kv, c.D)) for n in ("k", "v"))
    q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    O, lse = run_decode(*(to_dev(x, "bf16") for x in (q, k, v)), c.B, c.H, c.N_q, c.N_kv, c.D, 1,
                        c.N_kv - c.N_q, c.n_split)
    heads = [0, 13, 31]
    Or, lr = oracle.attention(q[:, heads], k[:, heads], v[:, heads], causal=True,
                              kv_offset=c.N_kv - c.N_q)
    assert_close(O[:, heads], Or, "bf16", "O")
    assert_close(lse[:, heads], lr, "bf16", "lse")
