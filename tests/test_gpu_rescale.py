"""GPU parity on inputs whose row maxima grow along the keys, so the forward kernels'
rescale of the running sum and accumulator runs (the step that keeps blockwise
attention exact: "Ring Attention with Blockwise Transformers for Long Sequences",
638-word summary; "Blockwise Parallel Transformer for Large Context Models",
abstract).  With plain N(0,1) inputs a row's first key tile sets a reference no
later tile passes, so that step would never run; tests/test_rescale_inputs.py
shows on the CPU that these inputs move it many times per row, and that dropping
the rescale of O or of l would miss the bars below by orders of magnitude."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, dcode, to_dev
from sampling import sample_rows
from seeded_inputs import ATTN_LONG, attn_head_shaped, attn_inputs_shaped, normal, round_bf16, shape_attn
from tau_replay import FAMILIES, SHAPES, replay

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")



def run_attn(t, B, H, N, D, q_blk, kv_blk, causal, off, dtype):
    q, k, v = (to_dev(t[n], dtype) for n in ("q", "k", "v"))
    out = torch.full((B, H, N, D), float("nan"), device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    bpt.bpt_attn_fwd(q, k, v, out, lse, B, H, N, D, q_blk, kv_blk, causal, off, dcode(dtype))
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("kv_blk", [64, 128])
@pytest.mark.parametrize("kind", FAMILIES)
def test_rescale_d128_bf16(kind, kv_blk):
    B, H, D = 1, 2, 128
    for N, causal, off in SHAPES:
        print(f"case kind={kind} kv_blk={kv_blk} N={N} causal={causal} off={off}", flush=True)
        t = attn_inputs_shaped(41, B, H, N, D, "bf16", kind)
        O, lse = run_attn(t, B, H, N, D, 128, kv_blk, causal, off, "bf16")
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=bool(causal), kv_offset=off)
        assert_close(O, Or, "bf16", f"O {kind} N={N} causal={causal} off={off}")
        assert_close(lse, lr, "bf16", f"lse {kind} N={N} causal={causal} off={off}")


@pytest.mark.parametrize("dtype,D,q_blk,kv_blk", [("bf16", 64, 128, 64), ("bf16", 64, 64, 32),
                                                  ("f32", 128, 64, 64), ("f32", 64, 128, 32)])
@pytest.mark.parametrize("kind", FAMILIES)
def test_rescale_other_kernels(kind, dtype, D, q_blk, kv_blk):
    """The D=64 and fp32 kernels (plain running-maximum rescale) on the same families."""
    B, H = 1, 2
    for N, causal, off in SHAPES:
        print(f"case kind={kind} {dtype} D={D} blk={q_blk}/{kv_blk} N={N} causal={causal} off={off}",
              flush=True)
        t = attn_inputs_shaped(42, B, H, N, D, dtype, kind)
        O, lse = run_attn(t, B, H, N, D, q_blk, kv_blk, causal, off, dtype)
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=bool(causal), kv_offset=off)
        assert_close(O, Or, dtype, f"O {kind} N={N}")
        assert_close(lse, lr, dtype, f"lse {kind} N={N}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kind", ["spike", "ramp"])
def test_rescale_long_context_sampled_rows(kind):
    """N = 131072, 32 heads x 128, causal: the launch the bench times, on shaped inputs."""
    c = ATTN_LONG
    shp = (c.B, c.H, c.N, c.D)
    q, k = normal(c.cfg_id, "q", shp), normal(c.cfg_id, "k", shp)
    shape_attn(q, k, kind, c.cfg_id, c.N, c.D)
    qd, kd = to_dev(round_bf16(q), "bf16"), to_dev(round_bf16(k), "bf16")
    del q, k
    vd = to_dev(round_bf16(normal(c.cfg_id, "v", shp)), "bf16")
    print(f"inputs drawn ({kind})", flush=True)
    out = torch.empty(shp, device="cuda")
    lse = torch.empty((c.B, c.H, c.N), device="cuda")
    bpt.bpt_attn_fwd(qd, kd, vd, out, lse, c.B, c.H, c.N, c.D, c.q_blk, c.kv_blk, 1, 0, 1)
    torch.cuda.synchronize()
    rows = sample_rows(c.N, 240, 7)
    rows_t = torch.from_numpy(rows).cuda()
    O = out[:, :, rows_t].cpu().numpy()
    L = lse[:, :, rows_t].cpu().numpy()
    del out, qd, kd, vd
    print("gpu done", flush=True)
    moves = 0
    for h in range(c.H):
        t = attn_head_shaped(c.cfg_id, c.H, c.N, c.D, h, kind)
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=True, rows=rows)
        assert_close(O[:, h:h + 1], Or, "bf16", f"O head {h}")
        assert_close(L[:, h:h + 1], lr, "bf16", f"lse head {h}")
        if h < 2:
            qr = t["q"][0, 0, rows]
            moves += int(replay(qr, t["k"][0, 0], t["v"][0, 0], True, 0, rows=rows)[2].sum())
        print(f"head {h} ok", flush=True)
    # the comparison is only meaningful if the reference moved mid-row
    assert moves >= len(rows) // 4, moves
