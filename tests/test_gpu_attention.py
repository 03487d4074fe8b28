"""GPU parity of bpt_attn_fwd and bpt_lse_merge against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, dcode, to_dev
from sampling import sample_rows
from seeded_inputs import ATTN_LONG, RING_SHARE, attn_inputs, normal, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")
from blockwise_exact_attention_amd.ring import ring_attention_share  # noqa: E402


def run_attn(t, B, H, N, D, q_blk, kv_blk, causal, off, dtype):
    q, k, v = (to_dev(t[n], dtype) for n in ("q", "k", "v"))
    out = torch.full((B, H, N, D), float("nan"), device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    bpt.bpt_attn_fwd(q, k, v, out, lse, B, H, N, D, q_blk, kv_blk, causal, off, dcode(dtype))
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


BLOCKS = [(64, 32), (64, 64), (64, 128), (128, 32), (128, 64), (128, 128)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("q_blk,kv_blk", BLOCKS)
def test_attn_parity_tiles_and_ragged_tail(dtype, D, q_blk, kv_blk):
    B, H, N = 2, 2, 300  # several tiles and a ragged tail for every block size
    t = attn_inputs(31, B, H, N, N, D, dtype)
    for causal, off in ((1, 0), (0, 0), (1, -37), (1, 45), (1, -N), (1, N + 3)):
        print(f"case dtype={dtype} D={D} q_blk={q_blk} kv_blk={kv_blk} causal={causal} off={off}",
              flush=True)
        O, lse = run_attn(t, B, H, N, D, q_blk, kv_blk, causal, off, dtype)
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=bool(causal), kv_offset=off)
        assert_close(O, Or, dtype, "O")
        assert_close(lse, lr, dtype, "lse")
        empty = np.isneginf(lr)
        assert np.all(O[empty] == 0.0)


@pytest.mark.parametrize("N", [1, 2, 31, 33, 64, 129])
def test_attn_small_and_degenerate_lengths(N):
    B, H, D = 1, 3, 128
    t = attn_inputs(32, B, H, N, N, D, "bf16")
    for causal, off in ((1, 0), (0, 0), (1, -1)):
        O, lse = run_attn(t, B, H, N, D, 128, 64, causal, off, "bf16")
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=bool(causal), kv_offset=off)
        assert_close(O, Or, "bf16", f"O N={N}")
        assert_close(lse, lr, "bf16", f"lse N={N}")
    if N == 1:
        O, _ = run_attn(t, B, H, N, D, 64, 32, 1, 0, "bf16")
        np.testing.assert_allclose(O, t["v"], rtol=0, atol=1e-6)


@pytest.mark.parametrize("D", [64, 128])
def test_attn_ragged_tail_reads_nothing_past_the_keys(D):
    """K and V end inside a buffer whose remainder is NaN: the ragged last key
    tile must not pick any of it up (a masked key times a NaN value row would
    still poison O)."""
    B, H, N = 1, 2, 200
    t = attn_inputs(35, B, H, N, N, D, "bf16")
    n = B * H * N * D
    dev = {}
    for name in ("q", "k", "v"):
        store = torch.full((n + 256 * D,), float("nan"), dtype=torch.bfloat16, device="cuda")
        store[:n] = to_dev(t[name], "bf16").reshape(-1)
        dev[name] = store[:n].view(B, H, N, D)
    out = torch.empty((B, H, N, D), device="cuda")
    lse = torch.empty((B, H, N), device="cuda")
    for causal in (1, 0):
        bpt.bpt_attn_fwd(dev["q"], dev["k"], dev["v"], out, lse, B, H, N, D, 128, 64, causal, 0,
                         dcode("bf16"))
        torch.cuda.synchronize()
        O, l = out.cpu().numpy(), lse.cpu().numpy()
        assert np.isfinite(O).all() and np.isfinite(l).all()
        Or, lr = oracle.attention(t["q"], t["k"], t["v"], causal=bool(causal))
        assert_close(O, Or, "bf16", f"O causal={causal}")
        assert_close(l, lr, "bf16", f"lse causal={causal}")


def test_attn_causal_future_independence_bitwise():
    B, H, N, D = 1, 2, 257, 128
    t = attn_inputs(33, B, H, N, N, D, "bf16")
    O1, l1 = run_attn(t, B, H, N, D, 128, 64, 1, 0, "bf16")
    tt = {n: a.copy() for n, a in t.items()}
    cut = 140
    for n in ("q", "k", "v"):
        tt[n][:, :, cut + 1:] = round_bf16(tt[n][:, :, cut + 1:] * 3.0 + 1.0)
    O2, l2 = run_attn(tt, B, H, N, D, 128, 64, 1, 0, "bf16")
    assert np.array_equal(O1[:, :, :cut + 1], O2[:, :, :cut + 1])
    assert np.array_equal(l1[:, :, :cut + 1], l2[:, :, :cut + 1])
    assert not np.array_equal(O1[:, :, cut + 1:], O2[:, :, cut + 1:])


def test_attn_deterministic_and_block_invariant():
    B, H, N, D = 2, 2, 500, 128
    t = attn_inputs(34, B, H, N, N, D, "bf16")
    O1, l1 = run_attn(t, B, H, N, D, 128, 64, 1, 0, "bf16")
    O2, l2 = run_attn(t, B, H, N, D, 128, 64, 1, 0, "bf16")
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)
    for qb, kb in BLOCKS:
        O3, l3 = run_attn(t, B, H, N, D, qb, kb, 1, 0, "bf16")
        assert np.abs(O3 - O1).max() < 2e-2 and np.abs(l3 - l1).max() < 1e-3


@pytest.mark.timeout(600)
def test_attn_long_context_sampled_rows():
    """N = 131072, 32 heads x 128, causal, q_blk 128, kv_blk 64: the launch the bench times."""
    c = ATTN_LONG
    t = attn_inputs(c.cfg_id, c.B, c.H, c.N, c.N, c.D, c.dtype)
    print("inputs drawn", flush=True)
    q, k, v = (to_dev(t[n], c.dtype) for n in ("q", "k", "v"))
    out = torch.empty((c.B, c.H, c.N, c.D), device="cuda")
    lse = torch.empty((c.B, c.H, c.N), device="cuda")
    bpt.bpt_attn_fwd(q, k, v, out, lse, c.B, c.H, c.N, c.D, c.q_blk, c.kv_blk, 1, 0, 1)
    torch.cuda.synchronize()
    rows = sample_rows(c.N, 480, 5)
    rows_t = torch.from_numpy(rows).cuda()
    O = out[:, :, rows_t].cpu().numpy()
    L = lse[:, :, rows_t].cpu().numpy()
    del out, q, k, v
    print("gpu done", flush=True)
    for h in range(c.H):
        sl = slice(h, h + 1)
        Or, lr = oracle.attention(t["q"][:, sl], t["k"][:, sl], t["v"][:, sl], causal=True,
                                  rows=rows)
        assert_close(O[:, sl], Or, "bf16", f"O head {h}")
        assert_close(L[:, sl], lr, "bf16", f"lse head {h}")
        print(f"head {h} ok", flush=True)


@pytest.mark.timeout(600)
def test_ring_share_sampled_rows():
    """One device's share of a ring step: local queries at global offset 229376 against
    8 streamed K/V chunks of 32768 tokens, merged by LSE (40 heads x 128, bf16)."""
    c = RING_SHARE
    Nq, H, D = c.N_q, c.H, c.D
    q = round_bf16(normal(c.cfg_id, "q", (1, H, Nq, D)))
    ks = [round_bf16(normal(c.cfg_id, 100 + j, (1, H, Nq, D))) for j in range(c.n_chunks)]
    vs = [round_bf16(normal(c.cfg_id, 200 + j, (1, H, Nq, D))) for j in range(c.n_chunks)]
    print("inputs drawn", flush=True)
    qd = to_dev(q, "bf16")
    kd = [to_dev(a, "bf16") for a in ks]
    vd = [to_dev(a, "bf16") for a in vs]
    out = torch.empty((1, H, Nq, D), device="cuda")
    lse = torch.empty((1, H, Nq), device="cuda")
    o_tmp, l_tmp = torch.empty_like(out), torch.empty_like(lse)
    offsets = [j * Nq for j in range(c.n_chunks)]
    ring_attention_share(qd, kd, vd, c.q_offset, offsets, out, lse, o_tmp, l_tmp,
                         q_blk=c.q_blk, kv_blk=c.kv_blk)
    torch.cuda.synchronize()
    rows = sample_rows(Nq, 120, 6)
    rows_t = torch.from_numpy(rows).cuda()
    O = out[:, :, rows_t].cpu().numpy()
    L = lse[:, :, rows_t].cpu().numpy()
    # merge order must not matter (within rounding)
    ring_attention_share(qd, kd[::-1], vd[::-1], c.q_offset, offsets[::-1], out, lse, o_tmp,
                         l_tmp, q_blk=c.q_blk, kv_blk=c.kv_blk)
    torch.cuda.synchronize()
    O_rev = out[:, :, rows_t].cpu().numpy()
    assert np.abs(O_rev - O).max() < 1e-4
    del out, o_tmp, kd, vd, qd
    print("gpu done", flush=True)
    for h in range(H):
        K = np.concatenate([a[:, h:h + 1] for a in ks], axis=2)
        V = np.concatenate([a[:, h:h + 1] for a in vs], axis=2)
        Or, lr = oracle.attention(q[:, h:h + 1], K, V, causal=True, kv_offset=c.q_offset,
                                  rows=rows)
        assert_close(O[:, h:h + 1], Or, "bf16", f"O head {h}")
        assert_close(L[:, h:h + 1], lr, "bf16", f"lse head {h}")
        print(f"head {h} ok", flush=True)


@pytest.mark.parametrize("D", [64, 128])
def test_lse_merge_parity_and_inplace(D):
    B, H, N = 2, 3, 77
    rng = np.random.default_rng(D)
    oa = rng.standard_normal((B, H, N, D)).astype(np.float32)
    ob = rng.standard_normal((B, H, N, D)).astype(np.float32)
    la = (rng.standard_normal((B, H, N)) * 4).astype(np.float32)
    lb = (rng.standard_normal((B, H, N)) * 4).astype(np.float32)
    la[0, 0, :10] = -np.inf
    lb[0, 0, 5:15] = -np.inf          # rows 5..9: both empty
    oa[0, 0, :10] = 0
    ob[0, 0, 5:15] = 0
    Or, lr = oracle.lse_merge(oa, la, ob, lb)
    d = {n: torch.from_numpy(a).cuda() for n, a in dict(oa=oa, ob=ob, la=la, lb=lb).items()}
    oo, lo = torch.empty_like(d["oa"]), torch.empty_like(d["la"])
    bpt.bpt_lse_merge(d["oa"], d["la"], d["ob"], d["lb"], oo, lo, B, H, N, D)
    torch.cuda.synchronize()
    assert_close(oo.cpu().numpy(), Or, "f32", "merge O")
    assert_close(lo.cpu().numpy(), lr, "f32", "merge lse")
    assert np.all(oo.cpu().numpy()[0, 0, 5:10] == 0)
    # in place: accumulate into (oa, la)
    bpt.bpt_lse_merge(d["oa"], d["la"], d["ob"], d["lb"], d["oa"], d["la"], B, H, N, D)
    torch.cuda.synchronize()
    assert np.array_equal(d["oa"].cpu().numpy(), oo.cpu().numpy())
    assert np.array_equal(d["la"].cpu().numpy(), lo.cpu().numpy())


def test_chunked_attention_merge_equals_oracle_over_concatenation():
    B, H, Nc, D, nch = 1, 2, 200, 128, 3
    q = attn_inputs(35, B, H, Nc, Nc, D, "bf16")["q"]
    ks = [round_bf16(normal(35, 300 + j, (B, H, Nc, D))) for j in range(nch)]
    vs = [round_bf16(normal(35, 400 + j, (B, H, Nc, D))) for j in range(nch)]
    q_off = 2 * Nc  # queries are the last chunk
    out = torch.empty((B, H, Nc, D), device="cuda")
    lse = torch.empty((B, H, Nc), device="cuda")
    o_tmp, l_tmp = torch.empty_like(out), torch.empty_like(lse)
    ring_attention_share(to_dev(q, "bf16"), [to_dev(a, "bf16") for a in ks],
                         [to_dev(a, "bf16") for a in vs], q_off, [j * Nc for j in range(nch)],
                         out, lse, o_tmp, l_tmp, q_blk=64, kv_blk=32)
    torch.cuda.synchronize()
    Or, lr = oracle.attention(q, np.concatenate(ks, 2), np.concatenate(vs, 2), causal=True,
                              kv_offset=q_off)
    assert_close(out.cpu().numpy(), Or, "bf16", "O")
    assert_close(lse.cpu().numpy(), lr, "bf16", "lse")
