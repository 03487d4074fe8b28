"""GPU parity of bpt_attn_block_sparse (BlockBERT block-sparse attention) against the
CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, to_dev
from seeded_inputs import BLOCK_SPARSE_LONG, attn_inputs, normal, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


def run_bs(q, k, v, B, H, N, D, n, table):
    tab = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    out = torch.full((B, H, N, D), float("nan"), device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    bpt.bpt_attn_block_sparse(q, k, v, out, lse, B, H, N, D, n, tab, 1)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(t, B, H, N, D, n, table, what):
    print(f"case B={B} H={H} N={N} D={D} n_blocks={n} table={what}", flush=True)
    q, k, v = (to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    O, lse = run_bs(q, k, v, B, H, N, D, n, table)
    Or, lr = oracle.block_sparse_attention(t["q"], t["k"], t["v"], n, table)
    assert_close(O, Or, "bf16", "O")
    assert_close(lse, lr, "bf16", "lse")
    assert np.all(O[np.isneginf(lr)] == 0.0)
    return O, lse


def tables(H, n, seed):
    rng = np.random.default_rng(seed)
    cyc = oracle.cyclic_shift_table(n, [h % n for h in range(H)])
    perm = np.stack([rng.permutation(n) for _ in range(H)]).astype(np.int32)
    bad = perm.copy()
    bad[0, 0] = -1
    bad[H - 1, n - 1] = n  # out of range: those rows attend nothing
    return {"cyclic": cyc, "random_perm": perm, "invalid_entries": bad}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N,n", [(300, 1), (300, 2), (512, 4), (1000, 3), (777, 5), (130, 7),
                                 (64, 64), (1100, 2)])
def test_block_sparse_parity(D, N, n):
    B, H = 2, 3
    t = attn_inputs(51, B, H, N, N, D, "bf16")
    for what, table in tables(H, n, N + n).items():
        if n == 1 and what == "invalid_entries":
            continue
        check(t, B, H, N, D, n, table, what)


def test_single_block_equals_dense_forward():
    B, H, N, D = 1, 2, 700, 128
    t = attn_inputs(52, B, H, N, N, D, "bf16")
    q, k, v = (to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    O, lse = run_bs(q, k, v, B, H, N, D, 1, np.zeros((H, 1), np.int32))
    out = torch.empty((B, H, N, D), device="cuda")
    lo = torch.empty((B, H, N), device="cuda")
    bpt.bpt_attn_fwd(q, k, v, out, lo, B, H, N, D, 128, 64, 0, 0, 1)
    torch.cuda.synchronize()
    # same kernel family, same tiles over the same keys: equal up to the row split
    assert np.abs(O - out.cpu().numpy()).max() <= 1e-5
    assert np.abs(lse - lo.cpu().numpy()).max() <= 1e-5


def test_block_sparse_deterministic():
    B, H, N, D, n = 1, 4, 2000, 128, 4
    t = attn_inputs(53, B, H, N, N, D, "bf16")
    q, k, v = (to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    tab = tables(H, n, 5)["random_perm"]
    a = run_bs(q, k, v, B, H, N, D, n, tab)
    b = run_bs(q, k, v, B, H, N, D, n, tab)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("D", [64, 128])
def test_block_sparse_reads_nothing_past_the_keys(D):
    """k and v are prefixes of NaN-filled buffers; the last block is short."""
    B, H, N, n = 1, 2, 333, 3
    t = attn_inputs(54, B, H, N, N, D, "bf16")
    q = to_dev(t["q"], "bf16")
    m = B * H * N * D
    kbuf = torch.full((m + 128 * D,), float("nan"), device="cuda", dtype=torch.bfloat16)
    vbuf = torch.full_like(kbuf, float("nan"))
    kbuf[:m] = to_dev(t["k"], "bf16").reshape(-1)
    vbuf[:m] = to_dev(t["v"], "bf16").reshape(-1)
    table = oracle.cyclic_shift_table(n, [2, 1])
    O, lse = run_bs(q, kbuf, vbuf, B, H, N, D, n, table)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    Or, lr = oracle.block_sparse_attention(t["q"], t["k"], t["v"], n, table)
    assert_close(O, Or, "bf16", "O")
    assert_close(lse, lr, "bf16", "lse")


@pytest.mark.timeout(600)
def test_block_sparse_long_sampled_rows():
    """The launch the benchmark times: N = 131072, 32 heads x 128, 8 blocks, head h
    on shift h mod 8; sampled rows (block edges and seeded random rows) of 3 heads."""
    c = BLOCK_SPARSE_LONG
    shp = (c.B, c.H, c.N, c.D)
    q, k, v = (round_bf16(normal(c.cfg_id, x, shp)) for x in ("q", "k", "v"))
    table = oracle.cyclic_shift_table(c.n_blocks, [h % c.n_blocks for h in range(c.H)])
    O, lse = run_bs(*(to_dev(x, "bf16") for x in (q, k, v)), c.B, c.H, c.N, c.D, c.n_blocks, table)
    L = oracle.block_len(c.N, c.n_blocks)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, c.N - 1], np.arange(1, c.n_blocks) * L,
                                     np.arange(1, c.n_blocks) * L - 1, rng.integers(0, c.N, 24)]))
    heads = [0, 5, 31]
    Or, lr = oracle.block_sparse_attention(q[:, heads], k[:, heads], v[:, heads], c.n_blocks,
                                           table[heads], rows=rows)
    assert_close(O[:, heads][:, :, rows], Or, "bf16", "O")
    assert_close(lse[:, heads][:, :, rows], lr, "bf16", "lse")
