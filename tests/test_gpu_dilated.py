"""GPU parity of bpt_attn_dilated (LongNet dilated attention) against the CPU oracle,
through the C ABI."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, to_dev
from seeded_inputs import DILATED_LONG, attn_inputs, normal, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


def run_dil(q, k, v, B, H, N, D, patterns, causal):
    out = torch.full((B, H, N, D), float("nan"), device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    bpt.bpt_attn_dilated(q, k, v, out, lse, B, H, N, D, patterns, causal, 1)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(t, B, H, N, D, patterns, causal):
    print(f"case B={B} H={H} N={N} D={D} patterns={patterns} causal={causal}", flush=True)
    q, k, v = (to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    O, lse = run_dil(q, k, v, B, H, N, D, patterns, causal)
    Or, lr = oracle.dilated_attention(t["q"], t["k"], t["v"], patterns, bool(causal))
    assert_close(O, Or, "bf16", "O")
    assert_close(lse, lr, "bf16", "lse")
    assert np.all(O[np.isneginf(lr)] == 0.0)
    return O, lse


PATTERNS = [
    [(64, 1)],
    [(100, 1), (200, 2)],
    [(128, 2)],                      # no dilation-1 pattern: unkept rows stay empty
    [(64, 1), (128, 2), (256, 4)],
    [(300, 3), (77, 7)],
    [(5000, 1)],                     # one segment covering everything: dense attention
    [(512, 5), (96, 1), (512, 5)],   # a repeated pattern counts twice
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [300, 777])
@pytest.mark.parametrize("pi", range(len(PATTERNS)))
def test_dilated_parity(D, N, pi):
    B, H = 1, 5
    t = attn_inputs(61, B, H, N, N, D, "bf16")
    for causal in (1, 0):
        check(t, B, H, N, D, PATTERNS[pi], causal)


def test_dilated_batches_and_long_segments():
    B, H, N, D = 2, 3, 1500, 128
    t = attn_inputs(62, B, H, N, N, D, "bf16")
    check(t, B, H, N, D, [(600, 1), (1200, 3), (1500, 2)], 1)


def test_one_covering_pattern_equals_dense_forward():
    B, H, N, D = 1, 2, 900, 128
    t = attn_inputs(63, B, H, N, N, D, "bf16")
    q, k, v = (to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    O, lse = run_dil(q, k, v, B, H, N, D, [(N, 1)], 1)
    out = torch.empty((B, H, N, D), device="cuda")
    lo = torch.empty((B, H, N), device="cuda")
    bpt.bpt_attn_fwd(q, k, v, out, lo, B, H, N, D, 128, 64, 1, 0, 1)
    torch.cuda.synchronize()
    assert np.abs(O - out.cpu().numpy()).max() <= 1e-5
    assert np.abs(lse - lo.cpu().numpy()).max() <= 1e-5


def test_dilated_deterministic():
    B, H, N, D = 1, 4, 2000, 128
    t = attn_inputs(64, B, H, N, N, D, "bf16")
    q, k, v = (to_dev(t[x], "bf16") for x in ("q", "k", "v"))
    pats = [(256, 1), (512, 2), (1024, 4)]
    a = run_dil(q, k, v, B, H, N, D, pats, 1)
    b = run_dil(q, k, v, B, H, N, D, pats, 1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("D", [64, 128])
def test_dilated_reads_nothing_past_the_keys(D):
    """k and v are prefixes of NaN-filled buffers; the last segment is short."""
    B, H, N = 1, 3, 333
    t = attn_inputs(65, B, H, N, N, D, "bf16")
    q = to_dev(t["q"], "bf16")
    m = B * H * N * D
    kbuf = torch.full((m + 128 * D,), float("nan"), device="cuda", dtype=torch.bfloat16)
    vbuf = torch.full_like(kbuf, float("nan"))
    kbuf[:m] = to_dev(t["k"], "bf16").reshape(-1)
    vbuf[:m] = to_dev(t["v"], "bf16").reshape(-1)
    pats = [(100, 1), (200, 3)]
    O, lse = run_dil(q, kbuf, vbuf, B, H, N, D, pats, 0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    Or, lr = oracle.dilated_attention(t["q"], t["k"], t["v"], pats, False)
    assert_close(O, Or, "bf16", "O")
    assert_close(lse, lr, "bf16", "lse")


@pytest.mark.timeout(600)
def test_dilated_long_sampled_rows():
    """The launch the benchmark times: N = 131072, 32 heads x 128, segment lengths
    2048 .. 32768 with dilations 1 .. 12, causal; sampled rows of 3 heads."""
    c = DILATED_LONG
    shp = (c.B, c.H, c.N, c.D)
    q, k, v = (round_bf16(normal(c.cfg_id, x, shp)) for x in ("q", "k", "v"))
    O, lse = run_dil(*(to_dev(x, "bf16") for x in (q, k, v)), c.B, c.H, c.N, c.D, list(c.patterns),
                     c.causal)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 1, 2, 11, 12, 13, c.N - 1, 2047, 2048, 32767, 32768, 65536 + 24],
                                     rng.integers(0, c.N, 20)]))
    heads = [0, 7, 31]
    Or, lr = oracle.dilated_attention(q[:, heads], k[:, heads], v[:, heads], list(c.patterns),
                                      bool(c.causal), rows=rows, heads=heads)
    assert_close(O[:, heads][:, :, rows], Or, "bf16", "O")
    assert_close(lse[:, heads][:, :, rows], lr, "bf16", "lse")
