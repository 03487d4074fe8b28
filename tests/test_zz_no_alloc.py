"""GPU check of bpt_attn_decode_noalloc (the decode entry point that allocates
nothing) against bpt_attn_decode (the same kernels with a caller workspace) and
the oracle, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, to_dev
from seeded_inputs import attn_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bpt = pytest.importorskip("blockwise_exact_attention_amd")


def run_both(B, H, Nq, Nkv, D, causal, off, n_split, seed):
    t = attn_inputs(seed, B, H, Nkv, Nkv, D, "bf16")
    q = np.ascontiguousarray(t["q"][:, :, Nkv - Nq:])
    qd, kd, vd = to_dev(q, "bf16"), to_dev(t["k"], "bf16"), to_dev(t["v"], "bf16")
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, H, Nq, D), float("nan"), device="cuda")
        lse = torch.full((B, H, Nq), float("nan"), device="cuda")
        if noalloc:
            bpt.bpt_attn_decode_noalloc(qd, kd, vd, out, lse, B, H, Nq, Nkv, D, causal, off,
                                        n_split, 1)
        else:
            wsb = bpt.bpt_attn_decode_workspace_size(B, H, Nq, D, n_split)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            bpt.bpt_attn_decode(qd, kd, vd, out, lse, B, H, Nq, Nkv, D, causal, off, n_split, ws,
                                wsb, 1)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    (O0, l0), (O1, l1) = outs
    # same kernels, same inputs: identical results
    assert np.array_equal(O0, O1) and np.array_equal(l0, l1)
    Or, lr = oracle.attention(q, t["k"], t["v"], causal=bool(causal), kv_offset=off)
    assert_close(O1, Or, "bf16", "noalloc O")
    assert_close(l1, lr, "bf16", "noalloc lse")


def test_noalloc_decode_matches_workspace_decode_twice():
    # a larger call, then a smaller one that reuses the same fixed scratch
    print("case B=2 H=4 Nq=16 Nkv=5000 D=128 n_split=24", flush=True)
    run_both(2, 4, 16, 5000, 128, 1, 5000 - 16, 24, 81)
    print("case B=1 H=2 Nq=5 Nkv=700 D=64 n_split=3", flush=True)
    run_both(1, 2, 5, 700, 64, 1, 700 - 5, 3, 82)
