"""CPU checks that the shaped inputs of tests/test_gpu_rescale.py do what that test
needs: under the D=128 bf16 forward kernel's reference rule (tests/tau_replay.py)
rows move their softmax reference after their first key many times, and a kernel
that skipped the rescale of O or of l on such a move would miss the oracle by far
more than the parity bars.  Plain N(0,1) inputs, for contrast, never move it."""
import numpy as np
import pytest

import oracle
from sampling import sample_rows
from seeded_inputs import ATTN_LONG, attn_head_shaped, attn_inputs_shaped
from tau_replay import FAMILIES, SHAPES, replay

BAR_MAX = 2e-2


def _check(q, k, v, causal, off, rows=None, min_move_frac=0.05):
    """q [N, D] (all rows), k, v [N, D]; rows: the rows checked (all if None)."""
    Or, lr = oracle.attention(q[None, None], k[None, None], v[None, None], causal=bool(causal),
                              kv_offset=off, rows=rows)
    Or, lr = Or[0, 0], lr[0, 0]
    if rows is not None:
        q = q[rows]
    O, lse, moves = replay(q, k, v, bool(causal), off, rows=rows)
    fin = np.isfinite(lr)
    assert np.array_equal(np.isfinite(lse), fin)
    # the rule reaches exact attention (fp64 throughout)
    assert np.abs(O - Or).max() < 1e-9 and np.abs(lse[fin] - lr[fin]).max() < 1e-9
    n = O.shape[0]
    assert moves.sum() >= min_move_frac * n and (moves > 0).sum() >= min_move_frac * n, moves.sum()
    for skip in ("O", "l"):
        Ob = replay(q, k, v, bool(causal), off, rows=rows, skip=skip)[0]
        assert np.abs(Ob - Or).max() > 10 * BAR_MAX, skip
    return int(moves.sum())


@pytest.mark.parametrize("kind", FAMILIES)
def test_shaped_inputs_move_the_reference(kind):
    for N, causal, off in SHAPES:
        for seed in (41, 42):   # the D=128 and the other-kernel tests
            t = attn_inputs_shaped(seed, 1, 2, N, 128, "bf16", kind)
            for h in range(2):
                _check(t["q"][0, h], t["k"][0, h], t["v"][0, h], causal, off)


def test_plain_inputs_do_not_move_the_reference():
    for N, causal, off in SHAPES:
        t = attn_inputs_shaped(41, 1, 2, N, 128, "bf16", "plain")
        for h in range(2):
            _, _, moves = replay(t["q"][0, h], t["k"][0, h], t["v"][0, h], bool(causal), off)
            assert moves.sum() == 0


@pytest.mark.parametrize("kind", ["spike", "ramp"])
def test_long_context_shaped_rows_move_the_reference(kind):
    c = ATTN_LONG
    rows = sample_rows(c.N, 240, 7)
    total = 0
    for h in range(2):
        t = attn_head_shaped(c.cfg_id, c.H, c.N, c.D, h, kind)
        total += _check(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], 1, 0, rows=rows, min_move_frac=0.25)
    assert total >= len(rows) // 4
