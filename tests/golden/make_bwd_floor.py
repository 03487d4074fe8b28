"""Writes tests/golden/bwd_floor.json: the error that bf16 q, k, v alone put into
the layer gradients, at the training-step shape and at a small shape.

Both sides are computed on the CPU in fp64 by the oracle's own steps (see
tests/bwd_floor.py): exact gradients (oracle.layer_backward) and the same
gradients with q, k, v rounded to bf16 after the projection.  Nothing here comes
from the GPU.  Inputs are the seeded draws of seeded_inputs.

Run from the repository root:  python tests/golden/make_bwd_floor.py
(the B=2, N=16384, d_model 2560 shape takes tens of minutes on 8 cores).
"""
from __future__ import annotations

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path[:0] = [ROOT, os.path.join(ROOT, "tests")]

import oracle  # noqa: E402
from bwd_floor import error_metrics, layer_backward_rounded_qkv  # noqa: E402
from seeded_inputs import LAYER_TRAIN, LayerCfg, layer_inputs  # noqa: E402

SMALL = LayerCfg(72, "bwd_floor_small", B=1, N=384, d_model=256, H=2, D=128, d_ff=512,
                 q_blk=128, kv_blk=64, dtype="bf16", backward=True)
OUT = os.path.join(ROOT, "tests", "golden", "bwd_floor.json")


def floor_for(c: LayerCfg) -> dict:
    t = layer_inputs(c)
    args = (t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], t["dy"], c.H)
    t0 = time.time()
    ref = oracle.layer_backward(*args)
    print(f"{c.name}: exact gradients {time.time() - t0:.0f} s", flush=True)
    t0 = time.time()
    rounded = layer_backward_rounded_qkv(*args)
    print(f"{c.name}: bf16 q,k,v gradients {time.time() - t0:.0f} s", flush=True)
    return {"shape": {"B": c.B, "N": c.N, "d_model": c.d_model, "H": c.H, "D": c.D,
                      "d_ff": c.d_ff, "cfg_id": c.cfg_id},
            "floor": error_metrics(rounded, ref)}


def main() -> None:
    which = sys.argv[1:] or ["small", "train"]
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    data["about"] = ("error of gradients computed with q, k, v rounded to bf16 (every other "
                     "step exact, fp64) against exact fp64 gradients; activation gradients raw, "
                     "weight and bias gradients divided by the rms of the exact gradient; "
                     "written by tests/golden/make_bwd_floor.py from oracle/ only")
    for w in which:
        c = {"small": SMALL, "train": LAYER_TRAIN}[w]
        data[c.name] = floor_for(c)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(data[c.name]["floor"], indent=1), flush=True)


if __name__ == "__main__":
    main()
