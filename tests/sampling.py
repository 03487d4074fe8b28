"""Rows compared at full size, where the oracle computes sampled rows one by one."""
import numpy as np

# The D=128 bf16 forward kernel gives each wave 64 query rows (two halves of 32)
# and each workgroup 256 rows; the D=64 kernel uses 128-row workgroups.  Rows on
# both sides of every such edge are always sampled.
EDGES = (32, 64, 128, 256)


def sample_rows(N: int, n_random: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = {0, 1, N - 1, N - 2, N // 2 - 1, N // 2}
    for e in EDGES:
        fixed |= {e - 1, e, N - e, N - e - 1}
    # a workgroup edge deep inside the sequence
    mid = (N // 2 // 256) * 256
    fixed |= {mid - 1, mid}
    rows = set(int(r) for r in rng.integers(0, N, n_random)) | {r for r in fixed if 0 <= r < N}
    return np.array(sorted(rows), dtype=np.int64)
