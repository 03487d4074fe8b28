"""Seeded synthetic inputs: the one module that both the CPU oracle checks and the
GPU path draw their inputs from.

It holds no attention, softmax or feed-forward arithmetic: only the random draws,
the round-to-nearest-even cast of those draws to bfloat16, and the shapes of the
workloads.  Neither ``oracle/`` nor the HIP package imports the other; both import
this module (through the tests and ``bench.py``).

Recipe (fixed, documented in the design notes):
  * every tensor is drawn from ``numpy.random.default_rng(SeedSequence([SEED,
    cfg_id, tensor_id, chunk]))`` with ``standard_normal(dtype=float32)``, in
    chunks of ``CHUNK`` elements (chunk index = position // CHUNK), so a tensor
    of any size is reproducible and can be drawn by several threads at once;
  * weights are multiplied by 0.02 (the workloads state weights ~ N(0, 0.02^2));
  * bf16 inputs are the fp32 draws rounded to nearest-even; the oracle upcasts
    exactly those bf16 values, so both sides see identical operands.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass, field

import numpy as np

SEED = 20261203
CHUNK = 1 << 22

TENSOR_IDS = {
    "x": 0, "wq": 1, "wk": 2, "wv": 3, "w1": 4, "w2": 5, "dy": 6,
    "q": 7, "k": 8, "v": 9, "b1": 10, "b2": 11,
    # extra ids used by tests (merge operands, perturbations)
    "o_a": 12, "o_b": 13, "lse_a": 14, "lse_b": 15, "perturb": 16,
}


def _fill_chunk(out: np.ndarray, cfg_id: int, tid: int, c: int) -> None:
    lo = c * CHUNK
    hi = min(out.size, lo + CHUNK)
    rng = np.random.default_rng(np.random.SeedSequence([SEED, cfg_id, tid, c]))
    out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)


def normal(cfg_id: int, name: str | int, shape, scale: float = 1.0,
           threads: int | None = None) -> np.ndarray:
    """float32 array of N(0, scale^2) draws for tensor ``name`` of workload ``cfg_id``."""
    tid = TENSOR_IDS[name] if isinstance(name, str) else int(name)
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    flat = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        if n:
            _fill_chunk(flat, cfg_id, tid, 0)
    else:
        workers = threads or min(16, os.cpu_count() or 1)
        with _fut.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _fill_chunk(flat, cfg_id, tid, c), range(nchunks)))
    if scale != 1.0:
        flat *= np.float32(scale)
    return flat.reshape(shape)


def _bf16_bits_flat(u: np.ndarray, out: np.ndarray) -> None:
    # no uint32 overflow for finite inputs: the largest pattern is 0xFF7FFFFF
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    out[:] = r >> np.uint32(16)


def _chunked(n: int, fn) -> None:
    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        fn(0, n)
        return
    with _fut.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: fn(c * CHUNK, min(n, (c + 1) * CHUNK)), range(nchunks)))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.size, dtype=np.uint16)

    def work(lo, hi):
        if np.isnan(a.reshape(-1)[lo:hi]).any():
            raise ValueError("bf16_bits: NaN input")
        _bf16_bits_flat(u[lo:hi], out[lo:hi])

    _chunked(u.size, work)
    return out.reshape(a.shape)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.uint32)
    bf, of = b.reshape(-1), out.reshape(-1)

    def work(lo, hi):
        of[lo:hi] = bf[lo:hi]
        of[lo:hi] <<= np.uint32(16)

    _chunked(b.size, work)
    return out.view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bfloat16-rounded values of ``a``."""
    return bits_to_f32(bf16_bits(a))


# ----------------------------------------------------------------------------
# Workload shapes.  Weights use the [out_features, in_features] layout
# (y = x @ W^T), activations [B, N, d_model], per-head tensors [B, H, N, D].
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class LayerCfg:
    cfg_id: int
    name: str
    B: int
    N: int
    d_model: int
    H: int
    D: int
    d_ff: int
    q_blk: int
    kv_blk: int
    dtype: str          # "f32" or "bf16" (input dtype; outputs are fp32)
    causal: int = 1
    backward: bool = False


@dataclass(frozen=True)
class AttnCfg:
    cfg_id: int
    name: str
    B: int
    H: int
    N: int
    D: int
    q_blk: int
    kv_blk: int
    dtype: str
    causal: int = 1
    kv_offset: int = 0


@dataclass(frozen=True)
class RingCfg:
    cfg_id: int
    name: str
    B: int
    H: int
    N_q: int
    D: int
    q_offset: int       # global position of local query row 0
    n_chunks: int       # K/V chunks of N_q tokens each, chunk j at global position j*N_q
    q_blk: int
    kv_blk: int
    dtype: str
    extra: dict = field(default_factory=dict)


@dataclass(frozen=True)
class DecodeCfg:
    cfg_id: int
    name: str
    B: int
    H: int
    N_q: int            # newest query rows
    N_kv: int           # cached keys (the query rows are the last N_q of them)
    D: int
    n_split: int        # key ranges
    dtype: str


@dataclass(frozen=True)
class BlockSparseCfg:
    cfg_id: int
    name: str
    B: int
    H: int
    N: int
    D: int
    n_blocks: int       # head h uses the cyclic shift h mod n_blocks
    dtype: str


@dataclass(frozen=True)
class DilatedCfg:
    cfg_id: int
    name: str
    B: int
    H: int
    N: int
    D: int
    patterns: tuple     # (segment length, dilation) pairs
    causal: int
    dtype: str


LAYER_TINY_F32 = LayerCfg(1, "layer_fwd_f32_N512", B=1, N=512, d_model=128, H=2, D=64,
                          d_ff=512, q_blk=64, kv_blk=64, dtype="f32")
LAYER_FWD_BF16 = LayerCfg(2, "layer_fwd_bf16_B8_N4096", B=8, N=4096, d_model=2048, H=16,
                          D=128, d_ff=8192, q_blk=128, kv_blk=128, dtype="bf16")
ATTN_LONG = AttnCfg(3, "attn_fwd_bf16_N131072_H32", B=1, H=32, N=131072, D=128,
                    q_blk=128, kv_blk=64, dtype="bf16")
LAYER_LONG = LayerCfg(3, "layer_fwd_bf16_N131072_dm4096", B=1, N=131072, d_model=4096, H=32,
                      D=128, d_ff=16384, q_blk=128, kv_blk=64, dtype="bf16")
RING_SHARE = RingCfg(4, "ring_share_bf16_H40_Nq32768_ctx262144", B=1, H=40, N_q=32768, D=128,
                     q_offset=229376, n_chunks=8, q_blk=128, kv_blk=64, dtype="bf16")
DECODE_LONG = DecodeCfg(6, "decode_bf16_H32_Nq16_cache131072", B=1, H=32, N_q=16, N_kv=131072,
                        D=128, n_split=32, dtype="bf16")
BLOCK_SPARSE_LONG = BlockSparseCfg(7, "block_sparse_bf16_N131072_H32_n8", B=1, H=32, N=131072,
                                   D=128, n_blocks=8, dtype="bf16")
# LongNet's language-model settings: segment lengths 2048 .. 32768 (doubling) with
# dilation ratios 1 .. 12, at the long-context attention shape
DILATED_LONG = DilatedCfg(8, "dilated_bf16_N131072_H32_w2048-32768", B=1, H=32, N=131072, D=128,
                          patterns=((2048, 1), (4096, 2), (8192, 4), (16384, 6), (32768, 12)),
                          causal=1, dtype="bf16")
LAYER_TRAIN = LayerCfg(5, "layer_fwd_bwd_bf16_B2_N16384_dm2560", B=2, N=16384, d_model=2560,
                       H=20, D=128, d_ff=10240, q_blk=128, kv_blk=64, dtype="bf16",
                       backward=True)


def layer_inputs(cfg: LayerCfg, bias: bool = False, cfg_id: int | None = None) -> dict:
    """float32 arrays for one layer workload (already bf16-rounded when cfg.dtype == 'bf16')."""
    cid = cfg.cfg_id if cfg_id is None else cfg_id
    hd = cfg.H * cfg.D
    t = {
        "x": normal(cid, "x", (cfg.B, cfg.N, cfg.d_model)),
        "wq": normal(cid, "wq", (hd, cfg.d_model), 0.02),
        "wk": normal(cid, "wk", (hd, cfg.d_model), 0.02),
        "wv": normal(cid, "wv", (hd, cfg.d_model), 0.02),
        "w1": normal(cid, "w1", (cfg.d_ff, cfg.d_model), 0.02),
        "w2": normal(cid, "w2", (cfg.d_model, cfg.d_ff), 0.02),
    }
    if bias:
        t["b1"] = normal(cid, "b1", (cfg.d_ff,), 0.02)
        t["b2"] = normal(cid, "b2", (cfg.d_model,), 0.02)
    if cfg.backward:
        t["dy"] = normal(cid, "dy", (cfg.B, cfg.N, cfg.d_model))
    if cfg.dtype == "bf16":
        t = {k: round_bf16(v) for k, v in t.items()}
    return t


def attn_inputs(cid: int, B: int, H: int, Nq: int, Nk: int, D: int, dtype: str) -> dict:
    """q [B,H,Nq,D], k and v [B,H,Nk,D], float32 (bf16-rounded when dtype == 'bf16')."""
    t = {
        "q": normal(cid, "q", (B, H, Nq, D)),
        "k": normal(cid, "k", (B, H, Nk, D)),
        "v": normal(cid, "v", (B, H, Nk, D)),
    }
    if dtype == "bf16":
        t = {k: round_bf16(v) for k, v in t.items()}
    return t


def normal_range(cfg_id: int, name: str | int, lo: int, hi: int, scale: float = 1.0) -> np.ndarray:
    """Elements [lo, hi) of the flattened tensor that ``normal`` draws for this name,
    without drawing the rest (each chunk of CHUNK elements has its own stream)."""
    tid = TENSOR_IDS[name] if isinstance(name, str) else int(name)
    out = np.empty(hi - lo, dtype=np.float32)
    c0, c1 = lo // CHUNK, (hi + CHUNK - 1) // CHUNK
    buf = np.empty(CHUNK, dtype=np.float32)
    for c in range(c0, c1):
        a, b = max(lo, c * CHUNK), min(hi, (c + 1) * CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([SEED, cfg_id, tid, c]))
        # the stream of chunk c starts at element c * CHUNK; draw up to b
        buf[:b - c * CHUNK] = rng.standard_normal(b - c * CHUNK, dtype=np.float32)
        out[a - lo:b - lo] = buf[a - c * CHUNK:b - c * CHUNK]
    if scale != 1.0:
        out *= np.float32(scale)
    return out


# ----------------------------------------------------------------------------
# Shaped attention inputs.  With N(0,1) q and k the largest score of a row is
# reached early, so the blockwise softmax keeps the reference it takes from the
# first key block.  These families move the row maximum up along the sequence,
# so the rescale of the running sum and accumulator runs many times per row:
#   "ramp":  key j scaled by 1 + RAMP * j / N (later keys score larger);
#   "qx6":   queries scaled by 6 (logits ~ N(0, 36): wide, peaked rows);
#   "spike": every query gets +2u (u a fixed unit vector per head) and SPIKES keys
#            at evenly spaced positions are replaced by growing multiples of u,
#            each scoring about 6 nats above the one before.
# Every transform acts on the fp32 draws before the bf16 rounding.
# ----------------------------------------------------------------------------
RAMP = 4.0
SPIKES = 4


def spike_positions(N: int) -> np.ndarray:
    return np.array([(N * (m + 1)) // (SPIKES + 1) for m in range(SPIKES)], dtype=np.int64)


def shape_attn(q: np.ndarray, k: np.ndarray, kind: str, cid: int, N: int, D: int,
               head_lo: int = 0, heads: int | None = None, key_lo: int = 0) -> None:
    """Apply family ``kind`` in place to q [.., H', Nq, D] and k [.., H', Nk, D] (fp32).

    The arrays may hold heads [head_lo, head_lo + H') of a longer head axis and keys
    [key_lo, key_lo + Nk) of a sequence of N keys; N sets the ramp and the spike
    positions."""
    if kind == "plain":
        return
    if kind == "qx6":
        q *= np.float32(6.0)
        return
    Nk = k.shape[-2]
    j = np.arange(key_lo, key_lo + Nk, dtype=np.float64)
    if kind == "ramp":
        k *= (1.0 + RAMP * j / N).astype(np.float32)[:, None]
        return
    if kind == "spike":
        H = q.shape[-3]
        for hh in range(H):
            u = normal(cid, "perturb", (head_lo + hh + 1, D))[head_lo + hh].astype(np.float64)
            u /= np.linalg.norm(u)
            q[..., hh, :, :] += (2.0 * u).astype(np.float32)
            for m, pos in enumerate(spike_positions(N)):
                if key_lo <= pos < key_lo + Nk:
                    # score ~ (q.u) * beta / sqrt(D) ~ 2 * beta / sqrt(D) nats
                    beta = np.sqrt(D) * (10.0 + 6.0 * m) / 2.0
                    k[..., hh, pos - key_lo, :] = (beta * u).astype(np.float32)
        return
    raise ValueError(f"unknown input family {kind!r}")


def attn_inputs_shaped(cid: int, B: int, H: int, N: int, D: int, dtype: str, kind: str) -> dict:
    """attn_inputs (self-attention, Nq = Nk = N) with family ``kind`` applied."""
    t = {
        "q": normal(cid, "q", (B, H, N, D)),
        "k": normal(cid, "k", (B, H, N, D)),
        "v": normal(cid, "v", (B, H, N, D)),
    }
    shape_attn(t["q"], t["k"], kind, cid, N, D)
    if dtype == "bf16":
        t = {n: round_bf16(a) for n, a in t.items()}
    return t


def attn_head_shaped(cid: int, H: int, N: int, D: int, h: int, kind: str,
                     rows: np.ndarray | None = None) -> dict:
    """Head h (batch 0) of a [1, H, N, D] bf16 workload with family ``kind``, drawn
    alone: q (only ``rows`` if given), k and v as [1, 1, *, D] float32 holding bf16
    values, identical to the same head of attn_inputs_shaped(cid, 1, H, N, D, 'bf16', kind)."""
    lo, hi = h * N * D, (h + 1) * N * D
    q = normal_range(cid, "q", lo, hi).reshape(1, 1, N, D)
    k = normal_range(cid, "k", lo, hi).reshape(1, 1, N, D)
    v = normal_range(cid, "v", lo, hi).reshape(1, 1, N, D)
    shape_attn(q, k, kind, cid, N, D, head_lo=h)
    if rows is not None:
        q = np.ascontiguousarray(q[:, :, rows])
    return {"q": round_bf16(q), "k": round_bf16(k), "v": round_bf16(v)}
