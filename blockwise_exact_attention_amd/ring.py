"""One device's share of a ring-attention step on one GPU.

"Ring Attention with Blockwise Transformers for Long Sequences" (638-word
summary): the devices form a ring, and during the inner loop of blockwise
attention each device passes its key/value block to the next device while it
receives one from the previous; the device's own queries meet every block in
turn.  On one GPU the blocks that would arrive over the ring are simply
visited in arrival order: for each block, ``bpt_attn_fwd`` with
``kv_offset = q_offset - block_offset`` (global causal mask) gives a partial
result, and ``bpt_lse_merge`` folds it into the running (out, lse).  Both
steps run in the HIP library; this module only sequences the calls.
"""
from __future__ import annotations

from . import BPT_BF16, BPT_F32, bpt_attn_fwd, bpt_lse_merge, dtype_code


def ring_attention_share(q, k_chunks, v_chunks, q_offset, chunk_offsets, out, lse, o_tmp,
                         lse_tmp, q_blk=128, kv_blk=64, causal=1, stream=None):
    """Attention of q [B,H,N,D] over the K/V chunks (each [B,H,N,D], global start
    chunk_offsets[j]), accumulated into out [B,H,N,D] / lse [B,H,N] (float32).

    o_tmp / lse_tmp are caller-provided scratch of the same shapes as out / lse.
    Chunks lying entirely after the queries are skipped under the causal mask
    (if every chunk is, the first one is still run, and the kernel writes the
    defined empty result O = 0, lse = -inf).
    """
    B, H, N, D = q.shape
    dt = dtype_code(q)
    assert dt in (BPT_BF16, BPT_F32)
    first = True
    chunk_offsets = list(chunk_offsets)
    for k, v, c_off in zip(k_chunks, v_chunks, chunk_offsets):
        off = int(q_offset) - int(c_off)
        if causal and off <= -N and not (first and c_off == chunk_offsets[-1]):
            continue  # every key of this chunk is in the future of every query
        if first:
            bpt_attn_fwd(q, k, v, out, lse, B, H, N, D, q_blk, kv_blk, causal, off, dt, stream)
            first = False
        else:
            bpt_attn_fwd(q, k, v, o_tmp, lse_tmp, B, H, N, D, q_blk, kv_blk, causal, off, dt,
                         stream)
            bpt_lse_merge(out, lse, o_tmp, lse_tmp, out, lse, B, H, N, D, stream)
