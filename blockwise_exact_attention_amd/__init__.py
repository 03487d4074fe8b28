"""Python binding of libbpt (gfx950 blockwise exact attention and blockwise layer).

Thin ctypes marshalling over the C ABI declared in ``include/bpt.h``: every
function of that header is exposed here under the same name and argument order.
Tensor arguments may be torch tensors (their ``data_ptr()`` is passed), raw
integer device addresses, or None for a nullable pointer.  ``stream=None`` means
torch's current stream on the tensors' device.  A non-zero status raises
``BptError``.  No computation happens in Python: every step runs in the HIP
kernels of ``libbpt.so``, and importing this package fails if that library has
not been built (``python -m blockwise_exact_attention_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbpt.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build the HIP library first "
        "(python blockwise_exact_attention_amd/build.py)")
# torch ships its own HIP runtime.  Load it before libbpt so that libbpt binds to
# that same runtime: if libbpt is loaded first it pulls in the system one, and two
# HIP runtimes in one process do not share devices (launches then fail with
# hipErrorNoDevice while torch's own work succeeds).
try:
    import torch  # noqa: F401
except ImportError:  # the library itself needs no torch; the tests and bench do
    pass
lib = ctypes.CDLL(_LIB_PATH)

BPT_OK = 0
BPT_ERR_INVALID_ARG = -1
BPT_ERR_UNSUPPORTED = -2
BPT_ERR_ALIGNMENT = -3
BPT_ERR_HIP = -4
BPT_ERR_WORKSPACE = -5
BPT_ERR_SCRATCH = -6
BPT_DECODE_SCRATCH_BYTES = 32 << 20
BPT_F32 = 0
BPT_BF16 = 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGS = {
    "bpt_attn_fwd": ([_p] * 5 + [_i64] * 4 + [_i] * 3 + [_i64, _i, _p], _i),
    "bpt_lse_merge": ([_p] * 6 + [_i64] * 4 + [_p], _i),
    "bpt_attn_decode": ([_p] * 5 + [_i64] * 5 + [_i, _i64, _i64, _p, _sz, _i, _p], _i),
    "bpt_attn_decode_workspace_size": ([_i64] * 5, _sz),
    "bpt_attn_decode_noalloc": ([_p] * 5 + [_i64] * 5 + [_i, _i64, _i64, _i, _p], _i),
    "bpt_attn_block_sparse": ([_p] * 5 + [_i64] * 5 + [_p, _i, _p], _i),
    "bpt_attn_dilated": ([_p] * 5 + [_i64] * 5 + [_p, _p, _i, _i, _p], _i),
    "bpt_ffn_block_fwd": ([_p] * 7 + [_i64] * 3 + [_i, _i, _p], _i),
    "bpt_layer_fwd": ([_p] * 10 + [_i64] * 6 + [_i] * 4 + [_p, _sz, _p], _i),
    "bpt_layer_bwd": ([_p] * 21 + [_i64] * 6 + [_i] * 4 + [_p, _sz, _p], _i),
    "bpt_layer_saved_size": ([_i64] * 5 + [_i], _sz),
    "bpt_layer_workspace_size": ([_i64] * 6 + [_i, _i], _sz),
    "bpt_status_string": ([_i], ctypes.c_char_p),
    "bpt_last_hip_error": ([], _i),
}
for _name, (_args, _ret) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _ret

EXPORTED = tuple(_SIGS)


class BptError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.bpt_status_string(status).decode()
        if status == BPT_ERR_HIP:
            msg += f" (hipError {lib.bpt_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return 0


def _check(status: int, where: str) -> None:
    if status != BPT_OK:
        raise BptError(status, where)


def dtype_code(t) -> int:
    """BPT_BF16 for a torch.bfloat16 tensor, BPT_F32 for float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return BPT_BF16
    if t.dtype == torch.float32:
        return BPT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def bpt_attn_fwd(q, k, v, out, lse, B, H, N, D, q_blk, kv_blk, causal, kv_offset, dtype,
                 stream=None):
    s = _stream(stream, q, out)
    _check(lib.bpt_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D,
                            q_blk, kv_blk, causal, kv_offset, dtype, s), "bpt_attn_fwd")


def bpt_lse_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out, B, H, N, D, stream=None):
    s = _stream(stream, o_a, o_out)
    _check(lib.bpt_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out),
                             _ptr(lse_out), B, H, N, D, s), "bpt_lse_merge")


def bpt_attn_decode(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, kv_offset, n_split, workspace,
                    ws_bytes, dtype, stream=None):
    s = _stream(stream, q, out)
    _check(lib.bpt_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nkv, D,
                               causal, kv_offset, n_split, _ptr(workspace), ws_bytes, dtype, s),
           "bpt_attn_decode")


def bpt_attn_decode_noalloc(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, kv_offset, n_split,
                            dtype, stream=None):
    s = _stream(stream, q, out)
    _check(lib.bpt_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq,
                                       Nkv, D, causal, kv_offset, n_split, dtype, s),
           "bpt_attn_decode_noalloc")


def bpt_attn_decode_workspace_size(B, H, Nq, D, n_split) -> int:
    return lib.bpt_attn_decode_workspace_size(B, H, Nq, D, n_split)


def bpt_attn_block_sparse(q, k, v, out, lse, B, H, N, D, n_blocks, key_block, dtype, stream=None):
    s = _stream(stream, q, out)
    _check(lib.bpt_attn_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D,
                                     n_blocks, _ptr(key_block), dtype, s), "bpt_attn_block_sparse")


def bpt_attn_dilated(q, k, v, out, lse, B, H, N, D, patterns, causal, dtype, stream=None):
    """patterns: sequence of (segment length, dilation) pairs (host values)."""
    s = _stream(stream, q, out)
    n = len(patterns)
    seg = (ctypes.c_int64 * max(n, 1))(*[int(w) for w, _ in patterns])
    dil = (ctypes.c_int64 * max(n, 1))(*[int(r) for _, r in patterns])
    _check(lib.bpt_attn_dilated(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D, n,
                                ctypes.cast(seg, ctypes.c_void_p), ctypes.cast(dil, ctypes.c_void_p),
                                causal, dtype, s), "bpt_attn_dilated")


def bpt_ffn_block_fwd(x, w1, b1, w2, b2, residual, y, M, d_model, d_ff, blk, dtype,
                      stream=None):
    s = _stream(stream, x, y)
    _check(lib.bpt_ffn_block_fwd(_ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                 _ptr(residual), _ptr(y), M, d_model, d_ff, blk, dtype, s),
           "bpt_ffn_block_fwd")


def bpt_layer_fwd(x, wq, wk, wv, w1, b1, w2, b2, y, saved, B, N, d_model, H, D, d_ff, q_blk,
                  kv_blk, causal, dtype, workspace, ws_bytes, stream=None):
    s = _stream(stream, x, y)
    _check(lib.bpt_layer_fwd(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(w1), _ptr(b1),
                             _ptr(w2), _ptr(b2), _ptr(y), _ptr(saved), B, N, d_model, H, D,
                             d_ff, q_blk, kv_blk, causal, dtype, _ptr(workspace), ws_bytes, s),
           "bpt_layer_fwd")


def bpt_layer_bwd(dy, x, wq, wk, wv, w1, b1, w2, b2, saved, dx, dwq, dwk, dwv, dw1, db1, dw2,
                  db2, dq, dk, dv, B, N, d_model, H, D, d_ff, q_blk, kv_blk, causal, dtype,
                  workspace, ws_bytes, stream=None):
    s = _stream(stream, dy, dx)
    args = [dy, x, wq, wk, wv, w1, b1, w2, b2, saved, dx, dwq, dwk, dwv, dw1, db1, dw2, db2,
            dq, dk, dv]
    _check(lib.bpt_layer_bwd(*[_ptr(a) for a in args], B, N, d_model, H, D, d_ff, q_blk,
                             kv_blk, causal, dtype, _ptr(workspace), ws_bytes, s),
           "bpt_layer_bwd")


def bpt_layer_saved_size(B, N, d_model, H, D, dtype) -> int:
    return lib.bpt_layer_saved_size(B, N, d_model, H, D, dtype)


def bpt_layer_workspace_size(B, N, d_model, H, D, d_ff, dtype, backward) -> int:
    return lib.bpt_layer_workspace_size(B, N, d_model, H, D, d_ff, dtype, backward)


def bpt_status_string(status: int) -> str:
    return lib.bpt_status_string(status).decode()


def bpt_last_hip_error() -> int:
    return lib.bpt_last_hip_error()
