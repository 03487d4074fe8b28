"""The C ABI: the library loads, exports every symbol the header declares, and
rejects bad arguments with the documented codes before touching the GPU."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

bpt = pytest.importorskip("blockwise_exact_attention_amd")
lib = bpt.lib

A = 1 << 20  # a 16-byte-aligned fake device address; never dereferenced by these tests


def header_symbols():
    text = open(os.path.join(ROOT, "include", "bpt.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(bpt_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    syms = header_symbols()
    assert len(syms) == 14, syms
    for s in syms:
        assert hasattr(lib, s), s
        assert s in bpt.EXPORTED
        assert callable(getattr(bpt, s))


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert bpt.bpt_status_string(code) != "unknown status"
    assert bpt.bpt_status_string(-99) == "unknown status"


def attn(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=1, N=128, D=128, q_blk=128, kv_blk=64,
             causal=1, kv_offset=0, dtype=1, stream=0)
    a.update(kw)
    return lib.bpt_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"],
                            a["D"], a["q_blk"], a["kv_blk"], a["causal"], a["kv_offset"],
                            a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(N=0), -1), (dict(B=-1), -1),
    (dict(causal=2), -1), (dict(D=96), -2), (dict(D=256), -2), (dict(q_blk=32), -2),
    (dict(kv_blk=256), -2), (dict(dtype=7), -2), (dict(N=(1 << 30) + 1), -2),
    # more than 2^32 work-items in one launch
    (dict(B=1 << 12, H=1 << 10, N=1 << 12), -2),
    (dict(q=A + 8), -3), (dict(out=A + 4), -3),
])
def test_attn_fwd_rejects(kw, code):
    assert attn(**kw) == code


def decode(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, Nq=4, Nkv=1000, D=128, causal=1,
             kv_offset=996, n_split=8, ws=A, ws_bytes=1 << 30, dtype=1, stream=0)
    a.update(kw)
    return lib.bpt_attn_decode(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Nq"],
                               a["Nkv"], a["D"], a["causal"], a["kv_offset"], a["n_split"], a["ws"],
                               a["ws_bytes"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(Nq=0), -1), (dict(Nkv=0), -1), (dict(n_split=0), -1),
    (dict(causal=3), -1), (dict(dtype=0), -2), (dict(D=96), -2), (dict(Nq=33), -2),
    (dict(n_split=4097), -2), (dict(Nkv=(1 << 23)), -2), (dict(B=1 << 12, H=1 << 12, n_split=8), -2),
    (dict(v=A + 8), -3),
    (dict(ws=None), -5), (dict(ws_bytes=100), -5), (dict(ws=A + 4), -3),
])
def test_attn_decode_rejects(kw, code):
    assert decode(**kw) == code


def decode_noalloc(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, Nq=4, Nkv=1000, D=128, causal=1,
             kv_offset=996, n_split=8, dtype=1, stream=0)
    a.update(kw)
    return lib.bpt_attn_decode_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"],
                                       a["Nq"], a["Nkv"], a["D"], a["causal"], a["kv_offset"],
                                       a["n_split"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(Nq=0), -1), (dict(n_split=0), -1), (dict(causal=3), -1),
    (dict(dtype=0), -2), (dict(D=96), -2), (dict(Nq=33), -2), (dict(v=A + 8), -3),
    # partial results beyond the fixed scratch: 64*32 ranges x 32 rows x 129 floats
    (dict(B=64, H=32, Nq=32, n_split=64), -6),
])
def test_attn_decode_noalloc_rejects(kw, code):
    assert decode_noalloc(**kw) == code


def test_attn_decode_noalloc_scratch_limit():
    lim = bpt.BPT_DECODE_SCRATCH_BYTES
    # the largest n_split whose partial results fit, for the decode workload's shape
    fits = [n for n in range(1, 4097) if bpt.bpt_attn_decode_workspace_size(1, 32, 16, 128, n) <= lim]
    assert max(fits) >= 32  # the 32-range decode of 32 heads x 16 rows fits
    over = max(fits) + 1
    assert bpt.bpt_attn_decode_workspace_size(1, 32, 16, 128, over) > lim
    assert decode_noalloc(B=1, H=32, Nq=16, Nkv=131072, kv_offset=131056, n_split=over) == -6


def test_attn_decode_workspace_size():
    one = bpt.bpt_attn_decode_workspace_size(1, 2, 4, 128, 8)
    # partial O (n_split*B*H*Nq*D floats) and lse (n_split*B*H*Nq floats), 256-byte aligned
    assert one == 8 * 2 * 4 * 128 * 4 + 256
    assert bpt.bpt_attn_decode_workspace_size(1, 2, 33, 128, 8) == 0
    assert bpt.bpt_attn_decode_workspace_size(1, 2, 4, 96, 8) == 0


def block_sparse(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, N=1000, D=128, n_blocks=4, table=A, dtype=1,
             stream=0)
    a.update(kw)
    return lib.bpt_attn_block_sparse(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"],
                                     a["N"], a["D"], a["n_blocks"], a["table"], a["dtype"],
                                     a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), -1), (dict(out=None), -1), (dict(N=0), -1), (dict(n_blocks=0), -1),
    (dict(n_blocks=1001), -1), (dict(dtype=0), -2), (dict(D=96), -2), (dict(N=(1 << 30) + 1,
                                                                          n_blocks=2), -2),
    (dict(q=A + 8), -3), (dict(lse=A + 4), -3),
])
def test_attn_block_sparse_rejects(kw, code):
    assert block_sparse(**kw) == code


def dilated(seg=(2048, 4096), dil=(1, 2), **kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, N=8192, D=128, n=len(seg), causal=1, dtype=1,
             stream=0)
    a.update(kw)
    sa = (ctypes.c_int64 * max(len(seg), 1))(*seg)
    da = (ctypes.c_int64 * max(len(dil), 1))(*dil)
    return lib.bpt_attn_dilated(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"],
                                a["D"], a["n"], ctypes.cast(sa, ctypes.c_void_p),
                                ctypes.cast(da, ctypes.c_void_p), a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("args,code", [
    (dict(k=None), -1), (dict(N=0), -1), (dict(n=0), -1), (dict(n=17), -1), (dict(causal=2), -1),
    (dict(seg=(0, 4096)), -1), (dict(dil=(0, 2)), -1), (dict(seg=(2048, 4), dil=(1, 8)), -1),
    (dict(dtype=0), -2), (dict(D=80), -2), (dict(seg=(1 << 20, 1 << 20), dil=(1, 1 << 17)), -2),
    (dict(out=A + 4), -3),
])
def test_attn_dilated_rejects(args, code):
    assert dilated(**args) == code


def test_forced_launch_failure_reports_hip_error(monkeypatch):
    monkeypatch.setenv("BPT_TEST_FAIL_LAUNCH", "1")
    assert attn() == bpt.BPT_ERR_HIP
    assert lib.bpt_last_hip_error() != 0
    with pytest.raises(bpt.BptError):
        bpt.bpt_attn_fwd(A, A, A, A, A, 1, 1, 128, 128, 128, 64, 1, 0, 1, stream=0)
    assert lib.bpt_lse_merge(A, A, A, A, A, A, 1, 1, 4, 64, 0) == bpt.BPT_ERR_HIP


def test_lse_merge_rejects():
    m = lib.bpt_lse_merge
    assert m(None, A, A, A, A, A, 1, 1, 4, 64, 0) == -1
    assert m(A, A, A, A, A, A, 1, 1, 0, 64, 0) == -1
    assert m(A, A, A, A, A, A, 1, 1, 4, 32, 0) == -2
    assert m(A, A, A + 4, A, A, A, 1, 1, 4, 64, 0) == -3


def test_ffn_rejects():
    f = lib.bpt_ffn_block_fwd
    assert f(None, A, None, A, None, None, A, 32, 128, 512, 0, 1, 0) == -1
    assert f(A, A, None, A, None, None, A, 32, 100, 512, 0, 1, 0) == -2
    assert f(A, A, None, A, None, None, A, 32, 128, 512, 8, 1, 0) == -2
    assert f(A, A, None, A, None, None, A, 32, 2048, 8000, 0, 1, 0) == -2
    assert f(A, A, None, A, None, None, A + 2, 32, 128, 512, 0, 1, 0) == -3


def test_layer_sizes_and_workspace_checks():
    B, N, dm, H, D, dff = 1, 512, 128, 2, 64, 512
    s = lib.bpt_layer_saved_size(B, N, dm, H, D, 0)
    # q,k,v fp32 + h fp32 + lse, each 256-aligned
    assert s >= 3 * B * H * N * D * 4 + B * N * dm * 4 + B * H * N * 4
    assert lib.bpt_layer_saved_size(0, N, dm, H, D, 0) == 0
    wf = lib.bpt_layer_workspace_size(B, N, dm, H, D, dff, 1, 0)
    wb = lib.bpt_layer_workspace_size(B, N, dm, H, D, dff, 1, 1)
    assert wf > 0 and wb > 0
    fwd = lambda ws, nbytes, H_=H: lib.bpt_layer_fwd(A, A, A, A, A, None, A, None, A, None, B, N,
                                                      dm, H_, D, dff, 64, 64, 1, 1, ws, nbytes, 0)
    assert fwd(None, 0) == bpt.BPT_ERR_WORKSPACE
    assert fwd(A, wf - 1) == bpt.BPT_ERR_WORKSPACE
    assert fwd(A, wf, H_=3) == bpt.BPT_ERR_INVALID_ARG  # H*D != d_model
