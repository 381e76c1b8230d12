"""The C-ABI library without a GPU: it loads, exports every symbol include/mla.h declares,
and rejects invalid arguments with status codes before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from deepseek_mla_amd import mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text))


def test_exports_match_header():
    declared = header_functions()
    assert declared == set(mla.EXPORTS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", mla.LIB_PATH]).decode()
    exported = set(re.findall(r" T (mla_[a-z0-9_]+)$", out, flags=re.M))
    assert declared <= exported
    L = mla.lib()
    for name in declared:
        assert getattr(L, name) is not None


def tiny():
    return mla.mla_dims(4, 64, 32, 16, 32, 128, 0.144, 10000.0)


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert mla.status_str(s).startswith("MLA_")
    assert "unknown" in mla.status_str(7)


def test_invalid_arguments_rejected_without_gpu():
    L = mla.lib()
    d = tiny()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    bad = mla.mla_dims(4, 64, 32, 15, 32, 128, 0.1, 10000.0)  # odd rope dim
    assert L.mla_absorb_q(None, 0, p, p, p, p, p, 4, None) == mla.ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(bad), 0, p, p, p, p, p, 4, None) == mla.ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(d), 0, None, p, p, p, p, 4, None) == mla.ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(d), 2, p, p, p, p, p, 4, None) == mla.ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(d), 0, p, p, p, p, p, -1, None) == mla.ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(d), 0, None, None, None, None, None, 0, None) == mla.OK
    # prefill: Q8_0 cache unsupported, bf16 needs the 512/64 latent row, dtype mix invalid
    assert L.mla_attn_prefill(ctypes.byref(d), 1, 2, p, p, 4, p, 8, p, None, 0, None, 0, None) == \
        mla.ERR_UNSUPPORTED
    assert L.mla_attn_prefill(ctypes.byref(d), 1, 1, p, p, 4, p, 8, p, None, 0, None, 0, None) == \
        mla.ERR_UNSUPPORTED
    assert L.mla_attn_prefill(ctypes.byref(d), 0, 1, p, p, 4, p, 8, p, None, 0, None, 0, None) == \
        mla.ERR_INVALID_ARG
    assert L.mla_attn_prefill(ctypes.byref(d), 0, 0, p, p, 4, p, 0, p, None, 0, None, 0, None) == \
        mla.ERR_INVALID_ARG
    # decode: workspace too small; Q8_0 needs a width multiple of 32 (tiny rows are 80 wide)
    ws = mla.mla_decode_workspace_bytes(d, 2, 100, 3)
    assert ws > 0
    assert L.mla_attn_decode(ctypes.byref(d), 0, 0, p, p, 80 * 4 * 100, p, 2, 100, 3, p, None,
                             p, ws - 1, None) == mla.ERR_WORKSPACE
    assert L.mla_attn_decode(ctypes.byref(d), 1, 2, p, p, 4000, p, 2, 100, 3, p, None, p, ws,
                             None) == mla.ERR_INVALID_ARG
    assert L.mla_attn_decode(ctypes.byref(d), 0, 0, p, p, 16, p, 2, 100, 3, p, None, p, ws,
                             None) == mla.ERR_INVALID_ARG  # stride shorter than a sequence
    assert L.mla_out_proj(ctypes.byref(d), 0, p, p, p, None, p, 3, None) == mla.ERR_INVALID_ARG
    assert L.mla_quantize_q8_0(p, p, 3, 80, None) == mla.ERR_INVALID_ARG
    assert L.mla_dequant_q8_0(p, p, 3, 0, None) == mla.ERR_INVALID_ARG


def test_host_helpers():
    assert mla.mla_q8_0_row_bytes(576) == 612
    assert mla.mla_q8_0_row_bytes(80) == -1
    assert mla.mla_heads_per_chunk(128, 131072.0, 8192) == 8
    assert mla.mla_heads_per_chunk(128, 4096.0, 256) == 8
    assert mla.mla_heads_per_chunk(128, 4096.0, 100) == 4
    assert mla.mla_heads_per_chunk(128, 4096.0, 0) == 128
    assert mla.mla_heads_per_chunk(7, 1000.0, 128) == 1
    v3 = mla.mla_dims(128, 512, 128, 64, 128, 7168, 0.0722, 10000.0)
    s = mla.mla_decode_auto_splits(v3, mla.BF16, 1, 32768)
    assert s >= 1
    assert mla.mla_decode_workspace_bytes(v3, 1, 32768, s) >= s * 128 * 513 * 4


def test_auto_split_counts_fill_the_cus_once():
    """The automatic split counts of the two V3 decodes give one workgroup per CU (256 CUs):
    bf16 at one sequence runs two 64-head groups per split, Q8_0 one 128-head workgroup per
    (sequence, split).  A split-count sweep on MI355X measured these counts fastest (more
    workgroups than CUs add a second round; fewer lengthen every workgroup's key range)."""
    v3 = mla.mla_dims(128, 512, 128, 64, 128, 7168, 0.0722, 10000.0)
    assert mla.mla_decode_auto_splits(v3, mla.BF16, 1, 32768) == 128
    assert mla.mla_decode_auto_splits(v3, mla.Q8_0, 4, 98304) == 64
    # short caches: never more splits than 32-row tiles allow work for
    s = mla.mla_decode_auto_splits(v3, mla.BF16, 1, 100)
    assert 1 <= s <= 100


def test_new_entry_points_validate_without_gpu():
    """Cache append, the materialised prefill, the Hadamard rotation and the wkv_b layout
    reject bad arguments before any launch (pointers are never dereferenced)."""
    L = mla.lib()
    d = tiny()  # R 64, Dr 16: W 80 (not a multiple of 32)
    p = ctypes.c_void_p(16)
    D = ctypes.byref(d)
    # cache append: Q8_0 needs W % 32 == 0; act/kv mix; T < 0; nulls; T == 0 is a no-op
    assert L.mla_cache_append(D, 0, 2, p, p, p, None, 3, p, 10, None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_append(D, 0, 1, p, p, p, None, 3, p, 10, None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_append(D, 0, 0, p, p, p, None, -1, p, 10, None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_append(D, 0, 0, None, p, p, None, 3, p, 10, None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_append(D, 0, 0, None, None, None, None, 0, None, 10, None) == mla.OK
    # Hadamard: R must be a power of two; outputs must not alias inputs
    r48 = mla.mla_dims(4, 48, 32, 16, 32, 128, 0.1, 10000.0)
    assert L.mla_cache_append_hadamard(ctypes.byref(r48), 0, 0, p, p, p, None, 3, p, 10,
                                       None) == mla.ERR_INVALID_ARG
    assert L.mla_hadamard_weights(ctypes.byref(r48), 0, p, p, ctypes.c_void_p(32),
                                  ctypes.c_void_p(48), None) == mla.ERR_INVALID_ARG
    assert L.mla_hadamard_weights(D, 0, p, ctypes.c_void_p(32), p, ctypes.c_void_p(48),
                                  None) == mla.ERR_INVALID_ARG
    # wkv_b layout: the merged type is act or Q8_0 (then R % 32 == 0)
    assert L.mla_wkv_b_merge(D, 0, 1, p, p, p, None) == mla.ERR_INVALID_ARG
    assert L.mla_wkv_b_merge(ctypes.byref(r48), 0, 2, p, p, p, None) == mla.ERR_INVALID_ARG
    assert L.mla_wkv_b_split(D, 1, 0, p, p, p, None) == mla.ERR_INVALID_ARG
    assert L.mla_wkv_b_split(D, 0, 0, p, None, p, None) == mla.ERR_INVALID_ARG
    # materialised prefill: bf16 DeepSeek head shape only; workspace checked
    v3 = mla.mla_dims(128, 512, 128, 64, 128, 7168, 0.0722, 10000.0)
    V = ctypes.byref(v3)
    args = lambda act, kv, ws, nb: (act, kv, p, p, p, 64, p, 256, p, p, None, p, None, None, 0,
                                    ws, nb, None)
    assert L.mla_prefill_materialized(D, *args(1, 1, p, 1 << 30)) == mla.ERR_UNSUPPORTED
    assert L.mla_prefill_materialized(V, *args(0, 0, p, 1 << 30)) == mla.ERR_UNSUPPORTED
    assert L.mla_prefill_materialized(V, *args(1, 2, p, 1 << 30)) == mla.ERR_UNSUPPORTED
    need = mla.mla_materialized_workspace_bytes(v3, 64, 256, 0)
    assert need > 0 and mla.mla_materialized_workspace_bytes(d, 64, 256, 0) == 0
    assert L.mla_prefill_materialized(V, *args(1, 1, ctypes.c_void_p(256), need - 1)) == \
        mla.ERR_WORKSPACE
    assert L.mla_prefill_materialized(V, *args(1, 1, ctypes.c_void_p(272), need)) == \
        mla.ERR_WORKSPACE  # not 256-byte aligned
    # wo and out come together
    a = list(args(1, 1, ctypes.c_void_p(256), need))
    a[10] = p  # wo given, out missing
    assert L.mla_prefill_materialized(V, *a) == mla.ERR_INVALID_ARG


def test_static_decode_validates_without_gpu():
    """The allocation-free decode rejects a call whose partials exceed its device array
    (and invalid arguments) before touching the GPU."""
    L = mla.lib()
    v3 = mla.mla_dims(128, 512, 128, 64, 128, 7168, 0.0722, 10000.0)
    V = ctypes.byref(v3)
    p = ctypes.c_void_p(16)
    # 64 sequences x 98304 rows, 10 splits each: 64 * 10 * 128 partial rows of 1 KB > 64 MiB
    assert L.mla_attn_decode_static(V, 1, 1, p, p, 98304 * 1152, p, 64, 98304, 10, p, None,
                                    None) == mla.ERR_WORKSPACE
    assert L.mla_attn_decode_static(None, 1, 1, p, p, 1152, p, 1, 1, 0, p, None,
                                    None) == mla.ERR_INVALID_ARG
    assert L.mla_attn_decode_static(V, 1, 1, None, p, 1152, p, 1, 1, 0, p, None,
                                    None) == mla.ERR_INVALID_ARG
    assert L.mla_attn_decode_static(V, 1, 1, None, None, 0, None, 0, 1, 0, None, None,
                                    None) == mla.OK
    assert mla.MLA_DECODE_STATIC_BYTES == 64 << 20


def test_vt_entry_points_validate_without_gpu():
    """The K + V^T cache entry points reject bad arguments before any launch."""
    L = mla.lib()
    v3 = mla.mla_dims(128, 512, 128, 64, 128, 7168, 0.0722, 10000.0)
    V = ctypes.byref(v3)
    D = ctypes.byref(tiny())
    p = ctypes.c_void_p(16)
    # transpose: bf16 and R 512 / Dr 64 only; vt_ld covers row1 rounded up to 32
    assert L.mla_cache_transpose_v(V, 1, p, 1152 * 100, 2, 0, 100, p, 512 * 64 * 2, 128,
                                   None) == mla.ERR_INVALID_ARG  # V^T rows overlap
    assert L.mla_cache_transpose_v(V, 1, p, 1152 * 99, 2, 0, 100, p, 512 * 128 * 2, 128,
                                   None) == mla.ERR_INVALID_ARG  # cache rows overlap
    assert L.mla_cache_transpose_v(V, 1, p, 1152 * 100, 1, 0, 100, p, 0, 96,
                                   None) == mla.ERR_INVALID_ARG  # vt_ld < 128
    assert L.mla_cache_transpose_v(V, 2, p, 612 * 100, 1, 0, 100, p, 0, 128,
                                   None) == mla.ERR_UNSUPPORTED
    assert L.mla_cache_transpose_v(D, 1, p, 160 * 100, 1, 0, 100, p, 0, 128,
                                   None) == mla.ERR_UNSUPPORTED
    assert L.mla_cache_transpose_v(V, 1, p, 1152, 1, 5, 4, p, 0, 128, None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_transpose_v(V, 1, p, 1152, 1, 0, 1, p, 0, (1 << 26) + 8,
                                   None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_transpose_v(V, 1, None, 1152, 1, 0, 1, p, 0, 32,
                                   None) == mla.ERR_INVALID_ARG
    assert L.mla_cache_transpose_v(V, 1, None, 0, 1, 7, 7, None, 0, 32, None) == mla.OK
    # decode: dtypes, vt_ld (multiple of 8, >= n_kv_max rounded up to 32), strides, workspace
    def dec(act=1, kv=1, kvs=1152 * 100, vts=512 * 128 * 2, ld=128, B=1, nmax=100, ws=p,
            wsb=1 << 30, dims=V, vt=p):
        return L.mla_attn_decode_vt(dims, act, kv, p, p, kvs, vt, vts, ld, p, B, nmax, 0, p,
                                    None, ws, wsb, None)
    assert dec(kv=2) == mla.ERR_UNSUPPORTED
    assert dec(act=0, kv=0) == mla.ERR_UNSUPPORTED
    assert dec(act=3) == mla.ERR_INVALID_ARG
    assert dec(dims=D) == mla.ERR_UNSUPPORTED
    assert dec(ld=96) == mla.ERR_INVALID_ARG
    assert dec(ld=132) == mla.ERR_INVALID_ARG
    assert dec(kvs=1152 * 100 + 8) == mla.ERR_INVALID_ARG
    assert dec(B=2, vts=512 * 64 * 2) == mla.ERR_INVALID_ARG
    assert dec(vt=ctypes.c_void_p(24)) == mla.ERR_INVALID_ARG
    assert dec(ws=None) == mla.ERR_INVALID_ARG
    need = mla.mla_decode_workspace_bytes(v3, 1, 100, 0)
    assert dec(wsb=need - 1) == mla.ERR_WORKSPACE
    assert L.mla_attn_decode_vt(V, 1, 1, None, None, 0, None, 0, 32, None, 0, 1, 0, None, None,
                                None, 0, None) == mla.OK
