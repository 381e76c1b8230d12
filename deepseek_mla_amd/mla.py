"""Thin Python binding of the C ABI in include/mla.h (argument marshalling only).

Every function has the C name and argument order; tensors are passed as device
pointers (torch tensors on the GPU, contiguous), `stream` defaults to torch's current
stream.  A non-zero status raises MLAError.  There is no fallback: if libmla.so is
missing the import of the library fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

F32, BF16, Q8_0 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4

# Every symbol include/mla.h declares.
EXPORTS = ("mla_absorb_q", "mla_attn_prefill", "mla_prefill_workspace_bytes",
           "mla_heads_per_chunk", "mla_decode_workspace_bytes",
           "mla_decode_auto_splits", "mla_attn_decode", "mla_attn_decode_static",
           "mla_cache_transpose_v", "mla_attn_decode_vt", "mla_out_proj",
           "mla_prefill_materialized",
           "mla_materialized_workspace_bytes", "mla_cache_append",
           "mla_cache_append_hadamard", "mla_hadamard_weights", "mla_wkv_b_merge",
           "mla_wkv_b_split",
           "mla_quantize_q8_0", "mla_dequant_q8_0", "mla_q8_0_row_bytes", "mla_status_str")


class MLAError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_str(status)}")


class mla_dims(ctypes.Structure):
    _fields_ = [("n_head", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope", ctypes.c_int32), ("qk_rope", ctypes.c_int32),
                ("v_head", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("scale", ctypes.c_float), ("rope_base", ctypes.c_float)]


def make_dims(d) -> mla_dims:
    """From any object with the mla_dims field names (e.g. synth.Dims)."""
    return mla_dims(d.n_head, d.kv_lora_rank, d.qk_nope, d.qk_rope, d.v_head, d.d_model,
                    float(d.scale), float(d.rope_base))


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run deepseek_mla_amd/build.py "
                              "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        D = ctypes.POINTER(mla_dims)
        sig = {
            "mla_absorb_q": ([D, ctypes.c_int, vp, vp, vp, vp, vp, i32, vp], ctypes.c_int),
            "mla_attn_prefill": ([D, ctypes.c_int, ctypes.c_int, vp, vp, i32, vp, i32, vp, vp,
                                  ctypes.c_uint32, vp, sz, vp], ctypes.c_int),
            "mla_prefill_workspace_bytes": ([D, ctypes.c_int, i32, i32, ctypes.c_uint32], sz),
            "mla_heads_per_chunk": ([i32, ctypes.c_double, ctypes.c_uint32], i32),
            "mla_decode_workspace_bytes": ([D, i32, i32, i32], sz),
            "mla_decode_auto_splits": ([D, ctypes.c_int, i32, i32], i32),
            "mla_attn_decode": ([D, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i32, i32, i32,
                                 vp, vp, vp, sz, vp], ctypes.c_int),
            "mla_attn_decode_static": ([D, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i32, i32,
                                        i32, vp, vp, vp], ctypes.c_int),
            "mla_cache_transpose_v": ([D, ctypes.c_int, vp, i64, i32, i32, i32, vp, i64, i32, vp],
                                      ctypes.c_int),
            "mla_attn_decode_vt": ([D, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i64, i32, vp,
                                    i32, i32, i32, vp, vp, vp, sz, vp], ctypes.c_int),
            "mla_out_proj": ([D, ctypes.c_int, vp, vp, vp, vp, vp, i32, vp], ctypes.c_int),
            "mla_prefill_materialized": ([D, ctypes.c_int, ctypes.c_int, vp, vp, vp, i32, vp, i32,
                                          vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, sz, vp],
                                         ctypes.c_int),
            "mla_materialized_workspace_bytes": ([D, i32, i32, ctypes.c_uint32], sz),
            "mla_cache_append_hadamard": ([D, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32, vp,
                                           i64, vp], ctypes.c_int),
            "mla_hadamard_weights": ([D, ctypes.c_int, vp, vp, vp, vp, vp], ctypes.c_int),
            "mla_wkv_b_merge": ([D, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp], ctypes.c_int),
            "mla_wkv_b_split": ([D, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp], ctypes.c_int),
            "mla_cache_append": ([D, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i32, vp, i64,
                                  vp], ctypes.c_int),
            "mla_quantize_q8_0": ([vp, vp, i64, i32, vp], ctypes.c_int),
            "mla_dequant_q8_0": ([vp, vp, i64, i32, vp], ctypes.c_int),
            "mla_q8_0_row_bytes": ([i32], i32),
            "mla_status_str": ([ctypes.c_int], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().mla_status_str(int(status)).decode()


def _p(t):
    """Device pointer of a tensor (None -> NULL).  Plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MLA library must be contiguous")
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str):
    if status != OK:
        raise MLAError(status, call)


def _d(dims):
    return ctypes.byref(dims if isinstance(dims, mla_dims) else make_dims(dims))


def mla_absorb_q(dims, act, q_nope, q_rope, pos, wk_b, q_cat, T, stream=None):
    _check(lib().mla_absorb_q(_d(dims), act, _p(q_nope), _p(q_rope), _p(pos), _p(wk_b), _p(q_cat),
                              T, _s(stream)), "mla_absorb_q")


def mla_prefill_workspace_bytes(dims, kv, T, n_kv, scratch_cap_mib=0):
    return lib().mla_prefill_workspace_bytes(_d(dims), kv, T, n_kv, scratch_cap_mib)


def prefill_workspace(dims, kv, T, n_kv, scratch_cap_mib=0, device="cuda"):
    """A workspace of the size mla_attn_prefill needs (None if it needs none)."""
    import torch
    n = mla_prefill_workspace_bytes(dims, kv, T, n_kv, scratch_cap_mib)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def mla_attn_prefill(dims, act, kv, q_cat, pos, T, kv_cache, n_kv, o_lat, lse=None,
                     scratch_cap_mib=0, workspace=None, stream=None):
    """workspace: a tensor from prefill_workspace() (allocated here when None)."""
    if workspace is None:
        workspace = prefill_workspace(dims, kv, T, n_kv, scratch_cap_mib, q_cat.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_attn_prefill(_d(dims), act, kv, _p(q_cat), _p(pos), T, _p(kv_cache), n_kv,
                                  _p(o_lat), _p(lse), scratch_cap_mib, _p(workspace), nbytes,
                                  _s(stream)),
           "mla_attn_prefill")


def mla_heads_per_chunk(n_head, size_mib, cap_mib):
    return lib().mla_heads_per_chunk(n_head, float(size_mib), cap_mib)


def mla_decode_workspace_bytes(dims, B, n_kv_max, n_splits=0):
    return lib().mla_decode_workspace_bytes(_d(dims), B, n_kv_max, n_splits)


def mla_decode_auto_splits(dims, kv, B, n_kv_max):
    return lib().mla_decode_auto_splits(_d(dims), kv, B, n_kv_max)


def mla_attn_decode(dims, act, kv, q_cat, kv_cache, kv_seq_stride_bytes, n_kv, B, n_kv_max,
                    n_splits, o_lat, lse, workspace, workspace_bytes, stream=None):
    _check(lib().mla_attn_decode(_d(dims), act, kv, _p(q_cat), _p(kv_cache), kv_seq_stride_bytes,
                                 _p(n_kv), B, n_kv_max, n_splits, _p(o_lat), _p(lse),
                                 _p(workspace), workspace_bytes, _s(stream)), "mla_attn_decode")


def mla_cache_transpose_v(dims, kv, kv_cache, kv_seq_stride_bytes, B, row0, row1, v_t,
                          vt_seq_stride_bytes, vt_ld, stream=None):
    _check(lib().mla_cache_transpose_v(_d(dims), kv, _p(kv_cache), kv_seq_stride_bytes, B, row0,
                                       row1, _p(v_t), vt_seq_stride_bytes, vt_ld, _s(stream)),
           "mla_cache_transpose_v")


def mla_attn_decode_vt(dims, act, kv, q_cat, kv_cache, kv_seq_stride_bytes, v_t,
                       vt_seq_stride_bytes, vt_ld, n_kv, B, n_kv_max, n_splits, o_lat, lse,
                       workspace, workspace_bytes, stream=None):
    _check(lib().mla_attn_decode_vt(_d(dims), act, kv, _p(q_cat), _p(kv_cache),
                                    kv_seq_stride_bytes, _p(v_t), vt_seq_stride_bytes, vt_ld,
                                    _p(n_kv), B, n_kv_max, n_splits, _p(o_lat), _p(lse),
                                    _p(workspace), workspace_bytes, _s(stream)),
           "mla_attn_decode_vt")


MLA_DECODE_STATIC_BYTES = 64 << 20  # include/mla.h


def mla_attn_decode_static(dims, act, kv, q_cat, kv_cache, kv_seq_stride_bytes, n_kv, B,
                           n_kv_max, n_splits, o_lat, lse, stream=None):
    _check(lib().mla_attn_decode_static(_d(dims), act, kv, _p(q_cat), _p(kv_cache),
                                        kv_seq_stride_bytes, _p(n_kv), B, n_kv_max, n_splits,
                                        _p(o_lat), _p(lse), _s(stream)), "mla_attn_decode_static")


def mla_out_proj(dims, act, o_lat, wv_b, wo, v_scratch, out, T, stream=None):
    _check(lib().mla_out_proj(_d(dims), act, _p(o_lat), _p(wv_b), _p(wo), _p(v_scratch), _p(out),
                              T, _s(stream)), "mla_out_proj")


def mla_materialized_workspace_bytes(dims, T, n_kv, scratch_cap_mib=0):
    return lib().mla_materialized_workspace_bytes(_d(dims), T, n_kv, scratch_cap_mib)


def materialized_workspace(dims, T, n_kv, scratch_cap_mib=0, device="cuda"):
    """A workspace of the size mla_prefill_materialized needs (256-byte aligned)."""
    import torch
    n = mla_materialized_workspace_bytes(dims, T, n_kv, scratch_cap_mib)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def mla_prefill_materialized(dims, act, kv, q_nope, q_rope, pos, T, kv_cache, n_kv, wk_b, wv_b,
                             v_out, wo=None, out=None, lse=None, scratch_cap_mib=0,
                             workspace=None, stream=None):
    """workspace: a tensor from materialized_workspace() (allocated here when None)."""
    if workspace is None:
        workspace = materialized_workspace(dims, T, n_kv, scratch_cap_mib, q_nope.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().mla_prefill_materialized(_d(dims), act, kv, _p(q_nope), _p(q_rope), _p(pos), T,
                                          _p(kv_cache), n_kv, _p(wk_b), _p(wv_b), _p(wo),
                                          _p(v_out), _p(out), _p(lse), scratch_cap_mib,
                                          _p(workspace), nbytes, _s(stream)),
           "mla_prefill_materialized")


def mla_cache_append(dims, act, kv, c_kv, k_rope, pos, T, cache, n_rows, dst_row=None,
                     stream=None):
    _check(lib().mla_cache_append(_d(dims), act, kv, _p(c_kv), _p(k_rope), _p(pos), _p(dst_row), T,
                                  _p(cache), n_rows, _s(stream)), "mla_cache_append")


def mla_cache_append_hadamard(dims, act, kv, c_kv, k_rope, pos, T, cache, n_rows, dst_row=None,
                              stream=None):
    _check(lib().mla_cache_append_hadamard(_d(dims), act, kv, _p(c_kv), _p(k_rope), _p(pos),
                                           _p(dst_row), T, _p(cache), n_rows, _s(stream)),
           "mla_cache_append_hadamard")


def mla_hadamard_weights(dims, act, wk_b, wv_b, wk_b_rot, wv_b_rot, stream=None):
    _check(lib().mla_hadamard_weights(_d(dims), act, _p(wk_b), _p(wv_b), _p(wk_b_rot),
                                      _p(wv_b_rot), _s(stream)), "mla_hadamard_weights")


def mla_wkv_b_merge(dims, act, out, wk_b, wv_b, wkv_b, stream=None):
    _check(lib().mla_wkv_b_merge(_d(dims), act, out, _p(wk_b), _p(wv_b), _p(wkv_b), _s(stream)),
           "mla_wkv_b_merge")


def mla_wkv_b_split(dims, inp, act, wkv_b, wk_b, wv_b, stream=None):
    _check(lib().mla_wkv_b_split(_d(dims), inp, act, _p(wkv_b), _p(wk_b), _p(wv_b), _s(stream)),
           "mla_wkv_b_split")


def mla_quantize_q8_0(x, rows, n_rows, width, stream=None):
    _check(lib().mla_quantize_q8_0(_p(x), _p(rows), n_rows, width, _s(stream)),
           "mla_quantize_q8_0")


def mla_dequant_q8_0(rows, out, n_rows, width, stream=None):
    _check(lib().mla_dequant_q8_0(_p(rows), _p(out), n_rows, width, _s(stream)),
           "mla_dequant_q8_0")


def mla_q8_0_row_bytes(width):
    return lib().mla_q8_0_row_bytes(width)
