"""CPU oracle for absorbed MLA (test infrastructure only).

Loads the plain C oracle (mla_oracle.c, float32 in/out, double accumulation)
through ctypes.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package; the GPU library never does, and this package never
imports the GPU library.

Every function takes and returns numpy arrays in the layouts documented in
mla_oracle.c.  The method follows the page "ik_llama.cpp MLA matrix absorption"
(czykbl.com/news/93068), sections 1, 3, 4 and 5; the Q8_0 format follows its
section 8.1 and the DeepSeek-V3 run of the KV-cache-rm page (trdm.cn/news/546512).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def build(force: bool = False) -> str:
    """Compile mla_oracle.c with gcc (OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i, d, f = ctypes.c_int, ctypes.c_double, ctypes.c_float
        L.orc_rope.argtypes = [_f32p, i, d, d, _f32p]
        L.orc_absorb_q.argtypes = [i, i, i, i, d, _f32p, _f32p, _i32p, _f32p, i, _f32p]
        L.orc_attention.argtypes = [i, i, i, d, _f32p, _i32p, i, _f32p, i, _f32p,
                                    ctypes.c_void_p]
        L.orc_out_proj.argtypes = [i, i, i, i, _f32p, _f32p, _f32p, i, ctypes.c_void_p, _f32p]
        L.orc_mla_unabsorbed.argtypes = [i, i, i, i, i, i, d, d, _f32p, _f32p, _i32p, i, _f32p,
                                         i, _f32p, _f32p, _f32p, ctypes.c_void_p, _f32p]
        L.orc_half_to_float.argtypes = [ctypes.c_uint16]
        L.orc_half_to_float.restype = f
        L.orc_float_to_half.argtypes = [f]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_q8_0_quantize.argtypes = [_f32p, ctypes.c_int64, i, _u8p]
        L.orc_q8_0_dequantize.argtypes = [_u8p, ctypes.c_int64, i, _f32p]
        L.orc_heads_per_chunk.argtypes = [i, d, i]
        L.orc_heads_per_chunk.restype = i
        L.orc_set_threads.argtypes = [i]
        L.orc_max_threads.restype = i
        _lib = L
    return _lib


def _c(a, dt=np.float32):
    return np.ascontiguousarray(a, dtype=dt)


def rope(x, pos, base=10000.0):
    """RoPE of one vector (adjacent pairs, angle pos * base^(-2i/dr))."""
    x = _c(x)
    y = np.empty_like(x)
    lib().orc_rope(x, x.shape[-1], float(pos), float(base), y)
    return y


def absorb_q(dims, q_nope, q_rope, pos, wk_b):
    """q_cat[t,h] = [wk_b[h] @ q_nope[t,h] | RoPE(q_rope[t,h], pos[t])]."""
    q_nope, q_rope, wk_b, pos = _c(q_nope), _c(q_rope), _c(wk_b), _c(pos, np.int32)
    T = q_nope.shape[0]
    H, R, Dn, Dr = dims.n_head, dims.kv_lora_rank, dims.qk_nope, dims.qk_rope
    q_cat = np.empty((T, H, R + Dr), dtype=np.float32)
    lib().orc_absorb_q(H, R, Dn, Dr, float(dims.rope_base), q_nope, q_rope, pos, wk_b, T, q_cat)
    return q_cat


def attention(dims, q_cat, pos, cache_rows):
    """Causal attention of q_cat [T,H,W] over cache rows [N,W]; returns (o_lat, lse)."""
    q_cat, pos, cache_rows = _c(q_cat), _c(pos, np.int32), _c(cache_rows)
    T, H, W = q_cat.shape
    R = dims.kv_lora_rank
    N = cache_rows.shape[0]
    o = np.empty((T, H, R), dtype=np.float32)
    lse = np.empty((T, H), dtype=np.float32)
    lib().orc_attention(H, R, dims.qk_rope, float(dims.scale), q_cat, pos, T, cache_rows, N, o,
                        lse.ctypes.data)
    return o, lse


def out_proj(dims, o_lat, wv_b, wo):
    """Returns (v [T, H*Dv], out [T, D]): v = wv_b . o_lat per head, out = wo . v."""
    o_lat, wv_b, wo = _c(o_lat), _c(wv_b), _c(wo)
    T = o_lat.shape[0]
    H, R, Dv, D = dims.n_head, dims.kv_lora_rank, dims.v_head, dims.d_model
    v = np.empty((T, H * Dv), dtype=np.float32)
    out = np.empty((T, D), dtype=np.float32)
    lib().orc_out_proj(H, R, Dv, D, o_lat, wv_b, wo, T, v.ctypes.data, out)
    return v, out


def mla_unabsorbed(dims, q_nope, q_rope, pos, cache_rows, wk_b, wv_b, wo):
    """Explicitly decompressed MLA (mode 0); returns (attn_v [T,H,Dv], out [T,D])."""
    q_nope, q_rope, pos = _c(q_nope), _c(q_rope), _c(pos, np.int32)
    cache_rows, wk_b, wv_b, wo = _c(cache_rows), _c(wk_b), _c(wv_b), _c(wo)
    T = q_nope.shape[0]
    H, R, Dn, Dr, Dv, D = (dims.n_head, dims.kv_lora_rank, dims.qk_nope, dims.qk_rope,
                           dims.v_head, dims.d_model)
    av = np.empty((T, H, Dv), dtype=np.float32)
    out = np.empty((T, D), dtype=np.float32)
    lib().orc_mla_unabsorbed(H, R, Dn, Dr, Dv, D, float(dims.scale), float(dims.rope_base),
                             q_nope, q_rope, pos, T, cache_rows, cache_rows.shape[0], wk_b, wv_b,
                             wo, av.ctypes.data, out)
    return av, out


def half_to_float(bits: int) -> float:
    return float(lib().orc_half_to_float(int(bits)))


def float_to_half(x: float) -> int:
    return int(lib().orc_float_to_half(float(x)))


def q8_0_row_bytes(width: int) -> int:
    return width // 32 * 34


def q8_0_quantize(x):
    """Quantise rows [..., width] (width % 32 == 0) to Q8_0 bytes [..., width/32*34]."""
    x = _c(x)
    width = x.shape[-1]
    assert width % 32 == 0
    n_rows = x.size // width
    out = np.empty(x.shape[:-1] + (q8_0_row_bytes(width),), dtype=np.uint8)
    lib().orc_q8_0_quantize(x, n_rows, width, out)
    return out


def q8_0_dequantize(b, width):
    b = _c(b, np.uint8)
    n_rows = b.size // q8_0_row_bytes(width)
    out = np.empty(b.shape[:-1] + (width,), dtype=np.float32)
    lib().orc_q8_0_dequantize(b, n_rows, width, out)
    return out


def bf16_round(x):
    """float32 -> nearest bfloat16 (ties to even), returned as float32 (NaN kept NaN)."""
    x = _c(x)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out).astype(np.float32)


def cache_rows_new(dims, c_kv, k_rope, pos):
    """The rows new tokens add to the latent cache: [c_kv[t] | RoPE(k_rope[t], pos[t])].

    Section 4 of the absorption page keeps, per token, the compressed latent and the
    rotated shared key side by side; the key is rotated at its own position once, when
    it enters the cache (the rule of the KV-cache page, section 2.3).  float32 [T, W]."""
    c_kv, k_rope, pos = _c(c_kv), _c(k_rope), _c(pos, np.int32)
    T = c_kv.shape[0]
    rows = np.empty((T, dims.kv_lora_rank + dims.qk_rope), dtype=np.float32)
    for t in range(T):
        rows[t, :dims.kv_lora_rank] = c_kv[t]
        rows[t, dims.kv_lora_rank:] = rope(k_rope[t], int(pos[t]), dims.rope_base)
    return rows


def cache_append(dims, kv, cache, c_kv, k_rope, pos, dst_row=None, hadamard=False):
    """Returns a copy of cache with the new rows stored at dst_row[t] (pos[t] if None).

    kv is "f32", "bf16" (cache float32 [N, W] holding bfloat16 values) or "q8_0" (cache
    uint8 [N, W/32*34]).  Destinations outside [0, N) are skipped.  hadamard: the latent
    part is rotated first (cache_rows_new_hadamard)."""
    rows = (cache_rows_new_hadamard if hadamard else cache_rows_new)(dims, c_kv, k_rope, pos)
    dst = np.asarray(pos if dst_row is None else dst_row, dtype=np.int64)
    out = np.array(cache, copy=True)
    if kv == "bf16":
        rows = bf16_round(rows)
    elif kv == "q8_0":
        rows = q8_0_quantize(rows)
    for t, r in enumerate(dst):
        if 0 <= r < out.shape[0]:
            out[r] = rows[t]
    return out


def hadamard(n: int) -> np.ndarray:
    """The normalised Walsh-Hadamard matrix of order n (a power of two), built by the
    doubling of the "llama.cpp KV cache" page, section 3.1: start from 1/sqrt(n) in the
    corner; each step copies the filled s x s block right and down and its negation to the
    lower right.  float64."""
    assert n > 0 and n & (n - 1) == 0
    h = np.zeros((n, n))
    h[0, 0] = 1.0 / np.sqrt(n)
    s = 1
    while s < n:
        blk = h[:s, :s].copy()
        h[s:2 * s, :s] = blk
        h[:s, s:2 * s] = blk
        h[s:2 * s, s:2 * s] = -blk
        s *= 2
    return h


def hadamard_weights(dims, wk_b, wv_b):
    """(H wk_b[h], wv_b[h] H) per head, float64 products rounded to float32."""
    h = hadamard(dims.kv_lora_rank)
    wk = np.einsum("lm,hmd->hld", h, np.asarray(wk_b, np.float64))
    wv = np.einsum("hdm,ml->hdl", np.asarray(wv_b, np.float64), h)
    return wk.astype(np.float32), wv.astype(np.float32)


def cache_rows_new_hadamard(dims, c_kv, k_rope, pos):
    """cache_rows_new with the latent part rotated: [H c_kv[t] | RoPE(k_rope[t], pos[t])]."""
    rows = cache_rows_new(dims, c_kv, k_rope, pos)
    h = hadamard(dims.kv_lora_rank)
    rows[:, :dims.kv_lora_rank] = (np.asarray(c_kv, np.float64) @ h.T).astype(np.float32)
    return rows


def wkv_b_merge(dims, wk_b, wv_b):
    """The merged attn_kv_b layout of the PR #394 page (section 2.1; rebuilt from the split
    pair as in its section 3.3): per head, the transposed wk_b ([Dn][R]) stacked over
    wv_b ([Dv][R]).  [H][Dn+Dv][R] float32."""
    wk_b = np.asarray(wk_b, np.float32)
    wv_b = np.asarray(wv_b, np.float32)
    return np.ascontiguousarray(np.concatenate([wk_b.transpose(0, 2, 1), wv_b], axis=1))


def wkv_b_split(dims, wkv_b):
    """Inverse of wkv_b_merge: (wk_b [H][R][Dn], wv_b [H][Dv][R])."""
    wkv_b = np.asarray(wkv_b, np.float32)
    Dn = dims.qk_nope
    return (np.ascontiguousarray(wkv_b[:, :Dn, :].transpose(0, 2, 1)),
            np.ascontiguousarray(wkv_b[:, Dn:, :]))


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's loops (timing only; results do not depend on it)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def heads_per_chunk(n_head: int, size_mib: float, cap_mib: int) -> int:
    return int(lib().orc_heads_per_chunk(int(n_head), float(size_mib), int(cap_mib)))


def mla_absorbed(dims, q_nope, q_rope, pos, cache_rows, wk_b, wv_b, wo):
    """The absorbed chain end to end; returns dict of q_cat, o_lat, lse, v, out."""
    q_cat = absorb_q(dims, q_nope, q_rope, pos, wk_b)
    o_lat, lse = attention(dims, q_cat, pos, cache_rows)
    v, out = out_proj(dims, o_lat, wv_b, wo)
    return {"q_cat": q_cat, "o_lat": o_lat, "lse": lse, "v": v, "out": out}
