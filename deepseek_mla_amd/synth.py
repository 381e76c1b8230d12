"""Seeded synthetic inputs for absorbed Multi-head Latent Attention.

This module only draws and formats inputs; it computes nothing of the attention
method itself.  Both the GPU path (bench, tests) and the CPU oracle's tests take
their inputs from here, so the two sides always see identical values.

Shapes follow the DeepSeek dimensions the pages describe (DeepSeek-V3 hparams in
"ik_llama.cpp PR #394" section 2.1: kv_lora_rank 512, rope 64, nope 128, V 128,
128 heads; DeepSeek-Lite: 16 heads, d_model 2048).  No weights or datasets exist
here: every tensor is a seeded normal draw.

Distributions (readings stated where the pages are silent):
  * latents c_kv, k_rope ~ N(0, 1); k_rope is taken as already rotated, i.e. the
    cached key part is post-RoPE (the llama.cpp KV-cache page, section 2.3,
    re-ropes cached keys on a shift, so the cache holds rotated keys).
  * queries q_nope, q_rope ~ N(0, 1).
  * weights ~ N(0, 1/fan_in): wk_b and wv_b up-project c_kv, fan_in = kv_lora_rank;
    wo takes the concatenated heads, fan_in = n_head * v_head.
  * draw order: q_nope, q_rope, c_kv, k_rope, wk_b, wv_b, wo, each as float64
    standard normals from numpy's PCG64, scaled, then cast to float32.
  * bf16 / Q8_0 modes: values are rounded to bf16 (round to nearest even) before
    either side sees them; the Q8_0 cache is quantised from the float32 latents.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Dims:
    n_head: int
    kv_lora_rank: int
    qk_nope: int
    qk_rope: int
    v_head: int
    d_model: int
    scale: float
    rope_base: float = 10000.0

    @property
    def row(self) -> int:
        """Width of one latent cache row: [c_kv | k_rope]."""
        return self.kv_lora_rank + self.qk_rope


def deepseek_dims(n_head: int, d_model: int) -> Dims:
    return Dims(n_head=n_head, kv_lora_rank=512, qk_nope=128, qk_rope=64, v_head=128,
                d_model=d_model, scale=1.0 / math.sqrt(128 + 64))


TINY = Dims(n_head=4, kv_lora_rank=64, qk_nope=32, qk_rope=16, v_head=32, d_model=128,
            scale=1.0 / math.sqrt(32 + 16))
LITE = deepseek_dims(16, 2048)
V3 = deepseek_dims(128, 7168)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    kind "prefill": T query tokens at positions pos0 .. pos0+T-1, causal over a
    single cache of n_kv rows.  kind "decode": n_seq sequences, each with its
    own cache of n_kv rows and one new query token at position n_kv-1.
    mode: "f32", "bf16" or "q8_0" (bf16 activations, Q8_0 cache).
    """
    name: str
    dims: Dims
    mode: str
    kind: str
    n_kv: int
    seed: int
    T: int = 1
    pos0: int = 0
    n_seq: int = 1
    scratch_cap_mib: int = 0

    @property
    def n_query(self) -> int:
        return self.T if self.kind == "prefill" else self.n_seq


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", TINY, "f32", "prefill", n_kv=64, seed=1, T=16, pos0=48),
    "lite_prefill": Workload("lite_prefill", LITE, "bf16", "prefill", n_kv=2048, seed=2, T=2048,
                             pos0=0),
    "v3_decode": Workload("v3_decode", V3, "bf16", "decode", n_kv=32768, seed=3, n_seq=1),
    "v3_long_prefill": Workload("v3_long_prefill", V3, "bf16", "prefill", n_kv=32768, seed=4,
                                T=8192, pos0=24576, scratch_cap_mib=8192),
    "v3_decode_q8": Workload("v3_decode_q8", V3, "q8_0", "decode", n_kv=98304, seed=5, n_seq=4),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, scale: float = 1.0, chunk: int = 1 << 24):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s)
        if scale != 1.0:
            v *= scale
        out[s:e] = v
    return out.reshape(shape)


def generate(dims: Dims, T: int, n_kv: int, seed: int, n_seq: int | None = None,
             mode: str = "f32", pos=None) -> dict:
    """Draw one layer's inputs.

    Returns float32 arrays (already bf16-rounded in bf16/q8_0 modes):
      q_nope [Q, H, Dn], q_rope [Q, H, Dr] (pre-RoPE), pos [Q] int32,
      c_kv [S, N, R], k_rope [S, N, Dr] (S = n_seq, or 1 for prefill),
      wk_b [H, R, Dn], wv_b [H, Dv, R], wo [D, H*Dv].
    For decode (n_seq given) Q = n_seq and pos[b] = n_kv - 1.
    """
    H, R, Dn, Dr, Dv, D = (dims.n_head, dims.kv_lora_rank, dims.qk_nope, dims.qk_rope,
                           dims.v_head, dims.d_model)
    rng = np.random.Generator(np.random.PCG64(seed))
    S = 1 if n_seq is None else n_seq
    Q = T if n_seq is None else n_seq
    out = {
        "q_nope": _normal(rng, (Q, H, Dn)),
        "q_rope": _normal(rng, (Q, H, Dr)),
        "c_kv": _normal(rng, (S, n_kv, R)),
        "k_rope": _normal(rng, (S, n_kv, Dr)),
        "wk_b": _normal(rng, (H, R, Dn), 1.0 / math.sqrt(R)),
        "wv_b": _normal(rng, (H, Dv, R), 1.0 / math.sqrt(R)),
        "wo": _normal(rng, (D, H * Dv), 1.0 / math.sqrt(H * Dv)),
    }
    if pos is None:
        pos = np.full(Q, n_kv - 1, dtype=np.int32) if n_seq is not None else \
            np.arange(n_kv - T, n_kv, dtype=np.int32)
    out["pos"] = np.ascontiguousarray(pos, dtype=np.int32)
    if mode in ("bf16", "q8_0"):
        for k in ("q_nope", "q_rope", "c_kv", "k_rope", "wk_b", "wv_b", "wo"):
            out[k] = round_bf16(out[k])
    return out


def generate_workload(w: Workload) -> dict:
    pos = None
    if w.kind == "prefill":
        pos = np.arange(w.pos0, w.pos0 + w.T, dtype=np.int32)
    return generate(w.dims, w.T, w.n_kv, w.seed,
                    n_seq=(w.n_seq if w.kind == "decode" else None), mode=w.mode, pos=pos)


def sample_tokens(T: int, k: int, seed: int) -> np.ndarray:
    """Sorted indices of k seeded draws from range(T) (without replacement) together with
    the first and the last token."""
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(k, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


def long_prefill_sample(T: int = 8192) -> np.ndarray:
    """The 64 query tokens of the long prefill that the CPU oracle computes (parity tests
    and the CPU baseline): 62 seeded draws plus the first and the last token."""
    sel = sample_tokens(T, 62, 62)
    assert len(sel) == 64 and sel[0] == 0 and sel[-1] == T - 1
    return sel


def cache_rows(c_kv: np.ndarray, k_rope: np.ndarray) -> np.ndarray:
    """Lay out latent cache rows [c_kv | k_rope] along the last axis (float32)."""
    return np.ascontiguousarray(np.concatenate([c_kv, k_rope], axis=-1), dtype=np.float32)
