"""Algorithmic FLOP and byte counts for absorbed MLA.

These are the closed forms behind the per-token comparison table of the page
"ik_llama.cpp MLA matrix absorption" (czykbl.com/news/93068), section 7, which
prints 81.92 KB / 1.15 KB cache per token and 0.08 M / 33.64 M / 0.28 M FLOP per
token for the decompressed, compressed-without-absorption and absorbed paths at
DeepSeek-V3 dimensions.  Counts are per (query token, cached token) pair for one
layer, with a multiply-add counted as 2 FLOP.  The benchmark prices throughput
with exactly these units.
"""
from __future__ import annotations

import numpy as np


def absorbed_flops_per_pair(d) -> int:
    """All heads: 2*(R+Dr) for the two-term score plus 2*R for the latent weighted sum."""
    return d.n_head * 2 * ((d.kv_lora_rank + d.qk_rope) + d.kv_lora_rank)


def decompressed_flops_per_pair(d) -> int:
    """Standard attention on decompressed K (Dn+Dr wide) and V (Dv wide)."""
    return d.n_head * 2 * (d.qk_nope + d.qk_rope + d.v_head)


def compressed_no_absorption_flops_per_pair(d) -> int:
    """Decompress k_nope and v of the cached token through wk_b / wv_b, then attend."""
    return 2 * d.kv_lora_rank * d.n_head * (d.qk_nope + d.v_head) + decompressed_flops_per_pair(d)


def decompressed_cache_bytes_per_token(d, elem_bytes: int = 2) -> int:
    return d.n_head * (d.qk_nope + d.qk_rope + d.v_head) * elem_bytes


def latent_cache_bytes_per_token(d, elem_bytes: int = 2) -> int:
    return (d.kv_lora_rank + d.qk_rope) * elem_bytes


def q8_0_row_bytes(width: int) -> int:
    """Q8_0: 32 int8 codes + one binary16 scale per 32 values."""
    if width % 32:
        raise ValueError("Q8_0 rows need a width that is a multiple of 32")
    return width // 32 * 34


def visible_pairs(pos, n_kv: int) -> int:
    """Causal (query, key) pairs: key j is visible to a query at pos iff j <= pos, j < n_kv."""
    pos = np.asarray(pos, dtype=np.int64)
    return int(np.clip(pos + 1, 0, n_kv).sum())


def attention_flops(d, pos, n_kv: int) -> int:
    return visible_pairs(pos, n_kv) * absorbed_flops_per_pair(d)


def decode_bytes(d, n_kv: int, n_seq: int, cache_row_bytes: int, act_bytes: int = 2) -> int:
    """Bytes one decode step must move: every sequence's cache rows, its query row
    [q_lat | q_rope] for all heads, and its latent output for all heads."""
    W, R, H = d.kv_lora_rank + d.qk_rope, d.kv_lora_rank, d.n_head
    return n_seq * (n_kv * cache_row_bytes + H * W * act_bytes + H * R * act_bytes)
