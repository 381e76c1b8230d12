"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every expected value here comes from a closed form, an identity, a special case
that reduces to a library routine (torch / numpy in float64), brute force, or a
number the pages print (tests/golden).  None comes from the GPU path.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from deepseek_mla_amd import accounting, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.sqrt((b ** 2).mean()), 1e-300))


def small_dims(H=4, R=64, Dn=32, Dr=16, Dv=32, D=96):
    return synth.Dims(n_head=H, kv_lora_rank=R, qk_nope=Dn, qk_rope=Dr, v_head=Dv, d_model=D,
                      scale=1.0 / math.sqrt(Dn + Dr))


def inputs(d, T, N, seed, pos=None):
    x = synth.generate(d, T, N, seed, pos=pos)
    x["rows"] = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    return x


# ------------------------------------------------------------ absorption ---

@pytest.mark.parametrize("name", ["tiny", "deepseek_dims"])
def test_absorbed_equals_unabsorbed(name):
    """Associativity (absorption page, section 3): attending on the latent cache
    with wk_b folded into q and wv_b applied late equals explicit decompression."""
    if name == "tiny":
        w = synth.WORKLOADS["tiny_f32"]
        d = w.dims
        x = synth.generate_workload(w)
        x["rows"] = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    else:
        d = synth.deepseek_dims(4, 256)
        x = inputs(d, 9, 41, seed=11, pos=np.array([0, 3, 17, 18, 30, 38, 39, 40, 40]))
    a = oracle.mla_absorbed(d, x["q_nope"], x["q_rope"], x["pos"], x["rows"], x["wk_b"],
                            x["wv_b"], x["wo"])
    av, out = oracle.mla_unabsorbed(d, x["q_nope"], x["q_rope"], x["pos"], x["rows"], x["wk_b"],
                                    x["wv_b"], x["wo"])
    assert rel_err(a["out"], out) <= 1e-6
    assert rel_err(a["v"].reshape(av.shape), av) <= 1e-6


def test_wk_b_layout_one_hot():
    """wk_b is [H][R][Dn]: a one-hot wk_b[h][a][b] = 1 copies q_nope[.., b] into
    q_lat[.., a] and nothing else; the rope part is RoPE(q_rope) untouched by wk_b."""
    d = small_dims()
    x = inputs(d, 3, 8, seed=5)
    wk = np.zeros_like(x["wk_b"])
    a_idx, b_idx = 7, 19
    wk[:, a_idx, b_idx] = 1.0
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], wk)
    R = d.kv_lora_rank
    expect = np.zeros((3, d.n_head, R), np.float32)
    expect[:, :, a_idx] = x["q_nope"][:, :, b_idx]
    assert np.array_equal(q[:, :, :R], expect)
    for t in range(3):
        for h in range(d.n_head):
            assert np.array_equal(q[t, h, R:], oracle.rope(x["q_rope"][t, h], x["pos"][t]))


def test_identity_absorption_when_dn_equals_r():
    """With Dn = R and wk_b[h] = I the absorbed query is the nope query itself."""
    d = small_dims(R=32, Dn=32)
    x = inputs(d, 4, 8, seed=6)
    wk = np.broadcast_to(np.eye(32, dtype=np.float32), (d.n_head, 32, 32)).copy()
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], wk)
    assert np.array_equal(q[:, :, :32], x["q_nope"])


def test_out_proj_layout_one_hot():
    """wv_b is [H][Dv][R] and wo is [D][H*Dv] with input column h*Dv+d."""
    d = small_dims()
    T = 2
    rng = np.random.default_rng(0)
    o_lat = rng.standard_normal((T, d.n_head, d.kv_lora_rank)).astype(np.float32)
    wv = np.zeros((d.n_head, d.v_head, d.kv_lora_rank), np.float32)
    wv[2, 5, 11] = 1.0  # v[t, head 2, dim 5] = o_lat[t, 2, 11]
    wo = np.zeros((d.d_model, d.n_head * d.v_head), np.float32)
    wo[13, 2 * d.v_head + 5] = 1.0  # out[t, 13] = v[t, head 2, dim 5]
    v, out = oracle.out_proj(d, o_lat, wv, wo)
    ev = np.zeros((T, d.n_head * d.v_head), np.float32)
    ev[:, 2 * d.v_head + 5] = o_lat[:, 2, 11]
    eo = np.zeros((T, d.d_model), np.float32)
    eo[:, 13] = o_lat[:, 2, 11]
    assert np.array_equal(v, ev)
    assert np.array_equal(out, eo)


def test_out_proj_vs_numpy_matmul():
    d = small_dims()
    rng = np.random.default_rng(1)
    T = 5
    o_lat = rng.standard_normal((T, d.n_head, d.kv_lora_rank)).astype(np.float32)
    wv = rng.standard_normal((d.n_head, d.v_head, d.kv_lora_rank)).astype(np.float32)
    wo = rng.standard_normal((d.d_model, d.n_head * d.v_head)).astype(np.float32)
    v, out = oracle.out_proj(d, o_lat, wv, wo)
    ev = np.einsum("hdl,thl->thd", wv.astype(np.float64), o_lat.astype(np.float64))
    eo = ev.reshape(T, -1) @ wo.astype(np.float64).T
    assert rel_err(v, ev.reshape(T, -1)) <= 1e-6
    assert rel_err(out, eo) <= 1e-6


# ------------------------------------------------------- softmax / causal ---

def test_zero_query_gives_prefix_means():
    """q = 0 makes every score 0, so o_lat[t] is the mean of the visible rows
    (pins normalisation and the inclusive causal boundary j <= pos) and
    lse = ln(number of visible keys)."""
    d = small_dims()
    N = 37
    pos = np.array([0, 1, 5, 20, 36, 50], np.int32)  # 50 >= N: all rows visible
    x = inputs(d, len(pos), N, seed=7, pos=pos)
    q = np.zeros((len(pos), d.n_head, d.row), np.float32)
    o, lse = oracle.attention(d, q, pos, x["rows"])
    c = x["c_kv"][0].astype(np.float64)
    for t, p in enumerate(pos):
        n = min(p + 1, N)
        expect = c[:n].mean(axis=0)
        for h in range(d.n_head):
            assert np.abs(o[t, h] - expect).max() <= 1e-6
            assert abs(lse[t, h] - math.log(n)) <= 1e-6


def test_single_key():
    """N = 1: the softmax of one score is 1, so o_lat = c_kv[0] and lse = s_0."""
    d = small_dims()
    x = inputs(d, 3, 1, seed=8, pos=np.array([0, 4, 9]))
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"])
    o, lse = oracle.attention(d, q, x["pos"], x["rows"])
    for t in range(3):
        for h in range(d.n_head):
            assert np.array_equal(o[t, h], x["rows"][0, :d.kv_lora_rank])
            s0 = d.scale * np.dot(q[t, h].astype(np.float64), x["rows"][0].astype(np.float64))
            assert abs(lse[t, h] - s0) <= 1e-5 * max(1.0, abs(s0))


def test_identical_rows():
    """If every cached row is the same, the output is that row for any query."""
    d = small_dims()
    x = inputs(d, 4, 16, seed=9, pos=np.array([0, 3, 9, 15]))
    rows = np.broadcast_to(x["rows"][3], x["rows"].shape).copy()
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"])
    o, _ = oracle.attention(d, q, x["pos"], rows)
    assert np.abs(o - rows[0, :d.kv_lora_rank]).max() <= 1e-6


def test_rows_sum_to_one():
    """A c_kv column of ones comes out as sum_j p_j = 1 (softmax rows sum to 1)."""
    d = small_dims()
    x = inputs(d, 6, 30, seed=10, pos=np.array([0, 2, 7, 13, 29, 29]))
    rows = x["rows"].copy()
    rows[:, 5] = 1.0
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"])
    o, _ = oracle.attention(d, q, x["pos"], rows)
    assert np.abs(o[:, :, 5] - 1.0).max() <= 1e-6


def test_causal_perturbation():
    """Rows after a query's position cannot change it: perturbing them by +-1e3
    leaves that query's output bit-identical."""
    d = small_dims()
    pos = np.array([3, 9, 10, 20], np.int32)
    x = inputs(d, 4, 32, seed=12, pos=pos)
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], pos, x["wk_b"])
    o1, l1 = oracle.attention(d, q, pos, x["rows"])
    rows = x["rows"].copy()
    rng = np.random.default_rng(3)
    rows[11:] += rng.choice([-1e3, 1e3], size=rows[11:].shape).astype(np.float32)
    o2, l2 = oracle.attention(d, q, pos, rows)
    assert np.array_equal(o1[:3], o2[:3]) and np.array_equal(l1[:3], l2[:3])
    assert not np.array_equal(o1[3], o2[3])


def _bruteforce_numpy(d, q, pos, rows):
    """Full masked [T, N] score matrix per head, float64, vectorised."""
    q = q.astype(np.float64)
    rows = rows.astype(np.float64)
    N = rows.shape[0]
    s = np.einsum("thw,nw->thn", q, rows) * d.scale
    mask = np.arange(N)[None, :] <= pos[:, None]
    s = np.where(mask[:, None, :], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    Z = e.sum(axis=-1, keepdims=True)
    o = np.einsum("thn,nl->thl", e / Z, rows[:, :d.kv_lora_rank])
    return o, (m + np.log(Z))[..., 0]


def test_attention_vs_numpy_bruteforce():
    d = synth.deepseek_dims(3, 64)
    pos = np.array([0, 1, 63, 64, 100, 129, 129], np.int32)
    x = inputs(d, len(pos), 130, seed=13, pos=pos)
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], pos, x["wk_b"])
    o, lse = oracle.attention(d, q, pos, x["rows"])
    eo, el = _bruteforce_numpy(d, q, pos, x["rows"])
    assert rel_err(o, eo) <= 1e-6
    assert np.abs(lse - el).max() <= 1e-5


def test_attention_is_mqa_sdpa():
    """Given q_cat, the latent attention is single-KV-head attention with K the
    full [c_kv | k_rope] row and V its first R columns (one KV head, K 576 and
    V 512 wide: PR #394 page, section 3.1).  Checked against torch's
    scaled_dot_product_attention on the CPU in float64 with an explicit mask."""
    torch = pytest.importorskip("torch")
    d = small_dims()
    pos = np.array([2, 5, 5, 19, 30, 31], np.int32)
    x = inputs(d, len(pos), 32, seed=14, pos=pos)
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], pos, x["wk_b"])
    o, _ = oracle.attention(d, q, pos, x["rows"])
    Q = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]      # [1,H,T,W]
    K = torch.from_numpy(x["rows"].astype(np.float64))[None, None]          # [1,1,N,W]
    V = K[..., :d.kv_lora_rank]
    K = K.expand(1, d.n_head, -1, -1)
    V = V.expand(1, d.n_head, -1, -1)
    mask = torch.arange(32)[None, :] <= torch.from_numpy(pos.astype(np.int64))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                           scale=d.scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert rel_err(o, ref) <= 1e-6


def test_split_score_equals_concatenated_dot():
    """Move elision (absorption page, section 5): the rope term and the latent
    term added separately equal one dot product over the adjacent row parts.
    Zeroing the rope query leaves only the latent term and vice versa."""
    d = small_dims()
    pos = np.array([7], np.int32)
    x = inputs(d, 1, 8, seed=15, pos=pos)
    q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], pos, x["wk_b"])
    R = d.kv_lora_rank
    q_lat_only = q.copy()
    q_lat_only[..., R:] = 0
    q_rope_only = q.copy()
    q_rope_only[..., :R] = 0
    _, l_lat = oracle.attention(d, q_lat_only, pos, x["rows"])
    _, l_rot = oracle.attention(d, q_rope_only, pos, x["rows"])
    rows = x["rows"].astype(np.float64)
    for h in range(d.n_head):
        s_lat = d.scale * rows[:, :R] @ q[0, h, :R].astype(np.float64)
        s_rot = d.scale * rows[:, R:] @ q[0, h, R:].astype(np.float64)
        lse = lambda s: s.max() + np.log(np.exp(s - s.max()).sum())
        assert abs(l_lat[0, h] - lse(s_lat)) <= 1e-5
        assert abs(l_rot[0, h] - lse(s_rot)) <= 1e-5


# ------------------------------------------------------------------ RoPE ---

def test_rope_closed_form():
    """Adjacent pair i rotates by pos * base^(-2i/dr): dr = 4, pos = 1 turns pair 0
    by 1 rad and pair 1 by 10000^(-1/2) = 0.01 rad."""
    x = np.array([1.0, 0.0, 0.0, 1.0], np.float32)
    y = oracle.rope(x, 1, 10000.0)
    expect = [math.cos(1.0), math.sin(1.0), -math.sin(0.01), math.cos(0.01)]
    assert np.allclose(y, expect, rtol=0, atol=1e-7)


def test_rope_invariants():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(64).astype(np.float32)
    k = rng.standard_normal(64).astype(np.float32)
    assert np.array_equal(oracle.rope(q, 0), q)  # position 0 is the identity
    y = oracle.rope(q, 12345)
    pairs = lambda v: np.hypot(v[0::2].astype(np.float64), v[1::2].astype(np.float64))
    assert np.allclose(pairs(y), pairs(q), rtol=1e-6)  # each pair keeps its norm
    # the score between RoPE(q, i) and RoPE(k, j) depends only on i - j
    s = [np.dot(oracle.rope(q, i).astype(np.float64), oracle.rope(k, j).astype(np.float64))
         for i, j in [(10, 3), (107, 100), (5007, 5000)]]
    assert max(s) - min(s) <= 1e-4


# ------------------------------------------------------------ binary16 ---

def test_half_conversion_matches_ieee():
    """binary16 conversion against numpy's IEEE float16 (round to nearest even)."""
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-8, 5, 3000),
        [0.0, -0.0, 65504.0, 65519.0, 65520.0, 70000.0, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8,
         1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -1.5, 1e-3]]).astype(np.float32)
    with np.errstate(over="ignore"):
        want_all = vals.astype(np.float16).view(np.uint16)
    for v, want in zip(vals, want_all):
        want = int(want)
        assert oracle.float_to_half(v) == want, v
    for bits in list(range(0, 0x7C00, 97)) + [1, 0x3FF, 0x400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF]:
        want = float(np.uint16(bits).view(np.float16))
        assert oracle.half_to_float(bits) == want


# ------------------------------------------------------------------ Q8_0 ---

def test_q8_0_exact_codes():
    """Values k/8 with max |k| = 127 give d = (127/8)/127 = 1/8 exactly, so the
    codes are k and dequantisation is exact."""
    k = np.clip(np.arange(-128, 128, dtype=np.int64), -127, 127).reshape(8, 32)
    k[:, 0] = 127
    x = (k / 8.0).astype(np.float32)
    b = oracle.q8_0_quantize(x.reshape(1, 256))
    blocks = b.reshape(8, 34)
    scale_bits = blocks[:, 0].astype(np.uint16) | (blocks[:, 1].astype(np.uint16) << 8)
    assert np.all(scale_bits == 0x3000)  # binary16 0.125: exponent -3 -> 12 << 10
    assert np.array_equal(blocks[:, 2:].view(np.int8).astype(np.int64), k)
    assert np.array_equal(oracle.q8_0_dequantize(b, 256).reshape(8, 32), k / 8.0)


def test_q8_0_round_half_away_and_zero_block():
    x = np.zeros((1, 64), np.float32)
    x[0, :6] = [127.0, 2.5, -2.5, 0.5, -0.5, 126.5]  # d = 1: ties round away from zero
    b = oracle.q8_0_quantize(x)
    q = b[0, 2:34].view(np.int8)
    assert list(q[:6]) == [127, 3, -3, 1, -1, 127]
    assert np.all(b[0, 34:] == 0)  # all-zero block: d = 0, codes 0
    assert oracle.q8_0_dequantize(b, 64)[0, 32:].tolist() == [0.0] * 32


def test_q8_0_roundtrip_bound():
    """|x - deq(q(x))| <= d/2 + 127*|d - half(d)| per block."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 576)).astype(np.float32) * 3
    y = oracle.q8_0_dequantize(oracle.q8_0_quantize(x), 576)
    xb = x.reshape(-1, 32).astype(np.float64)
    d = np.abs(xb).max(axis=1) / 127.0
    dh = d.astype(np.float16).astype(np.float64)
    bound = d / 2 + 127 * np.abs(d - dh) + 1e-12
    assert np.all(np.abs(xb - y.reshape(-1, 32)) <= bound[:, None] * (1 + 1e-6))


def test_q8_0_cache_size_matches_v3_log():
    g = json.load(open(os.path.join(GOLDEN, "q8_0_cache_size_v3.json")))
    row = accounting.q8_0_row_bytes(g["row_width"])
    assert row == oracle.q8_0_row_bytes(576) == 612
    mib = g["n_layer"] * g["n_ctx"] * row / 2 ** 20
    assert round(mib, g["printed_decimals"]) == g["printed_size_mib"]


# ------------------------------------------------------ head chunk planner ---

@pytest.mark.parametrize("n_head,size,cap,expect", [
    (128, 4096, 256, 8),      # 4096/16 = 256 <= 256: 16 iterations of 8 heads
    (128, 4096, 8192, 128),   # within the cap: no chunking
    (128, 4096, 0, 128),      # cap 0 = unlimited
    (128, 4096, 100, 4),      # (0,128) is raised to 128: 4096/32 = 128
    (128, 131072, 8192, 8),   # K x Q size of 8192 queries x 32768 keys x 128 heads, fp32
    (7, 1000, 128, 1),        # no divisor brings 1000 MiB under 128: one head at a time
    (16, 300, 128, 4),        # niter 2 -> 150 > 128; niter 4 -> 75
])
def test_heads_per_chunk(n_head, size, cap, expect):
    """The -amb divisor rule of the absorption page, section 8.3."""
    assert oracle.heads_per_chunk(n_head, size, cap) == expect


# ------------------------------------------------------ FLOP/byte table ---

def test_accounting_reproduces_page_table():
    g = json.load(open(os.path.join(GOLDEN, "accounting_absorption_table.json")))
    d = synth.V3
    assert round(accounting.decompressed_cache_bytes_per_token(d) / 1000, 2) == \
        g["kv_cache_per_token_decompressed_KB"]
    assert round(accounting.latent_cache_bytes_per_token(d) / 1000, 2) == \
        g["kv_cache_per_token_latent_KB"]
    assert round(accounting.decompressed_flops_per_pair(d) / 1e6, 2) == \
        g["flops_per_token_decompressed_M"]
    assert round(accounting.compressed_no_absorption_flops_per_pair(d) / 1e6, 2) == \
        g["flops_per_token_compressed_no_absorption_M"]
    assert round(accounting.absorbed_flops_per_pair(d) / 1e6, 2) == \
        g["flops_per_token_absorbed_M"]
    assert round(accounting.decompressed_cache_bytes_per_token(d) /
                 accounting.latent_cache_bytes_per_token(d)) == g["cache_reduction_approx"]
    assert round(accounting.compressed_no_absorption_flops_per_pair(d) /
                 accounting.absorbed_flops_per_pair(d), -1) == g["compute_reduction_approx"]
    assert round(100 * (1 - accounting.latent_cache_bytes_per_token(d) /
                        accounting.decompressed_cache_bytes_per_token(d)), 1) == \
        g["compression_rate_percent"]


# ---------------------------------------------------------- cache append ---

def _append_inputs(d, T, seed):
    rng = np.random.default_rng(seed)
    c_kv = rng.standard_normal((T, d.kv_lora_rank)).astype(np.float32)
    k_rope = rng.standard_normal((T, d.qk_rope)).astype(np.float32)
    return c_kv, k_rope


def test_cache_append_position_zero_is_concatenation():
    """At position 0 every rotation angle is 0: the new row is exactly [c_kv | k_rope]."""
    d = small_dims()
    c, k = _append_inputs(d, 5, 1)
    rows = oracle.cache_rows_new(d, c, k, np.zeros(5, np.int32))
    assert np.array_equal(rows, np.concatenate([c, k], axis=1))


def test_cache_append_rope_relative_position():
    """The score between a query rotated by mla_absorb_q's rule at position m and a key
    rotated on entry at position n depends on m - n only.  Closed form per pair i
    (complex view q = a + ib, k = c + id): Re(q conj(k) e^{i (m-n) theta_i}),
    theta_i = base^(-2i/Dr), evaluated in float64 here."""
    d = small_dims(H=1, Dr=16)
    rng = np.random.default_rng(5)
    q_rope = rng.standard_normal((3, 1, d.qk_rope)).astype(np.float32)
    kr = rng.standard_normal((3, d.qk_rope)).astype(np.float32)
    zero_nope = np.zeros((3, 1, d.qk_nope), np.float32)
    wk_b = np.zeros((1, d.kv_lora_rank, d.qk_nope), np.float32)
    m = np.array([7, 1000, 40000], np.int32)
    n = np.array([3, 999, 12345], np.int32)
    qc = oracle.absorb_q(d, zero_nope, q_rope, m, wk_b)[:, 0, d.kv_lora_rank:]
    kc = oracle.cache_rows_new(d, np.zeros((3, d.kv_lora_rank), np.float32), kr, n)
    kc = kc[:, d.kv_lora_rank:]
    for t in range(3):
        got = float(np.dot(qc[t].astype(np.float64), kc[t].astype(np.float64)))
        a, b = q_rope[t, 0, 0::2].astype(np.float64), q_rope[t, 0, 1::2].astype(np.float64)
        c, e = kr[t, 0::2].astype(np.float64), kr[t, 1::2].astype(np.float64)
        th = 10000.0 ** (-2.0 * np.arange(d.qk_rope // 2) / d.qk_rope)
        phi = (float(m[t]) - float(n[t])) * th
        want = float(((a * c + b * e) * np.cos(phi) - (b * c - a * e) * np.sin(phi)).sum())
        assert abs(got - want) <= 1e-5 * (1 + abs(want)), (t, got, want)
        # each rotated pair keeps its length
        pn = np.hypot(kc[t, 0::2].astype(np.float64), kc[t, 1::2].astype(np.float64))
        assert np.allclose(pn, np.hypot(c, e), rtol=1e-6)


def test_cache_append_destinations():
    """New rows land at pos[t] (or dst_row[t]); other rows, and tokens aimed outside
    [0, N), leave the cache unchanged."""
    d = small_dims()
    W = d.kv_lora_rank + d.qk_rope
    c, k = _append_inputs(d, 4, 2)
    pos = np.array([2, 9, -1, 5], np.int32)
    base = np.full((8, W), 7.0, np.float32)
    out = oracle.cache_append(d, "f32", base, c, k, pos)
    rows = oracle.cache_rows_new(d, c, k, pos)
    for r in range(8):
        want = {2: rows[0], 5: rows[3]}.get(r, base[r])
        assert np.array_equal(out[r], want)
    out2 = oracle.cache_append(d, "f32", base, c, k, pos, dst_row=np.array([0, 1, 7, 8]))
    assert np.array_equal(out2[[0, 1, 7]], rows[[0, 1, 2]])
    assert np.array_equal(out2[2:7], base[2:7])


def test_cache_append_q8_0_within_half_step():
    """A Q8_0 appended row dequantises to within half a quantisation step (d/2, plus the
    binary16 rounding of d times 127) of the float row, block by block."""
    d = small_dims(Dr=32)
    W = d.kv_lora_rank + d.qk_rope
    c, k = _append_inputs(d, 6, 3)
    pos = np.array([0, 1, 2, 3, 4, 5], np.int32)
    q = oracle.cache_append(d, "q8_0", np.zeros((6, W // 32 * 34), np.uint8), c, k, pos)
    rows = oracle.cache_rows_new(d, c, k, pos)
    deq = oracle.q8_0_dequantize(q, W)
    blk = rows.reshape(6, -1, 32)
    dstep = np.abs(blk).max(axis=2, keepdims=True) / 127.0
    bound = dstep / 2 + 127 * dstep * 2.0 ** -11 + 1e-12
    assert (np.abs(deq.reshape(blk.shape) - blk) <= bound).all()


def test_bf16_round_ties_and_library():
    """Round to nearest even at the halfway points, and agreement with torch's float32 ->
    bfloat16 conversion on random values."""
    torch = pytest.importorskip("torch")
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
                  np.inf, -0.0], np.float32)
    want = np.array([1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, np.inf, -0.0], np.float32)
    got = oracle.bf16_round(x)
    assert np.array_equal(got, want)
    assert np.signbit(got[5])
    r = np.random.default_rng(9).standard_normal(10000).astype(np.float32) * 100
    t = torch.from_numpy(r).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_round(r), t)


# ------------------------------------------------------ Hadamard rotation ---

def test_hadamard_matrix():
    """The page's doubling construction against the closed form
    H[i][j] = (-1)^popcount(i & j) / sqrt(n), the textbook orders 2 and 4, symmetry and
    orthonormality."""
    for n in (1, 2, 4, 8, 64, 512):
        h = oracle.hadamard(n)
        i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
        pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
        assert np.array_equal(h, (-1.0) ** pc / np.sqrt(n))
        assert np.array_equal(h, h.T)
        assert np.abs(h @ h - np.eye(n)).max() <= 1e-12
    s2 = 1 / np.sqrt(2)
    assert np.allclose(oracle.hadamard(2), [[s2, s2], [s2, -s2]], atol=0, rtol=0)
    assert np.array_equal(oracle.hadamard(4) * 2, [[1, 1, 1, 1], [1, -1, 1, -1],
                                                  [1, 1, -1, -1], [1, -1, -1, 1]])


def test_hadamard_rotation_preserves_the_layer():
    """A cache whose latent rows are rotated, read with the rotated weights, gives the
    plain layer (H H = I and associativity): absorbed chain on both sides, float32 I/O."""
    d = small_dims()  # R = 64
    x = inputs(d, 7, 30, seed=91, pos=np.array([0, 4, 9, 17, 23, 28, 29]))
    rows_rot = x["rows"].copy()
    h = oracle.hadamard(d.kv_lora_rank)
    rows_rot[:, :d.kv_lora_rank] = (x["rows"][:, :d.kv_lora_rank].astype(np.float64) @ h
                                    ).astype(np.float32)
    wk_r, wv_r = oracle.hadamard_weights(d, x["wk_b"], x["wv_b"])
    a = oracle.mla_absorbed(d, x["q_nope"], x["q_rope"], x["pos"], x["rows"], x["wk_b"],
                            x["wv_b"], x["wo"])
    b = oracle.mla_absorbed(d, x["q_nope"], x["q_rope"], x["pos"], rows_rot, wk_r, wv_r, x["wo"])
    assert rel_err(b["out"], a["out"]) <= 1e-5
    assert np.abs(b["lse"] - a["lse"]).max() <= 1e-5


def test_hadamard_append_rows():
    """cache_append with the rotation stores H c_kv (the closed-form matrix product) and
    leaves the RoPE part as the plain append does."""
    d = small_dims(Dr=32)
    c, k = _append_inputs(d, 5, 92)
    pos = np.array([3, 0, 7, 1, 2], np.int32)
    base = np.zeros((8, d.kv_lora_rank + d.qk_rope), np.float32)
    got = oracle.cache_append(d, "f32", base, c, k, pos, hadamard=True)
    plain = oracle.cache_append(d, "f32", base, c, k, pos)
    R = d.kv_lora_rank
    i, j = np.meshgrid(np.arange(R), np.arange(R), indexing="ij")
    hm = (-1.0) ** np.vectorize(lambda v: bin(int(v)).count("1"))(i & j) / np.sqrt(R)
    assert np.abs(got[pos, :R] - (hm @ c.astype(np.float64).T).T).max() <= 1e-6
    assert np.array_equal(got[:, R:], plain[:, R:])


def test_hadamard_q8_0_spreads_outlier_channels():
    """The page's claim on data it is made for: latents with a few large channels.  The
    Q8_0 cache of the rotated rows (read with the rotated weights) gives a layer output
    closer to the exact one than the Q8_0 cache of the plain rows."""
    d = small_dims(H=4, R=128, Dn=32, Dr=32, Dv=32, D=64)
    x = inputs(d, 8, 96, seed=93, pos=np.arange(88, 96))
    rng = np.random.default_rng(94)
    ch = rng.choice(d.kv_lora_rank, size=4, replace=False)
    rows = x["rows"].copy()
    rows[:, ch] *= 40.0
    exact = oracle.mla_absorbed(d, x["q_nope"], x["q_rope"], x["pos"], rows, x["wk_b"],
                                x["wv_b"], x["wo"])["out"]
    W = d.kv_lora_rank + d.qk_rope
    plain = oracle.q8_0_dequantize(oracle.q8_0_quantize(rows), W)
    out_plain = oracle.mla_absorbed(d, x["q_nope"], x["q_rope"], x["pos"], plain, x["wk_b"],
                                    x["wv_b"], x["wo"])["out"]
    h = oracle.hadamard(d.kv_lora_rank)
    rot = rows.copy()
    rot[:, :d.kv_lora_rank] = (rows[:, :d.kv_lora_rank].astype(np.float64) @ h).astype(np.float32)
    rot = oracle.q8_0_dequantize(oracle.q8_0_quantize(rot), W)
    wk_r, wv_r = oracle.hadamard_weights(d, x["wk_b"], x["wv_b"])
    out_rot = oracle.mla_absorbed(d, x["q_nope"], x["q_rope"], x["pos"], rot, wk_r, wv_r,
                                  x["wo"])["out"]
    e_plain, e_rot = rel_err(out_plain, exact), rel_err(out_rot, exact)
    assert e_rot < 0.5 * e_plain, (e_rot, e_plain)


# ------------------------------------------------------ merged wkv_b layout ---

def test_wkv_b_merged_rows_match_absorption_and_late_projection():
    """The merged rows' orientation pinned against the oracle's own absorption and late
    projection (separate C code): q_lat = wkv_b[h][:Dn]^T q_nope (the K rows seen from the
    query side) and v = wkv_b[h][Dn:] o_lat (the V rows); the split of the merge gives the
    pair back exactly."""
    d = small_dims(H=3, R=64, Dn=32, Dr=16, Dv=24, D=40)
    x = inputs(d, 4, 20, seed=101, pos=np.array([3, 9, 15, 19]))
    m = oracle.wkv_b_merge(d, x["wk_b"], x["wv_b"])
    assert m.shape == (3, 32 + 24, 64)
    q_cat = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"])
    want_q = np.einsum("hdl,thd->thl", m[:, :32, :].astype(np.float64),
                       x["q_nope"].astype(np.float64))
    assert rel_err(q_cat[:, :, :64], want_q) <= 1e-6
    o_lat, _ = oracle.attention(d, q_cat, x["pos"], x["rows"])
    v, _ = oracle.out_proj(d, o_lat, x["wv_b"], x["wo"])
    want_v = np.einsum("hel,thl->the", m[:, 32:, :].astype(np.float64), o_lat.astype(np.float64))
    assert rel_err(v.reshape(4, 3, 24), want_v) <= 1e-6
    wk, wv = oracle.wkv_b_split(d, m)
    assert np.array_equal(wk, x["wk_b"]) and np.array_equal(wv, x["wv_b"])
