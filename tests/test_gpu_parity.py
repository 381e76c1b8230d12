"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerance (for each output row x, i.e. one query's vector along the last axis):
max |x_gpu - x_oracle| <= tol * rms(x_oracle), with tol = 1e-4 in float32 mode and
2e-2 in bf16 / Q8_0 mode; outputs stored in bf16 are
additionally allowed half a bf16 ulp of the exact value (the rounding of the stored
result itself).  lse (always float32) is compared in absolute terms against tol.  Inputs are the same seeded
values on both sides (bf16-rounded, or Q8_0 bytes produced by the oracle's quantiser,
before either side sees them).  Q8_0 (de)quantisation is compared bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
from deepseek_mla_amd import synth
from oracle import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = compare.TOL


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from deepseek_mla_amd import mla
    mla.lib()  # fail loudly if the library is missing
    return "cuda"


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.sqrt((b ** 2).mean()), 1e-30))


def rel_err_stored(g, r, mode):
    return compare.row_error(g, r, mode)


def report(name, err, tol):
    print(f"  {name}: max|diff|/rms = {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.0e}"


def oracle_chain(dims, x, rows, qsel=None):
    """Oracle q_cat, o_lat, lse, v, out for the selected query rows."""
    q_nope, q_rope, pos = x["q_nope"], x["q_rope"], x["pos"]
    if qsel is not None:
        q_nope, q_rope, pos = q_nope[qsel], q_rope[qsel], pos[qsel]
    return oracle.mla_absorbed(dims, q_nope, q_rope, pos, rows, x["wk_b"], x["wv_b"], x["wo"])


ALL_STAGES = ("q_cat", "o_lat", "lse", "v", "out")


def check_stages(got, ref, mode, sel=None, stages=("q_cat", "o_lat", "lse", "out")):
    tol = TOL[mode]
    for k in stages:
        g = got[k] if sel is None else got[k][sel]
        r = ref[k]
        if k == "lse":  # lse is compared against the spread of scores it summarises
            err = float(np.abs(g - r).max())
            report(k + " (abs)", err, tol)
        else:
            report(k, rel_err_stored(g, r, mode), tol)


def small_prefill(dims, mode, T, N, seed, pos):
    x = synth.generate(dims, T, N, seed, mode=mode, pos=pos)
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    return x, rows


# ----------------------------------------------------------------- Q8_0 ---

def test_q8_0_dequant_bit_exact(dev):
    from deepseek_mla_amd import mla
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((37, 576)) * 2).astype(np.float32)
    x[3, 32:64] = 0.0  # a zero block
    x[5, :32] = 1e-3   # tiny scale
    b = oracle.q8_0_quantize(x)
    ref = oracle.q8_0_dequantize(b, 576)
    bt = torch.from_numpy(b).to(dev)
    out = torch.empty((37, 576), dtype=torch.float32, device=dev)
    mla.mla_dequant_q8_0(bt, out, 37, 576)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_q8_0_quantize_bit_exact(dev):
    from deepseek_mla_amd import mla
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((41, 576)) * 3).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :6] = [127.0, 2.5, -2.5, 0.5, -0.5, 126.5]
    x[1, 6:32] = 0.0
    ref = oracle.q8_0_quantize(x)
    rows = torch.empty((41, 612), dtype=torch.uint8, device=dev)
    mla.mla_quantize_q8_0(torch.from_numpy(x).to(dev), rows, 41, 576)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), ref)


# ---------------------------------------------------------- float32 path ---

def test_tiny_f32_chain(dev):
    """The tiny float32 layer (4 heads, R 64, 16 queries at 48..63 over 64 keys)."""
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["tiny_f32"]
    x = synth.generate_workload(w)
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    ref = oracle_chain(w.dims, x, rows)
    L = layer.for_workload(w, x)
    L.step()
    torch.cuda.synchronize()
    check_stages(L.outputs(), ref, "f32", stages=("q_cat", "o_lat", "lse", "v", "out"))


def test_f32_decode_splits(dev):
    from deepseek_mla_amd import layer
    d = synth.TINY
    N = 300
    x = synth.generate(d, 1, N, seed=23, n_seq=3)
    ref_o = []
    for b in range(3):
        rows = synth.cache_rows(x["c_kv"][b], x["k_rope"][b])
        ref_o.append(oracle_chain(d, {k: (v[b:b + 1] if k in ("q_nope", "q_rope", "pos") else v)
                                      for k, v in x.items()}, rows))
    for ns in (1, 2, 3, 7, 0):
        L = layer.LayerStep(d, "f32", "decode", x, N, n_splits=ns)
        L.step()
        torch.cuda.synchronize()
        got = L.outputs()
        for b in range(3):
            print(f" splits={ns} seq={b}")
            check_stages({k: v[b:b + 1] for k, v in got.items()}, ref_o[b], "f32")


# ------------------------------------------------------------- bf16 path ---

@pytest.mark.parametrize("T,N,pos0", [(1, 1, 0), (37, 37, 0), (200, 333, 133), (96, 500, 404)])
def test_bf16_prefill_small(dev, T, N, pos0):
    """Lite-dims prefill spanning several tiles with ragged ends."""
    from deepseek_mla_amd import layer
    d = synth.deepseek_dims(16, 2048)
    pos = np.arange(pos0, pos0 + T, dtype=np.int32)
    x, rows = small_prefill(d, "bf16", T, N, seed=31 + T, pos=pos)
    ref = oracle_chain(d, x, rows)
    L = layer.LayerStep(d, "bf16", "prefill", x, N)
    L.step()
    torch.cuda.synchronize()
    check_stages(L.outputs(), ref, "bf16")


@pytest.mark.parametrize("T,N", [(200, 333), (700, 1500)])
def test_bf16_prefill_unordered_positions(dev, T, N):
    """Query positions in no order and with repeats (not the last T rows of the cache): the
    cut prefill's work lists and key-part sizes are estimated from the usual layout, so this
    checks that only the schedule, never the result, depends on that estimate."""
    from deepseek_mla_amd import layer
    d = synth.deepseek_dims(16, 2048)
    rng = np.random.default_rng(37 + T)
    pos = rng.integers(0, N, size=T).astype(np.int32)
    pos[: T // 4] = N - 1  # several full rows
    rng.shuffle(pos)
    x, rows = small_prefill(d, "bf16", T, N, seed=41 + T, pos=pos)
    ref = oracle_chain(d, x, rows)
    L = layer.LayerStep(d, "bf16", "prefill", x, N)
    L.step()
    torch.cuda.synchronize()
    check_stages(L.outputs(), ref, "bf16")


def test_bf16_prefill_chunked_vs_unchunked_bitwise(dev):
    """Force real chunking with a T*N*H*4 intermediate above 128 MiB (16 heads)."""
    from deepseek_mla_amd import layer, mla
    d = synth.deepseek_dims(16, 2048)
    T, N = 1024, 2560  # 1024*2560*16*4 B = 160 MiB > 128 -> 2 chunks of 8 heads
    assert mla.mla_heads_per_chunk(16, T * N * 16 * 4 / 2 ** 20, 128) == 8
    pos = np.arange(N - T, N, dtype=np.int32)
    x, rows = small_prefill(d, "bf16", T, N, seed=42, pos=pos)
    L = layer.LayerStep(d, "bf16", "prefill", x, N)
    L.absorb()
    L.scratch_cap_mib = 0
    L.attend()
    torch.cuda.synchronize()
    o0, l0 = L.o_lat.clone(), L.lse.clone()
    L.scratch_cap_mib = 128
    L.attend()
    torch.cuda.synchronize()
    assert torch.equal(L.o_lat, o0) and torch.equal(L.lse, l0)
    # and sampled rows against the oracle
    sel = np.array([0, 1, 511, 1022, 1023])
    ref = oracle_chain(d, x, rows, qsel=sel)
    report("o_lat (sampled)", rel_err_stored(o0.float().cpu().numpy()[sel], ref["o_lat"], "bf16"),
           2e-2)


def test_bf16_prefill_causal_perturbation(dev):
    """Cache rows after a query's position cannot change its output (bitwise)."""
    from deepseek_mla_amd import layer
    d = synth.deepseek_dims(16, 2048)
    T, N = 64, 256
    pos = np.arange(N - T, N, dtype=np.int32)
    x, rows = small_prefill(d, "bf16", T, N, seed=43, pos=pos)
    L = layer.LayerStep(d, "bf16", "prefill", x, N)
    L.absorb()
    L.attend()
    torch.cuda.synchronize()
    o1 = L.o_lat.clone()
    cut = 220  # rows >= 220 only visible to queries with pos >= 220
    L.cache[:, cut:] += 1000.0
    L.attend()
    torch.cuda.synchronize()
    keep = pos < cut
    assert torch.equal(L.o_lat[torch.from_numpy(keep).to(dev)], o1[torch.from_numpy(keep).to(dev)])
    assert not torch.equal(L.o_lat, o1)


def test_bf16_prefill_score_jump_repass(dev):
    """A late key whose score exceeds the first tile's max by far more than 2^64 (base-2)
    triggers the kernel's repeated pass; the result still matches the oracle."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    T, N = 4, 300
    rng = np.random.default_rng(44)
    q = synth.round_bf16(rng.standard_normal((T, 16, 576)).astype(np.float32) * 0.1)
    rows = synth.round_bf16(rng.standard_normal((N, 576)).astype(np.float32) * 0.1)
    # key 250 aligned with query (3, 5): score = scale*400*|q|^2 ~ 166 nats, the rest ~0
    rows[250] = synth.round_bf16(q[3, 5] * 400.0)
    pos = np.array([100, 260, 280, 299], np.int32)
    ro, rl = oracle.attention(d, q, pos, rows)
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16)
    cd = torch.from_numpy(rows).to(dev).to(torch.bfloat16)
    pd = torch.from_numpy(pos).to(dev)
    o = torch.empty((T, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, 16), dtype=torch.float32, device=dev)
    mla.mla_attn_prefill(mla.make_dims(d), mla.BF16, mla.BF16, qd, pd, T, cd, N, o, lse)
    torch.cuda.synchronize()
    s_max = (d.scale * rows[250].astype(np.float64) @ q[3, 5].astype(np.float64))
    assert s_max > 60.0  # far beyond the frozen max's 44-nat margin
    report("o_lat", rel_err_stored(o.float().cpu().numpy(), ro, "bf16"), 2e-2)
    report("lse (abs)", float(np.abs(lse.cpu().numpy() - rl).max()), 2e-2)


@pytest.mark.parametrize("mode", ["bf16", "q8_0"])
def test_decode_splits(dev, mode):
    """V3-dims decode, 2 sequences of different lengths, split counts 1, 2, 3, 7, auto."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    Nmax, lens = 777, [777, 301]
    x = synth.generate(d, 1, Nmax, seed=51, n_seq=2, mode="bf16")
    x["pos"] = np.array([l - 1 for l in lens], np.int32)
    W = 576
    q_cat_ref, rows_f = [], []
    # both sides attend with the same bf16-rounded absorbed queries
    qc = synth.round_bf16(oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"]))
    for b in range(2):
        r = synth.cache_rows(x["c_kv"][b], x["k_rope"][b])
        if mode == "q8_0":
            r = oracle.q8_0_dequantize(oracle.q8_0_quantize(r), W)
        rows_f.append(r)
    ref = [oracle.attention(d, qc[b:b + 1], x["pos"][b:b + 1], rows_f[b][:lens[b]]) for b in range(2)]
    qd = torch.from_numpy(qc).to(dev).to(torch.bfloat16)
    if mode == "q8_0":
        qb, stride = q8_cache([synth.cache_rows(x["c_kv"][b], x["k_rope"][b]) for b in range(2)],
                              Nmax)
        cache, kv = torch.from_numpy(qb).to(dev), mla.Q8_0
    else:
        cache = torch.from_numpy(np.stack(rows_f)).to(dev).to(torch.bfloat16)
        stride, kv = 1152 * Nmax, mla.BF16
    nkv = torch.tensor(lens, dtype=torch.int32, device=dev)
    cd = mla.make_dims(d)
    for ns in (1, 2, 3, 7, 0):
        wsb = mla.mla_decode_workspace_bytes(cd, 2, Nmax, ns)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        o = torch.empty((2, 128, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((2, 128), dtype=torch.float32, device=dev)
        mla.mla_attn_decode(cd, mla.BF16, kv, qd, cache, stride, nkv, 2, Nmax, ns, o, lse, ws, wsb)
        torch.cuda.synchronize()
        for b in range(2):
            print(f" splits={ns} seq={b}")
            report("o_lat", rel_err_stored(o[b].float().cpu().numpy(), ref[b][0][0], mode),
                   TOL[mode])
            report("lse (abs)", float(np.abs(lse[b].cpu().numpy() - ref[b][1][0]).max()), TOL[mode])


def q8_cache(float_rows, Nmax):
    """Q8_0 bytes of each sequence (float rows [n, 576], n <= Nmax) in a [B][stride] uint8
    buffer, stride = 612*Nmax rounded up to 16 bytes (the decode ABI's alignment)."""
    stride = (612 * Nmax + 15) // 16 * 16
    buf = np.zeros((len(float_rows), stride), np.uint8)
    for b, r in enumerate(float_rows):
        q = oracle.q8_0_quantize(r).reshape(-1)
        buf[b, :q.size] = q
    return buf, stride


def _decode_run(d, q, rows_list, lens, mode, ns):
    """mla_attn_decode on B sequences (bf16 queries q [B,H,576]); rows_list holds the float
    rows (bf16-rounded) of each sequence.  Returns o_lat, lse as numpy."""
    from deepseek_mla_amd import mla
    B, H = q.shape[0], q.shape[1]
    Nmax = max(r.shape[0] for r in rows_list)
    pad = [np.concatenate([r, np.zeros((Nmax - r.shape[0], 576), np.float32)]) for r in rows_list]
    if mode == "q8_0":
        qb, stride = q8_cache(pad, Nmax)
        cache, kv = torch.from_numpy(qb).to(dev_name()), mla.Q8_0
    else:
        cache = torch.from_numpy(np.stack(pad)).to(dev_name()).to(torch.bfloat16)
        stride, kv = 1152 * Nmax, mla.BF16
    qd = torch.from_numpy(q).to(dev_name()).to(torch.bfloat16)
    nkv = torch.tensor(lens, dtype=torch.int32, device=dev_name())
    cd = mla.make_dims(d)
    wsb = mla.mla_decode_workspace_bytes(cd, B, Nmax, ns)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev_name())
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev_name())
    lse = torch.empty((B, H), dtype=torch.float32, device=dev_name())
    mla.mla_attn_decode(cd, mla.BF16, kv, qd, cache, stride, nkv, B, Nmax, ns, o, lse, ws, wsb)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def dev_name():
    return "cuda"


@pytest.mark.parametrize("mode", ["bf16", "q8_0"])
def test_decode_score_jump_repass(dev, mode):
    """Decode: a key whose score exceeds its split's first-tile max by far more than 2^64
    (base 2) triggers the repeated pass; split counts 1 and 3 put the key in a later tile
    of its split.  The result still matches the oracle.

    The jump row is made of half-integers with a maximum of 63.5 in every 32-value block,
    so its Q8_0 codes (scale 0.5) and their bf16 conversion are exact: a row some 400 times
    the size of the others would otherwise magnify the bf16 rounding of dequantised values
    (a documented step of the Q8_0 path) past the tolerance, and the test is about the
    repeated pass."""
    d = synth.deepseek_dims(128, 7168)
    N = 300
    rng = np.random.default_rng(45)
    q = synth.round_bf16(rng.standard_normal((1, 128, 576)).astype(np.float32) * 0.1)
    rows = synth.round_bf16(rng.standard_normal((N, 576)).astype(np.float32) * 0.1)
    jump = np.clip(np.round(q[0, 5].astype(np.float64) * 800.0), -127, 127).reshape(18, 32)
    for blk in jump:  # one code of +-127 per block: amax 63.5, scale exactly 0.5
        i = int(np.argmax(np.abs(blk)))
        blk[i] = 127.0 if blk[i] >= 0 else -127.0
    rows[250] = (jump.reshape(576) * 0.5).astype(np.float32)  # ~150 nats for head 5
    if mode == "q8_0":
        rows = oracle.q8_0_dequantize(oracle.q8_0_quantize(rows), 576)
    s_max = d.scale * rows[250].astype(np.float64) @ q[0, 5].astype(np.float64)
    assert s_max > 60.0
    ro, rl = oracle.attention(d, q, np.array([N - 1], np.int32), rows)
    for ns in (1, 3):
        o, lse = _decode_run(d, q, [rows], [N], mode, ns)
        print(f" splits={ns}")
        report("o_lat", rel_err_stored(o[0], ro[0], mode), TOL[mode])
        report("lse (abs)", float(np.abs(lse[0] - rl[0]).max()), TOL[mode])


@pytest.mark.parametrize("H", [16, 96])
def test_decode_partial_head_groups(dev, H):
    """Decode with head counts that leave a 64-head workgroup partly empty (16: one group;
    96: a full and a half group), 3 sequences of ragged length, bf16 and Q8_0 caches."""
    d = synth.deepseek_dims(H, 2048)
    lens = [33, 130, 77]
    rng = np.random.default_rng(46 + H)
    q = synth.round_bf16(rng.standard_normal((3, H, 576)).astype(np.float32) * 0.3)
    rows = [synth.round_bf16(rng.standard_normal((n, 576)).astype(np.float32)) for n in lens]
    for mode in ("bf16", "q8_0"):
        rr = rows if mode == "bf16" else [oracle.q8_0_dequantize(oracle.q8_0_quantize(r), 576)
                                          for r in rows]
        for ns in (1, 2, 0):
            o, lse = _decode_run(d, q, rr, lens, mode, ns)
            for b in range(3):
                ro, rl = oracle.attention(d, q[b:b + 1], np.array([lens[b] - 1], np.int32), rr[b])
                print(f" {mode} splits={ns} seq={b}")
                report("o_lat", rel_err_stored(o[b], ro[0], mode), TOL[mode])
                report("lse (abs)", float(np.abs(lse[b] - rl[0]).max()), TOL[mode])


# ------------------------------------------------------- full-size configs ---

def _sample(T, k, seed):
    return synth.sample_tokens(T, k, seed)


def test_lite_prefill_full(dev):
    """DeepSeek-Lite-shaped layer: 2048 causal tokens over 2048 rows, as the bench runs it."""
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["lite_prefill"]
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x)
    L.step()
    torch.cuda.synchronize()
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    sel = _sample(w.T, 24, 61)
    ref = oracle_chain(w.dims, x, rows, qsel=sel)
    check_stages(L.outputs(), ref, "bf16", sel=sel, stages=ALL_STAGES)


def test_v3_decode_full(dev):
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["v3_decode"]
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x)
    L.step()
    torch.cuda.synchronize()
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    ref = oracle_chain(w.dims, x, rows)
    check_stages(L.outputs(), ref, "bf16", stages=ALL_STAGES)


long_prefill_sample = synth.long_prefill_sample


def test_v3_long_prefill_sampled(dev):
    """8192 queries at 24576..32767 over 32768 rows with the 8192 MiB cap (8-head chunks);
    the oracle checks 64 queries (tokens 0 and 8191 among them), all 128 heads, every
    stage."""
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["v3_long_prefill"]
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x)
    L.step()
    torch.cuda.synchronize()
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    sel = long_prefill_sample(w.T)
    ref = oracle_chain(w.dims, x, rows, qsel=sel)
    check_stages(L.outputs(), ref, "bf16", sel=sel, stages=ALL_STAGES)


def test_v3_decode_q8_full(dev):
    """4 sequences x 98304 Q8_0 rows: every stage of every sequence against the oracle
    chain over the oracle's own dequantised rows (all 128 heads)."""
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["v3_decode_q8"]
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x)
    L.step()
    torch.cuda.synchronize()
    got = L.outputs()
    d = w.dims
    for b in range(w.n_seq):
        rows = synth.cache_rows(x["c_kv"][b], x["k_rope"][b])
        rows = oracle.q8_0_dequantize(oracle.q8_0_quantize(rows), 576)
        xb = {k: (v[b:b + 1] if k in ("q_nope", "q_rope", "pos") else v) for k, v in x.items()}
        ref = oracle_chain(d, xb, rows)
        print(f" seq {b}", flush=True)
        check_stages({k: v[b:b + 1] for k, v in got.items()}, ref, "q8_0", stages=ALL_STAGES)


@pytest.mark.parametrize("T", [1, 3, 8, 9])
def test_out_proj_few_and_many_tokens(dev, T):
    """Late projections at V3 dims across the few-token stream (T <= 8) and the matrix-core
    tile path (T = 9), against the oracle on the same bf16 inputs."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    x = synth.generate(d, 1, 8, seed=71, mode="bf16")
    rng = np.random.default_rng(72)
    o_lat = synth.round_bf16(rng.standard_normal((T, 128, 512)) * 0.2)
    rv, ro = oracle.out_proj(d, o_lat, x["wv_b"], x["wo"])
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)
    v = torch.empty((T, 128 * 128), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, 7168), dtype=torch.bfloat16, device=dev)
    mla.mla_out_proj(mla.make_dims(d), mla.BF16, tb(o_lat), tb(x["wv_b"]), tb(x["wo"]), v, out, T)
    torch.cuda.synchronize()
    report("v", rel_err_stored(v.float().cpu().numpy(), rv, "bf16"), 2e-2)
    report("out", rel_err_stored(out.float().cpu().numpy(), ro, "bf16"), 2e-2)


# ------------------------------------------------- projections, other shapes ---

@pytest.mark.parametrize("T", [37, 300])
def test_projections_ragged_dims(dev, T):
    """Absorption and late projections in bf16 at dims off the DeepSeek grid: Dn = 72 (a K
    that is not a whole number of 64-deep k-tiles: the 32-deep GEMM), Dv = 40 and
    d_model = 200 (partial 128-column output tiles of the LDS-staged GEMM), T ragged."""
    import dataclasses
    from deepseek_mla_amd import mla
    d = dataclasses.replace(synth.LITE, qk_nope=72, v_head=40, d_model=200,
                            scale=1.0 / math.sqrt(72 + 64))
    x = synth.generate(d, T, 8, seed=91, mode="bf16", pos=np.arange(T, dtype=np.int32) * 7)
    ref_q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"])
    rng = np.random.default_rng(92)
    o_lat = synth.round_bf16(rng.standard_normal((T, d.n_head, 512)) * 0.2)
    rv, ro = oracle.out_proj(d, o_lat, x["wv_b"], x["wo"])
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)
    q_cat = torch.empty((T, d.n_head, d.row), dtype=torch.bfloat16, device=dev)
    pos = torch.from_numpy(x["pos"]).to(dev)
    md = mla.make_dims(d)
    mla.mla_absorb_q(md, mla.BF16, tb(x["q_nope"]), tb(x["q_rope"]), pos, tb(x["wk_b"]), q_cat, T)
    v = torch.empty((T, d.n_head * d.v_head), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, d.d_model), dtype=torch.bfloat16, device=dev)
    mla.mla_out_proj(md, mla.BF16, tb(o_lat), tb(x["wv_b"]), tb(x["wo"]), v, out, T)
    torch.cuda.synchronize()
    report("q_cat", rel_err_stored(q_cat.float().cpu().numpy(), ref_q, "bf16"), 2e-2)
    report("v", rel_err_stored(v.float().cpu().numpy(), rv, "bf16"), 2e-2)
    report("out", rel_err_stored(out.float().cpu().numpy(), ro, "bf16"), 2e-2)


def test_rope_odd_width_f32(dev):
    """Query RoPE with a rope width that is not a multiple of 8 (the one-pair path) and
    positions up to 1e5, float32 mode."""
    import dataclasses
    from deepseek_mla_amd import mla
    d = dataclasses.replace(synth.TINY, qk_rope=6, scale=1.0 / math.sqrt(32 + 6))
    T = 19
    pos = (np.arange(T, dtype=np.int64) * 5261 % 100003).astype(np.int32)
    x = synth.generate(d, T, 8, seed=93, mode="f32", pos=pos)
    ref_q = oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"])
    tf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    q_cat = torch.empty((T, d.n_head, d.row), dtype=torch.float32, device=dev)
    mla.mla_absorb_q(mla.make_dims(d), mla.F32, tf(x["q_nope"]), tf(x["q_rope"]),
                     torch.from_numpy(x["pos"]).to(dev), tf(x["wk_b"]), q_cat, T)
    torch.cuda.synchronize()
    report("q_cat", rel_err_stored(q_cat.cpu().numpy(), ref_q, "f32"), 1e-4)


# --------------------------------------------------------- cache append ---

def _append_check(got, ref, d, mode, rows):
    """Appended rows: c_kv columns bit for bit.  The RoPE columns differ by the float32
    sine/cosine of the kernel against the oracle's double (a few 1e-7 absolute): float32
    within 1e-5 of the row's rms; bf16 within one bf16 ulp plus 1e-5; Q8_0 RoPE blocks
    one code apart with scales one binary16 ulp apart, c_kv blocks byte for byte."""
    R, W = d.kv_lora_rank, d.kv_lora_rank + d.qk_rope
    if mode == "q8_0":
        nb = W // 32
        g = got[rows].reshape(len(rows), nb, 34)
        r = ref[rows].reshape(len(rows), nb, 34)
        nc = R // 32
        assert np.array_equal(g[:, :nc], r[:, :nc])
        gs = g[:, nc:, :2].copy().view(np.uint16).astype(np.int32)
        rs = r[:, nc:, :2].copy().view(np.uint16).astype(np.int32)
        assert np.abs(gs - rs).max() <= 1
        gq = g[:, nc:, 2:].view(np.int8).astype(np.int32)
        rq = r[:, nc:, 2:].view(np.int8).astype(np.int32)
        assert np.abs(gq - rq).max() <= 1
        return
    g, r = got[rows].astype(np.float64), ref[rows].astype(np.float64)
    assert np.array_equal(g[:, :R], r[:, :R])
    if mode == "bf16":
        assert (np.abs(g[:, R:] - r[:, R:]) <= 2.0 ** -7 * np.abs(r[:, R:]) + 1e-5).all()
    else:
        report("rope", rel_err(g[:, R:], r[:, R:]), 1e-5)


def _append_run(d, mode, c_kv, k_rope, pos, n_rows, fill, dst_row=None):
    """mla_cache_append into a cache filled with `fill`; returns the cache as numpy
    (float32 values for f32 / bf16, bytes for Q8_0)."""
    from deepseek_mla_amd import mla
    W = d.kv_lora_rank + d.qk_rope
    T = c_kv.shape[0]
    act = mla.F32 if mode == "f32" else mla.BF16
    tdt = torch.float32 if mode == "f32" else torch.bfloat16
    if mode == "q8_0":
        cache = torch.full((n_rows, W // 32 * 34), fill, dtype=torch.uint8, device="cuda")
        kv = mla.Q8_0
    else:
        cache = torch.full((n_rows, W), fill, dtype=tdt, device="cuda")
        kv = act
    ct = torch.from_numpy(np.ascontiguousarray(c_kv)).to("cuda").to(tdt)
    kt = torch.from_numpy(np.ascontiguousarray(k_rope)).to("cuda").to(tdt)
    pt = torch.from_numpy(np.ascontiguousarray(pos, np.int32)).to("cuda")
    dt = None if dst_row is None else torch.from_numpy(np.asarray(dst_row, np.int64)).to("cuda")
    mla.mla_cache_append(mla.make_dims(d), act, kv, ct, kt, pt, T, cache, n_rows, dst_row=dt)
    torch.cuda.synchronize()
    return cache.cpu().numpy() if mode == "q8_0" else cache.float().cpu().numpy()


@pytest.mark.parametrize("mode", ["f32", "bf16", "q8_0"])
def test_cache_append_small(dev, mode):
    """77 tokens (a ragged count) at scattered positions up to 1e5 through dst_row, plus
    position-indexed rows, a token aimed below 0 and one past the end; every other row
    keeps its fill."""
    d = synth.TINY if mode == "f32" else synth.deepseek_dims(16, 2048)
    T, N = 77, 300
    rng = np.random.default_rng(61)
    c = rng.standard_normal((T, d.kv_lora_rank)).astype(np.float32)
    k = (rng.standard_normal((T, d.qk_rope)) * 3).astype(np.float32)
    if mode != "f32":
        c, k = synth.round_bf16(c), synth.round_bf16(k)
    # position-indexed: a permutation of distinct rows, one -1 and one N
    pos = rng.permutation(N)[:T].astype(np.int32)
    pos[5], pos[40] = -1, N
    fill = 0xAB if mode == "q8_0" else 7.0
    got = _append_run(d, mode, c, k, pos, N, fill)
    base = np.full_like(got, fill)
    ref = oracle.cache_append(d, mode, base, c, k, pos)
    hit = sorted(int(p) for p in pos if 0 <= p < N)
    assert len(hit) == T - 2
    _append_check(got, ref, d, mode, hit)
    miss = [r for r in range(N) if r not in set(hit)]
    assert np.array_equal(got[miss], base[miss])
    # explicit destinations with large rotation positions
    pos2 = (np.arange(T, dtype=np.int64) * 7919 % 100003).astype(np.int32)
    dst = rng.permutation(N)[:T].astype(np.int64)
    got2 = _append_run(d, mode, c, k, pos2, N, fill, dst_row=dst)
    ref2 = oracle.cache_append(d, mode, base, c, k, pos2, dst_row=dst)
    _append_check(got2, ref2, d, mode, sorted(int(r) for r in dst))
    print(f"  {mode}: {T} tokens, rows checked", flush=True)


@pytest.mark.parametrize("mode", ["bf16", "q8_0"])
def test_cache_append_then_decode(dev, mode):
    """Two V3 sequences (Nmax 300 rows each) filled entirely by mla_cache_append through
    dst_row = b*Nmax + pos, then attended by mla_attn_decode: the result matches the
    oracle's attention over the oracle's appended rows."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    W, Nmax, lens = 576, 300, [300, 123]
    rng = np.random.default_rng(62)
    c = synth.round_bf16(rng.standard_normal((2 * Nmax, 512)).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((2 * Nmax, 64)).astype(np.float32))
    pos = np.tile(np.arange(Nmax, dtype=np.int32), 2)
    dst = np.arange(2 * Nmax, dtype=np.int64)
    fill = 0 if mode == "q8_0" else 0.0
    got = _append_run(d, mode, c, k, pos, 2 * Nmax, fill, dst_row=dst)
    base = np.zeros_like(got)
    ref = oracle.cache_append(d, mode, base, c, k, pos, dst_row=dst)
    _append_check(got, ref, d, mode, list(range(2 * Nmax)))
    rows_ref = oracle.q8_0_dequantize(ref, W) if mode == "q8_0" else ref
    x = synth.generate(d, 1, 8, seed=63, n_seq=2, mode="bf16")
    qpos = np.array([l - 1 for l in lens], np.int32)
    qc = synth.round_bf16(oracle.absorb_q(d, x["q_nope"], x["q_rope"], qpos, x["wk_b"]))
    if mode == "q8_0":
        cache, stride, kv = torch.from_numpy(got).to(dev), 612 * Nmax, mla.Q8_0
    else:
        cache = torch.from_numpy(got).to(dev).to(torch.bfloat16)
        stride, kv = 1152 * Nmax, mla.BF16
    nkv = torch.tensor(lens, dtype=torch.int32, device=dev)
    cd = mla.make_dims(d)
    wsb = mla.mla_decode_workspace_bytes(cd, 2, Nmax, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    o = torch.empty((2, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, 128), dtype=torch.float32, device=dev)
    mla.mla_attn_decode(cd, mla.BF16, kv, torch.from_numpy(qc).to(dev).to(torch.bfloat16), cache,
                        stride, nkv, 2, Nmax, 0, o, lse, ws, wsb)
    torch.cuda.synchronize()
    for b in range(2):
        r = rows_ref[b * Nmax: b * Nmax + lens[b]]
        ro, rl = oracle.attention(d, qc[b:b + 1], qpos[b:b + 1], r)
        report("o_lat", rel_err_stored(o[b].float().cpu().numpy(), ro[0], mode), TOL[mode])
        report("lse (abs)", float(np.abs(lse[b].cpu().numpy() - rl[0]).max()), TOL[mode])


def test_cache_append_v3_long_prefill_rows(dev):
    """The long-context prefill's own append: 8192 new V3 tokens at positions
    24576..32767 into a 32768-row bf16 cache; every new row checked, every old row kept."""
    d = synth.deepseek_dims(128, 7168)
    T, N, p0 = 8192, 32768, 24576
    rng = np.random.default_rng(64)
    c = synth.round_bf16(rng.standard_normal((T, 512)).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((T, 64)).astype(np.float32))
    pos = np.arange(p0, p0 + T, dtype=np.int32)
    got = _append_run(d, "bf16", c, k, pos, N, 0.5)
    assert (got[:p0] == 0.5).all()
    new = oracle.bf16_round(oracle.cache_rows_new(d, c, k, pos))
    ref = np.full_like(got, 0.5)
    ref[p0:] = new
    _append_check(got, ref, d, "bf16", list(range(p0, N)))


def test_cache_append_v3_decode_q8_rows(dev):
    """The Q8_0 decode workload's append: one token per sequence for 4 sequences of
    98304 rows, each at its last row (position 98303), through dst_row."""
    d = synth.deepseek_dims(128, 7168)
    B, N = 4, 98304
    rng = np.random.default_rng(65)
    c = synth.round_bf16(rng.standard_normal((B, 512)).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((B, 64)).astype(np.float32))
    pos = np.full(B, N - 1, np.int32)
    dst = np.arange(B, dtype=np.int64) * N + (N - 1)
    got = _append_run(d, "q8_0", c, k, pos, B * N, 0x5A, dst_row=dst)
    rows = [int(r) for r in dst]
    ref = np.full_like(got, 0x5A)
    ref[rows] = oracle.q8_0_quantize(oracle.cache_rows_new(d, c, k, pos))
    _append_check(got, ref, d, "q8_0", rows)
    untouched = np.ones(B * N, bool)
    untouched[rows] = False
    assert (got[untouched] == 0x5A).all()


# ------------------------------------------- materialised prefill (pp_opt) ---

MAT_STAGES = ("lse", "v", "out")


@pytest.mark.parametrize("T,N,pos0", [(1, 1, 0), (37, 37, 0), (200, 333, 133), (300, 700, 400)])
def test_materialized_prefill_small(dev, T, N, pos0):
    """Lite dims (16 heads): ragged token blocks and key tiles.  v and out against the
    oracle's explicitly decompressed path, lse against its absorbed attention."""
    from deepseek_mla_amd import layer
    d = synth.deepseek_dims(16, 2048)
    pos = np.arange(pos0, pos0 + T, dtype=np.int32)
    x, rows = small_prefill(d, "bf16", T, N, seed=71 + T, pos=pos)
    ref = oracle_chain(d, x, rows)
    av, out = oracle.mla_unabsorbed(d, x["q_nope"], x["q_rope"], x["pos"], rows, x["wk_b"],
                                    x["wv_b"], x["wo"])
    ref["v"] = av.reshape(T, -1)
    ref["out"] = out
    L = layer.LayerStep(d, "bf16", "prefill", x, N, path="materialized")
    L.step()
    torch.cuda.synchronize()
    check_stages(L.outputs(), ref, "bf16", stages=MAT_STAGES)


def test_materialized_prefill_unordered_and_chunked(dev):
    """Positions in no order, with repeats and rows past the cache end; then the same call
    with a scratch cap that splits the 16 heads into chunks gives bitwise the same
    output."""
    from deepseek_mla_amd import layer, mla
    d = synth.deepseek_dims(16, 2048)
    T, N = 300, 700
    rng = np.random.default_rng(73)
    pos = rng.integers(0, N + 50, size=T).astype(np.int32)
    pos[:40] = N - 1
    rng.shuffle(pos)
    x, rows = small_prefill(d, "bf16", T, N, seed=74, pos=pos)
    ref = oracle_chain(d, x, rows)
    L = layer.LayerStep(d, "bf16", "prefill", x, N, path="materialized")
    L.step()
    torch.cuda.synchronize()
    got = L.outputs()
    check_stages(got, ref, "bf16", stages=MAT_STAGES)
    # T*N*H*4 B = 12.8 MiB; a 128 MiB cap cannot split it, so compare cap 0 against a
    # planner split forced through the smallest cap on a larger T*N
    T2, N2 = 1200, 2048
    pos2 = np.arange(N2 - T2, N2, dtype=np.int32)
    x2, _ = small_prefill(d, "bf16", T2, N2, seed=75, pos=pos2)
    assert mla.mla_heads_per_chunk(16, T2 * N2 * 16 * 4 / 2 ** 20, 128) < 16
    outs = []
    for cap in (0, 128):
        L2 = layer.LayerStep(d, "bf16", "prefill", x2, N2, scratch_cap_mib=cap,
                             path="materialized")
        L2.step()
        torch.cuda.synchronize()
        outs.append(L2.outputs())
    for k in MAT_STAGES:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_materialized_lite_full(dev):
    """The Lite prefill (2048 tokens over 2048 rows) on the materialised path, 24 sampled
    tokens against the oracle."""
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["lite_prefill"]
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x, path="materialized")
    L.step()
    torch.cuda.synchronize()
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    sel = _sample(w.T, 24, 76)
    ref = oracle_chain(w.dims, x, rows, qsel=sel)
    check_stages(L.outputs(), ref, "bf16", sel=sel, stages=MAT_STAGES)


def test_materialized_v3_long_sampled(dev):
    """The V3 long prefill (8192 tokens at 24576..32767 over 32768 rows, 8192 MiB cap:
    16 chunks of 8 heads) on the materialised path; 64 tokens (0 and 8191 among them), all
    128 heads."""
    from deepseek_mla_amd import layer
    w = synth.WORKLOADS["v3_long_prefill"]
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x, path="materialized")
    L.step()
    torch.cuda.synchronize()
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    sel = long_prefill_sample(w.T)
    ref = oracle_chain(w.dims, x, rows, qsel=sel)
    check_stages(L.outputs(), ref, "bf16", sel=sel, stages=MAT_STAGES)


# ------------------------------------------------ Hadamard-rotated cache ---

@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_hadamard_weights(dev, mode):
    """GPU rotated weights (fast transform in float32) against the oracle's float64 matrix
    products: float32 within 1e-5 of each row's rms, bf16 within one bf16 ulp + 1e-6."""
    from deepseek_mla_amd import mla
    d = synth.TINY if mode == "f32" else synth.deepseek_dims(16, 2048)
    x = synth.generate(d, 1, 4, seed=95, mode=mode)
    wk_r, wv_r = oracle.hadamard_weights(d, x["wk_b"], x["wv_b"])
    tdt = torch.float32 if mode == "f32" else torch.bfloat16
    act = mla.F32 if mode == "f32" else mla.BF16
    wk = torch.from_numpy(x["wk_b"]).to(dev).to(tdt)
    wv = torch.from_numpy(x["wv_b"]).to(dev).to(tdt)
    gk, gv = torch.empty_like(wk), torch.empty_like(wv)
    mla.mla_hadamard_weights(mla.make_dims(d), act, wk, wv, gk, gv)
    torch.cuda.synchronize()
    for name, g, r in (("wk_b", gk, wk_r), ("wv_b", gv, wv_r)):
        g = g.float().cpu().numpy().astype(np.float64)
        if mode == "f32":
            report(name, rel_err(g, r), 1e-5)
        else:
            assert (np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-6).all(), name


@pytest.mark.parametrize("mode", ["f32", "bf16", "q8_0"])
def test_cache_append_hadamard(dev, mode):
    """Rotated append: latent part H c_kv (float32 transform on the GPU, float64 in the
    oracle), RoPE part as in the plain append."""
    from deepseek_mla_amd import mla
    d = synth.TINY if mode == "f32" else synth.deepseek_dims(16, 2048)
    T, N = 45, 120
    rng = np.random.default_rng(96)
    c = rng.standard_normal((T, d.kv_lora_rank)).astype(np.float32)
    k = rng.standard_normal((T, d.qk_rope)).astype(np.float32)
    if mode != "f32":
        c, k = synth.round_bf16(c), synth.round_bf16(k)
    pos = rng.permutation(N)[:T].astype(np.int32)
    W = d.kv_lora_rank + d.qk_rope
    tdt = torch.float32 if mode == "f32" else torch.bfloat16
    act = mla.F32 if mode == "f32" else mla.BF16
    if mode == "q8_0":
        cache = torch.zeros((N, W // 32 * 34), dtype=torch.uint8, device=dev)
        kv = mla.Q8_0
    else:
        cache = torch.zeros((N, W), dtype=tdt, device=dev)
        kv = act
    mla.mla_cache_append_hadamard(mla.make_dims(d), act, kv, torch.from_numpy(c).to(dev).to(tdt),
                                  torch.from_numpy(k).to(dev).to(tdt),
                                  torch.from_numpy(pos).to(dev), T, cache, N)
    torch.cuda.synchronize()
    got = cache.cpu().numpy() if mode == "q8_0" else cache.float().cpu().numpy()
    ref = oracle.cache_append(d, mode, np.zeros_like(got), c, k, pos, hadamard=True)
    rows = sorted(int(p) for p in pos)
    if mode == "q8_0":
        g = got[rows].reshape(len(rows), -1, 34)
        r = ref[rows].reshape(len(rows), -1, 34)
        gs = g[:, :, :2].copy().view(np.uint16).astype(np.int32)
        rs = r[:, :, :2].copy().view(np.uint16).astype(np.int32)
        assert np.abs(gs - rs).max() <= 1
        gq = g[:, :, 2:].view(np.int8).astype(np.int32)
        rq = r[:, :, 2:].view(np.int8).astype(np.int32)
        assert np.abs(gq - rq).max() <= 1
    elif mode == "bf16":
        g, r = got[rows].astype(np.float64), ref[rows].astype(np.float64)
        assert (np.abs(g - r) <= 2.0 ** -7 * np.abs(r) + 1e-5).all()
    else:
        report("rows", rel_err(got[rows], ref[rows]), 1e-5)
    others = np.setdiff1d(np.arange(N), rows)
    assert not got[others].any()


def _q8_decode_layer(d, c, k, lens, Nmax, x, rotate):
    """Fill two Q8_0 caches by appends (rotated or not), rotate the weights on the GPU when
    asked, then absorb -> decode -> out_proj through the C ABI.  Returns out [2, D]."""
    from deepseek_mla_amd import mla
    cd = mla.make_dims(d)
    bt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
    W = d.kv_lora_rank + d.qk_rope
    cache = torch.zeros((2 * Nmax, W // 32 * 34), dtype=torch.uint8, device="cuda")
    pos = torch.from_numpy(np.tile(np.arange(Nmax, dtype=np.int32), 2)).to("cuda")
    append = mla.mla_cache_append_hadamard if rotate else mla.mla_cache_append
    dst = torch.arange(2 * Nmax, dtype=torch.int64, device="cuda")  # b * Nmax + pos
    append(cd, mla.BF16, mla.Q8_0, bt(c), bt(k), pos, 2 * Nmax, cache, 2 * Nmax, dst_row=dst)
    wk, wv = bt(x["wk_b"]), bt(x["wv_b"])
    if rotate:
        wk_r, wv_r = torch.empty_like(wk), torch.empty_like(wv)
        mla.mla_hadamard_weights(cd, mla.BF16, wk, wv, wk_r, wv_r)
        wk, wv = wk_r, wv_r
    qpos = torch.tensor([l - 1 for l in lens], dtype=torch.int32, device="cuda")
    H = d.n_head
    q_cat = torch.empty((2, H, W), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(cd, mla.BF16, bt(x["q_nope"]), bt(x["q_rope"]), qpos, wk, q_cat, 2)
    nkv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    wsb = mla.mla_decode_workspace_bytes(cd, 2, Nmax, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    o = torch.empty((2, H, d.kv_lora_rank), dtype=torch.bfloat16, device="cuda")
    mla.mla_attn_decode(cd, mla.BF16, mla.Q8_0, q_cat, cache, 612 * Nmax, nkv, 2, Nmax, 0, o,
                        None, ws, wsb)
    v = torch.empty((2, H * d.v_head), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((2, d.d_model), dtype=torch.bfloat16, device="cuda")
    mla.mla_out_proj(cd, mla.BF16, o, wv, bt(x["wo"]), v, out, 2)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("outliers", [False, True])
def test_hadamard_q8_0_decode_layer(dev, outliers):
    """V3 dims, two sequences (300 and 123 rows) written by appends into Q8_0 caches, plain
    and Hadamard-rotated (with rotated weights), decoded end to end through the C ABI.
    Parity: each against the oracle's layer over the oracle's own Q8_0 rows of the same
    kind (rotated rows with the oracle's rotated weights), within 2e-2.  Accuracy (the
    page's claim, reported): both against the exact layer over the unquantised rows; with
    four large latent channels the rotated cache must be the closer one."""
    d = synth.deepseek_dims(128, 7168)
    Nmax, lens = 300, [300, 123]
    W = 576
    rng = np.random.default_rng(97)
    c = rng.standard_normal((2 * Nmax, 512)).astype(np.float32)
    if outliers:
        c[:, rng.choice(512, size=4, replace=False)] *= 40.0
    c = synth.round_bf16(c)
    k = synth.round_bf16(rng.standard_normal((2 * Nmax, 64)).astype(np.float32))
    x = synth.generate(d, 1, 8, seed=98, n_seq=2, mode="bf16")
    pos = np.tile(np.arange(Nmax, dtype=np.int32), 2)
    qpos = [np.array([l - 1], np.int32) for l in lens]
    # the rotated weights as the layer holds them: bfloat16, rounded to nearest even
    wk_r, wv_r = (oracle.bf16_round(w) for w in oracle.hadamard_weights(d, x["wk_b"], x["wv_b"]))

    def layer(rows, wk, wv):
        return np.stack([oracle.mla_absorbed(d, x["q_nope"][b:b + 1], x["q_rope"][b:b + 1],
                                             qpos[b], rows[b * Nmax: b * Nmax + lens[b]], wk, wv,
                                             x["wo"])["out"][0] for b in range(2)])

    exact = layer(oracle.cache_rows_new(d, c, k, pos), x["wk_b"], x["wv_b"])
    acc = {}
    for rotate in (False, True):
        got = _q8_decode_layer(d, c, k, lens, Nmax, x, rotate)
        rows = (oracle.cache_rows_new_hadamard if rotate else oracle.cache_rows_new)(d, c, k, pos)
        rows = oracle.q8_0_dequantize(oracle.q8_0_quantize(rows), W)
        ref = layer(rows, wk_r, wv_r) if rotate else layer(rows, x["wk_b"], x["wv_b"])
        tag = "rotated" if rotate else "plain"
        report(f"out ({tag} Q8_0 cache, parity)", rel_err_stored(got, ref, "q8_0"), 2e-2)
        acc[rotate] = rel_err(got, exact)
        print(f"  out ({tag} Q8_0 cache) vs the exact layer: max|diff|/rms = {acc[rotate]:.3e}",
              flush=True)
    if outliers:
        assert acc[True] < acc[False]


# ------------------------------------------------------ merged wkv_b layout ---

@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_wkv_b_merge_split(dev, mode):
    """Merge (as act and as Q8_0) and split (from both) against the oracle's layout, bit
    for bit: pure data movement, the Q8_0 rows by the shared quantiser rule, the Q8_0
    split as d*q rounded to act."""
    from deepseek_mla_amd import mla
    d = synth.TINY if mode == "f32" else synth.deepseek_dims(16, 2048)
    x = synth.generate(d, 1, 4, seed=102, mode=mode)
    tdt = torch.float32 if mode == "f32" else torch.bfloat16
    act = mla.F32 if mode == "f32" else mla.BF16
    cd = mla.make_dims(d)
    H, R, Dn, Dv = d.n_head, d.kv_lora_rank, d.qk_nope, d.v_head
    wk = torch.from_numpy(x["wk_b"]).to(dev).to(tdt)
    wv = torch.from_numpy(x["wv_b"]).to(dev).to(tdt)
    ref = oracle.wkv_b_merge(d, x["wk_b"], x["wv_b"])
    merged = torch.empty((H, Dn + Dv, R), dtype=tdt, device=dev)
    mla.mla_wkv_b_merge(cd, act, act, wk, wv, merged)
    merged_q8 = torch.empty((H, Dn + Dv, R // 32 * 34), dtype=torch.uint8, device=dev)
    mla.mla_wkv_b_merge(cd, act, mla.Q8_0, wk, wv, merged_q8)
    torch.cuda.synchronize()
    assert np.array_equal(merged.float().cpu().numpy(), ref)
    ref_q8 = oracle.q8_0_quantize(ref)
    assert np.array_equal(merged_q8.cpu().numpy(), ref_q8)
    for src, kind in ((merged, act), (merged_q8, mla.Q8_0)):
        gk, gv = torch.empty_like(wk), torch.empty_like(wv)
        mla.mla_wkv_b_split(cd, kind, act, src, gk, gv)
        torch.cuda.synchronize()
        if kind == mla.Q8_0:
            deq = oracle.q8_0_dequantize(ref_q8, R)
            if mode == "bf16":
                deq = oracle.bf16_round(deq)
            want_k, want_v = oracle.wkv_b_split(d, deq)
        else:
            want_k, want_v = x["wk_b"], x["wv_b"]
        assert np.array_equal(gk.float().cpu().numpy(), want_k)
        assert np.array_equal(gv.float().cpu().numpy(), want_v)


# --------------------------------------------- cut prefill: workspace, empty rows ---

def test_bf16_prefill_cut_poisoned_workspace_and_empty_groups(dev):
    """A prefill that cuts its row groups into key parts, with a workspace filled with
    0x7f bytes (the caller need not initialise it): groups whose keys fit one part must not
    be merged from stale slots.  The first 130 tokens sit at position -1, so whole row
    groups see no key: their rows are zero and their lse -inf."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    T, N = 200, 333
    pos = np.arange(N - T, N, dtype=np.int32)
    pos[:130] = -1
    x, rows = small_prefill(d, "bf16", T, N, seed=111, pos=pos)
    ref = oracle_chain(d, x, rows)
    cd = mla.make_dims(d)
    nb = mla.mla_prefill_workspace_bytes(cd, mla.BF16, T, N, 0)
    assert nb > 0  # the cut mode
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device=dev)
    q_cat = torch.from_numpy(synth.round_bf16(ref["q_cat"])).to(dev).to(torch.bfloat16)
    cache = torch.from_numpy(rows).to(dev).to(torch.bfloat16)
    o = torch.empty((T, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, 16), dtype=torch.float32, device=dev)
    mla.mla_attn_prefill(cd, mla.BF16, mla.BF16, q_cat, torch.from_numpy(pos).to(dev), T, cache, N,
                         o, lse, 0, ws)
    torch.cuda.synchronize()
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.attention(d, synth.round_bf16(ref["q_cat"]), pos, rows)
    assert (got_o[:130] == 0).all() and np.isneginf(got_l[:130]).all()
    report("o_lat", rel_err_stored(got_o[130:], ro[130:], "bf16"), TOL["bf16"])
    report("lse (abs)", float(np.abs(got_l[130:] - rl[130:]).max()), TOL["bf16"])


# ------------------------------------------------- decode of many sequences ---

@pytest.mark.parametrize("B", [16, 40])
def test_decode_many_sequences(dev, B):
    """bf16 decode at V3 dims with B >= 16 sequences of different lengths (the batched-cache
    prefill kernel with key parts), against the oracle on sampled heads of every sequence and
    against the split decode kernel (explicit split count) on all heads."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(112 + B)
    Nmax = 1500
    lens = rng.integers(1, Nmax + 1, size=B).astype(np.int32)
    lens[0], lens[1] = Nmax, 1
    W = 576
    cache_f = synth.round_bf16(rng.standard_normal((B, Nmax, W)).astype(np.float32))
    q = synth.round_bf16(rng.standard_normal((B, 128, W)).astype(np.float32))
    cd = mla.make_dims(d)
    cache = torch.from_numpy(cache_f).to(dev).to(torch.bfloat16)
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16)
    nkv = torch.from_numpy(lens).to(dev)
    outs = []
    for ns in (0, 7):
        wsb = mla.mla_decode_workspace_bytes(cd, B, Nmax, ns)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        o = torch.empty((B, 128, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, 128), dtype=torch.float32, device=dev)
        mla.mla_attn_decode(cd, mla.BF16, mla.BF16, qd, cache, Nmax * W * 2, nkv, B, Nmax, ns, o,
                            lse, ws, wsb)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), lse.cpu().numpy()))
    heads = np.arange(0, 128, 16)
    for b in range(B):
        ro, rl = oracle.attention(d, q[b:b + 1][:, heads], np.array([lens[b] - 1], np.int32),
                                  cache_f[b, :lens[b]])
        report(f"o_lat seq {b}", rel_err_stored(outs[0][0][b][heads], ro[0], "bf16"), TOL["bf16"])
        assert np.abs(outs[0][1][b][heads] - rl[0]).max() <= TOL["bf16"]
    # two GPU results, each within TOL of the exact one (the split kernel's parity is tested
    # on its own above): they may differ by the sum
    report("o_lat vs split kernel", rel_err_stored(outs[0][0], outs[1][0], "bf16"), 2 * TOL["bf16"])


def test_decode_many_sequences_full_size(dev):
    """16 V3 sequences of 32768 bf16 rows (the batched-cache decode at the size the decode
    sweep times): every sequence against the oracle on 4 sampled heads."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    B, N, W = 16, 32768, 576
    g = torch.Generator(device="cpu").manual_seed(113)
    cache_f = synth.round_bf16(torch.randn((B, N, W), generator=g).numpy())
    q = synth.round_bf16(torch.randn((B, 128, W), generator=g).numpy())
    lens = np.full(B, N, np.int32)
    lens[3], lens[9] = 17, 20000
    cd = mla.make_dims(d)
    cache = torch.from_numpy(cache_f).to(dev).to(torch.bfloat16)
    wsb = mla.mla_decode_workspace_bytes(cd, B, N, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    o = torch.empty((B, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, 128), dtype=torch.float32, device=dev)
    mla.mla_attn_decode(cd, mla.BF16, mla.BF16, torch.from_numpy(q).to(dev).to(torch.bfloat16),
                        cache, N * W * 2, torch.from_numpy(lens).to(dev), B, N, 0, o, lse, ws, wsb)
    torch.cuda.synchronize()
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    heads = np.array([0, 37, 90, 127])
    for b in range(B):
        ro, rl = oracle.attention(d, q[b:b + 1][:, heads], np.array([lens[b] - 1], np.int32),
                                  cache_f[b, :lens[b]])
        report(f"o_lat seq {b}", rel_err_stored(got_o[b][heads], ro[0], "bf16"), TOL["bf16"])
        assert np.abs(got_l[b][heads] - rl[0]).max() <= TOL["bf16"]
