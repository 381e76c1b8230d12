"""The K + V^T cache form (absorption page, section 8.2: the -mla switch's mode 1 keeps a K
cache and a cache of V transposed): the transposition, and the decode that reads V^T.

* mla_cache_transpose_v is data movement: its output is checked bit for bit against the
  layout stated in the header (v_t[c][32 g + p] = row[32 g + pi(p)][c], pi swapping bits 2
  and 3), positions it must not touch keep their poison.
* mla_attn_decode_vt against the oracle (same tolerance as the bf16 decode), against
  mla_attn_decode on the same inputs, and bit for bit on caches whose softmax weights are
  all equal (o_lat is then the row itself).  The V^T rows past each sequence's end, and the
  cache rows past it, hold NaN: the kernel must not let them into the result.
"""
import numpy as np
import pytest

import oracle
from deepseek_mla_amd import synth
from oracle import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = compare.TOL["bf16"]
W, R = 576, 512
NAN16 = 0x7FC0  # a bf16 quiet NaN


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from deepseek_mla_amd import mla
    mla.lib()
    return "cuda"


def perm32(n):
    """Position -> key within each group of 32 (bits 2 and 3 swapped), for n positions."""
    p = np.arange(n)
    i = p & 31
    return (p & ~31) | (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1)


def bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def make_vt(d, cache, stride_rows, B, vt_ld, pieces):
    """v_t [B][512][vt_ld] bf16 filled with NaN, then transposed in the given row ranges."""
    from deepseek_mla_amd import mla
    vt = torch.full((B, R, vt_ld), 0, dtype=torch.int16, device="cuda")
    vt.fill_(NAN16)
    vt = vt.view(torch.bfloat16)
    cd = mla.make_dims(d)
    for r0, r1 in pieces:
        mla.mla_cache_transpose_v(cd, mla.BF16, cache, stride_rows * W * 2, B, r0, r1, vt,
                                  R * vt_ld * 2, vt_ld)
    torch.cuda.synchronize()
    return vt


def test_transpose_layout(dev):
    """Two sequences of 100 rows, transposed in pieces [0, 37), [37, 64), [64, 100) (row0
    inside a 32-key group); then a piece [100, 101) appended after a row is added."""
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(301)
    B, N, ld = 2, 104, 136
    rows = synth.round_bf16(rng.standard_normal((B, N, W)).astype(np.float32))
    cache = torch.from_numpy(rows).to("cuda").to(torch.bfloat16)
    vt = make_vt(d, cache, N, B, ld, [(0, 37), (37, 64), (64, 100)])
    got = bits_of(vt)
    src = synth.bf16_bits(rows)  # [B][N][W]
    key = perm32(ld)
    for n_written in (100, 101):
        if n_written == 101:
            make_vt_piece(d, cache, N, B, vt, ld, 100, 101)
            got = bits_of(vt)
        for b in range(B):
            for p in range(ld):
                k = key[p]
                if k < n_written:
                    assert (got[b, :, p] == src[b, k, :R]).all(), (b, p, k)
                else:
                    assert (got[b, :, p] == NAN16).all(), (b, p, k)
    print(f"  v_t of {B} x 101 rows: every position as the layout states", flush=True)


def make_vt_piece(d, cache, stride_rows, B, vt, vt_ld, r0, r1):
    from deepseek_mla_amd import mla
    mla.mla_cache_transpose_v(mla.make_dims(d), mla.BF16, cache, stride_rows * W * 2, B, r0, r1,
                              vt, R * vt_ld * 2, vt_ld)
    torch.cuda.synchronize()


def decode_both(d, qc, rows_pad, lens, Nmax, ns, vt_ld):
    """mla_attn_decode_vt and mla_attn_decode on the same inputs.  rows_pad [B][Nmax][576]
    float32 (bf16 values); rows past each length are replaced by NaN on the device."""
    from deepseek_mla_amd import mla
    B, H = qc.shape[0], qc.shape[1]
    cd = mla.make_dims(d)
    cache = torch.from_numpy(rows_pad).to("cuda").to(torch.bfloat16)
    vt = make_vt(d, cache, Nmax, B, vt_ld, [(0, Nmax)])
    for b in range(B):  # poison what lies past each sequence's end, in both caches
        cache[b, lens[b]:] = float("nan")
        past = torch.from_numpy(np.nonzero(perm32(vt_ld) >= lens[b])[0]).to("cuda")
        vt.view(torch.int16)[b][:, past] = NAN16
    qd = torch.from_numpy(qc).to("cuda").to(torch.bfloat16)
    nkv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    wsb = mla.mla_decode_workspace_bytes(cd, B, Nmax, ns)
    out = []
    for use_vt in (True, False):
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)  # NaN partials if anything is left unwritten
        o = torch.empty((B, H, R), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        if use_vt:
            mla.mla_attn_decode_vt(cd, mla.BF16, mla.BF16, qd, cache, Nmax * W * 2, vt,
                                   R * vt_ld * 2, vt_ld, nkv, B, Nmax, ns, o, lse, ws, wsb)
        else:
            mla.mla_attn_decode(cd, mla.BF16, mla.BF16, qd, cache, Nmax * W * 2, nkv, B, Nmax,
                                ns, o, lse, ws, wsb)
        torch.cuda.synchronize()
        out.append((o.float().cpu().numpy(), lse.cpu().numpy()))
    return out


def report(name, err, tol):
    print(f"  {name}: {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, name


@pytest.mark.parametrize("H", [128, 256, 16])
def test_decode_vt_ragged(dev, H):
    """3 sequences of 777, 301 and 33 rows (whole tiles, tail tiles, a split holding only a
    tail), split counts 1, 2, 3, 7 and automatic; 128 heads, 256 heads (two head groups),
    16 heads (one group, 112 of its rows unused)."""
    d = synth.deepseek_dims(H, 7168)
    rng = np.random.default_rng(311 + H)
    lens, Nmax = [777, 301, 33], 777
    rows = synth.round_bf16(rng.standard_normal((3, Nmax, W)).astype(np.float32))
    qc = synth.round_bf16(rng.standard_normal((3, H, W)).astype(np.float32) * 0.5)
    ref = [oracle.attention(d, qc[b:b + 1], np.array([lens[b] - 1], np.int32), rows[b, :lens[b]])
           for b in range(3)]
    for ns in (1, 2, 3, 7, 0):
        (ov, lv), (orow, lrow) = decode_both(d, qc, rows, lens, Nmax, ns, 800)
        for b in range(3):
            report(f"H={H} splits={ns} seq {b} o_lat vs oracle",
                   compare.row_error(ov[b], ref[b][0][0], "bf16"), TOL)
            report(f"H={H} splits={ns} seq {b} lse vs oracle",
                   float(np.abs(lv[b] - ref[b][1][0]).max()), TOL)
        # both within TOL of the exact result: they may differ by twice that
        report(f"H={H} splits={ns} o_lat vs mla_attn_decode",
               compare.row_error(ov, orow, "bf16"), 2 * TOL)


@pytest.mark.parametrize("n", [1, 77])
def test_decode_vt_equal_weights(dev, n):
    """8 sequences whose n rows (1, or 77 = two whole tiles and a tail) are one row: every
    softmax weight is equal and o_lat is that bf16 row, bit for bit, on 1 and 3 splits."""
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(321 + n)
    B, Nmax = 8, 200
    x = rng.standard_normal((B, W // 32, 32))
    x *= 10.0 ** rng.uniform(-6, 3, size=(B, W // 32, 1)) / np.abs(x).max(-1, keepdims=True)
    one = synth.round_bf16(x.reshape(B, W).astype(np.float32))
    rows = np.zeros((B, Nmax, W), np.float32)
    rows[:, :n] = one[:, None, :]
    qc = synth.round_bf16(rng.standard_normal((B, 128, W)).astype(np.float32) * 0.05)
    for ns in (1, 3):
        (ov, lv), _ = decode_both(d, qc, rows, [n] * B, Nmax, ns, 224)
        bad = int((ov != one[:, None, :R]).sum())
        print(f"  n={n} splits={ns}: o_lat elements differing {bad} of {ov.size}", flush=True)
        assert bad == 0
        s = d.scale * (qc.astype(np.float64) * one[:, None, :]).sum(-1) + np.log(n)
        mag = d.scale * np.abs(qc.astype(np.float64) * one[:, None, :]).sum(-1)
        assert (np.abs(lv - s) <= 2 * W * 2.0 ** -24 * mag + 4 * 2.0 ** -24 * np.abs(s)
                + 1e-6).all()


def test_decode_vt_full_size(dev):
    """The 32768-row V3 decode: a bf16 cache and its V^T copy, 128 heads, all heads against
    the oracle; and 4 sequences of 98304 rows (2^17 = vt_ld rounded up) on 8 sampled heads."""
    from deepseek_mla_amd import mla
    w = synth.WORKLOADS["v3_decode"]
    d = w.dims
    x = synth.generate_workload(w)
    qc = synth.round_bf16(oracle.absorb_q(d, x["q_nope"], x["q_rope"], x["pos"], x["wk_b"]))
    rows = synth.cache_rows(x["c_kv"][0], x["k_rope"][0])
    N = rows.shape[0]
    (ov, lv), (orow, _) = decode_both(d, qc, rows[None], [N], N, 0, N)
    ro, rl = oracle.attention(d, qc, x["pos"], rows)
    report("32768 rows o_lat vs oracle", compare.row_error(ov[0], ro[0], "bf16"), TOL)
    report("32768 rows lse vs oracle", float(np.abs(lv[0] - rl[0]).max()), TOL)
    report("32768 rows o_lat vs mla_attn_decode", compare.row_error(ov, orow, "bf16"), 2 * TOL)
    del ov, orow, x
    # 4 sequences, lengths ragged around the maximum
    g = torch.Generator(device="cpu").manual_seed(331)
    B, Nmax = 4, 98304
    cd = mla.make_dims(d)
    lens = np.array([Nmax, 98303, 65537, 17], np.int32)
    heads = np.array([0, 1, 31, 32, 63, 64, 100, 127])
    cache_f = synth.round_bf16(torch.randn((B, Nmax, W), generator=g).numpy())
    q = synth.round_bf16(torch.randn((B, 128, W), generator=g).numpy())
    ld = 98304
    cache = torch.from_numpy(cache_f).to("cuda").to(torch.bfloat16)
    vt = make_vt(d, cache, Nmax, B, ld, [(0, 50000), (50000, Nmax)])
    wsb = mla.mla_decode_workspace_bytes(cd, B, Nmax, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    o = torch.empty((B, 128, R), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 128), dtype=torch.float32, device="cuda")
    mla.mla_attn_decode_vt(cd, mla.BF16, mla.BF16, torch.from_numpy(q).to("cuda").to(torch.bfloat16),
                           cache, Nmax * W * 2, vt, R * ld * 2, ld, torch.from_numpy(lens).to("cuda"),
                           B, Nmax, 0, o, lse, ws, wsb)
    torch.cuda.synchronize()
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        ro, rl = oracle.attention(d, q[b:b + 1][:, heads], np.array([lens[b] - 1], np.int32),
                                  cache_f[b, :lens[b]])
        report(f"4 x 98304: seq {b} ({lens[b]} rows) o_lat",
               compare.row_error(got_o[b][heads], ro[0], "bf16"), TOL)
        report(f"4 x 98304: seq {b} lse", float(np.abs(got_l[b][heads] - rl[0]).max()), TOL)
