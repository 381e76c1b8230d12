"""GPU pins with exact answers: attention whose softmax weights are all equal.

With a single visible key (n_kv = 1, or every query at position 0), or with every visible
key holding the same row, every weight of a row's softmax is equal, so the latent output
is exactly that row's first R values: o_lat = sum_j p c / sum_j p = c.  The attention
kernels hold the cache rows in bfloat16 on their way into the matrix cores, so the answer
is bit-exact:
  * bf16 cache: o_lat equals the stored row, bit for bit;
  * Q8_0 cache: o_lat equals bf16_round(oracle.q8_0_dequantize(row))[:R] bit for bit, which
    pins the dequantisation inside the decode kernel's load path (scale times code, exact
    in float32, then the bf16 rounding of the tile) on both of its copy paths: dword
    copies of a tile that reaches past the sequence end, and 16-byte copies of tiles inside
    it.
lse is s + ln(n) for n equal scores s of the values the kernel holds (the bf16 row, or
the bf16 rounding of the dequantised row); it is compared within the float32 accumulation
error of the score (the sum of 576 products in some order).

The rows span a wide dynamic range (block maxima from 1e-6 to 1e3, so binary16 scales
from subnormal to large), with zero blocks and codes of +-127.
"""
import numpy as np
import pytest

import oracle
from deepseek_mla_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W, R = 576, 512


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from deepseek_mla_amd import mla
    mla.lib()
    return "cuda"


def wide_rows(rng, n):
    """n float32 rows of 576 values: each 32-value block a normal draw scaled to a maximum
    of 10^U(-6, 3); a few all-zero blocks."""
    x = rng.standard_normal((n, W // 32, 32))
    x /= np.abs(x).max(axis=-1, keepdims=True)
    x *= 10.0 ** rng.uniform(-6, 3, size=(n, W // 32, 1))
    x[rng.random((n, W // 32)) < 0.05] = 0.0
    return x.reshape(n, W).astype(np.float32)


def expected_rows(rows_f, mode):
    """What o_lat must hold for a row: the bf16 row itself, or the bf16 rounding of its
    Q8_0 dequantisation (oracle)."""
    if mode == "bf16":
        return synth.round_bf16(rows_f)
    return oracle.bf16_round(oracle.q8_0_dequantize(oracle.q8_0_quantize(rows_f), W))


def lse_bound(q, row, scale, n):
    """lse of n equal scores s = scale * q . row, and a bound on its float32 error."""
    q64, r64 = q.astype(np.float64), row.astype(np.float64)
    s = scale * (q64 * r64).sum(axis=-1)
    mag = scale * np.abs(q64 * r64).sum(axis=-1)
    return s + np.log(n), 2.0 * W * 2.0 ** -24 * mag + 4.0 * 2.0 ** -24 * np.abs(s) + 1e-6


def run_decode(d, q, caches, stride, lens, n_kv_max, mode, ns):
    from deepseek_mla_amd import mla
    B, H = q.shape[0], q.shape[1]
    cd = mla.make_dims(d)
    wsb = mla.mla_decode_workspace_bytes(cd, B, n_kv_max, ns)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, R), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    kv = mla.Q8_0 if mode == "q8_0" else mla.BF16
    mla.mla_attn_decode(cd, mla.BF16, kv, torch.from_numpy(q).to("cuda").to(torch.bfloat16),
                        caches, stride, torch.tensor(lens, dtype=torch.int32, device="cuda"), B,
                        n_kv_max, ns, o, lse, ws, wsb)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def pack(rows_per_seq, mode, n_kv_max):
    """Device cache of B sequences (rows_per_seq: list of float32 [n, 576]) and its stride."""
    B = len(rows_per_seq)
    if mode == "q8_0":
        stride = (612 * n_kv_max + 15) // 16 * 16
        buf = np.zeros((B, stride), np.uint8)
        for b, r in enumerate(rows_per_seq):
            qb = oracle.q8_0_quantize(r).reshape(-1)
            buf[b, :qb.size] = qb
        return torch.from_numpy(buf).to("cuda"), stride
    buf = np.zeros((B, n_kv_max, W), np.float32)
    for b, r in enumerate(rows_per_seq):
        buf[b, :r.shape[0]] = synth.round_bf16(r)
    return torch.from_numpy(buf).to("cuda").to(torch.bfloat16), n_kv_max * W * 2


def check_equal_weights(name, o, lse, want, q, row_for_lse, d, n):
    """o [H, R] must equal want [R] in every head; lse within the accumulation bound."""
    bad = int((o != want[None, :R]).sum())
    lt, tol = lse_bound(q, row_for_lse[None, :], d.scale, n)
    lerr = float((np.abs(lse - lt) / tol).max())
    print(f"  {name}: o_lat elements differing {bad} of {o.size}; lse max err / bound "
          f"{lerr:.3f}", flush=True)
    assert bad == 0, name
    assert lerr <= 1.0, name


@pytest.mark.parametrize("mode", ["bf16", "q8_0"])
@pytest.mark.parametrize("ns", [1, 3])
def test_decode_single_row(dev, mode, ns):
    """8 sequences of one row each, n_kv_max 200 (splits 1 and 3; with 3 splits of 96 keys
    the row's split holds one row and the other two none): o_lat is the row, bit for bit.
    The split's only tile reaches past the sequence end, so Q8_0 rows take the dword
    copies."""
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(201 + ns)
    B, n_kv_max = 8, 200
    rows_f = wide_rows(rng, B)
    want = expected_rows(rows_f, mode)
    q = synth.round_bf16(rng.standard_normal((B, 128, W)).astype(np.float32))
    cache, stride = pack([rows_f[b:b + 1] for b in range(B)], mode, n_kv_max)
    o, lse = run_decode(d, q, cache, stride, [1] * B, n_kv_max, mode, ns)
    for b in range(B):
        check_equal_weights(f"{mode} splits={ns} seq {b}", o[b], lse[b], want[b], q[b],
                            want[b], d, 1)


@pytest.mark.parametrize("mode", ["bf16", "q8_0"])
@pytest.mark.parametrize("n", [64, 77])
def test_decode_identical_rows(dev, mode, n):
    """2 sequences whose n rows are all one row (64: two whole tiles, the 16-byte Q8_0
    copies; 77: two whole tiles and a tail tile), one and two splits (77 rows in two
    splits: 64 rows of whole tiles, then a split of 13 rows in one tail tile)."""
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(211 + n)
    rows_f = wide_rows(rng, 2)
    want = expected_rows(rows_f, mode)
    q = synth.round_bf16(rng.standard_normal((2, 128, W)).astype(np.float32) * 0.05)
    seqs = [np.repeat(rows_f[b:b + 1], n, axis=0) for b in range(2)]
    cache, stride = pack(seqs, mode, n)
    for ns in (1, 2):
        o, lse = run_decode(d, q, cache, stride, [n, n], n, mode, ns)
        for b in range(2):
            check_equal_weights(f"{mode} n={n} splits={ns} seq {b}", o[b], lse[b], want[b], q[b],
                                want[b], d, n)


def test_decode_single_row_many_sequences(dev):
    """16 sequences of one row each with the automatic split count: the decode of many
    sequences that runs on the prefill kernel over the batched caches (bf16)."""
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(221)
    B, n_kv_max = 16, 1500
    rows_f = wide_rows(rng, B)
    want = expected_rows(rows_f, "bf16")
    q = synth.round_bf16(rng.standard_normal((B, 128, W)).astype(np.float32))
    cache, stride = pack([rows_f[b:b + 1] for b in range(B)], "bf16", n_kv_max)
    o, lse = run_decode(d, q, cache, stride, [1] * B, n_kv_max, "bf16", 0)
    for b in range(B):
        check_equal_weights(f"bf16 B=16 seq {b}", o[b], lse[b], want[b], q[b], want[b], d, 1)


@pytest.mark.parametrize("T,N", [(5, 1), (200, 333)])
def test_prefill_single_key(dev, T, N):
    """Prefill with every query at position 0 (Lite dims; N = 333 also runs the cut mode's
    work lists): each row sees key 0 only, so o_lat is row 0, bit for bit."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    rng = np.random.default_rng(231 + T)
    rows_f = np.concatenate([wide_rows(rng, 1),
                             rng.standard_normal((N - 1, W)).astype(np.float32)])
    rows = synth.round_bf16(rows_f)
    q = synth.round_bf16(rng.standard_normal((T, 16, W)).astype(np.float32))
    pos = np.zeros(T, np.int32)
    cd = mla.make_dims(d)
    o = torch.empty((T, 16, R), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 16), dtype=torch.float32, device="cuda")
    mla.mla_attn_prefill(cd, mla.BF16, mla.BF16, torch.from_numpy(q).to("cuda").to(torch.bfloat16),
                         torch.from_numpy(pos).to("cuda"), T,
                         torch.from_numpy(rows).to("cuda").to(torch.bfloat16), N, o, lse)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for t in range(T):
        check_equal_weights(f"prefill T={T} N={N} token {t}", o[t], lse[t], rows[0], q[t],
                            rows[0], d, 1)
