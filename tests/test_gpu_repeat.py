"""Run-to-run determinism and write bounds of the attention calls (GPU).

* Determinism: every attention path reduces in a fixed order (no floating-point atomics),
  so repeated calls on the same inputs return the same bits, also when the workspace is
  filled with random bytes between the calls (nothing may depend on its stale contents).
* Write bounds: outputs and workspaces are views into larger buffers whose guard bands
  (4 KB before and after) hold a byte pattern; after every call the guards must hold it
  unchanged.  The workspace view is exactly the size the library asked for, so the check
  also pins the workspace-size functions.  A stray write would land in a guard of the same
  allocation, so the check itself cannot fault.

Paths: the Lite-shaped prefill with cut row groups (work lists and the merge), the bf16
split decode, the Q8_0 decode (128 heads per workgroup), the batched decode that runs on
the prefill kernel, the K + V^T decode, the float32 decode and the materialised prefill;
then the projections (absorb and out-proj, few-token and GEMM kernels), the cache append
(bf16, Q8_0, Hadamard-rotated Q8_0: only the target rows may change) and the Q8_0 helpers.
"""
import numpy as np
import pytest

import oracle
from deepseek_mla_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W, R = 576, 512
GUARD = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from deepseek_mla_amd import mla
    mla.lib()
    return "cuda"


class Guarded:
    """A view of `shape` inside a byte buffer with GUARD bytes of PATTERN on each side."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.buf = torch.full((self.n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def intact(self):
        g = torch.cat([self.buf[:GUARD], self.buf[GUARD + self.n:]])
        return int((g != PATTERN).sum())

    def poison(self, gen):
        self.buf[GUARD:GUARD + self.n] = torch.randint(0, 256, (self.n,), dtype=torch.uint8,
                                                       device="cuda", generator=gen)


def workspace(nbytes):
    return Guarded((max(nbytes, 1),), torch.uint8)


def repeat_check(name, run, outs, ws, reps=3):
    """run() fills outs (Guarded views); compare every rep's bits with the first's, with
    the workspace and the outputs filled with fresh random bytes before each rep (so an
    output element left unwritten shows up as a difference), and check every guard after
    each rep."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    first = None
    for rep in range(reps):
        if ws is not None:
            ws.poison(gen)
        for o in outs:
            o.poison(gen)
        run()
        torch.cuda.synchronize()
        bits = [o.buf[GUARD:GUARD + o.n].cpu().numpy().copy() for o in outs]
        bad = sum(o.intact() for o in outs) + (ws.intact() if ws is not None else 0)
        diff = 0 if first is None else sum(int((a != b).sum()) for a, b in zip(bits, first))
        print(f"  {name} rep {rep}: guard bytes changed {bad}, bytes differing from rep 0 {diff}",
              flush=True)
        assert bad == 0, name
        assert diff == 0, name
        if first is None:
            first = bits


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch.bfloat16)


def test_prefill_cut_groups_repeat(dev):
    """Lite dims, 700 queries at 800..1499 over 1500 rows: row groups cut into key parts,
    per-CU work lists, partial rows in the workspace and the merge."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    rng = np.random.default_rng(401)
    T, N, H = 700, 1500, 16
    q = bf16_dev(rng.standard_normal((T, H, W)) * 0.5)
    cache = bf16_dev(rng.standard_normal((N, W)))
    pos = torch.arange(N - T, N, dtype=torch.int32, device="cuda")
    cd = mla.make_dims(d)
    wsb = mla.mla_prefill_workspace_bytes(cd, mla.BF16, T, N)
    assert wsb > 0  # the cut mode is what this test is about
    ws = workspace(wsb)
    o = Guarded((T, H, R), torch.bfloat16)
    lse = Guarded((T, H), torch.float32)

    def run():
        mla.mla_attn_prefill(cd, mla.BF16, mla.BF16, q, pos, T, cache, N, o.t, lse.t,
                             workspace=ws.t[:wsb])

    repeat_check("prefill (cut groups)", run, [o, lse], ws)


def _decode_inputs(rng, B, H, lens, n_max, mode):
    q = bf16_dev(rng.standard_normal((B, H, W)) * 0.3)
    rows = [rng.standard_normal((n, W)).astype(np.float32) for n in lens]
    if mode == "q8_0":
        stride = (612 * n_max + 15) // 16 * 16
        buf = np.zeros((B, stride), np.uint8)
        for b, r in enumerate(rows):
            qb = oracle.q8_0_quantize(r).reshape(-1)
            buf[b, :qb.size] = qb
        return q, torch.from_numpy(buf).to("cuda"), stride
    pad = np.zeros((B, n_max, W), np.float32)
    for b, r in enumerate(rows):
        pad[b, :r.shape[0]] = r
    return q, bf16_dev(pad), n_max * W * 2


@pytest.mark.parametrize("mode,B,n_splits", [("bf16", 2, 0), ("bf16", 2, 5), ("q8_0", 2, 0),
                                             ("q8_0", 3, 7), ("bf16", 16, 0)])
def test_decode_repeat(dev, mode, B, n_splits):
    """V3 dims (128 heads), ragged lengths: the 64-head split decode (bf16), the 128-head
    Q8_0 decode, and (B = 16, automatic splits) the decode on the prefill kernel."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(411 + B + n_splits)
    lens = [int(x) for x in rng.integers(200, 2100, size=B)]
    n_max = 2100
    q, cache, stride = _decode_inputs(rng, B, 128, lens, n_max, mode)
    kv = mla.Q8_0 if mode == "q8_0" else mla.BF16
    cd = mla.make_dims(d)
    nkv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    wsb = mla.mla_decode_workspace_bytes(cd, B, n_max, n_splits)
    ws = workspace(wsb)
    o = Guarded((B, 128, R), torch.bfloat16)
    lse = Guarded((B, 128), torch.float32)

    def run():
        mla.mla_attn_decode(cd, mla.BF16, kv, q, cache, stride, nkv, B, n_max, n_splits, o.t,
                            lse.t, ws.t, wsb)

    repeat_check(f"decode {mode} B={B} splits={n_splits}", run, [o, lse], ws)


def test_decode_vt_repeat(dev):
    """The K + V^T decode: every cache row transposed into a guarded V^T buffer, then the
    decode that reads it (the second sequence ends inside a tile)."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(421)
    B, n_max = 2, 1000
    lens = [1000, 613]
    q, cache, stride = _decode_inputs(rng, B, 128, lens, n_max, "bf16")
    cd = mla.make_dims(d)
    ld = (n_max + 31) // 32 * 32
    vt = Guarded((B, R, ld), torch.bfloat16)
    mla.mla_cache_transpose_v(cd, mla.BF16, cache, stride, B, 0, n_max, vt.t, R * ld * 2, ld)
    torch.cuda.synchronize()
    assert vt.intact() == 0
    nkv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    wsb = mla.mla_decode_workspace_bytes(cd, B, n_max, 0)
    ws = workspace(wsb)
    o = Guarded((B, 128, R), torch.bfloat16)
    lse = Guarded((B, 128), torch.float32)

    def run():
        mla.mla_attn_decode_vt(cd, mla.BF16, mla.BF16, q, cache, stride, vt.t, R * ld * 2, ld,
                               nkv, B, n_max, 0, o.t, lse.t, ws.t, wsb)

    repeat_check("decode K + V^T", run, [o, lse], ws)
    assert vt.intact() == 0


def test_decode_f32_repeat(dev):
    """The float32 path (tiny dims): float32 partials and combine."""
    from deepseek_mla_amd import mla
    d = synth.TINY
    Wt = d.kv_lora_rank + d.qk_rope
    rng = np.random.default_rng(431)
    B, n_max, H = 3, 300, d.n_head
    lens = [300, 1, 157]
    q = torch.from_numpy(rng.standard_normal((B, H, Wt)).astype(np.float32)).to("cuda")
    cache = torch.from_numpy(rng.standard_normal((B, n_max, Wt)).astype(np.float32)).to("cuda")
    cd = mla.make_dims(d)
    nkv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    wsb = mla.mla_decode_workspace_bytes(cd, B, n_max, 4)
    ws = workspace(wsb)
    o = Guarded((B, H, d.kv_lora_rank), torch.float32)
    lse = Guarded((B, H), torch.float32)

    def run():
        mla.mla_attn_decode(cd, mla.F32, mla.F32, q, cache, n_max * Wt * 4, nkv, B, n_max, 4,
                            o.t, lse.t, ws.t, wsb)

    repeat_check("decode f32", run, [o, lse], ws)


def test_materialized_repeat(dev):
    """The materialised prefill (Lite dims, 1200 queries over 2048 rows under a 128 MiB cap:
    the heads run in chunks): its decompressed K and V in the workspace, the attention and
    wo."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    T, N, H = 1200, 2048, 16
    x = synth.generate(d, T, N, seed=441, mode="bf16",
                       pos=np.arange(N - T, N, dtype=np.int32))
    to = lambda a: bf16_dev(a)  # noqa: E731
    q_nope, q_rope = to(x["q_nope"]), to(x["q_rope"])
    cache = to(synth.cache_rows(x["c_kv"][0], x["k_rope"][0]))
    wk_b, wv_b, wo = to(x["wk_b"]), to(x["wv_b"]), to(x["wo"])
    pos = torch.from_numpy(x["pos"]).to("cuda")
    cd = mla.make_dims(d)
    cap = 128  # MiB: below the whole problem's T*N*H*4 B, so the heads run in chunks
    assert mla.mla_heads_per_chunk(H, T * N * H * 4 / 2 ** 20, cap) < H
    wsb = mla.mla_materialized_workspace_bytes(cd, T, N, cap)
    ws = workspace(wsb)
    v = Guarded((T, H * 128), torch.bfloat16)
    out = Guarded((T, 2048), torch.bfloat16)
    lse = Guarded((T, H), torch.float32)

    def run():
        mla.mla_prefill_materialized(cd, mla.BF16, mla.BF16, q_nope, q_rope, pos, T, cache, N,
                                     wk_b, wv_b, v.t, wo=wo, out=out.t, lse=lse.t,
                                     scratch_cap_mib=cap, workspace=ws.t[:wsb])

    repeat_check("materialised prefill", run, [v, out, lse], ws)


@pytest.mark.parametrize("T", [5, 300])
def test_projections_repeat(dev, T):
    """mla_absorb_q and mla_out_proj (Lite dims; T = 5 takes the few-token kernels):
    q_cat, v and out bitwise repeatable, fully written, guards intact."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    x = synth.generate(d, T, T, seed=451 + T, mode="bf16")
    q_nope, q_rope, wk_b = bf16_dev(x["q_nope"]), bf16_dev(x["q_rope"]), bf16_dev(x["wk_b"])
    wv_b, wo = bf16_dev(x["wv_b"]), bf16_dev(x["wo"])
    pos = torch.from_numpy(x["pos"]).to("cuda")
    o_lat = bf16_dev(np.random.default_rng(452).standard_normal((T, 16, R)) * 0.2)
    cd = mla.make_dims(d)
    q_cat = Guarded((T, 16, W), torch.bfloat16)
    v = Guarded((T, 16 * 128), torch.bfloat16)
    out = Guarded((T, 2048), torch.bfloat16)
    repeat_check(f"absorb T={T}",
                 lambda: mla.mla_absorb_q(cd, mla.BF16, q_nope, q_rope, pos, wk_b, q_cat.t, T),
                 [q_cat], None)
    repeat_check(f"out_proj T={T}",
                 lambda: mla.mla_out_proj(cd, mla.BF16, o_lat, wv_b, wo, v.t, out.t, T),
                 [v, out], None)


@pytest.mark.parametrize("mode,hadamard", [("bf16", False), ("q8_0", False), ("q8_0", True)])
def test_cache_append_bounds(dev, mode, hadamard):
    """mla_cache_append (and the Hadamard-rotated form) into a cache of random bytes: only
    the target rows change, the guards around the cache stay intact, and a second append of
    the same tokens writes the same bits."""
    from deepseek_mla_amd import mla
    d = synth.deepseek_dims(16, 2048)
    rng = np.random.default_rng(461)
    T, n_rows = 37, 300
    pos = rng.choice(n_rows, size=T, replace=False).astype(np.int32)
    c_kv = bf16_dev(rng.standard_normal((T, R)))
    k_rope = bf16_dev(rng.standard_normal((T, 64)))
    pt = torch.from_numpy(pos).to("cuda")
    row_bytes = 612 if mode == "q8_0" else W * 2
    cache = Guarded((n_rows, row_bytes), torch.uint8)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(462)
    cache.poison(gen)
    before = cache.t.cpu().numpy().copy()
    kv = mla.Q8_0 if mode == "q8_0" else mla.BF16
    call = mla.mla_cache_append_hadamard if hadamard else mla.mla_cache_append
    target = np.zeros(n_rows, bool)
    target[pos] = True
    first = None
    for rep in range(2):
        call(mla.make_dims(d), mla.BF16, kv, c_kv, k_rope, pt, T, cache.t, n_rows)
        torch.cuda.synchronize()
        after = cache.t.cpu().numpy()
        changed_other = int((after[~target] != before[~target]).sum())
        diff = 0 if first is None else int((after[target] != first).sum())
        print(f"  append {mode}{' hadamard' if hadamard else ''} rep {rep}: other rows' bytes "
              f"changed {changed_other}, guard bytes changed {cache.intact()}, target bytes "
              f"differing from rep 0 {diff}", flush=True)
        assert changed_other == 0 and cache.intact() == 0 and diff == 0
        if first is None:
            first = after[target].copy()


def test_q8_0_helpers_bounds(dev):
    """mla_quantize_q8_0 and mla_dequant_q8_0 on 333 rows: outputs fully written and
    repeatable, guards intact."""
    from deepseek_mla_amd import mla
    rng = np.random.default_rng(471)
    n = 333
    x = torch.from_numpy(rng.standard_normal((n, W)).astype(np.float32)).to("cuda")
    rows = Guarded((n, 612), torch.uint8)
    repeat_check("quantize", lambda: mla.mla_quantize_q8_0(x, rows.t, n, W), [rows], None)
    out = Guarded((n, W), torch.float32)
    repeat_check("dequant", lambda: mla.mla_dequant_q8_0(rows.t, out.t, n, W), [out], None)
