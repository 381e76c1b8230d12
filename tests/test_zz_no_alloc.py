"""mla_attn_decode_static (the allocation-free decode, its workspace a device array of the
library) against mla_attn_decode with a caller workspace: same kernels, so the outputs
must agree bit for bit, and both against the oracle within the bf16 / Q8_0 tolerance.
Two calls in a row, the second smaller than the first (the array keeps the first call's
partials, which must not leak into the second)."""
import numpy as np
import pytest

import oracle
from deepseek_mla_amd import synth
from oracle import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from deepseek_mla_amd import mla
    mla.lib()
    return "cuda"


def _case(mode, B, lens, Nmax, seed):
    d = synth.deepseek_dims(128, 7168)
    rng = np.random.default_rng(seed)
    rows = [synth.round_bf16(rng.standard_normal((n, 576)).astype(np.float32)) for n in lens]
    q = synth.round_bf16(rng.standard_normal((B, 128, 576)).astype(np.float32) * 0.5)
    if mode == "q8_0":
        stride = (612 * Nmax + 15) // 16 * 16
        buf = np.zeros((B, stride), np.uint8)
        for b, r in enumerate(rows):
            qb = oracle.q8_0_quantize(r).reshape(-1)
            buf[b, :qb.size] = qb
        ref_rows = [oracle.q8_0_dequantize(oracle.q8_0_quantize(r), 576) for r in rows]
        cache = torch.from_numpy(buf).to("cuda")
    else:
        stride = Nmax * 1152
        buf = np.zeros((B, Nmax, 576), np.float32)
        for b, r in enumerate(rows):
            buf[b, :r.shape[0]] = r
        ref_rows = rows
        cache = torch.from_numpy(buf).to("cuda").to(torch.bfloat16)
    return d, q, cache, stride, ref_rows


def _run(fn, d, mode, q, cache, stride, lens, Nmax, ns):
    from deepseek_mla_amd import mla
    B = q.shape[0]
    cd = mla.make_dims(d)
    kv = mla.Q8_0 if mode == "q8_0" else mla.BF16
    o = torch.full((B, 128, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, 128), 7.0, dtype=torch.float32, device="cuda")
    qd = torch.from_numpy(q).to("cuda").to(torch.bfloat16)
    nkv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    if fn == "static":
        mla.mla_attn_decode_static(cd, mla.BF16, kv, qd, cache, stride, nkv, B, Nmax, ns, o, lse)
    else:
        wsb = mla.mla_decode_workspace_bytes(cd, B, Nmax, ns)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        mla.mla_attn_decode(cd, mla.BF16, kv, qd, cache, stride, nkv, B, Nmax, ns, o, lse, ws, wsb)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("mode", ["bf16", "q8_0"])
def test_static_decode_matches_workspace_decode(dev, mode):
    cases = [(3, [2000, 1500, 777], 2000, 0, 301), (2, [300, 41], 300, 3, 302)]
    for B, lens, Nmax, ns, seed in cases:  # the second call is smaller than the first
        d, q, cache, stride, ref_rows = _case(mode, B, lens, Nmax, seed)
        o_s, l_s = _run("static", d, mode, q, cache, stride, lens, Nmax, ns)
        o_w, l_w = _run("workspace", d, mode, q, cache, stride, lens, Nmax, ns)
        same = np.array_equal(o_s, o_w) and np.array_equal(l_s, l_w)
        print(f"  {mode} B={B} lens={lens} splits={ns}: static == workspace: {same}", flush=True)
        assert same
        for b in range(B):
            ro, rl = oracle.attention(d, q[b:b + 1], np.array([lens[b] - 1], np.int32),
                                      ref_rows[b])
            e = compare.row_error(o_s[b], ro[0], mode)
            print(f"    seq {b}: o_lat {e:.3e}, lse {np.abs(l_s[b] - rl[0]).max():.3e}", flush=True)
            assert e <= compare.TOL[mode]
            assert np.abs(l_s[b] - rl[0]).max() <= compare.TOL[mode]
