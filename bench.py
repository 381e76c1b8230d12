"""Benchmark: one absorbed-MLA layer step on one MI355X.

A step is the whole path on one batch of synthetic input already resident in HBM:
mla_absorb_q -> mla_attn_prefill (or mla_attn_decode) -> mla_out_proj.

Default workload (the headline line): the DeepSeek-V3-shaped long prefill (128 heads,
kv_lora_rank 512, rope 64, nope 128, v 128, d_model 7168; 8192 query tokens at positions
24576..32767, causal over a 32768-row bf16 latent cache, heads in -amb chunks under an
8192 MiB cap), the largest single-GPU configuration.  `value` is the metric's attention
TFLOP/s: the two-term score and the latent weighted sum priced per visible (query, key)
pair as in the absorption page's section 7 table (2 * (576 + 512) FLOP per head, a
multiply-add counted as 2), divided by the attention call's median duration (HIP events
on the launch stream).  The whole step's rate (absorption GEMM + attention + wv_b + wo
over the step's wall time) is reported beside it as `step_tflops`.

The other workloads run as entries under "workloads" (decode ones report latent-cache
GB/s of the attention kernels, prefill ones TFLOP/s); each entry carries its own roofline
object and the median / p10 / p90 of its per-iteration attention times.  Decode timing
rotates through several copies of the latent cache so that the 256 MB last-level cache
cannot hold it between steps.

`cpu_baseline` times the CPU oracle (test infrastructure) on this host's cores, threads
pinned, on the same workload: in full where it finishes in seconds, else on a fixed sample
whose time is extrapolated by visible-pair count (labelled so); a single-thread time on a
smaller sample is reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
MFMA_FLOP_PER_CLK = 256 * 4096  # chip-wide dense bf16 FLOP per clock

# HBM bytes per launch of the dominant kernel(s), from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes scaled by a 512 MiB copy (fetch x2.0, write x1.0); the summaries and commands are
# in profiles/.  Each figure is valid only for the kernel sources it was taken on (sha256
# prefix over the files listed, in order).
_CSRC = "deepseek_mla_amd/csrc/"
# the prefill kernel and its merge
PREFILL_SRC = tuple(_CSRC + f for f in ("flash_mfma.hip", "latent_tile.h", "lds_dma.h", "common.h"))
# the 64-head split decode and the combine
DECODE_SRC = tuple(_CSRC + f for f in ("decode_mfma.hip", "simt.hip", "latent_tile.h", "lds_dma.h",
                                       "common.h"))
# the 128-head split decode (Q8_0, K + V^T) and the combine
WIDE_DECODE_SRC = tuple(_CSRC + f for f in ("flash_mfma.hip", "simt.hip", "latent_tile.h",
                                            "lds_dma.h", "common.h"))
MATERIALIZED_SRC = tuple(_CSRC + f for f in ("flash_mha.hip", "latent_tile.h", "lds_dma.h",
                                             "common.h"))
TRAFFIC = {
    # workload: (bytes per launch, sources, sha256 prefix)
    "v3_long_prefill": (10849167437, PREFILL_SRC, "cf06df68df7e75e7"),
    "lite_prefill": (228780498, PREFILL_SRC, "cf06df68df7e75e7"),
    "v3_decode": (73657596, DECODE_SRC, "d3648251bb2fc5f5"),
    "v3_decode@vt": (141545802, WIDE_DECODE_SRC, "150288f17bf57c70"),
    "v3_decode_q8": (317920916, WIDE_DECODE_SRC, "150288f17bf57c70"),
    "v3_long_prefill@materialized": (3401259541, MATERIALIZED_SRC, "b55cdceb7076f3ef"),
}
# Sustained shader clock under each kernel's load (GHz): GRBM_GUI_ACTIVE cycles per
# dispatch over the dispatch's duration, from the counter summaries in profiles/; keyed
# like TRAFFIC.
CLOCK_GHZ = {
    "v3_long_prefill": (1.933, PREFILL_SRC, "cf06df68df7e75e7"),
    "v3_long_prefill@materialized": (1.921, MATERIALIZED_SRC, "b55cdceb7076f3ef"),
}


def _sources_sha(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _keyed(table, name):
    if name not in table:
        return None
    value, paths, sha = table[name]
    if _sources_sha(paths) != sha:
        return None  # kernels changed since the counters were taken
    return value


def measured_traffic(name):
    return _keyed(TRAFFIC, name)


def measured_clock(name):
    return _keyed(CLOCK_GHZ, name)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats(ms):
    ms = np.asarray(ms, np.float64)
    return {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
            "p90_ms": float(np.percentile(ms, 90)), "mean_ms": float(ms.mean()),
            "iterations": int(ms.size)}


def step_flops(w, pos) -> dict:
    from deepseek_mla_amd import accounting
    d = w.dims
    Q = len(pos)
    H, R, Dn, Dv, D = d.n_head, d.kv_lora_rank, d.qk_nope, d.v_head, d.d_model
    n_kv = w.n_kv
    if w.kind == "decode":
        attn = w.n_seq * n_kv * accounting.absorbed_flops_per_pair(d)
    else:
        attn = accounting.attention_flops(d, pos, n_kv)
    return {"absorb": 2 * Q * H * R * Dn, "attention": attn,
            "out_proj": 2 * Q * H * Dv * R + 2 * Q * D * H * Dv}


def attention_bytes(w) -> int:
    """Decode: latent rows of every sequence + q_cat and o_lat of every head (bf16)."""
    from deepseek_mla_amd import accounting
    d = w.dims
    W = d.kv_lora_rank + d.qk_rope
    row = accounting.q8_0_row_bytes(W) if w.mode == "q8_0" else W * 2
    return accounting.decode_bytes(d, w.n_kv, w.n_seq, row)


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """Measured device-to-device copy rate (read + write bytes per second, GB/s)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / s / 1e9


def time_workload(w, steps, warmup, copies=1, n_splits=0, path="absorbed"):
    import torch
    from deepseek_mla_amd import layer, synth
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x, cache_copies=copies, n_splits=n_splits, path=path)
    del x
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        L.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        L.absorb()
        e[1].record(stream)
        L.attend()
        e[2].record(stream)
        L.project()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    parts = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                      for e in ev])
    res = {"ms_per_step": wall * 1e3, "absorb_ms": float(np.median(parts[:, 0])),
           "attention_ms": float(np.median(parts[:, 1])),
           "out_proj_ms": float(np.median(parts[:, 2])), "attention_stats": stats(parts[:, 1])}
    res["cache_append"] = time_append(w, L, steps)
    if path == "vt":
        res["transpose_v_append"] = time_transpose_append(w, L, steps)
    pos = L.pos.cpu().numpy()
    del L
    torch.cuda.empty_cache()
    return res, pos


def time_append(w, L, reps):
    """mla_cache_append of the workload's new tokens (prefill: the T query tokens at their
    positions; decode: one token per sequence at its last row), timed on its own after
    the step (it is the call that precedes a step, not part of it)."""
    import torch
    from deepseek_mla_amd import mla
    d = w.dims
    R, Dr = d.kv_lora_rank, d.qk_rope
    W = R + Dr
    g = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    n_new = w.T if w.kind == "prefill" else w.n_seq
    c_kv = torch.randn((n_new, R), generator=g, device="cuda").to(L.tdt)
    k_rope = torch.randn((n_new, Dr), generator=g, device="cuda").to(L.tdt)
    if w.kind == "prefill":
        pos, dst, n_rows = L.pos, None, w.n_kv
    else:
        assert L.seq_stride == w.n_kv * L.row_bytes
        pos = torch.full((n_new,), w.n_kv - 1, dtype=torch.int32, device="cuda")
        dst = torch.arange(n_new, dtype=torch.int64, device="cuda") * w.n_kv + (w.n_kv - 1)
        n_rows = w.n_kv * w.n_seq
    cache = L.caches[0]
    stream = torch.cuda.current_stream()

    def run():
        mla.mla_cache_append(L.cdims, L.act, L.kv, c_kv, k_rope, pos, n_new, cache, n_rows,
                             dst_row=dst, stream=stream)

    def run_had():
        mla.mla_cache_append_hadamard(L.cdims, L.act, L.kv, c_kv, k_rope, pos, n_new, cache,
                                      n_rows, dst_row=dst, stream=stream)

    reps = max(min(reps, 50), 20)
    in_b = 4 if w.mode == "f32" else 2
    nbytes = n_new * (W * in_b + 4 + (8 if dst is not None else 0) + L.row_bytes)
    res = {"kernel": "cache_append_kernel", "tokens": n_new, "bytes_per_launch": nbytes,
           "bytes": "per token: c_kv + k_rope inputs, pos (+ dst_row), one cache row"}
    for key, fn in (("", run), ("hadamard_", run_had)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[key + "us_per_launch"] = us
        res[key + "GB/s"] = nbytes / (us * 1e-6) / 1e9
    res["frac_hbm"] = res["GB/s"] / HBM_PEAK_GBS
    return res


def time_transpose_append(w, L, reps):
    """mla_cache_transpose_v of one new row per sequence (its last row), the V^T upkeep
    that follows each cache append on the K + V^T path."""
    import torch
    from deepseek_mla_amd import mla
    R = w.dims.kv_lora_rank
    stream = torch.cuda.current_stream()

    def run():
        mla.mla_cache_transpose_v(L.cdims, L.kv, L.caches[0], L.seq_stride, L.n_seq, w.n_kv - 1,
                                  w.n_kv, L.vts[0], R * L.vt_ld * 2, L.vt_ld, stream=stream)

    for _ in range(3):
        run()
    reps = max(min(reps, 50), 20)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"kernel": "transpose_v_kernel", "rows": L.n_seq,
            "us_per_launch": e0.elapsed_time(e1) * 1e3 / reps}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Oracle coverage of each workload: prefill query-token sample (None = all tokens) for
# the multi-thread timing, and the smaller sample of the single-thread timing.
CPU_PLAN = {
    "tiny_f32": (None, None),
    "lite_prefill": (None, 64),
    "v3_long_prefill": ("long64", 2),
    "v3_decode": (None, None),
    "v3_decode_q8": (None, 1),
}


def _oracle_run(w, x, rows_of, seqs):
    """Runs the oracle chain over (sequence, query selection) pairs; returns seconds,
    the algorithmic FLOP and the visible pairs covered."""
    import oracle
    from deepseek_mla_amd import accounting
    d = w.dims
    dt, fl, pairs = 0.0, 0, 0
    for b, sel in seqs:
        rows = rows_of(b)
        t0 = time.perf_counter()
        oracle.mla_absorbed(d, x["q_nope"][sel], x["q_rope"][sel], x["pos"][sel], rows,
                            x["wk_b"], x["wv_b"], x["wo"])
        dt += time.perf_counter() - t0
        f = step_flops(w, x["pos"][sel])
        if w.kind == "decode":
            f["attention"] = accounting.absorbed_flops_per_pair(d) * w.n_kv
            pairs += w.n_kv
        else:
            pairs += accounting.visible_pairs(x["pos"][sel], w.n_kv)
        fl += sum(f.values())
    return dt, fl, pairs


def cpu_baseline(w):
    """The oracle (absorb + attention + out_proj, test infrastructure) on this host's cores
    with pinned threads, on the plan of CPU_PLAN; see the module docstring."""
    import oracle
    from deepseek_mla_amd import accounting, synth
    x = synth.generate_workload(w)
    d = w.dims
    threads = oracle.max_threads()  # OMP_NUM_THREADS, or every core the process may use
    multi, single = CPU_PLAN[w.name]
    cache = {}

    def rows_of(b):
        if b not in cache:
            cache.clear()
            r = synth.cache_rows(x["c_kv"][b], x["k_rope"][b])
            if w.mode == "q8_0":
                r = oracle.q8_0_dequantize(oracle.q8_0_quantize(r), r.shape[-1])
            cache[b] = r
        return cache[b]

    if w.kind == "prefill":
        all_tok = np.arange(w.T)
        sel = synth.long_prefill_sample(w.T) if multi == "long64" else all_tok
        seqs = [(0, sel)]
        sample = (f"{len(sel)} of {w.T} query tokens (tokens 0 and {w.T - 1} among them), "
                  f"all {d.n_head} heads" if multi == "long64" else
                  f"all {w.T} query tokens, all {d.n_head} heads")
        ssel = all_tok if single is None else sel[np.linspace(0, len(sel) - 1, single).astype(int)]
        sseqs = [(0, ssel)]
        total_pairs = accounting.visible_pairs(x["pos"], w.n_kv)
        total_flops = sum(step_flops(w, x["pos"]).values())
    else:
        seqs = [(b, np.array([b])) for b in range(w.n_seq)]
        sample = f"all {w.n_seq} sequences, all {d.n_head} heads, all {w.n_kv} rows"
        sseqs = seqs if single is None else seqs[:single]
        total_pairs = w.n_seq * w.n_kv
        total_flops = None
    dt, fl, pairs = _oracle_run(w, x, rows_of, seqs)
    oracle.set_threads(1)
    try:
        dt1, fl1, pairs1 = _oracle_run(w, x, rows_of, sseqs)
    finally:
        oracle.set_threads(threads)
    extrap = pairs < total_pairs
    full_s = dt * total_pairs / pairs
    full_s1 = dt1 * total_pairs / pairs1
    res = {"cores": threads, "kind": "oracle", "cpu": cpu_model(),
           "threads_pinned": os.environ.get("OMP_PROC_BIND", ""),
           "places": os.environ.get("OMP_PLACES", ""),
           "seconds": dt, "extrapolated": bool(extrap),
           "full_workload_seconds": full_s,
           "single_thread": {"seconds": dt1, "full_workload_seconds": full_s1,
                             "sample": (f"{len(sseqs[0][1])} query tokens" if w.kind == "prefill"
                                        else f"{len(sseqs)} of {w.n_seq} sequences")}}
    label = " (extrapolated by visible-pair count)" if extrap else ""
    if w.kind == "prefill":
        res.update({"value": fl / dt / 1e12, "unit": "TFLOP/s",
                    "sample": sample + "; full step (absorb, attention, out_proj)" + label})
        res["single_thread"]["value"] = fl1 / dt1 / 1e12
        if extrap:
            res["full_workload_flops"] = total_flops
    else:
        nbytes = attention_bytes(w)
        res.update({"value": nbytes / full_s / 1e9, "unit": "GB/s",
                    "sample": sample + "; full step, bytes = latent rows + q_cat + o_lat"})
        res["single_thread"]["value"] = nbytes / full_s1 / 1e9
    return res


def run_materialized(name, steps, warmup):
    """The materialised prefill (one mla_prefill_materialized call per step: rotation of the
    query rope, per head chunk the k_nope / v decompression and the attention, then wo)."""
    import torch
    from deepseek_mla_amd import accounting, layer, synth
    base = name.split("@")[0]
    w = synth.WORKLOADS[base]
    assert w.kind == "prefill"
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x, path="materialized")
    del x
    log(f"[bench] {name}: {steps} steps after {warmup} warmup")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        L.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        L.step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    calls = [e[0].elapsed_time(e[1]) for e in ev]
    ms = float(np.median(calls))
    pos = L.pos.cpu().numpy()
    del L
    torch.cuda.empty_cache()
    d = w.dims
    pairs = accounting.visible_pairs(pos, w.n_kv)
    attn = pairs * accounting.decompressed_flops_per_pair(d)
    decomp = 2 * w.n_kv * d.kv_lora_rank * d.n_head * (d.qk_nope + d.v_head)
    wo = 2 * len(pos) * d.d_model * d.n_head * d.v_head
    att = attn / (ms * 1e-3) / 1e12
    return {"workload": name,
            "roofline": {"kernel": "flash_mha_kernel (all head chunks of the call)",
                         "bound": "mfma", "achieved": att, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": att / BF16_PEAK_TFLOPS,
                         "traffic": measured_traffic(name),
                         "per_launch": "attention FLOP = visible pairs x 640 x heads, over the "
                                       "whole call (decompression GEMMs, wo and launch gaps "
                                       "included: a lower bound for the kernel)"},
            "path": "materialized (decompress k_nope / v, then 192/128 causal attention)",
            "ms_per_step": wall * 1e3, "call_ms": ms, "call_stats": stats(calls),
            "flops_performed": {"attention": attn, "decompression": decomp, "wo": wo},
            "performed_tflops": (attn + decomp + wo) / (ms * 1e-3) / 1e12}


def run_one(name, steps, warmup, with_cpu, n_splits=0):
    from deepseek_mla_amd import synth
    if name.endswith("@materialized"):
        return run_materialized(name, steps, warmup)
    path = "vt" if name.endswith("@vt") else "absorbed"
    w = synth.WORKLOADS[name.split("@")[0]]
    copies = 1
    if w.kind == "decode":
        # rotate caches so that the 256 MB last-level cache holds none of them between steps
        per = attention_bytes(w)
        copies = max(1, min(16, int(np.ceil(600e6 / per))))
    log(f"[bench] {name}: {steps} steps after {warmup} warmup, cache copies {copies}")
    res, pos = time_workload(w, steps, warmup, copies, n_splits, path)
    fl = step_flops(w, pos)
    total = sum(fl.values())
    entry = {"workload": name, "ms_per_step": res["ms_per_step"],
             "kernel_ms": {k: res[k] for k in ("absorb_ms", "attention_ms", "out_proj_ms")},
             "attention_stats": res["attention_stats"],
             "step_tflops": total / (res["ms_per_step"] * 1e-3) / 1e12,
             "cache_append": res["cache_append"]}
    if path == "vt":
        entry["path"] = ("K + V^T cache (absorption page, section 8.2, mode 1): "
                         "mla_attn_decode_vt over the bf16 rows and their transposed latent copy")
        entry["transpose_v_append"] = res["transpose_v_append"]
    clk = measured_clock(name)
    if w.kind == "prefill":
        ach = fl["attention"] / (res["attention_ms"] * 1e-3) / 1e12
        entry["value"] = ach
        entry["unit"] = "TFLOP/s"
        entry["attention_tflops"] = ach
        entry["roofline"] = {"kernel": "flash_prefill_bf16_kernel (+ prefill_merge_kernel for cut "
                                       "row groups)", "bound": "mfma",
                             "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": ach / BF16_PEAK_TFLOPS, "traffic": measured_traffic(name),
                             "per_launch": f"{fl['attention']} FLOP = visible pairs x "
                                           f"{2 * (2 * w.dims.kv_lora_rank + w.dims.qk_rope)}"
                                           f" x {w.dims.n_head} heads"}
        if clk:
            pk = MFMA_FLOP_PER_CLK * clk * 1e9 / 1e12
            entry["roofline"].update({"clock_ghz_measured": clk, "peak_at_measured_clock": pk,
                                      "frac_at_measured_clock": ach / pk})
    else:
        nbytes = attention_bytes(w)
        # the K + V^T form also reads the transposed latent rows (R bf16 per key)
        vt_bytes = w.n_seq * w.n_kv * w.dims.kv_lora_rank * 2 if path == "vt" else 0
        if path == "vt":
            entry["row_cache_gbs"] = nbytes / (res["attention_ms"] * 1e-3) / 1e9
        nbytes += vt_bytes
        ach = nbytes / (res["attention_ms"] * 1e-3) / 1e9
        entry["value"] = ach
        entry["unit"] = "GB/s"
        entry["attention_tflops"] = fl["attention"] / (res["attention_ms"] * 1e-3) / 1e12
        kern = ("flash_decode_w_kernel<VT> + combine_kernel" if path == "vt" else
                "flash_decode_w_kernel<Q8> + combine_kernel" if w.mode == "q8_0" else
                "flash_decode_kernel + combine_kernel")
        entry["roofline"] = {"kernel": kern, "bound": "hbm",
                             "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(name),
                             "mfma_frac": entry["attention_tflops"] / BF16_PEAK_TFLOPS,
                             "per_launch": f"{nbytes} B = {w.n_seq} x ({w.n_kv} latent rows "
                                           f"{'+ their V^T copy ' if vt_bytes else ''}+ "
                                           f"q_cat + o_lat of {w.dims.n_head} heads)"}
        if clk:
            entry["roofline"]["clock_ghz_measured"] = clk
    if with_cpu and path == "absorbed":
        t0 = time.perf_counter()
        entry["cpu_baseline"] = cpu_baseline(w)
        log(f"[bench] {name}: cpu baseline {time.perf_counter() - t0:.1f}s")
    log(f"[bench] {name}: {json.dumps(entry)}")
    return entry


def decode_batch_sweep(batches=(1, 4, 16, 64), n_kv=32768, reps=20):
    """mla_attn_decode (partials + combine) at V3 dims over batch sizes, random bf16 queries
    and caches made on the device (timing only), copies rotated past the MALL.  Prints one
    JSON line per batch size."""
    import math
    import torch
    from deepseek_mla_amd import mla, synth
    d = synth.deepseek_dims(128, 7168)
    cd = mla.make_dims(d)
    W, H, R = d.kv_lora_rank + d.qk_rope, d.n_head, d.kv_lora_rank
    for B in batches:
        per = B * n_kv * W * 2
        copies = max(1, min(8, math.ceil(700e6 / per)))
        caches = [torch.randn((B, n_kv, W), device="cuda").to(torch.bfloat16)
                  for _ in range(copies)]
        q = torch.randn((B, H, W), device="cuda").to(torch.bfloat16)
        nkv = torch.full((B,), n_kv, dtype=torch.int32, device="cuda")
        ns = mla.mla_decode_auto_splits(cd, mla.BF16, B, n_kv)
        wsb = mla.mla_decode_workspace_bytes(cd, B, n_kv, 0)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        o = torch.empty((B, H, R), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")

        def run(i):
            mla.mla_attn_decode(cd, mla.BF16, mla.BF16, q, caches[i % copies], n_kv * W * 2, nkv,
                                B, n_kv, 0, o, lse, ws, wsb)

        for i in range(3):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = B * (n_kv * W * 2 + H * W * 2 + H * R * 2)
        print(json.dumps({"sweep": "v3_decode_batch", "B": B, "splits": ns, "us": ms * 1e3,
                          "GB/s": nbytes / (ms * 1e-3) / 1e9,
                          "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}), flush=True)
        del caches, q, ws, o
        torch.cuda.empty_cache()


def decode_split_sweep(steps=60, warmup=5):
    """Decode attention time against the key split count: the V3 bf16 decode (1 x 32768 rows)
    and the V3 Q8_0 decode (4 x 98304 rows), each at a list of split counts around the
    library's automatic choice (median of the attention call over `steps` whole steps)."""
    from deepseek_mla_amd import mla, synth
    for name, splits in (("v3_decode", (32, 64, 96, 128, 160, 192, 256)),
                         ("v3_decode_q8", (16, 32, 48, 64, 96, 128))):
        w = synth.WORKLOADS[name]
        d = mla.make_dims(w.dims)
        auto = mla.mla_decode_auto_splits(d, mla.Q8_0 if w.mode == "q8_0" else mla.BF16,
                                          w.n_seq, w.n_kv)
        for ns in splits:
            res, _ = time_workload(w, steps, warmup, 1, ns)
            ms = res["attention_ms"]
            nbytes = attention_bytes(w)
            print(json.dumps({"sweep": name + "_splits", "splits": ns, "auto": auto,
                              "us": ms * 1e3, "p10_us": res["attention_stats"]["p10_ms"] * 1e3,
                              "p90_us": res["attention_stats"]["p90_ms"] * 1e3,
                              "GB/s": nbytes / (ms * 1e-3) / 1e9}), flush=True)


# Iterations per workload entry (the measurement protocol: 50 prefill, 200 decode).
PROTOCOL_STEPS = {"prefill": 50, "decode": 200}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_long_prefill")
    ap.add_argument("--extra", default="v3_decode,v3_decode@vt,v3_decode_q8,lite_prefill,"
                                       "lite_prefill@materialized,v3_long_prefill@materialized",
                    help="comma-separated extra workloads reported under 'workloads' ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode key splits per sequence (0 = the library's automatic choice)")
    ap.add_argument("--decode-batch-sweep", action="store_true",
                    help="only time V3 bf16 decode at B = 1, 4, 16, 64 (one JSON line each)")
    ap.add_argument("--decode-split-sweep", action="store_true",
                    help="only time the V3 bf16 and Q8_0 decodes over a range of split counts")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the design for sharding is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    # the CPU oracle's OpenMP threads are pinned to cores (read when its runtime loads)
    os.environ.setdefault("OMP_PROC_BIND", "close")
    os.environ.setdefault("OMP_PLACES", "cores")
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.decode_batch_sweep:
        from deepseek_mla_amd import mla
        mla.lib()
        decode_batch_sweep()
        return
    if args.decode_split_sweep:
        from deepseek_mla_amd import mla
        mla.lib()
        decode_split_sweep()
        return
    if args.calibrate_copy:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    from deepseek_mla_amd import mla, synth
    mla.lib()
    copy_gbs = copy_bandwidth()
    log(f"[bench] device copy: {copy_gbs:.0f} GB/s (read + write)")
    main_entry = run_one(args.workload, args.steps, args.warmup, not args.no_cpu_baseline,
                         args.splits)
    extras = []
    for name in [n for n in args.extra.split(",") if n and n != args.workload]:
        kind = synth.WORKLOADS[name.split("@")[0]].kind
        steps = PROTOCOL_STEPS[kind]
        extras.append(run_one(name, steps, args.warmup, not args.no_cpu_baseline, args.splits))
    # the materialised path against the absorbed step of the same workload
    absorbed = {e["workload"]: e["ms_per_step"] for e in [main_entry] + extras
                if "@" not in e["workload"]}
    attn_ms = {e["workload"]: e["kernel_ms"]["attention_ms"] for e in [main_entry] + extras
               if "@" not in e["workload"]}
    for e in extras:
        base = e["workload"].split("@")[0]
        if "@materialized" in e["workload"] and base in absorbed:
            e["speedup_vs_absorbed"] = absorbed[base] / e["ms_per_step"]
            e["speedup_note"] = "absorbed step ms (absorb + attention + out_proj) / this step ms"
        if "@vt" in e["workload"] and base in attn_ms:
            e["attention_speedup_vs_row_cache"] = attn_ms[base] / e["kernel_ms"]["attention_ms"]
    for e in [main_entry] + extras:
        if e["roofline"]["bound"] == "hbm":
            e["roofline"]["copy_gbs_measured"] = copy_gbs
            e["roofline"]["frac_of_measured_copy"] = e["roofline"]["achieved"] / copy_gbs
    w = synth.WORKLOADS[args.workload.split("@")[0]]
    line = {
        "metric": "MLA attention TFLOP/s (prefill) and latent-cache GB/s (decode), 1 MI355X",
        "value": main_entry["value"], "unit": main_entry["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_entry["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.mode != "f32" else "f32", "data": "synthetic",
        "config": {"workload": args.workload, "n_head": w.dims.n_head,
                   "kv_lora_rank": w.dims.kv_lora_rank, "qk_rope": w.dims.qk_rope,
                   "qk_nope": w.dims.qk_nope, "v_head": w.dims.v_head,
                   "d_model": w.dims.d_model, "query_tokens": w.n_query, "n_kv": w.n_kv,
                   "cache": w.mode, "scratch_cap_mib": w.scratch_cap_mib,
                   "value": "attention FLOP (visible pairs x 2176 x heads) / median attention "
                            "call time"},
        "roofline": main_entry["roofline"],
        "attention_stats": main_entry["attention_stats"],
        "kernel_ms": main_entry["kernel_ms"],
        "step_tflops": main_entry["step_tflops"],
        "copy_gbs_measured": copy_gbs,
        "cache_append": main_entry["cache_append"],
        "workloads": extras,
    }
    if "cpu_baseline" in main_entry:
        line["cpu_baseline"] = main_entry["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
