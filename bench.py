"""Benchmark: one absorbed-MLA layer step on one MI355X.

A step is the whole path on one batch of synthetic input already resident in HBM:
mla_absorb_q -> mla_attn_prefill (or mla_attn_decode) -> mla_out_proj.

Default workload (the headline line): the DeepSeek-Lite-shaped prefill layer
(16 heads, kv_lora_rank 512, rope 64, nope 128, v 128, d_model 2048; 2048 causal
tokens over a 2048-row bf16 latent cache).  `value` is the step's algorithmic FLOP
count (absorption GEMM + two-term attention + latent weighted sum + wv_b + wo, a
multiply-add counted as 2 FLOP; attention priced per visible (query, key) pair as
in the absorption page's section 7 table) divided by the step's wall time.

The V3-shaped configurations run as extra entries under "workloads" (decode ones
report latent-cache GB/s of the attention kernels, prefill ones TFLOP/s); each entry
carries its own roofline object.  Decode timing rotates through several copies of
the latent cache so that the 256 MB last-level cache cannot hold it between steps.

`cpu_baseline` times the CPU oracle (test infrastructure) on a bounded sample of the
same workload on this host's cores.
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
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

# HBM bytes per launch of the dominant kernel(s), from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes scaled by a 512 MiB copy (fetch x2.0, write x1.0); the summaries and commands are
# in profiles/.  Each figure is valid only for the kernel sources it was taken on (sha256
# prefix over the files listed, in order).
ABSORBED_SRC = ("deepseek_mla_amd/csrc/flash_mfma.hip", "deepseek_mla_amd/csrc/decode_mfma.hip",
                "deepseek_mla_amd/csrc/latent_tile.h", "deepseek_mla_amd/csrc/lds_dma.h",
                "deepseek_mla_amd/csrc/simt.hip", "deepseek_mla_amd/csrc/common.h")
MATERIALIZED_SRC = ("deepseek_mla_amd/csrc/flash_mha.hip", "deepseek_mla_amd/csrc/latent_tile.h",
                    "deepseek_mla_amd/csrc/lds_dma.h", "deepseek_mla_amd/csrc/common.h")
TRAFFIC = {
    # workload: (bytes per launch, sources, sha256 prefix)
    "lite_prefill": ((71.32e6 + 82.26e6) + (61.82e6 + 15.32e6), ABSORBED_SRC,
                     "be9298de0b078631"),                                         # prefill kernel + merge
    "v3_long_prefill": (9804.58e6 + 1195.38e6, ABSORBED_SRC, "be9298de0b078631"),
    "v3_decode": ((39.25e6 + 16.84e6) + (17.43e6 + 0.14e6), ABSORBED_SRC,
                  "be9298de0b078631"),                                            # partial kernel + combine
    "v3_decode_q8": ((245.75e6 + 16.84e6) + (17.43e6 + 0.54e6), ABSORBED_SRC, "be9298de0b078631"),
    "v3_long_prefill@materialized": (193.71e6 + 18.87e6, MATERIALIZED_SRC,
                                     "8bb3e0163161f07e"),                         # one 8-head chunk launch
}


def _sources_sha(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    if name not in TRAFFIC:
        return None
    value, paths, sha = TRAFFIC[name]
    if _sources_sha(paths) != sha:
        return None  # kernels changed since the counters were taken
    return value


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def time_workload(w, steps, warmup, copies=1, n_splits=0):
    import torch
    from deepseek_mla_amd import layer, synth
    x = synth.generate_workload(w)
    L = layer.for_workload(w, x, cache_copies=copies, n_splits=n_splits)
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
    res = {"ms_per_step": wall * 1e3, "absorb_ms": float(parts[:, 0].mean()),
           "attention_ms": float(parts[:, 1].mean()), "out_proj_ms": float(parts[:, 2].mean()),
           "attention_ms_min": float(parts[:, 1].min())}
    res["cache_append"] = time_append(w, L, steps)
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

    for _ in range(3):
        run()
    def run_had():
        mla.mla_cache_append_hadamard(L.cdims, L.act, L.kv, c_kv, k_rope, pos, n_new, cache,
                                      n_rows, dst_row=dst, stream=stream)

    reps = max(reps, 20)
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


def cpu_baseline(w, max_queries):
    """Oracle (absorb + attention + out_proj) on a bounded sample of the workload."""
    import oracle
    from deepseek_mla_amd import accounting, synth
    x = synth.generate_workload(w)
    d = w.dims
    if w.kind == "prefill":
        sel = np.unique(np.linspace(0, w.T - 1, min(max_queries, w.T)).astype(int))
        seqs = [(0, sel)]
        sample = f"{len(sel)} of {w.T} query tokens (evenly spaced), all {d.n_head} heads"
    else:
        nseq = min(w.n_seq, max(1, max_queries))
        seqs = [(b, np.array([b])) for b in range(nseq)]
        sample = f"{nseq} of {w.n_seq} sequences, all {d.n_head} heads, all {w.n_kv} rows"
    fl = 0
    dt = 0.0
    nbytes = 0
    for b, sel in seqs:
        rows = synth.cache_rows(x["c_kv"][b], x["k_rope"][b])
        if w.mode == "q8_0":
            rows = oracle.q8_0_dequantize(oracle.q8_0_quantize(rows), rows.shape[-1])
        t0 = time.perf_counter()
        oracle.mla_absorbed(d, x["q_nope"][sel], x["q_rope"][sel], x["pos"][sel], rows,
                            x["wk_b"], x["wv_b"], x["wo"])
        dt += time.perf_counter() - t0
        f = step_flops(w, x["pos"][sel])
        if w.kind == "decode":
            f["attention"] = accounting.absorbed_flops_per_pair(d) * w.n_kv
        fl += f["attention"] if w.kind == "decode" else sum(f.values())
        nbytes += attention_bytes(w) // w.n_seq
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    if w.kind == "prefill":
        return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": sample + "; full step (absorb, attention, out_proj)", "seconds": dt}
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": sample + "; full step, bytes = latent rows + q_cat + o_lat", "seconds": dt}


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
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    pos = L.pos.cpu().numpy()
    del L
    torch.cuda.empty_cache()
    d = w.dims
    pairs = accounting.visible_pairs(pos, w.n_kv)
    attn = pairs * accounting.decompressed_flops_per_pair(d)
    decomp = 2 * w.n_kv * d.kv_lora_rank * d.n_head * (d.qk_nope + d.v_head)
    wo = 2 * len(pos) * d.d_model * d.n_head * d.v_head
    absorbed = sum(step_flops(w, pos).values())
    att = attn / (ms * 1e-3) / 1e12
    return {"workload": name,
            "roofline": {"kernel": "flash_mha_kernel (all head chunks of the call)",
                         "bound": "mfma", "achieved": att, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": att / BF16_PEAK_TFLOPS,
                         "traffic": measured_traffic(name),
                         "per_launch": "attention FLOP = visible pairs x 640 x heads, over the "
                                       "whole call (decompression GEMMs, wo and launch gaps "
                                       "included: a lower bound for the kernel)"}, "path": "materialized (decompress k_nope / v, then 192/128 "
                                      "causal attention)",
            "ms_per_step": wall * 1e3, "call_ms": ms,
            "flops_performed": {"attention": attn, "decompression": decomp, "wo": wo},
            "performed_tflops": (attn + decomp + wo) / (ms * 1e-3) / 1e12,
            "absorbed_equivalent_tflops": absorbed / (ms * 1e-3) / 1e12,
            "note": "absorbed_equivalent_tflops prices the step with the absorbed path's "
                    "FLOP count (the same result, 3.4x more attention FLOPs per pair)"}


def run_one(name, steps, warmup, with_cpu, n_splits=0):
    from deepseek_mla_amd import synth
    if name.endswith("@materialized"):
        return run_materialized(name, steps, warmup)
    w = synth.WORKLOADS[name]
    copies = 1
    if w.kind == "decode":
        # rotate caches so that the 256 MB last-level cache holds none of them between steps
        per = attention_bytes(w)
        copies = max(1, min(16, int(np.ceil(600e6 / per))))
    log(f"[bench] {name}: {steps} steps after {warmup} warmup, cache copies {copies}")
    res, pos = time_workload(w, steps, warmup, copies, n_splits)
    fl = step_flops(w, pos)
    total = sum(fl.values())
    entry = {"workload": name, "ms_per_step": res["ms_per_step"],
             "kernel_ms": {k: res[k] for k in ("absorb_ms", "attention_ms", "out_proj_ms")},
             "step_tflops": total / (res["ms_per_step"] * 1e-3) / 1e12,
             "cache_append": res["cache_append"]}
    if w.kind == "prefill":
        ach = fl["attention"] / (res["attention_ms"] * 1e-3) / 1e12
        entry["value"] = entry["step_tflops"]
        entry["unit"] = "TFLOP/s"
        entry["attention_tflops"] = ach
        entry["roofline"] = {"kernel": "flash_prefill_bf16_kernel (+ prefill_merge_kernel for cut row groups)", "bound": "mfma",
                             "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": ach / BF16_PEAK_TFLOPS, "traffic": measured_traffic(name),
                             "per_launch": f"{fl['attention']} FLOP = visible pairs x "
                                           f"{2 * (2 * w.dims.kv_lora_rank + w.dims.qk_rope)}"
                                           f" x {w.dims.n_head} heads"}
    else:
        nbytes = attention_bytes(w)
        ach = nbytes / (res["attention_ms"] * 1e-3) / 1e9
        entry["value"] = ach
        entry["unit"] = "GB/s"
        entry["attention_tflops"] = fl["attention"] / (res["attention_ms"] * 1e-3) / 1e12
        entry["roofline"] = {"kernel": "flash_decode_kernel + combine_kernel", "bound": "hbm",
                             "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(name),
                             "mfma_frac": entry["attention_tflops"] / BF16_PEAK_TFLOPS,
                             "per_launch": f"{nbytes} B = {w.n_seq} x ({w.n_kv} latent rows + "
                                           f"q_cat + o_lat of {w.dims.n_head} heads)"}
    if with_cpu:
        t0 = time.perf_counter()
        mq = {"lite_prefill": 2048, "v3_long_prefill": 8, "v3_decode": 1, "v3_decode_q8": 1,
              "tiny_f32": 16}[name]
        entry["cpu_baseline"] = cpu_baseline(w, mq)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lite_prefill")
    ap.add_argument("--extra", default="v3_decode,v3_long_prefill,v3_decode_q8,"
                                       "lite_prefill@materialized,v3_long_prefill@materialized",
                    help="comma-separated extra workloads reported under 'workloads' ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode key splits per sequence (0 = the library's automatic choice)")
    ap.add_argument("--decode-batch-sweep", action="store_true",
                    help="only time V3 bf16 decode at B = 1, 4, 16, 64 (one JSON line each)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the design for sharding is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.decode_batch_sweep:
        from deepseek_mla_amd import mla
        mla.lib()
        decode_batch_sweep()
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
    from deepseek_mla_amd import mla
    mla.lib()
    main_entry = run_one(args.workload, args.steps, args.warmup, not args.no_cpu_baseline,
                         args.splits)
    extras = []
    for name in [n for n in args.extra.split(",") if n and n != args.workload]:
        steps = max(3, args.steps // 2) if "long" in name else args.steps
        extras.append(run_one(name, steps, args.warmup, not args.no_cpu_baseline, args.splits))
    from deepseek_mla_amd import synth
    w = synth.WORKLOADS[args.workload]
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
                   "cache": w.mode, "flop_count": "absorb + attention + out_proj per step"},
        "roofline": main_entry["roofline"],
        "kernel_ms": main_entry["kernel_ms"],
        "attention_tflops": main_entry.get("attention_tflops"),
        "cache_append": main_entry["cache_append"],
        "workloads": extras,
    }
    if "cpu_baseline" in main_entry:
        line["cpu_baseline"] = main_entry["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
