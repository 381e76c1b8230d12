"""One absorbed-MLA layer step on the GPU, driven through the C ABI.

A step is the whole path in the order of the absorption page, section 4:
mla_absorb_q -> mla_attn_prefill (or mla_attn_decode) -> mla_out_proj.  A prefill step
on the materialised path (section 8.4) is the single call mla_prefill_materialized
(decompression, attention and wo).  A decode step on the K + V^T path (section 8.2, the
-mla switch's mode 1) calls mla_attn_decode_vt on the row cache and its transposed latent
copy, built once by mla_cache_transpose_v.
Buffers are allocated once with torch (device memory only); every computation runs
in libmla.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import mla, synth

_MODE = {"f32": (mla.F32, mla.F32), "bf16": (mla.BF16, mla.BF16), "q8_0": (mla.BF16, mla.Q8_0)}


def _dev(a: np.ndarray, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype).contiguous()


class LayerStep:
    """Device buffers and launch sequence for one workload.

    inputs: dict from synth.generate / generate_workload (float32 numpy, bf16-rounded in
    bf16 / q8_0 modes).  For q8_0 the float32 latents are quantised on the device by
    mla_quantize_q8_0.
    """

    def __init__(self, dims: synth.Dims, mode: str, kind: str, inputs: dict, n_kv: int,
                 scratch_cap_mib: int = 0, n_splits: int = 0, cache_copies: int = 1,
                 device="cuda", path: str = "absorbed"):
        assert path in ("absorbed", "materialized", "vt")
        assert path != "materialized" or kind == "prefill"
        assert path != "vt" or (kind == "decode" and mode == "bf16")
        self.path = path
        self.dims, self.mode, self.kind = dims, mode, kind
        self.act, self.kv = _MODE[mode]
        self.cdims = mla.make_dims(dims)
        self.n_kv = n_kv
        self.scratch_cap_mib = scratch_cap_mib
        self.n_splits = n_splits
        H, R, Dr, Dv, D = dims.n_head, dims.kv_lora_rank, dims.qk_rope, dims.v_head, dims.d_model
        W = R + Dr
        tdt = torch.float32 if mode == "f32" else torch.bfloat16
        self.tdt = tdt
        self.q_nope = _dev(inputs["q_nope"], tdt, device)
        self.q_rope = _dev(inputs["q_rope"], tdt, device)
        self.pos = _dev(inputs["pos"], torch.int32, device)
        self.wk_b = _dev(inputs["wk_b"], tdt, device)
        self.wv_b = _dev(inputs["wv_b"], tdt, device)
        self.wo = _dev(inputs["wo"], tdt, device)
        self.T = int(self.q_nope.shape[0])
        S = inputs["c_kv"].shape[0]
        self.n_seq = S
        if mode == "q8_0":
            rb = mla.mla_q8_0_row_bytes(W)
            # sequences start 16-byte aligned: the stride is n_kv rows rounded up to 16 B
            self.cache = torch.empty((S, (n_kv * rb + 15) // 16 * 16), dtype=torch.uint8,
                                     device=device)
            for s in range(S):  # quantise one sequence at a time (bounded float32 staging)
                rows = _dev(synth.cache_rows(inputs["c_kv"][s], inputs["k_rope"][s]),
                            torch.float32, device)
                mla.mla_quantize_q8_0(rows, self.cache[s], n_kv, W)
                del rows
            self.row_bytes = rb
            self.seq_stride = int(self.cache.shape[1])
        else:
            rows = np.concatenate([inputs["c_kv"], inputs["k_rope"]], axis=-1)
            self.cache = _dev(rows, tdt, device)
            self.row_bytes = W * (4 if mode == "f32" else 2)
            self.seq_stride = n_kv * self.row_bytes
        # identical copies of the cache, used in rotation (keeps timing honest when the
        # cache would otherwise stay resident in the last-level cache between steps)
        self.caches = [self.cache] + [self.cache.clone() for _ in range(cache_copies - 1)]
        self._ci = 0
        self.q_cat = torch.empty((self.T, H, W), dtype=tdt, device=device)
        self.o_lat = torch.empty((self.T, H, R), dtype=tdt, device=device)
        self.lse = torch.empty((self.T, H), dtype=torch.float32, device=device)
        self.v = torch.empty((self.T, H * Dv), dtype=tdt, device=device)
        self.out = torch.empty((self.T, D), dtype=tdt, device=device)
        self.prefill_ws = (mla.prefill_workspace(self.cdims, self.kv, self.T, n_kv,
                                                 scratch_cap_mib, device)
                           if kind == "prefill" and path == "absorbed" else None)
        self.mat_ws = (mla.materialized_workspace(self.cdims, self.T, n_kv, scratch_cap_mib,
                                                  device)
                       if path == "materialized" else None)
        if kind == "decode":
            self.n_kv_dev = torch.full((S,), n_kv, dtype=torch.int32, device=device)
            wsb = mla.mla_decode_workspace_bytes(self.cdims, S, n_kv, n_splits)
            self.workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=device)
            self.ws_bytes = wsb
        if path == "vt":
            # each cache copy's V^T rows: [S][R][vt_ld], vt_ld = n_kv rounded up to 32
            self.vt_ld = (n_kv + 31) // 32 * 32
            self.vts = []
            for c in self.caches:
                vt = torch.empty((S, R, self.vt_ld), dtype=tdt, device=device)
                mla.mla_cache_transpose_v(self.cdims, self.kv, c, self.seq_stride, S, 0, n_kv, vt,
                                          R * self.vt_ld * 2, self.vt_ld)
                self.vts.append(vt)

    def absorb(self, stream=None):
        mla.mla_absorb_q(self.cdims, self.act, self.q_nope, self.q_rope, self.pos, self.wk_b,
                         self.q_cat, self.T, stream)

    def attend(self, stream=None):
        self.cache = self.caches[self._ci]
        ci = self._ci
        self._ci = (self._ci + 1) % len(self.caches)
        if self.path == "vt":
            mla.mla_attn_decode_vt(self.cdims, self.act, self.kv, self.q_cat, self.cache,
                                   self.seq_stride, self.vts[ci], self.dims.kv_lora_rank *
                                   self.vt_ld * 2, self.vt_ld, self.n_kv_dev, self.n_seq,
                                   self.n_kv, self.n_splits, self.o_lat, self.lse,
                                   self.workspace, self.ws_bytes, stream)
        elif self.kind == "prefill":
            mla.mla_attn_prefill(self.cdims, self.act, self.kv, self.q_cat, self.pos, self.T,
                                 self.cache, self.n_kv, self.o_lat, self.lse,
                                 self.scratch_cap_mib, self.prefill_ws, stream)
        else:
            mla.mla_attn_decode(self.cdims, self.act, self.kv, self.q_cat, self.cache,
                                self.seq_stride, self.n_kv_dev, self.n_seq, self.n_kv,
                                self.n_splits, self.o_lat, self.lse, self.workspace,
                                self.ws_bytes, stream)

    def project(self, stream=None):
        mla.mla_out_proj(self.cdims, self.act, self.o_lat, self.wv_b, self.wo, self.v, self.out,
                         self.T, stream)

    def materialized(self, stream=None):
        self.cache = self.caches[self._ci]
        self._ci = (self._ci + 1) % len(self.caches)
        mla.mla_prefill_materialized(self.cdims, self.act, self.kv, self.q_nope, self.q_rope,
                                     self.pos, self.T, self.cache, self.n_kv, self.wk_b,
                                     self.wv_b, self.v, wo=self.wo, out=self.out, lse=self.lse,
                                     scratch_cap_mib=self.scratch_cap_mib,
                                     workspace=self.mat_ws, stream=stream)

    def step(self, stream=None):
        if self.path == "materialized":
            self.materialized(stream)
            return
        self.absorb(stream)
        self.attend(stream)
        self.project(stream)

    def outputs(self) -> dict:
        """Host float32 copies of every stage's output."""
        f = lambda t: t.float().cpu().numpy()
        if self.path == "materialized":
            return {"lse": f(self.lse), "v": f(self.v), "out": f(self.out)}
        return {"q_cat": f(self.q_cat), "o_lat": f(self.o_lat), "lse": f(self.lse), "v": f(self.v),
                "out": f(self.out)}


def for_workload(w: synth.Workload, inputs: dict | None = None, **kw) -> LayerStep:
    if inputs is None:
        inputs = synth.generate_workload(w)
    return LayerStep(w.dims, w.mode, w.kind, inputs, w.n_kv,
                     scratch_cap_mib=kw.pop("scratch_cap_mib", w.scratch_cap_mib), **kw)
