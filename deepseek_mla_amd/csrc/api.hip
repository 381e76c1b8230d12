// C-ABI entry points (include/mla.h): argument validation, work planning and dispatch.
// Every check happens before the first launch; no call allocates device memory.
#include <math.h>

#include <mutex>

#include "common.h"

using namespace mla;

namespace {

constexpr int NUM_CUS = 256;  // MI355X: 8 XCDs x 32 CUs

bool dims_ok(const mla_dims *d) {
    return d && d->n_head > 0 && d->kv_lora_rank > 0 && d->qk_nope > 0 && d->qk_rope > 0 &&
           (d->qk_rope % 2) == 0 && d->v_head > 0 && d->d_model > 0 && isfinite(d->scale) &&
           d->rope_base > 0.0f;
}

bool act_ok(int act) { return act == MLA_F32 || act == MLA_BF16; }

// The bf16 attention kernels are specialised for the DeepSeek latent row [512 | 64].
bool bf16_attn_dims(const mla_dims *d) { return d->kv_lora_rank == 512 && d->qk_rope == 64; }

int hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

constexpr int SIMT_SPLIT_GRAIN = 64;
constexpr int MAX_SPLITS = 4096;  // largest split count accepted
constexpr int MFMA_SPLIT_GRAIN = 32;
// V^T row length limit: a 16-row copy's lane offsets (15 rows of 2 vt_ld bytes) stay 32-bit
constexpr int32_t MAX_VT_LD = 1 << 26;

// A Q8_0 cache with whole groups of 128 heads decodes on the wide kernel (128 heads per
// workgroup, every raw tile dequantised once for all of them).
bool decode_q8_wide(const mla_dims *d, int kv) {
    return kv == MLA_Q8_0 && d->n_head % decode_wide_heads() == 0;
}

// Splits that fill the CUs with workgroups of hpb heads (at least 4 tiles per split).
int splits_for(const mla_dims *d, int hpb, int B, int n_kv_max) {
    const int hgroups = (d->n_head + hpb - 1) / hpb;
    const int per_seq = (B * hgroups);
    int s = (NUM_CUS + per_seq - 1) / per_seq;
    // at least 4 tiles of 32 keys per split
    const int max_s = (n_kv_max + 127) / 128;
    if (s > max_s) s = max_s;
    return s < 1 ? 1 : s;
}

int auto_splits(const mla_dims *d, int kv, int B, int n_kv_max) {
    if (kv == MLA_F32) {
        int s = (n_kv_max + 255) / 256;
        return s < 1 ? 1 : (s > 64 ? 64 : s);
    }
    return splits_for(d, decode_q8_wide(d, kv) ? decode_wide_heads() : decode_heads_per_block(),
                      B, n_kv_max);
}

// split length (multiple of the kernel's key grain) and the resulting split count
void split_plan(int kv, int n_kv_max, int n_splits, int *len, int *count) {
    const int grain = kv == MLA_F32 ? SIMT_SPLIT_GRAIN : MFMA_SPLIT_GRAIN;
    int L = (n_kv_max + n_splits - 1) / n_splits;
    L = (L + grain - 1) / grain * grain;
    *len = L;
    *count = (n_kv_max + L - 1) / L;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char *mla_status_str(int status) {
    switch (status) {
    case MLA_OK: return "MLA_OK: success";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype not implemented";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
    default: return "unknown mla_status";
    }
}

int32_t mla_q8_0_row_bytes(int32_t width) {
    if (width <= 0 || width % 32) return -1;
    return width / 32 * 34;
}

int32_t mla_heads_per_chunk(int32_t n_head, double size_mib, uint32_t cap_mib) {
    if (n_head < 1) return n_head;
    if (cap_mib == 0) return n_head;
    double cap = cap_mib < 128 ? 128.0 : (double)cap_mib;
    if (!(size_mib > cap)) return n_head;
    int32_t heads = 1;
    for (int32_t niter = 2; niter <= n_head; ++niter) {
        if (n_head % niter == 0 && size_mib / niter <= cap) {
            heads = n_head / niter;
            break;
        }
    }
    return heads;
}

int mla_absorb_q(const mla_dims *d, mla_dtype act, const void *q_nope, const void *q_rope,
                 const int32_t *pos, const void *wk_b, void *q_cat, int32_t T, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || T < 0) return MLA_ERR_INVALID_ARG;
    if (T == 0) return MLA_OK;
    if (!q_nope || !q_rope || !pos || !wk_b || !q_cat) return MLA_ERR_INVALID_ARG;
    const int H = d->n_head, R = d->kv_lora_rank, Dn = d->qk_nope, Dr = d->qk_rope;
    const int W = R + Dr;
    hipStream_t st = as_stream(stream);
    hipError_t e;
    if (act == MLA_F32) {
        e = launch_gemm_nt_f32((const float *)q_nope, (const float *)wk_b, (float *)q_cat, T, R,
                               Dn, (int64_t)H * Dn, Dn, (int64_t)H * W, H, Dn, (int64_t)R * Dn, W,
                               st);
        if (e == hipSuccess)
            e = launch_rope_q<float>((const float *)q_rope, pos, (float *)q_cat, T, H, R, Dr,
                                     d->rope_base, st);
    } else {
        if (Dn % 8) return MLA_ERR_UNSUPPORTED;
        e = launch_absorb_bf16((const bf16 *)q_nope, (const bf16 *)q_rope, pos, (const bf16 *)wk_b,
                               (bf16 *)q_cat, T, H, R, Dn, Dr, d->rope_base, st);
    }
    return hip_status(e);
}

size_t mla_prefill_workspace_bytes(const mla_dims *d, mla_dtype kv, int32_t T, int32_t n_kv,
                                   uint32_t scratch_cap_mib) {
    if (!dims_ok(d) || T < 1 || n_kv < 1) return 0;
    if (kv != MLA_BF16 || !bf16_attn_dims(d)) return 0;
    const int H = d->n_head;
    const double size_mib = (double)T * (double)n_kv * (double)H * 4.0 / (1024.0 * 1024.0);
    const int hc = mla_heads_per_chunk(H, size_mib, scratch_cap_mib);
    return prefill_workspace_bytes(T, H, n_kv, hc);
}

int mla_attn_prefill(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_cat,
                     const int32_t *pos, int32_t T, const void *kv_cache, int32_t n_kv,
                     void *o_lat, float *lse, uint32_t scratch_cap_mib, void *workspace,
                     size_t workspace_bytes, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || T < 0 || n_kv < 1) return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && kv != MLA_BF16 && kv != MLA_Q8_0) return MLA_ERR_INVALID_ARG;
    if (kv == MLA_Q8_0) return MLA_ERR_UNSUPPORTED;
    if (kv != act) return MLA_ERR_INVALID_ARG;
    if (T == 0) return MLA_OK;
    if (!q_cat || !pos || !kv_cache || !o_lat) return MLA_ERR_INVALID_ARG;
    const int H = d->n_head;
    const double size_mib = (double)T * (double)n_kv * (double)H * 4.0 / (1024.0 * 1024.0);
    const int hc = mla_heads_per_chunk(H, size_mib, scratch_cap_mib);
    hipStream_t st = as_stream(stream);
    if (act == MLA_F32) {
        if (d->kv_lora_rank > 1024) return MLA_ERR_UNSUPPORTED;
        for (int h0 = 0; h0 < H; h0 += hc) {
            hipError_t e = launch_flash_simt_prefill(*d, (const float *)q_cat, pos, T,
                                                     (const float *)kv_cache, n_kv, h0, hc,
                                                     (float *)o_lat, lse, st);
            if (e != hipSuccess) return MLA_ERR_HIP;
        }
        return MLA_OK;
    }
    if (!bf16_attn_dims(d)) return MLA_ERR_UNSUPPORTED;
    if ((int64_t)T * hc > INT32_MAX / 2) return MLA_ERR_UNSUPPORTED;
    const size_t need = prefill_workspace_bytes(T, H, n_kv, hc);
    if (need && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
    return hip_status(launch_flash_prefill_bf16((const bf16 *)q_cat, pos, T, H,
                                                (const bf16 *)kv_cache, n_kv, hc, d->scale,
                                                (bf16 *)o_lat, lse, workspace, st));
}

int32_t mla_decode_auto_splits(const mla_dims *d, mla_dtype kv, int32_t B, int32_t n_kv_max) {
    if (!dims_ok(d) || B < 1 || n_kv_max < 1) return 0;
    return auto_splits(d, kv, B, n_kv_max);
}

// Decode of many sequences at once: with 128 heads (one row group of the prefill kernel per
// sequence) and at least DEC_GROUPED_MIN_B sequences, the bf16 decode runs on the prefill
// kernel over the batched caches (its key parts and their merge are the splits and their
// combine); that kernel's tile loop sustains more of the MFMA rate than the 64-head decode
// kernel's, and enough sequences fill the CUs.  Only with the automatic split count.
constexpr int DEC_GROUPED_MIN_B = 16;
static bool decode_grouped(const mla_dims *d, int kv, int B, int n_splits) {
    return kv == MLA_BF16 && n_splits == 0 && d->n_head == 128 && bf16_attn_dims(d) &&
           B >= DEC_GROUPED_MIN_B;
}

// Workspace bytes the decode of these arguments uses with a cache of type kv: the split
// partials (float32 on the float32 path, bfloat16 otherwise) and their lse, or the batched
// prefill's part buffers.  mla_decode_workspace_bytes reports the largest of these over the
// cache types.
static size_t decode_need_bytes(const mla_dims *d, int kv, int32_t B, int32_t n_kv_max,
                                int32_t n_splits);

size_t mla_decode_workspace_bytes(const mla_dims *d, int32_t B, int32_t n_kv_max,
                                  int32_t n_splits) {
    if (!dims_ok(d) || B < 1 || n_kv_max < 1 || n_splits < 0 || n_splits > MAX_SPLITS) return 0;
    int S = n_splits;
    if (S == 0) {
        // the largest automatic choice over cache types
        // (and the transposed-V decode, on 128-head workgroups)
        const int a = auto_splits(d, MLA_F32, B, n_kv_max), b = auto_splits(d, MLA_BF16, B, n_kv_max),
                  c = auto_splits(d, MLA_Q8_0, B, n_kv_max),
                  v = splits_for(d, decode_wide_heads(), B, n_kv_max);
        S = a > b ? a : b;
        S = S > c ? S : c;
        S = S > v ? S : v;
    }
    if (S > n_kv_max) S = n_kv_max;
    const size_t rows = (size_t)B * S * d->n_head;
    // partial outputs: float32 on the float32 path, bfloat16 otherwise; sized for the larger
    size_t bytes = align256(rows * d->kv_lora_rank * sizeof(float)) + align256(rows * sizeof(float));
    if (decode_grouped(d, MLA_BF16, B, n_splits)) {
        const size_t g = prefill_workspace_bytes(B, d->n_head, n_kv_max, 128, true);
        bytes = g > bytes ? g : bytes;
    }
    return bytes;
}

// mla_attn_decode with the workspace checked against the exact need of this cache type
// (mla_attn_decode's own check is against the larger size its callers are told).
static int decode_impl(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_cat,
                       const void *kv_cache, int64_t kv_seq_stride_bytes, const int32_t *n_kv,
                       int32_t B, int32_t n_kv_max, int32_t n_splits, void *o_lat, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream);

int mla_attn_decode(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_cat,
                    const void *kv_cache, int64_t kv_seq_stride_bytes, const int32_t *n_kv,
                    int32_t B, int32_t n_kv_max, int32_t n_splits, void *o_lat, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (dims_ok(d) && B > 0 && n_kv_max > 0 && n_splits >= 0 && n_splits <= MAX_SPLITS &&
        workspace_bytes < mla_decode_workspace_bytes(d, B, n_kv_max, n_splits))
        workspace_bytes = 0;  // smaller than this call's documented size: rejected below
    return decode_impl(d, act, kv, q_cat, kv_cache, kv_seq_stride_bytes, n_kv, B, n_kv_max,
                       n_splits, o_lat, lse, workspace, workspace_bytes, stream);
}

static int decode_impl(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_cat,
                       const void *kv_cache, int64_t kv_seq_stride_bytes, const int32_t *n_kv,
                       int32_t B, int32_t n_kv_max, int32_t n_splits, void *o_lat, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || B < 0 || n_kv_max < 1 || n_splits < 0 ||
        n_splits > MAX_SPLITS)
        return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && kv != MLA_BF16 && kv != MLA_Q8_0) return MLA_ERR_INVALID_ARG;
    if (kv == MLA_F32 && act != MLA_F32) return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && act != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (B == 0) return MLA_OK;
    if (!q_cat || !kv_cache || !n_kv || !o_lat || !workspace) return MLA_ERR_INVALID_ARG;
    const int W = d->kv_lora_rank + d->qk_rope;
    int64_t row_bytes;
    if (kv == MLA_Q8_0) {
        if (W % 32) return MLA_ERR_INVALID_ARG;
        row_bytes = (int64_t)W / 32 * 34;
    } else {
        row_bytes = (int64_t)W * (kv == MLA_F32 ? 4 : 2);
    }
    if (B > 1 && kv_seq_stride_bytes < row_bytes * n_kv_max) return MLA_ERR_INVALID_ARG;
    if (kv_seq_stride_bytes < 0 || kv_seq_stride_bytes % 16)
        return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && !bf16_attn_dims(d)) return MLA_ERR_UNSUPPORTED;
    if (kv == MLA_F32 && d->kv_lora_rank > 1024) return MLA_ERR_UNSUPPORTED;

    if (workspace_bytes < decode_need_bytes(d, kv, B, n_kv_max, n_splits)) return MLA_ERR_WORKSPACE;
    if (decode_grouped(d, kv, B, n_splits)) {
        if ((uintptr_t)workspace & 15) return MLA_ERR_INVALID_ARG;
        return hip_status(launch_flash_prefill_bf16(
            (const bf16 *)q_cat, nullptr, B, d->n_head, (const bf16 *)kv_cache, n_kv_max, 128,
            d->scale, (bf16 *)o_lat, lse, workspace, as_stream(stream), kv_seq_stride_bytes, n_kv));
    }
    int S = n_splits ? n_splits : auto_splits(d, kv, B, n_kv_max);
    if (S > n_kv_max) S = n_kv_max;
    int split_len, count;
    split_plan(kv, n_kv_max, S, &split_len, &count);
    const size_t rows = (size_t)B * count * d->n_head;
    const size_t po_elem = kv == MLA_F32 ? sizeof(float) : sizeof(bf16);
    void *part_o = workspace;
    float *part_lse = (float *)((char *)workspace + align256(rows * d->kv_lora_rank * po_elem));
    hipStream_t st = as_stream(stream);
    hipError_t e;
    if (kv == MLA_F32) {
        e = launch_flash_simt_decode(*d, (const float *)q_cat, (const float *)kv_cache,
                                     kv_seq_stride_bytes / 4, n_kv, n_kv_max, B, count, split_len,
                                     (float *)part_o, part_lse, st);
        if (e == hipSuccess)
            e = launch_combine<float, float>((const float *)part_o, part_lse, B, d->n_head,
                                             d->kv_lora_rank, count, (float *)o_lat, lse, st);
    } else {
        if (decode_q8_wide(d, kv))
            e = launch_flash_decode_q8_wide((const bf16 *)q_cat, kv_cache, kv_seq_stride_bytes, n_kv,
                                            n_kv_max, B, d->n_head, count, split_len, d->scale,
                                            (bf16 *)part_o, part_lse, st);
        else
            e = launch_flash_decode_bf16((const bf16 *)q_cat, kv_cache, kv == MLA_Q8_0,
                                         kv_seq_stride_bytes, n_kv, n_kv_max, B, d->n_head, count,
                                         split_len, d->scale, (bf16 *)part_o, part_lse, st);
        if (e == hipSuccess)
            e = launch_combine<bf16, bf16>((const bf16 *)part_o, part_lse, B, d->n_head,
                                           d->kv_lora_rank, count, (bf16 *)o_lat, lse, st);
    }
    return hip_status(e);
}

static size_t decode_need_bytes(const mla_dims *d, int kv, int32_t B, int32_t n_kv_max,
                                int32_t n_splits) {
    if (decode_grouped(d, kv, B, n_splits))
        return prefill_workspace_bytes(B, d->n_head, n_kv_max, 128, true);
    int S = n_splits ? n_splits : auto_splits(d, kv, B, n_kv_max);
    if (S > n_kv_max) S = n_kv_max;
    int split_len, count;
    split_plan(kv, n_kv_max, S, &split_len, &count);
    const size_t rows = (size_t)B * count * d->n_head;
    const size_t po_elem = kv == MLA_F32 ? sizeof(float) : sizeof(bf16);
    return align256(rows * d->kv_lora_rank * po_elem) + align256(rows * sizeof(float));
}

// The allocation-free decode: the workspace is a file-scope device array of
// MLA_DECODE_STATIC_BYTES, one copy per device (the runtime creates it when the library's
// code is loaded onto that device).  Host code never passes the array's name to a kernel:
// its device address, taken once per device with hipGetSymbolAddress, is kept in
// static_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[MLA_DECODE_STATIC_BYTES];

static std::mutex static_scratch_lock;
static void *static_scratch_ptr[64];

static int static_scratch(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> guard(static_scratch_lock);
    if (!static_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
        static_scratch_ptr[dev] = p;
    }
    *out = static_scratch_ptr[dev];
    return MLA_OK;
}

int mla_attn_decode_static(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_cat,
                           const void *kv_cache, int64_t kv_seq_stride_bytes,
                           const int32_t *n_kv, int32_t B, int32_t n_kv_max, int32_t n_splits,
                           void *o_lat, float *lse, void *stream) {
    if (!dims_ok(d) || B < 0 || n_kv_max < 1 || n_splits < 0 || n_splits > MAX_SPLITS)
        return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && kv != MLA_BF16 && kv != MLA_Q8_0) return MLA_ERR_INVALID_ARG;
    if (B == 0) return MLA_OK;
    if (decode_need_bytes(d, kv, B, n_kv_max, n_splits) > MLA_DECODE_STATIC_BYTES)
        return MLA_ERR_WORKSPACE;
    if (!q_cat || !kv_cache || !n_kv || !o_lat) return MLA_ERR_INVALID_ARG;
    void *ws = nullptr;
    const int s = static_scratch(&ws);
    if (s != MLA_OK) return s;
    return decode_impl(d, act, kv, q_cat, kv_cache, kv_seq_stride_bytes, n_kv, B, n_kv_max,
                       n_splits, o_lat, lse, ws, MLA_DECODE_STATIC_BYTES, stream);
}

int mla_cache_transpose_v(const mla_dims *d, mla_dtype kv, const void *kv_cache,
                          int64_t kv_seq_stride_bytes, int32_t B, int32_t row0, int32_t row1,
                          void *v_t, int64_t vt_seq_stride_bytes, int32_t vt_ld, void *stream) {
    if (!dims_ok(d) || B < 0 || B > 65535 || row0 < 0 || row1 < row0 || vt_ld < 1 ||
        vt_ld > MAX_VT_LD)
        return MLA_ERR_INVALID_ARG;
    if (kv != MLA_BF16) return kv == MLA_F32 || kv == MLA_Q8_0 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
    if (!bf16_attn_dims(d)) return MLA_ERR_UNSUPPORTED;
    if (B == 0 || row1 == row0) return MLA_OK;
    if (!kv_cache || !v_t) return MLA_ERR_INVALID_ARG;
    const int64_t row_bytes = (int64_t)(d->kv_lora_rank + d->qk_rope) * 2;
    const int64_t rows_need = ((int64_t)row1 + 31) / 32 * 32;  // whole 32-key groups
    if (vt_ld < rows_need || kv_seq_stride_bytes % 2 || vt_seq_stride_bytes % 2) return MLA_ERR_INVALID_ARG;
    if (B > 1 && (kv_seq_stride_bytes < row_bytes * row1 ||
                  vt_seq_stride_bytes < (int64_t)d->kv_lora_rank * vt_ld * 2))
        return MLA_ERR_INVALID_ARG;
    return hip_status(launch_transpose_v((const bf16 *)kv_cache, kv_seq_stride_bytes, B, row0, row1,
                                         (bf16 *)v_t, vt_seq_stride_bytes, vt_ld, as_stream(stream)));
}

int mla_attn_decode_vt(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_cat,
                       const void *kv_cache, int64_t kv_seq_stride_bytes, const void *v_t,
                       int64_t vt_seq_stride_bytes, int32_t vt_ld, const int32_t *n_kv, int32_t B,
                       int32_t n_kv_max, int32_t n_splits, void *o_lat, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!dims_ok(d) || B < 0 || n_kv_max < 1 || n_splits < 0 || n_splits > MAX_SPLITS ||
        vt_ld < 1 || vt_ld > MAX_VT_LD)
        return MLA_ERR_INVALID_ARG;
    if (act != MLA_BF16 || kv != MLA_BF16)
        return (act == MLA_F32 || act == MLA_BF16) && (kv == MLA_F32 || kv == MLA_Q8_0)
                   ? MLA_ERR_UNSUPPORTED
                   : MLA_ERR_INVALID_ARG;
    if (!bf16_attn_dims(d)) return MLA_ERR_UNSUPPORTED;
    if (B == 0) return MLA_OK;
    if (!q_cat || !kv_cache || !v_t || !n_kv || !o_lat || !workspace) return MLA_ERR_INVALID_ARG;
    const int64_t row_bytes = (int64_t)(d->kv_lora_rank + d->qk_rope) * 2;
    const int64_t rows_need = ((int64_t)n_kv_max + 31) / 32 * 32;
    if (kv_seq_stride_bytes < 0 || kv_seq_stride_bytes % 16 || vt_seq_stride_bytes < 0 ||
        vt_seq_stride_bytes % 16 || vt_ld % 8 || vt_ld < rows_need || ((uintptr_t)v_t & 15))
        return MLA_ERR_INVALID_ARG;
    if (B > 1 && (kv_seq_stride_bytes < row_bytes * n_kv_max ||
                  vt_seq_stride_bytes < (int64_t)d->kv_lora_rank * vt_ld * 2))
        return MLA_ERR_INVALID_ARG;
    int S = n_splits ? n_splits : splits_for(d, decode_wide_heads(), B, n_kv_max);
    if (S > n_kv_max) S = n_kv_max;
    int split_len, count;
    split_plan(MLA_BF16, n_kv_max, S, &split_len, &count);
    const size_t rows = (size_t)B * count * d->n_head;
    const size_t need = align256(rows * d->kv_lora_rank * sizeof(bf16)) + align256(rows * sizeof(float));
    if (workspace_bytes < need || workspace_bytes < mla_decode_workspace_bytes(d, B, n_kv_max, n_splits))
        return MLA_ERR_WORKSPACE;
    bf16 *part_o = (bf16 *)workspace;
    float *part_lse = (float *)((char *)workspace + align256(rows * d->kv_lora_rank * sizeof(bf16)));
    hipStream_t st = as_stream(stream);
    hipError_t e = launch_flash_decode_bf16_wide((const bf16 *)q_cat, kv_cache, kv_seq_stride_bytes,
                                                 v_t, vt_seq_stride_bytes, vt_ld, n_kv, n_kv_max, B,
                                                 d->n_head, count, split_len, d->scale, part_o,
                                                 part_lse, st);
    if (e == hipSuccess)
        e = launch_combine<bf16, bf16>(part_o, part_lse, B, d->n_head, d->kv_lora_rank, count,
                                       (bf16 *)o_lat, lse, st);
    return hip_status(e);
}

int mla_out_proj(const mla_dims *d, mla_dtype act, const void *o_lat, const void *wv_b,
                 const void *wo, void *v_scratch, void *out, int32_t T, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || T < 0) return MLA_ERR_INVALID_ARG;
    if (T == 0) return MLA_OK;
    if (!o_lat || !wv_b || !wo || !v_scratch || !out) return MLA_ERR_INVALID_ARG;
    const int H = d->n_head, R = d->kv_lora_rank, Dv = d->v_head, D = d->d_model;
    const int HDv = H * Dv;
    hipStream_t st = as_stream(stream);
    hipError_t e;
    if (act == MLA_F32) {
        e = launch_gemm_nt_f32((const float *)o_lat, (const float *)wv_b, (float *)v_scratch, T,
                               Dv, R, (int64_t)H * R, R, HDv, H, R, (int64_t)Dv * R, Dv, st);
        if (e == hipSuccess)
            e = launch_gemm_nt_f32((const float *)v_scratch, (const float *)wo, (float *)out, T, D,
                                   HDv, HDv, HDv, D, 1, 0, 0, 0, st);
    } else {
        if (R % 8 || Dv % 8) return MLA_ERR_UNSUPPORTED;
        const bf16 *ol = (const bf16 *)o_lat, *wv = (const bf16 *)wv_b, *w_o = (const bf16 *)wo;
        bf16 *v = (bf16 *)v_scratch;
        // few tokens (decode): both products are streams over the weights
        const bool few = gemv_nt_bf16_ok(ol, wv, T, R, (int64_t)H * R, R, R, (int64_t)Dv * R) &&
                         gemv_nt_bf16_ok(v, w_o, T, HDv, HDv, HDv, 0, 0);
        if (few) {
            e = launch_gemv_nt_bf16(ol, wv, v, T, Dv, R, (int64_t)H * R, R, HDv, H, R,
                                    (int64_t)Dv * R, Dv, st);
            if (e == hipSuccess)
                e = launch_gemv_nt_bf16(v, w_o, (bf16 *)out, T, D, HDv, HDv, HDv, D, 1, 0, 0, 0, st);
        } else {
            e = launch_gemm_nt_bf16(ol, wv, v, T, Dv, R, (int64_t)H * R, R, HDv, H, R,
                                    (int64_t)Dv * R, Dv, st);
            if (e == hipSuccess)
                e = launch_gemm_nt_bf16(v, w_o, (bf16 *)out, T, D, HDv, HDv, HDv, D, 1, 0, 0, 0, st);
        }
    }
    return hip_status(e);
}

int mla_quantize_q8_0(const float *x, void *rows, int64_t n_rows, int32_t width, void *stream) {
    if (width <= 0 || width % 32 || n_rows < 0) return MLA_ERR_INVALID_ARG;
    if (n_rows == 0) return MLA_OK;
    if (!x || !rows) return MLA_ERR_INVALID_ARG;
    return hip_status(launch_quantize_q8_0(x, (uint8_t *)rows, n_rows, width, as_stream(stream)));
}

int mla_dequant_q8_0(const void *rows, float *out, int64_t n_rows, int32_t width, void *stream) {
    if (width <= 0 || width % 32 || n_rows < 0) return MLA_ERR_INVALID_ARG;
    if (n_rows == 0) return MLA_OK;
    if (!rows || !out) return MLA_ERR_INVALID_ARG;
    return hip_status(launch_dequant_q8_0((const uint8_t *)rows, out, n_rows, width,
                                          as_stream(stream)));
}

// The materialised path's kernels are written for the DeepSeek head shape.
static bool materialized_dims(const mla_dims *d) {
    return d->qk_nope == 128 && d->qk_rope == 64 && d->v_head == 128 && d->kv_lora_rank % 8 == 0 &&
           d->scale > 0.0f;
}

static int materialized_hc(const mla_dims *d, int32_t T, int32_t n_kv, uint32_t cap) {
    const double size_mib = (double)T * (double)n_kv * (double)d->n_head * 4.0 / (1024.0 * 1024.0);
    return mla_heads_per_chunk(d->n_head, size_mib, cap);
}

size_t mla_materialized_workspace_bytes(const mla_dims *d, int32_t T, int32_t n_kv,
                                        uint32_t scratch_cap_mib) {
    if (!dims_ok(d) || T < 1 || n_kv < 1 || !materialized_dims(d)) return 0;
    return materialized_workspace_bytes(T, d->n_head, d->kv_lora_rank, n_kv,
                                        materialized_hc(d, T, n_kv, scratch_cap_mib));
}

int mla_prefill_materialized(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *q_nope,
                             const void *q_rope, const int32_t *pos, int32_t T,
                             const void *kv_cache, int32_t n_kv, const void *wk_b,
                             const void *wv_b, const void *wo, void *v_out, void *out, float *lse,
                             uint32_t scratch_cap_mib, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (!dims_ok(d) || !act_ok(act) || T < 0 || n_kv < 1) return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && kv != MLA_BF16 && kv != MLA_Q8_0) return MLA_ERR_INVALID_ARG;
    if (act != MLA_BF16 || kv != MLA_BF16 || !materialized_dims(d)) return MLA_ERR_UNSUPPORTED;
    if (T == 0) return MLA_OK;
    if (!q_nope || !q_rope || !pos || !kv_cache || !wk_b || !wv_b || !v_out) return MLA_ERR_INVALID_ARG;
    if ((wo == nullptr) != (out == nullptr)) return MLA_ERR_INVALID_ARG;
    const int H = d->n_head, R = d->kv_lora_rank;
    const int hc = materialized_hc(d, T, n_kv, scratch_cap_mib);
    const size_t need = materialized_workspace_bytes(T, H, R, n_kv, hc);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return MLA_ERR_WORKSPACE;
    hipStream_t st = as_stream(stream);
    hipError_t e = launch_prefill_materialized(
        (const bf16 *)q_nope, (const bf16 *)q_rope, pos, T, H, R, (const bf16 *)kv_cache, n_kv,
        (const bf16 *)wk_b, (const bf16 *)wv_b, hc, d->scale, d->rope_base, (bf16 *)v_out, lse,
        workspace, st);
    if (e == hipSuccess && wo) {
        const int HDv = H * d->v_head;
        e = launch_gemm_nt_bf16((const bf16 *)v_out, (const bf16 *)wo, (bf16 *)out, T, d->d_model,
                                HDv, HDv, HDv, d->d_model, 1, 0, 0, 0, st);
    }
    return hip_status(e);
}

static bool pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

static int cache_append_impl(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *c_kv,
                             const void *k_rope, const int32_t *pos, const int64_t *dst_row,
                             int32_t T, void *cache, int64_t n_rows, bool hadamard, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || T < 0 || n_rows < 0) return MLA_ERR_INVALID_ARG;
    if (kv != MLA_F32 && kv != MLA_BF16 && kv != MLA_Q8_0) return MLA_ERR_INVALID_ARG;
    if (kv != MLA_Q8_0 && kv != act) return MLA_ERR_INVALID_ARG;
    const int R = d->kv_lora_rank, Dr = d->qk_rope;
    if (kv == MLA_Q8_0 && (R + Dr) % 32) return MLA_ERR_INVALID_ARG;
    if ((int64_t)(R + Dr) * 4 > 65536) return MLA_ERR_UNSUPPORTED;
    if (T == 0) return MLA_OK;
    if (!c_kv || !k_rope || !pos || !cache) return MLA_ERR_INVALID_ARG;
    hipStream_t st = as_stream(stream);
    hipError_t e;
    if (act == MLA_F32)
        e = launch_cache_append<float>((const float *)c_kv, (const float *)k_rope, pos, dst_row, T,
                                       R, Dr, d->rope_base, kv, hadamard, cache, n_rows, st);
    else
        e = launch_cache_append<bf16>((const bf16 *)c_kv, (const bf16 *)k_rope, pos, dst_row, T, R,
                                      Dr, d->rope_base, kv, hadamard, cache, n_rows, st);
    return hip_status(e);
}

int mla_cache_append(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *c_kv,
                     const void *k_rope, const int32_t *pos, const int64_t *dst_row, int32_t T,
                     void *cache, int64_t n_rows, void *stream) {
    return cache_append_impl(d, act, kv, c_kv, k_rope, pos, dst_row, T, cache, n_rows, false,
                             stream);
}

int mla_cache_append_hadamard(const mla_dims *d, mla_dtype act, mla_dtype kv, const void *c_kv,
                              const void *k_rope, const int32_t *pos, const int64_t *dst_row,
                              int32_t T, void *cache, int64_t n_rows, void *stream) {
    if (!d || !pow2(d->kv_lora_rank)) return MLA_ERR_INVALID_ARG;
    return cache_append_impl(d, act, kv, c_kv, k_rope, pos, dst_row, T, cache, n_rows, true,
                             stream);
}

int mla_hadamard_weights(const mla_dims *d, mla_dtype act, const void *wk_b, const void *wv_b,
                         void *wk_b_rot, void *wv_b_rot, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || !pow2(d->kv_lora_rank)) return MLA_ERR_INVALID_ARG;
    if (!wk_b || !wv_b || !wk_b_rot || !wv_b_rot) return MLA_ERR_INVALID_ARG;
    if (wk_b == wk_b_rot || wv_b == wv_b_rot) return MLA_ERR_INVALID_ARG;
    if (d->kv_lora_rank > 16384) return MLA_ERR_UNSUPPORTED;
    hipStream_t st = as_stream(stream);
    const int H = d->n_head, R = d->kv_lora_rank, Dn = d->qk_nope, Dv = d->v_head;
    hipError_t e;
    if (act == MLA_F32)
        e = launch_hadamard_weights<float>((const float *)wk_b, (const float *)wv_b,
                                           (float *)wk_b_rot, (float *)wv_b_rot, H, R, Dn, Dv, st);
    else
        e = launch_hadamard_weights<bf16>((const bf16 *)wk_b, (const bf16 *)wv_b, (bf16 *)wk_b_rot,
                                          (bf16 *)wv_b_rot, H, R, Dn, Dv, st);
    return hip_status(e);
}

int mla_wkv_b_merge(const mla_dims *d, mla_dtype act, mla_dtype out, const void *wk_b,
                    const void *wv_b, void *wkv_b, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || (out != act && out != MLA_Q8_0)) return MLA_ERR_INVALID_ARG;
    if (!wk_b || !wv_b || !wkv_b) return MLA_ERR_INVALID_ARG;
    if (out == MLA_Q8_0 && d->kv_lora_rank % 32) return MLA_ERR_INVALID_ARG;
    const bool q8 = out == MLA_Q8_0;
    const int H = d->n_head, R = d->kv_lora_rank, Dn = d->qk_nope, Dv = d->v_head;
    hipStream_t st = as_stream(stream);
    hipError_t e = act == MLA_F32
                       ? launch_wkv_merge<float>((const float *)wk_b, (const float *)wv_b, wkv_b,
                                                 q8, H, R, Dn, Dv, st)
                       : launch_wkv_merge<bf16>((const bf16 *)wk_b, (const bf16 *)wv_b, wkv_b, q8,
                                                H, R, Dn, Dv, st);
    return hip_status(e);
}

int mla_wkv_b_split(const mla_dims *d, mla_dtype in, mla_dtype act, const void *wkv_b,
                    void *wk_b, void *wv_b, void *stream) {
    if (!dims_ok(d) || !act_ok(act) || (in != act && in != MLA_Q8_0)) return MLA_ERR_INVALID_ARG;
    if (!wk_b || !wv_b || !wkv_b) return MLA_ERR_INVALID_ARG;
    if (in == MLA_Q8_0 && d->kv_lora_rank % 32) return MLA_ERR_INVALID_ARG;
    const bool q8 = in == MLA_Q8_0;
    const int H = d->n_head, R = d->kv_lora_rank, Dn = d->qk_nope, Dv = d->v_head;
    hipStream_t st = as_stream(stream);
    hipError_t e = act == MLA_F32
                       ? launch_wkv_split<float>(wkv_b, q8, (float *)wk_b, (float *)wv_b, H, R, Dn,
                                                 Dv, st)
                       : launch_wkv_split<bf16>(wkv_b, q8, (bf16 *)wk_b, (bf16 *)wv_b, H, R, Dn, Dv,
                                                st);
    return hip_status(e);
}

}  // extern "C"
