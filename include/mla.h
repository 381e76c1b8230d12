/*
 * mla.h -- C ABI of the MI355X (gfx950) absorbed Multi-head Latent Attention library.
 *
 * The four calls follow the order in which the page "ik_llama.cpp MLA matrix
 * absorption" (czykbl.com/news/93068) applies the absorbed method, section 4:
 * project q_nope through wk_b into the latent space (mla_absorb_q), attend
 * directly on the latent cache (mla_attn_prefill / mla_attn_decode), then
 * decompress late through wv_b and apply wo (mla_out_proj).
 *
 * Conventions for every call
 *   - Pointers are device pointers unless stated otherwise.  The caller owns every
 *     buffer (weights, cache, activations, outputs, workspace); the library never
 *     allocates on these paths and never frees caller memory.
 *   - Tensors are dense, row-major, innermost dimension last.  Element type is given
 *     by the mla_dtype arguments.  Device pointers must be 16-byte aligned.
 *   - Launches are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *     Nothing synchronises.
 *   - Calls may come from several host threads at once.  The host-side plans the library
 *     keeps between calls (prefill work lists, kernel attributes) are guarded by a lock.
 *     Calls whose output or workspace buffers overlap must not run concurrently, on any
 *     stream.
 *   - Every call validates its arguments before launching anything and returns an
 *     mla_status; nothing aborts or exits.  A shape or dtype a kernel does not
 *     implement returns MLA_ERR_UNSUPPORTED: no call silently switches to another
 *     path.  A HIP launch error returns MLA_ERR_HIP.
 *
 * Notation: H heads, R = kv_lora_rank, Dn = qk_nope, Dr = qk_rope, Dv = v_head,
 * D = d_model, W = R + Dr (latent cache row width), T query tokens, N cached rows.
 *
 * Data types
 *   MLA_F32  : activations, weights, cache and o_lat in float32 (any dims).
 *   MLA_BF16 : activations, weights, cache and o_lat in bfloat16, float32
 *              accumulation; attention kernels need R = 512, Dr = 64 (the
 *              DeepSeek latent shape: K 576 / V 512 / rope 64, page "ik_llama.cpp
 *              PR #394", section 3.1).
 *   MLA_Q8_0 : cache only (attention decode): each 32-value run of a row is a
 *              34-byte block {binary16 scale d (little endian), int8 q[32]},
 *              value = d * q.  A 576-wide row is 612 bytes.  Activations bf16.
 *   lse outputs are always float32.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, odd Dr, bad dtype combination */
    MLA_ERR_UNSUPPORTED = -2, /* valid request that no kernel implements (see each call) */
    MLA_ERR_WORKSPACE = -3,   /* workspace smaller than the matching *_workspace_bytes() */
    MLA_ERR_HIP = -4          /* the HIP runtime reported an error on launch */
} mla_status;

typedef enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1, MLA_Q8_0 = 2 } mla_dtype;

/* Layer dimensions.  scale multiplies the score (DeepSeek: 1/sqrt(Dn + Dr));
 * rope_base is the RoPE frequency base (10000). */
typedef struct mla_dims {
    int32_t n_head, kv_lora_rank, qk_nope, qk_rope, v_head, d_model;
    float scale;
    float rope_base;
} mla_dims;

/* K absorption and query RoPE (absorption page, sections 3 and 4).
 *   q_cat[t][h][0:R]  = sum_d wk_b[h][l][d] * q_nope[t][h][d]   (q_lat; the
 *                       mul_mat(wk_b, q_nope) of section 4)
 *   q_cat[t][h][R:W]  = RoPE(q_rope[t][h], pos[t])  -- RoPE is not absorbable
 *                       (section 3): adjacent pairs (x[2i], x[2i+1]) rotated by
 *                       pos * rope_base^(-2i/Dr), angles in double precision.
 * q_nope [T][H][Dn], q_rope [T][H][Dr] (pre-RoPE), pos [T] int32 (device),
 * wk_b [H][R][Dn] (the split layout ggml {Dn,R,H} of the PR #394 page, section
 * 3.2), q_cat [T][H][W].  All of dtype act (MLA_F32 or MLA_BF16).
 * T == 0 is a no-op.  Errors: INVALID_ARG for nulls, T < 0, odd Dr, act Q8_0. */
int mla_absorb_q(const mla_dims *dims, mla_dtype act, const void *q_nope, const void *q_rope,
                 const int32_t *pos, const void *wk_b, void *q_cat, int32_t T, void *stream);

/* Causal attention on the latent cache (absorption page, sections 4 and 5).
 * For each query t and head h, key row j is visible iff j <= pos[t] and j < n_kv:
 *   s_j   = scale * (q_cat[t][h][0:R] . c_kv[j] + q_cat[t][h][R:W] . k_rope[j])
 *           (the two-term "move elision" score over the row's adjacent parts)
 *   o_lat[t][h] = sum_j softmax(s)_j * c_kv[j]       (the latent weighted sum)
 *   lse[t][h]   = log sum_j exp(s_j)                 (natural log)
 * Rows with no visible key get o_lat = 0 and lse = -inf.
 * q_cat [T][H][W] (act), pos [T] int32, kv_cache [n_kv][W] (kv dtype; row j holds the
 * token at position j, k_rope stored post-RoPE), o_lat [T][H][R] (act), lse [T][H]
 * float32 or NULL.
 * scratch_cap_mib is the -amb analogue (absorption page, section 8.3): with
 * size = T * n_kv * H * 4 bytes (the K x Q intermediate an unfused path would hold),
 * heads are processed in chunks of mla_heads_per_chunk(H, size, cap) heads.  0 means
 * unlimited; a value in (0, 128) is raised to 128.  The fused kernel holds no such
 * intermediate, so the cap only changes the work decomposition: results are
 * bitwise identical for every cap.
 * Supported: act == kv == MLA_F32 (any dims), act == kv == MLA_BF16 (R 512, Dr 64).
 * workspace: device memory of at least mla_prefill_workspace_bytes(dims, kv, T, n_kv,
 * scratch_cap_mib) bytes (may be NULL when that is 0).  When few row groups would leave
 * the longest ones setting the time, the bf16 kernel cuts every row's keys into parts
 * at fixed boundaries and merges the parts' partial results with the split-KV combine
 * (the same log-sum-exp merge as decode); the workspace holds those partials.  Its
 * contents need not be initialised.  Calls sharing a workspace must not overlap.
 * Errors: INVALID_ARG (nulls, T < 0, n_kv < 1, dtype mix), UNSUPPORTED (Q8_0 cache,
 * bf16 with other R/Dr), WORKSPACE (workspace missing or too small). */
int mla_attn_prefill(const mla_dims *dims, mla_dtype act, mla_dtype kv, const void *q_cat,
                     const int32_t *pos, int32_t T, const void *kv_cache, int32_t n_kv,
                     void *o_lat, float *lse, uint32_t scratch_cap_mib, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Workspace bytes mla_attn_prefill needs for these arguments (0: none).  Host-only;
 * returns 0 for invalid arguments. */
size_t mla_prefill_workspace_bytes(const mla_dims *dims, mla_dtype kv, int32_t T, int32_t n_kv,
                                   uint32_t scratch_cap_mib);

/* Heads per chunk for the -amb rule (absorption page, section 8.3): if
 * size_mib > cap, the smallest niter >= 2 with n_head % niter == 0 and
 * size_mib / niter <= cap gives n_head / niter heads per chunk (1 if none does);
 * cap 0 = unlimited, cap in (0,128) -> 128.  Host-only, never fails (returns
 * n_head for n_head < 1). */
int32_t mla_heads_per_chunk(int32_t n_head, double size_mib, uint32_t cap_mib);

/* Workspace bytes mla_attn_decode needs for B sequences of up to n_kv_max rows
 * with n_splits key splits per sequence (0 = the automatic choice).  Returns 0
 * for invalid arguments.  Host-only. */
size_t mla_decode_workspace_bytes(const mla_dims *dims, int32_t B, int32_t n_kv_max,
                                  int32_t n_splits);

/* The split count mla_attn_decode uses for n_splits == 0.  Host-only. */
int32_t mla_decode_auto_splits(const mla_dims *dims, mla_dtype kv, int32_t B, int32_t n_kv_max);

/* One decode step per sequence (absorption page, section 8: a separate kernel for
 * token generation).  Sequence b has n_kv[b] cache rows, its new token is already
 * appended, so its query (position n_kv[b]-1) sees every row.  The key range
 * [0, n_kv_max) is cut into n_splits contiguous splits; each split computes a
 * partial (o_s, lse_s) of the attention above over its rows, and a combine step
 * merges them:  lse = log sum_s exp(lse_s),  o_lat = sum_s exp(lse_s - lse) o_s.
 * Splits with no row contribute nothing (lse_s = -inf).
 * With n_splits == 0, a bf16 cache, H == 128 and B >= 16 the same computation runs on the
 * prefill kernel instead (one row group per sequence; its key parts, chosen by the
 * library, are the splits and merge by the same rule); the workspace size function
 * accounts for it.
 * q_cat [B][H][W] (act); kv_cache: sequence b's rows start at byte offset
 * b * kv_seq_stride_bytes (rows of W values for F32/BF16, of W/32*34 bytes for
 * Q8_0), the stride a multiple of 16 bytes (a Q8_0 sequence of N rows therefore takes
 * N*W/32*34 bytes rounded up to 16); n_kv [B] int32 on the device, each in
 * [1, n_kv_max]; o_lat [B][H][R] (act);
 * lse [B][H] float32 or NULL; workspace of at least
 * mla_decode_workspace_bytes(dims, B, n_kv_max, n_splits) bytes (device, 16-byte
 * aligned), contents need not be initialised.
 * Supported: act == kv == MLA_F32 (any dims); act == MLA_BF16 with kv MLA_BF16 or
 * MLA_Q8_0 (R 512, Dr 64).
 * Errors: INVALID_ARG, WORKSPACE, UNSUPPORTED as above. */
int mla_attn_decode(const mla_dims *dims, mla_dtype act, mla_dtype kv, const void *q_cat,
                    const void *kv_cache, int64_t kv_seq_stride_bytes, const int32_t *n_kv,
                    int32_t B, int32_t n_kv_max, int32_t n_splits, void *o_lat, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream);

/* The K + V^T cache form (absorption page, section 8.2: the -mla switch's mode 1 keeps a
 * K cache and a cache of V transposed).  Beside the row cache [c_kv | k_rope]
 * (bf16), each sequence holds the transpose of its latent part: v_t[c][p] for the R = 512
 * columns c, vt_ld positions p per column, bf16.  Within every aligned group of 32 keys
 * the position of key 32g + i is 32g + pi(i), pi swapping bits 2 and 3 of i (the order of
 * the decode kernel's score slots; pi is its own inverse).
 * mla_cache_transpose_v: writes v_t from the row cache for rows [row0, row1) of each of B
 *   sequences (sequence b's rows at b * kv_seq_stride_bytes, its v_t at
 *   b * vt_seq_stride_bytes); other positions are left as they are, so new rows can be
 *   added as they are appended.  vt_ld >= row1 rounded up to 32 and <= 2^26; B <= 65535.
 *   bf16 only.
 * mla_attn_decode_vt: mla_attn_decode (bf16 cache, same arguments, semantics and
 *   workspace size, mla_decode_workspace_bytes) with the O update reading V^T from v_t
 *   (rows [0, n_kv[b]) of v_t must have been written; positions up to n_kv_max rounded up
 *   to 32 are read and those past n_kv[b] ignored).  Workgroups of 128 heads; vt_ld a
 *   multiple of 8, >= n_kv_max rounded up to 32 and <= 2^26; strides multiples of 16
 *   bytes; v_t 16-byte aligned.
 * Errors: INVALID_ARG (nulls, sizes, strides, alignment), UNSUPPORTED (other dtypes or
 * dims: R 512 and Dr 64 as for the bf16 kernels), WORKSPACE. */
int mla_cache_transpose_v(const mla_dims *dims, mla_dtype kv, const void *kv_cache,
                          int64_t kv_seq_stride_bytes, int32_t B, int32_t row0, int32_t row1,
                          void *v_t, int64_t vt_seq_stride_bytes, int32_t vt_ld, void *stream);
int mla_attn_decode_vt(const mla_dims *dims, mla_dtype act, mla_dtype kv, const void *q_cat,
                       const void *kv_cache, int64_t kv_seq_stride_bytes, const void *v_t,
                       int64_t vt_seq_stride_bytes, int32_t vt_ld, const int32_t *n_kv,
                       int32_t B, int32_t n_kv_max, int32_t n_splits, void *o_lat, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Size of the device scratch array behind mla_attn_decode_static (bytes, per device). */
#define MLA_DECODE_STATIC_BYTES (64u << 20)

/* mla_attn_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The partial results live in a file-scope device array of
 * MLA_DECODE_STATIC_BYTES bytes, one per device, held from the library's load onto the
 * device until the process ends; the call allocates nothing (its first call on a device
 * looks up that device's array address once).  Same arguments, semantics, kernels and
 * results as mla_attn_decode.  The array needs no initialisation and keeps the last call's
 * partials.  All calls on one device share the one array: calls that may overlap in time
 * on one device (different streams, or host threads racing on one stream) race on it and
 * must be serialised by the caller.
 * Errors: as mla_attn_decode; WORKSPACE when this call's partials would need more than
 * MLA_DECODE_STATIC_BYTES (V3 dims: one or four sequences of up to 98304 rows with the
 * automatic split count fit; use mla_attn_decode with a workspace beyond that). */
int mla_attn_decode_static(const mla_dims *dims, mla_dtype act, mla_dtype kv, const void *q_cat,
                           const void *kv_cache, int64_t kv_seq_stride_bytes,
                           const int32_t *n_kv, int32_t B, int32_t n_kv_max, int32_t n_splits,
                           void *o_lat, float *lse, void *stream);

/* Late V decompression and output projection (absorption page, section 4):
 *   v[t][h*Dv + d] = sum_l wv_b[h][d][l] * o_lat[t][h][l]     (einsum bhqc,hdc->bhqd)
 *   out[t][e]      = sum_k wo[e][k] * v[t][k]                  (einsum hdD,bhqd->bqD)
 * o_lat [T][H][R], wv_b [H][Dv][R] (ggml {R,Dv,H} of the PR #394 page, section 3.2),
 * wo [D][H*Dv] (heads concatenated as reshape_2d(n_embd_head_v*n_head)),
 * v_scratch [T][H*Dv] (caller-owned; holds v afterwards), out [T][D]; all act.
 * Errors: INVALID_ARG (nulls, T < 0, act Q8_0). */
int mla_out_proj(const mla_dims *dims, mla_dtype act, const void *o_lat, const void *wv_b,
                 const void *wo, void *v_scratch, void *out, int32_t T, void *stream);

/* Q8_0 helpers (the 8-bit latent cache of the absorption page, section 8.1).
 * mla_quantize_q8_0: rows [n_rows][width] float32 -> Q8_0 bytes; per 32-block
 *   amax = max|x|, d = amax/127 (float32), q = round-half-away(x/d) clamped to
 *   [-127,127] (0 when d == 0), stored scale binary16(d) rounded to nearest even.
 * mla_dequant_q8_0: Q8_0 bytes -> float32, value = float(d) * q (exact).
 * width must be a positive multiple of 32 (else INVALID_ARG). */
int mla_quantize_q8_0(const float *x, void *rows, int64_t n_rows, int32_t width, void *stream);
int mla_dequant_q8_0(const void *rows, float *out, int64_t n_rows, int32_t width, void *stream);

/* Materialised prefill (the pp_opt path, absorption page, section 8.4): the same
 * attention as mla_absorb_q + mla_attn_prefill + mla_out_proj, computed the unabsorbed
 * way for long prompts over long caches.  Per chunk of heads (the -amb rule of section
 * 8.3 with the size of mla_attn_prefill) the keys and values are decompressed from the
 * cache once:  k_nope[h][j] = wk_b[h]^T c_kv[j] (Dn),  v[h][j] = wv_b[h] c_kv[j] (Dv),
 * then for every (t, h) and key j <= pos[t], j < n_kv:
 *   s_j = scale * ([q_nope[t][h] | RoPE(q_rope[t][h], pos[t])] . [k_nope[h][j] | k_rope[j]])
 *   v_out[t][h] = sum_j softmax(s)_j v[h][j],   lse[t][h] = log sum_j exp(s_j)
 * and, when wo is given, out[t] = wo . v_out[t] (heads concatenated).  Equal to the
 * absorbed chain by associativity (section 3); it needs 2(Dn+Dr+Dv) FLOP per visible
 * (query, key, head) instead of 2(2R+Dr), plus the decompression.
 * q_nope [T][H][Dn], q_rope [T][H][Dr] (pre-RoPE), pos [T] int32, kv_cache [n_kv][W],
 * wk_b [H][R][Dn], wv_b [H][Dv][R], wo [D][H*Dv] or NULL, v_out [T][H*Dv], out [T][D] or
 * NULL (both or neither of wo, out), lse [T][H] float32 or NULL.  Rows with no visible
 * key get v_out = 0 and lse = -inf.
 * workspace: at least mla_materialized_workspace_bytes(dims, T, n_kv, scratch_cap_mib)
 * bytes of device memory, 256-byte aligned, contents need not be initialised; it holds
 * the transposed wk_b, the rotated query rope and one head chunk's keys and values.
 * Supported: act == kv == MLA_BF16, Dn 128, Dr 64, Dv 128, R % 8 == 0, scale > 0.
 * Domain: q_nope and the decompressed k_nope and v are held in binary16 (IEEE half), so
 * every q_nope value and every k_nope[h][j], v[h][j] component must lie within +-65504;
 * the rope parts and all stored inputs and outputs stay bfloat16.  Outside that domain the
 * half conversion gives +-inf and the affected rows come out inf or NaN (or lose those
 * keys' contributions); the library does not scan the inputs to reject them.  The absorbed
 * chain (mla_absorb_q, mla_attn_prefill, mla_out_proj) has no such limit.
 * Errors: INVALID_ARG (nulls, T < 0, n_kv < 1), UNSUPPORTED (other dtypes or dims),
 * WORKSPACE (missing, too small or misaligned). */
int mla_prefill_materialized(const mla_dims *dims, mla_dtype act, mla_dtype kv,
                             const void *q_nope, const void *q_rope, const int32_t *pos,
                             int32_t T, const void *kv_cache, int32_t n_kv, const void *wk_b,
                             const void *wv_b, const void *wo, void *v_out, void *out, float *lse,
                             uint32_t scratch_cap_mib, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Workspace bytes of mla_prefill_materialized (0 for invalid or unsupported arguments).
 * Host-only. */
size_t mla_materialized_workspace_bytes(const mla_dims *dims, int32_t T, int32_t n_kv,
                                        uint32_t scratch_cap_mib);

/* Append new tokens to the latent cache (absorption page, section 4: the cache keeps
 * one row per token holding the compressed c_kv and the rotated shared key; section
 * 8.1: an 8-bit Q8_0 cache).  For token t:
 *   row = [ c_kv[t][0:R] | RoPE(k_rope[t], pos[t]) ]          (W = R + Dr values)
 * with the rotation of mla_absorb_q (adjacent pairs, angle pos * rope_base^(-2i/Dr)); the
 * key is rotated once, on entry (the "llama.cpp KV cache" page, section 2.3, re-rotates
 * cached keys on a shift, so the cache holds rotated keys),
 * written at cache row dst_row[t] (int64, device), or at row pos[t] when dst_row is
 * NULL, converted to the kv type: float32; bfloat16 rounded to nearest even; Q8_0 by
 * the rule of mla_quantize_q8_0 (bitwise the same bytes as quantizing the float32 row).
 * c_kv [T][R] and k_rope [T][Dr] (pre-RoPE) of dtype act, pos [T] int32 (device),
 * cache [n_rows][W] rows of kv dtype (Q8_0: W/32*34 bytes per row).  Tokens whose
 * destination row lies outside [0, n_rows) are skipped.  Two tokens with the same
 * destination race (either may win).  c_kv is taken as given: any normalisation
 * belongs to the projection that produced it.
 * Supported: act MLA_F32 or MLA_BF16 with kv == act, or kv MLA_Q8_0 (W % 32 == 0);
 * W <= 16384.  T == 0 is a no-op.
 * Errors: INVALID_ARG (nulls, T < 0, n_rows < 0, dtype mix, Q8_0 with W % 32 != 0),
 * UNSUPPORTED (W > 16384). */
int mla_cache_append(const mla_dims *dims, mla_dtype act, mla_dtype kv, const void *c_kv,
                     const void *k_rope, const int32_t *pos, const int64_t *dst_row, int32_t T,
                     void *cache, int64_t n_rows, void *stream);

/* Walsh-Hadamard-rotated latent cache (the "llama.cpp KV cache" page, section 3.1: keys
 * rotated by an orthonormal Hadamard matrix before quantisation spread the quantisation
 * noise over all dimensions; the query takes the same rotation, so scores are unchanged).
 * H is the page's normalised Sylvester matrix of order R (a power of two),
 * H[i][j] = (-1)^popcount(i & j) / sqrt(R): symmetric, H H = I.
 *
 * mla_cache_append_hadamard: mla_cache_append with the c_kv part of each new row replaced
 *   by H c_kv[t] before it is stored (RoPE part unchanged).  Same arguments, layouts and
 *   errors; R must be a power of two (else INVALID_ARG).
 * mla_hadamard_weights: the weights that make a rotated cache give the plain result,
 *   wk_b_rot[h] = H wk_b[h] ([R][Dn]) and wv_b_rot[h] = wv_b[h] H ([Dv][R]); computed once.
 *   Since c = H c', the score q_lat . c = (H q_lat) . c' and the output
 *   wv_b o_lat = (wv_b H) o_lat' (o_lat' attends on the rotated rows): mla_absorb_q with
 *   wk_b_rot, attention on the rotated cache and mla_out_proj with wv_b_rot compute the
 *   same layer as the plain chain.  act MLA_F32 or MLA_BF16 (outputs rounded to nearest
 *   even); outputs must not alias inputs.  Errors: INVALID_ARG (nulls, aliasing, R not a
 *   power of two), UNSUPPORTED (R > 16384). */
int mla_cache_append_hadamard(const mla_dims *dims, mla_dtype act, mla_dtype kv,
                              const void *c_kv, const void *k_rope, const int32_t *pos,
                              const int64_t *dst_row, int32_t T, void *cache, int64_t n_rows,
                              void *stream);
int mla_hadamard_weights(const mla_dims *dims, mla_dtype act, const void *wk_b, const void *wv_b,
                         void *wk_b_rot, void *wv_b_rot, void *stream);

/* Merged and split weight layouts (the page "ik_llama.cpp PR #394": section 2.1 names the
 * merged attn_kv_b tensor of ggml shape {R, H*(Dn+Dv)}, section 3.3 rebuilds it from the
 * split pair, with BF16 sources giving BF16 and other sources Q8_0).  Row-major:
 *   wkv_b[h][i][l] = wk_b[h][l][i]        for i <  Dn   (k_nope row i of head h)
 *   wkv_b[h][Dn+e][l] = wv_b[h][e][l]     for e <  Dv   (v row e of head h)
 * so that [k_nope | v] of head h = wkv_b[h] . c_kv.  wkv_b is [H][Dn+Dv][R] of type `out`
 * (act, an exact copy, or MLA_Q8_0: each R-wide row quantised as by mla_quantize_q8_0);
 * wk_b [H][R][Dn], wv_b [H][Dv][R] of type act (MLA_F32 or MLA_BF16).
 * mla_wkv_b_merge: split -> merged.  mla_wkv_b_split: merged (type `in`: act, or MLA_Q8_0
 * dequantised to d*q and rounded to act) -> split.
 * Errors: INVALID_ARG (nulls, dtype not act or Q8_0, Q8_0 with R % 32 != 0). */
int mla_wkv_b_merge(const mla_dims *dims, mla_dtype act, mla_dtype out, const void *wk_b,
                    const void *wv_b, void *wkv_b, void *stream);
int mla_wkv_b_split(const mla_dims *dims, mla_dtype in, mla_dtype act, const void *wkv_b,
                    void *wk_b, void *wv_b, void *stream);

/* Bytes of one Q8_0 row of `width` values (width/32*34), or -1 if width is not a
 * positive multiple of 32.  Host-only. */
int32_t mla_q8_0_row_bytes(int32_t width);

/* Static description of a status code.  Host-only. */
const char *mla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
