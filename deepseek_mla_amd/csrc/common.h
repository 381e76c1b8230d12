// Internal declarations shared by the HIP sources of the MLA library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // v_cvt_pk_bf16_f32 (RNE)

template <typename T> __device__ __forceinline__ float ld_f(const T *p);
template <> __device__ __forceinline__ float ld_f<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld_f<bf16>(const bf16 *p) { return (float)*p; }
template <typename T> __device__ __forceinline__ void st_f(T *p, float v);
template <> __device__ __forceinline__ void st_f<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_f<bf16>(bf16 *p, float v) { *p = (bf16)v; }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]).
#define MLA_WAIT_VMCNT(n)                                                                      \
    __builtin_amdgcn_s_waitcnt((((n)&0xF) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (0xF << 8)))

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once per device
// (the attribute is held per device).  `done` is the kernel's own bit mask of devices
// already set; concurrent callers may both set it, which is harmless.
inline hipError_t ensure_lds_limit(const void *fn, int bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// ---- launchers (implemented in the .hip sources; all return hipError_t of launch)

// f32 / generic SIMT path
hipError_t launch_gemm_nt_f32(const float *A, const float *B, float *C, int M, int N, int K,
                              int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                              int64_t sB, int64_t sC, hipStream_t st);
template <typename T>
hipError_t launch_rope_q(const T *q_rope, const int32_t *pos, T *q_cat, int T_, int H, int R,
                         int Dr, float base, hipStream_t st);
hipError_t launch_flash_simt_prefill(const mla_dims &d, const float *q_cat, const int32_t *pos,
                                     int T, const float *cache, int n_kv, int h0, int hc,
                                     float *o_lat, float *lse, hipStream_t st);
hipError_t launch_flash_simt_decode(const mla_dims &d, const float *q_cat, const float *cache,
                                    int64_t seq_stride_elems, const int32_t *n_kv, int n_kv_max,
                                    int B,
                                    int n_splits, int split_len, float *part_o, float *part_lse,
                                    hipStream_t st);
template <typename PT, typename OT>
hipError_t launch_combine(const PT *part_o, const float *part_lse, int B, int H, int R,
                          int n_splits, OT *o_lat, float *lse, hipStream_t st);
hipError_t launch_quantize_q8_0(const float *x, uint8_t *rows, int64_t n_rows, int width,
                                hipStream_t st);
hipError_t launch_dequant_q8_0(const uint8_t *rows, float *out, int64_t n_rows, int width,
                               hipStream_t st);

// bf16 MFMA path
template <typename TI>
hipError_t launch_cache_append(const TI *c_kv, const TI *k_rope, const int32_t *pos,
                               const int64_t *dst_row, int T, int R, int Dr, float base, int kv,
                               bool hadamard, void *cache, int64_t n_rows, hipStream_t st);
template <typename T>
hipError_t launch_wkv_merge(const T *wk_b, const T *wv_b, void *wkv_b, bool q8, int H, int R,
                            int Dn, int Dv, hipStream_t st);
template <typename T>
hipError_t launch_wkv_split(const void *wkv_b, bool q8, T *wk_b, T *wv_b, int H, int R, int Dn,
                            int Dv, hipStream_t st);
template <typename T>
hipError_t launch_hadamard_weights(const T *wk_b, const T *wv_b, T *wk_b_rot, T *wv_b_rot, int H,
                                   int R, int Dn, int Dv, hipStream_t st);
hipError_t launch_absorb_bf16(const bf16 *q_nope, const bf16 *q_rope, const int32_t *pos,
                              const bf16 *wk_b, bf16 *q_cat, int T, int H, int R, int Dn, int Dr,
                              float base, hipStream_t st);
hipError_t launch_gemm_nt_bf16(const bf16 *A, const bf16 *B, bf16 *C, int M, int N, int K,
                               int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                               int64_t sB, int64_t sC, hipStream_t st);
// the same product with a binary16 result (rounded to nearest even)
hipError_t launch_gemm_nt_bf16_f16out(const bf16 *A, const bf16 *B, f16 *C, int M, int N, int K,
                                      int64_t lda, int64_t ldb, int64_t ldc, int batch,
                                      int64_t sA, int64_t sB, int64_t sC, hipStream_t st);
// few-row NT product (M <= GEMV_MAX_M rows of A), a stream over B; see gemv.hip
constexpr int GEMV_MAX_M = 8;
bool gemv_nt_bf16_ok(const bf16 *A, const bf16 *B, int M, int K, int64_t lda, int64_t ldb,
                     int64_t sA, int64_t sB);
hipError_t launch_gemv_nt_bf16(const bf16 *A, const bf16 *B, bf16 *C, int M, int N, int K,
                               int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                               int64_t sB, int64_t sC, hipStream_t st);
// prefill key parts: parts per row group (keys per part in *ks), and the workspace the
// merge of parts needs (0 when every group is one part)
// batched: one cache per token (sequence), of seq_n_kv[t] rows at cache + t * seq_stride
// bytes, every row visible (decode of many sequences); needs hc == 128 (a group per token)
int prefill_parts(int T, int H, int n_kv, int *ks, bool batched = false);
size_t prefill_workspace_bytes(int T, int H, int n_kv, int hc, bool batched = false);
hipError_t launch_flash_prefill_bf16(const bf16 *q_cat, const int32_t *pos, int T, int H,
                                     const bf16 *cache, int n_kv, int hc, float scale,
                                     bf16 *o_lat, float *lse, void *ws, hipStream_t st,
                                     int64_t seq_stride = 0, const int32_t *seq_n_kv = nullptr);
// materialised (pp_opt) prefill: Dn 128, Dr 64, Dv 128; workspace bytes and the launch
size_t materialized_workspace_bytes(int T, int H, int R, int n_kv, int hc);
hipError_t launch_prefill_materialized(const bf16 *q_nope, const bf16 *q_rope, const int32_t *pos,
                                       int T, int H, int R, const bf16 *cache, int n_kv,
                                       const bf16 *wk_b, const bf16 *wv_b, int hc, float scale,
                                       float rope_base, bf16 *v_out, float *lse, void *ws,
                                       hipStream_t st);
// heads per workgroup of the decode kernel (the split planner fills the CUs with it)
int decode_heads_per_block();
// decode over a Q8_0 cache with 128 heads per workgroup (every raw tile dequantised once
// for all of them); same partial layout as launch_flash_decode_bf16
int decode_wide_heads();
hipError_t launch_flash_decode_q8_wide(const bf16 *q_cat, const void *cache,
                                       int64_t seq_stride_bytes, const int32_t *n_kv,
                                       int n_kv_max, int B, int H, int n_splits, int split_len,
                                       float scale, bf16 *part_o, float *part_lse,
                                       hipStream_t st);
// the same over a bf16 cache; with vt (the transposed latent rows of each sequence, vt_ld
// keys apart, keys in score-slot order within each 32-key group) the O update reads V^T from
// there instead of transposing the cache rows
hipError_t launch_flash_decode_bf16_wide(const bf16 *q_cat, const void *cache,
                                         int64_t seq_stride_bytes, const void *vt,
                                         int64_t vt_seq_stride_bytes, int64_t vt_ld,
                                         const int32_t *n_kv, int n_kv_max, int B, int H,
                                         int n_splits, int split_len, float scale, bf16 *part_o,
                                         float *part_lse, hipStream_t st);
// transposed latent rows (the V^T cache) from a bf16 cache: rows [row0, row1) of each of B
// sequences; keys in score-slot order (bits 2 and 3 of the index swapped) within each
// aligned 32-key group
hipError_t launch_transpose_v(const bf16 *cache, int64_t seq_stride_bytes, int B, int row0,
                              int row1, bf16 *vt, int64_t vt_seq_stride_bytes, int64_t vt_ld,
                              hipStream_t st);
hipError_t launch_flash_decode_bf16(const bf16 *q_cat, const void *cache, int cache_q8,
                                    int64_t seq_stride_bytes, const int32_t *n_kv, int n_kv_max,
                                    int B, int H,
                                    int n_splits, int split_len, float scale, bf16 *part_o,
                                    float *part_lse, hipStream_t st);

}  // namespace mla
