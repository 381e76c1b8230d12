// Generic (non-MFMA) kernels: the float32 path for any layer dims, the RoPE part of
// query absorption, the split-KV log-sum-exp combine, and Q8_0 (de)quantisation.
#include "common.h"

#include <math.h>

namespace mla {

// ---------------------------------------------------------------- NT GEMM (f32)
// C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]; 64x64 tiles, 256 threads, 4x4 outputs
// per thread, K staged through LDS in steps of 16.
constexpr int SG_TM = 64, SG_TN = 64, SG_TK = 16;

__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(const float *__restrict__ A,
                                                          const float *__restrict__ B,
                                                          float *__restrict__ C, int M, int N,
                                                          int K, int64_t lda, int64_t ldb,
                                                          int64_t ldc, int64_t sA, int64_t sB,
                                                          int64_t sC) {
    __shared__ float As[SG_TK][SG_TM + 4];
    __shared__ float Bs[SG_TK][SG_TN + 4];
    const int bz = blockIdx.z;
    A += bz * sA;
    B += bz * sB;
    C += bz * sC;
    const int m0 = blockIdx.y * SG_TM, n0 = blockIdx.x * SG_TN;
    const int tid = threadIdx.x;
    const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += SG_TK) {
        for (int e = tid; e < SG_TM * SG_TK; e += 256) {
            int r = e / SG_TK, kk = e % SG_TK;
            int gm = m0 + r, gk = k0 + kk;
            As[kk][r] = (gm < M && gk < K) ? A[gm * lda + gk] : 0.0f;
            int gn = n0 + r;
            Bs[kk][r] = (gn < N && gk < K) ? B[gn * ldb + gk] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < SG_TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[kk][tm + i];
                b[i] = Bs[kk][tn + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int gm = m0 + tm + i, gn = n0 + tn + j;
            if (gm < M && gn < N) C[gm * ldc + gn] = acc[i][j];
        }
}

hipError_t launch_gemm_nt_f32(const float *A, const float *B, float *C, int M, int N, int K,
                              int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                              int64_t sB, int64_t sC, hipStream_t st) {
    if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
    dim3 grid((N + SG_TN - 1) / SG_TN, (M + SG_TM - 1) / SG_TM, batch);
    hipLaunchKernelGGL(gemm_nt_f32_kernel, grid, dim3(256), 0, st, A, B, C, M, N, K, lda, ldb,
                       ldc, sA, sB, sC);
    return hipGetLastError();
}

// ------------------------------------------------------------------ query RoPE
// q_cat[t][h][R + 2i .. R + 2i+1] = rotation of (q_rope[t][h][2i], q_rope[t][h][2i+1]) by
// the angle pos[t] * base^(-2i/Dr).  The angle is formed and reduced to [-pi, pi] in
// double (at pos ~ 1e5 a float angle would be off by ~1e-2 rad); its sine and cosine are
// then taken in float (|error| ~1e-7) and the rotation is done in float.  A block takes
// RQ_TOK tokens: its threads first tabulate (cos, sin) per (token, pair) in LDS, then
// rotate 4 pairs (8 values) per step, all heads.  The first RQ_PRE groups of each thread
// are loaded before the angles are formed, so that their latency overlaps that work.
constexpr int RQ_TOK = 8, RQ_T = 256, RQ_PRE = 4;

// cos and sin of the RoPE angle pos * base^(-2i/Dr): the angle formed and reduced to
// [-pi, pi] in double, the sine and cosine taken in float.
__device__ __forceinline__ void rope_cs(int32_t pos, int i, int Dr, double log2_base, float *c,
                                        float *s) {
    constexpr double TWO_PI = 6.283185307179586;
    const double ang = (double)pos * exp2(-2.0 * (double)i / (double)Dr * log2_base);
    const double r = fma(-rint(ang / TWO_PI), TWO_PI, ang);
    sincosf((float)r, s, c);
}

template <typename T> struct Vec8;
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
        for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    }
    static __device__ __forceinline__ void store(float *p, const float *v) {
        const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        *(f32x4 *)p = a;
        *(f32x4 *)(p + 4) = b;
    }
};
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const bf16 *p, float *v) {
        const bf16x8 a = *(const bf16x8 *)p;
        for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
    }
    static __device__ __forceinline__ void store(bf16 *p, const float *v) {
        bf16x8 a;
        for (int i = 0; i < 8; ++i) a[i] = (bf16)v[i];
        *(bf16x8 *)p = a;
    }
};

template <typename T>
__global__ __launch_bounds__(RQ_T) void rope_q_kernel(const T *__restrict__ q_rope,
                                                      const int32_t *__restrict__ pos,
                                                      T *__restrict__ q_cat, int T_, int H, int R,
                                                      int Dr, float base, bool vec) {
    extern __shared__ float cs[];  // [RQ_TOK][Dr/2][2]
    const int t0 = blockIdx.x * RQ_TOK;
    const int half = Dr / 2;
    const int ntok = min(RQ_TOK, T_ - t0);
    const int quads = half / 4;  // groups of 4 pairs
    const int nvec = vec ? ntok * H * quads : 0;
    auto vrow = [&](int e, int &tt, int &g) {  // row (t, h) of group e; tt, g: token, group
        tt = e / (H * quads);
        const int rem = e % (H * quads);
        g = rem % quads;
        return (int64_t)(t0 + tt) * H + rem / quads;
    };
    float pre[RQ_PRE][8];
#pragma unroll
    for (int k = 0; k < RQ_PRE; ++k) {
        const int e = threadIdx.x + RQ_T * k;
        if (e < nvec) {
            int tt, g;
            const int64_t row = vrow(e, tt, g);
            Vec8<T>::load(q_rope + row * Dr + 8 * g, pre[k]);
        }
    }
    const double lb = log2((double)base);
    for (int j = threadIdx.x; j < ntok * half; j += blockDim.x) {
        const int tt = j / half;
        float sn, cn;
        rope_cs(pos[t0 + tt], j % half, Dr, lb, &cn, &sn);
        cs[2 * j] = cn;
        cs[2 * j + 1] = sn;
    }
    __syncthreads();
    const int W = R + Dr;
    auto rotate = [&](int e, const float *v) {
        int tt, g;
        const int64_t row = vrow(e, tt, g);
        float o[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float c = cs[2 * (tt * half + 4 * g + k)], sn = cs[2 * (tt * half + 4 * g + k) + 1];
            o[2 * k] = fmaf(v[2 * k], c, -v[2 * k + 1] * sn);
            o[2 * k + 1] = fmaf(v[2 * k], sn, v[2 * k + 1] * c);
        }
        Vec8<T>::store(q_cat + row * W + R + 8 * g, o);
    };
    if (vec) {  // Dr and R multiples of 8, 16-byte aligned bases: aligned 8-value accesses
#pragma unroll
        for (int k = 0; k < RQ_PRE; ++k)
            if (threadIdx.x + RQ_T * k < nvec) rotate(threadIdx.x + RQ_T * k, pre[k]);
        for (int e = threadIdx.x + RQ_T * RQ_PRE; e < nvec; e += RQ_T) {
            int tt, g;
            const int64_t row = vrow(e, tt, g);
            float v[8];
            Vec8<T>::load(q_rope + row * Dr + 8 * g, v);
            rotate(e, v);
        }
    } else {
        for (int e = threadIdx.x; e < ntok * H * half; e += blockDim.x) {
            const int tt = e / (H * half), rem = e % (H * half);
            const int h = rem / half, i = rem % half;
            const int64_t row = (int64_t)(t0 + tt) * H + h;
            const float a = ld_f(q_rope + row * Dr + 2 * i), b = ld_f(q_rope + row * Dr + 2 * i + 1);
            const float c = cs[2 * (tt * half + i)], sn = cs[2 * (tt * half + i) + 1];
            st_f(q_cat + row * W + R + 2 * i, fmaf(a, c, -b * sn));
            st_f(q_cat + row * W + R + 2 * i + 1, fmaf(a, sn, b * c));
        }
    }
}

template <typename T>
hipError_t launch_rope_q(const T *q_rope, const int32_t *pos, T *q_cat, int T_, int H, int R,
                         int Dr, float base, hipStream_t st) {
    if (T_ <= 0) return hipSuccess;
    const size_t shm = sizeof(float) * (size_t)RQ_TOK * Dr;
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    const bool vec = Dr % 8 == 0 && R % 8 == 0 && al16(q_rope) && al16(q_cat);
    hipLaunchKernelGGL(rope_q_kernel<T>, dim3((T_ + RQ_TOK - 1) / RQ_TOK), dim3(RQ_T), shm, st,
                       q_rope, pos, q_cat, T_, H, R, Dr, base, vec);
    return hipGetLastError();
}
template hipError_t launch_rope_q<float>(const float *, const int32_t *, float *, int, int, int,
                                         int, float, hipStream_t);
template hipError_t launch_rope_q<bf16>(const bf16 *, const int32_t *, bf16 *, int, int, int,
                                        int, float, hipStream_t);

// ------------------------------------------------------- SIMT flash attention (f32)
// One wave per (query row, head).  Keys are taken 64 at a time: lane i scores key
// j0+i (dot product over the W-wide row against the query held in LDS), the wave
// updates a running max / sum (online softmax), and each lane accumulates output
// columns lane, lane+64, ... of the latent weighted sum.
constexpr int SF_WAVES = 4;
constexpr int SF_MAXR = 16;  // R <= 64 * SF_MAXR

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Attends query row q (W floats in LDS) over cache rows [k0, k1) (row stride W).
// Returns normalised output in o[] (lane's columns) and lse (natural log; -inf if
// the range is empty).
__device__ void simt_attend(const float *qs, const float *__restrict__ rows, int k0, int k1,
                            int R, int W, float scale, float *o, float &lse_out) {
    const int lane = threadIdx.x & 63;
    const int nc = (R + 63) / 64;
    float m = -INFINITY, l = 0.0f;
    for (int c = 0; c < SF_MAXR; ++c) o[c] = 0.0f;
    for (int j0 = k0; j0 < k1; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        if (j < k1) {
            const float *row = rows + (int64_t)j * W;
            float acc = 0.0f;
            for (int e = 0; e < W; ++e) acc = fmaf(qs[e], row[e], acc);
            s = acc * scale;
        }
        const float cmax = wave_max(s);
        const float mnew = fmaxf(m, cmax);
        const float alpha = (m == -INFINITY) ? 0.0f : expf(m - mnew);
        const float p = (j < k1) ? expf(s - mnew) : 0.0f;
        l = l * alpha + wave_sum(p);
        for (int c = 0; c < SF_MAXR; ++c) o[c] *= alpha;
        m = mnew;
        const int cnt = min(64, k1 - j0);
        for (int i = 0; i < cnt; ++i) {
            const float pi = __shfl(p, i);
            const float *row = rows + (int64_t)(j0 + i) * W;
            for (int c = 0; c < nc; ++c) {
                int col = c * 64 + lane;
                if (col < R) o[c] = fmaf(pi, row[col], o[c]);
            }
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    for (int c = 0; c < SF_MAXR; ++c) o[c] *= inv;
    lse_out = l > 0.0f ? m + logf(l) : -INFINITY;
}

__global__ __launch_bounds__(256) void flash_simt_prefill_kernel(
    const float *__restrict__ q_cat, const int32_t *__restrict__ pos, int T, int H, int R, int W,
    const float *__restrict__ cache, int n_kv, int h0, int hc, float scale,
    float *__restrict__ o_lat, float *__restrict__ lse) {
    extern __shared__ float qsh[];  // [SF_WAVES][W]
    const int w = threadIdx.x / 64, lane = threadIdx.x & 63;
    const int row = blockIdx.x * SF_WAVES + w;  // flattened (t, head-in-chunk)
    if (row >= T * hc) return;
    const int t = row / hc, h = h0 + row % hc;
    float *qs = qsh + w * W;
    const float *q = q_cat + ((int64_t)t * H + h) * W;
    for (int e = lane; e < W; e += 64) qs[e] = q[e];
    __builtin_amdgcn_wave_barrier();
    int k1 = min(pos[t] + 1, n_kv);
    if (k1 < 0) k1 = 0;
    float o[SF_MAXR], ls;
    simt_attend(qs, cache, 0, k1, R, W, scale, o, ls);
    float *dst = o_lat + ((int64_t)t * H + h) * R;
    for (int c = 0; c < SF_MAXR; ++c) {
        int col = c * 64 + lane;
        if (col < R) dst[col] = o[c];
    }
    if (lse && lane == 0) lse[(int64_t)t * H + h] = ls;
}

hipError_t launch_flash_simt_prefill(const mla_dims &d, const float *q_cat, const int32_t *pos,
                                     int T, const float *cache, int n_kv, int h0, int hc,
                                     float *o_lat, float *lse, hipStream_t st) {
    const int W = d.kv_lora_rank + d.qk_rope;
    const int rows = T * hc;
    if (rows <= 0) return hipSuccess;
    dim3 grid((rows + SF_WAVES - 1) / SF_WAVES);
    hipLaunchKernelGGL(flash_simt_prefill_kernel, grid, dim3(64 * SF_WAVES),
                       sizeof(float) * SF_WAVES * W, st, q_cat, pos, T, d.n_head,
                       d.kv_lora_rank, W, cache, n_kv, h0, hc, d.scale, o_lat, lse);
    return hipGetLastError();
}

// Decode partials: block (row group, split, sequence).  part_o [B][S][H][R] (normalised
// within the split), part_lse [B][S][H].
__global__ __launch_bounds__(256) void flash_simt_decode_kernel(
    const float *__restrict__ q_cat, int H, int R, int W, const float *__restrict__ cache,
    int64_t seq_stride, const int32_t *__restrict__ n_kv, int n_kv_max, int n_splits,
    int split_len, float scale, float *__restrict__ part_o, float *__restrict__ part_lse) {
    extern __shared__ float qsh[];
    const int w = threadIdx.x / 64, lane = threadIdx.x & 63;
    const int h = blockIdx.x * SF_WAVES + w;
    const int s = blockIdx.y, b = blockIdx.z;
    if (h >= H) return;
    float *qs = qsh + w * W;
    const float *q = q_cat + ((int64_t)b * H + h) * W;
    for (int e = lane; e < W; e += 64) qs[e] = q[e];
    __builtin_amdgcn_wave_barrier();
    const int nk = min(n_kv[b], n_kv_max);  // rows past n_kv_max are never read
    const int k0 = s * split_len, k1 = min(k0 + split_len, nk);
    float o[SF_MAXR], ls;
    simt_attend(qs, cache + b * seq_stride, k0, max(k0, k1), R, W, scale, o, ls);
    const int64_t pi = ((int64_t)b * n_splits + s) * H + h;
    float *dst = part_o + pi * R;
    for (int c = 0; c < SF_MAXR; ++c) {
        int col = c * 64 + lane;
        if (col < R) dst[col] = o[c];
    }
    if (lane == 0) part_lse[pi] = ls;
}

hipError_t launch_flash_simt_decode(const mla_dims &d, const float *q_cat, const float *cache,
                                    int64_t seq_stride_elems, const int32_t *n_kv, int n_kv_max,
                                    int B,
                                    int n_splits, int split_len, float *part_o, float *part_lse,
                                    hipStream_t st) {
    const int W = d.kv_lora_rank + d.qk_rope;
    dim3 grid((d.n_head + SF_WAVES - 1) / SF_WAVES, n_splits, B);
    hipLaunchKernelGGL(flash_simt_decode_kernel, grid, dim3(64 * SF_WAVES),
                       sizeof(float) * SF_WAVES * W, st, q_cat, d.n_head, d.kv_lora_rank, W,
                       cache, seq_stride_elems, n_kv, n_kv_max, n_splits, split_len, d.scale, part_o,
                       part_lse);
    return hipGetLastError();
}

// ------------------------------------------------------------ split-KV combine
// lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s (partials o_s float32 on the
// float32 path, bfloat16 on the bf16 / Q8_0 path).  Splits with lse_s = -inf contribute
// nothing.  Block (b*H + h, slice of CB_COLS columns) of CB_T threads: thread
// (phase, group) takes 8 adjacent columns of splits phase + CB_PH * i.  It loads CB_U of
// its splits at once (lse and partial rows, all in flight together) and folds them into
// a running (max, sum, 8 weighted columns) with one rescale per batch; the CB_PH phases
// are then merged through LDS in a fixed order.
constexpr int CB_T = 256, CB_COLS = 128, CB_GROUPS = CB_COLS / 8, CB_PH = CB_T / CB_GROUPS;
constexpr int CB_U = 8;

template <typename PT, typename OT>
__global__ __launch_bounds__(CB_T) void combine_kernel(const PT *__restrict__ part_o,
                                                       const float *__restrict__ part_lse, int H,
                                                       int R, int S, OT *__restrict__ o_lat,
                                                       float *__restrict__ lse) {
    __shared__ float m_sh[CB_PH], l_sh[CB_PH];
    __shared__ float acc_sh[CB_PH][CB_COLS];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int grp = tid % CB_GROUPS, ph = tid / CB_GROUPS;
    const int c0 = blockIdx.y * CB_COLS + grp * 8;
    const float *pl = part_lse + (int64_t)b * S * H + h;
    const PT *po = part_o + ((int64_t)b * S * H + h) * R + c0;
    const int64_t stride = (int64_t)H * R;
    float m = -INFINITY, lsum = 0.0f;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s0 = ph; s0 < S; s0 += CB_PH * CB_U) {
        float x[CB_U], v[CB_U][8];
#pragma unroll
        for (int i = 0; i < CB_U; ++i) {
            const int s = s0 + i * CB_PH;
            x[i] = s < S ? pl[(int64_t)s * H] : -INFINITY;
            if (s < S && c0 < R) {
                if (R % 8 == 0) {  // rows of 8-column groups: aligned vector loads, no overrun
                    Vec8<PT>::load(po + (int64_t)s * stride, v[i]);
                } else {
                    for (int e = 0; e < 8; ++e)
                        v[i][e] = (c0 + e < R) ? ld_f(po + (int64_t)s * stride + e) : 0.0f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
            }
        }
        float mc = m;
#pragma unroll
        for (int i = 0; i < CB_U; ++i) mc = fmaxf(mc, x[i]);
        if (mc == -INFINITY) continue;  // no visible split yet
        const float r = __expf(m - mc);  // 0 while m = -inf (nothing accumulated)
        lsum *= r;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= r;
#pragma unroll
        for (int i = 0; i < CB_U; ++i) {
            if (x[i] == -INFINITY) continue;  // an empty split's row is never weighted
            const float wgt = __expf(x[i] - mc);
            lsum += wgt;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(wgt, v[i][e], acc[e]);
        }
        m = mc;
    }
    if (grp == 0) {  // every group of a phase holds the same max and sum
        m_sh[ph] = m;
        l_sh[ph] = lsum;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc_sh[ph][grp * 8 + e] = acc[e];
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < CB_PH; ++p) mx = fmaxf(mx, m_sh[p]);
    float f[CB_PH], sum = 0.0f;
#pragma unroll
    for (int p = 0; p < CB_PH; ++p) {
        f[p] = (mx == -INFINITY || m_sh[p] == -INFINITY) ? 0.0f : __expf(m_sh[p] - mx);
        sum += f[p] * l_sh[p];
    }
    if (tid < CB_COLS) {
        const int c = blockIdx.y * CB_COLS + tid;
        float tot = 0.0f;
#pragma unroll
        for (int p = 0; p < CB_PH; ++p) tot = fmaf(f[p], acc_sh[p][tid], tot);
        if (c < R) st_f(o_lat + ((int64_t)b * H + h) * R + c, sum > 0.0f ? tot / sum : 0.0f);
    }
    if (lse && blockIdx.y == 0 && tid == 0)
        lse[(int64_t)b * H + h] = sum > 0.0f ? mx + logf(sum) : -INFINITY;
}

template <typename PT, typename OT>
hipError_t launch_combine(const PT *part_o, const float *part_lse, int B, int H, int R,
                          int n_splits, OT *o_lat, float *lse, hipStream_t st) {
    dim3 grid(B * H, (R + CB_COLS - 1) / CB_COLS);
    hipLaunchKernelGGL((combine_kernel<PT, OT>), grid, dim3(CB_T), 0, st, part_o, part_lse, H,
                       R, n_splits, o_lat, lse);
    return hipGetLastError();
}
template hipError_t launch_combine<float, float>(const float *, const float *, int, int, int, int,
                                                 float *, float *, hipStream_t);
template hipError_t launch_combine<bf16, bf16>(const bf16 *, const float *, int, int, int, int,
                                               bf16 *, float *, hipStream_t);

// ------------------------------------------------------------------------ Q8_0
// One thread per 32-value block.  Block layout: binary16 scale (little endian) then
// 32 int8 codes; blocks are 34 bytes, so scales sit at 2-byte alignment.
// One 32-value block v -> 34 bytes at out (2-byte aligned).
__device__ __forceinline__ void q8_0_block(const float *v, uint8_t *out) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d = amax / 127.0f;
    const _Float16 hd = (_Float16)d;
    *(uint16_t *)out = __builtin_bit_cast(uint16_t, hd);
    for (int i = 0; i < 32; i += 2) {
        int q0 = 0, q1 = 0;
        if (d != 0.0f) {
            q0 = (int)fminf(fmaxf(roundf(v[i] / d), -127.0f), 127.0f);
            q1 = (int)fminf(fmaxf(roundf(v[i + 1] / d), -127.0f), 127.0f);
        }
        *(uint16_t *)(out + 2 + i) = (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
    }
}

__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float *__restrict__ x,
                                                            uint8_t *__restrict__ rows,
                                                            int64_t n_blocks, int nb_row,
                                                            int width) {
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= n_blocks) return;
    const int64_t r = blk / nb_row;
    const int b = (int)(blk % nb_row);
    q8_0_block(x + r * width + (int64_t)b * 32, rows + r * (int64_t)nb_row * 34 + (int64_t)b * 34);
}

__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t *__restrict__ rows,
                                                           float *__restrict__ out,
                                                           int64_t n_blocks, int nb_row,
                                                           int width) {
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= n_blocks) return;
    const int64_t r = blk / nb_row;
    const int b = (int)(blk % nb_row);
    const uint8_t *in = rows + r * (int64_t)nb_row * 34 + (int64_t)b * 34;
    const float d = (float)__builtin_bit_cast(_Float16, *(const uint16_t *)in);
    float *o = out + r * width + (int64_t)b * 32;
    for (int i = 0; i < 32; i += 2) {
        uint16_t pr = *(const uint16_t *)(in + 2 + i);
        o[i] = d * (float)(int8_t)(pr & 0xFF);
        o[i + 1] = d * (float)(int8_t)(pr >> 8);
    }
}

hipError_t launch_quantize_q8_0(const float *x, uint8_t *rows, int64_t n_rows, int width,
                                hipStream_t st) {
    const int nb = width / 32;
    const int64_t n = n_rows * nb;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       x, rows, n, nb, width);
    return hipGetLastError();
}

hipError_t launch_dequant_q8_0(const uint8_t *rows, float *out, int64_t n_rows, int width,
                               hipStream_t st) {
    const int nb = width / 32;
    const int64_t n = n_rows * nb;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       rows, out, n, nb, width);
    return hipGetLastError();
}

// ------------------------------------------------------------ merged wkv_b layout
// wkv_b[h] ([Dn + Dv][R]) stacks the transposed wk_b[h] ([R][Dn]) over wv_b[h] ([Dv][R]):
// row i < Dn is k_nope dim i, row Dn + e is v dim e (the merged attn_kv_b tensor of the page
// "ik_llama.cpp PR #394", section 2.1, reconstructed as in its section 3.3).

// element (h, i, l) of the merged tensor, read from the split pair
template <typename T>
__device__ __forceinline__ float wkv_elem(const T *wk_b, const T *wv_b, int h, int i, int l, int R,
                                          int Dn, int Dv) {
    return i < Dn ? ld_f(wk_b + ((int64_t)h * R + l) * Dn + i)
                  : ld_f(wv_b + ((int64_t)h * Dv + (i - Dn)) * R + l);
}

// merged = act type: one thread per element (writes coalesced along l)
template <typename T>
__global__ __launch_bounds__(256) void wkv_merge_kernel(const T *__restrict__ wk_b,
                                                        const T *__restrict__ wv_b,
                                                        T *__restrict__ wkv_b, int H, int R, int Dn,
                                                        int Dv) {
    const int64_t n = (int64_t)H * (Dn + Dv) * R;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int l = (int)(x % R);
    const int64_t hi = x / R;
    const int i = (int)(hi % (Dn + Dv)), h = (int)(hi / (Dn + Dv));
    st_f(wkv_b + x, wkv_elem(wk_b, wv_b, h, i, l, R, Dn, Dv));
}

// merged = Q8_0 rows of R values: one thread per 32-block (the block quantiser above)
template <typename T>
__global__ __launch_bounds__(256) void wkv_merge_q8_kernel(const T *__restrict__ wk_b,
                                                           const T *__restrict__ wv_b,
                                                           uint8_t *__restrict__ wkv_b, int H, int R,
                                                           int Dn, int Dv) {
    const int nb = R / 32;
    const int64_t n = (int64_t)H * (Dn + Dv) * nb;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int b = (int)(x % nb);
    const int64_t hi = x / nb;
    const int i = (int)(hi % (Dn + Dv)), h = (int)(hi / (Dn + Dv));
    float v[32];
    for (int j = 0; j < 32; ++j) v[j] = wkv_elem(wk_b, wv_b, h, i, 32 * b + j, R, Dn, Dv);
    q8_0_block(v, wkv_b + hi * (int64_t)nb * 34 + (int64_t)b * 34);
}

// split pair from the merged tensor (act type, or Q8_0 dequantised: d * q, exact in float)
template <typename T, bool Q8>
__global__ __launch_bounds__(256) void wkv_split_kernel(const void *__restrict__ wkv_b,
                                                        T *__restrict__ wk_b, T *__restrict__ wv_b,
                                                        int H, int R, int Dn, int Dv) {
    const int64_t n = (int64_t)H * (Dn + Dv) * R;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int l = (int)(x % R);
    const int64_t hi = x / R;
    const int i = (int)(hi % (Dn + Dv)), h = (int)(hi / (Dn + Dv));
    float val;
    if constexpr (Q8) {
        const uint8_t *blk = (const uint8_t *)wkv_b + hi * (int64_t)(R / 32) * 34 + (l / 32) * 34;
        const float d = (float)__builtin_bit_cast(_Float16, *(const uint16_t *)blk);
        val = d * (float)(int8_t)blk[2 + (l % 32)];
    } else {
        val = ld_f((const T *)wkv_b + x);
    }
    if (i < Dn)
        st_f(wk_b + ((int64_t)h * R + l) * Dn + i, val);
    else
        st_f(wv_b + ((int64_t)h * Dv + (i - Dn)) * R + l, val);
}

template <typename T>
hipError_t launch_wkv_merge(const T *wk_b, const T *wv_b, void *wkv_b, bool q8, int H, int R,
                            int Dn, int Dv, hipStream_t st) {
    const int64_t n = (int64_t)H * (Dn + Dv) * (q8 ? R / 32 : R);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (q8)
        hipLaunchKernelGGL(wkv_merge_q8_kernel<T>, grid, dim3(256), 0, st, wk_b, wv_b,
                           (uint8_t *)wkv_b, H, R, Dn, Dv);
    else
        hipLaunchKernelGGL(wkv_merge_kernel<T>, grid, dim3(256), 0, st, wk_b, wv_b, (T *)wkv_b, H,
                           R, Dn, Dv);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_wkv_split(const void *wkv_b, bool q8, T *wk_b, T *wv_b, int H, int R, int Dn,
                            int Dv, hipStream_t st) {
    const int64_t n = (int64_t)H * (Dn + Dv) * R;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (q8)
        hipLaunchKernelGGL((wkv_split_kernel<T, true>), grid, dim3(256), 0, st, wkv_b, wk_b, wv_b,
                           H, R, Dn, Dv);
    else
        hipLaunchKernelGGL((wkv_split_kernel<T, false>), grid, dim3(256), 0, st, wkv_b, wk_b, wv_b,
                           H, R, Dn, Dv);
    return hipGetLastError();
}
template hipError_t launch_wkv_merge<float>(const float *, const float *, void *, bool, int, int,
                                            int, int, hipStream_t);
template hipError_t launch_wkv_merge<bf16>(const bf16 *, const bf16 *, void *, bool, int, int, int,
                                           int, hipStream_t);
template hipError_t launch_wkv_split<float>(const void *, bool, float *, float *, int, int, int,
                                            int, hipStream_t);
template hipError_t launch_wkv_split<bf16>(const void *, bool, bf16 *, bf16 *, int, int, int, int,
                                           hipStream_t);

// ------------------------------------------------------------ Walsh-Hadamard rotation
// H (n = 2^k) is the normalised Sylvester matrix of the page "llama.cpp KV cache", section
// 3.1: H[i][j] = (-1)^popcount(i & j) / sqrt(n), symmetric and orthonormal (H H = I).
// y = H x by the fast transform: k butterfly stages (a, b) -> (a + b, a - b) over
// element pairs 2^s apart, then the 1/sqrt(n) scale; float32 throughout.  x is in LDS and
// every thread of the block takes part (the stages are separated by barriers).
__device__ __forceinline__ void fwht_lds(float *x, int n) {
    for (int h = 1; h < n; h <<= 1) {
        __syncthreads();
        for (int q = threadIdx.x; q < n / 2; q += blockDim.x) {
            const int i = (q / h) * 2 * h + (q % h);
            const float a = x[i], b = x[i + h];
            x[i] = a + b;
            x[i + h] = a - b;
        }
    }
    __syncthreads();
    const float sc = rsqrtf((float)n);
    for (int i = threadIdx.x; i < n; i += blockDim.x) x[i] *= sc;
    __syncthreads();
}

// out vector v = H . (in vector v), vector v's element i at
// (v / inner) * outer + (v % inner) + i * step (the same offsets in `in` and `out`).
template <typename T>
__global__ __launch_bounds__(256) void hadamard_vectors_kernel(const T *__restrict__ in,
                                                               T *__restrict__ out, int n,
                                                               int64_t inner, int64_t outer,
                                                               int64_t step) {
    extern __shared__ float hv[];
    const int64_t v = blockIdx.x;
    const int64_t base = (v / inner) * outer + (v % inner);
    for (int i = threadIdx.x; i < n; i += blockDim.x) hv[i] = ld_f(in + base + i * step);
    fwht_lds(hv, n);
    for (int i = threadIdx.x; i < n; i += blockDim.x) st_f(out + base + i * step, hv[i]);
}

template <typename T>
hipError_t launch_hadamard_weights(const T *wk_b, const T *wv_b, T *wk_b_rot, T *wv_b_rot, int H,
                                   int R, int Dn, int Dv, hipStream_t st) {
    const size_t shm = sizeof(float) * (size_t)R;
    // wk_b[h] is [R][Dn]: column d of head h (stride Dn) -> H . column
    hipLaunchKernelGGL(hadamard_vectors_kernel<T>, dim3((unsigned)H * Dn), dim3(256), shm, st, wk_b,
                       wk_b_rot, R, (int64_t)Dn, (int64_t)R * Dn, (int64_t)Dn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // wv_b[h] is [Dv][R]: each row (contiguous) -> row . H = (H . row^T)^T (H symmetric)
    hipLaunchKernelGGL(hadamard_vectors_kernel<T>, dim3((unsigned)H * Dv), dim3(256), shm, st, wv_b,
                       wv_b_rot, R, (int64_t)1, (int64_t)R, (int64_t)1);
    return hipGetLastError();
}
template hipError_t launch_hadamard_weights<float>(const float *, const float *, float *, float *,
                                                   int, int, int, int, hipStream_t);
template hipError_t launch_hadamard_weights<bf16>(const bf16 *, const bf16 *, bf16 *, bf16 *, int,
                                                  int, int, int, hipStream_t);

// ------------------------------------------------------------ latent cache append
// Row pos[t] of the cache <- [c_kv[t] (R) | RoPE(k_rope[t], pos[t]) (Dr)], stored as
// float32, bfloat16 (rounded to nearest even) or Q8_0 (the block quantiser above).  The
// rotation is the query's (rope_cs, adjacent pairs).  The destination row is row[t], or
// pos[t] when row is null; tokens whose destination lies outside [0, n_rows) are skipped.
// HAD: the c_kv part is rotated by H (fwht_lds) before it is stored.
// One wave per token; the row is assembled in LDS as float32, then stored.
template <typename TI, int KV, bool HAD>
__global__ __launch_bounds__(64) void cache_append_kernel(const TI *__restrict__ c_kv,
                                                          const TI *__restrict__ k_rope,
                                                          const int32_t *__restrict__ pos,
                                                          const int64_t *__restrict__ dst_row,
                                                          int R, int Dr, float base, void *cache,
                                                          int64_t n_rows) {
    extern __shared__ float row[];  // [R + Dr]
    const int t = blockIdx.x, l = threadIdx.x;
    const int32_t p = pos[t];
    const int64_t r = dst_row ? dst_row[t] : (int64_t)p;
    if (r < 0 || r >= n_rows) return;  // uniform
    const int W = R + Dr;
    for (int j = l; j < R; j += 64) row[j] = ld_f(c_kv + (int64_t)t * R + j);
    const double lb = log2((double)base);
    for (int i = l; i < Dr / 2; i += 64) {
        float c, s;
        rope_cs(p, i, Dr, lb, &c, &s);
        const float a = ld_f(k_rope + (int64_t)t * Dr + 2 * i), b = ld_f(k_rope + (int64_t)t * Dr + 2 * i + 1);
        row[R + 2 * i] = fmaf(a, c, -b * s);
        row[R + 2 * i + 1] = fmaf(a, s, b * c);
    }
    if constexpr (HAD) fwht_lds(row, R);  // ends on a barrier
    __syncthreads();
    if constexpr (KV == MLA_F32) {
        float *dst = (float *)cache + r * W;
        for (int j = l; j < W; j += 64) dst[j] = row[j];
    } else if constexpr (KV == MLA_BF16) {
        bf16 *dst = (bf16 *)cache + r * W;
        for (int j = l; j < W; j += 64) dst[j] = (bf16)row[j];
    } else {
        uint8_t *dst = (uint8_t *)cache + r * (W / 32 * 34);
        for (int b = l; b < W / 32; b += 64) q8_0_block(row + 32 * b, dst + 34 * b);
    }
}

template <typename TI, bool HAD>
static void launch_append_kv(const TI *c_kv, const TI *k_rope, const int32_t *pos,
                             const int64_t *dst_row, int T, int R, int Dr, float base, int kv,
                             void *cache, int64_t n_rows, hipStream_t st) {
    const size_t shm = sizeof(float) * (size_t)(R + Dr);
    if (kv == MLA_F32)
        hipLaunchKernelGGL((cache_append_kernel<TI, MLA_F32, HAD>), dim3(T), dim3(64), shm, st,
                           c_kv, k_rope, pos, dst_row, R, Dr, base, cache, n_rows);
    else if (kv == MLA_BF16)
        hipLaunchKernelGGL((cache_append_kernel<TI, MLA_BF16, HAD>), dim3(T), dim3(64), shm, st,
                           c_kv, k_rope, pos, dst_row, R, Dr, base, cache, n_rows);
    else
        hipLaunchKernelGGL((cache_append_kernel<TI, MLA_Q8_0, HAD>), dim3(T), dim3(64), shm, st,
                           c_kv, k_rope, pos, dst_row, R, Dr, base, cache, n_rows);
}

template <typename TI>
hipError_t launch_cache_append(const TI *c_kv, const TI *k_rope, const int32_t *pos,
                               const int64_t *dst_row, int T, int R, int Dr, float base, int kv,
                               bool hadamard, void *cache, int64_t n_rows, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (hadamard)
        launch_append_kv<TI, true>(c_kv, k_rope, pos, dst_row, T, R, Dr, base, kv, cache, n_rows, st);
    else
        launch_append_kv<TI, false>(c_kv, k_rope, pos, dst_row, T, R, Dr, base, kv, cache, n_rows,
                                    st);
    return hipGetLastError();
}
template hipError_t launch_cache_append<float>(const float *, const float *, const int32_t *,
                                               const int64_t *, int, int, int, float, int, bool,
                                               void *, int64_t, hipStream_t);
template hipError_t launch_cache_append<bf16>(const bf16 *, const bf16 *, const int32_t *,
                                              const int64_t *, int, int, int, float, int, bool,
                                              void *, int64_t, hipStream_t);

}  // namespace mla
