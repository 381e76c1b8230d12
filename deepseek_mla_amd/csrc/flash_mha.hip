// Materialised prefill (the pp_opt path of the page "ik_llama.cpp MLA matrix absorption",
// section 8.4): for long prompts over a long cache, each head's keys and values are
// decompressed from the latent cache once,
//   k_nope[h][j] = c_kv[j] . wk_b[h]      (Dn = 128 per key)
//   v[h][j]      = wv_b[h] . c_kv[j]      (Dv = 128 per key, stored transposed)
// and attention runs as ordinary causal multi-head attention with a 192-wide query
// [q_nope | RoPE(q_rope)] against [k_nope | k_rope] (k_rope read from the cache rows,
// shared by all heads) and a 128-wide value.  Per visible (query, key, head) that is
// 2 * (192 + 128) = 640 FLOP instead of the absorbed path's 2 * (576 + 512) = 2176.
// Heads run in chunks chosen by the -amb rule (section 8.3), which bounds the
// decompressed keys and values held at once.
//
// flash_mha_kernel<NW, NS>: a workgroup owns 32*NW query tokens of one head; wave w owns
// 32 of them.  Keys stream through LDS in tiles of 64 (LDS-direct copies, NS stages):
//   S^T[key][row] = K_tile (64 x 192) x Q^T          24 MFMA 32x32x16 per wave
//   O^T[dv][row] += V^T_tile (128 x 64) x P^T        16 MFMA 32x32x16 per wave
// The transposed products put one query row in each lane (lanes l and l^32 share it), so
// the softmax statistics are lane-local plus one exchange.  Inside each 16-key group of
// a tile, LDS row m holds key m with bits 2 and 3 swapped: the score slots a lane then
// holds are exactly the 8 consecutive keys the P^T operand of the value product needs,
// so the weights go from the score registers into the value MFMA without an exchange.
// Softmax: FlashAttention-2 recurrence in base 2 with a lazy reference: a row's weights
// are exp2(s - m) against a reference m that is raised (and the 128-wide accumulator and
// the denominator rescaled) only when a score exceeds it by more than 2^8, so weights
// stay below 256 (well inside binary16) and most tiles skip the rescale.
//
// Precision: the decompressed keys and values, the weights P and the query's nope part
// are held in binary16 (11 significant bits; the cache, the rope parts and all inputs
// stay bfloat16): with bfloat16 for these three intermediate roundings the result moves
// about 4x further from the exact one than with none at all, with binary16 it stays at
// the rounding of the stored output.  Values beyond binary16's range (|x| > 65504) in
// q_nope or in a decompressed key or value are outside this path's domain.
#include "latent_tile.h"  // static_for, lds_copy16

#include <algorithm>


namespace mla {

namespace mh {
constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int NK = 64;                         // keys per tile
constexpr int KN_BYTES = NK * DN * 2;          // 16384: k_nope rows, 256 B each
constexpr int KR_BYTES = NK * DR * 2;          // 8192: k_rope rows, 128 B each
constexpr int VT_BYTES = DV * NK * 2;          // 16384: V^T rows (one per dv), 128 B each
constexpr int STAGE = KN_BYTES + KR_BYTES + VT_BYTES;  // 40960
constexpr int COPIES = (KN_BYTES + KR_BYTES + VT_BYTES) / 1024;  // 40 copy instructions per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float TAU = 8.0f;                    // weights exp2(s - m) stay <= 2^TAU
}  // namespace mh

// LDS row of key k within a tile (bits 2 and 3 swapped; an involution).
__device__ __forceinline__ int mh_perm(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}
// Bank swizzles (LDS: 16 groups of 16 bytes).  k_nope rows are 256 B (16 groups): chunk c of
// row m sits at c ^ (m & 15), so 16 consecutive rows read at one chunk hit 16 groups.
// k_rope and V^T rows are 128 B (8 groups): odd rows take the upper half, and chunk c of
// row m sits at c ^ ((m >> 1) & 7).
__device__ __forceinline__ int kn_off(int m, int c) { return m * 256 + ((c ^ (m & 15)) << 4); }
__device__ __forceinline__ int h8_off(int m, int c) { return m * 128 + ((c ^ ((m >> 1) & 7)) << 4); }

// Issue the 40/NW copy instructions of wave w for the tile of keys key0 .. key0+63 into
// stage dst.  Keys past `last` re-read row `last` (k_nope, k_rope); V^T rows are padded
// with zeros up to a multiple of 64 keys, so whole tiles are always in bounds.
template <int NW>
__device__ __forceinline__ void mh_issue_tile(const uint8_t *kn, const uint8_t *cache,
                                              int64_t row_bytes, int rope_off, const uint8_t *vt,
                                              int64_t vt_pitch, int key0, int last,
                                              uint32_t dst, int w) {
    static_assert(NW == 4 || NW == 8, "copies split evenly over the waves");
    const int l = threadIdx.x & 63;
    // k_nope: instructions i = (16/NW) w + j cover LDS rows 4i .. 4i+3
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
        const int i = (16 / NW) * w + j;
        const int m = 4 * i + (l >> 4), s = l & 15;
        const int c = s ^ (m & 15);
        const int key = min(key0 + mh_perm(m), last);
        lds_copy16(kn + (int64_t)key0 * 256, (uint32_t)((key - key0) * 256 + c * 16),
                   dst + i * 1024);
    }
    // k_rope: instructions i = (8/NW) w + j cover LDS rows 8i .. 8i+7 (from the cache rows)
#pragma unroll
    for (int j = 0; j < 8 / NW; ++j) {
        const int i = (8 / NW) * w + j;
        const int m = 8 * i + (l >> 3), s = l & 7;
        const int c = s ^ ((m >> 1) & 7);
        const int key = min(key0 + mh_perm(m), last);
        lds_copy16(cache + (int64_t)key0 * row_bytes,
                   (uint32_t)((int64_t)(key - key0) * row_bytes + rope_off + c * 16),
                   dst + mh::KN_BYTES + i * 1024);
    }
    // V^T: instructions i = (16/NW) w + j cover dv rows 8i .. 8i+7 (keys key0 .. key0+63)
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
        const int i = (16 / NW) * w + j;
        const int dv = 8 * i + (l >> 3), s = l & 7;
        const int c = s ^ ((dv >> 1) & 7);
        lds_copy16(vt + (int64_t)key0 * 2, (uint32_t)(dv * vt_pitch + c * 16),
                   dst + mh::KN_BYTES + mh::KR_BYTES + i * 1024);
    }
}

// One (head, token block) per workgroup.  kn: [hc][n_kv][128], vt: [hc][128][vt_len] (binary16)
// (vt_len a multiple of 64, zero past n_kv), q_nope [T][H][128], q_rope_rot [T][H][64]
// (already rotated), cache rows of row_bytes with k_rope at rope_off.  Writes
// v_out[t][h*128 ..] (bf16, normalised) and lse[t][h] (natural log) for h = h0 + chunk head.
template <int NW, int NS>
__global__ __launch_bounds__(64 * NW) void flash_mha_kernel(
    const bf16 *__restrict__ q_nope, const bf16 *__restrict__ q_rope_rot,
    const int32_t *__restrict__ pos, int T, int H, int h0, int hc,
    const uint8_t *__restrict__ kn_all, const uint8_t *__restrict__ cache, int64_t row_bytes,
    int rope_off, const uint8_t *__restrict__ vt_all, int vt_len, int n_kv, float sc,
    bf16 *__restrict__ v_out, float *__restrict__ lse) {
    constexpr int ROWS = 32 * NW;                 // query tokens per workgroup
    constexpr int PER_WAVE = mh::COPIES / NW;     // copy instructions per wave per tile
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    uint8_t MLA_LDS *lds = (uint8_t MLA_LDS *)smem_raw;

    // block -> (head, token block): the blocks of one head share an XCD (block ids go
    // round-robin over the 8 XCDs) when hc is a multiple of 8; heaviest blocks first.
    const int nqb = (T + ROWS - 1) / ROWS;
    const int L = blockIdx.x;
    int hh, qr;
    if (hc % 8 == 0) {
        hh = (L & 7) + 8 * (L / (8 * nqb));
        qr = (L >> 3) % nqb;
    } else {
        hh = L / nqb;
        qr = L % nqb;
    }
    const int qb = nqb - 1 - qr;
    const int h = h0 + hh;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, hi = l >> 5, r = l & 31;
    const int t = qb * ROWS + 32 * w + r;
    const bool valid = t < T;
    const int tq = valid ? t : T - 1;
    int lim = valid ? min(pos[tq], n_kv - 1) : -1;

    // queries: fragment kk holds dims kk*16 + hi*8 .. +7 of the row (nope part in binary16)
    f16x8 qn16[8];
    bf16x8 qr16[4];
    {
        const bf16 *qn = q_nope + ((int64_t)tq * H + h) * mh::DN + hi * 8;
        const bf16 *qp = q_rope_rot + ((int64_t)tq * H + h) * mh::DR + hi * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 x = *(const bf16x8 *)(qn + kk * 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) qn16[kk][e] = (f16)(float)x[e];
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qr16[kk] = *(const bf16x8 *)(qp + kk * 16);
    }
    // key bounds: wave max / min of the row limits; every wave also reduces the limits of
    // all the workgroup's rows (lane l reads rows l, l + 64, ...) for the key range
    int wmax = lim, wmin = valid ? lim : INT32_MAX, gmax = -1;
#pragma unroll
    for (int i = 0; i < NW / 2; ++i) {
        const int tt = qb * ROWS + 64 * i + l;
        if (tt < T) gmax = max(gmax, min(pos[tt], n_kv - 1));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) gmax = max(gmax, __shfl_xor(gmax, o));
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        wmax = max(wmax, __shfl_xor(wmax, o));
        wmin = min(wmin, __shfl_xor(wmin, o));
    }
    wmax = __builtin_amdgcn_readfirstlane(wmax);
    wmin = __builtin_amdgcn_readfirstlane(wmin);
    const int kend = __builtin_amdgcn_readfirstlane(gmax) + 1;  // keys [0, kend) are seen
    const int ntiles = (kend + mh::NK - 1) / mh::NK;

    const uint8_t *kn = kn_all + (int64_t)hh * n_kv * mh::DN * 2;
    const uint8_t *vt = vt_all + (int64_t)hh * mh::DV * vt_len * 2;
    const int64_t vt_pitch = (int64_t)vt_len * 2;
    const int last = n_kv - 1;
    const uint32_t lbase = lds_u32(lds);

    // per-lane LDS offsets within a stage: K fragment of step kk (block j adds 8192 for
    // k_nope, 4096 for k_rope), V^T fragment of key step ks (dv block nb adds 4096)
    uint32_t koff[12], voff[4];
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
        koff[kk] = kk < 8 ? (uint32_t)kn_off(r, 2 * kk + hi)
                          : (uint32_t)(mh::KN_BYTES + h8_off(r, 2 * (kk - 8) + hi));
        asm volatile("" : "+v"(koff[kk]));
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        voff[ks] = (uint32_t)(mh::KN_BYTES + mh::KR_BYTES + h8_off(r, 2 * ks + hi));
        asm volatile("" : "+v"(voff[ks]));
    }

    f32x16 o[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[nb][e] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    // the query and bound loads must be complete before the copies (their completion is
    // tracked by counting outstanding vector-memory operations)
    // Copies run NS-1 tiles ahead.
    static_assert(NS == 2 || NS == 3, "one or two tiles in flight");
    constexpr int DEPTH = NS - 1;
    MLA_WAIT_VMCNT(0);
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
        if (s < ntiles)
            mh_issue_tile<NW>(kn, cache, row_bytes, rope_off, vt, vt_pitch, s * mh::NK, last,
                              lbase + s * mh::STAGE, w);

    for (int ti = 0; ti < ntiles; ++ti) {
        // tile ti landed (with more than one tile in flight, tile ti+1 may not have)
        if (DEPTH > 1 && ti + 1 < ntiles) {
            MLA_WAIT_VMCNT(PER_WAVE);
        } else {
            MLA_WAIT_VMCNT(0);
        }
        __syncthreads();  // tile ti landed everywhere; stages of tiles before ti-1 are free
        if (ti + DEPTH < ntiles)
            mh_issue_tile<NW>(kn, cache, row_bytes, rope_off, vt, vt_pitch, (ti + DEPTH) * mh::NK,
                              last, lbase + ((ti + DEPTH) % NS) * mh::STAGE, w);
        const int key0 = ti * mh::NK;
        if (key0 > wmax) continue;  // no row of this wave sees these keys
        const uint8_t MLA_LDS *st = lds + (ti % NS) * mh::STAGE;

        // scores: two 32-key blocks, slot e of block j is key
        // key0 + 32j + 16(e>>3) + 8hi + (e&7).  Step i = (kk, j) = (i/2, i%2); the K
        // fragment of step i + SA is read right after the MFMA of step i.
        // Masked keys ride on the chain's starting value: -inf stays -inf through every
        // finite product (edge tiles only); other tiles start from the constant 0.
        constexpr int SA = 6;
        auto kfrag = [&](int i) -> u32x4 {
            const int kk = i >> 1, j = i & 1;
            return *(const u32x4 MLA_LDS *)(st + koff[kk] + (kk < 8 ? 8192 : 4096) * j);
        };
        u32x4 ring[SA];
#pragma unroll
        for (int i = 0; i < SA; ++i) ring[i] = kfrag(i);
        f32x16 s[2];
        const bool edge = key0 + mh::NK - 1 > wmin;
        static_for<24>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int kk = i >> 1, j = i & 1;
            const u32x4 a = ring[i % SA];
            if constexpr (kk == 0) {
                if (edge) {
                    f32x16 b;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        b[e] = (key0 + 32 * j + 16 * (e >> 3) + 8 * hi + (e & 7) <= lim) ? 0.0f
                                                                                         : -INFINITY;
                    s[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                                  qn16[0], b, 0, 0, 0);
                } else {
                    const f32x16 z = {};
                    s[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                                  qn16[0], z, 0, 0, 0);
                }
            } else if constexpr (kk < 8) {
                s[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                              qn16[kk], s[j], 0, 0, 0);
            } else {
                s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                               qr16[kk - 8], s[j], 0, 0, 0);
            }
            if constexpr (i + SA < 24) ring[i % SA] = kfrag(i + SA);
            __builtin_amdgcn_sched_barrier(0);
        });
        // online softmax (base 2): running max over the row (this lane's 32 slots and the
        // partner lane's), rescale when it grows
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[j][e]);
        {
            const float y = __shfl_xor(tmax, 32);
            tmax = hi ? fmaxf(y, tmax) : fmaxf(tmax, y);
        }
        tmax *= sc;
        if (__builtin_amdgcn_ballot_w64(tmax > m + mh::TAU)) {  // also a row's first keys
            const float mnew = tmax > m + mh::TAU ? tmax : m;
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 when m = -inf
            lsum *= alpha;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[nb][e] *= alpha;
            m = mnew;
        }
        const float nmu = (m == -INFINITY) ? 0.0f : -m;
        f16x8 p[4];  // p[ks]: keys key0 + 16ks + 8hi .. +7
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(s[j][e], sc, nmu));
                lsum += pe;
                p[2 * j + (e >> 3)][e & 7] = (f16)pe;
            }
        // O^T += V^T P^T: A = V^T rows dv = 32nb + r, keys 16ks + 8hi .. +7 (chunk 2ks+hi)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const f16x8 a = *(const f16x8 MLA_LDS *)(st + voff[ks] + 4096 * nb);
                o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, p[ks], o[nb], 0, 0, 0);
            }
    }

    if (!valid) return;
    float ltot;
    {
        const float y = __shfl_xor(lsum, 32);
        ltot = hi ? y + lsum : lsum + y;
    }
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    bf16 *orow = v_out + ((int64_t)t * H + h) * mh::DV;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            bf16x4 v4;
#pragma unroll
            for (int b = 0; b < 4; ++b) v4[b] = f2bf(o[nb][4 * a + b] * inv);
            *(bf16x4 *)(orow + 32 * nb + 8 * a + 4 * hi) = v4;
        }
    if (lse && hi == 0)
        lse[(int64_t)t * H + h] = ltot > 0.0f ? (m + __log2f(ltot)) * mh::LN2 : -INFINITY;
}

// wk_b [H][R][Dn] -> wk_bT [H][Dn][R] (32 x 32 tiles through LDS).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16 *__restrict__ src,
                                                             bf16 *__restrict__ dst, int rows,
                                                             int cols) {
    __shared__ bf16 tile[32][33];
    const int64_t b = blockIdx.z;
    const bf16 *s = src + b * rows * cols;
    bf16 *d = dst + b * rows * cols;
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int i = ty; i < 32; i += 8)
        if (r0 + i < rows && c0 + tx < cols) tile[i][tx] = s[(int64_t)(r0 + i) * cols + c0 + tx];
    __syncthreads();
    for (int i = ty; i < 32; i += 8)
        if (c0 + i < cols && r0 + tx < rows) d[(int64_t)(c0 + i) * rows + r0 + tx] = tile[tx][i];
}

// Zero columns [from, pitch) of `rows` rows of a binary16 matrix with row pitch `pitch`.
__global__ __launch_bounds__(256) void zero_cols_kernel(f16 *__restrict__ x, int64_t rows,
                                                        int pitch, int from) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int w = pitch - from;
    if (i >= rows * w) return;
    x[(i / w) * pitch + from + (int)(i % w)] = (f16)0.0f;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// One chunk's attention launch.  8 waves (256 tokens) and 3 stages per workgroup, one
// workgroup per CU; when that grid would leave CUs idle (few tokens per head chunk), 4 waves
// (128 tokens) and 2 stages, two workgroups per CU.
template <int NW, int NS>
static hipError_t launch_mha(const bf16 *q_nope, const bf16 *qr, const int32_t *pos, int T, int H,
                             int h0, int nh, const f16 *kn, const bf16 *cache, int W, int R,
                             const f16 *vt, int vt_len, int n_kv, float sc, bf16 *v_out,
                             float *lse, hipStream_t st) {
    const size_t shm = (size_t)NS * mh::STAGE;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_lds_limit((const void *)flash_mha_kernel<NW, NS>, (int)shm, lds_set);
    if (e != hipSuccess) return e;
    const int nqb = (T + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((flash_mha_kernel<NW, NS>), dim3(nqb * nh), dim3(64 * NW), shm, st, q_nope,
                       qr, pos, T, H, h0, nh, (const uint8_t *)kn, (const uint8_t *)cache,
                       (int64_t)W * 2, R * 2, (const uint8_t *)vt, vt_len, n_kv, sc, v_out, lse);
    return hipGetLastError();
}

static int vt_len_of(int n_kv) { return (n_kv + mh::NK - 1) / mh::NK * mh::NK; }

size_t materialized_workspace_bytes(int T, int H, int R, int n_kv, int hc) {
    return al256((size_t)H * mh::DN * R * 2) + al256((size_t)T * H * mh::DR * 2) +
           al256((size_t)hc * n_kv * mh::DN * 2) + al256((size_t)hc * mh::DV * vt_len_of(n_kv) * 2);
}

hipError_t launch_prefill_materialized(const bf16 *q_nope, const bf16 *q_rope, const int32_t *pos,
                                       int T, int H, int R, const bf16 *cache, int n_kv,
                                       const bf16 *wk_b, const bf16 *wv_b, int hc, float scale,
                                       float rope_base, bf16 *v_out, float *lse, void *ws,
                                       hipStream_t st) {
    using namespace mh;
    uint8_t *p = (uint8_t *)ws;
    bf16 *wk_bT = (bf16 *)p;
    p += al256((size_t)H * DN * R * 2);
    bf16 *qr = (bf16 *)p;
    p += al256((size_t)T * H * DR * 2);
    f16 *kn = (f16 *)p;
    p += al256((size_t)hc * n_kv * DN * 2);
    f16 *vt = (f16 *)p;
    const int vt_len = vt_len_of(n_kv);
    const int W = R + DR;
    hipError_t e;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((DN + 31) / 32, (R + 31) / 32, H), dim3(256), 0,
                       st, wk_b, wk_bT, R, DN);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_rope_q<bf16>(q_rope, pos, qr, T, H, 0, DR, rope_base, st)) != hipSuccess)
        return e;
    int n_cu = 256;
    {
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    }
    for (int h0 = 0; h0 < H; h0 += hc) {
        const int nh = std::min(hc, H - h0);
        // k_nope[i][j][d] = sum_l c_kv[j][l] wk_b[h0+i][l][d]
        e = launch_gemm_nt_bf16_f16out(cache, wk_bT + (int64_t)h0 * DN * R, kn, n_kv, DN, R, W,
                                       R, DN, nh, 0, (int64_t)DN * R, (int64_t)n_kv * DN, st);
        if (e != hipSuccess) return e;
        // v^T[i][d][j] = sum_l wv_b[h0+i][d][l] c_kv[j][l]
        e = launch_gemm_nt_bf16_f16out(wv_b + (int64_t)h0 * DV * R, cache, vt, DV, n_kv, R, R, W,
                                       vt_len, nh, (int64_t)DV * R, 0, (int64_t)DV * vt_len, st);
        if (e != hipSuccess) return e;
        if (vt_len > n_kv) {
            const int64_t n = (int64_t)nh * DV * (vt_len - n_kv);
            hipLaunchKernelGGL(zero_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               st, vt, (int64_t)nh * DV, vt_len, n_kv);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const bool wide = (int64_t)((T + 255) / 256) * nh >= n_cu;
        e = wide ? launch_mha<8, 3>(q_nope, qr, pos, T, H, h0, nh, kn, cache, W, R, vt, vt_len, n_kv,
                                    scale * LOG2E, v_out, lse, st)
                 : launch_mha<4, 2>(q_nope, qr, pos, T, H, h0, nh, kn, cache, W, R, vt, vt_len, n_kv,
                                    scale * LOG2E, v_out, lse, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mla
