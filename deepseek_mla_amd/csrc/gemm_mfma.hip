// bf16 "NT" GEMM on gfx950 matrix cores:
//   C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]       (bf16 in, fp32 accumulate, bf16 out;
//                                                     binary16 out on request)
// Both operands are K-contiguous, which is the layout of all three projections of the
// absorbed path: q_lat = q_nope . wk_b[h]^T, v = o_lat . wv_b[h]^T, out = v . wo^T.
//
// Tile 128x128x32 per workgroup of 4 waves (2x2), each wave 64x64 as 2x2 blocks of
// v_mfma_f32_32x32x16_bf16.  Operand tiles are staged through LDS (double buffered)
// with a 16-byte-chunk XOR swizzle so that fragment reads are bank-conflict free.
#include "common.h"
#include "lds_dma.h"

#include <type_traits>

namespace mla {

constexpr int GB_M = 128, GB_N = 128, GB_K = 32;
constexpr int GB_ROWB = GB_K * 2;                 // 64 bytes per tile row
constexpr int GB_TILE_BYTES = GB_M * GB_ROWB;     // 8 KiB per operand tile

__device__ __forceinline__ int gswz(int row, int c) { return c ^ ((row >> 2) & 3); }

// fp32 -> output element (both conversions round to nearest even)
template <typename TO> __device__ __forceinline__ TO cvt_out(float x) { return (TO)x; }

template <typename TO>
__global__ __launch_bounds__(256) void gemm_nt_bf16_kernel(const bf16 *__restrict__ A,
                                                           const bf16 *__restrict__ B,
                                                           TO *__restrict__ C, int M, int N,
                                                           int K, int64_t lda, int64_t ldb,
                                                           int64_t ldc, int64_t sA, int64_t sB,
                                                           int64_t sC) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][GB_TILE_BYTES];  // [stage][A/B]
    const int bz = blockIdx.z;
    A += bz * sA;
    B += bz * sB;
    C += bz * sC;
    const int m0 = blockIdx.y * GB_M, n0 = blockIdx.x * GB_N;
    const int tid = threadIdx.x, w = tid / 64, l = tid & 63;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;

    // staging: each thread moves 2 chunks of 16 B for A and 2 for B per K step
    u32x4 ra[2], rb[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int ch = tid + i * 256;  // 0..511: row = ch / 4, c = ch % 4
            int r = ch >> 2, c = ch & 3;
            int gk = k0 + c * 8;
            int gm = m0 + r, gn = n0 + r;
            u32x4 z = {0, 0, 0, 0};
            ra[i] = (gm < M && gk < K) ? *(const u32x4 *)(A + gm * lda + gk) : z;
            rb[i] = (gn < N && gk < K) ? *(const u32x4 *)(B + gn * ldb + gk) : z;
        }
    };
    auto sstore = [&](int stg) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int ch = tid + i * 256;
            int r = ch >> 2, c = ch & 3;
            int off = r * GB_ROWB + gswz(r, c) * 16;
            *(u32x4 *)(&lds[stg][0][off]) = ra[i];
            *(u32x4 *)(&lds[stg][1][off]) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = (K + GB_K - 1) / GB_K;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int stg = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * GB_K);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[2], bfr[2];
            const int c = ks * 2 + (l >> 5);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int ra_ = wm + i * 32 + (l & 31);
                af[i] = *(const bf16x8 *)(&lds[stg][0][ra_ * GB_ROWB + gswz(ra_, c) * 16]);
                int rb_ = wn + i * 32 + (l & 31);
                bfr[i] = *(const bf16x8 *)(&lds[stg][1][rb_ * GB_ROWB + gswz(rb_, c) * 16]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) {
            sstore(stg ^ 1);
        }
        __syncthreads();
    }
    // D[m][n]: lane l holds column n = l%32, rows (e/4)*8 + (l/32)*4 + e%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int gn = n0 + wn + j * 32 + (l & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int gm = m0 + wm + i * 32 + (e >> 2) * 8 + (l >> 5) * 4 + (e & 3);
                if (gm < M && gn < N) C[gm * ldc + gn] = cvt_out<TO>(acc[i][j][e]);
            }
        }
}

// ---------------------------------------------------------------------------------
// Larger-tile form for K a multiple of 64: workgroup tile BM x 128 (BM = 256 or 128) x 64,
// 4 waves as 2 x 2, each wave (BM/2) x 64.  Operand tiles go straight from global memory
// to LDS (global_load_lds_dwordx4, one instruction per 8 rows of 128 B), NS stages deep
// (NS - 1 k-tiles in flight while one is consumed; 2 stages when K is only two k-tiles,
// so that two workgroups fit a CU).  In LDS, logical
// 16-byte chunk c of tile row r sits at chunk c ^ ((r >> 1) & 7) (the copies take their
// source chunk accordingly): the fragment reads of 8 consecutive rows then hit 8
// distinct bank groups.  The product is computed transposed, D^T[n][m] = B_tile A_tile^T,
// so that a lane ends up with 4 consecutive columns of one output row; the tile is staged
// in LDS as bf16 rows and written with 16-byte stores.
constexpr int GL_BN = 128, GL_BK = 64;
constexpr int GL_ROWB = GL_BK * 2;  // 128 B per tile row
constexpr int GL_OPITCH = GL_BN * 2 + 16;  // staged output row pitch: rows 4 banks apart
__host__ __device__ constexpr int gl_stage_bytes(int bm) { return (bm + GL_BN) * GL_ROWB; }
__device__ __forceinline__ int gl_swz(int r) { return (r >> 1) & 7; }

// Source offsets of this lane's copies, fixed for the whole K loop: wave w copies A rows
// [w*BM/4, (w+1)*BM/4) and B rows [32w, 32w + 32), 8 rows per instruction; rows past the
// matrix end re-read its last row (those results are not stored).
template <int BM>
struct GlPlan {
    uint32_t a[BM / 32], b[4];
    uint32_t wa, wb;  // LDS offsets of this wave's first A row and first B row in a stage
    __device__ __forceinline__ GlPlan(int M, int N, int64_t lda, int64_t ldb, int m0, int n0) {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < BM / 32; ++j) {
            const int r = w * (BM / 4) + 8 * j + (l >> 3);
            const int rr = min(m0 + r, M - 1) - m0;
            a[j] = (uint32_t)((int64_t)rr * lda * 2 + (((l & 7) ^ gl_swz(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = w * 32 + 8 * j + (l >> 3);
            const int rr = min(n0 + r, N - 1) - n0;
            b[j] = (uint32_t)((int64_t)rr * ldb * 2 + (((l & 7) ^ gl_swz(r)) << 4));
        }
        wa = (uint32_t)(w * (BM / 4) * GL_ROWB);
        wb = (uint32_t)(BM * GL_ROWB + w * 32 * GL_ROWB);
    }
    // copy instruction c (0 .. BM/32 + 3; A rows first, then B rows) of the k-tile whose
    // first elements are at asrc (A) and bsrc (B), into the stage at LDS address dst
    __device__ __forceinline__ void issue_one(const uint8_t *asrc, const uint8_t *bsrc,
                                              uint32_t dst, int c) const {
        if (c < BM / 32)
            lds_copy16(asrc, a[c], dst + wa + 8 * c * GL_ROWB);
        else
            lds_copy16(bsrc, b[c - BM / 32], dst + wb + 8 * (c - BM / 32) * GL_ROWB);
    }
    // copies of k-tile [k0, k0 + 64) into the stage at LDS address dst
    __device__ __forceinline__ void issue(const uint8_t *abase, const uint8_t *bbase, int k0,
                                          uint32_t dst) const {
#pragma unroll
        for (int c = 0; c < BM / 32 + 4; ++c) issue_one(abase + 2 * k0, bbase + 2 * k0, dst, c);
    }
};

// Query RoPE carried by the absorption GEMM (batch index = head h, C = q_cat of head h,
// row stride ldc): after its output tile, the workgroup of tile (n-tile x, rows from m0,
// head h) rotates the rope part of rows [m0 + x*rpb, m0 + (x+1)*rpb) (rpb = BM / gridDim.x,
// rounded up; every n-tile of a row range once), writing
// q_cat[t][h][R + 2i ..] from q_rope[t][h][2i ..] by the angle pos[t] * base^(-2i/Dr).  The
// angle is formed and reduced to [-pi, pi] in double (at pos ~ 1e5 a float angle would be
// off by ~1e-2 rad), its sine and cosine are taken in float.  q_rope == nullptr: none.
struct RopeTail {
    const bf16 *q_rope;
    const int32_t *pos;
    float base;
    int H, Dr, R;
};

__device__ __forceinline__ void rope_rows(const RopeTail &rp, bf16 *__restrict__ C, int64_t ldc,
                                          int h, int t0, int t1) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const int half = rp.Dr / 2;
    const double lb = log2((double)rp.base);
    constexpr double TWO_PI = 6.283185307179586;
    for (int j = threadIdx.x; j < (t1 - t0) * half; j += blockDim.x) {
        const int t = t0 + j / half, i = j % half;
        const double ang = (double)rp.pos[t] * exp2(-2.0 * (double)i / (double)rp.Dr * lb);
        const double r = fma(-rint(ang / TWO_PI), TWO_PI, ang);
        float sn, cn;
        sincosf((float)r, &sn, &cn);
        const bf16x2 x = *(const bf16x2 *)(rp.q_rope + ((int64_t)t * rp.H + h) * rp.Dr + 2 * i);
        const float a = (float)x[0], b = (float)x[1];
        const bf16x2 v = {(bf16)fmaf(a, cn, -b * sn), (bf16)fmaf(a, sn, b * cn)};
        *(bf16x2 *)(C + (int64_t)t * ldc + rp.R + 2 * i) = v;
    }
}

// Output tile of a workgroup of the two-stage form (K of at most two k-tiles: the absorption,
// whose M is the token count and whose batch is the heads).  Workgroups are dispatched
// round-robin over the 8 XCDs (workgroup i on XCD i % 8); when the grid divides evenly, each
// XCD takes a contiguous run of tiles, ordered in groups of GL_GM m-tiles (m fastest within a
// group), so that the workgroups an XCD runs at once share their A rows (and B rows) in its
// L2: V3 long-prefill absorption 0.567 -> 0.466 ms, Lite 23.6 -> 21.4 us.  The many-k-tile
// forms keep the plain order, which measured as fast or faster for their shapes.
constexpr int GL_GM = 4;
struct GlTile {
    int nx, my, bz;
};
__device__ __forceinline__ GlTile gl_tile_grouped() {
    const int nt = gridDim.x, mt = gridDim.y;
    const int total = nt * mt * (int)gridDim.z;
    int L = blockIdx.x + nt * (blockIdx.y + mt * blockIdx.z);
    if (total % 8 == 0) L = (L & 7) * (total >> 3) + (L >> 3);
    const int per_b = nt * mt;
    const int bz = L / per_b, r = L % per_b;
    const int g = r / (GL_GM * nt), rg = r % (GL_GM * nt);
    const int gm = min(GL_GM, mt - g * GL_GM);  // m-tiles in this group
    return {rg / gm, g * GL_GM + rg % gm, bz};
}

template <int BM, int NS, typename TO>
__global__ __launch_bounds__(256) void gemm_nt_bf16_lds_kernel(
    const bf16 *__restrict__ A, const bf16 *__restrict__ B, TO *__restrict__ C, int M, int N,
    int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sA, int64_t sB, int64_t sC,
    const RopeTail rope) {
    constexpr int MB = BM / 64;            // 32-row m blocks per wave
    constexpr int CP = BM / 32 + 4;        // copy instructions per wave per k-tile
    constexpr int SB = gl_stage_bytes(BM);
    static_assert(NS * SB <= 163840 && BM * GL_OPITCH <= NS * SB, "LDS budget");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    uint8_t MLA_LDS *lds = (uint8_t MLA_LDS *)lds_raw;
    const GlTile tile = NS == 2 ? gl_tile_grouped()
                                : GlTile{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    const int bz = tile.bz;
    A += bz * sA;
    B += bz * sB;
    C += bz * sC;
    const int m0 = tile.my * BM, n0 = tile.nx * GL_BN;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int wm = (w >> 1) * (BM / 2), wn = (w & 1) * 64;
    const uint32_t lbase = lds_u32(lds);
    const GlPlan<BM> plan(M, N, lda, ldb, m0, n0);
    const uint8_t *abase = (const uint8_t *)(A + (int64_t)m0 * lda);
    const uint8_t *bbase = (const uint8_t *)(B + (int64_t)n0 * ldb);

    f32x16 acc[2][MB];  // [n block][m block], D^T layout
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    // fragment rows of this lane: B-tile rows (n) as the MFMA A operand, A-tile rows (m)
    // as the MFMA B operand; logical chunk 2*ks + (l >> 5) for k step ks
    int boff[2], aoff[MB];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = wn + 32 * j + (l & 31);
        boff[j] = BM * GL_ROWB + r * GL_ROWB;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int r = wm + 32 * i + (l & 31);
        aoff[i] = r * GL_ROWB;
    }
    const int hi = l >> 5;
    auto chunk = [&](int rowoff, int ks) {  // byte offset of the lane's chunk in a row
        const int r = rowoff / GL_ROWB;
        return rowoff + ((((ks << 1) + hi) ^ gl_swz(r)) << 4);
    };

    const int nk = K / GL_BK;
    // With three or more stages, every stage receives a copy in the prologue and every
    // k-tile issues one, also past the last k-tile (the last one again, into the stage the
    // previous k-tile left, which nothing reads any more): the count of copy groups in flight
    // is then the same at every wait, and the copies need no branches.
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) plan.issue(abase, bbase, min(s, nk - 1) * GL_BK, lbase + s * SB);
    for (int kt = 0; kt < nk; ++kt) {
        // k-tile kt landed (the NS - 2 copy groups issued after its own may be in flight)
        MLA_WAIT_VMCNT((NS - 2) * CP);
        __syncthreads();  // k-tile kt landed everywhere; k-tile kt-1 no longer read
        // k-tile kt + NS - 1 goes into the stage k-tile kt-1 left.  With three or more stages,
        // one copy instruction after every other MFMA: issued together, the four waves' copies
        // queue in the CU's address unit and hold back the first MFMAs of the k-tile.  With
        // two (K of two k-tiles), all at once, and none past the last k-tile (the wait is for
        // every copy in flight there).
        constexpr bool SPREAD = NS > 2;
        const int nk0 = min(kt + NS - 1, nk - 1) * GL_BK;
        const uint8_t *asrc = abase + 2 * nk0, *bsrc = bbase + 2 * nk0;
        const uint32_t ndst = lbase + ((kt + NS - 1) % NS) * SB;
        const uint8_t MLA_LDS *st = lds + (kt % NS) * SB;
        if (!SPREAD && kt + 1 < nk) plan.issue(abase, bbase, nk0, ndst);
        // fragments of k step ks+1 are read while the MFMAs of step ks run
        bf16x8 bf[2][2], af[2][MB];
        auto fetch = [&](int ks, int b) {
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[b][j] = *(const bf16x8 MLA_LDS *)(st + chunk(boff[j], ks));
#pragma unroll
            for (int i = 0; i < MB; ++i) af[b][i] = *(const bf16x8 MLA_LDS *)(st + chunk(aoff[i], ks));
        };
        fetch(0, 0);
#pragma unroll
        for (int ks = 0; ks < GL_BK / 16; ++ks) {
            if (ks + 1 < GL_BK / 16) fetch(ks + 1, (ks + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);  // reads of step ks+1 go out before step ks's MFMAs
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[ks & 1][j], af[ks & 1][i],
                                                                        acc[j][i], 0, 0, 0);
                    const int q = (ks * 2 + j) * MB + i;  // MFMA index within the k-tile
                    if (SPREAD && q % 2 == 0 && q / 2 < CP) {
                        plan.issue_one(asrc, bsrc, ndst, q / 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    static_assert(2 * CP <= GL_BK / 16 * 2 * MB, "every copy instruction inside the k-tile's MFMAs");
    MLA_WAIT_VMCNT(0);  // the copies issued past the last k-tile land before the staging
    __syncthreads();    // stages free: staging of the output tile
    // lane: output row m = wm + 32i + (l & 31); columns n = wn + 32j + 8g + 4*hi + 0..3
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int m = wm + 32 * i + (l & 31);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = wn + 32 * j + 8 * g + 4 * hi;
                typedef TO tox4 __attribute__((ext_vector_type(4)));
                const tox4 v = {cvt_out<TO>(acc[j][i][4 * g]), cvt_out<TO>(acc[j][i][4 * g + 1]),
                                cvt_out<TO>(acc[j][i][4 * g + 2]), cvt_out<TO>(acc[j][i][4 * g + 3])};
                *(tox4 MLA_LDS *)(lds + m * GL_OPITCH + n * 2) = v;
            }
        }
    __syncthreads();
    // 16 chunks of 16 B per row; thread t takes chunks t, t + 256, ...
#pragma unroll
    for (int it = 0; it < BM / 16; ++it) {
        const int q = threadIdx.x + 256 * it;
        const int r = q >> 4, c = q & 15;
        if (m0 + r < M && n0 + 8 * c < N) {
            const uint8_t MLA_LDS *src = lds + r * GL_OPITCH + c * 16;
            const u32x2 a = *(const u32x2 MLA_LDS *)src;
            const u32x2 b = *(const u32x2 MLA_LDS *)(src + 8);
            const u32x4 v = {a[0], a[1], b[0], b[1]};
            *(u32x4 *)(C + (int64_t)(m0 + r) * ldc + n0 + 8 * c) = v;
        }
    }
    if constexpr (std::is_same<TO, bf16>::value) {
        if (rope.q_rope) {  // uniform
            const int rpb = (BM + (int)gridDim.x - 1) / (int)gridDim.x;
            const int t0 = m0 + tile.nx * rpb;
            rope_rows(rope, C, ldc, bz, min(t0, M), min(t0 + rpb, min(m0 + BM, M)));
        }
    }
}

template <int BM, int NS, typename TO>
static hipError_t launch_lds_gemm(const bf16 *A, const bf16 *B, TO *C, int M, int N, int K,
                                  int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                                  int64_t sB, int64_t sC, const RopeTail &rope, hipStream_t st) {
    static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
    const int shm = NS * gl_stage_bytes(BM);
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e =
        ensure_lds_limit((const void *)gemm_nt_bf16_lds_kernel<BM, NS, TO>, shm, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid((N + GL_BN - 1) / GL_BN, (M + BM - 1) / BM, batch);
    hipLaunchKernelGGL((gemm_nt_bf16_lds_kernel<BM, NS, TO>), grid, dim3(256), shm, st, A, B, C, M, N, K,
                       lda, ldb, ldc, sA, sB, sC, rope);
    return hipGetLastError();
}

// The LDS-staged kernel when the shape allows it (returns false otherwise, nothing launched).
template <typename TO>
static bool try_lds_gemm(const bf16 *A, const bf16 *B, TO *C, int M, int N, int K, int64_t lda,
                         int64_t ldb, int64_t ldc, int batch, int64_t sA, int64_t sB, int64_t sC,
                         const RopeTail &rope, hipStream_t st, hipError_t *e) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    if (!(K % GL_BK == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && ldc % 8 == 0 &&
          sA % 8 == 0 && sB % 8 == 0 && sC % 8 == 0 && al16(A) && al16(B) && al16(C)))
        return false;
    // K of two k-tiles: 128-row tiles, 2 stages (64 KB: two workgroups per CU).  Longer K:
    // 256-row tiles, 3 stages, when they still give two workgroups per CU, else 128-row
    // tiles, 4 stages.
    if (K <= 2 * GL_BK) {
        *e = launch_lds_gemm<128, 2, TO>(A, B, C, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, rope, st);
        return true;
    }
    const int64_t t256 = (int64_t)((N + GL_BN - 1) / GL_BN) * ((M + 255) / 256) * batch;
    if (t256 >= 512)
        *e = launch_lds_gemm<256, 3, TO>(A, B, C, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, rope, st);
    else
        *e = launch_lds_gemm<128, 4, TO>(A, B, C, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, rope, st);
    return true;
}

template <typename TO>
static hipError_t launch_gemm_any(const bf16 *A, const bf16 *B, TO *C, int M, int N, int K,
                                  int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                                  int64_t sB, int64_t sC, hipStream_t st) {
    if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
    hipError_t e = hipSuccess;
    const RopeTail none{nullptr, nullptr, 0.0f, 0, 0, 0};
    if (try_lds_gemm<TO>(A, B, C, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, none, st, &e))
        return e;
    dim3 grid((N + GB_N - 1) / GB_N, (M + GB_M - 1) / GB_M, batch);
    hipLaunchKernelGGL(gemm_nt_bf16_kernel<TO>, grid, dim3(256), 0, st, A, B, C, M, N, K, lda,
                       ldb, ldc, sA, sB, sC);
    return hipGetLastError();
}

hipError_t launch_gemm_nt_bf16(const bf16 *A, const bf16 *B, bf16 *C, int M, int N, int K,
                               int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                               int64_t sB, int64_t sC, hipStream_t st) {
    return launch_gemm_any<bf16>(A, B, C, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, st);
}

hipError_t launch_gemm_nt_bf16_f16out(const bf16 *A, const bf16 *B, f16 *C, int M, int N, int K,
                                      int64_t lda, int64_t ldb, int64_t ldc, int batch,
                                      int64_t sA, int64_t sB, int64_t sC, hipStream_t st) {
    return launch_gemm_any<f16>(A, B, C, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, st);
}

// Absorption: q_cat[t][h][:R] = wk_b[h] . q_nope[t][h] and the query RoPE into
// q_cat[t][h][R:].  For few tokens (decode) in one launch when the LDS-staged GEMM takes
// the shape (the rope rows ride on its workgroups: a second launch would cost more than
// the work); otherwise the GEMM and the RoPE kernel one after the other (riding on the
// GEMM, every head's workgroups would recompute the same angles).
hipError_t launch_absorb_bf16(const bf16 *q_nope, const bf16 *q_rope, const int32_t *pos,
                              const bf16 *wk_b, bf16 *q_cat, int T, int H, int R, int Dn, int Dr,
                              float base, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int W = R + Dr;
    const RopeTail rope{q_rope, pos, base, H, Dr, R};
    hipError_t e = hipSuccess;
    constexpr int FUSE_MAX_T = 64;
    if (T <= FUSE_MAX_T && Dr % 2 == 0 && R % 2 == 0 && ((uintptr_t)q_rope & 3) == 0 &&
        try_lds_gemm<bf16>(q_nope, wk_b, q_cat, T, R, Dn, (int64_t)H * Dn, Dn, (int64_t)H * W, H, Dn,
                     (int64_t)R * Dn, W, rope, st, &e))
        return e;
    e = launch_gemm_nt_bf16(q_nope, wk_b, q_cat, T, R, Dn, (int64_t)H * Dn, Dn, (int64_t)H * W, H,
                            Dn, (int64_t)R * Dn, W, st);
    if (e != hipSuccess) return e;
    return launch_rope_q<bf16>(q_rope, pos, q_cat, T, H, R, Dr, base, st);
}

}  // namespace mla
