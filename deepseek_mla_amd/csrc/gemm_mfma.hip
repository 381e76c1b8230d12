// bf16 "NT" GEMM on gfx950 matrix cores:
//   C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]       (bf16 in, fp32 accumulate, bf16 out)
// Both operands are K-contiguous, which is the layout of all three projections of the
// absorbed path: q_lat = q_nope . wk_b[h]^T, v = o_lat . wv_b[h]^T, out = v . wo^T.
//
// Tile 128x128x32 per workgroup of 4 waves (2x2), each wave 64x64 as 2x2 blocks of
// v_mfma_f32_32x32x16_bf16.  Operand tiles are staged through LDS (double buffered)
// with a 16-byte-chunk XOR swizzle so that fragment reads are bank-conflict free.
#include "common.h"

namespace mla {

constexpr int GB_M = 128, GB_N = 128, GB_K = 32;
constexpr int GB_ROWB = GB_K * 2;                 // 64 bytes per tile row
constexpr int GB_TILE_BYTES = GB_M * GB_ROWB;     // 8 KiB per operand tile

__device__ __forceinline__ int gswz(int row, int c) { return c ^ ((row >> 2) & 3); }

__global__ __launch_bounds__(256) void gemm_nt_bf16_kernel(const bf16 *__restrict__ A,
                                                           const bf16 *__restrict__ B,
                                                           bf16 *__restrict__ C, int M, int N,
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
                if (gm < M && gn < N) C[gm * ldc + gn] = f2bf(acc[i][j][e]);
            }
        }
}

hipError_t launch_gemm_nt_bf16(const bf16 *A, const bf16 *B, bf16 *C, int M, int N, int K,
                               int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                               int64_t sB, int64_t sC, hipStream_t st) {
    if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
    dim3 grid((N + GB_N - 1) / GB_N, (M + GB_M - 1) / GB_M, batch);
    hipLaunchKernelGGL(gemm_nt_bf16_kernel, grid, dim3(256), 0, st, A, B, C, M, N, K, lda, ldb,
                       ldc, sA, sB, sC);
    return hipGetLastError();
}

}  // namespace mla
