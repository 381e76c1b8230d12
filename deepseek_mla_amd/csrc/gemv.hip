// bf16 "NT" product for few rows of A (M <= GEMV_MAX_M), the decode-time shape of the
// late projections (v = o_lat . wv_b[h]^T per head, out = v . wo^T):
//   C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]      (bf16 in, fp32 accumulate, bf16 out)
// With M this small the product is a stream over B (HBM bound): a 128x128 matrix-core
// tile would waste all but M of its rows.  Each wave streams RPW rows of B with 16-byte
// loads (a wave reads 1 KB of one row per instruction), keeps the M rows of A for the
// same k range in registers, accumulates with v_dot2c_f32_bf16 (bf16 pairs, fp32 sum)
// and reduces across the wave at the end.  One or two rows of A: one row of B per wave and
// 16 k steps unrolled (many loads in flight); more rows of A: 4 rows of B per wave, so
// that each A fragment serves 4 rows.
#include "common.h"

namespace mla {

constexpr int GV_WAVES = 4;
template <int M> constexpr int gv_rpw() { return M <= 2 ? 1 : 4; }         // rows of B per wave
template <int M> constexpr int gv_rows() { return gv_rpw<M>() * GV_WAVES; }  // per workgroup
constexpr int GV_KSTEP = 64 * 8;                      // k covered by one wave iteration

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(const bf16x8 &a, const bf16x8 &b, float c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x2v x = {a[2 * j], a[2 * j + 1]};
        const bf16x2v y = {b[2 * j], b[2 * j + 1]};
        c = __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false);
    }
    return c;
}

template <int M>
__global__ __launch_bounds__(64 * GV_WAVES) void gemv_nt_bf16_kernel(
    const bf16 *__restrict__ A, const bf16 *__restrict__ B, bf16 *__restrict__ C, int N, int K,
    int64_t lda, int64_t ldb, int64_t ldc, int64_t sA, int64_t sB, int64_t sC) {
    const int z = blockIdx.y;
    A += z * sA;
    B += z * sB;
    C += z * sC;
    constexpr int RPW = gv_rpw<M>();
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int n0 = blockIdx.x * gv_rows<M>() + w * RPW;
    // rows past N re-read row N-1 (their sums are not stored)
    const bf16 *brow[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) brow[r] = B + (int64_t)min(n0 + r, N - 1) * ldb;
    float acc[RPW][M];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    constexpr int UNR = M <= 2 ? 16 : 4;
#pragma unroll UNR
    for (int k = l * 8; k < K; k += GV_KSTEP) {
        bf16x8 a[M], b[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) b[r] = *(const bf16x8 *)(brow[r] + k);
#pragma unroll
        for (int m = 0; m < M; ++m) a[m] = *(const bf16x8 *)(A + m * lda + k);
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = dot8(a[m], b[r], acc[r][m]);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v = acc[r][m];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
            if (l == 0 && n0 + r < N) C[m * ldc + n0 + r] = f2bf(v);
        }
}

template <int M>
static void launch_m(int batch, hipStream_t st, const bf16 *A, const bf16 *B, bf16 *C, int N,
                     int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sA, int64_t sB,
                     int64_t sC) {
    const dim3 grid((N + gv_rows<M>() - 1) / gv_rows<M>(), batch);
    hipLaunchKernelGGL(gemv_nt_bf16_kernel<M>, grid, dim3(64 * GV_WAVES), 0, st, A, B, C, N, K, lda,
                       ldb, ldc, sA, sB, sC);
}

bool gemv_nt_bf16_ok(const bf16 *A, const bf16 *B, int M, int K, int64_t lda, int64_t ldb,
                     int64_t sA, int64_t sB) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    return M >= 1 && M <= GEMV_MAX_M && K % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 &&
           sA % 8 == 0 && sB % 8 == 0 && al16(A) && al16(B);
}

hipError_t launch_gemv_nt_bf16(const bf16 *A, const bf16 *B, bf16 *C, int M, int N, int K,
                               int64_t lda, int64_t ldb, int64_t ldc, int batch, int64_t sA,
                               int64_t sB, int64_t sC, hipStream_t st) {
    if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
    if (!gemv_nt_bf16_ok(A, B, M, K, lda, ldb, sA, sB)) return hipErrorInvalidValue;
    switch (M) {
        case 1: launch_m<1>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        case 2: launch_m<2>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        case 3: launch_m<3>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        case 4: launch_m<4>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        case 5: launch_m<5>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        case 6: launch_m<6>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        case 7: launch_m<7>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
        default: launch_m<8>(batch, st, A, B, C, N, K, lda, ldb, ldc, sA, sB, sC); break;
    }
    return hipGetLastError();
}

}  // namespace mla
