// Fused flash-MLA attention on the latent cache, gfx950 (CDNA4) bf16 matrix cores.
//
// Method (page "ik_llama.cpp MLA matrix absorption", sections 4 and 5): every head
// attends to the same latent rows [c_kv (512) | k_rope (64)], with score
//   s_j = scale * (q_lat . c_kv[j] + q_rope' . k_rope[j])
// and output o_lat = softmax(s) . c_kv -- one KV head shared by all query rows.
//
// Work decomposition.  A workgroup owns 32*NW query rows (flattened (token, head)
// pairs in prefill, the heads of one sequence in decode); wave w owns 32 of them.
// The workgroup streams the cache in tiles of 32 rows; each tile is read from HBM
// once into LDS and used by every wave, i.e. by all of the workgroup's rows.
//   S^T[key][row] = K_tile (32x576, LDS) x Q^T (576x32, registers)   36 MFMA 32x32x16
//   O^T[col][row] += V^T (512x32, LDS via ds_read_b64_tr_b16) x P^T   32 MFMA 32x32x16
// Computing the transposed products puts one query row in each lane (lanes l and
// l^32 share a row), so the softmax statistics and the output rescale are lane-local.
// The same LDS tile serves as K (all 576 columns) and as V (first 512).
//
// Online softmax (FlashAttention-2 recurrence, KV-cache page section 3.3) in the
// base-2 domain with a frozen maximum: a row's reference max m is taken from its first
// visible tile and never raised in place, so the 512-wide fp32 output accumulator is
// only ever touched by MFMA inside the key loop (no rescale).  Weights exp2(s - m) may
// exceed 1; they stay finite while s - m <= 64 (fp32/bf16 range is 2^128).  A row
// whose score exceeds m + 64 is marked, keeps tracking its true max for the rest of
// the pass, and the workgroup repeats the pass once with the marked rows starting
// from their true max (unmarked rows recompute bit-identical values).
//
// LDS tile layout (32 keys, 38912 B).  The latent part (512 bf16 = 64 chunks of 16 B per
// key) sits in rows of pitch 1088 B, logical chunk c at chunk c ^ mask_a(k); the rope part
// (64 bf16 = 8 chunks) follows in rows of 128 B, chunk c at c ^ mask_b(k).  One copy
// instruction then moves one whole latent row (uniform global address, lane-contiguous
// LDS), and both the 16-byte K-fragment reads and the transposing V reads are free of
// bank conflicts (see mask_a and mask_b).
#include "latent_tile.h"

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

namespace mla {

// Per-wave attention state and the tile computation.
//
// Each wave computes the scores and the softmax of its own 32 rows; the four waves share
// their bf16 weights P through LDS, and wave w accumulates O for all 128 rows of the
// workgroup over its quarter of the latent columns (128 columns).  Every V^T fragment
// read from LDS then feeds four MFMAs (one per row block): each tile's V is read from
// LDS once per workgroup, while the score MFMAs are not duplicated.
struct WaveState {
    bf16x8 q[36];     // Q^T fragments of the own rows: lane l holds row l%32,
                      // dims kk*16 + (l/32)*8 .. +7
    f32x16 o[4][4];   // O^T: column block nb of this wave's quarter (columns
                      // 128w + nb*32 ..), row block rb (the rows of wave rb)
    float m;          // frozen reference max of the own row (scaled, log2 domain)
    float lsum;       // this lane's share of the own row's softmax denominator
    bool bad;         // a score exceeded m + FREEZE_LIMIT: this pass is discarded
};

// Score product S^T = K Q^T of the tile in stage t: 36 MFMAs on one accumulator chain.
// Step kk requests the K fragment of step kk + QK_AHEAD right after its MFMA, so LDS
// latency overlaps matrix work; fill(kk) places other work (the previous tile's softmax,
// copy issue) between the MFMAs.  Latent chunk 2kk + hi (kk < 32) is stored at
// 4*(kk/2) + ((2*(kk%2) + hi) ^ mask_a(k)): two lane-dependent bases plus compile-time
// offsets; the four rope chunks (kk = 32 .. 35) take one address each.
//
// Causal masking rides on the chain's starting value: in a tile where some row of the
// wave ends (edge, wave-uniform) a slot past the row's bound starts at -inf, which every
// finite product leaves at -inf, so its weight comes out 0; other tiles start at 0.
// Slot e of a lane holds key key0 + hi*4 + (e/4)*8 + e%4.
template <typename Fill>
__device__ __forceinline__ f32x16 score_tile(const WaveState &st, const uint8_t MLA_LDS *t,
                                             bool edge, int key0, int lim, Fill fill) {
    const int l = threadIdx.x & 63, hi = l >> 5;
    const int k = l & 31;
    const int ma = mask_a(k), mb = mask_b(k);
    const uint8_t MLA_LDS *rowa = t + k * fl::PA;
    const uint8_t MLA_LDS *rowb = t + fl::A_BYTES + k * fl::PB;
    const uint8_t MLA_LDS *kb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) kb[b] = rowa + (((2 * b + hi) ^ ma) * 16);
    auto kaddr = [&](int kk) -> const uint8_t MLA_LDS * {
        return kk < 32 ? kb[kk & 1] + (kk >> 1) * 64 : rowb + (((2 * (kk - 32) + hi) ^ mb) * 16);
    };
    f32x16 s;
    constexpr int QK_AHEAD = 6;
    bf16x8 a[QK_AHEAD];
#pragma unroll
    for (int kk = 0; kk < QK_AHEAD; ++kk) a[kk] = *(const bf16x8 MLA_LDS *)kaddr(kk);
    static_for<36>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        if constexpr (kk == 0) {
            if (edge) {
                const int rel = lim - key0 - (hi << 2);
                f32x16 b;
#pragma unroll
                for (int e = 0; e < 16; ++e) b[e] = ((e >> 2) * 8 + (e & 3) <= rel) ? 0.0f : -INFINITY;
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], st.q[0], b, 0, 0, 0);
            } else {
                const f32x16 z = {};
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], st.q[0], z, 0, 0, 0);
            }
        } else {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk % QK_AHEAD], st.q[kk], s, 0, 0, 0);
        }
        constexpr int nk = kk + QK_AHEAD;
        if constexpr (nk < 36) a[kk % QK_AHEAD] = *(const bf16x8 MLA_LDS *)kaddr(nk);
        fill(kc);
        __builtin_amdgcn_sched_barrier(0);
    });
    return s;
}

// Softmax set-up for the raw scores s of keys key0 .. key0+31 (masked keys already hold
// -inf, see score_tile).  The row's reference max is frozen at its first visible tile, so
// the tile max is only needed while some row of the wave has no reference yet or is
// marked (wave-uniform branch).  Returns the exponent offset -m.
__device__ __forceinline__ float softmax_prep(WaveState &st, const f32x16 &s, int key0, int lim,
                                              float sc) {
    if (__builtin_amdgcn_ballot_w64((st.m == -INFINITY && key0 <= lim) || st.bad)) {
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[e]);
        tmax = pair_max(tmax) * sc;  // sc > 0: max of scaled = scaled max
        if (st.m == -INFINITY) {
            st.m = tmax;  // first visible keys of this row (o and lsum are still zero)
        } else if (tmax > st.m + fl::FREEZE_LIMIT || st.bad) {
            st.bad = true;
            st.m = fmaxf(st.m, tmax);  // track the true max for the repeated pass
        }
    }
    return (st.m == -INFINITY) ? 0.0f : -st.m;
}

// Overflow test of the frozen max.  A weight above 2^FREEZE_LIMIT makes this lane's tile
// sum exceed it, so the exact test (tile max against m + FREEZE_LIMIT, as in
// softmax_prep) only runs when some lane's sum does.
__device__ __forceinline__ void softmax_check(WaveState &st, const f32x16 &s, float psum,
                                              float sc) {
    if (__builtin_amdgcn_ballot_w64(!(psum <= 0x1p64f))) {
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[e]);
        tmax = pair_max(tmax) * sc;
        if (st.m != -INFINITY && tmax > st.m + fl::FREEZE_LIMIT) {
            st.bad = true;
            st.m = fmaxf(st.m, tmax);
        }
    }
}
static_assert(fl::FREEZE_LIMIT == 64.0f, "softmax_check compares against 2^64");

// V^T fragment addressing of the tile in stage t for O^T += V^T P^T, over the column
// quarter `cq` (uniform).  Lane: key kin + 8*h (+16 ks) and 4 columns at colb of each
// 32-column block.  Row ks*16 + h*8 + kin has mask mask_a(h*8 + kin); chunk 4nb + c3
// (c3 < 4) is stored at 4nb + (c3 ^ mask): one base per row half plus compile-time
// offsets.
struct VAddr {
    const uint8_t MLA_LDS *vb[2];
    __device__ __forceinline__ VAddr(const uint8_t MLA_LDS *t, int cq) {
        const int l = threadIdx.x & 63;
        const int G = l >> 4, lam = l & 15;
        const int kin = (G >> 1) * 4 + (lam >> 2);     // key within an 8-key group
        const int colb = (G & 1) * 16 + 4 * (lam & 3);  // column within a 32-column block
        const int c3 = colb >> 3, cb = (colb & 7) * 2;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            vb[h] = t + cq * 256 + (h * 8 + kin) * fl::PA + ((c3 ^ mask_a(h * 8 + kin)) * 16) + cb;
    }
    __device__ __forceinline__ bf16x8 load(int i) const {  // step i = (ks, nb) = (i/4, i%4)
        const int off = (i >> 2) * 16 * fl::PA + (i & 3) * 64;
        return tr_pair(vb[0] + off, vb[1] + off);
    }
};

constexpr int PV_AHEAD = 2;  // V^T read-ahead in PV steps (four MFMAs each)

// Weight of key slot e (e < 16) of this lane: exp2(s*sc - m); masked keys give 0.
__device__ __forceinline__ void soft_piece(const f32x16 &s, int e, float sc, float nmu,
                                           float &psum, bf16x8 (&p)[2]) {
    const float pe = __builtin_amdgcn_exp2f(fmaf(s[e], sc, nmu));
    asm volatile("" ::"v"(pe));  // computed here, between the MFMAs (not sunk to its use)
    psum += pe;
    p[e >> 3][e & 7] = f2bf(pe);
}

// P^T fragment (B operand of 32x32x16) of wave rb's weights for key step ks, from the
// exchange buffer: lane l holds row l & 31 of wave rb, keys 16 ks + 8 (l >> 5) .. +7.
__device__ __forceinline__ bf16x8 get_p(const uint8_t MLA_LDS *pbuf, int rb, int ks) {
    return ((const bf16x8 MLA_LDS *)(pbuf + rb * 2048))[ks * 64 + (threadIdx.x & 63)];
}

// O^T += V^T P^T over the 32 keys of a tile for all four row blocks: 8 steps (ks, nb),
// each one V^T fragment and four MFMAs (the weights of wave rb's rows), with a read-ahead
// ring whose first PV_AHEAD entries the caller loaded; fill(j) follows MFMA j (32 MFMAs).
// pk[rb] holds the weights of key step 0 (loaded by the caller from pbuf); each is
// replaced by key step 1's right after its last use, so the weights take 16 registers.
template <typename VA, typename Fill>
__device__ __forceinline__ void pv_tile(WaveState &st, const VA &va_addr,
                                        bf16x8 (&va)[PV_AHEAD], const uint8_t MLA_LDS *pbuf,
                                        bf16x8 (&pk)[4], Fill fill) {
    static_for<8>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int nb = i & 3;
        static_for<4>([&](auto rc) {
            constexpr int rb = decltype(rc)::value;
            st.o[nb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % PV_AHEAD], pk[rb],
                                                                   st.o[nb][rb], 0, 0, 0);
            if constexpr (i == 3) pk[rb] = get_p(pbuf, rb, 1);
            if constexpr (rb == 3) {
                constexpr int ni = i + PV_AHEAD;
                if constexpr (ni < 8) va[i % PV_AHEAD] = va_addr.load(ni);
            }
            fill(std::integral_constant<int, 4 * i + rb>{});
            __builtin_amdgcn_sched_barrier(0);
        });
    });
}

// Softmax of one tile's raw scores s while the O update of the previous tile runs (one
// step per MFMA, 32 steps): step 0 masks and sets the reference, odd step 2e+1 computes
// weight e (about two VALU operations per MFMA, which issue in the MFMA's shadow), step
// 31 also tests for overflow.  The weights land in p, their sum in psum.
// The weights alone (step 2e+1 computes weight e), for an O update whose softmax set-up
// and overflow test run outside it.
struct SoftPieces {
    const f32x16 &s;
    bf16x8 (&p)[2];
    float &psum;
    const float nmu, sc;
    __device__ __forceinline__ void operator()(int i) const {
        if (i & 1) soft_piece(s, i >> 1, sc, nmu, psum, p);
    }
};

struct SoftFill {
    WaveState &st;
    f32x16 &s;
    bf16x8 (&p)[2];
    float &psum;
    float &nmu;
    int key0, lim;
    float sc;
    __device__ __forceinline__ void operator()(int i) const {
        if (i == 0) nmu = softmax_prep(st, s, key0, lim, sc);
        if (i & 1) soft_piece(s, i >> 1, sc, nmu, psum, p);
        if (i == 31) softmax_check(st, s, psum, sc);
    }
};

// Weight exchange buffer: 2 KB per wave (p[0] at lane*16, p[1] at 1024 + lane*16).
constexpr int PBUF_BYTES = 4 * 2048;
__device__ __forceinline__ void put_p(uint8_t MLA_LDS *pbuf, const bf16x8 (&p)[2]) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    bf16x8 MLA_LDS *slot = (bf16x8 MLA_LDS *)(pbuf + w * 2048);
    slot[l] = p[0];
    slot[64 + l] = p[1];
}
// Key step 0's weights of all four waves (pv_tile loads step 1's).
__device__ __forceinline__ void get_p0(const uint8_t MLA_LDS *pbuf, bf16x8 (&pk)[4]) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) pk[rb] = get_p(pbuf, rb, 0);
}

// Rows that are not valid load a valid row's query instead (their keys are all masked,
// so their scores never reach the softmax).
__device__ __forceinline__ void load_q(WaveState &st, const bf16 *__restrict__ qrow) {
    const int hi = (threadIdx.x & 63) >> 5;
    const bf16 *p = qrow + hi * 8;
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) st.q[kk] = *(const bf16x8 *)(p + kk * 16);
}

__device__ __forceinline__ void init_acc(WaveState &st, float m0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[nb][rb][e] = 0.0f;
    st.m = m0;
    st.lsum = 0.0f;
    st.bad = false;
}

// Stream keys [kbeg, kend) of the bf16 `rows` through LDS and attend every tile.
// pbuf: the weight exchange buffer (PBUF_BYTES of LDS).  AF: every tile of the stream lies
// inside the cache (a multiple of 32 rows, kbeg a multiple of 32).  The copies of the tile
// two ahead then go out in every iteration, past the stream's end as well (the cache's last
// 32 rows, into the stage the tile two back left, which nothing reads again): they need no
// branches, and every wait allows the same count of copies in flight.
template <int NW, int NS, bool AF>
__device__ __forceinline__ void stream_keys(WaveState &st, uint8_t MLA_LDS *lds,
                                            uint8_t MLA_LDS *pbuf,
                                            const uint8_t *__restrict__ rows, int n_rows,
                                            int kbeg, int kend, int lim, int wlim, float sc) {
    static_assert(NW == 4, "four row blocks and four column quarters per workgroup");
    if (kend <= kbeg) return;
    const int ntiles = (kend - kbeg + fl::NK - 1) / fl::NK;
    const int cq = threadIdx.x >> 6;  // column quarter of this wave
    // Finish every earlier vector-memory load (queries, row bounds) before the first tile
    // copy.  The compiler cannot see the copies; a load it still counted as pending would
    // get a wait for all outstanding vector-memory operations inside the tile loop, which
    // would also drain the tile copies in flight on every tile.
    MLA_WAIT_VMCNT(0);
    {
        constexpr int PER = 9;  // copy instructions per wave per tile (issue_tile_bf16)
        const int last = n_rows - 1;
#pragma unroll
        for (int s = 0; s < 2; ++s)
            if (AF || s < ntiles)
                issue_tile_bf16<NW>(rows, kbeg + min(s, ntiles - 1) * fl::NK, last,
                                    lds + s * fl::TILE_BYTES);
        // Iteration t: wait for tile t, scores of tile t (with the copy of tile t+2 into
        // the stage tile t-2 used, free since the barrier), then the O update of tile t-1
        // carrying the softmax of tile t.  Tile t-1 stays resident for its V reads.  The
        // weights of tile t stay in registers until the top barrier of iteration t+1, which
        // follows every wave's last read of the exchange buffer (the O update of tile t-1
        // reads key step 1's weights while it runs); they are written right after it, and
        // a second barrier after score step 2 makes all four waves' weights visible.
        static_assert(NS == 4, "tiles t-1 .. t+2 resident or in flight");
        constexpr int P_SYNC = 2, P_READ = 28;
        static_assert(P_SYNC < P_READ && P_READ + 4 <= 36 - PV_AHEAD, "score steps");
        bf16x8 pprev[2];  // the own rows' weights of tile t-1
        for (int ti = 0; ti < ntiles; ++ti) {
            if (AF || ti + 1 < ntiles) {
                MLA_WAIT_VMCNT(PER);
            } else {
                MLA_WAIT_VMCNT(0);
            }
            __syncthreads();
            if (ti > 0) put_p(pbuf, pprev);
            const int nx = ti + 2;
            uint8_t MLA_LDS *ndst = lds + (nx % NS) * fl::TILE_BYTES;
            const int nkey0 = kbeg + nx * fl::NK;
            const bool more = nx < ntiles;
            // Full tiles take the fast copy path spread over the score MFMAs; the one tile
            // reaching past the cache's last row clamps per row and is issued at once.
            const bool full = AF || nkey0 + fl::NK - 1 <= last;
            const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
            const int skey = AF ? min(nkey0, last - (fl::NK - 1)) : nkey0;
            const uint8_t *sbase = rows + (int64_t)(skey + 8 * wu) * fl::RB;
            const uint32_t dsts = lds_u32(ndst);
            const CopyPlan plan = make_copy_plan();
            if (!AF && more && !full) issue_tile_bf16<NW>(rows, nkey0, last, ndst);  // once per stream
            // The copy's 9 instructions are spread over the score MFMAs: issued together,
            // the four waves' 36 instructions queue behind each other in the CU's memory
            // address unit.
            const VAddr vprev(lds + ((ti + NS - 1) % NS) * fl::TILE_BYTES, cq);
            bf16x8 va[PV_AHEAD], pk[4];
            const int key0 = kbeg + ti * fl::NK;
            // The row bound is made opaque per tile: values the compiler would derive from
            // it once and keep across the loop end up spilled, and a spill reload pending at
            // the loop would bring a wait for all vector-memory operations into it.
            int lim_t = lim;
            asm volatile("" : "+v"(lim_t));
            f32x16 s = score_tile(st, lds + (ti % NS) * fl::TILE_BYTES, key0 + fl::NK - 1 > wlim, key0,
                                  lim_t, [&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                if constexpr (kk == P_SYNC) {
                    if (ti > 0) __syncthreads();  // every wave's weights of tile t-1 written
                }
                if constexpr (kk >= P_READ && kk < P_READ + 4) {
                    if (ti > 0) pk[kk - P_READ] = get_p(pbuf, kk - P_READ, 0);
                }
                if (ti > 0 && kk >= 36 - PV_AHEAD)
                    va[kk - (36 - PV_AHEAD)] = vprev.load(kk - (36 - PV_AHEAD));
            });
            float psum = 0.0f;
            // the reference (its wave-uniform branch runs before the O update: a branch
            // among the MFMAs would split the block and the weights would sink to its end)
            float nmu = softmax_prep(st, s, key0, lim_t, sc);
            bf16x8 pcur[2];
            const SoftPieces soft{s, pcur, psum, nmu, sc};
            // Copy parts go between the O-update MFMAs (even steps; the softmax takes the
            // odd ones): that phase leaves LDS bandwidth for the copies' writes, while the
            // score MFMAs already keep LDS busy with K-fragment reads.
            auto fill = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                soft(j);
                if constexpr ((j & 3) == 2 || j == 16) {
                    if (AF || (more && full))
                        issue_part_full<(j == 16 ? 8 : j >> 2)>(sbase, plan, dsts, wu);
                }
            };
            if (ti > 0) {
                pv_tile(st, vprev, va, pbuf, pk, fill);
            } else {
                static_for<32>(fill);
            }
            softmax_check(st, s, psum, sc);
            st.lsum += psum;
            pprev[0] = pcur[0];
            pprev[1] = pcur[1];
        }
        __syncthreads();  // every wave's last O update done
        put_p(pbuf, pprev);
        __syncthreads();
        {
            const VAddr vlast(lds + ((ntiles - 1) % NS) * fl::TILE_BYTES, cq);
            bf16x8 va[PV_AHEAD], pk[4];
#pragma unroll
            for (int i = 0; i < PV_AHEAD; ++i) va[i] = vlast.load(i);
            get_p0(pbuf, pk);
            pv_tile(st, vlast, va, pbuf, pk, [](int) {});
        }
        if (AF) MLA_WAIT_VMCNT(0);  // the copies past the stream's end land before the stages are reused
        __syncthreads();
    }
}

// Small shared integers live in the last bytes of the weight exchange buffer, which the
// key stream alone writes: the group's key range is read before the stream starts, the
// pass flag is written and read after it ends (the stream starts and ends on a barrier),
// and the denominators of finish take only the buffer's first 512 bytes.  The tile stages
// hold the query staging before the stream, so no pad there is free.
struct Misc {
    int flag, wmax[4], wmin[4];
};
static_assert(sizeof(Misc) <= PBUF_BYTES - 512, "misc clear of the denominators");
__device__ __forceinline__ Misc *misc_of(uint8_t *pbuf_generic) {
    return (Misc *)(pbuf_generic + PBUF_BYTES - 64);
}
static_assert(sizeof(Misc) <= 64, "misc fits the last 64 bytes");

// Runs the key stream for the workgroup, repeating it once if any row was marked.
template <int NW, int NS, bool AF>
__device__ __forceinline__ void attend_range(WaveState &st, uint8_t MLA_LDS *lds,
                                             uint8_t MLA_LDS *pbuf, int *flag,
                                             const uint8_t *__restrict__ rows, int n_rows,
                                             int kbeg, int kend, int lim, int wlim, float sc) {
    float m0 = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
        init_acc(st, m0);
        stream_keys<NW, NS, AF>(st, lds, pbuf, rows, n_rows, kbeg, kend, lim, wlim, sc);
        if (threadIdx.x == 0) *flag = 0;
        __syncthreads();
        if (__builtin_amdgcn_ballot_w64(st.bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
        __syncthreads();
        const int again = *flag;
        __syncthreads();
        if (!again) break;
        m0 = st.m;  // marked rows: their true max; others: unchanged reference
    }
}

// Final normalisation and output.  Each wave holds O for all 128 rows (row block rb: the
// rows of wave rb) over its column quarter; the waves share the row denominators through
// LDS.  The normalised bf16 rows are staged in LDS (the tile stages are free once the key
// stream ended) and written out one 1 KB row per instruction: stores straight from the
// MFMA layout would scatter 8 bytes per lane over 32 rows.  row_dst(r) gives the output
// row of workgroup row r (0 .. 127; own rows of wave w are 32w .. 32w+31), or nullptr
// for rows past the end.  Returns lse (natural log) of this lane's own row.
constexpr int OPITCH = 1032;  // staged row pitch: rows 2 banks apart, 8-byte writes conflict-free
constexpr int OSTAGE_BYTES = 128 * OPITCH;
template <typename RowDst>
__device__ __forceinline__ float finish(WaveState &st, uint8_t MLA_LDS *stage,
                                        uint8_t MLA_LDS *pbuf, RowDst row_dst) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // recomputed, not kept from before the key stream
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, hi = l >> 5;
    const float lt = pair_sum(st.lsum);
    float MLA_LDS *den = (float MLA_LDS *)pbuf;  // buffer free: the key stream ended on a barrier
    if (l < 32) den[w * 32 + l] = lt;
    __syncthreads();
    float inv[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const float x = den[rb * 32 + (l & 31)];
        inv[rb] = x > 0.0f ? 1.0f / x : 0.0f;
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int r = rb * 32 + (l & 31);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = w * 128 + nb * 32 + g * 8 + hi * 4;
                const f32x16 &o = st.o[nb][rb];
                const bf16x4 v = {f2bf(o[g * 4 + 0] * inv[rb]), f2bf(o[g * 4 + 1] * inv[rb]),
                                  f2bf(o[g * 4 + 2] * inv[rb]), f2bf(o[g * 4 + 3] * inv[rb])};
                *(bf16x4 MLA_LDS *)(stage + r * OPITCH + col * 2) = v;
            }
    }
    __syncthreads();
    for (int j = 0; j < 32; ++j) {
        const int r = w * 32 + j;
        bf16 *dst = row_dst(r);
        if (dst) {
            const uint8_t MLA_LDS *src = stage + r * OPITCH + l * 16;
            const u32x2 a = *(const u32x2 MLA_LDS *)src;
            const u32x2 b = *(const u32x2 MLA_LDS *)(src + 8);
            const u32x4 v = {a[0], a[1], b[0], b[1]};
            *(u32x4 *)(dst + l * 8) = v;
        }
    }
    return lt > 0.0f ? (st.m + __log2f(lt)) * fl::LN2 : -INFINITY;
}
static_assert(OSTAGE_BYTES <= 4 * fl::TILE_BYTES, "output staging fits the tile stages");

// Normalised rows in float32 (partial results that are merged later keep full precision:
// a merged row can be much smaller than its parts).  Row r goes to dst + r*R floats,
// written straight from the accumulators (16 bytes per lane: 32-byte runs per row).
// Returns lse (natural log) of this lane's own row.
__device__ __forceinline__ float finish_f32(WaveState &st, uint8_t MLA_LDS *pbuf,
                                            float *__restrict__ dst) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // recomputed, not kept from before the key stream
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, hi = l >> 5;
    const float lt = pair_sum(st.lsum);
    float MLA_LDS *den = (float MLA_LDS *)pbuf;  // buffer free: the key stream ended on a barrier
    if (l < 32) den[w * 32 + l] = lt;
    __syncthreads();
    float inv[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const float x = den[rb * 32 + (l & 31)];
        inv[rb] = x > 0.0f ? 1.0f / x : 0.0f;
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        float *row = dst + (int64_t)(rb * 32 + (l & 31)) * fl::R + w * 128 + hi * 4;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16 &o = st.o[nb][rb];
                const f32x4 v = {o[g * 4 + 0] * inv[rb], o[g * 4 + 1] * inv[rb],
                                 o[g * 4 + 2] * inv[rb], o[g * 4 + 3] * inv[rb]};
                *(f32x4 *)(row + nb * 32 + g * 8) = v;
            }
    }
    return lt > 0.0f ? (st.m + __log2f(lt)) * fl::LN2 : -INFINITY;
}

constexpr int PF_NW = 4, PF_NS = 4;
constexpr int PF_ROWS = 32 * PF_NW;  // rows per workgroup
constexpr int PF_MAX_PARTS = 16;     // key parts per row group (the merge keeps one weight each)
constexpr int PF_MAX_ITEMS = 1024;   // (row group, part) items when groups are cut
// Block order of a cut prefill (a kernel argument: 2 KB, within the argument limit).
constexpr int PF_LISTS = 256;       // workgroups of a cut prefill: one per CU, each with a list
struct PrefillOrder {
    uint16_t item[PF_MAX_ITEMS];  // unit * nparts + part, grouped by workgroup
    uint16_t start[PF_LISTS + 1];  // workgroup b takes item[start[b] .. start[b + 1])
};
static_assert(PF_MAX_PARTS <= 16, "the merge holds every part's log-sum-exp and row at once");

// Prefill.  Rows are the flattened (token, head-in-chunk) pairs of all head chunks; a
// group of 128 rows attends to its keys in parts of ks keys (part p: keys [p*ks,
// (p+1)*ks)), one workgroup per (group, part).  A group whose keys fit one part writes
// its rows directly.  Otherwise every part writes its normalised rows (float32) and their
// log-sum-exp to the workspace slot (group, part), part 0 records the group's part count,
// and prefill_merge_kernel merges the slots after this kernel.  The part boundaries
// depend only on ks, so a row's result does not depend on how rows are grouped (head
// chunks): a row whose keys all lie in one part merges that part with weight exactly 1.
// One (row group, head chunk, key part) item of the prefill; returns with the LDS free
// for the next item except for a final barrier (the caller's).  AF: see stream_keys.
template <bool AF>
__device__ __forceinline__ void prefill_item(
    int unit, int part, const bf16 *__restrict__ q_cat, const int32_t *__restrict__ pos, int T,
    int H, const uint8_t *__restrict__ cache, int n_kv, int hc, int n_groups, int n_chunks,
    float sc, bf16 *__restrict__ o_lat, float *__restrict__ lse, int ks, int nparts,
    float *__restrict__ ws_o, float *__restrict__ ws_lse, int *__restrict__ ws_np,
    int64_t seq_stride, const int32_t *__restrict__ seq_n_kv) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    uint8_t MLA_LDS *lds = (uint8_t MLA_LDS *)lds_raw;
    uint8_t MLA_LDS *pbuf = lds + PF_NS * fl::TILE_BYTES;
    Misc *misc = misc_of(lds_raw + PF_NS * fl::TILE_BYTES);
    const int chunk = unit % n_chunks;
    const int grp = n_groups - 1 - unit / n_chunks;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar
    const int rows_total = T * hc;
    // row (token t, head h) of lane l's row in wave `wave`; false past the last row
    auto row_of = [&](int l, int wave, int &t, int &h) {
        const int r = grp * PF_ROWS + wave * 32 + (l & 31);
        const bool v = r < rows_total;
        t = v ? r / hc : 0;
        h = chunk * hc + (v ? r % hc : 0);
        return v;
    };
    int t, h;
    const bool valid = row_of(threadIdx.x & 63, w, t, h);
    // Batched caches (seq_n_kv given; one token per group): the group's token is a sequence
    // with its own rows at cache + t * seq_stride, all of its seq_n_kv[t] rows visible.
    int n_rows = n_kv;
    if (seq_n_kv) {
        const int sq = __builtin_amdgcn_readfirstlane(grp);
        n_rows = min(seq_n_kv[sq], n_kv);
        cache += (int64_t)sq * seq_stride;
    }
    int lim = -1;
    if (valid) lim = seq_n_kv ? n_rows - 1 : min(pos[t], n_kv - 1);

    // key range of the group (max) and of each wave (min of the rows' last visible key)
    // Butterfly reductions within the wave, one barrier for the group (atomics on one LDS
    // word would be serialised lane by lane).
    int wmx = lim, wmn = lim;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        wmx = max(wmx, __shfl_xor(wmx, o));
        wmn = min(wmn, __shfl_xor(wmn, o));
    }
    if ((threadIdx.x & 63) == 0) {
        misc->wmax[w] = wmx;
        misc->wmin[w] = wmn;
    }
    __syncthreads();
    const int kend = max(max(misc->wmax[0], misc->wmax[1]), max(misc->wmax[2], misc->wmax[3])) + 1;
    // parts holding keys of this group; a group whose rows see no key at all still has
    // part 0, which writes its rows (zeros, lse -inf) after an empty key range
    const int np = max(1, (kend + ks - 1) / ks);
    if (part >= np) return;  // uniform: nothing to attend to
    WaveState st;
    load_q(st, q_cat + ((int64_t)t * H + h) * fl::W);
    const int wlim = misc->wmin[w];
    // Kept opaque: folded into the loop, a constant start leads the compiler to keep more
    // values live across the tile loop, which then spills.
    int kbeg = part * ks;
    asm volatile("" : "+s"(kbeg));
    attend_range<PF_NW, PF_NS, AF>(st, lds, pbuf, &misc->flag, cache, n_rows, kbeg,
                               min(kbeg + ks, kend), lim, wlim, sc);
    // Output rows are recomputed here from the thread index: values kept from before the
    // key stream would stay live across it, crowd out the tile loop's registers and come
    // back as spill reloads among the output stores (each reload waits for every store
    // issued before it).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int l = tid & 63;
    if (np == 1) {
        // the group's part count tells the merge that these rows are final (the workspace
        // is not initialised by the caller)
        if (nparts > 1 && threadIdx.x == 0) ws_np[chunk * n_groups + grp] = 1;
        const float ls = finish(st, lds, pbuf, [&](int r) -> bf16 * {
            const int rr = grp * PF_ROWS + r;
            if (rr >= rows_total) return nullptr;
            return o_lat + ((int64_t)(rr / hc) * H + chunk * hc + rr % hc) * fl::R;
        });
        int ta, ha;
        if (lse && row_of(l, w, ta, ha) && l < 32) lse[(int64_t)ta * H + ha] = ls;
        return;
    }
    const int gid = chunk * n_groups + grp;
    const int64_t slot = (int64_t)gid * nparts + part;
    if (part == 0 && threadIdx.x == 0) ws_np[gid] = np;
    const float ls = finish_f32(st, pbuf, ws_o + slot * PF_ROWS * fl::R);
    if (l < 32) ws_lse[slot * PF_ROWS + w * 32 + l] = ls;
}

// Blocks are dispatched in index order, round-robin over the 8 XCDs and over the shader
// engines inside each, and a block waits for a free CU on its engine even when other
// engines have one: neighbouring blocks must carry similar work.  With one part per
// group (large prefills), block b takes unit b; units (row group, head chunk) go
// heaviest group (latest tokens) first, the chunks of a group together.  With several
// parts (small prefills), one workgroup per CU works through its own list of (unit,
// part) items, balanced on the host by estimated work (order.start / order.item), so
// that neither the dispatch order nor per-workgroup start-up costs decide the balance.
template <bool AF>
__global__ __launch_bounds__(64 * PF_NW, 1) void flash_prefill_bf16_kernel(
    const bf16 *__restrict__ q_cat, const int32_t *__restrict__ pos, int T, int H,
    const uint8_t *__restrict__ cache, int n_kv, int hc, int n_groups, int n_chunks, float sc,
    bf16 *__restrict__ o_lat, float *__restrict__ lse, int ks, int nparts,
    float *__restrict__ ws_o, float *__restrict__ ws_lse, int *__restrict__ ws_np,
    int64_t seq_stride, const int32_t *__restrict__ seq_n_kv, const PrefillOrder order) {
    if (nparts == 1) {
        prefill_item<AF>(blockIdx.x, 0, q_cat, pos, T, H, cache, n_kv, hc, n_groups, n_chunks, sc,
                     o_lat, lse, ks, nparts, ws_o, ws_lse, ws_np, seq_stride, seq_n_kv);
        return;
    }
    const int k1 = order.start[blockIdx.x + 1];
    const int units = n_groups * n_chunks;
    for (int k = order.start[blockIdx.x]; k < k1; ++k) {
        const int it = order.item[k];
        if (it / nparts >= units) continue;  // not an item of this launch (uniform)
        prefill_item<AF>(it / nparts, it % nparts, q_cat, pos, T, H, cache, n_kv, hc, n_groups,
                     n_chunks, sc, o_lat, lse, ks, nparts, ws_o, ws_lse, ws_np, seq_stride,
                     seq_n_kv);
        __syncthreads();  // the item's output staging and exchange areas are free again
    }
}

// Merge of the key parts of the row groups that were cut (flash_prefill_bf16_kernel):
// lse = log sum_p exp(lse_p), o = sum_p exp(lse_p - lse) o_p, the split-KV combine.
// Block (group, slab of 4 rows); wave w takes one row, lane l columns 8l .. 8l+7.
// MAXP: the largest part count the kernel handles (each thread holds every part's row piece
// and lse at once, so fewer slots keep more waves resident).
constexpr int MG_ROWS = 4;
template <int MAXP>
__global__ __launch_bounds__(64 * MG_ROWS) void prefill_merge_kernel(
    int T, int H, int hc, int n_groups, int nparts, const int *__restrict__ ws_np,
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse, bf16 *__restrict__ o_lat,
    float *__restrict__ lse) {
    const int gid = blockIdx.x / (PF_ROWS / MG_ROWS);
    const int np = ws_np[gid];
    if (np <= 1) return;  // written directly by its only part
    const int chunk = gid / n_groups, grp = gid % n_groups;
    const int r = (blockIdx.x % (PF_ROWS / MG_ROWS)) * MG_ROWS + (threadIdx.x >> 6);
    const int rr = grp * PF_ROWS + r;
    if (rr >= T * hc) return;
    const int l = threadIdx.x & 63;
    const int64_t slot0 = (int64_t)gid * nparts;
    // the lse and the rows of every part are requested together (one memory latency)
    float lp[MAXP];
    f32x4 va[MAXP], vb[MAXP];
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < np) {
            lp[p] = ws_lse[(slot0 + p) * PF_ROWS + r];
            const float *src = ws_o + ((slot0 + p) * PF_ROWS + r) * fl::R + l * 8;
            va[p] = *(const f32x4 *)src;
            vb[p] = *(const f32x4 *)(src + 4);
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
        if (p < np) m = fmaxf(m, lp[p]);
    const int64_t orow = (int64_t)(rr / hc) * H + chunk * hc + rr % hc;
    if (m == -INFINITY) {  // a row that sees no key (a negative position): zeros, lse -inf
        const bf16x8 z = {};
        *(bf16x8 *)(o_lat + orow * fl::R + l * 8) = z;
        if (lse && l == 0) lse[orow] = -INFINITY;
        return;
    }
    float ssum = 0.0f;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
        if (p < np) ssum += expf(lp[p] - m);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < np) {
            const float wt = expf(lp[p] - m) / ssum;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += wt * va[p][e];
                acc[4 + e] += wt * vb[p][e];
            }
        }
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f2bf(acc[e]);
    *(bf16x8 *)(o_lat + orow * fl::R + l * 8) = o;
    if (lse && l == 0) lse[orow] = m + logf(ssum);
}

// Host estimate of an item's time on MI355X (microseconds, fitted to measured item
// durations of the persistent cut prefill): a fixed cost (queries, key bounds, output
// rows), a cost per 32-key tile, an extra for writing a part instead of the final rows,
// and the cost of an item whose part holds no keys.  Only schedules depend on it.
constexpr double PF_COST_FIXED = 13.8, PF_COST_TILE = 2.07, PF_COST_CUT = 1.4, PF_COST_EMPTY = 2.24;

// Estimated tiles of part p of row group g (counted from the first tokens) and whether
// the group is cut, for the usual prefill positions (the T tokens are the last T of the
// n_kv cached rows).
static int est_tiles(int g, int p, int ks, int T, int hc, int n_kv, bool *cut) {
    const int64_t last_row = std::min<int64_t>((int64_t)(g + 1) * PF_ROWS, (int64_t)T * hc) - 1;
    const int64_t kend = std::min<int64_t>(n_kv, (int64_t)n_kv - T + last_row / hc + 1);
    *cut = kend > ks;
    const int64_t k = std::max<int64_t>(0, std::min<int64_t>(ks, kend - (int64_t)p * ks));
    return (int)((k + fl::NK - 1) / fl::NK);
}
static double est_cost(int tiles, bool cut) {
    return tiles > 0 ? PF_COST_FIXED + PF_COST_TILE * tiles + (cut ? PF_COST_CUT : 0.0)
                     : PF_COST_EMPTY;
}

// Longest-processing-time-first assignment of n items (costs c) to nb workgroups;
// owner[k] is the workgroup of the k-th item in `sorted` (items by decreasing cost).
// Returns the largest workgroup load.
static double lpt_assign(const double *c, int n, int nb, uint16_t *sorted, uint16_t *owner) {
    for (int i = 0; i < n; ++i) sorted[i] = (uint16_t)i;
    std::stable_sort(sorted, sorted + n, [&](uint16_t a, uint16_t b) { return c[a] > c[b]; });
    std::vector<std::pair<double, int>> heap;
    for (int b = 0; b < nb; ++b) heap.push_back({0.0, b});
    auto gt = [](const std::pair<double, int> &x, const std::pair<double, int> &y) { return x > y; };
    std::make_heap(heap.begin(), heap.end(), gt);
    double worst = 0.0;
    for (int k = 0; k < n; ++k) {
        std::pop_heap(heap.begin(), heap.end(), gt);
        auto &top = heap.back();
        top.first += c[sorted[k]];
        if (owner) owner[k] = (uint16_t)top.second;
        worst = std::max(worst, top.first);
        std::push_heap(heap.begin(), heap.end(), gt);
    }
    return worst;
}

// The host-side plans below (key-part size, work lists) are kept for the next call with
// the same shape; this lock guards them, so calls from several host threads are safe.
static std::mutex plan_lock;

// Parts per row group and keys per part.  Few row groups (fewer than two per CU) leave
// the longest groups setting the time; their keys are then cut into up to 4 parts of a
// fixed size ks (a multiple of the 32-key tile).  ks is chosen to minimise the estimated
// time of the persistent schedule, computed for the unchunked grouping, so that it
// depends on (T, H, n_kv) only: the part boundaries, hence the results, do not depend on
// the head-chunk cap.  Part counts leave room for the extra groups of a chunked grouping
// within the work-list capacity.
int prefill_parts(int T, int H, int n_kv, int *ks, bool batched) {
    constexpr int NUM_CUS = 256;
    *ks = n_kv;
    const int64_t groups = ((int64_t)T * H + PF_ROWS - 1) / PF_ROWS;
    if (groups >= 2 * NUM_CUS || n_kv <= fl::NK) return 1;
    std::lock_guard<std::mutex> guard(plan_lock);
    static int64_t cache_key[4] = {-1, -1, -1, -1};
    static int cache_ks = 0;
    const int64_t key[4] = {T, H, n_kv, batched};
    if (std::equal(key, key + 4, cache_key)) {
        *ks = cache_ks;
        return (n_kv + cache_ks - 1) / cache_ks;
    }
    // items G * P must fit the work lists; G <= groups + H over every head chunking (one
    // chunk, G = groups, for batched caches)
    const int pmax =
        (int)std::min<int64_t>(PF_MAX_PARTS, PF_MAX_ITEMS / (batched ? groups : groups + H));
    double best = 1e30;
    int best_ks = n_kv;
    std::vector<double> c;
    std::vector<uint16_t> sorted;
    for (int P = 1; P <= std::max(1, pmax); ++P) {
        const int lo = P == 1 ? n_kv : (n_kv + P - 1) / P;
        const int hi = P == 1 ? n_kv : (n_kv + P - 2) / (P - 1) - 1;
        for (int k = (lo + fl::NK - 1) / fl::NK * fl::NK; k <= std::max(lo, hi); k += fl::NK) {
            if (P > 1 && (n_kv + k - 1) / k != P) continue;
            const int kk = P == 1 ? n_kv : k;
            c.assign((size_t)groups * P, 0.0);
            sorted.resize(c.size());
            for (int g = 0; g < (int)groups; ++g)
                for (int p = 0; p < P; ++p) {
                    bool cut;
                    const int t = est_tiles(g, p, kk, T, H, n_kv, &cut);
                    c[(size_t)g * P + p] = est_cost(t, P > 1 && cut);
                }
            const double m = lpt_assign(c.data(), (int)c.size(), NUM_CUS, sorted.data(), nullptr);
            if (m < best - 1e-9) {
                best = m;
                best_ks = kk;
            }
            if (P == 1) break;
        }
    }
    std::copy(key, key + 4, cache_key);
    cache_ks = best_ks;
    *ks = best_ks;
    return (n_kv + best_ks - 1) / best_ks;
}

size_t prefill_workspace_bytes(int T, int H, int n_kv, int hc, bool batched) {
    int ks;
    const int P = prefill_parts(T, H, n_kv, &ks, batched);
    if (P == 1) return 0;
    const int64_t G = (int64_t)(H / hc) * (((int64_t)T * hc + PF_ROWS - 1) / PF_ROWS);
    const size_t cnt = ((size_t)G * 4 + 255) & ~(size_t)255;  // part count per group
    const size_t ls = ((size_t)G * P * PF_ROWS * 4 + 255) & ~(size_t)255;
    return cnt + ls + (size_t)G * P * PF_ROWS * fl::R * 4;
}

// Work lists of a cut prefill (G units x P parts) into `order`; returns the number of
// lists (workgroups).
static int build_order(int64_t G, int P, int ks, int T, int hc, int n_kv, int n_groups,
                       int n_chunks, PrefillOrder &order) {
    const int n_items = (int)G * P;
    double cost[PF_MAX_ITEMS];
    for (int it = 0; it < n_items; ++it) {
        const int u = it / P, p = it % P;
        bool cut;
        const int t = est_tiles(n_groups - 1 - u / n_chunks, p, ks, T, hc, n_kv, &cut);
        cost[it] = est_cost(t, cut);
    }
    uint16_t sorted[PF_MAX_ITEMS], owner[PF_MAX_ITEMS];
    const int n_lists = std::min(PF_LISTS, n_items);
    lpt_assign(cost, n_items, n_lists, sorted, owner);
    int count[PF_LISTS];
    std::fill(count, count + n_lists, 0);
    for (int k = 0; k < n_items; ++k) ++count[owner[k]];
    order.start[0] = 0;
    for (int b = 0; b < n_lists; ++b) order.start[b + 1] = (uint16_t)(order.start[b] + count[b]);
    int fillp[PF_LISTS];
    for (int b = 0; b < n_lists; ++b) fillp[b] = order.start[b];
    for (int k = 0; k < n_items; ++k) order.item[fillp[owner[k]]++] = sorted[k];
    return n_lists;
}

hipError_t launch_flash_prefill_bf16(const bf16 *q_cat, const int32_t *pos, int T, int H,
                                     const bf16 *cache, int n_kv, int hc, float scale,
                                     bf16 *o_lat, float *lse, void *ws, hipStream_t st,
                                     int64_t seq_stride, const int32_t *seq_n_kv) {
    if (T <= 0) return hipSuccess;
    const int rows = T * hc;
    const int n_groups = (rows + PF_ROWS - 1) / PF_ROWS;
    const int n_chunks = H / hc;
    int ks;
    const bool batched = seq_n_kv != nullptr;
    if (batched && hc != PF_ROWS) return hipErrorInvalidValue;  // one sequence per group
    const int P = prefill_parts(T, H, n_kv, &ks, batched);
    const int64_t G = (int64_t)n_chunks * n_groups;
    int *ws_np = (int *)ws;
    float *ws_lse = (float *)((char *)ws + (((size_t)G * 4 + 255) & ~(size_t)255));
    float *ws_o = (float *)((char *)ws_lse + (((size_t)G * P * PF_ROWS * 4 + 255) & ~(size_t)255));
    if (P == 1) ws_np = nullptr, ws_lse = nullptr, ws_o = nullptr;
    const size_t shm = (size_t)PF_NS * fl::TILE_BYTES + PBUF_BYTES;
    static std::atomic<uint64_t> lds_set[2];
    // every tile inside the cache: n_kv rows in whole tiles, tiles aligned to 32 keys (key
    // parts are multiples of 32); batched caches have their own row counts
    const bool all_full = !seq_n_kv && n_kv >= fl::NK && n_kv % fl::NK == 0;
    auto kern = all_full ? flash_prefill_bf16_kernel<true> : flash_prefill_bf16_kernel<false>;
    hipError_t ea = ensure_lds_limit((const void *)kern, (int)shm, lds_set[all_full]);
    if (ea != hipSuccess) return ea;
    // Work lists of a cut prefill: items by decreasing estimated cost (tiles plus a fixed
    // per-item cost), each assigned to the least loaded of the PF_LISTS workgroups (longest
    // processing time first).  Estimated with the usual prefill positions (the T tokens
    // are the last T of the n_kv cached rows): only the schedule depends on this estimate,
    // never the results (every item is listed; one without keys returns at once).  The
    // lists depend only on (T, H, n_kv, hc); they are kept for the next call, and each
    // launch takes its own copy (made under the plan lock).
    if (P > 1 && G * P > PF_MAX_ITEMS) return hipErrorInvalidValue;  // prefill_parts leaves room
    PrefillOrder order;
    int n_lists = 0;
    if (P > 1) {
        std::lock_guard<std::mutex> guard(plan_lock);
        static PrefillOrder cached;
        static int64_t cached_key[5] = {-1, -1, -1, -1, -1};
        static int cached_lists = 0;
        const int64_t key[5] = {T, H, n_kv, hc, batched};
        if (!std::equal(key, key + 5, cached_key)) {
            cached_lists = build_order(G, P, ks, T, hc, n_kv, n_groups, n_chunks, cached);
            std::copy(key, key + 5, cached_key);
        }
        order = cached;
        n_lists = cached_lists;
    }
    const unsigned nblocks = P > 1 ? (unsigned)n_lists : (unsigned)G;
    hipLaunchKernelGGL(kern, dim3(nblocks), dim3(64 * PF_NW), shm,
                       st, q_cat, pos, T, H, (const uint8_t *)cache, n_kv, hc, n_groups, n_chunks,
                       scale * fl::LOG2E, o_lat, lse, ks, P, ws_o, ws_lse, ws_np, seq_stride,
                       seq_n_kv, order);
    if (P > 1) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (P <= 4)
            hipLaunchKernelGGL(prefill_merge_kernel<4>, dim3((unsigned)(G * (PF_ROWS / MG_ROWS))),
                               dim3(64 * MG_ROWS), 0, st, T, H, hc, n_groups, P, ws_np, ws_o,
                               ws_lse, o_lat, lse);
        else
            hipLaunchKernelGGL(prefill_merge_kernel<PF_MAX_PARTS>,
                               dim3((unsigned)(G * (PF_ROWS / MG_ROWS))), dim3(64 * MG_ROWS), 0, st,
                               T, H, hc, n_groups, P, ws_np, ws_o, ws_lse, o_lat, lse);
    }
    return hipGetLastError();
}


// ------------------------------------------------------------- wide decode kernels
//
// Token generation (absorption page, section 8: a separate decode kernel), one workgroup
// per (sequence, key split, group of 128 heads), with the prefill's wave structure: wave w
// owns heads 32w .. 32w+31 of the group, each wave scores all 32 keys of a tile for its own
// heads, and the four waves share their weights so that each wave accumulates O for all
// 128 heads over a quarter of the latent columns.  Every tile serves all 128 heads.  Partials are
// written exactly as the split decode kernel writes them (normalised bf16 rows and their
// lse), so the split-KV combine merges them.  Three cache forms:
//   DW_Q8   Q8_0 rows (section 8.1): every raw tile is dequantised once into the bf16 tile
//           layout, its tasks interleaved with the score and O-update MFMAs of the previous
//           tile; raw tiles land in 3 stages, two tiles ahead, bf16 tiles in 2.
//   DW_BF16 bf16 rows; V^T fragments read from the row-major tile (ds_read_b64_tr_b16), as
//           in prefill; 2 stages, one tile ahead.
//   DW_VT   bf16 rows for the scores and a separate transposed copy of their latent part
//           for the O update: section 8.2's mode 1, a K cache and a V^T cache.  The V^T
//           tile [512 columns][32 keys] is read with ds_read_b128 (one instruction per
//           fragment instead of two transposing ones) at the cost of 1 KB more per key;
//           2 stages, one tile ahead.
// Per tile t: the scores of tile t, the softmax, the weight exchange, then O += P V over
// tile t.
enum { DW_Q8 = 0, DW_BF16 = 1, DW_VT = 2 };
constexpr int DW_NS = 2;  // tile stages
constexpr int DW_NR = 3;  // raw Q8_0 stages
constexpr int VT_TILE = fl::R * fl::NK * 2;  // 32768 B: [512 columns][32 keys] bf16
constexpr int DW_HEADS = PF_ROWS;            // 128 heads
__host__ __device__ constexpr int dw_stage(int mode) {
    return mode == DW_VT ? fl::TILE_BYTES + VT_TILE : fl::TILE_BYTES;
}
__host__ __device__ constexpr int dw_stages(int mode) {
    return mode == DW_Q8 ? DW_NS * fl::TILE_BYTES + DW_NR * Q8_RAW_STAGE : DW_NS * dw_stage(mode);
}
// the stages, or the output staging of finish() once the key stream ended
__host__ __device__ constexpr int dw_front(int mode) {
    return dw_stages(mode) > OSTAGE_BYTES ? dw_stages(mode) : OSTAGE_BYTES;
}
static_assert(dw_front(DW_Q8) + PBUF_BYTES <= 163840 && dw_front(DW_VT) + PBUF_BYTES <= 163840,
              "LDS budget");

// V^T fragments from the transposed tile (A operand of 32x32x16: lane l holds column l & 31
// of a 32-column block and the 8 keys 16 ks + 8 (l >> 5) .. +7 of key step ks).  Column c's
// 64 bytes hold its 32 keys in the order of the score slots (bits 2 and 3 of the key index
// swapped, as the V^T cache stores them), so those 8 keys are 16 contiguous bytes; 16-byte
// chunk q of column c sits at q ^ ((c >> 2) & 3), which spreads the 16 columns a
// 16-lane read touches over the 16 bank groups.
struct VAddrT {
    const uint8_t MLA_LDS *b[2];
    __device__ __forceinline__ VAddrT(const uint8_t MLA_LDS *vt, int cq) {
        const int l = threadIdx.x & 63;
        const int col = cq * 128 + (l & 31);     // plus 32 nb, a multiple of 16
        const int swz = ((l & 31) >> 2) & 3;     // (col >> 2) & 3
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) b[ks] = vt + col * 64 + (((2 * ks + (l >> 5)) ^ swz) << 4);
    }
    __device__ __forceinline__ bf16x8 load(int i) const {  // step i = (ks, nb) = (i/4, i%4)
        return *(const bf16x8 MLA_LDS *)(b[i >> 2] + (i & 3) * 32 * 64);
    }
};

// Copy of the V^T tile of keys key0 .. key0+31 (32 instructions, 8 per wave): instruction i
// moves columns 16i .. 16i+15, lane l column 16i + (l >> 2), stored chunk l & 3 (logical
// chunk (l & 3) ^ ((l >> 4) & 3), the swizzle of that column).  vt: the sequence's V^T rows
// (ld keys apart, bf16); the 32 keys of the tile must lie inside the rows.
__device__ __forceinline__ void issue_part_vt(const uint8_t *vt, int64_t ld_bytes, int key0,
                                              uint32_t dst, int i) {
    const int l = threadIdx.x & 63;
    const uint32_t voff = (uint32_t)((l >> 2) * ld_bytes) + ((((l & 3) ^ ((l >> 4) & 3))) << 4);
    lds_copy16(vt + (int64_t)key0 * 2 + (int64_t)16 * i * ld_bytes, voff, dst + (uint32_t)(i * 1024));
}

// Zeroes the V^T tile entries of keys past the sequence end (nk rows; the tile starts at
// key0): their weights are 0, but the transposed rows hold whatever the caller left there.
__device__ __forceinline__ void zero_vt_tail(uint8_t MLA_LDS *vt, int key0, int nk) {
    for (int e = threadIdx.x; e < fl::R * 4; e += 64 * PF_NW) {
        const int c = e >> 2, q = e & 3;          // column, logical chunk
        uint8_t MLA_LDS *p = vt + c * 64 + ((q ^ ((c >> 2) & 3)) << 4);
        bf16x8 v = *(bf16x8 MLA_LDS *)p;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            const int pos = q * 8 + x;  // slot order: key = pos with bits 2 and 3 swapped
            const int key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1);
            if (key0 + key >= nk) v[x] = (bf16)0.0f;
        }
        *(bf16x8 MLA_LDS *)p = v;
    }
}

// Keys [kbeg, kend) of one sequence (nk rows; lim = nk - 1 is every row's last visible
// key).  rows: the sequence's cache rows; vt, vt_ld: its V^T rows (DW_VT).
template <int MODE>
__device__ __forceinline__ void stream_keys_w(WaveState &st, uint8_t MLA_LDS *lds,
                                              uint8_t MLA_LDS *pbuf,
                                              const uint8_t *__restrict__ rows,
                                              const uint8_t *__restrict__ vt, int64_t vt_ld,
                                              int nk, int kbeg, int kend, float sc) {
    constexpr int NW = PF_NW;
    if (kend <= kbeg) return;
    const int ntiles = (kend - kbeg + fl::NK - 1) / fl::NK;
    const int lim = nk - 1;
    const int cq = threadIdx.x >> 6;  // column quarter of this wave
    const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // only the sequence's last tile can reach past its end
    auto tail = [&](int j) { return kbeg + (j + 1) * fl::NK > nk; };
    auto stage = [&](int j) { return lds + (j & 1) * dw_stage(MODE); };
    [[maybe_unused]] uint8_t MLA_LDS *raw = lds + DW_NS * fl::TILE_BYTES;
    [[maybe_unused]] constexpr int PX = Q8_X4_INST / NW, PD = q8_inst_per_wave<NW>();
    [[maybe_unused]] auto cnt = [&](int j) { return j < ntiles ? (tail(j) ? PD : PX) : 0; };
    [[maybe_unused]] auto issue_raw = [&](int j) {
        uint8_t MLA_LDS *dst = raw + (j % DW_NR) * Q8_RAW_STAGE;
        if (tail(j))
            issue_tile_q8<NW>(rows, kbeg + j * fl::NK, nk, dst);
        else
            issue_tile_q8_full<NW>(rows, kbeg + j * fl::NK, dst);
    };
    // a whole tile's copies at once (bf16 forms: the first tile and the tail tile)
    [[maybe_unused]] auto issue_all = [&](int j) {
        const int key0 = kbeg + j * fl::NK;
        issue_tile_bf16<NW>(rows, key0, nk - 1, stage(j));
        if constexpr (MODE == DW_VT) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                issue_part_vt(vt, 2 * vt_ld, key0, lds_u32(stage(j) + fl::TILE_BYTES), 8 * wu + i);
        }
    };
    // Every earlier vector-memory load (queries, the sequence length) completes before the
    // first copy: the compiler does not see the copies (see lds_copy16).
    [[maybe_unused]] const Q8CopyParts<NW> qparts;
    MLA_WAIT_VMCNT(0);
    if constexpr (MODE == DW_Q8) {
        for (int j = 0; j < DW_NR; ++j)
            if (j < ntiles) issue_raw(j);
        wait_vm_q8(cnt(1) + cnt(2));  // raw tile 0 landed
        __syncthreads();
        DequantQ8{raw, lds, kbeg, nk}.all();
    } else {
        issue_all(0);
    }
    for (int t = 0; t < ntiles; ++t) {
        if constexpr (MODE == DW_Q8) {
            // raw tile t+1 landed (only raw tile t+2 may be in flight); the barrier also
            // orders the dequantisation of tile t, the O update of tile t-1 (whose stage
            // the dequantisation of tile t+1 overwrites) and the reads of raw tile t (whose
            // stage takes raw tile t+3)
            wait_vm_q8(cnt(t + 2));
            __syncthreads();
            // raw tile t+3 (into the stage raw tile t left): the tail tile's copies here, a
            // whole tile's spread over the score steps below
            if (t + 3 < ntiles && tail(t + 3)) issue_raw(t + 3);
        } else {
            // tile t landed; the barrier also orders the O update of tile t-1, whose stage
            // takes tile t+1
            MLA_WAIT_VMCNT(0);
            __syncthreads();
            if constexpr (MODE == DW_VT) {
                // (ordered before the O update by the exchange barrier below)
                if (tail(t)) zero_vt_tail(stage(t) + fl::TILE_BYTES, kbeg + t * fl::NK, nk);
            }
            if (t + 1 < ntiles && tail(t + 1)) issue_all(t + 1);
        }
        const uint8_t MLA_LDS *tile = stage(t);
        const bool next = t + 1 < ntiles;
        // the next bf16 tile's copies when it lies inside the sequence, spread over the
        // score steps (a copy instruction blocks its wave while the address unit is backed
        // up): K parts after steps 0, 4, .., 32, V^T parts after steps 2, 6, .., 30
        [[maybe_unused]] const bool fast = next && !tail(t + 1);
        [[maybe_unused]] const int nkey0 = kbeg + (t + 1) * fl::NK;
        [[maybe_unused]] const uint8_t *sbase = rows + (int64_t)(nkey0 + 8 * wu) * fl::RB;
        [[maybe_unused]] const uint32_t ndst = lds_u32(stage(t + 1));
        [[maybe_unused]] const CopyPlan plan = make_copy_plan();
        // Q8_0: the dequantisation of raw tile t+1, also after the split's last tile (it
        // then converts a stale raw stage into the free bf16 stage: both lie inside LDS, and
        // nothing reads the result), which keeps the tile loop free of branches around it
        [[maybe_unused]] const DequantQ8Pieces dqp(raw + ((t + 1) % DW_NR) * Q8_RAW_STAGE,
                                                   lds + ((t + 1) & 1) * fl::TILE_BYTES, nkey0, nk);
        [[maybe_unused]] const bool raw_fast = t + 3 < ntiles && !tail(t + 3);
        [[maybe_unused]] const uint8_t *rbase = rows + (int64_t)(kbeg + (t + 3) * fl::NK) * fl::Q8_RB;
        [[maybe_unused]] const uint32_t rstage = lds_u32(raw + ((t + 3) % DW_NR) * Q8_RAW_STAGE);
        [[maybe_unused]] DequantQ8::Words dw;
        [[maybe_unused]] DequantQ8Pieces::Mid mid;
        [[maybe_unused]] bf16x4 h0, h1;
        const int key0 = kbeg + t * fl::NK;
        int lim_t = lim;
        asm volatile("" : "+v"(lim_t));
        // Q8_0: the dequantisation of raw tile t+1 between the MFMAs, one piece per step:
        // task m (0 .. 4) is fetched after score step 7m, prepared after step 7m + 3 and
        // converted and stored after steps 7m + 4 and 7m + 5; raw copy instruction m of
        // tile t+3 follows step 7m + 1.  Tasks 5 .. 8 take the O-update steps 8(m - 5) + 0,
        // 3, 4 and 5 the same way.
        f32x16 s = score_tile(st, tile, key0 + fl::NK - 1 > lim, key0, lim_t, [&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            if constexpr (MODE == DW_Q8) {
                constexpr int m = kk / 7, r = kk % 7;
                if constexpr (m < 5) {
                    if constexpr (r == 0) dqp.fetch(m, dw);
                    if constexpr (r == 1) {
                        if (raw_fast) qparts.issue(rbase, rstage, m);
                    }
                    if constexpr (r == 3) dqp.prep(dw, mid);
                    if constexpr (r == 4) dqp.half(mid, 0, h0);
                    if constexpr (r == 5) {
                        dqp.half(mid, 1, h1);
                        dqp.store(m, h0, h1);
                    }
                }
            } else {
                if (fast) {
                    if constexpr (kk % 4 == 0) issue_part_full<kk / 4>(sbase, plan, ndst, wu);
                    if constexpr (MODE == DW_VT && kk % 4 == 2 && kk / 4 < 8)
                        issue_part_vt(vt, 2 * vt_ld, nkey0, ndst + fl::TILE_BYTES, 8 * wu + kk / 4);
                }
            }
        });
        static_assert(7 * 4 + 5 < 36 && 4 * 8 < 36 && Q8_X4_INST / NW == 5,
                      "every task, raw copy and bf16 copy inside the score steps");
        float nmu = 0.0f, psum = 0.0f;
        bf16x8 pcur[2];
        const SoftFill soft{st, s, pcur, psum, nmu, key0, lim_t, sc};
        static_for<32>(soft);
        st.lsum += psum;
        put_p(pbuf, pcur);
        __syncthreads();  // every wave's weights visible
        bf16x8 pk[4];
        get_p0(pbuf, pk);
        auto o_update = [&](const auto &va_addr) {
            bf16x8 va[PV_AHEAD];
#pragma unroll
            for (int i = 0; i < PV_AHEAD; ++i) va[i] = va_addr.load(i);
            pv_tile(st, va_addr, va, pbuf, pk, [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (MODE == DW_Q8) {
                    constexpr int m = 5 + j / 8, r = j % 8;
                    if constexpr (r == 0) dqp.fetch(m, dw);
                    if constexpr (r == 3) dqp.prep(dw, mid);
                    if constexpr (r == 4) dqp.half(mid, 0, h0);
                    if constexpr (r == 5) {
                        dqp.half(mid, 1, h1);
                        dqp.store(m, h0, h1);
                    }
                }
            });
        };
        if constexpr (MODE == DW_VT)
            o_update(VAddrT(tile + fl::TILE_BYTES, cq));
        else
            o_update(VAddr(tile, cq));
        static_assert(5 + 3 == DequantQ8::TASKS - 1, "four tasks in the O-update steps");
    }
    __syncthreads();
}

// Block (unit u = (b * n_splits + split) * hgroups + head group): blocks go round-robin
// over the XCDs; no two blocks share a tile, so no placement matters.
template <int MODE>
__global__ __launch_bounds__(64 * PF_NW, 1) void flash_decode_w_kernel(
    const bf16 *__restrict__ q_cat, int H, const uint8_t *__restrict__ cache, int64_t seq_stride,
    const uint8_t *__restrict__ vt, int64_t vt_seq_stride, int64_t vt_ld,
    const int32_t *__restrict__ n_kv, int n_kv_max, int n_splits, int split_len, int hgroups,
    float sc, bf16 *__restrict__ part_o, float *__restrict__ part_lse) {
    const int u = blockIdx.x;
    const int hg = u % hgroups;
    const int b = u / hgroups / n_splits, sp = (u / hgroups) % n_splits;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    uint8_t MLA_LDS *lds = (uint8_t MLA_LDS *)lds_raw;
    uint8_t MLA_LDS *pbuf = lds + dw_front(MODE);
    Misc *misc = misc_of(lds_raw + dw_front(MODE));
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nk = min(n_kv[b], n_kv_max);  // rows past n_kv_max are never read
    const int k0 = sp * split_len;
    const int k1 = min(k0 + split_len, nk);
    // heads past H load head H-1's query; their rows are never written
    const int h = min(hg * DW_HEADS + w * 32 + (int)(threadIdx.x & 31), H - 1);
    WaveState st;
    load_q(st, q_cat + ((int64_t)b * H + h) * fl::W);
    const uint8_t *rows = cache + b * seq_stride;
    const uint8_t *vts = MODE == DW_VT ? vt + b * vt_seq_stride : nullptr;
    float m0 = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
        init_acc(st, m0);
        stream_keys_w<MODE>(st, lds, pbuf, rows, vts, vt_ld, nk, k0, k1, sc);
        if (threadIdx.x == 0) misc->flag = 0;
        __syncthreads();
        if (__builtin_amdgcn_ballot_w64(st.bad) && (threadIdx.x & 63) == 0) atomicOr(&misc->flag, 1);
        __syncthreads();
        const int again = misc->flag;
        __syncthreads();
        if (!again) break;
        m0 = st.m;  // marked rows: their true max; others: unchanged reference
    }
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // recomputed, not kept across the key stream
    const int l = tid & 63;
    const int64_t pi = ((int64_t)b * n_splits + sp) * H + hg * DW_HEADS;
    const int hmax = H - hg * DW_HEADS;  // heads of this group
    const float ls = finish(st, lds, pbuf, [&](int r) -> bf16 * {
        return r < hmax ? part_o + (pi + r) * fl::R : nullptr;
    });
    const int r = __builtin_amdgcn_readfirstlane(tid >> 6) * 32 + (l & 31);
    if (l < 32 && r < hmax) part_lse[pi + r] = ls;
}

int decode_wide_heads() { return DW_HEADS; }

template <int MODE>
static hipError_t launch_w(const bf16 *q_cat, const void *cache, int64_t seq_stride_bytes,
                           const void *vt, int64_t vt_seq_stride_bytes, int64_t vt_ld,
                           const int32_t *n_kv, int n_kv_max, int B, int H, int n_splits,
                           int split_len, float scale, bf16 *part_o, float *part_lse,
                           hipStream_t st) {
    const int hgroups = (H + DW_HEADS - 1) / DW_HEADS;
    const int64_t nblocks = (int64_t)B * n_splits * hgroups;
    if (nblocks <= 0 || nblocks > INT32_MAX) return hipErrorInvalidValue;
    const int shm = dw_front(MODE) + PBUF_BYTES;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_lds_limit((const void *)flash_decode_w_kernel<MODE>, shm, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(flash_decode_w_kernel<MODE>, dim3((unsigned)nblocks), dim3(64 * PF_NW), shm,
                       st, q_cat, H, (const uint8_t *)cache, seq_stride_bytes,
                       (const uint8_t *)vt, vt_seq_stride_bytes, vt_ld, n_kv, n_kv_max, n_splits,
                       split_len, hgroups, scale * fl::LOG2E, part_o, part_lse);
    return hipGetLastError();
}

hipError_t launch_flash_decode_q8_wide(const bf16 *q_cat, const void *cache,
                                       int64_t seq_stride_bytes, const int32_t *n_kv,
                                       int n_kv_max, int B, int H, int n_splits, int split_len,
                                       float scale, bf16 *part_o, float *part_lse,
                                       hipStream_t st) {
    return launch_w<DW_Q8>(q_cat, cache, seq_stride_bytes, nullptr, 0, 0, n_kv, n_kv_max, B, H,
                           n_splits, split_len, scale, part_o, part_lse, st);
}

hipError_t launch_flash_decode_bf16_wide(const bf16 *q_cat, const void *cache,
                                         int64_t seq_stride_bytes, const void *vt,
                                         int64_t vt_seq_stride_bytes, int64_t vt_ld,
                                         const int32_t *n_kv, int n_kv_max, int B, int H,
                                         int n_splits, int split_len, float scale, bf16 *part_o,
                                         float *part_lse, hipStream_t st) {
    if (vt)
        return launch_w<DW_VT>(q_cat, cache, seq_stride_bytes, vt, vt_seq_stride_bytes, vt_ld,
                               n_kv, n_kv_max, B, H, n_splits, split_len, scale, part_o, part_lse,
                               st);
    return launch_w<DW_BF16>(q_cat, cache, seq_stride_bytes, nullptr, 0, 0, n_kv, n_kv_max, B, H,
                             n_splits, split_len, scale, part_o, part_lse, st);
}

// Transposed latent rows for the K + V^T cache form (absorption page, section 8.2, mode 1):
// vt[c][32 g + p] = cache[32 g + pi(p)][c] for the 512 latent columns c, pi swapping bits 2
// and 3 of the in-group index (an involution), so that a 16-byte run of a column holds the
// 8 keys one lane's score slots cover.  Block (32-key group, 64-column chunk, sequence);
// keys outside [row0, row1) are neither read nor written.
__global__ __launch_bounds__(256) void transpose_v_kernel(const bf16 *__restrict__ cache,
                                                          int64_t seq_stride, int row0, int row1,
                                                          bf16 *__restrict__ vt,
                                                          int64_t vt_seq_stride, int64_t vt_ld) {
    __shared__ bf16 t[fl::NK][64 + 2];
    const int kb = (row0 / fl::NK + (int)blockIdx.x) * fl::NK, c0 = (int)blockIdx.y * 64;
    const bf16 *src = cache + (int64_t)blockIdx.z * seq_stride;
    bf16 *dst = vt + (int64_t)blockIdx.z * vt_seq_stride;
    for (int i = threadIdx.x; i < fl::NK * 64; i += 256) {
        const int k = i >> 6, c = i & 63, key = kb + k;
        t[k][c] = (key >= row0 && key < row1) ? src[(int64_t)key * fl::W + c0 + c] : (bf16)0.0f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * fl::NK; i += 256) {
        const int c = i >> 5, p = i & 31;
        const int k = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
        const int key = kb + k;
        if (key >= row0 && key < row1) dst[(int64_t)(c0 + c) * vt_ld + kb + p] = t[k][c];
    }
}

hipError_t launch_transpose_v(const bf16 *cache, int64_t seq_stride_bytes, int B, int row0,
                              int row1, bf16 *vt, int64_t vt_seq_stride_bytes, int64_t vt_ld,
                              hipStream_t st) {
    if (row1 <= row0 || B <= 0) return hipSuccess;
    const int groups = (row1 - 1) / fl::NK - row0 / fl::NK + 1;
    hipLaunchKernelGGL(transpose_v_kernel, dim3((unsigned)groups, fl::R / 64, (unsigned)B),
                       dim3(256), 0, st, cache, seq_stride_bytes / 2, row0, row1, vt,
                       vt_seq_stride_bytes / 2, vt_ld);
    return hipGetLastError();
}

}  // namespace mla
