// Split-KV decode partials on the latent cache (bf16 or Q8_0 rows), gfx950 matrix cores.
//
// Method (page "ik_llama.cpp MLA matrix absorption", sections 4, 5 and 8): one new token
// per sequence attends to every cached row [c_kv (512) | k_rope (64)] with
//   s_j = scale * (q_lat . c_kv[j] + q_rope' . k_rope[j]),   o_lat = softmax(s) . c_kv,
// all heads sharing the one latent row (a single KV head).  Token generation has its own
// kernel (section 8); the key range is cut into splits, each of which emits a partial
// (o_s, lse_s) that the combine step merges with a log-sum-exp.
//
// Work decomposition.  A workgroup owns 64 heads of one sequence and one key split, and
// streams the split's rows through LDS in tiles of 32 (the tile layout of latent_tile.h,
// each tile read from HBM once and used by all 64 heads).  Decode has one query per head,
// so a workgroup with few heads leaves more workgroups for the key range: at 128 heads
// and one sequence, 2 head groups x 128 splits fill the 256 CUs while each workgroup
// loads only 64 query rows and writes only 64 partial rows (the query loads and the
// partial rows, not the cache, dominated a 128-head workgroup's traffic).
//
// Wave w = (key half kh = w & 1, head half hh = w >> 1):
//   scores   S^T[16 keys of half kh][32 heads of half hh]  = K Q^T over the 576 dims:
//            18 steps x 2 v_mfma_f32_16x16x32_bf16 sharing one K fragment (16 keys x 32
//            dims, 16 B per lane, conflict-free by the tile layout);
//   weights  P = exp2(S*scale*log2e - m) for its 16 x 32 block, written to an LDS weight
//            buffer [64 heads][32 keys];
//   output   O^T[128 columns of quarter w][all 64 heads] += V^T P^T over the tile's 32
//            keys: 4 column blocks x 2 key steps, each V^T fragment (ds_read_b64_tr_b16,
//            natural key order) feeding two v_mfma_f32_32x32x16_bf16 (two head blocks).
// The O update of tile t-1 runs between the score MFMAs of tile t; one workgroup barrier
// per tile orders the tile copies and the weight buffers (double-buffered).
//
// Softmax: the FlashAttention-2 recurrence (KV-cache page, section 3.3) with a frozen
// reference maximum m per head, taken from the split's first tile (the two key-half
// waves of a head agree through LDS) and never raised, so the accumulators are touched
// only by MFMA.  Weights exp2(s - m) stay finite while s - m <= 64; a score beyond that
// marks the workgroup, which repeats the pass once from the true maxima (exact either way).
#include "latent_tile.h"

namespace mla {

namespace dq {
constexpr int NW = 4;                          // waves per workgroup
constexpr int HPB = 64;                        // heads per workgroup
constexpr int KSTEPS = fl::W / 32;             // 18 score steps of 32 dims
constexpr int PBUF = HPB * fl::NK * 2;         // 4096 B: one weight buffer
constexpr int NS_BF16 = 4;                     // bf16 tile stages (tile t and 3 in flight)
constexpr int NRAW = 4;                        // raw Q8_0 stages (3 in flight)
constexpr int COPY_PER = 9;                    // copy instructions per wave per bf16 tile
constexpr int QCH = fl::W / 8;                 // 72 query chunks of 16 B per head
constexpr int QCOPY_PER = QCH / NW;            // 18 query copy instructions per wave
constexpr int OPITCH = 1032;                   // output staging row pitch (bytes)
// LDS: tile stages, then the weight buffers.  bf16: 4 stages.  Q8_0: 2 bf16 stages and
// 4 raw stages.  The query rows are staged once, before the key stream, over the
// stages that are still free: 2-3 (bf16) or the two bf16 stages (Q8_0).
__host__ __device__ constexpr int stage_bytes(bool q8) {
    return q8 ? 2 * fl::TILE_BYTES + NRAW * Q8_RAW_STAGE : NS_BF16 * fl::TILE_BYTES;
}
// weight buffers: two on the bf16 path (tile t's weights are written while tile t-1's
// are read), one on the Q8_0 path (a barrier separates writing and reading)
__host__ __device__ constexpr int npbuf(bool q8) { return q8 ? 1 : 2; }
__host__ __device__ constexpr int lds_bytes(bool q8) { return stage_bytes(q8) + npbuf(q8) * PBUF; }
__host__ __device__ constexpr int qstage_off(bool q8) { return q8 ? 0 : 2 * fl::TILE_BYTES; }
static_assert(lds_bytes(false) <= 163840 && lds_bytes(true) <= 163840, "LDS budget");
static_assert(QCH * HPB * 16 <= 2 * fl::TILE_BYTES, "query staging fits two bf16 stages");
static_assert(QCH % NW == 0, "query copies split evenly over the waves");
static_assert(HPB * OPITCH <= 2 * fl::TILE_BYTES, "output staging fits two stages");
// Small exchange areas live in the 64-byte pads of the latent rows of stage 0 (never
// written by tile copies nor read by fragment loads): the pass flag in row 0, the
// per-wave maxima of the reference exchange in rows 1..8 (16 floats each).
__device__ __forceinline__ uint32_t pad_off(int row) { return (uint32_t)(row * fl::PA + 1024); }
}  // namespace dq

// Per-lane state.  QK/softmax role: heads hh*32 + hb*16 + (l & 15), keys of half kh.
// Output role: heads hb2*32 + (l & 31), columns 128w + cb*32 + ...
struct DqState {
    bf16x8 q[2][dq::KSTEPS];  // Q^T fragments (B operand of 16x16x32): dims kk*32 + (l/16)*8
    f32x16 o[4][2];           // O^T blocks: column block cb, head block hb2
    float m[2];               // frozen reference max per head block (scaled, log2 domain)
    float lsum[2];            // this lane's share of the head's denominator
    bool bad;                 // a score exceeded m + FREEZE_LIMIT in this pass
};

// P^T fragments of the previous tile's weights (B operand of 32x32x16: lane l holds head
// hb2*32 + (l & 31), keys ks*16 + (l >> 5)*8 .. +7).
__device__ __forceinline__ void load_pt(const uint8_t MLA_LDS *pb, bf16x8 (&pt)[2][2]) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            pt[hb2][ks] = *(const bf16x8 MLA_LDS *)(pb + pbuf_r_off(hb2 * 32 + (l & 31), ks, l >> 5));
}

// Scores of one tile (stage t) for both head blocks: 18 steps, each one K fragment (read
// four steps ahead) feeding two 16x16x32 MFMAs.  Even and odd steps accumulate into
// separate chains (four in flight), summed at the end.  fill(kk) follows step kk.
//
// The score MFMAs are asm statements with VGPR accumulators: given the choice, the
// register allocator puts the chains into the AGPRs of O blocks and moves those blocks
// to VGPRs and back on every tile (112 extra instructions per tile, in a loop that is
// bound by instruction issue).  The chains start from a literal zero (no VALU write feeds
// an MFMA source), and since the compiler does not count wait states after an MFMA it
// cannot see, 20 of them separate the last MFMAs from the reads of their results.
template <typename KA, typename Fill>
__device__ __forceinline__ void score_tile_q(const DqState &st, const uint8_t MLA_LDS *t,
                                             const KA &ka, f32x4 (&s)[2], Fill fill) {
    f32x4 c[2][2];
    constexpr int AH = 4;
    bf16x8 a[AH];
#pragma unroll
    for (int kk = 0; kk < AH; ++kk) a[kk] = *(const bf16x8 MLA_LDS *)(t + ka.at(kk));
    static_for<dq::KSTEPS>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        constexpr int par = kk & 1;
        if constexpr (kk < 2) {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                             : "=&v"(c[hb][par]) : "v"(a[kk % AH]), "v"(st.q[hb][kk]));
        } else {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                             : "+v"(c[hb][par]) : "v"(a[kk % AH]), "v"(st.q[hb][kk]));
        }
        if constexpr (kk + AH < dq::KSTEPS)
            a[kk % AH] = *(const bf16x8 MLA_LDS *)(t + ka.at(kk + AH));
        fill(kc);
        __builtin_amdgcn_sched_barrier(0);
    });
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(c[0][0]), "+v"(c[0][1]), "+v"(c[1][0]), "+v"(c[1][1]));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[hb][e] = c[hb][0][e] + c[hb][1][e];
}

// O^T += V^T P^T over the tile's 32 keys: 8 V^T fragments (two reads ahead), each
// feeding two 32x32x16 MFMAs (head blocks); fill(i) follows step i.
template <typename VA, typename Fill>
__device__ __forceinline__ void update_tile_q(DqState &st, const uint8_t MLA_LDS *t,
                                              const VA &va, const bf16x8 (&pt)[2][2],
                                              Fill fill) {
    bf16x8 v[2];
    v[0] = va.load(t, 0, 0);
    v[1] = va.load(t, 0, 1);
    static_for<8>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int cb = i >> 1, ks = i & 1;
        st.o[cb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[ks], pt[0][ks], st.o[cb][0], 0, 0, 0);
        st.o[cb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[ks], pt[1][ks], st.o[cb][1], 0, 0, 0);
        if constexpr (cb + 1 < 4) v[ks] = va.load(t, cb + 1, ks);
        fill(ic);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Softmax of one tile's scores s (keys key0 + kh*16 + (l >> 4)*4 + e; keys >= kend are
// masked) into weights, written to the weight buffer pb, in 8 pieces so that it can run
// between the MFMAs of the previous tile's O update: 0 masks, 1..4 take two weights
// each, 5 and 6 write a head block's weights and add its sum, 7 tests for overflow.
// init (between pieces 0 and 1, uniform: contains a workgroup barrier) sets the
// reference max from this tile; both key halves agree through the row pads at lds0.
struct SoftQ {
    DqState &st;
    f32x4 (&s)[2];
    uint8_t MLA_LDS *pb;
    int key0, kend;
    float sc;
    float p[2][4];
    float psum[2];

    __device__ __forceinline__ void init(uint8_t MLA_LDS *lds0) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        float mx[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float x = fmaxf(fmaxf(s[hb][0], s[hb][1]), fmaxf(s[hb][2], s[hb][3]));
            mx[hb] = quad_max(x);
            if (l < 16) ((float MLA_LDS *)(lds0 + dq::pad_off(1 + w * 2 + hb)))[l] = mx[hb];
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float other =
                ((const float MLA_LDS *)(lds0 + dq::pad_off(1 + (w ^ 1) * 2 + hb)))[l & 15];
            // both halves evaluate max(half 0, half 1) in the same order
            const float m = (w & 1) ? fmaxf(other, mx[hb]) : fmaxf(mx[hb], other);
            st.m[hb] = m * sc;  // sc > 0: the scaled max
        }
    }

    __device__ __forceinline__ void piece(int i) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4;
        const int kh = w & 1, hh = w >> 1;
        if (i == 0) {
            const int kb = key0 + kh * 16 + g * 4;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[hb][e] = (kb + e < kend) ? s[hb][e] : -INFINITY;
            psum[0] = psum[1] = 0.0f;
        } else if (i <= 4) {
            const int hb = (i - 1) >> 1, e0 = ((i - 1) & 1) * 2;
#pragma unroll
            for (int e = e0; e < e0 + 2; ++e) {
                p[hb][e] = __builtin_amdgcn_exp2f(fmaf(s[hb][e], sc, -st.m[hb]));
                psum[hb] += p[hb][e];
            }
        } else if (i <= 6) {
            const int hb = i - 5;
            st.lsum[hb] += psum[hb];
            const bf16x4 pv = {f2bf(p[hb][0]), f2bf(p[hb][1]), f2bf(p[hb][2]), f2bf(p[hb][3])};
            *(bf16x4 MLA_LDS *)(pb + pbuf_w_off(hh * 32 + hb * 16 + (l & 15), kh, g)) = pv;
        } else {
            // a weight above 2^FREEZE_LIMIT makes the sum exceed it: only then test exactly
            if (__builtin_amdgcn_ballot_w64(!(psum[0] <= 0x1p64f) || !(psum[1] <= 0x1p64f))) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const float tmax =
                        fmaxf(fmaxf(s[hb][0], s[hb][1]), fmaxf(s[hb][2], s[hb][3])) * sc;
                    if (tmax > st.m[hb] + fl::FREEZE_LIMIT) {
                        st.bad = true;
                        st.m[hb] = fmaxf(st.m[hb], tmax);  // track the true max for the repeat
                    }
                }
            }
        }
    }
};
static_assert(fl::FREEZE_LIMIT == 64.0f, "SoftQ compares sums against 2^64");

// The whole softmax of one tile at once (init as in SoftQ).
__device__ __forceinline__ void softmax_tile(DqState &st, f32x4 (&s)[2], int key0, int kend,
                                             float sc, bool init, uint8_t MLA_LDS *lds0,
                                             uint8_t MLA_LDS *pb) {
    SoftQ sq{st, s, pb, key0, kend, sc, {}, {}};
    sq.piece(0);
    if (init) sq.init(lds0);
#pragma unroll
    for (int i = 1; i < 8; ++i) sq.piece(i);
}

// Query staging layout: 16-byte chunk c (of 72) of head h (of 64) at slot
// (c/8)*512 + h*8 + ((c%8) ^ (h%8)): blocks of 8 chunks (128 contiguous bytes of a row) per
// head, so that one copy instruction moves 8 heads x 128 B (8 lanes per row: 8 cache lines
// instead of 64 for a chunk of 64 heads), and the fragment reads of 16 consecutive heads
// meet at most 2 per bank group.
__device__ __forceinline__ int qslot(int c, int h) {
    return (c >> 3) * 512 + h * 8 + ((c & 7) ^ (h & 7));
}
// Copies of the workgroup's 64 query rows into the staging area: instruction i (wave w
// issues 18w .. 18w+17) fills slots 64i .. 64i+63, i.e. heads 8(i%8) .. +7 of chunk block
// i/8; heads past H re-read head H-1 (their outputs are discarded).
__device__ __forceinline__ void issue_query_copies(const bf16 *__restrict__ qb, int hbase, int H,
                                                   uint8_t MLA_LDS *qs) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int i0 = 0; i0 < dq::QCOPY_PER; ++i0) {
        const int i = w * dq::QCOPY_PER + i0;
        const int h = (i & 7) * 8 + (l >> 3);
        const int c = (i >> 3) * 8 + ((l & 7) ^ (h & 7));
        const uint32_t off = (uint32_t)min(hbase + h, H - 1) * (uint32_t)fl::RB + (uint32_t)(c * 16);
        lds_copy16((const uint8_t *)qb, off, lds_u32(qs + i * 1024));
    }
}

// Query fragments from the staging area into registers (lane l: head hh*32 + hb*16 + (l&15),
// dims kk*32 + (l>>4)*8 .. +7, i.e. chunk kk*4 + (l>>4)).
__device__ __forceinline__ void read_query(DqState &st, const uint8_t MLA_LDS *qs) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int hh = w >> 1, g = l >> 4;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const int h = hh * 32 + hb * 16 + (l & 15);
#pragma unroll
        for (int kk = 0; kk < dq::KSTEPS; ++kk)
            st.q[hb][kk] = *(const bf16x8 MLA_LDS *)(qs + qslot(kk * 4 + g, h) * 16);
    }
}

// Waits until at most n (0, 1 or 2; uniform) groups of `per` copy instructions of this
// wave are outstanding.
template <int PER>
__device__ __forceinline__ void wait_groups(int n) {
    if (n >= 2) {
        MLA_WAIT_VMCNT(2 * PER);
    } else if (n == 1) {
        MLA_WAIT_VMCNT(PER);
    } else {
        MLA_WAIT_VMCNT(0);
    }
}

static_assert(Q8_X4_INST / dq::NW == 5 && q8_inst_per_wave<dq::NW>() == 20,
              "wait_vm_q8 enumerates sums of 5 and 20");

// One pass over keys [k0, k1) of `rows` (nk rows in the sequence); Q8: rows are Q8_0.
// bf16: the O update of tile t-1 (with the softmax of tile t between its MFMAs) follows
// the scores of tile t; one barrier per tile; two tiles in flight.  Q8_0: each tile's
// scores, the dequantisation of the next raw tile, the softmax, a barrier and the O
// update; three raw tiles in flight.  first: also load the query rows (staged through
// LDS) at the start.
template <bool Q8>
__device__ __forceinline__ void dq_stream(DqState &st, uint8_t MLA_LDS *lds,
                                          const uint8_t *__restrict__ rows, int nk, int k0,
                                          int k1, float sc, bool have_m, bool first,
                                          const bf16 *__restrict__ qb, int hbase, int H) {
    // bf16 tiles take the masks of 16-row fragment reads; Q8_0 tiles keep those of the
    // dequantisation's writes
    using Masks = std::conditional_t<Q8, TileMasks, TileMasks16>;
    uint8_t MLA_LDS *pbuf = lds + dq::stage_bytes(Q8);
    uint8_t MLA_LDS *qs = lds + dq::qstage_off(Q8);
    const int w = threadIdx.x >> 6;
    const KAddr<Masks> ka(w & 1);
    const VAddrQ<Masks> va(w);
    const int ntiles = (k1 - k0 + fl::NK - 1) / fl::NK;
    // Every earlier vector-memory load (the sequence length) must be complete before the
    // first copy: the compiler does not see the copies, and a load it still counted as
    // pending would bring a wait for all vector-memory operations into the tile loop.
    MLA_WAIT_VMCNT(0);
    if (first) issue_query_copies(qb, hbase, H, qs);
    if constexpr (!Q8) {
        const int last = nk - 1;
        // tiles 0 and 1 now (stages 2-3 hold the query rows until they are read)
        for (int i = 0; i < 2; ++i)
            if (i < ntiles)
                issue_tile_bf16<dq::NW, Masks>(rows, k0 + i * fl::NK, last, lds + i * fl::TILE_BYTES);
        if (first) {
            wait_groups<dq::COPY_PER>(min(2, ntiles));  // the query copies (issued first)
            __syncthreads();
            read_query(st, qs);
            __syncthreads();
        }
        // Iteration t: scores of tile t (with the copy of tile t+2 issued between the
        // MFMAs, into the stage tile t-2 used), then the O update of tile t-1 with the
        // softmax of tile t between its MFMAs.  Tiles t-1 .. t+2 resident or in flight.
        const int wu = __builtin_amdgcn_readfirstlane(w);
        for (int t = 0; t < ntiles; ++t) {
            wait_groups<dq::COPY_PER>(min(1, ntiles - 1 - t));
            __syncthreads();  // tile t landed; iteration t-1 done everywhere
            const int nx = t + 2;
            const bool more = nx < ntiles;
            const int nkey0 = k0 + nx * fl::NK;
            const bool full = nkey0 + fl::NK - 1 <= last;
            uint8_t MLA_LDS *ndst = lds + (nx % dq::NS_BF16) * fl::TILE_BYTES;
            if (more && !full) issue_tile_bf16<dq::NW, Masks>(rows, nkey0, last, ndst);  // the tail tile
            const uint8_t *sbase = rows + (int64_t)(nkey0 + 8 * wu) * fl::RB;
            const uint32_t dsts = lds_u32(ndst);
            const CopyPlan plan = make_copy_plan<Masks>();
            f32x4 s[2];
            // Copy parts 0..5 follow score steps 0, 3, .. 15 and parts 6..8 the O-update
            // steps 1, 3, 5: a copy instruction blocks its wave while the CU's address
            // unit is backed up, so the 36 instructions of a tile are spread over the
            // whole iteration.
            const bool fast = more && full;
            score_tile_q(st, lds + (t % dq::NS_BF16) * fl::TILE_BYTES, ka, s, [&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                if constexpr (kk % 3 == 0) {
                    if (fast) issue_part_full<kk / 3>(sbase, plan, dsts, wu);
                }
            });
            uint8_t MLA_LDS *pw = pbuf + (t & 1) * dq::PBUF;
            if (t == 0) {
                if (fast) {
                    issue_part_full<6>(sbase, plan, dsts, wu);
                    issue_part_full<7>(sbase, plan, dsts, wu);
                    issue_part_full<8>(sbase, plan, dsts, wu);
                }
                softmax_tile(st, s, k0, k1, sc, !have_m, lds, pw);
            } else {
                SoftQ sq{st, s, pw, k0 + t * fl::NK, k1, sc, {}, {}};
                bf16x8 pt[2][2];
                load_pt(pbuf + ((t - 1) & 1) * dq::PBUF, pt);
                update_tile_q(st, lds + ((t - 1) % dq::NS_BF16) * fl::TILE_BYTES, va, pt,
                              [&](auto ic) {
                                  constexpr int i = decltype(ic)::value;
                                  sq.piece(i);
                                  if constexpr ((i & 1) == 1 && i < 7) {
                                      if (fast) issue_part_full<6 + (i >> 1)>(sbase, plan, dsts, wu);
                                  }
                              });
            }
        }
        __syncthreads();
        {
            bf16x8 pt[2][2];
            load_pt(pbuf + ((ntiles - 1) & 1) * dq::PBUF, pt);
            update_tile_q(st, lds + ((ntiles - 1) % dq::NS_BF16) * fl::TILE_BYTES, va, pt,
                          [](auto) {});
        }
        __syncthreads();
    } else {
        // Raw tiles: 16-byte copies (5 per wave) for tiles inside the sequence, dword
        // copies clamped to the sequence's last byte (20 per wave) for the one tile that
        // reaches past it, which can only be the split's last tile.
        constexpr int PX = Q8_X4_INST / dq::NW, PD = q8_inst_per_wave<dq::NW>();
        const bool tail = k0 + ntiles * fl::NK > nk;
        auto cnt = [&](int j) { return (tail && j == ntiles - 1) ? PD : PX; };
        uint8_t MLA_LDS *raw = lds + 2 * fl::TILE_BYTES;
        auto issue_raw = [&](int j) {
            uint8_t MLA_LDS *dst = raw + (j % dq::NRAW) * Q8_RAW_STAGE;
            if (tail && j == ntiles - 1) {
                issue_tile_q8<dq::NW>(rows, k0 + j * fl::NK, nk, dst);
            } else {
                issue_tile_q8_full<dq::NW>(rows, k0 + j * fl::NK, dst);
            }
        };
        // waits until raw tile j has landed, given that tiles up to `issued` were issued
        auto wait_raw = [&](int j, int issued) {
            int n = 0;
            for (int i = j + 1; i <= issued; ++i) n += cnt(i);
            wait_vm_q8(n);
        };
        for (int i = 0; i < dq::NRAW; ++i)
            if (i < ntiles) issue_raw(i);
        wait_raw(0, min(dq::NRAW, ntiles) - 1);  // raw tile 0 and the query copies before it
        __syncthreads();
        if (first) {
            read_query(st, qs);
            __syncthreads();  // the query staging (bf16 stages) is free
        }
        DequantQ8{raw, lds, k0, nk}.all();
        for (int t = 0; t < ntiles; ++t) {
            // raw tile t+1 landed (raw tiles up to t+3 issued)
            if (t + 1 < ntiles) wait_raw(t + 1, min(t + 3, ntiles - 1));
            __syncthreads();  // bf16 tile t complete; tile t-1's O update done everywhere
            if (t + 4 < ntiles) issue_raw(t + 4);
            const uint8_t MLA_LDS *tile = lds + (t & 1) * fl::TILE_BYTES;
            // the dequantisation of raw tile t+1 runs between the score MFMAs of tile t:
            // task m is fetched after score step 2m and converted after step 2m+2
            const bool next = t + 1 < ntiles;
            const DequantQ8 dqz{raw + ((t + 1) % dq::NRAW) * Q8_RAW_STAGE,
                                lds + ((t + 1) & 1) * fl::TILE_BYTES, k0 + (t + 1) * fl::NK, nk};
            DequantQ8::Words dw[2];
            f32x4 s[2];
            score_tile_q(st, tile, ka, s, [&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                if constexpr ((kk & 1) == 0) {
                    constexpr int m = kk >> 1;
                    if (next) {
                        if constexpr (m >= 1) dqz.convert(m - 1, dw[(m - 1) & 1]);
                        if constexpr (m < DequantQ8::TASKS) dw[m & 1] = dqz.load(m);
                    }
                }
            });
            static_assert(2 * (DequantQ8::TASKS - 1) < dq::KSTEPS, "all fetches inside the score steps");
            if (next) dqz.convert(DequantQ8::TASKS - 1, dw[(DequantQ8::TASKS - 1) & 1]);
            softmax_tile(st, s, k0 + t * fl::NK, k1, sc, t == 0 && !have_m, lds, pbuf);
            __syncthreads();  // weights visible
            bf16x8 pt[2][2];
            load_pt(pbuf, pt);
            update_tile_q(st, tile, va, pt, [](auto) {});
        }
        __syncthreads();
    }
}

// Decode partials.  Blocks are dispatched round-robin over the 8 XCDs (block i on XCD
// i % 8); the head groups of one (sequence, split) get block indices on the same XCD so
// that they stream the same rows through one L2.  units = B * n_splits key ranges.
template <bool Q8>
__global__ __launch_bounds__(64 * dq::NW, 1) void flash_decode_kernel(
    const bf16 *__restrict__ q_cat, int H, const uint8_t *__restrict__ cache, int64_t seq_stride,
    const int32_t *__restrict__ n_kv, int n_kv_max, int n_splits, int split_len, int hgroups,
    int units, float sc, bf16 *__restrict__ part_o, float *__restrict__ part_lse) {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int hg = j % hgroups;
    const int u = (j / hgroups) * 8 + xcd;
    if (u >= units) return;  // padding block (uniform)
    const int b = u / n_splits, sp = u % n_splits;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    uint8_t MLA_LDS *lds = (uint8_t MLA_LDS *)lds_raw;
    int *flag = (int *)(lds_raw + dq::pad_off(0));

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int hh = w >> 1;
    const int hbase = hg * dq::HPB;
    DqState st;
    const int nk = min(n_kv[b], n_kv_max);  // rows past n_kv_max are never read
    const int k0 = sp * split_len;
    const int k1 = min(k0 + split_len, nk);
    const uint8_t *rows = cache + b * seq_stride;
    const bf16 *qb = q_cat + (int64_t)b * H * fl::W;

    float m0[2] = {-INFINITY, -INFINITY};
    bool have_m = false;
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
                for (int e = 0; e < 16; ++e) st.o[cb][hb2][e] = 0.0f;
        st.m[0] = m0[0];
        st.m[1] = m0[1];
        st.lsum[0] = st.lsum[1] = 0.0f;
        st.bad = false;
        if (k1 > k0) dq_stream<Q8>(st, lds, rows, nk, k0, k1, sc, have_m, pass == 0, qb, hbase, H);
        if (threadIdx.x == 0) *flag = 0;
        __syncthreads();
        if (__builtin_amdgcn_ballot_w64(st.bad) && l == 0) atomicOr(flag, 1);
        __syncthreads();
        const int again = *flag;
        if (!again) break;
        // repeat from the true maxima: max over the four lanes and both key halves
        float MLA_LDS *xm = (float MLA_LDS *)lds;  // stages are free after the stream
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float mx = quad_max(st.m[hb]);
            if (l < 16) xm[(w * 2 + hb) * 16 + l] = mx;
            m0[hb] = mx;
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float other = xm[((w ^ 1) * 2 + hb) * 16 + (l & 15)];
            m0[hb] = (w & 1) ? fmaxf(other, m0[hb]) : fmaxf(m0[hb], other);
        }
        have_m = true;
        __syncthreads();
    }

    // Denominators: the four lanes of a head, then both key halves (through LDS).
    float MLA_LDS *den = (float MLA_LDS *)(lds + 2 * fl::TILE_BYTES);  // past the staging area
    int l2 = l;
    asm volatile("" : "+v"(l2));  // recomputed here rather than kept across the stream
    const int kh = w & 1;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const float ls = quad_sum(st.lsum[hb]);
        if (l2 < 16) den[kh * 64 + hh * 32 + hb * 16 + l2] = ls;
    }
    __syncthreads();
    const int64_t pi = ((int64_t)b * n_splits + sp) * H;
    // lse of the QK-role heads (key-half-0 waves write)
    if (kh == 0 && l2 < 16) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int hd = hh * 32 + hb * 16 + l2;
            const float lt = den[hd] + den[64 + hd];
            if (hbase + hd < H)
                part_lse[pi + hbase + hd] = lt > 0.0f ? (st.m[hb] + __log2f(lt)) * fl::LN2 : -INFINITY;
        }
    }
    // Normalised bf16 rows staged in LDS, then written one 1 KB row per instruction.
    uint8_t MLA_LDS *stg = lds;
#pragma unroll
    for (int hb2 = 0; hb2 < 2; ++hb2) {
        const int hd = hb2 * 32 + (l2 & 31);
        const float lt = den[hd] + den[64 + hd];
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int col = w * 128 + cb * 32 + q4 * 8 + (l2 >> 5) * 4;
                const f32x16 &o = st.o[cb][hb2];
                const bf16x4 v = {f2bf(o[q4 * 4 + 0] * inv), f2bf(o[q4 * 4 + 1] * inv),
                                  f2bf(o[q4 * 4 + 2] * inv), f2bf(o[q4 * 4 + 3] * inv)};
                *(bf16x4 MLA_LDS *)(stg + hd * dq::OPITCH + col * 2) = v;
            }
    }
    __syncthreads();
    for (int r = 0; r < dq::HPB / dq::NW; ++r) {
        const int hd = w * (dq::HPB / dq::NW) + r;
        if (hbase + hd < H) {
            const uint8_t MLA_LDS *src = stg + hd * dq::OPITCH + l2 * 16;
            const u32x2 a = *(const u32x2 MLA_LDS *)src;
            const u32x2 c = *(const u32x2 MLA_LDS *)(src + 8);
            const u32x4 v = {a[0], a[1], c[0], c[1]};
            *(u32x4 *)(part_o + (pi + hbase + hd) * fl::R + l2 * 8) = v;
        }
    }
}
static_assert(dq::HPB * dq::OPITCH <= 2 * fl::TILE_BYTES, "staging below the denominators");

int decode_heads_per_block() { return dq::HPB; }

hipError_t launch_flash_decode_bf16(const bf16 *q_cat, const void *cache, int cache_q8,
                                    int64_t seq_stride_bytes, const int32_t *n_kv, int n_kv_max,
                                    int B, int H, int n_splits, int split_len, float scale,
                                    bf16 *part_o, float *part_lse, hipStream_t st) {
    const int hgroups = (H + dq::HPB - 1) / dq::HPB;
    const int units = B * n_splits;
    const int nblocks = (units + 7) / 8 * 8 * hgroups;
    const float sc = scale * fl::LOG2E;
    if (cache_q8) {
        const int shm = dq::lds_bytes(true);
        static std::atomic<uint64_t> lds_set{0};
        const hipError_t e = ensure_lds_limit((const void *)flash_decode_kernel<true>, shm, lds_set);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(flash_decode_kernel<true>, dim3(nblocks), dim3(64 * dq::NW), shm, st,
                           q_cat, H, (const uint8_t *)cache, seq_stride_bytes, n_kv, n_kv_max,
                           n_splits, split_len, hgroups, units, sc, part_o, part_lse);
    } else {
        const int shm = dq::lds_bytes(false);
        static std::atomic<uint64_t> lds_set{0};
        const hipError_t e = ensure_lds_limit((const void *)flash_decode_kernel<false>, shm, lds_set);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(flash_decode_kernel<false>, dim3(nblocks), dim3(64 * dq::NW), shm, st,
                           q_cat, H, (const uint8_t *)cache, seq_stride_bytes, n_kv, n_kv_max,
                           n_splits, split_len, hgroups, units, sc, part_o, part_lse);
    }
    return hipGetLastError();
}

}  // namespace mla
