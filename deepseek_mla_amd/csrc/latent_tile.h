// Latent-cache tile layout in LDS and the copies that fill it (gfx950), shared by the
// prefill and decode attention kernels.
//
// A cache row is [c_kv (512 bf16) | k_rope (64 bf16)] (1152 B), or its Q8_0 form of 18
// blocks {binary16 scale, int8 q[32]} (612 B).  A tile holds 32 consecutive rows.
//
// LDS tile layout (32 keys, 38912 B).  The latent part (512 bf16 = 64 chunks of 16 B per
// key) sits in rows of pitch 1088 B, logical chunk c at chunk c ^ mask_a(k); the rope part
// (64 bf16 = 8 chunks) follows in rows of 128 B, chunk c at c ^ mask_b(k).  One copy
// instruction then moves one whole latent row (uniform global address, lane-contiguous
// LDS), and both the 16-byte K-fragment reads of 32 rows at one chunk (the 32x32x16 A
// operand) and the transposing V reads of 4 consecutive rows are free of bank conflicts
// (see mask_a and mask_b).  Tiles read 16 rows at a time take other masks (TileMasks16).
#pragma once

#include "common.h"
#include "lds_dma.h"

#include <type_traits>
#include <utility>

namespace mla {
// Calls f(std::integral_constant<int, K>) for K = 0 .. N-1 (fully unrolled, K usable in
// constant expressions).
template <typename F, int... K>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, K...>) {
    (f(std::integral_constant<int, K>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

namespace fl {
constexpr int R = 512, DR = 64, W = 576;
constexpr int RB = W * 2;         // 1152 bytes per bf16 row
constexpr int WCH = W / 8;        // 72 chunks of 16 B per row
constexpr int NK = 32;            // keys per tile
constexpr int PA = 1088;                    // latent row pitch: 1024 B + 64 B pad
constexpr int A_BYTES = NK * PA;            // 34816 B
constexpr int PB = 128;                     // rope row pitch
constexpr int TILE_BYTES = A_BYTES + NK * PB;  // 38912 B
constexpr int Q8_RB = W / 32 * 34;          // 612 B per Q8_0 row
constexpr int Q8_TILE_BYTES = NK * Q8_RB;   // 19584 B, 16-B aligned for aligned tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float FREEZE_LIMIT = 64.0f;  // log2 units a score may exceed the frozen max by
}  // namespace fl

// LDS has 64 banks of 4 B, i.e. 16 groups of 16 B.  ds_read_b128 serves a wave in four
// passes of 16 lanes: the lanes with equal bit 5 and equal parity of bits 2..4 (lane 0
// with lanes 1-3, 12-15, 20-23 and 24-27), measured with the bank-conflict counter.
// Latent rows: the pitch of 1088 B moves row k by 4k groups and the mask XORs the low
// two chunk bits with (k >> 2) & 3, so
//  - a pass of the 32x32x16 K fragment read (rows = lanes 0..31 at one chunk, i.e. rows
//    k, k + 12, k + 20, k + 24 for k = 0..3 and the like) lands in 16 distinct groups:
//    4 * (k & 3) picks the high part, the mask (four different quads) the low part;
//  - a ds_read_b64_tr_b16 pass (32 consecutive lanes) reads 4 consecutive rows (one mask
//    value) x 4 chunks: the rows pick distinct high parts, the chunks distinct low parts.
__device__ __forceinline__ int mask_a(int k) { return (k >> 2) & 3; }
// Rope rows (128 B = half a bank row): even and odd rows take the two halves, and bits
// (k1, k2, k3) of the row index as bits (2, 1, 0) of the mask spread 8 even (odd) rows
// over the 8 groups of their half.
__device__ __forceinline__ int mask_b(int k) {
    return (((k >> 1) & 1) << 2) | (((k >> 2) & 1) << 1) | ((k >> 3) & 1);
}
// Byte offset of logical chunk c (0 .. 71) of key k in a tile.
__device__ __forceinline__ int tile_off(int k, int c) {
    return c < 64 ? k * fl::PA + ((c ^ mask_a(k)) * 16)
                  : fl::A_BYTES + k * fl::PB + (((c - 64) ^ mask_b(k)) * 16);
}

// Lanes l and l^32 hold the same query row; these combine the pair (ds_bpermute).
// Both halves compute (x[l % 32] op x[32 + l % 32]), so the results are bit-identical.
__device__ __forceinline__ float pair_max(float x) {
    const float y = __shfl_xor(x, 32);
    return (threadIdx.x & 32) ? fmaxf(y, x) : fmaxf(x, y);
}
__device__ __forceinline__ float pair_sum(float x) {
    const float y = __shfl_xor(x, 32);
    return (threadIdx.x & 32) ? y + x : x + y;
}

__device__ __forceinline__ bf16x8 tr_pair(const uint8_t MLA_LDS *p0, const uint8_t MLA_LDS *p1) {
    s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS *)p0);
    s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS *)p1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Async copy of one bf16 tile (32 keys from key0; keys past `last` re-read key `last`,
// they are masked out of the softmax) into LDS stage `dst`.  Part i (0 .. 8) of wave w:
// parts 0..7 copy the latent row 8w + i (one instruction, uniform source row), part 8
// copies the rope rows 8w .. 8w+7 (one instruction).
// The chunk masks of the tile layout above, as a policy for the copies and the fragment
// addressing.
struct TileMasks {
    __device__ __forceinline__ static int a(int k) { return mask_a(k); }
    __device__ __forceinline__ static int b(int k) { return mask_b(k); }
};
// Masks for tiles whose K fragments are read 16 rows at a time (v_mfma_f32_16x16x32_bf16:
// lane l reads row l & 15 at chunk 4kk + (l >> 4)).  Measured on gfx950 (an in-bounds probe
// of each access form under the bank-conflict counter): ds_read_b128 serves a wave in four
// passes of 16 lanes, lanes with equal bit 5 and equal parity of bits 2..4 together, and a
// pass is conflict-free when its lanes hit distinct 16-byte groups of a 256-byte bank row.
// A pass of the 16-row fragment read holds rows k, k + 12 at chunk c and rows k + 4, k + 8
// at chunk c ^ 1 (k = 0..3); with mask_a the second pair lands on the first pair's groups
// (two passes per group of lanes).  Here a(k) = -(k >> 2) mod 4 gives the four rows of each
// k & 3 four different groups, and b(k) = k & 6 spreads the even and the odd rope rows of
// a pass over eight chunks each.  Rows k and k + 16 keep equal masks, and the transposing
// V reads (32 lanes per pass, four consecutive rows at four chunks) stay conflict-free with
// any row mask.
struct TileMasks16 {
    __device__ __forceinline__ static int a(int k) { return (4 - ((k >> 2) & 3)) & 3; }
    __device__ __forceinline__ static int b(int k) { return k & 6; }
};
// cw: the copying wave's index among the four that share the tile (uniform); Masks: the
// layout's chunk masks.
template <typename Masks = TileMasks>
__device__ __forceinline__ void issue_chunk_bf16_cw(const uint8_t *__restrict__ rows, int key0,
                                                    int last, uint8_t MLA_LDS *dst, int i, int w) {
    const int l = threadIdx.x & 63;
    if (i < 8) {
        const int k = w * 8 + i;
        const uint8_t *src = rows + (int64_t)min(key0 + k, last) * fl::RB;
        lds_copy16(src, (uint32_t)((l ^ Masks::a(k)) * 16), lds_u32(dst + k * fl::PA));
    } else {
        // rows past `last` are clamped per lane; offsets stay below 32 rows
        const int k = w * 8 + (l >> 3);
        const int kr = min(k, last - key0);
        lds_copy16(rows + (int64_t)key0 * fl::RB,
                   (uint32_t)(kr * fl::RB + fl::R * 2 + (((l & 7) ^ Masks::b(k)) * 16)),
                   lds_u32(dst + fl::A_BYTES + w * 1024));
    }
}

// Copy plan of a full tile (all 32 keys inside the cache) for wave w: one uniform source
// address per tile (key0 + 8w) plus a compile-time row step per instruction, and lane
// offsets fixed for the whole stream.  Latent row 8w + i uses mask_a(8w + i) =
// (2w + i/4) & 3, so rows i < 4 and i >= 4 take two lane offsets.  The rope instruction
// covers rows 8w .. 8w+7.  (The instruction's immediate offset is left at 0: it would
// move the LDS destination as well.)
struct CopyPlan {
    uint32_t va0, va1, vb;
};
template <typename Masks = TileMasks>
__device__ __forceinline__ CopyPlan make_copy_plan() {
    const int w = threadIdx.x >> 6;
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));  // recomputed where used, not kept live across the loop
    CopyPlan c;
    c.va0 = (uint32_t)((l ^ Masks::a(8 * w)) * 16);
    c.va1 = (uint32_t)((l ^ Masks::a(8 * w + 4)) * 16);
    c.vb = (uint32_t)((l >> 3) * fl::RB + fl::R * 2 + (((l & 7) ^ Masks::b(8 * w + (l >> 3))) * 16));
    return c;
}

// Part I (0 .. 8) of a full tile's copy for this wave: sbase = rows + (key0 + 8w) * 1152
// (uniform), dst = the LDS stage.
template <int I>
__device__ __forceinline__ void issue_part_full(const uint8_t *sbase, const CopyPlan &c,
                                                uint32_t dst, int w) {
    if constexpr (I < 8) {
        lds_copy16(sbase + I * fl::RB, I < 4 ? c.va0 : c.va1,
                   dst + (uint32_t)((8 * w + I) * fl::PA));
    } else {
        lds_copy16(sbase, c.vb, dst + (uint32_t)(fl::A_BYTES + w * 1024));
    }
}

template <int NW, typename Masks = TileMasks>
__device__ __forceinline__ void issue_tile_bf16(const uint8_t *__restrict__ rows, int key0,
                                                int last, uint8_t MLA_LDS *dst) {
    static_assert(NW == 4, "one latent row per instruction: 8 rows and one rope part per wave");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < 9; ++i) issue_chunk_bf16_cw<Masks>(rows, key0, last, dst, i, w);
}

// Issue the async copy of the raw Q8_0 bytes of a 32-row tile into LDS, one dword per
// lane (612-byte rows are dword aligned, not 16-byte aligned).  Dwords past the
// sequence's last row re-read its final dword; the dequant pass zeroes those rows.
// 80 instructions of 64 dwords cover the 4896-dword tile; the stage holds 20480 B.
constexpr int Q8_RAW_DW = fl::Q8_TILE_BYTES / 4;      // 4896
constexpr int Q8_RAW_INST = (Q8_RAW_DW + 63) / 64 + 3; // 80 (rounded up to a multiple of 4)
constexpr int Q8_RAW_STAGE = Q8_RAW_INST * 256;        // 20480 B
static_assert(Q8_RAW_INST * 64 >= Q8_RAW_DW, "raw tile coverage");

template <int NW>
__device__ __forceinline__ void issue_tile_q8(const uint8_t *__restrict__ rows, int key0,
                                              int n_rows, uint8_t MLA_LDS *dst) {
    static_assert(Q8_RAW_INST % NW == 0, "raw copies must split evenly over waves");
    constexpr int NI = Q8_RAW_INST / NW;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= NW) return;  // only waves 0 .. NW-1 copy
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));  // recompute offsets per call (see issue_tile_bf16)
    // tile-relative dword index of the sequence's last dword (uniform, 32-bit)
    const int64_t rem = (int64_t)(n_rows - key0) * (fl::Q8_RB / 4) - 1;
    const int last_rel = (int)(rem < Q8_RAW_INST * 64 ? rem : Q8_RAW_INST * 64);
    const uint8_t *gbase = rows + (int64_t)key0 * fl::Q8_RB;
    // inline-asm copies (lds_copy4): the compiler's wait tracking does not see them, so
    // it inserts no waits for them; every read of a copied tile follows a vmcnt wait and
    // a workgroup barrier placed by hand
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int inst = w * NI + i;
        const uint32_t off = (uint32_t)min(inst * 64 + l, last_rel) * 4u;
        lds_copy4(gbase, off, lds_u32(dst + inst * 256));
    }
}

// Copy of a raw Q8_0 tile whose 32 rows all lie inside the sequence, in 16-byte pieces
// (the tile's 19584 bytes are 1224 pieces, 16-byte aligned when the sequence base is):
// 20 instructions, Q8_X4_INST / NW per wave; instruction i, lane l moves piece
// min(64 i + l, 1223) to the same offset of the stage (lanes past the tile repeat the
// last piece into the stage's spare bytes).
constexpr int Q8_X4_INST = 20;
static_assert(Q8_X4_INST * 1024 >= fl::Q8_TILE_BYTES && Q8_X4_INST * 1024 <= Q8_RAW_STAGE,
              "16-byte raw copies cover the tile and stay inside the stage");
template <int NW>
__device__ __forceinline__ void issue_tile_q8_full(const uint8_t *__restrict__ rows, int key0,
                                                   uint8_t MLA_LDS *dst) {
    static_assert(Q8_X4_INST % NW == 0, "raw copies must split evenly over waves");
    constexpr int NI = Q8_X4_INST / NW;
    constexpr int LAST = fl::Q8_TILE_BYTES / 16 - 1;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    const uint8_t *gbase = rows + (int64_t)key0 * fl::Q8_RB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int inst = w * NI + i;
        lds_copy16(gbase, (uint32_t)min(inst * 64 + l, LAST) * 16u, lds_u32(dst + inst * 1024));
    }
}
// The same copy one instruction at a time, with the per-lane offsets formed once for a
// whole stream: instruction i of wave w moves pieces 64 (w NI + i) .. +63.
template <int NW>
struct Q8CopyParts {
    static constexpr int NI = Q8_X4_INST / NW;
    uint32_t off[NI];  // source byte offsets inside the tile (clamped to its last piece)
    uint32_t dst0;     // LDS offset of the wave's first instruction inside a stage
    __device__ __forceinline__ Q8CopyParts() {
        static_assert(Q8_X4_INST % NW == 0, "raw copies must split evenly over waves");
        constexpr int LAST = fl::Q8_TILE_BYTES / 16 - 1;
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int l = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < NI; ++i) off[i] = (uint32_t)min((w * NI + i) * 64 + l, LAST) * 16u;
        dst0 = (uint32_t)(w * NI * 1024);
    }
    // instruction i of the copy of the tile at gbase (the global image of its first row)
    // into the stage at LDS offset stage
    __device__ __forceinline__ void issue(const uint8_t *gbase, uint32_t stage, int i) const {
        lds_copy16(gbase, off[i], stage + dst0 + (uint32_t)(i * 1024));
    }
};
static_assert(fl::Q8_TILE_BYTES % 16 == 0, "a tile is a whole number of 16-byte pieces");

// Number of async-copy instructions a wave issues per Q8_0 tile (for vmcnt waits).
template <int NW> __host__ __device__ constexpr int q8_inst_per_wave() {
    return Q8_RAW_INST / NW;
}

// Waits until at most n of this wave's copy instructions are outstanding, n a sum of up
// to three Q8_0 tile counts of a 4-wave workgroup (5 each for whole tiles, 20 for the one
// tile that reaches past the sequence end): 0, 5, 10, 15, 20, 25 or 30.
__device__ __forceinline__ void wait_vm_q8(int n) {
    switch (n) {
    case 0: MLA_WAIT_VMCNT(0); break;
    case 5: MLA_WAIT_VMCNT(5); break;
    case 10: MLA_WAIT_VMCNT(10); break;
    case 15: MLA_WAIT_VMCNT(15); break;
    case 20: MLA_WAIT_VMCNT(20); break;
    case 25: MLA_WAIT_VMCNT(25); break;
    default: MLA_WAIT_VMCNT(30); break;
    }
}

// Dequantisation of a raw Q8_0 tile (LDS, the global byte image) into the bf16 tile
// layout (LDS), in tasks of one 16-byte output chunk: 8 values of one 32-value block.
// Thread x of the 256-thread workgroup takes row k = x / 8 and chunks c = x % 8 + 8 i,
// i = 0 .. 8 (32 rows x 72 chunks = 2304 tasks, 9 per thread), so that every offset is a
// per-thread base plus a constant: the block of chunk c starts 68 i bytes after that of
// chunk x % 8 (two 34-byte blocks per 8 chunks), and latent chunks land 128 i bytes apart
// (the row mask only permutes the low two chunk bits).  load(i) fetches the task's scale
// and the 2-3 dwords holding its 8 codes; convert(i) forms the values and writes the
// chunk, so that the two can sit between other work.  Value = float(d) * q, exact in
// float32 (an 11-bit by 8-bit product), then rounded to bf16.  The code with its sign bit
// flipped is the unsigned byte u = q + 128; two of them at a time become the binary16
// values 1024 + u (the byte placed under the exponent bits 0x64), and one mixed-precision
// fma per value forms d (1024 + u) - 1152 d = d q: the product of two binary16 values is
// exact in float32 and the sum is exact because the result is representable.  Rows with
// key0 + k >= n_rows are written as zeros.
struct DequantQ8 {
    const uint8_t MLA_LDS *raw;
    uint8_t MLA_LDS *dst;
    int key0, n_rows;
    static constexpr int TASKS = 9;
    static_assert(fl::NK * (fl::W / 8) == TASKS * 256, "9 chunk tasks per thread");

    struct Words {
        uint32_t w0, w1, w2;
        uint16_t d;
    };
    // per-thread bases: raw offset of the scale of chunk x % 8's block, byte offset of the
    // codes inside their first dword (0 or 2), LDS offset of the first latent chunk
    __device__ __forceinline__ static int row() { return (int)(threadIdx.x >> 3); }
    __device__ __forceinline__ static int blk0() {
        const int x = (int)threadIdx.x;
        return (x >> 3) * fl::Q8_RB + ((x >> 2) & 1) * 34;
    }
    __device__ __forceinline__ Words load(int i) const {
        const int x = (int)threadIdx.x;
        const int blk = blk0() + 68 * i;
        const int o = blk + 2 + (x & 3) * 8;
        const int a0 = o & ~3;
        Words r;
        r.w0 = *(const uint32_t MLA_LDS *)(raw + a0);
        r.w1 = *(const uint32_t MLA_LDS *)(raw + a0 + 4);
        r.w2 = *(const uint32_t MLA_LDS *)(raw + a0 + 8);  // inside the stage's spare bytes at the end
        r.d = *(const uint16_t MLA_LDS *)(raw + blk);
        return r;
    }
    __device__ __forceinline__ void convert(int i, const Words &r) const {
        const int x = (int)threadIdx.x, k = row();
        const uint32_t sh = (uint32_t)((blk0() + 2 + (x & 3) * 8) & 3);  // same for every i
        const uint32_t lo = __builtin_amdgcn_alignbyte(r.w1, r.w0, sh) ^ 0x80808080u;
        const uint32_t hi = __builtin_amdgcn_alignbyte(r.w2, r.w1, sh) ^ 0x80808080u;
        const bool valid = key0 + k < n_rows;
        const _Float16 dh = valid ? __builtin_bit_cast(_Float16, r.d) : (_Float16)0.0f;
        const float c = -1152.0f * (float)dh;  // exact: 9 * 2^7 times an 11-bit value
        constexpr uint32_t EXP = 0x64646464u;  // binary16 exponent byte of 1024
        const uint32_t h[4] = {__builtin_amdgcn_perm(EXP, lo, 0x05010400u),
                               __builtin_amdgcn_perm(EXP, lo, 0x05030402u),
                               __builtin_amdgcn_perm(EXP, hi, 0x05010400u),
                               __builtin_amdgcn_perm(EXP, hi, 0x05030402u)};
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f16x2 x = __builtin_bit_cast(f16x2, h[e]);
            v[2 * e] = f2bf(fmaf((float)x[0], (float)dh, c));
            v[2 * e + 1] = f2bf(fmaf((float)x[1], (float)dh, c));
        }
        const int c0 = x & 7;
        const int off = i < 8 ? k * fl::PA + ((c0 ^ mask_a(k)) << 4) + 128 * i
                              : fl::A_BYTES + k * fl::PB + ((c0 ^ mask_b(k)) << 4);
        *(bf16x8 MLA_LDS *)(dst + off) = v;
    }
    __device__ __forceinline__ void all() const {
#pragma unroll
        for (int i = 0; i < TASKS; ++i) convert(i, load(i));
    }
};
static_assert(fl::Q8_TILE_BYTES + 8 <= Q8_RAW_STAGE, "the last task's third word stays in the stage");

// The same dequantisation (same tasks, same arithmetic) cut into pieces of a few
// instructions, for a loop that places one piece after each of its MFMAs: fetch (the
// task's four LDS reads), prep (align the 8 codes, flip their sign bits, the block scale),
// then half 0 and half 1 (four values each: byte placement, mixed-precision fmas, bf16
// rounding), and store.  The per-thread LDS addresses are formed once per tile, so every
// task reads and writes at constant offsets from them.  Each piece pins its inputs and
// outputs with empty asm statements so that the compiler keeps it where it is placed.
struct DequantQ8Pieces {
    const uint8_t MLA_LDS *rw;  // first code dword of task 0 (task i: + 68 i)
    const uint8_t MLA_LDS *rs;  // scale of task 0's block
    uint8_t MLA_LDS *wa;        // latent output chunk of task 0 (task i < 8: + 128 i)
    uint8_t MLA_LDS *wb;        // rope output chunk (task 8)
    uint32_t sh;                // byte offset of the codes in their first dword (0 or 2)
    bool valid;                 // the thread's row lies inside the sequence

    struct Mid {
        uint32_t lo, hi;  // codes 0..3 and 4..7 with the sign bit flipped (u = q + 128)
        _Float16 d;       // block scale (0 for rows past the sequence end)
        float c;          // -1152 d
    };

    __device__ __forceinline__ DequantQ8Pieces(const uint8_t MLA_LDS *raw, uint8_t MLA_LDS *dst,
                                               int key0, int n_rows) {
        const int x = (int)threadIdx.x, k = x >> 3, c0 = x & 7;
        const int blk = k * fl::Q8_RB + ((x >> 2) & 1) * 34;
        const int o = blk + 2 + (x & 3) * 8;
        rw = raw + (o & ~3);
        rs = raw + blk;
        sh = (uint32_t)(o & 3);
        wa = dst + k * fl::PA + ((c0 ^ mask_a(k)) << 4);
        wb = dst + fl::A_BYTES + k * fl::PB + ((c0 ^ mask_b(k)) << 4);
        valid = key0 + k < n_rows;
    }
    __device__ __forceinline__ void fetch(int i, DequantQ8::Words &r) const {
        r.w0 = *(const uint32_t MLA_LDS *)(rw + 68 * i);
        r.w1 = *(const uint32_t MLA_LDS *)(rw + 68 * i + 4);
        r.w2 = *(const uint32_t MLA_LDS *)(rw + 68 * i + 8);
        r.d = *(const uint16_t MLA_LDS *)(rs + 68 * i);
    }
    __device__ __forceinline__ void prep(DequantQ8::Words &r, Mid &m) const {
        asm volatile("" : "+v"(r.w0), "+v"(r.w1), "+v"(r.w2), "+v"(r.d));
        m.lo = __builtin_amdgcn_alignbyte(r.w1, r.w0, sh) ^ 0x80808080u;
        m.hi = __builtin_amdgcn_alignbyte(r.w2, r.w1, sh) ^ 0x80808080u;
        m.d = valid ? __builtin_bit_cast(_Float16, r.d) : (_Float16)0.0f;
        m.c = -1152.0f * (float)m.d;  // exact: 9 * 2^7 times an 11-bit value
        asm volatile("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.d), "+v"(m.c));
    }
    __device__ __forceinline__ void half(Mid &m, int hf, bf16x4 &v) const {
        asm volatile("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.d), "+v"(m.c));
        constexpr uint32_t EXP = 0x64646464u;  // binary16 exponent byte of 1024
        const uint32_t src = hf ? m.hi : m.lo;
        const uint32_t h[2] = {__builtin_amdgcn_perm(EXP, src, 0x05010400u),
                               __builtin_amdgcn_perm(EXP, src, 0x05030402u)};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const f16x2 x = __builtin_bit_cast(f16x2, h[e]);
            v[2 * e] = f2bf(fmaf((float)x[0], (float)m.d, m.c));
            v[2 * e + 1] = f2bf(fmaf((float)x[1], (float)m.d, m.c));
        }
        asm volatile("" : "+v"(v));
    }
    __device__ __forceinline__ void store(int i, bf16x4 a, bf16x4 b) const {
        const bf16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        if (i < 8)
            *(bf16x8 MLA_LDS *)(wa + 128 * i) = v;
        else
            *(bf16x8 MLA_LDS *)wb = v;
    }
};


// ------------------------------------------------- 16-row score and weight-buffer layouts
// Shared by the attention kernels whose waves score 16 query rows (or heads) at a time
// with v_mfma_f32_16x16x32_bf16 and exchange their weights through a [64 rows][32 keys]
// LDS buffer.

// Byte offsets (within a tile stage) of the K fragment of score step kk for this lane:
// key kh*16 + (l & 15), logical chunk kk*4 + (l >> 4).  Latent chunks (kk < 16) are
// stored at kk*4 + ((l >> 4) ^ mask_a(key)): one base plus kk*64.  Keys k and k + 16 have
// the same masks, so key half 1 is key half 0 moved by 16 rows (compile-time offsets).
template <typename Masks = TileMasks>
struct KAddr {
    uint32_t a, r0, r1;
    __device__ __forceinline__ KAddr(int kh) {
        const int l = threadIdx.x & 63, g = l >> 4;
        const int k = kh * 16 + (l & 15);
        a = (uint32_t)(k * fl::PA + ((g ^ Masks::a(k)) << 4));
        r0 = (uint32_t)(fl::A_BYTES + k * fl::PB + ((g ^ Masks::b(k)) << 4));
        r1 = (uint32_t)(fl::A_BYTES + k * fl::PB + (((4 + g) ^ Masks::b(k)) << 4));
    }
    __device__ __forceinline__ uint32_t at(int kk) const {
        return kk < 16 ? a + (uint32_t)(kk * 64) : (kk == 16 ? r0 : r1);
    }
};

// Byte offsets of the V^T fragments (A operand of 32x32x16: lane l holds column l & 31
// of a 32-column block and keys (l >> 5)*8 .. +7 of a 16-key step) over the 128 latent
// columns of quarter cq.  Two transposing reads of 4 keys each: in its 16-lane group G,
// lane 4r + c addresses key (G >> 1)*8 + 4s + r and columns (G & 1)*16 + 4c .. +3 of the
// block; lane i of the group receives column (G & 1)*16 + i of those 4 keys.  The row
// mask mask_a depends only on (G >> 1, s), so step (cb, ks) adds a compile-time offset.
template <typename Masks = TileMasks>
struct VAddrQ {
    uint32_t b[2];
    __device__ __forceinline__ explicit VAddrQ(int cq) {
        const int l = threadIdx.x & 63;
        const int G = l >> 4, i = l & 15, r = i >> 2, c = i & 3;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int krow = (G >> 1) * 8 + s * 4 + r;
            const int mk = Masks::a(krow);  // the same for the 4 rows (krow >> 2 fixed) and at krow + 16
            b[s] = (uint32_t)(krow * fl::PA + cq * 256 + ((((G & 1) * 2 + (c >> 1)) ^ mk) << 4) +
                              ((c & 1) << 3));
        }
    }
    // fragment of column block cb, key step ks
    __device__ __forceinline__ bf16x8 load(const uint8_t MLA_LDS *t, int cb, int ks) const {
        const int off = ks * 16 * fl::PA + cb * 64;
        return tr_pair(t + b[0] + off, t + b[1] + off);
    }
};

// Weight buffer [64 rows][32 keys] bf16, 64 B per row, 16-byte chunk c of row h stored
// at c ^ ((h >> 2) & 3): the P^T reads (16 consecutive rows at one chunk) and the
// 8-byte weight writes are conflict-free.  pbuf_w_off: the 4 weights of keys
// kh*16 + g*4 .. +3; pbuf_r_off: the 8 weights of keys ks*16 + half*8 .. +7.
__device__ __forceinline__ uint32_t pbuf_w_off(int hd, int kh, int g) {
    const int chunk = 2 * kh + (g >> 1);
    return (uint32_t)(hd * 64 + ((chunk ^ ((hd >> 2) & 3)) << 4) + ((g & 1) << 3));
}
__device__ __forceinline__ uint32_t pbuf_r_off(int hd, int ks, int half) {
    const int chunk = 2 * ks + half;
    return (uint32_t)(hd * 64 + ((chunk ^ ((hd >> 2) & 3)) << 4));
}

// Max over the four lanes (l & 15) + 16g that hold the same row; all four get the
// result of the same fixed-order combination.
__device__ __forceinline__ float quad_max(float x) {
    const float a = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(a, __shfl_xor(a, 32));
}
__device__ __forceinline__ float quad_sum(float x) {
    const int l = threadIdx.x & 63;
    const float y = __shfl_xor(x, 16);
    const float a = (l & 16) ? y + x : x + y;
    const float z = __shfl_xor(a, 32);
    return (l & 32) ? z + a : a + z;
}

}  // namespace mla
