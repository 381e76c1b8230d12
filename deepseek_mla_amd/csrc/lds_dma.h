// LDS-direct copies (global memory straight into LDS, gfx950 global_load_lds).
#pragma once

#include "common.h"

namespace mla {

// One LDS-direct copy instruction: lane l moves 16 bytes from sbase + voff (sbase uniform)
// to LDS address lds_addr + 16*l (lds_addr uniform, through M0).  Written as inline asm so
// that the compiler's LDS wait tracking does not see it: the compiler follows the builtin
// form with a wait for every outstanding LDS read, which would drain the read rings of the
// tile loop.  Completion is tracked by hand: a vmcnt wait and a barrier precede every read
// of a copied tile, and no other vector-memory instruction is issued in the tile loop.
__device__ __forceinline__ void lds_copy16(const uint8_t *sbase, uint32_t voff,
                                           uint32_t lds_addr) {
    const uint64_t a = (uint64_t)sbase;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint64_t su = ((uint64_t)hi << 32) | lo;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(su), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory", "m0");
}

// Dword form of lds_copy16: lane l moves 4 bytes from sbase + voff to lds_addr + 4*l.
__device__ __forceinline__ void lds_copy4(const uint8_t *sbase, uint32_t voff, uint32_t lds_addr) {
    const uint64_t a = (uint64_t)sbase;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint64_t su = ((uint64_t)hi << 32) | lo;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(su), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t MLA_LDS *p) {
    return (uint32_t)(uintptr_t)p;
}

}  // namespace mla
