// gemm_common.hpp -- pieces shared by the gfx950 GEMM kernels (the
// block-scaled FP8 GEMM and the bf16 GEMM of the dequantized backward):
// the LDS layout of an operand stage and its MFMA fragments, the tile order,
// and the direct global->LDS copy.
//
// A stage holds 128 bytes of the contraction axis for every tile row (128
// FP8 codes or 64 bf16 values), split into eight 16-byte chunks; chunk c of
// tile row r sits at byte r*128 + ((c ^ (r & 7)) << 4), so that the
// fragment reads of 16 rows hit distinct banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace fp8blk {

// MFMA operand fragment of one row: lane group g = lane/16 takes the 16-byte
// chunks g and g+4 of the row's 128 K bytes, which is the K order of the
// 16x16x128 instruction (so the 32-wide MX scale blocks line up too).  Chunk
// c of tile row r sits at byte r*128 + ((c ^ (r & 7)) << 4) of a stage.
// frag_off gives a lane's two byte offsets for its fragment row; rows 16
// apart share them up to r*128, so sub-tiles differ by constant offsets.
struct FragOff {
    uint32_t o0, o1;
};

__device__ __forceinline__ FragOff frag_off(int row, int lane) {
    const int g = lane >> 4, sw = row & 7;
    return FragOff{(uint32_t)(row * 128 + ((g ^ sw) << 4)), (uint32_t)(row * 128 + (((g + 4) ^ sw) << 4))};
}

// Fragment at `delta` bytes (a multiple of 16 rows) past the offsets' row.
__device__ __forceinline__ v8i lds_frag(const uint8_t* stage, FragOff f, int delta) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(stage + f.o0 + delta);
    const uint4 x1 = *reinterpret_cast<const uint4*>(stage + f.o1 + delta);
    v8i r;
    r[0] = (int)x0.x; r[1] = (int)x0.y; r[2] = (int)x0.z; r[3] = (int)x0.w;
    r[4] = (int)x1.x; r[5] = (int)x1.y; r[6] = (int)x1.z; r[7] = (int)x1.w;
    return r;
}

// Tile index -> (tile row, tile col) with groups of GM tile rows walked
// column by column, so consecutive indices form GM x k patches.
__device__ __forceinline__ void grouped_tile(int64_t t, int64_t nbi, int64_t nbj, int64_t GM,
                                             int64_t& ti, int64_t& tj) {
    const int64_t per_group = GM * nbj;
    const int64_t group = t / per_group;
    const int64_t first = group * GM;
    const int64_t rows = nbi - first < GM ? nbi - first : GM;
    const int64_t r = t - group * per_group;
    ti = first + r % rows;
    tj = r / rows;
}

// Consecutive block ids are dealt round-robin to the 8 XCDs; renumber so
// that each XCD works on a contiguous range of logical tiles.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t total) {
    if (total % 8 != 0) return b;
    return (b % 8) * (total / 8) + b / 8;
}

// A value the whole block agrees on (read from LDS after a barrier), moved
// to scalar registers so that addresses built from it stay scalar.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding and leaves the LDS/scalar and export counters alone.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Direct copy of 16 bytes per lane from global memory into LDS
// (global_load_lds_dwordx4): lane l's bytes at gbase + voff land at LDS byte
// lds_wave + 16*l.  lds_wave and gbase must be wave-uniform (they go to M0
// and an SGPR pair); issued from inline assembly, so the compiler tracks no
// vector-memory load and inserts no wait for it: the caller waits on vmcnt.
__device__ __forceinline__ void dma16(uint32_t lds_wave, const void* gbase, uint32_t voff) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds_wave);
    const uint64_t gv = (uint64_t)(uintptr_t)gbase;
    // readfirstlane returns int: widen through uint32_t, never sign-extend
    const uint64_t gb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gv >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gv);
    uint32_t m0save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
                 "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(m0save) : "s"(la), "v"(voff), "s"(gb) : "memory");
}

}  // namespace fp8blk
