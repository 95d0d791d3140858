// decode.hip -- the few-token GEMM of rollout decoding (FProp with at most 64
// token rows, e.g. 64 x 4096 against a fused gate+up weight of 24576 x 4096):
// the weight streams from HBM once and is the whole cost.
//
// Same products and the same per-output arithmetic as the block-scaled GEMM
// (gemm.hip): per 128-wide K block one v_mfma_f32_16x16x128_f8f6f4 whose A
// operand is 16 weight rows and whose B operand is 16 tokens, fed with the
// same lane layout (lane group g = lane/16 holds the 16-byte chunks g and g+4
// of a row's block), its four results added into the fp32 accumulators with
// one FMA each by fl32(s_x * s_w), in ascending K blocks; for MXFP8 one
// scaled MFMA per block accumulating in the matrix core.  So every output is
// bit for bit what the training-size kernel gives: rollout computes exactly
// the training forward's rows.
//
// Layout on the chip:
//   * 96 weight rows per block (6 waves of 16): 24576 rows are 256 blocks,
//     one per compute unit;
//   * each wave streams its 16 weight rows straight into registers (a ring
//     of RING K blocks, two 16-byte loads per lane per block);
//   * the weight comes either row-major (the quantizer's [D x C] codes) or
//     in the decode layout written by launch_pack_decode: per group of 16
//     rows and K block, the two 1 KB halves of the MFMA operand exactly as
//     the lanes hold them (lane l = 16q + r: row r, 16-byte chunks q and
//     q+4).  Row-major, one load covers 64 bytes of 16 rows 4 KB apart; in
//     the decode layout it covers 1 KB of consecutive bytes and a wave reads
//     its 16 rows as one linear 64 KB stream, which HBM serves markedly
//     faster (measured reading a 24576 x 4096 weight: 16 x 64-byte pieces
//     per load reach 4.5 TB/s, 1 KB runs 5.4 TB/s).  MX scale words are
//     packed the same way, 16 rows of a K block in one 64-byte run;
//   * the tokens' codes and scales go through LDS in chunks of 4 K blocks
//     (32 KB, three buffers), copied global->LDS two chunks ahead by a
//     seventh, producer wave with a wait counter of its own; the six weight
//     waves issue nothing but their ring's loads, which the compiler sees and
//     waits for exactly, and meet the producer at one barrier per chunk.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

constexpr int DEC_WAVES = 6;                  // weight waves, 16 weight rows each
constexpr int DEC_ROWS = 16 * DEC_WAVES;      // weight rows per block
constexpr int DEC_THREADS = 64 * (DEC_WAVES + 1);   // + the producer wave
constexpr int DEC_CHUNK = 4;                  // K blocks per token chunk
constexpr int DEC_NBUF = 3;                   // token chunk buffers
constexpr int DEC_CHUNK_OPS = 32 + DEC_CHUNK; // the producer's copies per chunk (codes, then scales)

typedef int dec_v4i __attribute__((ext_vector_type(4)));

// LDS barrier that does not wait for outstanding global loads (the weight
// ring stays in flight across it).
__device__ __forceinline__ void dec_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// global_load_lds_dword: 4 bytes per lane from gbase + voff to LDS at
// lds_wave + 4*lane (wave-uniform lds_wave and gbase).
__device__ __forceinline__ void dma4(uint32_t lds_wave, const void* gbase, uint32_t voff) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds_wave);
    const uint64_t gv = (uint64_t)(uintptr_t)gbase;
    const uint64_t gb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gv >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gv);
    uint32_t m0save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
                 "global_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(m0save) : "s"(la), "v"(voff), "s"(gb) : "memory");
}

template <int SM, bool PACKED, int RING>
__global__ __launch_bounds__(DEC_THREADS, 1) void k_gemm_rows96(GemmArgs g) {
    // token chunk: [buffer][K block][64 token rows x 128 bytes], chunks
    // XOR-swizzled as in the large-tile kernel; scale words [buffer][K block][token]
    __shared__ __attribute__((aligned(16))) uint8_t xs_codes[DEC_NBUF][DEC_CHUNK][64 * 128];
    __shared__ __attribute__((aligned(16))) uint32_t xs_scale[DEC_NBUF][DEC_CHUNK][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t KB = (g.K + 127) / 128;
    const int64_t NC = (KB + DEC_CHUNK - 1) / DEC_CHUNK;
    const int64_t M = g.M;

    if (wave == DEC_WAVES) {
        // ------------------------------------------------ producer wave
        // Instruction i < 32 of a chunk copies pieces q = 64*i + lane: K block
        // i / 8, token row 8*(i % 8) + lane / 8, physical chunk lane % 8
        // holding logical chunk (lane % 8) ^ (row & 7), to LDS byte 16*q of
        // the buffer; instruction 32 + kk copies the scale words of K block kk
        // (lane = token).  Token rows past M read row M-1 (computed, never
        // stored); K blocks past the end read the last block.
        uint32_t voff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 8 * i + (lane >> 3), lch = (lane & 7) ^ (row & 7);
            const int64_t r = row < M ? row : M - 1;
            voff[i] = (uint32_t)(r * g.ldp + lch * 16);
        }
        const int64_t tok = lane < M ? lane : M - 1;
        const uint32_t soff = (uint32_t)(SM == SCALE_MX ? tok * g.ldsp : tok * g.ldsp * 4);
        const uint32_t lds_codes = (uint32_t)(uintptr_t)&xs_codes[0][0][0];
        const uint32_t lds_scale = (uint32_t)(uintptr_t)&xs_scale[0][0][0];
        const char* sP = static_cast<const char*>(g.sP);
        auto copy_chunk = [&](int64_t c) {
            const int buf = (int)(c % DEC_NBUF);
#pragma unroll
            for (int kk = 0; kk < DEC_CHUNK; ++kk) {
                const int64_t k = c * DEC_CHUNK + kk < KB ? c * DEC_CHUNK + kk : KB - 1;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    dma16(lds_codes + (uint32_t)(buf * DEC_CHUNK * 8192 + kk * 8192 + i * 1024), g.P + k * 128,
                          voff[i]);
            }
#pragma unroll
            for (int kk = 0; kk < DEC_CHUNK; ++kk) {
                const int64_t k = c * DEC_CHUNK + kk < KB ? c * DEC_CHUNK + kk : KB - 1;
                dma4(lds_scale + (uint32_t)((buf * DEC_CHUNK + kk) * 256), sP + k * 4, soff);
            }
        };
        copy_chunk(0);
        if (NC > 1) copy_chunk(1);
        for (int64_t c = 0; c < NC; ++c) {
            // chunk c has landed (chunk c+1's copies may still be in flight)
            if (c + 1 < NC) __builtin_amdgcn_s_waitcnt(vmcnt_imm(DEC_CHUNK_OPS));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            dec_lds_barrier();
            // every weight wave has finished chunk c-1: its buffer takes c+2
            if (c + 2 < NC) copy_chunk(c + 2);
        }
        return;
    }

    // ------------------------------------------------ weight waves
    const int64_t j0 = (int64_t)blockIdx.x * DEC_ROWS + wave * 16;      // the wave's first weight row
    const int64_t jl = j0 + (lane & 15) < g.Nn ? j0 + (lane & 15) : g.Nn - 1;
    // a wave wholly past the last row (last block only) reads row Nn-1's
    // codes and scales; its outputs are never stored
    const int64_t jb = j0 < g.Nn ? j0 : g.Nn - 1;
    const int gq = lane >> 4, sh = 8 * gq;
    // decode layout: the wave's group of 16 rows (the last group for waves
    // past the end)
    const int64_t ngrp = (g.Nn + 15) / 16;
    const int64_t grp = j0 / 16 < ngrp ? j0 / 16 : ngrp - 1;
    const uint8_t* wrow = PACKED ? g.Q + grp * KB * 2048 + 16 * lane : g.Q + jl * g.ldq + 16 * gq;
    constexpr int64_t kStep = PACKED ? 2048 : 128, kHalf = PACKED ? 1024 : 64;
    auto load_w = [&](int64_t kb) __attribute__((always_inline)) {
        const int64_t k = kb < KB ? kb : KB - 1;                         // past the end: reload the last
        const dec_v4i x0 = *reinterpret_cast<const dec_v4i*>(wrow + k * kStep);
        const dec_v4i x1 = *reinterpret_cast<const dec_v4i*>(wrow + k * kStep + kHalf);
        return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    };
    // weight scale of K block kb: the 128x128 block of the wave's rows (one
    // value per wave), or the MX word of this lane's row.  Loaded with the
    // block's codes, into the same ring, so that waiting for it never waits
    // for newer weight loads.
    const char* sQ = static_cast<const char*>(g.sQ);
    auto w_scale = [&](int64_t kb) __attribute__((always_inline)) -> uint32_t {
        const int64_t k = kb < KB ? kb : KB - 1;
        if constexpr (SM == SCALE_MX && PACKED)
            return *reinterpret_cast<const uint32_t*>(sQ + ((grp * KB + k) * 16 + (lane & 15)) * 4);
        else if constexpr (SM == SCALE_MX) return *reinterpret_cast<const uint32_t*>(sQ + jl * g.sq_rs + k * 4);
        else return *reinterpret_cast<const uint32_t*>(sQ + ((jb / 128) * g.sq_rs + k * g.sq_ks) * 4);
    };

    static_assert(RING % DEC_CHUNK == 0, "a ring pass covers whole token chunks");
    v8i wr[RING];
    uint32_t swr[RING];
#pragma unroll
    for (int r = 0; r < RING; ++r) {
        wr[r] = load_w(r);
        swr[r] = w_scale(r);
    }
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    v4f prev[4];
    float sprev[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) { prev[t] = v4f{0.f, 0.f, 0.f, 0.f}; sprev[t] = 0.f; }
    const FragOff pfo = frag_off(lane & 15, lane);                      // token row lane%16 of a group

    // One K block: ring slot u = kb % RING (compile-time once unrolled).
    auto step = [&](int64_t kb, const int u) __attribute__((always_inline)) {
        const int64_t c = kb / DEC_CHUNK;
        const int kk = u % DEC_CHUNK;
        if (kk == 0) dec_lds_barrier();                                  // chunk c has landed
        const int buf = (int)(c % DEC_NBUF);
        const uint8_t* xb = xs_codes[buf][kk];
        const uint32_t* sb = xs_scale[buf][kk];
        v8i bf[4];
        uint32_t xw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf[t] = lds_frag(xb, pfo, t * 16 * 128);
            xw[t] = sb[t * 16 + (lane & 15)];
        }
        const uint32_t ww = swr[u];
        const v8i af = wr[u];
        if constexpr (SM == SCALE_MX) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf[t], acc[t], 0, 0, 0, (int)((ww >> sh) & 0xFFu), 0, (int)((xw[t] >> sh) & 0xFFu));
        } else {
            v4f cur[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                cur[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[t], v4f{0.f, 0.f, 0.f, 0.f},
                                                                          0, 0, 0, 0, 0, 0);
            // promotion of the previous K block (its results are ready),
            // then this block's combined scales
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] = __builtin_fmaf(prev[t][r], sprev[t], acc[t][r]);
            const float sw = __uint_as_float(ww);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float sx = __uint_as_float(xw[t]);
                sx *= sw;
                sprev[t] = sx;
                prev[t] = cur[t];
            }
        }
        wr[u] = load_w(kb + RING);
        swr[u] = w_scale(kb + RING);
        __builtin_amdgcn_sched_barrier(0);                                // keep the K blocks in order
    };
    // Whole ring groups with no branch, so the compiler's waits count the ring
    // exactly, then the last partial group.
    int64_t kb0 = 0;
    for (; kb0 + RING <= KB; kb0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) step(kb0 + u, u);
    }
    if (kb0 < KB) {
#pragma unroll
        for (int u = 0; u < RING; ++u)
            if (kb0 + u < KB) step(kb0 + u, u);                          // uniform
    }
    if constexpr (SM != SCALE_MX) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = __builtin_fmaf(prev[t][r], sprev[t], acc[t][r]);
    }

    // ------------------------------------------------ epilogue
    // lane holds outputs (token t*16 + lane%16, weight rows j0 + 4*(lane/16) + r)
    const int64_t jw = j0 + 4 * gq;
    char* O = static_cast<char*>(g.O);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t i = t * 16 + (lane & 15);
        if (i >= M) continue;
        const v4f r = acc[t];
        if (g.out_f32) {
            float* o = reinterpret_cast<float*>(O) + i * g.ldo + jw;
            if (jw + 3 < g.Nn) {
                *reinterpret_cast<float4*>(o) = make_float4(r[0], r[1], r[2], r[3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (jw + q < g.Nn) o[q] = r[q];
            }
        } else {
            uint16_t* o = reinterpret_cast<uint16_t*>(O) + i * g.ldo + jw;
            if (jw + 3 < g.Nn) {
                uint2 v;
                v.x = f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16);
                v.y = f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16);
                *reinterpret_cast<uint2*>(o) = v;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (jw + q < g.Nn) o[q] = (uint16_t)f32_to_bf16(r[q]);
            }
        }
    }
}

bool rows96_applies(const GemmArgs& a) {
    return a.M >= 1 && a.M <= 64 && a.K >= 1 && a.group_mode == GROUP_NONE && a.ksplit <= 1 && a.beta == 0 &&
           (a.scale_mode == SCALE_Q_BLOCK || a.scale_mode == SCALE_MX) &&
           (a.Nn + DEC_ROWS - 1) / DEC_ROWS >= 128;
}

// Weight ring depth: 4 K blocks per wave measured fastest on the decode
// workload (8 and 12 add bytes in flight that delay the token copies
// queued behind them).
constexpr int kDecRing = 4;

template <bool PACKED>
static hipError_t launch_rows96(const GemmArgs& a, hipStream_t st) {
    const int64_t blocks = (a.Nn + DEC_ROWS - 1) / DEC_ROWS;
    if (blocks == 0 || a.M == 0 || a.K == 0) return hipSuccess;
    if (a.M > 64 || blocks > 0x7FFFFFFF || a.beta != 0) return hipErrorInvalidValue;
    if (a.scale_mode == SCALE_MX)
        k_gemm_rows96<SCALE_MX, PACKED, kDecRing><<<dim3((unsigned)blocks), DEC_THREADS, 0, st>>>(a);
    else if (a.scale_mode == SCALE_Q_BLOCK)
        k_gemm_rows96<SCALE_Q_BLOCK, PACKED, kDecRing><<<dim3((unsigned)blocks), DEC_THREADS, 0, st>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemm_rows96(const GemmArgs& a, hipStream_t st) { return launch_rows96<false>(a, st); }
hipError_t launch_gemm_decode_packed(const GemmArgs& a, hipStream_t st) { return launch_rows96<true>(a, st); }

// ------------------------------------------------------------ decode layout
// 16-byte piece p of the packed codes: lane l = p % 64, half h = (p / 64) % 2,
// K block k = (p / 128) % KB, group grp = p / (128 KB); it holds row
// 16 grp + l % 16, bytes 128 k + 16 (l / 16 + 4 h) .. +16 of the row-major
// codes (zeros for rows past D).  Scale word w: row 16 grp + w % 16 of
// K block (w / 16) % KB, grp = w / (16 KB): the row's four E8M0 bytes of that
// K block (127 for rows past D).
__global__ __launch_bounds__(256) void k_pack_decode(const uint8_t* __restrict__ wq, int64_t ldwq,
                                                     const uint8_t* __restrict__ we, int64_t ldwe,
                                                     int64_t D, int64_t KB, int64_t ngrp,
                                                     uint8_t* __restrict__ wp, uint32_t* __restrict__ wep) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t pieces = ngrp * KB * 128;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pieces; p += stride) {
        const int l = (int)(p & 63), h = (int)((p >> 6) & 1);
        const int64_t k = (p >> 7) % KB, grp = (p >> 7) / KB;
        const int64_t row = grp * 16 + (l & 15);
        dec_v4i v = {0, 0, 0, 0};
        if (row < D) v = *reinterpret_cast<const dec_v4i*>(wq + row * ldwq + k * 128 + 16 * ((l >> 4) + 4 * h));
        *reinterpret_cast<dec_v4i*>(wp + p * 16) = v;
    }
    if (we == nullptr) return;
    const int64_t words = ngrp * KB * 16;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words; w += stride) {
        const int64_t k = (w >> 4) % KB, grp = (w >> 4) / KB;
        const int64_t row = grp * 16 + (w & 15);
        wep[w] = row < D ? *reinterpret_cast<const uint32_t*>(we + row * ldwe + k * 4) : 0x7F7F7F7Fu;
    }
}

hipError_t launch_pack_decode(const uint8_t* wq, int64_t ldwq, const uint8_t* we, int64_t ldwe,
                              int64_t D, int64_t KB, uint8_t* wp, uint32_t* wep, hipStream_t st) {
    const int64_t ngrp = (D + 15) / 16;
    const int64_t pieces = ngrp * KB * 128;
    if (pieces == 0) return hipSuccess;
    int64_t blocks = (pieces + 255) / 256;
    if (blocks > 4096) blocks = 4096;                    // grid-stride beyond
    k_pack_decode<<<dim3((unsigned)blocks), 256, 0, st>>>(wq, ldwq, we, ldwe, D, KB, ngrp, wp, wep);
    return hipGetLastError();
}

}  // namespace fp8blk
