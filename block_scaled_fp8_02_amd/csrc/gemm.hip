// gemm.hip -- block-scaled FP8 GEMM on gfx950 MFMA (FProp, DGrad, WGrad,
// their grouped MoE forms, and the MXFP8 variant).
//
// Every GEMM of the linear layer is cast as
//     O[i][j] = sum_kb  sP[i][kb] * sQ[j][kb] * sum_{k in kb} P[i][k] Q[j][k]
// with P (M x K) and Q (Nn x K) FP8 E4M3 codes, both contiguous along the
// contraction axis K and grouped in 128-wide K blocks (Jet-RL notes,
// section 4.2; the summary page's note that the GEMM kernels perform the
// rescaling by the group and block scales and accumulate in FP32):
//   FProp  P = X  (1x128 scales per row),  Q = W   (128x128 block scales)
//   DGrad  P = dY (1x128 along D),         Q = W^T (block scales transposed)
//   WGrad  P = dY^T, Q = X^T (both 1x128 along the token axis, per row)
//
// Mapping to CDNA4:
//   * one v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-wide K block,
//     so its fp32 result is the block's partial sum; it is promoted into
//     the fp32 accumulator with one FMA by the combined scale;
//   * the MFMA A operand is the Q tile and the B operand the P tile, so each
//     lane's four results share one P row (one token) and, for the
//     128x128-scaled weight, one Q block: the combined scale is a single
//     value per lane and P sub-tile;
//   * P and Q tiles of one K block go global -> LDS by direct DMA
//     (global_load_lds_dwordx4, no register staging), double-buffered with
//     one barrier per K block; the next block's DMA and scale loads are in
//     flight while the current one is multiplied.  16-byte chunks are
//     XOR-swizzled by row (the DMA lane picks the source chunk that belongs
//     in its LDS slot), so the MFMA fragment reads are conflict-free;
//   * blocks are renumbered so that the tiles resident on one XCD (one L2)
//     at a time form a compact patch of the output and share operands;
//   * the MX variant feeds the E8M0 block scales to the scaled MFMA and
//     accumulates across all K blocks in the matrix core.
//
// The reduction order of an output element is fixed: ascending K blocks,
// one MFMA per block, one FMA per block (one scaled MFMA per block for MX).
// It does not depend on the tile shape or on M, which makes row i of the
// output a function of row i of P alone (rollout and training forward
// agree bit for bit).
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// MFMA operand fragment of one row: lane group g = lane/16 takes the 16-byte
// chunks g and g+4 of the row's 128 K bytes, which is the K order of the
// 16x16x128 instruction (so the 32-wide MX scale blocks line up too).
__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int lane) {
    const int g = lane >> 4;
    const int sw = row & 7;
    const uint4 x0 = *reinterpret_cast<const uint4*>(base + row * 128 + ((g ^ sw) << 4));
    const uint4 x1 = *reinterpret_cast<const uint4*>(base + row * 128 + (((g + 4) ^ sw) << 4));
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

// Row tile `tile` of the grouped (MoE) row enumeration -> rows [i0, ihi) of expert e.
__device__ __forceinline__ void find_row_tile(const int32_t* off, int64_t E, int64_t tile, int64_t BI,
                                              int64_t& i0, int64_t& ihi, int64_t& e_out) {
    int64_t acc = 0;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t a = off[e], b = off[e + 1];
        const int64_t tiles = (b - a + BI - 1) / BI;
        if (tile < acc + tiles) {
            i0 = a + (tile - acc) * BI;
            ihi = i0 + BI < b ? i0 + BI : b;
            e_out = e;
            return;
        }
        acc += tiles;
    }
    i0 = 0; ihi = 0; e_out = -1;
}

// BI x BJ block tile, NW waves, wave tile (16*TI) x (16*TJ).
template <int BI, int BJ, int TI, int TJ, int NW, int SM>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm(GemmArgs g) {
    constexpr int NT = 64 * NW;
    constexpr int WI = 16 * TI, WJ = 16 * TJ;
    constexpr int NWI = BI / WI, NWJ = BJ / WJ;
    static_assert(NWI * NWJ == NW, "wave grid must cover the block tile");
    static_assert(SM != SCALE_Q_BLOCK || (128 % WJ == 0), "a wave's Q rows must sit in one 128-row block");
    constexpr int STAGE = (BI + BJ) * 128;
    constexpr int NCH = (BI + BJ) * 8 / NT;                 // 16-byte DMA chunks per thread per stage
    static_assert(NCH * NT == (BI + BJ) * 8, "DMA chunks must divide evenly");
    static_assert(BI + BJ <= NT, "one scale loader per tile row");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    // Per K block, one 32-bit scale word per tile row (P rows, then Q rows):
    // the fp32 group/block scale, or for MX the four E8M0 bytes of the row's
    // four 32-wide sub-blocks.
    __shared__ __attribute__((aligned(16))) uint32_t sscale[2][NT];
    __shared__ int64_t tinfo[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave % NWI, wj = wave / NWI;

    // ---------------------------------------------------- tile setup
    const uint8_t* Q = g.Q;
    const char* sQ = static_cast<const char*>(g.sQ);
    char* O = static_cast<char*>(g.O);
    const size_t sq_elem = SM == SCALE_MX ? 1 : 4;
    const size_t o_elem = g.out_f32 ? 4 : 2;
    const int64_t nbj = (g.Nn + BJ - 1) / BJ;
    int64_t i0, ihi, j0, kbase = 0, KB = (g.K + 127) / 128;
    if (g.group_mode == GROUP_ROWS) {
        if (tid == 0) {
            int64_t a, b, e;
            find_row_tile(g.offsets, g.E, blockIdx.y, BI, a, b, e);
            tinfo[0] = a; tinfo[1] = b; tinfo[2] = e;
        }
        __syncthreads();
        i0 = tinfo[0]; ihi = tinfo[1];
        const int64_t e = tinfo[2];
        if (e < 0) return;                                         // whole block
        j0 = (int64_t)blockIdx.x * BJ;
        Q += e * g.q_estride;
        sQ += e * g.sq_estride * sq_elem;
    } else {
        const int64_t nbi = (g.M + BI - 1) / BI;
        int64_t ti, tj;
        grouped_tile(xcd_remap(blockIdx.x, nbi * nbj), nbi, nbj, 4, ti, tj);
        i0 = ti * BI;
        ihi = i0 + BI < g.M ? i0 + BI : g.M;
        j0 = tj * BJ;
        if (g.group_mode == GROUP_K) {
            const int64_t e = blockIdx.y;
            if (tid == 0) {
                int64_t P = 0;
                for (int64_t x = 0; x < e; ++x) P += (g.offsets[x + 1] - g.offsets[x] + 127) / 128 * 128;
                tinfo[0] = P / 128;
                tinfo[1] = (g.offsets[e + 1] - g.offsets[e] + 127) / 128;
            }
            __syncthreads();
            kbase = tinfo[0];
            KB = tinfo[1];
            O += e * g.o_estride * o_elem;
        }
    }
    const int64_t jhi = j0 + BJ < g.Nn ? j0 + BJ : g.Nn;

    // ---------------------------------------------------- DMA addressing
    // Chunk q = c*NT + tid of a stage lands at LDS byte 16*q: tile row q/8,
    // physical chunk q%8, which holds logical chunk (q%8) ^ (row&7).  Rows
    // c < NCP are P rows, the rest Q rows.  Sources are a block-uniform base
    // (SGPRs) plus a 32-bit per-lane offset; rows past the matrix edge are
    // clamped to its last row (they are computed but never stored).
    constexpr int NCP = BI * 8 / NT;
    static_assert(NCP * NT == BI * 8, "P rows must fill whole DMA rounds");
    const uint8_t* pbase = g.P + i0 * g.ldp + kbase * 128;
    const uint8_t* qbase = Q + j0 * g.ldq + kbase * 128;
    uint32_t soff[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int q = c * NT + tid, row = q >> 3, lch = (q & 7) ^ (row & 7);
        if (c < NCP) {
            const int64_t r = row < ihi - i0 ? row : ihi - i0 - 1;
            soff[c] = (uint32_t)(r * g.ldp + lch * 16);
        } else {
            const int64_t r = row - BI < jhi - j0 ? row - BI : jhi - j0 - 1;
            soff[c] = (uint32_t)(r * g.ldq + lch * 16);
        }
    }

    // ---------------------------------------------------- scale loader
    // Thread t < BI+BJ fetches the scale word of tile row t for each K block
    // (the others fetch a valid word they never use, which keeps the K loop
    // free of branches).
    const char* sbase;
    int64_t sstep;                                                  // bytes per K block
    if (tid < BI) {
        int64_t r = i0 + tid;
        r = r < ihi ? r : ihi - 1;
        sbase = static_cast<const char*>(g.sP) + (r * g.ldsp + (SM == SCALE_MX ? kbase * 4 : kbase)) * sq_elem;
        sstep = 4;
    } else {
        int64_t r = j0 + (tid < BI + BJ ? tid - BI : 0);
        r = r < jhi ? r : jhi - 1;
        const int64_t rr = SM == SCALE_Q_BLOCK ? r / 128 : r;
        sbase = sQ + (rr * g.sq_rs + (SM == SCALE_MX ? kbase * 4 : kbase * g.sq_ks)) * sq_elem;
        sstep = SM == SCALE_MX ? 4 : 4 * g.sq_ks;
    }
    auto load_scale = [&](int64_t kb) -> uint32_t {
        return *reinterpret_cast<const uint32_t*>(sbase + kb * sstep);
    };

    // global_load_lds_dwordx4 writes lane l's 16 bytes to LDS at m0 + 16*l.
    // It is issued from inline assembly so that the compiler, which cannot
    // tell the stage being filled from the stage being read, does not stall
    // the fragment reads on it; completion is awaited explicitly before the
    // barrier that ends each K step.  The DMAs of the next stage are spread
    // over the first Q sub-tiles of the current one, so that they queue
    // behind the matrix work instead of stalling every wave at once.
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
#define FP8B_DMA_PART(kb_, buf_, c0_, c1_)                                                         \
    do {                                                                                            \
        _Pragma("unroll") for (int c = (c0_); c < (c1_); ++c) {                                     \
            const uint32_t la = __builtin_amdgcn_readfirstlane(                                     \
                lds_base + (uint32_t)((buf_) * STAGE + (c * NT + wave * 64) * 16));                 \
            const uint64_t gv = (uint64_t)(uintptr_t)((c < NCP ? pbase : qbase) + (kb_) * 128);    \
            /* readfirstlane returns int: widen through uint32_t, never sign-extend */               \
            const uint64_t gb =                                                                     \
                ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gv >> 32)) << 32) |  \
                (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gv);                   \
            uint32_t m0save;                                                                        \
            asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"                                \
                         "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"                       \
                         : "=&s"(m0save) : "s"(la), "v"(soff[c]), "s"(gb) : "memory");             \
        }                                                                                           \
    } while (0)
    constexpr int DMA_PER_STEP = (NCH + TJ - 1) / TJ > 2 ? (NCH + TJ - 1) / TJ : 2;

    v4f acc[TJ][TI];
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
        for (int b = 0; b < TI; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    if (KB > 0) {
        FP8B_DMA_PART(0, 0, 0, NCH);
        sscale[0][tid] = load_scale(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const int prow_l = wi * WI + (lane & 15);                        // tile row of this lane's first P fragment
    const int qrow_l = BI + wj * WJ;                                 // tile row of this wave's first Q row
    const int sh = 8 * (lane >> 4);
    for (int64_t kb = 0; kb < KB; ++kb) {
        const int buf = (int)(kb & 1);
        const int64_t kn = kb + 1 < KB ? kb + 1 : kb;             // the last block reloads itself into
                                                                   // the idle stage: no branch in the loop
        const uint32_t snext = load_scale(kn);
        const uint8_t* base = smem + buf * STAGE;
        const uint32_t* sc = sscale[buf];

        // P fragments and P-side scales for the whole K block; Q fragments
        // stream through a two-deep register pipeline (the next Q sub-tile's
        // LDS reads are in flight while the current one is multiplied).
        v8i bf[TI];
        float sp[TI];
        int eb[TI];
#pragma unroll
        for (int t = 0; t < TI; ++t) {
            bf[t] = lds_frag(base, prow_l + t * 16, lane);
            const uint32_t w = sc[prow_l + t * 16];
            sp[t] = __uint_as_float(w);
            eb[t] = (int)((w >> sh) & 0xFFu);
        }
        if constexpr (SM == SCALE_Q_BLOCK) {
            const float sq = __uint_as_float(sc[qrow_l]);
#pragma unroll
            for (int t = 0; t < TI; ++t) sp[t] *= sq;                 // combined scale per P sub-tile
        }
        v8i af = lds_frag(base, qrow_l + (lane & 15), lane);
        uint4 sqa = *reinterpret_cast<const uint4*>(&sc[qrow_l + 4 * (lane >> 4)]);
        uint32_t eaw = sc[qrow_l + (lane & 15)];
        if constexpr (SM == SCALE_MX) {
#pragma unroll
            for (int a = 0; a < TJ; ++a) {
                if (a * DMA_PER_STEP < NCH)
                    FP8B_DMA_PART(kn, buf ^ 1, a * DMA_PER_STEP,
                                  (a + 1) * DMA_PER_STEP < NCH ? (a + 1) * DMA_PER_STEP : NCH);
                v8i af_n = af;
                uint32_t eaw_n = eaw;
                if (a + 1 < TJ) {
                    const int qr = qrow_l + (a + 1) * 16;
                    af_n = lds_frag(base, qr + (lane & 15), lane);
                    eaw_n = sc[qr + (lane & 15)];
                }
#pragma unroll
                for (int b = 0; b < TI; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af, bf[b], acc[a][b], 0, 0, 0, (int)((eaw >> sh) & 0xFFu), 0, eb[b]);
                af = af_n;
                eaw = eaw_n;
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // Software pipeline: step a issues the MFMAs of Q sub-tile a and
            // the promotion FMAs of sub-tile a-1, whose results are ready.
            v4f prev[TI];
            uint4 sqa_prev = sqa;
#pragma unroll
            for (int a = 0; a <= TJ; ++a) {
                if (a * DMA_PER_STEP < NCH)
                    FP8B_DMA_PART(kn, buf ^ 1, a * DMA_PER_STEP,
                                  (a + 1) * DMA_PER_STEP < NCH ? (a + 1) * DMA_PER_STEP : NCH);
                v8i af_n = af;
                uint4 sqa_n = sqa;
                if (a + 1 < TJ) {
                    const int qr = qrow_l + (a + 1) * 16;
                    af_n = lds_frag(base, qr + (lane & 15), lane);
                    if constexpr (SM == SCALE_Q_ROW) sqa_n = *reinterpret_cast<const uint4*>(&sc[qr + 4 * (lane >> 4)]);
                }
                v4f cur[TI];
                if (a < TJ) {
#pragma unroll
                    for (int b = 0; b < TI; ++b)
                        cur[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af, bf[b], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                }
                if (a > 0) {
#pragma unroll
                    for (int b = 0; b < TI; ++b) {
                        if constexpr (SM == SCALE_Q_BLOCK) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[a - 1][b][r] = __builtin_fmaf(prev[b][r], sp[b], acc[a - 1][b][r]);
                        } else {
                            acc[a - 1][b][0] = __builtin_fmaf(prev[b][0], sp[b] * __uint_as_float(sqa_prev.x), acc[a - 1][b][0]);
                            acc[a - 1][b][1] = __builtin_fmaf(prev[b][1], sp[b] * __uint_as_float(sqa_prev.y), acc[a - 1][b][1]);
                            acc[a - 1][b][2] = __builtin_fmaf(prev[b][2], sp[b] * __uint_as_float(sqa_prev.z), acc[a - 1][b][2]);
                            acc[a - 1][b][3] = __builtin_fmaf(prev[b][3], sp[b] * __uint_as_float(sqa_prev.w), acc[a - 1][b][3]);
                        }
                    }
                }
                if (a < TJ) {
#pragma unroll
                    for (int b = 0; b < TI; ++b) prev[b] = cur[b];
                }
                sqa_prev = sqa;
                af = af_n;
                sqa = sqa_n;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        sscale[buf ^ 1][tid] = snext;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");           // next stage's DMA has landed
        __syncthreads();
    }
#undef FP8B_DMA_PART

    // ---------------------------------------------------- epilogue
    const int64_t jw = j0 + wj * WJ;
#pragma unroll
    for (int a = 0; a < TJ; ++a) {
        const int64_t j = jw + a * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int b = 0; b < TI; ++b) {
            const int64_t i = i0 + wi * WI + b * 16 + (lane & 15);
            if (i >= ihi) continue;
            const v4f r = acc[a][b];
            if (g.out_f32) {
                float* o = reinterpret_cast<float*>(O) + i * g.ldo + j;
                if (j + 3 < g.Nn) {
                    float4 v = make_float4(r[0], r[1], r[2], r[3]);
                    if (g.beta) {
                        const float4 old = *reinterpret_cast<const float4*>(o);
                        v.x += old.x; v.y += old.y; v.z += old.z; v.w += old.w;
                    }
                    *reinterpret_cast<float4*>(o) = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (j + q < g.Nn) o[q] = g.beta ? o[q] + r[q] : r[q];
                }
            } else {
                uint16_t* o = reinterpret_cast<uint16_t*>(O) + i * g.ldo + j;
                if (j + 3 < g.Nn) {
                    uint2 v;
                    v.x = f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16);
                    v.y = f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16);
                    *reinterpret_cast<uint2*>(o) = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (j + q < g.Nn) o[q] = (uint16_t)f32_to_bf16(r[q]);
                }
            }
        }
    }
}

template <int BI, int BJ, int TI, int TJ, int NW, int SM>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
    const int64_t nbj = (a.Nn + BJ - 1) / BJ;
    const int64_t nbi = (a.M + BI - 1) / BI;
    dim3 grid;
    if (a.group_mode == GROUP_ROWS) {
        const int64_t rt = nbi + a.E;                              // bound on the experts' row tiles
        if (nbj == 0 || rt == 0) return hipSuccess;
        if (nbj > 0x7FFFFFFF || rt > 65535) return hipErrorInvalidValue;
        grid = dim3((unsigned)nbj, (unsigned)rt, 1);
    } else {
        const int64_t tiles = nbi * nbj;
        const int64_t z = a.group_mode == GROUP_K ? a.E : 1;
        if (tiles == 0 || z == 0) return hipSuccess;
        if (tiles > 0x7FFFFFFF || z > 65535) return hipErrorInvalidValue;
        grid = dim3((unsigned)tiles, (unsigned)z, 1);
    }
    k_gemm<BI, BJ, TI, TJ, NW, SM><<<grid, 64 * NW, 0, st>>>(a);
    return hipGetLastError();
}

template <int SM>
static hipError_t launch_sm(const GemmArgs& a, hipStream_t st) {
    // Small-M (decode) problems take 64x64 tiles so the weight stream is
    // spread over many blocks; large problems take 256x256 tiles with eight
    // waves (two per SIMD).  The per-element arithmetic is the same in both.
    if (a.group_mode == GROUP_NONE && a.M <= 64)
        return launch_cfg<64, 64, 4, 1, 4, SM>(a, st);
    return launch_cfg<256, 256, 4, 8, 8, SM>(a, st);        // 8 waves of 64 x 128
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    switch (a.scale_mode) {
        case SCALE_Q_BLOCK: return launch_sm<SCALE_Q_BLOCK>(a, st);
        case SCALE_Q_ROW: return launch_sm<SCALE_Q_ROW>(a, st);
        case SCALE_MX: return launch_sm<SCALE_MX>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8blk
