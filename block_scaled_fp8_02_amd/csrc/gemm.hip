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
// In every launch without a K split (every FProp, every WGrad, DGrad with
// more than 64 rows or a short contraction) it does not depend on the tile
// shape or on M, which makes row i of the output a function of row i of P
// alone (rollout and training forward agree bit for bit).  A K-split launch
// (few-row DGrad) sums ascending K ranges, each reduced as above, in
// ascending order: a different but equally fixed order, chosen from
// (M, Nn, K) alone.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// Experts one GROUP_K block walks through at most.
constexpr int MAX_EPB = 64;

// BI x BJ block tile, NW waves, wave tile (16*TI) x (16*TJ), NS LDS stages,
// GM the grouping (a template argument, so that the dense and row-grouped
// instances carry none of the expert-boundary code of GROUP_K).
template <int BI, int BJ, int TI, int TJ, int NW, int SM, int NS, int GM, bool PST = false>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm(GemmArgs g) {
    constexpr int NT = 64 * NW;
    constexpr int WI = 16 * TI, WJ = 16 * TJ;
    constexpr int NWI = BI / WI, NWJ = BJ / WJ;
    static_assert(NWI * NWJ == NW, "wave grid must cover the block tile");
    static_assert(SM != SCALE_Q_BLOCK || (128 % WJ == 0), "a wave's Q rows must sit in one 128-row block");
    constexpr int STAGE = (BI + BJ) * 128;
    constexpr int NCH = (BI + BJ) * 8 / NT;                 // 16-byte DMA chunks per thread per stage
    static_assert(NCH * NT == (BI + BJ) * 8, "DMA chunks must divide evenly");
    constexpr int NSL = (BI + BJ + NT - 1) / NT;           // scale words per thread per stage
    static_assert(NS >= 2, "at least double buffering");
    // vector-memory operations a thread issues per stage: NCH chunks + NSL scale words;
    // at the end of a K step the NS-2 newest stages may still be in flight
    constexpr int INFLIGHT = (NS - 2) * (NCH + NSL);
    static_assert(INFLIGHT <= 63, "vmcnt holds at most 63");
    // PST: a block walks tiles blockIdx.x, blockIdx.x + gridDim.x, ... (one
    // block per compute unit; launched for contractions of a few K blocks,
    // whose tiles are mostly output write).  The last K step of a tile copies
    // the next tile's first K block into the idle stage and the finished tile
    // leaves through the other stage, so the next tile's loads are in flight
    // while this one's stores drain.  Per-output arithmetic and K order are
    // those of the one-tile launch.
    constexpr bool PERSIST = PST && GM == GROUP_NONE && BI == 256 && BJ == 256;
    // the bf16 output tile fits in the stage buffers for the staged epilogue
    constexpr bool STAGED_OUT = BI * BJ * 2 <= NS * STAGE;

    __shared__ __attribute__((aligned(16))) uint8_t smem[NS * STAGE];
    // Per K block, one 32-bit scale word per tile row (P rows, then Q rows):
    // the fp32 group/block scale, or for MX the four E8M0 bytes of the row's
    // four 32-wide sub-blocks.  Filled by DMA like the operand stages.
    __shared__ __attribute__((aligned(16))) uint32_t sscale[NS][NSL * NT];
    __shared__ int64_t tinfo[4];
    __shared__ int32_t ekb[MAX_EPB];                                // GROUP_K: K blocks of each expert

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
    const int64_t nbi = (g.M + BI - 1) / BI;                        // dense forms
    const int64_t ntiles = nbi * nbj;
    int64_t vt = blockIdx.x;                                        // PERSIST: current tile
    int64_t i0, ihi, j0, kbase = 0, KB = (g.K + 127) / 128;
    int64_t e_first = 0, e_end = 1;                                 // GROUP_K: the block's experts
    if (GM == GROUP_ROWS) {
        if (tid < 64) {                                            // wave 0 locates the row tile
            const SegPos sp = wave_find_tile(g.offsets, g.E, blockIdx.y, BI, SegPos{0, 0, 0});
            if (tid == 0) {
                const bool ok = sp.e < g.E;
                const int64_t a = ok ? g.offsets[sp.e] + (blockIdx.y - sp.first) * BI : 0;
                const int64_t b = ok ? g.offsets[sp.e + 1] : 0;
                tinfo[0] = a; tinfo[1] = a + BI < b ? a + BI : b; tinfo[2] = ok ? sp.e : -1;
            }
        }
        __syncthreads();
        i0 = uniform64(tinfo[0]); ihi = uniform64(tinfo[1]);
        const int64_t e = uniform64(tinfo[2]);
        if (e < 0) return;                                         // whole block
        j0 = (int64_t)blockIdx.x * BJ;
        Q += e * g.q_estride;
        sQ += e * g.sq_estride * sq_elem;
    } else {
        int64_t ti, tj;
        grouped_tile(xcd_remap(blockIdx.x, ntiles), nbi, nbj, 4, ti, tj);
        i0 = ti * BI;
        ihi = i0 + BI < g.M ? i0 + BI : g.M;
        j0 = tj * BJ;
        if (GM == GROUP_K) {
            // experts [e_first, e_end) in turn, for the same output tile: their
            // K ranges are consecutive in the padded token axis, so the K loop
            // runs through all of them and stores one output tile per expert
            e_first = (int64_t)blockIdx.y * g.epb;
            e_end = e_first + g.epb < g.E ? e_first + g.epb : g.E;
            if (tid < 64) {                                        // wave 0: padded start, K blocks
                int64_t P = 0;
                for (int64_t x0 = 0; x0 < e_first; x0 += 64) {
                    const int64_t x = x0 + lane;
                    int64_t np = x < e_first ? ((int64_t)g.offsets[x + 1] - g.offsets[x] + 127) / 128 : 0;
#pragma unroll
                    for (int d = 32; d >= 1; d >>= 1) np += __shfl_xor(np, d);
                    P += np;
                }
                const int64_t x = e_first + lane;
                int64_t kx = x < e_end ? ((int64_t)g.offsets[x + 1] - g.offsets[x] + 127) / 128 : 0;
                if (lane < MAX_EPB) ekb[lane] = (int32_t)kx;
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) kx += __shfl_xor(kx, d);
                if (tid == 0) {
                    tinfo[0] = P;                                  // in 128-row blocks
                    tinfo[1] = kx;
                }
            }
            __syncthreads();
            kbase = uniform64(tinfo[0]);
            KB = uniform64(tinfo[1]);
        }
        if (GM == GROUP_NONE && g.ksplit > 1) {
            // K split: block row y runs K blocks [y * kb_split, (y + 1) * kb_split)
            // (ascending) into its own fp32 slice of partial sums
            kbase = (int64_t)blockIdx.y * g.kb_split;
            KB = KB - kbase < g.kb_split ? KB - kbase : g.kb_split;
            O += (int64_t)blockIdx.y * g.o_estride * (int64_t)o_elem;
        }
    }
    int64_t jhi = j0 + BJ < g.Nn ? j0 + BJ : g.Nn;

    // ---------------------------------------------------- DMA addressing
    // Chunk q = c*NT + tid of a stage lands at LDS byte 16*q: tile row q/8,
    // physical chunk q%8, which holds logical chunk (q%8) ^ (row&7).  Rows
    // c < NCP are P rows, the rest Q rows.  Sources are a block-uniform base
    // (SGPRs) plus a 32-bit per-lane offset; rows past the matrix edge are
    // clamped to its last row (they are computed but never stored).
    constexpr int NCP = BI * 8 / NT;
    static_assert(NCP * NT == BI * 8, "P rows must fill whole DMA rounds");
    const uint8_t* pbase;
    const uint8_t* qbase;
    uint32_t soff[NCH];

    // ---------------------------------------------------- scale loader
    // Tile row t = s*NT + tid (s < NSL) has its scale word fetched by this
    // thread for each K block; t >= BI+BJ fetches a valid word that is never
    // used, so that every thread issues the same DMA sequence.  BI is a
    // multiple of 64, so a wave's rows are all P rows or all Q rows: the
    // address is a wave-uniform base (SGPRs) plus a small per-lane offset.
    const char* sbase[NSL];                                         // wave-uniform, at K block 0
    int64_t sstep[NSL];                                             // bytes per K block
    uint32_t soffs[NSL];                                            // per lane
    static_assert(BI % 64 == 0, "P and Q scale rows must not share a wave");
    // wave-uniform scale base of slot sl for the tile at (i0_, j0_)
    auto sbase_of = [&](int64_t i0_, int64_t j0_, int sl) -> const char* {
        if (sl * NT + wave * 64 < BI)                               // the wave holds P rows
            return static_cast<const char*>(g.sP) + (i0_ * g.ldsp + (SM == SCALE_MX ? kbase * 4 : kbase)) * sq_elem;
        const int64_t rr0 = SM == SCALE_Q_BLOCK ? j0_ / 128 : j0_;
        return sQ + (rr0 * g.sq_rs + (SM == SCALE_MX ? kbase * 4 : kbase * g.sq_ks)) * sq_elem;
    };
    // copy addresses of the current tile (i0, ihi, j0, jhi, kbase)
    auto set_addr = [&]() {
        // an opaque copy of the thread index keeps the compiler from hoisting
        // per-lane terms out of the tile loop (live across the K loop, they
        // would cost registers there)
        int tx = tid;
        asm volatile("" : "+v"(tx));
        pbase = g.P + i0 * g.ldp + kbase * 128;
        qbase = Q + j0 * g.ldq + kbase * 128;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int q = c * NT + tx, row = q >> 3, lch = (q & 7) ^ (row & 7);
            if (c < NCP) {
                const int64_t r = row < ihi - i0 ? row : ihi - i0 - 1;
                soff[c] = (uint32_t)(r * g.ldp + lch * 16);
            } else {
                const int64_t r = row - BI < jhi - j0 ? row - BI : jhi - j0 - 1;
                soff[c] = (uint32_t)(r * g.ldq + lch * 16);
            }
        }
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
            const int t = sl * NT + tx;
            sbase[sl] = sbase_of(i0, j0, sl);
            if (sl * NT + wave * 64 < BI) {
                int64_t r = i0 + t;
                r = r < ihi ? r : ihi - 1;
                soffs[sl] = (uint32_t)((r - i0) * g.ldsp * sq_elem);
                sstep[sl] = 4;
            } else {
                int64_t r = j0 + (t < BI + BJ ? t - BI : 0);
                r = r < jhi ? r : jhi - 1;
                const int64_t rr = SM == SCALE_Q_BLOCK ? r / 128 : r;
                const int64_t rr0 = SM == SCALE_Q_BLOCK ? j0 / 128 : j0;
                soffs[sl] = (uint32_t)((rr - rr0) * g.sq_rs * sq_elem);
                sstep[sl] = SM == SCALE_MX ? 4 : 4 * g.sq_ks;
            }
        }
    };
    set_addr();

    // global_load_lds_dwordx4 writes lane l's 16 bytes to LDS at m0 + 16*l
    // (global_load_lds_dword: 4 bytes at m0 + 4*l).  Both are issued from
    // inline assembly, so the compiler tracks no vector-memory loads in the
    // K loop and inserts no waits of its own: completion is awaited
    // explicitly (vmcnt) before the barrier that ends each K step, leaving
    // the NS-2 newer stages in flight.  The DMAs of a stage are spread over
    // the first Q sub-tiles of a step, so that they queue behind the matrix
    // work instead of stalling every wave at once.
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
    const uint32_t lds_scale = (uint32_t)(uintptr_t)&sscale[0][0];
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
#define FP8B_DMA_SCALE(kb_, buf_)                                                                   \
    do {                                                                                            \
        _Pragma("unroll") for (int sl = 0; sl < NSL; ++sl) {                                        \
            const uint32_t la = __builtin_amdgcn_readfirstlane(                                     \
                lds_scale + (uint32_t)(((buf_) * NSL * NT + sl * NT + wave * 64) * 4));             \
            const uint64_t gv = (uint64_t)(uintptr_t)(sbase[sl] + (kb_) * sstep[sl]);               \
            const uint64_t gb =                                                                     \
                ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gv >> 32)) << 32) |  \
                (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gv);                   \
            uint32_t m0save;                                                                        \
            asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"                                \
                         "global_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"                         \
                         : "=&s"(m0save) : "s"(la), "v"(soffs[sl]), "s"(gb) : "memory");           \
        }                                                                                           \
    } while (0)
    constexpr int DMA_PER_STEP = (NCH + TJ - 1) / TJ > 2 ? (NCH + TJ - 1) / TJ : 2;

    v4f acc[TJ][TI];
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
        for (int b = 0; b < TI; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    auto prologue = [&]() {
        if (KB > 0) {
            // stages 0 .. NS-2 hold K blocks 0 .. NS-2 (the last block repeated
            // where there are fewer): every thread issues the same sequence
#pragma unroll
            for (int st = 0; st < NS - 1; ++st) {
                const int64_t kk = st < KB ? st : KB - 1;
                FP8B_DMA_PART(kk, st, 0, NCH);
                FP8B_DMA_SCALE(kk, st);
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFLIGHT));
        }
        __syncthreads();
    };
    prologue();

    const int prow_l = wi * WI + (lane & 15);                        // tile row of this lane's first P fragment
    const int qrow_l = BI + wj * WJ;                                 // tile row of this wave's first Q row
    // Direct epilogue: lane stores its 4 consecutive outputs of one row.
    auto store_direct = [&](char* Ob) {
        const int64_t jw = j0 + wj * WJ;
        // an opaque copy of the lane index keeps the compiler from hoisting
        // these addresses out of the expert loop (they would stay live
        // across the K loop and push its registers into scratch)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
    for (int a = 0; a < TJ; ++a) {
        const int64_t j = jw + a * 16 + 4 * (ln >> 4);
#pragma unroll
        for (int b = 0; b < TI; ++b) {
            const int64_t i = i0 + wi * WI + b * 16 + (ln & 15);
            if (i >= ihi) continue;
            const v4f r = acc[a][b];
            if (g.out_f32) {
                float* o = reinterpret_cast<float*>(Ob) + i * g.ldo + j;
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
                uint16_t* o = reinterpret_cast<uint16_t*>(Ob) + i * g.ldo + j;
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
    };

    // Staged epilogue of output rows [r0, r0 + rh) (whole waves' rows) in
    // bf16: the waves holding them write their accumulators to LDS at stile
    // (rows stride BJ*2 bytes; 8-byte column chunks XOR-swizzled by
    // 2*(row % 16), so that 16 rows' writes hit distinct banks and 16-byte
    // pairs stay whole), then every thread sends whole rows out as
    // contiguous 16-byte stores.  Ends with a barrier: stile is free again.
    constexpr int CPR = BJ / 4;                                      // 8-byte chunks per tile row
    constexpr int PPR = CPR / 2;                                     // 16-byte pairs per tile row
    auto store_staged = [&](char* Ob, uint8_t* stile, int r0, int rh) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (wi * WI >= r0 && wi * WI < r0 + rh) {
#pragma unroll
            for (int a = 0; a < TJ; ++a) {
                const int jl = wj * WJ + a * 16 + 4 * (ln >> 4);
#pragma unroll
                for (int b = 0; b < TI; ++b) {
                    const int il = wi * WI + b * 16 + (ln & 15) - r0;
                    const v4f r = acc[a][b];
                    uint2 v;
                    v.x = f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16);
                    v.y = f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16);
                    const int ch = (jl >> 2) ^ ((2 * (il & 15)) & (CPR - 1) & ~1);
                    *reinterpret_cast<uint2*>(stile + (il * CPR + ch) * 8) = v;
                }
            }
        }
        __syncthreads();
        const bool full_cols = jhi - j0 == BJ && (g.ldo % 8) == 0;
        // Streaming stores: the output leaves L2 with the epilogue instead of
        // as dirty lines that later traffic must write back (measured: the
        // quantizers that follow a GEMM in the training step run 3-4 us
        // faster, the MoE WGrads 3-8%).  A dense tile of at most 4 K blocks
        // is all output write, and there the L2 absorbing one round's burst
        // while the next round computes wins (K = 64 WGrad: 67 against 70 us).
        const bool streaming = GM != GROUP_NONE || KB > 4;
        int t0 = tid;                                                // opaque, as ln above
        asm volatile("" : "+v"(t0));
        for (int q = t0; q < rh * PPR; q += NT) {
            const int il = q / PPR, pp = q % PPR;
            const int64_t i = i0 + r0 + il;
            if (i < ihi) {
                const int ch = (2 * pp) ^ ((2 * (il & 15)) & (CPR - 1) & ~1);
                const uint4 v = *reinterpret_cast<const uint4*>(stile + (il * CPR + ch) * 8);
                const int64_t j = j0 + 8 * pp;
                uint16_t* o = reinterpret_cast<uint16_t*>(Ob) + i * g.ldo + j;
                if (full_cols && streaming) {
                    __builtin_nontemporal_store(v.x, reinterpret_cast<uint32_t*>(o));
                    __builtin_nontemporal_store(v.y, reinterpret_cast<uint32_t*>(o) + 1);
                    __builtin_nontemporal_store(v.z, reinterpret_cast<uint32_t*>(o) + 2);
                    __builtin_nontemporal_store(v.w, reinterpret_cast<uint32_t*>(o) + 3);
                } else if (full_cols) {
                    *reinterpret_cast<uint4*>(o) = v;
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (j + e < g.Nn) o[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
        __syncthreads();
    };
    // rows of one staged piece that fit in a single stage (whole waves)
    constexpr int RH = (STAGE / (BJ * 2)) / WI * WI;
    constexpr bool STAGED_PIECES = RH >= WI && BI % (RH > 0 ? RH : 1) == 0;
    static_assert(!PERSIST || (NS == 2 && STAGED_PIECES), "the persistent epilogue uses one of two stages");

    const FragOff pfo = frag_off(prow_l, lane);                      // this lane's P fragment row
    const FragOff qfo = frag_off(qrow_l + (lane & 15), lane);        // and Q fragment row
    const int sh = 8 * (lane >> 4);
    int buf = 0;                                                     // stage of K block kb
    int nbuf = NS - 1;                                               // stage that receives block kb + NS - 1
    int64_t ecur = e_first;                                          // expert whose K blocks run (GROUP_K)
    for (;;) {                                                       // tiles: one pass unless PERSIST
    // PERSIST: the block's next tile, and whether its first K block is copied
    // during this tile's last K step (both tiles whole, so that the per-lane
    // copy offsets are the same; otherwise the next tile fills its pipeline
    // after the epilogue, as a fresh launch would)
    bool pf = false;
    const uint8_t* pbase_n = pbase;
    const uint8_t* qbase_n = qbase;
    const char* sbase_n[NSL];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) sbase_n[sl] = sbase[sl];
    if constexpr (PERSIST) {
        const int64_t vn = vt + (int64_t)gridDim.x;
        if (vn < ntiles) {
            int64_t ti, tj;
            grouped_tile(xcd_remap(vn, ntiles), nbi, nbj, 4, ti, tj);
            const int64_t i0n = ti * BI, j0n = tj * BJ;
            pf = KB > 0 && ihi - i0 == BI && jhi - j0 == BJ && i0n + BI <= g.M && j0n + BJ <= g.Nn;
            pbase_n = g.P + i0n * g.ldp;
            qbase_n = Q + j0n * g.ldq;
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) sbase_n[sl] = sbase_of(i0n, j0n, sl);
        }
    }
    // K block copied during step kb: kb + NS - 1, the last block again past
    // the end (an idle stage, no branch in the loop), or with pf the next
    // tile's block 0 in the last step
    auto next_copy = [&](int64_t kb_) -> int64_t {
        if (PERSIST && pf && kb_ == KB - 1) {
            pbase = pbase_n;
            qbase = qbase_n;
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) sbase[sl] = sbase_n[sl];
            return 0;
        }
        return kb_ + NS - 1 < KB ? kb_ + NS - 1 : KB - 1;
    };
    int64_t kend = GM == GROUP_K ? uniform64(ekb[0]) : KB;
    int64_t kb = 0;
    if constexpr (SM == SCALE_Q_ROW && GM != GROUP_K && TJ >= 2) {
        // Rotated K loop for per-row scales on both sides (WGrad), whose
        // promotion costs two VALU operations per output and K block: the
        // MFMAs of a block's last Q sub-tile are issued after the barrier
        // that ends the block, from fragments already in registers, so the
        // matrix cores have work while the next block's first LDS reads are
        // in flight.  At kb = 0 that tail runs on zero fragments and zero
        // scales and adds exactly +0.  The arithmetic per output is the same
        // as in the loop below (measured 3% faster at the WGrad training
        // shape; no faster for the 128x128-scaled GEMMs, which keep the
        // plain loop).
        v8i bf[TI], af = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        float sp[TI];
        v4f prev[TI];
#pragma unroll
        for (int t = 0; t < TI; ++t) {
            bf[t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            sp[t] = 0.f;
            prev[t] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        uint4 sqa = make_uint4(0, 0, 0, 0), sqa_prev = sqa;
        auto promote = [&](int a, const v4f* pv, const float* spb, uint4 sq) {
#pragma unroll
            for (int b = 0; b < TI; ++b) {
                acc[a][b][0] = __builtin_fmaf(pv[b][0], spb[b] * __uint_as_float(sq.x), acc[a][b][0]);
                acc[a][b][1] = __builtin_fmaf(pv[b][1], spb[b] * __uint_as_float(sq.y), acc[a][b][1]);
                acc[a][b][2] = __builtin_fmaf(pv[b][2], spb[b] * __uint_as_float(sq.z), acc[a][b][2]);
                acc[a][b][3] = __builtin_fmaf(pv[b][3], spb[b] * __uint_as_float(sq.w), acc[a][b][3]);
            }
        };
        for (; kb < KB; ++kb) {
            const int64_t kn = next_copy(kb);
            const uint8_t* base = smem + buf * STAGE;
            const uint32_t* sc = sscale[buf];
            FP8B_DMA_SCALE(kn, nbuf);
            // tail of block kb-1: its last Q sub-tile, and the promotion of
            // the sub-tile before
            v4f cur[TI];
#pragma unroll
            for (int b = 0; b < TI; ++b)
                cur[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b], v4f{0.f, 0.f, 0.f, 0.f},
                                                                          0, 0, 0, 0, 0, 0);
            promote(TJ - 2, prev, sp, sqa_prev);
            float sp_old[TI];
#pragma unroll
            for (int b = 0; b < TI; ++b) {
                prev[b] = cur[b];
                sp_old[b] = sp[b];
            }
            sqa_prev = sqa;
            __builtin_amdgcn_sched_barrier(0);
            // block kb: P fragments and scales, first Q fragment
#pragma unroll
            for (int t = 0; t < TI; ++t) {
                bf[t] = lds_frag(base, pfo, t * 16 * 128);
                sp[t] = __uint_as_float(sc[prow_l + t * 16]);
            }
            af = lds_frag(base, qfo, 0);
            sqa = *reinterpret_cast<const uint4*>(&sc[qrow_l + 4 * (lane >> 4)]);
            // Q sub-tiles 0 .. TJ-2; step a promotes sub-tile a-1 (step 0 the
            // last one of block kb-1, with that block's scales)
#pragma unroll
            for (int a = 0; a + 1 < TJ; ++a) {
                if (a * DMA_PER_STEP < NCH)
                    FP8B_DMA_PART(kn, nbuf, a * DMA_PER_STEP,
                                  (a + 1) * DMA_PER_STEP < NCH ? (a + 1) * DMA_PER_STEP : NCH);
                const v8i af_n = lds_frag(base, qfo, (a + 1) * 16 * 128);
                const uint4 sqa_n = *reinterpret_cast<const uint4*>(&sc[qrow_l + (a + 1) * 16 + 4 * (lane >> 4)]);
#pragma unroll
                for (int b = 0; b < TI; ++b)
                    cur[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b], v4f{0.f, 0.f, 0.f, 0.f},
                                                                              0, 0, 0, 0, 0, 0);
                if (a == 0) promote(TJ - 1, prev, sp_old, sqa_prev);
                else promote(a - 1, prev, sp, sqa_prev);
#pragma unroll
                for (int b = 0; b < TI; ++b) prev[b] = cur[b];
                sqa_prev = sqa;
                af = af_n;
                sqa = sqa_n;
                __builtin_amdgcn_sched_barrier(0);
            }
            if ((TJ - 1) * DMA_PER_STEP < NCH) FP8B_DMA_PART(kn, nbuf, (TJ - 1) * DMA_PER_STEP, NCH);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFLIGHT));        // block kb + 1 has landed
            __syncthreads();                                         // (and af is in registers)
            buf = buf + 1 == NS ? 0 : buf + 1;
            nbuf = nbuf + 1 == NS ? 0 : nbuf + 1;
        }
        // tail of the last block
        v4f cur[TI];
#pragma unroll
        for (int b = 0; b < TI; ++b)
            cur[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b], v4f{0.f, 0.f, 0.f, 0.f},
                                                                      0, 0, 0, 0, 0, 0);
        promote(TJ - 2, prev, sp, sqa_prev);
        promote(TJ - 1, cur, sp, sqa);
    } else
    for (;;) {
    for (; kb < kend; ++kb) {
        const int64_t kn = next_copy(kb);
        const uint8_t* base = smem + buf * STAGE;
        const uint32_t* sc = sscale[buf];
        FP8B_DMA_SCALE(kn, nbuf);

        // P fragments and P-side scales for the whole K block; Q fragments
        // stream through a two-deep register pipeline (the next Q sub-tile's
        // LDS reads are in flight while the current one is multiplied).
        v8i bf[TI];
        float sp[TI];
        int eb[TI];
#pragma unroll
        for (int t = 0; t < TI; ++t) {
            bf[t] = lds_frag(base, pfo, t * 16 * 128);
            const uint32_t w = sc[prow_l + t * 16];
            sp[t] = __uint_as_float(w);
            eb[t] = (int)((w >> sh) & 0xFFu);
        }
        if constexpr (SM == SCALE_Q_BLOCK) {
            const float sq = __uint_as_float(sc[qrow_l]);
#pragma unroll
            for (int t = 0; t < TI; ++t) sp[t] *= sq;                 // combined scale per P sub-tile
        }
        v8i af = lds_frag(base, qfo, 0);
        uint4 sqa = *reinterpret_cast<const uint4*>(&sc[qrow_l + 4 * (lane >> 4)]);
        uint32_t eaw = sc[qrow_l + (lane & 15)];
        if constexpr (SM == SCALE_MX) {
#pragma unroll
            for (int a = 0; a < TJ; ++a) {
                if (a * DMA_PER_STEP < NCH)
                    FP8B_DMA_PART(kn, nbuf, a * DMA_PER_STEP,
                                  (a + 1) * DMA_PER_STEP < NCH ? (a + 1) * DMA_PER_STEP : NCH);
                v8i af_n = af;
                uint32_t eaw_n = eaw;
                if (a + 1 < TJ) {
                    const int qr = qrow_l + (a + 1) * 16;
                    af_n = lds_frag(base, qfo, (a + 1) * 16 * 128);
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
            // a wave tile narrower than the DMA spread issues the rest here
            if (TJ * DMA_PER_STEP < NCH) FP8B_DMA_PART(kn, nbuf, TJ * DMA_PER_STEP, NCH);
        } else {
            // Software pipeline: step a issues the MFMAs of Q sub-tile a and
            // the promotion FMAs of sub-tile a-1, whose results are ready.
            // Per-row Q scales (WGrad): step a reads sub-tile a's four scale
            // words, used at step a + 1, so two such vectors are live at once.
            v4f prev[TI];
            uint4 sqa_prev = sqa;
#pragma unroll
            for (int a = 0; a <= TJ; ++a) {
                if (a * DMA_PER_STEP < NCH)
                    FP8B_DMA_PART(kn, nbuf, a * DMA_PER_STEP,
                                  (a + 1) * DMA_PER_STEP < NCH ? (a + 1) * DMA_PER_STEP : NCH);
                v8i af_n = af;
                uint4 sqa_n = sqa;
                if (a + 1 < TJ) af_n = lds_frag(base, qfo, (a + 1) * 16 * 128);
                if constexpr (SM == SCALE_Q_ROW) {
                    if (a < TJ) sqa_n = *reinterpret_cast<const uint4*>(&sc[qrow_l + a * 16 + 4 * (lane >> 4)]);
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
                if constexpr (SM == SCALE_Q_ROW) sqa_prev = sqa_n;  // sub-tile a's scales, used at step a + 1
                af = af_n;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFLIGHT));            // block kb + 1 has landed
        __syncthreads();
        buf = buf + 1 == NS ? 0 : buf + 1;
        nbuf = nbuf + 1 == NS ? 0 : nbuf + 1;
    }
    if (GM != GROUP_K || ecur + 1 >= e_end) break;
    // expert boundary: the next expert's first K block has landed in stage
    // buf and nothing is in flight, so stage nbuf is free: this expert's tile
    // leaves through it in pieces of RH rows (or by direct stores), then the
    // next expert starts
    if (STAGED_PIECES && !g.out_f32) {
        for (int r0 = 0; r0 < BI; r0 += RH) store_staged(O + ecur * g.o_estride * o_elem, smem + nbuf * STAGE, r0, RH);
    } else {
        store_direct(O + ecur * g.o_estride * o_elem);
    }
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
        for (int b = 0; b < TI; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
    ++ecur;
    kend += uniform64(ekb[ecur - e_first]);
    }
    // the tail's repeated DMAs target idle stages (with pf: the next tile's
    // first block, in stage buf); let them land before the stage memory is
    // reused or the block exits
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    // ---------------------------------------------------- epilogue
    if (GM == GROUP_K) O += ecur * g.o_estride * o_elem;
    if constexpr (PERSIST) {
        if (g.out_f32) {
            store_direct(O);
        } else if (pf) {                                           // stage nbuf is free, buf is taken
            for (int r0 = 0; r0 < BI; r0 += RH) store_staged(O, smem + nbuf * STAGE, r0, RH);
        } else {
            store_staged(O, smem, 0, BI);                          // every stage is free
        }
        vt += (int64_t)gridDim.x;
        if (vt >= ntiles) return;
        int64_t ti, tj;
        grouped_tile(xcd_remap(vt, ntiles), nbi, nbj, 4, ti, tj);
        i0 = ti * BI;
        ihi = i0 + BI < g.M ? i0 + BI : g.M;
        j0 = tj * BJ;
        jhi = j0 + BJ < g.Nn ? j0 + BJ : g.Nn;
        set_addr();
#pragma unroll
        for (int a = 0; a < TJ; ++a)
#pragma unroll
            for (int b = 0; b < TI; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
        if (!pf) {                                                  // fill the pipeline afresh
            prologue();
            buf = 0;
            nbuf = NS - 1;
        }
        continue;
    }
    if (STAGED_OUT && !g.out_f32) {
        store_staged(O, smem, 0, BI);                              // every stage is free now
        return;
    }
    store_direct(O);
    return;
    }
#undef FP8B_DMA_PART
#undef FP8B_DMA_SCALE
}

template <int BI, int BJ, int TI, int TJ, int NW, int SM, int NS, int GM, bool PST = false>
static hipError_t launch_cfg(const GemmArgs& args, hipStream_t st) {
    GemmArgs a = args;
    a.epb = 1;
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
        int64_t z = 1;
        if (a.group_mode == GROUP_K) {
            // several experts per block, sized so that about three blocks per
            // compute unit remain (each expert holds only a few K blocks)
            int64_t epb = tiles * a.E / (3 * (int64_t)device_cu_count());
            epb = epb < 1 ? 1 : (epb > MAX_EPB ? MAX_EPB : epb);
            if (NS != 2) epb = 1;     // the boundary store needs an idle stage and no DMA in flight
            a.epb = epb;
            z = (a.E + epb - 1) / epb;
        }
        if (a.group_mode == GROUP_NONE && a.ksplit > 1) z = a.ksplit;
        if (tiles == 0 || z == 0) return hipSuccess;
        if (tiles > 0x7FFFFFFF || z > 65535) return hipErrorInvalidValue;
        int64_t gx = tiles;
        if constexpr (PST) {
            // persistent: one block per compute unit, a multiple of the 8
            // XCDs, so that block b and every tile it takes stay on XCD b % 8
            static_assert(GM == GROUP_NONE && BI == 256 && BJ == 256, "persistent form of the dense tiles only");
            if (a.ksplit > 1) return hipErrorInvalidValue;
            const int64_t cus = (int64_t)device_cu_count() / 8 * 8;
            if (cus >= 8 && gx > cus) gx = cus;
        }
        grid = dim3((unsigned)gx, (unsigned)z, 1);
    }
    k_gemm<BI, BJ, TI, TJ, NW, SM, NS, GM, PST><<<grid, 64 * NW, 0, st>>>(a);
    return hipGetLastError();
}

template <int SM>
static hipError_t launch_sm(const GemmArgs& a, hipStream_t st) {
    // Few rows (decode, M <= 64): the weight stream dominates.  A weight of
    // at least 128 groups of 96 rows (block or MX scales, no accumulation)
    // streams through registers, 96 rows per block (decode.hip; 64x24576x4096
    // in 28 us against 29 us on the 128-row tiles below).  Otherwise 128-row
    // tiles (8 waves of 64x16, 4 stages) for the K-split DGrad and wide
    // weights: each block re-reads the 64-row activation from L2 once per 128
    // weight rows, and the L2 traffic that saves outweighs idle compute units
    // (64x24576x4096: 34 us against 38 us with 32-row tiles).  Smaller weights
    // keep narrow tiles (32 or 16 rows) to spread over at least one block per
    // compute unit, with 4 or 8 stages in flight.  The per-element arithmetic
    // is the same in every configuration.
    if (a.M <= 64 && a.group_mode == GROUP_NONE) {
        if (rows96_applies(a)) return launch_gemm_rows96(a, st);
        // K split into ranges (few-row DGrad, where the output has too few
        // tiles to occupy the chip): 128-row weight tiles as for a large weight
        if (a.ksplit > 1) return launch_cfg<64, 128, 4, 1, 8, SM, 4, GROUP_NONE>(a, st);
        if ((a.Nn + 127) / 128 >= 192) return launch_cfg<64, 128, 4, 1, 8, SM, 4, GROUP_NONE>(a, st);
        if ((a.Nn + 31) / 32 >= 512) return launch_cfg<64, 32, 4, 1, 2, SM, 4, GROUP_NONE>(a, st);
        return launch_cfg<64, 16, 2, 1, 2, SM, 8, GROUP_NONE>(a, st);
    }
    // 8 waves of 64 x 128.  Only the pairings the entry points use are
    // instantiated: row-grouped (MoE FProp, DGrad) with 128x128 weight
    // scales, K-grouped (MoE WGrad) with per-row scales on both sides.
    // Contractions of at most 4 K blocks (e.g. the rollout-batch WGrad, K =
    // 64) are mostly output write: their tiles run persistently, each
    // block's next tile loading while its last one's stores drain (K = 64
    // WGrad of 24576 x 4096 measured in the notes of this change).
    if (a.group_mode == GROUP_NONE) {
        if ((a.K + 127) / 128 <= 4) return launch_cfg<256, 256, 4, 8, 8, SM, 2, GROUP_NONE, true>(a, st);
        return launch_cfg<256, 256, 4, 8, 8, SM, 2, GROUP_NONE>(a, st);
    }
    if constexpr (SM == SCALE_Q_BLOCK) {
        if (a.group_mode == GROUP_ROWS) return launch_cfg<256, 256, 4, 8, 8, SM, 2, GROUP_ROWS>(a, st);
    }
    if constexpr (SM == SCALE_Q_ROW) {
        if (a.group_mode == GROUP_K) return launch_cfg<256, 256, 4, 8, 8, SM, 2, GROUP_K>(a, st);
    }
    return hipErrorInvalidValue;
}

// Sum of the K ranges' fp32 partial outputs, ascending in the range index:
// four consecutive outputs of one row per thread.
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int64_t S, int64_t slice,
                                                   int64_t ldp, int64_t M, int64_t Nn, void* __restrict__ out,
                                                   bool out_f32, int64_t ldo) {
    const int64_t n4 = (Nn + 3) / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * n4) return;
    const int64_t i = idx / n4, j = (idx - i * n4) * 4;
    const int nv = Nn - j < 4 ? (int)(Nn - j) : 4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int64_t s = 0; s < S; ++s) {                               // loads issued ahead, sums in order
        const float* p = part + s * slice + i * ldp + j;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (nv == 4) {                                              // ldp and slice are multiples of 4
            const float4 w = *reinterpret_cast<const float4*>(p);
            v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < nv) v[q] = p[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = s == 0 ? v[q] : acc[q] + v[q];
    }
    if (out_f32) {
        float* o = static_cast<float*>(out) + i * ldo + j;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nv) o[q] = acc[q];
    } else {
        uint16_t* o = static_cast<uint16_t*>(out) + i * ldo + j;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nv) o[q] = (uint16_t)f32_to_bf16(acc[q]);
    }
}

hipError_t launch_split_sum(const float* part, int64_t S, int64_t slice, int64_t ldp, int64_t M, int64_t Nn,
                            void* out, bool out_f32, int64_t ldo, hipStream_t st) {
    const int64_t items = M * ((Nn + 3) / 4);
    if (items == 0) return hipSuccess;
    const int64_t blocks = (items + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    k_split_sum<<<dim3((unsigned)blocks), 256, 0, st>>>(part, S, slice, ldp, M, Nn, out, out_f32, ldo);
    return hipGetLastError();
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
