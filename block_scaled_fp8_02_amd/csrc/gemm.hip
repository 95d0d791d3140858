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
//   * 128-row tiles of P and Q are staged through LDS, double-buffered with
//     one barrier per K block; 16-byte chunks are XOR-swizzled by row so
//     the MFMA fragment reads are conflict-free;
//   * the MX variant feeds the E8M0 block scales to the scaled MFMA and
//     accumulates across all K blocks in the matrix core.
//
// The reduction order of an output element is fixed: ascending K blocks,
// one MFMA per block, one FMA per block.  It does not depend on the tile
// shape or on M, which makes row i of the output a function of row i of P
// alone (rollout and training forward agree bit for bit).
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

struct TileInfo {
    int64_t i0, ihi;        // P/O rows [i0, ihi) of this tile (ihi clipped to the segment)
    int64_t kbase, KB;      // first K block and number of K blocks
    int64_t e;              // expert (grouped modes), else 0
};

__device__ __forceinline__ void find_row_tile(const int32_t* off, int64_t E, int64_t tile, int64_t BI,
                                              TileInfo& ti) {
    int64_t acc = 0;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t a = off[e], b = off[e + 1];
        const int64_t tiles = (b - a + BI - 1) / BI;
        if (tile < acc + tiles) {
            ti.i0 = a + (tile - acc) * BI;
            ti.ihi = ti.i0 + BI < b ? ti.i0 + BI : b;
            ti.e = e;
            return;
        }
        acc += tiles;
    }
    ti.i0 = 0; ti.ihi = 0; ti.e = -1;
}

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

// BI x BJ block tile, 4 waves, wave tile (16*TI) x (16*TJ).
template <int BI, int BJ, int TI, int TJ, int SM>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g) {
    constexpr int WI = 16 * TI, WJ = 16 * TJ;
    constexpr int NWI = BI / WI, NWJ = BJ / WJ;
    static_assert(NWI * NWJ == 4, "four waves per block");
    static_assert(SM != SCALE_Q_BLOCK || (128 % WJ == 0), "a wave's Q rows must sit in one 128-row block");
    constexpr int PCH = BI * 8 / 256, QCH = BJ * 8 / 256;   // 16-byte chunks per thread per K block
    static_assert(PCH >= 1 && QCH >= 1, "tile too small for 256 loaders");
    constexpr int STAGE = (BI + BJ) * 128;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ int64_t tinfo[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave % NWI, wj = wave / NWI;

    // ---------------------------------------------------- tile setup
    TileInfo ti;
    const uint8_t* Q = g.Q;
    const char* sQ = static_cast<const char*>(g.sQ);
    char* O = static_cast<char*>(g.O);
    const int64_t j0 = (int64_t)blockIdx.x * BJ;
    const int64_t KBall = (g.K + 127) / 128;
    const size_t sq_elem = SM == SCALE_MX ? 1 : 4;
    const size_t o_elem = g.out_f32 ? 4 : 2;
    if (g.group_mode == GROUP_ROWS) {
        if (tid == 0) {
            TileInfo t0;
            find_row_tile(g.offsets, g.E, blockIdx.y, BI, t0);
            tinfo[0] = t0.i0; tinfo[1] = t0.ihi; tinfo[2] = t0.e;
        }
        __syncthreads();
        ti.i0 = tinfo[0]; ti.ihi = tinfo[1]; ti.e = tinfo[2];
        if (ti.e < 0) return;                                        // whole block
        ti.kbase = 0; ti.KB = KBall;
        Q += ti.e * g.q_estride;
        sQ += ti.e * g.sq_estride * sq_elem;
    } else if (g.group_mode == GROUP_K) {
        if (tid == 0) {
            int64_t P = 0;
            for (int64_t e = 0; e < (int64_t)blockIdx.z; ++e)
                P += (g.offsets[e + 1] - g.offsets[e] + 127) / 128 * 128;
            tinfo[0] = P / 128;
            tinfo[1] = (g.offsets[blockIdx.z + 1] - g.offsets[blockIdx.z] + 127) / 128;
        }
        __syncthreads();
        ti.kbase = tinfo[0]; ti.KB = tinfo[1];
        ti.i0 = (int64_t)blockIdx.y * BI;
        ti.ihi = ti.i0 + BI < g.M ? ti.i0 + BI : g.M;
        ti.e = blockIdx.z;
        O += ti.e * g.o_estride * o_elem;
    } else {
        ti.i0 = (int64_t)blockIdx.y * BI;
        ti.ihi = ti.i0 + BI < g.M ? ti.i0 + BI : g.M;
        ti.kbase = 0; ti.KB = KBall; ti.e = 0;
    }
    const int64_t jhi = j0 + BJ < g.Nn ? j0 + BJ : g.Nn;

    // ---------------------------------------------------- global -> LDS staging
    uint4 rp[PCH], rq[QCH];
    const uint8_t* gp[PCH];
    const uint8_t* gq[QCH];
#pragma unroll
    for (int c = 0; c < PCH; ++c) {
        const int idx = tid + 256 * c, row = idx >> 3, ch = idx & 7;
        int64_t r = ti.i0 + row;
        r = r < ti.ihi ? r : ti.ihi - 1;                            // clamp: rows past the edge are never stored
        gp[c] = g.P + r * g.ldp + ti.kbase * 128 + ch * 16;
    }
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
        const int idx = tid + 256 * c, row = idx >> 3, ch = idx & 7;
        int64_t r = j0 + row;
        r = r < jhi ? r : jhi - 1;
        gq[c] = Q + r * g.ldq + ti.kbase * 128 + ch * 16;
    }
    // ---------------------------------------------------- scale addressing
    // P rows of this lane's B fragments, Q rows of its A fragments.
    int64_t prow[TI];
#pragma unroll
    for (int t = 0; t < TI; ++t) {
        int64_t r = ti.i0 + wi * WI + t * 16 + (lane & 15);
        prow[t] = r < ti.ihi ? r : ti.ihi - 1;
    }
    const int64_t jw = j0 + wj * WJ;                               // first Q row of this wave

    v4f acc[TJ][TI];
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
        for (int b = 0; b < TI; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

#define FP8B_GLOAD(kb_)                                                                    \
    do {                                                                                   \
        _Pragma("unroll") for (int c = 0; c < PCH; ++c)                                    \
            rp[c] = *reinterpret_cast<const uint4*>(gp[c] + (kb_) * 128);                  \
        _Pragma("unroll") for (int c = 0; c < QCH; ++c)                                    \
            rq[c] = *reinterpret_cast<const uint4*>(gq[c] + (kb_) * 128);                  \
    } while (0)
#define FP8B_SSTORE(buf_)                                                                  \
    do {                                                                                   \
        uint8_t* sb_ = smem + (buf_) * STAGE;                                              \
        _Pragma("unroll") for (int c = 0; c < PCH; ++c) {                                  \
            const int idx = tid + 256 * c, row = idx >> 3, ch = idx & 7;                   \
            *reinterpret_cast<uint4*>(sb_ + row * 128 + ((ch ^ (row & 7)) << 4)) = rp[c];  \
        }                                                                                  \
        _Pragma("unroll") for (int c = 0; c < QCH; ++c) {                                  \
            const int idx = tid + 256 * c, row = BI + (idx >> 3), ch = idx & 7;            \
            *reinterpret_cast<uint4*>(sb_ + row * 128 + ((ch ^ (row & 7)) << 4)) = rq[c];  \
        }                                                                                  \
    } while (0)

    if (ti.KB > 0) {
        FP8B_GLOAD(0);
        FP8B_SSTORE(0);
    }
    __syncthreads();

    for (int64_t kb = 0; kb < ti.KB; ++kb) {
        const int buf = (int)(kb & 1);
        // unconditional prefetch (the last iteration re-reads its own block)
        // keeps the staging registers out of scratch memory
        FP8B_GLOAD(kb + 1 < ti.KB ? kb + 1 : kb);
        const int64_t kg = ti.kbase + kb;                          // global K-block index

        const uint8_t* base = smem + buf * STAGE;
        v8i af[TJ], bf[TI];
#pragma unroll
        for (int t = 0; t < TJ; ++t) af[t] = lds_frag(base, BI + wj * WJ + t * 16 + (lane & 15), lane);
#pragma unroll
        for (int t = 0; t < TI; ++t) bf[t] = lds_frag(base, wi * WI + t * 16 + (lane & 15), lane);

        if constexpr (SM == SCALE_MX) {
            const uint8_t* eP = static_cast<const uint8_t*>(g.sP);
            const uint8_t* eQ = reinterpret_cast<const uint8_t*>(sQ);
            const int kq = (int)(kg * 4 + (lane >> 4));
            int sa[TJ], sb[TI];
#pragma unroll
            for (int t = 0; t < TJ; ++t) {
                int64_t r = jw + t * 16 + (lane & 15);
                r = r < jhi ? r : jhi - 1;
                sa[t] = eQ[r * g.sq_rs + kq];
            }
#pragma unroll
            for (int t = 0; t < TI; ++t) sb[t] = eP[prow[t] * g.ldsp + kq];
#pragma unroll
            for (int a = 0; a < TJ; ++a)
#pragma unroll
                for (int b = 0; b < TI; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[a], bf[b], acc[a][b],
                                                                                  0, 0, 0, sa[a], 0, sb[b]);
        } else {
            const float* sPf = static_cast<const float*>(g.sP);
            const float* sQf = reinterpret_cast<const float*>(sQ);
            float sp[TI];
#pragma unroll
            for (int t = 0; t < TI; ++t) sp[t] = sPf[prow[t] * g.ldsp + kg];
            if constexpr (SM == SCALE_Q_BLOCK) {
                const float sq = sQf[(jw / 128) * g.sq_rs + kg * g.sq_ks];
                float cmb[TI];
#pragma unroll
                for (int t = 0; t < TI; ++t) cmb[t] = sp[t] * sq;
#pragma unroll
                for (int a = 0; a < TJ; ++a)
#pragma unroll
                    for (int b = 0; b < TI; ++b) {
                        const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af[a], bf[b], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[a][b][r] = __builtin_fmaf(pr[r], cmb[b], acc[a][b][r]);
                    }
            } else {
                float sq[TJ][4];
#pragma unroll
                for (int a = 0; a < TJ; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int64_t j = jw + a * 16 + 4 * (lane >> 4) + r;
                        j = j < jhi ? j : jhi - 1;
                        sq[a][r] = sQf[j * g.sq_rs + kg * g.sq_ks];
                    }
#pragma unroll
                for (int a = 0; a < TJ; ++a)
#pragma unroll
                    for (int b = 0; b < TI; ++b) {
                        const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af[a], bf[b], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[a][b][r] = __builtin_fmaf(pr[r], sp[b] * sq[a][r], acc[a][b][r]);
                    }
            }
        }

        if (kb + 1 < ti.KB) FP8B_SSTORE(buf ^ 1);
        __syncthreads();
    }

#undef FP8B_GLOAD
#undef FP8B_SSTORE

    // ---------------------------------------------------- epilogue
#pragma unroll
    for (int a = 0; a < TJ; ++a) {
        const int64_t j = jw + a * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int b = 0; b < TI; ++b) {
            const int64_t i = ti.i0 + wi * WI + b * 16 + (lane & 15);
            if (i >= ti.ihi) continue;
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

template <int BI, int BJ, int TI, int TJ, int SM>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
    const int64_t jt = (a.Nn + BJ - 1) / BJ;
    int64_t it, z = 1;
    if (a.group_mode == GROUP_ROWS) it = (a.M + BI - 1) / BI + a.E;
    else it = (a.M + BI - 1) / BI;
    if (a.group_mode == GROUP_K) z = a.E;
    if (jt == 0 || it == 0 || z == 0) return hipSuccess;
    if (jt > 0x7FFFFFFF || it > 65535 || z > 65535) return hipErrorInvalidValue;
    k_gemm<BI, BJ, TI, TJ, SM><<<dim3((unsigned)jt, (unsigned)it, (unsigned)z), 256, 0, st>>>(a);
    return hipGetLastError();
}

template <int SM>
static hipError_t launch_sm(const GemmArgs& a, hipStream_t st) {
    // Small-M (decode) problems take 64-row tiles so the weight stream is
    // spread over more blocks; the per-element arithmetic is identical.
    if (a.group_mode == GROUP_NONE && a.M <= 64)
        return launch_cfg<64, 128, 4, 2, SM>(a, st);
    return launch_cfg<128, 128, 4, 4, SM>(a, st);
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
