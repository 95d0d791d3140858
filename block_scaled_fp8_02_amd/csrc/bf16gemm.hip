// bf16gemm.hip -- the bf16 GEMM of the dequantized-backward mode on gfx950
// MFMA, and the transposing copies that give it its operands.
//
// The Miles MXFP8/NVFP4 blog's backward-mode section offers a backward in
// which DGrad and WGrad run as plain bf16 GEMMs: dY stays bf16 and the
// forward's FP8 operand (W for DGrad, X for WGrad) enters as its bf16
// dequantization.  Here:
//
//   k_gemm_bf16       O[i][j] (+)= sum_k P[i][k] Q[j][k] with P (M x K) and
//                     Q (Nn x K) bf16, both contiguous along K, fp32
//                     accumulation in the matrix cores, bf16 (nearest-even)
//                     or fp32 output;
//   k_transpose_bf16  out[c][r] = value of in[r][c] as bf16, for a bf16
//                     input (a copy) or FP8 codes dequantized as
//                     bf16(fl32(E4M3(q) * scale)) with 1x128, 128x128 or MX
//                     1x32 scales -- the K-contiguous operand copies.
//
// The GEMM is the block-scaled FP8 GEMM's tile machinery without the scales:
// 256x256 block tile, 8 waves of 64x128, two 64 KB LDS stages filled by
// direct global->LDS copies (128 bytes of K per tile row = 64 bf16 values),
// one barrier per K block.  The fragment a lane reads for one FP8 MFMA (the
// 16-byte chunks g and g+4 of a row, g = lane/16) feeds two bf16 MFMAs
// (v_mfma_f32_16x16x32_bf16, K 0..31 and 32..63 of the block); the
// instruction's K order within a chunk is the same for both operands, so the
// pairs it multiplies are the pairs of the dot product.  A contraction that
// is not a multiple of 64 ends in a partial block: chunks that start past the
// last valid element are fetched from chunk 0 of the same row (in bounds),
// and every element at k >= K is cleared in both operands' fragments before
// the last block's MFMAs, so whatever the row padding holds contributes
// exactly zero.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                    0, 0, 0);
}

__device__ __forceinline__ v4i lo4(const v8i& x) { return v4i{x[0], x[1], x[2], x[3]}; }
__device__ __forceinline__ v4i hi4(const v8i& x) { return v4i{x[4], x[5], x[6], x[7]}; }

// Mask word d (elements 2d, 2d+1) of a chunk with v valid leading elements.
__device__ __forceinline__ uint32_t chunk_mask(int v, int d) {
    return v > 2 * d + 1 ? 0xFFFFFFFFu : (v > 2 * d ? 0x0000FFFFu : 0u);
}

template <int BI, int BJ, int TI, int TJ, int NW, int NS>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm_bf16(Bf16GemmArgs g) {
    constexpr int NT = 64 * NW;
    constexpr int WI = 16 * TI, WJ = 16 * TJ;
    constexpr int NWI = BI / WI, NWJ = BJ / WJ;
    static_assert(NWI * NWJ == NW, "wave grid must cover the block tile");
    constexpr int STAGE = (BI + BJ) * 128;
    constexpr int NCH = (BI + BJ) * 8 / NT;                 // 16-byte chunks per thread per stage
    static_assert(NCH * NT == (BI + BJ) * 8, "copy chunks must divide evenly");
    constexpr int NCP = BI * 8 / NT;                        // of which P rows
    static_assert(NCP * NT == BI * 8, "P rows must fill whole copy rounds");
    static_assert(NS >= 2, "at least double buffering");
    constexpr int INFLIGHT = (NS - 2) * NCH;
    static_assert(INFLIGHT <= 63, "vmcnt holds at most 63");
    constexpr bool STAGED_OUT = BI * BJ * 2 <= NS * STAGE;

    __shared__ __attribute__((aligned(16))) uint8_t smem[NS * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave % NWI, wj = wave / NWI;

    const int64_t nbi = (g.M + BI - 1) / BI, nbj = (g.Nn + BJ - 1) / BJ;
    int64_t ti, tj;
    grouped_tile(xcd_remap(blockIdx.x, nbi * nbj), nbi, nbj, 4, ti, tj);
    const int64_t i0 = ti * BI, j0 = tj * BJ;
    const int64_t ihi = i0 + BI < g.M ? i0 + BI : g.M;
    const int64_t jhi = j0 + BJ < g.Nn ? j0 + BJ : g.Nn;
    const int64_t KB = (g.K + 63) / 64;                     // 64-wide K blocks
    const int64_t kchunks = (g.K + 7) / 8;                  // 8-element chunks holding data
    const int kb_last_valid = (int)(g.K - (KB - 1) * 64);   // valid elements of the last block, 1..64

    // Copy addressing as in the FP8 GEMM: chunk q = c*NT + tid of a stage
    // lands at LDS byte 16*q (tile row q/8, physical chunk q%8 holding
    // logical chunk (q%8) ^ (row&7)); rows past the edge are clamped.  The
    // last K block fetches its chunks past the data from chunk 0 instead.
    const uint8_t* pbase = reinterpret_cast<const uint8_t*>(g.P + i0 * g.ldp);
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(g.Q + j0 * g.ldq);
    uint32_t soff[NCH], soff_last[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int q = c * NT + tid, row = q >> 3, lch = (q & 7) ^ (row & 7);
        int64_t rbytes;
        if (c < NCP) {
            const int64_t r = row < ihi - i0 ? row : ihi - i0 - 1;
            rbytes = r * g.ldp * 2;
        } else {
            const int64_t r = row - BI < jhi - j0 ? row - BI : jhi - j0 - 1;
            rbytes = r * g.ldq * 2;
        }
        soff[c] = (uint32_t)(rbytes + lch * 16);
        const bool has_data = (KB - 1) * 8 + lch < kchunks;
        soff_last[c] = (uint32_t)(rbytes + (has_data ? lch : 0) * 16);
    }
    // This lane's fragment chunks are g and g+4 (g = lane/16) of every block:
    // masks of their valid elements in the last block.
    uint32_t kmask[8];
    {
        const int v0 = kb_last_valid - 8 * (lane >> 4), v1 = v0 - 32;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            kmask[d] = chunk_mask(v0, d);
            kmask[4 + d] = chunk_mask(v1, d);
        }
    }
    const bool ragged_k = (g.K & 63) != 0;

    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
    auto dma_part = [&](int64_t kb, int buf, int c0, int c1) {
        const bool last = kb == KB - 1;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (c < c0 || c >= c1) continue;
            dma16(lds_base + (uint32_t)(buf * STAGE + (c * NT + wave * 64) * 16),
                  (c < NCP ? pbase : qbase) + kb * 128, last ? soff_last[c] : soff[c]);
        }
    };
    constexpr int DMA_PER_STEP = (NCH + TJ - 1) / TJ > 2 ? (NCH + TJ - 1) / TJ : 2;

    v4f acc[TJ][TI];
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
        for (int b = 0; b < TI; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    if (KB > 0) {
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) dma_part(st < KB ? st : KB - 1, st, 0, NCH);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFLIGHT));
    }
    __syncthreads();

    const int prow_l = wi * WI + (lane & 15);
    const int qrow_l = BI + wj * WJ;
    const FragOff pfo = frag_off(prow_l, lane);
    const FragOff qfo = frag_off(qrow_l + (lane & 15), lane);
    auto masked = [&](v8i x) {
#pragma unroll
        for (int d = 0; d < 8; ++d) x[d] = (int)((uint32_t)x[d] & kmask[d]);
        return x;
    };
    int buf = 0, nbuf = NS - 1;
    for (int64_t kb = 0; kb < KB; ++kb) {
        const int64_t kn = kb + NS - 1 < KB ? kb + NS - 1 : KB - 1;   // past the end: reload the last
                                                                      // block into an idle stage
        const uint8_t* base = smem + buf * STAGE;
        const bool tail = ragged_k && kb == KB - 1;
        v8i bf[TI];
#pragma unroll
        for (int t = 0; t < TI; ++t) bf[t] = lds_frag(base, pfo, t * 16 * 128);
        v8i af = lds_frag(base, qfo, 0);
        if (tail) {
#pragma unroll
            for (int t = 0; t < TI; ++t) bf[t] = masked(bf[t]);
        }
#pragma unroll
        for (int a = 0; a < TJ; ++a) {
            if (a * DMA_PER_STEP < NCH)
                dma_part(kn, nbuf, a * DMA_PER_STEP, (a + 1) * DMA_PER_STEP);
            v8i af_n = af;
            if (a + 1 < TJ) af_n = lds_frag(base, qfo, (a + 1) * 16 * 128);
            if (tail) af = masked(af);
#pragma unroll
            for (int b = 0; b < TI; ++b) {
                acc[a][b] = mfma_bf16(lo4(af), lo4(bf[b]), acc[a][b]);
                acc[a][b] = mfma_bf16(hi4(af), hi4(bf[b]), acc[a][b]);
            }
            af = af_n;
            __builtin_amdgcn_sched_barrier(0);
        }
        if (TJ * DMA_PER_STEP < NCH) dma_part(kn, nbuf, TJ * DMA_PER_STEP, NCH);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFLIGHT));        // block kb + 1 has landed
        __syncthreads();
        buf = buf + 1 == NS ? 0 : buf + 1;
        nbuf = nbuf + 1 == NS ? 0 : nbuf + 1;
    }
    // the tail's repeated copies target idle stages; let them land before the
    // stage memory is reused or the block exits
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    // ---------------------------------------------------- epilogue
    // Lane holds outputs (i, j..j+3): i = i0 + wi*WI + b*16 + lane%16,
    // j = j0 + wj*WJ + a*16 + 4*(lane/16).
    char* O = static_cast<char*>(g.O);
    if (STAGED_OUT && !g.out_f32) {
        // bf16 tile through LDS (rows of BJ*2 bytes; 8-byte chunks swizzled
        // by 2*(row%16) so 16 rows' writes hit distinct banks), then whole
        // rows out as 16-byte stores
        constexpr int CPR = BJ / 4, PPR = CPR / 2;
        uint8_t* stile = smem;
#pragma unroll
        for (int a = 0; a < TJ; ++a) {
            const int jl = wj * WJ + a * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int b = 0; b < TI; ++b) {
                const int il = wi * WI + b * 16 + (lane & 15);
                const v4f r = acc[a][b];
                uint2 v;
                v.x = f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16);
                v.y = f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16);
                const int ch = (jl >> 2) ^ ((2 * (il & 15)) & (CPR - 1) & ~1);
                *reinterpret_cast<uint2*>(stile + (il * CPR + ch) * 8) = v;
            }
        }
        __syncthreads();
        const bool full_cols = jhi - j0 == BJ && (g.ldo % 8) == 0;
        for (int q = tid; q < BI * PPR; q += NT) {
            const int il = q / PPR, pp = q % PPR;
            const int64_t i = i0 + il;
            if (i >= ihi) continue;
            const int ch = (2 * pp) ^ ((2 * (il & 15)) & (CPR - 1) & ~1);
            const uint4 v = *reinterpret_cast<const uint4*>(stile + (il * CPR + ch) * 8);
            const int64_t j = j0 + 8 * pp;
            uint16_t* o = reinterpret_cast<uint16_t*>(O) + i * g.ldo + j;
            if (full_cols) {
                *reinterpret_cast<uint4*>(o) = v;
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (j + e < g.Nn) o[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
        return;
    }
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

hipError_t launch_gemm_bf16(const Bf16GemmArgs& a, hipStream_t st) {
    const int64_t tiles = ((a.M + 255) / 256) * ((a.Nn + 255) / 256);
    if (tiles == 0) return hipSuccess;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    k_gemm_bf16<256, 256, 4, 8, 8, 2><<<dim3((unsigned)tiles), 512, 0, st>>>(a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------
// Transposing copies: out[c][r] (row stride ldo, elements) from in[r][c].
// A 256-thread block covers 64 rows x 256 columns of the input; thread t
// takes rows 8*(t%8) .. +7 and columns 8*(t/8) .. +7 of it: eight row
// loads (16 bytes of bf16, or 8 bytes of codes), an 8x8 transpose of 16-bit
// values in registers, eight 16-byte stores (one output row each; the 8
// threads sharing a column group write one 128-byte run).  Input rows past
// `rows` read as zero, so the 16-byte store of a partial row group writes
// zeros at output columns [rows, round_up(rows, 8)), which lie inside the
// output row stride (ldo is a multiple of 8 >= rows).
// SRC: 0 bf16 input; 1 FP8 codes with 1x128 row-group scales s[r][c/128];
// 2 FP8 codes with 128x128 block scales s[r/128][c/128]; 3 FP8 codes with
// MX E8M0 bytes e[r][c/32].  FP8 code rows are padded to a multiple of 128,
// so 8 codes at any column below `cols` are in bounds.
// ---------------------------------------------------------------------
template <int SRC>
__global__ __launch_bounds__(256) void k_transpose_bf16(const void* __restrict__ in, int64_t ldi,
                                                        const void* __restrict__ sp, int64_t lds,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t* __restrict__ out, int64_t ldo) {
    const int64_t ncb = (cols + 255) / 256;
    const int64_t rb = blockIdx.x / ncb, cb = blockIdx.x - rb * ncb;
    const int t = threadIdx.x;
    const int64_t r0 = rb * 64 + 8 * (t & 7);
    const int64_t c0 = cb * 256 + 8 * (t >> 3);
    if (c0 >= cols || r0 >= rows) return;
    uint32_t w[8][4];                                           // w[i][d]: columns 2d, 2d+1 of row r0+i
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + i;
        if (r >= rows) {
#pragma unroll
            for (int d = 0; d < 4; ++d) w[i][d] = 0;
            continue;
        }
        if (SRC == 0) {
            // bf16 rows: 8 values are in bounds when c0 + 8 <= ldi (ldi is a
            // multiple of 8 >= cols); a partial group reads element by element
            const uint16_t* p = static_cast<const uint16_t*>(in) + r * ldi + c0;
            if (c0 + 8 <= cols) {
                const uint4 v = *reinterpret_cast<const uint4*>(p);
                w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
            } else {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = c0 + e < cols ? p[e] : 0u;
#pragma unroll
                for (int d = 0; d < 4; ++d) w[i][d] = h[2 * d] | (h[2 * d + 1] << 16);
            }
        } else {
            float sc;
            if (SRC == 3) {
                const int e = static_cast<const uint8_t*>(sp)[r * lds + c0 / 32];
                sc = __builtin_ldexpf(1.0f, e - 127);
            } else {
                const int64_t sr = SRC == 2 ? r / 128 : r;
                sc = static_cast<const float*>(sp)[sr * lds + c0 / 128];
            }
            const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(in) + r * ldi + c0);
            const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false);
            const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
            const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false);
            const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
            const float v[8] = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = c0 + e < cols ? f32_to_bf16(v[e] * sc) : 0u;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) w[i][dd] = h[2 * dd] | (h[2 * dd + 1] << 16);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t c = c0 + j;
        if (c >= cols) break;
        uint32_t o[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = w[2 * d][j >> 1], hi = w[2 * d + 1][j >> 1];
            o[d] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        *reinterpret_cast<uint4*>(out + c * ldo + r0) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

hipError_t launch_transpose_bf16(int src, const void* in, int64_t ldi, const void* s, int64_t lds,
                                 int64_t rows, int64_t cols, uint16_t* out, int64_t ldo, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t blocks = ((rows + 63) / 64) * ((cols + 255) / 256);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (src) {
        case 0: k_transpose_bf16<0><<<grid, 256, 0, st>>>(in, ldi, s, lds, rows, cols, out, ldo); break;
        case 1: k_transpose_bf16<1><<<grid, 256, 0, st>>>(in, ldi, s, lds, rows, cols, out, ldo); break;
        case 2: k_transpose_bf16<2><<<grid, 256, 0, st>>>(in, ldi, s, lds, rows, cols, out, ldo); break;
        case 3: k_transpose_bf16<3><<<grid, 256, 0, st>>>(in, ldi, s, lds, rows, cols, out, ldo); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fp8blk
