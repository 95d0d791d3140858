// quant.hip -- gfx950 quantizer kernels for the block-scaled FP8 path.
//
// Both kernels apply the quantizer Q of the Jet-RL notes (section 2.1):
// S = max|x| / 448 per group, code = E4M3(fl32(x / S)), nearest-even,
// saturating.  They differ in the grouping (section 4.2 of the notes; the
// summary page's weight and activation quantization paragraphs):
//   k_quant_rows    1x128 along the contiguous axis (X for FProp, dY for DGrad)
//   k_quant_tiles   128x128 tiles: weight blocks (optionally also the
//                   transposed codes), or 1x128 groups along the token axis
//                   written transposed (the WGrad operands), optionally with
//                   the row-wise copy from the same read of the input
//
// Data movement: every input element is read from HBM exactly once with
// 16-byte vector loads; codes leave as 8- or 16-byte stores.  The
// transposed copies go through a 16 KB LDS tile whose 8-byte chunks are
// XOR-swizzled so that neither the writes nor the row reads conflict.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// ---------------------------------------------------------------------
// 1x128 row-wise.  A 16-lane slot owns one group of 128 elements, 8 per
// lane; a 256-thread block owns 16 consecutive groups (row-major order).
// ---------------------------------------------------------------------
template <typename T, bool P2>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ x, int64_t cols, int64_t ldx,
                                                    uint8_t* __restrict__ q, int64_t ldq,
                                                    float* __restrict__ s, int64_t lds,
                                                    uint8_t* __restrict__ e8, int64_t lde,
                                                    uint32_t groups_per_row, uint32_t total_groups) {
    const uint32_t grp = blockIdx.x * 16u + (threadIdx.x >> 4);
    if (grp >= total_groups) return;                 // whole 16-lane slots exit together
    const uint32_t row = grp / groups_per_row;
    const uint32_t g = grp - row * groups_per_row;
    const int lane16 = threadIdx.x & 15;
    const int64_t col0 = (int64_t)g * 128 + lane16 * 8;
    const int valid = clamp_valid(cols - col0);
    float v[8];
    load8(x + (int64_t)row * ldx + col0, valid, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = max16(amax);
    const float S = block_scale<P2>(amax);
    const float P = prescale(S);
    const float Sp = S * P, r = recip32(Sp);
    float y[8];
    if (__all(P == 1.0f)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = quotient32(v[i], Sp, r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = quotient32(v[i] * P, Sp, r);
    }
    uint2 out;
    out.x = e4m3_pack4_q(y[0], y[1], y[2], y[3]);
    out.y = e4m3_pack4_q(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2*>(q + (int64_t)row * ldq + col0) = out;
    if (lane16 == 0) {
        s[(int64_t)row * lds + g] = S;
        if (P2 && e8 != nullptr) *reinterpret_cast<uint32_t*>(e8 + (int64_t)row * lde + 4 * (int64_t)g) = e8m0_x4(amax);
    }
}

// ---------------------------------------------------------------------
// Tile quantizer: 128x128 tiles, persistent blocks.
//
// One 256-thread block walks tiles k = blockIdx.x, +gridDim.x, ... in
// row-tile-major order; the next tile's input is loaded into registers
// while the current one is quantized, so every block keeps one tile of
// loads in flight.  Thread t owns rows 8*(t/16)..+7 and columns
// 8*(t%16)..+7 of a tile.
//
//   QT_WEIGHT     one scale per tile (128x128 weight blocks): codes q and,
//                 optionally, the same codes transposed (qT)
//   QT_COLS       1x128 groups along the row (token) axis: per-column
//                 scales, codes written transposed (qT, sT)
//   QT_COLS_ROWS  as QT_COLS, plus the row-wise 1x128 codes (q, s) from
//                 the same registers
//
// Grouped (MoE) token-axis mode: rows [offsets[e], offsets[e+1]) form
// expert e; its row tiles never cross the expert's end and its transposed
// codes start at the padded position P_e = sum_{e'<e} round_up(n_e', 128).
// Every block advances a cursor over the experts as its tile index grows.
// ---------------------------------------------------------------------
enum { QT_WEIGHT = 0, QT_COLS = 1, QT_COLS_ROWS = 2 };

struct QuantTileArgs {
    const void* x; int64_t rows, cols, ldx;
    const int32_t* offsets; int64_t E;
    uint8_t* q; int64_t ldq; float* s; int64_t lds;
    uint8_t* qT; int64_t ldqT; float* sT; int64_t ldsT;
    const float* xs; int64_t ldxs;  // FP8 input (requantization): 1x128 scales of x's codes
    uint8_t* e8; int64_t lde;       // power-of-two scales: E8M0 bytes of q's groups (nullable)
    uint8_t* e8T; int64_t ldeT;     // and of qT's groups (nullable)
    int64_t col_tiles;
    int64_t tiles;          // dense: exact tile count; grouped: an upper bound
};

// 8 rows x 8 columns of raw input per thread.
template <typename T> struct RawTile;
template <> struct RawTile<uint16_t> { uint4 w[8]; };
template <> struct RawTile<float> { uint4 w[16]; };
// FP8 codes and their row scales, as loaded: masking of rows past the tile
// and columns past `cols` waits for unpack_row, so that the loads of the
// next tile stay in flight while this one is quantized.
template <> struct RawTile<uint8_t> {
    uint2 w[8];
    float s[8];
    uint32_t klo, khi;      // byte mask of the columns inside `cols`
    uint32_t rows;          // bit p: row p lies inside the tile
};

__device__ __forceinline__ void load_raw_row(const uint16_t* p, int valid, RawTile<uint16_t>& rt, int i) {
    if (valid == 8) {
        rt.w[i] = *reinterpret_cast<const uint4*>(p);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = j < valid ? (uint32_t)p[j] : 0u;
        rt.w[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
}

__device__ __forceinline__ void load_raw_row(const float* p, int valid, RawTile<float>& rt, int i) {
    if (valid == 8) {
        rt.w[2 * i] = *reinterpret_cast<const uint4*>(p);
        rt.w[2 * i + 1] = *reinterpret_cast<const uint4*>(p + 4);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = j < valid ? __float_as_uint(p[j]) : 0u;
        rt.w[2 * i] = make_uint4(h[0], h[1], h[2], h[3]);
        rt.w[2 * i + 1] = make_uint4(h[4], h[5], h[6], h[7]);
    }
}

__device__ __forceinline__ void unpack_row(const RawTile<uint16_t>& rt, int i, float v[8]) {
    const uint4 w = rt.w[i];
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xFFFF0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

// fl32(E4M3(code) * s): the hardware conversion decodes exactly, one
// binary32 multiply applies the group scale.
__device__ __forceinline__ void unpack_row(const RawTile<uint8_t>& rt, int i, float v[8]) {
    const bool in = (rt.rows >> i) & 1u;
    const uint2 w = make_uint2(rt.w[i].x & (in ? rt.klo : 0u), rt.w[i].y & (in ? rt.khi : 0u));
    const float sc = rt.s[i];                          // finite: read from a row of the input
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    v[0] = a[0] * sc; v[1] = a[1] * sc; v[2] = b[0] * sc; v[3] = b[1] * sc;
    v[4] = c[0] * sc; v[5] = c[1] * sc; v[6] = d[0] * sc; v[7] = d[1] * sc;
}

__device__ __forceinline__ void unpack_row(const RawTile<float>& rt, int i, float v[8]) {
    const uint4 a = rt.w[2 * i], b = rt.w[2 * i + 1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

// A thread's 8x8 values, unpacked once into fp32 registers.
template <typename T> struct TileVals {
    float v[8][8];
    __device__ __forceinline__ void set(const RawTile<T>& rt) {
#pragma unroll
        for (int p = 0; p < 8; ++p) unpack_row(rt, p, v[p]);
    }
    __device__ __forceinline__ float operator()(int p, int j) const { return v[p][j]; }
};

// Where a tile lies: input rows [a, b), first column cb, first position of
// its transposed codes pos, row-tile index rt (scale row of QT_WEIGHT) and
// column-tile index ct.
struct TileAt {
    int64_t a, b, cb, pos, rt, ct;
    bool valid;
};

// Tiles are numbered in bands of QT_BAND row tiles walked column by column.
// With one row tile per band the tiles in flight at one time (one per
// resident block, consecutive numbers) cover whole rows of the input and of
// the row-wise codes, and each transposed code row in 128-byte pieces; wider
// bands trade input-row runs for transposed-row runs and measured slower
// (token-axis quantization of X [8192 x 12288]: 71 us with bands of 1 row
// tile, 76 us with 32).
constexpr int64_t QT_BAND = 1;

// Experts whose offsets a grouped tile quantizer keeps in LDS (more: read
// from global memory).
constexpr int QT_MAX_OFFS = 1025;

// offs: the experts' offsets (A.offsets, or the block's LDS copy of them).
__device__ __forceinline__ TileAt locate_tile(const QuantTileArgs& A, const int32_t* offs, int64_t k, SegPos& cur) {
    TileAt at;
    at.valid = k < A.tiles;
    const int64_t nr = A.tiles / A.col_tiles;                     // row tiles (grouped: an upper bound)
    const int64_t band = k / (QT_BAND * A.col_tiles);
    const int64_t r0 = band * QT_BAND;
    const int64_t rows_b = nr - r0 < QT_BAND ? nr - r0 : QT_BAND;
    const int64_t rin = k - band * QT_BAND * A.col_tiles;
    at.rt = r0 + (rows_b > 0 ? rin % rows_b : 0);
    at.ct = rows_b > 0 ? rin / rows_b : 0;
    at.cb = at.ct * 128;
    if (A.offsets == nullptr) {
        at.a = at.rt * 128;
        at.b = at.a + 128 < A.rows ? at.a + 128 : A.rows;
        at.pos = at.a;
        return at;
    }
    if (!at.valid) {
        at.a = at.b = at.pos = 0;
        return at;
    }
    // a block's row-tile index normally only grows; search afresh if not
    if (at.rt < cur.first) cur = SegPos{0, 0, 0};
    cur = wave_find_tile(offs, A.E, at.rt, 128, cur);
    at.valid = cur.e < A.E;
    if (!at.valid) {                                               // past the experts' last tile
        cur = SegPos{0, 0, 0};
        at.a = at.b = at.pos = 0;
        return at;
    }
    const int64_t hi = offs[cur.e + 1];
    const int64_t g = at.rt - cur.first;
    at.a = offs[cur.e] + 128 * g;
    at.b = at.a + 128 < hi ? at.a + 128 : hi;
    at.pos = cur.P + 128 * g;
    return at;
}

// FP8 input: 8 codes per row (always inside the 128-padded row) and the row's
// scale of this column tile.  A row past the tile reads the tile's first
// row instead; unpack_row turns it, and codes past `cols`, into zeros.
__device__ __forceinline__ void load_tile(const QuantTileArgs& A, const TileAt& at, int rg, int cg,
                                          RawTile<uint8_t>& raw) {
    const uint8_t* x = static_cast<const uint8_t*>(A.x);
    const int64_t c0 = at.cb + cg * 8;
    const int cvalid = clamp_valid(A.cols - c0);
    raw.klo = cvalid >= 4 ? ~0u : (1u << (8 * cvalid)) - 1u;
    raw.khi = cvalid >= 8 ? ~0u : (cvalid <= 4 ? 0u : (1u << (8 * (cvalid - 4))) - 1u);
    raw.rows = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = at.a + rg * 8 + p;
        const bool in = r < at.b;
        const int64_t rr = in ? r : at.a;
        raw.rows |= (in ? 1u : 0u) << p;
        raw.w[p] = *reinterpret_cast<const uint2*>(x + rr * A.ldx + c0);
        raw.s[p] = A.xs[rr * A.ldxs + at.ct];
    }
}

template <typename T>
__device__ __forceinline__ void load_tile(const QuantTileArgs& A, const TileAt& at, int rg, int cg, RawTile<T>& raw) {
    const T* x = static_cast<const T*>(A.x);
    const int64_t c0 = at.cb + cg * 8;
    const int cvalid = clamp_valid(A.cols - c0);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = at.a + rg * 8 + p;
        const bool in = r < at.b;
        load_raw_row(x + (in ? r : 0) * A.ldx + c0, in ? cvalid : 0, raw, p);
    }
}

// Codes of one thread's 8x8 values with one scale per row (PER_ROW) or
// per column: S = S_group*P, r = RN32(1/S), P = prescale(S_group).  The
// multiplication by P is skipped when every P of the tile is 1 (plain).
template <bool PER_ROW, bool SCALED, class V>
__device__ __forceinline__ void encode_8x8_v(const V& v, const float S[8], const float r[8], const float P[8],
                                             uint32_t lo[8], uint32_t hi[8]) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = PER_ROW ? p : j;
            y[j] = quotient32(SCALED ? v(p, j) * P[g] : v(p, j), S[g], r[g]);
        }
        lo[p] = e4m3_pack4_q(y[0], y[1], y[2], y[3]);
        hi[p] = e4m3_pack4_q(y[4], y[5], y[6], y[7]);
    }
}

template <bool PER_ROW, class V>
__device__ __forceinline__ void encode_8x8(bool plain, const V& v, const float S[8], const float r[8],
                                           const float P[8], uint32_t lo[8], uint32_t hi[8]) {
    if (plain)
        encode_8x8_v<PER_ROW, false>(v, S, r, P, lo, hi);
    else
        encode_8x8_v<PER_ROW, true>(v, S, r, P, lo, hi);
}

// Eight consecutive LDS floats.
__device__ __forceinline__ void lds_read8(const float* p, float o[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load, which would drain the next tile's prefetch at
// the first barrier of each tile; LDS writes only need lgkmcnt(0).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T, int MODE, bool P2>
__global__ __launch_bounds__(256, 2) void k_quant_tiles(QuantTileArgs A) {
    __shared__ __attribute__((aligned(16))) float red_col[16][128];   // [row slice][column]
    __shared__ __attribute__((aligned(16))) float red_row[16][128];   // [column slice][row]
    __shared__ __attribute__((aligned(16))) float sc_col[3][128];     // S*P, RN32(1/(S*P)), P per column
    __shared__ __attribute__((aligned(16))) float sc_row[3][128];     // the same per row
    __shared__ __attribute__((aligned(16))) uint8_t tileT[128 * 128];
    __shared__ float red4[4];
    __shared__ int scaled_flag;       // some group of the tile needs P != 1

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int rg = t >> 4, cg = t & 15;
    const bool want_qT = MODE != QT_WEIGHT || A.qT != nullptr;
    if (t == 0) scaled_flag = 0;

    // grouped: the experts' offsets, read once into LDS (each tile's expert
    // search then reads LDS instead of global memory)
    __shared__ int32_t soffs[QT_MAX_OFFS];
    const int32_t* offs = A.offsets;
    if (A.offsets != nullptr && A.E < QT_MAX_OFFS) {
        for (int64_t i = t; i <= A.E; i += 256) soffs[i] = A.offsets[i];
        offs = soffs;
        lds_barrier();
    }

    SegPos cur{0, 0, 0};
    int64_t k = blockIdx.x;
    TileAt at = locate_tile(A, offs, k, cur);
    RawTile<T> raw;
    if (at.valid) load_tile(A, at, rg, cg, raw);
    lds_barrier();

    for (; k < A.tiles; k += gridDim.x) {
        // grouped: the experts' row tiles are numbered without gaps, so the
        // first tile past the last expert ends the block's work (the launch
        // sizes the slots for the worst case)
        if (!at.valid) break;                                      // uniform
        const TileAt nx = locate_tile(A, offs, k + gridDim.x, cur);
        TileVals<T> v;
        v.set(raw);
        if (nx.valid) load_tile(A, nx, rg, cg, raw);            // next tile, while this one is quantized

        uint32_t lo[8], hi[8];
        if (MODE == QT_WEIGHT) {
            float m = 0.0f;
#pragma unroll
            for (int p = 0; p < 8; ++p)
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v(p, j)));
            m = max64(m);
            if (lane == 0) red4[wave] = m;
            lds_barrier();                                           // (1)
            m = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
            const float S = block_scale<P2>(m);
            if (t == 0) A.s[at.rt * A.lds + at.ct] = S;
            if (P2) {                                                  // E8M0 per row (q) and per column (qT)
                const uint32_t ew = e8m0_x4(m);
                if (t < 128) {
                    if (A.e8 != nullptr && at.a + t < at.b) *reinterpret_cast<uint32_t*>(A.e8 + (at.a + t) * A.lde + 4 * at.ct) = ew;
                } else if (A.e8T != nullptr && at.cb + t - 128 < A.cols) {
                    *reinterpret_cast<uint32_t*>(A.e8T + (at.cb + t - 128) * A.ldeT + 4 * at.rt) = ew;
                }
            }
            const float P = prescale(S);
            float Sv[8], rv[8], Pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) { Sv[i] = S * P; rv[i] = recip32(S * P); Pv[i] = P; }
            encode_8x8<true>(P == 1.0f, v, Sv, rv, Pv, lo, hi);       // P is uniform over the block
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int64_t row = at.a + rg * 8 + p;
                if (row < at.b) *reinterpret_cast<uint2*>(A.q + row * A.ldq + at.cb + cg * 8) = make_uint2(lo[p], hi[p]);
            }
        } else {
            // partial maxima: columns over this thread's 8 rows, rows over its 8 columns
            float cm[8], rm[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) cm[j] = 0.0f;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                float m = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float a = fabsf(v(p, j));
                    cm[j] = fmaxf(cm[j], a);
                    m = fmaxf(m, a);
                }
                rm[p] = m;
            }
            *reinterpret_cast<float4*>(&red_col[rg][cg * 8]) = make_float4(cm[0], cm[1], cm[2], cm[3]);
            *reinterpret_cast<float4*>(&red_col[rg][cg * 8 + 4]) = make_float4(cm[4], cm[5], cm[6], cm[7]);
            if (MODE == QT_COLS_ROWS) {
                *reinterpret_cast<float4*>(&red_row[cg][rg * 8]) = make_float4(rm[0], rm[1], rm[2], rm[3]);
                *reinterpret_cast<float4*>(&red_row[cg][rg * 8 + 4]) = make_float4(rm[4], rm[5], rm[6], rm[7]);
            }
            lds_barrier();                                           // (1)
            if (t < 128) {
                float m = red_col[0][t];
#pragma unroll
                for (int i = 1; i < 16; ++i) m = fmaxf(m, red_col[i][t]);
                const float S = block_scale<P2>(m), P = prescale(S);
                if (P2 && A.e8T != nullptr && at.cb + t < A.cols)
                    *reinterpret_cast<uint32_t*>(A.e8T + (at.cb + t) * A.ldeT + at.pos / 32) = e8m0_x4(m);
                sc_col[0][t] = S * P;
                sc_col[1][t] = recip32(S * P);
                sc_col[2][t] = P;
                if (P != 1.0f) scaled_flag = 1;
                if (at.cb + t < A.cols) A.sT[(at.cb + t) * A.ldsT + at.pos / 128] = S;
            } else if (MODE == QT_COLS_ROWS) {
                const int rr = t - 128;
                float m = red_row[0][rr];
#pragma unroll
                for (int i = 1; i < 16; ++i) m = fmaxf(m, red_row[i][rr]);
                const float S = block_scale<P2>(m), P = prescale(S);
                if (P2 && A.e8 != nullptr && at.a + rr < at.b)
                    *reinterpret_cast<uint32_t*>(A.e8 + (at.a + rr) * A.lde + 4 * at.ct) = e8m0_x4(m);
                sc_row[0][rr] = S * P;
                sc_row[1][rr] = recip32(S * P);
                sc_row[2][rr] = P;
                if (P != 1.0f) scaled_flag = 1;
                if (at.a + rr < at.b) A.s[(at.a + rr) * A.lds + at.ct] = S;
            }
            lds_barrier();                                           // (2)
            const bool plain = scaled_flag == 0;
            float Sv[8], rv[8], Pv[8];
            if (MODE == QT_COLS_ROWS) {
                lds_read8(&sc_row[0][rg * 8], Sv);
                lds_read8(&sc_row[1][rg * 8], rv);
                lds_read8(&sc_row[2][rg * 8], Pv);
                encode_8x8<true>(plain, v, Sv, rv, Pv, lo, hi);
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int64_t row = at.a + rg * 8 + p;
                    if (row < at.b) *reinterpret_cast<uint2*>(A.q + row * A.ldq + at.cb + cg * 8) = make_uint2(lo[p], hi[p]);
                }
            }
            lds_read8(&sc_col[0][cg * 8], Sv);
            lds_read8(&sc_col[1][cg * 8], rv);
            lds_read8(&sc_col[2][cg * 8], Pv);
            encode_8x8<false>(plain, v, Sv, rv, Pv, lo, hi);
        }

        if (want_qT) {
            uint32_t tlo[8], thi[8];
            transpose8x8_perm(lo, hi, tlo, thi);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint2*>(tileT + (cg * 8 + j) * 128 + ((rg ^ cg) << 3)) = make_uint2(tlo[j], thi[j]);
        }
        lds_barrier();                                               // (3)
        if (want_qT) {
            // 8 lanes per code row: every store instruction writes 8 whole
            // 128-byte rows.  Lane chunk ch holds logical 8-byte chunks 2ch and
            // 2ch+1, stored at physical (2ch)^s and (2ch+1)^s, s = crow/8: one
            // aligned 16-byte pair, its halves swapped when s is odd.
            const int ch = t & 7;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int crow = (t >> 3) + 32 * i;
                const int s8 = crow >> 3;
                const uint4 u = *reinterpret_cast<const uint4*>(tileT + crow * 128 + ((((2 * ch) ^ s8) & ~1) << 3));
                const uint4 w = (s8 & 1) ? make_uint4(u.z, u.w, u.x, u.y) : u;
                const int64_t c = at.cb + crow;
                if (c < A.cols) *reinterpret_cast<uint4*>(A.qT + c * A.ldqT + at.pos + 16 * ch) = w;
            }
        }
        if (MODE != QT_WEIGHT && t == 0) scaled_flag = 0;   // every wave has read it (before barrier 3)
        at = nx;
    }
}

// ---------------------------------------------------------------------
// Elementwise access to the codec (exhaustive device checks).
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode(const float* __restrict__ x, const float* __restrict__ s,
                                                int64_t n, uint8_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float y = x[i];
        if (s != nullptr) {
            const float S = s[i], P = prescale(S), Sp = S * P, r = recip32(Sp);
            const float xp = y * P, q0 = xp * r;
            // |x/S| beyond 2^10 saturates whatever its exact value (q0 may be
            // +-inf); below it quotient32's conditions hold
            y = fabsf(q0) < 1024.0f ? quotient32(xp, Sp, r) : q0;
        }
        out[i] = (uint8_t)e4m3_encode(y);
    }
}

// ---------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------
hipError_t launch_quant_rows(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             bool pow2, uint8_t* e8, int64_t lde, hipStream_t st) {
    const int64_t gpr = (cols + 127) / 128;
    const int64_t total = rows * gpr;
    if (total == 0) return hipSuccess;
    if (total > 0xFFFFFFF0ll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 15) / 16));
#define FP8B_ROWS(T_, P2_) \
    k_quant_rows<T_, P2_><<<grid, 256, 0, st>>>(static_cast<const T_*>(x), cols, ldx, q, ldq, s, lds, e8, lde, \
                                                 (uint32_t)gpr, (uint32_t)total)
    if (in_bf16) {
        if (pow2) FP8B_ROWS(uint16_t, true); else FP8B_ROWS(uint16_t, false);
    } else {
        if (pow2) FP8B_ROWS(float, true); else FP8B_ROWS(float, false);
    }
#undef FP8B_ROWS
    return hipGetLastError();
}

int device_cu_count() {
    static int cu_count[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int cus = dev < 64 ? cu_count[dev] : 0;
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (dev < 64) cu_count[dev] = cus;
    }
    return cus;
}

static int64_t tile_grid(int64_t tiles) {
    const int64_t g = 2 * (int64_t)device_cu_count();
    return tiles < g ? tiles : g;
}

template <int MODE>
static hipError_t launch_tiles(bool in_bf16, bool pow2, const QuantTileArgs& A, hipStream_t st) {
    const int64_t blocks = tile_grid(A.tiles);
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks);
    if (in_bf16) {
        if (pow2) k_quant_tiles<uint16_t, MODE, true><<<grid, 256, 0, st>>>(A);
        else k_quant_tiles<uint16_t, MODE, false><<<grid, 256, 0, st>>>(A);
    } else {
        if (pow2) k_quant_tiles<float, MODE, true><<<grid, 256, 0, st>>>(A);
        else k_quant_tiles<float, MODE, false><<<grid, 256, 0, st>>>(A);
    }
    return hipGetLastError();
}

hipError_t launch_quant_weight(const void* w, bool in_bf16, int64_t D, int64_t C, int64_t ldw,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               uint8_t* qT, int64_t ldqT,
                               bool pow2, uint8_t* e8, int64_t lde, uint8_t* e8T, int64_t ldeT, hipStream_t st) {
    if (D == 0 || C == 0) return hipSuccess;
    QuantTileArgs A{};
    A.x = w; A.rows = D; A.cols = C; A.ldx = ldw;
    A.offsets = nullptr; A.E = 0;
    A.q = q; A.ldq = ldq; A.s = s; A.lds = lds;
    A.qT = qT; A.ldqT = ldqT; A.sT = nullptr; A.ldsT = 0;
    A.e8 = e8; A.lde = lde; A.e8T = e8T; A.ldeT = ldeT;
    A.col_tiles = (C + 127) / 128;
    A.tiles = (D + 127) / 128 * A.col_tiles;
    return launch_tiles<QT_WEIGHT>(in_bf16, pow2, A, st);
}

hipError_t launch_quant_cols(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             const int32_t* offsets, int64_t E,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             bool pow2, uint8_t* e8T, int64_t ldeT, uint8_t* e8, int64_t lde, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    QuantTileArgs A{};
    A.x = x; A.rows = rows; A.cols = cols; A.ldx = ldx;
    A.offsets = offsets; A.E = offsets ? E : 0;
    A.q = q; A.ldq = ldq; A.s = s; A.lds = lds;
    A.qT = qT; A.ldqT = ldqT; A.sT = sT; A.ldsT = ldsT;
    A.e8 = e8; A.lde = lde; A.e8T = e8T; A.ldeT = ldeT;
    A.col_tiles = (cols + 127) / 128;
    // grouped: at most one partial tile per expert beyond rows/128
    A.tiles = ((rows + 127) / 128 + A.E) * A.col_tiles;
    return q != nullptr ? launch_tiles<QT_COLS_ROWS>(in_bf16, pow2, A, st)
                        : launch_tiles<QT_COLS>(in_bf16, pow2, A, st);
}

hipError_t launch_requant_cols(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                               int64_t rows, int64_t cols, const int32_t* offsets, int64_t E,
                               uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    QuantTileArgs A{};
    A.x = q; A.rows = rows; A.cols = cols; A.ldx = ldq;
    A.xs = s; A.ldxs = lds;
    A.offsets = offsets; A.E = offsets ? E : 0;
    A.qT = qT; A.ldqT = ldqT; A.sT = sT; A.ldsT = ldsT;
    A.col_tiles = (cols + 127) / 128;
    A.tiles = ((rows + 127) / 128 + A.E) * A.col_tiles;
    const int64_t blocks = tile_grid(A.tiles);
    if (blocks <= 0) return hipSuccess;
    k_quant_tiles<uint8_t, QT_COLS, false><<<dim3((unsigned)blocks), 256, 0, st>>>(A);
    return hipGetLastError();
}

hipError_t launch_encode(const float* x, const float* s, int64_t n, uint8_t* out, hipStream_t st) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    k_encode<<<dim3((unsigned)blocks), 256, 0, st>>>(x, s, n, out);
    return hipGetLastError();
}

}  // namespace fp8blk
