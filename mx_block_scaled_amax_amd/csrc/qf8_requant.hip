// qf8_requant.hip -- re-grouping of 1x128-quantized FP8 data into 128x1 groups, stored transposed.
//
// Pages (title, section):
//   [MP-FP8] "混合精度与 FP8 训练" (hs-black.github.io): section 10.5 (an activation quantized in
//            1x128 groups is needed in 128x1 groups by the weight-gradient GEMM; the groups do
//            not transpose, so the data is read, de-scaled, transposed, quantized again in
//            128x1 groups and written back), section 10.4 (those tensors take power-of-two
//            scale factors so that the second quantization adds no error).
//
// Definition: v = fl32(decode(q) / S_row_group) (the de-scaling of the dequantization kernels),
// then for every column c and every group g of 128 rows: amax over the group, S' (Eq.(1) or the
// power-of-two rule), qT[c][r] = sat_rne8(fl32(v * S')), scalesT[c][g] = S'. The result holds
// the transpose in 1x128 groups, ready for a GEMM that reduces over the rows of the input.
//
// Work: one workgroup of 512 threads per 128 x 128 tile. The tile's codes (16 KiB) and its 128
// row scales go to LDS with 16-byte loads; each thread then owns 4 columns x 8 rows (one dword
// of codes per row, two values per convert instruction) and de-scales them in registers. When a
// row's scale is a power of two (the rule the pages use for these tensors) the division is the
// multiplication by its exact reciprocal (the same correctly rounded quotient); a wave whose rows
// all exist and all have such scales multiplies without per-row branches, and with power-of-two
// output scales a wave whose columns are all finite casts without the saturating clamp (the
// products cannot exceed F8max there). Column maxima meet through a lane exchange and LDS; the new codes of a
// column's 8 rows go as 8 bytes into a second 16 KiB LDS tile, transposed (16-byte chunks
// permuted by column so the writes spread over the banks), and the workgroup stores each
// column's 128 new codes as one 128-byte line of qT.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kTile = 128;
constexpr int kRqThreads = 512;          // thread = 4 columns x 8 rows of the tile
constexpr int kWaves = kRqThreads / 64;

__device__ __forceinline__ int ot_offset(int c, int k) { return c * kTile + ((k ^ ((c >> 3) & 7)) << 4); }

template <int FMT>
__device__ __forceinline__ void decode4(uint32_t w, float *d) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f lo, hi;
    if constexpr (FMT == kE4M3) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
    }
    d[0] = lo.x; d[1] = lo.y; d[2] = hi.x; d[3] = hi.y;
}

// sat_rne8(fl32(x * s)) for products known to lie within +-F8max (power-of-two scale of a finite
// column amax): the clamp of cast4 is the identity there, so it is left out.
template <int FMT>
__device__ __forceinline__ uint32_t cast4_in_range(float x0, float x1, float x2, float x3, float s) {
    return cvt2_f32<FMT, true>(x2 * s, x3 * s, cvt2_f32<FMT, false>(x0 * s, x1 * s, 0u));
}

// 1/S exactly when S is a power of two whose reciprocal is a normal fp32 value (then x / S and
// x * (1/S) are the same correctly rounded quotient), else 0.
__device__ __forceinline__ float exact_reciprocal(float s) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t e = (u >> 23) & 0xFFu;
    if ((u & 0x807FFFFFu) != 0u || e < 1u || e > 253u) return 0.0f;
    return __uint_as_float((254u - e) << 23);
}

// De-scale rows 8rg .. 8rg+7, columns 4cg .. 4cg+3 of the tile (v = fl32(decode / S_row)) and take
// the column maxima of |v| as bit patterns. FULL: all 128 rows exist and every row scale has an
// exact reciprocal, so every row multiplies; otherwise each row multiplies or divides (the 32
// lanes of a row take the same side) and rows beyond the tile's end stay out of the maxima.
template <int FIN, bool FULL>
__device__ __forceinline__ void descale_rows(const uint8_t *qs, const float *srow, const float *srec, int rg, int cg,
                                             int nr, float (&v)[8][4], uint32_t (&m)[4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * rg + i;
        decode4<FIN>(((const uint32_t *)qs)[row * (kTile / 4) + cg], v[i]);
        const float rec = srec[row];
        if (FULL || rec != 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[i][j] *= rec;
        } else {
            const float sr = srow[row];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[i][j] = v[i][j] / sr;
        }
        if (FULL || row < nr) {
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = umax(m[j], __float_as_uint(v[i][j]) & 0x7FFFFFFFu);
        }
    }
}

// New codes of columns 4cg .. 4cg+3, rows 8rg .. 8rg+7: 8 bytes per column into the transposed
// LDS tile. CLAMP: the saturating cast; otherwise every product is known to lie within +-F8max.
template <int FOUT, bool CLAMP>
__device__ __forceinline__ void cast_columns(const float (&v)[8][4], const float *scol, uint8_t *ot, int rg, int cg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = 4 * cg + j;
        const float sc = scol[col];
        const uint32_t lo = CLAMP ? cast4<FOUT>(v[0][j], v[1][j], v[2][j], v[3][j], sc)
                                  : cast4_in_range<FOUT>(v[0][j], v[1][j], v[2][j], v[3][j], sc);
        const uint32_t hi = CLAMP ? cast4<FOUT>(v[4][j], v[5][j], v[6][j], v[7][j], sc)
                                  : cast4_in_range<FOUT>(v[4][j], v[5][j], v[6][j], v[7][j], sc);
        *(uint2 *)(ot + ot_offset(col, rg >> 1) + (rg & 1) * 8) = make_uint2(lo, hi);
    }
}

template <int FIN, int FOUT, bool POW2>
__global__ __launch_bounds__(kRqThreads) void requant_t_kernel(const uint8_t *__restrict__ q,
                                                               const float *__restrict__ scales, int64_t rows,
                                                               int64_t cols, int tiles_c, int tiles, int per_xcd,
                                                               uint8_t *__restrict__ qT, float *__restrict__ scalesT,
                                                               int32_t *nonfinite) {
    __shared__ __attribute__((aligned(16))) uint8_t qs[kTile * kTile];     // [row][col]
    __shared__ __attribute__((aligned(16))) uint8_t ot[kTile * kTile];     // [col][row], chunks permuted
    __shared__ __attribute__((aligned(16))) float srow[kTile], srec[kTile], scol[kTile];
    __shared__ __attribute__((aligned(4))) uint8_t snf[kTile];           // column amax non-finite
    __shared__ uint32_t part[kWaves][kTile];
    // workgroups are dealt to the 8 XCDs round-robin; each XCD takes a contiguous run of tiles in
    // row-major order, so the tiles of a tile row, which gather their row scales from the same
    // lines, share one L2 (dealt round-robin, every XCD fetched those lines again: 1.21x the
    // algorithmic bytes read instead of ~1.0x, at the same speed)
    const int b = blockIdx.x, local = b >> 3, tile = (b & 7) * per_xcd + local;
    if (local >= per_xcd || tile >= tiles) return;       // whole workgroup idle
    const int tr = tile / tiles_c, tc = tile - tr * tiles_c;
    const int64_t r0 = (int64_t)tr * kTile, c0 = (int64_t)tc * kTile;
    const int nr = rows - r0 < kTile ? (int)(rows - r0) : kTile;          // multiples of 16
    const int nc = cols - c0 < kTile ? (int)(cols - c0) : kTile;
    const int t = threadIdx.x;
    const int64_t gcols = (cols + 127) / 128;

    // codes and row scales of the tile into LDS
#pragma unroll
    for (int j = 0; j < kTile * kTile / 16 / kRqThreads; ++j) {
        const int k = t + j * kRqThreads, row = k >> 3, ch = k & 7;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < nr && ch * 16 < nc) v = *(const uint4 *)(q + (r0 + row) * cols + c0 + ch * 16);
        *(uint4 *)(qs + row * kTile + ch * 16) = v;
    }
    if (t < kTile) {
        const float sr = t < nr ? scales[(r0 + t) * gcols + tc] : 1.0f;
        srow[t] = sr;
        srec[t] = exact_reciprocal(sr);
    }
    __syncthreads();

    // columns 4cg .. 4cg+3, rows 8rg .. 8rg+7: de-scale (v = fl32(decode / S_row)), column maxima.
    // A wave whose 16 rows all exist and all have exact reciprocals (the usual case: power-of-two
    // row scales) takes the path without per-row branches.
    const int cg = t & 31, rg = t >> 5, wave = t >> 6;
    const float4 ra = *(const float4 *)(srec + 8 * rg), rb = *(const float4 *)(srec + 8 * rg + 4);
    const bool own_fast = 8 * rg + 8 <= nr && ra.x != 0.0f && ra.y != 0.0f && ra.z != 0.0f && ra.w != 0.0f &&
                          rb.x != 0.0f && rb.y != 0.0f && rb.z != 0.0f && rb.w != 0.0f;
    const bool fast = __builtin_amdgcn_ballot_w64(!own_fast) == 0u;
    float v[8][4];
    uint32_t m[4] = {0, 0, 0, 0};
    if (fast) descale_rows<FIN, true>(qs, srow, srec, rg, cg, nr, v, m);
    else descale_rows<FIN, false>(qs, srow, srec, rg, cg, nr, v, m);
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = umax(m[j], (uint32_t)__shfl_xor((int)m[j], 32));   // the wave's 16 rows
    if ((t & 63) < 32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[wave][4 * cg + j] = m[j];
    }
    __syncthreads();
    if (t < kTile) {                                     // column t: maximum over the 8 waves, new scale
        uint32_t mc = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mc = umax(mc, part[w][t]);
        const float sc = POW2 ? scale_pow2_from_amax_bits<FOUT>(mc) : scale_from_amax_bits<FOUT>(mc);
        scol[t] = sc;
        snf[t] = mc >= 0x7F800000u;
        if (t < nc) {
            scalesT[(c0 + t) * ((rows + 127) / 128) + tr] = sc;
            if (nonfinite && mc >= 0x7F800000u) *nonfinite = 1;
        }
    }
    __syncthreads();
    // power-of-two scales put every product of a finite column within +-F8max (S' <= F8max / amax),
    // so the saturating clamp is needed only for Eq.(1) scales or in a wave with a non-finite column
    const bool clamp = !POW2 || __builtin_amdgcn_ballot_w64(*(const uint32_t *)(snf + 4 * cg) != 0u) != 0u;

    // new codes: for each column, its 8 rows as 8 bytes of the transposed output tile
    if (clamp) cast_columns<FOUT, true>(v, scol, ot, rg, cg);
    else cast_columns<FOUT, false>(v, scol, ot, rg, cg);
    __syncthreads();

    // each column's 128 codes: one line of qT, written once, so non-temporal (cached stores took
    // 25.2 µs on 8192x7168 against 24.0; the code loads stay cached: non-temporal loads took 31.0)
#pragma unroll
    for (int j = 0; j < kTile * kTile / 16 / kRqThreads; ++j) {
        const int k = t + j * kRqThreads, col = k >> 3, ch = k & 7;
        if (col < nc && ch * 16 < nr)
            st_stream((uint4 *)(qT + (c0 + col) * rows + r0 + ch * 16), *(const uint4 *)(ot + ot_offset(col, ch)));
    }
}

}  // namespace

int launch_requant_t(const uint8_t *q, const float *scales, int64_t rows, int64_t cols, int fmt_in, int fmt_out,
                     int pow2, uint8_t *qT, float *scalesT, int32_t *nonfinite, hipStream_t s) {
    if (rows == 0 || cols == 0) return QF8_OK;
    const int tiles_r = (int)((rows + kTile - 1) / kTile), tiles_c = (int)((cols + kTile - 1) / kTile);
    const int tiles = tiles_r * tiles_c, per_xcd = (tiles + 7) / 8;
    const dim3 grid((unsigned)(8 * per_xcd)), block(kRqThreads);
#define QF8_RQ(FI, FO, P) hipLaunchKernelGGL((requant_t_kernel<FI, FO, P>), grid, block, 0, s, q, scales, rows, cols, \
                                             tiles_c, tiles, per_xcd, qT, scalesT, nonfinite)
#define QF8_RQP(FI, FO) do { if (pow2) QF8_RQ(FI, FO, true); else QF8_RQ(FI, FO, false); } while (0)
    if (fmt_in == QF8_E4M3) { if (fmt_out == QF8_E4M3) QF8_RQP(kE4M3, kE4M3); else QF8_RQP(kE4M3, kE5M2); }
    else { if (fmt_out == QF8_E4M3) QF8_RQP(kE5M2, kE4M3); else QF8_RQP(kE5M2, kE5M2); }
#undef QF8_RQP
#undef QF8_RQ
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
