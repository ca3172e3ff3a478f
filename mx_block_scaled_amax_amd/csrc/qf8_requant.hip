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
// Work: one workgroup of 256 threads per 128 x 128 tile. The tile's codes (16 KiB) and its 128
// row scales go to LDS with 16-byte loads; thread t then owns column t % 128 and 64 of its rows:
// it de-scales them in registers, the two halves of a column exchange their maxima through LDS,
// and the new codes are written, transposed, into a second 16 KiB LDS tile (16-byte chunks
// permuted by column so the writes spread over the banks). The workgroup stores each column's
// 128 new codes as one 128-byte line of qT.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kRqThreads = 256;
constexpr int kTile = 128;

__device__ __forceinline__ int ot_offset(int c, int k) { return c * kTile + ((k ^ ((c >> 3) & 7)) << 4); }

template <int FMT>
__device__ __forceinline__ float decode1(uint32_t code) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f d = FMT == kE4M3 ? __builtin_amdgcn_cvt_pk_f32_fp8(code, false) : __builtin_amdgcn_cvt_pk_f32_bf8(code, false);
    return d.x;
}

template <int FIN, int FOUT, bool POW2>
__global__ __launch_bounds__(kRqThreads) void requant_t_kernel(const uint8_t *__restrict__ q,
                                                               const float *__restrict__ scales, int64_t rows,
                                                               int64_t cols, int tiles_c, uint8_t *__restrict__ qT,
                                                               float *__restrict__ scalesT, int32_t *nonfinite) {
    __shared__ __attribute__((aligned(16))) uint8_t qs[kTile * kTile];     // [row][col]
    __shared__ __attribute__((aligned(16))) uint8_t ot[kTile * kTile];     // [col][row], chunks permuted
    __shared__ float srow[kTile];
    __shared__ uint32_t half_max[2][kTile];
    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
    const int64_t r0 = (int64_t)tr * kTile, c0 = (int64_t)tc * kTile;
    const int nr = rows - r0 < kTile ? (int)(rows - r0) : kTile;          // multiples of 16
    const int nc = cols - c0 < kTile ? (int)(cols - c0) : kTile;
    const int t = threadIdx.x;
    const int64_t gcols = (cols + 127) / 128;

    // codes and row scales of the tile into LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = t + j * kRqThreads, row = k >> 3, ch = k & 7;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < nr && ch * 16 < nc) v = *(const uint4 *)(q + (r0 + row) * cols + c0 + ch * 16);
        *(uint4 *)(qs + row * kTile + ch * 16) = v;
    }
    if (t < kTile) srow[t] = t < nr ? scales[(r0 + t) * gcols + tc] : 1.0f;
    __syncthreads();

    // column cl, rows 64h .. 64h+63: de-scale, column maximum
    const int cl = t & (kTile - 1), h = t >> 7;
    float v[64];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        const int row = 64 * h + i;
        v[i] = decode1<FIN>(qs[row * kTile + cl]) / srow[row];
        if (row < nr) m = umax(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    }
    half_max[h][cl] = m;
    __syncthreads();
    m = umax(half_max[0][cl], half_max[1][cl]);
    const float s = POW2 ? scale_pow2_from_amax_bits<FOUT>(m) : scale_from_amax_bits<FOUT>(m);

    // the column's new codes, transposed into the output tile
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t b = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) b |= cast1<FOUT>(v[16 * k + 4 * d + e], s) << (8 * e);
            w[d] = b;
        }
        *(uint4 *)(ot + ot_offset(cl, 4 * h + k)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (h == 0 && cl < nc) {
        scalesT[(c0 + cl) * ((rows + 127) / 128) + tr] = s;
        if (nonfinite && m >= 0x7F800000u) *nonfinite = 1;
    }
    __syncthreads();

    // each column's 128 codes: one line of qT
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = t + j * kRqThreads, col = k >> 3, ch = k & 7;
        if (col < nc && ch * 16 < nr)
            *(uint4 *)(qT + (c0 + col) * rows + r0 + ch * 16) = *(const uint4 *)(ot + ot_offset(col, ch));
    }
}

}  // namespace

int launch_requant_t(const uint8_t *q, const float *scales, int64_t rows, int64_t cols, int fmt_in, int fmt_out,
                     int pow2, uint8_t *qT, float *scalesT, int32_t *nonfinite, hipStream_t s) {
    if (rows == 0 || cols == 0) return QF8_OK;
    const int tiles_r = (int)((rows + kTile - 1) / kTile), tiles_c = (int)((cols + kTile - 1) / kTile);
    const dim3 grid((unsigned)tiles_r * (unsigned)tiles_c), block(kRqThreads);
#define QF8_RQ(FI, FO, P) hipLaunchKernelGGL((requant_t_kernel<FI, FO, P>), grid, block, 0, s, q, scales, rows, cols, \
                                             tiles_c, qT, scalesT, nonfinite)
#define QF8_RQP(FI, FO) do { if (pow2) QF8_RQ(FI, FO, true); else QF8_RQ(FI, FO, false); } while (0)
    if (fmt_in == QF8_E4M3) { if (fmt_out == QF8_E4M3) QF8_RQP(kE4M3, kE4M3); else QF8_RQP(kE4M3, kE5M2); }
    else { if (fmt_out == QF8_E4M3) QF8_RQP(kE5M2, kE4M3); else QF8_RQP(kE5M2, kE5M2); }
#undef QF8_RQP
#undef QF8_RQ
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
