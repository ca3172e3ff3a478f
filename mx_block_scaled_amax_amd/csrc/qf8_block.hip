// qf8_block.hip -- fine-grained current scaling: 1x128 per-token groups and 128x128 blocks.
//
// Pages (title, section):
//   [MP-FP8] "混合精度与 FP8 训练" (hs-black.github.io): section 10.2 (activations scaled per
//            1x128 group of one token, weights per 128x128 block), 10.3 (online quantization:
//            every group computes its own amax), 8.1 (S = F8max/amax, saturating cast).
//
// Scale rule: Eq.(1) S_g = F8max / amax_g, or (power-of-two option, [MP-FP8 10.4]) the largest
// power of two S_g with amax_g * S_g <= F8max.
// Both kernels are one HBM pass: load the group into registers, reduce its |x| maximum, derive
// S_g with one IEEE division, cast from the registers. Loads and stores are non-temporal.
//   1x128: a group of 128 BF16 is 16 lanes x 8 values, i.e. one DPP row, so the maximum is four
//          DPP steps; a workgroup handles 16 groups per pass and 4 passes (all loads issued
//          first). FP32 input uses 32 lanes per group.
//   128x128: one workgroup per block; 8 BF16 rows of 16-byte loads per thread, wave maximum
//          then a 4-entry LDS maximum.
// Groups at the right and bottom edges may be partial: lanes outside the tensor load zeros,
// which never raise a maximum, and store nothing.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kThreads = 256;

template <bool BF16>
__device__ __forceinline__ uint32_t vec_absmax_bits(uint4 v) {
    if constexpr (BF16) {
        uint32_t m = pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
        return umax(m & 0xFFFFu, m >> 16) << 16;
    } else {
        return umax(umax(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), umax(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
    }
}

// Codes of one 16-byte input vector. STREAM: non-temporal store (the 1x128 kernel); the 128x128
// kernel, whose workgroup writes a 128-row block in 128-byte pieces spread over 128 rows, runs
// faster with ordinary cached stores (63 vs 68 us on 7168x18432), measured both ways.
template <bool BF16, int FMT, bool STREAM>
__device__ __forceinline__ void store_cast(uint8_t *q, int64_t off, uint4 v, float s) {
    if constexpr (STREAM) {
        if constexpr (BF16) st_stream((uint2 *)(q + off), cast8_bf16<FMT>(v, s));
        else st_stream((uint32_t *)(q + off), cast4_f32<FMT>(v, s));
    } else {
        if constexpr (BF16) *(uint2 *)(q + off) = cast8_bf16<FMT>(v, s);
        else *(uint32_t *)(q + off) = cast4_f32<FMT>(v, s);
    }
}

template <int FMT, bool POW2>
__device__ __forceinline__ float group_scale(uint32_t m) {
    if constexpr (POW2) return scale_pow2_from_amax_bits<FMT>(m);
    else return scale_from_amax_bits<FMT>(m);
}

template <bool BF16, int FMT, bool POW2>
__global__ __launch_bounds__(kThreads) void block_1x128_kernel(const uint16_t *__restrict__ x16, int64_t cols,
                                                               int64_t gcols, int64_t ngroups, uint8_t *__restrict__ q,
                                                               float *__restrict__ scales, float *__restrict__ amax,
                                                               int32_t *nonfinite) {
    constexpr int VEC = BF16 ? 8 : 4;
    constexpr int LPG = 128 / VEC;          // lanes per group
    constexpr int GPP = kThreads / LPG;     // groups per pass
    constexpr int ITER = 4;
    const int sub = threadIdx.x % LPG, gslot = threadIdx.x / LPG;
    const char *xb = (const char *)x16;
    uint4 v[ITER];
    int64_t off[ITER], g[ITER];
    bool ok[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        g[it] = ((int64_t)blockIdx.x * ITER + it) * GPP + gslot;
        const int64_t r = g[it] / gcols, j = g[it] - r * gcols;
        const int64_t col = j * 128 + sub * VEC;
        ok[it] = g[it] < ngroups && col < cols;
        off[it] = r * cols + col;
        v[it] = ok[it] ? ld_stream((const uint4 *)(xb + off[it] * (BF16 ? 2 : 4))) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        uint32_t m = vec_absmax_bits<BF16>(v[it]);
        m = max_row16(m);
        if constexpr (!BF16) m = umax(m, (uint32_t)__shfl_xor((int)m, 16));
        const float s = group_scale<FMT, POW2>(m);
        if (ok[it]) {
            store_cast<BF16, FMT, true>(q, off[it], v[it], s);
            if (sub == 0) {
                scales[g[it]] = s;
                if (amax) amax[g[it]] = __uint_as_float(m);
                if (nonfinite && m >= 0x7F800000u) *nonfinite = 1;
            }
        }
    }
}

template <bool BF16, int FMT, bool POW2>
__global__ __launch_bounds__(kThreads) void block_128x128_kernel(const uint16_t *__restrict__ x16, int64_t rows,
                                                                 int64_t cols, int64_t gcols, uint8_t *__restrict__ q,
                                                                 float *__restrict__ scales, float *__restrict__ amax,
                                                                 int32_t *nonfinite) {
    constexpr int VEC = BF16 ? 8 : 4;
    constexpr int TPR = 128 / VEC;          // threads per block row
    constexpr int RPP = kThreads / TPR;     // rows per pass
    constexpr int PASSES = 128 / RPP;
    __shared__ uint32_t red[4];
    const int64_t bi = blockIdx.x / gcols, bj = blockIdx.x - bi * gcols;
    const int sub = threadIdx.x % TPR, rr = threadIdx.x / TPR;
    const int64_t col = bj * 128 + sub * VEC;
    const bool cok = col < cols;
    const char *xb = (const char *)x16;
    uint4 v[PASSES];
    uint32_t m = 0;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int64_t r = bi * 128 + p * RPP + rr;
        v[p] = (cok && r < rows) ? ld_stream((const uint4 *)(xb + (r * cols + col) * (BF16 ? 2 : 4))) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) m = umax(m, vec_absmax_bits<BF16>(v[p]));
    m = max_wave(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    const float s = group_scale<FMT, POW2>(m);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int64_t r = bi * 128 + p * RPP + rr;
        if (cok && r < rows) store_cast<BF16, FMT, false>(q, r * cols + col, v[p], s);
    }
    if (threadIdx.x == 0) {
        scales[blockIdx.x] = s;
        if (amax) amax[blockIdx.x] = __uint_as_float(m);
        if (nonfinite && m >= 0x7F800000u) *nonfinite = 1;
    }
}

}  // namespace

int launch_block(const void *x, int dtype, int64_t rows, int64_t cols, int block_rows, int fmt, int pow2, uint8_t *q,
                 float *scales, float *amax, int32_t *nonfinite, hipStream_t s) {
    const int64_t gcols = (cols + 127) / 128;
    const uint16_t *x16 = (const uint16_t *)x;
    if (rows == 0 || cols == 0) return QF8_OK;
    const bool bf = dtype == QF8_IN_BF16, e4 = fmt == QF8_E4M3;
    if (block_rows == 1) {
        const int64_t ngroups = rows * gcols;
        const int gpb = (bf ? 16 : 8) * 4;
        const dim3 grid((unsigned)((ngroups + gpb - 1) / gpb));
#define QF8_L1(BF, F, P) hipLaunchKernelGGL((block_1x128_kernel<BF, F, P>), grid, dim3(kThreads), 0, s, x16, cols, gcols, \
                                            ngroups, q, scales, amax, nonfinite)
#define QF8_L1P(BF, F) do { if (pow2) QF8_L1(BF, F, true); else QF8_L1(BF, F, false); } while (0)
        if (bf) { if (e4) QF8_L1P(true, kE4M3); else QF8_L1P(true, kE5M2); }
        else { if (e4) QF8_L1P(false, kE4M3); else QF8_L1P(false, kE5M2); }
#undef QF8_L1P
#undef QF8_L1
    } else {
        const dim3 grid((unsigned)(((rows + 127) / 128) * gcols));
#define QF8_L128(BF, F, P) hipLaunchKernelGGL((block_128x128_kernel<BF, F, P>), grid, dim3(kThreads), 0, s, x16, rows, \
                                              cols, gcols, q, scales, amax, nonfinite)
#define QF8_L128P(BF, F) do { if (pow2) QF8_L128(BF, F, true); else QF8_L128(BF, F, false); } while (0)
        if (bf) { if (e4) QF8_L128P(true, kE4M3); else QF8_L128P(true, kE5M2); }
        else { if (e4) QF8_L128P(false, kE4M3); else QF8_L128P(false, kE5M2); }
#undef QF8_L128P
#undef QF8_L128
    }
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
