// qf8_mx.hip -- MX quantization: 1x32 blocks with E8M0 shared scales, rowwise and columnwise
// (stored transposed) from one read of the high-precision tensor.
//
// Pages (title, section):
//   [MP-FP8]       "混合精度与 FP8 训练" (hs-black.github.io): section 13.1 (MX block = 32
//                  elements sharing an E8M0 power-of-two scale; shared exponent
//                  floor(log2 amax) - emax; elements divided by 2^X, then quantized with
//                  saturation; a tensor and its transpose are each quantized from the original).
//   [MXFP8-recipe] "NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" (51cto.com): section 4.1
//                  (amax over the 32 values; amax = 0 gives X = -127 and zero elements; OCP
//                  round-down versus the round-up exponent of Algorithm 1; saturating RNE of
//                  V/2^X), section 4.2 (each tensor kept quantized along both reduction axes).
//
// Work decomposition (one HBM read of x, every output written once):
//   A workgroup owns a tile of 128 rows x (64 * VEC) columns (VEC = 8 BF16 or 4 FP32 values per
//   16-byte load); each of its 4 waves owns 32 consecutive rows of the tile, and each lane owns
//   VEC consecutive columns of those rows, held in 32 x 16-byte registers.
//   * Columnwise blocks (32 rows x 1 column) are then entirely inside one lane: the block amax
//     is a register-only reduction, and the lane writes each column's 32 codes as 32
//     contiguous bytes of the transposed output q_colT[c][r0 .. r0+31].
//   * Rowwise blocks (1 row x 32 columns) span 32/VEC lanes (4 for BF16): the amax is two (or
//     three) DPP steps, and each lane writes its VEC codes of the row.
//   * The conversion is the gfx950 scaled convert (two values per instruction, divided by 2^X
//     given as an fp32 exponent); OCP round-down first clamps |x| to F8max * 2^X on the bit
//     pattern, since the instruction does not saturate. Round-up never exceeds F8max.
//   * Tiles are assigned so that each of the 8 XCDs (workgroups are dealt to XCDs round-robin)
//     receives a contiguous band of rows: the E8M0 rows and column-pieces written by
//     neighbouring tiles then meet in the same L2.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 128;
constexpr int kRowsPerWave = 32;

template <bool BF16, int FMT, int RND>
__device__ __forceinline__ uint32_t mx_byte(uint32_t absbits) {
    if constexpr (BF16) return mx_byte_bf16<FMT, RND>(absbits);
    else return mx_byte_f32<FMT, RND>(absbits);
}

template <bool BF16, int FMT, int RND, bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void mx_kernel(const uint4 *__restrict__ x, int rows, int cols,
                                                      uint8_t *__restrict__ q_row, uint8_t *__restrict__ s_row,
                                                      uint8_t *__restrict__ q_colT, uint8_t *__restrict__ s_colT,
                                                      int32_t *nonfinite, int tiles_c, int tiles, int per_xcd) {
    constexpr int VEC = BF16 ? 8 : 4;            // values per lane per row
    constexpr int LPB = 32 / VEC;                // lanes per rowwise block
    constexpr uint32_t ABS = BF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;

    const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
    const int t = xcd * per_xcd + local;
    if (local >= per_xcd || t >= tiles) return;  // whole workgroup idle
    const int tr = t / tiles_c, tc = t - tr * tiles_c;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r0 = tr * kTileRows + wave * kRowsPerWave;
    if (r0 >= rows) return;                      // whole wave idle
    const int c0 = (tc * 64 + lane) * VEC;
    const bool active = c0 < cols;               // whole rowwise blocks: cols % 32 == 0
    const int vcols = cols / VEC;

    // ---- load 32 rows x 16 bytes ----------------------------------------------------------
    uint32_t d[kRowsPerWave][4];
    const uint4 *p = x + (int64_t)r0 * vcols + c0 / VEC;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (active && r0 + i < rows) v = p[(int64_t)i * vcols];
        d[i][0] = v.x; d[i][1] = v.y; d[i][2] = v.z; d[i][3] = v.w;
    }

    uint32_t cmax[4] = {0, 0, 0, 0};             // columnwise |x| maxima (BF16: two per dword)
    bool bad = false;

    // ---- rowwise blocks, one row at a time; columnwise maxima accumulate -----------------
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        uint32_t m[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) m[k] = d[i][k] & ABS;
        if constexpr (COL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) cmax[k] = BF16 ? pk_max_u16(cmax[k], m[k]) : umax(cmax[k], m[k]);
        }
        if constexpr (ROW) {
            uint32_t a;
            if constexpr (BF16) {
                const uint32_t mm = pk_max_u16(pk_max_u16(m[0], m[1]), pk_max_u16(m[2], m[3]));
                a = max_quad(umax(mm & 0xFFFFu, mm >> 16));
            } else {
                a = max_oct(umax(umax(m[0], m[1]), umax(m[2], m[3])));
            }
            const uint32_t byte = mx_byte<BF16, FMT, RND>(a);
            bad |= byte == 255u;
            const float sc = __uint_as_float(byte << 23);
            const uint32_t zero_mask = a == 0u ? 0u : ~0u;            // all-zero block -> 0x00
            uint32_t v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = d[i][k];
            if constexpr (RND == kRoundDown) {                          // saturate before the cast
                if constexpr (BF16) {
                    const uint32_t cb = mx_clamp_bf16<FMT>(byte), cbp = cb | (cb << 16);
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[k] = bit_select(ABS, pk_min_u16(m[k], cbp), v[k]);
                } else {
                    const uint32_t cb = mx_clamp_f32<FMT>(byte);
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[k] = bit_select(ABS, umin(m[k], cb), v[k]);
                }
            }
            const bool st = active && r0 + i < rows;
            uint8_t *qr = q_row + (int64_t)(r0 + i) * cols + c0;
            if constexpr (BF16) {
                uint32_t o0 = cvt2_bf16_div2x<FMT, true>(v[1], sc, cvt2_bf16_div2x<FMT, false>(v[0], sc, 0u));
                uint32_t o1 = cvt2_bf16_div2x<FMT, true>(v[3], sc, cvt2_bf16_div2x<FMT, false>(v[2], sc, 0u));
                if (st) *(uint2 *)qr = make_uint2(o0 & zero_mask, o1 & zero_mask);
            } else {
                uint32_t o0 = cvt2_f32_div2x<FMT, true>(__uint_as_float(v[2]), __uint_as_float(v[3]), sc,
                              cvt2_f32_div2x<FMT, false>(__uint_as_float(v[0]), __uint_as_float(v[1]), sc, 0u));
                if (st) *(uint32_t *)qr = o0 & zero_mask;
            }
            // one lane of each block writes the scale byte; the lanes take turns by row
            if (st && (lane & (LPB - 1)) == (i & (LPB - 1)))
                s_row[(int64_t)(r0 + i) * (cols / 32) + c0 / 32] = (uint8_t)byte;
        }
    }

    // ---- columnwise blocks: VEC columns x 32 rows per lane ---------------------------------
    if constexpr (COL) {
        const int64_t srow = rows / 32;
        if constexpr (BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {                 // dword k holds columns 2k (low) and 2k+1
                const uint32_t alo = cmax[k] & 0xFFFFu, ahi = cmax[k] >> 16;
                const uint32_t blo = mx_byte<true, FMT, RND>(alo), bhi = mx_byte<true, FMT, RND>(ahi);
                bad |= (blo == 255u) | (bhi == 255u);
                const float slo = __uint_as_float(blo << 23), shi = __uint_as_float(bhi << 23);
                const uint32_t zlo = alo == 0u ? 0u : ~0u, zhi = ahi == 0u ? 0u : ~0u;
                uint32_t cbp = 0;
                if constexpr (RND == kRoundDown) cbp = mx_clamp_bf16<FMT>(blo) | (mx_clamp_bf16<FMT>(bhi) << 16);
                uint32_t olo[8], ohi[8];
#pragma unroll
                for (int g = 0; g < 8; ++g) {             // rows 4g .. 4g+3
                    uint32_t w[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[j] = d[4 * g + j][k];
                        if constexpr (RND == kRoundDown) w[j] = bit_select(ABS, pk_min_u16(w[j] & ABS, cbp), w[j]);
                    }
                    // gather one column's values of two consecutive rows into one dword
                    const uint32_t l01 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
                    const uint32_t l23 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
                    const uint32_t h01 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
                    const uint32_t h23 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
                    olo[g] = cvt2_bf16_div2x<FMT, true>(l23, slo, cvt2_bf16_div2x<FMT, false>(l01, slo, 0u)) & zlo;
                    ohi[g] = cvt2_bf16_div2x<FMT, true>(h23, shi, cvt2_bf16_div2x<FMT, false>(h01, shi, 0u)) & zhi;
                }
                if (active) {
                    uint4 *ql = (uint4 *)(q_colT + (int64_t)(c0 + 2 * k) * rows + r0);
                    uint4 *qh = (uint4 *)(q_colT + (int64_t)(c0 + 2 * k + 1) * rows + r0);
                    ql[0] = make_uint4(olo[0], olo[1], olo[2], olo[3]);
                    ql[1] = make_uint4(olo[4], olo[5], olo[6], olo[7]);
                    qh[0] = make_uint4(ohi[0], ohi[1], ohi[2], ohi[3]);
                    qh[1] = make_uint4(ohi[4], ohi[5], ohi[6], ohi[7]);
                    s_colT[(int64_t)(c0 + 2 * k) * srow + r0 / 32] = (uint8_t)blo;
                    s_colT[(int64_t)(c0 + 2 * k + 1) * srow + r0 / 32] = (uint8_t)bhi;
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {                 // column c0 + k
                const uint32_t a = cmax[k];
                const uint32_t byte = mx_byte<false, FMT, RND>(a);
                bad |= byte == 255u;
                const float sc = __uint_as_float(byte << 23);
                const uint32_t zm = a == 0u ? 0u : ~0u;
                uint32_t cb = 0;
                if constexpr (RND == kRoundDown) cb = mx_clamp_f32<FMT>(byte);
                uint32_t o[8];
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    float f[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t w = d[4 * g + j][k];
                        if constexpr (RND == kRoundDown) w = bit_select(ABS, umin(w & ABS, cb), w);
                        f[j] = __uint_as_float(w);
                    }
                    o[g] = cvt2_f32_div2x<FMT, true>(f[2], f[3], sc, cvt2_f32_div2x<FMT, false>(f[0], f[1], sc, 0u)) & zm;
                }
                if (active) {
                    uint4 *qc = (uint4 *)(q_colT + (int64_t)(c0 + k) * rows + r0);
                    qc[0] = make_uint4(o[0], o[1], o[2], o[3]);
                    qc[1] = make_uint4(o[4], o[5], o[6], o[7]);
                    s_colT[(int64_t)(c0 + k) * srow + r0 / 32] = (uint8_t)byte;
                }
            }
        }
    }
    if (bad && nonfinite) *nonfinite = 1;
}

template <bool BF16, int FMT, int RND>
void launch_dirs(const uint4 *x, int rows, int cols, uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT,
                 uint8_t *s_colT, int32_t *nonfinite, hipStream_t s) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int tiles_r = (rows + kTileRows - 1) / kTileRows;
    const int tiles_c = (cols + 64 * VEC - 1) / (64 * VEC);
    const int tiles = tiles_r * tiles_c;
    const int per_xcd = (tiles + 7) / 8;
    const dim3 grid(8 * per_xcd), block(kThreads);
    if (q_row && q_colT)
        hipLaunchKernelGGL((mx_kernel<BF16, FMT, RND, true, true>), grid, block, 0, s, x, rows, cols, q_row, s_row,
                           q_colT, s_colT, nonfinite, tiles_c, tiles, per_xcd);
    else if (q_row)
        hipLaunchKernelGGL((mx_kernel<BF16, FMT, RND, true, false>), grid, block, 0, s, x, rows, cols, q_row, s_row,
                           q_colT, s_colT, nonfinite, tiles_c, tiles, per_xcd);
    else
        hipLaunchKernelGGL((mx_kernel<BF16, FMT, RND, false, true>), grid, block, 0, s, x, rows, cols, q_row, s_row,
                           q_colT, s_colT, nonfinite, tiles_c, tiles, per_xcd);
}

}  // namespace

int launch_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int rnd, uint8_t *q_row,
              uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite, hipStream_t s) {
    if (rows == 0 || cols == 0) return QF8_OK;
    const uint4 *xv = (const uint4 *)x;
    const int r = (int)rows, c = (int)cols;
#define QF8_MX(BF, F, R) launch_dirs<BF, F, R>(xv, r, c, q_row, s_row, q_colT, s_colT, nonfinite, s)
    if (dtype == QF8_IN_BF16) {
        if (fmt == QF8_E4M3) { if (rnd == QF8_MX_ROUND_DOWN) QF8_MX(true, kE4M3, kRoundDown); else QF8_MX(true, kE4M3, kRoundUp); }
        else { if (rnd == QF8_MX_ROUND_DOWN) QF8_MX(true, kE5M2, kRoundDown); else QF8_MX(true, kE5M2, kRoundUp); }
    } else {
        if (fmt == QF8_E4M3) { if (rnd == QF8_MX_ROUND_DOWN) QF8_MX(false, kE4M3, kRoundDown); else QF8_MX(false, kE4M3, kRoundUp); }
        else { if (rnd == QF8_MX_ROUND_DOWN) QF8_MX(false, kE5M2, kRoundDown); else QF8_MX(false, kE5M2, kRoundUp); }
    }
#undef QF8_MX
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
