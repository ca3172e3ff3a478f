// qf8_fp4.hip -- FP4 (E2M1) quantization: MXFP4 (1x32 blocks with E8M0 scales, rowwise and
// columnwise from one read of x) and NVFP4 (1x16 blocks along rows with E4M3 block scales under
// one fp32 tensor scale).
//
// Pages (title, section):
//   [MP-FP8]       "混合精度与 FP8 训练" (hs-black.github.io): section 13.1 (MX rule: shared
//                  exponent floor(log2 amax) - emax, emax of E2M1 = 2, elements divided by 2^X and
//                  quantized with saturation; a tensor and its transpose each quantized from the
//                  original), section 13.2 (E2M1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6; NVFP4: a
//                  block of 16 shares an E4M3 scale amax/6, plus an fp32 tensor scale).
//   [MXFP8-recipe] "NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" (51cto.com): section 4.1 (the
//                  round-up exponent; amax = 0 gives X = -127 and zero elements).
//   [Ascend950]    Ascend 950 low-precision format guide: section 2.4 (MXFP4 = 32 FP4 values +
//                  one shared scale).
//
// Definitions (the readings the library documents):
//   MXFP4: X = floor(log2 amax) - 2 (round-down) or the smallest X with amax / 2^X <= 6
//     (round-up), clamped to [-127, 127]; byte = X + 127 (0xFF for a block with Inf/NaN);
//     code = sat_rne(E2M1, x / 2^X); amax = 0 gives zero codes.
//   NVFP4: S_t = fl32(2688 / A) (A the tensor amax; 1 for A = 0 or non-finite, FLT_MAX on
//     overflow); e_b = sat_rne(E4M3, amax_b * S_t / 6) and code = sat_rne(E2M1, x * S_t /
//     decode(e_b)), each rounded once from the exact quotient; a block whose e_b decodes to 0
//     gives zero codes of the elements' signs.
//   Codes are packed two per byte, element 2j in the low nibble of byte j.
//
// Conversion: v_cvt_scalef32_pk_fp4_{bf16,f32} turns two values into one byte of two E2M1 codes
// (the first value in the low nibble) in a chosen byte of its 32-bit result, dividing by 2^E
// where E is the exponent field of the fp32 scale operand minus 127, rounding to nearest even
// and saturating to +-6 (Inf too). Checked on gfx950 against an exact nearest-value reference
// for every BF16 value with all 255 scale exponents, and for every fp32 value below 16 in
// magnitude with scale 1 (a scale of 1.5 acts as 1: only the exponent field is used). So the MX
// path needs no separate clamp, and the NVFP4 path converts two fp32 estimates of x * S_t /
// decode(e_b) (one below, one above the exact quotient) with scale 1 and settles the rare elements
// where they disagree exactly (nv_elem_exact).
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 128;              // MXFP4 rowwise only
constexpr int kColTileRows = 256;           // MXFP4 with the columnwise direction
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerLane = kRowsPerWave / 2;
constexpr uint32_t kE2M1Emax = 2;              // 6 = 1.5 * 2^2
// NVFP4 blocks per thread and trip of the streaming kernel: two for BF16 input (their codes leave
// as 16-byte pieces through lane pairs; 30.5 against 31.3 µs on 16384x4096), one for FP32 (two
// took 75.6 against 74.3 µs).
template <bool BF16> constexpr int nv_passes_per_trip() { return BF16 ? 2 : 1; }

// E8M0 byte of an MXFP4 block from its |amax| bit pattern. For amax = 1.f * 2^E: round-down
// X = E - 2; round-up adds 1 when 1.f > 1.5, which is one carry into the exponent field from
// adding 0x3F (BF16, 7 mantissa bits, 1.5 = 0x40) or 0x3FFFFF (FP32). X is clamped below at -127
// by a saturating subtraction (subnormal or zero amax); a non-finite amax gives 0xFF.
template <bool BF16, int RND>
__device__ __forceinline__ uint32_t fp4_mx_byte(uint32_t a) {
    if constexpr (BF16) {
        const uint32_t e = (RND == kRoundUp ? a + 0x3Fu : a) >> 7;
        return a >= 0x7F80u ? 255u : __builtin_elementwise_sub_sat(e, kE2M1Emax);
    } else {
        const uint32_t e = (RND == kRoundUp ? a + 0x3FFFFFu : a) >> 23;
        return a >= 0x7F800000u ? 255u : __builtin_elementwise_sub_sat(e, kE2M1Emax);
    }
}

// Two BF16 values (one dword, the lower-addressed element in the low half) -> byte SEL of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_bf16(uint32_t old, uint32_t pair, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(v2bf16, pair), scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4_f32(uint32_t old, float a, float b, float scale) {
    return cvt_fp4_f32<SEL>(old, a, b, scale);
}

// Offset of the 8-byte unit u (rows 16u .. 16u+15, packed) of tile column c in the columnwise
// LDS tile of TR rows: one TR/2-byte line per column (two codes per byte). 128 rows: the lines
// of each group of 4 columns are permuted by bits 3-4 of c and the units' 16-byte pairs by bits
// 5-6, so that the 32 lanes of a half-wave, whose columns are 8 apart, write different banks.
// 256 rows: the 16-byte pairs of a line are permuted by bits 3-5 of c. A 16-byte pair (units
// 2j, 2j+1) stays contiguous and in order.
template <int TR>
__device__ __forceinline__ int fp4_col_offset(int c, int u) {
    if constexpr (TR == 128) return ((c ^ ((c >> 3) & 3)) << 6) + ((u ^ (((c >> 5) & 3) << 1)) << 3);
    else return c * (TR / 2) + ((((u >> 1) ^ ((c >> 3) & (TR / 32 - 1)))) << 4) + ((u & 1) << 3);
}

// ---------------------------------------------------------------------------------------------
// MXFP4: the tiling of the MXFP8 kernel, with TR rows per tile. A workgroup of TR / 32 waves
// owns TR rows x (32 * VEC) columns; lane l of a wave owns VEC columns (slot l % 32) of 16 rows
// (half l / 32 of the wave's 32 rows) in 16 x 16-byte registers. Rowwise: block amax over
// 32/VEC lanes by DPP, VEC codes of a row leave as VEC/2 bytes. Columnwise: a column's block
// spans lanes l and l ^ 32; each lane packs its 16 rows into 8 bytes per column, staged in
// LDS, and the workgroup writes each column's TR / 2 bytes of q_colT (and the E8M0 bytes of
// both directions) after one barrier. With the columnwise direction TR = 256: a tile column is
// then one whole 128-byte line of q_colT and its E8M0 bytes one 8-byte store (with 128 rows,
// half lines and 4-byte stores, the dual kernel took 41.8 instead of 39.1 µs on 16384x4096
// BF16 on MI355X; 512 rows took 43.4 µs).
template <bool BF16, int RND, bool ROW, bool COL, int TR>
__global__ __launch_bounds__(2 * TR) void mxfp4_kernel(const void *__restrict__ x, int rows, int cols,
                                                         uint8_t *__restrict__ q_row, uint8_t *__restrict__ s_row,
                                                         uint8_t *__restrict__ q_colT, uint8_t *__restrict__ s_colT,
                                                         int32_t *nonfinite, int tiles_c, int tiles, int per_xcd) {
    constexpr int VEC = BF16 ? 8 : 4;            // values per lane per row (one 16-byte load)
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int LPB = 32 / VEC;                // lanes per rowwise block
    constexpr int RPL = kRowsPerLane;
    constexpr int TILE_C = 32 * VEC;
    constexpr int NBLK = TILE_C / 32;            // rowwise blocks per tile row
    constexpr uint32_t ABS = BF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
    constexpr int NT = 2 * TR;                   // threads: one wave per 32 rows
    constexpr int NRB = TR / 32;                 // columnwise blocks per tile column

    __shared__ __attribute__((aligned(16))) uint8_t colbuf[COL ? TILE_C * (TR / 2) : 16];
    __shared__ __attribute__((aligned(16))) uint8_t scol[COL ? TILE_C * NRB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t srow[ROW ? TR * NBLK : 16];

    const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
    const int t = xcd * per_xcd + local;
    if (local >= per_xcd || t >= tiles) return;  // whole workgroup idle
    const int tr = t / tiles_c, tc = t - tr * tiles_c;
    const int tr0 = tr * TR, ct0 = tc * TILE_C;
    const int ncv = cols - ct0 < TILE_C ? cols - ct0 : TILE_C;
    const int trows = rows - tr0 < TR ? rows - tr0 : TR;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, half = lane >> 5, slot = lane & 31;
    const int r0 = tr0 + wave * kRowsPerWave;
    uint32_t seen = 0;

    if (r0 < rows) {
        const int c0 = ct0 + slot * VEC;
        const bool active = c0 < cols;           // rowwise blocks are whole: cols % 32 == 0
        const int wrows = rows - r0 < kRowsPerWave ? rows - r0 : kRowsPerWave;

        const uint32_t rowbytes = (uint32_t)cols * ESZ;
        const __amdgpu_buffer_rsrc_t xr = make_rsrc((const char *)x + (size_t)r0 * rowbytes,
                                                    (uint32_t)wrows * rowbytes);
        const uint32_t xvo = active ? (uint32_t)(half * RPL) * rowbytes + (uint32_t)c0 * ESZ : kOutOfRange;
        uint32_t d[RPL][4];
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const uint4 v = buf_load16<kNonTemporal>(xr, xvo, (uint32_t)i * rowbytes);
            d[i][0] = v.x; d[i][1] = v.y; d[i][2] = v.z; d[i][3] = v.w;
        }
        uint32_t cmax[4] = {0, 0, 0, 0};

        if constexpr (ROW) {
            const uint32_t qstride = (uint32_t)cols / 2;
            const __amdgpu_buffer_rsrc_t qr = make_rsrc(q_row + (size_t)r0 * qstride, (uint32_t)wrows * qstride);
            const uint32_t qvo = active ? (uint32_t)(half * RPL) * qstride + c0 / 2 : kOutOfRange;
            const uint32_t sstride = cols / 32;
            // Rows 2p and 2p + 1 leave through lane pairs: the even lane of a pair writes row 2p of
            // both lanes' columns, the odd lane row 2p + 1, after one DPP swap (8-byte pieces for
            // BF16, 4 for FP32). A pair's lanes are both active or both idle (cols % 32 == 0). The
            // swapped value comes from the zero-block select, never straight from a convert.
            static_assert(RPL % 2 == 0, "rowwise codes leave two rows at a time");
            const bool odd = (slot & 1) != 0;
            constexpr uint32_t kCodeBytes = VEC / 2;     // code bytes per lane and row
            const uint32_t qpo = !active ? kOutOfRange : odd ? qvo - kCodeBytes : qvo;
            uint32_t prev = 0u;                          // the codes of the pair's first row
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                uint32_t m[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) m[k] = d[i][k] & ABS;
                if constexpr (COL) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) cmax[k] = BF16 ? pk_max_u16(cmax[k], m[k]) : umax(cmax[k], m[k]);
                }
                uint32_t a;
                if constexpr (BF16) {
                    const uint32_t mm = pk_max_u16(pk_max_u16(m[0], m[1]), pk_max_u16(m[2], m[3]));
                    a = max_quad(umax(mm & 0xFFFFu, mm >> 16));
                } else {
                    a = max_oct(umax(umax(m[0], m[1]), umax(m[2], m[3])));
                }
                if constexpr (!COL) seen = umax(seen, a);
                const uint32_t byte = fp4_mx_byte<BF16, RND>(a);
                const float sc = __uint_as_float(byte << 23);
                if constexpr (BF16) {
                    uint32_t o = fp4_bf16<0>(0u, d[i][0], sc);
                    o = fp4_bf16<1>(o, d[i][1], sc);
                    o = fp4_bf16<2>(o, d[i][2], sc);
                    o = fp4_bf16<3>(o, d[i][3], sc);
                    if (a == 0u) o = 0u;                            // all-zero block: zero codes
                    if ((i & 1) == 0) {
                        prev = o;
                    } else {
                        const uint32_t r = dpp_mov<0xB1>(odd ? prev : o);
                        buf_store8(qr, qpo + (uint32_t)(odd ? i : i - 1) * qstride, 0u, odd ? r : prev, odd ? o : r);
                    }
                } else {
                    uint32_t o = fp4_f32<0>(0u, __uint_as_float(d[i][0]), __uint_as_float(d[i][1]), sc);
                    o = fp4_f32<1>(o, __uint_as_float(d[i][2]), __uint_as_float(d[i][3]), sc);
                    if (a == 0u) o = 0u;
                    if ((i & 1) == 0) {
                        prev = o;
                    } else {
                        const uint32_t r = dpp_mov<0xB1>(odd ? prev : o);
                        buf_store4(qr, qpo + (uint32_t)(odd ? i : i - 1) * qstride, 0u,
                                   odd ? ((r & 0xFFFFu) | (o << 16)) : ((prev & 0xFFFFu) | (r << 16)));
                    }
                }
                // every lane of the block writes the same byte to the same LDS slot
                srow[(wave * kRowsPerWave + half * RPL + i) * NBLK + slot / LPB] = (uint8_t)byte;
            }
            if constexpr (!COL) {
                // rowwise only: the wave's 32 rows of E8M0 bytes leave from LDS as one NBLK-byte store
                // per row (single byte stores from the lanes of every block cost more); the rows of
                // this wave are its own, so a wave-level fence orders the LDS bytes
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const int nbl = ncv / 32;
                const bool whole = nbl == NBLK && (sstride % NBLK) == 0 && (((uintptr_t)s_row) % NBLK) == 0;
                const __amdgpu_buffer_rsrc_t sw = make_rsrc(s_row + (size_t)r0 * sstride + ct0 / 32,
                                                            (uint32_t)wrows * sstride - ct0 / 32);
                if (lane < kRowsPerWave) {
                    const bool rv = lane < wrows;
                    const uint8_t *src = srow + (wave * kRowsPerWave + lane) * NBLK;
                    if constexpr (NBLK == 8) {
                        const uint2 w = *(const uint2 *)src;
                        if (whole) {
                            buf_store8(sw, rv ? (uint32_t)lane * sstride : kOutOfRange, 0u, w.x, w.y);
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                buf_store1(sw, (rv & (j < nbl)) ? (uint32_t)lane * sstride + j : kOutOfRange, 0u,
                                           (j < 4 ? w.x : w.y) >> (8 * (j & 3)));
                        }
                    } else {
                        const uint32_t w = *(const uint32_t *)src;
                        if (whole) {
                            buf_store4(sw, rv ? (uint32_t)lane * sstride : kOutOfRange, 0u, w);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                buf_store1(sw, (rv & (j < nbl)) ? (uint32_t)lane * sstride + j : kOutOfRange, 0u,
                                           w >> (8 * j));
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    cmax[k] = BF16 ? pk_max_u16(cmax[k], d[i][k] & ABS) : umax(cmax[k], d[i][k] & ABS);
        }

        if constexpr (COL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t other = (uint32_t)__shfl_xor((int)cmax[k], 32);
                cmax[k] = BF16 ? pk_max_u16(cmax[k], other) : umax(cmax[k], other);
            }
            const int unit = wave * 2 + half;    // 16-row chunk of the tile = 8-byte unit
            if constexpr (BF16) {
                const uint32_t mm = pk_max_u16(pk_max_u16(cmax[0], cmax[1]), pk_max_u16(cmax[2], cmax[3]));
                seen = umax(mm & 0xFFFFu, mm >> 16);
#pragma unroll
                for (int k = 0; k < 4; ++k) {     // dword k holds columns 2k (low half) and 2k+1
                    const uint32_t alo = cmax[k] & 0xFFFFu, ahi = cmax[k] >> 16;
                    const uint32_t blo = fp4_mx_byte<true, RND>(alo), bhi = fp4_mx_byte<true, RND>(ahi);
                    const float slo = __uint_as_float(blo << 23), shi = __uint_as_float(bhi << 23);
                    uint32_t olo[2] = {0u, 0u}, ohi[2] = {0u, 0u};
#pragma unroll
                    for (int g = 0; g < 8; ++g) {     // rows 2g, 2g+1 of the lane -> byte g
                        const uint32_t l = __builtin_amdgcn_perm(d[2 * g + 1][k], d[2 * g][k], 0x05040100u);
                        const uint32_t h = __builtin_amdgcn_perm(d[2 * g + 1][k], d[2 * g][k], 0x07060302u);
                        switch (g & 3) {
                            case 0: olo[g >> 2] = fp4_bf16<0>(olo[g >> 2], l, slo); ohi[g >> 2] = fp4_bf16<0>(ohi[g >> 2], h, shi); break;
                            case 1: olo[g >> 2] = fp4_bf16<1>(olo[g >> 2], l, slo); ohi[g >> 2] = fp4_bf16<1>(ohi[g >> 2], h, shi); break;
                            case 2: olo[g >> 2] = fp4_bf16<2>(olo[g >> 2], l, slo); ohi[g >> 2] = fp4_bf16<2>(ohi[g >> 2], h, shi); break;
                            default: olo[g >> 2] = fp4_bf16<3>(olo[g >> 2], l, slo); ohi[g >> 2] = fp4_bf16<3>(ohi[g >> 2], h, shi); break;
                        }
                    }
                    if (alo == 0u) olo[0] = olo[1] = 0u;
                    if (ahi == 0u) ohi[0] = ohi[1] = 0u;
                    const int clo = slot * VEC + 2 * k;
                    *(uint2 *)(colbuf + fp4_col_offset<TR>(clo, unit)) = make_uint2(olo[0], olo[1]);
                    *(uint2 *)(colbuf + fp4_col_offset<TR>(clo + 1, unit)) = make_uint2(ohi[0], ohi[1]);
                    if (half == 0) {
                        scol[clo * NRB + wave] = (uint8_t)blo;
                        scol[(clo + 1) * NRB + wave] = (uint8_t)bhi;
                    }
                }
            } else {
                seen = umax(umax(cmax[0], cmax[1]), umax(cmax[2], cmax[3]));
#pragma unroll
                for (int k = 0; k < 4; ++k) {     // tile column slot * 4 + k
                    const uint32_t a = cmax[k];
                    const uint32_t byte = fp4_mx_byte<false, RND>(a);
                    const float sc = __uint_as_float(byte << 23);
                    uint32_t o[2] = {0u, 0u};
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        const float f0 = __uint_as_float(d[2 * g][k]), f1 = __uint_as_float(d[2 * g + 1][k]);
                        switch (g & 3) {
                            case 0: o[g >> 2] = fp4_f32<0>(o[g >> 2], f0, f1, sc); break;
                            case 1: o[g >> 2] = fp4_f32<1>(o[g >> 2], f0, f1, sc); break;
                            case 2: o[g >> 2] = fp4_f32<2>(o[g >> 2], f0, f1, sc); break;
                            default: o[g >> 2] = fp4_f32<3>(o[g >> 2], f0, f1, sc); break;
                        }
                    }
                    if (a == 0u) o[0] = o[1] = 0u;
                    const int c = slot * VEC + k;
                    *(uint2 *)(colbuf + fp4_col_offset<TR>(c, unit)) = make_uint2(o[0], o[1]);
                    if (half == 0) scol[c * NRB + wave] = (uint8_t)byte;
                }
            }
        }
    }

    if constexpr (COL) {
        __syncthreads();
        // q_colT: column c of the tile -> q_colT[ct0 + c][tr0/2 .. (tr0 + trows)/2), 16 bytes a lane
        const uint32_t cstride = (uint32_t)rows / 2;
        const __amdgpu_buffer_rsrc_t qc = make_rsrc(q_colT + (size_t)ct0 * cstride + tr0 / 2,
                                                    (uint32_t)ncv * cstride - tr0 / 2);
#pragma unroll
        for (int e = threadIdx.x; e < TILE_C * NRB; e += NT) {
            const int c = e / NRB, j = e % NRB;  // 16-byte chunk j = rows 32j .. 32j+31
            const uint4 v = *(const uint4 *)(colbuf + fp4_col_offset<TR>(c, 2 * j));
            const uint32_t vo = (c < ncv && 32 * j < trows) ? (uint32_t)c * cstride + 16 * j : kOutOfRange;
            buf_store16<kNonTemporal>(qc, vo, 0u, v);
        }
        const uint32_t srb = (uint32_t)rows / 32;
        const int nb = trows / 32;
        const __amdgpu_buffer_rsrc_t scr = make_rsrc(s_colT + (size_t)ct0 * srb + tr0 / 32, (uint32_t)ncv * srb - tr0 / 32);
        const bool whole_c = nb == NRB && (srb % NRB) == 0 && (((uintptr_t)s_colT) % NRB) == 0;
        for (int c = threadIdx.x; c < TILE_C; c += NT) {
            if constexpr (NRB == 8) {
                const uint2 w = *(const uint2 *)(scol + c * 8);
                if (whole_c) {
                    buf_store8(scr, c < ncv ? (uint32_t)c * srb : kOutOfRange, 0u, w.x, w.y);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        buf_store1(scr, (c < ncv && j < nb) ? (uint32_t)c * srb + j : kOutOfRange, 0u,
                                   (j < 4 ? w.x : w.y) >> (8 * (j & 3)));
                }
            } else {
                const uint32_t w = *(const uint32_t *)(scol + c * 4);
                if (whole_c) {
                    buf_store4(scr, c < ncv ? (uint32_t)c * srb : kOutOfRange, 0u, w);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        buf_store1(scr, (c < ncv && j < nb) ? (uint32_t)c * srb + j : kOutOfRange, 0u, w >> (8 * j));
                }
            }
        }
        if constexpr (ROW) {
            const uint32_t ssb = (uint32_t)cols / 32;
            const int nbl = ncv / 32;
            const __amdgpu_buffer_rsrc_t srr = make_rsrc(s_row + (size_t)tr0 * ssb + ct0 / 32,
                                                         (uint32_t)trows * ssb - ct0 / 32);
            const bool whole_r = nbl == NBLK && (ssb % NBLK) == 0 && (((uintptr_t)s_row) % NBLK) == 0;
            for (int r = threadIdx.x; r < TR; r += NT) {
                const bool rv = r < trows;
                if constexpr (NBLK == 8) {
                    const uint2 w = *(const uint2 *)(srow + r * 8);
                    if (whole_r) {
                        buf_store8(srr, rv ? (uint32_t)r * ssb : kOutOfRange, 0u, w.x, w.y);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            buf_store1(srr, (rv && j < nbl) ? (uint32_t)r * ssb + j : kOutOfRange, 0u,
                                       (j < 4 ? w.x : w.y) >> (8 * (j & 3)));
                    }
                } else {
                    const uint32_t w = *(const uint32_t *)(srow + r * 4);
                    if (whole_r) {
                        buf_store4(srr, rv ? (uint32_t)r * ssb : kOutOfRange, 0u, w);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            buf_store1(srr, (rv && j < nbl) ? (uint32_t)r * ssb + j : kOutOfRange, 0u, w >> (8 * j));
                    }
                }
            }
        }
    }
    if (seen >= (BF16 ? 0x7F80u : 0x7F800000u) && nonfinite) *nonfinite = 1;
}

template <bool BF16, int RND>
void launch_mxfp4_dirs(const void *x, int rows, int cols, uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT,
                       uint8_t *s_colT, int32_t *nonfinite, hipStream_t s) {
    constexpr int VEC = BF16 ? 8 : 4;
    // the columnwise direction takes tiles of kColTileRows rows, so that a tile column's codes
    // are whole 128-byte lines of q_colT; rowwise alone keeps kTileRows
    const int tr = q_colT ? kColTileRows : kTileRows;
    const int tiles_r = (rows + tr - 1) / tr;
    const int tiles_c = (cols + 32 * VEC - 1) / (32 * VEC);
    const int tiles = tiles_r * tiles_c;
    const int per_xcd = (tiles + 7) / 8;
    const dim3 grid(8 * per_xcd), block(2 * tr);
    if (q_row && q_colT)
        hipLaunchKernelGGL((mxfp4_kernel<BF16, RND, true, true, kColTileRows>), grid, block, 0, s, x, rows, cols,
                           q_row, s_row, q_colT, s_colT, nonfinite, tiles_c, tiles, per_xcd);
    else if (q_row)
        hipLaunchKernelGGL((mxfp4_kernel<BF16, RND, true, false, kTileRows>), grid, block, 0, s, x, rows, cols,
                           q_row, s_row, q_colT, s_colT, nonfinite, tiles_c, tiles, per_xcd);
    else
        hipLaunchKernelGGL((mxfp4_kernel<BF16, RND, false, true, kColTileRows>), grid, block, 0, s, x, rows, cols,
                           q_row, s_row, q_colT, s_colT, nonfinite, tiles_c, tiles, per_xcd);
}

// ---------------------------------------------------------------------------------------------
// NVFP4: a thread works on blocks of 16 consecutive elements (cols % 16 == 0, so a block never
// crosses a row and block b of the flattened tensor is row b / (cols/16)), one per pass over the
// workgroup's 256 threads, two passes per trip for BF16 input (nv_passes_per_trip). Every
// workgroup first takes the tensor amax (the caller's value, or the fold of the amax pass's
// partials), S_t and the table of element factors; for each block a thread loads its 32 (BF16) or
// 64 (FP32) bytes, takes the block amax and the E4M3 block scale, converts the two bracketing
// estimates of every element and produces 8 bytes of codes and the scale byte. The elements whose
// two estimates disagree (those within about 2^-20 of an E2M1 midpoint) are recomputed exactly,
// each by its own lane.


template <bool BF16>
__global__ __launch_bounds__(kThreads) void nvfp4_kernel(const void *__restrict__ x, int64_t nblk,
                                                         const uint32_t *__restrict__ partials, int nparts,
                                                         const float *amax_in, uint8_t *__restrict__ q,
                                                         uint8_t *__restrict__ s_blk, float *tensor_scale,
                                                         float *amax_out, int32_t *nonfinite) {
    __shared__ uint32_t red[kThreads / 64];
    __shared__ float2 tab[128];                  // (r_lo, r_hi) per E4M3 block-scale code
    const uint32_t A = amax_in ? (__float_as_uint(*amax_in) & 0x7FFFFFFFu)
                               : block_max_bcast<kThreads>(fold_max<kThreads>(partials, nparts), red);
    const float st = nv_tensor_scale(A);
    nv_factor_table(tab, st);
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (tensor_scale) *tensor_scale = st;
        if (amax_out) *amax_out = __uint_as_float(A);
        if (nonfinite && A >= 0x7F800000u) *nonfinite = 1;
    }
    constexpr int NV = BF16 ? 2 : 4;             // 16-byte loads per block
    const uint4 *xv = (const uint4 *)x;
    __shared__ __attribute__((aligned(16))) uint8_t sbuf[2 * kThreads];
    __shared__ __attribute__((aligned(16))) float fbuf[kThreads * 16];   // a lane's elements, for the exact path
    // The workgroup's P * 256 consecutive blocks per trip have as many consecutive scale bytes:
    // gathered in LDS, they leave as P * 16 non-temporal 16-byte stores (single cached bytes from every thread
    // cost several times more per byte on this path); a ragged last trip or an s_blk that is not
    // 16-byte aligned stores bytes.
    const bool sb_aligned = (((uintptr_t)s_blk) & 15u) == 0;
    bool bad = false;
    // The codes (8 bytes) and the E4M3 scale byte of one block whose 16 values are in v.
    const auto block_codes = [&](const uint4 (&v)[NV], uint32_t &e) -> uint2 {
        float f[16];
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    f[8 * j + 2 * k] = __uint_as_float(w[k] << 16);
                    f[8 * j + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[4 * j] = __uint_as_float(v[j].x); f[4 * j + 1] = __uint_as_float(v[j].y);
                f[4 * j + 2] = __uint_as_float(v[j].z); f[4 * j + 3] = __uint_as_float(v[j].w);
            }
        }
        uint32_t a = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) a = umax(a, __float_as_uint(f[k]) & 0x7FFFFFFFu);
        if (a >= 0x7F800000u) bad = true;        // Inf/NaN block: E4M3 NaN scale code
        e = nv_block_code(a, st);
        const float2 r = tab[e];
        uint32_t o[2], h[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const float *g = f + 8 * w;
            // every byte of lo and hi is written by its four converts: BF16 starts them from input
            // words that are dead once unpacked instead of zeros
            uint32_t lo = BF16 ? v[w].x : 0u, hi = BF16 ? v[w].y : 0u;
            lo = fp4_f32<0>(lo, g[0] * r.x, g[1] * r.x, 1.0f);
            lo = fp4_f32<1>(lo, g[2] * r.x, g[3] * r.x, 1.0f);
            lo = fp4_f32<2>(lo, g[4] * r.x, g[5] * r.x, 1.0f);
            lo = fp4_f32<3>(lo, g[6] * r.x, g[7] * r.x, 1.0f);
            hi = fp4_f32<0>(hi, g[0] * r.y, g[1] * r.y, 1.0f);
            hi = fp4_f32<1>(hi, g[2] * r.y, g[3] * r.y, 1.0f);
            hi = fp4_f32<2>(hi, g[4] * r.y, g[5] * r.y, 1.0f);
            hi = fp4_f32<3>(hi, g[6] * r.y, g[7] * r.y, 1.0f);
            o[w] = lo; h[w] = hi;
        }
        // elements whose two estimates disagree (nibbles of d) are recomputed exactly, one per
        // loop trip and lane; the lane's values go through LDS so that the trip reads element k
        // by index
        uint64_t d = (uint64_t)(o[0] ^ h[0]) | ((uint64_t)(o[1] ^ h[1]) << 32);
        if (__builtin_amdgcn_ballot_w64(d != 0u) != 0u) {          // wave-uniform branch
            float4 *fl = (float4 *)(fbuf + threadIdx.x * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k) fl[k] = make_float4(f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
            const float dec = __builtin_amdgcn_cvt_f32_fp8(e, 0);
            uint64_t oc = (uint64_t)o[0] | ((uint64_t)o[1] << 32);
            while (d != 0u) {
                const int sh = __builtin_ctzll(d) & ~3;             // nibble of the lowest set bit
                d &= ~(0xFull << sh);
                const uint64_t c = nv_elem_exact(fbuf[threadIdx.x * 16 + (sh >> 2)], st, dec);
                oc = (oc & ~(0xFull << sh)) | (c << sh);
            }
            o[0] = (uint32_t)oc;
            o[1] = (uint32_t)(oc >> 32);
        }
        return make_uint2(o[0], o[1]);
    };
    // P passes of kThreads blocks per trip (BF16: 2, FP32: 1), all their loads in flight together.
    // With two whole passes, lane pairs store the codes as 16-byte pieces (after one DPP swap the
    // even lane writes its own and its partner's block of the first pass, the odd lane both of the
    // second; the swapped words come from selects, not straight from the converts).
    constexpr int P = nv_passes_per_trip<BF16>();
    for (int64_t base = (int64_t)blockIdx.x * (P * kThreads); base < nblk; base += (int64_t)gridDim.x * (P * kThreads)) {
        int64_t blk[P];
        bool valid[P];
        uint4 v[P][NV];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            blk[p] = base + p * kThreads + threadIdx.x;
            valid[p] = blk[p] < nblk;
            // loads without a branch: a thread past the last block reads the last block again and
            // zeroes what it read (nblk > 0)
            const int64_t lb = valid[p] ? blk[p] : nblk - 1;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const uint4 t = ld_stream(xv + lb * NV + j);
                v[p][j] = valid[p] ? t : make_uint4(0, 0, 0, 0);
            }
        }
        uint32_t e[P];
        uint2 o[P];
#pragma unroll
        for (int p = 0; p < P; ++p) o[p] = block_codes(v[p], e[p]);
        const bool whole = base + P * kThreads <= nblk;            // uniform over the workgroup
        if (P == 2 && whole) {
            const bool odd = (threadIdx.x & 1u) != 0u;
            const uint2 oa = o[0], ob = o[P - 1];
            const uint32_t rx = dpp_mov<0xB1>(odd ? oa.x : ob.x), ry = dpp_mov<0xB1>(odd ? oa.y : ob.y);
            const uint4 w = odd ? make_uint4(rx, ry, ob.x, ob.y) : make_uint4(oa.x, oa.y, rx, ry);
            st_stream((uint4 *)(q + (odd ? blk[P - 1] - 1 : blk[0]) * 8), w);
        } else {
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (valid[p]) st_stream((uint2 *)q + blk[p], o[p]);
        }
        if (sb_aligned && whole) {
#pragma unroll
            for (int p = 0; p < P; ++p) sbuf[p * kThreads + threadIdx.x] = (uint8_t)e[p];
            __syncthreads();
            if (threadIdx.x < P * kThreads / 16)
                st_stream((uint4 *)(s_blk + base) + threadIdx.x, *(const uint4 *)(sbuf + 16 * threadIdx.x));
            __syncthreads();                             // sbuf is written again by the next trip
        } else {
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (valid[p]) s_blk[blk[p]] = (uint8_t)e[p];
        }
    }
    if (bad && nonfinite) *nonfinite = 1;
}

// ---------------------------------------------------------------------------------------------
// FP4 de-scaling. Units of 8 codes (BF16 output) or 4 codes (FP32 output), taken in flattened
// order, one 16-byte output piece each: element i
// belongs to MX block i / 32 (cols % 32 == 0) or NVFP4 block i / 16 (cols % 16 == 0), whose scale
// bytes are contiguous in the same order. MXFP4: decode(c) * 2^X is exact in fp32 for every code
// and X >= -127 (at most two significant bits, at least 2^-128), or Inf, and NaN for byte 0xFF.
// NVFP4: code * decode(e_b) takes at most 16 x 128 values and is exact in fp32, so each workgroup
// fills an LDS table of fl32(decode(c) * decode(e) / S_t) (IEEE division, S_t read once) and
// every element is one lookup. BF16 output rounds to nearest even.
constexpr int kDqThreads = 256;
constexpr int kDqMaxGrid = 2048;

// E2M1 code -> value: 0, 0.5 (the subnormal), then 1.m * 2^(e-1); sign in bit 3 (-0 for code 8).
__device__ __forceinline__ float e2m1_value(int c) {
    const int m = c & 7;
    const float mag = m < 2 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)(m & 1), (m >> 1) - 1);
    return (c & 8) ? -mag : mag;
}

// A unit is UC codes whose output is one 16-byte piece: 8 codes (4 bytes) for BF16, 4 codes (2
// bytes) for FP32. Lane l of a wave handles unit base + l, so each store instruction writes one
// dense 1 KiB run (non-temporal); a lane writing its output as several 16-byte stores would
// leave every store instruction half- or quarter-dense over its span, which measured slower.
template <int NV, bool OUTBF16>
__global__ __launch_bounds__(kDqThreads) void dequant_fp4_kernel(const uint8_t *__restrict__ q,
                                                                 const uint8_t *__restrict__ sb,
                                                                 const float *__restrict__ tensor_scale,
                                                                 int64_t nunits, void *__restrict__ out) {
    constexpr int UC = OUTBF16 ? 8 : 4;                                  // codes per unit
    constexpr int UPT = 4;                                               // units per thread and pass
    constexpr int BSH = (NV ? 4 : 5) - (OUTBF16 ? 3 : 2);                // unit -> scale block: u >> BSH
    __shared__ float tab[NV ? 128 * 16 : 16];
    if constexpr (NV) {
        const float st = *tensor_scale;
        for (int i = threadIdx.x; i < 128 * 16; i += kDqThreads) {
            const int e = i >> 4, c = i & 15;
            const float dec = __builtin_amdgcn_cvt_f32_fp8(e, 0);        // NaN for 0x7F
            const float p = e2m1_value(c) * dec;                         // exact
            tab[i] = p / st;
        }
    } else {
        if (threadIdx.x < 16) tab[threadIdx.x] = e2m1_value((int)threadIdx.x);
    }
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kDqThreads * UPT;
    for (int64_t base = (int64_t)blockIdx.x * kDqThreads * UPT + threadIdx.x; base < nunits; base += stride) {
        uint32_t w[UPT], b[UPT];
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int64_t u = base + (int64_t)j * kDqThreads;
            w[j] = 0u; b[j] = 0u;
            if (u < nunits) {
                if constexpr (UC == 8) w[j] = *(const uint32_t *)(q + 4 * u);
                else w[j] = *(const uint16_t *)(q + 2 * u);
                b[j] = sb[u >> BSH];
            }
        }
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int64_t u = base + (int64_t)j * kDqThreads;
            if (u >= nunits) continue;
            float v[UC];
            if constexpr (NV) {
#pragma unroll
                for (int k = 0; k < UC; ++k) v[k] = tab[b[j] * 16 + ((w[j] >> (4 * k)) & 15u)];
            } else {
                const int X = (int)b[j] - 127;
#pragma unroll
                for (int k = 0; k < UC; ++k) {
                    const float d = tab[(w[j] >> (4 * k)) & 15u];
                    v[k] = b[j] == 0xFFu ? __uint_as_float(0x7FC00000u) : __builtin_ldexpf(d, X);
                }
            }
            uint4 o;
            if constexpr (OUTBF16) {
                o = make_uint4(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                               bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16));
            } else {
                o = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
            }
            st_stream((uint4 *)out + u, o);
        }
    }
}

int nvfp4_grid(int64_t nblk, int passes) {
    int64_t g = (nblk + (int64_t)kThreads * passes - 1) / ((int64_t)kThreads * passes);
    if (g > kMaxStreamGrid) g = kMaxStreamGrid;
    return (int)(g < 1 ? 1 : g);
}

}  // namespace

int launch_dequant_fp4(int nv, const uint8_t *q, const uint8_t *sb, const float *tensor_scale, int64_t n, void *out,
                       int out_dtype, hipStream_t s) {
    // units of 8 codes (BF16 output) or 4 codes (FP32 output); n is a multiple of 16
    const int64_t nunits = n / (out_dtype == QF8_OUT_BF16 ? 8 : 4);
    if (nunits == 0) return QF8_OK;
    int64_t g = (nunits + 4 * kDqThreads - 1) / (4 * kDqThreads);
    if (g > kDqMaxGrid) g = kDqMaxGrid;
    const dim3 grid((unsigned)g), block(kDqThreads);
    if (nv) {
        if (out_dtype == QF8_OUT_BF16)
            hipLaunchKernelGGL((dequant_fp4_kernel<1, true>), grid, block, 0, s, q, sb, tensor_scale, nunits, out);
        else
            hipLaunchKernelGGL((dequant_fp4_kernel<1, false>), grid, block, 0, s, q, sb, tensor_scale, nunits, out);
    } else {
        if (out_dtype == QF8_OUT_BF16)
            hipLaunchKernelGGL((dequant_fp4_kernel<0, true>), grid, block, 0, s, q, sb, tensor_scale, nunits, out);
        else
            hipLaunchKernelGGL((dequant_fp4_kernel<0, false>), grid, block, 0, s, q, sb, tensor_scale, nunits, out);
    }
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

int launch_mxfp4(const void *x, int dtype, int64_t rows, int64_t cols, int rnd, uint8_t *q_row, uint8_t *s_row,
                 uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite, hipStream_t s) {
    if (rows == 0 || cols == 0) return QF8_OK;
    const int r = (int)rows, c = (int)cols;
    if (dtype == QF8_IN_BF16) {
        if (rnd == QF8_MX_ROUND_DOWN) launch_mxfp4_dirs<true, kRoundDown>(x, r, c, q_row, s_row, q_colT, s_colT, nonfinite, s);
        else launch_mxfp4_dirs<true, kRoundUp>(x, r, c, q_row, s_row, q_colT, s_colT, nonfinite, s);
    } else {
        if (rnd == QF8_MX_ROUND_DOWN) launch_mxfp4_dirs<false, kRoundDown>(x, r, c, q_row, s_row, q_colT, s_colT, nonfinite, s);
        else launch_mxfp4_dirs<false, kRoundUp>(x, r, c, q_row, s_row, q_colT, s_colT, nonfinite, s);
    }
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}


int launch_nvfp4(const void *x, int dtype, int64_t n, const uint32_t *partials, int nparts, const float *amax_in,
                 uint8_t *q, uint8_t *s_blk, float *tensor_scale, float *amax_out, int32_t *nonfinite, hipStream_t s) {
    const int64_t nblk = n / 16;
    const int grid = nvfp4_grid(nblk, dtype == QF8_IN_BF16 ? nv_passes_per_trip<true>() : nv_passes_per_trip<false>());
    if (dtype == QF8_IN_BF16)
        hipLaunchKernelGGL(nvfp4_kernel<true>, dim3(grid), dim3(kThreads), 0, s, x, nblk, partials, nparts, amax_in, q,
                           s_blk, tensor_scale, amax_out, nonfinite);
    else
        hipLaunchKernelGGL(nvfp4_kernel<false>, dim3(grid), dim3(kThreads), 0, s, x, nblk, partials, nparts, amax_in,
                           q, s_blk, tensor_scale, amax_out, nonfinite);
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
