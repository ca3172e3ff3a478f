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
//   A workgroup owns a tile of 128 rows x (32 * VEC) columns (VEC = 8 BF16 or 4 FP32 values per
//   16-byte load); each of its 4 waves owns 32 consecutive rows of the tile. Lane l of a wave
//   owns VEC consecutive columns (column slot l % 32) of 16 rows (half l / 32 of the wave's
//   rows), held in 16 x 16-byte registers.
//   * A rowwise block (1 row x 32 columns) spans 32/VEC lanes (4 for BF16): its amax takes two
//     (or three) DPP steps. Lane pairs write two rows' codes at once: after a DPP swap the even
//     lane stores row 2p of both lanes' columns and the odd lane row 2p + 1 (2 * VEC bytes each).
//   * A columnwise block (32 rows x 1 column) is split over lanes l and l ^ 32: each lane folds
//     its 16 rows in registers and one cross-half exchange completes the amax. The lane's 16
//     codes per column go to an LDS tile [column][128 rows]; after a barrier the workgroup
//     writes every column's 128 rows of q_colT as whole 128-byte lines, and the E8M0 bytes of
//     both directions, also gathered in LDS, as 4- or 8-byte runs.
//   * The conversion is the gfx950 scaled convert (two values per instruction, divided by 2^X
//     given as an fp32 exponent). The instruction does not saturate: with OCP round-down a
//     value can land in (F8max, 2^(emax+1)) and come out as the overflow code, which is then
//     mapped to +-F8max on the packed codes (mx_saturate_codes). Round-up never exceeds F8max.
//   * All global accesses are raw-buffer operations on per-wave descriptors: row and column
//     strides become scalar offsets, lanes outside the tensor get an out-of-range offset (their
//     loads read 0, their stores are dropped), and no per-row 64-bit address math is needed.
//     The input loads and the whole-line q_colT stores carry the non-temporal hint.
//   * Tiles are assigned so that each of the 8 XCDs (workgroups are dealt to XCDs round-robin)
//     receives a contiguous band of rows: the E8M0 rows and columns written by neighbouring
//     tiles then meet in the same L2.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 128;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerLane = kRowsPerWave / 2;
static_assert(kRowsPerLane % 2 == 0, "rowwise codes leave two rows at a time");

template <bool BF16, int FMT, int RND>
__device__ __forceinline__ uint32_t mx_byte(uint32_t absbits) {
    if constexpr (BF16) return mx_byte_bf16<FMT, RND>(absbits);
    else return mx_byte_f32<FMT, RND>(absbits);
}

// Byte offset of 16-row chunk k of tile column c in the LDS staging tile: one 128-byte line per
// column, chunks permuted by column so that the lanes of one LDS write spread over the banks.
__device__ __forceinline__ int colbuf_offset(int c, int k) { return c * kTileRows + ((k ^ ((c >> 3) & 7)) << 4); }

template <bool BF16, int FMT, int RND, bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void mx_kernel(const void *__restrict__ x, int rows, int cols,
                                                      uint8_t *__restrict__ q_row, uint8_t *__restrict__ s_row,
                                                      uint8_t *__restrict__ q_colT, uint8_t *__restrict__ s_colT,
                                                      int32_t *nonfinite, int tiles_c, int tiles, int per_xcd) {
    constexpr int VEC = BF16 ? 8 : 4;            // values per lane per row (one 16-byte load)
    constexpr int ESZ = BF16 ? 2 : 4;            // bytes per input element
    constexpr int LPB = 32 / VEC;                // lanes per rowwise block
    constexpr int RPL = kRowsPerLane;
    constexpr int TILE_C = 32 * VEC;             // columns per tile
    constexpr int NBLK = TILE_C / 32;            // rowwise blocks per tile row
    constexpr uint32_t ABS = BF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;

    // LDS staging (columnwise pass only): codes [column][128 rows] (16-byte chunks swizzled),
    // E8M0 bytes of the columnwise blocks [column][4 row blocks] and of the rowwise blocks
    // [tile row][NBLK]
    __shared__ __attribute__((aligned(16))) uint8_t colbuf[COL ? TILE_C * kTileRows : 16];
    __shared__ __attribute__((aligned(16))) uint8_t scol[COL ? TILE_C * 4 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t srow[ROW ? kTileRows * NBLK : 16];

    const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
    const int t = xcd * per_xcd + local;
    if (local >= per_xcd || t >= tiles) return;  // whole workgroup idle
    const int tr = t / tiles_c, tc = t - tr * tiles_c;
    const int tr0 = tr * kTileRows;              // first row of the tile
    const int ct0 = tc * TILE_C;                 // first column of the tile
    const int ncv = cols - ct0 < TILE_C ? cols - ct0 : TILE_C;          // valid columns of the tile
    const int trows = rows - tr0 < kTileRows ? rows - tr0 : kTileRows;  // valid rows of the tile
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, half = lane >> 5, slot = lane & 31;
    const int r0 = tr0 + wave * kRowsPerWave;   // first row of the wave (uniform)
    uint32_t seen = 0;     // |x| maximum of everything the lane loaded (BF16 or FP32 bit pattern)

    if (r0 < rows) {                             // else the wave only joins the barrier
        const int c0 = ct0 + slot * VEC;         // first column of the lane
        const bool active = c0 < cols;           // rowwise blocks are whole: cols % 32 == 0
        const int wrows = rows - r0 < kRowsPerWave ? rows - r0 : kRowsPerWave;

        // ---- load 16 rows x 16 bytes -----------------------------------------------------
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

        uint32_t cmax[4] = {0, 0, 0, 0};         // columnwise |x| maxima (BF16: two per dword)

        // ---- rowwise blocks, one row at a time; columnwise maxima accumulate -------------
        if constexpr (ROW) {
            const __amdgpu_buffer_rsrc_t qr = make_rsrc(q_row + (size_t)r0 * cols, (uint32_t)wrows * cols);
            const uint32_t qvo = active ? (uint32_t)(half * RPL) * cols + c0 : kOutOfRange;
            const uint32_t sstride = cols / 32;
            // Rows 2p and 2p + 1 leave through lane pairs: the even lane of a pair writes row 2p of
            // both lanes' columns, the odd lane row 2p + 1, after one DPP swap of the codes each
            // sends (16-byte pieces for BF16, 8 for FP32: half the store instructions). A pair's
            // lanes are both active or both idle, since cols % 32 == 0. The swapped value is the
            // result of the zero-block select, written whole by one VALU instruction: a DPP move
            // never reads a convert's partially written destination.
            const bool odd = (slot & 1) != 0;
            constexpr uint32_t kCodes = VEC;             // code bytes per lane and row
            const uint32_t qpo = !active ? kOutOfRange : odd ? qvo - kCodes : qvo;
            uint32_t p0 = 0u, p1 = 0u;                   // the codes of the pair's first row
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
                const uint32_t byte = mx_byte<BF16, FMT, RND>(a);
                const float sc = __uint_as_float(byte << 23);
                const uint32_t *v = d[i];
                // The converts write two of the four code bytes into their "old" operand; m[0] and
                // m[2] are dead here, so their registers take the codes without a zeroing move.
                if constexpr (BF16) {
                    uint32_t o0 = cvt2_bf16_div2x<FMT, true>(v[1], sc, cvt2_bf16_div2x<FMT, false>(v[0], sc, m[0]));
                    uint32_t o1 = cvt2_bf16_div2x<FMT, true>(v[3], sc, cvt2_bf16_div2x<FMT, false>(v[2], sc, m[2]));
                    if constexpr (RND == kRoundDown) { o0 = mx_saturate_codes<FMT>(o0); o1 = mx_saturate_codes<FMT>(o1); }
                    if (a == 0u) o0 = o1 = 0u;                          // all-zero block: 0x00, not -0
                    if ((i & 1) == 0) {
                        p0 = o0; p1 = o1;
                    } else {
                        const uint32_t rx = dpp_mov<0xB1>(odd ? p0 : o0), ry = dpp_mov<0xB1>(odd ? p1 : o1);
                        const uint4 w = odd ? make_uint4(rx, ry, o0, o1) : make_uint4(p0, p1, rx, ry);
                        buf_store16(qr, qpo + (uint32_t)(odd ? i : i - 1) * cols, 0u, w);
                    }
                } else {
                    uint32_t o0 = cvt2_f32_div2x<FMT, true>(__uint_as_float(v[2]), __uint_as_float(v[3]), sc,
                                  cvt2_f32_div2x<FMT, false>(__uint_as_float(v[0]), __uint_as_float(v[1]), sc, m[0]));
                    if constexpr (RND == kRoundDown) o0 = mx_saturate_codes<FMT>(o0);
                    if (a == 0u) o0 = 0u;
                    if ((i & 1) == 0) {
                        p0 = o0;
                    } else {
                        const uint32_t r = dpp_mov<0xB1>(odd ? p0 : o0);
                        buf_store8(qr, qpo + (uint32_t)(odd ? i : i - 1) * cols, 0u, odd ? r : p0, odd ? o0 : r);
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

        // ---- columnwise blocks: VEC columns x 16 rows per lane, the other 16 rows in lane ^ 32
        if constexpr (COL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t other = (uint32_t)__shfl_xor((int)cmax[k], 32);
                cmax[k] = BF16 ? pk_max_u16(cmax[k], other) : umax(cmax[k], other);
            }
            const int chunk = wave * 2 + half;   // 16-row chunk of the tile
            if constexpr (BF16) {
                const uint32_t mm = pk_max_u16(pk_max_u16(cmax[0], cmax[1]), pk_max_u16(cmax[2], cmax[3]));
                seen = umax(mm & 0xFFFFu, mm >> 16);
            } else {
                seen = umax(umax(cmax[0], cmax[1]), umax(cmax[2], cmax[3]));
            }
            if constexpr (BF16) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {     // dword k holds columns 2k (low half) and 2k+1
                    const uint32_t alo = cmax[k] & 0xFFFFu, ahi = cmax[k] >> 16;
                    const uint32_t blo = mx_byte<true, FMT, RND>(alo), bhi = mx_byte<true, FMT, RND>(ahi);
                    const float slo = __uint_as_float(blo << 23), shi = __uint_as_float(bhi << 23);
                    uint32_t olo[4], ohi[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {     // rows 4g .. 4g+3 of the lane
                        uint32_t w[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) w[j] = d[4 * g + j][k];
                        // one column's values of two consecutive rows in one dword
                        const uint32_t l01 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
                        const uint32_t l23 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
                        const uint32_t h01 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
                        const uint32_t h23 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
                        // w[0] and w[2] are dead after the permutes: they take the codes
                        olo[g] = cvt2_bf16_div2x<FMT, true>(l23, slo, cvt2_bf16_div2x<FMT, false>(l01, slo, w[0]));
                        ohi[g] = cvt2_bf16_div2x<FMT, true>(h23, shi, cvt2_bf16_div2x<FMT, false>(h01, shi, w[2]));
                        if constexpr (RND == kRoundDown) {
                            olo[g] = mx_saturate_codes<FMT>(olo[g]);
                            ohi[g] = mx_saturate_codes<FMT>(ohi[g]);
                        }
                        if (alo == 0u) olo[g] = 0u;          // all-zero block: 0x00, not -0
                        if (ahi == 0u) ohi[g] = 0u;
                    }
                    const int clo = slot * VEC + 2 * k;           // tile column of the low half
                    *(uint4 *)(colbuf + colbuf_offset(clo, chunk)) = make_uint4(olo[0], olo[1], olo[2], olo[3]);
                    *(uint4 *)(colbuf + colbuf_offset(clo + 1, chunk)) = make_uint4(ohi[0], ohi[1], ohi[2], ohi[3]);
                    if (half == 0) {
                        scol[clo * 4 + wave] = (uint8_t)blo;
                        scol[(clo + 1) * 4 + wave] = (uint8_t)bhi;
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {     // tile column slot * 4 + k
                    const uint32_t a = cmax[k];
                    const uint32_t byte = mx_byte<false, FMT, RND>(a);
                    const float sc = __uint_as_float(byte << 23);
                    uint32_t o[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float f[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(d[4 * g + j][k]);
                        o[g] = cvt2_f32_div2x<FMT, true>(f[2], f[3], sc,
                                                         cvt2_f32_div2x<FMT, false>(f[0], f[1], sc, d[4 * g][k]));
                        if constexpr (RND == kRoundDown) o[g] = mx_saturate_codes<FMT>(o[g]);
                        if (a == 0u) o[g] = 0u;
                    }
                    const int c = slot * VEC + k;
                    *(uint4 *)(colbuf + colbuf_offset(c, chunk)) = make_uint4(o[0], o[1], o[2], o[3]);
                    if (half == 0) scol[c * 4 + wave] = (uint8_t)byte;
                }
            }
        }
    }

    // ---- the tile's staged outputs, written by the whole workgroup ---------------------------
    if constexpr (COL) {
        __syncthreads();
        // q_colT: column c of the tile -> q_colT[ct0 + c][tr0 .. tr0 + trows), 16 bytes per lane.
        // Thread t writes 16-row chunk t % 8 of tile columns t / 8 + 32 j. The offsets are 32-bit and
        // the validity tests are combined without short-circuit branches: after the barrier each
        // store costs a handful of instructions, which shortens the tail of every workgroup.
        const __amdgpu_buffer_rsrc_t qc = make_rsrc(q_colT + (size_t)ct0 * rows + tr0, (uint32_t)ncv * rows - tr0);
        const uint32_t urows = (uint32_t)rows, k = threadIdx.x & 7u, cb = threadIdx.x >> 3;
        const bool kv = (int)(16u * k) < trows;
#pragma unroll
        for (int j = 0; j < TILE_C / 32; ++j) {
            const uint32_t c = cb + 32u * j;
            const uint4 v = *(const uint4 *)(colbuf + colbuf_offset((int)c, (int)k));
            const uint32_t vo = (((int)c < ncv) & kv) ? c * urows + 16u * k : kOutOfRange;
            buf_store16<kNonTemporal>(qc, vo, 0u, v);
        }
        // s_colT: the tile's trows/32 bytes of column c, contiguous in s_colT[ct0 + c]; one column per
        // thread (TILE_C <= kThreads). Whole tiles store them as one word, a ragged last tile row
        // byte by byte (the choice is uniform over the workgroup).
        static_assert(TILE_C <= kThreads && kTileRows <= kThreads, "one column and one row per thread");
        const uint32_t srb = (uint32_t)rows / 32;
        const int nb = trows / 32;
        const __amdgpu_buffer_rsrc_t scr = make_rsrc(s_colT + (size_t)ct0 * srb + tr0 / 32, (uint32_t)ncv * srb - tr0 / 32);
        const bool whole_c = nb == 4 && (srb & 3u) == 0 && (((uintptr_t)s_colT) & 3u) == 0;
        const int ct = threadIdx.x;
        if (ct < TILE_C) {
            const uint32_t w = *(const uint32_t *)(scol + ct * 4);
            if (whole_c) {
                buf_store4(scr, ct < ncv ? (uint32_t)ct * srb : kOutOfRange, 0u, w);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    buf_store1(scr, ((ct < ncv) & (j < nb)) ? (uint32_t)ct * srb + j : kOutOfRange, 0u, w >> (8 * j));
            }
        }
        // s_row: row r of the tile -> its NBLK bytes s_row[tr0 + r][ct0/32 ...]; one row per thread
        if constexpr (ROW) {
            const uint32_t ssb = (uint32_t)cols / 32;
            const int nbl = ncv / 32;
            const __amdgpu_buffer_rsrc_t srr = make_rsrc(s_row + (size_t)tr0 * ssb + ct0 / 32,
                                                         (uint32_t)trows * ssb - ct0 / 32);
            const bool whole_r = nbl == NBLK && (ssb % NBLK) == 0 && (((uintptr_t)s_row) % NBLK) == 0;
            const int r = threadIdx.x;
            if (r < kTileRows) {
                const bool rv = r < trows;
                if constexpr (NBLK == 8) {
                    const uint2 w = *(const uint2 *)(srow + r * 8);
                    if (whole_r) {
                        buf_store8(srr, rv ? (uint32_t)r * ssb : kOutOfRange, 0u, w.x, w.y);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            buf_store1(srr, (rv & (j < nbl)) ? (uint32_t)r * ssb + j : kOutOfRange, 0u,
                                       (j < 4 ? w.x : w.y) >> (8 * (j & 3)));
                    }
                } else {
                    const uint32_t w = *(const uint32_t *)(srow + r * 4);
                    if (whole_r) {
                        buf_store4(srr, rv ? (uint32_t)r * ssb : kOutOfRange, 0u, w);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            buf_store1(srr, (rv & (j < nbl)) ? (uint32_t)r * ssb + j : kOutOfRange, 0u, w >> (8 * j));
                    }
                }
            }
        }
    }
    if (seen >= (BF16 ? 0x7F80u : 0x7F800000u) && nonfinite) *nonfinite = 1;
}

template <bool BF16, int FMT, int RND>
void launch_dirs(const void *x, int rows, int cols, uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT,
                 uint8_t *s_colT, int32_t *nonfinite, hipStream_t s) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int tiles_r = (rows + kTileRows - 1) / kTileRows;
    const int tiles_c = (cols + 32 * VEC - 1) / (32 * VEC);
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
    const int r = (int)rows, c = (int)cols;
#define QF8_MX(BF, F, R) launch_dirs<BF, F, R>(x, r, c, q_row, s_row, q_colT, s_colT, nonfinite, s)
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
