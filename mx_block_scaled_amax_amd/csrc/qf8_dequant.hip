// qf8_dequant.hip -- de-scaling of FP8 codes back to BF16 / FP32, and quantization error
// statistics of a quantized tensor against its high-precision source.
//
// Pages (title, section):
//   [MP-FP8]       "混合精度与 FP8 训练" (hs-black.github.io): section 8.1 (the code 22 of the
//                  worked example de-scales by S = 22400 to 22/22400; a GEMM multiplies its
//                  result back by 1/(S_X S_W)), 8.2 (the saturated 448 de-scales to 20), 7.2
//                  (watch amax, the share of values that underflow to zero, and saturation),
//                  13.1 (an MX element is a code times its block's power of two).
//   [Ascend950]    Ascend 950 low-precision format guide (hwcomputing.csdn.net): the HiF8 vs
//                  MXFP8 numerical analysis on DeepSeek-V4-Flash (SQNR and zero-rate per layer).
//
// Definitions the kernels compute:
//   scale factor S (per tensor or per group):  xhat = fl32(decode(q) / S), one IEEE division;
//   MX block byte b:                           xhat = decode(q) * 2^(b - 127), exact (ldexp),
//                                              NaN for b = 0xFF;
//   BF16 output: xhat rounded to nearest even.
//   statistics over the finite elements of x: signal = sum x^2, noise = sum (x - xhat)^2 in
//   fp64, and counts of nonzero x, of nonzero x with xhat = 0, of saturated elements (scaled
//   value beyond F8max before the cast: |fl32(x S)| > F8max, or |x| > F8max 2^X for MX) and of
//   Inf/NaN x (excluded from the rest).
//
// Work: a unit is 8 consecutive codes for BF16 output, 4 for FP32 output, 16 with statistics (4
// when a group's rows are only a multiple of 4 or 8 long), always inside one row, one group and
// one MX block, so its scale is looked up once. A workgroup tile is 256 threads x 32 codes (16
// with statistics), consecutive threads on consecutive units; a workgroup walks its tiles a grid
// stride apart and loads the next tile's codes, inputs and scale words before the current one's
// arithmetic, with only uniform branches and unconditional loads in that loop so that the
// compiler's wait counts stay exact. Codes decode with the gfx950 fp8/bf8 -> f32 converts
// (exact) and de-scale (MX: times 2^X; groups: IEEE division; one tensor scale: a 256-entry LDS
// table of decode(c) / S built per workgroup); each 8-code BF16 or 4-code FP32 unit leaves as one
// 16-byte store, consecutive lanes on consecutive pieces. With statistics, whole tiles sum
// without a per-element Inf/NaN filter (a wave whose x holds one starts over with the filter),
// the fp64 terms go to 4 independent running sums per thread, and the counts are popcounts of
// wave ballots on the scalar unit; each workgroup reduces its sums and counts in a fixed order
// into a 64-byte partial in the workspace, and one workgroup folds the partials in a fixed order:
// the same input always gives the same bits.
#include <type_traits>

#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kDqThreads = 256;
constexpr int kDqMaxGrid = 16384;
constexpr int kStatsGrid = 1024;                 // workgroups (= 64-byte partials) with statistics
static_assert(kStatsGrid % kDqThreads == 0, "whole partials per thread in the final fold");
static_assert(kStatsGrid * 64 <= kMaxStreamGrid * 4, "partials fit the workspace partial region");

enum { kModeScaled = 0, kModeBlock = 1, kModeMx = 2 };
enum { kNone = 0, kBF16 = 1, kFP32 = 2 };


struct StatsPart {                               // same layout as qf8_error_stats
    double signal, noise;
    uint64_t count, nonzero, zeroed, saturated, nonfinite, reserved;
};
static_assert(sizeof(StatsPart) == 64, "64-byte partials");

struct DqArgs {
    const uint8_t *q;
    int64_t n;
    uint32_t units;              // whole W-code units
    uint32_t upr;                // units per row (block, MX)
    uint64_t upr_mul;            // u / upr = (u * upr_mul) >> upr_shift for every u < 2^31
    uint32_t upr_shift;
    uint32_t br_shift;           // log2 of the block rows, 1 or 128 (block)
    uint32_t gcols;              // groups per row of the scale array (block)
    const float *scale;          // per-tensor S (scaled) or group scales (block)
    const uint8_t *sb;           // E8M0 bytes (MX)
    void *out;
    const void *x;
    StatsPart *parts;
};

template <int FMT>
__device__ __forceinline__ void decode4(uint32_t codes, float *v) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f lo, hi;
    if constexpr (FMT == kE4M3) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8(codes, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8(codes, true);
    }
    v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
}

// Running statistics of one thread: the fp64 sums in 4 independent chains (element k of a unit
// goes to chain k % 4; short dependency chains, fixed order), counts in u32.
struct Acc {
    double signal[4] = {0.0, 0.0, 0.0, 0.0}, noise[4] = {0.0, 0.0, 0.0, 0.0};
    uint32_t count = 0, nonzero = 0, zeroed = 0, saturated = 0, nonfinite = 0;
    __device__ __forceinline__ double signal_sum() const { return (signal[0] + signal[1]) + (signal[2] + signal[3]); }
    __device__ __forceinline__ double noise_sum() const { return (noise[0] + noise[1]) + (noise[2] + noise[3]); }
};

__device__ __forceinline__ bool finite_f32(float x) { return fabsf(x) <= 3.40282346638528859812e+38f; }

template <int W>
__device__ __forceinline__ void acc_add_unit(Acc &acc, const float *x, const float *xh, const bool *sat) {
    bool all_fin = true;
#pragma unroll
    for (int k = 0; k < W; ++k) all_fin = all_fin && finite_f32(x[k]);
    if (all_fin) {                 // the usual case, without the selects that drop Inf/NaN
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const double xd = (double)x[k], d = xd - (double)xh[k];
            acc.signal[k & 3] += xd * xd;
            acc.noise[k & 3] += d * d;
            const bool nz = x[k] != 0.0f;
            acc.nonzero += nz ? 1u : 0u;
            acc.zeroed += (nz && xh[k] == 0.0f) ? 1u : 0u;
            acc.saturated += sat[k] ? 1u : 0u;
        }
        acc.count += W;
        return;
    }
    // a unit with Inf/NaN: those elements add +0 to the sums (which leaves them unchanged) and
    // count as non-finite only
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const bool fin = finite_f32(x[k]);
        const double xd = fin ? (double)x[k] : 0.0, d = fin ? xd - (double)xh[k] : 0.0;
        acc.signal[k & 3] += xd * xd;
        acc.noise[k & 3] += d * d;
        acc.nonfinite += fin ? 0u : 1u;
        acc.count += fin ? 1u : 0u;
        const bool nz = fin && x[k] != 0.0f;
        acc.nonzero += nz ? 1u : 0u;
        acc.zeroed += (nz && xh[k] == 0.0f) ? 1u : 0u;
        acc.saturated += (fin && sat[k]) ? 1u : 0u;
    }
}

// Counts of one wave, kept as wave-uniform sums of ballot masks (on the scalar unit).
struct WaveCounts {
    uint32_t nonzero = 0, zeroed = 0, saturated = 0;
};

// The statistics of one unit for a whole wave in step, without the Inf/NaN filter: a non-finite
// x makes the lane's signal sum non-finite (a finite BF16/FP32 x^2 is below 2^256, so a finite sum
// of fewer than 2^33 of them stays finite), and a wave that finds one starts over with
// acc_add_unit. Counts go to wave-uniform sums: only where every lane of the wave takes the same
// path.
template <int W>
__device__ __forceinline__ void acc_add_unit_fast(Acc &acc, WaveCounts &wc, const float *x, const float *xh,
                                                  const bool *sat) {
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const double xd = (double)x[k], d = xd - (double)xh[k];
        acc.signal[k & 3] += xd * xd;
        acc.noise[k & 3] += d * d;
        const uint64_t nz = __builtin_amdgcn_ballot_w64(x[k] != 0.0f), z = __builtin_amdgcn_ballot_w64(xh[k] == 0.0f);
        wc.nonzero += (uint32_t)__builtin_popcountll(nz);
        wc.zeroed += (uint32_t)__builtin_popcountll(nz & z);
        wc.saturated += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(sat[k]));
    }
    acc.count += W;
}

__device__ __forceinline__ bool finite_f64(double v) { return fabs(v) <= 1.79769313486231570815e+308; }

// W consecutive elements of x (W = 4 or 16: the units of the statistics) of unit u in two steps:
// the raw dwords (BF16 pairs or fp32 bits), loaded a tile ahead, then their fp32 values.
template <int XK, int W>
constexpr int x_raw_dwords() { return XK == kBF16 ? W / 2 : W; }
template <int XK, int W>
__device__ __forceinline__ void load_x_raw(const void *x, uint32_t u, uint32_t *w) {
    static_assert(W == 4 || W == 16, "statistics units");
    constexpr int D = x_raw_dwords<XK, W>();
    const uint32_t *p = (const uint32_t *)x + (size_t)u * D;
    if constexpr (D % 4 == 0) {
#pragma unroll
        for (int k = 0; k < D / 4; ++k) {
            const uint4 a0 = ((const uint4 *)p)[k];
            w[4 * k] = a0.x; w[4 * k + 1] = a0.y; w[4 * k + 2] = a0.z; w[4 * k + 3] = a0.w;
        }
    } else {
        const uint2 a0 = *(const uint2 *)p;
        w[0] = a0.x; w[1] = a0.y;
    }
}
template <int XK, int W>
__device__ __forceinline__ void x_from_raw(const uint32_t *w, float *xv) {
    if constexpr (XK == kBF16) {
#pragma unroll
        for (int k = 0; k < W / 2; ++k) {
            xv[2 * k] = __uint_as_float(w[k] << 16);
            xv[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < W; ++k) xv[k] = __uint_as_float(w[k]);
    }
}
template <int XK>
__device__ __forceinline__ float load_x1(const void *x, int64_t e) {
    if constexpr (XK == kBF16) return __uint_as_float((uint32_t)((const uint16_t *)x)[e] << 16);
    else return ((const float *)x)[e];
}

template <int OUTK, int W>
__device__ __forceinline__ void store_out(void *out, uint32_t u, const float *v) {
    if constexpr (OUTK == kBF16) {
        uint32_t w[W / 2];
#pragma unroll
        for (int k = 0; k < W / 2; ++k) w[k] = bf16_rne(v[2 * k]) | (bf16_rne(v[2 * k + 1]) << 16);
        uint32_t *p = (uint32_t *)out + (size_t)u * (W / 2);
        if constexpr (W == 16) {
            ((uint4 *)p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
            ((uint4 *)p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
        } else if constexpr (W == 8) {
            st_stream((uint4 *)p, make_uint4(w[0], w[1], w[2], w[3]));
        } else {
            *(uint2 *)p = make_uint2(w[0], w[1]);
        }
    } else if constexpr (OUTK == kFP32) {
        uint4 *p = (uint4 *)out + (size_t)u * (W / 4);
#pragma unroll
        for (int k = 0; k < W / 4; ++k) {
            const uint4 o = make_uint4(__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                                       __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3]));
            if constexpr (W == 4) st_stream(p + k, o);
            else p[k] = o;
        }
    }
}
template <int OUTK>
__device__ __forceinline__ void store1(void *out, int64_t e, float v) {
    if constexpr (OUTK == kBF16) ((uint16_t *)out)[e] = (uint16_t)bf16_rne(v);
    else if constexpr (OUTK == kFP32) ((float *)out)[e] = v;
}

// How one unit is de-scaled: a scale factor S (divide), or for MX the multiplier 2^X (an exact
// power of two, subnormal for X = -127; fp32 denormals are kept, so the product rounds exactly as
// ldexp does).
struct UnitScale {
    float s;      // S; MX: F8max * 2^X for the saturation test, +Inf for the byte 0xFF
    float m;      // MX: 2^X, NaN for the byte 0xFF (every element of the block de-scales to NaN)
};

// Row of unit u (u < 2^31) without a division instruction sequence: the multiplier and shift are
// computed on the host (round-up reciprocal, exact below 2^31; see launch_dequant).
__device__ __forceinline__ uint32_t unit_row(const DqArgs &a, uint32_t u) {
    return (uint32_t)(((uint64_t)u * a.upr_mul) >> a.upr_shift);
}

// The raw scale word of unit u (W codes, all in one row and one group: cols % W == 0, W divides
// 32 and 128): the fp32 bits of its group scale, or its E8M0 byte. Loaded with the unit's codes.
template <int MODE, int W>
__device__ __forceinline__ uint32_t load_scale_raw(const DqArgs &a, uint32_t u) {
    if constexpr (MODE == kModeBlock) {
        const uint32_t r = unit_row(a, u), c = (u - r * a.upr) * W;
        return __float_as_uint(a.scale[(size_t)(r >> a.br_shift) * a.gcols + (c >> 7)]);
    } else if constexpr (MODE == kModeMx) {
        const uint32_t r = unit_row(a, u), c = (u - r * a.upr) * W;
        return a.sb[(size_t)r * (a.upr * W / 32) + (c >> 5)];
    } else {
        return 0u;
    }
}

template <int FMT, int MODE>
__device__ __forceinline__ UnitScale unit_scale(uint32_t raw, float s_tensor) {
    UnitScale us{s_tensor, 1.0f};
    if constexpr (MODE == kModeBlock) {
        us.s = __uint_as_float(raw);
    } else if constexpr (MODE == kModeMx) {
        const int xexp = (int)raw - 127;
        const bool nan = raw == 0xFFu;
        us.m = nan ? __uint_as_float(0x7FC00000u) : __builtin_ldexpf(1.0f, xexp);
        us.s = nan ? __builtin_inff() : __builtin_ldexpf(F8<FMT>::kMax, xexp);
    }
    return us;
}

template <int MODE>
__device__ __forceinline__ float descale(float v, const UnitScale &us) {
    if constexpr (MODE == kModeMx) return v * us.m;
    else return v / us.s;
}

template <int FMT, int MODE>
__device__ __forceinline__ bool saturates(float x, const UnitScale &us) {
    if constexpr (MODE == kModeMx) return fabsf(x) > us.s;
    else return fabsf(x * us.s) > F8<FMT>::kMax;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Fixed-order workgroup sum of the accumulator into one partial (thread 0 writes it). The
// wave-uniform counts of the whole-tile passes are added once per wave.
__device__ void block_store_partial(const Acc &acc, const WaveCounts &wcnt, StatsPart *dst) {
    __shared__ double sd[2][kDqThreads / 64];
    __shared__ uint32_t sc[5][kDqThreads / 64];
    const double sg = wave_sum(acc.signal_sum()), ns = wave_sum(acc.noise_sum());
    const uint32_t c0 = wave_sum(acc.count), c4 = wave_sum(acc.nonfinite);
    const uint32_t c1 = wave_sum(acc.nonzero) + __builtin_amdgcn_readfirstlane(wcnt.nonzero),
                   c2 = wave_sum(acc.zeroed) + __builtin_amdgcn_readfirstlane(wcnt.zeroed),
                   c3 = wave_sum(acc.saturated) + __builtin_amdgcn_readfirstlane(wcnt.saturated);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sd[0][w] = sg; sd[1][w] = ns;
        sc[0][w] = c0; sc[1][w] = c1; sc[2][w] = c2; sc[3][w] = c3; sc[4][w] = c4;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        StatsPart p{};
        for (int k = 0; k < kDqThreads / 64; ++k) {
            p.signal += sd[0][k]; p.noise += sd[1][k];
            p.count += sc[0][k]; p.nonzero += sc[1][k]; p.zeroed += sc[2][k]; p.saturated += sc[3][k];
            p.nonfinite += sc[4][k];
        }
        *dst = p;
    }
}

template <int P> using Pass = std::integral_constant<int, P>;
enum { kWhole = 0, kPart = 1, kRedo = 2 };   // a whole tile, the partial last tile, a statistics re-run

// W codes per unit. De-scaling alone takes 8 or 4, so that each lane moves one 16-byte piece of the
// output and consecutive lanes move consecutive pieces: 8 codes (an 8-byte load) make 16 bytes of
// BF16, 4 codes 16 bytes of FP32, and whole 16-byte outputs leave as non-temporal stores (a lane
// writing 32 bytes as two 16-byte stores leaves every store instruction half-dense over its span,
// which measured ~10% slower for this stream). With the statistics, 16-code units (one 16-byte
// load of codes) halve the per-unit overhead of the fp64 terms. 4-code units also serve rows that
// are only a multiple of 4 codes long (8-byte BF16 stores, cached so that L2 merges them). With
// one scale factor the workgroup first tabulates fl32(decode(c) / S) for all 256 codes in LDS, so
// an element costs a table read, not a division.
template <int FMT, int MODE, int OUTK, int XK, int W>
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(DqArgs a) {
    constexpr bool STATS = XK != kNone;
    static_assert(W == 16 || W == 8 || W == 4, "16-, 8- or 4-code units");
    // units per thread and tile: 32 codes, or 16 with the statistics (two tiles' raw inputs are
    // held at once, below)
    constexpr int UPT = (STATS ? 16 : 32) / W;
    constexpr int ND = W / 4;                     // dwords of codes per unit
    constexpr uint32_t kTile = kDqThreads * UPT;  // units of one workgroup tile
    __shared__ float tab[MODE == kModeScaled ? 256 : 1];
    float s_tensor = 1.0f;
    if constexpr (MODE == kModeScaled) {
        s_tensor = *a.scale;
        float v[4];
        decode4<FMT>(threadIdx.x, v);            // 256 threads: code = threadIdx.x
        tab[threadIdx.x] = v[0] / s_tensor;
        __syncthreads();
    }
    Acc acc;
    WaveCounts wcnt;
    const uint32_t stride = gridDim.x * kTile;
    constexpr int XD = STATS ? x_raw_dwords<XK == kNone ? kBF16 : XK, W == 8 ? 16 : W>() : 1;
    // one tile's inputs of this thread: codes, raw x and raw scale word of each of its units
    struct In {
        uint32_t c[UPT][ND];
        uint32_t x[UPT][XD];
        uint32_t s[UPT];
    };
    auto load = [&](auto pass, uint32_t base, In &in) {
        constexpr int P = decltype(pass)::value;
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const uint32_t u = base + j * kDqThreads + threadIdx.x;
            if (P == kWhole || u < a.units) {
                if constexpr (W == 16) {
                    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
                    const v4u c = __builtin_nontemporal_load((const v4u *)a.q + u);
                    in.c[j][0] = c.x; in.c[j][1] = c.y; in.c[j][2] = c.z; in.c[j][3] = c.w;
                } else if constexpr (W == 8) {
                    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
                    const v2u c = __builtin_nontemporal_load((const v2u *)a.q + u);
                    in.c[j][0] = c.x; in.c[j][1] = c.y;
                } else {
                    in.c[j][0] = __builtin_nontemporal_load((const uint32_t *)a.q + u);
                }
                if constexpr (STATS) load_x_raw<XK, W>(a.x, u, in.x[j]);
                in.s[j] = load_scale_raw<MODE, W>(a, u);
            }
        }
    };
    auto process = [&](auto pass, uint32_t base, const In &in) {
        constexpr int P = decltype(pass)::value;
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const uint32_t u = base + j * kDqThreads + threadIdx.x;
            if (P != kWhole && u >= a.units) continue;
            const UnitScale us = unit_scale<FMT, MODE>(in.s[j], s_tensor);
            float v[W];
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                if constexpr (MODE == kModeScaled) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[4 * d + k] = tab[(in.c[j][d] >> (8 * k)) & 0xFFu];
                } else {
                    decode4<FMT>(in.c[j][d], v + 4 * d);
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[4 * d + k] = descale<MODE>(v[4 * d + k], us);
                }
            }
            if constexpr (P != kRedo) store_out<OUTK, W>(a.out, u, v);
            if constexpr (STATS) {
                float xv[W];
                x_from_raw<XK, W>(in.x[j], xv);
                bool sat[W];
#pragma unroll
                for (int k = 0; k < W; ++k) sat[k] = saturates<FMT, MODE>(xv[k], us);
                if constexpr (P == kWhole) acc_add_unit_fast<W>(acc, wcnt, xv, v, sat);
                else acc_add_unit<W>(acc, xv, v, sat);
            }
        }
    };
    // Whole tiles first, each tile's loads issued one tile ahead of its arithmetic (two buffers,
    // unrolled by two). Every branch here is uniform over the workgroup and the loads and their
    // uses are unconditional, so the compiler's wait counts stay exact: the next tile's loads
    // remain in flight while the current one is de-scaled. Only a workgroup's last tile can be
    // partial (the tiles of one workgroup are a grid stride apart).
    In i0, i1;
    uint32_t base = blockIdx.x * kTile;
    if (base + kTile <= a.units) {
        load(Pass<kWhole>(), base, i0);
        if constexpr (STATS) {
            // Several tiles per workgroup (the grid is capped). One processing site per buffer:
            // past the workgroup's last whole tile the prefetch reads tile 0 again (an L2 hit,
            // never used). With the exit path processing a buffer as well, the compiler hoists
            // the arithmetic shared by both paths above the exit test and keeps twice the
            // registers live; the empty asm keeps the loads from sinking below the arithmetic.
            for (;;) {
                const uint32_t b1 = base + stride;
                const bool more1 = b1 + kTile <= a.units;
                load(Pass<kWhole>(), more1 ? b1 : 0u, i1);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                process(Pass<kWhole>(), base, i0);
                base = b1;
                if (!more1) break;
                const uint32_t b2 = b1 + stride;
                const bool more2 = b2 + kTile <= a.units;
                load(Pass<kWhole>(), more2 ? b2 : 0u, i0);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                process(Pass<kWhole>(), b1, i1);
                base = b2;
                if (!more2) break;
            }
        } else {
            // Mostly one tile per workgroup: the exit path processes the buffer itself, so no
            // workgroup fetches a tile it does not use.
            for (;;) {
                const uint32_t b1 = base + stride;
                if (b1 + kTile > a.units) { process(Pass<kWhole>(), base, i0); base = b1; break; }
                load(Pass<kWhole>(), b1, i1);
                __builtin_amdgcn_sched_barrier(0);
                process(Pass<kWhole>(), base, i0);
                const uint32_t b2 = b1 + stride;
                if (b2 + kTile > a.units) { process(Pass<kWhole>(), b1, i1); base = b2; break; }
                load(Pass<kWhole>(), b2, i0);
                __builtin_amdgcn_sched_barrier(0);
                process(Pass<kWhole>(), b1, i1);
                base = b2;
            }
        }
    }
    if (base < a.units) {
        load(Pass<kPart>(), base, i0);
        process(Pass<kPart>(), base, i0);
    }
    if constexpr (STATS) {
        if (__builtin_amdgcn_ballot_w64(!finite_f64(acc.signal_sum())) != 0u) {
            // Inf/NaN in this wave's x: the whole tiles above took them unfiltered, so the wave
            // starts over on every tile with the per-element filter (rare; no stores)
            acc = Acc();
            wcnt = WaveCounts();
            for (uint32_t b = blockIdx.x * kTile; b < a.units; b += stride) {
                load(Pass<kRedo>(), b, i0);
                process(Pass<kRedo>(), b, i0);
            }
        }
    }
    if (MODE == kModeScaled && blockIdx.x == 0) {            // the last n % W elements
        const int64_t e = (int64_t)a.units * W + threadIdx.x;
        if (e < a.n) {
            const UnitScale us{s_tensor, 1.0f};
            const float xh = tab[a.q[e]];
            store1<OUTK>(a.out, e, xh);
            if constexpr (STATS) {
                float xe[1] = {load_x1<XK>(a.x, e)}, xhv[1] = {xh};
                bool sat[1] = {saturates<FMT, MODE>(xe[0], us)};
                acc_add_unit<1>(acc, xe, xhv, sat);
            }
        }
    }
    if constexpr (STATS) block_store_partial(acc, wcnt, a.parts + blockIdx.x);
}

// One workgroup folds the partials in a fixed order: thread t takes partials t, t + 256, ...
// (all loads in flight at once), then a shuffle tree in each wave and the waves in order.
__global__ __launch_bounds__(kDqThreads) void stats_finalize_kernel(const StatsPart *parts, int nparts,
                                                                    qf8_error_stats *out) {
    constexpr int kPer = kStatsGrid / kDqThreads;
    StatsPart p[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = (int)threadIdx.x + r * kDqThreads;
        p[r] = parts[i < nparts ? i : 0];               // beyond nparts: partial 0 read, not used
    }
    double sg = 0.0, ns = 0.0;
    uint64_t c[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < kPer; ++r) {                   // + 0 for the unused ones (sums are >= 0)
        const bool in = (int)threadIdx.x + r * kDqThreads < nparts;
        sg += in ? p[r].signal : 0.0; ns += in ? p[r].noise : 0.0;
        c[0] += in ? p[r].count : 0; c[1] += in ? p[r].nonzero : 0; c[2] += in ? p[r].zeroed : 0;
        c[3] += in ? p[r].saturated : 0; c[4] += in ? p[r].nonfinite : 0;
    }
    sg = wave_sum(sg);
    ns = wave_sum(ns);
#pragma unroll
    for (int k = 0; k < 5; ++k) c[k] = wave_sum(c[k]);
    __shared__ double sd[2][kDqThreads / 64];
    __shared__ uint64_t sc[5][kDqThreads / 64];
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sd[0][w] = sg; sd[1][w] = ns;
#pragma unroll
        for (int k = 0; k < 5; ++k) sc[k][w] = c[k];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        qf8_error_stats r{};
        for (int k = 0; k < kDqThreads / 64; ++k) {
            r.signal += sd[0][k]; r.noise += sd[1][k];
            r.count += (int64_t)sc[0][k]; r.nonzero += (int64_t)sc[1][k]; r.zeroed += (int64_t)sc[2][k];
            r.saturated += (int64_t)sc[3][k]; r.nonfinite += (int64_t)sc[4][k];
        }
        *out = r;
    }
}

template <int FMT, int MODE, int OUTK, int XK>
void launch_t(const DqArgs &a, int w, int grid, hipStream_t s) {
    if constexpr (XK != kNone) {
        if (w == 16)
            hipLaunchKernelGGL((dequant_kernel<FMT, MODE, OUTK, XK, 16>), dim3(grid), dim3(kDqThreads), 0, s, a);
        else
            hipLaunchKernelGGL((dequant_kernel<FMT, MODE, OUTK, XK, 4>), dim3(grid), dim3(kDqThreads), 0, s, a);
    } else {
        if (w == 8)
            hipLaunchKernelGGL((dequant_kernel<FMT, MODE, OUTK, XK, 8>), dim3(grid), dim3(kDqThreads), 0, s, a);
        else
            hipLaunchKernelGGL((dequant_kernel<FMT, MODE, OUTK, XK, 4>), dim3(grid), dim3(kDqThreads), 0, s, a);
    }
}
template <int FMT, int MODE, int OUTK>
void by_x(int xk, const DqArgs &a, int w, int grid, hipStream_t s) {
    if (xk == kBF16) launch_t<FMT, MODE, OUTK, kBF16>(a, w, grid, s);
    else if (xk == kFP32) launch_t<FMT, MODE, OUTK, kFP32>(a, w, grid, s);
    else if constexpr (OUTK != kNone) launch_t<FMT, MODE, OUTK, kNone>(a, w, grid, s);
}
template <int FMT, int MODE>
void by_out(int outk, int xk, const DqArgs &a, int w, int grid, hipStream_t s) {
    if (outk == kBF16) by_x<FMT, MODE, kBF16>(xk, a, w, grid, s);
    else if (outk == kFP32) by_x<FMT, MODE, kFP32>(xk, a, w, grid, s);
    else by_x<FMT, MODE, kNone>(xk, a, w, grid, s);
}
template <int MODE>
void by_fmt(int fmt, int outk, int xk, const DqArgs &a, int w, int grid, hipStream_t s) {
    if (fmt == QF8_E4M3) by_out<kE4M3, MODE>(outk, xk, a, w, grid, s);
    else by_out<kE5M2, MODE>(outk, xk, a, w, grid, s);
}

}  // namespace

int launch_dequant(int mode, int fmt, const uint8_t *q, int64_t rows, int64_t cols, int block_rows,
                   const float *scale, const uint8_t *sb, void *out, int out_dtype, const void *x, int x_dtype,
                   qf8_error_stats *stats, void *ws, hipStream_t s) {
    const int64_t n = rows * cols;
    const int outk = out ? (out_dtype == QF8_IN_BF16 ? kBF16 : kFP32) : kNone;
    const int xk = stats ? (x_dtype == QF8_IN_BF16 ? kBF16 : kFP32) : kNone;
    // Units stay inside one row (and so one group / MX block). With the statistics: 16 codes where
    // rows allow it, else 4. De-scaling alone: 8 codes for BF16 output where rows allow it, else 4.
    const bool whole_rows = mode == kModeScaled;
    const int w = stats ? ((whole_rows || cols % 16 == 0) ? 16 : 4)
                        : ((whole_rows || cols % 8 == 0) && outk == kBF16 ? 8 : 4);
    DqArgs a{};
    a.q = q;
    a.n = n;
    a.units = (uint32_t)(n / w);
    a.upr = (uint32_t)(cols / w);
    // floor(u / d) = (u * m) >> (31 + l) for all u < 2^31 with l = ceil(log2 d), m = ceil(2^(31+l) / d):
    // m d - 2^(31+l) = e lies in [0, d), so u m / 2^(31+l) = u / d + u e / (d 2^(31+l)) and the
    // second term is below 2^31 / 2^(31+l) <= 1 / d, too small to reach the next integer
    {
        const uint64_t d = a.upr > 0 ? a.upr : 1u;
        uint32_t l = 0;
        while ((1ull << l) < d) ++l;
        a.upr_shift = 31u + l;
        a.upr_mul = ((1ull << a.upr_shift) + d - 1) / d;
    }
    a.br_shift = block_rows == 128 ? 7u : 0u;
    a.gcols = (uint32_t)((cols + 127) / 128);
    a.scale = scale;
    a.sb = sb;
    a.out = out;
    a.x = x;
    a.parts = stats ? (StatsPart *)((uint32_t *)ws + kPartialsOffsetWords) : nullptr;
    const int64_t per_wg = (int64_t)kDqThreads * (32 / w);
    int64_t grid = ((int64_t)a.units + per_wg - 1) / per_wg;
    const int cap = stats ? kStatsGrid : kDqMaxGrid;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    if (n > 0 || stats) {
        if (mode == kModeScaled) by_fmt<kModeScaled>(fmt, outk, xk, a, w, (int)grid, s);
        else if (mode == kModeBlock) by_fmt<kModeBlock>(fmt, outk, xk, a, w, (int)grid, s);
        else by_fmt<kModeMx>(fmt, outk, xk, a, w, (int)grid, s);
    }
    if (stats)
        hipLaunchKernelGGL(stats_finalize_kernel, dim3(1), dim3(kDqThreads), 0, s, a.parts, (int)grid, stats);
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
