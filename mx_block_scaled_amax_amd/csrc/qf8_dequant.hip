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
// one MX block, so its scale is looked up once. A thread takes 32 codes per iteration (16 with
// statistics), consecutive threads on consecutive units, and loads the next iteration's codes
// and inputs before the current one's arithmetic; decodes with the gfx950 fp8/bf8 -> f32 converts
// (exact), de-scales (MX: ldexp; groups: IEEE division; one tensor scale: a 256-entry LDS table
// of decode(c) / S built per workgroup) and stores each 8-code BF16 or 4-code FP32 unit as one
// 16-byte piece, consecutive lanes on consecutive pieces. With statistics, the fp64
// terms go to 4 independent running sums per thread (short dependency chains); each
// workgroup reduces its sums and counts in a fixed order into a 64-byte partial in the
// workspace, and one workgroup folds the partials in a fixed order: the same input always gives
// the same bits.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kDqThreads = 256;
constexpr int kDqMaxGrid = 16384;
constexpr int kStatsGrid = 1024;                 // workgroups (= 64-byte partials) with statistics
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

// W consecutive elements of x (W = 4 or 16: the units of the statistics) of unit u.
template <int XK, int W>
__device__ __forceinline__ void load_x(const void *x, uint32_t u, float *xv) {
    static_assert(W == 4 || W == 16, "statistics units");
    if constexpr (XK == kBF16) {
        const uint32_t *p = (const uint32_t *)x + (size_t)u * (W / 2);
        uint32_t w[W / 2];
        if constexpr (W == 16) {
            const uint4 a0 = ((const uint4 *)p)[0], a1 = ((const uint4 *)p)[1];
            w[0] = a0.x; w[1] = a0.y; w[2] = a0.z; w[3] = a0.w; w[4] = a1.x; w[5] = a1.y; w[6] = a1.z; w[7] = a1.w;
        } else {
            const uint2 a0 = *(const uint2 *)p;
            w[0] = a0.x; w[1] = a0.y;
        }
#pragma unroll
        for (int k = 0; k < W / 2; ++k) {
            xv[2 * k] = __uint_as_float(w[k] << 16);
            xv[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = (const float4 *)x + (size_t)u * (W / 4);
#pragma unroll
        for (int k = 0; k < W / 4; ++k) {
            const float4 f = p[k];
            xv[4 * k] = f.x; xv[4 * k + 1] = f.y; xv[4 * k + 2] = f.z; xv[4 * k + 3] = f.w;
        }
    }
}
// The same in two steps: the raw dwords (BF16 pairs or fp32 bits) of unit u, loaded a loop
// iteration ahead, then their fp32 values.
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

// How one unit is de-scaled: a scale factor S (divide) or an E8M0 byte (ldexp).
struct UnitScale {
    float s;      // S, or F8max * 2^X for MX saturation tests
    int xexp;     // X (MX)
    bool nan;     // MX byte 0xFF
};

// Row of unit u (u < 2^31) without a division instruction sequence: the multiplier and shift are
// computed on the host (round-up reciprocal, exact below 2^31; see launch_dequant).
__device__ __forceinline__ uint32_t unit_row(const DqArgs &a, uint32_t u) {
    return (uint32_t)(((uint64_t)u * a.upr_mul) >> a.upr_shift);
}

// Scale of unit u (W codes, all in one row and one group: cols % W == 0, W divides 32 and 128).
template <int FMT, int MODE, int W>
__device__ __forceinline__ UnitScale unit_scale(const DqArgs &a, uint32_t u, float s_tensor) {
    UnitScale us{s_tensor, 0, false};
    if constexpr (MODE == kModeBlock) {
        const uint32_t r = unit_row(a, u), c = (u - r * a.upr) * W;
        us.s = a.scale[(size_t)(r >> a.br_shift) * a.gcols + (c >> 7)];
    } else if constexpr (MODE == kModeMx) {
        const uint32_t r = unit_row(a, u), c = (u - r * a.upr) * W;
        const uint32_t b = a.sb[(size_t)r * (a.upr * W / 32) + (c >> 5)];
        us.nan = b == 0xFFu;
        us.xexp = (int)b - 127;
        us.s = __builtin_ldexpf(F8<FMT>::kMax, us.xexp);
    }
    return us;
}

template <int MODE>
__device__ __forceinline__ float descale(float v, const UnitScale &us) {
    if constexpr (MODE == kModeMx) return us.nan ? __uint_as_float(0x7FC00000u) : __builtin_ldexpf(v, us.xexp);
    else return v / us.s;
}

template <int FMT, int MODE>
__device__ __forceinline__ bool saturates(float x, const UnitScale &us) {
    if constexpr (MODE == kModeMx) return !us.nan && fabsf(x) > us.s;
    else return fabsf(x * us.s) > F8<FMT>::kMax;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Fixed-order workgroup sum of the accumulator into one partial (thread 0 writes it).
__device__ void block_store_partial(const Acc &acc, StatsPart *dst) {
    __shared__ double sd[2][kDqThreads / 64];
    __shared__ uint32_t sc[5][kDqThreads / 64];
    const double sg = wave_sum(acc.signal_sum()), ns = wave_sum(acc.noise_sum());
    const uint32_t c0 = wave_sum(acc.count), c1 = wave_sum(acc.nonzero), c2 = wave_sum(acc.zeroed),
                   c3 = wave_sum(acc.saturated), c4 = wave_sum(acc.nonfinite);
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

// W codes per unit. De-scaling alone takes 8 or 4, so that each lane moves one 16-byte piece of the
// output and consecutive lanes move consecutive pieces: 8 codes (an 8-byte load) make 16 bytes of
// BF16, 4 codes 16 bytes of FP32, and whole 16-byte outputs leave as non-temporal stores (a lane
// writing 32 bytes as two 16-byte stores leaves every store instruction half-dense over its span,
// which measured ~10% slower for this stream). With the statistics, whose fp64 terms make the
// kernel VALU-bound, 16-code units (one 16-byte load of codes) halve the per-unit overhead.
// 4-code units also serve rows that are only a multiple of 4 codes long (8-byte BF16 stores,
// cached so that L2 merges them). With one scale factor the workgroup first tabulates
// fl32(decode(c) / S) for all 256 codes in LDS, so an element costs a table read, not a division.
template <int FMT, int MODE, int OUTK, int XK, int W>
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(DqArgs a) {
    constexpr bool STATS = XK != kNone;
    static_assert(W == 16 || W == 8 || W == 4, "16-, 8- or 4-code units");
    // units per thread and iteration: 32 codes, or 16 with the statistics (two iterations' raw
    // inputs are held at once, below)
    constexpr int UPT = (STATS ? 16 : 32) / W;
    constexpr int ND = W / 4;                     // dwords of codes per unit
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
    const uint32_t stride = gridDim.x * kDqThreads * UPT;
    constexpr int XD = STATS ? x_raw_dwords<XK == kNone ? kBF16 : XK, W == 8 ? 16 : W>() : 1;
    // one iteration's codes and raw x, loaded one iteration ahead of their arithmetic (two
    // buffers, the loop unrolled by two), so that the loads of the next 32 codes per thread are in
    // flight during the current ones' de-scaling and statistics
    auto load_iter = [&](uint32_t base, uint32_t (&codes)[UPT][ND], uint32_t (&xr)[UPT][XD]) {
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const uint32_t u = base + j * kDqThreads + threadIdx.x;
            if (u < a.units) {
                if constexpr (W == 16) {
                    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
                    const v4u c = __builtin_nontemporal_load((const v4u *)a.q + u);
                    codes[j][0] = c.x; codes[j][1] = c.y; codes[j][2] = c.z; codes[j][3] = c.w;
                } else if constexpr (W == 8) {
                    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
                    const v2u c = __builtin_nontemporal_load((const v2u *)a.q + u);
                    codes[j][0] = c.x; codes[j][1] = c.y;
                } else {
                    codes[j][0] = __builtin_nontemporal_load((const uint32_t *)a.q + u);
                }
                if constexpr (STATS) load_x_raw<XK, W>(a.x, u, xr[j]);
            }
        }
    };
    auto process = [&](uint32_t base, const uint32_t (&codes)[UPT][ND], const uint32_t (&xr)[UPT][XD]) {
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const uint32_t u = base + j * kDqThreads + threadIdx.x;
            if (u >= a.units) continue;
            const UnitScale us = unit_scale<FMT, MODE, W>(a, u, s_tensor);
            float v[W];
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                if constexpr (MODE == kModeScaled) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[4 * d + k] = tab[(codes[j][d] >> (8 * k)) & 0xFFu];
                } else {
                    decode4<FMT>(codes[j][d], v + 4 * d);
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[4 * d + k] = descale<MODE>(v[4 * d + k], us);
                }
            }
            store_out<OUTK, W>(a.out, u, v);
            if constexpr (STATS) {
                float xv[W];
                x_from_raw<XK, W>(xr[j], xv);
                bool sat[W];
#pragma unroll
                for (int k = 0; k < W; ++k) sat[k] = saturates<FMT, MODE>(xv[k], us);
                acc_add_unit<W>(acc, xv, v, sat);
            }
        }
    };
    uint32_t c0[UPT][ND], c1[UPT][ND], x0[UPT][XD], x1[UPT][XD];
    uint32_t base = blockIdx.x * kDqThreads * UPT;
    if (base < a.units) load_iter(base, c0, x0);
    for (; base < a.units; base += 2 * stride) {
        const uint32_t b1 = base + stride;
        if (b1 < a.units) load_iter(b1, c1, x1);
        process(base, c0, x0);
        if (b1 >= a.units) break;
        if (b1 + stride < a.units) load_iter(b1 + stride, c0, x0);
        process(b1, c1, x1);
    }
    if (MODE == kModeScaled && blockIdx.x == 0) {            // the last n % W elements
        const int64_t e = (int64_t)a.units * W + threadIdx.x;
        if (e < a.n) {
            const UnitScale us{s_tensor, 0, false};
            const float xh = tab[a.q[e]];
            store1<OUTK>(a.out, e, xh);
            if constexpr (STATS) {
                float xe[1] = {load_x1<XK>(a.x, e)}, xhv[1] = {xh};
                bool sat[1] = {saturates<FMT, MODE>(xe[0], us)};
                acc_add_unit<1>(acc, xe, xhv, sat);
            }
        }
    }
    if constexpr (STATS) block_store_partial(acc, a.parts + blockIdx.x);
}

__global__ __launch_bounds__(kDqThreads) void stats_finalize_kernel(const StatsPart *parts, int nparts,
                                                                    qf8_error_stats *out) {
    double sg = 0.0, ns = 0.0;
    uint64_t c[5] = {0, 0, 0, 0, 0};
    for (int i = threadIdx.x; i < nparts; i += kDqThreads) {
        const StatsPart p = parts[i];
        sg += p.signal; ns += p.noise;
        c[0] += p.count; c[1] += p.nonzero; c[2] += p.zeroed; c[3] += p.saturated; c[4] += p.nonfinite;
    }
    __shared__ double sd[2][kDqThreads];
    __shared__ uint64_t sc[5][kDqThreads];
    sd[0][threadIdx.x] = sg; sd[1][threadIdx.x] = ns;
    for (int k = 0; k < 5; ++k) sc[k][threadIdx.x] = c[k];
    __syncthreads();
    for (int half = kDqThreads / 2; half > 0; half >>= 1) {     // fixed-order tree
        if ((int)threadIdx.x < half) {
            sd[0][threadIdx.x] += sd[0][threadIdx.x + half];
            sd[1][threadIdx.x] += sd[1][threadIdx.x + half];
            for (int k = 0; k < 5; ++k) sc[k][threadIdx.x] += sc[k][threadIdx.x + half];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        qf8_error_stats r;
        r.signal = sd[0][0]; r.noise = sd[1][0];
        r.count = (int64_t)sc[0][0]; r.nonzero = (int64_t)sc[1][0]; r.zeroed = (int64_t)sc[2][0];
        r.saturated = (int64_t)sc[3][0]; r.nonfinite = (int64_t)sc[4][0]; r.reserved = 0;
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
