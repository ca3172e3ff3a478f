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
// Work: a unit is 4 consecutive codes (one dword of q). A thread takes 4 units per iteration
// (consecutive threads on consecutive units, so each load instruction of a wave covers 256
// contiguous bytes of q), decodes with the gfx950 fp8/bf8 -> f32 converts (exact), de-scales
// and stores 4 BF16 (8 bytes) or 4 FP32 (16 bytes) per unit. Group scales and E8M0 bytes are
// read per unit and hit in cache. With statistics, each workgroup reduces its fp64 sums and
// counts in a fixed order into a 64-byte partial in the workspace, and one workgroup folds the
// partials in a fixed order: the same input always gives the same bits.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kDqThreads = 256;
constexpr int kUnitsPerThread = 4;
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
    uint32_t units;              // whole 4-code units
    uint32_t upr;                // units per row (block, MX)
    uint32_t br;                 // block rows (block)
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

// fp32 -> BF16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct Acc {
    double signal = 0.0, noise = 0.0;
    uint32_t count = 0, nonzero = 0, zeroed = 0, saturated = 0, nonfinite = 0;
    __device__ __forceinline__ void add(float x, float xh, bool sat) {
        if (!(fabsf(x) <= 3.40282346638528859812e+38f)) { ++nonfinite; return; }
        ++count;
        const double xd = (double)x, d = xd - (double)xh;
        signal += xd * xd;
        noise += d * d;
        if (x != 0.0f) {
            ++nonzero;
            if (xh == 0.0f) ++zeroed;
        }
        if (sat) ++saturated;
    }
};

template <int XK>
__device__ __forceinline__ void load_x4(const void *x, uint32_t u, float *xv) {
    if constexpr (XK == kBF16) {
        const uint2 w = ((const uint2 *)x)[u];
        xv[0] = __uint_as_float(w.x << 16); xv[1] = __uint_as_float(w.x & 0xFFFF0000u);
        xv[2] = __uint_as_float(w.y << 16); xv[3] = __uint_as_float(w.y & 0xFFFF0000u);
    } else {
        const float4 w = ((const float4 *)x)[u];
        xv[0] = w.x; xv[1] = w.y; xv[2] = w.z; xv[3] = w.w;
    }
}
template <int XK>
__device__ __forceinline__ float load_x1(const void *x, int64_t e) {
    if constexpr (XK == kBF16) return __uint_as_float((uint32_t)((const uint16_t *)x)[e] << 16);
    else return ((const float *)x)[e];
}

template <int OUTK>
__device__ __forceinline__ void store4(void *out, uint32_t u, const float *v) {
    if constexpr (OUTK == kBF16) {
        ((uint2 *)out)[u] = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
    } else if constexpr (OUTK == kFP32) {
        ((float4 *)out)[u] = make_float4(v[0], v[1], v[2], v[3]);
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

template <int FMT, int MODE>
__device__ __forceinline__ UnitScale unit_scale(const DqArgs &a, uint32_t u, float s_tensor) {
    UnitScale us{s_tensor, 0, false};
    if constexpr (MODE == kModeBlock) {
        const uint32_t r = u / a.upr, c = (u - r * a.upr) * 4u;
        us.s = a.scale[(size_t)(r / a.br) * a.gcols + (c >> 7)];
    } else if constexpr (MODE == kModeMx) {
        const uint32_t r = u / a.upr, c = (u - r * a.upr) * 4u;
        const uint32_t b = a.sb[(size_t)r * (a.upr >> 3) + (c >> 5)];
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
    const double sg = wave_sum(acc.signal), ns = wave_sum(acc.noise);
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

template <int FMT, int MODE, int OUTK, int XK>
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(DqArgs a) {
    constexpr bool STATS = XK != kNone;
    const float s_tensor = MODE == kModeScaled ? *a.scale : 1.0f;
    Acc acc;
    const uint32_t *q32 = (const uint32_t *)a.q;
    const uint32_t stride = gridDim.x * kDqThreads * kUnitsPerThread;
    for (uint32_t base = blockIdx.x * kDqThreads * kUnitsPerThread; base < a.units; base += stride) {
        uint32_t codes[kUnitsPerThread];
        float xv[kUnitsPerThread][4];
#pragma unroll
        for (int j = 0; j < kUnitsPerThread; ++j) {
            const uint32_t u = base + j * kDqThreads + threadIdx.x;
            codes[j] = u < a.units ? __builtin_nontemporal_load(q32 + u) : 0u;
            if constexpr (STATS) {
                if (u < a.units) load_x4<XK>(a.x, u, xv[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kUnitsPerThread; ++j) {
            const uint32_t u = base + j * kDqThreads + threadIdx.x;
            if (u >= a.units) continue;
            const UnitScale us = unit_scale<FMT, MODE>(a, u, s_tensor);
            float v[4];
            decode4<FMT>(codes[j], v);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = descale<MODE>(v[k], us);
            store4<OUTK>(a.out, u, v);
            if constexpr (STATS) {
#pragma unroll
                for (int k = 0; k < 4; ++k) acc.add(xv[j][k], v[k], saturates<FMT, MODE>(xv[j][k], us));
            }
        }
    }
    if (MODE == kModeScaled && blockIdx.x == 0) {            // the last n % 4 elements
        const int64_t e = (int64_t)a.units * 4 + threadIdx.x;
        if (e < a.n) {
            const UnitScale us{s_tensor, 0, false};
            float v[4];
            decode4<FMT>(a.q[e], v);
            const float xh = descale<MODE>(v[0], us);
            store1<OUTK>(a.out, e, xh);
            if constexpr (STATS) {
                const float xe = load_x1<XK>(a.x, e);
                acc.add(xe, xh, saturates<FMT, MODE>(xe, us));
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
void launch_t(const DqArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((dequant_kernel<FMT, MODE, OUTK, XK>), dim3(grid), dim3(kDqThreads), 0, s, a);
}
template <int FMT, int MODE, int OUTK>
void by_x(int xk, const DqArgs &a, int grid, hipStream_t s) {
    if (xk == kBF16) launch_t<FMT, MODE, OUTK, kBF16>(a, grid, s);
    else if (xk == kFP32) launch_t<FMT, MODE, OUTK, kFP32>(a, grid, s);
    else if constexpr (OUTK != kNone) launch_t<FMT, MODE, OUTK, kNone>(a, grid, s);
}
template <int FMT, int MODE>
void by_out(int outk, int xk, const DqArgs &a, int grid, hipStream_t s) {
    if (outk == kBF16) by_x<FMT, MODE, kBF16>(xk, a, grid, s);
    else if (outk == kFP32) by_x<FMT, MODE, kFP32>(xk, a, grid, s);
    else by_x<FMT, MODE, kNone>(xk, a, grid, s);
}
template <int MODE>
void by_fmt(int fmt, int outk, int xk, const DqArgs &a, int grid, hipStream_t s) {
    if (fmt == QF8_E4M3) by_out<kE4M3, MODE>(outk, xk, a, grid, s);
    else by_out<kE5M2, MODE>(outk, xk, a, grid, s);
}

}  // namespace

int launch_dequant(int mode, int fmt, const uint8_t *q, int64_t rows, int64_t cols, int block_rows,
                   const float *scale, const uint8_t *sb, void *out, int out_dtype, const void *x, int x_dtype,
                   qf8_error_stats *stats, void *ws, hipStream_t s) {
    const int64_t n = rows * cols;
    DqArgs a{};
    a.q = q;
    a.n = n;
    a.units = (uint32_t)(n / 4);
    a.upr = (uint32_t)(cols / 4);
    a.br = (uint32_t)(block_rows > 0 ? block_rows : 1);
    a.gcols = (uint32_t)((cols + 127) / 128);
    a.scale = scale;
    a.sb = sb;
    a.out = out;
    a.x = x;
    a.parts = stats ? (StatsPart *)((uint32_t *)ws + kPartialsOffsetWords) : nullptr;
    const int outk = out ? (out_dtype == QF8_IN_BF16 ? kBF16 : kFP32) : kNone;
    const int xk = stats ? (x_dtype == QF8_IN_BF16 ? kBF16 : kFP32) : kNone;
    const int64_t per_wg = (int64_t)kDqThreads * kUnitsPerThread;
    int64_t grid = ((int64_t)a.units + per_wg - 1) / per_wg;
    const int cap = stats ? kStatsGrid : kDqMaxGrid;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    if (n > 0 || stats) {
        const int md = mode;
        if (md == kModeScaled) by_fmt<kModeScaled>(fmt, outk, xk, a, (int)grid, s);
        else if (md == kModeBlock) by_fmt<kModeBlock>(fmt, outk, xk, a, (int)grid, s);
        else by_fmt<kModeMx>(fmt, outk, xk, a, (int)grid, s);
    }
    if (stats)
        hipLaunchKernelGGL(stats_finalize_kernel, dim3(1), dim3(kDqThreads), 0, s, a.parts, (int)grid, stats);
    return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP;
}

}  // namespace qf8
