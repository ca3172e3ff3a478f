// qf8_tensor.hip -- per-tensor current scaling, delayed scaling and the plain scaled cast.
//
// Pages (title, section):
//   [HiF8-train] "HiFloat8：高性能训练之路" (hifloat.gccorg.com blog): section 1.2 Eq.(1)-(4)
//                (current and delayed scaling, amax history, Interval), section 5.2 (first step
//                after a (re)start is current scaling).
//   [MP-FP8]     "混合精度与 FP8 训练" (hs-black.github.io): section 8.1 (S = F8max/amax,
//                saturation), 8.2 (delayed scaling fuses the amax into the producing pass).
//
// Kernels (all HBM-bandwidth bound; 256 threads, 16-byte vector loads):
//   amax_partials  -- each workgroup reduces a contiguous chunk of |x| bit patterns to one u32.
//   cast_current   -- each workgroup first folds all partials into amax and S (so no separate
//                     single-wave finalize launch is needed), then casts its chunk with
//                     non-temporal 16-byte loads and 16-byte stores.
//   cast_scaled    -- cast with a scale read from device memory; optionally also emits the
//                     chunk's partial max (the fused amax of a delayed-scaling step).
//   delayed_finalize -- one workgroup: amax of the step, FIFO push on update steps, next scale.
#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kAbs16x2 = 0x7FFF7FFFu;

__device__ __forceinline__ uint32_t block_max_bcast(uint32_t v, uint32_t *red) {
    v = max_wave(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint32_t m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    __syncthreads();
    return m;
}

// |x| maximum of one 16-byte vector, accumulated as fp32 bit patterns (BF16 kept packed).
template <bool BF16>
__device__ __forceinline__ uint32_t vec_absmax(uint32_t acc, uint4 v) {
    if constexpr (BF16) {
        acc = pk_max_u16(acc, v.x & kAbs16x2);
        acc = pk_max_u16(acc, v.y & kAbs16x2);
        acc = pk_max_u16(acc, v.z & kAbs16x2);
        acc = pk_max_u16(acc, v.w & kAbs16x2);
    } else {
        acc = umax(acc, v.x & 0x7FFFFFFFu);
        acc = umax(acc, v.y & 0x7FFFFFFFu);
        acc = umax(acc, v.z & 0x7FFFFFFFu);
        acc = umax(acc, v.w & 0x7FFFFFFFu);
    }
    return acc;
}
// accumulator -> fp32 bit pattern of |amax|
template <bool BF16>
__device__ __forceinline__ uint32_t acc_to_f32bits(uint32_t acc) {
    if constexpr (BF16) return umax(acc & 0xFFFFu, acc >> 16) << 16;
    else return acc;
}
template <bool BF16>
__device__ __forceinline__ uint32_t elem_bits(const void *x, int64_t i) {
    if constexpr (BF16) return (uint32_t)((const uint16_t *)x)[i] << 16;
    else return ((const uint32_t *)x)[i];
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(const void *__restrict__ x, int64_t n, int64_t nvec,
                                                                 int64_t chunk, uint32_t *__restrict__ partials) {
    constexpr int VEC = BF16 ? 8 : 4;
    __shared__ uint32_t red[4];
    const uint4 *xv = (const uint4 *)x;
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = beg + chunk < nvec ? beg + chunk : nvec;
    uint32_t a0 = 0, a1 = 0;
    int64_t i = beg + threadIdx.x;
    for (; i + 3 * kThreads < end; i += 4 * kThreads) {
        uint4 v0 = xv[i], v1 = xv[i + kThreads], v2 = xv[i + 2 * kThreads], v3 = xv[i + 3 * kThreads];
        a0 = vec_absmax<BF16>(a0, v0);
        a1 = vec_absmax<BF16>(a1, v1);
        a0 = vec_absmax<BF16>(a0, v2);
        a1 = vec_absmax<BF16>(a1, v3);
    }
    for (; i < end; i += kThreads) a0 = vec_absmax<BF16>(a0, xv[i]);
    uint32_t m = umax(acc_to_f32bits<BF16>(a0), acc_to_f32bits<BF16>(a1));
    if (blockIdx.x == gridDim.x - 1)                               // ragged tail
        for (int64_t e = nvec * VEC + threadIdx.x; e < n; e += kThreads) m = umax(m, elem_bits<BF16>(x, e) & 0x7FFFFFFFu);
    m = block_max_bcast(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// One output unit = 16 codes = 16 bytes, from UV 16-byte input vectors (2 BF16, 4 FP32).
template <bool BF16>
constexpr int unit_vectors() { return BF16 ? 2 : 4; }
template <bool BF16>
constexpr int unit_elems() { return 16; }

template <bool BF16, int FMT>
__device__ __forceinline__ uint4 cast_unit(const uint4 *v, float s) {
    if constexpr (BF16) {
        const uint2 a = cast8_bf16<FMT>(v[0], s), b = cast8_bf16<FMT>(v[1], s);
        return make_uint4(a.x, a.y, b.x, b.y);
    } else {
        return make_uint4(cast4_f32<FMT>(v[0], s), cast4_f32<FMT>(v[1], s), cast4_f32<FMT>(v[2], s),
                          cast4_f32<FMT>(v[3], s));
    }
}

// Casts units [beg, end) of the chunk plus, for the last chunk, the elements past the last whole
// unit. Streaming loads and stores (read once, written once). Returns the |x| maximum (fp32
// bits) of everything it read when FUSE.
template <bool BF16, int FMT, bool FUSE>
__device__ __forceinline__ uint32_t cast_chunk(const void *__restrict__ x, int64_t n, int64_t nunits, int64_t beg,
                                               int64_t end, bool last, float s, uint8_t *__restrict__ q) {
    constexpr int UV = unit_vectors<BF16>();
    const uint4 *xv = (const uint4 *)x;
    uint4 *qv = (uint4 *)q;
    uint32_t a0 = 0, a1 = 0;
    int64_t i = beg + threadIdx.x;
    for (; i + kThreads < end; i += 2 * kThreads) {          // two units per thread in flight
        uint4 v[2][UV];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int u = 0; u < UV; ++u) v[k][u] = ld_stream(xv + (i + k * kThreads) * UV + u);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if constexpr (FUSE) {
#pragma unroll
                for (int u = 0; u < UV; ++u) {
                    if (u & 1) a1 = vec_absmax<BF16>(a1, v[k][u]);
                    else a0 = vec_absmax<BF16>(a0, v[k][u]);
                }
            }
            st_stream(qv + i + k * kThreads, cast_unit<BF16, FMT>(v[k], s));
        }
    }
    for (; i < end; i += kThreads) {
        uint4 v[UV];
#pragma unroll
        for (int u = 0; u < UV; ++u) v[u] = ld_stream(xv + i * UV + u);
        if constexpr (FUSE) {
#pragma unroll
            for (int u = 0; u < UV; ++u) a0 = vec_absmax<BF16>(a0, v[u]);
        }
        st_stream(qv + i, cast_unit<BF16, FMT>(v, s));
    }
    uint32_t m = 0;
    if constexpr (FUSE) m = umax(acc_to_f32bits<BF16>(a0), acc_to_f32bits<BF16>(a1));
    if (last) {
        for (int64_t e = nunits * unit_elems<BF16>() + threadIdx.x; e < n; e += kThreads) {
            const uint32_t b = elem_bits<BF16>(x, e);
            if constexpr (FUSE) m = umax(m, b & 0x7FFFFFFFu);
            q[e] = (uint8_t)cast1<FMT>(__uint_as_float(b), s);
        }
    }
    return m;
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(kThreads) void cast_current_kernel(const void *__restrict__ x, int64_t n, int64_t nunits,
                                                                int64_t chunk, uint8_t *__restrict__ q,
                                                                const uint32_t *__restrict__ partials, int nparts,
                                                                float *amax_out, float *scale_out, int32_t *nonfinite) {
    __shared__ uint32_t red[4];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) m = umax(m, partials[i]);
    m = block_max_bcast(m, red);
    const float s = scale_from_amax_bits<FMT>(m);
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = beg + chunk < nunits ? beg + chunk : nunits;
    cast_chunk<BF16, FMT, false>(x, n, nunits, beg, end, blockIdx.x == gridDim.x - 1, s, q);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (amax_out) *amax_out = __uint_as_float(m);
        if (scale_out) *scale_out = s;
        if (nonfinite && m >= 0x7F800000u) *nonfinite = 1;
    }
}

template <bool BF16, int FMT, bool FUSE>
__global__ __launch_bounds__(kThreads) void cast_scaled_kernel(const void *__restrict__ x, int64_t n, int64_t nunits,
                                                               int64_t chunk, const float *__restrict__ scale,
                                                               uint8_t *__restrict__ q, float *scale_used,
                                                               uint32_t *__restrict__ partials) {
    __shared__ uint32_t red[4];
    const float s = *scale;
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = beg + chunk < nunits ? beg + chunk : nunits;
    uint32_t m = cast_chunk<BF16, FMT, FUSE>(x, n, nunits, beg, end, blockIdx.x == gridDim.x - 1, s, q);
    if constexpr (FUSE) {
        m = block_max_bcast(m, red);
        if (threadIdx.x == 0) partials[blockIdx.x] = m;
    }
    if (scale_used && blockIdx.x == 0 && threadIdx.x == 0) *scale_used = s;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void delayed_finalize_kernel(const uint32_t *__restrict__ partials, int nparts,
                                                                    float *history, int32_t *meta, float *scale,
                                                                    int hist_len, int n_guard, int update,
                                                                    float *amax_out, int32_t *nonfinite) {
    __shared__ uint32_t red[4];
    __shared__ int sh_count, sh_slot;
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) m = umax(m, partials[i]);
    m = block_max_bcast(m, red);
    const bool bad = m >= 0x7F800000u;
    if (threadIdx.x == 0) {
        if (amax_out) *amax_out = __uint_as_float(m);
        if (bad && nonfinite) *nonfinite = 1;
        int count = meta[0], head = meta[1], slot = -1;
        if (update && !bad) {                                        // append; drop the oldest when full
            if (count < hist_len) {                                  // head stays 0 while filling
                slot = count;
                meta[0] = ++count;
            } else {
                slot = head;
                meta[1] = head + 1 == hist_len ? 0 : head + 1;
            }
            history[slot] = __uint_as_float(m);
        }
        sh_count = count;
        sh_slot = slot;
    }
    __syncthreads();
    // estimate = max of the history: slots [0, count) are the valid ones, in any order. The slot
    // written above is taken from the register of thread 0, not re-read from memory.
    const int count = sh_count, slot = sh_slot;
    uint32_t e = 0;
    for (int i = threadIdx.x; i < count; i += kThreads)
        if (i != slot) e = umax(e, __float_as_uint(history[i]));
    if (threadIdx.x == 0 && slot >= 0) e = umax(e, m);
    e = block_max_bcast(e, red);
    if (threadIdx.x == 0) {
        const float margin = __uint_as_float((uint32_t)(127 - n_guard) << 23);   // 2^-N, exact
        *scale = scale_from_amax_bits<FMT>(e) * margin;
    }
}

__global__ void fill_u32_kernel(uint32_t *p, int64_t n, uint32_t value) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

inline int64_t vec_count(int64_t n, int dtype) { return n / (dtype == QF8_IN_BF16 ? 8 : 4); }
inline int64_t unit_count(int64_t n) { return n / 16; }
inline int64_t chunk_of(int64_t nvec, int grid) { return (nvec + grid - 1) / grid; }
inline int status_after_launch() { return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP; }

}  // namespace

int stream_grid(int64_t n, int dtype) {
    int64_t nvec = vec_count(n, dtype);
    int64_t g = (nvec + 2047) / 2048;
    if (g < 1) g = 1;
    if (g > kStreamGridCap) g = kStreamGridCap;
    return (int)g;
}

#define QF8_DISPATCH_DT_FMT(dtype, fmt, KERNEL_CALL)                                           \
    do {                                                                                       \
        if (dtype == QF8_IN_BF16 && fmt == QF8_E4M3) { constexpr bool BF16 = true; constexpr int FMT = kE4M3; KERNEL_CALL; } \
        else if (dtype == QF8_IN_BF16) { constexpr bool BF16 = true; constexpr int FMT = kE5M2; KERNEL_CALL; }               \
        else if (fmt == QF8_E4M3) { constexpr bool BF16 = false; constexpr int FMT = kE4M3; KERNEL_CALL; }                   \
        else { constexpr bool BF16 = false; constexpr int FMT = kE5M2; KERNEL_CALL; }                                        \
    } while (0)

int launch_amax_partials(const void *x, int dtype, int64_t n, uint32_t *partials, int grid, hipStream_t s) {
    const int64_t nvec = vec_count(n, dtype);
    const int64_t chunk = chunk_of(nvec, grid);
    if (dtype == QF8_IN_BF16)
        hipLaunchKernelGGL(amax_partials_kernel<true>, dim3(grid), dim3(kThreads), 0, s, x, n, nvec, chunk, partials);
    else
        hipLaunchKernelGGL(amax_partials_kernel<false>, dim3(grid), dim3(kThreads), 0, s, x, n, nvec, chunk, partials);
    return status_after_launch();
}

int launch_cast_current(const void *x, int dtype, int64_t n, int fmt, uint8_t *q, const uint32_t *partials,
                        int nparts, float *amax_out, float *scale_out, int32_t *nonfinite, int grid, hipStream_t s) {
    const int64_t nunits = unit_count(n);
    const int64_t chunk = chunk_of(nunits, grid);
    QF8_DISPATCH_DT_FMT(dtype, fmt,
        hipLaunchKernelGGL((cast_current_kernel<BF16, FMT>), dim3(grid), dim3(kThreads), 0, s, x, n, nunits, chunk, q,
                           partials, nparts, amax_out, scale_out, nonfinite));
    return status_after_launch();
}

int launch_cast_scaled(const void *x, int dtype, int64_t n, int fmt, const float *scale, uint8_t *q,
                       float *scale_used, uint32_t *partials_out, int grid, hipStream_t s) {
    const int64_t nunits = unit_count(n);
    const int64_t chunk = chunk_of(nunits, grid);
    if (partials_out)
        QF8_DISPATCH_DT_FMT(dtype, fmt,
            hipLaunchKernelGGL((cast_scaled_kernel<BF16, FMT, true>), dim3(grid), dim3(kThreads), 0, s, x, n, nunits,
                               chunk, scale, q, scale_used, partials_out));
    else
        QF8_DISPATCH_DT_FMT(dtype, fmt,
            hipLaunchKernelGGL((cast_scaled_kernel<BF16, FMT, false>), dim3(grid), dim3(kThreads), 0, s, x, n, nunits,
                               chunk, scale, q, scale_used, partials_out));
    return status_after_launch();
}

int launch_delayed_finalize(const uint32_t *partials, int nparts, float *history, int32_t *meta, float *scale,
                            int hist_len, int n_guard, int fmt, int update, float *amax_out,
                            int32_t *nonfinite, hipStream_t s) {
    if (fmt == QF8_E4M3)
        hipLaunchKernelGGL(delayed_finalize_kernel<kE4M3>, dim3(1), dim3(kThreads), 0, s, partials, nparts, history,
                           meta, scale, hist_len, n_guard, update, amax_out, nonfinite);
    else
        hipLaunchKernelGGL(delayed_finalize_kernel<kE5M2>, dim3(1), dim3(kThreads), 0, s, partials, nparts, history,
                           meta, scale, hist_len, n_guard, update, amax_out, nonfinite);
    return status_after_launch();
}

int launch_fill_u32(uint32_t *p, int64_t n, uint32_t value, hipStream_t s) {
    if (n <= 0) return QF8_OK;
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 1024) g = 1024;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, p, n, value);
    return status_after_launch();
}

}  // namespace qf8
