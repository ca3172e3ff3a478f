// qf8_tensor.hip -- per-tensor current scaling, delayed scaling and the plain scaled cast.
//
// Pages (title, section):
//   [HiF8-train] "HiFloat8：高性能训练之路" (hifloat.gccorg.com blog): section 1.2 Eq.(1)-(4)
//                (current and delayed scaling, amax history, Interval), section 5.2 (first step
//                after a (re)start is current scaling).
//   [MP-FP8]     "混合精度与 FP8 训练" (hs-black.github.io): section 8.1 (S = F8max/amax,
//                saturation), 8.2 (delayed scaling fuses the amax into the producing pass).
//
// All kernels are HBM-bandwidth bound. The tensor is cut into runs of 256 * kVecs 16-byte input
// vectors (8 BF16 or 4 FP32 values each); a workgroup of 256 threads loads a run (kVecs vectors
// per thread, consecutive threads on consecutive vectors) before converting it. Small runs and
// many workgroups measured fastest on MI355X for this 2:1 read:write stream. Up to
// kMaxStreamGrid runs there is one workgroup per run; larger tensors give each workgroup several
// runs. The elements past the last whole vector (fewer than 8 or 4) are handled by workgroup 0.
//   amax_partials   -- read-only pass, one u32 |amax| bit pattern per workgroup: at most
//                      kAmaxGrid workgroups of 1024 threads, 8 loads per thread in flight (few
//                      partials keep the fold every cast workgroup repeats small).
//   cast_current    -- every workgroup folds all partials into amax and S itself (so there is
//                      no separate single-wave finalize launch), then casts its run.
//   cast_scaled     -- cast with a scale read from device memory.
//   cast_fused      -- a delayed-scaling step's pass: cast with the scale in the device state;
//                      each wave raises one of 256 workspace amax slots (128 B apart) with a
//                      device-scope atomic max that it does not wait for.
//   delayed_finalize -- one 256-thread workgroup: the step's amax from the slots (one load per
//                      thread; the slots are cleared for the next step), FIFO push on update
//                      steps, next scale into the state. (A single-launch variant that let the
//                      last workgroup finalize measured slower: device-scope atomics from every
//                      workgroup to one address serialize at the memory side.)
//   per_tensor_onepass -- current scaling for large tensors in one HBM read (described below).
#include <atomic>
#include <mutex>

#include "qf8_device.h"
#include "qf8_internal.h"
#include "../../include/qf8.h"

namespace qf8 {
namespace {

constexpr int kThreads = 256;
constexpr int kVecs = 2;                        // 16-byte input vectors per thread and run
constexpr int kAmaxThreads = 1024;              // read-only amax pass: one 16-wave workgroup per CU
constexpr int kAmaxDepth = 8;                   //   16-byte loads per thread in flight
constexpr int kFinalizeThreads = 256;           // single-workgroup finalize: one slot per thread
constexpr int kOpThreads = 512;                 // single-pass kernel, FP8 output: 8 waves, 2 per SIMD
constexpr int kOpRegSlabs = 48;                 //   slabs held in VGPRs (4 VGPRs each)
constexpr int kOpLdsSlabs = 16;                 //   slabs held in LDS (8 KiB each)
// NVFP4 output: its write phase is VALU-bound (two code estimates per element, and the exact
// recomputation of the elements where they differ), so it runs 16 waves (4 per SIMD, 128 VGPRs
// each) to hide the latencies of that phase, and holds 18 slabs in VGPRs (one more, without
// spills, gained nothing) and 9 in LDS (16 KiB each): 432 KiB per workgroup instead of 480. On
// 16384x4096 BF16 that re-reads 20 MiB but took 52.0-52.8 µs against 54.4-54.6 µs with 8 waves
// holding 42 + 18 slabs of 8 KiB.
constexpr int kOpThreadsNv = 1024;
constexpr int kOpRegSlabsNv = 18;
constexpr int kOpLdsSlabsNv = 9;
constexpr uint32_t kAbs16x2 = 0x7FFF7FFFu;

// |x| maximum of one 16-byte vector, accumulated as bit patterns (BF16 kept packed).
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
// maximum of two accumulators (BF16: per 16-bit half)
template <bool BF16>
__device__ __forceinline__ uint32_t acc_max(uint32_t a, uint32_t b) {
    if constexpr (BF16) return pk_max_u16(a, b);
    else return umax(a, b);
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
constexpr int vec_elems() { return BF16 ? 8 : 4; }

// One run of vectors, loaded in one go: vector j of thread t is run * 256 * kVecs + j * 256 + t.
// Raw-buffer accesses on a per-run descriptor: lanes past the end of the tensor read zeros (which
// never raise a maximum) and their stores are dropped, so there is no branch around any access.
template <bool BF16>
struct Run {
    static constexpr uint32_t kOutBytes = BF16 ? 8 : 4;   // codes per 16-byte input vector
    uint4 v[kVecs];
    int64_t first;                                         // first vector of the run
    uint32_t nv;                                           // vectors of the run inside the tensor

    __device__ __forceinline__ void load(const void *x, int64_t nvec, int64_t run) {
        first = run * kThreads * kVecs;
        const int64_t rem = nvec - first;
        nv = rem < kThreads * kVecs ? (uint32_t)rem : (uint32_t)(kThreads * kVecs);
        const __amdgpu_buffer_rsrc_t r = make_rsrc((const uint4 *)x + first, nv * 16u);
#pragma unroll
        for (int j = 0; j < kVecs; ++j)
            v[j] = buf_load16<kNonTemporal>(r, (uint32_t)(j * kThreads + threadIdx.x) * 16u, 0u);
    }
    __device__ __forceinline__ uint32_t absmax() const {
        uint32_t a0 = 0, a1 = 0;
#pragma unroll
        for (int j = 0; j < kVecs; ++j) {
            if (j & 1) a1 = vec_absmax<BF16>(a1, v[j]);
            else a0 = vec_absmax<BF16>(a0, v[j]);
        }
        return umax(acc_to_f32bits<BF16>(a0), acc_to_f32bits<BF16>(a1));
    }
    template <int FMT>
    __device__ __forceinline__ void cast_store(uint8_t *q, float s) const {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(q + first * kOutBytes, nv * kOutBytes);
#pragma unroll
        for (int j = 0; j < kVecs; ++j) {
            const uint32_t off = (uint32_t)(j * kThreads + threadIdx.x) * kOutBytes;
            if constexpr (BF16) {
                const uint2 o = cast8_bf16<FMT>(v[j], s);
                buf_store8<kNonTemporal>(r, off, 0u, o.x, o.y);
            } else {
                buf_store4<kNonTemporal>(r, off, 0u, cast4_f32<FMT>(v[j], s));
            }
        }
    }
};

inline __device__ int64_t run_count(int64_t nvec) { return (nvec + kThreads * kVecs - 1) / (kThreads * kVecs); }

// The elements after the last whole vector (workgroup 0 only).
template <bool BF16>
__device__ __forceinline__ uint32_t tail_absmax(const void *x, int64_t n, int64_t nvec) {
    uint32_t m = 0;
    if (blockIdx.x == 0)
        for (int64_t e = nvec * vec_elems<BF16>() + threadIdx.x; e < n; e += kThreads)
            m = umax(m, elem_bits<BF16>(x, e) & 0x7FFFFFFFu);
    return m;
}
template <bool BF16, int FMT>
__device__ __forceinline__ void tail_cast(const void *x, int64_t n, int64_t nvec, float s, uint8_t *q) {
    if (blockIdx.x == 0)
        for (int64_t e = nvec * vec_elems<BF16>() + threadIdx.x; e < n; e += kThreads)
            q[e] = (uint8_t)cast1<FMT>(__uint_as_float(elem_bits<BF16>(x, e)), s);
}

// |x| maximum (fp32 bits) of the elements of one 16-byte vector (first element e0) that lie in
// [lo, hi): the whole vector's maximum when it lies inside, else element by element.
template <bool BF16>
__device__ __forceinline__ uint32_t vec_absmax_in(uint4 v, int64_t e0, int64_t lo, int64_t hi) {
    constexpr int E = vec_elems<BF16>();
    if (e0 >= hi || e0 + E <= lo) return 0u;
    if (e0 >= lo && e0 + E <= hi) return acc_to_f32bits<BF16>(vec_absmax<BF16>(0u, v));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const uint32_t b = BF16 ? (w[i >> 1] >> ((i & 1) * 16)) << 16 : w[i];
        if (e0 + i >= lo && e0 + i < hi) m = umax(m, b & 0x7FFFFFFFu);
    }
    return m;
}

// Read-only pass over batches of kAmaxThreads * kAmaxDepth vectors (all loads of a batch in flight
// together; a read-only stream needs more bytes in flight per CU than the cast kernels, which also
// have stores queued). Batches are dealt round-robin: at any moment the workgroups read
// neighbouring batches. (Contiguous per-workgroup chunks measured 1.5x slower at power-of-two
// chunk sizes, where every workgroup hits the same HBM channels at once.)
template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void amax_partials_kernel(const void *__restrict__ x, int64_t n, int64_t nvec,
                                                                     uint32_t *__restrict__ partials) {
    constexpr int64_t kBatch = (int64_t)kAmaxThreads * kAmaxDepth;
    __shared__ uint32_t red[kAmaxThreads / 64];
    const uint4 *xv = (const uint4 *)x;
    uint32_t a0 = 0, a1 = 0;
    for (int64_t first = (int64_t)blockIdx.x * kBatch; first < nvec; first += (int64_t)gridDim.x * kBatch) {
        const int64_t rem = nvec - first;
        const uint32_t nb = (uint32_t)(rem < kBatch ? rem : kBatch) * 16u;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(xv + first, nb);
        uint4 v[kAmaxDepth];
#pragma unroll
        for (int k = 0; k < kAmaxDepth; ++k)
            v[k] = buf_load16<kNonTemporal>(r, (uint32_t)(k * kAmaxThreads + threadIdx.x) * 16u, 0u);
#pragma unroll
        for (int k = 0; k < kAmaxDepth; ++k) {
            if (k & 1) a1 = vec_absmax<BF16>(a1, v[k]);
            else a0 = vec_absmax<BF16>(a0, v[k]);
        }
    }
    uint32_t m = umax(acc_to_f32bits<BF16>(a0), acc_to_f32bits<BF16>(a1));
    if (blockIdx.x == 0)                                        // elements after the last whole vector
        for (int64_t e = nvec * vec_elems<BF16>() + threadIdx.x; e < n; e += kAmaxThreads)
            m = umax(m, elem_bits<BF16>(x, e) & 0x7FFFFFFFu);
    m = block_max_bcast<kAmaxThreads>(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(kThreads) void cast_current_kernel(const void *__restrict__ x, int64_t n, int64_t nvec,
                                                                uint8_t *__restrict__ q,
                                                                const uint32_t *__restrict__ partials, int nparts,
                                                                float *amax_out, float *scale_out, int32_t *nonfinite) {
    __shared__ uint32_t red[4];
    const int64_t nruns = run_count(nvec);
    Run<BF16> r;
    r.load(x, nvec, blockIdx.x);               // the first run's loads overlap the partials fold
    uint32_t m = block_max_bcast<kThreads>(fold_max<kThreads>(partials, nparts), red);
    const float s = scale_from_amax_bits<FMT>(m);
    r.template cast_store<FMT>(q, s);
    for (int64_t run = blockIdx.x + gridDim.x; run < nruns; run += gridDim.x) {
        r.load(x, nvec, run);
        r.template cast_store<FMT>(q, s);
    }
    tail_cast<BF16, FMT>(x, n, nvec, s, q);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (amax_out) *amax_out = __uint_as_float(m);
        if (scale_out) *scale_out = s;
        if (nonfinite && m >= 0x7F800000u) *nonfinite = 1;
    }
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(kThreads) void cast_scaled_kernel(const void *__restrict__ x, int64_t n, int64_t nvec,
                                                               const float *__restrict__ scale, uint8_t *__restrict__ q) {
    const float s = *scale;
    for (int64_t run = blockIdx.x; run < run_count(nvec); run += gridDim.x) {
        Run<BF16> r;
        r.load(x, nvec, run);
        r.template cast_store<FMT>(q, s);
    }
    tail_cast<BF16, FMT>(x, n, nvec, s, q);
}

// Delayed-scaling state update, by one workgroup. m is the step's whole-tensor |amax| (reported,
// and the flag for Inf/NaN). The value appended on update steps is m itself, or with split set
// the maximum of the window: meta[2] holds the running maximum of the pieces measured since the
// last update step (mp = this step's piece), and a window that saw Inf/NaN appends nothing.
// The oldest entry is dropped when the FIFO is full. On update steps the next scale is derived
// from the history with the state's estimator (0 maximum, 1 newest entry, 2 mean as the fp32 sum
// from oldest to newest divided by the count); between them neither changes. The FIFO is
// slots [0, count) while filling (head 0), then a ring whose oldest entry is at head.
template <int FMT>
__device__ void delayed_update(uint32_t m, uint32_t mp, int split, float *history, int32_t *meta, float *scale,
                               int hist_len, int n_guard, int update, int estimator, float *amax_out,
                               int32_t *nonfinite, uint32_t *red, int *sh) {
    if (threadIdx.x == 0) {
        if (amax_out) *amax_out = __uint_as_float(m);
        if (m >= 0x7F800000u && nonfinite) *nonfinite = 1;
        uint32_t v = m;                                              // the value to append
        if (split) {
            const uint32_t w = umax((uint32_t)meta[2], mp);
            meta[2] = update ? 0 : (int32_t)w;                       // a window ends on update steps
            v = w;
        }
        int count = meta[0], head = meta[1], slot = -1;
        if (update && v < 0x7F800000u) {
            if (count < hist_len) {                                  // head stays 0 while filling
                slot = count;
                meta[0] = ++count;
            } else {
                slot = head;
                head = head + 1 == hist_len ? 0 : head + 1;
                meta[1] = head;
            }
            history[slot] = __uint_as_float(v);
        }
        sh[0] = count;
        sh[1] = slot;
        sh[2] = head;
        sh[3] = (int)v;
    }
    __syncthreads();
    if (!update) return;
    // The slot written above is taken from shared memory, not re-read from global memory.
    const int count = sh[0], slot = sh[1], head = sh[2];
    const uint32_t v = (uint32_t)sh[3];
    uint32_t e = 0;
    if (estimator == 0) {                      // maximum: slots [0, count) in any order
        for (int i = threadIdx.x; i < count; i += kFinalizeThreads)
            if (i != slot) e = umax(e, __float_as_uint(history[i]));
        if (threadIdx.x == 0 && slot >= 0) e = umax(e, v);
        e = block_max_bcast<kFinalizeThreads>(e, red);
    } else if (threadIdx.x == 0 && count > 0) {
        if (estimator == 1) {                  // the newest entry
            const int idx = (head + count - 1) % hist_len;
            e = idx == slot ? v : __float_as_uint(history[idx]);
        } else {                               // mean, summed oldest to newest in fp32
            float sum = 0.0f;
            for (int i = 0; i < count; ++i) {
                const int idx = (head + i) % hist_len;
                sum = sum + (idx == slot ? __uint_as_float(v) : history[idx]);
            }
            e = __float_as_uint(sum / (float)count);
        }
    }
    if (threadIdx.x == 0) {
        const float margin = __uint_as_float((uint32_t)(127 - n_guard) << 23);   // 2^-N, exact
        *scale = scale_from_amax_bits<FMT>(e) * margin;
    }
}

// Cast with the state's scale and raise the running |amax| maximum of one workspace slot per
// wave (device-scope atomic max, not waited for; waves spread over kSlotCount slots, each on
// its own 128-byte line, so no single address takes more than a few hundred updates).
// SPLIT: the wave also raises word 1 of its slot line with the maximum over the elements
// [lo, hi) only (the piece of the tensor a split-amax delayed step measures).
template <bool BF16, int FMT, bool SPLIT>
__global__ __launch_bounds__(kThreads) void cast_fused_kernel(const void *__restrict__ x, int64_t n, int64_t nvec,
                                                              const float *__restrict__ scale, uint8_t *__restrict__ q,
                                                              float *scale_used, uint32_t *slots, int64_t lo,
                                                              int64_t hi) {
    constexpr int E = vec_elems<BF16>();
    const float s = *scale;
    uint32_t m = tail_absmax<BF16>(x, n, nvec), mp = 0;
    if (SPLIT && blockIdx.x == 0)
        for (int64_t e = nvec * E + threadIdx.x; e < n; e += kThreads)
            if (e >= lo && e < hi) mp = umax(mp, elem_bits<BF16>(x, e) & 0x7FFFFFFFu);
    for (int64_t run = blockIdx.x; run < run_count(nvec); run += gridDim.x) {
        Run<BF16> r;
        r.load(x, nvec, run);
        r.template cast_store<FMT>(q, s);
        m = umax(m, r.absmax());
        if constexpr (SPLIT) {
            // vectors past the end of the tensor were loaded as zeros and add nothing
#pragma unroll
            for (int j = 0; j < kVecs; ++j)
                mp = umax(mp, vec_absmax_in<BF16>(r.v[j], (r.first + j * kThreads + threadIdx.x) * E, lo, hi));
        }
    }
    tail_cast<BF16, FMT>(x, n, nvec, s, q);
    m = max_wave(m);
    if constexpr (SPLIT) mp = max_wave(mp);
    if ((threadIdx.x & 63) == 0) {
        const uint32_t slot = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) % kSlotCount;
        __hip_atomic_fetch_max(slots + (size_t)slot * kBarLineWords, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (SPLIT && mp != 0u)
            __hip_atomic_fetch_max(slots + (size_t)slot * kBarLineWords + 1, mp, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && scale_used) *scale_used = s;
}

// ---------------------------------------------------------------------------------------------
// Single-HBM-pass current scaling. One workgroup of op_threads<OP>() threads per CU (grid = CU
// count, at most kBarMaxGroups). The tensor is cut into slabs of one 16-byte vector per thread;
// workgroup b owns slabs b, b + G, b + 2G, ... (neighbouring workgroups read neighbouring slabs,
// so every HBM channel is busy at once). Its first KR slabs stay in VGPRs and the next KL in LDS
// (loaded by direct-to-LDS DMA, no VGPR staging), so that a tensor up to
//   G * threads * (KR + KL) * 16 bytes   (FP8 output: 128 MiB on 256 CUs; NVFP4: 108 MiB)
// is read from HBM exactly once; slabs beyond that are reduced in the first pass and re-read
// for the cast.
//
// Grid barrier. A barrier word is 64 bits: running amax low, arrival count high. Arrival is in
// two levels, because device-scope atomics on one address are performed one after another at
// the memory side (256 workgroups x 2 atomics on a single word took ~8 µs on MI355X, groups of
// 16 bring it to ~2.5 µs):
//   every workgroup arrives at its group's word (groups of kBarGroup consecutive workgroups;
//     the word is words 16-17 of the release line of the group's first workgroup): a 32-bit
//     fetch_max on the low half, waiting for the returned value so the maximum is performed
//     before the arrival, then a 64-bit fetch_add of 2^32, whose returned value carries both the
//     count and the maximum of every earlier arrival.
//   the group's last arriver zeroes the group word and arrives the same way at the header word
//     (workspace words 0-1) with the group maximum, adding the group's size: the header counts
//     the workgroups of complete groups. The one that completes the header word
//     holds the final maximum: it zeroes that word and releases each other workgroup by
//     exchanging RELEASED | amax into words 0-1 of that workgroup's own 128-byte line (one line
//     per poller: no same-address polling).
//   every other workgroup polls its own line. If it is not released within the timeout it may
//     give up: mark the line GAVE_UP (compare-exchange from 0) and exit without casting, which
//     frees its CU for a workgroup that is not resident yet (another kernel may hold CUs). So
//     the kernel never depends on all workgroups being resident at once: it only gets slower.
//     A timed-out waiter gives up only while the workgroups of its shader engine that gave up
//     are fewer than a 32nd of those that have not arrived (at most G minus the header count),
//     so that about as many leave as are missing, on every shader engine, and the rest stay to
//     share the given-up slabs; otherwise it waits another timeout. After kGiveUpTimeouts time-outs it gives up anyway,
//     so that every resident workgroup leaves in the end whatever holds the CUs.
// Given-up slabs. The releaser learns from its exchanges which workgroups gave up. After casting
// kPublishAt of its held slabs it clears their lines, writes their numbers to a list (word 4 of
// lines 0, 1, ...) and ORs INFO | (count << 48) into the line of every released workgroup. Each
// released workgroup reads its line half-way through its held slabs and, when they are done,
// polls again if INFO was not there yet (the releaser is running, so the wait ends), clears the
// line, and if the count is not zero joins the releaser in casting the
// given-up slabs: units of 8 slabs (one stream_slabs8 call) are claimed from a counter (header
// word 3), and the last workgroup to finish (counted in header word 4) clears the list and the
// counters. So the workspace is back to all-zero when the kernel ends, and the slabs of a
// workgroup that gave up are spread over all the others.

constexpr int kBarGroup = 16;                       // workgroups per first-level barrier word
constexpr int kBarGroupWord = 16;                   // its u32 offset in the group's first line
constexpr uint64_t kLineReleased = 1ull << 32;
constexpr uint64_t kLineGaveUp = 2ull << 32;
constexpr uint64_t kLineInfo = 4ull << 32;          // + the number of given-up workgroups << 48
constexpr int kLineListWord = 4;                    // u32 offset of a list entry in its line
// The releaser sends INFO after this many register slabs (FP8 output; NVFP4, whose slabs are twice
// as large and slower to cast, after a third of them): by then its exchanges have returned (at 8
// it still waited for them, and being the last workgroup to start its casts, that cost the whole
// call ~0.3 us at 8192x8192).
constexpr int kPublishAtFp8 = 12;
constexpr int kClaimWord = 3, kDoneWord = 4;        // header words of the recast counters
// Workgroups that gave up, counted per shader engine (8 XCDs x 4 SEs; the count of bucket i is
// word kLineBucketWord of line i): a workgroup that is not resident waits for a CU of the XCD and
// shader engine the dispatcher picked for it, so every shader engine gives up its share of the
// missing workgroups, not only the first waiters to time out.
constexpr int kGiveUpBuckets = 32;
constexpr int kLineBucketWord = 5;                  // u32 offset of a bucket count in its line
constexpr int kGiveUpTimeouts = 8;                  // a waiter gives up at the latest after this many
// Default timeout of a waiter, in ticks of the 100 MHz real-time counter: 50 us, plus one tick
// per 500 KB of input (a tenth of the time the first pass takes to stream it at 5 TB/s), since
// the arrivals of a large streamed tensor spread wider (10-20 us at 1 GiB).
constexpr uint32_t kDefaultGiveUpTicks = 5000;
constexpr int64_t kGiveUpBytesPerTick = 500000, kGiveUpMaxExtra = 100000;   // the size term: 1 ms at most

template <bool BF16, int FMT>
__device__ __forceinline__ void cast_vec_store(__amdgpu_buffer_rsrc_t w, uint32_t off, uint4 v, float s) {
    if constexpr (BF16) {
        const uint2 o = cast8_bf16<FMT>(v, s);
        buf_store8<kNonTemporal>(w, off, 0u, o.x, o.y);
    } else {
        buf_store4<kNonTemporal>(w, off, 0u, cast4_f32<FMT>(v, s));
    }
}

// Per-tensor FP8 codes of two whole slabs, stored by lane pairs as 16-byte pieces (8 for FP32
// input): the even lane of a pair writes its vector's codes and its partner's from slab k, the odd
// lane both from slab k + 1, after one DPP swap of the codes each sends. v0 is the lane's vector
// index in slab k; every lane of the wave must be active.
template <bool BF16, int FMT>
__device__ __forceinline__ void cast_pair_store(__amdgpu_buffer_rsrc_t w, uint32_t v0, uint32_t vstep, uint4 a, uint4 b,
                                                float s) {
    const bool odd = (threadIdx.x & 1u) != 0u;
    const uint32_t v = odd ? v0 - 1u + vstep : v0;      // the pair's first vector in its slab
    if constexpr (BF16) {
        const uint2 A = cast8_bf16<FMT>(a, s), B = cast8_bf16<FMT>(b, s);
        const uint32_t rx = dpp_mov<0xB1>(odd ? A.x : B.x), ry = dpp_mov<0xB1>(odd ? A.y : B.y);
        const uint4 o = odd ? make_uint4(rx, ry, B.x, B.y) : make_uint4(A.x, A.y, rx, ry);
        buf_store16<kNonTemporal>(w, v * 8u, 0u, o);
    } else {
        const uint32_t A = cast4_f32<FMT>(a, s), B = cast4_f32<FMT>(b, s);
        const uint32_t r = dpp_mov<0xB1>(odd ? A : B);
        buf_store8<kNonTemporal>(w, v * 4u, 0u, odd ? r : A, odd ? B : r);
    }
}

// The single-pass kernel's outputs. kOpFp8: per-tensor FP8 cast (8 or 4 code bytes per 16-byte
// input vector). kOpNvfp4: NVFP4 with the tensor scale S_t: a 16-element block is 2 (BF16) or 4
// (FP32) vectors held by adjacent lanes, whose amax meets by DPP; each lane writes its 4 or 2
// code bytes and the block's first lane the E4M3 scale byte. All lanes must be active.
constexpr int kOpFp8 = 0, kOpNvfp4 = 1;
template <int OP> constexpr int op_threads() { return OP == kOpFp8 ? kOpThreads : kOpThreadsNv; }
template <int OP, bool BF16>
constexpr uint32_t op_out_bytes() { return OP == kOpFp8 ? (BF16 ? 8u : 4u) : (BF16 ? 4u : 2u); }

// NVFP4 codes of one input vector. Two estimates of every quotient x * S_t / decode(e_b), one
// below and one above the exact value (nv_factor_table), give codes lo and hi; where a nibble
// differs the quotient lies next to an E2M1 midpoint, and that element alone is recomputed
// exactly (nv_elem_exact) from the vector still in registers. The loop over the differing nibbles
// runs in the lanes that have any (about 1% of the vectors of a BF16 gradient).
template <bool BF16>
__device__ __forceinline__ uint32_t nv_vec_codes(uint4 v, float2 r, uint32_t e, float st) {
    // every byte of l and h is written by its four converts, so they start from input words that
    // are dead by then instead of zeros
    uint32_t l = v.x, h = v.y;
    if constexpr (BF16) {
        l = cvt_fp4_f32<0>(l, bf16_lo(v.x) * r.x, bf16_hi(v.x) * r.x, 1.0f);
        l = cvt_fp4_f32<1>(l, bf16_lo(v.y) * r.x, bf16_hi(v.y) * r.x, 1.0f);
        l = cvt_fp4_f32<2>(l, bf16_lo(v.z) * r.x, bf16_hi(v.z) * r.x, 1.0f);
        l = cvt_fp4_f32<3>(l, bf16_lo(v.w) * r.x, bf16_hi(v.w) * r.x, 1.0f);
        h = cvt_fp4_f32<0>(h, bf16_lo(v.x) * r.y, bf16_hi(v.x) * r.y, 1.0f);
        h = cvt_fp4_f32<1>(h, bf16_lo(v.y) * r.y, bf16_hi(v.y) * r.y, 1.0f);
        h = cvt_fp4_f32<2>(h, bf16_lo(v.z) * r.y, bf16_hi(v.z) * r.y, 1.0f);
        h = cvt_fp4_f32<3>(h, bf16_lo(v.w) * r.y, bf16_hi(v.w) * r.y, 1.0f);
    } else {
        l = cvt_fp4_f32<0>(l, __uint_as_float(v.x) * r.x, __uint_as_float(v.y) * r.x, 1.0f);
        l = cvt_fp4_f32<1>(l, __uint_as_float(v.z) * r.x, __uint_as_float(v.w) * r.x, 1.0f);
        h = cvt_fp4_f32<0>(h, __uint_as_float(v.x) * r.y, __uint_as_float(v.y) * r.y, 1.0f);
        h = cvt_fp4_f32<1>(h, __uint_as_float(v.z) * r.y, __uint_as_float(v.w) * r.y, 1.0f);
        l &= 0xFFFFu;                           // the FP32 vector's 4 codes fill two bytes
        h &= 0xFFFFu;
    }
    uint32_t d = l ^ h;
    if (d != 0u) {
        const float dec = __builtin_amdgcn_cvt_f32_fp8(e, 0);
        do {
            const uint32_t sh = (uint32_t)__builtin_ctz(d) & ~3u;     // nibble of the lowest set bit
            d &= ~(0xFu << sh);
            // element sh / 4 of the vector: BF16 nibble 2k + j is half j of word k, FP32 nibble k word k
            const uint32_t k = BF16 ? sh >> 3 : sh >> 2;
            const uint32_t w = k == 0u ? v.x : k == 1u ? v.y : k == 2u ? v.z : v.w;
            const float xe = BF16 ? __uint_as_float((sh & 4u) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
            l = (l & ~(0xFu << sh)) | (nv_elem_exact(xe, st, dec) << sh);
        } while (d != 0u);
    }
    return l;
}

// A block of 16 is 2 (BF16) or 4 (FP32) vectors held by adjacent lanes, whose amax meets by DPP;
// each lane writes its 4 or 2 code bytes and the block's first lane the E4M3 scale byte. All lanes
// must be active.
template <bool BF16>
__device__ __forceinline__ void nv_vec_store(__amdgpu_buffer_rsrc_t wq, __amdgpu_buffer_rsrc_t wsb, uint32_t vrel,
                                             uint4 v, float st, const float2 *tab) {
    uint32_t a = acc_to_f32bits<BF16>(vec_absmax<BF16>(0u, v));
    if constexpr (BF16) a = umax(a, dpp_mov<0xB1>(a));         // lanes 2j, 2j+1 hold one block
    else a = max_quad(a);                                       // lanes 4j .. 4j+3
    const uint32_t e = nv_block_code(a, st);
    const uint32_t o = nv_vec_codes<BF16>(v, tab[e], e, st);
    if constexpr (BF16) {
        buf_store4<kNonTemporal>(wq, vrel * 4u, 0u, o);
        if ((vrel & 1u) == 0u) buf_store1(wsb, vrel >> 1, 0u, e);
    } else {
        buf_store2(wq, vrel * 2u, 0u, o);
        if ((vrel & 3u) == 0u) buf_store1(wsb, vrel >> 2, 0u, e);
    }
}

template <int OP, bool BF16, int FMT>
__device__ __forceinline__ void op_vec_store(__amdgpu_buffer_rsrc_t wq, __amdgpu_buffer_rsrc_t wsb, uint32_t vrel,
                                             uint4 v, float s, const float2 *tab) {
    if constexpr (OP == kOpFp8) cast_vec_store<BF16, FMT>(wq, vrel * op_out_bytes<OP, BF16>(), v, s);
    else nv_vec_store<BF16>(wq, wsb, vrel, v, s, tab);
}

// Byte count of the vectors [first, nvec) clamped to one buffer descriptor's range.
__device__ __forceinline__ uint32_t span_bytes(int64_t first, int64_t nvec, uint32_t bytes_per_vec) {
    const int64_t rem = nvec - first;
    if (rem <= 0) return 0u;
    const int64_t b = rem * bytes_per_vec;
    return b < 0xFFFFFFFFll ? (uint32_t)b : 0xFFFFFFFFu;
}

// The eight slabs k, k + 1, ..., k + 7 of workgroup j (slab k of workgroup j is k * G + j):
// load, and cast + store when CAST, return the |x| maximum (accumulator form).
template <int OP, bool BF16, int FMT, bool CAST>
__device__ __forceinline__ uint32_t stream_slabs8(const uint4 *x, int64_t nvec, uint8_t *q, uint8_t *sb, int64_t k,
                                                  int j, int G, float s, const float2 *tab) {
    constexpr int NT = op_threads<OP>();
    constexpr uint32_t kOut = op_out_bytes<OP, BF16>();
    constexpr uint32_t kVpb = BF16 ? 2u : 4u;                      // vectors per NVFP4 block
    const uint32_t step = (uint32_t)G * NT * 16u;
    const int64_t first = (k * G + j) * NT;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(x + first, span_bytes(first, nvec, 16u));
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = buf_load16<kNonTemporal>(r, i * step + threadIdx.x * 16u, 0u);
    uint32_t a = 0;
    if constexpr (CAST) {
        const __amdgpu_buffer_rsrc_t w = make_rsrc(q + first * kOut, span_bytes(first, nvec, kOut));
        const __amdgpu_buffer_rsrc_t wsb = make_rsrc(OP == kOpNvfp4 ? sb + first / kVpb : q,
                                                     OP == kOpNvfp4 ? span_bytes(first, nvec, 1u) / kVpb : 0u);
#pragma unroll
        for (int i = 0; i < 8; ++i) op_vec_store<OP, BF16, FMT>(w, wsb, i * (step / 16u) + threadIdx.x, v[i], s, tab);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a = vec_absmax<BF16>(a, v[i]);
    }
    return a;
}

// One arrival at a barrier word [amax | count << 32] shared by `expected` arrivals: raise the
// maximum (waiting for the atomic to be performed, so it is in the word before this arrival is
// counted), then count. The last arrival gets true and the maximum over all arrivals in *total,
// and zeroes the word for the next call.
__device__ __forceinline__ bool arrive(uint64_t *word, uint32_t m, uint32_t inc, uint32_t expected, uint32_t &total) {
    const uint32_t prev = __hip_atomic_fetch_max((uint32_t *)word, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::"v"(prev) : "memory");
    const uint64_t old = __hip_atomic_fetch_add(word, (uint64_t)inc << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old >> 32) + inc != expected) return false;
    total = umax((uint32_t)old, m);
    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

template <bool BF16, int FMT, int OP>
__global__ __launch_bounds__(op_threads<OP>()) void per_tensor_onepass_kernel(
        const void *__restrict__ x, int64_t n, int64_t nvec, uint8_t *__restrict__ q, uint8_t *__restrict__ sb,
        uint32_t *ws, float *amax_out, float *scale_out, int32_t *nonfinite, uint32_t *amax_bits_out) {
    constexpr int NT = op_threads<OP>();
    constexpr int KR = OP == kOpFp8 ? kOpRegSlabs : kOpRegSlabsNv;
    constexpr int KL = OP == kOpFp8 ? kOpLdsSlabs : kOpLdsSlabsNv;
    constexpr uint32_t kOut = op_out_bytes<OP, BF16>();
    constexpr uint32_t kVpb = BF16 ? 2u : 4u;
    __shared__ uint4 held[KL * NT];
    __shared__ uint32_t red[NT / 64];
    __shared__ uint32_t sh[4];
    __shared__ uint16_t gave_up[kBarMaxGroups];
    __shared__ float2 nvtab[OP == kOpNvfp4 ? 128 : 1];            // NVFP4: (r_lo, r_hi) per E4M3 code
    const uint4 *xv = (const uint4 *)x;
    const int G = gridDim.x, b = blockIdx.x, t = threadIdx.x;
    const int64_t nslabs = (nvec + NT - 1) / NT;
    // held slabs: offsets below (KR + KL) * G * NT * 16 < 2^32 (G <= kBarMaxGroups)
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xv, span_bytes(0, nvec, 16u));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, span_bytes(0, nvec, kOut));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(OP == kOpNvfp4 ? sb : q, OP == kOpNvfp4 ? span_bytes(0, nvec, 1u) / kVpb : 0u);
    const uint32_t step = (uint32_t)G * NT * 16u;        // bytes between a workgroup's slabs
    const uint32_t base = ((uint32_t)b * NT + t) * 16u;

    // pass 1: slabs that are not held (maximum only), then the LDS-held slabs (DMA), then the
    // register-held slabs, all loads in flight together
    uint32_t a0 = 0;
    for (int64_t k = KR + KL; k * G + b < nslabs; k += 8)
        a0 = acc_max<BF16>(a0, stream_slabs8<OP, BF16, FMT, false>(xv, nvec, q, sb, k, b, G, 0.f, nvtab));
    a0 = acc_to_f32bits<BF16>(a0);
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
#pragma unroll
    for (int k = 0; k < KL; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)&held[k * NT + wave * 64],
                                                 16, base + (KR + k) * step, 0, 0, kNonTemporal);
    uint4 R[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) R[k] = buf_load16<kNonTemporal>(rx, base + k * step, 0u);
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        if (k & 1) c1 = vec_absmax<BF16>(c1, R[k]);
        else c0 = vec_absmax<BF16>(c0, R[k]);
    }
#pragma unroll
    for (int k = 0; k < KL; ++k) c1 = vec_absmax<BF16>(c1, held[k * NT + t]);
    uint32_t m = umax(a0, umax(acc_to_f32bits<BF16>(c0), acc_to_f32bits<BF16>(c1)));
    if (b == 0)                                                    // elements after the last vector
        for (int64_t e = nvec * vec_elems<BF16>() + t; e < n; e += NT) m = umax(m, elem_bits<BF16>(x, e) & 0x7FFFFFFFu);
    m = block_max_bcast<NT>(m, red);

    // grid barrier
    uint64_t *lines = (uint64_t *)(ws + kBarHeaderWords);
    uint64_t *own = lines + (size_t)b * (kBarLineWords / 2);
    if (t == 0) {
        // arrival in two levels: the group's word, then (the group's last arriver) the header word
        const int grp = b / kBarGroup;
        const uint32_t gsize = (uint32_t)min(kBarGroup, G - grp * kBarGroup);
        uint32_t role = 0, am = 0;
        uint32_t gm = 0;
        if (arrive(lines + (size_t)grp * kBarGroup * (kBarLineWords / 2) + kBarGroupWord / 2, m, 1u, gsize, gm) &&
            arrive((uint64_t *)ws, gm, gsize, (uint32_t)G, am))
            role = 1;
        if (role == 0) {
            const int64_t extra = nvec * 16 / kGiveUpBytesPerTick;
            const uint32_t limit = ws[2] ? ws[2] : kDefaultGiveUpTicks + (uint32_t)(extra < kGiveUpMaxExtra ? extra : kGiveUpMaxExtra);
            // XCC_ID[3:0] and HW_ID.SE_ID[14:13] of this wave
            const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
            const uint32_t se = __builtin_amdgcn_s_getreg(4 | (13 << 6) | (1 << 11));
            uint32_t *gcount = (uint32_t *)(lines + (size_t)((xcc * 4u + se) % kGiveUpBuckets) * (kBarLineWords / 2)) +
                               kLineBucketWord;
            uint64_t start = __builtin_amdgcn_s_memrealtime();
            uint64_t v;
            for (int timeouts = 1;; ) {
                v = __hip_atomic_load(own, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v != 0) break;
                if (__builtin_amdgcn_s_memrealtime() - start > limit) {
                    // give up while this bucket's share of the workgroups that have not arrived
                    // (the header counts those of complete groups) is not yet used, or after
                    // kGiveUpTimeouts time-outs
                    const uint32_t h = (uint32_t)(__hip_atomic_load((uint64_t *)ws, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
                    const uint32_t g = __hip_atomic_fetch_add(gcount, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (g < ((uint32_t)G - h + kGiveUpBuckets - 1) / kGiveUpBuckets || timeouts >= kGiveUpTimeouts) {
                        uint64_t expected = 0;
                        if (__hip_atomic_compare_exchange_strong(own, &expected, kLineGaveUp, __ATOMIC_RELAXED,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                            v = kLineGaveUp;        // stays counted in the give-up word
                            break;
                        }
                        v = expected;               // released meanwhile
                    }
                    // not given up: the count goes back down before this workgroup goes on
                    const uint32_t back = __hip_atomic_fetch_sub(gcount, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    asm volatile("" ::"v"(back));
                    if (v != 0) break;
                    ++timeouts;
                    start = __builtin_amdgcn_s_memrealtime();
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (v == kLineGaveUp) role = 2;
            else am = (uint32_t)v;                  // the line is cleared once INFO has come
        }
        sh[0] = role;
        sh[1] = am;
        sh[2] = 0;
    }
    __syncthreads();
    const uint32_t role = sh[0];
    if (role == 2) return;                          // the released workgroups cast this one's slabs
    m = sh[1];
    uint64_t xres = kLineReleased;                  // (what no exchange returns: the line was 0 or GAVE_UP)
    if (role == 1 && t < G && t != b)               // release: one line per thread (G <= NT)
        xres = __hip_atomic_exchange(lines + (size_t)t * (kBarLineWords / 2), kLineReleased | m, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    const float s = OP == kOpFp8 ? scale_from_amax_bits<FMT>(m) : nv_tensor_scale(m);
    if constexpr (OP == kOpNvfp4) {
        nv_factor_table(nvtab, s);
        __syncthreads();
    }

    // pass 2: cast the held slabs, then re-read and cast the rest (vector indices: vbase + k * vstep)
    const uint32_t vbase = (uint32_t)b * NT + t, vstep = step / 16u;
    // Given-up slabs (see the barrier description above): the releaser publishes after its first
    // kPublishAt register slabs, when its exchanges have returned; the others read INFO after
    // slab kInfoReadAt, well after that, and use it only at the end, so that neither waits.
    uint32_t ng = 0, info = 0;                      // info: the high half of the own line
    constexpr int kPublishAt = OP == kOpFp8 ? kPublishAtFp8 : KR / 3;
    constexpr int kInfoReadAt = OP == kOpFp8 ? KR / 2 : KR - 4;
    static_assert(kPublishAt + 8 <= kInfoReadAt && kInfoReadAt < KR, "INFO is read well after it is sent");
    // FP8 output: slabs k, k + 1 that are both whole leave through lane pairs as 16-byte pieces
    const auto pair_whole = [&](int k) { return ((int64_t)(k + 1) * G + b + 1) * NT <= nvec; };
    static_assert(OP != kOpFp8 || (KR % 2 == 0 && KL % 2 == 0), "FP8 held slabs go in pairs");
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        if constexpr (OP == kOpFp8) {
            if ((k & 1) == 0) {
                if (pair_whole(k)) {
                    cast_pair_store<BF16, FMT>(rq, vbase + k * vstep, vstep, R[k], R[k + 1], s);
                } else {
                    op_vec_store<OP, BF16, FMT>(rq, rsb, vbase + k * vstep, R[k], s, nvtab);
                    op_vec_store<OP, BF16, FMT>(rq, rsb, vbase + (k + 1) * vstep, R[k + 1], s, nvtab);
                }
            }
        } else {
            op_vec_store<OP, BF16, FMT>(rq, rsb, vbase + k * vstep, R[k], s, nvtab);
        }
        if (k == kPublishAt && role == 1) {
            const bool tell = xres == 0u;           // released by this thread's exchange: gets INFO
            if (xres == kLineGaveUp) {
                __hip_atomic_store(lines + (size_t)t * (kBarLineWords / 2), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                gave_up[atomicAdd(&sh[2], 1u)] = (uint16_t)t;
            }
            __syncthreads();
            ng = sh[2];
            if (ng != 0u) {                         // rare
                if ((uint32_t)t < ng) {
                    // an exchange whose result is waited for is performed before the barrier
                    // below, so the entry is in place before any INFO that announces it
                    const uint32_t old = __hip_atomic_exchange((uint32_t *)(lines + (size_t)t * (kBarLineWords / 2)) + kLineListWord,
                                                               (uint32_t)gave_up[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    asm volatile("" ::"v"(old));
                }
                __syncthreads();
            }
            if (tell)
                __hip_atomic_fetch_or(lines + (size_t)t * (kBarLineWords / 2), kLineInfo | (uint64_t)ng << 48,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (k == kInfoReadAt && role == 0 && t == 0)   // (32 bits: no dead half to wait for)
            info = __hip_atomic_load((uint32_t *)own + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int k = 0; k < KL; ++k) {
        if constexpr (OP == kOpFp8) {
            if ((k & 1) == 0) {
                if (pair_whole(KR + k)) {
                    cast_pair_store<BF16, FMT>(rq, vbase + (KR + k) * vstep, vstep, held[k * NT + t], held[(k + 1) * NT + t], s);
                } else {
                    op_vec_store<OP, BF16, FMT>(rq, rsb, vbase + (KR + k) * vstep, held[k * NT + t], s, nvtab);
                    op_vec_store<OP, BF16, FMT>(rq, rsb, vbase + (KR + k + 1) * vstep, held[(k + 1) * NT + t], s, nvtab);
                }
            }
        } else {
            op_vec_store<OP, BF16, FMT>(rq, rsb, vbase + (KR + k) * vstep, held[k * NT + t], s, nvtab);
        }
    }
    for (int64_t k = KR + KL; k * G + b < nslabs; k += 8)
        stream_slabs8<OP, BF16, FMT, true>(xv, nvec, q, sb, k, b, G, s, nvtab);

    if (role == 0) {                                // the releaser's INFO: how many gave up
        if (t == 0) {
            uint32_t v = info;
            while ((v & (uint32_t)(kLineInfo >> 32)) == 0u) {   // rare: not there yet when read above
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load((uint32_t *)own + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __hip_atomic_store(own, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sh[2] = v >> 16;                        // bits 48.. of the line word
        }
        __syncthreads();
        ng = sh[2];
    }
    if (ng != 0u) {                                 // rare: cast the given-up slabs together
        const int64_t most = (nslabs + G - 1) / G;                  // slabs of a workgroup at most
        const uint32_t upw = (uint32_t)((most + 7) / 8), units = ng * upw;
        for (;;) {
            __syncthreads();                        // the previous unit's sh[3] has been read
            if (t == 0) {
                const uint32_t u = __hip_atomic_fetch_add(ws + kClaimWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sh[3] = u;
                if (u < units)
                    sh[0] = __hip_atomic_load((uint32_t *)(lines + (size_t)(u / upw) * (kBarLineWords / 2)) + kLineListWord,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            const uint32_t u = sh[3];
            if (u >= units) break;
            const int j = (int)sh[0];
            const int64_t k = (int64_t)(u % upw) * 8;
            if (k * G + j < nslabs) stream_slabs8<OP, BF16, FMT, true>(xv, nvec, q, sb, k, j, G, s, nvtab);
        }
        if (t == 0 && __hip_atomic_fetch_add(ws + kDoneWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                          (uint32_t)G - ng - 1u) {  // the last one out: list and counters back to zero
            for (uint32_t i = 0; i < ng; ++i)
                __hip_atomic_store((uint32_t *)(lines + (size_t)i * (kBarLineWords / 2)) + kLineListWord, 0u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ws + kClaimWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ws + kDoneWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int i = 0; i < kGiveUpBuckets; ++i)
                __hip_atomic_store((uint32_t *)(lines + (size_t)i * (kBarLineWords / 2)) + kLineBucketWord, 0u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (role == 1) {
        if constexpr (OP == kOpFp8)          // NVFP4 sizes are whole vectors (n % 16 == 0)
            for (int64_t e = nvec * vec_elems<BF16>() + t; e < n; e += NT)
                q[e] = (uint8_t)cast1<FMT>(__uint_as_float(elem_bits<BF16>(x, e)), s);
        if (t == 0) {
            if (amax_out) *amax_out = __uint_as_float(m);
            if (scale_out) *scale_out = s;
            if (amax_bits_out) *amax_bits_out = m;
            if (nonfinite && m >= 0x7F800000u) *nonfinite = 1;
        }
    }
}

// The step's amax = maximum of the workspace slots (cleared again for the next step) and of
// nparts per-workgroup partials (the two-kernel current-scaling path of step 0), then the state
// update.
template <int FMT>
__global__ __launch_bounds__(kFinalizeThreads) void delayed_finalize_kernel(uint32_t *slots, const uint32_t *__restrict__ partials,
                                                                            int nparts, float *history, int32_t *meta,
                                                                            float *scale, int hist_len, int n_guard,
                                                                            int update, int estimator, int split,
                                                                            float *amax_out, int32_t *nonfinite) {
    static_assert(kFinalizeThreads == kSlotCount, "one slot per thread");
    __shared__ uint32_t red[kFinalizeThreads / 64];
    __shared__ int sh[4];
    uint32_t *own = slots + (size_t)threadIdx.x * kBarLineWords;
    uint32_t m = umax(own[0], fold_max<kFinalizeThreads>(partials, nparts)), mp = 0u;
    own[0] = 0u;
    if (split) {
        mp = own[1];
        own[1] = 0u;
    }
    m = block_max_bcast<kFinalizeThreads>(m, red);
    if (split) mp = block_max_bcast<kFinalizeThreads>(mp, red);
    delayed_update<FMT>(m, mp, split, history, meta, scale, hist_len, n_guard, update, estimator, amax_out, nonfinite,
                        red, sh);
}

__global__ void fill_u32_kernel(uint32_t *p, int64_t n, uint32_t value) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

inline int64_t vec_count(int64_t n, int dtype) { return n / (dtype == QF8_IN_BF16 ? 8 : 4); }
inline int status_after_launch() { return hipGetLastError() == hipSuccess ? QF8_OK : QF8_ERR_HIP; }

}  // namespace

int stream_grid(int64_t n, int dtype) {
    const int64_t per_run = (int64_t)kThreads * kVecs;
    int64_t g = (vec_count(n, dtype) + per_run - 1) / per_run;
    if (g > kMaxStreamGrid) g = kMaxStreamGrid;
    return (int)(g < 1 ? 1 : g);
}

int amax_grid(int64_t n, int dtype) {
    const int64_t per_wg = (int64_t)kAmaxThreads * kAmaxDepth;      // vectors of one full batch
    int64_t g = (vec_count(n, dtype) + per_wg - 1) / per_wg;
    if (g > kAmaxGrid) g = kAmaxGrid;
    return (int)(g < 1 ? 1 : g);
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
    if (dtype == QF8_IN_BF16)
        hipLaunchKernelGGL(amax_partials_kernel<true>, dim3(grid), dim3(kAmaxThreads), 0, s, x, n, nvec, partials);
    else
        hipLaunchKernelGGL(amax_partials_kernel<false>, dim3(grid), dim3(kAmaxThreads), 0, s, x, n, nvec, partials);
    return status_after_launch();
}

int launch_cast_current(const void *x, int dtype, int64_t n, int fmt, uint8_t *q, const uint32_t *partials,
                        int nparts, float *amax_out, float *scale_out, int32_t *nonfinite, int grid, hipStream_t s) {
    const int64_t nvec = vec_count(n, dtype);
    QF8_DISPATCH_DT_FMT(dtype, fmt,
        hipLaunchKernelGGL((cast_current_kernel<BF16, FMT>), dim3(grid), dim3(kThreads), 0, s, x, n, nvec, q,
                           partials, nparts, amax_out, scale_out, nonfinite));
    return status_after_launch();
}

int launch_cast_scaled(const void *x, int dtype, int64_t n, int fmt, const float *scale, uint8_t *q, int grid,
                       hipStream_t s) {
    const int64_t nvec = vec_count(n, dtype);
    QF8_DISPATCH_DT_FMT(dtype, fmt,
        hipLaunchKernelGGL((cast_scaled_kernel<BF16, FMT>), dim3(grid), dim3(kThreads), 0, s, x, n, nvec, scale, q));
    return status_after_launch();
}

int launch_cast_fused(const void *x, int dtype, int64_t n, int fmt, const float *scale, uint8_t *q,
                      float *scale_used, uint32_t *slots, int split, int64_t lo, int64_t hi, int grid,
                      hipStream_t s) {
    const int64_t nvec = vec_count(n, dtype);
    if (split)
        QF8_DISPATCH_DT_FMT(dtype, fmt,
            hipLaunchKernelGGL((cast_fused_kernel<BF16, FMT, true>), dim3(grid), dim3(kThreads), 0, s, x, n, nvec,
                               scale, q, scale_used, slots, lo, hi));
    else
        QF8_DISPATCH_DT_FMT(dtype, fmt,
            hipLaunchKernelGGL((cast_fused_kernel<BF16, FMT, false>), dim3(grid), dim3(kThreads), 0, s, x, n, nvec,
                               scale, q, scale_used, slots, (int64_t)0, (int64_t)0));
    return status_after_launch();
}

namespace {
constexpr int64_t kOnePassMinElems = 1 << 22;
constexpr int kMaxDevices = 64;
std::atomic<int> g_onepass_grid[kMaxDevices][2];   // 0 = not yet known, -1 = not usable
std::atomic<int> g_onepass_override[kMaxDevices];  // 0 = one workgroup per CU

int query_onepass_grid(int dtype) {
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::atomic<int> &slot = g_onepass_grid[dev][dtype == QF8_IN_BF16 ? 0 : 1];
    int g = slot.load(std::memory_order_relaxed);
    if (g != 0) return g;
    const void *fn = dtype == QF8_IN_BF16 ? (const void *)per_tensor_onepass_kernel<true, kE4M3, kOpFp8>
                                          : (const void *)per_tensor_onepass_kernel<false, kE4M3, kOpFp8>;
    g = -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kOpThreads, 0) == hipSuccess && occ >= 1 && cus >= 1)
        g = cus < kBarMaxGroups ? cus : kBarMaxGroups;
    slot.store(g, std::memory_order_relaxed);
    return g;
}
}  // namespace

int onepass_grid(int64_t n, int dtype) {
    if (n < kOnePassMinElems) return 0;
    const int g = query_onepass_grid(dtype);
    if (g <= 0) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return g;
    const int o = g_onepass_override[dev].load(std::memory_order_relaxed);
    return o > 0 ? o : g;
}

int set_onepass_grid(int grid) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QF8_ERR_HIP;
    g_onepass_override[dev].store(grid, std::memory_order_relaxed);
    return QF8_OK;
}

int launch_per_tensor_onepass(const void *x, int dtype, int64_t n, int fmt, uint8_t *q, uint32_t *ws,
                              float *amax_out, float *scale_out, int32_t *nonfinite, uint32_t *amax_bits_out,
                              int grid, hipStream_t s) {
    const int64_t nvec = vec_count(n, dtype);
    QF8_DISPATCH_DT_FMT(dtype, fmt,
        hipLaunchKernelGGL((per_tensor_onepass_kernel<BF16, FMT, kOpFp8>), dim3(grid), dim3(kOpThreads), 0, s, x, n,
                           nvec, q, (uint8_t *)nullptr, ws, amax_out, scale_out, nonfinite, amax_bits_out));
    return status_after_launch();
}

int launch_nvfp4_onepass(const void *x, int dtype, int64_t n, uint8_t *q, uint8_t *s_blk, uint32_t *ws,
                         float *tensor_scale, float *amax_out, int32_t *nonfinite, int grid, hipStream_t s) {
    const int64_t nvec = vec_count(n, dtype);
    if (dtype == QF8_IN_BF16)
        hipLaunchKernelGGL((per_tensor_onepass_kernel<true, kE4M3, kOpNvfp4>), dim3(grid), dim3(op_threads<kOpNvfp4>()), 0, s, x, n,
                           nvec, q, s_blk, ws, amax_out, tensor_scale, nonfinite, (uint32_t *)nullptr);
    else
        hipLaunchKernelGGL((per_tensor_onepass_kernel<false, kE4M3, kOpNvfp4>), dim3(grid), dim3(op_threads<kOpNvfp4>()), 0, s, x,
                           n, nvec, q, s_blk, ws, amax_out, tensor_scale, nonfinite, (uint32_t *)nullptr);
    return status_after_launch();
}

int launch_delayed_finalize(uint32_t *slots, const uint32_t *partials, int nparts, float *history, int32_t *meta,
                            float *scale, int hist_len, int n_guard, int fmt, int update, int estimator,
                            int split, float *amax_out, int32_t *nonfinite, hipStream_t s) {
    if (fmt == QF8_E4M3)
        hipLaunchKernelGGL(delayed_finalize_kernel<kE4M3>, dim3(1), dim3(kFinalizeThreads), 0, s, slots, partials, nparts,
                           history, meta, scale, hist_len, n_guard, update, estimator, split, amax_out, nonfinite);
    else
        hipLaunchKernelGGL(delayed_finalize_kernel<kE5M2>, dim3(1), dim3(kFinalizeThreads), 0, s, slots, partials, nparts,
                           history, meta, scale, hist_len, n_guard, update, estimator, split, amax_out, nonfinite);
    return status_after_launch();
}

// ---- the per-tensor workspace for callers that cannot allocate -------------------------------
// A file-scope device array with the layout of a caller's workspace: each GPU holds its own copy
// (each device loads its own copy of this code object) from load until the process ends. It starts
// zero (a device object without initializer is zero-filled when the code object is loaded), and
// every call leaves its barrier and slot words zero again, as with a caller's workspace. In host
// code `scratch` names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that address is handed
// to kernels.
static __device__ __align__(256) uint32_t scratch[kWorkspaceBytes / sizeof(uint32_t)];
static_assert(sizeof(scratch) >= kWorkspaceBytes, "the scratch array holds a whole workspace");

namespace {
std::atomic<uint32_t *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

int scratch_workspace(uint32_t **ws, size_t *ws_bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QF8_ERR_HIP;
    uint32_t *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return QF8_ERR_HIP;
            p = (uint32_t *)addr;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ws = p;
    *ws_bytes = sizeof(scratch);
    return QF8_OK;
}

int launch_fill_u32(uint32_t *p, int64_t n, uint32_t value, hipStream_t s) {
    if (n <= 0) return QF8_OK;
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 1024) g = 1024;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, p, n, value);
    return status_after_launch();
}

}  // namespace qf8
