// qf8_internal.h -- host-side launchers shared between the kernel files and the C ABI layer.
// Arguments are already validated by the ABI layer; each launcher only enqueues kernels and
// returns QF8_OK or QF8_ERR_HIP.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/qf8.h"

namespace qf8 {

// Per-tensor / delayed geometry: number of workgroups of the streaming kernels for n elements.
int stream_grid(int64_t n, int dtype);
// Workgroups (= partial maxima) of the per-tensor amax pass.
int amax_grid(int64_t n, int dtype);
constexpr int kAmaxGrid = 256;
constexpr int kMaxStreamGrid = 16384;  // workgroups of the streaming kernels at most (= partials)

// Workspace layout, in u32 words:
//   [0, kBarHeaderWords)      grid-barrier header: [0] running amax bits, [1] arrival count (one
//                             64-bit word), [2] give-up timeout of a waiting workgroup in 10 ns
//                             ticks (0 = the default: 50 us + 10 ns per 500 KB of input, the
//                             size term at most 1 ms), [3] [4] the single-pass kernel's counters
//                             of given-up slabs (claimed units, finished workgroups)
//   kBarMaxGroups lines of kBarLineWords words (128 B each): the release line of each workgroup
//                             (words 0-1), an entry of the given-up list (word 4), the count of
//                             workgroups that gave up on one shader engine (word 5 of lines
//                             0-31); words 16-17 of every 16th line are a first-level barrier
//                             word of the single-pass kernel
//   kSlotCount lines of kBarLineWords words: word 0 of each is a running |amax| maximum that the
//                             fused delayed-scaling cast raises atomically and the finalize
//                             kernel reads and clears
//   kMaxStreamGrid words      per-workgroup partial maxima of the two-kernel per-tensor path
// Everything before the partials must be zero before the first call; every call leaves it zero.
constexpr int kBarHeaderWords = 32;
constexpr int kBarLineWords = 32;
constexpr int kBarMaxGroups = 512;
constexpr int kSlotCount = 256;
constexpr size_t kSlotsOffsetWords = kBarHeaderWords + (size_t)kBarMaxGroups * kBarLineWords;
constexpr size_t kPartialsOffsetWords = kSlotsOffsetWords + (size_t)kSlotCount * kBarLineWords;
constexpr size_t kWorkspaceBytes = (kPartialsOffsetWords + kMaxStreamGrid) * sizeof(uint32_t);

// Single-pass per-tensor kernel: its grid for n elements of dtype on the current device (one
// workgroup per CU), or 0 when the two-kernel path is used instead (small tensors, or a device
// where one workgroup per CU does not fit).
int onepass_grid(int64_t n, int dtype);
// Overrides that grid on the current device (grid in [1, kBarMaxGroups], 0 = default).
int set_onepass_grid(int grid);
int launch_nvfp4_onepass(const void *x, int dtype, int64_t n, uint8_t *q, uint8_t *s_blk, uint32_t *ws,
                         float *tensor_scale, float *amax_out, int32_t *nonfinite, int grid, hipStream_t s);
int launch_per_tensor_onepass(const void *x, int dtype, int64_t n, int fmt, uint8_t *q, uint32_t *ws,
                              float *amax_out, float *scale_out, int32_t *nonfinite, uint32_t *amax_bits_out,
                              int grid, hipStream_t s);

int launch_dequant_fp4(int nv, const uint8_t *q, const uint8_t *sb, const float *tensor_scale, int64_t n, void *out,
                       int out_dtype, hipStream_t s);
int launch_mxfp4(const void *x, int dtype, int64_t rows, int64_t cols, int rnd, uint8_t *q_row, uint8_t *s_row,
                 uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite, hipStream_t s);
int launch_nvfp4(const void *x, int dtype, int64_t n, const uint32_t *partials, int nparts, const float *amax_in,
                 uint8_t *q, uint8_t *s_blk, float *tensor_scale, float *amax_out, int32_t *nonfinite, hipStream_t s);
int launch_amax_partials(const void *x, int dtype, int64_t n, uint32_t *partials, int grid, hipStream_t s);
int launch_cast_current(const void *x, int dtype, int64_t n, int fmt, uint8_t *q, const uint32_t *partials,
                        int nparts, float *amax_out, float *scale_out, int32_t *nonfinite, int grid, hipStream_t s);
int launch_cast_scaled(const void *x, int dtype, int64_t n, int fmt, const float *scale, uint8_t *q, int grid,
                       hipStream_t s);
int launch_cast_fused(const void *x, int dtype, int64_t n, int fmt, const float *scale, uint8_t *q,
                      float *scale_used, uint32_t *slots, int split, int64_t lo, int64_t hi, int grid,
                      hipStream_t s);
int launch_delayed_finalize(uint32_t *slots, const uint32_t *partials, int nparts, float *history, int32_t *meta,
                            float *scale, int hist_len, int n_guard, int fmt, int update, int estimator,
                            int split, float *amax_out, int32_t *nonfinite, hipStream_t s);
int launch_fill_u32(uint32_t *p, int64_t n, uint32_t value, hipStream_t s);
// The current device's file-scope workspace (quantize_per_tensor_noalloc): its device address and
// size, looked up once per device. QF8_ERR_HIP if the device or the symbol cannot be queried.
int scratch_workspace(uint32_t **ws, size_t *ws_bytes);

int launch_block(const void *x, int dtype, int64_t rows, int64_t cols, int block_rows, int fmt, int pow2, uint8_t *q,
                 float *scales, float *amax, int32_t *nonfinite, hipStream_t s);

// 1x128 groups of q [rows][cols] -> 1x128 groups of the transpose, stored qT [cols][rows] with
// scalesT [cols][ceil(rows/128)]; rows % 16 == 0 and cols % 16 == 0.
int launch_requant_t(const uint8_t *q, const float *scales, int64_t rows, int64_t cols, int fmt_in, int fmt_out,
                     int pow2, uint8_t *qT, float *scalesT, int32_t *nonfinite, hipStream_t s);

int launch_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int rnd, uint8_t *q_row,
              uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite, hipStream_t s);

// De-scaling and error statistics. mode: 0 = one scale factor (scale -> 1 fp32), 1 = groups of
// block_rows x 128 (scale -> the group scale array), 2 = MX (sb -> E8M0 bytes [rows][cols/32]).
// out and stats are each optional (not both absent); stats needs x and the workspace.
int launch_dequant(int mode, int fmt, const uint8_t *q, int64_t rows, int64_t cols, int block_rows,
                   const float *scale, const uint8_t *sb, void *out, int out_dtype, const void *x, int x_dtype,
                   qf8_error_stats *stats, void *ws, hipStream_t s);

}  // namespace qf8
