/*
 * qf8.h -- C ABI of libqf8.so: FP8 tensor quantization (amax -> scale -> saturating RNE cast)
 * on AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (title, section):
 *   [HiF8-train]   "HiFloat8：高性能训练之路" (hifloat.gccorg.com blog)
 *   [MP-FP8]       "混合精度与 FP8 训练" (hs-black.github.io, posts/scaling-mixed-precision)
 *   [MXFP8-recipe] "NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" (51cto.com)
 *   [Ascend950]    Ascend 950 low-precision format guide (hwcomputing.csdn.net), HiF8 vs
 *                  MXFP8 numerical analysis on DeepSeek-V4-Flash
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major and contiguous: element (r, c) of a [rows][cols] tensor is at
 *     r*cols + c. Input elements are BF16 (QF8_IN_BF16, raw 16-bit patterns) or FP32.
 *   - All tensor and scalar arguments named x, q, s_*, scale*, amax*, nonfinite, ws, history,
 *     meta are DEVICE pointers on the current HIP device. The caller owns every buffer; the
 *     library allocates nothing and keeps no pointer after a call returns, except through work
 *     already queued on the stream.
 *   - stream is a hipStream_t passed as void*; NULL is the null stream. Every call only
 *     enqueues work on that stream and returns; results are valid once the stream has
 *     synchronized. No call synchronizes the host.
 *   - Arithmetic: amax is an exact maximum of |x|; a scale F8max/amax is one IEEE fp32
 *     division rounded to nearest even; x*S is one fp32 multiplication; the cast to fp8 is
 *     round-to-nearest-even with saturation to +-F8max (F8max = 448 for E4M3, 57344 for E5M2).
 *     A scale is 1 when the amax it comes from is 0 or not finite, and FLT_MAX when F8max/amax
 *     overflows fp32.
 *   - nonfinite (nullable, device int32): set to 1 when the input holds Inf or NaN, never
 *     cleared by the library (the caller zeroes it). Outputs computed from non-finite input
 *     are outside the bit-exact contract except where stated.
 *   - Return value: QF8_OK or a negative qf8_status. Argument errors are detected on the host
 *     before anything is enqueued; QF8_ERR_HIP reports a failed kernel launch.
 *   - Calls are thread-safe. The only global state is a per-device cache of the CU count and
 *     kernel occupancy, filled on first use. Calls on the same output buffers, the same
 *     workspace or the same delayed state must be ordered by the caller (same stream or events).
 */
#ifndef QF8_H
#define QF8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qf8_fmt { QF8_E4M3 = 0, QF8_E5M2 = 1 } qf8_fmt;
typedef enum qf8_dtype { QF8_IN_BF16 = 0, QF8_IN_FP32 = 1 } qf8_dtype;
/* MX shared-exponent rounding ([MXFP8-recipe 4.1]): OCP round-down X = floor(log2 amax) - emax,
 * or the round-up X = ceil(log2(amax / F8max)) of the recipe's Algorithm 1. */
typedef enum qf8_mx_round { QF8_MX_ROUND_DOWN = 0, QF8_MX_ROUND_UP = 1 } qf8_mx_round;

typedef enum qf8_status {
    QF8_OK = 0,
    QF8_ERR_NULL = -1,       /* a required pointer is NULL */
    QF8_ERR_ENUM = -2,       /* fmt, dtype or rounding mode out of range */
    QF8_ERR_SHAPE = -3,      /* negative size, or a size the operation's grouping cannot take */
    QF8_ERR_ALIGN = -4,      /* a tensor or workspace pointer is not 16-byte aligned (scalars: 4-byte) */
    QF8_ERR_WORKSPACE = -5,  /* ws is NULL or smaller than qf8_workspace_bytes() */
    QF8_ERR_STATE = -6,      /* delayed-scaling state invalid or not initialised */
    QF8_ERR_HIP = -7         /* a HIP launch failed */
} qf8_status;

/* Human-readable name of a status code. Never NULL. */
const char *qf8_status_string(qf8_status status);

/* Bytes of device workspace quantize_per_tensor and quantize_delayed need for a tensor of
 * rows x cols elements of dtype (currently a constant of about 160 KiB): a grid-barrier region
 * (arrival counter, running maximum, one 128-byte release line per workgroup), 256 running
 * amax slots for the fused delayed-scaling cast, and per-workgroup partial maxima. The
 * workspace must be zero-filled once before its first use (for example with
 * qf8_workspace_init); every call leaves the barrier and slot regions zero again, so the same
 * workspace serves any number of later calls ordered on one stream. Two calls that may run at
 * the same time need two workspaces. Word 2 (u32) of the workspace, if non-zero, replaces the
 * default time after which a workgroup waiting at the grid barrier of the single-pass kernel
 * may give up and leave its slabs to the others (50 us plus 10 ns per 500 KB of input, the size
 * term at most 1 ms), in 10 ns ticks (tests set it tiny to exercise that path). */
size_t qf8_workspace_bytes(int64_t rows, int64_t cols, qf8_dtype dtype);

/* Sets the number of workgroups of the single-pass kernel (quantize_per_tensor from 2^22
 * elements, delayed-scaling step 0, quantize_nvfp4 with a measured amax) on the current device:
 * grid in [1, 512], or 0 for the default of one workgroup per CU. A tuning and test hook: a grid
 * larger than the number of workgroups that fit on the device at once still gives the same
 * bytes (after the give-up timeout about as many waiters leave as are missing, and the others
 * cast their slabs), only slower. The setting is per process and device and applies to calls made after it; calls
 * already enqueued keep their grid. Returns QF8_ERR_SHAPE for a grid outside [0, 512] (checked
 * before any HIP call), QF8_ERR_HIP if the current device cannot be queried. */
qf8_status qf8_set_onepass_grid(int grid);

/* Enqueues a zero fill of the qf8_workspace_bytes() bytes at ws (16-byte aligned, ws_bytes at
 * least that size) on stream. */
qf8_status qf8_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Scaled saturating cast (Eq.(2) of [HiF8-train 1.2], [MP-FP8 8.1]):
 *   q[i] = sat_rne8(fl32(x[i] * scale[0])),  i in [0, n).
 * x: n elements of dtype, 16-byte aligned. scale: one device fp32 value. q: n bytes, 16-byte
 * aligned. n >= 0 (n = 0 enqueues nothing). */
qf8_status qf8_cast_scaled(const void *x, qf8_dtype dtype, int64_t n, qf8_fmt fmt, const float *scale, uint8_t *q,
                           void *stream);

/* Per-tensor current scaling ([HiF8-train 1.2] Eq.(1)-(2); [MP-FP8 8.1]):
 *   amax = max |x|;  S = fl32(F8max / amax);  q = sat_rne8(fl32(x * S)).
 * x: rows*cols elements (any rows, cols >= 0), 16-byte aligned. q: rows*cols bytes, 16-byte
 * aligned. amax, scale: one device fp32 each (amax of an empty tensor is 0, its scale 1).
 * ws: qf8_workspace_bytes(rows, cols, dtype) bytes, 16-byte aligned, initialised as described
 * at qf8_workspace_bytes.
 * From 2^22 elements on: one kernel that reads x from HBM once. One workgroup per CU keeps up
 * to 128 MiB of the tensor in registers and LDS (on 256 CUs) across a grid barrier on the amax
 * and casts from there; the rest of a larger tensor is re-read. Below 2^22 elements: two
 * kernels (grid-wide partial maxima, then the cast; each cast workgroup folds the partials). */
qf8_status quantize_per_tensor(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt, uint8_t *q,
                               float *amax, float *scale, int32_t *nonfinite, void *ws, size_t ws_bytes,
                               void *stream);

/* quantize_per_tensor without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (minus ws, ws_bytes), results and errors as quantize_per_tensor; it allocates
 * nothing (no hipMalloc, hipFree or allocating library call). The workspace is a file-scope
 * device array of qf8_workspace_bytes() bytes (about 160 KiB) inside the library: each GPU the
 * library runs on holds its own copy until the process ends. Its size does not depend on the
 * tensor, so no shape quantize_per_tensor accepts is refused for lack of scratch (QF8_ERR_WORKSPACE
 * would mean a library built with a smaller array). The array starts zero and every call leaves it
 * zero again, so calls ordered on one stream need no set-up; calls that overlap on one GPU (two
 * streams or two threads without ordering between them) share that array and race. The first call
 * on a device looks the array's device address up (QF8_ERR_HIP if that fails). The give-up timeout
 * of the single-pass kernel is the default (word 2 of the array stays 0). */
qf8_status quantize_per_tensor_noalloc(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt,
                                       uint8_t *q, float *amax, float *scale, int32_t *nonfinite, void *stream);

/* Per-tensor delayed scaling ([HiF8-train 1.2] Eq.(3)-(4) and section 5.2; [MP-FP8 8.2]).
 * State: a FIFO of the last hist_len amax values kept on the device; the estimate is the
 * maximum over it; the scale a step uses is S = fl32(F8max / estimate) * 2^-n_guard.
 * Step 0 after init or reset has no history and runs current scaling (no margin). Every step
 * t >= 1 casts with the scale the history gave before the step; when t % interval == 0 (and
 * at step 0) the step's own amax is appended afterwards, dropping the oldest entry when the
 * FIFO is full, and the next scale is derived with the state's estimator. A non-finite amax is
 * never appended (it sets nonfinite instead).
 * history (hist_len fp32), meta (4 int32) and scale (1 fp32) are caller-owned device buffers
 * that must outlive every queued step; step is a host counter the library advances.
 * Checkpoint = copy history, meta, scale and step; resume = copy them back. */
typedef struct qf8_delayed_state {
    float *history;      /* device: hist_len fp32 slots */
    int32_t *meta;       /* device: [0] count, [1] head (oldest slot), [2] split-amax window
                            maximum (fp32 bits), [3] reserved */
    float *scale;        /* device: the scale the next delayed step uses */
    int32_t hist_len;    /* 1 .. 4096 */
    int32_t interval;    /* >= 1 */
    int32_t n_guard;     /* 0 .. 64 */
    int32_t fmt;         /* qf8_fmt */
    int64_t step;        /* host: number of steps since init or reset */
    int32_t magic;       /* set by qf8_delayed_init */
    int32_t estimator;   /* qf8_estimator (0 with qf8_delayed_init) */
    int32_t flags;       /* qf8_delayed_flags (0 with qf8_delayed_init) */
    int32_t reserved;
} qf8_delayed_state;

/* How the amax estimate is taken from the history ([HiF8-train 1.2]: the maximum of the buffer,
 * or another rule such as the most recent entry or the mean). The mean is the fp32 sum of the
 * entries from oldest to newest divided by the count in fp32. An empty history estimates 0. */
typedef enum qf8_estimator { QF8_EST_MAX = 0, QF8_EST_RECENT = 1, QF8_EST_MEAN = 2 } qf8_estimator;

/* QF8_DELAYED_SPLIT_AMAX: spread the amax measurement over the interval ([HiF8-train], the
 * section comparing HiF8 with FP8 and MXFP8: the tensor is cut into equal sub-tensors and one
 * is measured per step). The flattened tensor of n elements is cut into interval consecutive
 * pieces [floor(k n / I), floor((k+1) n / I)); step t >= 1 measures piece (t - 1) mod I, and
 * the update step t % I == 0 appends the maximum of the window's I piece amaxes (nothing when
 * one of them was Inf/NaN). Step 0 is unchanged. amax_out and nonfinite still describe the
 * whole tensor, which the fused pass reads anyway. */
typedef enum qf8_delayed_flags { QF8_DELAYED_SPLIT_AMAX = 1 } qf8_delayed_flags;

/* Fills the host fields, clears history/meta/scale on the device, step = 0; the estimator is the
 * maximum of the history. */
qf8_status qf8_delayed_init(qf8_delayed_state *st, float *history, int32_t *meta, float *scale, int hist_len,
                            int interval, int n_guard, qf8_fmt fmt, void *stream);
/* The same with an estimator (qf8_estimator) and flags (qf8_delayed_flags); other values give
 * QF8_ERR_ENUM. */
qf8_status qf8_delayed_init_ex(qf8_delayed_state *st, float *history, int32_t *meta, float *scale, int hist_len,
                               int interval, int n_guard, qf8_fmt fmt, qf8_estimator estimator, int flags,
                               void *stream);
/* Empties the history and sets step = 0, so the next step is current scaling again (the
 * restart after an anomaly, [HiF8-train 5.2]). */
qf8_status qf8_delayed_reset(qf8_delayed_state *st, void *stream);
/* One iteration on x (rows*cols elements, 16-byte aligned) -> q (16-byte aligned). fmt must be
 * the format the state was initialised with (QF8_ERR_STATE otherwise): the history holds amax
 * values whose scales are F8max of that format over the estimate.
 * scale_used (nullable): the scale this step cast with. amax_out (nullable): this step's true
 * amax over the whole tensor (computed in the same pass as the cast; only update steps append
 * it to the history, or with QF8_DELAYED_SPLIT_AMAX the window's maximum over its pieces).
 * ws: qf8_workspace_bytes(rows, cols, dtype) bytes, 16-byte aligned, initialised as described
 * at qf8_workspace_bytes.
 * Steps after the first are two kernel launches: the cast, which also raises atomic amax
 * maxima in the workspace, and a one-workgroup finalize that reads and clears them and updates
 * the state. A reuse step (not an update step, no QF8_DELAYED_SPLIT_AMAX) called with
 * scale_used, amax_out and nonfinite all NULL is the cast alone: its amax would only be
 * reported. Step 0 is the current-scaling path of quantize_per_tensor, then the finalize. */
qf8_status quantize_delayed(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt,
                            qf8_delayed_state *st, uint8_t *q, float *scale_used, float *amax_out, int32_t *nonfinite,
                            void *ws, size_t ws_bytes, void *stream);

/* Fine-grained current scaling ([MP-FP8 10.2] and 10.3): Eq.(1)-(2) applied to each group of
 * block_rows x block_cols elements on its own; (block_rows, block_cols) is (1, 128) (per-token
 * groups) or (128, 128) (weight blocks). Groups at the right and bottom edges may be partial.
 * x: [rows][cols] with cols % 8 == 0 (BF16) or cols % 4 == 0 (FP32), 16-byte aligned.
 * q: [rows][cols] bytes, 16-byte aligned.
 * scales: [ceil(rows/block_rows)][ceil(cols/block_cols)] fp32, the S_g of each group.
 * amax (nullable): same shape, each group's amax. */
qf8_status quantize_block(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, int block_rows, int block_cols,
                          qf8_fmt fmt, uint8_t *q, float *scales, float *amax, int32_t *nonfinite, void *stream);

/* Flags of quantize_block_ex and requantize_1x128_to_128x1. */
#define QF8_FLAG_POW2_SCALES 1   /* group scales are the largest power of two S with amax*S <= F8max */

/* quantize_block with flags. QF8_FLAG_POW2_SCALES ([MP-FP8 10.4]: the tensors re-grouped from
 * 1x128 to 128x1 use integer powers of two as scale factors, so the re-grouping adds no error):
 * S_g = 2^-X, X = ceil(log2(amax_g / F8max)) clamped to [-127, 127]; 1 for amax_g = 0 or
 * non-finite. Unknown flag bits give QF8_ERR_ENUM. quantize_block is this call with flags 0. */
qf8_status quantize_block_ex(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, int block_rows,
                             int block_cols, qf8_fmt fmt, int flags, uint8_t *q, float *scales, float *amax,
                             int32_t *nonfinite, void *stream);

/* Re-grouping of 1x128 groups into 128x1 groups ([MP-FP8 10.5]: read, de-scale, transpose,
 * quantize again, write back). Input: q [rows][cols] (fmt_in) with its 1x128 group scales
 * [rows][ceil(cols/128)] as quantize_block(_ex) writes them. Each value is de-scaled as
 * dequantize_block does (fl32(decode(q) / S)); every column's groups of 128 rows are quantized
 * again (fmt_out, Eq.(1) scales or QF8_FLAG_POW2_SCALES) and stored transposed: qT [cols][rows]
 * with scalesT [cols][ceil(rows/128)], i.e. the 1x128 groups of the transpose. With power-of-two
 * scales on both sides and fmt_in == fmt_out, every value whose re-scaled magnitude is at least
 * the smallest normal fp8 value is carried over exactly. rows % 16 == 0, cols % 16 == 0; q, qT
 * 16-byte aligned. nonfinite (nullable) is set when a group holds Inf/NaN. */
qf8_status requantize_1x128_to_128x1(const uint8_t *q, const float *scales, int64_t rows, int64_t cols,
                                     qf8_fmt fmt_in, qf8_fmt fmt_out, int flags, uint8_t *qT, float *scalesT,
                                     int32_t *nonfinite, void *stream);

/* MX quantization with 1x32 blocks and E8M0 shared scales ([MP-FP8 13.1]; [MXFP8-recipe 4.1]),
 * rowwise and/or columnwise from the same high-precision input in one pass.
 * Per block of 32: amax = 0 gives X = -127 and 32 zero bytes; otherwise X from the rounding
 * mode, clamped to [-127, 127]; scale byte = X + 127; element = sat_rne8(x / 2^X).
 *   rowwise   (q_row non-NULL): blocks run along a row. q_row [rows][cols],
 *             s_row [rows][cols/32]; needs cols % 32 == 0.
 *   columnwise (q_colT non-NULL): blocks run down a column and are stored transposed:
 *             q_colT [cols][rows], s_colT [cols][rows/32]; needs rows % 32 == 0 and
 *             rows <= 2^23.
 * At least one direction; s_row / s_colT are required with their q. x, q_row, q_colT 16-byte
 * aligned; rows, cols <= 2^24. A block holding Inf or NaN gets scale byte 0xFF and sets
 * nonfinite. One kernel launch for either or both directions. */
qf8_status quantize_mx_dual(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt, qf8_mx_round rnd,
                            uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite,
                            void *stream);

/* ---- FP4: E2M1 elements ([MP-FP8 13.2]: values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives; a
 * 4-bit code S.EE.M, sign in bit 3). Codes are packed two per byte, element 2j in the low
 * nibble of byte j and element 2j+1 in the high nibble. The cast rounds to nearest even and
 * saturates to +-6.
 *
 * MXFP4 ([MP-FP8 13.1]; [Ascend950 2.4]: 32 FP4 values share one E8M0 scale): the MX rule of
 * quantize_mx_dual with emax = 2 and largest value 6: round-down X = floor(log2 amax) - 2,
 * round-up X = ceil(log2(amax / 6)), clamped to [-127, 127]; amax = 0 gives X = -127 and zero
 * codes; byte = X + 127 (0xFF and nonfinite for a block with Inf/NaN); code = E2M1(x / 2^X).
 *   rowwise    (q_row non-NULL): q_row [rows][cols/2] packed along the row, s_row
 *              [rows][cols/32]; cols % 32 == 0.
 *   columnwise (q_colT non-NULL): blocks down a column, stored transposed: q_colT
 *              [cols][rows/2] (rows 2j, 2j+1 of a column in byte j), s_colT [cols][rows/32];
 *              rows % 32 == 0.
 * At least one direction; x, q_row, q_colT 16-byte aligned; cols % 8 (BF16) or % 4 (FP32);
 * rows, cols <= 2^24. One kernel launch. */
qf8_status quantize_mxfp4_dual(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_mx_round rnd,
                               uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite,
                               void *stream);

/* NVFP4 ([MP-FP8 13.2]: blocks of 16 along a row, each with an E4M3 scale amax_b / 6 that can
 * align the block maximum to 6, under one fp32 tensor scale because E4M3's range is too
 * small). The tensor scale maps the largest block scale onto E4M3's largest value 448, and each
 * element is divided by its block's real scale decode(e_b) / S_t:
 *   S_t = fl32(448 * 6 / A)  (A = tensor amax; 1 for A = 0 or non-finite; FLT_MAX on overflow)
 *   e_b = E4M3(amax_b * S_t / 6), saturating                           -> s_blk
 *   code = E2M1(x * S_t / decode(e_b)); zero codes of x's sign when decode(e_b) = 0   -> q
 * where E4M3(.) and E2M1(.) round the exact quotient once to the nearest value, ties to even.
 * De-scaled: xhat = code * decode(e_b) / S_t. A block with Inf/NaN gets the E4M3 NaN code 0x7F
 * and sets nonfinite. Layout: q [rows][cols/2] packed, s_blk [rows][cols/16]; cols % 16 == 0;
 * x and q 16-byte aligned. tensor_scale (required) receives S_t, amax_out (nullable) A.
 * amax_in (nullable, device fp32): a tensor amax from the caller (its magnitude is used, e.g.
 * from an amax history); then x is read once and ws may be NULL. Otherwise A is measured: from
 * 2^22 elements by the single-pass kernel of quantize_per_tensor (x held on chip across a grid
 * barrier, read once), below that by a read-only pass first. ws: qf8_workspace_bytes bytes,
 * 16-byte aligned, zero-initialised once as described at qf8_workspace_bytes. */
qf8_status quantize_nvfp4(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, const float *amax_in,
                          uint8_t *q, uint8_t *s_blk, float *tensor_scale, float *amax_out, int32_t *nonfinite,
                          void *ws, size_t ws_bytes, void *stream);

/* ---- Dequantization and quantization error statistics -------------------------------------
 * De-scaling ([MP-FP8 8.1]: the code 22 with S = 22400 gives 22/22400; [MP-FP8 8.2]: the
 * saturated 448 with S = 22.4 gives 20; [MP-FP8 13.1]: an MX element is a code times 2^X):
 *   scale factor S (per tensor, delayed step, or group):  xhat = fl32(decode(q) / S);
 *   MX E8M0 byte b:                    xhat = fl32(decode(q) * 2^(b - 127)), NaN for b = 0xFF.
 * Output out (nullable): [rows][cols] BF16 (xhat rounded to nearest even) or FP32.
 * Statistics (nullable; [MP-FP8 7.2] amax / underflow / saturation watch, [Ascend950] SQNR and
 * zero-rate): the source x (the tensor q was quantized from, same layout as q; for a
 * columnwise MX result that is x transposed) is read alongside and qf8_error_stats is written
 * to device memory. Sums are fp64 over the finite elements of x, reduced in a fixed order (the
 * same input gives the same bits); SQNR = 10 log10(signal / noise), zero-rate = zeroed /
 * nonzero (or / count). With stats, ws (qf8_workspace_bytes) holds per-workgroup partials.
 * At least one of out and stats must be given. q, out and x are 16-byte aligned; stats 8-byte;
 * out overlaps neither q nor x.
 * Sizes: rows * cols < 2^33. */
typedef enum qf8_out_dtype { QF8_OUT_BF16 = 0, QF8_OUT_FP32 = 1 } qf8_out_dtype;

typedef struct qf8_error_stats {
    double signal;      /* sum of x^2 over the finite elements of x */
    double noise;       /* sum of (x - xhat)^2 over the same elements */
    int64_t count;      /* finite elements of x */
    int64_t nonzero;    /* finite elements with x != 0 */
    int64_t zeroed;     /* of those, elements whose xhat is 0 */
    int64_t saturated;  /* elements whose scaled value exceeded F8max before the saturating cast:
                           |fl32(x * S)| > F8max, or |x| > F8max * 2^X for MX */
    int64_t nonfinite;  /* Inf/NaN elements of x, excluded from every other field */
    int64_t reserved;
} qf8_error_stats;

/* One scale factor for all n codes (per-tensor current or delayed scaling: pass the scale the
 * quantization used). scale: one device fp32. */
qf8_status dequantize_scaled(const uint8_t *q, int64_t n, qf8_fmt fmt, const float *scale, void *out,
                             qf8_out_dtype out_dtype, const void *x, qf8_dtype x_dtype, qf8_error_stats *stats,
                             void *ws, size_t ws_bytes, void *stream);

/* Groups of block_rows x block_cols ((1, 128) or (128, 128)) with their fp32 scales
 * [ceil(rows/block_rows)][ceil(cols/128)] as quantize_block writes them; cols % 4 == 0. */
qf8_status dequantize_block(const uint8_t *q, int64_t rows, int64_t cols, int block_rows, int block_cols, qf8_fmt fmt,
                            const float *scales, void *out, qf8_out_dtype out_dtype, const void *x, qf8_dtype x_dtype,
                            qf8_error_stats *stats, void *ws, size_t ws_bytes, void *stream);

/* MX blocks of 32 along each row of q [rows][cols] with E8M0 bytes s [rows][cols/32]: a rowwise
 * result, or a columnwise result in its transposed layout (q_colT, s_colT with rows = the
 * tensor's cols). cols % 32 == 0. */
qf8_status dequantize_mx(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols, qf8_fmt fmt, void *out,
                         qf8_out_dtype out_dtype, const void *x, qf8_dtype x_dtype, qf8_error_stats *stats, void *ws,
                         size_t ws_bytes, void *stream);

/* FP4 de-scaling (the FP4 counterpart of the calls above; no statistics). q is packed two codes
 * per byte as the FP4 quantizers write it; element i uses the scale of its block in flattened
 * order.
 *   dequantize_mxfp4: q [rows][cols/2], sb [rows][cols/32] E8M0 bytes (a columnwise result is
 *     passed as its transpose: q_colT with rows = cols of x); xhat = decode(c) * 2^(b - 127),
 *     exact in fp32 (Inf on overflow), NaN for b = 0xFF. cols % 32 == 0.
 *   dequantize_nvfp4: q [rows][cols/2], s_blk [rows][cols/16] E4M3 codes, tensor_scale (device
 *     fp32 S_t); xhat = fl32(decode(c) * decode(e_b) / S_t) (the product is exact), NaN for
 *     e_b = 0x7F. cols % 16 == 0.
 * out: [rows][cols] BF16 (round to nearest even) or FP32 (qf8_out_dtype). q and out 16-byte
 * aligned; rows * cols < 2^36. */
qf8_status dequantize_mxfp4(const uint8_t *q, const uint8_t *sb, int64_t rows, int64_t cols, void *out,
                            qf8_out_dtype out_dtype, void *stream);
qf8_status dequantize_nvfp4(const uint8_t *q, const uint8_t *s_blk, const float *tensor_scale, int64_t rows,
                            int64_t cols, void *out, qf8_out_dtype out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QF8_H */
