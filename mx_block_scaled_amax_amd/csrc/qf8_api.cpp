// qf8_api.cpp -- the C ABI declared in include/qf8.h: argument validation and kernel dispatch.
// Every check happens on the host before anything is enqueued; nothing here synchronizes.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

#include "../../include/qf8.h"
#include "qf8_internal.h"

namespace {

constexpr int32_t kDelayedMagic = 0x51463844;  // "QF8D"
constexpr int kMaxHistory = 4096;
constexpr int kMaxGuard = 64;
constexpr int64_t kMaxMxDim = 1 << 24;   // keeps every per-wave buffer offset below 2^31
// The columnwise FP8 output of one 256-column tile spans 256 * rows bytes of one buffer
// descriptor; the parking offset 2^31 of idle lanes must stay outside it.
constexpr int64_t kMaxMxColRows = 1 << 23;

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool fmt_ok(int fmt) { return fmt == QF8_E4M3 || fmt == QF8_E5M2; }
inline bool dtype_ok(int dt) { return dt == QF8_IN_BF16 || dt == QF8_IN_FP32; }
inline hipStream_t as_stream(void *s) { return (hipStream_t)s; }
// kernel launchers report an int status; the entry points return it as qf8_status
inline qf8_status status_of(int v) { return static_cast<qf8_status>(v); }

// rows, cols >= 0 and rows * cols representable
inline bool dims_ok(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return false;
    if (rows > 0 && cols > INT64_MAX / 16 / rows) return false;
    return true;
}

int check_delayed(const qf8_delayed_state *st) {
    if (!st) return QF8_ERR_NULL;
    if (st->magic != kDelayedMagic) return QF8_ERR_STATE;
    if (!st->history || !st->meta || !st->scale) return QF8_ERR_NULL;
    if (st->hist_len < 1 || st->hist_len > kMaxHistory || st->interval < 1 || st->n_guard < 0 ||
        st->n_guard > kMaxGuard || !fmt_ok(st->fmt) || st->step < 0 || st->estimator < 0 ||
        st->estimator > QF8_EST_MEAN || (st->flags & ~QF8_DELAYED_SPLIT_AMAX) != 0)
        return QF8_ERR_STATE;
    return QF8_OK;
}

}  // namespace

extern "C" {

const char *qf8_status_string(qf8_status status) {
    switch (status) {
        case QF8_OK: return "QF8_OK";
        case QF8_ERR_NULL: return "QF8_ERR_NULL: a required pointer is NULL";
        case QF8_ERR_ENUM: return "QF8_ERR_ENUM: format, dtype or rounding mode out of range";
        case QF8_ERR_SHAPE: return "QF8_ERR_SHAPE: size not accepted by this operation";
        case QF8_ERR_ALIGN: return "QF8_ERR_ALIGN: pointer not 16-byte aligned";
        case QF8_ERR_WORKSPACE: return "QF8_ERR_WORKSPACE: workspace missing or too small";
        case QF8_ERR_STATE: return "QF8_ERR_STATE: delayed-scaling state invalid";
        case QF8_ERR_HIP: return "QF8_ERR_HIP: kernel launch failed";
        default: return "unknown qf8 status";
    }
}

size_t qf8_workspace_bytes(int64_t rows, int64_t cols, qf8_dtype dtype) {
    (void)rows; (void)cols; (void)dtype;
    return qf8::kWorkspaceBytes;
}

qf8_status qf8_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return QF8_ERR_NULL;
    if (ws_bytes < qf8::kWorkspaceBytes) return QF8_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return QF8_ERR_ALIGN;
    return status_of(qf8::launch_fill_u32((uint32_t *)ws, (int64_t)(qf8::kWorkspaceBytes / 4), 0u,
                                          as_stream(stream)));
}

qf8_status qf8_set_onepass_grid(int grid) {
    if (grid < 0 || grid > qf8::kBarMaxGroups) return QF8_ERR_SHAPE;
    return status_of(qf8::set_onepass_grid(grid));
}

qf8_status qf8_cast_scaled(const void *x, qf8_dtype dtype, int64_t n, qf8_fmt fmt, const float *scale, uint8_t *q,
                           void *stream) {
    if (!dtype_ok(dtype) || !fmt_ok(fmt)) return QF8_ERR_ENUM;
    if (n < 0) return QF8_ERR_SHAPE;
    if (n == 0) return QF8_OK;
    if (!x || !scale || !q) return QF8_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return QF8_ERR_ALIGN;
    return status_of(qf8::launch_cast_scaled(x, dtype, n, fmt, scale, q, qf8::stream_grid(n, dtype),
                                             as_stream(stream)));
}

qf8_status quantize_per_tensor(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt, uint8_t *q,
                               float *amax, float *scale, int32_t *nonfinite, void *ws, size_t ws_bytes,
                               void *stream) {
    if (!dtype_ok(dtype) || !fmt_ok(fmt)) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols)) return QF8_ERR_SHAPE;
    const int64_t n = rows * cols;
    if ((n > 0 && (!x || !q)) || !amax || !scale) return QF8_ERR_NULL;
    if (!ws || ws_bytes < qf8::kWorkspaceBytes) return QF8_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(amax, 4) || !aligned(scale, 4) || !aligned(ws, 16) ||
        (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    const int g1 = qf8::onepass_grid(n, dtype);
    if (g1 > 0)
        return status_of(qf8::launch_per_tensor_onepass(x, dtype, n, fmt, q, (uint32_t *)ws, amax, scale, nonfinite,
                                                        nullptr, g1, s));
    uint32_t *partials = (uint32_t *)ws + qf8::kPartialsOffsetWords;
    const int agrid = qf8::amax_grid(n, dtype);
    int st = qf8::launch_amax_partials(x, dtype, n, partials, agrid, s);
    if (st != QF8_OK) return status_of(st);
    return status_of(qf8::launch_cast_current(x, dtype, n, fmt, q, partials, agrid, amax, scale, nonfinite,
                                              qf8::stream_grid(n, dtype), s));
}

qf8_status quantize_per_tensor_noalloc(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt,
                                       uint8_t *q, float *amax, float *scale, int32_t *nonfinite, void *stream) {
    // the argument checks of quantize_per_tensor come first, so a bad call touches no device state
    if (!dtype_ok(dtype) || !fmt_ok(fmt)) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols)) return QF8_ERR_SHAPE;
    const int64_t n = rows * cols;
    if ((n > 0 && (!x || !q)) || !amax || !scale) return QF8_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(amax, 4) || !aligned(scale, 4) ||
        (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    uint32_t *ws = nullptr;
    size_t ws_bytes = 0;
    const int st = qf8::scratch_workspace(&ws, &ws_bytes);
    if (st != QF8_OK) return status_of(st);
    if (ws_bytes < qf8::kWorkspaceBytes) return QF8_ERR_WORKSPACE;   // fixed size: every shape fits
    return status_of(quantize_per_tensor(x, dtype, rows, cols, fmt, q, amax, scale, nonfinite, ws, ws_bytes, stream));
}

qf8_status qf8_delayed_init_ex(qf8_delayed_state *st, float *history, int32_t *meta, float *scale, int hist_len,
                               int interval, int n_guard, qf8_fmt fmt, qf8_estimator estimator, int flags,
                               void *stream) {
    if (!st || !history || !meta || !scale) return QF8_ERR_NULL;
    if (!fmt_ok(fmt) || estimator < QF8_EST_MAX || estimator > QF8_EST_MEAN || (flags & ~QF8_DELAYED_SPLIT_AMAX))
        return QF8_ERR_ENUM;
    if (hist_len < 1 || hist_len > kMaxHistory || interval < 1 || n_guard < 0 || n_guard > kMaxGuard)
        return QF8_ERR_STATE;
    if (!aligned(history, 4) || !aligned(meta, 4) || !aligned(scale, 4)) return QF8_ERR_ALIGN;
    st->history = history;
    st->meta = meta;
    st->scale = scale;
    st->hist_len = hist_len;
    st->interval = interval;
    st->n_guard = n_guard;
    st->fmt = fmt;
    st->step = 0;
    st->magic = kDelayedMagic;
    st->estimator = estimator;
    st->flags = flags;
    st->reserved = 0;
    return status_of(qf8_delayed_reset(st, stream));
}

qf8_status qf8_delayed_init(qf8_delayed_state *st, float *history, int32_t *meta, float *scale, int hist_len,
                            int interval, int n_guard, qf8_fmt fmt, void *stream) {
    return status_of(qf8_delayed_init_ex(st, history, meta, scale, hist_len, interval, n_guard, fmt, QF8_EST_MAX, 0,
                                         stream));
}

qf8_status qf8_delayed_reset(qf8_delayed_state *st, void *stream) {
    int c = check_delayed(st);
    if (c != QF8_OK) return status_of(c);
    hipStream_t s = as_stream(stream);
    // cleared with a fill kernel rather than a memset, so a captured graph replays it correctly
    int r = qf8::launch_fill_u32((uint32_t *)st->history, st->hist_len, 0u, s);
    if (r == QF8_OK) r = qf8::launch_fill_u32((uint32_t *)st->meta, 4, 0u, s);
    if (r == QF8_OK) r = qf8::launch_fill_u32((uint32_t *)st->scale, 1, 0x3F800000u /* 1.0f */, s);
    if (r == QF8_OK) st->step = 0;
    return status_of(r);
}

qf8_status quantize_delayed(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt,
                            qf8_delayed_state *st, uint8_t *q, float *scale_used, float *amax_out, int32_t *nonfinite,
                            void *ws, size_t ws_bytes, void *stream) {
    int c = check_delayed(st);
    if (c != QF8_OK) return status_of(c);
    if (!dtype_ok(dtype) || !fmt_ok(fmt)) return QF8_ERR_ENUM;
    if (fmt != st->fmt) return QF8_ERR_STATE;     // the state was initialised for another format
    if (!dims_ok(rows, cols)) return QF8_ERR_SHAPE;
    const int64_t n = rows * cols;
    if (n > 0 && (!x || !q)) return QF8_ERR_NULL;
    if (!ws || ws_bytes < qf8::kWorkspaceBytes) return QF8_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(ws, 16) || (scale_used && !aligned(scale_used, 4)) ||
        (amax_out && !aligned(amax_out, 4)) || (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    uint32_t *partials = (uint32_t *)ws + qf8::kPartialsOffsetWords;
    uint32_t *slots = (uint32_t *)ws + qf8::kSlotsOffsetWords;
    const int grid = qf8::stream_grid(n, dtype);
    int r;
    if (st->step == 0) {
        // no history yet: current scaling (Eq.(1)-(2), no margin), then append this amax
        const int g1 = qf8::onepass_grid(n, dtype);
        int nparts = 0;
        if (g1 > 0) {              // the single-pass kernel leaves the amax in slot 0
            r = qf8::launch_per_tensor_onepass(x, dtype, n, st->fmt, q, (uint32_t *)ws, nullptr, scale_used, nullptr,
                                               slots, g1, s);
        } else {
            nparts = qf8::amax_grid(n, dtype);
            r = qf8::launch_amax_partials(x, dtype, n, partials, nparts, s);
            if (r == QF8_OK)
                r = qf8::launch_cast_current(x, dtype, n, st->fmt, q, partials, nparts, nullptr, scale_used, nullptr,
                                             grid, s);
        }
        if (r == QF8_OK)
            r = qf8::launch_delayed_finalize(slots, partials, nparts, st->history, st->meta, st->scale, st->hist_len,
                                             st->n_guard, st->fmt, 1, st->estimator, 0, amax_out, nonfinite, s);
    } else {
        // cast with the scale the history gave, fusing this step's amax into the pass (atomic
        // maxima in the workspace slots); then append the amax on update steps and compute the
        // next scale
        const int update = (st->step % st->interval) == 0;
        const int split = (st->flags & QF8_DELAYED_SPLIT_AMAX) != 0;
        int64_t lo = 0, hi = 0;
        if (split) {
            // piece k = (t - 1) mod I: [floor(k n / I), floor((k+1) n / I)), computed as
            // k (n / I) + k (n % I) / I so that no product exceeds I^2 < 2^62
            const int64_t I = st->interval, k = (st->step - 1) % I, qn = n / I, rn = n % I;
            lo = k * qn + (k * rn) / I;
            hi = (k + 1) * qn + ((k + 1) * rn) / I;
        }
        if (!update && !split && !scale_used && !amax_out && !nonfinite) {
            // a reuse step whose caller wants no diagnostics: the cast alone (its amax would
            // only be reported, and the state does not change)
            r = qf8::launch_cast_scaled(x, dtype, n, st->fmt, st->scale, q, grid, s);
            if (r == QF8_OK) st->step++;
            return status_of(r);
        }
        r = qf8::launch_cast_fused(x, dtype, n, st->fmt, st->scale, q, scale_used, slots, split, lo, hi, grid, s);
        if (r == QF8_OK)
            r = qf8::launch_delayed_finalize(slots, partials, 0, st->history, st->meta, st->scale, st->hist_len,
                                             st->n_guard, st->fmt, update, st->estimator, split, amax_out, nonfinite,
                                             s);
    }
    if (r == QF8_OK) st->step++;
    return status_of(r);
}

qf8_status quantize_block_ex(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, int block_rows,
                             int block_cols, qf8_fmt fmt, int flags, uint8_t *q, float *scales, float *amax,
                             int32_t *nonfinite, void *stream) {
    if (!dtype_ok(dtype) || !fmt_ok(fmt)) return QF8_ERR_ENUM;
    if (flags & ~QF8_FLAG_POW2_SCALES) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols)) return QF8_ERR_SHAPE;
    if (!((block_rows == 1 || block_rows == 128) && block_cols == 128)) return QF8_ERR_SHAPE;
    if (cols % (dtype == QF8_IN_BF16 ? 8 : 4) != 0) return QF8_ERR_SHAPE;
    if (rows > INT32_MAX || cols > INT32_MAX) return QF8_ERR_SHAPE;
    const int64_t ngroups = ((rows + block_rows - 1) / block_rows) * ((cols + 127) / 128);
    if (ngroups > INT32_MAX) return QF8_ERR_SHAPE;
    if (rows * cols == 0) return QF8_OK;
    if (!x || !q || !scales) return QF8_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4) || (amax && !aligned(amax, 4)) ||
        (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    return status_of(qf8::launch_block(x, dtype, rows, cols, block_rows, fmt, flags & QF8_FLAG_POW2_SCALES, q, scales,
                                       amax, nonfinite, as_stream(stream)));
}

qf8_status quantize_block(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, int block_rows, int block_cols,
                          qf8_fmt fmt, uint8_t *q, float *scales, float *amax, int32_t *nonfinite, void *stream) {
    return status_of(quantize_block_ex(x, dtype, rows, cols, block_rows, block_cols, fmt, 0, q, scales, amax,
                                       nonfinite, stream));
}

qf8_status requantize_1x128_to_128x1(const uint8_t *q, const float *scales, int64_t rows, int64_t cols,
                                     qf8_fmt fmt_in, qf8_fmt fmt_out, int flags, uint8_t *qT, float *scalesT,
                                     int32_t *nonfinite, void *stream) {
    if (!fmt_ok(fmt_in) || !fmt_ok(fmt_out)) return QF8_ERR_ENUM;
    if (flags & ~QF8_FLAG_POW2_SCALES) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || rows % 16 != 0 || cols % 16 != 0) return QF8_ERR_SHAPE;
    if (rows > INT32_MAX || cols > INT32_MAX || ((rows + 127) / 128) * ((cols + 127) / 128) > INT32_MAX)
        return QF8_ERR_SHAPE;
    if (rows * cols == 0) return QF8_OK;
    if (!q || !scales || !qT || !scalesT) return QF8_ERR_NULL;
    if (!aligned(q, 16) || !aligned(qT, 16) || !aligned(scales, 4) || !aligned(scalesT, 4) ||
        (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    return status_of(qf8::launch_requant_t(q, scales, rows, cols, fmt_in, fmt_out, flags & QF8_FLAG_POW2_SCALES, qT,
                                           scalesT, nonfinite, as_stream(stream)));
}

qf8_status quantize_mx_dual(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_fmt fmt, qf8_mx_round rnd,
                            uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite,
                            void *stream) {
    if (!dtype_ok(dtype) || !fmt_ok(fmt) || (rnd != QF8_MX_ROUND_DOWN && rnd != QF8_MX_ROUND_UP)) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || rows > kMaxMxDim || cols > kMaxMxDim) return QF8_ERR_SHAPE;
    if (!q_row && !q_colT) return QF8_ERR_NULL;
    if ((q_row && !s_row) || (q_colT && !s_colT)) return QF8_ERR_NULL;
    if (q_row && cols % 32 != 0) return QF8_ERR_SHAPE;
    if (q_colT && (rows % 32 != 0 || rows > kMaxMxColRows)) return QF8_ERR_SHAPE;
    if (cols % (dtype == QF8_IN_BF16 ? 8 : 4) != 0) return QF8_ERR_SHAPE;
    if (rows * cols == 0) return QF8_OK;
    if (!x) return QF8_ERR_NULL;
    if (!aligned(x, 16) || (q_row && !aligned(q_row, 16)) || (q_colT && !aligned(q_colT, 16)) ||
        (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    return status_of(qf8::launch_mx(x, dtype, rows, cols, fmt, rnd, q_row, s_row, q_colT, s_colT, nonfinite,
                                    as_stream(stream)));
}

qf8_status quantize_mxfp4_dual(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, qf8_mx_round rnd,
                               uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite,
                               void *stream) {
    if (!dtype_ok(dtype) || (rnd != QF8_MX_ROUND_DOWN && rnd != QF8_MX_ROUND_UP)) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || rows > kMaxMxDim || cols > kMaxMxDim) return QF8_ERR_SHAPE;
    if (!q_row && !q_colT) return QF8_ERR_NULL;
    if ((q_row && !s_row) || (q_colT && !s_colT)) return QF8_ERR_NULL;
    if (q_row && cols % 32 != 0) return QF8_ERR_SHAPE;
    if (q_colT && rows % 32 != 0) return QF8_ERR_SHAPE;
    if (cols % (dtype == QF8_IN_BF16 ? 8 : 4) != 0) return QF8_ERR_SHAPE;
    if (rows * cols == 0) return QF8_OK;
    if (!x) return QF8_ERR_NULL;
    if (!aligned(x, 16) || (q_row && !aligned(q_row, 16)) || (q_colT && !aligned(q_colT, 16)) ||
        (nonfinite && !aligned(nonfinite, 4)))
        return QF8_ERR_ALIGN;
    return status_of(qf8::launch_mxfp4(x, dtype, rows, cols, rnd, q_row, s_row, q_colT, s_colT, nonfinite,
                                       as_stream(stream)));
}

qf8_status quantize_nvfp4(const void *x, qf8_dtype dtype, int64_t rows, int64_t cols, const float *amax_in,
                          uint8_t *q, uint8_t *s_blk, float *tensor_scale, float *amax_out, int32_t *nonfinite,
                          void *ws, size_t ws_bytes, void *stream) {
    if (!dtype_ok(dtype)) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || cols % 16 != 0) return QF8_ERR_SHAPE;
    const int64_t n = rows * cols;
    if ((n > 0 && (!x || !q || !s_blk)) || !tensor_scale) return QF8_ERR_NULL;
    if (!amax_in && (!ws || ws_bytes < qf8::kWorkspaceBytes)) return QF8_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(tensor_scale, 4) || (amax_in && !aligned(amax_in, 4)) ||
        (amax_out && !aligned(amax_out, 4)) || (nonfinite && !aligned(nonfinite, 4)) || (ws && !aligned(ws, 16)))
        return QF8_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    uint32_t *partials = ws ? (uint32_t *)ws + qf8::kPartialsOffsetWords : nullptr;
    int nparts = 0;
    if (!amax_in && n > 0) {
        // large tensors: amax and cast in one read (the single-pass kernel of per-tensor scaling)
        const int g1 = qf8::onepass_grid(n, dtype);
        if (g1 > 0)
            return status_of(qf8::launch_nvfp4_onepass(x, dtype, n, q, s_blk, (uint32_t *)ws, tensor_scale, amax_out,
                                                       nonfinite, g1, s));
        // otherwise the read-only amax pass first
        nparts = qf8::amax_grid(n, dtype);
        const int r = qf8::launch_amax_partials(x, dtype, n, partials, nparts, s);
        if (r != QF8_OK) return status_of(r);
    }
    return status_of(qf8::launch_nvfp4(x, dtype, n, partials, nparts, amax_in, q, s_blk, tensor_scale, amax_out,
                                       nonfinite, s));
}

qf8_status dequantize_mxfp4(const uint8_t *q, const uint8_t *sb, int64_t rows, int64_t cols, void *out,
                            qf8_out_dtype out_dtype, void *stream) {
    if (out_dtype != QF8_OUT_BF16 && out_dtype != QF8_OUT_FP32) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || cols % 32 != 0 || rows * cols >= ((int64_t)1 << 36)) return QF8_ERR_SHAPE;
    const int64_t n = rows * cols;
    if (n == 0) return QF8_OK;
    if (!q || !sb || !out) return QF8_ERR_NULL;
    if (!aligned(q, 16) || !aligned(out, 16)) return QF8_ERR_ALIGN;
    return status_of(qf8::launch_dequant_fp4(0, q, sb, nullptr, n, out, out_dtype, as_stream(stream)));
}

qf8_status dequantize_nvfp4(const uint8_t *q, const uint8_t *s_blk, const float *tensor_scale, int64_t rows,
                            int64_t cols, void *out, qf8_out_dtype out_dtype, void *stream) {
    if (out_dtype != QF8_OUT_BF16 && out_dtype != QF8_OUT_FP32) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || cols % 16 != 0 || rows * cols >= ((int64_t)1 << 36)) return QF8_ERR_SHAPE;
    const int64_t n = rows * cols;
    if (n == 0) return QF8_OK;
    if (!q || !s_blk || !tensor_scale || !out) return QF8_ERR_NULL;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(tensor_scale, 4)) return QF8_ERR_ALIGN;
    return status_of(qf8::launch_dequant_fp4(1, q, s_blk, tensor_scale, n, out, out_dtype, as_stream(stream)));
}

}  // extern "C"

// ---- dequantization and error statistics ---------------------------------------------------
namespace {
constexpr int64_t kMaxDequantElems = (int64_t)1 << 33;   // 4-code units stay below 2^31

int check_dequant(const uint8_t *q, int64_t rows, int64_t cols, int fmt, void *out, int out_dtype, const void *x,
                  int x_dtype, qf8_error_stats *stats, void *ws, size_t ws_bytes) {
    if (!fmt_ok(fmt)) return QF8_ERR_ENUM;
    if (out && out_dtype != QF8_OUT_BF16 && out_dtype != QF8_OUT_FP32) return QF8_ERR_ENUM;
    if (stats && !dtype_ok(x_dtype)) return QF8_ERR_ENUM;
    if (!dims_ok(rows, cols) || rows * cols >= kMaxDequantElems) return QF8_ERR_SHAPE;
    if (!out && !stats) return QF8_ERR_NULL;
    const int64_t n = rows * cols;
    if (n > 0 && !q) return QF8_ERR_NULL;
    if (stats && ((n > 0 && !x) || !ws)) return QF8_ERR_NULL;
    if (stats && ws_bytes < qf8::kWorkspaceBytes) return QF8_ERR_WORKSPACE;
    if (!aligned(q, 16) || (out && !aligned(out, 16)) || (x && !aligned(x, 16)) || (stats && !aligned(stats, 8)) ||
        (ws && !aligned(ws, 16)))
        return QF8_ERR_ALIGN;
    return QF8_OK;
}
}  // namespace

extern "C" {

qf8_status dequantize_scaled(const uint8_t *q, int64_t n, qf8_fmt fmt, const float *scale, void *out,
                             qf8_out_dtype out_dtype, const void *x, qf8_dtype x_dtype, qf8_error_stats *stats,
                             void *ws, size_t ws_bytes, void *stream) {
    int c = check_dequant(q, 1, n, fmt, out, out_dtype, x, x_dtype, stats, ws, ws_bytes);
    if (c != QF8_OK) return status_of(c);
    if (!scale) return QF8_ERR_NULL;
    if (!aligned(scale, 4)) return QF8_ERR_ALIGN;
    if (n == 0 && !stats) return QF8_OK;
    return status_of(qf8::launch_dequant(0, fmt, q, 1, n, 1, scale, nullptr, out, out_dtype, x, x_dtype, stats, ws,
                                         as_stream(stream)));
}

qf8_status dequantize_block(const uint8_t *q, int64_t rows, int64_t cols, int block_rows, int block_cols, qf8_fmt fmt,
                            const float *scales, void *out, qf8_out_dtype out_dtype, const void *x, qf8_dtype x_dtype,
                            qf8_error_stats *stats, void *ws, size_t ws_bytes, void *stream) {
    int c = check_dequant(q, rows, cols, fmt, out, out_dtype, x, x_dtype, stats, ws, ws_bytes);
    if (c != QF8_OK) return status_of(c);
    if (!((block_rows == 1 || block_rows == 128) && block_cols == 128)) return QF8_ERR_SHAPE;
    if (cols % 4 != 0) return QF8_ERR_SHAPE;
    if (rows * cols > 0 && !scales) return QF8_ERR_NULL;
    if (scales && !aligned(scales, 4)) return QF8_ERR_ALIGN;
    if (rows * cols == 0 && !stats) return QF8_OK;
    return status_of(qf8::launch_dequant(1, fmt, q, rows, cols, block_rows, scales, nullptr, out, out_dtype, x,
                                         x_dtype, stats, ws, as_stream(stream)));
}

qf8_status dequantize_mx(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols, qf8_fmt fmt, void *out,
                         qf8_out_dtype out_dtype, const void *x, qf8_dtype x_dtype, qf8_error_stats *stats, void *ws,
                         size_t ws_bytes, void *stream) {
    int c = check_dequant(q, rows, cols, fmt, out, out_dtype, x, x_dtype, stats, ws, ws_bytes);
    if (c != QF8_OK) return status_of(c);
    if (cols % 32 != 0) return QF8_ERR_SHAPE;
    if (rows * cols > 0 && !s) return QF8_ERR_NULL;
    if (rows * cols == 0 && !stats) return QF8_OK;
    return status_of(qf8::launch_dequant(2, fmt, q, rows, cols, 1, nullptr, s, out, out_dtype, x, x_dtype, stats, ws,
                                         as_stream(stream)));
}

}  // extern "C"
