/*
 * qf8_oracle.c -- plain, slow CPU definition of FP8 tensor quantization.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. It shares no code, header, table or helper with the GPU library,
 * and the GPU library never calls it.
 *
 * Everything here is written for a reader to check by eye against the pages:
 *   [HiF8-train]   "HiFloat8：高性能训练之路" (hifloat.gccorg.com blog):
 *                  section 1.2 (current scaling, Eq.(1)-(2); delayed scaling, Eq.(3)-(4),
 *                  amax history, Interval) and section 5.2 (first step / restart is current).
 *   [MP-FP8]       "混合精度与 FP8 训练" (hs-black.github.io, posts/scaling-mixed-precision):
 *                  sections 2.1-2.3 (field layout, E4M3/E5M2, the 0.1 example), 3 (binades),
 *                  4.1 (round to nearest, ties to even), 8.1 (S = F8max/amax, saturation),
 *                  8.2 (delayed scaling, margin), 10.2 (1x128 and 128x128 groups),
 *                  13.1 (MX blocks of 32, E8M0 scale, shared exponent, the 5.3 example).
 *   [MXFP8-recipe] "NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" (51cto.com):
 *                  section 4.1 (amax = 0 gives X = -127, OCP round-down exponent, the
 *                  round-up exponent of Algorithm 1, saturating RNE cast of V/2^X).
 *   [Ascend950]    Ascend 950 low-precision format guide (hwcomputing.csdn.net): the HiF8 vs
 *                  MXFP8 numerical analysis on DeepSeek-V4-Flash (per-layer SQNR and zero-rate
 *                  of quantized weights, activations and KV cache).
 *   Dequantization and error statistics follow [MP-FP8] section 8.1 (the worked example
 *   de-scales the code 22 by S = 22400 to 22/22400 ~ 0.000982; a GEMM multiplies its result
 *   back by 1/(S_X S_W)), 8.2 (the saturated 50 -> 448 de-scales to 20) and 7.2 (watch amax,
 *   the fraction of values that underflow to zero, and saturation), and [Ascend950] (SQNR,
 *   zero-rate).
 *
 * Arithmetic: fp64 throughout. A value is rounded to fp32 exactly where the method keeps an
 * fp32 value (the scale factor S and the scaled product x*S). Both roundings are done by a cast
 * of an fp64 result to float: a product of two fp32 (or bf16 and fp32) values is exact in fp64,
 * and for a quotient of two fp32 values fp64 then fp32 rounding equals one correct fp32
 * rounding, because 53 >= 2*24 + 2 (double rounding is innocuous for +,-,*,/ under that bound).
 *
 * Readings where the pages are silent or garbled (each is listed with its reason in the design
 * notes of the repository):
 *   R1 the MX element step divides by 2^X (X = -6 multiplies by 64 in the 5.3 example);
 *   R2 the scaled value is rounded to fp32 before the fp8 rounding (Eq.(2)/(4) bodies are lost);
 *   R3 IEEE signed zero, except that an all-zero MX block writes 0x00 everywhere;
 *   R4 amax = 0 (tensor, group or delayed estimate) gives the base ratio 1; an fp32 overflow of
 *      F8max/amax gives FLT_MAX;
 *   R5 E8M0 byte = X + 127, 0xFF is NaN;
 *   R6 Inf/NaN input is outside the bit-exact contract: it sets the non-finite flag, a NaN
 *      element encodes to an fp8 NaN code, a non-finite amax gives S = 1 (tensor, group) or
 *      E8M0 byte 0xFF (MX block), and a delayed step never pushes a non-finite amax;
 *   R7 delayed: step 0 (after init or reset) is current scaling without the 2^-N margin; later
 *      steps scale with the history as it stood before the step, then append; the update
 *      steps are step % Interval == 0; an empty history estimate counts as amax = 0;
 *   R8 the OCP round-down exponent is floor(log2 amax) - emax (a difference, not a quotient);
 *   R9 de-scaling by a scale factor S divides in fp32: xhat = fl32(decode(q) / S) (the 22/22400
 *      example); an MX element is multiplied by its block's 2^X: xhat = fl32(decode(q) * 2^X),
 *      and an E8M0 byte 0xFF gives NaN;
 *   R10 a BF16 dequantized output is that fp32 value rounded to BF16 to nearest, ties to even;
 *   R11 error statistics over the finite elements of the source x: signal = sum x^2,
 *      noise = sum (x - xhat)^2 (SQNR = 10 log10(signal / noise)), nonzero = #(x != 0),
 *      zeroed = #(x != 0 and xhat == 0) (the zero-rate numerator), saturated = #(elements whose
 *      scaled value exceeded F8max before the saturating cast), nonfinite = #(Inf/NaN in x).
 *      Per-element terms are fp64 operations on exact fp64 copies of x and xhat; the sums run in
 *      index order (any other order differs only by fp64 rounding);
 *   R12 a power-of-two group scale ([MP-FP8 10.4]: the tensors that are re-grouped from 1x128 to
 *      128x1 take integer powers of two as scale factors) is the largest power of two S with
 *      amax * S <= F8max, i.e. S = 2^-X with X = ceil(log2(amax / F8max)) clamped to
 *      [-127, 127] (the exponent rule of the MX round-up recipe applied to the group), and 1 for
 *      amax = 0 or non-finite;
 *   R14 delayed-scaling estimators ([HiF8-train 1.2] names the maximum of the history and, as
 *      other rules, the most recent entry and the mean): max; the newest entry; the mean as the
 *      fp32 sum of the entries from oldest to newest (each addition rounded to fp32) divided by
 *      the count in fp32. An empty history estimates 0 under every rule;
 *   R13 the 1x128 -> 128x1 re-grouping ([MP-FP8 10.5]: read, dequantize, transpose, quantize
 *      again in 128x1 groups, write back) de-scales with R9 and quantizes the transposed fp32
 *      values in 1x128 groups along the rows of the transpose, so the result is stored
 *      transposed: qT [cols][rows], scalesT [cols][ceil(rows/128)].
 *   R15 the amax computation spread over the Interval steps ([HiF8-train], the section that
 *      compares HiF8 with FP8 and MXFP8: the tensor is cut into equal sub-tensors, one measured
 *      per step of the Interval): the flattened tensor is cut into I consecutive pieces
 *      [floor(k n / I), floor((k+1) n / I)); step t >= 1 measures piece (t - 1) mod I; the
 *      maximum of the I piece amaxes of the window t-I+1 .. t is appended on the update step
 *      t % I == 0 (the same schedule as whole-tensor updates), unless a piece of the window
 *      held Inf/NaN. Step 0 is current scaling with the whole amax as always. The reported
 *      amax and the non-finite flag still cover the whole tensor.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#include <float.h>

#define QF8O_E4M3 0
#define QF8O_E5M2 1
#define QF8O_E8M0 2
#define QF8O_E2M1 3

#define QF8O_BF16 0
#define QF8O_FP32 1

#define QF8O_ROUND_DOWN 0
#define QF8O_ROUND_UP 1

/* ---------------------------------------------------------------------------------------------
 * Number formats, from their definitions.
 * [MP-FP8 2.1]: sign, biased exponent, trailing mantissa; exponent field 0 = subnormal with the
 * minimum exponent; [MP-FP8 2.2]: E5M2 follows IEEE (all-ones exponent = Inf/NaN); E4M3 has no
 * Inf and one NaN pattern S.1111.111, so the all-ones exponent also holds finite values up to 448.
 * Bias is 2^(e-1) - 1. E2M1 ([MP-FP8 13.2]: the FP4 element of MXFP4 and NVFP4, values 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6 and their negatives) is the 4-bit code S.EE.M with bias 1 and no Inf/NaN;
 * code 1 is the one subnormal, 0.5.
 * ------------------------------------------------------------------------------------------- */
static int fmt_mbits(int fmt) { return fmt == QF8O_E4M3 ? 3 : fmt == QF8O_E2M1 ? 1 : 2; }
static int fmt_ebits(int fmt) { return fmt == QF8O_E4M3 ? 4 : fmt == QF8O_E2M1 ? 2 : 5; }
static int fmt_bias(int fmt) { return (1 << (fmt_ebits(fmt) - 1)) - 1; }
static int fmt_bits(int fmt) { return 1 + fmt_ebits(fmt) + fmt_mbits(fmt); }

double qf8o_decode(int fmt, unsigned code)
{
    code &= 0xFFu;
    if (fmt == QF8O_E8M0) {                   /* [MP-FP8 13.1]: a power of two, 8 exponent bits */
        if (code == 0xFFu) return NAN;        /* R5 */
        return ldexp(1.0, (int)code - 127);
    }
    int mb = fmt_mbits(fmt), eb = fmt_ebits(fmt), bias = fmt_bias(fmt);
    code &= (1u << fmt_bits(fmt)) - 1u;
    int s = (int)(code >> (eb + mb));
    int e = (int)(code >> mb) & ((1 << eb) - 1);
    int m = (int)code & ((1 << mb) - 1);
    int eall = (1 << eb) - 1;
    double v;
    if (fmt == QF8O_E4M3 && e == eall && m == (1 << mb) - 1) return NAN;
    if (fmt == QF8O_E5M2 && e == eall) {
        if (m != 0) return NAN;
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)                                /* subnormal: 0.m * 2^(1-bias) */
        v = ldexp((double)m, 1 - bias - mb);
    else                                       /* normal: 1.m * 2^(e-bias) */
        v = ldexp((double)((1 << mb) + m), e - bias - mb);
    return s ? -v : v;
}

/* Ascending list of the non-negative finite values. Codes 0, 1, 2, ... decode in increasing
 * order, so the index in the list is the code itself (checked by the test suite). */
static double g_vals[4][128];
static int g_nvals[4] = {0, 0, 0, 0};

static void build_table(int fmt)
{
    if (g_nvals[fmt]) return;
    int n = 0;
    for (unsigned c = 0; c < (1u << (fmt_bits(fmt) - 1)); ++c) {
        double v = qf8o_decode(fmt, c);
        if (!isfinite(v)) break;
        g_vals[fmt][n++] = v;
    }
    g_nvals[fmt] = n;
}

int qf8o_num_finite_nonneg(int fmt) { build_table(fmt); return g_nvals[fmt]; }
double qf8o_max_finite(int fmt) { build_table(fmt); return g_vals[fmt][g_nvals[fmt] - 1]; }

/* sat_rne8(y): nearest fp8 value, ties to the even code, with magnitudes at or above the largest
 * finite value clamped to it ([MP-FP8 4.1] RNE; [MP-FP8 8.1] overflow saturates, it is not
 * skipped; [MXFP8-recipe 4.1] the cast saturates). Sign kept, so -0 and negative values that
 * round to zero give 0x80 (R3). NaN gives the positive NaN code (R6). E2M1 has no NaN: its codes
 * are 4 bits with the sign in bit 3, and NaN gives +6 (outside the compared results, R6). */
unsigned qf8o_encode(int fmt, double y)
{
    build_table(fmt);
    const double *v = g_vals[fmt];
    int n = g_nvals[fmt];
    const unsigned sbit = 1u << (fmt_bits(fmt) - 1);
    if (isnan(y)) return fmt == QF8O_E2M1 ? (unsigned)(n - 1) : 0x7Fu;
    unsigned sign = signbit(y) ? sbit : 0u;
    double a = fabs(y);
    int i;
    if (a >= v[n - 1]) {
        i = n - 1;
    } else {
        int lo = 0, hi = n - 1;                /* invariant: v[lo] <= a < v[hi] */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (v[mid] <= a) lo = mid; else hi = mid;
        }
        i = lo;
        if (v[i] != a) {
            double midpoint = 0.5 * (v[i] + v[i + 1]);   /* exact: short dyadic rationals */
            if (a > midpoint) i = i + 1;
            else if (a == midpoint && (i & 1)) i = i + 1; /* tie: the even code */
        }
    }
    return sign | (unsigned)i;
}

/* sat_rne of the exact quotient num / den (den > 0), rounded once: the nearest value, ties to the
 * even code, saturated at the largest finite value, with num's sign. Every comparison is between
 * num and a value or midpoint of the format times den; the caller passes num and den such that
 * those products are exact in fp64 (then each test decides the exact quotient's side). */
unsigned qf8o_encode_ratio(int fmt, double num, double den)
{
    build_table(fmt);
    const double *v = g_vals[fmt];
    int n = g_nvals[fmt];
    const unsigned sbit = 1u << (fmt_bits(fmt) - 1);
    if (isnan(num) || !(den > 0.0)) return fmt == QF8O_E2M1 ? (unsigned)(n - 1) : 0x7Fu;
    unsigned sign = signbit(num) ? sbit : 0u;
    double a = fabs(num);
    int i;
    if (a >= v[n - 1] * den) {
        i = n - 1;
    } else {
        int lo = 0, hi = n - 1;                /* invariant: v[lo] * den <= a < v[hi] * den */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (v[mid] * den <= a) lo = mid; else hi = mid;
        }
        i = lo;
        if (v[i] * den != a) {
            double t = 0.5 * (v[i] + v[i + 1]) * den;    /* the midpoint, scaled: exact */
            if (a > t) i = i + 1;
            else if (a == t && (i & 1)) i = i + 1;       /* tie: the even code */
        }
    }
    return sign | (unsigned)i;
}

/* ---------------------------------------------------------------------------------------------
 * Inputs. BF16 is the upper half of an fp32 ([MP-FP8 2.2]); widening is exact.
 * ------------------------------------------------------------------------------------------- */
static double load_elem(const void *x, int dtype, int64_t i)
{
    uint32_t u;
    float f;
    if (dtype == QF8O_BF16) u = (uint32_t)((const uint16_t *)x)[i] << 16;
    else u = ((const uint32_t *)x)[i];
    memcpy(&f, &u, 4);
    return (double)f;
}

/* amax = max |x| over a set of elements ([HiF8-train 1.2]: ComputeAmax, e.g. torch.max of |x|;
 * [MXFP8-recipe 4.1]: amax = max |V_i| over the block). NaN anywhere gives NaN. */
typedef struct { double amax; int has_nan; } amax_acc;
static void acc_init(amax_acc *a) { a->amax = 0.0; a->has_nan = 0; }
static void acc_add(amax_acc *a, double v)
{
    if (isnan(v)) { a->has_nan = 1; return; }
    if (fabs(v) > a->amax) a->amax = fabs(v);
}
static double acc_value(const amax_acc *a) { return a->has_nan ? NAN : a->amax; }

double qf8o_amax(const void *x, int dtype, int64_t n)
{
    amax_acc a;
    acc_init(&a);
    for (int64_t i = 0; i < n; ++i) acc_add(&a, load_elem(x, dtype, i));
    return acc_value(&a);
}

/* Eq.(1) of [HiF8-train 1.2] / [MP-FP8 8.1]: S = F8max / amax, kept as fp32 (R4, R6). */
float qf8o_scale_from_amax(int fmt, double amax)
{
    if (!isfinite(amax)) return 1.0f;
    if (amax == 0.0) return 1.0f;
    float s = (float)(qf8o_max_finite(fmt) / amax);
    if (isinf(s)) s = FLT_MAX;
    return s;
}

/* Eq.(2)/(4): q = sat_rne8(fl32(x * S)) (R2). */
unsigned qf8o_cast_one(int fmt, double x, float scale)
{
    float p = (float)(x * (double)scale);
    return qf8o_encode(fmt, (double)p);
}

void qf8o_cast(const void *x, int dtype, int64_t n, int fmt, float scale, uint8_t *q)
{
    for (int64_t i = 0; i < n; ++i) q[i] = (uint8_t)qf8o_cast_one(fmt, load_elem(x, dtype, i), scale);
}

void qf8o_encode_f32(int fmt, const float *y, int64_t n, uint8_t *q)
{
    for (int64_t i = 0; i < n; ++i) q[i] = (uint8_t)qf8o_encode(fmt, (double)y[i]);
}

/* ---------------------------------------------------------------------------------------------
 * Per-tensor current scaling ([HiF8-train 1.2] Eq.(1)-(2)). Outputs q, amax and S.
 * ------------------------------------------------------------------------------------------- */
void qf8o_quantize_per_tensor(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                              uint8_t *q, float *amax_out, float *scale_out, int32_t *nonfinite)
{
    int64_t n = rows * cols;
    double amax = qf8o_amax(x, dtype, n);
    float s = qf8o_scale_from_amax(fmt, amax);
    qf8o_cast(x, dtype, n, fmt, s, q);
    if (amax_out) *amax_out = (float)amax;
    if (scale_out) *scale_out = s;
    if (nonfinite) *nonfinite = isfinite(amax) ? 0 : 1;
}

/* ---------------------------------------------------------------------------------------------
 * Per-tensor delayed scaling ([HiF8-train 1.2] Eq.(3)-(4); [MP-FP8 8.2]).
 * A fixed-capacity FIFO of past amax values; the estimate is its maximum; the true amax is
 * appended every Interval steps and the oldest entry drops out when the buffer is full.
 * S = F8max/estimate * 2^-N_guard. Step 0 (or the first step after a reset) has no history and
 * runs current scaling once ([HiF8-train 5.2]).
 * ------------------------------------------------------------------------------------------- */
#define QF8O_MAX_HIST 4096
typedef struct {
    int32_t hist_len, interval, n_guard, fmt;
    int32_t count, head;        /* head = slot of the oldest entry */
    int64_t step;
    int32_t estimator;          /* R14: 0 max, 1 most recent, 2 mean */
    int32_t split;              /* R15: amax measured on one of Interval sub-tensors per step */
    int32_t window_bad;         /* a sub-tensor of the current window held Inf/NaN */
    double window;              /* maximum of the sub-tensor amaxes measured in the window */
    float hist[QF8O_MAX_HIST];
} qf8o_delayed;

size_t qf8o_delayed_sizeof(void) { return sizeof(qf8o_delayed); }

int qf8o_delayed_init(qf8o_delayed *st, int hist_len, int interval, int n_guard, int fmt)
{
    if (hist_len < 1 || hist_len > QF8O_MAX_HIST || interval < 1 || n_guard < 0) return -1;
    memset(st, 0, sizeof(*st));
    st->hist_len = hist_len;
    st->interval = interval;
    st->n_guard = n_guard;
    st->fmt = fmt;
    return 0;
}

void qf8o_delayed_reset(qf8o_delayed *st)
{
    st->count = 0;
    st->head = 0;
    st->step = 0;
    st->window = 0.0;
    st->window_bad = 0;
    memset(st->hist, 0, sizeof(st->hist));
}

static void delayed_push(qf8o_delayed *st, float v)
{
    if (st->count < st->hist_len) {
        st->hist[(st->head + st->count) % st->hist_len] = v;
        st->count++;
    } else {
        st->hist[st->head] = v;                        /* overwrite the oldest */
        st->head = (st->head + 1) % st->hist_len;
    }
}

/* The amax estimate from the history ([HiF8-train 1.2]: the maximum of the buffer, or another
 * rule such as the most recent entry or the mean; R14). */
float qf8o_delayed_estimate(const qf8o_delayed *st)
{
    if (st->count == 0) return 0.0f;                   /* R7: empty history counts as 0 */
    if (st->estimator == 1)                            /* the newest entry */
        return st->hist[(st->head + st->count - 1) % st->hist_len];
    if (st->estimator == 2) {                          /* fp32 sum, oldest to newest, / count */
        float sum = 0.0f;
        for (int i = 0; i < st->count; ++i) sum = sum + st->hist[(st->head + i) % st->hist_len];
        return sum / (float)st->count;
    }
    float e = 0.0f;
    for (int i = 0; i < st->count; ++i)
        if (st->hist[(st->head + i) % st->hist_len] > e) e = st->hist[(st->head + i) % st->hist_len];
    return e;
}

int qf8o_delayed_set_estimator(qf8o_delayed *st, int estimator)
{
    if (estimator < 0 || estimator > 2) return -1;
    st->estimator = estimator;
    return 0;
}

int qf8o_delayed_set_split(qf8o_delayed *st, int split)
{
    if (split != 0 && split != 1) return -1;
    st->split = split;
    return 0;
}

/* R15: the sub-tensor a split-mode step t >= 1 measures. The flattened tensor of n elements is cut
 * into Interval near-equal consecutive pieces, piece k = [floor(k n / I), floor((k+1) n / I)),
 * and step t measures piece (t - 1) mod I, so the window of steps t-I+1 .. t that ends on an
 * update step (t % I == 0) has measured every piece once (R15). */
void qf8o_delayed_piece(int64_t step, int interval, int64_t n, int64_t *lo, int64_t *hi)
{
    int64_t k = (step - 1) % interval;
    *lo = (int64_t)(((__int128)k * n) / interval);
    *hi = (int64_t)(((__int128)(k + 1) * n) / interval);
}

/* The scale a step uses, from the state before the step. */
float qf8o_delayed_scale(const qf8o_delayed *st)
{
    float base = qf8o_scale_from_amax(st->fmt, (double)qf8o_delayed_estimate(st));
    return (float)((double)base * ldexp(1.0, -st->n_guard));
}

void qf8o_delayed_step(qf8o_delayed *st, const void *x, int dtype, int64_t rows, int64_t cols,
                       uint8_t *q, float *scale_used, float *amax_out, int32_t *nonfinite)
{
    int64_t n = rows * cols;
    double amax = qf8o_amax(x, dtype, n);
    float s;
    int update;
    if (st->step == 0) {                               /* current scaling, no margin (R7) */
        s = qf8o_scale_from_amax(st->fmt, amax);
        update = 1;
    } else {                                           /* scale from the history, then maybe append */
        s = qf8o_delayed_scale(st);
        update = (st->step % st->interval) == 0;
    }
    qf8o_cast(x, dtype, n, st->fmt, s, q);
    if (st->split && st->step > 0) {                   /* R15: fold this step's piece into the window */
        int64_t lo, hi;
        qf8o_delayed_piece(st->step, st->interval, n, &lo, &hi);
        size_t esz = dtype == QF8O_BF16 ? 2 : 4;
        double a = qf8o_amax((const char *)x + (size_t)lo * esz, dtype, hi - lo);
        if (!isfinite(a)) st->window_bad = 1;
        else if (a > st->window) st->window = a;
        if (update) {                                  /* the window ends: append its maximum */
            if (!st->window_bad) delayed_push(st, (float)st->window);
            st->window = 0.0;
            st->window_bad = 0;
        }
    } else if (update && isfinite(amax)) {
        delayed_push(st, (float)amax);
    }
    st->step++;
    if (scale_used) *scale_used = s;
    if (amax_out) *amax_out = (float)amax;
    if (nonfinite) *nonfinite = isfinite(amax) ? 0 : 1;
}

void qf8o_delayed_get(const qf8o_delayed *st, float *hist_oldest_first, int32_t *count, int64_t *step)
{
    for (int i = 0; i < st->count; ++i) hist_oldest_first[i] = st->hist[(st->head + i) % st->hist_len];
    *count = st->count;
    *step = st->step;
}

/* ---------------------------------------------------------------------------------------------
 * Fine-grained groups ([MP-FP8 10.2]; online, current-scaled per group [MP-FP8 10.3]):
 * rule Eq.(1)-(2) applied to every br x bc group on its own. Groups at the right and bottom
 * edges may be partial. Scales and amax are [ceil(rows/br)][ceil(cols/bc)] fp32.
 * ------------------------------------------------------------------------------------------- */
void qf8o_quantize_block(const void *x, int dtype, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                         int fmt, uint8_t *q, float *scales, float *amax_out, int32_t *nonfinite)
{
    int64_t gr = (rows + br - 1) / br, gc = (cols + bc - 1) / bc;
    int bad = 0;
    for (int64_t bi = 0; bi < gr; ++bi) {
        for (int64_t bj = 0; bj < gc; ++bj) {
            int64_t r0 = bi * br, r1 = r0 + br < rows ? r0 + br : rows;
            int64_t c0 = bj * bc, c1 = c0 + bc < cols ? c0 + bc : cols;
            amax_acc a;
            acc_init(&a);
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) acc_add(&a, load_elem(x, dtype, r * cols + c));
            double amax = acc_value(&a);
            float s = qf8o_scale_from_amax(fmt, amax);
            if (!isfinite(amax)) bad = 1;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c)
                    q[r * cols + c] = (uint8_t)qf8o_cast_one(fmt, load_elem(x, dtype, r * cols + c), s);
            if (scales) scales[bi * gc + bj] = s;
            if (amax_out) amax_out[bi * gc + bj] = (float)amax;
        }
    }
    if (nonfinite) *nonfinite = bad;
}

/* ---------------------------------------------------------------------------------------------
 * MX blocks of 32 with an E8M0 shared scale 2^X ([MP-FP8 13.1]; [MXFP8-recipe 4.1]).
 * emax is the exponent of the largest normal of the element format (E4M3: 8, E5M2: 15) and
 * destmax its largest finite value.
 * ------------------------------------------------------------------------------------------- */
int qf8o_emax(int fmt)
{
    int e;
    frexp(qf8o_max_finite(fmt), &e);
    return e - 1;
}

/* Returns X (before the +127 bias); amax must be finite and >= 0. */
int qf8o_mx_exponent(int fmt, int rnd, double amax)
{
    if (amax == 0.0) return -127;                        /* [MXFP8-recipe 4.1] */
    int e;
    frexp(amax, &e);                                     /* amax = m * 2^e, m in [0.5, 1) */
    int floor_log2 = e - 1;
    int X;
    if (rnd == QF8O_ROUND_DOWN) {
        X = floor_log2 - qf8o_emax(fmt);                 /* OCP: floor(log2 amax) - emax (R8) */
    } else {
        /* Algorithm 1: the exponent of amax/destmax rounded toward +inf, i.e. the smallest
         * integer X with amax / 2^X <= destmax. */
        double destmax = qf8o_max_finite(fmt);
        X = floor_log2 - qf8o_emax(fmt) - 1;
        while (amax > ldexp(destmax, X)) X++;
    }
    if (X < -127) X = -127;                              /* saturate to the E8M0 bounds */
    if (X > 127) X = 127;
    return X;
}

static void mx_group(const void *x, int dtype, int fmt, int rnd, const int64_t *idx,
                     uint8_t *qout, int64_t qstride, uint8_t *sbyte, int *bad)
{
    amax_acc a;
    acc_init(&a);
    for (int k = 0; k < 32; ++k) acc_add(&a, load_elem(x, dtype, idx[k]));
    double amax = acc_value(&a);
    if (!isfinite(amax)) {                               /* R6: outside the bit-exact contract */
        *bad = 1;
        *sbyte = 0xFF;
        for (int k = 0; k < 32; ++k) qout[k * qstride] = (uint8_t)qf8o_encode(fmt, load_elem(x, dtype, idx[k]));
        return;
    }
    int X = qf8o_mx_exponent(fmt, rnd, amax);
    *sbyte = (uint8_t)(X + 127);
    for (int k = 0; k < 32; ++k) {
        if (amax == 0.0) { qout[k * qstride] = 0x00; continue; }   /* zero block: every byte 0 */
        double v = load_elem(x, dtype, idx[k]) * ldexp(1.0, -X);  /* V_i / 2^X, exact (R1) */
        qout[k * qstride] = (uint8_t)qf8o_encode(fmt, v);
    }
}

/* Rowwise: groups of 32 along a row, q_row [rows][cols], s_row [rows][cols/32].
 * Columnwise: groups of 32 down a column, stored transposed: q_colT [cols][rows],
 * s_colT [cols][rows/32]. Either pair may be NULL. Both come from the same high-precision
 * input ([MP-FP8 13.1]: a tensor and its transpose are each quantized from the original). */
void qf8o_quantize_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int rnd,
                      uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite)
{
    int bad = 0;
    int64_t idx[32];
    if (q_row) {
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t g = 0; g < cols / 32; ++g) {
                for (int k = 0; k < 32; ++k) idx[k] = r * cols + g * 32 + k;
                mx_group(x, dtype, fmt, rnd, idx, q_row + r * cols + g * 32, 1, s_row + r * (cols / 32) + g, &bad);
            }
    }
    if (q_colT) {
        for (int64_t c = 0; c < cols; ++c)
            for (int64_t g = 0; g < rows / 32; ++g) {
                for (int k = 0; k < 32; ++k) idx[k] = (g * 32 + k) * cols + c;
                mx_group(x, dtype, fmt, rnd, idx, q_colT + c * rows + g * 32, 1, s_colT + c * (rows / 32) + g, &bad);
            }
    }
    if (nonfinite) *nonfinite = bad;
}

/* ---------------------------------------------------------------------------------------------
 * Dequantization (R9, R10) and quantization error statistics (R11).
 * ------------------------------------------------------------------------------------------- */

/* xhat = fl32(decode(q) / S): decode(q) and S are both fp32 values, so the fp64 quotient
 * rounded to fp32 is the correctly rounded fp32 quotient (53 >= 2*24 + 2). */
float qf8o_dequant_one(int fmt, unsigned code, float scale)
{
    return (float)(qf8o_decode(fmt, code) / (double)scale);
}

/* xhat = fl32(decode(q) * 2^X) with X = byte - 127; exact unless it overflows fp32. */
float qf8o_dequant_mx_one(int fmt, unsigned code, unsigned sbyte)
{
    if ((sbyte & 0xFFu) == 0xFFu) return NAN;
    return (float)ldexp(qf8o_decode(fmt, code), (int)(sbyte & 0xFFu) - 127);
}

void qf8o_dequant_scaled(const uint8_t *q, int64_t n, int fmt, float scale, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = qf8o_dequant_one(fmt, q[i], scale);
}

/* Each br x bc group divides by its own S_g; scales is [ceil(rows/br)][ceil(cols/bc)]. */
void qf8o_dequant_block(const uint8_t *q, int64_t rows, int64_t cols, int64_t br, int64_t bc, int fmt,
                        const float *scales, float *out)
{
    int64_t gc = (cols + bc - 1) / bc;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = qf8o_dequant_one(fmt, q[r * cols + c], scales[(r / br) * gc + c / bc]);
}

/* q [rows][cols] with blocks of 32 along each row and s [rows][cols/32] (a rowwise result, or
 * a columnwise result in its transposed layout). */
void qf8o_dequant_mx(const uint8_t *q, const uint8_t *sb, int64_t rows, int64_t cols, int fmt, float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = qf8o_dequant_mx_one(fmt, q[r * cols + c], sb[r * (cols / 32) + c / 32]);
}

/* fp32 -> BF16, round to nearest, ties to even (R10). The BF16 values are exactly the fp32
 * values whose low 16 bits are zero, with the same exponent range, and for finite values of one
 * sign the bit pattern grows with the magnitude. So the nearest BF16 value is the pattern
 * rounded to a multiple of 2^16: up when the dropped half exceeds 0x8000, down when below, and
 * at exactly 0x8000 (a tie) to the even result. Rounding up past the largest finite value gives
 * the Inf pattern, as IEEE overflow does. NaN stays NaN (quiet, sign kept). */
uint16_t qf8o_f32_to_bf16_one(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16, lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
    return (uint16_t)hi;
}

void qf8o_f32_to_bf16(const float *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = qf8o_f32_to_bf16_one(in[i]);
}

/* Statistics accumulator (R11). sums[0] = signal, sums[1] = noise; counts[0..4] = count,
 * nonzero, zeroed, saturated, nonfinite. */
static void stats_add(double *sums, int64_t *counts, double x, float xhat, int saturated)
{
    if (!isfinite(x)) { counts[4]++; return; }
    counts[0]++;
    sums[0] += x * x;
    double d = x - (double)xhat;
    sums[1] += d * d;
    if (x != 0.0) {
        counts[1]++;
        if (xhat == 0.0f) counts[2]++;
    }
    if (saturated) counts[3]++;
}

static void stats_clear(double *sums, int64_t *counts)
{
    sums[0] = sums[1] = 0.0;
    for (int k = 0; k < 5; ++k) counts[k] = 0;
}

/* A scale-factor element saturates when |fl32(x * S)| > F8max (the cast clips it). */
static int scaled_saturates(int fmt, double x, float scale)
{
    float p = (float)(x * (double)scale);
    return fabs((double)p) > qf8o_max_finite(fmt);
}

void qf8o_stats_scaled(const void *x, int dtype, const uint8_t *q, int64_t n, int fmt, float scale,
                       double *sums, int64_t *counts)
{
    stats_clear(sums, counts);
    for (int64_t i = 0; i < n; ++i) {
        double v = load_elem(x, dtype, i);
        stats_add(sums, counts, v, qf8o_dequant_one(fmt, q[i], scale), isfinite(v) && scaled_saturates(fmt, v, scale));
    }
}

void qf8o_stats_block(const void *x, int dtype, const uint8_t *q, int64_t rows, int64_t cols, int64_t br,
                      int64_t bc, int fmt, const float *scales, double *sums, int64_t *counts)
{
    int64_t gc = (cols + bc - 1) / bc;
    stats_clear(sums, counts);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t i = r * cols + c;
            float sg = scales[(r / br) * gc + c / bc];
            double v = load_elem(x, dtype, i);
            stats_add(sums, counts, v, qf8o_dequant_one(fmt, q[i], sg), isfinite(v) && scaled_saturates(fmt, v, sg));
        }
}

/* An MX element saturates when |x| / 2^X > F8max, i.e. |x| > F8max * 2^X (exact in fp64). */
void qf8o_stats_mx(const void *x, int dtype, const uint8_t *q, const uint8_t *sb, int64_t rows, int64_t cols,
                   int fmt, double *sums, int64_t *counts)
{
    stats_clear(sums, counts);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t i = r * cols + c;
            unsigned b = sb[r * (cols / 32) + c / 32];
            double v = load_elem(x, dtype, i);
            int sat = isfinite(v) && b != 0xFFu && fabs(v) > ldexp(qf8o_max_finite(fmt), (int)b - 127);
            stats_add(sums, counts, v, qf8o_dequant_mx_one(fmt, q[i], b), sat);
        }
}

/* ---------------------------------------------------------------------------------------------
 * Power-of-two group scales (R12) and the 1x128 -> 128x1 re-grouping (R13).
 * ------------------------------------------------------------------------------------------- */
float qf8o_scale_pow2(int fmt, double amax)
{
    if (!isfinite(amax) || amax == 0.0) return 1.0f;
    int X = qf8o_mx_exponent(fmt, QF8O_ROUND_UP, amax);   /* smallest X with amax / 2^X <= F8max */
    return (float)ldexp(1.0, -X);
}

/* quantize_block with a choice of scale rule: pow2 = 0 gives Eq.(1), pow2 = 1 gives R12. */
void qf8o_quantize_block_ex(const void *x, int dtype, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                            int fmt, int pow2, uint8_t *q, float *scales, float *amax_out, int32_t *nonfinite)
{
    int64_t gr = (rows + br - 1) / br, gc = (cols + bc - 1) / bc;
    int bad = 0;
    for (int64_t bi = 0; bi < gr; ++bi) {
        for (int64_t bj = 0; bj < gc; ++bj) {
            int64_t r0 = bi * br, r1 = r0 + br < rows ? r0 + br : rows;
            int64_t c0 = bj * bc, c1 = c0 + bc < cols ? c0 + bc : cols;
            amax_acc a;
            acc_init(&a);
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) acc_add(&a, load_elem(x, dtype, r * cols + c));
            double amax = acc_value(&a);
            float s = pow2 ? qf8o_scale_pow2(fmt, amax) : qf8o_scale_from_amax(fmt, amax);
            if (!isfinite(amax)) bad = 1;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c)
                    q[r * cols + c] = (uint8_t)qf8o_cast_one(fmt, load_elem(x, dtype, r * cols + c), s);
            if (scales) scales[bi * gc + bj] = s;
            if (amax_out) amax_out[bi * gc + bj] = (float)amax;
        }
    }
    if (nonfinite) *nonfinite = bad;
}

/* R13: q [rows][cols] in 1x128 groups with scales [rows][ceil(cols/128)] (format fmt_in) ->
 * qT [cols][rows] in 1x128 groups of the transpose (128x1 groups of the original) with scalesT
 * [cols][ceil(rows/128)] (format fmt_out, scale rule pow2_out). tmp: rows*cols floats. */
void qf8o_requant_1x128_to_128x1(const uint8_t *q, const float *scales, int64_t rows, int64_t cols,
                                 int fmt_in, int fmt_out, int pow2_out, float *tmp, uint8_t *qT,
                                 float *scalesT, int32_t *nonfinite)
{
    int64_t gc = (cols + 127) / 128;
    for (int64_t c = 0; c < cols; ++c)                    /* de-scale and transpose */
        for (int64_t r = 0; r < rows; ++r)
            tmp[c * rows + r] = qf8o_dequant_one(fmt_in, q[r * cols + c], scales[r * gc + c / 128]);
    qf8o_quantize_block_ex(tmp, QF8O_FP32, cols, rows, 1, 128, fmt_out, pow2_out, qT, scalesT, NULL, nonfinite);
}

/* ---------------------------------------------------------------------------------------------
 * FP4 ([MP-FP8 13.1-13.2]; [Ascend950 2.4] MXFP4 = 32 FP4 values + one shared scale).
 * R16 MXFP4: the MX rule of qf8o_quantize_mx with E2M1 elements (emax = 2, largest value 6): X
 *     = floor(log2 amax) - 2 (round-down) or the smallest X with amax / 2^X <= 6 (round-up),
 *     clamped to [-127, 127]; amax = 0 gives X = -127 and zero codes; a block with Inf/NaN gets
 *     scale byte 0xFF. Codes are stored two per byte, element 2j in the low nibble of byte j
 *     and element 2j+1 in the high nibble (the pages do not fix the order; this is the order
 *     of the OCP MX format).
 * R17 NVFP4: blocks of 16 along a row, one E4M3 block scale each and one fp32 tensor scale.
 *     The pages fix the block scale as amax_b / 6 stored in E4M3, divide each element by the
 *     stored block scale and round it to E2M1, and add the fp32 tensor scale because E4M3's range
 *     is too small, without its formula. Reading: the tensor scale S_t lifts every block scale
 *     into E4M3's range so that the largest lands on 448, and the stored code holds the block
 *     scale in those lifted units:
 *       S_t = fl32(448 * 6 / A) with A the tensor amax (1 for A = 0 or non-finite, FLT_MAX on
 *             overflow, as Eq.(1));
 *       e_b = sat_rne(E4M3, amax_b * S_t / 6)          (one rounding of the exact quotient);
 *       code = sat_rne(E2M1, x * S_t / decode(e_b))    (x divided by the real block scale
 *             decode(e_b) / S_t, one rounding of the exact quotient);
 *     a block whose e_b decodes to 0 (negligible against the tensor; it de-scales to 0 whatever
 *     its codes) encodes its elements as zeros of their signs. The pages' example (amax 5.3,
 *     S_t = 1): 5.3/6 = 0.883 -> E4M3 0.875, 5.3 / 0.875 = 6.06 -> 6, de-scaled 5.25. A block
 *     with Inf/NaN gets the E4M3 NaN code 0x7F and sets nonfinite.
 *     Both quotients are rounded from their exact values: qf8o_encode_ratio compares the
 *     numerator with the format's values and midpoints times the denominator, products that are
 *     exact in fp64 (the numerator x * S_t has at most 48 significant bits, the denominator at
 *     most 24, the values and midpoints at most 5).
 * ------------------------------------------------------------------------------------------- */

/* Pairs of 4-bit codes into bytes: out[j] = c[2j] | c[2j+1] << 4 (n even). */
void qf8o_pack_fp4(const uint8_t *codes, int64_t n, uint8_t *out)
{
    for (int64_t j = 0; j < n / 2; ++j)
        out[j] = (uint8_t)((codes[2 * j] & 0xFu) | ((codes[2 * j + 1] & 0xFu) << 4));
}

void qf8o_unpack_fp4(const uint8_t *packed, int64_t n, uint8_t *codes)
{
    for (int64_t j = 0; j < n / 2; ++j) {
        codes[2 * j] = packed[j] & 0xFu;
        codes[2 * j + 1] = packed[j] >> 4;
    }
}

/* R17: the tensor scale from the tensor amax. */
float qf8o_nvfp4_tensor_scale(double amax)
{
    if (!isfinite(amax) || amax == 0.0) return 1.0f;
    float s = (float)(448.0 * 6.0 / amax);
    if (isinf(s)) s = FLT_MAX;
    return s;
}

/* R17, for one block of 16 given its amax: the E4M3 block-scale code, amax_b * S_t / 6 rounded
 * once. */
unsigned qf8o_nvfp4_block(double amax_b, float s_t)
{
    return qf8o_encode_ratio(QF8O_E4M3, amax_b * (double)s_t, 6.0);
}

/* R17, one element of a block with block-scale code e: x * S_t / decode(e) rounded once to E2M1,
 * or a zero of x's sign when decode(e) is 0. */
unsigned qf8o_nvfp4_element(double x, float s_t, unsigned e)
{
    double dec = qf8o_decode(QF8O_E4M3, e);
    if (dec == 0.0) return signbit(x) ? 0x8u : 0x0u;
    return qf8o_encode_ratio(QF8O_E2M1, x * (double)s_t, dec);
}

/* x [rows][cols] (cols % 16 == 0) -> codes [rows][cols] (one 4-bit code per byte, unpacked),
 * s_blk [rows][cols/16] E4M3 codes, the tensor scale S_t and amax, nonfinite. amax_in (nullable):
 * a tensor amax given by the caller (its magnitude is used) in place of the measured one, as
 * when it comes from an amax history. */
void qf8o_quantize_nvfp4(const void *x, int dtype, int64_t rows, int64_t cols, const float *amax_in, uint8_t *codes,
                         uint8_t *s_blk, float *tensor_scale, float *amax_out, int32_t *nonfinite)
{
    double A = amax_in ? fabs((double)*amax_in) : qf8o_amax(x, dtype, rows * cols);
    float s_t = qf8o_nvfp4_tensor_scale(A);
    int bad = !isfinite(A);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / 16; ++g) {
            int64_t base = r * cols + g * 16;
            double a = qf8o_amax((const char *)x + (size_t)base * (dtype == QF8O_BF16 ? 2 : 4), dtype, 16);
            if (!isfinite(a)) {
                bad = 1;
                s_blk[r * (cols / 16) + g] = 0x7F;       /* the E4M3 NaN code */
                for (int k = 0; k < 16; ++k) codes[base + k] = 0;
                continue;
            }
            unsigned e = qf8o_nvfp4_block(a, s_t);
            s_blk[r * (cols / 16) + g] = (uint8_t)e;
            for (int k = 0; k < 16; ++k)
                codes[base + k] = (uint8_t)qf8o_nvfp4_element(load_elem(x, dtype, base + k), s_t, e);
        }
    if (tensor_scale) *tensor_scale = s_t;
    if (amax_out) *amax_out = (float)A;
    if (nonfinite) *nonfinite = bad;
}

/* De-scaling (R9 applied to FP4): MXFP4 decode(c) * 2^X, exact, NaN for byte 0xFF; NVFP4
 * fl32(decode(c) * decode(e_b) / S_t), where the product of the two short significands is exact. */
float qf8o_dequant_mxfp4_one(unsigned code, unsigned sbyte)
{
    if (sbyte == 0xFFu) return NAN;
    return (float)ldexp(qf8o_decode(QF8O_E2M1, code), (int)sbyte - 127);
}

float qf8o_dequant_nvfp4_one(unsigned code, unsigned e_code, float s_t)
{
    double p = qf8o_decode(QF8O_E2M1, code) * qf8o_decode(QF8O_E4M3, e_code);
    return (float)(p / (double)s_t);
}

void qf8o_dequant_nvfp4(const uint8_t *codes, const uint8_t *s_blk, int64_t rows, int64_t cols, float s_t, float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = qf8o_dequant_nvfp4_one(codes[r * cols + c], s_blk[r * (cols / 16) + c / 16], s_t);
}

void qf8o_dequant_mxfp4(const uint8_t *codes, const uint8_t *sb, int64_t rows, int64_t cols, float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = qf8o_dequant_mxfp4_one(codes[r * cols + c], sb[r * (cols / 32) + c / 32]);
}
