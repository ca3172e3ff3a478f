// qf8_device.h -- device-side building blocks for the gfx950 FP8 quantization kernels.
//
// Pages (title, section):
//   [MP-FP8]       "混合精度与 FP8 训练" (hs-black.github.io, posts/scaling-mixed-precision)
//   [MXFP8-recipe] "NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" (51cto.com)
//
// Number handling
//   * amax is taken as an integer maximum over |x| bit patterns (sign bit cleared). For
//     non-negative IEEE values the bit pattern orders like the value, so the maximum is exact
//     and independent of reduction order; Inf and NaN patterns sort above every finite value,
//     so a non-finite block is recognised from its amax alone.
//   * The fp8 encoders are the gfx950 conversion instructions, used only on operands inside
//     +-F8max: there they round to nearest even exactly ([MP-FP8 4.1]); outside they produce
//     NaN/Inf instead of saturating, so every caller clamps first ([MP-FP8 8.1] saturation;
//     [MXFP8-recipe 4.1] saturating cast).
//       - v_cvt_pk_{fp8,bf8}_f32: two fp32 values -> two E4M3/E5M2 bytes.
//       - v_cvt_scalef32_pk_{fp8,bf8}_{bf16,f32}: two values divided by 2^E, where E is the
//         exponent field of the fp32 scale operand minus 127 -- exactly V/2^X of an MX block
//         when the operand's bits are (X + 127) << 23 (X = -127 gives the bit pattern 0).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qf8 {

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

enum { kE4M3 = 0, kE5M2 = 1 };
enum { kRoundDown = 0, kRoundUp = 1 };

// Element formats ([MP-FP8 2.2]): largest finite value, and emax = exponent of that value.
template <int FMT> struct F8;
template <> struct F8<kE4M3> {
    static constexpr float kMax = 448.0f;         // 1.75 * 2^8
    static constexpr int kEmax = 8;
};
template <> struct F8<kE5M2> {
    static constexpr float kMax = 57344.0f;       // 1.75 * 2^15
    static constexpr int kEmax = 15;
};

// ---- bit helpers ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2u16, a),
                                                                  __builtin_bit_cast(v2u16, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(v2u16, a),
                                                                  __builtin_bit_cast(v2u16, b)));
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
// take the bits of `v` where `mask` is set, else the bits of `other`
__device__ __forceinline__ uint32_t bit_select(uint32_t mask, uint32_t v, uint32_t other) {
    return (v & mask) | (other & ~mask);
}

// ---- cross-lane maxima (all lanes of the group receive the result; every lane of the wave
// must be active, which the kernels guarantee by predicating only loads and stores) -------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// groups of 4 lanes: quad_perm [1,0,3,2] then [2,3,0,1]
__device__ __forceinline__ uint32_t max_quad(uint32_t v) {
    v = umax(v, dpp_mov<0xB1>(v));
    v = umax(v, dpp_mov<0x4E>(v));
    return v;
}
// groups of 8 lanes: quads, then each lane with its mirror in the half row
__device__ __forceinline__ uint32_t max_oct(uint32_t v) {
    v = max_quad(v);
    v = umax(v, dpp_mov<0x141>(v));                // row_half_mirror
    return v;
}
// groups of 16 lanes (one DPP row): quads, then rotate the row by 4 and by 8
__device__ __forceinline__ uint32_t max_row16(uint32_t v) {
    v = max_quad(v);
    v = umax(v, dpp_mov<0x124>(v));                // row_ror:4
    v = umax(v, dpp_mov<0x128>(v));                // row_ror:8
    return v;
}
__device__ __forceinline__ uint32_t max_wave(uint32_t v) {
    v = max_row16(v);
    v = umax(v, (uint32_t)__shfl_xor((int)v, 16));
    v = umax(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// ---- workgroup-wide maxima ------------------------------------------------------------------
// Maximum over the workgroup of NT threads, broadcast to every thread. red: NT/64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_max_bcast(uint32_t v, uint32_t *red) {
    constexpr int W = NT / 64;
    v = max_wave(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) m = umax(m, red[w]);
    __syncthreads();
    return m;
}

// Maximum of n u32 values by a workgroup of NT threads (each thread's share; combine with
// block_max_bcast). 16 independent loads per thread in flight per round.
template <int NT>
__device__ __forceinline__ uint32_t fold_max(const uint32_t *__restrict__ p, int n) {
    uint32_t m = 0;
    for (int base = 0; base < n; base += 16 * NT) {
        uint32_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = base + k * NT + (int)threadIdx.x;
            v[k] = i < n ? p[i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) m = umax(m, v[k]);
    }
    return m;
}

// ---- fp8 conversions -----------------------------------------------------------------------
// Two fp32 values inside +-F8max -> two bytes in half HI of `old` (other half kept).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2_f32(float a, float b, uint32_t old) {
    if constexpr (FMT == kE4M3) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}
// Two BF16 values (one dword, low half first) divided by 2^X, with scale2x = bits (X+127)<<23.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2_bf16_div2x(uint32_t pair, float scale2x, uint32_t old) {
    v2bf16 v = __builtin_bit_cast(v2bf16, pair);
    v2i16 o = __builtin_bit_cast(v2i16, old);
    v2i16 r;
    if constexpr (FMT == kE4M3) r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, v, scale2x, HI);
    else r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(o, v, scale2x, HI);
    return __builtin_bit_cast(uint32_t, r);
}
// Two FP32 values divided by 2^X.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2_f32_div2x(float a, float b, float scale2x, uint32_t old) {
    v2i16 o = __builtin_bit_cast(v2i16, old);
    v2i16 r;
    if constexpr (FMT == kE4M3) r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale2x, HI);
    else r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, a, b, scale2x, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// sat_rne8(fl32(x * s)) for four fp32 inputs -> four bytes (x[0] in the lowest byte).
template <int FMT>
__device__ __forceinline__ uint32_t cast4(float x0, float x1, float x2, float x3, float s) {
    constexpr float M = F8<FMT>::kMax;
    float y0 = __builtin_amdgcn_fmed3f(x0 * s, -M, M);
    float y1 = __builtin_amdgcn_fmed3f(x1 * s, -M, M);
    float y2 = __builtin_amdgcn_fmed3f(x2 * s, -M, M);
    float y3 = __builtin_amdgcn_fmed3f(x3 * s, -M, M);
    return cvt2_f32<FMT, true>(y2, y3, cvt2_f32<FMT, false>(y0, y1, 0u));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 BF16 (16 bytes) -> 8 fp8 bytes
template <int FMT>
__device__ __forceinline__ uint2 cast8_bf16(uint4 v, float s) {
    return make_uint2(cast4<FMT>(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y), s),
                      cast4<FMT>(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w), s));
}
// 4 FP32 (16 bytes) -> 4 fp8 bytes
template <int FMT>
__device__ __forceinline__ uint32_t cast4_f32(uint4 v, float s) {
    return cast4<FMT>(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w), s);
}
// one element, for ragged tails
template <int FMT>
__device__ __forceinline__ uint32_t cast1(float x, float s) {
    constexpr float M = F8<FMT>::kMax;
    return cvt2_f32<FMT, false>(__builtin_amdgcn_fmed3f(x * s, -M, M), 0.0f, 0u) & 0xFFu;
}

// ---- scales ----------------------------------------------------------------------------------
// Eq.(1): S = fl32(F8max / amax) from the fp32 bit pattern of amax; 1 for amax = 0 or
// non-finite, FLT_MAX when the quotient overflows. The division is IEEE (correctly rounded).
template <int FMT>
__device__ __forceinline__ float scale_from_amax_bits(uint32_t abits) {
    if (abits == 0u || abits >= 0x7F800000u) return 1.0f;
    float s = F8<FMT>::kMax / __uint_as_float(abits);
    return s > 3.40282346638528859812e+38f ? 3.40282346638528859812e+38f : s;
}

// MX E8M0 byte (= X + 127) from the |amax| bit pattern. For a finite amax = 1.f * 2^E:
// round-down X = E - emax; round-up adds 1 when 1.f > 1.75, which is ceil(log2(amax/F8max))
// because F8max = 1.75 * 2^emax. With e = the biased exponent field, round-up's "e + (1.f > 1.75)"
// is one carry: adding 0x1F (BF16) or 0x1FFFFF (FP32) to the bits carries into the exponent
// exactly when the 7 (23) mantissa bits exceed those of 1.75. X is clamped below at -127
// (subnormal or zero amax) by a saturating subtraction; a non-finite amax gives 0xFF.
template <int FMT, int RND>
__device__ __forceinline__ uint32_t mx_byte_bf16(uint32_t a) {
    const uint32_t e = (RND == kRoundUp ? a + 0x1Fu : a) >> 7;
    const uint32_t b = __builtin_elementwise_sub_sat(e, (uint32_t)F8<FMT>::kEmax);
    return a >= 0x7F80u ? 255u : b;
}
template <int FMT, int RND>
__device__ __forceinline__ uint32_t mx_byte_f32(uint32_t a) {
    const uint32_t e = (RND == kRoundUp ? a + 0x1FFFFFu : a) >> 23;
    const uint32_t b = __builtin_elementwise_sub_sat(e, (uint32_t)F8<FMT>::kEmax);
    return a >= 0x7F800000u ? 255u : b;
}
// Power-of-two group scale from the |amax| fp32 bit pattern: the largest power of two S with
// amax * S <= F8max, i.e. S = 2^-X with X the round-up MX exponent of the group (byte = X + 127
// is at most 247 for finite amax, so S = 2^(127 - byte) is a normal fp32 value with exponent
// field 254 - byte). amax = 0 or non-finite gives 1, like the Eq.(1) scale.
template <int FMT>
__device__ __forceinline__ float scale_pow2_from_amax_bits(uint32_t abits) {
    if (abits == 0u || abits >= 0x7F800000u) return 1.0f;
    const uint32_t byte = mx_byte_f32<FMT, kRoundUp>(abits);
    return __uint_as_float((254u - byte) << 23);
}

// Saturation of the round-down MX cast, applied to four packed codes after the scaled convert
// (which does not saturate). With the round-down exponent every |x| / 2^X is below 2^(emax+1),
// so a value can only overflow into (F8max, 2^(emax+1)); the convert then returns the overflow
// code (E4M3: 0x7F, NaN; E5M2: 0x7C, Inf) with the input's sign, and that code minus one is
// +-F8max. Every other code is left alone. Checked on gfx950 against clamping |x| to
// F8max * 2^X before the convert: identical for all finite BF16 inputs and all 255 scales.
template <int FMT>
__device__ __forceinline__ uint32_t mx_saturate_codes(uint32_t w) {
    if constexpr (FMT == kE4M3) {                 // bytes whose low 7 bits are all ones: 0x7F -> 0x7E
        return w ^ ((((w & 0x7F7F7F7Fu) + 0x01010101u) >> 7) & 0x01010101u);
    } else {                                      // bytes whose low 7 bits are 0x7C: 0x7C -> 0x7B
        // with bit 7 of every byte set, a byte minus one borrows from no other byte, and keeps
        // bit 7 unless its low 7 bits were zero, i.e. the code's were 0x7C
        const uint32_t y = (((w & 0x7F7F7F7Fu) ^ 0x7C7C7C7Cu) | 0x80808080u) - 0x01010101u;
        return w - ((~y & 0x80808080u) >> 7);
    }
}


// ---- NVFP4 block scaling (E2M1 codes under an E4M3 block scale and an fp32 tensor scale) -----
// S_t = fl32(448 * 6 / A) from the tensor |amax| bits (1 for A = 0 or non-finite, FLT_MAX on
// overflow). Per block: e_b = E4M3(amax_b * S_t / 6) and per element code = E2M1(x * S_t /
// decode(e_b)), each the nearest value of the exact quotient, ties to the even code (saturating);
// a block whose e_b decodes to 0 gives zero codes of the elements' signs, and a block with
// Inf/NaN gets the E4M3 NaN code 0x7F.
// Both quotients are found the same way. An fp32 estimate of the quotient is formed twice, pushed
// once below and once above the exact value by a factor (1 -/+ 2^-21 or 2^-20) larger than the
// estimate's own rounding error (at most three roundings of 2^-24). Rounding to the format is
// monotone, so when both estimates give the same code, so does the exact quotient. When they
// differ, the quotient lies within about 2^-20 of the midpoint t/d between the two codes, and
// fma(n1, n2, -t) = n1*n2 - t rounded once has the sign (and the zero) of the exact difference,
// which decides the side, or the tie.
__device__ __forceinline__ float nv_tensor_scale(uint32_t abits) {
    if (abits == 0u || abits >= 0x7F800000u) return 1.0f;
    const float s = 2688.0f / __uint_as_float(abits);
    return s > 3.40282346638528859812e+38f ? 3.40282346638528859812e+38f : s;
}
// E4M3 code of a non-negative fp32 value not above 448: the gfx950 convert rounds to nearest even.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
}
// e_b of a block from its |amax| bits and S_t.
__device__ __forceinline__ uint32_t nv_block_code(uint32_t amax_bits, float st) {
    if (amax_bits >= 0x7F800000u) return 0x7Fu;
    const float a = __uint_as_float(amax_bits);
    const float p = a * st;                       // inf when the caller's tensor amax is far too small
    constexpr float kSixthLo = (float)((1.0 / 6.0) * (1.0 - 0x1p-20));
    constexpr float kSixthHi = (float)((1.0 / 6.0) * (1.0 + 0x1p-20));
    // both estimates in one convert (byte 0 from below, byte 1 from above); the upper half of the
    // result comes from p's bits and is not used
    const uint32_t c2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(p * kSixthLo, 448.0f),
                                                                 fminf(p * kSixthHi, 448.0f), __float_as_int(p), false);
    const uint32_t clo = c2 & 0xFFu, chi = (c2 >> 8) & 0xFFu;
    if (clo == chi) return clo;
    // adjacent codes: 6 * their midpoint = 3 * (sum of the two values), exact in fp32
    const float t = 3.0f * (__builtin_amdgcn_cvt_f32_fp8(clo, 0) + __builtin_amdgcn_cvt_f32_fp8(chi, 0));
    const float s = __builtin_fmaf(a, st, -t);
    return s > 0.0f ? chi : s < 0.0f ? clo : ((clo & 1u) ? chi : clo);
}
// The element estimates' factors for every E4M3 block-scale code, written by threads 0..127 of the
// workgroup (S_t is one value for the whole tensor, so each block looks its pair up): (r_lo, r_hi)
// = fl32(S_t / decode(e)) times (1 - 2^-21, 1 + 2^-21). A code that decodes to 0 (and the NaN code)
// gets (0, 0), so its elements become signed zeros; a quotient S_t / decode(e) that overflows gets
// (0, Inf), so every nonzero element of such a block takes the exact path. The caller synchronizes
// before reading.
__device__ __forceinline__ void nv_factor_table(float2 *tab, float st) {
    const int e = (int)threadIdx.x;
    if (e < 128) {
        const float dec = __builtin_amdgcn_cvt_f32_fp8(e, 0);
        float2 f = make_float2(0.0f, 0.0f);
        if (e != 0x7F && dec != 0.0f) {
            const float r = st / dec;
            f = r <= 3.40282346638528859812e+38f ? make_float2(r * (1.0f - 0x1p-21f), r * (1.0f + 0x1p-21f))
                                                 : make_float2(0.0f, __builtin_inff());
        }
        tab[e] = f;
    }
}
// The exact E2M1 code of x * S_t / dec (dec > 0): the number of E2M1 midpoints (0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5) the exact quotient lies above, a tie counting when the even code is the upper
// one; saturation at 6 follows. Midpoint j lies between magnitudes j and j + 1, and being above it
// is monotone in j, so three comparisons find the count: midpoint 3, then 1 or 5, then 0, 2, 4 or
// 6. Each comparison is the sign of fma(|x|, S_t, -midpoint * dec), the exact difference rounded
// once (midpoint * dec is exact: 3 x 4 significant bits). A tie goes up at the odd midpoints
// 1, 3, 5 (the upper code is the even one) and stays at the even ones. NaN x gives zeros of its sign.
__device__ __forceinline__ uint32_t nv_elem_exact(float x, float st, float dec) {
    const float ax = __builtin_fabsf(x);
    const bool u4 = __builtin_fmaf(ax, st, -(1.75f * dec)) >= 0.0f;
    const bool u2 = __builtin_fmaf(ax, st, -((u4 ? 3.5f : 0.75f) * dec)) >= 0.0f;
    const float m = u4 ? (u2 ? 5.0f : 2.5f) : (u2 ? 1.25f : 0.25f);
    const bool u1 = __builtin_fmaf(ax, st, -(m * dec)) > 0.0f;
    const uint32_t c = (u4 ? 4u : 0u) + (u2 ? 2u : 0u) + (u1 ? 1u : 0u);
    return c | ((__float_as_uint(x) >> 31) << 3);
}
// Two fp32 values -> one byte of two E2M1 codes (first value in the low nibble) in byte SEL of
// `old`: v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to nearest even and saturates to +-6.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4_f32(uint32_t old, float a, float b, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// fp32 -> BF16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- buffer resources ------------------------------------------------------------------------
// Raw buffer descriptors (stride 0): addresses are base + voffset (per lane) + soffset (uniform),
// and any access whose offset reaches num_records is dropped (loads return 0). Kernels set the
// per-lane offset of idle lanes to kOutOfRange instead of branching around their accesses.
constexpr uint32_t kOutOfRange = 0x80000000u;
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
    // dword3 0x00020000: 32-bit data format, the value gfx9-family raw buffers use
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)num_bytes, 0x00020000);
}
// Cache policy operand: kCached (default) or kNonTemporal, the hint for data read once or
// written once in whole lines. Partial-line stores stay cached so that L2 can merge them.
constexpr int kCached = 0;
constexpr int kNonTemporal = 2;
template <int CP = kCached>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, CP);
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CP = kCached>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint4 v) {
    v4u32 w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)voff, (int)soff, CP);
}
template <int CP = kCached>
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lo, uint32_t hi) {
    v2u32 w = {lo, hi};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)voff, (int)soff, CP);
}
template <int CP = kCached>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, (int)soff, CP);
}
template <int CP = kCached>
__device__ __forceinline__ void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)voff, (int)soff, CP);
}
template <int CP = kCached>
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, (int)voff, (int)soff, CP);
}

// Non-temporal (streaming) global loads and stores for data touched exactly once.
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const v4u32 v = __builtin_nontemporal_load((const v4u32 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(uint4 *p, uint4 v) {
    const v4u32 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (v4u32 *)p);
}
__device__ __forceinline__ void st_stream(uint2 *p, uint2 v) {
    const v2u32 w = {v.x, v.y};
    __builtin_nontemporal_store(w, (v2u32 *)p);
}
__device__ __forceinline__ void st_stream(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }

}  // namespace qf8
