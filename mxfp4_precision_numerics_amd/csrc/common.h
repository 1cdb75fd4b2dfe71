// common.h - device helpers shared by the gfx950 kernels of libmxq.
//
// Casting strategy.  gfx950's packed converters (v_cvt_scalef32_pk_*,
// v_cvt_pk_fp8_f32) round to nearest even, handle subnormal results, and
// divide by a power-of-two scale exactly.  Their FP8 forms do not saturate
// (an out-of-range value becomes NaN/Inf) and encode NaN without its sign,
// so the kernels clamp magnitudes on the integer bit pattern first (positive
// IEEE values order like unsigned integers) and patch NaN codes afterwards.
// The result is the saturating round-to-nearest-even cast defined for the
// formats of the FP8 guide ("O panorama da precisao numerica": E4M3 up to
// +-448, E5M2 wider) and of MXFP4 (E2M1; the MoE FP4 page, "Metodologia").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum Fmt { E4M3 = 0, E5M2 = 1, E2M1 = 2 };

// Per-format constants.
template <int F> struct FmtInfo;
template <> struct FmtInfo<E4M3> {
    static constexpr int emax = 8;                       // 448 = 1.75 * 2^8
    static constexpr uint32_t max_f32 = 0x43E00000u;     // 448.0f
    static constexpr uint32_t max_bf16 = 0x43E0u;        // 448 as bf16
    static constexpr uint32_t max_mant_bf16 = 0x60u;     // .11 in 7 mantissa bits
    static constexpr uint32_t max_mant_f32 = 0x600000u;
    static constexpr uint32_t nan_code = 0x7Fu;
    static constexpr int mfma_code = 0;
};
template <> struct FmtInfo<E5M2> {
    static constexpr int emax = 15;                      // 57344 = 1.75 * 2^15
    static constexpr uint32_t max_f32 = 0x47600000u;     // 57344.0f
    static constexpr uint32_t max_bf16 = 0x4760u;
    static constexpr uint32_t max_mant_bf16 = 0x60u;
    static constexpr uint32_t max_mant_f32 = 0x600000u;
    static constexpr uint32_t nan_code = 0x7Fu;
    static constexpr int mfma_code = 1;
};
template <> struct FmtInfo<E2M1> {
    static constexpr int emax = 2;                       // 6 = 1.5 * 2^2
    static constexpr int mfma_code = 4;
};

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

// 2^e as a binary32 (e in [-127, 127]; 2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float exp2i(int e) {
    return as_float(e > -127 ? (uint32_t)(e + 127) << 23 : 0x00400000u);
}

// Block scale exponent from the block's largest magnitude, given as the
// biased binary32 exponent field E of amax (0 for zero/subnormal):
// e = clamp(floor(log2 amax) - emax, -127, 127).  A subnormal amax has
// floor(log2) < -126, so it lands on the lower clamp like zero does.
template <int F> __device__ __forceinline__ int block_exp(uint32_t E) {
    int e = (int)E - 127 - FmtInfo<F>::emax;
    return e < -127 ? -127 : e;
}

// --- packed 16-bit helpers (two bf16 per dword) --------------------------
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    v2u16 x = __builtin_bit_cast(v2u16, a), y = __builtin_bit_cast(v2u16, b);
    v2u16 r = __builtin_elementwise_max(x, y);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    v2u16 x = __builtin_bit_cast(v2u16, a), y = __builtin_bit_cast(v2u16, b);
    v2u16 r = __builtin_elementwise_min(x, y);
    return __builtin_bit_cast(uint32_t, r);
}

// Two 16-bit lanes: w + s where w != 0, else 0, for w <= 63 and w + s below
// 1024: min(w + s, w << 10) (packed adds, shifts and mins only).
__device__ __forceinline__ uint32_t pk_lsum_u16(uint32_t w, uint32_t s2) {
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    const v2u16 x = __builtin_bit_cast(v2u16, w), s = __builtin_bit_cast(v2u16, s2);
    const v2u16 ten = {10, 10};
    const v2u16 r = __builtin_elementwise_min(x + s, x << ten);
    return __builtin_bit_cast(uint32_t, r);
}

// --- conversions -------------------------------------------------------------
// Two bf16 (one dword, element 0 in the low half) divided by the power of two
// `scale`, to two FP8 codes placed in the low (hi=false) or high half of `old`.
template <int F>
__device__ __forceinline__ uint32_t cvt2_bf16_fp8(uint32_t old, uint32_t w, float scale, bool hi) {
    v2s o = __builtin_bit_cast(v2s, old);
    v2bf x = __builtin_bit_cast(v2bf, w);
    v2s r;
    if (F == E4M3) {
        r = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, x, scale, true)
               : __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, x, scale, false);
    } else {
        r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(o, x, scale, true)
               : __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(o, x, scale, false);
    }
    return __builtin_bit_cast(uint32_t, r);
}

// Two binary32 divided by `scale`, to two FP8 codes in the low/high half.
template <int F>
__device__ __forceinline__ uint32_t cvt2_f32_fp8(uint32_t old, float a, float b, float scale, bool hi) {
    v2s o = __builtin_bit_cast(v2s, old);
    v2s r;
    if (F == E4M3) {
        r = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, true)
               : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, false);
    } else {
        r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, a, b, scale, true)
               : __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, a, b, scale, false);
    }
    return __builtin_bit_cast(uint32_t, r);
}

// Two bf16 / two binary32 divided by `scale` to two E2M1 codes (one byte,
// element 0 in the low nibble) placed in byte `sel` of `old`.  The E2M1
// converters saturate at +-6 by themselves.
template <int SEL>
__device__ __forceinline__ uint32_t cvt2_bf16_fp4(uint32_t old, uint32_t w, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(v2bf, w), scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t cvt2_f32_fp4(uint32_t old, float a, float b, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// Saturating clamp of two bf16 magnitudes at `lim` (bf16 bits, both halves),
// sign kept.  Inputs must be finite.
__device__ __forceinline__ uint32_t clamp2_bf16(uint32_t w, uint32_t lim2) {
    return (w & 0x80008000u) | pk_min_u16(w & 0x7FFF7FFFu, lim2);
}
// Same for one binary32.
__device__ __forceinline__ uint32_t clamp_f32(uint32_t u, uint32_t lim) {
    uint32_t a = u & 0x7FFFFFFFu;
    return (u & 0x80000000u) | (a < lim ? a : lim);
}

// Per-tensor cast of one binary32 product y = fl32(x * scale) (any value) to
// an FP8 code: NaN -> 0x7F|sign, |y| >= max -> +-max, else RNE.  Two values
// at a time (the converter is packed); returns two codes in the low 16 bits.
template <int F>
__device__ __forceinline__ uint32_t cast2_sat_f32(float y0, float y1) {
    uint32_t u0 = as_uint(y0), u1 = as_uint(y1);
    uint32_t c0 = clamp_f32(u0, FmtInfo<F>::max_f32), c1 = clamp_f32(u1, FmtInfo<F>::max_f32);
    uint32_t r;
    if constexpr (F == E4M3)
        r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(as_float(c0), as_float(c1), 0, false);
    else
        r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(as_float(c0), as_float(c1), 0, false);
    r &= 0xFFFFu;
    if ((u0 & 0x7FFFFFFFu) > 0x7F800000u) r = (r & 0xFF00u) | 0x7Fu | ((u0 >> 24) & 0x80u);
    if ((u1 & 0x7FFFFFFFu) > 0x7F800000u) r = (r & 0x00FFu) | ((0x7Fu | ((u1 >> 24) & 0x80u)) << 8);
    return r;
}

// --- MX block codes and the expert MLP activation ------------------------------
// Codes and scale byte of 8 binary32 values (bit patterns) of one 32-element
// MX block whose largest magnitude (bit pattern, NaN/Inf included) is
// amax_bits: e = floor(log2 amax) - emax clamped at -127, each value clamped
// to the largest finite magnitude at that scale (saturation) and converted by
// the scaled RNE converter; a block holding NaN or Inf gets codes 0x7F and
// scale byte 0xFF.
template <int F>
__device__ __forceinline__ void mx_codes_row8(const uint32_t (&u)[8], uint32_t amax_bits, uint32_t& lo, uint32_t& hi,
                                              uint8_t& sbyte) {
    const bool bad = amax_bits >= 0x7F800000u;
    const int e = block_exp<F>(amax_bits >> 23);
    const float sc = exp2i(e);
    const uint32_t lim = (uint32_t)(e + 127 + FmtInfo<F>::emax) << 23 | FmtInfo<F>::max_mant_f32;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = as_float(clamp_f32(u[k], lim));
    lo = cvt2_f32_fp8<F>(0u, y[0], y[1], sc, false);
    lo = cvt2_f32_fp8<F>(lo, y[2], y[3], sc, true);
    hi = cvt2_f32_fp8<F>(0u, y[4], y[5], sc, false);
    hi = cvt2_f32_fp8<F>(hi, y[6], y[7], sc, true);
    if (bad) { lo = 0x7F7F7F7Fu; hi = 0x7F7F7F7Fu; }
    sbyte = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
}

// h = silu(g) * u in binary32, silu(g) = g / (1 + e^-g): the sigmoid from
// e^-|g| in (0, 1], which cannot overflow (very negative gates keep their
// subnormal products instead of 0), and the hardware reciprocal (1 ulp).
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    const float en = expf(-__builtin_fabsf(g));
    const float sg = (g >= 0.0f ? 1.0f : en) * __builtin_amdgcn_rcpf(1.0f + en);
    return g * sg * u;
}

// --- streaming memory access ----------------------------------------------------
// The casts read every input once and write every output once.  They use
// nontemporal loads and stores (the instructions' nt cache policy), which
// keep these streams from displacing cached lines; on gfx950 a 2:1 stream
// measured about 5.7 TB/s this way against about 3.3 TB/s with plain ones.
typedef unsigned nt_v4u __attribute__((ext_vector_type(4)));
typedef unsigned nt_v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const nt_v4u v = __builtin_nontemporal_load(reinterpret_cast<const nt_v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
    const nt_v2u v = __builtin_nontemporal_load(reinterpret_cast<const nt_v2u*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_nt4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
    __builtin_nontemporal_store(nt_v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_v4u*>(p));
}
__device__ __forceinline__ void st_nt8(void* p, uint2 v) {
    __builtin_nontemporal_store(nt_v2u{v.x, v.y}, reinterpret_cast<nt_v2u*>(p));
}
__device__ __forceinline__ void st_nt4(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_nt1(void* p, uint8_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint8_t*>(p));
}

// --- reductions ----------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// max over the 4 lanes of an aligned quad
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, 1, 64);
    v = v > o ? v : o;
    o = (uint32_t)__shfl_xor((int)v, 2, 64);
    return v > o ? v : o;
}

// max over lanes l, l^4, l^8, l^12 (4 lanes strided by 4)
__device__ __forceinline__ uint32_t quad4_max_u32(uint32_t v) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, 4, 64);
    v = v > o ? v : o;
    o = (uint32_t)__shfl_xor((int)v, 8, 64);
    return v > o ? v : o;
}

// Max over lanes l, l^4, l^8, l^12 of two 16-bit lanes at once.  Those four
// lanes share a DPP row of 16, so rotations of the row by 4 and by 8 reach
// them (no LDS crossbar).
__device__ __forceinline__ uint32_t quad4_max_pk16(uint32_t v) {
    v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
    return pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
}

// 4x4 byte transpose: r[i] holds bytes (row i, cols 0..3); on return r[j]
// holds bytes (rows 0..3, col j).
__device__ __forceinline__ void transpose4x4_bytes(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
    // __builtin_amdgcn_perm(hi, lo, sel): selector byte k < 4 takes lo's byte k,
    // 4..7 takes hi's byte k-4.
    uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
    uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
    uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    r0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    r1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    r2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    r3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

}  // namespace mxq
