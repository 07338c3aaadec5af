// MXFP8 (E4M3 elements, E8M0 scale per 32 elements) arithmetic on the device.
//
// arex-research.com "Cursor 放出 MoK", design section, closing paragraph: the
// layer runs in BF16 or MXFP8; weights are quantised ahead of time and the
// activations inside dispatch, the expert GEMMs and SwiGLU.  The pages name the
// format only; the rule is the OCP Microscaling (MX) v1.0 one:
//   scale 2^s, s = floor(log2(max |v|)) - 8, clamped to [-127, 127] (all-zero
//   block: s = -127); element = v / 2^s rounded to nearest-even on the E4M3 grid,
//   saturated to +-448.
#pragma once

#include "common.h"

namespace moe {

// s of a block whose largest magnitude is amax (>= 0, finite)
__device__ __forceinline__ int mx_scale_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int ef = (int)((u >> 23) & 0xffu);
    if (ef == 0) return -127;          // zero or subnormal maximum: s < -127 before the clamp
    const int s = ef - 127 - 8;        // floor(log2 amax) - 8 (ef <= 254 so s <= 119)
    return s < -127 ? -127 : s;
}

// E4M3 code of v (already divided by the block scale), round to nearest even,
// saturating; the sign bit is kept for zero results.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = __uint_as_float(u & 0x7fffffffu);
    if (a >= 448.0f) return sign | 0x7eu;
    if (a < 0.015625f) {                       // below 2^-6: quantum 2^-9 (subnormals)
        const uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8, 8 = 2^-6
        return sign | m;
    }
    // normal: keep 3 mantissa bits, round half to even at bit 20
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    const uint32_t e = (b >> 23) - 127u + 7u;  // biased E4M3 exponent, 1..15
    const uint32_t m = (b >> 20) & 7u;
    return sign | (e << 3) | m;
}

// Four values of one 32-element block whose scale exponent is s -> four codes,
// value q in byte q.  The packed conversion instruction rounds to nearest
// even and keeps the sign of zero results, like e4m3_code; with the
// magnitude clamped to 448 first (its saturation) it returned e4m3_code's
// byte for every float32 below 512 in magnitude, both signs, subnormals
// included (a scaled block element is below 2^9), checked on gfx950.  It is
// one instruction per two values where e4m3_code takes a dozen with a branch.
__device__ __forceinline__ float e4m3_clamp(float v, int s) {
    const float x = __builtin_amdgcn_ldexpf(v, -s);
    return __builtin_copysignf(__builtin_fminf(__builtin_fabsf(x), 448.0f), x);
}

__device__ __forceinline__ uint32_t e4m3_pack4(const float* v, int s) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(v[0], s), e4m3_clamp(v[1], s), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(v[2], s), e4m3_clamp(v[3], s), lo, true);
}

// Quantise 8 values that belong to one 32-element block whose scale exponent is s.
__device__ __forceinline__ uint2 e4m3_pack8(const float* v, int s) {
    return make_uint2(e4m3_pack4(v, s), e4m3_pack4(v + 4, s));
}

// ------------------------------------------------------------------ MXFP4
// E2M1 elements (the MXFP4 element type of OCP MX v1.0): magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6; the block scale is 2^(floor(log2 amax) - 2), 2 being the
// exponent of the largest value (6 = 1.5 * 2^2); round to nearest even,
// saturate to +-6; the sign bit is kept for zero results.
__device__ __forceinline__ int mx4_scale_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int ef = (int)((u >> 23) & 0xffu);
    if (ef == 0) return -127;
    const int s = ef - 127 - 2;
    return s < -127 ? -127 : s;
}

// E2M1 code (0..15) of v, already divided by the block scale
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 28) & 0x8u;
    const float a = __uint_as_float(u & 0x7fffffffu);
    // quantum: 0.5 below 2, 1 in [2, 4), 2 from 4; count of quanta rounded half to even
    float r;
    if (a < 2.0f) r = __builtin_rintf(a * 2.0f) * 0.5f;
    else if (a < 4.0f) r = __builtin_rintf(a);
    else r = __builtin_rintf(a * 0.5f) * 2.0f;
    uint32_t m;                        // index on the grid 0, .5, 1, 1.5, 2, 3, 4, 6
    if (r < 2.0f) m = (uint32_t)(r * 2.0f);          // 0..3 (r = 2 handled below)
    else if (r < 4.0f) m = 2u + (uint32_t)r;        // 2 -> 4, 3 -> 5
    else m = r < 6.0f ? 6u : 7u;                     // 4 -> 6, >= 6 saturates
    return sign | m;
}

// eight values of one 32-element block (scale exponent s) -> 8 codes, element
// 2q in the low nibble of byte q
__device__ __forceinline__ uint32_t e2m1_pack8(const float* v, int s) {
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) w |= e2m1_code(__builtin_amdgcn_ldexpf(v[q], -s)) << (4 * q);
    return w;
}

}  // namespace moe
