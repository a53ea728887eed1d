// MXFP8 (OCP Microscaling, E4M3 elements, E8M0 scales) helpers for the
// gfx950 kernels of libmoegmm.
//
// The A8W8-FP scenario of "MegaMoE" quantises activations in groups of 32
// consecutive elements along the reduction dimension, one E8M0 scale per
// group.  The conversion follows the OCP MX v1.0 definition:
//   shared exponent  X = floor(log2(max |v|)) - 8      (8: exponent of 448,
//                    the largest E4M3 normal), clamped to >= -127;
//                    an all-zero group takes X = -127
//   scale byte       X + 127
//   element          v / 2^X rounded to the nearest E4M3 value, ties to even,
//                    saturating at +-448 (E4M3 "FN" has no infinity).
// The division by 2^X is exact, so these decisions are exact functions of the
// fp32 input.  NaN inputs are not supported (they encode as +-448).
#pragma once

#include "common.h"

namespace moegmm {

constexpr int kMxGroup = 32;  // elements per shared scale

// Scale byte of a group whose largest magnitude is the finite fp32 `amax`:
// for a normal amax with biased exponent b, floor(log2 amax) = b - 127, so the
// byte is b - 8, clamped at 0 (subnormal or zero amax gives 0).
MOE_DEVICE uint32_t mx_scale_byte(float amax) {
    const uint32_t b = (__float_as_uint(amax) >> 23) & 0xFFu;
    return b > 8u ? b - 8u : 0u;
}

// 2^(127 - byte): multiplying by it maps a group onto the E4M3 grid.  Exact
// (a normal fp32) for every byte mx_scale_byte can return (at most 246).
MOE_DEVICE float mx_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// E4M3FN code of f (|f| < 512 after scaling), round to nearest even,
// saturating at 448.  With E = max(floor(log2 |f|), -6) the representable
// neighbours of |f| are multiples of 2^(E-3); rint picks the nearest (ties to
// even), and a carry into the next binade falls out of the code arithmetic
// ((E+7) << 3 is the code of 2^E, plus the mantissa steps).
MOE_DEVICE uint32_t e4m3_rne_sat(float f) {
    const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
    const float a = fminf(fabsf(f), 448.0f);
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
    e = e < -6 ? -6 : e;
    const float to_steps = __uint_as_float((uint32_t)(130 - e) << 23);  // 2^(3-e)
    const int m = (int)__builtin_rintf(a * to_steps);
    return sign | (uint32_t)(((e + 7) << 3) + m - 8);
}

// Largest of v over the 4 lanes of a quad (lanes 4q .. 4q+3), every lane of
// the quad getting it: two DPP quad permutes (lane ^ 1, then lane ^ 2) on
// the vector ALU instead of LDS-routed shuffles.  All lanes must be active.
MOE_DEVICE float quad_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // [1,0,3,2]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));  // [2,3,0,1]
    return v;
}

// Largest of v over lane pairs (2p, 2p+1), both lanes getting it (one DPP
// quad permute).  All lanes must be active.
MOE_DEVICE float pair_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // [1,0,3,2]
}

// Four values (already scaled) -> four codes packed little-endian.
MOE_DEVICE uint32_t e4m3_pack4(float a, float b, float c, float d) {
    return e4m3_rne_sat(a) | (e4m3_rne_sat(b) << 8) | (e4m3_rne_sat(c) << 16) |
           (e4m3_rne_sat(d) << 24);
}

}  // namespace moegmm
