// Device helpers shared by the gfx950 quantizer and GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsfp8 {

constexpr int kGroup = 128;         // 1x128 / 128x1 / 128x128 group edge
constexpr float kFp8Max = 448.0f;   // finfo(float8_e4m3fn).max
constexpr float kAmaxEps = 1e-12f;  // floor on a group's amax (all-zero groups)

// Element format of the codes. FP8_MAX is the format's finfo max ("Enable blockwise FP8 dense
// training kernels on ROCm", description): 448 for float8_e4m3fn, 240 for float8_e4m3fnuz, the
// format that page's MI300X runs use.
//   float8_e4m3fnuz has the bit layout of e4m3fn with the exponent bias raised by one, so a code
//   that is finite in both formats means half its e4m3fn value; it has no negative zero (0x80 is
//   its only NaN) and 0x7F is its largest finite value, 240. gfx950's conversion instruction
//   produces e4m3fn, so an fnuz code is the e4m3fn conversion of twice the value (same rounding
//   grid, scaled by two), with 0x80 replaced by 0x00 -- see encode4_in_range.
template <bool FNUZ>
struct Fp8Format {
    static constexpr float kMax = FNUZ ? 240.0f : 448.0f;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Low and high bf16 of a packed dword.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Quantization of one value already multiplied by the group multiplier: clamp to +-448 (keeps the
// sign of zero), then the hardware RNE fp32 -> e4m3fn conversion. Four values -> one dword, byte i
// holding value i.
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -kFp8Max), kFp8Max);
    b = fminf(fmaxf(b, -kFp8Max), kFp8Max);
    c = fminf(fmaxf(c, -kFp8Max), kFp8Max);
    d = fminf(fmaxf(d, -kFp8Max), kFp8Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0,1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);        // bytes 2,3
    return static_cast<uint32_t>(w);
}

// encode4 for values x * m of a group whose multiplier is m = fl(448 / amax_c) with |x| <= amax_c:
// then |fl(x * m)| <= 448 (1 + 2^-24)^2 rounded, at most two fp32 ulps above 448, and the
// conversion rounds every magnitude up to 464 (the tie between 448 and the next binade step,
// resolved to even) to 448 -- the clamp of encode4 can never change such a value, so it is left
// out.
//
// float8_e4m3fnuz (FNUZ): the values come from a group multiplier that group_scale<true> has
// already doubled (2 fl(240 / amax_c), exact), so they are exactly twice fl(x * fl(240 / amax_c))
// and at most a few ulps above 480. The e4m3fn conversion of twice a value v rounds on the fnuz
// grid of v scaled by two; magnitudes up to 464 (the tie between 448 and the step above, resolved
// to the even 448) give codes up to 0x7E (fnuz 224), larger ones the pattern 0x7F with the sign,
// which is fnuz's largest value 240 -- exactly the round-to-nearest-even, saturating result for
// |v| in (232, 240]. A value that rounds to zero keeps its sign in e4m3fn (0x80), which is NaN in
// fnuz: every 0x80 byte becomes 0x00.
__device__ __forceinline__ uint32_t drop_negative_zero(uint32_t w) {
    const uint32_t mag = w & 0x7F7F7F7Fu;
    // per byte: magnitude + 0x7F <= 0xFE, so no carry crosses bytes and bit 7 is set exactly when
    // the magnitude is non-zero
    const uint32_t nonzero = mag + 0x7F7F7F7Fu;
    return (w & nonzero & 0x80808080u) | mag;
}

template <bool FNUZ = false>
__device__ __forceinline__ uint32_t encode4_in_range(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return FNUZ ? drop_negative_zero(static_cast<uint32_t>(w)) : static_cast<uint32_t>(w);
}

// Group scale pair from the group's max magnitude: the stored (dequantizing) scale
// s = amax/FP8_MAX and the multiplier m = FP8_MAX/amax, both IEEE-correct fp32 divisions (the
// compiler's default fp32 division is correctly rounded; fp32 denormals are preserved). For fnuz
// the multiplier is returned doubled (exact), as encode4_in_range<true> expects.
struct GroupScale {
    float s;
    float m;
};

template <bool FNUZ = false>
__device__ __forceinline__ GroupScale group_scale(float amax) {
    constexpr float kMax = Fp8Format<FNUZ>::kMax;
    float a = fmaxf(amax, kAmaxEps);
    GroupScale g;
    g.s = a / kMax;
    g.m = kMax / a;
    if (FNUZ) g.m *= 2.0f;
    return g;
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15) of a non-negative float, via the
// unsigned order of the bit patterns (valid for non-negative, non-NaN values). Every lane of the
// row receives the result.
__device__ __forceinline__ uint32_t umax_row16(uint32_t v) {
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// Max over all 64 lanes of a wave (non-negative floats as bit patterns).
__device__ __forceinline__ uint32_t umax_wave(uint32_t v) {
    v = umax_row16(v);
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16)));
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 32)));
    return v;
}

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

}  // namespace bsfp8
