// Device-side building blocks shared by the split kernel and the GEMM kernels
// (gfx950 only).
//
// The split is the one of "Unlocking Tensor Core Performance for Machine
// Learning Interatomic Potentials", section "How Tensor Core FP32 bridges the
// hardware gap", Figure 1: three scaled BF16 pieces per FP32 value,
//     hi = R(a),  mid' = R(2^8 (a - hi)),  lo' = 2^8 (2^8 (a - hi) - mid'),
// R = round to nearest even, saturating at +-0x7F7F.  Every subtraction and
// power-of-two scaling below is exact for finite a, so a == hi + 2^-8 mid' +
// 2^-16 lo' and lo' needs no rounding (it has at most 8 significant bits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace emu {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A zeroed MFMA accumulator, written as eight 64-bit moves (v_mov_b64)
// instead of sixteen 32-bit ones: half the VALU issue slots for the clears
// that follow every output tile.  The asm is volatile so that the moves are
// neither merged into one shared zero register (which would then be copied)
// nor hoisted out of the loop that reuses the accumulator.
__device__ __forceinline__ f32x16_t zero_acc()
{
    typedef double f64x8_t __attribute__((ext_vector_type(8)));
    f64x8_t z;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        double d;
        asm volatile("v_mov_b64 %0, 0" : "=v"(d));
        z[j] = d;
    }
    return __builtin_bit_cast(f32x16_t, z);
}

// Largest finite FP32 whose BF16 rounding is finite (0x7F7F7FFF): clamping
// to it before R makes the conversion saturate exactly as R prescribes.
__device__ __forceinline__ float bf16_sat_limit() { return __uint_as_float(0x7F7F7FFFu); }

__device__ __forceinline__ float clamp_sat(float x)
{
    const float lim = bf16_sat_limit();
    return __builtin_amdgcn_fmed3f(x, -lim, lim);
}

// Round two floats to BF16 (round to nearest even; v_cvt_pk_bf16_f32) and
// pack them: x0 in bits 0..15, x1 in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1)
{
    f32x2_t v = {x0, x1};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float lo_half_value(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_half_value(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Split of a pair (a0, a1): packed hi, mid', lo' words (a0 in the low half).
// SAT_MID: clamp before rounding mid' (needed for exactness only when |a| is
// within 2^-15 of FLT_MAX).  Without it, a non-finite a propagates into mid'.
// Non-finite a: hi is clamped finite, and the residuals carry the NaN/inf.
template <bool SAT_MID>
__device__ __forceinline__ void split_pair(float a0, float a1, uint32_t& hi, uint32_t& mid,
                                           uint32_t& lo)
{
    hi = pack_bf16x2(clamp_sat(a0), clamp_sat(a1));
    const float m0 = (a0 - lo_half_value(hi)) * 256.0f;
    const float m1 = (a1 - hi_half_value(hi)) * 256.0f;
    mid = SAT_MID ? pack_bf16x2(clamp_sat(m0), clamp_sat(m1)) : pack_bf16x2(m0, m1);
    const float l0 = (m0 - lo_half_value(mid)) * 256.0f;
    const float l1 = (m1 - hi_half_value(mid)) * 256.0f;
    // l0, l1 are BF16 values: their upper halves are the pieces.
    lo = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
}

// x clamped to +-bf16_sat_limit() when finite (so that R saturates), passed
// through when +-inf or NaN (the clamp alone would make it finite).
__device__ __forceinline__ float sat_finite(float x)
{
    return __builtin_fabsf(x) <= __uint_as_float(0x7F7FFFFFu) ? clamp_sat(x) : x;
}

// Two-piece version (hi, mid') for the three-product mode: the same pieces
// as split_pair<true>, mid' saturating like hi (for |a| within 2^-15 of
// FLT_MAX, 2^8 (a - hi) rounds past the largest BF16).  For finite a the
// residual 2^8 (a - hi) is finite, so sat_finite only ever passes through the
// inf/NaN of a non-finite a, which then reaches the products through mid'.
__device__ __forceinline__ void split_pair_hm(float a0, float a1, uint32_t& hi, uint32_t& mid)
{
    hi = pack_bf16x2(clamp_sat(a0), clamp_sat(a1));
    const float m0 = (a0 - lo_half_value(hi)) * 256.0f;
    const float m1 = (a1 - hi_half_value(hi)) * 256.0f;
    mid = pack_bf16x2(sat_finite(m0), sat_finite(m1));
}

// The first NP pieces of a pair (a0 in the low half of each word):
// w[0] = hi, w[1] = mid', w[2] = lo'.  NP = 1 is the one-piece (hi only)
// rounding of the one-product mode, where a non-finite a keeps its hi =
// +-inf / NaN.
template <int NP>
__device__ __forceinline__ void split_pieces(float a0, float a1, uint32_t (&w)[NP])
{
    static_assert(NP >= 1 && NP <= 3, "one to three pieces");
    if constexpr (NP == 3)
        split_pair<true>(a0, a1, w[0], w[1], w[2]);
    else if constexpr (NP == 2)
        split_pair_hm(a0, a1, w[0], w[1]);
    else
        w[0] = pack_bf16x2(sat_finite(a0), sat_finite(a1));
}

}  // namespace emu
