// bsp_device.hpp -- device-side number formats and helpers for gfx950.
//
// Encoders work on the IEEE binary32 bit pattern with integer rounding
// (round to nearest, ties to even), so every result is a pure function of
// the input bits.  Formats:
//   E2M1 (NVFP4 element): values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}
//        [nopree.com, "End-to-End 4-Bit Training", section 先说为什么难];
//   E4M3 (OCP FP8 E4M3FN): bias 7, maximum 448, subnormals m * 2^-9;
//   E8M0: 2^(c - 127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsp {

constexpr uint32_t kF32_448 = 0x43E00000u;   // 448.0f
constexpr uint32_t kF32_6 = 0x40C00000u;     // 6.0f
constexpr float kFlushBelow = 1.17549435e-38f;  // 2^-126, smallest normal f32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round the 24-bit significand `mant` right by `shift` bits (1 <= shift <= 31),
// nearest even.
__device__ __forceinline__ uint32_t rne_shift(uint32_t mant, uint32_t shift) {
    uint32_t q = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1u);
    q += (rem > half) | ((rem == half) & (q & 1u));
    return q;
}

// E4M3 encode, nearest even, saturating at 448; sign copied from the input.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    uint32_t b = __float_as_uint(y);
    uint32_t sign = (b >> 24) & 0x80u;
    uint32_t a = b & 0x7FFFFFFFu;
    if (a >= kF32_448) return sign | 0x7Eu;
    if (a <= 0x3A800000u) return sign;              // |y| <= 2^-10 rounds to 0
    int e = (int)(a >> 23) - 127;                   // >= -10
    int ee = e < -6 ? -6 : e;                       // E4M3 subnormals share 2^-6's scale
    uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
    uint32_t q = rne_shift(mant, (uint32_t)(20 + (ee - e)));
    return sign | (uint32_t)(((ee + 6) << 3) + (int)q);
}

// Two E4M3 codes (a in bits 0-7, b in bits 8-15) with the gfx950 conversion
// V_CVT_PK_FP8_F32.  Checked exhaustively against e4m3_encode over every f32
// with |y| <= 448 (both signs, subnormals included): identical.  Inputs are
// clamped to +-448 first, which is exactly e4m3_encode's saturation.
__device__ __forceinline__ uint32_t e4m3x2_hw(float a, float b) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four E4M3 codes packed little-endian.
__device__ __forceinline__ uint32_t e4m3x4_hw(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Two E2M1 codes (a in the low nibble, b in the high nibble) with the gfx950
// conversion V_CVT_SCALEF32_PK_FP4_F32 at scale 1.  Checked exhaustively
// against e2m1_encode over every finite f32 (both signs): identical,
// including ties to even, saturation at 6 and signed zeros.
__device__ __forceinline__ uint32_t e2m1x2_hw(float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// E4M3 decode (code 0x7F / 0xFF never produced).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;  // m * 2^-9
    return (c & 0x80u) ? -mag : mag;
}

// E2M1 magnitude code of a >= 0 (f32 bits), nearest even, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_mag(float av) {
    uint32_t a = __float_as_uint(av);
    if (a >= kF32_6) return 7u;
    if (a <= 0x3E800000u) return 0u;                // <= 0.25
    int E = (int)(a >> 23) - 126;                   // biased E2M1 exponent, >= -1
    int EE = E < 1 ? 1 : E;
    uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
    uint32_t q = rne_shift(mant, (uint32_t)(22 + (EE - E)));
    return (uint32_t)(2 * (EE - 1)) + q;
}

// Signed E2M1 code of v: sign bit 3 from v.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    return ((__float_as_uint(v) >> 28) & 8u) | e2m1_mag(fabsf(v));
}

// E2M1 magnitude value of a 3-bit code.
__device__ __forceinline__ float e2m1_mag_value(uint32_t m) {
    // 0, 0.5, 1, 1.5, 2, 3, 4, 6: exponent field e = m >> 1, mantissa bit m & 1
    uint32_t e = m >> 1, b = m & 1u;
    float normal = __uint_as_float(((e + 126u) << 23) | (b << 22));
    return e ? normal : 0.5f * (float)b;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
    float v = e2m1_mag_value(c & 7u);
    return (c & 8u) ? -v : v;
}

// MXFP8 block exponent: smallest k with amax <= 448 * 2^k, within [-127, 119].
// From the f32 bits of amax = 1.f * 2^E: k = E - 8, plus one when f > 0.75.
__device__ __forceinline__ int mx_block_exponent(float amax) {
    uint32_t a = __float_as_uint(amax);
    int E = (int)(a >> 23) - 127;
    int k = E - 8 + ((a & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    if (a < 0x00800000u) k = -127;                  // zero or f32 subnormal
    k = k < -127 ? -127 : k;
    k = k > 119 ? 119 : k;
    return k;
}

// 2^k as an f32 for k in [-126, 127].
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// SwiGLU of one element: bf16 bits of silu(gate) * up, silu(z) =
// z / (1 + exp(-z)), the product rounded to bf16 (nearest even).  exp(-z) is
// the hardware base-2 exponential (V_EXP_F32) of -z log2(e) and the division
// the hardware reciprocal (V_RCP_F32) and a multiply: the argument's rounding
// (at most |z log2 e| units of 2^-24, |z| < 89 where it matters) and the two
// approximations keep silu(z) * up within 2^-16 of its exact value relative
// to it, far inside the half bf16 unit (2^-9) of the final rounding, so h is
// the correctly rounded bf16 value or its neighbour: within one bf16 unit.
// From z < -88.7 the exponential is inf and h is -0 times up (the exact value
// there is at most 3e-37 |up|).
__device__ __forceinline__ uint32_t swiglu_bf16(float gate, float up) {
    const float e = __builtin_amdgcn_exp2f(gate * -1.44269504088896341f);
    const float silu = gate * __builtin_amdgcn_rcpf(1.0f + e);
    return f32_to_bf16(silu * up);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// Exclusive prefix sum over a 256-thread workgroup of each thread's value,
// plus the workgroup total.  `wsum` holds four words of LDS; every thread
// must call this (it contains barriers).
__device__ __forceinline__ int64_t block256_excl_scan(int64_t v, int64_t *wsum, int64_t &total) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t incl = wave_incl_scan(v, lane);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int64_t run = incl - v;
    for (int w = 0; w < wv; w++) run += wsum[w];
    total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();   // wsum may be rewritten by the next call
    return run;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of two
// 32x32->64 multiplies with the Philox constants, high halves xor-ed into
// the other words with the round key, key advanced by the Weyl constants.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; r++) {
        // one V_MAD_U64_U32 per product gives both halves
        const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
        // three-input xor in one V_BITOP3_B32 (truth table 0x96)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
        c[0] = n0;
        c[1] = (uint32_t)p1;
        c[2] = n2;
        c[3] = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

}  // namespace bsp
