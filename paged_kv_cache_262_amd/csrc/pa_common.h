// Internal helpers shared by the gfx950 kernels of libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint16_t bf16_t;  // bf16 storage: the top 16 bits of an fp32 word

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ void store(float *p, float x) { *p = x; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ void store(bf16_t *p, float x) { *p = f32_to_bf16(x); }
};

// ---- cross-lane moves inside a 16-lane DPP row -----------------------------
// Control words of the GFX9 DPP encoding.
enum : int {
    DPP_XOR1 = 0xB1,         // quad_perm [1,0,3,2]
    DPP_XOR2 = 0x4E,         // quad_perm [2,3,0,1]
    DPP_HALF_MIRROR = 0x141, // lane i <-> 7-i inside each group of 8
    DPP_MIRROR = 0x140,      // lane i <-> 15-i inside each row of 16
    DPP_ROR8 = 0x128,        // rotate a row of 16 by 8 (i <-> i^8)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "group size");
    x += dpp<DPP_XOR1>(x);
    x += dpp<DPP_XOR2>(x);
    if (N >= 8) x += dpp<DPP_HALF_MIRROR>(x);
    if (N >= 16) x += dpp<DPP_MIRROR>(x);
    return x;
}

// Max over the whole wave of 64; every lane gets it.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<DPP_XOR1>(x));
    x = fmaxf(x, dpp<DPP_XOR2>(x));
    x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
    x = fmaxf(x, dpp<DPP_MIRROR>(x));
    float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---- e4m3 (OCP 8-bit float: bias 7, 3 mantissa bits, no infinities,
// S.1111.111 = NaN, largest finite 448, smallest subnormal 2^-9) --------------
// e4m3 code of y: nearest value, ties to the even code, saturating at +-448,
// NaN -> 0x7F.  Written from the format's definition (no hardware
// conversion), so these rules hold whatever an instruction would do.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t u = __float_as_uint(y);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7Fu;  // NaN
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fminf(__uint_as_float(u & 0x7fffffffu), 448.0f);
    uint32_t code;
    if (a < 0.015625f) {
        // below 2^-6: subnormal codes 0..7 step 2^-9 (8 rounds up to 2^-6)
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        // normal: keep 3 of fp32's 23 mantissa bits, round half to even; a
        // carry moves into the exponent.  Rebias the exponent 127 -> 7.
        uint32_t b = __float_as_uint(a);
        b += 0x7FFFFu + ((b >> 20) & 1u);
        code = (b >> 20) - (120u << 3);
    }
    return sign | code;
}


// log2(e): softmax runs in base 2, the scale carries the conversion.
constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa
