// Shared device helpers of the gfx950 canvas-denoising kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define DG_DEV __device__ __forceinline__

namespace dg {

typedef uint16_t bf16_t;                         // bf16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));  // MFMA bf16 operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));    // MFMA 16x16 accumulator
typedef long fp8x8_t;                            // 8 packed e4m3 codes (MFMA fp8 operand)
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));  // MFMA f16 operand
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- conversions
DG_DEV float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// Nearest binary16 of a float.  Finite values that would round beyond the
// largest finite binary16 (|v| >= 65520) saturate at +-65504 and set `range`;
// NaN and infinities pass through (the non-finite checks downstream see them).
DG_DEV _Float16 f32_to_f16_sat(float v, bool& range) {
    const float a = fabsf(v);
    const bool big = a >= 65520.f && a != __builtin_inff();
    range |= big;
    return (_Float16)(big ? copysignf(65504.f, v) : v);
}

DG_DEV bf16_t f32_to_bf16(float f) {            // round to nearest even
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// float -> OCP e4m3 code, round to nearest even, saturating at +-448.
DG_DEV uint32_t f32_to_e4m3(float x) {
    uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    float a = fabsf(x);
    if (!(a == a)) return 0x7fu;
    a = fminf(a, 448.0f);
    uint32_t code;
    if (a >= 0x1p-6f) {
        int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // a = 1.f * 2^e
        float q = rintf(ldexpf(a, 3 - e));                        // [8, 16]
        if (q >= 16.0f) { q = 8.0f; e += 1; }
        code = (uint32_t)((e + 7) << 3) | ((uint32_t)q - 8u);
    } else {
        code = (uint32_t)rintf(a * 512.0f);                       // subnormal steps of 2^-9
    }
    return sign | code;
}

template <typename T> DG_DEV float to_f32(T v);
template <> DG_DEV float to_f32<float>(float v) { return v; }
template <> DG_DEV float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> DG_DEV T from_f32(float v);
template <> DG_DEV float from_f32<float>(float v) { return v; }
template <> DG_DEV bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------- wave helpers
DG_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

DG_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror & Shaw, SC'11: 10 rounds; round multipliers on words
// 0 and 2, Weyl key schedule.
struct u32x4 { uint32_t x, y, z, w; };

DG_DEV u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        u32x4 n;
        n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
        n.y = (uint32_t)p1;
        n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
        n.w = (uint32_t)p0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

constexpr uint32_t kInitTag = 0x494E4954u;
constexpr uint32_t kGumbelTag = 0x47554D42u;
constexpr uint32_t kRenoiseTag = 0x524E5345u;

// u in (0,1), exact float: (2*(word>>9)+1) * 2^-24
DG_DEV float philox_open_uniform(uint32_t w) {
    return (float)(((w >> 9) << 1) | 1u) * 0x1p-24f;
}

}  // namespace dg
