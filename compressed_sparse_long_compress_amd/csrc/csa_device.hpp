// Device helpers shared by the libcsa kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round-to-nearest-even fp32 -> bf16 bits (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts
// (1, 2, 4, 8 within each 16-lane row; shifted-in lanes read 0) and the
// row broadcasts of lanes 15 and 31 into the following rows.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the same position in each
// 16-lane row) with the gfx950 row-swap permutes; every one of the four lanes
// gets the bitwise-identical result (each step adds or maxes one pair).
__device__ __forceinline__ float rows4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// RoPE on pair i (dims 2i, 2i+1 of the 64 rotary dims) at position pos:
// theta_i = base^(-2i/64), angle = pos * theta_i, both in fp64.
__device__ __forceinline__ void rope_cs(double pos, double base, int i, float& c, float& s) {
    double theta = pow(base, -2.0 * (double)i / 64.0);
    double sn, cs;
    sincos(pos * theta, &sn, &cs);
    c = (float)cs;
    s = (float)sn;
}

// Gradient sums that must not depend on the order of their terms (several rows or heads adding
// into one entry's gradient) accumulate in 64-bit fixed point: units of 2^-40, range +-2^23.
// Each term is rounded once to the nearest unit (ties away from zero); integer addition is
// associative, so the sum is the same bits whatever order the atomics land in.
constexpr double kFxUnit = 1099511627776.0;  // 2^40 units per 1.0
__device__ __forceinline__ long long f32_to_fx(float v) {
    // v = mant * 2^(ex - 150) for a normal float; times 2^40: mant * 2^(ex - 110), by integer shifts
    const uint32_t b = __float_as_uint(v);
    const int ex = (int)((b >> 23) & 0xFFu);
    const long long mant = (long long)((b & 0x7FFFFFu) | 0x800000u);
    const int sh = ex - 110;
    long long r;
    if (sh >= 0) r = mant << (sh < 39 ? sh : 39);                                   // |v| < 2^23 assumed
    else r = sh > -25 ? (mant + (1ll << (-sh - 1))) >> (-sh) : 0ll;               // below 2^-41: 0
    if (ex == 0) r = 0;                                                            // zero, subnormals
    return (b >> 31) ? -r : r;
}
__device__ __forceinline__ void fx_add(unsigned long long* p, float v) {
    atomicAdd(p, (unsigned long long)f32_to_fx(v));
}

// Order-preserving map float -> u32 (larger float, larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace csa
