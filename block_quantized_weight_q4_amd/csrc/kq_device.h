// kq_device.h -- device-side helpers shared by the libkq kernels (gfx950).
//
// Scalar conversions, codec field access and the MFMA operand types.  Every
// decode here works on the block bytes exactly as stored (little-endian
// fields; see include/kq.h for the three formats).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Codec { Q4_K = 0, Q8_0 = 1, TQ1 = 2 };
enum DType { F32 = 0, F16 = 1, BF16 = 2 };

template <int C> struct CodecInfo;
template <> struct CodecInfo<Q4_K> { static constexpr int QK = 256, BYTES = 144; };
template <> struct CodecInfo<Q8_0> { static constexpr int QK = 32, BYTES = 34; };
template <> struct CodecInfo<TQ1> { static constexpr int QK = 128, BYTES = 28; };

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(half_t, (uint16_t)bits16);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}
// binary32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
// binary32 -> binary16 bits, round to nearest even (the hardware conversion
// in the default rounding mode), overflow to infinity.  The empty asm pins f
// as a materialized fp32 value: without it the compiler may fold a producing
// fma into a mixed-precision fma that rounds once, straight to fp16, instead
// of rounding to fp32 first and then to fp16.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    asm volatile("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (half_t)f);
}

template <int DT> __device__ __forceinline__ float load_act(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_act<F32>(const void* p, int64_t i) {
    return ((const float*)p)[i];
}
template <> __device__ __forceinline__ float load_act<F16>(const void* p, int64_t i) {
    return half_bits_to_float(((const uint16_t*)p)[i]);
}
template <> __device__ __forceinline__ float load_act<BF16>(const void* p, int64_t i) {
    return bf16_bits_to_float(((const uint16_t*)p)[i]);
}

template <int DT> __device__ __forceinline__ void store_out(void* p, int64_t i, float v);
template <> __device__ __forceinline__ void store_out<F32>(void* p, int64_t i, float v) {
    ((float*)p)[i] = v;
}
template <> __device__ __forceinline__ void store_out<F16>(void* p, int64_t i, float v) {
    ((uint16_t*)p)[i] = float_to_half_bits(v);
}
template <> __device__ __forceinline__ void store_out<BF16>(void* p, int64_t i, float v) {
    ((uint16_t*)p)[i] = float_to_bf16_bits(v);
}

// ---------------------------------------------------------------- Q4_K fields
// Header = the first 16 bytes of a super-block as four little-endian words:
// h.x = d | dmin << 16, h.y/z/w = scale bytes S[0..3], S[4..7], S[8..11].
// Sub-blocks 0..3: scale = S[j] & 63, min = S[j+4] & 63.  Sub-blocks 4..7:
// low four bits from S[j+4] (scale low nibble, min high nibble), top two bits
// from S[j-4] >> 6 (scale) and S[j] >> 6 (min).
__device__ __forceinline__ void q4k_scale_min(const u32x4& h, int j, int& sc, int& m) {
    const uint32_t s0 = h.y, s4 = h.z, s8 = h.w;
    if (j < 4) {
        sc = (s0 >> (8 * j)) & 63;
        m = (s4 >> (8 * j)) & 63;
    } else {
        const int b = 8 * (j - 4);
        sc = ((s8 >> b) & 15) | (((s0 >> (b + 6)) & 3) << 4);
        m = ((s8 >> (b + 4)) & 15) | (((s4 >> (b + 6)) & 3) << 4);
    }
}
// All eight (scale, min) pairs at once, as packed bytes: sc[j] in byte j of
// the returned 64-bit words.
__device__ __forceinline__ void q4k_scales_all(const u32x4& h, uint32_t& sc_lo, uint32_t& sc_hi,
                                               uint32_t& m_lo, uint32_t& m_hi) {
    const uint32_t s0 = h.y, s4 = h.z, s8 = h.w;
    sc_lo = s0 & 0x3f3f3f3fu;
    m_lo = s4 & 0x3f3f3f3fu;
    sc_hi = (s8 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u);
    m_hi = ((s8 >> 4) & 0x0f0f0f0fu) | ((s4 >> 2) & 0x30303030u);
}

__device__ __forceinline__ float q4k_d(const u32x4& h) { return half_bits_to_float(h.x & 0xffffu); }
__device__ __forceinline__ float q4k_dmin(const u32x4& h) { return half_bits_to_float(h.x >> 16); }

// ---------------------------------------------------------------- TQ1 digits
// Base-3 digit `d` (0..4) of a code byte, minus one: the trit in {-1,0,1}.
__device__ __forceinline__ int tq1_trit(uint32_t code, int d) {
    // code / 3^d for code <= 255 by multiply-shift (exact for these ranges).
    uint32_t q;
    switch (d) {
    case 0: q = code; break;
    case 1: q = (code * 43691u) >> 17; break;   // /3
    case 2: q = (code * 7282u) >> 16; break;    // /9
    case 3: q = (code * 2428u) >> 16; break;    // /27
    default: q = (code * 810u) >> 16; break;    // /81
    }
    const uint32_t r = q - 3u * ((q * 43691u) >> 17);  // q mod 3
    return (int)r - 1;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// GLU activations (h = act(g) * u), kq_moe_glu's KQ_ACT_SILU and
// KQ_ACT_GELU_TANH
__device__ __forceinline__ float silu_fast(float z) { return z / (1.0f + __expf(-z)); }
// gelu with the tanh approximation, z/2 (1 + tanh(y)) with y = sqrt(2/pi)
// (z + 0.044715 z^3), written as z / (1 + e^(-2y)) (the same function)
__device__ __forceinline__ float gelu_tanh_fast(float z) {
    const float y2 = 1.5957691216057308f * z * (1.0f + 0.044715f * z * z);  // 2y
    return z / (1.0f + __expf(-y2));
}
// h = act(g) * u for the GLU epilogues; act is uniform over the launch
__device__ __forceinline__ float glu_act(int act, float g, float u) {
    return (act == 1 ? gelu_tanh_fast(g) : silu_fast(g)) * u;
}

}  // namespace kq
