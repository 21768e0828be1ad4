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

enum Codec { Q4_K = 0, Q8_0 = 1, TQ1 = 2, Q4_0 = 3, Q5_0 = 4, Q5_1 = 5, Q6_K = 6, Q2_K = 7, Q3_K = 8, Q5_K = 9 };
enum DType { F32 = 0, F16 = 1, BF16 = 2 };

template <int C> struct CodecInfo;
template <> struct CodecInfo<Q4_K> { static constexpr int QK = 256, BYTES = 144; };
template <> struct CodecInfo<Q8_0> { static constexpr int QK = 32, BYTES = 34; };
template <> struct CodecInfo<TQ1> { static constexpr int QK = 128, BYTES = 28; };
template <> struct CodecInfo<Q4_0> { static constexpr int QK = 32, BYTES = 18; };
template <> struct CodecInfo<Q5_0> { static constexpr int QK = 32, BYTES = 22; };
template <> struct CodecInfo<Q5_1> { static constexpr int QK = 32, BYTES = 24; };
template <> struct CodecInfo<Q6_K> { static constexpr int QK = 256, BYTES = 210; };
template <> struct CodecInfo<Q2_K> { static constexpr int QK = 256, BYTES = 84; };
template <> struct CodecInfo<Q3_K> { static constexpr int QK = 256, BYTES = 110; };
template <> struct CodecInfo<Q5_K> { static constexpr int QK = 256, BYTES = 176; };

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

// ---------------------------------------------------------------- exact scalar decode
// Weight c of a weight row, rounded once to fp32 (Q4_K: fused multiply-add of
// the exact d*sc*q and dmin*m; Q8_0 and TQ1: exact).  Slow (reads the block
// header per weight): for the rare exact fallback paths only.
template <int C> __device__ __forceinline__ float weight_exact(const uint8_t* row, int64_t c);
template <> __device__ __forceinline__ float weight_exact<Q4_K>(const uint8_t* row, int64_t c) {
    const uint8_t* blk = row + (c >> 8) * 144;
    const int w = (int)(c & 255), ch = w >> 6, hi = (w >> 5) & 1;
    u32x4 h;
    const uint16_t* p16 = (const uint16_t*)blk;
    h.x = p16[0] | ((uint32_t)p16[1] << 16);
    h.y = p16[2] | ((uint32_t)p16[3] << 16);
    h.z = p16[4] | ((uint32_t)p16[5] << 16);
    h.w = p16[6] | ((uint32_t)p16[7] << 16);
    int sc, m;
    q4k_scale_min(h, 2 * ch + hi, sc, m);
    const uint32_t q = (blk[16 + 32 * ch + (w & 31)] >> (4 * hi)) & 15u;
    return __builtin_fmaf(q4k_d(h) * (float)sc, (float)q, -(q4k_dmin(h) * (float)m));
}
template <> __device__ __forceinline__ float weight_exact<Q8_0>(const uint8_t* row, int64_t c) {
    const uint8_t* blk = row + (c >> 5) * 34;
    const uint32_t d = blk[0] | ((uint32_t)blk[1] << 8);
    return half_bits_to_float(d) * (float)(int8_t)blk[2 + (c & 31)];
}
template <> __device__ __forceinline__ float weight_exact<TQ1>(const uint8_t* row, int64_t c) {
    const uint8_t* blk = row + (c >> 7) * 28;
    const int col = (int)(c & 127);
    const int slot = col < 125 ? col / 5 : 25;
    const int digit = col < 125 ? col - 5 * slot : col - 125;
    const uint32_t s = blk[26] | ((uint32_t)blk[27] << 8);
    return (float)tq1_trit(blk[slot], digit) * half_bits_to_float(s);
}

// ---------------------------------------------------------------- GGUF Q4_0 / Q5_0 / Q5_1 / Q6_K
// The further GGUF blocks of mlx-native's codec table (GgmlType::Q4_0, Q5_0,
// Q5_1, Q6_K), in the GGUF layouts (see include/kq.h).  Chunk32<C>::decode
// gives the 32 weights of chunk q of a row, each the exact value rounded
// once to fp32: w[0..15] are the weights at columns xa.., w[16..31] at xb..
// Blocks of 18, 22 and 210 bytes are only 2-byte aligned (read as 16-bit
// words); Q5_1 blocks are 8-byte aligned.
template <int C> struct Chunk32;

// Q4_0 chunk q = block q: low nibble of quant byte i is weight i, the high
// nibble weight i + 16; weight d (q - 8) (exact: 11 + 4 bits).
template <> struct Chunk32<Q4_0> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const uint16_t* blk = (const uint16_t*)(row + q * 18);
        const float d = half_bits_to_float(blk[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t pair = blk[1 + i];  // quant bytes 2i, 2i + 1
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t b = (pair >> (8 * h)) & 0xffu;
                w[2 * i + h] = d * (float)((int)(b & 15u) - 8);
                w[16 + 2 * i + h] = d * (float)((int)(b >> 4) - 8);
            }
        }
        xa = q * 32;
        xb = xa + 16;
    }
};

// Q5_0 chunk q = block q: fp16 d, qh (32 bits: bit i is weight i's fifth
// bit), nibbles as in Q4_0; weight d (q - 16) (exact).
template <> struct Chunk32<Q5_0> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const uint16_t* blk = (const uint16_t*)(row + q * 22);
        const float d = half_bits_to_float(blk[0]);
        const uint32_t qh = blk[1] | ((uint32_t)blk[2] << 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t pair = blk[3 + i];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = 2 * i + h;
                const uint32_t b = (pair >> (8 * h)) & 0xffu;
                const int q0 = (int)((b & 15u) | (((qh >> j) & 1u) << 4));
                const int q1 = (int)((b >> 4) | (((qh >> (j + 16)) & 1u) << 4));
                w[j] = d * (float)(q0 - 16);
                w[16 + j] = d * (float)(q1 - 16);
            }
        }
        xa = q * 32;
        xb = xa + 16;
    }
};

// Q5_1 chunk q = block q: fp16 d, fp16 m, qh, nibbles; weight d q + m with
// one rounding (fused).
template <> struct Chunk32<Q5_1> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const uint32_t* blk = (const uint32_t*)(row + q * 24);
        const float d = half_bits_to_float(blk[0] & 0xffffu), m = half_bits_to_float(blk[0] >> 16);
        const uint32_t qh = blk[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = blk[2 + i];  // quant bytes 4i .. 4i + 3
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int j = 4 * i + h;
                const uint32_t b = (word >> (8 * h)) & 0xffu;
                const uint32_t q0 = (b & 15u) | (((qh >> j) & 1u) << 4);
                const uint32_t q1 = (b >> 4) | (((qh >> (j + 16)) & 1u) << 4);
                w[j] = __builtin_fmaf(d, (float)q0, m);
                w[16 + j] = __builtin_fmaf(d, (float)q1, m);
            }
        }
        xa = q * 32;
        xb = xa + 16;
    }
};

// Q6_K chunk q: super-block q / 8, weights 32p .. 32p + 31 (p = q % 8), i.e.
// half h = p / 4 and run u = p % 4 of it: weight l of the run takes the low
// bits of ql[64h + l + 32 (u % 2)] (low nibble for u < 2, high for u >= 2),
// the high bits (qh[32h + l] >> 2u) & 3 and the scale scales[8h + 2u + l/16];
// value (d scale) (q - 32): d * scale is exact, the product rounds once.
template <> struct Chunk32<Q6_K> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const uint8_t* blk = row + sb * 210;
        const uint16_t* ql = (const uint16_t*)(blk + 64 * h + 32 * (u & 1));
        const uint16_t* qh = (const uint16_t*)(blk + 128 + 32 * h);
        const float d = half_bits_to_float(*(const uint16_t*)(blk + 208));
        const uint16_t scw = *(const uint16_t*)(blk + 192 + 8 * h + 2 * u);  // scales l/16 = 0, 1
        const float s0 = d * (float)(int8_t)(scw & 0xffu), s1 = d * (float)(int8_t)(scw >> 8);
        const int lsh = 4 * (u >> 1), hsh = 2 * u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t lw = ql[i], hw = qh[i];  // bytes 2i, 2i + 1 of the run
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int l = 2 * i + e;
                const uint32_t lo4 = ((lw >> (8 * e)) >> lsh) & 15u;
                const uint32_t hi2 = ((hw >> (8 * e)) >> hsh) & 3u;
                const int qv = (int)(lo4 | (hi2 << 4)) - 32;
                w[l] = (l < 16 ? s0 : s1) * (float)qv;
            }
        }
        xa = sb * 256 + 32 * p;
        xb = xa + 16;
    }
};

// The super-blocks Q2_K and Q3_K are, like Q6_K, two halves of four 32-weight
// runs: chunk q is run u = q % 4 of half h = (q / 4) % 2 of super-block q / 8,
// i.e. weights 32 (q % 8) .. + 31; weight l of the run takes bits 2u, 2u + 1
// of quant byte 32h + l and the 16-weight scale 8h + 2u + l / 16.

// Q2_K (84 bytes, 4-byte aligned): scale bytes[16] (low nibble scale, high
// nibble min), qs[64], fp16 d, fp16 dmin; weight d sc q - dmin mn with
// d sc and dmin mn exact and one fused rounding.
template <> struct Chunk32<Q2_K> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const uint8_t* blk = row + sb * 84;
        const uint32_t dd = *(const uint32_t*)(blk + 80);
        const float d = half_bits_to_float(dd & 0xffffu), dmin = half_bits_to_float(dd >> 16);
        const uint32_t scw = *(const uint16_t*)(blk + 8 * h + 2 * u);
        const uint32_t* qs = (const uint32_t*)(blk + 16 + 32 * h);
        float sc[2], mn[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t b = (scw >> (8 * i)) & 0xffu;
            sc[i] = d * (float)(b & 15u);
            mn[i] = dmin * (float)(b >> 4);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t word = qs[i] >> (2 * u);  // bytes 4i .. 4i + 3 of the run
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int l = 4 * i + e;
                const float qv = (float)((word >> (8 * e)) & 3u);
                w[l] = __builtin_fmaf(sc[l >> 4], qv, -mn[l >> 4]);
            }
        }
        xa = sb * 256 + 32 * p;
        xb = xa + 16;
    }
};

// Q3_K (110 bytes, 2-byte aligned): hmask[32], qs[64], 12 scale bytes, fp16
// d.  The third quant bit of weight l of run (h, u) is bit 4h + u of hmask[l]
// (clear: the quant is 4 lower); quants lie in -4..3.  Scale i (stored + 32)
// has its low four bits in the low nibble of scale byte i (i < 8) or the high
// nibble of byte i - 8, and its top two bits at 2 (i / 4) in byte 8 + i % 4.
// The run's two scales 8h + 2u, 8h + 2u + 1 therefore sit in the 16-bit
// words at scale bytes 2u (nibble 4h) and 8 + 2 (u % 2) (bit 2 (2h + u / 2)).
// Weight (d sc) q: both products exact.
template <> struct Chunk32<Q3_K> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const uint8_t* blk = row + sb * 110;
        const float d = half_bits_to_float(*(const uint16_t*)(blk + 108));
        const uint32_t lw = *(const uint16_t*)(blk + 96 + 2 * u);
        const uint32_t tw = *(const uint16_t*)(blk + 104 + 2 * (u & 1));
        const int tsh = 2 * (2 * h + (u >> 1));
        float sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int lo = (int)((lw >> (8 * i + 4 * h)) & 15u);
            const int top = (int)((tw >> (8 * i + tsh)) & 3u);
            sc[i] = d * (float)((lo | (top << 4)) - 32);
        }
        const uint16_t* hm = (const uint16_t*)blk;
        const uint16_t* qs = (const uint16_t*)(blk + 32 + 32 * h);
        const int hsh = 4 * h + u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t qw = qs[i], hw = hm[i];  // bytes 2i, 2i + 1 of the run
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int l = 2 * i + e;
                const int low = (int)((qw >> (8 * e + 2 * u)) & 3u);
                const int third = (int)((hw >> (8 * e + hsh)) & 1u);
                w[l] = sc[l >> 4] * (float)(low + 4 * third - 4);
            }
        }
        xa = sb * 256 + 32 * p;
        xb = xa + 16;
    }
};

// Q5_K (176 bytes, 16-byte aligned): the 16-byte Q4_K head (fp16 d, dmin,
// packed 6-bit scales and mins), qh[32], qs[128] in the Q4_K nibble order.
// Chunk q is sub-block j = q % 8 of super-block q / 8: weight l takes nibble
// j % 2 of qs[32 (j / 2) + l] and bit j of qh[l] as its fifth bit; weight
// d sc q - dmin m with one fused rounding, as Q4_K.
template <> struct Chunk32<Q5_K> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int j = (int)q & 7;
        const uint8_t* blk = row + sb * 176;
        const u32x4 hd = *(const u32x4*)blk;
        int sc, m;
        q4k_scale_min(hd, j, sc, m);
        const float s = q4k_d(hd) * (float)sc, mn = q4k_dmin(hd) * (float)m;
        const u32x4* qh = (const u32x4*)(blk + 16);
        const u32x4* qs = (const u32x4*)(blk + 48 + 32 * (j >> 1));
        const int nsh = 4 * (j & 1);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const u32x4 hv = qh[v], qv = qs[v];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int l = 16 * v + i;
                const uint32_t qb = (qv[i >> 2] >> (8 * (i & 3))) & 0xffu;
                const uint32_t hb = (hv[i >> 2] >> (8 * (i & 3))) & 0xffu;
                const uint32_t qq = ((qb >> nsh) & 15u) | (((hb >> j) & 1u) << 4);
                w[l] = __builtin_fmaf(s, (float)qq, -mn);
            }
        }
        xa = sb * 256 + 32 * j;
        xb = xa + 16;
    }
};

// One weight of the further GGUF codecs, exactly (the exact fallback of the
// prefill GEMM): its chunk decoded, the element picked.
template <int C>
__device__ __forceinline__ float weight_exact_chunk(const uint8_t* row, int64_t c) {
    float w[32];
    int64_t xa, xb;
    Chunk32<C>::decode(row, c >> 5, w, xa, xb);
    // element (c - xa) of w[0..15] or 16 + (c - xb): picked by selects, so
    // that w stays in registers
    const int i = c - xa < 16 ? (int)(c - xa) : 16 + (int)(c - xb);
    float v = w[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) v = i == j ? w[j] : v;
    return v;
}
template <> __device__ __forceinline__ float weight_exact<Q4_0>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q4_0>(row, c); }
template <> __device__ __forceinline__ float weight_exact<Q5_0>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q5_0>(row, c); }
template <> __device__ __forceinline__ float weight_exact<Q5_1>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q5_1>(row, c); }
template <> __device__ __forceinline__ float weight_exact<Q6_K>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q6_K>(row, c); }
template <> __device__ __forceinline__ float weight_exact<Q2_K>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q2_K>(row, c); }
template <> __device__ __forceinline__ float weight_exact<Q3_K>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q3_K>(row, c); }
template <> __device__ __forceinline__ float weight_exact<Q5_K>(const uint8_t* row, int64_t c) { return weight_exact_chunk<Q5_K>(row, c); }

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
// h = act(g, u) for the GLU epilogues; act is uniform over the launch:
// 0 silu(g) u, 1 gelu(g) u, 2 silu(min(g, limit)) clip(u, -limit, limit)
// (mlx-kquant "bindings.cpp", moe_glu_gather_kq act='silu_limit'; the
// comparisons keep a NaN u as NaN, and a NaN g takes the limit)
__device__ __forceinline__ float glu_act(int act, float g, float u, float limit) {
    if (act == 2) {
        const float gc = g < limit ? g : limit;
        const float uc = u < -limit ? -limit : (u > limit ? limit : u);
        return silu_fast(gc) * uc;
    }
    return (act == 1 ? gelu_tanh_fast(g) : silu_fast(g)) * u;
}

// ---------------------------------------------------------------- routing
// Expert of routed row i of a routing with S slots per token.  With a shared
// expert (shexp) the last slot of every token is expert n_experts (the shared
// expert's own matrices) and ids holds the S - 1 routed ids per token; a
// routed id >= n_experts is returned as 0xffffffff (out of range either way).
__device__ __forceinline__ uint32_t slot_expert(const uint32_t* ids, int64_t i, int64_t S,
                                                int shexp, int64_t n_experts) {
    if (!shexp) return ids[i];
    const int64_t t = i / S, r = i - t * S;
    if (r == S - 1) return (uint32_t)n_experts;
    const uint32_t e = ids[t * (S - 1) + r];
    return (int64_t)e < n_experts ? e : 0xffffffffu;
}
// Weights of expert e: the stacked experts, or the shared expert's matrix
// for e == n_experts.
__device__ __forceinline__ const uint8_t* expert_base(const uint8_t* w, const uint8_t* w_sh,
                                                      int64_t e, int64_t n_experts, int64_t stride) {
    return (w_sh && e == n_experts) ? w_sh : w + e * stride;
}

}  // namespace kq
