// q4k_mfma.h -- exact matrix-core operands of Q4_K super-blocks (shared by
// the weight-streaming kernels).
//
// Lane layout of v_mfma_f32_16x16x32_f16 as used here: the activations are
// the A operand (lane = activation row b = lane % 16, k group g = lane / 16),
// the weights the B operand (lane = weight row n = lane % 16, the same k
// group g).  Lane group g owns quant bytes 32g..32g+31 of a super-block, i.e.
// weights 64g..64g+31 (low nibbles, sub-block 2g) and 64g+32..64g+63 (high
// nibbles, sub-block 2g+1).  MFMA i (0..7) takes from every lane group the 8
// weights at 64g + 32*(i/4) + 8*(i%4) .. +7, so a chain of 8 MFMAs covers the
// super-block.
//
// The weight operand is exact: a nibble q becomes the fp16 number 1024+q (or
// 1024+16q for a high nibble) with one AND-OR, and one packed fp16 FMA with
// (sc, -1024*sc) (or (sc/16, -64*sc)) turns it into sc*q <= 945, exact in
// fp16 because the FMA is fused.  The products sc*q*x are exact in the fp32
// MFMA accumulator.  A second chain with the 6-bit min as a broadcast operand
// gives sum_k m_j(k) * x_k, and per super-block the fp32 accumulator takes
// d * chain1 - dmin * chain2.
#pragma once

#include "kq_device.h"

namespace kq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_fma16(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_fma(__builtin_bit_cast(half2_t, a),
                                                        __builtin_bit_cast(half2_t, b),
                                                        __builtin_bit_cast(half2_t, c)));
}

__device__ __forceinline__ uint32_t h2pair(float v) {
    const uint32_t b = float_to_half_bits(v);
    return b | (b << 16);
}

__device__ __forceinline__ float4_t mfma16(const u32x4& a, const u32x4& b, const float4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// (a & mask) | magic in one VALU op.  gfx9 VOP3 encodings take no literal
// and one scalar operand, so the magic constant is passed in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic_v) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic_v));
    return r;
}

// Exact MFMA weight operands of one super-block row for lane group g.
struct Q4Operands {
    u32x4 w[8];          // MFMA i: sc*q at positions 64g + 32(i/4) + 8(i%4) + 0..7
    u32x4 m_lo, m_hi;     // (m, m) fp16 pairs of sub-blocks 2g and 2g+1
    float d, dmin;
};

// Lane constants for the scale decode: which packed word holds this lane's
// two sub-blocks (2g, 2g+1), and the v_perm selector that moves their two
// bytes into the 16-bit halves.
struct LaneSel {
    bool high;      // g >= 2: sub-blocks 4..7
    uint32_t sel;   // bytes 2(g%2), 2(g%2)+1 -> halves 0, 1
};
__device__ __forceinline__ LaneSel lane_sel(int g) {
    const uint32_t b = 2u * (uint32_t)(g & 1);
    return {g >= 2, 0x0c000c00u | b | ((b + 1u) << 16)};
}

__device__ __forceinline__ void q4k_operands(const u32x4& hd, const u32x4& q0, const u32x4& q1,
                                             const LaneSel& ls, uint32_t magic_v,
                                             Q4Operands& o) {
    // all eight 6-bit scales and mins as bytes (sub-block j in byte j % 4)
    uint32_t sc_lo, sc_hi, m_lo, m_hi;
    q4k_scales_all(hd, sc_lo, sc_hi, m_lo, m_hi);
    const uint32_t scw = ls.high ? sc_hi : sc_lo, mw = ls.high ? m_hi : m_lo;
    // (sc_2g, sc_2g+1) and (m_2g, m_2g+1) as u16 pairs, then exact fp16 via
    // 1024 + v - 1024
    const uint32_t sc_u = __builtin_amdgcn_perm(scw, scw, ls.sel);
    const uint32_t m_u = __builtin_amdgcn_perm(mw, mw, ls.sel);
    const half2_t k1024 = {(half_t)1024.0f, (half_t)1024.0f};
    const half2_t sc_h = __builtin_bit_cast(half2_t, sc_u | 0x64006400u) - k1024;
    const half2_t m_h = __builtin_bit_cast(half2_t, m_u | 0x64006400u) - k1024;
    // fold constants: low nibbles (1024+q)*sc - 1024*sc; high nibbles
    // (1024+16q)*(sc/16) - 64*sc
    const half2_t f = sc_h * half2_t{(half_t)1.0f, (half_t)0.0625f};
    const half2_t gk = sc_h * half2_t{(half_t)-1024.0f, (half_t)-64.0f};
    const uint32_t f_lo = __builtin_bit_cast(uint32_t, half2_t{f[0], f[0]});
    const uint32_t f_hi = __builtin_bit_cast(uint32_t, half2_t{f[1], f[1]});
    const uint32_t g_lo = __builtin_bit_cast(uint32_t, half2_t{gk[0], gk[0]});
    const uint32_t g_hi = __builtin_bit_cast(uint32_t, half2_t{gk[1], gk[1]});
    const uint32_t ml = __builtin_bit_cast(uint32_t, half2_t{m_h[0], m_h[0]});
    const uint32_t mh = __builtin_bit_cast(uint32_t, half2_t{m_h[1], m_h[1]});
    o.m_lo = u32x4{ml, ml, ml, ml};
    o.m_hi = u32x4{mh, mh, mh, mh};
    o.d = q4k_d(hd);
    o.dmin = q4k_dmin(hd);
    const uint32_t dw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t D = dw[2 * i + half];
            // bytes (b0, b1) and (b2, b3) spread into the two 16-bit lanes
            const uint32_t p01 = __builtin_amdgcn_perm(D, D, 0x0c010c00u);
            const uint32_t p23 = __builtin_amdgcn_perm(D, D, 0x0c030c02u);
            o.w[i][2 * half] = pk_fma16(and_or(p01, 0x000f000fu, magic_v), f_lo, g_lo);
            o.w[i][2 * half + 1] = pk_fma16(and_or(p23, 0x000f000fu, magic_v), f_lo, g_lo);
            o.w[4 + i][2 * half] = pk_fma16(and_or(p01, 0x00f000f0u, magic_v), f_hi, g_hi);
            o.w[4 + i][2 * half + 1] = pk_fma16(and_or(p23, 0x00f000f0u, magic_v), f_hi, g_hi);
        }
    }
}


__device__ __forceinline__ void store_val(void* y, int64_t i, int dt, float v) {
    if (dt == F32) store_out<F32>(y, i, v);
    else if (dt == F16) store_out<F16>(y, i, v);
    else store_out<BF16>(y, i, v);
}

}  // namespace kq
