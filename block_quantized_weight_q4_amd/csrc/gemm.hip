// gemm.hip -- prefill product Y[M,N] = X[M,K] * dequant(W)[N,K]^T (kq_qmm).
//
// mlx-kquant "bindings.cpp", quantized_matmul; Ternary Bonsai
// "ternel_packed_model.py", tq1_gemm (decode a weight once and reuse it
// across a whole block of activation rows on the matrix units).
//
// The contraction runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation.  A
// workgroup of eight waves owns a BM x BN output tile; per K step of 64 it
// decodes its BN x 64 weight tile once into LDS (so each decoded weight feeds
// BM rows) next to the BM x 64 activation tile.  The global loads of step k+1
// are issued before the MFMAs of step k and written to LDS after them, so
// memory latency overlaps the matrix work.
//
// Operand precision (the product must stay within 2e-3 * sum|x*w| of the
// exact one for 16-bit activations):
//  - Weights are decoded exactly in fp32 and rounded once to fp16.  Q4_K and
//    Q8_0 weights are integer multiples of 2^-24 (d and dmin are fp16), so a
//    weight below 2^-14 is an exact fp16 subnormal and any other keeps 11
//    significant bits: relative error <= 2^-11 for every block whose weights
//    stay below 65520.  TQ1 weights (digit - 1) * scale are exact.
//  - fp16 activations are used as they are.  bf16 activations carry 8
//    significant bits, which fp16 holds exactly within a window of 2^31: each
//    workgroup first finds, per activation row, the largest and smallest
//    nonzero magnitude over all of K, scales the row by 2^-e so that its
//    largest magnitude lies in [2^14, 2^15), and multiplies the row's results
//    by 2^e at the store (both exact).
//  - A tile with a weight that could reach 65520 (|d| or |dmin| too large,
//    Inf or NaN) or with an activation row outside the window (a nonzero
//    range above 2^31, bf16 subnormals, Inf or NaN) is recomputed by an exact
//    fp32 path instead, so no legal input loses precision silently.
#include "kq_device.h"
#include "kq_internal.h"
#include "pair32.h"

namespace kq {

constexpr int BK = 64, LDS_STRIDE = BK + 8;  // +8 halves: rows start in different banks

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// two fp32 values -> one dword of fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_h(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, half2v));
}
__device__ __forceinline__ float16_t mma_h(const u32x4& a, const u32x4& b, float16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}
// fp16 overflows at 65520 (round to nearest even); NaN compares false
__device__ __forceinline__ bool f16_safe(float bound) { return bound < 65520.0f; }

// ---------------------------------------------------------------- weight tiles
// One thread role = (tile row r, half h): 32 of the 64 weights of row r in a
// K step.  Raw bytes are fetched into registers (Raw), then decoded into 32
// floats and the tile columns they belong to.
template <int C> struct WTile;

// Q4_K: step s is chunk c = s%4 of super-block s/4 (sub-blocks 2c, 2c+1).
// Half h: quant bytes 32c+16h..+16 -> low nibbles to columns 16h+i, high
// nibbles to 32+16h+i.
template <> struct WTile<Q4_K> {
    struct Raw { u32x4 hd, q; };
    static __device__ __forceinline__ void fetch(const uint8_t* row, int s, int h, Raw& r, bool) {
        const uint8_t* blk = row + (s >> 2) * 144;
        r.hd = *(const u32x4*)blk;
        r.q = *(const u32x4*)(blk + 16 + 32 * (s & 3) + 16 * h);
    }
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi,
                                                  bool& big) {
        const int c = s & 3;
        int sc0, m0, sc1, m1;
        q4k_scale_min(r.hd, 2 * c, sc0, m0);
        q4k_scale_min(r.hd, 2 * c + 1, sc1, m1);
        const float d = q4k_d(r.hd), dmin = q4k_dmin(r.hd);
        const float s0 = d * (float)sc0, s1 = d * (float)sc1;
        const float n0 = -dmin * (float)m0, n1 = -dmin * (float)m1;
        // high nibbles are converted in place (16 q) against s1 / 16: the
        // product is the same, and each byte converts in one instruction
        const float s1h = s1 * 0.0625f;
        big |= !f16_safe(__builtin_fabsf(s0) * 15.0f + __builtin_fabsf(n0)) ||
               !f16_safe(__builtin_fabsf(s1h) * 240.0f + __builtin_fabsf(n1));
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t ml = r.q[i] & 0x0f0f0f0fu, mh = r.q[i] & 0xf0f0f0f0u;
            // opaque to the compiler, which would otherwise fold the masks
            // into one bit-field extract per nibble
            asm("" : "+v"(ml), "+v"(mh));
#pragma unroll
            for (int b = 0; b < 4; b += 2) {
                lo[2 * i + b / 2] = pack_h(__builtin_fmaf(s0, byte(ml, b), n0),
                                           __builtin_fmaf(s0, byte(ml, b + 1), n0));
                hi[2 * i + b / 2] = pack_h(__builtin_fmaf(s1h, byte(mh, b), n1),
                                           __builtin_fmaf(s1h, byte(mh, b + 1), n1));
            }
        }
        col_lo = 16 * h;
        col_hi = 32 + 16 * h;
    }
    // Quarter q of step s: quant bytes 32c+8q..+8 -> low nibbles to columns
    // 8q+i, high nibbles to 32+8q+i.
    struct RawQ { u32x4 hd; u32x2 q; };
    static __device__ __forceinline__ void fetch_q(const uint8_t* row, int s, int q, RawQ& r, bool) {
        const uint8_t* blk = row + (s >> 2) * 144;
        r.hd = *(const u32x4*)blk;
        r.q = *(const u32x2*)(blk + 16 + 32 * (s & 3) + 8 * q);
    }
    static __device__ __forceinline__ void decode_q(const RawQ& r, int s, int q, uint32_t (&lo)[4],
                                                    uint32_t (&hi)[4], int& col_lo, int& col_hi,
                                                    bool& big) {
        const int c = s & 3;
        int sc0, m0, sc1, m1;
        q4k_scale_min(r.hd, 2 * c, sc0, m0);
        q4k_scale_min(r.hd, 2 * c + 1, sc1, m1);
        const float d = q4k_d(r.hd), dmin = q4k_dmin(r.hd);
        const float s0 = d * (float)sc0, s1h = d * (float)sc1 * 0.0625f;
        const float n0 = -dmin * (float)m0, n1 = -dmin * (float)m1;
        big |= !f16_safe(__builtin_fabsf(s0) * 15.0f + __builtin_fabsf(n0)) ||
               !f16_safe(__builtin_fabsf(s1h) * 240.0f + __builtin_fabsf(n1));
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t ml = r.q[i] & 0x0f0f0f0fu, mh = r.q[i] & 0xf0f0f0f0u;
            asm("" : "+v"(ml), "+v"(mh));
#pragma unroll
            for (int b = 0; b < 4; b += 2) {
                lo[2 * i + b / 2] = pack_h(__builtin_fmaf(s0, byte(ml, b), n0),
                                           __builtin_fmaf(s0, byte(ml, b + 1), n0));
                hi[2 * i + b / 2] = pack_h(__builtin_fmaf(s1h, byte(mh, b), n1),
                                           __builtin_fmaf(s1h, byte(mh, b + 1), n1));
            }
        }
        col_lo = 8 * q;
        col_hi = 32 + 8 * q;
    }
};

// Q8_0: step s covers blocks 2s, 2s+1 (68 contiguous, 4-byte aligned bytes);
// half h reads exactly its 34-byte block: h = 0 takes dwords 0..7 and the
// 16-bit word at byte 32; h = 1 the 16-bit word at byte 34 (its scale) and
// dwords 9..16 (its quants, dword aligned).
template <> struct WTile<Q8_0> {
    struct Raw { uint32_t w[8]; uint32_t tail; };
    // Rows start on a 4-byte boundary only when the row size is a multiple of
    // 4 bytes (an even number of blocks); otherwise the block is read as
    // 16-bit words.
    static __device__ __forceinline__ void fetch(const uint8_t* row, int s, int h, Raw& r,
                                                 bool rows_4b_aligned) {
        const uint8_t* base = row + 68 * s;
        if (rows_4b_aligned) {
            const uint32_t* p = (const uint32_t*)base + (h ? 9 : 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) r.w[i] = p[i];
        } else {
            const uint16_t* p = (const uint16_t*)base + (h ? 18 : 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) r.w[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
        }
        r.tail = *(const uint16_t*)(base + (h ? 34 : 32));
    }
    // Both halves decode with the same instructions (the half differs per
    // lane): the words [w0..w7, tail] shifted right by 16 bits (h = 0, whose
    // quants start at byte 2) or not at all (h = 1) give the 32 quants in
    // order.  A quant byte xor 0x80 is q + 128, converted in one instruction,
    // and fma(d, q + 128, -128 d) is d q exactly (a zero weight comes out as
    // +0 whatever the sign of d).
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi,
                                                  bool& big) {
        uint32_t sh = h ? 0u : 16u;
        asm("" : "+v"(sh));  // one funnel shift by a register, not two selected
        const float d = half_bits_to_float(h ? r.tail : (r.w[0] & 0xffffu));
        const float nd = -128.0f * d;
        big |= !f16_safe(__builtin_fabsf(nd));
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
        uint32_t v[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t next = j < 7 ? r.w[j + 1] : r.tail;
            const uint32_t u = __builtin_amdgcn_alignbit(next, r.w[j], sh) ^ 0x80808080u;
            v[2 * j] = pack_h(__builtin_fmaf(d, byte(u, 0), nd), __builtin_fmaf(d, byte(u, 1), nd));
            v[2 * j + 1] = pack_h(__builtin_fmaf(d, byte(u, 2), nd), __builtin_fmaf(d, byte(u, 3), nd));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) lo[i] = v[i], hi[i] = v[8 + i];
        col_lo = 32 * h;
        col_hi = 32 * h + 16;
    }
    // Quarter q of step s: quants 16 (q%2) .. +15 of block q/2, i.e. columns
    // 16q .. 16q+15.  Block 0's quants start 2 bytes past a word, so its four
    // words are shifted by 16 bits with the first half-word after them;
    // block 1's quants start on a word.
    struct RawQ { uint32_t w[4]; uint32_t next; uint32_t sc; };
    static __device__ __forceinline__ void fetch_q(const uint8_t* row, int s, int q, RawQ& r,
                                                   bool rows_4b_aligned) {
        const int h = q >> 1, hh = q & 1;
        const uint8_t* blk = row + 68 * s + 34 * h;
        const uint8_t* qb = blk + 16 * hh + (h ? 2 : 0);
        if (rows_4b_aligned) {
            const uint32_t* p = (const uint32_t*)qb;
#pragma unroll
            for (int i = 0; i < 4; ++i) r.w[i] = p[i];
        } else {
            const uint16_t* p = (const uint16_t*)qb;
#pragma unroll
            for (int i = 0; i < 4; ++i) r.w[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
        }
        r.next = *(const uint16_t*)(blk + 16 + 16 * hh);
        r.sc = *(const uint16_t*)blk;
    }
    static __device__ __forceinline__ void decode_q(const RawQ& r, int s, int q, uint32_t (&lo)[4],
                                                    uint32_t (&hi)[4], int& col_lo, int& col_hi,
                                                    bool& big) {
        uint32_t sh = (q >> 1) ? 0u : 16u;
        asm("" : "+v"(sh));
        const float d = half_bits_to_float(r.sc);
        const float nd = -128.0f * d;
        big |= !f16_safe(__builtin_fabsf(nd));
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
        uint32_t v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t next = j < 3 ? r.w[j + 1] : r.next;
            const uint32_t u = __builtin_amdgcn_alignbit(next, r.w[j], sh) ^ 0x80808080u;
            v[2 * j] = pack_h(__builtin_fmaf(d, byte(u, 0), nd), __builtin_fmaf(d, byte(u, 1), nd));
            v[2 * j + 1] = pack_h(__builtin_fmaf(d, byte(u, 2), nd), __builtin_fmaf(d, byte(u, 3), nd));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = v[i], hi[i] = v[4 + i];
        col_lo = 16 * q;
        col_hi = 16 * q + 8;
    }
};

// TQ1_G128: step s is half s%2 of group s/2; half h takes the group's columns
// 32*qi .. 32*qi+31 with qi = 2*(s%2) + h.  Column c < 125 is digit c%5 of
// code byte c/5, columns 125..127 digits of the tail byte; w = (digit-1)*s.
template <> struct WTile<TQ1> {
    struct Raw { uint32_t w[7]; };
    static __device__ __forceinline__ void fetch(const uint8_t* row, int s, int h, Raw& r, bool) {
        const uint32_t* p = (const uint32_t*)(row + (s >> 1) * 28);
#pragma unroll
        for (int i = 0; i < 7; ++i) r.w[i] = p[i];
    }
    // Digits two at a time with packed 16-bit integer arithmetic.  A code byte c (<= 242) in fixed point, q = ceil(256 c /
    // 243), holds its base-3 digits as a fraction: digit k is the integer part
    // of 3 * ((q * 3^(4-k)) mod 256) / 256.  With the digit placed in the low
    // byte of the fp16 1024 (0x6400 | d), subtracting 1025 gives d - 1 exactly,
    // and the product with the fp16 scale is exact as well.
    // Column pairs C0 + 2i, C0 + 2i + 1 (i < NP) of the block.
    template <int C0, int NP>
    static __device__ __forceinline__ void cols_f16(const Raw& r, uint32_t (&v)[NP]) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
        constexpr int CL = C0 + 2 * NP - 1;  // last column
        constexpr int B0 = C0 / 5, B1 = CL < 125 ? CL / 5 : 25;
        uint32_t q[B1 - B0 + 1];
#pragma unroll
        for (int b = B0; b <= B1; ++b) {
            const uint32_t c = (r.w[b >> 2] >> (8 * (b & 3))) & 0xffu;
            q[b - B0] = (c * 17261u + 16240u) >> 14;  // ceil(256 c / 243) for c <= 255
        }
        const uint32_t scb = r.w[6] >> 16;
        const h16x2 sc2 = __builtin_bit_cast(h16x2, scb | (scb << 16));
        const h16x2 off = {(_Float16)-1025.0f, (_Float16)-1025.0f};
        constexpr uint32_t kPow3[5] = {1u, 3u, 9u, 27u, 81u};
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int col = C0 + 2 * i;
            const int b = col < 125 ? col / 5 : 25;
            const int dg = col < 125 ? col - 5 * b : col - 125;
            uint32_t qq, mm;
            if (dg <= 3) {  // both columns in byte b: digits dg, dg + 1
                qq = q[b - B0] * 0x10001u;
                mm = kPow3[4 - dg] | (kPow3[3 - dg] << 16);
            } else {        // digit 4 of byte b, digit 0 of byte b + 1
                qq = q[b - B0] | (q[b + 1 - B0] << 16);
                mm = 1u | (81u << 16);
            }
            u16x2 t = __builtin_bit_cast(u16x2, qq) * __builtin_bit_cast(u16x2, mm);
            t = __builtin_bit_cast(u16x2, __builtin_bit_cast(uint32_t, t) & 0x00ff00ffu) * (u16x2){3, 3};
            // [high byte of each half | 0x64]: 1024 + digit in fp16
            const uint32_t h = __builtin_amdgcn_perm(0x64646464u, __builtin_bit_cast(uint32_t, t), 0x04030401u);
            v[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(h16x2, h) + off) * sc2);
        }
    }
    // (weights are at most |scale| and never overflow fp16; Inf and NaN scales
    // give the same Inf and NaN products as the exact values)
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi,
                                                  bool&) {
        uint32_t v[16];
        switch (2 * (s & 1) + h) {
        case 0: cols_f16<0, 16>(r, v); break;
        case 1: cols_f16<32, 16>(r, v); break;
        case 2: cols_f16<64, 16>(r, v); break;
        default: cols_f16<96, 16>(r, v); break;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) lo[i] = v[i], hi[i] = v[8 + i];
        col_lo = 32 * h;
        col_hi = 32 * h + 16;
    }
    // Quarter q of step s: columns 16e..16e+15 of the block, e = 4 (s%2) + q.
    using RawQ = Raw;
    static __device__ __forceinline__ void fetch_q(const uint8_t* row, int s, int, RawQ& r, bool) {
        fetch(row, s, 0, r, true);
    }
    static __device__ __forceinline__ void decode_q(const RawQ& r, int s, int q, uint32_t (&lo)[4],
                                                    uint32_t (&hi)[4], int& col_lo, int& col_hi,
                                                    bool&) {
        uint32_t v[8];
        switch (4 * (s & 1) + q) {
        case 0: cols_f16<0, 8>(r, v); break;
        case 1: cols_f16<16, 8>(r, v); break;
        case 2: cols_f16<32, 8>(r, v); break;
        case 3: cols_f16<48, 8>(r, v); break;
        case 4: cols_f16<64, 8>(r, v); break;
        case 5: cols_f16<80, 8>(r, v); break;
        case 6: cols_f16<96, 8>(r, v); break;
        default: cols_f16<112, 8>(r, v); break;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = v[i], hi[i] = v[4 + i];
        col_lo = 16 * q;
        col_hi = 16 * q + 8;
    }
};

// The further GGUF codecs (Q4_0, Q5_0, Q5_1, Q6_K, Q2_K, Q3_K, Q5_K; layouts
// as in include/kq.h): half h of step s is the 32-weight chunk q = 2s + h of
// the row, i.e. columns 32h .. 32h + 31 of the step.  fetch() takes the
// chunk's fields into registers; decode() forms the 32 weights exactly in
// fp32 (one rounding for the codecs with an offset: Q5_1, Q2_K, Q5_K) and
// rounds each once to fp16; a weight that could reach 65520, or a NaN, sends
// the tile to the exact path.  Chunk q of a 32-weight codec is block q; of a
// 256-weight codec it is run q % 8 of super-block q / 8.
template <int C> struct GRaw;
template <int C> struct GChunk;

template <> struct GRaw<Q4_0> { uint32_t d, qs[4]; };
template <> struct GChunk<Q4_0> {
    static __device__ __forceinline__ void fetch(const uint8_t* row, int64_t q, GRaw<Q4_0>& r) {
        const uint8_t* blk = row + q * 18;
        r.d = *(const uint16_t*)blk;
        words<false>(blk + 2, r.qs);
    }
    static __device__ __forceinline__ void decode(const GRaw<Q4_0>& r, int64_t, float (&w)[32]) {
        const float d = half_bits_to_float(r.d);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t b = (r.qs[j >> 2] >> (8 * (j & 3))) & 0xffu;
            w[j] = d * (float)((int)(b & 15u) - 8);
            w[16 + j] = d * (float)((int)(b >> 4) - 8);
        }
    }
};

// Q5_0 and Q5_1: [qh, qs[4]] after d (and m)
template <> struct GRaw<Q5_0> { uint32_t d, v[5]; };
template <> struct GRaw<Q5_1> { uint32_t dm, v[5]; };
template <int C> struct GChunkQ5 {
    static __device__ __forceinline__ void fetch(const uint8_t* row, int64_t q, GRaw<C>& r) {
        const uint8_t* blk = row + q * (C == Q5_0 ? 22 : 24);
        if constexpr (C == Q5_0) {
            r.d = *(const uint16_t*)blk;
            words<false>(blk + 2, r.v);
        } else {
            r.dm = (uint32_t)((const uint16_t*)blk)[0] | ((uint32_t)((const uint16_t*)blk)[1] << 16);
            words<false>(blk + 4, r.v);
        }
    }
    static __device__ __forceinline__ void decode(const GRaw<C>& r, int64_t, float (&w)[32]) {
        float d, m = 0.f;
        if constexpr (C == Q5_0) d = half_bits_to_float(r.d);
        else d = half_bits_to_float(r.dm & 0xffffu), m = half_bits_to_float(r.dm >> 16);
        const uint32_t qh = r.v[0];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t b = (r.v[1 + (j >> 2)] >> (8 * (j & 3))) & 0xffu;
            const uint32_t q0 = (b & 15u) | (((qh >> j) & 1u) << 4);
            const uint32_t q1 = (b >> 4) | (((qh >> (j + 16)) & 1u) << 4);
            if constexpr (C == Q5_0) {
                w[j] = d * (float)((int)q0 - 16);
                w[16 + j] = d * (float)((int)q1 - 16);
            } else {
                w[j] = __builtin_fmaf(d, (float)q0, m);
                w[16 + j] = __builtin_fmaf(d, (float)q1, m);
            }
        }
    }
};
template <> struct GChunk<Q5_0> : GChunkQ5<Q5_0> {};
template <> struct GChunk<Q5_1> : GChunkQ5<Q5_1> {};

// Q6_K run (h, u): ql and qh bytes of the run, the run's two scales, d
template <> struct GRaw<Q6_K> { uint32_t ql[8], qh[8], sc, d; };
template <> struct GChunk<Q6_K> {
    static __device__ __forceinline__ void fetch(const uint8_t* row, int64_t q, GRaw<Q6_K>& r) {
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const uint8_t* blk = row + (q >> 3) * 210;
        words<false>(blk + 64 * h + 32 * (u & 1), r.ql);
        words<false>(blk + 128 + 32 * h, r.qh);
        r.sc = *(const uint16_t*)(blk + 192 + 8 * h + 2 * u);
        r.d = *(const uint16_t*)(blk + 208);
    }
    static __device__ __forceinline__ void decode(const GRaw<Q6_K>& r, int64_t q, float (&w)[32]) {
        const int u = (int)q & 3;
        const float d = half_bits_to_float(r.d);
        const float s0 = d * (float)(int8_t)(r.sc & 0xffu), s1 = d * (float)(int8_t)(r.sc >> 8);
        const int lsh = 4 * (u >> 1), hsh = 2 * u;
#pragma unroll
        for (int l = 0; l < 32; ++l) {
            const uint32_t lo4 = (r.ql[l >> 2] >> (8 * (l & 3) + lsh)) & 15u;
            const uint32_t hi2 = (r.qh[l >> 2] >> (8 * (l & 3) + hsh)) & 3u;
            w[l] = (l < 16 ? s0 : s1) * (float)((int)(lo4 | (hi2 << 4)) - 32);
        }
    }
};

// Q2_K run (h, u): the half's quant bytes, the run's scale/min bytes, d and dmin
template <> struct GRaw<Q2_K> { uint32_t qs[8], sc, dd; };
template <> struct GChunk<Q2_K> {
    static __device__ __forceinline__ void fetch(const uint8_t* row, int64_t q, GRaw<Q2_K>& r) {
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const uint8_t* blk = row + (q >> 3) * 84;
        words<false>(blk + 16 + 32 * h, r.qs);
        r.sc = *(const uint16_t*)(blk + 8 * h + 2 * u);
        r.dd = (uint32_t)((const uint16_t*)(blk + 80))[0] | ((uint32_t)((const uint16_t*)(blk + 80))[1] << 16);
    }
    static __device__ __forceinline__ void decode(const GRaw<Q2_K>& r, int64_t q, float (&w)[32]) {
        const int u = (int)q & 3;
        const float d = half_bits_to_float(r.dd & 0xffffu), dmin = half_bits_to_float(r.dd >> 16);
        float sc[2], mn[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t b = (r.sc >> (8 * i)) & 0xffu;
            sc[i] = d * (float)(b & 15u);
            mn[i] = dmin * (float)(b >> 4);
        }
#pragma unroll
        for (int l = 0; l < 32; ++l) {
            const float qv = (float)((r.qs[l >> 2] >> (8 * (l & 3) + 2 * u)) & 3u);
            w[l] = __builtin_fmaf(sc[l >> 4], qv, -mn[l >> 4]);
        }
    }
};

// Q3_K run (h, u): hmask and the half's quant bytes, the two scale words, d
template <> struct GRaw<Q3_K> { uint32_t hm[8], qs[8], lw, tw, d; };
template <> struct GChunk<Q3_K> {
    static __device__ __forceinline__ void fetch(const uint8_t* row, int64_t q, GRaw<Q3_K>& r) {
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const uint8_t* blk = row + (q >> 3) * 110;
        words<false>(blk, r.hm);
        words<false>(blk + 32 + 32 * h, r.qs);
        r.lw = *(const uint16_t*)(blk + 96 + 2 * u);
        r.tw = *(const uint16_t*)(blk + 104 + 2 * (u & 1));
        r.d = *(const uint16_t*)(blk + 108);
    }
    static __device__ __forceinline__ void decode(const GRaw<Q3_K>& r, int64_t q, float (&w)[32]) {
        const int p = (int)q & 7, h = p >> 2, u = p & 3;
        const float d = half_bits_to_float(r.d);
        const int tsh = 2 * (2 * h + (u >> 1));
        float sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int lo = (int)((r.lw >> (8 * i + 4 * h)) & 15u);
            const int top = (int)((r.tw >> (8 * i + tsh)) & 3u);
            sc[i] = d * (float)((lo | (top << 4)) - 32);
        }
        const int hsh = 4 * h + u;
#pragma unroll
        for (int l = 0; l < 32; ++l) {
            const int low = (int)((r.qs[l >> 2] >> (8 * (l & 3) + 2 * u)) & 3u);
            const int third = (int)((r.hm[l >> 2] >> (8 * (l & 3) + hsh)) & 1u);
            w[l] = sc[l >> 4] * (float)(low + 4 * third - 4);
        }
    }
};

// Q5_K sub-block j: the 16-byte head, qh[32], the sub-block's 32 nibble bytes
template <> struct GRaw<Q5_K> { u32x4 hd, qh0, qh1, qs0, qs1; };
template <> struct GChunk<Q5_K> {
    static __device__ __forceinline__ void fetch(const uint8_t* row, int64_t q, GRaw<Q5_K>& r) {
        const int j = (int)q & 7;
        const uint8_t* blk = row + (q >> 3) * 176;
        r.hd = *(const u32x4*)blk;
        r.qh0 = *(const u32x4*)(blk + 16);
        r.qh1 = *(const u32x4*)(blk + 32);
        r.qs0 = *(const u32x4*)(blk + 48 + 32 * (j >> 1));
        r.qs1 = *(const u32x4*)(blk + 64 + 32 * (j >> 1));
    }
    static __device__ __forceinline__ void decode(const GRaw<Q5_K>& r, int64_t q, float (&w)[32]) {
        const int j = (int)q & 7;
        int sc, m;
        q4k_scale_min(r.hd, j, sc, m);
        const float s = q4k_d(r.hd) * (float)sc, mn = q4k_dmin(r.hd) * (float)m;
        const int nsh = 4 * (j & 1);
#pragma unroll
        for (int l = 0; l < 32; ++l) {
            const uint32_t qb = ((l < 16 ? r.qs0 : r.qs1)[(l & 15) >> 2] >> (8 * (l & 3))) & 0xffu;
            const uint32_t hb = ((l < 16 ? r.qh0 : r.qh1)[(l & 15) >> 2] >> (8 * (l & 3))) & 0xffu;
            const uint32_t qq = ((qb >> nsh) & 15u) | (((hb >> j) & 1u) << 4);
            w[l] = __builtin_fmaf(s, (float)qq, -mn);
        }
    }
};

// Q4_0, Q5_0, Q5_1 straight to fp16 pairs: the integer v (q - 8, q - 16 or
// q) is exact in fp16 (1024 + q under the exponent pattern, minus the
// offset), and one packed fp16 multiply by d (or fma with d and m) forms each
// weight exactly and rounds it once, as the fp32 form would.  A weight that
// could reach 65520 (|d| times the largest |v|, plus |m|), or a NaN scale,
// sends the tile to the exact path.
template <int C>
__device__ __forceinline__ void legacy_pairs(const GRaw<C>& r, uint32_t (&lo)[8], uint32_t (&hi)[8],
                                             bool& big) {
    uint32_t qh = 0, dbits, mbits = 0;
    const uint32_t* qs;
    if constexpr (C == Q4_0) {
        dbits = r.d, qs = r.qs;
    } else if constexpr (C == Q5_0) {
        dbits = r.d, qh = r.v[0], qs = r.v + 1;
    } else {
        dbits = r.dm & 0xffffu, mbits = r.dm >> 16, qh = r.v[0], qs = r.v + 1;
    }
    const float d = half_bits_to_float(dbits), mf = half_bits_to_float(mbits);
    constexpr float vmax = C == Q4_0 ? 8.0f : C == Q5_0 ? 16.0f : 31.0f;
    big |= !f16_safe(__builtin_fabsf(d) * vmax + __builtin_fabsf(mf));
    const h2_t off = h2(C == Q4_0 ? 1032.f : C == Q5_0 ? 1040.f : 1024.f);
    const h2_t d2 = __builtin_bit_cast(h2_t, dbits | (dbits << 16));
    const h2_t m2 = __builtin_bit_cast(h2_t, mbits | (mbits << 16));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t l = qs[i] & 0x0f0f0f0fu, u = (qs[i] >> 4) & 0x0f0f0f0fu;
        if constexpr (C != Q4_0) {
            l |= spread4((qh >> (4 * i)) & 15u) << 4;
            u |= spread4((qh >> (16 + 4 * i)) & 15u) << 4;
        }
        uint32_t v[4];
        bytes_to_pairs(l, off, v[0], v[1]);
        bytes_to_pairs(u, off, v[2], v[3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h2_t vv = __builtin_bit_cast(h2_t, v[j]);
            v[j] = __builtin_bit_cast(uint32_t, C == Q5_1 ? __builtin_elementwise_fma(vv, d2, m2) : vv * d2);
        }
        lo[2 * i] = v[0], lo[2 * i + 1] = v[1], hi[2 * i] = v[2], hi[2 * i + 1] = v[3];
    }
}

template <int C> struct WTileGguf {
    using Raw = GRaw<C>;
    using RawQ = GRaw<C>;  // (quarters are not used for these codecs)
    static __device__ __forceinline__ void fetch(const uint8_t* row, int s, int h, Raw& r, bool) {
        GChunk<C>::fetch(row, 2 * (int64_t)s + h, r);
    }
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi,
                                                  bool& big) {
        if constexpr (C == Q4_0 || C == Q5_0 || C == Q5_1) {
            legacy_pairs<C>(r, lo, hi, big);
        } else {
            float w[32];
            GChunk<C>::decode(r, 2 * (int64_t)s + h, w);
            bool ok = true;
#pragma unroll
            for (int i = 0; i < 32; ++i) ok &= __builtin_fabsf(w[i]) < 65520.0f;  // false for NaN
            big |= !ok;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo[i] = pack_h(w[2 * i], w[2 * i + 1]);
                hi[i] = pack_h(w[16 + 2 * i], w[17 + 2 * i]);
            }
        }
        col_lo = 32 * h;
        col_hi = 32 * h + 16;
    }
};
template <> struct WTile<Q4_0> : WTileGguf<Q4_0> {};
template <> struct WTile<Q5_0> : WTileGguf<Q5_0> {};
template <> struct WTile<Q5_1> : WTileGguf<Q5_1> {};
template <> struct WTile<Q6_K> : WTileGguf<Q6_K> {};
template <> struct WTile<Q2_K> : WTileGguf<Q2_K> {};
template <> struct WTile<Q3_K> : WTileGguf<Q3_K> {};
template <> struct WTile<Q5_K> : WTileGguf<Q5_K> {};

constexpr bool is_gguf(int c) { return c >= Q4_0; }

// The per-step weight registers: halves (Raw) or quarters (RawQ).
template <bool Q, class WT> struct RawSel { using type = typename WT::Raw; };
template <class WT> struct RawSel<true, WT> { using type = typename WT::RawQ; };

// Activation modes of the GEMM kernel.
enum XMode {
    XM_F16 = 0,     // fp16 activations, used as they are
    XM_BF16 = 1,    // bf16 activations, row exponents found by each workgroup
    XM_SCALED = 2,  // fp16 rows pre-scaled by 2^-e, exponents in GemmArgs::xexp
};
constexpr int32_t kBadRow = INT32_MIN;  // an activation row outside the fp16 window

// The exact path of one tile: every output is the fp32 sum, in column
// order, of the exact activation (fp32) times the weight decoded exactly to
// fp32, with no fp16 operand.  Slow (each thread decodes its weight row once
// per group of eight activation rows); taken only by tiles whose weights or
// activations do not fit the fp16 operands.  Covers columns [c0, c1) of K
// (the workgroup's share when K is split).
template <int C, int BM, int BN, int NT>
__device__ __forceinline__ void gemm_tile_exact(const GemmArgs& a, int64_t row_bytes, int64_t m0,
                                                int64_t n0, int64_t c0, int64_t c1, int tid) {
    constexpr int RS = NT / BN;  // threads per weight row
    static_assert(RS >= 1 && NT % BN == 0, "tile shape");
    const int64_t gn = n0 + tid % BN;
    if (gn >= a.n) return;
    const uint8_t* wr = a.w + gn * row_bytes;
    float* part = a.part && gridDim.z > 1 ? a.part + (int64_t)blockIdx.z * a.m * a.n : nullptr;
    for (int r0 = tid / BN; r0 < BM; r0 += 8 * RS) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int64_t c = c0; c < c1; ++c) {
            const float wv = weight_exact<C>(wr, c);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t gm = m0 + r0 + RS * j;
                if (r0 + RS * j < BM && gm < a.m) {
                    const float xv = a.x_src_dt == BF16 ? load_act<BF16>(a.x_src, gm * a.k + c)
                                                        : load_act<F16>(a.x_src, gm * a.k + c);
                    acc[j] = __builtin_fmaf(xv, wv, acc[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t gm = m0 + r0 + RS * j;
            if (r0 + RS * j >= BM || gm >= a.m) continue;
            if (part) part[gm * a.n + gn] = acc[j];
            else if (a.y_dt == F32) store_out<F32>(a.y, gm * a.n + gn, acc[j]);
            else if (a.y_dt == F16) store_out<F16>(a.y, gm * a.n + gn, acc[j]);
            else store_out<BF16>(a.y, gm * a.n + gn, acc[j]);
        }
    }
}

template <int C, int XM, int BM, int BN, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW) void gemm_kernel(const GemmArgs a) {
    constexpr int NT = 64 * NW, WN = NW / 2;
    constexpr int TM = BM / 2, TN = BN / WN, FM = TM / 32, FN = TN / 32;
    static_assert(FM >= 1 && FN >= 1 && 2 * BN <= NT, "tile shape");
    constexpr int XP = BM * 8 / NT;  // 16-byte activation pieces per thread per step
    constexpr int ASZ = BM * LDS_STRIDE, BSZ = BN * LDS_STRIDE;
    constexpr bool ROWEXP = XM != XM_F16;  // results are scaled by 2^e per row
    using WT = WTile<C>;
    // two stages of [activation tile | weight tile]
    __shared__ __align__(16) uint16_t lds[2 * (ASZ + BSZ)];
    // scaled activations: each tile row's exponent e (results x 2^e)
    __shared__ int32_t xe_lds[ROWEXP ? BM : 1];
    __shared__ int32_t exact_flag;  // the tile takes the exact path
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t n = a.n, k = a.k, m = a.m;
    const uint16_t* __restrict__ x = a.x;
    const uint8_t* __restrict__ w = a.w;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
    const int64_t row_bytes = (k / CodecInfo<C>::QK) * CodecInfo<C>::BYTES;
    // this workgroup's K steps: [sb, sb + steps) of the whole product's
    const int total_steps = (int)((k + BK - 1) / BK);
    const int sb = SPLIT ? (int)blockIdx.z * a.split_steps : 0;
    const int steps = !SPLIT ? total_steps
                      : total_steps - sb < a.split_steps ? total_steps - sb : a.split_steps;

    // weight role: tile row wr and part wh of each step, a half (wh < 2) or,
    // when the threads are four times the tile's rows, a quarter (wh < 4), so
    // that every wave shares the decoding.  Q8_0 takes quarters only in
    // tiles of at most 128 activation rows (7-8 % faster there, 3-6 %
    // slower in the 256-row tiles, where half the threads decoding keeps the
    // rest on matrix work).  Neighbouring threads read the parts of one row
    // (contiguous bytes), except for TQ1, whose decoding branches on the
    // part: there each wave holds one part, so it runs one branch (measured
    // faster for TQ1, slower for the others).
    constexpr bool QM = 4 * BN == NT && (C != Q8_0 || BM <= 128) && !is_gguf(C);
    constexpr int NPART = QM ? 4 : 2;
    constexpr bool kWaveParts = C == TQ1;
    // codecs of 32-weight blocks: a row of an odd block count ends half way
    // through its last step
    constexpr bool HALF_TAIL = C == Q8_0 || C == Q4_0 || C == Q5_0 || C == Q5_1;
    const int wr = kWaveParts ? tid % BN : tid / NPART, wh = kWaveParts ? tid / BN : tid % NPART;
    const bool wrole = tid < NPART * BN;
    const int64_t wrow_idx = n0 + wr;
    const bool wr_valid = wrole && wrow_idx < n;
    const uint8_t* wrow = w + (wrow_idx < n ? wrow_idx : n - 1) * row_bytes;

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = float16_t{};

    // A thread stages 16-byte pieces p = tid + NT i (i < XP) of each step:
    // tile row p / 8, columns 8 (p % 8) .. +7.  The eight threads of one row
    // are eight neighbouring lanes of one wave.
    if (tid == 0) exact_flag = 0;
    __syncthreads();  // before any thread may raise it
    if constexpr (XM == XM_SCALED) {
        for (int r = tid; r < BM; r += NT) {
            const int32_t e = m0 + r < m ? a.xexp[m0 + r] : 0;
            xe_lds[r] = e == kBadRow ? 0 : e;
            if (e == kBadRow) exact_flag = 1;
        }
        __syncthreads();
    }
    if constexpr (XM == XM_BF16) {
        // Per row: the largest and the smallest nonzero magnitude over all of
        // K, as bf16 bit patterns without the sign (ordered like the values).
        // Packed 16-bit max/min over both halves of each dword; the minimum
        // runs over magnitude - 1, so a zero wraps to 0xffff and is ignored.
        u16x2 mx[XP], mn[XP];
#pragma unroll
        for (int i = 0; i < XP; ++i) mx[i] = u16x2{0, 0}, mn[i] = u16x2{0xffff, 0xffff};
        for (int s = 0; s < steps; ++s) {
#pragma unroll
            for (int i = 0; i < XP; ++i) {
                const int p = tid + NT * i, r = p >> 3, q = p & 7;
                const int64_t gm = m0 + r, c0 = (int64_t)s * BK + 8 * q;
                if (gm < m && c0 < k) {
                    const u32x4 v = *(const u32x4*)(x + gm * k + c0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u16x2 mag = __builtin_bit_cast(u16x2, v[j] & 0x7fff7fffu);
                        mx[i] = __builtin_elementwise_max(mx[i], mag);
                        mn[i] = __builtin_elementwise_min(mn[i], mag - u16x2{1, 1});
                    }
                }
            }
        }
        bool bad = false;
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            uint32_t hi = mx[i][0] > mx[i][1] ? mx[i][0] : mx[i][1];
            uint32_t lo = mn[i][0] < mn[i][1] ? mn[i][0] : mn[i][1];
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) {
                const uint32_t h2 = __shfl_xor(hi, off, 64), l2 = __shfl_xor(lo, off, 64);
                hi = h2 > hi ? h2 : hi;
                lo = l2 < lo ? l2 : lo;
            }
            // exponent fields of the largest and smallest nonzero magnitudes
            const int emax = (int)(hi >> 7), emin = (int)((lo + 1u) >> 7);
            const bool any = hi != 0u;
            const bool row_bad = any && (emax == 255 || emin == 0 || emax - emin > 31);
            const int e = any ? emax - 127 - 14 : 0;
            const int p = tid + NT * i;
            if ((p & 7) == 0) xe_lds[p >> 3] = e;
            bad |= row_bad;
        }
        if (bad) exact_flag = 1;
        __syncthreads();
    }
    bool wbig = false;  // a decoded weight could overflow fp16

    // registers holding the fetched-but-not-stashed step
    struct Regs {
        u32x4 xr[XP];
        typename RawSel<QM, WT>::type raw;
    };
    Regs ra;
    // With every thread owning a weight role (2 BN, or 4 BN in quarters, ==
    // threads) the step is branch-free: out-of-range pieces are read from a
    // valid address and replaced by zeros with selects, so the whole K step
    // is one scheduling region in which loads, decoding and MFMAs can
    // interleave.
    constexpr bool FULL = 2 * BN == NT || QM;
    auto fetch = [&](int sr, Regs& R) {
        const int s = sb + sr;  // step of the whole product
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + NT * i, r = p >> 3, q = p & 7;
            const int64_t gm = m0 + r;
            const int64_t c0 = (int64_t)s * BK + 8 * q;
            if (FULL) {
                // rows past m read row 0; for Q4_K and TQ1 (K a multiple of
                // the step) they are left as read, since they only reach
                // output rows that are not stored.  Q8_0 zeroes them and the
                // columns past k (rows of an odd block count), which keeps
                // its scheduling measured faster.
                const bool ok = gm < m && c0 < k;
                const u32x4 v = *(const u32x4*)(x + (ok ? gm * k + c0 : 0));
                R.xr[i] = (!HALF_TAIL || ok) ? v : u32x4{0u, 0u, 0u, 0u};
            } else {
                R.xr[i] = (gm < m && c0 < k) ? *(const u32x4*)(x + gm * k + c0) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if constexpr (QM) {
            // a Q8_0 quarter past the row end reads block 0 of the step instead
            const int qf = (C == Q8_0 && (int64_t)(2 * s + (wh >> 1)) * 32 >= k) ? (wh & 1) : wh;
            WT::fetch_q(wrow, s, qf, R.raw, (row_bytes & 3) == 0);
        } else if (FULL) {
            // a half past the row end reads the step's first block instead
            const int hf = (HALF_TAIL && (int64_t)(2 * s + wh) * 32 >= k) ? 0 : wh;
            WT::fetch(wrow, s, hf, R.raw, (row_bytes & 3) == 0);
        } else if (wrole && (!HALF_TAIL || (int64_t)(2 * s + wh) * 32 < k)) {
            WT::fetch(wrow, s, wh, R.raw, (row_bytes & 3) == 0);
        }
    };
    // write the fetched step into stage st: activations as they are, weights
    // decoded to the 16-bit operand type
    auto stash = [&](int sr, int st, const Regs& R) {
        const int s = sb + sr;  // step of the whole product
        uint16_t* As = lds + st * (ASZ + BSZ);
        uint16_t* Bs = As + ASZ;
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + NT * i, r = p >> 3, q = p & 7;
            u32x4 v = R.xr[i];
            if constexpr (XM == XM_BF16) {
                // bf16 -> fp32 is a shift; the power-of-two scale (ldexp: the
                // factor itself may lie outside fp32) and the conversion to
                // fp16 are exact inside the row's window
                const int ne = -xe_lds[r];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = pack_h(__builtin_ldexpf(__builtin_bit_cast(float, v[j] << 16), ne),
                                  __builtin_ldexpf(__builtin_bit_cast(float, v[j] & 0xffff0000u), ne));
            }
            *(u32x4*)&As[r * LDS_STRIDE + 8 * q] = v;
        }
        if constexpr (QM) {
            // rows past n are left as decoded (see below)
            uint32_t lo[4], hi[4];
            int cl, ch;
            WT::decode_q(R.raw, s, wh, lo, hi, cl, ch, wbig);
            if (C == Q8_0 && (int64_t)(2 * s + (wh >> 1)) * 32 >= k) {
                // a quarter past the row end (odd block count) would reach stored outputs
#pragma unroll
                for (int i = 0; i < 4; ++i) lo[i] = hi[i] = 0u;
            }
            *(u32x4*)&Bs[wr * LDS_STRIDE + cl] = u32x4{lo[0], lo[1], lo[2], lo[3]};
            *(u32x4*)&Bs[wr * LDS_STRIDE + ch] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        } else if (FULL || wrole) {
            uint32_t lo[8], hi[8];
            int cl, ch;
            // weight rows past n (read from row n-1) only reach output
            // columns that are not stored and are left as decoded, except
            // for Q8_0, which also zeroes a half past the row end (that one
            // would reach stored outputs)
            const bool live = !HALF_TAIL || (wr_valid && (int64_t)(2 * s + wh) * 32 < k);
            if (FULL) {
                WT::decode(R.raw, s, wh, lo, hi, cl, ch, wbig);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    lo[i] = live ? lo[i] : 0u;
                    hi[i] = live ? hi[i] : 0u;
                }
            } else if (live) {
                WT::decode(R.raw, s, wh, lo, hi, cl, ch, wbig);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0u;
                cl = C == Q4_K ? 16 * wh : 32 * wh;
                ch = C == Q4_K ? 32 + 16 * wh : 32 * wh + 16;  // (Q8_0 and the GGUF codecs alike)
            }
            *(u32x4*)&Bs[wr * LDS_STRIDE + cl] = u32x4{lo[0], lo[1], lo[2], lo[3]};
            *(u32x4*)&Bs[wr * LDS_STRIDE + cl + 8] = u32x4{lo[4], lo[5], lo[6], lo[7]};
            *(u32x4*)&Bs[wr * LDS_STRIDE + ch] = u32x4{hi[0], hi[1], hi[2], hi[3]};
            *(u32x4*)&Bs[wr * LDS_STRIDE + ch + 8] = u32x4{hi[4], hi[5], hi[6], hi[7]};
        }
    };
    auto frags = [&](int st, int ks, u32x4 (&af)[FM], u32x4 (&bf)[FN]) {
        const uint16_t* As = lds + st * (ASZ + BSZ);
        const uint16_t* Bs = As + ASZ;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *(const u32x4*)&As[(wm * TM + 32 * i + (lane & 31)) * LDS_STRIDE + 16 * ks + 8 * (lane >> 5)];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = *(const u32x4*)&Bs[(wn * TN + 32 * j + (lane & 31)) * LDS_STRIDE + 16 * ks + 8 * (lane >> 5)];
    };

    // Pipeline: LDS stage s%2 holds step s; while the MFMAs of step s run,
    // step s+1 (fetched earlier) is decoded into the other stage, and the
    // freed registers take the fetch of a later step.  One barrier per step,
    // which keeps the waves in phase, so a decode overlaps matrix work only
    // if it sits among the step's MFMAs.  Measured per codec:
    //  - Q4_K and TQ1: two register sets, fetching three steps ahead, and the
    //    decode after the second of the four MFMA sub-steps (loads have over
    //    a step to land, and the decode runs under the remaining MFMAs);
    //  - Q8_0: one register set, fetching two steps ahead, and the decode
    //    after the last sub-step (the loads have a whole step to land).
    // (the further GGUF codecs, whose raw fields take up to 20 registers, use
    // the one-set pipeline of Q8_0)
    constexpr bool ONESET = C == Q8_0 || is_gguf(C);
    constexpr int kAhead = ONESET ? 2 : 3;              // steps fetched ahead
    constexpr int kStashKs = ONESET ? BK / 16 - 1 : 1;  // sub-step the decode follows
    auto step = [&](int s, Regs& R) {
        const int st = s & 1;
        u32x4 af[FM], bf[FN];
        frags(st, 0, af, bf);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            u32x4 naf[FM], nbf[FN];
            if (ks + 1 < BK / 16) frags(st, ks + 1, naf, nbf);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mma_h(af[i], bf[j], acc[i][j]);
            // (on the last step the stash fills the idle stage with data
            // that is never read)
            if (ks == kStashKs && (FULL || s + 1 < steps)) stash(s + 1, st ^ 1, R);
            if (ks + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < FM; ++i) af[i] = naf[i];
#pragma unroll
                for (int j = 0; j < FN; ++j) bf[j] = nbf[j];
            }
        }
        if (FULL) fetch(s + kAhead < steps ? s + kAhead : steps - 1, R);
        else if (s + kAhead < steps) fetch(s + kAhead, R);
        __syncthreads();
    };
    fetch(0, ra);
    stash(0, 0, ra);
    if constexpr (kAhead == 3) {
        // step j's fetch lives in rb for odd j, in ra for even j
        Regs rb;
        if (steps > 1) fetch(1, rb);
        if (FULL) fetch(steps > 2 ? 2 : steps - 1, ra);
        else if (steps > 2) fetch(2, ra);
        __syncthreads();
        for (int s = 0; s < steps; s += 2) {
            step(s, rb);
            if (s + 1 < steps) step(s + 1, ra);
        }
    } else {
        if (steps > 1) fetch(1, ra);
        __syncthreads();
        for (int s = 0; s < steps; ++s) step(s, ra);
    }

    // a weight that could overflow fp16, or an activation row outside the
    // window: the whole tile is recomputed exactly
    if (wbig) exact_flag = 1;
    __syncthreads();
    if (exact_flag) {
        const int64_t c0 = (int64_t)sb * BK, c1 = c0 + (int64_t)steps * BK < k ? c0 + (int64_t)steps * BK : k;
        gemm_tile_exact<C, BM, BN, NT>(a, row_bytes, m0, n0, c0, c1, tid);
        return;
    }
    float* part = SPLIT ? a.part + (int64_t)blockIdx.z * m * n : nullptr;

    // epilogue: lane holds column l%32 and rows 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = n0 + wn * TN + 32 * j + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int lr = wm * TM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t row = m0 + lr;
                if (row < m) {
                    float o = acc[i][j][v];
                    if constexpr (ROWEXP) o = __builtin_ldexpf(o, xe_lds[lr]);
                    if (SPLIT) part[row * n + col] = o;
                    else if (a.y_dt == F32) store_out<F32>(a.y, row * n + col, o);
                    else if (a.y_dt == F16) store_out<F16>(a.y, row * n + col, o);
                    else store_out<BF16>(a.y, row * n + col, o);
                }
            }
        }
}

// y = sum over the K splits, in split order, of the fp32 partial sums
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t mn,
                                                            void* __restrict__ y, int y_dt) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < mn; i += (int64_t)gridDim.x * 256) {
        // the partials are fetched eight at a time, all in flight together,
        // and added in piece order
        float acc = part[i];
        for (int z0 = 1; z0 < splits; z0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = z0 + u < splits ? part[(int64_t)(z0 + u) * mn + i] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (z0 + u < splits) acc += v[u];
        }
        if (y_dt == F32) store_out<F32>(y, i, acc);
        else if (y_dt == F16) store_out<F16>(y, i, acc);
        else store_out<BF16>(y, i, acc);
    }
}

// bf16 activation rows -> fp16 rows scaled by 2^-e, one workgroup per row:
// e puts the row's largest magnitude in [2^14, 2^15), which keeps every
// element whose magnitude is within 2^31 of it exact.  A row with a larger
// range, bf16 subnormals, Inf or NaN gets e = kBadRow (and zeros): the GEMM
// tiles holding it take the exact path.
__global__ __launch_bounds__(256) void x16_kernel(const uint16_t* __restrict__ x, int64_t k,
                                                  uint16_t* __restrict__ x16,
                                                  int32_t* __restrict__ xexp) {
    __shared__ uint32_t red_hi[4], red_lo[4];
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * k;
    uint16_t* outr = x16 + row * k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t hi = 0u, lo = 0xffffu;
    // k is a multiple of 32: whole 16-byte pieces of 8 values
    for (int64_t c = 8 * (int64_t)tid; c < k; c += 8 * 256) {
        const u32x4 v = *(const u32x4*)(xr + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t mag = (v[j] >> (16 * h)) & 0x7fffu;
                hi = mag > hi ? mag : hi;
                const uint32_t m1 = (mag - 1u) & 0xffffu;  // a zero wraps to 0xffff
                lo = m1 < lo ? m1 : lo;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t h2 = __shfl_xor(hi, off, 64), l2 = __shfl_xor(lo, off, 64);
        hi = h2 > hi ? h2 : hi;
        lo = l2 < lo ? l2 : lo;
    }
    if (lane == 0) red_hi[wave] = hi, red_lo[wave] = lo;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi = red_hi[i] > hi ? red_hi[i] : hi;
        lo = red_lo[i] < lo ? red_lo[i] : lo;
    }
    const int emax = (int)(hi >> 7), emin = (int)((lo + 1u) >> 7);
    const bool any = hi != 0u;
    const bool bad = any && (emax == 255 || emin == 0 || emax - emin > 31);
    const int e = any ? emax - 127 - 14 : 0;
    if (tid == 0) xexp[row] = bad ? kBadRow : e;
    for (int64_t c = 8 * (int64_t)tid; c < k; c += 8 * 256) {
        u32x4 v = *(const u32x4*)(xr + c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = bad ? 0u
                       : pack_h(__builtin_ldexpf(__builtin_bit_cast(float, v[j] << 16), -e),
                                __builtin_ldexpf(__builtin_bit_cast(float, v[j] & 0xffff0000u), -e));
        *(u32x4*)(outr + c) = v;
    }
}

template <int C, int XM, int BM, int BN, int NW, bool SPLIT = true>
static void launch_tile(const GemmArgs& a, int splits, hipStream_t s) {
    const dim3 grid((unsigned)((a.n + BN - 1) / BN), (unsigned)((a.m + BM - 1) / BM),
                    (unsigned)splits),
        block(64 * NW);
    if constexpr (SPLIT) {
        if (splits > 1) {
            hipLaunchKernelGGL((gemm_kernel<C, XM, BM, BN, NW, true>), grid, block, 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((gemm_kernel<C, XM, BM, BN, NW, false>), grid, block, 0, s, a);
}

// Tile choice (eight waves, two per SIMD, measured on the prefill shapes):
// 256 x 256 while the grid holds at least 1.5 workgroups per CU (256 CUs),
// else 256 x 128 or 128 x 128 while it holds 0.75, else 64 x 128.  TQ1,
// whose weights cost the most to decode, takes 256 x 256 down to half a
// workgroup per CU and 128 x 128 below that.  Larger tiles reuse each
// decoded weight over more rows and each activation over more columns;
// smaller ones keep the CUs busy when there are few tiles.
//
// With a workspace, a product with fewer than 200 tiles of 256 x 128 (256 x
// 256 for TQ1) takes that tile and splits K into floor(256 / tiles) pieces
// of at least 8 steps, so that one round of at most 256 workgroups covers
// the product (a second, partly filled round costs more than the split
// saves).
// Measured with weights rotated through HBM: 4096 x 4096 x 512 Q4_K 49.6 ->
// 41.9 us and Q8_0 62.4 -> 44.6 us (256 x 128, four pieces); TQ1
// 5120 x 17408 x 512 218.8 -> 115.8 us (256 x 256, six pieces).
GemmPlan gemm_plan(int codec, int64_t n, int64_t k, int64_t m, bool may_split) {
    auto tiles = [&](int64_t bm, int64_t bn) { return ((n + bn - 1) / bn) * ((m + bm - 1) / bm); };
    GemmPlan p{};
    if (codec == TQ1) {
        // TQ1 weights cost the most to decode, and a tile decodes its weights
        // once for BM activation rows: the largest tile while it still gives
        // half a workgroup per compute unit
        if (tiles(256, 256) >= 128) p.bm = 256, p.bn = 256;
        else p.bm = 128, p.bn = 128;
    } else if (tiles(256, 256) >= 384) p.bm = 256, p.bn = 256;
    else if (tiles(256, 128) >= 192) p.bm = 256, p.bn = 128;
    else if (tiles(128, 128) >= 192) p.bm = 128, p.bn = 128;
    else p.bm = 64, p.bn = 128;
    p.tiles = tiles(p.bm, p.bn);
    const int64_t steps = (k + BK - 1) / BK;
    p.splits = 1;
    p.split_steps = (int)steps;
    const int bm = 256, bn = codec == TQ1 ? 256 : 128;
    const int64_t t = tiles(bm, bn);
    if (may_split && t < 200) {
        int64_t sp = 256 / t;
        if (sp > steps / 8) sp = steps / 8;
        if (sp > 1) {
            int64_t per = (steps + sp - 1) / sp;
            per = (per + 3) / 4 * 4;  // whole super-blocks of Q4_K
            p.bm = bm, p.bn = bn, p.tiles = t;
            p.split_steps = (int)per;
            p.splits = (int)((steps + per - 1) / per);
        }
    }
    return p;
}

template <int C, int XM>
static void launch_c(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    constexpr bool SP = XM != XM_BF16;  // (no workspace, so never split)
    if (p.bm == 256 && p.bn == 256) {
        // Q8_0 runs its 256 x 256 tiles with sixteen waves: half of them
        // decode, and the spare ones hide latency (10 % faster; Q4_K would
        // spill registers); only for grids of 384 tiles or more, which are
        // never split
        if constexpr (C == Q8_0) launch_tile<C, XM, 256, 256, 16, false>(a, 1, s);
        else launch_tile<C, XM, 256, 256, 8, SP>(a, p.splits, s);
    } else if (p.bm == 256) launch_tile<C, XM, 256, 128, 8, SP>(a, p.splits, s);
    else if (p.bm == 128) launch_tile<C, XM, 128, 128, 8, SP>(a, p.splits, s);
    else launch_tile<C, XM, 64, 128, 8, SP>(a, p.splits, s);
}

template <int XM>
static void launch_xm(int codec, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    switch (codec) {
    case Q4_K: launch_c<Q4_K, XM>(a, p, s); break;
    case Q8_0: launch_c<Q8_0, XM>(a, p, s); break;
    case Q4_0: launch_c<Q4_0, XM>(a, p, s); break;
    case Q5_0: launch_c<Q5_0, XM>(a, p, s); break;
    case Q5_1: launch_c<Q5_1, XM>(a, p, s); break;
    case Q6_K: launch_c<Q6_K, XM>(a, p, s); break;
    case Q2_K: launch_c<Q2_K, XM>(a, p, s); break;
    case Q3_K: launch_c<Q3_K, XM>(a, p, s); break;
    case Q5_K: launch_c<Q5_K, XM>(a, p, s); break;
    default: launch_c<TQ1, XM>(a, p, s); break;
    }
}

GemmWorkspace gemm_workspace(int codec, int64_t n, int64_t k, int64_t m, int x_dt) {
    const GemmPlan p = gemm_plan(codec, n, k, m, true);
    GemmWorkspace L{};
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    int64_t off = 0;
    if (x_dt == BF16) {
        L.xexp_off = off;
        off += up(m * 4);
        L.x16_off = off;
        off += up(m * k * 2);
    }
    L.part_off = off;
    if (p.splits > 1) off += up((int64_t)p.splits * m * n * 4);
    L.bytes = off;
    return L;
}

hipError_t launch_gemm(int codec, int x_dt, const void* w, int64_t n, int64_t k, const void* x,
                       int64_t m, void* y, int y_dt, void* ws, hipStream_t s) {
    GemmArgs a{};
    a.w = (const uint8_t*)w;
    a.n = n, a.k = k, a.m = m;
    a.x = (const uint16_t*)x;
    a.x_src = (const uint16_t*)x;
    a.x_src_dt = x_dt;
    a.y = y;
    a.y_dt = y_dt;
    const GemmPlan p = gemm_plan(codec, n, k, m, ws != nullptr);
    a.split_steps = p.split_steps;
    if (!ws) {
        // no workspace: bf16 rows are scaled inside each workgroup
        if (x_dt == BF16) launch_xm<XM_BF16>(codec, a, p, s);
        else launch_xm<XM_F16>(codec, a, p, s);
        return hipGetLastError();
    }
    const GemmWorkspace L = gemm_workspace(codec, n, k, m, x_dt);
    char* base = (char*)ws;
    if (x_dt == BF16) {
        int32_t* xexp = (int32_t*)(base + L.xexp_off);
        uint16_t* x16 = (uint16_t*)(base + L.x16_off);
        hipLaunchKernelGGL(x16_kernel, dim3((unsigned)m), dim3(256), 0, s, (const uint16_t*)x, k,
                           x16, xexp);
        a.x = x16;
        a.xexp = xexp;
    }
    if (p.splits > 1) a.part = (float*)(base + L.part_off);
    if (x_dt == BF16) launch_xm<XM_SCALED>(codec, a, p, s);
    else launch_xm<XM_F16>(codec, a, p, s);
    if (p.splits > 1) return launch_splitk_reduce(a.part, p.splits, m * n, y, y_dt, s);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int pieces, int64_t count, void* y, int y_dt,
                                hipStream_t s) {
    const int64_t blocks = (count + 255) / 256 < 4096 ? (count + 255) / 256 : 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, pieces,
                       count, y, y_dt);
    return hipGetLastError();
}

}  // namespace kq
