// pair32.h -- Q8_0 and the further GGUF codecs (Q4_0, Q5_0, Q5_1, Q6_K, Q2_K,
// Q3_K, Q5_K) decoded for fp16 activations: exact fp16 integer pairs and an
// affine scale per 16 weights, multiplied on v_dot2_f32_f16.  The block
// layouts are those of include/kq.h (the GGUF layouts of the codecs that
// mlx-native "quantized_matmul_id_ggml.rs" dispatches).
#pragma once
#include "kq_device.h"

namespace kq {

// For fp16 activations the further GGUF codecs skip fp32 weights: chunk q
// decodes to 16 fp16 pairs p[] of exact small integers (p[0..7]: weights
// 0..15, paired with activations [xa, xa+16); p[8..15]: weights 16..31 with
// [xb, xb+16)) and, per half h of 16 weights, w = A[h] * v + B[h].  The dot
// products run on v_dot2_f32_f16 (fp16 products are exact in fp32, sums in
// fp32), then sum w x = A * sum v x + B * sum x.  An integer v is formed as
// the fp16 1024 + v (the byte v under the exponent pattern 0x64) minus the
// offset, exactly.
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <int C> struct Pair32 { static constexpr bool ok = false, has_b = false; };

// bytes b0..b3 of t (each < 256) as two fp16 pairs (1024 + b0, 1024 + b1),
// (1024 + b2, 1024 + b3), minus `off` in each lane
__device__ __forceinline__ void bytes_to_pairs(uint32_t t, h2_t off, uint32_t& p01, uint32_t& p23) {
    p01 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, t, 0x04010400u)) - off);
    p23 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, t, 0x04030402u)) - off);
}
__device__ __forceinline__ h2_t h2(float v) { return h2_t{(_Float16)v, (_Float16)v}; }
// N consecutive little-endian dwords from a 2-byte-aligned address.  From
// global memory: 16-bit loads, which the compiler may merge (the vector
// memory path takes unaligned addresses).  From LDS (LDS = true): N + 1
// aligned dword reads realigned by v_alignbyte; the one extra dword must be
// readable (the LDS rows of the decode kernels end in a padding piece).
template <bool LDS, int N>
__device__ __forceinline__ void words(const uint8_t* p, uint32_t (&v)[N]) {
    if constexpr (LDS) {
        const uint32_t sh = (uint32_t)(uintptr_t)p & 3u;
        const uint32_t* b = (const uint32_t*)(p - sh);
        uint32_t t[N + 1];
#pragma unroll
        for (int i = 0; i <= N; ++i) t[i] = b[i];
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_alignbyte(t[i + 1], t[i], sh);
    } else {
        const uint16_t* q = (const uint16_t*)p;
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = (uint32_t)q[2 * i] | ((uint32_t)q[2 * i + 1] << 16);
    }
}
// bits 0..3 of t moved to bits 0, 8, 16, 24 (the four copies t << 7i do not
// overlap, so the product carries nothing)
__device__ __forceinline__ uint32_t spread4(uint32_t t) { return (t * 0x00204081u) & 0x01010101u; }

// Q4_0 / Q5_0 / Q5_1: v = q - 8 / q - 16 / q (A = d; Q5_1: B = m)
template <int C> struct PairLegacy {
    static constexpr bool ok = true, has_b = C == Q5_1;
    template <bool LDS = false>
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, uint32_t (&p)[16],
                                                  float (&A)[2], float (&B)[2], int64_t& xa, int64_t& xb) {
        constexpr int BB = C == Q4_0 ? 18 : C == Q5_0 ? 22 : 24;
        const uint8_t* blk = row + q * BB;
        // Q4_0: d, qs[16]; Q5_0: d, qh, qs[16]; Q5_1: d, m, qh, qs[16]
        constexpr int NW = C == Q4_0 ? 4 : 5;
        uint32_t wv[NW];
        words<LDS>(blk + (C == Q5_1 ? 4 : 2), wv);
        const float d = half_bits_to_float(*(const uint16_t*)blk);
        A[0] = A[1] = d;
        B[0] = B[1] = C == Q5_1 ? half_bits_to_float(*(const uint16_t*)(blk + 2)) : 0.f;
        const uint32_t qh = C == Q4_0 ? 0u : wv[0];
        const h2_t off = h2(C == Q4_0 ? 1032.f : C == Q5_0 ? 1040.f : 1024.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t qd = wv[NW - 4 + i];  // quant bytes 4i .. 4i + 3
            uint32_t lo = qd & 0x0f0f0f0fu, hi = (qd >> 4) & 0x0f0f0f0fu;
            if (C != Q4_0) {
                lo |= spread4((qh >> (4 * i)) & 15u) << 4;
                hi |= spread4((qh >> (16 + 4 * i)) & 15u) << 4;
            }
            bytes_to_pairs(lo, off, p[2 * i], p[2 * i + 1]);
            bytes_to_pairs(hi, off, p[8 + 2 * i], p[8 + 2 * i + 1]);
        }
        xa = q * 32;
        xb = xa + 16;
    }
};
template <> struct Pair32<Q4_0> : PairLegacy<Q4_0> {};
template <> struct Pair32<Q5_0> : PairLegacy<Q5_0> {};
template <> struct Pair32<Q5_1> : PairLegacy<Q5_1> {};

// Q8_0 (34-byte blocks, 2-byte aligned): v = q (int8; q + 128 under the
// exponent pattern, then minus 1152), A = d
template <> struct Pair32<Q8_0> {
    static constexpr bool ok = true, has_b = false;
    template <bool LDS = false>
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, uint32_t (&p)[16],
                                                  float (&A)[2], float (&B)[2], int64_t& xa, int64_t& xb) {
        const uint8_t* blk = row + q * 34;
        uint32_t qw[8];
        words<LDS>(blk + 2, qw);
        A[0] = A[1] = half_bits_to_float(*(const uint16_t*)blk);
        B[0] = B[1] = 0.f;
        const h2_t off = h2(1152.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) bytes_to_pairs(qw[i] ^ 0x80808080u, off, p[2 * i], p[2 * i + 1]);
        xa = q * 32;
        xb = xa + 16;
    }
};

// Q6_K: v = q - 32, A = d * scale of each 16 weights
template <> struct Pair32<Q6_K> {
    static constexpr bool ok = true, has_b = false;
    template <bool LDS = false>
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, uint32_t (&p)[16],
                                                  float (&A)[2], float (&B)[2], int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int r = (int)q & 7, h = r >> 2, u = r & 3;
        const uint8_t* blk = row + sb * 210;
        uint32_t lw[8], hw[8];
        words<LDS>(blk + 64 * h + 32 * (u & 1), lw);
        words<LDS>(blk + 128 + 32 * h, hw);
        const float d = half_bits_to_float(*(const uint16_t*)(blk + 208));
        const uint32_t scw = *(const uint16_t*)(blk + 192 + 8 * h + 2 * u);
        A[0] = d * (float)(int8_t)(scw & 0xffu);
        A[1] = d * (float)(int8_t)(scw >> 8);
        B[0] = B[1] = 0.f;
        const int lsh = 4 * (u >> 1), hsh = 2 * u;
        const h2_t off = h2(1056.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = ((lw[i] >> lsh) & 0x0f0f0f0fu) | (((hw[i] >> hsh) & 0x03030303u) << 4);
            bytes_to_pairs(v, off, p[2 * i], p[2 * i + 1]);
        }
        xa = sb * 256 + 32 * r;
        xb = xa + 16;
    }
};

// Q2_K: v = q, A = d * scale, B = -dmin * min of each 16 weights (blocks are
// 4-byte aligned)
template <> struct Pair32<Q2_K> {
    static constexpr bool ok = true, has_b = true;
    template <bool LDS = false>
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, uint32_t (&p)[16],
                                                  float (&A)[2], float (&B)[2], int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int r = (int)q & 7, h = r >> 2, u = r & 3;
        const uint8_t* blk = row + sb * 84;
        const uint32_t dd = *(const uint32_t*)(blk + 80);
        const float d = half_bits_to_float(dd & 0xffffu), dmin = half_bits_to_float(dd >> 16);
        const uint32_t scw = *(const uint16_t*)(blk + 8 * h + 2 * u);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t b = (scw >> (8 * i)) & 0xffu;
            A[i] = d * (float)(b & 15u);
            B[i] = -(dmin * (float)(b >> 4));
        }
        const uint32_t* qs = (const uint32_t*)(blk + 16 + 32 * h);
        const h2_t off = h2(1024.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) bytes_to_pairs((qs[i] >> (2 * u)) & 0x03030303u, off, p[2 * i], p[2 * i + 1]);
        xa = sb * 256 + 32 * r;
        xb = xa + 16;
    }
};

// Q3_K: v = q in -4..3, A = d * scale of each 16 weights (scale bytes as in
// the chunk decoder)
template <> struct Pair32<Q3_K> {
    static constexpr bool ok = true, has_b = false;
    template <bool LDS = false>
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, uint32_t (&p)[16],
                                                  float (&A)[2], float (&B)[2], int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int r = (int)q & 7, h = r >> 2, u = r & 3;
        const uint8_t* blk = row + sb * 110;
        const float d = half_bits_to_float(*(const uint16_t*)(blk + 108));
        const uint32_t lw = *(const uint16_t*)(blk + 96 + 2 * u);
        const uint32_t tw = *(const uint16_t*)(blk + 104 + 2 * (u & 1));
        const int tsh = 2 * (2 * h + (u >> 1));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int lo = (int)((lw >> (8 * i + 4 * h)) & 15u);
            const int top = (int)((tw >> (8 * i + tsh)) & 3u);
            A[i] = d * (float)((lo | (top << 4)) - 32);
        }
        B[0] = B[1] = 0.f;
        uint32_t hm[8], qs[8];
        words<LDS>(blk, hm);
        words<LDS>(blk + 32 + 32 * h, qs);
        const int hsh = 4 * h + u;
        const h2_t off = h2(1028.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = ((qs[i] >> (2 * u)) & 0x03030303u) | (((hm[i] >> hsh) & 0x01010101u) << 2);
            bytes_to_pairs(v, off, p[2 * i], p[2 * i + 1]);
        }
        xa = sb * 256 + 32 * r;
        xb = xa + 16;
    }
};

// Q5_K: v = q in 0..31, A = d * sc, B = -dmin * m of the sub-block (blocks
// are 16-byte aligned)
template <> struct Pair32<Q5_K> {
    static constexpr bool ok = true, has_b = true;
    template <bool LDS = false>
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, uint32_t (&p)[16],
                                                  float (&A)[2], float (&B)[2], int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int j = (int)q & 7;
        const uint8_t* blk = row + sb * 176;
        const u32x4 hd = *(const u32x4*)blk;
        int sc, m;
        q4k_scale_min(hd, j, sc, m);
        A[0] = A[1] = q4k_d(hd) * (float)sc;
        B[0] = B[1] = -(q4k_dmin(hd) * (float)m);
        const u32x4* qh = (const u32x4*)(blk + 16);
        const u32x4* qs = (const u32x4*)(blk + 48 + 32 * (j >> 1));
        const int nsh = 4 * (j & 1);
        const h2_t off = h2(1024.f);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const u32x4 hv = qh[v], qv = qs[v];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t t = ((qv[i] >> nsh) & 0x0f0f0f0fu) | (((hv[i] >> j) & 0x01010101u) << 4);
                bytes_to_pairs(t, off, p[8 * v + 2 * i], p[8 * v + 2 * i + 1]);
            }
        }
        xa = sb * 256 + 32 * j;
        xb = xa + 16;
    }
};

// ---------------------------------------------------------------- one lane's part of a chunk
// Pair8<C>::decode(row, q, g, b0, b1, A, B): lane group g (0..3) of chunk q
// of a row: the exact fp16 integers v of weights 4g .. 4g+3 (b0, two pairs,
// first 16-weight half) and 16+4g .. 16+4g+3 (b1, second half), and the
// half's affine scales w = A[h] v + B[h] -- the same values Pair32 gives for
// those weights.  These are one 16x16x16 MFMA operand slice each.  Reads
// realigned dwords from LDS.
template <int C> struct Pair8;

// four bytes (each < 256) as fp16 integers minus off: two pairs
__device__ __forceinline__ u32x2 bytes_pairs2(uint32_t t, h2_t off) {
    uint32_t a, b;
    bytes_to_pairs(t, off, a, b);
    return u32x2{a, b};
}

// The 32-weight blocks (one fp16 d, Q5_1 also an fp16 m) also fold the scale
// in: fold() gives the eight weights as fp16, each d*v (Q5_1: d*v + m by one
// fma) rounded once, and returns false when a weight of the block could reach
// 65520 or d or m is not finite (then decode() gives the exact form).
__device__ __forceinline__ uint32_t fold_pair(uint32_t v, h2_t d2, h2_t m2, bool with_m) {
    const h2_t vv = __builtin_bit_cast(h2_t, v);
    return __builtin_bit_cast(uint32_t, with_m ? __builtin_elementwise_fma(vv, d2, m2) : vv * d2);
}
__device__ __forceinline__ u32x2 fold_pairs(const u32x2& v, uint32_t dbits, uint32_t mbits, bool with_m) {
    const h2_t d2 = __builtin_bit_cast(h2_t, dbits | (dbits << 16));
    const h2_t m2 = __builtin_bit_cast(h2_t, mbits | (mbits << 16));
    const uint32_t v0 = v.x, v1 = v.y;
    return u32x2{fold_pair(v0, d2, m2, with_m), fold_pair(v1, d2, m2, with_m)};
}

template <> struct Pair8<Q8_0> {
    static constexpr bool has_b = false, foldable = true;
    static __device__ __forceinline__ void ints(const uint8_t* blk, int g, u32x2& b0, u32x2& b1) {
        uint32_t w0[1], w1[1];
        words<true>(blk + 2 + 4 * g, w0);
        words<true>(blk + 18 + 4 * g, w1);
        const h2_t off = h2(1152.f);
        b0 = bytes_pairs2(w0[0] ^ 0x80808080u, off);
        b1 = bytes_pairs2(w1[0] ^ 0x80808080u, off);
    }
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, int g, u32x2& b0, u32x2& b1,
                                                  float (&A)[2], float (&B)[2]) {
        const uint8_t* blk = row + q * 34;
        ints(blk, g, b0, b1);
        A[0] = A[1] = half_bits_to_float(*(const uint16_t*)blk);
        B[0] = B[1] = 0.f;
    }
    static __device__ __forceinline__ bool fold(const uint8_t* row, int64_t q, int g, u32x2& w0, u32x2& w1) {
        const uint8_t* blk = row + q * 34;
        u32x2 b0, b1;
        ints(blk, g, b0, b1);
        const uint32_t db = *(const uint16_t*)blk;
        w0 = fold_pairs(b0, db, 0u, false);
        w1 = fold_pairs(b1, db, 0u, false);
        return __builtin_fabsf(half_bits_to_float(db)) * 128.0f < 65520.0f;  // |v| <= 128; NaN fails
    }
};

template <int C> struct Pair8Legacy {
    static constexpr bool has_b = C == Q5_1, foldable = true;
    static constexpr int BB = C == Q4_0 ? 18 : C == Q5_0 ? 22 : 24, QS = C == Q4_0 ? 2 : C == Q5_0 ? 6 : 8;
    static __device__ __forceinline__ void ints(const uint8_t* blk, int g, u32x2& b0, u32x2& b1) {
        uint32_t qd[1];
        words<true>(blk + QS + 4 * g, qd);  // quant bytes 4g .. 4g + 3
        uint32_t lo = qd[0] & 0x0f0f0f0fu, hi = (qd[0] >> 4) & 0x0f0f0f0fu;
        if constexpr (C != Q4_0) {
            uint32_t qh[1];
            words<true>(blk + (C == Q5_0 ? 2 : 4), qh);
            lo |= spread4((qh[0] >> (4 * g)) & 15u) << 4;
            hi |= spread4((qh[0] >> (16 + 4 * g)) & 15u) << 4;
        }
        const h2_t off = h2(C == Q4_0 ? 1032.f : C == Q5_0 ? 1040.f : 1024.f);
        b0 = bytes_pairs2(lo, off);
        b1 = bytes_pairs2(hi, off);
    }
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, int g, u32x2& b0, u32x2& b1,
                                                  float (&A)[2], float (&B)[2]) {
        const uint8_t* blk = row + q * BB;
        ints(blk, g, b0, b1);
        A[0] = A[1] = half_bits_to_float(*(const uint16_t*)blk);
        B[0] = B[1] = C == Q5_1 ? half_bits_to_float(*(const uint16_t*)(blk + 2)) : 0.f;
    }
    static __device__ __forceinline__ bool fold(const uint8_t* row, int64_t q, int g, u32x2& w0, u32x2& w1) {
        const uint8_t* blk = row + q * BB;
        u32x2 b0, b1;
        ints(blk, g, b0, b1);
        const uint32_t db = *(const uint16_t*)blk, mb = C == Q5_1 ? *(const uint16_t*)(blk + 2) : 0u;
        w0 = fold_pairs(b0, db, mb, C == Q5_1);
        w1 = fold_pairs(b1, db, mb, C == Q5_1);
        constexpr float vmax = C == Q4_0 ? 8.0f : C == Q5_0 ? 16.0f : 31.0f;
        return __builtin_fabsf(half_bits_to_float(db)) * vmax + __builtin_fabsf(half_bits_to_float(mb)) < 65520.0f;
    }
};
template <> struct Pair8<Q4_0> : Pair8Legacy<Q4_0> {};
template <> struct Pair8<Q5_0> : Pair8Legacy<Q5_0> {};
template <> struct Pair8<Q5_1> : Pair8Legacy<Q5_1> {};

template <> struct Pair8<Q6_K> {
    static constexpr bool has_b = false, foldable = false;
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, int g, u32x2& b0, u32x2& b1,
                                                  float (&A)[2], float (&B)[2]) {
        const int r = (int)q & 7, h = r >> 2, u = r & 3;
        const uint8_t* blk = row + (q >> 3) * 210;
        const uint8_t* ql = blk + 64 * h + 32 * (u & 1);
        const uint8_t* qh = blk + 128 + 32 * h;
        uint32_t l0[1], l1[1], h0[1], h1[1];
        words<true>(ql + 4 * g, l0);
        words<true>(ql + 16 + 4 * g, l1);
        words<true>(qh + 4 * g, h0);
        words<true>(qh + 16 + 4 * g, h1);
        const float d = half_bits_to_float(*(const uint16_t*)(blk + 208));
        const uint32_t scw = *(const uint16_t*)(blk + 192 + 8 * h + 2 * u);
        A[0] = d * (float)(int8_t)(scw & 0xffu);
        A[1] = d * (float)(int8_t)(scw >> 8);
        B[0] = B[1] = 0.f;
        const int lsh = 4 * (u >> 1), hsh = 2 * u;
        const h2_t off = h2(1056.f);
        b0 = bytes_pairs2(((l0[0] >> lsh) & 0x0f0f0f0fu) | (((h0[0] >> hsh) & 0x03030303u) << 4), off);
        b1 = bytes_pairs2(((l1[0] >> lsh) & 0x0f0f0f0fu) | (((h1[0] >> hsh) & 0x03030303u) << 4), off);
    }
};

template <> struct Pair8<Q2_K> {
    static constexpr bool has_b = true, foldable = false;
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, int g, u32x2& b0, u32x2& b1,
                                                  float (&A)[2], float (&B)[2]) {
        const int r = (int)q & 7, h = r >> 2, u = r & 3;
        const uint8_t* blk = row + (q >> 3) * 84;
        const uint32_t* qs = (const uint32_t*)(blk + 16 + 32 * h);
        const uint32_t dd = *(const uint32_t*)(blk + 80);
        const float d = half_bits_to_float(dd & 0xffffu), dmin = half_bits_to_float(dd >> 16);
        const uint32_t scw = *(const uint16_t*)(blk + 8 * h + 2 * u);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t b = (scw >> (8 * i)) & 0xffu;
            A[i] = d * (float)(b & 15u);
            B[i] = -(dmin * (float)(b >> 4));
        }
        const h2_t off = h2(1024.f);
        b0 = bytes_pairs2((qs[g] >> (2 * u)) & 0x03030303u, off);
        b1 = bytes_pairs2((qs[4 + g] >> (2 * u)) & 0x03030303u, off);
    }
};

template <> struct Pair8<Q3_K> {
    static constexpr bool has_b = false, foldable = false;
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, int g, u32x2& b0, u32x2& b1,
                                                  float (&A)[2], float (&B)[2]) {
        const int r = (int)q & 7, h = r >> 2, u = r & 3;
        const uint8_t* blk = row + (q >> 3) * 110;
        const float d = half_bits_to_float(*(const uint16_t*)(blk + 108));
        const uint32_t lw = *(const uint16_t*)(blk + 96 + 2 * u);
        const uint32_t tw = *(const uint16_t*)(blk + 104 + 2 * (u & 1));
        const int tsh = 2 * (2 * h + (u >> 1));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int lo = (int)((lw >> (8 * i + 4 * h)) & 15u);
            const int top = (int)((tw >> (8 * i + tsh)) & 3u);
            A[i] = d * (float)((lo | (top << 4)) - 32);
        }
        B[0] = B[1] = 0.f;
        uint32_t m0[1], m1[1], s0[1], s1[1];
        words<true>(blk + 4 * g, m0);
        words<true>(blk + 16 + 4 * g, m1);
        words<true>(blk + 32 + 32 * h + 4 * g, s0);
        words<true>(blk + 32 + 32 * h + 16 + 4 * g, s1);
        const int hsh = 4 * h + u;
        const h2_t off = h2(1028.f);
        b0 = bytes_pairs2(((s0[0] >> (2 * u)) & 0x03030303u) | (((m0[0] >> hsh) & 0x01010101u) << 2), off);
        b1 = bytes_pairs2(((s1[0] >> (2 * u)) & 0x03030303u) | (((m1[0] >> hsh) & 0x01010101u) << 2), off);
    }
};

template <> struct Pair8<Q5_K> {
    static constexpr bool has_b = true, foldable = false;
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, int g, u32x2& b0, u32x2& b1,
                                                  float (&A)[2], float (&B)[2]) {
        const int j = (int)q & 7;
        const uint8_t* blk = row + (q >> 3) * 176;
        const u32x4 hd = *(const u32x4*)blk;
        int sc, m;
        q4k_scale_min(hd, j, sc, m);
        A[0] = A[1] = q4k_d(hd) * (float)sc;
        B[0] = B[1] = -(q4k_dmin(hd) * (float)m);
        const uint32_t* qh = (const uint32_t*)(blk + 16);
        const uint32_t* qs = (const uint32_t*)(blk + 48 + 32 * (j >> 1));
        const int nsh = 4 * (j & 1);
        const h2_t off = h2(1024.f);
        b0 = bytes_pairs2(((qs[g] >> nsh) & 0x0f0f0f0fu) | (((qh[g] >> j) & 0x01010101u) << 4), off);
        b1 = bytes_pairs2(((qs[4 + g] >> nsh) & 0x0f0f0f0fu) | (((qh[4 + g] >> j) & 0x01010101u) << 4), off);
    }
};

// sum over 16 weights of v * x (p: 8 pairs, xw: 8 fp16 activation pairs)
__device__ __forceinline__ float dot16(const uint32_t* p, const uint32_t* xw) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p[e]), __builtin_bit_cast(h2_t, xw[e]), s, false);
    return s;
}
__device__ __forceinline__ float sum16(const uint32_t* xw) {
    const h2_t one = h2(1.f);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_amdgcn_fdot2(one, __builtin_bit_cast(h2_t, xw[e]), s, false);
    return s;
}
// the 16 fp16 activations at x[i .. i + 16) as 8 pairs
__device__ __forceinline__ void load_x_pairs(const void* x, int64_t i, uint32_t* xw) {
    const u32x4* p = (const u32x4*)((const uint16_t*)x + i);
    const u32x4 a = p[0], b = p[1];
    xw[0] = a[0], xw[1] = a[1], xw[2] = a[2], xw[3] = a[3];
    xw[4] = b[0], xw[5] = b[1], xw[6] = b[2], xw[7] = b[3];
}

}  // namespace kq
