// gemm.hip -- prefill product Y[M,N] = X[M,K] * dequant(W)[N,K]^T (kq_qmm).
//
// mlx-kquant "bindings.cpp", quantized_matmul; Ternary Bonsai
// "ternel_packed_model.py", tq1_gemm (decode a weight once and reuse it
// across a whole block of activation rows on the matrix units).
//
// The contraction runs on v_mfma_f32_32x32x16 in the activation's 16-bit
// type (bf16 or fp16) with fp32 accumulation.  A workgroup of eight waves owns
// a BM x BN output tile; per K step of 64 it decodes its BN x 64 weight tile
// once into LDS (so each decoded weight feeds BM rows) next to the BM x 64
// activation tile.  The global loads of step k+1 are issued before the MFMAs
// of step k and written to LDS after them, so memory latency overlaps the
// matrix work.  Decoded weights are rounded once from fp32 to the 16-bit
// operand type (round to nearest even).
#include "kq_device.h"
#include "kq_internal.h"

namespace kq {

constexpr int BK = 64, LDS_STRIDE = BK + 8;  // +8 halves: rows start in different banks

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int XDT> struct Op16;
template <> struct Op16<BF16> {
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2));
    }
    static __device__ __forceinline__ float16_t mma(const u32x4& a, const u32x4& b, float16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Op16<F16> {
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, half2v));
    }
    static __device__ __forceinline__ float16_t mma(const u32x4& a, const u32x4& b, float16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
};

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
    template <int XDT>
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi) {
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
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t ml = r.q[i] & 0x0f0f0f0fu, mh = r.q[i] & 0xf0f0f0f0u;
            // opaque to the compiler, which would otherwise fold the masks
            // into one bit-field extract per nibble
            asm("" : "+v"(ml), "+v"(mh));
#pragma unroll
            for (int b = 0; b < 4; b += 2) {
                lo[2 * i + b / 2] = Op16<XDT>::pack(__builtin_fmaf(s0, byte(ml, b), n0),
                                                    __builtin_fmaf(s0, byte(ml, b + 1), n0));
                hi[2 * i + b / 2] = Op16<XDT>::pack(__builtin_fmaf(s1h, byte(mh, b), n1),
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
    template <int XDT>
    static __device__ __forceinline__ void decode_q(const RawQ& r, int s, int q, uint32_t (&lo)[4],
                                                    uint32_t (&hi)[4], int& col_lo, int& col_hi) {
        const int c = s & 3;
        int sc0, m0, sc1, m1;
        q4k_scale_min(r.hd, 2 * c, sc0, m0);
        q4k_scale_min(r.hd, 2 * c + 1, sc1, m1);
        const float d = q4k_d(r.hd), dmin = q4k_dmin(r.hd);
        const float s0 = d * (float)sc0, s1h = d * (float)sc1 * 0.0625f;
        const float n0 = -dmin * (float)m0, n1 = -dmin * (float)m1;
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t ml = r.q[i] & 0x0f0f0f0fu, mh = r.q[i] & 0xf0f0f0f0u;
            asm("" : "+v"(ml), "+v"(mh));
#pragma unroll
            for (int b = 0; b < 4; b += 2) {
                lo[2 * i + b / 2] = Op16<XDT>::pack(__builtin_fmaf(s0, byte(ml, b), n0),
                                                    __builtin_fmaf(s0, byte(ml, b + 1), n0));
                hi[2 * i + b / 2] = Op16<XDT>::pack(__builtin_fmaf(s1h, byte(mh, b), n1),
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
    template <int XDT>
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi) {
        uint32_t sh = h ? 0u : 16u;
        asm("" : "+v"(sh));  // one funnel shift by a register, not two selected
        const float d = half_bits_to_float(h ? r.tail : (r.w[0] & 0xffffu));
        const float nd = -128.0f * d;
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
        uint32_t v[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t next = j < 7 ? r.w[j + 1] : r.tail;
            const uint32_t u = __builtin_amdgcn_alignbit(next, r.w[j], sh) ^ 0x80808080u;
            v[2 * j] = Op16<XDT>::pack(__builtin_fmaf(d, byte(u, 0), nd), __builtin_fmaf(d, byte(u, 1), nd));
            v[2 * j + 1] = Op16<XDT>::pack(__builtin_fmaf(d, byte(u, 2), nd), __builtin_fmaf(d, byte(u, 3), nd));
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
    template <int XDT>
    static __device__ __forceinline__ void decode_q(const RawQ& r, int s, int q, uint32_t (&lo)[4],
                                                    uint32_t (&hi)[4], int& col_lo, int& col_hi) {
        uint32_t sh = (q >> 1) ? 0u : 16u;
        asm("" : "+v"(sh));
        const float d = half_bits_to_float(r.sc);
        const float nd = -128.0f * d;
        auto byte = [](uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xffu); };
        uint32_t v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t next = j < 3 ? r.w[j + 1] : r.next;
            const uint32_t u = __builtin_amdgcn_alignbit(next, r.w[j], sh) ^ 0x80808080u;
            v[2 * j] = Op16<XDT>::pack(__builtin_fmaf(d, byte(u, 0), nd), __builtin_fmaf(d, byte(u, 1), nd));
            v[2 * j + 1] = Op16<XDT>::pack(__builtin_fmaf(d, byte(u, 2), nd), __builtin_fmaf(d, byte(u, 3), nd));
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
    // fp16 activations: digits two at a time with packed 16-bit integer
    // arithmetic.  A code byte c (<= 242) in fixed point, q = ceil(256 c /
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
    template <int XDT, int C0, int NP>
    static __device__ __forceinline__ void cols(const Raw& r, uint32_t (&v)[NP]) {
        if constexpr (XDT == F16) {
            cols_f16<C0, NP>(r, v);
        } else {
            // bf16 activations: w = (digit - 1) * scale rounded to bf16
            const float sc = half_bits_to_float(r.w[6] >> 16);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                float t[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int col = C0 + 2 * i + e;
                    const int slot = col < 125 ? col / 5 : 25;
                    const int digit = col < 125 ? col - 5 * slot : col - 125;
                    const uint32_t code = (r.w[slot >> 2] >> (8 * (slot & 3))) & 0xffu;
                    t[e] = (float)tq1_trit(code, digit) * sc;
                }
                v[i] = Op16<XDT>::pack(t[0], t[1]);
            }
        }
    }
    template <int XDT>
    static __device__ __forceinline__ void decode(const Raw& r, int s, int h, uint32_t (&lo)[8],
                                                  uint32_t (&hi)[8], int& col_lo, int& col_hi) {
        uint32_t v[16];
        switch (2 * (s & 1) + h) {
        case 0: cols<XDT, 0, 16>(r, v); break;
        case 1: cols<XDT, 32, 16>(r, v); break;
        case 2: cols<XDT, 64, 16>(r, v); break;
        default: cols<XDT, 96, 16>(r, v); break;
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
    template <int XDT>
    static __device__ __forceinline__ void decode_q(const RawQ& r, int s, int q, uint32_t (&lo)[4],
                                                    uint32_t (&hi)[4], int& col_lo, int& col_hi) {
        uint32_t v[8];
        switch (4 * (s & 1) + q) {
        case 0: cols<XDT, 0, 8>(r, v); break;
        case 1: cols<XDT, 16, 8>(r, v); break;
        case 2: cols<XDT, 32, 8>(r, v); break;
        case 3: cols<XDT, 48, 8>(r, v); break;
        case 4: cols<XDT, 64, 8>(r, v); break;
        case 5: cols<XDT, 80, 8>(r, v); break;
        case 6: cols<XDT, 96, 8>(r, v); break;
        default: cols<XDT, 112, 8>(r, v); break;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = v[i], hi[i] = v[4 + i];
        col_lo = 16 * q;
        col_hi = 16 * q + 8;
    }
};

// The per-step weight registers: halves (Raw) or quarters (RawQ).
template <bool Q, class WT> struct RawSel { using type = typename WT::Raw; };
template <class WT> struct RawSel<true, WT> { using type = typename WT::RawQ; };

// ---------------------------------------------------------------- kernel
// BM x BN tile, NW waves as 2 x (NW/2), each a (BM/2) x (2BN/NW) sub-tile of
// 32x32 MFMA blocks.  With eight waves two share each SIMD, so one wave's
// weight decoding overlaps the other's matrix work.
template <int C, int XDT, int BM, int BN, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_kernel(const uint8_t* __restrict__ w, int64_t n,
                                                       int64_t k, const uint16_t* __restrict__ x,
                                                       int64_t m, void* __restrict__ y, int y_dt) {
    constexpr int NT = 64 * NW, WN = NW / 2;
    constexpr int TM = BM / 2, TN = BN / WN, FM = TM / 32, FN = TN / 32;
    static_assert(FM >= 1 && FN >= 1 && 2 * BN <= NT, "tile shape");
    constexpr int XP = BM * 8 / NT;  // 16-byte activation pieces per thread per step
    constexpr int ASZ = BM * LDS_STRIDE, BSZ = BN * LDS_STRIDE;
    using WT = WTile<C>;
    // two stages of [activation tile | weight tile]
    __shared__ __align__(16) uint16_t lds[2 * (ASZ + BSZ)];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
    const int64_t row_bytes = (k / CodecInfo<C>::QK) * CodecInfo<C>::BYTES;
    const int steps = (int)((k + BK - 1) / BK);

    // weight role: tile row wr and part wh of each step, a half (wh < 2) or,
    // when the threads are four times the tile's rows, a quarter (wh < 4), so
    // that every wave shares the decoding.  Q8_0 takes quarters only in
    // tiles of at most 128 activation rows (7-8 % faster there, 3-6 %
    // slower in the 256-row tiles, where half the threads decoding keeps the
    // rest on matrix work).  Neighbouring threads read the parts of one row
    // (contiguous bytes), except for TQ1, whose decoding branches on the
    // part: there each wave holds one part, so it runs one branch (measured
    // faster for TQ1, slower for the others).
    constexpr bool QM = 4 * BN == NT && (C != Q8_0 || BM <= 128);
    constexpr int NPART = QM ? 4 : 2;
    constexpr bool kWaveParts = C == TQ1;
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
    auto fetch = [&](int s, Regs& R) {
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
                R.xr[i] = (C != Q8_0 || ok) ? v : u32x4{0u, 0u, 0u, 0u};
            } else {
                R.xr[i] = (gm < m && c0 < k) ? *(const u32x4*)(x + gm * k + c0) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if constexpr (QM) {
            // a Q8_0 quarter past the row end reads block 0 of the step instead
            const int qf = (C == Q8_0 && (int64_t)(2 * s + (wh >> 1)) * 32 >= k) ? (wh & 1) : wh;
            WT::fetch_q(wrow, s, qf, R.raw, (row_bytes & 3) == 0);
        } else if (FULL) {
            // a Q8_0 half past the row end reads the step's first block instead
            const int hf = (C == Q8_0 && (int64_t)(2 * s + wh) * 32 >= k) ? 0 : wh;
            WT::fetch(wrow, s, hf, R.raw, (row_bytes & 3) == 0);
        } else if (wrole && ((C != Q8_0) || (int64_t)(2 * s + wh) * 32 < k)) {
            WT::fetch(wrow, s, wh, R.raw, (row_bytes & 3) == 0);
        }
    };
    // write the fetched step into stage st: activations as they are, weights
    // decoded to the 16-bit operand type
    auto stash = [&](int s, int st, const Regs& R) {
        uint16_t* As = lds + st * (ASZ + BSZ);
        uint16_t* Bs = As + ASZ;
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + NT * i, r = p >> 3, q = p & 7;
            *(u32x4*)&As[r * LDS_STRIDE + 8 * q] = R.xr[i];
        }
        if constexpr (QM) {
            // rows past n are left as decoded (see below)
            uint32_t lo[4], hi[4];
            int cl, ch;
            WT::template decode_q<XDT>(R.raw, s, wh, lo, hi, cl, ch);
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
            const bool live = (C != Q8_0) || (wr_valid && (int64_t)(2 * s + wh) * 32 < k);
            if (FULL) {
                WT::template decode<XDT>(R.raw, s, wh, lo, hi, cl, ch);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    lo[i] = live ? lo[i] : 0u;
                    hi[i] = live ? hi[i] : 0u;
                }
            } else if (live) {
                WT::template decode<XDT>(R.raw, s, wh, lo, hi, cl, ch);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0u;
                cl = C == Q4_K ? 16 * wh : 32 * wh;
                ch = C == Q4_K ? 32 + 16 * wh : 32 * wh + 16;
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
    constexpr int kAhead = C == Q8_0 ? 2 : 3;              // steps fetched ahead
    constexpr int kStashKs = C == Q8_0 ? BK / 16 - 1 : 1;  // sub-step the decode follows
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
                for (int j = 0; j < FN; ++j) acc[i][j] = Op16<XDT>::mma(af[i], bf[j], acc[i][j]);
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

    // epilogue: lane holds column l%32 and rows 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = n0 + wn * TN + 32 * j + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * TM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < m) {
                    const float o = acc[i][j][v];
                    if (y_dt == F32) store_out<F32>(y, row * n + col, o);
                    else if (y_dt == F16) store_out<F16>(y, row * n + col, o);
                    else store_out<BF16>(y, row * n + col, o);
                }
            }
        }
}

template <int C, int XDT, int BM, int BN, int NW>
static void launch_tile(const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y,
                        int y_dt, hipStream_t s) {
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM)), block(64 * NW);
    hipLaunchKernelGGL((gemm_kernel<C, XDT, BM, BN, NW>), grid, block, 0, s, (const uint8_t*)w, n,
                       k, (const uint16_t*)x, m, y, y_dt);
}

// Tile choice (eight waves, two per SIMD, measured on the prefill shapes):
// 256 x 256 while the grid holds at least 1.5 workgroups per CU (256 CUs),
// else 256 x 128 or 128 x 128 while it holds 0.75, else 64 x 128.  TQ1,
// whose weights cost the most to decode, takes 256 x 256 down to half a
// workgroup per CU and 128 x 128 below that.  Larger tiles reuse each
// decoded weight over more rows and each activation over more columns;
// smaller ones keep the CUs busy when there are few tiles.
template <int C, int XDT>
static void launch_c(const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y,
                     int y_dt, hipStream_t s) {
    auto tiles = [&](int64_t bm, int64_t bn) { return ((n + bn - 1) / bn) * ((m + bm - 1) / bm); };
    if (C == TQ1) {
        // TQ1 weights cost the most to decode, and a tile decodes its weights
        // once for BM activation rows: the largest tile while it still gives
        // half a workgroup per compute unit
        if (tiles(256, 256) >= 128) launch_tile<C, XDT, 256, 256, 8>(w, n, k, x, m, y, y_dt, s);
        else launch_tile<C, XDT, 128, 128, 8>(w, n, k, x, m, y, y_dt, s);
        return;
    }
    if (tiles(256, 256) >= 384) {
        // Q8_0 runs its 256 x 256 tiles with sixteen waves: half of them
        // decode, and the spare ones hide latency (10 % faster; Q4_K would
        // spill registers)
        if (C == Q8_0) launch_tile<C, XDT, 256, 256, 16>(w, n, k, x, m, y, y_dt, s);
        else launch_tile<C, XDT, 256, 256, 8>(w, n, k, x, m, y, y_dt, s);
    } else if (tiles(256, 128) >= 192) launch_tile<C, XDT, 256, 128, 8>(w, n, k, x, m, y, y_dt, s);
    else if (tiles(128, 128) >= 192) launch_tile<C, XDT, 128, 128, 8>(w, n, k, x, m, y, y_dt, s);
    else launch_tile<C, XDT, 64, 128, 8>(w, n, k, x, m, y, y_dt, s);
}

hipError_t launch_gemm(int codec, int x_dt, const void* w, int64_t n, int64_t k, const void* x,
                       int64_t m, void* y, int y_dt, hipStream_t s) {
    const bool bf = x_dt == BF16;
    switch (codec) {
    case Q4_K: bf ? launch_c<Q4_K, BF16>(w, n, k, x, m, y, y_dt, s) : launch_c<Q4_K, F16>(w, n, k, x, m, y, y_dt, s); break;
    case Q8_0: bf ? launch_c<Q8_0, BF16>(w, n, k, x, m, y, y_dt, s) : launch_c<Q8_0, F16>(w, n, k, x, m, y, y_dt, s); break;
    default: bf ? launch_c<TQ1, BF16>(w, n, k, x, m, y, y_dt, s) : launch_c<TQ1, F16>(w, n, k, x, m, y, y_dt, s); break;
    }
    return hipGetLastError();
}

}  // namespace kq
