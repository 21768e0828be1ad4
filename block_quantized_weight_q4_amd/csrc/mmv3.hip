// mmv3.hip -- decode products of up to four fp16 activation rows with Q4_K
// weights (kq_qmv / kq_qmm with m <= 4).
//
// mlx-kquant "bindings.cpp": quantized_matmul in the decode regime; the Q4_K
// super-block as the GGUF K-quant layout defines it (fp16 d and dmin, eight
// 6-bit scales and mins, 256 nibbles).
//
// Weights stream into LDS as in mmv2.hip: a workgroup owns 16 weight rows,
// K is walked in double-buffered chunks of C super-blocks copied with
// global->LDS loads.  The multiply is arranged so that no weight is scaled:
//
// - A nibble q taken with one AND is the fp16 subnormal q * 2^-24 (a high
//   nibble: 16q * 2^-24).  It is exact, and the matrix core multiplies it by
//   an fp16 activation exactly into fp32.
// - Lane group g of every MFMA supplies nibbles of chunk g of the
//   super-block (quant bytes 32g..32g+31: sub-blocks 2g and 2g+1), and the
//   A operand's rows are (sub-block j, activation row) pairs: row (j, 0)
//   holds the activations of sub-block j in the lanes of group j/2 and zeros
//   in the other groups.  After the super-block's eight MFMAs, output row
//   (j, 0) is sum_{k in j} x[k] q[n,k], the dot product that d * sc_j
//   multiplies, and the scales are applied to these fp32 results.
// - The min term dmin * m_j * sum_{k in j} x[k] uses the sub-block sums of
//   the activation row.
//
// A quant dword b0 b1 b2 b3 gives the nibble pairs (b0, b2) and (b1, b3) by
// masking alone, so inside every group of four columns the operands are in
// the order 0, 2, 1, 3.  The workgroup rewrites the activation row once, in
// that order, as 16-byte entries [x0 x2 x1 x3 | 0 0 0 0]: an entry read at its
// start is the operand of a low-nibble sub-block; read 8 bytes earlier (the
// previous entry's zero half) it is [0 0 0 0 | x0 x2 x1 x3], the operand of a
// high-nibble sub-block.  Lanes whose row has no activations in an MFMA keep
// zero operands and read nothing.  The kernel for two to four rows (below)
// keeps the activations in their natural order instead.
#include "kq_device.h"
#include "kq_internal.h"
#include "q4k_mfma.h"
#include "lds_dma.h"

namespace kq {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Sum of the four fp16 values in two packed words, in fp32.
__device__ __forceinline__ float sum4_h(uint32_t d0, uint32_t d1) {
    return (half_bits_to_float(d0 & 0xffffu) + half_bits_to_float(d0 >> 16)) +
           (half_bits_to_float(d1 & 0xffffu) + half_bits_to_float(d1 >> 16));
}

// Sum over the eight lanes of an aligned group of eight (every lane of the
// group receives the total).
__device__ __forceinline__ float sum8_lanes(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));
    return v;
}

template <int C, int W, int S>
struct Mmv3Layout {
    static constexpr int WPIECES = 16 * 9 * C;         // 16-byte weight pieces per chunk
    static constexpr int WBYTES = WPIECES * 16;        // one chunk buffer
    static constexpr int XP_OFF = S * WBYTES;          // rearranged activations
    static constexpr int XP_SB = 64 * 16;              // per super-block: 64 entries
    static_assert(WPIECES % 64 == 0, "a chunk of weights is whole 1 KB loads");
    // sub-block sums follow the rearranged activations, then the reduction
    __host__ __device__ static size_t xs_off(int nsb) { return XP_OFF + (size_t)nsb * XP_SB; }
    __host__ __device__ static size_t red_off(int nsb) { return xs_off(nsb) + (size_t)nsb * 32; }
    __host__ __device__ static size_t end_off(int nsb) { return red_off(nsb) + (size_t)(W - 1) * 2 * 64 * 4; }
    // the activation row as loaded (whole 1 KB loads): in the second chunk
    // buffer, idle until the main loop starts, when it fits; else past the end
    __host__ __device__ static size_t raw_bytes(int nsb) { return (size_t)((nsb * 32 + 63) / 64) * 1024; }
    __host__ __device__ static size_t raw_off(int nsb) {
        return (S == 2 && raw_bytes(nsb) <= (size_t)WBYTES) ? (size_t)WBYTES : end_off(nsb);
    }
    __host__ __device__ static size_t total(int nsb) {
        const size_t r = raw_off(nsb) + raw_bytes(nsb);
        return r > end_off(nsb) ? r : end_off(nsb);
    }
};

}  // namespace

template <int C, int W, int S>
__global__ __launch_bounds__(64 * W) void mmv3_q4k_f16_kernel(SkinnyArgs a) {
    using L = Mmv3Layout<C, W, S>;
    constexpr int WLOADS = L::WPIECES / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int ROWB = 9 * C * 16;                  // LDS bytes of one weight row per chunk
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int nsb = (int)(a.k / 256);
    const int nchunks = (nsb + C - 1) / C;
    uint8_t* xp = smem + L::XP_OFF;
    float* xs = (float*)(smem + L::xs_off(nsb));

    // ---- weight pieces of this lane, offsets from the tile's first row
    const uint8_t* wbase = a.w + n0 * a.row_bytes;
    uint32_t woff[WL_PER_WAVE], wq16[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int p = 64 * (wave + W * j) + lane;
        const int r = p / (9 * C), q = p - r * 9 * C;
        int64_t n = n0 + r;
        if (n >= a.n) n = a.n - 1;
        wq16[j] = 16u * (uint32_t)q;
        woff[j] = (uint32_t)((n - n0) * a.row_bytes) + wq16[j];
    }
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    auto issue = [&](int chunk, int dst_off) {
        uint8_t* dst = smem + dst_off;
        const int s0 = chunk * C;
        const int nsc = nsb - s0 < C ? nsb - s0 : C;
        const uint32_t cbase = (uint32_t)s0 * 144u;
        const uint32_t climit = (uint32_t)nsc * 144u;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                // pieces past the last super-block re-read a valid piece
                const uint32_t off = wq16[j] < climit ? woff[j] : woff[j] - wq16[j];
                dma16(wbase + cbase + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i)));
            }
        }
    };
    // ---- the activation row: copied into LDS as loaded, issued just before
    // the first weights so that it lands while they stream (loads complete
    // in order, so waiting for the weights' count leaves only the weights
    // outstanding), then rearranged once for all of K: entry t of
    // super-block s is [x(4t) x(4t+2) x(4t+1) x(4t+3) | 0 0 0 0] (t = 0..63,
    // 16 bytes).  The lanes of a wave take 64 consecutive entries (one
    // super-block), so each group of eight lanes holds one sub-block and
    // forms its sum.
    uint8_t* xraw = smem + L::raw_off(nsb);
    {
        const int xpieces = nsb * 32, xloads = (xpieces + 63) / 64;
        const uint8_t* xsrc = (const uint8_t*)a.x;
        for (int i = wave; i < xloads; i += W) {
            // lanes past the row re-read its last piece into the padding
            const int piece = 64 * i + lane < xpieces ? 64 * i + lane : xpieces - 1;
            dma16(xsrc + 16 * piece, __builtin_amdgcn_readfirstlane(lds_addr(xraw + 1024 * i)));
        }
    }
    for (int c = 0; c < S - 1 && c < nchunks; ++c) issue(c, c * L::WBYTES);
    wait_loads_le(wave_loads * (nchunks < S - 1 ? nchunks : S - 1));
    __syncthreads();
    for (int e0 = tid; e0 < nsb * 64; e0 += 64 * W) {
        const int sbg = e0 >> 6, t = e0 & 63;
        const u32x2 v = *(const u32x2*)(xraw + 8 * e0);
        const uint32_t p0 = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // x0 x2
        const uint32_t p1 = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // x1 x3
        *(u32x4*)(xp + sbg * L::XP_SB + 16 * t) = u32x4{p0, p1, 0u, 0u};
        const float sum = sum8_lanes(sum4_h(v.x, v.y));
        if ((t & 7) == 0) xs[8 * sbg + (t >> 3)] = sum;
    }

    // A operand: MFMA j takes from column group g the quant dword j of chunk
    // g (bytes 32g+4j..+3): low nibbles of sub-block 2g at columns 64g+4j..,
    // high nibbles of sub-block 2g+1 at 64g+32+4j..  Lane row r = (sub-block
    // r/2, activation row r%2) carries activations only where its sub-block
    // lies in chunk g, i.e. r/4 == g; the other lanes keep zero operands and
    // read nothing.
    const bool alive = (n_l >> 2) == g && (n_l & 1) == 0;
    const uint32_t abase_l = L::XP_OFF + ((n_l & 2) ? 16 * (16 * g + 8) - 8 : 16 * (16 * g));
    u32x4 A[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) A[j] = u32x4{0u, 0u, 0u, 0u};
    // scale selectors: output lane (n_l, g) holds rows 4g+v = (sub-block
    // 2g + v/2, v%2); rows v = 0 and 2 carry the product
    const LaneSel ls = lane_sel(g);

    float acc0 = 0.f, acc2 = 0.f;
    for (int c = 0; c < nchunks; ++c) {
        const int later = nchunks - 1 - c < S - 2 ? nchunks - 1 - c : S - 2;
        wait_loads_le(wave_loads * later);
        __syncthreads();
        if (c + S - 1 < nchunks) issue(c + S - 1, ((c + S - 1) % S) * L::WBYTES);
        const uint8_t* B = smem + (c % S) * L::WBYTES;
        const int nsc = nsb - c * C < C ? nsb - c * C : C;
        for (int sb = wave; sb < nsc; sb += W) {
            const int sbg = c * C + sb;
            // weights of row n_l: head and this lane group's 32 quant bytes
            const uint8_t* wr = B + n_l * ROWB + sb * 144;
            const u32x4 hd = *(const u32x4*)wr;
            const u32x4 q0 = *(const u32x4*)(wr + 16 + 32 * g), q1 = *(const u32x4*)(wr + 32 + 32 * g);
            const uint32_t qd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            if (alive) {
                const uint8_t* ap = smem + abase_l + (uint32_t)sbg * L::XP_SB;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const u32x2 alo = *(const u32x2*)(ap + 16 * j), ahi = *(const u32x2*)(ap + 16 * j + 8);
                    A[j] = u32x4{alo.x, alo.y, ahi.x, ahi.y};
                }
            }
            const f32x2 x2 = *(const f32x2*)(xs + 8 * sbg + 2 * g);
            __builtin_amdgcn_sched_barrier(0);
            float4_t da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t q = qd[j], q8 = q >> 8;
                const u32x4 Bq = u32x4{q & 0x000f000fu, q8 & 0x000f000fu, q & 0x00f000f0u, q8 & 0x00f000f0u};
                if (j & 1) db = mfma16(A[j], Bq, db);
                else da = mfma16(A[j], Bq, da);
            }
            const float d0 = da[0] + db[0], d2 = da[2] + db[2];
            // scales of sub-blocks 2g (low nibbles) and 2g+1 (high nibbles)
            uint32_t sc_lo, sc_hi, m_lo, m_hi;
            q4k_scales_all(hd, sc_lo, sc_hi, m_lo, m_hi);
            const uint32_t scw = ls.high ? sc_hi : sc_lo, mw = ls.high ? m_hi : m_lo;
            const uint32_t sc_u = __builtin_amdgcn_perm(scw, scw, ls.sel);
            const uint32_t m_u = __builtin_amdgcn_perm(mw, mw, ls.sel);
            const float d = q4k_d(hd), dmin = q4k_dmin(hd);
            const float s0 = d * 16777216.0f * (float)(sc_u & 0xffu);
            const float s1 = d * 1048576.0f * (float)((sc_u >> 16) & 0xffu);
            const float mm0 = dmin * (float)(m_u & 0xffu), mm1 = dmin * (float)((m_u >> 16) & 0xffu);
            acc0 += s0 * d0 - mm0 * x2[0];
            acc2 += s1 * d2 - mm1 * x2[1];
        }
    }
    __syncthreads();

    // ---- combine the waves, then the four column groups
    float* red = (float*)(smem + L::red_off(nsb));
    if (W > 1) {
        if (wave > 0) {
            red[((wave - 1) * 2 + 0) * 64 + lane] = acc0;
            red[((wave - 1) * 2 + 1) * 64 + lane] = acc2;
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            acc0 += red[((w - 1) * 2 + 0) * 64 + lane];
            acc2 += red[((w - 1) * 2 + 1) * 64 + lane];
        }
    }
    float y = acc0 + acc2;
    y += __shfl_xor(y, 16);
    y += __shfl_xor(y, 32);
    const int64_t n = n0 + n_l;
    if (g == 0 && n < a.n) store_val(a.y, n, a.y_dt, y);
}

// ---------------------------------------------------------------------------
// Up to four activation rows.  Activations stay in their natural order
// (quant bytes are spread into nibble pairs with v_perm instead), and the A
// operand's 16 rows are (chunk c, activation row b) pairs: lane group g
// supplies chunk g's nibbles, and row (c, b) holds x[b] only in lane group
// c.  Three accumulators per super-block: the low-nibble products (sub-block
// 2c), the high-nibble products (2c+1), and the min term, whose B operand
// is the 6-bit min broadcast over the sub-block (m * sum x exactly).
template <int C, int W>
struct Mmv3mLayout {
    static constexpr int WPIECES = 16 * 9 * C;
    static constexpr int WBYTES = WPIECES * 16;          // weights of one chunk
    static constexpr int XSTRIDE = 512 * C + 16;         // one staged activation row
    static constexpr int BUF = WBYTES + 4 * XSTRIDE;     // one chunk buffer
    static constexpr int RED_OFF = 2 * BUF;
    static constexpr int TOTAL = RED_OFF + (W - 1) * 4 * 64 * 4;
    static_assert(WPIECES % 64 == 0, "a chunk of weights is whole 1 KB loads");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <int C, int W>
__global__ __launch_bounds__(64 * W) void mmv3m_q4k_f16_kernel(SkinnyArgs a) {
    using L = Mmv3mLayout<C, W>;
    constexpr int WLOADS = L::WPIECES / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int XPIECES_ROW = 32 * C;
    constexpr int ROWB = 9 * C * 16;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int nsb = (int)(a.k / 256);
    const int nchunks = (nsb + C - 1) / C;
    const int m = (int)a.m;  // 1..4

    const uint8_t* wbase = a.w + n0 * a.row_bytes;
    uint32_t woff[WL_PER_WAVE], wq16[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int p = 64 * (wave + W * j) + lane;
        const int r = p / (9 * C), q = p - r * 9 * C;
        int64_t n = n0 + r;
        if (n >= a.n) n = a.n - 1;
        wq16[j] = 16u * (uint32_t)q;
        woff[j] = (uint32_t)((n - n0) * a.row_bytes) + wq16[j];
    }
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    {
        const int xl_total = m * (XPIECES_ROW / 64);
        wave_loads += xl_total > wave ? (xl_total - wave + W - 1) / W : 0;
    }
    auto issue = [&](int chunk) {
        uint8_t* dst = smem + (chunk & 1) * L::BUF;
        const int s0 = chunk * C;
        const int nsc = nsb - s0 < C ? nsb - s0 : C;
        const uint32_t cbase = (uint32_t)s0 * 144u;
        const uint32_t climit = (uint32_t)nsc * 144u;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t off = wq16[j] < climit ? woff[j] : woff[j] - wq16[j];
                dma16(wbase + cbase + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i)));
            }
        }
        const int xl_row = XPIECES_ROW / 64;
        for (int i = wave; i < m * xl_row; i += W) {
            const int r = i / xl_row, k = i - r * xl_row;
            int piece = 64 * k + lane;
            if (piece >= 32 * nsc) piece = 0;
            const uint8_t* src = (const uint8_t*)a.x + ((int64_t)r * a.x_row + (int64_t)s0 * 256) * 2 + 16 * piece;
            dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(dst + L::WBYTES + r * L::XSTRIDE + 1024 * k)));
        }
    };

    // lanes whose row (chunk n_l / 4, activation row n_l % 4) meets lane
    // group g's chunk read the activations; the others keep zero operands.
    // MFMA p of a half takes quant dwords 2p, 2p+1 of the chunk: sub-block
    // columns 8p..8p+7, i.e. activations 64g+8p.. (low) and 64g+32+8p.. (high)
    const int brow = n_l & 3;
    const bool alive = (n_l >> 2) == g && brow < m;
    u32x4 AL[4], AH[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) AL[p] = AH[p] = u32x4{0u, 0u, 0u, 0u};
    const LaneSel ls = lane_sel(g);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};

    issue(0);
    for (int c = 0; c < nchunks; ++c) {
        wait_loads_le(0);
        __syncthreads();
        if (c + 1 < nchunks) issue(c + 1);
        const uint8_t* B = smem + (c & 1) * L::BUF;
        const int nsc = nsb - c * C < C ? nsb - c * C : C;
        for (int sb = wave; sb < nsc; sb += W) {
            const uint8_t* wr = B + n_l * ROWB + sb * 144;
            const u32x4 hd = *(const u32x4*)wr;
            const u32x4 q0 = *(const u32x4*)(wr + 16 + 32 * g), q1 = *(const u32x4*)(wr + 32 + 32 * g);
            const uint32_t qd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            if (alive) {
                const uint8_t* ap = B + L::WBYTES + brow * L::XSTRIDE + sb * 512 + 128 * g;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    AL[p] = *(const u32x4*)(ap + 16 * p);
                    AH[p] = *(const u32x4*)(ap + 64 + 16 * p);
                }
            }
            // scales and mins of sub-blocks 2g (low nibbles) and 2g+1 (high)
            uint32_t sc_lo, sc_hi, m_lo, m_hi;
            q4k_scales_all(hd, sc_lo, sc_hi, m_lo, m_hi);
            const uint32_t scw = ls.high ? sc_hi : sc_lo, mw = ls.high ? m_hi : m_lo;
            const uint32_t sc_u = __builtin_amdgcn_perm(scw, scw, ls.sel);
            const uint32_t m_u = __builtin_amdgcn_perm(mw, mw, ls.sel);
            const half2_t m_h = __builtin_bit_cast(half2_t, m_u | 0x64006400u) -
                                half2_t{(half_t)1024.0f, (half_t)1024.0f};
            const uint32_t m0 = __builtin_bit_cast(uint32_t, half2_t{m_h[0], m_h[0]});
            const uint32_t m1 = __builtin_bit_cast(uint32_t, half2_t{m_h[1], m_h[1]});
            float4_t dl = {0.f, 0.f, 0.f, 0.f}, dh = {0.f, 0.f, 0.f, 0.f}, dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t qa = qd[2 * p], qb = qd[2 * p + 1];
                const uint32_t a01 = __builtin_amdgcn_perm(qa, qa, 0x0c010c00u), a23 = __builtin_amdgcn_perm(qa, qa, 0x0c030c02u);
                const uint32_t b01 = __builtin_amdgcn_perm(qb, qb, 0x0c010c00u), b23 = __builtin_amdgcn_perm(qb, qb, 0x0c030c02u);
                dl = mfma16(AL[p], u32x4{a01 & 0x000f000fu, a23 & 0x000f000fu, b01 & 0x000f000fu, b23 & 0x000f000fu}, dl);
                dh = mfma16(AH[p], u32x4{a01 & 0x00f000f0u, a23 & 0x00f000f0u, b01 & 0x00f000f0u, b23 & 0x00f000f0u}, dh);
                dm = mfma16(AL[p], u32x4{m0, m0, m0, m0}, dm);
                dm = mfma16(AH[p], u32x4{m1, m1, m1, m1}, dm);
            }
            const float d = q4k_d(hd), dmin = q4k_dmin(hd);
            const float s0 = d * 16777216.0f * (float)(sc_u & 0xffu);
            const float s1 = d * 1048576.0f * (float)((sc_u >> 16) & 0xffu);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += (s0 * dl[v] + s1 * dh[v]) - dmin * dm[v];
        }
    }
    __syncthreads();

    // ---- combine the waves, then the four column groups (lane (n_l, g)
    // holds activation rows v of sub-blocks 2g and 2g+1)
    float* red = (float*)(smem + L::RED_OFF);
    if (W > 1) {
        if (wave > 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) red[((wave - 1) * 4 + v) * 64 + lane] = acc[v];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += red[((w - 1) * 4 + v) * 64 + lane];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        acc[v] += __shfl_xor(acc[v], 16);
        acc[v] += __shfl_xor(acc[v], 32);
    }
    const int64_t n = n0 + n_l;
    if (g == 0 && n < a.n) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (v < m) store_val(a.y, v * a.y_row + n, a.y_dt, acc[v]);
    }
}

template <int C, int W>
static void launch_cfg3m(const SkinnyArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.n + 15) / 16));
    constexpr size_t lds = Mmv3mLayout<C, W>::TOTAL;
    hipLaunchKernelGGL((mmv3m_q4k_f16_kernel<C, W>), grid, dim3(64 * W), lds, s, a);
}

hipError_t launch_mmv3m_q4k(const SkinnyArgs& a, hipStream_t s) {
    if (a.k / 256 > 16) launch_cfg3m<8, 8>(a, s);
    else launch_cfg3m<4, 4>(a, s);
    return hipGetLastError();
}

template <int C, int W, int S>
static void launch_cfg3(const SkinnyArgs& a, hipStream_t s) {
    using L = Mmv3Layout<C, W, S>;
    const dim3 grid((unsigned)((a.n + 15) / 16));
    hipLaunchKernelGGL((mmv3_q4k_f16_kernel<C, W, S>), grid, dim3(64 * W),
                       L::total((int)(a.k / 256)), s, a);
}

// Launch shapes, measured on the decode shapes: four waves and four-block
// chunks up to K = 4096, eight and eight beyond.
bool mmv3_fits(int64_t k) {
    const int nsb = (int)(k / 256);
    const size_t lds = nsb > 16 ? Mmv3Layout<8, 8, 2>::total(nsb) : Mmv3Layout<4, 4, 2>::total(nsb);
    return lds <= 160 * 1024;
}

hipError_t launch_mmv3_q4k(const SkinnyArgs& a, hipStream_t s) {
    if (a.k / 256 > 16) launch_cfg3<8, 8, 2>(a, s);
    else launch_cfg3<4, 4, 2>(a, s);
    return hipGetLastError();
}

}  // namespace kq
