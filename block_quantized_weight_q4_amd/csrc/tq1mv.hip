// tq1mv.hip -- TQ1_G128 decode GEMV, one fp16 activation row (kq_qmv, m = 1).
//
// Ternary Bonsai "ternel_packed_model.py": format constants (28-byte block:
// 25 code bytes of five base-3 digits, a tail byte of three, fp16 scale) and
// the LUT23 GEMV section (decoding through a table instead of dividing each
// byte by powers of three).
//
// Here a code byte c = d0 + 3 d1 + 9 d2 + 27 (d3 + 3 d4) is decoded through
// two small tables: c mod 27 gives the trits (d0-1, d1-1, d2-1), c div 27 the
// trits (d3-1, d4-1), each as an 8-byte entry of fp16 values padded with
// zeros, so that the two entries side by side are exactly one 16x16x32 MFMA
// operand slice of eight fp16 values [d0 d1 d2 0 d3 d4 0 0] and both reads
// land in aligned register pairs.  The tables are 27 and 10 entries long, so
// lanes that read different entries never share an LDS bank and lanes that
// read the same entry are served by one broadcast.  The contraction order is
// permuted so that each lane group's eight MFMA k-slots are the five columns
// of one code byte: the activations are staged in LDS once per workgroup in
// the same 8-wide "slot" layout (columns 5s..5s+4 of byte s at positions
// 0 1 2 4 5, zeros elsewhere; the tail byte's slot holds columns 125..127).
// A block of 128 weights is 28 slots (25 code bytes, the tail, and the two
// scale bytes, whose activation slots are zero), i.e. seven MFMAs; the fp16
// scale multiplies each block's fp32 result.  All products (+-x or 0) are
// exact; accumulation is fp32.
//
// A workgroup owns 16 weight rows.  Their weights stream through LDS in
// chunks of 16 blocks (coalesced global->LDS copies, double buffered);
// the W waves (8 or 16) take the blocks of a chunk in turn and combine their
// partial sums through LDS at the end.  Each half block issues all of its table and
// activation reads before its first MFMA, so their LDS latency overlaps.
#include "kq_device.h"
#include "kq_internal.h"
#include "lds_dma.h"

#include <type_traits>

namespace kq {

namespace {

constexpr int kSlots = 28;            // MFMA slots per 128-weight block
// LDS tables of 8-byte entries: c mod 27 (27 entries), then from byte 256
// c div 27 (16 entries; those past 8 serve the scale bytes, whose activations
// are zero)
constexpr int kHiOff = 256;
constexpr int kLutBytes = kHiOff + 16 * 8;

__device__ __forceinline__ float4_t mfma_h(const u32x4& a, const u32x4& b, const float4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

}  // namespace

// Weights stream through LDS: chunks of CB blocks of the 16 rows, copied
// with coalesced global->LDS 16-byte loads (each row's chunk is 28 CB
// contiguous bytes) into NBUF buffers, up to NBUF - 1 chunks in flight.
// LDS rows are padded by one 16-byte piece so that the 16 lanes reading one
// dword of 16 rows hit 16 banks.
template <int W, int CB_>
struct TqCfg {
    static constexpr int CB = CB_;                             // blocks per chunk
    static constexpr int NBUF = 2;                             // chunk buffers
    static constexpr int ROW_PIECES = CB * 28 / 16 + 1;        // 16-byte pieces per LDS row (+1 pad)
    static constexpr int WBUF = 16 * ROW_PIECES * 16;          // bytes of one chunk buffer
    static_assert(CB % 4 == 0, "a chunk row must be a whole number of 16-byte pieces");
    // tables, chunk buffers, activation slots (3.5 bytes per column), reduction
    static constexpr size_t lds_bytes(int64_t nblk) {
        return (size_t)kLutBytes + NBUF * WBUF + (size_t)nblk * kSlots * 16 + (W - 1) * 16 * 4;
    }
};

// K pieces (split-K): with pnb > 0, workgroup (tile, piece) covers blocks
// [piece * pnb, piece * pnb + pnb) of its rows and stores its fp32 partial
// sums to part[piece * n + row] instead of y.
template <int W, int CB>
__global__ __launch_bounds__(64 * W) void tq1_mv_kernel(const uint8_t* __restrict__ w, int64_t n,
                                                        int64_t k, const uint16_t* __restrict__ x,
                                                        void* __restrict__ y, int y_dt, int pnb,
                                                        float* __restrict__ part) {
    using Cfg = TqCfg<W, CB>;
    constexpr int kCB = Cfg::CB, kNBuf = Cfg::NBUF, kRowPieces = Cfg::ROW_PIECES, kWBuf = Cfg::WBUF;
    constexpr int NPIECE = 16 * kRowPieces;
    constexpr int WLOADS = (NPIECE + 63) / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    extern __shared__ __align__(16) uint8_t smem[];
    u32x2* lut_lo = (u32x2*)smem;                                // [27]
    u32x2* lut_hi = (u32x2*)(smem + kHiOff);                     // [16]
    uint8_t* wbuf = smem + kLutBytes;                           // [kNBuf][kWBuf]
    u32x4* xs = (u32x4*)(smem + kLutBytes + kNBuf * kWBuf);     // [nblk * 28] slots
    const int nblk_row = (int)(k / 128);
    const int piece = (int)blockIdx.y;
    // blocks of this workgroup's piece of K (all of K without a split)
    const int nblk = pnb ? (nblk_row - piece * pnb < pnb ? nblk_row - piece * pnb : pnb) : nblk_row;
    x += (int64_t)piece * pnb * 128;
    float* red = (float*)((uint8_t*)xs + (size_t)nblk * kSlots * 16);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t row_bytes = (int64_t)nblk_row * 28;
    const int nchunks = (nblk + kCB - 1) / kCB;

    // ---- tables of trits as fp16: -1, 0, +1 for digits 0, 1, 2
    auto trit = [](uint32_t d) -> uint32_t { return d == 0 ? 0xbc00u : d == 1 ? 0x0000u : 0x3c00u; };
    if (tid < 27) lut_lo[tid] = u32x2{trit(tid % 3) | (trit((tid / 3) % 3) << 16), trit(tid / 9)};
    if (tid >= 64 && tid < 80) {
        const uint32_t j = tid - 64;
        lut_hi[j] = u32x2{trit(j % 3) | (trit((j / 3) % 3) << 16), 0u};
    }
    // ---- activations in slot layout: slot s < 25 of block b holds columns
    // 128b + 5s .. +4 at positions 0 1 2 4 5, slot 25 columns 128b + 125 .. 127
    // at positions 0 1 2, the rest zeros.  Each thread builds whole slots from
    // the (4-byte aligned) dwords that cover their columns.
    for (int i = tid; i < nblk * kSlots; i += 64 * W) {
        const int b = i / kSlots, sl = i - kSlots * b;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (sl < 26) {
            const int64_t col = 128 * (int64_t)b + 5 * sl;
            const uint32_t* p = (const uint32_t*)(x + (col & ~(int64_t)1));
            // columns (col & ~1) .. +5; the tail slot needs only .. +3, and
            // reading further would pass the end of the row
            const uint32_t d0 = p[0], d1 = p[1], d2 = sl < 25 ? p[2] : 0u;
            const bool odd = col & 1;
            const uint32_t e0 = odd ? __builtin_amdgcn_alignbit(d1, d0, 16) : d0;  // columns 0, 1
            const uint32_t e1 = odd ? __builtin_amdgcn_alignbit(d2, d1, 16) : d1;  // columns 2, 3
            const uint32_t e2 = odd ? d2 >> 16 : d2 & 0xffffu;                      // column 4
            v[0] = e0;
            v[1] = e1 & 0xffffu;
            v[2] = sl < 25 ? (e1 >> 16) | (e2 << 16) : 0u;
        }
        xs[i] = v;
    }
    // ---- weight pieces of this lane: LDS slot p = 64 i + lane is piece
    // p % kRowPieces of row p / kRowPieces (the last piece of a row is
    // padding and is not loaded)
    const uint8_t* wbase = w + n0 * row_bytes + (int64_t)piece * pnb * 28;
    uint32_t woff[WL_PER_WAVE], wq16[WL_PER_WAVE];
    bool wact[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int r = p / kRowPieces, q = p - r * kRowPieces;
        int64_t nr = n0 + r;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < 16 && q < kRowPieces - 1;
        wq16[j] = 16u * (uint32_t)q;
        woff[j] = (uint32_t)((nr - n0) * row_bytes) + wq16[j];
    }
    // load instructions this wave issues per chunk (every one of them has a
    // live lane: each group of 64 pieces holds pieces of a row)
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    auto issue = [&](int chunk) {
        uint8_t* dst = wbuf + (chunk % kNBuf) * kWBuf;
        const uint32_t cbase = (uint32_t)chunk * (kCB * 28);
        const int ncb = nblk - chunk * kCB < kCB ? nblk - chunk * kCB : kCB;
        const uint32_t climit = (uint32_t)ncb * 28u;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS && wact[j]) {
                // pieces past the last block re-read the chunk's first piece
                const uint32_t off = wq16[j] < climit ? woff[j] : woff[j] - wq16[j];
                dma16(wbase + cbase + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i)));
            }
        }
    };

    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int sh = 8 * g;  // this lane group's byte within each dword
    auto block = [&](int b, const uint32_t (&dw)[7]) {
        const u32x4* xb = xs + (int64_t)b * kSlots + g;
        // the table and activation reads of each half block are issued
        // before the first of its MFMAs waits on one
        float4_t c = {0.f, 0.f, 0.f, 0.f};
        auto half = [&](auto I0, auto N) {
            constexpr int i0 = decltype(I0)::value, nn = decltype(N)::value;
            u32x2 tl[nn], th[nn];
            u32x4 xa[nn];
#pragma unroll
            for (int t = 0; t < nn; ++t) {
                // slot 4i + g: byte g of dword i
                const uint32_t code = (dw[i0 + t] >> sh) & 0xffu;
                const uint32_t hi = (code * 19u) >> 9;  // code / 27 for code <= 255
                tl[t] = lut_lo[code - 27u * hi];
                th[t] = lut_hi[hi];
                xa[t] = xb[4 * (i0 + t)];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < nn; ++t) c = mfma_h(xa[t], u32x4{tl[t].x, tl[t].y, th[t].x, th[t].y}, c);
        };
        // two halves keep the live registers at or under 64, eight waves per SIMD
        half(std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
        half(std::integral_constant<int, 4>{}, std::integral_constant<int, 3>{});
        const float s = half_bits_to_float(dw[6] >> 16);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(s, c[v], acc[v]);
    };

    for (int c = 0; c < kNBuf - 1 && c < nchunks; ++c) issue(c);
    for (int c = 0; c < nchunks; ++c) {
        // chunks issued after chunk c so far: up to c + kNBuf - 2
        const int later = (nchunks - 1 < c + kNBuf - 2 ? nchunks - 1 : c + kNBuf - 2) - c;
        wait_loads_le(later * wave_loads);
        __syncthreads();
        // the buffer refilled here was read in iteration c - 1, which every
        // wave has finished at the barrier above
        if (c + kNBuf - 1 < nchunks) issue(c + kNBuf - 1);
        const uint8_t* B = wbuf + (c % kNBuf) * kWBuf + n_l * (kRowPieces * 16);
        const int ncb = nblk - c * kCB < kCB ? nblk - c * kCB : kCB;
        for (int bl = wave; bl < ncb; bl += W) {
            uint32_t dw[7];
#pragma unroll
            for (int q = 0; q < 7; ++q) dw[q] = *(const uint32_t*)(B + 28 * bl + 4 * q);
            block(c * kCB + bl, dw);
        }
    }

    // ---- lane (n_l, g) holds activation rows 4g+v of weight row n_l; row 0
    // is the product (the other rows repeat it)
    if (W > 1) {
        if (wave > 0 && g == 0) red[(wave - 1) * 16 + n_l] = acc[0];
        __syncthreads();
        if (wave > 0) return;
        for (int ww = 1; ww < W; ++ww) acc[0] += red[(ww - 1) * 16 + n_l];
    }
    if (part) {
        if (g == 0 && n0 + n_l < n) part[(int64_t)piece * n + n0 + n_l] = acc[0];
        return;
    }
    if (g == 0 && n0 + n_l < n) {
        const int64_t o = n0 + n_l;
        if (y_dt == F32) store_out<F32>(y, o, acc[0]);
        else if (y_dt == F16) store_out<F16>(y, o, acc[0]);
        else store_out<BF16>(y, o, acc[0]);
    }
}

// Rows must start on 16-byte boundaries (a multiple of four blocks per row)
// for the 16-byte copies, and the activation slots must fit in LDS.
// Chunks of 16 blocks (448 bytes of a row) keep every chunk of a row on the
// row's own 64-byte alignment; measured, chunks whose copies start on odd
// 16-byte boundaries (4, 12 or 20 blocks) stream 30-130 % slower.
// Short rows: eight waves (four workgroups per compute unit at 40 blocks).
// Long rows: sixteen waves (two workgroups per compute unit), so that a
// compute unit holding one of the few workgroups still has four waves per
// SIMD.
using TqShort = TqCfg<8, 16>;  // rows of fewer than 64 blocks
using TqLong = TqCfg<16, 16>;

bool tq1_mv_fits(int64_t k) {
    const int64_t nblk = k / 128;
    if (nblk % 4 != 0) return false;
    const size_t lds = nblk >= 64 ? TqLong::lds_bytes(nblk) : TqShort::lds_bytes(nblk);
    return lds <= 160 * 1024;
}

// Split-K for rows that fill few workgroups (Ternary Bonsai
// "ternel_packed_model.py", the split-K budget of its decode dispatches: a
// tensor whose rows yield few tiles runs one short chain on an idle GPU).
// Fewer than 512 row tiles of 16 are split into ceil(1024 / tiles) pieces of
// at least 16 blocks, each a whole number of four blocks (16-byte aligned
// copies).  Measured on 5120x17408: 17.2 -> 13.9 us with four pieces,
// reduction included; the 17408-row shape (1088 tiles) is not split.
int tq1_mv_pieces(int64_t n, int64_t k, int* pnb_out) {
    const int64_t tiles = (n + 15) / 16, nblk = k / 128;
    *pnb_out = 0;
    if (!tq1_mv_fits(k) || tiles >= 512) return 1;
    int64_t pieces = (1024 + tiles - 1) / tiles;
    if (pieces > nblk / 16) pieces = nblk / 16;
    if (pieces < 2) return 1;
    int64_t pnb = (nblk + pieces - 1) / pieces;
    pnb = (pnb + 3) / 4 * 4;
    pieces = (nblk + pnb - 1) / pnb;
    if (pieces < 2) return 1;
    *pnb_out = (int)pnb;
    return (int)pieces;
}

hipError_t launch_tq1_mv(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y, int y_dt,
                         hipStream_t s, int pnb, float* part) {
    const int64_t nblk = pnb ? pnb : k / 128;  // blocks per workgroup
    const int pieces = pnb ? (int)((k / 128 + pnb - 1) / pnb) : 1;
    const dim3 grid((unsigned)((n + 15) / 16), (unsigned)pieces);
    if (nblk >= 64) {
        hipLaunchKernelGGL((tq1_mv_kernel<16, 16>), grid, dim3(64 * 16), TqLong::lds_bytes(nblk), s, w,
                           n, k, x, y, y_dt, pnb, part);
    } else {
        hipLaunchKernelGGL((tq1_mv_kernel<8, 16>), grid, dim3(64 * 8), TqShort::lds_bytes(nblk), s, w,
                           n, k, x, y, y_dt, pnb, part);
    }
    return hipGetLastError();
}

}  // namespace kq
