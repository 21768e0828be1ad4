// tq1mv.hip -- TQ1_G128 decode GEMV, one fp16 activation row (kq_qmv, m = 1).
//
// Ternary Bonsai "ternel_packed_model.py": format constants (28-byte block:
// 25 code bytes of five base-3 digits, a tail byte of three, fp16 scale) and
// the LUT23 GEMV section (decoding through a table instead of dividing each
// byte by powers of three).
//
// Here a code byte c = d0 + 3 d1 + 9 (d2 + 3 d3 + 9 d4) is decoded through two
// small tables, as the page splits it: c mod 9 gives the trits (d0-1, d1-1)
// as an fp16 pair, c div 9 the trits (d2-1, d3-1, d4-1); together with three
// zeros they are eight fp16 values, exactly one 16x16x32 MFMA operand slice.
// The tables are 9 and 27 entries long, so lanes that read different entries
// never share an LDS bank and lanes that read the same entry are served by
// one broadcast.  The contraction order is permuted so that each lane group's eight
// MFMA k-slots are the five columns of one code byte: the activations are
// staged in LDS once per workgroup in the same 8-wide "slot" layout (columns
// 5s..5s+4 of byte s, then zeros; the tail byte's slot holds columns
// 125..127).  A block of 128 weights is 28 slots (25 code bytes, the tail,
// and the two scale bytes, whose activation slots are zero), i.e. seven
// MFMAs; the fp16 scale multiplies each block's fp32 result.  All products
// (+-x or 0) are exact; accumulation is fp32.
//
// A workgroup owns 16 weight rows.  Their weights stream through LDS in
// chunks of 16 blocks (coalesced global->LDS copies, double buffered); the W
// waves take the blocks of a chunk in turn and combine their partial sums
// through LDS at the end.  Each block issues all of its table and activation
// reads before its first MFMA, so their LDS latency overlaps.
#include "kq_device.h"
#include "kq_internal.h"
#include "lds_dma.h"

namespace kq {

namespace {

constexpr int kSlots = 28;            // MFMA slots per 128-weight block
// LDS tables: 9 dwords (two trits) then, from byte 64, 32 8-byte entries
// (three trits; entries past 26 serve the scale bytes, whose activations are
// zero)
constexpr int kLut3Off = 64;
constexpr int kLutBytes = kLut3Off + 32 * 8;

__device__ __forceinline__ float4_t mfma_h(const u32x4& a, const u32x4& b, const float4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

}  // namespace

// Weights stream through LDS: chunks of kCB blocks of the 16 rows, copied
// with coalesced global->LDS 16-byte loads (each row's chunk is 448
// contiguous bytes) and double buffered.  LDS rows are padded by one 16-byte
// piece so that the 16 lanes reading one dword of 16 rows hit 16 banks.
constexpr int kCB = 16;                       // blocks per chunk
constexpr int kRowPieces = kCB * 28 / 16 + 1; // 16-byte pieces per LDS row (+1 pad)
constexpr int kWBuf = 16 * kRowPieces * 16;   // bytes of one chunk buffer

template <int W>
__global__ __launch_bounds__(64 * W) void tq1_mv_kernel(const uint8_t* __restrict__ w, int64_t n,
                                                        int64_t k, const uint16_t* __restrict__ x,
                                                        void* __restrict__ y, int y_dt) {
    constexpr int NPIECE = 16 * kRowPieces;
    constexpr int WLOADS = (NPIECE + 63) / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* lut2 = (uint32_t*)smem;                            // [9]
    u32x2* lut3 = (u32x2*)(smem + kLut3Off);                     // [32]
    uint8_t* wbuf = smem + kLutBytes;                           // [2][kWBuf]
    u32x4* xs = (u32x4*)(smem + kLutBytes + 2 * kWBuf);         // [nblk * 28] slots
    const int nblk = (int)(k / 128);
    float* red = (float*)((uint8_t*)xs + (size_t)nblk * kSlots * 16);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t row_bytes = (int64_t)nblk * 28;
    const int nchunks = (nblk + kCB - 1) / kCB;

    // ---- tables of trits as fp16: -1, 0, +1 for digits 0, 1, 2
    auto trit = [](uint32_t d) -> uint32_t { return d == 0 ? 0xbc00u : d == 1 ? 0x0000u : 0x3c00u; };
    if (tid < 9) lut2[tid] = trit(tid % 3) | (trit(tid / 3) << 16);
    if (tid >= 64 && tid < 96) {
        const uint32_t j = tid - 64;
        lut3[j] = u32x2{trit(j % 3) | (trit((j / 3) % 3) << 16), trit((j / 9) % 3)};
    }
    // ---- activations in slot layout: slot s < 25 of block b holds columns
    // 128b + 5s .. +4, slot 25 columns 128b + 125 .. 127, the rest zeros.
    // Zero every slot, then scatter the columns read 8 at a time.
    for (int i = tid; i < nblk * kSlots; i += 64 * W) xs[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    {
        uint16_t* xh = (uint16_t*)xs;
        for (int i = tid; i < nblk * 16; i += 64 * W) {
            const u32x4 v = *(const u32x4*)(x + 8 * (int64_t)i);
            const int b = i >> 4, c0 = 8 * (i & 15);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = c0 + j;
                const int sl = c < 125 ? (c * 52429) >> 18 : 25;  // c / 5 for c < 128
                const int pos = c - 5 * sl;
                const uint32_t h = (v[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                xh[((b * kSlots + sl) << 3) + pos] = (uint16_t)h;
            }
        }
    }

    // ---- weight pieces of this lane: LDS slot p = 64 i + lane is piece
    // p % kRowPieces of row p / kRowPieces (the last piece of a row is
    // padding and is not loaded)
    const uint8_t* wbase = w + n0 * row_bytes;
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
    auto issue = [&](int chunk) {
        uint8_t* dst = wbuf + (chunk & 1) * kWBuf;
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
        // every table and activation read of the block is issued before the
        // first MFMA waits on one
        uint32_t t2[7];
        u32x2 t3[7];
        u32x4 xa[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            // slot 4i + g: byte g of dword i
            const uint32_t code = (dw[i] >> sh) & 0xffu;
            const uint32_t hi9 = (code * 57u) >> 9;  // code / 9 for code <= 255
            const uint32_t lo9 = code - 9u * hi9;
            t2[i] = lut2[lo9];
            t3[i] = lut3[hi9];
            xa[i] = xb[4 * i];
        }
        __builtin_amdgcn_sched_barrier(0);
        float4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 7; ++i) c = mfma_h(xa[i], u32x4{t2[i], t3[i].x, t3[i].y, 0u}, c);
        const float s = half_bits_to_float(dw[6] >> 16);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(s, c[v], acc[v]);
    };

    issue(0);
    for (int c = 0; c < nchunks; ++c) {
        wait_loads_le(0);
        __syncthreads();
        if (c + 1 < nchunks) issue(c + 1);
        const uint8_t* B = wbuf + (c & 1) * kWBuf + n_l * (kRowPieces * 16);
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
    if (g == 0 && n0 + n_l < n) {
        const int64_t o = n0 + n_l;
        if (y_dt == F32) store_out<F32>(y, o, acc[0]);
        else if (y_dt == F16) store_out<F16>(y, o, acc[0]);
        else store_out<BF16>(y, o, acc[0]);
    }
}

// LDS: tables, two weight buffers, activation slots (3.5 bytes per column),
// reduction.  Rows must start on 16-byte boundaries (a multiple of four
// blocks per row) for the 16-byte copies.
bool tq1_mv_fits(int64_t k) {
    return (k / 128) % 4 == 0 && kLutBytes + 2 * kWBuf + (k / 128) * kSlots * 16 + 7 * 16 * 4 <= 160 * 1024;
}

hipError_t launch_tq1_mv(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y, int y_dt,
                         hipStream_t s) {
    const int64_t nblk = k / 128;
    const dim3 grid((unsigned)((n + 15) / 16));
    const size_t base = (size_t)kLutBytes + 2 * kWBuf + (size_t)nblk * kSlots * 16;
    if (nblk >= 64) {
        hipLaunchKernelGGL(tq1_mv_kernel<8>, grid, dim3(512), base + 7 * 16 * 4, s, w, n, k, x, y, y_dt);
    } else {
        hipLaunchKernelGGL(tq1_mv_kernel<4>, grid, dim3(256), base + 3 * 16 * 4, s, w, n, k, x, y, y_dt);
    }
    return hipGetLastError();
}

}  // namespace kq
