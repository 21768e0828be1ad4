// cmv.hip -- decode GEMV (one fp16 activation row) for Q8_0 and the further
// GGUF codecs Q4_0, Q5_0, Q5_1, Q6_K, Q2_K, Q3_K and Q5_K (kq_qmv, m = 1).
//
// mlx-kquant "bindings.cpp": quantized_matmul in the decode regime; the
// codecs are the GGUF blocks that mlx-native "quantized_matmul_id_ggml.rs"
// dispatches (its mv_id kernel table), laid out as include/kq.h states.
//
// A workgroup owns 16 weight rows.  Their bytes stream through LDS in
// chunks of whole 16-byte-aligned units of blocks (coalesced global->LDS
// copies, double buffered); the activation row is copied into LDS once.
// Each lane takes one 32-weight chunk of R rows at a time: it decodes each
// row's chunk to exact fp16 integer pairs with an affine scale per 16
// weights (pair32.h) and multiplies them with the shared activations on
// v_dot2_f32_f16, so one activation read serves R rows.  Lanes of a wave
// that share a row are summed by lane shuffles, waves through LDS.
#include "kq_device.h"
#include "kq_internal.h"
#include "lds_dma.h"
#include "pair32.h"

namespace kq {

namespace {

// The smallest run of whole blocks whose bytes are a multiple of 16 (so
// every chunk of a 16-byte-aligned row starts 16-byte aligned): bytes and
// weights.
template <int C> struct Unit;
template <> struct Unit<Q8_0> { static constexpr int BYTES = 272, W = 256; };   // 8 blocks
template <> struct Unit<Q4_0> { static constexpr int BYTES = 144, W = 256; };   // 8 blocks
template <> struct Unit<Q5_0> { static constexpr int BYTES = 176, W = 256; };   // 8 blocks
template <> struct Unit<Q5_1> { static constexpr int BYTES = 192, W = 256; };   // 8 blocks
template <> struct Unit<Q6_K> { static constexpr int BYTES = 1680, W = 2048; }; // 8 super-blocks
template <> struct Unit<Q2_K> { static constexpr int BYTES = 336, W = 1024; };  // 4 super-blocks
template <> struct Unit<Q3_K> { static constexpr int BYTES = 880, W = 2048; };  // 8 super-blocks
template <> struct Unit<Q5_K> { static constexpr int BYTES = 176, W = 256; };   // 1 super-block
// With 4-byte copies (PB = 4) a unit need only be a whole number of dwords:
// Q6_K and Q3_K then stream rows of any whole number of 2 super-blocks.
template <int C, int PB> struct UnitP : Unit<C> {};
template <> struct UnitP<Q6_K, 4> { static constexpr int BYTES = 420, W = 512; };
template <> struct UnitP<Q3_K, 4> { static constexpr int BYTES = 220, W = 512; };
template <> struct UnitP<Q2_K, 4> { static constexpr int BYTES = 168, W = 512; };
template <int PB>
__device__ __forceinline__ void dma_piece(const void* src, uint32_t lds) {
    if constexpr (PB == 16) dma16(src, lds);
    else dma4(src, lds);
}

// W waves; CU units per chunk; R rows per lane task; PB bytes per copied
// piece (16: global_load_lds_dwordx4, 4: global_load_lds_dword)
template <int C, int W_, int CU_, int R_, int PB_ = 16>
struct CmvCfg {
    static constexpr int W = W_, CU = CU_, R = R_, PB = PB_;
    static constexpr int CHB = CU * UnitP<C, PB>::BYTES;      // chunk bytes of one row
    static constexpr int CHQ = CU * UnitP<C, PB>::W / 32;     // 32-weight chunks of one row per chunk
    // pieces per LDS row: the chunk, one piece of padding (read past by the
    // realigning dword reads), and one more if that count is even, so that
    // the 16 rows of a workgroup start on different bank groups
    static constexpr int ROW_PIECES = (CHB / PB + 1) | 1;
    static constexpr int ROW_BYTES = ROW_PIECES * PB;
    static constexpr int WBUF = 16 * ROW_BYTES;               // bytes of one chunk buffer (16 rows)
    static constexpr int NBUF = 2;
    static constexpr int RG = 16 / R;                         // row groups
    static constexpr int TASKS = RG * CHQ;                    // lane tasks per chunk
    static_assert(UnitP<C, PB>::BYTES % PB == 0, "units are whole pieces");
    static_assert(16 % R == 0 && 64 % RG == 0, "row groups tile a wave");
    static size_t lds_bytes(int64_t k) { return (size_t)NBUF * WBUF + (size_t)k * 2 + (size_t)W * 16 * 4; }
};

}  // namespace

template <int C, int W, int CU, int R, int PB = 16>
__global__ __launch_bounds__(64 * W) void cmv_kernel(const uint8_t* __restrict__ w, int64_t n, int64_t k,
                                                     const uint16_t* __restrict__ x, void* __restrict__ y,
                                                     int y_dt) {
    using Cfg = CmvCfg<C, W, CU, R, PB>;
    constexpr int kRowPieces = Cfg::ROW_PIECES, kWBuf = Cfg::WBUF, kNBuf = Cfg::NBUF, kRG = Cfg::RG;
    constexpr int NPIECE = 16 * kRowPieces;
    constexpr int WLOADS = (NPIECE + 63) / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* wbuf = smem;                                           // [kNBuf][kWBuf]
    uint16_t* xs = (uint16_t*)(smem + kNBuf * kWBuf);               // [k]
    float* red = (float*)(smem + kNBuf * kWBuf + (size_t)k * 2);    // [W][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t row_bytes = k / UnitP<C, PB>::W * UnitP<C, PB>::BYTES;  // (k is a whole number of units)
    const int nchunks = (int)(row_bytes / Cfg::CHB);                // whole chunks (k is a multiple of the chunk)

    // ---- the activation row into LDS (16-byte copies; k * 2 is a multiple of 16)
    // (lanes past the row's end issue nothing: a copy lands at 16 * lane
    // past its base, whatever the source)
    const int xpieces = (int)(k / 8);
    for (int p0 = 64 * wave; p0 < xpieces; p0 += 64 * W) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr((const uint8_t*)xs + 16 * (int64_t)p0));
        if (p0 + lane < xpieces) dma16(x + 8 * (int64_t)(p0 + lane), dst);
    }
    // ---- weight pieces of this lane: LDS piece p = 64 i + lane is piece
    // p % kRowPieces of row p / kRowPieces (pieces past the chunk are padding)
    const uint8_t* wbase = w + n0 * row_bytes;
    uint32_t woff[WL_PER_WAVE];
    bool wact[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int r = p / kRowPieces, q = p - r * kRowPieces;
        int64_t nr = n0 + r;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < 16 && q < Cfg::CHB / PB;
        woff[j] = (uint32_t)((nr - n0) * row_bytes) + (uint32_t)PB * (uint32_t)q;
    }
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    auto issue = [&](int chunk) {
        uint8_t* dst = wbuf + (chunk % kNBuf) * kWBuf;
        const uint8_t* src = wbase + (int64_t)chunk * Cfg::CHB;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                // padding pieces and pieces past the 16 rows are not copied
                // (every load instruction still has live lanes: each group of
                // 64 pieces holds pieces of a row)
                const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_addr(dst + 64 * PB * i));
                if (wact[j]) dma_piece<PB>(src + woff[j], dl);
            }
        }
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    const int rg = lane % kRG;  // this lane's row group: rows rg + kRG * j
    for (int c = 0; c < kNBuf - 1 && c < nchunks; ++c) issue(c);
    for (int c = 0; c < nchunks; ++c) {
        const int later = (nchunks - 1 < c + kNBuf - 2 ? nchunks - 1 : c + kNBuf - 2) - c;
        // the activation copies were issued before every weight chunk
        wait_loads_le(later * wave_loads);
        __syncthreads();
        if (c + kNBuf - 1 < nchunks) issue(c + kNBuf - 1);
        const uint8_t* B = wbuf + (c % kNBuf) * kWBuf;
        const int64_t kbase = (int64_t)c * (Cfg::CHQ * 32);
        for (int t = lane + 64 * wave; t < Cfg::TASKS; t += 64 * W) {
            const int cq = t / kRG;
            uint32_t p[R][16];
            float A[R][2], Bv[R][2];
            int64_t xa = 0, xb = 0;
#pragma unroll
            for (int j = 0; j < R; ++j)
                Pair32<C>::template decode<true>(B + (rg + kRG * j) * Cfg::ROW_BYTES, cq, p[j], A[j], Bv[j],
                                                 xa, xb);
            uint32_t xw[16];
            const u32x4* xp = (const u32x4*)(xs + kbase + xa);
            const u32x4* xq = (const u32x4*)(xs + kbase + xb);
            const u32x4 x0 = xp[0], x1 = xp[1], x2 = xq[0], x3 = xq[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) xw[e] = x0[e], xw[4 + e] = x1[e], xw[8 + e] = x2[e], xw[12 + e] = x3[e];
            float t0 = 0.f, t1 = 0.f;
            if (Pair32<C>::has_b) {
                t0 = sum16(xw);
                t1 = sum16(xw + 8);
            }
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float s = A[j][0] * dot16(p[j], xw);
                s = __builtin_fmaf(A[j][1], dot16(p[j] + 8, xw + 8), s);
                if (Pair32<C>::has_b) {
                    s = __builtin_fmaf(Bv[j][0], t0, s);
                    s = __builtin_fmaf(Bv[j][1], t1, s);
                }
                acc[j] += s;
            }
        }
    }

    // ---- lanes rg, rg + kRG, ... of every wave hold rows rg + kRG j
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int o = kRG; o < 64; o <<= 1)
            acc[j] += __shfl_xor(acc[j], o, 64);
    }
    if (lane < kRG) {
#pragma unroll
        for (int j = 0; j < R; ++j) red[wave * 16 + rg + kRG * j] = acc[j];
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float v = 0.f;
        for (int ww = 0; ww < W; ++ww) v += red[ww * 16 + lane];
        const int64_t o = n0 + lane;
        if (o < n) {
            if (y_dt == F32) store_out<F32>(y, o, v);
            else if (y_dt == F16) store_out<F16>(y, o, v);
            else store_out<BF16>(y, o, v);
        }
    }
}

// rows of this many weights and more take the LONG launch shapes
constexpr int64_t kLongRow = 8192;

// ---------------------------------------------------------------- 2..16 activation rows
// The same weight stream feeding the matrix cores: per 32-weight chunk two
// v_mfma_f32_16x16x16_f16 (one per 16-weight half), the activation rows as
// the A operand (rows past m read row 0 and are not stored) and the chunk's
// weights of the 16 rows as B.  Activations are staged per chunk next to the
// weights (8 or 16 rows).
// - The 32-weight blocks (Q8_0, Q4_0, Q5_0, Q5_1) fold their fp16 scale into
//   the weights (each weight rounded once to fp16, as in the prefill GEMM)
//   and the matrix cores accumulate across chunks.  A block whose weights
//   could overflow fp16 sends its wave to the exact form for that buffer.
// - The K-quants (and that exact form) multiply the exact fp16 integers of
//   Pair8; each half's fp32 result takes its weight row's scale A[h], and
//   B[h] times the half's activation sum (an MFMA against ones) for the
//   codecs with an offset.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4_t mfma4(const u32x2& a, const u32x2& b, const float4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b),
                                                 c, 0, 0, 0);
}

// W waves, CU units per chunk, S chunk buffers, MR staged activation rows
template <int C, int W_, int CU_, int S_, int MR_>
struct CmmCfg {
    static constexpr int W = W_, CU = CU_, S = S_, MR = MR_;
    static constexpr int CHB = CU * Unit<C>::BYTES, CHQ = CU * Unit<C>::W / 32, CHW = CHQ * 32;
    static constexpr int ROW_PIECES = (CHB / 16 + 1) | 1;
    static constexpr int WBUF = 16 * ROW_PIECES * 16;
    static constexpr int XSTRIDE = CHW * 2 + 16;                       // bytes per staged activation row
    static constexpr int XBUF = MR * XSTRIDE;
    static constexpr int BUF = WBUF + XBUF;                             // one stage: weights, activations
    static_assert((CHW * 2) % 1024 == 0, "an activation row's chunk is whole 1 KB copies");
    static constexpr size_t lds_bytes() { return S * (size_t)BUF; }
    static_assert(S >= 2 && W * 64 * 16 <= S * BUF, "buffers, and the final reduction fits in them");
};

template <int C, int W, int CU, int S, int MR>
__global__ __launch_bounds__(64 * W) void cmm_kernel(const uint8_t* __restrict__ w, int64_t n, int64_t k,
                                                     const uint16_t* __restrict__ x, int m,
                                                     void* __restrict__ y, int y_dt) {
    using Cfg = CmmCfg<C, W, CU, S, MR>;
    constexpr int kRowPieces = Cfg::ROW_PIECES, kBuf = Cfg::BUF, CHB = Cfg::CHB, CHQ = Cfg::CHQ;
    constexpr int NPIECE = 16 * kRowPieces, WLOADS = (NPIECE + 63) / 64, WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int XL_ROW = Cfg::CHW * 2 / 1024;                         // 1 KB copies per activation row
    constexpr int PER = CHQ / W;                                        // 32-weight chunks per wave and buffer
    static_assert(CHQ % W == 0, "the waves split a chunk buffer evenly");
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t row_bytes = k / Unit<C>::W * Unit<C>::BYTES;
    const int nchunks = (int)(row_bytes / CHB);
    const uint8_t* wbase = w + n0 * row_bytes;
    uint32_t woff[WL_PER_WAVE];
    bool wact[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j, p = 64 * i + lane;
        const int r = p / kRowPieces, q = p - r * kRowPieces;
        int64_t nr = n0 + r;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < 16 && q < CHB / 16;
        woff[j] = (uint32_t)((nr - n0) * row_bytes) + 16u * (uint32_t)q;
    }
    const int xl_total = m * XL_ROW;  // 1 KB activation copies per chunk
    // loads this wave issues per chunk: its weight copies, its share of the
    // activation copies
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    wave_loads += xl_total > wave ? (xl_total - wave + W - 1) / W : 0;
    auto issue = [&](int chunk) {
        uint8_t* dst = smem + (chunk % S) * kBuf;
        const uint8_t* src = wbase + (int64_t)chunk * CHB;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i));
                if (wact[j]) dma16(src + woff[j], dl);
            }
        }
        for (int i = wave; i < xl_total; i += W) {
            const int r = i / XL_ROW, c = i - r * XL_ROW;
            const uint8_t* xs = (const uint8_t*)(x + (int64_t)r * k + (int64_t)chunk * Cfg::CHW) + 1024 * c;
            dma16(xs + 16 * lane, __builtin_amdgcn_readfirstlane(
                                      lds_addr(dst + Cfg::WBUF + r * Cfg::XSTRIDE + 1024 * c)));
        }
    };

    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int xrow = n_l < m ? n_l : 0;
    const u32x2 ones = u32x2{0x3c003c00u, 0x3c003c00u};
    for (int c = 0; c < S - 1 && c < nchunks; ++c) issue(c);
    for (int c = 0; c < nchunks; ++c) {
        // chunks c + 1 .. c + S - 2 may stay in flight
        const int later = nchunks - 1 - c < S - 2 ? nchunks - 1 - c : S - 2;
        wait_loads_le(later * wave_loads);
        __syncthreads();  // chunk c has landed everywhere; every wave is done with chunk c - 1
        if (c + S - 1 < nchunks) issue(c + S - 1);
        const uint8_t* B = smem + (c % S) * kBuf;
        const uint8_t* wrow = B + n_l * (kRowPieces * 16);
        const uint8_t* xr = B + Cfg::WBUF + xrow * Cfg::XSTRIDE;
        // this wave's chunks: PER consecutive ones
        u32x2 a[PER][2];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int cq = wave * PER + i;
            a[i][0] = *(const u32x2*)(xr + 2 * (32 * cq + 4 * g));
            a[i][1] = *(const u32x2*)(xr + 2 * (32 * cq + 16 + 4 * g));
        }
        auto exact = [&](int i) {
            // unscaled integers on the matrix cores, each 16-weight half's
            // scale (and offset) applied to the fp32 results
            const int cq = wave * PER + i;
            u32x2 b0, b1;
            float A[2], Bv[2];
            Pair8<C>::decode(wrow, cq, g, b0, b1, A, Bv);
            const float4_t z = {0.f, 0.f, 0.f, 0.f};
            const float4_t c0 = mfma4(a[i][0], b0, z), c1 = mfma4(a[i][1], b1, z);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(A[0], c0[v], __builtin_fmaf(A[1], c1[v], acc[v]));
            if constexpr (Pair8<C>::has_b) {
                const float4_t s0 = mfma4(a[i][0], ones, z), s1 = mfma4(a[i][1], ones, z);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(Bv[0], s0[v], __builtin_fmaf(Bv[1], s1[v], acc[v]));
            }
        };
        if constexpr (Pair8<C>::foldable) {
            // the weights rounded once to fp16, accumulated by the matrix
            // cores; a wave holding a block whose weights could overflow fp16
            // takes the exact form for this chunk buffer
            u32x2 wv[PER][2];
            bool ok = true;
#pragma unroll
            for (int i = 0; i < PER; ++i) ok &= Pair8<C>::fold(wrow, wave * PER + i, g, wv[i][0], wv[i][1]);
            if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    acc = mfma4(a[i][0], wv[i][0], acc);
                    acc = mfma4(a[i][1], wv[i][1], acc);
                }
            } else {
                for (int i = 0; i < PER; ++i) exact(i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) exact(i);
        }
    }
    __syncthreads();  // every wave is done with the last chunk and no load is in flight
    float4_t* red = (float4_t*)smem;  // [W][64]
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int ww = 1; ww < W; ++ww) {
        const float4_t t = red[ww * 64 + lane];
        acc[0] += t[0], acc[1] += t[1], acc[2] += t[2], acc[3] += t[3];
    }
    // lane holds activation rows 4g + v of weight row n_l
    const int64_t o = n0 + n_l;
    if (o >= n) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = 4 * g + v;
        if (r >= m) continue;
        if (y_dt == F32) store_out<F32>(y, r * n + o, acc[v]);
        else if (y_dt == F16) store_out<F16>(y, r * n + o, acc[v]);
        else store_out<BF16>(y, r * n + o, acc[v]);
    }
}

// Launch shapes (waves, units per chunk), measured on the 14336x4096 and
// 4096x14336 GEMVs at 2, 4, 8 and 16 rows; rows of 8192 and more take LONG
// (256 workgroups on the 4096-row shape: sixteen waves each).  MR, the rows
// the activation buffer holds, is the fewest of 2, 4, 8, 16 that take m:
// smaller buffers let more workgroups share a compute unit (Q6_K at m = 2:
// 22.1 -> 16.6 us).  Deeper buffering (S > 2) measured slower: more LDS per
// workgroup only cuts occupancy.
template <int C, bool LONG, int MR> struct CmmPick {
    static constexpr int W = LONG ? 16 : MR == 16 ? 4 : 8;
    static constexpr int CU = LONG ? (MR == 16 ? 4 : 8) : (MR == 16 ? 2 : 4);
};
template <bool LONG, int MR> struct CmmPick<Q8_0, LONG, MR> {
    static constexpr int W = LONG ? 16 : 4, CU = LONG ? (MR == 16 ? 4 : 8) : 2;
};
template <bool LONG, int MR> struct CmmPick<Q5_K, LONG, MR> {
    static constexpr int W = LONG || MR == 16 ? 16 : 8;
    static constexpr int CU = LONG ? (MR == 16 ? 4 : 8) : MR == 16 ? 4 : MR == 8 ? 4 : 8;
};
template <bool LONG, int MR> struct CmmPick<Q2_K, LONG, MR> { static constexpr int W = LONG ? 16 : 8, CU = LONG ? 2 : 1; };
template <bool LONG, int MR> struct CmmPick<Q6_K, LONG, MR> { static constexpr int W = LONG ? 16 : 8, CU = 1; };
template <bool LONG, int MR> struct CmmPick<Q3_K, LONG, MR> { static constexpr int W = LONG ? 16 : 8, CU = 1; };

template <int C, bool LONG, int MR>
using CmmCfgR = CmmCfg<C, CmmPick<C, LONG, MR>::W, CmmPick<C, LONG, MR>::CU, 2, MR>;

// 16 staged rows fit in LDS for every codec but Q6_K, which takes 9..16 rows
// in two passes of 8
template <int C> constexpr bool kCmm16 = CmmCfgR<C, false, 16>::lds_bytes() <= 160 * 1024 &&
                                         CmmCfgR<C, true, 16>::lds_bytes() <= 160 * 1024;

template <int C, int MR>
static int cmm_variant_mr(int64_t k) {
    static_assert(CmmCfgR<C, true, MR>::lds_bytes() <= 160 * 1024 && CmmCfgR<C, false, MR>::lds_bytes() <= 160 * 1024,
                  "LDS budget");
    if (k <= 0) return -1;
    if (k >= kLongRow && k % CmmCfgR<C, true, MR>::CHW == 0) return 1;
    return k % CmmCfgR<C, false, MR>::CHW == 0 ? 0 : -1;
}
// the shape a product of m rows of k weights takes: 1 LONG, 0 the other, -1
// none (k is not a whole number of its chunks)
template <int C>
static int cmm_variant(int64_t k, int64_t m) {
    if (m <= 2) return cmm_variant_mr<C, 2>(k);
    if (m <= 4) return cmm_variant_mr<C, 4>(k);
    if (m <= 8 || !kCmm16<C>) return cmm_variant_mr<C, 8>(k);
    if constexpr (kCmm16<C>) return cmm_variant_mr<C, 16>(k);
    return -1;
}
bool cmm_fits(int codec, int64_t k, int64_t m) {
    if (m < 2 || m > 16) return false;
    switch (codec) {
    case Q8_0: return cmm_variant<Q8_0>(k, m) >= 0;
    case Q4_0: return cmm_variant<Q4_0>(k, m) >= 0;
    case Q5_0: return cmm_variant<Q5_0>(k, m) >= 0;
    case Q5_1: return cmm_variant<Q5_1>(k, m) >= 0;
    case Q6_K: return cmm_variant<Q6_K>(k, m) >= 0;
    case Q2_K: return cmm_variant<Q2_K>(k, m) >= 0;
    case Q3_K: return cmm_variant<Q3_K>(k, m) >= 0;
    case Q5_K: return cmm_variant<Q5_K>(k, m) >= 0;
    default: return false;
    }
}

template <int C, bool LONG, int MR>
static hipError_t cmm_go(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int m, void* y, int y_dt,
                         hipStream_t s) {
    using Cfg = CmmCfgR<C, LONG, MR>;
    hipLaunchKernelGGL((cmm_kernel<C, Cfg::W, Cfg::CU, Cfg::S, Cfg::MR>), dim3((unsigned)((n + 15) / 16)),
                       dim3(64 * Cfg::W), Cfg::lds_bytes(), s, w, n, k, x, m, y, y_dt);
    return hipGetLastError();
}
template <int C, int MR>
static hipError_t cmm_go_k(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int m, void* y, int y_dt,
                           hipStream_t s) {
    if (cmm_variant_mr<C, MR>(k) == 1) return cmm_go<C, true, MR>(w, n, k, x, m, y, y_dt, s);
    return cmm_go<C, false, MR>(w, n, k, x, m, y, y_dt, s);
}

template <int C>
static hipError_t cmm_launch_c(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int64_t m, void* y,
                               int y_dt, hipStream_t s) {
    if (m <= 2) return cmm_go_k<C, 2>(w, n, k, x, (int)m, y, y_dt, s);
    if (m <= 4) return cmm_go_k<C, 4>(w, n, k, x, (int)m, y, y_dt, s);
    if (m <= 8) return cmm_go_k<C, 8>(w, n, k, x, (int)m, y, y_dt, s);
    if constexpr (kCmm16<C>) {
        return cmm_go_k<C, 16>(w, n, k, x, (int)m, y, y_dt, s);
    } else {
        const size_t ysz = y_dt == F32 ? 4 : 2;
        const hipError_t e = cmm_go_k<C, 8>(w, n, k, x, 8, y, y_dt, s);
        if (e != hipSuccess) return e;
        return cmm_go_k<C, 8>(w, n, k, x + 8 * k, (int)m - 8, (uint8_t*)y + 8 * n * ysz, y_dt, s);
    }
}

hipError_t launch_cmm(int codec, const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int64_t m, void* y,
                      int y_dt, hipStream_t s) {
    switch (codec) {
    case Q8_0: return cmm_launch_c<Q8_0>(w, n, k, x, m, y, y_dt, s);
    case Q4_0: return cmm_launch_c<Q4_0>(w, n, k, x, m, y, y_dt, s);
    case Q5_0: return cmm_launch_c<Q5_0>(w, n, k, x, m, y, y_dt, s);
    case Q5_1: return cmm_launch_c<Q5_1>(w, n, k, x, m, y, y_dt, s);
    case Q6_K: return cmm_launch_c<Q6_K>(w, n, k, x, m, y, y_dt, s);
    case Q2_K: return cmm_launch_c<Q2_K>(w, n, k, x, m, y, y_dt, s);
    case Q3_K: return cmm_launch_c<Q3_K>(w, n, k, x, m, y, y_dt, s);
    default: return cmm_launch_c<Q5_K>(w, n, k, x, m, y, y_dt, s);
    }
}

// Launch shapes (measured on the 14336x4096 and 4096x14336 GEMVs): rows of
// fewer than 8192 weights take four waves, two rows per lane task; longer
// rows, whose few workgroups leave compute units short of waves, take more
// waves and longer chunks.
template <int C, bool LONG> struct CmvPick;
template <> struct CmvPick<Q8_0, false> { using Cfg = CmvCfg<Q8_0, 4, 4, 2>; };
template <> struct CmvPick<Q8_0, true> { using Cfg = CmvCfg<Q8_0, 16, 8, 1>; };
template <> struct CmvPick<Q4_0, false> { using Cfg = CmvCfg<Q4_0, 4, 4, 2>; };
template <> struct CmvPick<Q5_0, false> { using Cfg = CmvCfg<Q5_0, 4, 4, 2>; };
template <> struct CmvPick<Q5_1, false> { using Cfg = CmvCfg<Q5_1, 4, 4, 2>; };
template <> struct CmvPick<Q5_K, false> { using Cfg = CmvCfg<Q5_K, 8, 4, 1>; };
template <> struct CmvPick<Q2_K, false> { using Cfg = CmvCfg<Q2_K, 8, 2, 2>; };
template <> struct CmvPick<Q6_K, false> { using Cfg = CmvCfg<Q6_K, 8, 1, 1>; };
template <> struct CmvPick<Q3_K, false> { using Cfg = CmvCfg<Q3_K, 8, 2, 2>; };
template <> struct CmvPick<Q4_0, true> { using Cfg = CmvCfg<Q4_0, 16, 8, 1>; };
template <> struct CmvPick<Q5_0, true> { using Cfg = CmvCfg<Q5_0, 16, 8, 1>; };
template <> struct CmvPick<Q5_1, true> { using Cfg = CmvCfg<Q5_1, 16, 8, 1>; };
template <> struct CmvPick<Q5_K, true> { using Cfg = CmvCfg<Q5_K, 16, 8, 1>; };
template <> struct CmvPick<Q2_K, true> { using Cfg = CmvCfg<Q2_K, 8, 2, 2>; };
template <> struct CmvPick<Q6_K, true> { using Cfg = CmvCfg<Q6_K, 8, 1, 1>; };
template <> struct CmvPick<Q3_K, true> { using Cfg = CmvCfg<Q3_K, 8, 1, 1>; };


template <int C, bool LONG>
static bool fits_cfg(int64_t k) {
    using Cfg = typename CmvPick<C, LONG>::Cfg;
    return k % (Cfg::CHQ * 32) == 0 && Cfg::lds_bytes(k) <= 160 * 1024;
}
// Q6_K and Q3_K rows that are no whole number of their 2048-weight units
// stream by 4-byte copies in chunks of 1024 weights (or 512)
template <int C> constexpr bool kDword = C == Q6_K || C == Q3_K;
template <int C, int CU4> using CmvCfg4 = CmvCfg<C, 8, CU4, 1, 4>;

template <int C>
static bool fits16_c(int64_t k) {
    return k >= kLongRow ? fits_cfg<C, true>(k) : fits_cfg<C, false>(k);
}
template <int C>
static bool fits_c(int64_t k) {
    if (fits16_c<C>(k)) return true;
    if constexpr (kDword<C>) return k > 0 && k % 512 == 0 && CmvCfg4<C, 1>::lds_bytes(k) <= 160 * 1024;
    return false;
}

bool cmv_fits(int codec, int64_t k) {
    switch (codec) {
    case Q8_0: return fits_c<Q8_0>(k);
    case Q4_0: return fits_c<Q4_0>(k);
    case Q5_0: return fits_c<Q5_0>(k);
    case Q5_1: return fits_c<Q5_1>(k);
    case Q6_K: return fits_c<Q6_K>(k);
    case Q2_K: return fits_c<Q2_K>(k);
    case Q3_K: return fits_c<Q3_K>(k);
    case Q5_K: return fits_c<Q5_K>(k);
    default: return false;
    }
}

template <int C, bool LONG>
static hipError_t launch_cfg(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y, int y_dt,
                             hipStream_t s) {
    using Cfg = typename CmvPick<C, LONG>::Cfg;
    constexpr auto kern = cmv_kernel<C, Cfg::W, Cfg::CU, Cfg::R>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((n + 15) / 16)), dim3(64 * Cfg::W), Cfg::lds_bytes(k), s, w, n, k,
                       x, y, y_dt);
    return hipGetLastError();
}
template <int C, int CU4>
static hipError_t launch_cfg4(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y, int y_dt,
                              hipStream_t s) {
    using Cfg = CmvCfg4<C, CU4>;
    constexpr auto kern = cmv_kernel<C, Cfg::W, Cfg::CU, Cfg::R, 4>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((n + 15) / 16)), dim3(64 * Cfg::W), Cfg::lds_bytes(k), s, w, n, k,
                       x, y, y_dt);
    return hipGetLastError();
}
template <int C>
static hipError_t launch_c(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y, int y_dt,
                           hipStream_t s) {
    if constexpr (kDword<C>) {
        if (!fits16_c<C>(k))
            return k % 1024 == 0 ? launch_cfg4<C, 2>(w, n, k, x, y, y_dt, s) : launch_cfg4<C, 1>(w, n, k, x, y, y_dt, s);
    }
    return k >= kLongRow ? launch_cfg<C, true>(w, n, k, x, y, y_dt, s) : launch_cfg<C, false>(w, n, k, x, y, y_dt, s);
}

hipError_t launch_cmv(int codec, const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y,
                      int y_dt, hipStream_t s) {
    switch (codec) {
    case Q8_0: return launch_c<Q8_0>(w, n, k, x, y, y_dt, s);
    case Q4_0: return launch_c<Q4_0>(w, n, k, x, y, y_dt, s);
    case Q5_0: return launch_c<Q5_0>(w, n, k, x, y, y_dt, s);
    case Q5_1: return launch_c<Q5_1>(w, n, k, x, y, y_dt, s);
    case Q6_K: return launch_c<Q6_K>(w, n, k, x, y, y_dt, s);
    case Q2_K: return launch_c<Q2_K>(w, n, k, x, y, y_dt, s);
    case Q3_K: return launch_c<Q3_K>(w, n, k, x, y, y_dt, s);
    default: return launch_c<Q5_K>(w, n, k, x, y, y_dt, s);
    }
}

// ---------------------------------------------------------------- one token, expert-routed
// The one-row kernel's weight stream for the single-token MoE forms, with
// the expert ids read directly (no schedule), as moe_dec.hip does for Q4_K:
// - cglu1_kernel (kq_moe_glu, fp16 activations): grid (row tile, slot); the
//   slot expert's 16 gate rows and the same 16 up rows stream together (32
//   LDS rows), and one lane task decodes a 32-weight chunk of gate row i and
//   of up row i against one activation read.  h = act(gate, up) is formed
//   before the single store; a slot with an invalid id gets NaN rows.
// - cdown1_kernel (kq_qmm_id with scores): the down projection with the
//   weighted sum over the token's slots fused in.  The slots' activation rows
//   are staged once; the workgroup's 16 rows walk the slots' experts in slot
//   order as one row of S*k weights, and each lane task's partial sum is
//   scaled by its slot's router weight.  fp32 activations are split per slot
//   row into fp16 hi + lo parts of the row scaled by a power of two (its
//   largest magnitude in [2^14, 2^15): 22 significant bits), both on
//   v_dot2_f32_f16.  A token with an invalid id gets NaN outputs.

__device__ __forceinline__ void put_dt(void* y, int64_t i, int dt, float v) {
    if (dt == F32) store_out<F32>(y, i, v);
    else if (dt == F16) store_out<F16>(y, i, v);
    else store_out<BF16>(y, i, v);
}

// 16 fp32 values times 2^ne as fp16 hi and lo pairs (hi + lo holds 22
// significant bits of each); the exponent that puts a row's largest
// magnitude in [2^14, 2^15) (0 for a zero or non-finite maximum)
__device__ __forceinline__ void split16(const uint32_t (&v)[16], int ne, uint32_t (&hw)[8], uint32_t (&lw)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float f0 = __builtin_ldexpf(__builtin_bit_cast(float, v[2 * q]), ne);
        const float f1 = __builtin_ldexpf(__builtin_bit_cast(float, v[2 * q + 1]), ne);
        const _Float16 h0 = (_Float16)f0, h1 = (_Float16)f1;
        const _Float16 l0 = (_Float16)(f0 - (float)h0), l1 = (_Float16)(f1 - (float)h1);
        hw[q] = __builtin_bit_cast(uint32_t, h2_t{h0, h1});
        lw[q] = __builtin_bit_cast(uint32_t, h2_t{l0, l1});
    }
}
__device__ __forceinline__ int split_exponent(float mx) {
    int ex = 0;
    if (mx > 0.f && mx <= 3.402823466e38f) {
        __builtin_frexpf(mx, &ex);
        ex -= 15;
    }
    return ex;
}

template <int C, int W, int CU, int PB = 16>
__global__ __launch_bounds__(64 * W) void cglu1_kernel(SkinnyArgs a) {
    using Cfg = CmvCfg<C, W, CU, 2, PB>;
    constexpr int kRowPieces = Cfg::ROW_PIECES, kNBuf = 2, kWBuf = 2 * Cfg::WBUF;  // 32 LDS rows
    constexpr int NPIECE = 32 * kRowPieces, WLOADS = (NPIECE + 63) / 64, WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int TASKS = 16 * Cfg::CHQ;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* wbuf = smem;                                             // [kNBuf][32 rows]
    uint16_t* xs = (uint16_t*)(smem + kNBuf * kWBuf);                 // [k]
    float* red = (float*)(smem + kNBuf * kWBuf + (size_t)a.k * 2);    // [W][2][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = a.n, k = a.k, n0 = (int64_t)blockIdx.x * 16, slot = blockIdx.y;
    const uint32_t e = slot_expert(a.ids, slot, a.top_k, a.shexp, a.n_experts);
    if ((int64_t)e >= a.n_experts + a.shexp) {
        if (tid < 16 && n0 + tid < n) put_dt(a.y, slot * a.y_row + n0 + tid, a.y_dt, __builtin_nanf(""));
        return;
    }
    const int64_t row_bytes = a.row_bytes;
    const int nchunks = (int)(row_bytes / Cfg::CHB);
    const uint8_t* wg = expert_base(a.w, a.w_sh, e, a.n_experts, a.expert_stride) + n0 * row_bytes;
    const uint8_t* wu = expert_base(a.w2, a.w2_sh, e, a.n_experts, a.expert_stride) + n0 * row_bytes;

    // ---- the token's activation row into LDS
    const uint16_t* x = (const uint16_t*)a.x;
    const int xpieces = (int)(k / 8);
    for (int p0 = 64 * wave; p0 < xpieces; p0 += 64 * W) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr((const uint8_t*)xs + 16 * (int64_t)p0));
        if (p0 + lane < xpieces) dma16(x + 8 * (int64_t)(p0 + lane), dst);
    }
    // ---- weight pieces: LDS piece p = 64 i + lane is piece p % kRowPieces of
    // LDS row p / kRowPieces (rows 0..15 gate, 16..31 up)
    uint32_t woff[WL_PER_WAVE];
    bool wact[WL_PER_WAVE], wup[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int r = p / kRowPieces, q = p - r * kRowPieces;
        const int rr = r & 15;
        int64_t nr = n0 + rr;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < 32 && q < Cfg::CHB / PB;
        wup[j] = r >= 16;
        woff[j] = (uint32_t)((nr - n0) * row_bytes) + (uint32_t)PB * (uint32_t)q;
    }
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    auto issue = [&](int chunk) {
        uint8_t* dst = wbuf + (chunk % kNBuf) * kWBuf;
        const int64_t cb = (int64_t)chunk * Cfg::CHB;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_addr(dst + 64 * PB * i));
                if (wact[j]) dma_piece<PB>((wup[j] ? wu : wg) + cb + woff[j], dl);
            }
        }
    };

    float acc[2] = {0.f, 0.f};  // gate, up
    const int rg = lane & 15;   // this lane's row
    for (int c = 0; c < kNBuf - 1 && c < nchunks; ++c) issue(c);
    for (int c = 0; c < nchunks; ++c) {
        const int later = (nchunks - 1 < c + kNBuf - 2 ? nchunks - 1 : c + kNBuf - 2) - c;
        wait_loads_le(later * wave_loads);
        __syncthreads();
        if (c + kNBuf - 1 < nchunks) issue(c + kNBuf - 1);
        const uint8_t* B = wbuf + (c % kNBuf) * kWBuf;
        const int64_t kbase = (int64_t)c * (Cfg::CHQ * 32);
        for (int t = lane + 64 * wave; t < TASKS; t += 64 * W) {
            const int cq = t >> 4;
            uint32_t pw[2][16];
            float A[2][2], Bv[2][2];
            int64_t xa = 0, xb = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                Pair32<C>::template decode<true>(B + (rg + 16 * j) * Cfg::ROW_BYTES, cq, pw[j], A[j], Bv[j],
                                                 xa, xb);
            uint32_t xw[16];
            const u32x4* xp = (const u32x4*)(xs + kbase + xa);
            const u32x4* xq = (const u32x4*)(xs + kbase + xb);
            const u32x4 x0 = xp[0], x1 = xp[1], x2 = xq[0], x3 = xq[1];
#pragma unroll
            for (int q = 0; q < 4; ++q) xw[q] = x0[q], xw[4 + q] = x1[q], xw[8 + q] = x2[q], xw[12 + q] = x3[q];
            float t0 = 0.f, t1 = 0.f;
            if (Pair32<C>::has_b) {
                t0 = sum16(xw);
                t1 = sum16(xw + 8);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float sj = A[j][0] * dot16(pw[j], xw);
                sj = __builtin_fmaf(A[j][1], dot16(pw[j] + 8, xw + 8), sj);
                if (Pair32<C>::has_b) {
                    sj = __builtin_fmaf(Bv[j][0], t0, sj);
                    sj = __builtin_fmaf(Bv[j][1], t1, sj);
                }
                acc[j] += sj;
            }
        }
    }
    // ---- lanes rg, rg + 16, rg + 32, rg + 48 of every wave hold row rg
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        acc[j] += __shfl_xor(acc[j], 16, 64);
        acc[j] += __shfl_xor(acc[j], 32, 64);
    }
    if (lane < 16) red[(wave * 2 + 0) * 16 + lane] = acc[0], red[(wave * 2 + 1) * 16 + lane] = acc[1];
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float gs = 0.f, us = 0.f;
        for (int ww = 0; ww < W; ++ww) gs += red[(ww * 2 + 0) * 16 + lane], us += red[(ww * 2 + 1) * 16 + lane];
        if (n0 + lane < n) put_dt(a.y, slot * a.y_row + n0 + lane, a.y_dt, glu_act(a.act, gs, us, a.limit));
    }
}

template <int C, int W, int CU, int R, bool XF32>
__global__ __launch_bounds__(64 * W) void cdown1_kernel(DownMixArgs d) {
    using Cfg = CmvCfg<C, W, CU, R>;
    constexpr int kRowPieces = Cfg::ROW_PIECES, kWBuf = Cfg::WBUF, kNBuf = 2, kRG = Cfg::RG;
    constexpr int NPIECE = 16 * kRowPieces, WLOADS = (NPIECE + 63) / 64, WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int ESZ = XF32 ? 4 : 2;  // staged bytes per activation
    extern __shared__ __align__(16) uint8_t smem[];
    const int S = (int)d.top_k;
    const int64_t n = d.n, k = d.k, n0 = (int64_t)blockIdx.x * 16;
    uint8_t* wbuf = smem;                                               // [kNBuf][kWBuf]
    uint8_t* xs = smem + kNBuf * kWBuf;                                 // [S][k] staged activations
    int32_t* xe = (int32_t*)(xs + (size_t)S * k * ESZ);                 // [S] row exponents (fp32)
    float* red = (float*)(xe + 16);                                     // [W][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // a token with an invalid expert id has NaN outputs
    bool bad = false;
    for (int r = 0; r < S; ++r)
        bad |= (int64_t)slot_expert(d.ids, r, S, d.shexp, d.n_experts) >= d.n_experts + d.shexp;
    if (bad) {
        if (tid < 16 && n0 + tid < n) put_dt(d.y, n0 + tid, d.y_dt, __builtin_nanf(""));
        return;
    }
    const int64_t row_bytes = d.row_bytes;
    const int cps = (int)(row_bytes / Cfg::CHB);  // chunks per slot (k is a multiple of the chunk)
    const int nchunks = S * cps;

    // ---- the slots' activation rows into LDS (slot-major, ESZ bytes each)
    {
        const int64_t ppr = k * ESZ / 16;  // 16-byte pieces per row
        const int64_t total = S * ppr;
        const uint8_t* xb = (const uint8_t*)d.x;
        for (int64_t p0 = 64 * wave; p0 < total; p0 += 64 * W) {
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(xs + 16 * p0));
            const int64_t p = p0 + lane;
            if (p < total) {
                const int64_t r = p / ppr, q = p - r * ppr;
                dma16(xb + (d.slotted ? r * k * ESZ : 0) + 16 * q, dst);
            }
        }
    }
    // ---- weight pieces (as in cmv_kernel), from the expert of each chunk's slot
    uint32_t woff[WL_PER_WAVE];
    bool wact[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int r = p / kRowPieces, q = p - r * kRowPieces;
        int64_t nr = n0 + r;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < 16 && q < Cfg::CHB / 16;
        woff[j] = (uint32_t)((nr - n0) * row_bytes) + 16u * (uint32_t)q;
    }
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    auto issue = [&](int chunk) {
        uint8_t* dst = wbuf + (chunk % kNBuf) * kWBuf;
        const int r = chunk / cps, lc = chunk - r * cps;
        const uint8_t* src = expert_base(d.w, d.w_sh, slot_expert(d.ids, r, S, d.shexp, d.n_experts), d.n_experts,
                                         d.expert_stride) +
                             n0 * row_bytes + (int64_t)lc * Cfg::CHB;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i));
                if (wact[j]) dma16(src + woff[j], dl);
            }
        }
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    const int rg = lane % kRG;
    for (int c = 0; c < kNBuf - 1 && c < nchunks; ++c) issue(c);
    for (int c = 0; c < nchunks; ++c) {
        const int later = (nchunks - 1 < c + kNBuf - 2 ? nchunks - 1 : c + kNBuf - 2) - c;
        wait_loads_le(later * wave_loads);  // (the activation copies were issued before every weight chunk)
        __syncthreads();
        if (c + kNBuf - 1 < nchunks) issue(c + kNBuf - 1);
        if (XF32 && c == 0) {
            // each slot row's exponent, then its values scaled by 2^-e and
            // split in place into fp16 hi and lo: every 16 floats (64 bytes)
            // become 16 hi halves then 16 lo halves
            for (int r = wave; r < S; r += W) {
                const float* row = (const float*)xs + (int64_t)r * k;
                float mx = 0.f;
                for (int64_t i = lane; i < k; i += 64) mx = __builtin_fmaxf(mx, __builtin_fabsf(row[i]));
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o, 64));
                if (lane == 0) xe[r] = split_exponent(mx);
            }
            __syncthreads();
            for (int64_t gi = tid; gi < (int64_t)S * k / 16; gi += 64 * W) {
                const int ne = -xe[(gi * 16) / k];
                u32x4* g4 = (u32x4*)(xs + 64 * gi);
                uint32_t v[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 u = g4[q];
                    v[4 * q] = u.x, v[4 * q + 1] = u.y, v[4 * q + 2] = u.z, v[4 * q + 3] = u.w;
                }
                uint32_t hw[8], lw[8];
                split16(v, ne, hw, lw);
                g4[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                g4[1] = u32x4{hw[4], hw[5], hw[6], hw[7]};
                g4[2] = u32x4{lw[0], lw[1], lw[2], lw[3]};
                g4[3] = u32x4{lw[4], lw[5], lw[6], lw[7]};
            }
            __syncthreads();
        }
        const uint8_t* B = wbuf + (c % kNBuf) * kWBuf;
        const int r = c / cps;
        const float sc = d.scores[r];
        const int ex = XF32 ? xe[r] : 0;
        const int64_t kbase = (int64_t)r * k + (int64_t)(c - r * cps) * (Cfg::CHQ * 32);
        for (int t = lane + 64 * wave; t < Cfg::TASKS; t += 64 * W) {
            const int cq = t / kRG;
            uint32_t p[R][16];
            float A[R][2], Bv[R][2];
            int64_t xa = 0, xb = 0;
#pragma unroll
            for (int j = 0; j < R; ++j)
                Pair32<C>::template decode<true>(B + (rg + kRG * j) * (kRowPieces * 16), cq, p[j], A[j], Bv[j],
                                                 xa, xb);
            if constexpr (!XF32) {
                uint32_t xw[16];
                const u32x4* xp = (const u32x4*)((const uint16_t*)xs + kbase + xa);
                const u32x4* xq = (const u32x4*)((const uint16_t*)xs + kbase + xb);
                const u32x4 x0 = xp[0], x1 = xp[1], x2 = xq[0], x3 = xq[1];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xw[q] = x0[q], xw[4 + q] = x1[q], xw[8 + q] = x2[q], xw[12 + q] = x3[q];
                float t0 = 0.f, t1 = 0.f;
                if (Pair32<C>::has_b) {
                    t0 = sum16(xw);
                    t1 = sum16(xw + 8);
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float sj = A[j][0] * dot16(p[j], xw);
                    sj = __builtin_fmaf(A[j][1], dot16(p[j] + 8, xw + 8), sj);
                    if (Pair32<C>::has_b) {
                        sj = __builtin_fmaf(Bv[j][0], t0, sj);
                        sj = __builtin_fmaf(Bv[j][1], t1, sj);
                    }
                    acc[j] = __builtin_fmaf(sc, sj, acc[j]);
                }
            } else {
                // 16-element groups at (kbase + xa) / 16 and (kbase + xb) / 16:
                // 8 dwords of hi pairs, then 8 of lo pairs
                const u32x4* ga = (const u32x4*)(xs + 4 * (kbase + xa));
                const u32x4* gb = (const u32x4*)(xs + 4 * (kbase + xb));
                uint32_t ha[8], la[8], hb[8], lb[8];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const u32x4 u0 = ga[q], u1 = ga[2 + q], u2 = gb[q], u3 = gb[2 + q];
#pragma unroll
                    for (int z = 0; z < 4; ++z)
                        ha[4 * q + z] = u0[z], la[4 * q + z] = u1[z], hb[4 * q + z] = u2[z], lb[4 * q + z] = u3[z];
                }
                float t0 = 0.f, t1 = 0.f;
                if (Pair32<C>::has_b) {
                    t0 = sum16(ha) + sum16(la);
                    t1 = sum16(hb) + sum16(lb);
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float sj = A[j][0] * (dot16(p[j], ha) + dot16(p[j], la));
                    sj = __builtin_fmaf(A[j][1], dot16(p[j] + 8, hb) + dot16(p[j] + 8, lb), sj);
                    if (Pair32<C>::has_b) {
                        sj = __builtin_fmaf(Bv[j][0], t0, sj);
                        sj = __builtin_fmaf(Bv[j][1], t1, sj);
                    }
                    acc[j] += __builtin_ldexpf(sc * sj, ex);
                }
            }
        }
    }
    // ---- lanes rg, rg + kRG, ... of every wave hold rows rg + kRG j
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int o = kRG; o < 64; o <<= 1)
            acc[j] += __shfl_xor(acc[j], o, 64);
    }
    if (lane < kRG) {
#pragma unroll
        for (int j = 0; j < R; ++j) red[wave * 16 + rg + kRG * j] = acc[j];
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float v = 0.f;
        for (int ww = 0; ww < W; ++ww) v += red[ww * 16 + lane];
        if (n0 + lane < n) put_dt(d.y, n0 + lane, d.y_dt, v);
    }
}

// fp32 activation rows split once for every workgroup of cdown1s_kernel:
// one workgroup per row
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ x, int64_t k,
                                                         uint8_t* __restrict__ out, int32_t* __restrict__ xexp) {
    __shared__ float part[4];
    __shared__ int ex_s;
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const float* row = x + r * k;
    float mx = 0.f;
    for (int64_t c = tid; c < k; c += 256) mx = __builtin_fmaxf(mx, __builtin_fabsf(row[c]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0) part[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        ex_s = split_exponent(__builtin_fmaxf(__builtin_fmaxf(part[0], part[1]), __builtin_fmaxf(part[2], part[3])));
        xexp[r] = ex_s;
    }
    __syncthreads();
    const int ne = -ex_s;
    for (int64_t g = tid; g < k / 16; g += 256) {
        const u32x4* src = (const u32x4*)(row + 16 * g);
        uint32_t v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 u = src[q];
            v[4 * q] = u.x, v[4 * q + 1] = u.y, v[4 * q + 2] = u.z, v[4 * q + 3] = u.w;
        }
        uint32_t hw[8], lw[8];
        split16(v, ne, hw, lw);
        u32x4* dst = (u32x4*)(out + 64 * (r * (k / 16) + g));
        dst[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
        dst[1] = u32x4{hw[4], hw[5], hw[6], hw[7]};
        dst[2] = u32x4{lw[0], lw[1], lw[2], lw[3]};
        dst[3] = u32x4{lw[4], lw[5], lw[6], lw[7]};
    }
}

hipError_t launch_split_rows(const float* x, int64_t rows, int64_t k, uint8_t* out, int32_t* xexp, hipStream_t s) {
    hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)rows), dim3(256), 0, s, x, k, out, xexp);
    return hipGetLastError();
}

// The down projection with each chunk's activations staged beside its
// weights (no staging of all slots up front): fp16 activations (PRE false)
// or fp32 rows split by split_rows_kernel (PRE true: 64-byte groups of 16 hi
// and 16 lo halves, the row's exponent in d.xexp).
template <int C, int W, int CU, int R, bool PRE, int PB = 16>
__global__ __launch_bounds__(64 * W) void cdown1s_kernel(DownMixArgs d) {
    using Cfg = CmvCfg<C, W, CU, R, PB>;
    constexpr int kRowPieces = Cfg::ROW_PIECES, kWBuf = Cfg::WBUF, kNBuf = 2, kRG = Cfg::RG;
    constexpr int NPIECE = 16 * kRowPieces, WLOADS = (NPIECE + 63) / 64, WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int ESZ = PRE ? 4 : 2;                  // staged bytes per activation
    constexpr int XB = Cfg::CHQ * 32 * ESZ;           // activation bytes of one chunk
    constexpr int XL = XB / 1024;                     // 1 KB copies of them
    constexpr int BUF = kWBuf + XB;
    static_assert(XB % 1024 == 0, "a chunk's activations are whole 1 KB copies");
    extern __shared__ __align__(16) uint8_t smem[];
    float* red = (float*)(smem + kNBuf * BUF);        // [W][16]
    const int S = (int)d.top_k;
    const int64_t n = d.n, k = d.k, n0 = (int64_t)blockIdx.x * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // a token with an invalid expert id has NaN outputs
    bool bad = false;
    for (int r = 0; r < S; ++r)
        bad |= (int64_t)slot_expert(d.ids, r, S, d.shexp, d.n_experts) >= d.n_experts + d.shexp;
    if (bad) {
        if (tid < 16 && n0 + tid < n) put_dt(d.y, n0 + tid, d.y_dt, __builtin_nanf(""));
        return;
    }
    const int64_t row_bytes = d.row_bytes;
    const int cps = (int)(row_bytes / Cfg::CHB);  // chunks per slot
    const int nchunks = S * cps;
    const uint8_t* xsrc = (const uint8_t*)d.x;

    uint32_t woff[WL_PER_WAVE];
    bool wact[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int r = p / kRowPieces, q = p - r * kRowPieces;
        int64_t nr = n0 + r;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < 16 && q < Cfg::CHB / PB;
        woff[j] = (uint32_t)((nr - n0) * row_bytes) + (uint32_t)PB * (uint32_t)q;
    }
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    wave_loads += XL > wave ? (XL - wave + W - 1) / W : 0;
    auto issue = [&](int chunk) {
        uint8_t* dst = smem + (chunk % kNBuf) * BUF;
        const int r = chunk / cps, lc = chunk - r * cps;
        const uint8_t* src = expert_base(d.w, d.w_sh, slot_expert(d.ids, r, S, d.shexp, d.n_experts), d.n_experts,
                                         d.expert_stride) +
                             n0 * row_bytes + (int64_t)lc * Cfg::CHB;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_addr(dst + 64 * PB * i));
                if (wact[j]) dma_piece<PB>(src + woff[j], dl);
            }
        }
        const int64_t xr = d.slotted ? r : 0;
        const uint8_t* xs = xsrc + (xr * k + (int64_t)lc * (Cfg::CHQ * 32)) * ESZ;
        for (int i = wave; i < XL; i += W)
            dma16(xs + 1024 * i + 16 * lane, __builtin_amdgcn_readfirstlane(lds_addr(dst + kWBuf + 1024 * i)));
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    const int rg = lane % kRG;
    for (int c = 0; c < kNBuf - 1 && c < nchunks; ++c) issue(c);
    for (int c = 0; c < nchunks; ++c) {
        const int later = (nchunks - 1 < c + kNBuf - 2 ? nchunks - 1 : c + kNBuf - 2) - c;
        wait_loads_le(later * wave_loads);
        __syncthreads();
        if (c + kNBuf - 1 < nchunks) issue(c + kNBuf - 1);
        const uint8_t* B = smem + (c % kNBuf) * BUF;
        const uint8_t* X = B + kWBuf;
        const int r = c / cps;
        const float sc = d.scores[r];
        const int ex = PRE ? d.xexp[d.slotted ? r : 0] : 0;
        for (int t = lane + 64 * wave; t < Cfg::TASKS; t += 64 * W) {
            const int cq = t / kRG;
            uint32_t p[R][16];
            float A[R][2], Bv[R][2];
            int64_t xa = 0, xb = 0;
#pragma unroll
            for (int j = 0; j < R; ++j)
                Pair32<C>::template decode<true>(B + (rg + kRG * j) * Cfg::ROW_BYTES, cq, p[j], A[j], Bv[j],
                                                 xa, xb);
            if constexpr (!PRE) {
                uint32_t xw[16];
                const u32x4* xp = (const u32x4*)(X + 2 * xa);
                const u32x4* xq = (const u32x4*)(X + 2 * xb);
                const u32x4 x0 = xp[0], x1 = xp[1], x2 = xq[0], x3 = xq[1];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xw[q] = x0[q], xw[4 + q] = x1[q], xw[8 + q] = x2[q], xw[12 + q] = x3[q];
                float t0 = 0.f, t1 = 0.f;
                if (Pair32<C>::has_b) {
                    t0 = sum16(xw);
                    t1 = sum16(xw + 8);
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float sj = A[j][0] * dot16(p[j], xw);
                    sj = __builtin_fmaf(A[j][1], dot16(p[j] + 8, xw + 8), sj);
                    if (Pair32<C>::has_b) {
                        sj = __builtin_fmaf(Bv[j][0], t0, sj);
                        sj = __builtin_fmaf(Bv[j][1], t1, sj);
                    }
                    acc[j] = __builtin_fmaf(sc, sj, acc[j]);
                }
            } else {
                const u32x4* ga = (const u32x4*)(X + 4 * xa);
                const u32x4* gb = (const u32x4*)(X + 4 * xb);
                uint32_t ha[8], la[8], hb[8], lb[8];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const u32x4 u0 = ga[q], u1 = ga[2 + q], u2 = gb[q], u3 = gb[2 + q];
#pragma unroll
                    for (int z = 0; z < 4; ++z)
                        ha[4 * q + z] = u0[z], la[4 * q + z] = u1[z], hb[4 * q + z] = u2[z], lb[4 * q + z] = u3[z];
                }
                float t0 = 0.f, t1 = 0.f;
                if (Pair32<C>::has_b) {
                    t0 = sum16(ha) + sum16(la);
                    t1 = sum16(hb) + sum16(lb);
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float sj = A[j][0] * (dot16(p[j], ha) + dot16(p[j], la));
                    sj = __builtin_fmaf(A[j][1], dot16(p[j] + 8, hb) + dot16(p[j] + 8, lb), sj);
                    if (Pair32<C>::has_b) {
                        sj = __builtin_fmaf(Bv[j][0], t0, sj);
                        sj = __builtin_fmaf(Bv[j][1], t1, sj);
                    }
                    acc[j] += __builtin_ldexpf(sc * sj, ex);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int o = kRG; o < 64; o <<= 1)
            acc[j] += __shfl_xor(acc[j], o, 64);
    }
    if (lane < kRG) {
#pragma unroll
        for (int j = 0; j < R; ++j) red[wave * 16 + rg + kRG * j] = acc[j];
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float v = 0.f;
        for (int ww = 0; ww < W; ++ww) v += red[ww * 16 + lane];
        if (n0 + lane < n) put_dt(d.y, n0 + lane, d.y_dt, v);
    }
}

// Launch shapes of the single-token forms (the down projection's own table
// is the same: smaller chunks, which would let two of its workgroups share a
// compute unit, measured slower).
template <int C> struct RoutedPick { static constexpr int W = 8, CU = 4; };
template <> struct RoutedPick<Q2_K> { static constexpr int W = 8, CU = 1; };
template <> struct RoutedPick<Q6_K> { static constexpr int W = 8, CU = 1; };
template <> struct RoutedPick<Q3_K> { static constexpr int W = 8, CU = 1; };
template <int C> struct DownPick : RoutedPick<C> {};

// (Q6_K and Q3_K rows that are no whole number of 2048 weights: 4-byte
// copies, chunks of 1024 weights or 512, as in the one-row GEMV)
template <int C, int CU, int PB>
static size_t glu1_lds(int64_t k) {
    using Cfg = CmvCfg<C, RoutedPick<C>::W, CU, 2, PB>;
    return (size_t)2 * 2 * Cfg::WBUF + (size_t)k * 2 + (size_t)RoutedPick<C>::W * 2 * 16 * 4;
}
template <int C, int CU, int PB>
static size_t down1_lds(int64_t k, int64_t S, int mode) {
    using Cfg = CmvCfg<C, DownPick<C>::W, CU, 2, PB>;
    if (mode == 2) return (size_t)2 * Cfg::WBUF + (size_t)S * k * 4 + 16 * 4 + (size_t)DownPick<C>::W * 16 * 4;
    return (size_t)2 * (Cfg::WBUF + Cfg::CHQ * 32 * (mode == 1 ? 4 : 2)) + (size_t)DownPick<C>::W * 16 * 4;
}
// the routed forms' variant for k: 16 (the table's shape), 42 or 41 (4-byte
// copies, chunks of 2 or 1 units), 0 none
template <int C>
static int glu1_variant(int64_t k) {
    if (k <= 0) return 0;
    if (k % ((int64_t)RoutedPick<C>::CU * Unit<C>::W) == 0 && glu1_lds<C, RoutedPick<C>::CU, 16>(k) <= 160 * 1024)
        return 16;
    if constexpr (kDword<C>) {
        if (k % 1024 == 0 && glu1_lds<C, 2, 4>(k) <= 160 * 1024) return 42;
        if (k % 512 == 0 && glu1_lds<C, 1, 4>(k) <= 160 * 1024) return 41;
    }
    return 0;
}
template <int C>
static int down1_variant(int64_t k, int64_t S, int mode) {
    // (splitting inside the kernel: at most 16 slots, whose row exponents
    // take 16 words; that form has 16-byte copies only)
    if (k <= 0 || S < 1 || (mode == 2 && S > 16)) return 0;
    if (k % ((int64_t)DownPick<C>::CU * Unit<C>::W) == 0 && down1_lds<C, DownPick<C>::CU, 16>(k, S, mode) <= 160 * 1024)
        return 16;
    if constexpr (kDword<C>) {
        if (mode != 2 && k % 1024 == 0) return 42;
        if (mode != 2 && k % 512 == 0) return 41;
    }
    return 0;
}
template <int C>
static bool glu1_fits_c(int64_t k) { return glu1_variant<C>(k) != 0; }
template <int C>
static bool down1_fits_c(int64_t k, int64_t S, int mode) { return down1_variant<C>(k, S, mode) != 0; }
bool glu1_fits(int codec, int64_t k) {
    switch (codec) {
    case Q8_0: return glu1_fits_c<Q8_0>(k);
    case Q4_0: return glu1_fits_c<Q4_0>(k);
    case Q5_0: return glu1_fits_c<Q5_0>(k);
    case Q5_1: return glu1_fits_c<Q5_1>(k);
    case Q6_K: return glu1_fits_c<Q6_K>(k);
    case Q2_K: return glu1_fits_c<Q2_K>(k);
    case Q3_K: return glu1_fits_c<Q3_K>(k);
    case Q5_K: return glu1_fits_c<Q5_K>(k);
    default: return false;
    }
}
bool down1_fits(int codec, int64_t k, int64_t S, int mode) {
    switch (codec) {
    case Q8_0: return down1_fits_c<Q8_0>(k, S, mode);
    case Q4_0: return down1_fits_c<Q4_0>(k, S, mode);
    case Q5_0: return down1_fits_c<Q5_0>(k, S, mode);
    case Q5_1: return down1_fits_c<Q5_1>(k, S, mode);
    case Q6_K: return down1_fits_c<Q6_K>(k, S, mode);
    case Q2_K: return down1_fits_c<Q2_K>(k, S, mode);
    case Q3_K: return down1_fits_c<Q3_K>(k, S, mode);
    case Q5_K: return down1_fits_c<Q5_K>(k, S, mode);
    default: return false;
    }
}

template <int C, int CU, int PB>
static hipError_t glu1_go(const SkinnyArgs& a, hipStream_t s) {
    constexpr int W = RoutedPick<C>::W;
    hipLaunchKernelGGL((cglu1_kernel<C, W, CU, PB>), dim3((unsigned)((a.n + 15) / 16), (unsigned)a.top_k),
                       dim3(64 * W), (glu1_lds<C, CU, PB>(a.k)), s, a);
    return hipGetLastError();
}
template <int C>
static hipError_t glu1_c(const SkinnyArgs& a, hipStream_t s) {
    const int v = glu1_variant<C>(a.k);
    if constexpr (kDword<C>) {
        if (v == 42) return glu1_go<C, 2, 4>(a, s);
        if (v == 41) return glu1_go<C, 1, 4>(a, s);
    }
    return glu1_go<C, RoutedPick<C>::CU, 16>(a, s);
}
template <int C, int CU, int PB>
static hipError_t down1_go(const DownMixArgs& d, int mode, hipStream_t s) {
    constexpr int W = DownPick<C>::W;
    const dim3 grid((unsigned)((d.n + 15) / 16));
    const size_t lds = down1_lds<C, CU, PB>(d.k, d.top_k, mode);
    if constexpr (PB == 16) {
        if (mode == 2) {
            hipLaunchKernelGGL((cdown1_kernel<C, W, CU, 2, true>), grid, dim3(64 * W), lds, s, d);
            return hipGetLastError();
        }
    }
    if (mode == 1) hipLaunchKernelGGL((cdown1s_kernel<C, W, CU, 2, true, PB>), grid, dim3(64 * W), lds, s, d);
    else hipLaunchKernelGGL((cdown1s_kernel<C, W, CU, 2, false, PB>), grid, dim3(64 * W), lds, s, d);
    return hipGetLastError();
}
template <int C>
static hipError_t down1_c(const DownMixArgs& d, int mode, hipStream_t s) {
    const int v = down1_variant<C>(d.k, d.top_k, mode);
    if constexpr (kDword<C>) {
        if (v == 42) return down1_go<C, 2, 4>(d, mode, s);
        if (v == 41) return down1_go<C, 1, 4>(d, mode, s);
    }
    return down1_go<C, DownPick<C>::CU, 16>(d, mode, s);
}

hipError_t launch_glu1_gguf(int codec, const SkinnyArgs& a, hipStream_t s) {
    switch (codec) {
    case Q8_0: return glu1_c<Q8_0>(a, s);
    case Q4_0: return glu1_c<Q4_0>(a, s);
    case Q5_0: return glu1_c<Q5_0>(a, s);
    case Q5_1: return glu1_c<Q5_1>(a, s);
    case Q6_K: return glu1_c<Q6_K>(a, s);
    case Q2_K: return glu1_c<Q2_K>(a, s);
    case Q3_K: return glu1_c<Q3_K>(a, s);
    default: return glu1_c<Q5_K>(a, s);
    }
}
hipError_t launch_down1_gguf(int codec, const DownMixArgs& d, int mode, hipStream_t s) {
    switch (codec) {
    case Q8_0: return down1_c<Q8_0>(d, mode, s);
    case Q4_0: return down1_c<Q4_0>(d, mode, s);
    case Q5_0: return down1_c<Q5_0>(d, mode, s);
    case Q5_1: return down1_c<Q5_1>(d, mode, s);
    case Q6_K: return down1_c<Q6_K>(d, mode, s);
    case Q2_K: return down1_c<Q2_K>(d, mode, s);
    case Q3_K: return down1_c<Q3_K>(d, mode, s);
    default: return down1_c<Q5_K>(d, mode, s);
    }
}

// ---------------------------------------------------------------- routed tiles
// The expert-routed products over the schedule's tiles (one expert, up to 32
// rows gathered through the permutation): kq_qmm_id and the gate/up form of
// kq_moe_glu, for Q8_0 and the further GGUF codecs, as the batched decode
// kernel above computes them.  A workgroup of eight waves takes one tile and
// NT tiles of 16 weight rows (16 gate and 16 up rows each for the GLU), as
// many as LDS holds: the tile's activation rows, staged once per chunk of K
// beside the weights, feed all of them.  8 / NT waves share a row tile and
// split each chunk's 32-weight groups, their sums combined through LDS.  K is walked in chunks of 512 weights (256 for fp32
// activations where a codec's copy unit allows; 16-byte copies, or 4-byte
// ones for Q2_K, Q6_K and Q3_K).  Each 32-weight chunk of a weight row is
// decoded once and feeds the two 16-row MFMA groups of the tile: folded into
// fp16 weights for the 32-weight blocks with fp16 activations (exact form for
// a wave holding a block that could overflow fp16), exact integers with the
// scales applied in fp32 otherwise (the K-quants, and fp32 activations, held
// to tau = 1e-5).  fp32 activations: each row scaled by its power of two
// (row_exp_kernel) and split per chunk into fp16 hi + lo halves, both through
// the matrix cores, the result scaled back.
template <int C> constexpr int kCrmPB = (C == Q6_K || C == Q3_K || C == Q2_K) ? 4 : 16;
template <int C, int NT, bool GLU, bool XF32>
struct CrmCfg {
    static constexpr int PB = kCrmPB<C>;
    using U = UnitP<C, PB>;
    static constexpr int CHW = (XF32 && U::W <= 256) ? 256 : 512;
    static constexpr int CU = CHW / U::W, CHB = CU * U::BYTES, CHQ = CHW / 32;
    static constexpr int NM = GLU ? 2 : 1;
    static constexpr int ROW_PIECES = (CHB / PB + 1) | 1, ROW_BYTES = ROW_PIECES * PB;
    static constexpr int WROWS = 16 * NT * NM;                 // weight rows per workgroup
    static constexpr int WBUF = (WROWS * ROW_BYTES + 15) / 16 * 16;
    static constexpr int ESZ = XF32 ? 4 : 2;
    static constexpr int XSTRIDE = CHW * ESZ + 16;              // bytes per staged activation row
    static constexpr int XL_ROW = CHW * ESZ / 1024;             // 1 KB copies per row and chunk
    static constexpr int BUF = WBUF + 32 * XSTRIDE;
    static constexpr size_t LDS = 2 * (size_t)BUF > (size_t)8 * NM * 2 * 1024 ? 2 * (size_t)BUF : (size_t)8 * NM * 2 * 1024;
    static_assert(CHW % U::W == 0 && U::BYTES % PB == 0 && XL_ROW >= 1, "whole units and copies per chunk");
};
// the widest workgroup whose buffers fit in LDS
template <int C, bool GLU, bool XF32>
constexpr int crm_nt() {
    return CrmCfg<C, 8, GLU, XF32>::LDS <= 160 * 1024   ? 8
           : CrmCfg<C, 4, GLU, XF32>::LDS <= 160 * 1024 ? 4
           : CrmCfg<C, 2, GLU, XF32>::LDS <= 160 * 1024 ? 2
                                                        : 1;
}

template <int C, int NT, bool GLU, bool XF32>
__global__ __launch_bounds__(512) void crm_kernel(SkinnyArgs a) {
    using Cfg = CrmCfg<C, NT, GLU, XF32>;
    constexpr int W = 8, KS = W / NT;  // waves; waves per row tile
    constexpr int PB = Cfg::PB, NM = Cfg::NM, CHB = Cfg::CHB, CHQ = Cfg::CHQ, CHW = Cfg::CHW;
    constexpr int ROW_PIECES = Cfg::ROW_PIECES, ROW_BYTES = Cfg::ROW_BYTES, BUF = Cfg::BUF;
    constexpr int NPIECE = Cfg::WROWS * ROW_PIECES, WLOADS = (NPIECE + 63) / 64, WL_PER_WAVE = (WLOADS + W - 1) / W;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n = a.n, k = a.k, nb = (int64_t)blockIdx.x * (16 * NT);
    if ((int64_t)blockIdx.y >= (int64_t)a.ws[0]) return;
    const int32_t* tile = a.ws + a.tiles_off + 3 * (int64_t)blockIdx.y;
    const int64_t e = tile[0], row0 = tile[1];
    const int nrows = tile[2];
    const int32_t* perm = a.ws + a.perm_off;
    const int32_t* xexp = a.ws + a.xexp_off;
    const int64_t row_bytes = a.row_bytes;
    const int nchunks = (int)(k / CHW);
    const uint8_t* wb0 = expert_base(a.w, a.w_sh, e, a.n_experts, a.expert_stride) + nb * row_bytes;
    const uint8_t* wb1 = GLU ? expert_base(a.w2, a.w2_sh, e, a.n_experts, a.expert_stride) + nb * row_bytes : wb0;
    // the activation row of tile row r (rows past the tile read row 0 and are not stored)
    auto xrow_of = [&](int r) -> int64_t {
        const int64_t R = perm[row0 + (r < nrows ? r : 0)];
        return a.shared_x ? R / a.top_k : R;
    };

    // LDS row q of a chunk buffer: matrix q / (16 NT), weight row nb + q % (16 NT)
    uint32_t woff[WL_PER_WAVE];
    bool wact[WL_PER_WAVE], wsec[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int r = p / ROW_PIECES, q = p - r * ROW_PIECES;
        const int rr = r % (16 * NT);
        int64_t nr = nb + rr;
        if (nr >= n) nr = n - 1;
        wact[j] = i < WLOADS && r < Cfg::WROWS && q < CHB / PB;
        wsec[j] = r >= 16 * NT;
        woff[j] = (uint32_t)((nr - nb) * row_bytes) + (uint32_t)PB * (uint32_t)q;
    }
    const int xl_total = nrows * Cfg::XL_ROW;
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    wave_loads += xl_total > wave ? (xl_total - wave + W - 1) / W : 0;
    const uint8_t* xsrc = (const uint8_t*)a.x;
    auto issue = [&](int chunk) {
        uint8_t* dst = smem + (chunk & 1) * BUF;
        const int64_t cb = (int64_t)chunk * CHB;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_addr(dst + 64 * PB * i));
                if (wact[j]) dma_piece<PB>((wsec[j] ? wb1 : wb0) + cb + woff[j], dl);
            }
        }
        for (int i = wave; i < xl_total; i += W) {
            const int r = i / Cfg::XL_ROW, c = i - r * Cfg::XL_ROW;
            const uint8_t* src = xsrc + (xrow_of(r) * k + (int64_t)chunk * CHW) * Cfg::ESZ + 1024 * c;
            dma16(src + 16 * lane,
                  __builtin_amdgcn_readfirstlane(lds_addr(dst + Cfg::WBUF + r * Cfg::XSTRIDE + 1024 * c)));
        }
    };

    float4_t acc[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m][0] = acc[m][1] = float4_t{0.f, 0.f, 0.f, 0.f};
    const u32x2 ones = u32x2{0x3c003c00u, 0x3c003c00u};
    const float4_t z = {0.f, 0.f, 0.f, 0.f};
    issue(0);
    for (int c = 0; c < nchunks; ++c) {
        wait_loads_le(0);
        __syncthreads();  // chunk c has landed everywhere; every wave is done with chunk c - 1
        if (c + 1 < nchunks) issue(c + 1);
        const uint8_t* B = smem + (c & 1) * BUF;
        uint8_t* X = smem + (c & 1) * BUF + Cfg::WBUF;
        if constexpr (XF32) {
            // each row's values times 2^-e, split in place: every 16 values
            // (64 bytes) become 16 hi halves then 16 lo halves
            for (int gi = tid; gi < nrows * (CHW / 16); gi += 64 * W) {
                const int r = gi / (CHW / 16), grp = gi - r * (CHW / 16);
                const int ne = -xexp[xrow_of(r)];
                u32x4* g4 = (u32x4*)(X + r * Cfg::XSTRIDE + 64 * grp);
                uint32_t v[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 u = g4[q];
                    v[4 * q] = u.x, v[4 * q + 1] = u.y, v[4 * q + 2] = u.z, v[4 * q + 3] = u.w;
                }
                uint32_t hw[8], lw[8];
                split16(v, ne, hw, lw);
                g4[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                g4[1] = u32x4{hw[4], hw[5], hw[6], hw[7]};
                g4[2] = u32x4{lw[0], lw[1], lw[2], lw[3]};
                g4[3] = u32x4{lw[4], lw[5], lw[6], lw[7]};
            }
            __syncthreads();
        }
        // this wave's weight rows: row tile wave % NT of each matrix, and its
        // share wave / NT of the chunk's 32-weight groups
        const int rt = wave % NT;
        const uint8_t* wrow0 = B + (rt * 16 + n_l) * ROW_BYTES;
        const uint8_t* wrow1 = B + ((NT + rt) * 16 + n_l) * ROW_BYTES;
        for (int cq = wave / NT; cq < CHQ; cq += KS) {
            // activation operands of the two row groups: [group][half][hi, lo]
            u32x2 av[2][2][2];
#pragma unroll
            for (int G = 0; G < 2; ++G) {
                const uint8_t* xr = X + (16 * G + n_l) * Cfg::XSTRIDE;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if constexpr (XF32) {
                        const uint8_t* gp = xr + 4 * (32 * cq + 16 * h);
                        av[G][h][0] = *(const u32x2*)(gp + 8 * g);
                        av[G][h][1] = *(const u32x2*)(gp + 32 + 8 * g);
                    } else {
                        av[G][h][0] = *(const u32x2*)(xr + 2 * (32 * cq + 16 * h + 4 * g));
                    }
                }
            }
            bool folded = false;
            // (fp32 activations are held to tau = 1e-5: exact weights only)
            if constexpr (Pair8<C>::foldable && PB == 16 && !XF32) {
                u32x2 wv[NM][2];
                bool ok = Pair8<C>::fold(wrow0, cq, g, wv[0][0], wv[0][1]);
                if constexpr (GLU) ok &= Pair8<C>::fold(wrow1, cq, g, wv[NM - 1][0], wv[NM - 1][1]);
                if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
                    folded = true;
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int G = 0; G < 2; ++G)
#pragma unroll
                            for (int h = 0; h < 2; ++h) acc[m][G] = mfma4(av[G][h][0], wv[m][h], acc[m][G]);
                }
            }
            if (!folded) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    u32x2 b[2];
                    float A[2], Bv[2];
                    Pair8<C>::decode(m ? wrow1 : wrow0, cq, g, b[0], b[1], A, Bv);
#pragma unroll
                    for (int G = 0; G < 2; ++G) {
                        float4_t ch[2], sh[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            ch[h] = mfma4(av[G][h][0], b[h], z);
                            if constexpr (XF32) ch[h] = mfma4(av[G][h][1], b[h], ch[h]);
                            if constexpr (Pair8<C>::has_b) {
                                sh[h] = mfma4(av[G][h][0], ones, z);
                                if constexpr (XF32) sh[h] = mfma4(av[G][h][1], ones, sh[h]);
                            }
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            float t = __builtin_fmaf(A[0], ch[0][v], __builtin_fmaf(A[1], ch[1][v], acc[m][G][v]));
                            if constexpr (Pair8<C>::has_b)
                                t = __builtin_fmaf(Bv[0], sh[0][v], __builtin_fmaf(Bv[1], sh[1][v], t));
                            acc[m][G][v] = t;
                        }
                    }
                }
            }
        }
    }
    if constexpr (KS > 1) {
        __syncthreads();  // every wave is done with the last chunk and no copy is in flight
        float4_t* red = (float4_t*)smem;  // [KS][NT][NM][2][64]
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int G = 0; G < 2; ++G) red[((wave * NM + m) * 2 + G) * 64 + lane] = acc[m][G];
        __syncthreads();
        if (wave >= NT) return;
        for (int ks = 1; ks < KS; ++ks)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int G = 0; G < 2; ++G) {
                    const float4_t t = red[(((ks * NT + wave) * NM + m) * 2 + G) * 64 + lane];
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[m][G][v] += t[v];
                }
    }
    // lane holds tile rows 16 G + 4 g + v of weight row nb + 16 wave + n_l
    const int64_t col = nb + 16 * wave + n_l;
    if (col >= n) return;
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * G + 4 * g + v;
            if (r >= nrows) continue;
            const int64_t R = perm[row0 + r];
            float gv = acc[0][G][v], uv = acc[NM - 1][G][v];
            if constexpr (XF32) {
                const int ex = xexp[a.shared_x ? R / a.top_k : R];
                gv = __builtin_ldexpf(gv, ex);
                uv = __builtin_ldexpf(uv, ex);
            }
            put_dt(a.y, R * a.y_row + col, a.y_dt, GLU ? glu_act(a.act, gv, uv, a.limit) : gv);
        }
}

template <int C, bool GLU, bool XF32>
static bool crm_fits_g(int64_t k) {
    using Cfg = CrmCfg<C, crm_nt<C, GLU, XF32>(), GLU, XF32>;
    return k > 0 && k % Cfg::CHW == 0 && Cfg::LDS <= 160 * 1024;
}
template <int C>
static bool crm_fits_c(int64_t k, bool glu, bool xf32) {
    if (glu) return xf32 ? crm_fits_g<C, true, true>(k) : crm_fits_g<C, true, false>(k);
    return xf32 ? crm_fits_g<C, false, true>(k) : crm_fits_g<C, false, false>(k);
}
bool crm_fits(int codec, int64_t k, bool glu, bool xf32) {
    switch (codec) {
    case Q8_0: return crm_fits_c<Q8_0>(k, glu, xf32);
    case Q4_0: return crm_fits_c<Q4_0>(k, glu, xf32);
    case Q5_0: return crm_fits_c<Q5_0>(k, glu, xf32);
    case Q5_1: return crm_fits_c<Q5_1>(k, glu, xf32);
    case Q6_K: return crm_fits_c<Q6_K>(k, glu, xf32);
    case Q2_K: return crm_fits_c<Q2_K>(k, glu, xf32);
    case Q3_K: return crm_fits_c<Q3_K>(k, glu, xf32);
    case Q5_K: return crm_fits_c<Q5_K>(k, glu, xf32);
    default: return false;
    }
}
template <int C, bool GLU, bool XF32>
static hipError_t crm_go(const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s) {
    constexpr int NT = crm_nt<C, GLU, XF32>();
    hipLaunchKernelGGL((crm_kernel<C, NT, GLU, XF32>),
                       dim3((unsigned)((a.n + 16 * NT - 1) / (16 * NT)), (unsigned)grid_tiles), dim3(512),
                       (CrmCfg<C, NT, GLU, XF32>::LDS), s, a);
    return hipGetLastError();
}
template <int C>
static hipError_t crm_c(bool glu, bool xf32, const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s) {
    if (glu) return xf32 ? crm_go<C, true, true>(a, grid_tiles, s) : crm_go<C, true, false>(a, grid_tiles, s);
    return xf32 ? crm_go<C, false, true>(a, grid_tiles, s) : crm_go<C, false, false>(a, grid_tiles, s);
}
hipError_t launch_crm(int codec, bool glu, bool xf32, const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s) {
    switch (codec) {
    case Q8_0: return crm_c<Q8_0>(glu, xf32, a, grid_tiles, s);
    case Q4_0: return crm_c<Q4_0>(glu, xf32, a, grid_tiles, s);
    case Q5_0: return crm_c<Q5_0>(glu, xf32, a, grid_tiles, s);
    case Q5_1: return crm_c<Q5_1>(glu, xf32, a, grid_tiles, s);
    case Q6_K: return crm_c<Q6_K>(glu, xf32, a, grid_tiles, s);
    case Q2_K: return crm_c<Q2_K>(glu, xf32, a, grid_tiles, s);
    case Q3_K: return crm_c<Q3_K>(glu, xf32, a, grid_tiles, s);
    default: return crm_c<Q5_K>(glu, xf32, a, grid_tiles, s);
    }
}

}  // namespace kq
