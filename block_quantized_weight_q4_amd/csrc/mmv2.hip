// mmv2.hip -- decode-shaped Q4_K products on the matrix cores with fp16
// activations: kq_qmv and kq_qmm with 5 to 16 rows (fewer rows take the
// unscaled-nibble kernels of mmv3.hip), and the expert-routed forms when
// every schedule tile holds at most 16 rows (decode batches): kq_qmm_id and
// the fused gate/up SiLU of kq_moe_glu.
//
// mlx-kquant "bindings.cpp": quantized_matmul, gather_qmv_kq,
// moe_glu_gather_kq; mlx-native "quantized_matmul_id_ggml.rs": the
// expert-routed matvec.
//
// A workgroup owns 16 consecutive weight rows (of one or two matrices) for
// all of K.  Those rows are one contiguous stretch of memory, so K is walked
// in chunks of C super-blocks that the workgroup streams into LDS with
// global->LDS 16-byte loads, 64 consecutive pieces per instruction; the
// activation rows of the tile are staged the same way.  Chunks are double
// buffered: the loads of chunk j+1 are in flight while the waves multiply
// chunk j.  The multiply is the exact-operand scheme of q4k_mfma.h: sc*q as
// fp16 integers, the 6-bit min as a second MFMA chain, d and dmin applied
// once per super-block in fp32.
#include "kq_device.h"
#include "kq_internal.h"
#include "q4k_mfma.h"
#include "lds_dma.h"

namespace kq {

// NM sets of 16 weight rows: for the GLU the gate (set 0) and up (set 1)
// rows of one 16-row block, otherwise NM consecutive 16-row blocks.  C
// super-blocks per chunk, W waves, S chunk buffers in LDS (S-1 chunks in
// flight while one is multiplied).
template <int NM, bool GLU, int C, int W, int S>
__global__ __launch_bounds__(64 * W) void mmv2_q4k_f16_kernel(SkinnyArgs a) {
    static_assert(!GLU || NM == 2, "the GLU takes one gate and one up set");
    static_assert((NM * 16 * 9 * C) % 64 == 0, "a chunk of weights is whole 1 KB loads");
    constexpr int WPIECES = NM * 16 * 9 * C;   // 16-byte pieces of weights per chunk
    constexpr int WLOADS = WPIECES / 64;       // load instructions per chunk
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int XPIECES_ROW = 32 * C;        // pieces of one activation row per chunk
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (GLU ? 16 : 16 * NM);
    const int nsb = (int)(a.k / 256);
    const int nchunks = (nsb + C - 1) / C;

    // ---- rows of this tile
    int64_t expert = 0, row0, nrows;
    const int32_t* perm = nullptr;
    if (a.ws) {
        if ((int64_t)blockIdx.y >= (int64_t)a.ws[0]) return;
        const int32_t* tile = a.ws + a.tiles_off + 3 * (int64_t)blockIdx.y;
        expert = tile[0];
        row0 = tile[1];
        nrows = tile[2];
        perm = a.ws + a.perm_off;
    } else {
        row0 = (int64_t)blockIdx.y * 16;
        nrows = a.m - row0 < 16 ? a.m - row0 : 16;
    }

    // LDS: S buffers of [weights | activations]
    const int xstride = a.xstride;            // bytes between staged activation rows
    const int wbytes = WPIECES * 16;
    const int bufbytes = a.red_off / S;       // bytes of one buffer
    float* red = (float*)smem;                // over buffer 0, used after the last chunk

    // Per-lane byte offsets of this wave's weight pieces inside a chunk,
    // counted from the tile's first row (so they stay small for any matrix
    // size): piece p = 64*i + lane -> matrix m, row r, piece q of the row's chunk.
    const uint8_t* wbase[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
        wbase[m] = expert_base(GLU && m ? a.w2 : a.w, GLU && m ? a.w2_sh : a.w_sh, expert,
                               a.n_experts, a.expert_stride) + n0 * a.row_bytes;
    uint32_t woff[WL_PER_WAVE], wq16[WL_PER_WAVE];
    int wmat[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int i = wave + W * j;
        const int p = 64 * i + lane;
        const int m = p / (16 * 9 * C), rem = p - m * 16 * 9 * C;
        const int r = rem / (9 * C), q = rem - r * 9 * C;
        int64_t n = n0 + (GLU ? 0 : 16 * m) + r;
        if (n >= a.n) n = a.n - 1;
        wmat[j] = m < NM ? m : 0;
        wq16[j] = 16u * (uint32_t)q;
        woff[j] = (uint32_t)((n - n0) * a.row_bytes) + wq16[j];
    }
    // activation row pointers of the tile (scalar per row)
    auto xrow_ptr = [&](int r) -> const uint8_t* {
        int64_t xr = row0 + r;
        if (perm) xr = perm[xr];
        if (a.shared_x) xr /= a.top_k;  // routed row -> its token's activation row
        return (const uint8_t*)a.x + xr * a.x_row * 2;
    };

    // activation rows staged per chunk: one when every routed row belongs to
    // the same token (a single-token routing over shared activations)
    const int xrows = a.one_x_row ? 1 : (int)nrows;

    // load instructions this wave issues per chunk (the same for every chunk)
    int wave_loads = 0;
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) wave_loads += (wave + W * j < WLOADS) ? 1 : 0;
    {
        const int xl_total = xrows * (XPIECES_ROW / 64);
        wave_loads += xl_total > wave ? (xl_total - wave + W - 1) / W : 0;
    }

    auto issue = [&](int chunk, int dst_off) {
        uint8_t* dst = smem + dst_off;
        const int s0 = chunk * C;
        const int nsc = nsb - s0 < C ? nsb - s0 : C;   // super-blocks in this chunk
        const uint32_t cbase = (uint32_t)s0 * 144u;
        const uint32_t climit = (uint32_t)nsc * 144u;  // valid bytes per row
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                // pieces past the last super-block re-read a valid piece of
                // the row; they land in LDS but are never used
                const uint32_t off = wq16[j] < climit ? woff[j] : woff[j] - wq16[j];
                dma16(wbase[wmat[j]] + cbase + off,
                      __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i)));
            }
        }
        // activations: row r, pieces [0, 32*nsc); instruction k of a row
        // covers pieces [64k, 64k+64)
        const int xl_row = XPIECES_ROW / 64;
        const int xl_total = xrows * xl_row;
        for (int i = wave; i < xl_total; i += W) {
            const int r = i / xl_row, k = i - r * xl_row;
            int piece = 64 * k + lane;
            if (piece >= 32 * nsc) piece = 0;
            const uint8_t* src = xrow_ptr(r) + (size_t)s0 * 512 + 16 * piece;
            dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(dst + wbytes + r * xstride + 1024 * k)));
        }
    };

    float4_t acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = float4_t{0.f, 0.f, 0.f, 0.f};
    const LaneSel ls = lane_sel(g);
    uint32_t magic_v = 0x64006400u;
    asm volatile("" : "+v"(magic_v));
    // A-operand LDS offset of this lane: staged row b, or row 0 for a lane past
    // the tile (its MFMA output row is never stored)
    const int xlane = wbytes + (n_l < xrows ? n_l : 0) * xstride + 128 * g;

    // Order per chunk: wait for this wave's loads of chunk c (those of the
    // up to S-2 later chunks may stay in flight), barrier (all of chunk c has
    // landed and every wave is done with chunk c-1), then request chunk
    // c+S-1 into the buffer chunk c-1 used and multiply chunk c.
    for (int c = 0; c < S - 1 && c < nchunks; ++c) issue(c, c * bufbytes);
    for (int c = 0; c < nchunks; ++c) {
        const int later = nchunks - 1 - c < S - 2 ? nchunks - 1 - c : S - 2;
        wait_loads_le(wave_loads * later);
        __syncthreads();
        if (c + S - 1 < nchunks) issue(c + S - 1, ((c + S - 1) % S) * bufbytes);
        const uint8_t* B = smem + (c % S) * bufbytes;
        const int nsc = nsb - c * C < C ? nsb - c * C : C;
        for (int sb = wave; sb < nsc; sb += W) {
            u32x4 xa[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                xa[i] = *(const u32x4*)(B + xlane + sb * 512 + 64 * (i >> 2) + 16 * (i & 3));
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const uint8_t* wr = B + (m * 16 + n_l) * (9 * C * 16) + sb * 144;
                const u32x4 hd = *(const u32x4*)wr;
                const u32x4 q0 = *(const u32x4*)(wr + 16 + 32 * g);
                const u32x4 q1 = *(const u32x4*)(wr + 32 + 32 * g);
                Q4Operands op;
                q4k_operands(hd, q0, q1, ls, magic_v, op);
                float4_t c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    c1 = mfma16(xa[i], op.w[i], c1);
                    c2 = mfma16(xa[i], i < 4 ? op.m_lo : op.m_hi, c2);
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[m][v] += op.d * c1[v] - op.dmin * c2[v];
            }
        }
    }
    __syncthreads();

    // ---- combine the waves' partial sums
    if (W > 1) {
        if (wave > 0) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v) red[(((wave - 1) * NM + m) * 4 + v) * 64 + lane] = acc[m][v];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[m][v] += red[(((w - 1) * NM + m) * 4 + v) * 64 + lane];
    }

    // ---- store: lane holds activation rows b = 4g+v of weight row n_l of
    // each set
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t idx = 4 * g + v;
        if (idx >= nrows) continue;
        const int64_t orow = perm ? (int64_t)perm[row0 + idx] : row0 + idx;
        if (GLU) {
            const int64_t n = n0 + n_l;
            if (n < a.n) store_val(a.y, orow * a.y_row + n, a.y_dt, glu_act(a.act, acc[0][v], acc[1][v], a.limit));
        } else {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int64_t n = n0 + 16 * m + n_l;
                if (n < a.n) store_val(a.y, orow * a.y_row + n, a.y_dt, acc[m][v]);
            }
        }
    }
}

// The reduction area is only used after the last chunk's barrier, when every
// chunk buffer is idle and no copy is in flight, so it overlays buffer 0.
template <int NM, int C, int W, int S>
static constexpr size_t lds_cfg2(int64_t rows_max) {
    const int64_t wbytes = (int64_t)NM * 16 * 9 * C * 16;
    const int64_t bufbytes = (wbytes + rows_max * (512 * C + 16) + 15) / 16 * 16;
    const int64_t red = (int64_t)(W - 1) * NM * 4 * 64 * 4;
    return (size_t)(S * bufbytes > red ? S * bufbytes : red);
}

template <int NM, bool GLU, int C, int W, int S>
static void launch_cfg2(SkinnyArgs a, int64_t rows_max, int64_t tiles_y, hipStream_t s) {
    const int64_t wbytes = (int64_t)NM * 16 * 9 * C * 16;
    a.xstride = 512 * C + 16;                      // padded staged activation row
    const int64_t bufbytes = (wbytes + rows_max * a.xstride + 15) / 16 * 16;
    a.red_off = (int)(S * bufbytes);  // bytes of the chunk buffers
    const size_t lds = lds_cfg2<NM, C, W, S>(rows_max);
    const int64_t rows_wg = GLU ? 16 : 16 * NM;
    const dim3 grid((unsigned)((a.n + rows_wg - 1) / rows_wg), (unsigned)tiles_y);
    hipLaunchKernelGGL((mmv2_q4k_f16_kernel<NM, GLU, C, W, S>), grid, dim3(64 * W), lds, s, a);
}

// LDS per workgroup is at most 160 KB; the staged activation rows grow with
// the row count, so wide chunks are used only while they fit.  Measured on
// the decode shapes (batch 8): two buffers (one chunk in flight) beat deeper
// rings; sixteen waves on 8-block chunks for long rows, eight waves on
// 4-block chunks otherwise (the spare waves hide latency: only two to four
// workgroups fit per CU); pairs of 16-row tiles per workgroup were slower.
constexpr size_t kLdsMax = 160 * 1024;
static_assert(lds_cfg2<2, 2, 2, 2>(16) <= kLdsMax && lds_cfg2<1, 4, 8, 2>(16) <= kLdsMax,
              "the fallback shapes hold 16 staged activation rows");

hipError_t launch_mmv2_q4k(bool glu, const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s) {
    const int64_t rows_max = a.one_x_row ? 1 : a.ws ? (a.rows_cap < 16 ? a.rows_cap : 16) : a.m;
    const int64_t tiles = a.ws ? grid_tiles : (a.m + 15) / 16;
    const int64_t nsb = a.k / 256;
    if (glu) launch_cfg2<2, true, 2, 2, 2>(a, rows_max, tiles, s);
    else if (nsb > 16 && lds_cfg2<1, 8, 16, 2>(rows_max) <= kLdsMax)
        launch_cfg2<1, false, 8, 16, 2>(a, rows_max, tiles, s);
    else launch_cfg2<1, false, 4, 8, 2>(a, rows_max, tiles, s);
    return hipGetLastError();
}

}  // namespace kq
