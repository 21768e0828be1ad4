// mmv.hip -- weight-streaming Q4_K products on the matrix cores, fp16
// activations: the decode GEMV (kq_qmv), the expert-routed product
// (kq_qmm_id) and the fused gate/up SiLU GLU (kq_moe_glu).
//
// mlx-kquant "bindings.cpp": quantized_matmul, gather_qmm, moe_glu_gather_kq;
// mlx-native "quantized_matmul_id_ggml.rs": the expert-routed matvec and the
// grouped expert GEMM.
//
// Each wave multiplies 16 weight rows (per row tile) by up to 16 activation
// rows (per sub-tile) with the exact-operand scheme of q4k_mfma.h.
//
// Waves of a workgroup split the super-blocks of K (interleaved) and combine
// their partial sums through LDS at the end; there are no atomics, so results
// are deterministic.
#include "kq_device.h"
#include "kq_internal.h"
#include "q4k_mfma.h"

namespace kq {

// NT weight row tiles of 16 rows (for GLU: tile 0 = gate, tile 1 = up, same
// rows), MT activation sub-tiles of 16 rows, W waves splitting K.  The
// activations of the tile's rows are staged in LDS a.xch super-blocks at a
// time (row stride a.xstride halves, padded so the rows read by one MFMA
// operand fall in different banks); dynamic LDS holds them and, after them,
// the cross-wave reduction buffer.
template <int NT, int MT, int W, bool GLU>
__global__ __launch_bounds__(64 * W) void mmv_q4k_f16_kernel(SkinnyArgs a) {
    constexpr int NTILE = GLU ? 1 : NT;   // distinct 16-row groups of output
    extern __shared__ __align__(16) uint8_t smem[];
    uint16_t* xs = (uint16_t*)smem;
    float* red = (float*)(smem + a.red_off);
    const int XCH = a.xch, XSTRIDE = a.xstride;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NTILE;
    const int64_t nsb = a.k / 256;

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
        row0 = (int64_t)blockIdx.y * 16 * MT;
        nrows = a.m - row0 < 16 * MT ? a.m - row0 : 16 * MT;
    }
    const int subtiles = (int)((nrows + 15) / 16);

    // weight row pointers of this lane (B operand: row n = n_l)
    const uint8_t* wrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const uint8_t* base = (GLU && t == 1) ? a.w2 : a.w;
        int64_t n = n0 + (GLU ? 0 : 16 * t) + n_l;
        if (n >= a.n) n = a.n - 1;
        wrow[t] = base + expert * a.expert_stride + n * a.row_bytes;
    }

    float4_t acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = float4_t{0.f, 0.f, 0.f, 0.f};

    const LaneSel ls = lane_sel(g);
    uint32_t magic_v = 0x64006400u;
    asm volatile("" : "+v"(magic_v));  // keep the magic constant in a VGPR

    // A-operand LDS row of this lane per sub-tile: staged row b, or row 0 for
    // a lane past the tile (its MFMA output row is never stored)
    int xoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int b = 16 * mt + n_l;
        xoff[mt] = (b < nrows ? b : 0) * XSTRIDE + 64 * g;
    }

    // Weights of one super-block for every row tile; register double buffer
    // so each wait is for data requested an iteration earlier.
    u32x4 hd[NT], q0[NT], q1[NT];
    auto load_w = [&](int sb, u32x4 (&h)[NT], u32x4 (&w0)[NT], u32x4 (&w1)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint8_t* p = wrow[t] + (uint32_t)sb * 144u;
            h[t] = *(const u32x4*)p;
            w0[t] = *(const u32x4*)(p + 16 + 32 * g);
            w1[t] = *(const u32x4*)(p + 32 + 32 * g);
        }
    };
    const int nsb32 = (int)nsb;
    int s = wave;
    if (s < nsb32) load_w(s, hd, q0, q1);

    for (int c0 = 0; c0 < nsb32; c0 += XCH) {
        const int nch = nsb32 - c0 < XCH ? nsb32 - c0 : XCH;
        // ---- stage the activations of super-blocks [c0, c0+nch): for each
        // tile row, consecutive threads copy consecutive 16-byte pieces
        __syncthreads();
        {
            const int per_row = nch * 32;  // 16-byte pieces per staged row
            for (int r = 0; r < (int)nrows; ++r) {
                int64_t xr = row0 + r;
                if (perm) {
                    xr = perm[xr];
                    if (a.shared_x) xr /= a.top_k;
                }
                const u32x4* src = (const u32x4*)((const uint16_t*)a.x + xr * a.x_row + c0 * 256);
                u32x4* dst = (u32x4*)&xs[r * XSTRIDE];
                for (int q = tid; q < per_row; q += 64 * W) dst[q] = src[q];
            }
        }
        __syncthreads();

        for (; s < c0 + nch; s += W) {
            u32x4 nhd[NT], nq0[NT], nq1[NT];
            const bool more = s + W < nsb32;
            load_w(more ? s + W : s, nhd, nq0, nq1);
            Q4Operands op[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) q4k_operands(hd[t], q0[t], q1[t], ls, magic_v, op[t]);
            const int sl = (s - c0) * 256;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < subtiles) {
                    u32x4 xa[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        xa[i] = *(const u32x4*)&xs[xoff[mt] + sl + 32 * (i >> 2) + 8 * (i & 3)];
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        float4_t c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            c1 = mfma16(xa[i], op[t].w[i], c1);
                            c2 = mfma16(xa[i], i < 4 ? op[t].m_lo : op[t].m_hi, c2);
                        }
                        // lane holds rows b = 4g+v of weight row n_l: d, dmin of n_l
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[t][mt][v] += op[t].d * c1[v] - op[t].dmin * c2[v];
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) hd[t] = nhd[t], q0[t] = nq0[t], q1[t] = nq1[t];
        }
    }

    // ---- combine the waves' partial sums
    if (W > 1) {
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[(((wave - 1) * NT + t) * MT * 4 + mt * 4 + v) * 64 + lane] = acc[t][mt][v];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[t][mt][v] += red[(((w - 1) * NT + t) * MT * 4 + mt * 4 + v) * 64 + lane];
    }

    // ---- store: lane holds activation rows b = 4g+v, weight row n_l
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t idx = 16 * mt + 4 * g + v;
            if (idx >= nrows) continue;
            const int64_t orow = perm ? (int64_t)perm[row0 + idx] : row0 + idx;
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
                const int64_t n = n0 + 16 * t + n_l;
                if (n >= a.n) continue;
                const float val = GLU ? silu_fast(acc[0][mt][v]) * acc[1][mt][v] : acc[t][mt][v];
                store_val(a.y, orow * a.y_row + n, a.y_dt, val);
            }
        }
    }
}

template <int NT, int MT, int W, bool GLU>
static void launch_cfg(SkinnyArgs a, int64_t rows_max, int64_t tiles_y, hipStream_t s) {
    constexpr int NTILE = GLU ? 1 : NT;
    constexpr int64_t kXBudget = 56 * 1024;  // bytes of staged activations
    const int64_t nsb = a.k / 256;
    int64_t xch = kXBudget / (rows_max * (256 * 2) + 16);
    xch = xch < 1 ? 1 : xch > nsb ? nsb : xch;
    a.xch = (int)xch;
    a.xstride = (int)(xch * 256 + 8);
    const int64_t xbytes = (rows_max * a.xstride * 2 + 15) / 16 * 16;
    a.red_off = (int)xbytes;
    const size_t lds = (size_t)xbytes + (size_t)(W > 1 ? W - 1 : 0) * NT * MT * 4 * 64 * 4;
    const dim3 grid((unsigned)((a.n + 16 * NTILE - 1) / (16 * NTILE)), (unsigned)tiles_y);
    hipLaunchKernelGGL((mmv_q4k_f16_kernel<NT, MT, W, GLU>), grid, dim3(64 * W), lds, s, a);
}

// Dense: m <= 16 activation rows, one sub-tile.  W (waves splitting K) grows
// with K so every wave streams a few super-blocks and the grid stays large.
// Routed: schedule tiles of kMoeTileRows = 32 rows, two sub-tiles.
hipError_t launch_mmv_q4k(bool glu, const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s) {
    const int64_t nsb = a.k / 256;
    if (a.ws) {
        static_assert(kMoeTileRows == 32, "routed tiles are two 16-row sub-tiles");
        const int64_t rows_max = a.rows_cap < kMoeTileRows ? a.rows_cap : kMoeTileRows;
        if (glu) launch_cfg<2, 2, 4, true>(a, rows_max, grid_tiles, s);
        else launch_cfg<1, 2, 4, false>(a, rows_max, grid_tiles, s);
    } else {
        const int64_t tiles = (a.m + 15) / 16;
        const int64_t rows_max = a.m < 16 ? a.m : 16;
        if (nsb >= 32) launch_cfg<1, 1, 8, false>(a, rows_max, tiles, s);
        else launch_cfg<1, 1, 4, false>(a, rows_max, tiles, s);
    }
    return hipGetLastError();
}

}  // namespace kq
