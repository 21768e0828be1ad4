// moe_mm.hip -- expert-routed Q4_K products over schedule tiles of up to 32
// rows (prefill routings): kq_qmm_id and the fused gate/up SiLU of
// kq_moe_glu, with fp16 or fp32 activations.
//
// mlx-native "quantized_matmul_id_ggml.rs": the grouped expert GEMM (one
// dispatch over the expert-sorted rows, each expert's weight tile read once
// per row block) and its fused gate_up_silu form; mlx-kquant "bindings.cpp":
// gather_qmm and moe_glu_gather_kq (gate and up share each activation load).
//
// A workgroup takes one schedule tile (one expert, up to 32 rows gathered
// through the permutation) and a block of weight rows: 128 rows of the
// product, or 64 rows of both gate and up for the GLU.  The tile's activation
// rows are staged in LDS once per chunk of K and feed every weight row of the
// block, so activations are re-read once per 64-128 weight rows rather than
// once per 16.  Each wave streams its own 32 weight rows through registers
// (one super-block ahead) and multiplies them with the exact-operand scheme of
// q4k_mfma.h (sc*q as fp16 integers, 6-bit mins as a second MFMA chain, d and
// dmin per super-block in fp32).
//
// fp32 activations: each activation row r is scaled by 2^-e_r (e_r such that
// the row's largest magnitude lies in [2^14, 2^15): from a pre-pass over all
// rows, or found by the workgroup itself when tiles hold few rows) and split
// into fp16 hi + lo parts; both parts go through the MFMAs, and the row's
// result is scaled back by 2^e_r.  hi + lo carries 22 significant bits of
// each scaled element.
#include "kq_device.h"
#include "kq_internal.h"
#include "q4k_mfma.h"
#include "lds_dma.h"

namespace kq {

// ---------------------------------------------------------------- row scales
// e[r] such that max_c |x[r,c]| * 2^-e[r] lies in [2^14, 2^15); 0 for a row
// of zeros or with a non-finite maximum.
__device__ __forceinline__ int row_exponent(float mx) {
    int ex = 0;
    if (mx > 0.f && mx <= 3.402823466e38f) {
        frexpf(mx, &ex);  // mx = f * 2^ex, f in [0.5, 1)
        ex -= 15;
    }
    return ex;
}

__global__ __launch_bounds__(256) void row_exp_kernel(const float* __restrict__ x, int64_t k,
                                                      int32_t* __restrict__ e) {
    __shared__ float part[4];
    const int64_t r = blockIdx.x;
    const float* row = x + r * k;
    float mx = 0.f;
    for (int64_t c = threadIdx.x; c < k; c += 256) mx = fmaxf(mx, fabsf(row[c]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) e[r] = row_exponent(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])));
}

hipError_t launch_row_exp(const float* x, int64_t rows, int64_t k, int32_t* e, hipStream_t s) {
    hipLaunchKernelGGL(row_exp_kernel, dim3((unsigned)rows), dim3(256), 0, s, x, k, e);
    return hipGetLastError();
}

// ---------------------------------------------------------------- product
// W waves; B-set b in {0, 1} of a wave: for the GLU the gate (0) and up (1)
// rows n0 + 16*wave + 0..15, otherwise rows n0 + 16*(2*wave + b) + 0..15.
// XC super-blocks of activations are staged per chunk.
template <int W, bool GLU, bool XF32>
__global__ __launch_bounds__(64 * W) void moe_mm_kernel(SkinnyArgs a) {
    constexpr int ROWS = GLU ? 16 * W : 32 * W;  // output columns of the workgroup
    extern __shared__ __align__(16) uint8_t smem[];
    // fp32 x: [32][xstride] hi and lo parts (then the raw rows); fp16 x:
    // two [32][xstride] chunk buffers, filled alternately
    uint16_t* xh = (uint16_t*)smem;
    uint16_t* xl = (uint16_t*)(smem + a.red_off);
    const int XC = a.xch, XSTRIDE = a.xstride;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int nsb = (int)(a.k / 256);

    if ((int64_t)blockIdx.y >= (int64_t)a.ws[0]) return;
    const int32_t* tile = a.ws + a.tiles_off + 3 * (int64_t)blockIdx.y;
    const int64_t expert = tile[0], row0 = tile[1];
    const int nrows = tile[2];
    const int32_t* perm = a.ws + a.perm_off;
    const int64_t n0 = (int64_t)blockIdx.x * ROWS;
    auto x_row_of = [&](int r) -> int64_t {
        int64_t xr = perm[row0 + r];
        return a.shared_x ? xr / a.top_k : xr;
    };

    // per tile row: the activation row's element offset and, for fp32
    // activations, its scale exponent (found here for small tiles, else
    // from the pre-pass); published by the first chunk's barrier
    __shared__ int64_t xoffs[kMoeTileRows];
    __shared__ int sexp[kMoeTileRows];
    for (int r = wave; r < nrows; r += W) {
        const int64_t xr = x_row_of(r);
        int ex = 0;
        if (XF32) {
            if (a.xexp_local) {
                const float* row = (const float*)a.x + xr * a.x_row;
                float mx = 0.f;
                for (int64_t c = 4 * lane; c < a.k; c += 256) {
                    const float4_t v = *(const float4_t*)(row + c);
                    mx = fmaxf(fmaxf(mx, fmaxf(fabsf(v[0]), fabsf(v[1]))), fmaxf(fabsf(v[2]), fabsf(v[3])));
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
                ex = row_exponent(mx);
            } else {
                ex = a.ws[a.xexp_off + xr];
            }
        }
        if (lane == 0) {
            xoffs[r] = xr * a.x_row;
            sexp[r] = ex;
        }
    }

    const uint8_t* wrow[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const uint8_t* base = expert_base((GLU && b == 1) ? a.w2 : a.w, (GLU && b == 1) ? a.w2_sh : a.w_sh,
                                          expert, a.n_experts, a.expert_stride);
        int64_t n = n0 + (GLU ? 16 * wave : 16 * (2 * wave + b)) + n_l;
        if (n >= a.n) n = a.n - 1;
        wrow[b] = base + n * a.row_bytes;
    }

    float4_t acc[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[b][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    const LaneSel ls = lane_sel(g);
    uint32_t magic_v = 0x64006400u;
    asm volatile("" : "+v"(magic_v));
    const int subtiles = (nrows + 15) / 16;
    int xoff[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int r = 16 * mt + n_l;
        xoff[mt] = (r < nrows ? r : 0) * XSTRIDE + 64 * g;
    }

    u32x4 hd[2], q0[2], q1[2];
    // the weights of one super-block: kWLoads 16-byte loads per lane
    constexpr int kWLoads = 6;
    auto load_w = [&](int sb, u32x4 (&h)[2], u32x4 (&w0)[2], u32x4 (&w1)[2]) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint8_t* p = wrow[b] + (uint32_t)sb * 144u;
            h[b] = *(const u32x4*)p;
            w0[b] = *(const u32x4*)(p + 16 + 32 * g);
            w1[b] = *(const u32x4*)(p + 32 + 32 * g);
        }
    };

    // fp16 activations: the rows of chunk [c0, c0 + XC) are copied straight
    // into LDS one chunk ahead (a 1 KB load per row: XC = 2, rows of at
    // least 1 KB), so their latency overlaps the previous chunk's work.
    // Loads complete in order, so the compiler's own waits on the weight
    // registers stay correct (and only wait longer).
    auto issue_x = [&](int c0, uint16_t* dst) {
        const int nch = nsb - c0 < XC ? nsb - c0 : XC;
        const int pieces = nch * 32, loads = (pieces + 63) / 64;
        for (int r = wave; r < nrows; r += W) {
            const uint8_t* src = (const uint8_t*)((const uint16_t*)a.x + xoffs[r] + (int64_t)c0 * 256);
            for (int i = 0; i < loads; ++i) {
                // lanes past the chunk re-read its first piece into the row's padding
                const int piece = 64 * i + lane < pieces ? 64 * i + lane : 0;
                dma16(src + 16 * piece,
                      __builtin_amdgcn_readfirstlane(lds_addr((const uint8_t*)(dst + r * XSTRIDE) + 1024 * i)));
            }
        }
    };
    // fp32 activations: each chunk (one super-block) of the rows is copied
    // as loaded into a raw buffer one chunk ahead, then split into the hi
    // and lo rows in LDS.
    uint8_t* xraw = smem + 2 * a.red_off;  // [32][1 KB]
    auto issue_raw = [&](int c0) {
        for (int r = wave; r < nrows; r += W) {
            const uint8_t* src = (const uint8_t*)((const float*)a.x + xoffs[r] + (int64_t)c0 * 256);
            dma16(src + 16 * lane, __builtin_amdgcn_readfirstlane(lds_addr(xraw + 1024 * r)));
        }
    };
    __syncthreads();  // the row offsets and exponents
    if (!XF32) issue_x(0, xh);
    else issue_raw(0);
    // the first weights are requested after the first activation copies, so
    // that at every chunk boundary the loads issued after a chunk's copies
    // are exactly the kWLoads of the next super-block's weights, which stay
    // in flight across the wait
    load_w(0, hd, q0, q1);
    // The compiler waits for a weight register by counting only the loads it
    // issued itself, so a wait placed after the next chunk's copies would wait
    // for those copies too.  Taking the current weights before issuing the
    // copies keeps the copies' latency under this chunk's matrix work.
    auto weights_ready = [&]() {
#pragma unroll
        for (int b = 0; b < 2; ++b) asm volatile("" : "+v"(hd[b]), "+v"(q0[b]), "+v"(q1[b]));
    };
    const uint16_t* xcur = xh;

    int ci = 0;
    for (int c0 = 0; c0 < nsb; c0 += XC, ++ci) {
        const int nch = nsb - c0 < XC ? nsb - c0 : XC;
        if (!XF32) {
            // this wave's copies of chunk ci have landed (loads complete in
            // issue order; only the prefetched weights may be outstanding)
            wait_loads_le(kWLoads);
            __syncthreads();   // every wave's, and every wave is done with chunk ci - 1
            weights_ready();
            if (c0 + XC < nsb) issue_x(c0 + XC, (ci & 1) ? xh : xl);
            xcur = (ci & 1) ? xl : xh;
        } else {
            wait_loads_le(kWLoads);  // this wave's copies of the chunk have landed
            __syncthreads();   // every wave's, and every wave is done with the previous chunk
            // ---- split activation rows of super-block c0 (XC = 1): a wave
            // per row, lane q on columns 4q..4q+3
            for (int r = wave; r < nrows; r += W) {
                const float* src = (const float*)(xraw + 1024 * r);
                const int nex = -sexp[r];
                {
                    const int q = lane;
                    const float4_t v = *(const float4_t*)(src + 4 * q);
                    uint32_t hi[2], lo[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float s0 = ldexpf(v[2 * j], nex), s1 = ldexpf(v[2 * j + 1], nex);
                        const uint32_t h0 = float_to_half_bits(s0), h1 = float_to_half_bits(s1);
                        const uint32_t l0 = float_to_half_bits(s0 - half_bits_to_float(h0));
                        const uint32_t l1 = float_to_half_bits(s1 - half_bits_to_float(h1));
                        hi[j] = h0 | (h1 << 16);
                        lo[j] = l0 | (l1 << 16);
                    }
                    *(uint2*)&xh[r * XSTRIDE + 4 * q] = uint2{hi[0], hi[1]};
                    *(uint2*)&xl[r * XSTRIDE + 4 * q] = uint2{lo[0], lo[1]};
                }
            }
            __syncthreads();  // hi and lo rows ready, raw buffer free
            weights_ready();
            if (c0 + 1 < nsb) issue_raw(c0 + 1);
        }

        for (int sb = c0; sb < c0 + nch; ++sb) {
            u32x4 nhd[2], nq0[2], nq1[2];
            load_w(sb + 1 < nsb ? sb + 1 : sb, nhd, nq0, nq1);
            // the next super-block's loads go out before this one's decode
            __builtin_amdgcn_sched_barrier(0);
            Q4Operands op[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) q4k_operands(hd[b], q0[b], q1[b], ls, magic_v, op[b]);
            const int sl = (sb - c0) * 256;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                if (mt < subtiles) {
                    u32x4 xa[8], xb[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int o = xoff[mt] + sl + 32 * (i >> 2) + 8 * (i & 3);
                        xa[i] = *(const u32x4*)&xcur[o];
                        if (XF32) xb[i] = *(const u32x4*)&xl[o];
                    }
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        float4_t c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            c1 = mfma16(xa[i], op[b].w[i], c1);
                            c2 = mfma16(xa[i], i < 4 ? op[b].m_lo : op[b].m_hi, c2);
                        }
                        if (XF32) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                c1 = mfma16(xb[i], op[b].w[i], c1);
                                c2 = mfma16(xb[i], i < 4 ? op[b].m_lo : op[b].m_hi, c2);
                            }
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[b][mt][v] += op[b].d * c1[v] - op[b].dmin * c2[v];
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) hd[b] = nhd[b], q0[b] = nq0[b], q1[b] = nq1[b];
        }
    }

    // ---- store: lane holds activation rows 16*mt + 4g + v of weight row n_l
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int idx = 16 * mt + 4 * g + v;
            if (idx >= nrows) continue;
            const int64_t orow = perm[row0 + idx];
            // fp32 activations: the row's result scaled back by 2^e exactly
            auto back = [&](float v) { return XF32 ? ldexpf(v, sexp[idx]) : v; };
            if (GLU) {
                const int64_t n = n0 + 16 * wave + n_l;
                if (n < a.n)
                    store_val(a.y, orow * a.y_row + n, a.y_dt,
                              glu_act(a.act, back(acc[0][mt][v]), back(acc[1][mt][v]), a.limit));
            } else {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int64_t n = n0 + 16 * (2 * wave + b) + n_l;
                    if (n < a.n) store_val(a.y, orow * a.y_row + n, a.y_dt, back(acc[b][mt][v]));
                }
            }
        }
    }
}

// Staged activations, up to 32 rows (no more than the routing holds), each
// filled by direct-to-LDS copies one chunk ahead: fp16 activations in two
// buffers of two super-blocks per row (whole 1 KB copies); fp32 activations
// as hi and lo rows of one super-block beside a raw 1 KB row buffer.  About
// 66 KB for 32 rows, so two workgroups share a CU.
template <int W, bool GLU, bool XF32>
static void launch_mm(SkinnyArgs a, int64_t grid_tiles, hipStream_t s) {
    constexpr int ROWS = GLU ? 16 * W : 32 * W;
    const int64_t rows = a.rows_cap < kMoeTileRows ? a.rows_cap : kMoeTileRows;
    const int64_t xc = XF32 ? 1 : 2;
    a.xch = (int)xc;
    a.xstride = (int)(xc * 256 + 8);
    const int64_t part_bytes = (rows * a.xstride * 2 + 15) / 16 * 16;
    a.red_off = (int)part_bytes;  // start of the lo part, or of the second buffer
    const size_t lds = (size_t)(2 * part_bytes + (XF32 ? rows * 1024 : 0));
    const dim3 grid((unsigned)((a.n + ROWS - 1) / ROWS), (unsigned)grid_tiles);
    hipLaunchKernelGGL((moe_mm_kernel<W, GLU, XF32>), grid, dim3(64 * W), lds, s, a);
}

hipError_t launch_moe_mm(bool glu, int x_dt, const SkinnyArgs& a, int64_t grid_tiles,
                         hipStream_t s) {
    static_assert(kMoeTileRows == 32, "a schedule tile is two 16-row MFMA sub-tiles");
    if (x_dt == F32) {
        if (glu) launch_mm<4, true, true>(a, grid_tiles, s);
        else launch_mm<4, false, true>(a, grid_tiles, s);
    } else {
        if (glu) launch_mm<4, true, false>(a, grid_tiles, s);
        else launch_mm<4, false, false>(a, grid_tiles, s);
    }
    return hipGetLastError();
}

}  // namespace kq
