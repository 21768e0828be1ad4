// skinny.hip -- weight-streaming products for few activation rows:
// the decode GEMV (kq_qmv), the expert-routed product (kq_qmm_id) and the
// fused gate/up + SiLU GLU (kq_moe_glu).
//
// mlx-kquant "bindings.cpp": quantized_matmul, gather_qmm, moe_glu_gather_kq;
// mlx-native "quantized_matmul_id_ggml.rs": the expert-routed matvec and the
// grouped expert GEMM (each expert's weight rows read once per row tile).
//
// One wavefront owns one weight row.  Its 64 lanes stride over the row in
// 32-weight chunks; each chunk is decoded once into registers and applied to
// every activation row of the tile, and the wave reduces across lanes at the
// end.  Accumulation is fp32.
#include "kq_device.h"
#include "kq_internal.h"
#include "pair32.h"

namespace kq {

// ---------------------------------------------------------------- activations
template <int DT> struct Act16;
template <> struct Act16<F32> {
    static __device__ __forceinline__ void load(const void* x, int64_t i, float (&v)[16]) {
        const float4_t* p = (const float4_t*)((const float*)x + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4_t t = p[j];
            v[4 * j] = t[0], v[4 * j + 1] = t[1], v[4 * j + 2] = t[2], v[4 * j + 3] = t[3];
        }
    }
};
template <> struct Act16<F16> {
    static __device__ __forceinline__ void load(const void* x, int64_t i, float (&v)[16]) {
        const u32x4* p = (const u32x4*)((const uint16_t*)x + i);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 t = p[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * j + 2 * e] = half_bits_to_float(t[e] & 0xffffu);
                v[8 * j + 2 * e + 1] = half_bits_to_float(t[e] >> 16);
            }
        }
    }
};
template <> struct Act16<BF16> {
    static __device__ __forceinline__ void load(const void* x, int64_t i, float (&v)[16]) {
        const u32x4* p = (const u32x4*)((const uint16_t*)x + i);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 t = p[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * j + 2 * e] = __builtin_bit_cast(float, t[e] << 16);
                v[8 * j + 2 * e + 1] = __builtin_bit_cast(float, t[e] & 0xffff0000u);
            }
        }
    }
};

// ---------------------------------------------------------------- chunk decode
// Decode 32-weight chunk q of a weight row into w[0..31]; w[0..15] pair with
// activations [xa, xa+16) and w[16..31] with [xb, xb+16).
template <int C> struct Chunk;

// Q4_K chunk q: super-block q/8, quant bytes 32c+16h .. +16 (c = (q/2)%4,
// h = q%2): low nibbles are weights 64c+16h+i (sub-block 2c), high nibbles
// 64c+32+16h+i (sub-block 2c+1).
template <> struct Chunk<Q4_K> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const int64_t sb = q >> 3;
        const int c = (int)(q >> 1) & 3, h = (int)q & 1;
        const uint8_t* blk = row + sb * 144;
        const u32x4 hd = *(const u32x4*)blk;
        const u32x4 qb = *(const u32x4*)(blk + 16 + 32 * c + 16 * h);
        int sc0, m0, sc1, m1;
        q4k_scale_min(hd, 2 * c, sc0, m0);
        q4k_scale_min(hd, 2 * c + 1, sc1, m1);
        const float d = q4k_d(hd), dmin = q4k_dmin(hd);
        const float s0 = d * (float)sc0, s1 = d * (float)sc1;
        const float n0 = dmin * (float)m0, n1 = dmin * (float)m1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t byte = (qb[i >> 2] >> (8 * (i & 3))) & 0xffu;
            w[i] = __builtin_fmaf(s0, (float)(byte & 15u), -n0);
            w[16 + i] = __builtin_fmaf(s1, (float)(byte >> 4), -n1);
        }
        xa = sb * 256 + 64 * c + 16 * h;
        xb = xa + 32;
    }
};

// Q8_0 chunk q: block q (2-byte aligned, read as 16-bit words).
template <> struct Chunk<Q8_0> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const uint16_t* blk = (const uint16_t*)(row + q * 34);
        const float d = half_bits_to_float(blk[0]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t pair = blk[1 + i];
            w[2 * i] = d * (float)(int8_t)(pair & 0xffu);
            w[2 * i + 1] = d * (float)(int8_t)(pair >> 8);
        }
        xa = q * 32;
        xb = xa + 16;
    }
};

// TQ1 chunk q: group q/4, columns 32*(q%4) .. +32.
template <> struct Chunk<TQ1> {
    static __device__ __forceinline__ void decode(const uint8_t* row, int64_t q, float (&w)[32],
                                                  int64_t& xa, int64_t& xb) {
        const uint8_t* blk = row + (q >> 2) * 28;
        const int part = (int)q & 3;
        uint32_t words[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) words[i] = ((const uint32_t*)blk)[i];
        const float s = half_bits_to_float(words[6] >> 16);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int col = 32 * part + i;
            const int slot = col < 125 ? col / 5 : 25;
            const int digit = col < 125 ? col - 5 * slot : col - 125;
            const uint32_t code = (words[slot >> 2] >> (8 * (slot & 3))) & 0xffu;
            w[i] = (float)tq1_trit(code, digit) * s;
        }
        xa = (q >> 2) * 128 + 32 * part;
        xb = xa + 16;
    }
};

// the further GGUF codecs: the shared chunk decoders of kq_device.h
template <> struct Chunk<Q4_0> : Chunk32<Q4_0> {};
template <> struct Chunk<Q5_0> : Chunk32<Q5_0> {};
template <> struct Chunk<Q5_1> : Chunk32<Q5_1> {};
template <> struct Chunk<Q6_K> : Chunk32<Q6_K> {};
template <> struct Chunk<Q2_K> : Chunk32<Q2_K> {};
template <> struct Chunk<Q3_K> : Chunk32<Q3_K> {};
template <> struct Chunk<Q5_K> : Chunk32<Q5_K> {};

__device__ __forceinline__ void store_any(void* y, int64_t i, int dt, float v) {
    if (dt == F32) store_out<F32>(y, i, v);
    else if (dt == F16) store_out<F16>(y, i, v);
    else store_out<BF16>(y, i, v);
}

// ---------------------------------------------------------------- kernel
// Grid: x = weight rows / 4 (one wave per row), y = tiles.  Dense: tile t
// covers activation rows [t*MB, t*MB+MB).  Routed: tile t is entry t of the
// schedule (expert, row_start, num_rows); its rows are perm[row_start + i].
template <int C, int XDT, int MB, bool GLU>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= a.n) return;

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
        row0 = (int64_t)blockIdx.y * MB;
        nrows = a.m - row0 < MB ? a.m - row0 : MB;
    }

    const uint8_t* wrow = expert_base(a.w, a.w_sh, expert, a.n_experts, a.expert_stride) + j * a.row_bytes;
    const uint8_t* wrow2 =
        GLU ? expert_base(a.w2, a.w2_sh, expert, a.n_experts, a.expert_stride) + j * a.row_bytes : nullptr;
    const int64_t nchunks = a.k / 32;

    for (int64_t sub = 0; sub < nrows; sub += MB) {
        const int cnt = (int)(nrows - sub < MB ? nrows - sub : MB);
        int64_t xrow[MB], orow[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int64_t idx = row0 + sub + (i < cnt ? i : 0);
            const int64_t r = perm ? (int64_t)perm[idx] : idx;
            orow[i] = r;
            xrow[i] = perm && a.shared_x ? r / a.top_k : r;
        }
        float acc[MB], acc2[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i] = 0.f, acc2[i] = 0.f;

        if constexpr (XDT == F16 && Pair32<C>::ok) {
            for (int64_t q = lane; q < nchunks; q += 64) {
                uint32_t p[16], p2[16];
                float A[2], B[2], A2[2], B2[2];
                int64_t xa, xb;
                Pair32<C>::decode(wrow, q, p, A, B, xa, xb);
                if (GLU) Pair32<C>::decode(wrow2, q, p2, A2, B2, xa, xb);
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    if (i < cnt) {
                        uint32_t xw[16];
                        load_x_pairs(a.x, xrow[i] * a.x_row + xa, xw);
                        load_x_pairs(a.x, xrow[i] * a.x_row + xb, xw + 8);
                        float s = A[0] * dot16(p, xw);
                        s = __builtin_fmaf(A[1], dot16(p + 8, xw + 8), s);
                        float t0 = 0.f, t1 = 0.f;
                        if (Pair32<C>::has_b) {
                            t0 = sum16(xw);
                            t1 = sum16(xw + 8);
                            s = __builtin_fmaf(B[0], t0, s);
                            s = __builtin_fmaf(B[1], t1, s);
                        }
                        acc[i] += s;
                        if (GLU) {
                            float s2 = A2[0] * dot16(p2, xw);
                            s2 = __builtin_fmaf(A2[1], dot16(p2 + 8, xw + 8), s2);
                            if (Pair32<C>::has_b) {
                                s2 = __builtin_fmaf(B2[0], t0, s2);
                                s2 = __builtin_fmaf(B2[1], t1, s2);
                            }
                            acc2[i] += s2;
                        }
                    }
                }
            }
        } else
        for (int64_t q = lane; q < nchunks; q += 64) {
            float w[32], w2[32];
            int64_t xa, xb;
            Chunk<C>::decode(wrow, q, w, xa, xb);
            if (GLU) Chunk<C>::decode(wrow2, q, w2, xa, xb);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                if (i < cnt) {
                    float xv[16];
                    Act16<XDT>::load(a.x, xrow[i] * a.x_row + xa, xv);
                    float s = 0.f, s2 = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        s = __builtin_fmaf(w[e], xv[e], s);
                        if (GLU) s2 = __builtin_fmaf(w2[e], xv[e], s2);
                    }
                    Act16<XDT>::load(a.x, xrow[i] * a.x_row + xb, xv);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        s = __builtin_fmaf(w[16 + e], xv[e], s);
                        if (GLU) s2 = __builtin_fmaf(w2[16 + e], xv[e], s2);
                    }
                    acc[i] += s;
                    if (GLU) acc2[i] += s2;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            if (i < cnt) {
                const float g = wave_sum(acc[i]);
                float v = g;
                if (GLU) v = glu_act(a.act, g, wave_sum(acc2[i]), a.limit);
                if (lane == 0) store_any(a.y, orow[i] * a.y_row + j, a.y_dt, v);
            }
        }
    }
}

template <int C, int XDT, bool GLU>
static void launch_mb(const SkinnyArgs& a, int mb, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    switch (mb) {
    case 1: hipLaunchKernelGGL((skinny_kernel<C, XDT, 1, GLU>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((skinny_kernel<C, XDT, 4, GLU>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((skinny_kernel<C, XDT, 16, GLU>), grid, block, 0, s, a); break;
    }
}

template <int C, bool GLU>
static void launch_x(int x_dt, const SkinnyArgs& a, int mb, dim3 grid, hipStream_t s) {
    switch (x_dt) {
    case F32: launch_mb<C, F32, GLU>(a, mb, grid, s); break;
    case F16: launch_mb<C, F16, GLU>(a, mb, grid, s); break;
    default: launch_mb<C, BF16, GLU>(a, mb, grid, s); break;
    }
}

hipError_t launch_skinny(int codec, int x_dt, bool glu, const SkinnyArgs& a, int64_t grid_tiles,
                         hipStream_t s) {
    // Q4_K on the matrix cores: routed fp32 activations and routed tiles of
    // more than 16 rows take the grouped kernel (moe_mm.hip); decode shapes
    // with fp16 activations stream weights and activations through LDS
    // (mmv2.hip)
    if (codec == Q4_K && a.ws && (x_dt == F32 || (x_dt == F16 && a.rows_cap > 16))) {
        SkinnyArgs b = a;
        // fp32 row scales: small routings find them per workgroup, larger
        // ones in one pass over the activation rows
        b.xexp_local = a.rows_cap <= 16;
        if (x_dt == F32 && !b.xexp_local) {
            const int64_t x_rows = a.shared_x ? a.rows_cap / a.top_k : a.rows_cap;
            const hipError_t e = launch_row_exp((const float*)a.x, x_rows, a.k,
                                                const_cast<int32_t*>(a.ws) + a.xexp_off, s);
            if (e != hipSuccess) return e;
        }
        return launch_moe_mm(glu, x_dt, b, grid_tiles, s);
    }
    // Q8_0 and the further GGUF codecs over a schedule: routed tiles on the
    // matrix cores (cmv.hip)
    if ((codec >= Q4_0 || codec == Q8_0) && a.ws && (x_dt == F16 || x_dt == F32) &&
        crm_fits(codec, a.k, glu, x_dt == F32)) {
        if (x_dt == F32) {
            const int64_t x_rows = a.shared_x ? a.rows_cap / a.top_k : a.rows_cap;
            const hipError_t e = launch_row_exp((const float*)a.x, x_rows, a.k,
                                                const_cast<int32_t*>(a.ws) + a.xexp_off, s);
            if (e != hipSuccess) return e;
        }
        return launch_crm(codec, glu, x_dt == F32, a, grid_tiles, s);
    }
    // up to four dense fp16 activation rows: unscaled nibbles on the matrix
    // cores, scales applied to the fp32 sub-block sums (mmv3.hip)
    if (codec == Q4_K && x_dt == F16 && !a.ws && !glu && a.m == 1 && mmv3_fits(a.k))
        return launch_mmv3_q4k(a, s);
    if (codec == Q4_K && x_dt == F16 && !a.ws && !glu && a.m <= 4)
        return launch_mmv3m_q4k(a, s);
    if (codec == Q4_K && x_dt == F16 && (a.ws ? a.rows_cap <= 16 : a.m <= 16))
        return launch_mmv2_q4k(glu, a, grid_tiles, s);
    // TQ1 decode GEMV of one fp16 activation row: table-decoded MFMA operands
    if (codec == TQ1 && x_dt == F16 && !a.ws && !glu && a.m == 1 && tq1_mv_fits(a.k))
        return launch_tq1_mv(a.w, a.n, a.k, (const uint16_t*)a.x, a.y, a.y_dt, s);
    // Q8_0 and the further GGUF codecs, one fp16 activation row: weights
    // through LDS
    if ((codec >= Q4_0 || codec == Q8_0) && x_dt == F16 && !a.ws && !glu && a.m == 1 && cmv_fits(codec, a.k))
        return launch_cmv(codec, a.w, a.n, a.k, (const uint16_t*)a.x, a.y, a.y_dt, s);
    // ... and 2..16 rows (dense, the rows contiguous) on the matrix cores
    if ((codec >= Q4_0 || codec == Q8_0) && x_dt == F16 && !a.ws && !glu && a.m >= 2 && a.m <= 16 &&
        a.x_row == a.k && a.y_row == a.n && cmm_fits(codec, a.k, a.m))
        return launch_cmm(codec, a.w, a.n, a.k, (const uint16_t*)a.x, a.m, a.y, a.y_dt, s);
    int mb;
    int64_t tiles;
    if (a.ws) {
        mb = 16;
        tiles = grid_tiles;
    } else {
        mb = a.m <= 1 ? 1 : a.m <= 4 ? 4 : 16;
        tiles = (a.m + mb - 1) / mb;
    }
    const dim3 grid((unsigned)((a.n + 3) / 4), (unsigned)tiles);
    switch (codec) {
    case Q4_K: glu ? launch_x<Q4_K, true>(x_dt, a, mb, grid, s) : launch_x<Q4_K, false>(x_dt, a, mb, grid, s); break;
    case Q8_0: glu ? launch_x<Q8_0, true>(x_dt, a, mb, grid, s) : launch_x<Q8_0, false>(x_dt, a, mb, grid, s); break;
    case Q4_0: glu ? launch_x<Q4_0, true>(x_dt, a, mb, grid, s) : launch_x<Q4_0, false>(x_dt, a, mb, grid, s); break;
    case Q5_0: glu ? launch_x<Q5_0, true>(x_dt, a, mb, grid, s) : launch_x<Q5_0, false>(x_dt, a, mb, grid, s); break;
    case Q5_1: glu ? launch_x<Q5_1, true>(x_dt, a, mb, grid, s) : launch_x<Q5_1, false>(x_dt, a, mb, grid, s); break;
    case Q6_K: glu ? launch_x<Q6_K, true>(x_dt, a, mb, grid, s) : launch_x<Q6_K, false>(x_dt, a, mb, grid, s); break;
    case Q2_K: glu ? launch_x<Q2_K, true>(x_dt, a, mb, grid, s) : launch_x<Q2_K, false>(x_dt, a, mb, grid, s); break;
    case Q3_K: glu ? launch_x<Q3_K, true>(x_dt, a, mb, grid, s) : launch_x<Q3_K, false>(x_dt, a, mb, grid, s); break;
    case Q5_K: glu ? launch_x<Q5_K, true>(x_dt, a, mb, grid, s) : launch_x<Q5_K, false>(x_dt, a, mb, grid, s); break;
    default: glu ? launch_x<TQ1, true>(x_dt, a, mb, grid, s) : launch_x<TQ1, false>(x_dt, a, mb, grid, s); break;
    }
    return hipGetLastError();
}

}  // namespace kq
