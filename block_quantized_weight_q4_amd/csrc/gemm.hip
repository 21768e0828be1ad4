// gemm.hip -- prefill product Y[M,N] = X[M,K] * dequant(W)[N,K]^T (kq_qmm).
//
// mlx-kquant "bindings.cpp", quantized_matmul; Ternary Bonsai
// "ternel_packed_model.py", tq1_gemm (decode a weight once and reuse it
// across a whole block of activation rows on the matrix units).
//
// The contraction runs on MFMA in the activation's 16-bit type (bf16 or fp16)
// with fp32 accumulation.  Each K step the workgroup decodes its weight tile
// once into LDS (so every decoded weight feeds BM rows), stages the matching
// activation tile, and four waves each multiply a 64x64 sub-tile with
// 32x32x16 MFMAs.
#include "kq_device.h"
#include "kq_internal.h"

namespace kq {

constexpr int BM = 128, BN = 128, BK = 64, LDS_STRIDE = BK + 8;  // +8: bank spread

template <int XDT> struct Mfma;
template <> struct Mfma<BF16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ uint16_t cvt(float f) { return float_to_bf16_bits(f); }
    static __device__ __forceinline__ float16_t mma(const short8& a, const short8& b, float16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<F16> {
    typedef half8 vec;
    static __device__ __forceinline__ uint16_t cvt(float f) { return float_to_half_bits(f); }
    static __device__ __forceinline__ float16_t mma(const short8& a, const short8& b, float16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
};

// Decode this thread's 32 weights of the BK=64 step `s` for weight row n into
// v[0..31], destined for tile columns col0 .. col0+15 and col1 .. col1+15.
template <int C> struct TileFill;

// Q4_K: step s is chunk c = s%4 of super-block s/4 (sub-blocks 2c and 2c+1).
// Thread half h takes quant bytes 32c+16h..+16: low nibbles -> columns 16h+i,
// high nibbles -> 32+16h+i.
template <> struct TileFill<Q4_K> {
    static __device__ __forceinline__ bool fill(const uint8_t* row, int64_t k, int64_t s, int h,
                                                float (&v)[32], int& col0, int& col1) {
        const int64_t sb = s >> 2;
        const int c = (int)s & 3;
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
            v[i] = __builtin_fmaf(s0, (float)(byte & 15u), -n0);
            v[16 + i] = __builtin_fmaf(s1, (float)(byte >> 4), -n1);
        }
        col0 = 16 * h;
        col1 = 32 + 16 * h;
        return true;
    }
};

// Q8_0: step s covers blocks 2s and 2s+1; thread half h takes block 2s+h.
template <> struct TileFill<Q8_0> {
    static __device__ __forceinline__ bool fill(const uint8_t* row, int64_t k, int64_t s, int h,
                                                float (&v)[32], int& col0, int& col1) {
        const int64_t b = 2 * s + h;
        col0 = 32 * h;
        col1 = 32 * h + 16;
        if (b * 32 >= k) return false;
        const uint16_t* blk = (const uint16_t*)(row + b * 34);
        const float d = half_bits_to_float(blk[0]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t pair = blk[1 + i];
            v[2 * i] = d * (float)(int8_t)(pair & 0xffu);
            v[2 * i + 1] = d * (float)(int8_t)(pair >> 8);
        }
        return true;
    }
};

// TQ1: step s is half s%2 of group s/2; thread half h takes columns
// 64*(s%2) + 32h .. +32 of the group.
template <> struct TileFill<TQ1> {
    static __device__ __forceinline__ bool fill(const uint8_t* row, int64_t k, int64_t s, int h,
                                                float (&v)[32], int& col0, int& col1) {
        const uint8_t* blk = row + (s >> 1) * 28;
        const int base = 64 * ((int)s & 1) + 32 * h;
        uint32_t words[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) words[i] = ((const uint32_t*)blk)[i];
        const float sc = half_bits_to_float(words[6] >> 16);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int col = base + i;
            const int slot = col < 125 ? col / 5 : 25;
            const int digit = col < 125 ? col - 5 * slot : col - 125;
            const uint32_t code = (words[slot >> 2] >> (8 * (slot & 3))) & 0xffu;
            v[i] = (float)tq1_trit(code, digit) * sc;
        }
        col0 = 32 * h;
        col1 = 32 * h + 16;
        return true;
    }
};

template <int C, int XDT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ w, int64_t n,
                                                   int64_t k, const uint16_t* __restrict__ x,
                                                   int64_t m, void* __restrict__ y, int y_dt) {
    __shared__ uint16_t As[BM * LDS_STRIDE];
    __shared__ uint16_t Bs[BN * LDS_STRIDE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
    const int64_t row_bytes = (k / CodecInfo<C>::QK) * CodecInfo<C>::BYTES;

    float16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = float16_t{};

    // fill roles: tile row r = tid/2, half h = tid%2
    const int fr = tid >> 1, fh = tid & 1;
    const int64_t wrow_idx = n0 + fr;
    const uint8_t* wrow = w + (wrow_idx < n ? wrow_idx : n - 1) * row_bytes;
    const int64_t xrow_idx = m0 + fr;
    const uint16_t* xrow = x + (xrow_idx < m ? xrow_idx : 0) * k;

    const int64_t steps = (k + BK - 1) / BK;
    for (int64_t s = 0; s < steps; ++s) {
        // activation tile: row fr, columns 32*fh .. +32
        {
            u32x4 v[4] = {};
            const int64_t c0 = s * BK + 32 * fh;
            if (xrow_idx < m && c0 < k) {
                const u32x4* p = (const u32x4*)(xrow + c0);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = p[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) *(u32x4*)&As[fr * LDS_STRIDE + 32 * fh + 8 * i] = v[i];
        }
        // weight tile: decode once, round to the MFMA type
        {
            float v[32];
            int col0 = C == Q4_K ? 16 * fh : 32 * fh;
            int col1 = C == Q4_K ? 32 + 16 * fh : 32 * fh + 16;
            const bool ok = wrow_idx < n && TileFill<C>::fill(wrow, k, s, fh, v, col0, col1);
            if (!ok) {
#pragma unroll
                for (int i = 0; i < 32; ++i) v[i] = 0.f;
            }
            u32x4 p0, p1, p2, p3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p0[i] = Mfma<XDT>::cvt(v[2 * i]) | ((uint32_t)Mfma<XDT>::cvt(v[2 * i + 1]) << 16);
                p1[i] = Mfma<XDT>::cvt(v[8 + 2 * i]) | ((uint32_t)Mfma<XDT>::cvt(v[9 + 2 * i]) << 16);
                p2[i] = Mfma<XDT>::cvt(v[16 + 2 * i]) | ((uint32_t)Mfma<XDT>::cvt(v[17 + 2 * i]) << 16);
                p3[i] = Mfma<XDT>::cvt(v[24 + 2 * i]) | ((uint32_t)Mfma<XDT>::cvt(v[25 + 2 * i]) << 16);
            }
            *(u32x4*)&Bs[fr * LDS_STRIDE + col0] = p0;
            *(u32x4*)&Bs[fr * LDS_STRIDE + col0 + 8] = p1;
            *(u32x4*)&Bs[fr * LDS_STRIDE + col1] = p2;
            *(u32x4*)&Bs[fr * LDS_STRIDE + col1 + 8] = p3;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            short8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + 32 * i + (lane & 31);
                af[i] = *(const short8*)&As[r * LDS_STRIDE + 16 * ks + 8 * (lane >> 5)];
                const int c = wn * 64 + 32 * i + (lane & 31);
                bf[i] = *(const short8*)&Bs[c * LDS_STRIDE + 16 * ks + 8 * (lane >> 5)];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = Mfma<XDT>::mma(af[i], bf[j], acc[i][j]);
        }
        __syncthreads();
    }

    // epilogue: lane holds column l%32 and rows 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < m && col < n) {
                    const float o = acc[i][j][v];
                    if (y_dt == F32) store_out<F32>(y, row * n + col, o);
                    else if (y_dt == F16) store_out<F16>(y, row * n + col, o);
                    else store_out<BF16>(y, row * n + col, o);
                }
            }
        }
}

template <int C>
static void launch_c(int x_dt, const void* w, int64_t n, int64_t k, const void* x, int64_t m,
                     void* y, int y_dt, hipStream_t s) {
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM)), block(256);
    if (x_dt == BF16)
        hipLaunchKernelGGL((gemm_kernel<C, BF16>), grid, block, 0, s, (const uint8_t*)w, n, k,
                           (const uint16_t*)x, m, y, y_dt);
    else
        hipLaunchKernelGGL((gemm_kernel<C, F16>), grid, block, 0, s, (const uint8_t*)w, n, k,
                           (const uint16_t*)x, m, y, y_dt);
}

hipError_t launch_gemm(int codec, int x_dt, const void* w, int64_t n, int64_t k, const void* x,
                       int64_t m, void* y, int y_dt, hipStream_t s) {
    switch (codec) {
    case Q4_K: launch_c<Q4_K>(x_dt, w, n, k, x, m, y, y_dt, s); break;
    case Q8_0: launch_c<Q8_0>(x_dt, w, n, k, x, m, y, y_dt, s); break;
    default: launch_c<TQ1>(x_dt, w, n, k, x, m, y, y_dt, s); break;
    }
    return hipGetLastError();
}

}  // namespace kq
