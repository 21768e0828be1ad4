// quantize.hip -- float weights -> block bytes (kq_quantize) and the TQ1
// legality scan (kq_validate_tq1).
//
// mlx-kquant "bindings.cpp", quantize: float weights whose last dimension is
// a multiple of the codec's block size become the codec's wire bytes, with an
// optional importance vector of length K steering the K-quant encoder.
// Ternary Bonsai "ternel_packed_model.py", kernels section ("Bounds safety"):
// code legality is established at conversion, outside the product kernels.
//
// The encoders (the pages give the contract, not an algorithm):
//   Q8_0   d = fp16(max|w| / 127), q = clamp(rint(w * (1/d)), -127, 127)
//   TQ1    s = fp16(max|w|) per 128 weights, trit = clamp(rint(w * (1/s)), -1, 1)
//   Q4_K   per 32-weight sub-block the range [lo, hi] with lo = min(0, min w):
//          scale r = (hi - lo) / 15 and min mn = -lo (with an importance
//          vector, r is the best of eight shrunk candidates r (16 - t) / 16
//          under the importance-weighted squared error of the levels
//          lo + s q); d = fp16(max r / 63), dmin = fp16(max mn / 63),
//          sc = clamp(rint(r / d), 0, 63), m = clamp(rint(mn / dmin), 0, 63),
//          q = clamp(rint((w + dmin m) / (d sc)), 0, 15).
// Scales past 65504 are clamped to it.  Every step is one binary32 operation
// in a fixed order (no contraction into fused multiply-adds, correctly
// rounded division, rint to nearest even), so the bytes are reproducible
// bit for bit by any implementation of the same steps.
#include "kq_device.h"
#include "kq_internal.h"

#pragma clang fp contract(off)

namespace kq {

namespace {

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
    return v < lo ? lo : v > hi ? hi : v;
}

// fp16 bits of a non-negative scale, clamped to the largest finite fp16
__device__ __forceinline__ uint32_t scale_half(float v) {
    if (v > 65504.0f) v = 65504.0f;
    return float_to_half_bits(v);
}

template <int DT> __device__ __forceinline__ float wload(const void* w, int64_t i) {
    return load_act<DT>(w, i);
}

// ---------------------------------------------------------------- Q8_0
template <int DT>
__global__ __launch_bounds__(256) void quant_q8_0_kernel(const void* __restrict__ w, int64_t nblk,
                                                         uint8_t* __restrict__ out) {
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk;
         b += (int64_t)gridDim.x * 256) {
        float x[32];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            x[i] = wload<DT>(w, b * 32 + i);
            const float a = __builtin_fabsf(x[i]);
            if (a > amax) amax = a;
        }
        const uint32_t dh = scale_half(amax / 127.0f);
        const float d = half_bits_to_float(dh);
        const float inv = d > 0.0f ? 1.0f / d : 0.0f;
        uint16_t* o = (uint16_t*)(out + b * 34);  // 34-byte blocks: 2-byte aligned
        o[0] = (uint16_t)dh;
#pragma unroll
        for (int i = 0; i < 32; i += 2) {
            const int q0 = (int)clampf(__builtin_rintf(x[i] * inv), -127.0f, 127.0f);
            const int q1 = (int)clampf(__builtin_rintf(x[i + 1] * inv), -127.0f, 127.0f);
            o[1 + i / 2] = (uint16_t)((q0 & 0xff) | ((q1 & 0xff) << 8));
        }
    }
}

// ---------------------------------------------------------------- TQ1_G128
template <int DT>
__global__ __launch_bounds__(256) void quant_tq1_kernel(const void* __restrict__ w, int64_t nblk,
                                                        uint8_t* __restrict__ out) {
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk;
         b += (int64_t)gridDim.x * 256) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            const float a = __builtin_fabsf(wload<DT>(w, b * 128 + i));
            if (a > amax) amax = a;
        }
        const uint32_t sh = scale_half(amax);
        const float sv = half_bits_to_float(sh);
        const float inv = sv > 0.0f ? 1.0f / sv : 0.0f;
        uint32_t words[7] = {0u, 0u, 0u, 0u, 0u, 0u, 0u};
        for (int slot = 0; slot < 26; ++slot) {
            const int nd = slot < 25 ? 5 : 3;
            uint32_t code = 0, p = 1;
            for (int dgt = 0; dgt < nd; ++dgt) {
                const int c = slot < 25 ? 5 * slot + dgt : 125 + dgt;
                const float t = clampf(__builtin_rintf(wload<DT>(w, b * 128 + c) * inv), -1.0f, 1.0f);
                code += (uint32_t)((int)t + 1) * p;
                p *= 3u;
            }
            words[slot >> 2] |= code << (8 * (slot & 3));
        }
        words[6] |= sh << 16;  // bytes 26, 27: the scale
        uint32_t* o = (uint32_t*)(out + b * 28);  // 28-byte blocks: 4-byte aligned
#pragma unroll
        for (int i = 0; i < 7; ++i) o[i] = words[i];
    }
}

// ---------------------------------------------------------------- Q4_K
// Importance-weighted squared error of the levels lo + s q (q nearest,
// clamped to 0..15) over a sub-block, summed in order.
__device__ __forceinline__ float q4k_level_err(const float (&x)[32], const float (&imp)[32],
                                               float lo, float s) {
    float e = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float q = s > 0.0f ? clampf(__builtin_rintf((x[i] - lo) / s), 0.0f, 15.0f) : 0.0f;
        const float r = x[i] - (lo + s * q);
        e = e + imp[i] * (r * r);
    }
    return e;
}

// Eight lanes per super-block: lane j of the group owns sub-block j.
template <int DT>
__global__ __launch_bounds__(256) void quant_q4k_kernel(const void* __restrict__ w, int64_t k,
                                                        int64_t nblk,
                                                        const float* __restrict__ imatrix,
                                                        uint8_t* __restrict__ out) {
    const int lane = threadIdx.x & 63, j = lane & 7;
    const int64_t groups = (int64_t)gridDim.x * 32;  // super-blocks per pass of the grid
    for (int64_t b0 = (int64_t)blockIdx.x * 32; b0 < nblk; b0 += groups) {
        const int64_t b = b0 + (threadIdx.x >> 3);
        const bool live = b < nblk;  // whole groups of eight lanes share b
        const int64_t base = (live ? b : 0) * 256 + 32 * j;
        const int64_t col = (base % k);  // column of the sub-block's first weight
        float x[32], imp[32];
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            x[i] = wload<DT>(w, base + i);
            imp[i] = imatrix ? imatrix[col + i] : 0.0f;
            if (i == 0) hi = x[0];
            if (x[i] < lo) lo = x[i];
            if (x[i] > hi) hi = x[i];
        }
        float r = (hi - lo) / 15.0f;
        if (imatrix) {
            float best = 0.0f;
            int best_t = 0;
            for (int t = 0; t < 8; ++t) {
                const float s = (r * (float)(16 - t)) * 0.0625f;
                const float e = q4k_level_err(x, imp, lo, s);
                if (t == 0 || e < best) {
                    best = e;
                    best_t = t;
                }
            }
            r = (r * (float)(16 - best_t)) * 0.0625f;
        }
        const float mn = -lo;
        // maxima over the sub-blocks, starting from +0 (a zero range or min
        // of -0 must not give a negative-zero scale)
        float rmax = r > 0.0f ? r : 0.0f, mmax = mn > 0.0f ? mn : 0.0f;
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            const float r2 = __shfl_xor(rmax, off, 64), m2 = __shfl_xor(mmax, off, 64);
            rmax = r2 > rmax ? r2 : rmax;
            mmax = m2 > mmax ? m2 : mmax;
        }
        const uint32_t dh = scale_half(rmax / 63.0f), mh = scale_half(mmax / 63.0f);
        const float d = half_bits_to_float(dh), dmin = half_bits_to_float(mh);
        const int sc = d > 0.0f ? (int)clampf(__builtin_rintf(r / d), 0.0f, 63.0f) : 0;
        const int m = dmin > 0.0f ? (int)clampf(__builtin_rintf(mn / dmin), 0.0f, 63.0f) : 0;
        // the eight (scale, min) pairs in every lane of the group
        int scs[8], ms[8];
        const int g0 = lane & ~7;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            scs[i] = __shfl(sc, g0 + i, 64);
            ms[i] = __shfl(m, g0 + i, 64);
        }
        // this sub-block's quants, one per byte (4 per dword)
        const float step = d * (float)sc, offs = dmin * (float)m;
        uint32_t qb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xv = x[4 * i + e];
                const uint32_t q = step > 0.0f ? (uint32_t)clampf(__builtin_rintf((xv + offs) / step), 0.0f, 15.0f) : 0u;
                v |= q << (8 * e);
            }
            qb[i] = v;
        }
        // sub-blocks 2c (low nibbles) and 2c+1 (high nibbles) share the 32
        // quant bytes 32c..32c+31: the even lane combines them
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t other = (uint32_t)__shfl_xor((int)qb[i], 1, 64);
            qb[i] = qb[i] | (other << 4);
        }
        if (!live) continue;
        uint8_t* blk = out + b * 144;  // 144-byte blocks: 16-byte aligned
        if ((j & 1) == 0) {
            u32x4* qo = (u32x4*)(blk + 16 + 32 * (j >> 1));
            qo[0] = u32x4{qb[0], qb[1], qb[2], qb[3]};
            qo[1] = u32x4{qb[4], qb[5], qb[6], qb[7]};
        }
        if (j == 0) {
            // the GGUF K-quant packing: sub-blocks 0..3 in the low six bits
            // of bytes 0..3 (scales) and 4..7 (mins); sub-blocks 4..7 with
            // their low four bits in bytes 8..11 and their top two bits in the
            // top bits of bytes 0..7
            uint32_t S[3] = {0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S[0] |= (uint32_t)((scs[i] & 63) | ((scs[i + 4] >> 4) << 6)) << (8 * i);
                S[1] |= (uint32_t)((ms[i] & 63) | ((ms[i + 4] >> 4) << 6)) << (8 * i);
                S[2] |= (uint32_t)((scs[i + 4] & 15) | ((ms[i + 4] & 15) << 4)) << (8 * i);
            }
            *(u32x4*)blk = u32x4{dh | (mh << 16), S[0], S[1], S[2]};
        }
    }
}

// ---------------------------------------------------------------- TQ1 scan
__global__ __launch_bounds__(64) void zero_u64_kernel(unsigned long long* p) {
    if (threadIdx.x == 0) *p = 0ull;
}

__global__ __launch_bounds__(256) void tq1_illegal_kernel(const uint8_t* __restrict__ w,
                                                          int64_t nblk,
                                                          unsigned long long* __restrict__ count) {
    unsigned long long bad = 0ull;
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk;
         b += (int64_t)gridDim.x * 256) {
        const uint32_t* p = (const uint32_t*)(w + b * 28);
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            const uint32_t v = p[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int byte = 4 * i + e;
                const uint32_t c = (v >> (8 * e)) & 0xffu;
                if (byte < 25) bad += c > 242u;
                else if (byte == 25) bad += c > 26u;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)bad, off, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(bad >> 32), off, 64);
        bad += ((unsigned long long)hi << 32) | lo;
    }
    if ((threadIdx.x & 63) == 0 && bad) atomicAdd(count, bad);
}

template <int DT>
void launch_quant_dt(int codec, const void* w, int64_t rows, int64_t k, const float* imatrix,
                     uint8_t* out, hipStream_t s) {
    const int64_t nblk = rows * (k / (codec == Q4_K ? 256 : codec == Q8_0 ? 32 : 128));
    if (codec == Q4_K) {
        const int64_t wg = (nblk + 31) / 32;
        const unsigned grid = (unsigned)(wg < 65536 ? wg : 65536);
        hipLaunchKernelGGL(quant_q4k_kernel<DT>, dim3(grid), dim3(256), 0, s, w, k, nblk, imatrix,
                           out);
        return;
    }
    const int64_t wg = (nblk + 255) / 256;
    const unsigned grid = (unsigned)(wg < 65536 ? wg : 65536);
    if (codec == Q8_0) hipLaunchKernelGGL(quant_q8_0_kernel<DT>, dim3(grid), dim3(256), 0, s, w, nblk, out);
    else hipLaunchKernelGGL(quant_tq1_kernel<DT>, dim3(grid), dim3(256), 0, s, w, nblk, out);
}

}  // namespace

hipError_t launch_quantize(int codec, const void* w, int w_dt, int64_t rows, int64_t k,
                           const float* imatrix, void* out, hipStream_t s) {
    uint8_t* o = (uint8_t*)out;
    if (w_dt == F32) launch_quant_dt<F32>(codec, w, rows, k, imatrix, o, s);
    else if (w_dt == F16) launch_quant_dt<F16>(codec, w, rows, k, imatrix, o, s);
    else launch_quant_dt<BF16>(codec, w, rows, k, imatrix, o, s);
    return hipGetLastError();
}

hipError_t launch_tq1_illegal(const void* w, int64_t rows, int64_t k, unsigned long long* count,
                              hipStream_t s) {
    hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, s, count);
    const int64_t nblk = rows * (k / 128);
    const int64_t wg = (nblk + 255) / 256;
    const unsigned grid = (unsigned)(wg < 16384 ? (wg > 0 ? wg : 1) : 16384);
    hipLaunchKernelGGL(tq1_illegal_kernel, dim3(grid), dim3(256), 0, s, (const uint8_t*)w, nblk,
                       count);
    return hipGetLastError();
}

}  // namespace kq
