// dequant.hip -- block bytes -> dense fp32 / fp16 / bf16 (kq_dequantize).
//
// mlx-kquant "bindings.cpp", dequantize; Ternary Bonsai
// "ternel_packed_model.py", get_rows.  HBM-bound streaming: every thread
// reads one aligned slice of a block and writes 8..32 contiguous outputs, so
// reads and writes are coalesced across the wave.
//
// Exactness: every decoded weight is formed with one rounding in fp32.
//   Q4_K: (d*sc) and (d*sc)*q are exact (<= 21 significant bits), dmin*m is
//         exact (<= 17 bits); the final fused multiply-subtract rounds once.
//   Q8_0: d*q is exact (<= 19 bits).
//   TQ1:  (t-1)*s is exact.
//   Q4_0 / Q5_0: d*(q-8), d*(q-16) are exact; Q5_1: d*q+m fused, one
//         rounding; Q6_K and Q3_K: d*sc and (d*sc)*q are exact; Q2_K and
//         Q5_K: as Q4_K.
// fp16/bf16 outputs then round that fp32 value to nearest even.
#include "kq_device.h"
#include "kq_internal.h"

namespace kq {

// 8 consecutive outputs.  Outputs are written once and not read back here,
// so they are stored non-temporally (they need not stay in the caches).
template <int DT> struct Out8;
template <> struct Out8<F32> {
    static __device__ __forceinline__ void store(void* out, int64_t i, const float (&v)[8]) {
        float4_t* p = (float4_t*)((float*)out + i);
        __builtin_nontemporal_store(float4_t{v[0], v[1], v[2], v[3]}, p);
        __builtin_nontemporal_store(float4_t{v[4], v[5], v[6], v[7]}, p + 1);
    }
};
template <> struct Out8<F16> {
    static __device__ __forceinline__ void store(void* out, int64_t i, const float (&v)[8]) {
        u32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = float_to_half_bits(v[2 * j]) | ((uint32_t)float_to_half_bits(v[2 * j + 1]) << 16);
        __builtin_nontemporal_store(r, (u32x4*)((uint16_t*)out + i));
    }
};
template <> struct Out8<BF16> {
    static __device__ __forceinline__ void store(void* out, int64_t i, const float (&v)[8]) {
        u32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = float_to_bf16_bits(v[2 * j]) | ((uint32_t)float_to_bf16_bits(v[2 * j + 1]) << 16);
        __builtin_nontemporal_store(r, (u32x4*)((uint16_t*)out + i));
    }
};

// Q4_K: each thread writes V consecutive weights of one sub-block (V = 4 for
// fp32, 8 for 16-bit outputs: 16 bytes), so the lanes of a wave store
// consecutive 16-byte pieces and every store instruction is one contiguous
// 1 KB run.  Weight w of a super-block lies in chunk c = w / 64; its first 32
// weights are the low nibbles of quant bytes 32c.., the next 32 the high
// nibbles of the same bytes.
template <int DT>
__global__ __launch_bounds__(256) void dequant_q4k_kernel(const uint8_t* __restrict__ w,
                                                          void* __restrict__ out, int64_t nblocks) {
    constexpr int V = DT == F32 ? 4 : 8, TPB = 256 / V;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = t / TPB;
    if (b >= nblocks) return;
    const int w0 = V * (int)(t % TPB);
    const int c = w0 >> 6, off = w0 & 63, hi = off >> 5, byte0 = 32 * c + (off & 31);
    const uint8_t* blk = w + b * 144;
    const u32x4 hd = *(const u32x4*)blk;
    uint32_t q[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) q[i] = *(const uint32_t*)(blk + 16 + byte0 + 4 * i);
    int sc, m;
    q4k_scale_min(hd, 2 * c + hi, sc, m);
    const float sd = q4k_d(hd) * (float)sc, mn = q4k_dmin(hd) * (float)m;
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const uint32_t byte = (q[i >> 2] >> (8 * (i & 3))) & 0xffu;
        v[i] = __builtin_fmaf(sd, (float)((byte >> (4 * hi)) & 15u), -mn);
    }
    const int64_t base = b * 256 + w0;
    if (DT == F32) {
        __builtin_nontemporal_store(float4_t{v[0], v[1], v[2], v[3]}, (float4_t*)((float*)out + base));
    } else {
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = v[i % V];
        Out8<DT>::store(out, base, v8);
    }
}

// Q8_0: 4 threads per 34-byte block, 8 weights each.  Blocks are only 2-byte
// aligned, so quants are read as 16-bit words.
template <int DT>
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ w,
                                                           void* __restrict__ out, int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = t >> 2;
    if (b >= nblocks) return;
    const int h = t & 3;
    const uint16_t* blk = (const uint16_t*)(w + b * 34);
    const float d = half_bits_to_float(blk[0]);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pair = blk[1 + 4 * h + i];
        v[2 * i] = d * (float)(int8_t)(pair & 0xffu);
        v[2 * i + 1] = d * (float)(int8_t)(pair >> 8);
    }
    Out8<DT>::store(out, b * 32 + 8 * h, v);
}

// TQ1_G128: 16 threads per 28-byte block, 8 columns each.  Column c < 125 is
// digit c % 5 of code byte c / 5; columns 125..127 are digits 0..2 of the
// tail byte; weight = (digit - 1) * scale.
template <int DT>
__global__ __launch_bounds__(256) void dequant_tq1_kernel(const uint8_t* __restrict__ w,
                                                          void* __restrict__ out, int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = t >> 4;
    if (b >= nblocks) return;
    const int part = t & 15;
    const uint8_t* blk = w + b * 28;
    const float s = half_bits_to_float(*(const uint16_t*)(blk + 26));
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int col = 8 * part + i;
        const int slot = col < 125 ? col / 5 : 25;
        const int digit = col < 125 ? col - 5 * slot : col - 125;
        v[i] = (float)tq1_trit(blk[slot], digit) * s;
    }
    Out8<DT>::store(out, b * 128 + 8 * part, v);
}

// GGUF Q4_0 / Q5_0 / Q5_1 / Q6_K / Q2_K / Q3_K / Q5_K: one thread per 32-weight chunk, decoded
// by the shared chunk decoders (kq_device.h); the chunk's 32 outputs are
// contiguous.  Rows are contiguous in both the blocks and the output, so
// chunk g of the whole matrix is chunk g of one long row.
template <int C, int DT>
__global__ __launch_bounds__(256) void dequant_chunk32_kernel(const uint8_t* __restrict__ w,
                                                              void* __restrict__ out, int64_t nchunks) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= nchunks) return;
    float v[32];
    int64_t xa, xb;
    Chunk32<C>::decode(w, g, v, xa, xb);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = v[16 * h + i], b[i] = v[16 * h + 8 + i];
        const int64_t base = h ? xb : xa;
        Out8<DT>::store(out, base, a);
        Out8<DT>::store(out, base + 8, b);
    }
}

template <int DT>
static hipError_t launch_chunk32_dt(int codec, const void* w, int64_t nchunks, void* out,
                                    hipStream_t s) {
    // chunks of one launch: a multiple of 8 (Q6_K super-blocks hold 8), and
    // fewer than 2^31 work-items
    const int64_t piece = (int64_t)1 << 30;
    const int64_t bbytes = codec == Q4_0 ? 18 : codec == Q5_0 ? 22 : codec == Q5_1 ? 24
                         : codec == Q6_K ? 210 : codec == Q2_K ? 84 : codec == Q3_K ? 110 : 176;
    const int64_t per = codec == Q4_0 || codec == Q5_0 || codec == Q5_1 ? 1 : 8;  // chunks per block
    for (int64_t c0 = 0; c0 < nchunks; c0 += piece) {
        const int64_t nc = nchunks - c0 < piece ? nchunks - c0 : piece;
        const uint8_t* wp = (const uint8_t*)w + c0 / per * bbytes;
        void* op = (uint8_t*)out + c0 * 32 * (DT == F32 ? 4 : 2);
        const dim3 grid((unsigned)((nc + 255) / 256)), block(256);
        switch (codec) {
        case Q4_0: hipLaunchKernelGGL((dequant_chunk32_kernel<Q4_0, DT>), grid, block, 0, s, wp, op, nc); break;
        case Q5_0: hipLaunchKernelGGL((dequant_chunk32_kernel<Q5_0, DT>), grid, block, 0, s, wp, op, nc); break;
        case Q5_1: hipLaunchKernelGGL((dequant_chunk32_kernel<Q5_1, DT>), grid, block, 0, s, wp, op, nc); break;
        case Q6_K: hipLaunchKernelGGL((dequant_chunk32_kernel<Q6_K, DT>), grid, block, 0, s, wp, op, nc); break;
        case Q2_K: hipLaunchKernelGGL((dequant_chunk32_kernel<Q2_K, DT>), grid, block, 0, s, wp, op, nc); break;
        case Q3_K: hipLaunchKernelGGL((dequant_chunk32_kernel<Q3_K, DT>), grid, block, 0, s, wp, op, nc); break;
        default: hipLaunchKernelGGL((dequant_chunk32_kernel<Q5_K, DT>), grid, block, 0, s, wp, op, nc); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DT>
static hipError_t launch_dequant_dt(int codec, const void* w, int64_t nblocks, void* out,
                                    hipStream_t s) {
    const int tpb = codec == Q8_0 ? 4 : codec == Q4_K ? (DT == F32 ? 64 : 32) : 16;
    const int64_t bbytes = codec == Q8_0 ? 34 : codec == Q4_K ? 144 : 28;
    const int64_t obytes = (codec == Q8_0 ? 32 : codec == Q4_K ? 256 : 128) * (DT == F32 ? 4 : 2);
    // a dispatch counts its work-items in 32 bits: matrices past 2^31 threads
    // go in pieces
    const int64_t piece = ((int64_t)1 << 31) / tpb;
    for (int64_t b0 = 0; b0 < nblocks; b0 += piece) {
        const int64_t nb = nblocks - b0 < piece ? nblocks - b0 : piece;
        const uint8_t* wp = (const uint8_t*)w + b0 * bbytes;
        void* op = (uint8_t*)out + b0 * obytes;
        const dim3 grid((unsigned)((nb * tpb + 255) / 256)), block(256);
        switch (codec) {
        case Q4_K: hipLaunchKernelGGL(dequant_q4k_kernel<DT>, grid, block, 0, s, wp, op, nb); break;
        case Q8_0: hipLaunchKernelGGL(dequant_q8_0_kernel<DT>, grid, block, 0, s, wp, op, nb); break;
        default: hipLaunchKernelGGL(dequant_tq1_kernel<DT>, grid, block, 0, s, wp, op, nb); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_dequant(int codec, const void* w, int64_t rows, int64_t k, void* out, int out_dt,
                          hipStream_t s) {
    if (codec >= Q4_0) {
        const int64_t nchunks = rows * (k / 32);
        switch (out_dt) {
        case F32: return launch_chunk32_dt<F32>(codec, w, nchunks, out, s);
        case F16: return launch_chunk32_dt<F16>(codec, w, nchunks, out, s);
        default: return launch_chunk32_dt<BF16>(codec, w, nchunks, out, s);
        }
    }
    const int qk = codec == Q4_K ? 256 : codec == Q8_0 ? 32 : 128;
    const int64_t nblocks = rows * (k / qk);
    switch (out_dt) {
    case F32: return launch_dequant_dt<F32>(codec, w, nblocks, out, s);
    case F16: return launch_dequant_dt<F16>(codec, w, nblocks, out, s);
    default: return launch_dequant_dt<BF16>(codec, w, nblocks, out, s);
    }
}

}  // namespace kq
