// moe_dec.hip -- single-token MoE layers with Q4_K experts, reading the
// expert ids directly (no routing schedule):
// - the down projection with the weighted sum over slots fused in: y[n] =
//   sum over slots r, in order, of scores[r] * (W[ids[r]] row n . x_r), for
//   kq_qmm_id with scores and one token, fp16 or fp32 activations;
// - the gate/up product with SiLU, kq_moe_glu for one token with fp16
//   activations (at the end of the file).
//
// mlx-kquant "bindings.cpp": gather_qmv_mix_ns_kq (the expert matvecs of a
// token summed with its router weights in f32) and moe_glu_gather_kq;
// mlx-native "quantized_matmul_id_ggml.rs": the expert-routed matvec and its
// slotted input layout.
//
// Down projection:
// A workgroup owns 16 output rows and walks the token's slots in order,
// streaming each slot's expert rows through LDS in chunks (double buffered,
// as in the decode GEMV).  The multiply is that of mmv3.hip for up to four
// activation rows: unscaled nibbles as fp16 subnormals, A rows (chunk,
// activation row), low-nibble, high-nibble and min accumulators, scales
// applied to the fp32 results.  fp32 activations are split per super-block
// into two fp16 rows, hi + lo, of the values scaled by a power of two that
// puts the super-block's largest magnitude in [2^14, 2^15); the two rows
// are the two activation rows of the multiply, and the power of two is
// folded into the super-block's scales.  Each slot's contribution is
// multiplied by its router weight as it is accumulated, so no slot rows are
// written: one launch replaces the routed product and the mix.  A token
// with an invalid id gets NaN outputs.
#include "kq_device.h"
#include "kq_internal.h"
#include "q4k_mfma.h"
#include "lds_dma.h"

namespace kq {

namespace {

template <int C, int W, bool XF32>
struct DownMixLayout {
    static constexpr int WPIECES = 16 * 9 * C;
    static constexpr int WBYTES = WPIECES * 16;               // weights of one chunk
    static constexpr int XBYTES = C * 256 * (XF32 ? 4 : 2);   // activations of one chunk
    static constexpr int BUF = WBYTES + XBYTES;
    static constexpr int XP_OFF = 2 * BUF;                    // per-wave hi/lo rows (fp32 only)
    static constexpr int XP_BYTES = XF32 ? 2 * 512 : 0;
    static constexpr int RED_OFF = XP_OFF + W * XP_BYTES;
    static constexpr int TOTAL = RED_OFF + (W - 1) * 64 * 4;
    static_assert(WPIECES % 64 == 0 && XBYTES % 1024 == 0, "chunks are whole 1 KB loads");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Largest value over the wave: within each row of 16 lanes by DPP moves,
// then across the four rows by reading one lane of each.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max<0xb1>(v);   // quad_perm 1,0,3,2
    v = dpp_max<0x4e>(v);   // quad_perm 2,3,0,1
    v = dpp_max<0x141>(v);  // row_half_mirror
    v = dpp_max<0x140>(v);  // row_mirror
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

}  // namespace

template <int C, int W, bool XF32>
__global__ __launch_bounds__(64 * W) void moe_down_mix1_kernel(DownMixArgs a) {
    using L = DownMixLayout<C, W, XF32>;
    constexpr int WLOADS = L::WPIECES / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int XLOADS = L::XBYTES / 1024;
    constexpr int ROWB = 9 * C * 16;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int nsb = (int)(a.k / 256);
    const int nch = (nsb + C - 1) / C;         // chunks per slot
    const int nq = (int)a.top_k * nch;         // chunks of the whole token

    // a token with an invalid expert id has NaN outputs (with a shared
    // expert, slot top_k - 1 is expert n_experts)
    bool bad = false;
    for (int r = 0; r < a.top_k; ++r)
        bad |= (int64_t)slot_expert(a.ids, r, a.top_k, a.shexp, a.n_experts) >= a.n_experts + a.shexp;
    if (bad) {
        if (tid < 16 && n0 + tid < a.n) store_val(a.y, n0 + tid, a.y_dt, __builtin_nanf(""));
        return;
    }

    uint32_t woff[WL_PER_WAVE], wq16[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int p = 64 * (wave + W * j) + lane;
        const int r = p / (9 * C), q = p - r * 9 * C;
        int64_t n = n0 + r;
        if (n >= a.n) n = a.n - 1;
        wq16[j] = 16u * (uint32_t)q;
        woff[j] = (uint32_t)((n - n0) * a.row_bytes) + wq16[j];
    }
    // chunk q: slot q / nch, super-blocks [C (q % nch), +C) of that slot
    auto issue = [&](int qc) {
        uint8_t* dst = smem + (qc & 1) * L::BUF;
        const int r = qc / nch, s0 = (qc - r * nch) * C;
        const int nsc = nsb - s0 < C ? nsb - s0 : C;
        const uint8_t* wbase = expert_base(a.w, a.w_sh, slot_expert(a.ids, r, a.top_k, a.shexp, a.n_experts),
                                           a.n_experts, a.expert_stride) +
                               n0 * a.row_bytes + (uint32_t)s0 * 144u;
        const uint32_t climit = (uint32_t)nsc * 144u;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t off = wq16[j] < climit ? woff[j] : woff[j] - wq16[j];
                dma16(wbase + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i)));
            }
        }
        const uint8_t* xrow = (const uint8_t*)a.x + (a.slotted ? (int64_t)r * a.k * (XF32 ? 4 : 2) : 0) +
                              (int64_t)s0 * 256 * (XF32 ? 4 : 2);
        const int xvalid = nsc * 256 * (XF32 ? 4 : 2);  // bytes of this chunk's activations
        for (int i = wave; i < XLOADS; i += W) {
            int off = 1024 * i + 16 * lane;
            if (off >= xvalid) off = 0;
            dma16(xrow + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + L::WBYTES + 1024 * i)));
        }
    };

    // A rows (chunk n_l / 4, activation row n_l % 4): live in lane group
    // n_l / 4, for the rows that exist (one, or hi and lo for fp32)
    const int brow = n_l & 3;
    const bool alive = (n_l >> 2) == g && brow < (XF32 ? 2 : 1);
    u32x4 AL[4], AH[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) AL[p] = AH[p] = u32x4{0u, 0u, 0u, 0u};
    const LaneSel ls = lane_sel(g);
    uint8_t* xp = smem + L::XP_OFF + wave * L::XP_BYTES;
    float acc = 0.f;

    issue(0);
    for (int qc = 0; qc < nq; ++qc) {
        wait_loads_le(0);
        __syncthreads();
        if (qc + 1 < nq) issue(qc + 1);
        const int r = qc / nch, s0 = (qc - r * nch) * C;
        const int nsc = nsb - s0 < C ? nsb - s0 : C;
        const float score = a.scores[r];
        const uint8_t* B = smem + (qc & 1) * L::BUF;
        for (int sb = wave; sb < nsc; sb += W) {
            const uint8_t* wr = B + n_l * ROWB + sb * 144;
            const u32x4 hd = *(const u32x4*)wr;
            const u32x4 q0 = *(const u32x4*)(wr + 16 + 32 * g), q1 = *(const u32x4*)(wr + 32 + 32 * g);
            const uint32_t qd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            float scale = score;
            const uint8_t* abase;
            if (XF32) {
                // split this super-block's activations: lane l holds columns
                // 4l..4l+3; the largest magnitude sets the power of two
                const float4_t v = *(const float4_t*)(B + L::WBYTES + sb * 1024 + 16 * lane);
                float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                                           __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
                mx = wave_max(mx);
                int e = 0;
                if (mx > 0.f && mx <= 3.4e38f) {
                    const int ex = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 255u) - 127;
                    e = ex - 14;
                    if (e < -126) e = -126;
                }
                const float down = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);  // 2^-e
                scale = score * __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);       // 2^e
                uint32_t hi2[2], lo2[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float a0 = v[2 * i] * down, a1 = v[2 * i + 1] * down;
                    const uint32_t h0 = float_to_half_bits(a0), h1 = float_to_half_bits(a1);
                    hi2[i] = h0 | (h1 << 16);
                    lo2[i] = float_to_half_bits(a0 - half_bits_to_float(h0)) |
                             (float_to_half_bits(a1 - half_bits_to_float(h1)) << 16);
                }
                *(u32x2*)(xp + 8 * lane) = u32x2{hi2[0], hi2[1]};
                *(u32x2*)(xp + 512 + 8 * lane) = u32x2{lo2[0], lo2[1]};
                abase = xp + brow * 512 + 128 * g;
            } else {
                abase = B + L::WBYTES + sb * 512 + 128 * g;
            }
            if (alive) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    AL[p] = *(const u32x4*)(abase + 16 * p);
                    AH[p] = *(const u32x4*)(abase + 64 + 16 * p);
                }
            }
            uint32_t sc_lo, sc_hi, m_lo, m_hi;
            q4k_scales_all(hd, sc_lo, sc_hi, m_lo, m_hi);
            const uint32_t scw = ls.high ? sc_hi : sc_lo, mw = ls.high ? m_hi : m_lo;
            const uint32_t sc_u = __builtin_amdgcn_perm(scw, scw, ls.sel);
            const uint32_t m_u = __builtin_amdgcn_perm(mw, mw, ls.sel);
            const half2_t m_h = __builtin_bit_cast(half2_t, m_u | 0x64006400u) -
                                half2_t{(half_t)1024.0f, (half_t)1024.0f};
            const uint32_t m0 = __builtin_bit_cast(uint32_t, half2_t{m_h[0], m_h[0]});
            const uint32_t m1 = __builtin_bit_cast(uint32_t, half2_t{m_h[1], m_h[1]});
            float4_t dl = {0.f, 0.f, 0.f, 0.f}, dh = {0.f, 0.f, 0.f, 0.f}, dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t qa = qd[2 * p], qb = qd[2 * p + 1];
                const uint32_t a01 = __builtin_amdgcn_perm(qa, qa, 0x0c010c00u), a23 = __builtin_amdgcn_perm(qa, qa, 0x0c030c02u);
                const uint32_t b01 = __builtin_amdgcn_perm(qb, qb, 0x0c010c00u), b23 = __builtin_amdgcn_perm(qb, qb, 0x0c030c02u);
                dl = mfma16(AL[p], u32x4{a01 & 0x000f000fu, a23 & 0x000f000fu, b01 & 0x000f000fu, b23 & 0x000f000fu}, dl);
                dh = mfma16(AH[p], u32x4{a01 & 0x00f000f0u, a23 & 0x00f000f0u, b01 & 0x00f000f0u, b23 & 0x00f000f0u}, dh);
                dm = mfma16(AL[p], u32x4{m0, m0, m0, m0}, dm);
                dm = mfma16(AH[p], u32x4{m1, m1, m1, m1}, dm);
            }
            const float d = q4k_d(hd), dmin = q4k_dmin(hd);
            const float s0 = d * 16777216.0f * (float)(sc_u & 0xffu);
            const float s1 = d * 1048576.0f * (float)((sc_u >> 16) & 0xffu);
            // output rows 4g and 4g+1: this chunk's sub-blocks 2g, 2g+1 for
            // activation rows 0 and 1 (hi and lo; row 1 is zero for fp16)
            const float t = (s0 * (dl[0] + dl[1]) + s1 * (dh[0] + dh[1])) - dmin * (dm[0] + dm[1]);
            acc = __builtin_fmaf(scale, t, acc);
        }
    }
    __syncthreads();

    float* red = (float*)(smem + L::RED_OFF);
    if (W > 1) {
        if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) acc += red[(w - 1) * 64 + lane];
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    const int64_t n = n0 + n_l;
    if (g == 0 && n < a.n) store_val(a.y, n, a.y_dt, acc);
}

// ---------------------------------------------------------------------------
// Single-token gate/up with SiLU (kq_moe_glu, one token, fp16 activations):
// grid row y is slot y, whose expert id is read directly.  A workgroup owns
// the same 16 rows of the expert's gate and up matrices, so every staged
// activation feeds both; the multiply is the one above with one activation
// row, and h = silu(gate) * up is formed before the single store.
template <int C, int W>
__global__ __launch_bounds__(64 * W) void moe_glu1_kernel(SkinnyArgs a) {
    constexpr int WPIECES = 2 * 16 * 9 * C;        // gate rows, then up rows
    constexpr int WBYTES = WPIECES * 16;
    constexpr int XBYTES = C * 512;
    constexpr int BUF = WBYTES + XBYTES;
    constexpr int RED_OFF = 2 * BUF;
    static_assert(WPIECES % 64 == 0 && XBYTES % 1024 == 0, "chunks are whole 1 KB loads");
    constexpr int WLOADS = WPIECES / 64;
    constexpr int WL_PER_WAVE = (WLOADS + W - 1) / W;
    constexpr int XLOADS = XBYTES / 1024;
    constexpr int ROWB = 9 * C * 16;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t slot = blockIdx.y;
    const int nsb = (int)(a.k / 256);
    const int nchunks = (nsb + C - 1) / C;

    const uint32_t e = slot_expert(a.ids, slot, a.top_k, a.shexp, a.n_experts);
    if ((int64_t)e >= a.n_experts + a.shexp) {
        if (tid < 16 && n0 + tid < a.n) store_val(a.y, slot * a.y_row + n0 + tid, a.y_dt, __builtin_nanf(""));
        return;
    }
    const uint8_t* wb[2] = {expert_base(a.w, a.w_sh, e, a.n_experts, a.expert_stride) + n0 * a.row_bytes,
                            expert_base(a.w2, a.w2_sh, e, a.n_experts, a.expert_stride) + n0 * a.row_bytes};
    uint32_t woff[WL_PER_WAVE], wq16[WL_PER_WAVE];
    int wset[WL_PER_WAVE];
#pragma unroll
    for (int j = 0; j < WL_PER_WAVE; ++j) {
        const int p = 64 * (wave + W * j) + lane;
        const int st = p / (16 * 9 * C), rem = p - st * 16 * 9 * C;
        const int r = rem / (9 * C), q = rem - r * 9 * C;
        int64_t n = n0 + r;
        if (n >= a.n) n = a.n - 1;
        wset[j] = st < 2 ? st : 0;
        wq16[j] = 16u * (uint32_t)q;
        woff[j] = (uint32_t)((n - n0) * a.row_bytes) + wq16[j];
    }
    const uint8_t* xrow = (const uint8_t*)a.x;
    auto issue = [&](int chunk) {
        uint8_t* dst = smem + (chunk & 1) * BUF;
        const int s0 = chunk * C;
        const int nsc = nsb - s0 < C ? nsb - s0 : C;
        const uint32_t cbase = (uint32_t)s0 * 144u;
        const uint32_t climit = (uint32_t)nsc * 144u;
#pragma unroll
        for (int j = 0; j < WL_PER_WAVE; ++j) {
            const int i = wave + W * j;
            if (i < WLOADS) {
                const uint32_t off = wq16[j] < climit ? woff[j] : woff[j] - wq16[j];
                dma16(wb[wset[j]] + cbase + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * i)));
            }
        }
        const int xvalid = nsc * 512;
        for (int i = wave; i < XLOADS; i += W) {
            int off = 1024 * i + 16 * lane;
            if (off >= xvalid) off = 0;
            dma16(xrow + (int64_t)s0 * 512 + off, __builtin_amdgcn_readfirstlane(lds_addr(dst + WBYTES + 1024 * i)));
        }
    };

    const bool alive = (n_l >> 2) == g && (n_l & 3) == 0;
    u32x4 AL[4], AH[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) AL[p] = AH[p] = u32x4{0u, 0u, 0u, 0u};
    const LaneSel ls = lane_sel(g);
    float acc[2] = {0.f, 0.f};

    issue(0);
    for (int c = 0; c < nchunks; ++c) {
        wait_loads_le(0);
        __syncthreads();
        if (c + 1 < nchunks) issue(c + 1);
        const uint8_t* B = smem + (c & 1) * BUF;
        const int nsc = nsb - c * C < C ? nsb - c * C : C;
        for (int sb = wave; sb < nsc; sb += W) {
            if (alive) {
                const uint8_t* ap = B + WBYTES + sb * 512 + 128 * g;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    AL[p] = *(const u32x4*)(ap + 16 * p);
                    AH[p] = *(const u32x4*)(ap + 64 + 16 * p);
                }
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const uint8_t* wr = B + (st * 16 + n_l) * ROWB + sb * 144;
                const u32x4 hd = *(const u32x4*)wr;
                const u32x4 q0 = *(const u32x4*)(wr + 16 + 32 * g), q1 = *(const u32x4*)(wr + 32 + 32 * g);
                const uint32_t qd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                uint32_t sc_lo, sc_hi, m_lo, m_hi;
                q4k_scales_all(hd, sc_lo, sc_hi, m_lo, m_hi);
                const uint32_t scw = ls.high ? sc_hi : sc_lo, mw = ls.high ? m_hi : m_lo;
                const uint32_t sc_u = __builtin_amdgcn_perm(scw, scw, ls.sel);
                const uint32_t m_u = __builtin_amdgcn_perm(mw, mw, ls.sel);
                const half2_t m_h = __builtin_bit_cast(half2_t, m_u | 0x64006400u) -
                                    half2_t{(half_t)1024.0f, (half_t)1024.0f};
                const uint32_t m0 = __builtin_bit_cast(uint32_t, half2_t{m_h[0], m_h[0]});
                const uint32_t m1 = __builtin_bit_cast(uint32_t, half2_t{m_h[1], m_h[1]});
                float4_t dl = {0.f, 0.f, 0.f, 0.f}, dh = {0.f, 0.f, 0.f, 0.f}, dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t qa = qd[2 * p], qb = qd[2 * p + 1];
                    const uint32_t a01 = __builtin_amdgcn_perm(qa, qa, 0x0c010c00u), a23 = __builtin_amdgcn_perm(qa, qa, 0x0c030c02u);
                    const uint32_t b01 = __builtin_amdgcn_perm(qb, qb, 0x0c010c00u), b23 = __builtin_amdgcn_perm(qb, qb, 0x0c030c02u);
                    dl = mfma16(AL[p], u32x4{a01 & 0x000f000fu, a23 & 0x000f000fu, b01 & 0x000f000fu, b23 & 0x000f000fu}, dl);
                    dh = mfma16(AH[p], u32x4{a01 & 0x00f000f0u, a23 & 0x00f000f0u, b01 & 0x00f000f0u, b23 & 0x00f000f0u}, dh);
                    dm = mfma16(AL[p], u32x4{m0, m0, m0, m0}, dm);
                    dm = mfma16(AH[p], u32x4{m1, m1, m1, m1}, dm);
                }
                const float d = q4k_d(hd), dmin = q4k_dmin(hd);
                const float s0 = d * 16777216.0f * (float)(sc_u & 0xffu);
                const float s1 = d * 1048576.0f * (float)((sc_u >> 16) & 0xffu);
                acc[st] += (s0 * dl[0] + s1 * dh[0]) - dmin * dm[0];
            }
        }
    }
    __syncthreads();

    float* red = (float*)(smem + RED_OFF);
    if (W > 1) {
        if (wave > 0) {
            red[((wave - 1) * 2 + 0) * 64 + lane] = acc[0];
            red[((wave - 1) * 2 + 1) * 64 + lane] = acc[1];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            acc[0] += red[((w - 1) * 2 + 0) * 64 + lane];
            acc[1] += red[((w - 1) * 2 + 1) * 64 + lane];
        }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        acc[st] += __shfl_xor(acc[st], 16);
        acc[st] += __shfl_xor(acc[st], 32);
    }
    const int64_t n = n0 + n_l;
    if (g == 0 && n < a.n) store_val(a.y, slot * a.y_row + n, a.y_dt, glu_act(a.act, acc[0], acc[1], a.limit));
}

template <int C, int W>
static void launch_glu1(const SkinnyArgs& a, hipStream_t s) {
    constexpr size_t lds = 2 * (2 * 16 * 9 * C * 16 + C * 512) + (W - 1) * 2 * 64 * 4;
    const dim3 grid((unsigned)((a.n + 15) / 16), (unsigned)a.top_k);
    hipLaunchKernelGGL((moe_glu1_kernel<C, W>), grid, dim3(64 * W), lds, s, a);
}

hipError_t launch_moe_glu1(const SkinnyArgs& a, hipStream_t s) {
    launch_glu1<2, 2>(a, s);
    return hipGetLastError();
}

template <int C, int W, bool XF32>
static void launch_dm(const DownMixArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.n + 15) / 16));
    constexpr size_t lds = DownMixLayout<C, W, XF32>::TOTAL;
    hipLaunchKernelGGL((moe_down_mix1_kernel<C, W, XF32>), grid, dim3(64 * W), lds, s, a);
}

hipError_t launch_down_mix1(const DownMixArgs& a, bool x_f32, hipStream_t s) {
    if (x_f32) launch_dm<8, 8, true>(a, s);
    else launch_dm<8, 8, false>(a, s);
    return hipGetLastError();
}

}  // namespace kq
