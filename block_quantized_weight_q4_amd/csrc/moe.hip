// moe.hip -- expert routing schedule (with NaN rows for invalid ids) and slot-order mixing.
//
// mlx-kquant "bindings.cpp": expert_tile_map (fixed-size row tiles per expert segment,
// only the last partial, built on the GPU with no host sync),
// gather_qmv_mix_ns_kq (each slot accumulated in f32 weighted by its score);
// mlx-native "quantized_matmul_id_ggml.rs": map0 regroup with on-device id
// validation, NaN poison for invalid routing metadata.
#include "kq_device.h"
#include "kq_internal.h"

namespace kq {

// Invalid routing metadata (mlx-native "quantized_matmul_id_ggml.rs", the
// id contract of quantized_matmul_id_ggml and the map0 comment of its
// matrix-matrix dispatch): below kMmIdMinTokens tokens (the matrix-vector
// rule) an id >= E poisons the rows it touches; from kMmIdMinTokens tokens on
// (the matrix-matrix rule) an out-of-range id or an id repeated within a
// token poisons the entire output and the schedule gets no tiles, so no
// weight is read.
constexpr int64_t kMmIdMinTokens = 32;

// One workgroup of 256 threads builds the whole schedule:
//   1. histogram of ids into LDS counts (ids >= E counted as invalid)
//   2. exclusive scans: row offsets per expert and tile offsets per expert
//   3. stable scatter by one wave, 64 rows at a time in row order: each lane
//      finds the lanes holding the same expert with ballots over the id bits,
//      its rank among them, and the lowest such lane advances the cursor
//   4. tile descriptors (expert, row_start, num_rows) in expert order
//   5. matrix-matrix rule: a repeated id within a token shows up as two
//      neighbours of one expert's segment of the (stable) permutation that
//      belong to the same token; any defect then empties the tile list
//   6. (when an output is given) the poisoned rows -- those with an id >= E,
//      or every row under the matrix-matrix rule -- are written as NaN in that
//      output; the products never touch them
__global__ __launch_bounds__(256) void route_kernel(const uint32_t* __restrict__ ids, int64_t rows,
                                                    int64_t top_k, int64_t n_experts,
                                                    int32_t* __restrict__ ws,
                                                    int64_t counts_off, int64_t offsets_off,
                                                    int64_t perm_off, int64_t tiles_off,
                                                    int id_bits, void* __restrict__ poison_y,
                                                    int64_t poison_n, int poison_dt, int shexp) {
    extern __shared__ int32_t lds[];
    int32_t* counts = lds;                  // [E]
    int32_t* cursor = lds + n_experts;      // [E]
    int32_t* tstart = lds + 2 * n_experts;  // [E]
    __shared__ int32_t n_invalid, n_tiles, n_repeat;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool mm_rule = rows / top_k >= kMmIdMinTokens;
    // expert of routed row i: with a shared expert it is the last slot of
    // each token (expert n_experts - 1), the ids hold the others
    const int64_t real_e = n_experts - shexp;
    auto expert_of = [&](int64_t i) { return slot_expert(ids, i, top_k, shexp, real_e); };

    for (int64_t e = tid; e < n_experts; e += 256) counts[e] = 0;
    if (tid == 0) n_invalid = 0, n_repeat = 0;
    __syncthreads();
    for (int64_t i = tid; i < rows; i += 256) {
        const uint32_t e = expert_of(i);
        if ((int64_t)e < n_experts) atomicAdd(&counts[e], 1);
        else atomicAdd(&n_invalid, 1);
    }
    __syncthreads();

    // exclusive scans over experts, by wave 0
    if (wave == 0) {
        int32_t run_rows = 0, run_tiles = 0;
        for (int64_t base = 0; base < n_experts; base += 64) {
            const int64_t e = base + lane;
            const int32_t c = e < n_experts ? counts[e] : 0;
            const int32_t t = (c + kMoeTileRows - 1) / kMoeTileRows;
            int32_t ic = c, it = t;  // inclusive prefix within the 64
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int32_t uc = __shfl_up(ic, off, 64), ut = __shfl_up(it, off, 64);
                if (lane >= off) ic += uc, it += ut;
            }
            if (e < n_experts) {
                cursor[e] = run_rows + ic - c;
                tstart[e] = run_tiles + it - t;
            }
            run_rows += __shfl(ic, 63, 64);
            run_tiles += __shfl(it, 63, 64);
        }
        if (lane == 0) n_tiles = run_tiles;
    }
    __syncthreads();

    for (int64_t e = tid; e < n_experts; e += 256) {
        ws[counts_off + e] = counts[e];
        ws[offsets_off + e] = cursor[e];
    }
    if (tid == 0) ws[offsets_off + n_experts] = (int32_t)(rows - n_invalid);
    // tile descriptors
    for (int64_t e = tid; e < n_experts; e += 256) {
        const int32_t c = counts[e], start = cursor[e];
        int32_t t = tstart[e];
        for (int32_t r0 = 0; r0 < c; r0 += kMoeTileRows, ++t) {
            int32_t* d = ws + tiles_off + 3 * (int64_t)t;
            d[0] = (int32_t)e;
            d[1] = start + r0;
            d[2] = c - r0 < kMoeTileRows ? c - r0 : kMoeTileRows;
        }
    }
    __syncthreads();  // cursor[] is reused below after the reads above

    if (wave == 0) {
        for (int64_t base = 0; base < rows; base += 64) {
            const int64_t i = base + lane;
            const uint32_t e = i < rows ? expert_of(i) : 0xffffffffu;
            const bool valid = (int64_t)e < n_experts;
            uint64_t same = __ballot(valid);
            for (int b = 0; b < id_bits; ++b) {
                const bool bit = (e >> b) & 1u;
                const uint64_t bal = __ballot(bit);
                same &= bit ? bal : ~bal;
            }
            if (valid) {
                const uint64_t below = same & ((1ull << lane) - 1ull);
                const int32_t pos = cursor[e] + __popcll(below);
                ws[perm_off + pos] = (int32_t)i;
            }
            __builtin_amdgcn_wave_barrier();
            if (valid && (same & ((1ull << lane) - 1ull)) == 0ull)  // lowest lane of its expert
                cursor[e] += __popcll(same);
            __builtin_amdgcn_wave_barrier();
        }
    }

    if (mm_rule) {
        // the scatter's global writes of perm are visible to the whole
        // workgroup after the barrier
        __syncthreads();
        const int64_t valid = rows - n_invalid;
        int32_t rep = 0;
        for (int64_t p = tid; p + 1 < valid; p += 256) {
            const int32_t a = ws[perm_off + p], b = ws[perm_off + p + 1];
            rep += expert_of(a) == expert_of(b) && a / top_k == b / top_k;
        }
        if (rep) atomicAdd(&n_repeat, rep);
    }
    __syncthreads();
    const bool poison_all = mm_rule && n_invalid + n_repeat > 0;
    if (tid == 0) {
        ws[0] = poison_all ? 0 : n_tiles;
        ws[1] = n_invalid + n_repeat;
    }
    if (poison_y && n_invalid + n_repeat > 0) {
        const float v = __builtin_nanf("");
        for (int64_t i = 0; i < rows; ++i) {
            if (!poison_all && (int64_t)expert_of(i) < n_experts) continue;
            for (int64_t j = tid; j < poison_n; j += 256) {
                if (poison_dt == F32) store_out<F32>(poison_y, i * poison_n + j, v);
                else if (poison_dt == F16) store_out<F16>(poison_y, i * poison_n + j, v);
                else store_out<BF16>(poison_y, i * poison_n + j, v);
            }
        }
    }
}

hipError_t launch_route(const uint32_t* ids, int64_t rows, int64_t top_k, int64_t n_experts,
                        const MoeLayout& L, int32_t* ws, hipStream_t s, void* poison_y,
                        int64_t poison_n, int poison_dt, int shexp) {
    int bits = 1;
    while ((1ll << bits) < n_experts) ++bits;
    const size_t lds = (size_t)3 * n_experts * sizeof(int32_t);
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(256), lds, s, ids, rows, top_k, n_experts, ws,
                       L.counts_off, L.offsets_off, L.perm_off, L.tiles_off, bits, poison_y,
                       poison_n, poison_dt, shexp);
    return hipGetLastError();
}

// y[t, j] = sum over slots r = 0..top_k-1, in order, of scores[t,r] * slot[t*top_k+r, j]
// in fp32.  Poison: below kMmIdMinTokens tokens, NaN for a token with an id
// >= E; from kMmIdMinTokens tokens on, NaN everywhere when the schedule
// counted any defect (*n_defects, word 1 of the workspace).  Tokens are
// walked with a grid-sized stride, so any token count fits the grid.
__global__ __launch_bounds__(256) void mix_kernel(const uint32_t* __restrict__ ids,
                                                  const float* __restrict__ scores,
                                                  int64_t n_tokens, int64_t top_k,
                                                  int64_t n_experts, const int32_t* __restrict__ n_defects,
                                                  const float* __restrict__ slots,
                                                  int64_t n, void* __restrict__ y, int y_dt,
                                                  int shexp) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    const bool all_bad = n_tokens >= kMmIdMinTokens && *n_defects > 0;
    for (int64_t t = blockIdx.y; t < n_tokens; t += gridDim.y) {
        float acc = 0.f;
        bool bad = all_bad;
        for (int64_t r = 0; r < top_k; ++r) {
            const int64_t row = t * top_k + r;
            bad |= (int64_t)slot_expert(ids, row, top_k, shexp, n_experts - shexp) >= n_experts;
            acc = __builtin_fmaf(scores[row], slots[row * n + j], acc);
        }
        const float v = bad ? __builtin_nanf("") : acc;
        if (y_dt == F32) store_out<F32>(y, t * n + j, v);
        else if (y_dt == F16) store_out<F16>(y, t * n + j, v);
        else store_out<BF16>(y, t * n + j, v);
    }
}

hipError_t launch_mix(const uint32_t* ids, const float* scores, int64_t n_tokens, int64_t top_k,
                      int64_t n_experts, const int32_t* ws, const float* slots, int64_t n,
                      void* y, int y_dt, hipStream_t s, int shexp) {
    const int64_t gy = n_tokens < 65535 ? n_tokens : 65535;
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)gy);
    hipLaunchKernelGGL(mix_kernel, grid, dim3(256), 0, s, ids, scores, n_tokens, top_k, n_experts,
                       ws + 1, slots, n, y, y_dt, shexp);
    return hipGetLastError();
}

}  // namespace kq
