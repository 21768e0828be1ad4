// kq_internal.h -- host-side declarations shared by the libkq translation
// units (launchers behind the C ABI).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// Rows of a weight-streaming tile: one pass over a weight row serves up to
// this many activation rows.
constexpr int kMoeTileRows = 32;

// Layout of the MoE workspace (int32 words); see include/kq.h.
struct MoeLayout {
    int64_t n_experts, rows, max_tiles;
    int64_t counts_off, offsets_off, perm_off, tiles_off;  // word offsets
    int64_t xexp_off;        // word offset of the per-activation-row scale exponents
    int64_t route_words;     // words used by the schedule
    int64_t slot_off_bytes;  // start of the fp32 slot buffer
    int64_t slot_bytes;      // rows * n_out * 4
    int64_t total_bytes;
};
MoeLayout moe_layout(int64_t n_experts, int64_t n_tokens, int64_t top_k, int64_t n_out);

// Arguments of the weight-streaming ("skinny") product kernels.
struct SkinnyArgs {
    const uint8_t* w;      // weights (gate for GLU)
    const uint8_t* w2;     // up weights (GLU only)
    int64_t row_bytes;     // bytes per weight row
    int64_t expert_stride; // bytes between experts
    int64_t n, k;          // weight rows, columns
    const void* x;         // activations
    int64_t x_row;         // elements between consecutive activation rows
    int64_t top_k;         // routed: slots per token
    int shared_x;          // routed: x row = r / top_k (else r)
    int one_x_row;         // routed: all rows read one activation row (one token, shared x)
    const int32_t* ws;     // routed: workspace (schedule); null for dense
    // single-token gate/up without a schedule: grid row y is slot y, whose
    // expert is ids[y] (an id >= n_experts poisons the slot's output)
    const uint32_t* ids;
    int64_t n_experts;
    int64_t tiles_off, perm_off;
    int64_t xexp_off;      // routed, fp32 activations: word offset of row exponents
    int xexp_local;        // ... or found by each workgroup for its own rows
    int64_t m;             // dense: activation rows
    void* y;               // output
    int y_dt;              // output dtype
    int64_t y_row;         // elements between output rows
    int64_t rows_cap;      // routed: most rows any schedule tile can hold
    int act;               // GLU: KQ_ACT_SILU or KQ_ACT_GELU_TANH
    // set by the launchers of the matrix-core kernels
    int xch;               // super-blocks of activations staged per chunk
    int xstride;           // elements (or bytes) between staged activation rows
    int red_off;           // byte offset of a second LDS region
};

// Single-token MoE down projection with the slot mix fused in (moe_dec.hip).
struct DownMixArgs {
    const uint8_t* w;       // experts' weights
    int64_t expert_stride;  // bytes between experts
    int64_t row_bytes;
    int64_t n, k;
    const void* x;          // activations: [k] (shared) or [top_k, k] (slotted)
    int slotted;
    const uint32_t* ids;    // [top_k]
    const float* scores;    // [top_k]
    int64_t n_experts, top_k;
    void* y;                // [n]
    int y_dt;
};
hipError_t launch_down_mix1(const DownMixArgs& a, bool x_f32, hipStream_t s);
// Single-token gate/up with SiLU, expert ids read directly (moe_dec.hip).
hipError_t launch_moe_glu1(const SkinnyArgs& a, hipStream_t s);

hipError_t launch_dequant(int codec, const void* w, int64_t rows, int64_t k, void* out, int out_dt,
                          hipStream_t s);
hipError_t launch_skinny(int codec, int x_dt, bool glu, const SkinnyArgs& a, int64_t grid_tiles,
                         hipStream_t s);
hipError_t launch_mmv2_q4k(bool glu, const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s);
bool mmv3_fits(int64_t k);
hipError_t launch_mmv3_q4k(const SkinnyArgs& a, hipStream_t s);
hipError_t launch_mmv3m_q4k(const SkinnyArgs& a, hipStream_t s);
hipError_t launch_moe_mm(bool glu, int x_dt, const SkinnyArgs& a, int64_t grid_tiles,
                         hipStream_t s);
hipError_t launch_row_exp(const float* x, int64_t rows, int64_t k, int32_t* e, hipStream_t s);
bool tq1_mv_fits(int64_t k);
hipError_t launch_tq1_mv(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y,
                         int y_dt, hipStream_t s);
hipError_t launch_gemm(int codec, int x_dt, const void* w, int64_t n, int64_t k, const void* x,
                       int64_t m, void* y, int y_dt, hipStream_t s);
// Builds the schedule; with poison_y, also writes NaN to the rows of
// poison_y ([rows, poison_n] of poison_dt) whose id is invalid.
hipError_t launch_route(const uint32_t* ids, int64_t rows, int64_t n_experts, const MoeLayout& L,
                        int32_t* ws, hipStream_t s, void* poison_y = nullptr,
                        int64_t poison_n = 0, int poison_dt = 0);
hipError_t launch_mix(const uint32_t* ids, const float* scores, int64_t n_tokens, int64_t top_k,
                      int64_t n_experts, const float* slots, int64_t n, void* y, int y_dt,
                      hipStream_t s);


}  // namespace kq
