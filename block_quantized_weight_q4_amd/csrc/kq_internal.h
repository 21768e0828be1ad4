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
    int act;               // GLU: KQ_ACT_SILU, KQ_ACT_GELU_TANH or KQ_ACT_SILU_LIMIT
    float limit;           // GLU: the bound of KQ_ACT_SILU_LIMIT
    // shared expert: the last of top_k slots per token is expert n_experts,
    // whose matrices are w_sh (and w2_sh for the GLU's up projection)
    int shexp;
    const uint8_t* w_sh;
    const uint8_t* w2_sh;
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
    int shexp;              // the last of top_k slots is the shared expert w_sh
    const uint8_t* w_sh;
    const int32_t* xexp;    // x split by split_rows_kernel: each row's exponent (else null)
};
hipError_t launch_down_mix1(const DownMixArgs& a, bool x_f32, hipStream_t s);
// ... and for Q8_0 and the further GGUF codecs (cmv.hip): the down projection
// with the mix (fp16 or fp32 activations) and the gate/up form (fp16), where
// k is a whole number of the kernels' chunks and their buffers fit in LDS
// (mode 0: fp16 x; 1: fp32 x split beforehand by launch_split_rows; 2: fp32
// x split inside the kernel)
bool down1_fits(int codec, int64_t k, int64_t S, int mode);
hipError_t launch_down1_gguf(int codec, const DownMixArgs& d, int mode, hipStream_t s);
// fp32 rows -> per row: the exponent e (largest magnitude x 2^-e in
// [2^14, 2^15)) and every 16 values as 16 fp16 hi then 16 fp16 lo parts of
// x 2^-e (64 bytes)
hipError_t launch_split_rows(const float* x, int64_t rows, int64_t k, uint8_t* out, int32_t* xexp, hipStream_t s);
bool glu1_fits(int codec, int64_t k);
hipError_t launch_glu1_gguf(int codec, const SkinnyArgs& a, hipStream_t s);
// ... and their routed products over schedule tiles on the matrix cores
// (cmv.hip); fp32 activations need the row exponents of launch_row_exp
bool crm_fits(int codec, int64_t k, bool glu, bool xf32);
hipError_t launch_crm(int codec, bool glu, bool xf32, const SkinnyArgs& a, int64_t grid_tiles, hipStream_t s);
// Single-token gate/up with SiLU, expert ids read directly (moe_dec.hip).
hipError_t launch_moe_glu1(const SkinnyArgs& a, hipStream_t s);

// Encoders and the TQ1 legality scan (quantize.hip).
hipError_t launch_quantize(int codec, const void* w, int w_dt, int64_t rows, int64_t k,
                           const float* imatrix, void* out, hipStream_t s);
hipError_t launch_tq1_illegal(const void* w, int64_t rows, int64_t k, unsigned long long* count,
                              hipStream_t s);
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
// pieces of K for the TQ1 GEMV of n rows (1: no split); *pnb = blocks per piece
int tq1_mv_pieces(int64_t n, int64_t k, int* pnb);
// pnb > 0: K in pieces of pnb blocks, fp32 partials to part [pieces][n]
hipError_t launch_tq1_mv(const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y,
                         int y_dt, hipStream_t s, int pnb = 0, float* part = nullptr);
// y[i] = sum over pieces p in order of part[p * count + i], stored as y_dt
// decode GEMV of one fp16 activation row for the further GGUF codecs
// (cmv.hip): rows a whole number of its chunks long, LDS permitting
bool cmv_fits(int codec, int64_t k);
hipError_t launch_cmv(int codec, const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, void* y,
                      int y_dt, hipStream_t s);
// ... and of 2..16 fp16 activation rows on the matrix cores (passes of 8 rows)
bool cmm_fits(int codec, int64_t k, int64_t m);
hipError_t launch_cmm(int codec, const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int64_t m, void* y,
                      int y_dt, hipStream_t s);
hipError_t launch_splitk_reduce(const float* part, int pieces, int64_t count, void* y, int y_dt,
                                hipStream_t s);
// Prefill GEMM (gemm.hip).
struct GemmArgs {
    const uint8_t* w;
    int64_t n, k, m;
    const uint16_t* x;      // activations the matrix cores read (fp16 or bf16)
    const uint16_t* x_src;  // the caller's activations (exact path)
    int x_src_dt;           // F16 or BF16
    const int32_t* xexp;    // pre-scaled fp16 rows: exponent per row
    void* y;
    int y_dt;
    float* part;            // split K: fp32 partial sums [splits][m][n], else null
    int split_steps;        // K steps (of 64) per split
};
struct GemmPlan {
    int bm, bn, splits, split_steps;
    int64_t tiles;
};
// Caller-owned scratch of kq_qmm_ws (byte offsets, 256-aligned).
struct GemmWorkspace {
    int64_t xexp_off, x16_off, part_off, bytes;
};
GemmPlan gemm_plan(int codec, int64_t n, int64_t k, int64_t m, bool may_split);
GemmWorkspace gemm_workspace(int codec, int64_t n, int64_t k, int64_t m, int x_dt);
// ws null: no workspace (bf16 rows are scaled inside each workgroup, no
// split); else the layout of gemm_workspace.
hipError_t launch_gemm(int codec, int x_dt, const void* w, int64_t n, int64_t k, const void* x,
                       int64_t m, void* y, int y_dt, void* ws, hipStream_t s);
// Builds the schedule; with poison_y, also writes NaN to the poisoned rows
// of poison_y ([rows, poison_n] of poison_dt).
// Rows of poison_y are NaN-ed by the routing rule: below 32 tokens those with
// an id >= n_experts, from 32 tokens on all of them if any id is out of range
// or repeated within a token (then the schedule has no tiles).
// With shexp, rows counts top_k slots per token of which the last is the
// shared expert (routed ids: top_k - 1 per token) and n_experts counts it.
hipError_t launch_route(const uint32_t* ids, int64_t rows, int64_t top_k, int64_t n_experts,
                        const MoeLayout& L, int32_t* ws, hipStream_t s, void* poison_y = nullptr,
                        int64_t poison_n = 0, int poison_dt = 0, int shexp = 0);
hipError_t launch_mix(const uint32_t* ids, const float* scores, int64_t n_tokens, int64_t top_k,
                      int64_t n_experts, const int32_t* ws, const float* slots, int64_t n,
                      void* y, int y_dt, hipStream_t s, int shexp = 0);


}  // namespace kq
