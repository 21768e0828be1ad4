/*
 * kq.h -- C ABI of libkq: products against block-quantized weights on
 * AMD Instinct MI355X (gfx950).
 *
 * Every entry point takes plain pointers and sizes.  Unless stated otherwise
 * a pointer argument is DEVICE memory owned by the caller; the library never
 * allocates, frees or retains memory and never synchronizes the host.  All
 * work is enqueued on `stream` (a hipStream_t; NULL is the default stream) in
 * submission order, so consecutive calls on one stream need no extra
 * synchronization.  Arguments are validated completely before anything is
 * launched; on any error nothing is enqueued.
 *
 * Weight formats (row-major: row n holds k / QK consecutive blocks, and the
 * row stride is (k / QK) * block_bytes with no padding):
 *
 *   KQ_Q4_K      256 weights in 144 bytes: fp16 d, fp16 dmin, 12 bytes of
 *                packed 6-bit sub-block scales and mins, 128 bytes of 4-bit
 *                quants; w = d * sc_j * q - dmin * m_j.  The GGUF K-quant
 *                super-block that mlx-kquant "bindings.cpp" (dequantize,
 *                quantized_matmul: codec "q4_k") and mlx-native
 *                "quantized_matmul_id_ggml.rs" (GgmlType::Q4_K) operate on.
 *   KQ_Q8_0      32 weights in 34 bytes: fp16 d then 32 int8 quants;
 *                w = d * q.  ds4 "ds4_metal.m", struct block_q8_0 and the
 *                Q8_0 matvec arguments (row bytes (k / 32) * 34).
 *   KQ_TQ1_G128  128 weights in 28 bytes: 25 code bytes of five base-3
 *                digits each (place values 1, 3, 9, 27, 81), one tail byte of
 *                three digits, fp16 scale s; w = (digit - 1) * s.  Ternary
 *                Bonsai "ternel_packed_model.py", format constants, LUT23
 *                section and get_rows kernel.  Code bytes above 242 (tail
 *                above 26) are not valid input; legality is checked when
 *                weights are produced, not by these kernels.
 *
 * All multi-byte fields are little-endian.  fp16 is IEEE binary16; bf16 is
 * the upper half of an IEEE binary32.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kq_type { KQ_Q4_K = 0, KQ_Q8_0 = 1, KQ_TQ1_G128 = 2 } kq_type;

typedef enum kq_dtype { KQ_F32 = 0, KQ_F16 = 1, KQ_BF16 = 2 } kq_dtype;

typedef enum kq_status {
    KQ_OK = 0,
    KQ_ERR_INVALID_ARG = 1, /* bad size, null/misaligned pointer, overlap, k % QK */
    KQ_ERR_UNSUPPORTED = 2, /* a (type, dtype) combination that is not built */
    KQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    KQ_ERR_DEVICE = 4       /* the HIP runtime reported an error at launch */
} kq_status;

/* x layouts of kq_qmm_id: one activation row per token, shared by its
 * top_k slots ([T, k]), or one row per (token, slot) ([T, top_k, k]).
 * mlx-native "quantized_matmul_id_ggml.rs", IdMmInputLayout.
 *
 * KQ_REUSE_SCHEDULE, OR-ed into the layout of a kq_qmm_id call with scores,
 * skips building the routing schedule: the workspace must then hold the
 * schedule that the previous kq_moe_glu, kq_qmm_id or kq_moe_route call on
 * the same stream built from the same ids, n_tokens, top_k and n_experts,
 * unmodified since (the gate/up -> down sequence of one MoE layer).
 * mlx-native "quantized_matmul_id_ggml.rs", the scratch reused across the
 * expert dispatches of a layer.  Ignored when scores is NULL: that form's
 * rows with an invalid id are written while the schedule is built.  Also
 * ignored for a single token (n_tokens == 1): its calls read the ids
 * directly, and a kq_moe_glu call for one token may leave no schedule. */
enum { KQ_LAYOUT_SHARED = 0, KQ_LAYOUT_SLOTTED = 1, KQ_REUSE_SCHEDULE = 0x100 };

/* GLU activations of kq_moe_glu: h = act(gate) * up.
 * mlx-kquant "bindings.cpp", moe_glu_gather_kq: act='silu' (the default) or
 * 'gelu' (the tanh approximation).
 *   KQ_ACT_SILU       silu(z) = z / (1 + e^-z)
 *   KQ_ACT_GELU_TANH  gelu(z) = z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3)))
 * Any other value -> KQ_ERR_UNSUPPORTED. */
enum { KQ_ACT_SILU = 0, KQ_ACT_GELU_TANH = 1 };

/* Human-readable name of a status code (static storage). */
const char* kq_status_string(kq_status s);

/* Text of the last error raised on the calling thread (empty if none). */
const char* kq_last_error(void);

/* Weights per block (256 / 32 / 128) and bytes per block (144 / 34 / 28);
 * 0 for an unknown type. */
int kq_qk(kq_type t);
int kq_block_bytes(kq_type t);

/* Bytes of one weight row of k columns, or -1 if k is not a positive
 * multiple of the block size. */
int64_t kq_row_bytes(kq_type t, int64_t k);

/*
 * kq_dequantize -- decode a block matrix to dense floats.
 * mlx-kquant "bindings.cpp", dequantize (wire bytes whose last dimension is
 * a multiple of the block bytes -> float array); Ternary Bonsai
 * "ternel_packed_model.py", get_rows (one decoded weight per element).
 *
 *   w       [rows, k/QK blocks]   block bytes, 16-byte aligned
 *   out     [rows, k]             out_dt elements, row-major, 16-byte aligned
 *
 * Each value is the exact decoded weight rounded once to binary32 (ties to
 * even); fp16/bf16 outputs round that binary32 value again (ties to even).
 * Any size that fits in memory is accepted (large matrices are decoded by
 * several launches on the stream).
 * Errors: rows <= 0, k not a positive multiple of QK, null or misaligned
 * pointers, overlapping w/out -> KQ_ERR_INVALID_ARG.
 */
kq_status kq_dequantize(kq_type t, const void* w, int64_t rows, int64_t k, void* out,
                        kq_dtype out_dt, void* stream);

/*
 * kq_qmv / kq_qmm -- y = x @ dequant(w)^T.
 * mlx-kquant "bindings.cpp", quantized_matmul (x @ dequant(w), w laid out
 * [N, K] when transpose=True); Ternary Bonsai "ternel_packed_model.py",
 * tq1_matmul / tq1_gemm (x is (batch, columns), the result (batch, rows)).
 *
 *   w   [n, k/QK blocks]  block bytes, 16-byte aligned
 *   x   [m, k]            x_dt (f32, f16 or bf16), row-major, 16-byte aligned
 *   y   [m, n]            y_dt (f32, f16 or bf16), row-major, 16-byte aligned
 *
 * y[i, j] = sum_c x[i, c] * w[j, c], accumulated in fp32 and rounded once to
 * y_dt.  kq_qmv is the decode form (1 <= m <= 16, weights streamed once);
 * kq_qmm takes any m >= 1 and picks the decode form itself for small m.
 * Errors: n, k or m <= 0, k % QK != 0, n > 2^26, k > 2^24, m > 16 for kq_qmv,
 * null or misaligned pointers, y overlapping w or x -> KQ_ERR_INVALID_ARG.
 */
kq_status kq_qmv(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                 int64_t m, void* y, kq_dtype y_dt, void* stream);
kq_status kq_qmm(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                 int64_t m, void* y, kq_dtype y_dt, void* stream);

/*
 * kq_moe_workspace_bytes -- size of the caller-owned scratch that
 * kq_moe_route, kq_qmm_id and kq_moe_glu need for a routing of n_tokens x
 * top_k rows over n_experts experts, where n_out is the widest output row
 * (n) of any kq_qmm_id call with scores that will use it (0 if none).
 * mlx-native "quantized_matmul_id_ggml.rs", IdMmScratch / id_mm_scratch_bytes
 * (caller-owned, reusable scratch; no allocation per call).  Returns 0 on
 * invalid arguments.
 */
size_t kq_moe_workspace_bytes(int64_t n_experts, int64_t n_tokens, int64_t top_k, int64_t n_out);

/*
 * Workspace layout written by kq_moe_route (int32 words, from the start):
 *   [0]                       number of tiles
 *   [1]                       number of rows with an invalid id (>= n_experts)
 *   [2 .. 2+E)                counts[e]: rows routed to expert e
 *   [2+E .. 3+2E)             offsets[e]: exclusive prefix sum of counts
 *   [3+2E .. 3+2E+R)          perm: routed-row indices t*top_k+slot grouped by
 *                             expert (ascending), ascending within an expert
 *   [3+2E+R .. +3*max_tiles)  tiles (expert, row_start, num_rows): each
 *                             expert's segment cut into KQ_MOE_TILE_ROWS-row
 *                             tiles, only the last of which may be partial
 *   [.. +R)                   scratch: per-activation-row scale exponents
 *                             (written by products with fp32 activations)
 * with R = n_tokens * top_k and max_tiles = min(R, ceil(R / KQ_MOE_TILE_ROWS)
 * + n_experts).  The fp32 slot buffer of kq_qmm_id follows at the next
 * 256-byte boundary.
 */
#define KQ_MOE_TILE_ROWS 32

/*
 * kq_moe_route -- sort routed rows by expert and cut them into tiles.
 * mlx-kquant "bindings.cpp", expert_tile_map (fixed-size row tiles, only the
 * last tile of a segment partial, built on the GPU with no host sync; here
 * KQ_MOE_TILE_ROWS = 32 rows, two 16-row MFMA sub-tiles); mlx-native
 * "quantized_matmul_id_ggml.rs", map0 regroup (ids validated on the device).
 *
 *   ids        [n_tokens, top_k] uint32 expert ids (device)
 *   workspace  at least kq_moe_workspace_bytes(n_experts, n_tokens, top_k, 0)
 *
 * The ids are never read on the host.  An id >= n_experts is counted as
 * invalid and left out of the schedule.  kq_qmm_id and kq_moe_glu call this
 * themselves; it is exported so the schedule can be inspected.
 */
kq_status kq_moe_route(const uint32_t* ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kq_qmm_id -- expert-routed product (mul_mat_id / gather_qmm).
 * mlx-native "quantized_matmul_id_ggml.rs", module comment:
 *   e = ids[t*top_k + r];  y[t*top_k + r][j] = sum_c dequant(W[e][j][c]) * x[t][c]
 * with the slotted input of the _pooled_slotted variant; mlx-kquant
 * "bindings.cpp", gather_qmm / gather_qmv_kq, and gather_qmv_mix_ns_kq for the
 * mixed form (each slot accumulated in f32 weighted by its score).
 *
 *   w          [n_experts][n, k/QK blocks], experts expert_stride bytes apart
 *   x          [n_tokens, k] (KQ_LAYOUT_SHARED) or [n_tokens, top_k, k]
 *              (KQ_LAYOUT_SLOTTED), x_dt f32, f16 or bf16
 *   ids        [n_tokens, top_k] uint32
 *   scores     NULL: y is [n_tokens*top_k, n];
 *              else [n_tokens, top_k] float32 and y is [n_tokens, n] with
 *              y[t] = sum over slots r in order of scores[t,r] * (W[e] x)
 *   workspace  kq_moe_workspace_bytes(n_experts, n_tokens, top_k, n) bytes
 *
 * Each expert's weights are streamed once per call however many rows it
 * serves.  A row with an id >= n_experts reads no weights and is written as
 * NaN (for the mixed form: that token's output row).
 * Errors: zero or negative sizes, top_k outside 1..n_experts,
 * n_tokens*top_k > INT32_MAX, k % QK != 0, n > 2^26, k > 2^24, expert_stride
 * smaller than one expert's bytes, null/misaligned pointers, y overlapping its inputs or the
 * workspace -> KQ_ERR_INVALID_ARG; workspace too small -> KQ_ERR_WORKSPACE.
 */
kq_status kq_qmm_id(kq_type t, const void* w, int64_t n_experts, int64_t n, int64_t k,
                    int64_t expert_stride, const void* x, kq_dtype x_dt, int x_layout,
                    const uint32_t* ids, int64_t n_tokens, int64_t top_k, const float* scores,
                    void* y, kq_dtype y_dt, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * kq_moe_glu -- fused MoE gate/up projections with the GLU epilogue.
 * mlx-kquant "bindings.cpp", moe_glu_gather_kq: gate and up expert products
 * share each activation load and act(g) * u is applied in the same kernel;
 * mlx-native "quantized_matmul_id_ggml.rs", the fused gate_up_silu expert
 * GEMM (one schedule, one write of h).
 *
 *   gate_w, up_w  [n_experts][n, k/QK blocks], experts expert_stride apart
 *   x             [n_tokens, k] x_dt f32, f16 or bf16
 *   ids           [n_tokens, top_k] uint32
 *   h             [n_tokens, top_k, n] h_dt (f16, bf16 or f32):
 *                 h = silu(W_gate[e] x_t) * (W_up[e] x_t), fp32 inside
 *   workspace     kq_moe_workspace_bytes(n_experts, n_tokens, top_k, 0)
 *
 * Rows with an invalid id are written as NaN.  Errors as kq_qmm_id; an
 * unknown act -> KQ_ERR_UNSUPPORTED.
 */
kq_status kq_moe_glu(kq_type t, const void* gate_w, const void* up_w, int64_t n_experts,
                     int64_t n, int64_t k, int64_t expert_stride, const void* x, kq_dtype x_dt,
                     const uint32_t* ids, int64_t n_tokens, int64_t top_k, int act, void* h,
                     kq_dtype h_dt, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
