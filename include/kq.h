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
 * The further GGUF blocks that mlx-native "quantized_matmul_id_ggml.rs"
 * dispatches (GgmlType::Q4_0, Q5_0, Q5_1, Q6_K, Q2_K, Q3_K and Q5_K in its
 * mv_id / mm_id kernel tables).  The page names them without printing a
 * layout; these are the GGUF layouts:
 *   KQ_Q4_0      32 weights in 18 bytes: fp16 d, 16 bytes of nibbles (low
 *                nibble of byte i is weight i, high nibble weight i + 16);
 *                w = d * (q - 8).
 *   KQ_Q5_0      32 weights in 22 bytes: fp16 d, uint32 qh (bit i is weight
 *                i's fifth bit), 16 bytes of nibbles as in Q4_0;
 *                w = d * (q - 16).
 *   KQ_Q5_1      32 weights in 24 bytes: fp16 d, fp16 m, uint32 qh, 16 bytes
 *                of nibbles; w = d * q + m.
 *   KQ_Q6_K      256 weights in 210 bytes: ql[128] (low four bits), qh[64]
 *                (high two bits), int8 scales[16], fp16 d.  Weight
 *                128h + 32u + l (h < 2, u < 4, l < 32) takes the low (u < 2)
 *                or high nibble of ql[64h + 32(u % 2) + l], bits 2u..2u+1 of
 *                qh[32h + l] and scales[8h + 2u + l / 16];
 *                w = d * scale * (q - 32).
 *   KQ_Q2_K      256 weights in 84 bytes: 16 scale bytes (low nibble scale,
 *                high nibble min), qs[64], fp16 d, fp16 dmin.  Weight
 *                128h + 32u + l takes bits 2u..2u+1 of qs[32h + l] and scale
 *                byte 8h + 2u + l / 16; w = d * scale * q - dmin * min.
 *   KQ_Q3_K      256 weights in 110 bytes: hmask[32], qs[64], 12 bytes of
 *                packed 6-bit scales, fp16 d.  Weight 128h + 32u + l takes
 *                bits 2u..2u+1 of qs[32h + l] plus 4 times bit 4h + u of
 *                hmask[l], minus 4, and scale i = 8h + 2u + l / 16, whose low
 *                four bits are the low nibble of scale byte i (i < 8) or the
 *                high nibble of byte i - 8, and whose top two bits are bits
 *                2(i / 4)..2(i / 4)+1 of byte 8 + i % 4, stored plus 32;
 *                w = d * scale * q.
 *   KQ_Q5_K      256 weights in 176 bytes: fp16 d, fp16 dmin, the 12 scale
 *                and min bytes of Q4_K, qh[32], qs[128] in the Q4_K nibble
 *                order; weight 32j + l adds 16 times bit j of qh[l] to its
 *                Q4_K nibble; w = d * sc_j * q - dmin * m_j.
 * These seven are decoded and multiplied (kq_dequantize, the products and the
 * expert-routed forms) but not encoded (kq_quantize -> KQ_ERR_UNSUPPORTED).
 * Their prefill products (kq_qmm, m > 16, fp16 or bf16 activations) run on
 * the matrix-core GEMM with each weight rounded once to fp16, as for Q4_K and
 * Q8_0.  Their decode products of 2..16 fp16 activation rows (rows a whole
 * number of 1024 weights, 2048 for Q6_K and Q3_K) also run on the matrix
 * cores: Q4_0, Q5_0, Q5_1 and Q8_0 with each weight rounded once to fp16
 * (blocks whose weights could pass the fp16 range exactly), the K-quants with
 * exact fp16 integers and their scales applied in fp32.  Their single-token
 * MoE forms (kq_moe_glu with fp16 activations, kq_qmm_id with scores and
 * fp16 or fp32 activations; k a whole number of 1024 weights, 512 for Q6_K
 * and Q3_K) stream each slot's expert rows through LDS with exact fp16
 * integer pairs on the vector units; fp32 activation rows are split into
 * fp16 hi + lo (22 significant bits), once into the workspace's slot buffer
 * when n_slots * k <= n_slots * n.  Their expert-routed products over a
 * schedule (more than one token; k a whole number of 512 weights) run on the
 * matrix cores per schedule tile, as the batched decode products (fp32
 * activations with exact weights and fp16 hi + lo rows).  Their other
 * decode and expert-routed products run on the vector units with exact
 * weights.
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

typedef enum kq_type {
    KQ_Q4_K = 0,
    KQ_Q8_0 = 1,
    KQ_TQ1_G128 = 2,
    KQ_Q4_0 = 3,
    KQ_Q5_0 = 4,
    KQ_Q5_1 = 5,
    KQ_Q6_K = 6,
    KQ_Q2_K = 7,
    KQ_Q3_K = 8,
    KQ_Q5_K = 9
} kq_type;

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
 *   KQ_ACT_SILU_LIMIT h = silu(min(g, limit)) * clip(u, -limit, limit)
 *                     (act='silu_limit', deepseek-v4 LimitedSwiGLU; limit > 0;
 *                     kq_moe_glu_ex only, as it takes the limit)
 * The page's 'swiglu_clamp' (gpt-oss) is for mxfp4/nvfp4 weights only and is
 * not offered for these codecs.  Any other value -> KQ_ERR_UNSUPPORTED. */
enum { KQ_ACT_SILU = 0, KQ_ACT_GELU_TANH = 1, KQ_ACT_SILU_LIMIT = 2 };

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
 * kq_quantize -- encode float weights into block bytes.
 * mlx-kquant "bindings.cpp", quantize (float weights whose last dimension is
 * a multiple of the codec's block size -> the codec's wire bytes; an optional
 * 1-D float32 importance vector of length K steers the K-quant encoder).
 *
 *   w        [rows, k]            w_dt (f32, f16 or bf16), row-major, finite
 *   imatrix  [k] float32 >= 0, or NULL; Q4_K only (else KQ_ERR_UNSUPPORTED)
 *   out      [rows, k/QK blocks]  block bytes, 16-byte aligned
 *
 * The pages fix the contract, not an encoder; the encoders (binary32 steps in
 * a fixed order, so the bytes are reproducible bit for bit):
 *   Q8_0   d = fp16(max|w| / 127), q = clamp(rint(w * (1/d)), -127, 127).
 *   TQ1    s = fp16(max|w|) per 128 weights, trit = clamp(rint(w * (1/s)),
 *          -1, 1); every code byte is legal.
 *   Q4_K   per 32-weight sub-block, the min-max range [min(0, min w), max w]
 *          (with imatrix: the best of eight ranges shrunk towards the
 *          minimum, by importance-weighted squared error); d and dmin are
 *          the largest scale and min over 63 in fp16, the 6-bit sc and m the
 *          nearest multiples, q the nearest level clamped to 0..15.
 * Scales past 65504 are clamped to it.  A block decoded from the encoders'
 * output range (Q8_0 with a |q| of 127, TQ1 with a nonzero trit, Q4_K whose
 * sub-blocks use levels 0 and 15 and whose largest sc and m are 63) encodes
 * back to its own bytes.
 * Errors: rows or k <= 0, k % QK != 0, null or misaligned pointers, out
 * overlapping an input -> KQ_ERR_INVALID_ARG; the GGUF blocks other than Q4_K
 * and Q8_0 -> KQ_ERR_UNSUPPORTED (no encoder is built for them).
 */
kq_status kq_quantize(kq_type t, const void* w, kq_dtype w_dt, int64_t rows, int64_t k,
                      const float* imatrix, void* out, void* stream);

/*
 * kq_validate_tq1 -- count illegal TQ1_G128 code bytes (a full code byte
 * above 242, a tail byte above 26) in rows x k/128 blocks.  Ternary Bonsai
 * "ternel_packed_model.py", kernels section ("Bounds safety": legality is
 * enforced outside the product kernels, at conversion and at load).
 *
 *   w          [rows, k/128 blocks], 4-byte aligned (device)
 *   n_illegal  one uint64 in device memory, 8-byte aligned: the count
 *
 * The count is written on the stream (no host synchronization).  The product
 * kernels' outputs for weights with a nonzero count are unspecified.
 */
kq_status kq_validate_tq1(const void* w, int64_t rows, int64_t k, uint64_t* n_illegal,
                          void* stream);

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
 * Errors: n, k or m <= 0, k % QK != 0, n > 2^26, k > 2^24, m > 2^19 (m > 16
 * for kq_qmv), null or misaligned pointers, y overlapping w or x ->
 * KQ_ERR_INVALID_ARG.
 */
kq_status kq_qmv(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                 int64_t m, void* y, kq_dtype y_dt, void* stream);
kq_status kq_qmm(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                 int64_t m, void* y, kq_dtype y_dt, void* stream);

/*
 * kq_qmm_workspace_bytes / kq_qmm_ws -- kq_qmm with caller-owned scratch.
 * mlx-kquant "bindings.cpp", quantized_matmul (the same product); Ternary
 * Bonsai "ternel_packed_model.py", tq1_matmul (k_split: fp32 partial sums
 * over pieces of K, added in a second pass, for products whose output alone
 * does not fill the GPU); mlx-native "quantized_matmul_id_ggml.rs",
 * IdMmScratch (reusable caller-owned scratch, no allocation per call).
 *
 * y = x @ dequant(w)^T exactly as kq_qmm computes it (same arguments and
 * layouts, same error bound).  With the workspace:
 *   - bf16 activations are converted once per call to fp16 rows scaled by a
 *     power of two (without it, each output tile column converts its own
 *     copy of the activation rows);
 *   - a product with fewer output tiles than the GPU has compute units splits
 *     K across workgroups; the fp32 partial sums are added in a fixed order,
 *     so results are deterministic;
 *   - the TQ1_G128 decode product of one fp16 activation row (m = 1) whose
 *     rows fill fewer than 512 workgroups of 16 rows splits K the same way
 *     (Ternary Bonsai "ternel_packed_model.py", the split-K budget of its
 *     decode dispatches).
 *
 * kq_qmm_workspace_bytes returns the bytes kq_qmm_ws needs for these sizes
 * (0: none needed -- any other m <= 16 product, fp32 activations, or fp16
 * activations on a grid that is not split -- or invalid arguments).
 * workspace: device memory, 256-byte aligned, at least that many bytes,
 * overlapping neither the inputs nor y; its contents on entry are ignored
 * and on return unspecified.  Calls that share a workspace must not overlap
 * in time (use one stream, or one workspace per stream).
 * Errors: as kq_qmm; a missing, misaligned or too small workspace ->
 * KQ_ERR_WORKSPACE; a workspace overlapping w, x or y -> KQ_ERR_INVALID_ARG.
 */
size_t kq_qmm_workspace_bytes(kq_type t, int64_t n, int64_t k, int64_t m, kq_dtype x_dt);
kq_status kq_qmm_ws(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                    int64_t m, void* y, kq_dtype y_dt, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * kq_qmm_noalloc -- kq_qmm_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments as kq_qmm, same result as kq_qmm_ws (the same
 * kernels), with the scratch in a fixed array inside the library: one per
 * GPU, kq_qmm_noalloc_max_bytes() = 64 MiB, held until the process ends.
 * Nothing is allocated or freed by the call.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (concurrent streams or threads) race and give undefined results.
 * Serialize them (one stream), or use kq_qmm_ws with a workspace per stream.
 * Errors: as kq_qmm; a product whose kq_qmm_workspace_bytes() exceeds
 * kq_qmm_noalloc_max_bytes() -> KQ_ERR_WORKSPACE (nothing is launched).
 */
size_t kq_qmm_noalloc_max_bytes(void);
kq_status kq_qmm_noalloc(kq_type t, const void* w, int64_t n, int64_t k, const void* x,
                         kq_dtype x_dt, int64_t m, void* y, kq_dtype y_dt, void* stream);

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
 *   [0]                       number of tiles (0 when the matrix-matrix
 *                             rule poisons the whole operation)
 *   [1]                       number of rows with an id >= n_experts, plus,
 *                             from 32 tokens on, rows whose id repeats an
 *                             earlier slot of the same token
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
 * invalid and left out of the schedule; from 32 tokens on, repeated ids are
 * counted too and any defect leaves the schedule with no tiles (the rule of
 * kq_qmm_id).  kq_qmm_id and kq_moe_glu call this themselves; it is exported
 * so the schedule can be inspected.
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
 * serves.
 *
 * Invalid ids are data, not host errors (the ids are never read on the
 * host).  mlx-native "quantized_matmul_id_ggml.rs", the id contract of
 * quantized_matmul_id_ggml and the map0 comment of its matrix-matrix
 * dispatch, whose route threshold is 32 tokens:
 *   n_tokens < 32   (matrix-vector rule) a row with an id >= n_experts reads
 *                   no weights and is written as NaN (for the mixed form:
 *                   that token's output row); an id repeated within a token
 *                   is computed as written.
 *   n_tokens >= 32  (matrix-matrix rule) the top_k ids of a token must be
 *                   distinct and in range; otherwise the ENTIRE output is
 *                   NaN and no weights are read.
 * Errors: zero or negative sizes, top_k outside 1..n_experts,
 * n_tokens*top_k > INT32_MAX, more than 65535 schedule tiles
 * (min(R, ceil(R / KQ_MOE_TILE_ROWS) + n_experts) with R = n_tokens * top_k),
 * k % QK != 0, n > 2^26, k > 2^24, expert_stride
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
 * Invalid ids poison h by the rule of kq_qmm_id (below 32 tokens the h row
 * of an out-of-range id; from 32 tokens on all of h if any id is out of range
 * or repeated within a token).  Errors as kq_qmm_id; an unknown act ->
 * KQ_ERR_UNSUPPORTED.
 */
kq_status kq_moe_glu(kq_type t, const void* gate_w, const void* up_w, int64_t n_experts,
                     int64_t n, int64_t k, int64_t expert_stride, const void* x, kq_dtype x_dt,
                     const uint32_t* ids, int64_t n_tokens, int64_t top_k, int act, void* h,
                     kq_dtype h_dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kq_moe_glu_ex -- kq_moe_glu with every activation (KQ_ACT_SILU_LIMIT takes
 * `limit`) and an optional shared expert folded in as one extra, last slot.
 * mlx-kquant "bindings.cpp", moe_glu_gather_kq (act, limit) and
 * moe_glu_gather_shexp_kq (the block's shared expert as slot top_k, fed by
 * single-expert matrices row-shape-matched to the expert stack).
 *
 *   shexp_gate_w, shexp_up_w  [n, k/QK blocks] of type t (both, or both NULL)
 *   h   [n_tokens, top_k, n] without a shared expert, [n_tokens, top_k + 1, n]
 *       with one (slot top_k: act(W_sg x_t, W_su x_t))
 *   workspace  kq_moe_workspace_bytes(n_experts + 1, n_tokens, top_k + 1, 0)
 *       with a shared expert (it is routed as one more expert and slot)
 * The shared slot is never invalid; routed ids poison h by the rule of
 * kq_qmm_id.  Errors as kq_moe_glu; KQ_ACT_SILU_LIMIT with a limit that is
 * not a finite value > 0, or one of the two shared matrices NULL ->
 * KQ_ERR_INVALID_ARG.
 */
kq_status kq_moe_glu_ex(kq_type t, const void* gate_w, const void* up_w, int64_t n_experts,
                        int64_t n, int64_t k, int64_t expert_stride, const void* shexp_gate_w,
                        const void* shexp_up_w, const void* x, kq_dtype x_dt, const uint32_t* ids,
                        int64_t n_tokens, int64_t top_k, int act, float limit, void* h,
                        kq_dtype h_dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kq_qmm_id_mix_shexp -- the mixed down projection with the shared expert
 * as the last slot.  mlx-kquant "bindings.cpp", gather_qmv_mix_kq (every
 * slot, the last being the shared expert, accumulated in f32 weighted by its
 * score, replacing gather + weighted sum + shared add).
 *
 *   w        [n_experts][n, k/QK blocks], experts expert_stride apart
 *   shexp_w  [n, k/QK blocks] of type t
 *   x        [n_tokens, top_k + 1, k] (slotted; slot top_k feeds shexp_w)
 *   ids      [n_tokens, top_k] uint32 (the routed slots)
 *   scores   [n_tokens, top_k + 1] float32 (the last: the shared expert's)
 *   y        [n_tokens, n]: y[t] = sum over slots r in order of
 *            scores[t,r] * (W_r x[t,r]), W_r = W[ids[t,r]] or shexp_w
 *   flags    0 or KQ_REUSE_SCHEDULE (after a kq_moe_glu_ex call with the
 *            same shared-expert layout, ids, n_tokens and top_k)
 *   workspace  kq_moe_workspace_bytes(n_experts + 1, n_tokens, top_k + 1, n)
 * Invalid routed ids poison as in kq_qmm_id's mixed form.  Errors as
 * kq_qmm_id; NULL shexp_w or scores, unknown flags -> KQ_ERR_INVALID_ARG.
 */
kq_status kq_qmm_id_mix_shexp(kq_type t, const void* w, int64_t n_experts, int64_t n, int64_t k,
                              int64_t expert_stride, const void* shexp_w, const void* x,
                              kq_dtype x_dt, int flags, const uint32_t* ids, int64_t n_tokens,
                              int64_t top_k, const float* scores, void* y, kq_dtype y_dt,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
