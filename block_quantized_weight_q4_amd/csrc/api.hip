// api.hip -- the C ABI of libkq (include/kq.h): argument validation and
// kernel dispatch.  Everything is checked before anything is enqueued
// (mlx-native "quantized_matmul_id_ggml.rs", validate_id_call and the pooled
// pair variant: sizes, top_k range, K % QK, row-count limit, overlapping
// ranges); nothing here allocates, frees or synchronizes.
#include <mutex>
#include <string>

#include "../../include/kq.h"
#include "kq_device.h"
#include "kq_internal.h"

namespace {

thread_local std::string g_last_error;

kq_status fail(kq_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

int qk_of(int t) {
    switch (t) {
    case KQ_Q4_K: case KQ_Q6_K: case KQ_Q2_K: case KQ_Q3_K: case KQ_Q5_K: return 256;
    case KQ_TQ1_G128: return 128;
    case KQ_Q8_0: case KQ_Q4_0: case KQ_Q5_0: case KQ_Q5_1: return 32;
    default: return 0;
    }
}
int bb_of(int t) {
    switch (t) {
    case KQ_Q4_K: return 144;
    case KQ_Q8_0: return 34;
    case KQ_TQ1_G128: return 28;
    case KQ_Q4_0: return 18;
    case KQ_Q5_0: return 22;
    case KQ_Q5_1: return 24;
    case KQ_Q6_K: return 210;
    case KQ_Q2_K: return 84;
    case KQ_Q3_K: return 110;
    case KQ_Q5_K: return 176;
    default: return 0;
    }
}
// the codecs with an encoder (kq_quantize)
static bool has_encoder(int t) { return t == KQ_Q4_K || t == KQ_Q8_0 || t == KQ_TQ1_G128; }
int64_t elem_size(int dt) { return dt == KQ_F32 ? 4 : 2; }
bool valid_dt(int dt) { return dt == KQ_F32 || dt == KQ_F16 || dt == KQ_BF16; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// a*b with overflow detection (all operands non-negative)
bool mul_ok(int64_t a, int64_t b, int64_t& out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    out = a * b;
    return true;
}

struct Range {
    const void* p;
    int64_t bytes;
};
bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

kq_status launched(hipError_t e) {
    if (e != hipSuccess) return fail(KQ_ERR_DEVICE, std::string("HIP launch failed: ") + hipGetErrorString(e));
    g_last_error.clear();
    return KQ_OK;
}

// Common checks of a weight matrix [n, k] of type t.
kq_status check_weights(int t, const void* w, int64_t n, int64_t k, int64_t& row_bytes) {
    if (!qk_of(t)) return fail(KQ_ERR_UNSUPPORTED, "unknown weight type");
    if (n <= 0 || k <= 0) return fail(KQ_ERR_INVALID_ARG, "n and k must be positive");
    if (k % qk_of(t)) return fail(KQ_ERR_INVALID_ARG, "k must be a multiple of the block size");
    if (!w) return fail(KQ_ERR_INVALID_ARG, "null weight pointer");
    if (!aligned(w, 16)) return fail(KQ_ERR_INVALID_ARG, "weights must be 16-byte aligned");
    row_bytes = (k / qk_of(t)) * bb_of(t);
    return KQ_OK;
}

// Bounds of the product kernels: a dispatch counts its work-items per
// dimension in 32 bits (at most 32 threads per weight row), offsets inside
// one weight row, or a few rows of one tile, are 32-bit, and grid.y (tiles of
// activation rows, at least 16 rows each) stays below 65536.
constexpr int64_t kMaxN = (int64_t)1 << 26, kMaxK = (int64_t)1 << 24, kMaxM = (int64_t)1 << 19;

kq_status check_product_size(int64_t n, int64_t k) {
    if (n > kMaxN) return fail(KQ_ERR_INVALID_ARG, "n exceeds 2^26 weight rows");
    if (k > kMaxK) return fail(KQ_ERR_INVALID_ARG, "k exceeds 2^24 columns");
    return KQ_OK;
}

kq_status check_product(kq_type t, const void* w, int64_t n, int64_t k, const void* x,
                        kq_dtype x_dt, int64_t m, void* y, kq_dtype y_dt, int64_t& row_bytes) {
    kq_status st = check_weights(t, w, n, k, row_bytes);
    if (st) return st;
    if ((st = check_product_size(n, k))) return st;
    if (!valid_dt(x_dt) || !valid_dt(y_dt)) return fail(KQ_ERR_UNSUPPORTED, "unknown dtype");
    if (m <= 0) return fail(KQ_ERR_INVALID_ARG, "m must be positive");
    if (m > kMaxM) return fail(KQ_ERR_INVALID_ARG, "m exceeds 2^19 activation rows");
    if (!x || !y) return fail(KQ_ERR_INVALID_ARG, "null activation or output pointer");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(KQ_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    int64_t wb, xb, yb;
    if (!mul_ok(n, row_bytes, wb) || !mul_ok(m, k, xb) || !mul_ok(xb, elem_size(x_dt), xb) ||
        !mul_ok(m, n, yb) || !mul_ok(yb, elem_size(y_dt), yb))
        return fail(KQ_ERR_INVALID_ARG, "size overflow");
    if (overlap({y, yb}, {w, wb}) || overlap({y, yb}, {x, xb}))
        return fail(KQ_ERR_INVALID_ARG, "output overlaps an input");
    return KQ_OK;
}

}  // namespace

namespace kq {

MoeLayout moe_layout(int64_t n_experts, int64_t n_tokens, int64_t top_k, int64_t n_out) {
    MoeLayout L{};
    L.n_experts = n_experts;
    L.rows = n_tokens * top_k;
    // every tile holds at least one row, and each expert has at most one
    // partial tile
    const int64_t bound = (L.rows + kMoeTileRows - 1) / kMoeTileRows + n_experts;
    L.max_tiles = L.rows < bound ? L.rows : bound;
    L.counts_off = 2;
    L.offsets_off = L.counts_off + n_experts;
    L.perm_off = L.offsets_off + n_experts + 1;
    L.tiles_off = L.perm_off + L.rows;
    L.xexp_off = L.tiles_off + 3 * L.max_tiles;
    L.route_words = L.xexp_off + L.rows;
    L.slot_off_bytes = (L.route_words * 4 + 255) / 256 * 256;
    L.slot_bytes = L.rows * n_out * 4;
    L.total_bytes = L.slot_off_bytes + L.slot_bytes;
    return L;
}

}  // namespace kq

extern "C" {

const char* kq_status_string(kq_status s) {
    switch (s) {
    case KQ_OK: return "ok";
    case KQ_ERR_INVALID_ARG: return "invalid argument";
    case KQ_ERR_UNSUPPORTED: return "unsupported";
    case KQ_ERR_WORKSPACE: return "workspace too small";
    case KQ_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char* kq_last_error(void) { return g_last_error.c_str(); }

int kq_qk(kq_type t) { return qk_of(t); }
int kq_block_bytes(kq_type t) { return bb_of(t); }

int64_t kq_row_bytes(kq_type t, int64_t k) {
    if (!qk_of(t) || k <= 0 || k % qk_of(t)) return -1;
    return (k / qk_of(t)) * bb_of(t);
}

kq_status kq_dequantize(kq_type t, const void* w, int64_t rows, int64_t k, void* out,
                        kq_dtype out_dt, void* stream) {
    int64_t row_bytes;
    kq_status st = check_weights(t, w, rows, k, row_bytes);
    if (st) return st;
    if (!valid_dt(out_dt)) return fail(KQ_ERR_UNSUPPORTED, "unknown dtype");
    if (!out || !aligned(out, 16)) return fail(KQ_ERR_INVALID_ARG, "out must be non-null and 16-byte aligned");
    int64_t wb, ob;
    if (!mul_ok(rows, row_bytes, wb) || !mul_ok(rows, k, ob) || !mul_ok(ob, elem_size(out_dt), ob))
        return fail(KQ_ERR_INVALID_ARG, "size overflow");
    if (overlap({out, ob}, {w, wb})) return fail(KQ_ERR_INVALID_ARG, "output overlaps the weights");
    return launched(kq::launch_dequant(t, w, rows, k, out, out_dt, (hipStream_t)stream));
}

kq_status kq_quantize(kq_type t, const void* w, kq_dtype w_dt, int64_t rows, int64_t k,
                      const float* imatrix, void* out, void* stream) {
    if (!qk_of(t)) return fail(KQ_ERR_UNSUPPORTED, "unknown weight type");
    if (!has_encoder(t)) return fail(KQ_ERR_UNSUPPORTED, "no encoder for this weight type");
    if (!valid_dt(w_dt)) return fail(KQ_ERR_UNSUPPORTED, "unknown dtype");
    if (imatrix && t != KQ_Q4_K)
        return fail(KQ_ERR_UNSUPPORTED, "an importance vector steers the Q4_K encoder only");
    if (rows <= 0 || k <= 0) return fail(KQ_ERR_INVALID_ARG, "rows and k must be positive");
    if (k % qk_of(t)) return fail(KQ_ERR_INVALID_ARG, "k must be a multiple of the block size");
    if (!w || !out) return fail(KQ_ERR_INVALID_ARG, "null weight or output pointer");
    if (!aligned(w, (uintptr_t)elem_size(w_dt)) || !aligned(out, 16) || (imatrix && !aligned(imatrix, 4)))
        return fail(KQ_ERR_INVALID_ARG, "misaligned pointer (out: 16 bytes, w and imatrix: their element)");
    int64_t wb, ob;
    if (!mul_ok(rows, k, wb) || !mul_ok(wb, elem_size(w_dt), wb) ||
        !mul_ok(rows, (k / qk_of(t)) * bb_of(t), ob))
        return fail(KQ_ERR_INVALID_ARG, "size overflow");
    if (overlap({out, ob}, {w, wb}) || (imatrix && overlap({out, ob}, {imatrix, k * 4})))
        return fail(KQ_ERR_INVALID_ARG, "output overlaps an input");
    return launched(kq::launch_quantize(t, w, w_dt, rows, k, imatrix, out, (hipStream_t)stream));
}

kq_status kq_validate_tq1(const void* w, int64_t rows, int64_t k, uint64_t* n_illegal,
                          void* stream) {
    if (rows <= 0 || k <= 0) return fail(KQ_ERR_INVALID_ARG, "rows and k must be positive");
    if (k % 128) return fail(KQ_ERR_INVALID_ARG, "k must be a multiple of 128");
    if (!w || !n_illegal) return fail(KQ_ERR_INVALID_ARG, "null pointer");
    if (!aligned(w, 4) || !aligned(n_illegal, 8)) return fail(KQ_ERR_INVALID_ARG, "misaligned pointer");
    int64_t wb;
    if (!mul_ok(rows, (k / 128) * 28, wb)) return fail(KQ_ERR_INVALID_ARG, "size overflow");
    if (overlap({n_illegal, 8}, {w, wb})) return fail(KQ_ERR_INVALID_ARG, "count overlaps the weights");
    return launched(kq::launch_tq1_illegal(w, rows, k, (unsigned long long*)n_illegal,
                                           (hipStream_t)stream));
}

static kq_status dense_skinny(kq_type t, const void* w, int64_t n, int64_t k, int64_t row_bytes,
                              const void* x, kq_dtype x_dt, int64_t m, void* y, kq_dtype y_dt,
                              hipStream_t s) {
    kq::SkinnyArgs a{};
    a.w = (const uint8_t*)w;
    a.row_bytes = row_bytes;
    a.n = n;
    a.k = k;
    a.x = x;
    a.x_row = k;
    a.m = m;
    a.y = y;
    a.y_dt = y_dt;
    a.y_row = n;
    return launched(kq::launch_skinny(t, x_dt, false, a, 0, s));
}

kq_status kq_qmv(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                 int64_t m, void* y, kq_dtype y_dt, void* stream) {
    int64_t row_bytes;
    kq_status st = check_product(t, w, n, k, x, x_dt, m, y, y_dt, row_bytes);
    if (st) return st;
    if (m > 16) return fail(KQ_ERR_INVALID_ARG, "kq_qmv takes at most 16 activation rows");
    return dense_skinny(t, w, n, k, row_bytes, x, x_dt, m, y, y_dt, (hipStream_t)stream);
}

kq_status kq_qmm(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                 int64_t m, void* y, kq_dtype y_dt, void* stream) {
    int64_t row_bytes;
    kq_status st = check_product(t, w, n, k, x, x_dt, m, y, y_dt, row_bytes);
    if (st) return st;
    if (m <= 16 || x_dt == KQ_F32)
        return dense_skinny(t, w, n, k, row_bytes, x, x_dt, m, y, y_dt, (hipStream_t)stream);
    return launched(kq::launch_gemm(t, x_dt, w, n, k, x, m, y, y_dt, nullptr, (hipStream_t)stream));
}

// Scratch of the workspace forms.  The prefill GEMM (m > 16, 16-bit
// activations) takes the layout of kq::gemm_workspace.  Of the decode shapes,
// the TQ1 GEMV of one fp16 row splits K when its rows fill few workgroups,
// with fp32 partials [pieces][n]; the other decode products and the fp32
// path need no scratch.
static bool qmm_uses_gemm(kq_type, int64_t m, kq_dtype x_dt) { return m > 16 && x_dt != KQ_F32; }

static int64_t decode_split_bytes(kq_type t, int64_t n, int64_t k, int64_t m, kq_dtype x_dt,
                                  int* pnb) {
    *pnb = 0;
    if (t != KQ_TQ1_G128 || x_dt != KQ_F16 || m != 1) return 0;
    const int pieces = kq::tq1_mv_pieces(n, k, pnb);
    if (pieces < 2) {
        *pnb = 0;
        return 0;
    }
    return ((int64_t)pieces * n * 4 + 255) / 256 * 256;
}

static int64_t qmm_scratch_bytes(kq_type t, int64_t n, int64_t k, int64_t m, kq_dtype x_dt,
                                 int* pnb) {
    *pnb = 0;
    if (qmm_uses_gemm(t, m, x_dt)) return kq::gemm_workspace(t, n, k, m, x_dt).bytes;
    return decode_split_bytes(t, n, k, m, x_dt, pnb);
}

// The product of the workspace forms on scratch of `need` bytes at ws (or
// none when need is 0).
static kq_status qmm_with_scratch(kq_type t, const void* w, int64_t n, int64_t k, int64_t row_bytes,
                                  const void* x, kq_dtype x_dt, int64_t m, void* y, kq_dtype y_dt,
                                  int64_t need, int pnb, void* ws, hipStream_t s) {
    if (qmm_uses_gemm(t, m, x_dt))
        return launched(kq::launch_gemm(t, x_dt, w, n, k, x, m, y, y_dt, need > 0 ? ws : nullptr, s));
    if (need == 0) return dense_skinny(t, w, n, k, row_bytes, x, x_dt, m, y, y_dt, s);
    // the split TQ1 decode product (the only decode shape that takes scratch)
    const int pieces = (int)((k / 128 + pnb - 1) / pnb);
    hipError_t e = kq::launch_tq1_mv((const uint8_t*)w, n, k, (const uint16_t*)x, y, y_dt, s, pnb,
                                     (float*)ws);
    if (e == hipSuccess) e = kq::launch_splitk_reduce((const float*)ws, pieces, n, y, y_dt, s);
    return launched(e);
}

size_t kq_qmm_workspace_bytes(kq_type t, int64_t n, int64_t k, int64_t m, kq_dtype x_dt) {
    if (!qk_of(t) || n <= 0 || k <= 0 || m <= 0 || k % qk_of(t) || !valid_dt(x_dt)) return 0;
    if (n > kMaxN || k > kMaxK || m > kMaxM) return 0;
    int pnb;
    return (size_t)qmm_scratch_bytes(t, n, k, m, x_dt, &pnb);
}

kq_status kq_qmm_ws(kq_type t, const void* w, int64_t n, int64_t k, const void* x, kq_dtype x_dt,
                    int64_t m, void* y, kq_dtype y_dt, void* workspace, size_t workspace_bytes,
                    void* stream) {
    int64_t row_bytes;
    kq_status st = check_product(t, w, n, k, x, x_dt, m, y, y_dt, row_bytes);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    int pnb;
    const int64_t need = qmm_scratch_bytes(t, n, k, m, x_dt, &pnb);
    if (need > 0) {
        if (!workspace || !aligned(workspace, 256))
            return fail(KQ_ERR_WORKSPACE, "workspace must be non-null and 256-byte aligned");
        if ((int64_t)workspace_bytes < need)
            return fail(KQ_ERR_WORKSPACE, "workspace smaller than kq_qmm_workspace_bytes()");
        const int64_t xb = m * k * elem_size(x_dt), yb = m * n * elem_size(y_dt);
        if (overlap({workspace, need}, {w, n * row_bytes}) || overlap({workspace, need}, {x, xb}) ||
            overlap({workspace, need}, {y, yb}))
            return fail(KQ_ERR_INVALID_ARG, "workspace overlaps an input or the output");
    }
    return qmm_with_scratch(t, w, n, k, row_bytes, x, x_dt, m, y, y_dt, need, pnb, workspace, s);
}

// ---------------------------------------------------------------- kq_qmm_noalloc
// The scratch of kq_qmm_noalloc: one fixed array per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept
// per device.
static constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static kq_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KQ_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KQ_ERR_DEVICE, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(KQ_ERR_DEVICE, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KQ_OK;
}

size_t kq_qmm_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

kq_status kq_qmm_noalloc(kq_type t, const void* w, int64_t n, int64_t k, const void* x,
                         kq_dtype x_dt, int64_t m, void* y, kq_dtype y_dt, void* stream) {
    int64_t row_bytes;
    kq_status st = check_product(t, w, n, k, x, x_dt, m, y, y_dt, row_bytes);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    int pnb;
    const int64_t need = qmm_scratch_bytes(t, n, k, m, x_dt, &pnb);
    if (need > (int64_t)kNoAllocScratchBytes)
        return fail(KQ_ERR_WORKSPACE, "product needs more scratch than kq_qmm_noalloc holds "
                                      "(kq_qmm_workspace_bytes() > kq_qmm_noalloc_max_bytes())");
    void* ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws))) return st;
    return qmm_with_scratch(t, w, n, k, row_bytes, x, x_dt, m, y, y_dt, need, pnb, ws, s);
}

size_t kq_moe_workspace_bytes(int64_t n_experts, int64_t n_tokens, int64_t top_k, int64_t n_out) {
    if (n_experts <= 0 || n_tokens <= 0 || top_k <= 0 || n_out < 0) return 0;
    if (n_tokens > INT32_MAX / top_k) return 0;
    return (size_t)kq::moe_layout(n_experts, n_tokens, top_k, n_out).total_bytes;
}

static const int64_t kMaxExperts = 4096;
static const int64_t kMaxGridY = 65535;

// top_k and n_experts count a shared expert's slot when there is one;
// ids_per_token (0: top_k) is the number of ids per token the caller holds.
static kq_status check_routing(const uint32_t* ids, int64_t n_tokens, int64_t top_k,
                               int64_t n_experts, void* workspace, size_t workspace_bytes,
                               int64_t n_out, int64_t ids_per_token = 0) {
    if (!ids_per_token) ids_per_token = top_k;
    if (n_experts <= 0 || n_experts > kMaxExperts)
        return fail(KQ_ERR_INVALID_ARG, "n_experts must be in 1..4096");
    if (n_tokens <= 0) return fail(KQ_ERR_INVALID_ARG, "n_tokens must be positive");
    if (top_k <= 0 || top_k > n_experts) return fail(KQ_ERR_INVALID_ARG, "top_k must be in 1..n_experts");
    if (n_tokens > INT32_MAX / top_k) return fail(KQ_ERR_INVALID_ARG, "n_tokens * top_k exceeds INT32_MAX");
    if (!ids || !aligned(ids, 4)) return fail(KQ_ERR_INVALID_ARG, "ids must be non-null and 4-byte aligned");
    const kq::MoeLayout L = kq::moe_layout(n_experts, n_tokens, top_k, n_out);
    // the routed products put the schedule's tile slots on grid.y
    if (L.max_tiles > kMaxGridY)
        return fail(KQ_ERR_INVALID_ARG, "routing exceeds 65535 schedule tiles (n_tokens * top_k too large)");
    if (!workspace || !aligned(workspace, 256))
        return fail(KQ_ERR_WORKSPACE, "workspace must be non-null and 256-byte aligned");
    if ((int64_t)workspace_bytes < L.total_bytes)
        return fail(KQ_ERR_WORKSPACE, "workspace smaller than kq_moe_workspace_bytes()");
    if (overlap({workspace, L.total_bytes}, {ids, n_tokens * ids_per_token * 4}))
        return fail(KQ_ERR_INVALID_ARG, "workspace overlaps ids");
    return KQ_OK;
}

kq_status kq_moe_route(const uint32_t* ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                       void* workspace, size_t workspace_bytes, void* stream) {
    kq_status st = check_routing(ids, n_tokens, top_k, n_experts, workspace, workspace_bytes, 0);
    if (st) return st;
    const kq::MoeLayout L = kq::moe_layout(n_experts, n_tokens, top_k, 0);
    return launched(kq::launch_route(ids, L.rows, top_k, n_experts, L, (int32_t*)workspace,
                                     (hipStream_t)stream));
}

// Shared validation of the expert-routed calls.
// With a shared expert (shexp = 1; w_sh, and w2_sh for the GLU, are its
// matrices of n rows) the routing has top_k + 1 slots per token over
// n_experts + 1 experts, and scores / outputs count top_k + 1 slots.
static kq_status check_expert_call(kq_type t, const void* w, const void* w2, int64_t n_experts,
                                   int64_t n, int64_t k, int64_t expert_stride, const void* x,
                                   kq_dtype x_dt, int64_t x_rows, const uint32_t* ids,
                                   int64_t n_tokens, int64_t top_k, const float* scores, void* y,
                                   kq_dtype y_dt, int64_t y_rows, void* workspace,
                                   size_t workspace_bytes, int64_t n_out, int64_t& row_bytes,
                                   int shexp = 0, const void* w_sh = nullptr,
                                   const void* w2_sh = nullptr) {
    kq_status st = check_weights(t, w, n, k, row_bytes);
    if (st) return st;
    if ((st = check_product_size(n, k))) return st;
    if (w2 && !aligned(w2, 16)) return fail(KQ_ERR_INVALID_ARG, "weights must be 16-byte aligned");
    if (shexp && (!w_sh || (w2 && !w2_sh)))
        return fail(KQ_ERR_INVALID_ARG, "null shared-expert weights");
    if ((w_sh && !aligned(w_sh, 16)) || (w2_sh && !aligned(w2_sh, 16)))
        return fail(KQ_ERR_INVALID_ARG, "shared-expert weights must be 16-byte aligned");
    if (!valid_dt(x_dt) || !valid_dt(y_dt)) return fail(KQ_ERR_UNSUPPORTED, "unknown dtype");
    if (top_k <= 0 || top_k > n_experts) return fail(KQ_ERR_INVALID_ARG, "top_k must be in 1..n_experts");
    if (n_experts <= 0 || n_experts > kMaxExperts - shexp)
        return fail(KQ_ERR_INVALID_ARG, "n_experts out of range");
    st = check_routing(ids, n_tokens, top_k + shexp, n_experts + shexp, workspace, workspace_bytes,
                       n_out, top_k);
    if (st) return st;
    int64_t one;
    if (!mul_ok(n, row_bytes, one)) return fail(KQ_ERR_INVALID_ARG, "size overflow");
    if (expert_stride < one) return fail(KQ_ERR_INVALID_ARG, "expert_stride smaller than one expert");
    if (expert_stride % 16) return fail(KQ_ERR_INVALID_ARG, "expert_stride must be a multiple of 16");
    int64_t wb, xb, yb;
    if (!mul_ok(n_experts - 1, expert_stride, wb) || (wb += one) < one)
        return fail(KQ_ERR_INVALID_ARG, "size overflow");
    if (!x || !y || !aligned(x, 16) || !aligned(y, 16))
        return fail(KQ_ERR_INVALID_ARG, "x and y must be non-null and 16-byte aligned");
    if (scores && !aligned(scores, 4)) return fail(KQ_ERR_INVALID_ARG, "scores must be 4-byte aligned");
    if (!mul_ok(x_rows, k, xb) || !mul_ok(xb, elem_size(x_dt), xb) || !mul_ok(y_rows, n, yb) ||
        !mul_ok(yb, elem_size(y_dt), yb))
        return fail(KQ_ERR_INVALID_ARG, "size overflow");
    const kq::MoeLayout L = kq::moe_layout(n_experts + shexp, n_tokens, top_k + shexp, n_out);
    const Range ry{y, yb};
    if (overlap(ry, {w, wb}) || (w2 && overlap(ry, {w2, wb})) || overlap(ry, {x, xb}) ||
        overlap(ry, {ids, n_tokens * top_k * 4}) ||
        (scores && overlap(ry, {scores, n_tokens * (top_k + shexp) * 4})) ||
        overlap(ry, {workspace, L.total_bytes}) || overlap(ry, {w_sh, one}) ||
        overlap(ry, {w2_sh, one}))
        return fail(KQ_ERR_INVALID_ARG, "output overlaps an input or the workspace");
    if (overlap({workspace, L.total_bytes}, {x, xb}) || overlap({workspace, L.total_bytes}, {w, wb}) ||
        overlap({workspace, L.total_bytes}, {w_sh, one}) || overlap({workspace, L.total_bytes}, {w2_sh, one}))
        return fail(KQ_ERR_INVALID_ARG, "workspace overlaps an input");
    return KQ_OK;
}

// The routed product; with shexp (mixed and slotted only) the last of top_k
// + 1 slots per token is the shared expert w_sh.
static kq_status qmm_id_impl(kq_type t, const void* w, int64_t n_experts, int64_t n, int64_t k,
                             int64_t expert_stride, const void* w_sh, const void* x, kq_dtype x_dt,
                             int x_layout, const uint32_t* ids, int64_t n_tokens, int64_t top_k,
                             const float* scores, void* y, kq_dtype y_dt, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const int shexp = w_sh ? 1 : 0;
    const bool reuse = (x_layout & KQ_REUSE_SCHEDULE) != 0 && scores && n_tokens > 1;
    x_layout &= ~KQ_REUSE_SCHEDULE;
    if (x_layout != KQ_LAYOUT_SHARED && x_layout != KQ_LAYOUT_SLOTTED)
        return fail(KQ_ERR_INVALID_ARG, "unknown x layout");
    const int64_t S = top_k + shexp;  // slots per token
    const int64_t rows = (n_tokens > 0 && S > 0 && n_tokens <= INT32_MAX / S) ? n_tokens * S : 0;
    const int64_t x_rows = x_layout == KQ_LAYOUT_SHARED ? n_tokens : rows;
    const int64_t y_rows = scores ? n_tokens : rows;
    int64_t row_bytes;
    kq_status st = check_expert_call(t, w, nullptr, n_experts, n, k, expert_stride, x, x_dt, x_rows,
                                     ids, n_tokens, top_k, scores, y, y_dt, y_rows, workspace,
                                     workspace_bytes, scores ? n : 0, row_bytes, shexp, w_sh);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    // one token, mixed: the slots are summed as their expert rows stream,
    // with no schedule and no slot rows
    if (scores && n_tokens == 1 && t == KQ_Q4_K && (x_dt == KQ_F16 || x_dt == KQ_F32)) {
        kq::DownMixArgs d{};
        d.w = (const uint8_t*)w;
        d.expert_stride = expert_stride;
        d.row_bytes = row_bytes;
        d.n = n;
        d.k = k;
        d.x = x;
        d.slotted = x_layout == KQ_LAYOUT_SLOTTED;
        d.ids = ids;
        d.scores = scores;
        d.n_experts = n_experts;
        d.top_k = S;
        d.y = y;
        d.y_dt = y_dt;
        d.shexp = shexp;
        d.w_sh = (const uint8_t*)w_sh;
        return launched(kq::launch_down_mix1(d, x_dt == KQ_F32, s));
    }
    // ... and for Q8_0 and the further GGUF codecs where their kernel takes k.
    // fp32 rows are split into fp16 hi + lo once, into the workspace's slot
    // buffer (unused by this form) where they fit, else by each workgroup.
    const kq::MoeLayout L1 = kq::moe_layout(n_experts + shexp, 1, S, n);
    const int64_t x_rows1 = x_layout == KQ_LAYOUT_SLOTTED ? S : 1;
    const int mode1 = x_dt == KQ_F16 ? 0 : (x_rows1 * k * 4 <= L1.slot_bytes ? 1 : 2);
    if (scores && n_tokens == 1 && (t == KQ_Q8_0 || t >= KQ_Q4_0) && (x_dt == KQ_F16 || x_dt == KQ_F32) &&
        kq::down1_fits(t, k, S, mode1)) {
        kq::DownMixArgs d{};
        d.w = (const uint8_t*)w;
        d.expert_stride = expert_stride;
        d.row_bytes = row_bytes;
        d.n = n;
        d.k = k;
        d.x = x;
        d.slotted = x_layout == KQ_LAYOUT_SLOTTED;
        d.ids = ids;
        d.scores = scores;
        d.n_experts = n_experts;
        d.top_k = S;
        d.y = y;
        d.y_dt = y_dt;
        d.shexp = shexp;
        d.w_sh = (const uint8_t*)w_sh;
        if (mode1 == 1) {
            uint8_t* xsplit = (uint8_t*)workspace + L1.slot_off_bytes;
            int32_t* xexp = (int32_t*)workspace + L1.xexp_off;
            const hipError_t e = kq::launch_split_rows((const float*)x, x_rows1, k, xsplit, xexp, s);
            if (e != hipSuccess) return launched(e);
            d.x = xsplit;
            d.xexp = xexp;
        }
        return launched(kq::launch_down1_gguf(t, d, mode1, s));
    }
    const kq::MoeLayout L = kq::moe_layout(n_experts + shexp, n_tokens, S, scores ? n : 0);
    int32_t* ws = (int32_t*)workspace;
    // the unmixed form's rows with an invalid id are poisoned by the route;
    // the mixed form's tokens by the mix
    hipError_t e = hipSuccess;
    if (!reuse)
        e = scores ? kq::launch_route(ids, L.rows, S, n_experts + shexp, L, ws, s, nullptr, 0, 0, shexp)
                   : kq::launch_route(ids, L.rows, S, n_experts + shexp, L, ws, s, y, n, y_dt, shexp);
    if (e != hipSuccess) return launched(e);
    kq::SkinnyArgs a{};
    a.w = (const uint8_t*)w;
    a.w_sh = (const uint8_t*)w_sh;
    a.shexp = shexp;
    a.n_experts = n_experts;
    a.row_bytes = row_bytes;
    a.expert_stride = expert_stride;
    a.n = n;
    a.k = k;
    a.x = x;
    a.x_row = k;
    a.top_k = S;
    a.shared_x = x_layout == KQ_LAYOUT_SHARED;
    a.one_x_row = a.shared_x && n_tokens == 1;
    a.ws = ws;
    a.tiles_off = L.tiles_off;
    a.perm_off = L.perm_off;
    a.xexp_off = L.xexp_off;
    a.rows_cap = L.rows;
    if (scores) {
        float* slots = (float*)((char*)workspace + L.slot_off_bytes);
        a.y = slots;
        a.y_dt = KQ_F32;
        a.y_row = n;
        e = kq::launch_skinny(t, x_dt, false, a, L.max_tiles, s);
        if (e != hipSuccess) return launched(e);
        return launched(kq::launch_mix(ids, scores, n_tokens, S, n_experts + shexp, ws, slots, n, y,
                                       y_dt, s, shexp));
    }
    a.y = y;
    a.y_dt = y_dt;
    a.y_row = n;
    return launched(kq::launch_skinny(t, x_dt, false, a, L.max_tiles, s));
}

kq_status kq_qmm_id(kq_type t, const void* w, int64_t n_experts, int64_t n, int64_t k,
                    int64_t expert_stride, const void* x, kq_dtype x_dt, int x_layout,
                    const uint32_t* ids, int64_t n_tokens, int64_t top_k, const float* scores,
                    void* y, kq_dtype y_dt, void* workspace, size_t workspace_bytes,
                    void* stream) {
    return qmm_id_impl(t, w, n_experts, n, k, expert_stride, nullptr, x, x_dt, x_layout, ids,
                       n_tokens, top_k, scores, y, y_dt, workspace, workspace_bytes, stream);
}

kq_status kq_qmm_id_mix_shexp(kq_type t, const void* w, int64_t n_experts, int64_t n, int64_t k,
                              int64_t expert_stride, const void* shexp_w, const void* x,
                              kq_dtype x_dt, int flags, const uint32_t* ids, int64_t n_tokens,
                              int64_t top_k, const float* scores, void* y, kq_dtype y_dt,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (flags & ~KQ_REUSE_SCHEDULE) return fail(KQ_ERR_INVALID_ARG, "unknown flags");
    if (!shexp_w) return fail(KQ_ERR_INVALID_ARG, "null shared-expert weights");
    if (!scores) return fail(KQ_ERR_INVALID_ARG, "null scores");
    return qmm_id_impl(t, w, n_experts, n, k, expert_stride, shexp_w, x, x_dt,
                       KQ_LAYOUT_SLOTTED | flags, ids, n_tokens, top_k, scores, y, y_dt, workspace,
                       workspace_bytes, stream);
}

static kq_status moe_glu_impl(kq_type t, const void* gate_w, const void* up_w, int64_t n_experts,
                              int64_t n, int64_t k, int64_t expert_stride, const void* shexp_gate_w,
                              const void* shexp_up_w, const void* x, kq_dtype x_dt,
                              const uint32_t* ids, int64_t n_tokens, int64_t top_k, int act,
                              float limit, void* h, kq_dtype h_dt, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (act != KQ_ACT_SILU && act != KQ_ACT_GELU_TANH && act != KQ_ACT_SILU_LIMIT)
        return fail(KQ_ERR_UNSUPPORTED, "unknown GLU activation");
    if (act == KQ_ACT_SILU_LIMIT && !(limit > 0.0f && limit < __builtin_inff()))
        return fail(KQ_ERR_INVALID_ARG, "silu_limit needs a finite limit > 0");
    if (!up_w) return fail(KQ_ERR_INVALID_ARG, "null up weights");
    if ((shexp_gate_w == nullptr) != (shexp_up_w == nullptr))
        return fail(KQ_ERR_INVALID_ARG, "shared-expert gate and up weights go together");
    const int shexp = shexp_gate_w ? 1 : 0;
    const int64_t S = top_k + shexp;
    const int64_t rows = (n_tokens > 0 && S > 0 && n_tokens <= INT32_MAX / S) ? n_tokens * S : 0;
    int64_t row_bytes;
    kq_status st = check_expert_call(t, gate_w, up_w, n_experts, n, k, expert_stride, x, x_dt,
                                     n_tokens, ids, n_tokens, top_k, nullptr, h, h_dt, rows,
                                     workspace, workspace_bytes, 0, row_bytes, shexp, shexp_gate_w,
                                     shexp_up_w);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const kq::MoeLayout L = kq::moe_layout(n_experts + shexp, n_tokens, S, 0);
    int32_t* ws = (int32_t*)workspace;
    kq::SkinnyArgs a{};
    // one token with fp16 activations: each grid row is one slot, whose
    // expert id is read directly (no schedule)
    const bool direct = n_tokens == 1 && t == KQ_Q4_K && x_dt == KQ_F16;
    // (Q8_0 and the further GGUF codecs, where their kernel takes k)
    const bool direct_gguf = n_tokens == 1 && (t == KQ_Q8_0 || t >= KQ_Q4_0) && x_dt == KQ_F16 &&
                             kq::glu1_fits(t, k);
    if (direct || direct_gguf) {
        a.ids = ids;
        a.m = 1;
    } else {
        hipError_t e = kq::launch_route(ids, L.rows, S, n_experts + shexp, L, ws, s, h, n, h_dt, shexp);
        if (e != hipSuccess) return launched(e);
        a.ws = ws;
    }
    a.n_experts = n_experts;
    a.shexp = shexp;
    a.w = (const uint8_t*)gate_w;
    a.w2 = (const uint8_t*)up_w;
    a.w_sh = (const uint8_t*)shexp_gate_w;
    a.w2_sh = (const uint8_t*)shexp_up_w;
    a.row_bytes = row_bytes;
    a.expert_stride = expert_stride;
    a.n = n;
    a.k = k;
    a.x = x;
    a.x_row = k;
    a.top_k = S;
    a.shared_x = 1;
    a.one_x_row = n_tokens == 1;
    a.tiles_off = L.tiles_off;
    a.perm_off = L.perm_off;
    a.xexp_off = L.xexp_off;
    a.rows_cap = L.rows;
    a.y = h;
    a.y_dt = h_dt;
    a.y_row = n;
    a.act = act;
    a.limit = limit;
    if (direct) return launched(kq::launch_moe_glu1(a, s));
    if (direct_gguf) return launched(kq::launch_glu1_gguf(t, a, s));
    return launched(kq::launch_skinny(t, x_dt, true, a, L.max_tiles, s));
}

kq_status kq_moe_glu(kq_type t, const void* gate_w, const void* up_w, int64_t n_experts,
                     int64_t n, int64_t k, int64_t expert_stride, const void* x, kq_dtype x_dt,
                     const uint32_t* ids, int64_t n_tokens, int64_t top_k, int act, void* h,
                     kq_dtype h_dt, void* workspace, size_t workspace_bytes, void* stream) {
    if (act != KQ_ACT_SILU && act != KQ_ACT_GELU_TANH)
        return fail(KQ_ERR_UNSUPPORTED, "unknown GLU activation (silu_limit: kq_moe_glu_ex)");
    return moe_glu_impl(t, gate_w, up_w, n_experts, n, k, expert_stride, nullptr, nullptr, x, x_dt,
                        ids, n_tokens, top_k, act, 0.0f, h, h_dt, workspace, workspace_bytes,
                        stream);
}

kq_status kq_moe_glu_ex(kq_type t, const void* gate_w, const void* up_w, int64_t n_experts,
                        int64_t n, int64_t k, int64_t expert_stride, const void* shexp_gate_w,
                        const void* shexp_up_w, const void* x, kq_dtype x_dt, const uint32_t* ids,
                        int64_t n_tokens, int64_t top_k, int act, float limit, void* h,
                        kq_dtype h_dt, void* workspace, size_t workspace_bytes, void* stream) {
    return moe_glu_impl(t, gate_w, up_w, n_experts, n, k, expert_stride, shexp_gate_w, shexp_up_w,
                        x, x_dt, ids, n_tokens, top_k, act, limit, h, h_dt, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"
