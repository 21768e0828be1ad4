/*
 * kq_oracle.c -- plain, slow CPU oracle for block-quantized weight products.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Every routine follows a written definition directly: each block is decoded
 * field by field into its exact real value (held in a double), and every
 * product is a sequential fp64 sum with no blocking, reordering or fusion.
 * OpenMP only splits independent output rows across threads; the arithmetic
 * of each row is unchanged.
 *
 * Sources (titles of the pages the definitions come from):
 *  [KQ]  mlx-kquant "bindings.cpp" -- op docstrings of dequantize,
 *        quantized_matmul, moe_glu_gather_kq, gather_qmv_mix_ns_kq,
 *        gather_qmm, expert_tile_map.
 *  [MID] mlx-native "quantized_matmul_id_ggml.rs" -- module comment (the
 *        expert-routed product), validate_id_call, the NaN-poison contract.
 *  [DS4] ds4 "ds4_metal.m" -- struct block_q8_0 and the Q8_0 row stride.
 *  [TQ1] Ternary Bonsai "ternel_packed_model.py" -- format constants, the
 *        LUT23 section (trit weights 1,3,9,27,81), get_rows (digit/slot map,
 *        (trit-1)*scale).
 *  The Q4_K super-block (fp16 d and dmin, 12 bytes of packed 6-bit scales and
 *  mins, 128 bytes of nibbles; w = d*sc*q - dmin*m) is the GGUF K-quant block
 *  the [KQ] and [MID] pages name ("q4_k", GgmlType::Q4_K).  The pages never
 *  print its bit packing; the packing used here is the GGUF convention and is
 *  a documented reading, pinned by hand-built blocks in the tests.
 *
 * Parity status: every function below has pins in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_Q4_K = 0, OR_Q8_0 = 1, OR_TQ1 = 2 };
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* ------------------------------------------------------------------ */
/* Scalar conversions                                                   */
/* ------------------------------------------------------------------ */

/* IEEE binary16 bit pattern -> exact real value.  1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 is the subnormal range
 * (fraction * 2^-24), exponent 31 is Inf/NaN. */
double or_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 word. */
double or_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double or_f32_to_double(float f) { return (double)f; }

/* Round an exact real value to binary32 (C's conversion is round to nearest,
 * ties to even, under the default rounding mode). */
float or_round_f32(double v) { return (float)v; }

/* Round-to-nearest-even of v onto the grid of a binary format with p
 * significant bits and minimum normal exponent emin (below it the grid keeps
 * the spacing of the smallest binade: the subnormals).  Returns the rounded
 * real; overflow is left to the caller. */
static double rne_grid(double v, int p, int emin) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);           /* a = m * 2^e, m in [0.5, 1) -> exponent e-1 */
    int ex = e - 1;
    if (ex < emin) ex = emin; /* subnormal range shares the emin quantum */
    double quantum = ldexp(1.0, ex - (p - 1));
    double q = a / quantum;   /* exact: scaling by a power of two */
    double r = nearbyint(q);  /* ties to even under the default mode */
    double out = r * quantum;
    return v < 0 ? -out : out;
}

/* binary32 -> binary16 bits, round to nearest even, overflow to +-Inf. */
uint16_t or_float_to_half_rne(float f) {
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return 0x7E00;
    double r = rne_grid(v, 11, -14);
    double a = fabs(r);
    if (isinf(a) || a >= 65536.0) return sign | 0x7C00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal: a = n * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    }
    int e;
    double m = frexp(a, &e); /* a = m*2^e, m in [0.5,1) */
    int biased = (e - 1) + 15;
    uint16_t frac = (uint16_t)(ldexp(m, 11) - 1024.0);
    return sign | (uint16_t)(biased << 10) | frac;
}

/* binary32 -> bfloat16 bits, round to nearest even, overflow to +-Inf. */
uint16_t or_float_to_bf16_rne(float f) {
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return 0x7FC0;
    double r = rne_grid(v, 8, -126);
    double a = fabs(r);
    if (isinf(a) || a >= ldexp(1.0, 128)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -126)) {
        return sign | (uint16_t)ldexp(a, 133); /* n * 2^-133 */
    }
    int e;
    double m = frexp(a, &e);
    int biased = (e - 1) + 127;
    uint16_t frac = (uint16_t)(ldexp(m, 8) - 128.0);
    return sign | (uint16_t)(biased << 7) | frac;
}

static double act_value(const void* x, int dt, int64_t i) {
    switch (dt) {
    case OR_F32: return (double)((const float*)x)[i];
    case OR_F16: return or_half_to_double(((const uint16_t*)x)[i]);
    case OR_BF16: return or_bf16_to_double(((const uint16_t*)x)[i]);
    }
    return NAN;
}

/* ------------------------------------------------------------------ */
/* Block decoders (exact real values)                                  */
/* ------------------------------------------------------------------ */

static uint16_t le16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Q4_K sub-block j (0..7): 6-bit scale and 6-bit min from the 12 packed
 * bytes S[0..11].  Sub-blocks 0..3 keep their scale in the low six bits of
 * S[j] and their min in the low six bits of S[j+4].  Sub-blocks 4..7 take
 * their low four bits from S[j+4] (scale in the low nibble, min in the high
 * nibble) and their top two bits from the spare top bits of S[j-4] (scale)
 * and S[j] (min). */
void or_q4k_scale_min(const uint8_t* S, int j, int* sc, int* m) {
    if (j < 4) {
        *sc = S[j] & 63;
        *m = S[j + 4] & 63;
    } else {
        *sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
        *m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
}

/* Q4_K super-block: 256 weights.  Quant bytes Q[0..127] come in four chunks
 * of 32 bytes; chunk c feeds weights 64c..64c+63: the low nibbles of its 32
 * bytes are weights 64c..64c+31 (sub-block 2c) and the high nibbles are
 * weights 64c+32..64c+63 (sub-block 2c+1).  Each weight is
 * d * sc_j * q - dmin * m_j, computed exactly in double. */
void or_decode_q4k(const uint8_t* blk, double* out) {
    double d = or_half_to_double(le16(blk));
    double dmin = or_half_to_double(le16(blk + 2));
    const uint8_t* S = blk + 4;
    const uint8_t* Q = blk + 16;
    for (int c = 0; c < 4; ++c) {
        int sc0, m0, sc1, m1;
        or_q4k_scale_min(S, 2 * c, &sc0, &m0);
        or_q4k_scale_min(S, 2 * c + 1, &sc1, &m1);
        for (int l = 0; l < 32; ++l) {
            int lo = Q[32 * c + l] & 15;
            int hi = Q[32 * c + l] >> 4;
            out[64 * c + l] = d * sc0 * lo - dmin * m0;
            out[64 * c + 32 + l] = d * sc1 * hi - dmin * m1;
        }
    }
}

/* Q8_0 block (ds4 "struct block_q8_0"): fp16 d then 32 int8 quants. */
void or_decode_q8_0(const uint8_t* blk, double* out) {
    double d = or_half_to_double(le16(blk));
    for (int i = 0; i < 32; ++i) out[i] = d * (double)(int8_t)blk[2 + i];
}

/* TQ1_G128 block: 25 code bytes with five trits each, one tail byte with
 * three, then the fp16 scale.  Column c < 125 reads digit c mod 5 of slot
 * c / 5; columns 125..127 read digits 0..2 of the tail slot.  Digit d of a
 * code is floor(code / 3^d) mod 3 (trit weights 1, 3, 9, 27, 81) and the
 * weight is (digit - 1) * scale. */
void or_decode_tq1(const uint8_t* blk, double* out) {
    double s = or_half_to_double(le16(blk + 26));
    for (int c = 0; c < 128; ++c) {
        int slot, digit;
        if (c < 125) {
            slot = c / 5;
            digit = c - 5 * slot;
        } else {
            slot = 25;
            digit = c - 125;
        }
        int code = blk[slot];
        int p = 1;
        for (int i = 0; i < digit; ++i) p *= 3;
        int t = (code / p) % 3;
        out[c] = (double)(t - 1) * s;
    }
}

int or_qk(int type) {
    switch (type) {
    case OR_Q4_K: return 256;
    case OR_Q8_0: return 32;
    case OR_TQ1: return 128;
    }
    return 0;
}

int or_block_bytes(int type) {
    switch (type) {
    case OR_Q4_K: return 144;
    case OR_Q8_0: return 34;
    case OR_TQ1: return 28;
    }
    return 0;
}

static void decode_block(int type, const uint8_t* blk, double* out) {
    switch (type) {
    case OR_Q4_K: or_decode_q4k(blk, out); break;
    case OR_Q8_0: or_decode_q8_0(blk, out); break;
    case OR_TQ1: or_decode_tq1(blk, out); break;
    }
}

/* One weight row [k] of a row-major block matrix, exact. */
static void decode_row(int type, const uint8_t* w, int64_t row, int64_t k, double* out) {
    int qk = or_qk(type), bb = or_block_bytes(type);
    int64_t nb = k / qk;
    const uint8_t* r = w + row * nb * bb;
    for (int64_t b = 0; b < nb; ++b) decode_block(type, r + b * bb, out + b * qk);
}

/* [KQ] dequantize: wire bytes [rows, k/qk blocks] -> exact values [rows, k]. */
int or_dequant(int type, const uint8_t* w, int64_t rows, int64_t k, double* out) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) decode_row(type, w, r, k, out + r * k);
    return 0;
}

/* The stored result of dequantization in out_dt: the exact value rounded
 * once to binary32 (ties to even), and for fp16/bf16 outputs that binary32
 * value rounded again to the 16-bit format (ties to even) -- the result of
 * computing in fp32 and converting at the store. */
int or_dequant_store(int type, const uint8_t* w, int64_t rows, int64_t k, int out_dt, void* out) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            decode_row(type, w, r, k, row);
            for (int64_t c = 0; c < k; ++c) {
                float f = or_round_f32(row[c]);
                if (out_dt == OR_F32)
                    ((float*)out)[r * k + c] = f;
                else if (out_dt == OR_F16)
                    ((uint16_t*)out)[r * k + c] = or_float_to_half_rne(f);
                else
                    ((uint16_t*)out)[r * k + c] = or_float_to_bf16_rne(f);
            }
        }
        free(row);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Products                                                             */
/* ------------------------------------------------------------------ */

/* [KQ] quantized_matmul (transpose=True): y[m,n] = sum_k x[m,k] * w[n,k],
 * with w the dequantized [n,k] matrix.  Also returns s[m,n] = sum |x*w|,
 * the scale of the tolerance.  Sequential fp64 sum over k. */
int or_qmm(int type, const uint8_t* w, int64_t n, int64_t k, const void* x, int x_dt,
           int64_t m, double* y, double* s) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            decode_row(type, w, j, k, row);
            for (int64_t i = 0; i < m; ++i) {
                double acc = 0.0, mag = 0.0;
                for (int64_t c = 0; c < k; ++c) {
                    double t = act_value(x, x_dt, i * k + c) * row[c];
                    acc += t;
                    mag += fabs(t);
                }
                y[i * n + j] = acc;
                if (s) s[i * n + j] = mag;
            }
        }
        free(row);
    }
    return 0;
}

/* The same product restricted to a list of (m, n) output positions, for
 * checking sampled outputs of large problems one by one. */
int or_qmm_points(int type, const uint8_t* w, int64_t n, int64_t k, const void* x, int x_dt,
                  int64_t m, int64_t npts, const int64_t* pm, const int64_t* pn, double* y,
                  double* s) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t p = 0; p < npts; ++p) {
            int64_t i = pm[p], j = pn[p];
            if (i < 0 || i >= m || j < 0 || j >= n) {
                y[p] = NAN;
                if (s) s[p] = NAN;
                continue;
            }
            decode_row(type, w, j, k, row);
            double acc = 0.0, mag = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                double t = act_value(x, x_dt, i * k + c) * row[c];
                acc += t;
                mag += fabs(t);
            }
            y[p] = acc;
            if (s) s[p] = mag;
        }
        free(row);
    }
    return 0;
}

/* [MID] module comment + [KQ] gather_qmm / gather_qmv_kq /
 * gather_qmv_mix_ns_kq.  For each token t and slot r: e = ids[t,r];
 * row = W[e] (experts are expert_stride bytes apart) applied to x[t] (shared
 * layout, x is [T,k]) or x[t,r] (slotted layout, x is [T,top_k,k]).
 * Without scores: y[(t*top_k + r), n].  With scores: y[t, n] =
 * sum_r scores[t,r] * (W[e] x)[n], accumulated in slot order.  An id outside
 * [0, n_experts) poisons the rows it touches with NaN ([MID] contract). */
int or_qmm_id(int type, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
              int64_t expert_stride, const void* x, int x_dt, int slotted, const uint32_t* ids,
              int64_t T, int64_t top_k, const float* scores, double* y, double* s) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
    int64_t out_rows = scores ? T : T * top_k;
    for (int64_t i = 0; i < out_rows * n; ++i) {
        y[i] = 0.0;
        if (s) s[i] = 0.0;
    }
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t r = 0; r < top_k; ++r) {
                uint32_t e = ids[t * top_k + r];
                int64_t orow = scores ? t : t * top_k + r;
                int64_t xrow = slotted ? t * top_k + r : t;
                if ((int64_t)e >= n_experts) {
                    for (int64_t j = 0; j < n; ++j) {
                        y[orow * n + j] = NAN;
                        if (s) s[orow * n + j] = NAN;
                    }
                    continue;
                }
                const uint8_t* we = w + (int64_t)e * expert_stride;
                double wt = scores ? (double)scores[t * top_k + r] : 1.0;
                for (int64_t j = 0; j < n; ++j) {
                    decode_row(type, we, j, k, row);
                    double acc = 0.0, mag = 0.0;
                    for (int64_t c = 0; c < k; ++c) {
                        double tv = act_value(x, x_dt, xrow * k + c) * row[c];
                        acc += tv;
                        mag += fabs(tv);
                    }
                    y[orow * n + j] += wt * acc;
                    if (s) s[orow * n + j] += fabs(wt) * mag;
                }
            }
        }
        free(row);
    }
    return 0;
}

/* SiLU as defined: z / (1 + e^-z). */
double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* [KQ] moe_glu_gather_kq, act='gelu': GELU by its tanh approximation,
 * z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))). */
double or_gelu_tanh(double z) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* [KQ] moe_glu_gather_kq with act = 0 ('silu') or 1 ('gelu', tanh
 * approximation): for each token t and slot r with e = ids[t,r]:
 * g = W_gate[e] x_t, u = W_up[e] x_t, h = act(g) * u, giving h[T, top_k, n].
 * Also returns g, u and their |.|-sums sg, su (any of the extra outputs may
 * be NULL).  An invalid id poisons its h row with NaN. */
int or_moe_glu(int type, const uint8_t* gate_w, const uint8_t* up_w, int64_t n_experts,
               int64_t n, int64_t k, int64_t expert_stride, const void* x, int x_dt,
               const uint32_t* ids, int64_t T, int64_t top_k, int act, double* h, double* g,
               double* u, double* sg, double* su) {
    if (act != 0 && act != 1) return -3;
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
#pragma omp parallel
    {
        double* rg = (double*)malloc(sizeof(double) * k);
        double* ru = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t tr = 0; tr < T * top_k; ++tr) {
            int64_t t = tr / top_k;
            uint32_t e = ids[tr];
            for (int64_t j = 0; j < n; ++j) {
                int64_t o = tr * n + j;
                if ((int64_t)e >= n_experts) {
                    h[o] = NAN;
                    if (g) g[o] = NAN;
                    if (u) u[o] = NAN;
                    if (sg) sg[o] = NAN;
                    if (su) su[o] = NAN;
                    continue;
                }
                decode_row(type, gate_w + (int64_t)e * expert_stride, j, k, rg);
                decode_row(type, up_w + (int64_t)e * expert_stride, j, k, ru);
                double ag = 0, au = 0, mg = 0, mu = 0;
                for (int64_t c = 0; c < k; ++c) {
                    double xv = act_value(x, x_dt, t * k + c);
                    ag += xv * rg[c];
                    mg += fabs(xv * rg[c]);
                    au += xv * ru[c];
                    mu += fabs(xv * ru[c]);
                }
                h[o] = (act == 1 ? or_gelu_tanh(ag) : or_silu(ag)) * au;
                if (g) g[o] = ag;
                if (u) u[o] = au;
                if (sg) sg[o] = mg;
                if (su) su[o] = mu;
            }
        }
        free(rg);
        free(ru);
    }
    return 0;
}

/* Whole MoE layer in fp64 with no intermediate rounding: h from or_moe_glu
 * (kept in double), then out_t = sum_r scores[t,r] * W_down[e] h_{t,r}.
 * s_out[t,n] = sum_r |scores| * sum_j |W_down[e][n,j] * h_{t,r,j}|. */
int or_moe_layer(int type, const uint8_t* gate_w, const uint8_t* up_w, const uint8_t* down_w,
                 int64_t n_experts, int64_t hidden, int64_t ffn, int64_t gate_stride,
                 int64_t down_stride, const void* x, int x_dt, const uint32_t* ids, int64_t T,
                 int64_t top_k, const float* scores, double* out, double* s_out) {
    double* h = (double*)malloc(sizeof(double) * T * top_k * ffn);
    if (!h) return -2;
    int rc = or_moe_glu(type, gate_w, up_w, n_experts, ffn, hidden, gate_stride, x, x_dt, ids,
                        T, top_k, 0, h, NULL, NULL, NULL, NULL);
    if (rc) {
        free(h);
        return rc;
    }
    int qk = or_qk(type);
    if (ffn % qk) {
        free(h);
        return -1;
    }
    for (int64_t i = 0; i < T * hidden; ++i) {
        out[i] = 0.0;
        if (s_out) s_out[i] = 0.0;
    }
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * ffn);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t r = 0; r < top_k; ++r) {
                uint32_t e = ids[t * top_k + r];
                if ((int64_t)e >= n_experts) {
                    for (int64_t j = 0; j < hidden; ++j) {
                        out[t * hidden + j] = NAN;
                        if (s_out) s_out[t * hidden + j] = NAN;
                    }
                    continue;
                }
                double wt = (double)scores[t * top_k + r];
                const double* hr = h + (t * top_k + r) * ffn;
                for (int64_t j = 0; j < hidden; ++j) {
                    decode_row(type, down_w + (int64_t)e * down_stride, j, ffn, row);
                    double acc = 0.0, mag = 0.0;
                    for (int64_t c = 0; c < ffn; ++c) {
                        acc += row[c] * hr[c];
                        mag += fabs(row[c] * hr[c]);
                    }
                    out[t * hidden + j] += wt * acc;
                    if (s_out) s_out[t * hidden + j] += fabs(wt) * mag;
                }
            }
        }
        free(row);
    }
    free(h);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Expert routing schedule (integer work)                              */
/* ------------------------------------------------------------------ */

/* [KQ] expert_tile_map / [MID] expert regroup.  Routed rows are the flat
 * (token, slot) indices i = t*top_k + r.  counts[e] is the number of rows
 * with ids[i] == e; offsets is its exclusive prefix sum (offsets[E] = number
 * of valid rows); perm lists the rows grouped by expert in ascending expert
 * order, and in ascending i within an expert (a stable sort).  Rows with an
 * id >= E are not placed; their number is returned in *n_invalid.  The tile
 * map cuts each expert's segment into tiles of at most tile_rows rows, only
 * the last of which may be partial: (expert, row_start, num_rows), in
 * expert order.  Returns the number of tiles, or -1 if max_tiles is too
 * small. */
int64_t or_route(const uint32_t* ids, int64_t n_rows, int64_t n_experts, int64_t tile_rows,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* tiles,
                 int64_t max_tiles, int64_t* n_invalid) {
    int64_t bad = 0;
    for (int64_t e = 0; e < n_experts; ++e) counts[e] = 0;
    for (int64_t i = 0; i < n_rows; ++i) {
        if ((int64_t)ids[i] < n_experts)
            counts[ids[i]]++;
        else
            bad++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int64_t e = 0; e < n_experts; ++e)
        for (int64_t i = 0; i < n_rows; ++i)
            if ((int64_t)ids[i] == e) perm[pos++] = (int32_t)i;
    int64_t nt = 0;
    for (int64_t e = 0; e < n_experts; ++e) {
        for (int64_t start = 0; start < counts[e]; start += tile_rows) {
            if (nt >= max_tiles) return -1;
            int64_t len = counts[e] - start < tile_rows ? counts[e] - start : tile_rows;
            tiles[3 * nt + 0] = (int32_t)e;
            tiles[3 * nt + 1] = (int32_t)(offsets[e] + start);
            tiles[3 * nt + 2] = (int32_t)len;
            nt++;
        }
    }
    if (n_invalid) *n_invalid = bad;
    return nt;
}
