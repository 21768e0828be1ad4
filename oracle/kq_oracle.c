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
 *  Q4_0, Q5_0, Q5_1, Q6_K, Q2_K, Q3_K and Q5_K are the further GGUF blocks of
 *  the [MID] page's codec table (GgmlType::Q4_0 ... Q5_K and their mv_id / mm_id
 *  kernel names); the page names them without printing a layout, so their
 *  layouts below are the GGUF convention as well -- readings, pinned by
 *  hand-built blocks and an independent decoder in the tests.
 *
 * Parity status: every function below has pins in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    OR_Q4_K = 0, OR_Q8_0 = 1, OR_TQ1 = 2, OR_Q4_0 = 3, OR_Q5_0 = 4, OR_Q5_1 = 5, OR_Q6_K = 6,
    OR_Q2_K = 7, OR_Q3_K = 8, OR_Q5_K = 9
};
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

/* Q4_0 block (32 weights, 18 bytes): fp16 d, then 16 bytes of nibbles; the
 * low nibble of byte j is weight j and the high nibble weight j + 16, and a
 * weight is d * (q - 8). */
void or_decode_q4_0(const uint8_t* blk, double* out) {
    double d = or_half_to_double(le16(blk));
    for (int j = 0; j < 16; ++j) {
        out[j] = d * ((blk[2 + j] & 15) - 8);
        out[j + 16] = d * ((blk[2 + j] >> 4) - 8);
    }
}

/* The fifth bit of weight i (0..31) of a Q5_0 / Q5_1 block: bit i of the
 * 32-bit little-endian word qh. */
static int q5_high_bit(const uint8_t* qh, int i) { return (qh[i >> 3] >> (i & 7)) & 1; }

/* Q5_0 block (32 weights, 22 bytes): fp16 d, 4 bytes qh, 16 bytes of nibbles
 * laid out as in Q4_0; the 5-bit quant of weight i is its nibble plus 16
 * times bit i of qh, and the weight is d * (q - 16). */
void or_decode_q5_0(const uint8_t* blk, double* out) {
    double d = or_half_to_double(le16(blk));
    const uint8_t* qh = blk + 2;
    const uint8_t* qs = blk + 6;
    for (int j = 0; j < 16; ++j) {
        int q0 = (qs[j] & 15) | (q5_high_bit(qh, j) << 4);
        int q1 = (qs[j] >> 4) | (q5_high_bit(qh, j + 16) << 4);
        out[j] = d * (q0 - 16);
        out[j + 16] = d * (q1 - 16);
    }
}

/* Q5_1 block (32 weights, 24 bytes): fp16 d, fp16 m, 4 bytes qh, 16 bytes of
 * nibbles; quants as in Q5_0, and the weight is d * q + m. */
void or_decode_q5_1(const uint8_t* blk, double* out) {
    double d = or_half_to_double(le16(blk));
    double m = or_half_to_double(le16(blk + 2));
    const uint8_t* qh = blk + 4;
    const uint8_t* qs = blk + 8;
    for (int j = 0; j < 16; ++j) {
        int q0 = (qs[j] & 15) | (q5_high_bit(qh, j) << 4);
        int q1 = (qs[j] >> 4) | (q5_high_bit(qh, j + 16) << 4);
        out[j] = d * q0 + m;
        out[j + 16] = d * q1 + m;
    }
}

/* Q6_K super-block (256 weights, 210 bytes): ql[128] (low four bits), qh[64]
 * (high two bits), 16 signed 8-bit scales, fp16 d.  The block is two halves
 * of 128 weights; half h uses ql[64h..], qh[32h..] and scales[8h..].  Weight
 * 128h + 32u + l (u = 0..3, l = 0..31) has the low bits of byte
 * ql[64h + l + 32 (u % 2)] (the low nibble for u < 2, the high nibble for
 * u >= 2), the high bits (qh[32h + l] >> 2u) & 3, the scale
 * scales[8h + l / 16 + 2u], and the value d * scale * (q - 32). */
void or_decode_q6_k(const uint8_t* blk, double* out) {
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    const int8_t* sc = (const int8_t*)(blk + 192);
    double d = or_half_to_double(le16(blk + 208));
    for (int h = 0; h < 2; ++h)
        for (int u = 0; u < 4; ++u)
            for (int l = 0; l < 32; ++l) {
                int lowb = ql[64 * h + l + 32 * (u & 1)];
                int lo4 = u < 2 ? (lowb & 15) : (lowb >> 4);
                int hi2 = (qh[32 * h + l] >> (2 * u)) & 3;
                int q = lo4 | (hi2 << 4);
                out[128 * h + 32 * u + l] = d * (double)sc[8 * h + l / 16 + 2 * u] * (q - 32);
            }
}

/* Q2_K super-block (256 weights, 84 bytes): 16 scale bytes (low nibble the
 * scale, high nibble the min of 16 weights), qs[64] of 2-bit quants, fp16 d,
 * fp16 dmin.  Like Q6_K it is two halves of 128 weights, each four runs of
 * 32: weight 128h + 32u + l takes bits 2u..2u+1 of qs[32h + l] and scale
 * byte 8h + 2u + l / 16, and is d * scale * q - dmin * min. */
void or_decode_q2_k(const uint8_t* blk, double* out) {
    const uint8_t* sc = blk;
    const uint8_t* qs = blk + 16;
    double d = or_half_to_double(le16(blk + 80));
    double dmin = or_half_to_double(le16(blk + 82));
    for (int h = 0; h < 2; ++h)
        for (int u = 0; u < 4; ++u)
            for (int l = 0; l < 32; ++l) {
                int q = (qs[32 * h + l] >> (2 * u)) & 3;
                int s = sc[8 * h + 2 * u + l / 16];
                out[128 * h + 32 * u + l] = d * (s & 15) * q - dmin * (s >> 4);
            }
}

/* The 6-bit scale i (0..15) of a Q3_K super-block from its 12 packed bytes
 * S: the low four bits are the low nibble of S[i] for i < 8 and the high
 * nibble of S[i - 8] for i >= 8; the top two bits are bits 2 (i / 4) and
 * 2 (i / 4) + 1 of S[8 + i % 4].  The stored value is offset by 32. */
int or_q3k_scale(const uint8_t* S, int i) {
    int low = i < 8 ? (S[i] & 15) : (S[i - 8] >> 4);
    int top = (S[8 + i % 4] >> (2 * (i / 4))) & 3;
    return (low | (top << 4)) - 32;
}

/* Q3_K super-block (256 weights, 110 bytes): hmask[32], qs[64] of 2-bit
 * quants, 12 bytes of packed 6-bit scales, fp16 d.  Weight 128h + 32u + l
 * takes bits 2u..2u+1 of qs[32h + l] as its low bits and bit 4h + u of
 * hmask[l] as its third bit; a clear third bit subtracts 4, so the quant
 * lies in -4..3.  Its scale is scale 8h + 2u + l / 16, and the weight is
 * d * scale * q. */
void or_decode_q3_k(const uint8_t* blk, double* out) {
    const uint8_t* hm = blk;
    const uint8_t* qs = blk + 32;
    const uint8_t* S = blk + 96;
    double d = or_half_to_double(le16(blk + 108));
    for (int h = 0; h < 2; ++h)
        for (int u = 0; u < 4; ++u)
            for (int l = 0; l < 32; ++l) {
                int low = (qs[32 * h + l] >> (2 * u)) & 3;
                int third = (hm[l] >> (4 * h + u)) & 1;
                int q = low - (third ? 0 : 4);
                out[128 * h + 32 * u + l] = d * or_q3k_scale(S, 8 * h + 2 * u + l / 16) * q;
            }
}

/* Q5_K super-block (256 weights, 176 bytes): fp16 d, fp16 dmin, the 12 scale
 * and min bytes of Q4_K, qh[32], qs[128] of nibbles laid out as in Q4_K.
 * Weight 32j + l of sub-block j (0..7) has the nibble Q4_K gives it as its
 * low four bits and bit j of qh[l] as its fifth, and is
 * d * sc_j * q - dmin * m_j. */
void or_decode_q5_k(const uint8_t* blk, double* out) {
    double d = or_half_to_double(le16(blk));
    double dmin = or_half_to_double(le16(blk + 2));
    const uint8_t* S = blk + 4;
    const uint8_t* qh = blk + 16;
    const uint8_t* qs = blk + 48;
    for (int j = 0; j < 8; ++j) {
        int sc, m;
        or_q4k_scale_min(S, j, &sc, &m);
        for (int l = 0; l < 32; ++l) {
            int byte = qs[32 * (j / 2) + l];
            int nib = (j % 2) ? (byte >> 4) : (byte & 15);
            int q = nib | (((qh[l] >> j) & 1) << 4);
            out[32 * j + l] = d * sc * q - dmin * m;
        }
    }
}

int or_qk(int type) {
    switch (type) {
    case OR_Q4_K: return 256;
    case OR_Q8_0: return 32;
    case OR_TQ1: return 128;
    case OR_Q4_0: return 32;
    case OR_Q5_0: return 32;
    case OR_Q5_1: return 32;
    case OR_Q6_K: return 256;
    case OR_Q2_K: return 256;
    case OR_Q3_K: return 256;
    case OR_Q5_K: return 256;
    }
    return 0;
}

int or_block_bytes(int type) {
    switch (type) {
    case OR_Q4_K: return 144;
    case OR_Q8_0: return 34;
    case OR_TQ1: return 28;
    case OR_Q4_0: return 18;
    case OR_Q5_0: return 22;
    case OR_Q5_1: return 24;
    case OR_Q6_K: return 210;
    case OR_Q2_K: return 84;
    case OR_Q3_K: return 110;
    case OR_Q5_K: return 176;
    }
    return 0;
}

static void decode_block(int type, const uint8_t* blk, double* out) {
    switch (type) {
    case OR_Q4_K: or_decode_q4k(blk, out); break;
    case OR_Q8_0: or_decode_q8_0(blk, out); break;
    case OR_TQ1: or_decode_tq1(blk, out); break;
    case OR_Q4_0: or_decode_q4_0(blk, out); break;
    case OR_Q5_0: or_decode_q5_0(blk, out); break;
    case OR_Q5_1: or_decode_q5_1(blk, out); break;
    case OR_Q6_K: or_decode_q6_k(blk, out); break;
    case OR_Q2_K: or_decode_q2_k(blk, out); break;
    case OR_Q3_K: or_decode_q3_k(blk, out); break;
    case OR_Q5_K: or_decode_q5_k(blk, out); break;
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

/* [MID] quantized_matmul_id_ggml doc comment ("Errors") and the map0
 * comment of its matrix-matrix dispatch: device-produced ids are checked on
 * the device.  The matrix-vector route only bounds-checks: an out-of-range id
 * poisons the output row(s) it touches and repeated ids are computed as
 * written.  The matrix-matrix route, which the page takes from
 * MM_ID_ROUTING_THRESHOLD = 32 tokens on, also requires the top_k ids of each
 * token to be distinct, and any out-of-range or repeated id there poisons the
 * entire output, with no weight read.  The reading here: a call of n_tokens
 * >= 32 follows the matrix-matrix rule, a smaller one the matrix-vector
 * rule, whichever kernels compute it. */
#define OR_MM_ID_MIN_TOKENS 32

/* 1 when a routing of T tokens follows the matrix-matrix rule and holds an
 * out-of-range id or a token with a repeated id (the whole output is NaN). */
int or_routing_poisons_all(const uint32_t* ids, int64_t T, int64_t top_k, int64_t n_experts) {
    if (T < OR_MM_ID_MIN_TOKENS) return 0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t r = 0; r < top_k; ++r) {
            uint32_t e = ids[t * top_k + r];
            if ((int64_t)e >= n_experts) return 1;
            for (int64_t q = 0; q < r; ++q)
                if (ids[t * top_k + q] == e) return 1;
        }
    return 0;
}

static void fill_nan(double* a, int64_t count) {
    if (!a) return;
    for (int64_t i = 0; i < count; ++i) a[i] = NAN;
}

/* [MID] module comment + [KQ] gather_qmm / gather_qmv_kq /
 * gather_qmv_mix_ns_kq.  For each token t and slot r: e = ids[t,r];
 * row = W[e] (experts are expert_stride bytes apart) applied to x[t] (shared
 * layout, x is [T,k]) or x[t,r] (slotted layout, x is [T,top_k,k]).
 * Without scores: y[(t*top_k + r), n].  With scores: y[t, n] =
 * sum_r scores[t,r] * (W[e] x)[n], accumulated in slot order.  Invalid ids
 * poison the output as or_routing_poisons_all describes: below 32 tokens an
 * id outside [0, n_experts) poisons the rows it touches with NaN, from 32
 * tokens on an out-of-range or repeated id poisons the whole output. */
int or_qmm_id(int type, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
              int64_t expert_stride, const void* x, int x_dt, int slotted, const uint32_t* ids,
              int64_t T, int64_t top_k, const float* scores, double* y, double* s) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
    int64_t out_rows = scores ? T : T * top_k;
    if (or_routing_poisons_all(ids, T, top_k, n_experts)) {
        fill_nan(y, out_rows * n);
        fill_nan(s, out_rows * n);
        return 0;
    }
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

/* [KQ] moe_glu_gather_kq, act='silu_limit' (deepseek-v4 LimitedSwiGLU):
 * silu(min(g, limit)) * clip(u, -limit, limit), limit > 0. */
double or_silu_limit(double g, double u, double limit) {
    double gc = g < limit ? g : limit;
    double uc = u < -limit ? -limit : u > limit ? limit : u;
    return or_silu(gc) * uc;
}

static double glu_value(int act, double g, double u, double limit) {
    if (act == 1) return or_gelu_tanh(g) * u;
    if (act == 2) return or_silu_limit(g, u, limit);
    return or_silu(g) * u;
}

/* [KQ] moe_glu_gather_kq with act = 0 ('silu') or 1 ('gelu', tanh
 * approximation): for each token t and slot r with e = ids[t,r]:
 * g = W_gate[e] x_t, u = W_up[e] x_t, h = act(g) * u, giving h[T, top_k, n].
 * Also returns g, u and their |.|-sums sg, su (any of the extra outputs may
 * be NULL).  Invalid ids poison h as or_routing_poisons_all describes (below
 * 32 tokens only the h row of an out-of-range id). */
/* [KQ] moe_glu_gather_kq (act 0 'silu', 1 'gelu', 2 'silu_limit' with
 * limit > 0) and moe_glu_gather_shexp_kq: for each token t and slot r,
 * g = W_gate[e] x_t, u = W_up[e] x_t, h = act(g, u), giving h[T, S, n].
 * Without a shared expert S = top_k and e = ids[t, r]; with one (shexp_gate
 * and shexp_up non-NULL, single-expert matrices [n, k/QK blocks]) S = top_k
 * + 1 and the last slot of every token uses the shared expert's weights.
 * Also returns g, u and their |.|-sums sg, su (any extra output may be NULL).
 * Invalid routed ids poison h by the rule of or_routing_poisons_all (the
 * shared slot is never invalid; below 32 tokens only an out-of-range routed
 * id's row is NaN). */
int or_moe_glu_ex(int type, const uint8_t* gate_w, const uint8_t* up_w, int64_t n_experts,
                  int64_t n, int64_t k, int64_t expert_stride, const uint8_t* shexp_gate,
                  const uint8_t* shexp_up, const void* x, int x_dt, const uint32_t* ids, int64_t T,
                  int64_t top_k, int act, double limit, double* h, double* g, double* u,
                  double* sg, double* su) {
    if (act < 0 || act > 2) return -3;
    if (act == 2 && !(limit > 0.0)) return -4;
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
    int shexp = shexp_gate && shexp_up;
    int64_t S = top_k + shexp;
    if (or_routing_poisons_all(ids, T, top_k, n_experts)) {
        fill_nan(h, T * S * n);
        fill_nan(g, T * S * n);
        fill_nan(u, T * S * n);
        fill_nan(sg, T * S * n);
        fill_nan(su, T * S * n);
        return 0;
    }
#pragma omp parallel
    {
        double* rg = (double*)malloc(sizeof(double) * k);
        double* ru = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t ts = 0; ts < T * S; ++ts) {
            int64_t t = ts / S, r = ts % S;
            int shared = shexp && r == top_k;
            uint32_t e = shared ? 0u : ids[t * top_k + r];
            const uint8_t* wg = shared ? shexp_gate : gate_w + (int64_t)e * expert_stride;
            const uint8_t* wu = shared ? shexp_up : up_w + (int64_t)e * expert_stride;
            for (int64_t j = 0; j < n; ++j) {
                int64_t o = ts * n + j;
                if (!shared && (int64_t)e >= n_experts) {
                    h[o] = NAN;
                    if (g) g[o] = NAN;
                    if (u) u[o] = NAN;
                    if (sg) sg[o] = NAN;
                    if (su) su[o] = NAN;
                    continue;
                }
                decode_row(type, wg, j, k, rg);
                decode_row(type, wu, j, k, ru);
                double ag = 0, au = 0, mg = 0, mu = 0;
                for (int64_t c = 0; c < k; ++c) {
                    double xv = act_value(x, x_dt, t * k + c);
                    ag += xv * rg[c];
                    mg += fabs(xv * rg[c]);
                    au += xv * ru[c];
                    mu += fabs(xv * ru[c]);
                }
                h[o] = glu_value(act, ag, au, limit);
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

/* The same without a shared expert or a limit (act 0 or 1). */
int or_moe_glu(int type, const uint8_t* gate_w, const uint8_t* up_w, int64_t n_experts,
               int64_t n, int64_t k, int64_t expert_stride, const void* x, int x_dt,
               const uint32_t* ids, int64_t T, int64_t top_k, int act, double* h, double* g,
               double* u, double* sg, double* su) {
    if (act != 0 && act != 1) return -3;
    return or_moe_glu_ex(type, gate_w, up_w, n_experts, n, k, expert_stride, NULL, NULL, x, x_dt,
                         ids, T, top_k, act, 0.0, h, g, u, sg, su);
}

/* [KQ] gather_qmv_mix_kq: the mixed down projection with the shared expert
 * as the last of S = top_k + 1 slots: x is [T, S, k], scores [T, S] and
 * y[t] = sum over slots r in order of scores[t,r] * (W_r x[t,r]) with W_r =
 * W[ids[t,r]] for r < top_k and the shared matrix shexp_w ([n, k/QK
 * blocks]) for r = top_k.  s[t] = sum_r |scores| * sum_c |W_r x|.  Invalid
 * routed ids poison as in or_qmm_id. */
int or_qmm_id_mix_shexp(int type, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                        int64_t expert_stride, const uint8_t* shexp_w, const void* x, int x_dt,
                        const uint32_t* ids, int64_t T, int64_t top_k, const float* scores,
                        double* y, double* s) {
    int qk = or_qk(type);
    if (!qk || k % qk) return -1;
    int64_t S = top_k + 1;
    if (or_routing_poisons_all(ids, T, top_k, n_experts)) {
        fill_nan(y, T * n);
        fill_nan(s, T * n);
        return 0;
    }
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            int bad = 0;
            for (int64_t r = 0; r < top_k; ++r) bad |= (int64_t)ids[t * top_k + r] >= n_experts;
            for (int64_t j = 0; j < n; ++j) {
                y[t * n + j] = bad ? NAN : 0.0;
                if (s) s[t * n + j] = bad ? NAN : 0.0;
            }
            if (bad) continue;
            for (int64_t r = 0; r < S; ++r) {
                const uint8_t* wr = r == top_k ? shexp_w : w + (int64_t)ids[t * top_k + r] * expert_stride;
                double wt = (double)scores[t * S + r];
                for (int64_t j = 0; j < n; ++j) {
                    decode_row(type, wr, j, k, row);
                    double acc = 0.0, mag = 0.0;
                    for (int64_t c = 0; c < k; ++c) {
                        double tv = act_value(x, x_dt, (t * S + r) * k + c) * row[c];
                        acc += tv;
                        mag += fabs(tv);
                    }
                    y[t * n + j] += wt * acc;
                    if (s) s[t * n + j] += fabs(wt) * mag;
                }
            }
        }
        free(row);
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
    if (or_routing_poisons_all(ids, T, top_k, n_experts)) {
        fill_nan(out, T * hidden);
        fill_nan(s_out, T * hidden);
        return 0;
    }
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
/* Encoders: float weights -> block bytes                              */
/* ------------------------------------------------------------------ */
/* [KQ] quantize encodes float weights [rows, k] (k a multiple of the block
 * size) into the wire bytes of a codec, with an optional importance vector
 * of length k that steers the K-quant encoder; [TQ1] "Bounds safety": code
 * legality is established at conversion.  The pages fix the contract, not an
 * encoder; the encoders below are the plain readings stated with each.  All
 * arithmetic is binary32 (float variables, this file is compiled without
 * contraction into fused multiply-adds), divisions and square-free products
 * correctly rounded, rintf rounds to nearest even, and every sum runs in
 * index order, so a faithful implementation elsewhere produces the same
 * bytes.  Weights and importances must be finite (importances >= 0). */

static float act_f32(const void* x, int dt, int64_t i) { return (float)act_value(x, dt, i); }

/* binary32 -> fp16 bits, round to nearest even, with magnitudes past the
 * fp16 range clamped to 65504 (scales are never infinite). */
static uint16_t scale_to_half(float v) {
    if (v > 65504.0f) v = 65504.0f;
    return or_float_to_half_rne(v);
}

static float clampf(float v, float lo, float hi) { return v < lo ? lo : v > hi ? hi : v; }

/* Q8_0: d = fp16(max|w| / 127); q = clamp(rint(w * (1/d)), -127, 127). */
static void encode_q8_0(const float* w, uint8_t* blk) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    uint16_t dh = scale_to_half(amax / 127.0f);
    float d = (float)or_half_to_double(dh);
    float inv = d > 0.0f ? 1.0f / d : 0.0f;
    blk[0] = (uint8_t)(dh & 0xff);
    blk[1] = (uint8_t)(dh >> 8);
    for (int i = 0; i < 32; ++i) {
        float q = clampf(rintf(w[i] * inv), -127.0f, 127.0f);
        blk[2 + i] = (uint8_t)(int8_t)q;
    }
}

/* TQ1_G128: s = fp16(max|w|) over the 128 weights (absmax, so a decoded block
 * encodes back to its own bytes); trit t = clamp(rint(w * (1/s)), -1, 1),
 * stored as the base-3 digit t + 1: column c < 125 is digit c mod 5 of code
 * byte c / 5, columns 125..127 digits 0..2 of the tail byte (place values 1,
 * 3, 9, 27, 81); the scale's fp16 bits follow. */
static void encode_tq1(const float* w, uint8_t* blk) {
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) {
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    uint16_t sh = scale_to_half(amax);
    float sv = (float)or_half_to_double(sh);
    float inv = sv > 0.0f ? 1.0f / sv : 0.0f;
    for (int b = 0; b < 26; ++b) blk[b] = 0;
    for (int c = 0; c < 128; ++c) {
        int t = (int)clampf(rintf(w[c] * inv), -1.0f, 1.0f);
        int slot = c < 125 ? c / 5 : 25;
        int digit = c < 125 ? c - 5 * slot : c - 125;
        int p = 1;
        for (int i = 0; i < digit; ++i) p *= 3;
        blk[slot] = (uint8_t)(blk[slot] + (t + 1) * p);
    }
    blk[26] = (uint8_t)(sh & 0xff);
    blk[27] = (uint8_t)(sh >> 8);
}

/* Q4_K.  Per sub-block j of 32 weights: lo = min(0, min w), hi = max w,
 * range scale r_j = (hi - lo) / 15 and min mn_j = -lo, so that the 16 levels
 * lo + r_j q (q = 0..15) span [lo, hi].  With an importance vector the range
 * is the best of eight shrunk candidates r_j (16 - t) / 16 (t = 0..7, the
 * levels anchored at lo): the one with the smallest importance-weighted sum
 * of squared errors sum_i imp_i (w_i - (lo + s q_i))^2, q_i the nearest level
 * clamped to 0..15, ties to the smaller t.  Then d = fp16(max_j r_j / 63),
 * dmin = fp16(max_j mn_j / 63), sc_j = clamp(rint(r_j / d), 0, 63), m_j =
 * clamp(rint(mn_j / dmin), 0, 63), and each weight takes q = clamp(rint((w +
 * dmin m_j) / (d sc_j)), 0, 15) -- the nearest point of the grid the block
 * decodes to (0 where d sc_j = 0). */
static float q4k_level_err(const float* w, const float* imp, float lo, float s) {
    float e = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float q = s > 0.0f ? clampf(rintf((w[i] - lo) / s), 0.0f, 15.0f) : 0.0f;
        float r = w[i] - (lo + s * q);
        e = e + imp[i] * (r * r);
    }
    return e;
}

static void encode_q4k(const float* w, const float* imp, uint8_t* blk) {
    float rng[8], mn[8];
    for (int j = 0; j < 8; ++j) {
        const float* x = w + 32 * j;
        float lo = 0.0f, hi = x[0];
        for (int i = 0; i < 32; ++i) {
            if (x[i] < lo) lo = x[i];
            if (x[i] > hi) hi = x[i];
        }
        float r = (hi - lo) / 15.0f;
        if (imp) {
            float best = 0.0f;
            int best_t = 0;
            for (int t = 0; t < 8; ++t) {
                float s = (r * (float)(16 - t)) * 0.0625f;
                float e = q4k_level_err(x, imp + 32 * j, lo, s);
                if (t == 0 || e < best) {
                    best = e;
                    best_t = t;
                }
            }
            r = (r * (float)(16 - best_t)) * 0.0625f;
        }
        rng[j] = r;
        mn[j] = -lo;
    }
    float rmax = 0.0f, mmax = 0.0f;
    for (int j = 0; j < 8; ++j) {
        if (rng[j] > rmax) rmax = rng[j];
        if (mn[j] > mmax) mmax = mn[j];
    }
    uint16_t dh = scale_to_half(rmax / 63.0f), mh = scale_to_half(mmax / 63.0f);
    float d = (float)or_half_to_double(dh), dmin = (float)or_half_to_double(mh);
    int sc[8], m[8];
    for (int j = 0; j < 8; ++j) {
        sc[j] = d > 0.0f ? (int)clampf(rintf(rng[j] / d), 0.0f, 63.0f) : 0;
        m[j] = dmin > 0.0f ? (int)clampf(rintf(mn[j] / dmin), 0.0f, 63.0f) : 0;
    }
    blk[0] = (uint8_t)(dh & 0xff);
    blk[1] = (uint8_t)(dh >> 8);
    blk[2] = (uint8_t)(mh & 0xff);
    blk[3] = (uint8_t)(mh >> 8);
    /* the 6-bit packing that or_q4k_scale_min reads */
    uint8_t* S = blk + 4;
    for (int j = 0; j < 4; ++j) {
        S[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        S[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        S[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    uint8_t* Q = blk + 16;
    for (int c = 0; c < 4; ++c) {
        for (int l = 0; l < 32; ++l) {
            int qq[2];
            for (int h = 0; h < 2; ++h) {
                int j = 2 * c + h;
                float step = d * (float)sc[j];
                float off = dmin * (float)m[j];
                float x = w[64 * c + 32 * h + l];
                qq[h] = step > 0.0f ? (int)clampf(rintf((x + off) / step), 0.0f, 15.0f) : 0;
            }
            Q[32 * c + l] = (uint8_t)(qq[0] | (qq[1] << 4));
        }
    }
}

/* Encode rows x k weights of dtype w_dt (f32, f16 bits or bf16 bits) into
 * out (rows x k/QK blocks).  imatrix: NULL or k floats (Q4_K only). */
int or_quantize(int type, const void* w, int w_dt, int64_t rows, int64_t k, const float* imatrix,
                uint8_t* out) {
    int qk = or_qk(type), bb = or_block_bytes(type);
    if (!qk || k % qk) return -1;
    if (type != OR_Q4_K && type != OR_Q8_0 && type != OR_TQ1) return -1;  /* no encoder */
    int64_t nb = k / qk;
#pragma omp parallel
    {
        float* blockw = (float*)malloc(sizeof(float) * qk);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t b = 0; b < nb; ++b) {
                for (int i = 0; i < qk; ++i) blockw[i] = act_f32(w, w_dt, r * k + b * qk + i);
                uint8_t* blk = out + (r * nb + b) * bb;
                if (type == OR_Q4_K) encode_q4k(blockw, imatrix ? imatrix + b * qk : NULL, blk);
                else if (type == OR_Q8_0) encode_q8_0(blockw, blk);
                else encode_tq1(blockw, blk);
            }
        }
        free(blockw);
    }
    return 0;
}

/* [TQ1] "Bounds safety": number of illegal code bytes (a full slot above 242,
 * a tail above 26) in rows x k/128 blocks. */
int64_t or_tq1_illegal(const uint8_t* w, int64_t rows, int64_t k) {
    int64_t nb = rows * (k / 128), bad = 0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = w + b * 28;
        for (int s = 0; s < 25; ++s) bad += blk[s] > 242;
        bad += blk[25] > 26;
    }
    return bad;
}

/* ------------------------------------------------------------------ */
/* Expert routing schedule (integer work)                              */
/* ------------------------------------------------------------------ */

/* [KQ] expert_tile_map / [MID] expert regroup.  Routed rows are the flat
 * (token, slot) indices i = t*top_k + r of n_tokens x top_k ids.  counts[e]
 * is the number of rows with ids[i] == e; offsets is its exclusive prefix sum
 * (offsets[E] = number of rows with an in-range id); perm lists those rows
 * grouped by expert in ascending expert order, and in ascending i within an
 * expert (a stable sort).  Rows with an id >= E are not placed.  *n_invalid
 * counts them, plus (from 32 tokens on, the matrix-matrix rule of
 * or_routing_poisons_all) every row whose id repeats an earlier slot of the
 * same token.  The tile map cuts each expert's segment into tiles of at most
 * tile_rows rows, only the last of which may be partial: (expert, row_start,
 * num_rows), in expert order -- and is empty when the matrix-matrix rule
 * poisons the whole operation (no weights are read).  Returns the number of
 * tiles, or -1 if max_tiles is too small. */
int64_t or_route(const uint32_t* ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                 int64_t tile_rows, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* tiles, int64_t max_tiles, int64_t* n_invalid) {
    int64_t n_rows = n_tokens * top_k;
    int64_t bad = 0;
    for (int64_t e = 0; e < n_experts; ++e) counts[e] = 0;
    for (int64_t i = 0; i < n_rows; ++i) {
        if ((int64_t)ids[i] < n_experts)
            counts[ids[i]]++;
        else
            bad++;
    }
    if (n_tokens >= OR_MM_ID_MIN_TOKENS) {
        for (int64_t t = 0; t < n_tokens; ++t)
            for (int64_t r = 0; r < top_k; ++r) {
                uint32_t e = ids[t * top_k + r];
                if ((int64_t)e >= n_experts) continue;
                for (int64_t q = 0; q < r; ++q)
                    if (ids[t * top_k + q] == e) {
                        bad++;
                        break;
                    }
            }
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int64_t e = 0; e < n_experts; ++e)
        for (int64_t i = 0; i < n_rows; ++i)
            if ((int64_t)ids[i] == e) perm[pos++] = (int32_t)i;
    if (n_invalid) *n_invalid = bad;
    if (n_tokens >= OR_MM_ID_MIN_TOKENS && bad > 0) return 0;
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
    return nt;
}
