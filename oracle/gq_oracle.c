/*
 * gq_oracle.c -- plain, slow, CPU reference for products against ggml
 * block-quantized weights (Q4_0, Q4_K, Q5_K, Q6_K).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the GPU library and includes nothing from it.
 *
 * What it follows
 *  - "GGUF in transformers" (Hugging Face blog), section "Reusing ggml's Metal
 *    kernels", kernel table, row "ggml-quantization": the operation is a matrix
 *    product that reads the packed quantized weights directly, including only
 *    the selected experts of an MoE model.  Section "What is the GGUF file
 *    format?" and its size table name the Q4_K_M / Q6_K / Q5_K_M variants.
 *  - The block formats themselves are the public ggml ones; the pages name
 *    them but print no layout.  The reading used here (sizes, field order,
 *    bit positions, dequantisation formulas) is written out next to each
 *    function and listed as a reading in the design notes:
 *      Q4_0: 32 weights / 18 B,  w = d * (q - 8)
 *      Q4_K: 256 weights / 144 B, w = (d * sc) * q - dmin * m
 *      Q6_K: 256 weights / 210 B, w = (d * sc) * (q - 32)
 *      Q5_K: 256 weights / 176 B, w = (d * sc) * q - dmin * m (q 5-bit)
 *    The Q5_K layout is the least supported reading: the pages give only the
 *    Q5_K_M variant's file size; its pins are the size table and the
 *    reduction to Q4_K when the fifth-bit plane is zero.
 *  - Each factor is converted to fp32 first and the formula is evaluated left
 *    to right in fp32 (the only rounding step is Q4_K's subtraction; every
 *    product here is exact in fp32).  Dot products accumulate in fp64, one term
 *    at a time, in increasing k.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (see oracle/oracle.py).  No OpenMP, no SIMD intrinsics, no blocking.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q4_0 1
#define ORC_Q4_K 2
#define ORC_Q6_K 3
#define ORC_Q5_K 4

/* ---------------------------------------------------------------- fp16 ---- */

/* IEEE 754 binary16 -> binary32, by the definition of the format:
 * sign 1 bit, exponent 5 bits (bias 15), fraction 10 bits; exponent 0 is a
 * subnormal (fraction * 2^-24), exponent 31 is Inf/NaN. */
static float orc_half_to_float(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);
    }
    /* every finite binary16 value is exactly representable in binary32 */
    return (float)(sign ? -v : v);
}

static uint16_t orc_rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------ formats ---- */

int oracle_block_info(int type, int32_t* elems, int32_t* bytes) {
    switch (type) {
    case ORC_Q4_0: *elems = 32;  *bytes = 2 + 16;             return 0;
    case ORC_Q4_K: *elems = 256; *bytes = 2 + 2 + 12 + 128;   return 0;
    case ORC_Q6_K: *elems = 256; *bytes = 128 + 64 + 16 + 2;  return 0;
    case ORC_Q5_K: *elems = 256; *bytes = 2 + 2 + 12 + 32 + 128; return 0;
    default: return -1;
    }
}

/* Q4_0 block: d (fp16) at byte 0, then 16 bytes of 4-bit quants.  Weight i
 * (0..15) is the low nibble of quant byte i, weight i (16..31) the high nibble
 * of quant byte i-16.  w = d * (q - 8). */
static void orc_dequant_q4_0(const uint8_t* b, float* w) {
    float d = orc_half_to_float(orc_rd16(b));
    const uint8_t* qs = b + 2;
    for (int i = 0; i < 32; ++i) {
        int q = (i < 16) ? (qs[i] & 0x0f) : (qs[i - 16] >> 4);
        w[i] = d * (float)(q - 8);
    }
}

/* Q4_K 6-bit (scale, min) pair s (0..7) from the 12 packed scale bytes.
 * Pairs 0..3: low 6 bits of byte s (scale) and of byte s+4 (min).
 * Pairs 4..7: low nibble of byte s+4 plus the top two bits of byte s-4 as bits
 * 4..5 (scale); high nibble of byte s+4 plus the top two bits of byte s as
 * bits 4..5 (min). */
static void orc_q4k_scale_min(const uint8_t* sb, int s, int* sc, int* m) {
    if (s < 4) {
        *sc = sb[s] & 63;
        *m = sb[s + 4] & 63;
    } else {
        *sc = (sb[s + 4] & 0x0f) | ((sb[s - 4] >> 6) << 4);
        *m = (sb[s + 4] >> 4) | ((sb[s] >> 6) << 4);
    }
}

/* Q4_K super-block: d (fp16) @0, dmin (fp16) @2, 12 scale bytes @4, 128 quant
 * bytes @16.  Weights come in four chunks of 64; chunk c uses quant bytes
 * 32c..32c+31.  Within a chunk, weight j < 32 is the low nibble of byte 32c+j
 * (sub-block 2c), weight j >= 32 the high nibble of byte 32c+j-32 (sub-block
 * 2c+1).  w = (d * sc) * q - dmin * m with the sub-block's (sc, m). */
static void orc_dequant_q4_k(const uint8_t* b, float* w) {
    float d = orc_half_to_float(orc_rd16(b));
    float dmin = orc_half_to_float(orc_rd16(b + 2));
    const uint8_t* sb = b + 4;
    const uint8_t* qs = b + 16;
    for (int i = 0; i < 256; ++i) {
        int c = i / 64, j = i % 64;
        int sub = (j < 32) ? 2 * c : 2 * c + 1;
        int q = (j < 32) ? (qs[32 * c + j] & 0x0f) : (qs[32 * c + j - 32] >> 4);
        int sc, m;
        orc_q4k_scale_min(sb, sub, &sc, &m);
        float a = d * (float)sc;
        float p = a * (float)q;
        float mm = dmin * (float)m;
        w[i] = p - mm;
    }
}

/* Q6_K super-block: 128 bytes of low 4-bit parts (ql) @0, 64 bytes of high
 * 2-bit parts (qh) @128, 16 int8 scales @192, d (fp16) @208.  Weight i: half
 * h = i/128, r = i%128, group g = r/32, lane l = r%32.  Low four bits: byte
 * ql[64h + l + 32*(g%2)], low nibble for g < 2, high nibble for g >= 2.  High
 * two bits: bits 2g..2g+1 of qh[32h + l].  q = low | high << 4 (0..63).
 * Scale index 8h + r/16 (one int8 scale per 16 weights).
 * w = (d * sc) * (q - 32). */
static void orc_dequant_q6_k(const uint8_t* b, float* w) {
    const uint8_t* ql = b;
    const uint8_t* qh = b + 128;
    const int8_t* sc = (const int8_t*)(b + 192);
    float d = orc_half_to_float(orc_rd16(b + 208));
    for (int i = 0; i < 256; ++i) {
        int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
        int lbyte = ql[64 * h + l + 32 * (g % 2)];
        int low = (g < 2) ? (lbyte & 0x0f) : (lbyte >> 4);
        int high = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = low | (high << 4);
        float a = d * (float)sc[8 * h + r / 16];
        w[i] = a * (float)(q - 32);
    }
}

/* Q5_K super-block: Q4_K's header (d, dmin, the same 12 scale bytes) @0, then
 * 32 bytes of fifth bits (qh) @16, then Q4_K's 128 quant bytes @48.  Weight i
 * (chunk c = i/64, j = i%64) takes its low four bits exactly as in Q4_K and
 * its fifth bit from bit 2c (j < 32) or 2c+1 (j >= 32) of qh[j % 32]:
 * q = low | fifth << 4 (0..31).  w = (d * sc) * q - dmin * m. */
static void orc_dequant_q5_k(const uint8_t* b, float* w) {
    float d = orc_half_to_float(orc_rd16(b));
    float dmin = orc_half_to_float(orc_rd16(b + 2));
    const uint8_t* sb = b + 4;
    const uint8_t* qh = b + 16;
    const uint8_t* qs = b + 48;
    for (int i = 0; i < 256; ++i) {
        int c = i / 64, j = i % 64;
        int upper = j >= 32;
        int sub = 2 * c + upper;
        int low = upper ? (qs[32 * c + j - 32] >> 4) : (qs[32 * c + j] & 0x0f);
        int fifth = (qh[j % 32] >> sub) & 1;
        int q = low | (fifth << 4);
        int sc, m;
        orc_q4k_scale_min(sb, sub, &sc, &m);
        float a = d * (float)sc;
        float p = a * (float)q;
        float mn = dmin * (float)m;
        w[i] = p - mn;
    }
}

int oracle_dequant(int type, const uint8_t* blocks, int64_t n_blocks, float* out) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes)) return -1;
    for (int64_t i = 0; i < n_blocks; ++i) {
        const uint8_t* b = blocks + i * bytes;
        float* w = out + i * elems;
        if (type == ORC_Q4_0) orc_dequant_q4_0(b, w);
        else if (type == ORC_Q4_K) orc_dequant_q4_k(b, w);
        else if (type == ORC_Q5_K) orc_dequant_q5_k(b, w);
        else orc_dequant_q6_k(b, w);
    }
    return 0;
}

/* Row n of a matrix with K inputs: K/elems consecutive blocks, no padding. */
static int orc_dequant_row(int type, const uint8_t* W, int64_t n, int64_t K, float* row) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes)) return -1;
    int64_t nb = K / elems;
    return oracle_dequant(type, W + n * nb * bytes, nb, row);
}

/* ------------------------------------------------------------- matvec ---- */

/* y[b][n] = sum_k w[n][k] * x[b][k], every product and the running sum in
 * fp64, k increasing.  sumabs[b][n] = sum_k |w[n][k] * x[b][k]| (for the
 * per-element tolerance, which the caller scales).  x is [batch][K] fp32;
 * y and sumabs are [batch][N] fp64.  Rows are independent; the optional row
 * range lets a caller time or check a subset. */
int oracle_matvec_rows(int type, const uint8_t* W, int64_t N, int64_t K,
                       const float* x, int32_t batch, int64_t row0, int64_t row1,
                       double* y, double* sumabs) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes) || K % elems || row0 < 0 || row1 > N) return -1;
    float* row = (float*)malloc(sizeof(float) * (size_t)(K ? K : 1));
    if (!row) return -2;
    for (int64_t n = row0; n < row1; ++n) {
        orc_dequant_row(type, W, n, K, row);
        for (int32_t b = 0; b < batch; ++b) {
            const float* xb = x + (int64_t)b * K;
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)row[k] * (double)xb[k];
                s += p;
                a += fabs(p);
            }
            y[(int64_t)b * N + n] = s;
            sumabs[(int64_t)b * N + n] = a;
        }
    }
    free(row);
    return 0;
}

int oracle_matvec(int type, const uint8_t* W, int64_t N, int64_t K, const float* x,
                  int32_t batch, double* y, double* sumabs) {
    return oracle_matvec_rows(type, W, N, K, x, batch, 0, N, y, sumabs);
}

/* ---------------------------------------------------------- matvec_id ---- */

/* Routed experts ("the selected experts in an MoE model").  experts is
 * [n_experts][N][K/elems blocks]; ids is [n_tokens][top_k].  x is [n_tokens][K]
 * when x_per_slot == 0 (every slot of a token reads the token's vector) or
 * [n_tokens][top_k][K] when x_per_slot == 1 (each slot has its own input, as
 * for a down projection).
 *  route_w == NULL: y and sumabs are [n_tokens][top_k][N],
 *      y[t][j][n] = sum_k w_{ids[t][j]}[n][k] * x_{t,j}[k].
 *  route_w != NULL: y and sumabs are [n_tokens][N],
 *      y[t][n] = sum_{j} route_w[t][j] * (sum_k w_{ids[t][j]}[n][k] * x_{t,j}[k]),
 *      j increasing, all in fp64; sumabs[t][n] = sum_j |route_w[t][j]| *
 *      sum_k |w * x|.
 * An id outside [0, n_experts) contributes zero to y and to sumabs. */
int oracle_matvec_id(int type, const uint8_t* experts, int32_t n_experts, int64_t N, int64_t K,
                     const int32_t* ids, int32_t n_tokens, int32_t top_k,
                     const float* x, int32_t x_per_slot, const float* route_w,
                     double* y, double* sumabs) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes) || K % elems) return -1;
    int64_t expert_bytes = N * (K / elems) * bytes;
    float* row = (float*)malloc(sizeof(float) * (size_t)(K ? K : 1));
    if (!row) return -2;
    if (route_w) {
        memset(y, 0, sizeof(double) * (size_t)(n_tokens * N));
        memset(sumabs, 0, sizeof(double) * (size_t)(n_tokens * N));
    }
    for (int32_t t = 0; t < n_tokens; ++t) {
        for (int32_t j = 0; j < top_k; ++j) {
            int32_t e = ids[(int64_t)t * top_k + j];
            const float* xv = x_per_slot ? x + ((int64_t)t * top_k + j) * K : x + (int64_t)t * K;
            for (int64_t n = 0; n < N; ++n) {
                double s = 0.0, a = 0.0;
                if (e >= 0 && e < n_experts) {
                    orc_dequant_row(type, experts + (int64_t)e * expert_bytes, n, K, row);
                    for (int64_t k = 0; k < K; ++k) {
                        double p = (double)row[k] * (double)xv[k];
                        s += p;
                        a += fabs(p);
                    }
                }
                if (route_w) {
                    double r = (double)route_w[(int64_t)t * top_k + j];
                    y[(int64_t)t * N + n] += r * s;
                    sumabs[(int64_t)t * N + n] += fabs(r) * a;
                } else {
                    y[((int64_t)t * top_k + j) * N + n] = s;
                    sumabs[((int64_t)t * top_k + j) * N + n] = a;
                }
            }
        }
    }
    free(row);
    return 0;
}

/* ------------------------------------------------------------- matmul ---- */

/* Prefill product Y[m][n] = sum_k X[m][k] * w[n][k] for the listed rows m
 * only (X is [M][ldx] fp32, the caller expands bf16 exactly).  Output rows are
 * written densely: y[i][n] for rows[i].  fp64 as in oracle_matvec. */
int oracle_matmul_rows(int type, const uint8_t* W, int64_t N, int64_t K,
                       const float* X, int64_t ldx, const int64_t* rows, int64_t n_rows,
                       double* y, double* sumabs) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes) || K % elems) return -1;
    float* wrow = (float*)malloc(sizeof(float) * (size_t)(K ? K : 1));
    if (!wrow) return -2;
    for (int64_t n = 0; n < N; ++n) {
        orc_dequant_row(type, W, n, K, wrow);
        for (int64_t i = 0; i < n_rows; ++i) {
            const float* xr = X + rows[i] * ldx;
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)xr[k] * (double)wrow[k];
                s += p;
                a += fabs(p);
            }
            y[i * N + n] = s;
            sumabs[i * N + n] = a;
        }
    }
    free(wrow);
    return 0;
}

/* Same product for the listed columns n only: y[m][i] for cols[i], all M
 * rows (y is [M][n_cols]). */
int oracle_matmul_cols(int type, const uint8_t* W, int64_t N, int64_t K,
                       const float* X, int64_t M, int64_t ldx, const int64_t* cols, int64_t n_cols,
                       double* y, double* sumabs) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes) || K % elems) return -1;
    float* wrow = (float*)malloc(sizeof(float) * (size_t)(K ? K : 1));
    if (!wrow) return -2;
    for (int64_t i = 0; i < n_cols; ++i) {
        if (cols[i] < 0 || cols[i] >= N) { free(wrow); return -1; }
        orc_dequant_row(type, W, cols[i], K, wrow);
        for (int64_t m = 0; m < M; ++m) {
            const float* xr = X + m * ldx;
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)xr[k] * (double)wrow[k];
                s += p;
                a += fabs(p);
            }
            y[m * n_cols + i] = s;
            sumabs[m * n_cols + i] = a;
        }
    }
    free(wrow);
    return 0;
}

/* Checksum of the whole product without forming it (Freivalds): for sign
 * vectors u (length M) and v (length N),
 *   u^T Y v = sum_k (sum_m u_m X[m][k]) * (sum_n v_n w[n][k]),
 * and the tolerance term
 *   sum_k (sum_m |u_m| |X[m][k]|) * (sum_n |v_n| |w[n][k]|)
 * bounds sum_{m,n} |u_m| |v_n| sum_k |X[m][k] w[n][k]|.  Both in fp64, O(MK+NK). */
int oracle_matmul_checksum(int type, const uint8_t* W, int64_t N, int64_t K,
                           const float* X, int64_t M, int64_t ldx,
                           const double* u, const double* v,
                           double* checksum, double* tolerance_term) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes) || K % elems) return -1;
    double* xu = (double*)calloc((size_t)(K ? K : 1), sizeof(double));
    double* xa = (double*)calloc((size_t)(K ? K : 1), sizeof(double));
    double* wv = (double*)calloc((size_t)(K ? K : 1), sizeof(double));
    double* wa = (double*)calloc((size_t)(K ? K : 1), sizeof(double));
    float* wrow = (float*)malloc(sizeof(float) * (size_t)(K ? K : 1));
    if (!xu || !xa || !wv || !wa || !wrow) { free(xu); free(xa); free(wv); free(wa); free(wrow); return -2; }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double xe = (double)X[m * ldx + k];
            xu[k] += u[m] * xe;
            xa[k] += fabs(u[m]) * fabs(xe);
        }
    for (int64_t n = 0; n < N; ++n) {
        orc_dequant_row(type, W, n, K, wrow);
        for (int64_t k = 0; k < K; ++k) {
            wv[k] += v[n] * (double)wrow[k];
            wa[k] += fabs(v[n]) * fabs((double)wrow[k]);
        }
    }
    double c = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        c += xu[k] * wv[k];
        t += xa[k] * wa[k];
    }
    *checksum = c;
    *tolerance_term = t;
    free(xu); free(xa); free(wv); free(wa); free(wrow);
    return 0;
}

/* -------------------------------------------------- round-to-nearest ---- */

/* Round-to-nearest quantisers, only used to make round-trip test data (the
 * pages give no quantiser).  Each picks a per-block (or per-sub-block) grid
 * and rounds every value to its nearest grid point; fp16 fields are stored
 * round-to-nearest-even. */

static uint16_t orc_float_to_half(float f) {
    /* round-to-nearest-even binary32 -> binary16 via fp64 arithmetic on the
     * value (no bit tricks): scale into the 11-bit significand grid. */
    if (f != f) return 0x7e00;
    double a = fabs((double)f);
    uint16_t sign = (f < 0 || (f == 0 && signbit(f))) ? 0x8000 : 0;
    if (a == 0) return sign;
    if (a >= 65520.0) return sign | 0x7c00; /* rounds to Inf */
    int e;
    frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;          /* a in [2^ex, 2^(ex+1)) */
    if (ex < -14) ex = -14;  /* subnormal grid step 2^-24 */
    double step = ldexp(1.0, ex - 10);
    double q = nearbyint(a / step); /* default rounding: to nearest, ties even */
    double r = q * step;
    /* re-encode r exactly */
    if (r >= 65536.0) return sign | 0x7c00;
    if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
    frexp(r, &e);
    ex = e - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, ex - 10) - 1024.0);
    return sign | (uint16_t)((ex + 15) << 10) | frac;
}

static void orc_wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }

static int orc_clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Q4_0: d = amax / 7 (stored fp16), q = clamp(round(x / d) + 8, 0, 15).  The
 * round uses the stored (fp16-rounded) d, so every value lands on the nearest
 * point of the grid d * {-8..7} that it can reach. */
static void orc_quant_q4_0(const float* x, uint8_t* b) {
    float amax = 0.f;
    for (int i = 0; i < 32; ++i) if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    uint16_t dh = orc_float_to_half(amax / 7.0f);
    float d = orc_half_to_float(dh);
    orc_wr16(b, dh);
    uint8_t* qs = b + 2;
    memset(qs, 0, 16);
    for (int i = 0; i < 32; ++i) {
        int q = 8;
        if (d > 0) q = orc_clampi((int)nearbyint((double)x[i] / (double)d) + 8, 0, 15);
        if (i < 16) qs[i] |= (uint8_t)q;
        else qs[i - 16] |= (uint8_t)(q << 4);
    }
}

/* Q4_K: per sub-block of 32 an affine grid lo + step * {0..15} with
 * step = (max - lo) / 15 and lo = min(0, min x).  The super-block stores
 * d = max step / 63 and dmin = max(-lo) / 63 in fp16; each sub-block stores
 * sc = round(step / d), m = round(-lo / dmin) in 6 bits.  Values are then
 * rounded to the nearest point of the grid actually stored:
 * (d*sc) * q - dmin*m, q in 0..15. */
static void orc_quant_q4_k(const float* x, uint8_t* b) {
    float step[8], neg_lo[8];
    float smax = 0.f, mmax = 0.f;
    for (int s = 0; s < 8; ++s) {
        float lo = 0.f, hi = 0.f;
        for (int i = 0; i < 32; ++i) {
            float v = x[32 * s + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        step[s] = (hi - lo) / 15.0f;
        neg_lo[s] = -lo;
        if (step[s] > smax) smax = step[s];
        if (neg_lo[s] > mmax) mmax = neg_lo[s];
    }
    uint16_t dh = orc_float_to_half(smax / 63.0f), mh = orc_float_to_half(mmax / 63.0f);
    float d = orc_half_to_float(dh), dmin = orc_half_to_float(mh);
    orc_wr16(b, dh);
    orc_wr16(b + 2, mh);
    int sc[8], m[8];
    for (int s = 0; s < 8; ++s) {
        sc[s] = d > 0 ? orc_clampi((int)nearbyint((double)step[s] / (double)d), 0, 63) : 0;
        m[s] = dmin > 0 ? orc_clampi((int)nearbyint((double)neg_lo[s] / (double)dmin), 0, 63) : 0;
    }
    uint8_t* sb = b + 4;
    memset(sb, 0, 12);
    for (int s = 0; s < 4; ++s) {
        sb[s] = (uint8_t)((sc[s] & 63) | ((sc[s + 4] >> 4) << 6));
        sb[s + 4] = (uint8_t)((m[s] & 63) | ((m[s + 4] >> 4) << 6));
        sb[s + 8] = (uint8_t)((sc[s + 4] & 15) | ((m[s + 4] & 15) << 4));
    }
    uint8_t* qs = b + 16;
    memset(qs, 0, 128);
    for (int i = 0; i < 256; ++i) {
        int s = i / 32;
        float a = d * (float)sc[s];
        float mm = dmin * (float)m[s];
        int best = 0;
        double bestd = INFINITY;
        for (int q = 0; q < 16; ++q) { /* nearest stored grid point, first on ties */
            double g = (double)(a * (float)q - mm);
            double dd = fabs(g - (double)x[i]);
            if (dd < bestd) { bestd = dd; best = q; }
        }
        int c = i / 64, j = i % 64;
        if (j < 32) qs[32 * c + j] |= (uint8_t)best;
        else qs[32 * c + j - 32] |= (uint8_t)(best << 4);
    }
}

/* Q6_K: per sub-block of 16, sc = round(amax_s / (31 d)) as int8 with
 * d = max_s amax_s / (31 * 127) in fp16; q = clamp(round(x / (d sc)) + 32,
 * 0, 63).  Values round to the nearest point of the stored grid. */
static void orc_quant_q6_k(const float* x, uint8_t* b) {
    float amax[16], gmax = 0.f;
    for (int s = 0; s < 16; ++s) {
        amax[s] = 0.f;
        for (int i = 0; i < 16; ++i) if (fabsf(x[16 * s + i]) > amax[s]) amax[s] = fabsf(x[16 * s + i]);
        if (amax[s] > gmax) gmax = amax[s];
    }
    uint16_t dh = orc_float_to_half(gmax / (31.0f * 127.0f));
    float d = orc_half_to_float(dh);
    int8_t* sc = (int8_t*)(b + 192);
    for (int s = 0; s < 16; ++s)
        sc[s] = (int8_t)(d > 0 ? orc_clampi((int)nearbyint((double)amax[s] / (31.0 * (double)d)), -127, 127) : 0);
    orc_wr16(b + 208, dh);
    uint8_t* ql = b;
    uint8_t* qh = b + 128;
    memset(ql, 0, 128);
    memset(qh, 0, 64);
    for (int i = 0; i < 256; ++i) {
        int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
        float a = d * (float)sc[8 * h + r / 16];
        int best = 32;
        double bestd = INFINITY;
        for (int q = 0; q < 64; ++q) {
            double gv = (double)(a * (float)(q - 32));
            double dd = fabs(gv - (double)x[i]);
            if (dd < bestd) { bestd = dd; best = q; }
        }
        int li = 64 * h + l + 32 * (g % 2);
        if (g < 2) ql[li] |= (uint8_t)(best & 15);
        else ql[li] |= (uint8_t)((best & 15) << 4);
        qh[32 * h + l] |= (uint8_t)((best >> 4) << (2 * g));
    }
}

int oracle_quantize(int type, const float* x, int64_t n_blocks, uint8_t* out) {
    int32_t elems, bytes;
    if (oracle_block_info(type, &elems, &bytes) || type == ORC_Q5_K) return -1;  /* no Q5_K quantiser */
    for (int64_t i = 0; i < n_blocks; ++i) {
        if (type == ORC_Q4_0) orc_quant_q4_0(x + i * elems, out + i * bytes);
        else if (type == ORC_Q4_K) orc_quant_q4_k(x + i * elems, out + i * bytes);
        else orc_quant_q6_k(x + i * elems, out + i * bytes);
    }
    return 0;
}

/* ----------------------------------------------------- gated unit ---- */

/*
 * Gated feed-forward unit: h = act(g) * u elementwise, where g and u are the
 * gate and up products of the same vector.  "GGUF in transformers" (section
 * "Reusing ggml's Metal kernels") notes that a specialised kernel may merge
 * several operations; the models on the pages use gated blocks (Qwen3.5:
 * SiLU; Gemma 4: tanh-approximated GELU).  In fp64, by the definitions:
 *   act 0 (SiLU):      g / (1 + exp(-g))
 *   act 1 (GELU tanh): g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))
 */
int oracle_glu(const double* g, const double* u, int64_t n, int act, double* h) {
    if (act != 0 && act != 1) return 1;
    for (int64_t i = 0; i < n; ++i) {
        double a;
        if (act == 0) {
            a = g[i] / (1.0 + exp(-g[i]));
        } else {
            double c = sqrt(2.0 / acos(-1.0));  /* sqrt(2/pi) */
            a = 0.5 * g[i] * (1.0 + tanh(c * (g[i] + 0.044715 * g[i] * g[i] * g[i])));
        }
        h[i] = a * u[i];
    }
    return 0;
}

/* Exposed for the tests' fp16 pins. */
/* ------------------------------------------------------------ routing ---- */

/*
 * Softmax + top-k routing of mixture-of-experts tokens: the "topk" row of the
 * kernel table in "GGUF in transformers" (section "Reusing ggml's Metal
 * kernels") combines the two steps; the Show HN README ("How it works") has
 * the router score all 128 experts of a token and keep the top 8.
 *
 * For token t, ids[t][0..k) are the k experts with the largest logit, in
 * decreasing order of logit; equal logits go to the lower expert id first.
 * The weights are the softmax of the selected logits,
 *   weights[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0),   l_0 = the largest,
 * evaluated in fp64 (the fp32 logits convert exactly).  Logits are finite.
 */
int oracle_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                      int32_t* ids, double* weights) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return 1;
    unsigned char* taken = (unsigned char*)malloc((size_t)n_experts);
    if (!taken) return 2;
    for (int32_t t = 0; t < n_tokens; ++t) {
        const float* l = logits + (int64_t)t * n_experts;
        memset(taken, 0, (size_t)n_experts);
        for (int32_t j = 0; j < top_k; ++j) {
            /* largest remaining logit; scanning ids upwards with a strict
               comparison keeps the lower id among equal logits */
            int32_t best = -1;
            for (int32_t e = 0; e < n_experts; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * top_k + j] = best;
        }
        const double l0 = (double)l[ids[(int64_t)t * top_k]];
        double sum = 0.0;
        for (int32_t j = 0; j < top_k; ++j) {
            double e = exp((double)l[ids[(int64_t)t * top_k + j]] - l0);
            weights[(int64_t)t * top_k + j] = e;
            sum += e;
        }
        for (int32_t j = 0; j < top_k; ++j) weights[(int64_t)t * top_k + j] /= sum;
    }
    free(taken);
    return 0;
}

float oracle_half_to_float(uint16_t h) { return orc_half_to_float(h); }
uint16_t oracle_float_to_half(float f) { return orc_float_to_half(f); }
