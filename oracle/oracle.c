/*
 * Plain CPU oracle — TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark
 * CPU baseline).  Shares no code with the HIP library.
 *
 * Written from the GGUF block layouts (element formulas per format, restated
 * in the header of the seeded input generator) and the method as the llamay
 * pages describe it ("Architecture", "The package map": block layouts,
 * dequantisation and the fused W4A8 kernels in pkg/quant; MatVec/MatMul in
 * pkg/tensor).  Every loop is element by element; nothing is blocked, fused or
 * reordered beyond what the definitions below state.
 *
 * Build: cc -O2 -std=c11 -ffp-contract=off -fPIC -shared oracle.c -lm
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

enum { T_Q4_0 = 2, T_Q4_1 = 3, T_Q5_0 = 6, T_Q5_1 = 7, T_Q8_0 = 8, T_Q8_1 = 9, T_Q4_K = 12,
       T_Q6_K = 14 };

/* formats whose value adds a per-block minimum: d*q + m */
static int has_min(int type) { return type == T_Q4_1 || type == T_Q5_1; }

/* ---------------------------------------------------------------- fp16 -- */

double oracle_half_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

uint16_t oracle_float_to_half(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double v = fabs((double)f);                 /* exact */
    if (isnan(v)) return sign | 0x7e00;
    if (v >= 65520.0) return sign | 0x7c00;     /* 65520 is the tie above 65504 */
    if (v < ldexp(1.0, -14)) {
        /* subnormal range: integer count of 2^-24 units, ties to even;
         * a count of 1024 is the smallest normal, which the encoding absorbs */
        double units = nearbyint(v * ldexp(1.0, 24));
        return sign | (uint16_t)units;
    }
    int ex;
    frexp(v, &ex);                              /* v = fr * 2^ex, fr in [0.5,1) */
    int E = ex - 1;                             /* v in [2^E, 2^(E+1)) */
    double r = nearbyint(ldexp(v, 10 - E));     /* in [1024, 2048], ties to even */
    if (r == 2048.0) { r = 1024.0; E += 1; }
    if (E + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t rd32(const uint8_t* p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* ------------------------------------------------------- layouts ------- */

static int block_shape(int type, int* qk, int* nbytes) {
    switch (type) {
    case T_Q8_0: *qk = 32;  *nbytes = 34;  return 0;
    case T_Q4_0: *qk = 32;  *nbytes = 18;  return 0;
    case T_Q5_0: *qk = 32;  *nbytes = 22;  return 0;
    case T_Q4_1: *qk = 32;  *nbytes = 20;  return 0;
    case T_Q5_1: *qk = 32;  *nbytes = 24;  return 0;
    case T_Q8_1: *qk = 32;  *nbytes = 36;  return 0;
    case T_Q4_K: *qk = 256; *nbytes = 144; return 0;
    case T_Q6_K: *qk = 256; *nbytes = 210; return 0;
    default: return -1;
    }
}

static int check(int type, int64_t N, int64_t K, int* qk, int* nbytes) {
    if (block_shape(type, qk, nbytes)) return -1;
    if (N < 0 || K <= 0 || K % *qk) return -2;
    return 0;
}

/* Q4_K: the 12 scale bytes hold eight 6-bit (sc, m) pairs.  Sub-blocks 0..3
 * keep theirs in the low 6 bits of bytes j (sc) and j+4 (m); sub-blocks 4..7
 * keep their low 4 bits in byte j+4 (sc low nibble, m high nibble) and their
 * top 2 bits in the top 2 bits of bytes j-4 (sc) and j (m). */
static void q4k_scale_min(const uint8_t* s12, int j, int* sc, int* m) {
    if (j < 4) {
        *sc = s12[j] & 63;
        *m = s12[j + 4] & 63;
    } else {
        *sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
        *m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
    }
}

/* Element e (0 <= e < QK) of one block: stored code, sub-scale, sub-min. */
static void decode_elem(int type, const uint8_t* blk, int e, int* q, int* sc, int* mn) {
    *sc = 1;
    *mn = 0;
    switch (type) {
    case T_Q8_0:
        *q = (int8_t)blk[2 + e];
        break;
    case T_Q8_1:  /* d, then s = d*sum(q) (not part of the value), then the codes */
        *q = (int8_t)blk[4 + e];
        break;
    case T_Q4_1: {  /* d, m, then the nibbles as in Q4_0; m enters once per element */
        uint8_t byte = blk[4 + (e & 15)];
        *q = e < 16 ? (byte & 15) : (byte >> 4);
        *mn = 1;
        break;
    }
    case T_Q5_1: {  /* d, m, the fifth bits (LE u32), the nibbles */
        uint8_t byte = blk[8 + (e & 15)];
        int low4 = e < 16 ? (byte & 15) : (byte >> 4);
        int bit5 = (int)((rd32(blk + 4) >> e) & 1u);
        *q = low4 | (bit5 << 4);
        *mn = 1;
        break;
    }
    case T_Q4_0: {
        uint8_t byte = blk[2 + (e & 15)];
        *q = e < 16 ? (byte & 15) : (byte >> 4);
        break;
    }
    case T_Q5_0: {
        /* d (2 bytes), then the 32 fifth bits as one LE u32, then the low
         * nibbles packed as in Q4_0 */
        uint8_t byte = blk[6 + (e & 15)];
        int low4 = e < 16 ? (byte & 15) : (byte >> 4);
        int bit5 = (int)((rd32(blk + 2) >> e) & 1u);
        *q = low4 | (bit5 << 4);
        break;
    }
    case T_Q4_K: {
        int c = e / 64, r = e % 64;
        uint8_t byte = blk[16 + 32 * c + (r & 31)];
        *q = r < 32 ? (byte & 15) : (byte >> 4);
        q4k_scale_min(blk + 4, e / 32, sc, mn);
        break;
    }
    case T_Q6_K: {
        int h = e / 128, r = e % 128, k = r / 32, l = r % 32;
        uint8_t lb = blk[64 * h + 32 * (k & 1) + l];
        int low4 = k < 2 ? (lb & 15) : (lb >> 4);
        int high2 = (blk[128 + 32 * h + l] >> (2 * k)) & 3;
        *q = low4 | (high2 << 4);
        *sc = (int8_t)blk[192 + e / 16];
        break;
    }
    }
}

static void block_scales(int type, const uint8_t* blk, double* d, double* dmin) {
    *dmin = 0.0;
    if (type == T_Q6_K)
        *d = oracle_half_to_double(rd16(blk + 208));
    else
        *d = oracle_half_to_double(rd16(blk));
    if (type == T_Q4_K || has_min(type)) *dmin = oracle_half_to_double(rd16(blk + 2));
}

/* The integer weight factor that multiplies the activation code, and the
 * integer that multiplies dmin (Q4_K only):
 *   value = d * wint  (Q8_0, Q4_0, Q6_K)      value = d*wint - dmin*mint (Q4_K)
 * Q8_0: wint = q;  Q4_0: q-8;  Q5_0: q-16;  Q6_K: s_j*(q-32);
 * Q4_K: wint = sc_j*q, mint = m_j. */
static void elem_ints(int type, int q, int sc, int mn, int64_t* wint, int64_t* mint) {
    *mint = 0;
    switch (type) {
    case T_Q8_0: *wint = q; break;
    case T_Q4_0: *wint = q - 8; break;
    case T_Q5_0: *wint = q - 16; break;
    case T_Q8_1: *wint = q; break;
    case T_Q4_1:
    case T_Q5_1: *wint = q; *mint = mn; break;
    case T_Q6_K: *wint = (int64_t)sc * (q - 32); break;
    case T_Q4_K: *wint = (int64_t)sc * q; *mint = mn; break;
    }
}

int oracle_unpack(int type, const uint8_t* w, int64_t N, int64_t K, int32_t* q,
                  int32_t* sub_scale, int32_t* sub_min, double* d, double* dmin) {
    int qk, nbytes, rc = check(type, N, K, &qk, &nbytes);
    if (rc) return rc;
    int64_t nbq = K / qk;
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nbq; b++) {
            const uint8_t* blk = w + (n * nbq + b) * nbytes;
            double bd, bdmin;
            block_scales(type, blk, &bd, &bdmin);
            if (d) d[n * nbq + b] = bd;
            if (dmin) dmin[n * nbq + b] = bdmin;
            for (int e = 0; e < qk; e++) {
                int cq, csc, cmn;
                decode_elem(type, blk, e, &cq, &csc, &cmn);
                int64_t k = n * K + b * qk + e;
                if (q) q[k] = cq;
                if (sub_scale) sub_scale[k] = csc;
                if (sub_min) sub_min[k] = cmn;
            }
        }
    return 0;
}

/* Dequantised value of one element (per-format formula of the GGUF layout). */
static double elem_value(int type, int q, int sc, int mn, double d, double dmin) {
    switch (type) {
    case T_Q8_0: return d * q;
    case T_Q4_0: return d * (q - 8);
    case T_Q5_0: return d * (q - 16);
    case T_Q8_1: return d * q;
    case T_Q4_1:
    case T_Q5_1: return d * q + dmin;   /* dmin holds the block's m */
    case T_Q4_K: return d * sc * q - dmin * mn;
    case T_Q6_K: return d * sc * (q - 32);
    }
    return NAN;
}

int oracle_dequant(int type, const uint8_t* w, int64_t N, int64_t K, double* out) {
    int qk, nbytes, rc = check(type, N, K, &qk, &nbytes);
    if (rc) return rc;
    int64_t nbq = K / qk;
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nbq; b++) {
            const uint8_t* blk = w + (n * nbq + b) * nbytes;
            double bd, bdmin;
            block_scales(type, blk, &bd, &bdmin);
            for (int e = 0; e < qk; e++) {
                int cq, csc, cmn;
                decode_elem(type, blk, e, &cq, &csc, &cmn);
                out[n * K + b * qk + e] = elem_value(type, cq, csc, cmn, bd, bdmin);
            }
        }
    return 0;
}

/* ------------------------------------------- activation quantisation --- */

/* Q8_0 per 32-element block: amax = max|x|, d = amax/127 (f32, correctly
 * rounded), id = 1/d (0 when 1/d is not finite, i.e. d == 0 or d below about
 * 2^-128: such a block's fp16 scale is 0), code = round-half-away-from-zero(x*id)
 * with the product in f32; the stored scale is fp16(d). */
int oracle_quantize_act(const float* x, int64_t rows, int64_t K, uint8_t* out) {
    if (rows < 0 || K <= 0 || K % 32) return -2;
    int64_t nb = K / 32;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const float* xb = x + r * K + 32 * b;
            uint8_t* o = out + (r * nb + b) * 34;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(xb[i]));
            float d = amax / 127.0f;
            /* a block too small for 1/d to be finite in f32 (d < ~2^-128,
             * d == 0 included) gets all-zero codes: its fp16 scale is 0 */
            float r = 1.0f / d;
            float id = isinf(r) ? 0.0f : r;
            uint16_t dh = oracle_float_to_half(d);
            o[0] = (uint8_t)(dh & 255);
            o[1] = (uint8_t)(dh >> 8);
            for (int i = 0; i < 32; i++) {
                float v = xb[i] * id;
                o[2 + i] = (uint8_t)(int8_t)(int)roundf(v);
            }
        }
    return 0;
}

int oracle_dequant_act(const uint8_t* xq, int64_t rows, int64_t K, double* out) {
    if (rows < 0 || K <= 0 || K % 32) return -2;
    int64_t nb = K / 32;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t* blk = xq + (r * nb + b) * 34;
            double d = oracle_half_to_double(rd16(blk));
            for (int i = 0; i < 32; i++) out[r * K + 32 * b + i] = d * (int8_t)blk[2 + i];
        }
    return 0;
}

/* ----------------------------------------------------- multiply -------- */

/* One weight row decoded into per-element integers and per-element scales. */
typedef struct {
    int64_t* wint;   /* [K] */
    int64_t* mint;   /* [K] */
    double* d;       /* [K] block d of the element's block */
    double* dmin;    /* [K] */
} row_t;

static int row_alloc(row_t* r, int64_t K) {
    r->wint = malloc(sizeof(int64_t) * K);
    r->mint = malloc(sizeof(int64_t) * K);
    r->d = malloc(sizeof(double) * K);
    r->dmin = malloc(sizeof(double) * K);
    return (r->wint && r->mint && r->d && r->dmin) ? 0 : -4;
}

static void row_free(row_t* r) {
    free(r->wint); free(r->mint); free(r->d); free(r->dmin);
}

static void row_decode(int type, const uint8_t* wrow, int64_t K, int qk, int nbytes, row_t* r) {
    for (int64_t b = 0; b < K / qk; b++) {
        const uint8_t* blk = wrow + b * nbytes;
        double bd, bdmin;
        block_scales(type, blk, &bd, &bdmin);
        for (int e = 0; e < qk; e++) {
            int cq, csc, cmn;
            decode_elem(type, blk, e, &cq, &csc, &cmn);
            int64_t k = b * qk + e;
            elem_ints(type, cq, csc, cmn, &r->wint[k], &r->mint[k]);
            r->d[k] = bd;
            /* the factor of the subtracted min term: Q4_K dmin; Q4_1/Q5_1 add m */
            r->dmin[k] = has_min(type) ? -bdmin : bdmin;
        }
    }
}

/* Integer partial(s) of 32-element block b of one activation row. */
static void block_ints(const row_t* r, const uint8_t* arow, int64_t b, int64_t* I, int64_t* Q) {
    const uint8_t* ablk = arow + b * 34;
    *I = 0;
    *Q = 0;
    for (int i = 0; i < 32; i++) {
        int64_t a = (int8_t)ablk[2 + i];
        *I += r->wint[32 * b + i] * a;
        *Q += r->mint[32 * b + i] * a;
    }
}

static int fits32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }

int oracle_partials(int type, const uint8_t* w, int64_t N, int64_t K,
                    const uint8_t* xq, int64_t B, int32_t* P) {
    int qk, nbytes, rc = check(type, N, K, &qk, &nbytes);
    if (rc) return rc;
    if (B < 0) return -2;
    int64_t nb = K / 32, rb = (K / qk) * nbytes;
    int per = (type == T_Q4_K || has_min(type)) ? 2 : 1;
    row_t r;
    if (row_alloc(&r, K)) { row_free(&r); return -4; }
    for (int64_t n = 0; n < N; n++) {
        row_decode(type, w + n * rb, K, qk, nbytes, &r);
        for (int64_t m = 0; m < B; m++)
            for (int64_t b = 0; b < nb; b++) {
                int64_t I, Q;
                block_ints(&r, xq + m * nb * 34, b, &I, &Q);
                if (!fits32(I) || !fits32(Q)) { row_free(&r); return -3; }
                int32_t* o = P + ((m * N + n) * nb + b) * per;
                o[0] = (int32_t)I;
                if (per == 2) o[1] = (int32_t)Q;
            }
    }
    row_free(&r);
    return 0;
}

int oracle_matmul_f64(int type, const uint8_t* w, int64_t N, int64_t K,
                      const uint8_t* xq, int64_t B, double* y, double* A) {
    int qk, nbytes, rc = check(type, N, K, &qk, &nbytes);
    if (rc) return rc;
    if (B < 0) return -2;
    int64_t nb = K / 32, rb = (K / qk) * nbytes;
    row_t r;
    if (row_alloc(&r, K)) { row_free(&r); return -4; }
    for (int64_t n = 0; n < N; n++) {
        row_decode(type, w + n * rb, K, qk, nbytes, &r);
        for (int64_t m = 0; m < B; m++) {
            const uint8_t* arow = xq + m * nb * 34;
            double acc = 0.0, absacc = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                int64_t I, Q;
                block_ints(&r, arow, b, &I, &Q);
                double da = oracle_half_to_double(rd16(arow + b * 34));
                double dw = r.d[32 * b], dmw = r.dmin[32 * b];
                acc += da * (dw * (double)I - dmw * (double)Q);
                if (A)
                    for (int i = 0; i < 32; i++) {
                        int64_t k = 32 * b + i;
                        double wv = dw * (double)r.wint[k] - dmw * (double)r.mint[k];
                        double xv = da * (double)(int8_t)arow[b * 34 + 2 + i];
                        absacc += fabs(wv * xv);
                    }
            }
            if (y) y[m * N + n] = acc;
            if (A) A[m * N + n] = absacc;
        }
    }
    row_free(&r);
    return 0;
}

int oracle_dense_f64(int type, const uint8_t* w, int64_t N, int64_t K,
                     const uint8_t* xq, int64_t B, double* y) {
    int qk, nbytes, rc = check(type, N, K, &qk, &nbytes);
    if (rc) return rc;
    if (B < 0) return -2;
    double* wd = malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    double* xd = malloc(sizeof(double) * (size_t)(B * K > 0 ? B * K : 1));
    if (!wd || !xd) { free(wd); free(xd); return -4; }
    oracle_dequant(type, w, N, K, wd);
    oracle_dequant_act(xq, B, K, xd);
    for (int64_t m = 0; m < B; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += wd[n * K + k] * xd[m * K + k];
            y[m * N + n] = acc;
        }
    free(wd);
    free(xd);
    return 0;
}

int oracle_matmul_canon_f32(int type, const uint8_t* w, int64_t N, int64_t K,
                            const uint8_t* xq, int64_t B, float* y) {
    int qk, nbytes, rc = check(type, N, K, &qk, &nbytes);
    if (rc) return rc;
    if (B < 0) return -2;
    int64_t nb = K / 32, rb = (K / qk) * nbytes;
    row_t r;
    if (row_alloc(&r, K)) { row_free(&r); return -4; }
    for (int64_t n = 0; n < N; n++) {
        row_decode(type, w + n * rb, K, qk, nbytes, &r);
        for (int64_t m = 0; m < B; m++) {
            const uint8_t* arow = xq + m * nb * 34;
            float acc = 0.0f;
            for (int64_t c0 = 0; c0 < nb; c0 += 8) {
                float p = 0.0f;
                for (int64_t b = c0; b < nb && b < c0 + 8; b++) {
                    int64_t I, Q;
                    block_ints(&r, arow, b, &I, &Q);
                    float da = (float)oracle_half_to_double(rd16(arow + b * 34));
                    float dw = (float)r.d[32 * b];
                    p = fmaf((float)I, dw * da, p);
                    if (type == T_Q4_K || has_min(type)) {
                        float dmw = (float)r.dmin[32 * b];
                        p = fmaf(-(float)Q, dmw * da, p);
                    }
                }
                acc = acc + p;
            }
            y[m * N + n] = acc;
        }
    }
    row_free(&r);
    return 0;
}

/* SwiGLU gate of a decode FFN (llamay "Models and formats", the architectures
 * table: SwiGLU feed-forward in the llama / qwen2 family; the pages give no
 * formula, so the usual one is read): h = silu(g) * u with
 * silu(g) = g / (1 + e^-g).  Each element is evaluated in f64 in the order
 * t = exp(-g), s = g / (1 + t), h = s * u, and rounded once to f32. */
int oracle_swiglu(const float* g, const float* u, int64_t n, float* h) {
    if (n < 0) return -2;
    for (int64_t i = 0; i < n; i++) {
        const double gd = (double)g[i];
        const double t = exp(-gd);
        const double s = gd / (1.0 + t);
        h[i] = (float)(s * (double)u[i]);
    }
    return 0;
}

/* ------------------------------------- K-quants x Q8_K activations ----- */
/*
 * Q8_K: the 8-bit format of the K-quant family ("Models and formats", the
 * list of tensor formats, which names it next to Q2_K..Q6_K).  The pages do
 * not describe it; taken here: one block per 256 elements, 292 bytes: the
 * scale d as an f32 (LE), 256 int8 codes, then 16 int16 (LE) sums of the
 * codes of each 16-element group (stored for the kernels; the oracle
 * recomputes every sum it needs from the codes).  The quantisation rule is
 * the Q8_0 rule over 256 elements, with the f32 d kept as is: amax, d =
 * amax/127, id = 1/d (0 when 1/d is not finite), code = round-half-away(x*id).
 *
 * The multiply pairs it with Q4_K and Q6_K weights, whose sub-block scales
 * are integers, so one superblock's partial is one integer (two for Q4_K):
 *   Q4_K: P = sum_j sc_j sum_{k in j} q_k a_k,   Q = sum_j m_j sum_{k in j} a_k
 *   Q6_K: I = sum_j s_j sum_{k in j} (q_k - 32) a_k
 * and the superblock adds d_a (d P - dmin Q), or d_a d I.
 */

enum { Q8K_BYTES = 292 };

static float rdf32(const uint8_t* p) {
    uint32_t u = rd32(p);
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int oracle_quantize_act_q8k(const float* x, int64_t rows, int64_t K, uint8_t* out) {
    if (rows < 0 || K <= 0 || K % 256) return -2;
    int64_t nsb = K / 256;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t s = 0; s < nsb; s++) {
            const float* xb = x + r * K + 256 * s;
            uint8_t* o = out + (r * nsb + s) * Q8K_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < 256; i++) amax = fmaxf(amax, fabsf(xb[i]));
            float d = amax / 127.0f;
            float rcp = 1.0f / d;
            float id = isinf(rcp) ? 0.0f : rcp;
            uint32_t du;
            memcpy(&du, &d, 4);
            for (int i = 0; i < 4; i++) o[i] = (uint8_t)(du >> (8 * i));
            int8_t q[256];
            for (int i = 0; i < 256; i++) q[i] = (int8_t)(int)roundf(xb[i] * id);
            for (int i = 0; i < 256; i++) o[4 + i] = (uint8_t)q[i];
            for (int g = 0; g < 16; g++) {
                int sum = 0;
                for (int i = 0; i < 16; i++) sum += q[16 * g + i];
                o[260 + 2 * g] = (uint8_t)(sum & 255);
                o[261 + 2 * g] = (uint8_t)((sum >> 8) & 255);
            }
        }
    return 0;
}

int oracle_dequant_act_q8k(const uint8_t* xq, int64_t rows, int64_t K, double* out) {
    if (rows < 0 || K <= 0 || K % 256) return -2;
    int64_t nsb = K / 256;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t s = 0; s < nsb; s++) {
            const uint8_t* blk = xq + (r * nsb + s) * Q8K_BYTES;
            double d = (double)rdf32(blk);
            for (int i = 0; i < 256; i++) out[r * K + 256 * s + i] = d * (int8_t)blk[4 + i];
        }
    return 0;
}

static int check_q8k(int type, int64_t N, int64_t K, int64_t B, int* qk, int* nbytes) {
    if (type != T_Q4_K && type != T_Q6_K) return -1;
    int rc = check(type, N, K, qk, nbytes);
    if (rc) return rc;
    return B < 0 ? -2 : 0;
}

/* Integer partial(s) of superblock s of one Q8_K activation row. */
static void superblock_ints(const row_t* r, const uint8_t* arow, int64_t s, int64_t* I, int64_t* Q) {
    const uint8_t* ablk = arow + s * Q8K_BYTES;
    *I = 0;
    *Q = 0;
    for (int i = 0; i < 256; i++) {
        int64_t a = (int8_t)ablk[4 + i];
        *I += r->wint[256 * s + i] * a;
        *Q += r->mint[256 * s + i] * a;
    }
}

int oracle_partials_q8k(int type, const uint8_t* w, int64_t N, int64_t K,
                        const uint8_t* xq, int64_t B, int32_t* P) {
    int qk, nbytes, rc = check_q8k(type, N, K, B, &qk, &nbytes);
    if (rc) return rc;
    int64_t nsb = K / 256, rb = nsb * nbytes;
    int per = type == T_Q4_K ? 2 : 1;
    row_t r;
    if (row_alloc(&r, K)) { row_free(&r); return -4; }
    for (int64_t n = 0; n < N; n++) {
        row_decode(type, w + n * rb, K, qk, nbytes, &r);
        for (int64_t m = 0; m < B; m++)
            for (int64_t s = 0; s < nsb; s++) {
                int64_t I, Q;
                superblock_ints(&r, xq + m * nsb * Q8K_BYTES, s, &I, &Q);
                if (!fits32(I) || !fits32(Q)) { row_free(&r); return -3; }
                int32_t* o = P + ((m * N + n) * nsb + s) * per;
                o[0] = (int32_t)I;
                if (per == 2) o[1] = (int32_t)Q;
            }
    }
    row_free(&r);
    return 0;
}

int oracle_matmul_q8k_f64(int type, const uint8_t* w, int64_t N, int64_t K,
                          const uint8_t* xq, int64_t B, double* y, double* A) {
    int qk, nbytes, rc = check_q8k(type, N, K, B, &qk, &nbytes);
    if (rc) return rc;
    int64_t nsb = K / 256, rb = nsb * nbytes;
    row_t r;
    if (row_alloc(&r, K)) { row_free(&r); return -4; }
    for (int64_t n = 0; n < N; n++) {
        row_decode(type, w + n * rb, K, qk, nbytes, &r);
        for (int64_t m = 0; m < B; m++) {
            const uint8_t* arow = xq + m * nsb * Q8K_BYTES;
            double acc = 0.0, absacc = 0.0;
            for (int64_t s = 0; s < nsb; s++) {
                int64_t I, Q;
                superblock_ints(&r, arow, s, &I, &Q);
                double da = (double)rdf32(arow + s * Q8K_BYTES);
                double dw = r.d[256 * s], dmw = r.dmin[256 * s];
                acc += da * (dw * (double)I - dmw * (double)Q);
                if (A)
                    for (int i = 0; i < 256; i++) {
                        int64_t k = 256 * s + i;
                        double wv = dw * (double)r.wint[k] - dmw * (double)r.mint[k];
                        double xv = da * (double)(int8_t)arow[s * Q8K_BYTES + 4 + i];
                        absacc += fabs(wv * xv);
                    }
            }
            if (y) y[m * N + n] = acc;
            if (A) A[m * N + n] = absacc;
        }
    }
    row_free(&r);
    return 0;
}

/* The f32 order of the Q8_K path: per superblock s (in ascending order),
 *   Q4_K: p = fmaf((float)P, fl(d * d_a), +0); p = fmaf(-(float)Q, fl(dmin * d_a), p)
 *   Q6_K: p = fmaf((float)I, fl(d * d_a), +0)
 * where fl(d * d_a) is the f32 product of the fp16 weight scale and the f32
 * activation scale, rounded once, and (float)P rounds to nearest even when
 * |P| > 2^24; then y = ((+0 + p_0) + p_1) + ... */
int oracle_matmul_q8k_canon_f32(int type, const uint8_t* w, int64_t N, int64_t K,
                                const uint8_t* xq, int64_t B, float* y) {
    int qk, nbytes, rc = check_q8k(type, N, K, B, &qk, &nbytes);
    if (rc) return rc;
    int64_t nsb = K / 256, rb = nsb * nbytes;
    row_t r;
    if (row_alloc(&r, K)) { row_free(&r); return -4; }
    for (int64_t n = 0; n < N; n++) {
        row_decode(type, w + n * rb, K, qk, nbytes, &r);
        for (int64_t m = 0; m < B; m++) {
            const uint8_t* arow = xq + m * nsb * Q8K_BYTES;
            float acc = 0.0f;
            for (int64_t s = 0; s < nsb; s++) {
                int64_t I, Q;
                superblock_ints(&r, arow, s, &I, &Q);
                float da = rdf32(arow + s * Q8K_BYTES);
                float sd = (float)r.d[256 * s] * da;
                float p = fmaf((float)I, sd, 0.0f);
                if (type == T_Q4_K) {
                    float sm = (float)r.dmin[256 * s] * da;
                    p = fmaf(-(float)Q, sm, p);
                }
                acc = acc + p;
            }
            y[m * N + n] = acc;
        }
    }
    row_free(&r);
    return 0;
}

/* ------------------------------------------ load-time repack (Q8_K path) -- */
/*
 * The pages' own benchmark runs with the weights repacked when the file is
 * loaded ("Architecture", bench transcript header: repack on) and do not say
 * into what.  The repack here serves the prefill multiply against Q8_K
 * activations: each element's integer weight factor wint (Q4_K: sc_j * q;
 * Q6_K: s_j * (q - 32)) stored as two int8 digits, wint = 64 * hi + lo with
 * lo = wint mod 64 in 0..63, so that one superblock's integer partial is
 * 64 * sum(hi * a) + sum(lo * a), sums of int8 products.  Layout, for N rows
 * in tiles of 32 (row n in tile n / 32, position r = n % 32) and superblocks
 * s = 0..K/256-1: region (t * (K/256) + s) of 16896 bytes holds
 *   bytes 1024 * (2j + g) + 16 * (32 h + r) + i, for element e = 32 j + 16 h + i
 *     of superblock s: digit g (0: lo, 1: hi, as int8) of row n's element e;
 *   bytes 16384 + 16 r .. + 15: row n's f32 d (the fp16 d, widened), f32
 *     dmin (Q4_K; 0 for Q6_K), then the eight 6-bit mins m_0..m_7 (Q4_K; 0
 *     for Q6_K), all little-endian;
 * rows n >= N of the last tile are all zero.
 */
enum { PREP_REGION = 16896, PREP_REC = 16384 };

int64_t oracle_prepared_bytes(int type, int64_t N, int64_t K) {
    int qk, nbytes;
    if (type != T_Q4_K && type != T_Q6_K) return -1;
    if (check(type, N, K, &qk, &nbytes)) return -2;
    return (N + 31) / 32 * (K / 256) * PREP_REGION;
}

static void wr32(uint8_t* p, uint32_t v) {
    for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}

int oracle_prepare_q8k(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* out) {
    int64_t bytes = oracle_prepared_bytes(type, N, K);
    if (bytes < 0) return (int)bytes;
    memset(out, 0, (size_t)bytes);
    int qk, nbytes;
    check(type, N, K, &qk, &nbytes);
    int64_t nsb = K / 256;
    for (int64_t n = 0; n < N; n++)
        for (int64_t s = 0; s < nsb; s++) {
            const uint8_t* blk = w + (n * nsb + s) * nbytes;
            uint8_t* reg = out + ((n / 32) * nsb + s) * PREP_REGION;
            int r = (int)(n % 32);
            for (int e = 0; e < 256; e++) {
                int q, sc, mn;
                int64_t wint, mint;
                decode_elem(type, blk, e, &q, &sc, &mn);
                elem_ints(type, q, sc, mn, &wint, &mint);
                int64_t lo = ((wint % 64) + 64) % 64;
                int64_t hi = (wint - lo) / 64;
                int j = e / 32, h = (e % 32) / 16, i = e % 16;
                reg[1024 * (2 * j) + 16 * (32 * h + r) + i] = (uint8_t)lo;
                reg[1024 * (2 * j + 1) + 16 * (32 * h + r) + i] = (uint8_t)(int8_t)hi;
            }
            double d, dmin;
            block_scales(type, blk, &d, &dmin);
            float fd = (float)d, fdmin = (float)dmin;
            uint32_t ud, udmin;
            memcpy(&ud, &fd, 4);
            memcpy(&udmin, &fdmin, 4);
            uint8_t* rec = reg + PREP_REC + 16 * r;
            wr32(rec, ud);
            wr32(rec + 4, udmin);
            if (type == T_Q4_K)
                for (int j = 0; j < 8; j++) {
                    int sc, mn;
                    q4k_scale_min(blk + 4, j, &sc, &mn);
                    rec[8 + j] = (uint8_t)mn;
                }
        }
    return 0;
}
