/* Drives every function of the CPU oracle under ASan/UBSan on small inputs of
 * every weight format: random bytes for the weight blocks (any byte pattern
 * is a block), activations with zero, tiny and large blocks.  Checks the
 * oracle's own consistency (f64 result against the dense f64 product and the
 * canonical f32 replay within 1e-4 sum|w x|).  Exit status 0 = all held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}

static int run(int type, int64_t N, int64_t K, int64_t B, int qk, int bb) {
    const int64_t nb = K / 32, rb = K / qk * bb, per = (type == 12 || type == 3 || type == 7) ? 2 : 1;
    uint8_t* w = malloc((size_t)(N * rb));
    float* x = malloc(sizeof(float) * (size_t)(B * K));
    uint8_t* xq = malloc((size_t)(B * nb * 34));
    int32_t* P = malloc(sizeof(int32_t) * (size_t)(B * N * nb * per));
    double *y = malloc(sizeof(double) * (size_t)(B * N)), *A = malloc(sizeof(double) * (size_t)(B * N));
    double* yd = malloc(sizeof(double) * (size_t)(B * N));
    float* yc = malloc(sizeof(float) * (size_t)(B * N));
    double* dq = malloc(sizeof(double) * (size_t)(N * K));
    double* xa = malloc(sizeof(double) * (size_t)(B * K));
    int32_t *q = malloc(sizeof(int32_t) * (size_t)(N * K)), *sc = malloc(sizeof(int32_t) * (size_t)(N * K));
    int32_t* mn = malloc(sizeof(int32_t) * (size_t)(N * K));
    double *d = malloc(sizeof(double) * (size_t)(N * K)), *dm = malloc(sizeof(double) * (size_t)(N * K));
    int bad = 0;
    for (int64_t i = 0; i < N * rb; i++) w[i] = (uint8_t)next();
    /* keep the fp16 scales finite: clear the top exponent bit of every d field */
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < K / qk; b++) {
            uint8_t* blk = w + n * rb + b * bb;
            if (type == 14) blk[209] &= 0x3F;
            else {
                blk[1] &= 0x3F;
                if (type == 12 || type == 3 || type == 7) blk[3] &= 0x3F;
            }
        }
    for (int64_t i = 0; i < B * K; i++) x[i] = (float)((int)(next() % 2001) - 1000) / 250.0f;
    for (int i = 0; i < 32 && i < K; i++) x[i] = 0.0f;                    /* an all-zero block */
    if (K >= 64) for (int i = 32; i < 64; i++) x[i] *= 1e-7f;             /* fp16 d underflows */
    bad |= oracle_quantize_act(x, B, K, xq) != 0;
    bad |= oracle_unpack(type, w, N, K, q, sc, mn, d, dm) != 0;
    bad |= oracle_dequant(type, w, N, K, dq) != 0;
    bad |= oracle_dequant_act(xq, B, K, xa) != 0;
    bad |= oracle_partials(type, w, N, K, xq, B, P) != 0;
    bad |= oracle_matmul_f64(type, w, N, K, xq, B, y, A) != 0;
    bad |= oracle_dense_f64(type, w, N, K, xq, B, yd) != 0;
    bad |= oracle_matmul_canon_f32(type, w, N, K, xq, B, yc) != 0;
    for (int64_t i = 0; i < B * N; i++) {
        if (!(fabs(y[i] - yd[i]) <= 1e-9 * A[i] + 1e-300)) bad = 1;
        if (!(fabs((double)yc[i] - y[i]) <= 1e-4 * A[i])) bad = 1;
    }
    if (qk == 256) {  /* the Q8_K path of the K-quants */
        uint8_t* xk = malloc((size_t)(B * (K / 256) * 292));
        int32_t* Pk = malloc(sizeof(int32_t) * (size_t)(B * N * (K / 256) * 2));
        float* yk = malloc(sizeof(float) * (size_t)(B * N));
        bad |= oracle_quantize_act_q8k(x, B, K, xk) != 0;
        bad |= oracle_dequant_act_q8k(xk, B, K, xa) != 0;
        bad |= oracle_partials_q8k(type, w, N, K, xk, B, Pk) != 0;
        bad |= oracle_matmul_q8k_f64(type, w, N, K, xk, B, y, A) != 0;
        bad |= oracle_matmul_q8k_canon_f32(type, w, N, K, xk, B, yk) != 0;
        for (int64_t i = 0; i < B * N; i++)
            if (!(fabs((double)yk[i] - y[i]) <= 1e-4 * A[i])) bad = 1;
        free(xk); free(Pk); free(yk);
    }
    float h[64], gg[64], uu[64];
    for (int i = 0; i < 64; i++) {
        gg[i] = (float)((int)(next() % 4001) - 2000) / 20.0f;
        uu[i] = (float)((int)(next() % 201) - 100) / 10.0f;
    }
    gg[0] = -1000.0f;
    gg[1] = 1000.0f;
    bad |= oracle_swiglu(gg, uu, 64, h) != 0;
    (void)oracle_half_to_double((uint16_t)next());
    (void)oracle_float_to_half(3.0e38f);
    /* refusals */
    bad |= oracle_partials(4, w, N, K, xq, B, P) == 0;
    bad |= oracle_quantize_act(x, B, 40, xq) == 0;
    free(w); free(x); free(xq); free(P); free(y); free(A); free(yd); free(yc); free(dq); free(xa);
    free(q); free(sc); free(mn); free(d); free(dm);
    if (bad) fprintf(stderr, "oracle check failed: type %d N %ld K %ld B %ld\n", type, (long)N, (long)K, (long)B);
    return bad;
}

int main(void) {
    const int types[8][3] = {{8, 32, 34}, {2, 32, 18}, {6, 32, 22}, {3, 32, 20},
                             {7, 32, 24}, {9, 32, 36}, {12, 256, 144}, {14, 256, 210}};
    int bad = 0;
    for (int t = 0; t < 8; t++) {
        const int qk = types[t][1];
        bad |= run(types[t][0], 1, qk, 1, qk, types[t][2]);
        bad |= run(types[t][0], 7, qk == 32 ? 416 : 768, 3, qk, types[t][2]);
        bad |= run(types[t][0], 3, 1024, 5, qk, types[t][2]);
    }
    if (bad) return 1;
    printf("oracle checks ok\n");
    return 0;
}
