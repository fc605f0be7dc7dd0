/*
 * Plain CPU oracle for the fused dequantise-and-multiply of GGUF block-quantised
 * weights against Q8_0-quantised activations.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library shares
 * no code, header, table or helper with it, and neither includes the other.
 *
 * What it computes (llamay "Architecture", section "The package map": pkg/quant
 * holds the block layouts, dequantisation and the fused W4A8 kernels;
 * pkg/tensor holds MatVec for decode and MatMul for prefill):
 *
 *   y[m][n] = sum_k  w^[n][k] * x^[m][k]
 *
 * where w^ is the dequantised weight (per the GGUF block layout) and x^ is the
 * dequantised Q8_0 activation.  Everything is plain scalar C: activation
 * quantisation in f32 (it decides integer codes, so it takes the kernel's
 * precision), integer partials in int64, and results in f64.
 *
 * Type ids are the GGUF ones: Q4_0 = 2, Q4_1 = 3, Q5_0 = 6, Q5_1 = 7, Q8_0 = 8,
 * Q8_1 = 9, Q4_K = 12, Q6_K = 14.
 * All functions return 0 on success and a negative value on a bad argument
 * (-1 unknown type, -2 bad shape, -3 a partial does not fit in int32).
 */
#ifndef GQMV_ORACLE_H
#define GQMV_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* fp16 bits -> exact double; f32 -> fp16 bits, round to nearest even,
 * subnormals kept, overflow to infinity. */
double   oracle_half_to_double(uint16_t h);
uint16_t oracle_float_to_half(float f);

/* Q8_0 activation quantisation of x[rows][K] (K % 32 == 0) into
 * rows*(K/32) blocks of 34 bytes: fp16 d (LE) then 32 int8 codes. */
int oracle_quantize_act(const float* x, int64_t rows, int64_t K, uint8_t* out);

/* Field-by-field unpack of an N x K weight blob.  Per element: the stored code
 * q[N*K] (Q8_0/Q8_1 signed, Q4_0/Q4_1/Q4_K 0..15, Q5_0/Q5_1 0..31, Q6_K 0..63),
 * its sub-block scale sub_scale[N*K] (Q4_K sc_j, Q6_K s_j, else 1) and min
 * sub_min[N*K] (Q4_K m_j, Q4_1/Q5_1 1, else 0).  Per block of QK elements:
 * d[N*K/QK] and dmin[N*K/QK] (Q4_K dmin, Q4_1/Q5_1 the block's m, else 0).
 * Values: d*q (Q8_0, Q8_1), d*(q-8) (Q4_0), d*(q-16) (Q5_0), d*q + m
 * (Q4_1, Q5_1), d*sc_j*q - dmin*m_j (Q4_K), d*s_j*(q-32) (Q6_K).  Any output
 * pointer may be NULL. */
int oracle_unpack(int type, const uint8_t* w, int64_t N, int64_t K, int32_t* q,
                  int32_t* sub_scale, int32_t* sub_min, double* d, double* dmin);

/* Dequantised weights, f64 [N][K]. */
int oracle_dequant(int type, const uint8_t* w, int64_t N, int64_t K, double* out);

/* Dequantised Q8_0 activations, f64 [rows][K]. */
int oracle_dequant_act(const uint8_t* xq, int64_t rows, int64_t K, double* out);

/* Exact integer partial per (m, n, 32-element block b), layout [B][N][K/32]:
 *   Q8_0, Q8_1: sum w*a     Q4_0: sum (q-8)*a     Q5_0: sum (q-16)*a
 *   Q6_K: sum s_j*(q-32)*a
 *   Q4_K: two integers per block, layout [B][N][K/32][2]:
 *         P = sum sc_j*q*a  and  Q = sum m_j*a
 *   Q4_1, Q5_1: the same pair with P = sum q*a and Q = sum a               */
int oracle_partials(int type, const uint8_t* w, int64_t N, int64_t K,
                    const uint8_t* xq, int64_t B, int32_t* P);

/* y[B][N] in f64 from the per-block partials and fp16 scales, blocks in
 * ascending order; A[B][N] = sum_k |w^ * x^| (either may be NULL). */
int oracle_matmul_f64(int type, const uint8_t* w, int64_t N, int64_t K,
                      const uint8_t* xq, int64_t B, double* y, double* A);

/* y[B][N] in f64 straight from the dequantised matrices, element by element. */
int oracle_dense_f64(int type, const uint8_t* w, int64_t N, int64_t K,
                     const uint8_t* xq, int64_t B, double* y);

/* y[B][N] in f32 following the documented f32 reduction order: blocks are
 * grouped into chunks of 8 (256 elements; the last chunk may be short); each
 * chunk starts at +0 and adds its block terms in ascending order, each term
 * added with one rounding (fmaf of the exact partial and the exact product of
 * the two fp16 scales; Q4_K adds +P*(d*da) then -Q*(dmin*da), Q4_1/Q5_1
 * +P*(d*da) then +Q*(m*da)); y is the chunk sums added in ascending order
 * starting from +0. */
int oracle_matmul_canon_f32(int type, const uint8_t* w, int64_t N, int64_t K,
                            const uint8_t* xq, int64_t B, float* y);

/* SwiGLU of a decode FFN, element by element: h = silu(g) * u with
 * silu(g) = g / (1 + exp(-g)), evaluated in f64 as t = exp(-g),
 * s = g / (1 + t), h = s * u and rounded once to f32. */
int oracle_swiglu(const float* g, const float* u, int64_t n, float* h);

/* ---- K-quant weights (Q4_K = 12, Q6_K = 14) x Q8_K activations ----
 * Q8_K block: 256 elements in 292 bytes: f32 d (LE), int8 codes[256], int16
 * sums of each 16-element group of codes (LE).  Quantisation as Q8_0 over
 * 256 elements with d kept in f32.  K % 256 == 0. */
int oracle_quantize_act_q8k(const float* x, int64_t rows, int64_t K, uint8_t* out);
int oracle_dequant_act_q8k(const uint8_t* xq, int64_t rows, int64_t K, double* out);
/* Per superblock s: Q4_K [B][N][K/256][2] = (sum_j sc_j sum q a, sum_j m_j sum a);
 * Q6_K [B][N][K/256] = sum_j s_j sum (q-32) a.  Other types: -1. */
int oracle_partials_q8k(int type, const uint8_t* w, int64_t N, int64_t K,
                        const uint8_t* xq, int64_t B, int32_t* P);
/* y = sum_s d_a (d P - dmin Q) (Q4_K) or d_a d I (Q6_K) in f64; A = sum |w^ x^|. */
int oracle_matmul_q8k_f64(int type, const uint8_t* w, int64_t N, int64_t K,
                          const uint8_t* xq, int64_t B, double* y, double* A);
/* The f32 order of the Q8_K path: per superblock in order,
 * p = fmaf((float)P, fl(d*d_a), +0) then (Q4_K) p = fmaf(-(float)Q,
 * fl(dmin*d_a), p); y = ((+0 + p_0) + p_1) + ... */
int oracle_matmul_q8k_canon_f32(int type, const uint8_t* w, int64_t N, int64_t K,
                                const uint8_t* xq, int64_t B, float* y);

/* ---- Load-time repack of Q4_K / Q6_K weights for the Q8_K path ----
 * Each element's integer weight factor as two int8 digits (wint = 64 hi + lo,
 * lo in 0..63) in 32-row tiles, one 16896-byte region per (tile, superblock):
 * digit g of row 32t + r, element 32j + 16h + i at byte 1024(2j + g) +
 * 16(32h + r) + i; at 16384 + 16r the row's f32 d, f32 dmin and (Q4_K) its
 * eight 6-bit mins; rows past N zero.  Other types: -1. */
int64_t oracle_prepared_bytes(int type, int64_t N, int64_t K);
int oracle_prepare_q8k(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* out);

#ifdef __cplusplus
}
#endif
#endif
