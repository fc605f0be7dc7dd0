/*
 * qmv.h — C-ABI of the MI355X (gfx950) fused dequantise-and-multiply library
 * for GGUF block-quantised weights (libqmv.so).
 *
 * What it computes.  The llamay pages ("Architecture", section "The package
 * map") put the block layouts, dequantisation and fused W4A8 kernels in
 * pkg/quant, and in pkg/tensor a matrix-vector product used while decoding
 * and a matrix-matrix product used for the prompt; the same page's bench
 * transcript reports prefill limited by arithmetic and decode by memory.  Here that is, for a weight matrix W (N rows of K
 * elements, GGUF block layout) and f32 activations X (rows of K elements):
 *
 *     xq      = Q8_0(X)                           (per 32-element block:
 *               d = amax/127 in f32, codes = round-half-away(x * (1/d))
 *               (0 when 1/d is not finite), stored scale fp16(d))
 *     Y[m][n] = sum over 32-blocks b of  d_w(n,b) * d_a(m,b) * I(m,n,b)
 *
 * with I the exact integer dot product of the block's weight codes and
 * activation codes (Q4_0 codes offset by -8, Q5_0 codes by -16, Q6_K codes by
 * -32 and weighted by the 16-element sub-scale; Q4_K contributes
 * d*sc_j*sum(q*a) - dmin*m_j*sum(a); Q4_1 and Q5_1, whose values are d*q + m,
 * contribute d*sum(q*a) + m*sum(a); Q8_0 and Q8_1 d*sum(q*a)).
 *
 * Floating-point order (fixed, identical for every entry point, batch size
 * and launch shape, so that every row of a batched or prefill call is
 * bit-identical to the batch-1 call on that row — the pages' claim that
 * output does not depend on batch composition, "llamay" docs, "The three
 * claims", and that batched prefill equals sequential decode, "Architecture",
 * "The forward pass"):
 *   the K/32 blocks of a row are cut into chunks of 8 blocks (256 elements;
 *   the last chunk may be shorter).  Each chunk sum starts at +0 and adds its
 *   blocks in ascending order, each block term added with ONE rounding to f32
 *   (an fma of the exact integer partial with the exact product of the two
 *   fp16 scales; Q4_K adds its +d and then its -dmin term, Q4_1 / Q5_1 their
 *   +d and then their +m term, m times the f32 product d_a * sum(a)).  Y is
 *   the chunk sums added in ascending order starting from +0.
 *
 * Weight layout.  Row n of W occupies bytes [n*R, (n+1)*R) of w, R =
 * (K/QK)*block_bytes: Q8_0 (type 8) 32 elements / 34 bytes, Q4_0 (type 2)
 * 32 / 18, Q5_0 (type 6) 32 / 22, Q4_1 (type 3) 32 / 20, Q5_1 (type 7)
 * 32 / 24, Q8_1 (type 9) 32 / 36 (its stored s = d*sum(q) is not read),
 * Q4_K (type 12) 256 / 144, Q6_K (type 14) 256 / 210 — a GGUF 2-D tensor
 * with K (ne0) contiguous.  The formats are
 * the ones the pages list ("Models and formats", section "Tensor formats");
 * the byte layouts are the GGUF block structures, which the pages do not
 * print.  Q5_0 is the format of most matrices in the pages' own Qwen2.5-0.5B
 * file (the tensor histogram of its info transcript).  Blocks need not be aligned; w itself must
 * be 16-byte aligned.  X and Y are dense row-major f32, 4-byte aligned (a
 * 16-byte aligned x lets the quantisation run inside the multiply).
 *
 * Ownership.  The caller owns and allocates every buffer (device memory).
 * The library allocates nothing, keeps no per-call state, never synchronises,
 * and enqueues all work asynchronously on `stream` (a hipStream_t; NULL = the
 * null stream).  Calls are thread-safe.  x, xq and y must not overlap w or
 * each other.
 *
 * Errors.  Every argument is checked on the host before anything is enqueued;
 * a failed check returns a negative code and enqueues nothing.  A failed
 * launch returns QMV_ELAUNCH.  qmv_strerror() names what is accepted.
 *
 * Preconditions not checked (data lives on the device): activations finite,
 * and each 32-block's amax at most 127 * 65504.  A block whose d = amax/127
 * is too small for 1/d to be finite in f32 (d below about 2^-128) is
 * quantised like an all-zero block (codes 0; its fp16 scale is 0 anyway).
 */
#ifndef QMV_H
#define QMV_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* GGUF tensor type ids. */
enum qmv_type {
    QMV_Q4_0 = 2, QMV_Q4_1 = 3, QMV_Q5_0 = 6, QMV_Q5_1 = 7, QMV_Q8_0 = 8, QMV_Q8_1 = 9,
    QMV_Q4_K = 12, QMV_Q6_K = 14
};

enum qmv_status {
    QMV_OK = 0,
    QMV_EINVAL_TYPE = -1,        /* type is not one of qmv_type */
    QMV_EINVAL_SHAPE = -2,       /* N, K, rows or batch out of range */
    QMV_EINVAL_PTR = -3,         /* NULL or misaligned pointer */
    QMV_ELAUNCH = -4,            /* the HIP launch failed */
    QMV_EUNSUPPORTED_DEVICE = -5, /* the current device is not gfx950 */
    QMV_ETOO_LARGE = -6          /* qmv_launch_noalloc: the activation scratch for B rows of
                                    K elements exceeds QMV_NOALLOC_MAX_ACT_BYTES */
};

/* Limits: 1 <= N <= 2^31-1; 32 <= K <= 2^20, K % 32 == 0 (K % 256 == 0 for
 * Q4_K and Q6_K, whose rows must be whole 256-element superblocks — the pages
 * fall back from Q4_K to Q4_0 for exactly that reason, "Models and formats",
 * quantize transcript); 1 <= B <= 16 for qmv_launch; 1 <= M <= 2^24 for
 * qmm_launch. */
#define QMV_MAX_K (1 << 20)
#define QMV_MAX_BATCH 16
#define QMV_MAX_M (1 << 24)
#define QMV_MAX_GROUP 8

/* Bytes of activation scratch `xq` for `rows` rows of K elements.  The first
 * rows*(K/32)*34 bytes are the Q8_0 blocks (fp16 d little-endian, then 32
 * int8 codes, blocks in row-major order); the rest holds private staging
 * copies in the layouts the kernels for that many rows read (only those are
 * written).  Returns 0 for an invalid shape. */
size_t qmv_act_bytes(int64_t rows, int64_t K);

/* Quantise x [rows][K] (f32, 4-byte aligned) to Q8_0 into xq (16-byte
 * aligned, qmv_act_bytes(rows, K) bytes): the Q8_0 blocks and the staging
 * copy.  With x == NULL, the Q8_0 blocks already in xq (first rows*(K/32)*34
 * bytes, e.g. produced elsewhere) are taken as the input and only the staging
 * copy is rebuilt from them.  The 8-bit activation format of the W4A8 path
 * ("Architecture", "The package map"). */
int quantize_act_q8_0(const float* x, void* xq, int64_t rows, int64_t K, void* stream);

/* Decode GEMV (MatVec): y[B][N] = x[B][K] * W^T for 1 <= B <= 16.
 * If x is non-NULL it is quantised into xq first, leaving xq exactly as
 * quantize_act_q8_0 would (for B <= 4 the quantisation runs inside the GEMV
 * kernel, one launch, unless the kernel's workgroups would between them read
 * x more bytes than the weights hold; then it is a launch of its own); if x
 * is NULL, xq must already hold a complete quantize_act_q8_0 result for
 * these B rows and K, which is used as is (so several matrices can share one
 * quantisation).  xq: qmv_act_bytes(B, K) bytes, 16-byte aligned.  Decode is
 * memory-bound ("Architecture", bench transcript), so every weight byte is
 * read once per call whatever B is ("A request, end to end": a batch reads
 * the weights once rather than once per sequence). */
int qmv_launch(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t B,
               void* xq, float* y, void* stream);

/* One GEMV of a grouped decode launch (qmv_launch_group). */
typedef struct qmv_gemv {
    const void* w;   /* weight blob as for qmv_launch */
    int64_t N, K;
    const float* x;  /* [B][K] f32 activations, or NULL for all entries (xq staged) */
    void* xq;        /* qmv_act_bytes(B, K) bytes: receives the quantisation when x is given,
                        or holds it when x is NULL.  May be NULL only with x given and
                        16-byte aligned, and only when the whole group runs as one launch
                        that needs no scratch (B <= 4 and every entry's activation rows fit
                        the kernel's LDS); otherwise a NULL xq is refused with
                        QMV_EINVAL_PTR, whatever the other entries hold */
    float* y;        /* [B][N] */
} qmv_gemv;

/* Several independent decode GEMVs of one weight type and one batch B, such
 * as the gate, up and down projections of a decode step, in one launch when
 * the lane-per-chunk kernel takes them all (B <= 4), so that they share the
 * launch latency and the chip instead of running one after another; larger B
 * runs them one after another.  Either every entry quantises its own x, or
 * every entry reads a staged xq (x NULL).  1 <= count <= QMV_MAX_GROUP.
 * Entry k gives bit-identical y (and xq, when written) to qmv_launch(type,
 * w, N, K, x, B, xq, y) on its own.  Entries must not write to memory that
 * another entry reads or writes. */
int qmv_launch_group(int type, int64_t B, const qmv_gemv* g, int count, void* stream);

/* Bytes of scratch `xq` for qmv_launch_gateup_swiglu with B rows, N
 * outputs and K inputs: the activation quantisation as for qmv_launch
 * (qmv_act_bytes(B, K) laid out the same way, first), then room for the two
 * intermediate products when the pair does not run as one launch.  Returns 0
 * for an invalid shape. */
size_t qmv_gateup_act_bytes(int64_t B, int64_t N, int64_t K);

/* Gate and up projections of a SwiGLU feed-forward block in decode, fused:
 * h[B][N] = silu(x * Wg^T) * (x * Wu^T), with silu(g) = g / (1 + e^-g) — the
 * feed-forward gate of the llama family ("Models and formats", architectures
 * table).  Each product is bit-identical to qmv_launch on its own weights;
 * each element of h is then evaluated in f64 as t = exp(-g), s = g / (1 + t),
 * s * u and rounded once to f32.  w_gate and w_up are two N x K blobs of one
 * type (as for qmv_launch); 1 <= B <= 16.  x: [B][K] f32 (4-byte aligned),
 * quantised into xq as qmv_launch does, or NULL to use the quantisation
 * already staged at the start of xq (as quantize_act_q8_0 leaves it).  xq:
 * qmv_gateup_act_bytes(B, N, K) bytes, 16-byte aligned.  h: [B][N] f32,
 * 4-byte aligned; feed it to qmv_launch as the down projection's x.  For
 * B <= 4 and K <= 8192 (and activation rows that fit the kernel's LDS) the
 * pair is one launch in which each wave multiplies matching rows of both
 * matrices and writes h; otherwise the two GEMVs run one after another and a
 * third launch forms h.  h must not overlap x, xq or the weights. */
int qmv_launch_gateup_swiglu(int type, const void* w_gate, const void* w_up, int64_t N,
                             int64_t K, const float* x, int64_t B, void* xq, float* h,
                             void* stream);

/* qmv_launch_gateup_swiglu that also leaves h quantised for the down
 * projection: hq (qmv_act_bytes(B, N) bytes, 16-byte aligned, not
 * overlapping the other buffers) receives exactly what quantize_act_q8_0(h,
 * hq, B, N) would write, so that qmv_launch(type_down, w_down, N_down, N,
 * NULL, B, hq, y, stream) can follow with no quantisation launch of its own.
 * h is still written.  N must be whole 32-element blocks (32 <= N <= 2^20,
 * N % 32 == 0; else QMV_EINVAL_SHAPE).  When each workgroup of the paired
 * launch can own whole 32-row blocks of h (B <= 4, Q4_0 / Q5_0 / Q8_0 / Q4_K
 * / Q6_K weights, K such that a wave takes 4, 8 or 16 gate/up row pairs,
 * e.g. K = 256 .. 2048 or the 896 of the pages' Qwen2.5-0.5B) the
 * quantisation runs in that same launch: the workgroup gathers its 32 values
 * of h in LDS and quantises them; otherwise a quantisation launch follows.  The SwiGLU chain of a decode step in the
 * pages' architecture table ("Models and formats") then takes two launches. */
int qmv_launch_gateup_swiglu_q8(int type, const void* w_gate, const void* w_up, int64_t N,
                                int64_t K, const float* x, int64_t B, void* xq, float* h,
                                void* hq, void* stream);

/* Prefill GEMM (MatMul): y[M][N] = x[M][K] * W^T for any M >= 1.  Prefill
 * is the arithmetic-bound phase ("Architecture", bench transcript): for
 * M > 16 the integer block dots run on the matrix cores (f16 MFMA, which is
 * exact on these small integers); M <= 16 runs the GEMV.  Same x / xq
 * contract as qmv_launch with qmv_act_bytes(M, K) bytes.  Each row of y is
 * bit-identical to qmv_launch with B = 1 on that row. */
int qmm_launch(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t M,
               void* xq, float* y, void* stream);

/* Test hook: the exact int32 per-block partials that the kernels scale and
 * accumulate, produced by the weight decode and integer dot of the same
 * kernel that qmv_launch runs for these B rows (the lane-per-chunk kernel
 * for B <= 4, the MFMA kernel otherwise).  xq must hold quantize_act_q8_0's
 * Q8_0 blocks for B rows, 1 <= B <= 16; the hook first rebuilds the private
 * part of xq from them (the Q8_0 blocks are not changed).  P layout
 * [B][N][K/32] int32; for Q4_K [B][N][K/32][2] = (sc_j * sum q*a,
 * m_j * sum a), for Q4_1 and Q5_1 [B][N][K/32][2] = (sum q*a, sum a). */
int qmv_partials_launch(int type, const void* w, int64_t N, int64_t K, void* xq,
                        int64_t B, int32_t* P, void* stream);

/* Test hook for prefill: as qmv_partials_launch, from the kernel that
 * qmm_launch runs for M rows (the prefill GEMM for M > 16), 1 <= M <= 2^24;
 * P holds M rows in the same layout.  For Q4_K / Q4_1 / Q5_1 the GEMM forms
 * only the first integer on the matrix cores (its min term multiplies the
 * exact f32 product d_a * S); the second is reported as m_j (Q4_K, decoded
 * by the GEMM) times S, the sum of the staged activation codes it
 * multiplies. */
int qmm_partials_launch(int type, const void* w, int64_t N, int64_t K, void* xq,
                        int64_t M, int32_t* P, void* stream);

/* ---- K-quant weights x Q8_K activations ----
 * Q8_K is the 8-bit activation format of the K-quant family (listed with the
 * tensor formats, "Models and formats"; its layout is not on the pages): one
 * block per 256 elements, 292 bytes: f32 d (LE), 256 int8 codes, then 16
 * int16 sums of each 16-code group (LE).  Quantised as Q8_0 is, over 256
 * elements, with d kept in f32: amax, d = amax/127, codes =
 * round-half-away(x * (1/d)) (0 when 1/d is not finite).  Against Q4_K and
 * Q6_K weights (the only types these calls accept; others return
 * QMV_EINVAL_TYPE; K % 256 == 0) a whole superblock reduces to integers
 * (Q4_K: P = sum_j sc_j sum q*a and Q = sum_j m_j sum a; Q6_K:
 * I = sum_j s_j sum (q-32)*a), scaled once per superblock in this f32 order:
 *   p = fma((float)P, fl(d * d_a), +0), then for Q4_K
 *   p = fma(-(float)Q, fl(dmin * d_a), p); y = ((+0 + p_0) + p_1) + ...
 * over the superblocks in ascending order, fl() one f32 rounding of the
 * product of the fp16 weight scale and the f32 activation scale, (float)P
 * rounded to nearest even.  Every row of qmm_launch_q8k and of
 * qmv_launch_q8k with B > 1 is bit-identical to qmv_launch_q8k with B = 1 on
 * that row.  Results differ from the Q8_0 path (a different quantisation of
 * x). */

/* Bytes of activation scratch for `rows` rows of K elements on the Q8_K
 * path: the Q8_K blocks (rows * K/256 * 292 bytes, row-major) first, then
 * private staging.  Returns 0 for an invalid shape (K % 256 != 0 included). */
size_t qmv_act_bytes_q8k(int64_t rows, int64_t K);

/* Quantise x [rows][K] (f32, 4-byte aligned) to Q8_K into xq
 * (qmv_act_bytes_q8k(rows, K) bytes, 16-byte aligned), or with x == NULL
 * rebuild the private staging from Q8_K blocks already at the start of xq. */
int quantize_act_q8_k(const float* x, void* xq, int64_t rows, int64_t K, void* stream);

/* Decode GEMV on the Q8_K path: y[B][N] = x[B][K] * W^T, 1 <= B <= 16, W
 * Q4_K or Q6_K.  x given: quantised into xq first; x NULL: xq holds a
 * complete quantize_act_q8_k result for these B rows.  B <= 4 runs the
 * lane-per-chunk kernel (one launch), B = 5..16 (and B <= 4 with rows too
 * long for that kernel's LDS staging) the batched int8-MFMA kernel
 * (v_mfma_i32_16x16x32_i8, sub-block scales applied to the exact int32
 * block sums, f32 scaling once per superblock); both read the weights
 * once. */
int qmv_launch_q8k(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t B,
                   void* xq, float* y, void* stream);

/* Several independent decode GEMVs of one K-quant type (Q4_K or Q6_K, else
 * QMV_EINVAL_TYPE) and one batch B on the Q8_K path, such as the q, k and v
 * projections of a decode step: entry k gives bit-identical y (and xq, when
 * written) to qmv_launch_q8k(type, w, N, K, x, B, xq, y) on its own.  Every
 * entry needs its xq (qmv_act_bytes_q8k(B, K) bytes, 16-byte aligned; NULL:
 * QMV_EINVAL_PTR); either every entry quantises its x into it (one launch
 * each) or every entry reads it staged (x NULL; entries may share one xq).
 * For B = 5..16 with every entry of one K, the products are one launch of
 * the batched int8-MFMA kernel (a grid row per entry); otherwise they run
 * one after another.  1 <= count <= QMV_MAX_GROUP.  Entries must not write
 * to memory that another entry reads or writes. */
int qmv_launch_group_q8k(int type, int64_t B, const qmv_gemv* g, int count, void* stream);

/* The gate and up projections of a SwiGLU feed-forward block in decode on
 * the Q8_K path (as qmv_launch_gateup_swiglu on the Q8_0 path): h[B][N] =
 * silu(x * Wg^T) * (x * Wu^T), w_gate and w_up two N x K blobs of one type,
 * Q4_K or Q6_K (else QMV_EINVAL_TYPE), K % 256 == 0, 1 <= B <= 16.  Each
 * product is bit-identical to qmv_launch_q8k on its own weights; each
 * element of h is then evaluated in f64 as t = exp(-g), s = g / (1 + t),
 * s * u and rounded once to f32.  x: [B][K] f32 (4-byte aligned), quantised
 * into xq first (one launch), or NULL to use the quantize_act_q8_k result
 * already in xq (qmv_act_bytes_q8k(B, K) bytes, 16-byte aligned).  One
 * launch of the batched int8-MFMA kernel multiplies matching 16-row tiles of
 * both matrices and writes h (4-byte aligned, not overlapping x, xq or the
 * weights). */
int qmv_launch_gateup_swiglu_q8k(int type, const void* w_gate, const void* w_up, int64_t N,
                                 int64_t K, const float* x, int64_t B, void* xq, float* h,
                                 void* stream);

/* Prefill GEMM on the Q8_K path: y[M][N] = x[M][K] * W^T for any M >= 1
 * (M <= 16 runs as qmv_launch_q8k).  The integer superblock partials run on
 * the int8 matrix cores (v_mfma_i32_32x32x32_i8). */
int qmm_launch_q8k(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t M,
                   void* xq, float* y, void* stream);

/* Test hook: the exact int32 superblock partials of the kernel that
 * qmv_launch_q8k / qmm_launch_q8k runs for M rows (1 <= M <= 2^24), from the
 * Q8_K blocks in xq (the private staging is rebuilt from them first).  P
 * layout: Q4_K [M][N][K/256][2] = (P, Q); Q6_K [M][N][K/256] = I. */
int qmv_partials_q8k_launch(int type, const void* w, int64_t N, int64_t K, void* xq,
                            int64_t M, int32_t* P, void* stream);

/* ---- Load-time repack for the Q8_K prefill GEMM (opt-in) ----
 * The pages' benchmark runs with the weights repacked at load ("Architecture",
 * bench transcript header) without saying into what.  Here the repack serves
 * the arithmetic-bound prefill: it stores each Q4_K / Q6_K element's integer
 * weight factor (Q4_K: sc_j * q; Q6_K: s_j * (q - 32)) as the two int8 digits
 * the int8 matrix cores take (v = 64 * hi + lo, lo in 0..63), in the order
 * one MFMA operand load reads them, with the scales split out, so that the
 * GEMM does no unpacking.  Layout (N rows in tiles of 32, t = n / 32,
 * r = n % 32; superblocks s = 0..K/256-1): region t * (K/256) + s of 16896
 * bytes holds at byte 1024 * (2j + g) + 16 * (32h + r) + i digit g (0: lo,
 * 1: hi, int8) of row n's element 32j + 16h + i of superblock s, and at byte
 * 16384 + 16r row n's f32 d (its fp16 d widened), f32 dmin (Q4_K, else 0)
 * and eight 6-bit mins (Q4_K, else 0), little-endian; rows n >= N are zero.
 * It takes 16896 / (32 * 144) = 3.7x the Q4_K bytes and 2.5x the Q6_K bytes:
 * the decode GEMVs, which are bound by weight bytes, keep reading the GGUF
 * blob; the repacked copy is for prefill only.  Results are bit-identical to
 * qmm_launch_q8k on the blob it was made from. */

/* Bytes of the repacked layout of an N x K Q4_K / Q6_K matrix; 0 for another
 * type or an invalid shape (K % 256 != 0 included). */
size_t qmv_prepared_bytes(int type, int64_t N, int64_t K);

/* Repack the GGUF blob w (as for qmv_launch) into wp (qmv_prepared_bytes
 * bytes, 16-byte aligned, caller-owned, not overlapping w), asynchronously on
 * `stream`.  Q4_K and Q6_K only (else QMV_EINVAL_TYPE). */
int qmv_prepare(int type, const void* w, int64_t N, int64_t K, void* wp, void* stream);

/* qmm_launch_q8k on repacked weights: y[M][N] = x[M][K] * W^T for any
 * M >= 1, on the int8-MFMA GEMM for every M (no GEMV on this layout).  wp:
 * qmv_prepare's output for this type, N and K; x / xq / y as qmm_launch_q8k. */
int qmm_launch_q8k_prepared(int type, const void* wp, int64_t N, int64_t K, const float* x,
                            int64_t M, void* xq, float* y, void* stream);

/* Test hook: the exact superblock partials of qmm_launch_q8k_prepared's
 * kernel for M rows, in qmv_partials_q8k_launch's layout. */
int qmm_partials_q8k_prepared_launch(int type, const void* wp, int64_t N, int64_t K, void* xq,
                                     int64_t M, int32_t* P, void* stream);

/* Decode GEMV for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc): the
 * same multiply and result as qmv_launch(type, w, N, K, x, B, xq, y, stream)
 * with x given, bit for bit, but the activation scratch is a fixed array
 * inside the library (one per GPU, QMV_NOALLOC_MAX_ACT_BYTES bytes, held
 * until the process ends) instead of a caller-supplied xq.  The call
 * allocates nothing.  x [B][K] f32 must be non-NULL (4-byte aligned); y
 * [B][N] f32.  Shapes as qmv_launch; in addition qmv_act_bytes(B, K) must not
 * exceed QMV_NOALLOC_MAX_ACT_BYTES, else QMV_ETOO_LARGE (this admits every
 * K <= 65536 at B = 16).  Every call on one GPU uses that GPU's one scratch
 * array: calls that may overlap in time on one GPU (other streams, other
 * host threads without ordering) race on it and must be serialised by the
 * caller; calls in one stream are ordered and safe.  Nothing in the scratch
 * needs to start at zero: each call writes every byte it reads. */
#define QMV_NOALLOC_MAX_ACT_BYTES ((size_t)8 << 20)
int qmv_launch_noalloc(int type, const void* w, int64_t N, int64_t K, const float* x,
                       int64_t B, float* y, void* stream);

/* Static text for a status code. */
const char* qmv_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
