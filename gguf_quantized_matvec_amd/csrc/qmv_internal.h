// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libqmv.so.  Not part of the public interface (include/qmv.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

// Activation scratch `xq` for `rows` rows of K elements:
//   [0, pub)            Q8_0 blocks, row-major: fp16 d (LE) + 32 int8 codes
//   [priv0, ...)        private staging copies (every offset 256-aligned):
//   for the MFMA kernels, in groups of 16 rows (G = ceil(rows/16); rows past
//   `rows` are zero):
//     codes  [G][nb][64][8] int8   the 16x16x32 MFMA A-operand of block b:
//                                  lane l = m + 16*kg holds codes
//                                  a[16g+m][32b + 8kg .. 32b + 8kg + 7]
//     da     [G][nb][16] f32       f32 value of the fp16 block scale
//     ca     [G][nb][16] f32       da * S (exact in f32)
//     S      [G][nb][16] int32     sum of the block's 32 codes
//   for the lane-per-chunk dot kernels, row-major over the `rows` rows:
//     rcodes [rows][K] int8        codes in element order
//     rda    [rows][nb] f32        as da
//     rca    [rows][nb] f32        as ca
//     rs16   [rows][nb] int32      sums of the two 16-element halves as two
//                                  int16: low half = elements 0..15
//   for the prefill GEMM (f16 MFMA; small integers are exact in f16):
//     hcodes [rows][K] f16         codes as f16 values
//     hda    [rows][nb] u16        fp16 bits of the block scale
struct ActLayout {
    int64_t nb, G, pub, priv0, codes, da, ca, S, rcodes, rda, rca, rs16, hcodes, hda, total;
};

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

inline ActLayout act_layout(int64_t rows, int64_t K) {
    ActLayout L;
    L.nb = K / 32;
    L.G = (rows + 15) / 16;
    L.pub = rows * L.nb * 34;
    L.priv0 = align256(L.pub);
    L.codes = L.priv0;
    L.da = align256(L.codes + L.G * L.nb * 512);
    L.ca = align256(L.da + L.G * L.nb * 64);
    L.S = align256(L.ca + L.G * L.nb * 64);
    L.rcodes = align256(L.S + L.G * L.nb * 64);
    L.rda = align256(L.rcodes + rows * K);
    L.rca = align256(L.rda + rows * L.nb * 4);
    L.rs16 = align256(L.rca + rows * L.nb * 4);
    L.hcodes = align256(L.rs16 + rows * L.nb * 4);
    L.hda = align256(L.hcodes + rows * K * 2);
    L.total = align256(L.hda + rows * L.nb * 2);
    return L;
}

// Activation scratch for the K-quant x Q8_K path, rows of K elements
// (K % 256 == 0):
//   [0, pub)           Q8_K blocks, row-major: f32 d (LE), 32 x 8 int8
//                      codes, 16 int16 sums of 16-code groups (292 bytes)
//   then (256-aligned) the row-major staging that the kernels read:
//     rcodes [rows][K] int8    codes in element order
//     rda    [rows][K/32] f32  d of the element's superblock, per 32 codes
//     rs16   [rows][K/32] i32  sums of the two 16-code halves of each 32
//                              codes, as two int16 (low half = first)
//     rsd    [rows][K/256][16] int8  the superblock's eight 32-code sums S_j
//                              as two digits, S = 64 hi + lo, lo = S & 63:
//                              lo of S_0..S_3, hi of S_0..S_3, lo of
//                              S_4..S_7, hi of S_4..S_7 (the operands of the
//                              Q4_K min-term MFMAs)
// (rcodes, rda, rs16: the layout of the lane-per-chunk GEMV's Q8_0 staging,
// so that kernel stages either; rca is not used on this path and aliases
// rda).
//   For rows <= 16 (gcodes != 0) also the copy the batched decode kernel
//   reads, in the operand order of v_mfma_i32_16x16x32_i8, per superblock c:
//     gcodes [c][p = 0..3][lane 0..63][16]  lane l = m + 16 kg: row m's codes
//                                           8kg..8kg+7 of block 2p, then of
//                                           block 2p+1
//     gda    [c][16] f32                    row m's Q8_K d
//     gsd    [c][16][16] int8               row m's sum digits, as in rsd
//   (entries of rows m >= rows are not written: they only ever feed outputs
//   of rows that are not stored).
struct ActLayoutK {
    int64_t nb, nsb, pub, rcodes, rda, rs16, rsd, gcodes, gda, gsd, total;
};
inline ActLayoutK act_layout_q8k(int64_t rows, int64_t K) {
    ActLayoutK L;
    L.nb = K / 32;
    L.nsb = K / 256;
    L.pub = rows * L.nsb * 292;
    L.rcodes = (L.pub + 255) & ~int64_t(255);
    L.rda = (L.rcodes + rows * K + 255) & ~int64_t(255);
    L.rs16 = (L.rda + rows * L.nb * 4 + 255) & ~int64_t(255);
    L.rsd = (L.rs16 + rows * L.nb * 4 + 255) & ~int64_t(255);
    L.total = (L.rsd + rows * L.nsb * 16 + 255) & ~int64_t(255);
    L.gcodes = L.gda = L.gsd = 0;
    if (rows <= 16) {
        L.gcodes = L.total;
        L.gda = L.gcodes + L.nsb * 4096;
        L.gsd = (L.gda + L.nsb * 64 + 255) & ~int64_t(255);
        L.total = (L.gsd + L.nsb * 256 + 255) & ~int64_t(255);
    }
    return L;
}

// One GEMV of a (possibly grouped) decode launch.
struct GemvDesc {
    const uint8_t* w;
    int64_t N, K;
    const float* x;   // non-NULL: quantised by the launch
    uint8_t* xq;      // staged quantisation (x NULL), or where to write it (may be NULL if x given)
    float* y;
};

// Bytes of one weight row.
inline int64_t row_bytes(int type, int64_t K) {
    switch (type) {
    case 2: return K / 32 * 18;     // Q4_0
    case 3: return K / 32 * 20;     // Q4_1
    case 6: return K / 32 * 22;     // Q5_0
    case 7: return K / 32 * 24;     // Q5_1
    case 9: return K / 32 * 36;     // Q8_1
    case 8: return K / 32 * 34;     // Q8_0
    case 12: return K / 256 * 144;  // Q4_K
    case 14: return K / 256 * 210;  // Q6_K
    }
    return 0;
}

// Which private staging copies a quantisation writes: only those that the
// multiply for that many rows reads.
enum Staging : int {
    ST_ROW = 1,   // rcodes, rda, rca, rs16 (lane-per-chunk GEMV)
    ST_MFMA = 2,  // codes, da, ca, S (MFMA GEMV and the partials hook)
    ST_F16 = 4,   // hcodes, hda and rca (prefill GEMM)
};
int staging_for(int64_t rows, int64_t K);
// Whether launch_qmv_group runs the whole group as one launch of the
// lane-per-chunk kernel (then an entry with x given may leave xq NULL, as
// long as its x is 16-byte aligned).
bool group_is_one_launch(const GemvDesc* d, int count, int64_t rows);

// Kernel launchers (qmv_kernels.hip).  Arguments are already validated.
// Each returns 0 or a hipError_t value.  x != NULL: the launch quantises x
// into xq first (fused into the multiply where that kernel can).
int launch_quantize(const float* x, uint8_t* xq, int64_t rows, int64_t K, int staging,
                    hipStream_t s);
int launch_rebuild(uint8_t* xq, int64_t rows, int64_t K, int staging, hipStream_t s);
int launch_qmv(int type, const uint8_t* w, int64_t N, int64_t K, const float* x, uint8_t* xq,
               int64_t rows, float* y, hipStream_t s);
// count GEMVs of one type and row count: one launch if the lane-per-chunk
// kernel takes them all (and all or none quantise x), else one after another.
int launch_qmv_group(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t s);
// Gate/up pair of a SwiGLU FFN: h[rows][N] = silu(x Wg^T) * (x Wu^T).  xq
// holds gateup_act_bytes(rows, N, K) bytes.
bool gateup_is_one_launch(int64_t rows, int64_t K);
inline int64_t gateup_act_bytes(int64_t rows, int64_t N, int64_t K) {
    return align256(act_layout(rows, K).total) + 2 * align256(rows * N * 4);
}
// hq != NULL: h quantised to Q8_0 into hq as quantize_act_q8_0(h, hq, rows,
// N) leaves it, inside the paired launch when gateup_quantises_h().
int launch_gateup(int type, const uint8_t* wg, const uint8_t* wu, int64_t N, int64_t K,
                  const float* x, uint8_t* xq, int64_t rows, float* h, hipStream_t s,
                  uint8_t* hq = nullptr);
bool gateup_quantises_h(int type, int64_t rows, int64_t N, int64_t K);
int launch_partials(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* xq,
                    int64_t rows, int32_t* P, hipStream_t s);
int launch_qmm(int type, const uint8_t* w, int64_t N, int64_t K, const float* x, uint8_t* xq,
               int64_t rows, float* y, hipStream_t s);
// K-quant (Q4_K, Q6_K) x Q8_K path.  x given: quantise it into xq first
// (x == NULL for launch_quantize_q8k: rebuild the staging from the Q8_K
// blocks already in xq).  P != NULL: the exact superblock partials go to P.
int launch_quantize_q8k(const float* x, uint8_t* xq, int64_t rows, int64_t K, hipStream_t s);
// Several GEMVs on the Q8_K path (1..16 rows; x of every entry, if given,
// quantised into its xq first): one launch of the batched kernel when the
// rows take it and every entry has the same K, else one after another.
int launch_group_q8k(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t s);
// Gate/up pair with the SwiGLU on the Q8_K path (1..16 rows): x (if given)
// quantised into xq, then one launch of the batched kernel writing h.
int launch_gateup_q8k(int type, const uint8_t* wg, const uint8_t* wu, int64_t N, int64_t K,
                      const float* x, uint8_t* xq, int64_t rows, float* h, hipStream_t s);
int launch_qmv_q8k(int type, const uint8_t* w, int64_t N, int64_t K, const float* x, uint8_t* xq,
                   int64_t rows, float* y, int32_t* P, hipStream_t s);
// The int8-MFMA GEMM of the Q8_K path (qmm8k_kernels.hip), any rows >= 1;
// prepared: w is the load-time repacked layout (launch_prepare_q8k).
int launch_gemm_q8k(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
                    int64_t M, float* y, int32_t* P, bool prepared, hipStream_t s);
// Load-time repack of a Q4_K / Q6_K blob for the Q8_K GEMM: its size in
// bytes, the repack, and the GEMM on it (x given or P: quantise first).
int64_t prepared_bytes_q8k(int type, int64_t N, int64_t K);
int launch_prepare_q8k(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* out,
                       hipStream_t s);
int launch_qmm_q8k_prepared(int type, const uint8_t* wp, int64_t N, int64_t K, const float* x,
                            uint8_t* xq, int64_t rows, float* y, int32_t* P, hipStream_t s);
// Device address of the current device's fixed activation scratch for
// qmv_launch_noalloc (qmv_noalloc.hip), or NULL with *err set.
uint8_t* noalloc_scratch(int* err);
// Prefill GEMM on f16 MFMA (qmm_kernels.hip), for rows > 16.
// P != NULL: the test hook; the exact block partials go to P instead of y.
int launch_gemm(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                float* y, hipStream_t s, int32_t* P = nullptr);
// Partials of the kernel qmm_launch runs at M rows (the GEMM for M > 16).
int launch_qmm_partials(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* xq,
                        int64_t M, int32_t* P, hipStream_t s);

}  // namespace qmv
