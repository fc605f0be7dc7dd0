// Prefill GEMM (MatMul) for gfx950: Y[M][N] = X[M][K] * W^T with GGUF block
// weights and Q8_0 activations, on MFMA.
//
// The pages call prefill arithmetic-bound (llamay "Architecture", bench
// transcript), so this is the one place the path is a dense contraction.  Its
// cost is not the integer dot but the per-block scaling: every (row, column,
// 32-block) needs its own f32 term added in the documented order.  Two facts
// measured on the hardware keep that to one VALU fma per output and block:
//   * f16 MFMA on small integers is exact: codes (|a| <= 127; weights with
//     the sub-scale folded in, |w| <= 945 for Q4_K and <= 4096 and even or
//     <= 2048 for Q6_K) are exact in f16, their products and sums (< 2^24)
//     are exact in the f32 accumulator, so v_mfma_f32_32x32x16_f16 returns
//     the exact integer block partial;
//   * the product of two fp16 values is exact in f32 (subnormals included),
//     so a rank-1 MFMA (one nonzero k) gives every d_w * d_a of a 32x32 tile.
// Then p = fma(I, d_w*d_a, p) is exactly the term the GEMV adds, and rows are
// bit-identical to the batch-1 GEMV.  Q4_K's min term is fma(-(dmin*m_j),
// d_a*S, p) with both products exact (S: the block's activation code sum),
// which is the same real product as the documented (m_j*S)*(dmin*d_a).
//
// Tiling: a workgroup of 8 waves owns 128 x 128 outputs; wave w computes rows
// 64*(w&1) .. +63 and columns 32*(w>>1) .. +31 (2 x 1 MFMA tiles of 32 x 32),
// two waves per SIMD.  K is walked 128 elements (4 blocks) per step.  The
// activation tile (f16 codes) goes global -> LDS directly with
// global_load_lds into a double buffer; each thread fetches one weight block
// into registers, decodes it to f16 into LDS after the previous step is
// consumed, and then issues the next step's loads, which stay in flight
// while the 4 blocks are multiplied.  Per block and wave the multiply is 6
// MFMAs (2 x (2 integer + 1 rank-1 scale)) against 32 VALU fmas (64 for
// Q4_K), read from ready-made LDS operands.  LDS rows are XOR swizzled in 16-byte
// pieces so that MFMA fragment reads hit all banks.  Workgroups are ordered
// in groups of 8 M-tiles and mapped so that each XCD runs a contiguous range
// of them: concurrently resident workgroups on one XCD share activation and
// weight tiles through its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int T_Q4_0 = 2, T_Q4_1 = 3, T_Q5_0 = 6, T_Q5_1 = 7, T_Q8_0 = 8, T_Q8_1 = 9,
              T_Q4_K = 12, T_Q6_K = 14;
// Formats whose block term has a second part fed by the activation code sums
// (Q4_K's sub-block mins; the block minimum m of Q4_1 / Q5_1).
template <int FMT> constexpr bool has_min_term() {
    return FMT == T_Q4_K || FMT == T_Q4_1 || FMT == T_Q5_1;
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int SB = 4;               // 32-element blocks per K step
constexpr int PR = 4 * SB;          // 16-byte pieces per tile row per step
constexpr int NA = 2;               // activation steps resident in LDS (1 in flight)

template <int FMT> struct GFmt;
template <> struct GFmt<T_Q8_0> { static constexpr int QK = 32, BB = 34; };
template <> struct GFmt<T_Q4_0> { static constexpr int QK = 32, BB = 18; };
template <> struct GFmt<T_Q5_0> { static constexpr int QK = 32, BB = 22; };
template <> struct GFmt<T_Q4_1> { static constexpr int QK = 32, BB = 20; };
template <> struct GFmt<T_Q5_1> { static constexpr int QK = 32, BB = 24; };
template <> struct GFmt<T_Q8_1> { static constexpr int QK = 32, BB = 36; };
template <> struct GFmt<T_Q4_K> { static constexpr int QK = 256, BB = 144; };
template <> struct GFmt<T_Q6_K> { static constexpr int QK = 256, BB = 210; };

__device__ __forceinline__ _Float16 h_of_bits(uint32_t b) {
    const uint16_t u = (uint16_t)b;
    _Float16 h;
    __builtin_memcpy(&h, &u, 2);
    return h;
}

// Weight bytes one staging thread fetches per step: one 32-element block of
// one row (K-quants: the fields of the superblock that block uses).
template <int FMT> struct WRaw;
template <> struct WRaw<T_Q8_0> { uint32_t v[9]; };    // 34 B
template <> struct WRaw<T_Q4_0> { uint32_t v[5]; };    // 18 B
template <> struct WRaw<T_Q5_0> { uint32_t v[6]; };    // 22 B
template <> struct WRaw<T_Q4_1> { uint32_t v[5]; };    // 20 B
template <> struct WRaw<T_Q5_1> { uint32_t v[6]; };    // 24 B
template <> struct WRaw<T_Q8_1> { uint32_t v[9]; };    // 36 B
template <> struct WRaw<T_Q4_K> { uint32_t hdr[4]; uint32_t q[8]; };   // d, dmin, sc12; 32 B of qs
template <> struct WRaw<T_Q6_K> { uint32_t ql[8]; uint32_t qh[8]; uint32_t sd; };  // s pair | d << 16

// Block b (< nb) of a weight row.
template <int FMT>
__device__ __forceinline__ void fetch_w(const uint8_t* row, int b, WRaw<FMT>& r) {
    if constexpr (GFmt<FMT>::QK == 32) {
        __builtin_memcpy(r.v, row + (int64_t)b * GFmt<FMT>::BB, GFmt<FMT>::BB);
    } else if constexpr (FMT == T_Q4_K) {
        const uint8_t* sb = row + (int64_t)144 * (b >> 3);
        const int j = b & 7;
        __builtin_memcpy(r.hdr, sb, 16);
        __builtin_memcpy(r.q, sb + 16 + 32 * (j >> 1), 32);
    } else {
        const uint8_t* sb = row + (int64_t)210 * (b >> 3);
        const int bb = b & 7, h = bb >> 2, kk = bb & 3;
        __builtin_memcpy(r.ql, sb + 64 * h + 32 * (kk & 1), 32);
        __builtin_memcpy(r.qh, sb + 128 + 32 * h, 32);
        uint16_t sp, d;
        __builtin_memcpy(&sp, sb + 192 + 2 * bb, 2);
        __builtin_memcpy(&d, sb + 208, 2);
        r.sd = (uint32_t)sp | ((uint32_t)d << 16);
    }
}

// f16 pair from 16-bit integers v < 1024 in the low bits of each half: the
// bits 0x6400 | v are the f16 value 1024 + v, so subtracting 1024 + bias
// exactly gives v - bias.
__device__ __forceinline__ uint32_t pk_ints_to_f16(uint32_t two, float bias) {
    const uint32_t bits = two | 0x64006400u;
    h2 v;
    __builtin_memcpy(&v, &bits, 4);
    const _Float16 off = (_Float16)(1024.0f + bias);
    const h2 o = {off, off};
    v = v - o;
    uint32_t out;
    __builtin_memcpy(&out, &v, 4);
    return out;
}

// 4 small integers in the bytes of `q` -> two dwords of packed f16 (q - bias)
__device__ __forceinline__ void bytes_to_f16(uint32_t q, float bias, uint32_t& o0, uint32_t& o1) {
    o0 = pk_ints_to_f16(__builtin_amdgcn_perm(0u, q, 0x0c010c00u), bias);
    o1 = pk_ints_to_f16(__builtin_amdgcn_perm(0u, q, 0x0c030c02u), bias);
}

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, _Float16 s) {
    h2 v;
    __builtin_memcpy(&v, &a, 4);
    const h2 ss = {s, s};
    v = v * ss;
    uint32_t out;
    __builtin_memcpy(&out, &v, 4);
    return out;
}

// Scale words of a decoded block, as the multiply reads them.
struct WScale {
    uint32_t d;    // fp16 bits of the block / superblock d
    uint32_t x1;   // Q4_K: f32 bits of dmin * m_j;  Q6_K (unscaled codes): s0 | s1 << 16
    int mn;        // Q4_K: the 6-bit min m_j (the partials hook reports m_j * S)
};

// Decode block b of the fetched bytes into 32 f16 values (16 dwords, element
// order).  Q4_K folds the 6-bit sub-scale into the codes (sc*q <= 945);
// Q6_K folds the int8 sub-scales in when FOLD (|s*(q-32)| <= 2048, or even
// and <= 4096: exact in f16), else leaves q - 32 and returns s0, s1.
template <int FMT, bool FOLD>
__device__ __forceinline__ void decode_w(const WRaw<FMT>& r, int b, uint32_t (&o)[16], WScale& s) {
    if constexpr (FMT == T_Q8_0 || FMT == T_Q8_1) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(r.v);
        s.d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
        constexpr int QS = FMT == T_Q8_0 ? 2 : 4;  // Q8_1 keeps s = d*sum(q) in bytes 2-3
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q;
            __builtin_memcpy(&q, blk + QS + 4 * i, 4);
            // int8 x -> x ^ 0x80 = x + 128 in [0, 255]; minus 128 after the f16 trick
            bytes_to_f16(q ^ 0x80808080u, 128.0f, o[2 * i], o[2 * i + 1]);
        }
    } else if constexpr (FMT == T_Q4_0) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(r.v);
        s.d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t q;
            __builtin_memcpy(&q, blk + 2 + 4 * i, 4);
            bytes_to_f16(q & 0x0F0F0F0Fu, 8.0f, o[2 * i], o[2 * i + 1]);                // 0..15
            bytes_to_f16((q >> 4) & 0x0F0F0F0Fu, 8.0f, o[8 + 2 * i], o[8 + 2 * i + 1]);  // 16..31
        }
    } else if constexpr (FMT == T_Q4_1 || FMT == T_Q5_1) {
        // codes 0..15 / 0..31 as f16; the block minimum is the second term:
        // x1 = -m, so that the epilogue's fma(-x1, d_a S, p) adds m d_a S
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(r.v);
        s.d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
        s.x1 = __float_as_uint(-(float)h_of_bits((uint32_t)blk[2] | ((uint32_t)blk[3] << 8)));
        constexpr int QS = FMT == T_Q4_1 ? 4 : 8;
        uint32_t h = 0;
        if constexpr (FMT == T_Q5_1) __builtin_memcpy(&h, blk + 4, 4);
        auto spread4 = [](uint32_t v) { return (__umul24(v, 0x204081u) & 0x01010101u) << 4; };
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t q;
            __builtin_memcpy(&q, blk + QS + 4 * i, 4);
            uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
            if constexpr (FMT == T_Q5_1) {
                lo |= spread4((h >> (4 * i)) & 15u);
                hi |= spread4((h >> (16 + 4 * i)) & 15u);
            }
            bytes_to_f16(lo, 0.0f, o[2 * i], o[2 * i + 1]);            // 0..15
            bytes_to_f16(hi, 0.0f, o[8 + 2 * i], o[8 + 2 * i + 1]);    // 16..31
        }
    } else if constexpr (FMT == T_Q5_0) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(r.v);
        s.d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
        uint32_t h;
        __builtin_memcpy(&h, blk + 2, 4);
        // fifth bit j of the block -> bit 4 of code j (see spread4)
        auto spread4 = [](uint32_t v) { return (__umul24(v, 0x204081u) & 0x01010101u) << 4; };
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t q;
            __builtin_memcpy(&q, blk + 6 + 4 * i, 4);
            const uint32_t lo = (q & 0x0F0F0F0Fu) | spread4((h >> (4 * i)) & 15u);
            const uint32_t hi = ((q >> 4) & 0x0F0F0F0Fu) | spread4((h >> (16 + 4 * i)) & 15u);
            bytes_to_f16(lo, 16.0f, o[2 * i], o[2 * i + 1]);            // 0..15
            bytes_to_f16(hi, 16.0f, o[8 + 2 * i], o[8 + 2 * i + 1]);    // 16..31
        }
    } else if constexpr (FMT == T_Q4_K) {
        const int j = b & 7;  // sub-block
        s.d = r.hdr[0] & 0xFFFFu;
        // byte i of the 12 packed scale bytes (selects, not a dynamic index)
        auto s12 = [&r](int i) -> int {
            const uint32_t d = i < 4 ? r.hdr[1] : (i < 8 ? r.hdr[2] : r.hdr[3]);
            return (int)((d >> (8 * (i & 3))) & 0xFFu);
        };
        int sc, mn;
        if (j < 4) {
            sc = s12(j) & 63;
            mn = s12(j + 4) & 63;
        } else {
            sc = (s12(j + 4) & 15) | ((s12(j - 4) >> 6) << 4);
            mn = (s12(j + 4) >> 4) | ((s12(j) >> 6) << 4);
        }
        const float dmin = (float)h_of_bits(r.hdr[0] >> 16);
        s.x1 = __float_as_uint(dmin * (float)mn);  // exact: 11-bit x 6-bit
        s.mn = mn;
        const _Float16 sch = (_Float16)(float)sc;
        const int sh = 4 * (j & 1);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t f0, f1;
            bytes_to_f16((r.q[i] >> sh) & 0x0F0F0F0Fu, 0.0f, f0, f1);
            o[2 * i] = pk_mul(f0, sch);
            o[2 * i + 1] = pk_mul(f1, sch);
        }
    } else {
        const int bb = b & 7, kk = bb & 3;
        s.d = r.sd >> 16;
        const int s0 = (int8_t)(r.sd & 0xFF), s1 = (int8_t)((r.sd >> 8) & 0xFF);
        s.x1 = (uint32_t)(s0 & 0xFFFF) | ((uint32_t)s1 << 16);
        const int lsh = 4 * (kk >> 1);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t lo = (r.ql[i] >> lsh) & 0x0F0F0F0Fu;
            const uint32_t hi = ((r.qh[i] >> (2 * kk)) & 0x03030303u) << 4;
            bytes_to_f16(lo | hi, 32.0f, o[2 * i], o[2 * i + 1]);
        }
        if constexpr (FOLD) {
            const _Float16 f0 = (_Float16)(float)s0, f1 = (_Float16)(float)s1;
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = pk_mul(o[i], f0);
#pragma unroll
            for (int i = 8; i < 16; i++) o[i] = pk_mul(o[i], f1);
        }
    }
}

// Workgroup -> (tile_m, tile_n): XCD x (= blockIdx % 8) gets a contiguous
// range of logical tiles; logical tiles run in groups of GROUP_M M-tiles with
// the N-tile advancing slowest inside a group.
constexpr int GROUP_M = 8;
__device__ __forceinline__ void tile_of(int64_t wg, int64_t tilesM, int64_t tilesN, int64_t& tm,
                                        int64_t& tn) {
    const int64_t nt = tilesM * tilesN;
    const int64_t x = wg & 7, k = wg >> 3;
    int64_t base = 0;
    for (int64_t xx = 0; xx < x; xx++) base += (nt - xx + 7) >> 3;
    const int64_t t = base + k;
    const int64_t group = t / (GROUP_M * tilesN);
    const int64_t first_m = group * GROUP_M;
    const int64_t gm = tilesM - first_m < GROUP_M ? tilesM - first_m : GROUP_M;
    const int64_t r = t - group * GROUP_M * tilesN;
    tm = first_m + r % gm;
    tn = r / gm;
}

// LDS of the workgroup.  Tile rows hold SB blocks x 32 f16 = 256 bytes as 16
// pieces of 16 bytes; piece q of row r sits in slot r*16 + (q ^ (r & 15)), so
// the 8 lanes of each ds_read_b128 pass (consecutive rows) hit different banks.
// The scale products run as rank-1 MFMAs whose operands are read ready-made:
// ra[b][r] = (d_a, 0, ..., 0) for activation row r (row TM is all zero, for
// the lanes that hold k = 8..15), rw[b][r] = d_w in all 8 halves.
// T = TM = TN: the workgroup tile.
template <int T> struct Smem {
    uint4 w[T * PR];      // decoded weights (f16)
    uint4 ra[SB][T + 1];  // rank-1 A operands (fp16 d_a at k = 0)
    uint4 rw[SB][T];      // rank-1 B operands (fp16 d_w broadcast)
    float ca[SB][T];      // Q4_K: d_a * S (S = the block's code sum)
    uint32_t x1[SB][T];   // see WScale::x1
};
// The partials hook's extra staging: per step, the code sum S of each
// activation row's block and the Q4_K min m_j of each weight row's block.
template <int T> struct SmemPart {
    int S[SB][T];
    int mn[SB][T];
};
__device__ __forceinline__ int slot(int row, int q) { return row * PR + (q ^ (row & 15)); }

using Even = std::integral_constant<int, 0>;
using Odd = std::integral_constant<int, 1>;

// NW waves per workgroup: NW = 8 owns 128 x 128 outputs (each wave 64 x 32,
// two MFMA tiles), NW = 4 owns 64 x 64 (each wave one 32 x 32 tile) for
// grids that would not fill the chip with the larger tile.
// PART: the test hook; instead of scaling and accumulating, each block's
// exact integer partial(s) go to P[m][n][b] (two per block for the formats
// with a minimum term), y unused.
template <int FMT, int NW, bool PART = false>
__global__ __launch_bounds__(64 * NW) void k_gemm(const uint8_t* __restrict__ w, int64_t N, int64_t K,
                                                  const uint8_t* __restrict__ xq, ActLayout L,
                                                  int64_t M, int64_t tilesM, int64_t tilesN,
                                                  float* __restrict__ y, int32_t* __restrict__ P) {
    using F = GFmt<FMT>;
    constexpr int TM = 16 * NW, TN = 16 * NW;  // workgroup tile
    constexpr int WT = NW / 4;                 // 32 x 32 MFMA tiles per wave (along M)
    // The activation ring (f16 codes of NA = 2 steps) lives in two separate
    // LDS objects: while the next step is copied into one by global_load_lds,
    // the multiply reads the other, and the compiler, seeing two objects,
    // does not make those reads wait for the copy in flight (with one object
    // it must).
    __shared__ uint4 lds_a0[TM * PR];
    __shared__ uint4 lds_a1[TM * PR];
    __shared__ Smem<TM> lds_rest;
    Smem<TM>* const sm = &lds_rest;
    __shared__ SmemPart<PART ? TM : 1> lds_part;
    auto a_buf = [&](auto par) -> uint4* {
        if constexpr (decltype(par)::value == 0) return lds_a0;
        else return lds_a1;
    };
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    int64_t tm, tn;
    tile_of(blockIdx.x, tilesM, tilesN, tm, tn);
    const int64_t m0 = tm * TM, n0 = tn * TN;
    const int nb = (int)(K >> 5);
    const int H = (nb + SB - 1) / SB;   // K steps
    const int64_t R = (K / F::QK) * F::BB;

    // staging role: tile row sr (activation row m0 + sr, weight row n0 + sr),
    // block sk of the step
    const int sr = tid >> 2, sk = tid & 3;
    const int64_t am = m0 + sr < M ? m0 + sr : M - 1;  // clamp: rows past M are discarded
    const int64_t wr = n0 + sr < N ? n0 + sr : N - 1;
    const uint16_t* ahda = reinterpret_cast<const uint16_t*>(xq + L.hda) + am * nb;
    const float* arca = reinterpret_cast<const float*>(xq + L.rca) + am * nb;
    const uint8_t* wrow = w + wr * R;
    if (tid < SB) sm->ra[tid][TM] = make_uint4(0, 0, 0, 0);

    // activation tile by global_load_lds: each wave instruction fills 64
    // consecutive slots = 4 tile rows; wave wv fills rows 16wv .. 16wv + 15;
    // lane l: row 16wv + 4i + l/16, slot l%16, which holds piece
    // (l%16) ^ (row & 15).  Source pointers advance 256 bytes per step.
    const uint8_t* asrc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int row = 16 * wv + 4 * i + (lane >> 4);
        const int piece = (lane & 15) ^ (row & 15);
        const int64_t arow = m0 + row < M ? m0 + row : M - 1;
        asrc[i] = xq + L.hcodes + (arow * K + 8 * piece) * 2;
    }
    auto issue_a = [&](int h, auto par) {
        const bool ragged = SB * h + SB > nb;  // uniform: only the last step of a ragged K
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint8_t* src = asrc[i] + (int64_t)h * (SB * 64);
            if (ragged) {
                // blocks past the row end: fetch any in-row bytes, never read
                const int row = 16 * wv + 4 * i + (lane >> 4);
                const int piece = (lane & 15) ^ (row & 15);
                const int blk = SB * h + (piece >> 2);
                if (blk >= nb) src -= (int64_t)(blk - (nb - 1)) * 64;
            }
            __builtin_amdgcn_global_load_lds(
                src, (lds_void*)(a_buf(par) + (16 * wv + 4 * i) * PR), 16, 0, 0);
        }
    };

    // weight bytes and activation scales of the next step, in registers;
    // every thread always loads (a clamped block past the end of K), so that
    // consuming them also waits for the earlier activation loads of the same
    // step (vector memory loads complete in order)
    struct Raw {
        WRaw<FMT> w;
        uint32_t da;
        float ca;
        bool have;
    };
    auto fetch = [&](int h, Raw& r) {
        const int b = SB * h + sk;
        r.have = b < nb;
        const int bc = r.have ? b : nb - 1;
        fetch_w<FMT>(wrow, bc, r.w);
        r.da = ahda[bc];
        if (has_min_term<FMT>()) r.ca = arca[bc];
    };

    // accumulators of tile i: chunk sum p and running sum yv
    v16f p[WT], yv[WT];
#pragma unroll
    for (int i = 0; i < WT; i++)
#pragma unroll
        for (int e = 0; e < 16; e++) p[i][e] = yv[i][e] = 0.0f;

    const int lr = lane & 31, kq = lane >> 5;  // MFMA lane roles
    const v16f zero16 = {};
    // fragment slots: A rows 32 WT wm + 32i + lr, B rows 32wn + lr; piece
    // 4*bk + 2hh + kq holds k = 16hh + 8kq .. +8 of block bk
    const int arow0 = 32 * WT * wm + lr, brow = 32 * wn + lr;

    // step h reads activation buffer P = h % 2 and fills the other
    auto step = [&](int h, Raw& r, auto par) {
        constexpr int PB = decltype(par)::value;
        const int nbh = min(SB, nb - SB * h);
        bool odd_big = false;
        if constexpr (FMT == T_Q6_K) {
            const int s0 = (int8_t)(r.w.sd & 0xFF), s1 = (int8_t)((r.w.sd >> 8) & 0xFF);
            odd_big = r.have && (((s0 & 1) && (s0 > 64 || s0 < -64)) ||
                                 ((s1 & 1) && (s1 > 64 || s1 < -64)));
        }
        // B1: step h-1 is consumed (its W tile and activation slot are free)
        const bool unfolded = __syncthreads_or(odd_big) != 0;
        {
            uint32_t o[16];
            WScale f{};
            if (FMT == T_Q6_K && unfolded)
                decode_w<FMT, false>(r.w, SB * h + sk, o, f);
            else
                decode_w<FMT, true>(r.w, SB * h + sk, o, f);
            if (!r.have) f.d = 0;
#pragma unroll
            for (int q = 0; q < 4; q++)
                sm->w[slot(sr, 4 * sk + q)] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
            const uint32_t dd = f.d | (f.d << 16);
            sm->rw[sk][sr] = make_uint4(dd, dd, dd, dd);
            sm->ra[sk][sr] = make_uint4(r.da, 0, 0, 0);
            if (has_min_term<FMT>()) sm->ca[sk][sr] = r.ca;
            if (has_min_term<FMT>() || FMT == T_Q6_K) sm->x1[sk][sr] = f.x1;
            if constexpr (PART) {
                // S: the sum of the staged activation codes of the block (the
                // f16 values the matrix cores multiply), exact in int
                int S = 0;
                if (has_min_term<FMT>() && r.have) {
                    const _Float16* hc = reinterpret_cast<const _Float16*>(xq + L.hcodes) +
                                         am * K + 32 * (int64_t)(SB * h + sk);
#pragma unroll
                    for (int i = 0; i < 32; i++) S += (int)(float)hc[i];
                }
                lds_part.S[sk][sr] = S;
                lds_part.mn[sk][sr] = f.mn;
            }
        }
        // B2: the W tile is staged; this wave's activation loads of step h
        // completed before its weight loads of step h were consumed above
        __syncthreads();
        if (h + 1 < H) {
            issue_a(h + 1, std::integral_constant<int, 1 - PB>{});  // in flight while step h is multiplied
            fetch(h + 1, r);
        }
        const uint4* A = a_buf(par);
        // the multiply of one step; UNF: Q6_K codes were staged without their
        // sub-scales (a scale that cannot be folded exactly occurs in the step)
        auto multiply = [&](auto unf_tag) {
            constexpr bool UNF = decltype(unf_tag)::value;
#pragma unroll
            for (int bk = 0; bk < SB; bk++) {
                if (bk < nbh) {
                    v8h Af[WT][2], Bf[2], Ra[WT], Rw;
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
#pragma unroll
                        for (int i = 0; i < WT; i++) {
                            const uint4 va = A[slot(arow0 + 32 * i, 4 * bk + 2 * hh + kq)];
                            __builtin_memcpy(&Af[i][hh], &va, 16);
                        }
                        const uint4 vb = sm->w[slot(brow, 4 * bk + 2 * hh + kq)];
                        __builtin_memcpy(&Bf[hh], &vb, 16);
                    }
                    {
#pragma unroll
                        for (int i = 0; i < WT; i++) {
                            const uint4 ri = sm->ra[bk][kq ? TM : arow0 + 32 * i];
                            __builtin_memcpy(&Ra[i], &ri, 16);
                        }
                        const uint4 rb = sm->rw[bk][brow];
                        __builtin_memcpy(&Rw, &rb, 16);
                    }
                    const uint32_t x1 = (has_min_term<FMT>() || FMT == T_Q6_K) ? sm->x1[bk][brow] : 0u;
                    if constexpr (PART) {
                        // the exact integers of the block, as the MFMAs form them
                        constexpr int per = has_min_term<FMT>() ? 2 : 1;
                        const int64_t n = n0 + brow, b = (int64_t)SB * h + bk;
#pragma unroll
                        for (int i = 0; i < WT; i++) {
                            v16f I;
                            if constexpr (FMT == T_Q6_K && UNF) {
                                const v16f I0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][0], Bf[0], zero16, 0, 0, 0);
                                const v16f I1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][1], Bf[1], zero16, 0, 0, 0);
                                const float s0 = (float)(int16_t)(x1 & 0xFFFF), s1 = (float)((int)x1 >> 16);
#pragma unroll
                                for (int e = 0; e < 16; e++) I[e] = fmaf(s0, I0[e], s1 * I1[e]);
                            } else {
                                I = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][0], Bf[0], zero16, 0, 0, 0);
                                I = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][1], Bf[1], I, 0, 0, 0);
                            }
#pragma unroll
                            for (int e = 0; e < 16; e++) {
                                const int rl = 32 * WT * wm + 32 * i + 8 * (e >> 2) + 4 * kq + (e & 3);
                                const int64_t m = m0 + rl;
                                if (m < M && n < N) {
                                    int32_t* o = P + ((m * N + n) * nb + b) * per;
                                    o[0] = (int32_t)I[e];
                                    if constexpr (per == 2) {
                                        const int S = lds_part.S[bk][rl];
                                        o[1] = FMT == T_Q4_K ? lds_part.mn[bk][brow] * S : S;
                                    }
                                }
                            }
                        }
                        continue;
                    }
#pragma unroll
                    for (int i = 0; i < WT; i++) {
                        const v16f S = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ra[i], Rw, zero16, 0, 0, 0);
                        if constexpr (FMT == T_Q6_K && UNF) {
                            const v16f I0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][0], Bf[0], zero16, 0, 0, 0);
                            const v16f I1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][1], Bf[1], zero16, 0, 0, 0);
                            const float s0 = (float)(int16_t)(x1 & 0xFFFF), s1 = (float)((int)x1 >> 16);
#pragma unroll
                            for (int e = 0; e < 16; e++) {
                                const float I = fmaf(s0, I0[e], s1 * I1[e]);  // exact integer
                                p[i][e] = fmaf(I, S[e], p[i][e]);
                            }
                        } else {
                            v16f I = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][0], Bf[0], zero16, 0, 0, 0);
                            I = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i][1], Bf[1], I, 0, 0, 0);
#pragma unroll
                            for (int e = 0; e < 16; e++) p[i][e] = fmaf(I[e], S[e], p[i][e]);
                            if constexpr (has_min_term<FMT>()) {
                                // element e of the lane is row 8(e/4) + 4kq + e%4 of the tile
                                const float nX = -__uint_as_float(x1);
                                const float* cr = &sm->ca[bk][32 * WT * wm + 32 * i + 4 * kq];
#pragma unroll
                                for (int g = 0; g < 4; g++) {
                                    const float4 c4 = *reinterpret_cast<const float4*>(cr + 8 * g);
                                    p[i][4 * g + 0] = fmaf(nX, c4.x, p[i][4 * g + 0]);
                                    p[i][4 * g + 1] = fmaf(nX, c4.y, p[i][4 * g + 1]);
                                    p[i][4 * g + 2] = fmaf(nX, c4.z, p[i][4 * g + 2]);
                                    p[i][4 * g + 3] = fmaf(nX, c4.w, p[i][4 * g + 3]);
                                }
                            }
                        }
                    }
                }
            }
        };
        if (FMT == T_Q6_K && unfolded)
            multiply(std::true_type{});
        else
            multiply(std::false_type{});
        // end of a 256-element chunk (two steps) or of K: add it, in chunk order
        if ((h & 1) || h + 1 == H) {
#pragma unroll
            for (int i = 0; i < WT; i++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    yv[i][e] = yv[i][e] + p[i][e];
                    p[i][e] = 0.0f;
                }
        }
    };

    Raw r;
    issue_a(0, Even{});
    fetch(0, r);
    for (int h = 0; h < H; h += 2) {
        step(h, r, Even{});
        if (h + 1 < H) step(h + 1, r, Odd{});
    }

    if constexpr (PART) return;
    // lane l, element e of tile i: row 8(e/4) + 4kq + e%4, column lr
    const int64_t n = n0 + 32 * wn + lr;
#pragma unroll
    for (int i = 0; i < WT; i++)
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int64_t m = m0 + 32 * WT * wm + 32 * i + 8 * (e >> 2) + 4 * kq + (e & 3);
            if (m < M && n < N) y[m * N + n] = yv[i][e];
        }
}

// Workgroups of 128 x 128 outputs, unless so few of them cover the output
// that half the 256 CUs or more would idle: then 64 x 64 tiles (four times
// the workgroups; measured slower per output than the larger tile, faster
// when the larger one leaves most of the chip empty).
template <int FMT>
int launch_gemm_t(const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                  float* y, int32_t* P, hipStream_t s) {
    const ActLayout L = act_layout(M, K);
    int64_t tilesM = (M + 127) / 128, tilesN = (N + 127) / 128;
    if (tilesM * tilesN > 128) {
        if (P)
            hipLaunchKernelGGL((k_gemm<FMT, 8, true>), dim3((unsigned)(tilesM * tilesN)), dim3(512),
                               0, s, w, N, K, xq, L, M, tilesM, tilesN, y, P);
        else
            hipLaunchKernelGGL((k_gemm<FMT, 8>), dim3((unsigned)(tilesM * tilesN)), dim3(512), 0,
                               s, w, N, K, xq, L, M, tilesM, tilesN, y, P);
    } else {
        tilesM = (M + 63) / 64;
        tilesN = (N + 63) / 64;
        if (P)
            hipLaunchKernelGGL((k_gemm<FMT, 4, true>), dim3((unsigned)(tilesM * tilesN)), dim3(256),
                               0, s, w, N, K, xq, L, M, tilesM, tilesN, y, P);
        else
            hipLaunchKernelGGL((k_gemm<FMT, 4>), dim3((unsigned)(tilesM * tilesN)), dim3(256), 0,
                               s, w, N, K, xq, L, M, tilesM, tilesN, y, P);
    }
    return (int)hipGetLastError();
}

}  // namespace

int launch_gemm(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                float* y, hipStream_t s, int32_t* P) {
    switch (type) {
    case T_Q8_0: return launch_gemm_t<T_Q8_0>(w, N, K, xq, M, y, P, s);
    case T_Q4_0: return launch_gemm_t<T_Q4_0>(w, N, K, xq, M, y, P, s);
    case T_Q5_0: return launch_gemm_t<T_Q5_0>(w, N, K, xq, M, y, P, s);
    case T_Q4_1: return launch_gemm_t<T_Q4_1>(w, N, K, xq, M, y, P, s);
    case T_Q5_1: return launch_gemm_t<T_Q5_1>(w, N, K, xq, M, y, P, s);
    case T_Q8_1: return launch_gemm_t<T_Q8_1>(w, N, K, xq, M, y, P, s);
    case T_Q4_K: return launch_gemm_t<T_Q4_K>(w, N, K, xq, M, y, P, s);
    case T_Q6_K: return launch_gemm_t<T_Q6_K>(w, N, K, xq, M, y, P, s);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace qmv
