// HIP kernels for gfx950 (CDNA4): Q8_0 activation quantisation and the fused
// dequantise-and-multiply of GGUF block-quantised weights (Q8_0, Q4_0, Q4_K,
// Q6_K) against Q8_0 activations.
//
// The method (llamay "Architecture", section "The package map": the fused W4A8
// kernels of pkg/quant behind MatVec / MatMul of pkg/tensor) multiplies block
// codes in integers and applies the fp16 block scales afterwards.  Here the
// integer block dots run on int8 MFMA (v_mfma_i32_16x16x32_i8: one 32-element
// block per instruction, 16 activation rows x 16 weight rows), and the f32
// scale-and-accumulate follows one fixed order for every launch shape (see
// include/qmv.h), so a row's result never depends on the batch around it
// (llamay docs front page, "The three claims": determinism, claimed for any
// mix of requests in a batch).
//
// Decode is memory-bound ("Architecture", bench transcript), so the weight
// stream is the thing to get right: each wave owns 16 weight rows and walks
// their 256-element chunks; the 16 row spans of a chunk are fetched with
// coalesced 16-byte loads into the wave's LDS slice, one chunk ahead (register
// prefetch), and every lane then decodes its 8 codes of a block straight from
// LDS at whatever byte alignment the GGUF layout leaves them.
//
// Built with -ffp-contract=off: every float operation below is the one
// written, in the order written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <utility>

#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int T_Q4_0 = 2, T_Q4_1 = 3, T_Q5_0 = 6, T_Q5_1 = 7, T_Q8_0 = 8, T_Q8_1 = 9,
              T_Q4_K = 12, T_Q6_K = 14;
// Formats whose block term has a second, minimum part fed by the activation
// code sums: Q4_K (sub-block mins, subtracted) and Q4_1 / Q5_1 (d*q + m).
template <int FMT> constexpr bool has_min_term() {
    return FMT == T_Q4_K || FMT == T_Q4_1 || FMT == T_Q5_1;
}

// Batch sizes up to this run on the lane-per-chunk v_dot4 kernel, larger ones on MFMA.
constexpr int DOT_MAX_ROWS = 4;
// ... as long as their activation rows fit in a workgroup's LDS.
constexpr int DOT_MAX_ACT_LDS = 96 * 1024;
// On the Q8_K path, batches from this size up to 16 rows run the batched
// MFMA kernel (k_bdot8k), smaller ones the lane-per-chunk kernel.
constexpr int BDOT_MIN_ROWS = 5;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    _Float16 f;
    __builtin_memcpy(&f, &h, 2);
    return (float)f;
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
    _Float16 f = (_Float16)x;  // round to nearest even, subnormals kept
    uint16_t h;
    __builtin_memcpy(&h, &f, 2);
    return h;
}

template <typename T>
__device__ __forceinline__ T ld(const uint8_t* p) {
    T v;
    __builtin_memcpy(&v, p, sizeof(T));
    return v;
}

// ------------------------------------------------------------ quantise ----
// id = 1/d, or 0 when 1/d is not finite in f32 (d == 0, or d below about
// 2^-128, a subnormal amax): such a block gets all-zero codes, like an
// all-zero block (its fp16 scale is 0 anyway), instead of the undefined
// integer conversion of an infinite x * id.
__device__ __forceinline__ float inv_scale(float d) {
    const float r = 1.0f / d;
    return __builtin_isinf(r) ? 0.0f : r;
}

// Q8_0 of one 32-element block: amax, d = amax/127 (correctly rounded f32
// divide), id = inv_scale(d), codes = round-half-away(x*id),
// stored scale fp16(d); dval = f32 value of the stored scale.  A16: xb is
// 16-byte aligned (float4 loads); otherwise only 4-byte alignment is assumed.
template <bool A16>
__device__ __forceinline__ void quant_block(const float* __restrict__ xb, uint8_t (&q)[32],
                                            uint16_t& h, float& dval) {
    float v[32];
    if constexpr (A16) {
        const float4* x4 = reinterpret_cast<const float4*>(xb);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float4 f = x4[j];
            v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++) v[i] = xb[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    const float d = amax / 127.0f;
    const float id = inv_scale(d);
#pragma unroll
    for (int i = 0; i < 32; i++) q[i] = (uint8_t)(int8_t)(int)roundf(v[i] * id);
    h = float_to_half_bits(d);
    dval = half_bits_to_float(h);
}

__device__ __forceinline__ void store_public(uint8_t* pub, const uint8_t (&q)[32], uint16_t h) {
    uint8_t blk[34];
    blk[0] = (uint8_t)(h & 255);
    blk[1] = (uint8_t)(h >> 8);
#pragma unroll
    for (int i = 0; i < 32; i++) blk[2 + i] = q[i];
    __builtin_memcpy(pub, blk, 34);
}

// Sum of the block's codes, and the two int16 half sums packed (low = 0..15).
__device__ __forceinline__ void code_sums(const uint8_t (&q)[32], int& S, int32_t& s16) {
    int lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) lo += (int8_t)q[i];
#pragma unroll
    for (int i = 16; i < 32; i++) hi += (int8_t)q[i];
    S = lo + hi;
    s16 = (int32_t)(((uint32_t)lo & 0xFFFFu) | ((uint32_t)hi << 16));
}

// The row-major staging of block b of row r (the lane-per-chunk kernels).
__device__ __forceinline__ void store_row_staging(uint8_t* xq, const ActLayout& L, int64_t r,
                                                  int64_t K, int64_t b, const uint8_t (&q)[32],
                                                  float dval, int S, int32_t s16) {
    const int64_t nb = L.nb;
    uint4* rc = reinterpret_cast<uint4*>(xq + L.rcodes + r * K + 32 * b);
    uint32_t wv[8];
    __builtin_memcpy(wv, q, 32);
    rc[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    rc[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
    reinterpret_cast<float*>(xq + L.rda)[r * nb + b] = dval;
    reinterpret_cast<float*>(xq + L.rca)[r * nb + b] = dval * (float)S;
    reinterpret_cast<int32_t*>(xq + L.rs16)[r * nb + b] = s16;
}

// Quantise x (or, FROM_PUBLIC, take codes and d from the Q8_0 blocks already
// in xq) and write the staging copies selected by `staging`.  One thread per
// (row, block); with ST_MFMA over the 16-row-padded range, whose padding
// rows get zero codes and scales in that copy.
// One 32-block quantised by an aligned group of 8 lanes, 4 elements each
// (lane sub = lane & 7 holds elements 4 sub .. 4 sub + 3): the amax and the
// code sums by lane shuffles (every lane of the wave takes part), then each
// live lane writes its 4 codes into the public block at pub and into the row
// staging at rc, and lane 0 of the group the scale and sums at index bi of
// rda / rca / rs16.  The arithmetic per element is quant_block's, so the
// bytes are the same as k_quantize's.
__device__ __forceinline__ void quant_block8(const float (&v)[4], int sub, bool live, uint8_t* pub,
                                             uint8_t* rc, float* rda, float* rca, int32_t* rs16,
                                             int64_t bi) {
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float d = amax / 127.0f;
    const float id = inv_scale(d);
    uint32_t c4 = 0;
    int s4 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int c = (int)roundf(v[i] * id);
        c4 |= ((uint32_t)c & 0xFFu) << (8 * i);
        s4 += c;
    }
    int s16 = s4 + __shfl_xor(s4, 1);
    s16 += __shfl_xor(s16, 2);               // the sum of this lane's 16-code half
    const int s16o = __shfl_xor(s16, 4);     // the other half's
    if (!live) return;
    const uint16_t h = float_to_half_bits(d);
    const float dval = half_bits_to_float(h);
    uint16_t* pc = reinterpret_cast<uint16_t*>(pub + 2 + 4 * sub);  // 2-byte aligned
    pc[0] = (uint16_t)(c4 & 0xFFFFu);
    pc[1] = (uint16_t)(c4 >> 16);
    *reinterpret_cast<uint32_t*>(rc + 4 * sub) = c4;
    if (sub == 0) {
        *reinterpret_cast<uint16_t*>(pub) = h;
        rda[bi] = dval;
        rca[bi] = dval * (float)(s16 + s16o);
        rs16[bi] = (int32_t)(((uint32_t)s16 & 0xFFFFu) | ((uint32_t)s16o << 16));
    }
}

template <bool FROM_PUBLIC, bool A16>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ x,
                                                  uint8_t* __restrict__ xq, int64_t rows,
                                                  int64_t K, ActLayout L, int staging) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nb = L.nb;
    const int64_t span = (staging & ST_MFMA) ? 16 * L.G : rows;
    if (t >= span * nb) return;
    const int64_t r = t / nb, b = t - r * nb;
    uint8_t q[32];
    float dval = 0.0f;
    if (r < rows) {
        uint8_t* pub = xq + (r * nb + b) * 34;
        if (!FROM_PUBLIC) {
            uint16_t h;
            quant_block<A16>(x + r * K + 32 * b, q, h, dval);
            store_public(pub, q, h);
        } else {
            uint8_t blk[34];
            __builtin_memcpy(blk, pub, 34);
#pragma unroll
            for (int i = 0; i < 32; i++) q[i] = blk[2 + i];
            dval = half_bits_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++) q[i] = 0;
    }
    int S;
    int32_t s16;
    code_sums(q, S, s16);
    if (staging & ST_MFMA) {
        const int64_t g = r >> 4;
        const int m = (int)(r & 15);
        const int64_t gb = g * nb + b;
        uint8_t* codes = xq + L.codes + gb * 512;
#pragma unroll
        for (int kg = 0; kg < 4; kg++) {
            uint64_t v = 0;
#pragma unroll
            for (int j = 0; j < 8; j++) v |= (uint64_t)q[8 * kg + j] << (8 * j);
            *reinterpret_cast<uint64_t*>(codes + (m + 16 * kg) * 8) = v;
        }
        reinterpret_cast<float*>(xq + L.da)[gb * 16 + m] = dval;
        reinterpret_cast<float*>(xq + L.ca)[gb * 16 + m] = dval * (float)S;
        reinterpret_cast<int32_t*>(xq + L.S)[gb * 16 + m] = S;
    }
    if (r >= rows) return;
    if (staging & ST_ROW) store_row_staging(xq, L, r, K, b, q, dval, S, s16);
    if (staging & ST_F16) {
        // f16 copy for the GEMM (code values are exact in f16), and d_a * S
        uint4* hc = reinterpret_cast<uint4*>(xq + L.hcodes + (r * K + 32 * b) * 2);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t hw[4];
#pragma unroll
            for (int t2 = 0; t2 < 4; t2++) {
                const _Float16 lo = (_Float16)(float)(int8_t)q[8 * j + 2 * t2];
                const _Float16 hi = (_Float16)(float)(int8_t)q[8 * j + 2 * t2 + 1];
                uint16_t ul, uh;
                __builtin_memcpy(&ul, &lo, 2);
                __builtin_memcpy(&uh, &hi, 2);
                hw[t2] = (uint32_t)ul | ((uint32_t)uh << 16);
            }
            hc[j] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        }
        uint16_t dbits = 0;
        {
            const _Float16 dh = (_Float16)dval;  // exact: dval came from fp16
            __builtin_memcpy(&dbits, &dh, 2);
        }
        reinterpret_cast<uint16_t*>(xq + L.hda)[r * nb + b] = dbits;
        reinterpret_cast<float*>(xq + L.rca)[r * nb + b] = dval * (float)S;
    }
}

// ------------------------------------------------------------- formats ----
// QK: elements per GGUF block; BB: bytes per block; CB: bytes of one full
// 256-element chunk of a row; PPS: 16-byte pieces that cover one chunk span
// at the worst alignment the layout allows (Q4_K spans are always 16-byte
// aligned: 144 | 16*9 and w is 16-byte aligned; the others only 2-byte).
template <int FMT> struct Fmt;
template <> struct Fmt<T_Q8_0> { static constexpr int QK = 32, BB = 34, CB = 272, PPS = 18; };
template <> struct Fmt<T_Q4_0> { static constexpr int QK = 32, BB = 18, CB = 144, PPS = 10; };
template <> struct Fmt<T_Q5_0> { static constexpr int QK = 32, BB = 22, CB = 176, PPS = 12; };
// 20-, 24- and 36-byte blocks keep every span 4-byte aligned
template <> struct Fmt<T_Q4_1> { static constexpr int QK = 32, BB = 20, CB = 160, PPS = 11; };
template <> struct Fmt<T_Q5_1> { static constexpr int QK = 32, BB = 24, CB = 192, PPS = 13; };
template <> struct Fmt<T_Q8_1> { static constexpr int QK = 32, BB = 36, CB = 288, PPS = 19; };
template <> struct Fmt<T_Q4_K> { static constexpr int QK = 256, BB = 144, CB = 144, PPS = 9; };
template <> struct Fmt<T_Q6_K> { static constexpr int QK = 256, BB = 210, CB = 210, PPS = 14; };

template <int FMT> constexpr int span_stride() { return 16 * Fmt<FMT>::PPS + 16; }
template <int FMT> constexpr int F_QK() { return Fmt<FMT>::QK; }
template <int FMT> constexpr int F_BB() { return Fmt<FMT>::BB; }
template <int FMT> constexpr int pieces_per_lane() { return (16 * Fmt<FMT>::PPS + 63) / 64; }

// ------------------------------------------------------- weight stream ----
// A tile is 16 consecutive weight rows; its bytes are one contiguous range
// [n0*R, (n0+16)*R) of the blob.  Offsets inside a tile fit in 32 bits
// (16 * R <= 16 * (2^20/32) * 34 bytes).
struct TileRef {
    const uint8_t* base;  // w + n0*R
    int nrows;            // rows of the tile that exist (1..16)
    uint32_t left;        // blob bytes from base to the end of the blob
    bool fast;            // whole tile present and >= 16 bytes of blob after it
};

__device__ __forceinline__ TileRef make_tile(const uint8_t* w, int64_t wbytes, int64_t N,
                                             int64_t R, int64_t tile) {
    TileRef t;
    const int64_t n0 = tile * 16;
    t.base = w + n0 * R;
    t.nrows = (int)(N - n0 < 16 ? N - n0 : 16);
    const int64_t left = wbytes - n0 * R;
    t.left = (uint32_t)(left < 0x7fffffff ? left : 0x7fffffff);
    t.fast = t.nrows == 16 && 16 * R + 16 <= left;
    return t;
}

// Global -> registers: the 16 row spans of chunk c, as 16-byte pieces aligned
// down from each span start.  Piece p of the wave is lane p%64 of step p/64;
// it belongs to span p/PPS at offset 16*(p%PPS).  Pieces past a span's end
// are not loaded.  Only the last tile of a blob takes the guarded path, which
// reads its final partial piece bytewise instead of running past the blob.
// The two paths are separate loops: interleaved per piece, the merge after
// each piece makes the compiler wait for every load already issued before it
// may write the next piece's register, leaving one piece in flight per lane.
template <int FMT>
__device__ __forceinline__ void fetch_chunk(const TileRef& t, uint32_t R, int c, int nbc,
                                            int lane, uint4 (&reg)[pieces_per_lane<FMT>()]) {
    using F = Fmt<FMT>;
    const uint32_t len = F::QK == 32 ? nbc * F::BB : F::BB;
    if (t.fast) {
#pragma unroll
        for (int k = 0; k < pieces_per_lane<FMT>(); k++) {
            const int p = k * 64 + lane;
            const int n = p / F::PPS, j = p - n * F::PPS;
            const uint32_t s = n * R + c * F::CB;
            const uint32_t off = (s & ~15u) + 16 * j;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (n < 16 && off < s + len) v = *reinterpret_cast<const uint4*>(t.base + off);
            reg[k] = v;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < pieces_per_lane<FMT>(); k++) {
        const int p = k * 64 + lane;
        const int n = p / F::PPS, j = p - n * F::PPS;
        const uint32_t s = n * R + c * F::CB;
        const uint32_t off = (s & ~15u) + 16 * j;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < t.nrows && off < s + len) {
            if (off + 16 <= t.left) {
                v = *reinterpret_cast<const uint4*>(t.base + off);
            } else {
                uint32_t b[4] = {0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 16; i++)
                    if (off + i < t.left) b[i >> 2] |= (uint32_t)t.base[off + i] << (8 * (i & 3));
                v = make_uint4(b[0], b[1], b[2], b[3]);
            }
        }
        reg[k] = v;
    }
}

template <int FMT>
__device__ __forceinline__ void stage_chunk(uint8_t* wl, int lane,
                                            const uint4 (&reg)[pieces_per_lane<FMT>()]) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int k = 0; k < pieces_per_lane<FMT>(); k++) {
        const int p = k * 64 + lane;
        const int n = p / F::PPS, j = p - n * F::PPS;
        if (n < 16) *reinterpret_cast<uint4*>(wl + n * span_stride<FMT>() + 16 * j) = reg[k];
    }
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Q5_0 fifth bits: the 4 bits of h (0..15) moved to bit 4 of bytes 0..3.
// h * 0x204081 places copies of h at bits 0, 7, 14 and 21 with no carries,
// so bit 8j of the product is bit j of h.
__device__ __forceinline__ uint32_t spread4(uint32_t h) {
    return (__umul24(h, 0x204081u) & 0x01010101u) << 4;
}

// Bytewise x - bias for bytes x in [0, 2*bias): add 128, subtract, flip bit 7
// (no borrow crosses a byte because every byte of x|0x80.. is >= 128).
__device__ __forceinline__ uint64_t bytes_minus(uint64_t x, uint64_t bias8) {
    const uint64_t hi = 0x8080808080808080ull;
    return ((x | hi) - bias8) ^ hi;
}

// ---------------------------------------------------- activation stream ----
// Activation side of one chunk: the lane's A operand of each of the 8 blocks,
// and 2 of the chunk's 8 x 16 scale values (da, and ca for Q4_K).  The
// staging copy always holds 16 rows per group (padding rows are zero), so
// the loads need no row guard.
struct ActRef {
    const uint8_t* codes;  // group's codes + lane*8
    const float* da;       // group's da
    const float* ca;       // group's ca
};

__device__ __forceinline__ ActRef make_act(const uint8_t* xq, const ActLayout& L, int64_t g,
                                           int lane) {
    ActRef a;
    a.codes = xq + L.codes + g * L.nb * 512 + lane * 8;
    a.da = reinterpret_cast<const float*>(xq + L.da) + g * L.nb * 16;
    a.ca = reinterpret_cast<const float*>(xq + L.ca) + g * L.nb * 16;
    return a;
}

struct ActRegs {
    long a[8];
    float2 da, ca;
};

template <int FMT>
__device__ __forceinline__ void fetch_act(const ActRef& A, int c, int nbc, int lane,
                                          ActRegs& r) {
#pragma unroll
    for (int bb = 0; bb < 8; bb++)
        r.a[bb] = bb < nbc ? *reinterpret_cast<const long*>(A.codes + (8 * c + bb) * 512) : 0;
    const int sb = lane >> 3;   // scale block: 8 blocks x 16 rows, two per lane
    const int sbc = sb < nbc ? sb : nbc - 1;
    const uint32_t o = (8 * c + sbc) * 16 + 2 * (lane & 7);
    float2 da = *reinterpret_cast<const float2*>(A.da + o);
    float2 ca = make_float2(0.f, 0.f);
    if (has_min_term<FMT>()) ca = *reinterpret_cast<const float2*>(A.ca + o);
    const bool ok = sb < nbc;
    r.da = ok ? da : make_float2(0.f, 0.f);
    r.ca = ok ? ca : make_float2(0.f, 0.f);
}

// ------------------------------------------------------------ one chunk ----
// The 8 (or fewer) blocks of chunk c for the 16 rows staged at wl and the
// activation rows of the A operand.  Lane (nn = l%16, kg = l/16) decodes its
// row's 8 codes of each block; the MFMA result of lane l, element i, is
// (activation row 4*kg + i, weight row nn).  Non-PARTIALS: p[i] is the chunk
// sum of rows 4*kg + i for i < NI (NI = 1, 2 or 4 rows per lane are needed).
// PARTIALS: the exact integer partials are written to P instead.
struct PartialsOut {
    int32_t* P;
    const int32_t* S;  // group's S + 4*kg
    int64_t N, row0, n;
    int nb, Bg, nrows;
};

template <int FMT, int NI, bool PARTIALS>
__device__ __forceinline__ void chunk_math(const uint8_t* rb, const float* sl, const long (&acur)[8],
                                           int c, int nbc, int kg, float (&p)[NI],
                                           const PartialsOut& po) {
    // All LDS reads of the chunk are issued first (the lane's weight bytes of
    // every block and its rows' activation scales), so the wave pays one LDS
    // round trip per chunk rather than one per block.  Blocks past nbc read
    // bytes inside the wave's slice that are never used.
    uint64_t q[8];       // per block (Q8_0, Q4_0); per 32-byte quarter (Q4_K, Q6_K ql)
    uint16_t dq[8];      // per-block fp16 d (Q8_0, Q4_0)
    uint64_t qh[2];      // Q6_K high bits, per 128-element half
    uint32_t h5[8];      // Q5_0, Q5_1: the block's fifth bits, the lane's 8 in the low byte
    uint16_t mq[8];      // Q4_1, Q5_1: per-block fp16 m
    uint4 hdr;           // Q4_K: d, dmin, 12 scale bytes; Q6_K: the 16 sub-scales
    uint16_t d6 = 0;     // Q6_K d
    if (F_QK<FMT>() == 32) {
        // field offsets: codes, fifth-bit word
        constexpr int QS = FMT == T_Q8_0 ? 2 : FMT == T_Q8_1 ? 4 : FMT == T_Q4_0 ? 2
                         : FMT == T_Q4_1 ? 4 : FMT == T_Q5_0 ? 6 : 8;
        constexpr int QH = FMT == T_Q5_0 ? 2 : 4;
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
            const uint8_t* blk = rb + F_BB<FMT>() * bb;
            dq[bb] = ld<uint16_t>(blk);
            if (FMT == T_Q8_0 || FMT == T_Q8_1) {
                q[bb] = ld<uint64_t>(blk + QS + 8 * kg);
            } else {
                // lanes kg = 2, 3 take the high nibbles: one per-lane shift
                q[bb] = ld<uint64_t>(blk + QS + 8 * (kg & 1)) >> (2 * (kg & 2));
            }
            if (FMT == T_Q5_0 || FMT == T_Q5_1) h5[bb] = ld<uint32_t>(blk + QH) >> (8 * kg);
            if (FMT == T_Q4_1 || FMT == T_Q5_1) mq[bb] = ld<uint16_t>(blk + 2);
        }
    } else if (FMT == T_Q4_K) {
        hdr = ld<uint4>(rb);
#pragma unroll
        for (int j = 0; j < 4; j++) q[j] = ld<uint64_t>(rb + 16 + 32 * j + 8 * kg);
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++) q[j] = ld<uint64_t>(rb + 32 * j + 8 * kg);
        qh[0] = ld<uint64_t>(rb + 128 + 8 * kg);
        qh[1] = ld<uint64_t>(rb + 160 + 8 * kg);
        hdr = ld<uint4>(rb + 192);
        d6 = ld<uint16_t>(rb + 208);
    }
    float dav[8][4], cav[8][4];
    if (!PARTIALS) {
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
            const float* sp = sl + bb * 16 + 4 * kg;
#pragma unroll
            for (int i = 0; i < 4; i++) dav[bb][i] = cav[bb][i] = 0.0f;
            if (NI == 1) {
                dav[bb][0] = sp[0];
                if (has_min_term<FMT>()) cav[bb][0] = sp[128];
            } else if (NI == 2) {
                const float2 d2 = *reinterpret_cast<const float2*>(sp);
                dav[bb][0] = d2.x; dav[bb][1] = d2.y;
                if (has_min_term<FMT>()) {
                    const float2 c2 = *reinterpret_cast<const float2*>(sp + 128);
                    cav[bb][0] = c2.x; cav[bb][1] = c2.y;
                }
            } else {
                const float4 d4 = *reinterpret_cast<const float4*>(sp);
                dav[bb][0] = d4.x; dav[bb][1] = d4.y; dav[bb][2] = d4.z; dav[bb][3] = d4.w;
                if (has_min_term<FMT>()) {
                    const float4 c4 = *reinterpret_cast<const float4*>(sp + 128);
                    cav[bb][0] = c4.x; cav[bb][1] = c4.y; cav[bb][2] = c4.z; cav[bb][3] = c4.w;
                }
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // per-chunk fields of the K-quant superblock
    float dw = 0.0f, dmw = 0.0f;
    uint32_t s12[3] = {hdr.y, hdr.z, hdr.w};
    if (FMT == T_Q4_K) {
        dw = half_bits_to_float((uint16_t)(hdr.x & 0xFFFF));
        dmw = half_bits_to_float((uint16_t)(hdr.x >> 16));
    }
    if (FMT == T_Q6_K) dw = half_bits_to_float(d6);
    const uint32_t sc6[4] = {hdr.x, hdr.y, hdr.z, hdr.w};
#pragma unroll
    for (int i = 0; i < NI; i++) p[i] = 0.0f;

#pragma unroll
    for (int bb = 0; bb < 8; bb++) {
        if (F_QK<FMT>() == 32 && bb >= nbc) break;
        const long a = acur[bb];
        const v4i zero = {0, 0, 0, 0};
        // Exact integer partial of (row 4kg+i, this lane's weight row).  The
        // K-quant sub-scale products use the full-rate 24-bit multiply: the
        // MFMA sums (|.| < 2^16) and the 6- or 8-bit scales fit its operands.
        v4i I;
        int mn = 0;
        if (FMT == T_Q8_0 || FMT == T_Q8_1) {
            dw = half_bits_to_float(dq[bb]);
            I = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, (long)q[bb], zero, 0, 0, 0);
        } else if (FMT == T_Q4_1) {
            dw = half_bits_to_float(dq[bb]);
            mn = 1;
            I = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, (long)(q[bb] & 0x0F0F0F0F0F0F0F0Full), zero,
                                                     0, 0, 0);
        } else if (FMT == T_Q5_1) {
            dw = half_bits_to_float(dq[bb]);
            mn = 1;
            const uint64_t b5 = ((uint64_t)spread4((h5[bb] >> 4) & 15u) << 32) | spread4(h5[bb] & 15u);
            I = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                a, (long)((q[bb] & 0x0F0F0F0F0F0F0F0Full) | b5), zero, 0, 0, 0);
        } else if (FMT == T_Q4_0) {
            dw = half_bits_to_float(dq[bb]);
            const uint64_t wc = bytes_minus(q[bb] & 0x0F0F0F0F0F0F0F0Full, 0x0808080808080808ull);
            I = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, (long)wc, zero, 0, 0, 0);
        } else if (FMT == T_Q5_0) {
            dw = half_bits_to_float(dq[bb]);
            const uint64_t b5 = ((uint64_t)spread4((h5[bb] >> 4) & 15u) << 32) | spread4(h5[bb] & 15u);
            const uint64_t wc = bytes_minus((q[bb] & 0x0F0F0F0F0F0F0F0Full) | b5, 0x1010101010101010ull);
            I = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, (long)wc, zero, 0, 0, 0);
        } else if (FMT == T_Q4_K) {
            // 6-bit scale and min of sub-block bb (two per 12 bytes)
            const uint8_t* sb = reinterpret_cast<const uint8_t*>(s12);
            int sc;
            if (bb < 4) {
                sc = sb[bb] & 63;
                mn = sb[bb + 4] & 63;
            } else {
                sc = (sb[bb + 4] & 15) | ((sb[bb - 4] >> 6) << 4);
                mn = (sb[bb + 4] >> 4) | ((sb[bb] >> 6) << 4);
            }
            uint64_t raw = q[bb >> 1];
            if (bb & 1) raw >>= 4;
            const v4i acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                a, (long)(raw & 0x0F0F0F0F0F0F0F0Full), zero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; i++) I[i] = __mul24(sc, acc[i]);
        } else {  // Q6_K
            const int h = bb >> 2, kq = bb & 3;
            uint64_t ql = q[2 * h + (kq & 1)];
            if (kq & 2) ql >>= 4;
            const uint64_t q6 = (ql & 0x0F0F0F0F0F0F0F0Full) |
                                (((qh[h] >> (2 * kq)) & 0x0303030303030303ull) << 4);
            const uint64_t wc = bytes_minus(q6, 0x2020202020202020ull);
            const uint32_t sw = sc6[bb >> 1] >> (16 * (bb & 1));
            const int s0 = (int8_t)(sw & 0xFF), s1 = (int8_t)((sw >> 8) & 0xFF);
            // the two 16-element halves carry different sub-scales: one MFMA
            // per half, the other half's codes zeroed
            const long lo = kg < 2 ? (long)wc : 0, hi = kg < 2 ? 0 : (long)wc;
            const v4i acc0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, lo, zero, 0, 0, 0);
            const v4i acc1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, hi, zero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; i++) I[i] = __mul24(s0, acc0[i]) + __mul24(s1, acc1[i]);
        }

        if (PARTIALS) {
            const int b = 8 * c + bb;
            int4 S4 = make_int4(0, 0, 0, 0);
            if (has_min_term<FMT>()) S4 = *reinterpret_cast<const int4*>(po.S + b * 16);
            const int Sv[4] = {S4.x, S4.y, S4.z, S4.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = 4 * kg + i;
                if (m < po.Bg && po.n < po.nrows) {
                    const int64_t o = ((po.row0 + m) * po.N + po.n) * po.nb + b;
                    if (has_min_term<FMT>()) {
                        po.P[2 * o] = I[i];
                        po.P[2 * o + 1] = mn * Sv[i];
                    } else {
                        po.P[o] = I[i];
                    }
                }
            }
        } else {
            // second term: Q4_K -(dmin m_j)(d_a S); Q4_1 / Q5_1 +m (d_a S)
            float cw = 0.0f;
            if (FMT == T_Q4_K) cw = -(dmw * (float)mn);
            if (FMT == T_Q4_1 || FMT == T_Q5_1) cw = half_bits_to_float(mq[bb]);
#pragma unroll
            for (int i = 0; i < NI; i++) {
                p[i] = fmaf((float)I[i], dw * dav[bb][i], p[i]);
                if (has_min_term<FMT>()) p[i] = fmaf(cw, cav[bb][i], p[i]);
            }
        }
    }
}

// ------------------------------------------------------------- kernels ----
// Each wave's LDS slice: the 16 row spans of its chunk, then the chunk's
// activation scales [2][8][16] f32 (da, ca).
template <int FMT> constexpr int wave_lds() { return 16 * span_stride<FMT>() + 1024; }

template <int FMT>
__device__ __forceinline__ void stage_all(uint8_t* wl, float* sl, int lane,
                                          const uint4 (&reg)[pieces_per_lane<FMT>()],
                                          const ActRegs& nxt, long (&acur)[8]) {
    stage_chunk<FMT>(wl, lane, reg);
    *reinterpret_cast<float2*>(sl + 2 * lane) = nxt.da;
    if (has_min_term<FMT>()) *reinterpret_cast<float2*>(sl + 128 + 2 * lane) = nxt.ca;
#pragma unroll
    for (int bb = 0; bb < 8; bb++) acur[bb] = nxt.a[bb];
    wave_sync();
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Tall matrices: every wave is independent and walks whole tiles, chunk after
// chunk, keeping one chunk of prefetch in flight across tile boundaries.
template <int FMT, int NI>
__global__ __launch_bounds__(256) void k_qmv_rows(const uint8_t* __restrict__ w, int64_t wbytes,
                                                  int64_t N, int64_t K,
                                                  const uint8_t* __restrict__ xq, ActLayout L,
                                                  int64_t rows, int64_t tiles,
                                                  float* __restrict__ y) {
    using F = Fmt<FMT>;
    constexpr int NP = pieces_per_lane<FMT>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    uint8_t* wl = smem + wv * wave_lds<FMT>();
    float* sl = reinterpret_cast<float*>(wl + 16 * span_stride<FMT>());
    const int nb = (int)(K >> 5), C = (nb + 7) >> 3;
    const int64_t Rl = (K / F::QK) * F::BB;
    const uint32_t R = (uint32_t)Rl;
    const int nn = lane & 15, kg = lane >> 4;
    const int64_t TG = tiles * L.G;
    const int64_t TW = (int64_t)gridDim.x * (blockDim.x >> 6);
    int64_t tg = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
    if (tg >= TG) return;

    uint4 reg[NP];
    ActRegs nxt;
    long acur[8];
    int c = 0;
    TileRef t = make_tile(w, wbytes, N, Rl, tg % tiles);
    ActRef A = make_act(xq, L, tg / tiles, lane);
    {
        const int nbc = F::QK == 32 ? min(8, nb) : 8;
        fetch_chunk<FMT>(t, R, 0, nbc, lane, reg);
        fetch_act<FMT>(A, 0, nbc, lane, nxt);
    }
    float yacc[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) yacc[i] = 0.0f;
    const PartialsOut none{};
    while (true) {
        const int nbc = F::QK == 32 ? min(8, nb - 8 * c) : 8;
        stage_all<FMT>(wl, sl, lane, reg, nxt, acur);
        const TileRef tc = t;
        const int64_t tgc = tg;
        const int cc = c;
        // advance to the next item and prefetch it
        if (++c == C) {
            c = 0;
            tg += TW;
            if (tg < TG) {
                t = make_tile(w, wbytes, N, Rl, tg % tiles);
                A = make_act(xq, L, tg / tiles, lane);
            }
        }
        if (tg < TG) {
            const int nbcn = F::QK == 32 ? min(8, nb - 8 * c) : 8;
            fetch_chunk<FMT>(t, R, c, nbcn, lane, reg);
            fetch_act<FMT>(A, c, nbcn, lane, nxt);
        }
        const uint8_t* rb = wl + nn * span_stride<FMT>() + ((nn * R + cc * F::CB) & 15);
        float p[NI];
        chunk_math<FMT, NI, false>(rb, sl, acur, cc, nbc, kg, p, none);
        wave_sync();
#pragma unroll
        for (int i = 0; i < NI; i++) yacc[i] = yacc[i] + p[i];
        if (cc == C - 1) {
            const int64_t g = tgc / tiles, n0 = (tgc % tiles) * 16;
            const int Bg = (int)(rows - 16 * g < 16 ? rows - 16 * g : 16);
#pragma unroll
            for (int i = 0; i < NI; i++) {
                const int m = 4 * kg + i;
                if (m < Bg && nn < tc.nrows) y[(16 * g + m) * N + n0 + nn] = yacc[i];
                yacc[i] = 0.0f;
            }
            if (tg >= TG) break;
        }
    }
}

// Short matrices: KS waves of one workgroup share a tile and take its chunks
// round-robin; after every round the chunk sums are combined in chunk order
// through LDS.  PARTIALS: write the int32 partials instead (test hook).
template <int FMT, int NI, bool PARTIALS>
__global__ __launch_bounds__(512) void k_qmv_split(const uint8_t* __restrict__ w, int64_t wbytes,
                                                   int64_t N, int64_t K,
                                                   const uint8_t* __restrict__ xq, ActLayout L,
                                                   int64_t rows, int64_t tiles,
                                                   float* __restrict__ y, int32_t* __restrict__ P) {
    using F = Fmt<FMT>;
    constexpr int NP = pieces_per_lane<FMT>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6), KS = blockDim.x >> 6;
    uint8_t* wl = smem + wv * wave_lds<FMT>();
    float* sl = reinterpret_cast<float*>(wl + 16 * span_stride<FMT>());
    float* pbuf = reinterpret_cast<float*>(smem + KS * wave_lds<FMT>());
    const int64_t tile = blockIdx.x % tiles, g = blockIdx.x / tiles;
    const int64_t n0 = tile * 16;
    const int Bg = (int)(rows - 16 * g < 16 ? rows - 16 * g : 16);
    const int nb = (int)(K >> 5), C = (nb + 7) >> 3;
    const int64_t Rl = (K / F::QK) * F::BB;
    const uint32_t R = (uint32_t)Rl;
    const int nn = lane & 15, kg = lane >> 4;
    const TileRef t = make_tile(w, wbytes, N, Rl, tile);
    const ActRef A = make_act(xq, L, g, lane);
    PartialsOut po{};
    if (PARTIALS) {
        po.P = P;
        po.S = reinterpret_cast<const int32_t*>(xq + L.S) + g * nb * 16 + 4 * kg;
        po.N = N; po.row0 = 16 * g; po.n = n0 + nn; po.nb = nb; po.Bg = Bg; po.nrows = (int)N;
    }

    float yacc = 0.0f;
    uint4 reg[NP];
    ActRegs nxt;
    long acur[8];
    if (wv < C) {
        const int nbc0 = F::QK == 32 ? min(8, nb - 8 * wv) : 8;
        fetch_chunk<FMT>(t, R, wv, nbc0, lane, reg);
        fetch_act<FMT>(A, wv, nbc0, lane, nxt);
    }
    for (int r0 = 0; r0 < C; r0 += KS) {
        const int c = r0 + wv;
        float p[NI];
        if (c < C) {
            stage_all<FMT>(wl, sl, lane, reg, nxt, acur);
            const int nbc = F::QK == 32 ? min(8, nb - 8 * c) : 8;
            const int cn = c + KS;
            if (cn < C) {
                const int nbcn = F::QK == 32 ? min(8, nb - 8 * cn) : 8;
                fetch_chunk<FMT>(t, R, cn, nbcn, lane, reg);
                fetch_act<FMT>(A, cn, nbcn, lane, nxt);
            }
            const uint8_t* rb = wl + nn * span_stride<FMT>() + ((nn * R + c * F::CB) & 15);
            chunk_math<FMT, NI, PARTIALS>(rb, sl, acur, c, nbc, kg, p, po);
            wave_sync();
            if (!PARTIALS) {
#pragma unroll
                for (int i = 0; i < NI; i++)
                    if (4 * kg + i < Bg) pbuf[wv * 256 + (4 * kg + i) * 16 + nn] = p[i];
            }
        }
        if (!PARTIALS) {
            __syncthreads();
            const int nact = min(KS, C - r0);
            if (threadIdx.x < 16 * Bg)
                for (int w2 = 0; w2 < nact; w2++) yacc = yacc + pbuf[w2 * 256 + threadIdx.x];
            __syncthreads();
        }
    }
    if (!PARTIALS && threadIdx.x < 16 * Bg) {
        const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
        if (n < t.nrows) y[(16 * g + m) * N + n0 + n] = yacc;
    }
}

// SwiGLU of one output element: silu(g) * u with silu(g) = g / (1 + e^-g),
// evaluated in f64 as t = exp(-g), s = g / (1 + t), h = s * u and rounded
// once to f32 (the llama-family feed-forward gate; llamay "Models and
// formats", architectures table).
__device__ __forceinline__ float swiglu(float g, float u) {
    const double gd = (double)g;
    const double t = exp(-gd);
    const double s = gd / (1.0 + t);
    return (float)(s * (double)u);
}

// ------------------------------------- batched decode on the Q8_K path ----
// 5..16 activation rows against Q4_K / Q6_K weights with Q8_K activations
// (one f32 scale per 256 activations): a workgroup owns a tile of 16 weight
// rows, and its KS waves take the tile's superblocks round-robin.  A wave
// streams the 16 rows' bytes of its superblock as 16-byte pieces into its LDS
// slice (as k_qmv_split does), then lane (nn = l%16, kg = l/16) takes weight
// row nn's codes 8kg..8kg+7 of each 32-element block, one
// v_mfma_i32_16x16x32_i8 per block (Q6_K: two, one per 16-element sub-block,
// the other half's codes zeroed); result element i is activation row 4kg+i.
// The activation operands come from the quantiser's copy in operand order
// (four 16-byte loads per lane and superblock, each wave instruction reading
// 1 KB contiguously; the rows' scales in one more).  The sub-block scales
// multiply the exact int32 block sums, so a superblock reduces to the
// integers of the Q8_K order and is scaled in f32 once, not once per 32
// elements as on the Q8_0 path.  Q4_K's min term Q = sum_j m_j S_j runs as
// two more MFMAs: the rows' eight 32-code sums as two int8 digits (from the
// quantiser) against the eight 6-bit mins, in k-group 0 only.  Every
// superblock's f32 results wait in LDS until a window of BDOT_WINDOW
// superblocks is done; then they are added to y in ascending superblock
// order.  PART: the integer partials are written instead (test hook).
// PAIR: the workgroup takes tile t of two matrices of one shape (the gate
// and up projections), walks the first one's superblocks and then the
// second's, sums each in its own order and writes h = silu(g) * u.
constexpr int BDOT_WINDOW = 32;

struct ActRegsK {
    uint4 a[4];   // blocks 2p, 2p+1: activation row l%16, codes 8kg..8kg+7 of each
    float4 da;    // Q8_K d of activation rows 4kg..4kg+3
    uint4 sd;     // Q4_K, k-group 0: row l%16's digits of S_0..S_7 (lo 0-3, hi 0-3, lo 4-7, hi 4-7)
};

// The activation side of superblock c from the quantiser's operand-order
// copy (gc, gd, gs: its uniform starts; 32-bit offsets on uniform bases keep
// one register per address).
template <int FMT>
__device__ __forceinline__ void fetch_act_k(const uint8_t* __restrict__ gc,
                                            const uint8_t* __restrict__ gd,
                                            const uint8_t* __restrict__ gs, int c, int lane,
                                            ActRegsK& r) {
    const uint32_t co = (uint32_t)c * 4096u + (uint32_t)lane * 16u;
#pragma unroll
    for (int p = 0; p < 4; p++) r.a[p] = *reinterpret_cast<const uint4*>(gc + (co + 1024u * p));
    r.da = *reinterpret_cast<const float4*>(gd + ((uint32_t)c * 64u + 16u * (uint32_t)(lane >> 4)));
    if constexpr (FMT == T_Q4_K)
        r.sd = lane < 16 ? *reinterpret_cast<const uint4*>(gs + ((uint32_t)c * 256u + 16u * (uint32_t)lane))
                         : make_uint4(0, 0, 0, 0);
}

// The integer partials of one superblock (rb: weight row nn's bytes of it in
// LDS) for activation rows 4kg+i: Q4_K Pi = sum_j sc_j sum q a and
// Qi = sum_j m_j S_j; Q6_K Pi = sum_j s_j sum (q - 32) a.  dw, dmw: the
// superblock's fp16 d and dmin, widened.
template <int FMT>
__device__ __forceinline__ void superblock_k(const uint8_t* rb, const ActRegsK& A, int kg,
                                             int (&Pi)[4], int (&Qi)[4], float& dw, float& dmw) {
    const v4i zero = {0, 0, 0, 0};
    auto act = [&](int j) -> long {
        const uint4 v = A.a[j >> 1];
        return (j & 1) ? (long)(((uint64_t)v.w << 32) | v.z) : (long)(((uint64_t)v.y << 32) | v.x);
    };
#pragma unroll
    for (int i = 0; i < 4; i++) Pi[i] = Qi[i] = 0;
    if constexpr (FMT == T_Q4_K) {
        const uint4 hdr = ld<uint4>(rb);
        uint64_t q[4];
#pragma unroll
        for (int j = 0; j < 4; j++) q[j] = ld<uint64_t>(rb + 16 + 32 * j + 8 * kg);
        dw = half_bits_to_float((uint16_t)(hdr.x & 0xFFFF));
        dmw = half_bits_to_float((uint16_t)(hdr.x >> 16));
        const uint32_t s12[3] = {hdr.y, hdr.z, hdr.w};
        const uint8_t* sb = reinterpret_cast<const uint8_t*>(s12);
        uint64_t mins = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            int sc, mn;
            if (j < 4) {
                sc = sb[j] & 63;
                mn = sb[j + 4] & 63;
            } else {
                sc = (sb[j + 4] & 15) | ((sb[j - 4] >> 6) << 4);
                mn = (sb[j + 4] >> 4) | ((sb[j] >> 6) << 4);
            }
            mins |= (uint64_t)mn << (8 * j);
            uint64_t raw = q[j >> 1];
            if (j & 1) raw >>= 4;
            const v4i acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                act(j), (long)(raw & 0x0F0F0F0F0F0F0F0Full), zero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; i++) Pi[i] = __mul24(sc, acc[i]) + Pi[i];
        }
        // min term: k-group 0 carries the S_j digits against m_j, j = 0..7
        const long bm = kg == 0 ? (long)mins : 0;
        const long slo = (long)(((uint64_t)A.sd.z << 32) | A.sd.x);
        const long shi = (long)(((uint64_t)A.sd.w << 32) | A.sd.y);
        const v4i ql = __builtin_amdgcn_mfma_i32_16x16x32_i8(slo, bm, zero, 0, 0, 0);
        const v4i qh = __builtin_amdgcn_mfma_i32_16x16x32_i8(shi, bm, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) Qi[i] = ql[i] + 64 * qh[i];
    } else {
        uint64_t q[4], qh[2];
#pragma unroll
        for (int j = 0; j < 4; j++) q[j] = ld<uint64_t>(rb + 32 * j + 8 * kg);
        qh[0] = ld<uint64_t>(rb + 128 + 8 * kg);
        qh[1] = ld<uint64_t>(rb + 160 + 8 * kg);
        const uint4 scv = ld<uint4>(rb + 192);
        dw = half_bits_to_float(ld<uint16_t>(rb + 208));
        dmw = 0.0f;
        const uint32_t sc6[4] = {scv.x, scv.y, scv.z, scv.w};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int h = j >> 2, kq = j & 3;
            uint64_t ql = q[2 * h + (kq & 1)];
            if (kq & 2) ql >>= 4;
            const uint64_t q6 = (ql & 0x0F0F0F0F0F0F0F0Full) |
                                (((qh[h] >> (2 * kq)) & 0x0303030303030303ull) << 4);
            const uint64_t wc = bytes_minus(q6, 0x2020202020202020ull);
            const uint32_t sw = sc6[j >> 1] >> (16 * (j & 1));
            const int s0 = (int8_t)(sw & 0xFF), s1 = (int8_t)((sw >> 8) & 0xFF);
            const long lo = kg < 2 ? (long)wc : 0, hi = kg < 2 ? 0 : (long)wc;
            const v4i acc0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act(j), lo, zero, 0, 0, 0);
            const v4i acc1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act(j), hi, zero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; i++) Pi[i] = __mul24(s0, acc0[i]) + __mul24(s1, acc1[i]) + Pi[i];
        }
    }
}

// (Q4_K: at most 128 VGPRs, i.e. 4 waves per SIMD; with one register more,
// 3 waves, the 14336 x 4096 GEMV at 16 rows took 16.5 us against 13.0)
// The work of one workgroup on weight tile `tile` (the kernels below).
template <int FMT, bool PART, bool PAIR>
__device__ __forceinline__ void bdot_tile(const uint8_t* __restrict__ w,
                                          const uint8_t* __restrict__ w2, int64_t wbytes,
                                          int64_t N, int64_t K, const uint8_t* __restrict__ xq,
                                          const ActLayoutK& L, int64_t rows,
                                          float* __restrict__ y, int32_t* __restrict__ P,
                                          int64_t tile) {
    using F = Fmt<FMT>;
    constexpr int NP = pieces_per_lane<FMT>();
    constexpr int SL = 16 * span_stride<FMT>();  // a wave's weight slice
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6), KS = blockDim.x >> 6;
    uint8_t* wl = smem + wv * SL;
    float* pbuf = reinterpret_cast<float*>(smem + KS * SL);  // [window][256]
    const int64_t n0 = tile * 16;
    const int Bg = (int)(rows < 16 ? rows : 16);
    const int C = (int)(K >> 8);
    const int64_t Rl = (int64_t)C * F::BB;
    const uint32_t R = (uint32_t)Rl;
    const int nn = lane & 15, kg = lane >> 4;
    const TileRef t = make_tile(w, wbytes, N, Rl, tile);
    const TileRef t2 = PAIR ? make_tile(w2, wbytes, N, Rl, tile) : t;
    const int CT = PAIR ? 2 * C : C;  // superblocks walked: the first matrix's, then the second's
    const uint8_t* gc = xq + L.gcodes;
    const uint8_t* gd = xq + L.gda;
    const uint8_t* gs = xq + L.gsd;
    auto fetch = [&](int cc, uint4 (&rg)[NP], ActRegsK& a) {
        const bool second = PAIR && cc >= C;
        const int c1 = second ? cc - C : cc;
        fetch_chunk<FMT>(second ? t2 : t, R, c1, 8, lane, rg);
        fetch_act_k<FMT>(gc, gd, gs, c1, lane, a);
    };

    uint4 reg[NP];
    ActRegsK nxt;
    if (wv < CT) fetch(wv, reg, nxt);
    float yacc = 0.0f, yacc2 = 0.0f;
    // the wave's superblocks are c = wv (mod KS), in ascending order across
    // the windows: the one in flight at a window's end is its first of the next
    int c = wv;
    for (int w0 = 0; w0 < CT; w0 += BDOT_WINDOW) {
        const int w1 = CT - w0 < BDOT_WINDOW ? CT : w0 + BDOT_WINDOW;
        for (; c < w1; c += KS) {
            stage_chunk<FMT>(wl, lane, reg);
            const ActRegsK cur = nxt;
            wave_sync();
            const int cn = c + KS;
            if (cn < CT) fetch(cn, reg, nxt);
            const int c1 = PAIR && c >= C ? c - C : c;  // superblock within its matrix
            const uint8_t* rb = wl + nn * span_stride<FMT>() + ((nn * R + c1 * F::CB) & 15);
            int Pi[4], Qi[4];
            float dw, dmw;
            superblock_k<FMT>(rb, cur, kg, Pi, Qi, dw, dmw);
            wave_sync();  // the slice is read: the next superblock may overwrite it
            const int64_t n = n0 + nn;
            if constexpr (PART) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = 4 * kg + i;
                    if (m < Bg && n < N) {
                        const int64_t o = ((int64_t)m * N + n) * C + c1;
                        if constexpr (FMT == T_Q4_K) {
                            P[2 * o] = Pi[i];
                            P[2 * o + 1] = Qi[i];
                        } else {
                            P[o] = Pi[i];
                        }
                    }
                }
            } else {
                const float da[4] = {cur.da.x, cur.da.y, cur.da.z, cur.da.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = 4 * kg + i;
                    float p = fmaf((float)Pi[i], dw * da[i], 0.0f);
                    if constexpr (FMT == T_Q4_K) p = fmaf(-(float)Qi[i], dmw * da[i], p);
                    if (m < Bg) pbuf[(c - w0) * 256 + m * 16 + nn] = p;
                }
            }
        }
        if constexpr (!PART) {
            __syncthreads();
            if (threadIdx.x < 16 * Bg) {
                for (int cc = 0; cc < w1 - w0; cc++) {
                    const float v = pbuf[cc * 256 + threadIdx.x];
                    if (!PAIR || w0 + cc < C)
                        yacc = yacc + v;
                    else
                        yacc2 = yacc2 + v;
                }
            }
            __syncthreads();
        }
    }
    if (!PART && threadIdx.x < 16 * Bg) {
        const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
        if (n < t.nrows) y[(int64_t)m * N + n0 + n] = PAIR ? swiglu(yacc, yacc2) : yacc;
    }
}

template <int FMT, bool PART, bool PAIR = false>
__global__ __launch_bounds__(512, FMT == T_Q4_K ? 4 : 1) void k_bdot8k(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ w2, int64_t wbytes, int64_t N,
    int64_t K, const uint8_t* __restrict__ xq, ActLayoutK L, int64_t rows, float* __restrict__ y,
    int32_t* __restrict__ P) {
    bdot_tile<FMT, PART, PAIR>(w, w2, wbytes, N, K, xq, L, rows, y, P, blockIdx.x);
}

// Several GEMVs of one K in one launch: job blockIdx.y, its tile blockIdx.x
// (workgroups past a job's tiles exit at once).
struct BdotJob {
    const uint8_t* w;
    const uint8_t* xq;
    float* y;
    int64_t N;
};
// A grouped launch's grid is flat: entry k owns workgroups
// [start[k], start[k+1]), one per 16-row tile, so no workgroup is surplus.
struct BdotJobs {
    BdotJob j[8];
    int start[9];
    int count;
};

template <int FMT>
__global__ __launch_bounds__(512, FMT == T_Q4_K ? 4 : 1) void k_bdot8k_group(
    BdotJobs jobs, int64_t K, ActLayoutK L, int64_t rows) {
    int k = 0;
    while (k + 1 < jobs.count && (int)blockIdx.x >= jobs.start[k + 1]) k++;
    const BdotJob& J = jobs.j[k];
    const int64_t tile = (int64_t)blockIdx.x - jobs.start[k];
    const int64_t wbytes = J.N * (K / 256) * Fmt<FMT>::BB;
    bdot_tile<FMT, false, false>(J.w, J.w, wbytes, J.N, K, J.xq, L, rows, J.y, nullptr, tile);
}

// ------------------------------------------------- lane-per-chunk GEMV ----
// For a few activation rows (B <= 4) the MFMA tile would be mostly empty and
// the per-lane decode overhead of 8 codes per block dominates.  Here every
// lane owns one 256-element chunk of one weight row: it streams the chunk's
// bytes straight into registers (16-byte loads at the chunk's own, possibly
// 2-byte, alignment), decodes all of them in-lane, and takes the block dots
// with v_dot4_i32_i8 against the row-major staging copy of the activations.
// Field offsets inside a chunk are compile-time constants, so unaligned fields
// cost one v_alignbyte each.  The integer partials are exact and the f32
// sequence per block is the documented one, so results are bit-identical to
// the MFMA kernels.

template <int N, class Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// dword at compile-time byte offset O of a register array holding bytes in order
template <int O, int NW>
__device__ __forceinline__ uint32_t dw_at(const uint32_t (&r)[NW]) {
    static_assert(O >= 0 && O + 4 <= 4 * NW, "field outside the chunk registers");
    if constexpr (O % 4 == 0)
        return r[O / 4];
    else
        return __builtin_amdgcn_alignbyte(r[O / 4 + 1], r[O / 4], O % 4);
}
template <int O, int NW>
__device__ __forceinline__ uint32_t half_at(const uint32_t (&r)[NW]) {
    return (r[O / 4] >> (8 * (O % 4))) & 0xFFFFu;
}
template <int O, int NW>
__device__ __forceinline__ int sbyte_at(const uint32_t (&r)[NW]) {
    return __builtin_amdgcn_sbfe((int)r[O / 4], 8 * (O % 4), 8);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Dwords of one chunk as loaded from the 4-byte-aligned address at or below
// the chunk start (chunks start 2-byte aligned; 16-byte loads at 2-byte
// alignment lose a quarter of the bandwidth, at 4-byte alignment nothing);
// realign_chunk then shifts them down by 0 or 2 bytes.
template <int FMT> struct DotFmt;
// NWD = ceil(CB/4) dwords after the shift, plus the one the shift reads from
// (formats whose chunks are always 4-byte aligned need no shift).
template <> struct DotFmt<T_Q8_0> { static constexpr int NWD = 69; };  // 272 B: 68 + 1
template <> struct DotFmt<T_Q4_0> { static constexpr int NWD = 37; };  // 144 B: 36 + 1
template <> struct DotFmt<T_Q5_0> { static constexpr int NWD = 45; };  // 176 B: 44 + 1
template <> struct DotFmt<T_Q4_1> { static constexpr int NWD = 40; };  // 160 B, aligned
template <> struct DotFmt<T_Q5_1> { static constexpr int NWD = 48; };  // 192 B, aligned
template <> struct DotFmt<T_Q8_1> { static constexpr int NWD = 72; };  // 288 B, aligned
template <> struct DotFmt<T_Q4_K> { static constexpr int NWD = 36; };  // 144 B, aligned
template <> struct DotFmt<T_Q6_K> { static constexpr int NWD = 54; };  // 210 B: 53 + 1
template <int FMT> constexpr bool chunk_aligned4() { return Fmt<FMT>::BB % 4 == 0; }

template <int FMT>
__device__ __forceinline__ void load_chunk_regs(const uint8_t* w, int64_t off, int64_t wbytes,
                                                bool guarded, uint32_t (&r)[DotFmt<FMT>::NWD]) {
    constexpr int NWD = DotFmt<FMT>::NWD;
    const int64_t off4 = off & ~int64_t(3);
    const uint32_t* p = reinterpret_cast<const uint32_t*>(w + off4);
    if (!guarded) {
        __builtin_memcpy(r, p, 4 * NWD);
    } else {
        // blob end inside the loaded range: dwords, then the final half dword
#pragma unroll
        for (int j = 0; j < NWD; j++) {
            const int64_t g = off4 + 4 * j;
            r[j] = g + 4 <= wbytes ? p[j]
                 : g + 2 <= wbytes ? (uint32_t)*reinterpret_cast<const uint16_t*>(w + g) : 0u;
        }
    }
}

// Shift the loaded dwords down by the chunk's offset inside its first dword
// (0 or 2 bytes), so that r[] holds the chunk from byte 0.  Separate from the
// loads so that the wait for them falls just before the chunk is used.
template <int FMT>
__device__ __forceinline__ void realign_chunk(int64_t off, uint32_t (&r)[DotFmt<FMT>::NWD]) {
    constexpr int NWD = DotFmt<FMT>::NWD;
    if constexpr (!chunk_aligned4<FMT>()) {
        const uint32_t sh = (uint32_t)(off & 3);  // 0 or 2
        // skipped when every chunk of the wave is 4-byte aligned (e.g. all
        // rows of a whole number of 8-byte spans)
        if (__builtin_amdgcn_ballot_w64(sh != 0) != 0) {
#pragma unroll
            for (int j = 0; j < NWD - 1; j++) r[j] = __builtin_amdgcn_alignbyte(r[j + 1], r[j], sh);
        }
    }
}

// Activation rows staged in LDS by the workgroup: codes of chunk c of row m
// at codes + c*272 (256 bytes + 16 of padding, so lanes on different chunks
// hit different banks); per-block scale words da, ca and s16 (two int16
// half-block sums) at [b].
struct ActRow {
    const uint8_t* codes;
    const float* da;
    const float* ca;
    const int32_t* s16;
};
constexpr int ACT_CHUNK_STRIDE = 272;

__device__ __forceinline__ void act_block(const ActRow& A, int b, uint32_t (&a)[8]) {
    const uint4* q = reinterpret_cast<const uint4*>(A.codes + (b >> 3) * ACT_CHUNK_STRIDE +
                                                    (b & 7) * 32);
    const uint4 lo = q[0], hi = q[1];
    a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
    a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
}

// LDS bytes of B staged activation rows of K elements.
__host__ __device__ inline int act_lds_row_bytes(int64_t K) {
    const int64_t nb = K / 32, C = (nb + 7) / 8;
    return (int)((C * ACT_CHUNK_STRIDE + 3 * nb * 4 + 15) & ~int64_t(15));
}

// p[m] = sum over the chunk's blocks in order (documented f32 order).
// Where a partials launch writes the exact integers of the lane's row:
// P[m][row][b] (two per block, [..][b][2], for the formats with a minimum term).
struct PartOut {
    int32_t* row;     // P + row * nb * per
    int64_t mstride;  // N * nb * per: from activation row m to m + 1
};

// PART: instead of scaling and accumulating, store each block's exact
// integer partial(s) (the ones the documented f32 order scales) to po.
template <int FMT, int B, bool PART = false>
__device__ __forceinline__ void dot_chunk(const uint32_t (&r)[DotFmt<FMT>::NWD],
                                          const ActRow (&A)[B], int c, int nbc, float (&p)[B],
                                          PartOut po = PartOut{}) {
    constexpr int per = has_min_term<FMT>() ? 2 : 1;
    // the integer(s) of block b, activation row m (only when PART)
    auto emit = [&](int m, int b, bool on, int I, int Q) {
        if constexpr (PART) {
            if (on) {
                int32_t* o = po.row + m * po.mstride + (int64_t)b * per;
                o[0] = I;
                if constexpr (per == 2) o[1] = Q;
            }
        }
    };
#pragma unroll
    for (int m = 0; m < B; m++) p[m] = 0.0f;
    // 32-element formats: the blocks of a short last chunk (bb >= nbc) are
    // computed too and their terms dropped by a select, so that the block
    // loop has no branch (nbc differs between lanes) and the LDS reads of
    // later blocks can be issued ahead.  Their activation bytes lie in the
    // chunk's padding and the following row fields, inside the staged copy.
    if constexpr (FMT == T_Q8_0) {
        static_for<8>([&](auto BB) {
            constexpr int bb = BB;
            const bool on = bb < nbc;
            const int b = 8 * c + bb;
            const float dw = half_bits_to_float(half_at<34 * bb>(r));
            uint32_t w[8];
            static_for<8>([&](auto I) { w[I] = dw_at<34 * bb + 2 + 4 * I>(r); });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 8; i++) D = dot4(w[i], a[i], D);
                emit(m, b, on, D, 0);
                const float t = fmaf((float)D, dw * A[m].da[b], p[m]);
                p[m] = on ? t : p[m];
            }
        });
    } else if constexpr (FMT == T_Q4_0) {
        static_for<8>([&](auto BB) {
            constexpr int bb = BB;
            const bool on = bb < nbc;
            const int b = 8 * c + bb;
            const float dw = half_bits_to_float(half_at<18 * bb>(r));
            uint32_t lo[4], hi[4];
            static_for<4>([&](auto I) {
                const uint32_t q = dw_at<18 * bb + 2 + 4 * I>(r);
                lo[I] = q & 0x0F0F0F0Fu;
                hi[I] = (q >> 4) & 0x0F0F0F0Fu;
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) D = dot4(lo[i], a[i], D);
#pragma unroll
                for (int i = 0; i < 4; i++) D = dot4(hi[i], a[4 + i], D);
                const int s16 = A[m].s16[b];
                const int S = (int)(int16_t)(s16 & 0xFFFF) + (s16 >> 16);
                emit(m, b, on, D - 8 * S, 0);
                const float t = fmaf((float)(D - 8 * S), dw * A[m].da[b], p[m]);
                p[m] = on ? t : p[m];
            }
        });
    } else if constexpr (FMT == T_Q8_1) {
        static_for<8>([&](auto BB) {
            constexpr int bb = BB;
            const bool on = bb < nbc;
            const int b = 8 * c + bb;
            const float dw = half_bits_to_float(half_at<36 * bb>(r));
            uint32_t w[8];
            static_for<8>([&](auto I) { w[I] = dw_at<36 * bb + 4 + 4 * I>(r); });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 8; i++) D = dot4(w[i], a[i], D);
                emit(m, b, on, D, 0);
                const float t = fmaf((float)D, dw * A[m].da[b], p[m]);
                p[m] = on ? t : p[m];
            }
        });
    } else if constexpr (FMT == T_Q4_1 || FMT == T_Q5_1) {
        // d, m, [fifth bits,] nibbles; term P (d d_a) then + m (d_a S)
        constexpr int BBY = Fmt<FMT>::BB, QS = FMT == T_Q4_1 ? 4 : 8;
        static_for<8>([&](auto BB) {
            constexpr int bb = BB;
            const bool on = bb < nbc;
            const int b = 8 * c + bb;
            const float dw = half_bits_to_float(half_at<BBY * bb>(r));
            const float mw = half_bits_to_float(half_at<BBY * bb + 2>(r));
            uint32_t h = 0;
            if constexpr (FMT == T_Q5_1) h = dw_at<BBY * bb + 4>(r);
            uint32_t lo[4], hi[4];
            static_for<4>([&](auto I) {
                const uint32_t q = dw_at<BBY * bb + QS + 4 * I>(r);
                lo[I] = q & 0x0F0F0F0Fu;
                hi[I] = (q >> 4) & 0x0F0F0F0Fu;
                if constexpr (FMT == T_Q5_1) {
                    lo[I] |= spread4((h >> (4 * I)) & 15u);
                    hi[I] |= spread4((h >> (16 + 4 * I)) & 15u);
                }
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) D = dot4(lo[i], a[i], D);
#pragma unroll
                for (int i = 0; i < 4; i++) D = dot4(hi[i], a[4 + i], D);
                if constexpr (PART) {
                    const int s16 = A[m].s16[b];
                    emit(m, b, on, D, (int)(int16_t)(s16 & 0xFFFF) + (s16 >> 16));
                }
                float t = fmaf((float)D, dw * A[m].da[b], p[m]);
                t = fmaf(mw, A[m].ca[b], t);
                p[m] = on ? t : p[m];
            }
        });
    } else if constexpr (FMT == T_Q5_0) {
        static_for<8>([&](auto BB) {
            constexpr int bb = BB;
            const bool on = bb < nbc;
            const int b = 8 * c + bb;
            const float dw = half_bits_to_float(half_at<22 * bb>(r));
            const uint32_t h = dw_at<22 * bb + 2>(r);
            uint32_t lo[4], hi[4];
            static_for<4>([&](auto I) {
                const uint32_t q = dw_at<22 * bb + 6 + 4 * I>(r);
                lo[I] = (q & 0x0F0F0F0Fu) | spread4((h >> (4 * I)) & 15u);
                hi[I] = ((q >> 4) & 0x0F0F0F0Fu) | spread4((h >> (16 + 4 * I)) & 15u);
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) D = dot4(lo[i], a[i], D);
#pragma unroll
                for (int i = 0; i < 4; i++) D = dot4(hi[i], a[4 + i], D);
                const int s16 = A[m].s16[b];
                const int S = (int)(int16_t)(s16 & 0xFFFF) + (s16 >> 16);
                emit(m, b, on, D - 16 * S, 0);
                const float t = fmaf((float)(D - 16 * S), dw * A[m].da[b], p[m]);
                p[m] = on ? t : p[m];
            }
        });
    } else if constexpr (FMT == T_Q4_K) {
        const float d = half_bits_to_float(half_at<0>(r));
        const float dmin = half_bits_to_float(half_at<2>(r));
        static_for<8>([&](auto BB) {
            constexpr int j = BB;
            const int b = 8 * c + j;
            // 6-bit scale and min of sub-block j (bytes 4..15 of the superblock)
            int sc, mn;
            if constexpr (j < 4) {
                sc = (int)((dw_at<4 + (j & ~3)>(r) >> (8 * (j & 3))) & 63);
                mn = (int)((dw_at<8>(r) >> (8 * j)) & 63);
            } else {
                const uint32_t s_hi = dw_at<12>(r) >> (8 * (j - 4));   // byte j+4
                const uint32_t s_lo = dw_at<4>(r) >> (8 * (j - 4));    // byte j-4
                const uint32_t s_mid = dw_at<8>(r) >> (8 * (j - 4));   // byte j
                sc = (int)((s_hi & 15) | (((s_lo >> 6) & 3) << 4));
                mn = (int)(((s_hi >> 4) & 15) | (((s_mid >> 6) & 3) << 4));
            }
            const float cw = dmin * (float)mn;
            uint32_t q[8];
            static_for<8>([&](auto I) {
                q[I] = (dw_at<16 + 32 * (j >> 1) + 4 * I>(r) >> (4 * (j & 1))) & 0x0F0F0F0Fu;
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 8; i++) D = dot4(q[i], a[i], D);
                if constexpr (PART) {
                    const int s16 = A[m].s16[b];
                    emit(m, b, true, sc * D, mn * ((int)(int16_t)(s16 & 0xFFFF) + (s16 >> 16)));
                }
                p[m] = fmaf((float)(sc * D), d * A[m].da[b], p[m]);
                p[m] = fmaf(-cw, A[m].ca[b], p[m]);
            }
        });
    } else {  // Q6_K
        const float d = half_bits_to_float(half_at<208>(r));
        static_for<8>([&](auto BB) {
            constexpr int bb = BB, h = bb >> 2, kq = bb & 3;
            const int b = 8 * c + bb;
            const int s0 = sbyte_at<192 + 2 * bb>(r), s1 = sbyte_at<193 + 2 * bb>(r);
            uint32_t q[8];
            static_for<8>([&](auto I) {
                const uint32_t ql = dw_at<64 * h + 32 * (kq & 1) + 4 * I>(r);
                const uint32_t qh = dw_at<128 + 32 * h + 4 * I>(r);
                q[I] = ((ql >> (4 * (kq >> 1))) & 0x0F0F0F0Fu) |
                       (((qh >> (2 * kq)) & 0x03030303u) << 4);
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D0 = 0, D1 = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) D0 = dot4(q[i], a[i], D0);
#pragma unroll
                for (int i = 4; i < 8; i++) D1 = dot4(q[i], a[i], D1);
                const int s16 = A[m].s16[b];
                const int S0 = (int)(int16_t)(s16 & 0xFFFF), S1 = s16 >> 16;
                const int I = s0 * (D0 - 32 * S0) + s1 * (D1 - 32 * S1);
                emit(m, b, true, I, 0);
                p[m] = fmaf((float)I, d * A[m].da[b], p[m]);
            }
        });
    }
}

// The same chunk (one K-quant superblock c) against Q8_K activations: the
// integer sub-block scales fold into one superblock partial (Q4_K: P and Q,
// Q6_K: I), scaled once: p = fma((float)P, fl(d d_a), +0) [then
// fma(-(float)Q, fl(dmin d_a), p)], d_a the activation superblock's f32
// scale (staged per 32 codes; [8c] is the superblock's).  PART: store the
// superblock partials instead, at po.row[m * po.mstride + c * per].
template <int FMT, int B, bool PART = false>
__device__ __forceinline__ void dot_chunk_q8k(const uint32_t (&r)[DotFmt<FMT>::NWD],
                                              const ActRow (&A)[B], int c, float (&p)[B],
                                              PartOut po = PartOut{}) {
    if constexpr (FMT == T_Q4_K) {
        const float d = half_bits_to_float(half_at<0>(r));
        const float dmin = half_bits_to_float(half_at<2>(r));
        int Pv[B], Qv[B];
#pragma unroll
        for (int m = 0; m < B; m++) Pv[m] = Qv[m] = 0;
        static_for<8>([&](auto BB) {
            constexpr int j = BB;
            const int b = 8 * c + j;
            int sc, mn;
            if constexpr (j < 4) {
                sc = (int)((dw_at<4 + (j & ~3)>(r) >> (8 * (j & 3))) & 63);
                mn = (int)((dw_at<8>(r) >> (8 * j)) & 63);
            } else {
                const uint32_t s_hi = dw_at<12>(r) >> (8 * (j - 4));
                const uint32_t s_lo = dw_at<4>(r) >> (8 * (j - 4));
                const uint32_t s_mid = dw_at<8>(r) >> (8 * (j - 4));
                sc = (int)((s_hi & 15) | (((s_lo >> 6) & 3) << 4));
                mn = (int)(((s_hi >> 4) & 15) | (((s_mid >> 6) & 3) << 4));
            }
            uint32_t q[8];
            static_for<8>([&](auto I) {
                q[I] = (dw_at<16 + 32 * (j >> 1) + 4 * I>(r) >> (4 * (j & 1))) & 0x0F0F0F0Fu;
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D = 0;
#pragma unroll
                for (int i = 0; i < 8; i++) D = dot4(q[i], a[i], D);
                const int s16 = A[m].s16[b];
                Pv[m] += sc * D;
                Qv[m] += mn * ((int)(int16_t)(s16 & 0xFFFF) + (s16 >> 16));
            }
        });
#pragma unroll
        for (int m = 0; m < B; m++) {
            if constexpr (PART) {
                int32_t* o = po.row + m * po.mstride + (int64_t)c * 2;
                o[0] = Pv[m];
                o[1] = Qv[m];
            }
            const float da = A[m].da[8 * c];
            const float t = fmaf((float)Pv[m], d * da, 0.0f);
            p[m] = fmaf(-(float)Qv[m], dmin * da, t);
        }
    } else {  // Q6_K
        const float d = half_bits_to_float(half_at<208>(r));
        int Iv[B];
#pragma unroll
        for (int m = 0; m < B; m++) Iv[m] = 0;
        static_for<8>([&](auto BB) {
            constexpr int bb = BB, h = bb >> 2, kq = bb & 3;
            const int b = 8 * c + bb;
            const int s0 = sbyte_at<192 + 2 * bb>(r), s1 = sbyte_at<193 + 2 * bb>(r);
            uint32_t q[8];
            static_for<8>([&](auto I) {
                const uint32_t ql = dw_at<64 * h + 32 * (kq & 1) + 4 * I>(r);
                const uint32_t qh = dw_at<128 + 32 * h + 4 * I>(r);
                q[I] = ((ql >> (4 * (kq >> 1))) & 0x0F0F0F0Fu) |
                       (((qh >> (2 * kq)) & 0x03030303u) << 4);
            });
#pragma unroll
            for (int m = 0; m < B; m++) {
                uint32_t a[8];
                act_block(A[m], b, a);
                int D0 = 0, D1 = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) D0 = dot4(q[i], a[i], D0);
#pragma unroll
                for (int i = 4; i < 8; i++) D1 = dot4(q[i], a[i], D1);
                const int s16 = A[m].s16[b];
                const int S0 = (int)(int16_t)(s16 & 0xFFFF), S1 = s16 >> 16;
                Iv[m] += s0 * (D0 - 32 * S0) + s1 * (D1 - 32 * S1);
            }
        });
#pragma unroll
        for (int m = 0; m < B; m++) {
            if constexpr (PART) po.row[m * po.mstride + c] = Iv[m];
            p[m] = fmaf((float)Iv[m], d * A[m].da[8 * c], 0.0f);
        }
    }
}

// One GEMV of a launch (a launch may carry several, of one format and one
// row count B): weights, shape, output, and the activations: x to quantise
// in the kernel (FUSED), or the staged quantisation in xq.
struct DotJob {
    const uint8_t* w;
    const uint8_t* w2;  // paired launch (gate/up + SwiGLU): the up blob; w is the gate blob
    float* y;
    const float* x;   // FUSED: f32 activations [B][K]
    uint8_t* xq;      // staged quantisation; FUSED: written by the job's first workgroup (may be NULL)
    int64_t N, K, wbytes;
    int64_t rcodes, rda, rca, rs16;  // offsets of the row-major staging in xq
    // paired launch with the quantisation of h (MODE_PAIRED_Q): the Q8_0
    // blocks and row staging of h go to hq (layout act_layout(B, N))
    uint8_t* hq;
    int64_t hnb, hrcodes, hrda, hrca, hrs16;
};
constexpr int MAX_JOBS = 8;
// A grouped launch's grid is flat: job k owns workgroups [start[k],
// start[k+1]), so no workgroup is surplus (a 2-D grid with a row per job,
// each as wide as the largest, measured 8.8 against 7.5 us for an 8B-class
// q/k/v group: the exiting workgroups of the smaller jobs still take their
// turn at dispatch).  A workgroup finds its job with a few scalar compares
// and loads the job's fields with one dependent kernel-argument load.
struct DotJobs {
    int count;
    int waves;            // waves per workgroup (4 or 8), as launched
    DotJob j[MAX_JOBS];
    int start[MAX_JOBS + 1];
};

// floor(a / b) for 0 <= a < 4096 and 1 <= b <= 64, through the f32
// reciprocal: (a + 1/2) / b lies at least 1/(2b) >= 1/128 from an integer,
// and the rounding of a + 1/2 (exact), rcp(b) (1 ulp) and the product keeps
// the result within 4096 * 2^-21 = 1/512 of it.
__device__ __forceinline__ int small_div(int a, int b) {
    return (int)(((float)a + 0.5f) * __builtin_amdgcn_rcpf((float)b));
}

// Work units: C <= 64 chunks per row: a unit is G = floor(64/C) rows, C
// lanes per row (LPR = C), one chunk per lane; C > 64: a unit is one row,
// in passes of 64 chunks.  (Waves start at a limited rate per XCD, about
// one per 25 ns measured, so packing rows tightly into the 64 lanes, rather
// than into power-of-two lane groups, shortens the launch.)  Every wave takes one unit; a workgroup is 4
// (or 8) waves sharing the activation rows staged in LDS.  Each lane streams its
// chunk straight into registers, issued before the activations are staged.
// Chunk sums are added in chunk order per row through a small LDS buffer,
// and each row's result is stored once, at the end.

// Launch modes of the dot kernel: a group of GEMVs (job = blockIdx.y), one
// GEMV, or one gate/up pair whose rows are computed side by side and leave
// h = silu(gate) * up instead of two outputs.
// MODE_PARTIALS: one GEMV on staged activations whose y is an int32 buffer
// receiving the exact block partials instead (the test hook).
// MODE_PAIRED_Q: MODE_PAIRED whose workgroups (of 32/GP waves, up to 8)
// each own one 32-element block of h per activation row and also write its
// Q8_0 quantisation (public block and row staging) for the down projection
constexpr int MODE_GROUP = 0, MODE_SINGLE = 1, MODE_PAIRED = 2, MODE_PARTIALS = 3,
              MODE_PAIRED_Q = 4;

// Q8K: the activations are staged Q8_K (K-quant formats only, not FUSED):
// each chunk is scaled once per superblock (dot_chunk_q8k).
// Loads whose count the compiler can see (LEAN): with every chunk of the
// launch whole (K a multiple of 256), each lane loads a full window from
// inside the blob with no branch around the loads, so that the waits for the
// activation loads issued before them count past the weight loads instead of
// draining every load (a path that skips its loads at a join forces that).
// Q6_K keeps the guarded loads, which measured faster for it.
template <int FMT> constexpr bool lean_loads() { return FMT != T_Q6_K; }

template <int FMT, int B, bool FUSED, int MODE, bool Q8K = false, bool WHOLE = false>
__global__ __launch_bounds__(512) void k_dot(DotJobs jobs) {
    constexpr bool PAIRED = MODE == MODE_PAIRED || MODE == MODE_PAIRED_Q;
    using F = Fmt<FMT>;
    constexpr int NWD = DotFmt<FMT>::NWD;
    constexpr bool LEAN = WHOLE && lean_loads<FMT>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // this workgroup's job (one kernel-argument round trip)
    DotJob J;
    int64_t bx = blockIdx.x;  // the workgroup's index within its job
    if constexpr (MODE != MODE_GROUP) {
        J = jobs.j[0];
    } else {
        int k = 0;
        while (k + 1 < jobs.count && (int)blockIdx.x >= jobs.start[k + 1]) k++;
        J = jobs.j[k];
        bx = (int64_t)blockIdx.x - jobs.start[k];
    }
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int64_t N = J.N, K = J.K;
    const int nb = (int)(K >> 5), C = (nb + 7) >> 3;
    const int rowb = act_lds_row_bytes(K);
    float (*pbuf)[64] = reinterpret_cast<float (*)[64]>(smem + B * rowb + wv * B * 256);

    const int64_t R = (K / F::QK) * F::BB;
    const int LPR = C <= 64 ? C : 64, G = 64 / LPR;  // lanes per row, rows per unit
    const int PR = (C + 63) >> 6;  // passes (1 unless C > 64)
    // output rows per unit: G, or G/2 gate/up pairs (lane rows 0..GP-1 take
    // gate rows, GP..2GP-1 the same up rows; the launcher ensures C <= 32)
    const int GP = PAIRED ? G >> 1 : G;
    const int64_t units = C <= 64 ? (N + GP - 1) / GP : N;
    const int lrow = small_div(lane, LPR), lchunk = lane - lrow * LPR;  // this lane's row in the unit, chunk
    if (bx * jobs.waves >= units) return;  // past the job's units (its last workgroup's idle waves)
    const int64_t u = bx * jobs.waves + wv;
    const bool active = u < units;

    auto chunk_of = [&](int q, int64_t& row, int& c) {
        // lanes past the unit's G rows (64 % C of them) get a row past N: idle
        if constexpr (PAIRED)
            row = lrow < 2 * GP ? u * GP + (lrow < GP ? lrow : lrow - GP) : N;
        else
            row = C <= 64 ? (lrow < G ? u * G + lrow : N) : u;
        c = C <= 64 ? lchunk : 64 * q + lane;
    };
    const uint8_t* wsrc = PAIRED && lrow >= GP ? J.w2 : J.w;
    auto issue = [&](int q, uint32_t (&r)[NWD]) {
        int64_t row;
        int c;
        chunk_of(q, row, c);
        const bool valid = active && row < N && c < C;
        if constexpr (LEAN) {
            // whole chunks: a row is C chunks of CB bytes, a multiple of 4,
            // so every chunk starts 4-byte aligned (the blob is 16-byte
            // aligned) and is exactly its CB / 4 dwords; lanes past the rows
            // read chunk 0 (their sums are dropped)
            static_assert(F::CB % 4 == 0, "lean loads need 4-byte chunks");
            const int64_t off = valid ? row * R + (int64_t)c * F::CB : 0;
            __builtin_memcpy(r, reinterpret_cast<const uint32_t*>(wsrc + off), F::CB);
#pragma unroll
            for (int i = F::CB / 4; i < NWD; i++) r[i] = 0;
        } else {
            const int64_t off = row * R + (int64_t)c * F::CB;
            const bool near_end = valid && off + 4 * NWD > J.wbytes;
            if (valid) {
                load_chunk_regs<FMT>(wsrc, off, J.wbytes, __builtin_amdgcn_ballot_w64(near_end) != 0, r);
            } else {
#pragma unroll
                for (int i = 0; i < NWD; i++) r[i] = 0;
            }
        }
    };

    // first chunk in flight while the activations are staged
    uint32_t r[NWD];
    // non-fused: the first pass of the activation copy is loaded into
    // registers and stored to LDS after the weights are issued.  A long copy
    // (>= 256 pieces) is loaded before the weights, so that it is not queued
    // behind them (loads complete in issue order); a short one after them.
    constexpr int SP = 4, SW = 2;  // 16-byte code pieces / scale words per thread in that pass
    uint4 pc[SP];
    uint32_t pw[SW][3];
    const int npc = B * nb * 2, nwd = B * nb;
    const bool copy_first = npc >= 256;
    if constexpr (!FUSED && LEAN) {
        // LEAN: the copy always goes first; every thread of a pass that has
        // work loads (a clamped index), so the loads are not behind branches
        const uint8_t* xq = J.xq;
        const int bd = blockDim.x;
#pragma unroll
        for (int uu = 0; uu < SP; uu++) {
            if (uu * bd < npc) {
                const int i = min((int)threadIdx.x + uu * bd, npc - 1);
                const int m = i / (2 * nb), k = i - m * 2 * nb;
                pc[uu] = reinterpret_cast<const uint4*>(xq + J.rcodes + (int64_t)m * K)[k];
            }
        }
#pragma unroll
        for (int uu = 0; uu < SW; uu++) {
            if (uu * bd < nwd) {
                const int i = min((int)threadIdx.x + uu * bd, nwd - 1);
                pw[uu][0] = reinterpret_cast<const uint32_t*>(xq + J.rda)[i];
                pw[uu][1] = reinterpret_cast<const uint32_t*>(xq + J.rca)[i];
                pw[uu][2] = reinterpret_cast<const uint32_t*>(xq + J.rs16)[i];
            }
        }
        issue(0, r);
    } else if constexpr (!FUSED) {
        const uint8_t* xq = J.xq;
        if (!copy_first) issue(0, r);
#pragma unroll
        for (int uu = 0; uu < SP; uu++) {
            const int i = threadIdx.x + uu * blockDim.x;  // piece i: row i / (2nb), piece i % (2nb)
            if (i < npc) {
                const int m = i / (2 * nb), k = i - m * 2 * nb;
                pc[uu] = reinterpret_cast<const uint4*>(xq + J.rcodes + (int64_t)m * K)[k];
            }
        }
#pragma unroll
        for (int uu = 0; uu < SW; uu++) {
            const int i = threadIdx.x + uu * blockDim.x;  // word i: row i / nb, block i % nb
            if (i < nwd) {
                pw[uu][0] = reinterpret_cast<const uint32_t*>(xq + J.rda)[i];
                pw[uu][1] = reinterpret_cast<const uint32_t*>(xq + J.rca)[i];
                pw[uu][2] = reinterpret_cast<const uint32_t*>(xq + J.rs16)[i];
            }
        }
        if (copy_first) issue(0, r);
    }

    // stage the B activation rows: codes (per-chunk padded), da, ca, s16
    ActRow A[B];
#pragma unroll
    for (int m = 0; m < B; m++) {
        uint8_t* base = smem + m * rowb;
        A[m].codes = base;
        A[m].da = reinterpret_cast<const float*>(base + C * ACT_CHUNK_STRIDE);
        A[m].ca = A[m].da + nb;
        A[m].s16 = reinterpret_cast<const int32_t*>(A[m].ca + nb);
    }
    if constexpr (FUSED) {
        // four lanes per block, 8 elements each: the block's amax and code
        // sums by lane shuffles, then the same d, id and codes as k_quantize
        const bool writer = bx == 0 && J.xq != nullptr;
        const float* x = J.x;
        uint8_t* xq = J.xq;
        const int total = 4 * B * nb;  // (block, quarter) tasks; whole blocks stay in one pass
        constexpr int UNR = 2;         // passes whose x loads are issued together
        // a long activation is loaded ahead of the weights (loads complete in
        // issue order), a short one behind them; formats with long chunks
        // (Q8_0, Q6_K) always load the weights first, which keeps the chunk
        // registers free during the quantisation
        // LEAN: x goes first for the short-chunk formats whatever its
        // length, and every thread of a pass that has work loads (a clamped
        // index), so the loads are not behind branches
        const bool x_first = NWD <= 40 && (LEAN || total > 256);
        const int bd = blockDim.x;
        float4 xf[UNR][2];
        auto load_x = [&](int pass) {
#pragma unroll
          for (int uu = 0; uu < UNR; uu++) {
            const int i0 = (pass * UNR + uu) * bd;
            if (LEAN ? i0 < total : i0 + (int)threadIdx.x < total) {
              const int i = min((int)threadIdx.x + i0, total - 1);
              const int blk = i >> 2, part = i & 3;
              const int m = blk / nb, b = blk - m * nb;
              const float4* xb = reinterpret_cast<const float4*>(x + (int64_t)m * K + 32 * b + 8 * part);
              xf[uu][0] = xb[0];
              xf[uu][1] = xb[1];
            }
          }
        };
        if constexpr (LEAN) {
            if constexpr (NWD <= 40) {
                load_x(0);
                issue(0, r);
            } else {
                issue(0, r);
                load_x(0);
            }
        } else {
            if (!x_first) issue(0, r);
            load_x(0);
            if (x_first) issue(0, r);  // every lane takes pass 0
        }
        for (int pass = 0; pass == 0 || pass * UNR * bd < total; pass++) {
          if (pass > 0) load_x(pass);
          const int i0 = threadIdx.x + pass * UNR * blockDim.x;
#pragma unroll
          for (int uu = 0; uu < UNR; uu++) {
            const int i = i0 + uu * blockDim.x;
            if (i >= total) break;
            const int blk = i >> 2, part = i & 3;
            const int m = blk / nb, b = blk - m * nb;
            const float4 f0 = xf[uu][0], f1 = xf[uu][1];
            const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; k++) amax = fmaxf(amax, fabsf(v[k]));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            const float d = amax / 127.0f;
            const float id = inv_scale(d);
            uint32_t c2[2] = {0u, 0u};
            int sp = 0;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const int qv = (int)roundf(v[k] * id);
                sp += qv;
                c2[k >> 2] |= ((uint32_t)qv & 0xFFu) << (8 * (k & 3));
            }
            const uint16_t h = float_to_half_bits(d);
            const float dval = half_bits_to_float(h);
            const int s01 = sp + __shfl_xor(sp, 1);     // parts 0+1 (lanes 0, 1), 2+3 (lanes 2, 3)
            const int s23 = __shfl_xor(s01, 2);
            uint8_t* base = smem + m * rowb;
            *reinterpret_cast<uint2*>(base + (b >> 3) * ACT_CHUNK_STRIDE + (b & 7) * 32 + 8 * part) =
                make_uint2(c2[0], c2[1]);
            float* dda = reinterpret_cast<float*>(base + C * ACT_CHUNK_STRIDE);
            const int S = s01 + s23;
            const int32_t s16 = (int32_t)(((uint32_t)s01 & 0xFFFFu) | ((uint32_t)s23 << 16));
            if (part == 0) {
                dda[b] = dval;
                dda[nb + b] = dval * (float)S;
                reinterpret_cast<int32_t*>(dda + 2 * nb)[b] = s16;
            }
            if (writer) {
                uint8_t* pub = xq + ((int64_t)m * nb + b) * 34;
                __builtin_memcpy(pub + 2 + 8 * part, c2, 8);
                *reinterpret_cast<uint2*>(xq + J.rcodes + (int64_t)m * K + 32 * b + 8 * part) =
                    make_uint2(c2[0], c2[1]);
                if (part == 0) {
                    const uint8_t hb[2] = {(uint8_t)(h & 255), (uint8_t)(h >> 8)};
                    __builtin_memcpy(pub, hb, 2);
                    reinterpret_cast<float*>(xq + J.rda)[m * nb + b] = dval;
                    reinterpret_cast<float*>(xq + J.rca)[m * nb + b] = dval * (float)S;
                    reinterpret_cast<int32_t*>(xq + J.rs16)[m * nb + b] = s16;
                }
            }
          }
        }
    } else {
        const uint8_t* xq = J.xq;
        // piece k of row m goes to chunk k/16, offset (k%16)*16 of the padded row
        auto put_piece = [&](int i, uint4 v) {
            const int m = i / (2 * nb), k = i - m * 2 * nb;
            *reinterpret_cast<uint4*>(smem + m * rowb + (k >> 4) * ACT_CHUNK_STRIDE + (k & 15) * 16) = v;
        };
        auto put_words = [&](int i, uint32_t da, uint32_t ca, uint32_t s16) {
            const int m = i / nb, b = i - m * nb;
            uint32_t* dd = reinterpret_cast<uint32_t*>(smem + m * rowb + C * ACT_CHUNK_STRIDE);
            dd[b] = da;
            dd[nb + b] = ca;
            dd[2 * nb + b] = s16;
        };
#pragma unroll
        for (int uu = 0; uu < SP; uu++) {
            const int i = threadIdx.x + uu * blockDim.x;
            if (i < npc) put_piece(i, pc[uu]);
        }
#pragma unroll
        for (int uu = 0; uu < SW; uu++) {
            const int i = threadIdx.x + uu * blockDim.x;
            if (i < nwd) put_words(i, pw[uu][0], pw[uu][1], pw[uu][2]);
        }
        // the rest (long rows): load and store
        for (int i = threadIdx.x + SP * blockDim.x; i < npc; i += blockDim.x) {
            const int m = i / (2 * nb), k = i - m * 2 * nb;
            put_piece(i, reinterpret_cast<const uint4*>(xq + J.rcodes + (int64_t)m * K)[k]);
        }
        for (int i = threadIdx.x + SW * blockDim.x; i < nwd; i += blockDim.x)
            put_words(i, reinterpret_cast<const uint32_t*>(xq + J.rda)[i],
                      reinterpret_cast<const uint32_t*>(xq + J.rca)[i],
                      reinterpret_cast<const uint32_t*>(xq + J.rs16)[i]);
    }
    __syncthreads();
    if (!active) return;

    float yacc[B];
#pragma unroll
    for (int j = 0; j < B; j++) yacc[j] = 0.0f;
    for (int q = 0; q < PR; q++) {
        int64_t row;
        int c;
        chunk_of(q, row, c);
        const bool valid = row < N && c < C;
        const int nbc = F::QK == 32 ? min(8, nb - 8 * c) : 8;
        float p[B];
        if constexpr (MODE == MODE_PARTIALS) {
            if (valid) {
                constexpr int per = has_min_term<FMT>() ? 2 : 1;
                realign_chunk<FMT>(row * R + (int64_t)c * F::CB, r);
                if constexpr (Q8K) {
                    const PartOut po{reinterpret_cast<int32_t*>(J.y) + row * C * per, N * C * per};
                    dot_chunk_q8k<FMT, B, true>(r, A, c, p, po);
                } else {
                    const PartOut po{reinterpret_cast<int32_t*>(J.y) + row * nb * per,
                                     N * nb * per};
                    dot_chunk<FMT, B, true>(r, A, c, nbc, p, po);
                }
            }
            if (q + 1 < PR) issue(q + 1, r);
            continue;
        }
        if (valid) {
            realign_chunk<FMT>(row * R + (int64_t)c * F::CB, r);
            if constexpr (Q8K)
                dot_chunk_q8k<FMT, B>(r, A, c, p);
            else
                dot_chunk<FMT, B>(r, A, c, nbc, p);
        } else {
#pragma unroll
            for (int m = 0; m < B; m++) p[m] = 0.0f;
        }
        if (q + 1 < PR) issue(q + 1, r);  // registers are free again
#pragma unroll
        for (int m = 0; m < B; m++) pbuf[m][lane] = p[m];
        wave_sync();
        // lane t < G*B (in steps of 64) adds row t%G's chunks for row m = t/G
        const int cnt = C <= 64 ? C : min(64, C - 64 * q);
#pragma unroll
        for (int j = 0; j < B; j++) {
            const int t = lane + 64 * j;
            if (t < G * B) {
                const int m = small_div(t, G), rl = t - m * G;
                for (int k = 0; k < cnt; k++) yacc[j] = yacc[j] + pbuf[m][rl * LPR + k];
            }
        }
        wave_sync();
    }
    if constexpr (MODE == MODE_PARTIALS) return;
    if constexpr (PAIRED) {
        // the gate and up sums of each output row meet in LDS; the gate
        // lane writes h = silu(gate) * up
#pragma unroll
        for (int j = 0; j < B; j++) {
            const int t = lane + 64 * j;
            if (t < G * B) {
                const int m = small_div(t, G), rl = t - m * G;
                pbuf[m][rl] = yacc[j];
            }
        }
        wave_sync();
        // MODE_PAIRED_Q: this workgroup's 32 rows of h (row 32 blockIdx.x + i
        // at hb[m][i]) for the quantisation below
        float* hb = reinterpret_cast<float*>(smem + B * rowb + jobs.waves * B * 256);
#pragma unroll
        for (int j = 0; j < B; j++) {
            const int t = lane + 64 * j;
            if (t < G * B) {
                const int m = small_div(t, G), rl = t - m * G;
                const int64_t orow = u * GP + rl;
                if (rl < GP && orow < N) {
                    const float hv = swiglu(yacc[j], pbuf[m][GP + rl]);
                    J.y[m * N + orow] = hv;
                    if constexpr (MODE == MODE_PAIRED_Q) hb[m * 32 + (int)(orow & 31)] = hv;
                }
            }
        }
        if constexpr (MODE == MODE_PAIRED_Q) {
            // every wave of the workgroup is active (N % 32 == 0, 32/GP waves)
            __syncthreads();
            if (wv == 0) {
                // lanes 8 m .. 8 m + 7 quantise row m's block (block index
                // blockIdx.x of the N/32 blocks of h)
                const int m = lane >> 3, sub = lane & 7;
                const bool live = m < B;
                float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (live) {
#pragma unroll
                    for (int i = 0; i < 4; i++) v[i] = hb[m * 32 + 4 * sub + i];
                }
                const int64_t b = blockIdx.x, hnb = J.hnb, mm = live ? m : 0;
                uint8_t* hq = J.hq;
                quant_block8(v, sub, live, hq + (mm * hnb + b) * 34, hq + J.hrcodes + mm * N + 32 * b,
                             reinterpret_cast<float*>(hq + J.hrda), reinterpret_cast<float*>(hq + J.hrca),
                             reinterpret_cast<int32_t*>(hq + J.hrs16), mm * hnb + b);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < B; j++) {
        const int t = lane + 64 * j;
        if (t < G * B) {
            const int m = small_div(t, G), rl = t - m * G;
            const int64_t orow = C <= 64 ? u * G + rl : u;
            if (orow < N) J.y[m * N + orow] = yacc[j];
        }
    }
}

// h = silu(g) * u element by element (the gate/up pair's fallback path).
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ g,
                                                const float* __restrict__ u,
                                                float* __restrict__ h, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) h[i] = swiglu(g[i], u[i]);
}

// Workgroups of the dot kernel for one GEMV: one wave per unit, 4 per group.
// paired: a gate/up pair (a unit holds G/2 rows of each).
inline int64_t dot_blocks(int type, int64_t N, int64_t K, int waves, bool paired = false) {
    const int nb = (int)(K / 32), C = (nb + 7) / 8;
    int64_t G = 64 / (C <= 64 ? C : 64);  // rows per unit, as k_dot
    if (paired) G >>= 1;
    (void)type;
    const int64_t units = C <= 64 ? (N + G - 1) / G : N;
    return (units + waves - 1) / waves;
}

inline size_t dot_shmem(int B, int64_t K, int waves) {
    return (size_t)B * act_lds_row_bytes(K) + (size_t)waves * B * 256;
}

// Raise a kernel's dynamic-LDS limit to the full 160 KB, once per kernel and
// device.  The state is atomic, so concurrent first calls from several host
// threads are safe (both may set the attribute, which is idempotent); a
// failure is returned to the caller and retried on the next call.
inline int raise_lds_limit(const void* kernel, std::atomic<int> (&state)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return (int)hipErrorInvalidDevice;
    std::atomic<int>* st = dev >= 0 && dev < 64 ? &state[dev] : nullptr;
    if (st && st->load(std::memory_order_acquire) == 1) return 0;
    const hipError_t rc =
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (rc != hipSuccess) return (int)rc;
    if (st) st->store(1, std::memory_order_release);
    return 0;
}

template <int FMT, int B, bool FUSED, int MODE, bool Q8K, bool WHOLE>
int launch_dot_variant(const DotJobs& jobs, int64_t blocks, size_t shmem, hipStream_t s) {
    static std::atomic<int> lds_state[64];
    const int arc = raise_lds_limit(
        reinterpret_cast<const void*>(&k_dot<FMT, B, FUSED, MODE, Q8K, WHOLE>), lds_state);
    if (arc) return arc;
    hipLaunchKernelGGL((k_dot<FMT, B, FUSED, MODE, Q8K, WHOLE>), dim3((unsigned)blocks),
                       dim3(64 * jobs.waves), shmem, s, jobs);
    return (int)hipGetLastError();
}

// WHOLE: every job's rows are whole 256-element chunks (always for the
// 256-element formats), which the lean loads need.
template <int FMT, int B, bool FUSED, int MODE, bool Q8K = false>
int launch_dot_kernel(const DotJobs& jobs, int64_t blocks, size_t shmem, hipStream_t s) {
    if constexpr (Fmt<FMT>::QK == 256 || !lean_loads<FMT>()) {
        return launch_dot_variant<FMT, B, FUSED, MODE, Q8K, lean_loads<FMT>()>(jobs, blocks, shmem,
                                                                                 s);
    } else {
        bool whole = true;
        for (int k = 0; k < jobs.count; k++) whole = whole && jobs.j[k].K % 256 == 0;
        return whole ? launch_dot_variant<FMT, B, FUSED, MODE, Q8K, true>(jobs, blocks, shmem, s)
                     : launch_dot_variant<FMT, B, FUSED, MODE, Q8K, false>(jobs, blocks, shmem, s);
    }
}

// The formats whose paired launch can also quantise h (the others run the
// quantisation as a launch of its own)
constexpr bool pairedq_format(int fmt) {
    return fmt == T_Q4_0 || fmt == T_Q5_0 || fmt == T_Q8_0 || fmt == T_Q4_K || fmt == T_Q6_K;
}

template <int FMT, int B, bool FUSED>
int launch_dot_jobs(const DotJobs& jobs, bool paired, int64_t blocks, size_t shmem,
                    hipStream_t s) {
    if (paired && jobs.j[0].hq) {
        if constexpr (pairedq_format(FMT))
            return launch_dot_kernel<FMT, B, FUSED, MODE_PAIRED_Q>(jobs, blocks, shmem, s);
        return (int)hipErrorInvalidValue;
    }
    if (paired) return launch_dot_kernel<FMT, B, FUSED, MODE_PAIRED>(jobs, blocks, shmem, s);
    return jobs.count == 1 ? launch_dot_kernel<FMT, B, FUSED, MODE_SINGLE>(jobs, blocks, shmem, s)
                           : launch_dot_kernel<FMT, B, FUSED, MODE_GROUP>(jobs, blocks, shmem, s);
}

template <int FMT>
int launch_dot_rows(const DotJobs& jobs, int64_t rows, bool fused, bool paired, int64_t blocks,
                    size_t shmem, hipStream_t s) {
    switch (rows) {
    case 1: return fused ? launch_dot_jobs<FMT, 1, true>(jobs, paired, blocks, shmem, s)
                         : launch_dot_jobs<FMT, 1, false>(jobs, paired, blocks, shmem, s);
    case 2: return fused ? launch_dot_jobs<FMT, 2, true>(jobs, paired, blocks, shmem, s)
                         : launch_dot_jobs<FMT, 2, false>(jobs, paired, blocks, shmem, s);
    case 3: return fused ? launch_dot_jobs<FMT, 3, true>(jobs, paired, blocks, shmem, s)
                         : launch_dot_jobs<FMT, 3, false>(jobs, paired, blocks, shmem, s);
    default: return fused ? launch_dot_jobs<FMT, 4, true>(jobs, paired, blocks, shmem, s)
                          : launch_dot_jobs<FMT, 4, false>(jobs, paired, blocks, shmem, s);
    }
}

// One launch of the dot kernel over `count` GEMVs of one type and row count.
// up != NULL: one gate/up pair (d[0].w the gate blob, up the up blob, count
// 1) whose output d[0].y receives h = silu(gate) * up.  waves: 4 or 8 waves
// per workgroup, or 0 to choose by the grid size.
int launch_dot(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t s,
               const uint8_t* up = nullptr, int waves = 0, uint8_t* hq = nullptr) {
    if (count < 1 || count > MAX_JOBS) return (int)hipErrorInvalidValue;
    const bool paired = up != nullptr;
    if (paired && count != 1) return (int)hipErrorInvalidValue;
    DotJobs jobs{};
    jobs.count = count;
    int64_t blocks = 0;
    size_t shmem = 0;
    const bool fused = d[0].x != nullptr;
    // 4-wave workgroups, unless that grid would just overrun the 256 CUs:
    // then 8-wave workgroups fit the same waves in one round of workgroups
    // (one per CU) instead of leaving a second round for a few CUs.
    int64_t blocks4 = 0;
    for (int k = 0; k < count; k++) blocks4 += dot_blocks(type, d[k].N, d[k].K, 4, paired);
    jobs.waves = waves ? waves : blocks4 > 256 && blocks4 <= 512 ? 8 : 4;
    // Jobs in decreasing workgroup count along the flat grid (the largest
    // GEMV's workgroups are dispatched first).
    int order[MAX_JOBS];
    for (int k = 0; k < count; k++) {
        int at = k;
        const int64_t bk = dot_blocks(type, d[k].N, d[k].K, 4);
        while (at > 0 && dot_blocks(type, d[order[at - 1]].N, d[order[at - 1]].K, 4) < bk) {
            order[at] = order[at - 1];
            at--;
        }
        order[at] = k;
    }
    for (int jk = 0; jk < count; jk++) {
        const int k = order[jk];
        const ActLayout L = act_layout(rows, d[k].K);
        DotJob& J = jobs.j[jk];
        J.w = d[k].w;
        J.w2 = up;
        J.y = d[k].y;
        J.x = d[k].x;
        J.xq = d[k].xq;
        J.N = d[k].N;
        J.K = d[k].K;
        J.wbytes = d[k].N * row_bytes(type, d[k].K);
        J.rcodes = L.rcodes;
        J.rda = L.rda;
        J.rca = L.rca;
        J.rs16 = L.rs16;
        J.hq = hq;
        if (hq) {
            const ActLayout H = act_layout(rows, d[k].N);
            J.hnb = H.nb;
            J.hrcodes = H.rcodes;
            J.hrda = H.rda;
            J.hrca = H.rca;
            J.hrs16 = H.rs16;
        }
        const int64_t bk = dot_blocks(type, d[k].N, d[k].K, jobs.waves, paired);
        if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
        jobs.start[jk] = (int)blocks;
        blocks += bk;  // the flat grid: every job's workgroups in turn
        const size_t sh = dot_shmem((int)rows, d[k].K, jobs.waves) + (hq ? rows * 32 * 4 : 0);
        shmem = sh > shmem ? sh : shmem;
    }
    if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    switch (type) {
    case T_Q8_0: return launch_dot_rows<T_Q8_0>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q4_0: return launch_dot_rows<T_Q4_0>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q5_0: return launch_dot_rows<T_Q5_0>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q4_1: return launch_dot_rows<T_Q4_1>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q5_1: return launch_dot_rows<T_Q5_1>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q8_1: return launch_dot_rows<T_Q8_1>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q4_K: return launch_dot_rows<T_Q4_K>(jobs, rows, fused, paired, blocks, shmem, s);
    case T_Q6_K: return launch_dot_rows<T_Q6_K>(jobs, rows, fused, paired, blocks, shmem, s);
    }
    return (int)hipErrorInvalidValue;
}

// Rows of the 16-row activation group each lane needs (see chunk_math).
inline int ni_for(int64_t rows) { return rows == 1 ? 1 : rows == 2 ? 2 : 4; }

template <int FMT, int NI>
int launch_qmv_ni(const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t rows,
                  float* y, int32_t* P, hipStream_t s, bool partials) {
    using F = Fmt<FMT>;
    const ActLayout L = act_layout(rows, K);
    const int64_t tiles = (N + 15) / 16;
    const int nb = (int)(K / 32), C = (nb + 7) / 8;
    const int64_t TG = tiles * L.G;
    const int64_t wbytes = N * (K / F::QK) * F::BB;
    // Enough tiles to fill the chip with independent waves: persistent waves
    // walking whole tiles.  Otherwise split each tile's chunks over the waves
    // of a workgroup (<= 8 waves keeps its LDS under 64 KB).
    const int64_t CHIP_WAVES = 256 * 16;
    if (!partials && TG >= 2048) {
        const int64_t per = (TG + CHIP_WAVES - 1) / CHIP_WAVES;  // tiles per wave
        const int64_t waves = (TG + per - 1) / per;
        const int64_t blocks = (waves + 3) / 4;
        hipLaunchKernelGGL((k_qmv_rows<FMT, NI>), dim3((unsigned)blocks), dim3(256),
                           4 * wave_lds<FMT>(), s, w, wbytes, N, K, xq, L, rows, tiles, y);
        return (int)hipGetLastError();
    }
    int KS = 1;
    while (KS < 8 && TG * KS < 4096 && KS * 2 <= C) KS *= 2;
    // the in-order combine gives one thread to each of the 16*rows outputs
    const int need = (int)((16 * (rows < 16 ? rows : 16) + 63) / 64);
    if (!partials && KS < need) KS = need;
    const size_t shmem = (size_t)KS * wave_lds<FMT>() + (partials ? 0 : (size_t)KS * 1024);
    if (partials)
        hipLaunchKernelGGL((k_qmv_split<FMT, 4, true>), dim3((unsigned)TG), dim3(64 * KS), shmem, s,
                           w, wbytes, N, K, xq, L, rows, tiles, y, P);
    else
        hipLaunchKernelGGL((k_qmv_split<FMT, NI, false>), dim3((unsigned)TG), dim3(64 * KS), shmem,
                           s, w, wbytes, N, K, xq, L, rows, tiles, y, P);
    return (int)hipGetLastError();
}

template <int FMT>
int launch_qmv_t(const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t rows,
                 float* y, int32_t* P, hipStream_t s, bool partials) {
    switch (ni_for(rows)) {
    case 1: return launch_qmv_ni<FMT, 1>(w, N, K, xq, rows, y, P, s, partials);
    case 2: return launch_qmv_ni<FMT, 2>(w, N, K, xq, rows, y, P, s, partials);
    default: return launch_qmv_ni<FMT, 4>(w, N, K, xq, rows, y, P, s, partials);
    }
}

// The lane-per-chunk kernel takes up to DOT_MAX_ROWS rows whose activations fit
// in a workgroup's LDS; everything else up to 16 rows runs on MFMA.
bool use_dot(int64_t rows, int64_t K) {
    return rows <= DOT_MAX_ROWS && rows * act_lds_row_bytes(K) + 8 * rows * 256 <= DOT_MAX_ACT_LDS;
}

// The same quantisation for the row staging alone (the decode GEMV's, B <= 4),
// 8 lanes per 32-block, 4 elements per lane: coalesced loads, every lane
// writing its own 4 codes.
template <bool A16>
__global__ __launch_bounds__(256) void k_quantize_row(const float* __restrict__ x,
                                                      uint8_t* __restrict__ xq, int64_t rows,
                                                      int64_t K, ActLayout L) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nb = L.nb;
    const int64_t blk = t >> 3;               // uniform over each group of 8 lanes
    const bool live = blk < rows * nb;        // (the shuffles below take every lane)
    const int sub = (int)(t & 7);
    const int64_t r = live ? blk / nb : 0, b = live ? blk - r * nb : 0;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
        const float* xb = x + r * K + 32 * b + 4 * sub;
        if constexpr (A16) {
            const float4 f = *reinterpret_cast<const float4*>(xb);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) v[i] = xb[i];
        }
    }
    quant_block8(v, sub, live, xq + (r * nb + b) * 34, xq + L.rcodes + r * K + 32 * b,
                 reinterpret_cast<float*>(xq + L.rda), reinterpret_cast<float*>(xq + L.rca),
                 reinterpret_cast<int32_t*>(xq + L.rs16), r * nb + b);
}

}  // namespace

bool group_is_one_launch(const GemvDesc* d, int count, int64_t rows) {
    bool one = count >= 1 && count <= MAX_JOBS;
    for (int k = 0; k < count && one; k++)
        one = use_dot(rows, d[k].K) && ((d[k].x != nullptr) == (d[0].x != nullptr));
    return one;
}

int staging_for(int64_t rows, int64_t K) {
    if (rows > 16) return ST_F16;
    return use_dot(rows, K) ? ST_ROW : ST_MFMA;
}

int launch_quantize(const float* x, uint8_t* xq, int64_t rows, int64_t K, int staging,
                    hipStream_t s) {
    const ActLayout L = act_layout(rows, K);
    if (staging == ST_ROW) {
        const unsigned grid = (unsigned)((rows * L.nb * 8 + 255) / 256);
        if (aligned16(x))
            hipLaunchKernelGGL((k_quantize_row<true>), dim3(grid), dim3(256), 0, s, x, xq, rows, K, L);
        else
            hipLaunchKernelGGL((k_quantize_row<false>), dim3(grid), dim3(256), 0, s, x, xq, rows, K, L);
        return (int)hipGetLastError();
    }
    const int64_t threads = ((staging & ST_MFMA) ? 16 * L.G : rows) * L.nb;
    if (aligned16(x))
        hipLaunchKernelGGL((k_quantize<false, true>), dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, s, x, xq, rows, K, L, staging);
    else
        hipLaunchKernelGGL((k_quantize<false, false>), dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, s, x, xq, rows, K, L, staging);
    return (int)hipGetLastError();
}

int launch_rebuild(uint8_t* xq, int64_t rows, int64_t K, int staging, hipStream_t s) {
    const ActLayout L = act_layout(rows, K);
    const int64_t threads = ((staging & ST_MFMA) ? 16 * L.G : rows) * L.nb;
    hipLaunchKernelGGL((k_quantize<true, true>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, nullptr, xq, rows, K, L, staging);
    return (int)hipGetLastError();
}

int launch_qmv(int type, const uint8_t* w, int64_t N, int64_t K, const float* x, uint8_t* xq,
               int64_t rows, float* y, hipStream_t s) {
    if (use_dot(rows, K)) {
        // quantisation fused into the kernel when x is given, unless the
        // workgroups' re-reads of x would exceed the weight bytes: then one
        // quantise launch first
        // (measured on the 8B-class down projection, 4096 x 14336 Q6_K: the
        // separate quantise launch plus the staged GEMV, 18.7 us, beats the
        // fused GEMV in 8-wave workgroups, which halve the re-reads, 20.7 us)
        const int64_t wbytes = N * row_bytes(type, K);
        if (x && (!aligned16(x) || dot_blocks(type, N, K, 4) * rows * K * 4 > wbytes)) {
            const int rc = launch_quantize(x, xq, rows, K, ST_ROW, s);
            if (rc) return rc;
            x = nullptr;
        }
        const GemvDesc d{w, N, K, x, xq, y};
        return launch_dot(type, &d, 1, rows, s);
    }
    if (!xq) return (int)hipErrorInvalidValue;  // the MFMA path reads a staged xq
    if (x) {
        const int rc = launch_quantize(x, xq, rows, K, ST_MFMA, s);
        if (rc) return rc;
    }
    switch (type) {
    case T_Q8_0: return launch_qmv_t<T_Q8_0>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q4_0: return launch_qmv_t<T_Q4_0>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q5_0: return launch_qmv_t<T_Q5_0>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q4_1: return launch_qmv_t<T_Q4_1>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q5_1: return launch_qmv_t<T_Q5_1>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q8_1: return launch_qmv_t<T_Q8_1>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q4_K: return launch_qmv_t<T_Q4_K>(w, N, K, xq, rows, y, nullptr, s, false);
    case T_Q6_K: return launch_qmv_t<T_Q6_K>(w, N, K, xq, rows, y, nullptr, s, false);
    }
    return (int)hipErrorInvalidValue;
}

int launch_qmv_group(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t s) {
    if (group_is_one_launch(d, count, rows)) {
        // the fused quantisation reads x with 16-byte loads: an entry whose x
        // is only 4-byte aligned is quantised by a launch of its own first
        GemvDesc e[MAX_JOBS];
        bool restaged = false;
        for (int k = 0; k < count; k++) {
            e[k] = d[k];
            if (d[k].x && !aligned16(d[k].x)) restaged = true;
        }
        if (restaged) {
            for (int k = 0; k < count; k++) {
                if (!e[k].xq) return (int)hipErrorInvalidValue;
                const int rc = launch_quantize(e[k].x, e[k].xq, rows, e[k].K, ST_ROW, s);
                if (rc) return rc;
                e[k].x = nullptr;
            }
        }
        return launch_dot(type, e, count, rows, s);
    }
    for (int k = 0; k < count; k++)  // one after another: each needs its xq
        if (!d[k].xq) return (int)hipErrorInvalidValue;
    for (int k = 0; k < count; k++) {
        const int rc = launch_qmv(type, d[k].w, d[k].N, d[k].K, d[k].x, d[k].xq, rows, d[k].y, s);
        if (rc) return rc;
    }
    return 0;
}

template <int FMT>
int launch_dot_partials_t(const DotJobs& jobs, int64_t rows, int64_t blocks, size_t shmem,
                          hipStream_t s) {
    switch (rows) {
    case 1: return launch_dot_kernel<FMT, 1, false, MODE_PARTIALS>(jobs, blocks, shmem, s);
    case 2: return launch_dot_kernel<FMT, 2, false, MODE_PARTIALS>(jobs, blocks, shmem, s);
    case 3: return launch_dot_kernel<FMT, 3, false, MODE_PARTIALS>(jobs, blocks, shmem, s);
    default: return launch_dot_kernel<FMT, 4, false, MODE_PARTIALS>(jobs, blocks, shmem, s);
    }
}

int launch_partials(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* xq,
                    int64_t rows, int32_t* P, hipStream_t s) {
    if (use_dot(rows, K)) {
        // the lane-per-chunk kernel, which qmv_launch runs at this many rows:
        // stage its copy from the Q8_0 blocks, then the kernel writes P
        int rc = launch_rebuild(xq, rows, K, ST_ROW, s);
        if (rc) return rc;
        const ActLayout L = act_layout(rows, K);
        DotJobs jobs{};
        jobs.count = 1;
        jobs.waves = 4;
        DotJob& J = jobs.j[0];
        J.w = w;
        J.w2 = nullptr;
        J.y = reinterpret_cast<float*>(P);
        J.x = nullptr;
        J.xq = xq;
        J.N = N;
        J.K = K;
        J.wbytes = N * row_bytes(type, K);
        J.rcodes = L.rcodes;
        J.rda = L.rda;
        J.rca = L.rca;
        J.rs16 = L.rs16;
        const int64_t blocks = dot_blocks(type, N, K, 4);
        const size_t shmem = dot_shmem((int)rows, K, 4);
        switch (type) {
        case T_Q8_0: return launch_dot_partials_t<T_Q8_0>(jobs, rows, blocks, shmem, s);
        case T_Q4_0: return launch_dot_partials_t<T_Q4_0>(jobs, rows, blocks, shmem, s);
        case T_Q5_0: return launch_dot_partials_t<T_Q5_0>(jobs, rows, blocks, shmem, s);
        case T_Q4_1: return launch_dot_partials_t<T_Q4_1>(jobs, rows, blocks, shmem, s);
        case T_Q5_1: return launch_dot_partials_t<T_Q5_1>(jobs, rows, blocks, shmem, s);
        case T_Q8_1: return launch_dot_partials_t<T_Q8_1>(jobs, rows, blocks, shmem, s);
        case T_Q4_K: return launch_dot_partials_t<T_Q4_K>(jobs, rows, blocks, shmem, s);
        case T_Q6_K: return launch_dot_partials_t<T_Q6_K>(jobs, rows, blocks, shmem, s);
        }
        return (int)hipErrorInvalidValue;
    }
    // otherwise the MFMA path: stage its copy from the Q8_0 blocks
    const int rc = launch_rebuild(xq, rows, K, ST_MFMA, s);
    if (rc) return rc;
    switch (type) {
    case T_Q8_0: return launch_qmv_ni<T_Q8_0, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q4_0: return launch_qmv_ni<T_Q4_0, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q5_0: return launch_qmv_ni<T_Q5_0, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q4_1: return launch_qmv_ni<T_Q4_1, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q5_1: return launch_qmv_ni<T_Q5_1, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q8_1: return launch_qmv_ni<T_Q8_1, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q4_K: return launch_qmv_ni<T_Q4_K, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    case T_Q6_K: return launch_qmv_ni<T_Q6_K, 4>(w, N, K, xq, rows, nullptr, P, s, true);
    }
    return (int)hipErrorInvalidValue;
}

int launch_qmm_partials(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* xq,
                        int64_t M, int32_t* P, hipStream_t s) {
    if (M <= 16) return launch_partials(type, w, N, K, xq, M, P, s);
    const int rc = launch_rebuild(xq, M, K, ST_F16, s);
    if (rc) return rc;
    return launch_gemm(type, w, N, K, xq, M, nullptr, s, P);
}

namespace {
template <int FMT, int MODE>
int launch_dot_q8k_t(const DotJobs& jobs, int64_t rows, int64_t blocks, size_t shmem,
                     hipStream_t s) {
    switch (rows) {
    case 1: return launch_dot_kernel<FMT, 1, false, MODE, true>(jobs, blocks, shmem, s);
    case 2: return launch_dot_kernel<FMT, 2, false, MODE, true>(jobs, blocks, shmem, s);
    case 3: return launch_dot_kernel<FMT, 3, false, MODE, true>(jobs, blocks, shmem, s);
    default: return launch_dot_kernel<FMT, 4, false, MODE, true>(jobs, blocks, shmem, s);
    }
}
}  // namespace

// The batched Q8_K kernel for BDOT_MIN_ROWS..16 activation rows: one
// workgroup per 16-row weight tile, KS waves sharing its superblocks (more
// waves when the tiles alone would leave the chip short of work; at least
// enough threads for the in-order combine of 16 x rows outputs).
int launch_bdot_q8k(int type, const uint8_t* w, const uint8_t* w2, int64_t N, int64_t K,
                    const uint8_t* xq, int64_t rows, float* y, int32_t* P, hipStream_t s) {
    const int64_t tiles = (N + 15) / 16;
    const int C = (int)(K / 256), CT = w2 ? 2 * C : C;
    const ActLayoutK L = act_layout_q8k(rows, K);
    if (tiles > INT32_MAX || rows < 1 || rows > 16 || !L.gcodes || (w2 && P))
        return (int)hipErrorInvalidValue;
    // 8 waves per tile (measured best at 8 wherever a tile has 8 superblocks),
    // fewer when it has fewer; at least one thread per output for the combine
    int KS = 1;
    while (KS < 8 && KS * 2 <= CT) KS *= 2;
    const int need = (int)((16 * rows + 63) / 64);
    if (!P && KS < need) KS = need;
    const int64_t wbytes = N * row_bytes(type, K);
    const size_t pb = P ? 0 : (size_t)(CT < BDOT_WINDOW ? CT : BDOT_WINDOW) * 1024;
    const dim3 grid((unsigned)tiles), block(64 * KS);
    if (type == T_Q4_K) {
        const size_t sh = (size_t)KS * 16 * span_stride<T_Q4_K>() + pb;
        if (P)
            hipLaunchKernelGGL((k_bdot8k<T_Q4_K, true>), grid, block, sh, s, w, w, wbytes, N, K,
                               xq, L, rows, y, P);
        else if (w2)
            hipLaunchKernelGGL((k_bdot8k<T_Q4_K, false, true>), grid, block, sh, s, w, w2, wbytes,
                               N, K, xq, L, rows, y, P);
        else
            hipLaunchKernelGGL((k_bdot8k<T_Q4_K, false>), grid, block, sh, s, w, w, wbytes, N, K,
                               xq, L, rows, y, P);
    } else {
        const size_t sh = (size_t)KS * 16 * span_stride<T_Q6_K>() + pb;
        if (P)
            hipLaunchKernelGGL((k_bdot8k<T_Q6_K, true>), grid, block, sh, s, w, w, wbytes, N, K,
                               xq, L, rows, y, P);
        else if (w2)
            hipLaunchKernelGGL((k_bdot8k<T_Q6_K, false, true>), grid, block, sh, s, w, w2, wbytes,
                               N, K, xq, L, rows, y, P);
        else
            hipLaunchKernelGGL((k_bdot8k<T_Q6_K, false>), grid, block, sh, s, w, w, wbytes, N, K,
                               xq, L, rows, y, P);
    }
    return (int)hipGetLastError();
}

int launch_group_q8k(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t s) {
    if (count < 1 || count > 8) return (int)hipErrorInvalidValue;
    const int64_t K = d[0].K;
    bool one = rows >= BDOT_MIN_ROWS && rows <= 16;
    for (int k = 0; k < count; k++) one = one && d[k].K == K;
    for (int k = 0; k < count; k++) {
        if (d[k].x) {
            const int rc = launch_quantize_q8k(d[k].x, d[k].xq, rows, d[k].K, s);
            if (rc) return rc;
        }
    }
    if (!one) {
        // one after another, each as qmv_launch_q8k on its staged xq
        for (int k = 0; k < count; k++) {
            const int rc = launch_qmv_q8k(type, d[k].w, d[k].N, d[k].K, nullptr, d[k].xq, rows,
                                          d[k].y, nullptr, s);
            if (rc) return rc;
        }
        return 0;
    }
    const int C = (int)(K / 256);
    const ActLayoutK L = act_layout_q8k(rows, K);
    BdotJobs jobs{};
    jobs.count = count;
    int64_t tiles = 0;
    for (int k = 0; k < count; k++) {
        jobs.j[k] = BdotJob{d[k].w, d[k].xq, d[k].y, d[k].N};
        if (tiles > INT32_MAX) return (int)hipErrorInvalidValue;
        jobs.start[k] = (int)tiles;
        tiles += (d[k].N + 15) / 16;
    }
    if (tiles > INT32_MAX || !L.gcodes) return (int)hipErrorInvalidValue;
    jobs.start[count] = (int)tiles;
    // the single launch's wave count and LDS (one K, so one choice)
    int KS = 1;
    while (KS < 8 && KS * 2 <= C) KS *= 2;
    const int need = (int)((16 * rows + 63) / 64);
    if (KS < need) KS = need;
    const size_t pb = (size_t)(C < BDOT_WINDOW ? C : BDOT_WINDOW) * 1024;
    const dim3 grid((unsigned)tiles), block(64 * KS);
    if (type == T_Q4_K)
        hipLaunchKernelGGL(k_bdot8k_group<T_Q4_K>, grid, block,
                           (size_t)KS * 16 * span_stride<T_Q4_K>() + pb, s, jobs, K, L, rows);
    else
        hipLaunchKernelGGL(k_bdot8k_group<T_Q6_K>, grid, block,
                           (size_t)KS * 16 * span_stride<T_Q6_K>() + pb, s, jobs, K, L, rows);
    return (int)hipGetLastError();
}

int launch_gateup_q8k(int type, const uint8_t* wg, const uint8_t* wu, int64_t N, int64_t K,
                      const float* x, uint8_t* xq, int64_t rows, float* h, hipStream_t s) {
    if (x) {
        const int rc = launch_quantize_q8k(x, xq, rows, K, s);
        if (rc) return rc;
    }
    return launch_bdot_q8k(type, wg, wu, N, K, xq, rows, h, nullptr, s);
}

int launch_qmv_q8k(int type, const uint8_t* w, int64_t N, int64_t K, const float* x, uint8_t* xq,
                   int64_t rows, float* y, int32_t* P, hipStream_t s) {
    // x given: quantise it; the partials hook rebuilds the staging from the
    // Q8_K blocks; otherwise xq is used as staged
    if (x || P) {
        const int rc = launch_quantize_q8k(x, xq, rows, K, s);
        if (rc) return rc;
    }
    // BDOT_MIN_ROWS..16 rows: the batched MFMA kernel; prefill: the GEMM
    if (rows > 16) return launch_gemm_q8k(type, w, N, K, xq, rows, y, P, false, s);
    if (rows >= BDOT_MIN_ROWS) return launch_bdot_q8k(type, w, nullptr, N, K, xq, rows, y, P, s);
    // fewer rows run the lane-per-chunk kernel (one launch), unless their
    // activation rows do not fit its LDS: then the batched kernel too
    if (!use_dot(rows, K)) return launch_bdot_q8k(type, w, nullptr, N, K, xq, rows, y, P, s);
    const ActLayoutK L = act_layout_q8k(rows, K);
    const int per = type == T_Q4_K ? 2 : 1;
    for (int64_t r0 = 0; r0 < rows; r0 += 4) {
        const int64_t rg = rows - r0 < 4 ? rows - r0 : 4;
        DotJobs jobs{};
        jobs.count = 1;
        jobs.waves = 4;
        DotJob& J = jobs.j[0];
        J.w = w;
        J.w2 = nullptr;
        // rows r0.. of the output (or of the partials) and of the staging
        J.y = P ? reinterpret_cast<float*>(P + r0 * N * (K / 256) * per) : y + r0 * N;
        J.x = nullptr;
        J.xq = xq;
        J.N = N;
        J.K = K;
        J.wbytes = N * row_bytes(type, K);
        J.rcodes = L.rcodes + r0 * K;
        J.rda = L.rda + r0 * L.nb * 4;
        J.rca = J.rda;  // not read on this path
        J.rs16 = L.rs16 + r0 * L.nb * 4;
        const int64_t blocks4 = dot_blocks(type, N, K, 4);
        if (blocks4 > 256 && blocks4 <= 512) jobs.waves = 8;
        const int64_t blocks = dot_blocks(type, N, K, jobs.waves);
        const size_t shmem = dot_shmem((int)rg, K, jobs.waves);
        if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
        int rc = (int)hipErrorInvalidValue;
        switch (type) {
        case T_Q4_K: rc = P ? launch_dot_q8k_t<T_Q4_K, MODE_PARTIALS>(jobs, rg, blocks, shmem, s)
                            : launch_dot_q8k_t<T_Q4_K, MODE_SINGLE>(jobs, rg, blocks, shmem, s);
            break;
        case T_Q6_K: rc = P ? launch_dot_q8k_t<T_Q6_K, MODE_PARTIALS>(jobs, rg, blocks, shmem, s)
                            : launch_dot_q8k_t<T_Q6_K, MODE_SINGLE>(jobs, rg, blocks, shmem, s);
            break;
        }
        if (rc) return rc;
    }
    return 0;
}

bool gateup_is_one_launch(int64_t rows, int64_t K) {
    const int64_t C = (K / 32 + 7) / 8;
    return use_dot(rows, K) && C <= 32;  // at least one gate/up row pair per wave
}

// The paired launch also quantises h when its workgroups, of 32/GP waves,
// cover whole 32-element blocks of h: GP (gate/up row pairs per wave)
// divides 32 and is at least 4 (workgroups of up to 8 waves: with 16, at
// K = 4096, one workgroup fits a CU and the launch took 22.0 us against 18.5
// for the plain pair plus about 3 for the quantisation launch), N is whole
// blocks, and the down projection reads the row staging.
bool gateup_quantises_h(int type, int64_t rows, int64_t N, int64_t K) {
    if (!gateup_is_one_launch(rows, K) || N % 32 || staging_for(rows, N) != ST_ROW) return false;
    if (!(type == T_Q4_0 || type == T_Q5_0 || type == T_Q8_0 || type == T_Q4_K || type == T_Q6_K))
        return false;
    const int C = (int)((K / 32 + 7) / 8), GP = (64 / C) >> 1;
    return GP >= 4 && 32 % GP == 0;
}

int launch_gateup(int type, const uint8_t* wg, const uint8_t* wu, int64_t N, int64_t K,
                  const float* x, uint8_t* xq, int64_t rows, float* h, hipStream_t s,
                  uint8_t* hq) {
    if (gateup_is_one_launch(rows, K)) {
        // one launch: each wave takes matching gate and up rows (the
        // quantisation fused as in qmv_launch, with the same rule for when
        // the workgroups' re-reads of x call for a launch of its own)
        if (x && (!aligned16(x) ||
                  dot_blocks(type, N, K, 4, true) * rows * K * 4 > 2 * N * row_bytes(type, K))) {
            const int rc = launch_quantize(x, xq, rows, K, ST_ROW, s);
            if (rc) return rc;
            x = nullptr;
        }
        const GemvDesc d{wg, N, K, x, xq, h};
        if (hq && gateup_quantises_h(type, rows, N, K)) {
            const int C = (int)((K / 32 + 7) / 8), GP = (64 / C) >> 1;
            return launch_dot(type, &d, 1, rows, s, wu, 32 / GP, hq);
        }
        const int rc = launch_dot(type, &d, 1, rows, s, wu);
        if (rc || !hq) return rc;
        return launch_quantize(h, hq, rows, N, staging_for(rows, N), s);
    }
    // otherwise: quantise once, gate and up into the scratch after the
    // activation copy, then the SwiGLU
    const int64_t act = align256(act_layout(rows, K).total);
    float* gt = reinterpret_cast<float*>(xq + act);
    float* ut = reinterpret_cast<float*>(xq + act + align256(rows * N * 4));
    int rc = 0;
    if (x && (rc = launch_quantize(x, xq, rows, K, staging_for(rows, K), s))) return rc;
    if ((rc = launch_qmv(type, wg, N, K, nullptr, xq, rows, gt, s))) return rc;
    if ((rc = launch_qmv(type, wu, N, K, nullptr, xq, rows, ut, s))) return rc;
    const int64_t n = rows * N;
    hipLaunchKernelGGL(k_swiglu, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gt, ut, h, n);
    if ((rc = (int)hipGetLastError()) || !hq) return rc;
    return launch_quantize(h, hq, rows, N, staging_for(rows, N), s);
}

int launch_qmm(int type, const uint8_t* w, int64_t N, int64_t K, const float* x, uint8_t* xq,
               int64_t rows, float* y, hipStream_t s) {
    if (rows <= 16) return launch_qmv(type, w, N, K, x, xq, rows, y, s);
    if (x) {
        const int rc = launch_quantize(x, xq, rows, K, ST_F16, s);
        if (rc) return rc;
    }
    return launch_gemm(type, w, N, K, xq, rows, y, s);
}

}  // namespace qmv
