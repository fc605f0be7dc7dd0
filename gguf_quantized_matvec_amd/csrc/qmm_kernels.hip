// Prefill GEMM (MatMul) for gfx950: Y[M][N] = X[M][K] * W^T with GGUF block
// weights and Q8_0 activations, on MFMA.
//
// The pages call prefill arithmetic-bound (llamay "Architecture", bench
// transcript), so this is the one place the path is a dense contraction.  Its
// cost is not the integer dot but the per-block scaling: every (row, column,
// 32-block) needs its own f32 term added in the documented order.  Two facts
// measured on the hardware keep that to one VALU fma per output and block:
//   * f16 MFMA on small integers is exact: codes (|a| <= 127; weights |w| <=
//     945 after folding Q4_K's 6-bit sub-scale in) are exact in f16, their
//     products and sums (< 2^24) are exact in the f32 accumulator, so
//     v_mfma_f32_32x32x16_f16 returns the exact integer block partial;
//   * the product of two fp16 values is exact in f32 (subnormals included),
//     so a rank-1 MFMA (one nonzero k) gives every d_w * d_a of a 32x32 tile.
// Then p = fma(I, d_w*d_a, p) is exactly the term the GEMV adds, and rows are
// bit-identical to the batch-1 GEMV.
//
// Tiling: a workgroup owns 128 x 128 outputs (4 waves of 64 x 64, each 2 x 2
// MFMA tiles of 32 x 32) and walks K one 256-element chunk (8 blocks) at a
// time.  Each thread fetches half a chunk of one activation row and one weight
// row into registers; after the chunk in LDS has been consumed it decodes the
// weights to f16 and stores both, then issues the loads of the next chunk,
// which stay in flight while the 8 blocks are multiplied.  LDS rows are XOR
// swizzled in 16-byte pieces so that MFMA fragment reads spread over all
// banks.  Workgroups are ordered in groups of 8 M-tiles and mapped so that
// each XCD runs a contiguous range of them: concurrently resident workgroups
// on one XCD share activation and weight tiles through its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int T_Q4_0 = 2, T_Q8_0 = 8, T_Q4_K = 12, T_Q6_K = 14;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int TM = 128, TN = 128;

template <int FMT> struct GFmt;
template <> struct GFmt<T_Q8_0> { static constexpr int QK = 32, BB = 34; };
template <> struct GFmt<T_Q4_0> { static constexpr int QK = 32, BB = 18; };
template <> struct GFmt<T_Q4_K> { static constexpr int QK = 256, BB = 144; };
template <> struct GFmt<T_Q6_K> { static constexpr int QK = 256, BB = 210; };

__device__ __forceinline__ uint32_t ldu16(const uint8_t* p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8);
}
__device__ __forceinline__ _Float16 h_of_bits(uint32_t b) {
    const uint16_t u = (uint16_t)b;
    _Float16 h;
    __builtin_memcpy(&h, &u, 2);
    return h;
}
__device__ __forceinline__ float f_of_hbits(uint32_t b) { return (float)h_of_bits(b); }

// Scale fields of one weight row and 32-block.
struct WRow {
    uint32_t d;     // fp16 bits: block / superblock d
    uint32_t dmin;  // Q4_K: fp16 bits of dmin
    int sc, mn;     // Q4_K: 6-bit scale and min of the sub-block
    int s0, s1;     // Q6_K: int8 sub-scales of the two 16-element halves
};

// Weight bytes one staging thread fetches per chunk: the four 32-blocks
// 4*half .. 4*half+3 of its row's chunk (K-quants: the superblock's header
// and the quarter of codes those sub-blocks use).
template <int FMT> struct WRaw;
template <> struct WRaw<T_Q8_0> { uint32_t v[34]; };   // 4 x 34 B
template <> struct WRaw<T_Q4_0> { uint32_t v[18]; };   // 4 x 18 B
template <> struct WRaw<T_Q4_K> { uint32_t hdr[4]; uint32_t q[16]; };   // 16 B + 64 B of qs
template <> struct WRaw<T_Q6_K> { uint32_t ql[16]; uint32_t qh[8]; uint32_t s[2]; uint32_t d; };

// Fetch chunk c, half `half` of a weight row (blocks are 2-byte aligned).
template <int FMT>
__device__ __forceinline__ void fetch_w(const uint8_t* row, int c, int half, int nbc,
                                        WRaw<FMT>& r) {
    if constexpr (FMT == T_Q8_0 || FMT == T_Q4_0) {
        constexpr int BB = FMT == T_Q8_0 ? 34 : 18;
        const uint8_t* p = row + (int64_t)(8 * c + 4 * half) * BB;
        const int nblk = nbc - 4 * half;  // blocks of this half that exist (ragged last chunk)
        if (nblk >= 4) {
            __builtin_memcpy(r.v, p, 4 * BB);
        } else {
#pragma unroll
            for (int i = 0; i < BB; i++) r.v[i] = 0;
            for (int k = 0; k < nblk; k++) __builtin_memcpy(reinterpret_cast<uint8_t*>(r.v) + k * BB, p + k * BB, BB);
        }
    } else if constexpr (FMT == T_Q4_K) {
        const uint8_t* sb = row + (int64_t)144 * c;
        __builtin_memcpy(r.hdr, sb, 16);
        __builtin_memcpy(r.q, sb + 16 + 64 * half, 64);
    } else {
        const uint8_t* sb = row + (int64_t)210 * c;
        __builtin_memcpy(r.ql, sb + 64 * half, 64);
        __builtin_memcpy(r.qh, sb + 128 + 32 * half, 32);
        __builtin_memcpy(r.s, sb + 192 + 8 * half, 8);
        r.d = ldu16(sb + 208);
    }
}

// f16 pair (lo, hi) from 16-bit integers in the low bits of each half: the
// bits 0x6400 | v are the f16 value 1024 + v (v < 1024), so subtracting
// 1024 + bias exactly gives v - bias.
__device__ __forceinline__ uint32_t pk_ints_to_f16(uint32_t two, float bias) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
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

template <typename T>
__device__ __forceinline__ T byte_at(const uint32_t* v, int o) {
    return (T)reinterpret_cast<const uint8_t*>(v)[o];
}

// Decode block k (0..3) of the fetched half-chunk: 32 f16 codes (16 dwords,
// element order) and the block's scale fields.
template <int FMT>
__device__ __forceinline__ void decode_blk(const WRaw<FMT>& r, int k, int half, uint32_t (&o)[16],
                                           WRow& s) {
    if constexpr (FMT == T_Q8_0) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(r.v) + 34 * k;
        s.d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q;
            __builtin_memcpy(&q, blk + 2 + 4 * i, 4);
            // int8 x -> x ^ 0x80 = x + 128 in [0, 255]; minus 128 after the f16 trick
            bytes_to_f16(q ^ 0x80808080u, 128.0f, o[2 * i], o[2 * i + 1]);
        }
    } else if constexpr (FMT == T_Q4_0) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(r.v) + 18 * k;
        s.d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t q;
            __builtin_memcpy(&q, blk + 2 + 4 * i, 4);
            bytes_to_f16(q & 0x0F0F0F0Fu, 8.0f, o[2 * i], o[2 * i + 1]);                // 0..15
            bytes_to_f16((q >> 4) & 0x0F0F0F0Fu, 8.0f, o[8 + 2 * i], o[8 + 2 * i + 1]);  // 16..31
        }
    } else if constexpr (FMT == T_Q4_K) {
        const int j = 4 * half + k;  // sub-block
        s.d = r.hdr[0] & 0xFFFFu;
        s.dmin = r.hdr[0] >> 16;
        const uint8_t* s12 = reinterpret_cast<const uint8_t*>(r.hdr) + 4;
        if (j < 4) {
            s.sc = s12[j] & 63;
            s.mn = s12[j + 4] & 63;
        } else {
            s.sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
            s.mn = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
        }
        // codes q (0..15) times the sub-scale: sc*q <= 945 is exact in f16
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const _Float16 sch = (_Float16)(float)s.sc;
        const h2 sc2 = {sch, sch};
        const int base = 8 * (k >> 1);  // dword of qs[32*(j>>1)] inside this half's 64 bytes
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t nib = ((k & 1) ? (r.q[base + i] >> 4) : r.q[base + i]) & 0x0F0F0F0Fu;
            uint32_t f0, f1;
            bytes_to_f16(nib, 0.0f, f0, f1);
            h2 v0, v1;
            __builtin_memcpy(&v0, &f0, 4);
            __builtin_memcpy(&v1, &f1, 4);
            v0 = v0 * sc2;
            v1 = v1 * sc2;
            __builtin_memcpy(&o[2 * i], &v0, 4);
            __builtin_memcpy(&o[2 * i + 1], &v1, 4);
        }
    } else {
        const int kq = k;  // block 4*half + k of the superblock: h = half, kq = k
        s.d = r.d;
        s.s0 = byte_at<int8_t>(r.s, 2 * k);
        s.s1 = byte_at<int8_t>(r.s, 2 * k + 1);
        const int lbase = 8 * (kq & 1);  // dword of ql[32*(kq&1)] inside this half's 64 bytes
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t lo = ((kq & 2) ? (r.ql[lbase + i] >> 4) : r.ql[lbase + i]) & 0x0F0F0F0Fu;
            const uint32_t hi = ((r.qh[i] >> (2 * kq)) & 0x03030303u) << 4;
            bytes_to_f16(lo | hi, 32.0f, o[2 * i], o[2 * i + 1]);
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

// LDS of one chunk (8 blocks) of a 128 x 128 tile.  Tile rows hold 8 blocks x
// 32 f16 = 512 bytes as 32 pieces of 16 bytes; piece q of row r is stored at
// slot q ^ (r & 31) so the 32 rows a fragment read touches hit different banks.
struct Chunk {
    uint4 a[TM * 32];     // activation codes (f16)
    uint4 w[TN * 32];     // decoded weights (f16)
    uint32_t da[8][TM];   // fp16 bits of the activation block scales
    uint32_t dw[8][TN];   // fp16 bits of the weight d
    uint32_t x1[8][TN];   // Q4_K: dmin bits | m_j << 16;  Q6_K: s0 | s1 << 16
};
__device__ __forceinline__ int slot(int row, int q) { return row * 32 + (q ^ (row & 31)); }

template <int FMT>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ w, int64_t N, int64_t K,
                                              const uint8_t* __restrict__ xq, ActLayout L,
                                              int64_t M, int64_t tilesM, int64_t tilesN,
                                              float* __restrict__ y) {
    using F = GFmt<FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    Chunk& cs = *reinterpret_cast<Chunk*>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    int64_t tm, tn;
    tile_of(blockIdx.x, tilesM, tilesN, tm, tn);
    const int64_t m0 = tm * TM, n0 = tn * TN;
    const int nb = (int)(K >> 5), C = (nb + 7) >> 3;
    const int64_t R = (K / F::QK) * F::BB;

    // staging role: row srow, half shalf (blocks 4*shalf .. 4*shalf+3 of a chunk)
    const int srow = tid >> 1, shalf = tid & 1;
    const int64_t am = m0 + srow < M ? m0 + srow : M - 1;  // clamp: rows past M are discarded
    const int64_t wr = n0 + srow < N ? n0 + srow : N - 1;
    const uint8_t* arow = xq + L.hcodes + am * K * 2;
    const uint16_t* ahda = reinterpret_cast<const uint16_t*>(xq + L.hda) + am * nb;
    const uint8_t* wrow = w + wr * R;

    // next chunk, in registers
    uint4 ra[16];
    uint32_t rda[4];
    WRaw<FMT> rw;
    auto fetch = [&](int c) {
        const int nbc = min(8, nb - 8 * c);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int b = 8 * c + 4 * shalf + k;
            const bool ok = 4 * shalf + k < nbc;
            const uint4* src = reinterpret_cast<const uint4*>(arow + (int64_t)(ok ? b : 0) * 64);
#pragma unroll
            for (int q = 0; q < 4; q++) ra[4 * k + q] = ok ? src[q] : make_uint4(0, 0, 0, 0);
            rda[k] = ok ? ahda[b] : 0u;
        }
        fetch_w<FMT>(wrow, c, shalf, nbc, rw);
    };
    auto stage = [&](int c) {
        const int nbc = min(8, nb - 8 * c);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int bk = 4 * shalf + k;  // block inside the chunk
#pragma unroll
            for (int q = 0; q < 4; q++) cs.a[slot(srow, 4 * bk + q)] = ra[4 * k + q];
            cs.da[bk][srow] = rda[k];
            uint32_t o[16];
            WRow f;
            decode_blk<FMT>(rw, k, shalf, o, f);
            if (bk >= nbc) f.d = 0;  // ragged last chunk: the missing blocks add nothing
#pragma unroll
            for (int q = 0; q < 4; q++)
                cs.w[slot(srow, 4 * bk + q)] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
            cs.dw[bk][srow] = f.d;
            if (FMT == T_Q4_K) cs.x1[bk][srow] = f.dmin | ((uint32_t)f.mn << 16);
            if (FMT == T_Q6_K) cs.x1[bk][srow] = (uint32_t)(f.s0 & 0xFFFF) | ((uint32_t)f.s1 << 16);
        }
    };

    // accumulators: chunk sum p and running sum yv, per 32x32 tile (i, j)
    v16f p[2][2], yv[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) p[i][j][e] = yv[i][j][e] = 0.0f;

    const int lr = lane & 31, kq = lane >> 5;  // MFMA lane roles
    const v16f zero16 = {};
    fetch(0);
    for (int c = 0; c < C; c++) {
        __syncthreads();  // the previous chunk is fully consumed
        stage(c);
        __syncthreads();
        if (c + 1 < C) fetch(c + 1);  // streams while this chunk is multiplied
        const int nbc = min(8, nb - 8 * c);
        for (int bk = 0; bk < nbc; bk++) {
            // fragments: A rows 64wm + 32i + lr, B rows 64wn + 32j + lr; piece
            // 4*bk + 2h + kq holds k = 16h + 8kq .. +8 of block bk
            v8h A[2][2], Bf[2][2];
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int ra_ = 64 * wm + 32 * i + lr, rb_ = 64 * wn + 32 * i + lr;
                    const uint4 va = cs.a[slot(ra_, 4 * bk + 2 * h + kq)];
                    const uint4 vb = cs.w[slot(rb_, 4 * bk + 2 * h + kq)];
                    __builtin_memcpy(&A[i][h], &va, 16);
                    __builtin_memcpy(&Bf[i][h], &vb, 16);
                }
            // rank-1 operands of the scale products: only k = 0 is nonzero
            v8h Ra[2], Rw[2], Rm[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const v8h za = {};
                Ra[i] = za;
                Rw[i] = za;
                Rm[i] = za;
                if (kq == 0) {
                    Ra[i][0] = h_of_bits(cs.da[bk][64 * wm + 32 * i + lr]);
                    Rw[i][0] = h_of_bits(cs.dw[bk][64 * wn + 32 * i + lr]);
                    if (FMT == T_Q4_K) Rm[i][0] = h_of_bits(cs.x1[bk][64 * wn + 32 * i + lr] & 0xFFFFu);
                }
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const v16f S =
                        __builtin_amdgcn_mfma_f32_32x32x16_f16(Ra[i], Rw[j], zero16, 0, 0, 0);
                    if constexpr (FMT == T_Q6_K) {
                        const v16f I0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][0], Bf[j][0], zero16, 0, 0, 0);
                        const v16f I1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][1], Bf[j][1], zero16, 0, 0, 0);
                        const uint32_t s01 = cs.x1[bk][64 * wn + 32 * j + lr];
                        const float s0 = (float)(int16_t)(s01 & 0xFFFF), s1 = (float)((int)s01 >> 16);
#pragma unroll
                        for (int e = 0; e < 16; e++) {
                            const float I = fmaf(s0, I0[e], s1 * I1[e]);  // exact integer
                            p[i][j][e] = fmaf(I, S[e], p[i][j][e]);
                        }
                    } else {
                        v16f I = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][0], Bf[j][0], zero16, 0, 0, 0);
                        I = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][1], Bf[j][1], I, 0, 0, 0);
                        if constexpr (FMT == T_Q4_K) {
                            // Q = m_j * sum(a): B operand is m_j at every k
                            const _Float16 mh = (_Float16)(float)(cs.x1[bk][64 * wn + 32 * j + lr] >> 16);
                            v8h Mb;
#pragma unroll
                            for (int t = 0; t < 8; t++) Mb[t] = mh;
                            v16f Q = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][0], Mb, zero16, 0, 0, 0);
                            Q = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][1], Mb, Q, 0, 0, 0);
                            const v16f S2 =
                                __builtin_amdgcn_mfma_f32_32x32x16_f16(Ra[i], Rm[j], zero16, 0, 0, 0);
#pragma unroll
                            for (int e = 0; e < 16; e++) {
                                p[i][j][e] = fmaf(I[e], S[e], p[i][j][e]);
                                p[i][j][e] = fmaf(-Q[e], S2[e], p[i][j][e]);
                            }
                        } else {
#pragma unroll
                            for (int e = 0; e < 16; e++) p[i][j][e] = fmaf(I[e], S[e], p[i][j][e]);
                        }
                    }
                }
        }
        // end of the chunk: add it, in chunk order
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    yv[i][j][e] = yv[i][j][e] + p[i][j][e];
                    p[i][j][e] = 0.0f;
                }
    }

    // lane l, element e of tile (i, j): row 8(e/4) + 4kq + e%4, column lr
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t n = n0 + 64 * wn + 32 * j + lr;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * kq + (e & 3);
                if (m < M && n < N) y[m * N + n] = yv[i][j][e];
            }
        }
}

template <int FMT>
int launch_gemm_t(const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                  float* y, hipStream_t s) {
    const ActLayout L = act_layout(M, K);
    const int64_t tilesM = (M + TM - 1) / TM, tilesN = (N + TN - 1) / TN;
    static bool attr_set = false;  // the chunk tiles need more than the default 64 KB of LDS
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<FMT>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)sizeof(Chunk));
        if (e != hipSuccess) return (int)e;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_gemm<FMT>), dim3((unsigned)(tilesM * tilesN)), dim3(256), sizeof(Chunk),
                       s, w, N, K, xq, L, M, tilesM, tilesN, y);
    return (int)hipGetLastError();
}

}  // namespace

int launch_gemm(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                float* y, hipStream_t s) {
    switch (type) {
    case T_Q8_0: return launch_gemm_t<T_Q8_0>(w, N, K, xq, M, y, s);
    case T_Q4_0: return launch_gemm_t<T_Q4_0>(w, N, K, xq, M, y, s);
    case T_Q4_K: return launch_gemm_t<T_Q4_K>(w, N, K, xq, M, y, s);
    case T_Q6_K: return launch_gemm_t<T_Q6_K>(w, N, K, xq, M, y, s);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace qmv
