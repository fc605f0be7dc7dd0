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
// (llamay docs, "The three claims": same output regardless of batch
// composition).
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

#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int T_Q4_0 = 2, T_Q8_0 = 8, T_Q4_K = 12, T_Q6_K = 14;

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
// Q8_0 per 32-element block: amax, d = amax/127 (correctly rounded f32
// divide), id = 1/d (0 for an all-zero block), codes = round-half-away(x*id),
// stored scale fp16(d).  One thread per (row, block) of the 16-row-padded
// range; padding rows get zero codes and scales in the staging copy.
// FROM_PUBLIC: take codes and d from the Q8_0 blocks already in xq instead.
template <bool FROM_PUBLIC>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ x,
                                                  uint8_t* __restrict__ xq, int64_t rows,
                                                  int64_t K, ActLayout L) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nb = L.nb;
    if (t >= 16 * L.G * nb) return;
    const int64_t r = t / nb, b = t - r * nb;
    uint8_t q[32];
    float dval = 0.0f;
    if (r < rows) {
        uint8_t* pub = xq + (r * nb + b) * 34;
        if (!FROM_PUBLIC) {
            float v[32];
            const float4* xb = reinterpret_cast<const float4*>(x + r * K + 32 * b);
#pragma unroll
            for (int j = 0; j < 8; j++) {
                float4 f = xb[j];
                v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
            const float d = amax / 127.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
            for (int i = 0; i < 32; i++) q[i] = (uint8_t)(int8_t)(int)roundf(v[i] * id);
            const uint16_t h = float_to_half_bits(d);
            uint8_t blk[34];
            blk[0] = (uint8_t)(h & 255);
            blk[1] = (uint8_t)(h >> 8);
#pragma unroll
            for (int i = 0; i < 32; i++) blk[2 + i] = q[i];
            __builtin_memcpy(pub, blk, 34);
            dval = half_bits_to_float(h);
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
    const int64_t g = r >> 4;
    const int m = (int)(r & 15);
    const int64_t gb = g * nb + b;
    uint8_t* codes = xq + L.codes + gb * 512;
    int S = 0;
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
        uint64_t v = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            v |= (uint64_t)q[8 * kg + j] << (8 * j);
            S += (int8_t)q[8 * kg + j];
        }
        *reinterpret_cast<uint64_t*>(codes + (m + 16 * kg) * 8) = v;
    }
    reinterpret_cast<float*>(xq + L.da)[gb * 16 + m] = dval;
    reinterpret_cast<float*>(xq + L.ca)[gb * 16 + m] = dval * (float)S;
    reinterpret_cast<int32_t*>(xq + L.S)[gb * 16 + m] = S;
}

// ------------------------------------------------------------- formats ----
// QK: elements per GGUF block; BB: bytes per block; CB: bytes of one full
// 256-element chunk of a row; PPS: 16-byte pieces that cover one chunk span
// at the worst alignment the layout allows (Q4_K spans are always 16-byte
// aligned: 144 | 16*9 and w is 16-byte aligned; the others only 2-byte).
template <int FMT> struct Fmt;
template <> struct Fmt<T_Q8_0> { static constexpr int QK = 32, BB = 34, CB = 272, PPS = 18; };
template <> struct Fmt<T_Q4_0> { static constexpr int QK = 32, BB = 18, CB = 144, PPS = 10; };
template <> struct Fmt<T_Q4_K> { static constexpr int QK = 256, BB = 144, CB = 144, PPS = 9; };
template <> struct Fmt<T_Q6_K> { static constexpr int QK = 256, BB = 210, CB = 210, PPS = 14; };

template <int FMT> constexpr int span_stride() { return 16 * Fmt<FMT>::PPS + 16; }
template <int FMT> constexpr int pieces_per_lane() { return (16 * Fmt<FMT>::PPS + 63) / 64; }

// The final piece of the whole blob may run past its end: read it bytewise.
__device__ __attribute__((noinline)) uint4 tail_piece(const uint8_t* w, int64_t off,
                                                      int64_t wbytes) {
    uint32_t v[4] = {0, 0, 0, 0};
    for (int i = 0; i < 16; i++)
        if (off + i < wbytes) v[i >> 2] |= (uint32_t)w[off + i] << (8 * (i & 3));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Global -> registers: the 16 row spans of chunk c (rows n0..n0+15), as
// 16-byte pieces aligned down from each span start.  Piece p of the wave is
// lane p%64 of step p/64; it belongs to span p/PPS, offset 16*(p%PPS).
template <int FMT>
__device__ __forceinline__ void fetch_chunk(const uint8_t* __restrict__ w, int64_t wbytes,
                                            int64_t n0, int64_t N, int64_t R, int c, int nbc,
                                            int lane, uint4 (&reg)[pieces_per_lane<FMT>()]) {
    using F = Fmt<FMT>;
    const int len = F::QK == 32 ? nbc * F::BB : F::BB;
#pragma unroll
    for (int t = 0; t < pieces_per_lane<FMT>(); t++) {
        const int p = t * 64 + lane;
        const int n = p / F::PPS, j = p - n * F::PPS;
        reg[t] = make_uint4(0, 0, 0, 0);
        if (n < 16 && n0 + n < N) {
            const int64_t s = (n0 + n) * R + (int64_t)c * F::CB;
            const int64_t off = (s & ~int64_t(15)) + 16 * j;
            if (off < s + len) {
                if (off + 16 <= wbytes)
                    reg[t] = *reinterpret_cast<const uint4*>(w + off);
                else
                    reg[t] = tail_piece(w, off, wbytes);
            }
        }
    }
}

template <int FMT>
__device__ __forceinline__ void stage_chunk(uint8_t* wl, int lane,
                                            const uint4 (&reg)[pieces_per_lane<FMT>()]) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int t = 0; t < pieces_per_lane<FMT>(); t++) {
        const int p = t * 64 + lane;
        const int n = p / F::PPS, j = p - n * F::PPS;
        if (n < 16) *reinterpret_cast<uint4*>(wl + n * span_stride<FMT>() + 16 * j) = reg[t];
    }
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bytewise x - bias for bytes x in [0, 2*bias): add 128, subtract, flip bit 7
// (no borrow crosses a byte because every byte of x|0x80.. is >= 128).
__device__ __forceinline__ uint64_t bytes_minus(uint64_t x, uint64_t bias8) {
    const uint64_t hi = 0x8080808080808080ull;
    return ((x | hi) - bias8) ^ hi;
}

// --------------------------------------------------------------- GEMV -----
// Grid: one workgroup per (16 activation rows g, 16 weight rows); KS waves per
// workgroup split the chunks of those rows round-robin (chunk r0 + wave).
// After every round the chunk sums are combined in chunk order through LDS,
// so the f32 order is the documented one whatever KS is.
// PARTIALS: write the int32 block partials instead (test hook).
template <int FMT, bool PARTIALS>
__global__ __launch_bounds__(512) void k_qmv(const uint8_t* __restrict__ w, int64_t wbytes,
                                             int64_t N, int64_t K, const uint8_t* __restrict__ xq,
                                             ActLayout L, int64_t rows, int64_t tiles,
                                             float* __restrict__ y, int32_t* __restrict__ P) {
    using F = Fmt<FMT>;
    constexpr int STRIDE = span_stride<FMT>();
    constexpr int NP = pieces_per_lane<FMT>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, KS = blockDim.x >> 6;
    uint8_t* wl = smem + wv * (16 * STRIDE);
    float* pbuf = reinterpret_cast<float*>(smem + KS * 16 * STRIDE);
    const int64_t tile = blockIdx.x % tiles, g = blockIdx.x / tiles;
    const int64_t n0 = tile * 16;
    const int Bg = (int)(rows - 16 * g < 16 ? rows - 16 * g : 16);
    const int nb = (int)(K >> 5), C = (nb + 7) >> 3;
    const int64_t R = (K / F::QK) * F::BB;
    const int nn = lane & 15, kg = lane >> 4;
    const uint8_t* acodes = xq + L.codes + g * nb * 512 + lane * 8;
    const float* ada = reinterpret_cast<const float*>(xq + L.da) + g * nb * 16 + 4 * kg;
    const float* aca = reinterpret_cast<const float*>(xq + L.ca) + g * nb * 16 + 4 * kg;
    const int32_t* aS = reinterpret_cast<const int32_t*>(xq + L.S) + g * nb * 16 + 4 * kg;
    const bool a_ok = nn < Bg;          // this lane's A-operand row exists
    const bool s_ok = 4 * kg < Bg;      // some of this lane's 4 output rows exist

    float yacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    uint4 reg[NP];
    if (wv < C) {
        const int nbc0 = F::QK == 32 ? min(8, nb - 8 * wv) : 8;
        fetch_chunk<FMT>(w, wbytes, n0, N, R, wv, nbc0, lane, reg);
    }
    for (int r0 = 0; r0 < C; r0 += KS) {
        const int c = r0 + wv;
        float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (c < C) {
            stage_chunk<FMT>(wl, lane, reg);
            wave_sync();
            const int nbc = F::QK == 32 ? min(8, nb - 8 * c) : 8;
            const int cn = c + KS;
            if (cn < C) {
                const int nbcn = F::QK == 32 ? min(8, nb - 8 * cn) : 8;
                fetch_chunk<FMT>(w, wbytes, n0, N, R, cn, nbcn, lane, reg);
            }
            const int delta = (int)(((n0 + nn) * R + (int64_t)c * F::CB) & 15);
            const uint8_t* rb = wl + nn * STRIDE + delta;

            // per-chunk fields of the K-quant superblock
            float dw = 0.0f, dmw = 0.0f;
            uint32_t s12[3] = {0, 0, 0};
            if (FMT == T_Q4_K) {
                dw = half_bits_to_float(ld<uint16_t>(rb));
                dmw = half_bits_to_float(ld<uint16_t>(rb + 2));
                s12[0] = ld<uint32_t>(rb + 4);
                s12[1] = ld<uint32_t>(rb + 8);
                s12[2] = ld<uint32_t>(rb + 12);
            }
            if (FMT == T_Q6_K) dw = half_bits_to_float(ld<uint16_t>(rb + 208));

#pragma unroll
            for (int bb = 0; bb < 8; bb++) {
                if (F::QK == 32 && bb >= nbc) break;
                const int64_t b = (int64_t)8 * c + bb;
                const long a = a_ok ? *reinterpret_cast<const long*>(acodes + b * 512) : 0;
                const v4i zero = {0, 0, 0, 0};
                v4i acc, acc1 = zero;
                int sc = 0, mn = 0, s0 = 0, s1 = 0;
                if (FMT == T_Q8_0) {
                    const uint8_t* blk = rb + 34 * bb;
                    dw = half_bits_to_float(ld<uint16_t>(blk));
                    const long wc = ld<long>(blk + 2 + 8 * kg);
                    acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, wc, zero, 0, 0, 0);
                } else if (FMT == T_Q4_0) {
                    const uint8_t* blk = rb + 18 * bb;
                    dw = half_bits_to_float(ld<uint16_t>(blk));
                    uint64_t raw = ld<uint64_t>(blk + 2 + 8 * (kg & 1));
                    if (kg & 2) raw >>= 4;
                    const uint64_t wc =
                        bytes_minus(raw & 0x0F0F0F0F0F0F0F0Full, 0x0808080808080808ull);
                    acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, (long)wc, zero, 0, 0, 0);
                } else if (FMT == T_Q4_K) {
                    // 6-bit scale and min of sub-block bb (two per 12 bytes)
                    const uint8_t* sb = reinterpret_cast<const uint8_t*>(s12);
                    if (bb < 4) {
                        sc = sb[bb] & 63;
                        mn = sb[bb + 4] & 63;
                    } else {
                        sc = (sb[bb + 4] & 15) | ((sb[bb - 4] >> 6) << 4);
                        mn = (sb[bb + 4] >> 4) | ((sb[bb] >> 6) << 4);
                    }
                    uint64_t raw = ld<uint64_t>(rb + 16 + 32 * (bb >> 1) + 8 * kg);
                    if (bb & 1) raw >>= 4;
                    const uint64_t wc = raw & 0x0F0F0F0F0F0F0F0Full;
                    acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, (long)wc, zero, 0, 0, 0);
                } else {  // Q6_K
                    const int h = bb >> 2, kq = bb & 3;
                    uint64_t ql = ld<uint64_t>(rb + 64 * h + 32 * (kq & 1) + 8 * kg);
                    const uint64_t qh = ld<uint64_t>(rb + 128 + 32 * h + 8 * kg);
                    if (kq & 2) ql >>= 4;
                    const uint64_t q6 = (ql & 0x0F0F0F0F0F0F0F0Full) |
                                        (((qh >> (2 * kq)) & 0x0303030303030303ull) << 4);
                    const uint64_t wc = bytes_minus(q6, 0x2020202020202020ull);
                    s0 = (int8_t)rb[192 + 2 * bb];
                    s1 = (int8_t)rb[192 + 2 * bb + 1];
                    // the two 16-element halves carry different sub-scales:
                    // one MFMA per half, the other half's codes zeroed
                    const long lo = kg < 2 ? (long)wc : 0, hi = kg < 2 ? 0 : (long)wc;
                    acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, lo, zero, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, hi, zero, 0, 0, 0);
                }

                if (PARTIALS) {
                    int4 S4 = make_int4(0, 0, 0, 0);
                    if (FMT == T_Q4_K && s_ok) S4 = *reinterpret_cast<const int4*>(aS + b * 16);
                    const int Sv[4] = {S4.x, S4.y, S4.z, S4.w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int m = 4 * kg + i;
                        if (m < Bg && n0 + nn < N) {
                            const int64_t o = ((16 * g + m) * N + n0 + nn) * nb + b;
                            if (FMT == T_Q4_K) {
                                P[2 * o] = sc * acc[i];
                                P[2 * o + 1] = mn * Sv[i];
                            } else if (FMT == T_Q6_K) {
                                P[o] = s0 * acc[i] + s1 * acc1[i];
                            } else {
                                P[o] = acc[i];
                            }
                        }
                    }
                } else {
                    float4 da4 = make_float4(0.f, 0.f, 0.f, 0.f), ca4 = da4;
                    if (s_ok) {
                        da4 = *reinterpret_cast<const float4*>(ada + b * 16);
                        if (FMT == T_Q4_K) ca4 = *reinterpret_cast<const float4*>(aca + b * 16);
                    }
                    const float dav[4] = {da4.x, da4.y, da4.z, da4.w};
                    const float cav[4] = {ca4.x, ca4.y, ca4.z, ca4.w};
                    const float cw = FMT == T_Q4_K ? dmw * (float)mn : 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        if (4 * kg + i < Bg) {
                            if (FMT == T_Q4_K) {
                                p[i] = fmaf((float)(sc * acc[i]), dw * dav[i], p[i]);
                                p[i] = fmaf(-cw, cav[i], p[i]);
                            } else if (FMT == T_Q6_K) {
                                p[i] = fmaf((float)(s0 * acc[i] + s1 * acc1[i]), dw * dav[i], p[i]);
                            } else {
                                p[i] = fmaf((float)acc[i], dw * dav[i], p[i]);
                            }
                        }
                    }
                }
            }
            wave_sync();
        }
        if (!PARTIALS) {
            if (c < C) {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (4 * kg + i < Bg) pbuf[wv * 256 + (4 * kg + i) * 16 + nn] = p[i];
            }
            __syncthreads();
            const int nact = min(KS, C - r0);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int e = threadIdx.x + k * blockDim.x;
                if (e < 16 * Bg)
                    for (int w2 = 0; w2 < nact; w2++) yacc[k] = yacc[k] + pbuf[w2 * 256 + e];
            }
            __syncthreads();
        }
    }
    if (!PARTIALS) {
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int e = threadIdx.x + k * blockDim.x;
            if (e < 16 * Bg) {
                const int m = e >> 4, n = e & 15;
                if (n0 + n < N) y[(16 * g + m) * N + n0 + n] = yacc[k];
            }
        }
    }
}

template <int FMT, bool PARTIALS>
int launch_qmv_t(const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t rows,
                 float* y, int32_t* P, hipStream_t s) {
    using F = Fmt<FMT>;
    const ActLayout L = act_layout(rows, K);
    const int64_t tiles = (N + 15) / 16;
    const int nb = (int)(K / 32), C = (nb + 7) / 8;
    const int64_t wgs = tiles * L.G;
    int KS = 1;
    while (KS < 8 && wgs * KS < 2048 && KS * 2 <= C) KS *= 2;
    const size_t shmem = (size_t)KS * 16 * span_stride<FMT>() + (PARTIALS ? 0 : (size_t)KS * 1024);
    const int64_t wbytes = N * (K / F::QK) * F::BB;
    hipLaunchKernelGGL((k_qmv<FMT, PARTIALS>), dim3((unsigned)wgs), dim3(64 * KS), shmem, s, w,
                       wbytes, N, K, xq, L, rows, tiles, y, P);
    return (int)hipGetLastError();
}

}  // namespace

int launch_quantize(const float* x, uint8_t* xq, int64_t rows, int64_t K, hipStream_t s) {
    const ActLayout L = act_layout(rows, K);
    const int64_t threads = 16 * L.G * L.nb;
    hipLaunchKernelGGL(k_quantize<false>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, x, xq, rows, K, L);
    return (int)hipGetLastError();
}

int launch_rebuild(uint8_t* xq, int64_t rows, int64_t K, hipStream_t s) {
    const ActLayout L = act_layout(rows, K);
    const int64_t threads = 16 * L.G * L.nb;
    hipLaunchKernelGGL(k_quantize<true>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, nullptr, xq, rows, K, L);
    return (int)hipGetLastError();
}

int launch_qmv(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
               int64_t rows, float* y, hipStream_t s) {
    switch (type) {
    case T_Q8_0: return launch_qmv_t<T_Q8_0, false>(w, N, K, xq, rows, y, nullptr, s);
    case T_Q4_0: return launch_qmv_t<T_Q4_0, false>(w, N, K, xq, rows, y, nullptr, s);
    case T_Q4_K: return launch_qmv_t<T_Q4_K, false>(w, N, K, xq, rows, y, nullptr, s);
    case T_Q6_K: return launch_qmv_t<T_Q6_K, false>(w, N, K, xq, rows, y, nullptr, s);
    }
    return (int)hipErrorInvalidValue;
}

int launch_partials(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
                    int64_t rows, int32_t* P, hipStream_t s) {
    switch (type) {
    case T_Q8_0: return launch_qmv_t<T_Q8_0, true>(w, N, K, xq, rows, nullptr, P, s);
    case T_Q4_0: return launch_qmv_t<T_Q4_0, true>(w, N, K, xq, rows, nullptr, P, s);
    case T_Q4_K: return launch_qmv_t<T_Q4_K, true>(w, N, K, xq, rows, nullptr, P, s);
    case T_Q6_K: return launch_qmv_t<T_Q6_K, true>(w, N, K, xq, rows, nullptr, P, s);
    }
    return (int)hipErrorInvalidValue;
}

int launch_qmm(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
               int64_t rows, float* y, hipStream_t s) {
    return launch_qmv(type, w, N, K, xq, rows, y, s);
}

}  // namespace qmv
