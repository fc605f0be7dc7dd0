// K-quant weights (Q4_K, Q6_K) x Q8_K activations on gfx950: the Q8_K
// quantiser and the prefill GEMM on int8 MFMA.
//
// Q8_K is the 8-bit format of the K-quant family ("Models and formats", the
// list of tensor formats): one f32 scale per 256 activations.  Against it,
// the integer sub-block scales of Q4_K / Q6_K fold into the integer partial
// of a whole superblock, so the f32 scaling runs once per 256 elements
// instead of once per 32 (include/qmv.h states the f32 order):
//   Q4_K: P = sum_j sc_j sum_k q a,  Q = sum_j m_j sum_k a
//   Q6_K: I = sum_j s_j sum_k (q - 32) a
//
// The GEMM keeps the whole superblock on the int8 matrix cores
// (v_mfma_i32_32x32x32_i8), exactly: each weight element's value sc*q
// (Q4_K, 0..945) or s*(q-32) (Q6_K, -4096..4064) is split into two int8
// digits, v = 64*hi + lo with lo in 0..63, and the superblock partial is
// ACC_lo + 64*ACC_hi of two int32 accumulators.  Q4_K's min term Q runs on
// the matrix cores too: the eight 32-code sums S_j of an activation row, split
// the same way, against the row's eight m_j, in one otherwise-zero MFMA per
// digit.  The VALU then does per superblock and output: P, (float)P, the
// scale product, one or two fma and the add in superblock order.
//
// Tiling: a workgroup of 4 waves owns 128 weight rows (32 per wave: lane l
// decodes row l%32's codes for its half of each 32-element block straight
// from the GGUF bytes into MFMA B operands) x 32*WM activation rows, staged
// per superblock in LDS (double buffered, one barrier per superblock); the
// next superblock's weight bytes and activation rows are loaded into
// registers while the current one is multiplied.
//
// Built with -ffp-contract=off: every float operation is the one written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int T_Q4_K = 12, T_Q6_K = 14;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef short s2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    const uint16_t u = (uint16_t)h;
    _Float16 f;
    __builtin_memcpy(&f, &u, 2);
    return (float)f;
}

// id = 1/d, or 0 when 1/d is not finite (the block quantises to zero codes)
__device__ __forceinline__ float inv_scale(float d) {
    const float r = 1.0f / d;
    return __builtin_isinf(r) ? 0.0f : r;
}

// ------------------------------------------------------------ quantise ----
// One wave per (row, superblock), 4 elements per lane: amax over the wave,
// d = amax/127, codes = round-half-away(x * id); the public Q8_K block and
// the row-major staging (codes, d per 32 codes, the two 16-code sums of each
// 32 codes, the digits of each 32-code sum), and for at most 16 rows the
// MFMA-order copy of the batched decode kernel.  FROM_PUBLIC: take codes and
// d from the Q8_K block in xq.
template <bool FROM_PUBLIC, bool A16>
__global__ __launch_bounds__(256) void k_quantize_q8k(const float* __restrict__ x,
                                                      uint8_t* __restrict__ xq, int64_t rows,
                                                      int64_t K, ActLayoutK L) {
    const int lane = threadIdx.x & 63;
    const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (task >= rows * L.nsb) return;  // uniform per wave
    const int64_t r = task / L.nsb, sb = task - r * L.nsb;
    uint8_t* pub = xq + task * 292;
    uint32_t c4 = 0;
    float d;
    if constexpr (!FROM_PUBLIC) {
        const float* xb = x + r * K + 256 * sb + 4 * lane;
        float v[4];
        if constexpr (A16) {
            const float4 f = *reinterpret_cast<const float4*>(xb);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) v[i] = xb[i];
        }
        float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        d = amax / 127.0f;
        const float id = inv_scale(d);
#pragma unroll
        for (int i = 0; i < 4; i++) c4 |= ((uint32_t)(int)roundf(v[i] * id) & 0xFFu) << (8 * i);
        if (lane == 0) *reinterpret_cast<float*>(pub) = d;
        *reinterpret_cast<uint32_t*>(pub + 4 + 4 * lane) = c4;
    } else {
        d = *reinterpret_cast<const float*>(pub);
        c4 = *reinterpret_cast<const uint32_t*>(pub + 4 + 4 * lane);
    }
    int s4 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) s4 += (int)(int8_t)(c4 >> (8 * i));
    int s16 = s4 + __shfl_xor(s4, 1);
    s16 += __shfl_xor(s16, 2);                   // sum of the lane's 16-code group
    const int s16b = __shfl_xor(s16, 4);         // the other group of its 32 codes
    if (!FROM_PUBLIC && (lane & 3) == 0)
        *reinterpret_cast<int16_t*>(pub + 260 + 2 * (lane >> 2)) = (int16_t)s16;
    *reinterpret_cast<uint32_t*>(xq + L.rcodes + r * K + 256 * sb + 4 * lane) = c4;
    if ((lane & 7) == 0) {
        const int64_t b = r * L.nb + 8 * sb + (lane >> 3);
        reinterpret_cast<float*>(xq + L.rda)[b] = d;
        reinterpret_cast<int32_t*>(xq + L.rs16)[b] =
            (int32_t)(((uint32_t)s16 & 0xFFFFu) | ((uint32_t)s16b << 16));
    }
    if ((lane & 7) == 0) {
        // the block's 32-code sum (|S| <= 4064) as two digits: block j's lo
        // at byte 8 (j / 4) + j % 4, its hi 4 bytes later
        const int j = lane >> 3, S = s16 + s16b;
        const uint8_t lo = (uint8_t)(S & 63), hi = (uint8_t)((S >> 6) & 0xFF);
        const int at = 8 * (j >> 2) + (j & 3);
        uint8_t* sd = xq + L.rsd + task * 16 + at;
        sd[0] = lo;
        sd[4] = hi;
        if (L.gsd) {
            uint8_t* gs = xq + L.gsd + sb * 256 + r * 16 + at;
            gs[0] = lo;
            gs[4] = hi;
        }
    }
    if (L.gcodes) {
        // element 4 lane + t is byte 8 kg + 4 (lane & 1) + t of block j:
        // j = lane / 8, kg = (lane % 8) / 2
        const int j = lane >> 3, kg = (lane & 7) >> 1;
        uint8_t* gb = xq + L.gcodes + sb * 4096;
        *reinterpret_cast<uint32_t*>(gb + (j >> 1) * 1024 + (r + 16 * kg) * 16 + (j & 1) * 8 +
                                     4 * (lane & 1)) = c4;
        if (lane == 0) reinterpret_cast<float*>(xq + L.gda)[sb * 16 + r] = d;
    }
}

// ---------------------------------------------------------------- GEMM ----
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes at a 2-byte aligned address (Q6_K superblocks are 210 bytes):
// the dwords from the 4-byte aligned address below it, shifted down.  The
// fifth dword is read only when p is not 4-byte aligned, so that no byte past
// p + 16 is touched (the last field of the blob's last superblock).
__device__ __forceinline__ uint4 ld16_a2(const uint8_t* p) {
    const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3);
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p - sh);
    uint32_t v[5];
    __builtin_memcpy(v, q, 16);
    v[4] = sh ? q[4] : 0u;
    return make_uint4(__builtin_amdgcn_alignbyte(v[1], v[0], sh),
                      __builtin_amdgcn_alignbyte(v[2], v[1], sh),
                      __builtin_amdgcn_alignbyte(v[3], v[2], sh),
                      __builtin_amdgcn_alignbyte(v[4], v[3], sh));
}

// The bytes of one superblock that one lane (weight row, half h of every
// 32-element block: elements 16h..16h+15) needs.
template <int FMT> struct WRawK;
template <> struct WRawK<T_Q4_K> {
    uint4 hdr;    // d, dmin, 12 scale bytes
    uint4 qs[4];  // qs[32c + 16h .. +16], c = 0..3 (blocks 2c, 2c+1: low, high nibbles)
};
template <> struct WRawK<T_Q6_K> {
    uint4 ql[4];  // ql[64hh + 32kk + 16h .. +16], index 2hh + kk
    uint4 qh[2];  // qh[32hh + 16h .. +16]
    uint4 sc;     // bytes 192..207: the 16 sub-scales
    uint32_t d;   // bytes 208, 209: fp16 d
};

template <int FMT>
__device__ __forceinline__ void fetch_wk(const uint8_t* sbp, int h, WRawK<FMT>& r) {
    if constexpr (FMT == T_Q4_K) {
        const uint4* p = reinterpret_cast<const uint4*>(sbp);  // 144-byte superblocks, 16-aligned
        r.hdr = p[0];
#pragma unroll
        for (int c = 0; c < 4; c++) r.qs[c] = p[1 + 2 * c + h];
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) r.ql[i] = ld16_a2(sbp + 64 * (i >> 1) + 32 * (i & 1) + 16 * h);
#pragma unroll
        for (int i = 0; i < 2; i++) r.qh[i] = ld16_a2(sbp + 128 + 32 * i + 16 * h);
        r.sc = ld16_a2(sbp + 192);
        uint16_t d16;
        __builtin_memcpy(&d16, sbp + 208, 2);
        r.d = d16;
    }
}

__device__ __forceinline__ uint32_t u4_at(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Q4_K: 6-bit scale and min of sub-block j from the 12 scale bytes.
__device__ __forceinline__ void q4k_sc_m(const uint4& hdr, int j, int& sc, int& mn) {
    auto byte = [&](int i) -> int { return (int)((u4_at(hdr, 1 + (i >> 2)) >> (8 * (i & 3))) & 0xFFu); };
    if (j < 4) {
        sc = byte(j) & 63;
        mn = byte(j + 4) & 63;
    } else {
        sc = (byte(j + 4) & 15) | ((byte(j - 4) >> 6) << 4);
        mn = (byte(j + 4) >> 4) | ((byte(j) >> 6) << 4);
    }
}

// Two int8 digits of 4 values v = f * c (c: 4 codes, one per byte, minus
// `off`; f the sub-block's integer scale): v = 64 hi + lo, lo in 0..63.
// Computed in 16-bit lanes (|v| <= 4096).
__device__ __forceinline__ void digits4(uint32_t codes, int off, int f, uint32_t& lo, uint32_t& hi) {
    const s2 vo = {(short)off, (short)off}, vf = {(short)f, (short)f};
    const s2 a = __builtin_bit_cast(s2, codes & 0x00FF00FFu) - vo;          // codes 0, 2
    const s2 b = __builtin_bit_cast(s2, (codes >> 8) & 0x00FF00FFu) - vo;   // codes 1, 3
    const s2 va = a * vf, vb = b * vf;
    const s2 m63 = {63, 63}, six = {6, 6};
    const uint32_t la = __builtin_bit_cast(uint32_t, (s2)(va & m63));
    const uint32_t lb = __builtin_bit_cast(uint32_t, (s2)(vb & m63));
    const uint32_t ha = __builtin_bit_cast(uint32_t, (s2)(va >> six)) & 0x00FF00FFu;
    const uint32_t hb = __builtin_bit_cast(uint32_t, (s2)(vb >> six)) & 0x00FF00FFu;
    lo = la | (lb << 8);
    hi = ha | (hb << 8);
}

// Digits of the lane's 16 weight values of block j (elements 16h..16h+15).
template <int FMT>
__device__ __forceinline__ void decode_block(const WRawK<FMT>& r, int j, int h, v4i& wlo, v4i& whi) {
    uint32_t codes[4];
    int f, off;
    if constexpr (FMT == T_Q4_K) {
        int mn;
        q4k_sc_m(r.hdr, j, f, mn);
        off = 0;
        const uint4 q = r.qs[j >> 1];
        const int sh = 4 * (j & 1);
#pragma unroll
        for (int i = 0; i < 4; i++) codes[i] = (u4_at(q, i) >> sh) & 0x0F0F0F0Fu;
    } else {
        const int hh = j >> 2, k = j & 3;
        const uint4 ql = r.ql[2 * hh + (k & 1)], qh = r.qh[hh];
        const int lsh = 4 * (k >> 1), hsh = 2 * k;
#pragma unroll
        for (int i = 0; i < 4; i++)
            codes[i] = ((u4_at(ql, i) >> lsh) & 0x0F0F0F0Fu) | (((u4_at(qh, i) >> hsh) & 0x03030303u) << 4);
        f = (int)(int8_t)((u4_at(r.sc, (2 * j + h) >> 2) >> (8 * ((2 * j + h) & 3))) & 0xFFu);
        off = 32;
    }
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; i++) digits4(codes[i], off, f, lo[i], hi[i]);
    wlo = (v4i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
    whi = (v4i){(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// LDS of one superblock step: the activation tile (TM rows x 256 code bytes
// as 16 pieces of 16 bytes; piece q of row r in slot 16 r + (q ^ (r & 15)),
// so that the lanes of one ds_read_b128 pass hit different banks), the rows'
// f32 scales and (Q4_K) the digits of their eight 32-code sums (16 bytes a
// row, as the quantiser leaves them).
// (d and sd are sized for every wave's copy instruction, whatever TM, so
// that each wave issues the same number of copies; slots past the tile's
// rows hold duplicates that are not read)
template <int TM> struct StageK {
    uint4 a[TM * 16];
    float d[256];
    uint4 sd[256];
};

// Load-time repacked weights (qmv_prepare): per 32-row tile and superblock a
// region of 16 digit slabs of 1 KB (slab 2j + g: digit g of block j; lane l's
// 16 bytes at 16 l, l = 32 h + row, i.e. exactly its MFMA B operand), then
// the 32 rows' 16-byte scale records (f32 d, f32 dmin, Q4_K's eight mins).
constexpr int PREP_REGION = 16896, PREP_REC = 16384;

// s_waitcnt with vmcnt = 17 (the repacked kernel's weight loads of one
// superblock: 16 digit slabs and a scale record), expcnt and lgkmcnt 0
constexpr int WAIT_VM17 = (1 << 14) | 1;

// WM: 32-row MFMA tiles per wave along M (the workgroup's 32*WM activation
// rows).  PART: write the exact superblock partials to P instead of y.
// PREP: w holds the repacked layout instead of the GGUF blob.
template <int FMT, int WM, bool PART, bool PREP>
__global__ __launch_bounds__(256, WM >= 4 ? 1 : 2) void k_gemm8k(const uint8_t* __restrict__ w, int64_t N,
                                                   int64_t K, const uint8_t* __restrict__ xq,
                                                   ActLayoutK L, int64_t M, int64_t tilesM,
                                                   int64_t tilesN, float* __restrict__ y, int64_t gm,
                                                   int32_t* __restrict__ P) {
    constexpr int TM = 32 * WM;
    // the two stages are separate LDS objects, so that reads of one are not
    // ordered behind the asynchronous copies into the other
    __shared__ StageK<TM> st0, st1;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 31, h = lane >> 5;
    // workgroup -> tile: XCD x (= blockIdx % 8) takes a contiguous range of
    // tiles in an order that runs through groups of gm M-tiles, M fastest
    // within a group, so that the workgroups resident on one XCD share a few
    // weight tiles and a bounded set of activation tiles through its L2
    // (with all M-tiles of the grid resident at once the activations did not
    // fit and were fetched again for every pair of weight tiles)
    int64_t tm, tn;
    {
        const int64_t nt = tilesM * tilesN, per = (nt + 7) >> 3, rem = nt & 7;
        const int64_t x8 = blockIdx.x & 7, k8 = blockIdx.x >> 3;
        const int64_t t = (rem == 0 || x8 < rem) ? x8 * per + k8
                                                 : rem * per + (x8 - rem) * (per - 1) + k8;
        const int64_t G = gm < tilesM ? gm : tilesM;
        const int64_t grp = t / (G * tilesN), i = t - grp * G * tilesN;
        const int64_t gr = tilesM - grp * G < G ? tilesM - grp * G : G;
        tm = grp * G + i % gr;
        tn = i / gr;
    }
    const int64_t m0 = tm * TM, n0 = tn * 128;
    const int nsb = (int)(K >> 8), nb = (int)(K >> 5);
    constexpr int SBB = FMT == T_Q4_K ? 144 : 210;
    const int64_t n = n0 + 32 * wv + lr;
    // direct: the lane's GGUF row; repacked: the wave's 32-row tile (the
    // last one for a wave wholly past N, whose outputs are not stored)
    const uint8_t* wrow;
    if constexpr (PREP) {
        const int64_t T = (N + 31) >> 5, tile = (n0 >> 5) + wv;
        wrow = w + (tile < T ? tile : T - 1) * nsb * PREP_REGION;
    } else {
        wrow = w + (n < N ? n : N - 1) * ((int64_t)nsb * SBB);
    }
    auto arow = [&](int row) -> int64_t { return m0 + row < M ? m0 + row : M - 1; };

    // asynchronous global -> LDS copy of superblock s into stage `dst`: each
    // wave instruction fills 64 consecutive 16-byte slots (4 tile rows); wave
    // wv fills rows [TM/4 wv, TM/4 (wv+1)); lane l of instruction i: slot
    // 16 r + u with r = TM/4 wv + 4i + l/16, u = l % 16, i.e. piece u ^ (r & 15)
    constexpr int RPW = TM / 4;  // tile rows per wave
    // copy sources: a base uniform over the workgroup (the tile's first
    // row) and 32-bit per-lane offsets (a tile's rows span < 2^27 bytes in
    // each staging array), which keeps one register per address
    const uint8_t* abase = xq + L.rcodes + m0 * K;
    const uint8_t* dbase = xq + L.rda + m0 * nb * 4;
    const uint8_t* sbase = xq + L.rsd + m0 * nsb * 16;
    uint32_t aoff[RPW / 4];
#pragma unroll
    for (int i = 0; i < RPW / 4; i++) {
        const int r = RPW * wv + 4 * i + (lane >> 4);
        aoff[i] = (uint32_t)((arow(r) - m0) * K + 16 * ((lane & 15) ^ (r & 15)));
    }
    const int drow = 64 * wv + lane;  // the row whose f32 scale this lane stages
    const uint32_t doff = (uint32_t)((arow(drow < TM ? drow : 0) - m0) * nb * 4);
    const uint32_t soff = (uint32_t)((arow(drow < TM ? drow : 0) - m0) * nsb * 16);
    // (the global operands are passed as plain void pointers: given as typed
    // pointer arithmetic, the host pass of this compiler drops the kernel)
    auto issue = [&](int s, StageK<TM>* __restrict__ dst) {
#pragma unroll
        for (int i = 0; i < RPW / 4; i++)
            __builtin_amdgcn_global_load_lds((const void*)(abase + (aoff[i] + 256u * s)),
                                             (lds_void*)&dst->a[16 * (RPW * wv + 4 * i)], 16, 0, 0);
        // the rows' f32 scales, one dword per lane (row 64 wv + lane)
        __builtin_amdgcn_global_load_lds((const void*)(dbase + (doff + 32u * s)), (lds_void*)&dst->d[64 * wv],
                                         4, 0, 0);
        if constexpr (FMT == T_Q4_K) {
            // the rows' sum digits, 16 bytes per row (row 64 wv + lane)
            __builtin_amdgcn_global_load_lds((const void*)(sbase + (soff + 16u * s)),
                                             (lds_void*)&dst->sd[64 * wv], 16, 0, 0);
        }
    };
    // the copies one issue() makes per wave, and an s_waitcnt that lets
    // exactly those stay in flight (expcnt and lgkmcnt not waited for)
    constexpr int NCOPY = RPW / 4 + 1 + (FMT == T_Q4_K ? 1 : 0);
    constexpr int WAIT_COPIES = NCOPY | (7 << 4) | (15 << 8);

    float yacc[WM][16];
#pragma unroll
    for (int t = 0; t < WM; t++)
#pragma unroll
        for (int e = 0; e < 16; e++) yacc[t][e] = 0.0f;
    const v16i zero16 = {};

    WRawK<FMT> wcur, wnext;   // direct: the raw bytes of this and the next superblock
    v4i wd[16];               // repacked: this superblock's digit slabs (refilled
    uint4 rec, recn;          // with the next one's as they are used), scale records
    auto slab = [&](int s, int i) -> v4i {
        return *reinterpret_cast<const v4i*>(wrow + (int64_t)s * PREP_REGION + 1024 * i + 16 * lane);
    };
    auto record = [&](int s) -> uint4 {
        return *reinterpret_cast<const uint4*>(wrow + (int64_t)s * PREP_REGION + PREP_REC + 16 * lr);
    };
    issue(0, &st0);
    if constexpr (PREP) {
#pragma unroll
        for (int i = 0; i < 16; i++) wd[i] = slab(0, i);
        rec = record(0);
    } else {
        fetch_wk<FMT>(wrow, h, wcur);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // one superblock on stage `cur` (the next one is copied into `nxt`)
    // (the stages as restrict pointers: once inlined, the LDS reads of `cur`
    // carry alias scopes that tell the wait-count pass they do not depend on
    // the asynchronous copies into `nxt`)
    auto step = [&](int s, StageK<TM>* __restrict__ cur, StageK<TM>* __restrict__ nxt) {
        // the next superblock (repacked: the last step copies and loads its
        // own again, into a stage that is not read any more: no branch, so
        // that the wait counts below stay exact)
        const int sn = s + 1 < nsb ? s + 1 : s;
        if (PREP || s + 1 < nsb) issue(sn, nxt);
        if constexpr (PREP) {
            // this superblock's weights (loaded during the previous step,
            // before these copies) have arrived; the copies stay in flight
            __builtin_amdgcn_s_waitcnt(WAIT_COPIES);
            // the 17 weight loads below are the wave's last vector-memory
            // operations of the step, after the copies
            __builtin_amdgcn_sched_barrier(0);
            recn = record(sn);
        } else if (s + 1 < nsb) {
            fetch_wk<FMT>(wrow + (int64_t)(s + 1) * SBB, h, wnext);
        }
        v16i alo[WM], ahi[WM];
#pragma unroll
        for (int t = 0; t < WM; t++) alo[t] = ahi[t] = zero16;
        // the activation operands of block j (tile t: rows 32 t + lr), read
        // from LDS one block ahead of their MFMAs (repacked: nothing else
        // hides the LDS latency)
        auto a_op = [&](int j, int t) -> v4i {
            const int r = 32 * t + lr;
            return __builtin_bit_cast(v4i, cur->a[16 * r + ((2 * j + h) ^ (r & 15))]);
        };
        v4i acur[WM];
#pragma unroll
        for (int t = 0; t < WM; t++) acur[t] = a_op(0, t);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            v4i wlo, whi;
            if constexpr (PREP) {
                wlo = wd[2 * j];
                whi = wd[2 * j + 1];
            } else {
                decode_block<FMT>(wcur, j, h, wlo, whi);
            }
            v4i anxt[WM];
#pragma unroll
            for (int t = 0; t < WM; t++) anxt[t] = a_op(j < 7 ? j + 1 : 7, t);
#pragma unroll
            for (int t = 0; t < WM; t++) {
                alo[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(acur[t], wlo, alo[t], 0, 0, 0);
                ahi[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(acur[t], whi, ahi[t], 0, 0, 0);
                acur[t] = anxt[t];
            }
            if constexpr (PREP) {
                wd[2 * j] = slab(sn, 2 * j);
                wd[2 * j + 1] = slab(sn, 2 * j + 1);
            }
        }
        float dw, dmw = 0.0f;
        v4i bm = {0, 0, 0, 0};
        if constexpr (PREP) {
            dw = __builtin_bit_cast(float, rec.x);
            dmw = __builtin_bit_cast(float, rec.y);
            bm = (v4i){(int)(h ? rec.w : rec.z), 0, 0, 0};
        } else if constexpr (FMT == T_Q4_K) {
            dw = half_bits_to_float(wcur.hdr.x & 0xFFFFu);
            dmw = half_bits_to_float(wcur.hdr.x >> 16);
            // Q4_K min term operands: m_j, j = 4h..4h+3, in bytes 0..3
            uint32_t mb = 0;
#pragma unroll
            for (int t2 = 0; t2 < 4; t2++) {
                int sc, mn;
                q4k_sc_m(wcur.hdr, 4 * h + t2, sc, mn);
                mb |= (uint32_t)mn << (8 * t2);
            }
            bm = (v4i){(int)mb, 0, 0, 0};
        } else {
            dw = half_bits_to_float(wcur.d);
        }
        // per tile: lane l, element e = activation row 32t + 8(e/4) + 4h +
        // e%4, weight row n (column lr)
#pragma unroll
        for (int t = 0; t < WM; t++) {
            int Qv[16];
            if constexpr (FMT == T_Q4_K) {
                // the row's 32-code sums S_j (j = 4h..4h+3) as two int8 digits
                // (from the quantiser) against m_j, in an otherwise-zero MFMA
                // per digit
                const uint2 sd2 = *reinterpret_cast<const uint2*>(
                    reinterpret_cast<const uint8_t*>(&cur->sd[32 * t + lr]) + 8 * h);
                const uint32_t slo = sd2.x, shi = sd2.y;
                const v16i ql = __builtin_amdgcn_mfma_i32_32x32x32_i8((v4i){(int)slo, 0, 0, 0}, bm, zero16, 0, 0, 0);
                const v16i qh = __builtin_amdgcn_mfma_i32_32x32x32_i8((v4i){(int)shi, 0, 0, 0}, bm, zero16, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; e++) Qv[e] = ql[e] + 64 * qh[e];
            }
            if constexpr (PART) {
                constexpr int per = FMT == T_Q4_K ? 2 : 1;
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int64_t m = m0 + 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
                    if (m < M && n < N) {
                        int32_t* o = P + ((m * N + n) * nsb + s) * per;
                        o[0] = alo[t][e] + 64 * ahi[t][e];
                        if constexpr (per == 2) o[1] = Qv[e];
                    }
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const float4 d4 = *reinterpret_cast<const float4*>(&cur->d[32 * t + 8 * g + 4 * h]);
                    const float da[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int e = 4 * g + i;
                        const int Pv = alo[t][e] + 64 * ahi[t][e];
                        float p = fmaf((float)Pv, dw * da[i], 0.0f);
                        if constexpr (FMT == T_Q4_K) p = fmaf(-(float)Qv[e], dmw * da[i], p);
                        yacc[t][e] = yacc[t][e] + p;
                    }
                }
            }
            // one tile's epilogue at a time: keeps the min-term MFMA results
            // of the other tiles from being held live at once
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (PREP) {
            rec = recn;
            // this wave's copies into `nxt` are complete (they precede the
            // 17 weight loads, which stay in flight), then every wave's; the
            // barrier is a plain s_barrier so that no wait for the weight
            // loads is added before it
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(WAIT_VM17);
            asm volatile("s_barrier" ::: "memory");
        } else {
            if (s + 1 < nsb) wcur = wnext;
            // this wave's copies into `nxt` are complete, then every wave's
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    };
    if constexpr (PREP) {
        // two straight-line steps per iteration, the odd one after the loop
        int s = 0;
        for (; s + 1 < nsb; s += 2) {
            step(s, &st0, &st1);
            step(s + 1, &st1, &st0);
        }
        if (s < nsb) step(s, &st0, &st1);
        __builtin_amdgcn_s_waitcnt(0);  // the last step's repeated copies and loads
    } else {
        for (int s = 0; s < nsb; s += 2) {
            step(s, &st0, &st1);
            if (s + 1 < nsb) step(s + 1, &st1, &st0);
        }
    }
    if constexpr (PART) return;
#pragma unroll
    for (int t = 0; t < WM; t++)
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int64_t m = m0 + 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
            if (m < M && n < N) y[m * N + n] = yacc[t][e];
        }
}

template <int FMT, int WM, bool PREP>
int launch_gemm8k_t(const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                    float* y, int32_t* P, hipStream_t s) {
    const ActLayoutK L = act_layout_q8k(M, K);
    const int64_t tilesM = (M + 32 * WM - 1) / (32 * WM), tilesN = (N + 127) / 128;
    const int64_t grid = tilesM * tilesN;
    if (grid > INT32_MAX) return (int)hipErrorInvalidValue;
    // M-tiles per group of the tile order (measured at M = 2048 on the
    // 8B-class shapes, weights from HBM: repacked 494-654 TOPS with every
    // M-tile in one group against 615-806 with 16; direct +5-8 % with 8)
    const int64_t gm = PREP ? 16 : 8;
    if (P)
        hipLaunchKernelGGL((k_gemm8k<FMT, WM, true, PREP>), dim3((unsigned)grid), dim3(256), 0, s,
                           w, N, K, xq, L, M, tilesM, tilesN, y, gm, P);
    else
        hipLaunchKernelGGL((k_gemm8k<FMT, WM, false, PREP>), dim3((unsigned)grid), dim3(256), 0, s,
                           w, N, K, xq, L, M, tilesM, tilesN, y, gm, P);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- repack ----
// One thread per (tile, superblock, block j, lane l = 32 h + row): the two
// digit slabs' 16 bytes of that lane, from the same decode as the direct
// GEMM; lanes j = 0 also write their row's scale record.  Rows past N: zero.
template <int FMT>
__global__ __launch_bounds__(256) void k_prepare_q8k(const uint8_t* __restrict__ w, int64_t N,
                                                     int64_t K, uint8_t* __restrict__ out,
                                                     int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int l = (int)(idx & 63), j = (int)((idx >> 6) & 7);
    const int64_t ts = idx >> 9, nsb = K >> 8;
    const int64_t t = ts / nsb, s = ts - t * nsb;
    const int r = l & 31, h = l >> 5;
    const int64_t n = 32 * t + r;
    uint8_t* reg = out + ts * PREP_REGION;
    v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    uint4 rc = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) {
        constexpr int SBB = FMT == T_Q4_K ? 144 : 210;
        const uint8_t* sbp = w + (n * nsb + s) * SBB;
        WRawK<FMT> raw;
        fetch_wk<FMT>(sbp, h, raw);
        decode_block<FMT>(raw, j, h, lo, hi);
        if constexpr (FMT == T_Q4_K) {
            rc.x = __builtin_bit_cast(uint32_t, half_bits_to_float(raw.hdr.x & 0xFFFFu));
            rc.y = __builtin_bit_cast(uint32_t, half_bits_to_float(raw.hdr.x >> 16));
            uint32_t m[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 8; k++) {
                int sc, mn;
                q4k_sc_m(raw.hdr, k, sc, mn);
                m[k >> 2] |= (uint32_t)mn << (8 * (k & 3));
            }
            rc.z = m[0];
            rc.w = m[1];
        } else {
            rc.x = __builtin_bit_cast(uint32_t, half_bits_to_float(raw.d));
        }
    }
    *reinterpret_cast<v4i*>(reg + 1024 * (2 * j) + 16 * l) = lo;
    *reinterpret_cast<v4i*>(reg + 1024 * (2 * j + 1) + 16 * l) = hi;
    if (j == 0 && h == 0) *reinterpret_cast<uint4*>(reg + PREP_REC + 16 * r) = rc;
}

}  // namespace

int launch_quantize_q8k(const float* x, uint8_t* xq, int64_t rows, int64_t K, hipStream_t s) {
    const ActLayoutK L = act_layout_q8k(rows, K);
    const int64_t tasks = rows * L.nsb;
    const unsigned blocks = (unsigned)((tasks + 3) / 4);
    if (!x)
        hipLaunchKernelGGL((k_quantize_q8k<true, true>), dim3(blocks), dim3(256), 0, s, x, xq, rows,
                           K, L);
    else if (aligned16(x))
        hipLaunchKernelGGL((k_quantize_q8k<false, true>), dim3(blocks), dim3(256), 0, s, x, xq,
                           rows, K, L);
    else
        hipLaunchKernelGGL((k_quantize_q8k<false, false>), dim3(blocks), dim3(256), 0, s, x, xq,
                           rows, K, L);
    return (int)hipGetLastError();
}

// Direct: Q6_K takes 128 activation rows per workgroup (4 MFMA tiles per
// wave: each decoded weight value feeds 4 MFMAs, one wave per SIMD) when that
// still gives the chip a few rounds of workgroups, else 64 or 32; Q4_K at most
// 64 (its decode and min-term MFMAs do not fit the registers of 4 tiles).
// Repacked (no decode to amortise): 64 rows, two waves per SIMD so that one
// wave's f32 epilogue overlaps the other's MFMAs, when that gives at least
// 256 workgroups; else 32.  (Measured on the 8B-class shapes at M = 512 and
// 2048: 128-row tiles were 10-45 % slower than 64 on every repacked shape.)
int launch_gemm_q8k(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
                    int64_t M, float* y, int32_t* P, bool prepared, hipStream_t s) {
    const int64_t tn = (N + 127) / 128;
    if (prepared) {
        const bool w2 = M > 32 && ((M + 63) / 64) * tn >= 256;
        switch (type) {
        case T_Q4_K: return w2 ? launch_gemm8k_t<T_Q4_K, 2, true>(w, N, K, xq, M, y, P, s)
                               : launch_gemm8k_t<T_Q4_K, 1, true>(w, N, K, xq, M, y, P, s);
        case T_Q6_K: return w2 ? launch_gemm8k_t<T_Q6_K, 2, true>(w, N, K, xq, M, y, P, s)
                               : launch_gemm8k_t<T_Q6_K, 1, true>(w, N, K, xq, M, y, P, s);
        }
        return (int)hipErrorInvalidValue;
    }
    const int wm = M <= 32 ? 1 : ((M + 127) / 128) * tn >= 512 ? 4 : 2;
    switch (type) {
    case T_Q4_K: return wm >= 2 ? launch_gemm8k_t<T_Q4_K, 2, false>(w, N, K, xq, M, y, P, s)
                                : launch_gemm8k_t<T_Q4_K, 1, false>(w, N, K, xq, M, y, P, s);
    case T_Q6_K: return wm == 4 ? launch_gemm8k_t<T_Q6_K, 4, false>(w, N, K, xq, M, y, P, s)
                      : wm == 2 ? launch_gemm8k_t<T_Q6_K, 2, false>(w, N, K, xq, M, y, P, s)
                                : launch_gemm8k_t<T_Q6_K, 1, false>(w, N, K, xq, M, y, P, s);
    }
    return (int)hipErrorInvalidValue;
}

int launch_qmm_q8k_prepared(int type, const uint8_t* wp, int64_t N, int64_t K, const float* x,
                            uint8_t* xq, int64_t rows, float* y, int32_t* P, hipStream_t s) {
    if (x || P) {
        const int rc = launch_quantize_q8k(x, xq, rows, K, s);
        if (rc) return rc;
    }
    return launch_gemm_q8k(type, wp, N, K, xq, rows, y, P, true, s);
}

int64_t prepared_bytes_q8k(int type, int64_t N, int64_t K) {
    return (N + 31) / 32 * (K / 256) * PREP_REGION;
}

int launch_prepare_q8k(int type, const uint8_t* w, int64_t N, int64_t K, uint8_t* out,
                       hipStream_t s) {
    const int64_t total = (N + 31) / 32 * (K / 256) * 512;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    if (type == T_Q4_K)
        hipLaunchKernelGGL(k_prepare_q8k<T_Q4_K>, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K,
                           out, total);
    else
        hipLaunchKernelGGL(k_prepare_q8k<T_Q6_K>, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K,
                           out, total);
    return (int)hipGetLastError();
}

}  // namespace qmv
