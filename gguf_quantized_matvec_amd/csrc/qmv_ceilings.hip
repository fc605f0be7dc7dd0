// Measurement kernels (libqmv_ceilings.so, include/qmv_ceilings.h): what this
// chip actually reaches on the three resources the multiply is bound by, so
// that the fractions reported against the vendor peaks can be read against
// measured ceilings too.  Not part of the product path.
//
//   * a streaming read of HBM (16-byte loads, every load of a wave issued
//     before any is used), plain and with the nontemporal hint that the
//     decode GEMVs put on their weight loads;
//   * loops of independent int8 and f16 MFMAs with operands in registers
//     (v_mfma_i32_32x32x32_i8, v_mfma_f32_32x32x16_f16);
//   * the prefill GEMM's scale epilogue alone: chains of f32 fma, one per
//     output and 32-element block.
//
// Built with the library's flags (no packed-fp32 instructions), so the fma
// rate is the one the GEMM's epilogue can use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmv_ceilings.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Workgroup b reads bytes [b*256*L*16, (b+1)*256*L*16): thread t loads the
// 16-byte pieces t, t+256, ..., t+(L-1)*256 (each load instruction of a wave
// covers 1 KB contiguously), all in flight together, then xors them into one
// word.  NT: the loads carry the nontemporal hint, as the weight loads of
// the decode GEMVs do.
template <int L, bool NT>
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ buf,
                                                     uint32_t* __restrict__ sink) {
    const uint4* p = buf + (size_t)blockIdx.x * 256 * L + threadIdx.x;
    v4u v[L];
#pragma unroll
    for (int i = 0; i < L; i++) {
        const v4u* q = reinterpret_cast<const v4u*>(p + 256 * i);
        v[i] = NT ? __builtin_nontemporal_load(q) : *q;
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < L; i++) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int L, bool NT>
int stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    const size_t per_block = 256 * L * 16;
    if (!buf || !sink || bytes < per_block || bytes % per_block ||
        (reinterpret_cast<uintptr_t>(buf) & 15) || bytes / per_block > 0x7fffffff)
        return -2;
    hipLaunchKernelGGL((k_stream_read<L, NT>), dim3((unsigned)(bytes / per_block)), dim3(256), 0,
                       stream, static_cast<const uint4*>(buf), sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Four independent accumulator chains per wave, so that issue, not the
// dependency between MFMAs, sets the rate.
__global__ __launch_bounds__(256) void k_mfma_i8(int32_t* __restrict__ out, int iters, int seed) {
    const v4i a = {seed + (int)threadIdx.x, 3, 5, 7};
    const v4i b = {11, seed, 13, 17};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; i++) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) s += c0[j] ^ c1[j] ^ c2[j] ^ c3[j];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_mfma_f16(float* __restrict__ out, int iters, int seed) {
    v8h a, b;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        a[j] = (_Float16)(float)((seed + j + (int)threadIdx.x) & 7);
        b[j] = (_Float16)(float)((seed + 3 * j) & 7);
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; i++) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) s += c0[j] + c1[j] + c2[j] + c3[j];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// 16 outputs per lane (a 32 x 32 MFMA tile's share), each taking one
// p = fma(I, s, p) per block, I and s changing every block as in the GEMM.
__global__ __launch_bounds__(256) void k_epilogue(float* __restrict__ out, int iters, float seed) {
    float p[16], I[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
        p[j] = 0.0f;
        I[j] = seed + (float)(j + (int)threadIdx.x);
    }
    float s = seed * 0.5f;
    for (int i = 0; i < iters; i++) {
#pragma unroll
        for (int j = 0; j < 16; j++) p[j] = fmaf(I[j], s, p[j]);
        s = s * 0.999f;  // one more VALU op per 16 fmas: the scale of the next block
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) r += p[j];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

// The decode GEMV's weight-load pattern alone: C lanes per row (one
// 16*NP-byte chunk each), floor(64/C) rows per wave, every chunk's 16-byte
// loads in flight together; each lane xors its words and stores only when the
// result is zero, so that the loads stay but hardly any bytes are written.
template <int NP>
__global__ __launch_bounds__(256) void k_chunk_read(const uint4* __restrict__ w, int64_t rows, int C,
                                                    uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int G = 64 / C, lrow = lane / C, c = lane - lrow * C;
    const int64_t row = wave * G + lrow;
    if (lrow >= G || row >= rows) return;
    const uint4* p = w + (row * C + c) * NP;
    v4u v[NP];
#pragma unroll
    for (int i = 0; i < NP; i++) v[i] = *reinterpret_cast<const v4u*>(p + i);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < NP; i++) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == 0) sink[wave * 64 + lane] = 1u;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int qmv_ceil_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    return stream_read<16, false>(buf, bytes, sink, static_cast<hipStream_t>(stream));
}
int qmv_ceil_stream_read_nt(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    return stream_read<8, true>(buf, bytes, sink, static_cast<hipStream_t>(stream));
}

int qmv_ceil_chunk_read(const void* w, int64_t rows, int64_t chunks, int64_t chunk_bytes,
                        uint32_t* sink, void* stream) {
    if (!w || !sink || (reinterpret_cast<uintptr_t>(w) & 15) || rows < 1 || chunks < 1 ||
        chunks > 64 || (chunk_bytes != 144 && chunk_bytes != 272))
        return -2;
    const int64_t G = 64 / chunks, waves = (rows + G - 1) / G, blocks = (waves + 3) / 4;
    if (blocks > 0x7fffffff) return -2;
    const uint4* p = static_cast<const uint4*>(w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (chunk_bytes == 144)
        hipLaunchKernelGGL(k_chunk_read<9>, dim3((unsigned)blocks), dim3(256), 0, s, p, rows,
                           (int)chunks, sink);
    else
        hipLaunchKernelGGL(k_chunk_read<17>, dim3((unsigned)blocks), dim3(256), 0, s, p, rows,
                           (int)chunks, sink);
    return launched();
}

int qmv_ceil_mfma_i8(int32_t* out, int blocks, int iters, void* stream) {
    if (!out || blocks < 1 || iters < 1) return -2;
    hipLaunchKernelGGL(k_mfma_i8, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out, iters, blocks);
    return launched();
}

int qmv_ceil_mfma_f16(float* out, int blocks, int iters, void* stream) {
    if (!out || blocks < 1 || iters < 1) return -2;
    hipLaunchKernelGGL(k_mfma_f16, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out, iters, blocks);
    return launched();
}

int qmv_ceil_epilogue(float* out, int blocks, int iters, void* stream) {
    if (!out || blocks < 1 || iters < 1) return -2;
    hipLaunchKernelGGL(k_epilogue, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out, iters, 1.0f + (float)(blocks & 7));
    return launched();
}

}  // extern "C"
