/*
 * qmv_ceilings.h — measurement kernels of libqmv_ceilings.so: the rates this
 * MI355X actually reaches on the resources the multiply of libqmv.so is bound
 * by (HBM reads for decode; int8 / f16 MFMA and the f32 scale epilogue for
 * prefill, which the llamay "Architecture" page's bench transcript reports
 * as the memory-bound and the arithmetic-bound phase).  Not part of the
 * product path; the caller times the launches on `stream`.
 *
 * Each call checks its arguments on the host (returns -2 and launches
 * nothing when one is bad), enqueues one kernel on `stream` (a hipStream_t)
 * and returns 0, or -4 when the launch fails.  All buffers are device memory
 * owned by the caller; nothing is allocated or synchronised.
 */
#ifndef QMV_CEILINGS_H
#define QMV_CEILINGS_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of buf (16-byte aligned; bytes a multiple of 65536) once with
 * 16-byte loads, one 64 KB slice per 256-thread workgroup with every load of
 * a thread in flight together; sink receives bytes/16/16 uint32 words. */
int qmv_ceil_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* As qmv_ceil_stream_read with the nontemporal hint on every load (the
 * cache policy of the decode GEMVs' weight loads) and 8 loads per thread:
 * one 32 KB slice per workgroup, bytes a multiple of 32768; sink receives
 * bytes/128 uint32 words. */
int qmv_ceil_stream_read_nt(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* The decode GEMV's weight-load pattern with nothing else: a blob of `rows`
 * rows of `chunks` chunks (1..64) of `chunk_bytes` bytes (144 or 272, the
 * 256-element chunks of Q4_K / Q4_0 and of Q8_0), w 16-byte aligned; each
 * lane loads one chunk whole (chunks lanes per row, 64 / chunks rows per
 * wave, workgroups of 4 waves).  sink receives at most 64 uint32 words per
 * wave (ceil(rows / (64 / chunks)) waves), and in practice none: a lane
 * stores only when the xor of its chunk's words is zero. */
int qmv_ceil_chunk_read(const void* w, int64_t rows, int64_t chunks, int64_t chunk_bytes,
                        uint32_t* sink, void* stream);

/* `blocks` workgroups of 4 waves, each wave issuing 4*iters
 * v_mfma_i32_32x32x32_i8 (65536 int8 operations each) in four independent
 * chains; out receives blocks*256 int32 words. */
int qmv_ceil_mfma_i8(int32_t* out, int blocks, int iters, void* stream);

/* As qmv_ceil_mfma_i8 with v_mfma_f32_32x32x16_f16 (32768 operations each);
 * out receives blocks*256 floats. */
int qmv_ceil_mfma_f16(float* out, int blocks, int iters, void* stream);

/* The prefill GEMM's scale epilogue alone: every thread runs 16 chains of
 * p = fma(I, s, p), iters steps each (16*iters fmas, one per output and
 * 32-element block); out receives blocks*256 floats. */
int qmv_ceil_epilogue(float* out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif
