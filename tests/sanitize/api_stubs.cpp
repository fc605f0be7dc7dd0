// Host-only stand-ins for the kernel launchers of libqmv.so and for the two
// HIP device queries, so that the C-ABI layer (qmv_api.cpp) can be built with
// AddressSanitizer / UndefinedBehaviorSanitizer and driven on a machine
// without a GPU.  Each launcher records its arguments; nothing is launched.
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../gguf_quantized_matvec_amd/csrc/qmv_internal.h"
#include "api_stubs.h"

LastCall g_last;

static int record(const char* what, int type, int64_t N, int64_t K, int64_t rows, const void* x,
                  const void* xq, const void* y) {
    g_last.calls++;
    g_last.what = what;
    g_last.type = type;
    g_last.N = N;
    g_last.K = K;
    g_last.rows = rows;
    g_last.x = x;
    g_last.xq = xq;
    g_last.y = y;
    return 0;
}

extern "C" hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t* p, int) {
    memset(p, 0, sizeof(*p));
    strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
    return hipSuccess;
}

namespace qmv {
static uint8_t g_scratch[QMV_NOALLOC_MAX_ACT_BYTES_STUB];
uint8_t* noalloc_scratch(int* err) {
    *err = 0;
    return g_scratch;
}
int staging_for(int64_t rows, int64_t K) {
    if (rows > 16) return ST_F16;
    return rows <= 4 && K <= 16384 ? ST_ROW : ST_MFMA;
}
bool group_is_one_launch(const GemvDesc* d, int count, int64_t rows) {
    bool one = count >= 1 && count <= 8;
    for (int k = 0; k < count && one; k++)
        one = staging_for(rows, d[k].K) == ST_ROW && ((d[k].x != nullptr) == (d[0].x != nullptr));
    return one;
}
int launch_quantize(const float* x, uint8_t* xq, int64_t rows, int64_t K, int, hipStream_t) {
    return record("quantize", 0, 0, K, rows, x, xq, nullptr);
}
int launch_rebuild(uint8_t* xq, int64_t rows, int64_t K, int, hipStream_t) {
    return record("rebuild", 0, 0, K, rows, nullptr, xq, nullptr);
}
int launch_qmv(int type, const uint8_t*, int64_t N, int64_t K, const float* x, uint8_t* xq,
               int64_t rows, float* y, hipStream_t) {
    return record("qmv", type, N, K, rows, x, xq, y);
}
int launch_qmv_group(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t) {
    g_last.group_count = count;
    return record("group", type, d[0].N, d[0].K, rows, d[0].x, d[0].xq, d[0].y);
}
int launch_partials(int type, const uint8_t*, int64_t N, int64_t K, uint8_t* xq, int64_t rows,
                    int32_t* P, hipStream_t) {
    return record("partials", type, N, K, rows, nullptr, xq, P);
}
int launch_qmm_partials(int type, const uint8_t*, int64_t N, int64_t K, uint8_t* xq, int64_t M,
                        int32_t* P, hipStream_t) {
    return record("qmm_partials", type, N, K, M, nullptr, xq, P);
}
int launch_qmm(int type, const uint8_t*, int64_t N, int64_t K, const float* x, uint8_t* xq,
               int64_t rows, float* y, hipStream_t) {
    return record("qmm", type, N, K, rows, x, xq, y);
}
int launch_gateup(int type, const uint8_t*, const uint8_t*, int64_t N, int64_t K, const float* x,
                  uint8_t* xq, int64_t rows, float* h, hipStream_t, uint8_t* hq) {
    g_last.hq = hq;
    return record(hq ? "gateup_q8" : "gateup", type, N, K, rows, x, xq, h);
}
int launch_group_q8k(int type, const GemvDesc* d, int count, int64_t rows, hipStream_t) {
    g_last.group_count = count;
    return record("group_q8k", type, d[0].N, d[0].K, rows, d[0].x, d[0].xq, d[0].y);
}
int launch_gateup_q8k(int type, const uint8_t*, const uint8_t*, int64_t N, int64_t K,
                      const float* x, uint8_t* xq, int64_t rows, float* h, hipStream_t) {
    return record("gateup_q8k", type, N, K, rows, x, xq, h);
}
int launch_quantize_q8k(const float* x, uint8_t* xq, int64_t rows, int64_t K, hipStream_t) {
    return record("quantize_q8k", 0, 0, K, rows, x, xq, nullptr);
}
int launch_qmv_q8k(int type, const uint8_t*, int64_t N, int64_t K, const float* x, uint8_t* xq,
                   int64_t rows, float* y, int32_t* P, hipStream_t) {
    return record(P ? "partials_q8k" : "qmv_q8k", type, N, K, rows, x, xq, P ? (void*)P : (void*)y);
}
int launch_qmm_q8k_prepared(int type, const uint8_t*, int64_t N, int64_t K, const float* x,
                            uint8_t* xq, int64_t rows, float* y, int32_t* P, hipStream_t) {
    return record(P ? "partials_q8k_prepared" : "qmm_q8k_prepared", type, N, K, rows, x, xq,
                  P ? (void*)P : (void*)y);
}
int64_t prepared_bytes_q8k(int, int64_t N, int64_t K) { return (N + 31) / 32 * (K / 256) * 16896; }
int launch_prepare_q8k(int type, const uint8_t*, int64_t N, int64_t K, uint8_t* out, hipStream_t) {
    return record("prepare", type, N, K, 0, nullptr, out, nullptr);
}
}  // namespace qmv
