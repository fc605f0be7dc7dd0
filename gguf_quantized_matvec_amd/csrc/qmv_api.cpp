// C-ABI of libqmv.so (declared in include/qmv.h): argument checks on the host,
// a device check, and dispatch to the kernels.  Nothing is allocated and
// nothing is synchronised; every check runs before any HIP call, so a refused
// call has no effect at all.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/qmv.h"
#include "qmv_internal.h"

namespace {

int elems_per_block(int type) {
    switch (type) {
    case QMV_Q8_0:
    case QMV_Q4_0:
    case QMV_Q5_0:
    case QMV_Q4_1:
    case QMV_Q5_1:
    case QMV_Q8_1: return 32;
    case QMV_Q4_K:
    case QMV_Q6_K: return 256;
    }
    return 0;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_weights(int type, const void* w, int64_t N, int64_t K) {
    const int qk = elems_per_block(type);
    if (!qk) return QMV_EINVAL_TYPE;
    if (N < 1 || N > INT32_MAX || K < 32 || K > QMV_MAX_K || K % qk) return QMV_EINVAL_SHAPE;
    if (!w || !aligned(w, 16)) return QMV_EINVAL_PTR;
    return QMV_OK;
}

// Cached per device: 1 = gfx950, 2 = something else.
std::atomic<int> g_dev_ok[64];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QMV_EUNSUPPORTED_DEVICE;
    if (dev < 64) {
        const int v = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (v) return v == 1 ? QMV_OK : QMV_EUNSUPPORTED_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QMV_EUNSUPPORTED_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? QMV_OK : QMV_EUNSUPPORTED_DEVICE;
}

int launched(int hip_rc) { return hip_rc == 0 ? QMV_OK : QMV_ELAUNCH; }

// Shared front half of qmv_launch / qmm_launch.
int matmul_common(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t rows,
                  int64_t max_rows, void* xq, float* y, void* stream, bool gemm) {
    int rc = check_weights(type, w, N, K);
    if (rc) return rc;
    if (rows < 1 || rows > max_rows) return QMV_EINVAL_SHAPE;
    if (!xq || !y || !aligned(xq, 16) || !aligned(y, 4)) return QMV_EINVAL_PTR;
    if (x && !aligned(x, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* q = static_cast<uint8_t*>(xq);
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    return launched(gemm ? qmv::launch_qmm(type, wb, N, K, x, q, rows, y, s)
                         : qmv::launch_qmv(type, wb, N, K, x, q, rows, y, s));
}

}  // namespace

extern "C" {

size_t qmv_act_bytes(int64_t rows, int64_t K) {
    if (rows < 1 || rows > QMV_MAX_M || K < 32 || K > QMV_MAX_K || K % 32) return 0;
    return (size_t)qmv::act_layout(rows, K).total;
}

int quantize_act_q8_0(const float* x, void* xq, int64_t rows, int64_t K, void* stream) {
    if (rows < 1 || rows > QMV_MAX_M || K < 32 || K > QMV_MAX_K || K % 32) return QMV_EINVAL_SHAPE;
    if (!xq || !aligned(xq, 16) || (x && !aligned(x, 4))) return QMV_EINVAL_PTR;
    const int rc = check_device();
    if (rc) return rc;
    uint8_t* q = static_cast<uint8_t*>(xq);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int st = qmv::staging_for(rows, K);
    return launched(x ? qmv::launch_quantize(x, q, rows, K, st, s)
                      : qmv::launch_rebuild(q, rows, K, st, s));
}

int qmv_launch(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t B,
               void* xq, float* y, void* stream) {
    return matmul_common(type, w, N, K, x, B, QMV_MAX_BATCH, xq, y, stream, false);
}

int qmv_launch_group(int type, int64_t B, const qmv_gemv* g, int count, void* stream) {
    if (!g) return QMV_EINVAL_PTR;
    if (count < 1 || count > QMV_MAX_GROUP || B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    const bool quantise = g[0].x != nullptr;
    qmv::GemvDesc d[QMV_MAX_GROUP];
    for (int k = 0; k < count; k++) {
        const int rc = check_weights(type, g[k].w, g[k].N, g[k].K);
        if (rc) return rc;
        if ((g[k].x != nullptr) != quantise) return QMV_EINVAL_PTR;
        if (!g[k].y || !aligned(g[k].y, 4)) return QMV_EINVAL_PTR;
        if (g[k].x && !aligned(g[k].x, 4)) return QMV_EINVAL_PTR;
        if (!g[k].x && !g[k].xq) return QMV_EINVAL_PTR;
        if (g[k].xq && !aligned(g[k].xq, 16)) return QMV_EINVAL_PTR;
        d[k] = qmv::GemvDesc{static_cast<const uint8_t*>(g[k].w), g[k].N, g[k].K, g[k].x,
                             static_cast<uint8_t*>(g[k].xq), g[k].y};
    }
    // xq may be left NULL only when the whole group (every entry's K and B)
    // runs as one fused launch and no entry's x needs a quantise launch of
    // its own (x not 16-byte aligned); every other path quantises into xq
    // first.  Decided for the whole group before anything is launched.
    bool any_null = false, any_unaligned = false;
    for (int k = 0; k < count; k++) {
        any_null |= g[k].xq == nullptr;
        any_unaligned |= g[k].x != nullptr && !aligned(g[k].x, 16);
    }
    if (any_null && (any_unaligned || !qmv::group_is_one_launch(d, count, B)))
        return QMV_EINVAL_PTR;
    const int rc = check_device();
    if (rc) return rc;
    return launched(qmv::launch_qmv_group(type, d, count, B, static_cast<hipStream_t>(stream)));
}

size_t qmv_gateup_act_bytes(int64_t B, int64_t N, int64_t K) {
    if (B < 1 || B > QMV_MAX_BATCH || N < 1 || N > INT32_MAX || K < 32 || K > QMV_MAX_K ||
        K % 32)
        return 0;
    return (size_t)qmv::gateup_act_bytes(B, N, K);
}

int qmv_launch_gateup_swiglu(int type, const void* w_gate, const void* w_up, int64_t N,
                             int64_t K, const float* x, int64_t B, void* xq, float* h,
                             void* stream) {
    int rc = check_weights(type, w_gate, N, K);
    if (rc) return rc;
    if ((rc = check_weights(type, w_up, N, K))) return rc;
    if (B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    if (!xq || !h || !aligned(xq, 16) || !aligned(h, 4)) return QMV_EINVAL_PTR;
    if (x && !aligned(x, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    return launched(qmv::launch_gateup(type, static_cast<const uint8_t*>(w_gate),
                                       static_cast<const uint8_t*>(w_up), N, K, x,
                                       static_cast<uint8_t*>(xq), B, h,
                                       static_cast<hipStream_t>(stream)));
}

int qmv_launch_gateup_swiglu_q8(int type, const void* w_gate, const void* w_up, int64_t N,
                                int64_t K, const float* x, int64_t B, void* xq, float* h,
                                void* hq, void* stream) {
    int rc = check_weights(type, w_gate, N, K);
    if (rc) return rc;
    if ((rc = check_weights(type, w_up, N, K))) return rc;
    if (B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    // h is the next projection's activation: whole 32-element blocks
    if (N < 32 || N > QMV_MAX_K || N % 32) return QMV_EINVAL_SHAPE;
    if (!xq || !h || !hq || !aligned(xq, 16) || !aligned(h, 4) || !aligned(hq, 16))
        return QMV_EINVAL_PTR;
    if (x && !aligned(x, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    return launched(qmv::launch_gateup(type, static_cast<const uint8_t*>(w_gate),
                                       static_cast<const uint8_t*>(w_up), N, K, x,
                                       static_cast<uint8_t*>(xq), B, h,
                                       static_cast<hipStream_t>(stream),
                                       static_cast<uint8_t*>(hq)));
}

int qmm_launch(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t M,
               void* xq, float* y, void* stream) {
    return matmul_common(type, w, N, K, x, M, QMV_MAX_M, xq, y, stream, true);
}

int qmv_partials_launch(int type, const void* w, int64_t N, int64_t K, void* xq,
                        int64_t B, int32_t* P, void* stream) {
    int rc = check_weights(type, w, N, K);
    if (rc) return rc;
    if (B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    if (!xq || !P || !aligned(xq, 16) || !aligned(P, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    return launched(qmv::launch_partials(type, static_cast<const uint8_t*>(w), N, K,
                                         static_cast<uint8_t*>(xq), B, P,
                                         static_cast<hipStream_t>(stream)));
}

int qmm_partials_launch(int type, const void* w, int64_t N, int64_t K, void* xq,
                        int64_t M, int32_t* P, void* stream) {
    int rc = check_weights(type, w, N, K);
    if (rc) return rc;
    if (M < 1 || M > QMV_MAX_M) return QMV_EINVAL_SHAPE;
    if (!xq || !P || !aligned(xq, 16) || !aligned(P, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    return launched(qmv::launch_qmm_partials(type, static_cast<const uint8_t*>(w), N, K,
                                             static_cast<uint8_t*>(xq), M, P,
                                             static_cast<hipStream_t>(stream)));
}

size_t qmv_act_bytes_q8k(int64_t rows, int64_t K) {
    if (rows < 1 || rows > QMV_MAX_M || K < 256 || K > QMV_MAX_K || K % 256) return 0;
    return (size_t)qmv::act_layout_q8k(rows, K).total;
}

int quantize_act_q8_k(const float* x, void* xq, int64_t rows, int64_t K, void* stream) {
    if (rows < 1 || rows > QMV_MAX_M || K < 256 || K > QMV_MAX_K || K % 256) return QMV_EINVAL_SHAPE;
    if (!xq || !aligned(xq, 16) || (x && !aligned(x, 4))) return QMV_EINVAL_PTR;
    const int rc = check_device();
    if (rc) return rc;
    return launched(qmv::launch_quantize_q8k(x, static_cast<uint8_t*>(xq), rows, K,
                                             static_cast<hipStream_t>(stream)));
}

namespace {
// prepared: w is the repacked layout of qmv_prepare (checked like a blob:
// the type, the shape, a 16-byte aligned pointer).
int q8k_common(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t rows,
               int64_t max_rows, void* xq, float* y, int32_t* P, void* stream,
               bool prepared = false) {
    if (type != QMV_Q4_K && type != QMV_Q6_K) return QMV_EINVAL_TYPE;
    int rc = check_weights(type, w, N, K);
    if (rc) return rc;
    if (rows < 1 || rows > max_rows) return QMV_EINVAL_SHAPE;
    if (!xq || !aligned(xq, 16)) return QMV_EINVAL_PTR;
    if (P ? !aligned(P, 4) : (!y || !aligned(y, 4))) return QMV_EINVAL_PTR;
    if (x && !aligned(x, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    uint8_t* xb = static_cast<uint8_t*>(xq);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (prepared) return launched(qmv::launch_qmm_q8k_prepared(type, wb, N, K, x, xb, rows, y, P, s));
    return launched(qmv::launch_qmv_q8k(type, wb, N, K, x, xb, rows, y, P, s));
}
}  // namespace

size_t qmv_prepared_bytes(int type, int64_t N, int64_t K) {
    if (type != QMV_Q4_K && type != QMV_Q6_K) return 0;
    if (N < 1 || N > INT32_MAX || K < 256 || K > QMV_MAX_K || K % 256) return 0;
    return (size_t)qmv::prepared_bytes_q8k(type, N, K);
}

int qmv_prepare(int type, const void* w, int64_t N, int64_t K, void* wp, void* stream) {
    if (type != QMV_Q4_K && type != QMV_Q6_K) return QMV_EINVAL_TYPE;
    int rc = check_weights(type, w, N, K);
    if (rc) return rc;
    if (!wp || !aligned(wp, 16)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    return launched(qmv::launch_prepare_q8k(type, static_cast<const uint8_t*>(w), N, K,
                                            static_cast<uint8_t*>(wp),
                                            static_cast<hipStream_t>(stream)));
}

int qmm_launch_q8k_prepared(int type, const void* wp, int64_t N, int64_t K, const float* x,
                            int64_t M, void* xq, float* y, void* stream) {
    return q8k_common(type, wp, N, K, x, M, QMV_MAX_M, xq, y, nullptr, stream, true);
}

int qmm_partials_q8k_prepared_launch(int type, const void* wp, int64_t N, int64_t K, void* xq,
                                     int64_t M, int32_t* P, void* stream) {
    if (!P) return QMV_EINVAL_PTR;
    return q8k_common(type, wp, N, K, nullptr, M, QMV_MAX_M, xq, nullptr, P, stream, true);
}

int qmv_launch_q8k(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t B,
                   void* xq, float* y, void* stream) {
    return q8k_common(type, w, N, K, x, B, QMV_MAX_BATCH, xq, y, nullptr, stream);
}

int qmm_launch_q8k(int type, const void* w, int64_t N, int64_t K, const float* x, int64_t M,
                   void* xq, float* y, void* stream) {
    return q8k_common(type, w, N, K, x, M, QMV_MAX_M, xq, y, nullptr, stream);
}

int qmv_launch_group_q8k(int type, int64_t B, const qmv_gemv* g, int count, void* stream) {
    if (type != QMV_Q4_K && type != QMV_Q6_K) return QMV_EINVAL_TYPE;
    if (!g) return QMV_EINVAL_PTR;
    if (count < 1 || count > QMV_MAX_GROUP || B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    const bool quantise = g[0].x != nullptr;
    qmv::GemvDesc d[QMV_MAX_GROUP];
    for (int k = 0; k < count; k++) {
        const int rc = check_weights(type, g[k].w, g[k].N, g[k].K);
        if (rc) return rc;
        if ((g[k].x != nullptr) != quantise) return QMV_EINVAL_PTR;
        if (!g[k].y || !aligned(g[k].y, 4)) return QMV_EINVAL_PTR;
        if (g[k].x && !aligned(g[k].x, 4)) return QMV_EINVAL_PTR;
        if (!g[k].xq || !aligned(g[k].xq, 16)) return QMV_EINVAL_PTR;
        d[k] = qmv::GemvDesc{static_cast<const uint8_t*>(g[k].w), g[k].N, g[k].K, g[k].x,
                             static_cast<uint8_t*>(g[k].xq), g[k].y};
    }
    const int rc = check_device();
    if (rc) return rc;
    return launched(qmv::launch_group_q8k(type, d, count, B, static_cast<hipStream_t>(stream)));
}

int qmv_launch_gateup_swiglu_q8k(int type, const void* w_gate, const void* w_up, int64_t N,
                                 int64_t K, const float* x, int64_t B, void* xq, float* h,
                                 void* stream) {
    if (type != QMV_Q4_K && type != QMV_Q6_K) return QMV_EINVAL_TYPE;
    int rc = check_weights(type, w_gate, N, K);
    if (rc) return rc;
    if ((rc = check_weights(type, w_up, N, K))) return rc;
    if (B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    if (!xq || !h || !aligned(xq, 16) || !aligned(h, 4)) return QMV_EINVAL_PTR;
    if (x && !aligned(x, 4)) return QMV_EINVAL_PTR;
    if ((rc = check_device())) return rc;
    return launched(qmv::launch_gateup_q8k(type, static_cast<const uint8_t*>(w_gate),
                                           static_cast<const uint8_t*>(w_up), N, K, x,
                                           static_cast<uint8_t*>(xq), B, h,
                                           static_cast<hipStream_t>(stream)));
}

int qmv_partials_q8k_launch(int type, const void* w, int64_t N, int64_t K, void* xq,
                            int64_t M, int32_t* P, void* stream) {
    if (!P) return QMV_EINVAL_PTR;
    return q8k_common(type, w, N, K, nullptr, M, QMV_MAX_M, xq, nullptr, P, stream);
}

int qmv_launch_noalloc(int type, const void* w, int64_t N, int64_t K, const float* x,
                       int64_t B, float* y, void* stream) {
    int rc = check_weights(type, w, N, K);
    if (rc) return rc;
    if (B < 1 || B > QMV_MAX_BATCH) return QMV_EINVAL_SHAPE;
    if (!x || !y || !aligned(x, 4) || !aligned(y, 4)) return QMV_EINVAL_PTR;
    if ((size_t)qmv::act_layout(B, K).total > QMV_NOALLOC_MAX_ACT_BYTES) return QMV_ETOO_LARGE;
    if ((rc = check_device())) return rc;
    int err = 0;
    uint8_t* xq = qmv::noalloc_scratch(&err);
    if (!xq) return QMV_ELAUNCH;
    return launched(qmv::launch_qmv(type, static_cast<const uint8_t*>(w), N, K, x, xq, B, y,
                                    static_cast<hipStream_t>(stream)));
}

const char* qmv_strerror(int code) {
    switch (code) {
    case QMV_OK: return "ok";
    case QMV_EINVAL_TYPE:
        return "unsupported weight type: accepted are Q4_0 (2), Q4_1 (3), Q5_0 (6), Q5_1 (7), "
               "Q8_0 (8), Q8_1 (9), Q4_K (12), Q6_K (14)";
    case QMV_EINVAL_SHAPE:
        return "bad shape: need 1 <= N <= 2^31-1, 32 <= K <= 2^20 with K % 32 == 0 "
               "(K % 256 == 0 for Q4_K/Q6_K), 1 <= B <= 16 for qmv_launch (use qmm_launch "
               "for more rows), 1 <= M <= 2^24 for qmm_launch";
    case QMV_EINVAL_PTR:
        return "bad pointer: w and xq must be non-NULL, w and xq 16-byte aligned, x, y and P "
               "4-byte aligned (x may be NULL to use xq as staged; a group entry may leave xq "
               "NULL only when the group runs as one launch and its x is 16-byte aligned)";
    case QMV_ELAUNCH: return "HIP kernel launch failed";
    case QMV_EUNSUPPORTED_DEVICE: return "current device is not an MI355X (gfx950)";
    case QMV_ETOO_LARGE:
        return "too large for qmv_launch_noalloc: qmv_act_bytes(B, K) must be at most "
               "QMV_NOALLOC_MAX_ACT_BYTES (8 MiB; every K <= 65536 at B <= 16); use qmv_launch "
               "with a caller-supplied xq for larger shapes";
    }
    return "unknown status code";
}

}  // extern "C"
