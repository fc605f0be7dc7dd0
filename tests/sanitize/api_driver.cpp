// Drives every entry point of the C-ABI layer under ASan/UBSan with the
// stand-in launchers of api_stubs.cpp: refusals return the documented codes
// and launch nothing; accepted calls reach the right launcher with the
// caller's arguments.  Exit status 0 = every check held.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/qmv.h"
#include "api_stubs.h"

static int g_fail = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            g_fail = 1;                                                     \
        }                                                                   \
    } while (0)

alignas(256) static unsigned char W[1 << 16];
alignas(256) static float X[1 << 14];
alignas(256) static unsigned char XQ[1 << 16];
alignas(256) static float Y[1 << 14];

int main() {
    const int calls0 = g_last.calls;
    // refusals: nothing reaches a launcher
    CHECK(qmv_launch(4, W, 16, 32, X, 1, XQ, Y, nullptr) == QMV_EINVAL_TYPE);
    CHECK(qmv_launch(QMV_Q4_K, W, 16, 896, X, 1, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_launch(QMV_Q8_0, W + 8, 16, 32, X, 1, XQ, Y, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_launch(QMV_Q8_0, W, 16, 32, (float*)((char*)X + 2), 1, XQ, Y, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_launch(QMV_Q8_0, W, 16, 32, X, 17, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_launch(QMV_Q8_0, W, 0, 32, X, 1, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_launch(QMV_Q8_0, W, 16, (1 << 20) + 32, X, 1, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmm_launch(QMV_Q4_0, W, 16, 32, X, 0, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmm_launch(QMV_Q4_0, W, 16, 32, X, (1 << 24) + 1, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(quantize_act_q8_0(X, XQ, 1, 40, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(quantize_act_q8_0(X, XQ + 4, 1, 32, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_partials_launch(QMV_Q8_0, W, 16, 32, XQ, 17, (int32_t*)Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmm_partials_launch(QMV_Q8_0, W, 16, 32, XQ, 0, (int32_t*)Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_launch_noalloc(QMV_Q8_0, W, 16, 1 << 17, X, 16, Y, nullptr) == QMV_ETOO_LARGE);
    CHECK(qmv_launch_noalloc(QMV_Q8_0, W, 16, 32, nullptr, 1, Y, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_launch_gateup_swiglu(QMV_Q4_0, W, nullptr, 16, 32, X, 1, XQ, Y, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_launch_gateup_swiglu(QMV_Q4_0, W, W, 16, 32, X, 17, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    {
        qmv_gemv gv[9];
        for (auto& e : gv) e = qmv_gemv{W, 16, 32, X, XQ, Y};
        CHECK(qmv_launch_group(QMV_Q8_0, 1, gv, 0, nullptr) == QMV_EINVAL_SHAPE);
        CHECK(qmv_launch_group(QMV_Q8_0, 1, gv, 9, nullptr) == QMV_EINVAL_SHAPE);
        CHECK(qmv_launch_group(QMV_Q8_0, 1, nullptr, 1, nullptr) == QMV_EINVAL_PTR);
        gv[1].x = nullptr;  // x given for one entry only
        CHECK(qmv_launch_group(QMV_Q8_0, 1, gv, 2, nullptr) == QMV_EINVAL_PTR);
        gv[1].x = X;
        gv[0].xq = nullptr;  // NULL xq with a long-K entry: not one launch
        gv[1].K = 1 << 17;
        CHECK(qmv_launch_group(QMV_Q8_0, 1, gv, 2, nullptr) == QMV_EINVAL_PTR);
    }
    CHECK(qmv_launch_q8k(QMV_Q4_0, W, 16, 256, X, 1, XQ, Y, nullptr) == QMV_EINVAL_TYPE);
    CHECK(qmv_launch_q8k(QMV_Q4_K, W, 16, 512 + 32, X, 1, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_launch_q8k(QMV_Q6_K, W, 16, 256, X, 17, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmm_launch_q8k(QMV_Q6_K, W, 16, 256, X, 0, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmm_launch_q8k(QMV_Q6_K, W, 16, 256, X, 40, XQ + 4, Y, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_partials_q8k_launch(QMV_Q4_K, W, 16, 256, XQ, 3, nullptr, nullptr) == QMV_EINVAL_PTR);
    CHECK(quantize_act_q8_k(X, XQ, 1, 128, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_act_bytes_q8k(1, 128) == 0 && qmv_act_bytes_q8k(0, 256) == 0);
    CHECK(g_last.calls == calls0);

    // accepted calls reach the launcher with the caller's arguments
    CHECK(qmv_launch(QMV_Q4_K, W, 300, 4096, X, 3, XQ, Y, nullptr) == QMV_OK);
    CHECK(g_last.calls == calls0 + 1 && g_last.type == QMV_Q4_K && g_last.N == 300 &&
          g_last.K == 4096 && g_last.rows == 3 && g_last.x == X && g_last.xq == XQ && g_last.y == Y);
    // 4-byte aligned x is accepted (the library quantises it on its own)
    CHECK(qmv_launch(QMV_Q8_0, W, 16, 32, X + 1, 1, XQ, Y, nullptr) == QMV_OK);
    CHECK(qmm_launch(QMV_Q6_K, W, 64, 1024, nullptr, 2048, XQ, Y, nullptr) == QMV_OK);
    CHECK(!strcmp(g_last.what, "qmm") && g_last.rows == 2048 && g_last.x == nullptr);
    CHECK(quantize_act_q8_0(X, XQ, 5, 64, nullptr) == QMV_OK && !strcmp(g_last.what, "quantize"));
    CHECK(quantize_act_q8_0(nullptr, XQ, 5, 64, nullptr) == QMV_OK && !strcmp(g_last.what, "rebuild"));
    CHECK(qmv_partials_launch(QMV_Q4_1, W, 16, 64, XQ, 5, (int32_t*)Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "partials"));
    CHECK(qmm_partials_launch(QMV_Q4_1, W, 16, 64, XQ, 40, (int32_t*)Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "qmm_partials") && g_last.rows == 40);
    CHECK(qmv_launch_noalloc(QMV_Q5_0, W, 16, 4096, X, 16, Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "qmv") && g_last.xq != nullptr && g_last.xq != XQ);
    CHECK(qmv_launch_gateup_swiglu(QMV_Q4_0, W, W + 256, 48, 896, X, 2, XQ, Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "gateup") && g_last.N == 48 && g_last.rows == 2);
    CHECK(qmv_launch_gateup_swiglu_q8(QMV_Q4_K, W, W + 256, 64, 4096, X, 1, XQ, Y, XQ + 4096,
                                      nullptr) == QMV_OK &&
          !strcmp(g_last.what, "gateup_q8") && g_last.hq == XQ + 4096);
    CHECK(qmv_launch_gateup_swiglu_q8(QMV_Q4_K, W, W + 256, 48 + 8, 4096, X, 1, XQ, Y, XQ + 4096,
                                      nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmv_launch_gateup_swiglu_q8(QMV_Q4_K, W, W + 256, 64, 4096, X, 1, XQ, Y, nullptr,
                                      nullptr) == QMV_EINVAL_PTR);
    CHECK(qmv_launch_gateup_swiglu_q8k(QMV_Q6_K, W, W + 256, 40, 1024, X, 16, XQ, Y, nullptr) ==
              QMV_OK &&
          !strcmp(g_last.what, "gateup_q8k") && g_last.N == 40 && g_last.rows == 16 && g_last.y == Y);
    CHECK(qmv_launch_gateup_swiglu_q8k(QMV_Q4_0, W, W + 256, 40, 1024, X, 1, XQ, Y, nullptr) ==
          QMV_EINVAL_TYPE);
    CHECK(qmv_launch_gateup_swiglu_q8k(QMV_Q4_K, W, W + 256, 40, 1024 + 32, X, 1, XQ, Y, nullptr) ==
          QMV_EINVAL_SHAPE);
    {
        qmv_gemv gk[3] = {{W, 16, 1024, nullptr, XQ, Y}, {W, 24, 1024, nullptr, XQ, Y},
                          {W, 8, 1024, nullptr, XQ, Y}};
        CHECK(qmv_launch_group_q8k(QMV_Q4_K, 16, gk, 3, nullptr) == QMV_OK &&
              !strcmp(g_last.what, "group_q8k") && g_last.group_count == 3 && g_last.rows == 16);
        gk[1].xq = nullptr;
        CHECK(qmv_launch_group_q8k(QMV_Q4_K, 16, gk, 3, nullptr) == QMV_EINVAL_PTR);
    }
    {
        qmv_gemv gv[3] = {{W, 16, 32, X, XQ, Y}, {W, 24, 64, X, nullptr, Y}, {W, 8, 96, X, nullptr, Y}};
        CHECK(qmv_launch_group(QMV_Q8_0, 2, gv, 3, nullptr) == QMV_OK &&
              !strcmp(g_last.what, "group") && g_last.group_count == 3);
    }
    CHECK(qmm_launch_q8k(QMV_Q4_K, W, 48, 4096, X, 2048, XQ, Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "qmv_q8k") && g_last.rows == 2048 && g_last.x == X);
    CHECK(qmv_partials_q8k_launch(QMV_Q6_K, W, 48, 512, XQ, 7, (int32_t*)Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "partials_q8k") && g_last.x == nullptr);
    CHECK(quantize_act_q8_k(X, XQ, 3, 512, nullptr) == QMV_OK && !strcmp(g_last.what, "quantize_q8k"));
    CHECK(qmv_prepare(QMV_Q4_K, W, 33, 512, XQ, nullptr) == QMV_OK && !strcmp(g_last.what, "prepare") &&
          g_last.N == 33);
    CHECK(qmv_prepare(QMV_Q4_0, W, 33, 512, XQ, nullptr) == QMV_EINVAL_TYPE);
    CHECK(qmv_prepare(QMV_Q6_K, W, 33, 512, XQ + 8, nullptr) == QMV_EINVAL_PTR);
    CHECK(qmm_launch_q8k_prepared(QMV_Q6_K, W, 48, 512, X, 5, XQ, Y, nullptr) == QMV_OK &&
          !strcmp(g_last.what, "qmm_q8k_prepared") && g_last.rows == 5);
    CHECK(qmm_launch_q8k_prepared(QMV_Q6_K, W, 48, 500, X, 5, XQ, Y, nullptr) == QMV_EINVAL_SHAPE);
    CHECK(qmm_partials_q8k_prepared_launch(QMV_Q4_K, W, 48, 512, XQ, 9, (int32_t*)Y, nullptr) ==
              QMV_OK && !strcmp(g_last.what, "partials_q8k_prepared") && g_last.x == nullptr);
    CHECK(qmv_prepared_bytes(QMV_Q4_K, 33, 512) == 2 * 2 * 16896);
    CHECK(qmv_prepared_bytes(QMV_Q8_0, 33, 512) == 0 && qmv_prepared_bytes(QMV_Q6_K, 33, 500) == 0);
    // sizes
    CHECK(qmv_act_bytes(1, 896) == 24576);
    CHECK(qmv_act_bytes(0, 32) == 0 && qmv_act_bytes(1, 48) == 0);
    CHECK(qmv_gateup_act_bytes(1, 4864, 896) == 24576 + 2 * 19456);
    for (int code = -7; code <= 1; code++) CHECK(qmv_strerror(code) != nullptr);
    if (g_fail) return 1;
    printf("api checks ok\n");
    return 0;
}
