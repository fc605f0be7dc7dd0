// Record of the last stand-in launcher call (api_stubs.cpp).
#pragma once
#include <stdint.h>

#define QMV_NOALLOC_MAX_ACT_BYTES_STUB (8u << 20)

struct LastCall {
    int calls = 0;
    const char* what = "";
    int type = 0;
    int64_t N = 0, K = 0, rows = 0;
    const void* x = nullptr;
    const void* xq = nullptr;
    const void* y = nullptr;
    int group_count = 0;
    const void* hq = nullptr;
};
extern LastCall g_last;
