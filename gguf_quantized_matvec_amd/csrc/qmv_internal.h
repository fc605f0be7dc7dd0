// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libqmv.so.  Not part of the public interface (include/qmv.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

// Activation scratch `xq` for `rows` rows of K elements:
//   [0, pub)            Q8_0 blocks, row-major: fp16 d (LE) + 32 int8 codes
//   [priv0, ...)        private staging copy, in groups of 16 rows
//                       (G = ceil(rows/16); rows past `rows` are zero):
//     codes  [G][nb][64][8] int8   the 16x16x32 MFMA A-operand of block b:
//                                  lane l = m + 16*kg holds codes
//                                  a[16g+m][32b + 8kg .. 32b + 8kg + 7]
//     da     [G][nb][16] f32       f32 value of the fp16 block scale
//     ca     [G][nb][16] f32       da * S (exact in f32)
//     S      [G][nb][16] int32     sum of the block's 32 codes
struct ActLayout {
    int64_t nb, G, pub, priv0, codes, da, ca, S, total;
};

inline ActLayout act_layout(int64_t rows, int64_t K) {
    ActLayout L;
    L.nb = K / 32;
    L.G = (rows + 15) / 16;
    L.pub = rows * L.nb * 34;
    L.priv0 = (L.pub + 255) & ~int64_t(255);
    L.codes = L.priv0;
    L.da = L.codes + L.G * L.nb * 512;
    L.ca = L.da + L.G * L.nb * 64;
    L.S = L.ca + L.G * L.nb * 64;
    L.total = L.S + L.G * L.nb * 64;
    return L;
}

// Kernel launchers (qmv_kernels.hip).  Arguments are already validated.
// Each returns 0 or a hipError_t value.
int launch_quantize(const float* x, uint8_t* xq, int64_t rows, int64_t K, hipStream_t s);
int launch_rebuild(uint8_t* xq, int64_t rows, int64_t K, hipStream_t s);
int launch_qmv(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
               int64_t rows, float* y, hipStream_t s);
int launch_partials(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
                    int64_t rows, int32_t* P, hipStream_t s);
int launch_qmm(int type, const uint8_t* w, int64_t N, int64_t K, const uint8_t* xq,
               int64_t rows, float* y, hipStream_t s);

}  // namespace qmv
