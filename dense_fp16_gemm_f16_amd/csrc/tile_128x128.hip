// Kernels of the 128x128 block tiles (see kernels.h): the default one
// (register-staged path on v_mfma_f32_32x32x16_f16) and the one on
// v_mfma_f32_16x16x32_f16 in every path (C = A B^T only).  Both share their
// direct-to-LDS kernels, which are instantiated once, here.
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_128x128(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg128, true, Cfg128d>(p, g, cus, s) : launch<Cfg128, false, Cfg128d>(p, g, cus, s);
}

hipError_t launch_128x128_m16(const Params &p, int g, int cus, hipStream_t s) {
    return launch<Cfg128m16, false>(p, g, cus, s);
}

}  // namespace gemm_f16
