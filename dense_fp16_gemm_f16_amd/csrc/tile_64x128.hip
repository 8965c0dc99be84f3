// Kernels of the 64x128 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_64x128(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg64x128, true, Cfg64x128d>(p, g, cus, s) : launch<Cfg64x128, false, Cfg64x128d>(p, g, cus, s);
}

}  // namespace gemm_f16
