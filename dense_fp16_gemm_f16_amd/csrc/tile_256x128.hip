// Kernels of the 256x128 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_256x128(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg256x128, true, Cfg256x128d>(p, g, cus, s) : launch<Cfg256x128, false, Cfg256x128d>(p, g, cus, s);
}

}  // namespace gemm_f16
