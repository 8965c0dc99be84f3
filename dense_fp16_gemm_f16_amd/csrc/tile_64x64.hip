// Kernels of the 64x64 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_64x64(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg64, true, Cfg64d>(p, g, cus, s) : launch<Cfg64, false, Cfg64d>(p, g, cus, s);
}

}  // namespace gemm_f16
