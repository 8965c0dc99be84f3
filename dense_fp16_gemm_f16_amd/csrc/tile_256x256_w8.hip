// Kernels of the 256x256 8-wave block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_256x256_w8(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg256w8, true, Cfg256w8>(p, g, cus, s) : launch<Cfg256w8, false, Cfg256w8>(p, g, cus, s);
}

}  // namespace gemm_f16
