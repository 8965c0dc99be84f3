// Kernels of the 256x256 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_256x256(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg256, true, Cfg256d>(p, g, cus, s) : launch<Cfg256, false, Cfg256d>(p, g, cus, s);
}

}  // namespace gemm_f16
