// Kernels of the 128x256 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_128x256(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg128x256, true, Cfg128x256d>(p, g, cus, s) : launch<Cfg128x256, false, Cfg128x256d>(p, g, cus, s);
}

}  // namespace gemm_f16
