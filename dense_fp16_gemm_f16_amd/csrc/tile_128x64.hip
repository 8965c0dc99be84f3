// Kernels of the 128x64 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_128x64(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg128x64, true, Cfg128x64d>(p, g, cus, s) : launch<Cfg128x64, false, Cfg128x64d>(p, g, cus, s);
}

}  // namespace gemm_f16
