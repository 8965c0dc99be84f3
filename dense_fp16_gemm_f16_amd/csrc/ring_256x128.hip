// The ring kernel's variants on the 256x128 block tile (see kernels.h): those
// whose ring fits (variants 1, 2, 3, 4, 5, 6), instantiated explicitly so that
// every one has its host-side launch stub.
#include "kernels.h"

namespace gemm_f16 {

template __global__ void gemm_f16_ring_kernel<Cfg256x128d, 64, 2, false>(const Params);
template __global__ void gemm_f16_ring_kernel<Cfg256x128d, 64, 3, false>(const Params);
template __global__ void gemm_f16_ring_kernel<Cfg256x128d, 32, 2, false>(const Params);
template __global__ void gemm_f16_ring_kernel<Cfg256x128d, 32, 3, false>(const Params);
template __global__ void gemm_f16_ring_kernel<Cfg256x128d, 32, 4, false>(const Params);
template __global__ void gemm_f16_ring_kernel<Cfg256x128d, 64, 2, true>(const Params);

hipError_t launch_ring_256x128(int variant, const Params &p, hipStream_t s) { return launch_ring<Cfg256x128d>(variant, p, s); }

}  // namespace gemm_f16
