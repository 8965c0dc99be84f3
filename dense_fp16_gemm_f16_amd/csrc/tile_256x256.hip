// Kernels of the 256x256 block tile (see kernels.h).
#include "kernels.h"

namespace gemm_f16 {

hipError_t launch_256x256(bool nn, const Params &p, int g, int cus, hipStream_t s) {
    return nn ? launch<Cfg256, true, Cfg256d>(p, g, cus, s) : launch<Cfg256, false, Cfg256d>(p, g, cus, s);
}

}  // namespace gemm_f16

#ifdef GEMM_F16_TRACE
// The profiling build's access to this unit's trace words (the 256x256
// kernels').  Both copy synchronously on the current device; they return
// the hipError_t of the copy, or -1 for a size beyond the array.
extern "C" int gemm_f16_trace_read(void *host, size_t bytes) {
    if (bytes > sizeof(gemm_f16::gemm_trace)) return -1;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gemm_f16::gemm_trace), bytes, 0, hipMemcpyDeviceToHost);
}
extern "C" int gemm_f16_trace_clear() {
    static unsigned long long zeros[sizeof(gemm_f16::gemm_trace) / sizeof(unsigned long long)];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(gemm_f16::gemm_trace), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
}
#endif
