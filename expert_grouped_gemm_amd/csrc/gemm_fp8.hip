// The persistent expert-GEMM kernel instantiated for fp8 (e4m3 codes with fp32 block scales) operands.
#include "gemm_device.h"

namespace moe {

hipError_t launch_gemm_fp8(const GemmParams& P, int G, hipStream_t s) {
  hipLaunchKernelGGL(moe_gemm_kernel<true>, dim3(G), dim3(gemm_threads(true)), 0, s, P);
  return hipGetLastError();
}

const void* gemm_kernel_fp8() { return reinterpret_cast<const void*>(moe_gemm_kernel<true>); }

}  // namespace moe
