// The persistent expert-GEMM kernel instantiated for bf16 operands.
#include "gemm_device.h"

namespace moe {

hipError_t launch_gemm_bf16(const GemmParams& P, int G, hipStream_t s) {
  hipLaunchKernelGGL(moe_gemm_kernel<false>, dim3(G), dim3(gemm_threads(false)), 0, s, P);
  return hipGetLastError();
}

const void* gemm_kernel_bf16() { return reinterpret_cast<const void*>(moe_gemm_kernel<false>); }

}  // namespace moe
