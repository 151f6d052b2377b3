// The persistent expert-GEMM kernel instantiated for e4m3 activations (fp32
// block scales) against MXFP4 weights (E2M1 codes with E8M0 block scales).
#include "gemm_device.h"

namespace moe {

hipError_t launch_gemm_w4a8(const GemmParams& P, int G, hipStream_t s) {
  hipLaunchKernelGGL(moe_gemm_kernel<OT_W4A8>, dim3(G), dim3(gemm_threads(true)), 0, s, P);
  return hipGetLastError();
}

const void* gemm_kernel_w4a8() { return reinterpret_cast<const void*>(moe_gemm_kernel<OT_W4A8>); }

}  // namespace moe
