// Weighted combine: Cui et al., "Fine-grained Computation-Communication
// Overlap via Tile-level Signaling and Scheduling for MoE", Section 2.1 step
// (5) (the owner forms the gate-weighted sum of the returned expert outputs);
// X-Stage, Section 2.2 (Combine aggregates the top-k results with the router
// weights).
//
// Y[q] = sum_{p in [tok_off[q], tok_off[q+1])} comb_w[p] * combine_buf[p],
// in ascending slot order, fp32 fused multiply-add, rounded once to bf16.
// Deterministic: each output element is owned by one lane, no atomics.
// Streaming: every lane moves 8 contiguous columns per slot (32 bytes of
// fp32, or 16 of bf16 with a bf16 buffer) and stores 16 bytes of bf16; one
// workgroup per output row at a time.
// The slot range comes from device memory (a caller's tok_off): a range that
// does not lie inside [0, cap) gives a NaN row and reads nothing.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16_IN>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ buf,
                                                      const int32_t* __restrict__ tok_off,
                                                      const float* __restrict__ comb_w, int T, int d, int cap,
                                                      uint16_t* __restrict__ Y, float* __restrict__ Y32) {
  for (int q = blockIdx.x; q < T; q += gridDim.x)
    combine_row<BF16_IN>(buf, tok_off, comb_w, q, d, cap, Y, Y32, threadIdx.x, blockDim.x);
}

}  // namespace

hipError_t launch_combine(const moe_problem_t& p, const void* combine_buf, const int32_t* tok_off,
                          const float* comb_w, void* Y, float* Y_fp32, hipStream_t s) {
  const int blocks = p.T < 8192 ? p.T : 8192;
  const int cap = (int)row_capacity(p);
  if (p.flags & MOE_FLAG_BF16_COMBINE_BUF)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(256), 0, s, combine_buf, tok_off, comb_w, p.T, p.d,
                       cap, static_cast<uint16_t*>(Y), Y_fp32);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(256), 0, s, combine_buf, tok_off, comb_w, p.T,
                       p.d, cap, static_cast<uint16_t*>(Y), Y_fp32);
  return hipGetLastError();
}

}  // namespace moe
