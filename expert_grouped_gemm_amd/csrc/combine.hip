// Weighted combine: Cui et al., "Fine-grained Computation-Communication
// Overlap via Tile-level Signaling and Scheduling for MoE", Section 2.1 step
// (5) (the owner forms the gate-weighted sum of the returned expert outputs);
// X-Stage, Section 2.2 (Combine aggregates the top-k results with the router
// weights).
//
// Y[q] = sum_{p in [tok_off[q], tok_off[q+1])} comb_w[p] * combine_buf[p],
// in ascending slot order, fp32 fused multiply-add, rounded once to bf16.
// Deterministic: each output element is owned by one lane, no atomics.
// Streaming: every lane moves 32 contiguous bytes of fp32 per slot and
// stores 16 bytes of bf16; one workgroup per output row at a time.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ buf,
                                                      const int32_t* __restrict__ tok_off,
                                                      const float* __restrict__ comb_w, int T, int d,
                                                      uint16_t* __restrict__ Y, float* __restrict__ Y32) {
  const int vec = d >> 3;  // 8 columns per lane-step
  for (int q = blockIdx.x; q < T; q += gridDim.x) {
    const int p0 = tok_off[q], p1 = tok_off[q + 1];
    for (int c = threadIdx.x; c < vec; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      for (int p = p0; p < p1; ++p) {
        const float wgt = comb_w[p];
        const float4* src = reinterpret_cast<const float4*>(buf + (size_t)p * d) + 2 * c;
        const float4 u = src[0], v = src[1];
        acc[0] = fmaf(wgt, u.x, acc[0]);
        acc[1] = fmaf(wgt, u.y, acc[1]);
        acc[2] = fmaf(wgt, u.z, acc[2]);
        acc[3] = fmaf(wgt, u.w, acc[3]);
        acc[4] = fmaf(wgt, v.x, acc[4]);
        acc[5] = fmaf(wgt, v.y, acc[5]);
        acc[6] = fmaf(wgt, v.z, acc[6]);
        acc[7] = fmaf(wgt, v.w, acc[7]);
      }
      uint4 o;
      o.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
      o.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
      o.z = f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
      o.w = f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
      reinterpret_cast<uint4*>(Y + (size_t)q * d)[c] = o;
      if (Y32) {
        float4* dst = reinterpret_cast<float4*>(Y32 + (size_t)q * d) + 2 * c;
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_problem_t& p, const float* combine_buf, const int32_t* tok_off,
                          const float* comb_w, void* Y, float* Y_fp32, hipStream_t s) {
  const int blocks = p.T < 8192 ? p.T : 8192;
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, combine_buf, tok_off, comb_w, p.T, p.d,
                     static_cast<uint16_t*>(Y), Y_fp32);
  return hipGetLastError();
}

}  // namespace moe
