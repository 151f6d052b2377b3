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
__device__ __forceinline__ void load8(const void* buf, size_t row, int d, int c, float (&v)[8]) {
  if constexpr (BF16_IN) {
    const uint4 u = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(buf) + row * d)[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(buf) + row * d) + 2 * c;
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16_IN>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ buf,
                                                      const int32_t* __restrict__ tok_off,
                                                      const float* __restrict__ comb_w, int T, int d, int cap,
                                                      uint16_t* __restrict__ Y, float* __restrict__ Y32) {
  const int vec = d >> 3;  // 8 columns per lane-step
  for (int q = blockIdx.x; q < T; q += gridDim.x) {
    const int p0 = tok_off[q], p1 = tok_off[q + 1];
    const bool ok = 0 <= p0 && p0 <= p1 && p1 <= cap;
    for (int c = threadIdx.x; c < vec; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = ok ? 0.0f : __builtin_nanf("");
      if (ok) {
        for (int p = p0; p < p1; ++p) {
          const float wgt = comb_w[p];
          float v[8];
          load8<BF16_IN>(buf, (size_t)p, d, c, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wgt, v[i], acc[i]);
        }
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
