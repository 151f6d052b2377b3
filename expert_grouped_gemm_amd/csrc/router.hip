// Top-k router: Cui et al., "Fine-grained Computation-Communication Overlap
// via Tile-level Signaling and Scheduling for MoE", Section 2.1 step (1)
// (per-token expert assignments and gate weights from a probability
// distribution, top-k kept); gate weights are the softmax over the k kept
// logits.
//
// One wavefront per token. Each lane holds ceil(E/64) logits (E <= 1024, so
// at most 16). Selection runs k rounds of a wave-wide max over 64-bit keys
// (order-preserving fp32 bits << 32 | ~expert), so the larger logit wins and
// equal logits go to the lower expert index; -0.0 is folded into +0.0 first
// so that the two tie. Memory traffic is one coalesced read of the logits row.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;                       // -0.0 ties +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);          // monotone in v
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Inverse of the order-preserving map: the logit a key was built from.
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t y = __shfl_xor(x, off, 64);
    x = y > x ? y : x;
  }
  return x;
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ counts_global) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  constexpr int kMaxPer = 16;
  float v[kMaxPer];
  const int per = (E + 63) >> 6;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < per && e < E) ? row[e] : 0.0f;
  }
  uint32_t taken = 0;  // bit i: slot i of this lane already selected (or absent)
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i)
    if (!(i < per && lane + 64 * i < E)) taken |= 1u << i;

  int my_e = -1;       // lane j keeps slot j's expert and logit
  float my_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;  // below every finite key
    int best_i = -1;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (!(taken & (1u << i))) {
        const uint64_t key = route_key(v[i], lane + 64 * i);
        if (key > best) { best = key; best_i = i; }
      }
    }
    const uint64_t win = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)win);
    if (best_i >= 0 && best == win) taken |= 1u << best_i;  // unique winner: keys carry the index
    if (lane == j) {
      my_e = e;
      my_v = key_value(win);
    }
  }

  // softmax over the k selected logits, summed in slot order
  const float m = __shfl(my_v, 0, 64);
  const float ex = (lane < k) ? expf(my_v - m) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, j, 64);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = ex / sum;
    if (counts_global) atomicAdd(&counts_global[my_e], 1);
  }
}

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_route(const moe_problem_t& p, const float* logits, int32_t* idx, float* w,
                        int32_t* counts_global, hipStream_t s) {
  if (counts_global) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3((p.E_global + 255) / 256), dim3(256), 0, s, counts_global,
                       p.E_global);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = (p.T + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(64 * kRouteWaves), 0, s, logits, p.T, p.E_global,
                     p.k, idx, w, counts_global);
  return hipGetLastError();
}

}  // namespace moe
