// Top-k router: Cui et al., "Fine-grained Computation-Communication Overlap
// via Tile-level Signaling and Scheduling for MoE", Section 2.1 step (1)
// (per-token expert assignments and gate weights from a probability
// distribution, top-k kept); gate weights are the softmax over the k kept
// logits.
//
// One wavefront per token. Each lane holds ceil(E/64) logits (E <= 1024, so
// at most 16); lane l's slot i is expert l + 64 i. Selection runs k rounds:
// each lane proposes its largest untaken logit (the lowest slot among equal
// ones), a wave-wide fp32 max finds the round's value, and a wave-wide min
// over the expert index of the lanes that hold it breaks ties toward the
// lower expert. -0.0 compares equal to +0.0, so the two tie. Both wave
// reductions use in-row DPP moves and four lane reads, no LDS round trips.
// Memory traffic is one coalesced read of the logits row.
#include <limits.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block
constexpr int kRouteCountWaves = 8;  // wavefronts of the fused router's per-chunk block

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// Every lane's value combined over its 16-lane row (quad swaps, then the
// half-row and row mirrors), then the four rows through lane reads.
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, __int_as_float(dpp<0xB1>(__float_as_int(x))));   // quad_perm [1,0,3,2]
  x = fmaxf(x, __int_as_float(dpp<0x4E>(__float_as_int(x))));   // quad_perm [2,3,0,1]
  x = fmaxf(x, __int_as_float(dpp<0x141>(__float_as_int(x))));  // row_half_mirror
  x = fmaxf(x, __int_as_float(dpp<0x140>(__float_as_int(x))));  // row_mirror
  const int xi = __float_as_int(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(xi, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(xi, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(xi, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int wave_min_i32(int x) {
  x = min(x, dpp<0xB1>(x));
  x = min(x, dpp<0x4E>(x));
  x = min(x, dpp<0x141>(x));
  x = min(x, dpp<0x140>(x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Route token row `row` (E logits) with the whole wavefront: lane j < k
// ends with slot j's expert (*my_e) and gate weight (*my_w).
template <int PER>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane, int& my_e,
                                            float& my_w) {
  // PER = ceil(E / 64) logits per lane (1, 2, 4, 8 or 16): the selection
  // scans only the slots that exist
  float v[PER];
  uint32_t taken = 0;  // bit i: slot i of this lane already selected (or absent)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const bool present = e < E;
    v[i] = present ? row[e] : 0.0f;
    if (!present) taken |= 1u << i;
  }

  my_e = -1;  // lane j keeps slot j's expert and logit
  float my_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    float best = -__builtin_huge_valf();
    int best_i = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (!(taken & (1u << i)) && (best_i < 0 || v[i] > best)) {
        best = v[i];
        best_i = i;
      }
    const float vmax = wave_max_f32(best);
    const int e = wave_min_i32(best_i >= 0 && best == vmax ? lane + 64 * best_i : INT_MAX);
    if (lane == (e & 63)) taken |= 1u << (e >> 6);
    if (lane == j) {
      my_e = e;
      my_v = vmax;
    }
  }

  // softmax over the k selected logits, summed in slot order
  const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  const float ex = (lane < k) ? expf(my_v - m) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  my_w = ex / sum;
}

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ counts_global) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefronts: the DPP reductions need every lane
  int my_e;
  float my_w;
  route_token<PER>(logits + (size_t)t * E, E, k, lane, my_e, my_w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = my_w;
    if (counts_global) atomicAdd(&counts_global[my_e], 1);
  }
}

// moe_layer_forward's first launch: routing fused with the dispatch's count.
// Block b routes the tokens of dispatch chunk b (chunk / k tokens, one
// wavefront per token in turn) and counts their local assignments per
// expert in LDS (blk_counts[e][b]) and per output row (tok_cnt[q(t)]), as the
// dispatch's count kernel does from topk_idx. Block 0 also starts the call's
// device-side state: the error words and the next launch's scan-done flag.
template <int PER>
__global__ __launch_bounds__(512) void route_count_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int S, int chunk_tok, int e_begin, int El, int nblk,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          int32_t* __restrict__ blk_counts,
                                                          int32_t* __restrict__ tok_cnt,
                                                          int32_t* __restrict__ meta) {
  extern __shared__ int32_t hist[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) {
    meta[META_ERR] = 0;
    meta[META_ARG_ERR] = 0;
    meta[META_SCAN_DONE] = 0;
  }
  for (int e = threadIdx.x; e < El; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int t0 = b * chunk_tok, t1 = min(T, t0 + chunk_tok);
  for (int t = t0 + w; t < t1; t += kRouteCountWaves) {
    int my_e;
    float my_w;
    route_token<PER>(logits + (size_t)t * E, E, k, lane, my_e, my_w);
    const bool local = lane < k && (unsigned)(my_e - e_begin) < (unsigned)El;
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = my_w;
    }
    if (local) atomicAdd(&hist[my_e - e_begin], 1);
    const int c = __popcll(__ballot(local));
    if (lane == 0) tok_cnt[y_row_of_token(t, T, S)] = c;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += blockDim.x) blk_counts[(size_t)e * nblk + b] = hist[e];
}

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_route_count(const moe_problem_t& p, const Layout& L, const float* logits, int32_t* idx, float* w,
                              int32_t* blk_counts, int32_t* tok_cnt, int32_t* meta, hipStream_t s) {
  const int per = (p.E_global + 63) >> 6;  // E_global <= 1024 (validated)
  const int chunk_tok = L.chunk / p.k;      // the dispatch chunk is a whole number of tokens
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(L.nblk), dim3(64 * kRouteCountWaves), L.E_l * 4, s, logits, p.T, p.E_global, p.k,
                       p.num_segments, chunk_tok, p.e_begin, L.E_l, L.nblk, idx, w, blk_counts, tok_cnt, meta);
  };
  if (per <= 1) go(route_count_kernel<1>);
  else if (per <= 2) go(route_count_kernel<2>);
  else if (per <= 4) go(route_count_kernel<4>);
  else if (per <= 8) go(route_count_kernel<8>);
  else go(route_count_kernel<16>);
  return hipGetLastError();
}

hipError_t launch_route(const moe_problem_t& p, const float* logits, int32_t* idx, float* w,
                        int32_t* counts_global, hipStream_t s) {
  if (counts_global) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3((p.E_global + 255) / 256), dim3(256), 0, s, counts_global,
                       p.E_global);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = (p.T + kRouteWaves - 1) / kRouteWaves;
  const int per = (p.E_global + 63) >> 6;  // E_global <= 1024 (validated)
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * kRouteWaves), 0, s, logits, p.T, p.E_global, p.k, idx, w,
                       counts_global);
  };
  if (per <= 1) go(route_topk_kernel<1>);
  else if (per <= 2) go(route_topk_kernel<2>);
  else if (per <= 4) go(route_topk_kernel<4>);
  else if (per <= 8) go(route_topk_kernel<8>);
  else go(route_topk_kernel<16>);
  return hipGetLastError();
}

}  // namespace moe
