// Dispatch of the local share as an on-GPU permutation: Cui et al., "Fine-
// grained Computation-Communication Overlap via Tile-level Signaling and
// Scheduling for MoE", Section 2.1 step (2) (tokens go to the experts that
// host them) and Section 3.2 (per-expert row layout built before the grouped
// GEMM); X-Stage, Section 2.2 (Dispatch precedes Linear-1).
//
// Assignment a = t*k + j is local when topk_idx[a] lies in [e_begin, e_end).
// Rows of one expert are ordered by ascending a (a stable counting sort), so
// the permutation is unique and needs no atomics:
//   1. count   : one wavefront per chunk of assignments (at most 512 chunks),
//                LDS histogram of local experts -> blk_counts[e][chunk]
//   2. scan    : one block; per-expert chunk prefixes, totals, offsets;
//                per-output-row local counts -> tok_off (exclusive scan)
//   3. scatter : one wavefront per chunk, walking its assignments in order;
//                the rank of an assignment among equal experts in a group of
//                64 comes from a ballot over lanes (a match-any loop), the
//                running base per expert from LDS.
//   4. gather  : X_perm[r] = X[row_src[r] / k], 16-byte lanes, coalesced.
#include "moe_internal.h"
#include "plan_device.h"

namespace moe {
namespace {

// Chunk b holds assignments [b*chunk, (b+1)*chunk); one wavefront per chunk,
// four chunks per 256-thread block, a private LDS histogram per wavefront.
// blk_counts is expert-major, [E_l][nblk], so that the scan's per-expert
// prefix reads contiguous memory.
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                             int S, int chunk, int e_begin, int El, int nblk,
                                                             int32_t* __restrict__ blk_counts,
                                                             int32_t* __restrict__ tok_cnt,
                                                             int32_t* __restrict__ meta) {
  const int Tk = T * k;
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // the error words report this call only
    meta[META_ERR] = 0;
    meta[META_ARG_ERR] = 0;
  }
  extern __shared__ int32_t hist_all[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + w;
  int32_t* hist = hist_all + w * El;
  for (int e = lane; e < El; e += 64) hist[e] = 0;
  __syncthreads();
  if (b < nblk) {
    const int a0 = b * chunk, a1 = min(Tk, a0 + chunk);
    for (int a = a0 + lane; a < a1; a += 64) {
      const int e = idx[a] - e_begin;
      if ((unsigned)e < (unsigned)El) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  if (b < nblk)
    for (int e = lane; e < El; e += 64) blk_counts[(size_t)e * nblk + b] = hist[e];
  // local slots of each token, stored at its output row q
  for (int t = blockIdx.x * 256 + threadIdx.x; t < T; t += gridDim.x * 256) {
    int c = 0;
    for (int j = 0; j < k; ++j) c += (unsigned)(idx[(size_t)t * k + j] - e_begin) < (unsigned)El;
    tok_cnt[y_row_of_token(t, T, S)] = c;
  }
}

// Exclusive scan over a 1024-thread block; returns the exclusive prefix of v
// and the block total in *total.
__device__ int block_exclusive_scan_1024(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  if (threadIdx.x < 16) {
    int s = sh[threadIdx.x];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(s, off, 16);
      if ((int)threadIdx.x >= off) s += y;
    }
    sh[16 + threadIdx.x] = s;  // inclusive over waves
  }
  __syncthreads();
  const int wave_base = wv ? sh[16 + wv - 1] : 0;
  *total = sh[16 + 15];
  const int r = wave_base + x - v;
  __syncthreads();
  return r;
}

// One block. (1) Per expert (one wavefront per expert, eight chunks per lane
// loaded together): exclusive prefix of its chunk counts, in place, and the
// expert total. (2) offsets = exclusive scan of the totals; A. (3) tok_off:
// exclusive scan of the local-slot counts of the output rows.
// A routing whose local assignments exceed the row capacity (a caller's
// topk_idx that lists an expert twice for one token) sets the capacity error
// bit and A = 0: the scatter then stores only what fits, the gather nothing,
// and the expert GEMM's own check of the offsets stops it.
__device__ __forceinline__ void scan_body(const int32_t* __restrict__ tok_cnt, int T, int El, int nblk, int cap,
                                          int32_t* __restrict__ blk_counts, int32_t* __restrict__ counts,
                                          int32_t* __restrict__ offsets, int32_t* __restrict__ tok_off,
                                          int32_t* __restrict__ meta) {
  __shared__ int sh[64];
  __shared__ int tot[1024];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Step 3's output-row counts of this wavefront's segment are loaded first,
  // into registers when they fit, so their latency overlaps step 1.
  constexpr int kRowRegs = 8;
  const int segw = ((T + 15) / 16 + 63) / 64 * 64;
  const int qa = min(T, w * segw), qb = min(T, qa + segw);
  const bool rows_in_regs = segw <= 64 * kRowRegs;
  int rc[kRowRegs];
#pragma unroll
  for (int u = 0; u < kRowRegs; ++u) {
    const int q = qa + u * 64 + lane;
    rc[u] = rows_in_regs && q < qb ? tok_cnt[q] : 0;
  }
  for (int e = w; e < El; e += 16) {
    int run = 0;
    for (int g0 = 0; g0 < nblk; g0 += 512) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = g0 + u * 64 + lane;
        v[u] = b < nblk ? blk_counts[(size_t)e * nblk + b] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int x = v[u];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        const int b = g0 + u * 64 + lane;
        if (b < nblk) blk_counts[(size_t)e * nblk + b] = run + x - v[u];
        run += __shfl(x, 63, 64);
      }
    }
    if (lane == 0) tot[e] = run;
  }
  __syncthreads();
  int A;
  const int e = threadIdx.x;
  const int off = block_exclusive_scan_1024(e < El ? tot[e] : 0, sh, &A);
  if (e < El) {
    counts[e] = tot[e];
    offsets[e] = off;
  }
  if (e == 0) {
    offsets[El] = A;
    meta[META_A] = A <= cap ? A : 0;
    if (A > cap)
      __hip_atomic_fetch_or(meta + META_ARG_ERR, (int)ARG_ERR_DISPATCH_CAP, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
  }
  // output rows: wavefront w owns a contiguous segment of q and reads it
  // 64 consecutive rows at a time (coalesced), or has it in registers;
  // segment totals are scanned across the 16 wavefronts in LDS.
  int wsum = 0;
  if (rows_in_regs) {
#pragma unroll
    for (int u = 0; u < kRowRegs; ++u) wsum += rc[u];
  } else {
#pragma unroll 4
    for (int q = qa + lane; q < qb; q += 64) wsum += tok_cnt[q];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
  if (lane == 0) sh[32 + w] = wsum;
  __syncthreads();
  int run = 0, total = 0;
  for (int i = 0; i < 16; ++i) {
    const int v = sh[32 + i];
    run += i < w ? v : 0;
    total += v;
  }
  if (rows_in_regs) {
#pragma unroll
    for (int u = 0; u < kRowRegs; ++u) {
      const int q = qa + u * 64 + lane;
      const int c = rc[u];
      int x = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (q < qb) tok_off[q] = run + x - c;
      run += __shfl(x, 63, 64);
    }
  } else {
#pragma unroll 4
    for (int q0 = qa; q0 < qb; q0 += 64) {
      const int q = q0 + lane;
      const int c = q < qb ? tok_cnt[q] : 0;
      int x = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (q < qb) tok_off[q] = run + x - c;
      run += __shfl(x, 63, 64);
    }
  }
  if (threadIdx.x == 0) tok_off[T] = total;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ tok_cnt, int T, int El,
                                                             int nblk, int cap, int32_t* __restrict__ blk_counts,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tok_off,
                                                             int32_t* __restrict__ meta) {
  scan_body(tok_cnt, T, El, nblk, cap, blk_counts, counts, offsets, tok_off, meta);
}

// One wavefront per chunk, walking its assignments in order, 64 at a time.
// A token's k experts are distinct, so within one expert the order is the
// order of the tokens; the rank of a lane among the lanes of its group that
// hold the same expert comes from a ballot (a match-any loop), the running
// base of each expert (offset + chunk prefix) from LDS.
// Chunk b of the assignments, walked by one wavefront (lane = 0..63) whose
// running[] (El ints of LDS) already holds each expert's base for the chunk.
// With X_scale set (the fused e4m3 path, where Linear-1 reads X itself), the
// wavefront also writes the gathered row scales X_perm_scale[c * cap + pos].
__device__ __forceinline__ void scatter_chunk(int b, int lane, int32_t* running, const int32_t* __restrict__ idx,
                                              const float* __restrict__ w, int T, int k, int S, int chunk,
                                              int e_begin, int El, int cap, const int32_t* __restrict__ tok_off,
                                              int32_t* __restrict__ row_src, int32_t* __restrict__ row_dst,
                                              float* __restrict__ comb_w, const float* __restrict__ X_scale,
                                              int dblocks, float* __restrict__ X_perm_scale) {
  const int Tk = T * k;
  const int a0 = b * chunk;
  const int a1 = min(Tk, a0 + chunk);
  int next = (a0 + lane < a1) ? idx[a0 + lane] : 0;
  for (int g = a0; g < a1; g += 64) {
    const int a = g + lane;
    const int e = (a < a1) ? next - e_begin : -1;
    if (g + 64 < a1) next = (a + 64 < a1) ? idx[a + 64] : 0;  // next group's experts, loaded early
    const bool local = (unsigned)e < (unsigned)El;
    uint64_t pending = __ballot(local);
    int pos = 0;
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int v = __shfl(e, leader, 64);
      const uint64_t same = __ballot(local && e == v);
      const int base = running[v];
      if (local && e == v) pos = base + __popcll(same & ((1ull << lane) - 1ull));
      if (lane == leader) running[v] = base + __popcll(same);
      pending &= ~same;
    }
    if (local) {
      const int t = a / k, j = a - t * k;
      int before = 0;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
        if (jj < j) before += (unsigned)(idx[(size_t)t * k + jj] - e_begin) < (unsigned)El;
      const int slot = tok_off[y_row_of_token(t, T, S)] + before;
      if (pos < cap) {  // only a routing past the capacity (reported by the scan) fails these
        row_src[pos] = a;
        row_dst[pos] = slot;
      }
      if (slot < cap) comb_w[slot] = w[a];
      if (X_scale && pos < cap)
        for (int c = 0; c < dblocks; ++c) X_perm_scale[(size_t)c * cap + pos] = X_scale[(size_t)(t >> 7) * dblocks + c];
    }
  }
}

// One wavefront per chunk, walking its assignments in order, 64 at a time.
// A token's k experts are distinct, so within one expert the order is the
// order of the tokens; the rank of a lane among the lanes of its group that
// hold the same expert comes from a ballot (a match-any loop), the running
// base of each expert (offset + chunk prefix) from LDS.
__global__ __launch_bounds__(64) void dispatch_scatter_kernel(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ w, int T, int k, int S,
                                                              int chunk, int e_begin, int El, int nblk, int cap,
                                                              const int32_t* __restrict__ blk_prefix,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ tok_off,
                                                              int32_t* __restrict__ row_src,
                                                              int32_t* __restrict__ row_dst,
                                                              float* __restrict__ comb_w) {
  extern __shared__ int32_t running[];
  const int lane = threadIdx.x;
  for (int e = lane; e < El; e += 64) running[e] = offsets[e] + blk_prefix[(size_t)e * nblk + blockIdx.x];
  __syncthreads();
  scatter_chunk(blockIdx.x, lane, running, idx, w, T, k, S, chunk, e_begin, El, cap, tok_off, row_src, row_dst,
                comb_w, nullptr, 0, nullptr);
}

// X_perm[r, :] = X[row_src[r] / k, :] for r < A; fp8 also gathers the row's
// block scales: X_perm_scale[c * cap + r] = X_scale[(t / 128) * (d / 128) + c].
__global__ __launch_bounds__(256) void dispatch_gather_kernel(const uint8_t* __restrict__ X,
                                                              const float* __restrict__ X_scale, int k,
                                                              int row_bytes, int dblocks, int cap,
                                                              const int32_t* __restrict__ row_src,
                                                              const int32_t* __restrict__ meta,
                                                              uint8_t* __restrict__ X_perm,
                                                              float* __restrict__ X_perm_scale) {
  const int A = meta[META_A];
  const int vecs = row_bytes >> 4;
  for (int r = blockIdx.x; r < A; r += gridDim.x) {
    const int t = row_src[r] / k;
    const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)t * row_bytes);
    uint4* dst = reinterpret_cast<uint4*>(X_perm + (size_t)r * row_bytes);
    for (int i = threadIdx.x; i < vecs; i += blockDim.x) dst[i] = src[i];
    if (X_scale) {
      for (int c = threadIdx.x; c < dblocks; c += blockDim.x)
        X_perm_scale[(size_t)c * cap + r] = X_scale[(size_t)(t >> 7) * dblocks + c];
    }
  }
}

struct FusedDispatch {
  const int32_t* idx;
  const float* w;
  int T, k, S, chunk, e_begin, El, nblk, cap;
  int32_t* blk_counts;
  const int32_t* tok_cnt;
  int32_t* counts;
  int32_t* offsets;
  int32_t* tok_off;
  int32_t* row_src;
  int32_t* row_dst;
  float* comb_w;
  const float* X_scale;  // e4m3 activations: their block scales, gathered per row into X_perm_scale
  int dblocks;
  float* X_perm_scale;
  int32_t* meta;
  // the expert GEMM's planning step
  int N1, G, wave_experts, sort_bands, Pmax, nblk_done;
  int32_t* blk_done;
  int32_t* band_expert;
  int32_t* band_row0;
  int32_t* band_rows;
  int32_t* l2_full;
  int32_t* wave_band0;
};

// moe_layer_forward's dispatch, one launch after the fused router: block 0
// runs the scan (per-expert chunk bases, counts, offsets, tok_off), raises
// meta[META_SCAN_DONE] with a device-scope release, then runs the expert
// GEMM's planning step (row bands, readiness counters); every other block
// waits for the flag (thread 0 polls, bounded; a timeout sets the error flag
// and the block stores nothing), acquires, and scatters 16 chunks, one per
// wavefront. Block 0 is dispatched first and waits for nothing, so the wait
// always ends. The router kernel cleared the flag.
__global__ __launch_bounds__(1024) void scan_plan_scatter_kernel(FusedDispatch F) {
  if (blockIdx.x == 0) {
    scan_body(F.tok_cnt, F.T, F.El, F.nblk, F.cap, F.blk_counts, F.counts, F.offsets, F.tok_off, F.meta);
    __syncthreads();  // (a workgroup barrier also orders the block's global stores before thread 0's release)
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(F.meta + META_SCAN_DONE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the scatter blocks run while this block plans the row bands
    plan_body(F.offsets, F.El, F.cap, F.N1, F.G, F.wave_experts, F.sort_bands, F.Pmax,
              ARG_ERR_OFFSETS | ARG_ERR_ROW_DST, F.blk_done, F.nblk_done, F.band_expert, F.band_row0, F.band_rows,
              F.l2_full, F.wave_band0, F.meta);
    return;
  }
  __shared__ int ok;
  if (threadIdx.x == 0) {
    int spins = 0, good = 1;
    while (__hip_atomic_load(F.meta + META_SCAN_DONE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(F.meta + META_ERR, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        good = 0;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ok = good;
  }
  __syncthreads();
  if (!ok) return;
  extern __shared__ int32_t running_all[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = (blockIdx.x - 1) * 16 + w;
  int32_t* running = running_all + w * F.El;
  if (b < F.nblk)
    for (int e = lane; e < F.El; e += 64) running[e] = F.offsets[e] + F.blk_counts[(size_t)e * F.nblk + b];
  __syncthreads();
  if (b < F.nblk)
    scatter_chunk(b, lane, running, F.idx, F.w, F.T, F.k, F.S, F.chunk, F.e_begin, F.El, F.cap, F.tok_off,
                  F.row_src, F.row_dst, F.comb_w, F.X_scale, F.dblocks, F.X_perm_scale);
}

}  // namespace

hipError_t launch_scan_plan_scatter(const moe_problem_t& p, const Layout& L, char* ws, const float* X_scale,
                                    const int32_t* idx, const float* w, int32_t* counts, int32_t* offsets,
                                    int32_t* row_src, int32_t* row_dst, int32_t* tok_off, float* comb_w,
                                    float* X_perm_scale, hipStream_t s) {
  const int G = gemm_grid(p);
  if (G <= 0) return hipErrorInvalidDevice;
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;
  const TileChoice tc = choose_tiles(p, L, G);
  FusedDispatch F{};
  F.idx = idx;
  F.w = w;
  F.T = p.T;
  F.k = p.k;
  F.S = p.num_segments;
  F.chunk = L.chunk;
  F.e_begin = p.e_begin;
  F.El = L.E_l;
  F.nblk = L.nblk;
  F.cap = L.cap;
  F.blk_counts = reinterpret_cast<int32_t*>(ws + L.blk_counts);
  F.tok_cnt = reinterpret_cast<const int32_t*>(ws + L.tok_cnt);
  F.counts = counts;
  F.offsets = offsets;
  F.tok_off = tok_off;
  F.row_src = row_src;
  F.row_dst = row_dst;
  F.comb_w = comb_w;
  F.X_scale = fp8 ? X_scale : nullptr;
  F.dblocks = p.d / 128;
  F.X_perm_scale = fp8 ? X_perm_scale : nullptr;
  F.meta = reinterpret_cast<int32_t*>(ws + L.pub.meta);
  F.N1 = p.f / (32 * tc.nnb1);
  F.G = G;
  F.wave_experts = p.wave_experts;
  F.sort_bands = resolve_schedule(p) == MOE_SCHED_EXPERT_WAVE ? 0 : 1;
  F.Pmax = L.Pmax;
  F.blk_done = reinterpret_cast<int32_t*>(ws + L.blk_done);
  F.nblk_done = fp8 ? L.Pmax * (p.f / 128) : 0;
  F.band_expert = reinterpret_cast<int32_t*>(ws + L.band_expert);
  F.band_row0 = reinterpret_cast<int32_t*>(ws + L.band_row0);
  F.band_rows = reinterpret_cast<int32_t*>(ws + L.band_rows);
  F.l2_full = reinterpret_cast<int32_t*>(ws + L.l2_full);
  F.wave_band0 = reinterpret_cast<int32_t*>(ws + L.wave_band0);
  const int blocks = 1 + (L.nblk + 15) / 16;
  hipLaunchKernelGGL(scan_plan_scatter_kernel, dim3(blocks), dim3(1024), 16 * L.E_l * 4, s, F);
  return hipGetLastError();
}

hipError_t launch_dispatch(const moe_problem_t& p, const Layout& L, const DispatchScratch& sc, const void* X,
                           const float* X_scale, const int32_t* idx, const float* w, int32_t* counts,
                           int32_t* offsets, int32_t* row_src, int32_t* row_dst, int32_t* tok_off,
                           float* comb_w, void* X_perm, float* X_perm_scale, hipStream_t s) {
  const int El = L.E_l;
  int32_t* blk = sc.blk_counts;
  int32_t* meta = sc.meta;
  int32_t* tok_cnt = sc.tok_cnt;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3((L.nblk + 3) / 4), dim3(256), 4 * El * 4, s, idx, p.T, p.k,
                     p.num_segments, L.chunk, p.e_begin, El, L.nblk, blk, tok_cnt, meta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, tok_cnt, p.T, El, L.nblk, L.cap, blk,
                     counts, offsets, tok_off, meta);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(L.nblk), dim3(64), El * 4, s, idx, w, p.T, p.k,
                     p.num_segments, L.chunk, p.e_begin, El, L.nblk, L.cap, blk, offsets, tok_off, row_src,
                     row_dst, comb_w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  const int row_bytes = p.d * (fp8 ? 1 : 2);
  const int blocks = L.cap < 8192 ? (L.cap > 0 ? L.cap : 1) : 8192;
  hipLaunchKernelGGL(dispatch_gather_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t*>(X),
                     fp8 ? X_scale : nullptr, p.k, row_bytes, p.d / 128, L.cap, row_src, meta,
                     static_cast<uint8_t*>(X_perm), X_perm_scale);
  return hipGetLastError();
}

}  // namespace moe
