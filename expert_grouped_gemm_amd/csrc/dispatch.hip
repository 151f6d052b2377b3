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
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ tok_cnt, int T, int El,
                                                             int nblk, int cap,
                                                             int32_t* __restrict__ blk_counts,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tok_off,
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
  const int Tk = T * k;
  const int a0 = blockIdx.x * chunk;
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
    }
  }
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

}  // namespace

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
