// The expert GEMM's planning step as a device function of one 1024-thread
// block: the planning kernel of moe_expert_forward runs it alone, the fused
// dispatch kernel of moe_layer_forward runs it after its scan.
#pragma once

#include "moe_internal.h"

namespace moe {

// Row bands from the per-expert offsets, zeroed l2_full counters, and the
// expert waves (fewest consecutive experts whose Linear-1 tiles reach the grid,
// or a fixed number of experts per wave).
// The offsets come from device memory the host never sees (a caller's, or
// the dispatch's): unless they are non-decreasing with 0 <= offsets[0] and
// offsets[E_l] <= cap, the plan has no band, so no tile runs and nothing is
// stored, and the error bit is set for moe_check_workspace.
__device__ __forceinline__ void plan_body(const int32_t* __restrict__ offsets, int El, int cap, int N1,
                                                    int G, int wave_experts, int sort_bands, int Pmax,
                                                    int clear_bits,
                                                    int32_t* __restrict__ blk_done,
                                                    int nblk_done, int32_t* __restrict__ band_expert,
                                                    int32_t* __restrict__ band_row0,
                                                    int32_t* __restrict__ band_rows, int32_t* __restrict__ l2_full,
                                                    int32_t* __restrict__ wave_band0, int32_t* __restrict__ meta) {
  __shared__ int start[1025];
  __shared__ int sh[64];
  for (int i = threadIdx.x; i < Pmax; i += blockDim.x) l2_full[i] = 0;
  for (int i = threadIdx.x; i < nblk_done; i += blockDim.x) blk_done[i] = 0;
  if (threadIdx.x == 0) {
    meta[META_ERR] = 0;  // the flag reports this call only
    meta[META_TRACE_N] = 0;
    __hip_atomic_fetch_and(meta + META_ARG_ERR, ~clear_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int e = threadIdx.x;
  int cnt = 0, nb = 0;
  bool bad = false;
  if (e < El) {
    const int lo = offsets[e], hi = offsets[e + 1];
    cnt = hi - lo;
    bad = cnt < 0 || (e == 0 && lo < 0) || (e == El - 1 && hi > cap);
    nb = (cnt + kBM - 1) / kBM;
  }
  if (__syncthreads_or(bad)) {
    if (threadIdx.x == 0) {
      meta[META_P] = 0;
      meta[META_A] = 0;
      meta[META_NWAVES] = 0;
      __hip_atomic_fetch_or(meta + META_ARG_ERR, (int)ARG_ERR_OFFSETS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  // block exclusive scan of nb
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = nb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < 16; ++i) { const int v = sh[i]; sh[i] = s; s += v; }
    sh[16] = s;
  }
  __syncthreads();
  const int first = sh[wv] + x - nb;
  __shared__ int row_off[1025];
  if (e < El) {
    start[e] = first;
    row_off[e] = offsets[e];
  }
  if (threadIdx.x == 0) {
    start[El] = sh[16];
    row_off[El] = offsets[El];
  }
  __syncthreads();
  // Band table. Band q (in expert order) belongs to the last expert whose
  // first band is <= q (binary search over start[]; experts without rows have
  // start[e] == start[e + 1] and are skipped). With sort_bands the table is
  // ordered by the band's 32-row blocks, largest first, stably: a static
  // round-robin over the tiles then gives every workgroup a similar mix of
  // tile sizes. The order of the bands changes no result, only which tiles
  // run together.
  const int Ptot = start[El];
  __shared__ int cls_base[9];
  if (threadIdx.x < 9) cls_base[threadIdx.x] = 0;
  __syncthreads();
  auto band_of = [&](int q, int& ex, int& r0, int& rows) {
    int lo = 0, hi = El - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= q) lo = mid;
      else hi = mid - 1;
    }
    const int i = q - start[lo];
    ex = lo;
    r0 = row_off[lo] + i * kBM;
    rows = min(kBM, row_off[lo + 1] - row_off[lo] - i * kBM);
  };
  if (sort_bands) {
    // class c = 8 - blocks (0: a full band); bases = exclusive sums over classes
    for (int q = threadIdx.x; q < Ptot; q += blockDim.x) {
      int ex, r0, rows;
      band_of(q, ex, r0, rows);
      atomicAdd(&cls_base[8 - ((rows + 31) >> 5)], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int s0 = 0;
      for (int c = 0; c < 9; ++c) { const int v = cls_base[c]; cls_base[c] = s0; s0 += v; }
    }
    __syncthreads();
  }
  for (int q0 = 0; q0 < Ptot; q0 += blockDim.x) {
    const int q = q0 + threadIdx.x;
    int ex = 0, r0 = 0, rows = 0, pos = q;
    if (q < Ptot) band_of(q, ex, r0, rows);
    if (sort_bands) {
      // stable rank among this chunk's bands of the same class: a ballot per
      // class in every wavefront, the per-wavefront counts exchanged once
      __shared__ int wave_cls[16][8];
      const int cls = q < Ptot ? 8 - ((rows + 31) >> 5) : 9;
      uint64_t mine = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint64_t bal = __ballot(cls == c);
        if (lane == c) wave_cls[wv][c] = __popcll(bal);
        if (cls == c) mine = bal;
      }
      __syncthreads();
      if (cls < 8) {
        int before = 0;
        for (int i = 0; i < wv; ++i) before += wave_cls[i][cls];
        pos = cls_base[cls] + before + __popcll(mine & ((1ull << lane) - 1ull));
      }
      __syncthreads();
      if (threadIdx.x < 8) {
        int total = 0;
        for (int i = 0; i < 16; ++i) total += wave_cls[i][threadIdx.x];
        cls_base[threadIdx.x] += total;
      }
      __syncthreads();
    }
    if (q < Ptot) {
      band_expert[pos] = ex | (row_off[ex + 1] - row_off[ex] <= kBM ? kBandSingle : 0);
      band_row0[pos] = r0;
      band_rows[pos] = rows;
    }
  }
  if (threadIdx.x == 0) {
    meta[META_P] = Ptot;
    meta[META_A] = offsets[El];
    int nw = 0, tiles = 0, e0 = 0;
    wave_band0[0] = 0;
    for (int ex = 0; ex < El; ++ex) {
      tiles += (start[ex + 1] - start[ex]) * N1;
      const bool close = wave_experts > 0 ? (ex + 1 - e0 >= wave_experts) : (tiles >= G);
      if (close || ex == El - 1) {
        wave_band0[++nw] = start[ex + 1];
        tiles = 0;
        e0 = ex + 1;
      }
    }
    meta[META_NWAVES] = nw;
  }
}


}  // namespace moe
