// Host side of the persistent grouped expert GEMM: persistent-grid size, tile
// shape choice, the planning kernel (row bands, readiness counters, expert
// waves) and the launch sequence of each schedule. The kernel itself is in
// gemm_device.h.
#include "gemm_device.h"

namespace moe {
namespace {

// Row bands from the per-expert offsets, zeroed l2_full counters, and the
// expert waves (fewest consecutive experts whose Linear-1 tiles reach the grid,
// or a fixed number of experts per wave).
// The offsets come from device memory the host never sees (a caller's, or
// the dispatch's): unless they are non-decreasing with 0 <= offsets[0] and
// offsets[E_l] <= cap, the plan has no band, so no tile runs and nothing is
// stored, and the error bit is set for moe_check_workspace.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int El, int cap, int N1,
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
      band_expert[pos] = ex;
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

}  // namespace

int gemm_grid(const moe_problem_t& p) {
  static thread_local int cached_dev = -1;
  static thread_local int cached_grid = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_kernel_bf16(),
                                                     gemm_threads(false), 0) != hipSuccess)
      return 0;
    cached_grid = prop.multiProcessorCount * (occ > 0 ? occ : 1);
    cached_dev = dev;
  }
  int g = cached_grid;
  if (p.grid > 0 && p.grid < g) g = p.grid;  // never above the co-resident limit
  if (g > 1 && (g & 1)) --g;                  // pair instances need an even grid
  return g;
}

// Wide tiles (256 weight rows) by default: per weight byte they load half as
// many band rows, and per MFMA half as many LDS fragments, as narrow ones;
// they were measured faster on every workload shape, bandwidth-bound (one
// band per expert) and compute-bound alike. Linear-2 tiles need d % 256 == 0.
// The raster groups 4 row bands: the 32 tiles an XCD runs at once then share
// 4 bands and 8 weight tiles through its L2.
TileChoice choose_tiles(const moe_problem_t& p, const Layout&, int) {
  TileChoice c{4, 4, 4};
  if (p.flags & MOE_FLAG_TILE_NARROW) c.nnb1 = c.nnb2 = 2;
  if (p.d % 256) c.nnb2 = 2;
  if (p.flags & MOE_FLAG_BAND_MAJOR) c.group_m = 1;
  return c;
}

// MOE_SCHED_AUTO (X-Stage, Section 6.3). The wave and interleaved orders
// shape remote-store bursts; with the Linear-2 epilogue storing into local
// HBM there is no drain to shape (every ΔT_iss of X-Stage Eq. 14 is zero), and
// what they cost stays: a device-scope publish per Linear-1 tile, weight
// locality shared with the other Linear, and Linear-2 tiles left at the end.
// Per-tile spans and whole-layer rates on every workload shape put the two
// separate launches first, so AUTO is SEPARATE.
int resolve_schedule(const moe_problem_t& p) {
  return p.sched == MOE_SCHED_AUTO ? MOE_SCHED_SEPARATE : p.sched;
}

hipError_t launch_expert_forward(const moe_problem_t& p, const Layout& L, char* ws, const void* X_perm,
                                 const float* X_perm_scale, const int32_t* offsets, const int32_t* row_dst,
                                 const void* W1, const void* W1_scale, const void* W2,
                                 const void* W2_scale, void* combine_buf, hipStream_t s, int32_t* row_done,
                                 int row_done_len, bool after_dispatch) {
  const int G = gemm_grid(p);
  if (G <= 0) return hipErrorInvalidDevice;
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  const int sched = resolve_schedule(p);
  GemmParams P{};
  P.X = static_cast<const uint8_t*>(X_perm);
  P.W1 = static_cast<const uint8_t*>(W1);
  P.W2 = static_cast<const uint8_t*>(W2);
  P.H = reinterpret_cast<uint8_t*>(ws + L.pub.h);
  P.C = combine_buf;
  P.Xs = X_perm_scale;
  const bool w4 = p.dtype == MOE_DTYPE_W4A8_MXFP4;
  P.W1s = w4 ? nullptr : static_cast<const float*>(W1_scale);
  P.W2s = w4 ? nullptr : static_cast<const float*>(W2_scale);
  P.W1e = w4 ? static_cast<const uint8_t*>(W1_scale) : nullptr;
  P.W2e = w4 ? static_cast<const uint8_t*>(W2_scale) : nullptr;
  P.Hs = fp8 ? reinterpret_cast<float*>(ws + L.pub.h_scale) : nullptr;
  P.Hf = fp8 ? reinterpret_cast<float*>(ws + L.pub.h_f32) : nullptr;
  P.cap = L.cap;
  P.row_dst = row_dst;
  P.band_expert = reinterpret_cast<const int32_t*>(ws + L.band_expert);
  P.band_row0 = reinterpret_cast<const int32_t*>(ws + L.band_row0);
  P.band_rows = reinterpret_cast<const int32_t*>(ws + L.band_rows);
  P.l2_full = reinterpret_cast<int32_t*>(ws + L.l2_full);
  P.meta = reinterpret_cast<int32_t*>(ws + L.pub.meta);
  P.wave_band0 = reinterpret_cast<const int32_t*>(ws + L.wave_band0);
  P.d = p.d;
  P.f = p.f;
  const TileChoice tc = choose_tiles(p, L, G);
  P.nnb1 = tc.nnb1;
  P.nnb2 = tc.nnb2;
  P.group_m = tc.group_m;
  P.N1 = p.f / (32 * tc.nnb1);
  P.N2 = p.d / (64 * tc.nnb2);
  P.ready = fp8 ? p.f / 128 : P.N1;
  if (p.flags & MOE_FLAG_TEST_WAIT_TIMEOUT) P.ready = 0x7FFFFFFF;  // no band ever becomes ready
  P.blk_done = reinterpret_cast<int32_t*>(ws + L.blk_done);
  P.trace = L.pub.tile_trace_capacity ? reinterpret_cast<uint64_t*>(ws + L.pub.tile_trace) : nullptr;
  P.trace_cap = (int)L.pub.tile_trace_capacity;
  P.keep_hf = (p.flags & MOE_FLAG_KEEP_H_F32) ? 1 : 0;
  P.row_done = row_done;
  P.row_done_len = row_done_len;
  P.c_bf16 = (p.flags & MOE_FLAG_BF16_COMBINE_BUF) ? 1 : 0;
  // Anti-starvation knee (X-Stage Eq. 16): D = b_n K / (2 h) with b_n the weight
  // rows of a Linear-1 tile, K the participating workgroups and h = f, i.e.
  // the row bands one sweep of the grid covers (G / N1 here). The knee is a
  // lower bound that assumes every workgroup advances through Linear-1 at the
  // same pace. But a workgroup that takes a Linear-2 tile issues no Linear-1
  // tile for as long as that tile lasts, about f / d Linear-1 tiles of the
  // same width (the K extents are f and d), so the phase skew between
  // workgroups, and with it the lead, grows by that factor. Default lead:
  // max(knee, 8) * max(1, f / d), rounded up. Measured on the Mixtral shape
  // (f / d = 3.5): D = 8 left Linear-2 tiles waiting 41 us each on average
  // and the schedule 12% behind D = 32.
  int D = p.lead_D;
  if (D <= 0) {
    D = (G + P.N1 - 1) / P.N1;
    if (D < 8) D = 8;
    if (p.f > p.d) D = (int)(((int64_t)D * p.f + p.d - 1) / p.d);
  }
  P.lead_D = D;

  // expert waves need expert-contiguous bands; the other schedules take them largest first
  const int sort_bands = sched == MOE_SCHED_EXPERT_WAVE ? 0 : 1;
  // a standalone call clears every error bit; after the dispatch of the same
  // call, only the GEMM's own
  const int clear_bits = after_dispatch ? (ARG_ERR_OFFSETS | ARG_ERR_ROW_DST) : ARG_ERR_ALL;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, L.E_l, L.cap, P.N1, G, p.wave_experts,
                     sort_bands, L.Pmax, clear_bits,
                     P.blk_done, fp8 ? L.Pmax * (p.f / 128) : 0, reinterpret_cast<int32_t*>(ws + L.band_expert), reinterpret_cast<int32_t*>(ws + L.band_row0),
                     reinterpret_cast<int32_t*>(ws + L.band_rows), P.l2_full,
                     reinterpret_cast<int32_t*>(ws + L.wave_band0), P.meta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto launch = [&](int mode) {
    P.mode = mode;
    return w4 ? launch_gemm_w4a8(P, G, s) : fp8 ? launch_gemm_fp8(P, G, s) : launch_gemm_bf16(P, G, s);
  };
  if (sched == MOE_SCHED_SEPARATE) {
    if ((e = launch(MODE_SEP_L1)) != hipSuccess) return e;
    return launch(MODE_SEP_L2);
  }
  return launch(sched == MOE_SCHED_EXPERT_WAVE ? MODE_WAVE : MODE_INTERLEAVED);
}

}  // namespace moe
