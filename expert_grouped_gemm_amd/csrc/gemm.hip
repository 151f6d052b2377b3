// Host side of the persistent grouped expert GEMM: persistent-grid size, tile
// shape choice, the planning kernel (row bands, readiness counters, expert
// waves) and the launch sequence of each schedule. The kernel itself is in
// gemm_device.h.
#include "gemm_device.h"
#include "plan_device.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int El, int cap, int N1,
                                                    int G, int wave_experts, int sort_bands, int Pmax,
                                                    int clear_bits, int32_t* __restrict__ blk_done,
                                                    int nblk_done, int32_t* __restrict__ band_expert,
                                                    int32_t* __restrict__ band_row0,
                                                    int32_t* __restrict__ band_rows, int32_t* __restrict__ l2_full,
                                                    int32_t* __restrict__ wave_band0, int32_t* __restrict__ meta) {
  plan_body(offsets, El, cap, N1, G, wave_experts, sort_bands, Pmax, clear_bits, blk_done, nblk_done, band_expert,
            band_row0, band_rows, l2_full, wave_band0, meta);
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

namespace {

// The GEMM launches' parameters for problem p on workspace ws (everything but
// the mode and the combine).
GemmParams gemm_params(const moe_problem_t& p, const Layout& L, char* ws, int G, const void* X_rows,
                       const float* X_perm_scale, const int32_t* row_dst, const void* W1, const void* W1_scale,
                       const void* W2, const void* W2_scale, void* combine_buf, int32_t* row_done,
                       int row_done_len) {
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  const bool w4 = p.dtype == MOE_DTYPE_W4A8_MXFP4;
  GemmParams P{};
  P.X = static_cast<const uint8_t*>(X_rows);
  P.W1 = static_cast<const uint8_t*>(W1);
  P.W2 = static_cast<const uint8_t*>(W2);
  P.H = reinterpret_cast<uint8_t*>(ws + L.pub.h);
  P.C = combine_buf;
  P.Xs = X_perm_scale;
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
  P.a_k = 1;
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
  return P;
}

// The GEMM launch(es) of the problem's schedule.
hipError_t launch_gemm_schedule(const moe_problem_t& p, GemmParams P, int G, hipStream_t s) {
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;
  const bool w4 = p.dtype == MOE_DTYPE_W4A8_MXFP4;
  const int sched = resolve_schedule(p);
  auto launch = [&](int mode) {
    P.mode = mode;
    return w4 ? launch_gemm_w4a8(P, G, s) : fp8 ? launch_gemm_fp8(P, G, s) : launch_gemm_bf16(P, G, s);
  };
  if (sched == MOE_SCHED_SEPARATE) {
    hipError_t e = launch(MODE_SEP_L1);
    if (e != hipSuccess) return e;
    return launch(MODE_SEP_L2);
  }
  return launch(sched == MOE_SCHED_EXPERT_WAVE ? MODE_WAVE : MODE_INTERLEAVED);
}

}  // namespace

hipError_t launch_expert_forward(const moe_problem_t& p, const Layout& L, char* ws, const void* X_perm,
                                 const float* X_perm_scale, const int32_t* offsets, const int32_t* row_dst,
                                 const void* W1, const void* W1_scale, const void* W2,
                                 const void* W2_scale, void* combine_buf, hipStream_t s, int32_t* row_done,
                                 int row_done_len, bool after_dispatch) {
  const int G = gemm_grid(p);
  if (G <= 0) return hipErrorInvalidDevice;
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;
  GemmParams P = gemm_params(p, L, ws, G, X_perm, X_perm_scale, row_dst, W1, W1_scale, W2, W2_scale, combine_buf,
                             row_done, row_done_len);
  // expert waves need expert-contiguous bands; the other schedules take them largest first
  const int sort_bands = resolve_schedule(p) == MOE_SCHED_EXPERT_WAVE ? 0 : 1;
  // a standalone call clears every error bit; after the dispatch of the same
  // call, only the GEMM's own
  const int clear_bits = after_dispatch ? (ARG_ERR_OFFSETS | ARG_ERR_ROW_DST) : ARG_ERR_ALL;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, L.E_l, L.cap, P.N1, G, p.wave_experts,
                     sort_bands, L.Pmax, clear_bits, P.blk_done, fp8 ? L.Pmax * (p.f / 128) : 0,
                     reinterpret_cast<int32_t*>(ws + L.band_expert), reinterpret_cast<int32_t*>(ws + L.band_row0),
                     reinterpret_cast<int32_t*>(ws + L.band_rows), P.l2_full,
                     reinterpret_cast<int32_t*>(ws + L.wave_band0), P.meta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm_schedule(p, P, G, s);
}

// moe_layer_forward's expert GEMMs: the fused dispatch kernel has already
// planned the row bands, and Linear-1 gathers each band's rows from X
// through row_src (assignment a is token a / k).
hipError_t launch_expert_forward_fused(const moe_problem_t& p, const Layout& L, char* ws, const void* X,
                                       const int32_t* row_src, const float* X_perm_scale, const int32_t* row_dst,
                                       const void* W1, const void* W1_scale, const void* W2, const void* W2_scale,
                                       void* combine_buf, hipStream_t s) {
  const int G = gemm_grid(p);
  if (G <= 0) return hipErrorInvalidDevice;
  GemmParams P = gemm_params(p, L, ws, G, X, X_perm_scale, row_dst, W1, W1_scale, W2, W2_scale, combine_buf,
                             nullptr, 0);
  P.a_src = row_src;
  P.a_k = p.k;
  return launch_gemm_schedule(p, P, G, s);
}

}  // namespace moe
