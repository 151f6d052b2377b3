// Internal declarations of the MI355X MoE library: workspace layout, tile
// constants and the kernel launchers each .hip file provides.
#pragma once

#include <vector>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_mi355x.h"

namespace moe {

// Grouped-GEMM tiling. A tile holds NNB * 64 weight rows, NNB = 2 (narrow) or
// 4 (wide): a Linear-1 tile covers NNB * 32 SwiGLU columns (as many gate rows
// plus as many up rows), a Linear-2 tile NNB * 64 output columns.
constexpr int kBM = 256;          // rows per row band (scheduler row)
// Threads of the expert-GEMM workgroup: 8 wavefronts, two per SIMD (256
// registers each), for both operand types. (fp8 with 4 wavefronts, one per
// SIMD, left the matrix unit idle while the only wavefront promoted each K
// block's partial sums: 8% slower on Linear-1, 10% on Linear-2.)
constexpr int gemm_threads(bool) { return 512; }
constexpr int kGemmLds = 160 * 1024;  // the whole LDS of a CU: one persistent workgroup per CU

constexpr int kMetaInts = 64;
enum MetaSlot {
  META_A = 0, META_P = 1, META_ERR = 2, META_NWAVES = 3, META_TRACE_N = 4, META_ARG_ERR = 5,
  // moe_layer_forward's fused dispatch kernel: the scan-done flag, cleared by
  // the router kernel that starts each call
  META_SCAN_DONE = 6
};
// Bits of meta[META_ARG_ERR]: device-side checks of arguments the host cannot
// see (they live in device memory). A call that uses a workspace clears the
// whole word when it starts (the workspace may hold anything before its first
// use); inside moe_layer_forward the expert GEMM clears only its own bits, so
// the dispatch's report survives until moe_check_workspace reads it.
enum ArgErr { ARG_ERR_DISPATCH_CAP = 1, ARG_ERR_OFFSETS = 2, ARG_ERR_ROW_DST = 4, ARG_ERR_ALL = 7 };

// band_expert[p] of the band table: the band's local expert, plus
// kBandSingle if the band is its expert's only one (the expert has at most
// kBM rows, so every weight byte of the expert is read by this band alone).
constexpr int32_t kBandSingle = 1 << 30;
constexpr int32_t kBandExpertMask = kBandSingle - 1;

enum GemmMode { MODE_SEP_L1 = 0, MODE_SEP_L2 = 1, MODE_WAVE = 2, MODE_INTERLEAVED = 3 };

// Spin limit of a Linear-2 tile waiting for its row's Linear-1 tiles (each
// probe sleeps ~0.05 us plus one memory round trip): well under a second.
constexpr int kSpinLimit = 1 << 19;

struct Layout {
  moe_workspace_layout_t pub;
  // internal
  size_t blk_counts;   // int32 [E_l, nblk]
  size_t tok_cnt;      // int32 [T] local slots per output row
  size_t band_expert;  // int32 [Pmax]
  size_t band_row0;    // int32 [Pmax]
  size_t band_rows;    // int32 [Pmax]
  size_t l2_full;      // int32 [Pmax]
  size_t wave_band0;   // int32 [E_l + 1]
  size_t blk_done;     // int32 [Pmax, f/128] (fp8 only)
  int cap, E_l, nblk, chunk, Pmax;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Dispatch chunk size in assignments: a whole number of tokens (k
// assignments each, so the fused router can count a chunk's tokens), at
// least 64 (one wavefront step), as small as possible while the [chunks, E_l]
// count matrix keeps at most 512 chunks and 2^20 entries.
inline int dispatch_chunk(int64_t Tk, int El, int k) {
  int64_t nmax = (1 << 20) / (El > 0 ? El : 1);
  if (nmax > 512) nmax = 512;
  if (nmax < 1) nmax = 1;
  int64_t per = (Tk + nmax - 1) / nmax;
  if (per < 64) per = 64;
  per = (per + k - 1) / k * k;
  return (int)per;
}

// Rows the workspace holds for the expert GEMM: every local assignment a
// routing can give (T * min(k, E_l)), or more for a padded row layout.
inline int64_t row_capacity(const moe_problem_t& p) {
  const int El = p.e_end - p.e_begin;
  const int64_t cap = (int64_t)p.T * (p.k < El ? p.k : El);
  return p.row_capacity > cap ? (int64_t)p.row_capacity : cap;
}

inline Layout make_layout(const moe_problem_t& p) {
  Layout L{};
  const int El = p.e_end - p.e_begin;
  const int64_t cap = row_capacity(p);
  const bool fp8 = p.dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  const size_t esz = fp8 ? 1 : 2;
  L.cap = (int)cap;
  L.E_l = El;
  L.chunk = dispatch_chunk((int64_t)p.T * p.k, El, p.k);
  L.nblk = (int)(((int64_t)p.T * p.k + L.chunk - 1) / L.chunk);
  L.Pmax = (int)((cap + kBM - 1) / kBM) + El;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.pub.meta = take(kMetaInts * 4);
  L.blk_counts = take((size_t)L.nblk * El * 4);
  L.tok_cnt = take((size_t)p.T * 4);
  L.band_expert = take((size_t)L.Pmax * 4);
  L.band_row0 = take((size_t)L.Pmax * 4);
  L.band_rows = take((size_t)L.Pmax * 4);
  L.l2_full = take((size_t)L.Pmax * 4);
  L.wave_band0 = take((size_t)(El + 1) * 4);
  L.blk_done = take(fp8 ? (size_t)L.Pmax * (p.f / 128) * 4 : 0);
  L.pub.topk_idx = take((size_t)p.T * p.k * 4);
  L.pub.topk_w = take((size_t)p.T * p.k * 4);
  L.pub.counts = take((size_t)El * 4);
  L.pub.offsets = take((size_t)(El + 1) * 4);
  L.pub.row_src = take(cap * 4);
  L.pub.row_dst = take(cap * 4);
  L.pub.tok_off = take((size_t)(p.T + 1) * 4);
  L.pub.comb_w = take(cap * 4);
  L.pub.x_perm = take(cap * p.d * esz);
  L.pub.x_perm_scale = take(fp8 ? cap * (p.d / 128) * 4 : 0);
  L.pub.h = take(cap * p.f * esz);
  L.pub.h_scale = take(fp8 ? cap * (p.f / 128) * 4 : 0);
  L.pub.combine_buf = take(cap * p.d * ((p.flags & MOE_FLAG_BF16_COMBINE_BUF) ? 2 : 4));
  L.pub.h_f32 = take(fp8 ? cap * p.f * 4 : 0);
  // a bound on the tiles of one call: every band at the narrow widths
  // (f / 64 Linear-1 tiles and d / 128 Linear-2 tiles)
  L.pub.tile_trace_capacity =
      (p.flags & MOE_FLAG_TILE_TRACE) ? (size_t)L.Pmax * (size_t)(p.f / 64 + p.d / 128) : 0;
  L.pub.tile_trace = take(L.pub.tile_trace_capacity * sizeof(moe_tile_record_t));
  L.pub.total = o;
  return L;
}

// Launchers (each returns the first HIP error, hipSuccess otherwise).
hipError_t launch_route(const moe_problem_t& p, const float* logits, int32_t* idx, float* w,
                        int32_t* counts_global, hipStream_t s);

// The dispatch's own scratch: per-(expert, chunk) counts [E_l, nblk], local
// slots per output row [T], and the meta words (A, error bits).
struct DispatchScratch {
  int32_t* blk_counts;
  int32_t* tok_cnt;
  int32_t* meta;
};
inline DispatchScratch dispatch_scratch(const Layout& L, char* ws) {
  return {reinterpret_cast<int32_t*>(ws + L.blk_counts), reinterpret_cast<int32_t*>(ws + L.tok_cnt),
          reinterpret_cast<int32_t*>(ws + L.pub.meta)};
}

hipError_t launch_dispatch(const moe_problem_t& p, const Layout& L, const DispatchScratch& sc, const void* X,
                           const float* X_scale, const int32_t* idx, const float* w, int32_t* counts,
                           int32_t* offsets, int32_t* row_src, int32_t* row_dst, int32_t* tok_off,
                           float* comb_w, void* X_perm, float* X_perm_scale, hipStream_t s);

hipError_t launch_expert_forward(const moe_problem_t& p, const Layout& L, char* ws, const void* X_perm,
                                 const float* X_perm_scale, const int32_t* offsets, const int32_t* row_dst,
                                 const void* W1, const void* W1_scale, const void* W2,
                                 const void* W2_scale, void* combine_buf, hipStream_t s,
                                 int32_t* row_done = nullptr, int row_done_len = 0, bool after_dispatch = false);

hipError_t launch_combine(const moe_problem_t& p, const void* combine_buf, const int32_t* tok_off,
                          const float* comb_w, void* Y, float* Y_fp32, hipStream_t s);

// moe_layer_forward's fused launches (route and dispatch counts; scan, band
// plan and scatter; the expert GEMMs with Linear-1 gathering its rows from X;
// then the combine kernel).
hipError_t launch_route_count(const moe_problem_t& p, const Layout& L, const float* logits, int32_t* idx, float* w,
                              int32_t* blk_counts, int32_t* tok_cnt, int32_t* meta, hipStream_t s);
hipError_t launch_scan_plan_scatter(const moe_problem_t& p, const Layout& L, char* ws, const float* X_scale,
                                    const int32_t* idx, const float* w, int32_t* counts, int32_t* offsets,
                                    int32_t* row_src, int32_t* row_dst, int32_t* tok_off, float* comb_w,
                                    float* X_perm_scale, hipStream_t s);
hipError_t launch_expert_forward_fused(const moe_problem_t& p, const Layout& L, char* ws, const void* X,
                                       const int32_t* row_src, const float* X_perm_scale, const int32_t* row_dst,
                                       const void* W1, const void* W1_scale, const void* W2, const void* W2_scale,
                                       void* combine_buf, hipStream_t s);

// Owner-aligned return path (validated arguments; see moe_owner_plan,
// moe_owner_gather and moe_segment_copy).
struct OwnerPlanSizes {
  int64_t R, bands, remote_bands, segments, recv_rows;
};
OwnerPlanSizes owner_plan_build(const moe_problem_t& p, const int32_t* idx, int local, int tb, int x,
                                std::vector<int32_t>& row_src, std::vector<int32_t>& expert_off,
                                std::vector<int32_t>& bands, std::vector<int32_t>& sched,
                                std::vector<int32_t>& segs, std::vector<int32_t>& recv_start);
hipError_t launch_owner_gather(const moe_problem_t& p, const void* X, const float* X_scale, const int32_t* row_src,
                               int R, void* X_pad, float* X_pad_scale, int cap, hipStream_t s);
hipError_t launch_segment_copy(const moe_problem_t& p, const float* O_pad, int R, const int32_t* segs, int n_seg,
                               float* recv, int R_recv, hipStream_t s);
hipError_t launch_segment_copy_wait(const moe_problem_t& p, const float* O_pad, int R, const int32_t* segs,
                                    int n_seg, float* recv, int R_recv, const int32_t* row_done, int32_t* err,
                                    int grid, hipStream_t s);

// Store-burst probe (validated arguments; see moe_store_burst_probe).
hipError_t launch_store_burst(int K, int B, int reps, double gap_us, void* buf, size_t buf_bytes, uint64_t* rec,
                              hipStream_t s);

// The schedule a problem runs (MOE_SCHED_AUTO resolved).
int resolve_schedule(const moe_problem_t& p);

// Persistent-grid size for the grouped GEMM on the current device.
int gemm_grid(const moe_problem_t& p);

// Expert-GEMM tile widths (nnb1, nnb2: 2 = 128 weight rows per tile, 4 = 256)
// and row bands per raster group, from the problem's flags and shape.
struct TileChoice {
  int nnb1, nnb2, group_m;
};
TileChoice choose_tiles(const moe_problem_t& p, const Layout& L, int G);

// Shared device helpers -------------------------------------------------------

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Eight consecutive columns (8 c .. 8 c + 7) of combine-buffer row p as fp32.
template <bool BF16_IN>
__device__ __forceinline__ void combine_load8(const void* buf, size_t p, int d, int c, float (&v)[8]) {
  if constexpr (BF16_IN) {
    const uint4 u = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(buf) + p * d)[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(buf) + p * d) + 2 * c;
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// The weighted combine of output row q (Cui et al., Section 2.1 step (5)):
// Y[q] = sum over slots p in [tok_off[q], tok_off[q+1]) of comb_w[p] *
// buf[p], ascending p, fp32 fused multiply-add, rounded once to bf16 (and
// the fp32 sums to Y32 if set). Threads tid, tid + nthr, ... take 8 columns
// each. A slot range outside [0, cap) gives a NaN row and reads nothing.
template <bool BF16_IN>
__device__ __forceinline__ void combine_row(const void* buf, const int32_t* tok_off, const float* comb_w, int q,
                                            int d, int cap, uint16_t* Y, float* Y32, int tid, int nthr) {
  const int vec = d >> 3;
  const int p0 = tok_off[q], p1 = tok_off[q + 1];
  const bool ok = 0 <= p0 && p0 <= p1 && p1 <= cap;
  for (int c = tid; c < vec; c += nthr) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = ok ? 0.0f : __builtin_nanf("");
    if (ok) {
      for (int p = p0; p < p1; ++p) {
        const float wgt = comb_w[p];
        float v[8];
        combine_load8<BF16_IN>(buf, (size_t)p, d, c, v);
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

// Output row of token t with S destination segments.
__host__ __device__ __forceinline__ int y_row_of_token(int t, int T, int S) {
  return (t % S) * (T / S) + t / S;
}

}  // namespace moe
