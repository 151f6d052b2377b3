// Host side of the C ABI declared in include/moe_mi355x.h: argument checks,
// workspace layout and the launch order of the share's stages (route ->
// dispatch -> grouped expert GEMM -> combine) on the caller's stream.
#include <string.h>

#include "moe_internal.h"

namespace moe {
const void* gemm_kernel_bf16();
const void* gemm_kernel_fp8();
const void* gemm_kernel_w4a8();
const void* segment_copy_wait_kernel_ptr();
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
}  // namespace moe

namespace {

thread_local int g_last_hip_error = 0;

moe_status_t hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

moe_status_t check_problem(const moe_problem_t* p) {
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  if (p->dtype != MOE_DTYPE_BF16 && p->dtype != MOE_DTYPE_FP8_E4M3 && p->dtype != MOE_DTYPE_W4A8_MXFP4)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->sched < MOE_SCHED_EXPERT_WAVE || p->sched > MOE_SCHED_AUTO) return MOE_ERR_INVALID_ARGUMENT;
  if (p->flags & ~(uint32_t)(MOE_FLAG_FP32_Y_DEBUG | MOE_FLAG_BF16_COMBINE_BUF | MOE_FLAG_TILE_NARROW |
                                MOE_FLAG_TILE_WIDE | MOE_FLAG_BAND_MAJOR | MOE_FLAG_TILE_TRACE | MOE_FLAG_KEEP_H_F32 |
                                MOE_FLAG_TEST_WAIT_TIMEOUT))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((p->flags & MOE_FLAG_TILE_NARROW) && (p->flags & MOE_FLAG_TILE_WIDE)) return MOE_ERR_INVALID_ARGUMENT;
  if (p->lead_D < 0 || p->wave_experts < 0 || p->grid < 0 || p->row_capacity < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->T < 1 || p->d < 1 || p->f < 1 || p->E_global < 1 || p->k < 1) return MOE_ERR_UNSUPPORTED;
  if (p->E_global > 1024 || p->k > 16 || p->k > p->E_global) return MOE_ERR_UNSUPPORTED;
  if (p->e_begin < 0 || p->e_begin >= p->e_end || p->e_end > p->E_global) return MOE_ERR_UNSUPPORTED;
  if (p->num_segments < 1 || p->T % p->num_segments) return MOE_ERR_UNSUPPORTED;
  if (p->d % 128 || p->f % 128) return MOE_ERR_UNSUPPORTED;
  const int64_t cap = moe::row_capacity(*p);
  // 32-bit row and element indices inside the kernels
  if ((int64_t)p->T * p->k > (1ll << 30) || cap * p->d > (1ll << 31) - 1 || cap * p->f > (1ll << 31) - 1)
    return MOE_ERR_UNSUPPORTED;
  if (p->dtype != MOE_DTYPE_BF16) {
    if (p->quant_block != 128 || p->f % 128 || p->T % 128) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status_t check_ws(const moe::Layout& L, const void* ws, size_t bytes) {
  if (!ws) return MOE_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(ws) % 256) return MOE_ERR_INVALID_ARGUMENT;
  if (bytes < L.pub.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

// Whether a copier wavefront fits on a SIMD beside the expert GEMM's
// wavefronts (two per SIMD): their register counts, as the runtime reports
// them, rounded up to the allocation granule of 8, within the 512 registers
// per lane of a SIMD.
bool copier_fits_beside_gemm(int dtype) {
  hipFuncAttributes g{}, c{};
  const void* gemm = dtype == MOE_DTYPE_BF16 ? moe::gemm_kernel_bf16()
                     : dtype == MOE_DTYPE_FP8_E4M3 ? moe::gemm_kernel_fp8() : moe::gemm_kernel_w4a8();
  const bool fp8 = dtype != MOE_DTYPE_BF16;
  if (hipFuncGetAttributes(&g, gemm) != hipSuccess) return false;
  if (hipFuncGetAttributes(&c, moe::segment_copy_wait_kernel_ptr()) != hipSuccess) return false;
  auto granule = [](int r) { return (r + 7) / 8 * 8; };
  const int waves_per_simd = moe::gemm_threads(fp8) / 64 / 4;
  return waves_per_simd * granule(g.numRegs) + granule(c.numRegs) <= 512;
}

}  // namespace

extern "C" {

MOE_API size_t moe_workspace_size(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return moe::make_layout(*p).pub.total;
}

MOE_API moe_status_t moe_workspace_get_layout(const moe_problem_t* p, moe_workspace_layout_t* out) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_INVALID_ARGUMENT;
  *out = moe::make_layout(*p).pub;
  return MOE_OK;
}

MOE_API moe_status_t moe_route_topk(const moe_problem_t* p, const float* logits, int32_t* topk_idx,
                                    float* topk_w, int32_t* counts_global, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  hipError_t e = moe::launch_route(*p, logits, topk_idx, topk_w, counts_global, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_dispatch(const moe_problem_t* p, const void* X, const float* X_scale,
                                  const int32_t* topk_idx, const float* topk_w, int32_t* counts,
                                  int32_t* offsets, int32_t* row_src, int32_t* row_dst, int32_t* tok_off,
                                  float* comb_w, void* X_perm, float* X_perm_scale, void* workspace,
                                  size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  if (!X || !topk_idx || !topk_w || !counts || !offsets || !row_src || !row_dst || !tok_off || !comb_w ||
      !X_perm)
    return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 != (X_scale != nullptr) || fp8 != (X_perm_scale != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(X) || !aligned16(X_perm)) return MOE_ERR_INVALID_ARGUMENT;
  moe::Layout L = moe::make_layout(*p);
  if ((st = check_ws(L, workspace, ws_bytes)) != MOE_OK) return st;
  hipError_t e = moe::launch_dispatch(*p, L, moe::dispatch_scratch(L, static_cast<char*>(workspace)), X, X_scale,
                                      topk_idx, topk_w, counts,
                                      offsets, row_src, row_dst, tok_off, comb_w, X_perm, X_perm_scale,
                                      (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const void* X, const float* X_scale,
                                          const int32_t* topk_idx, const float* topk_w, int32_t* counts,
                                          int32_t* offsets, int32_t* row_src, int32_t* row_dst, int32_t* tok_off,
                                          float* comb_w, void* X_perm, float* X_perm_scale, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  if (!X || !topk_idx || !topk_w || !counts || !offsets || !row_src || !row_dst || !tok_off || !comb_w ||
      !X_perm)
    return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 != (X_scale != nullptr) || fp8 != (X_perm_scale != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(X) || !aligned16(X_perm)) return MOE_ERR_INVALID_ARGUMENT;
  const moe::Layout L = moe::make_layout(*p);
  // the dispatch's scratch, packed: meta words, per-chunk counts, per-row counts
  const size_t meta_b = moe::align_up(moe::kMetaInts * 4, 256);
  const size_t blk_b = moe::align_up((size_t)L.nblk * L.E_l * 4, 256);
  const size_t tok_b = moe::align_up((size_t)p->T * 4, 256);
  if (meta_b + blk_b + tok_b > moe::noalloc_scratch_bytes()) return MOE_ERR_UNSUPPORTED;
  void* base = nullptr;
  hipError_t e = moe::noalloc_scratch(&base);
  if (e != hipSuccess) return hip_fail(e);
  char* sc = static_cast<char*>(base);
  const moe::DispatchScratch scratch{reinterpret_cast<int32_t*>(sc + meta_b),
                                     reinterpret_cast<int32_t*>(sc + meta_b + blk_b), reinterpret_cast<int32_t*>(sc)};
  e = moe::launch_dispatch(*p, L, scratch, X, X_scale, topk_idx, topk_w, counts, offsets, row_src, row_dst, tok_off,
                           comb_w, X_perm, X_perm_scale, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_expert_forward(const moe_problem_t* p, const void* X_perm, const float* X_perm_scale,
                                        const int32_t* offsets, const int32_t* row_dst, const void* W1,
                                        const void* W1_scale, const void* W2, const void* W2_scale,
                                        void* combine_buf, void* workspace, size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  if (!X_perm || !offsets || !row_dst || !W1 || !W2 || !combine_buf) return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 != (X_perm_scale != nullptr) || fp8 != (W1_scale != nullptr) || fp8 != (W2_scale != nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(X_perm) || !aligned16(W1) || !aligned16(W2) || !aligned16(combine_buf))
    return MOE_ERR_INVALID_ARGUMENT;
  moe::Layout L = moe::make_layout(*p);
  if ((st = check_ws(L, workspace, ws_bytes)) != MOE_OK) return st;
  hipError_t e = moe::launch_expert_forward(*p, L, static_cast<char*>(workspace), X_perm, X_perm_scale, offsets,
                                            row_dst, W1, W1_scale, W2, W2_scale, combine_buf,
                                            (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_combine(const moe_problem_t* p, const void* combine_buf, const int32_t* tok_off,
                                 const float* comb_w, void* Y, float* Y_fp32, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!combine_buf || !tok_off || !comb_w || !Y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(combine_buf) || !aligned16(Y) || (Y_fp32 && !aligned16(Y_fp32))) return MOE_ERR_INVALID_ARGUMENT;
  hipError_t e = moe::launch_combine(*p, combine_buf, tok_off, comb_w, Y, Y_fp32, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_layer_forward(const moe_problem_t* p, const void* X, const float* X_scale,
                                       const float* logits, const void* W1, const void* W1_scale,
                                       const void* W2, const void* W2_scale, void* Y, float* Y_fp32,
                                       void* workspace, size_t ws_bytes, int32_t* topk_idx_out,
                                       float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                       int32_t* row_src_out, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  if (!X || !logits || !W1 || !W2 || !Y) return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 != (X_scale != nullptr) || fp8 != (W1_scale != nullptr) || fp8 != (W2_scale != nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((p->flags & MOE_FLAG_FP32_Y_DEBUG) && !Y_fp32) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(X) || !aligned16(W1) || !aligned16(W2) || !aligned16(Y) || (Y_fp32 && !aligned16(Y_fp32)))
    return MOE_ERR_INVALID_ARGUMENT;
  for (const void* q : {(const void*)topk_idx_out, (const void*)topk_w_out, (const void*)counts_out,
                        (const void*)offsets_out, (const void*)row_src_out})
    if (q && (reinterpret_cast<uintptr_t>(q) & 3)) return MOE_ERR_INVALID_ARGUMENT;
  moe::Layout L = moe::make_layout(*p);
  if ((st = check_ws(L, workspace, ws_bytes)) != MOE_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  auto I = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const moe_workspace_layout_t& W = L.pub;
  // a caller's output takes the place of its workspace region
  int32_t* idx = topk_idx_out ? topk_idx_out : I(W.topk_idx);
  float* wts = topk_w_out ? topk_w_out : F(W.topk_w);
  int32_t* counts = counts_out ? counts_out : I(W.counts);
  int32_t* offsets = offsets_out ? offsets_out : I(W.offsets);
  int32_t* row_src = row_src_out ? row_src_out : I(W.row_src);
  // Five launches with the separate schedule, four with the fused ones:
  // route + dispatch counts; scan + row-band plan + scatter; the expert
  // GEMM(s), Linear-1 gathering its rows from X; the weighted combine.
  float* xps = fp8 ? F(W.x_perm_scale) : nullptr;
  hipError_t e = moe::launch_route_count(*p, L, logits, idx, wts, I(L.blk_counts), I(L.tok_cnt), I(W.meta), s);
  if (e == hipSuccess)
    e = moe::launch_scan_plan_scatter(*p, L, ws, X_scale, idx, wts, counts, offsets, row_src, I(W.row_dst),
                                      I(W.tok_off), F(W.comb_w), xps, s);
  if (e == hipSuccess)
    e = moe::launch_expert_forward_fused(*p, L, ws, X, row_src, xps, I(W.row_dst), W1, W1_scale, W2, W2_scale,
                                         ws + W.combine_buf, s);
  if (e == hipSuccess) e = moe::launch_combine(*p, ws + W.combine_buf, I(W.tok_off), F(W.comb_w), Y, Y_fp32, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_check_workspace(const moe_problem_t* p, void* workspace, size_t ws_bytes,
                                         void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  moe::Layout L = moe::make_layout(*p);
  if ((st = check_ws(L, workspace, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  int32_t* meta = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + L.pub.meta);
  int32_t host[moe::META_ARG_ERR + 1] = {};
  hipError_t e = hipMemcpyAsync(host, meta, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  const bool timed_out = host[moe::META_ERR] != 0, bad_arg = (host[moe::META_ARG_ERR] & moe::ARG_ERR_ALL) != 0;
  if (timed_out || bad_arg) {
    const int32_t zero = 0;
    e = hipMemcpyAsync(meta + moe::META_ERR, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(meta + moe::META_ARG_ERR, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e);
    return timed_out ? MOE_ERR_DEADLOCK : MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

MOE_API moe_status_t moe_store_burst_probe(int K, int B, int reps, double gap_us, void* buf, size_t buf_bytes,
                                           uint64_t* rec, size_t rec_bytes, void* stream) {
  if (K < 1 || K > 4096 || B < 1024 || (B % 1024) != 0 || reps < 1 || reps > 100000) return MOE_ERR_INVALID_ARGUMENT;
  if (!(gap_us >= 0.0 && gap_us <= 1e5)) return MOE_ERR_INVALID_ARGUMENT;  // also rejects NaN
  if (gap_us * reps > 2e6) return MOE_ERR_INVALID_ARGUMENT;                // at most 2 s of gaps per launch
  if (!buf || !rec) return MOE_ERR_INVALID_ARGUMENT;
  if (((buf_bytes / (size_t)K) & ~(size_t)1023) < (size_t)B) return MOE_ERR_INVALID_ARGUMENT;
  if (rec_bytes < ((size_t)2 * K * reps + 1) * sizeof(uint64_t)) return MOE_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(rec) % 8) return MOE_ERR_INVALID_ARGUMENT;
  const hipError_t e = moe::launch_store_burst(K, B, reps, gap_us, buf, buf_bytes, rec, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_owner_plan(const moe_problem_t* p, const int32_t* topk_idx, int local_rank, int tb_M,
                                    int x_bands, int32_t* row_src, int64_t row_cap, int32_t* expert_off,
                                    int32_t* bands, int32_t* schedule, int32_t* segments, int64_t band_cap,
                                    int32_t* recv_start, moe_owner_plan_sizes_t* sizes) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!topk_idx || !sizes) return MOE_ERR_INVALID_ARGUMENT;
  if (local_rank < 0 || local_rank >= p->num_segments || tb_M < 1 || tb_M > 4096 || x_bands < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  std::vector<int32_t> rs, eo, bd, sc, sg, rv;
  moe::OwnerPlanSizes z = moe::owner_plan_build(*p, topk_idx, local_rank, tb_M, x_bands, rs, eo, bd, sc, sg, rv);
  if (z.R > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  sizes->R = z.R;
  sizes->bands = z.bands;
  sizes->remote_bands = z.remote_bands;
  sizes->segments = z.segments;
  sizes->recv_rows = z.recv_rows;
  if (!row_src && !expert_off && !bands && !schedule && !segments && !recv_start) return MOE_OK;
  if (!row_src || !expert_off || !bands || !schedule || !segments || !recv_start) return MOE_ERR_INVALID_ARGUMENT;
  if (row_cap < z.R || band_cap < z.bands) return MOE_ERR_WORKSPACE_TOO_SMALL;
  memcpy(row_src, rs.data(), rs.size() * sizeof(int32_t));
  memcpy(expert_off, eo.data(), eo.size() * sizeof(int32_t));
  memcpy(bands, bd.data(), bd.size() * sizeof(int32_t));
  memcpy(schedule, sc.data(), sc.size() * sizeof(int32_t));
  memcpy(segments, sg.data(), sg.size() * sizeof(int32_t));
  memcpy(recv_start, rv.data(), rv.size() * sizeof(int32_t));
  return MOE_OK;
}

MOE_API moe_status_t moe_owner_gather(const moe_problem_t* p, const void* X, const float* X_scale,
                                      const int32_t* row_src, int64_t R, void* X_pad, float* X_pad_scale,
                                      void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  const int64_t cap = moe::row_capacity(*p);
  if (R < 0 || R > (int64_t)INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 != (X_scale != nullptr) || fp8 != (X_pad_scale != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 && R > cap) return MOE_ERR_UNSUPPORTED;  // the scale rows are laid out with the workspace's capacity
  if (R > 0 && (!X || !row_src || !X_pad || !aligned16(X) || !aligned16(X_pad))) return MOE_ERR_INVALID_ARGUMENT;
  hipError_t e = moe::launch_owner_gather(*p, X, X_scale, row_src, (int)R, X_pad, X_pad_scale, (int)cap,
                                          (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_segment_copy(const moe_problem_t* p, const float* O_pad, int64_t R,
                                      const int32_t* segments, int64_t n_segments, float* recv, int64_t R_recv,
                                      void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (R < 0 || R > (int64_t)INT32_MAX || R_recv < 0 || R_recv > (int64_t)INT32_MAX || n_segments < 0 ||
      n_segments > (int64_t)INT32_MAX)
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_segments > 0 && (!O_pad || !segments || !recv || !aligned16(O_pad) || !aligned16(recv)))
    return MOE_ERR_INVALID_ARGUMENT;
  hipError_t e = moe::launch_segment_copy(*p, O_pad, (int)R, segments, (int)n_segments, recv, (int)R_recv,
                                          (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_expert_forward_signal(const moe_problem_t* p, const void* X_perm,
                                               const float* X_perm_scale, const int32_t* offsets,
                                               const int32_t* row_dst, const void* W1, const void* W1_scale,
                                               const void* W2, const void* W2_scale, void* combine_buf,
                                               int32_t* row_done, int64_t row_done_len, void* workspace,
                                               size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->dtype != MOE_DTYPE_BF16;  // e4m3 activations (and their scales)
  if (!X_perm || !offsets || !row_dst || !W1 || !W2 || !combine_buf || !row_done) return MOE_ERR_INVALID_ARGUMENT;
  if (row_done_len < 1 || row_done_len > (int64_t)INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
  if (fp8 != (X_perm_scale != nullptr) || fp8 != (W1_scale != nullptr) || fp8 != (W2_scale != nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(X_perm) || !aligned16(W1) || !aligned16(W2) || !aligned16(combine_buf))
    return MOE_ERR_INVALID_ARGUMENT;
  moe::Layout L = moe::make_layout(*p);
  if ((st = check_ws(L, workspace, ws_bytes)) != MOE_OK) return st;
  hipError_t e = moe::launch_expert_forward(*p, L, static_cast<char*>(workspace), X_perm, X_perm_scale, offsets,
                                            row_dst, W1, W1_scale, W2, W2_scale, combine_buf, (hipStream_t)stream,
                                            row_done, (int)row_done_len);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API moe_status_t moe_segment_copy_wait(const moe_problem_t* p, const float* O_pad, int64_t R,
                                           const int32_t* segments, int64_t n_segments, float* recv,
                                           int64_t R_recv, const int32_t* row_done, int64_t row_done_len,
                                           int32_t* err, int grid, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (R < 0 || R > (int64_t)INT32_MAX || R_recv < 0 || R_recv > (int64_t)INT32_MAX || n_segments < 0 ||
      n_segments > (int64_t)INT32_MAX || grid < 0 || grid > 1024 || (int64_t)p->d * 32 > (int64_t)INT32_MAX)
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_segments > 0 && (!O_pad || !segments || !recv || !row_done || !err || !aligned16(O_pad) || !aligned16(recv)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_segments > 0 && row_done_len < (R + 31) / 32) return MOE_ERR_INVALID_ARGUMENT;
  // A copier wavefront must fit on a SIMD beside the GEMM's two (the fp8
  // GEMM's take the whole register file): otherwise every wait would time out.
  if (!copier_fits_beside_gemm(p->dtype)) return MOE_ERR_UNSUPPORTED;
  hipError_t e = moe::launch_segment_copy_wait(*p, O_pad, (int)R, segments, (int)n_segments, recv, (int)R_recv,
                                               row_done, err, grid ? grid : 256, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

MOE_API const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported problem shape";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEADLOCK: return "persistent pipeline wait timed out";
  }
  return "unknown status";
}

MOE_API int moe_last_hip_error(void) { return g_last_hip_error; }

MOE_API const char* moe_version(void) { return "0.1.0"; }

MOE_API int moe_schedule_of(const moe_problem_t* p) {
  if (!p || p->sched < MOE_SCHED_EXPERT_WAVE || p->sched > MOE_SCHED_AUTO) return -1;
  return moe::resolve_schedule(*p);
}

MOE_API double moe_tile_clock_hz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0.0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0.0;
  return khz > 0 ? khz * 1e3 : 0.0;
}

}  // extern "C"
