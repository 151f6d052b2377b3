// Owner-aligned return path: Cui et al., "Fine-grained Computation-
// Communication Overlap via Tile-level Signaling and Scheduling for MoE".
//   * Section 3.2.1 and Algorithm 1 (layout part): inside each local expert,
//     rows grouped by the rank that owns their token, remote ranks ascending
//     and the own rank last; each remote group zero-padded to a multiple of
//     the tile height tb_M so that every row band has a single owner.
//   * Section 3.2.2 and Algorithm 1 (schedule part): experts with more remote
//     row bands first, all remote bands before any local band.
//   * Section 3.2.3: per band, destination, receive-buffer offset, valid rows.
//   * Section 3.3.2 / Figure 3b: a group's first and last transfer segments
//     hold one band, the middle ones up to x bands.
// The owner of token t is rank t mod S (S = p->num_segments), the map of the
// eight-segment workloads. Inside a group rows keep ascending assignment id.
// The receive buffer holds S regions, one per rank, each in (expert,
// assignment id) order. On one GPU the own rank's group is copied too, so the
// buffer is complete; its bands are marked local-only.
//
// Like the page's plan construction, the plan is built on the host from the
// routing; the device side is the padded gather and the segment copy.
#include <algorithm>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace {

// X_pad[r] = X[row_src[r] / k] for a valid assignment id, zero otherwise.
// One workgroup per row at a time, 16 bytes per lane.
__global__ __launch_bounds__(256) void owner_gather_kernel(const uint16_t* __restrict__ X,
                                                           const int32_t* __restrict__ row_src, int R, int Tk,
                                                           int k, int d, uint16_t* __restrict__ X_pad) {
  const int vec = d >> 3;
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const int a = row_src[r];
    uint4* dst = reinterpret_cast<uint4*>(X_pad + (size_t)r * d);
    if (a >= 0 && a < Tk) {
      const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)(a / k) * d);
      for (int c = threadIdx.x; c < vec; c += blockDim.x) dst[c] = src[c];
    } else {
      for (int c = threadIdx.x; c < vec; c += blockDim.x) dst[c] = make_uint4(0, 0, 0, 0);
    }
  }
}

// fp8: the e4m3 codes of X[row_src[r] / k] (16 bytes per lane) and the row's
// block scales, X_pad_scale[c * cap + r] = X_scale[t / 128][c] (the K-block-
// major layout the grouped GEMM reads); a zero row gets codes 0 and scale 1.
__global__ __launch_bounds__(256) void owner_gather_fp8_kernel(const uint8_t* __restrict__ X,
                                                               const float* __restrict__ Xs,
                                                               const int32_t* __restrict__ row_src, int R, int Tk,
                                                               int k, int d, int cap, uint8_t* __restrict__ X_pad,
                                                               float* __restrict__ X_pad_scale) {
  const int vec = d >> 4, db = d >> 7;
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const int a = row_src[r];
    const bool valid = a >= 0 && a < Tk;
    const int t = valid ? a / k : 0;
    uint4* dst = reinterpret_cast<uint4*>(X_pad + (size_t)r * d);
    const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)t * d);
    for (int c = threadIdx.x; c < vec; c += blockDim.x) dst[c] = valid ? src[c] : make_uint4(0, 0, 0, 0);
    for (int c = threadIdx.x; c < db; c += blockDim.x)
      X_pad_scale[(size_t)c * cap + r] = valid ? Xs[(size_t)(t >> 7) * db + c] : 1.0f;
  }
}

// One segment per blockIdx.x; blockIdx.y (32 of them) strides its rows, so a
// segment of up to 32 rows has a workgroup per row. A segment is
// (src row, rows, dst row, dest); one whose rows fall outside [0, R) or
// [0, R_recv) is skipped.
__global__ __launch_bounds__(256) void segment_copy_kernel(const float* __restrict__ O_pad, int R,
                                                           const int32_t* __restrict__ seg, int R_recv, int d,
                                                           float* __restrict__ recv) {
  const int* s = seg + 4 * blockIdx.x;
  const int src = s[0], n = s[1], dst = s[2];
  if (src < 0 || n < 0 || dst < 0 || src > R - n || dst > R_recv - n) return;
  const int vec = d >> 2;
  for (int i = blockIdx.y; i < n; i += gridDim.y) {
    const float4* a = reinterpret_cast<const float4*>(O_pad + (size_t)(src + i) * d);
    float4* b = reinterpret_cast<float4*>(recv + (size_t)(dst + i) * d);
    for (int c = threadIdx.x; c < vec; c += blockDim.x) b[c] = a[c];
  }
}

// Segment transfer that runs beside the expert GEMM (Cui et al., Section
// 3.3.1-3.3.3: a consumer that polls the producer's tile flags and issues
// each segment once its tiles are stored). A small persistent grid walks the
// segments in plan order (segment q, q + gridDim.x, ...). In every wavefront
// lane 0 waits until every 32-row block b the segment touches counts
// min(32, R - 32 b) * d stored elements in row_done, polling with
// device-scope loads and a bounded spin; a timeout sets *err, and that and
// every later segment is then skipped. The wavefront then copies its share
// of the segment's columns. Wavefronts do not synchronise with each other:
// each copies only what it has itself seen ready.
//
// The kernel uses no LDS, so it never takes LDS a GEMM workgroup needs: the
// GEMM's persistent workgroups (the whole LDS of a CU each) stay resident
// beside it. A segment's rows are first read after their blocks are
// complete, rows are whole 128-byte lines (d % 128 == 0) and the launch
// starts with the kernel-entry acquire, so neither the CU's L1 nor its XCD's
// L2 holds a stale copy. O_pad is written by another kernel while this one
// runs, so it is neither const nor restrict here, and a workgroup-scope
// acquire fence after the poll keeps the compiler from moving a row load
// above it (an agent-scope acquire would also invalidate the L2, which the
// cache argument above makes unnecessary).
__global__ __launch_bounds__(256) void segment_copy_wait_kernel(float* O_pad, int R,
                                                                const int32_t* __restrict__ seg, int n_seg,
                                                                int R_recv, int d,
                                                                const int32_t* __restrict__ row_done,
                                                                int32_t* __restrict__ err,
                                                                float* __restrict__ recv) {
  const int lane = threadIdx.x & 63;
  const int vec = d >> 2;
  for (int q = blockIdx.x; q < n_seg; q += gridDim.x) {
    const int* s = seg + 4 * q;
    const int src = s[0], n = s[1], dst = s[2];
    if (src < 0 || n <= 0 || dst < 0 || src > R - n || dst > R_recv - n) continue;
    int ok = 1;
    if (lane == 0) {
      for (int b = src >> 5; ok && b <= (src + n - 1) >> 5; ++b) {
        const int need = (R - (b << 5) < 32 ? R - (b << 5) : 32) * d;
        int spins = 0;
        while (__hip_atomic_load(row_done + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(64);  // about 2 us between polls: little issue and memory traffic beside the GEMM
          if (++spins > kSpinLimit) {
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = 0;
            break;
          }
        }
      }
    }
    ok = __shfl(ok, 0, 64);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (!ok) continue;
    for (int i = 0; i < n; ++i) {
      const float4* a = reinterpret_cast<const float4*>(O_pad + (size_t)(src + i) * d);
      float4* b = reinterpret_cast<float4*>(recv + (size_t)(dst + i) * d);
      for (int c = threadIdx.x; c < vec; c += blockDim.x) b[c] = a[c];
    }
  }
}

}  // namespace

OwnerPlanSizes owner_plan_build(const moe_problem_t& p, const int32_t* idx, int local, int tb, int x,
                                std::vector<int32_t>& row_src, std::vector<int32_t>& expert_off,
                                std::vector<int32_t>& bands, std::vector<int32_t>& sched,
                                std::vector<int32_t>& segs, std::vector<int32_t>& recv_start) {
  const int T = p.T, k = p.k, S = p.num_segments, El = p.e_end - p.e_begin;
  // groups[el * S + r]: ascending assignment ids of expert el owned by rank r
  std::vector<std::vector<int32_t>> groups((size_t)El * S);
  for (int a = 0; a < T * k; ++a) {
    const int el = idx[a] - p.e_begin;
    if (el >= 0 && el < El) groups[(size_t)el * S + (a / k) % S].push_back(a);
  }
  std::vector<int> order;
  for (int r = 0; r < S; ++r)
    if (r != local) order.push_back(r);
  order.push_back(local);
  std::vector<int64_t> recv_rows(S, 0);
  row_src.clear();
  expert_off.assign(1, 0);
  bands.clear();
  std::vector<int> remote_bands(El, 0);
  for (int el = 0; el < El; ++el) {
    for (int r : order) {
      const auto& g = groups[(size_t)el * S + r];
      const int n = (int)g.size();
      const int padded = r == local ? n : (n + tb - 1) / tb * tb;
      const int first = (int)row_src.size();
      row_src.insert(row_src.end(), g.begin(), g.end());
      row_src.insert(row_src.end(), padded - n, -1);
      for (int b0 = 0; b0 < padded; b0 += tb) {
        const int valid = n - b0 < tb ? (n - b0 > 0 ? n - b0 : 0) : tb;
        bands.insert(bands.end(), {el, r, first + b0, valid, (int32_t)(recv_rows[r] + b0)});
        if (r != local) ++remote_bands[el];
      }
      recv_rows[r] += n;
    }
    expert_off.push_back((int32_t)row_src.size());
  }
  const int nb = (int)(bands.size() / 5);
  recv_start.assign(S + 1, 0);
  for (int r = 0; r < S; ++r) recv_start[r + 1] = recv_start[r] + (int32_t)recv_rows[r];
  // remote-first schedule: experts by descending remote band count, ties by index
  std::vector<int> ex(El);
  for (int el = 0; el < El; ++el) ex[el] = el;
  std::stable_sort(ex.begin(), ex.end(), [&](int a, int b) { return remote_bands[a] > remote_bands[b]; });
  std::vector<std::vector<int>> bands_of((size_t)El * S);  // bands of each (expert, rank) group, in order
  for (int b = 0; b < nb; ++b) bands_of[(size_t)bands[5 * b] * S + bands[5 * b + 1]].push_back(b);
  sched.clear();
  for (int el : ex)
    for (int r : order)
      if (r != local) sched.insert(sched.end(), bands_of[(size_t)el * S + r].begin(), bands_of[(size_t)el * S + r].end());
  const int n_remote = (int)sched.size();
  for (int el = 0; el < El; ++el)
    sched.insert(sched.end(), bands_of[(size_t)el * S + local].begin(), bands_of[(size_t)el * S + local].end());
  // transfer segments, in the order each group's first band is scheduled
  segs.clear();
  std::vector<char> seen((size_t)El * S, 0);
  for (int b : sched) {
    const size_t g = (size_t)bands[5 * b] * S + bands[5 * b + 1];
    if (seen[g]) continue;
    seen[g] = 1;
    const auto& m = bands_of[g];
    const int n = (int)m.size();
    auto emit = [&](int i0, int cnt) {
      int valid = 0;
      for (int i = i0; i < i0 + cnt; ++i) valid += bands[5 * m[i] + 3];
      const int dest = bands[5 * m[i0] + 1];
      segs.insert(segs.end(), {bands[5 * m[i0] + 2], valid, recv_start[dest] + bands[5 * m[i0] + 4], dest});
    };
    if (n <= 2) {
      for (int i = 0; i < n; ++i) emit(i, 1);
    } else {
      emit(0, 1);
      for (int i = 1; i < n - 1; i += x) emit(i, (n - 1 - i) < x ? (n - 1 - i) : x);
      emit(n - 1, 1);
    }
  }
  OwnerPlanSizes z;
  z.R = (int64_t)row_src.size();
  z.bands = nb;
  z.remote_bands = n_remote;
  z.segments = (int64_t)(segs.size() / 4);
  z.recv_rows = recv_start[S];
  return z;
}

hipError_t launch_owner_gather(const moe_problem_t& p, const void* X, const float* X_scale, const int32_t* row_src,
                               int R, void* X_pad, float* X_pad_scale, int cap, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int blocks = R < 8192 ? R : 8192;
  if (p.dtype != MOE_DTYPE_BF16) {
    hipLaunchKernelGGL(owner_gather_fp8_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t*>(X),
                       X_scale, row_src, R, p.T * p.k, p.k, p.d, cap, static_cast<uint8_t*>(X_pad), X_pad_scale);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(owner_gather_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t*>(X), row_src,
                     R, p.T * p.k, p.k, p.d, static_cast<uint16_t*>(X_pad));
  return hipGetLastError();
}

hipError_t launch_segment_copy(const moe_problem_t& p, const float* O_pad, int R, const int32_t* segs, int n_seg,
                               float* recv, int R_recv, hipStream_t s) {
  if (n_seg == 0) return hipSuccess;
  hipLaunchKernelGGL(segment_copy_kernel, dim3(n_seg, 32), dim3(256), 0, s, O_pad, R, segs, R_recv, p.d, recv);
  return hipGetLastError();
}

hipError_t launch_segment_copy_wait(const moe_problem_t& p, const float* O_pad, int R, const int32_t* segs,
                                    int n_seg, float* recv, int R_recv, const int32_t* row_done, int32_t* err,
                                    int grid, hipStream_t s) {
  if (n_seg == 0) return hipSuccess;
  const int g = grid < n_seg ? grid : n_seg;
  hipLaunchKernelGGL(segment_copy_wait_kernel, dim3(g), dim3(256), 0, s, const_cast<float*>(O_pad), R, segs, n_seg,
                     R_recv, p.d, row_done, err, recv);
  return hipGetLastError();
}

const void* segment_copy_wait_kernel_ptr() { return reinterpret_cast<const void*>(segment_copy_wait_kernel); }

}  // namespace moe
