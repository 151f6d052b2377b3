// Persistent grouped expert GEMM with a SwiGLU Linear-1 epilogue and a
// combine-store Linear-2 epilogue, on gfx950 bf16 MFMA.
//
// What it computes (X-Stage: An Overlooked Pipeline Stage for Communication-
// Computation Overlap in DiT Inference, Section 2.2 "MegaMoE Execution"):
// per local expert e and expert-contiguous row r of X_perm,
//   Linear-1 + SwiGLU : H[r, j]  = bf16( silu(W1[e][j] . x_r) * (W1[e][f+j] . x_r) )
//   Linear-2          : C[row_dst[r], n] = W2[e][n] . H[r]          (fp32)
//
// How the work is cut (Cui et al., Section 3.3.1: one rank-wide persistent
// kernel walks a unified tile list, each item an (expert, tile) pair, with
// the expert's pointers substituted per item; X-Stage Algorithm 1 for the
// ordering):
//   - a row band p is up to kBM = 256 consecutive rows of one expert; bands
//     are listed expert by expert (row p of the scheduler);
//   - a Linear-1 tile is (p, n1): 64 SwiGLU columns = 64 gate + 64 up rows of
//     W1[e]; a Linear-2 tile is (p, n2): 128 output columns;
//   - the K loop streams 128-byte slices of every row through a three-stage
//     LDS ring filled by direct global->LDS loads (global_load_lds_dwordx4),
//     so the weight tile is read from HBM once per band and reused by every
//     row of the band;
//   - 4 wavefronts, 2 (rows) x 2 (columns); a wavefront owns the 32-row
//     blocks {wm, wm+2, ...} of the band and two 32-column blocks, one
//     v_mfma_f32_32x32x16_bf16 accumulator each; the number of 32-row blocks
//     is a template parameter, so empty blocks cost neither loads nor MFMAs.
//
// Schedules (X-Stage Section 4.2, Algorithm 1, Figure 4):
//   MODE_SEP_L1/L2    every Linear-1 tile, then (next launch) every Linear-2 tile
//   MODE_WAVE         experts grouped into waves; a wave's Linear-1 tiles, then
//                     its Linear-2 tiles; each Linear-2 tile waits on l2_full[p]
//   MODE_INTERLEAVED  per pair-instance g (two workgroups, roles r = 0, 1) two
//                     cursors k1, k2 advance by the instance count; a Linear-2
//                     tile of row p2 = k2 / P2 is emitted only when the Linear-1
//                     row p1 = k1 / P1 leads it by at least D rows, otherwise
//                     the next Linear-1 tile; the N-tile of a pair cursor is
//                     n = 2 (k mod P) + r.
// l2_full[p] counts stored Linear-1 tiles of row p (X-Stage Section 4.2,
// "Condition 2"): the Linear-1 epilogue publishes with an agent-scope release
// after its H stores, a Linear-2 tile of row p acquires once it reaches the
// number of Linear-1 tiles per row. A workgroup only waits on rows at least
// D >= 1 behind its own Linear-1 cursor, so the smallest unfinished Linear-1
// row always belongs to a workgroup that is not waiting (no deadlock while
// the whole grid is resident: one workgroup per CU). Waits are bounded; a
// timeout sets the sticky error flag meta[META_ERR].
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

struct GemmParams {
  const uint8_t* X;       // X_perm [cap, d] (bf16 or e4m3 codes)
  const uint8_t* W1;      // [E_l, 2f, d]
  const uint8_t* W2;      // [E_l, d, f]
  uint8_t* H;             // [cap, f] Linear-2 operand (bf16 or e4m3 codes)
  float* C;               // combine_buf [cap, d]
  // fp8 only: block scales and the fp32 SwiGLU output before quantisation
  const float* Xs;        // [d/128, cap]  scale of X_perm row r, K block c at c*cap + r
  const float* W1s;       // [E_l, 2f/128, d/128]
  const float* W2s;       // [E_l, d/128, f/128]
  float* Hs;              // [f/128, cap]
  float* Hf;              // [cap, f] fp32
  int cap;
  const int32_t* row_dst;
  const int32_t* band_expert;
  const int32_t* band_row0;
  const int32_t* band_rows;
  int32_t* l2_full;
  int32_t* blk_done;      // fp8: [Pmax, f/128] Linear-1 tiles stored per (band, 128-column block)
  int32_t* meta;
  const int32_t* wave_band0;
  int d, f;
  int N1, N2;             // Linear-1 tiles per row band (f / 64), Linear-2 tiles (d / 128)
  int mode;
  int lead_D;
  int ready;              // l2_full value at which a row band's H is complete (N1, or f/128 with fp8)
};

struct Tile {
  const uint8_t* A;       // first row of the band (X_perm or H)
  const uint8_t* Bg;      // weight rows 0..63 of the tile
  const uint8_t* Bu;      // weight rows 64..127 of the tile
  size_t lda, ldb;        // row pitch in bytes
  int rows;               // valid rows of the band (1..256)
  int row0;               // first X_perm / H row of the band
  int n;                  // N-tile index
  int ktiles;             // K bytes / 128
  // fp8 only
  const float* As;        // row scales of K block 0 for the band's first row (next block: + cap)
  const float* Sg;        // weight block scales of rows 0..63 along K (one per 128-byte stage)
  const float* Su;        // weight block scales of rows 64..127
  int cap_stride;         // elements between consecutive K blocks of the row scales
};

// LDS ring geometry per number of 32-row blocks MB: a stage holds MB*32 rows
// of the band plus the 128 weight rows, 128 bytes of K each; with fp8 also the
// 256 row scales of the stage's K block (1 KiB).
__host__ __device__ constexpr int stage_a_bytes(int MB) { return MB * 32 * kKBytes; }
__host__ __device__ constexpr int stage_b_bytes() { return kBNW * kKBytes; }
__host__ __device__ constexpr int stage_bytes(int MB, bool FP8) {
  return stage_a_bytes(MB) + stage_b_bytes() + (FP8 ? kBM * 4 : 0);
}
__host__ __device__ constexpr int ring_stages(int MB, bool FP8) {
  return kGemmLds / stage_bytes(MB, FP8) > 8 ? 8 : kGemmLds / stage_bytes(MB, FP8);
}
// global -> LDS loads issued per lane per stage
__host__ __device__ constexpr int stage_loads(int MB, bool FP8) { return MB + 4 + (FP8 ? 1 : 0); }

// 16-byte chunk c of row `row` in a stage: rows are 128 bytes, the chunk index
// is XOR-swizzled with (row / 2) mod 8 so that the 16 rows a 16-lane phase of
// ds_read_b128 touches spread over all 64 LDS banks.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kKBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() would also
// drain every outstanding global load (vmcnt(0)), which would empty the
// prefetch ring; global->LDS completion is tracked explicitly with
// wait_vmcnt instead.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8));
}

// One pipeline stage: K bytes [kt*128, kt*128+128) of the band's first 32*MB
// rows and of the tile's 128 weight rows (and, with fp8, the 256 row scales of
// K block kt). Every lane issues stage_loads(MB, FP8) loads; lane i of a
// 16-byte instruction lands at LDS base + 16*i (8 rows of 128 B), lane i of a
// 4-byte instruction at base + 4*i.
template <int MB, bool FP8>
__device__ __forceinline__ void issue_stage(const Tile& t, int kt, lds_t* st) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = kt * kKBytes;
  const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r0 = (i * 4 + w) * 8;
    const int r = r0 + sub;
    const int gr = r < t.rows ? r : t.rows - 1;  // rows past the band re-read its last row
    const uint8_t* g = t.A + (size_t)gr * t.lda + kb + ((slot ^ ((r >> 1) & 7)) << 4);
    __builtin_amdgcn_global_load_lds(g, st + r0 * kKBytes, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r0 = (i * 4 + w) * 8;
    const int r = r0 + sub;
    const uint8_t* base = r < 64 ? t.Bg : t.Bu;
    const uint8_t* g = base + (size_t)(r & 63) * t.ldb + kb + ((slot ^ ((r >> 1) & 7)) << 4);
    __builtin_amdgcn_global_load_lds(g, st + stage_a_bytes(MB) + r0 * kKBytes, 16, 0, 0);
  }
  if constexpr (FP8) {
    const int r = w * 64 + lane;
    const int gr = r < t.rows ? r : t.rows - 1;
    const float* g = t.As + (size_t)kt * t.cap_stride + gr;
    __builtin_amdgcn_global_load_lds(g, st + stage_a_bytes(MB) + stage_b_bytes() + w * 256, 4, 0, 0);
  }
}

// MFMAs of one stage for a wavefront that owns NMB row blocks {wm, wm+2, ...}
// and weight rows {nb*64 + wn*32 .. +32} for nb = 0, 1.
// The K order inside a stage is a permutation shared by both operands (lane
// half h of an MFMA reads the same chunk indices of its A row and B row), so
// the sum over K is unchanged.
template <int NMB>
__device__ __forceinline__ void compute_stage(const lds_t* sa, const lds_t* sb, int wm, int wn,
                                              f32x16 (&acc)[NMB][2]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int chunk = ks * 2 + hi;
    bf16x8 b[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      b[nb] = *(const lds_bf16x8*)(sb + lds_off(nb * 64 + wn * 32 + lr, chunk));
#pragma unroll
    for (int mi = 0; mi < NMB; ++mi) {
      const int row = (wm + 2 * mi) * 32 + lr;
      const bf16x8 a = *(const lds_bf16x8*)(sa + lds_off(row, chunk));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[nb], acc[mi][nb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ i32x8 lds_read_32B(const lds_t* base, int row, int chunk0) {
  const i32x4 lo = *(const lds_i32x4*)(base + lds_off(row, chunk0));
  const i32x4 hi = *(const lds_i32x4*)(base + lds_off(row, chunk0 + 1));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// fp8 stage: the stage is exactly one 128-wide K block, so the block's MFMA
// sum (two v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales) is
// promoted into the fp32 accumulator with the row's activation scale times
// the weight block's scale: acc += partial * sx[row] * sw[nb].
template <int NMB>
__device__ __forceinline__ void compute_stage_fp8(const lds_t* sa, const lds_t* sb, const lds_t* ss, float swg,
                                                  float swu, int wm, int wn, f32x16 (&acc)[NMB][2]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, hi = lane >> 5;
  i32x8 b[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) b[ks][nb] = lds_read_32B(sb, nb * 64 + wn * 32 + lr, ks * 4 + hi * 2);
  const f32x16 zero = {};
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int mb = wm + 2 * mi;
    f32x16 part[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i32x8 a = lds_read_32B(sa, mb * 32 + lr, ks * 4 + hi * 2);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        part[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[ks][nb], ks ? part[nb] : zero, 0, 0, 0,
                                                                   127, 0, 127);
    }
    // the lane's rows of block mb: mb*32 + 8*g + 4*hi + (0..3), g = 0..3
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 sx = *(const lds_f32x4*)(ss + (mb * 32 + 8 * g + 4 * hi) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        acc[mi][0][i] = fmaf(part[0][i], sx[j] * swg, acc[mi][0][i]);
        acc[mi][1][i] = fmaf(part[1][i], sx[j] * swu, acc[mi][1][i]);
      }
    }
  }
}

// Load p[i] where p and i are the same in every lane, through the scalar
// cache (a read-only weight scale): a vector load here would be counted by
// vmcnt and force a wait that drains the global->LDS prefetch ring.
__device__ __forceinline__ float uniform_load(const float* p, int i) {
  const uint64_t a = reinterpret_cast<uint64_t>(p + i);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return *reinterpret_cast<const __attribute__((address_space(4))) float*>(((uint64_t)hi << 32) | lo);
}

template <int MB, int NMB, bool FP8>
__device__ __forceinline__ void compute_any(const Tile& t, const lds_t* st, int kt, int wm, int wn,
                                            f32x16 (&acc)[NMB][2]) {
  if constexpr (FP8) {
    const float swg = uniform_load(t.Sg, kt), swu = uniform_load(t.Su, kt);
    compute_stage_fp8<NMB>(st, st + stage_a_bytes(MB), st + stage_a_bytes(MB) + stage_b_bytes(), swg, swu, wm,
                           wn, acc);
  } else {
    compute_stage<NMB>(st, st + stage_a_bytes(MB), wm, wn, acc);
  }
}

// Accumulator element i of a 32x32 block sits at row 8*(i/4) + 4*(lane/32) + i%4,
// column lane%32.
template <int NMB, bool L1, bool FP8>
__device__ __forceinline__ void epilogue(const GemmParams& P, const Tile& t, int wm, int wn,
                                         const f32x16 (&acc)[NMB][2]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int mb = wm + 2 * mi;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = mb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
      if (m < t.rows) {
        if constexpr (L1) {
          const float g = acc[mi][0][i], u = acc[mi][1][i];
          const float act = g / (1.0f + expf(-g)) * u;
          const int col = t.n * kBN1 + wn * 32 + lr;
          const size_t at = (size_t)(t.row0 + m) * P.f + col;
          if constexpr (FP8) P.Hf[at] = act;  // quantised per row band once all its tiles are stored
          else reinterpret_cast<uint16_t*>(P.H)[at] = f32_to_bf16_rne(act);
        } else {
          const int dst = P.row_dst[t.row0 + m];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int col = t.n * kBN2 + nb * 64 + wn * 32 + lr;
            P.C[(size_t)dst * P.d + col] = acc[mi][nb][i];
          }
        }
      }
    }
  }
}

// Drain the last R+1 stages of the ring: stage kt is complete once at most R
// stages (R * stage_loads loads per lane) are still in flight.
template <int MB, int NMB, bool FP8, int R>
__device__ __forceinline__ void drain(const Tile& t, lds_t* lds, int rd, int kt, int wm, int wn,
                                      f32x16 (&acc)[NMB > 0 ? NMB : 1][2]) {
  constexpr int S = ring_stages(MB, FP8), SB = stage_bytes(MB, FP8);
  wait_vmcnt<R * stage_loads(MB, FP8)>();
  lds_barrier();
  if constexpr (NMB > 0) compute_any<MB, NMB, FP8>(t, lds + rd * SB, kt, wm, wn, acc);
  if constexpr (R > 0) drain<MB, NMB, FP8, R - 1>(t, lds, rd + 1 == S ? 0 : rd + 1, kt + 1, wm, wn, acc);
}

// The whole tile for one wavefront role: every wavefront runs the same number
// of loads and barriers; NMB (its share of the MB row blocks) only changes the
// MFMA and epilogue work, and the accumulators stay inside this function.
// The LDS ring has ring_stages(MB) stages of stage_bytes(MB): as many as fit
// in 160 KiB, so that S-1 stages of weight bytes are in flight per CU.
template <int MB, int NMB, bool L1, bool FP8>
__device__ __forceinline__ void tile_body(const GemmParams& P, const Tile& t, lds_t* lds, int wm, int wn) {
  constexpr int S = ring_stages(MB, FP8), SB = stage_bytes(MB, FP8), LD = stage_loads(MB, FP8);
  f32x16 acc[NMB > 0 ? NMB : 1][2];
#pragma unroll
  for (int a = 0; a < (NMB > 0 ? NMB : 1); ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  const int KT = t.ktiles;
  if (KT < S) {
    // the whole K extent fits in the ring
    for (int kt = 0; kt < KT; ++kt) issue_stage<MB, FP8>(t, kt, lds + kt * SB);
    wait_vmcnt<0>();
    lds_barrier();
    if constexpr (NMB > 0)
      for (int kt = 0; kt < KT; ++kt) compute_any<MB, NMB, FP8>(t, lds + kt * SB, kt, wm, wn, acc);
  } else {
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue_stage<MB, FP8>(t, s, lds + s * SB);
    int rd = 0, wr = S - 1, kt = 0;
    for (; kt + S - 1 < KT; ++kt) {
      wait_vmcnt<(S - 2) * LD>();  // this lane's loads of stage kt have landed
      lds_barrier();               // ... everyone's; and slot wr (stage kt-1) is no longer read
      issue_stage<MB, FP8>(t, kt + S - 1, lds + wr * SB);
      if constexpr (NMB > 0) compute_any<MB, NMB, FP8>(t, lds + rd * SB, kt, wm, wn, acc);
      rd = rd + 1 == S ? 0 : rd + 1;
      wr = wr + 1 == S ? 0 : wr + 1;
    }
    drain<MB, NMB, FP8, S - 2>(t, lds, rd, kt, wm, wn, acc);
  }
  lds_barrier();  // LDS ring free for the next tile
  if constexpr (NMB > 0) epilogue<NMB, L1, FP8>(P, t, wm, wn, acc);
}

template <int MB, bool L1, bool FP8>
__device__ __forceinline__ void run_tile(const GemmParams& P, const Tile& t, lds_t* lds) {
  const int w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  if (wm == 0) tile_body<MB, (MB + 1) / 2, L1, FP8>(P, t, lds, wm, wn);
  else tile_body<MB, MB / 2, L1, FP8>(P, t, lds, wm, wn);
}

template <bool L1, bool FP8>
__device__ __forceinline__ void dispatch_tile(const GemmParams& P, const Tile& t, lds_t* lds) {
  switch ((t.rows + 31) >> 5) {
    case 1: run_tile<1, L1, FP8>(P, t, lds); break;
    case 2: run_tile<2, L1, FP8>(P, t, lds); break;
    case 3: run_tile<3, L1, FP8>(P, t, lds); break;
    case 4: run_tile<4, L1, FP8>(P, t, lds); break;
    case 5: run_tile<5, L1, FP8>(P, t, lds); break;
    case 6: run_tile<6, L1, FP8>(P, t, lds); break;
    case 7: run_tile<7, L1, FP8>(P, t, lds); break;
    default: run_tile<8, L1, FP8>(P, t, lds); break;
  }
}

// Wait until row band p's H is complete. Thread 0 polls l2_full[p] with
// device-scope loads (they bypass the CU's L1 and see the value the
// producers' device-scope atomics left), then the workgroup proceeds.
//
// No cache invalidation is needed before the H loads: a band's H lines are
// first read only after the band is complete (only Linear-2 tiles of band p
// read them, and only after this wait), rows are whole multiples of 128-byte
// lines so no line is shared by two bands, and every launch starts with the
// kernel-entry acquire; so neither this CU's L1 nor its XCD's L2 can hold a
// stale copy. Invalidating the L2 here would instead discard the weight and
// activation lines the other 31 CUs of the XCD are reusing.
__device__ __forceinline__ void wait_row_ready(const GemmParams& P, int p) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(&P.l2_full[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < P.ready) {
      // after one timeout in this call every later wait gives up at once
      if (__hip_atomic_load(&P.meta[META_ERR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(&P.meta[META_ERR], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Make this workgroup's global stores visible at device scope, then let
// thread 0 add `inc` to a readiness counter (returned: its old value, in
// thread 0): every wave waits for its own stores to be
// acknowledged (vmcnt(0)), the barrier orders that before thread 0, whose
// device-scope release writes the XCD's L2 back before the increment.
__device__ __forceinline__ int publish(int32_t* counter, int inc) {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    old = __hip_atomic_fetch_add(counter, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return old;
}

// fp8: per row, per 128 columns of the band's fp32 SwiGLU output, scale =
// amax / 448 (1 for an all-zero block) and code = e4m3(value / scale), round
// to nearest even; 16 lanes per (row, block), 8 values per lane.
__device__ void quantize_band(const GemmParams& P, int row0, int rows) {
  const int fb = P.f >> 7;
  const int grp = threadIdx.x >> 4, q = threadIdx.x & 15;
  for (int it = grp; it < rows * fb; it += kGemmThreads / 16) {
    const int r = row0 + it / fb, c = it % fb;
    const float4* src = reinterpret_cast<const float4*>(P.Hf + (size_t)r * P.f + c * 128 + q * 8);
    const float4 v0 = src[0], v1 = src[1];
    float amax = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                       fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0.x / scale, v0.y / scale, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0.z / scale, v0.w / scale, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v1.x / scale, v1.y / scale, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v1.z / scale, v1.w / scale, hi, true);
    *reinterpret_cast<uint2*>(P.H + (size_t)r * P.f + c * 128 + q * 8) = make_uint2((uint32_t)lo, (uint32_t)hi);
    if (q == 0) P.Hs[(size_t)c * P.cap + r] = scale;
  }
}

// fp8: quantise column block j (128 SwiGLU columns) of a row band: per row,
// scale = amax / 448 (1 for an all-zero block) and code = e4m3(value /
// scale), round to nearest even. 16 lanes per row (8 values each), 16 rows per
// pass; the loads of four passes are issued before any is used.
__device__ void quantize_block(const GemmParams& P, int row0, int rows, int j) {
  const int rr = threadIdx.x >> 4, q = threadIdx.x & 15;
  const int col = j * 128 + q * 8;
  for (int base = 0; base < rows; base += 64) {
    float4 v[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + u * 16 + rr;
      if (r < rows) {
        const float4* src = reinterpret_cast<const float4*>(P.Hf + (size_t)(row0 + r) * P.f + col);
        v[u][0] = src[0];
        v[u][1] = src[1];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + u * 16 + rr;
      if (r >= rows) continue;  // uniform across the 16 lanes of a row
      const float4 a = v[u][0], b = v[u][1];
      float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                         fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
      const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a.x / scale, a.y / scale, 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(a.z / scale, a.w / scale, lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(b.x / scale, b.y / scale, 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(b.z / scale, b.w / scale, hi, true);
      *reinterpret_cast<uint2*>(P.H + (size_t)(row0 + r) * P.f + col) = make_uint2((uint32_t)lo, (uint32_t)hi);
      if (q == 0) P.Hs[(size_t)j * P.cap + row0 + r] = scale;
    }
  }
}

// After a Linear-1 tile's stores. bf16 (fused schedules only): count the tile
// in l2_full[p]; the band is ready at N1. fp8: tiles 2j and 2j+1 cover column
// block j; each counts itself in blk_done[p][j], and the second of the two
// (old value 1; every one of the block's Hf stores is then published)
// quantises the block and counts it in l2_full[p]; the band is ready at N1/2.
template <bool FP8>
__device__ __forceinline__ void finish_l1_tile(const GemmParams& P, const Tile& t, int p, bool fused, lds_t* lds) {
  if constexpr (!FP8) {
    if (fused) publish(P.l2_full + p, 1);
  } else {
    const int j = t.n >> 1;
    __attribute__((address_space(3))) int* flag = (__attribute__((address_space(3))) int*)lds;
    const int old = publish(P.blk_done + (size_t)p * (P.f >> 7) + j, 1);
    if (threadIdx.x == 0) *flag = old;
    __syncthreads();
    const bool second = *flag == 1;
    __syncthreads();  // the ring (and the flag in it) is reused by the next tile
    if (second) {
      quantize_block(P, t.row0, t.rows, j);
      publish(P.l2_full + p, 1);
    }
  }
}

template <bool L1, bool FP8>
__device__ __forceinline__ void do_tile(const GemmParams& P, int p, int n, bool fused, lds_t* lds) {
  constexpr int esz = FP8 ? 1 : 2;
  Tile t;
  const int e = P.band_expert[p];
  t.row0 = P.band_row0[p];
  t.rows = P.band_rows[p];
  t.n = n;
  t.cap_stride = P.cap;
  if constexpr (L1) {
    t.lda = (size_t)P.d * esz;
    t.ldb = (size_t)P.d * esz;
    t.A = P.X + (size_t)t.row0 * t.lda;
    const uint8_t* We = P.W1 + (size_t)e * 2 * P.f * t.ldb;
    t.Bg = We + (size_t)(n * kBN1) * t.ldb;
    t.Bu = We + (size_t)(P.f + n * kBN1) * t.ldb;
    t.ktiles = P.d * esz / kKBytes;
    if constexpr (FP8) {
      const int db = P.d >> 7, fb2 = (2 * P.f) >> 7;
      t.As = P.Xs + t.row0;
      t.Sg = P.W1s + ((size_t)e * fb2 + (n * kBN1) / 128) * db;
      t.Su = P.W1s + ((size_t)e * fb2 + (P.f + n * kBN1) / 128) * db;
    }
  } else {
    t.lda = (size_t)P.f * esz;
    t.ldb = (size_t)P.f * esz;
    t.A = P.H + (size_t)t.row0 * t.lda;
    t.Bg = P.W2 + ((size_t)e * P.d + (size_t)n * kBN2) * t.ldb;
    t.Bu = t.Bg + (size_t)64 * t.ldb;
    t.ktiles = P.f * esz / kKBytes;
    if constexpr (FP8) {
      t.As = P.Hs + t.row0;
      t.Sg = P.W2s + ((size_t)e * (P.d >> 7) + n) * (P.f >> 7);
      t.Su = t.Sg;
    }
    if (fused) wait_row_ready(P, p);
  }
  dispatch_tile<L1, FP8>(P, t, lds);
  if constexpr (L1) finish_l1_tile<FP8>(P, t, p, fused, lds);
}

template <bool FP8>
__global__ __launch_bounds__(kGemmThreads, 1) void moe_gemm_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmLds];
  lds_t* lds = (lds_t*)smem;  // address-space cast to the LDS window
  const int G = gridDim.x;
  const int b = blockIdx.x;
  // Workgroups are dealt round-robin to the 8 XCDs: make consecutive logical
  // ids share an XCD so a row band's tiles (same A rows) share one L2.
  const int lid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int Pb = P.meta[META_P];
  switch (P.mode) {
    case MODE_SEP_L1:
      for (int i = lid; i < Pb * P.N1; i += G) do_tile<true, FP8>(P, i / P.N1, i % P.N1, false, lds);
      break;
    case MODE_SEP_L2:
      for (int i = lid; i < Pb * P.N2; i += G) do_tile<false, FP8>(P, i / P.N2, i % P.N2, false, lds);
      break;
    case MODE_WAVE: {
      const int nw = P.meta[META_NWAVES];
      for (int wv = 0; wv < nw; ++wv) {
        const int pb0 = P.wave_band0[wv], pb1 = P.wave_band0[wv + 1];
        for (int i = lid; i < (pb1 - pb0) * P.N1; i += G)
          do_tile<true, FP8>(P, pb0 + i / P.N1, i % P.N1, true, lds);
        for (int i = lid; i < (pb1 - pb0) * P.N2; i += G)
          do_tile<false, FP8>(P, pb0 + i / P.N2, i % P.N2, true, lds);
      }
      break;
    }
    default: {  // MODE_INTERLEAVED
      const int g = lid >> 1, r = lid & 1, Gp = G >> 1;
      const int P1 = (P.N1 + 1) >> 1, P2 = (P.N2 + 1) >> 1;
      const int end1 = Pb * P1, end2 = Pb * P2;
      int k1 = g, k2 = g;
      while (k1 < end1 || k2 < end2) {
        const int p1 = k1 < end1 ? k1 / P1 : 0x3FFFFFFF;
        const int p2 = k2 / P2;
        if (k2 < end2 && p2 + P.lead_D <= p1) {
          const int n = 2 * (k2 % P2) + r;
          if (n < P.N2) do_tile<false, FP8>(P, p2, n, true, lds);
          k2 += Gp;
        } else {
          const int n = 2 * (k1 % P1) + r;
          if (n < P.N1) do_tile<true, FP8>(P, p1, n, true, lds);
          k1 += Gp;
        }
      }
      break;
    }
  }
}

// Row bands from the per-expert offsets, zeroed l2_full counters, and the
// expert waves (fewest consecutive experts whose Linear-1 tiles reach the grid,
// or a fixed number of experts per wave).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int El, int N1, int G,
                                                    int wave_experts, int Pmax, int32_t* __restrict__ blk_done,
                                                    int nblk_done, int32_t* __restrict__ band_expert,
                                                    int32_t* __restrict__ band_row0,
                                                    int32_t* __restrict__ band_rows, int32_t* __restrict__ l2_full,
                                                    int32_t* __restrict__ wave_band0, int32_t* __restrict__ meta) {
  __shared__ int start[1025];
  __shared__ int sh[64];
  for (int i = threadIdx.x; i < Pmax; i += blockDim.x) l2_full[i] = 0;
  for (int i = threadIdx.x; i < nblk_done; i += blockDim.x) blk_done[i] = 0;
  if (threadIdx.x == 0) meta[META_ERR] = 0;  // the flag reports this call only
  const int e = threadIdx.x;
  int cnt = 0, nb = 0;
  if (e < El) {
    cnt = offsets[e + 1] - offsets[e];
    nb = (cnt + kBM - 1) / kBM;
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
  if (e < El) {
    start[e] = first;
    const int r0 = offsets[e];
    for (int i = 0; i < nb; ++i) {
      band_expert[first + i] = e;
      band_row0[first + i] = r0 + i * kBM;
      band_rows[first + i] = min(kBM, cnt - i * kBM);
    }
  }
  if (threadIdx.x == 0) start[El] = sh[16];
  __syncthreads();
  if (threadIdx.x == 0) {
    const int Ptot = start[El];
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(moe_gemm_kernel<false>),
                                                     kGemmThreads, 0) != hipSuccess)
      return 0;
    cached_grid = prop.multiProcessorCount * (occ > 0 ? occ : 1);
    cached_dev = dev;
  }
  int g = cached_grid;
  if (p.grid > 0 && p.grid < g) g = p.grid;  // never above the co-resident limit
  if (g > 1 && (g & 1)) --g;                  // pair instances need an even grid
  return g;
}

hipError_t launch_expert_forward(const moe_problem_t& p, const Layout& L, char* ws, const void* X_perm,
                                 const float* X_perm_scale, const int32_t* offsets, const int32_t* row_dst,
                                 const void* W1, const float* W1_scale, const void* W2,
                                 const float* W2_scale, float* combine_buf, hipStream_t s) {
  const int G = gemm_grid(p);
  if (G <= 0) return hipErrorInvalidDevice;
  const bool fp8 = p.dtype == MOE_DTYPE_FP8_E4M3;
  GemmParams P{};
  P.X = static_cast<const uint8_t*>(X_perm);
  P.W1 = static_cast<const uint8_t*>(W1);
  P.W2 = static_cast<const uint8_t*>(W2);
  P.H = reinterpret_cast<uint8_t*>(ws + L.pub.h);
  P.C = combine_buf;
  P.Xs = X_perm_scale;
  P.W1s = W1_scale;
  P.W2s = W2_scale;
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
  P.N1 = p.f / kBN1;
  P.N2 = p.d / kBN2;
  P.ready = fp8 ? p.f / 128 : P.N1;
  P.blk_done = reinterpret_cast<int32_t*>(ws + L.blk_done);
  // Anti-starvation knee (X-Stage Eq. 16): D = b_n K / (2 h) with b_n the weight
  // rows of a Linear-1 tile (128), K the participating workgroups and h = f,
  // i.e. the rows one sweep of the grid covers. The knee is a lower bound;
  // below 8 rows Linear-2 tiles were measured to spin on the Mixtral shape
  // (f = 14336: knee 2), so the default lead is max(knee, 8).
  int D = p.lead_D;
  if (D <= 0) {
    D = (G + P.N1 - 1) / P.N1;
    if (D < 8) D = 8;
  }
  P.lead_D = D;

  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, L.E_l, P.N1, G, p.wave_experts, L.Pmax,
                     P.blk_done, fp8 ? L.Pmax * (p.f / 128) : 0, reinterpret_cast<int32_t*>(ws + L.band_expert), reinterpret_cast<int32_t*>(ws + L.band_row0),
                     reinterpret_cast<int32_t*>(ws + L.band_rows), P.l2_full,
                     reinterpret_cast<int32_t*>(ws + L.wave_band0), P.meta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto launch = [&](int mode) {
    P.mode = mode;
    if (fp8) hipLaunchKernelGGL(moe_gemm_kernel<true>, dim3(G), dim3(kGemmThreads), 0, s, P);
    else hipLaunchKernelGGL(moe_gemm_kernel<false>, dim3(G), dim3(kGemmThreads), 0, s, P);
    return hipGetLastError();
  };
  if (p.sched == MOE_SCHED_SEPARATE) {
    if ((e = launch(MODE_SEP_L1)) != hipSuccess) return e;
    return launch(MODE_SEP_L2);
  }
  return launch(p.sched == MOE_SCHED_EXPERT_WAVE ? MODE_WAVE : MODE_INTERLEAVED);
}

}  // namespace moe
