// Device side of the persistent grouped expert GEMM with a SwiGLU Linear-1 epilogue and a
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
//   - a tile holds NNB * 64 weight rows, NNB = 2 (narrow) or 4 (wide): a
//     Linear-1 tile (p, n1) covers NNB * 32 SwiGLU columns, i.e. as many gate
//     rows and as many up rows of W1[e]; a Linear-2 tile (p, n2) covers
//     NNB * 64 output columns;
//   - the K loop streams 128-byte slices of every row through an LDS ring of
//     as many stages as fit in 160 KiB, filled by direct global->LDS loads
//     (global_load_lds_dwordx4), so the weight tile is read once per band and
//     reused by every row of the band;
//   - 8 wavefronts, two per SIMD (while one waits on LDS or on its loads the
//     other issues MFMAs), in a WM (rows) x WN (columns) grid: 2 x 4 for
//     wide tiles, 4 x 2 for narrow ones. A wavefront owns the 32-row blocks
//     {wm, wm+WM, ...} of the band and, in each half of the weight rows,
//     NNB/WN 32-column blocks, one v_mfma_f32_32x32x16_bf16 accumulator each;
//     a Linear-1 wavefront thus holds the gate and the up column of every
//     SwiGLU output it owns. The number of 32-row blocks (rounded up to a
//     multiple of WM) is a template parameter, so a short band costs fewer
//     loads and MFMAs;
//   - every schedule walks its tile lists in groups of group_m row bands,
//     N-tile by N-tile inside a group, so the tiles that run at the same time
//     on one XCD share both their row bands and their weight tiles through
//     that XCD's L2.
//
// Schedules (X-Stage Section 4.2, Algorithm 1, Figure 4):
//   MODE_SEP_L1/L2    every Linear-1 tile, then (next launch) every Linear-2 tile
//   MODE_WAVE         experts grouped into waves; a wave's Linear-1 tiles, then
//                     its Linear-2 tiles; each Linear-2 tile waits on l2_full[p]
//   MODE_INTERLEAVED  per pair-instance g (two workgroups, roles r = 0, 1) two
//                     cursors k1, k2 advance by the instance count over the
//                     (row band, pair column) lists of Linear-1 and Linear-2,
//                     both walked in raster groups of group_m bands; a Linear-2
//                     tile of band p2 is emitted only when the first band of
//                     the Linear-1 cursor's group leads p2 by at least D bands
//                     (with group_m = 1: the Linear-1 cursor's band, as in the
//                     algorithm), otherwise the next Linear-1 tile; the N-tile
//                     of pair column c is n = 2 c + r. With wide Linear-2
//                     tiles, the pair columns of a last, partly idle round
//                     run after a workgroup's Linear-1 tiles as narrow
//                     tiles dealt over all workgroups.
// l2_full[p] counts stored Linear-1 tiles of row p (X-Stage Section 4.2,
// "Condition 2"): the Linear-1 epilogue publishes with an agent-scope release
// after its H stores, a Linear-2 tile of row p acquires once it reaches the
// number of Linear-1 tiles per row. A workgroup only waits on bands that lie
// in raster groups before its own Linear-1 cursor's group, whose Linear-1
// tiles all precede its cursor; so the workgroup holding the earliest
// unfinished Linear-1 tile either runs it or waits on a band that is already
// complete (no deadlock while the whole grid is resident: one workgroup per
// CU). A workgroup in the narrow tail holds no Linear-1 tile. Waits are bounded; a
// timeout sets the sticky error flag meta[META_ERR].
#pragma once

#include "moe_internal.h"

namespace moe {

struct GemmParams {
  const uint8_t* X;       // X_perm [cap, d] (bf16 or e4m3 codes)
  const uint8_t* W1;      // [E_l, 2f, d]
  const uint8_t* W2;      // [E_l, d, f]
  uint8_t* H;             // [cap, f] Linear-2 operand (bf16 or e4m3 codes)
  void* C;                // combine_buf [cap, d]: fp32, or bf16 with c_bf16
  // fp8 only: block scales and the fp32 SwiGLU output before quantisation
  const float* Xs;        // [d/128, cap]  scale of X_perm row r, K block c at c*cap + r
  const float* W1s;       // [E_l, 2f/128, d/128] (e4m3 weights)
  const float* W2s;       // [E_l, d/128, f/128]
  const uint8_t* W1e;     // MXFP4 weights: E8M0 scales [E_l, 2f, d/32]
  const uint8_t* W2e;     // [E_l, d, f/32]
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
  int N1, N2;             // Linear-1 tiles per row band (f / (32 nnb1)), Linear-2 tiles (d / (64 nnb2))
  int nnb1, nnb2;         // tile width (2 or 4) of the Linear-1 and Linear-2 tiles
  int group_m;            // row bands per raster group of the tile lists
  int mode;
  int lead_D;
  int ready;              // l2_full value at which a row band's H is complete (N1, or f/128 with fp8)
  uint64_t* trace;        // tile records of 5 words (moe_tile_record_t), or null: no timing
  int trace_cap;          // records the trace region holds
  int keep_hf;            // fp8: wide Linear-1 tiles also store their fp32 SwiGLU values in Hf
  int32_t* row_done;      // or null: per 32-row block of output rows, output elements stored (Linear-2)
  int row_done_len;       // blocks row_done holds
  int c_bf16;             // the Linear-2 epilogue rounds its outputs to bf16 (MOE_FLAG_BF16_COMBINE_BUF)
  // Linear-1 gathers its rows (moe_layer_forward): band row r is X row
  // a_src[r] / a_k (X is then the token rows, not X_perm); null: X_perm rows
  const int32_t* a_src;
  int a_k;
};

// Launch the persistent expert-GEMM kernel of one operand type (bf16 in
// gemm_bf16.hip, fp8 in gemm_fp8.hip: each type is its own translation unit
// so the two compile in parallel) on G workgroups, and the kernel's address
// for occupancy queries.
hipError_t launch_gemm_bf16(const GemmParams& P, int G, hipStream_t s);
hipError_t launch_gemm_fp8(const GemmParams& P, int G, hipStream_t s);
hipError_t launch_gemm_w4a8(const GemmParams& P, int G, hipStream_t s);
const void* gemm_kernel_bf16();

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
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) int lds_i32;


struct Tile {
  const uint8_t* A;       // first row of the band (X_perm or H)
  const uint8_t* Bg;      // first half of the tile's weight rows (Linear-1: the gate rows)
  const uint8_t* Bu;      // second half (Linear-1: the matching up rows)
  size_t lda, ldb;        // row pitch in bytes
  int rows;               // valid rows of the band (1..256)
  int row0;               // first X_perm / H row of the band
  int n;                  // N-tile index, in units of this tile's width
  int nnb;                // width: NNB * 64 weight rows
  int ktiles;             // K bytes / stage_k_bytes
  int krot;               // pipeline stage kt streams K slice (kt + krot) mod ktiles
  bool once;              // the expert's only row band: each weight byte is read once per launch
  // fp8 activations only
  const float* As;        // row scales of K block 0 for the band's first row (next block: + cap)
  const float* Sg;        // fp8 weights: block scales of the first half along K (one per 128-byte stage)
  const float* Su;        // fp8 weights: block scales of the second half
  int cap_stride;         // elements between consecutive K blocks of the row scales
  // MXFP4 weights only: E8M0 bytes, K/32 per weight row (4 per 128-wide stage)
  const uint8_t* Eg;      // scale row of the first weight row of the first half
  const uint8_t* Eu;      // ... of the second half
  size_t epitch;          // bytes between consecutive scale rows
  // Linear-1 with gathered rows: band row r is row a_src[r] / a_k of A
  // (which then points at X); null: row row0 + r
  const int32_t* a_src;
  int a_k;
  // byte offset from A of the row this lane loads, one per band-row load
  // instruction of a stage (filled at the start of the tile, once its
  // row-block count is known). The ring loads address a uniform base plus a
  // 32-bit per-lane offset (the instructions' SGPR-base form, one VGPR per
  // load instead of two).
  uint32_t arow[8];
};

// Operand types of the expert GEMM (the template parameter OT): bf16
// activations and weights; e4m3 activations and e4m3 weights with fp32
// 128x128 block scales; e4m3 activations and MXFP4 weights (E2M1 elements,
// one E8M0 scale per 32 along K).
enum OperandType { OT_BF16 = 0, OT_FP8 = 1, OT_W4A8 = 2 };
__host__ __device__ constexpr bool mxfp4_weights(int OT) { return OT == OT_W4A8; }

// K bytes per row per pipeline stage: 64 bf16 values, or for fp8 one 128-wide
// scale block of e4m3 values. (64-byte bf16 stages, which double the ring
// depth of a wide tile, were measured no faster on the compute-bound shapes
// and slower on the bandwidth-bound ones.)
__host__ __device__ constexpr int stage_k_bytes(bool) { return 128; }

// Bytes a weight row contributes to one stage: the stage's K extent (64
// bf16, or 128 e4m3 values) in the weight format; MXFP4 packs 128 values in
// 64 bytes.
__host__ __device__ constexpr int stage_kb_bytes(int OT) { return mxfp4_weights(OT) ? 64 : stage_k_bytes(OT); }

// LDS ring geometry per number of 32-row blocks MB and tile width NNB: a stage
// holds MB*32 rows of the band plus the NNB*64 weight rows, one stage's K of
// each; with fp8 activations also the 256 row scales of the stage's K block
// (1 KiB), and either the block's two fp32 weight scales (padded to 16
// bytes) or, for MXFP4 weights, one dword of four E8M0 scales per weight row.
__host__ __device__ constexpr int stage_a_bytes(int MB, int OT) { return MB * 32 * stage_k_bytes(OT); }
__host__ __device__ constexpr int stage_b_bytes(int NNB, int OT) { return NNB * 64 * stage_kb_bytes(OT); }
__host__ __device__ constexpr int stage_scale_bytes(int NNB, int OT) {
  return OT == OT_FP8 ? kBM * 4 + 16 : OT == OT_W4A8 ? kBM * 4 + NNB * 64 * 4 : 0;
}
__host__ __device__ constexpr int stage_bytes(int MB, int NNB, int OT) {
  return stage_a_bytes(MB, OT) + stage_b_bytes(NNB, OT) + stage_scale_bytes(NNB, OT);
}
__host__ __device__ constexpr int ring_stages(int MB, int NNB, int OT) {
  return kGemmLds / stage_bytes(MB, NNB, OT) > 8 ? 8 : kGemmLds / stage_bytes(MB, NNB, OT);
}
// Wavefronts that issue the ring's global -> LDS loads. The CU accepts about
// one such 1 KiB instruction per 22 cycles, so a 64 KiB stage takes about
// 1400 cycles to issue, and a wavefront blocked at an issue runs no MFMA.
// One wavefront per SIMD (the last four) issues the whole stage, after the
// step's barrier, while the other wavefront of its SIMD already runs its
// MFMAs. With every wavefront issuing its share before the barrier, the
// issue and the MFMAs ran one after the other: per-phase cycle counts of
// the Mixtral Linear-1 K loop gave 17-33% of each step to issuing and 12-20%
// to the barrier behind it, against 1.5% waiting for data. Every operand
// type splits this way: W4A8 share GEMM 358 -> 316 us, fp8 381 -> 372 us
// (fp8 only once the loads' addresses became 32-bit offsets; with 64-bit
// addresses its loaders spilled inside the K loop and the split lost 1%).
__host__ __device__ constexpr int loader_waves(int) { return 4; }

// Weight rows of an expert with a single row band are read once per launch:
// no other tile of the launch reads them again. Their ring loads then carry
// the non-temporal hint, so that the weight stream does not displace what is
// reused (the band rows, H, the combine buffer) from the L2 and the
// last-level cache. Measured on the DeepSeek-style share (every expert one
// band): Linear-1 365 -> 332 us, Linear-2 220 -> 211 us, fp8 GEMM 362 -> 330
// us; the counted L2 misses were the same, the hint changed what the misses
// cost. On experts with several bands (Mixtral, DiT) the hint made every
// launch slower (4-5%): their weights are read again by the other bands.
// MXFP4 weight rows are excluded: a stage takes 64 bytes of a row, half a
// 128-byte line, and the next stage the other half, which a streamed line no
// longer holds (the W4A8 share's Linear-1 183 -> 191 us with the hint).
__host__ __device__ constexpr bool streams_once(int OT) { return stage_kb_bytes(OT) == 128; }
constexpr int kCpolNT = 2;  // cache-policy operand of the global -> LDS load: nt

// global -> LDS loads issued per loader lane per stage: 16 bytes each, plus
// two 4-byte loads with e4m3 activations (the row scales and the weight
// scales). The band rows take a whole number of instructions per loader
// wavefront plus, when they do not divide evenly, one partial instruction in
// every loader wavefront.
__host__ __device__ constexpr int stage_a_rows_per_round(int OT) {
  return loader_waves(OT) * 64 * 16 / stage_k_bytes(OT);
}
__host__ __device__ constexpr int stage_b_rows_per_round(int OT) {
  return loader_waves(OT) * 64 * 16 / stage_kb_bytes(OT);
}
__host__ __device__ constexpr int stage_loads(int MB, int NNB, int OT) {
  return (MB * 32 + stage_a_rows_per_round(OT) - 1) / stage_a_rows_per_round(OT) +
         NNB * 64 / stage_b_rows_per_round(OT) + (OT ? 2 : 0);
}

// Wavefront grid of a tile of width NNB: WM wavefront rows x WN wavefront
// columns; each wavefront owns CPH = NNB / WN 32-column blocks in each half
// of the tile's weight rows (half = NNB * 32 rows: the gate rows of a
// Linear-1 tile, or the first half of a Linear-2 tile's output columns).
template <int NNB, int OT>
struct WaveGrid {
  static constexpr int W = gemm_threads(OT) / 64;
  static_assert(W == 4 || W == 8, "wavefront grid");
  static constexpr int WN = (W == 8 && NNB == 4) ? 4 : 2;
  static constexpr int WM = W / WN;
  static constexpr int CPH = NNB / WN;
  static constexpr int NCB = 2 * CPH;  // accumulator columns per wavefront
  static_assert(CPH >= 1, "a wavefront owns at least one block per half");
};

// Weight row (tile-relative) of column block c of half h owned by wavefront
// column wn, for lane row lr; the same index gives the output column.
template <int NNB, int OT>
__device__ __forceinline__ int wave_col(int h, int c, int wn, int lr) {
  return h * (NNB * 32) + (c * WaveGrid<NNB, OT>::WN + wn) * 32 + lr;
}

// 16-byte chunk c of row `row` in a stage of KB-byte rows. The chunk index is
// XOR-swizzled so that the 16 consecutive rows a 16-lane phase of
// ds_read_b128 touches spread over all 64 LDS banks (256 bytes): 128-byte rows
// pair up in a bank line, so the swizzle is (row / 2) mod 8.
template <int KB>
__device__ __forceinline__ int chunk_swizzle(int row) {
  static_assert(KB == 128 || KB == 64, "stage row size");
  // 64-byte rows (MXFP4 weights): four rows share a bank line, and a phase
  // reads one 16-byte chunk of 16 consecutive rows
  return KB == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}
template <int KB>
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * KB + ((chunk ^ chunk_swizzle<KB>(row)) << 4);
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

// One pipeline stage: K bytes [kt*KB, kt*KB+KB) of the band's first 32*MB
// rows and of the tile's NNB*64 weight rows (and, with fp8, the 256 row scales
// of K block kt and the block's two weight scales), in stage_loads(MB, NNB,
// OT) load instructions per lane:
// first the band rows, then the weight rows, then the scales. Lane i of a
// 16-byte instruction lands at LDS base + 16*i (64/CH rows of KB bytes, CH =
// KB/16 chunks per row), lane i of a 4-byte instruction at base + 4*i.
// issue_load issues instruction j of the stage; only the loader wavefronts
// call it (w below is the loader index). NT: the weight rows are loaded
// non-temporally (see streams_once).
template <int MB, int NNB, int OT, bool NT>
__device__ __forceinline__ void issue_load(const Tile& t, int kt, lds_t* st, int tid, int j) {
  constexpr int KB = stage_k_bytes(OT), CH = KB / 16, RPI = 64 / CH;
  constexpr int NW = loader_waves(OT), ROUND = NW * RPI;
  static_assert(ROUND == stage_a_rows_per_round(OT), "rows per load round");
  // weight rows: KBB bytes each (64 for MXFP4), RPIB rows per instruction
  constexpr int KBB = stage_kb_bytes(OT), CHB = KBB / 16, RPIB = 64 / CHB, ROUNDB = NW * RPIB;
  static_assert(ROUNDB == stage_b_rows_per_round(OT), "weight rows per load round");
  // NAF full rounds of band rows, then REM rows (a multiple of 32) spread over
  // the loader wavefronts: REM / NW rows each, the other lanes idle
  constexpr int NAF = MB * 32 / ROUND, REM = MB * 32 - NAF * ROUND, NA = NAF + (REM ? 1 : 0);
  constexpr int NBW = NNB * 64 / ROUNDB, half = NNB * 32;
  static_assert(NBW * ROUNDB == NNB * 64 && REM % NW == 0 && REM / NW <= RPI, "stage rows per wavefront");
  // (the wavefront index as a scalar: every instruction's rows then lie in
  // one half of the weight rows, whose base is a uniform choice)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) - (gemm_threads(OT) / 64 - NW), lane = tid & 63;
  if (j < NA) {
    constexpr int RPW = REM / NW;  // rows per wavefront in the partial round
    const int sub = lane / CH, slot = lane % CH;
    const bool part = REM && j == NAF;
    const int r0 = part ? NAF * ROUND + w * RPW : (j * NW + w) * RPI;
    const int r = r0 + sub;
    const uint8_t* g = t.A + (t.arow[j] + (uint32_t)(kt * KB + ((slot ^ chunk_swizzle<KB>(r)) << 4)));
    if (!part || sub < RPW) __builtin_amdgcn_global_load_lds(g, st + r0 * KB, 16, 0, 0);
  } else if (j < NA + NBW) {
    const int sub = lane / CHB, slot = lane % CHB;
    const int r0 = ((j - NA) * NW + w) * RPIB;
    const int r = r0 + sub;
    const uint8_t* base = r0 < half ? t.Bg : t.Bu;
    const uint8_t* g =
        base + (uint32_t)((r & (half - 1)) * (uint32_t)t.ldb + kt * KBB + ((slot ^ chunk_swizzle<KBB>(r)) << 4));
    __builtin_amdgcn_global_load_lds(g, st + stage_a_bytes(MB, OT) + r0 * KBB, 16, 0, NT ? kCpolNT : 0);
  } else if constexpr (OT != OT_BF16) {
    lds_t* ss = st + stage_a_bytes(MB, OT) + stage_b_bytes(NNB, OT);
    if (j == NA + NBW) {
      // the 256 row scales: kBM / NW per wavefront, one 4-byte lane each
      constexpr int PER = kBM / NW;
      const int r = w * PER + lane;
      const int gr = r < t.rows ? r : t.rows - 1;
      const float* g = t.As + (uint32_t)(kt * (uint32_t)t.cap_stride + gr);
      if (lane < PER) __builtin_amdgcn_global_load_lds(g, ss + w * PER * 4, 4, 0, 0);
    } else if constexpr (mxfp4_weights(OT)) {
      // the weight rows' E8M0 scales of this stage: one dword (four 32-wide
      // blocks) per weight row, NNB * 64 / NW rows per wavefront
      constexpr int PERB = NNB * 64 / NW;
      const int r = w * PERB + lane;
      const uint8_t* base = w * PERB < half ? t.Eg : t.Eu;
      const uint8_t* g = base + (uint32_t)((r & (half - 1)) * (uint32_t)t.epitch + kt * 4);
      if (lane < PERB) __builtin_amdgcn_global_load_lds(g, ss + kBM * 4 + w * PERB * 4, 4, 0, 0);
    } else {
      // the block's two weight scales (first and second half of the weight
      // rows) after the row scales. Every loader wavefront loads them, the
      // same 8 bytes, so that all loaders issue the same number of loads per
      // stage; kept in the stage, they need no scalar load in the MFMA loop.
      const float* g = lane == 0 ? t.Sg + kt : t.Su + kt;
      if (lane < 2) __builtin_amdgcn_global_load_lds(g, ss + kBM * 4, 4, 0, 0);
    }
  }
}

// The A (band) row each band-row load instruction j of this lane reads, as
// issue_load lays the stage out: rows past the band re-read its last row;
// with gathered rows, band row r is A row a_src[row0 + r] / a_k.
template <int MB, int NNB, int OT>
__device__ __forceinline__ void fill_arow(Tile& t, int tid) {
  constexpr int KB = stage_k_bytes(OT), CH = KB / 16, RPI = 64 / CH;
  constexpr int NW = loader_waves(OT), ROUND = NW * RPI;
  constexpr int NAF = MB * 32 / ROUND, REM = MB * 32 - NAF * ROUND, NA = NAF + (REM ? 1 : 0);
  static_assert(NA <= 8, "band-row load instructions per stage");
  const int w = (tid >> 6) - (gemm_threads(OT) / 64 - NW), sub = (tid & 63) / CH;
  if (w < 0) return;  // not a loader
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    constexpr int RPW = REM / NW;
    const bool part = REM && j == NAF;
    const int r = (part ? NAF * ROUND + w * RPW : (j * NW + w) * RPI) + sub;
    const int gr = r < t.rows ? r : t.rows - 1;
    // gathered: X row a_src[row0 + r] / k from X; else band row r from the
    // band's first row (t.A points there). 32 bits suffice: the problem
    // limits keep cap * d and cap * f (cap >= T) below 2^31 elements of at
    // most 2 bytes.
    t.arow[j] = (uint32_t)(t.a_src ? t.a_src[t.row0 + gr] / t.a_k : gr) * (uint32_t)t.lda;
  }
}

// The K loop of every Linear-2 tile of local expert e starts at slice
// (e * kKRot) mod ktiles and wraps around. The tiles running at the same time
// on different XCDs (different experts' bands) then stream different column
// offsets of their weight rows; at a power-of-two row pitch (W2 rows of 2 f
// bytes) they would otherwise all hit the same HBM channels together.
// Measured: the Linear-2 launch of the DeepSeek-style share (4 KiB rows)
// 10-13% faster; Linear-1, whose rows are d elements long, gained nothing and
// does not rotate. The start depends on the expert alone, not on the band a
// row falls in, so every output element is summed in one fixed K order
// whatever the tile width, schedule, grid or the order of the tokens.
constexpr int kKRot = 5;

// K slice streamed by pipeline stage kt of tile t.
__device__ __forceinline__ int kslice(const Tile& t, int kt) {
  const int s = kt + t.krot;
  return s >= t.ktiles ? s - t.ktiles : s;
}

template <int MB, int NNB, int OT, bool NT>
__device__ __forceinline__ void issue_stage(const Tile& t, int kt, lds_t* st, int tid) {
  const int ks = kslice(t, kt);
#pragma unroll
  for (int j = 0; j < stage_loads(MB, NNB, OT); ++j) issue_load<MB, NNB, OT, NT>(t, ks, st, tid, j);
}

// MFMAs of one stage for a wavefront that owns NMB row blocks {wm, wm+2, ...}
// and weight rows {nb*64 + wn*32 .. +32} for nb = 0 .. NNB-1.
// The K order inside a stage is a permutation shared by both operands (lane
// half h of an MFMA reads the same chunk indices of its A row and B row), so
// the sum over K is unchanged.
// The weight rows are the MFMA's A operand and the band rows its B operand,
// so each 32x32 accumulator holds the transposed block: lane l has band row
// l % 32 and, in elements 4q .. 4q+3, the four consecutive output columns
// 8q + 4 (l / 32) + 0..3. The epilogue then stores four columns of one row
// per instruction (16 bytes of fp32, 8 of bf16) instead of one.
// A loader wavefront (split loads) passes NL > 0 and issue(j) for the
// next stage's load instructions j = 0 .. NL-1, issued in NP batches at the
// starts of evenly spaced K steps. Measured (Linear-1 and
// Linear-2 together, same box): for loaders owning 4 row blocks (the
// 256-row bands of the compute-bound Mixtral and DiT shapes) one batch at
// the start of the stage is best (+2% and +4.6% on the GEMM against all
// wavefronts loading before the barrier; 4 or 16 batches were 2% slower
// than one); for loaders owning 2 (the bandwidth-bound DeepSeek-style bands
// of about 126 rows) four batches are (+1.5%; one batch +0.4%). Each batch
// is an ordering point for the LDS fragment reads after it, so the stage
// reads K step ks+1's fragments into a second register set before the batch
// and the MFMAs of step ks: Mixtral 1050 -> 1106 TFLOP/s, the DiT GEMM 1920
// -> 1856 us against fragments read just in time.
template <int NMB>
constexpr int load_points() { return NMB >= 3 ? 1 : 4; }
struct NoLoads {
  __device__ void operator()(int) const {}
};
template <int NMB, int NNB, int NL = 0, class Issue = NoLoads>
__device__ __forceinline__ void compute_stage(const lds_t* sa, const lds_t* sb, int tid,
                                              f32x16 (&acc)[NMB][WaveGrid<NNB, false>::NCB],
                                              const Issue& issue = Issue()) {
  using G = WaveGrid<NNB, false>;
  constexpr int KB = stage_k_bytes(false), NKS = KB / 32;
  const int lane = tid & 63, w = tid >> 6, wm = w % G::WM, wn = w / G::WM;
  const int lr = lane & 31, hi = lane >> 5;
  // fragments of K step ks+1 are read before the load batch and the MFMAs of
  // step ks, so no load issue stands between a fragment read and its MFMA
  bf16x8 fb[2][G::NCB], fa[2][NMB];
  auto read = [&](int ks, int buf) {
    const int chunk = ks * 2 + hi;
#pragma unroll
    for (int nb = 0; nb < G::NCB; ++nb)
      fb[buf][nb] = *(const lds_bf16x8*)(sb + lds_off<KB>(wave_col<NNB, false>(nb / G::CPH, nb % G::CPH, wn, lr), chunk));
#pragma unroll
    for (int mi = 0; mi < NMB; ++mi)
      fa[buf][mi] = *(const lds_bf16x8*)(sa + lds_off<KB>((wm + G::WM * mi) * 32 + lr, chunk));
  };
  read(0, 0);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks + 1 < NKS) read(ks + 1, (ks + 1) & 1);
    if constexpr (NL > 0) {
      constexpr int NP = load_points<NMB>() < NKS ? load_points<NMB>() : NKS;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (ks == p * NKS / NP)
#pragma unroll
          for (int j = p * NL / NP; j < (p + 1) * NL / NP; ++j) issue(j);
    }
#pragma unroll
    for (int mi = 0; mi < NMB; ++mi)
#pragma unroll
      for (int nb = 0; nb < G::NCB; ++nb)
        acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][nb], fa[ks & 1][mi], acc[mi][nb], 0, 0, 0);
  }
}

__device__ __forceinline__ i32x8 lds_read_32B(const lds_t* base, int row, int chunk0) {
  const i32x4 lo = *(const lds_i32x4*)(base + lds_off<128>(row, chunk0));
  const i32x4 hi = *(const lds_i32x4*)(base + lds_off<128>(row, chunk0 + 1));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// fp8 stage: the stage is exactly one 128-wide K block, so the block's MFMA
// sum (two v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales) is
// promoted into the fp32 accumulator with the row's activation scale times
// the weight block's scale: acc += partial * sx[row] * sw, with sw = swg for
// the first half of the weight rows and swu for the second. As in the bf16
// stage, the weight rows are the MFMA's A operand, so the accumulators hold
// transposed blocks (a lane has one band row).
template <int NMB, int NNB>
__device__ __forceinline__ void compute_stage_fp8(const lds_t* sa, const lds_t* sb, const lds_t* ss, float swg,
                                                  float swu, int tid, f32x16 (&acc)[NMB][WaveGrid<NNB, true>::NCB]) {
  using G = WaveGrid<NNB, true>;
  const int lane = tid & 63, w = tid >> 6, wm = w % G::WM, wn = w / G::WM;
  const int lr = lane & 31, hi = lane >> 5;
  const f32x16 zero = {};
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int mb = wm + G::WM * mi;
    f32x16 part[G::NCB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i32x8 a = lds_read_32B(sa, mb * 32 + lr, ks * 4 + hi * 2);
#pragma unroll
      for (int nb = 0; nb < G::NCB; ++nb) {
        // weight fragments are read per row block, not kept: with two
        // wavefronts per SIMD a wavefront has 256 registers
        const i32x8 b = lds_read_32B(sb, wave_col<NNB, true>(nb / G::CPH, nb % G::CPH, wn, lr), ks * 4 + hi * 2);
        part[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, ks ? part[nb] : zero, 0, 0, 0, 127, 0, 127);
      }
    }
    // transposed blocks (weights as the A operand): the lane's one row of
    // block mb is mb*32 + lr, so one activation scale serves all 16 elements
    const float sx = *(const lds_f32*)(ss + (mb * 32 + lr) * 4);
    const float sg = sx * swg, su = sx * swu;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int nb = 0; nb < G::NCB; ++nb) acc[mi][nb][i] = fmaf(part[nb][i], nb < G::CPH ? sg : su, acc[mi][nb][i]);
  }
}

// MXFP4-weight stage: one 128-wide K block of e4m3 activations against E2M1
// weights. The scaled MFMA applies each lane's E8M0 byte to the values that
// lane holds, so in each 64-wide step lane half h (lanes 32h .. 32h + 31)
// holds 32 consecutive K values of its weight row, elements [32h, 32h + 32)
// of the step: one MX block, whose scale it passes. The matrix unit pairs
// the 4-bit operand's first 16 values with K positions [16h, 16h + 16) of
// the e4m3 operand and its next 16 with [32 + 16h, +16), so the activation
// fragment of lane half h is chunks h and 2 + h of the step (16 bytes each),
// not chunks 2h and 2h + 1 as in the fp8 x fp8 product. (Measured on gfx950
// with one-hot products, the 4-bit operand in the B position; the pairing is
// the operand formats', and holds with the 4-bit operand as A, where it sits
// now for the transposed accumulators: the W4A8 parity tests compare every
// element.) The activation side runs at unit scale and the stage's partial
// sum is promoted with the row's fp32 activation scale: acc += partial * sx.
template <int NMB, int NNB>
__device__ __forceinline__ void compute_stage_w4(const lds_t* sa, const lds_t* sb, const lds_t* ss, int tid,
                                                 f32x16 (&acc)[NMB][WaveGrid<NNB, OT_W4A8>::NCB]) {
  using G = WaveGrid<NNB, OT_W4A8>;
  const int lane = tid & 63, w = tid >> 6, wm = w % G::WM, wn = w / G::WM;
  const int lr = lane & 31, hi = lane >> 5;
  const f32x16 zero = {};
  // the scale dword (four E8M0 bytes, one per 32-wide block) of each weight
  // row this lane holds, read once per stage
  int sw[G::NCB];
#pragma unroll
  for (int nb = 0; nb < G::NCB; ++nb)
    sw[nb] = *(const lds_i32*)(ss + kBM * 4 + wave_col<NNB, OT_W4A8>(nb / G::CPH, nb % G::CPH, wn, lr) * 4);
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int mb = wm + G::WM * mi;
    f32x16 part[G::NCB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i32x4 a0 = *(const lds_i32x4*)(sa + lds_off<128>(mb * 32 + lr, ks * 4 + hi));
      const i32x4 a1 = *(const lds_i32x4*)(sa + lds_off<128>(mb * 32 + lr, ks * 4 + 2 + hi));
      const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int nb = 0; nb < G::NCB; ++nb) {
        const int row = wave_col<NNB, OT_W4A8>(nb / G::CPH, nb % G::CPH, wn, lr);
        const i32x4 q = *(const lds_i32x4*)(sb + lds_off<64>(row, ks * 2 + hi));
        const i32x8 b = {q[0], q[1], q[2], q[3], 0, 0, 0, 0};
        const int sc = (sw[nb] >> (8 * (ks * 2 + hi))) & 0xFF;
        // the E2M1 weights as the A operand (cbsz = 4, with their E8M0
        // scale), the e4m3 activations as B (blgp = 0, unit scale)
        part[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, ks ? part[nb] : zero, 4, 0, 0, sc, 0, 127);
      }
    }
    // transposed blocks: one activation scale (row mb*32 + lr) per lane
    const float sx = *(const lds_f32*)(ss + (mb * 32 + lr) * 4);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int nb = 0; nb < G::NCB; ++nb) acc[mi][nb][i] = fmaf(part[nb][i], sx, acc[mi][nb][i]);
  }
}

template <int MB, int NMB, int NNB, int OT>
__device__ __forceinline__ void compute_any(const Tile& t, const lds_t* st, int kt, int tid,
                                            f32x16 (&acc)[NMB][WaveGrid<NNB, OT>::NCB]) {
  if constexpr (mxfp4_weights(OT)) {
    const lds_t* ss = st + stage_a_bytes(MB, OT) + stage_b_bytes(NNB, OT);
    compute_stage_w4<NMB, NNB>(st, st + stage_a_bytes(MB, OT), ss, tid, acc);
  } else if constexpr (OT) {
    static_assert(stage_k_bytes(true) == 128, "an fp8 stage is one 128-wide scale block");
    const lds_t* ss = st + stage_a_bytes(MB, OT) + stage_b_bytes(NNB, OT);
    const float swg = *(const lds_f32*)(ss + kBM * 4), swu = *(const lds_f32*)(ss + kBM * 4 + 4);
    compute_stage_fp8<NMB, NNB>(st, st + stage_a_bytes(MB, OT), ss, swg, swu, tid, acc);
  } else {
    compute_stage<NMB, NNB>(st, st + stage_a_bytes(MB, OT), tid, acc);
  }
}

// Whether a Linear-1 tile owns whole 128-column quantisation blocks of H
// (e4m3 H, wide tiles) and stages them in LDS.
template <int NNB, bool L1, int OT>
constexpr bool stages_block_in_lds() { return OT && L1 && NNB * 32 == 128; }

// The accumulators hold transposed blocks (the compute stages take the
// weight rows as the MFMA's A operand), so lane l owns band row l % 32 of
// each row block and, in elements 4q .. 4q+3, four consecutive output
// columns 8q + 4 (l / 32) + 0..3.
// fp8 / MXFP4 Linear-1 tiles of the wide width own a whole 128-column
// quantisation block: they stage its fp32 SwiGLU values in the (free) LDS
// ring as [rows][128] floats and quantise from there (quantize_block_from);
// narrow ones store them to H_f32 and pair up through blk_done.
// SwiGLU of one output element, silu(g) * u = g u / (1 + e^-g), with the
// hardware exp2 and reciprocal (about 1 ulp each, no IEEE division). Its error
// of a few fp32 ulp is far below the bf16 rounding or e4m3 quantisation of H
// that follows, and the exact expf and division cost epilogue time: DiT
// 750 -> 767 TFLOP/s, Mixtral 1110 -> 1131. For g below about -88.7 the
// exponential overflows and the result is a signed zero, where the exact
// value is below 1e-36 in magnitude.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}

template <int NMB, int NNB, bool L1, int OT>
__device__ __forceinline__ void epilogue_rows(const GemmParams& P, const Tile& t, int tid,
                                              const f32x16 (&acc)[NMB][WaveGrid<NNB, OT>::NCB], lds_t* lds) {
  using G = WaveGrid<NNB, OT>;
  const int lane = tid & 63, w = tid >> 6, wm = w % G::WM, wn = w / G::WM;
  const int lr = lane & 31, hi = lane >> 5;
  // Linear-2: every row's destination is loaded before the first store. As
  // far as the compiler knows a store may alias row_dst, so a load placed
  // after one waits for a memory round trip of its own, once per row block.
  int dsts[NMB];
  if constexpr (!L1) {
#pragma unroll
    for (int mi = 0; mi < NMB; ++mi) {
      const int m = (wm + G::WM * mi) * 32 + lr;
      dsts[mi] = m < t.rows ? P.row_dst[t.row0 + m] : 0;
    }
  }
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int m = (wm + G::WM * mi) * 32 + lr;
    if (m >= t.rows) continue;
    if constexpr (L1 && OT != OT_BF16) {
      // gate block c pairs with up block c of the second half: the same SwiGLU columns
      float* frow = P.Hf + (size_t)(t.row0 + m) * P.f + t.n * (NNB * 32);
#pragma unroll
      for (int c = 0; c < G::CPH; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = acc[mi][c][4 * q + e], u = acc[mi][G::CPH + c][4 * q + e];
            a[e] = silu_mul(g, u);
          }
          const int cb = wave_col<NNB, OT>(0, c, wn, 0) + 8 * q + 4 * hi;
          const float4 v = make_float4(a[0], a[1], a[2], a[3]);
          if constexpr (stages_block_in_lds<NNB, L1, OT>()) {
            *reinterpret_cast<lds_f32x4*>(lds + (m * 128 + cb) * 4) = f32x4{a[0], a[1], a[2], a[3]};
            if (P.keep_hf) *reinterpret_cast<float4*>(frow + cb) = v;
          } else {
            *reinterpret_cast<float4*>(frow + cb) = v;  // quantised once both halves are stored
          }
        }
      }
    } else if constexpr (L1) {
      // gate block c pairs with up block c of the second half: the same SwiGLU columns
      uint16_t* hrow = reinterpret_cast<uint16_t*>(P.H) + (size_t)(t.row0 + m) * P.f + t.n * (NNB * 32);
#pragma unroll
      for (int c = 0; c < G::CPH; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t packed[2];
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float g0 = acc[mi][c][4 * q + e], u0 = acc[mi][G::CPH + c][4 * q + e];
            const float g1 = acc[mi][c][4 * q + e + 1], u1 = acc[mi][G::CPH + c][4 * q + e + 1];
            const float a0 = silu_mul(g0, u0), a1 = silu_mul(g1, u1);
            packed[e / 2] = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
          }
          const int col = wave_col<NNB, OT>(0, c, wn, 0) + 8 * q + 4 * hi;
          *reinterpret_cast<uint2*>(hrow + col) = make_uint2(packed[0], packed[1]);
        }
      }
    } else {
      // a destination row outside the buffer (a caller's row_dst) is not
      // stored but reported
      const int dst = dsts[mi];
      if ((unsigned)dst >= (unsigned)P.cap) {
        __hip_atomic_fetch_or(P.meta + META_ARG_ERR, (int)ARG_ERR_ROW_DST, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        continue;
      }
#pragma unroll
      for (int nb = 0; nb < G::NCB; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = t.n * (NNB * 64) + wave_col<NNB, OT>(nb / G::CPH, nb % G::CPH, wn, 0) + 8 * q + 4 * hi;
          const float v[4] = {acc[mi][nb][4 * q], acc[mi][nb][4 * q + 1], acc[mi][nb][4 * q + 2],
                              acc[mi][nb][4 * q + 3]};
          if (P.c_bf16) {
            const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
            const uint32_t up = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.C) + (size_t)dst * P.d + col) = make_uint2(lo, up);
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(P.C) + (size_t)dst * P.d + col) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }
}

// Orders a wavefront's LDS accesses on either side of it, for values that
// other lanes of the same wavefront wrote or still read.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Linear-2 outputs (fp32) through the LDS, for a tile after which the ring is
// free. A lane holds four consecutive columns of one row, so a direct store
// instruction writes 32 bytes into each of 32 rows; such stores issue at
// about 24 GB/s per CU (the DiT and Mixtral epilogues: 256 KiB in 10-11 us).
// Here each wavefront moves one 32 x 32 block at a time through its own
// 4 KiB of LDS (16-byte chunks XOR-swizzled by row) and reads it back eight
// rows per instruction, so that every store writes whole 128-byte lines.
template <int NMB, int NNB, int OT>
__device__ __forceinline__ void epilogue_l2_staged(const GemmParams& P, const Tile& t, int tid,
                                                   const f32x16 (&acc)[NMB][WaveGrid<NNB, OT>::NCB], lds_t* lds) {
  using G = WaveGrid<NNB, OT>;
  const int lane = tid & 63, w = tid >> 6, wm = w % G::WM, wn = w / G::WM;
  const int lr = lane & 31, hi = lane >> 5;
  const int sr = lane >> 3, sc = lane & 7;  // read-back: rows sr + 8 j, 16-byte chunk sc
  lds_t* wl = lds + w * 4096;
  float* C = reinterpret_cast<float*>(P.C);
  int dsts[NMB];
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int m = (wm + G::WM * mi) * 32 + lr;
    dsts[mi] = m < t.rows ? P.row_dst[t.row0 + m] : -1;
  }
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    const int m = (wm + G::WM * mi) * 32 + lr;
    int dst = dsts[mi];
    // a destination row outside the buffer (a caller's row_dst) is not
    // stored but reported
    if (m < t.rows && (unsigned)dst >= (unsigned)P.cap)
      __hip_atomic_fetch_or(P.meta + META_ARG_ERR, (int)ARG_ERR_ROW_DST, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((unsigned)dst >= (unsigned)P.cap) dst = -1;
    int rdst[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rdst[j] = __shfl(dst, sr + 8 * j, 64);
#pragma unroll
    for (int nb = 0; nb < G::NCB; ++nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<lds_f32x4*>(wl + lr * 128 + (((2 * q + hi) ^ (lr & 7)) << 4)) =
            f32x4{acc[mi][nb][4 * q], acc[mi][nb][4 * q + 1], acc[mi][nb][4 * q + 2], acc[mi][nb][4 * q + 3]};
      wave_lds_sync();
      f32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = sr + 8 * j;
        v[j] = *reinterpret_cast<lds_f32x4*>(wl + r * 128 + ((sc ^ (r & 7)) << 4));
      }
      wave_lds_sync();
      const int col = t.n * (NNB * 64) + wave_col<NNB, OT>(nb / G::CPH, nb % G::CPH, wn, 0) + 4 * sc;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (rdst[j] >= 0)
          *reinterpret_cast<float4*>(C + (size_t)rdst[j] * P.d + col) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
    }
  }
}

// stage: the LDS ring is free (no successor stages were issued into it), and
// the caller runs a workgroup barrier after this before the ring is refilled.
template <int NMB, int NNB, bool L1, int OT>
__device__ __forceinline__ void epilogue(const GemmParams& P, const Tile& t, int tid,
                                         const f32x16 (&acc)[NMB][WaveGrid<NNB, OT>::NCB], lds_t* lds, bool stage) {
  if constexpr (!L1) {
    if (stage) {
      epilogue_l2_staged<NMB, NNB, OT>(P, t, tid, acc, lds);
      return;
    }
  }
  epilogue_rows<NMB, NNB, L1, OT>(P, t, tid, acc, lds);
}

// Drain the last R+1 stages of the ring: stage kt is complete once at most R
// stages (R * stage_loads loads per lane) are still in flight.
template <int MB, int NMB, int NNB, int OT, int R>
__device__ __forceinline__ void drain(const Tile& t, lds_t* lds, int rd, int kt, int tid,
                                      f32x16 (&acc)[NMB > 0 ? NMB : 1][WaveGrid<NNB, OT>::NCB]) {
  constexpr int S = ring_stages(MB, NNB, OT), SB = stage_bytes(MB, NNB, OT);
  wait_vmcnt<R * stage_loads(MB, NNB, OT)>();
  lds_barrier();
  if constexpr (NMB > 0) compute_any<MB, NMB, NNB, OT>(t, lds + rd * SB, kt, tid, acc);
  if constexpr (R > 0) drain<MB, NMB, NNB, OT, R - 1>(t, lds, rd + 1 == S ? 0 : rd + 1, kt + 1, tid, acc);
}

// The whole tile: every wavefront runs the same barriers and owns NMB of the
// MB row blocks; the loader wavefronts also issue the ring's loads. The
// accumulators stay inside this function.
// The LDS ring has ring_stages(MB, NNB) stages of stage_bytes(MB, NNB): as
// many as fit in 160 KiB (at least 2), so that S-1 stages are in flight per CU.
// The thread index is made opaque to the optimiser at the start of the tile:
// the per-lane address offsets derived from it (row * pitch products)
// are then computed once per tile instead of being hoisted, for every tile
// shape of the persistent loop at once, to the kernel entry where they would
// stay live (and spill) for the whole launch.
// Cross-tile prefetch (bf16 tiles of at most four row blocks, separate
// schedule): a tile whose successor on the same workgroup has its shape (row
// blocks and width) issues the successor's first ring stages after its own
// K loop, before its epilogue, so that the stores and the next loads
// overlap. Measured (same box): the DeepSeek-style share's GEMM (bands of
// about 126 rows) 589 -> 583 us; on 256-row tiles it paid nothing (DiT: the
// Linear-2 epilogue slowed from 10.8 to 11.4 us, its stores queued behind
// the loads, as much as the K loop gained) or lost (Mixtral's GEMM 1.8%
// slower), so those tiles do not prefetch. `next` is the
// successor if `has_next`, `issued` reports whether its stages were issued,
// `pre` tells a tile that its own first stages are already in flight.
struct Chain {
  Tile next;
  bool has_next = false;
  bool pre = false;
  bool issued = false;
};

// Roles of a wavefront in the K loop: a loader (ROLE_LOADER) or not
// (ROLE_COMPUTE). The role is a template parameter, chosen once per tile, so
// that each role's K loop is straight-line code with its own accumulators.
enum { ROLE_LOADER = 1, ROLE_COMPUTE = 2 };

template <int MB, int NMB, int NNB, bool L1, int OT, int ROLE, bool NT>
__device__ __forceinline__ void tile_body(const GemmParams& P, const Tile& t0, lds_t* lds, uint64_t& t_main,
                                          Chain& ch) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  Tile t = t0;
  fill_arow<MB, NNB, OT>(t, tid);
  constexpr int S = ring_stages(MB, NNB, OT), SB = stage_bytes(MB, NNB, OT), LD = stage_loads(MB, NNB, OT);
  static_assert(S >= 2, "the LDS ring needs two stages");
  f32x16 acc[NMB > 0 ? NMB : 1][WaveGrid<NNB, OT>::NCB];
#pragma unroll
  for (int a = 0; a < (NMB > 0 ? NMB : 1); ++a)
#pragma unroll
    for (int b = 0; b < WaveGrid<NNB, OT>::NCB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  const int KT = t.ktiles;
  constexpr bool loader = ROLE == ROLE_LOADER;
  // A tile whose first stages its predecessor issued waits for all of them
  // (and the predecessor's epilogue stores, issued after them) at once.
  if (ch.pre) wait_vmcnt<0>();
  if (KT < S) {
    // the whole K extent fits in the ring
    if constexpr (loader) {
      if (!ch.pre)
        for (int kt = 0; kt < KT; ++kt) issue_stage<MB, NNB, OT, NT>(t, kt, lds + kt * SB, tid);
    }
    wait_vmcnt<0>();
    lds_barrier();
    if constexpr (NMB > 0)
      for (int kt = 0; kt < KT; ++kt) compute_any<MB, NMB, NNB, OT>(t, lds + kt * SB, kt, tid, acc);
  } else {
    if constexpr (loader) {
      if (!ch.pre) {
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue_stage<MB, NNB, OT, NT>(t, s, lds + s * SB, tid);
      }
    }
    int rd = 0, wr = S - 1, kt = 0;
    for (; kt + S - 1 < KT; ++kt) {
      // One barrier per step. It shows stage kt complete (each loader waited
      // for its own loads of it) and every wavefront done with stage kt-1,
      // whose slot wr the loaders then refill while the other wavefront of
      // their SIMD already runs this stage's MFMAs. (With every wavefront
      // issuing its share of the refill before the step's wait, a second
      // barrier closed each step and the issue and the MFMAs ran one after
      // the other: see loader_waves.)
      wait_vmcnt<(S - 2) * LD>();  // a loader's loads of stage kt have landed
      lds_barrier();               // ... every loader's
      if constexpr (loader) {
        const int ks = kslice(t, kt + S - 1);
        lds_t* st = lds + wr * SB;
        if constexpr (NMB > 0 && OT == OT_BF16) {
          compute_stage<NMB, NNB, LD>(lds + rd * SB, lds + rd * SB + stage_a_bytes(MB, OT), tid, acc,
                                      [&](int j) { issue_load<MB, NNB, OT, NT>(t, ks, st, tid, j); });
        } else {
          // e4m3 activations: the whole stage at once, then the MFMAs
#pragma unroll
          for (int j = 0; j < LD; ++j) issue_load<MB, NNB, OT, NT>(t, ks, st, tid, j);
          if constexpr (NMB > 0) compute_any<MB, NMB, NNB, OT>(t, lds + rd * SB, kt, tid, acc);
        }
      } else if constexpr (NMB > 0) {
        compute_any<MB, NMB, NNB, OT>(t, lds + rd * SB, kt, tid, acc);
      }
      rd = rd + 1 == S ? 0 : rd + 1;
      wr = wr + 1 == S ? 0 : wr + 1;
    }
    drain<MB, NMB, NNB, OT, S - 2>(t, lds, rd, kt, tid, acc);
  }
  lds_barrier();  // LDS ring free for the next tile
  if (P.trace) t_main = __builtin_amdgcn_s_memrealtime();
  if constexpr (OT == OT_BF16 && MB <= 4) {
    // the successor's first stages, if it has this tile's shape (the bf16
    // epilogue leaves the LDS alone, so the ring is free from here on)
    if (ch.has_next) {
      const Tile& n0 = ch.next;
      constexpr int WM = WaveGrid<NNB, OT>::WM;
      const int nmb = WM == 2 ? min((n0.rows + 31) >> 5, 8) : (n0.rows <= 128 ? 4 : 8);
      if (n0.nnb == NNB && nmb == MB && (streams_once(OT) && n0.once) == NT) {
        if constexpr (loader) {
          Tile tn = n0;
          fill_arow<MB, NNB, OT>(tn, tid);
          const int ns = tn.ktiles < S ? tn.ktiles : S - 1;
          for (int s = 0; s < ns; ++s) issue_stage<MB, NNB, OT, NT>(tn, s, lds + s * SB, tid);
        }
        ch.issued = true;
      }
    }
  }
  // Linear-2 stages its fp32 outputs through the free ring; every wavefront
  // (also one without row blocks) then meets at a barrier before the next
  // tile's loads refill the ring.
  const bool stage = !L1 && !ch.issued && !P.c_bf16;
  if constexpr (NMB > 0) epilogue<NMB, NNB, L1, OT>(P, t, tid, acc, lds, stage);
  if (stage) lds_barrier();
}

// MB = the band's 32-row blocks. With two wavefront rows (WM = 2) wavefront
// row 0 owns blocks {0, 2, ...}, i.e. ceil(MB / 2), and row 1 floor(MB / 2),
// so an odd count costs no MFMAs on absent blocks, and the stage (and with
// it the ring depth) is sized to the band: three 52 KiB stages of a 160-row
// band fit in the LDS where 192-row ones would leave two. With four
// wavefront rows MB is rounded up to a multiple of 4 (rows past the band
// re-read its last row and are not stored).
template <int MB, int NNB, bool L1, int OT, int ROLE, bool NT>
__device__ __forceinline__ void run_tile_role(const GemmParams& P, const Tile& t, lds_t* lds, uint64_t& t_main,
                                              Chain& ch) {
  constexpr int WM = WaveGrid<NNB, OT>::WM;
  if constexpr (WM == 2 && (MB & 1)) {
    if (((threadIdx.x >> 6) % WM) == 0) tile_body<MB, (MB + 1) / 2, NNB, L1, OT, ROLE, NT>(P, t, lds, t_main, ch);
    else tile_body<MB, MB / 2, NNB, L1, OT, ROLE, NT>(P, t, lds, t_main, ch);
  } else {
    static_assert(MB % WM == 0, "row blocks per wavefront row");
    tile_body<MB, MB / WM, NNB, L1, OT, ROLE, NT>(P, t, lds, t_main, ch);
  }
}

// The last loader_waves(OT) wavefronts take the loader role (the wavefront
// index through readfirstlane, so the role test is a uniform scalar branch).
template <int MB, int NNB, bool L1, int OT, bool NT>
__device__ __forceinline__ void run_tile(const GemmParams& P, const Tile& t, lds_t* lds, uint64_t& t_main,
                                         Chain& ch) {
  static_assert(loader_waves(OT) < gemm_threads(OT) / 64, "loaders and compute-only wavefronts");
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= gemm_threads(OT) / 64 - loader_waves(OT))
    run_tile_role<MB, NNB, L1, OT, ROLE_LOADER, NT>(P, t, lds, t_main, ch);
  else
    run_tile_role<MB, NNB, L1, OT, ROLE_COMPUTE, NT>(P, t, lds, t_main, ch);
}

template <int NNB, bool L1, int OT, bool NT>
__device__ __forceinline__ void dispatch_tile(const GemmParams& P, const Tile& t, lds_t* lds, uint64_t& t_main,
                                              Chain& ch) {
  if constexpr (WaveGrid<NNB, OT>::WM == 2) {
    switch ((t.rows + 31) >> 5) {
      case 1: run_tile<1, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      case 2: run_tile<2, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      case 3: run_tile<3, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      case 4: run_tile<4, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      case 5: run_tile<5, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      case 6: run_tile<6, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      case 7: run_tile<7, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
      default: run_tile<8, NNB, L1, OT, NT>(P, t, lds, t_main, ch); break;
    }
  } else {
    static_assert(WaveGrid<NNB, OT>::WM == 4, "wavefront rows");
    if (t.rows <= 128) run_tile<4, NNB, L1, OT, NT>(P, t, lds, t_main, ch);
    else run_tile<8, NNB, L1, OT, NT>(P, t, lds, t_main, ch);
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

// fp8: quantise column block j (128 SwiGLU columns) of a row band: per row,
// scale = amax / 448 (1 for an all-zero block) and code = e4m3(value /
// scale), round to nearest even. 16 lanes per row (8 values each), one row
// per 16 threads per pass; the loads of four passes are issued before any is
// used.
// The values come from Hf (in HBM) or, for a block a wide tile staged, from
// the LDS ring ([rows][128] floats); the arithmetic is the same.
template <bool FROM_LDS>
__device__ __forceinline__ void quantize_block_from(const GemmParams& P, int row0, int rows, int j,
                                                    const lds_t* lds) {
  constexpr int RPP = gemm_threads(true) / 16;  // rows per pass
  const int rr = threadIdx.x >> 4, q = threadIdx.x & 15;
  const int col = j * 128 + q * 8;
  for (int base = 0; base < rows; base += 4 * RPP) {
    float4 v[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + u * RPP + rr;
      if (r < rows) {
        if constexpr (FROM_LDS) {
          typedef __attribute__((address_space(3))) const float lds_f;
          lds_f* src = reinterpret_cast<lds_f*>(lds) + r * 128 + q * 8;
          v[u][0] = make_float4(src[0], src[1], src[2], src[3]);
          v[u][1] = make_float4(src[4], src[5], src[6], src[7]);
        } else {
          const float4* src = reinterpret_cast<const float4*>(P.Hf + (size_t)(row0 + r) * P.f + col);
          v[u][0] = src[0];
          v[u][1] = src[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + u * RPP + rr;
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

__device__ void quantize_block(const GemmParams& P, int row0, int rows, int j) {
  quantize_block_from<false>(P, row0, rows, j, nullptr);
}

// After a Linear-1 tile's stores. bf16 (fused schedules only): count the tile
// in l2_full[p]; the band is ready at N1. fp8: the 128-column block j is
// covered by 128 / (32 nnb1) tiles (2 narrow, 1 wide). A wide tile staged
// its block in the LDS ring (the epilogue) and quantises it from there, with
// no round trip through HBM and no device-scope counter. Narrow tiles each count themselves in blk_done[p][j] at
// device scope, and the second (every Hf store of the block is then
// published) quantises it. In the fused schedules the quantised block is
// counted in l2_full[p]; the band is ready at f / 128. The separate schedule
// needs no counting for Linear-2: its launch starts after this one ends.
template <int OT>
__device__ __forceinline__ void finish_l1_tile(const GemmParams& P, const Tile& t, int p, bool fused, lds_t* lds) {
  if constexpr (!OT) {
    if (fused) publish(P.l2_full + p, 1);
  } else {
    const int bn1 = t.nnb * 32;
    const int j = (t.n * bn1) >> 7;
    const int need = 128 / bn1;
    if (need == 1) {
      __syncthreads();  // every wave's values are in the LDS block
      quantize_block_from<true>(P, t.row0, t.rows, j, lds);
      __syncthreads();  // the ring is reused by the next tile
      if (fused) publish(P.l2_full + p, 1);
      return;
    }
    __attribute__((address_space(3))) int* flag = (__attribute__((address_space(3))) int*)lds;
    const int old = publish(P.blk_done + (size_t)p * (P.f >> 7) + j, 1);
    if (threadIdx.x == 0) *flag = old;
    __syncthreads();
    const bool second = *flag == need - 1;
    __syncthreads();  // the ring (and the flag in it) is reused by the next tile
    if (second) {
      quantize_block(P, t.row0, t.rows, j);
      if (fused) publish(P.l2_full + p, 1);
    }
  }
}

// After a Linear-2 tile's stores, with P.row_done set: publish the tile's
// output elements per 32-row block of rows (row_done[b] += rows of the tile
// in block b times its output columns). A block of the layout is complete
// once it counts min(32, R - 32 b) * d. This is the tile-level signal of Cui
// et al., Section 3.3.1 (a flag published after each output tile), counted
// per row block so that a reader needs no knowledge of the tile order.
__device__ __forceinline__ void finish_l2_tile(const GemmParams& P, const Tile& t) {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int cols = t.nnb * 64, r1 = t.row0 + t.rows;
    for (int b = t.row0 >> 5; b <= (r1 - 1) >> 5; ++b) {
      if (b >= P.row_done_len) break;
      const int lo = t.row0 > (b << 5) ? t.row0 : (b << 5);
      const int hi = r1 < (b << 5) + 32 ? r1 : (b << 5) + 32;
      __hip_atomic_fetch_add(P.row_done + b, (hi - lo) * cols, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Tile timing (P.trace set): once every wavefront's epilogue stores (and
// publication) are done, thread 0 takes a record slot from the device-scope
// counter meta[META_TRACE_N] and writes the tile's four clock readings and
// its identity. The extra barrier makes t_end the time the whole tile left
// the CU.
__device__ __forceinline__ void record_tile(const GemmParams& P, bool l1, int p, int n, int nnb, uint64_t t_start,
                                            uint64_t t_ready, uint64_t t_main) {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    const int slot = __hip_atomic_fetch_add(P.meta + META_TRACE_N, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (slot < P.trace_cap) {
      uint64_t* r = P.trace + (size_t)slot * 5;
      r[0] = t_start;
      r[1] = t_ready;
      r[2] = t_main;
      r[3] = t_end;
      r[4] = (uint64_t)(l1 ? 1 : 2) | ((uint64_t)nnb << 2) | ((uint64_t)blockIdx.x << 8) | ((uint64_t)n << 24) |
             ((uint64_t)p << 40);
    }
  }
}

template <bool L1, int OT>
__device__ __forceinline__ Tile make_tile(const GemmParams& P, int p, int n, int nnb) {
  constexpr int esz = OT ? 1 : 2;
  Tile t;
  const int eb = P.band_expert[p], e = eb & kBandExpertMask;
  t.once = (eb & kBandSingle) != 0;
  t.row0 = P.band_row0[p];
  t.rows = P.band_rows[p];
  t.n = n;
  t.nnb = nnb;
  t.cap_stride = P.cap;
  // weight rows: K elements of esz bytes, or K/2 bytes of packed MXFP4
  constexpr bool W4 = mxfp4_weights(OT);
  if constexpr (L1) {
    const int bn = nnb * 32;  // SwiGLU columns: bn gate rows and bn up rows
    t.lda = (size_t)P.d * esz;
    t.ldb = W4 ? (size_t)P.d / 2 : (size_t)P.d * esz;
    // rows by t.arow: X row a_src[row0 + r] / k from X itself, or X_perm row
    // row0 + r from the band's first row
    t.A = P.a_src ? P.X : P.X + (size_t)t.row0 * t.lda;
    t.a_src = P.a_src;
    t.a_k = P.a_k;
    const uint8_t* We = P.W1 + (size_t)e * 2 * P.f * t.ldb;
    t.Bg = We + (size_t)(n * bn) * t.ldb;
    t.Bu = We + (size_t)(P.f + n * bn) * t.ldb;
    t.ktiles = P.d * esz / stage_k_bytes(OT);
    t.krot = 0;
    if constexpr (W4) {
      t.As = P.Xs + t.row0;
      t.epitch = (size_t)P.d / 32;
      const uint8_t* Es = P.W1e + (size_t)e * 2 * P.f * t.epitch;
      t.Eg = Es + (size_t)(n * bn) * t.epitch;
      t.Eu = Es + (size_t)(P.f + n * bn) * t.epitch;
    } else if constexpr (OT) {
      const int db = P.d >> 7, fb2 = (2 * P.f) >> 7;
      t.As = P.Xs + t.row0;
      t.Sg = P.W1s + ((size_t)e * fb2 + (n * bn) / 128) * db;
      t.Su = P.W1s + ((size_t)e * fb2 + (P.f + n * bn) / 128) * db;
    }
  } else {
    const int bn = nnb * 64;  // output columns
    t.lda = (size_t)P.f * esz;
    t.ldb = W4 ? (size_t)P.f / 2 : (size_t)P.f * esz;
    t.A = P.H + (size_t)t.row0 * t.lda;
    t.a_src = nullptr;
    t.a_k = 1;
    t.Bg = P.W2 + ((size_t)e * P.d + (size_t)n * bn) * t.ldb;
    t.Bu = t.Bg + (size_t)(bn / 2) * t.ldb;
    t.ktiles = P.f * esz / stage_k_bytes(OT);
    t.krot = (e * kKRot) % t.ktiles;
    if constexpr (W4) {
      t.As = P.Hs + t.row0;
      t.epitch = (size_t)P.f / 32;
      t.Eg = P.W2e + ((size_t)e * P.d + (size_t)n * bn) * t.epitch;
      t.Eu = t.Eg + (size_t)(bn / 2) * t.epitch;
    } else if constexpr (OT) {
      t.As = P.Hs + t.row0;
      t.Sg = P.W2s + ((size_t)e * (P.d >> 7) + (n * bn) / 128) * (P.f >> 7);
      t.Su = P.W2s + ((size_t)e * (P.d >> 7) + (n * bn + bn / 2) / 128) * (P.f >> 7);
    }
  }
  return t;
}

template <bool L1, int OT>
__device__ __forceinline__ void do_tile(const GemmParams& P, int p, int n, int nnb, bool fused, lds_t* lds,
                                        Chain& ch) {
  uint64_t t_start = 0, t_ready = 0, t_main = 0;
  if (P.trace) t_start = __builtin_amdgcn_s_memrealtime();
  const Tile t = make_tile<L1, OT>(P, p, n, nnb);
  if constexpr (!L1) {
    if (fused) wait_row_ready(P, p);
  }
  if (P.trace) t_ready = __builtin_amdgcn_s_memrealtime();
  bool nt = false;
  if constexpr (streams_once(OT)) nt = t.once;
  if (nt) {
    if constexpr (streams_once(OT)) {
      if (nnb == 4) dispatch_tile<4, L1, OT, true>(P, t, lds, t_main, ch);
      else dispatch_tile<2, L1, OT, true>(P, t, lds, t_main, ch);
    }
  } else {
    if (nnb == 4) dispatch_tile<4, L1, OT, false>(P, t, lds, t_main, ch);
    else dispatch_tile<2, L1, OT, false>(P, t, lds, t_main, ch);
  }
  if constexpr (L1) finish_l1_tile<OT>(P, t, p, fused, lds);
  if constexpr (!L1) {
    if (P.row_done) finish_l2_tile(P, t);
  }
  if (P.trace) record_tile(P, L1, p, n, nnb, t_start, t_ready, t_main);
}

// Tile i of a list of nb row bands x N tiles, walked in groups of gm bands:
// inside a group N-tile by N-tile, the group's bands fastest. Consecutive
// tiles (which run at the same time, on one XCD) then share gm row bands and
// a few weight tiles instead of one band and many weight tiles.
__device__ __forceinline__ void raster(int i, int nb, int N, int gm, int& p, int& n) {
  const int span = gm * N;
  const int grp = i / span, base = grp * gm;
  const int rows = min(gm, nb - base);
  const int j = i - grp * span;
  p = base + j % rows;
  n = j / rows;
}

// One launch of the separate schedule: every tile of one Linear over nb row
// bands x N tiles of width nnb, in raster order. When the tiles are wide and
// the last round of the persistent grid would be partly idle (a tail of
// fewer than G tiles), that tail runs as twice as many half-width tiles:
// wide tile n of a band is exactly narrow tiles 2n and 2n+1, with the same K
// order, so the last round keeps every workgroup busy for half as long.
template <bool L1, int OT>
__device__ __forceinline__ void separate_tiles(const GemmParams& P, int nb, int N, int nnb, int lid, int G,
                                               lds_t* lds) {
  const int total = nb * N;
  const int cut = (nnb == 4 && total % G) ? total / G * G : total;
  const int end = cut + 2 * (total - cut);
  // tile i of the list: band, N-tile and width
  auto coords = [&](int i, int& p, int& n, int& w) {
    if (i < cut) {
      raster(i, nb, N, P.group_m, p, n);
      w = nnb;
    } else {
      const int j = i - cut;
      raster(cut + (j >> 1), nb, N, P.group_m, p, n);
      n = 2 * n + (j & 1);
      w = 2;
    }
  };
  bool pre = false;
  for (int i = lid; i < end; i += G) {
    int p, n, w;
    coords(i, p, n, w);
    Chain ch;
    ch.pre = pre;
    if (OT == OT_BF16 && i + G < end) {
      int p2, n2, w2;
      coords(i + G, p2, n2, w2);
      ch.next = make_tile<L1, OT>(P, p2, n2, w2);
      ch.has_next = true;
    }
    do_tile<L1, OT>(P, p, n, w, false, lds, ch);
    pre = ch.issued;
  }
}

template <int OT>
__global__ __launch_bounds__(gemm_threads(OT), 1) void moe_gemm_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmLds];
  lds_t* lds = (lds_t*)smem;  // address-space cast to the LDS window
  const int G = gridDim.x;
  const int b = blockIdx.x;
  // Workgroups are dealt round-robin to the 8 XCDs: make consecutive logical
  // ids share an XCD so a row band's tiles (same A rows) share one L2.
  const int lid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int Pb = P.meta[META_P];
  int p, n;
  Chain none;  // the fused schedules prefetch nothing across tiles
  switch (P.mode) {
    case MODE_SEP_L1:
      separate_tiles<true, OT>(P, Pb, P.N1, P.nnb1, lid, G, lds);
      break;
    case MODE_SEP_L2:
      separate_tiles<false, OT>(P, Pb, P.N2, P.nnb2, lid, G, lds);
      break;
    case MODE_WAVE: {
      const int nw = P.meta[META_NWAVES];
      for (int wv = 0; wv < nw; ++wv) {
        const int pb0 = P.wave_band0[wv], pb1 = P.wave_band0[wv + 1];
        for (int i = lid; i < (pb1 - pb0) * P.N1; i += G) {
          raster(i, pb1 - pb0, P.N1, P.group_m, p, n);
          do_tile<true, OT>(P, pb0 + p, n, P.nnb1, true, lds, none);
        }
        for (int i = lid; i < (pb1 - pb0) * P.N2; i += G) {
          raster(i, pb1 - pb0, P.N2, P.group_m, p, n);
          do_tile<false, OT>(P, pb0 + p, n, P.nnb2, true, lds, none);
        }
      }
      break;
    }
    default: {  // MODE_INTERLEAVED
      const int g = lid >> 1, r = lid & 1, Gp = G >> 1;
      const int P1 = (P.N1 + 1) >> 1, P2 = (P.N2 + 1) >> 1;
      const int end1 = Pb * P1, end2 = Pb * P2;
      const int span1 = P.group_m * P1;
      // With wide Linear-2 tiles, a last round that would leave pairs idle
      // (end2 not a multiple of Gp) runs after this loop as narrow tiles
      // spread over every workgroup, as in the separate schedule.
      const int cut2 = (P.nnb2 == 4 && end2 % Gp) ? end2 / Gp * Gp : end2;
      int k1 = g, k2 = g;
      while (k1 < end1 || k2 < cut2) {
        // first band of k1's raster group: every Linear-1 tile of a lower band
        // comes before k1 in the Linear-1 order
        const int b1 = k1 < end1 ? (k1 / span1) * P.group_m : 0x3FFFFFFF;
        int p2 = 0, c2 = 0;
        if (k2 < cut2) raster(k2, Pb, P2, P.group_m, p2, c2);
        if (k2 < cut2 && p2 + P.lead_D <= b1) {
          const int n = 2 * c2 + r;
          if (n < P.N2) do_tile<false, OT>(P, p2, n, P.nnb2, true, lds, none);
          k2 += Gp;
        } else {
          int p1, c1;
          raster(k1, Pb, P1, P.group_m, p1, c1);
          const int n = 2 * c1 + r;
          if (n < P.N1) do_tile<true, OT>(P, p1, n, P.nnb1, true, lds, none);
          k1 += Gp;
        }
      }
      // The tail: pair unit cut2 + (j >> 2) holds wide tiles 2 c2 and 2 c2 + 1,
      // i.e. narrow tiles 4 c2 .. 4 c2 + 3 (those of a wide tile past N2 do not
      // exist). A workgroup gets here only after its own Linear-1 tiles, so
      // every readiness wait below is on tiles that workgroups still in the
      // loop above issue.
      for (int j = lid; j < 4 * (end2 - cut2); j += G) {
        int p2, c2;
        raster(cut2 + (j >> 2), Pb, P2, P.group_m, p2, c2);
        if (2 * c2 + ((j >> 1) & 1) < P.N2) do_tile<false, OT>(P, p2, 4 * c2 + (j & 3), 2, true, lds, none);
      }
      break;
    }
  }
}

}  // namespace
}  // namespace moe
