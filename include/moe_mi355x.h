/*
 * moe_mi355x.h -- C ABI of one GPU's share of a Mixture-of-Experts layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (Cui et al., "Fine-grained Computation-Communication Overlap via
 * Tile-level Signaling and Scheduling for MoE", Section 2.1; Xian et al.,
 * "X-Stage: An Overlooked Pipeline Stage for Communication-Computation
 * Overlap in DiT Inference", Section 2.2 "MegaMoE Execution"):
 *
 *   route    : per token, the k largest router logits (descending, ties to
 *              the lower expert index) and gate weights = softmax over those
 *              k logits;
 *   dispatch : the assignments whose expert lies in this GPU's share
 *              [e_begin, e_end) are permuted into expert-contiguous rows
 *              (ascending assignment id a = t*k + j inside an expert);
 *   experts  : per row, h = W1[e] x (2f outputs), act = silu(h[0:f]) * h[f:2f],
 *              act rounded to the Linear-2 operand type, o = W2[e] act;
 *   combine  : Y[q(t)] = sum over the token's local slots j (ascending) of
 *              w[t,j] * o[t,j], accumulated in fp32 and rounded once to bf16;
 *              tokens with no local expert get 0. With S destination segments
 *              token t is written to row q(t) = (t mod S) * (T/S) + t div S
 *              (S contiguous segments of T/S rows), otherwise q(t) = t.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller, 16-byte
 *     aligned, row-major, densely packed. The library never allocates or
 *     frees memory: intermediates live in a caller-provided workspace of at
 *     least moe_workspace_size(p) bytes (256-byte aligned).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream). Returning MOE_OK means "enqueued", not "finished".
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and no output is touched.
 *   - A failed HIP launch returns MOE_ERR_HIP; moe_last_hip_error() gives the
 *     hipError_t of that failure (per host thread).
 *   - Calls on one stream are ordered; calls that share a workspace must not
 *     overlap in time (same or different streams).
 *   - Router logits must be finite; NaN logits give unspecified routing.
 *
 * Shape limits (MOE_ERR_UNSUPPORTED otherwise): 1 <= k <= min(16, E_global),
 * E_global <= 1024, 0 <= e_begin < e_end <= E_global, T >= 1, T % S == 0,
 * d % 128 == 0, f % 128 == 0 (fp8 also T % 128 == 0 and
 * quant_block == 128).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad enum, inconsistent sizes */
  MOE_ERR_UNSUPPORTED = 2,        /* shape outside the limits above */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4,                /* a HIP runtime call failed */
  MOE_ERR_DEADLOCK = 5            /* a persistent-pipeline wait timed out (reported by moe_check_workspace) */
} moe_status_t;

typedef enum {
  MOE_DTYPE_BF16 = 0,             /* X, W1, W2 bfloat16; H bfloat16 */
  MOE_DTYPE_FP8_E4M3 = 1,         /* X, W1, W2 OCP E4M3FN codes with fp32 block scales; H e4m3 with
                                     one fp32 scale per row and 128 columns */
  MOE_DTYPE_W4A8_MXFP4 = 2        /* X e4m3 with fp32 block scales as above (H too); W1, W2 in OCP MXFP4:
                                     E2M1 codes, two per byte (the even element in the low nibble), and
                                     one E8M0 scale byte per 32 consecutive elements along K. The
                                     low-bit weight variant (W4A8) of X-Stage's evaluation, Section 5 */
} moe_dtype_t;

/* Tile schedule of the grouped expert GEMMs (X-Stage, Section 4.2 "MegaMoE:
 * Capacity-Aware Scheduling across Expert Waves", Algorithm 1 and Figure 4). */
typedef enum {
  MOE_SCHED_EXPERT_WAVE = 0,      /* one persistent launch; local experts grouped into waves; a wave's
                                     Linear-1 tiles, then its Linear-2 tiles, then the next wave */
  MOE_SCHED_INTERLEAVED = 1,      /* one persistent launch; Linear-1 and Linear-2 tile streams merged:
                                     a Linear-2 tile of row p2 is taken only when the Linear-1 cursor
                                     leads by at least lead_D rows, otherwise a Linear-1 tile */
  MOE_SCHED_SEPARATE = 2,         /* one persistent launch for every Linear-1 tile, then one for every
                                     Linear-2 tile (stream order is the only dependency) */
  MOE_SCHED_AUTO = 3              /* chosen at run time (X-Stage, Section 6.3: pick the schedule per
                                     routing and working set). The expert-wave and interleaved orders
                                     exist to spread remote-store bursts; this library's epilogues
                                     store into local HBM, where nothing drains them, so the choice is
                                     MOE_SCHED_SEPARATE, which needs no cross-workgroup readiness
                                     counters (measured fastest on every workload shape here) */
} moe_sched_t;

/* Flags (moe_problem_t.flags). Bits 0 and 1 select output and buffer
 * precisions; the tile-shape controls (bits 2-4) give bit-identical results
 * whatever their combination (each output element is computed by one tile
 * with the same K order) and exist for tests and tuning: by default the
 * widths and the raster order are chosen from the shape. */
enum {
  MOE_FLAG_NONE = 0u,
  MOE_FLAG_FP32_Y_DEBUG = 1u << 0,     /* moe_layer_forward also returns the fp32 sums of Y before their
                                          bf16 rounding in Y_fp32. A non-NULL Y_fp32 alone requests them
                                          too; with the flag set Y_fp32 must not be NULL */
  MOE_FLAG_BF16_COMBINE_BUF = 1u << 1, /* the token-ordered combine buffer holds bf16 instead of fp32: the
                                          Linear-2 epilogue rounds each expert output to bf16 (RNE) and the
                                          combine reads bf16. Halves the buffer's bytes, at the price of a
                                          second rounding of every output (measured, not the default) */
  MOE_FLAG_TILE_NARROW = 1u << 2,      /* every tile 128 weight rows wide */
  MOE_FLAG_TILE_WIDE = 1u << 3,        /* 256 weight rows wide wherever the shape allows (Linear-2 tiles
                                          need d % 256 == 0); may not be combined with MOE_FLAG_TILE_NARROW */
  MOE_FLAG_BAND_MAJOR = 1u << 4,       /* walk the expert-GEMM tile lists row band by row band instead of
                                          in groups of bands */
  MOE_FLAG_TILE_TRACE = 1u << 5,       /* record one span per expert-GEMM tile in the workspace region
                                          tile_trace (moe_tile_record_t); costs a few clock reads per tile */
  MOE_FLAG_KEEP_H_F32 = 1u << 6,       /* fp8: also store every fp32 SwiGLU value (the H quantiser's input)
                                          in the workspace region h_f32. Without it, wide Linear-1 tiles
                                          quantise from on-chip memory and leave h_f32 unwritten. For
                                          verification; costs 4 bytes of HBM writes per H element */
  MOE_FLAG_TEST_WAIT_TIMEOUT = 1u << 7 /* tests of the timeout path only: the fused schedules' readiness
                                          target is made unreachable, so their first Linear-2 wait gives up
                                          after its bounded spin (about a second), every later wait at once,
                                          and moe_check_workspace reports MOE_ERR_DEADLOCK. Outputs are
                                          then invalid. The separate schedule has no such wait */
};

/* One expert-GEMM tile as recorded with MOE_FLAG_TILE_TRACE: the per-tile
 * spans that X-Stage, Section 5.2.3, measures to test its Eq. 15 (mainloop
 * against epilogue stores). Times are reads of the device-wide constant-rate
 * clock (s_memrealtime; its rate is moe_tile_clock_hz()):
 * t_start when the workgroup takes the tile, t_ready once its inputs are
 * ready (a Linear-2 tile of a fused schedule first waits for its row band's
 * Linear-1 tiles), t_main_end after the K loop, t_end after the epilogue
 * stores (and, for Linear-1 in the fused schedules or fp8, after publishing
 * them). info packs kind (bits 0-1: 1 = Linear-1, 2 = Linear-2), the tile
 * width NNB (bits 2-4; 128 or 256 weight rows for 2 or 4), the workgroup
 * (bits 8-23), the N-tile index in units of its width (bits 24-39) and the row
 * band (bits 40-63). The region holds tile_trace_capacity records; the
 * number written is meta[4] (records past the capacity are dropped). */
typedef struct moe_tile_record {
  uint64_t t_start, t_ready, t_main_end, t_end;
  uint64_t info;
} moe_tile_record_t;

typedef struct moe_problem {
  int32_t T;             /* tokens */
  int32_t d;             /* hidden size */
  int32_t f;             /* expert intermediate size (W1 has 2f rows: gate [0,f), up [f,2f)) */
  int32_t E_global;      /* experts the router chooses from */
  int32_t k;             /* experts per token */
  int32_t e_begin;       /* this GPU's experts: [e_begin, e_end); E_l = e_end - e_begin */
  int32_t e_end;
  int32_t dtype;         /* moe_dtype_t */
  int32_t quant_block;   /* fp8 block edge (128); ignored for bf16 */
  int32_t num_segments;  /* S >= 1: destination segments of the output rows */
  int32_t sched;         /* moe_sched_t */
  int32_t lead_D;        /* interleaved: minimum row-band lead of Linear-1 over Linear-2 (>= 1);
                            0 = the anti-starvation knee of X-Stage Eq. 16 (at least 8),
                            times max(1, f / d), the Linear-2 : Linear-1 tile-time ratio */
  int32_t wave_experts;  /* expert-wave: experts per wave; 0 = fewest experts whose Linear-1
                            tiles fill the persistent grid */
  int32_t grid;          /* persistent workgroups; 0 = one per compute unit */
  uint32_t flags;        /* MOE_FLAG_* bits; 0 = tile shapes chosen from the problem's shape */
  int32_t row_capacity;  /* rows the workspace holds for the expert GEMM: 0 = T * min(k, E_l), the most
                            local assignments a routing can give; larger (>= that) for a padded row
                            layout such as the owner-aligned one below, whose R can exceed it */
} moe_problem_t;

/* Byte offsets of the intermediates inside a workspace (for inspection by
 * tests and callers). cap = the row capacity: T * min(k, E_l), or
 * p->row_capacity if set. moe_layer_forward writes every region except one
 * whose output the caller passes in its place, and x_perm (its Linear-1
 * reads each row band's X rows where they are). */
typedef struct moe_workspace_layout {
  size_t topk_idx;      /* int32 [T, k]                                     */
  size_t topk_w;        /* fp32  [T, k]                                     */
  size_t counts;        /* int32 [E_l]      local assignments per expert     */
  size_t offsets;       /* int32 [E_l + 1]  exclusive prefix sum of counts   */
  size_t row_src;       /* int32 [cap]      assignment id of expert-ordered row r */
  size_t row_dst;       /* int32 [cap]      token-order slot of expert-ordered row r */
  size_t tok_off;       /* int32 [T + 1]    first token-order slot of output row q */
  size_t comb_w;        /* fp32  [cap]      gate weight of token-order slot p */
  size_t x_perm;        /* elem  [cap, d]   gathered rows (bf16, or e4m3 codes) */
  size_t x_perm_scale;  /* fp32  [d/128, cap] fp8 only: scale of row r, column block c at c*cap + r */
  size_t h;             /* elem  [cap, f]   SwiGLU output (bf16, or e4m3 codes) */
  size_t h_scale;       /* fp32  [f/128, cap] fp8 only */
  size_t h_f32;         /* fp32  [cap, f]   fp8 only: SwiGLU output before its e4m3 quantisation */
  size_t combine_buf;   /* fp32  [cap, d]   Linear-2 output in token-order slots */
  size_t meta;          /* int32 [64]       meta[0] = A (local assignments), meta[1] = row bands,
                                            meta[2] = 1 if a readiness wait of the last expert-GEMM
                                            call timed out, meta[4] = tile records written
                                            (MOE_FLAG_TILE_TRACE), meta[5] = device-side argument
                                            errors (bits: 1 = more local assignments than the row
                                            capacity, 2 = offsets not monotone or past the row
                                            capacity, 4 = a row_dst outside the row capacity) */
  size_t tile_trace;    /* moe_tile_record_t [tile_trace_capacity]; empty without MOE_FLAG_TILE_TRACE */
  size_t tile_trace_capacity;  /* records (a bound on the tiles of one call) */
  size_t total;         /* = moe_workspace_size */
} moe_workspace_layout_t;

/* Workspace bytes for any entry point below (0 if the problem is invalid). */
MOE_API size_t moe_workspace_size(const moe_problem_t* p);

/* Fills *out with the workspace layout of problem p. */
MOE_API moe_status_t moe_workspace_get_layout(const moe_problem_t* p, moe_workspace_layout_t* out);

/* Top-k router (Cui et al. Section 2.1 step (1)).
 *   logits        fp32 [T, E_global]
 *   topk_idx      int32 [T, k]   out: selected global expert ids, slot order
 *   topk_w        fp32 [T, k]    out: gate weights (sum to 1 per token)
 *   counts_global int32 [E_global] out, may be NULL: assignments per global expert (sum T*k) */
MOE_API moe_status_t moe_route_topk(const moe_problem_t* p, const float* logits, int32_t* topk_idx,
                                    float* topk_w, int32_t* counts_global, void* stream);

/* Dispatch to this GPU's experts (Cui et al. Section 2.1 step (2), as an
 * on-GPU permutation). Inputs: X [T, d] (bf16, or e4m3 codes with X_scale
 * fp32 [T/128, d/128]; X_scale must be NULL for bf16), topk_idx, topk_w.
 * Outputs: counts, offsets, row_src, row_dst, tok_off, comb_w (see the
 * layout struct for shapes), X_perm [cap, d] (row r = X row of token
 * row_src[r] / k) and, for fp8, X_perm_scale [d/128, cap]. Rows >= A of the
 * cap-sized outputs are left untouched. */
MOE_API moe_status_t moe_dispatch(const moe_problem_t* p, const void* X, const float* X_scale,
                                  const int32_t* topk_idx, const float* topk_w, int32_t* counts,
                                  int32_t* offsets, int32_t* row_src, int32_t* row_dst, int32_t* tok_off,
                                  float* comb_w, void* X_perm, float* X_perm_scale, void* workspace,
                                  size_t ws_bytes, void* stream);

/* moe_dispatch without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels, with their scratch (per-chunk expert
 * counts, per-row slot counts, a few status words) in a library-owned device
 * array of 8 MiB per GPU, created with the library's code object and kept
 * until the process ends. The call itself allocates nothing. Arguments and
 * outputs as for moe_dispatch; a problem whose scratch exceeds the array
 * (about 2 MiB of counts plus 4 bytes per token: more than about 1.5 million
 * tokens) gives MOE_ERR_UNSUPPORTED before any launch. Every call on one GPU
 * uses that GPU's one array, so calls that overlap in time on one GPU (two
 * streams, two host threads) race and give undefined results; calls in
 * stream order are safe. A routing with more local assignments than the row
 * capacity shows as offsets[E_l] > cap (rows past it are not stored), as
 * there is no workspace to carry the error word. */
MOE_API moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const void* X, const float* X_scale,
                                          const int32_t* topk_idx, const float* topk_w, int32_t* counts,
                                          int32_t* offsets, int32_t* row_src, int32_t* row_dst, int32_t* tok_off,
                                          float* comb_w, void* X_perm, float* X_perm_scale, void* stream);

/* Grouped expert FFN over the expert-contiguous rows (X-Stage Section 2.2;
 * schedule per p->sched). W1 [E_l, 2f, d], W2 [E_l, d, f] (bf16, or e4m3 codes
 * with W1_scale fp32 [E_l, 2f/128, d/128], W2_scale fp32 [E_l, d/128, f/128];
 * MXFP4: W1 uint8 [E_l, 2f, d/2], W2 uint8 [E_l, d, f/2] with W1_scale uint8
 * E8M0 [E_l, 2f, d/32], W2_scale uint8 E8M0 [E_l, d, f/32]).
 * Writes combine_buf [cap, d] (fp32, or bf16 with MOE_FLAG_BF16_COMBINE_BUF):
 * row row_dst[r] = W2[e] act(r). The intermediate H lives in the workspace.
 * offsets/row_dst as from moe_dispatch. Device-side checks (reported by
 * moe_check_workspace as MOE_ERR_INVALID_ARGUMENT): offsets must be
 * non-decreasing with 0 <= offsets[0] and offsets[E_l] <= cap, otherwise no
 * tile runs and combine_buf and H are left untouched; a row whose row_dst lies
 * outside [0, cap) is not stored. */
MOE_API moe_status_t moe_expert_forward(const moe_problem_t* p, const void* X_perm, const float* X_perm_scale,
                                        const int32_t* offsets, const int32_t* row_dst, const void* W1,
                                        const void* W1_scale, const void* W2, const void* W2_scale,
                                        void* combine_buf, void* workspace, size_t ws_bytes, void* stream);

/* Weighted combine (Cui et al. Section 2.1 step (5)): Y bf16 [T, d] in
 * output-row order q; Y_fp32 [T, d] (may be NULL) gets the same sums before
 * the bf16 rounding. combine_buf [cap, d] is fp32, or bf16 with
 * MOE_FLAG_BF16_COMBINE_BUF. Deterministic: fixed slot order, no atomics. A
 * row q whose slot range [tok_off[q], tok_off[q+1]) does not lie inside
 * [0, cap) is written as NaN (a device-side check; nothing outside the
 * buffers is read). */
MOE_API moe_status_t moe_combine(const moe_problem_t* p, const void* combine_buf, const int32_t* tok_off,
                                 const float* comb_w, void* Y, float* Y_fp32, void* stream);

/* The whole share, Cui et al. Section 2.1 steps (1)-(5) as one GPU's local
 * pipeline (dispatch and return become on-GPU permutations) and X-Stage
 * Section 2.2 "MegaMoE Execution" (Dispatch, Linear-1, activation, Linear-2,
 * Combine): route -> dispatch -> grouped Linear-1 + SwiGLU -> grouped
 * Linear-2 -> combine on one stream, with row counts kept on the device (no
 * host synchronisation), in five launches (four with the expert-wave or
 * interleaved schedule): the router with the dispatch's counts; the scan,
 * the expert GEMM's row-band plan and the scatter; the grouped GEMM(s), whose
 * Linear-1 gathers each band's rows from X through row_src instead of a
 * permuted copy; the weighted combine. The results are those of the
 * component calls, bit for bit. Inputs as for the component calls; Y bf16 [T, d]
 * (segment-major with S > 1); Y_fp32 [T, d] or NULL (see
 * MOE_FLAG_FP32_Y_DEBUG). The optional outputs, each DEVICE memory or NULL,
 * receive the routing and dispatch results: topk_idx_out int32 [T, k],
 * topk_w_out fp32 [T, k], counts_out int32 [E_l], offsets_out int32
 * [E_l + 1], row_src_out int32 [cap] (rows >= A untouched). A non-NULL output
 * is written in place of its workspace region, which the call then leaves
 * unwritten. Every other intermediate is left in the workspace at
 * moe_workspace_get_layout's offsets, except x_perm, which is not formed
 * (x_perm_scale is: the e4m3 path's Linear-1 reads the row scales from it). */
MOE_API moe_status_t moe_layer_forward(const moe_problem_t* p, const void* X, const float* X_scale,
                                       const float* logits, const void* W1, const void* W1_scale,
                                       const void* W2, const void* W2_scale, void* Y, float* Y_fp32,
                                       void* workspace, size_t ws_bytes, int32_t* topk_idx_out,
                                       float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                       int32_t* row_src_out, void* stream);

/* Synchronises `stream` and reads the workspace's error words (meta[2],
 * meta[5]), which the calls that can set them clear when they start:
 * MOE_ERR_DEADLOCK if a persistent-pipeline wait of the most recent
 * expert-GEMM call on this workspace timed out, MOE_ERR_INVALID_ARGUMENT if a
 * device-side check of the last dispatch or expert-GEMM call failed (its
 * outputs are then invalid). Clears both words. */
MOE_API moe_status_t moe_check_workspace(const moe_problem_t* p, void* workspace, size_t ws_bytes,
                                         void* stream);

/* Owner-aligned return path (Cui et al., Section 3.2.1 remote-owner-aligned
 * row layout, Section 3.2.2 remote-first tile schedule and Algorithm 1,
 * Section 3.2.3 combine plan, Section 3.3.2 / Figure 3b segment-granular
 * transfer, Section 4.5 padding bound). The share's tokens belong to S =
 * p->num_segments ranks, token t to rank t mod S; local_rank is this GPU's.
 *
 * moe_owner_plan (HOST pointers, no GPU call; topk_idx int32 [T, k] as from
 * moe_route_topk, copied to the host). Inside each local expert the rows
 * are grouped by owner rank, remote ranks ascending and local_rank last,
 * ascending assignment id a = t*k + j inside a group; every remote group is
 * padded with zero rows (row_src = -1) to a multiple of tb_M (1..4096), the
 * local group is not. Outputs:
 *   row_src    int32 [R]          assignment id of padded row r, -1 = zero row
 *   expert_off int32 [E_l + 1]    first padded row of each expert (expert_off[E_l] = R)
 *   bands      int32 [bands, 5]   per row band of tb_M rows (a local group's last
 *                                 band may be shorter): local expert, owner rank,
 *                                 first row, valid rows, row offset inside the
 *                                 owner's receive region; in layout order
 *   schedule   int32 [bands]      band ids, remote-first: experts by descending
 *                                 remote band count (ties: lower expert first),
 *                                 their remote bands, then every local band
 *   segments   int32 [segments, 4] transfer segments: source row in the layout,
 *                                 valid rows, destination row in the receive
 *                                 buffer, owner rank. Per (expert, rank) group
 *                                 the first and last segment hold one band and the
 *                                 middle ones up to x_bands (>= 1); listed in the
 *                                 order their first band is scheduled
 *   recv_start int32 [S + 1]      first receive-buffer row of each rank's region;
 *                                 a region holds its rank's rows in (expert, a) order
 *   sizes      R, bands, remote_bands, segments, recv_rows (always filled).
 * With every array NULL only `sizes` is filled. row_cap < R or band_cap <
 * bands gives MOE_ERR_WORKSPACE_TOO_SMALL (sizes filled, arrays untouched);
 * R >= 2^31 gives MOE_ERR_UNSUPPORTED. */
typedef struct moe_owner_plan_sizes {
  int64_t R, bands, remote_bands, segments, recv_rows;
} moe_owner_plan_sizes_t;
MOE_API moe_status_t moe_owner_plan(const moe_problem_t* p, const int32_t* topk_idx, int local_rank, int tb_M,
                                    int x_bands, int32_t* row_src, int64_t row_cap, int32_t* expert_off,
                                    int32_t* bands, int32_t* schedule, int32_t* segments, int64_t band_cap,
                                    int32_t* recv_start, moe_owner_plan_sizes_t* sizes);

/* Gather into the owner-aligned layout. DEVICE pointers: X [T, d] (bf16, or
 * e4m3 codes with X_scale fp32 [T/128, d/128]; X_scale must be NULL for
 * bf16), row_src int32 [R] from moe_owner_plan. X_pad [R, d] out: row r =
 * X[row_src[r] / k], or zeros where row_src[r] is -1 (ids outside [0, T*k)
 * also give zeros). fp8: X_pad_scale fp32 [d/128, cap] out, cap = the row
 * capacity of p (T * min(k, E_l), or p->row_capacity): row r's block scales
 * at c * cap + r (the layout moe_expert_forward reads; 1 for a zero row);
 * R > cap gives MOE_ERR_UNSUPPORTED. moe_expert_forward then runs on X_pad
 * with offsets = expert_off and row_dst[r] = r, writing the layout's expert
 * outputs O_pad fp32 [R, d]; this needs R <= cap, so a padded layout sets
 * p->row_capacity to at least R (moe_owner_plan reports R). */
MOE_API moe_status_t moe_owner_gather(const moe_problem_t* p, const void* X, const float* X_scale,
                                      const int32_t* row_src, int64_t R, void* X_pad, float* X_pad_scale,
                                      void* stream);

/* Segment transfer (DEVICE pointers): for every segment (src, rows, dst, rank)
 * of moe_owner_plan, recv[dst + i] = O_pad[src + i] for i < rows (fp32 rows of
 * d). A segment whose rows fall outside [0, R) or [0, R_recv) is skipped. */
MOE_API moe_status_t moe_segment_copy(const moe_problem_t* p, const float* O_pad, int64_t R,
                                      const int32_t* segments, int64_t n_segments, float* recv, int64_t R_recv,
                                      void* stream);

/* Overlapped segment transfer (Cui et al., Section 3.3.1 tile-level signaling
 * and Section 3.3.3 producer-consumer co-scheduling, on one GPU).
 *
 * moe_expert_forward_signal: moe_expert_forward that also publishes, after
 * every Linear-2 tile's stores, the tile's output elements per 32-row block
 * of rows: row_done[b] += (rows of the tile in block b) * (its columns),
 * after a device-scope release. Block b of an R-row layout is complete at
 * min(32, R - 32 b) * d. row_done: DEVICE int32 [row_done_len], zero at the
 * call (the caller clears it), at least ceil(R / 32) blocks; counts past
 * row_done_len are dropped.
 *
 * moe_segment_copy_wait: moe_segment_copy whose segments each wait until
 * their rows' blocks are complete in row_done (ceil(R / 32) <= row_done_len).
 * R is the layout's row count, expert_off[E_l] of the plan: the GEMM stores
 * exactly those rows, so the last block's target is taken from it (O_pad
 * must hold at least R rows, and may hold more),
 * so it can run on a second stream beside moe_expert_forward_signal (launch
 * it after the clearing of row_done is ordered before it). Enqueue the
 * GEMM first and the copier second: two streams may share one hardware
 * queue, and a copier enqueued first on a shared queue would hold the GEMM
 * back until its waits time out; in the other order the worst case is that
 * the copier runs after the GEMM. grid persistent
 * workgroups (1..1024; 0 = 256, one per compute unit) walk the segments in plan order; they use no
 * LDS, so the GEMM's workgroups stay resident beside them. Waits are
 * bounded: a timeout (about a second) sets *err (DEVICE int32, zero at the
 * call) to 1, and that and every later segment are skipped. The call gives
 * MOE_ERR_UNSUPPORTED when the register counts the runtime reports for the
 * problem's expert-GEMM kernel (two wavefronts per SIMD) and for the copier
 * do not fit one SIMD's 512 registers per lane together: then no copier
 * wavefront could run beside the GEMM's workgroups and every wait would time
 * out (the fp8 GEMM, at 256 registers per wavefront, is such a case). */
MOE_API moe_status_t moe_expert_forward_signal(const moe_problem_t* p, const void* X_perm,
                                               const float* X_perm_scale, const int32_t* offsets,
                                               const int32_t* row_dst, const void* W1, const void* W1_scale,
                                               const void* W2, const void* W2_scale, void* combine_buf,
                                               int32_t* row_done, int64_t row_done_len, void* workspace,
                                               size_t ws_bytes, void* stream);
MOE_API moe_status_t moe_segment_copy_wait(const moe_problem_t* p, const float* O_pad, int64_t R,
                                           const int32_t* segments, int64_t n_segments, float* recv,
                                           int64_t R_recv, const int32_t* row_done, int64_t row_done_len,
                                           int32_t* err, int grid, void* stream);

MOE_API const char* moe_status_string(moe_status_t s);
MOE_API int moe_last_hip_error(void);
/* Library version, e.g. "0.1.0". */
MOE_API const char* moe_version(void);
/* Store-burst probe: the local-memory form of the periodic and isolated
 * burst microbenchmarks of X-Stage, Section 3.1, whose timings calibrate the
 * Burst-Gap parameters (T_iss^0, R, Q; Section 3.2-3.5, Eqs. 1-7) for vector
 * stores the CUs issue into their own HBM.
 *   K producers (1..4096; one wavefront each) start together and repeat
 *   `reps` times (1..100000): a burst of B bytes (a multiple of 1024, at
 *   least 1024) of 16-byte stores, then a gap of gap_us microseconds
 *   (0..100000, and reps * gap_us at most 2 s) with no memory traffic. Producer k writes its own ring of
 *   buf_bytes / K bytes (rounded down to 1 KiB; at least B) of `buf`
 *   (device memory, contents overwritten).
 *   rec: device memory of at least (2 K reps + 1) 64-bit words; word
 *   2 (k reps + r) is producer k's clock reading at the start of burst r,
 *   the next word the reading once its last store has issued; the last word
 *   is the common start time. Clock rate: moe_tile_clock_hz().
 *   Invalid arguments return MOE_ERR_INVALID_ARGUMENT before any launch. */
MOE_API moe_status_t moe_store_burst_probe(int K, int B, int reps, double gap_us, void* buf, size_t buf_bytes,
                                           uint64_t* rec, size_t rec_bytes, void* stream);

/* The schedule `p` runs: p->sched, with MOE_SCHED_AUTO resolved; -1 if
 * p->sched is not a moe_sched_t. */
MOE_API int moe_schedule_of(const moe_problem_t* p);
/* Frequency in Hz of the clock the moe_tile_record_t readings count (the
 * current device's constant-rate wall clock), or 0 if HIP cannot report it. */
MOE_API double moe_tile_clock_hz(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
