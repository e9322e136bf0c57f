/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts forward path.
 *
 * The library computes, for T tokens, the complete single-GPU MoE forward
 * pass: score the tokens (router top-k), reorder them onto experts, run the
 * variable-size per-expert SwiGLU GEMMs and combine the results back with
 * the routing weights.
 *
 * Source of the operation.  [R] is the Pith review page of "Cross-Platform
 * Fused MoE Dispatch in Triton: Portable Expert Routing Without CUDA"
 * (arXiv 2605.23911), which also carries the paper's abstract:
 *   - [R] "The reading": the four steps above.
 *   - [R] "What carries the argument": gate and up projections computed from
 *     one shared load of each input tile, SiLU applied in registers so the
 *     two intermediates never reach global memory; a grouped GEMM whose
 *     fixed-size blocks map to (expert, token-offset) pairs.
 *   - [R] "Assumptions & free parameters": softmax or sigmoid router, top-k,
 *     SwiGLU FFN (paper Eq. (1)-(4)); BLOCK_M fixed per launch.
 *   - abstract: router scoring, token permutation, expert GEMMs, weighted
 *     output combination.
 *
 * Conventions for every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are
 *     dense row-major.
 *   - Data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory and never synchronises the
 *     stream; every kernel is enqueued on `hip_stream` (a hipStream_t; NULL
 *     means the default stream) and the call returns at once.
 *   - All argument checks run on the host before any HIP call.  On failure
 *     the entry point returns a negative moe_status, enqueues nothing and
 *     leaves every output untouched.  A failed launch returns MOE_ERR_HIP;
 *     faults inside a kernel surface at the caller's next synchronisation.
 *   - Calls are re-entrant.  Concurrent calls are safe on distinct streams
 *     with distinct workspaces; calls that share a workspace must be
 *     ordered on one stream.
 *   - The contents of the workspace after a call are unspecified.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

/* Limits of the library (violations return MOE_ERR_UNSUPPORTED). */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 16
#define MOE_MAX_ROWS (1 << 20)   /* T * top_k */

enum moe_score {
    MOE_SCORE_SOFTMAX = 0,  /* softmax over the logits                    */
    MOE_SCORE_SIGMOID = 1   /* logistic sigmoid of each logit             */
};

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL                 */
    MOE_ERR_SHAPE = -2,       /* negative or zero size where one is needed  */
    MOE_ERR_TOPK = -3,        /* top_k < 1 or top_k > E                     */
    MOE_ERR_ALIGN = -4,       /* d or ffn not a multiple of 64, or a pointer
                                 not 16-byte aligned (workspace: 256)       */
    MOE_ERR_WORKSPACE = -5,   /* workspace smaller than the size query      */
    MOE_ERR_UNSUPPORTED = -6, /* beyond the library limits, bad option      */
    MOE_ERR_HIP = -7,         /* a HIP launch or record call failed         */
    MOE_ERR_STATIC_LIMIT = -8 /* moe_forward_static: the problem needs more
                                 than MOE_STATIC_WORKSPACE_BYTES of workspace */
};

/* Size of the device array moe_forward_static uses as its workspace (one
 * array per GPU the library runs on, held until the process ends). */
#define MOE_STATIC_WORKSPACE_BYTES (256u << 20)

/* Optional knobs of moe_forward_ex / moe_route.  Zero-initialise for the
 * automatic choices. */
typedef struct moe_options {
    /* Rows per schedule block (BLOCK_M, [R] "Assumptions & free
     * parameters": fixed for one launch).  0 = automatic: the smallest size
     * >= 128 that holds the mean rows per expert plus three standard
     * deviations of a uniform router; else one of 16, 32, 64, 128, 192, or
     * 256 (asked for only: the LDS-staged tiles at 256 rows -- the narrow
     * gate/up tile and down variant 2, so d a multiple of 256 -- not with
     * the unfused ablation, gather mode 3, the folded combination or the
     * fused down projection, else MOE_ERR_UNSUPPORTED).  Blocks hold up to
     * block_rows rows; the GEMMs skip 16-row subtiles past a block's last
     * row.  The gate/up GEMM may take its own blocks of 256 rows (see
     * schedule). */
    int block_rows;
    /* Split of the down projection's reduction (ffn) into this many parts
     * whose partial sums the combination adds in a fixed order.  0 =
     * automatic (an upper bound chosen on the host; the kernels then take
     * the parts from the routed block count on the device, see
     * moe_plan_info.split_on_device); else 1..8, used as given. */
    int split_k;
    /* Tile variant of the fused gate/up GEMM.  0 = automatic; k >= 1 selects
     * compiled variant k-1 for the chosen block_rows (which must then be set
     * explicitly).  BM = 64 has variants 0 (256 columns per workgroup) and 1
     * (128 columns); BM = 128 has variants 0 (128 columns, 8 waves), 1
     * (64 columns), 2 (256 columns, 8 waves, weights staged in LDS;
     * the last column tile may be partial) and 3 (128 columns, 8 waves of
     * one 16-column subtile, weights staged in LDS in three stages; the
     * stream-K schedule's tile) -- 2 and 3 not with gather_mode 3, else
     * MOE_ERR_UNSUPPORTED; BM = 192 has variants 0 (128 columns, 8 waves),
     * 1 (112 columns, 7 waves) and 2 (224 columns, 7 waves, weights staged
     * in LDS; the last column tile may be partial; not with gather_mode 3,
     * else MOE_ERR_UNSUPPORTED -- automatic at BM = 192 where ffn is a
     * multiple of 224 or the launch is large);
     * every other BM has variant 0 only. */
    int tile_variant;
    /* Tile variant of the down GEMM, like tile_variant (block_rows must be
     * set).  BM = 128 and 192 have variants 0 and 1 (256 columns per
     * workgroup: 4 waves of 64 and 8 waves of 32 at BM = 128, the reverse
     * at BM = 192), 2 (256 columns, 8 waves of 32, weights staged in LDS;
     * only when d is a multiple of 256) and 3 (64 columns per wave staged
     * in LDS: 512 columns, 8 waves at BM = 128; 448 columns, 7 waves at
     * BM = 192; the last column tile may be partial) and, at BM = 128, 4
     * (the same 64 columns per wave in 7 waves: 448 columns); variants 2
     * to 4 only when the combination is not folded into the down GEMM,
     * else MOE_ERR_UNSUPPORTED.  Automatic: variant 3 on launches with many
     * workgroups and at least six column tiles per block -- at BM = 128
     * variant 4 instead where d is a multiple of 448 and its workgroups
     * fill whole rounds of 256 better -- else 2 where it fits; every other
     * BM has variant 0 only.  0 = automatic.  All variants give the same
     * bytes (the same per-output K order). */
    int down_variant;
    /* K-start rotation of the GEMMs: a workgroup starts its reduction at a
     * step derived from its schedule block (2), from its own id (3) or from
     * its expert (4), and wraps around.  0 = automatic (per expert), 1 =
     * off.  Results are deterministic either way; rounding differs
     * slightly. */
    int rotate;
    /* Routing kernels.  0 = automatic: one workgroup does the route,
     * histogram, scan, schedule and reorder when T <= 1024, E <= 32 and
     * T*E*top_k <= 32768; else two launches (the route, then one workgroup
     * for the histogram, scan, schedule and reorder) when
     * ceil(T*top_k/64)*E <= 16384; else three launches; 1 = the
     * one-workgroup kernel (MOE_ERR_UNSUPPORTED beyond T <= 1024 and
     * E <= 64); 2 = three launches; 3 = two launches
     * (MOE_ERR_UNSUPPORTED beyond ceil(T*top_k/64)*E <= 16384).  Same
     * results either way. */
    int routing_kernels;
    /* Row gather of moe_forward.  0 = automatic (1 when 2*T*d < 2^31);
     * 1 = the fused gate/up GEMM reads each sorted row straight from x
     * through perm (no x_perm buffer); 2 = a gather kernel writes x_perm to
     * the workspace first; 3 = as 2, with x_perm stored in K-step tiles
     * (for each group of 16 sorted rows, each 64-column step is 2 KiB
     * contiguous), so the GEMM's per-step activation reads are contiguous.
     * Same results either way. */
    int gather_mode;
    /* SwiGLU ablation.  0 = fused (default): gate and up products from one
     * shared activation tile, SiLU and the product in registers, h written
     * once.  1 = unfused: a gate GEMM and an up GEMM each read the
     * activation rows and write a bf16 product [A, ffn] to the workspace,
     * and a third kernel forms h = bf16(silu(g) * u).  The workspace grows
     * by 4*A*ffn bytes; results differ from the fused path by the two extra
     * bf16 roundings. */
    int unfused_swiglu;
    /* Workgroup order of the GEMMs.  0 = automatic (grouped when about 128
     * or more schedule blocks are expected), 1 = plain (workgroup i
     * takes block i / tiles, tile i % tiles), 2 = grouped by XCD: each of
     * the 8 XCDs runs a contiguous range of (block, tile) ids, so a block's
     * rows are fetched into one L2; 3 = longest first: as plain, but over
     * the blocks in decreasing row count (an order the routing kernels
     * build on the device; moe_route's block_order), so that under skewed
     * routing the heavy blocks start first and light ones fill the tail.
     * Same results either way (with rotate = 3, rounding differs). */
    int xcd_order;
    /* Weighted combination.  The number of launches is a free choice of the
     * method, fusion depth against launch overhead ([R] "Assumptions & free
     * parameters").  0 = automatic (the separate kernel, measured faster on
     * every workload shape), 1 = its own kernel after the down GEMM, 2 = folded
     * into the down GEMM: each of its workgroups counts the partial rows it
     * wrote per (token, column tile), and the workgroup that writes the last
     * of a token's top_k * split partials of a tile also writes that token's
     * output columns of the tile -- the same sums in the same fixed order as
     * the separate kernel, so the output bytes are the same either way.  The
     * routing kernels clear the counters (4*T*ceil(d/256) bytes or fewer of
     * workspace) on every call. */
    int fold_combine;
    /* Down projection fused into the gate/up GEMM, for small problems
     * (again fewer launches, [R] "Assumptions & free parameters").  0 =
     * automatic, 1 = off, 2 = on: each (block, column tile) workgroup of the
     * gate/up GEMM keeps its SwiGLU tile in LDS and multiplies it by the
     * matching columns of W_down, writing one fp32 partial [A, d] per column
     * tile; the weighted combination adds those partials in tile order (the
     * split of the down reduction is then the number of column tiles, and
     * split_k and fold_combine do not apply).  No h buffer, no down GEMM
     * launch; the workspace holds ceil(ffn / tile) * A * d * 4 bytes of
     * partials.  Compiled for block_rows 64 (tile variant 1), 128 (variant
     * 1, taken automatically when tile_variant is 0) and 192 (variant 0);
     * other combinations and the unfused ablation return
     * MOE_ERR_UNSUPPORTED when 2 is asked for.  Rounding differs from the
     * separate down GEMM (other summation order). */
    int fuse_down;
    /* Schedule of the fused gate/up GEMM: the skew-aware dynamic work
     * assignment the method leaves as future work ([R] abstract; "Editorial
     * extensions").  0 = automatic: schedule 3's table with its merge rule
     * where it can run, else 1.  1 = one workgroup per (schedule block,
     * column tile) unit, in rounds of the GPU's 256 CUs, 2 = stream-K: 256
     * persistent workgroups share the K steps of all units evenly -- the
     * unit count is the routed block count times the column tiles, read on
     * the device -- so a skewed routing that leaves a ragged last round, or
     * fewer units than CUs, still keeps every CU streaming.  A unit split
     * between workgroups is finished by the workgroup that completes it,
     * adding the fp32 partial sums in K order (deterministic).  Runs the
     * 128-row tile with one 16-column subtile per wave (variant 3 of
     * tile_variant): block_rows must be 0 (taken as 128) or 128,
     * tile_variant 0 or 4, and
     * not with the unfused ablation, the fused down projection or gather
     * mode 3 (else MOE_ERR_UNSUPPORTED when 2 is asked for).  The
     * workspace grows by 2 * 256 partial slots of 128 KiB and one counter
     * per unit, which the routing kernels clear on every call.  Rounding
     * differs from schedule 1 where a unit is split (other association of
     * the K sum).  3 = variable block rows: the routing kernels build a
     * second block table for the gate/up GEMM in which an expert with more
     * than 128 rows takes blocks of 256 rows (the last one holding the
     * rest), so its weight tile is read once per 256 rows; the GEMM runs
     * the 128-row narrow tile on blocks of up to 128 rows and the same tile
     * at 256 rows on the others, in one launch.  The down GEMM keeps the
     * 128-row blocks.  Asked for, the table always merges; automatic (0), it
     * merges only when the 128-row table needs more than one round of 256
     * workgroups and the merged one at most one, and is the 128-row table
     * otherwise.  Same conditions as 2 (block_rows 0 or 128, tile_variant 0
     * or 4, not with the unfused ablation, the fused down projection,
     * gather mode 3, the XCD-grouped or longest-first orders: else
     * MOE_ERR_UNSUPPORTED when 3 is asked for); the workspace grows by 12
     * bytes per block.  With the K start rotated per expert (the automatic
     * rotation) or not rotated, the bytes equal schedule 1's. */
    int schedule;
    /* NULL, or 7 hipEvent_t handles created by the caller (for instance
     * with moe_timer_create).  events[0] is recorded on the stream before
     * the first kernel and events[i] right after kernel i (1 route, 2
     * histogram+scan+schedule, 3 reorder+gather, 4 fused gate/up SwiGLU
     * GEMM (or the three unfused kernels), 5 down GEMM, 6 weighted
     * combination).  With the one-workgroup
     * routing kernel, events 1 and 2 are both recorded after it; with the
     * gather inside the GEMM, event 3 follows the routing directly; with
     * the combination folded, events 5 and 6 both follow the down GEMM.
     * NULL entries are skipped.  moe_route records 0..3 only. */
    void *const *stage_events;
} moe_options;

/* Returns MOE_ABI_VERSION. */
int moe_abi_version(void);

/* Static text for a moe_status value (never NULL). */
const char *moe_status_string(int status);

/* Host-only size query: bytes of workspace moe_forward needs for these
 * sizes with the automatic options.  T = 0 gives 0.  Same checks and error
 * codes as moe_forward (pointer checks aside). */
int moe_workspace_size(int T, int d, int ffn, int E, int top_k, size_t *bytes);

/* As moe_workspace_size for moe_forward_ex with options `opt` (NULL means
 * automatic). */
int moe_workspace_size_ex(int T, int d, int ffn, int E, int top_k, const moe_options *opt,
                          size_t *bytes);

/* Host-only: the block_rows (BLOCK_M) and split_k (parts of the down
 * reduction) the library would use for these sizes and options, and whether
 * the down projection is fused into the gate/up GEMM (fused_down: 1 or 0).
 * Any output pointer may be NULL. */
int moe_plan(int T, int d, int ffn, int E, int top_k, const moe_options *opt,
             int *block_rows, int *split_k, int *fused_down);

/* What moe_forward_ex would launch for these sizes and options. */
typedef struct moe_plan_info {
    int block_rows;        /* BLOCK_M of the schedule                          */
    int split_k;           /* parts of the down reduction (column tiles of the
                              gate/up GEMM when the down projection is fused) */
    int fused_down;        /* 1: the down projection runs inside the gate/up GEMM */
    int routing_launches;  /* 1, 2 or 3 kernels for route, histogram/scan/
                              schedule and reorder                            */
    int gather_launch;     /* 1: a separate gather kernel writes x_perm        */
    int gate_up_variant;   /* tile variant of the gate/up GEMM (moe_options)   */
    int down_variant;      /* tile variant of the down GEMM (-1 when fused)    */
    int unfused_swiglu;    /* 1: the ablation's three kernels replace the fused GEMM */
    int fold_combine;      /* 1: the combination runs in the down GEMM         */
    int xcd_grouped;       /* 1: GEMM workgroups grouped by XCD                */
    int launches;          /* kernels per forward pass                         */
    int split_on_device;   /* 1: split_k is an upper bound; the down GEMM and
                              the combination take the number of parts from
                              the routed block count on the device: the split
                              whose workgroup count (blocks x column tiles x
                              parts) is nearest to one round of 256, at least
                              1 and at most split_k                           */
    int stream_k;          /* 1: the gate/up GEMM runs the stream-K schedule   */
    int variable_rows;     /* 1: the gate/up GEMM runs over the variable-size
                              block table, merged when one round needs it;
                              2: merged always (schedule 3); 0: not        */
    long long var_table_offset; /* byte offsets in the workspace of that table
                              ([nb_max, 3] int32: expert, first row, rows)  */
    long long var_count_offset; /* and of its block count (int32; -1 when the
                              routing kernels kept the fixed table), for
                              inspection after a call; -1 when not built   */
} moe_plan_info;

/* Host-only: fills *info with the launch plan moe_forward_ex would follow.
 * Same checks and error codes as moe_workspace_size_ex; info NULL returns
 * MOE_ERR_NULL.  T = 0 plans nothing (every field 0). */
int moe_plan_ex(int T, int d, int ffn, int E, int top_k, const moe_options *opt,
                moe_plan_info *info);

/*
 * The MoE forward pass ([R] "The reading"; abstract).
 *
 *   x             bf16 [T, d]           token activations
 *   router_logits fp32 [T, E]           router logits (finite values)
 *   W_gate_up     bf16 [E, 2*ffn, d]    per expert: gate rows [0, ffn),
 *                                       then up rows [ffn, 2*ffn)
 *   W_down        bf16 [E, d, ffn]      per expert down projection
 *   top_k         experts per token, 1..min(E, 16)
 *   renormalize   softmax: 1 = softmax over the top_k selected logits,
 *                 0 = softmax over all E logits, then take the top_k;
 *                 sigmoid: 1 = divide by the sum of the top_k sigmoids
 *   out           bf16 [T, d]           written; must not alias an input
 *   score_func    MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID
 *   workspace     device buffer of at least moe_workspace_size bytes,
 *                 256-byte aligned
 *
 * Computes, for each token t,
 *   out[t] = bf16_rne( sum_j w[t,j] * Wd[e_j] (silu(Wg[e_j] x_t) * Wu[e_j] x_t) )
 * where e_0..e_{k-1} are the top_k experts by logit (descending, equal
 * logits to the lower expert index) and w[t,j] their routing weights.
 * Constraints: T >= 0 (T = 0 is a no-op), 1 <= E <= 512, d and ffn
 * positive multiples of 64, T*top_k <= 2^20, pointers 16-byte aligned.
 * Deterministic: the same inputs give bitwise the same out.
 */
int moe_forward(const uint16_t *x, const float *router_logits, const uint16_t *W_gate_up,
                const uint16_t *W_down, int top_k, int renormalize, uint16_t *out,
                int T, int d, int ffn, int E, int score_func,
                void *workspace, size_t workspace_bytes, void *hip_stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as moe_forward with the automatic options,
 * with the workspace taken from a fixed device array inside the library
 * (MOE_STATIC_WORKSPACE_BYTES, one per GPU) instead of a caller's buffer.
 * Nothing is allocated or freed by this call.
 *
 * Arguments, layouts, ownership and checks as moe_forward (the caller still
 * passes x, router_logits, the weights and out).  The array belongs to the
 * GPU of hip_stream (the current device for a NULL stream); its address is
 * looked up once per GPU, on the first call there.
 *
 * Errors: as moe_forward, plus MOE_ERR_STATIC_LIMIT (nothing enqueued) when
 * moe_workspace_size for these sizes exceeds MOE_STATIC_WORKSPACE_BYTES --
 * Mixtral-shaped T <= 512 and DeepSeek-V3-shaped T <= 512 fit; and
 * MOE_ERR_HIP when the device or the array's address cannot be obtained.
 *
 * Every call on one GPU shares that GPU's array, and each call leaves its
 * own intermediates there: calls on one GPU must be ordered (one stream, or
 * streams synchronised with each other); calls that overlap race on the
 * array and give wrong results.  The array starts with no contract: the
 * kernels write every byte they read within a call. */
int moe_forward_static(const uint16_t *x, const float *router_logits, const uint16_t *W_gate_up,
                       const uint16_t *W_down, int top_k, int renormalize, uint16_t *out,
                       int T, int d, int ffn, int E, int score_func, void *hip_stream);

/* moe_forward with options (NULL = automatic, identical to moe_forward).
 * The workspace must hold moe_workspace_size_ex(..., opt, ...) bytes. */
int moe_forward_ex(const uint16_t *x, const float *router_logits, const uint16_t *W_gate_up,
                   const uint16_t *W_down, int top_k, int renormalize, uint16_t *out,
                   int T, int d, int ffn, int E, int score_func, const moe_options *opt,
                   void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Router scores ([R] "The reading": tokens are scored before they are
 * routed; "Assumptions & free parameters", Eq. (1)-(4): the standard router,
 * a linear map of each token's hidden state to one score per expert):
 *
 *   logits[t][e] = sum_c x[t][c] * W_router[e][c]
 *
 *   x         bf16 [T, d]   token activations
 *   W_router  bf16 [E, d]   one row per expert (K-contiguous, like the
 *                           expert weights)
 *   logits    fp32 [T, E]   written (fp32 accumulation; deterministic: the
 *                           reduction over d is split into a fixed number
 *                           of parts for these sizes, added in part order)
 *   workspace device buffer of moe_router_workspace_size bytes (256-byte
 *             aligned; may be NULL when that size is 0) for the partial sums
 *
 * Constraints: T >= 0 (T = 0 is a no-op), 1 <= E <= 512, d a positive
 * multiple of 64 with 64*d < 2^31, T <= 2^20, pointers 16-byte aligned.
 * Enqueued on hip_stream.
 */
int moe_router_logits(const uint16_t *x, const uint16_t *W_router, float *logits, int T, int d,
                      int E, void *workspace, size_t workspace_bytes, void *hip_stream);

/* Host-only size query for moe_router_logits. */
int moe_router_workspace_size(int T, int d, int E, size_t *bytes);

/* moe_forward_ex from the hidden states: the router scores of
 * moe_router_logits, then the forward pass on them; when the scores are
 * computed in several partial sums, the routing kernel adds them (in the
 * same order) as it reads them.  logits_out (fp32 [T, E], 16-byte aligned)
 * receives the scores (bitwise those of moe_router_logits), or may be NULL.
 * Same workspace size as moe_forward_ex; the constraints of both calls
 * apply.  The stage events (opt) time the forward pass after the router
 * GEMM: events[0] is recorded after it. */
int moe_forward_router(const uint16_t *x, const uint16_t *W_router, const uint16_t *W_gate_up,
                       const uint16_t *W_down, int top_k, int renormalize, uint16_t *out,
                       float *logits_out, int T, int d, int ffn, int E, int score_func,
                       const moe_options *opt, void *workspace, size_t workspace_bytes,
                       void *hip_stream);

/* Host-only size query for moe_route. */
int moe_route_workspace_size(int T, int E, int top_k, const moe_options *opt, size_t *bytes);

/*
 * Routing only: the first three kernels of moe_forward, with their results
 * copied to caller buffers ([R] "The reading": scoring and reordering;
 * "What carries the argument": the (expert, token-offset) block table).
 * A = T*top_k.  Every output may be NULL (not produced):
 *   topk_ids int32 [T, top_k]   experts of each token, descending logit,
 *                               equal logits to the lower index
 *   topk_w   fp32  [T, top_k]   routing weights (as in moe_forward)
 *   counts   int32 [E]          rows routed to each expert
 *   offsets  int32 [E+1]        exclusive prefix sum of counts
 *   perm     int32 [A]          sorted row p -> flat index t*top_k + j;
 *                               rows of one expert keep ascending flat index
 *   inv      int32 [A]          flat index -> sorted row
 *   blocks   int32 [nb_max, 2]  (expert, first sorted row) of each block of
 *                               up to block_rows rows of one expert, experts
 *                               ascending; nb_max = ceil(A/BM) + min(E, A)
 *   nb       int32 [1]          number of valid blocks (device)
 *   block_order int32 [nb_max]  the blocks longest first (the launch order
 *                               of xcd_order = 3): a stable sort of the
 *                               block indices by decreasing row count --
 *                               the full blocks in block order, then each
 *                               expert's partial last block by rows
 *                               descending, equal rows to the lower expert
 *   x, x_perm  bf16 [T, d] and [A, d]: if both are non-NULL, x_perm[p] =
 *                               x[perm[p] / top_k] is also written (d > 0,
 *                               a multiple of 64)
 *   bm_used  HOST int [1]       the block_rows used
 * The workspace must hold moe_route_workspace_size bytes.
 */
int moe_route(const float *router_logits, int T, int E, int top_k, int renormalize, int score_func,
              const moe_options *opt,
              int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets,
              int32_t *perm, int32_t *inv, int32_t *blocks, int32_t *nb, int32_t *block_order,
              const uint16_t *x, int d, uint16_t *x_perm, int *bm_used,
              void *workspace, size_t workspace_bytes, void *hip_stream);

/* Thin wrappers over HIP events for timing the stages of moe_forward_ex
 * (moe_options.stage_events).  The events are created without a
 * system-scope fence on record: they time work, they do not make its results
 * visible to the host.  Each returns a moe_status. */
int moe_timer_create(void **event);
int moe_timer_destroy(void *event);
/* Records `event` on hip_stream (NULL = the default stream), for timing a
 * call that takes no stage events (e.g. moe_router_logits). */
int moe_timer_record(void *event, void *hip_stream);
/* Milliseconds between two recorded events; waits for `stop` to complete. */
int moe_timer_elapsed_ms(void *start, void *stop, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
