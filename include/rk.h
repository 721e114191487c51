/*
 * rk.h -- C ABI of librk: request-centric masked multi-head attention
 * (forward and backward) with time RoPE, for AMD Instinct MI355X (gfx950).
 *
 * One packed buffer holds R requests.  Each request is one user sequence:
 * optional PROFILE tokens, HISTORY tokens, optional same-day REALTIME
 * tokens and N CANDIDATE (target) tokens, in that order.  Every token
 * carries an int64 timestamp in seconds.  The operations exported:
 *
 *   rk_mask_plan        classify every 128 x 64 (query x key) tile of every
 *                       request as EMPTY / PARTIAL / FULL with its exact
 *                       visible-pair count, list the non-empty key tiles of
 *                       each query tile (CSR) and build the launch schedule;
 *   rk_time_rope        rotate Q or K by time RoPE;
 *   rk_masked_attn_fwd  softmax(Q K^T * scale + M) V over the plan, with
 *                       optional fused time RoPE;
 *   rk_masked_attn_bwd  its gradients with respect to Q, K and V;
 *   rk_pointwise_attn_fwd
 *                       HSTU's pointwise (SiLU) attention over the same plan;
 *   rk_compress_layout / rk_prune_layout / rk_gather_sum
 *                       LazFormer's history compression and per-layer
 *                       history pruning, before and between layers;
 *   rk_pruned_history_length_ex / rk_prune_layout_ex / rk_gather_mean
 *                       SORT's query pruning: exponential schedule and the
 *                       pooled form.
 *
 * Sources (titles and sections of the pages this library follows):
 *  - CADET: Context-Conditioned Ads CTR Prediction With a Decoder-Only
 *    Transformer -- "why mask the most recent hour in training" (delay
 *    mask equation), "time encoding and self-gating" (time RoPE equation),
 *    "how to score hundreds of candidates in 50 ms" (candidates appended to
 *    the user sequence, seeing the history but not each other; a
 *    FlashAttention kernel that skips fully masked blocks; packed
 *    variable-length sequences with start/end offsets).
 *  - SORT: A Systematically Optimized Ranking Transformer for
 *    Industrial-scale Recommenders -- section 3.1 (U2U, C2U, C2C regions),
 *    section 3.2.1 (sliding-window local attention in U2U), section 4
 *    (sparse attention operator that skips fully masked blocks).
 *  - LazFormer -- section 2.3, equations 19-21 (allowed relation with
 *    window W; -inf mask; SparseAttn = softmax(QK^T/sqrt(d_k) + M) V).
 *  - MTGR (Meituan generative recommendation, blog post) -- model
 *    structure, "mixed dynamic mask".
 *  - HSTU, appendix H (M-FALCON): one pass with the modified causal mask
 *    equals separate causal passes per candidate.
 *
 * Visibility of key j for query i of the same request (p = request-local
 * position, t = timestamp, S = {PROFILE, HISTORY}):
 *   key j is a CANDIDATE          : visible iff i == j;
 *   i in S, j in S                : with RK_STATIC_BIDIRECTIONAL always;
 *                                   otherwise p_j <= p_i, and
 *                                   (window == 0 or p_i - p_j < window or
 *                                    p_i >= |S| - global_tail), and
 *                                   (delay == 0 or t_j <= t_i - delay);
 *   i in S, j REALTIME            : never;
 *   i REALTIME, j in S            : always;
 *   i REALTIME, j REALTIME        : p_j <= p_i and t_j <= t_i;
 *   i CANDIDATE, j in S           : always;
 *   i CANDIDATE, j REALTIME       : t_j < t_i.
 * A query with no visible key outputs 0 (log-sum-exp -inf).
 *
 * Conventions
 *  - Every device buffer is owned by the caller.  The library never
 *    allocates device memory: the plan lives in a caller-provided
 *    workspace whose size is computed on the host.
 *  - All work is asynchronous on the caller's stream (`stream` is a
 *    hipStream_t; NULL means the default stream).  Argument validation is
 *    synchronous and happens before anything is enqueued; a call that
 *    returns an error has enqueued nothing.
 *  - Checks that need device data (segment order, timestamp order) are
 *    recorded by rk_mask_plan on the device and reported by rk_plan_stats.
 *    Every kernel that runs over a plan whose checks failed stores NaN in
 *    each value it writes (O, LSE, dQ, dK, dV, the pointwise output), so a
 *    misused plan is visible even to a caller that never reads the stats.
 *  - No global mutable state: concurrent calls on distinct plans and
 *    buffers are safe.
 *  - Every struct starts with `struct_size` (= sizeof of the struct the
 *    caller was compiled against).
 */
#ifndef RK_H
#define RK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RK_ABI_VERSION 4

typedef enum rk_status {
  RK_OK = 0,
  RK_ERR_INVALID_ARG = 1,         /* NULL pointer, bad size, bad offsets or parameters */
  RK_ERR_SEGMENT_ORDER = 2,       /* segment kinds out of order or out of range (device check) */
  RK_ERR_UNSORTED_TIME = 3,       /* timestamps not non-decreasing where required (device check) */
  RK_ERR_UNSUPPORTED = 4,         /* dtype / d_head / alignment / size not supported */
  RK_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace smaller than the size query returned */
  RK_ERR_HIP = 6                  /* a HIP runtime call failed */
} rk_status;

typedef enum rk_dtype { RK_F32 = 0, RK_BF16 = 1 } rk_dtype;

/* Segment kinds (per token, uint8).  Non-decreasing inside a request. */
enum { RK_SEG_PROFILE = 0, RK_SEG_HISTORY = 1, RK_SEG_REALTIME = 2, RK_SEG_CANDIDATE = 3 };

/* Tile classes of the plan. */
enum { RK_TILE_EMPTY = 0, RK_TILE_PARTIAL = 1, RK_TILE_FULL = 2 };

#define RK_TILE_Q 128 /* query rows per tile */
#define RK_TILE_K 64  /* key columns per tile */
#define RK_SPLIT_SLOTS 768 /* extra attention launch slots of a RK_QUERY_CANDIDATES_ONLY
                              plan's work list, and the rows of its split table */

/* rk_mask_params.flags */
#define RK_STATIC_BIDIRECTIONAL 0x1u /* PROFILE+HISTORY mutually visible (MTGR static part) */
#define RK_QUERY_CANDIDATES_ONLY 0x2u /* serving call (HSTU, App. H, M-FALCON): the launch
                                         schedule covers only the query tiles that hold at
                                         least one CANDIDATE row, so rk_masked_attn_fwd
                                         writes O / LSE rows of those tiles only (rows
                                         elsewhere are left as they were).  Masks, tile
                                         classes, counts, CSR and totals are those of the
                                         whole batch.  When few such tiles exist, the key
                                         range of each is cut into chunks run by separate
                                         workgroups whose partial softmax results a merge
                                         pass combines (more attention workspace). */
#define RK_PLAN_BACKWARD 0x4u /* also build the key-major tables rk_masked_attn_bwd needs:
                                 for every block of 128 keys (k-tiles 2 kb and 2 kb + 1 of a
                                 request), the ascending list of 128-row query tiles with a
                                 visible pair in either k-tile (FULL only when both k-tiles
                                 exist and are FULL, else PARTIAL), and a schedule of (key
                                 block, head) work items.  Not allowed with
                                 RK_QUERY_CANDIDATES_ONLY. */

/* Segment-kind bits of rk_rope_params.kinds: bit k selects kind k. */
#define RK_KIND_BIT(k) (1u << (k))

/* rk_attn_args.flags */
#define RK_ATTN_REFERENCE_KERNEL 0x1u /* force the plain (non-MFMA) kernel */
#define RK_ATTN_K_PREROTATED 0x2u     /* with rope and / or qk_norm: K was already
                                         prepared by rk_time_rope or rk_qk_norm_rope (same
                                         parameters and anchors); only Q is transformed */

/*
 * A packed batch (CADET, "how to score hundreds of candidates": all tokens
 * of a batch in one buffer plus per-sequence start/end offsets).
 *   req_offsets_host/_dev : int32 [num_requests + 1]; [0] == 0,
 *                           non-decreasing, [num_requests] == total_tokens.
 *                           Host and device copies must hold equal values.
 *   seg_kind_dev          : uint8 [total_tokens], RK_SEG_*; non-decreasing
 *                           inside each request.
 *   timestamps_dev        : int64 [total_tokens], seconds.  Must be
 *                           non-decreasing inside REALTIME and, when the
 *                           static part is causal and delay > 0, inside
 *                           PROFILE and inside HISTORY (each on its own).
 *                           In that mode the keys a static row sees by the
 *                           delay rule are a prefix of PROFILE and a prefix
 *                           of HISTORY, and they must form one run of
 *                           positions: profile tokens dated at the anchor
 *                           ("now", the pages give them no time) or dated
 *                           no later than the first history token always
 *                           do; profile times interleaved with history
 *                           times can leave a row with two runs, which is
 *                           reported as RK_ERR_UNSORTED_TIME.
 *   anchors_dev           : int64 [num_requests]; time origin of each
 *                           request's RoPE angles (any value; outputs of
 *                           the attention do not depend on it).
 * All device arrays must stay valid and unchanged while a plan built from
 * the batch is in use.
 */
typedef struct rk_batch {
  uint32_t struct_size;
  int32_t num_requests;
  int32_t total_tokens;
  const int32_t* req_offsets_host;
  const int32_t* req_offsets_dev;
  const uint8_t* seg_kind_dev;
  const int64_t* timestamps_dev;
  const int64_t* anchors_dev;
} rk_batch;

/* Mask parameters (CADET delay mask; SORT / LazFormer window; MTGR static part). */
typedef struct rk_mask_params {
  uint32_t struct_size;
  uint32_t flags;       /* RK_STATIC_BIDIRECTIONAL, RK_QUERY_CANDIDATES_ONLY,
                           RK_PLAN_BACKWARD, or 0 */
  int64_t delay;        /* Delta_delay in timestamp units, >= 0; 0 = off */
  int32_t window;       /* keys kept including self, >= 0; 0 = off */
  int32_t global_tail;  /* LazFormer (section 2.3, eq. 19-21) G >= 0: the last G static
                           (profile + history) positions of a request are global queries,
                           exempt from the window (still causal, still delayed) */
} rk_mask_params;

/* Time RoPE (CADET, "time encoding"): pair (2i, 2i+1), i = 0 .. d/2-1, of a
 * token with time t in request r is rotated counter-clockwise by
 *   alpha_i = (t - anchor_r) * phi_min / dt_max * base^(2i/d).
 * dt_max is in timestamp units (1 year = 31,536,000 s on the page). */
typedef struct rk_rope_params {
  uint32_t struct_size;
  uint32_t kinds; /* rk_time_rope only: rotate tokens whose segment kind k has
                     RK_KIND_BIT(k) set, leave the other rows of x_out as they
                     were; 0 = every token.  Must be 0 in rk_attn_args.rope.
                     A serving call rotates the CANDIDATE keys into a buffer
                     whose history keys were rotated once before (HSTU,
                     App. H: history K/V cached across candidate batches). */
  double phi_min; /* > 0 */
  double dt_max;  /* > 0 */
  double base;    /* > 0 */
} rk_rope_params;

/* QK Norm (TM20K section 2: QK Norm after the query / key projections keeps
 * extreme scores in check; SORT section 3.3.2: RMSNorm on Q and K before the
 * scores): every [d_head] row of Q and K becomes
 *   x / sqrt(mean(x^2) + eps) * gamma,
 * applied before time RoPE.  One gain vector for Q and one for K, shared by
 * every head (the pages give no shape); NULL gains are 1. */
typedef struct rk_qk_norm_params {
  uint32_t struct_size;
  float eps;             /* > 0 */
  const float* gamma_q;  /* device fp32 [d_head] or NULL */
  const float* gamma_k;  /* device fp32 [d_head] or NULL */
} rk_qk_norm_params;

typedef struct rk_plan rk_plan;

/* Host-side description of a plan.  Byte offsets are relative to the start
 * of the plan workspace; the arrays there are valid once the stream has
 * executed rk_mask_plan's work. */
typedef struct rk_plan_info {
  uint32_t struct_size;
  int32_t num_requests;
  int32_t total_tokens;
  int32_t num_heads;
  int64_t num_qtiles;          /* sum over requests of ceil(L_r / 128) */
  int64_t num_tiles;           /* sum over requests of ceil(L_r/128)*ceil(L_r/64) */
  int64_t num_sched_slots;     /* one slot per (q-tile, head) work item, LPT / XCD order */
  const void* workspace;
  size_t off_tile_class;       /* uint8 [num_tiles], RK_TILE_*, requests in order, row-major [qt][kt] */
  size_t off_tile_count;       /* int32 [num_tiles], visible pairs per tile */
  size_t off_qtile_ptr;        /* int32 [num_qtiles + 1], CSR row pointers */
  size_t off_ktile_idx;        /* int32 [num_tiles] (first qtile_ptr[num_qtiles] used), request-local kt, ascending */
  size_t off_row_desc;         /* int32 [total_tokens][2]: visible keys of a query = [lo, hi) plus bit 31 of hi = self */
  size_t off_sched;            /* int32 [num_sched_slots]: work item = qtile * num_heads + head, or -1 */
  int64_t num_work_slots;      /* RK_QUERY_CANDIDATES_ONLY plans: grid size of the attention
                                  (num_sched_slots + RK_SPLIT_SLOTS), else 0 (the grid is the
                                  schedule) */
  size_t off_work;             /* int32 [num_work_slots][4]: (item, first, end, part) = CSR
                                  entries [first, end) of the item's q-tile (end -1: all of
                                  them); part >= 0 names the partial result of a split item;
                                  item -1 = idle slot.  With RK_SPLIT_SLOTS / 2 or more
                                  scheduled items it mirrors the schedule (whole items);
                                  with fewer it lists them in schedule order, in chunks */
  size_t off_splits;           /* int32 [RK_SPLIT_SLOTS][4]: (item, first part, parts, 0) of
                                  each split item, item -1 past the last */
  /* key-major tables, filled for RK_PLAN_BACKWARD plans (offsets 0 and
     num_ksched_slots 0 otherwise) */
  int64_t num_kblocks;         /* sum over requests of ceil(L_r / 128): key blocks of 128 */
  int64_t num_ksched_slots;    /* one slot per (key block, head) work item, LPT / XCD order */
  size_t off_kt_ptr;           /* int32 [num_kblocks + 1], CSR row pointers per global key
                                  block */
  size_t off_qtile_word;       /* int32 [kt_ptr[num_kblocks]]: request-local query tile, ascending,
                                  | (1 << 31) when the tile is PARTIAL */
  size_t off_ksched;           /* int32 [num_ksched_slots]: work item = global key block *
                                  num_heads + head, or -1 */
} rk_plan_info;

/* Totals of a plan (per head). */
typedef struct rk_plan_totals {
  uint32_t struct_size;
  uint32_t device_errors;      /* bit 0: segment order/kind, bit 1: timestamp order,
                                  bit 2: a static row's delayed keys form two runs */
  int64_t visible_pairs;       /* sum of all tile counts */
  int64_t full_tiles;
  int64_t partial_tiles;
  int64_t empty_tiles;
  int32_t work_entries;        /* slots of the work list in use or mirrored from the
                                  schedule (RK_QUERY_CANDIDATES_ONLY) */
  int32_t split_items;         /* items whose key range is split */
} rk_plan_totals;

/*
 * Attention arguments.  Q, K, V, O are [token, head, d] views with d
 * contiguous and the given element strides.  d_head is any multiple of 8
 * from 8 to 128 (CADET's 88, for example): the kernels run at the next
 * instance width (64 or 128 on the matrix cores, 32, 64 or 128 on the plain
 * kernel) with zero columns that never touch the tensors.  dtype RK_BF16:
 * bf16 inputs and output, fp32 accumulation and softmax, bf16 MFMA (needs
 * 16-byte aligned base pointers and strides that are multiples of 8;
 * RK_ATTN_REFERENCE_KERNEL selects the plain kernel).  dtype RK_F32: fp32
 * throughout on the plain kernel.
 *   lse       : optional float [num_heads][total_tokens], natural-log
 *               log-sum-exp of the scaled scores; -inf for empty rows.
 *   scale     : score scale; 0 selects 1/sqrt(d_head).
 *   rope      : NULL = inputs are used as given; otherwise Q and K are
 *               rotated by time RoPE with the plan's batch timestamps and
 *               anchors (Q while it is staged, K by a pass into the
 *               workspace, or not at all with RK_ATTN_K_PREROTATED, e.g.
 *               for a cache of rotated history keys).
 *   workspace : device memory of at least rk_attn_workspace_size bytes,
 *               256-byte aligned (may be NULL when that size is 0).
 *   qk_norm   : NULL, or QK Norm applied to Q and K before time RoPE (Q
 *               while it is staged, K by the pass into the workspace unless
 *               RK_ATTN_K_PREROTATED); d_head in {32, 64, 128}.
 * O must not overlap Q, K, V or the workspace.
 */
typedef struct rk_attn_args {
  uint32_t struct_size;
  uint32_t flags;
  rk_dtype dtype;
  int32_t num_heads;
  int32_t d_head;
  int32_t reserved;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t o_stride_tok, o_stride_head;
  float scale;
  float reserved2;
  const rk_rope_params* rope;
  void* workspace;
  size_t workspace_bytes;
  const rk_qk_norm_params* qk_norm;
} rk_attn_args;

/* Name of a status code (static string). */
const char* rk_status_string(rk_status s);

/* ABI version (RK_ABI_VERSION of the library). */
int32_t rk_abi_version(void);

/*
 * Bytes of plan workspace needed for `b` and `num_heads` (host only; reads
 * b->req_offsets_host).  Errors: RK_ERR_INVALID_ARG.
 */
rk_status rk_plan_workspace_size(const rk_batch* b, int32_t num_heads, size_t* bytes);

/*
 * Build the tile plan of a batch (CADET "50 ms" section: skip fully masked
 * blocks; SORT section 4: block computation with a mask pre-check that
 * skips fully masked blocks).
 *   workspace : device memory, 256-byte aligned, >= rk_plan_workspace_size.
 *               Owned by the caller; must outlive every use of the plan.
 *   plan_out  : receives a small host object, freed with rk_plan_destroy
 *               (after the last work that uses it has completed).
 * Per tile (qt, kt) of request r, covering request-local query rows
 * [128 qt, 128 qt + 128) and keys [64 kt, 64 kt + 64): count = visible
 * in-range pairs; FULL iff all 8192 cells are in range and visible; EMPTY
 * iff count == 0; PARTIAL otherwise.  The schedule orders the query tiles
 * of each (request, head) by descending non-empty tile count and spreads
 * (request, head) groups over the chip's eight XCDs.
 * Host tables computed from req_offsets_host reach the GPU through pinned
 * host blocks the library keeps for this (at most 64, each 64 KiB or more,
 * reused as the planner kernels finish reading them, held until the process
 * ends); with all of them in use, or while `stream` is being captured into
 * a graph (a replay reads the source again; the plan's own host copy, kept
 * until rk_plan_destroy, still holds it), the call copies its tables up
 * with hipMemcpyAsync instead.  The call is asynchronous either way.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_UNSUPPORTED (more than 2^31-1 tiles
 * or work items), RK_ERR_WORKSPACE_TOO_SMALL, RK_ERR_HIP.
 */
rk_status rk_mask_plan(const rk_batch* b, const rk_mask_params* m, int32_t num_heads,
                       void* workspace, size_t workspace_bytes, rk_plan** plan_out,
                       void* stream);

/* Host-side plan description (no device access).  Errors: INVALID_ARG. */
rk_status rk_plan_get_info(const rk_plan* p, rk_plan_info* out);

/*
 * Synchronise `stream`, then read the plan's totals and device checks.
 * Returns RK_ERR_SEGMENT_ORDER or RK_ERR_UNSORTED_TIME when the batch
 * broke the segment or time order (the totals are still filled in), and
 * RK_ERR_HIP on a runtime failure.
 */
rk_status rk_plan_stats(const rk_plan* p, rk_plan_totals* out, void* stream);

/* Free the host object of a plan (the workspace stays the caller's). */
void rk_plan_destroy(rk_plan* p);

/*
 * Time RoPE (CADET, "time encoding and self-gating"): rotate x_in into
 * x_out (same shape [total_tokens, num_heads, d_head], element strides as
 * given; in place allowed when the strides are equal).  Angles use
 * (t - anchor_r) computed exactly in int64; the phase is reduced in
 * double precision before sin/cos.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_UNSUPPORTED (d_head odd or > 128),
 * RK_ERR_HIP.
 */
rk_status rk_time_rope(const rk_batch* b, const rk_rope_params* r, const void* x_in, void* x_out,
                       rk_dtype dtype, int32_t num_heads, int32_t d_head,
                       int64_t in_stride_tok, int64_t in_stride_head,
                       int64_t out_stride_tok, int64_t out_stride_head, void* stream);

/*
 * QK Norm then time RoPE in one pass (the K side of a forward with qk_norm,
 * e.g. to fill a cache of prepared keys for RK_ATTN_K_PREROTATED): every row
 * x of x_in [total_tokens, num_heads, d_head] becomes
 * rotate(x / sqrt(mean(x^2) + eps) * gamma) in x_out; r may be NULL (norm
 * only).  gamma: device fp32 [d_head] or NULL (gain 1).  Strides and kinds as
 * in rk_time_rope.  Errors: RK_ERR_INVALID_ARG, RK_ERR_UNSUPPORTED (d_head not
 * in {32, 64, 128}), RK_ERR_HIP.
 */
rk_status rk_qk_norm_rope(const rk_batch* b, const rk_rope_params* r, float eps,
                          const float* gamma, const void* x_in, void* x_out, rk_dtype dtype,
                          int32_t num_heads, int32_t d_head, int64_t in_stride_tok,
                          int64_t in_stride_head, int64_t out_stride_tok,
                          int64_t out_stride_head, void* stream);

/* Workspace bytes rk_masked_attn_fwd needs for `a` on plan `p` (host only):
 * the rotated K when the call rotates K ([total_tokens][num_heads][d_head] of
 * dtype), plus, for RK_QUERY_CANDIDATES_ONLY plans, 2 * RK_SPLIT_SLOTS partial
 * results of 128 rows x (d_head + 2) floats (about 52 MB at d_head = 64). */
rk_status rk_attn_workspace_size(const rk_plan* p, const rk_attn_args* a, size_t* bytes);

/*
 * Masked attention forward over a plan (TM20K section 2.1 / LazFormer
 * eq. 21: softmax(Q K^T / sqrt(d) + M) V with M = 0 on visible pairs and
 * -inf elsewhere).  EMPTY tiles are never read; the per-element mask is
 * evaluated on PARTIAL tiles only.  One launch over the plan's schedule.
 * Errors: RK_ERR_INVALID_ARG (including num_heads != the plan's),
 * RK_ERR_UNSUPPORTED, RK_ERR_WORKSPACE_TOO_SMALL, RK_ERR_HIP.
 */
rk_status rk_masked_attn_fwd(const rk_plan* p, const rk_attn_args* a, void* stream);

/* Bytes of the library's scratch array on each GPU (128 MiB), used by
 * rk_masked_attn_fwd_noalloc. */
#define RK_STATIC_SCRATCH_BYTES (128u << 20)

/*
 * rk_masked_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation, kernels and results, with the workspace
 * taken from an array the library holds on each GPU instead of from the
 * caller.  a->workspace must be NULL and a->workspace_bytes 0.  The array
 * (RK_STATIC_SCRATCH_BYTES) is placed on a GPU when the library's scratch
 * module is first used there and stays until the process ends; this call
 * allocates nothing.  The array of the current device is used.  Every call
 * on one GPU shares that array: calls that may overlap on one GPU (different
 * streams, or host threads without ordering) race and must be serialised by
 * the caller; calls in order on one stream are safe.  Nothing in the array
 * needs to start at zero (every byte a call reads it wrote earlier in the
 * same call).
 * Errors: as rk_masked_attn_fwd; RK_ERR_INVALID_ARG when a workspace is
 * passed; RK_ERR_WORKSPACE_TOO_SMALL when rk_attn_workspace_size for `a`
 * exceeds RK_STATIC_SCRATCH_BYTES (e.g. K rotated by the call for more than
 * 128 MiB of keys: pass K pre-rotated instead).
 */
rk_status rk_masked_attn_fwd_noalloc(const rk_plan* p, const rk_attn_args* a, void* stream);

/*
 * Backward arguments.  Q, K, V, O, dO, dQ, dK, dV are [token, head, d]
 * views with d contiguous and the given element strides, all of `dtype`
 * (RK_BF16: fp32 accumulation, bf16 MFMA for d_head == 64 with 16-byte
 * aligned base pointers and strides that are multiples of 8; RK_F32: fp32
 * throughout).  d_head in {32, 64, 128}.
 *   q, k, v, rope, scale, flags : exactly as given to rk_masked_attn_fwd
 *               (RK_ATTN_REFERENCE_KERNEL, RK_ATTN_K_PREROTATED).
 *   o, lse    : that forward call's outputs; lse (float [num_heads]
 *               [total_tokens], natural log, -inf for empty rows) is
 *               required.
 *   d_o       : upstream gradient dLoss/dO.
 *   dq, dk, dv: outputs, every row written (0 for a query that sees no key
 *               and for a key that no query sees).  dQ and dK are the
 *               gradients with respect to the tensors passed in: with rope
 *               and without RK_ATTN_K_PREROTATED they are taken back
 *               through the rotation (with respect to the unrotated Q, K);
 *               with RK_ATTN_K_PREROTATED dk is the gradient with respect to
 *               the rotated K that was passed.
 *   workspace : device memory of at least rk_attn_bwd_workspace_size bytes,
 *               256-byte aligned.
 * Outputs must not overlap the inputs, each other or the workspace.
 */
typedef struct rk_attn_bwd_args {
  uint32_t struct_size;
  uint32_t flags;
  rk_dtype dtype;
  int32_t num_heads;
  int32_t d_head;
  int32_t reserved;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t do_stride_tok, do_stride_head;
  int64_t dq_stride_tok, dq_stride_head;
  int64_t dk_stride_tok, dk_stride_head;
  int64_t dv_stride_tok, dv_stride_head;
  float scale;
  float reserved2;
  const rk_rope_params* rope;
  void* workspace;
  size_t workspace_bytes;
  const rk_qk_norm_params* qk_norm; /* NULL, or the forward's QK Norm: the gradients are taken
                                       back through it (not with RK_ATTN_K_PREROTATED) */
  float* dgamma_q;  /* with qk_norm and its gamma_q: device fp32 [d_head], dLoss/dgamma_q
                       summed over tokens and heads; else ignored */
  float* dgamma_k;  /* likewise for gamma_k */
} rk_attn_bwd_args;

/* Workspace bytes rk_masked_attn_bwd needs for `a` on plan `p` (host only):
 * rowsum(dO * O) and the log2-unit LSE ([num_heads][total_tokens] fp32
 * each), plus, with rope or qk_norm, the rotated (normalised) Q and, unless
 * RK_ATTN_K_PREROTATED, K ([total_tokens][num_heads][d_head] of dtype
 * each), plus, with a QK Norm gain, the gain gradients' partial sums
 * (d_head fp32 per 512 rows of total_tokens * num_heads, per gain). */
rk_status rk_attn_bwd_workspace_size(const rk_plan* p, const rk_attn_bwd_args* a, size_t* bytes);

/*
 * Masked attention backward over a plan built with RK_PLAN_BACKWARD: the
 * gradients of a loss with respect to Q, K and V, given dLoss/dO, for the
 * forward softmax(Q K^T * scale + M) V of rk_masked_attn_fwd (TM20K
 * section 2.1, LazFormer eq. 21; trained with the delay mask as in
 * CADET, "why mask the most recent hour in training").  With P the masked
 * row softmax: dV = P^T dO; dS = P * (dO V^T - rowsum(dO * O)); dQ =
 * scale * dS K; dK = scale * dS^T Q.  P is recomputed from the forward's
 * log-sum-exp.  Two launches: one per (query tile, head) over the
 * query-major CSR writes dQ, one per (key block of 128, head) over the
 * key-major CSR writes dK and dV; EMPTY tiles are never read and the per-element mask
 * runs on PARTIAL tiles only.  With qk_norm (TM20K section 2: RMSNorm of the
 * rows of Q and K before the rotation, y = x * r * gamma, r = 1 /
 * sqrt(mean(x^2) + eps)) the two launches run on the normalised rows and a
 * pass per operand takes their gradients g back through the norm in place:
 * dx = r * gamma * g - x * r^3 * sum_j(gamma_j g_j x_j) / d_head, and
 * dgamma = sum over tokens and heads of g * x * r (bf16 operands: g is
 * rounded to bf16 once before that pass).  No atomics: results are
 * deterministic.
 * Errors: RK_ERR_INVALID_ARG (plan without RK_PLAN_BACKWARD, num_heads !=
 * the plan's, lse NULL, a gain without its gradient pointer, qk_norm with
 * RK_ATTN_K_PREROTATED, ...), RK_ERR_UNSUPPORTED, RK_ERR_WORKSPACE_TOO_SMALL,
 * RK_ERR_HIP.
 */
rk_status rk_masked_attn_bwd(const rk_plan* p, const rk_attn_bwd_args* a, void* stream);

/*
 * HSTU pointwise aggregated attention (HSTU eq. 2): over the same plan and
 * mask as rk_masked_attn_fwd,
 *   O_i = sum over visible j of SiLU(scale * q_i . k_j + rab_ij) v_j,
 * SiLU(x) = x / (1 + exp(-x)), with no normalisation (the pointwise form
 * keeps the number of related history points in the output).  rab^{p,t}
 * is shared by every head (the page): rab_ij = pos_bias[min(|p_i - p_j|,
 * num_pos_buckets - 1)] + time_bias[min(floor(log2(1 + |t_i - t_j|)),
 * num_time_buckets - 1)] (p request-local positions, t timestamps; the page
 * only says "a bucketing function of the time difference"); a NULL table
 * adds nothing.  No time RoPE (HSTU's rab carries position and time).
 */
typedef struct rk_pointwise_args {
  uint32_t struct_size;
  uint32_t flags;            /* RK_ATTN_REFERENCE_KERNEL or 0 */
  rk_dtype dtype;            /* RK_BF16 (bf16 MFMA for d_head == 64, 16-byte aligned rows) or
                                RK_F32; d_head in {32, 64, 128} */
  int32_t num_heads;
  int32_t d_head;
  int32_t num_pos_buckets;   /* 1 .. 4096 when pos_bias is set */
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t o_stride_tok, o_stride_head;
  float scale;               /* multiplies Q K^T; 0 selects 1 (no scale is printed) */
  int32_t num_time_buckets;  /* 1 .. 64 when time_bias is set */
  const float* pos_bias;     /* device fp32 [num_pos_buckets] or NULL */
  const float* time_bias;    /* device fp32 [num_time_buckets] or NULL */
} rk_pointwise_args;

/* With a RK_QUERY_CANDIDATES_ONLY plan (the serving call of HSTU App. H:
 * candidates against the cached history) only the O rows of query tiles that
 * hold a CANDIDATE row are written, each tile as in the full call; other rows
 * are left as they were.  The key range of a tile is never split (there is no
 * softmax state to merge).
 * Errors: RK_ERR_INVALID_ARG (including num_heads != the plan's),
 * RK_ERR_UNSUPPORTED, RK_ERR_HIP. */
rk_status rk_pointwise_attn_fwd(const rk_plan* p, const rk_pointwise_args* a, void* stream);

/* ---- LazFormer pre-passes (section 2.3): history compression and per-layer
 * history pruning.  The layout functions run on the host (they read host
 * copies of the segment kinds and timestamps, O(total_tokens)) and describe
 * each output token as a contiguous range of input rows; rk_gather_sum then
 * moves the feature rows (Q, K, V, hidden states, any width) on the device.
 * Readings where the page leaves the order open: histories are in time
 * order; the `keep` most recent history tokens are kept; the older ones are
 * summed in groups counted back from the kept part (a short group can only
 * be the oldest); a group carries its newest member's timestamp; pruning
 * drops the oldest history tokens; PROFILE, REALTIME and CANDIDATE tokens are
 * never compressed or pruned. */

/* Host copy of a packed layout. */
typedef struct rk_host_layout {
  uint32_t struct_size;
  int32_t num_requests;
  int32_t total_tokens;
  int32_t reserved;
  const int32_t* req_offsets; /* [num_requests + 1], as in rk_batch */
  const uint8_t* seg_kind;    /* [total_tokens] */
  const int64_t* timestamps;  /* [total_tokens]; HISTORY non-decreasing per request */
} rk_host_layout;

/* Caller-allocated host arrays receiving an output layout.  `capacity` is
 * the number of tokens the arrays hold; a call whose output is longer
 * returns RK_ERR_WORKSPACE_TOO_SMALL with total_tokens set to the length it
 * needs and writes nothing else (capacity 0 with NULL arrays is a size
 * query).  req_offsets must hold num_requests + 1 entries. */
typedef struct rk_layout_out {
  uint32_t struct_size;
  int32_t capacity;
  int32_t total_tokens;  /* set by the call */
  int32_t reserved;
  int32_t* req_offsets;  /* [num_requests + 1] */
  uint8_t* seg_kind;     /* [capacity] */
  int64_t* timestamps;   /* [capacity] */
  int32_t* ranges;       /* [capacity][2]: output token i = sum of input rows
                            [ranges[2i], ranges[2i+1]) */
} rk_layout_out;

/*
 * Group-sum compression (LazFormer eq. 16-18): per request with L HISTORY
 * tokens, the ell = min(L, keep) most recent stay as they are and the L - ell
 * older ones become ceil((L - ell) / group) group sums.  Output order per
 * request: PROFILE, group sums (oldest first), kept HISTORY, REALTIME,
 * CANDIDATE.  keep >= 0, group >= 1.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_SEGMENT_ORDER, RK_ERR_UNSORTED_TIME
 * (history out of time order), RK_ERR_WORKSPACE_TOO_SMALL (see
 * rk_layout_out).
 */
rk_status rk_compress_layout(const rk_host_layout* in, int32_t keep, int32_t group,
                             rk_layout_out* out);

/* History positions kept at layer `layer` (1-based) of `num_layers`
 * (LazFormer eq. 22): min(l_tilde, max(n_min, Round[l_tilde - (layer - 1) /
 * (num_layers - 1) * (l_tilde - n_min)])), Round taking halves away from
 * zero; l_tilde when num_layers == 1.  Errors: RK_ERR_INVALID_ARG. */
rk_status rk_pruned_history_length(int32_t l_tilde, int32_t n_min, int32_t layer,
                                   int32_t num_layers, int32_t* n_out);

/*
 * Input layout of layer `layer` (LazFormer eq. 22, "the next layer receives
 * the most recent history and all targets"): per request r, the last
 * N = rk_pruned_history_length(l_tilde[r], ...) HISTORY tokens of `in` and
 * every other token, in order.  l_tilde: host [num_requests], each request's
 * compressed history length (the first layer's).
 * Errors: as rk_compress_layout.
 */
rk_status rk_prune_layout(const rk_host_layout* in, const int32_t* l_tilde, int32_t n_min,
                          int32_t layer, int32_t num_layers, rk_layout_out* out);

/*
 * y[i] = sum over input rows j in [ranges[2i], ranges[2i+1]) of x[j], for
 * i < n_out, each row `width` elements of `dtype` (fp32 accumulation; RK_BF16
 * rounds once, to nearest even).  ranges: device int32 [n_out][2] (from a
 * layout function); ranges are clamped to [0, n_in), so a bad range reads
 * no memory outside x.  Rows are `x_stride` / `y_stride` elements apart.
 * y must not overlap x.  HBM-bound: reads the input rows once, writes the
 * output rows once.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_HIP.
 */
rk_status rk_gather_sum(const int32_t* ranges, int32_t n_out, int32_t n_in, const void* x,
                        int64_t x_stride, void* y, int64_t y_stride, int32_t width,
                        rk_dtype dtype, void* stream);

/* ---- SORT query pruning (section 3.2.2) -------------------------------
 * The page prunes the user side (history and profile; candidates are never
 * pruned) layer by layer with three strategies, linear, exponential and
 * pooling, whose formulas did not survive on the page.  Readings taken
 * (the plainest the text supports; none can be checked against a printed
 * formula):
 *   linear      : LazFormer eq. 22 (rk_pruned_history_length), the same
 *                 even-step shrink;
 *   exponential : N^l = min(l_tilde, max(n_min, Round(l_tilde * decay^(l -
 *                 1)))), Round taking halves away from zero, decay in
 *                 (0, 1] the per-layer factor;
 *   pooling     : pruning with either schedule in which the pruned history
 *                 tokens of a request are averaged into one token, placed
 *                 where they were (before the kept history) and dated as
 *                 their newest member, so their global content survives.
 * Only HISTORY tokens are pruned, oldest first (as in rk_prune_layout);
 * PROFILE, REALTIME and CANDIDATE tokens stay. */
typedef enum rk_prune_schedule {
  RK_PRUNE_LINEAR = 0,  /* LazFormer eq. 22 over num_layers */
  RK_PRUNE_EXP = 1      /* decay^(layer - 1) */
} rk_prune_schedule;

typedef struct rk_prune_params {
  uint32_t struct_size;
  int32_t schedule;    /* rk_prune_schedule */
  int32_t n_min;       /* floor of the kept history length, >= 0 */
  int32_t layer;       /* 1-based */
  int32_t num_layers;  /* RK_PRUNE_LINEAR: >= layer */
  int32_t pool;        /* nonzero: the pruned tokens become one mean-pooled token */
  double decay;        /* RK_PRUNE_EXP: in (0, 1] */
} rk_prune_params;

/* History positions kept at p->layer by p->schedule (pooling aside).
 * Errors: RK_ERR_INVALID_ARG. */
rk_status rk_pruned_history_length_ex(int32_t l_tilde, const rk_prune_params* p,
                                      int32_t* n_out);

/*
 * Input layout of layer p->layer: per request r, the last
 * rk_pruned_history_length_ex(l_tilde[r], p) HISTORY tokens of `in` and every
 * other token, in order; with p->pool, one more HISTORY token where the
 * pruned ones were, whose range covers them all (move the rows with
 * rk_gather_mean: a kept token's range is one row, so the mean is the row).
 * Errors: as rk_compress_layout.
 */
rk_status rk_prune_layout_ex(const rk_host_layout* in, const int32_t* l_tilde,
                             const rk_prune_params* p, rk_layout_out* out);

/* As rk_gather_sum, with each output row divided by its range length (an
 * empty range gives zeros).  Errors: as rk_gather_sum. */
rk_status rk_gather_mean(const int32_t* ranges, int32_t n_out, int32_t n_in, const void* x,
                         int64_t x_stride, void* y, int64_t y_stride, int32_t width,
                         rk_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RK_H */
