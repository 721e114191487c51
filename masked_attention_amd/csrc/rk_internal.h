// Internal declarations shared by the host ABI (api.cpp) and the HIP
// kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rk.h"

namespace rk {

constexpr int kTileQ = RK_TILE_Q;
constexpr int kTileK = RK_TILE_K;
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dispatched round-robin
// Work items one XCD runs at once in the forward (32 CUs x 3 workgroups;
// the backward's kernels run 2 per CU and take the same blocks).  Consecutive (request, head) groups of a queue are packed
// into blocks of at most this many items (a larger group is a block of its
// own); blocks run one after another and the groups of a block are
// interleaved by rank, so about as many groups are in flight as when they
// run one after another, without a saw-tooth of item sizes.
constexpr int kInterleaveItems = 96;
constexpr int kMaxHalfD = 64;     // d_head <= 128

// Per-request metadata in the plan workspace.  tok_off .. tile_off are
// filled on the host; seg[] starts as len on the host and the device
// records the first position of each segment kind.
struct ReqMeta {
  int32_t tok_off;   // first global token
  int32_t len;       // L_r
  int32_t qt_off;    // first global q-tile
  int32_t nqt;       // ceil(L / 128)
  int32_t nkt;       // ceil(L / 64)
  int32_t kt_off;    // first global 128-key block (backward key-major tables)
  int64_t tile_off;  // first tile in tile_class / tile_count
  int32_t seg[4];    // request-local start of PROFILE, HISTORY, REALTIME, CANDIDATE
};
static_assert(sizeof(ReqMeta) == 48, "ReqMeta layout");

// (request, head) group of the launch schedule, placed in one XCD queue.
struct Group {
  int32_t req;
  int32_t head;
  int32_t base;   // first slot index inside its queue
  int32_t count;  // number of q-tiles (= work items)
};

// Device words of plan totals: errors are OR-ed in by the segment kernel
// (starts at zero from the host upload); the counts are written by the
// scan kernel from per-q-tile partial sums.
struct PlanTotals {
  unsigned long long visible_pairs;
  unsigned long long full_tiles;
  unsigned long long partial_tiles;
  unsigned long long empty_tiles;
  unsigned int errors;  // kErrSegment | kErrTime | kErrStaticSplit
  int n_work;           // work-list entries (candidates-only plans)
  int n_splits;         // items split into partial results
  int n_act;            // active schedule slots (candidates-only plans)
  unsigned int info;    // kInfoHistoryUnsorted (not an error)
  unsigned int pad[3];
};

// Work list of a candidates-only plan: launch slot b of the attention runs
// CSR entries [kbeg, kend) of work item `item` (q-tile * H + head); part >= 0
// means the item's key range is split and this slot writes partial result
// `part`, merged by the combine kernel.
struct WorkEntry {
  int32_t item, kbeg, kend, part;
};
// What a forward kernel needs to start one launch slot's work, written by
// the planner next to the slot's schedule or work entry so that a
// workgroup's first memory access (one 48-byte scalar load) hands it the
// request geometry, the CSR range and its first two entries: the Q loads
// and the first key tiles' copies then go out one memory latency after
// launch instead of four (schedule -> q-tile's request -> request -> CSR).
struct ItemRec {
  int32_t tok_off;  // first global token of the request
  int32_t len;      // request length
  int32_t row0;     // first row of the q-tile, request-local
  int32_t head;     // -1: the slot has no work
  int32_t e0;       // first CSR entry of the slot's range
  int32_t n;        // CSR entries in the range
  int32_t req;      // request
  int32_t part;     // partial-result index of a split chunk, -1 for a whole item
  int32_t w0, w1;   // CSR words e0 and e0 + 1 (w1 = w0 when n < 2; both 0 when n == 0)
  int32_t pad[2];
};
static_assert(sizeof(ItemRec) == 48, "ItemRec layout");

// An item split into parts [part0, part0 + nparts).
struct SplitEntry {
  int32_t item, part0, nparts, pad;
};

// Splitting: aim at about kSplitTarget launch slots of work (one round of
// the attention kernel at three workgroups per CU on 256 CUs), chunks of at
// least kSplitMinChunk key tiles, fewer than kMaxParts partial results.
constexpr int kSplitTarget = RK_SPLIT_SLOTS;
constexpr int kSplitMinChunk = 8;
constexpr int kMaxParts = 2 * kSplitTarget;

constexpr unsigned kErrSegment = 1u;      // segment kinds out of order or out of range
constexpr unsigned kErrTime = 2u;         // timestamps out of order where the mask needs order
constexpr unsigned kErrStaticSplit = 4u;  // a static row's visible keys would form two runs
                                          // (profile times interleaved with history times)
// Some HISTORY segment is not in time order (allowed when no delay rule
// searches it): kernels must not take a history tile's time range from its
// end keys.
constexpr unsigned kInfoHistoryUnsorted = 1u;

// Device pointers of a plan (all inside the caller's workspace).
struct PlanDev {
  ReqMeta* req;            // [R]
  int32_t* qt_req;         // [NQ] request of each global q-tile
  Group* groups;           // [G] sorted by (queue, base)
  int32_t* queue_start;    // [kNumXcd + 1] first group of each queue
  int32_t* group_of;       // [R * H] index in groups of (request, head), -1 for empty requests
  int2* row_desc;          // [T]
  int32_t* tile_count;     // [NT]
  uint8_t* tile_class;     // [NT]
  int32_t* qt_nnz;         // [NQ] non-empty k-tiles of each q-tile
  int64_t* qt_pairs;       // [NQ] visible pairs of each q-tile
  int32_t* qt_full;        // [NQ] FULL k-tiles of each q-tile
  uint32_t* qt_flags;      // [NQ] device-check errors | info << 16 of each q-tile's rows
  int32_t* qtile_ptr;      // [NQ + 1]
  int32_t* ktile_idx;      // [NT]
  int32_t* ktile_word;     // [NT] CSR entry for the kernels: kt | (PARTIAL << 31)
  int32_t* qorder;         // [NQ]
  int32_t* sched;          // [slots]
  int32_t* ilv;            // blocks of the schedule: [G] first group of each group's block,
                           // [G] offset in ilv of the block's table: K (largest count),
                           // then C(k) = sum over its groups of min(count, k), k = 0..K
  WorkEntry* work;         // [slots + kSplitTarget] (candidates-only plans)
  ItemRec* irec;           // [slots + kSplitTarget] record of every forward launch slot
  SplitEntry* splits;      // [kSplitTarget]
  int32_t* act_slots;      // [kSplitTarget / 2] active schedule slots, arrival order
  PlanTotals* totals;
  // key-major tables (plans built with RK_PLAN_BACKWARD) over key blocks of
  // 128 keys (k-tiles 2 kb and 2 kb + 1 of the request)
  int32_t* kt_req;         // [NK] request of each global key block
  Group* kgroups;          // [G] (request, head) groups of key-block work items
  int32_t* kqueue_start;   // [kNumXcd + 1]
  int32_t* kt_nnz;         // [NK] non-empty q-tiles of each key block
  int32_t* kt_ptr;         // [NK + 1] CSR row pointers
  int32_t* qtile_word;     // [NT] CSR entry: request-local qt | (PARTIAL << 31)
  int32_t* korder;         // [NK] key blocks of each request by descending kt_nnz
  int32_t* ksched;         // [kslots] work item = key block * H + head, or -1
  int32_t* kilv;           // blocks of the key-major schedule, laid out as ilv
};

}  // namespace rk

struct rk_plan {
  int32_t R, T, H;
  int64_t NQ, NT, G, slots, max_queue;
  int64_t NK, kslots;       // global 128-key blocks; key-major launch slots
  int64_t grid;             // attention launch size: slots, or slots + kSplitTarget with a work list
  int64_t delay;
  int32_t window;
  int32_t global_tail;
  uint32_t flags;
  // batch device arrays (caller-owned)
  const int32_t* req_offsets_dev;
  const uint8_t* seg_kind_dev;
  const int64_t* timestamps_dev;
  const int64_t* anchors_dev;
  void* workspace;
  size_t workspace_bytes;
  size_t off_req, off_qt_req, off_groups, off_queue_start, off_row_desc, off_tile_count,
      off_tile_class, off_qt_nnz, off_qt_pairs, off_qt_full, off_qtile_ptr, off_ktile_idx, off_ktile_word, off_qorder,
      off_sched, off_work, off_splits, off_act, off_totals, host_blob_bytes, total_bytes,
      off_kt_req, off_kgroups, off_kqueue_start, off_kt_nnz, off_kt_ptr, off_qtile_word,
      off_korder, off_ksched, off_ilv, off_kilv, off_group_of, off_irec, off_qt_flags;
  rk::PlanDev dev;
  // host copy of the first host_blob_bytes of the workspace when it went
  // up by an asynchronous copy (kept alive for it), else null
  unsigned char* host_blob;
};

namespace rk {

// 1 when the plan's device checks passed, NaN otherwise.  Every kernel that
// runs over a plan multiplies what it stores by this, so a plan built from a
// batch that broke the segment or time order gives NaN rows, not silently
// wrong ones.
__device__ __forceinline__ float plan_poison(const unsigned* plan_err) {
  return *plan_err ? __builtin_nanf("") : 1.f;
}

// RoPE frequency table in revolutions per timestamp unit:
// w_rev[i] = phi_min / dt_max * base^(2i/d) / (2 pi).
struct RopeTab {
  double w_rev[kMaxHalfD];
};

// ---- launchers (defined in the .hip files); return hipSuccess or an error
// staged: the plan's host tables in a pinned host block the first kernel
// reads (null: already in the workspace); stage_done: set to 1 by the GPU
// once that block has been read (null with staged null).
hipError_t launch_plan(const rk_plan* p, const unsigned char* staged, unsigned* stage_done,
                       hipStream_t s);
// kinds: rotate only tokens whose segment kind k has bit k set (0 = all).
// norm: RMSNorm of every [d] row (x / sqrt(mean(x^2) + eps) * gamma, gamma
// NULL = 1) before the rotation; needs d in {32, 64, 128}.  A zero table
// rotates by nothing (cos 0 = 1, sin 0 = 0 exactly).
hipError_t launch_rope(int32_t R, int32_t T, const int32_t* req_offsets, const int64_t* ts,
                       const int64_t* anchors, const uint8_t* kind, unsigned kinds,
                       const RopeTab& tab, const void* x_in, void* x_out, rk_dtype dt, int H, int d,
                       int64_t in_st, int64_t in_sh, int64_t out_st, int64_t out_sh,
                       hipStream_t s, bool norm = false, float eps = 0.f,
                       const float* gamma = nullptr);

struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  float scale;
  int H, d, T;
  int dp;                   // the kernels' tile width: d rounded up to an instance (32, 64
                            // or 128); columns d .. dp - 1 are zero in registers and LDS,
                            // never read from or written to the tensors
  bool rope_q;              // transform Q while staging: rotate by `tab` (all zero
                            // for no rotation), fold the scale in (K is ready)
  bool norm_q;              // RMSNorm Q before the rotation (QK Norm)
  float eps;
  const float* gamma_q;     // [d] or null
  float* part;              // partial results of split items, or null
  const unsigned* plan_err; // the plan's device error word (plan_poison)
  const int64_t* ts;
  const int64_t* anchors;
  RopeTab tab;
};

// Backward launch description.  q and k are the rotated Q' and K' when
// rope is on (rotated by a pass into the workspace, or K given rotated);
// unrot_q / unrot_k ask the kernels to take dQ / dK back through the
// rotation (R^T) in their epilogue.  dsum and lse2 ([H][T] fp32, in the
// workspace) are written by the dQ kernel and read by the dK/dV kernel:
// dsum = rowsum(dO * O), lse2 = the forward log-sum-exp in log2 units
// (+inf for rows that see nothing).
struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, do_st, do_sh, dq_st, dq_sh, dk_st,
      dk_sh, dv_st, dv_sh;
  float scale;
  int H, d, T;
  bool unrot_q, unrot_k;
  float* dsum;
  float* lse2;
  const unsigned* plan_err; // the plan's device error word (plan_poison)
  const int64_t* ts;
  const int64_t* anchors;
  RopeTab tab;
};

hipError_t launch_attn_bwd_reference(const rk_plan* p, const BwdLaunch& a, rk_dtype dt,
                                     hipStream_t s);
hipError_t launch_attn_bwd_mfma_bf16_d64(const rk_plan* p, const BwdLaunch& a, hipStream_t s);

// y[i] = sum of input rows [ranges[2i], ranges[2i+1]) clamped to [0, n_in),
// or their mean (mean; 0 for an empty range).
hipError_t launch_gather_sum(const int32_t* ranges, int n_out, int n_in, const void* x,
                             int64_t xs, void* y, int64_t ys, int width, rk_dtype dt,
                             hipStream_t s, bool mean);

// HSTU pointwise attention launch description.
struct PwLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  float scale;
  int H, d, T;
  const float* pos_bias;  // [np] or null
  const float* time_bias; // [nt] or null
  int np, nt;
  const unsigned* plan_err; // the plan's device error word (plan_poison)
  const int64_t* ts;
};

hipError_t launch_pointwise_reference(const rk_plan* p, const PwLaunch& a, rk_dtype dt,
                                      hipStream_t s);
hipError_t launch_pointwise_mfma_bf16_d64(const rk_plan* p, const PwLaunch& a, hipStream_t s);

hipError_t launch_attn_reference(const rk_plan* p, const AttnLaunch& a, rk_dtype dt,
                                 hipStream_t s);
// bf16 MFMA forward; d_head 64 or 128
hipError_t launch_attn_mfma_bf16(const rk_plan* p, const AttnLaunch& a, hipStream_t s);
// Device address of the library's scratch array on the current GPU
// (RK_STATIC_SCRATCH_BYTES, 256-byte aligned), looked up on the first call
// per device (scratch.hip).
hipError_t static_scratch(void** out);
// Merge the partial results of split items into O / LSE.  to_log2 / to_nat
// convert the kernels' reference max into log2 / natural units.
hipError_t launch_attn_combine(const rk_plan* p, const AttnLaunch& a, rk_dtype dt, float to_log2,
                               float to_nat, hipStream_t s);

// Backward through QK Norm, in place on the gradient rows g (see
// norm_bwd.hip): rows = T * H rows of d elements, row (tok, head) at
// tok * st + head * sh.  partial: norm_bwd_blocks(rows) * d floats, or null
// when there is no gain (then dgamma is null too).
struct NormBwdArgs {
  const void* x;  // the rows before the norm
  int64_t x_st, x_sh;
  void* g;        // dLoss/dy in, dLoss/dx out
  int64_t g_st, g_sh;
  const float* gamma;  // [d] or null (gain 1)
  float eps;
  int64_t rows;
  int H;
  float* partial;
  float* dgamma;  // [d] or null
};
constexpr int kRowsPerNormBlock = 512;
inline int64_t norm_bwd_blocks(int64_t rows) {
  return (rows + kRowsPerNormBlock - 1) / kRowsPerNormBlock;
}
hipError_t launch_norm_bwd(const NormBwdArgs& a, rk_dtype dt, int d, hipStream_t s);

}  // namespace rk
