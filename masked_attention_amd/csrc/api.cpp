// C ABI of librk (declared in include/rk.h): argument validation, plan
// workspace layout, the host side of the launch schedule, and dispatch to
// the HIP kernels.  Validation is synchronous and precedes every enqueue.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "rk_internal.h"

using rk::Group;
using rk::kNumXcd;
using rk::PlanTotals;
using rk::ReqMeta;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kInt32Max = 2147483647;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Pinned, fine-grained (coherent) host blocks that carry a plan's host
// tables to the GPU: the first planner kernel reads them in place and
// copies them into the workspace, so a plan needs no copy-engine transfer
// and no wait of the compute queue on one.  The first word of a block is 1
// while the block is free and 0 while a plan's first kernel may still read
// it; the planner's second kernel, which starts after the first has ended,
// sets it back to 1.  Blocks stay allocated until the process ends.  With
// kMaxBlocks leased at once (plans issued far ahead of the GPU) a plan goes
// up by an asynchronous copy instead.
class StagingPool {
 public:
  static constexpr size_t kHeader = 256;
  static constexpr size_t kMinBlock = size_t(64) << 10;
  static constexpr size_t kMaxBlocks = 64;
  struct Lease {
    unsigned char* data = nullptr;
    unsigned* done = nullptr;
  };
  Lease acquire(size_t bytes) {
    std::lock_guard<std::mutex> lock(mu_);
    for (const Block& b : blocks_) {
      if (b.cap - kHeader >= bytes && __atomic_load_n(b.done, __ATOMIC_ACQUIRE) == 1u) {
        __atomic_store_n(b.done, 0u, __ATOMIC_RELAXED);
        return {b.base + kHeader, b.done};
      }
    }
    if (blocks_.size() >= kMaxBlocks) return {};
    size_t cap = kMinBlock;
    while (cap - kHeader < bytes) cap *= 2;
    void* mem = nullptr;
    if (hipHostMalloc(&mem, cap, hipHostMallocCoherent | hipHostMallocPortable) != hipSuccess) {
      (void)hipGetLastError();
      return {};
    }
    const Block b{static_cast<unsigned char*>(mem), cap, static_cast<unsigned*>(mem)};
    *b.done = 0u;
    blocks_.push_back(b);
    return {b.base + kHeader, b.done};
  }

 private:
  struct Block {
    unsigned char* base;
    size_t cap;
    unsigned* done;
  };
  std::mutex mu_;
  std::vector<Block> blocks_;
};

StagingPool& staging_pool() {
  static StagingPool* pool = new StagingPool;  // never destroyed: blocks live to process end
  return *pool;
}

// Sizes and host-side tables derived from req_offsets_host.
struct Layout {
  int32_t R = 0, T = 0, H = 0;
  int64_t NQ = 0, NT = 0, G = 0, max_queue = 0, slots = 0;
  int64_t NK = 0, kslots = 0;
  std::vector<ReqMeta> req;
  std::vector<int32_t> qt_req;
  std::vector<Group> groups;        // sorted by (queue, base)
  std::vector<int32_t> queue_start; // kNumXcd + 1
  std::vector<int32_t> kt_req;      // key-major counterparts
  std::vector<Group> kgroups;
  std::vector<int32_t> kqueue_start;
  std::vector<int32_t> group_of;    // see PlanDev::group_of
  std::vector<int32_t> ilv;         // see PlanDev::ilv
  std::vector<int32_t> kilv;        // the same for kgroups
  size_t ilv_cap = 0;               // int32 entries reserved for ilv (and for kilv)
  size_t off_ilv = 0, off_kilv = 0, off_group_of = 0;
  size_t off_req = 0, off_qt_req = 0, off_groups = 0, off_queue_start = 0, off_totals = 0,
         host_blob = 0, off_row_desc = 0, off_tile_count = 0, off_tile_class = 0, off_qt_nnz = 0,
         off_qt_pairs = 0, off_qt_full = 0, off_qt_flags = 0,
         off_qtile_ptr = 0, off_ktile_idx = 0, off_ktile_word = 0, off_qorder = 0, off_sched = 0,
         off_work = 0, off_irec = 0, off_splits = 0, off_act = 0, off_kt_req = 0, off_kgroups = 0,
         off_kqueue_start = 0, off_kt_nnz = 0, off_kt_ptr = 0, off_qtile_word = 0,
         off_korder = 0, off_ksched = 0, total = 0;
};

// Place (request, head) groups of `count(r)` work items each on the eight
// XCD queues: requests by descending weight, each group on the least-loaded
// queue.  Returns the longest queue; fills `out` sorted by (queue, base) and
// `qstart` (kNumXcd + 1 entries) when asked.
template <typename CountFn>
int64_t place_groups(int32_t R, int32_t H, const int32_t* o, const std::vector<int64_t>& weight,
                     CountFn count, bool fill, std::vector<Group>* out,
                     std::vector<int32_t>* qstart) {
  std::vector<Group> gs;
  std::vector<int> gq;
  int64_t counts[kNumXcd] = {0};
  std::vector<int32_t> order;
  for (int32_t r = 0; r < R; ++r)
    if (o[r + 1] > o[r]) order.push_back(r);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t c) { return weight[a] > weight[c]; });
  int64_t loads[kNumXcd] = {0};
  for (int32_t r : order) {
    const int32_t n = count(r);
    for (int32_t h = 0; h < H; ++h) {
      int q = 0;
      for (int j = 1; j < kNumXcd; ++j)
        if (loads[j] < loads[q]) q = j;
      Group g;
      g.req = r;
      g.head = h;
      g.base = (int32_t)std::min<int64_t>(counts[q], kInt32Max);
      g.count = n;
      loads[q] += weight[r];
      counts[q] += n;
      if (fill) {
        gs.push_back(g);
        gq.push_back(q);
      }
    }
  }
  int64_t mq = 0;
  for (int j = 0; j < kNumXcd; ++j) mq = std::max(mq, counts[j]);
  if (fill) {
    qstart->assign(kNumXcd + 1, 0);
    for (int j = 0; j < kNumXcd; ++j) {
      (*qstart)[j] = (int32_t)out->size();
      for (size_t i = 0; i < gs.size(); ++i)
        if (gq[i] == j) out->push_back(gs[i]);  // bases increase within a queue
    }
    (*qstart)[kNumXcd] = (int32_t)out->size();
  }
  return mq;
}

// Blocks of a schedule: consecutive groups of a queue packed while their
// items total at most kInterleaveItems (a larger group is a block of its
// own); inside a block the groups are sorted by count, largest first, all
// get the block's first slot as base, and the block's slots take every
// group's largest item, then every group's second largest, ...  Fills `ilv`
// as PlanDev::ilv describes (2 G + sum over blocks of K + 2 entries, at
// most 2 G + sum over groups of count + 2).
void build_blocks(std::vector<Group>* groups, const std::vector<int32_t>& qstart, int64_t G,
                  std::vector<int32_t>* ilv) {
  ilv->clear();
  if (G == 0) return;
  std::vector<Group>& gs = *groups;
  ilv->assign(2 * (size_t)G, 0);
  for (int q = 0; q < kNumXcd; ++q) {
    int32_t b = qstart[q];
    const int32_t e = qstart[q + 1];
    while (b < e) {
      int32_t f = b + 1;
      int64_t items = gs[b].count;
      while (f < e && items + gs[f].count <= rk::kInterleaveItems) items += gs[f++].count;
      const int32_t base = gs[b].base;  // the block's first slot
      std::stable_sort(gs.begin() + b, gs.begin() + f,
                       [](const Group& x, const Group& y) { return x.count > y.count; });
      const int32_t K = gs[b].count;
      const int32_t table = (int32_t)ilv->size();
      ilv->push_back(K);
      for (int32_t k = 0; k <= K; ++k) {
        int64_t c = 0;
        for (int32_t g = b; g < f; ++g) c += std::min(gs[g].count, k);
        ilv->push_back((int32_t)c);
      }
      for (int32_t g = b; g < f; ++g) {
        gs[g].base = base;
        (*ilv)[g] = b;
        (*ilv)[G + g] = table;
      }
      b = f;
    }
  }
}

rk_status check_batch(const rk_batch* b) {
  if (!b || b->struct_size < sizeof(rk_batch)) return RK_ERR_INVALID_ARG;
  if (b->num_requests < 0 || b->total_tokens < 0) return RK_ERR_INVALID_ARG;
  if (!b->req_offsets_host) return RK_ERR_INVALID_ARG;
  const int32_t* o = b->req_offsets_host;
  if (o[0] != 0) return RK_ERR_INVALID_ARG;
  for (int32_t r = 0; r < b->num_requests; ++r)
    if (o[r + 1] < o[r]) return RK_ERR_INVALID_ARG;
  if (o[b->num_requests] != b->total_tokens) return RK_ERR_INVALID_ARG;
  if (b->num_requests > 0 && (!b->req_offsets_dev || !b->anchors_dev)) return RK_ERR_INVALID_ARG;
  if (b->total_tokens > 0 && (!b->seg_kind_dev || !b->timestamps_dev)) return RK_ERR_INVALID_ARG;
  return RK_OK;
}

rk_status make_layout(const rk_batch* b, int32_t H, bool with_tables, Layout* L) {
  rk_status st = check_batch(b);
  if (st != RK_OK) return st;
  if (H < 1) return RK_ERR_INVALID_ARG;
  L->R = b->num_requests;
  L->T = b->total_tokens;
  L->H = H;
  const int32_t* o = b->req_offsets_host;
  int64_t nq = 0, nt = 0, nk = 0;
  if (with_tables) L->req.resize(L->R);
  std::vector<int64_t> weight(L->R);
  for (int32_t r = 0; r < L->R; ++r) {
    const int32_t len = o[r + 1] - o[r];
    // 64-bit sums: a request may hold up to INT32_MAX tokens
    const int32_t nqt = (int32_t)(((int64_t)len + rk::kTileQ - 1) / rk::kTileQ);
    const int32_t nkt = (int32_t)(((int64_t)len + rk::kTileK - 1) / rk::kTileK);
    if (with_tables) {
      ReqMeta& m = L->req[r];
      m.tok_off = o[r];
      m.len = len;
      m.qt_off = (int32_t)std::min<int64_t>(nq, kInt32Max);
      m.nqt = nqt;
      m.nkt = nkt;
      m.kt_off = (int32_t)std::min<int64_t>(nk, kInt32Max);  // key blocks of 128 keys
      m.tile_off = nt;
      for (int k = 0; k < 4; ++k) m.seg[k] = len;
    }
    weight[r] = (int64_t)nqt * nkt;
    nq += nqt;
    nk += nqt;  // the backward's key blocks have the q-tile's 128 positions
    nt += (int64_t)nqt * nkt;
  }
  if (nt >= kInt32Max || nq * (int64_t)H >= kInt32Max || nk * (int64_t)H >= kInt32Max)
    return RK_ERR_UNSUPPORTED;
  L->NQ = nq;
  L->NT = nt;
  L->NK = nk;

  // Launch schedules: (request, head) groups, heaviest first, each placed on
  // the least-loaded of the eight XCD queues (dense tile count as weight);
  // one for query-tile items, one for key-tile items (backward).
  auto nqt_of = [&](int32_t r) {
    return (int32_t)(((int64_t)o[r + 1] - o[r] + rk::kTileQ - 1) / rk::kTileQ);
  };
  auto nkb_of = nqt_of;  // 128-key blocks of the backward's key-major items
  L->max_queue = place_groups(L->R, H, o, weight, nqt_of, with_tables, &L->groups,
                              &L->queue_start);
  L->slots = L->max_queue * kNumXcd;
  int64_t ng = 0;
  for (int32_t r = 0; r < L->R; ++r) ng += (o[r + 1] > o[r]) ? H : 0;
  L->G = ng;
  L->ilv_cap = 2 * (size_t)L->G;
  for (int32_t r = 0; r < L->R; ++r)
    if (o[r + 1] > o[r]) L->ilv_cap += (size_t)H * (2 + (size_t)nqt_of(r));
  if (with_tables) {
    build_blocks(&L->groups, L->queue_start, L->G, &L->ilv);
    L->group_of.assign((size_t)L->R * H, -1);
    for (int64_t ga = 0; ga < L->G; ++ga)
      L->group_of[(size_t)L->groups[ga].req * H + L->groups[ga].head] = (int32_t)ga;
  }
  const int64_t kmax = place_groups(L->R, H, o, weight, nkb_of, with_tables, &L->kgroups,
                                    &L->kqueue_start);
  L->kslots = kmax * kNumXcd;
  if (with_tables) build_blocks(&L->kgroups, L->kqueue_start, L->G, &L->kilv);
  if (L->slots >= kInt32Max || L->kslots >= kInt32Max) return RK_ERR_UNSUPPORTED;
  if (with_tables) {
    L->qt_req.resize(nq);
    L->kt_req.resize(nk);
    for (int32_t r = 0; r < L->R; ++r) {
      for (int32_t i = 0; i < L->req[r].nqt; ++i) L->qt_req[L->req[r].qt_off + i] = r;
      for (int32_t i = 0; i < L->req[r].nqt; ++i) L->kt_req[L->req[r].kt_off + i] = r;
    }
  }

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L->off_req = take(sizeof(ReqMeta) * (size_t)L->R);
  L->off_qt_req = take(sizeof(int32_t) * (size_t)nq);
  L->off_groups = take(sizeof(Group) * (size_t)L->G);
  L->off_queue_start = take(sizeof(int32_t) * (kNumXcd + 1));
  L->off_totals = take(sizeof(PlanTotals));
  L->off_kt_req = take(sizeof(int32_t) * (size_t)nk);
  L->off_kgroups = take(sizeof(Group) * (size_t)L->G);
  L->off_kqueue_start = take(sizeof(int32_t) * (kNumXcd + 1));
  L->off_ilv = take(sizeof(int32_t) * L->ilv_cap);
  L->off_kilv = take(sizeof(int32_t) * L->ilv_cap);
  L->off_group_of = take(sizeof(int32_t) * (size_t)L->R * (size_t)H);
  L->host_blob = off;
  L->off_row_desc = take(sizeof(int2) * (size_t)L->T);
  L->off_tile_count = take(sizeof(int32_t) * (size_t)nt);
  L->off_tile_class = take((size_t)nt);
  L->off_qt_nnz = take(sizeof(int32_t) * (size_t)nq);
  L->off_qt_pairs = take(sizeof(int64_t) * (size_t)nq);
  L->off_qt_full = take(sizeof(int32_t) * (size_t)nq);
  L->off_qt_flags = take(sizeof(uint32_t) * (size_t)nq);
  L->off_qtile_ptr = take(sizeof(int32_t) * (size_t)(nq + 1));
  L->off_ktile_idx = take(sizeof(int32_t) * (size_t)nt);
  L->off_ktile_word = take(sizeof(int32_t) * (size_t)nt);
  L->off_qorder = take(sizeof(int32_t) * (size_t)nq);
  L->off_sched = take(sizeof(int32_t) * (size_t)L->slots);
  L->off_work = take(sizeof(rk::WorkEntry) * (size_t)(L->slots + rk::kSplitTarget));
  L->off_irec = take(sizeof(rk::ItemRec) * (size_t)(L->slots + rk::kSplitTarget));
  L->off_splits = take(sizeof(rk::SplitEntry) * (size_t)rk::kSplitTarget);
  L->off_act = take(sizeof(int32_t) * (size_t)(rk::kSplitTarget / 2));
  L->off_kt_nnz = take(sizeof(int32_t) * (size_t)nk);
  L->off_kt_ptr = take(sizeof(int32_t) * (size_t)(nk + 1));
  L->off_qtile_word = take(sizeof(int32_t) * (size_t)nt);
  L->off_korder = take(sizeof(int32_t) * (size_t)nk);
  L->off_ksched = take(sizeof(int32_t) * (size_t)L->kslots);
  L->total = off;
  return RK_OK;
}

rk_status check_rope(const rk_rope_params* r) {
  if (!r || r->struct_size < sizeof(rk_rope_params)) return RK_ERR_INVALID_ARG;
  if (r->kinds & ~0xfu) return RK_ERR_INVALID_ARG;  // four segment kinds
  if (!(std::isfinite(r->phi_min) && std::isfinite(r->dt_max) && std::isfinite(r->base)))
    return RK_ERR_INVALID_ARG;
  if (!(r->phi_min > 0 && r->dt_max > 0 && r->base > 0)) return RK_ERR_INVALID_ARG;
  return RK_OK;
}

rk_status check_norm(const rk_qk_norm_params* n, int d) {
  if (!n || n->struct_size < sizeof(rk_qk_norm_params)) return RK_ERR_INVALID_ARG;
  if (!(std::isfinite(n->eps) && n->eps > 0.f)) return RK_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return RK_ERR_UNSUPPORTED;
  return RK_OK;
}

rk::RopeTab make_tab(const rk_rope_params* r, int d) {
  rk::RopeTab t;
  std::memset(&t, 0, sizeof(t));
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d / 2 && i < rk::kMaxHalfD; ++i)
    t.w_rev[i] = r->phi_min / r->dt_max * std::pow(r->base, 2.0 * i / d) / two_pi;
  return t;
}

size_t elem_size(rk_dtype dt) { return dt == RK_F32 ? 4 : 2; }

// An enum argument as the int the (C or ctypes) caller stored.  Values
// outside the enumerators are not valid C++ enum values, so validation reads
// the representation instead of the enum.
template <typename E>
int enum_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool valid_dtype(const rk_dtype& dt) {
  const int v = enum_int(dt);
  return v == RK_F32 || v == RK_BF16;
}

}  // namespace

extern "C" {

const char* rk_status_string(rk_status s) {
  // C and ctypes callers may pass any int; read its representation rather
  // than the enum value (values outside the enumerators are not valid C++
  // enum values).
  switch (enum_int(s)) {
    case RK_OK: return "ok";
    case RK_ERR_INVALID_ARG: return "invalid argument";
    case RK_ERR_SEGMENT_ORDER: return "segment kinds out of order or out of range";
    case RK_ERR_UNSORTED_TIME: return "timestamps not in order where required";
    case RK_ERR_UNSUPPORTED: return "unsupported configuration";
    case RK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RK_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t rk_abi_version(void) { return RK_ABI_VERSION; }

rk_status rk_plan_workspace_size(const rk_batch* b, int32_t num_heads, size_t* bytes) {
  if (!bytes) return RK_ERR_INVALID_ARG;
  Layout L;
  rk_status st = make_layout(b, num_heads, false, &L);
  if (st != RK_OK) return st;
  *bytes = L.total;
  return RK_OK;
}

rk_status rk_mask_plan(const rk_batch* b, const rk_mask_params* m, int32_t num_heads,
                       void* workspace, size_t workspace_bytes, rk_plan** plan_out, void* stream) {
  if (!plan_out) return RK_ERR_INVALID_ARG;
  *plan_out = nullptr;
  if (!m || m->struct_size < sizeof(rk_mask_params)) return RK_ERR_INVALID_ARG;
  if (m->delay < 0 || m->window < 0 || m->global_tail < 0 ||
      (m->flags & ~(RK_STATIC_BIDIRECTIONAL | RK_QUERY_CANDIDATES_ONLY | RK_PLAN_BACKWARD)))
    return RK_ERR_INVALID_ARG;
  if ((m->flags & RK_QUERY_CANDIDATES_ONLY) && (m->flags & RK_PLAN_BACKWARD))
    return RK_ERR_INVALID_ARG;
  Layout L;
  rk_status st = make_layout(b, num_heads, true, &L);
  if (st != RK_OK) return st;
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0) return RK_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return RK_ERR_WORKSPACE_TOO_SMALL;

  rk_plan* p = new (std::nothrow) rk_plan();
  if (!p) return RK_ERR_INVALID_ARG;
  p->R = L.R;
  p->T = L.T;
  p->H = L.H;
  p->NQ = L.NQ;
  p->NT = L.NT;
  p->G = L.G;
  p->slots = L.slots;
  p->max_queue = L.max_queue;
  p->NK = L.NK;
  p->kslots = L.kslots;
  p->grid = (m->flags & RK_QUERY_CANDIDATES_ONLY) && L.slots > 0 ? L.slots + rk::kSplitTarget
                                                                 : L.slots;
  p->delay = m->delay;
  p->window = m->window;
  p->global_tail = m->global_tail;
  p->flags = m->flags;
  p->req_offsets_dev = b->req_offsets_dev;
  p->seg_kind_dev = b->seg_kind_dev;
  p->timestamps_dev = b->timestamps_dev;
  p->anchors_dev = b->anchors_dev;
  p->workspace = workspace;
  p->workspace_bytes = workspace_bytes;
  p->off_req = L.off_req;
  p->off_qt_req = L.off_qt_req;
  p->off_groups = L.off_groups;
  p->off_queue_start = L.off_queue_start;
  p->off_row_desc = L.off_row_desc;
  p->off_tile_count = L.off_tile_count;
  p->off_tile_class = L.off_tile_class;
  p->off_qt_nnz = L.off_qt_nnz;
  p->off_qt_pairs = L.off_qt_pairs;
  p->off_qt_full = L.off_qt_full;
  p->off_qt_flags = L.off_qt_flags;
  p->off_qtile_ptr = L.off_qtile_ptr;
  p->off_ktile_idx = L.off_ktile_idx;
  p->off_ktile_word = L.off_ktile_word;
  p->off_qorder = L.off_qorder;
  p->off_sched = L.off_sched;
  p->off_work = L.off_work;
  p->off_irec = L.off_irec;
  p->off_splits = L.off_splits;
  p->off_act = L.off_act;
  p->off_totals = L.off_totals;
  p->off_kt_req = L.off_kt_req;
  p->off_kgroups = L.off_kgroups;
  p->off_kqueue_start = L.off_kqueue_start;
  p->off_kt_nnz = L.off_kt_nnz;
  p->off_kt_ptr = L.off_kt_ptr;
  p->off_qtile_word = L.off_qtile_word;
  p->off_korder = L.off_korder;
  p->off_ksched = L.off_ksched;
  p->off_ilv = L.off_ilv;
  p->off_kilv = L.off_kilv;
  p->off_group_of = L.off_group_of;
  p->host_blob_bytes = L.host_blob;
  p->total_bytes = L.total;

  unsigned char* ws = (unsigned char*)workspace;
  rk::PlanDev& D = p->dev;
  D.req = (ReqMeta*)(ws + L.off_req);
  D.qt_req = (int32_t*)(ws + L.off_qt_req);
  D.groups = (Group*)(ws + L.off_groups);
  D.queue_start = (int32_t*)(ws + L.off_queue_start);
  D.totals = (PlanTotals*)(ws + L.off_totals);
  D.row_desc = (int2*)(ws + L.off_row_desc);
  D.tile_count = (int32_t*)(ws + L.off_tile_count);
  D.tile_class = (uint8_t*)(ws + L.off_tile_class);
  D.qt_nnz = (int32_t*)(ws + L.off_qt_nnz);
  D.qt_pairs = (int64_t*)(ws + L.off_qt_pairs);
  D.qt_full = (int32_t*)(ws + L.off_qt_full);
  D.qt_flags = (uint32_t*)(ws + L.off_qt_flags);
  D.qtile_ptr = (int32_t*)(ws + L.off_qtile_ptr);
  D.ktile_idx = (int32_t*)(ws + L.off_ktile_idx);
  D.ktile_word = (int32_t*)(ws + L.off_ktile_word);
  D.qorder = (int32_t*)(ws + L.off_qorder);
  D.sched = (int32_t*)(ws + L.off_sched);
  D.work = (rk::WorkEntry*)(ws + L.off_work);
  D.irec = (rk::ItemRec*)(ws + L.off_irec);
  D.splits = (rk::SplitEntry*)(ws + L.off_splits);
  D.act_slots = (int32_t*)(ws + L.off_act);
  D.kt_req = (int32_t*)(ws + L.off_kt_req);
  D.kgroups = (Group*)(ws + L.off_kgroups);
  D.kqueue_start = (int32_t*)(ws + L.off_kqueue_start);
  D.kt_nnz = (int32_t*)(ws + L.off_kt_nnz);
  D.kt_ptr = (int32_t*)(ws + L.off_kt_ptr);
  D.qtile_word = (int32_t*)(ws + L.off_qtile_word);
  D.korder = (int32_t*)(ws + L.off_korder);
  D.ksched = (int32_t*)(ws + L.off_ksched);
  D.ilv = (int32_t*)(ws + L.off_ilv);
  D.kilv = (int32_t*)(ws + L.off_kilv);
  D.group_of = (int32_t*)(ws + L.off_group_of);

  // The host tables: read in place by the first planner kernel from a
  // pinned block when one is free (and the batch has tokens, so that the
  // kernel runs), else copied up from the plan's own host buffer.  Under
  // stream capture the copy is used: a replayed graph reads its source
  // again, which the plan's own buffer still holds and a reused block
  // would not.
  hipStream_t s = (hipStream_t)stream;
  bool may_stage = false;
  if (L.NQ > 0) {
    hipStreamCaptureStatus capture = hipStreamCaptureStatusActive;
    if (hipStreamIsCapturing(s, &capture) == hipSuccess)
      may_stage = capture == hipStreamCaptureStatusNone;
    else
      (void)hipGetLastError();  // the query's own error; take the copy
  }
  const StagingPool::Lease lease =
      may_stage ? staging_pool().acquire(L.host_blob) : StagingPool::Lease{};
  unsigned char* blob = lease.data;
  if (!blob) {
    p->host_blob = (unsigned char*)std::malloc(L.host_blob ? L.host_blob : 1);
    if (!p->host_blob) {
      delete p;
      return RK_ERR_INVALID_ARG;
    }
    blob = p->host_blob;
  }
  std::memset(blob, 0, L.host_blob);  // totals start at zero
  if (L.R) std::memcpy(blob + L.off_req, L.req.data(), sizeof(ReqMeta) * L.R);
  if (L.NQ) std::memcpy(blob + L.off_qt_req, L.qt_req.data(), sizeof(int32_t) * L.NQ);
  if (L.G) std::memcpy(blob + L.off_groups, L.groups.data(), sizeof(Group) * L.G);
  std::memcpy(blob + L.off_queue_start, L.queue_start.data(), sizeof(int32_t) * (kNumXcd + 1));
  if (L.NK) std::memcpy(blob + L.off_kt_req, L.kt_req.data(), sizeof(int32_t) * L.NK);
  if (L.G) std::memcpy(blob + L.off_kgroups, L.kgroups.data(), sizeof(Group) * L.G);
  std::memcpy(blob + L.off_kqueue_start, L.kqueue_start.data(), sizeof(int32_t) * (kNumXcd + 1));
  if (!L.ilv.empty()) std::memcpy(blob + L.off_ilv, L.ilv.data(), sizeof(int32_t) * L.ilv.size());
  if (!L.kilv.empty())
    std::memcpy(blob + L.off_kilv, L.kilv.data(), sizeof(int32_t) * L.kilv.size());
  if (!L.group_of.empty())
    std::memcpy(blob + L.off_group_of, L.group_of.data(), sizeof(int32_t) * L.group_of.size());

  hipError_t e;
  if (lease.data) {
    // a failed launch leaves the block marked in use: a kernel that did
    // start may still read it
    e = rk::launch_plan(p, lease.data, lease.done, s);
  } else {
    e = hipMemcpyAsync(workspace, p->host_blob, L.host_blob, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = rk::launch_plan(p, nullptr, nullptr, s);
  }
  if (e != hipSuccess) {
    std::free(p->host_blob);
    delete p;
    return RK_ERR_HIP;
  }
  *plan_out = p;
  return RK_OK;
}

rk_status rk_plan_get_info(const rk_plan* p, rk_plan_info* out) {
  if (!p || !out || out->struct_size < sizeof(rk_plan_info)) return RK_ERR_INVALID_ARG;
  out->num_requests = p->R;
  out->total_tokens = p->T;
  out->num_heads = p->H;
  out->num_qtiles = p->NQ;
  out->num_tiles = p->NT;
  out->num_sched_slots = p->slots;
  out->workspace = p->workspace;
  out->off_tile_class = p->off_tile_class;
  out->off_tile_count = p->off_tile_count;
  out->off_qtile_ptr = p->off_qtile_ptr;
  out->off_ktile_idx = p->off_ktile_idx;
  out->off_row_desc = p->off_row_desc;
  out->off_sched = p->off_sched;
  const bool wl = p->grid > p->slots;
  out->num_work_slots = wl ? p->grid : 0;
  out->off_work = wl ? p->off_work : 0;
  out->off_splits = wl ? p->off_splits : 0;
  const bool bw = (p->flags & RK_PLAN_BACKWARD) != 0;
  out->num_kblocks = p->NK;
  out->num_ksched_slots = bw ? p->kslots : 0;
  out->off_kt_ptr = bw ? p->off_kt_ptr : 0;
  out->off_qtile_word = bw ? p->off_qtile_word : 0;
  out->off_ksched = bw ? p->off_ksched : 0;
  return RK_OK;
}

rk_status rk_plan_stats(const rk_plan* p, rk_plan_totals* out, void* stream) {
  if (!p || !out || out->struct_size < sizeof(rk_plan_totals)) return RK_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return RK_ERR_HIP;
  PlanTotals t;
  if (hipMemcpy(&t, p->dev.totals, sizeof(t), hipMemcpyDeviceToHost) != hipSuccess) return RK_ERR_HIP;
  out->device_errors = t.errors;
  out->visible_pairs = (int64_t)t.visible_pairs;
  out->full_tiles = (int64_t)t.full_tiles;
  out->partial_tiles = (int64_t)t.partial_tiles;
  out->empty_tiles = (int64_t)t.empty_tiles;
  out->work_entries = t.n_work;
  out->split_items = t.n_splits;
  if (t.errors & rk::kErrSegment) return RK_ERR_SEGMENT_ORDER;
  if (t.errors & (rk::kErrTime | rk::kErrStaticSplit)) return RK_ERR_UNSORTED_TIME;
  return RK_OK;
}

void rk_plan_destroy(rk_plan* p) {
  if (!p) return;
  std::free(p->host_blob);
  delete p;
}

rk_status rk_time_rope(const rk_batch* b, const rk_rope_params* r, const void* x_in, void* x_out,
                       rk_dtype dtype, int32_t num_heads, int32_t d_head, int64_t in_stride_tok,
                       int64_t in_stride_head, int64_t out_stride_tok, int64_t out_stride_head,
                       void* stream) {
  rk_status st = check_batch(b);
  if (st != RK_OK) return st;
  if ((st = check_rope(r)) != RK_OK) return st;
  if (!valid_dtype(dtype)) return RK_ERR_INVALID_ARG;
  if (num_heads < 1 || d_head < 2) return RK_ERR_INVALID_ARG;
  if ((d_head & 1) || d_head > 2 * rk::kMaxHalfD) return RK_ERR_UNSUPPORTED;
  if (in_stride_tok < 0 || in_stride_head < 0 || out_stride_tok < 0 || out_stride_head < 0)
    return RK_ERR_INVALID_ARG;
  if (b->total_tokens > 0 && (!x_in || !x_out)) return RK_ERR_INVALID_ARG;
  if (x_in == x_out && (in_stride_tok != out_stride_tok || in_stride_head != out_stride_head))
    return RK_ERR_INVALID_ARG;
  const rk::RopeTab tab = make_tab(r, d_head);
  hipError_t e = rk::launch_rope(b->num_requests, b->total_tokens, b->req_offsets_dev,
                                 b->timestamps_dev, b->anchors_dev, b->seg_kind_dev, r->kinds, tab,
                                 x_in, x_out, dtype, num_heads, d_head, in_stride_tok,
                                 in_stride_head, out_stride_tok, out_stride_head,
                                 (hipStream_t)stream);
  return e == hipSuccess ? RK_OK : RK_ERR_HIP;
}

rk_status rk_qk_norm_rope(const rk_batch* b, const rk_rope_params* r, float eps,
                          const float* gamma, const void* x_in, void* x_out, rk_dtype dtype,
                          int32_t num_heads, int32_t d_head, int64_t in_stride_tok,
                          int64_t in_stride_head, int64_t out_stride_tok,
                          int64_t out_stride_head, void* stream) {
  rk_status st = check_batch(b);
  if (st != RK_OK) return st;
  if (r && (st = check_rope(r)) != RK_OK) return st;
  if (!valid_dtype(dtype)) return RK_ERR_INVALID_ARG;
  if (num_heads < 1 || !(std::isfinite(eps) && eps > 0.f)) return RK_ERR_INVALID_ARG;
  if (d_head != 32 && d_head != 64 && d_head != 128) return RK_ERR_UNSUPPORTED;
  if (in_stride_tok < 0 || in_stride_head < 0 || out_stride_tok < 0 || out_stride_head < 0)
    return RK_ERR_INVALID_ARG;
  if (b->total_tokens > 0 && (!x_in || !x_out)) return RK_ERR_INVALID_ARG;
  if (x_in == x_out && (in_stride_tok != out_stride_tok || in_stride_head != out_stride_head))
    return RK_ERR_INVALID_ARG;
  rk::RopeTab tab;
  std::memset(&tab, 0, sizeof(tab));  // no rope: rotation by zero
  if (r) tab = make_tab(r, d_head);
  hipError_t e = rk::launch_rope(b->num_requests, b->total_tokens, b->req_offsets_dev,
                                 b->timestamps_dev, b->anchors_dev, b->seg_kind_dev,
                                 r ? r->kinds : 0u, tab, x_in, x_out, dtype, num_heads, d_head,
                                 in_stride_tok, in_stride_head, out_stride_tok, out_stride_head,
                                 (hipStream_t)stream, true, eps, gamma);
  return e == hipSuccess ? RK_OK : RK_ERR_HIP;
}

}  // extern "C"

namespace {

rk_status check_attn(const rk_plan* p, const rk_attn_args* a) {
  if (!p || !a || a->struct_size < sizeof(rk_attn_args)) return RK_ERR_INVALID_ARG;
  if (!valid_dtype(a->dtype)) return RK_ERR_INVALID_ARG;
  if (a->num_heads != p->H) return RK_ERR_INVALID_ARG;
  // any multiple of 8 up to 128 (the kernels pad to an instance width);
  // QK Norm keeps to 32, 64 and 128 (check_norm)
  if (a->d_head < 8 || a->d_head > 128 || (a->d_head % 8) != 0) return RK_ERR_UNSUPPORTED;
  if (a->flags & ~(RK_ATTN_REFERENCE_KERNEL | RK_ATTN_K_PREROTATED)) return RK_ERR_INVALID_ARG;
  if ((a->flags & RK_ATTN_K_PREROTATED) && !a->rope && !a->qk_norm) return RK_ERR_INVALID_ARG;
  if (a->qk_norm) {
    rk_status s = check_norm(a->qk_norm, a->d_head);
    if (s != RK_OK) return s;
  }
  if (p->T > 0 && (!a->q || !a->k || !a->v || !a->o)) return RK_ERR_INVALID_ARG;
  const int64_t st[8] = {a->q_stride_tok, a->q_stride_head, a->k_stride_tok, a->k_stride_head,
                         a->v_stride_tok, a->v_stride_head, a->o_stride_tok, a->o_stride_head};
  for (int64_t x : st)
    if (x < 0) return RK_ERR_INVALID_ARG;
  if (!(std::isfinite(a->scale) && a->scale >= 0.f)) return RK_ERR_INVALID_ARG;
  if (a->rope) {
    rk_status s = check_rope(a->rope);
    if (s != RK_OK) return s;
    if (a->rope->kinds != 0) return RK_ERR_INVALID_ARG;  // the attention rotates every row
  }
  return RK_OK;
}

bool mfma_eligible(const rk_attn_args* a) {
  return a->dtype == RK_BF16 && !(a->flags & RK_ATTN_REFERENCE_KERNEL);
}

// Instance width of the forward kernel that runs: d_head rounded up to 64
// or 128 (MFMA) or to 32, 64 or 128 (plain kernel).
int kernel_dp(const rk_attn_args* a) {
  const int d = a->d_head;
  if (mfma_eligible(a)) return d <= 64 ? 64 : 128;
  return d <= 32 ? 32 : d <= 64 ? 64 : 128;
}

bool mfma_aligned(const rk_attn_args* a, bool k_in_workspace) {
  auto al = [](const void* ptr) { return ((uintptr_t)ptr % 16) == 0; };
  // strides multiples of 8 elements (16-byte rows) and small enough that a
  // key tile's per-thread byte offsets fit in 32 bits
  auto st = [](int64_t x) { return (x % 8) == 0 && x <= (int64_t(1) << 24); };
  bool ok = al(a->q) && al(a->v) && al(a->o) && st(a->q_stride_tok) && st(a->q_stride_head) &&
            st(a->v_stride_tok) && st(a->v_stride_head) && st(a->o_stride_tok) &&
            st(a->o_stride_head);
  if (!k_in_workspace) ok = ok && al(a->k) && st(a->k_stride_tok) && st(a->k_stride_head);
  if (a->qk_norm && a->qk_norm->gamma_q) ok = ok && al(a->qk_norm->gamma_q);  // 16-byte loads
  return ok;
}

// Attention workspace: [rotated K, when the call rotates K][partial results
// of split items, for plans with a work list].
size_t attn_k_bytes(const rk_plan* p, const rk_attn_args* a) {
  if ((!a->rope && !a->qk_norm) || (a->flags & RK_ATTN_K_PREROTATED)) return 0;
  return align_up((size_t)p->T * (size_t)a->num_heads * (size_t)a->d_head * elem_size(a->dtype));
}

size_t attn_part_bytes(const rk_plan* p, const rk_attn_args* a) {
  if (p->grid <= p->slots) return 0;
  return align_up((size_t)rk::kMaxParts * rk::kTileQ * (size_t)(kernel_dp(a) + 2) * sizeof(float));
}

size_t attn_ws_bytes(const rk_plan* p, const rk_attn_args* a) {
  return attn_k_bytes(p, a) + attn_part_bytes(p, a);
}

}  // namespace

extern "C" {

rk_status rk_attn_workspace_size(const rk_plan* p, const rk_attn_args* a, size_t* bytes) {
  if (!bytes) return RK_ERR_INVALID_ARG;
  rk_status st = check_attn(p, a);
  if (st != RK_OK) return st;
  *bytes = attn_ws_bytes(p, a);
  return RK_OK;
}

rk_status rk_masked_attn_fwd(const rk_plan* p, const rk_attn_args* a, void* stream) {
  rk_status st = check_attn(p, a);
  if (st != RK_OK) return st;
  const size_t need = attn_ws_bytes(p, a);
  if (need > 0) {
    if (!a->workspace || ((uintptr_t)a->workspace % kAlign) != 0) return RK_ERR_INVALID_ARG;
    if (a->workspace_bytes < need) return RK_ERR_WORKSPACE_TOO_SMALL;
  }
  const bool use_mfma = mfma_eligible(a);
  // K is prepared (normalised and / or rotated) by a pass into the
  // workspace unless the caller did it
  const bool k_rotate = (a->rope || a->qk_norm) && !(a->flags & RK_ATTN_K_PREROTATED);
  if (use_mfma && !mfma_aligned(a, k_rotate)) return RK_ERR_UNSUPPORTED;

  rk::AttnLaunch L;
  std::memset(&L, 0, sizeof(L));
  L.q = a->q;
  L.k = a->k;
  L.v = a->v;
  L.o = a->o;
  L.lse = a->lse;
  L.q_st = a->q_stride_tok;
  L.q_sh = a->q_stride_head;
  L.k_st = a->k_stride_tok;
  L.k_sh = a->k_stride_head;
  L.v_st = a->v_stride_tok;
  L.v_sh = a->v_stride_head;
  L.o_st = a->o_stride_tok;
  L.o_sh = a->o_stride_head;
  L.scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->d_head);
  L.H = a->num_heads;
  L.d = a->d_head;
  L.dp = kernel_dp(a);
  L.T = p->T;
  L.ts = p->timestamps_dev;
  L.plan_err = &p->dev.totals->errors;
  L.anchors = p->anchors_dev;
  hipStream_t s = (hipStream_t)stream;
  if (a->rope || a->qk_norm) {
    // Q is transformed while staged: rotated (a zero table rotates by
    // nothing) after the optional norm
    if (a->rope) L.tab = make_tab(a->rope, a->d_head);
    L.rope_q = true;
  }
  if (a->qk_norm) {
    L.norm_q = true;
    L.eps = a->qk_norm->eps;
    L.gamma_q = a->qk_norm->gamma_q;
  }
  if (attn_part_bytes(p, a))
    L.part = (float*)((unsigned char*)a->workspace + attn_k_bytes(p, a));
  if (k_rotate) {
    // K is rotated once into the workspace ([T, H, d] dense); Q is rotated
    // by the attention kernel while it is staged.
    const int64_t hd = (int64_t)a->num_heads * a->d_head;
    hipError_t e = rk::launch_rope(p->R, p->T, p->req_offsets_dev, p->timestamps_dev,
                                   p->anchors_dev, p->seg_kind_dev, 0u, L.tab, a->k, a->workspace,
                                   a->dtype,
                                   a->num_heads, a->d_head, a->k_stride_tok, a->k_stride_head, hd,
                                   a->d_head, s, a->qk_norm != nullptr,
                                   a->qk_norm ? a->qk_norm->eps : 0.f,
                                   a->qk_norm ? a->qk_norm->gamma_k : nullptr);
    if (e != hipSuccess) return RK_ERR_HIP;
    L.k = a->workspace;
    L.k_st = hd;
    L.k_sh = a->d_head;
  }
  hipError_t e = use_mfma ? rk::launch_attn_mfma_bf16(p, L, s)
                          : rk::launch_attn_reference(p, L, a->dtype, s);
  if (e == hipSuccess && L.part) {
    // units of the kernels' reference max m: the MFMA kernel keeps it in log2
    // units of the scaled score when it folds scale * log2(e) into a rotated
    // Q, in raw dot-product units otherwise; the plain kernel in natural units
    // of the scaled score
    const float log2e = 1.4426950408889634f, ln2 = 0.6931471805599453f;
    float to_log2, to_nat;
    if (use_mfma && L.rope_q) { to_log2 = 1.f; to_nat = ln2; }
    else if (use_mfma) { to_log2 = L.scale * log2e; to_nat = L.scale; }
    else { to_log2 = log2e; to_nat = 1.f; }
    e = rk::launch_attn_combine(p, L, a->dtype, to_log2, to_nat, s);
  }
  return e == hipSuccess ? RK_OK : RK_ERR_HIP;
}

rk_status rk_masked_attn_fwd_noalloc(const rk_plan* p, const rk_attn_args* a, void* stream) {
  rk_status st = check_attn(p, a);
  if (st != RK_OK) return st;
  // the library's scratch array takes the place of the workspace
  if (a->workspace || a->workspace_bytes) return RK_ERR_INVALID_ARG;
  const size_t need = attn_ws_bytes(p, a);
  if (need > (size_t)RK_STATIC_SCRATCH_BYTES) return RK_ERR_WORKSPACE_TOO_SMALL;
  rk_attn_args b;
  std::memcpy(&b, a, sizeof(b));
  if (need > 0) {
    void* ws = nullptr;
    if (rk::static_scratch(&ws) != hipSuccess) return RK_ERR_HIP;
    b.workspace = ws;
    b.workspace_bytes = (size_t)RK_STATIC_SCRATCH_BYTES;
  }
  return rk_masked_attn_fwd(p, &b, stream);
}

rk_status rk_pointwise_attn_fwd(const rk_plan* p, const rk_pointwise_args* a, void* stream) {
  if (!p || !a || a->struct_size < sizeof(rk_pointwise_args)) return RK_ERR_INVALID_ARG;
  if (!valid_dtype(a->dtype) || a->num_heads != p->H) return RK_ERR_INVALID_ARG;
  if (a->d_head != 32 && a->d_head != 64 && a->d_head != 128) return RK_ERR_UNSUPPORTED;
  if (a->flags & ~RK_ATTN_REFERENCE_KERNEL) return RK_ERR_INVALID_ARG;
  if (p->T > 0 && (!a->q || !a->k || !a->v || !a->o)) return RK_ERR_INVALID_ARG;
  const int64_t st[8] = {a->q_stride_tok, a->q_stride_head, a->k_stride_tok, a->k_stride_head,
                         a->v_stride_tok, a->v_stride_head, a->o_stride_tok, a->o_stride_head};
  for (int64_t x : st)
    if (x < 0) return RK_ERR_INVALID_ARG;
  if (!std::isfinite(a->scale)) return RK_ERR_INVALID_ARG;
  if (a->pos_bias && (a->num_pos_buckets < 1 || a->num_pos_buckets > 4096)) return RK_ERR_INVALID_ARG;
  if (a->time_bias && (a->num_time_buckets < 1 || a->num_time_buckets > 64))
    return RK_ERR_INVALID_ARG;
  const bool use_mfma =
      enum_int(a->dtype) == RK_BF16 && a->d_head == 64 && !(a->flags & RK_ATTN_REFERENCE_KERNEL);
  if (use_mfma) {
    auto al = [](const void* ptr) { return ((uintptr_t)ptr % 16) == 0; };
    for (int64_t x : st)
      if ((x % 8) != 0 || x > (int64_t(1) << 24)) return RK_ERR_UNSUPPORTED;
    if (!al(a->q) || !al(a->k) || !al(a->v) || !al(a->o)) return RK_ERR_UNSUPPORTED;
  }
  rk::PwLaunch L;
  std::memset(&L, 0, sizeof(L));
  L.q = a->q;
  L.k = a->k;
  L.v = a->v;
  L.o = a->o;
  L.q_st = a->q_stride_tok;
  L.q_sh = a->q_stride_head;
  L.k_st = a->k_stride_tok;
  L.k_sh = a->k_stride_head;
  L.v_st = a->v_stride_tok;
  L.v_sh = a->v_stride_head;
  L.o_st = a->o_stride_tok;
  L.o_sh = a->o_stride_head;
  L.scale = a->scale != 0.f ? a->scale : 1.f;
  L.H = a->num_heads;
  L.d = a->d_head;
  L.T = p->T;
  L.pos_bias = a->pos_bias;
  L.time_bias = a->time_bias;
  L.np = a->pos_bias ? a->num_pos_buckets : 1;
  L.nt = a->time_bias ? a->num_time_buckets : 1;
  L.ts = p->timestamps_dev;
  L.plan_err = &p->dev.totals->errors;
  hipError_t e = use_mfma ? rk::launch_pointwise_mfma_bf16_d64(p, L, (hipStream_t)stream)
                          : rk::launch_pointwise_reference(p, L, a->dtype, (hipStream_t)stream);
  return e == hipSuccess ? RK_OK : RK_ERR_HIP;
}

}  // extern "C"

namespace {

rk_status check_bwd(const rk_plan* p, const rk_attn_bwd_args* a) {
  if (!p || !a || a->struct_size < sizeof(rk_attn_bwd_args)) return RK_ERR_INVALID_ARG;
  if (!(p->flags & RK_PLAN_BACKWARD)) return RK_ERR_INVALID_ARG;
  if (!valid_dtype(a->dtype)) return RK_ERR_INVALID_ARG;
  if (a->num_heads != p->H) return RK_ERR_INVALID_ARG;
  if (a->d_head != 32 && a->d_head != 64 && a->d_head != 128) return RK_ERR_UNSUPPORTED;
  if (a->flags & ~(RK_ATTN_REFERENCE_KERNEL | RK_ATTN_K_PREROTATED)) return RK_ERR_INVALID_ARG;
  if ((a->flags & RK_ATTN_K_PREROTATED) && !a->rope) return RK_ERR_INVALID_ARG;
  if (a->qk_norm) {
    rk_status s = check_norm(a->qk_norm, a->d_head);
    if (s != RK_OK) return s;
    // the gradient of K is taken back through the norm, so K comes as is
    if (a->flags & RK_ATTN_K_PREROTATED) return RK_ERR_INVALID_ARG;
    if ((a->qk_norm->gamma_q && !a->dgamma_q) || (a->qk_norm->gamma_k && !a->dgamma_k))
      return RK_ERR_INVALID_ARG;
  }
  if (p->T > 0 && (!a->q || !a->k || !a->v || !a->o || !a->d_o || !a->lse || !a->dq || !a->dk ||
                   !a->dv))
    return RK_ERR_INVALID_ARG;
  const int64_t st[16] = {a->q_stride_tok,  a->q_stride_head,  a->k_stride_tok,  a->k_stride_head,
                          a->v_stride_tok,  a->v_stride_head,  a->o_stride_tok,  a->o_stride_head,
                          a->do_stride_tok, a->do_stride_head, a->dq_stride_tok, a->dq_stride_head,
                          a->dk_stride_tok, a->dk_stride_head, a->dv_stride_tok, a->dv_stride_head};
  for (int64_t x : st)
    if (x < 0) return RK_ERR_INVALID_ARG;
  if (!(std::isfinite(a->scale) && a->scale >= 0.f)) return RK_ERR_INVALID_ARG;
  if (a->rope) {
    rk_status s = check_rope(a->rope);
    if (s != RK_OK) return s;
    if (a->rope->kinds != 0) return RK_ERR_INVALID_ARG;
  }
  return RK_OK;
}

bool bwd_mfma_eligible(const rk_attn_bwd_args* a) {
  return a->dtype == RK_BF16 && a->d_head == 64 && !(a->flags & RK_ATTN_REFERENCE_KERNEL);
}

// Row-aligned views for the MFMA kernels: 16-byte base pointers, strides
// that are multiples of 8 elements and small enough for 32-bit byte offsets.
bool bwd_mfma_aligned(const rk_attn_bwd_args* a, bool q_in_ws, bool k_in_ws) {
  auto al = [](const void* ptr) { return ((uintptr_t)ptr % 16) == 0; };
  auto st = [](int64_t x) { return (x % 8) == 0 && x <= (int64_t(1) << 24); };
  bool ok = al(a->v) && al(a->o) && al(a->d_o) && al(a->dq) && al(a->dk) && al(a->dv);
  const int64_t s[12] = {a->v_stride_tok,  a->v_stride_head,  a->o_stride_tok,  a->o_stride_head,
                         a->do_stride_tok, a->do_stride_head, a->dq_stride_tok, a->dq_stride_head,
                         a->dk_stride_tok, a->dk_stride_head, a->dv_stride_tok, a->dv_stride_head};
  for (int64_t x : s) ok = ok && st(x);
  if (!q_in_ws) ok = ok && al(a->q) && st(a->q_stride_tok) && st(a->q_stride_head);
  if (!k_in_ws) ok = ok && al(a->k) && st(a->k_stride_tok) && st(a->k_stride_head);
  return ok;
}

// Backward workspace: [rowsum(dO*O) H*T fp32][lse2 H*T fp32][rotated
// (normalised) Q][rotated (normalised) K][gain gradient partials of Q][of K].
struct BwdWs {
  size_t dsum = 0, lse2 = 0, q = 0, k = 0, pq = 0, pk = 0, total = 0;
};

BwdWs bwd_ws(const rk_plan* p, const rk_attn_bwd_args* a) {
  BwdWs w;
  const size_t ht = (size_t)p->T * (size_t)a->num_heads;
  const size_t rows = ht * (size_t)a->d_head * elem_size(a->dtype);
  size_t off = 0;
  w.dsum = off;
  off = align_up(off + ht * sizeof(float));
  w.lse2 = off;
  off = align_up(off + ht * sizeof(float));
  if (a->rope || a->qk_norm) {
    w.q = off;
    off = align_up(off + rows);
    if (!(a->flags & RK_ATTN_K_PREROTATED)) {
      w.k = off;
      off = align_up(off + rows);
    }
  }
  if (a->qk_norm) {
    const size_t part = (size_t)rk::norm_bwd_blocks((int64_t)ht) * (size_t)a->d_head * sizeof(float);
    if (a->qk_norm->gamma_q) {
      w.pq = off;
      off = align_up(off + part);
    }
    if (a->qk_norm->gamma_k) {
      w.pk = off;
      off = align_up(off + part);
    }
  }
  w.total = off;
  return w;
}

// The pass that takes dQ or dK back through QK Norm (in place).
hipError_t norm_bwd(const rk_plan* p, const rk_attn_bwd_args* a, const void* x, int64_t x_st,
                    int64_t x_sh, void* g, int64_t g_st, int64_t g_sh, const float* gamma,
                    float* partial, float* dgamma, hipStream_t s) {
  rk::NormBwdArgs n;
  n.x = x;
  n.x_st = x_st;
  n.x_sh = x_sh;
  n.g = g;
  n.g_st = g_st;
  n.g_sh = g_sh;
  n.gamma = gamma;
  n.eps = a->qk_norm->eps;
  n.rows = (int64_t)p->T * a->num_heads;
  n.H = a->num_heads;
  n.partial = gamma ? partial : nullptr;
  n.dgamma = gamma ? dgamma : nullptr;
  return rk::launch_norm_bwd(n, a->dtype, a->d_head, s);
}

}  // namespace

extern "C" {

rk_status rk_attn_bwd_workspace_size(const rk_plan* p, const rk_attn_bwd_args* a, size_t* bytes) {
  if (!bytes) return RK_ERR_INVALID_ARG;
  rk_status st = check_bwd(p, a);
  if (st != RK_OK) return st;
  *bytes = bwd_ws(p, a).total;
  return RK_OK;
}

rk_status rk_masked_attn_bwd(const rk_plan* p, const rk_attn_bwd_args* a, void* stream) {
  rk_status st = check_bwd(p, a);
  if (st != RK_OK) return st;
  const BwdWs w = bwd_ws(p, a);
  hipStream_t s = (hipStream_t)stream;
  if (p->T == 0) {
    // nothing to write but the gain gradients, which are zero
    if (a->qk_norm) {
      hipError_t e = norm_bwd(p, a, nullptr, 0, 0, nullptr, 0, 0, a->qk_norm->gamma_q, nullptr,
                              a->dgamma_q, s);
      if (e == hipSuccess)
        e = norm_bwd(p, a, nullptr, 0, 0, nullptr, 0, 0, a->qk_norm->gamma_k, nullptr,
                     a->dgamma_k, s);
      if (e != hipSuccess) return RK_ERR_HIP;
    }
    return RK_OK;
  }
  if (!a->workspace || ((uintptr_t)a->workspace % kAlign) != 0) return RK_ERR_INVALID_ARG;
  if (a->workspace_bytes < w.total) return RK_ERR_WORKSPACE_TOO_SMALL;
  const bool rope = a->rope != nullptr;
  const bool norm = a->qk_norm != nullptr;
  // Q and K are rotated (and normalised) into the workspace; K unless the
  // caller gave it rotated
  const bool prep = rope || norm;
  const bool k_prep = prep && !(a->flags & RK_ATTN_K_PREROTATED);
  const bool use_mfma = bwd_mfma_eligible(a);
  if (use_mfma && !bwd_mfma_aligned(a, prep, k_prep)) return RK_ERR_UNSUPPORTED;

  unsigned char* ws = (unsigned char*)a->workspace;
  rk::BwdLaunch L;
  std::memset(&L, 0, sizeof(L));
  L.q = a->q;
  L.k = a->k;
  L.v = a->v;
  L.o = a->o;
  L.dout = a->d_o;
  L.lse = a->lse;
  L.dq = a->dq;
  L.dk = a->dk;
  L.dv = a->dv;
  L.q_st = a->q_stride_tok;
  L.q_sh = a->q_stride_head;
  L.k_st = a->k_stride_tok;
  L.k_sh = a->k_stride_head;
  L.v_st = a->v_stride_tok;
  L.v_sh = a->v_stride_head;
  L.o_st = a->o_stride_tok;
  L.o_sh = a->o_stride_head;
  L.do_st = a->do_stride_tok;
  L.do_sh = a->do_stride_head;
  L.dq_st = a->dq_stride_tok;
  L.dq_sh = a->dq_stride_head;
  L.dk_st = a->dk_stride_tok;
  L.dk_sh = a->dk_stride_head;
  L.dv_st = a->dv_stride_tok;
  L.dv_sh = a->dv_stride_head;
  L.scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->d_head);
  L.H = a->num_heads;
  L.d = a->d_head;
  L.T = p->T;
  L.dsum = (float*)(ws + w.dsum);
  L.lse2 = (float*)(ws + w.lse2);
  L.ts = p->timestamps_dev;
  L.plan_err = &p->dev.totals->errors;
  L.anchors = p->anchors_dev;
  const int64_t hd = (int64_t)a->num_heads * a->d_head;
  const float eps = norm ? a->qk_norm->eps : 0.f;
  if (prep) {
    // Q (and K unless given rotated) are normalised (QK Norm) and rotated
    // once into the workspace ([T, H, d] dense; a zero table rotates by
    // nothing); the kernels take dQ (dK) back through the rotation.
    if (rope) L.tab = make_tab(a->rope, a->d_head);
    hipError_t e = rk::launch_rope(p->R, p->T, p->req_offsets_dev, p->timestamps_dev,
                                   p->anchors_dev, p->seg_kind_dev, 0u, L.tab, a->q, ws + w.q,
                                   a->dtype, a->num_heads, a->d_head, a->q_stride_tok,
                                   a->q_stride_head, hd, a->d_head, s, norm, eps,
                                   norm ? a->qk_norm->gamma_q : nullptr);
    if (e != hipSuccess) return RK_ERR_HIP;
    L.q = ws + w.q;
    L.q_st = hd;
    L.q_sh = a->d_head;
    L.unrot_q = rope;
    if (k_prep) {
      e = rk::launch_rope(p->R, p->T, p->req_offsets_dev, p->timestamps_dev, p->anchors_dev,
                          p->seg_kind_dev, 0u, L.tab, a->k, ws + w.k, a->dtype, a->num_heads,
                          a->d_head, a->k_stride_tok, a->k_stride_head, hd, a->d_head, s, norm,
                          eps, norm ? a->qk_norm->gamma_k : nullptr);
      if (e != hipSuccess) return RK_ERR_HIP;
      L.k = ws + w.k;
      L.k_st = hd;
      L.k_sh = a->d_head;
      L.unrot_k = rope;
    }
  }
  hipError_t e = use_mfma ? rk::launch_attn_bwd_mfma_bf16_d64(p, L, s)
                          : rk::launch_attn_bwd_reference(p, L, a->dtype, s);
  if (e == hipSuccess && norm) {
    // dQ and dK hold the gradients of the normalised rows: take them back
    // through the norm in place, with the gains' gradients
    e = norm_bwd(p, a, a->q, a->q_stride_tok, a->q_stride_head, a->dq, a->dq_stride_tok,
                 a->dq_stride_head, a->qk_norm->gamma_q, (float*)(ws + w.pq), a->dgamma_q, s);
    if (e == hipSuccess)
      e = norm_bwd(p, a, a->k, a->k_stride_tok, a->k_stride_head, a->dk, a->dk_stride_tok,
                   a->dk_stride_head, a->qk_norm->gamma_k, (float*)(ws + w.pk), a->dgamma_k, s);
  }
  return e == hipSuccess ? RK_OK : RK_ERR_HIP;
}

}  // extern "C"
