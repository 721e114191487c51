// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer against a library whose host code carries the
// same instrumentation (tests/test_abi_sanitizers.py builds and runs it).
// Every call here returns from argument validation before any HIP call, so
// no GPU is needed; a sanitizer report or a wrong status fails the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "rk.h"

static int failures = 0;

#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

// Device pointers are never dereferenced by the validation paths: any
// non-null value stands in for them.
static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static rk_batch make_batch(const std::vector<int32_t>& offs, int32_t total) {
  rk_batch b;
  std::memset(&b, 0, sizeof(b));
  b.struct_size = sizeof(rk_batch);
  b.num_requests = (int32_t)offs.size() - 1;
  b.total_tokens = total;
  b.req_offsets_host = offs.data();
  b.req_offsets_dev = static_cast<const int32_t*>(fake(0x1000));
  b.seg_kind_dev = static_cast<const uint8_t*>(fake(0x2000));
  b.timestamps_dev = static_cast<const int64_t*>(fake(0x3000));
  b.anchors_dev = static_cast<const int64_t*>(fake(0x4000));
  return b;
}

static void check_status_strings() {
  EXPECT(rk_abi_version() == RK_ABI_VERSION);
  for (int s = 0; s <= 6; ++s) EXPECT(std::strlen(rk_status_string((rk_status)s)) > 0);
  EXPECT(rk_status_string((rk_status)99) != nullptr);
}

static void check_workspace_size() {
  size_t n = 0;
  std::vector<int32_t> offs = {0, 10, 10, 300};
  rk_batch b = make_batch(offs, 300);
  EXPECT(rk_plan_workspace_size(&b, 4, &n) == RK_OK);
  EXPECT(n > 0 && n % 256 == 0);
  // a large batch: 64 requests of 20001 tokens
  std::vector<int32_t> big(65);
  for (int i = 0; i <= 64; ++i) big[i] = 20001 * i;
  rk_batch bb = make_batch(big, big.back());
  EXPECT(rk_plan_workspace_size(&bb, 8, &n) == RK_OK);
  EXPECT(n >= (size_t)64 * 157 * 313 * 10);
  // bad offsets
  std::vector<int32_t> o1 = {1, 10}, o2 = {0, 10, 5}, o3 = {0, 10, 20};
  rk_batch b1 = make_batch(o1, 10), b2 = make_batch(o2, 5), b3 = make_batch(o3, 19);
  EXPECT(rk_plan_workspace_size(&b1, 4, &n) == RK_ERR_INVALID_ARG);
  EXPECT(rk_plan_workspace_size(&b2, 4, &n) == RK_ERR_INVALID_ARG);
  EXPECT(rk_plan_workspace_size(&b3, 4, &n) == RK_ERR_INVALID_ARG);
  EXPECT(rk_plan_workspace_size(&b, 0, &n) == RK_ERR_INVALID_ARG);
  EXPECT(rk_plan_workspace_size(nullptr, 1, &n) == RK_ERR_INVALID_ARG);
  EXPECT(rk_plan_workspace_size(&b, 1, nullptr) == RK_ERR_INVALID_ARG);
  rk_batch b4 = b;
  b4.struct_size = 8;
  EXPECT(rk_plan_workspace_size(&b4, 1, &n) == RK_ERR_INVALID_ARG);
  rk_batch b5 = b;
  b5.seg_kind_dev = nullptr;
  EXPECT(rk_plan_workspace_size(&b5, 1, &n) == RK_ERR_INVALID_ARG);
  rk_batch b6 = b;
  b6.req_offsets_host = nullptr;
  EXPECT(rk_plan_workspace_size(&b6, 1, &n) == RK_ERR_INVALID_ARG);
  rk_batch b7 = make_batch(offs, 300);
  b7.num_requests = -1;
  EXPECT(rk_plan_workspace_size(&b7, 1, &n) == RK_ERR_INVALID_ARG);
}

static void check_mask_plan() {
  std::vector<int32_t> offs = {0, 100, 300};
  rk_batch b = make_batch(offs, 300);
  size_t n = 0;
  EXPECT(rk_plan_workspace_size(&b, 2, &n) == RK_OK);
  rk_mask_params m;
  std::memset(&m, 0, sizeof(m));
  m.struct_size = sizeof(m);
  m.delay = 3600;
  rk_plan* h = nullptr;
  EXPECT(rk_mask_plan(&b, &m, 2, fake(1 << 20), n - 256, &h, nullptr) ==
         RK_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(h == nullptr);
  EXPECT(rk_mask_plan(&b, &m, 2, fake((1 << 20) + 8), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_mask_plan(&b, &m, 2, nullptr, n, &h, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_mask_plan(&b, nullptr, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_mask_plan(&b, &m, 2, fake(1 << 20), n, nullptr, nullptr) == RK_ERR_INVALID_ARG);
  rk_mask_params bad = m;
  bad.delay = -1;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  bad = m;
  bad.window = -3;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  bad = m;
  bad.flags = 8;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  bad.flags = RK_QUERY_CANDIDATES_ONLY | RK_PLAN_BACKWARD;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  bad.flags = RK_QUERY_CANDIDATES_ONLY | 8u;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  bad = m;
  bad.global_tail = -1;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
  bad = m;
  bad.struct_size = 4;
  EXPECT(rk_mask_plan(&b, &bad, 2, fake(1 << 20), n, &h, nullptr) == RK_ERR_INVALID_ARG);
}

static void check_time_rope() {
  std::vector<int32_t> offs = {0, 100};
  rk_batch b = make_batch(offs, 100);
  rk_rope_params r;
  std::memset(&r, 0, sizeof(r));
  r.struct_size = sizeof(r);
  r.phi_min = 1e-4;
  r.dt_max = 31536000.0;
  r.base = 6e5;
  void* x = fake(1 << 20);
  void* y = fake(1 << 21);
  EXPECT(rk_time_rope(&b, &r, x, y, RK_BF16, 2, 63, 128, 64, 128, 64, nullptr) ==
         RK_ERR_UNSUPPORTED);
  EXPECT(rk_time_rope(&b, &r, x, y, RK_BF16, 2, 256, 512, 256, 512, 256, nullptr) ==
         RK_ERR_UNSUPPORTED);
  EXPECT(rk_time_rope(&b, &r, x, y, RK_BF16, 0, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_time_rope(&b, &r, x, y, (rk_dtype)7, 2, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_time_rope(&b, &r, nullptr, y, RK_BF16, 2, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_time_rope(&b, &r, x, y, RK_BF16, 2, 64, -1, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_time_rope(&b, &r, x, x, RK_BF16, 2, 64, 128, 64, 256, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  rk_rope_params bad = r;
  bad.phi_min = 0.0;
  EXPECT(rk_time_rope(&b, &bad, x, y, RK_BF16, 2, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  bad = r;
  bad.kinds = RK_KIND_BIT(4);  // only four segment kinds exist
  EXPECT(rk_time_rope(&b, &bad, x, y, RK_BF16, 2, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  bad = r;
  bad.base = std::nan("");
  EXPECT(rk_time_rope(&b, &bad, x, y, RK_BF16, 2, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_time_rope(nullptr, &r, x, y, RK_BF16, 2, 64, 128, 64, 128, 64, nullptr) ==
         RK_ERR_INVALID_ARG);
}

static void check_attention_without_plan() {
  rk_attn_args a;
  std::memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = RK_BF16;
  a.num_heads = 1;
  a.d_head = 64;
  size_t n = 0;
  EXPECT(rk_masked_attn_fwd(nullptr, &a, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_attn_workspace_size(nullptr, &a, &n) == RK_ERR_INVALID_ARG);
  rk_plan_totals t;
  std::memset(&t, 0, sizeof(t));
  t.struct_size = sizeof(t);
  EXPECT(rk_plan_stats(nullptr, &t, nullptr) == RK_ERR_INVALID_ARG);
  rk_plan_info info;
  std::memset(&info, 0, sizeof(info));
  info.struct_size = sizeof(info);
  EXPECT(rk_plan_get_info(nullptr, &info) == RK_ERR_INVALID_ARG);
  rk_plan_destroy(nullptr);
  rk_attn_bwd_args g;
  std::memset(&g, 0, sizeof(g));
  g.struct_size = sizeof(g);
  g.dtype = RK_BF16;
  g.num_heads = 1;
  g.d_head = 64;
  EXPECT(rk_masked_attn_bwd(nullptr, &g, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_masked_attn_bwd(nullptr, nullptr, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_attn_bwd_workspace_size(nullptr, &g, &n) == RK_ERR_INVALID_ARG);
}

static void check_layouts() {
  // two requests: PROFILE x1, HISTORY x5, CANDIDATE x2 | HISTORY x3
  std::vector<int32_t> offs = {0, 8, 11};
  std::vector<uint8_t> kind = {0, 1, 1, 1, 1, 1, 3, 3, 1, 1, 1};
  std::vector<int64_t> ts = {5, 10, 20, 30, 40, 50, 60, 60, 1, 2, 3};
  rk_host_layout in;
  std::memset(&in, 0, sizeof(in));
  in.struct_size = sizeof(in);
  in.num_requests = 2;
  in.total_tokens = 11;
  in.req_offsets = offs.data();
  in.seg_kind = kind.data();
  in.timestamps = ts.data();
  std::vector<int32_t> o2(3);
  rk_layout_out out;
  std::memset(&out, 0, sizeof(out));
  out.struct_size = sizeof(out);
  out.req_offsets = o2.data();
  // size query, then the call with exactly that capacity
  EXPECT(rk_compress_layout(&in, 2, 2, &out) == RK_ERR_WORKSPACE_TOO_SMALL);
  const int32_t n = out.total_tokens;
  EXPECT(n == 10);  // request 0: 1 + 2 groups + 2 kept + 2; request 1: 1 group + 2 kept
  std::vector<uint8_t> k2(n);
  std::vector<int64_t> t2(n);
  std::vector<int32_t> r2(2 * n);
  out.capacity = n;
  out.seg_kind = k2.data();
  out.timestamps = t2.data();
  out.ranges = r2.data();
  EXPECT(rk_compress_layout(&in, 2, 2, &out) == RK_OK);
  EXPECT(o2[1] == 7 && o2[2] == 10);
  EXPECT(r2[2] == 1 && r2[3] == 2 && r2[4] == 2 && r2[5] == 4);  // short group is the oldest
  EXPECT(t2[2] == 30);                                           // newest member's time
  std::vector<int32_t> lt = {5, 3};
  EXPECT(rk_prune_layout(&in, lt.data(), 1, 2, 2, &out) == RK_OK);
  EXPECT(out.total_tokens == 5);  // 1 + 1 + 2 | 1
  EXPECT(rk_prune_layout(&in, nullptr, 1, 2, 2, &out) == RK_ERR_INVALID_ARG);
  EXPECT(rk_prune_layout(&in, lt.data(), 1, 3, 2, &out) == RK_ERR_INVALID_ARG);
  EXPECT(rk_compress_layout(&in, -1, 2, &out) == RK_ERR_INVALID_ARG);
  EXPECT(rk_compress_layout(&in, 1, 0, &out) == RK_ERR_INVALID_ARG);
  EXPECT(rk_compress_layout(nullptr, 1, 1, &out) == RK_ERR_INVALID_ARG);
  EXPECT(rk_compress_layout(&in, 1, 1, nullptr) == RK_ERR_INVALID_ARG);
  ts[3] = 1;  // history out of time order
  EXPECT(rk_compress_layout(&in, 1, 1, &out) == RK_ERR_UNSORTED_TIME);
  ts[3] = 30;
  kind[2] = 0;  // PROFILE after HISTORY
  EXPECT(rk_compress_layout(&in, 1, 1, &out) == RK_ERR_SEGMENT_ORDER);
  kind[2] = 9;  // not a segment kind
  EXPECT(rk_compress_layout(&in, 1, 1, &out) == RK_ERR_SEGMENT_ORDER);
  kind[2] = 1;
  offs[2] = 12;  // last offset != total_tokens
  EXPECT(rk_compress_layout(&in, 1, 1, &out) == RK_ERR_INVALID_ARG);
  offs[2] = 11;
  int32_t m = 0;
  EXPECT(rk_pruned_history_length(1152, 128, 3, 5, &m) == RK_OK && m == 640);
  EXPECT(rk_pruned_history_length(1152, 128, 0, 5, &m) == RK_ERR_INVALID_ARG);
  EXPECT(rk_pruned_history_length(1152, 128, 1, 5, nullptr) == RK_ERR_INVALID_ARG);
  EXPECT(rk_gather_sum(nullptr, 1, 1, nullptr, 1, nullptr, 1, 1, (rk_dtype)5, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_gather_sum(nullptr, 0, 0, nullptr, 0, nullptr, 0, 0, RK_F32, nullptr) == RK_OK);
  // SORT query pruning: exponential schedule, pooled layout
  rk_prune_params pp;
  std::memset(&pp, 0, sizeof(pp));
  pp.struct_size = sizeof(pp);
  pp.schedule = RK_PRUNE_EXP;
  pp.n_min = 0;
  pp.layer = 2;
  pp.decay = 0.5;
  EXPECT(rk_pruned_history_length_ex(5, &pp, &m) == RK_OK && m == 3);  // 2.5 rounds away from 0
  pp.pool = 1;
  EXPECT(rk_prune_layout_ex(&in, lt.data(), &pp, &out) == RK_OK);
  // request 0 keeps 3 of 5 history tokens (+1 pooled), request 1 keeps 2 of 3 (+1 pooled)
  EXPECT(out.total_tokens == 10 && o2[1] == 7 && o2[2] == 10);
  EXPECT(r2[2] == 1 && r2[3] == 3 && t2[1] == 20);  // pooled rows [1, 3), newest member's time
  pp.decay = 0.0;
  EXPECT(rk_pruned_history_length_ex(5, &pp, &m) == RK_ERR_INVALID_ARG);
  EXPECT(rk_prune_layout_ex(&in, lt.data(), &pp, &out) == RK_ERR_INVALID_ARG);
  pp.decay = 0.5;
  pp.schedule = 7;
  EXPECT(rk_pruned_history_length_ex(5, &pp, &m) == RK_ERR_INVALID_ARG);
  EXPECT(rk_pruned_history_length_ex(5, nullptr, &m) == RK_ERR_INVALID_ARG);
  EXPECT(rk_prune_layout_ex(&in, lt.data(), nullptr, &out) == RK_ERR_INVALID_ARG);
  EXPECT(rk_gather_mean(nullptr, 1, 1, nullptr, 1, nullptr, 1, 1, (rk_dtype)5, nullptr) ==
         RK_ERR_INVALID_ARG);
  EXPECT(rk_gather_mean(nullptr, 0, 0, nullptr, 0, nullptr, 0, 0, RK_F32, nullptr) == RK_OK);
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--self-test") == 0) {
    // proves the instrumentation is live: AddressSanitizer must stop here
    volatile int* p = new int[4];
    p[4] = 1;
    delete[] p;
    return 0;
  }
  check_status_strings();
  check_workspace_size();
  check_mask_plan();
  check_time_rope();
  check_attention_without_plan();
  check_layouts();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
