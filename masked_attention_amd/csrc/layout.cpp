// LazFormer pre-passes on the host (section 2.3): group-sum compression of
// long histories (eq. 16-18) and the per-layer history length and pruning of
// eq. 22; SORT's query pruning (section 3.2.2) with its exponential schedule
// and its pooled form.  Each output token is described by a contiguous range
// of input rows; the rows themselves move on the device (rk_gather_sum,
// rk_gather_mean).
#include <cmath>
#include <cstring>
#include <vector>

#include "rk_internal.h"

namespace {

struct Tok {
  uint8_t kind;
  int64_t time;
  int32_t b, e;  // input rows [b, e)
};

rk_status check_layout(const rk_host_layout* in) {
  if (!in || in->struct_size < sizeof(rk_host_layout)) return RK_ERR_INVALID_ARG;
  if (in->num_requests < 0 || in->total_tokens < 0 || !in->req_offsets) return RK_ERR_INVALID_ARG;
  const int32_t* o = in->req_offsets;
  if (o[0] != 0 || o[in->num_requests] != in->total_tokens) return RK_ERR_INVALID_ARG;
  for (int32_t r = 0; r < in->num_requests; ++r)
    if (o[r + 1] < o[r]) return RK_ERR_INVALID_ARG;
  if (in->total_tokens > 0 && (!in->seg_kind || !in->timestamps)) return RK_ERR_INVALID_ARG;
  for (int32_t r = 0; r < in->num_requests; ++r) {
    for (int32_t j = o[r]; j < o[r + 1]; ++j) {
      if (in->seg_kind[j] > RK_SEG_CANDIDATE) return RK_ERR_SEGMENT_ORDER;
      if (j > o[r] && in->seg_kind[j] < in->seg_kind[j - 1]) return RK_ERR_SEGMENT_ORDER;
      if (j > o[r] && in->seg_kind[j] == RK_SEG_HISTORY && in->seg_kind[j - 1] == RK_SEG_HISTORY &&
          in->timestamps[j] < in->timestamps[j - 1])
        return RK_ERR_UNSORTED_TIME;
    }
  }
  return RK_OK;
}

rk_status check_out(const rk_layout_out* out, int32_t R) {
  if (!out || out->struct_size < sizeof(rk_layout_out) || out->capacity < 0) return RK_ERR_INVALID_ARG;
  (void)R;
  return RK_OK;
}

// Emit the tokens of every request through `build` (which appends the
// request's output tokens to a vector) into `out`.
template <typename Build>
rk_status emit(const rk_host_layout* in, rk_layout_out* out, Build build) {
  std::vector<Tok> toks;
  std::vector<int32_t> offs(in->num_requests + 1, 0);
  for (int32_t r = 0; r < in->num_requests; ++r) {
    build(r, toks);
    if (toks.size() > (size_t)2147483647) return RK_ERR_UNSUPPORTED;
    offs[r + 1] = (int32_t)toks.size();
  }
  const int32_t n = (int32_t)toks.size();
  out->total_tokens = n;
  if (n > out->capacity) return RK_ERR_WORKSPACE_TOO_SMALL;
  if (!out->req_offsets || (n > 0 && (!out->seg_kind || !out->timestamps || !out->ranges)))
    return RK_ERR_INVALID_ARG;
  std::memcpy(out->req_offsets, offs.data(), sizeof(int32_t) * offs.size());
  for (int32_t i = 0; i < n; ++i) {
    out->seg_kind[i] = toks[i].kind;
    out->timestamps[i] = toks[i].time;
    out->ranges[2 * i] = toks[i].b;
    out->ranges[2 * i + 1] = toks[i].e;
  }
  return RK_OK;
}

// dv: the dtype argument as the int a C caller passed (read without
// loading an enum that may hold no enumerator)
rk_status gather(const int32_t* ranges, int32_t n_out, int32_t n_in, const void* x,
                 int64_t x_stride, void* y, int64_t y_stride, int32_t width, int dv,
                 void* stream, bool mean) {
  if (dv != RK_F32 && dv != RK_BF16) return RK_ERR_INVALID_ARG;
  if (n_out < 0 || n_in < 0 || width < 0 || x_stride < 0 || y_stride < 0) return RK_ERR_INVALID_ARG;
  if (n_out == 0 || width == 0) return RK_OK;
  if (!ranges || !y || (n_in > 0 && !x) || y_stride < width) return RK_ERR_INVALID_ARG;
  if (n_in > 0 && x_stride < width) return RK_ERR_INVALID_ARG;
  hipError_t e = rk::launch_gather_sum(ranges, n_out, n_in, x, x_stride, y, y_stride, width,
                                       (rk_dtype)dv, (hipStream_t)stream, mean);
  return e == hipSuccess ? RK_OK : RK_ERR_HIP;
}


}  // namespace

extern "C" {

rk_status rk_compress_layout(const rk_host_layout* in, int32_t keep, int32_t group,
                             rk_layout_out* out) {
  rk_status st = check_layout(in);
  if (st != RK_OK) return st;
  if ((st = check_out(out, in->num_requests)) != RK_OK) return st;
  if (keep < 0 || group < 1) return RK_ERR_INVALID_ARG;
  const int32_t* o = in->req_offsets;
  const uint8_t* k = in->seg_kind;
  const int64_t* t = in->timestamps;
  return emit(in, out, [&](int32_t r, std::vector<Tok>& v) {
    // segments are contiguous (kinds non-decreasing): history = [h0, h1)
    int32_t h0 = o[r], h1 = o[r];
    while (h0 < o[r + 1] && k[h0] < RK_SEG_HISTORY) ++h0;
    h1 = h0;
    while (h1 < o[r + 1] && k[h1] == RK_SEG_HISTORY) ++h1;
    for (int32_t j = o[r]; j < h0; ++j) v.push_back({k[j], t[j], j, j + 1});
    const int32_t L = h1 - h0;
    const int32_t ell = L < keep ? L : keep;
    const int32_t n_old = L - ell;
    // groups counted back from the kept part: the first (oldest) may be short
    const int32_t n_groups = (int32_t)(((int64_t)n_old + group - 1) / group);
    for (int32_t g = 0; g < n_groups; ++g) {
      const int32_t e = h0 + n_old - (n_groups - 1 - g) * group;
      const int32_t b = e - group > h0 ? e - group : h0;
      v.push_back({(uint8_t)RK_SEG_HISTORY, t[e - 1], b, e});
    }
    for (int32_t j = h0 + n_old; j < h1; ++j) v.push_back({k[j], t[j], j, j + 1});
    for (int32_t j = h1; j < o[r + 1]; ++j) v.push_back({k[j], t[j], j, j + 1});
  });
}

rk_status rk_pruned_history_length(int32_t l_tilde, int32_t n_min, int32_t layer,
                                   int32_t num_layers, int32_t* n_out) {
  if (!n_out || l_tilde < 0 || n_min < 0 || num_layers < 1 || layer < 1 || layer > num_layers)
    return RK_ERR_INVALID_ARG;
  if (num_layers == 1) {
    *n_out = l_tilde;
    return RK_OK;
  }
  const double val =
      (double)l_tilde - (double)(layer - 1) / (double)(num_layers - 1) * ((double)l_tilde - n_min);
  const double rnd = val >= 0 ? std::floor(val + 0.5) : -std::floor(-val + 0.5);
  double n = rnd > n_min ? rnd : (double)n_min;
  if (n > l_tilde) n = l_tilde;
  *n_out = (int32_t)n;
  return RK_OK;
}

rk_status rk_prune_layout(const rk_host_layout* in, const int32_t* l_tilde, int32_t n_min,
                          int32_t layer, int32_t num_layers, rk_layout_out* out) {
  rk_status st = check_layout(in);
  if (st != RK_OK) return st;
  if ((st = check_out(out, in->num_requests)) != RK_OK) return st;
  if (!l_tilde && in->num_requests > 0) return RK_ERR_INVALID_ARG;
  std::vector<int32_t> keep(in->num_requests);
  for (int32_t r = 0; r < in->num_requests; ++r)
    if ((st = rk_pruned_history_length(l_tilde[r], n_min, layer, num_layers, &keep[r])) != RK_OK)
      return st;
  const int32_t* o = in->req_offsets;
  const uint8_t* k = in->seg_kind;
  const int64_t* t = in->timestamps;
  return emit(in, out, [&](int32_t r, std::vector<Tok>& v) {
    int32_t n_hist = 0;
    for (int32_t j = o[r]; j < o[r + 1]; ++j) n_hist += k[j] == RK_SEG_HISTORY;
    int32_t drop = n_hist - keep[r] > 0 ? n_hist - keep[r] : 0;  // oldest history tokens
    for (int32_t j = o[r]; j < o[r + 1]; ++j) {
      if (k[j] == RK_SEG_HISTORY && drop > 0) {
        --drop;
        continue;
      }
      v.push_back({k[j], t[j], j, j + 1});
    }
  });
}

rk_status rk_pruned_history_length_ex(int32_t l_tilde, const rk_prune_params* p,
                                      int32_t* n_out) {
  if (!p || p->struct_size < sizeof(rk_prune_params) || !n_out) return RK_ERR_INVALID_ARG;
  if (p->schedule == RK_PRUNE_LINEAR)
    return rk_pruned_history_length(l_tilde, p->n_min, p->layer, p->num_layers, n_out);
  if (p->schedule != RK_PRUNE_EXP) return RK_ERR_INVALID_ARG;
  if (l_tilde < 0 || p->n_min < 0 || p->layer < 1 || !(p->decay > 0.0 && p->decay <= 1.0))
    return RK_ERR_INVALID_ARG;
  // l_tilde * decay^(layer - 1), rounded half away from zero, floored at
  // n_min and capped at l_tilde
  const double val = (double)l_tilde * std::pow(p->decay, (double)(p->layer - 1));
  double n = std::floor(val + 0.5);
  if (n < p->n_min) n = p->n_min;
  if (n > l_tilde) n = l_tilde;
  *n_out = (int32_t)n;
  return RK_OK;
}

rk_status rk_prune_layout_ex(const rk_host_layout* in, const int32_t* l_tilde,
                             const rk_prune_params* p, rk_layout_out* out) {
  rk_status st = check_layout(in);
  if (st != RK_OK) return st;
  if ((st = check_out(out, in->num_requests)) != RK_OK) return st;
  if (!p || p->struct_size < sizeof(rk_prune_params)) return RK_ERR_INVALID_ARG;
  if (!l_tilde && in->num_requests > 0) return RK_ERR_INVALID_ARG;
  std::vector<int32_t> keep(in->num_requests);
  for (int32_t r = 0; r < in->num_requests; ++r)
    if ((st = rk_pruned_history_length_ex(l_tilde[r], p, &keep[r])) != RK_OK) return st;
  const int32_t* o = in->req_offsets;
  const uint8_t* k = in->seg_kind;
  const int64_t* t = in->timestamps;
  const bool pool = p->pool != 0;
  return emit(in, out, [&](int32_t r, std::vector<Tok>& v) {
    int32_t n_hist = 0;
    for (int32_t j = o[r]; j < o[r + 1]; ++j) n_hist += k[j] == RK_SEG_HISTORY;
    const int32_t drop = n_hist - keep[r] > 0 ? n_hist - keep[r] : 0;  // oldest history tokens
    int32_t seen = 0;
    for (int32_t j = o[r]; j < o[r + 1]; ++j) {
      if (k[j] == RK_SEG_HISTORY && seen < drop) {
        // history is contiguous: the dropped tokens are rows [j, j + drop)
        // and, pooled, become one token dated as their newest member
        if (pool && seen == 0) v.push_back({(uint8_t)RK_SEG_HISTORY, t[j + drop - 1], j, j + drop});
        ++seen;
        continue;
      }
      v.push_back({k[j], t[j], j, j + 1});
    }
  });
}

rk_status rk_gather_sum(const int32_t* ranges, int32_t n_out, int32_t n_in, const void* x,
                        int64_t x_stride, void* y, int64_t y_stride, int32_t width,
                        rk_dtype dtype, void* stream) {
  int dv;
  std::memcpy(&dv, &dtype, sizeof dv);
  return gather(ranges, n_out, n_in, x, x_stride, y, y_stride, width, dv, stream, false);
}

rk_status rk_gather_mean(const int32_t* ranges, int32_t n_out, int32_t n_in, const void* x,
                         int64_t x_stride, void* y, int64_t y_stride, int32_t width,
                         rk_dtype dtype, void* stream) {
  int dv;
  std::memcpy(&dv, &dtype, sizeof dv);
  return gather(ranges, n_out, n_in, x, x_stride, y, y_stride, width, dv, stream, true);
}

}  // extern "C"
