// Mask planner: row descriptors, 128x64 tile classification with exact
// visible-pair counts, per-query-tile CSR of non-empty key tiles, and the
// XCD-aware launch schedule.
//
// The visibility rule (CADET delay mask; SORT U2U/C2U/C2C and local window;
// LazFormer eq. 19-21; MTGR mixed dynamic mask) gives every query row a
// visible key set that is one interval [lo, hi) of request-local positions
// plus, for candidates, the row itself:
//   static query, causal   : [max(0, p-W+1), p+1) intersected, with a delay,
//                            with the keys dated at or before t_i - delay:
//                            a prefix of PROFILE and a prefix of HISTORY
//                            (each segment is in time order, so one binary
//                            search per segment).  Their union is one run
//                            when every profile key is that old (profile
//                            dated before the history), when no profile key
//                            is (profile dated at the anchor, "now"), or
//                            when one of the two parts falls outside the
//                            causal window; a row left with two runs is
//                            reported as a timestamp-order error.
//                            lo = 0 for the last G static rows (global tail)
//   static query, bidir.   : [0, end of static)
//   real-time query        : [0, p+1)  (static part, then real-time events up
//                            to itself; sorted times make t_j <= t_i implied)
//   candidate query        : [0, end of static + #real-time events with
//                            t_j < t_i) plus itself.
// Tile counts are sums of interval overlaps, so they are exact integers.
#include <climits>

#include "rk_internal.h"

namespace rk {
namespace {

// Number of keys in ts[0, n) (non-decreasing) with value <= x, or < x with
// kStrict, helped by samples of ts held in LDS: samp[j] = ts[j * step] for
// j < ceil(n / step) (at most kSamples).  The samples that pass bracket the
// answer to one step of positions, (p_{k-1}, p_k], searched in memory; with
// step 1 no memory is read.  On unsorted ts (which the row checks report)
// the result is still in [0, n].
constexpr int kSamples = 256;  // one per thread of the block

// Where the first planner kernel finds the plan's host tables: in the
// workspace already (blob null), or in a pinned host block that it reads
// directly, copying 16-byte words [lo16, hi16) (the tables past the request
// records) into the workspace; request records are written by the blocks
// that read them.
struct PlanSource {
  const ReqMeta* req;
  const int32_t* qt_req;
  const uint4* blob;
  uint4* dst;
  int64_t lo16, hi16;
  int R;
};
template <bool kStrict>
__device__ __forceinline__ int count_sampled(const int64_t* __restrict__ ts, int n, int64_t x,
                                             const long long* samp, int step) {
  if (n <= 0) return 0;
  const int m = (n + step - 1) / step;
  int a = 0, b = m;
  while (a < b) {
    const int mid = (a + b) >> 1;
    if (kStrict ? samp[mid] < x : samp[mid] <= x) a = mid + 1; else b = mid;
  }
  int lo = a == 0 ? 0 : (a - 1) * step + 1;
  int hi = a == m ? n : a * step;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (kStrict ? ts[mid] < x : ts[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Sum over the 64 lanes of a wave (integers: order does not matter).
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive scan of one int per thread over a block of blockDim.x (<= 1024)
// threads.  Returns the exclusive prefix; *total receives the block sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* smem, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) smem[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      int t = smem[w];
      smem[w] = run;
      run += t;
    }
    smem[16] = run;
  }
  __syncthreads();
  int res = smem[wave] + x - v;
  *total = smem[16];
  __syncthreads();
  return res;
}

// Block-wide sum of one value per thread (blockDim.x a multiple of 64,
// at most 1024): wave sums, then the waves' sums in order.  Every thread
// gets the total.
__device__ __forceinline__ long long block_sum(long long v, long long* red) {
  v = wave_sum(v);
  const int nw = (int)(blockDim.x >> 6);
  __syncthreads();  // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

// Request-local starts of segment kinds 1..3 of one request (lo_s[k - 1] =
// number of tokens of kind < k; kinds are non-decreasing inside a request)
// by a sampled search over its kinds: each round takes 256 evenly spaced
// samples of every boundary's window and keeps the one gap that holds the
// boundary, so a window of n positions takes ceil(log_256 n) rounds (two
// at 20,000 tokens).  Kinds out of order (reported by the row checks)
// still give values in [0, L].  lo_s, hi_s: __shared__ int[3].
__device__ void seg_search(const uint8_t* __restrict__ kr, int L, int* lo_s, int* hi_s) {
  const int t = threadIdx.x;  // blockDim.x == 256
  if (t < 3) {
    lo_s[t] = 0;
    hi_s[t] = L;
  }
  __syncthreads();
  while (lo_s[0] < hi_s[0] || lo_s[1] < hi_s[1] || lo_s[2] < hi_s[2]) {
    int lo[3], hi[3], step[3], c[3];
    bool below[3];
    // the three boundaries' samples are loaded together, then counted
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      lo[k] = lo_s[k];
      hi[k] = hi_s[k];
      const int n = hi[k] - lo[k];  // the boundary lies in [lo, hi]
      step[k] = n > 0 ? (n - 1) / 256 + 1 : 1;
      const int64_t pos = lo[k] + (int64_t)t * step[k];
      below[k] = n > 0 && pos < hi[k] && kr[pos] <= k;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) c[k] = __syncthreads_count(below[k]);
    if (t < 3) {
      const int k = t;
      if (hi[k] > lo[k]) {
        if (c[k] == 0) {
          hi_s[k] = lo[k];  // the window's first token already has kind >= k + 1
        } else {
          // sample c - 1 is below kind k + 1, sample c (if any) is not
          lo_s[k] = lo[k] + (c[k] - 1) * step[k] + 1;
          hi_s[k] = (int)min((int64_t)hi[k], (int64_t)lo[k] + (int64_t)c[k] * step[k]);
        }
      }
    }
    __syncthreads();
  }
}

// Request-local starts of kinds 1..3 (lo_s[k - 1] = tokens of kind < k)
// by counting over the whole request in one memory round: each thread
// counts the kinds in its 16-byte words of [tok_off, tok_off + L) (a word
// that is not wholly inside the T-byte array is read byte by byte, inside
// the request only).  Equal to seg_search's result when kinds are
// non-decreasing; any kinds give values in [0, L].  Ends with a barrier.
constexpr int kSegCountMax = 16384;  // longer requests use seg_search
__device__ void seg_count(const uint8_t* __restrict__ kind, int64_t tok_off, int L, int64_t T,
                          int* lo_s, long long* red) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(kind);
  const uintptr_t rs = base + (uintptr_t)tok_off, re = rs + (uintptr_t)L;
  const uintptr_t w0 = rs & ~(uintptr_t)15;
  const int nw = (int)((re - w0 + 15) >> 4);
  long long c = 0;  // tokens of kind <= 0, <= 1, <= 2 in bits 0, 21, 42
  auto tally = [&](unsigned b) {
    c += (long long)(b <= 0u) + ((long long)(b <= 1u) << 21) + ((long long)(b <= 2u) << 42);
  };
  for (int w = threadIdx.x; w < nw; w += blockDim.x) {
    const uintptr_t a = w0 + 16 * (uintptr_t)w;
    const int jb = rs > a ? (int)(rs - a) : 0;
    const int je = re < a + 16 ? (int)(re - a) : 16;
    if (a >= base && a + 16 <= base + (uintptr_t)T) {
      const uint4 v = *reinterpret_cast<const uint4*>(a);
      const unsigned wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j >= jb && j < je) tally((wd[j >> 2] >> (8 * (j & 3))) & 0xffu);
    } else {
      for (int j = jb; j < je; ++j) tally(*reinterpret_cast<const uint8_t*>(a + j));
    }
  }
  c = block_sum(c, red);
  if (threadIdx.x < 3) lo_s[threadIdx.x] = (int)((c >> (21 * threadIdx.x)) & ((1 << 21) - 1));
  __syncthreads();
}

// Record of a launch slot without work.
__device__ __forceinline__ ItemRec no_item_rec() {
  ItemRec rc;
  rc.tok_off = rc.len = rc.row0 = rc.e0 = rc.n = rc.req = rc.w0 = rc.w1 = 0;
  rc.head = rc.part = -1;
  rc.pad[0] = rc.pad[1] = 0;
  return rc;
}

// Record of item (q-tile * H + head) over CSR entries [kbeg, kend) of its
// row (kend < 0: the whole row); the CSR must be complete.
__device__ __forceinline__ ItemRec item_rec(const PlanDev& P, int item, int kbeg, int kend,
                                            int part, int H) {
  if (item < 0) return no_item_rec();
  const int qg = item / H;
  const int r = P.qt_req[qg];
  const ReqMeta m = P.req[r];
  ItemRec rc = no_item_rec();
  rc.tok_off = m.tok_off;
  rc.len = m.len;
  rc.row0 = (qg - m.qt_off) * kTileQ;
  rc.head = item - qg * H;
  rc.e0 = P.qtile_ptr[qg] + kbeg;
  rc.n = kend >= 0 ? kend - kbeg : P.qtile_ptr[qg + 1] - rc.e0;
  rc.req = r;
  rc.part = part;
  rc.w0 = rc.n > 0 ? P.ktile_word[rc.e0] : 0;
  rc.w1 = rc.n > 1 ? P.ktile_word[rc.e0 + 1] : rc.w0;
  return rc;
}

// One block (256 threads) per global q-tile: the request's segment starts
// (a counting pass over its kinds, or a sampled search beyond
// kSegCountMax tokens; the request's first q-tile records them), the order
// checks and visible interval (row descriptor) of each of its 128 rows, and
// the exact visible count and class of each of its k-tiles with the
// q-tile's partial totals (non-empty, FULL, pairs, check flags).  It also
// marks its share of the launch schedule idle and, when the host tables
// come from a pinned host block, copies them into the workspace; the CSR
// kernel writes the items.
//
// Row checks: segment kinds non-decreasing and in range; real-time events
// in time order; PROFILE and HISTORY each in time order when the delay rule
// searches them (an out-of-order history is otherwise only noted).
//
// Tile counts: from the extremes of the rows' intervals [lo, hi) (lo_max,
// hi_min, lo_min, hi_max over the q-tile's rows) most k-tiles [c0, c1) are
// decided without visiting the rows: a tile with lo_max <= c0 and c1 <=
// hi_min holds nrows * (c1 - c0) pairs (a row's own key, if in the tile,
// is inside its interval), FULL when that is 128 * 64; a tile with c0 >=
// hi_max or c1 <= lo_min that holds no row's own position is EMPTY.  The
// rest (diagonal, window and delay boundaries) are listed in LDS and
// counted row by row, the block's lanes spread over the list.
__global__ __launch_bounds__(256) void plan_rows_tiles_kernel(
    PlanDev P, PlanSource src, const uint8_t* __restrict__ kind, const int64_t* __restrict__ ts,
    int64_t T, int64_t delay, int window, int global_tail, int bidir, int check_static_time,
    int slots) {
  __shared__ int2 d[kTileQ];
  __shared__ unsigned long long pairs_s;
  __shared__ int nnz_s, full_s;
  __shared__ int lim[4];  // lo_max, hi_min, lo_min, hi_max
  __shared__ int lo_s[3], hi_s[3];
  __shared__ long long samp[3][kSamples];  // PROFILE, HISTORY, REALTIME sample times
  __shared__ unsigned flags_s;              // errors | info << 16 of the q-tile's rows
  __shared__ long long red[16];
  __shared__ int slow[256];                 // k-tiles counted row by row
  __shared__ int nslow_s;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t gstride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t x = (int64_t)g * blockDim.x + tid; x < slots; x += gstride) {
    P.sched[x] = -1;
    P.irec[x] = no_item_rec();
  }
  if (src.blob) {
    // host tables past the request records, into the workspace
    for (int64_t x = src.lo16 + (int64_t)g * blockDim.x + tid; x < src.hi16; x += gstride)
      src.dst[x] = src.blob[x];
    // records of empty requests (a request with q-tiles writes its own below)
    for (int64_t x = (int64_t)g * blockDim.x + tid; x < src.R; x += gstride) {
      const ReqMeta e = src.req[x];
      if (e.nqt == 0) P.req[x] = e;
    }
  }
  const int r = src.qt_req[g];
  const ReqMeta m = src.req[r];
  const int qt = g - m.qt_off;
  const int L = m.len;
  const int row0 = qt * kTileQ;
  const int nrows = min(kTileQ, L - row0);
  const int64_t* tr = ts + m.tok_off;
  // this thread's row (threads below nrows): kind and time of it and of the
  // row before, loaded ahead of the segment pass so that the two overlap
  int s_row = 0, s_prev = 0;
  int64_t t_row = 0, t_prev = 0;
  if (tid < nrows) {
    const int64_t i = (int64_t)m.tok_off + row0 + tid;
    s_row = kind[i];
    t_row = ts[i];
    if (row0 + tid > 0) {
      s_prev = kind[i - 1];
      t_prev = ts[i - 1];
    }
  }
  // the request's first q-tile writes the request's record with its segment
  // starts (words kSeg.. of the record)
  constexpr int kSeg = offsetof(ReqMeta, seg) / 4;
  static_assert(offsetof(ReqMeta, seg) % 4 == 0 && sizeof(ReqMeta) == 4 * (kSeg + 4),
                "segment starts close the request record");
  int rec_word = 0;
  if (qt == 0 && tid < kSeg) rec_word = reinterpret_cast<const int*>(src.req + r)[tid];
  if (tid == 0) {
    flags_s = 0;
    nslow_s = 0;
  }
  if (L <= kSegCountMax)
    seg_count(kind, m.tok_off, L, T, lo_s, red);
  else
    seg_search(kind + m.tok_off, L, lo_s, hi_s);
  if (qt == 0 && tid < kSeg + 4)
    reinterpret_cast<int*>(P.req + r)[tid] =
        tid < kSeg ? rec_word : (tid == kSeg ? 0 : lo_s[tid - kSeg - 1]);
  // segment boundaries, made monotone and clamped so that any device data
  // yields in-range descriptors
  const int a_rt = min(max(lo_s[RK_SEG_REALTIME - 1], 0), L);
  const int a_c = min(max(lo_s[RK_SEG_CANDIDATE - 1], a_rt), L);
  const int a_h = min(max(lo_s[RK_SEG_HISTORY - 1], 0), a_rt);
  if (tid == 0) {
    pairs_s = 0; nnz_s = 0; full_s = 0;
    lim[0] = INT_MIN; lim[1] = INT_MAX; lim[2] = INT_MAX; lim[3] = INT_MIN;
  }
  // Samples of the three time-ordered runs the rows search (profile and
  // history for the delay cut, real-time for a candidate's events), one
  // load per thread, so each row's search reads memory for one step of
  // positions only.
  const bool cut_static = !bidir && delay > 0;
  const int n_rt = a_c - a_rt;
  const int st_p = max(1, (a_h + kSamples - 1) / kSamples);
  const int st_h = max(1, (a_rt - a_h + kSamples - 1) / kSamples);
  const int st_r = max(1, (n_rt + kSamples - 1) / kSamples);
  if (cut_static) {
    if (tid * st_p < a_h) samp[0][tid] = tr[tid * st_p];
    if (tid * st_h < a_rt - a_h) samp[1][tid] = tr[a_h + tid * st_h];
  }
  if (a_c < L && tid * st_r < n_rt) samp[2][tid] = tr[a_rt + tid * st_r];
  __syncthreads();
  if (tid < kTileQ) {
    int2 desc = make_int2(0, 0);
    if (tid < nrows) {
      const int p = row0 + tid;
      const int i = m.tok_off + p;
      unsigned err = 0, info = 0;
      int s = s_row;
      if (s > RK_SEG_CANDIDATE) { err |= kErrSegment; s = RK_SEG_CANDIDATE; }
      if (p > 0) {
        int prev = s_prev;
        if (prev > RK_SEG_CANDIDATE) prev = RK_SEG_CANDIDATE;
        if (s < prev) {
          err |= kErrSegment;
        } else if (s == prev && t_row < t_prev) {
          if (s == RK_SEG_REALTIME || (check_static_time && s <= RK_SEG_HISTORY)) err |= kErrTime;
          if (s == RK_SEG_HISTORY) info = kInfoHistoryUnsorted;
        }
      }
      int lo = 0, hi = 0, diag = 0;
      if (s <= RK_SEG_HISTORY) {
        if (bidir) {
          hi = a_rt;
        } else {
          hi = min(p + 1, a_rt);
          // the last global_tail static positions are global queries (no window)
          lo = (window > 0 && p < a_rt - global_tail) ? max(0, p - window + 1) : 0;
          if (delay > 0) {
            // keys dated at or before the cut: [0, cp) of PROFILE and
            // [a_h, a_h + ch) of HISTORY
            const int64_t cut = t_row - delay;
            const int cp = count_sampled<false>(tr, a_h, cut, samp[0], st_p);
            const int ch = count_sampled<false>(tr + a_h, a_rt - a_h, cut, samp[1], st_h);
            const bool prof_run = min(cp, hi) > lo;
            const bool hist_run = min(a_h + ch, hi) > max(a_h, lo);
            if (cp == a_h) {
              hi = min(hi, a_h + ch);  // the whole profile, then a history prefix
            } else if (hist_run) {
              if (prof_run) err |= kErrStaticSplit;  // two runs
              lo = max(lo, a_h);
              hi = min(hi, a_h + ch);
            } else {
              hi = min(hi, cp);
            }
          }
        }
      } else if (s == RK_SEG_REALTIME) {
        hi = p + 1;
      } else {
        hi = a_rt + count_sampled<true>(tr + a_rt, n_rt, t_row, samp[2], st_r);
        diag = 1;
      }
      if (hi <= lo) { lo = 0; hi = 0; }
      desc = make_int2(lo, (int)((unsigned)hi | ((unsigned)diag << 31)));
      P.row_desc[i] = desc;
      if (err | info) atomicOr(&flags_s, err | (info << 16));
    }
    d[tid] = desc;
  }
  __syncthreads();
  if (tid < kTileQ) {  // waves 0 and 1: the rows' extremes
    const bool ok = tid < nrows;
    const int lo = d[tid].x, hi = d[tid].y & 0x7fffffff;
    int v0 = ok ? lo : INT_MIN, v1 = ok ? hi : INT_MAX, v2 = ok ? lo : INT_MAX,
        v3 = ok ? hi : INT_MIN;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      v0 = max(v0, __shfl_xor(v0, o, 64));
      v1 = min(v1, __shfl_xor(v1, o, 64));
      v2 = min(v2, __shfl_xor(v2, o, 64));
      v3 = max(v3, __shfl_xor(v3, o, 64));
    }
    if ((tid & 63) == 0) {
      atomicMax(&lim[0], v0);
      atomicMin(&lim[1], v1);
      atomicMin(&lim[2], v2);
      atomicMax(&lim[3], v3);
    }
  }
  __syncthreads();
  const int lo_max = lim[0], hi_min = lim[1], lo_min = lim[2], hi_max = lim[3];
  // K-tiles decided from the extremes (FULL or EMPTY) are written at once;
  // the others of each chunk of 256 are listed and counted row by row with
  // the block's lanes spread over them: S = 2^j lanes per listed tile
  // (S * listed <= 256, S <= 64), each over 128 / S rows, meeting by
  // shuffles.
  const int64_t trow = m.tile_off + (int64_t)qt * m.nkt;
  unsigned long long pairs = 0;
  int nnz = 0, nfull = 0;
  auto put = [&](int kt, int cnt) {
    const uint8_t cls =
        cnt == 0 ? RK_TILE_EMPTY : (cnt == kTileQ * kTileK ? RK_TILE_FULL : RK_TILE_PARTIAL);
    P.tile_count[trow + kt] = cnt;
    P.tile_class[trow + kt] = cls;
    pairs += cnt;
    nnz += cnt > 0;
    nfull += cls == RK_TILE_FULL;
  };
  for (int kt0 = 0; kt0 < m.nkt; kt0 += blockDim.x) {  // uniform trip count
    const int kt = kt0 + tid;
    if (kt < m.nkt) {
      const int c0 = kt * kTileK;
      const int c1 = min(L, c0 + kTileK);
      // every row's interval covers the tile's keys (then so does it hold
      // each row's own key if in the tile): nrows * width pairs, FULL when
      // that is 8192
      const bool cover = lo_max <= c0 && c1 <= hi_min;
      const bool empty = (c0 >= hi_max || c1 <= lo_min) && (c1 <= row0 || c0 >= row0 + nrows);
      if (cover)
        put(kt, nrows * (c1 - c0));
      else if (empty)
        put(kt, 0);
      else
        slow[atomicAdd(&nslow_s, 1)] = kt;
    }
    __syncthreads();
    const int ns = nslow_s;
    int S = 64;
    while (S > 1 && S * ns > (int)blockDim.x) S >>= 1;
    const int slice = tid & (S - 1);
    const int per = kTileQ / S;  // rows of a lane: slice * per .. + per
    const int t0 = slice * per, t1 = min(nrows, t0 + per);
    // every lane of a tile's group runs the same trip count and takes the
    // same branch, so the shuffles below see all S lanes
    for (int j0 = 0; j0 < ns; j0 += (int)blockDim.x / S) {
      const int j = j0 + tid / S;
      int cnt = 0, ktj = 0;
      if (j < ns) {
        ktj = slow[j];
        const int c0 = ktj * kTileK;
        const int c1 = min(L, c0 + kTileK);
        for (int t = t0; t < t1; ++t) {
          const int lo = d[t].x;
          const int hi = d[t].y & 0x7fffffff;
          const int a = max(lo, c0), b = min(hi, c1);
          cnt += max(0, b - a);
          if (d[t].y < 0) {
            const int pr = row0 + t;
            if (pr >= c0 && pr < c1 && !(pr >= lo && pr < hi)) cnt += 1;
          }
        }
      }
      for (int o = 1; o < S; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
      if (j < ns && slice == 0) put(ktj, cnt);
    }
    if (kt0 + (int)blockDim.x < m.nkt) {  // the list is reused by the next chunk
      __syncthreads();
      if (tid == 0) nslow_s = 0;
      __syncthreads();
    }
  }
  // block sums: wave sums, then one LDS atomic per wave
  pairs = wave_sum(pairs);
  nnz = wave_sum(nnz);
  nfull = wave_sum(nfull);
  if ((tid & 63) == 0) {
    atomicAdd(&pairs_s, pairs);
    atomicAdd(&nnz_s, nnz);
    atomicAdd(&full_s, nfull);
  }
  __syncthreads();
  if (tid == 0) {
    P.qt_nnz[g] = nnz_s;
    P.qt_full[g] = full_s;
    P.qt_pairs[g] = (int64_t)pairs_s;
    P.qt_flags[g] = flags_s;
  }
}

// Blocks 0 .. NQ - 1, one per global q-tile: the start of its CSR row (the
// non-empty k-tiles of all earlier q-tiles), its rank among its request's
// q-tiles (descending non-empty count, ties by index), the ascending list
// of its non-empty k-tiles, and its H items' slots of the blocked XCD
// schedule (slot_of below, inverted: the item of group ga at rank k sits
// at queue position base + C(k) + (ga - first group of its block)).  With
// sched_mode 2 (candidates-only plans) only q-tiles holding a candidate row
// are scheduled (the others' slots stay idle) and their slots are counted
// and collected, in arrival order, for the work list.  Block NQ: the
// plan's totals.
__global__ __launch_bounds__(256) void plan_csr_sched_kernel(PlanDev P, int NQ, int64_t NT, int H,
                                                             int G, int sched_mode,
                                                             unsigned* stage_done) {
  __shared__ int smem[32];
  __shared__ int act_base;
  __shared__ long long red[16];
  __shared__ int w01[2];  // the row's first two CSR words
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  if (g == NQ) {
    __shared__ unsigned flags_s;
    if (tid == 0) flags_s = 0;
    long long nnz = 0, pairs = 0, nfull = 0;
    unsigned fl = 0;
    for (int i = tid; i < NQ; i += blockDim.x) {
      nnz += P.qt_nnz[i];
      pairs += P.qt_pairs[i];
      nfull += P.qt_full[i];
      fl |= P.qt_flags[i];
    }
    nnz = block_sum(nnz, red);  // its barriers also order flags_s = 0 before the ORs
    pairs = block_sum(pairs, red);
    nfull = block_sum(nfull, red);
    if (fl) atomicOr(&flags_s, fl);
    __syncthreads();
    if (tid == 0) {
      P.qtile_ptr[NQ] = (int)nnz;
      P.totals->visible_pairs = (unsigned long long)pairs;
      P.totals->full_tiles = (unsigned long long)nfull;
      P.totals->partial_tiles = (unsigned long long)(nnz - nfull);
      P.totals->empty_tiles = (unsigned long long)(NT - nnz);
      P.totals->errors = flags_s & 0xffffu;
      P.totals->info = flags_s >> 16;
      // the first kernel, the only reader of the staged host tables, has
      // ended: their host block may be reused
      if (stage_done) __hip_atomic_store(stage_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return;
  }
  const int r = P.qt_req[g];
  const ReqMeta m = P.req[r];
  const int qt = g - m.qt_off;
  long long acc = 0;
  for (int i = tid; i < g; i += blockDim.x) acc += P.qt_nnz[i];
  const int base = (int)block_sum(acc, red);
  const int na = P.qt_nnz[g];
  long long rk = 0;
  for (int j = tid; j < m.nqt; j += blockDim.x) {
    const int nb = P.qt_nnz[m.qt_off + j];
    rk += (nb > na) || (nb == na && j < qt);
  }
  const int rank = (int)block_sum(rk, red);
  if (tid == 0) {
    P.qtile_ptr[g] = base;
    P.qorder[m.qt_off + rank] = g;
  }
  const int64_t row = m.tile_off + (int64_t)qt * m.nkt;
  int run = 0;
  for (int k0 = 0; k0 < m.nkt; k0 += blockDim.x) {
    const int kt = k0 + tid;
    const int flag = kt < m.nkt && P.tile_count[row + kt] > 0;
    int total;
    const int ex = block_exclusive_scan(flag, smem, &total);
    if (flag) {
      const int word =
          (int)((unsigned)kt | ((unsigned)(P.tile_class[row + kt] == RK_TILE_PARTIAL) << 31));
      P.ktile_idx[base + run + ex] = kt;
      P.ktile_word[base + run + ex] = word;
      if (run + ex < 2) w01[run + ex] = word;
    }
    run += total;
  }
  const int first_cand = m.seg[RK_SEG_CANDIDATE];  // == len without candidates
  const bool keep =
      sched_mode == 1 || (first_cand < m.len && (qt + 1) * kTileQ > first_cand);
  if (keep) {  // uniform over the block
    __syncthreads();
    if (sched_mode == 2) {
      if (tid == 0) act_base = atomicAdd(&P.totals->n_act, H);
      __syncthreads();
    }
    ItemRec rc = no_item_rec();
    rc.tok_off = m.tok_off;
    rc.len = m.len;
    rc.row0 = qt * kTileQ;
    rc.e0 = base;
    rc.n = na;
    rc.req = r;
    rc.w0 = na > 0 ? w01[0] : 0;
    rc.w1 = na > 1 ? w01[1] : rc.w0;
    for (int h = tid; h < H; h += blockDim.x) {
      const int ga = P.group_of[(int64_t)r * H + h];
      const int f = P.ilv[ga];                  // first group of ga's block
      const int* C = P.ilv + P.ilv[G + ga] + 1;  // the block's C(k)
      const int idx = P.groups[f].base + C[rank] + (ga - f);
      int q = 0;
      while (q < kNumXcd - 1 && ga >= P.queue_start[q + 1]) ++q;
      const int64_t slot = (int64_t)idx * kNumXcd + q;
      P.sched[slot] = g * H + h;
      rc.head = h;
      P.irec[slot] = rc;
      if (sched_mode == 2 && act_base + h < kSplitTarget / 2) P.act_slots[act_base + h] = (int)slot;
    }
  }
}

// Rank sort of n tiles of one request by non-empty count, descending, ties
// by tile index: order[rank] = off + tile.  One block.
__device__ __forceinline__ void rank_order(int n, int off, const int* __restrict__ nnz,
                                           int* __restrict__ order, int* chunk) {
  for (int a0 = 0; a0 < n; a0 += blockDim.x) {
    const int a = a0 + threadIdx.x;
    const int na = a < n ? nnz[a] : 0;
    int rank = 0;
    for (int b0 = 0; b0 < n; b0 += 1024) {
      const int nb = min(1024, n - b0);
      const int nb4 = (nb + 3) & ~3;
      __syncthreads();
      // pad to a multiple of four with a value that never ranks above a
      // tile (counts are >= 0) and never ties
      for (int t = threadIdx.x; t < nb4; t += blockDim.x) chunk[t] = t < nb ? nnz[b0 + t] : INT_MIN;
      __syncthreads();
      if (a < n) {
        // four counts per LDS read, several reads in flight
#pragma unroll 4
        for (int t = 0; t < nb4; t += 4) {
          const int4 v = *(const int4*)&chunk[t];
          const int i0 = b0 + t;
          rank += (v.x > na) || (v.x == na && i0 < a);
          rank += (v.y > na) || (v.y == na && i0 + 1 < a);
          rank += (v.z > na) || (v.z == na && i0 + 2 < a);
          rank += (v.w > na) || (v.w == na && i0 + 3 < a);
        }
      }
    }
    if (a < n) order[off + rank] = off + a;
  }
}

// The group `ga` and rank `k` whose item sits at position `idx` of XCD
// queue `q` of a blocked schedule (groups sorted by (queue, base), the
// groups of a block share the block's first slot as base; ilv as
// PlanDev::ilv describes); ga = -1 for a slot past the block's items.
__device__ void slot_of(const Group* groups, const int32_t* qstart, const int32_t* ilv, int G,
                        int q, int idx, int* ga, int* k) {
  int a = qstart[q], b = qstart[q + 1];
  *ga = -1;
  *k = -1;
  if (a >= b) return;
  // the block holding the slot (the last group with base <= idx is one of it)
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (groups[mid].base <= idx) a = mid; else b = mid;
  }
  const int f = ilv[a];                    // first group of the block
  const int* T = ilv + ilv[G + a];         // K, then C(0..K)
  const int K = T[0];
  const int* C = T + 1;
  const int local = idx - groups[f].base;
  if (local < 0 || local >= C[K]) return;
  // rank k of every group of the block with more than k items, k = 0, 1, ...
  int lo = 0, hi = K;  // C[lo] <= local < C[hi]; C increases strictly
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (C[mid] <= local) lo = mid; else hi = mid;
  }
  *k = lo;
  *ga = f + (local - C[lo]);
}

// Work list of a candidates-only plan (blocks of 1024 threads over the
// launch slots).  With at least kSplitTarget / 2 active items the list
// mirrors the schedule (whole items, kend = -1).  With fewer, block 0 builds
// it alone from the active slots the CSR kernel collected: they are put
// back in slot order (rank by slot), and an item whose CSR holds n key tiles
// is cut into c = ceil(n / C) chunks of equal length (to one tile), where
// C = max(kSplitMinChunk, ceil(total tiles / kSplitTarget)).  Then sum(c) <=
// target + items < 1.5 * target entries, and the parts of split items number
// fewer than kMaxParts.  Slots past the last entry, and split slots past the
// last split item, get item -1.
__global__ __launch_bounds__(1024) void plan_work_kernel(PlanDev P, int slots, int grid, int H) {
  constexpr int kMaxAct = kSplitTarget / 2;
  constexpr int kHead = 2 * kSplitTarget;  // block 0 owns slots [0, kHead) when splitting
  __shared__ int smem[32];
  __shared__ long long tiles_sh[16];
  __shared__ int s_slot[kMaxAct], s_item[kMaxAct], s_n[kMaxAct];
  __shared__ int s_c[kMaxAct], s_w[kMaxAct], s_p[kMaxAct];  // chunks, first entry, first part
  const int t = threadIdx.x;
  const int n_act = P.totals->n_act;
  const bool split = n_act < kMaxAct;
  if (!split) {
    const int s = blockIdx.x * blockDim.x + t;
    if (s < grid && s >= slots) {  // slots below: the CSR kernel wrote their records
      P.work[s] = WorkEntry{-1, 0, 0, -1};
      P.irec[s] = no_item_rec();
    } else if (s < slots) {
      P.work[s] = WorkEntry{P.sched[s], 0, -1, -1};
    }
    if (blockIdx.x == 0) {
      for (int k = t; k < kSplitTarget; k += blockDim.x) P.splits[k] = SplitEntry{-1, 0, 0, 0};
      if (t == 0) {
        P.totals->n_work = slots;
        P.totals->n_splits = 0;
      }
    }
    return;
  }
  if (blockIdx.x > 0) {
    const int s = blockIdx.x * blockDim.x + t;
    if (s >= kHead && s < grid) {
      P.work[s] = WorkEntry{-1, 0, 0, -1};
      P.irec[s] = no_item_rec();
    }
    return;
  }
  int slot = 0x7fffffff, item = -1, n = 0;
  if (t < n_act) {
    slot = P.act_slots[t];
    item = P.sched[slot];
    const int qg = item / H;
    n = P.qtile_ptr[qg + 1] - P.qtile_ptr[qg];
    s_slot[t] = slot;
  }
  long long v = n;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((t & 63) == 0) tiles_sh[t >> 6] = v;
  __syncthreads();
  long long total_tiles = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total_tiles += tiles_sh[w];
  if (t < n_act) {
    int r = 0;
    for (int u = 0; u < n_act; ++u) r += s_slot[u] < slot;
    s_item[r] = item;
    s_n[r] = n;
  }
  __syncthreads();
  if (t < n_act) {
    item = s_item[t];
    n = s_n[t];
  }
  const long long cl = (total_tiles + kSplitTarget - 1) / kSplitTarget;
  const int C = (int)max((long long)kSplitMinChunk, cl);
  const int c = t < n_act ? max(1, (n + C - 1) / C) : 0;
  int w_tot, p_tot, s_tot;
  const int w = block_exclusive_scan(c, smem, &w_tot);
  const int part = block_exclusive_scan(c > 1 ? c : 0, smem, &p_tot);
  const int sp = block_exclusive_scan(c > 1 ? 1 : 0, smem, &s_tot);
  if (c > 1) P.splits[sp] = SplitEntry{item, part, c, 0};
  if (t < n_act) {
    s_c[t] = c;
    s_w[t] = w;
    s_p[t] = c > 1 ? part : -1;
  }
  __syncthreads();
  // entry e of the list: chunk e - s_w[i] of the last item i with s_w[i] <=
  // e; one entry per thread, so their records' loads go out together.
  // Chunk lengths differ by at most one and none is empty (c <= n).
  for (int e = t; e < w_tot; e += blockDim.x) {
    int a = 0, b = n_act - 1;
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (s_w[mid] <= e) a = mid; else b = mid - 1;
    }
    const int j = e - s_w[a], ci = s_c[a], ni = s_n[a], it = s_item[a];
    const int kb = (int)((long long)j * ni / ci), ke = (int)((long long)(j + 1) * ni / ci);
    const int pi = ci > 1 ? s_p[a] + j : -1;
    P.irec[e] = item_rec(P, it, kb, ke, pi, H);
    P.work[e] = WorkEntry{it, kb, ke, pi};
  }
  for (int s = w_tot + t; s < min(grid, kHead); s += blockDim.x) {
    P.work[s] = WorkEntry{-1, 0, 0, -1};
    P.irec[s] = no_item_rec();
  }
  for (int k = s_tot + t; k < kSplitTarget; k += blockDim.x) P.splits[k] = SplitEntry{-1, 0, 0, 0};
  if (t == 0) {
    P.totals->n_work = w_tot;
    P.totals->n_splits = s_tot;
  }
}

// ---- key-major tables (backward) -------------------------------------

// Key block kb of a request covers k-tiles 2 kb and 2 kb + 1 (the second
// may not exist).  A q-tile has a visible pair in the block when it has one
// in either k-tile; the entry is FULL only when both k-tiles exist and are
// FULL (every other block entry gets the per-element mask).
__device__ __forceinline__ bool kblock_nonempty(const PlanDev& P, const ReqMeta& m, int qt,
                                                int kb) {
  const int64_t row = m.tile_off + (int64_t)qt * m.nkt;
  const int k0 = 2 * kb, k1 = 2 * kb + 1;
  return P.tile_count[row + k0] > 0 || (k1 < m.nkt && P.tile_count[row + k1] > 0);
}
__device__ __forceinline__ bool kblock_full(const PlanDev& P, const ReqMeta& m, int qt, int kb) {
  const int64_t row = m.tile_off + (int64_t)qt * m.nkt;
  const int k0 = 2 * kb, k1 = 2 * kb + 1;
  return k1 < m.nkt && P.tile_class[row + k0] == RK_TILE_FULL &&
         P.tile_class[row + k1] == RK_TILE_FULL;
}

// One block per global key block: number of q-tiles with a visible pair in it.
__global__ __launch_bounds__(256) void plan_kcount_kernel(PlanDev P) {
  __shared__ int cnt_s;
  const int g = blockIdx.x;
  const ReqMeta m = P.req[P.kt_req[g]];
  const int kb = g - m.kt_off;
  if (threadIdx.x == 0) cnt_s = 0;
  __syncthreads();
  int c = 0;
  for (int qt = threadIdx.x; qt < m.nqt; qt += blockDim.x) c += kblock_nonempty(P, m, qt, kb);
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) atomicAdd(&cnt_s, c);
  __syncthreads();
  if (threadIdx.x == 0) P.kt_nnz[g] = cnt_s;
}

// Single block: kt_ptr = exclusive scan of kt_nnz.
__global__ __launch_bounds__(1024) void plan_kscan_kernel(PlanDev P, int NK) {
  __shared__ int smem[32];
  int carry = 0;
  for (int base = 0; base < NK; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const int v = i < NK ? P.kt_nnz[i] : 0;
    int total;
    const int ex = block_exclusive_scan(v, smem, &total);
    if (i < NK) P.kt_ptr[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) P.kt_ptr[NK] = carry;
}

// One block per key block: ascending list of its non-empty q-tiles, with
// the PARTIAL bit.
__global__ __launch_bounds__(256) void plan_kfill_kernel(PlanDev P) {
  __shared__ int smem[32];
  const int g = blockIdx.x;
  const ReqMeta m = P.req[P.kt_req[g]];
  const int kb = g - m.kt_off;
  const int base = P.kt_ptr[g];
  int run = 0;
  for (int q0 = 0; q0 < m.nqt; q0 += blockDim.x) {
    const int qt = q0 + threadIdx.x;
    const int flag = qt < m.nqt && kblock_nonempty(P, m, qt, kb);
    int total;
    const int ex = block_exclusive_scan(flag, smem, &total);
    if (flag)
      P.qtile_word[base + run + ex] =
          (int)((unsigned)qt | ((unsigned)(!kblock_full(P, m, qt, kb)) << 31));
    run += total;
  }
}

// One block per request: key blocks by descending non-empty q-tile count.
__global__ __launch_bounds__(256) void plan_ksort_kernel(PlanDev P) {
  __shared__ __attribute__((aligned(16))) int chunk[1024];
  const ReqMeta m = P.req[blockIdx.x];
  rank_order(m.nqt, m.kt_off, P.kt_nnz + m.kt_off, P.korder, chunk);
}

// One thread per key-major launch slot (same XCD mapping as the query-major
// schedule): item = global k-tile * H + head, or -1.
__global__ void plan_ksched_kernel(PlanDev P, int64_t slots, int H, int G) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= slots) return;
  int ga = -1, k = -1;
  slot_of(P.kgroups, P.kqueue_start, P.kilv, G, (int)(s % kNumXcd), (int)(s / kNumXcd), &ga,
          &k);
  int item = -1;
  if (ga >= 0) {
    const Group grp = P.kgroups[ga];
    if (k >= 0 && k < grp.count) {
      const ReqMeta m = P.req[grp.req];
      item = P.korder[m.kt_off + k] * H + grp.head;
    }
  }
  P.ksched[s] = item;
}

}  // namespace

hipError_t launch_plan(const rk_plan* p, const unsigned char* staged, unsigned* stage_done,
                       hipStream_t s) {
  const PlanDev& P = p->dev;
  PlanSource src{};
  if (staged) {
    // the first kernel reads the request records and q-tile table from the
    // host block and copies the rest of the host tables into the workspace
    src.req = reinterpret_cast<const ReqMeta*>(staged + p->off_req);
    src.qt_req = reinterpret_cast<const int32_t*>(staged + p->off_qt_req);
    src.blob = reinterpret_cast<const uint4*>(staged);
    src.dst = reinterpret_cast<uint4*>(p->workspace);
    src.lo16 = (int64_t)(p->off_qt_req / 16);
    src.hi16 = (int64_t)(p->host_blob_bytes / 16);
    src.R = p->R;
  } else {
    src.req = P.req;
    src.qt_req = P.qt_req;
  }
  const bool cand_only = (p->flags & RK_QUERY_CANDIDATES_ONLY) != 0;
  if (p->NQ > 0) {
    // one block per global q-tile (NQ > 0 whenever T > 0)
    const int check_static = (!(p->flags & RK_STATIC_BIDIRECTIONAL)) && p->delay > 0;
    hipLaunchKernelGGL(plan_rows_tiles_kernel, dim3((unsigned)p->NQ), dim3(256), 0, s, P, src,
                       p->seg_kind_dev, p->timestamps_dev, (int64_t)p->T, p->delay, p->window,
                       p->global_tail,
                       (int)((p->flags & RK_STATIC_BIDIRECTIONAL) != 0), check_static,
                       (int)p->slots);
  }
  // blocks 0 .. NQ - 1 per q-tile, block NQ the totals (zero tiles: totals only)
  hipLaunchKernelGGL(plan_csr_sched_kernel, dim3((unsigned)(p->NQ + 1)), dim3(256), 0, s, P,
                     (int)p->NQ, p->NT, p->H, (int)p->G, cand_only ? 2 : 1, stage_done);
  if (cand_only && p->slots > 0 && p->grid > p->slots)
    hipLaunchKernelGGL(plan_work_kernel, dim3((unsigned)((p->grid + 1023) / 1024)), dim3(1024), 0,
                       s, P, (int)p->slots, (int)p->grid, p->H);
  if ((p->flags & RK_PLAN_BACKWARD) && p->NK > 0) {
    hipLaunchKernelGGL(plan_kcount_kernel, dim3((unsigned)p->NK), dim3(256), 0, s, P);
    hipLaunchKernelGGL(plan_kscan_kernel, dim3(1), dim3(1024), 0, s, P, (int)p->NK);
    hipLaunchKernelGGL(plan_kfill_kernel, dim3((unsigned)p->NK), dim3(256), 0, s, P);
    hipLaunchKernelGGL(plan_ksort_kernel, dim3(p->R), dim3(256), 0, s, P);
    hipLaunchKernelGGL(plan_ksched_kernel, dim3((unsigned)((p->kslots + 255) / 256)), dim3(256), 0,
                       s, P, p->kslots, p->H, (int)p->G);
  }
  return hipGetLastError();
}

}  // namespace rk
