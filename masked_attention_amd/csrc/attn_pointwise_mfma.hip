// HSTU pointwise aggregated attention (HSTU eq. 2), bf16, d_head = 64,
// CDNA4 MFMA:
//   O_i = sum over visible j of SiLU(scale q_i . k_j + rab_ij) v_j,
//   rab_ij = pos_bias[min(|p_i - p_j|, np - 1)]
//          + time_bias[min(floor(log2(1 + |t_i - t_j|)), nt - 1)],
// over the same plan (row descriptors, CSR of non-empty key tiles, launch
// schedule) as the softmax forward.  No normalisation and no running max:
// each key tile adds its weighted values to O directly.
//
// Work item = (query tile of 128 rows, head); 4 waves of 32 rows, one query
// per lane, the transposed products of the softmax kernel:
//   Y^T (64 keys x 32 queries) = K Q'^T + C    8 x mfma 32x32x16
//   W' = Y / (1 + 2^Y) (+ rab in Y units), masked keys 0, packed to bf16
//   O^T (64 d x 32 queries) += V^T W'^T        8 x mfma
// in units where Y = -log2(e) x for x = scale q . k (+ rab): Q' carries
// -scale * log2(e) and the bias tables -log2(e), so that SiLU(x) =
// x / (1 + e^-x) = -ln2 * Y / (1 + 2^Y) costs one exp2, one add, one
// reciprocal and one multiply per score; the -ln2 is applied to O at the
// end.
// The relative bias.  Both buckets are monotone in |p_i - p_j| and
// |t_i - t_j|, so for one row over one key tile the bias is constant when
// the bucket at both ends of the tile's position and time ranges is the
// same and the ranges do not cross zero; the time range is the min / max
// of the tile's key timestamps (one wave reduction per tile).  When that
// holds for every lane of the wave, the constant enters the QK^T product
// as its initial accumulator (C = the bias in Y units) and costs nothing
// per score; otherwise (tiles near the diagonal or across a bucket edge) the
// wave evaluates the bias per score from the tables in LDS.
#include "cdna4_common.h"

namespace rk {
namespace {

using namespace cdna4;

constexpr int D = 64;
constexpr int kThreads = 256;
constexpr int TILE_ELEMS = kTileK * D;  // 64 rows x 64 bf16 = 8 KB
constexpr int kMaxPos = 4096;
constexpr int kMaxTime = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct PwView {
  const ReqMeta* req;
  const int32_t* qt_req;
  const int2* row_desc;
  const int32_t* qtile_ptr;
  const int32_t* ktile_word;
  const int32_t* sched;
  const unsigned* info;  // plan info word (kInfoHistoryUnsorted)
};

// LDS K / V tiles: 64 rows of 128 bytes, 16-byte chunk c of row r in slot
// c ^ kswz(r) (K) or c ^ vswz(r) (V).  gfx950's LDS has 64 four-byte banks,
// two rows per bank line, and serves a K row read 16 lanes (rows) at a
// time: even and odd rows each need 8 distinct slots, kswz(r) = (r / 2)
// mod 8.  A V transposing read (4 consecutive rows from a multiple of 4,
// 4 chunks over 32 lanes) takes 16 distinct bank groups with vswz.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }

// floor(log2(1 + |dt|)) capped at nt - 1
__device__ __forceinline__ int time_bucket(int64_t dt, int nt) {
  const uint64_t x = 1ull + (uint64_t)(dt < 0 ? -dt : dt);
  return min(63 - __clzll((long long)x), nt - 1);
}

__device__ __forceinline__ int64_t wave_min64(int64_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_xor(v, o, 64);
    v = u < v ? u : v;
  }
  return v;
}
__device__ __forceinline__ int64_t wave_max64(int64_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_xor(v, o, 64);
    v = u > v ? u : v;
  }
  return v;
}

struct Tabs {
  float pos[kMaxPos];
  float time[kMaxTime];
};

// W' = Y / (1 + 2^Y) (Y = the scaled score in -log2(e) units, + rab in the
// same units) packed to bf16 as the B operands of the PV
// product (step s: accumulator block s / 2, registers 8 (s % 2) .. +7).
// Register r of block mb holds key c0 + 32 mb + 8 (r / 4) + 4 hh + r % 4.
// kBias: the bias varies over the tile and is read from the tables per
// score (otherwise it is constant and already in the accumulator);
// kPartial: masked keys get W = 0 (visible-key bits w0 / w1, shifted by
// 4 hh).
template <bool kBias, bool kPartial>
__device__ __forceinline__ void pw_weights(bf16x8 (&pb)[4], const f32x16& s0, const f32x16& s1,
                                           int w0, int w1, const int64_t* tk,
                                           const Tabs& tab, int c0, int hh, int row, int64_t ti,
                                           const PwLaunch& A, bool has_pos, bool has_time) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int mb = s >> 1;
    const f32x16& src = mb ? s1 : s0;
    const int r0 = 8 * (s & 1);
    bf16x2_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = r0 + 2 * j + e;
        float x = src[r];
        if (kBias) {
          const int kk = 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);  // key offset in the tile
          if (has_pos) {
            const int dp = row - (c0 + kk);
            x += tab.pos[min(dp < 0 ? -dp : dp, A.np - 1)];
          }
          if (has_time) x += tab.time[time_bucket(ti - tk[kk], A.nt)];
        }
        float wv = x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x));
        if (kPartial) {
          const unsigned bit = 8u * (unsigned)(r >> 2) + (unsigned)(r & 3);
          const int m = __builtin_amdgcn_sbfe(mb ? w1 : w0, bit, 1u);  // 0 or -1
          wv = __int_as_float(__float_as_int(wv) & m);
        }
        w[j][e] = (__bf16)wv;
      }
    }
    __builtin_memcpy(&pb[s], w, 16);
  }
}

// One key tile for one wave.  seg_sorted: the tile's keys all lie in one
// segment whose timestamps are non-decreasing (REALTIME, or HISTORY when
// the planner found every history in time order), so their time range is
// given by the first and the last key.
__device__ __forceinline__ void pw_tile(f32x16& o0, f32x16& o1, const unsigned short* kb,
                                        const unsigned short* vb, const int64_t* tk,
                                        const Tabs& tab, const bf16x8 (&q)[4], int kt, bool partial,
                                        int L, int li, int hh, int lo, int hi, int self, int row,
                                        int64_t ti, const PwLaunch& A, bool has_pos,
                                        bool has_time, const ReqMeta& m, bool hist_sorted) {
  const int c0 = kt * kTileK;
  const int nr = min(L - c0, kTileK);  // keys of the tile inside the request
  // ---- is the bias constant over this tile for the lane's row?
  bool fast = true;
  float cb = 0.f;
  if (has_pos) {
    const int dlo = row - (c0 + nr - 1), dhi = row - c0;  // p_i - p_j over the tile
    if (dlo >= A.np - 1 || dhi <= -(A.np - 1)) cb += tab.pos[A.np - 1];
    else fast = false;
  }
  if (has_time) {
    const int c1 = c0 + nr;
    const bool seg_sorted =
        (hist_sorted && c0 >= m.seg[RK_SEG_HISTORY] && c1 <= m.seg[RK_SEG_REALTIME]) ||
                            (c0 >= m.seg[RK_SEG_REALTIME] && c1 <= m.seg[RK_SEG_CANDIDATE]);
    int64_t tmin, tmax;
    if (seg_sorted) {
      tmin = tk[0];
      tmax = tk[nr - 1];
    } else {
      const int lane = threadIdx.x & 63;
      const int64_t t = tk[lane];
      tmin = wave_min64(lane < nr ? t : INT64_MAX);
      tmax = wave_max64(lane < nr ? t : INT64_MIN);
    }
    const int64_t a = ti - tmax, b = ti - tmin;  // t_i - t_j over the tile
    if (a >= 0 || b <= 0) {
      const int b1 = time_bucket(a, A.nt), b2 = time_bucket(b, A.nt);
      if (b1 == b2) cb += tab.time[b1];
      else fast = false;
    } else {
      fast = false;
    }
  }
  const bool uniform = !__any(!fast);
  const float init = uniform ? cb : 0.f;

  // ---- S^T = K Q^T + C
  f32x16 s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { s0[r] = init; s1[r] = init; }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cc = 2 * s + hh;
    const bf16x8 k0 = as_bf16x8(*(const uint4*)&kb[li * 64 + 8 * (cc ^ kswz(li))]);
    const bf16x8 k1 = as_bf16x8(*(const uint4*)&kb[(32 + li) * 64 + 8 * (cc ^ kswz(32 + li))]);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q[s], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, q[s], s1, 0, 0, 0);
  }

  // ---- W' = Y / (1 + 2^Y) (+ rab), masked keys 0; one code path per
  // (bias per score, mask) case, chosen per tile and wave
  bf16x8 pb[4];
  int w0 = -1, w1 = -1;
  if (partial) {
    const uint64_t vis = tile_vis_bits(c0, lo, hi, self, row) >> (4 * hh);
    w0 = (int)(unsigned)vis;
    w1 = (int)(unsigned)(vis >> 32);
  }
  if (uniform) {
    if (partial)
      pw_weights<false, true>(pb, s0, s1, w0, w1, tk, tab, c0, hh, row, ti, A, has_pos,
                              has_time);
    else
      pw_weights<false, false>(pb, s0, s1, w0, w1, tk, tab, c0, hh, row, ti, A, has_pos,
                               has_time);
  } else {
    if (partial)
      pw_weights<true, true>(pb, s0, s1, w0, w1, tk, tab, c0, hh, row, ti, A, has_pos,
                             has_time);
    else
      pw_weights<true, false>(pb, s0, s1, w0, w1, tk, tab, c0, hh, row, ti, A, has_pos,
                              has_time);
  }

  // ---- O^T += V^T W^T (V^T by transposing reads, keys in register order)
  const int g = (li >> 4) + 2 * hh;
  const int i = li & 15;
  const int rr = i >> 2;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int d0 = 32 * mb + 16 * (g & 1);
      const int col = d0 + 4 * (i & 3);
      const int ka = 16 * s + 4 * hh + rr;
      const int kb2 = ka + 8;
      const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          RK_LDS_PTR(v4i16, &vb[ka * 64 + 8 * ((col >> 3) ^ vswz(ka)) + (col & 7)]));
      const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          RK_LDS_PTR(v4i16, &vb[kb2 * 64 + 8 * ((col >> 3) ^ vswz(kb2)) + (col & 7)]));
      bf16x8 va;
      __builtin_memcpy(&va, &lo4, 8);
      __builtin_memcpy((char*)&va + 8, &hi4, 8);
      if (mb == 0)
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], o0, 0, 0, 0);
      else
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], o1, 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kThreads, 3) void pw_mfma_bf16_d64_kernel(PwView P, PwLaunch A) {
  __shared__ __attribute__((aligned(1024))) unsigned short K0[TILE_ELEMS], K1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) unsigned short V0[TILE_ELEMS], V1[TILE_ELEMS];
  // key timestamps of each stage: 64 used; dword copies of 256 bytes fill
  // [0, 512) and read out of range (zeros) past the request's end
  __shared__ __attribute__((aligned(16))) int64_t T0[kTileK], T1[kTileK];
  __shared__ Tabs tab;

  const int item = ldc(P.sched, blockIdx.x);
  if (item < 0) return;
  const float pz = plan_poison(A.plan_err);
  const int qg = item / A.H;
  const int head = item - qg * A.H;
  const int req = ldc(P.qt_req, qg);
  const ReqMeta m = ldc(P.req, req);
  const int qt = qg - m.qt_off;
  const int L = m.len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int li = lane & 31;
  const int row = qt * kTileQ + wv * 32 + li;
  const bool rvalid = row < L;
  const int tokq = m.tok_off + row;
  const int tokc = m.tok_off + min(row, L - 1);

  // the row: Q fragments (d = 16 s + 8 hh .. +7), time, descriptor
  const unsigned short* Qp = (const unsigned short*)A.q + (int64_t)tokc * A.q_st + (int64_t)head * A.q_sh;
  bf16x8 q[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 u = *(const uint4*)(Qp + 16 * s + 8 * hh);
    q[s] = as_bf16x8(rvalid ? u : make_uint4(0, 0, 0, 0));
  }
  const int64_t ti = A.ts[tokc];
  const int2 dsc = P.row_desc[tokc];
  const int lo = rvalid ? dsc.x : 0;
  const int hi = rvalid ? dsc.y & 0x7fffffff : 0;
  const int self = rvalid && dsc.y < 0;
  const bool has_pos = A.pos_bias != nullptr, has_time = A.time_bias != nullptr;
  const bool hist_sorted = !(ldc(P.info, 0) & kInfoHistoryUnsorted);
  // scores and biases in -log2(e) units (the -ln2 goes onto O at the end)
  for (int x = tid; x < A.np && has_pos; x += kThreads) tab.pos[x] = -kLog2e * A.pos_bias[x];
  for (int x = tid; x < A.nt && has_time; x += kThreads) tab.time[x] = -kLog2e * A.time_bias[x];
#pragma unroll
  for (int s = 0; s < 4; ++s) q[s] = scale_bf16x8(q[s], -kLog2e * A.scale);

  const char* Kb = (const char*)((const unsigned short*)A.k + (int64_t)m.tok_off * A.k_st + (int64_t)head * A.k_sh);
  const char* Vb = (const char*)((const unsigned short*)A.v + (int64_t)m.tok_off * A.v_st + (int64_t)head * A.v_sh);
  const char* Tb = (const char*)(A.ts + m.tok_off);
  const unsigned kst_b = (unsigned)A.k_st * 2u, vst_b = (unsigned)A.v_st * 2u;
  unsigned koff[2], voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qq = (2 * wv + j) * 64 + lane;
    const int r = qq >> 3, slot = qq & 7;
    koff[j] = (unsigned)r * kst_b + 16u * (unsigned)(slot ^ kswz(r));
    voff[j] = (unsigned)r * vst_b + 16u * (unsigned)(slot ^ vswz(r));
  }
  // Each wave zeroes the K and V rows its own copies fill in both stages:
  // any byte a copy leaves unwritten stays finite.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int o = (2 * wv + j) * 512 + 8 * lane;
    *(uint4*)&K0[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&K1[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&V0[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&V1[o] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  auto issue = [&](unsigned short* kd, unsigned short* vd, int64_t* td, int kt) {
    const int c0 = kt * kTileK;
    const unsigned last = (unsigned)min(L - c0, kTileK) - 1u;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kb + (int64_t)c0 * kst_b), 0, (int)(last * kst_b + 2u * D), (int)kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vb + (int64_t)c0 * vst_b), 0, (int)(last * vst_b + 2u * D), (int)kBufferFlags);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, RK_LDS_PTR(void, kd + (2 * wv + j) * 512), 16,
                                               koff[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, RK_LDS_PTR(void, vd + (2 * wv + j) * 512), 16,
                                               voff[j], 0, 0, 0);
    }
    if (wv == 0) {
      const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(Tb + 8 * (int64_t)c0), 0, (int)(8u * (last + 1u)), (int)kBufferFlags);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tr, RK_LDS_PTR(void, (char*)td + 256 * j), 4,
                                                 256u * j + 4u * lane, 0, 0, 0);
    }
  };

  f32x16 o0, o1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { o0[r] = 0.f; o1[r] = 0.f; }

  const int e0 = ldc(P.qtile_ptr, qg);
  const int n = ldc(P.qtile_ptr, qg + 1) - e0;
  int w_cur = n > 0 ? ldc(P.ktile_word, e0) : 0;
  issue(K0, V0, T0, w_cur & 0x7fffffff);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < n; it += 2) {
    {
      const int w_nxt = ldc(P.ktile_word, e0 + min(it + 1, n - 1));
      issue(K1, V1, T1, w_nxt & 0x7fffffff);
      pw_tile(o0, o1, K0, V0, T0, tab, q, w_cur & 0x7fffffff, w_cur < 0, L, li, hh, lo, hi,
              self, row, ti, A, has_pos, has_time, m, hist_sorted);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      w_cur = w_nxt;
    }
    if (it + 1 < n) {
      const int w_nxt = ldc(P.ktile_word, e0 + min(it + 2, n - 1));
      issue(K0, V0, T0, w_nxt & 0x7fffffff);
      pw_tile(o0, o1, K1, V1, T1, tab, q, w_cur & 0x7fffffff, w_cur < 0, L, li, hh, lo, hi,
              self, row, ti, A, has_pos, has_time, m, hist_sorted);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      w_cur = w_nxt;
    }
  }

  if (!rvalid) return;
  const float oscale = -0.6931471805599453f * pz;  // -ln2
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    o0[r] *= oscale;
    o1[r] *= oscale;
  }
  unsigned short* Op = (unsigned short*)A.o + (int64_t)tokq * A.o_st + (int64_t)head * A.o_sh;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int d = 8 * g + 4 * hh;
    *(uint2*)(Op + d) = make_uint2(pack_bf16x2(o0[4 * g], o0[4 * g + 1]),
                                   pack_bf16x2(o0[4 * g + 2], o0[4 * g + 3]));
    *(uint2*)(Op + 32 + d) = make_uint2(pack_bf16x2(o1[4 * g], o1[4 * g + 1]),
                                        pack_bf16x2(o1[4 * g + 2], o1[4 * g + 3]));
  }
}

}  // namespace

hipError_t launch_pointwise_mfma_bf16_d64(const rk_plan* p, const PwLaunch& a, hipStream_t s) {
  if (p->slots == 0) return hipSuccess;
  PwView P{p->dev.req, p->dev.qt_req, p->dev.row_desc, p->dev.qtile_ptr, p->dev.ktile_word,
           p->dev.sched, &p->dev.totals->info};
  hipLaunchKernelGGL(pw_mfma_bf16_d64_kernel, dim3((unsigned)p->slots), dim3(kThreads), 0, s, P,
                     a);
  return hipGetLastError();
}

}  // namespace rk
