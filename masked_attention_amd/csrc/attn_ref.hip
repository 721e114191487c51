// Plain masked-attention forward over the tile plan (no matrix cores).
//
// One 128-thread workgroup per (query tile, head) work item, one thread per
// query row.  K and V tiles of 64 keys are staged in LDS as fp32; every
// thread computes its 64 scores, applies the per-element mask on PARTIAL
// tiles only, and keeps an fp32 online softmax (running max m, sum l) and
// output accumulator.  Serves the fp32 path (exact to fp32 rounding), bf16
// with d_head other than 64, and a cross-check of the MFMA kernel.  The
// instance width D is d_head rounded up to 32, 64 or 128; columns past
// d_head are zero and never touch memory.
//
// Visibility of key c for query row p (request-local): c in [lo, hi), or
// c == p when the row is a candidate (bit 31 of hi), from the plan's row
// descriptors.  A row with no visible key writes 0 and lse = -inf.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __hip_bfloat16* p) {
  return __uint_as_float(((unsigned)(*(const unsigned short*)p)) << 16);
}
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(__hip_bfloat16* p, float v) {
  unsigned u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  *(unsigned short*)p = (unsigned short)(u >> 16);
}

struct PlanView {
  const ReqMeta* req;
  const int32_t* qt_req;
  const int2* row_desc;
  const int32_t* qtile_ptr;
  const int32_t* ktile_word;
  const int32_t* sched;
  const WorkEntry* work;  // launch slot -> (item, CSR range, part), or null
};

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_ref_kernel(PlanView P, AttnLaunch A) {
  __shared__ float Ks[kTileK][D];
  __shared__ float Vs[kTileK][D];
  __shared__ double w[kMaxHalfD];
  int item, kbeg = 0, kend = -1, part = -1;
  if (P.work) {
    const WorkEntry we = P.work[blockIdx.x];
    item = we.item;
    kbeg = we.kbeg;
    kend = we.kend;
    part = we.part;
  } else {
    item = P.sched[blockIdx.x];
  }
  if (item < 0) return;
  const int qg = item / A.H;
  const int head = item - qg * A.H;
  const ReqMeta m = P.req[P.qt_req[qg]];
  const int qt = qg - m.qt_off;
  const int L = m.len;
  const int t = threadIdx.x;
  const int p = qt * kTileQ + t;
  const bool valid = p < L;
  const int tok = m.tok_off + p;
  if (A.rope_q && t < D / 2) w[t] = A.tab.w_rev[t];
  __syncthreads();

  const T* Q = (const T*)A.q;
  const T* K = (const T*)A.k;
  const T* V = (const T*)A.v;
  float q[D];
#pragma unroll
  for (int c = 0; c < D; ++c)
    q[c] = valid && c < A.d ? ld(Q + (int64_t)tok * A.q_st + (int64_t)head * A.q_sh + c) : 0.f;
  if (A.norm_q && valid) {
    // QK Norm before the rotation
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) ss = fmaf(q[c], q[c], ss);
    const float rstd = rsqrtf(ss / (float)A.d + A.eps);
#pragma unroll
    for (int c = 0; c < D; ++c) q[c] *= rstd * (A.gamma_q && c < A.d ? A.gamma_q[c] : 1.f);
  }
  if (A.rope_q && valid) {
    const int64_t dt = A.ts[tok] - A.anchors[P.qt_req[qg]];
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const double rev = (double)dt * w[i];
      const float f = (float)(rev - rint(rev));
      float sn, cs;
      sincosf(6.283185307179586f * f, &sn, &cs);
      const float x0 = q[2 * i], x1 = q[2 * i + 1];
      q[2 * i] = x0 * cs - x1 * sn;
      q[2 * i + 1] = x0 * sn + x1 * cs;
    }
  }
  int lo = 0, hi = 0, self = 0;
  if (valid) {
    const int2 dsc = P.row_desc[tok];
    lo = dsc.x;
    hi = dsc.y & 0x7fffffff;
    self = dsc.y < 0;
  }

  float mrow = -INFINITY, lsum = 0.f;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;

  const int e0 = P.qtile_ptr[qg] + kbeg;
  const int e1 = kend >= 0 ? P.qtile_ptr[qg] + kend : P.qtile_ptr[qg + 1];
  for (int e = e0; e < e1; ++e) {
    const int kw = P.ktile_word[e];
    const int kt = kw & 0x7fffffff;
    const bool partial = kw < 0;
    __syncthreads();
    for (int x = t; x < kTileK * D; x += blockDim.x) {
      const int j = x / D, c = x - j * D;
      const int key = kt * kTileK + j;
      const bool in = key < L && c < A.d;
      const int64_t kk = (int64_t)(m.tok_off + key);
      Ks[j][c] = in ? ld(K + kk * A.k_st + (int64_t)head * A.k_sh + c) : 0.f;
      Vs[j][c] = in ? ld(V + kk * A.v_st + (int64_t)head * A.v_sh + c) : 0.f;
    }
    __syncthreads();
    float s[kTileK];
    float mx = -INFINITY;
    for (int j = 0; j < kTileK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(q[c], Ks[j][c], dot);
      float v = dot * A.scale;
      if (partial) {
        const int key = kt * kTileK + j;
        const bool vis = (key >= lo && key < hi) || (self && key == p);
        if (!vis) v = -INFINITY;
      }
      s[j] = v;
      mx = fmaxf(mx, v);
    }
    const float mnew = fmaxf(mrow, mx);
    if (mnew == -INFINITY) continue;  // nothing visible to this row yet
    const float alpha = expf(mrow - mnew);  // 0 when mrow == -inf
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
    for (int j = 0; j < kTileK; ++j) {
      const float pj = expf(s[j] - mnew);
      lsum += pj;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(pj, Vs[j][c], acc[c]);
    }
    mrow = mnew;
  }

  if (!valid) return;
  if (part >= 0) {
    // partial result of a split item: O unnormalised, running max, sum
    float* pp = A.part + (int64_t)part * (kTileQ * (D + 2));
#pragma unroll
    for (int c = 0; c < D; ++c) pp[t * D + c] = acc[c];
    pp[kTileQ * D + t] = mrow;
    pp[kTileQ * D + kTileQ + t] = lsum;
    return;
  }
  T* O = (T*)A.o;
  const float pz = plan_poison(A.plan_err);
  const float inv = (lsum > 0.f ? 1.f / lsum : 0.f) * pz;
#pragma unroll
  for (int c = 0; c < D; ++c)
    if (c < A.d) st(O + (int64_t)tok * A.o_st + (int64_t)head * A.o_sh + c, acc[c] * inv);
  if (A.lse) A.lse[(int64_t)head * A.T + tok] = (lsum > 0.f ? mrow + logf(lsum) : -INFINITY) * pz;
}

template <typename T, int D>
hipError_t launch_ref(const rk_plan* p, const AttnLaunch& a, hipStream_t s) {
  const bool wl = p->grid > p->slots;
  PlanView P{p->dev.req, p->dev.qt_req, p->dev.row_desc, p->dev.qtile_ptr, p->dev.ktile_word,
             p->dev.sched, wl ? p->dev.work : nullptr};
  hipLaunchKernelGGL((attn_ref_kernel<T, D>), dim3((unsigned)p->grid), dim3(128), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_reference(const rk_plan* p, const AttnLaunch& a, rk_dtype dt, hipStream_t s) {
  if (p->slots == 0) return hipSuccess;
  if (a.d > a.dp) return hipErrorInvalidValue;
  if (dt == RK_F32) {
    if (a.dp == 32) return launch_ref<float, 32>(p, a, s);
    if (a.dp == 64) return launch_ref<float, 64>(p, a, s);
    if (a.dp == 128) return launch_ref<float, 128>(p, a, s);
  } else {
    if (a.dp == 32) return launch_ref<__hip_bfloat16, 32>(p, a, s);
    if (a.dp == 64) return launch_ref<__hip_bfloat16, 64>(p, a, s);
    if (a.dp == 128) return launch_ref<__hip_bfloat16, 128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rk
