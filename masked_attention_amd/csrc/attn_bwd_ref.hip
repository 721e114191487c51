// Plain masked-attention backward over the tile plan (no matrix cores).
//
// Gradients of a loss with respect to Q, K, V given dO, for the forward
// softmax(Q K^T * scale + M) V (TM20K section 2.1; LazFormer eq. 21).  With
// P recomputed from the forward's log-sum-exp:
//   dV = P^T dO,  dS = P * (dO V^T - D),  D_i = dO_i . O_i,
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// Two launches, no atomics:
//   dq kernel   : one 128-thread workgroup per (query tile, head) of the
//                 query-major schedule, one thread per query row; walks the
//                 row's non-empty key tiles (K, V staged in LDS as fp32);
//                 also writes D and the log-sum-exp in log2 units for the
//                 second launch;
//   dkdv kernel : one 128-thread workgroup per (key block of 128 keys,
//                 head) of the key-major schedule, one thread per key; walks
//                 the block's non-empty query tiles in chunks of 32 rows (Q, dO,
//                 log-sum-exp, D and row descriptors staged in LDS).
// The per-element mask (visible interval [lo, hi) plus the candidate self
// link, from the plan's row descriptors) runs on PARTIAL tiles only.  With
// time RoPE, Q and K arrive rotated; dQ and dK are taken back through the
// rotation (the transpose of a rotation by alpha is the rotation by -alpha)
// before they are written.  Serves fp32, bf16 with d_head other than 64,
// and a cross-check of the MFMA kernels.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

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

struct BwdPlanView {
  const ReqMeta* req;
  const int32_t* qt_req;
  const int32_t* kt_req;
  const int2* row_desc;
  const int32_t* qtile_ptr;
  const int32_t* ktile_word;
  const int32_t* kt_ptr;
  const int32_t* qtile_word;
  const int32_t* sched;
  const int32_t* ksched;
};

// Rotate pairs of x[D] by -alpha_i = -(t - anchor) * omega_i (w: revolutions
// per time unit, in LDS).
template <int D>
__device__ __forceinline__ void unrotate(float (&x)[D], int64_t dt, const double* w) {
#pragma unroll
  for (int i = 0; i < D / 2; ++i) {
    const double rev = (double)dt * w[i];
    const float f = (float)(rev - rint(rev));
    float sn, cs;
    sincosf(6.283185307179586f * f, &sn, &cs);
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = x0 * cs + x1 * sn;
    x[2 * i + 1] = -x0 * sn + x1 * cs;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_bwd_ref_dq_kernel(BwdPlanView P, BwdLaunch A) {
  __shared__ float Ks[kTileK][D];
  __shared__ float Vs[kTileK][D];
  __shared__ double w[kMaxHalfD];
  const int item = P.sched[blockIdx.x];
  if (item < 0) return;
  const int qg = item / A.H;
  const int head = item - qg * A.H;
  const int req = P.qt_req[qg];
  const ReqMeta m = P.req[req];
  const int qt = qg - m.qt_off;
  const int L = m.len;
  const int t = threadIdx.x;
  const int p = qt * kTileQ + t;
  const bool valid = p < L;
  const int tok = m.tok_off + p;
  if (A.unrot_q && t < D / 2) w[t] = A.tab.w_rev[t];
  __syncthreads();

  const T* Q = (const T*)A.q;
  const T* K = (const T*)A.k;
  const T* V = (const T*)A.v;
  const T* O = (const T*)A.o;
  const T* dO = (const T*)A.dout;
  float q[D], g[D], acc[D];
  float dsum = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? ld(Q + (int64_t)tok * A.q_st + (int64_t)head * A.q_sh + c) : 0.f;
    g[c] = valid ? ld(dO + (int64_t)tok * A.do_st + (int64_t)head * A.do_sh + c) : 0.f;
    const float o = valid ? ld(O + (int64_t)tok * A.o_st + (int64_t)head * A.o_sh + c) : 0.f;
    dsum = fmaf(g[c], o, dsum);
    acc[c] = 0.f;
  }
  int lo = 0, hi = 0, self = 0;
  float lse2 = INFINITY;
  if (valid) {
    const int2 dsc = P.row_desc[tok];
    lo = dsc.x;
    hi = dsc.y & 0x7fffffff;
    self = dsc.y < 0;
    const float l = A.lse[(int64_t)head * A.T + tok];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;  // empty row: every P is 0
    A.dsum[(int64_t)head * A.T + tok] = dsum;
    A.lse2[(int64_t)head * A.T + tok] = lse2;
  }
  const float c2 = A.scale * kLog2e;

  const int e0 = P.qtile_ptr[qg], e1 = P.qtile_ptr[qg + 1];
  for (int e = e0; e < e1; ++e) {
    const int kw = P.ktile_word[e];
    const int kt = kw & 0x7fffffff;
    const bool partial = kw < 0;
    __syncthreads();
    for (int x = t; x < kTileK * D; x += blockDim.x) {
      const int j = x / D, c = x - j * D;
      const int key = kt * kTileK + j;
      const bool in = key < L;
      const int64_t kk = (int64_t)(m.tok_off + key);
      Ks[j][c] = in ? ld(K + kk * A.k_st + (int64_t)head * A.k_sh + c) : 0.f;
      Vs[j][c] = in ? ld(V + kk * A.v_st + (int64_t)head * A.v_sh + c) : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < kTileK; ++j) {
      const int key = kt * kTileK + j;
      if (partial && !((key >= lo && key < hi) || (self && key == p))) continue;
      if (!partial && key >= L) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(q[c], Ks[j][c], s);
        dp = fmaf(g[c], Vs[j][c], dp);
      }
      const float pr = exp2f(s * c2 - lse2);
      const float ds = pr * (dp - dsum);
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, Ks[j][c], acc[c]);
    }
  }
  if (!valid) return;
  const float sc = A.scale * plan_poison(A.plan_err);
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] *= sc;
  if (A.unrot_q) unrotate<D>(acc, A.ts[tok] - A.anchors[req], w);
  T* dQ = (T*)A.dq;
#pragma unroll
  for (int c = 0; c < D; ++c) st(dQ + (int64_t)tok * A.dq_st + (int64_t)head * A.dq_sh + c, acc[c]);
}

constexpr int kChunk = 32;  // query rows staged at a time by the dK/dV kernel

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_bwd_ref_dkdv_kernel(BwdPlanView P, BwdLaunch A) {
  __shared__ float Qs[kChunk][D];
  __shared__ float Gs[kChunk][D];
  __shared__ float ls[kChunk], ds_[kChunk];
  __shared__ int2 dsc[kChunk];
  __shared__ double w[kMaxHalfD];
  const int item = P.ksched[blockIdx.x];
  if (item < 0) return;
  const int kg = item / A.H;
  const int head = item - kg * A.H;
  const int req = P.kt_req[kg];
  const ReqMeta m = P.req[req];
  const int kb = kg - m.kt_off;  // key block of 128 keys
  const int L = m.len;
  const int t = threadIdx.x;
  const int j = kb * 128 + t;  // this thread's key (request-local)
  const bool valid = j < L;
  const int tokk = m.tok_off + j;
  if (A.unrot_k && t < D / 2) w[t] = A.tab.w_rev[t];
  __syncthreads();

  const T* Q = (const T*)A.q;
  const T* K = (const T*)A.k;
  const T* V = (const T*)A.v;
  const T* dO = (const T*)A.dout;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    k[c] = valid ? ld(K + (int64_t)tokk * A.k_st + (int64_t)head * A.k_sh + c) : 0.f;
    v[c] = valid ? ld(V + (int64_t)tokk * A.v_st + (int64_t)head * A.v_sh + c) : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const float c2 = A.scale * kLog2e;
  const int e0 = P.kt_ptr[kg], e1 = P.kt_ptr[kg + 1];
  for (int e = e0; e < e1; ++e) {
    const int qw = P.qtile_word[e];
    const int qt = qw & 0x7fffffff;
    const bool partial = qw < 0;
    for (int r0 = 0; r0 < kTileQ; r0 += kChunk) {
      const int row0 = qt * kTileQ + r0;
      if (row0 >= L) break;
      __syncthreads();
      for (int x = t; x < kChunk * D; x += blockDim.x) {
        const int i = x / D, c = x - i * D;
        const int row = row0 + i;
        const bool in = row < L;
        const int64_t tq = (int64_t)(m.tok_off + row);
        Qs[i][c] = in ? ld(Q + tq * A.q_st + (int64_t)head * A.q_sh + c) : 0.f;
        Gs[i][c] = in ? ld(dO + tq * A.do_st + (int64_t)head * A.do_sh + c) : 0.f;
      }
      if (t < kChunk) {
        const int row = row0 + t;
        const bool in = row < L;
        const int64_t tq = (int64_t)(m.tok_off + row);
        ls[t] = in ? A.lse2[(int64_t)head * A.T + tq] : INFINITY;
        ds_[t] = in ? A.dsum[(int64_t)head * A.T + tq] : 0.f;
        dsc[t] = in ? P.row_desc[tq] : make_int2(0, 0);
      }
      __syncthreads();
      if (!valid) continue;
      for (int i = 0; i < kChunk; ++i) {
        const int row = row0 + i;
        if (row >= L) break;
        if (partial) {
          const int lo = dsc[i].x, hi = dsc[i].y & 0x7fffffff;
          const bool self = dsc[i].y < 0;
          if (!((j >= lo && j < hi) || (self && j == row))) continue;
        }
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s = fmaf(Qs[i][c], k[c], s);
          dp = fmaf(Gs[i][c], v[c], dp);
        }
        const float pr = exp2f(s * c2 - ls[i]);
        const float dsv = pr * (dp - ds_[i]);
#pragma unroll
        for (int c = 0; c < D; ++c) {
          dv[c] = fmaf(pr, Gs[i][c], dv[c]);
          dk[c] = fmaf(dsv, Qs[i][c], dk[c]);
        }
      }
    }
  }
  if (!valid) return;
  const float pz = plan_poison(A.plan_err);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    dk[c] *= A.scale * pz;
    dv[c] *= pz;
  }
  if (A.unrot_k) unrotate<D>(dk, A.ts[tokk] - A.anchors[req], w);
  T* dK = (T*)A.dk;
  T* dV = (T*)A.dv;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    st(dK + (int64_t)tokk * A.dk_st + (int64_t)head * A.dk_sh + c, dk[c]);
    st(dV + (int64_t)tokk * A.dv_st + (int64_t)head * A.dv_sh + c, dv[c]);
  }
}

template <typename T, int D>
hipError_t launch_bwd_ref(const rk_plan* p, const BwdLaunch& a, hipStream_t s) {
  BwdPlanView P{p->dev.req,     p->dev.qt_req,    p->dev.kt_req,     p->dev.row_desc,
                p->dev.qtile_ptr, p->dev.ktile_word, p->dev.kt_ptr,   p->dev.qtile_word,
                p->dev.sched,   p->dev.ksched};
  hipLaunchKernelGGL((attn_bwd_ref_dq_kernel<T, D>), dim3((unsigned)p->slots), dim3(128), 0, s, P,
                     a);
  hipLaunchKernelGGL((attn_bwd_ref_dkdv_kernel<T, D>), dim3((unsigned)p->kslots), dim3(128), 0, s,
                     P, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_reference(const rk_plan* p, const BwdLaunch& a, rk_dtype dt,
                                     hipStream_t s) {
  if (p->slots == 0 || p->kslots == 0) return hipSuccess;
  if (dt == RK_F32) {
    if (a.d == 32) return launch_bwd_ref<float, 32>(p, a, s);
    if (a.d == 64) return launch_bwd_ref<float, 64>(p, a, s);
    if (a.d == 128) return launch_bwd_ref<float, 128>(p, a, s);
  } else {
    if (a.d == 32) return launch_bwd_ref<__hip_bfloat16, 32>(p, a, s);
    if (a.d == 64) return launch_bwd_ref<__hip_bfloat16, 64>(p, a, s);
    if (a.d == 128) return launch_bwd_ref<__hip_bfloat16, 128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rk
