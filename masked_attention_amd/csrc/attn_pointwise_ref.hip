// Plain HSTU pointwise aggregated attention over the tile plan (HSTU eq. 2;
// no matrix cores): O_i = sum over visible j of SiLU(scale q_i . k_j +
// rab_ij) v_j, rab_ij = pos_bias[min(|p_i - p_j|, np - 1)] +
// time_bias[min(floor(log2(1 + |t_i - t_j|)), nt - 1)].
//
// One 128-thread workgroup per (query tile, head), one thread per query
// row, K, V and the key timestamps staged in LDS per 64-key tile; the mask
// (visible interval plus the candidate self link) runs on PARTIAL tiles
// only.  Serves fp32, bf16 with d_head other than 64, and a cross-check of
// the MFMA kernel.
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

// floor(log2(1 + |dt|)) capped at nt - 1: the index of the highest set bit
__device__ __forceinline__ int time_bucket(int64_t dt, int nt) {
  const uint64_t x = 1ull + (uint64_t)(dt < 0 ? -dt : dt);
  return min(63 - __clzll((long long)x), nt - 1);
}

template <typename T, int D>
__global__ __launch_bounds__(128) void pw_ref_kernel(const ReqMeta* __restrict__ req,
                                                     const int32_t* __restrict__ qt_req,
                                                     const int2* __restrict__ row_desc,
                                                     const int32_t* __restrict__ qtile_ptr,
                                                     const int32_t* __restrict__ ktile_word,
                                                     const int32_t* __restrict__ sched,
                                                     PwLaunch A) {
  __shared__ float Ks[kTileK][D];
  __shared__ float Vs[kTileK][D];
  __shared__ int64_t Ts[kTileK];
  const int item = sched[blockIdx.x];
  if (item < 0) return;
  const int qg = item / A.H;
  const int head = item - qg * A.H;
  const ReqMeta m = req[qt_req[qg]];
  const int qt = qg - m.qt_off;
  const int L = m.len;
  const int t = threadIdx.x;
  const int p = qt * kTileQ + t;
  const bool valid = p < L;
  const int tok = m.tok_off + p;
  const T* Q = (const T*)A.q;
  const T* K = (const T*)A.k;
  const T* V = (const T*)A.v;
  float q[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? ld(Q + (int64_t)tok * A.q_st + (int64_t)head * A.q_sh + c) : 0.f;
    acc[c] = 0.f;
  }
  int lo = 0, hi = 0, self = 0;
  int64_t ti = 0;
  if (valid) {
    const int2 dsc = row_desc[tok];
    lo = dsc.x;
    hi = dsc.y & 0x7fffffff;
    self = dsc.y < 0;
    ti = A.ts[tok];
  }
  const int e0 = qtile_ptr[qg], e1 = qtile_ptr[qg + 1];
  for (int e = e0; e < e1; ++e) {
    const int kw = ktile_word[e];
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
    if (t < kTileK) {
      const int key = kt * kTileK + t;
      Ts[t] = key < L ? A.ts[m.tok_off + key] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    for (int j = 0; j < kTileK; ++j) {
      const int key = kt * kTileK + j;
      if (key >= L) break;
      if (partial && !((key >= lo && key < hi) || (self && key == p))) continue;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(q[c], Ks[j][c], dot);
      float x = dot * A.scale;
      if (A.pos_bias) x += A.pos_bias[min(abs(p - key), A.np - 1)];
      if (A.time_bias) x += A.time_bias[time_bucket(ti - Ts[j], A.nt)];
      const float w = x / (1.f + expf(-x));
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(w, Vs[j][c], acc[c]);
    }
  }
  if (!valid) return;
  const float pz = plan_poison(A.plan_err);
  T* O = (T*)A.o;
#pragma unroll
  for (int c = 0; c < D; ++c) st(O + (int64_t)tok * A.o_st + (int64_t)head * A.o_sh + c, acc[c] * pz);
}

template <typename T, int D>
hipError_t launch_pw(const rk_plan* p, const PwLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL((pw_ref_kernel<T, D>), dim3((unsigned)p->slots), dim3(128), 0, s,
                     p->dev.req, p->dev.qt_req, p->dev.row_desc, p->dev.qtile_ptr,
                     p->dev.ktile_word, p->dev.sched, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pointwise_reference(const rk_plan* p, const PwLaunch& a, rk_dtype dt,
                                      hipStream_t s) {
  if (p->slots == 0) return hipSuccess;
  if (dt == RK_F32) {
    if (a.d == 32) return launch_pw<float, 32>(p, a, s);
    if (a.d == 64) return launch_pw<float, 64>(p, a, s);
    if (a.d == 128) return launch_pw<float, 128>(p, a, s);
  } else {
    if (a.d == 32) return launch_pw<__hip_bfloat16, 32>(p, a, s);
    if (a.d == 64) return launch_pw<__hip_bfloat16, 64>(p, a, s);
    if (a.d == 128) return launch_pw<__hip_bfloat16, 128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rk
