// Time RoPE (CADET, "time encoding and self-gating"): pair (2i, 2i+1) of a
// token at time t in request r turns by alpha_i = (t - anchor_r) * omega_i,
// omega_i = phi_min / dt_max * base^(2i/d).  The time difference is exact in
// int64; the phase is formed in revolutions in double precision and reduced
// to [-1/2, 1/2] before an fp32 sin/cos, so large Unix times lose nothing.
//
// HBM-bound elementwise pass: the angle of a (token, pair) is computed once
// and applied to every head.  Aligned rows with d % 8 == 0 take the 16-byte
// vector form; anything else the one-pair-per-thread form.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const __hip_bfloat16* p) {
  return __uint_as_float(((unsigned)(*(const unsigned short*)p)) << 16);
}
__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *(float2*)p = make_float2(a, b);
}
__device__ __forceinline__ unsigned short f2bf(float f) {
  // round to nearest even (inputs are finite)
  unsigned u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
__device__ __forceinline__ void store_pair(__hip_bfloat16* p, float a, float b) {
  *(unsigned*)p = (unsigned)f2bf(a) | ((unsigned)f2bf(b) << 16);
}

// Is a token of segment kind k among the kinds to rotate (bit k of kinds)?
__device__ __forceinline__ bool selected(uint8_t k, unsigned kinds) {
  return k < 4 && ((kinds >> k) & 1u);
}

// Sum of v over the n lanes (power of two, n <= 64, aligned) holding one row.
__device__ __forceinline__ float row_sum(float v, int n) {
  for (int o = 1; o < n; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T, bool kNorm>
__global__ __launch_bounds__(256) void rope_kernel(int R, int Tn, const int32_t* __restrict__ offs,
                                                   const int64_t* __restrict__ ts,
                                                   const int64_t* __restrict__ anchors,
                                                   const uint8_t* __restrict__ kind,
                                                   unsigned kinds, RopeTab tab, const T* x, T* y,
                                                   int H, int d,
                                                   int64_t ist, int64_t ish, int64_t ost,
                                                   int64_t osh, float eps,
                                                   const float* __restrict__ gamma) {
  __shared__ double w[kMaxHalfD];
  const int half = d >> 1;
  if ((int)threadIdx.x < half) w[threadIdx.x] = tab.w_rev[threadIdx.x];
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)Tn * half) return;
  const int tok = (int)(gid / half);
  const int i = (int)(gid - (int64_t)tok * half);
  if (kinds && !selected(kind[tok], kinds)) return;
  // request of the token: last r with offs[r] <= tok
  int a = 0, b = R;
  while (a < b) {
    const int m = (a + b) >> 1;
    if (offs[m] <= tok) a = m + 1; else b = m;
  }
  const int r = a > 0 ? a - 1 : 0;
  const double rev = (double)(ts[tok] - anchors[r]) * w[i];
  const float f = (float)(rev - rint(rev));
  float sn, cs;
  sincosf(6.283185307179586f * f, &sn, &cs);
  const T* xp = x + (int64_t)tok * ist + 2 * i;
  T* yp = y + (int64_t)tok * ost + 2 * i;
  // with kNorm the d / 2 lanes of a token (consecutive, aligned: d / 2
  // divides 64 and 256) hold one row per head and reduce it together
  const float g0 = kNorm && gamma ? gamma[2 * i] : 1.f;
  const float g1 = kNorm && gamma ? gamma[2 * i + 1] : 1.f;
  for (int h = 0; h < H; ++h) {
    float x0 = load_elem(xp + (int64_t)h * ish);
    float x1 = load_elem(xp + (int64_t)h * ish + 1);
    if (kNorm) {
      const float rstd = rsqrtf(row_sum(x0 * x0 + x1 * x1, half) / (float)d + eps);
      x0 *= rstd * g0;
      x1 *= rstd * g1;
    }
    store_pair(yp + (int64_t)h * osh, x0 * cs - x1 * sn, x0 * sn + x1 * cs);
  }
}

// Vector form for d % 8 == 0 with 16-byte aligned rows: one thread per
// (token, group of four pairs); 16-byte (bf16) or 2 x 16-byte (fp32)
// accesses per head.
template <typename T, bool kNorm>
__global__ __launch_bounds__(256) void rope8_kernel(int R, int Tn, const int32_t* __restrict__ offs,
                                                    const int64_t* __restrict__ ts,
                                                    const int64_t* __restrict__ anchors,
                                                    const uint8_t* __restrict__ kind,
                                                    unsigned kinds, RopeTab tab, const T* x, T* y,
                                                    int H, int d,
                                                    int64_t ist, int64_t ish, int64_t ost,
                                                    int64_t osh, float eps,
                                                    const float* __restrict__ gamma) {
  __shared__ double w[kMaxHalfD];
  const int half = d >> 1;
  if ((int)threadIdx.x < half) w[threadIdx.x] = tab.w_rev[threadIdx.x];
  __syncthreads();
  const int groups = d >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)Tn * groups) return;
  const int tok = (int)(gid / groups);
  const int g = (int)(gid - (int64_t)tok * groups);
  if (kinds && !selected(kind[tok], kinds)) return;
  int a = 0, b = R;
  while (a < b) {
    const int m = (a + b) >> 1;
    if (offs[m] <= tok) a = m + 1; else b = m;
  }
  const int r = a > 0 ? a - 1 : 0;
  const double dt = (double)(ts[tok] - anchors[r]);
  float sn[4], cs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double rev = dt * w[4 * g + j];
    const float f = (float)(rev - rint(rev));
    sincosf(6.283185307179586f * f, &sn[j], &cs[j]);
  }
  const T* xp = x + (int64_t)tok * ist + 8 * g;
  T* yp = y + (int64_t)tok * ost + 8 * g;
  float gm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) gm[j] = kNorm && gamma ? gamma[8 * g + j] : 1.f;
  // Heads in chunks of kHc: the chunk's loads go out before any of its
  // stores, so they are in flight together (input and output may be the
  // same rows, and each thread reads and writes only its own elements, so
  // loading ahead of the stores is safe in place too).
  constexpr int kHc = 4;
  constexpr int kW = sizeof(T) == 2 ? 1 : 2;  // 16-byte words per head
  for (int h0 = 0; h0 < H; h0 += kHc) {
    uint4 raw[kHc][kW];
#pragma unroll
    for (int k = 0; k < kHc; ++k)
      if (h0 + k < H)
#pragma unroll
        for (int q = 0; q < kW; ++q)
          raw[k][q] = *(const uint4*)(xp + (int64_t)(h0 + k) * ish + 4 * q);
#pragma unroll
    for (int k = 0; k < kHc; ++k) {
      if (h0 + k >= H) break;
      const int h = h0 + k;
      float v[8];
      if constexpr (sizeof(T) == 2) {
        const unsigned u[4] = {raw[k][0].x, raw[k][0].y, raw[k][0].z, raw[k][0].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = __uint_as_float(u[j] << 16);
          v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < kW; ++q) {
          v[4 * q] = __uint_as_float(raw[k][q].x);
          v[4 * q + 1] = __uint_as_float(raw[k][q].y);
          v[4 * q + 2] = __uint_as_float(raw[k][q].z);
          v[4 * q + 3] = __uint_as_float(raw[k][q].w);
        }
      }
      if (kNorm) {
        // the d / 8 lanes of a token (consecutive, aligned) hold one row
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
        const float rstd = rsqrtf(row_sum(ss, groups) / (float)d + eps);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= rstd * gm[j];
      }
      float o[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = v[2 * j] * cs[j] - v[2 * j + 1] * sn[j];
        o[2 * j + 1] = v[2 * j] * sn[j] + v[2 * j + 1] * cs[j];
      }
      if constexpr (sizeof(T) == 2) {
        unsigned u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          u[j] = (unsigned)f2bf(o[2 * j]) | ((unsigned)f2bf(o[2 * j + 1]) << 16);
        *(uint4*)(yp + (int64_t)h * osh) = make_uint4(u[0], u[1], u[2], u[3]);
      } else {
        *(float4*)(yp + (int64_t)h * osh) = make_float4(o[0], o[1], o[2], o[3]);
        *(float4*)(yp + (int64_t)h * osh + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}

}  // namespace

hipError_t launch_rope(int32_t R, int32_t T, const int32_t* req_offsets, const int64_t* ts,
                       const int64_t* anchors, const uint8_t* kind, unsigned kinds,
                       const RopeTab& tab, const void* x_in, void* x_out, rk_dtype dt, int H, int d,
                       int64_t in_st, int64_t in_sh, int64_t out_st, int64_t out_sh,
                       hipStream_t s, bool norm, float eps, const float* gamma) {
  if (T == 0) return hipSuccess;
  const int64_t v = 16 / (dt == RK_F32 ? 4 : 2);  // elements per 16 bytes
  const bool vec = (d % 8 == 0) && ((uintptr_t)x_in % 16 == 0) && ((uintptr_t)x_out % 16 == 0) &&
                   in_st % v == 0 && in_sh % v == 0 && out_st % v == 0 && out_sh % v == 0;
  const int per = vec ? 8 : 2;  // elements of a row per thread
  const int64_t n = (int64_t)T * (d / per);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
#define RK_ROPE_LAUNCH(KERNEL, TY, NORM)                                                         \
  hipLaunchKernelGGL((KERNEL<TY, NORM>), grid, block, 0, s, R, T, req_offsets, ts, anchors, kind, \
                     kinds, tab, (const TY*)x_in, (TY*)x_out, H, d, in_st, in_sh, out_st, out_sh,  \
                     eps, gamma)
  if (vec) {
    if (dt == RK_F32) {
      if (norm) RK_ROPE_LAUNCH(rope8_kernel, float, true);
      else RK_ROPE_LAUNCH(rope8_kernel, float, false);
    } else {
      if (norm) RK_ROPE_LAUNCH(rope8_kernel, __hip_bfloat16, true);
      else RK_ROPE_LAUNCH(rope8_kernel, __hip_bfloat16, false);
    }
  } else {
    if (dt == RK_F32) {
      if (norm) RK_ROPE_LAUNCH(rope_kernel, float, true);
      else RK_ROPE_LAUNCH(rope_kernel, float, false);
    } else {
      if (norm) RK_ROPE_LAUNCH(rope_kernel, __hip_bfloat16, true);
      else RK_ROPE_LAUNCH(rope_kernel, __hip_bfloat16, false);
    }
  }
#undef RK_ROPE_LAUNCH
  return hipGetLastError();
}

}  // namespace rk
