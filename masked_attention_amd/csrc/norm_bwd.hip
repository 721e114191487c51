// Backward through QK Norm (TM20K section 2; SORT section 3.3.2: RMSNorm of
// every [d] row of Q and K before the scores).  The attention backward runs
// on the normalised rows and leaves g = dLoss/dy in the gradient buffer;
// this pass takes it back through y = x * r * gamma, r = 1 / sqrt(mean(x^2)
// + eps), in place:
//   dx = r * gamma * g - x * r^3 * sum_j(gamma_j g_j x_j) / d,
// and sums dgamma = sum over rows of g * x * r.
//
// HBM-bound: every row of x and g is read once and dx written once.  A row
// is spread over d / 4 lanes (4 consecutive elements each); its two sums
// meet through shuffles among those lanes.  Each block handles a fixed
// range of kRowsPerNormBlock rows and writes its dgamma partial (summed in a
// fixed order over lanes and waves); a second kernel adds the partials in
// block order, so dgamma does not depend on scheduling.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __hip_bfloat16* p) {
  return __uint_as_float(((unsigned)(*(const unsigned short*)p)) << 16);
}
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(__hip_bfloat16* p, float v) {
  unsigned u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even (finite values)
  *(unsigned short*)p = (unsigned short)(u >> 16);
}

// Sum over the `width` consecutive lanes of a row group (width a power of 2).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rmsnorm_bwd_kernel(NormBwdArgs a) {
  constexpr int kLpr = D / 4;          // lanes per row
  constexpr int kRpw = 64 / kLpr;      // rows per wave and pass
  constexpr int kRpp = 4 * kRpw;       // rows per block and pass
  __shared__ float part[4][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane % kLpr;           // element group of the lane: 4 j .. 4 j + 3
  const int rw = lane / kLpr;          // row of the lane inside the wave's pass
  const T* x = (const T*)a.x;
  T* g = (T*)a.g;
  float gam[4] = {1.f, 1.f, 1.f, 1.f};
  if (a.gamma) {
#pragma unroll
    for (int e = 0; e < 4; ++e) gam[e] = a.gamma[4 * j + e];
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerNormBlock;
  for (int pass = 0; pass < kRowsPerNormBlock / kRpp; ++pass) {
    const int64_t row = r0 + (int64_t)pass * kRpp + wv * kRpw + rw;
    // a row's lanes are in or out together, and shuffle only among themselves
    if (row < a.rows) {
      const int64_t tok = row / a.H, head = row - tok * a.H;
      const T* xp = x + tok * a.x_st + head * a.x_sh + 4 * j;
      T* gp = g + tok * a.g_st + head * a.g_sh + 4 * j;
      float xv[4], gv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[e] = ld(xp + e);
        gv[e] = ld(gp + e);
      }
      float ss = 0.f, tt = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss = fmaf(xv[e], xv[e], ss);
        tt = fmaf(gam[e] * gv[e], xv[e], tt);
      }
      ss = group_sum<kLpr>(ss);
      tt = group_sum<kLpr>(tt);
      const float r = rsqrtf(ss * (1.f / D) + a.eps);
      const float c = r * r * r * tt * (1.f / D);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st(gp + e, r * gam[e] * gv[e] - xv[e] * c);
        acc[e] = fmaf(gv[e] * xv[e], r, acc[e]);
      }
    }
  }
  if (!a.partial) return;
  // dgamma partial: lanes with the same j across the wave's rows, then the
  // four waves, always in the same order
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = acc[e];
#pragma unroll
    for (int o = kLpr; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    acc[e] = v;
  }
  if (rw == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wv][4 * j + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D)
    a.partial[(int64_t)blockIdx.x * D + threadIdx.x] =
        ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
        part[3][threadIdx.x];
}

// dgamma[i] = sum over blocks b of partial[b][i].  The groups of d threads
// of one workgroup take the blocks in a fixed interleaved order (four
// running sums each, added in a fixed order), then the groups are added in
// order: the result does not depend on scheduling.
constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void gamma_reduce_kernel(const float* partial,
                                                                      int64_t nblk, int d,
                                                                      float* dgamma) {
  __shared__ float sums[kReduceThreads];
  const int groups = kReduceThreads / d;  // d in {32, 64, 128}
  const int grp = threadIdx.x / d, i = threadIdx.x - grp * d;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  const int64_t step = 4 * (int64_t)groups;
  int64_t b = grp;
  for (; b + 3 * groups < nblk; b += step) {
    s0 += partial[b * d + i];
    s1 += partial[(b + groups) * d + i];
    s2 += partial[(b + 2 * groups) * d + i];
    s3 += partial[(b + 3 * groups) * d + i];
  }
  for (; b < nblk; b += groups) s0 += partial[b * d + i];
  sums[threadIdx.x] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  if ((int)threadIdx.x < d) {
    float t = 0.f;
    for (int k = 0; k < groups; ++k) t += sums[k * d + threadIdx.x];
    dgamma[threadIdx.x] = t;
  }
}

template <typename T, int D>
hipError_t launch_t(const NormBwdArgs& a, hipStream_t s) {
  const int64_t nblk = norm_bwd_blocks(a.rows);
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, D>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
  if (a.partial && a.dgamma)
    hipLaunchKernelGGL(gamma_reduce_kernel, dim3(1), dim3(kReduceThreads), 0, s, a.partial, nblk,
                       D, a.dgamma);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_bwd(const NormBwdArgs& a, rk_dtype dt, int d, hipStream_t s) {
  if (a.rows == 0) {
    // no rows: the gain gradients are zero (the reduction over no blocks
    // writes them; a kernel rather than a memset, so the call can be captured)
    if (!a.dgamma) return hipSuccess;
    if (d != 32 && d != 64 && d != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gamma_reduce_kernel, dim3(1), dim3(kReduceThreads), 0, s, a.partial,
                       (int64_t)0, d, a.dgamma);
    return hipGetLastError();
  }
  if (dt == RK_F32) {
    if (d == 32) return launch_t<float, 32>(a, s);
    if (d == 64) return launch_t<float, 64>(a, s);
    if (d == 128) return launch_t<float, 128>(a, s);
  } else {
    if (d == 32) return launch_t<__hip_bfloat16, 32>(a, s);
    if (d == 64) return launch_t<__hip_bfloat16, 64>(a, s);
    if (d == 128) return launch_t<__hip_bfloat16, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rk
