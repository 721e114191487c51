// Row gather-sum for the LazFormer pre-passes (section 2.3, eq. 16-18 and
// 22): y[i] = sum of input rows [b_i, e_i) for every output row i.  Group
// sums (compression) and plain row selection (pruning) are both such ranges.
// With kMean the sum is divided by the range length (SORT's pooled query
// pruning: the pruned history rows averaged into one).
//
// HBM-bound: every input row is read once and every output row written once.
// Lanes across the row: 16-byte loads (8 bf16 or 4 fp32 per lane) when rows
// are 16-byte aligned, one element per lane otherwise; a row narrower than
// half a wave's reach shares the wave with others (2^rpw_log2 output rows
// per wave, e.g. two at 4 heads x 64 bf16), so no lane idles.  Eight input
// rows are loaded before they are added, so a group sum keeps eight loads
// in flight instead of waiting for each; fp32 accumulation in input order,
// one rounding on the store.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(__hip_bfloat16 v) {
  return __uint_as_float(((unsigned)(*(const unsigned short*)&v)) << 16);
}
__device__ __forceinline__ unsigned short f2bf(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even (finite inputs)
  return (unsigned short)(u >> 16);
}
__device__ __forceinline__ void from_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void from_f(__hip_bfloat16* p, float v) {
  *(unsigned short*)p = f2bf(v);
}

constexpr int kWaves = 4;  // waves per 256-thread block

// V elements per lane per access: 16 bytes when vectorised, else 1.
template <typename T, bool kVec, bool kMean>
__global__ __launch_bounds__(256) void gather_sum_kernel(const int2* __restrict__ ranges,
                                                         int n_out, int n_in,
                                                         const T* __restrict__ x, int64_t xs,
                                                         T* __restrict__ y, int64_t ys,
                                                         int width, int rpw_log2) {
  constexpr int V = kVec ? 16 / (int)sizeof(T) : 1;
  const int lane = threadIdx.x & 63;
  const int lanes = 64 >> rpw_log2;  // lanes of one output row
  const int sl = lane & (lanes - 1);
  const int i = (((int)blockIdx.x * kWaves + (int)(threadIdx.x >> 6)) << rpw_log2) +
                (lane >> (6 - rpw_log2));
  if (i >= n_out) return;
  const int2 rg = ranges[i];
  const int b = min(max(rg.x, 0), n_in);
  const int e = min(max(rg.y, b), n_in);
  const float scale = kMean && e > b ? 1.f / (float)(e - b) : 1.f;
  for (int c = sl * V; c < width; c += lanes * V) {
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    const T* src = x + (int64_t)b * xs + c;
    int j = b;
    for (; j + 8 <= e; j += 8, src += 8 * xs) {
      if (kVec) {
        uint4 u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) u[k] = *(const uint4*)(src + k * xs);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          T vals[V];
          __builtin_memcpy(vals, &u[k], 16);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] += to_f(vals[v]);
        }
      } else {
        T u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) u[k] = src[k * xs];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[0] += to_f(u[k]);
      }
    }
    for (; j < e; ++j, src += xs) {
      if (kVec) {
        const uint4 u = *(const uint4*)src;
        T vals[V];
        __builtin_memcpy(vals, &u, 16);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += to_f(vals[v]);
      } else {
        acc[0] += to_f(*src);
      }
    }
    T* dst = y + (int64_t)i * ys + c;
    if (kVec) {
      T vals[V];
#pragma unroll
      for (int v = 0; v < V; ++v) from_f(&vals[v], kMean ? acc[v] * scale : acc[v]);
      uint4 u;
      __builtin_memcpy(&u, vals, 16);
      *(uint4*)dst = u;
    } else {
      from_f(dst, kMean ? acc[0] * scale : acc[0]);
    }
  }
}

template <typename T, bool kMean>
hipError_t launch(const int2* ranges, int n_out, int n_in, const void* x, int64_t xs, void* y,
                  int64_t ys, int width, hipStream_t s) {
  const int per = 16 / (int)sizeof(T);
  const bool vec = ((uintptr_t)x % 16) == 0 && ((uintptr_t)y % 16) == 0 && width % per == 0 &&
                   xs % per == 0 && ys % per == 0;
  // output rows per wave: as many as fit whole in 64 lanes, at most 8
  const int chunks = vec ? width / per : width;
  int rpw_log2 = 0;
  while (rpw_log2 < 3 && chunks <= (32 >> rpw_log2)) ++rpw_log2;
  const int rows_per_block = kWaves << rpw_log2;
  const dim3 grid((unsigned)((n_out + rows_per_block - 1) / rows_per_block));
  if (vec)
    hipLaunchKernelGGL((gather_sum_kernel<T, true, kMean>), grid, dim3(256), 0, s, ranges, n_out,
                       n_in, (const T*)x, xs, (T*)y, ys, width, rpw_log2);
  else
    hipLaunchKernelGGL((gather_sum_kernel<T, false, kMean>), grid, dim3(256), 0, s, ranges, n_out,
                       n_in, (const T*)x, xs, (T*)y, ys, width, rpw_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_sum(const int32_t* ranges, int n_out, int n_in, const void* x,
                             int64_t xs, void* y, int64_t ys, int width, rk_dtype dt,
                             hipStream_t s, bool mean) {
  if (n_out == 0) return hipSuccess;
  const int2* rg = (const int2*)ranges;
  if (dt == RK_F32)
    return mean ? launch<float, true>(rg, n_out, n_in, x, xs, y, ys, width, s)
                : launch<float, false>(rg, n_out, n_in, x, xs, y, ys, width, s);
  return mean ? launch<__hip_bfloat16, true>(rg, n_out, n_in, x, xs, y, ys, width, s)
              : launch<__hip_bfloat16, false>(rg, n_out, n_in, x, xs, y, ys, width, s);
}

}  // namespace rk
