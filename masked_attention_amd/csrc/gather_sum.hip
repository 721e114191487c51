// Row gather-sum for the LazFormer pre-passes (section 2.3, eq. 16-18 and
// 22): y[i] = sum of input rows [b_i, e_i) for every output row i.  Group
// sums (compression) and plain row selection (pruning) are both such ranges.
// With kMean the sum is divided by the range length (SORT's pooled query
// pruning: the pruned history rows averaged into one).
//
// HBM-bound: every input row is read once and every output row written once.
// One wave per output row, lanes across the row: 16-byte loads (8 bf16 or 4
// fp32 per lane) when rows are 16-byte aligned, one element per lane
// otherwise; fp32 accumulation, one rounding on the store.
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

constexpr int kWaves = 4;  // output rows per 256-thread block

// V elements per lane per access: 16 bytes when vectorised, else 1.
template <typename T, bool kVec, bool kMean>
__global__ __launch_bounds__(256) void gather_sum_kernel(const int2* __restrict__ ranges,
                                                         int n_out, int n_in,
                                                         const T* __restrict__ x, int64_t xs,
                                                         T* __restrict__ y, int64_t ys,
                                                         int width) {
  constexpr int V = kVec ? 16 / (int)sizeof(T) : 1;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (i >= n_out) return;
  const int2 rg = ranges[i];
  const int b = min(max(rg.x, 0), n_in);
  const int e = min(max(rg.y, b), n_in);
  const float scale = kMean && e > b ? 1.f / (float)(e - b) : 1.f;
  for (int c = lane * V; c < width; c += 64 * V) {
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    for (int j = b; j < e; ++j) {
      const T* src = x + (int64_t)j * xs + c;
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
  const dim3 grid((unsigned)((n_out + kWaves - 1) / kWaves));
  if (vec)
    hipLaunchKernelGGL((gather_sum_kernel<T, true, kMean>), grid, dim3(256), 0, s, ranges, n_out,
                       n_in, (const T*)x, xs, (T*)y, ys, width);
  else
    hipLaunchKernelGGL((gather_sum_kernel<T, false, kMean>), grid, dim3(256), 0, s, ranges, n_out,
                       n_in, (const T*)x, xs, (T*)y, ys, width);
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
