// Device helpers shared by the MFMA kernels of the backward and the
// pointwise attention (CDNA4, gfx950): operand vector types, bf16 packing,
// scalar-cache loads of uniform values, LDS address casts and the buffer
// descriptor flags of direct global -> LDS copies.
#pragma once

#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr unsigned kBufferFlags = 0x00020000u;  // raw buffer, 32-bit data format

#define RK_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// A wave-uniform value read through the scalar cache.
template <typename T>
__device__ __forceinline__ T ldc(const T* p, int64_t i) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(4))) T*)p)[i];
#else
  return p[i];  // host pass of the single-source compile; never executed
#endif
}

// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  unsigned u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// x * c for the eight bf16 of a fragment, rounded back to bf16 (to nearest
// even).
__device__ __forceinline__ bf16x8 scale_bf16x8(const bf16x8& x, float c) {
  uint4 u;
  __builtin_memcpy(&u, &x, 16);
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
  unsigned o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(bf_lo(w[j]) * c, bf_hi(w[j]) * c);
  return as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
}

// Visible keys of a 64-key tile starting at c0 for one query row, as a
// 64-bit set: the row's interval [lo, hi) clipped to the tile plus, for a
// candidate (self), its own position.
__device__ __forceinline__ uint64_t tile_vis_bits(int c0, int lo, int hi, int self, int row) {
  const int a = min(max(lo - c0, 0), 64), b = min(max(hi - c0, 0), 64);
  const uint64_t below_b = b >= 64 ? ~0ull : (1ull << b) - 1ull;
  const uint64_t below_a = a >= 64 ? ~0ull : (1ull << a) - 1ull;
  uint64_t vis = below_b & ~below_a;
  const int sr = row - c0;
  if (self && sr >= 0 && sr < 64) vis |= 1ull << sr;
  return vis;
}

}  // namespace cdna4
}  // namespace rk
