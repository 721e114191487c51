// Merge of split work items (candidates-only plans with a work list).
//
// The key range of a split (query tile, head) item was cut into chunks of
// CSR entries; each chunk's slot left, per query row, its unnormalised output
// O_j = sum_k exp(s_k - m_j) v_k, its reference max m_j and its sum
// l_j = sum_k exp(s_k - m_j).  Softmax over the union of the chunks is
//   M = max_j m_j,  w_j = exp(m_j - M),  O = sum_j w_j O_j / sum_j w_j l_j,
//   LSE = M + log(sum_j w_j l_j),
// the same rescaling the online softmax applies between key tiles (HSTU,
// App. H, M-FALCON; the flash-decoding split of a long key range).  The
// kernels keep m in their own units; to_log2 and to_nat convert it.
//
// d_head / 4 threads per query row, each owning four d values (one 16-byte
// load per part), so a split item's 128 rows spread over d_head / 16
// workgroups of 512 threads.  Parts are read sixteen at a time (their loads
// in flight together) and merged with the online rescaling, so the running
// max is never re-read.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(__hip_bfloat16* p, float v) {
  unsigned u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  *(unsigned short*)p = (unsigned short)(u >> 16);
}

constexpr int kGroup = 16;  // parts read together
constexpr int kThreads = 512;

// workgroups per split item at width D: 128 rows of D / 4 threads
template <int D>
constexpr int blocks_per_item() { return kTileQ * (D / 4) / kThreads; }

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const ReqMeta* req,
                                                                const int32_t* qt_req,
                                                                const SplitEntry* splits,
                                                                AttnLaunch A, float to_log2,
                                                                float to_nat) {
  constexpr int kQ = 4;           // d values of this thread
  constexpr int kV = 1;           // float4 loads per part
  constexpr int kTpr = D / kQ;    // threads per row
  constexpr int kStride = kTileQ * (D + 2);
  const SplitEntry se = splits[blockIdx.x / blocks_per_item<D>()];
  if (se.item < 0) return;
  const int qg = se.item / A.H;
  const int head = se.item - qg * A.H;
  const ReqMeta m = req[qt_req[qg]];
  const int rl = (int)(blockIdx.x % blocks_per_item<D>()) * (kThreads / kTpr) +
                 (int)threadIdx.x / kTpr;
  const int c0 = ((int)threadIdx.x % kTpr) * kQ;
  const int row = (qg - m.qt_off) * kTileQ + rl;
  if (row >= m.len) return;
  const int tok = m.tok_off + row;
  const float* base = A.part + (int64_t)se.part0 * kStride;

  float M = -INFINITY, l = 0.f;
  float acc[kQ];
#pragma unroll
  for (int c = 0; c < kQ; ++c) acc[c] = 0.f;
  for (int j0 = 0; j0 < se.nparts; j0 += kGroup) {
    float mj[kGroup], lj[kGroup];
    float4 v[kGroup][kV];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      // past the last part: re-read it with weight 0
      const float* pj = base + min(j0 + u, se.nparts - 1) * kStride;
      mj[u] = j0 + u < se.nparts ? pj[kTileQ * D + rl] : -INFINITY;
      lj[u] = pj[kTileQ * D + kTileQ + rl];
      const float4* o4 = (const float4*)(pj + rl * D + c0);
#pragma unroll
      for (int c = 0; c < kV; ++c) v[u][c] = o4[c];
    }
    float gm = mj[0];
#pragma unroll
    for (int u = 1; u < kGroup; ++u) gm = fmaxf(gm, mj[u]);
    const float Mn = fmaxf(M, gm);
    if (Mn == -INFINITY) continue;  // nothing visible to the row so far
    const float alpha = exp2f((M - Mn) * to_log2);  // 0 while M is -inf
    l *= alpha;
#pragma unroll
    for (int c = 0; c < kQ; ++c) acc[c] *= alpha;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      // a part that saw nothing of the row has m = -inf and weight 0
      const float w = exp2f((mj[u] - Mn) * to_log2);
      l = fmaf(w, lj[u], l);
#pragma unroll
      for (int c = 0; c < kV; ++c) {
        acc[4 * c] = fmaf(w, v[u][c].x, acc[4 * c]);
        acc[4 * c + 1] = fmaf(w, v[u][c].y, acc[4 * c + 1]);
        acc[4 * c + 2] = fmaf(w, v[u][c].z, acc[4 * c + 2]);
        acc[4 * c + 3] = fmaf(w, v[u][c].w, acc[4 * c + 3]);
      }
    }
    M = Mn;
  }
  const float pz = plan_poison(A.plan_err);
  const float inv = (l > 0.f ? 1.f / l : 0.f) * pz;
  T* O = (T*)A.o + (int64_t)tok * A.o_st + (int64_t)head * A.o_sh + c0;
#pragma unroll
  for (int c = 0; c < kQ; ++c)
    if (c0 + c < A.d) st(O + c, acc[c] * inv);  // columns past d_head are padding
  if (A.lse && c0 == 0)
    A.lse[(int64_t)head * A.T + tok] = (l > 0.f ? M * to_nat + logf(l) : -INFINITY) * pz;
}

template <typename T, int D>
hipError_t launch(const rk_plan* p, const AttnLaunch& a, float to_log2, float to_nat,
                  hipStream_t s) {
  // at most kSplitTarget / 2 items are split
  hipLaunchKernelGGL((attn_combine_kernel<T, D>),
                     dim3((unsigned)(kSplitTarget / 2 * blocks_per_item<D>())), dim3(kThreads), 0,
                     s, p->dev.req, p->dev.qt_req, p->dev.splits, a, to_log2, to_nat);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_combine(const rk_plan* p, const AttnLaunch& a, rk_dtype dt, float to_log2,
                               float to_nat, hipStream_t s) {
  if (p->grid <= p->slots || a.part == nullptr) return hipSuccess;
  // the parts have the producing kernel's width dp
  if (a.d > a.dp) return hipErrorInvalidValue;
  if (dt == RK_F32) {
    if (a.dp == 32) return launch<float, 32>(p, a, to_log2, to_nat, s);
    if (a.dp == 64) return launch<float, 64>(p, a, to_log2, to_nat, s);
    if (a.dp == 128) return launch<float, 128>(p, a, to_log2, to_nat, s);
  } else {
    if (a.dp == 32) return launch<__hip_bfloat16, 32>(p, a, to_log2, to_nat, s);
    if (a.dp == 64) return launch<__hip_bfloat16, 64>(p, a, to_log2, to_nat, s);
    if (a.dp == 128) return launch<__hip_bfloat16, 128>(p, a, to_log2, to_nat, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rk
