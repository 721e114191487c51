// Masked flash-attention forward, bf16 inputs, d_head = 64, CDNA4 MFMA.
//
// Work item = (query tile of 128 rows, head); one 256-thread workgroup
// (4 wave64s, 32 query rows per wave).  The item walks the plan's CSR of
// non-empty 64-key tiles in ascending order; EMPTY tiles are never touched
// and the per-element mask runs on PARTIAL tiles only.
//
// Per 64-key tile and wave:
//   S^T (64 keys x 32 queries) = K_tile (64 x 64) * Q_w^T   8 x mfma 32x32x16 bf16
//   online softmax in fp32 (exp2 with log2(e) folded into the scale; the
//   running max is only moved, and O rescaled, when it grows by > 2^8)
//   O^T (64 d x 32 queries) += V_tile^T * P^T               8 x mfma 32x32x16 bf16
// Computing the transposed products puts one query per lane (lane % 32) in
// both accumulators, so the row max needs one exchange with lane ^ 32 and
// the rescale of O by exp2(m_old - m_new) is lane-local.
//
// Operand layouts (v_mfma_f32_32x32x16_bf16, lane l, half h = l / 32):
//   A[m][k]: lane holds m = l % 32, k = 8h .. 8h+7
//   B[k][n]: lane holds n = l % 32, k = 8h .. 8h+7
//   D[m][n]: lane holds n = l % 32, m = 8 (r/4) + 4h + (r%4), r = 0..15
// For P^T V^T the 16-key slice of step s is consumed in the key order that
// the S^T accumulator already holds (k = 8h + e  ->  key 16 s + 8 (e/4) +
// 4h + e%4); V^T is read from LDS in the same order, so P never moves
// between lanes.
//
// LDS (double-buffered, one barrier per tile):
//   K  [64 keys][72]  row-major, 16-byte rows padded to avoid conflicts
//   V^T[64 d][68]     transposed while staging; word index XOR 8 on rows
//                     16..31 / 48..63 spreads the transposing stores
// Q is rotated by time RoPE while it is loaded (fp32, hardware sin/cos on a
// phase reduced to [-1/2, 1/2] revolution); K arrives pre-rotated.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 64;
constexpr int KS = 72;  // K row stride (elements)
constexpr int VS = 68;  // V^T row stride (elements)
constexpr int KBUF = kTileK * KS;
constexpr int VBUF = D * VS;
constexpr float kRescaleLog2 = 8.f;

struct PlanView {
  const ReqMeta* req;
  const int32_t* qt_req;
  const int2* row_desc;
  const int32_t* qtile_ptr;
  const int32_t* ktile_word;
  const int32_t* sched;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

// V^T physical word of (row d, logical word w): XOR 8 on rows with bit 4 set.
__device__ __forceinline__ int vt_word(int d, int w) { return w ^ (((d >> 4) & 1) << 3); }

__global__ __launch_bounds__(256, 2) void attn_mfma_bf16_d64_kernel(PlanView P, AttnLaunch A) {
  __shared__ __attribute__((aligned(16))) unsigned short Ks[2 * KBUF];
  __shared__ __attribute__((aligned(16))) unsigned short Vt[2 * VBUF];
  __shared__ double wtab[D / 2];

  const int item = P.sched[blockIdx.x];
  if (item < 0) return;
  const int qg = item / A.H;
  const int head = item - qg * A.H;
  const int req = P.qt_req[qg];
  const ReqMeta m = P.req[req];
  const int qt = qg - m.qt_off;
  const int L = m.len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int hh = lane >> 5;   // lane half
  const int li = lane & 31;   // query column of this lane
  const int row = qt * kTileQ + wv * 32 + li;
  const bool rvalid = row < L;
  const int tokq = m.tok_off + row;

  if (A.rope_q && tid < D / 2) wtab[tid] = A.tab.w_rev[tid];
  __syncthreads();

  // ---- Q fragment: lane holds Q[row][16 s + 8 hh .. +7] for s = 0..3
  bf16x8 qb[4];
  {
    const unsigned short* Qp = (const unsigned short*)A.q + (int64_t)tokq * A.q_st + (int64_t)head * A.q_sh;
    double dtd = 0.0;
    if (A.rope_q && rvalid) dtd = (double)(A.ts[tokq] - A.anchors[req]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (rvalid) raw = *(const uint4*)(Qp + 16 * s + 8 * hh);
      if (A.rope_q) {
        unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * s + 4 * hh + j;  // pair index
          const double rev = dtd * wtab[i];
          const float f = (float)(rev - rint(rev));
          const float sn = __builtin_amdgcn_sinf(f);
          const float cs = __builtin_amdgcn_cosf(f);
          const float x0 = bf_lo(w[j]), x1 = bf_hi(w[j]);
          w[j] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
        }
        raw = make_uint4(w[0], w[1], w[2], w[3]);
      }
      qb[s] = as_bf16x8(raw);
    }
  }

  int lo = 0, hi = 0, self = 0;
  if (rvalid) {
    const int2 dsc = P.row_desc[tokq];
    lo = dsc.x;
    hi = dsc.y & 0x7fffffff;
    self = dsc.y < 0;
  }

  // ---- staging roles
  const int kk = tid >> 3;       // K: keys kk and kk + 32
  const int kpart = tid & 7;     // 8-element slice of d
  const int vp = tid >> 3;       // V: key pair (2 vp, 2 vp + 1)
  const int vpart = tid & 7;
  const unsigned short* Kb = (const unsigned short*)A.k + (int64_t)m.tok_off * A.k_st + (int64_t)head * A.k_sh;
  const unsigned short* Vb = (const unsigned short*)A.v + (int64_t)m.tok_off * A.v_st + (int64_t)head * A.v_sh;

  // per-thread element offsets inside a key tile (loop invariant)
  const int64_t ko0 = (int64_t)kk * A.k_st + 8 * kpart;
  const int64_t ko1 = (int64_t)(kk + 32) * A.k_st + 8 * kpart;
  const int64_t vo0 = (int64_t)(2 * vp) * A.v_st + 8 * vpart;
  const int64_t vo1 = (int64_t)(2 * vp + 1) * A.v_st + 8 * vpart;
  uint4 rk0, rk1, rv0, rv1;
  // Loads are unconditional so the compiler can count them: rows past the
  // end of the request (ragged last tile only) re-read the last row, whose
  // finite values meet a -inf score (that tile is always PARTIAL) and P = 0.
  auto gload = [&](int kt) {
    const int c0 = kt * kTileK;
    const unsigned short* kb = Kb + (int64_t)c0 * A.k_st;
    const unsigned short* vb = Vb + (int64_t)c0 * A.v_st;
    if (c0 + kTileK <= L) {
      rk0 = *(const uint4*)(kb + ko0);
      rk1 = *(const uint4*)(kb + ko1);
      rv0 = *(const uint4*)(vb + vo0);
      rv1 = *(const uint4*)(vb + vo1);
    } else {
      const int last = L - 1 - c0;
      rk0 = *(const uint4*)(kb + (int64_t)min(kk, last) * A.k_st + 8 * kpart);
      rk1 = *(const uint4*)(kb + (int64_t)min(kk + 32, last) * A.k_st + 8 * kpart);
      rv0 = *(const uint4*)(vb + (int64_t)min(2 * vp, last) * A.v_st + 8 * vpart);
      rv1 = *(const uint4*)(vb + (int64_t)min(2 * vp + 1, last) * A.v_st + 8 * vpart);
    }
  };
  auto lstore = [&](int buf) {
    *(uint4*)&Ks[buf * KBUF + kk * KS + 8 * kpart] = rk0;
    *(uint4*)&Ks[buf * KBUF + (kk + 32) * KS + 8 * kpart] = rk1;
    unsigned* vt = (unsigned*)&Vt[buf * VBUF];
    const unsigned a[4] = {rv0.x, rv0.y, rv0.z, rv0.w};
    const unsigned b[4] = {rv1.x, rv1.y, rv1.z, rv1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 8 * vpart + 2 * j;
      // element (key 2vp, d0) pairs with (key 2vp+1, d0) into one word
      vt[d0 * (VS / 2) + vt_word(d0, vp)] = (a[j] & 0xffffu) | (b[j] << 16);
      vt[(d0 + 1) * (VS / 2) + vt_word(d0 + 1, vp)] = (a[j] >> 16) | (b[j] & 0xffff0000u);
    }
  };

  f32x16 o0, o1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { o0[r] = 0.f; o1[r] = 0.f; }
  float mref = -INFINITY, lsum = 0.f;
  const float sl2 = A.scale * 1.4426950408889634f;
  const float thr = kRescaleLog2 / sl2;  // in raw score units

  const int e0 = P.qtile_ptr[qg];
  const int n = P.qtile_ptr[qg + 1] - e0;
  // CSR words are software-pipelined two tiles ahead and the prefetch is
  // unconditional (the last iteration re-reads its own tile into the idle
  // buffer), so the loop body has no data-dependent branches around loads.
  int kw_cur = 0, kw_nxt = 0;
  if (n > 0) {
    kw_cur = P.ktile_word[e0];
    kw_nxt = P.ktile_word[e0 + min(1, n - 1)];
    gload(kw_cur & 0x7fffffff);
    lstore(0);
  }
  // Everything loaded before the loop (Q fragment, row descriptor) is
  // complete here, so inside the loop only the next tile's prefetch is
  // outstanding when the MFMAs start.
  asm volatile("s_waitcnt vmcnt(0)");
  __syncthreads();

  for (int it = 0; it < n; ++it) {
    const int buf = it & 1;
    const int kt = kw_cur & 0x7fffffff;
    const bool partial = kw_cur < 0;
    gload(kw_nxt & 0x7fffffff);
    const int kw_nn = P.ktile_word[e0 + min(it + 2, n - 1)];

    // S^T = K Q^T
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
    const unsigned short* kb = &Ks[buf * KBUF];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 a0 = as_bf16x8(*(const uint4*)&kb[li * KS + 16 * s + 8 * hh]);
      const bf16x8 a1 = as_bf16x8(*(const uint4*)&kb[(32 + li) * KS + 16 * s + 8 * hh]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[s], s1, 0, 0, 0);
    }

    if (partial) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * kTileK + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool v0 = (key >= lo && key < hi) || (self && key == row);
        const bool v1 = (key + 32 >= lo && key + 32 < hi) || (self && key + 32 == row);
        if (!v0) s0[r] = -INFINITY;
        if (!v1) s1[r] = -INFINITY;
      }
    }

    float mx = s0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescale: the reference max m_ref only moves when a row's max
    // exceeds it by more than kRescaleLog2 (in log2 units), so P <= 2^8.
    // The decision is made for the whole wave at once.
    const float mnew = fmaxf(mref, mx);
    const bool grow = mnew > mref + thr;
    if (__any(grow)) {
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mref - mnew) * sl2);
      lsum *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) { o0[r] *= alpha; o1[r] *= alpha; }
      mref = mnew;
    }
    const float nb = mref == -INFINITY ? 0.f : -mref * sl2;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], sl2, nb));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], sl2, nb));
      psum += s0[r] + s1[r];
    }
    lsum += psum;

    // P^T as B operands: step s takes accumulator block s/2, registers
    // 8 (s%2) .. 8 (s%2) + 7
    bf16x8 pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x16& src = (s < 2) ? s0 : s1;
      const int r0 = 8 * (s & 1);
      const uint4 w = make_uint4(pack_bf16x2(src[r0 + 0], src[r0 + 1]),
                                 pack_bf16x2(src[r0 + 2], src[r0 + 3]),
                                 pack_bf16x2(src[r0 + 4], src[r0 + 5]),
                                 pack_bf16x2(src[r0 + 6], src[r0 + 7]));
      pb[s] = as_bf16x8(w);
    }

    // O^T += V^T P^T
    const unsigned* vt = (const unsigned*)&Vt[buf * VBUF];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int w0 = 8 * s + 2 * hh;  // keys 16 s + 4 hh .. +3  (logical words w0, w0+1)
      {
        const int d = li;
        const unsigned* rowp = vt + d * (VS / 2);
        const uint2 x = *(const uint2*)(rowp + vt_word(d, w0));
        const uint2 y = *(const uint2*)(rowp + vt_word(d, w0 + 4));
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(x.x, x.y, y.x, y.y)), pb[s], o0, 0, 0, 0);
      }
      {
        const int d = 32 + li;
        const unsigned* rowp = vt + d * (VS / 2);
        const uint2 x = *(const uint2*)(rowp + vt_word(d, w0));
        const uint2 y = *(const uint2*)(rowp + vt_word(d, w0 + 4));
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(x.x, x.y, y.x, y.y)), pb[s], o1, 0, 0, 0);
      }
    }

    lstore(buf ^ 1);
    __syncthreads();
    kw_cur = kw_nxt;
    kw_nxt = kw_nn;
  }

  // ---- epilogue: O = O^T / l, lanes of both halves hold distinct d values
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (!rvalid) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  unsigned short* Op = (unsigned short*)A.o + (int64_t)tokq * A.o_st + (int64_t)head * A.o_sh;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int d = 8 * g + 4 * hh;
    *(uint2*)(Op + d) = make_uint2(pack_bf16x2(o0[4 * g] * inv, o0[4 * g + 1] * inv),
                                   pack_bf16x2(o0[4 * g + 2] * inv, o0[4 * g + 3] * inv));
    *(uint2*)(Op + 32 + d) = make_uint2(pack_bf16x2(o1[4 * g] * inv, o1[4 * g + 1] * inv),
                                        pack_bf16x2(o1[4 * g + 2] * inv, o1[4 * g + 3] * inv));
  }
  if (A.lse && hh == 0)
    A.lse[(int64_t)head * A.T + tokq] = ltot > 0.f ? mref * A.scale + logf(ltot) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_mfma_bf16_d64(const rk_plan* p, const AttnLaunch& a, hipStream_t s) {
  if (p->slots == 0) return hipSuccess;
  PlanView P{p->dev.req, p->dev.qt_req, p->dev.row_desc, p->dev.qtile_ptr, p->dev.ktile_word,
             p->dev.sched};
  hipLaunchKernelGGL(attn_mfma_bf16_d64_kernel, dim3((unsigned)p->slots), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace rk
