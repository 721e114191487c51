// Masked flash-attention forward, bf16 inputs, d_head = 64, CDNA4 MFMA.
//
// Work item = (query tile of 128 rows, head); one 256-thread workgroup
// (4 wave64s, 32 query rows per wave).  The item walks the plan's CSR of
// non-empty 64-key tiles in ascending order; EMPTY tiles are never touched
// and the per-element mask runs on PARTIAL tiles only.
//
// Per 64-key tile and wave:
//   S^T (64 keys x 32 queries) = K_tile (64 x 64) * Q_w^T      8 x mfma 32x32x16
//   P = exp2(S - m), packed to bf16; row sum in fp32
//   O^T (64 d x 32 queries) += V_tile^T * P^T                  8 x mfma 32x32x16
// With time RoPE, Q is loaded pre-multiplied by scale * log2(e) (folded in
// before its single bf16 rounding), so the scores come out of the matrix
// core in log2 units.  m is the row's reference (0 at the start); it is
// not tracked per tile but re-derived from the tile's scores only when a
// lane's tile sum of P exceeds 2^32 or is not a number, or falls below
// 2^-32 while the lane has accumulated nothing.  Any P kept is therefore
// <= 2^32, far from fp32 overflow, and bf16 P keeps its relative precision
// at any magnitude.
//
// Operand layouts (v_mfma_f32_32x32x16_bf16, lane l, half h = l / 32):
//   A[m][k]: lane holds m = l % 32, k = 8h .. 8h+7
//   B[k][n]: lane holds n = l % 32, k = 8h .. 8h+7
//   D[m][n]: lane holds n = l % 32, m = 8 (r/4) + 4h + (r%4), r = 0..15
// Computing the transposed products puts one query per lane (lane % 32) in
// both accumulators; the two lane halves hold different keys of the same
// query.  For P^T V^T the 16-key slice of step s is consumed in the key
// order the S^T accumulator already holds (k = 8h + e  ->  key 16 s +
// 8 (e/4) + 4h + e%4); V^T is read in that order with transposing LDS
// reads, so P never moves between lanes.
//
// LDS: three stages of K and V tiles (64 rows x 128 bytes each, unpadded,
// XOR-swizzled 16-byte chunks, 48 KB per workgroup), filled by buffer loads
// that write LDS directly two tiles ahead of their use; one barrier per
// tile.  Q is rotated by time RoPE while it is
// loaded (fp32, hardware sin/cos on a phase reduced to [-1/2, 1/2]
// revolution); K arrives pre-rotated.
#include <hip/hip_bf16.h>

#include "rk_internal.h"

namespace rk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile geometry for d_head D (64 or 128): a K or V tile is 64 rows of 2 D
// bytes (8 KB at d = 64); each wave moves D / 32 one-kilobyte pieces of it.
template <int D>
constexpr int tile_elems() { return kTileK * D; }
template <int D>
constexpr int wave_copies() { return D / 32; }
// A lane's tile sum above this (or not a number) makes the wave re-derive
// the reference max.
constexpr float kMaxTileSum = 4294967296.f;  // 2^32
// A lane with nothing accumulated whose tile sum is below this re-derives
// the reference max (the row's P would otherwise lose range).
constexpr float kMinTileSum = 2.3283064365386963e-10f;  // 2^-32
[[maybe_unused]] constexpr unsigned kBufferFlags = 0x00020000u;  // raw buffer, 32-bit data format

struct PlanView {
  const ItemRec* irec;  // launch slot -> item record
  const int2* row_desc;
  const int32_t* ktile_word;
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


template <typename T>
__device__ __forceinline__ T ldc(const T* p, int64_t i) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(4))) T*)p)[i];
#else
  return p[i];  // host pass of the single-source compile; never executed
#endif
}

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef short v4i16 __attribute__((ext_vector_type(4)));

// LDS tiles hold 64 rows of 2 D bytes (D / 8 sixteen-byte slots), unpadded.
// Logical 16-byte chunk c of row r sits in slot c ^ kswz(r) for K and
// c ^ vswz(r) for V.  gfx950's LDS serves a ds_read_b128 sixteen lanes at a
// time over 64 four-byte banks (256 bytes), so
//  - at D = 64 the 16 rows a lane group reads at one chunk (two rows per
//    256-byte bank line) must take 8 distinct slots among the even rows and
//    among the odd rows: kswz(r) = (r / 2) mod 8 (r mod 8 would put rows r
//    and r + 8 on the same banks: a two-way conflict the LDS counters
//    showed on every K read);
//  - at D = 128 a row fills the bank line, so the 16 rows take 16 distinct
//    slots: kswz(r) = r mod 16;
//  - a ds_read_b64_tr_b16 group (4 consecutive V rows starting at a
//    multiple of 4, 2 chunks each) takes 8 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 64 ? (r >> 1) & 7 : r & 15; }
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }

// Q fragment: lane holds Q[row][16 s + 8 hh .. +7] * qmul, s = 0..3,
// rotated by time RoPE when asked (fp32 math, hardware sin/cos on a phase
// reduced to [-1/2, 1/2] revolution), rounded once to bf16.  The raw
// loads are issued first (QRaw) and consumed later (finish_q), so that the
// first key tile's copies are in flight while Q arrives and is rotated.
template <int D>
struct QRaw {
  uint4 v[D / 16];
  int64_t t;  // timestamp of the row
  int2 dsc;   // row descriptor
};

// A row past the end of the request reads the request's last token and is
// zeroed in finish_q (it is never written).  Chunks past d_head (a padded
// instance) are not read and are zero.
template <int D>
__device__ __forceinline__ QRaw<D> load_q_raw(const AttnLaunch& A, const int2* row_desc,
                                              int tokq_c, int head, int hh, bool rope, int d) {
  QRaw<D> r;
  const unsigned short* Qp = (const unsigned short*)A.q + (int64_t)tokq_c * A.q_st + (int64_t)head * A.q_sh;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    r.v[s] = 16 * s + 8 * hh < d ? *(const uint4*)(Qp + 16 * s + 8 * hh) : make_uint4(0, 0, 0, 0);
  r.t = rope ? A.ts[tokq_c] : 0;
  r.dsc = row_desc[tokq_c];
  return r;
}

// With kNorm (QK Norm) the row is first scaled by 1 / sqrt(mean(x^2) + eps)
// and the gain gamma[d] (NULL: 1); the two lane halves hold the two halves
// of the row and meet through one lane ^ 32 exchange.
template <bool kRope, bool kNorm, int D>
__device__ __forceinline__ void finish_q(bf16x8 (&qb)[D / 16], const QRaw<D>& raw, bool valid,
                                         int64_t anchor, const RopeTab& tab, int hh, float qmul,
                                         float eps, const float* gamma) {
  const double dtd = (double)(raw.t - anchor);
  float nscale[D / 16][8];
  if (kNorm) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const unsigned w[4] = {raw.v[s].x, raw.v[s].y, raw.v[s].z, raw.v[s].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ss = fmaf(bf_lo(w[j]), bf_lo(w[j]), ss);
        ss = fmaf(bf_hi(w[j]), bf_hi(w[j]), ss);
      }
    }
    ss += __shfl_xor(ss, 32, 64);
    const float rstd = rsqrtf(ss * (1.f / D) + eps);  // QK Norm runs only with d == D
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      float4 g0 = make_float4(1.f, 1.f, 1.f, 1.f), g1 = g0;
      if (gamma) {
        g0 = *(const float4*)(gamma + 16 * s + 8 * hh);
        g1 = *(const float4*)(gamma + 16 * s + 8 * hh + 4);
      }
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) nscale[s][e] = rstd * gv[e];
    }
  }
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    unsigned w[4] = {raw.v[s].x, raw.v[s].y, raw.v[s].z, raw.v[s].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x0 = bf_lo(w[j]), x1 = bf_hi(w[j]);
      if (kNorm) {
        x0 *= nscale[s][2 * j];
        x1 *= nscale[s][2 * j + 1];
      }
      if (kRope) {
        // pair 8 s + 4 hh + j: both candidates are uniform loads, hh picks
        const double w = hh ? tab.w_rev[8 * s + 4 + j] : tab.w_rev[8 * s + j];
        const double rev = dtd * w;
        const float f = (float)(rev - rint(rev));
        const float sn = __builtin_amdgcn_sinf(f);
        const float cs = __builtin_amdgcn_cosf(f);
        const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
        x0 = y0;
        x1 = y1;
      }
      w[j] = valid ? pack_bf16x2(x0 * qmul, x1 * qmul) : 0u;
    }
    qb[s] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// Per-lane byte offsets of the direct buffer -> LDS copies.  A wave's
// 16-byte-per-lane buffer load with the LDS bit fills 1 KB of LDS
// contiguously (lane l at byte 16 l): 512 / D rows of D / 8 chunks (8 rows
// at d = 64).  Wave w issues copies j = 0 .. D / 32 - 1, piece
// (D / 32) w + j of both the K and the V tile; the offsets are relative to
// the tile's first row and do not change.  A chunk past d_head (a padded
// instance) gets an offset past every buffer's range: its copy loads
// nothing from memory and its LDS slot keeps the zero it was given.
constexpr unsigned kOutOfRange = 0x80000000u;
template <int D>
struct CopyMap {
  unsigned koff[D / 32];
  unsigned voff[D / 32];
};

template <int D>
__device__ __forceinline__ CopyMap<D> copy_map(int wv, int lane, unsigned kst_b, unsigned vst_b,
                                                int d) {
  CopyMap<D> c;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int q = (D / 32 * wv + j) * 64 + lane;
    const int r = q / (D / 8), slot = q % (D / 8);
    // lane q writes physical slot q % (D / 8) of row r: logical chunk slot ^ swizzle
    const int ck = slot ^ kswz<D>(r), cv = slot ^ vswz(r);
    c.koff[j] = 8 * ck < d ? (unsigned)r * kst_b + 16u * (unsigned)ck : kOutOfRange;
    c.voff[j] = 8 * cv < d ? (unsigned)r * vst_b + 16u * (unsigned)cv : kOutOfRange;
  }
  return c;
}

// Issue the copies of key tile kt into LDS buffers kd / vd.  The buffer
// descriptor of each tile ends at the last byte of its last token, so the
// rows past the end of the request (ragged last tile only) are out of
// range and load zeros; that tile is always PARTIAL, so their scores are
// masked.
template <int D>
__device__ __forceinline__ void tile_copy(unsigned short* kd, unsigned short* vd, const CopyMap<D>& c,
                                          const char* Kb, const char* Vb, unsigned kst_b,
                                          unsigned vst_b, int kt, int L, int wv) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins do not exist in the host pass
  const int c0 = kt * kTileK;
  const unsigned last = (unsigned)min(L - c0, kTileK) - 1u;  // last row inside the request
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Kb + (int64_t)c0 * kst_b), 0, (int)(last * kst_b + 2u * D), (int)kBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Vb + (int64_t)c0 * vst_b), 0, (int)(last * vst_b + 2u * D), (int)kBufferFlags);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, LDS_PTR(void, kd + (D / 32 * wv + j) * 512), 16,
                                             c.koff[j], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, LDS_PTR(void, vd + (D / 32 * wv + j) * 512), 16,
                                             c.voff[j], 0, 0, 0);
  }
#endif
}

// Mask of one tile on the S^T accumulators: the lane's query sees key
// c0 + 8 g + 4 hh + e (g, e = 0..3) in register 4 g + e of s0, and that key
// + 32 in s1.  The visible keys of the row inside the tile, as a 64-bit
// set, are its interval [lo, hi) clipped to the tile plus, for a candidate,
// its own position; after a shift by 4 hh, register r of s0 tests bit
// 8 (r / 4) + r % 4 of the low word and s1 the same bit of the high word.
// A hidden score becomes -inf by a bit select against the sign-extended
// test bit (no lane masks involved).
__device__ __forceinline__ void mask_tile(f32x16& s0, f32x16& s1, int kt, int hh, int lo, int hi,
                                          int self, int row) {
  const int c0 = kt * kTileK;
  const int a = min(max(lo - c0, 0), kTileK), b = min(max(hi - c0, 0), kTileK);
  const uint64_t below_b = b >= 64 ? ~0ull : (1ull << b) - 1ull;
  const uint64_t below_a = a >= 64 ? ~0ull : (1ull << a) - 1ull;
  uint64_t vis = below_b & ~below_a;
  const int sr = row - c0;
  if (self && sr >= 0 && sr < kTileK) vis |= 1ull << sr;
  vis >>= 4 * hh;
  const int w0 = (int)(unsigned)vis, w1 = (int)(unsigned)(vis >> 32);
  const int ninf = (int)0xff800000u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const unsigned bit = 8u * (unsigned)(r >> 2) + (unsigned)(r & 3);
    const int m0 = __builtin_amdgcn_sbfe(w0, bit, 1u);  // 0 or -1
    const int m1 = __builtin_amdgcn_sbfe(w1, bit, 1u);
    s0[r] = __int_as_float((__float_as_int(s0[r]) & m0) | (ninf & ~m0));
    s1[r] = __int_as_float((__float_as_int(s1[r]) & m1) | (ninf & ~m1));
  }
}

// S^T = K Q^T + c for the wave's 32 queries (c: initial accumulator).
template <int D>
__device__ __forceinline__ void scores(f32x16& s0, f32x16& s1, const unsigned short* kb,
                                       const bf16x8 (&q)[D / 16], const f32x16& c, int li,
                                       int hh) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int cc = 2 * s + hh;  // logical chunk: d = 16 s + 8 hh .. +7
    const bf16x8 k0 = as_bf16x8(*(const uint4*)&kb[li * D + 8 * (cc ^ kswz<D>(li))]);
    const bf16x8 k1 = as_bf16x8(*(const uint4*)&kb[(32 + li) * D + 8 * (cc ^ kswz<D>(32 + li))]);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q[s], s == 0 ? c : s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, q[s], s == 0 ? c : s1, 0, 0, 0);
  }
}

// P = exp2((S - sh) * mul) (sh only when kShift, mul only when kScale),
// packed to bf16 as the B operands of the PV product (step s: accumulator
// block s/2, registers 8 (s%2)..+7).  S is left as it is.  Returns the
// lane's sum of the fp32 values (plain adds: they issue alongside the
// matrix cores, unlike the packed-bf16 dot products).
template <bool kShift, bool kScale>
__device__ __forceinline__ float probs(bf16x8 (&pb)[4], const f32x16& s0, const f32x16& s1,
                                       float sh, float mul) {
  float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f32x16& src = (s < 2) ? s0 : s1;
    const int r0 = 8 * (s & 1);
    bf16x2_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x0 = src[r0 + 2 * j], x1 = src[r0 + 2 * j + 1];
      if (kShift) { x0 -= sh; x1 -= sh; }
      if (kScale) { x0 *= mul; x1 *= mul; }
      const float p0 = __builtin_amdgcn_exp2f(x0), p1 = __builtin_amdgcn_exp2f(x1);
      w[j][0] = (__bf16)p0;
      w[j][1] = (__bf16)p1;
      sum0 += p0;
      sum1 += p1;
    }
    __builtin_memcpy(&pb[s], w, 16);
  }
  return sum0 + sum1;
}

// Does query `row` see any key of tile kt?  Every row of a FULL tile does;
// on a PARTIAL tile, its interval [lo, hi) or its own position must fall in
// the tile.
__device__ __forceinline__ bool row_sees(int kt, bool partial, int lo, int hi, int self, int row) {
  const int c0 = kt * kTileK;
  return !partial || (lo < c0 + kTileK && hi > c0) || (self && row >= c0 && row < c0 + kTileK);
}

// Scores of tile kt from K in global memory: the same bf16 rows in the same
// product order as from LDS, so the same values.  Rows past the request's
// end read its last row; the tile is then PARTIAL and they are masked.
template <int D>
__device__ __forceinline__ void scores_global(f32x16& s0, f32x16& s1, const unsigned short* Kh,
                                              int64_t k_st, int kt, int L, int d,
                                              const bf16x8 (&q)[D / 16], const f32x16& negm,
                                              int li, int hh) {
  const int c0 = kt * kTileK;
  const unsigned short* r0 = Kh + (int64_t)min(c0 + li, L - 1) * k_st + 8 * hh;
  const unsigned short* r1 = Kh + (int64_t)min(c0 + 32 + li, L - 1) * k_st + 8 * hh;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    // chunks past d_head are zero, as in LDS
    const bool in = 16 * s + 8 * hh < d;
    const bf16x8 k0 = as_bf16x8(in ? *(const uint4*)(r0 + 16 * s) : make_uint4(0, 0, 0, 0));
    const bf16x8 k1 = as_bf16x8(in ? *(const uint4*)(r1 + 16 * s) : make_uint4(0, 0, 0, 0));
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q[s], s == 0 ? negm : s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, q[s], s == 0 ? negm : s1, 0, 0, 0);
  }
}

// O^T accumulators of one wave, 32 d values per block (d = 64 uses the first
// two).  Named members rather than an array: an array indexed by a loop
// counter stays in memory until the loops are unrolled, and the register
// allocation that comes out of that is much larger.
struct OAcc {
  f32x16 b0, b1, b2, b3;
};

__device__ __forceinline__ f32x16 acc_get(const OAcc& o, int mb) {
  return mb == 0 ? o.b0 : mb == 1 ? o.b1 : mb == 2 ? o.b2 : o.b3;
}

__device__ __forceinline__ void acc_mfma(OAcc& o, int mb, const bf16x8& a, const bf16x8& b) {
  if (mb == 0)
    o.b0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o.b0, 0, 0, 0);
  else if (mb == 1)
    o.b1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o.b1, 0, 0, 0);
  else if (mb == 2)
    o.b2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o.b2, 0, 0, 0);
  else
    o.b3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o.b3, 0, 0, 0);
}

// One 64-key tile for one wave (32 queries): scores, mask, P, O^T += V^T
// P^T.  kb / vb are the tile's LDS buffers.  Scores are in log2 units when
// kPreScaled (Q carries scale * log2(e)); otherwise they are raw dot
// products and mul = scale * log2(e) is applied before exp2.
//
// The QK product starts from negm, which holds -m for the lane's row in
// all 16 registers (m starts at 0), so the fast path takes P = exp2(S) as
// it comes out of the matrix core.  The wave re-derives the reference from
// this tile's shifted scores instead when a lane's tile sum exceeds 2^32
// (or is not a number), or when a lane that has accumulated nothing sees a
// key of this tile and its sum is below 2^-32 (P would lose range).  A row
// with nothing accumulated (O = 0 and l = 0) moves m to the tile's max, up
// or down; any other row moves m up by the tile's excess over it, with O
// and l rescaled.  That path recomputes the tile's scores from K in global
// memory, so the scores need not stay live once P is packed.
template <bool kPreScaled, int D>
__device__ __forceinline__ void tile_step(OAcc& o, f32x16& negm, float& mref,
                                          float& lsum, const unsigned short* kb,
                                          const unsigned short* vb, const bf16x8 (&q)[D / 16],
                                          int kt,
                                          bool partial, int li, int hh, int lo, int hi, int self,
                                          int row, float mul, const unsigned short* Kh,
                                          int64_t k_st, int L, int d) {
  f32x16 s0, s1;
  scores<D>(s0, s1, kb, q, negm, li, hh);
  if (partial) mask_tile(s0, s1, kt, hh, lo, hi, self, row);
  bf16x8 pb[4];
  float ts = probs<false, !kPreScaled>(pb, s0, s1, 0.f, mul);
  const bool big = !(ts <= kMaxTileSum);
  const bool tiny =
      lsum == 0.f && ts < kMinTileSum && row_sees(kt, partial, lo, hi, self, row);
  if (__any(big || tiny)) {
    // the scores are recomputed, so they need not stay live past the packing
    scores_global<D>(s0, s1, Kh, k_st, kt, L, d, q, negm, li, hh);
    if (partial) mask_tile(s0, s1, kt, hh, lo, hi, self, row);
    float mx = s0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float lrow = lsum + __shfl_xor(lsum, 32, 64);
    float sh;
    if (lrow == 0.f) {
      sh = mx == -INFINITY ? 0.f : mx;  // nothing of this tile visible: m stays
    } else {
      sh = fmaxf(mx, 0.f);
      if (sh > 0.f) {
        const float alpha = __builtin_amdgcn_exp2f(kPreScaled ? -sh : -sh * mul);
        lsum *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          o.b0[r] *= alpha;
          o.b1[r] *= alpha;
          if (D > 64) {
            o.b2[r] *= alpha;
            o.b3[r] *= alpha;
          }
        }
      }
    }
    mref += sh;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] -= sh;
    ts = probs<true, !kPreScaled>(pb, s0, s1, sh, mul);
  }
  lsum += ts;

  // V^T fragments by transposing reads: in each 16-lane group g, lane i
  // points at V[k + (i >> 2)][d0 + 4 (i & 3)] and receives V[k..k+3][d0 + i].
  const int g = (li >> 4) + 2 * hh;  // 16-lane group of this lane
  const int i = li & 15;
  const int rr = i >> 2;             // row offset inside the 4-row group
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const int d0 = 32 * mb + 16 * (g & 1);
      const int col = d0 + 4 * (i & 3);
      const int ka = 16 * s + 4 * hh + rr;      // keys for e = 0..3
      const int kb2 = ka + 8;                   // keys for e = 4..7
      const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(v4i16, &vb[ka * D + 8 * ((col >> 3) ^ vswz(ka)) + (col & 7)]));
      const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(v4i16, &vb[kb2 * D + 8 * ((col >> 3) ^ vswz(kb2)) + (col & 7)]));
      bf16x8 va;
      __builtin_memcpy(&va, &lo4, 8);
      __builtin_memcpy((char*)&va + 8, &hi4, 8);
      acc_mfma(o, mb, va, pb[s]);
    }
  }
}

// End of a pipeline step: this wave's copies other than its four most
// recent (the step's own) have landed and its LDS reads are done
// (vmcnt(4) lgkmcnt(0)), then the workgroup meets.  A bare barrier: the
// fence of __syncthreads would also wait for the copies still in flight.
// The empty asm statements keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0074u);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kThreads = 256;  // 4 waves, 32 query rows each

// kPreScaled: Q is rotated by time RoPE in the kernel and rounded to bf16
// anyway, so scale * log2(e) is folded in before that single rounding.
// Without RoPE, Q is used exactly as given and the scale is applied to the
// fp32 scores instead.
//
// d = 64 keeps three LDS stages (48 KB, three workgroups per CU); d = 128
// keeps two (64 KB, two workgroups per CU, which is also what its registers
// allow), so a copy has one step to land instead of two.
//
// kPad: d_head is below D (a padded instance); the exact instances keep no
// trace of the padding logic.
template <bool kPreScaled, bool kNorm, int D, bool kPad>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_bf16_kernel(PlanView P, AttnLaunch A) {
  constexpr int kStages = D <= 64 ? 3 : 2;
  constexpr int kTile = tile_elems<D>();
  constexpr int kWc = wave_copies<D>();
  // The stages as separate objects, so the compiler can tell the buffers
  // being filled from the one being read.
  __shared__ __attribute__((aligned(1024))) unsigned short K0[kTile], K1[kTile],
      K2[kStages == 3 ? kTile : 8];
  __shared__ __attribute__((aligned(1024))) unsigned short V0[kTile], V1[kTile],
      V2[kStages == 3 ? kTile : 8];

  const int dh = kPad ? A.d : D;  // d_head
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  // Each wave zeroes the V rows its own copies fill (pieces kWc wv .. +kWc
  // - 1 of every stage) and waits for those writes before its first copy:
  // whatever a copy leaves unwritten then stays finite, so a masked key
  // (P = 0) adds exactly 0 to O.  No other wave touches these rows, so no
  // barrier.  This comes first, while the only memory accesses in flight
  // are the slot's own record and arguments, so the wait delays nothing.
  // A padded instance (d_head < D) zeroes K too: its padding columns meet
  // Q's zeros in the scores.
#pragma unroll
  for (int j = 0; j < kWc; ++j) {
    *(uint4*)&V0[(kWc * wv + j) * 512 + 8 * lane] = make_uint4(0, 0, 0, 0);
    *(uint4*)&V1[(kWc * wv + j) * 512 + 8 * lane] = make_uint4(0, 0, 0, 0);
    if (kStages == 3) *(uint4*)&V2[(kWc * wv + j) * 512 + 8 * lane] = make_uint4(0, 0, 0, 0);
    if (kPad) {
      *(uint4*)&K0[(kWc * wv + j) * 512 + 8 * lane] = make_uint4(0, 0, 0, 0);
      *(uint4*)&K1[(kWc * wv + j) * 512 + 8 * lane] = make_uint4(0, 0, 0, 0);
      if (kStages == 3) *(uint4*)&K2[(kWc * wv + j) * 512 + 8 * lane] = make_uint4(0, 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  // a slot runs a whole item or a CSR range of one (split chunk)
  const ItemRec ir = ldc(P.irec, blockIdx.x);
  if (ir.head < 0) return;
  const float pz = plan_poison(A.plan_err);
  const int head = ir.head;
  const int L = ir.len;
  const int part = ir.part;

  const int hh = lane >> 5;   // lane half
  const int li = lane & 31;   // query column of this lane
  const int row = ir.row0 + wv * 32 + li;
  const bool rvalid = row < L;
  const int tokq = ir.tok_off + row;

  const float sl2 = A.scale * 1.4426950408889634f;  // scale * log2(e)
  // Q's loads go out first, then the first key tile's copies; Q is rotated
  // while those copies land.
  const QRaw<D> qraw =
      load_q_raw<D>(A, P.row_desc, ir.tok_off + min(row, L - 1), head, hh, kPreScaled, dh);
  const int64_t anchor = kPreScaled ? ldc(A.anchors, ir.req) : 0;

  const char* Kb = (const char*)((const unsigned short*)A.k + (int64_t)ir.tok_off * A.k_st + (int64_t)head * A.k_sh);
  const char* Vb = (const char*)((const unsigned short*)A.v + (int64_t)ir.tok_off * A.v_st + (int64_t)head * A.v_sh);
  // row strides in bytes (32-bit per-lane offsets: the host limits strides)
  const unsigned kst_b = (unsigned)A.k_st * 2u, vst_b = (unsigned)A.v_st * 2u;
  const CopyMap<D> cm = copy_map<D>(wv, lane, kst_b, vst_b, dh);
  OAcc o;
  f32x16 negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;
  o.b0 = o.b1 = o.b2 = o.b3 = negm;
  float mref = 0.f, lsum = 0.f;

  const int e0 = ir.e0;
  const int n = ir.n;
  // Three stages: step i computes tile i from stage i % 3 while the copies
  // of tile i + 2 fill stage (i + 2) % 3 (which held tile i - 1): every copy
  // has two steps to land.  The wait before the barrier that ends step i
  // leaves the step's own copies (two of K, two of V per wave) in flight and
  // covers those of tile i + 1.  The loop is unrolled by three so each stage
  // is a distinct LDS object.  Two stages: step i computes tile i while the
  // copies of tile i + 1 fill the other stage, and waits for all of them.
  // Copies past the last tile re-read the last tile into an idle stage (no
  // branch around loads; making them conditional measured slower); an item
  // without key tiles still copies the request's first tile (in bounds,
  // never read), so the copies are unconditional and Q's loads can be
  // waited for without waiting for them.
  const int w_cur0 = ir.w0;
  const int w_cur1 = ir.w1;
  int w_cur = w_cur0, w_nxt = w_cur1;
  tile_copy<D>(K0, V0, cm, Kb, Vb, kst_b, vst_b, w_cur0 & 0x7fffffff, L, wv);
  if (kStages == 3) tile_copy<D>(K1, V1, cm, Kb, Vb, kst_b, vst_b, w_cur1 & 0x7fffffff, L, wv);
  bf16x8 q[D / 16];
  finish_q<kPreScaled, kNorm, D>(q, qraw, rvalid, anchor, A.tab, hh, kPreScaled ? sl2 : 1.f,
                                 A.eps, A.gamma_q);
  const int lo = rvalid ? qraw.dsc.x : 0;
  const int hi = rvalid ? qraw.dsc.y & 0x7fffffff : 0;
  const int self = rvalid && qraw.dsc.y < 0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const unsigned short* Kh = (const unsigned short*)Kb;
  if (kStages == 3) {
    for (int it = 0; it < n; it += 3) {
      {
        const int w_nn = ldc(P.ktile_word, e0 + min(it + 2, n - 1));
        tile_copy<D>(K2, V2, cm, Kb, Vb, kst_b, vst_b, w_nn & 0x7fffffff, L, wv);
        tile_step<kPreScaled, D>(o, negm, mref, lsum, K0, V0, q, w_cur & 0x7fffffff, w_cur < 0,
                                 li, hh, lo, hi, self, row, sl2, Kh, A.k_st, L, dh);
        step_barrier();
        w_cur = w_nxt;
        w_nxt = w_nn;
      }
      if (it + 1 < n) {
        const int w_nn = ldc(P.ktile_word, e0 + min(it + 3, n - 1));
        tile_copy<D>(K0, V0, cm, Kb, Vb, kst_b, vst_b, w_nn & 0x7fffffff, L, wv);
        tile_step<kPreScaled, D>(o, negm, mref, lsum, K1, V1, q, w_cur & 0x7fffffff, w_cur < 0,
                                 li, hh, lo, hi, self, row, sl2, Kh, A.k_st, L, dh);
        step_barrier();
        w_cur = w_nxt;
        w_nxt = w_nn;
      }
      if (it + 2 < n) {
        const int w_nn = ldc(P.ktile_word, e0 + min(it + 4, n - 1));
        tile_copy<D>(K1, V1, cm, Kb, Vb, kst_b, vst_b, w_nn & 0x7fffffff, L, wv);
        tile_step<kPreScaled, D>(o, negm, mref, lsum, K2, V2, q, w_cur & 0x7fffffff, w_cur < 0,
                                 li, hh, lo, hi, self, row, sl2, Kh, A.k_st, L, dh);
        step_barrier();
        w_cur = w_nxt;
        w_nxt = w_nn;
      }
    }
  } else {
    for (int it = 0; it < n; it += 2) {
      {
        tile_copy<D>(K1, V1, cm, Kb, Vb, kst_b, vst_b, w_nxt & 0x7fffffff, L, wv);
        tile_step<kPreScaled, D>(o, negm, mref, lsum, K0, V0, q, w_cur & 0x7fffffff, w_cur < 0,
                                 li, hh, lo, hi, self, row, sl2, Kh, A.k_st, L, dh);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        w_cur = w_nxt;
        w_nxt = ldc(P.ktile_word, e0 + min(it + 2, n - 1));
      }
      if (it + 1 < n) {
        tile_copy<D>(K0, V0, cm, Kb, Vb, kst_b, vst_b, w_nxt & 0x7fffffff, L, wv);
        tile_step<kPreScaled, D>(o, negm, mref, lsum, K1, V1, q, w_cur & 0x7fffffff, w_cur < 0,
                                 li, hh, lo, hi, self, row, sl2, Kh, A.k_st, L, dh);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        w_cur = w_nxt;
        w_nxt = ldc(P.ktile_word, e0 + min(it + 3, n - 1));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy outlives the item

  // ---- epilogue: O = O^T / l; lanes of both halves hold distinct d values
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (!rvalid) return;
  if (part >= 0) {
    // partial result of a split item: O unnormalised, reference max, sum
    float* pp = A.part + (int64_t)part * (kTileQ * (D + 2));
    const int rl = wv * 32 + li;
    float* orow = pp + rl * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const f32x16 ob = acc_get(o, mb);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * mb + 8 * g + 4 * hh;
        *(float4*)(orow + d) = make_float4(ob[4 * g], ob[4 * g + 1], ob[4 * g + 2], ob[4 * g + 3]);
      }
    }
    if (hh == 0) {
      pp[kTileQ * D + rl] = ltot > 0.f ? mref : -INFINITY;  // -inf: nothing seen
      pp[kTileQ * D + kTileQ + rl] = ltot;
    }
    return;
  }
  const float inv = (ltot > 0.f ? 1.f / ltot : 0.f) * pz;
  unsigned short* Op = (unsigned short*)A.o + (int64_t)tokq * A.o_st + (int64_t)head * A.o_sh;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    const f32x16 ob = acc_get(o, mb);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * mb + 8 * g + 4 * hh;
      if (d < dh)  // columns past d_head are padding
        *(uint2*)(Op + d) = make_uint2(pack_bf16x2(ob[4 * g] * inv, ob[4 * g + 1] * inv),
                                       pack_bf16x2(ob[4 * g + 2] * inv, ob[4 * g + 3] * inv));
    }
  }
  if (A.lse && hh == 0)
    A.lse[(int64_t)head * A.T + tokq] =
        (ltot > 0.f ? mref * (kPreScaled ? 0.6931471805599453f : A.scale) + logf(ltot)
                    : -INFINITY) * pz;
}

template <int D, bool kPad>
hipError_t launch_d(const PlanView& P, const AttnLaunch& a, dim3 grid, hipStream_t s) {
  // QK Norm runs only at the exact widths
  if (a.rope_q && a.norm_q && !kPad)
    hipLaunchKernelGGL((attn_mfma_bf16_kernel<true, true, D, false>), grid, dim3(kThreads), 0, s,
                       P, a);
  else if (a.norm_q)
    return hipErrorInvalidValue;
  else if (a.rope_q)
    hipLaunchKernelGGL((attn_mfma_bf16_kernel<true, false, D, kPad>), grid, dim3(kThreads), 0, s,
                       P, a);
  else
    hipLaunchKernelGGL((attn_mfma_bf16_kernel<false, false, D, kPad>), grid, dim3(kThreads), 0, s,
                       P, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma_bf16(const rk_plan* p, const AttnLaunch& a, hipStream_t s) {
  if (p->slots == 0) return hipSuccess;
  PlanView P{p->dev.irec, p->dev.row_desc, p->dev.ktile_word};
  const dim3 grid((unsigned)p->grid);
  if (a.d > a.dp) return hipErrorInvalidValue;
  if (a.dp == 128) return a.d == 128 ? launch_d<128, false>(P, a, grid, s)
                                      : launch_d<128, true>(P, a, grid, s);
  if (a.dp == 64) return a.d == 64 ? launch_d<64, false>(P, a, grid, s)
                                   : launch_d<64, true>(P, a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace rk
