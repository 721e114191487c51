// Masked flash-attention backward, bf16 inputs, d_head = 64, CDNA4 MFMA.
//
// Gradients of a loss given dO for O = softmax(Q K^T * scale + M) V (TM20K
// section 2.1, LazFormer eq. 21), with P recomputed from the forward's
// log-sum-exp (in log2 units: lse2) and D_i = dO_i . O_i:
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Two launches, no atomics (results are deterministic):
//
// dq kernel -- work item (query tile of 128 rows, head) of the query-major
//   schedule; 4 waves, 32 query rows each, walking the query tile's CSR of
//   non-empty 64-key tiles (K and V double-buffered in LDS).  Per key tile
//   and wave, with one query per lane as in the forward kernel:
//     S^T  (64 x 32) = K Q^T                     8 x mfma 32x32x16
//     P^T = exp2(S^T * scale log2(e) - lse2)     (mask on PARTIAL tiles)
//     dP^T (64 x 32) = V dO^T                    8 x mfma
//     dS^T = P^T * (dP^T - D), packed to bf16 in the key order of the
//            accumulator (as P^T in the forward)
//     dQ^T (64 x 32) += K^T dS^T                 8 x mfma (K^T by
//            transposing LDS reads)
//   Its prologue computes D and lse2 of its rows and stores them for the
//   second launch.
//
// dkdv kernel -- work item (key block of 128 keys, head) of the key-major
//   schedule; 4 waves: wave w owns keys 32 w .. +31 of the block (their K
//   and V fragments stay in registers) and walks all 128 rows of each
//   visited query tile in four 32-row blocks (Q, dO, lse2, D and row
//   descriptors double-buffered in LDS).  Per 32-row block and wave, with
//   one key per lane:
//     S  (32 q x 32 keys) = Q K^T                4 x mfma
//     P = exp2(S * scale log2(e) - lse2_q)       (mask on PARTIAL tiles)
//     dP (32 x 32) = dO V^T                      4 x mfma
//     dS = P * (dP - D_q)
//     dV^T (64 x 32) += dO^T P                   4 x mfma (dO^T and Q^T by
//     dK^T (64 x 32) += Q^T dS                   4 x mfma  transposing reads)
//
// With time RoPE, Q and K arrive rotated (a pass into the workspace, or K
// given rotated); dQ and dK are taken back through the rotation (rotation by
// -alpha) in fp32 before their single rounding to bf16.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (lane l, half h = l / 32):
//   A[m][k]: lane holds m = l % 32, k = 8h .. 8h+7
//   B[k][n]: lane holds n = l % 32, k = 8h .. 8h+7
//   D[m][n]: lane holds n = l % 32, m = 8 (r/4) + 4h + (r%4), r = 0..15
// An accumulator therefore feeds the B operand of the next product directly
// when the next contraction runs over its m index, taken in the order the
// registers hold it; the A operand is then read in that order with
// transposing LDS reads.
//
// LDS tiles hold rows of 128 bytes (eight 16-byte slots), unpadded; logical
// chunk c of row r sits in slot c ^ swz(r), swz(r) = 2 (r & 3) + ((r >> 2) & 1).
// The transposing reads (rows 4k .. 4k + 3, four chunks over 32 lanes) are
// free of bank conflicts on gfx950's 64-bank LDS; the row reads (16 rows at
// one chunk) meet a two-way conflict between rows r and r + 8.  A swizzle
// free of both needs a 16-row period, which stops rows r and r + 8 of a
// transposing read from sharing an address register (+1 KB immediate): it
// took the dq kernel from 166 to 190 VGPRs (3 to 2 waves per SIMD) and the
// dK/dV kernel to 256 with spills, and measured 0.6 % slower, so this one
// stays.
#include "cdna4_common.h"

namespace rk {
namespace {

using namespace cdna4;

constexpr int D = 64;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

#define LDS_PTR RK_LDS_PTR

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

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// 16-byte chunk c (8 bf16) of row r of an LDS tile
__device__ __forceinline__ bf16x8 lds_chunk(const unsigned short* t, int r, int c) {
  return as_bf16x8(*(const uint4*)&t[r * 64 + 8 * (c ^ swz(r))]);
}

// A operand of X^T (m = d, k = 16 rows in accumulator order) from an LDS
// tile X [rows][64] by transposing reads: lane li of half hh receives
// X[r][32 mb + li] for r = r0 + 8 (e / 4) + 4 hh + e % 4, e = 0..7.
__device__ __forceinline__ bf16x8 lds_tr(const unsigned short* t, int r0, int mb, int li, int hh) {
  const int g = (li >> 4) + 2 * hh;  // 16-lane group
  const int i = li & 15;
  const int col = 32 * mb + 16 * (g & 1) + 4 * (i & 3);
  const int ra = r0 + 4 * hh + (i >> 2);
  const int rb = ra + 8;
  const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      LDS_PTR(v4i16, &t[ra * 64 + 8 * ((col >> 3) ^ swz(ra)) + (col & 7)]));
  const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      LDS_PTR(v4i16, &t[rb * 64 + 8 * ((col >> 3) ^ swz(rb)) + (col & 7)]));
  bf16x8 a;
  __builtin_memcpy(&a, &lo4, 8);
  __builtin_memcpy((char*)&a + 8, &hi4, 8);
  return a;
}

// Per-lane byte offset of a direct buffer -> LDS copy: one wave's 16-byte
// per-lane load fills 1 KB of LDS (8 rows) contiguously; copy j of a tile
// fills rows 8 j .. 8 j + 7, and lane l lands in slot l & 7 of row 8 j + l / 8,
// so it fetches logical chunk slot ^ swz(row).
__device__ __forceinline__ unsigned copy_off(int j, int lane, unsigned st_b) {
  const int r = 8 * j + (lane >> 3), slot = lane & 7;
  return (unsigned)r * st_b + 16u * (unsigned)(slot ^ swz(r));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, unsigned st_b,
                                                            int nrows) {
  // ends at the last byte of the last valid row: later rows load zeros
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0,
                                           nrows > 0 ? (int)((unsigned)(nrows - 1) * st_b + 2u * D)
                                                     : 0,
                                           (int)kBufferFlags);
}

__device__ __forceinline__ void copy_rows(unsigned short* dst, __amdgpu_buffer_rsrc_t rs, int j,
                                          unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, dst + j * 512), 16, off, 0, 0, 0);
}

// Mask of one 64-key tile on S^T accumulators (one query per lane): key
// c0 + 8 g + 4 hh + e is in register 4 g + e of s0, that key + 32 in s1.
__device__ __forceinline__ void mask_keys(f32x16& s0, f32x16& s1, int kt, int hh, int lo, int hi,
                                          int self, int row) {
  const uint64_t vis = tile_vis_bits(kt * kTileK, lo, hi, self, row) >> (4 * hh);
  const int w0 = (int)(unsigned)vis, w1 = (int)(unsigned)(vis >> 32);
  const int ninf = (int)0xff800000u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const unsigned bit = 8u * (unsigned)(r >> 2) + (unsigned)(r & 3);
    const int m0 = __builtin_amdgcn_sbfe(w0, bit, 1u);
    const int m1 = __builtin_amdgcn_sbfe(w1, bit, 1u);
    s0[r] = __int_as_float((__float_as_int(s0[r]) & m0) | (ninf & ~m0));
    s1[r] = __int_as_float((__float_as_int(s1[r]) & m1) | (ninf & ~m1));
  }
}

// Rotate the pairs of a d-layout accumulator (lane half hh holds
// d = 8 (r/4) + 4 hh + r % 4 in x0 and d + 32 in x1) by -alpha_i,
// alpha_i = dt * omega_i, and scale them.  Pair i = d / 2.
__device__ __forceinline__ void unrotate_acc(f32x16& x0, f32x16& x1, int64_t dt,
                                             const RopeTab& tab, int hh, float mul, bool rot) {
  const double dtd = (double)dt;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    f32x16& x = half ? x1 : x0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 4 * g + 2 * j;
        float a0 = x[r] * mul, a1 = x[r + 1] * mul;
        if (rot) {
          // pair 16 half + 4 g + 2 hh + j: both candidates are uniform loads
          const int i0 = 16 * half + 4 * g + j;
          const double w = hh ? tab.w_rev[i0 + 2] : tab.w_rev[i0];
          const double rev = dtd * w;
          const float f = (float)(rev - rint(rev));
          const float sn = __builtin_amdgcn_sinf(f);
          const float cs = __builtin_amdgcn_cosf(f);
          const float y0 = a0 * cs + a1 * sn, y1 = a1 * cs - a0 * sn;
          a0 = y0;
          a1 = y1;
        }
        x[r] = a0;
        x[r + 1] = a1;
      }
    }
  }
}

// Store a d-layout accumulator pair (d and d + 32, see unrotate_acc) as a
// bf16 row.
__device__ __forceinline__ void store_row(unsigned short* p, const f32x16& x0, const f32x16& x1,
                                          int hh) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int d = 8 * g + 4 * hh;
    *(uint2*)(p + d) = make_uint2(pack_bf16x2(x0[4 * g], x0[4 * g + 1]),
                                  pack_bf16x2(x0[4 * g + 2], x0[4 * g + 3]));
    *(uint2*)(p + 32 + d) = make_uint2(pack_bf16x2(x1[4 * g], x1[4 * g + 1]),
                                       pack_bf16x2(x1[4 * g + 2], x1[4 * g + 3]));
  }
}

// ===========================================================================
// dq kernel
// ===========================================================================

constexpr int TILE_ELEMS = kTileK * D;  // 64 rows x 64 bf16 = 8 KB

// X^T (64 keys x 32 queries) = X_tile Y_w^T + c, X from LDS (row reads), Y
// fragments in registers (lane = query), c the lane's query's constant in
// every accumulator register.
__device__ __forceinline__ void prod_keys(f32x16& s0, f32x16& s1, const unsigned short* t,
                                          const bf16x8 (&y)[4], float c, int li, int hh) {
#pragma unroll
  for (int r = 0; r < 16; ++r) { s0[r] = c; s1[r] = c; }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = 2 * s + hh;  // d = 16 s + 8 hh .. +7
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_chunk(t, li, c), y[s], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_chunk(t, 32 + li, c), y[s], s1, 0, 0, 0);
  }
}

__device__ __forceinline__ void dq_tile(f32x16& dq0, f32x16& dq1, const unsigned short* kb,
                                        const unsigned short* vb, const bf16x8 (&q)[4],
                                        const bf16x8 (&g)[4], int kt, bool partial, int li, int hh,
                                        int lo, int hi, int self, int row, float lse2,
                                        float dsum) {
  // q carries scale * log2(e), so the products start from -lse2 and -D and
  // come out as the exponent of P^T and as dP^T - D
  f32x16 s0, s1, p0, p1;
  prod_keys(s0, s1, kb, q, -lse2, li, hh);
  if (partial) mask_keys(s0, s1, kt, hh, lo, hi, self, row);
  prod_keys(p0, p1, vb, g, -dsum, li, hh);
  // dS^T = P^T (dP^T - D), packed as the B operand of step s (accumulator
  // block s / 2, registers 8 (s % 2) .. +7)
  bf16x8 ds[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f32x16& sa = (s < 2) ? s0 : s1;
    const f32x16& pa = (s < 2) ? p0 : p1;
    const int r0 = 8 * (s & 1);
    bf16x2_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pr0 = __builtin_amdgcn_exp2f(sa[r0 + 2 * j]);
      const float pr1 = __builtin_amdgcn_exp2f(sa[r0 + 2 * j + 1]);
      w[j][0] = (__bf16)(pr0 * pa[r0 + 2 * j]);
      w[j][1] = (__bf16)(pr1 * pa[r0 + 2 * j + 1]);
    }
    __builtin_memcpy(&ds[s], w, 16);
  }
  // dQ^T += K^T dS^T
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    dq0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr(kb, 16 * s, 0, li, hh), ds[s], dq0, 0, 0, 0);
    dq1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr(kb, 16 * s, 1, li, hh), ds[s], dq1, 0, 0, 0);
  }
}

template <bool kUnrot>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq_kernel(BwdPlanView P, BwdLaunch A) {
  __shared__ __attribute__((aligned(1024))) unsigned short K0[TILE_ELEMS], K1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) unsigned short V0[TILE_ELEMS], V1[TILE_ELEMS];
  const int item = ldc(P.sched, blockIdx.x);
  if (item < 0) return;
  const float pz = plan_poison(A.plan_err);
  const int qg = item / A.H;
  const int head = item - qg * A.H;
  const int req = ldc(P.qt_req, qg);
  const ReqMeta m = ldc(P.req, req);
  const int qt = qg - m.qt_off;
  const int L = m.len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int li = lane & 31;
  const int row = qt * kTileQ + wv * 32 + li;
  const bool rvalid = row < L;
  const int tokq = m.tok_off + row;
  const int tokc = m.tok_off + min(row, L - 1);  // in-bounds row for the loads

  // row inputs: Q, dO, O fragments (d = 16 s + 8 hh .. +7), lse, descriptor
  const unsigned short* Qp = (const unsigned short*)A.q + (int64_t)tokc * A.q_st + (int64_t)head * A.q_sh;
  const unsigned short* Gp = (const unsigned short*)A.dout + (int64_t)tokc * A.do_st + (int64_t)head * A.do_sh;
  const unsigned short* Op = (const unsigned short*)A.o + (int64_t)tokc * A.o_st + (int64_t)head * A.o_sh;
  uint4 qr[4], gr[4], orow[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qr[s] = *(const uint4*)(Qp + 16 * s + 8 * hh);
    gr[s] = *(const uint4*)(Gp + 16 * s + 8 * hh);
    orow[s] = *(const uint4*)(Op + 16 * s + 8 * hh);
  }
  const float lse = A.lse[(int64_t)head * A.T + tokc];
  const int2 dsc = P.row_desc[tokc];

  const char* Kb = (const char*)((const unsigned short*)A.k + (int64_t)m.tok_off * A.k_st + (int64_t)head * A.k_sh);
  const char* Vb = (const char*)((const unsigned short*)A.v + (int64_t)m.tok_off * A.v_st + (int64_t)head * A.v_sh);
  const unsigned kst_b = (unsigned)A.k_st * 2u, vst_b = (unsigned)A.v_st * 2u;
  unsigned koff[2], voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    koff[j] = copy_off(2 * wv + j, lane, kst_b);
    voff[j] = copy_off(2 * wv + j, lane, vst_b);
  }
  // Each wave zeroes the rows its own copies fill in both stages, so any
  // byte a copy leaves unwritten is finite (masked keys then add exactly 0).
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int o = (2 * wv + j) * 512 + 8 * lane;
    *(uint4*)&K0[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&K1[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&V0[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&V1[o] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  const int e0 = ldc(P.qtile_ptr, qg);
  const int n = ldc(P.qtile_ptr, qg + 1) - e0;
  auto issue = [&](unsigned short* kd, unsigned short* vd, int kt) {
    const int c0 = kt * kTileK;
    const int nr = min(L - c0, kTileK);
    const __amdgpu_buffer_rsrc_t kr = rows_rsrc(Kb + (int64_t)c0 * kst_b, kst_b, nr);
    const __amdgpu_buffer_rsrc_t vr = rows_rsrc(Vb + (int64_t)c0 * vst_b, vst_b, nr);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      copy_rows(kd, kr, 2 * wv + j, koff[j]);
      copy_rows(vd, vr, 2 * wv + j, voff[j]);
    }
  };
  int w_cur = n > 0 ? ldc(P.ktile_word, e0) : 0;
  issue(K0, V0, w_cur & 0x7fffffff);

  // finish the row inputs while the first copies land
  bf16x8 q[4], g[4];
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const unsigned wq[4] = {qr[s].x, qr[s].y, qr[s].z, qr[s].w};
    const unsigned wg[4] = {gr[s].x, gr[s].y, gr[s].z, gr[s].w};
    const unsigned wo[4] = {orow[s].x, orow[s].y, orow[s].z, orow[s].w};
    unsigned zq[4], zg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dpart = fmaf(bf_lo(wg[j]), bf_lo(wo[j]), dpart);
      dpart = fmaf(bf_hi(wg[j]), bf_hi(wo[j]), dpart);
      zq[j] = rvalid ? wq[j] : 0u;
      zg[j] = rvalid ? wg[j] : 0u;
    }
    q[s] = as_bf16x8(make_uint4(zq[0], zq[1], zq[2], zq[3]));
    g[s] = as_bf16x8(make_uint4(zg[0], zg[1], zg[2], zg[3]));
  }
  const float dsum = rvalid ? dpart + __shfl_xor(dpart, 32, 64) : 0.f;
  const float lse2 = (rvalid && lse != -INFINITY) ? lse * kLog2e : INFINITY;
  if (rvalid && hh == 0) {
    A.dsum[(int64_t)head * A.T + tokq] = dsum;
    A.lse2[(int64_t)head * A.T + tokq] = lse2;
  }
  const int lo = rvalid ? dsc.x : 0;
  const int hi = rvalid ? dsc.y & 0x7fffffff : 0;
  const int self = rvalid && dsc.y < 0;
  // scores in log2 units straight from the matrix cores
#pragma unroll
  for (int s = 0; s < 4; ++s) q[s] = scale_bf16x8(q[s], A.scale * kLog2e);

  f32x16 dq0, dq1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { dq0[r] = 0.f; dq1[r] = 0.f; }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < n; it += 2) {
    {
      const int w_nxt = ldc(P.ktile_word, e0 + min(it + 1, n - 1));
      issue(K1, V1, w_nxt & 0x7fffffff);
      dq_tile(dq0, dq1, K0, V0, q, g, w_cur & 0x7fffffff, w_cur < 0, li, hh, lo, hi, self, row,
              lse2, dsum);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      w_cur = w_nxt;
    }
    if (it + 1 < n) {
      const int w_nxt = ldc(P.ktile_word, e0 + min(it + 2, n - 1));
      issue(K0, V0, w_nxt & 0x7fffffff);
      dq_tile(dq0, dq1, K1, V1, q, g, w_cur & 0x7fffffff, w_cur < 0, li, hh, lo, hi, self, row,
              lse2, dsum);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      w_cur = w_nxt;
    }
  }

  if (!rvalid) return;
  const int64_t dt = kUnrot ? ldc(A.ts, tokq) - ldc(A.anchors, req) : 0;
  unrotate_acc(dq0, dq1, dt, A.tab, hh, A.scale * pz, kUnrot);
  store_row((unsigned short*)A.dq + (int64_t)tokq * A.dq_st + (int64_t)head * A.dq_sh, dq0, dq1,
            hh);
}

// ===========================================================================
// dkdv kernel
// ===========================================================================

constexpr int QTILE_ELEMS = kTileQ * D;  // 128 rows x 64 bf16 = 16 KB

// LDS stage of one query tile: Q, dO, lse2, D and the row descriptors.
// The last three are filled by dword copies (64 lanes x 4 bytes = 256 bytes
// each; rows past the request's end read out of range and write zeros).
struct QStage {
  unsigned short q[QTILE_ELEMS];
  unsigned short g[QTILE_ELEMS];
  float lse2[kTileQ];
  float dsum[kTileQ];
  int2 desc[kTileQ];
};

// S or dP block (32 query rows x 32 keys): X_rows (LDS, row reads, lane =
// query row of the A operand) times the wave's key fragments (B operand).
__device__ __forceinline__ f32x16 prod_rows(const unsigned short* t, int r0,
                                            const bf16x8 (&kf)[4], int li, int hh) {
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_chunk(t, r0 + li, 2 * s + hh), kf[s], acc,
                                                  0, 0, 0);
  return acc;
}

__device__ __forceinline__ void dkdv_block(f32x16& dk0, f32x16& dk1, f32x16& dv0, f32x16& dv1,
                                           const QStage& st, int r0, const bf16x8 (&kf)[4],
                                           const bf16x8 (&vf)[4], bool partial, int qrow0,
                                           int key, int li, int hh, float c2) {
  f32x16 s = prod_rows(st.q, r0, kf, li, hh);
  f32x16 dp = prod_rows(st.g, r0, vf, li, hh);
  // rows of register r: r0 + 8 (r / 4) + 4 hh + r % 4
  bf16x8 pb[2], db[2];
  pb[0] = pb[1] = db[0] = db[1] = as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int rb = r0 + 8 * gq + 4 * hh;
    const float4 l4 = *(const float4*)&st.lse2[rb];
    const float4 d4 = *(const float4*)&st.dsum[rb];
    const float la[4] = {l4.x, l4.y, l4.z, l4.w};
    const float da[4] = {d4.x, d4.y, d4.z, d4.w};
    float pv[4], dsv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = s[4 * gq + e];
      if (partial) {
        const int2 dd = st.desc[rb + e];
        const int lo = dd.x, hi = dd.y & 0x7fffffff;
        const int q = qrow0 + rb + e;
        const bool vis = (key >= lo && key < hi) || (dd.y < 0 && key == q);
        x = vis ? x : -INFINITY;
      }
      pv[e] = __builtin_amdgcn_exp2f(fmaf(x, c2, -la[e]));
      dsv[e] = pv[e] * (dp[4 * gq + e] - da[e]);
    }
    // B operand of step gq / 2: registers 8 (gq % 2) .. +7 of the block
    const unsigned pw0 = pack_bf16x2(pv[0], pv[1]), pw1 = pack_bf16x2(pv[2], pv[3]);
    const unsigned dw0 = pack_bf16x2(dsv[0], dsv[1]), dw1 = pack_bf16x2(dsv[2], dsv[3]);
    const int sidx = gq >> 1, half = gq & 1;
    uint4 pu, du;
    __builtin_memcpy(&pu, &pb[sidx], 16);
    __builtin_memcpy(&du, &db[sidx], 16);
    if (half == 0) { pu.x = pw0; pu.y = pw1; du.x = dw0; du.y = dw1; }
    else           { pu.z = pw0; pu.w = pw1; du.z = dw0; du.w = dw1; }
    pb[sidx] = as_bf16x8(pu);
    db[sidx] = as_bf16x8(du);
  }
  // dV^T += dO^T P, dK^T += Q^T dS (contraction over the block's 32 rows)
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int rr = r0 + 16 * s2;
    dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr(st.g, rr, 0, li, hh), pb[s2], dv0, 0, 0, 0);
    dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr(st.g, rr, 1, li, hh), pb[s2], dv1, 0, 0, 0);
    dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr(st.q, rr, 0, li, hh), db[s2], dk0, 0, 0, 0);
    dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr(st.q, rr, 1, li, hh), db[s2], dk1, 0, 0, 0);
  }
}

template <bool kUnrot>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dkdv_kernel(BwdPlanView P, BwdLaunch A) {
  __shared__ __attribute__((aligned(1024))) QStage S0, S1;
  const int item = ldc(P.ksched, blockIdx.x);
  if (item < 0) return;
  const float pz = plan_poison(A.plan_err);
  const int kg = item / A.H;
  const int head = item - kg * A.H;
  const int req = ldc(P.kt_req, kg);
  const ReqMeta m = ldc(P.req, req);
  const int kb = kg - m.kt_off;  // key block of 128 keys
  const int L = m.len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int li = lane & 31;
  const int key = kb * 128 + 32 * wv + li;  // this lane's key (request-local)
  const bool kvalid = key < L;
  const int tokk = m.tok_off + key;
  const int tokc = m.tok_off + min(key, L - 1);

  // the wave's key fragments (B operands: lane = key, d = 16 s + 8 hh .. +7)
  const unsigned short* Kp = (const unsigned short*)A.k + (int64_t)tokc * A.k_st + (int64_t)head * A.k_sh;
  const unsigned short* Vp = (const unsigned short*)A.v + (int64_t)tokc * A.v_st + (int64_t)head * A.v_sh;
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 a = *(const uint4*)(Kp + 16 * s + 8 * hh);
    const uint4 b = *(const uint4*)(Vp + 16 * s + 8 * hh);
    kf[s] = as_bf16x8(kvalid ? a : make_uint4(0, 0, 0, 0));
    vf[s] = as_bf16x8(kvalid ? b : make_uint4(0, 0, 0, 0));
  }

  const char* Qb = (const char*)((const unsigned short*)A.q + (int64_t)m.tok_off * A.q_st + (int64_t)head * A.q_sh);
  const char* Gb = (const char*)((const unsigned short*)A.dout + (int64_t)m.tok_off * A.do_st + (int64_t)head * A.do_sh);
  const char* Lb = (const char*)(A.lse2 + (int64_t)head * A.T + m.tok_off);
  const char* Db = (const char*)(A.dsum + (int64_t)head * A.T + m.tok_off);
  const char* Rb = (const char*)(P.row_desc + m.tok_off);
  const unsigned qst_b = (unsigned)A.q_st * 2u, gst_b = (unsigned)A.do_st * 2u;
  // copies per stage: 16 of Q and 16 of dO (1 KB each, 4 + 4 per wave) plus
  // eight dword copies of 256 bytes (two per wave): lse2 (2), D (2) and the
  // row descriptors (4)
  unsigned qoff[4], goff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qoff[j] = copy_off(4 * wv + j, lane, qst_b);
    goff[j] = copy_off(4 * wv + j, lane, gst_b);
  }
  // Zero both stages' Q and dO rows this wave fills (any unwritten byte
  // stays finite: a masked row then adds exactly 0).
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = (4 * wv + j) * 512 + 8 * lane;
    *(uint4*)&S0.q[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&S0.g[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&S1.q[o] = make_uint4(0, 0, 0, 0);
    *(uint4*)&S1.g[o] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  auto issue = [&](QStage& st, int qt) {
    const int r0 = qt * kTileQ;
    const int nr = min(L - r0, kTileQ);
    const __amdgpu_buffer_rsrc_t qr = rows_rsrc(Qb + (int64_t)r0 * qst_b, qst_b, nr);
    const __amdgpu_buffer_rsrc_t gr = rows_rsrc(Gb + (int64_t)r0 * gst_b, gst_b, nr);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      copy_rows(st.q, qr, 4 * wv + j, qoff[j]);
      copy_rows(st.g, gr, 4 * wv + j, goff[j]);
    }
    {
      // wave 0: lse2, wave 1: D, waves 2 and 3: row descriptor halves
      const char* base = wv == 0 ? Lb + 4 * r0 : (wv == 1 ? Db + 4 * r0 : Rb + 8 * r0);
      const int bytes = wv >= 2 ? 8 * nr : 4 * nr;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, (int)kBufferFlags);
      char* dst = wv == 0 ? (char*)st.lse2 : (wv == 1 ? (char*)st.dsum : (char*)st.desc);
      const int part0 = wv == 3 ? 2 : 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int part = part0 + j;  // 256-byte part of the array
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, dst + 256 * part), 4,
                                                 256u * part + 4u * lane, 0, 0, 0);
      }
    }
  };

  f32x16 dk0, dk1, dv0, dv1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { dk0[r] = 0.f; dk1[r] = 0.f; dv0[r] = 0.f; dv1[r] = 0.f; }
  const float c2 = A.scale * kLog2e;

  const int e0 = ldc(P.kt_ptr, kg);
  const int n = ldc(P.kt_ptr, kg + 1) - e0;
  int w_cur = n > 0 ? ldc(P.qtile_word, e0) : 0;
  issue(S0, w_cur & 0x7fffffff);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < n; it += 2) {
    {
      const int w_nxt = ldc(P.qtile_word, e0 + min(it + 1, n - 1));
      issue(S1, w_nxt & 0x7fffffff);
      const int qrow0 = (w_cur & 0x7fffffff) * kTileQ;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        dkdv_block(dk0, dk1, dv0, dv1, S0, 32 * b, kf, vf, w_cur < 0, qrow0, key, li, hh, c2);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      w_cur = w_nxt;
    }
    if (it + 1 < n) {
      const int w_nxt = ldc(P.qtile_word, e0 + min(it + 2, n - 1));
      issue(S0, w_nxt & 0x7fffffff);
      const int qrow0 = (w_cur & 0x7fffffff) * kTileQ;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        dkdv_block(dk0, dk1, dv0, dv1, S1, 32 * b, kf, vf, w_cur < 0, qrow0, key, li, hh, c2);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      w_cur = w_nxt;
    }
  }

  if (!kvalid) return;
  const int64_t dt = kUnrot ? ldc(A.ts, tokk) - ldc(A.anchors, req) : 0;
  unrotate_acc(dk0, dk1, dt, A.tab, hh, A.scale * pz, kUnrot);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    dv0[r] *= pz;
    dv1[r] *= pz;
  }
  store_row((unsigned short*)A.dk + (int64_t)tokk * A.dk_st + (int64_t)head * A.dk_sh, dk0, dk1,
            hh);
  store_row((unsigned short*)A.dv + (int64_t)tokk * A.dv_st + (int64_t)head * A.dv_sh, dv0, dv1,
            hh);
}

}  // namespace

hipError_t launch_attn_bwd_mfma_bf16_d64(const rk_plan* p, const BwdLaunch& a, hipStream_t s) {
  if (p->slots == 0 || p->kslots == 0) return hipSuccess;
  BwdPlanView P{p->dev.req,       p->dev.qt_req,     p->dev.kt_req, p->dev.row_desc,
                p->dev.qtile_ptr, p->dev.ktile_word, p->dev.kt_ptr, p->dev.qtile_word,
                p->dev.sched,     p->dev.ksched};
  if (a.unrot_q)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<true>, dim3((unsigned)p->slots), dim3(kThreads), 0, s,
                       P, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<false>, dim3((unsigned)p->slots), dim3(kThreads), 0, s,
                       P, a);
  if (a.unrot_k)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<true>, dim3((unsigned)p->kslots), dim3(kThreads), 0,
                       s, P, a);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<false>, dim3((unsigned)p->kslots), dim3(kThreads), 0,
                       s, P, a);
  return hipGetLastError();
}

}  // namespace rk
