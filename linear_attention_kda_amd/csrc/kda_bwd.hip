// Backward pass of the chunkwise KDA forward for gfx950 (MI355X).
//
// Per chunk (64 tokens of one sequence and head; local rows r, i; S the chunk's
// start state, S' its end state), with G the within-chunk inclusive cumsum of g,
// Gam = exp(G), gam = exp(G_last) [core.today "Kimi Linear 특집", ch.4 혁신 2,
// state-update equation and its chunkwise form]:
//   kg = K*Gam, qg = Q*Gam, kh = K/Gam, kp = kh*gam
//   A  = strict_lower(diag(b) kg kh^T),  T = (I + A)^-1
//   R  = V - kg S,  U = T diag(b) R,  M = lower_incl(qg kh^T)
//   O  = scale (qg S + M U),  S' = Diag(gam) S + kp^T U
// Reverse mode, given dO' = scale dO and dSn = dL/dS' (written out here):
//   dU  = M^T dO' + kp dSn                dM  = lower_incl(dO' U^T)
//   dY  = T^T dU                          dA  = strict_lower(-dY U^T)
//   dqg = dO' S^T + dM kh                 dkp = U dSn^T
//   dkg = diag(b) (dA kh - dY S^T)        dkh = dM^T qg + dA^T diag(b) kg
//   dV  = diag(b) dY                      db_r = sum_j dY_rj R_rj + sum_i dA_ri (kg kh^T)_ri
//   dS  = Diag(gam) dSn + qg^T dO' - kg^T diag(b) dY           (gradient at S)
// and through the gates: dq = dqg Gam, dk = dkg Gam + dkh/Gam + dkp gam/Gam,
//   dG_r = dqg qg + dkg kg - dkh kh - dkp kp (per channel),
//   dG_last = sum_r dkp kp + gam * rowsum(S * dSn),  dg_t = sum_{r >= t} dG_r + dG_last.
// kh = K/Gam is never formed: over a whole chunk exp(-G) overflows fp32 long before
// the recurrence does.  Every product that pairs exp(G_r) with exp(-G_i) -- P, M and
// the terms dM kh, dA kh and dkh through the gates -- is evaluated directly as
// sum_i W_ri x_i exp(G_r - G_i) per channel with the 16-row block references of the
// forward pass (bwd_pm_kernel, bwd_gated_kernel), so the backward accepts every g the
// forward accepts; the other products only see Gam <= 1, kp = K exp(G_last - G) <= 1
// and the state.
// The only serial dependency is dS across chunks: with F = kg^T diag(b) T^T
// (128 x 64) and X = qg^T dO' (128 x 128), both chunk-local,
//   dU = kp dSn + M^T dO',   dS = Diag(gam) dSn - F dU + X.
//
// Layout: the forward pass writes every chunk's start state (fp32) to slot
// n + floor(bos_n / 64) + c of sequence n's chunk c (slots are distinct across
// sequences); batch index b = slot * H + h addresses every per-chunk tile.
// Everything here is fp32: the chunk-local products run as batched tiled GEMMs
// (fp32 matrix cores), the serial recurrence in eight workgroups per (sequence,
// head), one per 16 value columns.  launch_bwd_streams (at the end) orders the
// launches on the caller's stream and a second one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int C = 64;

__device__ __forceinline__ float bf2f_u16(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ int64_t seq_bos(const BwdParams& p, int n) {
  return p.cu ? (int64_t)p.cu[n] : (int64_t)n * p.T;
}
__device__ __forceinline__ int64_t seq_len_of(const BwdParams& p, int n) {
  return p.cu ? (int64_t)p.cu[n + 1] - p.cu[n] : p.T;
}

// Sequence owning slot s: the largest n with n + floor(bos_n / 64) <= s.
__device__ __forceinline__ int slot_seq(const BwdParams& p, int64_t s) {
  int lo = 0, hi = p.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mid + seq_bos(p, mid) / C <= s) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- batched GEMM
// C[b] = rs[b] (.) (alpha op(A[b]) op(B[b]) + D[b]), then masked; row-major fp32.
// op(A) is M x K: A stored [m][k] (TA false) or [k][m] (TA true); its k-th column
// is scaled by ks[b][k] when ks is given.  op(B) is K x N: B stored [k][n] (TB
// false) or [n][k] (TB true).  rs scales output rows.  mask: 0 none, 1 keep
// n < m, 2 keep n <= m.  One workgroup computes a 64 x 64 or 64 x 128 tile; M, N,
// K are multiples of 64, 64 and 16.
//
// The products run on the fp32 matrix cores (16 x 16 x 4 per instruction, fp32
// operands and accumulation): twice the rate of unpacked fp32 FMAs.  Each wave
// owns a quarter of the tile as 2 x (NT / 32) blocks; for step k of four, lane
// (q4, m16) supplies op(A)[16i + m16][k] and op(B)[k][16j + m16] with k = 4s + q4,
// and holds C[16i + 4q4 + t][16j + m16] (t < 4) of each block.
typedef float bg_f32x4 __attribute__((ext_vector_type(4)));

// k-major tiles; a row stride of 16 mod 32 floats puts lane groups q4 and q4 + 1
// on disjoint banks for the operand reads.  NT is the tile's width (64 or 128).
// Column c of row k is stored at bg_col(k, c) = c ^ 8 ((k >> 2) & 3): a transposed
// operand is staged four k rows per group of lanes (rows 4 apart: the same banks
// with this stride), and the XOR puts the four groups on different banks; it
// moves whole 8-column blocks, so runs of four columns stay together, and the
// reads take one k per step, whose XOR is a constant there.
template <int NT>
struct BgTiles {
  float A[16][80];
  float B[16][NT + 16];
};

__device__ __forceinline__ int bg_col(int k, int c) { return c ^ (8 * ((k >> 2) & 3)); }

// acc += sign * op(A) op(B) over K for the 64 x NT tile at (m0, n0); op(A)'s
// k-th column is scaled by ks[k] when ks is given (sign is +-1: exact).  Wave w
// owns rows 32 (w / 2) .. +31 and columns (NT / 2)(w % 2) .. + NT / 2 - 1.
template <int NT, bool TA, bool TB>
__device__ __forceinline__ void bg_accumulate(bg_f32x4 (&acc)[2][NT / 32], BgTiles<NT>& sm,
                                              const float* A, int lda, const float* B, int ldb,
                                              int K, const float* ks, float sign, int m0, int n0) {
  constexpr int JN = NT / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, m16 = lane & 15, q4 = lane >> 4;
  const int wm = 32 * (wave >> 1), wn = (NT / 2) * (wave & 1);
  for (int k0 = 0; k0 < K; k0 += 16) {
    if (!TA) {
      const int m = tid >> 2, k = (tid & 3) * 4;
      const float4 v = *reinterpret_cast<const float4*>(A + (int64_t)(m0 + m) * lda + k0 + k);
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.A[k + e][bg_col(k + e, m)] = (ks ? vv[e] * ks[k0 + k + e] : vv[e]) * sign;
    } else {
      const int k = tid >> 4, m = (tid & 15) * 4;
      const float4 v = *reinterpret_cast<const float4*>(A + (int64_t)(k0 + k) * lda + m0 + m);
      const float s = (ks ? ks[k0 + k] : 1.f) * sign;
      *reinterpret_cast<float4*>(&sm.A[k][bg_col(k, m)]) = make_float4(v.x * s, v.y * s, v.z * s, v.w * s);
    }
#pragma unroll
    for (int h = 0; h < NT / 64; ++h) {
      if (!TB) {
        const int k = tid >> 4, n = 64 * h + (tid & 15) * 4;
        *reinterpret_cast<float4*>(&sm.B[k][bg_col(k, n)]) =
            *reinterpret_cast<const float4*>(B + (int64_t)(k0 + k) * ldb + n0 + n);
      } else {
        const int n = 64 * h + (tid >> 2), k = (tid & 3) * 4;
        const float4 v = *reinterpret_cast<const float4*>(B + (int64_t)(n0 + n) * ldb + k0 + k);
        const int nc = bg_col(k, n);   // rows k .. k + 3 share the XOR
        sm.B[k][nc] = v.x; sm.B[k + 1][nc] = v.y; sm.B[k + 2][nc] = v.z; sm.B[k + 3][nc] = v.w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int k = 4 * s4 + q4;
      const float a0 = sm.A[k][bg_col(k, wm + m16)], a1 = sm.A[k][bg_col(k, wm + 16 + m16)];
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const float bj = sm.B[k][bg_col(k, wn + 16 * j + m16)];
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bj, acc[0][j], 0, 0, 0);
        acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bj, acc[1][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
}

// C = rs (.) (alpha acc + D), masked, for the tile at (m0, n0) of batch b.
template <int NT>
__device__ __forceinline__ void bg_store(const bg_f32x4 (&acc)[2][NT / 32], const GemmArgs& a,
                                         int64_t b, int m0, int n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m16 = lane & 15, q4 = lane >> 4;
  const int wm = 32 * (wave >> 1), wn = (NT / 2) * (wave & 1);
  float* Cb = a.C + b * a.sC;
  const float* Db = a.Dm ? a.Dm + b * a.sD : nullptr;
  const float* rs = a.rs ? a.rs + b * a.srs : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m0 + wm + 16 * i + 4 * q4 + t;
      const float r = rs ? rs[m] : 1.f;
#pragma unroll
      for (int j = 0; j < NT / 32; ++j) {
        const int n = n0 + wn + 16 * j + m16;
        float v = a.alpha * acc[i][j][t];
        if (Db) v += Db[(int64_t)m * a.ldd + n];
        v *= r;
        if ((a.mask == 1 && n >= m) || (a.mask == 2 && n > m)) v = 0.f;
        Cb[(int64_t)m * a.ldc + n] = v;
      }
    }
}

template <int NT>
__device__ __forceinline__ void bg_zero(bg_f32x4 (&acc)[2][NT / 32]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT / 32; ++j) acc[i][j] = bg_f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int NT, bool TA, bool TB>
__global__ void __launch_bounds__(256) bgemm_kernel(GemmArgs a) {
  __shared__ BgTiles<NT> sm;
  const int n0 = blockIdx.x * NT, m0 = blockIdx.y * 64;
  const int64_t b = blockIdx.z;
  bg_f32x4 acc[2][NT / 32];
  bg_zero<NT>(acc);
  bg_accumulate<NT, TA, TB>(acc, sm, a.A + b * a.sA, a.lda, a.B + b * a.sB, a.ldb, a.K,
                            a.ks ? a.ks + b * a.sks : nullptr, 1.f, m0, n0);
  bg_store<NT>(acc, a, b, m0, n0);
}

// ---------------------------------------------------------------- chunk prep
// One workgroup per batch (slot, head): loads the chunk's rows (zero past the
// sequence), forms G, the gated tiles K Gam, Q Gam and K exp(G_last - G) (all <= 1
// for g <= 0), dO' = scale dO and the per-row beta.  Thread t owns channels
// 4 (t % 32) .. +3 of rows 8 (t / 32) .. +7: 16-byte loads of g, 8-byte loads of
// q, k, v and dO, 16-byte stores of every tile; the exponentials are exp2 of
// G log2(e).
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p, BwdTiles w) {
  const int64_t bidx = blockIdx.x;   // the group's batch (tile index)
  const int64_t slot = p.slot0 + bidx / p.H;
  const int h = (int)(bidx % p.H);
  const int n = slot_seq(p, slot);
  const int64_t bos = seq_bos(p, n), len = seq_len_of(p, n);
  const int64_t c = slot - (n + bos / C);
  const int64_t rest = len - c * C;
  const int valid = (c < 0 || rest <= 0) ? 0 : rest < C ? (int)rest : C;
  const int t = threadIdx.x;
  const int64_t HD = (int64_t)p.H * D;
  if (t < C) w.beta[bidx * C + t] = t < valid ? p.beta[(bos + c * C + t) * p.H + h] : 0.f;
  if (t == 0) w.valid[bidx] = valid;
  constexpr float kLog2e = 1.4426950408889634f;
  const int c4 = 4 * (t & 31), rg = t >> 5, r0 = 8 * rg;
  const int64_t tok0 = bos + c * C;
  // G: inclusive cumsum over the chunk (natural log): each thread sums its 8 rows in
  // registers, then adds the totals of the row groups before it
  __shared__ float4 tot[8][32];
  float4 gv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + i;
    gv[i] = r < valid ? *reinterpret_cast<const float4*>(&p.g[((tok0 + r) * p.H + h) * D + c4])
                      : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    gv[i].x += gv[i - 1].x; gv[i].y += gv[i - 1].y; gv[i].z += gv[i - 1].z; gv[i].w += gv[i - 1].w;
  }
  tot[rg][t & 31] = gv[7];
  __syncthreads();
  float4 off = make_float4(0.f, 0.f, 0.f, 0.f), gl = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 v = tot[k][t & 31];
    if (k < rg) { off.x += v.x; off.y += v.y; off.z += v.z; off.w += v.w; }
    gl.x += v.x; gl.y += v.y; gl.z += v.z; gl.w += v.w;
  }
  const float glast[4] = {gl.x, gl.y, gl.z, gl.w};
  if (rg == 0)
    *reinterpret_cast<float4*>(&w.gam[bidx * D + c4]) =
        make_float4(exp2f(gl.x * kLog2e), exp2f(gl.y * kLog2e), exp2f(gl.z * kLog2e), exp2f(gl.w * kLog2e));
  const int64_t tb = bidx * (C * D);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + i;
    const int64_t row = (tok0 + r) * HD + (int64_t)h * D + c4;
    const bool in = r < valid;
    const uint2 zero = make_uint2(0u, 0u);
    const uint2 qu = in ? *reinterpret_cast<const uint2*>(&p.q[row]) : zero;
    const uint2 ku = in ? *reinterpret_cast<const uint2*>(&p.k[row]) : zero;
    const uint2 vu = in ? *reinterpret_cast<const uint2*>(&p.v[row]) : zero;
    const uint2 du = in ? *reinterpret_cast<const uint2*>(&p.dout[row]) : zero;
    const float qf[4] = {bf2f_u16(qu.x & 0xffffu), bf2f_u16(qu.x >> 16), bf2f_u16(qu.y & 0xffffu), bf2f_u16(qu.y >> 16)};
    const float kf[4] = {bf2f_u16(ku.x & 0xffffu), bf2f_u16(ku.x >> 16), bf2f_u16(ku.y & 0xffffu), bf2f_u16(ku.y >> 16)};
    const float vf[4] = {bf2f_u16(vu.x & 0xffffu), bf2f_u16(vu.x >> 16), bf2f_u16(vu.y & 0xffffu), bf2f_u16(vu.y >> 16)};
    const float df[4] = {bf2f_u16(du.x & 0xffffu), bf2f_u16(du.x >> 16), bf2f_u16(du.y & 0xffffu), bf2f_u16(du.y >> 16)};
    const float gr[4] = {gv[i].x + off.x, gv[i].y + off.y, gv[i].z + off.z, gv[i].w + off.w};
    float o_g[4], o_kg[4], o_qg[4], o_kp[4], o_d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float eg = exp2f(gr[e] * kLog2e);
      o_g[e] = gr[e];
      o_kg[e] = kf[e] * eg;
      o_qg[e] = qf[e] * eg;
      o_kp[e] = kf[e] * exp2f((glast[e] - gr[e]) * kLog2e);
      o_d[e] = p.scale * df[e];
    }
    const int64_t o = tb + r * D + c4;
    *reinterpret_cast<float4*>(&w.G[o]) = make_float4(o_g[0], o_g[1], o_g[2], o_g[3]);
    *reinterpret_cast<float4*>(&w.kg[o]) = make_float4(o_kg[0], o_kg[1], o_kg[2], o_kg[3]);
    *reinterpret_cast<float4*>(&w.qg[o]) = make_float4(o_qg[0], o_qg[1], o_qg[2], o_qg[3]);
    *reinterpret_cast<float4*>(&w.kp[o]) = make_float4(o_kp[0], o_kp[1], o_kp[2], o_kp[3]);
    *reinterpret_cast<float4*>(&w.vv[o]) = make_float4(vf[0], vf[1], vf[2], vf[3]);
    *reinterpret_cast<float4*>(&w.dO[o]) = make_float4(o_d[0], o_d[1], o_d[2], o_d[3]);
  }
}

// ---------------------------------------------------------------- block references
// For a chunk with G the cumulative log-decay, X_b = G at the last row of block b - 1
// (X_0 = 0, X_4 = G_last), rows r in block rb and i in block ib <= rb:
//   exp(G_r - G_i) = F_r w(rb, ib) H_i,  F_r = exp(G_r - X_rb),  H_i = exp(X_{ib+1} - G_i),
//   w(rb, ib) = exp(X_rb - X_{ib+1})
// per channel.  For g <= 0, F, H <= 1 and w <= 1 off the diagonal blocks; on a diagonal
// block w = exp(-sum of g over the block), finite while that sum stays below ~88 -- the
// forward pass's own limit [core.today "Kimi Linear 특집", ch.4 혁신 2, chunkwise form].
// Block pairs are numbered p = rb (rb + 1) / 2 + ib.
constexpr int kPairs = 10;

__device__ __forceinline__ int bwd_pair(int rb, int ib) { return rb * (rb + 1) / 2 + ib; }

// exp(x) for a natural-log argument on the hardware exp2 (one multiply and v_exp_f32; the
// rounding of x log2(e) adds a relative error of about |x| 6e-8, results below 2^-126 flush)
__device__ __forceinline__ float exp_n(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Sequence, head, first row and valid rows of the group's batch bidx (a tile index).
__device__ __forceinline__ void bwd_chunk_rows(const BwdParams& p, int64_t bidx, int& h, int64_t& bos,
                                               int64_t& c, int& valid, int& n) {
  const int64_t gb = p.slot0 * p.H + bidx;
  const int64_t slot = gb / p.H;
  h = (int)(gb % p.H);
  n = slot_seq(p, slot);
  bos = seq_bos(p, n);
  const int64_t len = seq_len_of(p, n);
  c = slot - (n + bos / C);
  const int64_t rest = len - c * C;
  valid = (c < 0 || rest <= 0) ? 0 : rest < C ? (int)rest : C;
}

// ---------------------------------------------------------------- P, A and M
// P = strict_lower(K K^T gated), A = diag(beta) P, M = lower_incl(Q K^T gated):
// P_ri = sum_c k_rc k_ic exp(G_rc - G_ic) = sum_c (k F)_rc (k H)_ic w(rb, ib)_c, and M
// likewise with q in the row operand, on the fp32 matrix cores (16 x 16 x 4).  One
// workgroup per batch; each wave takes two or three of the ten lower block pairs (both
// products share the column operand), the blocks above the diagonal are zero.  The
// channels go through LDS in two halves of 64 (the products accumulate over both), so
// that two workgroups fit a CU; the second half's loads are issued before the first
// half's products.
constexpr int PMH = 64;        // channels per half
constexpr int PMS = PMH + 4;   // row stride (fp32) of the staged operands
struct alignas(16) PmSmem {
  float kF[C][PMS];
  float qF[C][PMS];
  float kH[C][PMS];
  float wf[kPairs][PMH];
  float X[5][PMH];
  float beta[C];
};

// One half's contribution to pair pr's P and M tiles (lane holds rows 16 rb + 4 q4 + t,
// column 16 ib + m16).
__device__ __forceinline__ void pm_pair_acc(const PmSmem& sm, int pr, bg_f32x4& ap, bg_f32x4& am) {
  const int rb = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
  const int ib = pr - rb * (rb + 1) / 2;
  const int lane = threadIdx.x & 63, q4 = lane >> 4, m16 = lane & 15;
  // channel 16j + 4q4 + s4 of instruction s4: four consecutive channels per lane
#pragma unroll
  for (int j = 0; j < PMH / 16; ++j) {
    const int c0 = 16 * j + 4 * q4;
    const float4 kf = *reinterpret_cast<const float4*>(&sm.kF[16 * rb + m16][c0]);
    const float4 qf = *reinterpret_cast<const float4*>(&sm.qF[16 * rb + m16][c0]);
    const float4 kh = *reinterpret_cast<const float4*>(&sm.kH[16 * ib + m16][c0]);
    const float4 wv = *reinterpret_cast<const float4*>(&sm.wf[pr][c0]);
    const float av[4] = {kf.x, kf.y, kf.z, kf.w}, qv[4] = {qf.x, qf.y, qf.z, qf.w};
    const float bv[4] = {kh.x * wv.x, kh.y * wv.y, kh.z * wv.z, kh.w * wv.w};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      ap = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s4], bv[s4], ap, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[s4], bv[s4], am, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void pm_pair_store(const PmSmem& sm, const BwdTiles& w, int64_t bidx, int pr,
                                              const bg_f32x4& ap, const bg_f32x4& am) {
  const int rb = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
  const int ib = pr - rb * (rb + 1) / 2;
  const int lane = threadIdx.x & 63, q4 = lane >> 4, m16 = lane & 15;
  const int i = 16 * ib + m16;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = 16 * rb + 4 * q4 + t;
    const float pv = i < r ? ap[t] : 0.f;
    const int64_t o = bidx * (C * C) + (int64_t)r * C + i;
    w.P[o] = pv;
    w.A[o] = sm.beta[r] * pv;
    w.M[o] = i <= r ? am[t] : 0.f;
  }
}

// Thread t's share of one channel half: channels 4 (t % 16) .. +3 of the half, rows
// 4 (t / 16) .. +3 (G as formed by the prep, k and q from the inputs), and the block
// references of its 16-row block b = t / 64: X_b (zero for b = 0) and X_{b+1}, with X_j
// the G row 16 j - 1.
struct PmLoads {
  float4 G[4], xb, xe;
  uint2 k[4], q[4];
};

__device__ __forceinline__ void pm_load(const BwdParams& p, const BwdTiles& w, int64_t bidx, int h,
                                        int64_t bos, int64_t c, int valid, int half, PmLoads& L) {
  const int t = threadIdx.x, c4 = PMH * half + 4 * (t & 15), rg = t >> 4, b = rg >> 2;
  const int HD = p.H * D;
  const float* Gb = w.G + bidx * (C * D);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * rg + i;
    L.G[i] = *reinterpret_cast<const float4*>(Gb + r * D + c4);
    const bool in = r < valid;
    const int64_t row = (bos + c * C + (in ? r : 0)) * (int64_t)HD + (int64_t)h * D + c4;
    L.k[i] = in ? *reinterpret_cast<const uint2*>(p.k + row) : make_uint2(0u, 0u);
    L.q[i] = in ? *reinterpret_cast<const uint2*>(p.q + row) : make_uint2(0u, 0u);
  }
  L.xb = b == 0 ? make_float4(0.f, 0.f, 0.f, 0.f)
                : *reinterpret_cast<const float4*>(Gb + (16 * b - 1) * D + c4);
  L.xe = *reinterpret_cast<const float4*>(Gb + (16 * b + 15) * D + c4);
}

// The half's operands into LDS: K F, Q F, K H, the block references and the pair
// factors w(rb, ib) = exp(X_rb - X_{ib+1}).  Ends with a barrier.
__device__ __forceinline__ void pm_stage(PmSmem& sm, const PmLoads& L) {
  const int t = threadIdx.x, cl = 4 * (t & 15), rg = t >> 4;
  const float xb[4] = {L.xb.x, L.xb.y, L.xb.z, L.xb.w};
  const float xe[4] = {L.xe.x, L.xe.y, L.xe.z, L.xe.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * rg + i;
    const float g4[4] = {L.G[i].x, L.G[i].y, L.G[i].z, L.G[i].w};
    const float kf[4] = {bf2f_u16(L.k[i].x & 0xffff), bf2f_u16(L.k[i].x >> 16),
                         bf2f_u16(L.k[i].y & 0xffff), bf2f_u16(L.k[i].y >> 16)};
    const float qf[4] = {bf2f_u16(L.q[i].x & 0xffff), bf2f_u16(L.q[i].x >> 16),
                         bf2f_u16(L.q[i].y & 0xffff), bf2f_u16(L.q[i].y >> 16)};
    float kF[4], qF[4], kH[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float F = exp_n(g4[e] - xb[e]), H = exp_n(xe[e] - g4[e]);
      kF[e] = kf[e] * F;
      qF[e] = qf[e] * F;
      kH[e] = kf[e] * H;
    }
    *reinterpret_cast<float4*>(&sm.kF[r][cl]) = make_float4(kF[0], kF[1], kF[2], kF[3]);
    *reinterpret_cast<float4*>(&sm.qF[r][cl]) = make_float4(qF[0], qF[1], qF[2], qF[3]);
    *reinterpret_cast<float4*>(&sm.kH[r][cl]) = make_float4(kH[0], kH[1], kH[2], kH[3]);
  }
  // the first row group of each block holds X_b and X_{b+1}
  if ((rg & 3) == 0) {
    const int b = rg >> 2;
    if (b == 0) *reinterpret_cast<float4*>(&sm.X[0][cl]) = L.xb;
    *reinterpret_cast<float4*>(&sm.X[b + 1][cl]) = L.xe;
  }
  __syncthreads();  // the block references in LDS
  for (int x = t; x < kPairs * PMH; x += 256) {
    const int pr = x / PMH, cc = x % PMH;
    const int rb = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
    const int ib = pr - rb * (rb + 1) / 2;
    sm.wf[pr][cc] = exp_n(sm.X[rb][cc] - sm.X[ib + 1][cc]);
  }
  __syncthreads();
}

// pairs (0,0) (1,0) (3,2); (1,1) (2,0) (2,1); (2,2) (3,0); (3,1) (3,3)
// (one 4-bit pair index per slot, no table in memory)
__device__ __forceinline__ int pm_wave_pair(int wave, int k) {
  const unsigned packed = wave == 0 ? 0x810u : wave == 1 ? 0x432u : wave == 2 ? 0x65u : 0x97u;
  return (int)((packed >> (4 * k)) & 15u);
}

__global__ void __launch_bounds__(256, 2) bwd_pm_kernel(BwdParams p, BwdTiles w) {
  __shared__ PmSmem sm;
  const int64_t bidx = blockIdx.x;
  int h, valid, n;
  int64_t bos, c;
  bwd_chunk_rows(p, bidx, h, bos, c, valid, n);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  if (t < C) sm.beta[t] = w.beta[bidx * C + t];
  PmLoads L;
  pm_load(p, w, bidx, h, bos, c, valid, 0, L);
  pm_stage(sm, L);
  pm_load(p, w, bidx, h, bos, c, valid, 1, L);   // in flight during the first half's products
  // blocks above the diagonal
  for (int x = t; x < C * C; x += 256) {
    const int r = x / C, i = x % C;
    if ((i >> 4) > (r >> 4)) {
      const int64_t o = bidx * (C * C) + x;
      w.P[o] = 0.f;
      w.A[o] = 0.f;
      w.M[o] = 0.f;
    }
  }
  const bg_f32x4 z4 = bg_f32x4{0.f, 0.f, 0.f, 0.f};
  bg_f32x4 ap[3] = {z4, z4, z4}, am[3] = {z4, z4, z4};
  const int npairs = wave < 2 ? 3 : 2;
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (k < npairs) pm_pair_acc(sm, pm_wave_pair(wave, k), ap[k], am[k]);
  __syncthreads();  // the first half's operands are read
  pm_stage(sm, L);
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (k < npairs) pm_pair_acc(sm, pm_wave_pair(wave, k), ap[k], am[k]);
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (k < npairs) pm_pair_store(sm, w, bidx, pm_wave_pair(wave, k), ap[k], am[k]);
}

// ---------------------------------------------------------------- gated triangle products
// The gradient terms that pair exp(G_r) with exp(-G_i), per channel c:
//   dqi_r = sum_{i <= r} dM_ri k_i exp(G_r - G_i)          (dM kh, through qg's gate)
//   dka_r = beta_r sum_{i < r} dA_ri k_i exp(G_r - G_i)    (diag(b) dA kh, through kg's gate)
//   dkh_i = sum_{r >= i} (dM_ri q_r + dA_ri beta_r k_r) exp(G_r - G_i)   (dkh through kh)
// With the block references, dqi_r = F_r sum_{ib <= rb} w(rb, ib) [dM_(rb,ib) (k H)_ib]_r and
// dkh_i = H_i sum_{rb >= ib} w(rb, ib) [dM_(rb,ib)^T (q F)_rb + dA_(rb,ib)^T (b k F)_rb]_i, each
// bracket a 16 x 16 x 16 product on the fp32 matrix cores (dM, dA are already masked).  One
// workgroup per (batch, 32-channel slice); wave v forms row block v of dqi and dka and row
// block v of dkh, five block products of each kind per wave.  The same workgroup then
// finishes its channels: the gradients through each gate, ungated,
//   dq  = (dO' S^T) Gam + dqi                        (dqg Gam)
//   dkg = -diag(b) (dY S^T) Gam + dka                 (dkg Gam)
//   dkh                                               (dkh / Gam, formed ungated)
//   dkp = (U dSn^T) exp(G_last - G)                   (dkp gam / Gam)
// so that dqg qg = dq q, dkg kg = dkg' k, dkh kh = dkh' k and dkp kp = dkp' k; then
// dG_r = dq q + (dkg - dkh - dkp) k per channel, dq, dk = dkg + dkh + dkp, and
// dg_t = sum_{r >= t} dG_r + dG_last with dG_last = sum_r dkp k + the state term.
constexpr int GSL = 32, GSS = GSL + 4;
struct alignas(16) GatedSmem {
  union {
    float kH[C][GSS];
    float dG[C][GSS];      // per row and channel, once the products are done
  };
  union {
    float qF[C][GSS];
    float gl[16][GSL];     // partial sums of dkp k over rows, once the products are done
  };
  float bkF[C][GSS];
  float G[C][GSS];
  float dM[C][C + 4];
  float dA[C][C + 4];
  float wf[kPairs][GSL];
  float X[5][GSL];
  float part[8][GSL];      // sums of dG over 8-row groups, for the reverse sum
  float beta[C];
};

__global__ void __launch_bounds__(256) bwd_gated_kernel(BwdParams p, BwdTiles w) {
  __shared__ GatedSmem sm;
  const int64_t bidx = blockIdx.x / (D / GSL);
  const int c0 = (blockIdx.x % (D / GSL)) * GSL;
  int h, valid, n;
  int64_t bos, c;
  bwd_chunk_rows(p, bidx, h, bos, c, valid, n);
  if (valid == 0) return;  // the finalize writes nothing for this batch
  const int t = threadIdx.x;
  const int HD = p.H * D;
  const float* Gb = w.G + bidx * (C * D) + c0;
  // every load first: thread t takes channels 4 (t % 8) .. +3 of the slice and rows
  // 2 (t / 8) .. +1 (G, k, q), and 16 entries each of dM and dA
  const int cg = t & 7, rg = t >> 3, c4 = 4 * cg;
  const int b = rg >> 3;  // the 16-row block of this thread's rows
  const float bt = t < C ? w.beta[bidx * C + t] : 0.f;
  float4 Gv[2], mv[4], av[4];
  uint2 kv[2], qv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 2 * rg + i;
    Gv[i] = *reinterpret_cast<const float4*>(Gb + r * D + c4);
    const bool in = r < valid;
    const int64_t row = (bos + c * C + (in ? r : 0)) * (int64_t)HD + (int64_t)h * D + c0 + c4;
    kv[i] = in ? *reinterpret_cast<const uint2*>(p.k + row) : make_uint2(0u, 0u);
    qv[i] = in ? *reinterpret_cast<const uint2*>(p.q + row) : make_uint2(0u, 0u);
  }
  // the block references of this thread's block: X_b (zero for b = 0) and X_{b+1}, with
  // X_j the G row 16 j - 1 (loaded as such: an indexed register array would go to scratch)
  const float4 xb4 = b == 0 ? make_float4(0.f, 0.f, 0.f, 0.f)
                            : *reinterpret_cast<const float4*>(Gb + (16 * b - 1) * D + c4);
  const float4 xe4 = *reinterpret_cast<const float4*>(Gb + (16 * b + 15) * D + c4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = t + 256 * j, r = x >> 4, i4 = (x & 15) * 4;
    mv[j] = *reinterpret_cast<const float4*>(w.dM + bidx * (C * C) + r * C + i4);
    av[j] = *reinterpret_cast<const float4*>(w.dA + bidx * (C * C) + r * C + i4);
  }
  // the finishing step's operands at the product layout (lane (q4, m16) of wave v:
  // rows 16 v + 4 q4 + e, channels 16 ct + m16 of the slice): issued now, used last
  const int v0 = t >> 6, q40 = (t & 63) >> 4, m160 = t & 15;
  float fq[2][4], fk[2][4], fp[2][4];
  uint32_t kq[2][4];   // k (low half) and q (high half) as bf16
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * v0 + 4 * q40 + e, cc = 16 * ct + m160;
      const int64_t o = bidx * (C * D) + (int64_t)r * D + c0 + cc;
      fq[ct][e] = w.dqg[o];
      fk[ct][e] = w.dkg[o];
      fp[ct][e] = w.dkp[o];
      const bool in = r < valid;
      const int64_t row = (bos + c * C + (in ? r : 0)) * (int64_t)HD + (int64_t)h * D + c0 + cc;
      kq[ct][e] = in ? (uint32_t)p.k[row] | ((uint32_t)p.q[row] << 16) : 0u;
    }
  if (t < C) sm.beta[t] = bt;
  if ((rg & 7) == 0) {  // the first row group of each block
    if (b == 0) *reinterpret_cast<float4*>(&sm.X[0][c4]) = xb4;
    *reinterpret_cast<float4*>(&sm.X[b + 1][c4]) = xe4;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = t + 256 * j, r = x >> 4, i4 = (x & 15) * 4;
    *reinterpret_cast<float4*>(&sm.dM[r][i4]) = mv[j];
    *reinterpret_cast<float4*>(&sm.dA[r][i4]) = av[j];
  }
  __syncthreads();  // beta
  {
    const float xb[4] = {xb4.x, xb4.y, xb4.z, xb4.w};
    const float xe[4] = {xe4.x, xe4.y, xe4.z, xe4.w};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 2 * rg + i;
      const float g4[4] = {Gv[i].x, Gv[i].y, Gv[i].z, Gv[i].w};
      const float kf[4] = {bf2f_u16(kv[i].x & 0xffff), bf2f_u16(kv[i].x >> 16),
                           bf2f_u16(kv[i].y & 0xffff), bf2f_u16(kv[i].y >> 16)};
      const float qf[4] = {bf2f_u16(qv[i].x & 0xffff), bf2f_u16(qv[i].x >> 16),
                           bf2f_u16(qv[i].y & 0xffff), bf2f_u16(qv[i].y >> 16)};
      const float br = sm.beta[r];
      float kH[4], qF[4], bkF[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float F = exp_n(g4[e] - xb[e]), H = exp_n(xe[e] - g4[e]);
        kH[e] = kf[e] * H;
        qF[e] = qf[e] * F;
        bkF[e] = br * kf[e] * F;
      }
      *reinterpret_cast<float4*>(&sm.G[r][c4]) = Gv[i];
      *reinterpret_cast<float4*>(&sm.kH[r][c4]) = make_float4(kH[0], kH[1], kH[2], kH[3]);
      *reinterpret_cast<float4*>(&sm.qF[r][c4]) = make_float4(qF[0], qF[1], qF[2], qF[3]);
      *reinterpret_cast<float4*>(&sm.bkF[r][c4]) = make_float4(bkF[0], bkF[1], bkF[2], bkF[3]);
    }
    for (int x = t; x < kPairs * GSL; x += 256) {
      const int pr = x / GSL, ch = x % GSL;
      const int rb = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
      const int ib = pr - rb * (rb + 1) / 2;
      sm.wf[pr][ch] = exp_n(sm.X[rb][ch] - sm.X[ib + 1][ch]);
    }
  }
  __syncthreads();
  const int v = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63, q4 = lane >> 4, m16 = lane & 15;
  const bg_f32x4 z4 = bg_f32x4{0.f, 0.f, 0.f, 0.f};
  float dqi[2][4], dka[2][4], dkh[2][4];
  // ---- row form: rows of block rb = v
  {
    const int rb = v;
    bg_f32x4 aq[2] = {z4, z4}, ak[2] = {z4, z4};
    for (int ib = 0; ib <= rb; ++ib) {
      bg_f32x4 tq[2] = {z4, z4}, tk[2] = {z4, z4};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int i = 16 * ib + 4 * s4 + q4;  // the contraction row of this lane
        const float am = sm.dM[16 * rb + m16][i], aa = sm.dA[16 * rb + m16][i];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const float bk = sm.kH[i][16 * ct + m16];
          tq[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(am, bk, tq[ct], 0, 0, 0);
          tk[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(aa, bk, tk[ct], 0, 0, 0);
        }
      }
      const int pr = bwd_pair(rb, ib);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float wv = sm.wf[pr][16 * ct + m16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          aq[ct][e] = fmaf(wv, tq[ct][e], aq[ct][e]);
          ak[ct][e] = fmaf(wv, tk[ct][e], ak[ct][e]);
        }
      }
    }
    // lane holds rows 16 rb + 4 q4 + e, channel 16 ct + m16 of the slice
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * q4 + e, cc = 16 * ct + m16;
        const float F = exp_n(sm.G[r][cc] - sm.X[rb][cc]);
        dqi[ct][e] = F * aq[ct][e];
        dka[ct][e] = sm.beta[r] * F * ak[ct][e];
      }
  }
  // ---- column form: rows of block ib = v
  {
    const int ib = v;
    bg_f32x4 ah[2] = {z4, z4};
    for (int rb = ib; rb < 4; ++rb) {
      bg_f32x4 th[2] = {z4, z4};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int r = 16 * rb + 4 * s4 + q4;  // the contraction row of this lane
        const float am = sm.dM[r][16 * ib + m16], aa = sm.dA[r][16 * ib + m16];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          th[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(am, sm.qF[r][16 * ct + m16], th[ct], 0, 0, 0);
          th[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(aa, sm.bkF[r][16 * ct + m16], th[ct], 0, 0, 0);
        }
      }
      const int pr = bwd_pair(rb, ib);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float wv = sm.wf[pr][16 * ct + m16];
#pragma unroll
        for (int e = 0; e < 4; ++e) ah[ct][e] = fmaf(wv, th[ct][e], ah[ct][e]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * ib + 4 * q4 + e, cc = 16 * ct + m16;
        const float H = exp_n(sm.X[ib + 1][cc] - sm.G[i][cc]);
        dkh[ct][e] = H * ah[ct][e];
      }
  }
  __syncthreads();  // every read of kH and qF is done: dG and gl overlay them
  // ---- finish the slice's channels: dq, dk, and dG for the reverse sum
  {
    float glp[2] = {0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * v + 4 * q4 + e, cc = 16 * ct + m16;
        const float G = sm.G[r][cc];
        const float eg = exp_n(G), el = exp_n(sm.G[C - 1][cc] - G);
        const float dq = fq[ct][e] * eg + dqi[ct][e];
        const float dkg = fk[ct][e] * eg + dka[ct][e];
        const float dkp = fp[ct][e] * el;
        const float kf = bf2f_u16((uint16_t)(kq[ct][e] & 0xffff));
        const float qf = bf2f_u16((uint16_t)(kq[ct][e] >> 16));
        sm.dG[r][cc] = dq * qf + (dkg - dkh[ct][e] - dkp) * kf;
        glp[ct] += dkp * kf;
        if (r < valid) {
          const int64_t row = (bos + c * C + r) * (int64_t)HD + (int64_t)h * D + c0 + cc;
          p.dq[row] = dq;
          p.dk[row] = dkg + dkh[ct][e] + dkp;
        }
      }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) sm.gl[4 * v + q4][16 * ct + m16] = glp[ct];
  }
  __syncthreads();
  // dg_t = dG_last + sum_{r >= t} dG_r, with dG_last the kp terms of every row and the
  // state's direct share: thread t takes channel t % 32 and rows 8 (t / 32) .. +7; the
  // eight row groups' sums go through LDS, then each thread walks its rows last first
  {
    const int ch = t & (GSL - 1), g8 = t >> 5;
    float dgv[8], part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dgv[i] = sm.dG[8 * g8 + i][ch];
      part += dgv[i];
    }
    sm.part[g8][ch] = part;
    float run = w.dgl[bidx * D + c0 + ch];
#pragma unroll
    for (int x = 0; x < 16; ++x) run += sm.gl[x][ch];
    __syncthreads();  // the row groups' sums
#pragma unroll
    for (int g = 1; g < 8; ++g)
      if (g > g8) run += sm.part[g][ch];
    float* dg = p.dg + ((bos + c * C) * (int64_t)p.H + h) * D + c0 + ch;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      const int r = 8 * g8 + i;
      run += dgv[i];
      if (r < valid) dg[(int64_t)r * p.H * D] = run;
    }
  }
}

// ---------------------------------------------------------------- T = (I + A)^-1
// A strictly lower 64 x 64; thread j forms column j by forward substitution.
__global__ void __launch_bounds__(64) bwd_inverse_kernel(const float* A, float* T) {
  __shared__ float As[C][C + 1];
  const int64_t b = blockIdx.x;
  const int j = threadIdx.x;
  for (int r = 0; r < C; ++r) As[r][j] = A[b * C * C + r * C + j];
  __syncthreads();
  float col[C];
#pragma unroll
  for (int r = 0; r < C; ++r) {
    float v = r == j ? 1.f : 0.f;
    if (r > j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s = fmaf(As[r][i], col[i], s);
      v = -s;
    }
    col[r] = v;
  }
#pragma unroll
  for (int r = 0; r < C; ++r) T[b * C * C + r * C + j] = col[r];
}

// ---------------------------------------------------------------- serial dS
// Column j of dS depends only on column j of dSn (Diag(gam), kp and F act on
// rows), so each (sequence, head) runs as D / 16 workgroups of 16 value columns.
// Chunks last to first: dSn(c) is stored for the chunk's gradient products, the
// chunk's dU = kp dSn + M^T dO' is formed and stored, and
// dS = Diag(gam) dSn - F dU + qg^T dO' becomes the next dSn (the same as
// Diag(gam) dSn - F (kp dSn) + X with X = qg^T dO' - F M^T dO').  The sequence's
// initial-state gradient is the last dS.
//  * Both products run on the fp32 matrix cores (16x16x4): wave w forms rows
//    16w .. 16w+15 of dU = kp dSn + M^T dO' and rows 32w .. 32w+31 of dS.  The k index of a
//    product is permuted so that each lane's A operand is one contiguous run
//    (k = 32q + s for P, 16q + s for F P over steps s), loaded as float4s.
//  * dS stays in the MFMA accumulators (rows 32w + 16it + 4q + t, column m); a
//    transposed copy in LDS is the B operand of the next chunk's kp dSn, and dU
//    goes through LDS (transposed) as the B operand of F dU.
//  * The operands (kp, F, qg^T dO', M^T dO', gam) of the next two chunks are in flight
//    while a chunk computes: three register sets in rotation, the loop unrolled by three
//    so that no copy between sets waits for a load.
//  * The 8 column slices of one (sequence, head) run on one XCD (workgroups go
//    to the XCDs round robin), so the chunk's kp and F, which every slice reads,
//    come from that XCD's L2 after the first slice's fetch.
struct ScanOps {
  float4 kp[8];       // kp[16w + m][32q .. 32q + 31]
  float4 f[2][4];     // F[32w + 16it + m][16q .. 16q + 15]
  float x[2][4];      // (qg^T dO')[32w + 16it + 4q + t][j0 + m]
  float mt[4];        // (M^T dO')[16w + 4q + t][j0 + m]
  float4 gam[2];      // gam[32w + 16it + 4q .. + 3]
};

__device__ __forceinline__ void scan_fetch(const BwdTiles& w, int64_t bidx, int j0, int wave, int q, int m,
                                           ScanOps& o) {
  const float* kp = w.kp + bidx * (C * D) + (16 * wave + m) * D + 32 * q;
#pragma unroll
  for (int i = 0; i < 8; ++i) o.kp[i] = *reinterpret_cast<const float4*>(kp + 4 * i);
  const float* mt = w.MtdO + bidx * (C * D) + (size_t)(16 * wave + 4 * q) * D + j0 + m;
#pragma unroll
  for (int t = 0; t < 4; ++t) o.mt[t] = mt[(size_t)t * D];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const float* F = w.F + bidx * (D * C) + (32 * wave + 16 * it + m) * C + 16 * q;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.f[it][i] = *reinterpret_cast<const float4*>(F + 4 * i);
    const int r0 = 32 * wave + 16 * it + 4 * q;
    const float* X = w.X + bidx * (D * D) + (size_t)r0 * D + j0 + m;
#pragma unroll
    for (int t = 0; t < 4; ++t) o.x[it][t] = X[(size_t)t * D];
    o.gam[it] = *reinterpret_cast<const float4*>(w.gam + bidx * D + r0);
  }
}

__global__ void __launch_bounds__(256) bwd_ds_scan_kernel(BwdParams p, BwdTiles w) {
  constexpr int DSW = 16, DSC = D / DSW;
  __shared__ float dsT[DSW][D + 4];   // dSn, transposed: dsT[j][k]
  __shared__ float pT[DSW][C + 4];    // dU = kp dSn + M^T dO', transposed: pT[j][r]
  // workgroup b: slice (b / 8) % DSC of pair (b / (8 DSC)) * 8 + b % 8, so that all
  // slices of a pair share b % 8 (their XCD)
  const int b = blockIdx.x;
  const int pair = (b / (8 * DSC)) * 8 + b % 8, j0 = ((b / 8) % DSC) * DSW;
  if (pair >= p.nseq * p.H) return;   // the same for the whole workgroup
  const int n = pair / p.H, h = pair % p.H;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63, q = lane >> 4, m = lane & 15;
  const int64_t bos = seq_bos(p, n), len = seq_len_of(p, n);
  const int nch = (int)((len + C - 1) / C);
  const size_t sd = (size_t)D * D;
  // the sequence's chunks in this group's slots: c_lo .. c_hi - 1 (chunk c is slot
  // s_first + c); a sequence without chunks belongs to the group holding slot s_first
  const int64_t s_first = n + bos / C;
  const int64_t lo = p.slot0 > s_first ? p.slot0 - s_first : 0;
  const int64_t hi = p.slot1 - s_first < nch ? p.slot1 - s_first : nch;
  if (nch == 0 ? (s_first < p.slot0 || s_first >= p.slot1) : lo >= hi) return;  // uniform
  const int c_lo = (int)lo, c_hi = (int)hi;
  // this lane's dS entries: rows 32w + 16it + 4q + tt, column j0 + m; the scan starts
  // from dL/dS_final at the sequence's last chunk, else from the group above's carry
  bg_f32x4 ds[2];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const size_t e = (size_t)(32 * wave + 16 * it + 4 * q + tt) * D + j0 + m;
      float v = 0.f;
      if (c_hi < nch) {
        v = p.carry_in[(size_t)h * sd + e];
      } else if (p.dsT) {
        const size_t o = ((size_t)n * p.H + h) * sd + e;
        v = p.dsT_fp32 ? static_cast<const float*>(p.dsT)[o] : bf2f_u16(static_cast<const uint16_t*>(p.dsT)[o]);
      }
      ds[it][tt] = v;
    }
#pragma unroll
  for (int it = 0; it < 2; ++it)
    *reinterpret_cast<float4*>(&dsT[m][32 * wave + 16 * it + 4 * q]) = make_float4(ds[it][0], ds[it][1], ds[it][2], ds[it][3]);
  const int64_t b_first = (s_first - p.slot0) * p.H + h;   // tile index of chunk 0 (may be negative)
  auto fetch = [&](int c, ScanOps& o) __attribute__((always_inline)) {
    scan_fetch(w, b_first + (int64_t)c * p.H, j0, wave, q, m, o);
  };
  // one chunk of the recurrence with its operands in `cur`
  auto step = [&](int c, const ScanOps& cur) __attribute__((always_inline)) {
    const int64_t bidx = b_first + (int64_t)c * p.H;
    {  // dSn(c) for the chunk's gradient products
      float* dsn = w.dSn + bidx * sd;
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          dsn[(size_t)(32 * wave + 16 * it + 4 * q + tt) * D + j0 + m] = ds[it][tt];
    }
    {  // dU rows 16w .. 16w+15 = kp dSn + M^T dO', k = 32q + s, in four independent chains
      bg_f32x4 acc[4] = {};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 bv = *reinterpret_cast<const float4*>(&dsT[m][32 * q + 4 * i]);
        const float av[4] = {cur.kp[i].x, cur.kp[i].y, cur.kp[i].z, cur.kp[i].w};
        const float bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bw[e], acc[e], 0, 0, 0);
      }
      const bg_f32x4 pv = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      float du[4];
      float* dug = w.dU + bidx * (C * D) + (size_t)(16 * wave + 4 * q) * D + j0 + m;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        du[tt] = pv[tt] + cur.mt[tt];
        dug[(size_t)tt * D] = du[tt];
      }
      *reinterpret_cast<float4*>(&pT[m][16 * wave + 4 * q]) = make_float4(du[0], du[1], du[2], du[3]);
    }
    __syncthreads();  // dU complete; every read of dsT done
    // dS = gam (.) dSn + qg^T dO' - F dU, k = 16q + s, in two independent chains per row tile
    {
      bg_f32x4 acc[2][2] = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 bv = *reinterpret_cast<const float4*>(&pT[m][16 * q + 4 * i]);
        const float bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const float av[4] = {cur.f[it][i].x, cur.f[it][i].y, cur.f[it][i].z, cur.f[it][i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[it][e & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bw[e], acc[it][e & 1], 0, 0, 0);
        }
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const float gv[4] = {cur.gam[it].x, cur.gam[it].y, cur.gam[it].z, cur.gam[it].w};
        const bg_f32x4 fp = acc[it][0] + acc[it][1];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) ds[it][tt] = fmaf(gv[tt], ds[it][tt], cur.x[it][tt]) - fp[tt];
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it)
      *reinterpret_cast<float4*>(&dsT[m][32 * wave + 16 * it + 4 * q]) = make_float4(ds[it][0], ds[it][1], ds[it][2], ds[it][3]);
    __syncthreads();  // the new dS is in place; every read of pT done
  };
  // Chunks last to first with two chunks' operands in flight ahead of the one being
  // computed: three operand sets in rotation, the loop unrolled by three so that no
  // copy between sets waits for a load.
  ScanOps o0, o1, o2;
  if (c_hi - 1 >= c_lo) fetch(c_hi - 1, o0);
  if (c_hi - 2 >= c_lo) fetch(c_hi - 2, o1);
  __syncthreads();
  for (int c = c_hi - 1; c >= c_lo; c -= 3) {
    if (c - 2 >= c_lo) fetch(c - 2, o2);
    step(c, o0);
    if (c - 1 < c_lo) break;
    if (c - 3 >= c_lo) fetch(c - 3, o0);
    step(c - 1, o1);
    if (c - 2 < c_lo) break;
    if (c - 4 >= c_lo) fetch(c - 4, o1);
    step(c - 2, o2);
  }
  // the sequence's initial-state gradient, or the carry for the group below
  float* o = c_lo > 0 ? p.carry_out + (size_t)h * sd : p.ds0 ? p.ds0 + ((size_t)n * p.H + h) * sd : nullptr;
  if (o != nullptr) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o[(size_t)(32 * wave + 16 * it + 4 * q + tt) * D + j0 + m] = ds[it][tt];
  }
}

// The scan's launch: 16-column slices, eight per (sequence, head); the grid is a
// multiple of 64 workgroups (the XCD-aware mapping) and the extra ones exit at once.
void launch_ds_scan(const BwdParams& p, const BwdTiles& w, hipStream_t s) {
  const int64_t pairs = (int64_t)p.nseq * p.H;
  const int64_t groups = (pairs + 7) / 8;
  hipLaunchKernelGGL(bwd_ds_scan_kernel, dim3((unsigned)(groups * 8 * (D / 16))), dim3(256), 0, s, p, w);
}

// ---------------------------------------------------------------- rows past the sequences
// With cu_seqlens, rows cu_seqlens[num_seqs] .. T - 1 belong to no sequence and get
// zero gradients (every other row is written by the finalize and dbeta / dv
// kernels).  Their extent is known on the device only, so a kernel clears them.
__global__ void __launch_bounds__(256) bwd_clear_tail_kernel(BwdParams p) {
  const int64_t r0 = p.cu[p.nseq];
  const int64_t n = (p.T - r0) * p.H;   // (row, head) pairs to clear
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n * (D / 4); i += stride) {
    const int64_t o = r0 * p.H * (D / 4) + i;   // float4 index
    reinterpret_cast<float4*>(p.dq)[o] = z;
    reinterpret_cast<float4*>(p.dk)[o] = z;
    reinterpret_cast<float4*>(p.dv)[o] = z;
    reinterpret_cast<float4*>(p.dg)[o] = z;
    if (i < n) p.dbeta[r0 * p.H + i] = 0.f;
  }
}

// ---------------------------------------------------------------- gates and scatter
// Terms that need no gated gradient, on the side stream while the gated terms run:
//  * the state's direct share of dG_last, gam_c sum_j S_cj dSn_cj per channel c;
//  * dbeta_r = sum_j dY_rj R_rj + sum_i dA_ri P_ri and dv_r = beta_r dY_r per row.
// Sixteen lanes share a row, each with eight consecutive entries (coalesced), and
// their sums meet through lane exchanges within the sixteen.
__global__ void __launch_bounds__(256) bwd_state_term_kernel(BwdParams p, BwdTiles w) {
  const int64_t bidx = blockIdx.x;
  if (w.valid[bidx] == 0) return;
  const int t = threadIdx.x, jq = t & 15;
  const float* S = w.S + bidx * (size_t)(D * D);
  const float* dsn = w.dSn + bidx * (size_t)(D * D);
#pragma unroll 2
  for (int it = 0; it < D / 16; ++it) {
    const int r = 16 * it + (t >> 4);
    const float4 a0 = *reinterpret_cast<const float4*>(S + (size_t)r * D + 8 * jq);
    const float4 a1 = *reinterpret_cast<const float4*>(S + (size_t)r * D + 8 * jq + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(dsn + (size_t)r * D + 8 * jq);
    const float4 b1 = *reinterpret_cast<const float4*>(dsn + (size_t)r * D + 8 * jq + 4);
    float sum = a0.x * b0.x + a0.y * b0.y + a0.z * b0.z + a0.w * b0.w +
                a1.x * b1.x + a1.y * b1.y + a1.z * b1.z + a1.w * b1.w;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
    if (jq == 0) w.dgl[bidx * D + r] = sum * w.gam[bidx * D + r];
  }
}

__global__ void __launch_bounds__(256) bwd_dbeta_dv_kernel(BwdParams p, BwdTiles w) {
  const int64_t bidx = blockIdx.x;
  const int valid = w.valid[bidx];
  if (valid == 0) return;
  const int64_t slot = p.slot0 + bidx / p.H;
  const int h = (int)(bidx % p.H);
  const int n = slot_seq(p, slot);
  const int64_t bos = seq_bos(p, n);
  const int64_t c = slot - (n + bos / C);
  const int t = threadIdx.x, jq = t & 15;
  const int64_t tb = bidx * (C * D);
  const float* beta = w.beta + bidx * C;
#pragma unroll
  for (int it = 0; it < C / 16; ++it) {
    const int r = 16 * it + (t >> 4);
    const float* dy = w.dY + tb + (size_t)r * D + 8 * jq;
    const float* rr = w.R + tb + (size_t)r * D + 8 * jq;
    const float* da = w.dA + bidx * C * C + (size_t)r * C + 4 * jq;
    const float* pp = w.P + bidx * C * C + (size_t)r * C + 4 * jq;
    const float4 y0 = *reinterpret_cast<const float4*>(dy), y1 = *reinterpret_cast<const float4*>(dy + 4);
    const float4 q0 = *reinterpret_cast<const float4*>(rr), q1 = *reinterpret_cast<const float4*>(rr + 4);
    const float4 a = *reinterpret_cast<const float4*>(da), b = *reinterpret_cast<const float4*>(pp);
    float sum = y0.x * q0.x + y0.y * q0.y + y0.z * q0.z + y0.w * q0.w +
                y1.x * q1.x + y1.y * q1.y + y1.z * q1.z + y1.w * q1.w +
                a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
    if (r < valid) {
      const int64_t row = (bos + c * C + r) * (int64_t)p.H + h;
      if (jq == 0) p.dbeta[row] = sum;
      const float br = beta[r];
      float* dv = p.dv + row * D + 8 * jq;
      *reinterpret_cast<float4*>(dv) = make_float4(br * y0.x, br * y0.y, br * y0.z, br * y0.w);
      *reinterpret_cast<float4*>(dv + 4) = make_float4(br * y1.x, br * y1.y, br * y1.z, br * y1.w);
    }
  }
}

template <int NT>
void gemm_nt(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.N / NT, a.M / 64, a.batches), block(256);
  if (!ta && !tb) hipLaunchKernelGGL((bgemm_kernel<NT, false, false>), grid, block, 0, s, a);
  else if (!ta && tb) hipLaunchKernelGGL((bgemm_kernel<NT, false, true>), grid, block, 0, s, a);
  else if (ta && !tb) hipLaunchKernelGGL((bgemm_kernel<NT, true, false>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((bgemm_kernel<NT, true, true>), grid, block, 0, s, a);
}

// 64 x 128 tiles where N allows (op(A) is then read once per row block), else 64 x 64.
void gemm(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  if (a.N % 128 == 0) gemm_nt<128>(ta, tb, a, s);
  else gemm_nt<64>(ta, tb, a, s);
}

// op(A) M x K times op(B) K x N over every batch; strides are per-batch element counts.
GemmArgs mm(int M, int N, int K, const float* A, int64_t sA, int lda, const float* B, int64_t sB,
            int ldb, float* Cm, int64_t sC, int ldc, int batches) {
  GemmArgs a{};
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.sA = sA; a.lda = lda;
  a.B = B; a.sB = sB; a.ldb = ldb;
  a.C = Cm; a.sC = sC; a.ldc = ldc;
  a.alpha = 1.f;
  a.batches = batches;
  return a;
}

}  // namespace


hipError_t launch_bwd_scan_only(const BwdParams& p, hipStream_t s) {
  const BwdTiles w{};
  BwdParams q = p;   // without tokens sequence n sits at slot n: one group of every slot
  q.slot0 = 0;
  q.slot1 = (int64_t)p.nseq + 1;
  launch_ds_scan(q, w, s);
  return hipGetLastError();
}

hipError_t launch_bwd_chunk_local(const BwdParams& p, const BwdTiles& w, int64_t batches, hipStream_t s) {
  const int NB = (int)batches;
  const int64_t t1 = C * D, t2 = C * C, t3 = D * D, tf = D * C;
  // chunk tiles
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(NB), dim3(256), 0, s, p, w);
  // P = strict_lower(K K^T gated), A = diag(b) P, M = lower_incl(Q K^T gated)
  hipLaunchKernelGGL(bwd_pm_kernel, dim3(NB), dim3(256), 0, s, p, w);
  hipLaunchKernelGGL(bwd_inverse_kernel, dim3(NB), dim3(64), 0, s, w.A, w.T);
  // the scan's chunk-local operands: MtdO = M^T dO';  F = kg^T diag(b) T^T;  X = qg^T dO'
  {
    gemm(true, false, mm(C, D, C, w.M, t2, C, w.dO, t1, D, w.MtdO, t1, D, NB), s);
    GemmArgs f = mm(D, C, C, w.kg, t1, D, w.T, t2, C, w.F, tf, C, NB);
    f.ks = w.beta; f.sks = C;
    gemm(true, true, f, s);
    gemm(true, false, mm(D, D, C, w.qg, t1, D, w.dO, t1, D, w.X, t3, D, NB), s);
  }
  return hipGetLastError();
}

// Products that need the checkpoints but not the state gradients: R, U and dM.
// They may run beside the scan.
hipError_t launch_bwd_state_products(const BwdParams& p, const BwdTiles& w, int64_t batches,
                                     hipStream_t s) {
  const int NB = (int)batches;
  const int64_t t1 = C * D, t2 = C * C, t3 = D * D;
  // R = V - kg S;  U = T diag(b) R
  GemmArgs a = mm(C, D, D, w.kg, t1, D, w.S, t3, D, w.R, t1, D, NB);
  a.alpha = -1.f; a.Dm = w.vv; a.sD = t1; a.ldd = D;
  gemm(false, false, a, s);
  GemmArgs u = mm(C, D, C, w.T, t2, C, w.R, t1, D, w.U, t1, D, NB);
  u.ks = w.beta; u.sks = C;
  gemm(false, false, u, s);
  GemmArgs dm = mm(C, C, D, w.dO, t1, D, w.U, t1, D, w.dM, t2, C, NB);  // dM = lower_incl(dO' U^T)
  dm.mask = 2;
  gemm(false, true, dm, s);
  (void)p;
  return hipGetLastError();
}

// dO' S^T: needs the checkpoints only, and only the gated kernel reads it.
void launch_dos(const BwdTiles& w, int NB, hipStream_t s) {
  const int64_t t1 = C * D, t3 = D * D;
  gemm(false, true, mm(C, D, D, w.dO, t1, D, w.S, t3, D, w.dqg, t1, D, NB), s);
}

// The serial recurrence of dS over chunks: it reads only chunk-local tiles.
hipError_t launch_bwd_scan(const BwdParams& p, const BwdTiles& w, hipStream_t s) {
  launch_ds_scan(p, w, s);
  return hipGetLastError();
}

// The gradient products after the scan.  dY = T^T dU needs the scan only (it forms
// dU); dA = strict_lower(-dY U^T), -diag(b) dY S^T and the gated terms
// also need the state products (U, dM); dkp = U dSn^T needs both but nothing else
// here, so it may run beside them.
void launch_dy(const BwdTiles& w, int NB, hipStream_t s) {  // dY = T^T dU (the scan formed dU)
  const int64_t t1 = C * D, t2 = C * C;
  gemm(true, false, mm(C, D, C, w.T, t2, C, w.dU, t1, D, w.dY, t1, D, NB), s);
}

void launch_dkp(const BwdTiles& w, int NB, hipStream_t s) {
  const int64_t t1 = C * D, t3 = D * D;
  gemm(false, true, mm(C, D, D, w.U, t1, D, w.dSn, t3, D, w.dkp, t1, D, NB), s);  // dkp = U dSn^T
}

void launch_da(const BwdTiles& w, int NB, hipStream_t s) {
  const int64_t t1 = C * D, t2 = C * C;
  GemmArgs da = mm(C, C, D, w.dY, t1, D, w.U, t1, D, w.dA, t2, C, NB);  // dA = strict_lower(-dY U^T)
  da.alpha = -1.f; da.mask = 1;
  gemm(false, true, da, s);
}

void launch_dkg(const BwdTiles& w, int NB, hipStream_t s) {
  const int64_t t1 = C * D, t3 = D * D;
  GemmArgs k1 = mm(C, D, D, w.dY, t1, D, w.S, t3, D, w.dkg, t1, D, NB);  // -diag(b) dY S^T
  k1.rs = w.beta; k1.srs = C; k1.alpha = -1.f;
  gemm(false, true, k1, s);
}

// dM kh, diag(b) dA kh and dkh through the gates, with block references, and the
// final dq, dk and dg of every valid row
void launch_gated(const BwdParams& p, const BwdTiles& w, int NB, hipStream_t s) {
  hipLaunchKernelGGL(bwd_gated_kernel, dim3((unsigned)NB * (D / GSL)), dim3(256), 0, s, p, w);
}

hipError_t launch_bwd_streams(const Params& fwd, int fwd_splits, const BwdParams& p0, const BwdTiles& w0,
                              int64_t slots, int64_t group_slots, float* carry, hipStream_t hs,
                              hipStream_t side) {
  // Per group, caller's stream:  chunk-local tiles | scan (and dU) | dY | (forward) dkg,
  //                   dO' S^T | (state products) dA | (side terms) gated terms with dq, dk, dg
  //                   | (side) end
  // Side stream:      (fork) forward with checkpoints, first group only | (chunk-local) R, U,
  //                   dM | (scan) dkp, the state term of dG_last | (dA) dbeta, dv
  // Once the fork is recorded, the caller's stream always waits for the side stream
  // before this returns, so that later work on it (and the workspace's next use)
  // follows everything enqueued here; each group's tiles are reused by the next group
  // only after that group's end on both streams.
  hipEvent_t ev[8] = {};
  enum { kFork, kFwd, kLocal, kProducts, kScan, kSideTerms, kDA, kJoin };
  hipError_t err = hipSuccess;
  for (int i = 0; i < 8 && err == hipSuccess; ++i) err = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
  if (err == hipSuccess && p0.cu != nullptr) {
    hipLaunchKernelGGL(bwd_clear_tail_kernel, dim3(512), dim3(256), 0, hs, p0);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipEventRecord(ev[kFork], hs);
  if (err == hipSuccess) {
    auto on_side = [&](hipEvent_t after, auto&& launch) {  // side stream: wait, then enqueue
      if (err == hipSuccess) err = hipStreamWaitEvent(side, after, 0);
      if (err == hipSuccess) err = launch();
    };
    auto on_hs = [&](auto&& launch) {
      if (err == hipSuccess) {
        launch();
        err = hipGetLastError();
      }
    };
    const size_t sd = (size_t)D * D * p0.H;
    int k = 0;
    for (int64_t slot1 = slots; slot1 > 0 && err == hipSuccess; slot1 -= group_slots, ++k) {
      const int64_t slot0 = slot1 > group_slots ? slot1 - group_slots : 0;
      BwdParams p = p0;
      p.slot0 = slot0;
      p.slot1 = slot1;
      p.carry_in = carry ? carry + ((k + 1) & 1) * sd : nullptr;
      p.carry_out = carry ? carry + (k & 1) * sd : nullptr;
      BwdTiles w = w0;
      w.S = w0.S + (size_t)slot0 * sd;
      const int64_t batches = (slot1 - slot0) * p.H;
      const int NB = (int)batches;
      if (k == 0) {
        on_side(ev[kFork], [&] { return launch_fwd(fwd, fwd_splits, side); });
        if (err == hipSuccess) err = hipEventRecord(ev[kFwd], side);   // the checkpoints exist
      }
      if (err == hipSuccess) err = launch_bwd_chunk_local(p, w, batches, hs);
      if (err == hipSuccess) err = hipEventRecord(ev[kLocal], hs);
      on_side(ev[kLocal], [&] { return launch_bwd_state_products(p, w, batches, side); });
      if (err == hipSuccess) err = hipEventRecord(ev[kProducts], side);
      if (err == hipSuccess) err = launch_bwd_scan(p, w, hs);
      if (err == hipSuccess) err = hipEventRecord(ev[kScan], hs);
      on_side(ev[kScan], [&] {
        launch_dkp(w, NB, side);
        hipLaunchKernelGGL(bwd_state_term_kernel, dim3(NB), dim3(256), 0, side, p, w);
        return hipGetLastError();
      });
      if (err == hipSuccess) err = hipEventRecord(ev[kSideTerms], side);
      // the products that need only dY and the checkpoints run while the side stream
      // finishes the state products
      on_hs([&] { launch_dy(w, NB, hs); });
      if (err == hipSuccess) err = hipStreamWaitEvent(hs, ev[kFwd], 0);
      on_hs([&] {
        launch_dkg(w, NB, hs);
        launch_dos(w, NB, hs);
      });
      if (err == hipSuccess) err = hipStreamWaitEvent(hs, ev[kProducts], 0);
      on_hs([&] { launch_da(w, NB, hs); });
      if (err == hipSuccess) err = hipEventRecord(ev[kDA], hs);
      on_side(ev[kDA], [&] {
        hipLaunchKernelGGL(bwd_dbeta_dv_kernel, dim3(NB), dim3(256), 0, side, p, w);
        return hipGetLastError();
      });
      if (err == hipSuccess) err = hipStreamWaitEvent(hs, ev[kSideTerms], 0);
      on_hs([&] { launch_gated(p, w, NB, hs); });
      // the group's end on both streams before the next group reuses the tiles
      if (err == hipSuccess) err = hipEventRecord(ev[kJoin], side);
      if (err == hipSuccess) err = hipStreamWaitEvent(hs, ev[kJoin], 0);
    }
    if (err != hipSuccess) {  // the side stream's work may be unordered: wait on the host
      (void)hipStreamSynchronize(side);
    }
  }
  for (hipEvent_t e : ev)
    if (e != nullptr) (void)hipEventDestroy(e);
  return err;
}

}  // namespace kda
