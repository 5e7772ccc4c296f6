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
// The only serial dependency is dS across chunks: with F = kg^T diag(b) T^T
// (128 x 64) and X = qg^T dO' - F M^T dO' (128 x 128), both chunk-local,
//   dS = Diag(gam) dSn - F (kp dSn) + X.
//
// Layout: the forward pass writes every chunk's start state (fp32) to slot
// n + floor(bos_n / 64) + c of sequence n's chunk c (slots are distinct across
// sequences); batch index b = slot * H + h addresses every per-chunk tile.
// Everything here is fp32: the chunk-local products run as batched tiled GEMMs
// (fp32 matrix cores), the serial recurrence in four workgroups per (sequence, head), one per
// 32 value columns.
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
// and holds C[16i + 4q4 + t][16j + m16] (t < 4) of each block.  Where an output
// is a sum of two products, both accumulate in the same registers (bgemm2_kernel).
typedef float bg_f32x4 __attribute__((ext_vector_type(4)));

// k-major tiles; a row stride of 16 mod 32 floats puts lane groups q4 and q4 + 1
// on disjoint banks for the operand reads.  NT is the tile's width (64 or 128).
template <int NT>
struct BgTiles {
  float A[16][80];
  float B[16][NT + 16];
};

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
      for (int e = 0; e < 4; ++e) sm.A[k + e][m] = (ks ? vv[e] * ks[k0 + k + e] : vv[e]) * sign;
    } else {
      const int k = tid >> 4, m = (tid & 15) * 4;
      const float4 v = *reinterpret_cast<const float4*>(A + (int64_t)(k0 + k) * lda + m0 + m);
      const float s = (ks ? ks[k0 + k] : 1.f) * sign;
      *reinterpret_cast<float4*>(&sm.A[k][m]) = make_float4(v.x * s, v.y * s, v.z * s, v.w * s);
    }
#pragma unroll
    for (int h = 0; h < NT / 64; ++h) {
      if (!TB) {
        const int k = tid >> 4, n = 64 * h + (tid & 15) * 4;
        *reinterpret_cast<float4*>(&sm.B[k][n]) =
            *reinterpret_cast<const float4*>(B + (int64_t)(k0 + k) * ldb + n0 + n);
      } else {
        const int n = 64 * h + (tid >> 2), k = (tid & 3) * 4;
        const float4 v = *reinterpret_cast<const float4*>(B + (int64_t)(n0 + n) * ldb + k0 + k);
        sm.B[k][n] = v.x; sm.B[k + 1][n] = v.y; sm.B[k + 2][n] = v.z; sm.B[k + 3][n] = v.w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int k = 4 * s4 + q4;
      const float a0 = sm.A[k][wm + m16], a1 = sm.A[k][wm + 16 + m16];
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const float bj = sm.B[k][wn + 16 * j + m16];
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

// Two 64 x 64 products that share their right operand, X1 B^T and X2 B^T, with B
// staged once (all three stored [64][K]).  `o1` carries X1, B and the first output
// (mask, alpha, row scale); `o1b`, if its C is set, stores the same accumulators a
// second time with its own mask, alpha and row scale; `o2` carries X2 in A and the
// second output.  Used for P = strict_lower(kg kh^T) with A = diag(beta) P and
// M = lower_incl(qg kh^T), and for dM = lower_incl(dO' U^T) with
// dA = strict_lower(-dY U^T).
__global__ void __launch_bounds__(256) bgemm_shared_b_kernel(GemmArgs o1, GemmArgs o1b, GemmArgs o2) {
  __shared__ float Bs[16][80];   // B^T slice, [k][n]
  __shared__ float X1s[16][80];  // X1^T slice, [k][m]
  __shared__ float X2s[16][80];  // X2^T slice, [k][m]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, m16 = lane & 15, q4 = lane >> 4;
  const int wm = 32 * (wave >> 1), wn = 32 * (wave & 1);
  const int64_t b = blockIdx.z;
  const float* x1 = o1.A + b * o1.sA;
  const float* bm = o1.B + b * o1.sB;
  const float* x2 = o2.A + b * o2.sA;
  bg_f32x4 acc1[2][2], acc2[2][2];
  bg_zero<64>(acc1);
  bg_zero<64>(acc2);
  for (int k0 = 0; k0 < o1.K; k0 += 16) {
    // rows tid / 4 of X1, X2 and B, four consecutive k each
    const int r = tid >> 2, k = (tid & 3) * 4;
    const float4 v1 = *reinterpret_cast<const float4*>(x1 + (int64_t)r * o1.lda + k0 + k);
    const float4 v2 = *reinterpret_cast<const float4*>(x2 + (int64_t)r * o2.lda + k0 + k);
    const float4 vb = *reinterpret_cast<const float4*>(bm + (int64_t)r * o1.ldb + k0 + k);
    X1s[k][r] = v1.x; X1s[k + 1][r] = v1.y; X1s[k + 2][r] = v1.z; X1s[k + 3][r] = v1.w;
    X2s[k][r] = v2.x; X2s[k + 1][r] = v2.y; X2s[k + 2][r] = v2.z; X2s[k + 3][r] = v2.w;
    Bs[k][r] = vb.x; Bs[k + 1][r] = vb.y; Bs[k + 2][r] = vb.z; Bs[k + 3][r] = vb.w;
    __syncthreads();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int kk = 4 * s4 + q4;
      const float b0 = Bs[kk][wn + m16], b1 = Bs[kk][wn + 16 + m16];
      const float a0 = X1s[kk][wm + m16], a1 = X1s[kk][wm + 16 + m16];
      const float c0 = X2s[kk][wm + m16], c1 = X2s[kk][wm + 16 + m16];
      acc1[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc1[0][0], 0, 0, 0);
      acc1[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc1[0][1], 0, 0, 0);
      acc1[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc1[1][0], 0, 0, 0);
      acc1[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc1[1][1], 0, 0, 0);
      acc2[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(c0, b0, acc2[0][0], 0, 0, 0);
      acc2[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(c0, b1, acc2[0][1], 0, 0, 0);
      acc2[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(c1, b0, acc2[1][0], 0, 0, 0);
      acc2[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(c1, b1, acc2[1][1], 0, 0, 0);
    }
    __syncthreads();
  }
  bg_store<64>(acc1, o1, b, 0, 0);
  if (o1b.C) bg_store<64>(acc1, o1b, b, 0, 0);
  bg_store<64>(acc2, o2, b, 0, 0);
}

// A sum of two products in one pass, C = rs (.) (op(A) op(B) + sign2 op(A2) op(B2)),
// so that the first product never goes through memory.
struct Gemm2Args {
  GemmArgs a;                              // first product, output, row scale, mask
  const float* A2; int64_t sA2; int lda2;
  const float* B2; int64_t sB2; int ldb2;
  int K2;
  const float* ks2; int64_t sks2;
  float sign2;                             // +-1
};

template <int NT, bool TA, bool TB, bool TA2, bool TB2>
__global__ void __launch_bounds__(256) bgemm2_kernel(Gemm2Args g) {
  __shared__ BgTiles<NT> sm;
  const GemmArgs& a = g.a;
  const int n0 = blockIdx.x * NT, m0 = blockIdx.y * 64;
  const int64_t b = blockIdx.z;
  bg_f32x4 acc[2][NT / 32];
  bg_zero<NT>(acc);
  bg_accumulate<NT, TA, TB>(acc, sm, a.A + b * a.sA, a.lda, a.B + b * a.sB, a.ldb, a.K,
                            a.ks ? a.ks + b * a.sks : nullptr, 1.f, m0, n0);
  bg_accumulate<NT, TA2, TB2>(acc, sm, g.A2 + b * g.sA2, g.lda2, g.B2 + b * g.sB2, g.ldb2, g.K2,
                              g.ks2 ? g.ks2 + b * g.sks2 : nullptr, g.sign2, m0, n0);
  bg_store<NT>(acc, a, b, m0, n0);
}

// ---------------------------------------------------------------- chunk prep
// One workgroup per batch (slot, head): loads the chunk's rows (zero past the
// sequence), forms G, the gated tiles, dO' = scale dO and the per-row beta.
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p, BwdTiles w) {
  const int64_t bidx = blockIdx.x;
  const int64_t slot = bidx / p.H;
  const int h = (int)(bidx % p.H);
  const int n = slot_seq(p, slot);
  const int64_t bos = seq_bos(p, n), len = seq_len_of(p, n);
  const int64_t c = slot - (n + bos / C);
  const int64_t rest = len - c * C;
  const int valid = (c < 0 || rest <= 0) ? 0 : rest < C ? (int)rest : C;
  const int t = threadIdx.x;
  const int HD = p.H * D;
  if (t < C) w.beta[bidx * C + t] = t < valid ? p.beta[(bos + c * C + t) * p.H + h] : 0.f;
  if (t == 0) w.valid[bidx] = valid;
  // thread t: channel t % 128, rows 32 (t / 128) .. +31
  const int ch = t & 127, half = t >> 7, r0 = 32 * half;
  // G: inclusive cumsum over the chunk (natural log): each thread sums its 32 rows in
  // registers, then the second half adds the first half's total
  __shared__ float tot[2][D];
  float gv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int r = r0 + i;
    gv[i] = r < valid ? p.g[((bos + c * C + r) * p.H + h) * D + ch] : 0.f;
  }
#pragma unroll
  for (int i = 1; i < 32; ++i) gv[i] += gv[i - 1];
  tot[half][ch] = gv[31];
  __syncthreads();
  const float off = half ? tot[0][ch] : 0.f;
  const float Glast = tot[0][ch] + tot[1][ch];
  const float gam = expf(Glast);
  if (half == 0) w.gam[bidx * D + ch] = gam;
  const int64_t tb = bidx * (C * D);
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const int r = r0 + i;
    const int64_t row = (bos + c * C + r) * (int64_t)HD + (int64_t)h * D + ch;
    const bool in = r < valid;
    const float qf = in ? bf2f_u16(p.q[row]) : 0.f;
    const float kf = in ? bf2f_u16(p.k[row]) : 0.f;
    const float vf = in ? bf2f_u16(p.v[row]) : 0.f;
    const float df = in ? p.scale * bf2f_u16(p.dout[row]) : 0.f;
    const float G = gv[i] + off;
    const float e = expf(G), ei = expf(-G);
    const int64_t o = tb + r * D + ch;
    w.G[o] = G;
    w.kg[o] = kf * e;
    w.qg[o] = qf * e;
    w.kh[o] = kf * ei;
    w.kp[o] = kf * ei * gam;
    w.vv[o] = vf;
    w.dO[o] = df;
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
// rows), so each (sequence, head) runs as D / DSW workgroups of DSW value
// columns.  Chunks last to first: dSn(c) is stored for the chunk's gradient
// products, then dS = Diag(gam) dSn - F (kp dSn) + X becomes the next dSn.  The
// sequence's initial-state gradient is the last dS.  The loop is serial and
// VALU-bound inside a workgroup of four waves, so with few (sequence, head)
// pairs the columns are cut finer (DSW 16) to occupy more compute units and
// halve each workgroup's work per chunk.
template <int DSW>
__global__ void __launch_bounds__(256) bwd_ds_scan_kernel(BwdParams p, BwdTiles w) {
  constexpr int DSC = D / DSW;       // workgroups per (sequence, head)
  constexpr int CG = DSW / 4;        // column groups of 4
  constexpr int RP = C * CG / 256;   // rows of P per thread
  constexpr int RF = D * CG / 256;   // rows of dS per thread
  static_assert(RP >= 1 && RF >= 1 && C * CG % 256 == 0, "slice width");
  __shared__ float ds[D][DSW + 4];   // dSn, then the new dS (this workgroup's columns)
  __shared__ float pp[C][DSW + 4];   // P = kp dSn
  const int pair = blockIdx.x / DSC, j0 = (blockIdx.x % DSC) * DSW;
  const int n = pair / p.H, h = pair % p.H;
  const int t = threadIdx.x;
  const int64_t bos = seq_bos(p, n), len = seq_len_of(p, n);
  const int nch = (int)((len + C - 1) / C);
  const size_t sd = (size_t)D * D;
  for (int x = t; x < D * DSW; x += 256) {   // dS_final (or zero)
    const int r = x / DSW, j = x % DSW;
    float v = 0.f;
    if (p.dsT) {
      const size_t o = ((size_t)n * p.H + h) * sd + (size_t)r * D + j0 + j;
      v = p.dsT_fp32 ? static_cast<const float*>(p.dsT)[o] : bf2f_u16(static_cast<const uint16_t*>(p.dsT)[o]);
    }
    ds[r][j] = v;
  }
  __syncthreads();
  const int jb = (t % CG) * 4;   // 4 of this workgroup's columns
  for (int c = nch - 1; c >= 0; --c) {
    const int64_t bidx = (n + bos / C + c) * p.H + h;
    float* dsn = w.dSn + bidx * sd;
    for (int x = t; x < D * DSW; x += 256) dsn[(size_t)(x / DSW) * D + j0 + x % DSW] = ds[x / DSW][x % DSW];
    {  // P = kp dSn: rows RP (t / CG) .. +RP-1
      const float* kp = w.kp + bidx * (C * D);
      const int r0 = (t / CG) * RP;
      float acc[RP][4] = {};
      for (int k = 0; k < D; k += 4) {
        float av[RP][4];
#pragma unroll
        for (int i = 0; i < RP; ++i) {
          const float4 a4 = *reinterpret_cast<const float4*>(&kp[(r0 + i) * D + k]);
          av[i][0] = a4.x; av[i][1] = a4.y; av[i][2] = a4.z; av[i][3] = a4.w;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float4 bv = *reinterpret_cast<const float4*>(&ds[k + kk][jb]);
#pragma unroll
          for (int i = 0; i < RP; ++i) {
            acc[i][0] = fmaf(av[i][kk], bv.x, acc[i][0]); acc[i][1] = fmaf(av[i][kk], bv.y, acc[i][1]);
            acc[i][2] = fmaf(av[i][kk], bv.z, acc[i][2]); acc[i][3] = fmaf(av[i][kk], bv.w, acc[i][3]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < RP; ++i)
        *reinterpret_cast<float4*>(&pp[r0 + i][jb]) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
    __syncthreads();
    {  // dS = gam (.) dSn - F P + X: rows RF (t / CG) .. +RF-1
      const float* F = w.F + bidx * (D * C);
      const float* X = w.X + bidx * sd;
      const float* gam = w.gam + bidx * D;
      const int c0 = (t / CG) * RF;
      float acc[RF][4];
#pragma unroll
      for (int i = 0; i < RF; ++i) {
        const float g = gam[c0 + i];
        const float4 xv = *reinterpret_cast<const float4*>(&X[(size_t)(c0 + i) * D + j0 + jb]);
        acc[i][0] = g * ds[c0 + i][jb] + xv.x;
        acc[i][1] = g * ds[c0 + i][jb + 1] + xv.y;
        acc[i][2] = g * ds[c0 + i][jb + 2] + xv.z;
        acc[i][3] = g * ds[c0 + i][jb + 3] + xv.w;
      }
      for (int r = 0; r < C; r += 4) {
        float fv[RF][4];
#pragma unroll
        for (int i = 0; i < RF; ++i) {
          const float4 f4 = *reinterpret_cast<const float4*>(&F[(c0 + i) * C + r]);
          fv[i][0] = f4.x; fv[i][1] = f4.y; fv[i][2] = f4.z; fv[i][3] = f4.w;
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float4 bv = *reinterpret_cast<const float4*>(&pp[r + rr][jb]);
#pragma unroll
          for (int i = 0; i < RF; ++i) {
            acc[i][0] = fmaf(-fv[i][rr], bv.x, acc[i][0]); acc[i][1] = fmaf(-fv[i][rr], bv.y, acc[i][1]);
            acc[i][2] = fmaf(-fv[i][rr], bv.z, acc[i][2]); acc[i][3] = fmaf(-fv[i][rr], bv.w, acc[i][3]);
          }
        }
      }
      __syncthreads();  // every read of dSn and P is done
#pragma unroll
      for (int i = 0; i < RF; ++i)
        *reinterpret_cast<float4*>(&ds[c0 + i][jb]) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
    __syncthreads();
  }
  if (p.ds0) {
    float* o = p.ds0 + ((size_t)n * p.H + h) * sd;
    for (int x = t; x < D * DSW; x += 256) o[(size_t)(x / DSW) * D + j0 + x % DSW] = ds[x / DSW][x % DSW];
  }
}

// The scan's launch: 32-column slices once four per (sequence, head) fill the
// 256 compute units, 16-column slices below that.
void launch_ds_scan(const BwdParams& p, const BwdTiles& w, hipStream_t s) {
  const int64_t pairs = (int64_t)p.nseq * p.H;
  if (pairs * (D / 32) >= 256)
    hipLaunchKernelGGL(bwd_ds_scan_kernel<32>, dim3((unsigned)(pairs * (D / 32))), dim3(256), 0, s, p, w);
  else
    hipLaunchKernelGGL(bwd_ds_scan_kernel<16>, dim3((unsigned)(pairs * (D / 16))), dim3(256), 0, s, p, w);
}

// ---------------------------------------------------------------- gates and scatter
// One workgroup per batch: dq, dk, dv, dg, dbeta of the chunk's rows.
__global__ void __launch_bounds__(256) bwd_finalize_kernel(BwdParams p, BwdTiles w) {
  const int64_t bidx = blockIdx.x;
  const int valid = w.valid[bidx];
  if (valid == 0) return;
  const int64_t slot = bidx / p.H;
  const int h = (int)(bidx % p.H);
  const int n = slot_seq(p, slot);
  const int64_t bos = seq_bos(p, n);
  const int64_t c = slot - (n + bos / C);
  const int t = threadIdx.x, ch = t & 127, half = t >> 7;
  const int HD = p.H * D;
  const int64_t tb = bidx * (C * D);
  const float* beta = w.beta + bidx * C;
  __shared__ float dGs[C][D];
  __shared__ float red[2][D];
  __shared__ float rowsum[D];
  __shared__ float dbs[C];
  // per row: dG, dq, dk, dv; per channel: dG_last pieces
  float glast = 0.f;
  for (int r = half; r < C; r += 2) {
    const int64_t o = tb + r * D + ch;
    const float G = w.G[o];
    const float e = expf(G), ei = expf(-G);
    const float gam = w.gam[bidx * D + ch];
    const float dqg = w.dqg[o], dkg = w.dkg[o], dkh = w.dkh[o], dkp = w.dkp[o];
    // k and q straight from the inputs (exact in fp32; zero past the sequence's end)
    const int64_t row = (bos + c * C + r) * (int64_t)HD + (int64_t)h * D + ch;
    const float kf = r < valid ? bf2f_u16(p.k[row]) : 0.f;
    const float qf = r < valid ? bf2f_u16(p.q[row]) : 0.f;
    const float kp = kf * ei * gam;
    dGs[r][ch] = dqg * qf * e + dkg * kf * e - dkh * kf * ei - dkp * kp;
    glast += dkp * kp;
    if (r < valid) {
      p.dq[row] = dqg * e;
      p.dk[row] = dkg * e + dkh * ei + dkp * gam * ei;
      p.dv[row] = beta[r] * w.dY[o];
    }
  }
  red[half][ch] = glast;
  // dgam_direct: gam_c times the row sum over j of S * dSn for every channel c.  Sixteen
  // lanes share a row, each with eight consecutive entries (coalesced), and their sums
  // meet through lane exchanges within the sixteen.
  {
    const float* S = w.S + bidx * (size_t)(D * D);
    const float* dsn = w.dSn + bidx * (size_t)(D * D);
    const int jq = t & 15;
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
      if (jq == 0) rowsum[r] = sum;
    }
    __syncthreads();
    red[half][ch] += half == 0 ? rowsum[ch] * w.gam[bidx * D + ch] : 0.f;
  }
  __syncthreads();
  if (half == 0) {
    const float dGlast = red[0][ch] + red[1][ch];
    // dg_t = sum_{r >= t} dG_r + dG_last
    float run = dGlast;
    for (int r = C - 1; r >= 0; --r) {
      run += dGs[r][ch];
      if (r < valid) p.dg[((bos + c * C + r) * (int64_t)p.H + h) * D + ch] = run;
    }
  }
  // dbeta_r = sum_j dY_rj R_rj + sum_i dA_ri P_ri: sixteen lanes per row, as above
  {
    const int jq = t & 15;
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
      if (jq == 0) dbs[r] = sum;
    }
  }
  __syncthreads();
  if (t < valid) p.dbeta[(bos + c * C + t) * p.H + h] = dbs[t];
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

// C = op(A) op(B) + sign2 op(A2) op(B2) with `first`'s output, row scale and mask;
// `second` supplies A2, B2, K2 and the column scale of op(A2).
template <bool TA, bool TB, bool TA2, bool TB2>
void gemm2(const GemmArgs& first, const GemmArgs& second, float sign2, hipStream_t s) {
  Gemm2Args g{};
  g.a = first;
  g.A2 = second.A; g.sA2 = second.sA; g.lda2 = second.lda;
  g.B2 = second.B; g.sB2 = second.sB; g.ldb2 = second.ldb;
  g.K2 = second.K; g.ks2 = second.ks; g.sks2 = second.sks;
  g.sign2 = sign2;
  if (first.N % 128 == 0)
    hipLaunchKernelGGL((bgemm2_kernel<128, TA, TB, TA2, TB2>), dim3(first.N / 128, first.M / 64, first.batches),
                       dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((bgemm2_kernel<64, TA, TB, TA2, TB2>), dim3(first.N / 64, first.M / 64, first.batches),
                       dim3(256), 0, s, g);
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

size_t bwd_tile_floats() { return BwdTiles::floats_per_batch(); }

hipError_t launch_bwd_scan_only(const BwdParams& p, hipStream_t s) {
  const BwdTiles w{};
  launch_ds_scan(p, w, s);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, const BwdTiles& w, int64_t batches, hipStream_t s) {
  const int NB = (int)batches;
  const int64_t t1 = C * D, t2 = C * C, t3 = D * D, tf = D * C;
  // chunk tiles
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(NB), dim3(256), 0, s, p, w);
  // A = strict_lower(diag(b) kg kh^T), P = strict_lower(kg kh^T), M = lower_incl(qg kh^T)
  {
    GemmArgs p1 = mm(C, C, D, w.kg, t1, D, w.kh, t1, D, w.P, t2, C, NB);
    p1.mask = 1;
    GemmArgs a1 = p1;
    a1.C = w.A; a1.rs = w.beta; a1.srs = C;
    GemmArgs m2 = mm(C, C, D, w.qg, t1, D, w.kh, t1, D, w.M, t2, C, NB);
    m2.mask = 2;
    hipLaunchKernelGGL(bgemm_shared_b_kernel, dim3(1, 1, NB), dim3(256), 0, s, p1, a1, m2);
  }
  hipLaunchKernelGGL(bwd_inverse_kernel, dim3(NB), dim3(64), 0, s, w.A, w.T);
  // R = V - kg S;  U = T diag(b) R
  {
    GemmArgs a = mm(C, D, D, w.kg, t1, D, w.S, t3, D, w.R, t1, D, NB);
    a.alpha = -1.f; a.Dm = w.vv; a.sD = t1; a.ldd = D;
    gemm(false, false, a, s);
    GemmArgs u = mm(C, D, C, w.T, t2, C, w.R, t1, D, w.U, t1, D, NB);
    u.ks = w.beta; u.sks = C;
    gemm(false, false, u, s);
  }
  // MtdO = M^T dO';  F = kg^T diag(b) T^T;  X = qg^T dO' - F MtdO
  {
    gemm(true, false, mm(C, D, C, w.M, t2, C, w.dO, t1, D, w.MtdO, t1, D, NB), s);
    GemmArgs f = mm(D, C, C, w.kg, t1, D, w.T, t2, C, w.F, tf, C, NB);
    f.ks = w.beta; f.sks = C;
    gemm(true, true, f, s);
    gemm2<true, false, false, false>(mm(D, D, C, w.qg, t1, D, w.dO, t1, D, w.X, t3, D, NB),
                                     mm(D, D, C, w.F, tf, C, w.MtdO, t1, D, nullptr, 0, 0, NB), -1.f, s);
  }
  // serial recurrence of dS over chunks
  launch_ds_scan(p, w, s);
  // chunk gradients
  {
    GemmArgs du = mm(C, D, D, w.kp, t1, D, w.dSn, t3, D, w.dU, t1, D, NB);  // dU = kp dSn + MtdO
    du.Dm = w.MtdO; du.sD = t1; du.ldd = D;
    gemm(false, false, du, s);
    gemm(true, false, mm(C, D, C, w.T, t2, C, w.dU, t1, D, w.dY, t1, D, NB), s);  // dY = T^T dU
    {
      GemmArgs dm = mm(C, C, D, w.dO, t1, D, w.U, t1, D, w.dM, t2, C, NB);  // dM = lower_incl(dO' U^T)
      dm.mask = 2;
      GemmArgs da = mm(C, C, D, w.dY, t1, D, w.U, t1, D, w.dA, t2, C, NB);  // dA = strict_lower(-dY U^T)
      da.alpha = -1.f; da.mask = 1;
      GemmArgs none{};
      hipLaunchKernelGGL(bgemm_shared_b_kernel, dim3(1, 1, NB), dim3(256), 0, s, dm, none, da);
    }
    gemm2<false, true, false, false>(mm(C, D, D, w.dO, t1, D, w.S, t3, D, w.dqg, t1, D, NB),  // dO' S^T
                                     mm(C, D, C, w.dM, t2, C, w.kh, t1, D, nullptr, 0, 0, NB),  // + dM kh
                                     1.f, s);
    gemm(false, true, mm(C, D, D, w.U, t1, D, w.dSn, t3, D, w.dkp, t1, D, NB), s);  // dkp = U dSn^T
    GemmArgs k1 = mm(C, D, C, w.dA, t2, C, w.kh, t1, D, w.dkg, t1, D, NB);  // diag(b)(dA kh - dY S^T)
    k1.rs = w.beta; k1.srs = C;
    gemm2<false, false, false, true>(k1, mm(C, D, D, w.dY, t1, D, w.S, t3, D, nullptr, 0, 0, NB), -1.f, s);
    GemmArgs h2 = mm(C, D, C, w.dA, t2, C, w.kg, t1, D, nullptr, 0, 0, NB);  // + dA^T diag(b) kg
    h2.ks = w.beta; h2.sks = C;
    gemm2<true, false, true, false>(mm(C, D, C, w.dM, t2, C, w.qg, t1, D, w.dkh, t1, D, NB), h2,  // dM^T qg
                                    1.f, s);
  }
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3(NB), dim3(256), 0, s, p, w);
  return hipGetLastError();
}

}  // namespace kda
