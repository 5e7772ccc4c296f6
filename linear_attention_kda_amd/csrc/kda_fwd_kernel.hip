// Fused chunkwise Kimi Delta Attention forward kernel for gfx950 (MI355X).
//
// Recurrence (per sequence and head) [core.today "Kimi Linear 특집", ch.4 혁신 2,
// state-update equation; ch.4 혁신 1, channel-wise gate; ch.2, readout]:
//   S_t = (Diag(a_t) - b_t k_t (k_t * a_t)^T) S_{t-1} + b_t k_t v_t^T,  a_t = exp(g_t)
//   o_t = scale * S_t^T q_t
// evaluated 64 tokens at a time with the WY/UT form of the diagonal-plus-low-rank
// transition [same page, ch.4 혁신 2, chunkwise remark].  For one chunk with start
// state S (128 x 128, S[c][j]: c key channel, j value channel), local rows r, i,
// G = within-chunk inclusive cumsum of g, Gamma = exp(G):
//   A[r][i] = b_r sum_c k_rc k_ic exp(G_rc - G_ic)   (i < r)      (L = I + A)
//   Y       = V - (K*Gamma) S
//   U       = L^-1 diag(b) Y          (= b_r times the delta-rule error of row r)
//   M[r][i] = sum_c q_rc k_ic exp(G_rc - G_ic)        (i <= r)
//   O       = scale * ((Q*Gamma) S + M U)
//   S'      = Diag(Gamma_last) S + (K * exp(G_last - G))^T U
//
// Mapping: one workgroup of 4 waves owns one (sequence, head, value-column slice)
// and walks its chunks in order.  The fp32 state slice lives in MFMA accumulator
// registers for the whole sequence (never in LDS or HBM); each wave owns 16*JT
// value columns.  The value-independent per-chunk work (gating, A, M, the
// diagonal-block inverses) is recomputed by every value slice of a head.
// Per chunk:  gating (VALU, exp2) -> LDS operand tiles -> A and M tiles (bf16
// MFMA 16x16x32) and the four 16x16 diagonal-block inverses (fp32 VALU forward
// substitution) -> per-wave state pass: Y (MFMA), block forward substitution
// for U (MFMA 16x16x16), O (MFMA, written straight to HBM), S update (MFMA).
// The next chunk's q/k/v/g/beta loads are issued right after the gating step and
// stay in flight during the MFMA work.
//
// Exponent ranges: every exp factor that multiplies an MFMA operand is <= 1,
// except exp(G_r - G_{end of r's 16-row block}) on the diagonal blocks of A and
// M, which is bounded by the decay inside one 16-token block (this is why the
// per-channel sum of -g over such a block must stay below ~88 in natural log).
//
// MFMA operand layouts used below (64 lanes, q = lane/16, m = lane%16):
//  16x16x32 bf16:  A[m][8q+e], B[8q+e][m] (e < 8),  D[4q+t][m] (t < 4)
//  16x16x16 bf16:  A[m][4q+e], B[4q+e][m] (e < 4),  D[4q+t][m]
// A contraction may permute its k index as long as both operands agree; the
// state path uses k-slot e <-> k = 32ks + 4q + e (e < 4), 32ks + 16 + 4q + e-4
// (e >= 4), which is exactly what two D-layout tiles (rows 32ks..+15 and
// 32ks+16..+31) hold per lane, so accumulators feed the next product directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // head dimension
constexpr int NT = 256;      // threads per workgroup (4 waves)
constexpr int TS = D + 8;    // row stride (bf16) of token-major [64][128] tiles: 272 B
constexpr int CS = C + 4;    // row stride (bf16) of channel-major [.][64] tiles: 136 B
constexpr int QS = C + 4;    // row stride (bf16) of [64][64] tiles: 136 B
constexpr int LS = 16 + 4;   // row stride (bf16) of the diagonal-block inverses
constexpr int NS = 16 + 4;   // row stride (fp32) of the diagonal blocks of A
constexpr float LOG2E = 1.4426950408889634f;

// Shared-memory plan (bytes); one workgroup per CU.
template <int NV>
struct alignas(16) Smem {
  __bf16 kr[C * TS];    // K * exp(G - X_b)            row operand of A      (<= 1)
  __bf16 qr[C * TS];    // Q * exp(G - X_b)            row operand of M      (<= 1)
  __bf16 kh[C * TS];    // K * exp(X_{b+1} - G)        column operand of A, M (<= 1)
  __bf16 kg[C * TS];    // K * Gamma                   for Y = V - (K*Gamma) S
  __bf16 qg[C * TS];    // Q * Gamma                   for O = (Q*Gamma) S + ...
  __bf16 kpt[D * CS];   // (K * exp(G_last - G))^T     channel-major, state update
  __bf16 vt[NV * CS];   // V^T (this slice's columns)  channel-major
  __bf16 mm[C * QS];    // M (lower incl. diagonal), zero elsewhere
  __bf16 an[C * QS];    // -A on the off-diagonal 16x16 blocks
  __bf16 li[C * LS];    // inverses of the 4 diagonal blocks of L = I + A
  float nd[4 * 16 * NS];  // diagonal 16x16 blocks of A (fp32)
  float gamc[D];        // exp(G_last) per channel
  float beta[C];
  float seg[8 * D];     // per 8-row group, per channel: sum of g*log2(e)
  float pf[10 * D];     // exp(X_rb - X_{ib+1}) per (rb, ib <= rb) pair and channel
  int order;            // sequence chosen for this workgroup
};

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(pack2(a, b), pack2(c, d));
}

__device__ __forceinline__ void unpack4(uint2 u, float* f) {
  bf16x2 lo = __builtin_bit_cast(bf16x2, u.x);
  bf16x2 hi = __builtin_bit_cast(bf16x2, u.y);
  f[0] = bf2f(lo[0]);
  f[1] = bf2f(lo[1]);
  f[2] = bf2f(hi[0]);
  f[3] = bf2f(hi[1]);
}

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Two 4-element bf16 runs (8-byte aligned) -> one 16x16x32 operand.
__device__ __forceinline__ bf16x8 ld2x4(const __bf16* p0, const __bf16* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0);
  uint2 b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x4 ld4(const __bf16* p) {
  return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}

__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
  return __builtin_bit_cast(bf16x4, pack4(v[0], v[1], v[2], v[3]));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// (rb, ib) enumeration of the 10 lower-triangular 16x16 block pairs.
__device__ __forceinline__ int pair_rb(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ int pair_ib(int p) { return p - (pair_rb(p) * (pair_rb(p) + 1)) / 2; }

// Raw inputs of one chunk held by one thread: rows 8*rg..8*rg+7, channels 4*cg..4*cg+3.
template <int NV>
struct ChunkRegs {
  float4 g[8];
  uint2 q[8];
  uint2 k[8];
  uint32_t v[8][NV / 64];  // NV/32 bf16 values per row
  float beta;
};

template <int NV>
__device__ __forceinline__ void load_chunk(ChunkRegs<NV>& R, const Params& p, int64_t tok0,
                                           int valid, int h, int j0, int tid) {
  const int rg = tid >> 5, cg = tid & 31;
  const int64_t HD = (int64_t)p.H * D;
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) {
    const int row = rg * 8 + r8;
    if (row < valid) {
      const int64_t base = (tok0 + row) * HD + (int64_t)h * D;
      R.g[r8] = *reinterpret_cast<const float4*>(p.g + base + 4 * cg);
      R.q[r8] = *reinterpret_cast<const uint2*>(p.q + base + 4 * cg);
      R.k[r8] = *reinterpret_cast<const uint2*>(p.k + base + 4 * cg);
      if constexpr (NV == 128) {
        uint2 t = *reinterpret_cast<const uint2*>(p.v + base + j0 + 4 * cg);
        R.v[r8][0] = t.x;
        R.v[r8][1] = t.y;
      } else {
        R.v[r8][0] = *reinterpret_cast<const uint32_t*>(p.v + base + j0 + 2 * cg);
      }
    } else {
      R.g[r8] = make_float4(0.f, 0.f, 0.f, 0.f);
      R.q[r8] = make_uint2(0u, 0u);
      R.k[r8] = make_uint2(0u, 0u);
#pragma unroll
      for (int x = 0; x < NV / 64; ++x) R.v[r8][x] = 0u;
    }
  }
  R.beta = 0.f;
  if (tid < C && tid < valid) R.beta = p.beta[(tok0 + tid) * p.H + h];
}

template <int JT>
__global__ void __launch_bounds__(NT, 1) kda_fwd_kernel(Params p) {
  constexpr int NV = 64 * JT;  // value columns per workgroup
  __shared__ Smem<NV> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, m16 = lane & 15;

  // ---- workgroup -> (sequence rank, head, value slice); slices of one head share an XCD
  const int nsplit = 128 / NV;
  const int pairs = p.nseq * p.H;
  const int grp = blockIdx.x / (8 * nsplit);
  const int rem = blockIdx.x % (8 * nsplit);
  const int split = rem / 8;
  const int pidx = grp * 8 + (rem % 8);
  if (pidx >= pairs) return;
  const int rank = pidx / p.H;
  const int h = pidx % p.H;
  const int j0 = split * NV;

  // ---- longest sequence first: rank -> sequence index (ties by index)
  int n = rank;
  if (p.cu != nullptr && p.nseq > 1 && p.nseq <= kSortLimit) {
    int* lens = reinterpret_cast<int*>(sm.kr);  // scratch before the first chunk
    for (int i = tid; i < p.nseq; i += NT) lens[i] = p.cu[i + 1] - p.cu[i];
    __syncthreads();
    for (int i = tid; i < p.nseq; i += NT) {
      const int li = lens[i];
      int rk = 0;
      for (int j = 0; j < p.nseq; ++j) {
        const int lj = lens[j];
        rk += (lj > li) || (lj == li && j < i);
      }
      if (rk == rank) sm.order = i;
    }
    __syncthreads();
    n = sm.order;
  }
  const int64_t bos = p.cu ? (int64_t)p.cu[n] : (int64_t)n * p.T;
  const int64_t len = p.cu ? (int64_t)p.cu[n + 1] - bos : p.T;

  // ---- constant LDS: M tiles above the block diagonal that the 32-wide k-steps touch
  for (int x = tid; x < 16 * 16; x += NT) {
    const int r = x >> 4, i = x & 15;
    sm.mm[r * QS + 16 + i] = (__bf16)0.f;          // block (0, 1)
    sm.mm[(32 + r) * QS + 48 + i] = (__bf16)0.f;   // block (2, 3)
  }

  // ---- state slice: wave owns value columns jw = j0 + 16*JT*wave + 16*jt + m16;
  // Sacc[ct][jt][t] = S[16ct + 4q4 + t][jw]
  f32x4 Sacc[8][JT];
  const int jw_base = j0 + 16 * JT * wave;
  const size_t sbase = ((size_t)n * p.H + h) * (size_t)(D * D);
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const size_t off = sbase + (size_t)(16 * ct + 4 * q4 + t) * D + jw_base + 16 * jt + m16;
        float s = 0.f;
        if (p.s0 != nullptr)
          s = p.s0_fp32 ? reinterpret_cast<const float*>(p.s0)[off]
                        : bf2f(reinterpret_cast<const __bf16*>(p.s0)[off]);
        Sacc[ct][jt][t] = s;
      }
  bf16x8 Sfrag[4][JT];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) Sfrag[ks][jt] = cat(cvt4(Sacc[2 * ks][jt]), cvt4(Sacc[2 * ks + 1][jt]));

  const int nchunks = (int)((len + C - 1) / C);
  const int rg = tid >> 5, cg = tid & 31;
  const int blk = rg >> 1;  // 16-row block of this thread's rows

  ChunkRegs<NV> R;
  if (nchunks > 0) load_chunk<NV>(R, p, bos, (int)(len < C ? len : C), h, j0, tid);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int64_t tok0 = bos + (int64_t)ch * C;
    const int valid = (int)((len - (int64_t)ch * C) < C ? (len - (int64_t)ch * C) : C);

    // ================= gating, part 1: chunk-local cumulative log2-decay
    float lg[8][4];
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      lg[r8][0] = R.g[r8].x * LOG2E;
      lg[r8][1] = R.g[r8].y * LOG2E;
      lg[r8][2] = R.g[r8].z * LOG2E;
      lg[r8][3] = R.g[r8].w * LOG2E;
      if (r8 > 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) lg[r8][e] += lg[r8 - 1][e];
    }
    *reinterpret_cast<float4*>(&sm.seg[rg * D + 4 * cg]) =
        make_float4(lg[7][0], lg[7][1], lg[7][2], lg[7][3]);
    __syncthreads();  // (1) also: every wave has finished the previous chunk's state pass

    // ================= gating, part 2: reference points and operand tiles
    float X[5][4];   // X[b] = G (log2) at the last row of block b-1; X[0] = 0; X[4] = G_last
    float off[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) X[0][e] = 0.f;
    {
      float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float4 s = *reinterpret_cast<const float4*>(&sm.seg[r * D + 4 * cg]);
        if (r == rg) {
          off[0] = run[0]; off[1] = run[1]; off[2] = run[2]; off[3] = run[3];
        }
        run[0] += s.x; run[1] += s.y; run[2] += s.z; run[3] += s.w;
        if (r & 1)
#pragma unroll
          for (int e = 0; e < 4; ++e) X[(r + 1) >> 1][e] = run[e];
      }
    }
    float Xb[4], Xb1[4], eXb[4], eCX[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // runtime block index -> select (keeps X in registers)
      Xb[e] = blk == 0 ? X[0][e] : blk == 1 ? X[1][e] : blk == 2 ? X[2][e] : X[3][e];
      Xb1[e] = blk == 0 ? X[1][e] : blk == 1 ? X[2][e] : blk == 2 ? X[3][e] : X[4][e];
      eXb[e] = exp2f(Xb[e]);
      eCX[e] = exp2f(X[4][e] - Xb1[e]);
    }
    float kpv[8][4];  // K * exp(G_last - G), kept for the channel-major writes
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int row = rg * 8 + r8;
      float qf[4], kf[4];
      unpack4(R.q[r8], qf);
      unpack4(R.k[r8], kf);
      float kr[4], qr[4], kh[4], kg[4], qg[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float G = off[e] + lg[r8][e];
        const float F = exp2f(G - Xb[e]);   // <= 1
        const float Hh = exp2f(Xb1[e] - G); // <= 1
        kr[e] = kf[e] * F;
        qr[e] = qf[e] * F;
        kh[e] = kf[e] * Hh;
        kg[e] = kr[e] * eXb[e];
        qg[e] = qr[e] * eXb[e];
        kpv[r8][e] = kh[e] * eCX[e];
      }
      const int o = row * TS + 4 * cg;
      *reinterpret_cast<uint2*>(&sm.kr[o]) = pack4(kr[0], kr[1], kr[2], kr[3]);
      *reinterpret_cast<uint2*>(&sm.qr[o]) = pack4(qr[0], qr[1], qr[2], qr[3]);
      *reinterpret_cast<uint2*>(&sm.kh[o]) = pack4(kh[0], kh[1], kh[2], kh[3]);
      *reinterpret_cast<uint2*>(&sm.kg[o]) = pack4(kg[0], kg[1], kg[2], kg[3]);
      *reinterpret_cast<uint2*>(&sm.qg[o]) = pack4(qg[0], qg[1], qg[2], qg[3]);
    }
    // channel-major K' and V^T: per channel, 8 consecutive rows as two 4-row runs
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = (4 * cg + e) * CS + rg * 8;
      *reinterpret_cast<uint2*>(&sm.kpt[o]) = pack4(kpv[0][e], kpv[1][e], kpv[2][e], kpv[3][e]);
      *reinterpret_cast<uint2*>(&sm.kpt[o + 4]) = pack4(kpv[4][e], kpv[5][e], kpv[6][e], kpv[7][e]);
    }
    {
      constexpr int VPT = NV / 32;  // value columns per thread
#pragma unroll
      for (int e = 0; e < VPT; ++e) {
        float vv[8];
#pragma unroll
        for (int r8 = 0; r8 < 8; ++r8) {
          const bf16x2 two = __builtin_bit_cast(bf16x2, R.v[r8][e >> 1]);
          vv[r8] = bf2f(two[e & 1]);
        }
        const int o = (VPT * cg + e) * CS + rg * 8;
        *reinterpret_cast<uint2*>(&sm.vt[o]) = pack4(vv[0], vv[1], vv[2], vv[3]);
        *reinterpret_cast<uint2*>(&sm.vt[o + 4]) = pack4(vv[4], vv[5], vv[6], vv[7]);
      }
    }
    // pair factors exp(X_rb - X_{ib+1}); this thread's row group covers pairs rg, rg+8
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int pr = rg + 8 * pp;
      if (pr < 10) {
        const int rb = pair_rb(pr), ib = pair_ib(pr);
        float4 f;
        float* fp = reinterpret_cast<float*>(&f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xr = rb == 0 ? X[0][e] : rb == 1 ? X[1][e] : rb == 2 ? X[2][e] : X[3][e];
          const float xi = ib == 0 ? X[1][e] : ib == 1 ? X[2][e] : ib == 2 ? X[3][e] : X[4][e];
          fp[e] = exp2f(xr - xi);
        }
        *reinterpret_cast<float4*>(&sm.pf[pr * D + 4 * cg]) = f;
      }
    }
    if (rg == 0)
      *reinterpret_cast<float4*>(&sm.gamc[4 * cg]) =
          make_float4(exp2f(X[4][0]), exp2f(X[4][1]), exp2f(X[4][2]), exp2f(X[4][3]));
    if (tid < C) sm.beta[tid] = R.beta;

    // prefetch the next chunk's raw inputs (in flight during the MFMA work below)
    if (ch + 1 < nchunks) {
      const int64_t rest = len - (int64_t)(ch + 1) * C;
      load_chunk<NV>(R, p, tok0 + C, (int)(rest < C ? rest : C), h, j0, tid);
    }
    __syncthreads();  // (2) operand tiles ready

    // ================= A (waves 0,1) and M (waves 2,3) 16x16 tiles
    {
      const bool isM = wave >= 2;
      const __bf16* rowsrc = isM ? sm.qr : sm.kr;
      const int p0 = (wave & 1) ? 5 : 0;
      for (int pr = p0; pr < p0 + 5; ++pr) {
        const int rb = pair_rb(pr), ib = pair_ib(pr);
        const bool scaled = ib != rb - 1;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int c0 = 32 * ks + 8 * q4;
          bf16x8 rf = ld8(&rowsrc[(16 * rb + m16) * TS + c0]);
          if (scaled) {
            const float4 f0 = *reinterpret_cast<const float4*>(&sm.pf[pr * D + c0]);
            const float4 f1 = *reinterpret_cast<const float4*>(&sm.pf[pr * D + c0 + 4]);
            const float fs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) rf[e] = (__bf16)(bf2f(rf[e]) * fs[e]);
          }
          const bf16x8 cf = ld8(&sm.kh[(16 * ib + m16) * TS + c0]);
          acc = mfma32(cf, rf, acc);  // D[i][r]: lane holds (r = m16, i = 4q4 + t)
        }
        const int r = 16 * rb + m16;
        float v4[4];
        if (!isM) {
          const float br = sm.beta[r];
#pragma unroll
          for (int t = 0; t < 4; ++t) v4[t] = (16 * ib + 4 * q4 + t < r) ? br * acc[t] : 0.f;
          if (ib == rb) {
            *reinterpret_cast<float4*>(&sm.nd[(rb * 16 + m16) * NS + 4 * q4]) =
                make_float4(v4[0], v4[1], v4[2], v4[3]);
          } else {
            *reinterpret_cast<uint2*>(&sm.an[r * QS + 16 * ib + 4 * q4]) =
                pack4(-v4[0], -v4[1], -v4[2], -v4[3]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) v4[t] = (16 * ib + 4 * q4 + t <= r) ? acc[t] : 0.f;
          *reinterpret_cast<uint2*>(&sm.mm[r * QS + 16 * ib + 4 * q4]) = pack4(v4[0], v4[1], v4[2], v4[3]);
        }
      }
      if (!isM) {
        // inverse of the unit lower-triangular diagonal blocks this wave just wrote:
        // lanes 0-15 -> block 2*wave, lanes 16-31 -> block 2*wave+1 (lanes 32-63 mirror)
        lds_fence();
        const int b = 2 * wave + ((lane >> 4) & 1);
        const int j = m16;
        const float* N = &sm.nd[b * 16 * NS];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = (r == j) ? 1.f : 0.f;
#pragma unroll
          for (int kk = 0; kk < r; ++kk) s -= N[r * NS + kk] * x[kk];
          x[r] = s;
        }
        if (lane < 32) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sm.li[(16 * b + r) * LS + j] = (__bf16)x[r];
        }
      }
    }
    __syncthreads();  // (3) M, -A, L_bb^-1 ready

    // ================= state pass for this wave's value columns
    // Y = V - (K*Gamma) S  ->  Z = beta * Y   (D-layout: rows 16it + 4q4 + t, column m16)
    f32x4 Z[4][JT];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) Z[it][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const __bf16* rowp = &sm.kg[(16 * it + m16) * TS + 32 * ks + 4 * q4];
        const bf16x8 a = ld2x4(rowp, rowp + 16);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Z[it][jt] = mfma32(a, Sfrag[ks][jt], Z[it][jt]);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float4 bb = *reinterpret_cast<const float4*>(&sm.beta[16 * it + 4 * q4]);
      const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const int jl = 16 * JT * wave + 16 * jt + m16;  // column within this slice
        float vv[4];
        unpack4(*reinterpret_cast<const uint2*>(&sm.vt[jl * CS + 16 * it + 4 * q4]), vv);
#pragma unroll
        for (int t = 0; t < 4; ++t) Z[it][jt][t] = bv[t] * (vv[t] - Z[it][jt][t]);
      }
    }
    // U = L^-1 Z by block forward substitution: U_b = Linv_b (Z_b - sum_{b'<b} A_bb' U_b')
    bf16x4 U[4][JT];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bf16x4 linv = ld4(&sm.li[(16 * b + m16) * LS + 4 * q4]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        f32x4 z = Z[b][jt];
#pragma unroll
        for (int bp = 0; bp < b; ++bp) {
          const bf16x4 an = ld4(&sm.an[(16 * b + m16) * QS + 16 * bp + 4 * q4]);
          z = mfma16(an, U[bp][jt], z);
        }
        // z = hi + lo in bf16 (the rounding of z would otherwise reach U in full)
        const bf16x4 zh = cvt4(z);
        f32x4 zl;
#pragma unroll
        for (int t = 0; t < 4; ++t) zl[t] = z[t] - bf2f(zh[t]);
        f32x4 u = mfma16(linv, zh, f32x4{0.f, 0.f, 0.f, 0.f});
        u = mfma16(linv, cvt4(zl), u);
        U[b][jt] = cvt4(u);
      }
    }
    // O^T = S^T (Q*Gamma)^T + U^T M^T  ->  lane holds O[r = 16rt + m16][j = 16jt + 4q4 + t]
    {
      const int64_t HD = (int64_t)p.H * D;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + m16;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const __bf16* rowp = &sm.qg[r * TS + 32 * ks + 4 * q4];
            o = mfma32(Sfrag[ks][jt], ld2x4(rowp, rowp + 16), o);
          }
#pragma unroll
          for (int ks = 0; ks <= (rt >> 1); ++ks) {
            const __bf16* rowp = &sm.mm[r * QS + 32 * ks + 4 * q4];
            o = mfma32(cat(U[2 * ks][jt], U[2 * ks + 1][jt]), ld2x4(rowp, rowp + 16), o);
          }
          if (r < valid) {
            const int64_t addr = (tok0 + r) * HD + (int64_t)h * D + jw_base + 16 * jt + 4 * q4;
            *reinterpret_cast<uint2*>(p.out + addr) =
                pack4(p.scale * o[0], p.scale * o[1], p.scale * o[2], p.scale * o[3]);
          }
        }
      }
    }
    // S <- Diag(Gamma_last) S + K'^T U
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const float4 gc = *reinterpret_cast<const float4*>(&sm.gamc[16 * ct + 4 * q4]);
      const float gv[4] = {gc.x, gc.y, gc.z, gc.w};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        f32x4 s = Sacc[ct][jt];
#pragma unroll
        for (int t = 0; t < 4; ++t) s[t] *= gv[t];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const __bf16* rowp = &sm.kpt[(16 * ct + m16) * CS + 32 * ks + 4 * q4];
          s = mfma32(ld2x4(rowp, rowp + 16), cat(U[2 * ks][jt], U[2 * ks + 1][jt]), s);
        }
        Sacc[ct][jt] = s;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) Sfrag[ks][jt] = cat(cvt4(Sacc[2 * ks][jt]), cvt4(Sacc[2 * ks + 1][jt]));
  }

  // ---- final state
  if (p.s1 != nullptr) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const size_t off = sbase + (size_t)(16 * ct + 4 * q4 + t) * D + jw_base + 16 * jt + m16;
          if (p.s1_fp32) reinterpret_cast<float*>(p.s1)[off] = Sacc[ct][jt][t];
          else reinterpret_cast<__bf16*>(p.s1)[off] = (__bf16)Sacc[ct][jt][t];
        }
  }
}

}  // namespace

hipError_t launch_fwd(const Params& p, int nsplit, hipStream_t stream) {
  const int pairs = p.nseq * p.H;
  const int groups = (pairs + 7) / 8;
  const dim3 grid(groups * 8 * nsplit), block(NT);
  if (nsplit == 1) {
    hipLaunchKernelGGL(kda_fwd_kernel<2>, grid, block, 0, stream, p);
  } else if (nsplit == 2) {
    hipLaunchKernelGGL(kda_fwd_kernel<1>, grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
