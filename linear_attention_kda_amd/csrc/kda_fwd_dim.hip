// Chunkwise Kimi Delta Attention forward at head dimension D = K = V = 256 for
// gfx950 (MI355X).  The templates below are written for D in {64, 256}; only
// D = 256 is launched: head dimension 64 runs on the fused kernel
// (kda_fwd_hd64_kernel.hip), which is faster.
//
// The recurrence and its chunkwise algebra are those of the fused d = 128 kernel
// [core.today "Kimi Linear 특집", ch.4 혁신 2, state-update equation and the
// chunkwise remark; ch.4 혁신 1, channel-wise gate; ch.2, readout].  Per chunk of
// 64 tokens (local rows r, i), with G the within-chunk inclusive cumsum of g and
// S the chunk's start state (D x D, S[c][j]: c key channel, j value channel):
//   A[r][i] = b_r sum_c k_rc k_ic exp(G_rc - G_ic)   (i < r),   Tb = (I + A)^-1 diag(b)
//   M[r][i] = sum_c q_rc k_ic exp(G_rc - G_ic)       (i <= r)
//   Y = V - (K * exp(G)) S,   U = Tb Y
//   O = scale ((Q * exp(G)) S + M U),   S' = Diag(exp(G_last)) S + (K * exp(G_last - G))^T U
//
// Two launches instead of one fused pipeline (the d = 128 kernel's LDS plan does
// not scale to D = 256):
//  1. dim_prep_kernel, one workgroup per (chunk, head), every chunk in parallel,
//     writes the chunk's record: kg = K exp(G), qg = Q exp(G) ([64][D] bf16),
//     kpt = (K exp(G_last - G))^T ([D][64] bf16), Tb as bf16 high and low parts
//     ([64][64] each), M ([64][64] bf16, zero above the diagonal) and
//     gam = exp(G_last) ([D] fp32).  A and M come from bf16 MFMA over panels of
//     64 channels; the unit-lower inverse is fp32 forward substitution.
//  2. dim_state_kernel, one workgroup per (sequence, head, value slice of 64
//     columns at D = 64, 128 at D = 256),
//     walks the chunks in order with the fp32 state slice in MFMA accumulators.
//     U = Tb Y splits both operands into bf16 high and low parts (three
//     products) so that the solve stays close to fp32.  The next chunk's record
//     and value slice are loaded into registers while the current one computes
//     and are staged through LDS.
//
// Exponent references in the prep: the rows of 16-row block b use X_b = G at the
// last row of block b-1 (X_0 = 0).  Row operands K exp(G - X_rb), Q exp(G - X_rb)
// and the column operand K exp(X_{ib+1} - G) are <= 1; the tile of block pair
// (rb, ib) scales the column operand per channel by exp(X_rb - X_{ib+1}), which is
// <= 1 off the diagonal and bounded by one block's decay on it: the per-channel
// sum of -g over 16 tokens must stay below ~88 (natural log), the domain limit of
// the d = 128 kernel as well.
//
// MFMA 16x16x32 bf16 operand layout (64 lanes, q = lane / 16, m = lane % 16):
// A[m][8q+e], B[8q+e][m], D[4q+t][m].  Where a product consumes accumulators as
// its B operand, both operands use the k order e <-> 32ks + 4q + e (e < 4),
// 32ks + 16 + 4q + e - 4 (e >= 4), which is what two D-layout tiles hold per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int C = 64;          // chunk length
constexpr int PS = 64 + 8;     // row stride (bf16) of the prep's 64-wide LDS tiles: 144 B
constexpr int RS = 64 + 4;     // row stride (bf16) of the record's 64-wide tiles: 136 B
constexpr int NT = 256;        // threads per prep workgroup
// State workgroups: 16 value columns per wave; 64 columns (4 waves) at D = 64,
// 128 columns (8 waves) at D = 256, where the per-chunk operands are 4x larger.
template <int D>
struct Slice {
  static constexpr int nv = D == 256 ? 128 : 64;   // value columns per workgroup
  static constexpr int nt = 4 * nv;                // threads
  static constexpr int occ = D == 256 ? 1 : 2;     // workgroups per CU (LDS-bound)
};
constexpr int AS = 64 + 4;     // LDS row stride (fp32) of A
constexpr float LOG2E = 1.4426950408889634f;
constexpr int kLptMax = 256;   // longest-first ordering of the state workgroups up to this many sequences

// Byte offsets inside the record of one (chunk, head).  Rows are padded exactly
// as the state kernel's LDS tiles (4 bf16 per row: row strides of 2 dwords modulo
// the 32 LDS banks, so that the 8-byte operand reads of 16 rows spread over every
// bank) so that staging a record is a straight copy; the padding is never written
// or read.
template <int D>
struct Rec {
  static constexpr int ks = D + 4;     // row stride (bf16) of kg and qg
  static constexpr int kg = 0;
  static constexpr int qg = kg + C * ks * 2;
  static constexpr int kpt = qg + C * ks * 2;
  static constexpr int thi = kpt + D * RS * 2;
  static constexpr int tlo = thi + C * RS * 2;
  static constexpr int mm = tlo + C * RS * 2;
  static constexpr int gam = mm + C * RS * 2;
  static constexpr int bytes = gam + D * 4;
};
static_assert(Rec<64>::bytes % 256 == 0 && Rec<256>::bytes % 256 == 0, "records stay 256-byte aligned");

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) {  // 16-byte aligned
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Two 4-element runs (8-byte aligned) -> one operand in the permuted k order.
__device__ __forceinline__ bf16x8 ld2x4(const __bf16* p0, const __bf16* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
  bf16x4 r;
  r[0] = (__bf16)v[0];
  r[1] = (__bf16)v[1];
  r[2] = (__bf16)v[2];
  r[3] = (__bf16)v[3];
  return r;
}

__device__ __forceinline__ f32x4 up4(bf16x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Buffer descriptor over `bytes` bytes from `base`: loads beyond the range return
// zero and stores beyond it are dropped (raw buffer, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ int64_t seq_bos(const DimParams& p, int n) {
  return p.cu ? (int64_t)__builtin_amdgcn_readfirstlane(p.cu[n]) : (int64_t)n * p.T;
}
__device__ __forceinline__ int64_t seq_len(const DimParams& p, int n) {
  return p.cu ? (int64_t)__builtin_amdgcn_readfirstlane(p.cu[n + 1]) -
                    __builtin_amdgcn_readfirstlane(p.cu[n])
              : p.T;
}

// Sequence owning record slot s: the largest n with n + floor(bos_n / 64) <= s.
__device__ __forceinline__ int slot_seq(const DimParams& p, int64_t s) {
  int lo = 0, hi = p.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mid + seq_bos(p, mid) / C <= s) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ============================================================================ prep
// Block pairs (rb, ib), ib <= rb, numbered 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0)
// 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3).
template <int PR>
struct Pair {
  static constexpr int rb = PR < 1 ? 0 : PR < 3 ? 1 : PR < 6 ? 2 : 3;
  static constexpr int ib = PR - rb * (rb + 1) / 2;
};

struct PrepSmem {
  union {
    struct {
      __bf16 kr[C * PS];   // K exp(G - X_rb)   A row operand
      __bf16 qr[C * PS];   // Q exp(G - X_rb)   M row operand
    };
    float as[C * AS];      // A (beta-scaled, strictly lower), after the last panel
  };
  union {
    struct {
      __bf16 kh[C * PS];   // K exp(X_{ib+1} - G)   column operand
      __bf16 kt[C * PS];   // (K exp(G_last - G))^T of the panel: [channel][row]
    };
    float ts[C * AS];      // T = (I + A)^-1 (lower blocks), after the last panel
  };
  union {
    struct {
      float bt[4][64];     // per row block and channel: sum of g log2(e)
      float pf[10][64];    // exp2(X_rb - X_{ib+1}) per pair and channel
    };
    float wb[3][256];      // sum_m A_{rb,m} T_{m,ib} of one level of the inverse, after the panels
  };
  float bs[C];             // beta of the chunk
};

// One 64-channel panel's contribution to the A and M tiles of pair PR.
template <int PR>
__device__ __forceinline__ void pair_panel(const PrepSmem& sm, int q4, int m16, f32x4& a, f32x4& m) {
  constexpr int rb = Pair<PR>::rb, ib = Pair<PR>::ib;
  constexpr bool scaled = ib != rb - 1;   // the factor is 1 for ib = rb - 1
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c0 = 32 * ks + 8 * q4;
    bf16x8 cf = ld8(&sm.kh[(16 * ib + m16) * PS + c0]);
    if constexpr (scaled) {
      const float4 f0 = *reinterpret_cast<const float4*>(&sm.pf[PR][c0]);
      const float4 f1 = *reinterpret_cast<const float4*>(&sm.pf[PR][c0 + 4]);
      const float fs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) cf[e] = (__bf16)((float)cf[e] * fs[e]);
    }
    const bf16x8 kf = ld8(&sm.kr[(16 * rb + m16) * PS + c0]);
    const bf16x8 qf = ld8(&sm.qr[(16 * rb + m16) * PS + c0]);
    a = mfma32(cf, kf, a);   // D[i][r]: lane (q4, m16) holds i = 16 ib + 4 q4 + t, r = 16 rb + m16
    m = mfma32(cf, qf, m);
  }
}

// A (beta-scaled, strictly lower) into LDS and M (lower incl. the diagonal) into the record.
template <int D, int PR>
__device__ __forceinline__ void pair_store(PrepSmem& sm, __amdgpu_buffer_rsrc_t rrec, int q4, int m16,
                                           f32x4 a, f32x4 m) {
  constexpr int rb = Pair<PR>::rb, ib = Pair<PR>::ib;
  const int r = 16 * rb + m16;
  const float br = sm.bs[r];
  float va[4];
  uint16_t vm[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = 16 * ib + 4 * q4 + t;
    va[t] = i < r ? br * a[t] : 0.f;
    vm[t] = f2bf(i <= r ? m[t] : 0.f);
  }
  *reinterpret_cast<float4*>(&sm.as[r * AS + 16 * ib + 4 * q4]) = make_float4(va[0], va[1], va[2], va[3]);
  const uint2 mv = make_uint2(vm[0] | ((uint32_t)vm[1] << 16), vm[2] | ((uint32_t)vm[3] << 16));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, mv),
                                        rrec, (r * RS + 16 * ib + 4 * q4) * 2, Rec<D>::mm, 0);
}

template <int D, bool GS>
__global__ void __launch_bounds__(NT) dim_prep_kernel(DimParams p) {
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, m16 = lane & 15;
  const int h = blockIdx.x % p.H;
  const int64_t slot = blockIdx.x / p.H;
  const int n = slot_seq(p, slot);
  const int64_t bos = seq_bos(p, n), len = seq_len(p, n);
  const int64_t c = slot - n - bos / C;
  if (c * C >= len) return;   // past the sequence's last chunk (the same for the whole workgroup)
  const int64_t row0 = bos + c * C;
  const int rows = (int)(len - c * C < C ? len - c * C : C);
  const int hs = p.H * D;      // token stride of q, k, g (elements); the host bounds H * D
  // descriptors over the chunk's rows: rows past the sequence read as zero
  const size_t t0 = (size_t)row0 * hs + (size_t)h * D;
  const auto rq = rsrc(p.q + t0, ((rows - 1) * hs + D) * 2);
  const auto rk = rsrc(p.k + t0, ((rows - 1) * hs + D) * 2);
  const auto rg = GS ? rsrc(p.g + (size_t)row0 * p.H + h, ((rows - 1) * p.H + 1) * 4)
                     : rsrc(p.g + t0, ((rows - 1) * hs + D) * 4);
  const auto rb_ = rsrc(p.beta + (size_t)row0 * p.H + h, ((rows - 1) * p.H + 1) * 4);
  const auto rrec = rsrc(p.ws + ((size_t)slot * p.H + h) * Rec<D>::bytes, Rec<D>::bytes);

  if (tid < C) sm.bs[tid] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb_, tid * p.H * 4, 0, 0));

  f32x4 aA[3], aM[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) aA[j] = aM[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // raw loads of one panel (channels 64 pc + lane, rows 16 wave .. +15), issued a
  // panel ahead so that they overlap the previous panel's tile products
  float graw[16];
  uint32_t kraw[16], qraw[16];
  auto load_panel = [&](int pc) {
    const int ch = 64 * pc + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * wave + i;
      graw[i] = GS ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, 0, r * p.H * 4, 0))
                   : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, ch * 4, r * hs * 4, 0));
      kraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rk, ch * 2, r * hs * 2, 0);
      qraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rq, ch * 2, r * hs * 2, 0);
    }
  };
  load_panel(0);

  for (int pc = 0; pc < D / 64; ++pc) {
    const int ch = 64 * pc + lane;
    float gl[16], kv[16], qv[16];
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      run += graw[i] * LOG2E;
      gl[i] = run;
      kv[i] = __uint_as_float(kraw[i] << 16);
      qv[i] = __uint_as_float(qraw[i] << 16);
    }
    sm.bt[wave][lane] = run;
    __syncthreads();
    float X[5];
    X[0] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) X[b + 1] = X[b] + sm.bt[b][lane];
    const float xr = wave == 0 ? X[0] : wave == 1 ? X[1] : wave == 2 ? X[2] : X[3];
    const float xn = wave == 0 ? X[1] : wave == 1 ? X[2] : wave == 2 ? X[3] : X[4];
    const float xl = X[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * wave + i;
      const float G = xr + gl[i];
      const float eg = ex2(G);
      __builtin_amdgcn_raw_buffer_store_b16(f2bf(kv[i] * eg), rrec, ch * 2, Rec<D>::kg + r * Rec<D>::ks * 2, 0);
      __builtin_amdgcn_raw_buffer_store_b16(f2bf(qv[i] * eg), rrec, ch * 2, Rec<D>::qg + r * Rec<D>::ks * 2, 0);
      sm.kt[lane * PS + r] = (__bf16)(kv[i] * ex2(xl - G));
      const float er = ex2(G - xr);
      sm.kr[r * PS + lane] = (__bf16)(kv[i] * er);
      sm.qr[r * PS + lane] = (__bf16)(qv[i] * er);
      sm.kh[r * PS + lane] = (__bf16)(kv[i] * ex2(xn - G));
    }
    if (wave == 0) {
      sm.pf[0][lane] = ex2(X[0] - X[1]);
      sm.pf[1][lane] = ex2(X[1] - X[1]);
      sm.pf[2][lane] = ex2(X[1] - X[2]);
      sm.pf[3][lane] = ex2(X[2] - X[1]);
      sm.pf[4][lane] = ex2(X[2] - X[2]);
      sm.pf[5][lane] = ex2(X[2] - X[3]);
      sm.pf[6][lane] = ex2(X[3] - X[1]);
      sm.pf[7][lane] = ex2(X[3] - X[2]);
      sm.pf[8][lane] = ex2(X[3] - X[3]);
      sm.pf[9][lane] = ex2(X[3] - X[4]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ex2(xl)), rrec, ch * 4, Rec<D>::gam, 0);
    }
    __syncthreads();
    if (pc + 1 < D / 64) load_panel(pc + 1);
    // kp^T rows of this panel: 64 channels x 128 bytes
#pragma unroll
    for (int x = tid; x < 64 * 8; x += NT) {
      const int cr = x >> 3, part = x & 7;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, *reinterpret_cast<const uint4*>(&sm.kt[cr * PS + 8 * part])), rrec,
          (cr * RS + 8 * part) * 2, Rec<D>::kpt + 64 * pc * RS * 2, 0);
    }
    switch (wave) {
      case 0:
        pair_panel<0>(sm, q4, m16, aA[0], aM[0]);
        pair_panel<1>(sm, q4, m16, aA[1], aM[1]);
        pair_panel<8>(sm, q4, m16, aA[2], aM[2]);
        break;
      case 1:
        pair_panel<2>(sm, q4, m16, aA[0], aM[0]);
        pair_panel<3>(sm, q4, m16, aA[1], aM[1]);
        pair_panel<4>(sm, q4, m16, aA[2], aM[2]);
        break;
      case 2:
        pair_panel<5>(sm, q4, m16, aA[0], aM[0]);
        pair_panel<6>(sm, q4, m16, aA[1], aM[1]);
        break;
      default:
        pair_panel<7>(sm, q4, m16, aA[0], aM[0]);
        pair_panel<9>(sm, q4, m16, aA[1], aM[1]);
        break;
    }
    __syncthreads();   // the panel tiles are rewritten next (and A, T overlay them)
  }

  switch (wave) {
    case 0:
      pair_store<D, 0>(sm, rrec, q4, m16, aA[0], aM[0]);
      pair_store<D, 1>(sm, rrec, q4, m16, aA[1], aM[1]);
      pair_store<D, 8>(sm, rrec, q4, m16, aA[2], aM[2]);
      break;
    case 1:
      pair_store<D, 2>(sm, rrec, q4, m16, aA[0], aM[0]);
      pair_store<D, 3>(sm, rrec, q4, m16, aA[1], aM[1]);
      pair_store<D, 4>(sm, rrec, q4, m16, aA[2], aM[2]);
      break;
    case 2:
      pair_store<D, 5>(sm, rrec, q4, m16, aA[0], aM[0]);
      pair_store<D, 6>(sm, rrec, q4, m16, aA[1], aM[1]);
      break;
    default:
      pair_store<D, 7>(sm, rrec, q4, m16, aA[0], aM[0]);
      pair_store<D, 9>(sm, rrec, q4, m16, aA[1], aM[1]);
      break;
  }
  // M is zero above the diagonal blocks: (rb, ib) = (0,1..3), (1,2..3), (2,3)
  for (int x = tid; x < 6 * 64; x += NT) {
    const int blk = x >> 6, e = x & 63;   // 16 rows x 4 runs of 4 per block
    const int rb = blk < 3 ? 0 : blk < 5 ? 1 : 2;
    const int ib = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
    const int r = 16 * rb + (e >> 2), i = 16 * ib + 4 * (e & 3);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rrec,
                                          (r * RS + i) * 2, Rec<D>::mm, 0);
  }
  __syncthreads();

  // T = (I + A)^-1 by 16-row blocks: the diagonal blocks by forward substitution
  // (wave b, lane j < 16: column j of block b), then level by level
  //   T_{rb,ib} = -T_{rb,rb} sum_{m=ib}^{rb-1} A_{rb,m} T_{m,ib},  rb - ib = 1, 2, 3
  // (from (I + A) T = I: the off-diagonal blocks of I + A are those of A).
  if (lane < 16) {
    const int b0 = 16 * wave, j = lane;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) {
        if (i & 1) s1 = fmaf(sm.as[(b0 + r) * AS + b0 + i], col[i], s1);
        else s0 = fmaf(sm.as[(b0 + r) * AS + b0 + i], col[i], s0);
      }
      col[r] = r == j ? 1.f : -(s0 + s1);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.ts[(b0 + r) * AS + b0 + j] = col[r];
  }
  __syncthreads();
  {
    const int i16 = tid >> 4, j16 = tid & 15;
#pragma unroll
    for (int L = 1; L < 4; ++L) {
#pragma unroll
      for (int ib = 0; ib + L < 4; ++ib) {
        const int rb = ib + L;
        float w0 = 0.f, w1 = 0.f;
#pragma unroll
        for (int k = 16 * ib; k < 16 * rb; ++k) {
          const float t = sm.as[(16 * rb + i16) * AS + k] * sm.ts[k * AS + 16 * ib + j16];
          if (k & 1) w1 += t;
          else w0 += t;
        }
        sm.wb[ib][tid] = w0 + w1;
      }
      __syncthreads();
#pragma unroll
      for (int ib = 0; ib + L < 4; ++ib) {
        const int rb = ib + L;
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) t = fmaf(sm.ts[(16 * rb + i16) * AS + 16 * rb + k], sm.wb[ib][16 * k + j16], t);
        sm.ts[(16 * rb + i16) * AS + 16 * ib + j16] = -t;
      }
      __syncthreads();
    }
  }
  // Tb = T diag(beta) as bf16 high and low parts: thread t, row t / 4, columns 16 (t % 4) .. +15
  {
    const int r = tid >> 2, cb = tid & 3;
    uint32_t hv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 16 * cb + 2 * e + u;
        x2[u] = cb > (r >> 4) ? 0.f : sm.ts[r * AS + j] * sm.bs[j];
      }
      const __bf16 h0 = (__bf16)x2[0], h1 = (__bf16)x2[1];
      const __bf16 l0 = (__bf16)(x2[0] - (float)h0), l1 = (__bf16)(x2[1] - (float)h1);
      hv[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lv[e] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    const int off = (r * RS + 16 * cb) * 2;
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{hv[0], hv[1], hv[2], hv[3]}, rrec, off, Rec<D>::thi, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{hv[4], hv[5], hv[6], hv[7]}, rrec, off + 16, Rec<D>::thi, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{lv[0], lv[1], lv[2], lv[3]}, rrec, off, Rec<D>::tlo, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{lv[4], lv[5], lv[6], lv[7]}, rrec, off + 16, Rec<D>::tlo, 0);
  }
}

// ============================================================================ state pass
template <int D>
struct StateSmem {
  alignas(16) char rec[Rec<D>::bytes];      // the chunk's record, byte for byte
  __bf16 vs[C * (Slice<D>::nv + 8)];       // V of the chunk, this workgroup's columns
  int lens[kLptMax];
  int order;
  __device__ const __bf16* tile(int off) const { return reinterpret_cast<const __bf16*>(rec + off); }
};

template <int D>
struct Pieces {   // 16-byte pieces of one chunk's operands per thread: the record, then V
  static constexpr int nt = Slice<D>::nt;
  static constexpr int rec = Rec<D>::bytes / 16;
  static constexpr int full = rec / nt;                  // record rounds every thread takes
  static constexpr int tail = rec - full * nt;           // threads with one more piece
  static constexpr int vp = Slice<D>::nv / 8;            // V pieces per row
  static constexpr int vr = C * vp / nt;                 // V rounds
  static constexpr int per_thread = full + (tail ? 1 : 0) + vr;
  static_assert(C * vp % nt == 0, "V pieces spread evenly");
};

// The next chunk's record and V slice into registers.  Pieces past the record,
// and V rows past the sequence, read as zero through the descriptors.
template <int D>
__device__ __forceinline__ void chunk_load(u32x4* buf, __amdgpu_buffer_rsrc_t rrec,
                                           __amdgpu_buffer_rsrc_t rv, int vrow_bytes, int tid) {
  using P = Pieces<D>;
#pragma unroll
  for (int i = 0; i < P::full + (P::tail ? 1 : 0); ++i)
    buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rrec, (tid + P::nt * i) * 16, 0, 0);
#pragma unroll
  for (int i = 0; i < P::vr; ++i) {
    const int y = tid + P::nt * i, row = y / P::vp, part = y % P::vp;
    buf[P::full + (P::tail ? 1 : 0) + i] =
        __builtin_amdgcn_raw_buffer_load_b128(rv, row * vrow_bytes + 16 * part, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void chunk_stage(StateSmem<D>& sm, const u32x4* buf, int tid) {
  using P = Pieces<D>;
  constexpr int VS = Slice<D>::nv + 8;
#pragma unroll
  for (int i = 0; i < P::full; ++i)
    *reinterpret_cast<u32x4*>(sm.rec + 16 * (tid + P::nt * i)) = buf[i];
  if (P::tail && tid < P::tail)
    *reinterpret_cast<u32x4*>(sm.rec + 16 * (tid + P::nt * P::full)) = buf[P::full];
#pragma unroll
  for (int i = 0; i < P::vr; ++i) {
    const int y = tid + P::nt * i;
    *reinterpret_cast<u32x4*>(&sm.vs[(y / P::vp) * VS + 8 * (y % P::vp)]) =
        buf[P::full + (P::tail ? 1 : 0) + i];
  }
}

template <int D>
__global__ void __launch_bounds__(Slice<D>::nt, Slice<D>::occ) dim_state_kernel(DimParams p) {
  constexpr int KS = Rec<D>::ks;
  constexpr int NV = Slice<D>::nv;
  constexpr int VS = NV + 8;
  constexpr int NTS = Slice<D>::nt;
  constexpr int NCB = D / 16;   // 16-row tiles of the state slice per wave
  constexpr int NKS = D / 32;   // k-steps over the channels
  constexpr int KG = D == 64 ? 2 : 1;   // k-steps per group of the first products
  constexpr int NSL = D / NV;   // value slices per (sequence, head)
  __shared__ StateSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4_ = lane >> 4, m16_ = lane & 15;

  // workgroup -> (rank, head, value slice); the slices of one (sequence, head) share an XCD
  const int grp = blockIdx.x / (8 * NSL), rem = blockIdx.x % (8 * NSL);
  const int split = rem / 8;
  const int pidx = grp * 8 + rem % 8;
  const int rank = pidx / p.H, h = pidx % p.H;
  if (rank >= p.nseq) return;
  int n = rank;
  if (p.cu != nullptr && p.nseq > 1 && p.nseq <= kLptMax) {   // longest sequences first
    for (int s = tid; s < p.nseq; s += NTS) sm.lens[s] = p.cu[s + 1] - p.cu[s];
    __syncthreads();
    for (int s = tid; s < p.nseq; s += NTS) {
      const int ls = sm.lens[s];
      int rk = 0;
      for (int j = 0; j < p.nseq; ++j) {
        const int lj = sm.lens[j];
        rk += (lj > ls) || (lj == ls && j < s);
      }
      if (rk == rank) sm.order = s;
    }
    __syncthreads();
    n = __builtin_amdgcn_readfirstlane(sm.order);
  }
  const int64_t bos = seq_bos(p, n), len = seq_len(p, n);
  const int nch = (int)((len + C - 1) / C);
  const int jw = split * NV + 16 * wave;   // this wave's first value column
  const size_t hs = (size_t)p.H * D;
  const size_t sbase = ((size_t)n * p.H + h) * D * D;

  // the state slice: st[cb][t] = S[16 cb + 4 q4 + t][jw + m16]
  f32x4 st[NCB];
  const size_t soff = sbase + (size_t)(4 * q4_) * D + jw + m16_;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p.s0 != nullptr) {
    if (p.s0_fp32) {
      const float* s = static_cast<const float*>(p.s0) + soff;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[cb][t] = s[(16 * cb + t) * D];
    } else {
      const uint16_t* s = static_cast<const uint16_t*>(p.s0) + soff;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[cb][t] = bf2f(s[(16 * cb + t) * D]);
    }
  }

  const int64_t slot0 = n + bos / C;
  const int hsb = p.H * D * 2;   // token stride of v and out in bytes; the host bounds H * D
  auto rows_of = [&](int c) { return (int)(len - (int64_t)c * C < C ? len - (int64_t)c * C : C); };
  auto rec_of = [&](int c) {
    return rsrc(p.ws + ((size_t)(slot0 + c) * p.H + h) * Rec<D>::bytes, Rec<D>::bytes);
  };
  // this slice's V columns of the chunk's rows (later rows read as zero)
  auto v_of = [&](int c) {
    return rsrc(p.v + (size_t)(bos + (int64_t)c * C) * hs + (size_t)h * D + split * NV,
                (rows_of(c) - 1) * hsb + NV * 2);
  };

  u32x4 buf[Pieces<D>::per_thread];
  if (nch > 0) chunk_load<D>(buf, rec_of(0), v_of(0), hsb, tid);

  for (int c = 0; c < nch; ++c) {
    // lane indices through an empty asm: addresses are formed where they are used
    // instead of being kept live across the loop
    int ti = tid, q4 = q4_, m16 = m16_;
    asm volatile("" : "+v"(ti), "+v"(q4), "+v"(m16));
    __syncthreads();   // the previous chunk's operands are no longer read
    chunk_stage<D>(sm, buf, ti);
    __syncthreads();
    if (c + 1 < nch) chunk_load<D>(buf, rec_of(c + 1), v_of(c + 1), hsb, ti);

    // The products of each phase read their LDS operand fragments first: the
    // scheduling groups keep the reads ahead of the MFMAs, so that LDS latency is
    // paid once per group instead of once per product.
    // V of this wave's columns, read now and used after the first products
    float vv[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int t = 0; t < 4; ++t) vv[rb][t] = (float)sm.vs[(16 * rb + 4 * q4 + t) * VS + 16 * wave + m16];

    // P1 = kg S, P2 = qg S (rows 16 rb + 4 q4 + t, column jw + m16), KG k-steps per group
    f32x4 p1[4], p2[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) p1[rb] = p2[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < NKS; k0 += KG) {
      bf16x8 ka[KG][4], qa[KG][4];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const __bf16* kp = sm.tile(Rec<D>::kg) + (16 * rb + m16) * KS + 32 * (k0 + kk) + 4 * q4;
          const __bf16* qp = sm.tile(Rec<D>::qg) + (16 * rb + m16) * KS + 32 * (k0 + kk) + 4 * q4;
          ka[kk][rb] = ld2x4(kp, kp + 16);
          qa[kk][rb] = ld2x4(qp, qp + 16);
        }
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const bf16x8 sf = cat(cvt4(st[2 * (k0 + kk)]), cvt4(st[2 * (k0 + kk) + 1]));
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          p1[rb] = mfma32(ka[kk][rb], sf, p1[rb]);
          p2[rb] = mfma32(qa[kk][rb], sf, p2[rb]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8 * KG, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 8 * KG, 0);   // then the products
      __builtin_amdgcn_sched_barrier(0);
    }
    // Tb fragments of the solve: block pairs (ib, ks) with ks <= ib / 2
    bf16x8 tha[6], tla[6];
#pragma unroll
    for (int e = 0; e < 6; ++e) {
      const int ib = e < 2 ? e : 2 + (e - 2) / 2, ks = e < 2 ? 0 : (e - 2) % 2;
      const __bf16* th = sm.tile(Rec<D>::thi) + (16 * ib + m16) * RS + 32 * ks + 4 * q4;
      const __bf16* tl = sm.tile(Rec<D>::tlo) + (16 * ib + m16) * RS + 32 * ks + 4 * q4;
      tha[e] = ld2x4(th, th + 16);
      tla[e] = ld2x4(tl, tl + 16);
    }
    // Y = V - P1 as bf16 high and low parts, in the permuted k order over rows
    bf16x8 zh[2], zl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x4 hi[2], lo[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int rb = 2 * ks + s;
        f32x4 y;
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] = vv[rb][t] - p1[rb][t];
        hi[s] = cvt4(y);
        lo[s] = cvt4(y - up4(hi[s]));
      }
      zh[ks] = cat(hi[0], hi[1]);
      zl[ks] = cat(lo[0], lo[1]);
    }
    // U = Tb Y (Tb is lower triangular: block row ib needs k-steps 0 .. ib / 2)
    f32x4 u[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) u[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 6; ++e) {
      const int ib = e < 2 ? e : 2 + (e - 2) / 2, ks = e < 2 ? 0 : (e - 2) % 2;
      u[ib] = mfma32(tha[e], zh[ks], u[ib]);
      u[ib] = mfma32(tha[e], zl[ks], u[ib]);
      u[ib] = mfma32(tla[e], zh[ks], u[ib]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 18, 0);
    __builtin_amdgcn_sched_barrier(0);
    // M fragments, read before the output products
    bf16x8 ma[6];
#pragma unroll
    for (int e = 0; e < 6; ++e) {
      const int rb = e < 2 ? e : 2 + (e - 2) / 2, ks = e < 2 ? 0 : (e - 2) % 2;
      const __bf16* mp = sm.tile(Rec<D>::mm) + (16 * rb + m16) * RS + 32 * ks + 4 * q4;
      ma[e] = ld2x4(mp, mp + 16);
    }
    bf16x8 uf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) uf[ks] = cat(cvt4(u[2 * ks]), cvt4(u[2 * ks + 1]));

    // O = scale (P2 + M U); rows past the sequence are dropped by the descriptor
    const auto ro = rsrc(p.out + (size_t)(bos + (int64_t)c * C) * hs + (size_t)h * D + jw,
                         (rows_of(c) - 1) * hsb + 32);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 o = p2[rb];
#pragma unroll
      for (int ks = 0; ks <= rb / 2; ++ks) o = mfma32(ma[rb < 2 ? rb : 2 + 2 * (rb - 2) + ks], uf[ks], o);
      // lane-dependent row part in the vector offset, the block's row in the scalar one
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_raw_buffer_store_b16(f2bf(p.scale * o[t]), ro, (4 * q4 + t) * hsb + m16 * 2,
                                              16 * rb * hsb, 0);
    }

    // S' = Diag(gam) S + kpt U, four 16-row tiles per group
#pragma unroll
    for (int c0 = 0; c0 < NCB; c0 += 4) {
      bf16x8 kf[4][2];
      float4 gm[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        gm[cc] = *reinterpret_cast<const float4*>(sm.rec + Rec<D>::gam + (16 * (c0 + cc) + 4 * q4) * 4);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const __bf16* kp = sm.tile(Rec<D>::kpt) + (16 * (c0 + cc) + m16) * RS + 32 * ks + 4 * q4;
          kf[cc][ks] = ld2x4(kp, kp + 16);
        }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int cb = c0 + cc;
        st[cb][0] *= gm[cc].x;
        st[cb][1] *= gm[cc].y;
        st[cb][2] *= gm[cc].z;
        st[cb][3] *= gm[cc].w;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st[cb] = mfma32(kf[cc][ks], uf[ks], st[cb]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (p.s1 != nullptr) {
    if (p.s1_fp32) {
      float* s = static_cast<float*>(p.s1) + soff;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int t = 0; t < 4; ++t) s[(16 * cb + t) * D] = st[cb][t];
    } else {
      uint16_t* s = static_cast<uint16_t*>(p.s1) + soff;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int t = 0; t < 4; ++t) s[(16 * cb + t) * D] = f2bf(st[cb][t]);
    }
  }
}

template <int D>
hipError_t launch_dim(const DimParams& p, hipStream_t stream) {
  if (p.slots > 0) {
    const dim3 grid((unsigned)(p.slots * p.H));
    if (p.g_scalar) hipLaunchKernelGGL((dim_prep_kernel<D, true>), grid, dim3(NT), 0, stream, p);
    else hipLaunchKernelGGL((dim_prep_kernel<D, false>), grid, dim3(NT), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t wgs = ((int64_t)p.nseq * p.H + 7) / 8 * 8 * (D / Slice<D>::nv);
  hipLaunchKernelGGL(dim_state_kernel<D>, dim3((unsigned)wgs), dim3(Slice<D>::nt), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t dim_record_bytes(int D) { return D == 256 ? (size_t)Rec<256>::bytes : 0; }

int64_t dim_slots(int64_t nseq, int64_t rows) { return nseq + (rows + C - 1) / C + 1; }

hipError_t launch_fwd_dim(const DimParams& p, hipStream_t stream) {
  if (p.D == 256) return launch_dim<256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
