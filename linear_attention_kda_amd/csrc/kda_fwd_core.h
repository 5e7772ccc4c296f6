// Fused chunkwise Kimi Delta Attention forward kernel for gfx950 (MI355X).
//
// Recurrence (per sequence and head) [core.today "Kimi Linear 특집", ch.4 혁신 2,
// state-update equation; ch.4 혁신 1, channel-wise gate; ch.2, readout]:
//   S_t = (Diag(a_t) - b_t k_t (k_t * a_t)^T) S_{t-1} + b_t k_t v_t^T,  a_t = exp(g_t)
//   o_t = scale * S_t^T q_t
// evaluated 64 tokens at a time with the WY/UT form of the diagonal-plus-low-rank
// transition [same page, ch.4 혁신 2, chunkwise remark].  For one chunk with start
// state S (128 x 128, S[c][j]: c key channel, j value channel), local rows r, i,
// G = within-chunk inclusive cumsum of g:
//   A[r][i] = b_r sum_c k_rc k_ic exp(G_rc - G_ic)   (i < r)      (L = I + A)
//   Y       = V - (K * exp(G)) S
//   U       = L^-1 diag(b) Y          (= b_r times the delta-rule error of row r)
//   M[r][i] = sum_c q_rc k_ic exp(G_rc - G_ic)        (i <= r)
//   O       = scale * ((Q * exp(G)) S + M U)
//   S'      = Diag(exp(G_last)) S + (K * exp(G_last - G))^T U
//
// Exponent bookkeeping.  The chunk splits into four 16-row blocks; X_b is G at
// the last row of block b-1 (X_0 = 0, X_4 = G_last).  With F_r = exp(G_r - X_b)
// and H_r = exp(X_{b+1} - G_r) for r in block b (both <= 1):
//  * Kr = K*F and Qr = Q*F are the row operands of A and M, Kh = K*H the column
//    operand; tile (rb, ib) takes the per-channel factor exp(X_rb - X_{ib+1}) on
//    the column operand, shared by the A and M tiles of the pair (<= 1 off the
//    diagonal, 1 for ib = rb-1, and bounded by one block's decay on the diagonal:
//    the per-channel sum of -g over a 16-token block must stay below ~88 in
//    natural log);
//  * K*exp(G) = Kr * exp(X_b), Q*exp(G) = Qr * exp(X_b) (both <= 1);
//  * K*exp(G_last - G) = Kh * exp(G_last - X_{b+1}).
// F and H are running products of a = exp(g) along the rows.
// Chunk-level reference: when exp(+-G) stays within 2^+-96 on every channel of a
// chunk (the common case), the tiles use G itself as the reference instead --
// rows K*exp(G) and Q*exp(G) (the operands the state products use anyway),
// column K*exp(-G) -- and no pair needs a per-channel factor.
//
// Mapping: one workgroup of 8 waves owns one (sequence, head, value-column slice)
// and walks its chunks in order as a two-stage pipeline with three barriers per
// chunk (phases A, B, C):
//  * waves 0-3 ("state waves") run chunk c: phase A  Y and (Q exp(G)) S;
//    phase B  U by block forward substitution, the output, the state update.
//    The fp32 state slice (16*JT value columns per wave) lives in MFMA
//    accumulator registers for the whole sequence.
//  * waves 4-7 ("prep waves") prepare chunk c+1: phase A  the inverses of the
//    diagonal blocks of L for chunk c and the row sums of g for chunk c+1;
//    phase B  gating (VALU, exp2) into the operand tiles; phase C  V^T and the
//    state-update operand of chunk c+1, then the loads of chunk c+2.
//  * in phase C the state waves build the A and M tiles of chunk c+1 from the
//    gated tiles, two or three pairs of 16-row blocks (both tiles) per wave.
// Each tile is rewritten only after the phase in which the state waves last read
// it.  The value-independent per-chunk work is recomputed by every value slice.
//
// MFMA operand layouts used below (64 lanes, q = lane/16, m = lane%16):
//  16x16x32 bf16:  A[m][8q+e], B[8q+e][m] (e < 8),  D[4q+t][m] (t < 4)
//  16x16x16 bf16:  A[m][4q+e], B[4q+e][m] (e < 4),  D[4q+t][m]
// A contraction may permute its k index as long as both operands agree; the
// state path uses k-slot e <-> k = 32ks + 4q + e (e < 4), 32ks + 16 + 4q + e-4
// (e >= 4), which is exactly what two D-layout tiles (rows 32ks..+15 and
// 32ks+16..+31) hold per lane, so accumulators feed the next product directly.
//
// This header holds the device code of the fused kernel; each translation unit
// that includes it instantiates the variants it launches (kda_fwd_kernel.hip:
// per-channel gate, kda_gdn_kernel.hip: scalar gate).
#pragma once

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
constexpr int NT = 512;      // threads per workgroup: 4 state waves + 4 prep waves
constexpr int NP = 256;      // prep threads
constexpr int TS = D + 4;    // row stride (bf16) of token-major [64][128] tiles: 264 B
constexpr int CS = C + 12;   // row stride (bf16) of channel-major [.][64] tiles: 152 B (room for tcol)
constexpr int QS = C + 4;    // row stride (bf16) of [64][64] tiles: 136 B
constexpr int LS = 16 + 4;   // row stride (fp32) of the diagonal-block inverses
constexpr int NS = 16 + 4;   // row stride (fp32) of the diagonal blocks of A
constexpr float LOG2E = 1.4426950408889634f;

// Shared-memory plan; one workgroup per CU.
template <int NV>
struct alignas(16) Smem {
  __bf16 kg[C * TS];    // K * exp(G)                  for Y = V - (K exp(G)) S
  __bf16 qg[C * TS];    // Q * exp(G)                  for O = (Q exp(G)) S + ...
  __bf16 kr[C * TS];    // K * F                       A row operand
  __bf16 qr[C * TS];    // Q * F                       M row operand
  __bf16 kh[C * TS];    // K * H                       A and M column operand
  __bf16 kpt[D * CS];   // (K * exp(G_last - G))^T     channel-major, state update
  __bf16 vt[NV * CS];   // V^T (this slice's columns)  channel-major
  __bf16 mm[C * QS];    // M (lower incl. diagonal; blocks above the diagonal unused)
  __bf16 an[C * QS];    // -A on the off-diagonal 16x16 blocks
  float li[C * LS];     // inverses of the 4 diagonal blocks of L = I + A (fp32)
  float ndt[4 * 16 * NS];  // diagonal 16x16 blocks of A (beta-scaled, fp32): [b][r][i]
  float gamc[D];        // exp(G_last) per channel
  float beta[C];        // beta of the chunk in the state pass
  float pbeta[C];       // beta of the chunk being prepared
  float seg[8 * D];     // per 8-row group and channel: sum of g*log2(e)
  float pf[10 * D];     // exp(X_rb - X_{ib+1}) per (rb, ib <= rb) pair and channel
  int order;            // task chosen for this workgroup
  int chunk_ref;        // the chunk being prepared uses the chunk-level exponent reference
};

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

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
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
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


__device__ __forceinline__ bf16x4 ld4(const __bf16* p) {
  return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}

__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
  return __builtin_bit_cast(bf16x4, pack4(v[0], v[1], v[2], v[3]));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Column offset of the channel-major tiles V^T and K'^T: the 64 columns of row r
// start at column 4 ((r >> 4) & 3) of its 76.  The prep's 8-byte stores put rows 4
// apart in one instruction, and 8-byte LDS accesses are served 16 lanes at a time
// over 32 banks, where rows 4 apart fall 8 banks apart (24 with the 38-dword rows):
// four lanes would share each bank pair.  The offset spreads them; the readers take
// 16 consecutive rows, which share one offset (known where the row block is).
__device__ __forceinline__ int tcol(int row, int col) { return col + 4 * ((row >> 4) & 3); }

// (rb, ib) enumeration of the 10 lower-triangular 16x16 block pairs.
__device__ __forceinline__ int pair_rb(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ int pair_ib(int p) { return p - (pair_rb(p) * (pair_rb(p) + 1)) / 2; }

// The A and M tiles of block pair PR = (rb, ib): lane (q4, m16) gets
// tile[r = 16rb + m16][i = 16ib + 4q4 + t] of sum_c row[r][c] col[i][c].
// Writes -A off the diagonal, A's diagonal block (fp32, beta-scaled, for the
// inverse), and M without the attention scale (the output applies it), each
// masked to its triangle.
//  * chunk reference (FAST): rows -K exp(G) (A) and Q exp(G) (M), the
//    tiles the state products use; column K exp(-G).
//  * block references: rows Kr = K F (A) and Qr = Q F (M), column Kh = K H
//    scaled per channel by exp(X_rb - X_{ib+1}) (skipped for ib == rb - 1,
//    where the factor is 1).
template <int NV, int PR, bool FAST, int DK>
__device__ __forceinline__ void tile_pair(Smem<NV>& sm, int q4, int m16) {
  constexpr int rb = PR < 1 ? 0 : PR < 3 ? 1 : PR < 6 ? 2 : 3;
  constexpr int ib = PR - rb * (rb + 1) / 2;
  constexpr bool scaled = !FAST && ib != rb - 1;
  const __bf16* krow = FAST ? sm.kg : sm.kr;
  const __bf16* qrow = FAST ? sm.qg : sm.qr;
  constexpr int KS = DK / 32;  // 32-channel slices (channels past DK are zero)
  bf16x8 cf[KS], kf[KS], qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = 32 * ks + 8 * q4;
    const __bf16* cp = &sm.kh[(16 * ib + m16) * TS + c0];
    const __bf16* kp = &krow[(16 * rb + m16) * TS + c0];
    const __bf16* qp = &qrow[(16 * rb + m16) * TS + c0];
    cf[ks] = ld2x4(cp, cp + 4);
    kf[ks] = ld2x4(kp, kp + 4);
    qf[ks] = ld2x4(qp, qp + 4);
  }
  if constexpr (scaled) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * ks + 8 * q4;
      const float4 f0 = *reinterpret_cast<const float4*>(&sm.pf[PR * D + c0]);
      const float4 f1 = *reinterpret_cast<const float4*>(&sm.pf[PR * D + c0 + 4]);
      const float fs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) cf[ks][e] = (__bf16)(bf2f(cf[ks][e]) * fs[e]);
    }
  }
  f32x4 ta = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 tm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    ta = mfma32(cf[ks], kf[ks], ta);  // D[i][r]
    tm = mfma32(cf[ks], qf[ks], tm);
  }
  const int r = 16 * rb + m16;
  const float br = FAST ? -sm.pbeta[r] : sm.pbeta[r];  // the FAST row operand is -K exp(G)
  float va[4], vm[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int i = 16 * ib + 4 * q4 + tt;
    va[tt] = (i < r) ? br * ta[tt] : 0.f;
    vm[tt] = (i <= r) ? tm[tt] : 0.f;
  }
  if constexpr (ib == rb) {
    *reinterpret_cast<float4*>(&sm.ndt[(rb * 16 + m16) * NS + 4 * q4]) =
        make_float4(va[0], va[1], va[2], va[3]);
  } else {
    *reinterpret_cast<uint2*>(&sm.an[r * QS + 16 * ib + 4 * q4]) =
        pack4(-va[0], -va[1], -va[2], -va[3]);
  }
  *reinterpret_cast<uint2*>(&sm.mm[r * QS + 16 * ib + 4 * q4]) = pack4(vm[0], vm[1], vm[2], vm[3]);
}

template <int NV, bool FAST, int DK>
__device__ __forceinline__ void tile_pairs(Smem<NV>& sm, int wave, int q4, int m16) {
  switch (wave) {
    case 0:
      tile_pair<NV, 0, FAST, DK>(sm, q4, m16);
      tile_pair<NV, 1, FAST, DK>(sm, q4, m16);
      tile_pair<NV, 8, FAST, DK>(sm, q4, m16);
      break;
    case 1:
      tile_pair<NV, 2, FAST, DK>(sm, q4, m16);
      tile_pair<NV, 3, FAST, DK>(sm, q4, m16);
      tile_pair<NV, 4, FAST, DK>(sm, q4, m16);
      break;
    case 2:
      tile_pair<NV, 5, FAST, DK>(sm, q4, m16);
      tile_pair<NV, 6, FAST, DK>(sm, q4, m16);
      break;
    default:
      tile_pair<NV, 7, FAST, DK>(sm, q4, m16);
      tile_pair<NV, 9, FAST, DK>(sm, q4, m16);
      break;
  }
}

// Phase C tile work of state wave `wave` (0..3, wave-uniform): pairs (0,0) (1,0)
// (3,2); (1,1) (2,0) (2,1); (2,2) (3,0); (3,1) (3,3) -- with block references
// the seven pairs that scale their column operand spread two per wave.  The
// pairs of a wave are independent straight-line code, so their loads and
// products overlap.
template <int NV, int DK>
__device__ __forceinline__ void build_tiles(Smem<NV>& sm, int wave, int q4_, int m16_) {
  // lane indices through an empty asm: the tile addresses are then formed here on
  // every call instead of being kept live (or spilled) across the whole loop
  int q4 = q4_, m16 = m16_;
  asm volatile("" : "+v"(q4), "+v"(m16));
  if (__builtin_amdgcn_readfirstlane(sm.chunk_ref)) tile_pairs<NV, true, DK>(sm, wave, q4, m16);
  else tile_pairs<NV, false, DK>(sm, wave, q4, m16);
}

struct Work {
  int64_t bos;     // first token of the run
  int64_t len;     // tokens in the run
  int h;           // head
  int j0;          // first value column of this workgroup's slice
  int nchunks;
  int s0_mode;     // start state: 0 zero, 1 bf16 at s0, 2 fp32 at s0, 3 identity
  int s1_fp32;     // end state stored as fp32 (else bf16)
  int vzero;       // values read as zero
  int o_lane;      // outputs are a fix-up block's O0, stored in the fix-up's lane order
  const void* s0;  // this (sequence, head)'s 128 x 128 start state
  void* s1;        // where its end state goes, or null
  __bf16* o;       // output rows of the run's first chunk for head h (bf16)
  int orow;        // elements between output rows (H * 128, or 128 in a fix-up block)
  int64_t ochunk;  // elements between the first rows of consecutive chunks
  uint16_t* sb;    // also the end state in the fix-up's bf16 operand order, or null
  float* ck;       // checkpoint of the run's first chunk (chunk c at + c * H * 128 * 128), or null
};

// Buffer descriptor over `bytes` bytes from `base`; loads beyond the range return
// zero and stores beyond it are dropped (raw buffer, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Wave-wide integer scans and reductions on DPP row shifts and row broadcasts
// (lanes shifted in from outside a row read zero).
template <int ctrl, int rmask = 0xf>
__device__ __forceinline__ int dpp_in(int x) {
  return __builtin_amdgcn_update_dpp(0, x, ctrl, rmask, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes: within rows of 16 by doubling
// shifts, then row 0's total into rows 1 and 3, lane 31's into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_in<0x111>(x);        // row_shr:1
  x += dpp_in<0x112>(x);        // row_shr:2
  x += dpp_in<0x114>(x);        // row_shr:4
  x += dpp_in<0x118>(x);        // row_shr:8
  x += dpp_in<0x142, 0xa>(x);   // row_bcast:15
  x += dpp_in<0x143, 0xc>(x);   // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// Maximum of non-negative values over the 64 lanes.
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, dpp_in<0x111>(x));
  x = max(x, dpp_in<0x112>(x));
  x = max(x, dpp_in<0x114>(x));
  x = max(x, dpp_in<0x118>(x));
  x = max(x, dpp_in<0x142, 0xa>(x));
  x = max(x, dpp_in<0x143, 0xc>(x));
  return __builtin_amdgcn_readlane(x, 63);
}

// ============================================================================ prep waves
// Prep thread t (0..255) owns rows 8*rg..8*rg+7 and channels 4*cg..4*cg+3 of a chunk.
template <int NV>
struct ChunkRegs {
  float4 g[8];
  uint2 q[8];
  uint2 k[8];
  uint32_t v[8][NV / 64];  // NV/32 bf16 values per row
  float beta;
};

// Buffer descriptors for chunk `ch` of the sequence.  Each tensor's descriptor
// starts at the chunk's first row and covers exactly its `valid` rows, so rows
// past the end of a partial last chunk read as zero (zero rows leave the
// recurrence unchanged: k = 0, v = 0, beta = 0, g = 0).
struct ChunkSrc {
  __amdgpu_buffer_rsrc_t g, q, k, v, b;
};

template <bool GS, int DK>
__device__ __forceinline__ ChunkSrc chunk_src(const Params& p, const Work& w, int ch) {
  const int64_t tok0 = w.bos + (int64_t)ch * C;
  const int64_t rest = w.len - (int64_t)ch * C;
  // chunks past the end of the sequence get empty descriptors: every load is zero
  const int valid = rest <= 0 ? 0 : rest < C ? (int)rest : C;
  const int HD = p.H * DK;
  const int64_t base = tok0 * HD + (int64_t)w.h * DK;
  ChunkSrc s;
  // the gate: per channel [rows][H][DK], or one value per token and head [rows][H]
  s.g = GS ? rsrc(p.g + tok0 * p.H + w.h, valid * p.H * 4) : rsrc(p.g + base, valid * HD * 4);
  s.q = rsrc(p.q + base, valid * HD * 2);
  s.k = rsrc(p.k + base, valid * HD * 2);
  s.v = rsrc(p.v + base + w.j0, w.vzero ? 0 : valid * HD * 2);
  s.b = rsrc(p.beta + tok0 * p.H + w.h, valid * p.H * 4);
  return s;
}

// Prep thread t loads rows 8*rg..8*rg+7, channels 4*cg..4*cg+3 (rg = t/32,
// cg = t%32), in pieces so that each register set is refilled as soon as the
// previous chunk has consumed it.  With a head dimension DK < 128 the channels
// from DK on read as zero: those lanes take an offset past every descriptor's
// range (2^31: above any range, and with the row offset still below 2^32, since
// H * DK <= 2^22), so the chunk runs as a 128-channel one whose extra key
// channels are zero and leave the recurrence unchanged.
template <int DK>
__device__ __forceinline__ int chan_offset(int cg, int vo) {
  if constexpr (DK == 128) return vo;
  else return 4 * cg < DK ? vo : (int)0x80000000u;
}

template <int NV, bool GS, int DK>
__device__ __forceinline__ void load_g(ChunkRegs<NV>& R, const ChunkSrc& s, int HD, int t) {
  const int rg = t >> 5, cg = t & 31;
  if constexpr (GS) {
    // one gate per row, the same for the thread's four channels
    const int H = HD / DK;
    const int vo = chan_offset<DK>(cg, rg * 8 * H * 4);
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(s.g, vo, r8 * H * 4, 0));
      R.g[r8] = make_float4(x, x, x, x);
    }
    return;
  }
  const int vo = chan_offset<DK>(cg, rg * 8 * HD * 4 + 16 * cg);  // lane part; the row goes in soffset
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) {
    const f32x4 gv = __builtin_amdgcn_raw_buffer_load_b128(s.g, vo, r8 * HD * 4, 0);
    R.g[r8] = make_float4(gv[0], gv[1], gv[2], gv[3]);
  }
}

template <int NV, int DK>
__device__ __forceinline__ void load_qk(ChunkRegs<NV>& R, const ChunkSrc& s, int HD, int t, int r8) {
  const int rg = t >> 5, cg = t & 31;
  const int vo = chan_offset<DK>(cg, rg * 8 * HD * 2 + 8 * cg);
  const auto qv = __builtin_amdgcn_raw_buffer_load_b64(s.q, vo, r8 * HD * 2, 0);
  const auto kv = __builtin_amdgcn_raw_buffer_load_b64(s.k, vo, r8 * HD * 2, 0);
  R.q[r8] = make_uint2(qv[0], qv[1]);
  R.k[r8] = make_uint2(kv[0], kv[1]);
}

template <int NV>
__device__ __forceinline__ void load_v(ChunkRegs<NV>& R, const ChunkSrc& s, int HD, int t) {
  const int rg = t >> 5, cg = t & 31;
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) {
    if constexpr (NV == 128) {
      const auto vv = __builtin_amdgcn_raw_buffer_load_b64(s.v, rg * 8 * HD * 2 + 8 * cg, r8 * HD * 2, 0);
      R.v[r8][0] = vv[0];
      R.v[r8][1] = vv[1];
    } else {
      R.v[r8][0] = __builtin_amdgcn_raw_buffer_load_b32(s.v, rg * 8 * HD * 2 + 4 * cg, r8 * HD * 2, 0);
    }
  }
}

template <int NV>
__device__ __forceinline__ void load_beta(ChunkRegs<NV>& R, const ChunkSrc& s, int H, int t) {
  R.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(s.b, (t & 63) * H * 4, 0, 0));
}

template <int NV, bool GS, int DK>
__device__ __forceinline__ void load_chunk(ChunkRegs<NV>& R, const Params& p, const Work& w,
                                           int ch, int t) {
  const ChunkSrc s = chunk_src<GS, DK>(p, w, ch);
  const int HD = p.H * DK;
  // the scheduling barriers keep this issue order, which the loop's memory-counter
  // waits assume on entry as well
  load_beta<NV>(R, s, p.H, t);
  __builtin_amdgcn_sched_barrier(0);
  load_g<NV, GS, DK>(R, s, HD, t);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) load_qk<NV, DK>(R, s, HD, t, r8);
  __builtin_amdgcn_sched_barrier(0);
  load_v<NV>(R, s, HD, t);
}

// Value of x in lane `src` of this lane's 16-lane row (DPP row broadcast).
template <int src>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                           0x150 + src, 0xF, 0xF, false));
}

// Inverse of the diagonal block b of L = I + A (A strictly lower, beta-scaled, fp32
// rows in ndt), written to li in fp32.  One wave: lane (q4, m16) holds
// X[r = m16][j = 4q4 + t], t < 4, and the right-looking substitution
// X[r][.] -= N[r][i] X[i][.] (all r at once; N[r][i] = 0 for r <= i) takes row i
// from lane i of the same 16-lane row once it is final.
template <int i>
__device__ __forceinline__ void inverse_step(float (&x)[4], const float (&n)[16]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) x[t] = fmaf(-n[i], row_bcast<i>(x[t]), x[t]);
}

template <int NV>
__device__ __forceinline__ void diag_inverse(Smem<NV>& sm, int b, int q4, int m16) {
  const float* Nr = &sm.ndt[(b * 16 + m16) * NS];
  float n[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(&Nr[4 * c]);
    n[4 * c] = v.x; n[4 * c + 1] = v.y; n[4 * c + 2] = v.z; n[4 * c + 3] = v.w;
  }
  float x[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) x[t] = (m16 == 4 * q4 + t) ? 1.f : 0.f;
  inverse_step<0>(x, n);  inverse_step<1>(x, n);  inverse_step<2>(x, n);
  inverse_step<3>(x, n);  inverse_step<4>(x, n);  inverse_step<5>(x, n);
  inverse_step<6>(x, n);  inverse_step<7>(x, n);  inverse_step<8>(x, n);
  inverse_step<9>(x, n);  inverse_step<10>(x, n); inverse_step<11>(x, n);
  inverse_step<12>(x, n); inverse_step<13>(x, n); inverse_step<14>(x, n);
  *reinterpret_cast<float4*>(&sm.li[(16 * b + m16) * LS + 4 * q4]) = make_float4(x[0], x[1], x[2], x[3]);
}

template <int NV, bool GS, int DK>
__device__ __forceinline__ void prep_loop(Smem<NV>& sm, const Params& p, const Work& w) {
  const int t = threadIdx.x - (NT - NP);   // 0..255
  const int pw = __builtin_amdgcn_readfirstlane(t >> 6);  // prep wave 0..3 (wave-uniform)
  const int lane = t & 63, q4 = lane >> 4, m16 = lane & 15;
  const int rg = t >> 5, cg = t & 31;
  const int blk = pw;                      // 16-row block of this thread's rows
  const bool second = (rg & 1) != 0;       // rows 8..15 of the block
  constexpr int VPT = NV / 32;             // value columns per thread
  const int HD = p.H * DK;
  // wave-uniform 0/1 selectors of this wave's block (multiplied in, never branched on)
  const float m0 = blk == 0 ? 1.f : 0.f, m1 = blk == 1 ? 1.f : 0.f;
  const float m2 = blk == 2 ? 1.f : 0.f, m3 = blk == 3 ? 1.f : 0.f;
  // Each half-wave (pw, second) produces one per-channel factor: the seven pairs
  // that scale their column operand, exp(X_rb - X_{ib+1}), and exp(G_last) in the
  // eighth slot.  Its exponent is sum_k wx[k] X[k] (X[0] = 0 drops out).
  const int slot = 2 * pw + (second ? 1 : 0);
  const int spr = slot == 0 ? 0 : slot == 1 ? 2 : slot == 2 ? 3 : slot == 3 ? 5
                : slot == 4 ? 6 : slot == 5 ? 7 : slot == 6 ? 9 : -1;  // -1: exp(G_last)
  float wx[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    if (spr < 0) {
      wx[k] = k == 4 ? 1.f : 0.f;
    } else {
      const int rb = pair_rb(spr), ib = pair_ib(spr);
      wx[k] = (k == rb ? 1.f : 0.f) - (k == ib + 1 ? 1.f : 0.f);
    }
  }

  ChunkRegs<NV> R;
  load_chunk<NV, GS, DK>(R, p, w, 0, t);

  // Iteration it prepares chunk pc = it + 1 while the state waves run chunk it.
  // The loop body has no branches around its loads, so the memory-counter waits
  // stay exact; the state waves' last chunk is finished after the loop.
  for (int it = -1; it < w.nchunks - 1; ++it) {
    const int pc = it + 1;
    uint2 kpt_hold[4][2];                  // channel 4cg+e: rows 8rg..8rg+3, 8rg+4..8rg+7
    float4 gamc_hold;
    float pother[4];                       // exp2 of the other half-block's sum (A -> B)
    float sother[4], sown[4];              // the other half-block's and this group's sums

    // ---- phase A: inverses for chunk `it` (used in the state waves' phase B); for
    // chunk pc the 8-row sums of g*log2(e), the decays a = exp(g), and the
    // block-local H pass: H_r = H_{r+1} a_{r+1}, last row first, and K * H
    if (it >= 0) diag_inverse(sm, pw, q4, m16);
    {
      float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        float4& g = R.g[r8];
        g.x *= LOG2E; g.y *= LOG2E; g.z *= LOG2E; g.w *= LOG2E;
        s[0] += g.x; s[1] += g.y; s[2] += g.z; s[3] += g.w;
      }
      *reinterpret_cast<float4*>(&sm.seg[rg * D + 4 * cg]) = make_float4(s[0], s[1], s[2], s[3]);
      // the other half of this block is lane ^ 32 of the same wave
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s[e]), __float_as_uint(s[e]),
                                                          false, false);
        sown[e] = s[e];
        sother[e] = __uint_as_float(second ? p32[0] : p32[1]);
        pother[e] = ex2(sother[e]);
      }
      if (t < C) sm.pbeta[t] = R.beta;
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        R.g[r8] = make_float4(ex2(R.g[r8].x), ex2(R.g[r8].y), ex2(R.g[r8].z), ex2(R.g[r8].w));
        // the decays are formed here, not rematerialised next to their uses in phase B
        asm volatile("" : "+v"(R.g[r8].x), "+v"(R.g[r8].y), "+v"(R.g[r8].z), "+v"(R.g[r8].w));
      }
    }
    __syncthreads();  // (A) the state waves are done with K exp(G), Q exp(G), V^T, beta

    // ---- phase B: gated operand tiles of chunk pc
    {
      const ChunkSrc nsrc = chunk_src<GS, DK>(p, w, pc + 1);
      // beta of the next chunk is fetched first: the next phase A waits only for
      // beta and g (the memory counter retires loads in order)
      if (t < C) sm.beta[t] = R.beta;
      load_beta<NV>(R, nsrc, p.H, t);
      // X[k] = G (log2) at the last row of block k-1 per channel (X[0] = 0,
      // X[4] = G_last): running sums of the 8-row group sums.
      float X[5][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) X[0][e] = 0.f;
      {
        float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float4 sg = *reinterpret_cast<const float4*>(&sm.seg[r * D + 4 * cg]);
          run[0] += sg.x; run[1] += sg.y; run[2] += sg.z; run[3] += sg.w;
          if (r & 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) X[(r + 1) >> 1][e] = run[e];
          }
        }
      }
      gamc_hold = make_float4(ex2(X[4][0]), ex2(X[4][1]), ex2(X[4][2]), ex2(X[4][3]));
      // Chunk-level reference when exp(+-G) stays within 2^+-96 on every channel
      // (G falls along the chunk for g <= 0, so G_last bounds it); otherwise the
      // 16-row block references.  All prep waves reach the same decision.
      float xmn = X[1][0], xmx = X[1][0];
#pragma unroll
      for (int k = 1; k < 5; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xmn = fminf(xmn, X[k][e]);
          xmx = fmaxf(xmx, X[k][e]);
        }
      const int span = __float_as_int(fmaxf(-xmn, 4.f * xmx));
      const bool chunk_ref = wave_max(span) < __float_as_int(96.f);
      if (t == 0) sm.chunk_ref = chunk_ref ? 1 : 0;
      if (chunk_ref) {
        // G before this thread's first row (Xg) and after its last row (Xe)
        float nE[4], Hc[4], ig[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float Xb = m1 * X[1][e] + m2 * X[2][e] + m3 * X[3][e];
          const float Xg = second ? Xb + sother[e] : Xb;
          nE[e] = -ex2(Xg);
          Hc[e] = ex2(X[4][e] - (Xg + sown[e]));
          ig[e] = ex2(-X[4][e]);
        }
        // last row first: K' = K exp(G_last - G) and K exp(-G) = K' exp(-G_last)
        uint32_t kpw[4][4];
#pragma unroll
        for (int r8 = 7; r8 >= 0; --r8) {
          float kf[4], kp[4], kh[4];
          unpack4(R.k[r8], kf);
          const float4 av = R.g[r8];
          const float ar[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kp[e] = kf[e] * Hc[e];
            kh[e] = kp[e] * ig[e];
            Hc[e] *= ar[e];
          }
          if (r8 & 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) kpw[e][r8 >> 1] = __float_as_uint(kp[e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) kpw[e][r8 >> 1] = pack2(kp[e], __uint_as_float(kpw[e][r8 >> 1]));
          }
          *reinterpret_cast<uint2*>(&sm.kh[(rg * 8 + r8) * TS + 4 * cg]) = pack4(kh[0], kh[1], kh[2], kh[3]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kpt_hold[e][0] = make_uint2(kpw[e][0], kpw[e][1]);
          kpt_hold[e][1] = make_uint2(kpw[e][2], kpw[e][3]);
        }
        // first row first: -K exp(G) and Q exp(G)
#pragma unroll
        for (int r8 = 0; r8 < 8; ++r8) {
          float qf[4], kf[4], kg[4], qg[4];
          unpack4(R.q[r8], qf);
          unpack4(R.k[r8], kf);
          const float4 av = R.g[r8];
          const float ar[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            nE[e] *= ar[e];
            kg[e] = kf[e] * nE[e];
            qg[e] = -(qf[e] * nE[e]);
          }
          const int o = (rg * 8 + r8) * TS + 4 * cg;
          *reinterpret_cast<uint2*>(&sm.kg[o]) = pack4(kg[0], kg[1], kg[2], kg[3]);
          *reinterpret_cast<uint2*>(&sm.qg[o]) = pack4(qg[0], qg[1], qg[2], qg[3]);
        }
      } else {
        // 16-row block references: block-local H pass, H_r = H_{r+1} a_{r+1}, last row first
        {
          float Hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) Hv[e] = second ? 1.f : pother[e];  // H of the last row
#pragma unroll
          for (int r8 = 7; r8 >= 0; --r8) {
            float kf[4], kh[4];
            unpack4(R.k[r8], kf);
            const float4 av = R.g[r8];
            const float ar[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              kh[e] = kf[e] * Hv[e];
              Hv[e] *= ar[e];
            }
            *reinterpret_cast<uint2*>(&sm.kh[(rg * 8 + r8) * TS + 4 * cg]) = pack4(kh[0], kh[1], kh[2], kh[3]);
          }
        }
        float eCX[4], eXb[4];
        {
          float fs[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float Xb = m1 * X[1][e] + m2 * X[2][e] + m3 * X[3][e];
            const float Xb1 = m0 * X[1][e] + m1 * X[2][e] + m2 * X[3][e] + m3 * X[4][e];
            eCX[e] = ex2(X[4][e] - Xb1);
            eXb[e] = ex2(Xb);
            fs[e] = ex2(wx[1] * X[1][e] + wx[2] * X[2][e] + wx[3] * X[3][e] + wx[4] * X[4][e]);
          }
          // this half-wave's pair factor
          if (spr >= 0) *reinterpret_cast<float4*>(&sm.pf[spr * D + 4 * cg]) = make_float4(fs[0], fs[1], fs[2], fs[3]);
        }
        // Hc_r = H_r exp(G_last - X_{b+1}) (the state-update operand K' = K * Hc)
        float Hc[8][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Hc[7][e] = (second ? 1.f : pother[e]) * eCX[e];
#pragma unroll
        for (int r8 = 6; r8 >= 0; --r8) {
          const float4 av = R.g[r8 + 1];
          Hc[r8][0] = Hc[r8 + 1][0] * av.x; Hc[r8][1] = Hc[r8 + 1][1] * av.y;
          Hc[r8][2] = Hc[r8 + 1][2] * av.z; Hc[r8][3] = Hc[r8 + 1][3] * av.w;
        }
        // F_r = F_{r-1} a_r, first row first: row operands K * F, Q * F, the state
        // operands -K * exp(G) = -K * F * exp(X_b), Q * exp(G), and K'
        {
          uint32_t kpw[4][4];  // K' of row pairs (2j, 2j+1), per channel
          float F[4], nXb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            F[e] = second ? pother[e] : 1.f;  // F of the row before
            nXb[e] = -eXb[e];
          }
#pragma unroll
          for (int r8 = 0; r8 < 8; ++r8) {
            const int row = rg * 8 + r8;
            float qf[4], kf[4], kr[4], qr[4], kg[4], qg[4], kp[4];
            unpack4(R.q[r8], qf);
            unpack4(R.k[r8], kf);
            const float4 av = R.g[r8];
            const float ar[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              F[e] *= ar[e];
              kr[e] = kf[e] * F[e];
              qr[e] = qf[e] * F[e];
              kg[e] = kr[e] * nXb[e];   // -K exp(G)
              qg[e] = qr[e] * eXb[e];   // Q exp(G)
              kp[e] = kf[e] * Hc[r8][e];
            }
            if (r8 & 1) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
              kpw[e][r8 >> 1] = pack2(__uint_as_float(kpw[e][r8 >> 1]), kp[e]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) kpw[e][r8 >> 1] = __float_as_uint(kp[e]);
            }
            const int o = row * TS + 4 * cg;
            *reinterpret_cast<uint2*>(&sm.kr[o]) = pack4(kr[0], kr[1], kr[2], kr[3]);
            *reinterpret_cast<uint2*>(&sm.qr[o]) = pack4(qr[0], qr[1], qr[2], qr[3]);
            *reinterpret_cast<uint2*>(&sm.kg[o]) = pack4(kg[0], kg[1], kg[2], kg[3]);
            *reinterpret_cast<uint2*>(&sm.qg[o]) = pack4(qg[0], qg[1], qg[2], qg[3]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kpt_hold[e][0] = make_uint2(kpw[e][0], kpw[e][1]);
            kpt_hold[e][1] = make_uint2(kpw[e][2], kpw[e][3]);
          }
        }
      }
      load_g<NV, GS, DK>(R, nsrc, HD, t);  // the decays of this chunk are consumed
    }
    __syncthreads();  // (B) the state waves are done with -A, M, K'^T and exp(G_last)

    // ---- phase C: state-update operand, exp(G_last) and V^T of chunk pc (the state
    // waves build its A and M tiles meanwhile)
    {
      // q, k and v of chunk pc are consumed once V^T is stored; the next chunk's are
      // fetched after this phase's stores, which would otherwise wait behind the
      // issue of the loads
      const ChunkSrc nsrc = chunk_src<GS, DK>(p, w, pc + 1);
      // V^T (channel-major)
#pragma unroll
      for (int e = 0; e < VPT; ++e) {
        // column e of this thread: the low (even e) or high half of each row's word,
        // two rows per 32-bit word
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t pw2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pw2[j] = __builtin_amdgcn_perm(R.v[2 * j + 1][e >> 1], R.v[2 * j][e >> 1], sel);
        const int row = VPT * cg + e;
        *reinterpret_cast<uint2*>(&sm.vt[row * CS + tcol(row, rg * 8)]) = make_uint2(pw2[0], pw2[1]);
        *reinterpret_cast<uint2*>(&sm.vt[row * CS + tcol(row, rg * 8 + 4)]) = make_uint2(pw2[2], pw2[3]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * cg + e;
        *reinterpret_cast<uint2*>(&sm.kpt[row * CS + tcol(row, rg * 8)]) = kpt_hold[e][0];
        *reinterpret_cast<uint2*>(&sm.kpt[row * CS + tcol(row, rg * 8 + 4)]) = kpt_hold[e][1];
      }
      if (rg == 0) *reinterpret_cast<float4*>(&sm.gamc[4 * cg]) = gamc_hold;
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) load_qk<NV, DK>(R, nsrc, HD, t, r8);
      load_v<NV>(R, nsrc, HD, t);
    }
    __syncthreads();  // (C) chunk pc fully published
  }
  // the state waves' last chunk: its inverses, then the same three barriers
  if (w.nchunks > 0) diag_inverse(sm, pw, q4, m16);
  __syncthreads();
  __syncthreads();
  __syncthreads();
}

// ============================================================================ state waves
template <int JT, int DK>
__device__ __forceinline__ void state_loop(Smem<64 * JT>& sm, const Params& p, const Work& w) {
  constexpr int CT = DK / 16;   // 16-row tiles of the state (key channels)
  constexpr int KS = DK / 32;   // 32-channel slices of the products over the key channels
  const int tid = threadIdx.x;
  const int wave = tid >> 6;  // 0..3
  const int lane = tid & 63, q4 = lane >> 4, m16 = lane & 15;
  const int jw_base = w.j0 + 16 * JT * wave;   // first global value column of this wave
  const int jl_base = 16 * JT * wave;          // first column within the slice

  // Sacc[ct][jt][t] = S[16ct + 4q4 + t][jw_base + 16jt + m16]
  f32x4 Sacc[CT][JT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) Sacc[ct][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (w.s0_mode == 3) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          Sacc[ct][jt][t] = (16 * ct + 4 * q4 + t == jw_base + 16 * jt + m16) ? 1.f : 0.f;
  } else if (w.s0_mode == 2) {
    const float* s0 = reinterpret_cast<const float*>(w.s0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          Sacc[ct][jt][t] = s0[(16 * ct + 4 * q4 + t) * DK + jw_base + 16 * jt + m16];
  } else if (w.s0_mode == 1) {
    const __bf16* s0 = reinterpret_cast<const __bf16*>(w.s0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          Sacc[ct][jt][t] = bf2f(s0[(16 * ct + 4 * q4 + t) * DK + jw_base + 16 * jt + m16]);
  }

  for (int it = -1; it < w.nchunks; ++it) {
    const bool act = it >= 0;
    const int64_t rest = w.len - (int64_t)it * C;
    const int valid = rest < C ? (int)rest : C;
    f32x4 Z[4][JT];   // beta * Y, rows 16b + 4q4 + t, column m16
    f32x4 O[4][JT];   // O^T: row j = 16jt + 4q4 + t, column r = 16rt + m16

    // ---- phase A: Y = V - (K exp(G)) S -> Z = beta * Y;  O^T = S^T (Q exp(G))^T
    // (the prep waves store -K exp(G) and Q exp(G))
    if (DK == 128 && act && w.ck != nullptr) {  // the state entering this chunk, for the backward pass
      // one lane offset; the row and column-tile terms are scalar offsets
      const auto crs = rsrc(w.ck + (size_t)it * p.H * (D * D), D * D * 4);
      const int lo = ((4 * q4) * D + jw_base + m16) * 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Sacc[ct][jt][t]), crs, lo,
                                                  ((16 * ct + t) * D + 16 * jt) * 4, 0);
    }
    if (act) {
      // Z starts at V and accumulates (-K exp(G)) S
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const int jl = jl_base + 16 * jt + m16;
          float vv[4];
          unpack4(*reinterpret_cast<const uint2*>(&sm.vt[jl * CS + tcol(jl, 16 * b + 4 * q4)]), vv);
          Z[b][jt] = f32x4{vv[0], vv[1], vv[2], vv[3]};
          O[b][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      // one 32-channel slice of the bf16 state copy at a time (k-slot order of the
      // products), so that only a quarter of it is live
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 Sfrag[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Sfrag[jt] = cat(cvt4(Sacc[2 * ks][jt]), cvt4(Sacc[2 * ks + 1][jt]));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const __bf16* kp = &sm.kg[(16 * b + m16) * TS + 32 * ks + 4 * q4];
          const __bf16* qp = &sm.qg[(16 * b + m16) * TS + 32 * ks + 4 * q4];
          const bf16x8 ka = ld2x4(kp, kp + 16);
          const bf16x8 qa = ld2x4(qp, qp + 16);
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) {
            Z[b][jt] = mfma32(ka, Sfrag[jt], Z[b][jt]);
            O[b][jt] = mfma32(Sfrag[jt], qa, O[b][jt]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float4 bb = *reinterpret_cast<const float4*>(&sm.beta[16 * b + 4 * q4]);
        const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t) Z[b][jt][t] *= bv[t];
      }
    }
    __syncthreads();  // (A)

    // ---- phase B: U = L^-1 Z (block forward substitution), output, state update
    if (act) {
      bf16x4 U[4][JT];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // row m16 of the block's inverse, Li[m16][4q4 + e], and z in its D layout are
        // exactly the operands of a 16x16x16 product; U = Li z with z split into
        // high and low bf16 parts (z carries the cancellation of V - (K exp(G)) S;
        // Li in bf16 costs no measurable accuracy)
        const float4 lv = *reinterpret_cast<const float4*>(&sm.li[(16 * b + m16) * LS + 4 * q4]);
        const bf16x4 lh = cvt4(f32x4{lv.x, lv.y, lv.z, lv.w});
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          f32x4 z = Z[b][jt];
#pragma unroll
          for (int bp = 0; bp < b; ++bp) {
            const bf16x4 an = ld4(&sm.an[(16 * b + m16) * QS + 16 * bp + 4 * q4]);
            z = mfma16(an, U[bp][jt], z);
          }
          const bf16x4 zh = cvt4(z);
          const bf16x4 zl = cvt4(f32x4{z[0] - bf2f(zh[0]), z[1] - bf2f(zh[1]), z[2] - bf2f(zh[2]), z[3] - bf2f(zh[3])});
          f32x4 u = mfma16(lh, zh, f32x4{0.f, 0.f, 0.f, 0.f});
          u = mfma16(lh, zl, u);
          U[b][jt] = cvt4(u);
        }
      }
      // O^T += U^T M^T, store (rows past `valid` fall outside the descriptor).  An O0
      // block goes in the order its fix-up reads it: the 8 bytes of lane l of wave w for
      // row block rt and column tile jt at (((4 w + rt) JT + jt) 64 + l) 8, every store one
      // contiguous 512-byte run (rows past `valid` are written too; their fix-up outputs
      // are dropped)
      const bool olane = w.o_lane != 0;
      const auto orsrc = rsrc(w.o + (int64_t)it * w.ochunk, olane ? C * D * 2 : valid * w.orow * 2);
      const int ovo = olane ? lane * 8 : (m16 * w.orow + jw_base + 4 * q4) * 2;  // lane part of the offset
      const int swave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + m16;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          f32x4 o = O[rt][jt];
#pragma unroll
          for (int ks = 0; ks <= (rt >> 1); ++ks) {
            const __bf16* rowp = &sm.mm[r * QS + 32 * ks + 4 * q4];
            // M block (rt, rt + 1) is zero: its half of the k range is zero in both
            // operands (the LDS above the diagonal is never written).  The chain keeps
            // one MFMA shape: a 16x16x16 issued right behind a 16x16x32 whose result it
            // accumulates onto has given wrong sums on gfx950.
            if ((rt & 1) == 0 && ks == (rt >> 1))
              o = mfma32(cat(U[2 * ks][jt], bf16x4{}), cat(ld4(rowp), bf16x4{}), o);
            else
              o = mfma32(cat(U[2 * ks][jt], U[2 * ks + 1][jt]), ld2x4(rowp, rowp + 16), o);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) o[t] *= p.scale;  // Q exp(G) and M are unscaled
          const uint2 ov = pack4(o[0], o[1], o[2], o[3]);
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, ov), orsrc, ovo,
              olane ? ((4 * swave + rt) * JT + jt) * 512 : 16 * rt * w.orow * 2 + 32 * jt, 0);
        }
      }
      // S <- Diag(exp(G_last)) S + K'^T U
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float4 gc = *reinterpret_cast<const float4*>(&sm.gamc[16 * ct + 4 * q4]);
        const float gv[4] = {gc.x, gc.y, gc.z, gc.w};
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          f32x4 s = Sacc[ct][jt];
#pragma unroll
          for (int t = 0; t < 4; ++t) s[t] *= gv[t];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int row = 16 * ct + m16;
            const __bf16* rowp = &sm.kpt[row * CS];
            s = mfma32(ld2x4(rowp + tcol(row, 32 * ks + 4 * q4), rowp + tcol(row, 32 * ks + 16 + 4 * q4)),
                       cat(U[2 * ks][jt], U[2 * ks + 1][jt]), s);
          }
          Sacc[ct][jt] = s;
        }
      }
    }
    __syncthreads();  // (B)

    // ---- phase C: A and M tiles of the next chunk
    if (it + 1 < w.nchunks) build_tiles<64 * JT, DK>(sm, __builtin_amdgcn_readfirstlane(wave), q4, m16);
    __syncthreads();  // (C)
  }

  if (w.s1 != nullptr) {
    if (w.s1_fp32) {
      float* s1 = reinterpret_cast<float*>(w.s1);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            s1[(16 * ct + 4 * q4 + t) * DK + jw_base + 16 * jt + m16] = Sacc[ct][jt][t];
    } else {
      __bf16* s1 = reinterpret_cast<__bf16*>(w.s1);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            s1[(16 * ct + 4 * q4 + t) * DK + jw_base + 16 * jt + m16] = (__bf16)Sacc[ct][jt][t];
    }
  }
  if (w.sb != nullptr) {
    // element (k, j) at [k/32][j/16][16 ((k/8) % 4) + j % 16][k % 8] (k, j < DK): this
    // lane's rows 16ct + 4q4 .. +3 of column j are four consecutive entries
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const int k0 = 16 * ct + 4 * q4;
        const int jg = (jw_base >> 4) + jt;
        uint16_t* dst = w.sb + (((k0 >> 5) * (DK / 16) + jg) * 64 + 16 * ((k0 >> 3) & 3) + m16) * 8 + (k0 & 7);
        *reinterpret_cast<uint2*>(dst) = pack4(Sacc[ct][jt][0], Sacc[ct][jt][1], Sacc[ct][jt][2], Sacc[ct][jt][3]);
      }
  }
}

// ============================================================================ segment plan
// The recurrence is affine in the state: over any run of tokens, the end state
// is S_end = A S_start + B, where A is the product of the run's transition
// matrices (Diag(a_t) - b_t k_t (k_t * a_t)^T) and B the end state from a zero
// start [core.today "Kimi Linear 특집", ch.4 혁신 2, state-update equation].  The
// same holds for every output: o_t = scale (A_t S_start + B_t)^T q_t.  A
// sequence of c > M chunks is therefore cut into segments of M chunks (the last
// one shorter).  Segment 0 runs from the true initial state.  Every later
// segment p runs twice, in parallel with everything else: from a zero start with
// its values (outputs O0_t into a workspace, end state B_p) and from the
// identity with zero values (outputs Q~_t = scale A_t^T q_t into the output
// rows, end state A_p).  A scan S_{p+1} = A_p S_p + B_p then gives every start
// state, and the fix-up o_t = O0_t + S_p^T Q~_t completes the outputs.
//
// M is the shortest segment for which the whole job -- every chunk once, plus
// once more for each chunk past a sequence's first segment -- spread over the
// compute units takes at most 95% of M chunk-steps (kSlackNum / kSlackDen); the
// longest task then bounds the run only by that margin.  Every workgroup of
// the three kernels computes the same plan from the sequence lengths (integer
// arithmetic only).

constexpr int kNoSplit = 0x7fffffff;

__device__ __forceinline__ int64_t seq_len(const Params& p, int i) {
  return p.cu ? (int64_t)p.cu[i + 1] - p.cu[i] : p.T;
}

// The plan in LDS (ints).
struct PlanView {
  int* hdr;   // [0] M (kNoSplit: nothing split) [1] task groups [2] state slots
              // [3] split sequences [4] fix-up units of segment 1 [5] of later segments
              // [6] chunks of the longest sequence
  int* lens;  // [N]   chunks of each sequence
  int* goff;  // [N+1] first task group of each sequence
  int* soff;  // [N+1] first state slot (slot of segment p >= 1: soff + p - 1)
  int* xoff;  // [N+1] split sequences before it
  int* uoff;  // [N+1] first fix-up unit of segment 1
  int* voff;  // [N+1] first fix-up unit of the later segments
  int* tok;   // [N+1] first token of each sequence (with cu_seqlens only)
  int* glen;  // [N + 2 emax] chunks of each task group
  int* gseq;  //              its sequence
  int* gk;    //              its kind: 0 segment 0; 2p-1 zero start, 2p identity start of segment p
};

__host__ __device__ constexpr int plan_ints(int N, int emax, bool groups) {
  return 8 + N + 6 * (N + 1) + (groups ? 3 * (N + 2 * emax) : 0);
}

__device__ __forceinline__ PlanView plan_view(int* base, int N, int emax) {
  PlanView v;
  v.hdr = base;
  v.lens = base + 8;
  v.goff = v.lens + N;
  v.soff = v.goff + N + 1;
  v.xoff = v.soff + N + 1;
  v.uoff = v.xoff + N + 1;
  v.voff = v.uoff + N + 1;
  v.tok = v.voff + N + 1;
  v.glen = v.tok + N + 1;
  v.gseq = v.glen + N + 2 * emax;
  v.gk = v.gseq + N + 2 * emax;
  return v;
}

struct SeqCounts {
  int groups, slots, split, units1, units2;
};

// Task groups, state slots, split flag and fix-up units (one per chunk and
// head) of segment 1 and of the later segments, for a sequence of c chunks.
__device__ __forceinline__ SeqCounts seq_counts(int c, int M, int H) {
  SeqCounts r{1, 0, 0, 0, 0};
  if (M != kNoSplit && c > M) {
    const int P = (c + M - 1) / M;
    r.groups = 2 * P - 1;
    r.slots = P - 1;
    r.split = 1;
    r.units1 = H * min(c - M, M);
    r.units2 = H * max(c - 2 * M, 0);
  }
  return r;
}

// Builds the plan; every thread of the workgroup calls it (it holds barriers).
__device__ void build_plan(const Params& p, const PlanView& v, bool groups) {
  const int N = p.nseq, tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < N; i += nt) v.lens[i] = (int)((seq_len(p, i) + C - 1) / C);
  if (p.cu)
    for (int i = tid; i <= N; i += nt) v.tok[i] = p.cu[i];
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    int mx = 0, sum = 0;
    for (int i = lane; i < N; i += 64) {
      mx = max(mx, v.lens[i]);
      sum += v.lens[i];
    }
    mx = wave_max(mx);
    sum = wave_sum(sum);
    // fits(m): segments of m chunks balance the device, and the workspace holds
    // their state slots (emax) and fix-up output blocks (ucap); each condition
    // only gets easier as m grows
    auto fits = [&](int m) {
      int extra = 0, slots = 0;
      for (int i = lane; i < N; i += 64) {
        extra += max(0, v.lens[i] - m);
        slots += v.lens[i] > m ? (v.lens[i] - 1) / m : 0;
      }
      extra = wave_sum(extra);
      slots = wave_sum(slots);
      return (long long)kSlackDen * p.H * ((long long)sum + extra) <= (long long)kSlackNum * m * p.cus &&
             slots <= p.emax && (long long)p.H * extra <= p.ucap;
    };
    int M = kNoSplit;
    if (p.emax > 0 && mx > p.seg_min && fits(mx)) {
      int lo = p.seg_min, hi = mx;  // fits(hi)
      while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        if (fits(mid)) hi = mid;
        else lo = mid + 1;
      }
      if (hi < mx) M = hi;
    }
    // exclusive prefix sums over contiguous runs of sequences, one run per lane
    const int per = (N + 63) / 64;
    const int i0 = min(N, lane * per), i1 = min(N, i0 + per);
    int sg = 0, ss = 0, sx = 0, su = 0, sv = 0;
    for (int i = i0; i < i1; ++i) {
      const SeqCounts r = seq_counts(v.lens[i], M, p.H);
      sg += r.groups;
      ss += r.slots;
      sx += r.split;
      su += r.units1;
      sv += r.units2;
    }
    int eg = wave_incl_scan(sg) - sg, es = wave_incl_scan(ss) - ss;
    int ex = wave_incl_scan(sx) - sx, eu = wave_incl_scan(su) - su, ev = wave_incl_scan(sv) - sv;
    for (int i = i0; i < i1; ++i) {
      const SeqCounts r = seq_counts(v.lens[i], M, p.H);
      v.goff[i] = eg;
      v.soff[i] = es;
      v.xoff[i] = ex;
      v.uoff[i] = eu;
      v.voff[i] = ev;
      eg += r.groups;
      es += r.slots;
      ex += r.split;
      eu += r.units1;
      ev += r.units2;
    }
    if (lane == 63) {  // its run ends at N: the running sums are the totals
      v.goff[N] = eg;
      v.soff[N] = es;
      v.xoff[N] = ex;
      v.uoff[N] = eu;
      v.voff[N] = ev;
      v.hdr[0] = M;
      v.hdr[1] = eg;
      v.hdr[2] = es;
      v.hdr[3] = ex;
      v.hdr[4] = eu;
      v.hdr[5] = ev;
      v.hdr[6] = mx;
    }
  }
  __syncthreads();
  if (groups) {
    const int M = v.hdr[0];
    for (int i = tid; i < N; i += nt) {
      const int c = v.lens[i], g = v.goff[i];
      const bool split = M != kNoSplit && c > M;
      v.glen[g] = split ? M : c;
      v.gseq[g] = i;
      v.gk[g] = 0;
      if (split) {
        const int P = (c + M - 1) / M;
        for (int sp = 1; sp < P; ++sp) {
          const int len = min(M, c - sp * M);
#pragma unroll
          for (int kind = 0; kind < 2; ++kind) {
            const int gg = g + 2 * sp - 1 + kind;
            v.glen[gg] = len;
            v.gseq[gg] = i;
            v.gk[gg] = 2 * sp - 1 + kind;
          }
        }
      }
    }
    __syncthreads();
  }
}

// Smallest i in [0, N) with off[i + 1] > x (off non-decreasing, off[N] > x).
__device__ __forceinline__ int find_seq(const int* off, int N, int x) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (off[mid + 1] > x) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// ============================================================================ main kernel
// GS: the gate is one scalar per token and head (Gated DeltaNet), broadcast over
// the key channels as it is loaded; everything after the load is the KDA path.
template <int JT, bool GS, int DK>
__global__ void __launch_bounds__(NT, 1) kda_fwd_kernel(Params p) {
  constexpr int NV = 64 * JT;  // value columns per workgroup
  static_assert(DK == 128 || (DK == 64 && JT == 1), "head dimension 128, or 64 in one slice");
  __shared__ Smem<NV> sm;
  static_assert(plan_ints(kSortLimit, 512, true) * 4 <= 5 * sizeof(sm.kg),
                "the plan fits in the operand tiles");
  const int tid = threadIdx.x;
  // the tail kernel's publication counters start at zero
  if (blockIdx.x == 0 && p.state_flags != nullptr)
    for (int i = tid; i < p.emax * p.H; i += NT) p.state_flags[i] = 0;

  // ---- workgroup -> (task rank, head, value slice); slices of one head share an XCD
  const int nsplit = DK / NV;
  const int grp = blockIdx.x / (8 * nsplit);
  const int rem = blockIdx.x % (8 * nsplit);
  const int split = rem / 8;
  const int pidx = grp * 8 + (rem % 8);
  const int rank = pidx / p.H;
  Work w;
  w.h = pidx % p.H;
  w.j0 = split * NV;

  // ---- task of this rank: longest first (ties by sequence, then segment)
  int n = rank, kind = 0, M = kNoSplit, slot0 = 0;
  int ubase1 = 0, ubase2 = 0;  // first fix-up unit of (n, h) in segment 1 / in the later ones
  const bool planned = p.nseq <= kSortLimit && (p.emax > 0 || (p.cu != nullptr && p.nseq > 1));
  if (planned) {
    const PlanView v = plan_view(reinterpret_cast<int*>(sm.kg), p.nseq, p.emax);
    build_plan(p, v, true);
    const int G = __builtin_amdgcn_readfirstlane(v.hdr[1]);
    if (rank >= G) return;  // the same for the whole workgroup
    for (int g = tid; g < G; g += NT) {
      const int lg = v.glen[g];
      int rk = 0;
      for (int j = 0; j < G; ++j) {
        const int lj = v.glen[j];
        rk += (lj > lg) || (lj == lg && j < g);
      }
      if (rk == rank) sm.order = g;
    }
    __syncthreads();
    const int g = __builtin_amdgcn_readfirstlane(sm.order);
    n = __builtin_amdgcn_readfirstlane(v.gseq[g]);
    kind = __builtin_amdgcn_readfirstlane(v.gk[g]);
    M = __builtin_amdgcn_readfirstlane(v.hdr[0]);
    slot0 = __builtin_amdgcn_readfirstlane(v.soff[n]);
    if (kind != 0) {  // fix-up units numbered by head, then chunk (the tail kernel's order)
      const int c = __builtin_amdgcn_readfirstlane(v.lens[n]);
      ubase1 = __builtin_amdgcn_readfirstlane(v.uoff[n]) + w.h * min(c - M, M);
      ubase2 = __builtin_amdgcn_readfirstlane(v.hdr[4]) + __builtin_amdgcn_readfirstlane(v.voff[n]) +
               w.h * (c - 2 * M);
    }
    __syncthreads();  // the scratch is reused by the prep waves
  } else if (rank >= p.nseq) {
    return;
  }

  // sequence bounds, made wave-uniform so that every buffer descriptor is scalar
  int64_t bos, len;
  if (p.cu) {
    const int c0 = __builtin_amdgcn_readfirstlane(p.cu[n]);
    const int c1 = __builtin_amdgcn_readfirstlane(p.cu[n + 1]);
    bos = c0;
    len = (int64_t)c1 - c0;
  } else {
    bos = (int64_t)n * p.T;
    len = p.T;
  }
  const size_t hd2 = (size_t)w.h * (D * D);   // a state slot of the split workspace (its
                                               // first DK x DK entries used, row stride DK)
  const size_t hdk = (size_t)w.h * (DK * DK);  // the head's state in s0 / s1
  const bool seq_split = M != kNoSplit && len > (int64_t)M * C;
  if (kind == 0) {  // the sequence, or its first segment, from the true initial state
    w.bos = bos;
    w.len = seq_split ? (int64_t)M * C : len;
    w.s0_mode = p.s0 == nullptr ? 0 : p.s0_fp32 ? 2 : 1;
    w.s0 = p.s0 == nullptr ? nullptr
         : static_cast<const char*>(p.s0) + ((size_t)n * p.H * (DK * DK) + hdk) * (p.s0_fp32 ? 4 : 2);
    w.sb = nullptr;
    if (seq_split) {  // the start state of segment 1, also as the fix-up operand
      w.s1 = p.st + ((size_t)slot0 * p.H) * (D * D) + hd2;
      w.s1_fp32 = 1;
      w.sb = p.sb + ((size_t)slot0 * p.H) * (D * D) + hd2;
    } else {
      w.s1 = p.s1 == nullptr ? nullptr
           : static_cast<char*>(p.s1) + ((size_t)n * p.H * (DK * DK) + hdk) * (p.s1_fp32 ? 4 : 2);
      w.s1_fp32 = p.s1_fp32;
    }
    w.o = reinterpret_cast<__bf16*>(p.out) + w.bos * (p.H * DK) + (int64_t)w.h * DK;
    w.orow = p.H * DK;
    w.ochunk = (int64_t)C * p.H * DK;
    w.o_lane = 0;
    w.vzero = 0;
    w.ck = p.ckpt == nullptr ? nullptr : p.ckpt + ((size_t)(n + bos / C) * p.H + w.h) * (D * D);
  } else {  // segment sp >= 1 from a zero start (odd kind) or from the identity (even kind)
    const int sp = (kind + 1) >> 1;
    const bool ident = (kind & 1) == 0;
    const int64_t off = (int64_t)sp * M * C;
    w.bos = bos + off;
    w.len = len - off < (int64_t)M * C ? len - off : (int64_t)M * C;
    w.s0_mode = ident ? 3 : 0;
    w.s0 = nullptr;
    w.s1 = p.st + ((size_t)((ident ? 1 : 2) * p.emax + slot0 + sp - 1) * p.H) * (D * D) + hd2;
    w.s1_fp32 = 1;
    if (ident) {  // Q~ into the output rows
      w.o = reinterpret_cast<__bf16*>(p.out) + w.bos * (p.H * DK) + (int64_t)w.h * DK;
      w.orow = p.H * DK;
      w.ochunk = (int64_t)C * p.H * DK;
      w.o_lane = 0;
    } else {      // O0 into the fix-up blocks of its units, one 64 x 128 block per chunk
                  // (its first DK columns used)
      const int ub = sp == 1 ? ubase1 : ubase2 + (sp - 2) * M;
      w.o = reinterpret_cast<__bf16*>(p.o0) + (int64_t)ub * (C * D);
      w.orow = D;
      w.ochunk = (int64_t)C * D;
      w.o_lane = 1;
    }
    w.ck = nullptr;
    w.vzero = ident ? 1 : 0;
    w.sb = nullptr;
  }
  w.nchunks = (int)((w.len + C - 1) / C);

  // Both roles execute the same barrier sequence; the branch is uniform per wave.
  if (__builtin_amdgcn_readfirstlane(tid >> 6) < 4) state_loop<JT, DK>(sm, p, w);
  else prep_loop<NV, GS, DK>(sm, p, w);
}

}  // namespace
}  // namespace kda
