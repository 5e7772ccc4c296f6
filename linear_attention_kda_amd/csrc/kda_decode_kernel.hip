// Recurrent KDA decode step for gfx950 (MI355X): one token per sequence.
//
// Per sequence n and head h, with the D x D state S (S[i][j]: i key channel,
// j value channel) [core.today "Kimi Linear 특집", ch.4 혁신 2, state-update
// equation; ch.4 혁신 1, channel-wise gate; ch.2, readout]:
//   S~  = Diag(exp(g)) S                      (decay first)
//   e   = v - S~^T k                          (delta-rule error, per value column)
//   S'  = S~ + beta k e^T                     (rank-1 write)
//   o   = scale S'^T q = scale (S~^T q + beta (k . q) e)
// The state is the only sizeable operand (64 KiB fp32 per head at D = 128), so
// the step is bound by reading and writing it once; the fixed state size is why
// decoding cost does not grow with the context [same page, decoding-speed
// comparison].
//
// Mapping: one workgroup per (sequence, head) at D = 64 and 128, two (128 value
// columns each; columns never mix) at D = 256.  With NC columns per workgroup,
// thread t owns value columns 4 (t % (NC/4)) .. +3 and key rows t / (NC/4) + RG r,
// RG = threads / (NC/4) row groups: every state row slice is read by NC/4
// consecutive threads as one contiguous run.  D = 128: 512 threads, 16 row groups
// of 8 rows; D = 64: 256 threads, 16 groups of 4 rows; D = 256: 1024 threads, 32
// groups of 8 rows.  Eight rows of four columns per thread (32 state values) kept
// the most loads in flight: at D = 128 it reached 77% of HBM bandwidth against 70%
// with 256 threads of 16 rows.  The two column dot products (S~^T k, S~^T q) are summed over
// the row groups in LDS; the state stays in registers between its load and its
// store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((ext_vector_type(4))) float v4f;
typedef __attribute__((ext_vector_type(2))) unsigned v2u;

template <int D>
struct Dec {
  static constexpr int nt = D == 256 ? 1024 : D == 128 ? 512 : 256;   // threads per workgroup
  static constexpr int cs = D == 256 ? 2 : 1;         // workgroups per (sequence, head), by columns
  static constexpr int nc = D / cs;                   // value columns per workgroup
  static constexpr int cg = nc / 4;                   // column groups of 4
  static constexpr int rg = nt / cg;                  // row groups
  static constexpr int rpt = D / rg;                  // rows per thread
};
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float bf2f_u16(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// GS: one gate per token and head (Gated DeltaNet), the same decay for every
// key channel [core.today "Kimi Linear 특집", ch.4 혁신 1].
template <int D, bool F32, bool GS>
__global__ void __launch_bounds__(Dec<D>::nt) kda_decode_kernel(DecodeParams p) {
  constexpr int CG = Dec<D>::cg, RG = Dec<D>::rg, RPT = Dec<D>::rpt, NC = Dec<D>::nc;
  __shared__ float vk[D], vq[D], va[D];   // k, q and exp(g) of the token
  __shared__ float part[2][RG][NC];       // per row group: partial S~^T k and S~^T q
  __shared__ float kq_part[D / 64];

  const int pair = blockIdx.x / Dec<D>::cs;
  const int c0 = (blockIdx.x % Dec<D>::cs) * NC;   // first value column of this workgroup
  const int n = pair / p.H, h = pair % p.H;
  const int slot = p.idx != nullptr ? __builtin_amdgcn_readfirstlane(p.idx[n]) : n;
  if (slot < 0) return;  // padding entry: no state, no output (the same for the whole workgroup)
  const int t = threadIdx.x, cb = t % CG, rg = t / CG;
  const size_t tok = (size_t)n * p.H + h;

  // stage the token's vectors; k . q by the first D / 64 waves
  if (t < D) {
    const float kf = bf2f_u16(p.k[tok * D + t]);
    const float qf = bf2f_u16(p.q[tok * D + t]);
    vk[t] = kf;
    vq[t] = qf;
    va[t] = __builtin_amdgcn_exp2f((GS ? p.g[tok] : p.g[tok * D + t]) * LOG2E);
    float s = kf * qf;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((t & 63) == 0) kq_part[t >> 6] = s;
  }
  // this thread's RPT rows of its 4 columns
  const size_t sbase = ((size_t)slot * p.H + h) * (size_t)(D * D) + c0 + 4 * cb;
  float4 srow[RPT];
  if constexpr (F32) {
    const float* s = static_cast<const float*>(p.state) + sbase;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      // the state is touched once per step: nontemporal loads and stores
      const v4f t4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(s + (size_t)(rg + RG * r) * D));
      srow[r] = make_float4(t4[0], t4[1], t4[2], t4[3]);
    }
  } else {
    const uint16_t* s = static_cast<const uint16_t*>(p.state) + sbase;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const v2u u = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(s + (size_t)(rg + RG * r) * D));
      srow[r] = make_float4(__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                            __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u));
    }
  }
  __syncthreads();

  // decay and the partial dot products over this thread's rows
  float dk[4] = {0.f, 0.f, 0.f, 0.f}, dq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg + RG * r;
    const float a = va[i], ki = vk[i], qi = vq[i];
    srow[r].x *= a; srow[r].y *= a; srow[r].z *= a; srow[r].w *= a;
    dk[0] += srow[r].x * ki; dk[1] += srow[r].y * ki; dk[2] += srow[r].z * ki; dk[3] += srow[r].w * ki;
    dq[0] += srow[r].x * qi; dq[1] += srow[r].y * qi; dq[2] += srow[r].z * qi; dq[3] += srow[r].w * qi;
  }
  *reinterpret_cast<float4*>(&part[0][rg][4 * cb]) = make_float4(dk[0], dk[1], dk[2], dk[3]);
  *reinterpret_cast<float4*>(&part[1][rg][4 * cb]) = make_float4(dq[0], dq[1], dq[2], dq[3]);
  __syncthreads();

  // column sums, error and output for this thread's 4 columns
  float sk[4] = {0.f, 0.f, 0.f, 0.f}, sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g8 = 0; g8 < RG; ++g8) {
    const float4 a = *reinterpret_cast<const float4*>(&part[0][g8][4 * cb]);
    const float4 b = *reinterpret_cast<const float4*>(&part[1][g8][4 * cb]);
    sk[0] += a.x; sk[1] += a.y; sk[2] += a.z; sk[3] += a.w;
    sq[0] += b.x; sq[1] += b.y; sq[2] += b.z; sq[3] += b.w;
  }
  const float beta = p.beta[tok];
  float kq = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) kq += kq_part[w];
  float be[4];
  {
    const uint2 vu = *reinterpret_cast<const uint2*>(p.v + tok * D + c0 + 4 * cb);
    const float vv[4] = {__uint_as_float(vu.x << 16), __uint_as_float(vu.x & 0xffff0000u),
                         __uint_as_float(vu.y << 16), __uint_as_float(vu.y & 0xffff0000u)};
    float o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      be[c] = beta * (vv[c] - sk[c]);
      o[c] = p.scale * (sq[c] + kq * be[c]);
    }
    if (rg == 0)
      *reinterpret_cast<uint2*>(p.out + tok * D + c0 + 4 * cb) = make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
  }

  // S' = S~ + k (beta e)^T, stored in place
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float ki = vk[rg + RG * r];
    srow[r].x += ki * be[0]; srow[r].y += ki * be[1]; srow[r].z += ki * be[2]; srow[r].w += ki * be[3];
  }
  if constexpr (F32) {
    float* s = static_cast<float*>(p.state) + sbase;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      __builtin_nontemporal_store(v4f{srow[r].x, srow[r].y, srow[r].z, srow[r].w},
                                  reinterpret_cast<v4f*>(s + (size_t)(rg + RG * r) * D));
  } else {
    uint16_t* s = static_cast<uint16_t*>(p.state) + sbase;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      __builtin_nontemporal_store(v2u{pack2_bf16(srow[r].x, srow[r].y), pack2_bf16(srow[r].z, srow[r].w)},
                                  reinterpret_cast<v2u*>(s + (size_t)(rg + RG * r) * D));
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.nseq * p.H * Dec<D>::cs)), block(Dec<D>::nt);
  if (p.g_scalar) {
    if (p.state_fp32) hipLaunchKernelGGL((kda_decode_kernel<D, true, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((kda_decode_kernel<D, false, true>), grid, block, 0, stream, p);
  } else {
    if (p.state_fp32) hipLaunchKernelGGL((kda_decode_kernel<D, true, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((kda_decode_kernel<D, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.D == 128) return launch_decode_d<128>(p, stream);
  if (p.D == 64) return launch_decode_d<64>(p, stream);
  if (p.D == 256) return launch_decode_d<256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
