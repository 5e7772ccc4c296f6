// Launch of the fused chunkwise KDA forward kernel (per-channel gate) and of the
// scan / fix-up kernel that finishes sequences split into affine segments.  The
// fused kernel itself is in kda_fwd_core.h.
//
// The scalar-gate variant is instantiated in kda_gdn_kernel.hip, a translation
// unit of its own: with both variants in one module the compiler's inlining and
// register allocation for the per-channel kernel changed (256 VGPRs with spills
// instead of 252 without), which cost about a tenth of its throughput.
#include "kda_fwd_core.h"

namespace kda {
namespace {

// ============================================================================ scan and fix-up
// Two launches follow the main kernel when sequences were split.
//  * phase 0: the scan, one unit per (split sequence, head, 16-column block of
//    the state): S_1 is segment 0's end state; for p = 1 .. P-1 it forms
//    S_{p+1} = A_p S_p + B_p in fp32 and stores the bf16 operand copy of S_p for
//    p >= 2 (segment 0's task stored that of S_1); S_P is the final state.  The
//    same launch fixes up the outputs of segment 1, which need only S_1.
//  * phase 1: the output fix-up of the later segments.
// A fix-up unit is one chunk of one (sequence, head): o_t = O0_t + S_p^T Q~_t,
// with Q~ read from (and o written back to) the output rows.  Every load of a
// unit is issued at its start.  Wave w forms output columns 32w..32w+31 as
// O^T = S_p^T Q~^T on bf16 MFMA 16x16x32; Q~ is staged through LDS so that each
// wave reads all 64 tokens.  The plan lives in dynamic LDS (plan_ints(N, 0,
// false) ints); every launch walks its units in a grid-stride loop.
constexpr int TAIL_NT = 256;
constexpr int SLT = D + 4;  // row stride (fp32) of the scan's state block, stored transposed

__device__ __forceinline__ void split_hilo(const float* f, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (__bf16)f[e];
    lo[e] = (__bf16)(f[e] - bf2f(hi[e]));
  }
}

// One scan unit: columns 16cb .. 16cb+15 of the states of split sequence
// `sidx`, head h.  The block lives transposed in LDS, slt[j][k].  A_p S_p runs on
// bf16 16x16x32 products of high and low parts (the low-by-low term dropped);
// wave w forms rows 32w .. 32w+31.
__device__ __forceinline__ void scan_unit(const Params& p, const PlanView& v, int M, int u, float* slt) {
  const int N = p.nseq, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, m16 = lane & 15;
  const size_t slot_stride = (size_t)p.H * (D * D);
  // u = (split sequence * 8 + column block) * H + head: the eight column blocks of one
  // (sequence, head), which all read the same A_p, land on one XCD when 8 divides H
  // (workgroups go to XCDs round robin)
  const int sidx = u / (p.H * 8), cb = (u / p.H) % 8, h = u % p.H;
  const int i = __builtin_amdgcn_readfirstlane(find_seq(v.xoff, N, sidx));
  const int c = __builtin_amdgcn_readfirstlane(v.lens[i]), P = (c + M - 1) / M;
  const int slot0 = __builtin_amdgcn_readfirstlane(v.soff[i]);
  const size_t hd2 = (size_t)h * (D * D);
  {  // S_1 (row-major in the workspace) -> slt
    const float* s1 = p.st + slot0 * slot_stride + hd2 + 16 * cb;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int k = 16 * x + (tid >> 4), j = tid & 15;
      slt[j * SLT + k] = s1[(size_t)k * D + j];
    }
  }
  __syncthreads();
  for (int sp = 1; sp < P; ++sp) {
    const int slot = slot0 + sp - 1;
    // rows 32w + 16it + m16 of A_p (k = 32ks + 8q4 .. +7) and the matching
    // entries of B_p, all loads in flight before the products
    const float* am = p.st + ((size_t)p.emax + slot) * slot_stride + hd2;
    const float* bm = p.st + ((size_t)2 * p.emax + slot) * slot_stride + hd2 + 16 * cb + m16;
    float4 ar[2][4][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float* rp = am + (size_t)(32 * wave + 16 * it + m16) * D + 32 * ks + 8 * q4;
        ar[it][ks][0] = *reinterpret_cast<const float4*>(rp);
        ar[it][ks][1] = *reinterpret_cast<const float4*>(rp + 4);
      }
    f32x4 acc[2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[it][t] = bm[(size_t)(32 * wave + 16 * it + 4 * q4 + t) * D];
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the products
    if (sp >= 2) {  // fix-up operand copy of S_p: element (k, j) at [k/32][j/16][16 ((k/8)%4) + j%16][k%8]
      const int ks = tid >> 6;
      const float4 f0 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4]);
      const float4 f1 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4 + 4]);
      const uint2 lo = pack4(f0.x, f0.y, f0.z, f0.w), hi = pack4(f1.x, f1.y, f1.z, f1.w);
      uint16_t* dst = p.sb + slot * slot_stride + hd2 + ((ks * 8 + cb) * 64 + lane) * 8;
      *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // B operand: S_p[32ks + 8q4 + e][m16] = slt[m16][32ks + 8q4 + e]
      const float4 g0 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4]);
      const float4 g1 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4 + 4]);
      const float sf[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      bf16x8 sh, sl;
      split_hilo(sf, sh, sl);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const float af[8] = {ar[it][ks][0].x, ar[it][ks][0].y, ar[it][ks][0].z, ar[it][ks][0].w,
                             ar[it][ks][1].x, ar[it][ks][1].y, ar[it][ks][1].z, ar[it][ks][1].w};
        bf16x8 ah, al;
        split_hilo(af, ah, al);
        acc[it] = mfma32(ah, sh, acc[it]);
        acc[it] = mfma32(ah, sl, acc[it]);
        acc[it] = mfma32(al, sh, acc[it]);
      }
    }
    __syncthreads();  // every read of S_p is done
    // lane holds S_{p+1}[32w + 16it + 4q4 + t][m16]: four consecutive entries of slt row m16
#pragma unroll
    for (int it = 0; it < 2; ++it)
      *reinterpret_cast<float4*>(&slt[m16 * SLT + 32 * wave + 16 * it + 4 * q4]) =
          make_float4(acc[it][0], acc[it][1], acc[it][2], acc[it][3]);
    __syncthreads();
  }
  if (p.s1 != nullptr) {
    const size_t base = ((size_t)i * p.H) * (D * D) + hd2 + 16 * cb;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int k = 16 * x + (tid >> 4), j = tid & 15;
      const float val = slt[j * SLT + k];
      if (p.s1_fp32) static_cast<float*>(p.s1)[base + (size_t)k * D + j] = val;
      else static_cast<__bf16*>(p.s1)[base + (size_t)k * D + j] = (__bf16)val;
    }
  }
  __syncthreads();  // before the next unit overwrites the block
}

// Fix-up units: one per (sequence, head, chunk past the first segment), numbered
// within a sequence by head, then chunk, so that consecutive units share the
// segment start state S_p.  Segment-1 units (seg0 = 1) cover chunks M ..
// M + min(c - M, M) - 1, later-segment units (seg0 = 2) chunks 2M .. c - 1.
struct FixUnit {
  int i, h, ch, slot, valid;
  int64_t tok0;
};

__device__ __forceinline__ FixUnit fix_decode(const Params& p, const PlanView& v, int M, const int* off,
                                              int seg0, int u) {
  FixUnit f;
  f.i = __builtin_amdgcn_readfirstlane(find_seq(off, p.nseq, u));
  const int r = u - __builtin_amdgcn_readfirstlane(off[f.i]);
  const int c = __builtin_amdgcn_readfirstlane(v.lens[f.i]);
  const int n = seg0 == 1 ? min(c - M, M) : c - 2 * M;  // chunks per head in this range
  f.h = r / n;
  f.ch = seg0 * M + r % n;
  f.slot = __builtin_amdgcn_readfirstlane(v.soff[f.i]) + f.ch / M - 1;
  int64_t bos, len;
  if (p.cu) {  // from the plan in LDS: no global load on the unit's critical path
    const int c0 = __builtin_amdgcn_readfirstlane(v.tok[f.i]);
    const int c1 = __builtin_amdgcn_readfirstlane(v.tok[f.i + 1]);
    bos = c0;
    len = (int64_t)c1 - c0;
  } else {
    bos = (int64_t)f.i * p.T;
    len = p.T;
  }
  f.tok0 = bos + (int64_t)f.ch * C;
  const int64_t rest = len - (int64_t)f.ch * C;
  f.valid = rest < C ? (int)rest : C;
  return f;
}

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Q~ rows of the unit's chunk (rows past `valid` read as zero) and its O0 entries.
struct FixLoads {
  u32x4 qv[4];
  u32x2 zv[4][2];
};

__device__ __forceinline__ void fix_issue(const Params& p, const FixUnit& f, FixLoads& L) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, m16 = lane & 15;
  const int HD = p.H * D;
  const auto orsrc = rsrc(p.out + f.tok0 * HD + (int64_t)f.h * D, f.valid * HD * 2);
  const auto zrsrc = rsrc(p.o0 + f.tok0 * HD + (int64_t)f.h * D, f.valid * HD * 2);
#pragma unroll
  for (int x = 0; x < 4; ++x)
    L.qv[x] = __builtin_amdgcn_raw_buffer_load_b128(orsrc, ((16 * x + (tid >> 4)) * HD + 8 * (tid & 15)) * 2, 0, 0);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      L.zv[tt][jj] = __builtin_amdgcn_raw_buffer_load_b64(
          zrsrc, ((16 * tt + m16) * HD + 16 * (2 * wave + jj) + 4 * q4) * 2, 0, 0);
}

// S_p^T as the products' A operand (bf16, the order the segment's first run wrote).
__device__ __forceinline__ void fix_state(const Params& p, const FixUnit& f, bf16x8 (&sa)[4][2]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const __bf16* sbp = reinterpret_cast<const __bf16*>(p.sb) + ((size_t)f.slot * p.H + f.h) * (D * D);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      sa[ks][jj] = *reinterpret_cast<const bf16x8*>(sbp + ((ks * 8 + 2 * wave + jj) * 64 + lane) * 8);
}

// This workgroup's contiguous share of `units` fix-up units, spread over the
// workgroups first .. gridDim.x - 1: o = O0 + S_p^T Q~ for every row of each
// unit's chunk.  The next unit's loads are in flight while the current one is
// multiplied; S_p is reloaded only when the segment or head changes.
__device__ void fix_range(const Params& p, const PlanView& v, int M, const int* off, int seg0, int units,
                          __bf16* ot, int first) {
  const int G = gridDim.x - first, b = blockIdx.x - first;
  const int u_lo = (int)((int64_t)units * b / G), u_hi = (int)((int64_t)units * (b + 1) / G);
  if (u_lo >= u_hi) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, m16 = lane & 15;
  const int HD = p.H * D;
  FixUnit cur = fix_decode(p, v, M, off, seg0, u_lo);
  FixLoads L;
  fix_issue(p, cur, L);
  bf16x8 sa[4][2];
  fix_state(p, cur, sa);
  for (int u = u_lo; u < u_hi; ++u) {
    // stage Q~ of the current unit (its B operand order) in LDS
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      uint2* dst = reinterpret_cast<uint2*>(&ot[(16 * x + (tid >> 4)) * TS + 8 * (tid & 15)]);
      dst[0] = make_uint2(L.qv[x][0], L.qv[x][1]);
      dst[1] = make_uint2(L.qv[x][2], L.qv[x][3]);
    }
    f32x4 z[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float f[4];
        unpack4(make_uint2(L.zv[tt][jj][0], L.zv[tt][jj][1]), f);
        z[tt][jj] = f32x4{f[0], f[1], f[2], f[3]};
      }
    const FixUnit f = cur;
    const bool more = u + 1 < u_hi;
    if (more) {
      cur = fix_decode(p, v, M, off, seg0, u + 1);
      fix_issue(p, cur, L);  // the next unit's loads fly during this unit's products
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const __bf16* bp = &ot[(16 * tt + m16) * TS + 32 * ks + 8 * q4];
        const bf16x8 bb = ld2x4(bp, bp + 4);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) z[tt][jj] = mfma32(sa[ks][jj], bb, z[tt][jj]);
      }
    }
    // lane holds o[token 16tt + m16][columns 16jt + 4q4 .. +3], jt = 2 wave + jj
    const auto orsrc = rsrc(p.out + f.tok0 * HD + (int64_t)f.h * D, f.valid * HD * 2);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint2 ov = pack4(z[tt][jj][0], z[tt][jj][1], z[tt][jj][2], z[tt][jj][3]);
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(u32x2, ov), orsrc,
            ((16 * tt + m16) * HD + 16 * (2 * wave + jj) + 4 * q4) * 2, 0, 0);
      }
    if (more && (cur.slot != f.slot || cur.h != f.h)) fix_state(p, cur, sa);
    __syncthreads();  // before the next unit's staging
  }
}

__global__ void __launch_bounds__(TAIL_NT, 3) kda_tail_kernel(Params p, int phase) {
  extern __shared__ int plan_lds[];
  __shared__ __attribute__((aligned(16))) float slt[16 * SLT];
  __shared__ __attribute__((aligned(16))) __bf16 ot[C * TS];
  const int N = p.nseq;
  const PlanView v = plan_view(plan_lds, N, 0);
  build_plan(p, v, false);
  // wave-uniform unit values keep every buffer descriptor scalar
  const int M = __builtin_amdgcn_readfirstlane(v.hdr[0]);
  if (M == kNoSplit) return;
  if (phase == 0) {
    // scan units spread over the grid, then every workgroup's share of the
    // segment-1 fix-ups (they need only S_1, written by the main kernel)
    const int nscan = __builtin_amdgcn_readfirstlane(v.hdr[3]) * p.H * 8;
    for (int u = blockIdx.x; u < nscan; u += gridDim.x) scan_unit(p, v, M, u, slt);
    // with workgroups to spare, the fix-ups go to those without a scan unit and run
    // beside the scan instead of after it
    const int first = nscan < (int)gridDim.x ? nscan : 0;
    if ((int)blockIdx.x >= first)
      fix_range(p, v, M, v.uoff, 1, __builtin_amdgcn_readfirstlane(v.hdr[4]), ot, first);
  } else {
    fix_range(p, v, M, v.voff, 2, __builtin_amdgcn_readfirstlane(v.hdr[5]), ot, 0);
  }
}

}  // namespace

int workspace_slots(int cus, int H) { return (H > 0 && H < cus) ? cus / H + 1 : 0; }

WorkspaceLayout workspace_layout(int64_t rows, int H, int emax) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout l;
  l.o0 = 0;
  l.st = up((size_t)rows * H * D * 2);
  l.sb = l.st + up((size_t)3 * emax * H * D * D * 4);
  l.total = l.sb + up((size_t)emax * H * D * D * 2);
  return l;
}

hipError_t launch_fwd(const Params& p, int nsplit, hipStream_t stream) {
  if (nsplit != 1 && nsplit != 2) return hipErrorInvalidValue;
  if (p.emax > 0 && (nsplit != 1 || p.o0 == nullptr || p.st == nullptr || p.sb == nullptr))
    return hipErrorInvalidValue;
  // task groups: every sequence, plus two runs per extra segment (fewer than
  // 2 * emax of them when splitting)
  const int64_t groups = (int64_t)p.nseq + (p.emax > 0 && p.nseq <= kSortLimit ? 2 * (int64_t)p.emax : 0);
  const int64_t wgs = (groups * p.H + 7) / 8 * 8 * nsplit;
  const dim3 block(NT);
  hipError_t err;
  if (p.g_scalar) {
    err = launch_fwd_main_scalar_gate(p, nsplit, (unsigned)wgs, stream);
  } else {
    if (nsplit == 1) hipLaunchKernelGGL((kda_fwd_kernel<2, false>), dim3((unsigned)wgs), block, 0, stream, p);
    else hipLaunchKernelGGL((kda_fwd_kernel<1, false>), dim3((unsigned)wgs), block, 0, stream, p);
    err = hipGetLastError();
  }
  if (err != hipSuccess || p.emax == 0 || p.nseq > kSortLimit) return err;
  const size_t plan_bytes = (size_t)plan_ints(p.nseq, 0, false) * sizeof(int);
  hipLaunchKernelGGL(kda_tail_kernel, dim3(3 * p.cus), dim3(TAIL_NT), plan_bytes, stream, p, 0);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kda_tail_kernel, dim3(3 * p.cus), dim3(TAIL_NT), plan_bytes, stream, p, 1);
  return hipGetLastError();
}

}  // namespace kda
