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
// One launch follows the main kernel when sequences were split.
//  * Scan units, one per (split sequence, head, 16-column block of the state), in
//    the first workgroups: S_1 is segment 0's end state; for p = 1 .. P-1 a unit
//    forms S_{p+1} = A_p S_p + B_p in fp32, and in step p >= 2 it stores the bf16
//    fix-up operand of S_p and then publishes it (below); S_P is the final state.
//  * Fix-up units: one chunk of one (sequence, head), o_t = O0_t + S_p^T Q~_t,
//    with Q~ read from (and o written back to) the output rows.  Units of segment
//    1 need only S_1, which the main kernel stored; a unit of a later segment
//    first waits until every column block of its S_p has been published.
// Publication: the scan's stores of the operand copy are device-scope (sc1, written
// through to the point of coherence of all XCDs), every wave waits for its stores
// to complete, and after a barrier one thread adds 1 to the (slot, head) counter
// with a device-scope atomic.  A waiting workgroup polls the counter with
// device-scope loads until it reaches the number of column blocks, then reads the
// copy with device-scope loads, so no XCD's L2 can serve it stale.  The counters
// are zeroed by the main kernel.  Scan units never wait, and they occupy the
// lowest workgroup indices, which are dispatched first, so a waiting workgroup
// never holds back the work it waits for; the wait is bounded all the same.
// Every load of a fix-up unit is issued at its start.  Wave w forms output columns
// 32w..32w+31 as O^T = S_p^T Q~^T on bf16 MFMA 16x16x32; Q~ is staged through LDS
// so that each wave reads all 64 tokens.  The plan lives in dynamic LDS
// (plan_ints(N, 0, false) ints).
constexpr int TAIL_NT = 256;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
// cache policy of a buffer access: device scope (sc1), coherent across the XCDs
constexpr int kDeviceScope = 16;
// polls of a publication counter before a wait gives up (~1-2 s): reached only if the
// scan never published, which would be a defect; the unit then runs on whatever the
// operand holds instead of hanging the device
constexpr int kWaitPolls = 1 << 20;
constexpr int SLT = D + 4;  // row stride (fp32) of the scan's state block, stored transposed

__device__ __forceinline__ void split_hilo(const float* f, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (__bf16)f[e];
    lo[e] = (__bf16)(f[e] - bf2f(hi[e]));
  }
}

// One scan unit: columns 16cb .. 16cb+15 of the states of split sequence
// `sidx`, head h, at head dimension DK (the states are DK x DK with row stride
// DK, in slots of 128 x 128).  The block lives transposed in LDS, slt[j][k].
// A_p S_p runs on bf16 16x16x32 products of high and low parts (the low-by-low
// term dropped); wave w forms rows DK/4 w .. DK/4 w + DK/4 - 1.
template <int DK>
__device__ __forceinline__ void scan_unit(const Params& p, const PlanView& v, int M, int u, float* slt) {
  constexpr int NB = DK / 16;   // 16-column blocks of a state
  constexpr int KS = DK / 32;   // 32-row slices of the product's k range
  constexpr int IT = DK / 64;   // 16-row tiles per wave
  const int N = p.nseq, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, m16 = lane & 15;
  const size_t slot_stride = (size_t)p.H * (D * D);
  // u = (split sequence * NB + column block) * H + head: the column blocks of one
  // (sequence, head), which all read the same A_p, land on one XCD when 8 divides H
  // (workgroups go to XCDs round robin)
  const int sidx = u / (p.H * NB), cb = (u / p.H) % NB, h = u % p.H;
  const int i = __builtin_amdgcn_readfirstlane(find_seq(v.xoff, N, sidx));
  const int c = __builtin_amdgcn_readfirstlane(v.lens[i]), P = (c + M - 1) / M;
  const int slot0 = __builtin_amdgcn_readfirstlane(v.soff[i]);
  const size_t hd2 = (size_t)h * (D * D);
  {  // S_1 (row-major in the workspace) -> slt
    const float* s1 = p.st + slot0 * slot_stride + hd2 + 16 * cb;
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int k = 16 * x + (tid >> 4), j = tid & 15;
      slt[j * SLT + k] = s1[(size_t)k * DK + j];
    }
  }
  __syncthreads();
  for (int sp = 1; sp < P; ++sp) {
    const int slot = slot0 + sp - 1;
    // rows DK/4 w + 16it + m16 of A_p (k = 32ks + 8q4 .. +7) and the matching
    // entries of B_p, all loads in flight before the products
    const float* am = p.st + ((size_t)p.emax + slot) * slot_stride + hd2;
    const float* bm = p.st + ((size_t)2 * p.emax + slot) * slot_stride + hd2 + 16 * cb + m16;
    const int row0 = (DK / 4) * wave;
    float4 ar[IT][KS][2];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float* rp = am + (size_t)(row0 + 16 * it + m16) * DK + 32 * ks + 8 * q4;
        ar[it][ks][0] = *reinterpret_cast<const float4*>(rp);
        ar[it][ks][1] = *reinterpret_cast<const float4*>(rp + 4);
      }
    f32x4 acc[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[it][t] = bm[(size_t)(row0 + 16 * it + 4 * q4 + t) * DK];
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the products
    // fix-up operand copy of S_p: element (k, j) at [k/32][j/16][16 ((k/8)%4) + j%16][k%8],
    // one 32-row slice per wave
    if (sp >= 2 && wave < KS) {  // device-scope stores: published after the products
      const int ks = wave;
      const float4 f0 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4]);
      const float4 f1 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4 + 4]);
      const uint2 lo = pack4(f0.x, f0.y, f0.z, f0.w), hi = pack4(f1.x, f1.y, f1.z, f1.w);
      const auto srs = rsrc(p.sb + slot * slot_stride + hd2, D * D * 2);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{lo.x, lo.y, hi.x, hi.y}, srs,
                                             ((ks * NB + cb) * 64 + lane) * 16, 0, kDeviceScope);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // B operand: S_p[32ks + 8q4 + e][m16] = slt[m16][32ks + 8q4 + e]
      const float4 g0 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4]);
      const float4 g1 = *reinterpret_cast<const float4*>(&slt[m16 * SLT + 32 * ks + 8 * q4 + 4]);
      const float sf[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      bf16x8 sh, sl;
      split_hilo(sf, sh, sl);
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const float af[8] = {ar[it][ks][0].x, ar[it][ks][0].y, ar[it][ks][0].z, ar[it][ks][0].w,
                             ar[it][ks][1].x, ar[it][ks][1].y, ar[it][ks][1].z, ar[it][ks][1].w};
        bf16x8 ah, al;
        split_hilo(af, ah, al);
        acc[it] = mfma32(ah, sh, acc[it]);
        acc[it] = mfma32(ah, sl, acc[it]);
        acc[it] = mfma32(al, sh, acc[it]);
      }
    }
    if (sp >= 2) __builtin_amdgcn_s_waitcnt(0);  // this wave's copy stores have completed
    __syncthreads();  // every read of S_p is done
    if (sp >= 2 && tid == 0)  // publish the copy of S_p (column block cb)
      __hip_atomic_fetch_add(p.state_flags + (size_t)slot * p.H + h, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    // lane holds S_{p+1}[row0 + 16it + 4q4 + t][m16]: four consecutive entries of slt row m16
#pragma unroll
    for (int it = 0; it < IT; ++it)
      *reinterpret_cast<float4*>(&slt[m16 * SLT + row0 + 16 * it + 4 * q4]) =
          make_float4(acc[it][0], acc[it][1], acc[it][2], acc[it][3]);
    __syncthreads();
  }
  if (p.s1 != nullptr) {
    const size_t base = ((size_t)i * p.H + h) * (DK * DK) + 16 * cb;
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int k = 16 * x + (tid >> 4), j = tid & 15;
      const float val = slt[j * SLT + k];
      if (p.s1_fp32) static_cast<float*>(p.s1)[base + (size_t)k * DK + j] = val;
      else static_cast<__bf16*>(p.s1)[base + (size_t)k * DK + j] = (__bf16)val;
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
  int ob;          // the unit's O0 block: units of segment 1 first, then the later ones
  int64_t tok0;
};

__device__ __forceinline__ FixUnit fix_decode(const Params& p, const PlanView& v, int M, const int* off,
                                              int seg0, int u) {
  FixUnit f;
  f.i = __builtin_amdgcn_readfirstlane(find_seq(off, p.nseq, u));
  f.ob = seg0 == 1 ? u : __builtin_amdgcn_readfirstlane(v.hdr[4]) + u;
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


// At head dimension DK: a row of Q~ is DK/8 loads of 16 bytes, so 2048/DK rows go
// in one pass of the 256 threads; wave w forms output columns DK/4 w .. + DK/4 - 1
// (JJ = DK/64 tiles of 16).
template <int DK>
struct FixShape {
  static constexpr int TPR = DK / 8;        // threads per Q~ row
  static constexpr int RPS = TAIL_NT / TPR;  // Q~ rows per pass
  static constexpr int QP = C / RPS;        // passes over the chunk's 64 rows
  static constexpr int JJ = DK / 64;        // 16-column output tiles per wave
  static constexpr int KS = DK / 32;        // 32-channel slices of the products
  static constexpr int NB = DK / 16;        // 16-column blocks of a state
};

// Q~ rows of the unit's chunk (rows past `valid` read as zero) and its O0 entries.
template <int DK>
struct FixLoads {
  u32x4 qv[FixShape<DK>::QP];
  u32x2 zv[4][FixShape<DK>::JJ];
};

template <int DK>
__device__ __forceinline__ void fix_issue(const Params& p, const FixUnit& f, FixLoads<DK>& L) {
  using F = FixShape<DK>;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int HD = p.H * DK;
  const auto orsrc = rsrc(p.out + f.tok0 * HD + (int64_t)f.h * DK, f.valid * HD * 2);
  // the O0 block in the order the main kernel stored it: lane l of wave w reads rows
  // 16 tt + m16, columns 16 (JJ w + jj) + 4 q4 .. +3 from (((4 w + tt) JJ + jj) 64 + l) 8
  const auto zrsrc = rsrc(p.o0 + (int64_t)f.ob * (C * D), C * D * 2);
#pragma unroll
  for (int x = 0; x < F::QP; ++x)
    L.qv[x] = __builtin_amdgcn_raw_buffer_load_b128(
        orsrc, ((F::RPS * x + tid / F::TPR) * HD + 8 * (tid % F::TPR)) * 2, 0, 0);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int jj = 0; jj < F::JJ; ++jj)
      L.zv[tt][jj] = __builtin_amdgcn_raw_buffer_load_b64(
          zrsrc, lane * 8, ((4 * wave + tt) * F::JJ + jj) * 512, 0);
}

// S_p^T as the products' A operand (bf16, the order the segment's first run or the
// scan wrote).  LATER: a state the scan published in this launch, read at device scope
// once its counter is full.
template <int DK, bool LATER>
__device__ __forceinline__ void fix_state(const Params& p, const FixUnit& f,
                                          bf16x8 (&sa)[FixShape<DK>::KS][FixShape<DK>::JJ]) {
  using F = FixShape<DK>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (LATER) {
    if (threadIdx.x == 0) {
      const int* flag = p.state_flags + (size_t)f.slot * p.H + f.h;
      for (int n = 0; n < kWaitPolls; ++n) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= F::NB) break;
        __builtin_amdgcn_s_sleep(4);
      }
    }
    __syncthreads();
  }
  const auto srs = rsrc(p.sb + ((size_t)f.slot * p.H + f.h) * (D * D), D * D * 2);
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks)
#pragma unroll
    for (int jj = 0; jj < F::JJ; ++jj) {
      const int off = ((ks * F::NB + F::JJ * wave + jj) * 64 + lane) * 16;
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, LATER ? kDeviceScope : 0);
      sa[ks][jj] = __builtin_bit_cast(bf16x8, x);
    }
}

// Fix-up units [u_lo, u_hi) of this workgroup: o = O0 + S_p^T Q~ for every row
// of each unit's chunk.  The next unit's loads are in flight while the current
// one is multiplied; S_p is reloaded only when the segment or head changes.
template <int DK, int SEG0>
__device__ void fix_range(const Params& p, const PlanView& v, int M, const int* off,
                          int u_lo, int u_hi, __bf16* ot) {
  constexpr int seg0 = SEG0;
  using F = FixShape<DK>;
  if (u_lo >= u_hi) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, m16 = lane & 15;
  const int HD = p.H * DK;
  FixUnit cur = fix_decode(p, v, M, off, seg0, u_lo);
  FixLoads<DK> L;
  fix_issue<DK>(p, cur, L);
  bf16x8 sa[F::KS][F::JJ];
  fix_state<DK, SEG0 == 2>(p, cur, sa);
  for (int u = u_lo; u < u_hi; ++u) {
    // stage Q~ of the current unit (its B operand order) in LDS
#pragma unroll
    for (int x = 0; x < F::QP; ++x) {
      uint2* dst = reinterpret_cast<uint2*>(&ot[(F::RPS * x + tid / F::TPR) * TS + 8 * (tid % F::TPR)]);
      dst[0] = make_uint2(L.qv[x][0], L.qv[x][1]);
      dst[1] = make_uint2(L.qv[x][2], L.qv[x][3]);
    }
    f32x4 z[4][F::JJ];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < F::JJ; ++jj) {
        float f[4];
        unpack4(make_uint2(L.zv[tt][jj][0], L.zv[tt][jj][1]), f);
        z[tt][jj] = f32x4{f[0], f[1], f[2], f[3]};
      }
    const FixUnit f = cur;
    const bool more = u + 1 < u_hi;
    if (more) {
      cur = fix_decode(p, v, M, off, seg0, u + 1);
      fix_issue<DK>(p, cur, L);  // the next unit's loads fly during this unit's products
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int ks = 0; ks < F::KS; ++ks) {
        const __bf16* bp = &ot[(16 * tt + m16) * TS + 32 * ks + 8 * q4];
        const bf16x8 bb = ld2x4(bp, bp + 4);
#pragma unroll
        for (int jj = 0; jj < F::JJ; ++jj) z[tt][jj] = mfma32(sa[ks][jj], bb, z[tt][jj]);
      }
    }
    // lane holds o[token 16tt + m16][columns 16jt + 4q4 .. +3], jt = JJ wave + jj.  The
    // rows go out through the Q~ tile (every wave's reads of it are done at the barrier):
    // each thread stores 16 bytes that continue its neighbour's along the row, instead of
    // 8 bytes in each of 16 rows per instruction
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < F::JJ; ++jj)
        *reinterpret_cast<uint2*>(&ot[(16 * tt + m16) * TS + 16 * (F::JJ * wave + jj) + 4 * q4]) =
            pack4(z[tt][jj][0], z[tt][jj][1], z[tt][jj][2], z[tt][jj][3]);
    __syncthreads();
    const auto orsrc = rsrc(p.out + f.tok0 * HD + (int64_t)f.h * DK, f.valid * HD * 2);
#pragma unroll
    for (int x = 0; x < F::QP; ++x) {  // rows past `valid` fall outside the descriptor
      const int row = F::RPS * x + tid / F::TPR, c8 = 8 * (tid % F::TPR);
      const uint2 a = *reinterpret_cast<const uint2*>(&ot[row * TS + c8]);
      const uint2 b = *reinterpret_cast<const uint2*>(&ot[row * TS + c8 + 4]);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{a.x, a.y, b.x, b.y}, orsrc, (row * HD + c8) * 2, 0, 0);
    }
    if (more && (cur.slot != f.slot || cur.h != f.h)) fix_state<DK, SEG0 == 2>(p, cur, sa);
    __syncthreads();  // before the next unit's staging
  }
}

template <int DK>
__global__ void __launch_bounds__(TAIL_NT, 3) kda_tail_kernel(Params p) {
  extern __shared__ int plan_lds[];
  __shared__ __attribute__((aligned(16))) float slt[16 * SLT];
  __shared__ __attribute__((aligned(16))) __bf16 ot[C * TS];
  const int N = p.nseq;
  const PlanView v = plan_view(plan_lds, N, 0);
  build_plan(p, v, false);
  // wave-uniform unit values keep every buffer descriptor scalar
  const int M = __builtin_amdgcn_readfirstlane(v.hdr[0]);
  if (M == kNoSplit) return;
  const int G = gridDim.x, b = blockIdx.x;
  // Scan units go to the first S workgroups (each may take several); at least a
  // compute unit's worth of workgroups remains for the fix-ups.
  const int nscan = __builtin_amdgcn_readfirstlane(v.hdr[3]) * p.H * (DK / 16);
  const int S = min(nscan, G - p.cus);
  if (b < S)
    for (int u = b; u < nscan; u += S) scan_unit<DK>(p, v, M, u, slt);
  // Segment-1 fix-ups need only S_1.  With a scan of several steps they go to the
  // workgroups without scan units; a one-step scan (two segments at most) ends long
  // before them, and then every workgroup takes its share, after its scan units.
  const int F1 = __builtin_amdgcn_readfirstlane(v.hdr[4]);
  const int mx = __builtin_amdgcn_readfirstlane(v.hdr[6]);
  const bool one_step = (mx + M - 1) / M <= 2;
  const int first = one_step ? 0 : S;
  if (b >= first)
    fix_range<DK, 1>(p, v, M, v.uoff, (int)((int64_t)F1 * (b - first) / (G - first)),
                     (int)((int64_t)F1 * (b - first + 1) / (G - first)), ot);
  // Later segments: only workgroups without scan units wait for published states.
  const int F2 = __builtin_amdgcn_readfirstlane(v.hdr[5]);
  if (b >= S && F2 > 0)
    fix_range<DK, 2>(p, v, M, v.voff, (int)((int64_t)F2 * (b - S) / (G - S)),
                     (int)((int64_t)F2 * (b - S + 1) / (G - S)), ot);
}

}  // namespace

int workspace_slots(int cus, int H) { return (H > 0 && H < cus) ? cus / H + 1 : 0; }

WorkspaceLayout workspace_layout(int64_t ucap, int H, int emax) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout l;
  l.o0 = 0;
  l.st = up((size_t)ucap * kUnitBytes);
  l.sb = l.st + up((size_t)3 * emax * H * D * D * 4);
  l.flag = l.sb + up((size_t)emax * H * D * D * 2);
  l.total = l.flag + up((size_t)emax * H * 4);
  return l;
}

size_t workspace_slot_bytes(int H) { return (size_t)H * D * D * (3 * 4 + 2); }

hipError_t launch_fwd(const Params& p, int nsplit, hipStream_t stream) {
  if (nsplit != 1 && nsplit != 2) return hipErrorInvalidValue;
  if (p.dk != 128 && (p.dk != 64 || nsplit != 1 || p.ckpt != nullptr)) return hipErrorInvalidValue;
  if (p.emax > 0 && (nsplit != 1 || p.o0 == nullptr || p.st == nullptr || p.sb == nullptr ||
                     p.state_flags == nullptr))
    return hipErrorInvalidValue;
  // task groups: every sequence, plus two runs per extra segment (fewer than
  // 2 * emax of them when splitting)
  const int64_t groups = (int64_t)p.nseq + (p.emax > 0 && p.nseq <= kSortLimit ? 2 * (int64_t)p.emax : 0);
  const int64_t wgs = (groups * p.H + 7) / 8 * 8 * nsplit;
  const dim3 block(NT);
  hipError_t err;
  if (p.dk == 64) {  // one 64-column slice, either gate
    err = launch_fwd_main_hd64(p, (unsigned)wgs, stream);
  } else if (p.g_scalar) {
    err = launch_fwd_main_scalar_gate(p, nsplit, (unsigned)wgs, stream);
  } else {
    if (nsplit == 1) hipLaunchKernelGGL((kda_fwd_kernel<2, false, 128>), dim3((unsigned)wgs), block, 0, stream, p);
    else hipLaunchKernelGGL((kda_fwd_kernel<1, false, 128>), dim3((unsigned)wgs), block, 0, stream, p);
    err = hipGetLastError();
  }
  if (err != hipSuccess || p.emax == 0 || p.nseq > kSortLimit) return err;
  const size_t plan_bytes = (size_t)plan_ints(p.nseq, 0, false) * sizeof(int);
  if (p.dk == 64) hipLaunchKernelGGL(kda_tail_kernel<64>, dim3(3 * p.cus), dim3(TAIL_NT), plan_bytes, stream, p);
  else hipLaunchKernelGGL(kda_tail_kernel<128>, dim3(3 * p.cus), dim3(TAIL_NT), plan_bytes, stream, p);
  return hipGetLastError();
}

}  // namespace kda
