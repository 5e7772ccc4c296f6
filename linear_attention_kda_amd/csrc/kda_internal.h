// Internal launch interface between the C ABI (kda_api.cpp) and the gfx950 kernels.
#ifndef KDA_INTERNAL_H_
#define KDA_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Sequences are ordered longest-first, and long ones split into segments, only
// when there are at most this many packed sequences; beyond it workgroups
// follow the packing order and every sequence runs whole.
constexpr int kSortLimit = 1024;

// Shortest sequence (in 64-token chunks) that may be split into segments.
constexpr int kSegMinDefault = 8;
// Segment length rule: the shortest M for which H * (chunks + chunks past the
// first segment) <= kSlackNum / kSlackDen * M * compute units.  The slack keeps
// a little imbalance rather than splitting more: each split chunk costs an
// extra identity-start run and a fix-up, while the last tasks of a nearly
// balanced run finish with most of the device idle (and its power budget free).
constexpr int kSlackNum = 19, kSlackDen = 20;

struct Params {
  const uint16_t* q;      // bf16 [rows][H][128]
  const uint16_t* k;
  const uint16_t* v;
  const float* g;         // fp32 [rows][H][128], or [rows][H] when g_scalar
  const float* beta;      // fp32 [rows][H]
  uint16_t* out;          // bf16 [rows][H][128]
  const void* s0;         // [N][H][128][128] or null
  void* s1;               // [N][H][128][128] or null
  const int32_t* cu;      // [N+1] or null
  int64_t T;              // tokens per batch row (fixed-length mode)
  float scale;
  int s0_fp32;
  int s1_fp32;
  int nseq;               // N: sequences (varlen) or batch rows
  int H;
  // Sequence splitting (all zero / null: every sequence runs whole).
  int cus;                // parallel width the segment plan fills (compute units)
  int seg_min;            // shortest sequence, in chunks, that may be split
  int emax;               // segment state slots in the workspace; 0 disables splitting
  uint16_t* o0;           // bf16 [rows][H][128]: outputs of later segments from a zero state
  float* st;              // fp32 [3][emax][H][128][128]: segment start states, A maps, B states
  uint16_t* sb;           // bf16 [emax][H][128*128]: segment start states, fix-up operand order
  // Backward support: the fp32 state at the start of every chunk, at slot
  // n + floor(bos_n / 64) + c of sequence n's chunk c ([slots][H][128][128]), or
  // null.  Requires emax = 0 (no sequence splitting).
  float* ckpt;
  int g_scalar;           // one gate per token and head (Gated DeltaNet)
};

// Workspace bytes for splitting with `emax` state slots over `rows` packed
// rows of H heads, and the offsets of its three parts.
struct WorkspaceLayout {
  size_t o0, st, sb, total;
};
WorkspaceLayout workspace_layout(int64_t rows, int H, int emax);

// State slots a plan can use on `cus` compute units with H heads: the plan
// never needs more than cus / H extra segments.
int workspace_slots(int cus, int H);

// One decode step: one token per sequence, state updated in place.
struct DecodeParams {
  const uint16_t* q;      // bf16 [N][H][D]
  const uint16_t* k;
  const uint16_t* v;
  const float* g;         // fp32 [N][H][D], or [N][H] when g_scalar
  const float* beta;      // fp32 [N][H]
  uint16_t* out;          // bf16 [N][H][D]
  int g_scalar;           // one gate per token and head (Gated DeltaNet)
  int D;                  // head dimension: 64, 128 or 256
  void* state;            // [slots][H][D][D], bf16 or fp32
  const int32_t* idx;     // [N] state slot of each sequence (negative: skip), or null (slot n)
  float scale;
  int state_fp32;
  int nseq;
  int H;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// ---- backward
struct BwdParams {
  const uint16_t* q;      // bf16 [rows][H][128]
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;   // bf16 [rows][H][128]: dL/do
  const float* g;         // fp32 [rows][H][128]
  const float* beta;      // fp32 [rows][H]
  const int32_t* cu;      // [N+1] or null
  int64_t T;              // tokens per batch row (fixed-length mode)
  float scale;
  int nseq;
  int H;
  const void* dsT;        // dL/dS_final [N][H][128][128] or null
  int dsT_fp32;
  float* dq;              // fp32 [rows][H][128]
  float* dk;
  float* dv;
  float* dg;
  float* dbeta;           // fp32 [rows][H]
  float* ds0;             // fp32 [N][H][128][128] or null
};

// Per-chunk fp32 tiles of the backward, each an array over batches b = slot * H + h.
struct BwdTiles {
  // [b][64][128]
  float *G, *kg, *qg, *kh, *kp, *vv, *dO, *R, *U, *MtdO, *dU, *dY, *dqg, *dkg, *dkh, *dkp;
  float *A, *P, *M, *T, *dM, *dA;   // [b][64][64]
  float* F;                          // [b][128][64]
  float *S, *X, *dSn;                // [b][128][128]; S: chunk start states (the checkpoints)
  float* beta;                       // [b][64]
  float* gam;                        // [b][128]
  int* valid;                        // [b]
  static constexpr size_t floats_per_batch() {
    return 16 * 64 * 128 + 6 * 64 * 64 + 128 * 64 + 3 * 128 * 128 + 64 + 128 + 1;
  }
};

struct GemmArgs {
  int M, N, K, batches;
  const float* A; int64_t sA; int lda;
  const float* B; int64_t sB; int ldb;
  float* C; int64_t sC; int ldc;
  const float* Dm; int64_t sD; int ldd;   // added before the row scale, or null
  const float* rs; int64_t srs;           // row scale of the output, or null
  const float* ks; int64_t sks;           // scale of op(A)'s k-th column, or null
  float alpha;
  int mask;                               // 0 none, 1 keep n < m, 2 keep n <= m
};

size_t bwd_tile_floats();
hipError_t launch_bwd(const BwdParams& p, const BwdTiles& w, int64_t batches, hipStream_t stream);
// The initial-state gradients alone, for calls without tokens.
hipError_t launch_bwd_scan_only(const BwdParams& p, hipStream_t stream);

// Forward pass at head dimension D = K = V in {64, 256}: a chunk-parallel
// prep kernel writes one record of per-chunk operands for every (chunk, head)
// into the workspace, then a serial kernel walks each (sequence, head, 64
// value columns) through its chunks.  Chunk c of sequence n uses record slot
// n + floor(bos_n / 64) + c; dim_slots() bounds the slot count.
struct DimParams {
  const uint16_t* q;      // bf16 [rows][H][D]
  const uint16_t* k;
  const uint16_t* v;
  const float* g;         // fp32 [rows][H][D], or [rows][H] when g_scalar
  const float* beta;      // fp32 [rows][H]
  uint16_t* out;          // bf16 [rows][H][D]
  const void* s0;         // [N][H][D][D] or null
  void* s1;               // [N][H][D][D] or null
  const int32_t* cu;      // [N+1] or null
  int64_t T;              // tokens per batch row (fixed-length mode)
  int64_t slots;          // record slots in the workspace
  float scale;
  int s0_fp32;
  int s1_fp32;
  int nseq;
  int H;
  int D;
  int g_scalar;
  char* ws;               // [slots][H] records of dim_record_bytes(D) bytes
};
size_t dim_record_bytes(int D);
int64_t dim_slots(int64_t nseq, int64_t rows);
hipError_t launch_fwd_dim(const DimParams& p, hipStream_t stream);

// Enqueue the forward pass; nsplit in {1, 2} value-column slices per (sequence,
// head).  With p.emax > 0 (nsplit must be 1) long sequences may be split, and
// the segment scan and output fix-up kernels follow the main kernel.
hipError_t launch_fwd(const Params& p, int nsplit, hipStream_t stream);
// The fused kernel alone with the scalar gate (p.g_scalar), wgs workgroups.
hipError_t launch_fwd_main_scalar_gate(const Params& p, int nsplit, unsigned wgs, hipStream_t stream);

}  // namespace kda

#endif  // KDA_INTERNAL_H_
