// Internal launch interface between the C ABI (kda_api.cpp) and the gfx950 kernels.
#ifndef KDA_INTERNAL_H_
#define KDA_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

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
  int ucap;               // fix-up units the workspace's output blocks hold
  uint16_t* o0;           // bf16 [ucap][64][128]: outputs of later segments from a zero
                          // state, one 64-row block per fix-up unit (sequence, head, chunk)
  float* st;              // fp32 [3][emax][H][128][128]: segment start states, A maps, B states
  uint16_t* sb;           // bf16 [emax][H][128*128]: segment start states, fix-up operand order
  int* state_flags;       // [emax][H]: scan column blocks that have published the fix-up
                          // operand of that slot's start state (zeroed by the main kernel)
  // Backward support: the fp32 state at the start of every chunk, at slot
  // n + floor(bos_n / 64) + c of sequence n's chunk c ([slots][H][128][128]), or
  // null.  Requires emax = 0 (no sequence splitting).
  float* ckpt;
  int g_scalar;           // one gate per token and head (Gated DeltaNet)
  // Key/value head dimension: 128, or 64 (q, k, v, g, out and the states laid out
  // with 64 channels; the kernel runs it as a 128-channel problem whose key
  // channels past 64 are zero, in one 64-column value slice).  The split
  // workspace keeps its 128 x 128 slots and 64 x 128 output blocks; at 64 their
  // first 64 x 64 entries (row stride 64) and first 64 columns are used.
  int dk;
};

// Workspace bytes for splitting with `emax` state slots and `ucap` fix-up
// units of H heads, and the offsets of its three parts.
struct WorkspaceLayout {
  size_t o0, st, sb, flag, total;
};
WorkspaceLayout workspace_layout(int64_t ucap, int H, int emax);
// Bytes of one state slot (all heads) and of one fix-up unit's output block.
size_t workspace_slot_bytes(int H);
constexpr size_t kUnitBytes = 64 * 128 * 2;

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
  // The slot group of one pass: batches b = slot * H + h with slot0 <= slot < slot1.
  // The per-chunk tiles hold the group's batches only (tile index b - slot0 * H).
  // A sequence that continues past slot1 starts its state-gradient scan from
  // carry_in; one that continues below slot0 leaves its dS in carry_out (both
  // [H][128][128]; at most one sequence crosses each group boundary).
  int64_t slot0;
  int64_t slot1;
  const float* carry_in;
  float* carry_out;
};

// Per-chunk fp32 tiles of the backward, each an array over batches b = slot * H + h.
struct BwdTiles {
  // [b][64][128]
  float *G, *kg, *qg, *kp, *vv, *dO, *R, *U, *MtdO, *dU, *dY, *dqg, *dkg, *dkp;
  float *A, *P, *M, *T, *dM, *dA;   // [b][64][64]
  float* F;                          // [b][128][64]
  float *X, *dSn;                    // [b][128][128]
  float* S;                          // [b][128][128]: chunk start states (the checkpoints); an
                                     // array over every slot, S pointing at the group's first batch
  float* beta;                       // [b][64]
  float* gam;                        // [b][128]
  float* dgl;                        // [b][128]: the state's direct share of dG_last
  int* valid;                        // [b]
  // fp32 words per batch of a group, and of the checkpoints (every slot)
  static constexpr size_t floats_per_batch() {
    return 14 * 64 * 128 + 6 * 64 * 64 + 128 * 64 + 2 * 128 * 128 + 64 + 2 * 128 + 1;
  }
  static constexpr size_t ckpt_floats_per_batch() { return 128 * 128; }
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

// The backward pass on two streams: the checkpointing forward pass (`fwd`, with
// fwd_splits value slices) and the products that need the checkpoints run on
// `side` beside the chunk-local tiles and the state-gradient scan on `hs`; `hs`
// waits for `side` before the last kernel, so that everything enqueued is ordered
// before later work on `hs`.  The chunk slots go in groups of at most group_slots,
// the last group first, each group through every part below with the tiles of
// `w` (sized for one group; w.S the checkpoints of every slot); the forward pass
// runs once, before the first group's state products.  `carry` holds two
// [H][128][128] state-gradient buffers (null when one group covers every slot).
// Parts, in dependency order:
//  * chunk_local: the tiles that need no state checkpoint (prep, P / A / M, the
//    inverse, M^T dO', F and X);
//  * state_products: R, U and dM, after chunk_local and the forward pass;
//  * scan: the state gradients over the chunks, after chunk_local only;
//  * then dY (after the scan, which forms dU), -diag(b) dY S^T and dO' S^T (after the
//    forward pass), dA (after the state products), dkp and the state term of dG_last
//    (after the scan and the state products, on `side`), the gated terms with dq, dk
//    and dg (after all of these), dbeta and dv (after dA, on `side`).
hipError_t launch_bwd_chunk_local(const BwdParams& p, const BwdTiles& w, int64_t batches, hipStream_t stream);
hipError_t launch_bwd_state_products(const BwdParams& p, const BwdTiles& w, int64_t batches,
                                     hipStream_t stream);
hipError_t launch_bwd_scan(const BwdParams& p, const BwdTiles& w, hipStream_t stream);
hipError_t launch_bwd_streams(const Params& fwd, int fwd_splits, const BwdParams& p, const BwdTiles& w,
                              int64_t slots, int64_t group_slots, float* carry, hipStream_t hs,
                              hipStream_t side);
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

// A caller-provided workspace: the forward pass sizes its plan to it instead of
// taking memory from the library's pool.
struct ExtWorkspace {
  void* ptr;
  size_t bytes;
};

// kda_fwd / kda_gdn_fwd (g_scalar), with the workspace from `ext` instead of the
// library's pool when ext is not null.
kda_status fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    float scale, const void* initial_state, int initial_dtype, void* final_state,
                    int final_dtype, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                    int64_t T, int32_t H, int32_t K, int32_t V, void* out, void* stream,
                    bool g_scalar, const ExtWorkspace* ext);
// Records the text of a failure (kda_last_error) and returns st.
kda_status record_failure(kda_status st, const char* text);

// Enqueue the forward pass; nsplit in {1, 2} value-column slices per (sequence,
// head).  With p.emax > 0 (nsplit must be 1) long sequences may be split, and
// the segment scan and output fix-up kernels follow the main kernel.  At
// p.dk = 64, nsplit must be 1 and there are no checkpoints.
hipError_t launch_fwd(const Params& p, int nsplit, hipStream_t stream);
// The fused kernel alone with the scalar gate (p.g_scalar), wgs workgroups.
hipError_t launch_fwd_main_scalar_gate(const Params& p, int nsplit, unsigned wgs, hipStream_t stream);
// The fused kernel alone at head dimension 64 (either gate), wgs workgroups.
hipError_t launch_fwd_main_hd64(const Params& p, unsigned wgs, hipStream_t stream);

}  // namespace kda

#endif  // KDA_INTERNAL_H_
