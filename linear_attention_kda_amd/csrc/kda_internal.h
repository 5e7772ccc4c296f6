// Internal launch interface between the C ABI (kda_api.cpp) and the gfx950 kernels.
#ifndef KDA_INTERNAL_H_
#define KDA_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Sequences longer-first ordering is computed on the device for at most this
// many packed sequences; beyond it workgroups follow the packing order.
constexpr int kSortLimit = 1024;

struct Params {
  const uint16_t* q;      // bf16 [rows][H][128]
  const uint16_t* k;
  const uint16_t* v;
  const float* g;         // fp32 [rows][H][128]
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
};

// Enqueue the forward pass; nsplit in {1, 2} value-column slices per (sequence, head).
hipError_t launch_fwd(const Params& p, int nsplit, hipStream_t stream);

}  // namespace kda

#endif  // KDA_INTERNAL_H_
