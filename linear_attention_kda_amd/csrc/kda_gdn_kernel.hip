// The fused chunkwise forward kernel with one gate per token and head (Gated
// DeltaNet) [core.today "Kimi Linear 특집", ch.4 혁신 1]: the kernel of
// kda_fwd_core.h with the gate broadcast over the key channels as it is loaded.
// It is instantiated here, apart from the per-channel variant, so that each
// variant is compiled in a module of its own.
#include "kda_fwd_core.h"

namespace kda {

hipError_t launch_fwd_main_scalar_gate(const Params& p, int nsplit, unsigned wgs, hipStream_t stream) {
  const dim3 block(NT);
  if (nsplit == 1) hipLaunchKernelGGL((kda_fwd_kernel<2, true, 128>), dim3(wgs), block, 0, stream, p);
  else hipLaunchKernelGGL((kda_fwd_kernel<1, true, 128>), dim3(wgs), block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
