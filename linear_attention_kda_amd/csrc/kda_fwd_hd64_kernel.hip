// The fused chunkwise forward kernel at head dimension 64 (K = V = 64), with
// either gate [core.today "Kimi Linear 특집", ch.4 혁신 1 and 혁신 2]: the kernel of
// kda_fwd_core.h reading 64 channels per head, with the key channels past 64 set
// to zero, in one 64-column value slice per (sequence, head, segment).  Zero key channels
// contribute nothing to K K^T, Q K^T, (K exp(G)) S or the state update, and the
// state rows they index stay zero.  It is instantiated here, in a module of its
// own, so that the 128-channel variants compile as before.
#include "kda_fwd_core.h"

namespace kda {

hipError_t launch_fwd_main_hd64(const Params& p, unsigned wgs, hipStream_t stream) {
  const dim3 block(NT);
  if (p.g_scalar) hipLaunchKernelGGL((kda_fwd_kernel<1, true, 64>), dim3(wgs), block, 0, stream, p);
  else hipLaunchKernelGGL((kda_fwd_kernel<1, false, 64>), dim3(wgs), block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
