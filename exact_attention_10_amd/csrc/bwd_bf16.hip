// Backward attention, bf16 (gfx950) -- launcher placeholder until the kernels land.
#include "internal.h"
namespace attn {
size_t bwd_workspace_bytes(int B, int Hq, int Sq) {
  return ((size_t)B * Hq * Sq * sizeof(float) + 255) / 256 * 256;
}
hipError_t launch_bwd_bf16(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
