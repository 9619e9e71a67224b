// K5: MoC attention backward (placeholder until the kernels land).
#include "attn_common.h"

namespace moc_host {

size_t attn_bwd_workspace(const moc_layout* lay, int S) {
  (void)lay;
  (void)S;
  return 256;
}

hipError_t launch_attn_bwd(const moc_layout*, const moc_varlen*, const void*, const void*,
                           const void*, const void*, const float*, const void*, float, void*,
                           void*, void*, void*, size_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moc_host
