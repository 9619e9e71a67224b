// Device check of the layout content (the check word of moc_layout.check): one workgroup reads
// the chunk offsets and shot ids once and ORs the violations into the word, which every kernel
// of the same call reads first (layout_rejected).
#include "layout_check.h"
#include "moc_common.h"

namespace moc {

__global__ __launch_bounds__(256) void layout_check_kernel(const int32_t* __restrict__ off,
                                                           const int32_t* __restrict__ shot,
                                                           int C, int L, int tb, int te,
                                                           uint32_t* __restrict__ word) {
  __shared__ uint32_t acc;
  if (threadIdx.x == 0) acc = 0u;
  __syncthreads();
  const uint32_t bits = check_layout_bits(off, shot, C, L, tb, te, threadIdx.x, blockDim.x);
  if (bits) atomicOr(&acc, bits);
  __syncthreads();
  if (threadIdx.x == 0 && acc) atomicOr(word, acc);
}

}  // namespace moc

namespace moc_host {

hipError_t launch_layout_check(const moc_layout* lay, hipStream_t st) {
  hipLaunchKernelGGL(moc::layout_check_kernel, dim3(1), dim3(256), 0, st, lay->chunk_offsets,
                     lay->chunk_shot, lay->C, lay->L, lay->text_begin, lay->text_end,
                     lay->check);
  return hipGetLastError();
}

uint32_t layout_check_host(const int32_t* off, const int32_t* shot, int C, int L, int tb,
                           int te) {
  return moc::check_layout_bits(off, shot, C, L, tb, te, 0, 1);
}

}  // namespace moc_host
