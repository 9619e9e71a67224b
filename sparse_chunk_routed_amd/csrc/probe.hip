// Benchmark helper, not part of libmoc and not a step of the layer: register-only MFMA loops
// that show the matrix-core rate this chip sustains under its clock and power limits (bf16
// 32x32x16, and fp8 32x32x64 with E8M0 block scales), next to which the attention kernels' MFMA
// rates are read. Built on its own into libmoc_bench_probe.so, which only the benchmark loads.
//
//   int moc_bench_probe_mfma(int fp8, int blocks, int iters, float* sink, void* stream)
//     Launches `blocks` workgroups of 4 waves on `stream` (a hipStream_t); every wave runs `iters`
//     rounds of 8 independent 32x32x16 bf16 MFMAs (fp8 = 0) or 32x32x64 e4m3 MFMAs with unit
//     scales (fp8 = 1) and writes one float per thread to sink (device float [blocks * 256]).
//     FLOPs = blocks * 4 * iters * 8 * 2 * 32 * 32 * (16 or 64). Returns 0 when launched, 1 on a
//     bad argument, 2 when the launch fails.
#include "moc_common.h"

namespace moc {

typedef __attribute__((ext_vector_type(8))) int probe_i32x8;

// Every wave runs `iters` rounds of 8 independent accumulation chains (no dependency stalls),
// operands in registers; the sums go to sink so that nothing is optimised away.
template <bool FP8>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x16{};
  if constexpr (FP8) {
    probe_i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x30303030 + lane;  // small finite e4m3 codes
      b[i] = 0x28282828 + i;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 0x7f7f7f7f,
                                                                  0, 0x7f7f7f7f);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<__bf16>(0.001f * static_cast<float>(lane + i));
      b[i] = static_cast<__bf16>(0.002f * static_cast<float>(lane - i));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace moc

extern "C" int moc_bench_probe_mfma(int fp8, int blocks, int iters, float* sink, void* stream) {
  if ((fp8 != 0 && fp8 != 1) || blocks < 1 || blocks > 65535 || iters < 1 || iters > 10000000 ||
      !sink)
    return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL((moc::mfma_probe_kernel<true>), dim3(blocks), dim3(256), 0, st, iters,
                       sink);
  else
    hipLaunchKernelGGL((moc::mfma_probe_kernel<false>), dim3(blocks), dim3(256), 0, st, iters,
                       sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
