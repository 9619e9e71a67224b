// K1: mean-pooled chunk keys (the chunk descriptor of the MoC router).
//
// Source: "Mixture of Contexts for Long Video Generation | Summary", §3.1 (each chunk is scored
// through the mean of its keys) and §3.3 / the jxzklqfsx.com write-up, section 計算效率
// (segmented mean computed on the fly, chunks of very different sizes).
//
// kbar[b,h,c,:] = RN32( RN64(sum_{t in c} K[b,h,t,:]) / n_c ). The sum is carried as an
// unevaluated double-double (hi + lo) built from error-free TwoSum steps, so the result does
// not depend on the summation order: every bf16 input and every fp32 input whose exponents
// span less than ~80 binades is summed exactly before the single binary64 division.
//
// Work decomposition: one workgroup per (b, h, chunk) and column half (bf16, d = 128: 1,356
// chunks of a 12-head headline layer would otherwise leave a ragged last round of workgroups).
// A chunk is a contiguous run of n_c rows of d elements, so the workgroup streams its columns
// with 16-byte coalesced loads; each thread owns 16/sizeof(T) consecutive columns of every
// RPI-th row. HBM-bound: one read of K.
#include "moc_common.h"

namespace moc {

__device__ __forceinline__ void dd_add(double& hi, double& lo, double x) {
  double s = hi + x;                       // TwoSum(hi, x) = (s, e), s + e == hi + x exactly
  double bp = s - hi;
  double e = (hi - (s - bp)) + (x - bp);
  lo += e;
  hi = s;
}

__device__ __forceinline__ void dd_merge(double& hi, double& lo, double bhi, double blo) {
  double s = hi + bhi;
  double bp = s - hi;
  double e = (hi - (s - bp)) + (bhi - bp);
  lo = lo + blo + e;
  hi = s;
}

// PARTIAL: instead of the mean, write the chunk's double-double sum (hi, lo) to part
// [B*H][C][D][2], for sums over groups of chunks (outer-loop routing's segment features).
// NS: workgroups per chunk, each owning D / NS consecutive columns (blockIdx.z), so that more,
// shorter workgroups leave a shorter tail; the columns' sums are independent.
template <typename T, int D, bool PARTIAL = false, int NS = 1>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ K,
                                                   const int32_t* __restrict__ off,
                                                   float* __restrict__ kbar, int L, int C,
                                                   const uint32_t* __restrict__ chk,
                                                   double* __restrict__ part = nullptr) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int DW = D / NS;       // columns of this workgroup
  constexpr int TPR = DW / VEC;    // threads per row
  constexpr int RPI = 256 / TPR;   // rows per pass
  __shared__ double sh[2][RPI][DW];
  if (layout_rejected(chk)) return;

  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int col0 = static_cast<int>(blockIdx.z) * DW;
  const int r0 = off[c];
  const int n = off[c + 1] - r0;
  const T* base = K + (static_cast<size_t>(bh) * L + r0) * D + col0;
  const int tr = threadIdx.x / TPR;
  const int tc = threadIdx.x % TPR;

  double hi[VEC], lo[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) { hi[i] = 0.0; lo[i] = 0.0; }

  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  int r = tr;
  // four rows in flight per thread
  for (; r + 3 * RPI < n; r += 4 * RPI) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(r + u * RPI) * D + tc * VEC);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) dd_add(hi[i], lo[i], static_cast<double>(to_f32<T>(e[i])));
    }
  }
  for (; r < n; r += RPI) {
    u32x4 v = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(r) * D + tc * VEC);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int i = 0; i < VEC; ++i) dd_add(hi[i], lo[i], static_cast<double>(to_f32<T>(e[i])));
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    sh[0][tr][tc * VEC + i] = hi[i];
    sh[1][tr][tc * VEC + i] = lo[i];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < DW; j += blockDim.x) {
    double h = 0.0, l = 0.0;
    for (int k = 0; k < RPI; ++k) dd_merge(h, l, sh[0][k][j], sh[1][k][j]);
    if constexpr (PARTIAL) {
      double* o = part + ((static_cast<size_t>(bh) * C + c) * D + col0 + j) * 2;
      o[0] = h;
      o[1] = l;
      continue;
    }
    // renormalise, then the binary64 sum is the rounded value of h + l
    double s = h + l;
    double mean = s / static_cast<double>(n);
    kbar[(static_cast<size_t>(bh) * C + c) * D + col0 + j] = static_cast<float>(mean);
  }
}

}  // namespace moc

namespace moc_host {

template <typename T, int D>
static hipError_t launch_pool_t(const moc_layout* lay, const void* K, float* kbar,
                                hipStream_t st) {
  // two workgroups per chunk (each 128 bytes of every bf16 row at d = 128) where the grid
  // would otherwise be only a few rounds of workgroups deep
  constexpr int NS = (sizeof(T) == 2 && D == 128) ? 2 : 1;
  dim3 grid(lay->C, lay->B * lay->H, NS);
  hipLaunchKernelGGL((moc::pool_kernel<T, D, false, NS>), grid, dim3(256), 0, st,
                     static_cast<const T*>(K), lay->chunk_offsets, kbar, lay->L, lay->C,
                     lay->check);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_pool_partial_t(const moc_layout* lay, const void* X, double* part,
                                        hipStream_t st) {
  dim3 grid(lay->C, lay->B * lay->H);
  hipLaunchKernelGGL((moc::pool_kernel<T, D, true>), grid, dim3(256), 0, st,
                     static_cast<const T*>(X), lay->chunk_offsets, nullptr, lay->L, lay->C,
                     lay->check, part);
  return hipGetLastError();
}

// Double-double chunk sums [B*H][C][d][2] of X (outer-loop routing's segment features).
hipError_t launch_pool_partial(const moc_layout* lay, const void* X, double* part,
                               hipStream_t st) {
  if (lay->dtype == MOC_BF16) {
    return lay->d == 128 ? launch_pool_partial_t<moc::bf16_t, 128>(lay, X, part, st)
                         : launch_pool_partial_t<moc::bf16_t, 64>(lay, X, part, st);
  }
  return lay->d == 128 ? launch_pool_partial_t<float, 128>(lay, X, part, st)
                       : launch_pool_partial_t<float, 64>(lay, X, part, st);
}

hipError_t launch_pool(const moc_layout* lay, const void* K, float* kbar, hipStream_t st) {
  if (lay->dtype == MOC_BF16) {
    return lay->d == 128 ? launch_pool_t<moc::bf16_t, 128>(lay, K, kbar, st)
                         : launch_pool_t<moc::bf16_t, 64>(lay, K, kbar, st);
  }
  return lay->d == 128 ? launch_pool_t<float, 128>(lay, K, kbar, st)
                       : launch_pool_t<float, 64>(lay, K, kbar, st);
}

}  // namespace moc_host
