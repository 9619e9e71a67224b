// MXFP8 quantisation of Q or K rows for the quantised-scores attention.
//
// Source: "Mixture of Contexts for Long Video Generation | Summary" §5 Conclusion, the
// jxzklqfsx.com write-up (section 結論) and the docswell slides (slide 21) name quantisation
// among the directions for faster kernels, without fixing a format. The format here is OCP Microscaling
// MXFP8: E4M3 elements (OCP OFP8: bias 7, largest finite 448) and per block of 32 consecutive
// elements of a row one E8M0 scale 2^E with E = floor(log2(max |x|)) - 8, clamped below at
// -127. An element is x * 2^-E (exact: a power-of-two scaling of a bf16 value) rounded to the
// nearest E4M3 value, ties to even, after saturation to +-448 (the hardware conversion
// v_cvt_pk_fp8_f32 rounds to nearest even and keeps the sign of a zero result).
#include "moc_common.h"

namespace moc {

typedef __attribute__((ext_vector_type(4))) uint32_t mx_u32x4;

// One thread per 32-element block of a row of the padded [B*H][Lp][D] output: reads 64 bytes
// of bf16, writes 32 code bytes and one scale byte. Rows >= L are written as zeros.
template <int D>
__global__ __launch_bounds__(256) void mx_quant_kernel(const bf16_t* __restrict__ X, int L, int Lp,
                                                       int64_t nblk, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  constexpr int NB = D / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nblk) return;
  const int64_t row = i / NB;  // over B*H*Lp
  const int blk = static_cast<int>(i % NB);
  const int64_t bh = row / Lp;
  const int r = static_cast<int>(row % Lp);
  mx_u32x4 out0 = {0u, 0u, 0u, 0u}, out1 = {0u, 0u, 0u, 0u};
  uint32_t sc = 0;
  if (r < L) {
    const mx_u32x4* src =
        reinterpret_cast<const mx_u32x4*>(X + (bh * L + r) * D + blk * 32);
    float f[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const mx_u32x4 w = src[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
        f[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(f[e]));
    // floor(log2(amax)) - 8 from the exponent field; a zero or subnormal amax gives -127
    int E = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;
    if (E < -127) E = -127;
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - E) << 23);  // 2^-E
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(f[4 * k + e] * inv, -448.f), 448.f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
      w[k] = static_cast<uint32_t>(pk);
    }
    out0 = mx_u32x4{w[0], w[1], w[2], w[3]};
    out1 = mx_u32x4{w[4], w[5], w[6], w[7]};
    sc = static_cast<uint32_t>(E + 127);
  }
  mx_u32x4* dst = reinterpret_cast<mx_u32x4*>(codes + row * D + blk * 32);
  dst[0] = out0;
  dst[1] = out1;
  scales[row * NB + blk] = static_cast<uint8_t>(sc);
}

// Quantised values: V [B*H][L][D] bf16 -> tiles [B*H][Lp/64][D][80] bytes. Per 64-key tile and
// dim d, the row holds the MXFP8 codes of V[key][d] for the tile's keys in two blocks of 32
// (same rule as above, blocks along the keys, aligned to key 0), position p of a block holding
// key p with bits 3 and 4 swapped (the order in which the attention's P^T operand holds its
// keys), then the two E8M0 scale codes at bytes 64 and 65, zeros at 66-79. Keys >= L are zero.
// One thread per (tile, d); a workgroup stages 256 / D tiles of V in LDS.
constexpr int kVqRowBytes = 80;

__device__ __forceinline__ int swap_bits34(int p) {
  return (p & ~24) | ((p & 8) << 1) | ((p & 16) >> 1);
}

template <int D>
__global__ __launch_bounds__(256) void mx_quant_v_kernel(const bf16_t* __restrict__ V, int L,
                                                         int ntiles, uint8_t* __restrict__ out,
                                                         const uint32_t* __restrict__ chk) {
  constexpr int TPB = 256 / D;   // tiles per workgroup
  constexpr int PITCH = D + 8;   // bf16 per staged key row
  __shared__ __attribute__((aligned(16))) bf16_t tile[TPB * 64 * PITCH];
  if (layout_rejected(chk)) return;
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * TPB;
  for (int e = threadIdx.x; e < TPB * 64 * (D / 8); e += 256) {
    const int r = e / (D / 8), c = e % (D / 8);   // r = staged key row over the TPB tiles
    const int key = t0 * 64 + r;
    mx_u32x4 v = {0u, 0u, 0u, 0u};
    if (key < L)
      v = *reinterpret_cast<const mx_u32x4*>(V + (static_cast<size_t>(bh) * L + key) * D + c * 8);
    *reinterpret_cast<mx_u32x4*>(tile + r * PITCH + c * 8) = v;
  }
  __syncthreads();
  const int tt = threadIdx.x / D, d = threadIdx.x % D;
  const int ti = t0 + tt;
  if (ti >= ntiles) return;
  uint32_t w[20];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float f[32];
#pragma unroll
    for (int k = 0; k < 32; ++k)
      f[k] = __uint_as_float(static_cast<uint32_t>(tile[(tt * 64 + 32 * b + k) * PITCH + d]) << 16);
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(f[k]));
    int E = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;
    if (E < -127) E = -127;
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - E) << 23);  // 2^-E
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = fminf(fmaxf(f[swap_bits34(4 * q + e)] * inv, -448.f), 448.f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
      w[8 * b + q] = static_cast<uint32_t>(pk);
    }
    if (b == 0) w[16] = static_cast<uint32_t>(E + 127);
    else w[16] |= static_cast<uint32_t>(E + 127) << 8;
  }
  w[17] = w[18] = w[19] = 0u;
  mx_u32x4* dst = reinterpret_cast<mx_u32x4*>(
      out + ((static_cast<size_t>(bh) * ntiles + ti) * D + d) * kVqRowBytes);
#pragma unroll
  for (int c = 0; c < 5; ++c) dst[c] = mx_u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
}

}  // namespace moc

namespace moc_host {

int attn_vt_rows(int L);

hipError_t launch_mx_quantize(const moc_layout* lay, const void* X, uint8_t* codes,
                              uint8_t* scales, hipStream_t st) {
  const int Lp = attn_vt_rows(lay->L);
  const int64_t nblk = static_cast<int64_t>(lay->B) * lay->H * Lp * (lay->d / 32);
  const int64_t grid = (nblk + 255) / 256;
  const moc::bf16_t* x = static_cast<const moc::bf16_t*>(X);
  if (lay->d == 128)
    hipLaunchKernelGGL((moc::mx_quant_kernel<128>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, st, x, lay->L, Lp, nblk, codes, scales, lay->check);
  else
    hipLaunchKernelGGL((moc::mx_quant_kernel<64>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, st, x, lay->L, Lp, nblk, codes, scales, lay->check);
  return hipGetLastError();
}

size_t mx_quantize_v_bytes(const moc_layout* lay) {
  const int Lp = attn_vt_rows(lay->L);
  return static_cast<size_t>(lay->B) * lay->H * (Lp / 64) * lay->d * moc::kVqRowBytes;
}

hipError_t launch_mx_quantize_v(const moc_layout* lay, const void* V, uint8_t* out,
                                hipStream_t st) {
  const int ntiles = attn_vt_rows(lay->L) / 64;
  const int BH = lay->B * lay->H;
  const moc::bf16_t* v = static_cast<const moc::bf16_t*>(V);
  if (lay->d == 128)
    hipLaunchKernelGGL((moc::mx_quant_v_kernel<128>), dim3((ntiles + 1) / 2, BH), dim3(256), 0,
                       st, v, lay->L, ntiles, out, lay->check);
  else
    hipLaunchKernelGGL((moc::mx_quant_v_kernel<64>), dim3((ntiles + 3) / 4, BH), dim3(256), 0,
                       st, v, lay->L, ntiles, out, lay->check);
  return hipGetLastError();
}

}  // namespace moc_host
