// Direct-to-LDS staging and swizzled MFMA operand reads for the bf16 attention kernels.
//
// Tiles cover 64 keys on 64-aligned positions of the (b, h) key axis. K rows (D bf16 each) and
// V^T rows (64 keys of one dim, from a transposed copy of V) are copied global -> LDS with
// 16-byte global_load_lds (lane l of a wave lands at base + 16 l), so staging uses no VGPRs
// and no VALU. Both tiles use an XOR swizzle of 16-byte chunks instead of padding:
//   K   [64][D]:  chunk c of row r is stored at chunk c ^ (r & (D/8 - 1))
//   V^T [D][64]:  chunk c of row d is stored at chunk c ^ ((d >> 1) & 7)
// which keeps the MFMA operand reads below free of bank conflicts.
//
// Key order: S^T = K Q^T is computed with lane m of the A operand reading K row pi(m),
//   pi(8a + 4b + c) = 16 (a >> 1) + 8 b + 4 (a & 1) + c,   (a = 0..3, b = 0..1, c = 0..3)
// so output value i (0..15) of lane group g holds key 16 (i >> 3) + 8 g + (i & 7) of the
// 32-key block: each lane's P values for one 16-key MFMA step are 8 contiguous keys, the V^T
// operand of O^T += V^T P^T is one 16-byte read.
#pragma once

#include "attn_common.h"

namespace moc {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// 16-byte global -> LDS copy; lane l lands at lds_base + 16 l (lds_base is wave-uniform)
__device__ __forceinline__ void copy16_to_lds(const void* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)const_cast<void*>(src), (lds_ptr_t)lds_base, 16, 0, 0);
}

__device__ __forceinline__ int kperm(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// key (within the 64-key tile) of S^T output value i of block kb for lane group g
__device__ __forceinline__ int key_of_perm(int kb, int i, int g) {
  return kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
}

template <int D>
struct LdsTiles {
  static constexpr int KBYTES = kBN * D * 2;        // K tile
  static constexpr int VBYTES = D * kBN * 2;        // V^T tile
  static constexpr int STAGE = KBYTES + VBYTES;     // bytes per stage
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
};

// Issue the direct-to-LDS copies of one (K, V^T) tile. NW waves; every wave issues
// (64*KCH + D*8) / (64 * NW) 16-byte loads per lane. K rows past `kmax` are clamped to it
// (their scores are masked), V^T reads stay inside the padded transposed copy.
template <int D, int NW>
__device__ __forceinline__ void stage_tile_async(char* stage, const bf16_t* __restrict__ Kbh,
                                                 const bf16_t* __restrict__ Vtbh, int Lp,
                                                 int tbase, int kmax) {
  using LT = LdsTiles<D>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int KBLK = LT::KBYTES / 1024;  // 1 KB blocks of the K tile
  constexpr int VBLK = LT::VBYTES / 1024;
  static_assert(KBLK % NW == 0 && VBLK % NW == 0, "tile split over waves");
#pragma unroll
  for (int j = 0; j < KBLK / NW; ++j) {
    const int blk = wv * (KBLK / NW) + j;
    const int e = blk * 64 + lane;             // 16-byte chunk index within the tile
    const int r = e / LT::KCH, c = e % LT::KCH;
    const int cg = c ^ (r & (LT::KCH - 1));    // global chunk stored at this LDS chunk
    int key = tbase + r;
    key = key < kmax ? key : kmax;
    const bf16_t* src = Kbh + static_cast<size_t>(key) * D + cg * 8;
    copy16_to_lds(src, stage + blk * 1024);
  }
#pragma unroll
  for (int j = 0; j < VBLK / NW; ++j) {
    const int blk = wv * (VBLK / NW) + j;
    const int e = blk * 64 + lane;
    const int d = e >> 3, c = e & 7;
    const int cg = c ^ ((d >> 1) & 7);
    const bf16_t* src = Vtbh + static_cast<size_t>(d) * Lp + tbase + cg * 8;
    copy16_to_lds(src, stage + LT::KBYTES + blk * 1024);
  }
}

// S^T block kb (32 keys x 32 queries) with the permuted key order.
template <int D>
__device__ __forceinline__ f32x16 score_block_swz(const char* stage, const QFrag<bf16_t, D>& qf,
                                                  int kb, int ql, int g) {
  f32x16 acc = {};
  const int r = kb * 32 + kperm(ql);
  const char* row = stage + r * (D * 2);
  const int sw = r & (D / 8 - 1);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int ch = (2 * kk + g) ^ sw;
    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + ch * 16));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.q[kk], acc, 0, 0, 0);
  }
  return acc;
}

// O^T[db] += V^T P^T for one 64-key tile (P^T in the permuted output layout, fp32).
template <int D>
__device__ __forceinline__ void pv_swz(const char* stage, const f32x16 (&p)[2],
                                       f32x16 (&acc)[D / 32], int ql, int g) {
  using LT = LdsTiles<D>;
  const char* vt = stage + LT::KBYTES;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kb = ks >> 1, hh = ks & 1;
    bf16x8 pb;
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) pb[ii] = static_cast<__bf16>(p[kb][8 * hh + ii]);
    const int c = 4 * kb + 2 * hh + g;  // 8-key chunk of this lane group
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + ql;
      const int ch = c ^ ((d >> 1) & 7);
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vt + d * 128 + ch * 16));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
    }
  }
}

}  // namespace moc
