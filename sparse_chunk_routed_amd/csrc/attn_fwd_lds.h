// Direct-to-LDS staging and MFMA operand reads for the bf16 attention kernels.
//
// Tiles cover 64 keys on 64-aligned positions of the (b, h) key axis. K rows (D bf16 each) and
// V^T rows (64 keys of one dim, from a transposed copy of V) are copied global -> LDS with
// 16-byte global_load_lds (lane l of a wave lands at base + 16 l), so staging uses no VGPRs
// and no VALU. Both tiles are stored row-major with one spare 16-byte chunk per row:
//   K   [64][D/8 + 1] chunks,   V^T [D][9] chunks
// With these odd row pitches (in chunks), the 16 lanes that one LDS read pass serves land on 16
// different 16-byte bank slots, and every operand read of a lane is one base address plus a
// compile-time offset (no per-step address registers). The copy of a 1 KB block walks the
// padded positions in order; a position that is padding copies a valid chunk that is never read.
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

// 16-byte global -> LDS copy: lane l reads gbase + voff (voff per lane, gbase wave-uniform)
// and lands at LDS byte address lds + 16 l (lds wave-uniform). Issued as inline asm so that
// the compiler adds no waits for it (its alias tracking of these copies is too coarse and would
// drain copies meant to stay in flight); the asm has no register outputs, and the callers wait
// for completion with an explicit s_waitcnt vmcnt and a barrier before any wave reads the stage.
__device__ __forceinline__ void copy16_to_lds(const void* gbase, uint32_t voff, uint32_t lds) {
  // the base and the LDS address are wave-uniform; make that visible (a no-op for values the
  // compiler already keeps in scalar registers)
  // (readfirstlane returns a signed int: both halves go through uint32_t, no sign extension)
  const uint64_t gb = reinterpret_cast<uint64_t>(gbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(gb)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(gb >> 32)));
  gbase = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
  lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds)));
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(gbase), "s"(lds)
      : "memory", "m0");
}

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)const_cast<void*>(p)));
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
  static constexpr int KCH = D / 8;                       // 16-byte chunks of one K row
  static constexpr int KROW = KCH + 1;                    // padded K row pitch (chunks)
  static constexpr int VROW = kBN / 8 + 1;                // padded V^T row pitch (chunks)
  static constexpr int KBLK = (kBN * KROW + 63) / 64;     // 1 KB copy blocks of the K tile
  static constexpr int VBLK = (D * VROW + 63) / 64;       // 1 KB copy blocks of the V^T tile
  static constexpr int KBYTES = KBLK * 1024;
  static constexpr int VBYTES = VBLK * 1024;
  static constexpr int STAGE = KBYTES + VBYTES;           // bytes per stage
};

// Direct-to-LDS copies of one wave for one stage. The wave copies blocks w, w + NW, ... of the
// K tile and of the V^T tile (1 KB each, one 16-byte chunk per lane); the per-lane source
// offsets are computed once, so issuing a stage costs a few scalar instructions per copy.
template <int D, int NW>
struct StageCopier {
  using LT = LdsTiles<D>;
  static constexpr int KI = (LT::KBLK + NW - 1) / NW;  // most K blocks per wave
  static constexpr int VI = (LT::VBLK + NW - 1) / NW;  // most V^T blocks per wave
  int wv;
  uint32_t krow[KI];   // tile row (key) of this lane's chunk
  uint32_t kcol[KI];   // byte offset of the chunk within the row (padding chunks copy chunk 0)
  uint32_t voff[VI];   // byte offset within the V^T tile of this (b, h): d * Lp * 2 + chunk * 16

  __device__ __forceinline__ void init(int wave, int lane, int Lp) {
    wv = wave;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int pos = (wv + i * NW) * 64 + lane;  // padded chunk position
      int r = pos / LT::KROW, c = pos % LT::KROW;
      if (c >= LT::KCH) c = 0;
      if (r >= kBN) r = kBN - 1;
      krow[i] = r;
      kcol[i] = c * 16;
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int pos = (wv + i * NW) * 64 + lane;
      int d = pos / LT::VROW, c = pos % LT::VROW;
      if (c >= kBN / 8) c = 0;
      if (d >= D) d = D - 1;
      voff[i] = static_cast<uint32_t>(d) * Lp * 2 + c * 16;
    }
  }

  // this wave's copies per stage
  __device__ __forceinline__ int count() const {
    return LT::KBLK / NW + (wv < LT::KBLK % NW) + LT::VBLK / NW + (wv < LT::VBLK % NW);
  }

  // Copy K rows kbase .. kbase+63 (rows past kmax are clamped to it; their scores are masked)
  // and V^T keys vbase .. vbase+63 into the stage at LDS byte address `lds`.
  __device__ __forceinline__ void issue(uint32_t lds, const bf16_t* Kbh, int kbase, int kmax,
                                        const bf16_t* Vtbh, int vbase) const {
    const bf16_t* kb = Kbh + static_cast<size_t>(kbase) * D;
    const uint32_t lim = static_cast<uint32_t>(kmax - kbase);  // >= 0: kbase <= kmax
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      if (i * NW + NW > LT::KBLK && wv + i * NW >= LT::KBLK) break;
      const uint32_t r = krow[i] < lim ? krow[i] : lim;
      copy16_to_lds(kb, r * (D * 2) + kcol[i], lds + (wv + i * NW) * 1024);
    }
    const bf16_t* vb = Vtbh + vbase;
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      if (i * NW + NW > LT::VBLK && wv + i * NW >= LT::VBLK) break;
      copy16_to_lds(vb, voff[i], lds + LT::KBYTES + (wv + i * NW) * 1024);
    }
  }
};

// X [B*H][L][D] -> X^T [B*H][D][Lp] (Lp = L rounded up to 64, zero padded), so that tiles of 64
// aligned keys read each dim's 64 keys as 128 contiguous bytes (V for the forward, K for the
// backward's dQ). One workgroup per 64-row tile of one (b, h).
template <int D>
__global__ __launch_bounds__(256) void transpose_rows_kernel(const bf16_t* __restrict__ V,
                                                             bf16_t* __restrict__ Vt, int L,
                                                             int Lp,
                                                             const uint32_t* __restrict__ chk) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[kBN * (D + 8)];
  if (layout_rejected(chk)) return;
  const int bh = blockIdx.y;
  const int k0 = blockIdx.x * kBN;
  for (int e = threadIdx.x; e < kBN * D / 8; e += blockDim.x) {
    const int r = e / (D / 8), c = e % (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + r < L) v = *reinterpret_cast<const u32x4*>(V + (static_cast<size_t>(bh) * L + k0 + r) * D + c * 8);
    *reinterpret_cast<u32x4*>(tile + r * (D + 8) + c * 8) = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < D * (kBN / 8); e += blockDim.x) {
    const int d = e / (kBN / 8), c = e % (kBN / 8);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(tile[(c * 8 + 2 * i) * (D + 8) + d]) |
             (static_cast<uint32_t>(tile[(c * 8 + 2 * i + 1) * (D + 8) + d]) << 16);
    *reinterpret_cast<u32x4*>(Vt + (static_cast<size_t>(bh) * D + d) * Lp + k0 + c * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

// S^T of one 64-key tile: blocks kb = 0, 1 (32 keys x 32 queries each) with the permuted key
// order. The two accumulation chains are interleaved so that consecutive MFMAs never depend on
// each other.
template <int D>
__device__ __forceinline__ void score_tile_swz(const char* stage, const QFrag<bf16_t, D>& qf,
                                               f32x16 (&s)[2], int ql, int g) {
  using LT = LdsTiles<D>;
  const char* row0 = stage + (LT::KROW * kperm(ql) + g) * 16;
  const char* row1 = row0 + LT::KROW * 32 * 16;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row0 + kk * 32));
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row1 + kk * 32));
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf.q[kk], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf.q[kk], s[1], 0, 0, 0);
  }
}

// O^T[db] += V^T P^T for one 64-key tile, P^T packed to bf16 in the permuted output layout:
// pb[ks] holds values 8 (ks & 1) .. 8 (ks & 1) + 7 of S^T block ks >> 1. The first NPRE V^T
// operands (in (ks, db) order) were read ahead of time into pre (pv_preload).
template <int D, int VOFF, int NPRE>
__device__ __forceinline__ void pv_swz_packed(const char* stage, const bf16x8 (&pb)[4],
                                              f32x16 (&acc)[D / 32], int ql, int g,
                                              const bf16x8* pre) {
  using LT = LdsTiles<D>;
  const char* vt = stage + VOFF + (LT::VROW * ql + g) * 16;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int i = ks * (D / 32) + db;
      const bf16x8 a = i < NPRE ? pre[i]
                                : __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                                 vt + (db * 32 * LT::VROW + 2 * ks) * 16));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], acc[db], 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void pv_swz_packed(const char* stage, const bf16x8 (&pb)[4],
                                              f32x16 (&acc)[D / 32], int ql, int g) {
  pv_swz_packed<D, LdsTiles<D>::KBYTES, 0>(stage, pb, acc, ql, g, nullptr);
}

// The first NPRE V^T operand reads of pv_swz_packed for a stage, issued early (by a wave that
// is not running MFMAs at the time, so that its LDS reads overlap the other wave's).
template <int D, int VOFF, int NPRE>
__device__ __forceinline__ void pv_preload(const char* stage, bf16x8* pre, int ql, int g) {
  using LT = LdsTiles<D>;
  const char* vt = stage + VOFF + (LT::VROW * ql + g) * 16;
#pragma unroll
  for (int i = 0; i < NPRE; ++i) {
    const int ks = i / (D / 32), db = i % (D / 32);
    pre[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                            vt + (db * 32 * LT::VROW + 2 * ks) * 16));
  }
}

// ---------------------------------------------------------------------------------------------
// Quantised scores: K and Q as MXFP8 (e4m3 codes, one E8M0 scale per 32 dims), S^T = K Q^T on
// the block-scaled fp8 MFMA (32x32x64: each lane holds 32 codes of its row, bytes 0-15 from the
// first 32-dim block of the step and bytes 16-31 from the second; lane group h supplies the
// scale of block h of the step for its row).
//
// Stage layout: 64 code rows of D bytes with one spare 16-byte chunk per row (odd pitch, as for
// the bf16 rows), one 1 KB block holding the 64 keys' scale bytes (D/32 per key, key-major),
// then the V^T tile of the bf16 layout.
template <int D>
struct MxTiles {
  static constexpr int NB = D / 32;                       // scale bytes per row
  static constexpr int KCH = D / 16;                      // 16-byte chunks of one code row
  static constexpr int KROW = KCH + 1;                    // padded code row pitch (chunks)
  static constexpr int KBLK = (kBN * KROW + 63) / 64;     // 1 KB copy blocks of the code rows
  static constexpr int SOFF = KBLK * 1024;                // the scale block
  static constexpr int KBYTES = SOFF + 1024;
  static constexpr int VBLK = LdsTiles<D>::VBLK;
  static constexpr int VBYTES = VBLK * 1024;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int SCH = kBN * NB / 16;               // 16-byte chunks of the tile's scales
};

// Quantised values: V as MXFP8 along the keys, in the tile layout written by moc_mx_quantize_v:
// per 64-key tile, D rows of kVqRow bytes - the row's 64 e4m3 codes (position p of each 32-key
// block holds key p with bits 3 and 4 swapped, so that a lane's 16-byte operand read holds the
// keys of its P^T values), the E8M0 scales of the tile's two 32-key blocks, zero padding. The
// stage takes the tile verbatim after the MX K tile: the 80-byte pitch is 5 chunks (odd), so
// the 16 lanes of a read pass land on distinct bank slots.
constexpr int kVqRow = 80;

template <int D>
struct MxvTiles {
  static constexpr int VOFF = MxTiles<D>::KBYTES;
  static constexpr int VBLK = D * kVqRow / 1024;   // 1 KB copy blocks of the V tile
  static constexpr int STAGE = VOFF + VBLK * 1024;
  static_assert(D * kVqRow % 1024 == 0, "the V tile is a whole number of copy blocks");
};

// Direct-to-LDS copies of one wave for one MX stage: blocks w, w + NW, ... of the code rows and
// scale block (KBLK + 1 blocks) and of the V tile (the bf16 V^T tile, or with QV the quantised
// V tile, which is contiguous in global memory). Code and scale rows are padded to a multiple
// of 64 rows in global memory, so no row is clamped.
template <int D, int NW, bool QV = false>
struct MxStageCopier {
  using MT = MxTiles<D>;
  static constexpr int KB = MT::KBLK + 1;
  static constexpr int VB = QV ? MxvTiles<D>::VBLK : MT::VBLK;
  static constexpr int VO = QV ? MxvTiles<D>::VOFF : MT::KBYTES;
  static constexpr int KI = (KB + NW - 1) / NW;
  static constexpr int VI = (VB + NW - 1) / NW;
  static constexpr int NBASE = KB / NW + VB / NW;  // fewest copies of a wave per stage
  int wv;
  uint32_t koff[KI];   // byte offset within the tile's code rows, or within its scale bytes
  uint32_t voff[VI];

  __device__ __forceinline__ void init(int wave, int lane, int Lp) {
    wv = wave;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int blk = wv + i * NW;
      if (blk < MT::KBLK) {
        const int pos = blk * 64 + lane;
        int r = pos / MT::KROW, c = pos % MT::KROW;
        if (c >= MT::KCH) c = 0;
        if (r >= kBN) r = kBN - 1;
        koff[i] = static_cast<uint32_t>(r * D + c * 16);
      } else {
        koff[i] = static_cast<uint32_t>((lane % MT::SCH) * 16);  // lanes past the scales repeat
      }
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int pos = (wv + i * NW) * 64 + lane;
      if constexpr (QV) {
        voff[i] = static_cast<uint32_t>(pos < VB * 64 ? pos : VB * 64 - 1) * 16;
      } else {
        int d = pos / LdsTiles<D>::VROW, c = pos % LdsTiles<D>::VROW;
        if (c >= kBN / 8) c = 0;
        if (d >= D) d = D - 1;
        voff[i] = static_cast<uint32_t>(d) * Lp * 2 + c * 16;
      }
    }
  }

  __device__ __forceinline__ int count() const {
    return KB / NW + (wv < KB % NW) + VB / NW + (wv < VB % NW);
  }

  // codes/scales of keys kbase .. kbase+63, and the V tile of those keys: V^T keys vbase ..
  // vbase+63 of vsrc (bf16 V^T of this (b, h)), or with QV the tile that starts at vsrc
  __device__ __forceinline__ void issue(uint32_t lds, const uint8_t* Kc, const uint8_t* Ks,
                                        int kbase, const void* vsrc, int vbase) const {
    const uint8_t* kc = Kc + static_cast<size_t>(kbase) * D;
    const uint8_t* ks = Ks + static_cast<size_t>(kbase) * MT::NB;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int blk = wv + i * NW;
      if (i * NW + NW > KB && blk >= KB) break;
      if (blk < MT::KBLK) copy16_to_lds(kc, koff[i], lds + blk * 1024);
      else copy16_to_lds(ks, koff[i], lds + blk * 1024);
    }
    const void* vb = QV ? vsrc : static_cast<const void*>(static_cast<const bf16_t*>(vsrc) + vbase);
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      if (i * NW + NW > VB && wv + i * NW >= VB) break;
      copy16_to_lds(vb, voff[i], lds + VO + (wv + i * NW) * 1024);
    }
  }
};

typedef __attribute__((ext_vector_type(8))) int i32x8;

// The B operand (Q^T) of the scaled fp8 score MFMA for one query row: per 64-dim step m, the
// lane's 32 codes (dims 64m + 16g .. +15 and 64m + 32 + 16g .. +15), and the row's scale codes
// shifted so that byte 2m holds the scale of block 2m + g.
template <int D>
struct MxQFrag {
  static constexpr int NM = D / 64;
  i32x8 q[NM];
  uint32_t sc;
  __device__ __forceinline__ void load(const uint8_t* __restrict__ row,
                                       const uint8_t* __restrict__ srow, int g) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 64 * m + 16 * g);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 64 * m + 32 + 16 * g);
      q[m] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                   static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                   static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    }
    if constexpr (D == 128) sc = *reinterpret_cast<const uint32_t*>(srow) >> (8 * g);
    else sc = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(srow)) >> (8 * g);
  }
};

// one block-scaled fp8 MFMA (e4m3 x e4m3); OP selects the scale byte of both operands
template <int OP>
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, const f32x16& c,
                                          uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OP, static_cast<int>(sa),
                                                         OP, static_cast<int>(sb));
}

// S^T of one 64-key tile from an MX stage (blocks kb = 0, 1; the permuted key order of the bf16
// tiles)
template <int D>
__device__ __forceinline__ void score_tile_mx(const char* stage, const MxQFrag<D>& qf,
                                             f32x16 (&s)[2], int ql, int g) {
  using MT = MxTiles<D>;
  const int k0 = kperm(ql), k1 = 32 + kperm(ql);
  const char* row0 = stage + MT::KROW * k0 * 16;
  const char* row1 = stage + MT::KROW * k1 * 16;
  uint32_t sa0, sa1;
  if constexpr (D == 128) {
    sa0 = *reinterpret_cast<const uint32_t*>(stage + MT::SOFF + 4 * k0) >> (8 * g);
    sa1 = *reinterpret_cast<const uint32_t*>(stage + MT::SOFF + 4 * k1) >> (8 * g);
  } else {
    sa0 = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(stage + MT::SOFF + 2 * k0)) >> (8 * g);
    sa1 = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(stage + MT::SOFF + 2 * k1)) >> (8 * g);
  }
  auto arow = [&](const char* row, int m) __attribute__((always_inline)) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + (4 * m + g) * 16);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + (4 * m + 2 + g) * 16);
    return i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                 static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                 static_cast<int>(hi[2]), static_cast<int>(hi[3])};
  };
  s[0] = f32x16{};
  s[1] = f32x16{};
  s[0] = mfma_mx<0>(arow(row0, 0), qf.q[0], s[0], sa0, qf.sc);
  s[1] = mfma_mx<0>(arow(row1, 0), qf.q[0], s[1], sa1, qf.sc);
  if constexpr (D == 128) {
    s[0] = mfma_mx<2>(arow(row0, 1), qf.q[1], s[0], sa0, qf.sc);
    s[1] = mfma_mx<2>(arow(row1, 1), qf.q[1], s[1], sa1, qf.sc);
  }
}

// O^T[db] += V^T P^T for one 64-key tile on the block-scaled fp8 MFMA: A = the quantised V tile
// (row d = 32 db + ql; lane group g reads bytes 16 g .. +15 and 32 + 16 g .. +15, and the scale
// byte of block g of the row), B = P^T as e4m3 codes (pb bytes 0-15: values 0-15 of S^T block
// 0, bytes 16-31: of block 1; those are the keys that the swapped positions of the V rows
// hold), with unit scale. Three LDS reads per MFMA.
template <int D, int VOFF>
__device__ __forceinline__ void pv_mxv(const char* stage, const i32x8& pb,
                                       f32x16 (&acc)[D / 32], int ql, int g) {
  const char* vrow = stage + VOFF + ql * kVqRow;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const char* r = vrow + db * 32 * kVqRow;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + 16 * g);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + 32 + 16 * g);
    const uint32_t sa = *reinterpret_cast<const uint32_t*>(r + 64) >> (8 * g);
    const i32x8 a = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]),
                          static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                          static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                          static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    acc[db] = mfma_mx<0>(a, pb, acc[db], sa, 127u);
  }
}

// Operand reads consumed up to and including MFMA i of an MFMA half-step: NPV P.V MFMAs of PVR
// reads each, the first NPRE reads of them preloaded, then the score MFMAs, SFIRST reads before
// the first of them and SREADS per MFMA.
constexpr int half_step_reads(int i, int npv, int npre, int sfirst, int sreads, int pvr = 1) {
  return i < npv ? ((i + 1) * pvr - npre > 0 ? (i + 1) * pvr - npre : 0)
                 : (npv * pvr - npre) + sfirst + sreads * (i - npv + 1);
}

// sched_group_barrier pattern that keeps the reads A ahead of the MFMAs that consume them: before
// MFMA i, the reads of MFMAs up to i plus A more are issued (all NR at the end).
template <int NM, int NR, int A, int NPV, int NPRE, int SFIRST, int SREADS, int PVR = 1, int I = 0>
__device__ __forceinline__ void sched_lead_reads() {
  static_assert(half_step_reads(NM - 1, NPV, NPRE, SFIRST, SREADS, PVR) == NR,
                "the read count of the half-step does not match its MFMAs");
  if constexpr (I < NM) {
    constexpr int want = half_step_reads(I, NPV, NPRE, SFIRST, SREADS, PVR) + A;
    constexpr int prev_want =
        I == 0 ? 0 : half_step_reads(I - 1, NPV, NPRE, SFIRST, SREADS, PVR) + A;
    constexpr int cur = want < NR ? want : NR;
    constexpr int prev = prev_want < NR ? prev_want : NR;
    if constexpr (cur > prev) __builtin_amdgcn_sched_group_barrier(0x100, cur - prev, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_lead_reads<NM, NR, A, NPV, NPRE, SFIRST, SREADS, PVR, I + 1>();
  }
}

}  // namespace moc
