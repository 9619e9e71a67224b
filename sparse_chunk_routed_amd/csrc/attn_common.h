// Building blocks shared by the attention kernels: MFMA fragments, LDS tile staging.
//
// Formulation ("transposed" flash attention): per 32-query block we compute
//   S^T = K Q^T   (MFMA A = a 32-key slice of K from LDS, B = Q^T fragment in registers)
//   O^T += V^T P^T (MFMA A = V^T slice from a transposed LDS tile, B = P^T straight from the
//                   S^T accumulator registers)
// With the 32x32 MFMA output layout every lane holds values of ONE query (lane % 32) and 16
// keys / dims of a 32-block, so the online softmax needs a single cross-lane exchange (lanes l
// and l^32) per tile and the rescale of O is lane-local. A wave owns QB query blocks, so each
// K / V^T fragment read from LDS feeds QB MFMAs.
//
// gfx950 MFMA layouts used (wave64, 32x32 output):
//   v_mfma_f32_32x32x16_bf16: A[m][k] lane l holds m = l%32, k = 8*(l/32)+0..7;
//                             B[k][n] lane l holds n = l%32, k = 8*(l/32)+0..7;
//   v_mfma_f32_32x32x2_f32:   A lane l holds m = l%32, k = l/32; B lane l holds n = l%32, k = l/32;
//   output D[m][n], 16 floats per lane: n = l%32, m = 8*(i/4) + 4*(l/32) + (i%4), i = 0..15.
// Any permutation of the contraction index applied to both A and B gives the same product;
// the P^T operand uses the output layout's key order directly and V^T is read in that order.
#pragma once

#include "moc_common.h"

namespace moc {

constexpr int kBN = 64;  // keys per tile

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

template <typename T, int D, int NT = 256>
struct Tiles;

// bf16: K tile [64][D+8], V^T tile [D][64+4] (row strides chosen for conflict-free reads:
// 16-byte K reads by 16 consecutive rows, 8-byte V^T reads by 32 consecutive dims).
// NT threads cooperate in staging a tile.
template <int D, int NT>
struct Tiles<bf16_t, D, NT> {
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = kBN + 4;
  static constexpr int KK = D / 16;         // MFMA k-steps over d for S^T
  static constexpr int VEC = 8;             // elements per 16-byte vector
  static constexpr int TPR = D / VEC;       // threads per K row
  static constexpr int KRP = NT / TPR;      // K rows per pass
  static constexpr int KV = kBN / KRP;      // K vectors per thread
  static constexpr int DG = D / VEC;        // V dim groups
  // threads per dim group (each stages whole key pairs; 32 pairs per 64-key tile)
  static constexpr int TPD = (NT / DG) < (kBN / 2) ? (NT / DG) : (kBN / 2);
  static constexpr int VV = kBN / TPD;      // V vectors (rows) per thread, in pairs
  static constexpr int VACT = DG * TPD;     // threads that stage V
  static constexpr int STAGE = kBN * KSTR + D * VSTR;  // elements of one K + V^T stage
  static_assert(VV >= 2 && VV % 2 == 0, "V rows are staged in key pairs");
  static_assert(KV >= 1 && KRP * KV == kBN, "K tile split");
};

template <int D, int NT>
struct Tiles<float, D, NT> {
  static constexpr int KSTR = D + 1;
  static constexpr int VSTR = kBN + 1;
  static constexpr int KK = D / 2;
  static constexpr int VEC = 4;
  static constexpr int TPR = D / VEC;
  static constexpr int KRP = NT / TPR;
  static constexpr int KV = kBN / KRP;
  static constexpr int DG = D / VEC;
  static constexpr int TPD = (NT / DG) < kBN ? (NT / DG) : kBN;
  static constexpr int VV = kBN / TPD;
  static constexpr int VACT = DG * TPD;
  static constexpr int STAGE = kBN * KSTR + D * VSTR;
  static_assert(KV >= 1 && KRP * KV == kBN, "K tile split");
};

// Registers holding one K tile and one V tile between the global load and the LDS store
// (NT threads cooperate).
template <typename T, int D, int NT = 256>
struct TileRegs {
  using TL = Tiles<T, D, NT>;
  u32x4 k[TL::KV];
  u32x4 v[TL::VV];

  // rows key0 .. key0+63 of the (b,h) slab; rows at or beyond kend read as zero
  __device__ __forceinline__ void load(const T* __restrict__ Kbh, const T* __restrict__ Vbh,
                                       int key0, int kend) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < TL::KV; ++j) {
      const int idx = tid + j * NT;
      const int row = idx / TL::TPR, col = idx % TL::TPR;
      const int key = key0 + row;
      k[j] = key < kend ? *reinterpret_cast<const u32x4*>(Kbh + static_cast<size_t>(key) * D + col * TL::VEC)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    if (TL::VACT < NT && tid >= TL::VACT) return;
    const int dg = tid / TL::TPD, r0 = tid % TL::TPD;
#pragma unroll
    for (int j = 0; j < TL::VV; ++j) {
      const int row = v_row(r0, j);
      const int key = key0 + row;
      v[j] = key < kend ? *reinterpret_cast<const u32x4*>(Vbh + static_cast<size_t>(key) * D + dg * TL::VEC)
                        : u32x4{0u, 0u, 0u, 0u};
    }
  }

  __device__ __forceinline__ static int v_row(int r0, int j) {
    if constexpr (sizeof(T) == 2) {
      return 2 * (r0 + (j >> 1) * TL::TPD) + (j & 1);  // key pairs (2kp, 2kp+1)
    } else {
      return r0 + j * TL::TPD;
    }
  }

  __device__ __forceinline__ void store(T* Ks, T* Vt) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < TL::KV; ++j) {
      const int idx = tid + j * NT;
      const int row = idx / TL::TPR, col = idx % TL::TPR;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(Ks + row * TL::KSTR + col * TL::VEC) = k[j];
      } else {
        float* dst = reinterpret_cast<float*>(Ks) + row * TL::KSTR + col * TL::VEC;
        dst[0] = __uint_as_float(k[j].x); dst[1] = __uint_as_float(k[j].y);
        dst[2] = __uint_as_float(k[j].z); dst[3] = __uint_as_float(k[j].w);
      }
    }
    if (TL::VACT < NT && tid >= TL::VACT) return;
    const int dg = tid / TL::TPD, r0 = tid % TL::TPD;
    if constexpr (sizeof(T) == 2) {
      uint32_t* vt = reinterpret_cast<uint32_t*>(Vt);
#pragma unroll
      for (int jp = 0; jp < TL::VV / 2; ++jp) {
        const int kp = r0 + jp * TL::TPD;
        const u32x4 a = v[2 * jp], b = v[2 * jp + 1];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t aw = a[w], bw = b[w];
          // dims dg*8 + 2w (low halves) and dg*8 + 2w + 1 (high halves), keys 2kp, 2kp+1
          vt[((dg * 8 + 2 * w) * TL::VSTR) / 2 + kp] = (aw & 0xffffu) | (bw << 16);
          vt[((dg * 8 + 2 * w + 1) * TL::VSTR) / 2 + kp] = (aw >> 16) | (bw & 0xffff0000u);
        }
      }
    } else {
      float* vt = reinterpret_cast<float*>(Vt);
#pragma unroll
      for (int j = 0; j < TL::VV; ++j) {
        const int row = v_row(r0, j);
#pragma unroll
        for (int w = 0; w < 4; ++w) vt[(dg * 4 + w) * TL::VSTR + row] = __uint_as_float(v[j][w]);
      }
    }
  }
};

// Q^T fragment of the lane's query (B operand of S^T = K Q^T).
template <typename T, int D>
struct QFrag;

template <int D>
struct QFrag<bf16_t, D> {
  bf16x8 q[D / 16];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ qrow, int g) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      q[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * g));
  }
};

template <int D>
struct QFrag<float, D> {
  float q[D / 2];
  __device__ __forceinline__ void load(const float* __restrict__ qrow, int g) {
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) q[kk] = qrow[2 * kk + g];
  }
};

// S^T blocks (32 keys of block kb x 32 queries) for QB query blocks; each K fragment read
// from LDS feeds QB MFMAs.
template <int D, int QB>
__device__ __forceinline__ void score_blocks(const bf16_t* Ks, const QFrag<bf16_t, D> (&qf)[QB],
                                             int kb, int ql, int g, f32x16 (&s)[QB]) {
  using TL = Tiles<bf16_t, D>;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
  const bf16_t* kr = Ks + (kb * 32 + ql) * TL::KSTR + 8 * g;
#pragma unroll
  for (int kk = 0; kk < TL::KK; ++kk) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * kk));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb].q[kk], s[qb], 0, 0, 0);
  }
}

template <int D, int QB>
__device__ __forceinline__ void score_blocks(const float* Ks, const QFrag<float, D> (&qf)[QB],
                                             int kb, int ql, int g, f32x16 (&s)[QB]) {
  using TL = Tiles<float, D>;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
  const float* kr = Ks + (kb * 32 + ql) * TL::KSTR + g;
#pragma unroll
  for (int kk = 0; kk < TL::KK; ++kk) {
    const float a = kr[2 * kk];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[qb].q[kk], s[qb], 0, 0, 0);
  }
}

// Key (within the 64-key tile) of output value i of block kb for lane group g.
__device__ __forceinline__ int key_of(int kb, int i, int g) {
  return kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
}

// O^T[qb][db] += V^T[db-block] P^T[qb] for one 64-key tile. p[qb][kb] holds P^T in the S^T
// output layout (fp32); it is converted to bf16 per 16-key step.
template <int D, int QB>
__device__ __forceinline__ void pv_accumulate(const bf16_t* Vt, const f32x16 (&p)[QB][2],
                                              f32x16 (&acc)[QB][D / 32], int ql, int g) {
  using TL = Tiles<bf16_t, D>;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kb = ks >> 1, hh = ks & 1;
    bf16x8 pb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) pb[qb][ii] = static_cast<__bf16>(p[qb][kb][8 * hh + ii]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16_t* vr = Vt + (db * 32 + ql) * TL::VSTR + kb * 32 + 16 * hh + 4 * g;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], acc[qb][db], 0, 0, 0);
    }
  }
}

template <int D, int QB>
__device__ __forceinline__ void pv_accumulate(const float* Vt, const f32x16 (&p)[QB][2],
                                              f32x16 (&acc)[QB][D / 32], int ql, int g) {
  using TL = Tiles<float, D>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int key = key_of(kb, ii, g);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float a = Vt[(db * 32 + ql) * TL::VSTR + key];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[qb][kb][ii], acc[qb][db], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling threshold (log2 units): the reference max of the online softmax is only moved
// when a tile's max exceeds it by more than this, so P stays below 2^kRescale.
constexpr float kRescale = 8.0f;

}  // namespace moc
