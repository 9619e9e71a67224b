// K4: MoC attention forward over the routed key sets.
//
// Source: "Mixture of Contexts for Long Video Generation | Summary" §3.1 (attention of q_i over
// the keys/values of its routed set, softmax(q K_Omega^T / sqrt(d)) V_Omega), §3.2 (every query
// also attends all caption tokens and its own shot); jxzklqfsx.com write-up, sections
// 固定的跨模態選擇 / 固定的鏡頭內選擇 and 計算效率 (prior art: one variable-length
// flash-attention call over packed (query, key) groups - replaced here by two block-sparse
// kernels).
//
// Omega(t) = text range U own-shot range U routed chunks, which are disjoint, so the softmax
// over Omega is the log-sum-exp merge of independent partial softmaxes:
//   K4a (routed): one workgroup per tile of <= 128 queries gathered from one (b, h, chunk)
//        bucket; the chunk's K/V are streamed once per tile; writes a normalised partial
//        output row and its LSE for each (query, routed chunk) into the workspace.
//   K4b (anchor): one workgroup per tile of <= 128 consecutive queries of one shot (or the
//        text); streams text keys then own-shot keys; the epilogue merges the query's routed
//        partials in ascending chunk order (deterministic) and writes O and LSE.
// Both are exp2-domain online-softmax flash loops on MFMA (see attn_common.h), 4 waves x 32
// queries, 64-key tiles staged through LDS with the next tile's global loads in flight.
#include "attn_common.h"

namespace moc {

constexpr int kBM = 128;  // queries per workgroup

struct AttnParams {
  int B, H, L, C, S;
  int max_tiles;
  float scale_log2;  // softmax_scale * log2(e)
};

enum { MODE_ANCHOR = 0, MODE_ROUTED = 1 };

template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ off, AttnParams p, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ bucket_off,
    const int32_t* __restrict__ bucket_q, const int32_t* __restrict__ slot,
    float* __restrict__ pO, float* __restrict__ plse, T* __restrict__ O,
    float* __restrict__ lse) {
  using TL = Tiles<T, D>;
  __shared__ __attribute__((aligned(16))) T lds[TL::LDS_ELEMS];
  T* Ks = lds;
  T* Vt = lds + kBN * TL::KSTR;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, q_lo, nq;            // tile queries: bucket positions or consecutive tokens
  int r1a, r1b, r2a, r2b;      // key ranges
  int bstart = 0;
  if constexpr (MODE == MODE_ANCHOR) {
    bh = lid / p.max_tiles;
    const int tile = lid % p.max_tiles;
    if (tile >= n_tiles[0]) return;
    const int32_t* a = tiles + 6 * tile;
    q_lo = a[0];
    nq = a[1] - a[0];
    r1a = a[2]; r1b = a[3]; r2a = a[4]; r2b = a[5];
  } else {
    if (lid >= n_tiles[0]) return;
    const int bucket = tiles[2 * lid];
    const int start = tiles[2 * lid + 1];
    bh = bucket / p.C;
    const int c = bucket % p.C;
    bstart = bucket_off[bucket] + start;
    const int rem = bucket_off[bucket + 1] - bstart;
    nq = rem < kBM ? rem : kBM;
    q_lo = 0;
    r1a = off[c]; r1b = off[c + 1]; r2a = 0; r2b = 0;
  }

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int r = wv * 32 + ql;   // query row within the tile
  const bool valid = r < nq;
  int t;
  if constexpr (MODE == MODE_ANCHOR) {
    t = q_lo + (valid ? r : nq - 1);
  } else {
    t = bucket_q[bstart + (valid ? r : nq - 1)];
  }

  const size_t bh_off = static_cast<size_t>(bh) * p.L * D;
  const T* Kbh = K + bh_off;
  const T* Vbh = V + bh_off;
  QFrag<T, D> qf;
  qf.load(Q + bh_off + static_cast<size_t>(t) * D, g);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m = -__builtin_inff();
  float lsum = 0.f;

  const int n1 = (r1b - r1a + kBN - 1) / kBN;
  const int n2 = (r2b - r2a + kBN - 1) / kBN;
  const int ntot = n1 + n2;

  TileRegs<T, D> regs;
  auto tile_pos = [&](int j, int& key0, int& kend) {
    if (j < n1) { key0 = r1a + j * kBN; kend = r1b; }
    else { key0 = r2a + (j - n1) * kBN; kend = r2b; }
  };
  {
    int key0, kend;
    tile_pos(0, key0, kend);
    regs.load(Kbh, Vbh, key0, kend);
    regs.store(Ks, Vt);
  }
  __syncthreads();

  for (int j = 0; j < ntot; ++j) {
    int key0, kend;
    tile_pos(j, key0, kend);
    const bool has_next = j + 1 < ntot;
    if (has_next) {
      int nk0, nke;
      tile_pos(j + 1, nk0, nke);
      regs.load(Kbh, Vbh, nk0, nke);
    }
    f32x16 s[2];
    s[0] = score_block<D>(Ks, qf, 0, ql, g);
    s[1] = score_block<D>(Ks, qf, 1, ql, g);
    const int nvalid = kend - key0;  // keys at or beyond nvalid are masked
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[kb][i] * p.scale_log2;
        x = key_of(kb, i, g) < nvalid ? x : -__builtin_inff();
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(s[kb][i] - m);
        s[kb][i] = pv;
        lsum += pv;
      }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    pv_accumulate<D>(Vt, s, acc, ql, g);
    __syncthreads();
    if (has_next) {
      regs.store(Ks, Vt);
      __syncthreads();
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / ltot;
  float lse2 = m + fast_log2(ltot);  // base-2 log-sum-exp of the scaled scores
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] *= inv;

  if (!valid) return;
  if constexpr (MODE == MODE_ROUTED) {
    const size_t pos = static_cast<size_t>(bstart) + r;
    float* prow = pO + pos * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 v = {acc[db][4 * jj + 0], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]};
        *reinterpret_cast<f32x4*>(prow + db * 32 + 8 * jj + 4 * g) = v;
      }
    if (g == 0) plse[pos] = lse2;  // kept in base 2 inside the workspace
  } else {
    const size_t row = static_cast<size_t>(bh) * p.L + t;
    const int32_t* sl = slot + row * p.S;
    float M = lse2, wsum = 1.f;
    for (int j = 0; j < p.S; ++j) {
      const int pos = sl[j];
      if (pos < 0) break;
      const float lj = plse[pos];
      const float Mn = fmaxf(M, lj);
      const float so = fast_exp2(M - Mn), sn = fast_exp2(lj - Mn);
      const float* prow = pO + static_cast<size_t>(pos) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(prow + db * 32 + 8 * jj + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * jj + e] = acc[db][4 * jj + e] * so + v[e] * sn;
        }
      wsum = wsum * so + sn;
      M = Mn;
    }
    const float winv = 1.f / wsum;
    T* orow = O + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        T* dst = orow + db * 32 + 8 * jj + 4 * g;
        if constexpr (sizeof(T) == 2) {
          uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 0] * winv)) |
                        (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 1] * winv)) << 16);
          uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 2] * winv)) |
                        (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 3] * winv)) << 16);
          *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{acc[db][4 * jj + 0] * winv, acc[db][4 * jj + 1] * winv,
                                                 acc[db][4 * jj + 2] * winv, acc[db][4 * jj + 3] * winv};
        }
      }
    if (g == 0) lse[row] = (M + fast_log2(wsum)) * kLn2;
  }
}

}  // namespace moc

namespace moc_host {

using moc::AttnParams;

template <typename T, int D>
static hipError_t launch_fwd_t(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                               const void* K, const void* V, float scale, void* O, float* lse,
                               float* pO, float* plse, hipStream_t st) {
  AttnParams p;
  p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = vl->S;
  p.scale_log2 = scale * moc::kLog2e;
  const T* q = static_cast<const T*>(Q);
  const T* k = static_cast<const T*>(K);
  const T* v = static_cast<const T*>(V);
  if (vl->S > 0 && vl->max_rtiles > 0) {
    p.max_tiles = vl->max_rtiles;
    hipLaunchKernelGGL((moc::attn_fwd_kernel<T, D, moc::MODE_ROUTED>), dim3(vl->max_rtiles),
                       dim3(256), 0, st, q, k, v, lay->chunk_offsets, p, vl->rtiles,
                       vl->n_rtiles, vl->bucket_off, vl->bucket_q, vl->slot, pO, plse,
                       static_cast<T*>(O), lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  p.max_tiles = vl->max_atiles;
  hipLaunchKernelGGL((moc::attn_fwd_kernel<T, D, moc::MODE_ANCHOR>),
                     dim3(vl->max_atiles * lay->B * lay->H), dim3(256), 0, st, q, k, v,
                     lay->chunk_offsets, p, vl->atiles, vl->n_atiles, vl->bucket_off,
                     vl->bucket_q, vl->slot, pO, plse, static_cast<T*>(O), lse);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                           const void* K, const void* V, float scale, void* O, float* lse,
                           float* pO, float* plse, hipStream_t st) {
  if (lay->dtype == MOC_BF16)
    return lay->d == 128 ? launch_fwd_t<moc::bf16_t, 128>(lay, vl, Q, K, V, scale, O, lse, pO, plse, st)
                         : launch_fwd_t<moc::bf16_t, 64>(lay, vl, Q, K, V, scale, O, lse, pO, plse, st);
  return lay->d == 128 ? launch_fwd_t<float, 128>(lay, vl, Q, K, V, scale, O, lse, pO, plse, st)
                       : launch_fwd_t<float, 64>(lay, vl, Q, K, V, scale, O, lse, pO, plse, st);
}

}  // namespace moc_host
