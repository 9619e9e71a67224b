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
//   K4a (routed): one workgroup per tile of <= 256 queries gathered from one (b, h, chunk)
//        bucket; the chunk's K/V are streamed once per tile; writes a normalised partial
//        output row and its base-2 LSE for each (query, routed chunk) into the workspace.
//   K4b (anchor): one workgroup per tile of <= 256 consecutive queries of one shot (or the
//        text); streams text keys then own-shot keys; the epilogue merges the query's routed
//        partials in ascending chunk order (deterministic) and writes O and LSE.
// Both are exp2-domain online-softmax flash loops on MFMA (S^T = K Q^T, O^T += V^T P^T; a lane
// owns one query), 8 waves x 32 queries per workgroup, 64-key tiles, lazy rescaling of the
// running max (only when it grows by more than 2^8). The bf16 kernel runs its two wave groups
// half a tile apart so that one group's MFMAs overlap the other group's softmax, with K and
// V^T tiles copied global -> LDS without registers into four rotating stages (attn_fwd_lds.h);
// with MXFP8 codes for Q and K (quantised scores) S runs on the block-scaled fp8 MFMA. The fp32
// kernel stages tiles through registers into a double-buffered LDS ring.
#include <type_traits>

#include "attn_common.h"
#include "attn_fwd_lds.h"

namespace moc {

#ifndef MOC_ATTN_QB
#define MOC_ATTN_QB 1
#endif
#ifndef MOC_ATTN_NW
#define MOC_ATTN_NW 8
#endif
constexpr int kQB = MOC_ATTN_QB;       // 32-query blocks per wave
constexpr int kNW = MOC_ATTN_NW;       // waves per workgroup
constexpr int kNT = 64 * kNW;          // threads per workgroup
constexpr int kBM = kNW * 32 * kQB;    // queries per workgroup
#ifndef MOC_ATTN_RA
#define MOC_ATTN_RA 4
#endif
constexpr int kReadAhead = MOC_ATTN_RA;  // LDS operand reads in flight ahead of the MFMAs
#ifndef MOC_ATTN_PRE
#define MOC_ATTN_PRE 4
#endif
// V^T operands of a wave's next MFMA half-step read during its softmax half-step
constexpr int kPre = MOC_ATTN_PRE;

struct AttnParams {
  int B, H, L, C, S;
  int max_tiles;
  float scale_log2;  // softmax_scale * log2(e)
  const uint32_t* chk;  // layout check word (moc_layout.check) or NULL
};

enum { MODE_ANCHOR = 0, MODE_ROUTED = 1 };

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kNT) void attn_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ off, AttnParams p, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ bucket_off,
    const int32_t* __restrict__ bucket_q, const int32_t* __restrict__ slot,
    float* __restrict__ pO, float* __restrict__ plse, T* __restrict__ O,
    float* __restrict__ lse) {
  using TL = Tiles<T, D, kNT>;
  constexpr int QB = kQB;
  __shared__ __attribute__((aligned(16))) T lds[2 * TL::STAGE];
  if (layout_rejected(p.chk)) return;

  // The grid is an upper bound of the work list (its length lives on the device): blocks
  // past the real count exit, and the rest are remapped so that each XCD takes a contiguous
  // range of the real work items.
  int bh, q_lo, nq;            // tile queries: bucket positions or consecutive tokens
  int r1a, r1b, r2a, r2b;      // key ranges
  int bstart = 0;
  if constexpr (MODE == MODE_ANCHOR) {
    const int nt = n_tiles[0];
    const int nwork = nt * p.B * p.H;
    if (static_cast<int>(blockIdx.x) >= nwork) return;
    const int lid = xcd_remap(blockIdx.x, nwork);
    bh = lid / nt;
    const int tile = lid % nt;
    const int32_t* a = tiles + 6 * tile;
    q_lo = a[0];
    nq = a[1] - a[0];
    r1a = a[2]; r1b = a[3]; r2a = a[4]; r2b = a[5];
  } else {
    const int nwork = n_tiles[0];
    if (static_cast<int>(blockIdx.x) >= nwork) return;
    const int lid = xcd_remap(blockIdx.x, nwork);
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
  int rows[QB];
  int tok[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    rows[qb] = wv * 32 * QB + qb * 32 + ql;
    const int rr = rows[qb] < nq ? rows[qb] : nq - 1;
    if constexpr (MODE == MODE_ANCHOR) tok[qb] = q_lo + rr;
    else tok[qb] = bucket_q[bstart + rr];
  }

  const size_t bh_off = static_cast<size_t>(bh) * p.L * D;
  const T* Kbh = K + bh_off;
  const T* Vbh = V + bh_off;
  QFrag<T, D> qf[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qf[qb].load(Q + bh_off + static_cast<size_t>(tok[qb]) * D, g);

  f32x16 acc[QB][D / 32];
  float m_ref[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[qb][db] = f32x16{};
    m_ref[qb] = -__builtin_inff();
    lsum[qb] = 0.f;
  }
  const float c2 = p.scale_log2;

  const int n1 = (r1b - r1a + kBN - 1) / kBN;
  const int n2 = (r2b - r2a + kBN - 1) / kBN;
  const int ntot = n1 + n2;
  auto tile_pos = [&](int j, int& key0, int& kend) __attribute__((always_inline)) {
    if (j < n1) { key0 = r1a + j * kBN; kend = r1b; }
    else { key0 = r2a + (j - n1) * kBN; kend = r2b; }
  };

  TileRegs<T, D, kNT> regs;
  {
    int key0, kend;
    tile_pos(0, key0, kend);
    regs.load(Kbh, Vbh, key0, kend);
    regs.store(lds, lds + kBN * TL::KSTR);
    if (ntot > 1) {
      tile_pos(1, key0, kend);
      regs.load(Kbh, Vbh, key0, kend);
    }
  }
  __syncthreads();

  for (int j = 0; j < ntot; ++j) {
    T* cur = lds + (j & 1) * TL::STAGE;
    if (j + 1 < ntot) {
      T* nxt = lds + ((j + 1) & 1) * TL::STAGE;
      regs.store(nxt, nxt + kBN * TL::KSTR);
    }
    if (j + 2 < ntot) {
      int key0, kend;
      tile_pos(j + 2, key0, kend);
      regs.load(Kbh, Vbh, key0, kend);
    }
    const T* Ks = cur;
    const T* Vt = cur + kBN * TL::KSTR;

    f32x16 s[QB][2];
    {
      f32x16 s0[QB], s1[QB];
      score_blocks<D, QB>(Ks, qf, 0, ql, g, s0);
      score_blocks<D, QB>(Ks, qf, 1, ql, g, s1);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) { s[qb][0] = s0[qb]; s[qb][1] = s1[qb]; }
    }
    int key0, kend;
    tile_pos(j, key0, kend);
    const int nvalid = kend - key0;
    if (nvalid < kBN) {  // ragged last tile of a range: mask keys past its end
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (key_of(kb, i, g) >= nvalid) s[qb][kb][i] = -__builtin_inff();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
      // move the reference max only when this tile exceeds it by more than 2^kRescale
      if (__builtin_amdgcn_ballot_w64(mx > m_ref[qb] + kRescale)) {
        const float m_new = fmaxf(m_ref[qb], mx);
        const float alpha = fast_exp2(m_ref[qb] - m_new);
        m_ref[qb] = m_new;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[qb][db] *= alpha;
      }
      const float neg = -m_ref[qb];
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(s[qb][0][i], c2, neg));
        const float p1 = fast_exp2(__builtin_fmaf(s[qb][1][i], c2, neg));
        s[qb][0][i] = p0;
        s[qb][1][i] = p1;
        l0 += p0;
        l1 += p1;
      }
      lsum[qb] += l0 + l1;
    }
    pv_accumulate<D, QB>(Vt, s, acc, ql, g);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const float inv = 1.f / ltot;
    const float lse2 = m_ref[qb] + fast_log2(ltot);  // base-2 log-sum-exp of the scaled scores
    const int r = rows[qb];
    if (r >= nq) continue;
    if constexpr (MODE == MODE_ROUTED) {
      const size_t pos = static_cast<size_t>(bstart) + r;
      float* prow = pO + pos * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 v = {acc[qb][db][4 * jj + 0] * inv, acc[qb][db][4 * jj + 1] * inv,
                           acc[qb][db][4 * jj + 2] * inv, acc[qb][db][4 * jj + 3] * inv};
          *reinterpret_cast<f32x4*>(prow + db * 32 + 8 * jj + 4 * g) = v;
        }
      if (g == 0) plse[pos] = lse2;  // kept in base 2 inside the workspace
    } else {
      const int t = tok[qb];
      const size_t row = static_cast<size_t>(bh) * p.L + t;
      const int32_t* sl = slot + row * p.S;
      f32x16 (&o)[D / 32] = acc[qb];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= inv;
      float M = lse2, wsum = 1.f;
      for (int jsl = 0; jsl < p.S; ++jsl) {
        const int pos = sl[jsl];
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
            for (int e = 0; e < 4; ++e) o[db][4 * jj + e] = o[db][4 * jj + e] * so + v[e] * sn;
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
            const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(o[db][4 * jj + 0] * winv)) |
                                (static_cast<uint32_t>(f32_to_bf16(o[db][4 * jj + 1] * winv)) << 16);
            const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(o[db][4 * jj + 2] * winv)) |
                                (static_cast<uint32_t>(f32_to_bf16(o[db][4 * jj + 3] * winv)) << 16);
            *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{o[db][4 * jj + 0] * winv, o[db][4 * jj + 1] * winv,
                                                   o[db][4 * jj + 2] * winv, o[db][4 * jj + 3] * winv};
          }
        }
      if (g == 0) lse[row] = (M + fast_log2(wsum)) * kLn2;
    }
  }
}


// Operand formats of the LDS-staged forward: bf16 Q, K, V; MXFP8 Q and K (quantised scores);
// MXFP8 Q, K and V (quantised scores and values).
enum { QNT_NONE = 0, QNT_SCORES = 1, QNT_VALUES = 2 };

// bf16 attention forward: same work decomposition and epilogue as attn_fwd_kernel; two wave
// groups half a tile apart, K and V^T tiles staged by direct-to-LDS copies into padded
// 64-key-aligned tiles (four rotating stages) and the permuted key order of attn_fwd_lds.h.
// QNT_SCORES: Q and K are MXFP8 codes and scales (rows padded to Lp), S on the block-scaled fp8
// MFMA. QNT_VALUES: also V, as the quantised tiles of moc_mx_quantize_v (Vt points at them),
// and P.V on the block-scaled fp8 MFMA with P^T rounded to e4m3.
template <int D, int MODE, int QNT>
__device__ __forceinline__ void attn_fwd_lds_body(
    const void* __restrict__ Qv, const void* __restrict__ Kv, const uint8_t* __restrict__ Qs,
    const uint8_t* __restrict__ Ks, const void* __restrict__ Vt, int Lp,
    const int32_t* __restrict__ off, AttnParams p, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int32_t* __restrict__ ctr,
    const int32_t* __restrict__ bucket_off, const int32_t* __restrict__ bucket_q,
    const int32_t* __restrict__ slot, float* __restrict__ pO, float* __restrict__ plse,
    bf16_t* __restrict__ O, float* __restrict__ lse) {
  using LT = LdsTiles<D>;
  using MT = MxTiles<D>;
  constexpr bool MX = QNT != QNT_NONE;
  constexpr bool QV = QNT == QNT_VALUES;
  static_assert(kNW == 8, "two groups of four waves");
  constexpr int STAGE = QV ? MxvTiles<D>::STAGE : MX ? MT::STAGE : LT::STAGE;
  // V tile within a stage
  constexpr int VOFF = QV ? MxvTiles<D>::VOFF : MX ? MT::KBYTES : LT::KBYTES;
  // four stage buffers as distinct objects, so that the compiler can tell the LDS written by
  // the in-flight direct-to-LDS copies from the stage being read (no forced wait between them)
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[STAGE];
  if (layout_rejected(p.chk)) return;

  int bh, q_lo, nq, r1a, r1b, r2a, r2b, bstart = 0;
  if constexpr (MODE == MODE_ANCHOR) {
    // an item of this XCD's range (about an eighth of the total cost; the range starts are at
    // n_tiles[1 ..], stored by the index inversion), or of another XCD's once this one's is
    // used up; one item per workgroup
    __shared__ int s_item;
    if (threadIdx.x == 0)
      s_item = claim_item(n_tiles + 1, ctr, static_cast<int>(blockIdx.x) % kXcds);
    __syncthreads();
    const int lid = s_item;
    if (lid < 0) return;
    const int nt = n_tiles[0];
    bh = lid / nt;
    const int32_t* a = tiles + 6 * (lid % nt);
    q_lo = a[0];
    nq = a[1] - a[0];
    r1a = a[2]; r1b = a[3]; r2a = a[4]; r2b = a[5];
  } else {
    const int nwork = n_tiles[0];
    if (static_cast<int>(blockIdx.x) >= nwork) return;
    const int lid = xcd_remap(blockIdx.x, nwork);
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

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int ql = lane & 31, g = lane >> 5;
  const int row = wv * 32 + ql;
  int tok;
  {
    const int rr = row < nq ? row : nq - 1;
    if constexpr (MODE == MODE_ANCHOR) tok = q_lo + rr;
    else tok = bucket_q[bstart + rr];
  }
  // s_waitcnt vmcnt(n) lgkmcnt(0), n = this wave's copies of one stage: all but the newest
  // stage's copies have landed
  std::conditional_t<MX, MxStageCopier<D, kNW, QV>, StageCopier<D, kNW>> cp;
  cp.init(wv, lane, Lp);
  const int ncopy = cp.count();
  auto wait_but_newest = [&]() __attribute__((always_inline)) {
    constexpr int NB = MX ? MxStageCopier<D, kNW, QV>::NBASE : LT::KBLK / kNW + LT::VBLK / kNW;
    if (ncopy == NB) __builtin_amdgcn_s_waitcnt(0x0070 | NB);
    else if (ncopy == NB + 1) __builtin_amdgcn_s_waitcnt(0x0070 | (NB + 1));
    else __builtin_amdgcn_s_waitcnt(0x0070 | (NB + 2));
  };
  const size_t bh_off = static_cast<size_t>(bh) * p.L * D;
  const size_t bhp = static_cast<size_t>(bh) * Lp;  // MX rows are padded to Lp per (b, h)
  const bf16_t* Kbh = static_cast<const bf16_t*>(Kv) + bh_off;
  const uint8_t* Kcbh = static_cast<const uint8_t*>(Kv) + bhp * D;
  const uint8_t* Ksbh = Ks + bhp * MT::NB;
  const bf16_t* Vtbh = static_cast<const bf16_t*>(Vt) + static_cast<size_t>(bh) * D * Lp;
  // quantised V tiles of this (b, h): Lp / 64 tiles of D rows
  const uint8_t* Vqbh = static_cast<const uint8_t*>(Vt) + static_cast<size_t>(bh) * Lp * D * kVqRow / kBN;
  std::conditional_t<MX, MxQFrag<D>, QFrag<bf16_t, D>> qf;
  if constexpr (MX)
    qf.load(static_cast<const uint8_t*>(Qv) + (bhp + tok) * D, Qs + (bhp + tok) * MT::NB, g);
  else
    qf.load(static_cast<const bf16_t*>(Qv) + bh_off + static_cast<size_t>(tok) * D, g);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_ref = -__builtin_inff();
  float lsum = 0.f;
  const float c2 = p.scale_log2;

  // 64-aligned tiles covering [r1a, r1b) then [r2a, r2b)
  const int m1a = r1a >> 6, n1 = r1b > r1a ? ((r1b - 1) >> 6) - m1a + 1 : 0;
  const int m2a = r2a >> 6, n2 = r2b > r2a ? ((r2b - 1) >> 6) - m2a + 1 : 0;
  const int ntot = n1 + n2;
  auto tile_of = [&](int j, int& base, int& lo, int& hi) __attribute__((always_inline)) {
    int ra, rb;
    if (j < n1) { base = (m1a + j) * kBN; ra = r1a; rb = r1b; }
    else { base = (m2a + j - n1) * kBN; ra = r2a; rb = r2b; }
    lo = ra > base ? ra - base : 0;
    hi = rb - base < kBN ? rb - base : kBN;
  };
  const int kmax = p.L - 1;
  auto tile_base = [&](int j) __attribute__((always_inline)) { return j < n1 ? (m1a + j) * kBN : (m2a + j - n1) * kBN; };
  // Stage j (0 <= j < ntot) holds K and V^T of tile j, in buffer j % 4.
  const uint32_t lds0 = lds_addr(st0), lds1 = lds_addr(st1), lds2 = lds_addr(st2),
                 lds3 = lds_addr(st3);
  auto issue = [&](int j, uint32_t lds) __attribute__((always_inline)) {
    if (j >= ntot) return;
    const int base = tile_base(j);
    if constexpr (QV) cp.issue(lds, Kcbh, Ksbh, base, Vqbh + static_cast<size_t>(base / kBN) * D * kVqRow, base);
    else if constexpr (MX) cp.issue(lds, Kcbh, Ksbh, base, Vtbh, base);
    else cp.issue(lds, Kbh, base, kmax, Vtbh, base);
  };

  // Two wave groups (waves 0-3 and 4-7; wave w and w+4 run on the same SIMD) work on the same
  // key tiles half a step apart: in every half-step one group issues MFMAs (O += V P of the
  // previous tile, then S of the current one) while the other runs the softmax of its current
  // tile on the VALU, so the matrix cores of each SIMD stay busy during the exp / max / sum
  // work. Half-step t ends with a workgroup barrier; group 0 runs MFMAs on even t, group 1 on
  // odd t. A wave streams its MFMA operands from LDS at a bounded rate of its own, so during
  // its softmax half-step it also reads the first kPre V^T operands of the P.V that follows
  // (preload): the two waves of a SIMD then read LDS at the same time. Stage j is read in
  // half-steps 2j (S, group 0) to 2j+3 (P.V, group 1); its copies are issued in half-step 2j-4
  // (group 1) or 2j-3 (group 0), both softmax half-steps, into the buffer of stage j-4, and
  // waited for at the end of half-step 2j-1.
  f32x16 s[2];
  bf16x8 pb[4];  // P^T of the previous tile, packed for the four 16-key MFMA steps
  i32x8 pb8;     // QNT_VALUES: P^T of the previous tile as e4m3 codes (one 64-key MFMA step)
  auto scores = [&](const char* st) __attribute__((always_inline)) {
    if constexpr (MX) score_tile_mx<D>(st, qf, s, ql, g);
    else score_tile_swz<D>(st, qf, s, ql, g);
  };
  bf16x8 pre[kPre > 0 ? kPre : 1];  // V^T operands read ahead for the next P.V
  auto preload = [&](const char* st) __attribute__((always_inline)) {
    if constexpr (kPre > 0 && !QV) pv_preload<D, VOFF, kPre>(st, pre, ql, g);
  };
  // steady MFMA half-step: O += V P of tile j-1 (stage stp), then S of tile j (stage stc)
  auto mfma_full = [&](const char* stp, const char* stc) __attribute__((always_inline)) {
    if constexpr (QV) pv_mxv<D, VOFF>(stp, pb8, acc, ql, g);
    else pv_swz_packed<D, VOFF, kPre>(stp, pb, acc, ql, g, pre);
    scores(stc);
    // operand reads run kReadAhead ahead of the MFMAs that use them, all the way to the last
    // MFMA (bounded registers; an even spread of the reads over the MFMAs fell behind the
    // last ones, which then each waited for their operand)
    if constexpr (QV) {
      // P.V: three reads per MFMA (two code halves and the scale word); S as below
      constexpr int NM = D / 32 + 2 * (D / 64);
      constexpr int NR = 3 * (D / 32) + 4 * (D / 64) + 2;
      sched_lead_reads<NM, NR, kReadAhead, D / 32, 0, 2, 2, 3>();
    } else if constexpr (MX) {
      // P.V: one read per MFMA (less the preloaded ones); S: two code reads per MFMA and two
      // scale reads per tile
      constexpr int NM = 4 * (D / 32) + 2 * (D / 64);
      constexpr int NR = 4 * (D / 32) - kPre + 4 * (D / 64) + 2;
      sched_lead_reads<NM, NR, kReadAhead, 4 * (D / 32), kPre, 2, 2>();
    } else {
      constexpr int NM = 4 * (D / 32) + 2 * (D / 16);
      constexpr int NR = NM - kPre;
      sched_lead_reads<NM, NR, kReadAhead, 4 * (D / 32), kPre, 0, 1>();
    }
  };
  // last MFMA half-step: O += V P of the last tile
  auto mfma_last = [&]() __attribute__((always_inline)) {
    const int r = (ntot - 1) & 3;
    const char* st = r == 0 ? st0 : r == 1 ? st1 : r == 2 ? st2 : st3;
    if constexpr (QV) {
      pv_mxv<D, VOFF>(st, pb8, acc, ql, g);
    } else {
      if (r == 0) pv_swz_packed<D, VOFF, kPre>(st0, pb, acc, ql, g, pre);
      else if (r == 1) pv_swz_packed<D, VOFF, kPre>(st1, pb, acc, ql, g, pre);
      else if (r == 2) pv_swz_packed<D, VOFF, kPre>(st2, pb, acc, ql, g, pre);
      else pv_swz_packed<D, VOFF, kPre>(st3, pb, acc, ql, g, pre);
    }
  };
  auto valu_half = [&](int j) __attribute__((always_inline)) {
    int base, lo, hi;
    tile_of(j, base, lo, hi);
    if (lo > 0 || hi < kBN) {  // partial tile at a range edge: mask keys outside [lo, hi)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = key_of_perm(kb, i, g);
          if (k < lo || k >= hi) s[kb][i] = -__builtin_inff();
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescale)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }
    const float neg = -m_ref;
    float l0 = 0.f, l1 = 0.f;
    if constexpr (QV) {
      // P^T as e4m3 codes, round to nearest even (values are at most 2^kRescale = 256, below
      // the e4m3 maximum 448); the row sum keeps the unrounded values
      int w[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = fast_exp2(__builtin_fmaf(s[0][4 * k + e], c2, neg));
          b[e] = fast_exp2(__builtin_fmaf(s[1][4 * k + e], c2, neg));
          l0 += a[e];
          l1 += b[e];
        }
        w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false);
        w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(a[2], a[3], w[k], true);
        w[4 + k] = __builtin_amdgcn_cvt_pk_fp8_f32(b[0], b[1], 0, false);
        w[4 + k] = __builtin_amdgcn_cvt_pk_fp8_f32(b[2], b[3], w[4 + k], true);
      }
      pb8 = i32x8{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(s[0][i], c2, neg));
        const float p1 = fast_exp2(__builtin_fmaf(s[1][i], c2, neg));
        pb[i >> 3][i & 7] = static_cast<__bf16>(p0);
        pb[2 + (i >> 3)][i & 7] = static_cast<__bf16>(p1);
        l0 += p0;
        l1 += p1;
      }
    }
    lsum += l0 + l1;
  };
  // workgroup barrier that no instruction is scheduled across; copies in flight stay in flight
  // (a fenced __syncthreads would wait for them)
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // stage i complete (its first read is in the next half-step); stage i+1 may stay in flight
  auto wait_stage = [&](int i) __attribute__((always_inline)) {
    if (i + 1 < ntot) wait_but_newest();
    else __builtin_amdgcn_s_waitcnt(0x0070);
  };

  if (ntot > 0) {
    issue(0, lds0);
    issue(1, lds1);
    wait_stage(0);
    bar();
    if (wv < 4) {
      // group 0: half-step 2j = MFMAs (P.V of tile j-1, S of tile j), 2j+1 = softmax of tile j
      scores(st0);
      bar();
      issue(2, lds2);
      preload(st0);
      valu_half(0);
      wait_stage(1);
      bar();
      auto step = [&](int j, const char* stp, const char* stc, uint32_t lds_j2) __attribute__((always_inline)) {
        mfma_full(stp, stc);
        bar();
        issue(j + 2, lds_j2);  // the buffer of stage j-2, last read in half-step 2j-1
        preload(stc);
        valu_half(j);
        wait_stage(j + 1);
        bar();
      };
      for (int j = 1; j < ntot; j += 4) {
        step(j, st0, st1, lds3);
        if (j + 1 < ntot) step(j + 1, st1, st2, lds0);
        if (j + 2 < ntot) step(j + 2, st2, st3, lds1);
        if (j + 3 < ntot) step(j + 3, st3, st0, lds2);
      }
      mfma_last();  // half-step 2 ntot
      bar();
      bar();  // idle half-step 2 ntot + 1
    } else {
      // group 1: idle half-step 0, then 2j+1 = MFMAs of tiles j-1 / j, 2j+2 = softmax of tile j
      issue(2, lds2);
      bar();
      scores(st0);
      wait_stage(1);
      bar();
      issue(3, lds3);
      preload(st0);
      valu_half(0);
      bar();
      auto step = [&](int j, const char* stp, const char* stc, uint32_t lds_j3) __attribute__((always_inline)) {
        mfma_full(stp, stc);
        wait_stage(j + 1);
        bar();
        issue(j + 3, lds_j3);  // the buffer of stage j-1, last read in half-step 2j+1
        preload(stc);
        valu_half(j);
        bar();
      };
      for (int j = 1; j < ntot; j += 4) {
        step(j, st0, st1, lds0);
        if (j + 1 < ntot) step(j + 1, st1, st2, lds1);
        if (j + 2 < ntot) step(j + 2, st2, st3, lds2);
        if (j + 3 < ntot) step(j + 3, st3, st0, lds3);
      }
      mfma_last();  // half-step 2 ntot + 1
      bar();
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / ltot;
  const float lse2 = m_ref + fast_log2(ltot);
  if (row >= nq) return;
  if constexpr (MODE == MODE_ROUTED) {
    const size_t pos = static_cast<size_t>(bstart) + row;
    float* prow = pO + pos * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<f32x4*>(prow + db * 32 + 8 * jj + 4 * g) =
            f32x4{acc[db][4 * jj] * inv, acc[db][4 * jj + 1] * inv, acc[db][4 * jj + 2] * inv,
                  acc[db][4 * jj + 3] * inv};
    if (g == 0) plse[pos] = lse2;
  } else {
    const size_t trow = static_cast<size_t>(bh) * p.L + tok;
    const int32_t* sl = slot + trow * p.S;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] *= inv;
    float M = lse2, wsum = 1.f;
    for (int jsl = 0; jsl < p.S; ++jsl) {
      const int pos = sl[jsl];
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
    bf16_t* orow = O + trow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 0] * winv)) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 1] * winv)) << 16);
        const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 2] * winv)) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 3] * winv)) << 16);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * g) = u32x2{w0, w1};
      }
    if (g == 0) lse[trow] = (M + fast_log2(wsum)) * kLn2;
  }
}

// bf16 Q, K, V (MX = false) or MXFP8 Q and K (MX = true)
template <int D, int MODE, bool MX>
__global__ __launch_bounds__(kNT) void attn_fwd_bf16_kernel(
    const void* __restrict__ Qv, const void* __restrict__ Kv, const uint8_t* __restrict__ Qs,
    const uint8_t* __restrict__ Ks, const void* __restrict__ Vt, int Lp,
    const int32_t* __restrict__ off, AttnParams p, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int32_t* __restrict__ ctr,
    const int32_t* __restrict__ bucket_off, const int32_t* __restrict__ bucket_q,
    const int32_t* __restrict__ slot, float* __restrict__ pO, float* __restrict__ plse,
    bf16_t* __restrict__ O, float* __restrict__ lse) {
  attn_fwd_lds_body<D, MODE, MX ? QNT_SCORES : QNT_NONE>(Qv, Kv, Qs, Ks, Vt, Lp, off, p, tiles,
                                                          n_tiles, ctr, bucket_off, bucket_q,
                                                          slot, pO, plse, O, lse);
}

// MXFP8 Q, K and V (quantised scores and values)
template <int D, int MODE>
__global__ __launch_bounds__(kNT) void attn_fwd_mxv_kernel(
    const void* __restrict__ Qv, const void* __restrict__ Kv, const uint8_t* __restrict__ Qs,
    const uint8_t* __restrict__ Ks, const void* __restrict__ Vq, int Lp,
    const int32_t* __restrict__ off, AttnParams p, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int32_t* __restrict__ ctr,
    const int32_t* __restrict__ bucket_off, const int32_t* __restrict__ bucket_q,
    const int32_t* __restrict__ slot, float* __restrict__ pO, float* __restrict__ plse,
    bf16_t* __restrict__ O, float* __restrict__ lse) {
  attn_fwd_lds_body<D, MODE, QNT_VALUES>(Qv, Kv, Qs, Ks, Vq, Lp, off, p, tiles, n_tiles, ctr,
                                         bucket_off, bucket_q, slot, pO, plse, O, lse);
}

}  // namespace moc

namespace moc_host {

using moc::AttnParams;

int attn_tile_rows() { return moc::kBM; }

// rows of the transposed V copy: L rounded up to the 64-key tile
int attn_vt_rows(int L) { return (L + moc::kBN - 1) / moc::kBN * moc::kBN; }

// X [BH][L][d] -> X^T [BH][d][Lp] (bf16), the only instantiation of the transpose kernel
hipError_t launch_transpose_rows(const void* X, void* Xt, int BH, int L, int Lp, int d,
                                 const uint32_t* chk, hipStream_t st) {
  using moc::bf16_t;
  if (d == 128)
    hipLaunchKernelGGL((moc::transpose_rows_kernel<128>), dim3(Lp / moc::kBN, BH), dim3(256), 0,
                       st, static_cast<const bf16_t*>(X), static_cast<bf16_t*>(Xt), L, Lp, chk);
  else
    hipLaunchKernelGGL((moc::transpose_rows_kernel<64>), dim3(Lp / moc::kBN, BH), dim3(256), 0,
                       st, static_cast<const bf16_t*>(X), static_cast<bf16_t*>(Xt), L, Lp, chk);
  return hipGetLastError();
}

size_t attn_fwd_vt_bytes(const moc_layout* lay) {
  if (lay->dtype != MOC_BF16) return 0;
  return static_cast<size_t>(lay->B) * lay->H * lay->d * attn_vt_rows(lay->L) * 2;
}

template <typename T, int D>
static hipError_t launch_fwd_t(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                               const void* K, const void* V, float scale, void* O, float* lse,
                               float* pO, float* plse, hipStream_t st) {
  AttnParams p;
  p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = vl->S;
  p.scale_log2 = scale * moc::kLog2e;
  p.chk = vl->status;
  const T* q = static_cast<const T*>(Q);
  const T* k = static_cast<const T*>(K);
  const T* v = static_cast<const T*>(V);
  if (vl->S > 0 && vl->max_rtiles > 0) {
    p.max_tiles = vl->max_rtiles;
    hipLaunchKernelGGL((moc::attn_fwd_kernel<T, D, moc::MODE_ROUTED>), dim3(vl->max_rtiles),
                       dim3(moc::kNT), 0, st, q, k, v, lay->chunk_offsets, p, vl->rtiles,
                       vl->n_rtiles, vl->bucket_off, vl->bucket_q, vl->slot, pO, plse,
                       static_cast<T*>(O), lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  p.max_tiles = vl->max_atiles;
  hipLaunchKernelGGL((moc::attn_fwd_kernel<T, D, moc::MODE_ANCHOR>),
                     dim3(vl->max_atiles * lay->B * lay->H), dim3(moc::kNT), 0, st, q, k, v,
                     lay->chunk_offsets, p, vl->atiles, vl->n_atiles, vl->bucket_off,
                     vl->bucket_q, vl->slot, pO, plse, static_cast<T*>(O), lse);
  return hipGetLastError();
}

// bf16 forward; with Qs/Ks non-null, Q and K are MXFP8 codes (rows padded to Lp) and scales
template <int D>
static hipError_t launch_fwd_bf16(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                                  const void* K, const uint8_t* Qs, const uint8_t* Ks,
                                  const void* V, float scale, void* O, float* lse, float* pO,
                                  float* plse, void* vt_ws, hipStream_t st) {
  using moc::bf16_t;
  AttnParams p;
  p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = vl->S;
  p.scale_log2 = scale * moc::kLog2e;
  p.chk = vl->status;
  const int Lp = attn_vt_rows(lay->L);
  bf16_t* Vt = static_cast<bf16_t*>(vt_ws);
  hipError_t e = launch_transpose_rows(V, Vt, lay->B * lay->H, lay->L, Lp, D, vl->status, st);
  if (e != hipSuccess) return e;
  const bool mx = Qs != nullptr;
  if (vl->S > 0 && vl->max_rtiles > 0) {
    p.max_tiles = vl->max_rtiles;
    if (mx)
      hipLaunchKernelGGL((moc::attn_fwd_bf16_kernel<D, moc::MODE_ROUTED, true>),
                         dim3(vl->max_rtiles), dim3(moc::kNT), 0, st, Q, K, Qs, Ks, Vt, Lp,
                         lay->chunk_offsets, p, vl->rtiles, vl->n_rtiles, nullptr, vl->bucket_off,
                         vl->bucket_q, vl->slot, pO, plse, static_cast<bf16_t*>(O), lse);
    else
      hipLaunchKernelGGL((moc::attn_fwd_bf16_kernel<D, moc::MODE_ROUTED, false>),
                         dim3(vl->max_rtiles), dim3(moc::kNT), 0, st, Q, K, Qs, Ks, Vt, Lp,
                         lay->chunk_offsets, p, vl->rtiles, vl->n_rtiles, nullptr, vl->bucket_off,
                         vl->bucket_q, vl->slot, pO, plse, static_cast<bf16_t*>(O), lse);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  p.max_tiles = vl->max_atiles;
  const int grid = moc::kXcds * moc::xcd_slots(vl->max_atiles, lay->B * lay->H);
  if (mx)
    hipLaunchKernelGGL((moc::attn_fwd_bf16_kernel<D, moc::MODE_ANCHOR, true>), dim3(grid),
                       dim3(moc::kNT), 0, st, Q, K, Qs, Ks, Vt, Lp, lay->chunk_offsets, p,
                       vl->atiles, vl->n_atiles, vl->n_atiles + moc::kCtrFwd, vl->bucket_off,
                       vl->bucket_q, vl->slot, pO,
                       plse, static_cast<bf16_t*>(O), lse);
  else
    hipLaunchKernelGGL((moc::attn_fwd_bf16_kernel<D, moc::MODE_ANCHOR, false>), dim3(grid),
                       dim3(moc::kNT), 0, st, Q, K, Qs, Ks, Vt, Lp, lay->chunk_offsets, p,
                       vl->atiles, vl->n_atiles, vl->n_atiles + moc::kCtrFwd, vl->bucket_off,
                       vl->bucket_q, vl->slot, pO,
                       plse, static_cast<bf16_t*>(O), lse);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                           const void* K, const void* V, float scale, void* O, float* lse,
                           float* pO, float* plse, void* vt_ws, hipStream_t st) {
  if (lay->dtype == MOC_BF16)
    return lay->d == 128
               ? launch_fwd_bf16<128>(lay, vl, Q, K, nullptr, nullptr, V, scale, O, lse, pO, plse, vt_ws, st)
               : launch_fwd_bf16<64>(lay, vl, Q, K, nullptr, nullptr, V, scale, O, lse, pO, plse, vt_ws, st);
  return lay->d == 128 ? launch_fwd_t<float, 128>(lay, vl, Q, K, V, scale, O, lse, pO, plse, st)
                       : launch_fwd_t<float, 64>(lay, vl, Q, K, V, scale, O, lse, pO, plse, st);
}

// quantised scores and values: Q and K as MXFP8 codes and scales (rows padded to Lp), V as the
// quantised tiles of moc_mx_quantize_v
template <int D>
static hipError_t launch_fwd_mxv_d(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                                   const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                                   const uint8_t* Vq, float scale, void* O, float* lse, float* pO,
                                   float* plse, hipStream_t st) {
  using moc::bf16_t;
  AttnParams p;
  p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = vl->S;
  p.scale_log2 = scale * moc::kLog2e;
  p.chk = vl->status;
  const int Lp = attn_vt_rows(lay->L);
  hipError_t e;
  if (vl->S > 0 && vl->max_rtiles > 0) {
    p.max_tiles = vl->max_rtiles;
    hipLaunchKernelGGL((moc::attn_fwd_mxv_kernel<D, moc::MODE_ROUTED>), dim3(vl->max_rtiles),
                       dim3(moc::kNT), 0, st, Qc, Kc, Qs, Ks, Vq, Lp, lay->chunk_offsets, p,
                       vl->rtiles, vl->n_rtiles, nullptr, vl->bucket_off, vl->bucket_q, vl->slot, pO,
                       plse, static_cast<bf16_t*>(O), lse);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  p.max_tiles = vl->max_atiles;
  hipLaunchKernelGGL((moc::attn_fwd_mxv_kernel<D, moc::MODE_ANCHOR>),
                     dim3(moc::kXcds * moc::xcd_slots(vl->max_atiles, lay->B * lay->H)),
                     dim3(moc::kNT), 0, st, Qc, Kc, Qs,
                     Ks, Vq, Lp, lay->chunk_offsets, p, vl->atiles, vl->n_atiles,
                     vl->n_atiles + moc::kCtrFwd, vl->bucket_off, vl->bucket_q, vl->slot, pO, plse,
                     static_cast<bf16_t*>(O), lse);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_mxv(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                               const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                               const uint8_t* Vq, float scale, void* O, float* lse, float* pO,
                               float* plse, hipStream_t st) {
  return lay->d == 128
             ? launch_fwd_mxv_d<128>(lay, vl, Qc, Qs, Kc, Ks, Vq, scale, O, lse, pO, plse, st)
             : launch_fwd_mxv_d<64>(lay, vl, Qc, Qs, Kc, Ks, Vq, scale, O, lse, pO, plse, st);
}

// quantised scores: Q and K as MXFP8 codes and scales (rows padded to Lp), V bf16
hipError_t launch_attn_fwd_mx(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                              const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                              const void* V, float scale, void* O, float* lse, float* pO,
                              float* plse, void* vt_ws, hipStream_t st) {
  return lay->d == 128
             ? launch_fwd_bf16<128>(lay, vl, Qc, Kc, Qs, Ks, V, scale, O, lse, pO, plse, vt_ws, st)
             : launch_fwd_bf16<64>(lay, vl, Qc, Kc, Qs, Ks, V, scale, O, lse, pO, plse, vt_ws, st);
}

}  // namespace moc_host
