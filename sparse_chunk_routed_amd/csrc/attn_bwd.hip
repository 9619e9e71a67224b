// K5: MoC attention backward with the routed sets held fixed.
//
// Source: "Mixture of Contexts for Long Video Generation | Summary" §3.1 and Appendix A (top-k is
// a discrete, non-differentiable choice; gradients reach the keys/values that were selected,
// and the summarised implementation wraps the attention in a custom autograd function).
//
// For every attended pair (t, j), with x_tj = scale q_t.k_j and P_tj = exp(x_tj - lse_t):
//   dV_j += P_tj dO_t;  dP_tj = dO_t.v_j;  dS_tj = P_tj (dP_tj - D_t) with D_t = dO_t.O_t;
//   dQ_t += scale dS_tj k_j;  dK_j += scale dS_tj q_t.
// Pairs come in the same blocks as the forward: anchor (a query tile x text U own-shot keys)
// and routed (a bucket of gathered queries x one chunk). The kernels:
//   prep      D_t and the base-2 LSE per query row.
//   images    the dQ kernel's 64-key tile images (K rows, V rows, K^T) and the dK/dV kernel's
//             32-query tile images (Q and dO rows, their transposes, lse2 and D) of the whole
//             sequence and of every routed bucket (padded to 32 rows, pads have P = 0), each
//             laid out as the kernel's LDS stage so that staging is a linear copy.
//   dq        query-centric, like the forward (S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T):
//             routed tiles write fp32 partial rows per (query, routed chunk); anchor tiles
//             merge those partials in ascending chunk order and write dQ.
//   dkdv      key-centric: a workgroup owns 128 keys of one chunk (4 waves x 32) and streams
//             the query blocks of the chunk's shot (anchor) and then of the chunk's routed
//             bucket, accumulating dV += P^T dO and dK += dS^T Q in registers (S = Q K^T).
//   text      text keys are attended by every query: their key tiles are split over query
//             ranges into fp32 partials, summed here in a fixed order.
// No float atomics anywhere, so the result is deterministic. The separate dQ and dK/dV passes
// recompute S and dP (7 GEMM-units per pair instead of 5).
#include "attn_common.h"
#include "attn_bwd_lds.h"

namespace moc {

constexpr int kBwdQNW = 8;                 // dq: waves (32 queries each) per workgroup
constexpr int kBwdQNT = 64 * kBwdQNW;
constexpr int kBwdQBM = 32 * kBwdQNW;      // queries per dq workgroup (= varlen tile rows)
constexpr int kBwdKNW = 4;                 // dkdv: waves (32 keys each) per workgroup
constexpr int kBwdKNT = 64 * kBwdKNW;
constexpr int kBwdKR = 32 * kBwdKNW;       // keys per key tile
constexpr int kBwdQT = 32;                 // queries per dkdv step
constexpr int kTextSplitRows = 16384;      // queries per text-key split
constexpr int kDqAhead = 3;                // dq: LDS operand reads in flight per MFMA sequence
constexpr int kDkdvAhead = 3;              // dkdv: LDS operand reads in flight per MFMA sequence

struct BwdParams {
  int B, H, L, C, S, max_tiles;
  int Lp;  // L rounded up to 64: row stride of the per-(b, h) statistics and transposed copies
  int text_begin, text_len, n_split;
  float scale_log2;  // softmax_scale * log2(e)
  float scale;
  const uint32_t* chk;  // layout check word (moc_layout.check) or NULL
};

enum { BMODE_ANCHOR = 0, BMODE_ROUTED = 1 };

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// D_t = sum_d dO[t,d] O[t,d]; lse2_t = lse_t * log2(e)
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16_t* __restrict__ O,
                                                       const bf16_t* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ Dq,
                                                       float* __restrict__ lse2, int64_t rows,
                                                       int L, int Lp,
                                                       const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + c * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) s += bf_lo(a[w]) * bf_lo(b[w]) + bf_hi(a[w]) * bf_hi(b[w]);
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (row < rows && c == 0) {
    const int64_t out = (row / L) * Lp + row % L;  // statistics rows are Lp apart
    Dq[out] = s;
    lse2[out] = lse[row] * kLog2e;
  }
}

// Query-centric dQ (bf16), built like the forward kernel: 8 waves x 32 queries, 64-key aligned
// tiles of K rows, V rows and K^T copied global -> LDS without registers (K^T from a transposed
// copy of K), two wave groups half a tile apart. Per tile a wave computes S^T = K Q^T and
// dP^T = V dO^T (lane = query, 16 keys), the VALU forms dS^T = P (dP - D) with
// P = exp2(S scale log2(e) - lse2), and dQ^T += K^T dS^T accumulates in registers. Skewed stage
// j holds K and V of tile j and K^T of tile j-1: a group's MFMA half-step runs dQ of tile j-1
// and S, dP of tile j, while the other group computes dS of its current tile.
template <int D, int MODE>
__global__ __launch_bounds__(kBwdQNT) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const char* __restrict__ kvimg, const bf16_t* __restrict__ dO,
    const float* __restrict__ Dq, const float* __restrict__ lse2,
    const int32_t* __restrict__ off, BwdParams p, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int32_t* __restrict__ ctr,
    const int32_t* __restrict__ bucket_off, const int32_t* __restrict__ bucket_q,
    const int32_t* __restrict__ slot, float* __restrict__ dQp, bf16_t* __restrict__ dQ) {
  static_assert(kBwdQNW == 8, "two groups of four waves");
  using LT = LdsTiles<D>;
  using KI = KvImage<D>;
  using CP = KvStageCopier<D, kBwdQNW>;
  __shared__ __attribute__((aligned(1024))) char st0[KI::BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[KI::BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[KI::BYTES];
  if (layout_rejected(p.chk)) return;

  // upper-bound grid: blocks past the device-side work count exit; the rest take the real work
  // items per XCD (anchor items: claimed from the cost-balanced ranges that the index inversion
  // stores after the anchor tile count, from other XCDs' ranges once this XCD's is used up)
  int bh, q_lo, nq, r1a, r1b, r2a, r2b, bstart = 0;
  if constexpr (MODE == BMODE_ANCHOR) {
    __shared__ int s_item;
    if (threadIdx.x == 0)
      s_item = claim_item(n_tiles + 1, ctr, static_cast<int>(blockIdx.x) % kXcds);
    __syncthreads();
    const int lid = s_item;
    if (lid < 0) return;
    const int nt = n_tiles[0];
    bh = lid / nt;
    const int32_t* a = tiles + 6 * (lid % nt);
    q_lo = a[0]; nq = a[1] - a[0];
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
    nq = rem < kBwdQBM ? rem : kBwdQBM;
    q_lo = 0;
    r1a = off[c]; r1b = off[c + 1]; r2a = 0; r2b = 0;
  }
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int ql = lane & 31, g = lane >> 5;
  const int r = wv * 32 + ql;
  const int rr = r < nq ? r : nq - 1;
  int t;
  if constexpr (MODE == BMODE_ANCHOR) t = q_lo + rr;
  else t = bucket_q[bstart + rr];

  CP cp;
  cp.init(wv, lane);
  const int ncopy = cp.count();
  auto wait_but_newest = [&]() __attribute__((always_inline)) {
    constexpr int NB = KI::NBLK / kBwdQNW;
    if (ncopy == NB) __builtin_amdgcn_s_waitcnt(0x0070 | NB);
    else __builtin_amdgcn_s_waitcnt(0x0070 | (NB + 1));
  };
  const size_t bh_off = static_cast<size_t>(bh) * p.L * D;
  const char* imgbh = kvimg + static_cast<size_t>(bh) * (p.Lp / kBN) * KI::BYTES;
  QFrag<bf16_t, D> qf, dof;
  qf.load(Q + bh_off + static_cast<size_t>(t) * D, g);
  dof.load(dO + bh_off + static_cast<size_t>(t) * D, g);
  const size_t trow = static_cast<size_t>(bh) * p.L + t;
  const size_t srow = static_cast<size_t>(bh) * p.Lp + t;
  const float l2 = lse2[srow];
  const float dd = Dq[srow];
  const float c2 = p.scale_log2;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  const int m1a = r1a >> 6, n1 = r1b > r1a ? ((r1b - 1) >> 6) - m1a + 1 : 0;
  const int m2a = r2a >> 6, n2 = r2b > r2a ? ((r2b - 1) >> 6) - m2a + 1 : 0;
  const int ntot = n1 + n2;
  auto tile_base = [&](int j) __attribute__((always_inline)) { return j < n1 ? (m1a + j) * kBN : (m2a + j - n1) * kBN; };
  auto tile_of = [&](int j, int& lo, int& hi) __attribute__((always_inline)) {
    int base, ra, rb;
    if (j < n1) { base = (m1a + j) * kBN; ra = r1a; rb = r1b; }
    else { base = (m2a + j - n1) * kBN; ra = r2a; rb = r2b; }
    lo = ra > base ? ra - base : 0;
    hi = rb - base < kBN ? rb - base : kBN;
  };
  const uint32_t lds0 = lds_addr(st0), lds1 = lds_addr(st1), lds2 = lds_addr(st2);
  // stage j: K and V rows of tile j, K^T of tile j-1 (clamped past the ends: loaded, unread)
  auto issue = [&](int j, uint32_t lds) __attribute__((always_inline)) {
    if (j > ntot || ntot == 0) return;
    const int tr = tile_base(j < ntot ? j : ntot - 1) / kBN;
    const int tt = tile_base(j > 0 ? j - 1 : 0) / kBN;
    cp.issue(lds, imgbh + static_cast<size_t>(tr) * KI::BYTES,
             imgbh + static_cast<size_t>(tt) * KI::BYTES);
  };

  f32x16 s[2], dp[2];
  bf16x8 dsb[4];  // dS^T of the previous tile, packed for the four 16-key MFMA steps
  auto sdp = [&](const char* st) __attribute__((always_inline)) {
    score_tile_swz<D>(st, qf, s, ql, g);
    score_tile_swz<D>(st + LT::KBYTES, dof, dp, ql, g);
  };
  auto mfma_full = [&](const char* st) __attribute__((always_inline)) {
    // dQ^T += K^T dS^T: the K^T tile sits after the two row tiles, in the V^T position of a
    // forward stage whose K tile starts one row tile later
    pv_swz_packed<D>(st + LT::KBYTES, dsb, acc, ql, g);
    sdp(st);
    // operand reads run kDqAhead ahead of their MFMAs (bounded registers)
    constexpr int NM = 4 * (D / 32) + 4 * (D / 16);
    __builtin_amdgcn_sched_group_barrier(0x100, kDqAhead, 0);
#pragma unroll
    for (int i = 0; i < NM - kDqAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kDqAhead, 0);
  };
  auto mfma_last = [&]() __attribute__((always_inline)) {
    const int rl = ntot % 3;
    if (rl == 0) pv_swz_packed<D>(st0 + LT::KBYTES, dsb, acc, ql, g);
    else if (rl == 1) pv_swz_packed<D>(st1 + LT::KBYTES, dsb, acc, ql, g);
    else pv_swz_packed<D>(st2 + LT::KBYTES, dsb, acc, ql, g);
  };
  auto valu_half = [&](int j) __attribute__((always_inline)) {
    int lo, hi;
    tile_of(j, lo, hi);
    if (lo > 0 || hi < kBN) {  // partial tile at a range edge: keys outside [lo, hi) get P = 0
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = key_of_perm(kb, i, g);
          if (k < lo || k >= hi) s[kb][i] = -__builtin_inff();
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(s[0][i], c2, -l2));
      const float p1 = fast_exp2(__builtin_fmaf(s[1][i], c2, -l2));
      dsb[i >> 3][i & 7] = static_cast<__bf16>(p0 * (dp[0][i] - dd));
      dsb[2 + (i >> 3)][i & 7] = static_cast<__bf16>(p1 * (dp[1][i] - dd));
    }
  };
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_next = [&](int i) __attribute__((always_inline)) {
    if (i + 2 <= ntot) wait_but_newest();
    else __builtin_amdgcn_s_waitcnt(0x0070);
  };

  if (ntot > 0) {
    issue(0, lds0);
    issue(1, lds1);
    wait_but_newest();
    bar();
    if (wv < 4) {
      // group 0: half-step 2j = MFMAs of stage j, 2j+1 = dS of tile j (+ copies of stage j+2)
      sdp(st0);
      bar();
      issue(2, lds2);
      valu_half(0);
      wait_next(0);
      bar();
      auto step = [&](int j, const char* cur, uint32_t nxt2) __attribute__((always_inline)) {
        mfma_full(cur);
        bar();
        issue(j + 2, nxt2);
        valu_half(j);
        wait_next(j);
        bar();
      };
      for (int j = 1; j < ntot; j += 3) {
        step(j, st1, lds0);
        if (j + 1 < ntot) step(j + 1, st2, lds1);
        if (j + 2 < ntot) step(j + 2, st0, lds2);
      }
      mfma_last();
      bar();
      wait_next(ntot);
      bar();
    } else {
      // group 1: idle half-step 0, then 2j+1 = MFMAs of stage j, 2j+2 = dS of tile j
      issue(2, lds2);
      bar();
      sdp(st0);
      wait_next(0);
      bar();
      issue(3, lds0);
      valu_half(0);
      bar();
      auto step = [&](int j, const char* cur, uint32_t cur_lds) __attribute__((always_inline)) {
        mfma_full(cur);
        wait_next(j);
        bar();
        issue(j + 3, cur_lds);
        valu_half(j);
        bar();
      };
      for (int j = 1; j < ntot; j += 3) {
        step(j, st1, lds1);
        if (j + 1 < ntot) step(j + 1, st2, lds2);
        if (j + 2 < ntot) step(j + 2, st0, lds0);
      }
      mfma_last();
      wait_next(ntot);
      bar();
    }
  }

  if (r >= nq) return;
  if constexpr (MODE == BMODE_ROUTED) {
    float* prow = dQp + (static_cast<size_t>(bstart) + r) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<f32x4*>(prow + db * 32 + 8 * jj + 4 * g) =
            f32x4{acc[db][4 * jj], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]};
  } else {
    const int32_t* sl = slot + trow * p.S;
    for (int js = 0; js < p.S; ++js) {
      const int pos = sl[js];
      if (pos < 0) break;
      const float* prow = dQp + static_cast<size_t>(pos) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(prow + db * 32 + 8 * jj + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * jj + e] += v[e];
        }
    }
    bf16_t* orow = dQ + trow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 0] * p.scale)) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 1] * p.scale)) << 16);
        const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 2] * p.scale)) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * jj + 3] * p.scale)) << 16);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * g) = u32x2{w0, w1};
      }
  }
}

// Key-centric dK/dV (bf16). A workgroup owns a key tile's 128 keys (4 waves x 32; K and V rows
// in registers as B operands) and streams 32-query blocks: first its anchor range (the keys'
// shot, or a split of all queries for text keys) from the sequence's blocks, then the chunk's
// routed bucket from the gathered blocks. Blocks are staged by register-free copies (two
// stages). Per block a wave computes S = Q K^T and dP = dO V^T (lane = key; the Q and dO rows
// are read in a permuted order so that each lane's values come in runs of 8 queries),
// P = exp2(S scale log2(e) - lse2) and dS = P (dP - D) on the VALU, then dV += P^T dO and
// dK += dS^T Q with P^T and dS^T straight from registers. Two workgroups share a CU (at most
// 256 registers), so one's MFMAs overlap the other's VALU. Video keys are complete at the end
// (bf16 out); text keys write fp32 partials of their query split.
template <int D>
__global__ __launch_bounds__(kBwdKNT, 2) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ K, const bf16_t* __restrict__ V, BwdParams p,
    const int32_t* __restrict__ ktiles, const int32_t* __restrict__ n_ktiles,
    const char* __restrict__ qblocks, const char* __restrict__ gblocks,
    const int32_t* __restrict__ gstart, const int32_t* __restrict__ kranges,
    int32_t* __restrict__ ctr, float* __restrict__ textK, float* __restrict__ textV,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV) {
  using QTl = QTiles<D>;
  using CP = QTileCopier<D, kBwdKNW>;
  __shared__ __attribute__((aligned(1024))) char st0[QTl::BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[QTl::BYTES];
  if (layout_rejected(p.chk)) return;

  // an item of this XCD's range of (b, h, key tile) items (bwd_key_split_kernel), or of another
  // XCD's once this one's is used up; one item per workgroup
  __shared__ int s_item;
  if (threadIdx.x == 0)
    s_item = claim_item(kranges, ctr, static_cast<int>(blockIdx.x) % kXcds);
  __syncthreads();
  const int lid = s_item;
  if (lid < 0) return;
  const int nt = n_ktiles[0];
  const int bh = lid / nt;
  const int32_t* kt6 = ktiles + 6 * (lid % nt);
  const int k0 = kt6[0], k1 = kt6[1], c = kt6[2], qa = kt6[3], qb = kt6[4], sp = kt6[5];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int ql = lane & 31, g = lane >> 5;
  const int key = k0 + wv * 32 + ql;
  const int kl = key < k1 ? key : k1 - 1;
  const size_t bh_off = static_cast<size_t>(bh) * p.L * D;
  QFrag<bf16_t, D> kf, vf;
  kf.load(K + bh_off + static_cast<size_t>(kl) * D, g);
  vf.load(V + bh_off + static_cast<size_t>(kl) * D, g);
  // Retire these loads before any copy is issued: their first use would otherwise be inside the
  // tile loop, where the compiler's wait for them would also wait for copies in flight. The asm
  // "uses" every fragment here, so the compiler waits for the loads at this point.
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) asm volatile("" ::"v"(kf.q[kk]), "v"(vf.q[kk]));
  const float c2 = p.scale_log2;

  CP cp;
  cp.init(wv, lane);
  const int ncopy = cp.count();
  auto wait_but_newest = [&]() __attribute__((always_inline)) {
    constexpr int NB = QTl::NBLK / kBwdKNW;
    if (ncopy == NB) __builtin_amdgcn_s_waitcnt(0x0070 | NB);
    else __builtin_amdgcn_s_waitcnt(0x0070 | (NB + 1));
  };

  f32x16 accK[D / 32], accV[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    accK[db] = f32x16{};
    accV[db] = f32x16{};
  }
  const int nqt = qb > qa ? ((qb - 1) >> 5) - (qa >> 5) + 1 : 0;
  const int qbase0 = qa & ~31;
  // anchor queries: the sequence's query blocks from qa's; routed queries of this chunk: the
  // bucket's gathered blocks (pads have P = 0)
  const char* ab = qblocks + (static_cast<size_t>(bh) * (p.Lp >> 5) + (qa >> 5)) * QTl::BYTES;
  const char* gb = gblocks;
  int ngt = 0;
  if (c >= 0) {
    const int bucket = bh * p.C + c;
    const int g0 = gstart[bucket];
    ngt = (gstart[bucket + 1] - g0) >> 5;
    gb += static_cast<size_t>(g0 >> 5) * QTl::BYTES;
  }
  const int ntot = nqt + ngt;
  const uint32_t lds0 = lds_addr(st0), lds1 = lds_addr(st1);
  auto issue = [&](int j, uint32_t lds) __attribute__((always_inline)) {
    if (j >= ntot) return;
    const char* blk = j < nqt ? ab + static_cast<size_t>(j) * QTl::BYTES
                              : gb + static_cast<size_t>(j - nqt) * QTl::BYTES;
    cp.issue(lds, blk);
  };
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const int rq = QTl::RROW * kperm(ql) + g;  // permuted row of this lane's A operand (chunks)
  // the operand reads of an MFMA sequence run kDkdvAhead ahead of their MFMAs: an LDS read
  // takes longer than one MFMA, so fewer in flight leave every MFMA waiting on its operand
  // (and more do not fit the 256 registers)
  auto pace = [&](int nm) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, kDkdvAhead, 0);
    for (int i = 0; i < nm - kDkdvAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kDkdvAhead, 0);
  };
  // One 32-query tile, in the order S -> P -> dV, dP -> dS -> dK, so that at most one 32x32
  // score block and one packed block are live next to the accumulators (dS uses the packed P).
  auto tile = [&](int j, const char* cur) __attribute__((always_inline)) {
    const char* qr = cur + QTl::Q_OFF + rq * 16;
    const char* orr = cur + QTl::DO_OFF + rq * 16;
    // this lane's column of the transposed tiles: the (ks, db) operands are immediate offsets
    const char* tr = cur + (QTl::TROW * ql + g) * 16;
    const float* stl = reinterpret_cast<const float*>(cur + QTl::ST_OFF);
    const int qbase = qbase0 + 32 * j;
    const bool partial = j < nqt && (qbase < qa || qbase + 32 > qb);
    // S = Q K^T (lane = key; value i of lane group g is query 16 (i >> 3) + 8 g + (i & 7))
    f32x16 sp = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 aq = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + kk * 32));
      sp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf.q[kk], sp, 0, 0, 0);
    }
    pace(D / 16);
    // P = exp2(S scale log2(e) - lse2), zero for queries outside [qa, qb) (only the first and
    // last anchor tiles are partial: one branch per tile)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 la = *reinterpret_cast<const f32x4*>(stl + 16 * h + 8 * g);
      const f32x4 lb = *reinterpret_cast<const f32x4*>(stl + 16 * h + 8 * g + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * h + e;
        sp[i] = fast_exp2(__builtin_fmaf(sp[i], c2, -(e < 4 ? la[e] : lb[e - 4])));
      }
    }
    if (partial) {
      const int lo = qa - qbase - 8 * g, hi = qb - qbase - 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 16 * (i >> 3) + (i & 7);
        if (off < lo || off >= hi) sp[i] = 0.f;
      }
    }
    bf16x8 pa[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[h][e] = static_cast<__bf16>(sp[8 * h + e]);
    // dV += P^T dO (B operand: dO^T rows, 8 queries each)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int toff = QTl::DOT_OFF + (QTl::TROW * 32 * db + 2 * ks) * 16;  // compile-time
        const bf16x8 bo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tr + toff));
        accV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], bo, accV[db], 0, 0, 0);
      }
    pace(2 * (D / 32));
    // dP = dO V^T
    f32x16 dp = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 ao = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(orr + kk * 32));
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf.q[kk], dp, 0, 0, 0);
    }
    pace(D / 16);
    // dS = P (dP - D), with the same bf16-rounded P that entered dV
    bf16x8 da[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 da4 = *reinterpret_cast<const f32x4*>(stl + 32 + 16 * h + 8 * g);
      const f32x4 db4 = *reinterpret_cast<const f32x4*>(stl + 32 + 16 * h + 8 * g + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * h + e;
        const float pr = static_cast<float>(pa[h][e]);
        da[h][e] = static_cast<__bf16>(pr * (dp[i] - (e < 4 ? da4[e] : db4[e - 4])));
      }
    }
    // dK += dS^T Q (B operand: Q^T rows)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int toff = QTl::QT_OFF + (QTl::TROW * 32 * db + 2 * ks) * 16;  // compile-time
        const bf16x8 bq = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tr + toff));
        accK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks], bq, accK[db], 0, 0, 0);
      }
    pace(2 * (D / 32));
  };

  if (ntot > 0) {
    issue(0, lds0);
    issue(1, lds1);
    if (ntot > 1) wait_but_newest();
    else __builtin_amdgcn_s_waitcnt(0x0070);
    bar();
    // tile j reads stage j & 1; only tile j+1's copies are in flight while it runs, and they
    // must land before the barrier; after it, the freed buffer takes tile j+2
    auto step = [&](int j, const char* cur, uint32_t cur_lds) __attribute__((always_inline)) {
      tile(j, cur);
      __builtin_amdgcn_s_waitcnt(0x0070);
      bar();
      issue(j + 2, cur_lds);
    };
    for (int j = 0; j < ntot; j += 2) {
      step(j, st0, lds0);
      if (j + 1 < ntot) step(j + 1, st1, lds1);
    }
  }

  // output: accumulator rows are the wave's keys (value i: key 8 (i >> 2) + 4 g + (i & 3)),
  // columns the dims (lane & 31 of each 32-dim block). Video keys are complete: dK = scale
  // dS^T Q and dV in bf16. Text keys hold one query split: fp32 partials.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kk = k0 + wv * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
    if (kk >= k1) continue;
    if (c >= 0) {
      const size_t r = (static_cast<size_t>(bh) * p.L + kk) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        dK[r + db * 32 + ql] = f32_to_bf16(accK[db][i] * p.scale);
        dV[r + db * 32 + ql] = f32_to_bf16(accV[db][i]);
      }
    } else {
      const size_t r = ((static_cast<size_t>(bh) * p.n_split + sp) * p.text_len +
                        (kk - p.text_begin)) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        textK[r + db * 32 + ql] = accK[db][i];
        textV[r + db * 32 + ql] = accV[db][i];
      }
    }
  }
}

// Key tile images of the dQ kernel (KvImage layout), one workgroup per 64-key tile of a (b, h):
// K and V rows into the padded row layout, K^T through LDS into the padded transposed layout;
// padding bytes and rows past L are zero.
template <int D>
__global__ __launch_bounds__(256) void bwd_kvimage_kernel(const bf16_t* __restrict__ K,
                                                          const bf16_t* __restrict__ V, int L,
                                                          int Lp, char* __restrict__ img,
                                                          const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  using LT = LdsTiles<D>;
  using KI = KvImage<D>;
  constexpr int PITCH = D + 8;  // bf16
  __shared__ __attribute__((aligned(16))) bf16_t sk[kBN * PITCH];
  const int bh = blockIdx.y, k0 = blockIdx.x * kBN;
  const bf16_t* Kbh = K + static_cast<size_t>(bh) * L * D;
  const bf16_t* Vbh = V + static_cast<size_t>(bh) * L * D;
  char* out = img + (static_cast<size_t>(bh) * (Lp / kBN) + blockIdx.x) * KI::BYTES;
  for (int e = threadIdx.x; e < kBN * LT::KCH; e += 256) {
    const int r = e / LT::KCH, c = e % LT::KCH;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + r < L) v = *reinterpret_cast<const u32x4*>(Kbh + static_cast<size_t>(k0 + r) * D + c * 8);
    *reinterpret_cast<u32x4*>(sk + r * PITCH + c * 8) = v;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < KI::NBLK * 64; u += 256) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (u < KI::ROWBLK * 64) {
      const bool isv = u >= LT::KBLK * 64;
      const int pu = u % (LT::KBLK * 64);
      const int r = pu / LT::KROW, c = pu % LT::KROW;
      if (r < kBN && c < LT::KCH && k0 + r < L) {
        if (isv) v = *reinterpret_cast<const u32x4*>(Vbh + static_cast<size_t>(k0 + r) * D + c * 8);
        else v = *reinterpret_cast<const u32x4*>(sk + r * PITCH + c * 8);
      }
    } else {
      // K^T row d: 16-byte piece c holds keys 8 c .. 8 c + 7 of dim d
      const int pu = u - KI::ROWBLK * 64;
      const int d = pu / LT::VROW, c = pu % LT::VROW;
      if (d < D && c < kBN / 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * c + 2 * e;
          v[e] = static_cast<uint32_t>(sk[r * PITCH + d]) |
                 (static_cast<uint32_t>(sk[(r + 1) * PITCH + d]) << 16);
        }
      }
    }
    *reinterpret_cast<u32x4*>(out + static_cast<size_t>(u) * 16) = v;
  }
}

// Start of every (b, h, chunk) bucket's gathered rows: sizes rounded up to 32, scanned in
// bucket order; gstart[NB] is the total. One workgroup.
__global__ __launch_bounds__(1024) void bwd_gather_scan_kernel(const int32_t* __restrict__ bucket_off,
                                                               int NB,
                                                               int32_t* __restrict__ gstart,
                                                               const uint32_t* __restrict__ chk) {
  __shared__ int32_t part[1024];
  if (layout_rejected(chk)) return;
  const int per = (NB + 1023) / 1024;
  const int a = threadIdx.x * per;
  const int e = a + per < NB ? a + per : NB;
  auto padded = [&](int i) { return (bucket_off[i + 1] - bucket_off[i] + 31) & ~31; };
  int sum = 0;
  for (int i = a; i < e; ++i) sum += padded(i);
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = static_cast<int>(threadIdx.x) >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
  for (int i = a; i < e; ++i) {
    gstart[i] = run;
    run += padded(i);
  }
  if (threadIdx.x == 1023) gstart[NB] = part[1023];
}

// The key-centric kernel's (b, h, key tile) items in kXcds contiguous ranges of about equal
// cost: an item costs its 32-query blocks (the anchor query range's, plus the gathered blocks
// of its chunk's bucket, known once gstart is) and kKeyTileFixed. Range x starts at the first
// item whose cost prefix reaches x / kXcds of the total, kept within xcd_slots(max_ktiles, BH)
// items. One workgroup of 1024: per-thread sums over contiguous items, a block scan, then the
// thread whose items hold a range start finds it. out[x], x = 0..kXcds.
__global__ __launch_bounds__(1024) void bwd_key_split_kernel(
    const int32_t* __restrict__ ktiles, const int32_t* __restrict__ n_ktiles,
    const int32_t* __restrict__ gstart, int C, int BH, int max_ktiles,
    int32_t* __restrict__ out, const uint32_t* __restrict__ chk) {
  __shared__ long long part[1024];
  __shared__ long long raw[kXcds];
  if (layout_rejected(chk)) return;
  const int nkt = n_ktiles[0];
  const long long nwork = static_cast<long long>(nkt) * BH;
  auto cost = [&](long long lid) -> long long {
    const int bh = static_cast<int>(lid / nkt);
    const int32_t* kt = ktiles + 6 * (lid % nkt);
    const int c = kt[2], qa = kt[3], qb = kt[4];
    long long n = qb > qa ? ((qb - 1) >> 5) - (qa >> 5) + 1 : 0;
    if (c >= 0) {
      const int b = bh * C + c;
      n += (gstart[b + 1] - gstart[b]) >> 5;
    }
    return n + kKeyTileFixed;
  };
  const long long per = (nwork + 1023) / 1024;
  const long long a = threadIdx.x * per;
  const long long e = a + per < nwork ? a + per : nwork;
  long long sum = 0;
  for (long long i = a; i < e; ++i) sum += cost(i);
  part[threadIdx.x] = sum;
  if (threadIdx.x < kXcds) raw[threadIdx.x] = nwork;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const long long v = static_cast<int>(threadIdx.x) >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  const long long total = part[1023];
  const long long incl = part[threadIdx.x], excl = incl - sum;
  for (int x = 1; x < kXcds; ++x) {
    const long long target = total * x / kXcds;
    if (target <= 0) {
      if (threadIdx.x == 0) raw[x] = 0;
    } else if (excl < target && target <= incl) {
      long long run = excl;
      for (long long i = a; i < e; ++i) {
        run += cost(i);
        if (run >= target) {
          raw[x] = i + 1;
          break;
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long slots = xcd_slots(max_ktiles, BH);
    long long prev = 0;
    out[0] = 0;
    for (int x = 1; x < kXcds; ++x) {
      long long lo = raw[x];
      const long long lo_min = nwork - (kXcds - x) * slots;
      if (lo < prev) lo = prev;
      if (lo < lo_min) lo = lo_min;
      if (lo > prev + slots) lo = prev + slots;
      if (lo > nwork) lo = nwork;
      out[x] = static_cast<int32_t>(lo);
      prev = lo;
    }
    out[kXcds] = static_cast<int32_t>(nwork);
  }
}

// Query tile images (QTiles layout) for the key-centric kernel: 32 queries' Q and dO rows, their
// transposes and lse2, D, padded exactly as the kernel stages them. tok[r] is the query of row
// r, or -1 for a pad (zero rows, lse2 = +inf so that P = 0, D = 0); padding bytes are zero.
// Called by a whole workgroup of 256.
template <int D>
__device__ __forceinline__ void build_qblock(const bf16_t* __restrict__ Qbh,
                                             const bf16_t* __restrict__ dObh,
                                             const float* __restrict__ l2bh,
                                             const float* __restrict__ Dbh, const int32_t* tok,
                                             bf16_t* sq, bf16_t* so, float* sst,
                                             char* __restrict__ img) {
  using QTl = QTiles<D>;
  constexpr int PITCH = D + 4;  // bf16; rows 8 apart land 16 banks apart
  constexpr int CPR = D / 8;    // 16-byte pieces per row
  constexpr int RU = QTl::RBLK * 64, TU = QTl::TBLK * 64;  // 16-byte units per region
  if (threadIdx.x < 32) {
    const int t = tok[threadIdx.x];
    sst[threadIdx.x] = t >= 0 ? l2bh[t] : __builtin_inff();
    sst[32 + threadIdx.x] = t >= 0 ? Dbh[t] : 0.f;
  }
  for (int id = threadIdx.x; id < 32 * CPR; id += 256) {
    const int r = id / CPR, c = id % CPR;
    const int t = tok[r];
    u32x4 vq = {0u, 0u, 0u, 0u}, vo = {0u, 0u, 0u, 0u};
    if (t >= 0) {
      vq = *reinterpret_cast<const u32x4*>(Qbh + static_cast<size_t>(t) * D + c * 8);
      vo = *reinterpret_cast<const u32x4*>(dObh + static_cast<size_t>(t) * D + c * 8);
    }
    u32x2* lq = reinterpret_cast<u32x2*>(sq + r * PITCH + c * 8);
    u32x2* lo = reinterpret_cast<u32x2*>(so + r * PITCH + c * 8);
    lq[0] = u32x2{vq[0], vq[1]};
    lq[1] = u32x2{vq[2], vq[3]};
    lo[0] = u32x2{vo[0], vo[1]};
    lo[1] = u32x2{vo[2], vo[3]};
  }
  __syncthreads();
  // every 16-byte unit of the image, in order (coalesced stores)
  for (int u = threadIdx.x; u < QTl::NBLK * 64; u += 256) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (u < 2 * RU) {
      const bf16_t* src = u < RU ? sq : so;
      const int pu = u % RU;
      const int r = pu / QTl::RROW, c = pu % QTl::RROW;
      if (r < QTl::T && c < CPR) {
        const u32x2* l = reinterpret_cast<const u32x2*>(src + r * PITCH + c * 8);
        const u32x2 a = l[0], b = l[1];
        v = u32x4{a[0], a[1], b[0], b[1]};
      }
    } else if (u < 2 * RU + 2 * TU) {
      // transposed row d: 16-byte piece c4 holds queries 8 c4 .. 8 c4 + 7 of dim d
      const bf16_t* src = u < 2 * RU + TU ? sq : so;
      const int pu = (u - 2 * RU) % TU;
      const int d = pu / QTl::TROW, c4 = pu % QTl::TROW;
      if (d < D && c4 < QTl::T / 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * c4 + 2 * e;
          v[e] = static_cast<uint32_t>(src[r * PITCH + d]) |
                 (static_cast<uint32_t>(src[(r + 1) * PITCH + d]) << 16);
        }
      }
    } else {
      const int pu = u - 2 * RU - 2 * TU;  // lse2 in units 0-7, D in 8-15
      if (pu < 16) v = *reinterpret_cast<const u32x4*>(sst + 4 * pu);
    }
    *reinterpret_cast<u32x4*>(img + static_cast<size_t>(u) * 16) = v;
  }
  __syncthreads();
}

// QB_SEQ: the blocks of every (b, h)'s sequence, Lp / 32 per (b, h) (rows past L are pads);
// a workgroup builds 8 blocks. QB_ROUTED: the blocks of the routed buckets, one routed tile (256
// bucket positions) per workgroup; each bucket is padded to a multiple of 32 rows and starts
// at gstart[bucket].
enum { QB_SEQ = 0, QB_ROUTED = 1 };

template <int D, int MODE>
__global__ __launch_bounds__(256) void bwd_qblock_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ dO, const float* __restrict__ Dq,
    const float* __restrict__ lse2, BwdParams p, const int32_t* __restrict__ rtiles,
    const int32_t* __restrict__ n_rtiles, const int32_t* __restrict__ bucket_off,
    const int32_t* __restrict__ bucket_q, const int32_t* __restrict__ gstart,
    char* __restrict__ blocks) {
  using QTl = QTiles<D>;
  __shared__ __attribute__((aligned(16))) bf16_t sq[32 * (D + 4)];
  __shared__ __attribute__((aligned(16))) bf16_t so[32 * (D + 4)];
  __shared__ int32_t tok[32];
  __shared__ __attribute__((aligned(16))) float sst[64];
  if (layout_rejected(p.chk)) return;
  int bh, first, end, b0 = 0, n = 0;
  size_t blk0;  // block index of position `first`
  if (MODE == QB_SEQ) {
    bh = blockIdx.y;
    first = blockIdx.x * kBwdQBM;
    end = first + kBwdQBM < p.Lp ? first + kBwdQBM : p.Lp;
    n = p.L;
    blk0 = static_cast<size_t>(bh) * (p.Lp >> 5) + (first >> 5);
  } else {
    if (static_cast<int>(blockIdx.x) >= n_rtiles[0]) return;
    const int bucket = rtiles[2 * blockIdx.x];
    first = rtiles[2 * blockIdx.x + 1];
    bh = bucket / p.C;
    b0 = bucket_off[bucket];
    n = bucket_off[bucket + 1] - b0;
    const int np = (n + 31) & ~31;
    end = first + kBwdQBM < np ? first + kBwdQBM : np;
    blk0 = static_cast<size_t>(gstart[bucket] + first) >> 5;
  }
  const bf16_t* Qbh = Q + static_cast<size_t>(bh) * p.L * D;
  const bf16_t* dObh = dO + static_cast<size_t>(bh) * p.L * D;
  const float* l2bh = lse2 + static_cast<size_t>(bh) * p.Lp;
  const float* Dbh = Dq + static_cast<size_t>(bh) * p.Lp;
  for (int i0 = first; i0 < end; i0 += 32) {
    if (threadIdx.x < 32) {
      const int idx = i0 + threadIdx.x;
      tok[threadIdx.x] = idx < n ? (MODE == QB_SEQ ? idx : bucket_q[b0 + idx]) : -1;
    }
    __syncthreads();
    build_qblock<D>(Qbh, dObh, l2bh, Dbh, tok, sq, so, sst,
                    blocks + (blk0 + ((i0 - first) >> 5)) * QTl::BYTES);
  }
}

// Text keys: dK, dV = the sum of the per-split partials, in split order.
template <int D>
__global__ __launch_bounds__(256) void bwd_text_reduce_kernel(const float* __restrict__ textK,
                                                              const float* __restrict__ textV,
                                                              BwdParams p,
                                                              bf16_t* __restrict__ dK,
                                                              bf16_t* __restrict__ dV) {
  if (layout_rejected(p.chk)) return;
  const int64_t n = static_cast<int64_t>(p.B) * p.H * p.text_len * D;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int dim = static_cast<int>(e % D);
  const int64_t rt = e / D;
  const int tk = static_cast<int>(rt % p.text_len);
  const int64_t bh = rt / p.text_len;
  float sk = 0.f, sv = 0.f;
  for (int s = 0; s < p.n_split; ++s) {
    const size_t idx = ((static_cast<size_t>(bh) * p.n_split + s) * p.text_len + tk) * D + dim;
    sk += textK[idx];
    sv += textV[idx];
  }
  const size_t out = (static_cast<size_t>(bh) * p.L + p.text_begin + tk) * D + dim;
  dK[out] = f32_to_bf16(sk * p.scale);
  dV[out] = f32_to_bf16(sv);
}

}  // namespace moc

namespace moc_host {

using moc::BwdParams;

int attn_bwd_key_rows() { return moc::kBwdKR; }

int attn_bwd_text_split(int L) {
  const int n = (L + moc::kTextSplitRows - 1) / moc::kTextSplitRows;
  return n < 1 ? 1 : n;
}

namespace {
struct BwdSizes {
  size_t dq, l2, dqp, textk, textv, kv, qb, gb, gstart;
  size_t total() const { return dq + l2 + dqp + textk + textv + kv + qb + gb + gstart; }
};
int kt_rows(int L) { return (L + moc::kBN - 1) / moc::kBN * moc::kBN; }
size_t al(size_t x) { return (x + 255) / 256 * 256; }
// gathered rows of the routed buckets: each bucket padded to a multiple of 32
size_t gather_rows(const moc_layout* lay, size_t sel) {
  const size_t nb = static_cast<size_t>(lay->B) * lay->H * lay->C;
  return (sel + 31 * nb + 31) / 32 * 32;
}
// sel: routed (query, chunk) rows the workspace holds (the varlen capacity)
BwdSizes bwd_sizes(const moc_layout* lay, size_t sel) {
  BwdSizes z;
  const size_t text = static_cast<size_t>(lay->text_end - lay->text_begin);
  const size_t ns = static_cast<size_t>(attn_bwd_text_split(lay->L));
  // D and lse2 rows are padded to Lp per (b, h) (16-byte aligned 32-query slices)
  const size_t prow = static_cast<size_t>(lay->B) * lay->H * kt_rows(lay->L);
  z.dq = al(sizeof(float) * prow);
  z.l2 = al(sizeof(float) * prow);
  z.dqp = al(sizeof(float) * (sel > 0 ? sel : 1) * lay->d);
  const size_t tp = static_cast<size_t>(lay->B) * lay->H * ns * (text > 0 ? text : 1) * lay->d;
  z.textk = al(sizeof(float) * tp);
  z.textv = al(sizeof(float) * tp);
  // key tile images of the dQ kernel, Lp / 64 per (b, h)
  const size_t kvtile = lay->d == 128 ? moc::KvImage<128>::BYTES : moc::KvImage<64>::BYTES;
  z.kv = al(static_cast<size_t>(lay->B) * lay->H * (kt_rows(lay->L) / moc::kBN) * kvtile);
  // 32-query blocks of the dK/dV kernel: the sequence's (Lp / 32 per (b, h)) and the routed
  // buckets' (each bucket padded to a multiple of 32 rows: at most sel + 31 per bucket)
  const size_t nb = static_cast<size_t>(lay->B) * lay->H * lay->C;
  const size_t gtile = lay->d == 128 ? moc::QTiles<128>::BYTES : moc::QTiles<64>::BYTES;
  z.qb = al(static_cast<size_t>(lay->B) * lay->H * (kt_rows(lay->L) / 32) * gtile);
  z.gb = al(gather_rows(lay, sel) / 32 * gtile);
  z.gstart = al((nb + 1 + 16) * sizeof(int32_t));  // + the key-tile ranges per XCD
  return z;
}
}  // namespace

size_t attn_bwd_workspace(const moc_layout* lay, int64_t routed_rows) {
  return bwd_sizes(lay, static_cast<size_t>(routed_rows)).total();
}

template <int D>
static hipError_t launch_bwd_t(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                               const void* K, const void* V, const void* O, const float* lse,
                               const void* dO, float scale, void* dQ, void* dK, void* dV,
                               void* ws, hipStream_t st) {
  using moc::bf16_t;
  const BwdSizes z = bwd_sizes(lay, static_cast<size_t>(vl->routed_cap));
  char* w = static_cast<char*>(ws);
  float* Dq = reinterpret_cast<float*>(w); w += z.dq;
  float* l2 = reinterpret_cast<float*>(w); w += z.l2;
  float* dqp = reinterpret_cast<float*>(w); w += z.dqp;
  float* textK = reinterpret_cast<float*>(w); w += z.textk;
  float* textV = reinterpret_cast<float*>(w); w += z.textv;
  char* kvimg = w; w += z.kv;
  char* qblocks = w; w += z.qb;
  char* gblocks = w; w += z.gb;
  int32_t* gstart = reinterpret_cast<int32_t*>(w); w += z.gstart;
  const int Lp = kt_rows(lay->L);
  int32_t* kranges = gstart + static_cast<size_t>(lay->B) * lay->H * lay->C + 1;

  const bf16_t* q = static_cast<const bf16_t*>(Q);
  const bf16_t* k = static_cast<const bf16_t*>(K);
  const bf16_t* v = static_cast<const bf16_t*>(V);
  const bf16_t* o = static_cast<const bf16_t*>(O);
  const bf16_t* g = static_cast<const bf16_t*>(dO);
  const int64_t rows = static_cast<int64_t>(lay->B) * lay->H * lay->L;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((moc::bwd_prep_kernel<D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                     o, g, lse, Dq, l2, rows, lay->L, Lp, vl->status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdParams p{};
  p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = vl->S;
  p.text_begin = lay->text_begin;
  p.text_len = lay->text_end - lay->text_begin;
  p.n_split = vl->n_text_split;
  p.scale_log2 = scale * moc::kLog2e;
  p.scale = scale;
  p.Lp = Lp;
  p.chk = vl->status;
  const int BH = lay->B * lay->H;
  hipLaunchKernelGGL((moc::bwd_kvimage_kernel<D>), dim3(Lp / moc::kBN, BH), dim3(256), 0, st, k,
                     v, lay->L, Lp, kvimg, vl->status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int NB = BH * lay->C;
  hipLaunchKernelGGL(moc::bwd_gather_scan_kernel, dim3(1), dim3(1024), 0, st, vl->bucket_off, NB,
                     gstart, vl->status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(moc::bwd_key_split_kernel, dim3(1), dim3(1024), 0, st, vl->ktiles,
                     vl->n_ktiles, gstart, lay->C, BH, vl->max_ktiles, kranges, vl->status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((moc::bwd_qblock_kernel<D, moc::QB_SEQ>),
                     dim3((Lp + moc::kBwdQBM - 1) / moc::kBwdQBM, BH), dim3(256), 0, st, q, g, Dq,
                     l2, p, vl->rtiles, vl->n_rtiles, vl->bucket_off, vl->bucket_q, gstart,
                     qblocks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (vl->S > 0 && vl->max_rtiles > 0) {
    hipLaunchKernelGGL((moc::bwd_qblock_kernel<D, moc::QB_ROUTED>), dim3(vl->max_rtiles),
                       dim3(256), 0, st, q, g, Dq, l2, p, vl->rtiles, vl->n_rtiles,
                       vl->bucket_off, vl->bucket_q, gstart, gblocks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (vl->S > 0 && vl->max_rtiles > 0) {
    p.max_tiles = vl->max_rtiles;
    hipLaunchKernelGGL((moc::bwd_dq_kernel<D, moc::BMODE_ROUTED>), dim3(vl->max_rtiles),
                       dim3(moc::kBwdQNT), 0, st, q, kvimg, g, Dq, l2, lay->chunk_offsets,
                       p, vl->rtiles, vl->n_rtiles, nullptr, vl->bucket_off, vl->bucket_q,
                       vl->slot, dqp, static_cast<bf16_t*>(dQ));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  p.max_tiles = vl->max_atiles;
  hipLaunchKernelGGL((moc::bwd_dq_kernel<D, moc::BMODE_ANCHOR>),
                     dim3(moc::kXcds * moc::xcd_slots(vl->max_atiles, lay->B * lay->H)),
                     dim3(moc::kBwdQNT), 0, st, q, kvimg,
                     g, Dq, l2, lay->chunk_offsets, p, vl->atiles, vl->n_atiles,
                     vl->n_atiles + moc::kCtrDq, vl->bucket_off, vl->bucket_q, vl->slot, dqp,
                     static_cast<bf16_t*>(dQ));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  p.max_tiles = vl->max_ktiles;
  hipLaunchKernelGGL((moc::bwd_dkdv_kernel<D>),
                     dim3(moc::kXcds * moc::xcd_slots(vl->max_ktiles, lay->B * lay->H)),
                     dim3(moc::kBwdKNT), 0, st, k, v, p, vl->ktiles, vl->n_ktiles, qblocks,
                     gblocks, gstart, kranges, vl->n_atiles + moc::kCtrDkdv, textK, textV,
                     static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.text_len > 0) {
    const int64_t n = static_cast<int64_t>(lay->B) * lay->H * p.text_len * D;
    hipLaunchKernelGGL((moc::bwd_text_reduce_kernel<D>), dim3((n + 255) / 256), dim3(256), 0, st,
                       textK, textV, p, static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV));
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attn_bwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                           const void* K, const void* V, const void* O, const float* lse,
                           const void* dO, float scale, void* dQ, void* dK, void* dV, void* ws,
                           size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  if (lay->dtype != MOC_BF16) return hipErrorNotSupported;
  if (vl->tile_rows != moc::kBwdQBM) return hipErrorInvalidValue;
  return lay->d == 128 ? launch_bwd_t<128>(lay, vl, Q, K, V, O, lse, dO, scale, dQ, dK, dV, ws, st)
                       : launch_bwd_t<64>(lay, vl, Q, K, V, O, lse, dO, scale, dQ, dK, dV, ws, st);
}

}  // namespace moc_host
