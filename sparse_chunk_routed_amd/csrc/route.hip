// K2: MoC routing - score every query against the pooled chunk keys, mask, top-k, and the
// training-time drop-off / drop-in noise.
//
// Sources: "Mixture of Contexts for Long Video Generation | Summary" §3.1 (parameter-free
// dot-product router, independent per head, drop-off p ~ U(0, p_max) removing floor(p k)
// chunks, drop-in m ~ Poisson(lambda) added chunks), §3.2 (causal mask on optional edges
// i -> j with j >= i, mandatory text and own-shot links); jxzklqfsx.com write-up, section
// 計算效率 (mandatory links are masked before top-k so they take no routing budget).
//
// Candidate chunk c for query t: not text, not in the query's own shot, and c < chunk(t) when
// causal. Score s_c = q_t . kbar_c with exact products and binary32 accumulation. Top-k is a
// register insertion list per thread; an exact tie keeps the lower chunk id. The result is
// written ascending by chunk id, -1 padded to S entries.
//
// Noise (a fixed reading of "at random"): a counter-based SplitMix64 word per (seed, b, h, t,
// stream, j); p = (word >> 8) * 2^-24 * p_max; nd = min(floor(p * k), |T|) picks, each
// idx = (word * remaining) >> 32 over the ascending list of what remains. Drop-in: m is the
// first i with word < Thr_i (Poisson CDF thresholds, truncated at m_cap); picks from the
// ascending candidates not in the original top-k, the same way (the idx-th set bit of the
// allowed-and-unused chunk mask).
//
// Work decomposition: bf16 queries are scored on MFMA (32 queries per wave against 32-chunk
// blocks of kbar split into three bf16 terms). For C <= 128, route_mfma_persist_kernel stages
// the terms once per workgroup and loops over query tiles; its top list holds order-preserving
// integer keys (score bits, low 7 bits = 127 - chunk id), so an insertion is one integer
// max/min pair and scores within 2^-16 relative of each other order by lower chunk id. Larger
// C uses route_mfma_kernel (one tile per workgroup, kbar staged in blocks of 128 chunks, exact
// float ordering). fp32 queries use route_kernel: one thread per query, 256 queries per
// workgroup, one (b,h) per grid row; kbar for the (b,h) is staged through LDS in blocks of
// chunks and read by broadcast.
#include <mutex>

#include "attn_common.h"
#include "moc_params.h"

namespace moc {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t h32(uint64_t seed, int bh, int L, int t, int stream, int j) {
  uint64_t ctr = ((((static_cast<uint64_t>(bh) * L + t) * 4u + stream) << 8) | static_cast<uint64_t>(j));
  return static_cast<uint32_t>(mix64(seed + (ctr + 1) * 0x9E3779B97F4A7C15ull) >> 32);
}

// Optional candidate mask of outer-loop routing: bit c of row (bh, chunk of the query).
__device__ __forceinline__ const uint32_t* cmask_row(const RouteParams& p, int bh, int cq) {
  return p.cmask ? p.cmask + (static_cast<size_t>(bh) * p.C + cq) * p.cmask_w : nullptr;
}
__device__ __forceinline__ bool cmask_ok(const uint32_t* row, int c) {
  return !row || ((row[c >> 5] >> (c & 31)) & 1u);
}

// Final selection of one query: T = the first min(k_eff, n_allowed) entries of the sorted
// top list (bs descending, ties by lower chunk id), drop-off / drop-in, ascending write-out.
template <int KMAX, bool NOISE>
__device__ __forceinline__ void finish_query(const float (&bs)[KMAX], const int (&bc)[KMAX],
                                             int n_allowed, const RouteParams& p, int bh, int t,
                                             int cq, int sq, const int32_t* s_shot,
                                             int32_t* __restrict__ sel,
                                             int32_t* __restrict__ nsel) {
  constexpr int MC = NOISE ? MOC_MAX_DROP_IN : 0;
  const int L = p.L, C = p.C;
  (void)bs;

  // T = the first min(k_eff, n_allowed) entries; make everything else invalid.
  const int nT = p.k_eff < n_allowed ? p.k_eff : n_allowed;
  int f[KMAX + MC];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) f[i] = (i < nT && bc[i] >= 0) ? bc[i] : 0x7fffffff;
#pragma unroll
  for (int i = KMAX; i < KMAX + MC; ++i) f[i] = 0x7fffffff;
  // ascending by chunk id (odd-even transposition network over the static slots)
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
#pragma unroll
    for (int i = (r & 1); i + 1 < KMAX; i += 2)
      if (f[i] > f[i + 1]) { int x = f[i]; f[i] = f[i + 1]; f[i + 1] = x; }
  int nout = 0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) nout += f[i] != 0x7fffffff;

  if constexpr (NOISE) {
    int orig[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) orig[i] = f[i];
    const int nTv = nout;
    if (p.drop_off) {
      uint32_t r = h32(p.seed, bh, L, t, 0, 0);
      double u = static_cast<double>(r >> 8) * 0x1p-24;
      double pp = u * static_cast<double>(p.p_max);
      int nd = static_cast<int>(floor(pp * static_cast<double>(p.k_eff)));
      if (nd > nout) nd = nout;
      for (int j = 0; j < nd; ++j) {
        uint32_t w = h32(p.seed, bh, L, t, 1, j);
        int idx = static_cast<int>((static_cast<uint64_t>(w) * static_cast<uint64_t>(nout)) >> 32);
        // survivors are f[0..nout) ascending: remove f[idx] and shift the tail up
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
          const int nx = (i + 1 < KMAX) ? f[i + 1] : 0x7fffffff;
          if (i >= idx) f[i] = nx;
        }
        --nout;
      }
    }
    if (p.drop_in) {
      uint32_t r = h32(p.seed, bh, L, t, 2, 0);
      int m = p.m_cap;
      for (int i = 0; i < p.m_cap; ++i) {
        if (static_cast<uint64_t>(r) < p.thr[i]) { m = i; break; }
      }
      int npool = n_allowed - nTv;
      int nadd = m < npool ? m : npool;
      if (nadd > 0) {
        // The pool in ascending order is the allowed chunks - [0, lim) without the text chunks
        // [x0, x1) and the own shot [s0, s1) (both contiguous) - minus the original top-k and
        // the chunks picked so far. A pick is the idx-th set bit of that set, found 32 chunks
        // at a time.
        int s0 = cq, s1 = cq + 1;
        while (s0 > 0 && s_shot[s0 - 1] == sq) --s0;
        while (s1 < C && s_shot[s1] == sq) ++s1;
        int x0 = C, x1 = C;
        for (int c = 0; c < C; ++c)
          if (s_shot[c] < 0) { x0 = c; break; }
        for (int c = x0; c < C && s_shot[c] < 0; ++c) x1 = c + 1;
        const int lim = p.causal ? cq : C;
        auto range_bits = [](int a, int b, int w) -> uint32_t {
          const int lo = a - 32 * w > 0 ? a - 32 * w : 0;
          const int hi = b - 32 * w < 32 ? b - 32 * w : 32;
          if (hi <= lo) return 0u;
          const uint32_t ones = hi - lo == 32 ? 0xffffffffu : ((1u << (hi - lo)) - 1u);
          return ones << lo;
        };
        const uint32_t* crow = cmask_row(p, bh, cq);
        auto pool_word = [&](int w, int npicked) -> uint32_t {
          uint32_t bits = range_bits(0, lim, w) & ~range_bits(x0, x1, w) & ~range_bits(s0, s1, w);
          if (crow) bits &= crow[w];
#pragma unroll
          for (int i = 0; i < KMAX; ++i)
            if (orig[i] != 0x7fffffff && (orig[i] >> 5) == w) bits &= ~(1u << (orig[i] & 31));
#pragma unroll
          for (int i = KMAX; i < KMAX + MC; ++i)
            if (i - KMAX < npicked && (f[i] >> 5) == w) bits &= ~(1u << (f[i] & 31));
          return bits;
        };
        const int nw = (C + 31) >> 5;
        for (int j = 0; j < nadd; ++j) {
          uint32_t w = h32(p.seed, bh, L, t, 3, j);
          int idx = static_cast<int>((static_cast<uint64_t>(w) * static_cast<uint64_t>(npool - j)) >> 32);
          int pick = -1;
          for (int wd = 0; wd < nw && pick < 0; ++wd) {
            uint32_t bits = pool_word(wd, j);
            const int cnt = popc(bits);
            if (idx >= cnt) { idx -= cnt; continue; }
            for (int i = 0; i < idx; ++i) bits &= bits - 1u;  // drop the idx lowest set bits
            pick = 32 * wd + __builtin_ctz(bits);
          }
#pragma unroll
          for (int i = KMAX; i < KMAX + MC; ++i) if (i - KMAX == j) f[i] = pick;
          ++nout;
        }
      }
      // ascending over all slots
#pragma unroll
      for (int r2 = 0; r2 < KMAX + MC; ++r2)
#pragma unroll
        for (int i = (r2 & 1); i + 1 < KMAX + MC; i += 2)
          if (f[i] > f[i + 1]) { int x = f[i]; f[i] = f[i + 1]; f[i + 1] = x; }
    }
  }

  int32_t* so = sel + (static_cast<size_t>(bh) * L + t) * p.S;
#pragma unroll
  for (int i = 0; i < KMAX + MC; ++i)
    if (i < p.S) so[i] = f[i] == 0x7fffffff ? -1 : f[i];
  for (int i = KMAX + MC; i < p.S; ++i) so[i] = -1;
  nsel[static_cast<size_t>(bh) * L + t] = nout;
}

template <typename T, int D, int KMAX, bool NOISE>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ Q,
                                                    const float* __restrict__ kbar,
                                                    const int32_t* __restrict__ off_g,
                                                    const int32_t* __restrict__ shot_g,
                                                    RouteParams p, int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ nsel) {
  constexpr int CB = 16384 / D;  // chunks per LDS block (64 KB of fp32)
  __shared__ float kb[CB * D];
  __shared__ int32_t s_off[MOC_MAX_C + 1];
  __shared__ int32_t s_shot[MOC_MAX_C];
  if (layout_rejected(p.chk)) return;

  const int L = p.L, C = p.C;
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * 256;
  const int t = t0 + threadIdx.x;
  const bool live = t < L;

  for (int i = threadIdx.x; i <= C; i += 256) s_off[i] = off_g[i];
  for (int i = threadIdx.x; i < C; i += 256) s_shot[i] = shot_g[i];
  __syncthreads();

  const int tq = live ? t : L - 1;
  const int cq = chunk_of(s_off, C, tq);
  const int sq = s_shot[cq];
  const uint32_t* crow = cmask_row(p, bh, cq);
  // highest chunk any thread of this block may need
  int c_end = C;
  if (p.causal) {
    int tl = t0 + 255 < L ? t0 + 255 : L - 1;
    c_end = chunk_of(s_off, C, tl);  // candidates satisfy c < chunk(t) <= chunk(tl)
  }

  float q[D];
  {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    constexpr int VEC = 16 / sizeof(T);
    const u32x4* qr = reinterpret_cast<const u32x4*>(Q + (static_cast<size_t>(bh) * L + tq) * D);
#pragma unroll
    for (int v = 0; v < D / VEC; ++v) {
      u32x4 raw = qr[v];
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int i = 0; i < VEC; ++i) q[v * VEC + i] = to_f32<T>(e[i]);
    }
  }

  float bs[KMAX];
  int bc[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) { bs[i] = -__builtin_inff(); bc[i] = -1; }
  int n_allowed = 0;

  const float* kbh = kbar + static_cast<size_t>(bh) * C * D;
  for (int cb0 = 0; cb0 < c_end; cb0 += CB) {
    const int ncb = (c_end - cb0) < CB ? (c_end - cb0) : CB;
    __syncthreads();
    for (int i = threadIdx.x; i < ncb * D / 4; i += 256)
      reinterpret_cast<f32x4*>(kb)[i] = reinterpret_cast<const f32x4*>(kbh + static_cast<size_t>(cb0) * D)[i];
    __syncthreads();
    for (int cc = 0; cc < ncb; ++cc) {
      const int c = cb0 + cc;
      const int sc = s_shot[c];
      const bool ok = live && sc >= 0 && sc != sq && (!p.causal || c < cq) && cmask_ok(crow, c);
      if (!__builtin_amdgcn_ballot_w64(ok)) continue;
      const f32x4* kr = reinterpret_cast<const f32x4*>(kb + cc * D);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int j = 0; j < D / 4; ++j) {
        f32x4 kv = kr[j];
        a0 = __builtin_fmaf(q[4 * j + 0], kv.x, a0);
        a1 = __builtin_fmaf(q[4 * j + 1], kv.y, a1);
        a2 = __builtin_fmaf(q[4 * j + 2], kv.z, a2);
        a3 = __builtin_fmaf(q[4 * j + 3], kv.w, a3);
      }
      if (!ok) continue;
      ++n_allowed;
      float cs = (a0 + a1) + (a2 + a3);
      int ci = c;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {  // strict '>' keeps earlier (lower-id) chunks ahead on ties
        const bool take = cs > bs[i];
        const float ts = take ? bs[i] : cs;
        const int tc = take ? bc[i] : ci;
        bs[i] = take ? cs : bs[i];
        bc[i] = take ? ci : bc[i];
        cs = ts;
        ci = tc;
      }
    }
  }
  if (!live) return;
  finish_query<KMAX, NOISE>(bs, bc, n_allowed, p, bh, t, cq, sq, s_shot, sel, nsel);
}


// kbar (fp32) -> three bf16 terms hi + mid + lo per element (each the round-to-nearest-even of
// what the previous terms leave), laid out [B*H][3][C][D]. With bf16 queries every product
// q * term is exact in fp32, so the three MFMA passes score against kbar to about 2^-25.
template <int D>
__global__ __launch_bounds__(256) void route_split_kernel(const float* __restrict__ kbar,
                                                          bf16_t* __restrict__ split, int C,
                                                          int64_t n,
                                                          const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n) return;
  const int64_t per = static_cast<int64_t>(C) * D;
  const int64_t bh = e / per;
  const int64_t r = e % per;
  const float x = kbar[e];
  const bf16_t hi = f32_to_bf16(x);
  const float r1 = x - bf16_to_f32(hi);
  const bf16_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  const bf16_t lo = f32_to_bf16(r2);
  bf16_t* o = split + bh * 3 * per + r;
  o[0] = hi;
  o[per] = mid;
  o[2 * per] = lo;
}

// Routing for bf16 queries on MFMA: each wave scores 32 queries against 32-chunk blocks,
// S^T = kbar_block Q^T summed over the three bf16 terms (fp32 accumulation). In the 32x32
// output layout a lane holds one query and 16 chunks of the block (lanes l and l^32 split the
// block), visited in ascending chunk order; each lane keeps its own top list, then the two
// lists of a query are merged (ties by lower chunk id) and the even half-wave finishes.
template <int D, int KMAX, bool NOISE>
__global__ __launch_bounds__(512) void route_mfma_kernel(const bf16_t* __restrict__ Q,
                                                         const bf16_t* __restrict__ split,
                                                         const int32_t* __restrict__ off_g,
                                                         const int32_t* __restrict__ shot_g,
                                                         RouteParams p, int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ nsel) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  constexpr int NW = 8;
  constexpr int QPB = 32 * NW;
  constexpr int CB = 128;            // chunks per LDS stage
  constexpr int KSTR = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t ks[3 * CB * KSTR];
  __shared__ int32_t s_off[MOC_MAX_C + 1];
  __shared__ int32_t s_shot[MOC_MAX_C];
  if (layout_rejected(p.chk)) return;

  const int L = p.L, C = p.C;
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * QPB;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int t = t0 + wv * 32 + ql;
  const bool live = t < L;
  const int tq = live ? t : L - 1;

  for (int i = threadIdx.x; i <= C; i += blockDim.x) s_off[i] = off_g[i];
  for (int i = threadIdx.x; i < C; i += blockDim.x) s_shot[i] = shot_g[i];
  __syncthreads();
  const int cq = chunk_of(s_off, C, tq);
  const int sq = s_shot[cq];
  // chunk limits: candidates satisfy c < chunk(t) <= chunk(last query) under causal routing
  int c_blk = C, c_wave = C;
  if (p.causal) {
    const int tb = t0 + QPB - 1 < L ? t0 + QPB - 1 : L - 1;
    const int tw = t0 + wv * 32 + 31 < L ? t0 + wv * 32 + 31 : L - 1;
    c_blk = chunk_of(s_off, C, tb);
    c_wave = chunk_of(s_off, C, tw);
  }

  QFrag<bf16_t, D> qf;
  qf.load(Q + (static_cast<size_t>(bh) * L + tq) * D, g);

  // Candidate test as index ranges: the query's own shot is the chunk range [s0, s1) (shots
  // are contiguous) and the text chunks are [x0, x1); under causal routing c < chunk(t) and
  // not in the own shot means c < s0.
  int s0 = cq, s1 = cq + 1;
  while (s0 > 0 && s_shot[s0 - 1] == sq) --s0;
  while (s1 < C && s_shot[s1] == sq) ++s1;
  int x0 = C, x1 = C;
  for (int c = 0; c < C; ++c)
    if (s_shot[c] < 0) { x0 = c; break; }
  for (int c = x0; c < C && s_shot[c] < 0; ++c) x1 = c + 1;
  const int lim = live ? (p.causal ? s0 : C) : 0;
  const uint32_t* crow = cmask_row(p, bh, cq);

  float bs[KMAX];
  int bc[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) { bs[i] = -__builtin_inff(); bc[i] = -1; }
  int n_allowed = 0;

  const size_t per = static_cast<size_t>(C) * D;
  const bf16_t* sp = split + static_cast<size_t>(bh) * 3 * per;
  for (int cb0 = 0; cb0 < c_blk; cb0 += CB) {
    const int ncb = (c_blk - cb0) < CB ? (c_blk - cb0) : CB;
    __syncthreads();
    constexpr int VPR = D / 8;  // 16-byte vectors per row
    for (int v = threadIdx.x; v < 3 * ncb * VPR; v += blockDim.x) {
      const int term = v / (ncb * VPR);
      const int rem = v % (ncb * VPR);
      const int c = rem / VPR, col = rem % VPR;
      *reinterpret_cast<u32x4*>(ks + (term * CB + c) * KSTR + col * 8) =
          *reinterpret_cast<const u32x4*>(sp + term * per + static_cast<size_t>(cb0 + c) * D + col * 8);
    }
    __syncthreads();
    for (int b32 = 0; b32 < ncb; b32 += 32) {
      if (cb0 + b32 >= c_wave) break;  // wave-uniform: no candidate of this wave beyond here
      f32x16 acc = {};
#pragma unroll
      for (int term = 0; term < 3; ++term) {
        const bf16_t* kr = ks + (term * CB + b32 + ql) * KSTR + 8 * g;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * kk));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.q[kk], acc, 0, 0, 0);
        }
      }
      const int cend = lim < cb0 + ncb ? lim : cb0 + ncb;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = cb0 + b32 + 8 * (i >> 2) + 4 * g + (i & 3);
        const bool ok = c < cend && (c < x0 || c >= x1) && (c < s0 || c >= s1) &&
                        cmask_ok(crow, c);
        n_allowed += ok ? 1 : 0;
        if (!(ok && acc[i] > bs[KMAX - 1])) continue;  // cannot enter the top list
        float cs = acc[i];
        int ci = c;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {  // strict '>' keeps earlier (lower-id) chunks ahead
          const bool take = cs > bs[k];
          const float ts = take ? bs[k] : cs;
          const int tc = take ? bc[k] : ci;
          bs[k] = take ? cs : bs[k];
          bc[k] = take ? ci : bc[k];
          cs = ts;
          ci = tc;
        }
      }
    }
  }
  // merge the partner lane's list (disjoint chunk sets: ties go to the lower chunk id)
  const int n_all = n_allowed + __shfl_xor(n_allowed, 32);
  float ps[KMAX];
  int pc[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) { ps[k] = __shfl_xor(bs[k], 32); pc[k] = __shfl_xor(bc[k], 32); }
#pragma unroll
  for (int m = 0; m < KMAX; ++m) {
    float cs = ps[m];
    int ci = pc[m];
    if (ci < 0) continue;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const bool take = cs > bs[k] || (cs == bs[k] && (bc[k] < 0 || ci < bc[k]));
      const float ts = take ? bs[k] : cs;
      const int tc = take ? bc[k] : ci;
      bs[k] = take ? cs : bs[k];
      bc[k] = take ? ci : bc[k];
      cs = ts;
      ci = tc;
    }
  }
  if (!live || g != 0) return;
  finish_query<KMAX, NOISE>(bs, bc, n_all, p, bh, t, cq, sq, s_shot, sel, nsel);
}


// Persistent form of route_mfma_kernel for C <= kRouteCB: a workgroup stages the three kbar
// terms of its (b, h) once and then scores the 256-query tiles gx, gx + G, gx + 2G, ... of that
// (b, h) with no further barriers; the next tile's queries are loaded while the current tile is
// scored. The interleaved tile order balances the causal work, which grows along the sequence.
constexpr int kRouteCB = 128;

template <int D, int KMAX, bool NOISE, int NW>
__global__ __launch_bounds__(64 * NW) void route_mfma_persist_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ split,
    const int32_t* __restrict__ off_g, const int32_t* __restrict__ shot_g, RouteParams p,
    int32_t* __restrict__ sel, int32_t* __restrict__ nsel) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  constexpr int QPB = 32 * NW;
  constexpr int KSTR = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t ks[3 * kRouteCB * KSTR];
  __shared__ int32_t s_off[MOC_MAX_C + 1];
  __shared__ int32_t s_shot[MOC_MAX_C];
  __shared__ int32_t s_sh0[kRouteCB], s_sh1[kRouteCB];  // chunk range [s_sh0, s_sh1) of c's shot
  if (layout_rejected(p.chk)) return;

  const int L = p.L, C = p.C;
  const int bh = blockIdx.y;
  const int G = gridDim.x;
  const int ntile = (L + QPB - 1) / QPB;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ql = lane & 31, g = lane >> 5;

  for (int i = threadIdx.x; i <= C; i += blockDim.x) s_off[i] = off_g[i];
  for (int i = threadIdx.x; i < C; i += blockDim.x) s_shot[i] = shot_g[i];
  {
    const size_t per = static_cast<size_t>(C) * D;
    const bf16_t* sp = split + static_cast<size_t>(bh) * 3 * per;
    constexpr int VPR = D / 8;  // 16-byte vectors per row
    // LDS rows [chunk][term]: a wave's reads of one 32-chunk block are one base address plus
    // immediate offsets; rows of chunks C..kRouteCB-1 are zero, so that their (masked) scores
    // stay finite
    for (int v = threadIdx.x; v < 3 * kRouteCB * VPR; v += blockDim.x) {
      const int term = v / (kRouteCB * VPR);
      const int rem = v % (kRouteCB * VPR);
      const int c = rem / VPR, col = rem % VPR;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (c < C)
        x = *reinterpret_cast<const u32x4*>(sp + term * per + static_cast<size_t>(c) * D + col * 8);
      *reinterpret_cast<u32x4*>(ks + (c * 3 + term) * KSTR + col * 8) = x;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    const int sc = s_shot[c];
    int a = c, b = c + 1;
    while (a > 0 && s_shot[a - 1] == sc) --a;
    while (b < C && s_shot[b] == sc) ++b;
    s_sh0[c] = a;
    s_sh1[c] = b;
  }
  __syncthreads();
  // text chunks [x0, x1) (contiguous), the same for every query
  int x0 = C, x1 = C;
  for (int c = 0; c < C; ++c)
    if (s_shot[c] < 0) { x0 = c; break; }
  for (int c = x0; c < C && s_shot[c] < 0; ++c) x1 = c + 1;

  int tile = blockIdx.x;
  if (tile >= ntile) return;
  auto tok_of = [&](int tl) __attribute__((always_inline)) {
    const int t = tl * QPB + wv * 32 + ql;
    return t < L ? t : L - 1;
  };
  QFrag<bf16_t, D> qf, qn;
  qf.load(Q + (static_cast<size_t>(bh) * L + tok_of(tile)) * D, g);
  for (; tile < ntile; tile += G) {
    const int t0 = tile * QPB;
    const int t = t0 + wv * 32 + ql;
    const bool live = t < L;
    const int tq = live ? t : L - 1;
    // the next tile's queries load while this one is scored
    if (tile + G < ntile) qn.load(Q + (static_cast<size_t>(bh) * L + tok_of(tile + G)) * D, g);
    const int cq = chunk_of(s_off, C, tq);
    const int sq = s_shot[cq];
    int c_wave = C;
    if (p.causal) {
      const int tw = t0 + wv * 32 + 31 < L ? t0 + wv * 32 + 31 : L - 1;
      c_wave = chunk_of(s_off, C, tw);
    }
    const int s0 = s_sh0[cq], s1 = s_sh1[cq];
    const int lim = live ? (p.causal ? s0 : C) : 0;
    // allowed chunks of this query as a bit set: [0, lim) without the text and own-shot ranges
    auto range_bits = [](int a, int b, int w) -> uint32_t {
      const int lo = a - 32 * w > 0 ? a - 32 * w : 0;
      const int hi = b - 32 * w < 32 ? b - 32 * w : 32;
      if (hi <= lo) return 0u;
      const uint32_t ones = hi - lo == 32 ? 0xffffffffu : ((1u << (hi - lo)) - 1u);
      return ones << lo;
    };
    uint32_t okw[kRouteCB / 32];
    int n_all = 0;
    const uint32_t* crow = cmask_row(p, bh, cq);
#pragma unroll
    for (int w = 0; w < kRouteCB / 32; ++w) {
      okw[w] = range_bits(0, lim, w) & ~range_bits(x0, x1, w) & ~range_bits(s0, s1, w);
      if (crow) okw[w] &= w < p.cmask_w ? crow[w] : 0u;
      n_all += popc(okw[w]);
    }

    // top list as order-preserving keys: the score's bits mapped to a signed int that orders
    // like the float, low 7 bits replaced by 127 - chunk id (C <= 128), so one integer max
    // orders by score and, within 2^-16 relative, by lower chunk id. An empty slot is INT_MIN.
    int tk[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) tk[i] = static_cast<int>(0x80000000u);
    for (int b32 = 0; b32 < C; b32 += 32) {
      if (b32 >= c_wave) break;  // wave-uniform: no candidate of this wave beyond here
      // Candidates outside the allowed set start from -inf, so their score stays -inf and its
      // key ranks below every finite score (above the empty slot); finish_query keeps only
      // the first min(k, #allowed) keys, which are then all allowed. A block allowed for the
      // whole wave skips this.
      const uint32_t okb = okw[b32 >> 5] >> (4 * g);  // bit 8 j + r: chunk b32 + 8 j + 4 g + r
      f32x16 acc = {};
      if (__builtin_amdgcn_ballot_w64((okb & 0x0f0f0f0fu) != 0x0f0f0f0fu) != 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = __builtin_amdgcn_sbfe(static_cast<int>(okb), 8 * (i >> 2) + (i & 3), 1);
          acc[i] = __int_as_float(~m & static_cast<int>(0xff800000u));
        }
      }
      const bf16_t* kr = ks + (b32 + ql) * 3 * KSTR + 8 * g;
#pragma unroll
      for (int term = 0; term < 3; ++term) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kr + term * KSTR + 16 * kk));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.q[kk], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = b32 + 8 * (i >> 2) + 4 * g + (i & 3);
        const float sc = acc[i];  // (a bit cast of the vector element itself reads element 0)
        const int bits = __float_as_int(sc);
        int key = bits ^ ((bits >> 31) & 0x7fffffff);
        key = (key & ~127) | (127 - c);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int hi = key > tk[k] ? key : tk[k];
          key = key > tk[k] ? tk[k] : key;
          tk[k] = hi;
        }
      }
    }
    // merge the partner lane's list (the two lanes hold disjoint chunks); read all of it
    // before either lane updates its own
    int pk[KMAX];
#pragma unroll
    for (int m = 0; m < KMAX; ++m) pk[m] = __shfl_xor(tk[m], 32);
#pragma unroll
    for (int m = 0; m < KMAX; ++m) {
      int key = pk[m];
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int hi = key > tk[k] ? key : tk[k];
        key = key > tk[k] ? tk[k] : key;
        tk[k] = hi;
      }
    }
    float bs[KMAX];
    int bc[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      bs[k] = 0.f;  // not used by finish_query
      bc[k] = tk[k] == static_cast<int>(0x80000000u) ? -1 : 127 - (tk[k] & 127);
    }
    if (live && g == 0) finish_query<KMAX, NOISE>(bs, bc, n_all, p, bh, t, cq, sq, s_shot, sel, nsel);
    qf = qn;
  }
}

}  // namespace moc

namespace moc {

// Scratch of moc_route_noalloc: the three bf16 terms of kbar ([B*H][3][C][d], as route_split_kernel
// writes them), for callers that cannot allocate. One copy per GPU, kept until the process ends
// and shared by every call on that GPU. In host code `scratch` only names the symbol: kernels get
// the device address that route_noalloc_scratch() looks up.
constexpr size_t kRouteScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

}  // namespace moc

namespace moc_host {

using moc::RouteParams;

constexpr int kMaxDevices = 64;

size_t route_noalloc_limit() { return moc::kRouteScratchBytes; }

// Device address of `scratch` on the current device, looked up once per device (with that device
// current) and cached; nullptr with the HIP error in *err when the lookup fails.
void* route_noalloc_scratch(hipError_t* err) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(moc::scratch));
    if (*err != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

template <typename T, int D, int KMAX, bool NOISE>
static hipError_t launch_route_t(const moc_layout* lay, const RouteParams& p, const void* Q,
                                 const float* kbar, int32_t* sel, int32_t* nsel, void* ws,
                                 hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    // bf16 queries: split kbar into the workspace, then score on MFMA
    moc::bf16_t* split = static_cast<moc::bf16_t*>(ws);
    const int64_t n = static_cast<int64_t>(lay->B) * lay->H * lay->C * D;
    hipLaunchKernelGGL((moc::route_split_kernel<D>), dim3((n + 255) / 256), dim3(256), 0, st,
                       kbar, split, lay->C, n, p.chk);
    const int ntile = (lay->L + 255) / 256;
    const int BH = lay->B * lay->H;
    if (lay->C <= moc::kRouteCB) {
      // at most one workgroup per CU (one round), each taking every G-th query tile of its
      // (b, h); 16 waves per workgroup where the registers of a query allow it (no noise,
      // top-k <= 4), else 8
      constexpr int NW = (NOISE || KMAX > 4) ? 8 : 16;
      const int ntp = (lay->L + 32 * NW - 1) / (32 * NW);
      int G = 256 / BH;
      if (G < 1) G = 1;
      if (G > ntp) G = ntp;
      hipLaunchKernelGGL((moc::route_mfma_persist_kernel<D, KMAX, NOISE, NW>), dim3(G, BH),
                         dim3(64 * NW), 0, st, static_cast<const moc::bf16_t*>(Q), split,
                         lay->chunk_offsets, lay->chunk_shot, p, sel, nsel);
    } else {
      hipLaunchKernelGGL((moc::route_mfma_kernel<D, KMAX, NOISE>), dim3(ntile, BH), dim3(512),
                         0, st, static_cast<const moc::bf16_t*>(Q), split, lay->chunk_offsets,
                         lay->chunk_shot, p, sel, nsel);
    }
  } else {
    (void)ws;
    dim3 grid((lay->L + 255) / 256, lay->B * lay->H);
    hipLaunchKernelGGL((moc::route_kernel<T, D, KMAX, NOISE>), grid, dim3(256), 0, st,
                       static_cast<const T*>(Q), kbar, lay->chunk_offsets, lay->chunk_shot, p,
                       sel, nsel);
  }
  return hipGetLastError();
}

template <typename T, int D, bool NOISE>
static hipError_t launch_route_k(const moc_layout* lay, const RouteParams& p, const void* Q,
                                 const float* kbar, int32_t* sel, int32_t* nsel, void* ws,
                                 hipStream_t st) {
  if (p.k_eff <= 2) return launch_route_t<T, D, 2, NOISE>(lay, p, Q, kbar, sel, nsel, ws, st);
  if (p.k_eff <= 4) return launch_route_t<T, D, 4, NOISE>(lay, p, Q, kbar, sel, nsel, ws, st);
  if (p.k_eff <= 8) return launch_route_t<T, D, 8, NOISE>(lay, p, Q, kbar, sel, nsel, ws, st);
  if (p.k_eff <= 16) return launch_route_t<T, D, 16, NOISE>(lay, p, Q, kbar, sel, nsel, ws, st);
  return launch_route_t<T, D, 32, NOISE>(lay, p, Q, kbar, sel, nsel, ws, st);
}

template <typename T, int D>
static hipError_t launch_route_n(const moc_layout* lay, const RouteParams& p, const void* Q,
                                 const float* kbar, int32_t* sel, int32_t* nsel, void* ws,
                                 hipStream_t st) {
  if (p.drop_off || p.drop_in) return launch_route_k<T, D, true>(lay, p, Q, kbar, sel, nsel, ws, st);
  return launch_route_k<T, D, false>(lay, p, Q, kbar, sel, nsel, ws, st);
}

size_t route_workspace(const moc_layout* lay) {
  if (lay->dtype != MOC_BF16) return 0;
  return static_cast<size_t>(lay->B) * lay->H * lay->C * lay->d * 3 * sizeof(moc::bf16_t);
}

hipError_t launch_route(const moc_layout* lay, const RouteParams& p, const void* Q,
                        const float* kbar, int32_t* sel, int32_t* nsel, void* ws, hipStream_t st) {
  if (lay->dtype == MOC_BF16) {
    return lay->d == 128 ? launch_route_n<moc::bf16_t, 128>(lay, p, Q, kbar, sel, nsel, ws, st)
                         : launch_route_n<moc::bf16_t, 64>(lay, p, Q, kbar, sel, nsel, ws, st);
  }
  return lay->d == 128 ? launch_route_n<float, 128>(lay, p, Q, kbar, sel, nsel, ws, st)
                       : launch_route_n<float, 64>(lay, p, Q, kbar, sel, nsel, ws, st);
}

}  // namespace moc_host
