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
// ascending candidates not in the original top-k, the same way.
//
// Work decomposition: one thread per query, 256 queries per workgroup, one (b,h) per
// grid row; kbar for the (b,h) is staged through LDS in blocks of chunks and read by broadcast.
#include "moc_common.h"
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

template <typename T, int D, int KMAX, bool NOISE>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ Q,
                                                    const float* __restrict__ kbar,
                                                    const int32_t* __restrict__ off_g,
                                                    const int32_t* __restrict__ shot_g,
                                                    RouteParams p, int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ nsel) {
  constexpr int CB = 16384 / D;  // chunks per LDS block (64 KB of fp32)
  constexpr int MC = NOISE ? MOC_MAX_DROP_IN : 0;
  __shared__ float kb[CB * D];
  __shared__ int32_t s_off[MOC_MAX_C + 1];
  __shared__ int32_t s_shot[MOC_MAX_C];

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
      const bool ok = live && sc >= 0 && sc != sq && (!p.causal || c < cq);
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
      for (int j = 0; j < nadd; ++j) {
        uint32_t w = h32(p.seed, bh, L, t, 3, j);
        int idx = static_cast<int>((static_cast<uint64_t>(w) * static_cast<uint64_t>(npool - j)) >> 32);
        int cnt = 0;
        int pick = -1;
        for (int c = 0; c < C && pick < 0; ++c) {
          const int sc = s_shot[c];
          if (!(sc >= 0 && sc != sq && (!p.causal || c < cq))) continue;
          bool used = false;
#pragma unroll
          for (int i = 0; i < KMAX; ++i) used |= orig[i] == c;
#pragma unroll
          for (int i = KMAX; i < KMAX + MC; ++i) used |= f[i] == c;
          if (used) continue;
          if (cnt == idx) pick = c;
          ++cnt;
        }
#pragma unroll
        for (int i = KMAX; i < KMAX + MC; ++i) if (i - KMAX == j) f[i] = pick;
        ++nout;
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

}  // namespace moc

namespace moc_host {

using moc::RouteParams;

template <typename T, int D, int KMAX, bool NOISE>
static hipError_t launch_route_t(const moc_layout* lay, const RouteParams& p, const void* Q,
                                 const float* kbar, int32_t* sel, int32_t* nsel,
                                 hipStream_t st) {
  dim3 grid((lay->L + 255) / 256, lay->B * lay->H);
  hipLaunchKernelGGL((moc::route_kernel<T, D, KMAX, NOISE>), grid, dim3(256), 0, st,
                     static_cast<const T*>(Q), kbar, lay->chunk_offsets, lay->chunk_shot, p,
                     sel, nsel);
  return hipGetLastError();
}

template <typename T, int D, bool NOISE>
static hipError_t launch_route_k(const moc_layout* lay, const RouteParams& p, const void* Q,
                                 const float* kbar, int32_t* sel, int32_t* nsel,
                                 hipStream_t st) {
  if (p.k_eff <= 2) return launch_route_t<T, D, 2, NOISE>(lay, p, Q, kbar, sel, nsel, st);
  if (p.k_eff <= 4) return launch_route_t<T, D, 4, NOISE>(lay, p, Q, kbar, sel, nsel, st);
  if (p.k_eff <= 8) return launch_route_t<T, D, 8, NOISE>(lay, p, Q, kbar, sel, nsel, st);
  if (p.k_eff <= 16) return launch_route_t<T, D, 16, NOISE>(lay, p, Q, kbar, sel, nsel, st);
  return launch_route_t<T, D, 32, NOISE>(lay, p, Q, kbar, sel, nsel, st);
}

template <typename T, int D>
static hipError_t launch_route_n(const moc_layout* lay, const RouteParams& p, const void* Q,
                                 const float* kbar, int32_t* sel, int32_t* nsel,
                                 hipStream_t st) {
  if (p.drop_off || p.drop_in) return launch_route_k<T, D, true>(lay, p, Q, kbar, sel, nsel, st);
  return launch_route_k<T, D, false>(lay, p, Q, kbar, sel, nsel, st);
}

hipError_t launch_route(const moc_layout* lay, const RouteParams& p, const void* Q,
                        const float* kbar, int32_t* sel, int32_t* nsel, hipStream_t st) {
  if (lay->dtype == MOC_BF16) {
    return lay->d == 128 ? launch_route_n<moc::bf16_t, 128>(lay, p, Q, kbar, sel, nsel, st)
                         : launch_route_n<moc::bf16_t, 64>(lay, p, Q, kbar, sel, nsel, st);
  }
  return lay->d == 128 ? launch_route_n<float, 128>(lay, p, Q, kbar, sel, nsel, st)
                       : launch_route_n<float, 64>(lay, p, Q, kbar, sel, nsel, st);
}

}  // namespace moc_host
