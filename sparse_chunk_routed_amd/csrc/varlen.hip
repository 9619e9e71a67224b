// K3: index inversion - per-query chunk lists -> per-(b, h, chunk) query buckets.
//
// Source: jxzklqfsx.com write-up of the MoC paper, section 計算效率 (boundary tables built
// with prefix sums, and every (query group, key group) pair packed into one variable-length
// attention problem); "Mixture of Contexts for Long Video Generation | Summary" §3.3.
//
// The routed part of the attention runs chunk-centric: all queries that picked chunk c form a
// bucket, tiles of gathered queries then read chunk c's keys and values once per tile. This
// pass builds, without any host synchronisation:
//   bucket_off[B*H*C+1]  exclusive prefix of bucket sizes,
//   bucket_q[...]        query ids per bucket, ascending (stable counting sort),
//   slot[B,H,L,S]        bucket position of each (query, selection), -1 padding,
//   rtiles / n_rtiles    routed work tiles (bucket, first position), tile_rows queries each,
//   atiles / n_atiles    anchor work tiles (query range + text range + own-shot range),
//   pair_count[B,H]      sum_t |Omega(t)| as int64.
//
// Steps: (a) per 256-query tile, an LDS bitmap [chunk][256 bits] of who picked what -> counts;
// (b) per bucket, exclusive scan over query tiles; (c) one workgroup scans bucket totals and
// emits tiles and pair counts; (d) per query tile, rank = popcount of the bitmap bits below
// the query -> stable scatter.
#include "moc_common.h"
#include "moc_params.h"

namespace moc {

constexpr int kInvTile = 256;          // queries per inversion tile
constexpr int kInvWords = kInvTile / 32;

__device__ __forceinline__ void build_bitmap(uint32_t* bm, const int32_t* __restrict__ sel,
                                             const int32_t* __restrict__ nsel, int bh, int tile,
                                             const VarlenParams& p) {
  for (int i = threadIdx.x; i < p.C * kInvWords; i += blockDim.x) bm[i] = 0u;
  __syncthreads();
  const int t = tile * kInvTile + threadIdx.x;
  if (t < p.L) {
    const size_t row = static_cast<size_t>(bh) * p.L + t;
    const int n = nsel[row];
    for (int j = 0; j < n; ++j) {
      const int c = sel[row * p.S + j];
      atomicOr(&bm[c * kInvWords + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void inv_count_kernel(const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ nsel,
                                                        VarlenParams p,
                                                        int32_t* __restrict__ counts) {
  __shared__ uint32_t bm[MOC_MAX_C * kInvWords];
  if (layout_rejected(p.chk)) return;
  const int tile = blockIdx.x, bh = blockIdx.y;
  build_bitmap(bm, sel, nsel, bh, tile, p);
  for (int c = threadIdx.x; c < p.C; c += blockDim.x) {
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kInvWords; ++w) cnt += popc(bm[c * kInvWords + w]);
    counts[(static_cast<size_t>(bh) * p.C + c) * p.nqt + tile] = cnt;
  }
}

// Exclusive scan of one bucket's per-tile counts (in place); bucket total -> totals.
__global__ __launch_bounds__(256) void inv_scan_bucket_kernel(int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ totals,
                                                              int nqt,
                                                              const uint32_t* __restrict__ chk) {
  __shared__ int32_t part[256];
  if (layout_rejected(chk)) return;
  int32_t* row = counts + static_cast<size_t>(blockIdx.x) * nqt;
  const int per = (nqt + 255) / 256;
  const int a = threadIdx.x * per;
  const int e = a + per < nqt ? a + per : nqt;
  int s = 0;
  for (int i = a; i < e; ++i) s += row[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
  for (int i = a; i < e; ++i) {
    int v = row[i];
    row[i] = run;
    run += v;
  }
  if (threadIdx.x == 255) totals[blockIdx.x] = part[255];
}

// Block-wide exclusive scan over n values with 1024 threads (values read via `get`).
template <typename Get, typename Put>
__device__ int64_t block_exclusive_scan(int n, Get get, Put put, int64_t* part) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int a = threadIdx.x * per;
  const int e = a + per < n ? a + per : n;
  int64_t s = 0;
  for (int i = a; i < e; ++i) s += get(i);
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < static_cast<int>(blockDim.x); off <<= 1) {
    int64_t v = static_cast<int>(threadIdx.x) >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int64_t run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
  for (int i = a; i < e; ++i) {
    int64_t v = get(i);
    put(i, run);
    run += v;
  }
  int64_t total = part[blockDim.x - 1];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(1024) void inv_global_kernel(
    const int32_t* __restrict__ totals, const int32_t* __restrict__ off_g,
    const int32_t* __restrict__ shot_g, VarlenParams p, int32_t* __restrict__ bucket_off,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ rtiles, int32_t* __restrict__ n_rtiles,
    int32_t* __restrict__ atiles, int32_t* __restrict__ n_atiles, int32_t* __restrict__ ktiles,
    int32_t* __restrict__ n_ktiles, int64_t* __restrict__ pair_count) {
  __shared__ int64_t part[1024];
  __shared__ int64_t s_anchor;
  __shared__ int32_t off[MOC_MAX_C + 1];
  __shared__ int32_t shot[MOC_MAX_C];
  // tile emission tables: anchor groups (text, shots) and per-chunk key tile starts
  __shared__ int32_t g_q0[MOC_MAX_C + 1], g_q1[MOC_MAX_C + 1], g_base[MOC_MAX_C + 1];
  __shared__ int32_t g_text[MOC_MAX_C + 1];
  __shared__ int32_t k_base[MOC_MAX_C], k_q0[MOC_MAX_C], k_q1[MOC_MAX_C];
  __shared__ int32_t s_ng, s_nsp, s_ntxt_k;
  if (layout_rejected(p.chk)) return;
  // the serial tile emission below walks the layout: keep it in LDS, not in global memory
  for (int i = threadIdx.x; i <= p.C; i += blockDim.x) off[i] = off_g[i];
  for (int i = threadIdx.x; i < p.C; i += blockDim.x) shot[i] = shot_g[i];
  __syncthreads();
  const int NB = p.B * p.H * p.C;
  const int BM = p.tile_rows;
  // bucket offsets
  int64_t tot = block_exclusive_scan(
      NB, [&](int i) -> int64_t { return totals[i]; },
      [&](int i, int64_t v) { bucket_off[i] = static_cast<int32_t>(v); }, part);
  if (threadIdx.x == 0) bucket_off[NB] = static_cast<int32_t>(tot);
  // routed tiles: ceil(total / BM) per bucket
  int64_t ntile = block_exclusive_scan(
      NB, [&](int i) -> int64_t { return (totals[i] + BM - 1) / BM; },
      [&](int i, int64_t v) { tile_base[i] = static_cast<int32_t>(v); }, part);
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += blockDim.x) {
    const int nt = (totals[i] + BM - 1) / BM;
    const int base = tile_base[i];
    for (int k = 0; k < nt; ++k) {
      rtiles[2 * (base + k) + 0] = i;
      rtiles[2 * (base + k) + 1] = k * BM;
    }
  }
  if (threadIdx.x == 0) n_rtiles[0] = static_cast<int32_t>(ntile);
  // Anchor tiles (shared by all (b,h)) and backward key tiles. Thread 0 lays out where each
  // group's tiles start (the text, then every shot; the text keys, then every video chunk);
  // all threads then write the tiles, in the same order a serial walk would.
  const int tb = p.text_begin, te = p.text_end;
  const int nt_txt = te - tb;
  const int KR = p.key_rows;
  if (threadIdx.x == 0) {
    int ng = 0, n = 0;
    int64_t anchor = 0;
    if (nt_txt > 0) {
      g_q0[ng] = tb; g_q1[ng] = te; g_base[ng] = n; g_text[ng] = 1; ++ng;
      n += (nt_txt + BM - 1) / BM;
      anchor += static_cast<int64_t>(nt_txt) * nt_txt;
    }
    int c = 0;
    while (c < p.C) {
      const int sh = shot[c];
      if (sh < 0) { k_q0[c] = 0; k_q1[c] = 0; ++c; continue; }
      const int c0 = c;
      while (c < p.C && shot[c] == sh) ++c;
      const int q0 = off[c0], q1 = off[c];
      for (int cc = c0; cc < c; ++cc) { k_q0[cc] = q0; k_q1[cc] = q1; }
      g_q0[ng] = q0; g_q1[ng] = q1; g_base[ng] = n; g_text[ng] = 0; ++ng;
      n += (q1 - q0 + BM - 1) / BM;
      anchor += static_cast<int64_t>(q1 - q0) * (nt_txt + (q1 - q0));
    }
    s_ng = ng;
    n_atiles[0] = n;
    s_anchor = anchor;
    // text key tiles: key blocks x the query splits that are not empty (a prefix of them)
    int nk = 0, nsp = 0;
    if (nt_txt > 0) {
      const int qs = (p.L + p.n_text_split - 1) / p.n_text_split;
      while (nsp < p.n_text_split && nsp * qs < p.L) ++nsp;
      nk = ((nt_txt + KR - 1) / KR) * nsp;
    }
    s_nsp = nsp;
    s_ntxt_k = nk;
    for (int cc = 0; cc < p.C; ++cc) {
      k_base[cc] = nk;
      if (shot[cc] >= 0) nk += (off[cc + 1] - off[cc] + KR - 1) / KR;
    }
    n_ktiles[0] = nk;
  }
  __syncthreads();
  for (int gi = 0; gi < s_ng; ++gi) {
    const int q0 = g_q0[gi], q1 = g_q1[gi];
    const int nt = (q1 - q0 + BM - 1) / BM;
    for (int k = threadIdx.x; k < nt; k += blockDim.x) {
      const int q = q0 + k * BM;
      int32_t* a = atiles + 6 * (g_base[gi] + k);
      a[0] = q; a[1] = q + BM < q1 ? q + BM : q1;
      a[2] = tb; a[3] = te;
      a[4] = g_text[gi] ? 0 : q0; a[5] = g_text[gi] ? 0 : q1;
    }
  }
  if (nt_txt > 0) {
    const int qs = (p.L + p.n_text_split - 1) / p.n_text_split;
    for (int i = threadIdx.x; i < s_ntxt_k; i += blockDim.x) {
      const int k0 = tb + (i / s_nsp) * KR, sp = i % s_nsp;
      const int qa = sp * qs;
      const int qb = qa + qs < p.L ? qa + qs : p.L;
      int32_t* a = ktiles + 6 * i;
      a[0] = k0; a[1] = k0 + KR < te ? k0 + KR : te;
      a[2] = -1; a[3] = qa; a[4] = qb; a[5] = sp;
    }
  }
  for (int cc = 0; cc < p.C; ++cc) {
    if (shot[cc] < 0) continue;
    const int a0 = off[cc], a1 = off[cc + 1];
    const int nt = (a1 - a0 + KR - 1) / KR;
    for (int k = threadIdx.x; k < nt; k += blockDim.x) {
      const int k0 = a0 + k * KR;
      int32_t* a = ktiles + 6 * (k_base[cc] + k);
      a[0] = k0; a[1] = k0 + KR < a1 ? k0 + KR : a1;
      a[2] = cc; a[3] = k_q0[cc]; a[4] = k_q1[cc]; a[5] = -1;
    }
  }
  __syncthreads();
  // pair counts: anchor pairs + routed chunk sizes, one wave per (b, h) (integer sums: exact in
  // any order)
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int bh = threadIdx.x >> 6; bh < p.B * p.H; bh += nw) {
    long long s = 0;
    for (int c = lane; c < p.C; c += 64)
      s += static_cast<long long>(totals[bh * p.C + c]) * (off[c + 1] - off[c]);
    for (int w = 32; w > 0; w >>= 1) s += __shfl_xor(s, w);
    if (lane == 0) pair_count[bh] = s_anchor + s;
  }
}

__global__ __launch_bounds__(256) void inv_scatter_kernel(const int32_t* __restrict__ sel,
                                                          const int32_t* __restrict__ nsel,
                                                          const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ bucket_off,
                                                          VarlenParams p,
                                                          int32_t* __restrict__ bucket_q,
                                                          int32_t* __restrict__ slot) {
  __shared__ uint32_t bm[MOC_MAX_C * kInvWords];
  if (layout_rejected(p.chk)) return;
  const int tile = blockIdx.x, bh = blockIdx.y;
  build_bitmap(bm, sel, nsel, bh, tile, p);
  const int t = tile * kInvTile + threadIdx.x;
  if (t >= p.L) return;
  const size_t row = static_cast<size_t>(bh) * p.L + t;
  const int n = nsel[row];
  const int w = threadIdx.x >> 5;
  const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
  for (int j = 0; j < n; ++j) {
    const int c = sel[row * p.S + j];
    const uint32_t* b = bm + c * kInvWords;
    int rank = popc(b[w] & below);
    for (int k = 0; k < w; ++k) rank += popc(b[k]);
    const size_t bucket = static_cast<size_t>(bh) * p.C + c;
    const int pos = bucket_off[bucket] + counts[bucket * p.nqt + tile] + rank;
    bucket_q[pos] = t;
    slot[row * p.S + j] = pos;
  }
  for (int j = n; j < p.S; ++j) slot[row * p.S + j] = -1;
}

// Guard of an attention call: the routing's total routed rows against the capacity its
// workspace was sized for, and the layout check word, into the varlen status word that every
// kernel of the call reads first (layout_rejected).
__global__ void varlen_guard_kernel(const int32_t* __restrict__ total, int64_t cap,
                                    const uint32_t* __restrict__ layout_word,
                                    uint32_t* __restrict__ status) {
  uint32_t st = 0u;
  if (static_cast<int64_t>(total[0]) > cap) st |= MOC_VARLEN_OVER_CAPACITY;
  if (layout_word != nullptr && layout_word[0] != 0u) st |= MOC_VARLEN_BAD_LAYOUT;
  status[0] = st;
}

}  // namespace moc

namespace moc_host {

using moc::VarlenParams;

hipError_t launch_varlen_guard(const moc_layout* lay, const moc_varlen* vl, hipStream_t st) {
  const int64_t nb = static_cast<int64_t>(lay->B) * lay->H * lay->C;
  hipLaunchKernelGGL(moc::varlen_guard_kernel, dim3(1), dim3(1), 0, st, vl->bucket_off + nb,
                     vl->routed_cap, lay->check, vl->status);
  return hipGetLastError();
}

hipError_t launch_varlen(const moc_layout* lay, const VarlenParams& p, const int32_t* sel,
                         const int32_t* nsel, int32_t* counts, int32_t* totals,
                         int32_t* tile_base, const moc_varlen* out, int64_t* pair_count,
                         hipStream_t st) {
  const int BH = lay->B * lay->H;
  const int NB = BH * lay->C;
  // with S == 0 every nsel is 0: the counts, totals and tiles simply come out empty
  hipLaunchKernelGGL(moc::inv_count_kernel, dim3(p.nqt, BH), dim3(256), 0, st, sel, nsel, p,
                     counts);
  hipLaunchKernelGGL(moc::inv_scan_bucket_kernel, dim3(NB), dim3(256), 0, st, counts, totals,
                     p.nqt, p.chk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moc::inv_global_kernel, dim3(1), dim3(1024), 0, st, totals,
                     lay->chunk_offsets, lay->chunk_shot, p, out->bucket_off, tile_base,
                     out->rtiles, out->n_rtiles, out->atiles, out->n_atiles, out->ktiles,
                     out->n_ktiles, pair_count);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moc::inv_scatter_kernel, dim3(p.nqt, BH), dim3(256), 0, st, sel, nsel,
                     counts, out->bucket_off, p, out->bucket_q, out->slot);
  return hipGetLastError();
}

}  // namespace moc_host
