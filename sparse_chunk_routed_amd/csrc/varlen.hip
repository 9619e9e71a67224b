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

// The bitmap lives in dynamic LDS, C * kInvWords words (launches pass that size), so that small
// layouts leave room for more workgroups per CU.
extern __shared__ uint32_t inv_bitmap[];

__device__ __forceinline__ void build_bitmap(uint32_t* bm, const int32_t* __restrict__ sel,
                                             const int32_t* __restrict__ nsel, int bh, int tile,
                                             const VarlenParams& p) {
  for (int i = threadIdx.x; i < p.C * kInvWords; i += blockDim.x) bm[i] = 0u;
  __syncthreads();
  const int t = tile * kInvTile + threadIdx.x;
  if (t < p.L) {
    const size_t row = static_cast<size_t>(bh) * p.L + t;
    const int32_t* sr = sel + row * p.S;
    const int n = nsel[row];
    const uint32_t bit = 1u << (threadIdx.x & 31);
    uint32_t* col = bm + (threadIdx.x >> 5);
    // the selection row is read four entries at a time whatever n is (all S entries exist),
    // so the first loads go out together with the load of n
    for (int j0 = 0; j0 < p.S; j0 += 4) {
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = j0 + u < p.S ? sr[j0 + u] : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n) atomicOr(col + c[u] * kInvWords, bit);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void inv_count_kernel(const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ nsel,
                                                        VarlenParams p,
                                                        int32_t* __restrict__ counts) {
  uint32_t* bm = inv_bitmap;
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

// Two running sums scanned together over one workgroup.
struct Sum2 {
  long long a, b;
};

// Block-wide exclusive scan of n pairs: thread t takes the contiguous items [t*per, t*per+per),
// the threads' sums are scanned in each wave with lane shuffles and across waves through `wsum`
// (2 * waves entries). get(i) -> Sum2, put(i, exclusive prefix). Returns the totals; every
// thread must call it.
template <typename Get, typename Put>
__device__ Sum2 block_scan2(int n, Get get, Put put, long long* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = static_cast<int>(blockDim.x) >> 6;
  const int per = (n + static_cast<int>(blockDim.x) - 1) / static_cast<int>(blockDim.x);
  const int i0 = tid * per;
  const int i1 = i0 + per < n ? i0 + per : n;
  long long sa = 0, sb = 0;
  for (int i = i0; i < i1; ++i) {
    const Sum2 v = get(i);
    sa += v.a;
    sb += v.b;
  }
  long long ia = sa, ib = sb;  // inclusive scan inside the wave
  for (int d = 1; d < 64; d <<= 1) {
    const long long ta = __shfl_up(ia, d), tb = __shfl_up(ib, d);
    if (lane >= d) {
      ia += ta;
      ib += tb;
    }
  }
  if (lane == 63) {
    wsum[2 * wave] = ia;
    wsum[2 * wave + 1] = ib;
  }
  __syncthreads();
  long long pa = 0, pb = 0, tot_a = 0, tot_b = 0;
  for (int w = 0; w < nw; ++w) {
    const long long xa = wsum[2 * w], xb = wsum[2 * w + 1];
    if (w < wave) {
      pa += xa;
      pb += xb;
    }
    tot_a += xa;
    tot_b += xb;
  }
  long long ra = pa + ia - sa, rb = pb + ib - sb;
  for (int i = i0; i < i1; ++i) {
    const Sum2 v = get(i);
    put(i, Sum2{ra, rb});
    ra += v.a;
    rb += v.b;
  }
  __syncthreads();  // wsum is reused by the next scan
  return Sum2{tot_a, tot_b};
}

// Writes the tiles of nseg segments (segment s: `cnt` tiles from index `base`, seg(s, base,
// cnt)). Groups of kSegLanes lanes take one segment each and write its tiles on consecutive
// lanes: emit(s, k, base + k). Segments hold a few tiles each (a bucket's rows or a chunk's
// keys), so narrow groups keep most of the workgroup's lanes busy.
constexpr int kSegLanes = 8;

template <typename Seg, typename Emit>
__device__ void emit_segments(int nseg, Seg seg, Emit emit) {
  const int sub = threadIdx.x % kSegLanes;
  const int ngroups = static_cast<int>(blockDim.x) / kSegLanes;
  for (int s = threadIdx.x / kSegLanes; s < nseg; s += ngroups) {
    int base = 0, cnt = 0;
    seg(s, base, cnt);
    for (int k = sub; k < cnt; k += kSegLanes) emit(s, k, base + k);
  }
}

// One workgroup of 1024 threads: bucket offsets, routed tiles, anchor tiles, backward key tiles
// and pair counts. Every step is a block scan or a parallel write; the layout walk (which chunks
// start and end a shot, where each group's tiles begin) is one scan over the chunks.
__global__ __launch_bounds__(1024) void inv_global_kernel(
    const int32_t* __restrict__ totals, const int32_t* __restrict__ off_g,
    const int32_t* __restrict__ shot_g, VarlenParams p, int32_t* __restrict__ bucket_off,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ rtiles, int32_t* __restrict__ n_rtiles,
    int32_t* __restrict__ atiles, int32_t* __restrict__ n_atiles, int32_t* __restrict__ ktiles,
    int32_t* __restrict__ n_ktiles, int64_t* __restrict__ pair_count) {
  __shared__ long long wsum[32];
  __shared__ int32_t off[MOC_MAX_C + 1];
  __shared__ int32_t shot[MOC_MAX_C];
  __shared__ int32_t grp[MOC_MAX_C];     // anchor group of each shot chunk
  __shared__ int32_t k_base[MOC_MAX_C];  // first backward key tile of each chunk
  // anchor groups: the text, then every run of chunks with one shot id
  __shared__ int32_t g_q0[MOC_MAX_C + 1], g_q1[MOC_MAX_C + 1], g_base[MOC_MAX_C + 1];
  __shared__ long long g_cost[MOC_MAX_C + 2];  // exclusive prefix of the groups' tile costs
  if (layout_rejected(p.chk)) return;
  for (int i = threadIdx.x; i <= p.C; i += blockDim.x) off[i] = off_g[i];
  for (int i = threadIdx.x; i < p.C; i += blockDim.x) shot[i] = shot_g[i];
  __syncthreads();
  const int NB = p.B * p.H * p.C;
  const int BM = p.tile_rows;
  const int KR = p.key_rows;
  const int tb = p.text_begin, te = p.text_end;
  const int nt_txt = te - tb;
  const int has_text = nt_txt > 0 ? 1 : 0;

  // bucket offsets and the first routed tile of each bucket (ceil(rows / BM) tiles per bucket)
  const Sum2 rt = block_scan2(
      NB,
      [&](int i) -> Sum2 {
        const int t = totals[i];
        return Sum2{t, (t + BM - 1) / BM};
      },
      [&](int i, Sum2 v) {
        bucket_off[i] = static_cast<int32_t>(v.a);
        tile_base[i] = static_cast<int32_t>(v.b);
      },
      wsum);
  if (threadIdx.x == 0) {
    bucket_off[NB] = static_cast<int32_t>(rt.a);
    n_rtiles[0] = static_cast<int32_t>(rt.b);
  }

  // The layout walk. A chunk starts a group when its shot id differs from the previous chunk's
  // (text chunks, shot -1, belong to no group); its backward key tiles are ceil(size / KR).
  auto starts = [&](int c) { return shot[c] >= 0 && (c == 0 || shot[c - 1] != shot[c]); };
  auto ends = [&](int c) { return shot[c] >= 0 && (c == p.C - 1 || shot[c + 1] != shot[c]); };
  int nsp = 0, nk_txt = 0;  // text key tiles: key blocks x the non-empty query splits
  if (has_text) {
    const int qs = (p.L + p.n_text_split - 1) / p.n_text_split;
    nsp = (p.L + qs - 1) / qs;
    if (nsp > p.n_text_split) nsp = p.n_text_split;
    nk_txt = ((nt_txt + KR - 1) / KR) * nsp;
  }
  const Sum2 wk = block_scan2(
      p.C,
      [&](int c) -> Sum2 {
        return Sum2{starts(c) ? 1 : 0,
                    shot[c] >= 0 ? (off[c + 1] - off[c] + KR - 1) / KR : 0};
      },
      [&](int c, Sum2 v) {
        // a shot chunk belongs to the last group started at or before it
        grp[c] = has_text + static_cast<int>(v.a) + (starts(c) ? 1 : 0) - 1;
        k_base[c] = nk_txt + static_cast<int>(v.b);
      },
      wsum);
  const int ng = has_text + static_cast<int>(wk.a);
  if (threadIdx.x == 0) {
    n_ktiles[0] = nk_txt + static_cast<int>(wk.b);
    if (has_text) {
      g_q0[0] = tb;
      g_q1[0] = te;
    }
  }
  for (int c = threadIdx.x; c < p.C; c += blockDim.x) {
    if (starts(c)) g_q0[grp[c]] = off[c];
    if (ends(c)) g_q1[grp[c]] = off[c + 1];
  }
  __syncthreads();

  // anchor tiles per group, and the anchor pairs of one (b, h): text^2, plus every shot query
  // against the text and its own shot
  const Sum2 an = block_scan2(
      ng,
      [&](int g) -> Sum2 {
        const long long n = g_q1[g] - g_q0[g];
        return Sum2{(n + BM - 1) / BM,
                    (has_text && g == 0) ? n * n : n * (nt_txt + n)};
      },
      [&](int g, Sum2 v) { g_base[g] = static_cast<int32_t>(v.a); }, wsum);
  if (threadIdx.x == 0) n_atiles[0] = static_cast<int32_t>(an.a);
  const long long anchor_pairs = an.b;

  // The anchor items (b, h, tile) in kXcds contiguous ranges of about equal cost, a tile
  // costing its 64-key tiles (text range, then own shot) plus kAnchorTileFixed; range x starts
  // at the first item whose cost prefix reaches x / kXcds of the total, kept within the
  // xcd_slots workgroups of an XCD. Stored at n_atiles[1 + x], x = 0..kXcds.
  auto ktiles64 = [](int a, int b) { return b > a ? ((b - 1) >> 6) - (a >> 6) + 1 : 0; };
  const Sum2 gc = block_scan2(
      ng,
      [&](int g) -> Sum2 {
        const long long n = (g_q1[g] - g_q0[g] + BM - 1) / BM;
        const bool text = has_text && g == 0;
        const long long per = ktiles64(tb, te) + (text ? 0 : ktiles64(g_q0[g], g_q1[g])) +
                              kAnchorTileFixed;
        return Sum2{n * per, 0};
      },
      [&](int g, Sum2 v) { g_cost[g] = v.a; }, wsum);
  __shared__ long long raw_lo[kXcds];
  const int nt_all = static_cast<int>(an.a);
  const long long Ch = gc.a;  // cost of one (b, h)
  const long long nwork = static_cast<long long>(nt_all) * p.B * p.H;
  if (threadIdx.x == 0) g_cost[ng] = Ch;
  __syncthreads();
  if (threadIdx.x >= 1 && threadIdx.x < kXcds) {
    const int x = threadIdx.x;
    long long lo = nwork;
    if (Ch > 0) {
      const long long target = Ch * p.B * p.H * x / kXcds;
      const long long bh = target / Ch, r = target - bh * Ch;
      int a = 0, b = ng - 1;  // last group whose cost prefix is at most r (g_cost[0] = 0)
      while (a < b) {
        const int m = (a + b + 1) >> 1;
        if (g_cost[m] <= r) a = m;
        else b = m - 1;
      }
      const int nt_g = (g_q1[a] - g_q0[a] + BM - 1) / BM;
      const long long per = (g_cost[a + 1] - g_cost[a]) / nt_g;
      lo = bh * nt_all + g_base[a] + (r - g_cost[a] + per - 1) / per;
    }
    raw_lo[x] = lo;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long slots = xcd_slots(p.max_atiles, p.B * p.H);
    long long prev = 0;
    n_atiles[1] = 0;
    for (int x = 1; x < kXcds; ++x) {
      long long lo = raw_lo[x];
      const long long lo_min = nwork - (kXcds - x) * slots;
      if (lo < prev) lo = prev;
      if (lo < lo_min) lo = lo_min;
      if (lo > prev + slots) lo = prev + slots;
      if (lo > nwork) lo = nwork;
      n_atiles[1 + x] = static_cast<int32_t>(lo);
      prev = lo;
    }
    n_atiles[1 + kXcds] = static_cast<int32_t>(nwork);
  }

  // routed tiles: (bucket, first position)
  emit_segments(
      NB,
      [&](int i, int& base, int& cnt) {
        base = tile_base[i];
        cnt = (totals[i] + BM - 1) / BM;
      },
      [&](int i, int k, int t) {
        rtiles[2 * t + 0] = i;
        rtiles[2 * t + 1] = k * BM;
      });
  // anchor tiles: query range, text range, own-shot range (empty for the text group)
  emit_segments(
      ng,
      [&](int g, int& base, int& cnt) {
        base = g_base[g];
        cnt = (g_q1[g] - g_q0[g] + BM - 1) / BM;
      },
      [&](int g, int k, int t) {
        const int q0 = g_q0[g], q1 = g_q1[g];
        const bool text = has_text && g == 0;
        const int q = q0 + k * BM;
        int32_t* a = atiles + 6 * t;
        a[0] = q; a[1] = q + BM < q1 ? q + BM : q1;
        a[2] = tb; a[3] = te;
        a[4] = text ? 0 : q0; a[5] = text ? 0 : q1;
      });
  // backward key tiles: the text keys against each query split, then every shot chunk's keys
  if (has_text) {
    const int qs = (p.L + p.n_text_split - 1) / p.n_text_split;
    for (int i = threadIdx.x; i < nk_txt; i += blockDim.x) {
      const int k0 = tb + (i / nsp) * KR, sp = i % nsp;
      const int qa = sp * qs;
      const int qb = qa + qs < p.L ? qa + qs : p.L;
      int32_t* a = ktiles + 6 * i;
      a[0] = k0; a[1] = k0 + KR < te ? k0 + KR : te;
      a[2] = -1; a[3] = qa; a[4] = qb; a[5] = sp;
    }
  }
  emit_segments(
      p.C,
      [&](int c, int& base, int& cnt) {
        base = k_base[c];
        cnt = shot[c] >= 0 ? (off[c + 1] - off[c] + KR - 1) / KR : 0;
      },
      [&](int c, int k, int t) {
        const int a0 = off[c], a1 = off[c + 1];
        const int k0 = a0 + k * KR;
        int32_t* a = ktiles + 6 * t;
        a[0] = k0; a[1] = k0 + KR < a1 ? k0 + KR : a1;
        a[2] = c; a[3] = g_q0[grp[c]]; a[4] = g_q1[grp[c]]; a[5] = -1;
      });

  // pair counts: anchor pairs + routed chunk sizes, one wave per (b, h) (integer sums: exact in
  // any order)
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int bh = threadIdx.x >> 6; bh < p.B * p.H; bh += nw) {
    long long s = 0;
    for (int c = lane; c < p.C; c += 64)
      s += static_cast<long long>(totals[bh * p.C + c]) * (off[c + 1] - off[c]);
    for (int w = 32; w > 0; w >>= 1) s += __shfl_xor(s, w);
    if (lane == 0) pair_count[bh] = anchor_pairs + s;
  }
}

__global__ __launch_bounds__(256) void inv_scatter_kernel(const int32_t* __restrict__ sel,
                                                          const int32_t* __restrict__ nsel,
                                                          const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ bucket_off,
                                                          VarlenParams p,
                                                          int32_t* __restrict__ bucket_q,
                                                          int32_t* __restrict__ slot) {
  uint32_t* bm = inv_bitmap;
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
                                    uint32_t* __restrict__ status, int32_t* __restrict__ ctr) {
  // the claim counters of the call's range-split kernels start from zero
  for (int i = kCtrFwd; i < kCtrEnd; ++i) ctr[i] = 0;
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
                     vl->routed_cap, lay->check, vl->status, vl->n_atiles);
  return hipGetLastError();
}

hipError_t launch_varlen(const moc_layout* lay, const VarlenParams& p, const int32_t* sel,
                         const int32_t* nsel, int32_t* counts, int32_t* totals,
                         int32_t* tile_base, const moc_varlen* out, int64_t* pair_count,
                         hipStream_t st) {
  const int BH = lay->B * lay->H;
  const int NB = BH * lay->C;
  // with S == 0 every nsel is 0: the counts, totals and tiles simply come out empty
  const size_t bm_bytes = sizeof(uint32_t) * lay->C * moc::kInvWords;
  hipLaunchKernelGGL(moc::inv_count_kernel, dim3(p.nqt, BH), dim3(256), bm_bytes, st, sel, nsel,
                     p, counts);
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
  hipLaunchKernelGGL(moc::inv_scatter_kernel, dim3(p.nqt, BH), dim3(256), bm_bytes, st, sel, nsel,
                     counts, out->bucket_off, p, out->bucket_q, out->slot);
  return hipGetLastError();
}

}  // namespace moc_host
