// K2b: outer-loop context routing - a coarse router over large context segments.
//
// Source: "Mixture of Contexts for Long Video Generation | Summary", Appendix I. Routing runs on
// two levels there for long autoregressive generation: whole segments are ranked first, by
// comparing averaged features of the current block of queries with averaged features of each
// other segment, and the ordinary chunk router then only looks inside the few best segments
// (the mandatory context stays attached).
//
// Segments are given as groups of whole chunks (seg_chunk[nseg+1]); a query's block is its own
// segment. The pass, without host synchronisation:
//   (a) segment token offsets and kinds (text / video) from the layout;
//   (b) qseg / kseg: the segment means of Q and of K: the chunk pooling kernel's double-double
//       chunk sums, merged per segment in chunk order, one binary64 division, RN to binary32
//       (the pooling rule of the chunk means, applied to the segment's tokens);
//   (c) per (b, h, query segment) one wave scores the candidate segments (video, not itself,
//       earlier when causal; binary32 dot products summed in a fixed tree order) and keeps the
//       top min(M, #candidates), an exact tie keeping the lower segment id;
//   (d) per (b, h, chunk) the candidate mask row of the inner router: the chunks of the chunk's
//       own segment and of the segments picked for it.
#include "moc_common.h"
#include "moc_params.h"

namespace moc {

__global__ __launch_bounds__(256) void outer_seg_kernel(const int32_t* __restrict__ chunk_offsets,
                                                        const int32_t* __restrict__ chunk_shot,
                                                        const int32_t* __restrict__ seg_chunk,
                                                        int nseg, int32_t* __restrict__ seg_tok,
                                                        int32_t* __restrict__ seg_text,
                                                        const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  for (int s = threadIdx.x; s <= nseg; s += blockDim.x) {
    seg_tok[s] = chunk_offsets[seg_chunk[s]];
    if (s < nseg) seg_text[s] = chunk_shot[seg_chunk[s]] < 0 ? 1 : 0;
  }
}

// Segment means from the double-double chunk sums part [B*H][C][D][2]: one workgroup per
// (segment, b*h), one thread per dim, the segment's chunks merged in ascending order.
template <int D>
__global__ __launch_bounds__(D) void outer_seg_mean_kernel(const double* __restrict__ part,
                                                           const int32_t* __restrict__ seg_chunk,
                                                           const int32_t* __restrict__ seg_tok,
                                                           int C, int nseg,
                                                           float* __restrict__ feat,
                                                           const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  const int sg = blockIdx.x, bh = blockIdx.y, j = threadIdx.x;
  double h = 0.0, l = 0.0;
  for (int c = seg_chunk[sg]; c < seg_chunk[sg + 1]; ++c) {
    const double* pc = part + ((static_cast<size_t>(bh) * C + c) * D + j) * 2;
    const double bhi = pc[0], blo = pc[1];
    // double-double merge (TwoSum of the high parts, low parts added)
    const double s = h + bhi;
    const double bp = s - h;
    const double e = (h - (s - bp)) + (bhi - bp);
    l = l + blo + e;
    h = s;
  }
  const double n = static_cast<double>(seg_tok[sg + 1] - seg_tok[sg]);
  feat[(static_cast<size_t>(bh) * nseg + sg) * D + j] = static_cast<float>((h + l) / n);
}

// One wave per (query segment, b*h). Lane l holds dims l, l + 64, ... of the query feature.
template <int D>
__global__ __launch_bounds__(64) void outer_route_kernel(const float* __restrict__ qseg,
                                                         const float* __restrict__ kseg,
                                                         const int32_t* __restrict__ seg_text,
                                                         int nseg, int M, int Ms, int causal,
                                                         int32_t* __restrict__ seg_sel,
                                                         int32_t* __restrict__ seg_nsel,
                                                         const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  constexpr int DPL = D / 64;
  const int sq = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const float* q = qseg + (static_cast<size_t>(bh) * nseg + sq) * D;
  float qv[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) qv[i] = q[lane + 64 * i];
  float bs[MOC_MAX_TOPM];
  int bc[MOC_MAX_TOPM];
#pragma unroll
  for (int i = 0; i < MOC_MAX_TOPM; ++i) { bs[i] = -__builtin_inff(); bc[i] = -1; }
  int ncand = 0;
  for (int s = 0; s < nseg; ++s) {
    if (seg_text[s] || s == sq || (causal && s >= sq)) continue;  // uniform over the wave
    ++ncand;
    const float* k = kseg + (static_cast<size_t>(bh) * nseg + s) * D;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) part = __builtin_fmaf(qv[i], k[lane + 64 * i], part);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    float cs = __shfl(part, 0);  // one value for every lane
    int ci = s;
#pragma unroll
    for (int k2 = 0; k2 < MOC_MAX_TOPM; ++k2) {  // strict '>': the lower id stays ahead on ties
      if (k2 >= M) break;
      const bool take = cs > bs[k2];
      const float ts = take ? bs[k2] : cs;
      const int tc = take ? bc[k2] : ci;
      bs[k2] = take ? cs : bs[k2];
      bc[k2] = take ? ci : bc[k2];
      cs = ts;
      ci = tc;
    }
  }
  if (lane != 0) return;
  const int n = ncand < M ? ncand : M;
  // ascending by segment id
  int f[MOC_MAX_TOPM];
#pragma unroll
  for (int i = 0; i < MOC_MAX_TOPM; ++i) f[i] = (i < n) ? bc[i] : 0x7fffffff;
#pragma unroll
  for (int r = 0; r < MOC_MAX_TOPM; ++r)
#pragma unroll
    for (int i = (r & 1); i + 1 < MOC_MAX_TOPM; i += 2)
      if (f[i] > f[i + 1]) { const int x = f[i]; f[i] = f[i + 1]; f[i + 1] = x; }
  int32_t* out = seg_sel + (static_cast<size_t>(bh) * nseg + sq) * Ms;
  for (int i = 0; i < Ms; ++i) out[i] = i < n ? f[i] : -1;
  seg_nsel[static_cast<size_t>(bh) * nseg + sq] = n;
}

// Bits of chunks [a, b) in 32-chunk word w.
__device__ __forceinline__ uint32_t outer_range_bits(int a, int b, int w) {
  const int lo = a - 32 * w > 0 ? a - 32 * w : 0;
  const int hi = b - 32 * w < 32 ? b - 32 * w : 32;
  if (hi <= lo) return 0u;
  const uint32_t ones = hi - lo == 32 ? 0xffffffffu : ((1u << (hi - lo)) - 1u);
  return ones << lo;
}

// One workgroup per (chunk, b*h): the candidate mask row of the chunk's queries.
__global__ __launch_bounds__(64) void outer_mask_kernel(const int32_t* __restrict__ seg_chunk,
                                                        int nseg,
                                                        const int32_t* __restrict__ seg_sel,
                                                        const int32_t* __restrict__ seg_nsel,
                                                        int Ms, int C, int W,
                                                        uint32_t* __restrict__ cmask,
                                                        const uint32_t* __restrict__ chk) {
  if (layout_rejected(chk)) return;
  const int cq = blockIdx.x, bh = blockIdx.y;
  // the segment holding chunk cq: the last s with seg_chunk[s] <= cq
  int lo = 0, hi = nseg;  // seg_chunk[lo] <= cq < seg_chunk[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_chunk[mid] <= cq) lo = mid;
    else hi = mid;
  }
  const int sq = lo;
  const int32_t* ss = seg_sel + (static_cast<size_t>(bh) * nseg + sq) * Ms;
  const int n = seg_nsel[static_cast<size_t>(bh) * nseg + sq];
  for (int w = threadIdx.x; w < W; w += blockDim.x) {
    uint32_t bits = outer_range_bits(seg_chunk[sq], seg_chunk[sq + 1], w);
    for (int j = 0; j < n; ++j) {
      const int s = ss[j];
      bits |= outer_range_bits(seg_chunk[s], seg_chunk[s + 1], w);
    }
    cmask[(static_cast<size_t>(bh) * C + cq) * W + w] = bits;
  }
}

}  // namespace moc

namespace moc_host {

hipError_t launch_pool_partial(const moc_layout* lay, const void* X, double* part,
                               hipStream_t st);

namespace {
size_t al(size_t x) { return (x + 255) / 256 * 256; }
struct OuterSizes {
  size_t tok, text, feat, part;
  size_t total() const { return tok + text + 2 * feat + part; }
};
OuterSizes outer_sizes(const moc_layout* lay) {
  OuterSizes z;
  z.tok = al(sizeof(int32_t) * (MOC_MAX_SEG + 1));
  z.text = al(sizeof(int32_t) * MOC_MAX_SEG);
  z.feat = al(sizeof(float) * static_cast<size_t>(lay->B) * lay->H * MOC_MAX_SEG * lay->d);
  z.part = al(sizeof(double) * 2 * static_cast<size_t>(lay->B) * lay->H * lay->C * lay->d);
  return z;
}
}  // namespace

size_t outer_workspace(const moc_layout* lay) { return outer_sizes(lay).total(); }

hipError_t launch_route_outer(const moc_layout* lay, const int32_t* seg_chunk, int nseg, int M,
                              int causal, const void* Q, const void* K, int32_t* seg_sel,
                              int32_t* seg_nsel, uint32_t* cmask, void* ws, hipStream_t st) {
  const OuterSizes z = outer_sizes(lay);
  char* w = static_cast<char*>(ws);
  int32_t* seg_tok = reinterpret_cast<int32_t*>(w); w += z.tok;
  int32_t* seg_text = reinterpret_cast<int32_t*>(w); w += z.text;
  float* qseg = reinterpret_cast<float*>(w); w += z.feat;
  float* kseg = reinterpret_cast<float*>(w); w += z.feat;
  double* part = reinterpret_cast<double*>(w); w += z.part;
  hipLaunchKernelGGL(moc::outer_seg_kernel, dim3(1), dim3(256), 0, st, lay->chunk_offsets,
                     lay->chunk_shot, seg_chunk, nseg, seg_tok, seg_text, lay->check);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int BH = lay->B * lay->H;
  // chunk sums in parallel over all chunks, then one merge per segment (Q, then K)
  for (int pass = 0; pass < 2; ++pass) {
    if ((e = launch_pool_partial(lay, pass == 0 ? Q : K, part, st)) != hipSuccess) return e;
    float* feat = pass == 0 ? qseg : kseg;
    if (lay->d == 128)
      hipLaunchKernelGGL((moc::outer_seg_mean_kernel<128>), dim3(nseg, BH), dim3(128), 0, st,
                         part, seg_chunk, seg_tok, lay->C, nseg, feat, lay->check);
    else
      hipLaunchKernelGGL((moc::outer_seg_mean_kernel<64>), dim3(nseg, BH), dim3(64), 0, st,
                         part, seg_chunk, seg_tok, lay->C, nseg, feat, lay->check);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int Ms = M < nseg ? M : nseg;
  if (lay->d == 128)
    hipLaunchKernelGGL((moc::outer_route_kernel<128>), dim3(nseg, BH), dim3(64), 0, st, qseg,
                       kseg, seg_text, nseg, Ms, Ms, causal, seg_sel, seg_nsel, lay->check);
  else
    hipLaunchKernelGGL((moc::outer_route_kernel<64>), dim3(nseg, BH), dim3(64), 0, st, qseg,
                       kseg, seg_text, nseg, Ms, Ms, causal, seg_sel, seg_nsel, lay->check);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int W = (lay->C + 31) / 32;
  hipLaunchKernelGGL(moc::outer_mask_kernel, dim3(lay->C, BH), dim3(64), 0, st, seg_chunk, nseg,
                     seg_sel, seg_nsel, Ms, lay->C, W, cmask, lay->check);
  return hipGetLastError();
}

}  // namespace moc_host
