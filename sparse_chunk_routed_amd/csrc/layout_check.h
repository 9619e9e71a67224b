// Layout content check, the same code on the host and on the device.
//
// A layout is a list of content-aligned chunks ("Mixture of Contexts for Long Video Generation |
// Summary", §3.2: chunks follow frame, shot and caption boundaries; jxzklqfsx.com write-up,
// 計算效率: the boundary tables of the packed sequence): offsets [C+1] that start at 0, increase
// strictly and end at L; one shot id per chunk, -1 exactly for the chunks of the caption range
// [tb, te), which is a union of whole chunks; and every shot's chunks next to each other.
// check_layout_bits() returns the violations as bits (0 = a valid layout). It reads only
// off[0..C] and shot[0..C-1], whatever they hold.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moc {

enum : uint32_t {
  kLayoutBadStart = 1u,       // off[0] != 0
  kLayoutNotIncreasing = 2u,  // off[c+1] <= off[c] for some c
  kLayoutBadEnd = 4u,         // off[C] != L
  kLayoutBadShotId = 8u,      // a shot id below -1
  kLayoutBadText = 16u,       // a chunk straddles [tb, te), or shot -1 is not exactly the text
  kLayoutShotSplit = 32u,     // a shot's chunks are not contiguous
};

// Violations seen by one worker of `nworkers` (worker w checks chunks w, w + nworkers, ...);
// the OR over all workers is the layout's result.
__host__ __device__ inline uint32_t check_layout_bits(const int32_t* off, const int32_t* shot,
                                                      int C, int L, int tb, int te, int w,
                                                      int nworkers) {
  uint32_t bits = 0;
  if (w == 0) {
    if (off[0] != 0) bits |= kLayoutBadStart;
    if (off[C] != L) bits |= kLayoutBadEnd;
  }
  for (int c = w; c < C; c += nworkers) {
    const int a = off[c], b = off[c + 1], s = shot[c];
    if (b <= a) bits |= kLayoutNotIncreasing;
    if (s < -1) bits |= kLayoutBadShotId;
    const bool inside = tb < te && tb <= a && b <= te;
    const bool overlap = a < te && tb < b;
    if ((overlap && !inside) || inside != (s == -1)) bits |= kLayoutBadText;
    // c starts a run of shot s: no other run of the same shot may start anywhere else
    if (s >= 0 && (c == 0 || shot[c - 1] != s)) {
      for (int e = 0; e < C; ++e)
        if (e != c && shot[e] == s && (e == 0 || shot[e - 1] != s)) bits |= kLayoutShotSplit;
    }
  }
  return bits;
}

}  // namespace moc
