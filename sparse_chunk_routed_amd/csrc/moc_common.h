// Shared device helpers for the MoC kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moc.h"

namespace moc {

typedef uint16_t bf16_t;  // raw bfloat16 storage

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin across them

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even float -> bf16 (hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, h);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Map a physical block id to a logical one so that every XCD works on a contiguous range of
// logical work items (blocks are handed to XCDs round-robin: block b runs on XCD b % 8).
// Neighbouring logical tiles share K/V, so this keeps the sharing inside one XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  int xcd = b % kXcds;
  int idx = b / kXcds;
  int per = n / kXcds;
  int rem = n % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ int popc(uint32_t x) { return __builtin_popcount(x); }

// Work split over the XCDs: the (b, h, tile) items of the anchor attention kernels and of the
// key-centric backward are cut into kXcds contiguous ranges of about equal cost (range starts
// computed on the device before the launch), and each XCD runs its range with this many
// workgroup slots: a quarter more than an equal split by count, so that ranges of cheaper
// items still fit. max_tiles bounds the tiles of one (b, h).
__host__ __device__ inline int xcd_slots(int max_tiles, int BH) {
  const long long n = static_cast<long long>(max_tiles) * BH;
  return static_cast<int>((n * 5 / 4 + kXcds - 1) / kXcds);
}
// cost of one anchor tile: its 64-key tiles plus a fixed start-up and epilogue share
constexpr int kAnchorTileFixed = 4;

// Claim counters of the XCD ranges, in the VARLEN workspace after the anchor tile count and its
// range starts (n_atiles[kCtrFwd + y] etc.); every attention call's guard kernel zeroes them.
constexpr int kCtrFwd = 16, kCtrDq = 24, kCtrDkdv = 32, kCtrEnd = 40;

// The work item of a workgroup of a range-split kernel: the next unclaimed item of its own XCD's
// range (ranges[x] .. ranges[x + 1]), else of the other ranges in turn, so that an XCD whose
// range runs out early takes over the rest of a slower one. ctr[y] counts the claims on range
// y and only grows. Returns -1 when every range is used up. Called by one thread.
__device__ inline int claim_item(const int32_t* ranges, int32_t* ctr, int x) {
  for (int k = 0; k < kXcds; ++k) {
    const int y = (x + k) % kXcds;
    const int n = ranges[y + 1] - ranges[y];
    if (k > 0 && __hip_atomic_load(ctr + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n)
      continue;
    const int i = atomicAdd(ctr + y, 1);
    if (i < n) return ranges[y] + i;
  }
  return -1;
}
// cost of one backward key tile: its 32-query blocks plus a fixed start-up and epilogue share
constexpr int kKeyTileFixed = 2;

// The layout check word of the call (moc_layout.check, NULL when the check is off): a kernel
// whose call's layout failed the device check returns at its start, before reading anything the
// layout would index.
__device__ __forceinline__ bool layout_rejected(const uint32_t* check) {
  return check != nullptr && *check != 0u;
}

// Chunk containing token t: largest c with off[c] <= t (off has C+1 entries).
__device__ __forceinline__ int chunk_of(const int32_t* off, int C, int t) {
  int lo = 0, hi = C - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moc

// Launch-side helpers (host code in the .hip translation units).
namespace moc_host {

struct LaunchCtx {
  hipStream_t stream;
};

}  // namespace moc_host
