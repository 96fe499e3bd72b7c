// Work items of the split-sequence decode, shared by the decode kernels and the
// combine kernel (gfx950).
//
// For each (sequence b, kv head h) the quantized blocks [0, Q_b/G) are cut into
// splits of `bps` blocks, and the ring tokens [Q_b, S_b) into chunks of `rc`
// tokens (at least one chunk, possibly empty, so every pair has a partial
// state). Items are numbered sequence by sequence, then head by head, then
// split by split, quantized splits first.
#pragma once

#include "common.h"

namespace kvq {

struct ItemCounts {
  int nq;   // quantized splits
  int nr;   // ring chunks (>= 1)
};

__host__ __device__ inline ItemCounts items_of(int Q, int S, int G, int bps, int rc, int nq_max, int nr_max,
                                                bool* too_long) {
  ItemCounts c;
  const int nblk = Q / G;
  c.nq = (nblk + bps - 1) / bps;
  if (c.nq > nq_max) {
    c.nq = nq_max;
    *too_long = true;
  }
  const int r = S - Q;
  c.nr = r > 0 ? (r + rc - 1) / rc : 1;
  if (c.nr > nr_max) c.nr = nr_max;   // r <= ring capacity bounds it already
  return c;
}

#ifdef __HIPCC__
// Per-workgroup item table in LDS: prefix[b] = items before sequence b
// (per kv head), computed from the device-side lengths. All threads call it.
__device__ inline void build_prefix(const Geom& g, const int32_t* __restrict__ state, int bps, int rc, int nq_max,
                                    int nr_max, int* prefix, bool report_too_long) {
  bool too_long = false;
  for (int b = threadIdx.x; b < g.B; b += blockDim.x) {
    const ItemCounts c = items_of(state[4 * b + kStateQ], state[4 * b + kStateS], g.G, bps, rc, nq_max, nr_max,
                                  &too_long);
    prefix[b + 1] = c.nq + c.nr;
  }
  if (too_long && report_too_long) atomicOr(const_cast<int32_t*>(&state[4 * g.B]), KVQ_DEV_TOO_LONG);
  __syncthreads();
  if (threadIdx.x == 0) {
    prefix[0] = 0;
    for (int b = 0; b < g.B; ++b) prefix[b + 1] += prefix[b];
  }
  __syncthreads();
}

struct ItemRef {
  int b, h, item, cb;   // cb = items of this (sequence, head)
};

__device__ __forceinline__ ItemRef locate_item(const Geom& g, const int* prefix, int w) {
  int lo = 0, hi = g.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.Hkv * prefix[mid] <= w) lo = mid; else hi = mid - 1;
  }
  ItemRef r;
  r.b = lo;
  r.cb = prefix[lo + 1] - prefix[lo];
  const int rem = w - g.Hkv * prefix[lo];
  r.h = rem / r.cb;
  r.item = rem % r.cb;
  return r;
}
#endif

}  // namespace kvq
