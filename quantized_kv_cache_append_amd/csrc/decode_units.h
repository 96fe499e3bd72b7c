// Work units of the split-sequence decode, shared by the decode kernels and the
// combine kernel (gfx950).
//
// Every (sequence b, kv head h) pair ("pair" p = b*H_kv + h) contributes:
//   - ring units: its full-precision tokens [Q_b, S_b) in runs of `rc` tokens;
//   - big units of `ub` quantized blocks covering its leading blocks;
//   - then up to kTailUnits medium units of `um` blocks and up to kTailUnits
//     small units of `us` blocks (one set) covering its last blocks.
// A kernel that partitions the units statically over its waves instead asks
// for units of a fixed number of sets (`unit_sets`): then every quantized unit
// is a big unit of that size and there are no medium or small units.
// Units are numbered section by section -- all ring units, then all big, all
// medium and all small units -- and within a section by sequence, kv head and
// position. Waves take units in that order, so the latency-bound ring units
// start first and the units shrink towards the end of the launch, which keeps
// the last waves from idling the GPU. Each unit leaves one partial softmax state per
// query head of its group in slot u of the workspace; the combine kernel merges
// the partials of each pair.
//
// The unit sizes follow from the total number of quantized blocks on the
// device (about kUnitsTarget big units in all), so they depend only on the
// lengths and the configuration: the partition -- and with it every rounding
// in the result -- is the same from run to run, whichever wave takes a unit.
#pragma once

#include "common.h"

namespace kvq {

// About 2 big units per wave slot of a 256-CU GPU at 2 waves per SIMD: a
// unit change costs a few microseconds of a wave's time (its partial state,
// the next unit's lookup and first loads), so units are as large as the tail
// allows; the cap keeps ragged batches with many tiny sets balanced.
constexpr int kUnitsTarget = 4096;
constexpr int kMaxUnitSets = 16;     // cap on the sets of one big unit
constexpr int kTailUnits = 2;        // medium and small units per pair (at most)

// Plan words, at the start of the workspace (written by the decode kernel, read
// by the combine kernel) and in each decode workgroup's LDS.
enum {
  kPlanUnits = 0,   // units in all
  kPlanSec = 1,     // units in all of sections 0..3 (ring, big, medium, small): words 1..4
  kPlanUb = 5,      // blocks per big unit
  kPlanUm = 6,      // blocks per medium unit
  kPlanUs = 7,      // blocks per small unit
  kPlanRc = 8,      // ring tokens per ring unit
  kPlanTails = 9,   // medium and small units per pair (at most): kTailUnits or 0
  kPlanHdr = 12,    // then pre[s][B + 1] for each section s: exclusive prefix over
};                  // sequences of the section's units of one kv head; then the
                    // lengths the plan was built from: Q[B] (tokens of the low-bit
                    // blocks the units stream: all quantized blocks but the FP8
                    // tier's), S[B] (tokens after the sink) and R[B] (the ring's
                    // first token: every quantized token before it)
constexpr int kSections = 4;

__host__ __device__ inline int plan_ints(int B) { return kPlanHdr + kSections * (B + 1) + 3 * B; }
__host__ __device__ inline int plan_seq_off(int B) { return kPlanHdr + kSections * (B + 1); }
inline size_t plan_bytes(int B) { return ((size_t)plan_ints(B) * 4 + 255) & ~(size_t)255; }
// LDS bytes a decode workgroup reserves for its copy of the plan (16-byte aligned)
__host__ __device__ inline int plan_lds_bytes(int B) { return (plan_ints(B) * 4 + 15) & ~15; }

// Upper bound on the units when no sequence has more than max_blk quantized
// blocks, sets hold nb_set blocks and ring units rc tokens: ceil(C/rc) ring
// units per pair, at most max(kUnitsTarget, P*ceil(max_blk/(kMaxUnitSets*nb_set)))
// + P big units, and at most kTailUnits medium and kTailUnits small units per
// pair.
inline size_t units_max(const Geom& g, int max_blk, int nb_set, int rc, int unit_sets = 0) {
  const size_t P = (size_t)g.B * g.Hkv;
  const size_t ring = P * (size_t)((g.C + rc - 1) / rc);
  if (unit_sets > 0) {
    const size_t ub = (size_t)unit_sets * nb_set;
    return ring + P * ((max_blk + ub - 1) / ub);
  }
  const size_t cap = (size_t)kMaxUnitSets * nb_set;
  const size_t big = std::max<size_t>(kUnitsTarget, P * ((max_blk + cap - 1) / cap));
  return ring + big + P + 2 * P * kTailUnits;
}

// Blocks of sequence b's pair in each quantized section: big units cover
// [0, body), medium [body, body + mid), small [body + mid, nblk).
struct Tail {
  int mid, small;
};
__host__ __device__ inline Tail tail_of(int nblk, int um, int us, int tails) {
  Tail t;
  t.small = nblk < tails * us ? nblk : tails * us;
  const int rest = nblk - t.small;
  t.mid = rest < tails * um ? rest : tails * um;
  return t;
}

#ifdef __HIPCC__
// Inclusive prefix sum over the 64 lanes with row shifts and row broadcasts
// (DPP: no LDS round trips on the plan's critical path at kernel start).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr 1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr 2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr 4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr 8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast 15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast 31 -> rows 2, 3
  return x;
}
// Build the plan in LDS (`plan`, plan_ints(B) ints) from the device-side
// lengths: the first wave does all of it (one lane per sequence, 64 sequences
// at a time), the others wait at the closing barrier; every thread of the
// workgroup calls it. Sequences with more than max_blk quantized blocks are cut
// to max_blk (the caller's max_seq_tokens was too small) and, if
// report_too_long, flag KVQ_DEV_TOO_LONG.
__device__ inline void build_unit_plan(const Geom& g, int32_t* state, int max_blk, int nb_set, int rc, int* plan,
                                       bool report_too_long, int unit_sets = 0) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int* seqQ = plan + plan_seq_off(g.B);
    int* seqS = seqQ + g.B;
    int* seqR = seqS + g.B;
    // pass 1: lengths into the plan, quantized sets in all
    int sets = 0;
    bool too_long = false;
    for (int b = lane; b < g.B; b += 64) {
      const int Q = state[4 * b + kStateQ], S = max(state[4 * b + kStateS] - g.P, 0);   // tokens after the sink
      seqQ[b] = (Q / g.G - min(Q / g.G, g.W)) * g.G;   // the FP8 tier's blocks are read elsewhere
      seqS[b] = S;
      seqR[b] = Q;
      const int nblk = seqQ[b] / g.G;
      too_long |= nblk > max_blk;
      sets += (min(nblk, max_blk) + nb_set - 1) / nb_set;
    }
    if (too_long && report_too_long) atomicOr(&state[4 * g.B], KVQ_DEV_TOO_LONG);
    sets = __builtin_amdgcn_readlane(wave_incl_scan(sets), 63);
    const long long tot = (long long)sets * g.Hkv;
    int ub_sets = (int)((tot + kUnitsTarget - 1) / kUnitsTarget);
    ub_sets = max(1, min(kMaxUnitSets, ub_sets));
    if (unit_sets > 0) ub_sets = unit_sets;
    const int tails = unit_sets > 0 ? 0 : kTailUnits;
    const int ub = ub_sets * nb_set, um = unit_sets > 0 ? ub : max(1, ub_sets / 4) * nb_set;
    const int us = unit_sets > 0 ? ub : nb_set;
    // pass 2: units per section and sequence, exclusive prefixes over sequences
    int carry[kSections] = {0, 0, 0, 0};
    for (int b0 = 0; b0 < g.B; b0 += 64) {
      const int b = b0 + lane;
      int cnt[kSections] = {0, 0, 0, 0};
      if (b < g.B) {
        const int Q = seqQ[b], S = seqS[b], R0 = seqR[b];
        const int nblk = min(Q / g.G, max_blk);
        const Tail t = tail_of(nblk, um, us, tails);
        cnt[0] = (min(max(S - R0, 0), g.C) + rc - 1) / rc;
        cnt[1] = (nblk - t.mid - t.small + ub - 1) / ub;
        cnt[2] = (t.mid + um - 1) / um;
        cnt[3] = (t.small + us - 1) / us;
      }
      int inc[kSections];
#pragma unroll
      for (int k = 0; k < kSections; ++k) inc[k] = wave_incl_scan(cnt[k]);
#pragma unroll
      for (int k = 0; k < kSections; ++k) {
        if (b < g.B) plan[kPlanHdr + k * (g.B + 1) + b] = carry[k] + inc[k] - cnt[k];
        carry[k] += __builtin_amdgcn_readlane(inc[k], 63);
      }
    }
    if (lane == 0) {
      int tot_units = 0;
#pragma unroll
      for (int k = 0; k < kSections; ++k) {
        plan[kPlanHdr + k * (g.B + 1) + g.B] = carry[k];
        plan[kPlanSec + k] = g.Hkv * carry[k];
        tot_units += g.Hkv * carry[k];
      }
      plan[kPlanUnits] = tot_units;
      plan[kPlanUb] = ub;
      plan[kPlanUm] = um;
      plan[kPlanUs] = us;
      plan[kPlanRc] = rc;
      plan[kPlanTails] = tails;
    }
  }
  __syncthreads();
}

// What unit u is.
struct Unit {
  int b, h;
  bool ring;
  int begin, end;   // ring: token range; else quantized block range
};

// Largest b in [0, B) with pre[b] * Hkv <= v (pre non-decreasing, pre[0] = 0).
__device__ __forceinline__ int find_seq(const int* pre, int B, int Hkv, int v) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (Hkv * pre[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Unit u of the plan (in LDS: every read of it is an LDS read). Sequences are
// cut to max_blk quantized blocks, as when the plan was built.
__device__ inline Unit locate_unit(const Geom& g, const int* plan, int u, int max_blk) {
  int v = u, sec = 0;
  while (sec < kSections - 1 && v >= plan[kPlanSec + sec]) {
    v -= plan[kPlanSec + sec];
    ++sec;
  }
  const int* pre = plan + kPlanHdr + sec * (g.B + 1);
  const int b = find_seq(pre, g.B, g.Hkv, v);
  const int n = pre[b + 1] - pre[b];
  v -= g.Hkv * pre[b];
  Unit r;
  r.b = b;
  r.h = v / n;
  const int i = v % n;
  r.ring = sec == 0;
  const int Q = plan[plan_seq_off(g.B) + b];
  if (sec == 0) {
    const int S = plan[plan_seq_off(g.B) + g.B + b];
    const int rc = plan[kPlanRc];
    r.begin = plan[plan_seq_off(g.B) + 2 * g.B + b] + i * rc;
    r.end = min(S, r.begin + rc);
  } else {
    const int nblk = min(Q / g.G, max_blk);
    const int um = plan[kPlanUm], us = plan[kPlanUs];
    const Tail t = tail_of(nblk, um, us, plan[kPlanTails]);
    const int body = nblk - t.mid - t.small;
    const int size = sec == 1 ? plan[kPlanUb] : (sec == 2 ? um : us);
    const int start = sec == 1 ? 0 : (sec == 2 ? body : body + t.mid);
    const int stop = sec == 1 ? body : (sec == 2 ? body + t.mid : nblk);
    r.begin = start + i * size;
    r.end = min(stop, r.begin + size);
  }
  return r;
}

// Static partition of the plan's units over W persistent waves: contiguous
// ranges, in plan order, of equal estimated cost (bytes streamed; a ring
// unit costs `ring_cost`, a quantized unit its blocks times `rec_bytes`).
// The cost is piecewise linear over the sections, so each wave finds its range
// in O(1) and no work is claimed at run time; every unit still writes its own
// partial state. All values are wave-uniform.
struct UnitRange {
  int begin, end;
};
// (fp32 arithmetic: a boundary shared by two waves is the same expression on
// the same inputs for both, and unit_at is monotone in c, so the ranges tile
// [0, units) exactly whatever the rounding; 64-bit integer division would cost
// the launch thousands of instructions before its first load.)
__device__ inline UnitRange static_unit_range(const int* plan, float ring_cost, float rec_bytes, int wv, int W) {
  int nsec[kSections];
  float cost[kSections];
#pragma unroll
  for (int k = 0; k < kSections; ++k) nsec[k] = __builtin_amdgcn_readfirstlane(plan[kPlanSec + k]);
  cost[0] = ring_cost;
  cost[1] = (float)__builtin_amdgcn_readfirstlane(plan[kPlanUb]) * rec_bytes;
  cost[2] = (float)__builtin_amdgcn_readfirstlane(plan[kPlanUm]) * rec_bytes;
  cost[3] = (float)__builtin_amdgcn_readfirstlane(plan[kPlanUs]) * rec_bytes;
  float total = 0.f;
  int units = 0;
#pragma unroll
  for (int k = 0; k < kSections; ++k) {
    total += (float)nsec[k] * cost[k];
    units += nsec[k];
  }
  // first unit whose start cost is >= c
  // (branch-free: the section is found with selects, the result made scalar)
  auto unit_at = [&](float c) -> int {
    float cbase = 0.f;
    int ubase = 0, r = units;
    bool found = false;
#pragma unroll
    for (int k = 0; k < kSections; ++k) {
      const float sec = (float)nsec[k] * cost[k];
      const bool here = !found && nsec[k] > 0 && c <= cbase + sec;
      const int i = min(nsec[k], (int)ceilf((c - cbase) * __builtin_amdgcn_rcpf(cost[k])));
      r = here ? ubase + max(i, 0) : r;
      found = found || here;
      cbase += sec;
      ubase += nsec[k];
    }
    return __builtin_amdgcn_readfirstlane(r);
  };
  const float per_wave = total / (float)W;
  UnitRange r;
  r.begin = wv == 0 ? 0 : unit_at(per_wave * (float)wv);
  r.end = wv + 1 == W ? units : unit_at(per_wave * (float)(wv + 1));
  return r;
}

// Slot of the i-th partial of pair (b, h): its units section by section.
struct PairUnits {
  int n;                      // partials of the pair
  int cnt[kSections];         // per section
  int first[kSections];       // first slot per section
  // branch-free: the last section that starts at or before i (empty sections
  // start where the next one does)
  __device__ __forceinline__ int slot(int i) const {
    int r = first[0] + i, start = 0;
#pragma unroll
    for (int k = 1; k < kSections; ++k) {
      start += cnt[k - 1];
      r = i >= start ? first[k] + (i - start) : r;
    }
    return r;
  }
};
__device__ inline PairUnits pair_units(const Geom& g, const int* plan, int b, int h) {
  PairUnits p;
  p.n = 0;
  int base = 0;
#pragma unroll
  for (int k = 0; k < kSections; ++k) {
    const int* pre = plan + kPlanHdr + k * (g.B + 1);
    p.cnt[k] = pre[b + 1] - pre[b];
    p.first[k] = base + g.Hkv * pre[b] + h * p.cnt[k];
    p.n += p.cnt[k];
    base += plan[kPlanSec + k];
  }
  return p;
}
#endif

}  // namespace kvq
