// Split-sequence decode attention over the packed cache, and the combine of the
// split partial states (gfx950).
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026": section "KIVI (2024)" (dequantization with per-channel
//        key and per-token value parameters), innovation 3 (codes unpacked from
//        32-bit words in registers), innovation 4 (the full-precision window is
//        read by the same attention pass as the low-bit history).
//   [P3] encorp.ai, "La compression du cache KV est une décision
//        d'infrastructure ...": every decoded token streams the cache from HBM,
//        so the kernel is organised around that stream.
//   [P1] ai-automate.fr, "KV-cache compressé et modèles 4-bit ...", Minima-KV:
//        partial attention states combined by a globally normalised online
//        softmax -- the split/combine used here.
//
// Work decomposition (decode_units.h). Each (sequence b, kv head h) gives one
// unit for its ring tokens and units of consecutive quantized blocks; the unit
// counts come from the device-side lengths, so ragged batches need no host
// synchronisation. Each unit leaves a partial state (running max m, sum l,
// unnormalised o[d]) per query head of the group, scores in log2 units (the
// query is pre-multiplied by softmax_scale * log2 e, so exp becomes exp2); the
// combine kernel merges them.
//
// This file holds the plan, the combine and the generic VALU path (head_dim 64
// or 128, any supported group size, n_g <= 8), used for configurations the
// MFMA path (decode_fast.h) has no instantiation for: scores lane-per-token
// with the key scale folded into the query (q~ = q * s_K) and the zero-point
// term added once per block, values lane-per-channel.
#include <algorithm>

#include "common.h"
#include "decode_units.h"

namespace kvq {

namespace {

constexpr int kWaves = 4;
constexpr int kRingAll = 1 << 30;   // ring tokens per ring unit of the generic kernel: all of them

template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_generic_kernel(
    Geom g, const uint8_t* __restrict__ blocks, const int32_t* __restrict__ table,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring, int32_t* __restrict__ state,
    const uint16_t* __restrict__ q, float qscale, int max_blk, int* __restrict__ ws_plan, float* __restrict__ ws) {
  constexpr int CPL = D / 64;   // channels per lane
  extern __shared__ int smem[];
  int* plan = smem;
  const int pints = plan_ints(g.B);
  float* scratch = reinterpret_cast<float*>(smem + plan_lds_bytes(g.B) / 4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* qt = scratch + wave * (kNgMax * D + kNgMax * 64);   // [8][D]
  float* pb = qt + kNgMax * D;                               // [8][64]

  // the whole ring of a pair is one unit (kRingAll tokens per ring unit)
  build_unit_plan(g, state, max_blk, 1, kRingAll, plan, blockIdx.x == 0);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < pints; i += blockDim.x) ws_plan[i] = plan[i];

  const int units = plan[kPlanUnits];
  const int ng = g.ng;
  for (int w = blockIdx.x * kWaves + wave; w < units; w += gridDim.x * kWaves) {
    const Unit un = locate_unit(g, plan, w, max_blk);
    const int b = un.b, h = un.h;
    const int pair = b * g.Hkv + h;
    const int Q = state[4 * b + kStateQ];
    const int S = max(state[4 * b + kStateS] - g.P, 0);   // tokens after the sink

    float qv[kNgMax][CPL], o[kNgMax][CPL], m[kNgMax], l[kNgMax];
#pragma unroll
    for (int j = 0; j < kNgMax; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        o[j][k] = 0.f;
        qv[j][k] = (j < ng) ? in_to_f32<BF16>(q[((size_t)b * g.Hq + h * ng + j) * D + lane + 64 * k]) * qscale : 0.f;
      }
    }

    // online softmax update for one tile of up to 64 tokens (lane = token)
    auto softmax_tile = [&](float (&sc)[kNgMax], bool valid) {
#pragma unroll
      for (int j = 0; j < kNgMax; ++j) {
        if (j >= ng) break;
        const float s = valid ? sc[j] : -INFINITY;
        const float bm = wave_max(s);
        const float mn = fmaxf(m[j], bm);
        const float alpha = (m[j] == -INFINITY) ? 0.f : exp2f(m[j] - mn);
        const float p = (valid && s != -INFINITY) ? exp2f(s - mn) : 0.f;   // (-inf: a masked token)
        l[j] = l[j] * alpha + wave_sum(p);
        m[j] = mn;
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[j][k] *= alpha;
        pb[j * 64 + lane] = p;
      }
      wave_lds_fence();
    };

    if (!un.ring) {
      // ---- quantized blocks of this unit ----
      // (rotated keys: the query is rotated the same way, H q' * 8 / D)
      if (g.rot & KVQ_ROTATE_KEYS) {
#pragma unroll
        for (int j = 0; j < kNgMax; ++j)
          if (j < ng) wht_row_strided<CPL>(qv[j], 8.0f / D);
      }
      const int blk0 = un.begin, blk1 = un.end;
      const int kP = 32 / g.kb;
      const uint32_t kmask = (1u << g.kb) - 1, vmask = (1u << g.vb) - 1;
      for (int blk = blk0; blk < blk1; ++blk) {
        const uint8_t* rec = block_record(g, blocks, table, b, h, blk);
        if (rec == nullptr) continue;
        const uint16_t* ks = reinterpret_cast<const uint16_t*>(rec + g.rec_ks);
        const uint16_t* kz = reinterpret_cast<const uint16_t*>(rec + g.rec_kz);
        float kap[kNgMax];
#pragma unroll
        for (int j = 0; j < kNgMax; ++j) kap[j] = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int c = lane + 64 * k;
          const float s = f16_to_f32(ks[c]), z = f16_to_f32(kz[c]);
#pragma unroll
          for (int j = 0; j < kNgMax; ++j) {
            if (j >= ng) break;
            qt[j * D + c] = qv[j][k] * s;
            kap[j] += qv[j][k] * z;
          }
        }
#pragma unroll
        for (int j = 0; j < kNgMax; ++j)
          if (j < ng) kap[j] = wave_sum(kap[j]);
        wave_lds_fence();

        // scores, lane = token of the block
        const bool valid = lane < g.G;
        float sc[kNgMax];
#pragma unroll
        for (int j = 0; j < kNgMax; ++j) sc[j] = 0.f;
        if (valid) {
          const uint32_t* kw = reinterpret_cast<const uint32_t*>(rec + g.rec_kc) + (size_t)lane * g.k_words;
          for (int wd = 0; wd < g.k_words; ++wd) {
            const uint32_t word = kw[wd];
            for (int sl = 0; sl < kP; ++sl) {
              const float code = (float)((word >> (sl * g.kb)) & kmask);
              const int c = wd * kP + sl;
#pragma unroll
              for (int j = 0; j < kNgMax; ++j)
                if (j < ng) sc[j] += qt[j * D + c] * code;
            }
          }
        }
#pragma unroll
        for (int j = 0; j < kNgMax; ++j) sc[j] = sc[j] + kap[j];
        softmax_tile(sc, valid);

        // values, lane = channel
        const uint16_t* vs = reinterpret_cast<const uint16_t*>(rec + g.rec_vs);
        const uint16_t* vz = reinterpret_cast<const uint16_t*>(rec + g.rec_vz);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int c = lane + 64 * k;
          const int gr = c / g.GV;
          const uint32_t* vw = reinterpret_cast<const uint32_t*>(rec + g.rec_vc);
          const int cpos = ((c & 15) * (D / 16) + (c >> 4)) * 8;   // stream position of (t=0, c)
          for (int t = 0; t < g.G; ++t) {
            const int bit = (cpos + (t >> 3) * 8 * D + (t & 7)) * g.vb;
            const float code = (float)((vw[bit >> 5] >> (bit & 31)) & vmask);
            const float val = f16_to_f32(vs[gr * g.G + t]) * code + f16_to_f32(vz[gr * g.G + t]);
#pragma unroll
            for (int j = 0; j < kNgMax; ++j)
              if (j < ng) o[j][k] += pb[j * 64 + t] * val;
          }
        }
        wave_lds_fence();
      }
    } else {
      // ---- full-precision ring tokens of this pair ----
      const int r0 = un.begin, r1 = un.end;
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int j = 0; j < kNgMax; ++j)
          if (j < ng) qt[j * D + lane + 64 * k] = qv[j][k];
      wave_lds_fence();
      for (int t0 = r0; t0 < r1; t0 += 64) {
        const int t = t0 + lane;
        const bool valid = t < r1;
        float sc[kNgMax];
#pragma unroll
        for (int j = 0; j < kNgMax; ++j) sc[j] = 0.f;
        if (valid) {
          const uint16_t* kr = k_ring + ((size_t)pair * g.C + (t % g.C)) * D;
          for (int c = 0; c < D; ++c) {
            const float x = in_to_f32<BF16>(kr[c]);
#pragma unroll
            for (int j = 0; j < kNgMax; ++j)
              if (j < ng) sc[j] += qt[j * D + c] * x;
          }
        }
        if (g.T > 1) {   // query row j is token S - T + j % T (after the sink): later tokens are masked
#pragma unroll
          for (int j = 0; j < kNgMax; ++j)
            if (j < ng && t > S - g.T + j % g.T) sc[j] = -INFINITY;
        }
        softmax_tile(sc, valid);
        const int nt = min(64, r1 - t0);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int c = lane + 64 * k;
          for (int tt = 0; tt < nt; ++tt) {
            const float x = in_to_f32<BF16>(v_ring[((size_t)pair * g.C + ((t0 + tt) % g.C)) * D + c]);
#pragma unroll
            for (int j = 0; j < kNgMax; ++j)
              if (j < ng) o[j][k] += pb[j * 64 + tt] * x;
          }
        }
        wave_lds_fence();
      }
    }

    // partial state of this unit, per query head of the group
#pragma unroll
    for (int j = 0; j < kNgMax; ++j) {
      if (j >= ng) break;
      float* dst = ws + ((size_t)w * ng + j) * (D + 2);
#pragma unroll
      for (int k = 0; k < CPL; ++k) dst[lane + 64 * k] = o[j][k];
      if (lane == 0) {
        dst[D] = m[j];
        dst[D + 1] = l[j];
      }
    }
  }
}

// Merge the partial states of one (sequence, query head) (scores in log2
// units): with M = max m_i, o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.
// The units of the pair come from the plan the decode kernel left in the
// workspace. One workgroup of WPR waves per output row, lane holding D/64
// channels: wave w takes batches w, w + WPR, ... of kCombineBatch partials,
// each batch one round of loads (lane i also fetches m and l of partial i;
// a batch of fewer partials issues only the loads it needs),
// merged into a running maximum; with WPR > 1 the waves' states are then
// merged through LDS by wave 0. The kernel is bound by dispatch and load
// latency, not bandwidth: rows with many partials (long sequences cut into
// many units) take WPR = 4 so that each wave has one round of loads, rows with
// few take one wave per workgroup, which spreads them over every compute unit
// (four rows per workgroup measured 1.4 us slower per step than one). Batches
// of 48 rather than 64 partials: fewer registers, and 3.9 us less per launch on
// 1024 one-wave rows (0.5-0.7 us less on 256 rows of four waves).
constexpr int kCombineBatch = 48;
constexpr int kLoadStep = 8;   // granularity of a short batch's loads
// Waves per workgroup of the sink and FP8-tier side launches (one output row,
// or one round of a row, per wave).
constexpr int kSideWaves = 1;

// ROTV (values pre-rotated): the quantized units' partials (after the side
// states and the pair's ring units) sum in the rotated coordinates, kept apart
// and taken back through H y * 8 / D once per row: o = (sum_plain + H sum_rot
// * 8 / D) / L.
template <int D, bool SIDE, int WPR, bool ROTV>
__global__ __launch_bounds__(64 * WPR) void combine_kernel(Geom g, const int* __restrict__ plan,
                                                          const float* ws,   // (not restrict: the
                                                          // compiler barrier below must order its loads)
                                                          const float* __restrict__ side_parts, int nside,
                                                          float* __restrict__ out) {
  constexpr int CPL = D / 64;   // channels per lane
  const int lane = threadIdx.x & 63;
  const int wave = WPR == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = blockIdx.x;
  if (row >= g.B * g.Hq) return;
  const int b = row / g.Hq, hq = row % g.Hq;
  const int h = hq / g.ng, j = hq % g.ng;
  const PairUnits pu = pair_units(g, plan, b, h);
  const size_t stride = (size_t)g.ng * (D + 2);
  const float* src0 = ws + (size_t)j * (D + 2);

  float m = -INFINITY, L = 0.f, acc[CPL], accq[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = accq[k] = 0.f;
  const int q0 = (SIDE ? nside : 0) + pu.cnt[0];   // partials from q0 on are quantized units
  // partial i: the side states (sink, FP8 tier rounds) first, then the pair's units
  const size_t side_stride = (size_t)g.B * g.Hq * (D + 2);
  const float* side0 = side_parts + (size_t)row * (D + 2);
  auto part = [&](int i) -> const float* {
    if constexpr (SIDE)
      return i < nside ? side0 + (size_t)i * side_stride : src0 + (size_t)pu.slot(i - nside) * stride;
    else
      return src0 + (size_t)pu.slot(i) * stride;
  };
  const int nparts = (SIDE ? nside : 0) + pu.n;
  for (int i0 = wave * kCombineBatch; i0 < nparts; i0 += WPR * kCombineBatch) {
    const int cnt = min(kCombineBatch, nparts - i0);
    const int lim = __builtin_amdgcn_readfirstlane((cnt + kLoadStep - 1) / kLoadStep * kLoadStep);
    // lane u locates partial i0 + u once (in parallel); load u takes its address
    // from lane u (two lane reads instead of a scalar slot search per load)
    const float* mine = part(i0 + min(lane, cnt - 1));
    const uint64_t mine_bits = reinterpret_cast<uint64_t>(mine);
    float v[kCombineBatch][CPL];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (u < lim) {   // (loads of a short batch stop at the next multiple of kLoadStep)
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)mine_bits, u < cnt ? u : 0);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(mine_bits >> 32), u < cnt ? u : 0);
        const float* src = reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo) + CPL * lane;
        if constexpr (CPL == 2) {
          const float2 x = *reinterpret_cast<const float2*>(src);
          v[u][0] = x.x;
          v[u][1] = x.y;
        } else {
#pragma unroll
          for (int k = 0; k < CPL; ++k) v[u][k] = src[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) v[u][k] = 0.f;
      }
    }
    const float2 ml = *reinterpret_cast<const float2*>(mine + D);
    asm volatile("" ::: "memory");   // the whole batch is in flight before the first wait
    const float mi = lane < cnt ? ml.x : -INFINITY, li = lane < cnt ? ml.y : 0.f;
    const float mn = fmaxf(m, wave_max(mi));
    if (mn == -INFINITY) continue;   // wave-uniform: nothing but empty partials so far
    const float a = m == -INFINITY ? 0.f : exp2f(m - mn);
    const float w = mi == -INFINITY ? 0.f : exp2f(mi - mn);   // weight of partial i0 + lane
    L = L * a + wave_sum(w * li);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      acc[k] *= a;
      if constexpr (ROTV) accq[k] *= a;
    }
#pragma unroll
    for (int c = 0; c < kCombineBatch / kLoadStep; ++c) {
      if (c * kLoadStep >= lim) break;   // (wave-uniform: a short batch merges only what it loaded)
#pragma unroll
      for (int k8 = 0; k8 < kLoadStep; ++k8) {
        const int u = c * kLoadStep + k8;
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));   // 0 past cnt
        if (ROTV && i0 + u >= q0) {
#pragma unroll
          for (int k = 0; k < CPL; ++k) accq[k] = wu == 0.f ? accq[k] : fmaf(wu, v[u][k], accq[k]);
        } else {
#pragma unroll
          for (int k = 0; k < CPL; ++k) acc[k] = wu == 0.f ? acc[k] : fmaf(wu, v[u][k], acc[k]);   // (empty partials: o unset)
        }
      }
    }
    m = mn;
  }
  if constexpr (WPR > 1) {
    __shared__ float s_ml[WPR][2];
    __shared__ float s_acc[WPR][D];
    __shared__ float s_accq[ROTV ? WPR : 1][D];
    if (lane == 0) {
      s_ml[wave][0] = m;
      s_ml[wave][1] = L;
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      s_acc[wave][CPL * lane + k] = acc[k];
      if constexpr (ROTV) s_accq[wave][CPL * lane + k] = accq[k];
    }
    __syncthreads();
    if (wave != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < WPR; ++x) M = fmaxf(M, s_ml[x][0]);
    L = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] = accq[k] = 0.f;
#pragma unroll
    for (int x = 0; x < WPR; ++x) {
      const float mx = s_ml[x][0];
      if (mx == -INFINITY) continue;   // a wave that saw no partial (or only empty ones)
      const float wx = exp2f(mx - M);
      L = fmaf(wx, s_ml[x][1], L);
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        acc[k] = fmaf(wx, s_acc[x][CPL * lane + k], acc[k]);
        if constexpr (ROTV) accq[k] = fmaf(wx, s_accq[x][CPL * lane + k], accq[k]);
      }
    }
  }
  if constexpr (ROTV) {   // the quantized share back from the rotated coordinates
    if constexpr (CPL == 2) wht_row_pairs(accq[0], accq[1], 8.0f / D);
    else wht_row_strided<CPL>(accq, 8.0f / D);
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] += accq[k];
  }
  float* dst = out + (size_t)row * D + CPL * lane;
#pragma unroll
  for (int k = 0; k < CPL; ++k) dst[k] = L > 0.f ? acc[k] / L : 0.f;
}

// Partial softmax state of the sink tokens of one (sequence b, query head):
// the first min(S_b, P) tokens, kept in full precision (attention sink: the
// zubnet.ai survey's paragraph on StreamingLLM's sink tokens, the encorp.ai
// OSCAR section). One wave per output row and 64 tokens per round, all of a
// round's loads issued together: lane t scores token t against the scaled
// query (held in LDS), then lane l accumulates channels D/64 * l .. over the
// round's tokens. Scores in log2 units like every other partial; written in
// the partial layout {o[D], m, l}, the empty state (m = -inf, l = 0) for
// S_b == 0.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kSideWaves) void sink_kernel(Geom g, const uint16_t* __restrict__ k_sink,
                                                                  const uint16_t* __restrict__ v_sink,
                                                                  const int32_t* __restrict__ state,
                                                                  const uint16_t* __restrict__ q, float qscale,
                                                                  float* __restrict__ out_part) {
  constexpr int CPL = D / 64;             // channels per lane in the P.V phase
  constexpr int VEC = D / 8;              // 16-byte vectors per row
  constexpr int VW = CPL == 1 ? 1 : CPL / 2;   // words per lane of a value row (d = 64: a half word)
  __shared__ float lq[kSideWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = blockIdx.x * kSideWaves + wave;
  if (row >= g.B * g.Hq) return;
  const int b = row / g.Hq, h = (row % g.Hq) / g.ng;
  // row j of a T-token query block is token S_b - T + j % T: it sees sink rows up to there
  const int S_b = state[4 * b + kStateS];
  const int n = __builtin_amdgcn_readfirstlane(max(min(min(S_b, g.P), S_b - g.T + (row % g.Hq) % g.ng % g.T + 1), 0));
  float* qs = lq[wave];
#pragma unroll
  for (int k = 0; k < CPL; ++k) qs[CPL * lane + k] = in_to_f32<BF16>(q[(size_t)row * D + CPL * lane + k]) * qscale;
  wave_lds_fence();
  const size_t pair_row0 = (size_t)(b * g.Hkv + h) * g.P;
  float m = -INFINITY, l = 0.f, acc[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = 0.f;
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int cnt = min(64, n - t0);   // wave-uniform
    // this round's loads: lane's key row (token t0 + lane), and its channels of every value row
    const uint4* kr = reinterpret_cast<const uint4*>(k_sink + (pair_row0 + t0 + min(lane, cnt - 1)) * D);
    uint4 kv[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) kv[i] = kr[i];
    uint32_t vw[64][VW];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (16 * c >= cnt) break;   // wave-uniform: only the chunks of 16 tokens the round has
#pragma unroll
      for (int u = 16 * c; u < 16 * c + 16; ++u) {
        const uint16_t* vr = v_sink + (pair_row0 + t0 + min(u, cnt - 1)) * D + CPL * lane;
        if constexpr (CPL == 1) {
          vw[u][0] = vr[0];
        } else {
#pragma unroll
          for (int k = 0; k < VW; ++k) vw[u][k] = reinterpret_cast<const uint32_t*>(vr)[k];
        }
      }
    }
    // score of token t0 + lane
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float4 qa = *reinterpret_cast<const float4*>(qs + 8 * i);
      const float4 qb = *reinterpret_cast<const float4*>(qs + 8 * i + 4);
      const uint32_t w[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
      s = fmaf(qa.x, in_to_f32<BF16>(w[0] & 0xffffu), s);
      s = fmaf(qa.y, in_to_f32<BF16>(w[0] >> 16), s);
      s = fmaf(qa.z, in_to_f32<BF16>(w[1] & 0xffffu), s);
      s = fmaf(qa.w, in_to_f32<BF16>(w[1] >> 16), s);
      s = fmaf(qb.x, in_to_f32<BF16>(w[2] & 0xffffu), s);
      s = fmaf(qb.y, in_to_f32<BF16>(w[2] >> 16), s);
      s = fmaf(qb.z, in_to_f32<BF16>(w[3] & 0xffffu), s);
      s = fmaf(qb.w, in_to_f32<BF16>(w[3] >> 16), s);
    }
    s = lane < cnt ? s : -INFINITY;
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
    const float p = lane < cnt ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] *= alpha;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (16 * c >= cnt) break;
#pragma unroll
      for (int u = 16 * c; u < 16 * c + 16; ++u) {
        const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), u));   // 0 past cnt
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const uint32_t w = vw[u][k / 2];
          acc[k] = fmaf(pu, in_to_f32<BF16>(CPL == 1 ? w : (k % 2 ? (w >> 16) : (w & 0xffffu))), acc[k]);
        }
      }
    }
    m = mn;
  }
  float* dst = out_part + (size_t)row * (D + 2);
#pragma unroll
  for (int k = 0; k < CPL; ++k) dst[CPL * lane + k] = acc[k];
  if (lane == 0) {
    dst[D] = m;
    dst[D + 1] = l;
  }
}

// Partial softmax states of the FP8 tier of one (sequence b, query head): the
// W most recent quantized blocks, read from their FP8 records ([P1]
// ai-automate.fr, section on Minima-KV: recent pages in FP8, one online
// softmax over both formats). One wave per (output row, round of 64 tier
// tokens), all of its loads issued together, each writing its own side
// partial (the empty state past the tier's end): lane t scores token t as
// s_K(t) * sum_c q'_c e4m3(k_tc) against the scaled query in LDS; then lane l
// accumulates channels D/64 * l .. as sum_t (p_t s_V(t)) e4m3(v_tc). Every
// query of a T-token block sees these blocks (they precede the window).
typedef float f32x2v __attribute__((ext_vector_type(2)));
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kSideWaves) void fp8_kernel(Geom g, const uint8_t* __restrict__ fp8,
                                                                 const int32_t* __restrict__ state,
                                                                 const uint16_t* __restrict__ q, float qscale,
                                                                 int rounds, float* __restrict__ out_part) {
  constexpr int CPL = D / 64;   // channels per lane in the P.V phase
  constexpr int VEC = D / 16;   // 16-byte vectors per code row
  __shared__ float lq[kSideWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int idx = blockIdx.x * kSideWaves + wave;   // round * (B * H_q) + row
  if (idx >= g.B * g.Hq * rounds) return;
  const int row = idx % (g.B * g.Hq), round = idx / (g.B * g.Hq);
  const int b = row / g.Hq, h = (row % g.Hq) / g.ng;
  const int nblk = __builtin_amdgcn_readfirstlane(state[4 * b + kStateQ] / g.G);
  const int f0 = nblk - min(nblk, g.W);
  const int n = (nblk - f0) * g.G;   // tokens of the tier
  float* qs = lq[wave];
#pragma unroll
  for (int k = 0; k < CPL; ++k) qs[CPL * lane + k] = in_to_f32<BF16>(q[(size_t)row * D + CPL * lane + k]) * qscale;
  wave_lds_fence();
  const uint8_t* pair_recs = fp8 + (size_t)(b * g.Hkv + h) * g.W * g.rec8;
  // record of tier token i (0 <= i < n): block f0 + i / G, row i % G
  auto rec_of = [&](int i) { return pair_recs + (size_t)((f0 + i / g.G) % g.W) * g.rec8; };
  const size_t ks_off = (size_t)g.G * D, vc_off = ks_off + 2 * g.G, vs_off = vc_off + (size_t)g.G * D;
  float m = -INFINITY, l = 0.f, acc[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = 0.f;
  const int t0 = 64 * round;
  if (t0 < n) {
    const int cnt = min(64, n - t0);   // wave-uniform
    const int mine = t0 + min(lane, cnt - 1);
    const uint8_t* mrec = rec_of(mine);
    const int mrow = mine % g.G;
    uint4 kv[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) kv[i] = reinterpret_cast<const uint4*>(mrec + (size_t)mrow * D)[i];
    const float sk = f16_to_f32(*reinterpret_cast<const uint16_t*>(mrec + ks_off + 2 * mrow));
    const float sv = f16_to_f32(*reinterpret_cast<const uint16_t*>(mrec + vs_off + 2 * mrow));
    uint32_t vw[64];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (16 * c >= cnt) break;   // wave-uniform: only the chunks of 16 tokens the round has
#pragma unroll
      for (int u = 16 * c; u < 16 * c + 16; ++u) {
        const int i = t0 + min(u, cnt - 1);
        const uint8_t* vr = rec_of(i) + vc_off + (size_t)(i % g.G) * D + CPL * lane;
        vw[u] = CPL == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(vr) : (uint32_t)*vr;
      }
    }
    // score of token t0 + lane
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const uint32_t w[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 qa = *reinterpret_cast<const float4*>(qs + 16 * i + 4 * e);
        const f32x2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[e], false);
        const f32x2v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[e], true);
        dot = fmaf(qa.x, lo.x, dot);
        dot = fmaf(qa.y, lo.y, dot);
        dot = fmaf(qa.z, hi.x, dot);
        dot = fmaf(qa.w, hi.y, dot);
      }
    }
    const float s = lane < cnt ? dot * sk : -INFINITY;
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
    const float p = lane < cnt ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    const float pv = p * sv;   // the token's value scale folded into its probability
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] *= alpha;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (16 * c >= cnt) break;
#pragma unroll
      for (int u = 16 * c; u < 16 * c + 16; ++u) {
        const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pv), u));   // 0 past cnt
        const f32x2v x = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[u], false);
        acc[0] = fmaf(pu, x.x, acc[0]);
        if constexpr (CPL == 2) acc[1] = fmaf(pu, x.y, acc[1]);
      }
    }
    m = mn;
  }
  float* dst = out_part + ((size_t)round * g.B * g.Hq + row) * (D + 2);
#pragma unroll
  for (int k = 0; k < CPL; ++k) dst[CPL * lane + k] = acc[k];
  if (lane == 0) {
    dst[D] = m;
    dst[D + 1] = l;
  }
}

template <int D, bool BF16>
hipError_t launch_generic(const Geom& g, const kvq_cache& c, const void* q, float scale, const DecodePlan& plan,
                          void* ws, hipStream_t s) {
  const int wgs = (int)std::min<size_t>((plan.units_max + kWaves - 1) / kWaves, 2048);
  const size_t lds = (size_t)plan_lds_bytes(g.B) + (size_t)kWaves * (kNgMax * D + kNgMax * 64) * 4;
  hipLaunchKernelGGL((decode_generic_kernel<D, BF16>), dim3(wgs), dim3(256), lds, s, g,
                     static_cast<const uint8_t*>(c.blocks), c.block_table,
                     static_cast<const uint16_t*>(c.k_ring), static_cast<const uint16_t*>(c.v_ring), c.state,
                     static_cast<const uint16_t*>(q), scale * 1.4426950408889634f, plan.max_blk,
                     static_cast<int*>(ws), reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan_bytes(g.B)));
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(const Geom& g, int max_seq_tokens) {
  DecodePlan p{};
  int nb_set = 1, rc = kRingAll, us = 0;
  // (every specialised kernel rotates the query for a rotated cache)
  p.fast = fast_supported(g, &nb_set, &rc, &us);
  p.nb_set = p.fast ? nb_set : 1;
  p.ring_chunk = p.fast ? rc : kRingAll;
  p.unit_sets = p.fast ? us : 0;
  p.max_blk = std::max(max_seq_tokens - g.R, 0) / g.G;
  p.units_max = units_max(g, p.max_blk, p.nb_set, p.ring_chunk, p.unit_sets);
  p.ws_bytes = plan_bytes(g.B) + p.units_max * (size_t)g.ng * (size_t)(g.d + 2) * 4;
  p.fp8_rounds = (g.W * g.G + 63) / 64;   // FP8 tier: one side partial per 64 of its tokens
  p.nside = (g.P > 0 ? 1 : 0) + p.fp8_rounds;
  p.side_off = 0;
  if (p.nside > 0) {   // side partials per output row, 16-byte aligned
    p.side_off = (p.ws_bytes + 15) & ~(size_t)15;
    p.ws_bytes = p.side_off + (size_t)p.nside * g.B * g.Hq * (g.d + 2) * 4;
  }
  return p;
}

namespace {
template <int D, bool BF16>
hipError_t launch_sink(const Geom& g, const kvq_cache& c, const void* q, float scale, const DecodePlan& plan,
                       void* ws, hipStream_t s) {
  const int grid = (g.B * g.Hq + kSideWaves - 1) / kSideWaves;
  hipLaunchKernelGGL((sink_kernel<D, BF16>), dim3(grid), dim3(64 * kSideWaves), 0, s, g,
                     static_cast<const uint16_t*>(c.k_sink), static_cast<const uint16_t*>(c.v_sink), c.state,
                     static_cast<const uint16_t*>(q), scale * 1.4426950408889634f,
                     reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan.side_off));
  return hipGetLastError();
}
template <int D, bool BF16>
hipError_t launch_fp8(const Geom& g, const kvq_cache& c, const void* q, float scale, const DecodePlan& plan,
                      void* ws, hipStream_t s) {
  const int grid = (g.B * g.Hq * plan.fp8_rounds + kSideWaves - 1) / kSideWaves;
  const size_t slot = g.P > 0 ? (size_t)g.B * g.Hq * (D + 2) * 4 : 0;   // after the sink's
  hipLaunchKernelGGL((fp8_kernel<D, BF16>), dim3(grid), dim3(64 * kSideWaves), 0, s, g,
                     static_cast<const uint8_t*>(c.fp8), c.state, static_cast<const uint16_t*>(q),
                     scale * 1.4426950408889634f, plan.fp8_rounds,
                     reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan.side_off + slot));
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_partials(const Geom& g, const kvq_cache& c, const void* q, float scale,
                                  const DecodePlan& plan, void* ws, hipStream_t s) {
  const bool bf16 = g.dtype == KVQ_BF16;
  if (g.P > 0) {
    const hipError_t e = g.d == 128 ? (bf16 ? launch_sink<128, true>(g, c, q, scale, plan, ws, s)
                                            : launch_sink<128, false>(g, c, q, scale, plan, ws, s))
                                    : (bf16 ? launch_sink<64, true>(g, c, q, scale, plan, ws, s)
                                            : launch_sink<64, false>(g, c, q, scale, plan, ws, s));
    if (e != hipSuccess) return e;
  }
  if (g.W > 0) {
    const hipError_t e = g.d == 128 ? (bf16 ? launch_fp8<128, true>(g, c, q, scale, plan, ws, s)
                                            : launch_fp8<128, false>(g, c, q, scale, plan, ws, s))
                                    : (bf16 ? launch_fp8<64, true>(g, c, q, scale, plan, ws, s)
                                            : launch_fp8<64, false>(g, c, q, scale, plan, ws, s));
    if (e != hipSuccess) return e;
  }
  if (plan.fast) return launch_decode_fast(g, c, q, scale, plan, ws, s);
  if (g.d == 128)
    return bf16 ? launch_generic<128, true>(g, c, q, scale, plan, ws, s)
                : launch_generic<128, false>(g, c, q, scale, plan, ws, s);
  return bf16 ? launch_generic<64, true>(g, c, q, scale, plan, ws, s)
              : launch_generic<64, false>(g, c, q, scale, plan, ws, s);
}

namespace {
template <int D, bool SIDE>
hipError_t launch_combine(bool wide, bool rotv, const Geom& g, const int* planp, const float* parts,
                          const float* side, int ns, float* out, hipStream_t s) {
  const dim3 gd(g.B * g.Hq);
  if (wide) {
    if (rotv) hipLaunchKernelGGL((combine_kernel<D, SIDE, 4, true>), gd, dim3(256), 0, s, g, planp, parts, side, ns, out);
    else hipLaunchKernelGGL((combine_kernel<D, SIDE, 4, false>), gd, dim3(256), 0, s, g, planp, parts, side, ns, out);
  } else {
    if (rotv) hipLaunchKernelGGL((combine_kernel<D, SIDE, 1, true>), gd, dim3(64), 0, s, g, planp, parts, side, ns, out);
    else hipLaunchKernelGGL((combine_kernel<D, SIDE, 1, false>), gd, dim3(64), 0, s, g, planp, parts, side, ns, out);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_combine(const Geom& g, const kvq_cache& c, float* out, const DecodePlan& plan, void* ws,
                                 hipStream_t s) {
  (void)c;
  const int* planp = static_cast<const int*>(ws);
  const float* parts = reinterpret_cast<const float*>(static_cast<const uint8_t*>(ws) + plan_bytes(g.B));
  const float* side = reinterpret_cast<const float*>(static_cast<const uint8_t*>(ws) + plan.side_off);
  const int ns = plan.nside;
  // partial states a row can have: its pair's share of the unit bound, plus the side states.
  // Four waves per row only while all of them fit on the GPU at once (rows * 4
  // waves within 256 CUs x 32 wave slots): with more rows than that, the extra
  // waves cost more than the shorter chains save (measured on 3072 rows).
  const size_t per_row = plan.units_max / ((size_t)g.B * g.Hkv) + (size_t)ns;
  const bool wide = per_row > kCombineBatch && (size_t)g.B * g.Hq * 4 <= 8192;
  const bool rotv = (g.rot & KVQ_ROTATE_VALUES) != 0;
  if (g.d == 128) {
    if (ns > 0) return launch_combine<128, true>(wide, rotv, g, planp, parts, side, ns, out, s);
    return launch_combine<128, false>(wide, rotv, g, planp, parts, side, ns, out, s);
  }
  if (ns > 0) return launch_combine<64, true>(wide, rotv, g, planp, parts, side, ns, out, s);
  return launch_combine<64, false>(wide, rotv, g, planp, parts, side, ns, out, s);
}

}  // namespace kvq
