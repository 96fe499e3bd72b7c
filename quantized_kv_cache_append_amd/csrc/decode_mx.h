// Decode path for one query head per kv head with 2-bit keys and values,
// G = G_V = 32, head_dim 128 (gfx950): both products on the block-scaled
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4), the packed codes fed to
// them as fp4 operands. Kernel template, instantiated in
// decode_fast_dispatch.hip.
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026": section "KIVI (2024)" -- keys quantized per channel,
//        values per token, each group with its own min/max parameters, recent
//        tokens in full precision; innovation 3 -- 16 INT2 codes per 32-bit
//        word, unpacked in registers; innovation 4 -- the window of recent
//        tokens is read by the same attention pass.
//   [P3] encorp.ai, "La compression du cache KV est une décision
//        d'infrastructure ...": decode streams the cache from HBM and is bound
//        by that traffic.
//
// Arithmetic (log2 units, q' = q * softmax_scale * log2 e), as in the other
// decode paths:
//   score_t = sum_c (q'_c s_c) code_tc + kappa,  kappa = sum_c q'_c z_c   (per block)
//   o_c     = sum_t (p_t s_tj) code_tc + lambda_j, lambda_j = sum_t p_t z_tj
//
// Why the matrix cores, although a single query row makes both products
// matrix-vector: a 2-bit code placed in a nibble is an exact fp4 (e2m1) value
// c/2, so the codes go to the MFMA after three bit operations per 16 codes,
// and the real-valued operand (q~ = q' s_K per block, p~ = p s_V per value
// group) takes the otherwise idle rows: its values, in units of 2^(e - 4)
// where 2^e bounds them over the row, are written as three signed base-32
// digits and an e4m3 remainder, x = D0 + D1/32 + D2/1024 + r/32768 (integers
// |D_k| <= 16 and |r| <= 16: e4m3 holds every integer up to 16 exactly), one
// row each, and the per-row E8M0 block scale of the instruction restores each
// row's weight; the remainder's rounding leaves out at most 2^-19 of the row
// maximum. Why digits and not limbs of each value's own significand:
// the instruction does not sum its products exactly. Measured on gfx950, each
// run of 8 consecutive k is aligned to its largest product and bits more than
// about 2^13 below it are dropped (256 + 2^-9 sums to 256), while the sums of
// the runs are exact. A row of digits holds only small integers, so each of its
// products (at most 16 * 1.5, on a grid of 0.5) survives that alignment and the
// row's sum is exact; only the remainder row loses bits, far below the digits.
// Each score or output is then the fp32 sum of its four rows. This leaves the
// vector ALUs about a third of the instructions per token of the fp32 path.
//
// Work of one wave: units of whole sets of 4 blocks (128 tokens), the next
// set's loads in flight while a set is computed. Lane l = 16 g + n:
//   score MFMA (one per 16-token tile i; A = q~ digit rows, rows 4 blk + k; B =
//     key codes of tokens 16 i + n, channels 32 g .. 32 g + 31): lane group g
//     holds the four digit rows of block g, so the scores of block g's tokens
//     32 g + n and 32 g + 16 + n are sums of the lane's own accumulators;
//   P.V MFMA (one per 16-channel tile; A = p~ digit rows, rows 4 j + k; B =
//     value codes of channel 16 nt + n, tokens 32 g .. 32 g + 31): lane group
//     g holds the digit rows of value group g, so outputs 32 g + n and
//     32 g + 16 + n are sums of its own accumulators;
//   the q~ digit rows of block g, kappa, the p~ digit rows and lambda of group g are
//     built by the 16 lanes of lane group g (8 channels or 8 tokens each).
// Operand layouts of the instruction (measured): an fp4 operand lane of group
// g holds k = 32 g .. 32 g + 31 (nibble j = k - 32 g); an fp8 operand lane
// holds k = 16 g .. 16 g + 15 in bytes 0..15 and 64 + 16 g .. 64 + 16 g + 15
// in bytes 16..31; the block scale of row r for k in [32 b, 32 b + 32) comes
// from lane r + 16 b. The k order of the codes (even slots of a word, then odd
// slots) is followed by the digit-row images the builders write to LDS.
#pragma once

#include "common.h"
#include "decode_mha.h"
#include "decode_units.h"

namespace kvq {
namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kSetBlk = 4;         // blocks per set
constexpr int kSetTok = 128;       // tokens per set
constexpr int kRows = 4;           // A-operand rows per real-valued operand: 3 digits + remainder
constexpr int kRingTok = 32;       // ring tokens per ring unit: every load of a unit in flight at once
constexpr int kRingWeight = 3;     // cost of a ring byte in quarters of a quantized byte (measured: a 16 KB ring unit takes about as long as a 12 KB set)
constexpr int kUnitSets = 1;       // sets per quantized unit: the static partition cuts at set granularity
constexpr float kRescaleLog2 = 8.0f;
constexpr int kCodeScale = 128;    // E8M0 2^1: an fp4 code nibble reads c / 2

template <bool BF16_, bool PAGED_>
struct Cfg {
  static constexpr int KB = 2, VB = 2, G = 32, GV = 32, D = 128;
  static constexpr bool BF16 = BF16_, PAGED = PAGED_;
  static constexpr int NGR = D / GV;   // value groups (4: one per lane group)
  // record sections
  static constexpr int REC_KC = 0;
  static constexpr int REC_KS = G * D * KB / 8;
  static constexpr int REC_KZ = REC_KS + 2 * D;
  static constexpr int REC_VC = REC_KZ + 2 * D;
  static constexpr int REC_VS = REC_VC + G * D * VB / 8;
  static constexpr int REC_VZ = REC_VS + 2 * NGR * G;
  static constexpr int REC = REC_VZ + 2 * NGR * G;
  // per-wave LDS (bytes)
  static constexpr int L_Q = 4 * D;          // q' (fp32)
  static constexpr int L_P = 4 * kSetTok;    // p of the set's tokens (fp32; also the ring units' p)
  static constexpr int L_A = 64 * 32;        // one A-operand image: 32 bytes per lane
  static constexpr int L_WAVE = L_Q + L_P + 2 * L_A;
  using Ring = mha::Cfg<KB, VB, G, GV, BF16, PAGED>;   // ring units run the fp32 routine
  static_assert(NGR == 4 && kSetBlk == 4, "lane group g = block g of a set = value group g");
};

// ---------------------------------------------------------------------------------
// Building blocks
// ---------------------------------------------------------------------------------

// Write x0..x7 (|x| < 16, in units of the first digit) as kRows e4m3 rows of
// an A-operand image: rows 0 .. kRows - 2 hold the signed base-32 digits
// D_k = round(t_k), t_0 = x, t_(k+1) = 32 (t_k - D_k) (|t_k| <= 16, so the
// digits are integers in [-16, 16], exact in e4m3), the last row t_(kRows-1)
// rounded to e4m3. Row k's value of x_e goes to byte e/2 of dword `off_even` (e even) or
// `off_odd` (e odd) of row row0 + k, where a row's lane image starts at
// 32 (row + 16 g) bytes.
__device__ __forceinline__ void write_digit_rows(uint8_t* img, int row0, int off_even, int off_odd, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = k + 1 < kRows ? __builtin_rintf(x[e]) : x[e];
    int ev = __builtin_amdgcn_cvt_pk_fp8_f32(d[0], d[2], 0, false);
    ev = __builtin_amdgcn_cvt_pk_fp8_f32(d[4], d[6], ev, true);
    int od = __builtin_amdgcn_cvt_pk_fp8_f32(d[1], d[3], 0, false);
    od = __builtin_amdgcn_cvt_pk_fp8_f32(d[5], d[7], od, true);
    uint8_t* row = img + 32 * (row0 + k);
    *reinterpret_cast<int*>(row + off_even) = ev;
    *reinterpret_cast<int*>(row + off_odd) = od;
    if (k + 1 < kRows) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (x[e] - d[e]) * 32.0f;   // exact
    }
  }
}

// Exponent e with max|x| < 2^e over the 16 lanes of a DPP row (every lane gets
// it), floored so that the rows' scales stay inside E8M0's range.
__device__ __forceinline__ int row_exponent(float amax) {
  amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x121, 0xF, 0xF, false)));
  amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x122, 0xF, 0xF, false)));
  amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x124, 0xF, 0xF, false)));
  amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x128, 0xF, 0xF, false)));
  return max(__builtin_amdgcn_frexp_expf(amax), -100);
}

// E8M0 scale byte of A-operand row r (= 4 j + k) of this lane, from the
// exponents e_j of the four lane groups: row k of a value written in units of
// 2^(e - 4) weighs 2^(e - 4 - 5k).
__device__ __forceinline__ int row_scale(int e_lane, int lane) {
  const int r = lane & 15;
  const int e0 = __builtin_amdgcn_readlane(e_lane, 0), e1 = __builtin_amdgcn_readlane(e_lane, 16);
  const int e2 = __builtin_amdgcn_readlane(e_lane, 32), e3 = __builtin_amdgcn_readlane(e_lane, 48);
  const int j = r >> 2;
  const int e = j == 0 ? e0 : (j == 1 ? e1 : (j == 2 ? e2 : e3));
  return 127 + e - 4 - 5 * (r & 3);
}

// Even and odd 2-bit slots of a code word as fp4 nibbles (k order of the
// operands: even slots of the word, then odd slots).
__device__ __forceinline__ uint32_t even_slots(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t odd_slots(uint32_t w) { return (w >> 2) & 0x33333333u; }

__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, int scale_a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, kCodeScale);
}

template <class C>
__device__ __forceinline__ float in_val(uint32_t bits16) {
  return C::BF16 ? __uint_as_float(bits16 << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ float h2f(uint32_t w, int hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? (w >> 16) : w));
}

// ---------------------------------------------------------------------------------
// The quantized units [first, units) of a wave, in order, as one stream of
// sets: each set's loads go out while the previous set is computed, across
// unit boundaries. locate(u) gives unit u's span (called for increasing u).
// ---------------------------------------------------------------------------------
template <class C, class Locate>
__device__ __forceinline__ void quant_stream(const Geom& g, float* __restrict__ lq, float* __restrict__ lp,
                                             uint8_t* __restrict__ qimg, uint8_t* __restrict__ pimg,
                                             const uint8_t* __restrict__ blocks, const int32_t* __restrict__ table,
                                             const uint16_t* __restrict__ q, float qscale, int units, int first,
                                             mha::Span first_span, Locate locate, float* __restrict__ ws) {
  constexpr int D = C::D;
  const int lane = threadIdx.x & 63, n = lane & 15, gq = lane >> 4;

  struct SetBuf {
    uint2 kc[8];     // key codes of tile i: token 16 i + n, channels 32 gq .. 32 gq + 31
    uint4 ks, kz;    // key scale / zero of block gq, channels 8 n .. 8 n + 7
    uint4 vc[4];     // value-code chunk (run rr, channel n) of block gq, rr = 0..3
    uint4 vs, vz;    // value scale / zero of group gq, tokens 8 (n % 4) .. + 7 of block n / 4
    uint32_t qw;     // the unit's query, channels 2 lane and 2 lane + 1
  };
  auto rec_of = [&](mha::Span sp, int blk) -> const uint8_t* {
    return mha::span_rec<typename C::Ring>(g, blocks, table, sp, blk);
  };
  auto load_set = [&](SetBuf& b, mha::Span sp, int si) {
    const int blk0 = sp.begin + si * kSetBlk;
    b.qw = reinterpret_cast<const uint32_t*>(q + ((size_t)sp.b * g.Hq + sp.h) * D)[lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t* r = rec_of(sp, blk0 + i / 2) + C::REC_KC + (16 * (i % 2) + n) * (D / 4) + 8 * gq;
      b.kc[i] = *reinterpret_cast<const uint2*>(r);
    }
    const uint8_t* rg = rec_of(sp, blk0 + gq);
    b.ks = *reinterpret_cast<const uint4*>(rg + C::REC_KS + 16 * n);
    b.kz = *reinterpret_cast<const uint4*>(rg + C::REC_KZ + 16 * n);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) b.vc[rr] = *reinterpret_cast<const uint4*>(rg + C::REC_VC + (rr * 16 + n) * 16);
    const uint8_t* rv = rec_of(sp, blk0 + n / 4) + 64 * gq + 16 * (n % 4);
    b.vs = *reinterpret_cast<const uint4*>(rv + C::REC_VS);
    b.vz = *reinterpret_cast<const uint4*>(rv + C::REC_VZ);
  };
  auto blk_ok = [&](mha::Span sp, int blk) -> bool {
    if (blk >= sp.end) return false;
    if constexpr (!C::PAGED) return true;
    const int page = table[(size_t)sp.b * g.max_blocks + blk];
    return page >= 0 && page < g.num_pages;
  };

  // running state of the current unit
  float m_run, l_lane, lam_lane;
  v4f acc[8];

  const bool rot_q = (g.rot & KVQ_ROTATE_KEYS) != 0;
  auto compute_set = [&](const SetBuf& cb, mha::Span cur, bool new_query) {
    const int blk0 = cur.begin;
    if (new_query) {   // a new pair's first set: its query into LDS
      float x0 = in_val<C>(cb.qw & 0xffffu) * qscale, x1 = in_val<C>(cb.qw >> 16) * qscale;
      // (rotated keys: the blocks hold R(k) = H k / 8, so the query is rotated
      // the same way, H q' * 8 / D, and the scores are unchanged)
      if (rot_q) wht_row_pairs(x0, x1, 8.0f / D);
      *reinterpret_cast<float2*>(lq + 2 * lane) = make_float2(x0, x1);
      wave_lds_fence();
    }
    // ---- q~ digit rows of block gq, channels 8n .. 8n + 7, and kappa of block gq ----
    float kap;
    {
      const float4 qa = *reinterpret_cast<const float4*>(lq + 8 * n);
      const float4 qb = *reinterpret_cast<const float4*>(lq + 8 * n + 4);
      const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      const uint32_t sw[4] = {cb.ks.x, cb.ks.y, cb.ks.z, cb.ks.w};
      const uint32_t zw[4] = {cb.kz.x, cb.kz.y, cb.kz.z, cb.kz.w};
      float x[8], amax = 0.f;
      kap = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = qv[e] * h2f(sw[e / 2], e & 1);
        kap = fmaf(qv[e], h2f(zw[e / 2], e & 1), kap);
        amax = fmaxf(amax, fabsf(x[e]));
      }
      kap = mha::row_sum16(kap);
      const int ex = row_exponent(amax);
      const float nrm = __builtin_amdgcn_ldexpf(1.0f, 4 - ex);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= nrm;
      // channels 8n + e sit at k = 16 (n / 2) + 4 (n % 2) + 8 (e % 2) + e / 2
      const int kb = 16 * (n / 2) + 4 * (n % 2);
      const int lg = (kb % 64) / 16, off = 16 * (kb / 64) + kb % 16;
      write_digit_rows(qimg + 32 * 16 * lg, 4 * gq, off, off + 8, x);
      const int sc = row_scale(ex, lane);
      wave_lds_fence();
      const v8i a = *reinterpret_cast<const v8i*>(qimg + 32 * lane);
      // ---- scores: tile i = tokens 16 i .. 16 i + 15, block i / 2 ----
      float s0 = -INFINITY, s1 = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint2 w = cb.kc[i];
        const v8i bop = {(int)even_slots(w.x), (int)odd_slots(w.x), (int)even_slots(w.y), (int)odd_slots(w.y),
                         0, 0, 0, 0};
        const v4f d = mfma_fp8_fp4(a, sc, bop, v4f{0.f, 0.f, 0.f, 0.f});
        const float t = (d[0] + d[1]) + (d[2] + d[3]);
        if (i % 2 == 0) s0 = gq == i / 2 ? t : s0;
        else s1 = gq == i / 2 ? t : s1;
      }
      const bool ok = blk_ok(cur, blk0 + gq);
      s0 = ok ? s0 + kap : -INFINITY;
      s1 = ok ? s1 + kap : -INFINITY;
      // ---- online softmax, lazily rescaled ----
      const float mx = mha::wave_max64(fmaxf(s0, s1));
      if (mx > m_run + kRescaleLog2) {   // wave-uniform
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
        m_run = mx;
        l_lane *= alpha;
        lam_lane *= alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] *= alpha;
      }
      const float p0 = s0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s0 - m_run);
      const float p1 = s1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s1 - m_run);
      l_lane += p0 + p1;
      lp[32 * gq + n] = p0;
      lp[32 * gq + 16 + n] = p1;
    }
    wave_lds_fence();
    // ---- p~ digit rows of value group gq, tokens 8n .. 8n + 7 (run n), and lambda ----
    {
      const float4 pa = *reinterpret_cast<const float4*>(lp + 8 * n);
      const float4 pb = *reinterpret_cast<const float4*>(lp + 8 * n + 4);
      const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      const uint32_t sw[4] = {cb.vs.x, cb.vs.y, cb.vs.z, cb.vs.w};
      const uint32_t zw[4] = {cb.vz.x, cb.vz.y, cb.vz.z, cb.vz.w};
      float x[8], amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = pv[e] * h2f(sw[e / 2], e & 1);
        lam_lane = fmaf(pv[e], h2f(zw[e / 2], e & 1), lam_lane);
        amax = fmaxf(amax, fabsf(x[e]));
      }
      const int ex = row_exponent(amax);
      const float nrm = __builtin_amdgcn_ldexpf(1.0f, 4 - ex);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= nrm;
      // token 8n + e of the set sits at k = 8n + (e even: e / 2, odd: 4 + e / 2)
      const int lg = (n % 8) / 2, off = 16 * (n / 8) + 8 * (n % 2);
      write_digit_rows(pimg + 32 * 16 * lg, 4 * gq, off, off + 4, x);
      const int sc = row_scale(ex, lane);
      wave_lds_fence();
      const v8i a = *reinterpret_cast<const v8i*>(pimg + 32 * lane);
      // ---- P.V: tile nt = channels 16 nt .. 16 nt + 15 (value group nt / 2) ----
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // word m of a chunk: low half channel 16 (2m) + n, high half 16 (2m + 1) + n
        // (tiles 2m and 2m + 1); k order of run rr: tokens 0, 2, 4, 6 (even
        // slots), then 1, 3, 5, 7
        uint32_t ev[4], od[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t w = m == 0 ? cb.vc[rr].x : (m == 1 ? cb.vc[rr].y : (m == 2 ? cb.vc[rr].z : cb.vc[rr].w));
          ev[rr] = even_slots(w);
          od[rr] = odd_slots(w);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t sel = h == 0 ? 0x05040100u : 0x07060302u;
          v8i bop;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) bop[rr] = (int)__builtin_amdgcn_perm(od[rr], ev[rr], sel);
          bop[4] = bop[5] = bop[6] = bop[7] = 0;
          acc[2 * m + h] = mfma_fp8_fp4(a, sc, bop, acc[2 * m + h]);
        }
      }
    }
    wave_lds_fence();   // the images and p are rewritten by the next set
  };

  // the unit's result: lane group gq owns channels 32 gq + n and 32 gq + 16 + n
  auto finish_unit = [&](float* __restrict__ out_part) {
    const float lsum = mha::wave_sum64(l_lane);
    const float lam = mha::row_sum16(lam_lane);
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float t = (acc[nt][0] + acc[nt][1]) + (acc[nt][2] + acc[nt][3]);
      if (nt % 2 == 0) o0 = gq == nt / 2 ? t : o0;
      else o1 = gq == nt / 2 ? t : o1;
    }
    out_part[32 * gq + n] = o0 + lam;
    out_part[32 * gq + 16 + n] = o1 + lam;
    if (lane == 0) {
      out_part[D] = m_run;
      out_part[D + 1] = lsum;
    }
  };

  // Every unit is one set; two register buffers alternate (the loads of unit
  // k + 1 are in flight while unit k is computed). Consecutive units that
  // continue the same pair share one running state: the state's partial goes
  // to the slot of the run's last unit and the other slots get an empty
  // partial (m = -inf, l = 0), which the combine skips.
  SetBuf b0, b1;
  int k = first;
  mha::Span s0 = first_span, s1 = first_span;
  load_set(b0, s0, 0);
  bool cont = false;
  auto step = [&](const SetBuf& cb, SetBuf& pf) -> bool {
    const bool more = k + 1 < units;   // wave-uniform
    if (more) {
      s1 = locate(k + 1);
      load_set(pf, s1, 0);
    }
    if (!cont) {
      m_run = -INFINITY;
      l_lane = 0.f;
      lam_lane = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    compute_set(cb, s0, !cont);
    const bool nc = more && s1.b == s0.b && s1.h == s0.h && s1.begin == s0.end;   // wave-uniform
    float* out_part = ws + (size_t)k * (D + 2);
    if (nc) {
      if (lane == 0) *reinterpret_cast<float2*>(out_part + D) = make_float2(-INFINITY, 0.f);
    } else {
      finish_unit(out_part);
    }
    cont = nc;
    ++k;
    s0 = s1;
    return more;
  };
  while (step(b0, b1) && step(b1, b0)) {
  }
}

// ------------------------------------------------------------------------------------
// The kernel: persistent waves, each with a fixed range of the plan's units;
// ring units run the fp32 routine of the multi-head path.
// ------------------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mx_kernel(
    Geom g, const uint8_t* __restrict__ blocks, const int32_t* __restrict__ table,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring, int32_t* __restrict__ state,
    const uint16_t* __restrict__ q, float qscale, int max_blk, int* __restrict__ ws_plan, float* __restrict__ ws) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* plan = reinterpret_cast<int*>(smem);
  const int pints = plan_ints(g.B);
  const int pre_bytes = plan_lds_bytes(g.B);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t* wl = smem + pre_bytes + wave * C::L_WAVE;
  float* lq = reinterpret_cast<float*>(wl);
  float* lp = reinterpret_cast<float*>(wl + C::L_Q);
  uint8_t* qimg = wl + C::L_Q + C::L_P;
  uint8_t* pimg = qimg + C::L_A;
  mha::WaveLds<typename C::Ring> L;   // the ring routine uses q' and p only
  L.q = lq;
  L.qt = nullptr;
  L.kap = nullptr;
  L.p = lp;
  L.pv = nullptr;

  build_unit_plan(g, state, max_blk, kSetBlk, kRingTok, plan, blockIdx.x == 0, kUnitSets);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < pints; i += blockDim.x) ws_plan[i] = plan[i];
  const UnitRange range = static_unit_range(plan, (float)(kRingTok * 4 * C::D * kRingWeight / 4), (float)C::REC,
                                            (int)blockIdx.x * kWaves + wave, (int)gridDim.x * kWaves);
  int u = range.begin;
  const int u_end = range.end;
  const int ring_units = __builtin_amdgcn_readfirstlane(plan[kPlanSec]);
  auto span_of = [&](int uu) -> mha::Span {
    const Unit un = locate_unit(g, plan, uu, max_blk);
    mha::Span sp;
    sp.b = __builtin_amdgcn_readfirstlane(un.b);
    sp.h = __builtin_amdgcn_readfirstlane(un.h);
    sp.begin = __builtin_amdgcn_readfirstlane(un.begin);
    sp.end = __builtin_amdgcn_readfirstlane(un.end);
    return sp;
  };
  // The quantized units of a pair are consecutive and one set each: the unit
  // after `last` continues its pair while blocks remain (no plan lookup).
  mha::Span last{};
  int last_u = -2, last_stop = 0;
  auto next_span = [&](int uu) -> mha::Span {
    if (uu == last_u + 1 && last.end < last_stop) {
      last.begin = last.end;
      last.end = min(last_stop, last.end + kSetBlk * kUnitSets);
    } else {
      last = span_of(uu);
      last_stop = min(__builtin_amdgcn_readfirstlane(plan[plan_seq_off(g.B) + last.b]) / C::G, max_blk);
    }
    last_u = uu;
    return last;
  };
  for (; u < u_end && u < ring_units; ++u) {
    const mha::Span sp = span_of(u);
    mha::ring_unit<typename C::Ring, kRingTok>(g, L, k_ring, v_ring, q, qscale, sp.b, sp.h, sp.begin, sp.end,
                                               ws + (size_t)u * (C::D + 2));
  }
  if (u < u_end) {
    quant_stream<C>(g, lq, lp, qimg, pimg, blocks, table, q, qscale, u_end, u, next_span(u), next_span, ws);
  }
}

template <class C>
hipError_t launch_mx(const Geom& g, const kvq_cache& c, const void* q, float scale, int max_blk, void* ws,
                     hipStream_t s) {
  const size_t lds = (size_t)plan_lds_bytes(g.B) + (size_t)kWaves * C::L_WAVE;
  const int grid = persistent_grid(decode_mx_kernel<C>, lds);
  hipLaunchKernelGGL((decode_mx_kernel<C>), dim3(grid), dim3(256), lds, s, g,
                     static_cast<const uint8_t*>(c.blocks), c.block_table, static_cast<const uint16_t*>(c.k_ring),
                     static_cast<const uint16_t*>(c.v_ring), c.state, static_cast<const uint16_t*>(q),
                     scale * 1.4426950408889634f, max_blk, static_cast<int*>(ws),
                     reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan_bytes(g.B)));
  return hipGetLastError();
}

}  // namespace mx
}  // namespace kvq
