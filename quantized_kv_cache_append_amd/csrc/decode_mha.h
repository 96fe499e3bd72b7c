// Decode path for one query head per kv head (multi-head attention), head_dim
// 128 (gfx950): kernel template, instantiated in decode_fast_dispatch.hip.
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026": section "KIVI (2024)" -- keys quantized per channel,
//        values per token, each group with its own min/max parameters, recent
//        tokens in full precision; innovation 3 -- codes packed 16 (INT2) or 8
//        (INT4) per 32-bit word and unpacked in registers; innovation 4 -- the
//        window of recent tokens is read by the same attention pass.
//   [P3] encorp.ai, "La compression du cache KV est une décision
//        d'infrastructure ...": decode streams the cache from HBM and is bound
//        by that traffic.
//
// With a single query row per kv head the score and P.V products are matrix
// times vector: there is no contraction for the matrix cores to share, so this
// path stays on the vector ALUs and is built around the HBM stream -- a few
// wide, fully coalesced loads per lane per set of 64 tokens, exact integer to
// fp32 code conversion and fp32 FMAs (no operand splitting), few registers so
// that several waves share each SIMD.
//
// Arithmetic (log2 units, q' = q * softmax_scale * log2 e):
//   score_t = sum_c (q'_c s_c) code_tc + sum_c q'_c z_c            (keys, per block)
//   o_c     = sum_t (p_t s_tj) code_tc + sum_t p_t z_tj, j = c / G_V (values)
// A set is 64 tokens (64/G blocks); the next set's loads are in flight while a
// set is computed. Score phase: lane = token, reading its key code row. P.V
// phase: lane (n = lane % 16, r = lane / 16) owns channels c = 16 cj + n
// (cj < 8) and the runs of 8 tokens r and r + 4, each run's codes one
// contiguous chunk of the value-code layout.
#pragma once

#include "common.h"
#include "decode_units.h"

namespace kvq {
namespace mha {

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kSetTok = 64;     // tokens per set (one per lane in the score phase)
constexpr int kTokLane = kSetTok / 64;
constexpr int kRingTok = 64;    // ring tokens per ring unit
constexpr float kRescaleLog2 = 8.0f;

template <int KB_, int VB_, int G_, int GV_, bool BF16_, bool PAGED_>
struct Cfg {
  static constexpr int KB = KB_, VB = VB_, G = G_, GV = GV_;
  static constexpr bool BF16 = BF16_, PAGED = PAGED_;
  static constexpr int D = 128;
  static constexpr int NBS = kSetTok / G;          // blocks per set
  static constexpr int NGR = D / GV;               // value groups
  static constexpr int KROW = D * KB / 8;          // key code bytes per token
  static constexpr int KW = KROW / 4;              // key code words per token
  static constexpr int VRUN = 8 * VB;              // value code bytes per (run of 8 tokens, c % 16)
  static constexpr int VW = VRUN / 4;
  static constexpr int RUNS = kSetTok / 8;         // runs of 8 tokens per set
  static constexpr int RPL = RUNS / 4;             // runs per lane
  // record sections
  static constexpr int REC_KC = 0;
  static constexpr int REC_KS = G * KROW;
  static constexpr int REC_KZ = REC_KS + 2 * D;
  static constexpr int REC_VC = REC_KZ + 2 * D;
  static constexpr int REC_VS = REC_VC + G * D * VB / 8;
  static constexpr int REC_VZ = REC_VS + 2 * NGR * G;
  static constexpr int REC = REC_VZ + 2 * NGR * G;
  // scale/zero bytes per set (both sections, all blocks of the set), loaded as 16-byte chunks
  static constexpr int KSZ_SET = NBS * 4 * D;
  static constexpr int VSZ_SET = NBS * 4 * NGR * G;
  static constexpr int KSZ_LD = (KSZ_SET + 1023) / 1024;   // 16-byte loads per lane
  static constexpr int VSZ_LD = (VSZ_SET + 1023) / 1024;
  // per-wave LDS (floats)
  static constexpr int L_Q = D;               // q'
  static constexpr int QT_STRIDE = D + 4;     // per-block rows 16 B apart in bank: the two blocks'
                                              // broadcast reads of a set fall in different banks
  static constexpr int L_QT = NBS * QT_STRIDE; // q' * s_K per block of the set
  static constexpr int L_KAP = 16;            // kappa per block (NBS <= 4)
  static constexpr int L_P = kSetTok;         // p per token of the set
  static constexpr int L_PV = NGR * kSetTok;  // p * s_V per group and token
  static constexpr int L_WAVE = L_Q + L_QT + L_KAP + L_P + L_PV;
  static_assert(G == 16 || G == 32 || G == 64, "blocks of 16, 32 or 64 tokens");
  static_assert(GV >= 16 && D % GV == 0, "value groups of whole 16-channel tiles");
  static_assert(KB == 2 || KB == 4, "2- or 4-bit keys");
  static_assert(VB == 2 || VB == 4, "2- or 4-bit values");
};

template <class C>
__device__ __forceinline__ float in_val(uint32_t bits16) {
  return C::BF16 ? __uint_as_float(bits16 << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ float h2f_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float h2f_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// sum over the 16 lanes of a DPP row (every lane gets the row's total)
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));   // row_ror 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));   // row_ror 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));   // row_ror 4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));   // row_ror 8
  return x;
}
// sum over the four lanes n, n+16, n+32, n+48
__device__ __forceinline__ float rows_sum4(float x) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}
// Reductions over the wave with row rotations (DPP) and row swaps (no LDS
// traffic); every lane gets the result.
__device__ __forceinline__ float wave_sum64(float v) { return rows_sum4(row_sum16(v)); }
__device__ __forceinline__ float wave_max64(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Byte k of w as a float (the compiler selects v_cvt_f32_ubyte<k>).
template <int K>
__device__ __forceinline__ float ubyte(uint32_t w) {
  return (float)((w >> (8 * K)) & 0xffu);
}

// The masked word with its known bits hidden from the compiler, which would
// otherwise narrow each byte read to a 2- or 4-bit field extract plus a
// conversion instead of one byte conversion.
__device__ __forceinline__ uint32_t opaque(uint32_t m) {
  asm("" : "+v"(m));
  return m;
}

// Codes of one 32-bit word as floats, in word order (slot i at bits [i*b, (i+1)*b)).
template <int B>
__device__ __forceinline__ void word_codes(uint32_t w, float (&out)[32 / B]) {
  if constexpr (B == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t m = opaque((w >> (2 * k)) & 0x03030303u);   // byte j holds slot 4j + k
      out[k] = ubyte<0>(m);
      out[4 + k] = ubyte<1>(m);
      out[8 + k] = ubyte<2>(m);
      out[12 + k] = ubyte<3>(m);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t m = opaque((w >> (4 * k)) & 0x0F0F0F0Fu);   // byte j holds slot 2j + k
      out[k] = ubyte<0>(m);
      out[2 + k] = ubyte<1>(m);
      out[4 + k] = ubyte<2>(m);
      out[6 + k] = ubyte<3>(m);
    }
  }
}

// A run of quantized blocks [begin, end) of (sequence b, kv head h).
struct Span {
  int b, h, begin, end;
};

template <class C>
__device__ __forceinline__ const uint8_t* span_rec(const Geom& g, const uint8_t* __restrict__ blocks,
                                                   const int32_t* __restrict__ table, Span sp, int blk) {
  blk = min(blk, sp.end - 1);
  if constexpr (!C::PAGED) {
    return blocks + (((size_t)sp.b * g.Hkv + sp.h) * g.max_blocks + blk) * (size_t)C::REC;
  } else {
    int page = table[(size_t)sp.b * g.max_blocks + blk];
    page = (page >= 0 && page < g.num_pages) ? page : 0;
    return blocks + ((size_t)page * g.Hkv + sp.h) * (size_t)C::REC;
  }
}

template <class C>
struct WaveLds {
  float* q;     // [D] q'
  float* qt;    // [NBS][D] q' * s_K
  float* kap;   // [16] kappa per block
  float* p;     // [64] p per set token
  float* pv;    // [NGR][64] p * s_V
};

// ---------------------------------------------------------------------------------
// Ring tokens [t0, t1) (at most RT <= 64) of one pair: lane = token for the
// scores (fp16/bf16 key row against q' in LDS), lane = 2 channels for P.V.
// ---------------------------------------------------------------------------------
template <class C, int RT = kRingTok>
__device__ __forceinline__ void ring_unit(const Geom& g, const WaveLds<C>& L, const uint16_t* __restrict__ k_ring,
                                          const uint16_t* __restrict__ v_ring, const uint16_t* __restrict__ q,
                                          float qscale, int b, int h, int t0, int t1,
                                          float* __restrict__ out_part) {
  constexpr int D = C::D;
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)(b * g.Hkv + h) * g.C;
  const int n = t1 - t0;
  // ring slot of token t0 + u (u < n <= C): one wrap at most
  const int s0 = t0 % g.C;
  auto slot = [&](int u) { return s0 + u - (s0 + u >= g.C ? g.C : 0); };
  // every load of the unit goes out together: the query, the key row of token
  // t0 + lane and the lane's two channels of all value rows (rows past t1
  // read row t0 and get probability 0)
  const uint32_t qw = reinterpret_cast<const uint32_t*>(q + ((size_t)b * g.Hq + h) * D)[lane];
  const bool valid = lane < n;
  const uint4* krow = reinterpret_cast<const uint4*>(k_ring + (base + slot(valid ? lane : 0)) * D);
  uint4 kr[D / 8];
#pragma unroll
  for (int k = 0; k < D / 8; ++k) kr[k] = krow[k];
  // (uniform row address + one shared lane offset: scalar-base addressing)
  const uint8_t* vpair = reinterpret_cast<const uint8_t*>(v_ring + base * D);
  const uint32_t loff = 4u * (uint32_t)lane;
  static_assert(RT % 4 == 0 && RT <= 64, "ring units of at most 64 tokens");
  uint32_t vv[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u)
    vv[u] = *reinterpret_cast<const uint32_t*>(vpair + (size_t)slot(u < n ? u : 0) * (2 * D) + loff);
  *reinterpret_cast<float2*>(L.q + 2 * lane) =
      make_float2(in_val<C>(qw & 0xffffu) * qscale, in_val<C>(qw >> 16) * qscale);
  wave_lds_fence();
  // score of token t0 + lane
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < D / 8; ++k) {
    const uint4 kw = kr[k];
    const float4 qa = *reinterpret_cast<const float4*>(L.q + 8 * k);
    const float4 qb = *reinterpret_cast<const float4*>(L.q + 8 * k + 4);
    acc[0] = fmaf(qa.x, in_val<C>(kw.x & 0xffffu), acc[0]);
    acc[1] = fmaf(qa.y, in_val<C>(kw.x >> 16), acc[1]);
    acc[2] = fmaf(qa.z, in_val<C>(kw.y & 0xffffu), acc[2]);
    acc[3] = fmaf(qa.w, in_val<C>(kw.y >> 16), acc[3]);
    acc[0] = fmaf(qb.x, in_val<C>(kw.z & 0xffffu), acc[0]);
    acc[1] = fmaf(qb.y, in_val<C>(kw.z >> 16), acc[1]);
    acc[2] = fmaf(qb.z, in_val<C>(kw.w & 0xffffu), acc[2]);
    acc[3] = fmaf(qb.w, in_val<C>(kw.w >> 16), acc[3]);
  }
  const float s = valid ? (acc[0] + acc[1]) + (acc[2] + acc[3]) : -INFINITY;
  const float m = wave_max64(s);
  const float p = valid ? __builtin_amdgcn_exp2f(s - m) : 0.f;
  const float l = wave_sum64(p);
  L.p[lane] = p;
  wave_lds_fence();
  // P.V: lane holds channels 2l, 2l+1
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int u4 = 0; u4 < RT / 4; ++u4) {
    const float4 pp = *reinterpret_cast<const float4*>(L.p + 4 * u4);
    const float pq[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = vv[4 * u4 + e];
      o0 = fmaf(pq[e], in_val<C>(w & 0xffffu), o0);
      o1 = fmaf(pq[e], in_val<C>(w >> 16), o1);
    }
  }
  *reinterpret_cast<float2*>(out_part + 2 * lane) = make_float2(o0, o1);
  if (lane == 0) {
    out_part[D] = m;
    out_part[D + 1] = l;
  }
  wave_lds_fence();   // L.p is rewritten by the next unit
}

// ---------------------------------------------------------------------------------
// The quantized units of a wave, from `first` on, as one stream of sets: the
// last set of a unit already loads the first set (and query) of the next unit.
// ---------------------------------------------------------------------------------
template <class C, class Locate, class Issue, class Claim>
__device__ __forceinline__ void quant_stream(const Geom& g, const WaveLds<C>& L, const uint8_t* __restrict__ blocks,
                                             const int32_t* __restrict__ table, const uint16_t* __restrict__ q,
                                             float qscale, int units, int first, Span first_span, int claimed,
                                             Locate locate, Issue issue, Claim claim, float* __restrict__ ws) {
  constexpr int D = C::D, G = C::G, NBS = C::NBS, NGR = C::NGR;
  const int lane = threadIdx.x & 63, n = lane & 15, rr = lane >> 4;

  // ---- register buffers of one set ----
  struct SetBuf {
    uint4 kc[kTokLane][C::KW / 4];   // key code rows of tokens lane (+ 64 ...)
    uint4 ksz[C::KSZ_LD];            // 16-byte chunks of the set's key scale/zero sections
    uint4 vc[C::RPL][C::VW / 4];     // value code chunks of runs rr, rr + 4, ...
    uint4 vsz[C::VSZ_LD];            // 16-byte chunks of the set's value scale/zero sections
    uint32_t qw;                     // the unit's query, channels 2 lane and 2 lane + 1
  };
  SetBuf cb;   // the set being computed (the next one loads into a second buffer meanwhile)

  // chunk k of lane of the set's [block][scale|zero] sections of `bytes_per_block`
  auto sz_chunk = [&](int k, int bytes_per_block, int& bi, int& off) {
    const int o = (k * 64 + lane) * 16;
    bi = o / bytes_per_block;
    off = o % bytes_per_block;
  };
  auto load_set = [&](SetBuf& b, Span sp, int si) {
    const int blk0 = sp.begin + si * NBS;
    b.qw = reinterpret_cast<const uint32_t*>(q + ((size_t)sp.b * g.Hq + sp.h) * D)[lane];
#pragma unroll
    for (int tl = 0; tl < kTokLane; ++tl) {
      const int tok = lane + 64 * tl;
      const uint8_t* r = span_rec<C>(g, blocks, table, sp, blk0 + tok / G) + C::REC_KC + (tok % G) * C::KROW;
#pragma unroll
      for (int k = 0; k < C::KW / 4; ++k) b.kc[tl][k] = reinterpret_cast<const uint4*>(r)[k];
    }
#pragma unroll
    for (int k = 0; k < C::KSZ_LD; ++k) {
      int bi, off;
      sz_chunk(k, 4 * D, bi, off);
      bi = bi < NBS ? bi : NBS - 1;
      b.ksz[k] = *reinterpret_cast<const uint4*>(span_rec<C>(g, blocks, table, sp, blk0 + bi) + C::REC_KS + off);
    }
#pragma unroll
    for (int h2 = 0; h2 < C::RPL; ++h2) {
      const int run = rr + 4 * h2;   // set-relative run of 8 tokens
      const int bi = run / (G / 8), R = run % (G / 8);
      const uint8_t* r = span_rec<C>(g, blocks, table, sp, blk0 + bi) + C::REC_VC + (R * 16 + n) * C::VRUN;
#pragma unroll
      for (int k = 0; k < C::VW / 4; ++k) b.vc[h2][k] = reinterpret_cast<const uint4*>(r)[k];
    }
#pragma unroll
    for (int k = 0; k < C::VSZ_LD; ++k) {
      int bi, off;
      sz_chunk(k, 4 * NGR * G, bi, off);
      bi = bi < NBS ? bi : NBS - 1;
      b.vsz[k] = *reinterpret_cast<const uint4*>(span_rec<C>(g, blocks, table, sp, blk0 + bi) + C::REC_VS + off);
    }
  };
  auto blk_ok = [&](Span sp, int blk) -> bool {
    if (blk >= sp.end) return false;
    if constexpr (!C::PAGED) return true;
    const int page = table[(size_t)sp.b * g.max_blocks + blk];
    return page >= 0 && page < g.num_pages;
  };

  // running state of the current unit
  float m_run, l_lane, lam_k[C::VSZ_LD], o[8];
  int lam_grp[C::VSZ_LD];   // value group of the lane's zero chunk k (-1: a scale chunk)
#pragma unroll
  for (int k = 0; k < C::VSZ_LD; ++k) {
    int bi, off;
    sz_chunk(k, 4 * NGR * G, bi, off);
    lam_grp[k] = (bi < NBS && off >= 2 * NGR * G) ? ((off - 2 * NGR * G) / 2) / G : -1;
  }

  const bool rot_q = (g.rot & KVQ_ROTATE_KEYS) != 0;
  auto run_set = [&](Span cur, int si, Span nsp, int nsi) {
    const int blk0 = cur.begin + si * NBS;
    // the next set's loads go out first and stay in flight through this set
    SetBuf nb;
    load_set(nb, nsp, nsi);
    if (si == 0) {   // a unit's first set: its query (prefetched with the set) into LDS
      float x0 = in_val<C>(cb.qw & 0xffffu) * qscale, x1 = in_val<C>(cb.qw >> 16) * qscale;
      // (rotated keys: the blocks hold R(k) = H k / 8, so the query is rotated
      // the same way, H q' * 8 / D, and the scores are unchanged)
      if (rot_q) wht_row_pairs(x0, x1, 8.0f / D);
      *reinterpret_cast<float2*>(L.q + 2 * lane) = make_float2(x0, x1);
      wave_lds_fence();
    }
    // ---- q~ = q' * s_K and kappa partials from the key scale/zero chunks ----
#pragma unroll
    for (int k = 0; k < C::KSZ_LD; ++k) {
      int bi, off;
      sz_chunk(k, 4 * D, bi, off);
      if (bi < NBS) {
        const bool zero = off >= 2 * D;
        const int c0 = (off % (2 * D)) / 2;   // 8 channels c0..c0+7
        const float4 qa = *reinterpret_cast<const float4*>(L.q + c0);
        const float4 qb = *reinterpret_cast<const float4*>(L.q + c0 + 4);
        const uint4 w = cb.ksz[k];
        const float x[8] = {qa.x * h2f_lo(w.x), qa.y * h2f_hi(w.x), qa.z * h2f_lo(w.y), qa.w * h2f_hi(w.y),
                            qb.x * h2f_lo(w.z), qb.y * h2f_hi(w.z), qb.z * h2f_lo(w.w), qb.w * h2f_hi(w.w)};
        if (!zero) {
          float* dst = L.qt + bi * C::QT_STRIDE + c0;
          *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
        // every lane of a 16-lane row holds the same (block, section)
        const float kp = row_sum16(((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7])));
        if (zero && (lane & 15) == 0) L.kap[bi] = kp;
      }
    }
    wave_lds_fence();
    // ---- scores of tokens lane and lane + 64 ----
    float s[kTokLane];
#pragma unroll
    for (int tl = 0; tl < kTokLane; ++tl) {
      const int tok = lane + 64 * tl;
      const int sbi = tok / G;
      const bool valid = blk_ok(cur, blk0 + sbi);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      const float* qt = L.qt + sbi * C::QT_STRIDE;
#pragma unroll
      for (int wi = 0; wi < C::KW; ++wi) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(&cb.kc[tl][wi / 4])[wi % 4];
        constexpr int PER = 32 / C::KB;   // channels per word
        float cf[PER];
        word_codes<C::KB>(w, cf);
#pragma unroll
        for (int e4 = 0; e4 < PER / 4; ++e4) {
          const float4 qv = *reinterpret_cast<const float4*>(qt + PER * wi + 4 * e4);
          acc[0] = fmaf(qv.x, cf[4 * e4 + 0], acc[0]);
          acc[1] = fmaf(qv.y, cf[4 * e4 + 1], acc[1]);
          acc[2] = fmaf(qv.z, cf[4 * e4 + 2], acc[2]);
          acc[3] = fmaf(qv.w, cf[4 * e4 + 3], acc[3]);
        }
      }
      s[tl] = valid ? ((acc[0] + acc[1]) + (acc[2] + acc[3])) + L.kap[sbi] : -INFINITY;
      asm volatile("" ::: "memory");   // one token's operands live at a time
    }

    // ---- online softmax, lazily rescaled ----
    float smax = s[0];
#pragma unroll
    for (int tl = 1; tl < kTokLane; ++tl) smax = fmaxf(smax, s[tl]);
    const float mx = wave_max64(smax);
    if (mx > m_run + kRescaleLog2) {   // wave-uniform
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
      m_run = mx;
      l_lane *= alpha;
#pragma unroll
      for (int k = 0; k < C::VSZ_LD; ++k) lam_k[k] *= alpha;
#pragma unroll
      for (int cj = 0; cj < 8; ++cj) o[cj] *= alpha;
    }
#pragma unroll
    for (int tl = 0; tl < kTokLane; ++tl) {
      const float p = s[tl] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[tl] - m_run);
      l_lane += p;
      L.p[lane + 64 * tl] = p;
    }
    wave_lds_fence();

    // ---- p~ = p * s_V and lambda partials from the value scale/zero chunks ----
#pragma unroll
    for (int k = 0; k < C::VSZ_LD; ++k) {
      int bi, off;
      sz_chunk(k, 4 * NGR * G, bi, off);
      if (bi < NBS) {
        const bool zero = off >= 2 * NGR * G;
        const int e0 = (off % (2 * NGR * G)) / 2;   // entries e0..e0+7 of [NGR][G]
        const int j = e0 / G, t = bi * G + e0 % G;  // group, set-relative first token
        const float4 pa = *reinterpret_cast<const float4*>(L.p + t);
        const float4 pb = *reinterpret_cast<const float4*>(L.p + t + 4);
        const uint4 w = cb.vsz[k];
        const float x[8] = {pa.x * h2f_lo(w.x), pa.y * h2f_hi(w.x), pa.z * h2f_lo(w.y), pa.w * h2f_hi(w.y),
                            pb.x * h2f_lo(w.z), pb.y * h2f_hi(w.z), pb.z * h2f_lo(w.w), pb.w * h2f_hi(w.w)};
        if (!zero) {
          float* dst = L.pv + j * kSetTok + t;
          *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
        } else {
          lam_k[k] += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
        }
      }
    }
    // next set's key data can load now
    wave_lds_fence();

    // ---- P.V: channels 16 cj + n over the lane's two runs ----
#pragma unroll
    for (int h2 = 0; h2 < C::RPL; ++h2) {
      const int t0 = 8 * (rr + 4 * h2);   // set-relative first token of the run
#pragma unroll
      for (int wi = 0; wi < C::VW; ++wi) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(&cb.vc[h2][wi / 4])[wi % 4];
        constexpr int PER = 32 / C::VB;   // codes per word = (channels per word) x 8 tokens
        float cf[PER];
        word_codes<C::VB>(w, cf);
        // entry i of the run's stream: channel index cj = i / 8, token t0 + i % 8
#pragma unroll
        for (int c8 = 0; c8 < PER / 8; ++c8) {
          const int cj = (PER / 8) * wi + c8;
          const int j = (16 * cj + n) / C::GV;
          const float4 pa = *reinterpret_cast<const float4*>(L.pv + j * kSetTok + t0);
          const float4 pb = *reinterpret_cast<const float4*>(L.pv + j * kSetTok + t0 + 4);
          float a = o[cj];
          a = fmaf(pa.x, cf[8 * c8 + 0], a);
          a = fmaf(pa.y, cf[8 * c8 + 1], a);
          a = fmaf(pa.z, cf[8 * c8 + 2], a);
          a = fmaf(pa.w, cf[8 * c8 + 3], a);
          a = fmaf(pb.x, cf[8 * c8 + 4], a);
          a = fmaf(pb.y, cf[8 * c8 + 5], a);
          a = fmaf(pb.z, cf[8 * c8 + 6], a);
          a = fmaf(pb.w, cf[8 * c8 + 7], a);
          o[cj] = a;
        }
      }
      asm volatile("" ::: "memory");   // one run's operands live at a time
    }
    cb = nb;
    wave_lds_fence();   // L.qt, L.p and L.pv are rewritten by the next set
  };

  // the unit's result: o_c = sum over the 4 run lanes + lambda(group of c)
  auto finish_unit = [&](float* __restrict__ out_part) {
    const float lsum = wave_sum64(l_lane);
    // lambda of group j: the zero-chunk partials of every lane whose chunk
    // belongs to group j, summed over the wave
    float lam[NGR];
#pragma unroll
    for (int j = 0; j < NGR; ++j) {
      float x = 0.f;
#pragma unroll
      for (int k = 0; k < C::VSZ_LD; ++k) x += lam_grp[k] == j ? lam_k[k] : 0.f;
      lam[j] = wave_sum64(x);
    }
#pragma unroll
    for (int cj = 0; cj < 8; ++cj) {
      const float v = rows_sum4(o[cj]);
      if (rr == 0) out_part[16 * cj + n] = v + lam[(16 * cj + n) / C::GV];
    }
    if (lane == 0) {
      out_part[D] = m_run;
      out_part[D + 1] = lsum;
    }
    wave_lds_fence();
  };

  int u = first;
  Span cur = first_span;
  load_set(cb, cur, 0);
  while (true) {
    m_run = -INFINITY;
    l_lane = 0.f;
#pragma unroll
    for (int k = 0; k < C::VSZ_LD; ++k) lam_k[k] = 0.f;
#pragma unroll
    for (int cj = 0; cj < 8; ++cj) o[cj] = 0.f;
    const int nsets = (cur.end - cur.begin + NBS - 1) / NBS;
    for (int si = 0; si + 1 < nsets; ++si) run_set(cur, si, cur, si + 1);
    const int nu = claim(claimed);
    const bool more = nu < units;
    const Span nxt = more ? locate(nu) : cur;
    run_set(cur, nsets - 1, nxt, more ? 0 : nsets - 1);
    finish_unit(ws + (size_t)u * (D + 2));
    if (!more) break;
    u = nu;
    cur = nxt;
    claimed = issue();
  }
}

// ------------------------------------------------------------------------------------
// The kernel: persistent waves taking units from the work queues (as the
// matrix-core path does).
// ------------------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mha_kernel(
    Geom g, const uint8_t* __restrict__ blocks, const int32_t* __restrict__ table,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring, int32_t* __restrict__ state,
    const uint16_t* __restrict__ q, float qscale, int max_blk, int* __restrict__ ws_plan, float* __restrict__ ws) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* plan = reinterpret_cast<int*>(smem);
  const int pints = plan_ints(g.B);
  const int pre_bytes = plan_lds_bytes(g.B);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* wl = reinterpret_cast<float*>(smem + pre_bytes) + wave * C::L_WAVE;
  WaveLds<C> L;
  L.q = wl;
  L.qt = L.q + C::L_Q;
  L.kap = L.qt + C::L_QT;
  L.p = L.kap + C::L_KAP;
  L.pv = L.p + C::L_P;

  build_unit_plan(g, state, max_blk, C::NBS, kRingTok, plan, blockIdx.x == 0);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < pints; i += blockDim.x) ws_plan[i] = plan[i];
  const int units = plan[kPlanUnits];
  const int queue = blockIdx.x % kQueues;
  const int qwaves = (int)(gridDim.x / kQueues) * kWaves;
  int* counter = state + state_queue_word(g.B, queue);
  int* done = state + state_done_word(g.B);
  auto issue = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(counter, 1);
    return v;
  };
  auto claim = [&](int raw) -> int { return queue + kQueues * (qwaves + __builtin_amdgcn_readfirstlane(raw)); };
  auto span_of = [&](int uu) -> Span {
    const Unit un = locate_unit(g, plan, uu, max_blk);
    Span sp;
    sp.b = __builtin_amdgcn_readfirstlane(un.b);
    sp.h = __builtin_amdgcn_readfirstlane(un.h);
    sp.begin = __builtin_amdgcn_readfirstlane(un.begin);
    sp.end = __builtin_amdgcn_readfirstlane(un.end);
    return sp;
  };

  int u = queue + kQueues * ((int)(blockIdx.x / kQueues) * kWaves + wave);
  int claimed = issue();
  while (u < units && u < plan[kPlanSec]) {
    const Span sp = span_of(u);
    ring_unit<C>(g, L, k_ring, v_ring, q, qscale, sp.b, sp.h, sp.begin, sp.end, ws + (size_t)u * (C::D + 2));
    u = claim(claimed);
    claimed = issue();
  }
  if (u < units)
    quant_stream<C>(g, L, blocks, table, q, qscale, units, u, span_of(u), claimed, span_of, issue, claim, ws);
  // All of this wave's claims have returned, so once every wave has counted
  // itself here no claim is outstanding and the counters can be re-armed (no
  // fence: the partial states reach the combine kernel at the launch boundary).
  if (lane == 0) {
    if (atomicAdd(done, 1) == (int)gridDim.x * kWaves - 1) {
      for (int k = 0; k < kQueues; ++k) atomicExch(state + state_queue_word(g.B, k), 0);
      atomicExch(done, 0);
    }
  }
}

template <class C>
hipError_t launch_mha(const Geom& g, const kvq_cache& c, const void* q, float scale, int max_blk, void* ws,
                      hipStream_t s) {
  const size_t lds = (size_t)plan_lds_bytes(g.B) + (size_t)kWaves * C::L_WAVE * 4;
  const int grid = persistent_grid(decode_mha_kernel<C>, lds);
  hipLaunchKernelGGL((decode_mha_kernel<C>), dim3(grid), dim3(256), lds, s, g,
                     static_cast<const uint8_t*>(c.blocks), c.block_table, static_cast<const uint16_t*>(c.k_ring),
                     static_cast<const uint16_t*>(c.v_ring), c.state, static_cast<const uint16_t*>(q),
                     scale * 1.4426950408889634f, max_blk, static_cast<int*>(ws),
                     reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan_bytes(g.B)));
  return hipGetLastError();
}

}  // namespace mha
}  // namespace kvq
