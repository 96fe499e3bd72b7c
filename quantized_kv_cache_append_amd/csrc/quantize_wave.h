// Quantize-and-pack of one block by one wave, head_dim 128 (gfx950): the
// flush path for the configurations the workloads use (any other shape runs
// the workgroup routine in append_flush.hip).
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026": section "KIVI (2024)" -- keys per channel over a group
//        of tokens, values per token over a group of channels, each group with
//        its own min/max parameters; innovation 3 -- 16 INT2 or 8 INT4 codes per
//        32-bit word.
//
// Both tiles are read straight from the ring into registers, each in the lane
// layout that keeps its groups inside a lane, so no statistic needs a cross-lane
// reduction and nothing goes through LDS:
//   keys:   lane l holds channels 2l and 2l+1 of all G tokens (one coalesced
//           4-byte load per token row); a key code word (16 INT2 / 8 INT4
//           channels of one token) is the OR of the contributions of the 8 / 4
//           lanes that hold its channels;
//   values: lane l holds token l % G and the slice l / G of 128 G / 64 channels
//           (16-byte loads); a value code word (8 tokens of one or two channels)
//           is the OR of the 8 lanes that hold those tokens.
// The group arithmetic is formula F, shared with the workgroup routine.
#pragma once

#include "common.h"

namespace kvq {

// Formula F on one group whose min and max are known (fp32 IEEE steps, round to
// nearest even, no fused multiply-add). Returns the fp16 bits of scale and
// zero and the reciprocal used for the codes (0 for a constant group).
struct GroupParams {
  uint16_t s16, z16;
  float zf, inv;
};
__device__ __forceinline__ GroupParams group_params(float mn, float mx, int bits) {
  GroupParams p;
  p.z16 = f32_to_f16_bits(mn);
  const float qmax = (float)((1 << bits) - 1);
  const float range = __fsub_rn(mx, mn);
  p.s16 = f32_to_f16_bits(__fdiv_rn(range, qmax));
  const float sf = f16_to_f32(p.s16);
  p.zf = f16_to_f32(p.z16);
  p.inv = (sf == 0.0f) ? 0.0f : __fdiv_rn(1.0f, sf);
  return p;
}
__device__ __forceinline__ uint32_t group_code(float x, const GroupParams& p, int bits) {
  if (p.inv == 0.0f) return 0u;
  const float t = __fmul_rn(__fsub_rn(x, p.zf), p.inv);
  const float qmax = (float)((1 << bits) - 1);
  const float r = fminf(fmaxf(rintf(t), 0.0f), qmax);
  return (uint32_t)r;
}

namespace qwave {

template <bool BF16_, int G_, int KB_, int VB_, int GV_>
struct Cfg {
  static constexpr bool BF16 = BF16_;
  static constexpr int G = G_, KB = KB_, VB = VB_, GV = GV_, D = 128;
  static constexpr int KW = D * KB / 32;     // key code words per token
  static constexpr int KLPW = 16 / KB;       // lanes per key code word (2 channels per lane)
  static constexpr int SL = D * G / 64;      // value channels per lane
  static constexpr int SLV = SL / 8;         // 16-byte value loads per lane
  static constexpr int NGR = D / GV;         // value groups per token
  static_assert(G == 16 || G == 32 || G == 64, "blocks of 16, 32 or 64 tokens");
  static_assert(KB == 2 || KB == 4, "2- or 4-bit keys");
  static_assert(VB == 2 || VB == 4, "2- or 4-bit values");
  static_assert(GV <= SL && SL % GV == 0, "a value group inside one lane's channel slice");
};

// OR over aligned groups of 4 / 8 lanes; every lane gets its group's result.
__device__ __forceinline__ uint32_t or4(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return x;
}
__device__ __forceinline__ uint32_t or8(uint32_t x) {
  x = or4(x);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return x;
}

// Walsh-Hadamard pre-rotation of a value row held as SL consecutive channels
// per lane (lane l: channels (l / G) SL ..; the row's other channels in lanes
// l ^ G, l ^ 2G, ...), in the order of the stored-side definition: stages
// h = 1, 2, ..., 64, each (a, b) -> (a + b, a - b) rounded to fp32, the stages
// below SL inside the lane, the others with the partner lane; then x 1/8.
template <int SL, int G>
__device__ __forceinline__ void rotate_value_row(float (&x)[SL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 1; h < SL; h <<= 1)
#pragma unroll
    for (int j = 0; j < SL / 2; ++j) {
      const int i = (j / h) * 2 * h + j % h;
      const float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
#pragma unroll
  for (int m = 1; m * SL < 128; m <<= 1) {   // stage h = m SL: the partner is lane ^ m G
    const bool upper = ((lane / G) & m) != 0;
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const float p = __shfl_xor(x[k], m * G, 64);
      x[k] = upper ? p - x[k] : x[k] + p;
    }
  }
#pragma unroll
  for (int k = 0; k < SL; ++k) x[k] *= 0.125f;
}

// Quantize tokens blk*G .. blk*G+G-1 of ring `pair` into record `rec`. Called
// by all 64 lanes of one wave; the ring rows must be visible to the wave. With
// ROT the rows of the sides g.rot names are rotated first, in registers: a key
// row is spread over the wave (wht_row_pairs), a value row over 128 / SL lanes
// (at G = 64 the rotated rows exceed the register file by 32 values per lane,
// which the compiler spills: still 6.6x the workgroup routine's rate).
template <class Q, bool ROT = false>
__device__ __forceinline__ void quantize_block(const Geom& g, uint8_t* __restrict__ rec,
                                               const uint16_t* __restrict__ k_ring,
                                               const uint16_t* __restrict__ v_ring, int pair, int blk) {
  constexpr int G = Q::G, D = Q::D, KB = Q::KB, VB = Q::VB, GV = Q::GV;
  const int lane = threadIdx.x & 63;
  // ring slot of token t: base + t, wrapping at most once (G <= C)
  const int base = (int)(((long long)blk * G) % g.C);
  const size_t pair_row = (size_t)pair * g.C;
  auto row = [&](int t) -> size_t {
    int s = base + t;
    s -= s >= g.C ? g.C : 0;
    return (pair_row + s) * D;
  };

  // ---- loads: keys (lane = channel pair), values (lane = token x slice) ----
  uint32_t kd[G];
#pragma unroll
  for (int t = 0; t < G; ++t) kd[t] = reinterpret_cast<const uint32_t*>(k_ring + row(t))[lane];
  const int vt = lane % G, cbase = (lane / G) * Q::SL;
  uint4 vd[Q::SLV];
  auto load_values = [&]() {
    const uint4* src = reinterpret_cast<const uint4*>(v_ring + row(vt) + cbase);
#pragma unroll
    for (int k = 0; k < Q::SLV; ++k) vd[k] = src[k];
  };
  // (rotated: the value rows are loaded once the keys are done, so that the
  // rotated key rows and value slice are never live together)
  if constexpr (!ROT) load_values();

  // rotated key rows (fp32): channels 2 lane, 2 lane + 1 of each token
  float kr0[ROT ? G : 1], kr1[ROT ? G : 1];
  if constexpr (ROT) {
    const bool rk = (g.rot & KVQ_ROTATE_KEYS) != 0;
#pragma unroll
    for (int t = 0; t < G; ++t) {
      kr0[t] = in_to_f32<Q::BF16>(kd[t] & 0xffffu);
      kr1[t] = in_to_f32<Q::BF16>(kd[t] >> 16);
      if (rk) wht_row_pairs(kr0[t], kr1[t], 0.125f);
    }
  }
  auto key0 = [&](int t) -> float {
    if constexpr (ROT) return kr0[t];
    else return in_to_f32<Q::BF16>(kd[t] & 0xffffu);
  };
  auto key1 = [&](int t) -> float {
    if constexpr (ROT) return kr1[t];
    else return in_to_f32<Q::BF16>(kd[t] >> 16);
  };

  // ---- keys: one group per channel over the G tokens ----
  {
    float mn0 = key0(0), mx0 = mn0;
    float mn1 = key1(0), mx1 = mn1;
#pragma unroll
    for (int t = 1; t < G; ++t) {
      const float x0 = key0(t), x1 = key1(t);
      mn0 = fminf(mn0, x0);
      mx0 = fmaxf(mx0, x0);
      mn1 = fminf(mn1, x1);
      mx1 = fmaxf(mx1, x1);
    }
    const GroupParams p0 = group_params(mn0, mx0, KB), p1 = group_params(mn1, mx1, KB);
    reinterpret_cast<uint32_t*>(rec + g.rec_ks)[lane] = (uint32_t)p0.s16 | ((uint32_t)p1.s16 << 16);
    reinterpret_cast<uint32_t*>(rec + g.rec_kz)[lane] = (uint32_t)p0.z16 | ((uint32_t)p1.z16 << 16);
    // channel 2l sits at slot (2l) % (32 / KB) of word (2l) / (32 / KB) of its token
    const int sh = ((2 * lane) % (32 / KB)) * KB;
    const int sub = lane % Q::KLPW;   // token (within a store group) this lane stores
    uint32_t* kc = reinterpret_cast<uint32_t*>(rec + g.rec_kc);
#pragma unroll
    for (int t0 = 0; t0 < G; t0 += Q::KLPW) {
      uint32_t mine = 0;
#pragma unroll
      for (int k = 0; k < Q::KLPW; ++k) {
        const int t = t0 + k;
        const uint32_t c0 = group_code(key0(t), p0, KB);
        const uint32_t c1 = group_code(key1(t), p1, KB);
        uint32_t w = (c0 << sh) | (c1 << (sh + KB));
        w = KB == 2 ? or8(w) : or4(w);
        mine = sub == k ? w : mine;
      }
      // lane l stores word l / KLPW of token t0 + l % KLPW
      kc[(t0 + sub) * Q::KW + lane / Q::KLPW] = mine;
    }
  }

  // ---- values: one group per (token, GV channels) ----
  if constexpr (ROT) load_values();
  {
    uint16_t* vs = reinterpret_cast<uint16_t*>(rec + g.rec_vs);
    uint16_t* vz = reinterpret_cast<uint16_t*>(rec + g.rec_vz);
    auto vraw = [&](int c) -> float {   // channel cbase + c of token vt
      const uint32_t w = reinterpret_cast<const uint32_t*>(&vd[c / 8])[(c % 8) / 2];
      return in_to_f32<Q::BF16>((c & 1) ? (w >> 16) : (w & 0xffffu));
    };
    float vr[ROT ? Q::SL : 1];   // the rotated row slice (fp32)
    if constexpr (ROT) {
#pragma unroll
      for (int c = 0; c < Q::SL; ++c) vr[c] = vraw(c);
      if (g.rot & KVQ_ROTATE_VALUES) rotate_value_row<Q::SL, G>(vr);
    }
    auto vval = [&](int c) -> float {
      if constexpr (ROT) return vr[c];
      else return vraw(c);
    };
    GroupParams p[Q::SL / GV];
#pragma unroll
    for (int j = 0; j < Q::SL / GV; ++j) {
      float mn = vval(j * GV), mx = mn;
#pragma unroll
      for (int c = 1; c < GV; ++c) {
        const float x = vval(j * GV + c);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      p[j] = group_params(mn, mx, VB);
      const int jg = cbase / GV + j;   // group index within the token
      vs[jg * G + vt] = p[j].s16;
      vz[jg * G + vt] = p[j].z16;
    }
    // code stream position of (t, c): ((t/8*16 + c%16) * (D/16) + c/16) * 8 + t%8,
    // LSB first; a word holds VB == 2: 8 tokens of channels c and c+16 (c/16
    // even), VB == 4: 8 tokens of channel c
    uint32_t* vc = reinterpret_cast<uint32_t*>(rec + g.rec_vc);
    const int r = vt % 8, t8 = vt / 8;
    constexpr int NW = VB == 2 ? Q::SL / 2 : Q::SL;   // words per 8-lane group
    uint32_t words[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      if constexpr (VB == 2) {
        const int cl = (u / 16) * 32 + u % 16;   // local channel with (c/16) even
        const uint32_t a = group_code(vval(cl), p[cl / GV], VB);
        const uint32_t b = group_code(vval(cl + 16), p[(cl + 16) / GV], VB);
        words[u] = or8((a << (2 * r)) | (b << (16 + 2 * r)));
      } else {
        const uint32_t a = group_code(vval(u), p[u / GV], VB);
        words[u] = or8(a << (4 * r));
      }
    }
    // lane r of each 8-lane group stores words r, r + 8, ...
#pragma unroll
    for (int u0 = 0; u0 < NW; u0 += 8) {
      uint32_t mine = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) mine = r == k ? words[u0 + k] : mine;
      const int u = u0 + r;
      int W;
      if constexpr (VB == 2) {
        const int c = cbase + (u / 16) * 32 + u % 16;   // c / 16 even
        W = ((t8 * 16 + c % 16) * (D / 16) + c / 16) / 2;
      } else {
        const int c = cbase + u;
        W = (t8 * 16 + c % 16) * (D / 16) + c / 16;
      }
      vc[W] = mine;
    }
  }
}

}  // namespace qwave
}  // namespace kvq
