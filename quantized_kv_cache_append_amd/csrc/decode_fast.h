// MFMA decode path for head_dim 128 (gfx950): kernel template. Instantiated per
// configuration in decode_fast_*.hip.
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
//   [P1] ai-automate.fr, "KV-cache compressé et modèles 4-bit ...", Minima-KV:
//        partial attention states merged by an online softmax.
//
// Arithmetic. With x_hat = code*s + z, the score of token t for query q is
//   q . k_hat_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c ,
// so per block the key scale is folded into the query (q~ = q * s_K) and the
// zero-point term kappa = q . z_K is one dot product per block; likewise
//   o_c = sum_t (p_t s_tj) code_tc + sum_t p_t z_tj          (j = group of c).
// The contractions run on MFMA (v_mfma_f32_16x16x32_bf16): codes 0..15 are
// exact in bf16 (unpacked with the scaled fp4/fp8 -> bf16 conversions), and the
// real-valued operand (q~ or p~) is split into a bf16 high part and a bf16
// remainder, two MFMAs accumulating in fp32 -- about 16 significant bits per
// product term instead of bf16's 8.
//
// Layout of one wave's work item: a run of quantized blocks of one (sequence,
// kv head), processed in "sets" of NB blocks whose NB*NG (block, head) pairs
// are the 16 columns of the score MFMA; or a chunk of up to 32 ring tokens.
// Scores come out as D[token][(block, head)]; after the online-softmax update
// the probabilities, scaled per value group and split hi/lo, go through LDS
// into the A operand of the P.V MFMA (rows = head hi / head lo, k = tokens,
// columns = 16 channels). The value codes are stored in 8-token chunks so that
// each lane's B operand is one contiguous 16- (INT2) or 32-byte (INT4) load.
#pragma once

#include <type_traits>

#include "common.h"
#include "decode_units.h"

namespace kvq {
namespace fast {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kRingChunk = 32;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// --- exact code unpacking --------------------------------------------------------
// 8 codes of one 8-element run (LSB first) -> 4 bf16 pairs in the k order
// (0,2) (1,3) (4,6) (5,7). INT2: a 2-bit code c placed in a nibble reads as
// fp4 e2m1 c/2, so a scale of 2 gives c exactly. INT4: a 4-bit code in a byte
// reads as fp8 e4m3 c*2^-9 (subnormals and the first binade are evenly
// spaced), so a scale of 2^9 gives c exactly.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t src) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 2.0f, SEL));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t src) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 512.0f, HI));
}
// Both 16-bit halves of an INT2 word (two runs of 8 codes).
__device__ __forceinline__ void unpack_int2_word(uint32_t w, uint4& lo_run, uint4& hi_run) {
  const uint32_t e0 = w & 0x33333333u, e1 = (w >> 2) & 0x33333333u;
  lo_run.x = fp4x2_to_bf16x2<0>(e0);
  lo_run.y = fp4x2_to_bf16x2<0>(e1);
  lo_run.z = fp4x2_to_bf16x2<1>(e0);
  lo_run.w = fp4x2_to_bf16x2<1>(e1);
  hi_run.x = fp4x2_to_bf16x2<2>(e0);
  hi_run.y = fp4x2_to_bf16x2<2>(e1);
  hi_run.z = fp4x2_to_bf16x2<3>(e0);
  hi_run.w = fp4x2_to_bf16x2<3>(e1);
}
// One INT4 word (one run of 8 codes).
__device__ __forceinline__ uint4 unpack_int4_word(uint32_t w) {
  const uint32_t e0 = w & 0x0F0F0F0Fu, e1 = (w >> 4) & 0x0F0F0F0Fu;
  uint4 r;
  r.x = fp8x2_to_bf16x2<false>(e0);
  r.y = fp8x2_to_bf16x2<false>(e1);
  r.z = fp8x2_to_bf16x2<true>(e0);
  r.w = fp8x2_to_bf16x2<true>(e1);
  return r;
}
// k position of element e of a run of 8 (its own inverse).
__host__ __device__ constexpr int kperm(int e) { return (e & 4) | ((e & 1) << 1) | ((e >> 1) & 1); }

// --- hi/lo splits -------------------------------------------------------------------
// Two floats to a bf16 pair, each rounded to nearest even (low half = a). Written
// as the instruction itself: from the vector-of-bf16 form the compiler converted
// the low element a second time to get it back as a float.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// a times the fp16 in the low (HI = false) or high half of s, rounded once: one
// mixed-precision FMA with a zero addend instead of a conversion and a multiply.
template <bool HI>
__device__ __forceinline__ float mul_f16(float a, uint32_t s) {
  float x;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(x) : "v"(a), "v"(s));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(x) : "v"(a), "v"(s));
  return x;
}
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (the subtraction is exact):
// about 16 significant bits per value in two bf16 operands. Six instructions
// per pair of values.
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(x0, x1);
  const float r0 = x0 - __uint_as_float(hi << 16);
  const float r1 = x1 - __uint_as_float(hi & 0xffff0000u);
  lo = pk_bf16(r0, r1);
}
__device__ __forceinline__ void split_f16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const f16x2v h = {(_Float16)x0, (_Float16)x1};
  hi = __builtin_bit_cast(uint32_t, h);
  const float h0 = (float)h[0], h1 = (float)h[1];
  const f16x2v l = {(_Float16)(x0 - h0), (_Float16)(x1 - h1)};
  lo = __builtin_bit_cast(uint32_t, l);
}
__device__ __forceinline__ float lo_half_f16(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float hi_half_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// --- cross-lane helpers ---------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int K>
__device__ __forceinline__ float ror(float x) { return dpp<0x120 + K>(x); }

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// Combine x over the lanes holding the same head: columns n = blk*NG + head
// of every 16-lane row (unused columns must hold the identity), then the four
// rows. Every lane of a used column ends with the head's total.
template <int NG, typename Op>
__device__ __forceinline__ float reduce_head(float x, int n, Op op) {
  if constexpr (NG == 6) {
    const float a = ror<6>(x);    // lane n <- lane n-6
    const float b = ror<10>(x);   // lane n <- lane n+6
    x = op(x, n < 6 ? b : a);
  } else {
    if constexpr (NG <= 1) x = op(x, ror<1>(x));
    if constexpr (NG <= 2) x = op(x, ror<2>(x));
    if constexpr (NG <= 4) x = op(x, ror<4>(x));
    if constexpr (NG <= 8) x = op(x, ror<8>(x));
  }
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
// Combine over the four rows only (same lane position).
template <typename Op>
__device__ __forceinline__ float reduce_rows(float x, Op op) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

template <int NG_, int KB_, int VB_, int G_, int GV_, bool BF16_, bool PAGED_>
struct Cfg {
  static constexpr int NG = NG_, KB = KB_, VB = VB_, G = G_, GV = GV_;
  static constexpr bool BF16 = BF16_, PAGED = PAGED_;
  static constexpr int D = 128;
  static constexpr int NB = (16 / NG) < 4 ? (16 / NG) : 4;   // blocks per set
  static constexpr int NCOL = NB * NG;                         // used score columns
  static constexpr int TPB = G / 16;                           // 16-token tiles per block
  static constexpr int SET_TOK = NB * G;
  static constexpr int KS_SET = SET_TOK / 32;                  // P.V k-steps per set
  static constexpr int NGR = D / GV;                           // value groups
  static constexpr int KROW = D * KB / 8;                      // key code bytes per token
  static constexpr int KLANE = KROW / 4;                       // per lane group
  static constexpr int VLANE = 8 * VB;                         // value code bytes per lane per k-step
  // record sections
  static constexpr int REC_KC = 0;
  static constexpr int REC_KS = G * KROW;
  static constexpr int REC_KZ = REC_KS + 2 * D;
  static constexpr int REC_VC = REC_KZ + 2 * D;
  static constexpr int REC_VS = REC_VC + G * D * VB / 8;
  static constexpr int REC_VZ = REC_VS + 2 * NGR * G;
  static constexpr int REC = REC_VZ + 2 * NGR * G;
  // the scale/zero sections of a record (scales then zero-points, contiguous)
  static constexpr int KSEC = REC_VC - REC_KS;                       // 4 D bytes
  static constexpr int VSEC = REC - REC_VS;                          // 4 NGR G bytes
  // a set's sections are loaded once, a contiguous share per lane, and staged
  // in LDS; each lane then reads the scales of its own column and channels
  static constexpr int KSZ_LANE = NB * KSEC / 64;
  static constexpr int VSZ_LANE = NB * VSEC / 64;
  // waves per SIMD: the 6-head group (32-token sets, the fewest registers and
  // LDS) runs three, which keeps more of its loads in flight; the others two
  static constexpr int WAVES_PER_SIMD = NG == 6 ? 3 : 2;
  // per-wave LDS (bytes). A query row takes QS floats: 4 more than D, so that the
  // rows of the group start 4 banks apart and the lanes of one row of the
  // operand layout, which read the same channels of different heads, do not
  // collide on a bank.
  static constexpr int QS = D + 4;
  static constexpr int LDS_Q = NG * QS * 4;
  static constexpr int LDS_A = KS_SET * NGR * 4 * 2 * NG * 16;
  static constexpr int LDS_O = 2 * NG * D * 4;
  static constexpr int LDS_P = kRingChunk * NG * 4;
  static constexpr int LDS_BUF = (LDS_A > LDS_O ? (LDS_A > LDS_P ? LDS_A : LDS_P) : (LDS_O > LDS_P ? LDS_O : LDS_P));
  static constexpr int LDS_ALPHA = 16 * 4;
  static constexpr int LDS_LAM = NG * NGR * 4;
  static constexpr int LDS_ZERO = 16;
  static constexpr int LDS_KS = NB * KSEC;
  static constexpr int LDS_VS = NB * VSEC;
  static constexpr int LDS_WAVE = LDS_Q + LDS_BUF + LDS_KS + LDS_VS + LDS_ALPHA + LDS_LAM + LDS_ZERO;
  static_assert(NG == 1 || NG == 2 || NG == 4 || NG == 6 || NG == 8, "column reductions exist for these groups");
  static_assert(NB >= 2, "query group must fit two blocks in 16 columns");
  static_assert(G % 16 == 0 && SET_TOK % 32 == 0, "sets must be whole P.V k-steps");
  static_assert(GV >= 16 && D % GV == 0, "value groups must cover whole 16-channel tiles");
  static_assert(KSEC == 4 * D && REC_KZ == REC_KS + 2 * D && REC_VZ == REC_VS + VSEC / 2, "sections contiguous");
  static_assert((KSZ_LANE == 8 || KSZ_LANE == 16 || KSZ_LANE == 32) && KSEC % KSZ_LANE == 0, "key share");
  static_assert((VSZ_LANE == 8 || VSZ_LANE == 16 || VSZ_LANE == 32) && VSEC % VSZ_LANE == 0, "value share");
};

// Pointer to block `blk` of (b, h); nullptr if a paged entry is out of range.
template <class C>
__device__ __forceinline__ const uint8_t* rec_ptr(const Geom& g, const uint8_t* blocks, const int32_t* table, int b,
                                                  int h, int blk) {
  if constexpr (!C::PAGED) return blocks + (((size_t)b * g.Hkv + h) * g.max_blocks + blk) * (size_t)C::REC;
  const int page = table[(size_t)b * g.max_blocks + blk];
  if (page < 0 || page >= g.num_pages) return nullptr;
  return blocks + ((size_t)page * g.Hkv + h) * (size_t)C::REC;
}

template <int NBYTES>
struct Chunk;
template <>
struct Chunk<8> {
  uint2 v;
};
template <>
struct Chunk<16> {
  uint4 v;
};
template <>
struct Chunk<32> {
  uint4 a, b;
};
template <int NBYTES>
__device__ __forceinline__ Chunk<NBYTES> load_chunk(const uint8_t* p) {
  Chunk<NBYTES> c;
  if constexpr (NBYTES == 8) {
    c.v = *reinterpret_cast<const uint2*>(p);
  } else if constexpr (NBYTES == 16) {
    c.v = *reinterpret_cast<const uint4*>(p);
  } else {
    c.a = *reinterpret_cast<const uint4*>(p);
    c.b = *reinterpret_cast<const uint4*>(p + 16);
  }
  return c;
}

template <int NBYTES>
__device__ __forceinline__ void store_chunk(uint8_t* p, const Chunk<NBYTES>& c) {
  if constexpr (NBYTES == 8) {
    *reinterpret_cast<uint2*>(p) = c.v;
  } else if constexpr (NBYTES == 16) {
    *reinterpret_cast<uint4*>(p) = c.v;
  } else {
    *reinterpret_cast<uint4*>(p) = c.a;
    *reinterpret_cast<uint4*>(p + 16) = c.b;
  }
}

// Key-code A operand of k-step ks from a lane's chunk of one token row
// (channels 32g .. 32g+31): k position kperm(e) of k-step ks is channel
// 32g + 8ks + e.
template <class C>
__device__ __forceinline__ void key_operands(const Chunk<C::KLANE>& ch, uint4 (&a)[4]) {
  if constexpr (C::KB == 2) {
    unpack_int2_word(ch.v.x, a[0], a[1]);
    unpack_int2_word(ch.v.y, a[2], a[3]);
  } else {
    a[0] = unpack_int4_word(ch.v.x);
    a[1] = unpack_int4_word(ch.v.y);
    a[2] = unpack_int4_word(ch.v.z);
    a[3] = unpack_int4_word(ch.v.w);
  }
}
// Value-code B operands of the 8 column tiles (channel 16nt + n) from a lane's
// chunk: 8 channels x 8 tokens.
template <class C>
__device__ __forceinline__ void value_operands(const Chunk<C::VLANE>& ch, uint4 (&bop)[8]) {
  if constexpr (C::VB == 2) {
    unpack_int2_word(ch.v.x, bop[0], bop[1]);
    unpack_int2_word(ch.v.y, bop[2], bop[3]);
    unpack_int2_word(ch.v.z, bop[4], bop[5]);
    unpack_int2_word(ch.v.w, bop[6], bop[7]);
  } else {
    bop[0] = unpack_int4_word(ch.a.x);
    bop[1] = unpack_int4_word(ch.a.y);
    bop[2] = unpack_int4_word(ch.a.z);
    bop[3] = unpack_int4_word(ch.a.w);
    bop[4] = unpack_int4_word(ch.b.x);
    bop[5] = unpack_int4_word(ch.b.y);
    bop[6] = unpack_int4_word(ch.b.z);
    bop[7] = unpack_int4_word(ch.b.w);
  }
}

template <class C>
__device__ __forceinline__ float in_val(uint32_t bits16) {
  return C::BF16 ? __uint_as_float(bits16 << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Scores are in log2 units. The running maximum of a head is only moved (and
// the accumulated state rescaled) when a new score exceeds it by more than
// this, so probabilities stay below 2^8 and most sets skip the rescale.
constexpr float kRescaleLog2 = 8.0f;

// Per-wave LDS regions.
template <class C>
struct WaveLds {
  float* qs;        // [NG][D] query scaled to log2 units
  uint8_t* buf;     // P.V A operands / item outputs / ring probabilities
  uint8_t* ks;      // [NB][KSEC] key scale / zero sections of the set being computed
  uint8_t* vs;      // [NB][VSEC] value scale / zero sections
  float* alpha;     // [16] per P.V row
  float* lam;       // [NG][NGR]
  uint4* zero16;
};

// ---------------------------------------------------------------------------------
// The full-precision ring tokens [t_begin, t_end) of one (sequence, kv head), in
// chunks of 32: scores on MFMA (A = key rows as stored, B = query hi/lo),
// online softmax across the chunks, P.V on the vector ALUs. Needs the scaled
// query in L.qs. Query row n sees ring tokens up to last + n % T (a block of
// T query tokens is causal; T = 1: last = the ring's last token).
// ---------------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void ring_unit(const Geom& g, const WaveLds<C>& L, const uint16_t* __restrict__ k_ring,
                                          const uint16_t* __restrict__ v_ring, int pair, int t_begin, int t_end,
                                          int last, float* __restrict__ out_part) {
  constexpr int NG = C::NG, D = C::D;
  const int lane = threadIdx.x & 63, gq = lane >> 4, n = lane & 15;
  const int last_n = last + n % g.T;   // this lane's head column sees tokens up to here
  // B operand: q' hi/lo, column n = head, k position e of k-step ks = channel 32gq + 8ks + e
  uint4 bq_hi[4], bq_lo[4];
  float escale = 1.0f;
  if constexpr (!C::BF16) {
    // fp16 operands: bring the largest |q'| near 2^14 (an exact power of two)
    float mx = 0.f;
    for (int idx = lane; idx < NG * D; idx += 64) mx = fmaxf(mx, fabsf(L.qs[(idx / D) * C::QS + idx % D]));
    mx = wave_max(mx);
    escale = ldexpf(1.0f, mx > 0.f ? 14 - ilogbf(mx) : 0);
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 32 * gq + 8 * ks + 2 * r;
      const float x0 = n < NG ? L.qs[n * C::QS + c] * escale : 0.f;
      const float x1 = n < NG ? L.qs[n * C::QS + c + 1] * escale : 0.f;
      if constexpr (C::BF16) split_bf16(x0, x1, hi[r], lo[r]);
      else split_f16(x0, x1, hi[r], lo[r]);
    }
    bq_hi[ks] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    bq_lo[ks] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  const float inv_escale = 1.0f / escale;   // exact: a power of two
  const size_t ring_base = (size_t)pair * g.C;
  float m_run = -INFINITY, l_run = 0.f;   // per lane: head n (lanes n < NG)
  float o0[NG], o1[NG];                   // per lane: channels 2*lane, 2*lane+1 of every head
#pragma unroll
  for (int j = 0; j < NG; ++j) o0[j] = o1[j] = 0.f;
  float* pl = reinterpret_cast<float*>(L.buf);   // [32 tokens][NG]

  for (int t0 = t_begin; t0 < t_end; t0 += kRingChunk) {
    const int t1 = min(t_end, t0 + kRingChunk);
    // value rows of the chunk (rows past t1 read row t0 and get probability 0)
    // and key rows, all in flight together
    uint32_t vv[kRingChunk];
#pragma unroll
    for (int u = 0; u < kRingChunk; ++u) {
      const int t = t0 + u < t1 ? t0 + u : t0;
      vv[u] = *reinterpret_cast<const uint32_t*>(v_ring + (ring_base + t % g.C) * D + 2 * lane);
    }
    uint4 ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = t0 + 16 * tt + n;   // A row = token
      const uint16_t* krow = k_ring + (ring_base + (t < t1 ? t : t0) % g.C) * D + 32 * gq;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[tt][ks] = *reinterpret_cast<const uint4*>(krow + 8 * ks);
    }
    float s[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (C::BF16) {
          acc = mfma_bf16(ka[tt][ks], bq_hi[ks], acc);
          acc = mfma_bf16(ka[tt][ks], bq_lo[ks], acc);
        } else {
          acc = mfma_f16(ka[tt][ks], bq_hi[ks], acc);
          acc = mfma_f16(ka[tt][ks], bq_lo[ks], acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * tt + 4 * gq + i;   // D row = token, column n = head
        s[tt][i] = (n < NG && tok < t1 && tok <= last_n) ? acc[i] * inv_escale : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][i]);
    mx = reduce_rows(mx, OpMax{});
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = s[tt][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[tt][i] - m_new);
        lsum += p;
        if (n < NG) pl[(16 * tt + 4 * gq + i) * NG + n] = p;
      }
    lsum = reduce_rows(lsum, OpAdd{});
    l_run = l_run * alpha + lsum;
    if (gq == 0 && n < NG) L.alpha[n] = alpha;
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float a = L.alpha[j];
      o0[j] *= a;
      o1[j] *= a;
    }
#pragma unroll
    for (int u = 0; u < kRingChunk; ++u) {
      const float v0 = in_val<C>(vv[u] & 0xffffu), v1 = in_val<C>(vv[u] >> 16);
      const float* prow = pl + u * NG;
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const float p = prow[j];   // 0 for rows past t1
        o0[j] = fmaf(p, v0, o0[j]);
        o1[j] = fmaf(p, v1, o1[j]);
      }
    }
    wave_lds_fence();   // pl and alpha are rewritten by the next chunk
  }
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    float* dst = out_part + j * (D + 2);
    *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(o0[j], o1[j]);
  }
  if (gq == 0 && n < NG) {
    out_part[n * (D + 2) + D] = m_run;
    out_part[n * (D + 2) + D + 1] = l_run;
  }
}

// ---------------------------------------------------------------------------------
// Quantized blocks: a wave's stream of units.
// ---------------------------------------------------------------------------------

// A run of quantized blocks [begin, end) of (sequence b, kv head h).
struct Span {
  int b, h, begin, end;
};

// Record of block blk of span sp (blk is clamped into the span). The dense store
// keeps a pair's blocks contiguous; the paged store looks the page up (an
// out-of-range page reads page 0 and the block is masked out).
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

// The quantized units of a wave, from `first` on, taking the next unit from the
// queue counter: one continuous stream of sets in which the last set of a unit
// already prefetches the first set (and the query) of the next one, so a new
// unit costs no memory round trip. Each unit's partial state goes to its slot.
// `issue()` starts a claim on the queue (its raw answer, valid in lane 0),
// `claim(raw)` turns the answer into a unit index, `locate(u)` gives a
// quantized unit's span.
template <class C, class Locate, class Issue, class Claim>
__device__ __forceinline__ void quant_stream(const Geom& g, const WaveLds<C>& L, const uint8_t* __restrict__ blocks,
                                             const int32_t* __restrict__ table, const uint16_t* __restrict__ q,
                                             float qscale, int units, int first, Span first_span, int claimed,
                                             Locate locate, Issue issue, Claim claim, float* __restrict__ ws) {
  constexpr int NG = C::NG, D = C::D, NB = C::NB, TPB = C::TPB, NGR = C::NGR, KS_SET = C::KS_SET;
  constexpr int QW = NG * D / 128;   // query words per lane
  const int lane = threadIdx.x & 63, gq = lane >> 4, n = lane & 15;
  const int cbk = n / NG, chd = n % NG;   // column's block within the set, column's head
  const bool col_used = n < C::NCOL;

  // ---- register buffers for one set, refilled right after their last use ----
  // (The scale / zero sections are loaded once per set, a contiguous share per
  // lane, and staged in LDS at the top of the set: a per-lane copy of the
  // sections its column needs would hold them 8 to 16 times over, about 60
  // registers that the waves need for loads in flight.)
  Chunk<C::KSZ_LANE> ksz;       // this lane's share of the set's key scale / zero sections
  Chunk<C::KLANE> kc[NB][TPB];  // key code rows
  Chunk<C::VSZ_LANE> vsz;       // this lane's share of the value scale / zero sections
  Chunk<C::VLANE> vc[KS_SET];   // value code chunks

  // The paged store reads a set's page numbers once, ahead of its record
  // loads (raw values: an out-of-range page reads page 0 and its block is
  // masked out), where a set spans at most two blocks; with four, the extra
  // registers spill and each record load reads its own page number instead.
  // The dense store needs none. The table index is the same in every lane.
  constexpr bool EARLY = C::PAGED && NB <= 2;
  auto set_pages = [&](Span sp, int si, int (&pg)[NB]) {
    if constexpr (EARLY) {
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
        const int idx = __builtin_amdgcn_readfirstlane(sp.b * g.max_blocks + min(sp.begin + si * NB + bi, sp.end - 1));
        pg[bi] = table[idx];
      }
    }
  };
  auto pick_page = [&](const int (&pg)[NB], int bi) -> int {
    int page = pg[0];
#pragma unroll
    for (int k = 1; k < NB; ++k) page = bi == k ? pg[k] : page;
    return page;
  };
  auto page_in_range = [&](int page) -> bool { return page >= 0 && page < g.num_pages; };
  // record of block bi of set si of span sp
  auto set_rec = [&](Span sp, int si, int bi, const int (&pg)[NB]) -> const uint8_t* {
    if constexpr (!EARLY) {
      return span_rec<C>(g, blocks, table, sp, sp.begin + si * NB + bi);
    } else {
      int page = pick_page(pg, bi);
      page = page_in_range(page) ? page : 0;
      return blocks + ((size_t)page * g.Hkv + sp.h) * (size_t)C::REC;
    }
  };

  // loaders for set si of span sp, whose pages are pg
  auto load_ksz = [&](Span sp, int si, const int (&pg)[NB]) {
    const int byte = lane * C::KSZ_LANE;   // of the set's NB sections
    ksz = load_chunk<C::KSZ_LANE>(set_rec(sp, si, byte / C::KSEC, pg) + C::REC_KS + byte % C::KSEC);
  };
  auto load_kc = [&](Span sp, int si, const int (&pg)[NB]) {
    const int off = C::REC_KC + n * C::KROW + gq * C::KLANE;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      const uint8_t* p = set_rec(sp, si, bi, pg) + off;
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) kc[bi][tt] = load_chunk<C::KLANE>(p + 16 * tt * C::KROW);
    }
  };
  auto load_vsz = [&](Span sp, int si, const int (&pg)[NB]) {
    const int byte = lane * C::VSZ_LANE;
    vsz = load_chunk<C::VSZ_LANE>(set_rec(sp, si, byte / C::VSEC, pg) + C::REC_VS + byte % C::VSEC);
  };
  auto load_vc = [&](Span sp, int si, const int (&pg)[NB]) {
#pragma unroll
    for (int ks = 0; ks < KS_SET; ++ks) {
      const int tok = 32 * ks + 8 * gq;   // set-relative first token of this lane group's run
      // for G >= 32 the k-step lies in one block (wave-uniform); G = 16 spans two
      const int bi = C::G >= 32 ? (32 * ks) / C::G : tok / C::G;
      const uint8_t* p = set_rec(sp, si, bi, pg);
      const int g8 = (tok % C::G) / 8;
      vc[ks] = load_chunk<C::VLANE>(p + C::REC_VC + (g8 * 16 + n) * C::VLANE);
    }
  };
  // the query of span sp: raw words, then scaled into L.qs
  auto query_words = [&](Span sp, uint32_t (&w)[QW]) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(q + ((size_t)sp.b * g.Hq + (size_t)sp.h * NG) * D);
#pragma unroll
    for (int k = 0; k < QW; ++k) w[k] = src[lane + 64 * k];
  };
  // (with rotated keys the quantized blocks hold R(k) = H k / 8: their scores
  // take the query rotated the same way, H q' * 8 / D, since R(k) . H q' 8 / D = k . q')
  const bool rot_q = (g.rot & KVQ_ROTATE_KEYS) != 0;
  auto store_query = [&](const uint32_t (&w)[QW]) {
#pragma unroll
    for (int k = 0; k < QW; ++k) {   // word lane + 64k holds channels 2*lane, 2*lane+1 of row k
      float x0 = in_val<C>(w[k] & 0xffffu) * qscale, x1 = in_val<C>(w[k] >> 16) * qscale;
      if (rot_q) wht_row_pairs(x0, x1, 8.0f / D);
      *reinterpret_cast<float2*>(L.qs + k * C::QS + 2 * lane) = make_float2(x0, x1);
    }
  };

  // running state of the current unit: per lane for its column's head
  float m_ref, l_part, lam[NGR];
  f32x4 dpv[8];
  bool page_ok = true;   // the page of this lane's column block in the set being computed is in range (EARLY)

  // One set si of span cur; prefetches set nsi of span nsp into each register
  // buffer right after its last use (always a valid set, so the loads are never
  // under a branch and stay in flight across the loop).
  // Issue priority: the waves that share a SIMD do not progress alike (the
  // older one wins arbitration between equals), so each wave's base priority
  // alternates with its set count -- whichever of them is on an odd set goes
  // first -- and the score phase (below) sits two levels above both. A/B on one
  // box: Llama-3 GQA INT4 272 -> 263.5 us, paged 265 -> 260 us, 70B unchanged.
  int sets_done = 0;
  auto run_set = [&](Span cur, int si, Span nsp, int nsi) {
    const bool odd = (sets_done++ & 1) != 0;
    int pgn[NB];   // pages of the prefetched set, read before its first record load
    set_pages(nsp, nsi, pgn);
    const int my_b = cur.begin + si * NB + cbk;
    bool my_blk = col_used && my_b < cur.end && page_ok;
    if constexpr (C::PAGED && !EARLY)
      my_blk = my_blk && page_in_range(table[(size_t)cur.b * g.max_blocks + min(my_b, cur.end - 1)]);
    // ---- the set's scale / zero sections into LDS; the next set's are loaded at once ----
    store_chunk<C::KSZ_LANE>(L.ks + lane * C::KSZ_LANE, ksz);
    store_chunk<C::VSZ_LANE>(L.vs + lane * C::VSZ_LANE, vsz);
    load_ksz(nsp, nsi, pgn);
    load_vsz(nsp, nsi, pgn);
    wave_lds_fence();
    // ---- B operand: q~ = q' * s_K (hi/lo) and kappa = q' . z_K for the column ----
    uint4 bhi[4], blo[4];
    float kap = 0.f;
    {
      const float* qrow = L.qs + chd * C::QS + 32 * gq;
      const uint8_t* ksec = L.ks + cbk * C::KSEC + 2 * 32 * gq;   // channels 32gq.. of the column's block
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // channels 32gq + 8ks + (0..7) as fp16 pairs
        const uint4 sv = *reinterpret_cast<const uint4*>(ksec + 16 * ks);
        const uint4 zv = *reinterpret_cast<const uint4*>(ksec + 2 * D + 16 * ks);
        const float4 qa = *reinterpret_cast<const float4*>(qrow + 8 * ks);
        const float4 qb = *reinterpret_cast<const float4*>(qrow + 8 * ks + 4);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        const uint32_t s2[4] = {sv.x, sv.y, sv.z, sv.w}, z2[4] = {zv.x, zv.y, zv.z, zv.w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ze = (e & 1) ? hi_half_f16(z2[e >> 1]) : lo_half_f16(z2[e >> 1]);
          x[e] = (e & 1) ? mul_f16<true>(qv[e], s2[e >> 1]) : mul_f16<false>(qv[e], s2[e >> 1]);
          kap = fmaf(qv[e], ze, kap);
        }
        uint32_t hi[4], lo[4];
        // register r holds k positions 2r, 2r+1 = elements kperm(2r), kperm(2r+1)
        split_bf16(x[0], x[2], hi[0], lo[0]);
        split_bf16(x[1], x[3], hi[1], lo[1]);
        split_bf16(x[4], x[6], hi[2], lo[2]);
        split_bf16(x[5], x[7], hi[3], lo[3]);
        bhi[ks] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        blo[ks] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
      kap = reduce_rows(kap, OpAdd{});
    }

    // ---- scores: D[token][column] for every tile of every block of the set ----
    // (the wave issuing its score MFMAs goes first: the other wave of the
    // SIMD fills the matrix-core cycles with its vector work; measured 3%
    // faster on the INT4 layer, neutral elsewhere)
    if (odd) __builtin_amdgcn_s_setprio(3);
    else __builtin_amdgcn_s_setprio(2);
    float sc[TPB][4];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[tt][i] = -INFINITY;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      const bool mine = cbk == bi;
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        uint4 a[4];
        key_operands<C>(kc[bi][tt], a);
        f32x4 acc = {kap, kap, kap, kap};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          acc = mfma_bf16(a[ks], bhi[ks], acc);
          acc = mfma_bf16(a[ks], blo[ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[tt][i] = mine ? acc[i] : sc[tt][i];
      }
    }
    if (odd) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    load_kc(nsp, nsi, pgn);
    if (!my_blk) {
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[tt][i] = -INFINITY;
    }

    // ---- online softmax (log2 units), lazily rescaled ----
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[tt][i]);
    mx = reduce_head<NG>(mx, n, OpMax{});
    const bool grow = col_used && mx > m_ref + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int j = 0; j < NGR; ++j) lam[j] *= alpha;
      // row r of the P.V accumulators holds head r % NG (hi rows, then lo rows)
      if (gq == 0) L.alpha[n] = n < 2 * NG ? alpha : 1.f;
      wave_lds_fence();
      const float4 ar = *reinterpret_cast<const float4*>(L.alpha + 4 * gq);
      const float a4[4] = {ar.x, ar.y, ar.z, ar.w};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dpv[nt][i] *= a4[i];
    }
    // exp2(-inf - m) is 0 for a finite m, so masked scores need no test of
    // their own; m_ref is still -inf only while every score of the head was
    // masked (a set wholly on out-of-range pages), and then all of them are.
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float p[TPB][4];
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tt][i] = __builtin_amdgcn_exp2f(sc[tt][i] - m_use);
        psum += p[tt][i];
      }
    l_part += psum;

    // ---- p~ = p * s_V per value group, hi/lo, into the P.V A operand in LDS ----
    // (every used column writes, so the slots of a missing block hold zeros)
    if (col_used) {
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const int T = cbk * C::G + 16 * tt + 4 * gq;   // set-relative token of p[tt][0]
        const int ks = T >> 5, gp = (T >> 3) & 3, kvb = (T >> 2) & 1;
#pragma unroll
        for (int j = 0; j < NGR; ++j) {
          // value group j of the lane's 4 tokens
          const uint8_t* vsec = L.vs + cbk * C::VSEC + 2 * (j * C::G + 16 * tt + 4 * gq);
          const uint2 sv = *reinterpret_cast<const uint2*>(vsec);
          const uint2 zv = *reinterpret_cast<const uint2*>(vsec + C::VSEC / 2);
          const float z4[4] = {lo_half_f16(zv.x), hi_half_f16(zv.x), lo_half_f16(zv.y), hi_half_f16(zv.y)};
          const float x[4] = {mul_f16<false>(p[tt][0], sv.x), mul_f16<true>(p[tt][1], sv.x),
                              mul_f16<false>(p[tt][2], sv.y), mul_f16<true>(p[tt][3], sv.y)};
#pragma unroll
          for (int i = 0; i < 4; ++i) lam[j] = fmaf(p[tt][i], z4[i], lam[j]);
          uint32_t hi02, lo02, hi13, lo13;
          split_bf16(x[0], x[2], hi02, lo02);
          split_bf16(x[1], x[3], hi13, lo13);
          uint8_t* base = L.buf + (((ks * NGR + j) * 4 + gp) * 2 * NG) * 16 + kvb * 8;
          *reinterpret_cast<uint2*>(base + chd * 16) = make_uint2(hi02, hi13);
          *reinterpret_cast<uint2*>(base + (NG + chd) * 16) = make_uint2(lo02, lo13);
        }
      }
    }
    wave_lds_fence();

    // ---- P.V: D[head hi|lo][channel] += p~ . code ----
#pragma unroll
    for (int ks = 0; ks < KS_SET; ++ks) {
      uint4 av[NGR];
#pragma unroll
      for (int j = 0; j < NGR; ++j)
        av[j] = *reinterpret_cast<const uint4*>(
            n < 2 * NG ? L.buf + (((ks * NGR + j) * 4 + gq) * 2 * NG + n) * 16 : reinterpret_cast<uint8_t*>(L.zero16));
      uint4 bv[8];
      value_operands<C>(vc[ks], bv);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) dpv[nt] = mfma_bf16(av[(16 * nt) / C::GV], bv[nt], dpv[nt]);
    }
    load_vc(nsp, nsi, pgn);
    wave_lds_fence();
    if constexpr (EARLY) page_ok = page_in_range(pick_page(pgn, cbk));
  };

  // the unit's result: per head h', o = D[h'] + D[NG+h'] + lam(h', group)
  auto finish_unit = [&](float* __restrict__ out_part) {
    const float lsum = reduce_head<NG>(col_used ? l_part : 0.f, n, OpAdd{});
    float lm[NGR];
#pragma unroll
    for (int j = 0; j < NGR; ++j) lm[j] = reduce_head<NG>(col_used ? lam[j] : 0.f, n, OpAdd{});
    float* ol = reinterpret_cast<float*>(L.buf);   // [2NG][D]
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * gq + i;
        if (r < 2 * NG) ol[r * D + 16 * nt + n] = dpv[nt][i];
      }
    if (gq == 0 && n < NG) {
#pragma unroll
      for (int j = 0; j < NGR; ++j) L.lam[n * NGR + j] = lm[j];
      out_part[n * (D + 2) + D] = m_ref;
      out_part[n * (D + 2) + D + 1] = lsum;
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = lane + 64 * k;
        out_part[j * (D + 2) + c] = ol[j * D + c] + ol[(NG + j) * D + c] + L.lam[j * NGR + c / C::GV];
      }
    wave_lds_fence();   // L.buf and L.lam are rewritten by the next unit
  };

  int u = first;
  Span cur = first_span;
  {
    uint32_t w[QW];
    query_words(cur, w);
    store_query(w);
    wave_lds_fence();
  }
  {
    int pg0[NB];
    set_pages(cur, 0, pg0);
    load_ksz(cur, 0, pg0);
    load_kc(cur, 0, pg0);
    load_vsz(cur, 0, pg0);
    load_vc(cur, 0, pg0);
    if constexpr (EARLY) page_ok = page_in_range(pick_page(pg0, cbk));
  }
  while (true) {
    m_ref = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int j = 0; j < NGR; ++j) lam[j] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) dpv[nt] = {0.f, 0.f, 0.f, 0.f};
    const int nsets = (cur.end - cur.begin + NB - 1) / NB;
    for (int si = 0; si + 1 < nsets; ++si) run_set(cur, si, cur, si + 1);
    // last set: its prefetch is the next unit's first set (or, at the end of
    // the stream, this set again: cache hits)
    const int nu = claim(claimed);
    const bool more = nu < units;
    const Span nxt = more ? locate(nu) : cur;
    uint32_t qn[QW];
    query_words(nxt, qn);
    run_set(cur, nsets - 1, nxt, more ? 0 : nsets - 1);
    finish_unit(ws + (size_t)u * NG * (D + 2));
    if (!more) break;
    store_query(qn);
    wave_lds_fence();
    u = nu;
    cur = nxt;
    claimed = issue();
  }
}

// The query of (sequence b, kv head h), scaled to log2 units, into L.qs: one
// batch of independent loads, then the LDS writes.
template <class C>
__device__ __forceinline__ void load_query(const Geom& g, const WaveLds<C>& L, const uint16_t* __restrict__ q,
                                           float qscale, int b, int h) {
  constexpr int QW = C::NG * C::D / 128;   // 32-bit words per lane
  const int lane = threadIdx.x & 63;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(q + ((size_t)b * g.Hq + (size_t)h * C::NG) * C::D);
  uint32_t w[QW];
#pragma unroll
  for (int k = 0; k < QW; ++k) w[k] = src[lane + 64 * k];
#pragma unroll
  for (int k = 0; k < QW; ++k)   // word lane + 64k holds channels 2*lane, 2*lane+1 of row k
    *reinterpret_cast<float2*>(L.qs + k * C::QS + 2 * lane) =
        make_float2(in_val<C>(w[k] & 0xffffu) * qscale, in_val<C>(w[k] >> 16) * qscale);
  wave_lds_fence();
}

// ------------------------------------------------------------------------------------
// The kernel: persistent waves (C::WAVES_PER_SIMD per SIMD). The units are dealt to kQueues
// queues (unit u to queue u % kQueues) served by the workgroups with
// blockIdx.x % kQueues == queue -- with the usual round-robin placement of
// workgroups that is one queue per XCD, so the counters, each on its own cache
// line, are not all hit by every wave. A wave's first unit of its queue is
// fixed by its index; later ones come from the queue's counter in the state
// words. The last wave to finish re-arms the counters. 4 waves per workgroup
// share the unit plan in LDS and nothing else.
// ------------------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD))) void decode_fast_kernel(
    Geom g, const uint8_t* __restrict__ blocks, const int32_t* __restrict__ table,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring, int32_t* __restrict__ state,
    const uint16_t* __restrict__ q, float qscale, int max_blk, int* __restrict__ ws_plan, float* __restrict__ ws) {
  constexpr int NG = C::NG, D = C::D;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* plan = reinterpret_cast<int*>(smem);
  const int pints = plan_ints(g.B);
  const int pre_bytes = plan_lds_bytes(g.B);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t* wl = smem + pre_bytes + wave * C::LDS_WAVE;
  WaveLds<C> L;
  L.qs = reinterpret_cast<float*>(wl);
  L.buf = wl + C::LDS_Q;
  L.ks = L.buf + C::LDS_BUF;
  L.vs = L.ks + C::LDS_KS;
  L.alpha = reinterpret_cast<float*>(L.vs + C::LDS_VS);
  L.lam = L.alpha + 16;
  L.zero16 = reinterpret_cast<uint4*>(L.lam + NG * C::NGR);

  build_unit_plan(g, state, max_blk, C::NB, kRingChunk, plan, blockIdx.x == 0);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < pints; i += blockDim.x) ws_plan[i] = plan[i];
  if (lane == 0) *L.zero16 = make_uint4(0, 0, 0, 0);
  const int units = plan[kPlanUnits];
  // queue of this workgroup; gridDim.x is a multiple of kQueues
  const int queue = blockIdx.x % kQueues;
  const int qwaves = (int)(gridDim.x / kQueues) * kWaves;   // waves serving the queue
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

  // ring units come first in every queue; the claim for the next unit is in
  // flight while a unit runs
  int u = queue + kQueues * ((int)(blockIdx.x / kQueues) * kWaves + wave);
  int claimed = issue();
  while (u < units && u < plan[kPlanSec]) {
    const Span sp = span_of(u);
    load_query<C>(g, L, q, qscale, sp.b, sp.h);
    // ring tokens count after the sink; the last query token is the ring's last, S' - 1
    const int s_post = plan[plan_seq_off(g.B) + g.B + sp.b];
    ring_unit<C>(g, L, k_ring, v_ring, sp.b * g.Hkv + sp.h, sp.begin, sp.end, s_post - g.T,
                 ws + (size_t)u * NG * (D + 2));
    u = claim(claimed);
    claimed = issue();
  }
  if (u < units) quant_stream<C>(g, L, blocks, table, q, qscale, units, u, span_of(u), claimed, span_of, issue, claim, ws);
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
hipError_t launch_fast(const Geom& g, const kvq_cache& c, const void* q, float scale, int max_blk, void* ws,
                       hipStream_t s) {
  const size_t lds = (size_t)plan_lds_bytes(g.B) + (size_t)kWaves * C::LDS_WAVE;
  const int grid = persistent_grid(decode_fast_kernel<C>, lds);
  hipLaunchKernelGGL((decode_fast_kernel<C>), dim3(grid), dim3(256), lds, s, g,
                     static_cast<const uint8_t*>(c.blocks), c.block_table, static_cast<const uint16_t*>(c.k_ring),
                     static_cast<const uint16_t*>(c.v_ring), c.state, static_cast<const uint16_t*>(q),
                     scale * kLog2e, max_blk, static_cast<int*>(ws),
                     reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan_bytes(g.B)));
  return hipGetLastError();
}

}  // namespace fast
}  // namespace kvq
