// Append into the full-precision ring, and flush = quantize + pack the oldest
// complete blocks (gfx950).
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026": section "KIVI (2024)" -- keys are quantized per channel
//        and values per token, each group with its own min/max parameters, and
//        the most recent tokens stay in full precision; innovation 3 -- 16 INT2
//        or 8 INT4 codes per 32-bit word; innovation 4 -- a window of the most
//        recent tokens in full precision next to the low-bit history.
//   [P2] zubnet.ai survey, quantization family: keep every token, lower the bits.
//
// A block (G tokens of one kv head) is quantized either by one wave, straight
// from the ring in registers (quantize_wave.h: head_dim 128 and the key/value
// bits and groups the workloads use), or, for any other shape, by one
// workgroup: the tile is staged in LDS with 16-byte loads, column (key) and
// row-group (value) min/max are taken from LDS, codes go to LDS and the packed
// words are written with consecutive lanes on consecutive words.
//
// Three kernels share the block routines:
//   append_kernel        copies new rows into the ring (grid: pair x 64-token chunk);
//   flush_kernel         quantizes the complete blocks past the window of
//                        every pair: all (sequence, kv head, block) items in
//                        one list, each worker a contiguous, equal share;
//   append_flush_kernel  both, one workgroup per pair -- the decode-step path,
//                        one launch instead of two.
// Lengths live on the device: the workgroups read (Q_b, S_b), and the last of
// them to finish (an arrival counter in the state words) publishes the new
// values, so no host synchronisation is needed.
#include "common.h"
#include "quantize_wave.h"

namespace kvq {

namespace {

constexpr int kAppendTokensPerWG = 64;
constexpr int kThreads = 256;

// LDS of the block routine: raw tile [G][d] x 2 (16-bit), codes [G][d] x 2
// (8-bit); with the pre-rotation the tiles are fp32 instead.
__host__ __device__ inline size_t block_lds_bytes(int G, int d, bool rot = false) {
  return (size_t)(rot ? 10 : 6) * G * d;
}

// Walsh-Hadamard pre-rotation of every row of an fp32 tile [G][d] in LDS
// (patricehuetz.fr, "TurboQuant : les cinq innovations", innovation 1): for
// h = 1, 2, ..., d/2 each pair (i, i + h) of a row with bit h of i clear becomes
// (x_i + x_{i+h}, x_i - x_{i+h}), rounded to fp32; the last stage also takes the
// factor 1/8 (exact). Four threads per row, each holding CPT = d/4 consecutive
// channels in registers: the stages h < CPT run inside a thread, h = CPT and
// 2 CPT between the threads (partners lane ^ 1, lane ^ 2), so the tile is read
// and written once. All threads of the workgroup call it; ends with a barrier.
// One butterfly stage between the threads of a row: the partner (lane ^ M,
// through a quad permutation) holds the channels M * CPT away.
template <int CPT, int M>
__device__ __forceinline__ void rotate_cross(float (&x)[CPT], int q) {
  const bool upper = (q & M) != 0;
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    const float o = __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x[e]), M == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false));
    const float r = upper ? __fsub_rn(o, x[e]) : __fadd_rn(x[e], o);
    x[e] = M == 2 ? __fmul_rn(r, 0.125f) : r;
  }
}
template <int CPT>
__device__ __forceinline__ void rotate_rows_reg(float* f, int G) {
  constexpr int d = 4 * CPT;
  const int q = threadIdx.x & 3;
  for (int t0 = 0; t0 < G; t0 += kThreads / 4) {
    const int t = t0 + (int)(threadIdx.x >> 2);
    const bool live = t < G;   // the same for the four threads of a row
    float* row = f + (size_t)(live ? t : 0) * d + q * CPT;
    float x[CPT];
#pragma unroll
    for (int e = 0; e < CPT; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + e);
      x[e] = v.x;
      x[e + 1] = v.y;
      x[e + 2] = v.z;
      x[e + 3] = v.w;
    }
#pragma unroll
    for (int h = 1; h < CPT; h <<= 1)
#pragma unroll
      for (int j = 0; j < CPT / 2; ++j) {
        const int i = (j / h) * 2 * h + j % h;
        const float a = x[i], b = x[i + h];
        x[i] = __fadd_rn(a, b);
        x[i + h] = __fsub_rn(a, b);
      }
    rotate_cross<CPT, 1>(x, q);   // h = CPT: partner lane ^ 1
    rotate_cross<CPT, 2>(x, q);   // h = 2 CPT (the last stage): partner lane ^ 2
    if (live) {
#pragma unroll
      for (int e = 0; e < CPT; e += 4) *reinterpret_cast<float4*>(row + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
    }
  }
  __syncthreads();
}
__device__ __forceinline__ void rotate_rows(float* f, int G, int d) {
  __syncthreads();   // (the tile's writes before any thread reads another's)
  if (d == 128) rotate_rows_reg<32>(f, G);
  else rotate_rows_reg<16>(f, G);
}

// Quantize tokens blk*G .. blk*G+G-1 of ring `pair` into record `rec`; with ROT
// the rows of the sides g.rot names are rotated first (rotate_rows).
// Called by all kThreads threads of the workgroup; ends with a barrier.
template <bool BF16, bool ROT = false>
__device__ void quantize_block(const Geom& g, uint8_t* __restrict__ rec, const uint16_t* __restrict__ k_ring,
                               const uint16_t* __restrict__ v_ring, int pair, int blk, uint8_t* smem) {
  const int G = g.G, d = g.d, tid = threadIdx.x;
  uint16_t* s_k = reinterpret_cast<uint16_t*>(smem);   // [G][d] (without rotation)
  uint16_t* s_v = s_k + G * d;                         // [G][d]
  float* f_k = reinterpret_cast<float*>(smem);         // [G][d] (with rotation)
  float* f_v = f_k + G * d;
  uint8_t* s_kc = ROT ? reinterpret_cast<uint8_t*>(f_v + G * d) : reinterpret_cast<uint8_t*>(s_v + G * d);   // [G][d]
  uint8_t* s_vc = s_kc + G * d;                              // [d][G] value codes

  const int vec_per_tok = d / 8;
  for (int idx = tid; idx < G * vec_per_tok; idx += kThreads) {
    const int t = idx / vec_per_tok, v = idx % vec_per_tok;
    const int slot = (blk * G + t) % g.C;
    const size_t src = ((size_t)pair * g.C + slot) * d + (size_t)v * 8;
    const uint4 kw = *reinterpret_cast<const uint4*>(k_ring + src);
    const uint4 vw = *reinterpret_cast<const uint4*>(v_ring + src);
    if constexpr (ROT) {
      const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f_k[t * d + v * 8 + 2 * e] = in_to_f32<BF16>(kk[e] & 0xffffu);
        f_k[t * d + v * 8 + 2 * e + 1] = in_to_f32<BF16>(kk[e] >> 16);
        f_v[t * d + v * 8 + 2 * e] = in_to_f32<BF16>(vv[e] & 0xffffu);
        f_v[t * d + v * 8 + 2 * e + 1] = in_to_f32<BF16>(vv[e] >> 16);
      }
    } else {
      *reinterpret_cast<uint4*>(&s_k[t * d + v * 8]) = kw;
      *reinterpret_cast<uint4*>(&s_v[t * d + v * 8]) = vw;
    }
  }
  __syncthreads();
  if constexpr (ROT) {
    if (g.rot & KVQ_ROTATE_KEYS) rotate_rows(f_k, G, d);
    if (g.rot & KVQ_ROTATE_VALUES) rotate_rows(f_v, G, d);
  }
  // element (t, c) of the key / value tile, as fp32
  auto kx = [&](int t, int c) -> float { return ROT ? f_k[t * d + c] : in_to_f32<BF16>(s_k[t * d + c]); };
  auto vx = [&](int t, int c) -> float { return ROT ? f_v[t * d + c] : in_to_f32<BF16>(s_v[t * d + c]); };

  uint16_t* ks = reinterpret_cast<uint16_t*>(rec + g.rec_ks);
  uint16_t* kz = reinterpret_cast<uint16_t*>(rec + g.rec_kz);
  uint16_t* vs = reinterpret_cast<uint16_t*>(rec + g.rec_vs);
  uint16_t* vz = reinterpret_cast<uint16_t*>(rec + g.rec_vz);

  // keys: one group per channel over the G tokens
  for (int c = tid; c < d; c += kThreads) {
    float mn = kx(0, c), mx = mn;
    for (int t = 1; t < G; ++t) {
      const float x = kx(t, c);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const GroupParams p = group_params(mn, mx, g.kb);
    ks[c] = p.s16;
    kz[c] = p.z16;
    for (int t = 0; t < G; ++t) s_kc[t * d + c] = (uint8_t)group_code(kx(t, c), p, g.kb);
  }
  // values: one group per (token, G_V consecutive channels)
  const int ngr = d / g.GV;
  for (int idx = tid; idx < G * ngr; idx += kThreads) {
    const int t = idx / ngr, j = idx % ngr;
    const int c0 = j * g.GV;
    float mn = vx(t, c0), mx = mn;
    for (int c = 1; c < g.GV; ++c) {
      const float x = vx(t, c0 + c);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const GroupParams p = group_params(mn, mx, g.vb);
    vs[j * G + t] = p.s16;
    vz[j * G + t] = p.z16;
    for (int c = 0; c < g.GV; ++c)
      s_vc[(c0 + c) * G + t] = (uint8_t)group_code(vx(t, c0 + c), p, g.vb);
  }
  __syncthreads();

  // keys: word w of token t holds channels w*P .. w*P+P-1, LSB first
  uint32_t* kc = reinterpret_cast<uint32_t*>(rec + g.rec_kc);
  const int kP = 32 / g.kb;
  for (int idx = tid; idx < G * g.k_words; idx += kThreads) {
    const int t = idx / g.k_words, w = idx % g.k_words;
    const uint8_t* src = &s_kc[t * d + w * kP];
    uint32_t word = 0;
    for (int i = 0; i < kP; ++i) word |= (uint32_t)src[i] << (i * g.kb);
    kc[idx] = word;
  }
  // values in 8-token chunks: code (t, c) at stream position
  // ((t/8 * 16 + c%16) * (d/16) + c/16) * 8 + t%8, LSB first
  uint32_t* vc = reinterpret_cast<uint32_t*>(rec + g.rec_vc);
  const int vP = 32 / g.vb;
  const int nt_count = d / 16;
  for (int idx = tid; idx < G * d * g.vb / 32; idx += kThreads) {
    uint32_t word = 0;
    for (int i = 0; i < vP; ++i) {
      const int pos = idx * vP + i;
      const int rest = pos >> 3;
      const int nt = rest % nt_count, rest2 = rest / nt_count;
      const int t = (rest2 >> 4) * 8 + (pos & 7);
      const int c = nt * 16 + (rest2 & 15);
      word |= (uint32_t)s_vc[c * G + t] << (i * g.vb);
    }
    vc[idx] = word;
  }
  __syncthreads();
}

// Copy tokens i in [t_lo, t_hi) of pair `pair` from the new rows into the ring,
// new row i at ring position base + i (>= 0 for every copied row; positions
// count the tokens after the sink), 16-byte vectors.
__device__ __forceinline__ void copy_to_ring(const Geom& g, const uint16_t* __restrict__ k_new,
                                             const uint16_t* __restrict__ v_new, int n_max, uint16_t* k_ring,
                                             uint16_t* v_ring, int pair, int base, int t_lo, int t_hi) {
  const int vec_per_tok = g.d / 8;
  for (int idx = threadIdx.x; idx < (t_hi - t_lo) * vec_per_tok; idx += kThreads) {
    const int i = t_lo + idx / vec_per_tok;
    const int v = idx % vec_per_tok;
    const int slot = (base + i) % g.C;
    const size_t src = ((size_t)pair * n_max + i) * g.d + (size_t)v * 8;
    const size_t dst = ((size_t)pair * g.C + slot) * g.d + (size_t)v * 8;
    *reinterpret_cast<uint4*>(k_ring + dst) = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(v_ring + dst) = *reinterpret_cast<const uint4*>(v_new + src);
  }
}

// Copy tokens i in [t_lo, t_hi) of pair `pair` from the new rows into sink
// rows S + i (all below P).
__device__ __forceinline__ void copy_to_sink(const Geom& g, const uint16_t* __restrict__ k_new,
                                             const uint16_t* __restrict__ v_new, int n_max, uint16_t* k_sink,
                                             uint16_t* v_sink, int pair, int S, int t_lo, int t_hi) {
  const int vec_per_tok = g.d / 8;
  for (int idx = threadIdx.x; idx < (t_hi - t_lo) * vec_per_tok; idx += kThreads) {
    const int i = t_lo + idx / vec_per_tok;
    const int v = idx % vec_per_tok;
    const size_t src = ((size_t)pair * n_max + i) * g.d + (size_t)v * 8;
    const size_t dst = ((size_t)pair * g.P + S + i) * g.d + (size_t)v * 8;
    *reinterpret_cast<uint4*>(k_sink + dst) = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(v_sink + dst) = *reinterpret_cast<const uint4*>(v_new + src);
  }
}

// Where n new tokens of a sequence of S tokens go: rows [0, n_sink) to sink
// rows S.., the others to the ring (row i at ring position S + i - P); `post`
// is the sequence's token count after the sink once they are in.
struct AppendSplit {
  int n_sink, post;
};
__device__ __forceinline__ AppendSplit append_split(const Geom& g, int S, int n) {
  AppendSplit a;
  a.n_sink = min(max(g.P - S, 0), n);
  a.post = max(S + n - g.P, 0);
  return a;
}

// Tokens after the sink of a sequence of S tokens.
__device__ __forceinline__ int post_sink(const Geom& g, int S) { return max(S - g.P, 0); }

// Blocks a flush takes for a sequence with Q quantized of S tokens after the
// sink, and how many of those fit under max_blocks.
struct FlushPlan {
  int nfl, nok;
};
__device__ __forceinline__ FlushPlan flush_plan(const Geom& g, int Q, int S) {
  const int r = S - Q;
  FlushPlan f;
  f.nfl = (r >= g.R + g.G) ? (r - g.R) / g.G : 0;
  f.nok = min(f.nfl, max(g.max_blocks - Q / g.G, 0));
  return f;
}

__global__ __launch_bounds__(kThreads) void append_kernel(Geom g, const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new,
                                                          const int32_t* __restrict__ n_new, int n_max,
                                                          uint16_t* __restrict__ k_ring,
                                                          uint16_t* __restrict__ v_ring,
                                                          uint16_t* __restrict__ k_sink,
                                                          uint16_t* __restrict__ v_sink, int32_t* __restrict__ state) {
  const int pair = blockIdx.x;
  const int b = pair / g.Hkv;
  __shared__ int s_S, s_n, s_ok;
  if (threadIdx.x == 0) {
    const int Q = state[4 * b + kStateQ];
    const int S = state[4 * b + kStateS];
    const int n = n_new ? n_new[b] : n_max;
    const bool count_ok = n >= 0 && n <= n_max;
    s_S = S;
    s_n = n;
    s_ok = count_ok ? (append_split(g, S, n).post - Q <= g.C ? 1 : 2) : 0;   // 1 ok, 2 ring full, 0 bad count
  }
  __syncthreads();
  if (s_ok == 1) {
    const int t0 = blockIdx.y * kAppendTokensPerWG, t1 = min(t0 + kAppendTokensPerWG, s_n);
    const int ns = append_split(g, s_S, s_n).n_sink;
    copy_to_sink(g, k_new, v_new, n_max, k_sink, v_sink, pair, s_S, t0, min(t1, ns));
    copy_to_ring(g, k_new, v_new, n_max, k_ring, v_ring, pair, s_S - g.P, max(t0, ns), t1);
  }
  __syncthreads();
  if (threadIdx.x == 0 && last_arrival(&state[4 * b + kStateAppendCnt], g.Hkv * gridDim.y)) {
    if (s_ok == 1)
      state[4 * b + kStateS] = s_S + s_n;
    else
      atomicOr(&state[4 * g.B], s_ok == 0 ? KVQ_DEV_BAD_COUNT : KVQ_DEV_RESIDUAL_FULL);
  }
}

// FP8 record of block `blk` of `pair` from its ring rows ([P1] ai-automate.fr,
// section on Minima-KV: recent pages kept in FP8). Formula F8 per token row
// x: s = fp16(max|x| / 448) (IEEE divide, then round to nearest even);
// s == 0 -> codes 0; else code_c = e4m3(clamp(x_c / s, -448, 448)), the
// packed conversion rounding to nearest even. One wave: tokens t0, t0 + dt, ...
template <bool BF16>
__device__ inline void write_fp8_rows(const Geom& g, uint8_t* __restrict__ rec8, const uint16_t* __restrict__ k_ring,
                                      const uint16_t* __restrict__ v_ring, int pair, int blk, int t0, int dt) {
  const int lane = threadIdx.x & 63;
  const bool two = g.d == 128;   // channels per lane: 2 (d = 128) or 1 (d = 64)
  for (int t = t0; t < g.G; t += dt) {
    const size_t row = ((size_t)pair * g.C + (size_t)((blk * g.G + t) % g.C)) * g.d;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = (kv == 0 ? k_ring : v_ring) + row;
      float x0, x1 = 0.f;
      if (two) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src + 2 * lane);
        x0 = in_to_f32<BF16>(w & 0xffffu);
        x1 = in_to_f32<BF16>(w >> 16);
      } else {
        x0 = in_to_f32<BF16>(src[lane]);
      }
      const float a = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(a, 448.0f));
      const float s = f16_to_f32(s16);
      float y0 = 0.f, y1 = 0.f;
      if (s != 0.f) {   // wave-uniform
        y0 = fminf(fmaxf(__fdiv_rn(x0, s), -448.0f), 448.0f);
        y1 = fminf(fmaxf(__fdiv_rn(x1, s), -448.0f), 448.0f);
      }
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      uint8_t* codes = rec8 + (kv == 0 ? 0 : (size_t)g.G * g.d + 2 * g.G) + (size_t)t * g.d;
      if (two)
        *reinterpret_cast<uint16_t*>(codes + 2 * lane) = (uint16_t)pk;
      else
        codes[lane] = (uint8_t)pk;
      if (lane == 0)
        *reinterpret_cast<uint16_t*>(rec8 + (kv == 0 ? (size_t)g.G * g.d : 2 * (size_t)g.G * g.d + 2 * g.G) +
                                     2 * t) = s16;
    }
  }
}

// The two block routines behind one interface: Workers blocks at a time per
// workgroup (the wave routine: one per wave; the workgroup routine: one).
// fp8() writes the block's FP8 record (every wave of a workgroup worker
// takes a share of its tokens).
// The workgroup routine; ROT: with the Walsh-Hadamard pre-rotation of the sides
// g.rot names (every rotated configuration takes this routine).
template <bool BF16, bool ROT = false>
struct WgBlock {
  static constexpr int kWorkers = 1;
  __device__ static void fp8(const Geom& g, uint8_t* rec8, const uint16_t* kr, const uint16_t* vr, int pair,
                             int blk) {
    write_fp8_rows<BF16>(g, rec8, kr, vr, pair, blk, (int)(threadIdx.x >> 6), kThreads / 64);
  }
  __host__ __device__ static size_t lds(const Geom& g) { return block_lds_bytes(g.G, g.d, ROT); }
  __device__ static void run(const Geom& g, uint8_t* rec, const uint16_t* kr, const uint16_t* vr, int pair,
                             int blk, uint8_t* smem) {
    quantize_block<BF16, ROT>(g, rec, kr, vr, pair, blk, smem);
  }
};
template <class Q, bool ROT = false>
struct WaveBlock {
  static constexpr int kWorkers = kThreads / 64;
  __device__ static void fp8(const Geom& g, uint8_t* rec8, const uint16_t* kr, const uint16_t* vr, int pair,
                             int blk) {
    write_fp8_rows<Q::BF16>(g, rec8, kr, vr, pair, blk, 0, 1);
  }
  __host__ __device__ static size_t lds(const Geom&) { return 0; }
  __device__ static void run(const Geom& g, uint8_t* rec, const uint16_t* kr, const uint16_t* vr, int pair,
                             int blk, uint8_t*) {
    qwave::quantize_block<Q, ROT>(g, rec, kr, vr, pair, blk);
  }
};

// Blocks k0, k0 + stride, ... below nok of pair (b, h), by this thread's
// worker (wave or workgroup); `bad` is set for a missing page. Blocks that end
// up among the W most recent (the FP8 tier) also get their FP8 record, at
// slot blk mod W of the pair (blocks older than that never share a slot with
// them).
template <class P>
__device__ __forceinline__ void flush_blocks(const Geom& g, uint8_t* blocks, const int32_t* table, uint8_t* fp8,
                                             const uint16_t* k_ring, const uint16_t* v_ring, int pair, int b, int h,
                                             int Q, int k0, int stride, int nok, int* bad, uint8_t* smem) {
  const int worker = P::kWorkers > 1 ? (int)(threadIdx.x / (kThreads / P::kWorkers)) : 0;
  const int fp8_from = Q / g.G + nok - g.W;   // first block of the tier after this flush
  for (int k = k0 * P::kWorkers + worker; k < nok; k += stride * P::kWorkers) {
    const int blk = Q / g.G + k;
    uint8_t* rec = const_cast<uint8_t*>(block_record(g, blocks, table, b, h, blk));
    if (rec == nullptr) {
      if (threadIdx.x % (kThreads / P::kWorkers) == 0) *bad = 1;
      continue;
    }
    P::run(g, rec, k_ring, v_ring, pair, blk, smem);
    if (g.W > 0 && blk >= fp8_from) P::fp8(g, fp8 + ((size_t)pair * g.W + blk % g.W) * g.rec8, k_ring, v_ring, pair, blk);
  }
}

// Bulk flush. Every workgroup reads the lengths of all sequences and lays out
// one list of items, (sequence b, kv head h, block k) with k fastest, from the
// exclusive prefix of the sequences' flushable block counts (in LDS after the
// block routine's tile). Worker w of W takes items w, w + W, w + 2W, ...: a
// ragged batch is balanced over the whole grid whatever its lengths, and the
// workers in flight at one time stream consecutive blocks (contiguous ranges
// per worker put them a power-of-two stride apart, which measured 20% slower
// on the Llama-2 layer). The last workgroup to finish publishes every sequence's
// new Q_b (arrival counter: sequence 0's flush counter word).
template <class P>
__global__ __launch_bounds__(kThreads) void flush_kernel(Geom g, uint8_t* __restrict__ blocks,
                                                         const int32_t* __restrict__ table, uint8_t* __restrict__ fp8,
                                                         const uint16_t* __restrict__ k_ring,
                                                         const uint16_t* __restrict__ v_ring,
                                                         int32_t* __restrict__ state) {
  extern __shared__ uint8_t smem[];
  int* s_pre = reinterpret_cast<int*>(smem + P::lds(g));   // [B + 1] exclusive prefix of nok_b
  int* s_Q = s_pre + g.B + 1;                              // [B] Q_b as read at the start
  __shared__ int s_wave[kThreads / 64];
  __shared__ int s_bad, s_full, s_last;
  const int B = g.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // this thread's run of sequences: one round of state loads, nok_b into
  // s_pre, then a block-wide exclusive scan turns them into the prefix
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = min((int)threadIdx.x * per, B), b1 = min(b0 + per, B);
  if (threadIdx.x == 0) {
    s_bad = 0;
    s_full = 0;
  }
  int run = 0, full = 0;
  for (int b = b0; b < b1; ++b) {
    const int Q = state[4 * b + kStateQ];
    const FlushPlan f = flush_plan(g, Q, post_sink(g, state[4 * b + kStateS]));
    s_Q[b] = Q;
    s_pre[b] = f.nok;
    run += f.nok;
    full |= f.nok < f.nfl;
  }
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (full) atomicOr(&s_full, 1);
  int acc = incl - run;
  for (int w = 0; w < wave; ++w) acc += s_wave[w];
  for (int b = b0; b < b1; ++b) {
    const int nok = s_pre[b];
    s_pre[b] = acc;
    acc += nok;
  }
  if (threadIdx.x == kThreads - 1) s_pre[B] = acc;
  __syncthreads();

  // (the item bookkeeping is uniform over a worker: scalar registers, so
  // that the block routine keeps every vector register it had)
  const long long total = (long long)__builtin_amdgcn_readfirstlane(s_pre[B]) * g.Hkv;
  const int worker =
      P::kWorkers > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x / (kThreads / P::kWorkers))) : 0;
  const long long nworkers = (long long)gridDim.x * P::kWorkers;
  for (long long i = (long long)blockIdx.x * P::kWorkers + worker; i < total; i += nworkers) {
    // the item's sequence: the largest b with pre[b] * Hkv <= i (it has blocks)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)__builtin_amdgcn_readfirstlane(s_pre[mid]) * g.Hkv <= i) lo = mid;
      else hi = mid - 1;
    }
    const int b = lo;
    const int pre_b = __builtin_amdgcn_readfirstlane(s_pre[b]);
    const int nok = __builtin_amdgcn_readfirstlane(s_pre[b + 1]) - pre_b;
    const int r = (int)(i - (long long)pre_b * g.Hkv);   // < nok * Hkv
    const int h = r / nok, k = r % nok;
    const int Q = __builtin_amdgcn_readfirstlane(s_Q[b]);
    const int blk = Q / g.G + k;
    const int pair = b * g.Hkv + h;
    uint8_t* rec = const_cast<uint8_t*>(block_record(g, blocks, table, b, h, blk));
    if (rec == nullptr) {
      if (threadIdx.x % (kThreads / P::kWorkers) == 0) s_bad = 1;
      continue;
    }
    P::run(g, rec, k_ring, v_ring, pair, blk, smem);
    // blocks that end up among the W most recent (the FP8 tier) also get
    // their FP8 record, at slot blk mod W of the pair
    if (g.W > 0 && blk >= Q / g.G + nok - g.W)
      P::fp8(g, fp8 + ((size_t)pair * g.W + blk % g.W) * g.rec8, k_ring, v_ring, pair, blk);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_bad) atomicOr(&state[4 * B], KVQ_DEV_BAD_PAGE);
    s_last = last_arrival(&state[kStateFlushCnt], gridDim.x);
  }
  __syncthreads();
  if (s_last) {   // every workgroup has finished: publish the new lengths
    for (int b = b0; b < b1; ++b) state[4 * b + kStateQ] = s_Q[b] + (s_pre[b + 1] - s_pre[b]) * g.G;
    if (threadIdx.x == 0 && s_full) atomicOr(&state[4 * B], KVQ_DEV_BLOCKS_FULL);
  }
}

// Append then flush, one workgroup per (sequence, kv head): the decode-step
// path. Every workgroup of a sequence derives the same new lengths from the
// same (Q_b, S_b, n_b); the last to finish publishes them.
template <class P>
__global__ __launch_bounds__(kThreads) void append_flush_kernel(Geom g, const uint16_t* __restrict__ k_new,
                                                                const uint16_t* __restrict__ v_new,
                                                                const int32_t* __restrict__ n_new, int n_max,
                                                                uint8_t* __restrict__ blocks,
                                                                const int32_t* __restrict__ table,
                                                                uint8_t* __restrict__ fp8,
                                                                uint16_t* __restrict__ k_ring,
                                                                uint16_t* __restrict__ v_ring,
                                                                uint16_t* __restrict__ k_sink,
                                                                uint16_t* __restrict__ v_sink,
                                                                int32_t* __restrict__ state) {
  extern __shared__ uint8_t smem[];
  const int pair = blockIdx.x;
  const int b = pair / g.Hkv, h = pair % g.Hkv;
  __shared__ int s_Q, s_S, s_n, s_ok, s_nfl, s_nok, s_bad;
  // the first kThreads 16-byte vectors of the new rows are loaded before the
  // lengths (a decode step's whole append): the two round trips overlap
  const int vec_per_tok = g.d / 8;
  uint4 pk = make_uint4(0, 0, 0, 0), pv = pk;
  if ((int)threadIdx.x < n_max * vec_per_tok) {
    const size_t src = (size_t)pair * n_max * g.d + (size_t)threadIdx.x * 8;
    pk = *reinterpret_cast<const uint4*>(k_new + src);
    pv = *reinterpret_cast<const uint4*>(v_new + src);
  }
  if (threadIdx.x == 0) {
    const int Q = state[4 * b + kStateQ];
    const int S = state[4 * b + kStateS];
    const int n = n_new ? n_new[b] : n_max;
    const bool count_ok = n >= 0 && n <= n_max;
    const int post = count_ok ? append_split(g, S, n).post : 0;
    const int ok = count_ok ? (post - Q <= g.C ? 1 : 2) : 0;
    const FlushPlan f = flush_plan(g, Q, ok == 1 ? post : post_sink(g, S));
    s_Q = Q;
    s_S = S;
    s_n = n;
    s_ok = ok;
    s_nfl = f.nfl;
    s_nok = f.nok;
    s_bad = 0;
  }
  __syncthreads();
  if (s_ok == 1) {   // rows [0, ns) to sink rows S.., the others to ring position S - P + i
    const int ns = append_split(g, s_S, s_n).n_sink;
    for (int idx = threadIdx.x; idx < s_n * vec_per_tok; idx += kThreads) {
      const int i = idx / vec_per_tok, v = idx % vec_per_tok;
      uint4 kw = pk, vw = pv;
      if (idx >= kThreads) {
        const size_t src = ((size_t)pair * n_max + i) * g.d + (size_t)v * 8;
        kw = *reinterpret_cast<const uint4*>(k_new + src);
        vw = *reinterpret_cast<const uint4*>(v_new + src);
      }
      size_t dst;
      uint16_t *kd, *vd;
      if (i < ns) {
        dst = ((size_t)pair * g.P + s_S + i) * g.d + (size_t)v * 8;
        kd = k_sink;
        vd = v_sink;
      } else {
        dst = ((size_t)pair * g.C + (s_S - g.P + i) % g.C) * g.d + (size_t)v * 8;
        kd = k_ring;
        vd = v_ring;
      }
      *reinterpret_cast<uint4*>(kd + dst) = kw;
      *reinterpret_cast<uint4*>(vd + dst) = vw;
    }
  }
  // the block routine reads the ring through plain loads: make this
  // workgroup's ring writes visible to all of its threads first
  __threadfence_block();
  __syncthreads();
  flush_blocks<P>(g, blocks, table, fp8, k_ring, v_ring, pair, b, h, s_Q, 0, 1, s_nok, &s_bad, smem);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_bad) atomicOr(&state[4 * g.B], KVQ_DEV_BAD_PAGE);
    if (s_ok != 1) atomicOr(&state[4 * g.B], s_ok == 0 ? KVQ_DEV_BAD_COUNT : KVQ_DEV_RESIDUAL_FULL);
    if (last_arrival(&state[4 * b + kStateAppendCnt], g.Hkv)) {
      if (s_ok == 1) state[4 * b + kStateS] = s_S + s_n;
      state[4 * b + kStateQ] = s_Q + s_nok * g.G;
      if (s_nok < s_nfl) atomicOr(&state[4 * g.B], KVQ_DEV_BLOCKS_FULL);
    }
  }
}

}  // namespace

hipError_t launch_append(const Geom& g, const kvq_cache& c, const void* k_new, const void* v_new,
                         const int32_t* n_new, int n_max, hipStream_t s) {
  const int chunks = (n_max + kAppendTokensPerWG - 1) / kAppendTokensPerWG;
  dim3 grid(g.B * g.Hkv, chunks > 0 ? chunks : 1);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kThreads), 0, s, g,
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), n_new,
                     n_max, static_cast<uint16_t*>(c.k_ring), static_cast<uint16_t*>(c.v_ring),
                     static_cast<uint16_t*>(c.k_sink), static_cast<uint16_t*>(c.v_sink), c.state);
  return hipGetLastError();
}

namespace {

template <class P>
hipError_t launch_flush_p(const Geom& g, const kvq_cache& c, hipStream_t s) {
  // A ring of C slots holds at most (C - R) / G complete blocks past the
  // window: enough workers for that many blocks of every pair, at most the
  // workgroups that stay resident at once (each pays the length prologue once;
  // a decode-sized flush stays small).
  const long long max_items = (long long)std::max((g.C - g.R) / g.G, 1) * g.B * g.Hkv;
  const int per_wg = P::kWorkers;
  const size_t lds = P::lds(g) + (size_t)(2 * g.B + 1) * sizeof(int);
  const int resident = persistent_grid(flush_kernel<P>, lds);
  const int wgs = (int)std::max(1LL, std::min((max_items + per_wg - 1) / per_wg, (long long)resident));
  hipLaunchKernelGGL((flush_kernel<P>), dim3(wgs), dim3(kThreads), lds, s, g,
                     static_cast<uint8_t*>(c.blocks), c.block_table, static_cast<uint8_t*>(c.fp8),
                     static_cast<const uint16_t*>(c.k_ring),
                     static_cast<const uint16_t*>(c.v_ring), c.state);
  return hipGetLastError();
}

template <class P>
hipError_t launch_append_flush_p(const Geom& g, const kvq_cache& c, const void* k_new, const void* v_new,
                                 const int32_t* n_new, int n_max, hipStream_t s) {
  hipLaunchKernelGGL((append_flush_kernel<P>), dim3(g.B * g.Hkv), dim3(kThreads), P::lds(g), s, g,
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), n_new, n_max,
                     static_cast<uint8_t*>(c.blocks), c.block_table, static_cast<uint8_t*>(c.fp8),
                     static_cast<uint16_t*>(c.k_ring),
                     static_cast<uint16_t*>(c.v_ring), static_cast<uint16_t*>(c.k_sink),
                     static_cast<uint16_t*>(c.v_sink), c.state);
  return hipGetLastError();
}

using FlushFn = hipError_t (*)(const Geom&, const kvq_cache&, hipStream_t);
using AppendFlushFn = hipError_t (*)(const Geom&, const kvq_cache&, const void*, const void*, const int32_t*, int,
                                     hipStream_t);
struct QuantEntry {
  int G, kb, vb, GV, dtype;
  FlushFn flush, flush_rot;                      // plain and pre-rotated rows
  AppendFlushFn append_flush, append_flush_rot;
};
template <bool BF16, int G, int KB, int VB, int GV>
QuantEntry wave_entry() {
  using Q = qwave::Cfg<BF16, G, KB, VB, GV>;
  using P = WaveBlock<Q>;
  using PR = WaveBlock<Q, true>;
  return QuantEntry{G, KB, VB, GV, BF16 ? KVQ_BF16 : KVQ_F16, &launch_flush_p<P>, &launch_flush_p<PR>,
                    &launch_append_flush_p<P>, &launch_append_flush_p<PR>};
}
// head_dim 128: the key/value bits and groups of the workloads, fp16 and bf16
#define KVQ_WAVE(G, KB, VB, GV) wave_entry<false, G, KB, VB, GV>(), wave_entry<true, G, KB, VB, GV>()
const QuantEntry* find_wave(const Geom& g) {
  static const QuantEntry kTable[] = {
      KVQ_WAVE(32, 2, 2, 32), KVQ_WAVE(32, 4, 4, 32), KVQ_WAVE(64, 2, 2, 64), KVQ_WAVE(16, 4, 2, 32),
  };
  if (g.d != 128) return nullptr;
  for (const QuantEntry& e : kTable)
    if (e.G == g.G && e.kb == g.kb && e.vb == g.vb && e.GV == g.GV && e.dtype == g.dtype) return &e;
  return nullptr;
}
#undef KVQ_WAVE

}  // namespace

hipError_t launch_flush(const Geom& g, const kvq_cache& c, hipStream_t s) {
  const QuantEntry* e = find_wave(g);
  if (g.rot != 0) {
    if (e) return e->flush_rot(g, c, s);
    return g.dtype == KVQ_BF16 ? launch_flush_p<WgBlock<true, true>>(g, c, s)
                               : launch_flush_p<WgBlock<false, true>>(g, c, s);
  }
  if (e) return e->flush(g, c, s);
  return g.dtype == KVQ_BF16 ? launch_flush_p<WgBlock<true>>(g, c, s) : launch_flush_p<WgBlock<false>>(g, c, s);
}

hipError_t launch_append_flush(const Geom& g, const kvq_cache& c, const void* k_new, const void* v_new,
                               const int32_t* n_new, int n_max, hipStream_t s) {
  if (n_max > kAppendTokensPerWG) {
    // a large append keeps the parallel copy and the parallel flush
    hipError_t e = launch_append(g, c, k_new, v_new, n_new, n_max, s);
    return e != hipSuccess ? e : launch_flush(g, c, s);
  }
  const QuantEntry* e = find_wave(g);
  if (g.rot != 0) {
    if (e) return e->append_flush_rot(g, c, k_new, v_new, n_new, n_max, s);
    return g.dtype == KVQ_BF16 ? launch_append_flush_p<WgBlock<true, true>>(g, c, k_new, v_new, n_new, n_max, s)
                               : launch_append_flush_p<WgBlock<false, true>>(g, c, k_new, v_new, n_new, n_max, s);
  }
  if (e) return e->append_flush(g, c, k_new, v_new, n_new, n_max, s);
  return g.dtype == KVQ_BF16 ? launch_append_flush_p<WgBlock<true>>(g, c, k_new, v_new, n_new, n_max, s)
                             : launch_append_flush_p<WgBlock<false>>(g, c, k_new, v_new, n_new, n_max, s);
}

}  // namespace kvq
