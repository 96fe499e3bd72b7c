// Shared device/host definitions of libkvq (gfx950).
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026" -- section "KIVI (2024)" (per-channel keys, per-token
//        values, own min/max parameters, full-precision recent tokens),
//        innovation 3 (dense INT2/INT4 packing into 32-bit words, 16-token
//        blocks for paged attention), innovation 4 (residual window).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kvq.h"

namespace kvq {

// Everything a kernel needs to know about one cache layer. Plain data, passed
// by value as a kernel argument.
struct Geom {
  int B, Hq, Hkv, d, ng;
  int kb, vb, G, GV, R, C;
  int max_blocks, num_pages, dtype;
  // record section offsets (bytes) and sizes
  int rec_kc, rec_ks, rec_kz, rec_vc, rec_vs, rec_vz, rec_bytes;
  int k_words;   // uint32 words of K codes per token: d*kb/32
  int v_words;   // uint32 words of V codes per channel: G*vb/32
  int P;         // sink: leading tokens of a sequence kept in full precision
  int T;         // queries per (sequence, query head): the T newest tokens, causal; Hq and ng count them
  int W;         // FP8 tier: most recent quantized blocks also kept (and read) as FP8 records
  int rec8;      // bytes of one FP8 record: K codes [G][d], K scales [G], V codes [G][d], V scales [G]
  int rot;       // Walsh-Hadamard pre-rotation: KVQ_ROTATE_KEYS | KVQ_ROTATE_VALUES bits
};

// Query rows per kv head one launch serves (n_g times T).
constexpr int kNgMax = 8;

// Fill the derived fields of a Geom from a validated config.
inline Geom make_geom(const kvq_config& c) {
  Geom g{};
  g.B = c.batch; g.Hq = c.num_q_heads; g.Hkv = c.num_kv_heads; g.d = c.head_dim;
  g.ng = c.num_q_heads / c.num_kv_heads;
  g.kb = c.k_bits; g.vb = c.v_bits; g.G = c.k_group; g.GV = c.v_group;
  g.R = c.residual; g.C = c.res_capacity;
  g.max_blocks = c.max_blocks; g.num_pages = c.num_pages; g.dtype = c.dtype;
  g.k_words = g.d * g.kb / 32;
  g.v_words = g.G * g.vb / 32;
  g.rec_kc = 0;
  g.rec_ks = g.G * g.k_words * 4;
  g.rec_kz = g.rec_ks + 2 * g.d;
  g.rec_vc = g.rec_kz + 2 * g.d;
  g.rec_vs = g.rec_vc + g.d * g.v_words * 4;
  g.rec_vz = g.rec_vs + 2 * (g.d / g.GV) * g.G;
  g.rec_bytes = g.rec_vz + 2 * (g.d / g.GV) * g.G;
  g.P = c.sink;
  g.T = 1;
  g.W = c.fp8_blocks;
  g.rec8 = 2 * g.G * g.d + 4 * g.G;
  g.rot = c.rotate;
  return g;
}

// State words per sequence: {Q_b, S_b, flush arrivals, append arrivals};
// then the sticky error word (4B), the decode's finished-wave counter
// (4B + 1), and the decode's work-queue counters, one per 128-byte line
// (4B + kQueueStride * (k + 1), k < kQueues).
constexpr int kStateQ = 0, kStateS = 1, kStateFlushCnt = 2, kStateAppendCnt = 3;
constexpr int kQueues = 8;        // decode work queues (counters on separate cache lines)
constexpr int kQueueStride = 32;  // int32 words between queue counters
__host__ __device__ inline int state_words(int B) { return 4 * B + kQueueStride * (kQueues + 1); }
__host__ __device__ inline int state_done_word(int B) { return 4 * B + 1; }
__host__ __device__ inline int state_queue_word(int B, int k) { return 4 * B + kQueueStride * (k + 1); }

#ifdef __HIPCC__
// ---- conversions --------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
template <bool BF16>
__device__ __forceinline__ float in_to_f32(uint32_t bits16) {
  return BF16 ? bf16_to_f32(bits16) : f16_to_f32(bits16);
}
// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---- addressing ---------------------------------------------------------------
// Record of block `blk` of (sequence b, kv head h); nullptr for a page index
// outside the pool.
__device__ __forceinline__ const uint8_t* block_record(const Geom& g, const uint8_t* blocks,
                                                       const int32_t* table, int b, int h, int blk) {
  if (table == nullptr)
    return blocks + (((size_t)b * g.Hkv + h) * g.max_blocks + blk) * (size_t)g.rec_bytes;
  const int page = table[(size_t)b * g.max_blocks + blk];
  if (page < 0 || page >= g.num_pages) return nullptr;
  return blocks + ((size_t)page * g.Hkv + h) * (size_t)g.rec_bytes;
}

// ---- wave helpers (wave64) ----------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
// ---- Walsh-Hadamard transform of one row held by a wave ------------------------
// H x * scale (H the Sylvester Hadamard matrix) for a row of 128 channels held as
// lane l: (x[2l], x[2l+1]), in the butterfly order of the flush's pre-rotation
// (h = 1, 2, ..., 64; the pair (c, c + h) becomes (x_c + x_{c+h}, x_c - x_{c+h})).
// Stage h = 1 is inside the lane, stage h = 2m pairs lane l with lane l ^ m.
__device__ __forceinline__ void wht_row_pairs(float& x0, float& x1, float scale) {
  const int lane = threadIdx.x & 63;
  const float a = x0 + x1, b = x0 - x1;
  x0 = a;
  x1 = b;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float p0 = __shfl_xor(x0, m, 64), p1 = __shfl_xor(x1, m, 64);
    const bool upper = (lane & m) != 0;   // this lane holds the (c + h) side
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
  }
  x0 *= scale;
  x1 *= scale;
}
// The same for a row of 64 * CPL channels held as lane l: x[k] = channel l + 64k
// (stages h = 1 .. 32 across lanes, h = 64 inside the lane).
template <int CPL>
__device__ __forceinline__ void wht_row_strided(float (&x)[CPL], float scale) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const float p = __shfl_xor(x[k], m, 64);
      x[k] = upper ? p - x[k] : x[k] + p;
    }
  }
  if constexpr (CPL == 2) {
    const float a = x[0] + x[1], b = x[0] - x[1];
    x[0] = a;
    x[1] = b;
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k) x[k] *= scale;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data: waits for the wave's outstanding LDS operations only (global loads in
// flight stay in flight) and keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// One thread per workgroup calls this after the workgroup's work is done.
// Returns true for exactly one caller among `total` arrivals on `counter`,
// after every other arrival; that caller also re-arms the counter to 0.
// No fences: callers use it only to let one workgroup publish values that all
// of them computed alike from what they read before arriving (the length
// words); nothing written by another workgroup is read after it, and the
// next kernel sees every write at the launch boundary. (A device-scope fence
// here is an L2 write-back per workgroup.)
__device__ __forceinline__ bool last_arrival(int* counter, int total) {
  const int old = atomicAdd(counter, 1);
  if (old == total - 1) {
    atomicExch(counter, 0);
    return true;
  }
  return false;
}
// Persistent grid of a kernel of 256-thread workgroups: as many workgroups as
// stay resident at once (from the runtime's occupancy for this kernel and LDS
// size), rounded up to a multiple of the decode work queues. The answer is
// remembered per kernel (each instantiation has its own table), device and LDS
// size, since the occupancy query is slow next to a launch. The table is the
// library's only state across calls; a mutex guards it, so host threads may
// launch concurrently.
template <class K>
inline int persistent_grid(K kernel, size_t lds_bytes) {
  struct Memo {
    int dev;
    size_t lds;
    int grid;
  };
  static std::mutex lock;
  static Memo memo[16] = {};
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  {
    std::lock_guard<std::mutex> g(lock);
    for (int i = 0; i < used; ++i)
      if (memo[i].dev == dev && memo[i].lds == lds_bytes) return memo[i].grid;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds_bytes) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int grid = (cus * per_cu + kQueues - 1) / kQueues * kQueues;
  std::lock_guard<std::mutex> g(lock);
  if (used < 16) memo[used++] = Memo{dev, lds_bytes, grid};
  return grid;
}
#endif

// Launch wrappers (defined in the .hip files). Return hipSuccess or the error.
hipError_t launch_append(const Geom& g, const kvq_cache& c, const void* k_new, const void* v_new,
                         const int32_t* n_new, int n_max, hipStream_t s);
hipError_t launch_flush(const Geom& g, const kvq_cache& c, hipStream_t s);
hipError_t launch_append_flush(const Geom& g, const kvq_cache& c, const void* k_new, const void* v_new,
                               const int32_t* n_new, int n_max, hipStream_t s);
struct DecodePlan;
hipError_t launch_decode_partials(const Geom& g, const kvq_cache& c, const void* q, float scale,
                                  const DecodePlan& plan, void* ws, hipStream_t s);
hipError_t launch_decode_combine(const Geom& g, const kvq_cache& c, float* out, const DecodePlan& plan, void* ws,
                                 hipStream_t s);

// Decode work decomposition shared by the workspace sizing and the kernels.
struct DecodePlan {
  bool fast;          // MFMA kernel (else the generic VALU kernel)
  int nb_set;         // blocks per set (unit sizes are whole sets)
  int ring_chunk;     // ring tokens per ring unit
  int unit_sets;      // fixed sets per quantized unit (0: sized from the lengths)
  int max_blk;        // quantized blocks per (sequence, kv head) the workspace is sized for
  size_t units_max;   // upper bound on work units
  int fp8_rounds;     // side partial states of the FP8 tier per output row (64 of its tokens each)
  int nside;          // side partial states per output row: the sink's (P > 0), then the FP8 tier's
  size_t side_off;    // byte offset of the side partial states, [nside][B * H_q][d + 2]; 0 if none
  size_t ws_bytes;    // workspace bytes: the unit plan, the partial states, then the side ones
};
DecodePlan plan_decode(const Geom& g, int max_seq_tokens);

// Specialised paths (decode_fast_dispatch.hip): whether a configuration has an
// instantiation, its blocks per set, ring tokens per ring unit and fixed sets
// per unit (0: sized from the lengths), and the launch.
bool fast_supported(const Geom& g, int* blocks_per_set, int* ring_chunk, int* unit_sets);
hipError_t launch_decode_fast(const Geom& g, const kvq_cache& c, const void* q, float scale, const DecodePlan& p,
                              void* ws, hipStream_t s);

}  // namespace kvq
