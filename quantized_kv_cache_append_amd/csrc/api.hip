// Host side of the C ABI declared in include/kvq.h: argument validation, byte
// layout arithmetic and kernel launches on the caller's stream. No allocation;
// the state kept across calls is the launch-grid table of persistent_grid()
// (common.h) and, for kvq_decode_attention_noalloc, one device array per GPU
// (below) with its address.
//
// Sources:
//   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
//        l'art en 2026": section "Le problème" gives the dense cache size
//        2*L*H*d*S*bytes that the packed layout shrinks; innovation 3 fixes the
//        packing density (16 INT2 / 8 INT4 per 32-bit word) and 16-token blocks
//        for paged caches.
#include <cmath>
#include <cstring>

#include "common.h"

using kvq::Geom;

namespace {

// Every decode workgroup keeps a copy of the unit plan (16 + 7B ints) in LDS
// beside its four waves' buffers (at most 4 x 15 KB); at B = 1024 that is at
// most 89 KB, inside gfx950's 160 KB per workgroup.
constexpr int kMaxBatch = 1024;
constexpr int kMaxSink = 1 << 20;   // sink tokens per sequence
constexpr int kMaxFp8Blocks = 4096;  // FP8 blocks per (sequence, kv head)

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

kvq_status validate(const kvq_config* c) {
  if (c == nullptr) return KVQ_ERR_INVALID_ARG;
  if (c->batch <= 0 || c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 ||
      c->k_group <= 0 || c->v_group <= 0 || c->residual < 0 || c->res_capacity <= 0 || c->max_blocks < 0 ||
      c->num_pages < 0 || c->sink < 0 || c->fp8_blocks < 0)
    return KVQ_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  if (c->dtype != KVQ_F16 && c->dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if ((c->k_bits != 2 && c->k_bits != 4) || (c->v_bits != 2 && c->v_bits != 4)) return KVQ_ERR_UNSUPPORTED;
  if (c->head_dim % c->v_group != 0) return KVQ_ERR_INVALID_ARG;
  if (c->res_capacity < c->residual + c->k_group) return KVQ_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (!pow2_in(c->k_group, 16, 64) || !pow2_in(c->v_group, 16, 64)) return KVQ_ERR_UNSUPPORTED;
  if (c->num_q_heads / c->num_kv_heads > 8) return KVQ_ERR_UNSUPPORTED;
  if (c->batch > kMaxBatch) return KVQ_ERR_UNSUPPORTED;
  if (c->sink > kMaxSink) return KVQ_ERR_UNSUPPORTED;
  if (c->fp8_blocks > kMaxFp8Blocks) return KVQ_ERR_UNSUPPORTED;
  if ((long long)c->k_group * c->v_bits < 32) return KVQ_ERR_UNSUPPORTED;
  if (c->rotate & ~(KVQ_ROTATE_KEYS | KVQ_ROTATE_VALUES)) return KVQ_ERR_INVALID_ARG;
  if (c->rotate != 0 && c->fp8_blocks > 0) return KVQ_ERR_UNSUPPORTED;   // the FP8 tier stores unrotated rows
  return KVQ_OK;
}

kvq_status validate_cache(const kvq_config* c, const kvq_cache* k) {
  if (k == nullptr || k->blocks == nullptr || k->k_ring == nullptr || k->v_ring == nullptr ||
      k->state == nullptr)
    return KVQ_ERR_INVALID_ARG;
  if ((c->num_pages > 0) != (k->block_table != nullptr)) return KVQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k->blocks) | reinterpret_cast<uintptr_t>(k->k_ring) |
       reinterpret_cast<uintptr_t>(k->v_ring)) & 15)
    return KVQ_ERR_INVALID_ARG;
  if (c->sink > 0 && (k->k_sink == nullptr || k->v_sink == nullptr ||
                      ((reinterpret_cast<uintptr_t>(k->k_sink) | reinterpret_cast<uintptr_t>(k->v_sink)) & 15)))
    return KVQ_ERR_INVALID_ARG;
  if (c->fp8_blocks > 0 && (k->fp8 == nullptr || (reinterpret_cast<uintptr_t>(k->fp8) & 15)))
    return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

kvq_status launched(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

// The most tokens a sequence can hold: the sink, max_blocks quantized blocks
// and a full ring.
long long capacity_tokens(const kvq_config* c) {
  return (long long)c->sink + (long long)c->max_blocks * c->k_group + c->res_capacity;
}
// Rows of one append that can never fit: the sink takes at most P, the ring
// at most res_capacity.
bool append_fits(const kvq_config* c, int32_t n_max) { return (long long)n_max <= (long long)c->sink + c->res_capacity; }

}  // namespace

extern "C" {

kvq_status kvq_layout_bytes(const kvq_config* cfg, kvq_layout* out) {
  const kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if (out == nullptr) return KVQ_ERR_INVALID_ARG;
  const Geom g = kvq::make_geom(*cfg);
  out->record = (size_t)g.rec_bytes;
  if (cfg->num_pages > 0) {
    out->blocks = (size_t)cfg->num_pages * g.Hkv * g.rec_bytes;
    out->block_table = (size_t)g.B * cfg->max_blocks * sizeof(int32_t);
  } else {
    out->blocks = (size_t)g.B * g.Hkv * (size_t)cfg->max_blocks * g.rec_bytes;
    out->block_table = 0;
  }
  out->ring = (size_t)g.B * g.Hkv * (size_t)g.C * g.d * 2;
  out->state = (size_t)kvq::state_words(g.B) * sizeof(int32_t);
  out->sink = (size_t)g.B * g.Hkv * (size_t)g.P * g.d * 2;
  out->fp8_record = g.W > 0 ? (size_t)g.rec8 : 0;
  out->fp8 = (size_t)g.B * g.Hkv * (size_t)g.W * out->fp8_record;
  return KVQ_OK;
}

}  // extern "C"

namespace {
// Geometry of a call with T queries per (sequence, query head): the T newest
// tokens act as T query heads each, row j of a kv head's n_g * T rows being
// token S_b - T + j % T. T <= R keeps all of them in the ring, so every
// quantized block is seen by every query.
kvq_status query_geom(const kvq_config* cfg, int32_t T, Geom& g) {
  if (T < 1 || (T > 1 && T > cfg->residual)) return KVQ_ERR_INVALID_ARG;
  g = kvq::make_geom(*cfg);
  if ((long long)g.ng * T > kvq::kNgMax) return KVQ_ERR_UNSUPPORTED;
  g.Hq *= T;
  g.ng *= T;
  g.T = T;
  return KVQ_OK;
}
}  // namespace

extern "C" {

kvq_status kvq_workspace_size_multi(const kvq_config* cfg, int32_t max_seq_tokens, int32_t T, size_t* bytes) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if (bytes == nullptr || max_seq_tokens < 0) return KVQ_ERR_INVALID_ARG;
  Geom g;
  if ((st = query_geom(cfg, T, g)) != KVQ_OK) return st;
  *bytes = kvq::plan_decode(g, max_seq_tokens).ws_bytes;
  return KVQ_OK;
}

kvq_status kvq_workspace_size(const kvq_config* cfg, int32_t max_seq_tokens, size_t* bytes) {
  return kvq_workspace_size_multi(cfg, max_seq_tokens, 1, bytes);
}

kvq_status kvq_append(const kvq_config* cfg, const kvq_cache* cache, const void* k_new, const void* v_new,
                      const int32_t* n_new, int32_t n_max, void* stream) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if ((st = validate_cache(cfg, cache)) != KVQ_OK) return st;
  if (k_new == nullptr || v_new == nullptr || n_max < 0) return KVQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15) return KVQ_ERR_INVALID_ARG;
  if (!append_fits(cfg, n_max)) return KVQ_ERR_CAPACITY;
  if (n_max == 0) return KVQ_OK;
  return launched(kvq::launch_append(kvq::make_geom(*cfg), *cache, k_new, v_new, n_new, n_max,
                                     static_cast<hipStream_t>(stream)));
}

kvq_status kvq_append_flush(const kvq_config* cfg, const kvq_cache* cache, const void* k_new, const void* v_new,
                            const int32_t* n_new, int32_t n_max, void* stream) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if ((st = validate_cache(cfg, cache)) != KVQ_OK) return st;
  if (k_new == nullptr || v_new == nullptr || n_max < 0) return KVQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15) return KVQ_ERR_INVALID_ARG;
  if (!append_fits(cfg, n_max)) return KVQ_ERR_CAPACITY;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_max == 0) return launched(kvq::launch_flush(kvq::make_geom(*cfg), *cache, s));
  return launched(kvq::launch_append_flush(kvq::make_geom(*cfg), *cache, k_new, v_new, n_new, n_max, s));
}

kvq_status kvq_flush_residual(const kvq_config* cfg, const kvq_cache* cache, void* stream) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if ((st = validate_cache(cfg, cache)) != KVQ_OK) return st;
  return launched(kvq::launch_flush(kvq::make_geom(*cfg), *cache, static_cast<hipStream_t>(stream)));
}

namespace {
// Shared argument checks of the decode entry points; fills g, plan and scale.
kvq_status decode_args(const kvq_config* cfg, const kvq_cache* cache, int32_t max_seq_tokens, void* workspace,
                       size_t workspace_bytes, float softmax_scale, Geom& g, kvq::DecodePlan& plan,
                       float& scale, int32_t T = 1) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if ((st = validate_cache(cfg, cache)) != KVQ_OK) return st;
  if (max_seq_tokens < 0 || !std::isfinite(softmax_scale)) return KVQ_ERR_INVALID_ARG;
  if (max_seq_tokens > capacity_tokens(cfg)) return KVQ_ERR_CAPACITY;
  if ((st = query_geom(cfg, T, g)) != KVQ_OK) return st;
  plan = kvq::plan_decode(g, max_seq_tokens);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return KVQ_ERR_WORKSPACE;
  scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)g.d);
  return KVQ_OK;
}
}  // namespace

kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q, float* out,
                                float softmax_scale, int32_t max_seq_tokens, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (q == nullptr || out == nullptr) return KVQ_ERR_INVALID_ARG;
  Geom g;
  kvq::DecodePlan plan;
  float scale;
  const kvq_status st = decode_args(cfg, cache, max_seq_tokens, workspace, workspace_bytes, softmax_scale, g, plan, scale);
  if (st != KVQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kvq::launch_decode_partials(g, *cache, q, scale, plan, workspace, s) != hipSuccess) return KVQ_ERR_LAUNCH;
  return launched(kvq::launch_decode_combine(g, *cache, out, plan, workspace, s));
}

kvq_status kvq_decode_attention_multi(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t T,
                                      float* out, float softmax_scale, int32_t max_seq_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (q == nullptr || out == nullptr) return KVQ_ERR_INVALID_ARG;
  Geom g;
  kvq::DecodePlan plan;
  float scale;
  const kvq_status st =
      decode_args(cfg, cache, max_seq_tokens, workspace, workspace_bytes, softmax_scale, g, plan, scale, T);
  if (st != KVQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kvq::launch_decode_partials(g, *cache, q, scale, plan, workspace, s) != hipSuccess) return KVQ_ERR_LAUNCH;
  return launched(kvq::launch_decode_combine(g, *cache, out, plan, workspace, s));
}

kvq_status kvq_decode_partials(const kvq_config* cfg, const kvq_cache* cache, const void* q, float softmax_scale,
                               int32_t max_seq_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr) return KVQ_ERR_INVALID_ARG;
  Geom g;
  kvq::DecodePlan plan;
  float scale;
  const kvq_status st = decode_args(cfg, cache, max_seq_tokens, workspace, workspace_bytes, softmax_scale, g, plan, scale);
  if (st != KVQ_OK) return st;
  return launched(kvq::launch_decode_partials(g, *cache, q, scale, plan, workspace, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_combine(const kvq_config* cfg, const kvq_cache* cache, float* out, int32_t max_seq_tokens,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (out == nullptr) return KVQ_ERR_INVALID_ARG;
  Geom g;
  kvq::DecodePlan plan;
  float scale;
  const kvq_status st = decode_args(cfg, cache, max_seq_tokens, workspace, workspace_bytes, 0.f, g, plan, scale);
  if (st != KVQ_OK) return st;
  return launched(kvq::launch_decode_combine(g, *cache, out, plan, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- the decode entry point that allocates nothing -----------------------------------
namespace {
// The decode workspace of kvq_decode_attention_noalloc: one array per GPU the
// library runs on, held until the process ends. Host code must not use its name
// as an address (that is a host-side stand-in): the device address is taken once
// per device with hipGetSymbolAddress and kept in scratch_ptr.
constexpr size_t kScratchBytes = KVQ_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_lock;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first
// call on that device, with the device current).
kvq_status scratch_of_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_lock);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KVQ_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return KVQ_OK;
}
}  // namespace

extern "C" {

kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache, const void* q, float* out,
                                        float softmax_scale, int32_t max_seq_tokens, void* stream) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if ((st = validate_cache(cfg, cache)) != KVQ_OK) return st;
  if (q == nullptr || out == nullptr || max_seq_tokens < 0 || !std::isfinite(softmax_scale))
    return KVQ_ERR_INVALID_ARG;
  if (max_seq_tokens > capacity_tokens(cfg)) return KVQ_ERR_CAPACITY;
  size_t need = 0;
  if ((st = kvq_workspace_size(cfg, max_seq_tokens, &need)) != KVQ_OK) return st;
  if (need > kScratchBytes) return KVQ_ERR_WORKSPACE;   // before any device call
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != KVQ_OK) return st;
  return kvq_decode_attention(cfg, cache, q, out, softmax_scale, max_seq_tokens, ws, kScratchBytes, stream);
}

kvq_status kvq_get_device_error(const kvq_config* cfg, const kvq_cache* cache, void* stream,
                                int32_t* err) {
  const kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if (cache == nullptr || cache->state == nullptr || err == nullptr) return KVQ_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t word = 0;
  if (hipMemcpyAsync(&word, cache->state + 4 * cfg->batch, sizeof(word), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return KVQ_ERR_LAUNCH;
  *err = word;
  return KVQ_OK;
}

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "request exceeds the cache's capacity";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
