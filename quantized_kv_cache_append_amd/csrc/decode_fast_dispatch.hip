// Instantiations of the MFMA decode path (decode_fast.h) and their dispatch.
//
// One instantiation per cache configuration the workloads use (query group,
// key/value bits, key and value group sizes, input dtype); any other
// configuration runs the generic kernel in decode.hip.
#include "decode_fast.h"

namespace kvq {

namespace {

struct FastEntry {
  int ng, kb, vb, G, GV, dtype;
  bool paged;
  int nb_set;
  hipError_t (*launch)(const Geom&, const kvq_cache&, const void*, float, int, int, void*, hipStream_t);
};

template <int NG, int KB, int VB, int G, int GV, bool BF16, bool PAGED>
constexpr FastEntry entry() {
  using C = fast::Cfg<NG, KB, VB, G, GV, BF16, PAGED>;
  return FastEntry{NG, KB, VB, G, GV, BF16 ? KVQ_BF16 : KVQ_F16, PAGED, C::NB, &fast::launch_fast<C>};
}

// dense and paged store of each configuration
#define KVQ_FAST(NG, KB, VB, G, GV, BF16) entry<NG, KB, VB, G, GV, BF16, false>(), entry<NG, KB, VB, G, GV, BF16, true>()

constexpr FastEntry kFast[] = {
    KVQ_FAST(1, 2, 2, 32, 32, false),   // MHA, INT2, G = G_V = 32, fp16 (a Llama-2-7B-shaped layer)
    KVQ_FAST(1, 2, 2, 32, 32, true),
    KVQ_FAST(4, 4, 4, 32, 32, true),    // GQA 4, INT4 (a Llama-3-8B-shaped layer)
    KVQ_FAST(4, 2, 2, 32, 32, true),    // GQA 4, INT2
    KVQ_FAST(8, 2, 2, 64, 64, true),    // GQA 8, INT2, G = G_V = 64 (a 70B-shaped layer)
    KVQ_FAST(6, 4, 2, 16, 32, true),    // GQA 6, INT4 keys / INT2 values, 16-token pages
};
#undef KVQ_FAST

const FastEntry* find(const Geom& g) {
  if (g.d != 128) return nullptr;
  for (const FastEntry& e : kFast)
    if (e.ng == g.ng && e.kb == g.kb && e.vb == g.vb && e.G == g.G && e.GV == g.GV && e.dtype == g.dtype &&
        e.paged == (g.num_pages > 0))
      return &e;
  return nullptr;
}

}  // namespace

int fast_ring_chunk() { return fast::kRingChunk; }

bool fast_supported(const Geom& g, int* blocks_per_set) {
  const FastEntry* e = find(g);
  if (e && blocks_per_set) *blocks_per_set = e->nb_set;
  return e != nullptr;
}

// Persistent grid: two 4-wave workgroups per compute unit (the kernel is built
// for 2 waves per SIMD), rounded up to a multiple of the work queues.
int persistent_grid() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * kQueues;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = (2 * cus + kQueues - 1) / kQueues * kQueues;
  }
  return cached[dev];
}

hipError_t launch_decode_fast(const Geom& g, const kvq_cache& c, const void* q, float scale, const DecodePlan& p,
                              void* ws, hipStream_t s) {
  const FastEntry* e = find(g);
  if (e == nullptr) return hipErrorInvalidValue;
  return e->launch(g, c, q, scale, p.max_blk, persistent_grid(), ws, s);
}

}  // namespace kvq
