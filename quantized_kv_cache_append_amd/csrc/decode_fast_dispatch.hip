// Instantiations of the MFMA decode path (decode_fast.h) and of the
// multi-head (one query head per kv head) path (decode_mha.h), and their
// dispatch.
//
// One instantiation per cache configuration the workloads use (query group,
// key/value bits, key and value group sizes, input dtype, dense or paged);
// any other configuration runs the generic kernel in decode.hip.
#include "decode_fast.h"
#include "decode_mha.h"
#include "decode_mx.h"

namespace kvq {

namespace {

using LaunchFn = hipError_t (*)(const Geom&, const kvq_cache&, const void*, float, int, void*, hipStream_t);

struct FastEntry {
  int ng, kb, vb, G, GV, dtype;
  bool paged;
  int nb_set;      // blocks per set
  int ring_chunk;  // ring tokens per ring unit
  int unit_sets;   // fixed sets per quantized unit (0: sized from the lengths)
  bool rot_ok;     // takes caches with pre-rotated keys and/or values
  LaunchFn launch;
};

template <int NG, int KB, int VB, int G, int GV, bool BF16, bool PAGED>
FastEntry mfma_entry() {
  using C = fast::Cfg<NG, KB, VB, G, GV, BF16, PAGED>;
  return FastEntry{NG, KB, VB, G, GV, BF16 ? KVQ_BF16 : KVQ_F16, PAGED, C::NB, fast::kRingChunk, 0, true,
                   &fast::launch_fast<C>};
}
template <bool BF16, bool PAGED>
FastEntry mx_entry() {
  using C = mx::Cfg<BF16, PAGED>;
  return FastEntry{1, C::KB, C::VB, C::G, C::GV, BF16 ? KVQ_BF16 : KVQ_F16, PAGED, mx::kSetBlk, mx::kRingTok,
                   mx::kUnitSets, true, &mx::launch_mx<C>};
}
template <int KB, int VB, int G, int GV, bool BF16, bool PAGED>
FastEntry mha_entry() {
  using C = mha::Cfg<KB, VB, G, GV, BF16, PAGED>;
  return FastEntry{1, KB, VB, G, GV, BF16 ? KVQ_BF16 : KVQ_F16, PAGED, C::NBS, mha::kRingTok, 0, true,
                   &mha::launch_mha<C>};
}

// dense and paged store of each configuration
#define KVQ_MFMA(NG, KB, VB, G, GV, BF16) \
  mfma_entry<NG, KB, VB, G, GV, BF16, false>(), mfma_entry<NG, KB, VB, G, GV, BF16, true>()
#define KVQ_MHA(KB, VB, G, GV, BF16) mha_entry<KB, VB, G, GV, BF16, false>(), mha_entry<KB, VB, G, GV, BF16, true>()
#define KVQ_MX(BF16) mx_entry<BF16, false>(), mx_entry<BF16, true>()

const FastEntry* table() {
  static const FastEntry kFast[] = {
      KVQ_MX(false),                       // MHA, INT2, G = G_V = 32, fp16 (a Llama-2-7B-shaped layer)
      KVQ_MX(true),
      KVQ_MHA(4, 4, 32, 32, false),        // MHA, INT4
      KVQ_MHA(4, 4, 32, 32, true),
      KVQ_MFMA(4, 4, 4, 32, 32, true),     // GQA 4, INT4 (a Llama-3-8B-shaped layer)
      KVQ_MFMA(4, 2, 2, 32, 32, true),     // GQA 4, INT2
      KVQ_MFMA(8, 2, 2, 64, 64, true),     // GQA 8, INT2, G = G_V = 64 (a 70B-shaped layer)
      KVQ_MFMA(6, 4, 2, 16, 32, true),     // GQA 6, INT4 keys / INT2 values, 16-token pages
      // query blocks of T tokens (T * n_g query rows): MHA fp16 INT2 with T = 4 and 8,
      // GQA 4 INT2 / INT4 with T = 2
      KVQ_MFMA(4, 2, 2, 32, 32, false),
      KVQ_MFMA(8, 2, 2, 32, 32, false),
      KVQ_MFMA(8, 2, 2, 32, 32, true),
      KVQ_MFMA(8, 4, 4, 32, 32, true),
  };
  return kFast;
}
constexpr int kEntries = 24;
#undef KVQ_MFMA
#undef KVQ_MHA
#undef KVQ_MX

const FastEntry* find(const Geom& g) {
  if (g.d != 128) return nullptr;
  const FastEntry* t = table();
  for (int i = 0; i < kEntries; ++i) {
    const FastEntry& e = t[i];
    if (e.ng == g.ng && e.kb == g.kb && e.vb == g.vb && e.G == g.G && e.GV == g.GV && e.dtype == g.dtype &&
        e.paged == (g.num_pages > 0) && (g.rot == 0 || e.rot_ok))
      return &e;
  }
  return nullptr;
}

}  // namespace

bool fast_supported(const Geom& g, int* blocks_per_set, int* ring_chunk, int* unit_sets) {
  const FastEntry* e = find(g);
  if (e && blocks_per_set) *blocks_per_set = e->nb_set;
  if (e && ring_chunk) *ring_chunk = e->ring_chunk;
  if (e && unit_sets) *unit_sets = e->unit_sets;
  return e != nullptr;
}

hipError_t launch_decode_fast(const Geom& g, const kvq_cache& c, const void* q, float scale, const DecodePlan& p,
                              void* ws, hipStream_t s) {
  const FastEntry* e = find(g);
  if (e == nullptr) return hipErrorInvalidValue;
  return e->launch(g, c, q, scale, p.max_blk, ws, s);
}

}  // namespace kvq
