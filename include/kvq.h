/*
 * kvq.h -- C ABI of libkvq: KIVI-style asymmetric low-bit KV-cache append,
 * residual flush (quantize + pack) and single-token decode attention over the
 * packed cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [P2] zubnet.ai, survey of KV-cache compression techniques (H2O, KIVI, MLA,
 *        StreamingLLM): quantization family -- keep every token, lower the bits;
 *        KIVI quantizes keys per channel and values per token.
 *   [P3] encorp.ai, "La compression du cache KV est une décision
 *        d'infrastructure, pas un débat sur les modèles": decode is bound by
 *        HBM traffic, not FLOPs.
 *   [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de
 *        l'art en 2026": section "Le problème" (cache bytes = 2*L*H*d*S*bytes),
 *        section "KIVI (2024)" (per-channel keys, per-token values, own min/max
 *        parameters, INT2 with a full-precision residual of recent tokens),
 *        innovation 3 (16 INT2 or 8 INT4 codes per 32-bit word; 16-token blocks
 *        for paged attention), innovation 4 (the most recent tokens stay in
 *        full precision and attention reads both parts transparently).
 *   [P1] ai-automate.fr, "KV-cache compressé et modèles 4-bit ...", section on
 *        Minima-KV: partial attention states merged by a globally normalised
 *        online softmax.
 *   FP8 tier: [P1], section on Minima-KV (recent and protected pages kept in
 *        FP8, older pages compacted to low bits, one online softmax over
 *        both).
 *   Multi-token query: [P3], section on EpiCache (block-wise prefill); [P4],
 *        introduction (compatible with block decoding).
 *   Attention sink: [P2], paragraph on the eviction family (StreamingLLM keeps
 *        the first tokens as attention sinks beside a recent window); [P3],
 *        section on OSCAR (sink and recent tokens kept in BF16, the history
 *        compressed to INT2).
 *
 * Memory model. The caller owns every buffer (sized with kvq_layout_bytes and
 * kvq_workspace_size). The library allocates nothing and borrows the pointers
 * for the duration of a call; it enqueues its kernels on the caller's HIP
 * stream (passed as void*; NULL is the default stream). All pointers in
 * kvq_cache and every tensor argument are DEVICE pointers. The state the
 * library keeps across calls is a host-side table of launch grid sizes per
 * (device, kernel, LDS bytes), filled on first use under a mutex, and the
 * device array of kvq_decode_attention_noalloc (one per GPU, with its address):
 * calls from several host threads are safe as long as they do not share a
 * cache or a workspace (or, for the no-allocation call, a GPU).
 *
 * One kvq_cache is one layer. For each (sequence b, kv head h), with a sink of
 * P >= 0 tokens (kvq_config.sink; P = 0: none):
 *   - tokens [0, min(S_b, P)) sit in the full-precision sink buffers, row t;
 *     they are never quantized;
 *   - tokens [P, P + Q_b) are quantized, in blocks of G tokens (a "record"
 *     each; block j holds tokens P + jG .. P + jG + G - 1);
 *   - tokens [P + Q_b, S_b) sit in a full-precision ring buffer of
 *     res_capacity slots; token t lives in slot (t - P) mod res_capacity;
 *   - after kvq_flush_residual, R <= S_b - P - Q_b < R + G whenever
 *     S_b - P >= R, i.e. Q_b = G * floor(max(S_b - P - R, 0) / G).
 * With P = 0 the sink is absent and everything else reads as written.
 *
 * FP8 tier (kvq_config.fp8_blocks = W > 0): the W most recent quantized
 * blocks of each (sequence, kv head), j >= n_b - W with n_b = Q_b / G, also
 * have an FP8 record in the `fp8` store, and attention reads them there
 * instead of their low-bit records (which are written as always). FP8 record
 * of a block (formula F8 per token row x of d values, fp32 IEEE steps, round
 * to nearest even: s = fp16(max|x| / 448); s == 0 -> codes 0; else code_c =
 * e4m3(clamp(x_c / s, -448, 448)); x_hat = e4m3_value(code) * s):
 *   K codes  uint8 [G][d]  e4m3, token-major
 *   K scale  fp16  [G]
 *   V codes  uint8 [G][d]
 *   V scale  fp16  [G]
 * Store: [B][H_kv][W] records; block j of a pair lives in slot j mod W.
 *
 * Walsh-Hadamard pre-rotation (kvq_config.rotate; [P4], "TurboQuant : les cinq
 * innovations", innovation 1: a WHT of the key and value vectors before
 * quantization spreads outliers over every dimension and is inverted on the
 * dequantized vectors). With KVQ_ROTATE_KEYS (KVQ_ROTATE_VALUES) every key
 * (value) token row x of a flushed block is replaced, before formula F, by
 * R(x) = H x / 8: H the d x d Sylvester Hadamard matrix (H_1 = [1], H_2n =
 * [[H_n, H_n], [H_n, -H_n]]), applied in fp32 as radix-2 butterflies -- for h =
 * 1, 2, ..., d/2, each pair (i, i + h) with bit h of i clear becomes
 * (x_i + x_{i+h}, x_i - x_{i+h}) -- then multiplied by 1/8 (exact). Records
 * then hold the rotated rows' codes, scales and zero-points; the ring and the
 * sink keep the original rows. Attention reads a dequantized rotated row y
 * back as H y * 8 / d (H H = d I): decode rotates the query instead for the
 * quantized keys, and applies H * 8 / d once per output row to the quantized
 * tokens' share of the value sum. Not with the FP8 tier (KVQ_ERR_UNSUPPORTED).
 *
 * Record of one block (little-endian, sections in this order, no padding):
 *   K codes  uint32 [G][d*k_bits/32]   token-major; word w of token t holds
 *                                       channels w*32/k_bits.. , LSB first
 *                                       (slot i at bits [i*b, (i+1)*b))
 *   K scale  fp16   [d]                 per channel over the block's G tokens
 *   K zero   fp16   [d]
 *   V codes  G*d*v_bits/8 bytes in 8-token chunks: the code of (token t,
 *            channel c) is entry pos(t,c) of an LSB-first stream of v_bits-wide
 *            codes packed into little-endian uint32 words, with
 *              pos(t,c) = ((t/8 * 16 + c%16) * (d/16) + c/16) * 8 + t%8
 *            (for each run of 8 tokens, for each c%16, for each c/16: that
 *            channel's 8 codes in token order)
 *   V scale  fp16   [d/G_V][G]          per (channel group, token)
 *   V zero   fp16   [d/G_V][G]
 * Dense store: records at [B][H_kv][max_blocks]. Paged store: one page holds
 * the records of one block for all H_kv heads, records at [num_pages][H_kv],
 * and block_table[b][j] names the page of block j of sequence b.
 *
 * Quantizer (formula F, every step an fp32 IEEE operation rounded to nearest
 * even, no fused multiply-add), per group x_1..x_n (a key channel over G
 * tokens, or G_V channels of one value token):
 *   z = fp16(min x);  s = fp16(fp32(max x - min x) / (2^b - 1));
 *   s == 0 -> all codes 0;  else inv = fp32(1/s),
 *   code_i = clamp(round_half_even(fp32(fp32(x_i - z) * inv)), 0, 2^b - 1);
 *   x_hat = code*s + z.
 * Input values whose group minimum lies outside the fp16 normal range are
 * outside the supported domain (results stay deterministic).
 *
 * Errors. Argument errors are reported synchronously, before any launch:
 * KVQ_ERR_CAPACITY when the request cannot fit the cache as configured (an
 * append larger than the sink plus the ring, or a max_seq_tokens beyond what
 * the sink, max_blocks blocks and the ring can hold). Conditions only the
 * device can see (ring full, flush past max_blocks, page index out of range)
 * skip the affected work and OR a KVQ_DEV_* bit into the cache's sticky error
 * word (read it with kvq_get_device_error). No call aborts or throws.
 *
 * Streams and graphs. Every call that takes a stream only enqueues kernels on
 * it: no allocation, memset, copy or synchronisation. Append, flush and decode
 * calls may therefore be captured in a HIP graph and replayed, provided the
 * caller passes the workspace and a max_seq_tokens that covers every length
 * the replays reach (the captured value is fixed). kvq_get_device_error
 * copies to the host and is not capturable.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1,   /* null pointer, non-positive or inconsistent size */
  KVQ_ERR_UNSUPPORTED = 2,   /* a well-formed configuration with no kernel in this build */
  KVQ_ERR_CAPACITY = 3,      /* the request exceeds what the cache as configured can hold */
  KVQ_ERR_WORKSPACE = 4,     /* workspace smaller than kvq_workspace_size() */
  KVQ_ERR_LAUNCH = 5,        /* the HIP runtime rejected a launch or a copy */
} kvq_status;

enum { KVQ_F16 = 0, KVQ_BF16 = 1 };
enum { KVQ_ROTATE_KEYS = 1, KVQ_ROTATE_VALUES = 2 };

/* Bits of the device-side sticky error word. */
enum {
  KVQ_DEV_RESIDUAL_FULL = 1, /* an append would overflow the ring: that sequence's tokens were not taken */
  KVQ_DEV_BLOCKS_FULL = 2,   /* a flush needed a block index >= max_blocks: it stopped there */
  KVQ_DEV_BAD_PAGE = 4,      /* a block_table entry was outside [0, num_pages): that block was skipped */
  KVQ_DEV_BAD_COUNT = 8,     /* an n_new[b] outside [0, n_max]: that sequence took nothing */
  KVQ_DEV_TOO_LONG = 16,     /* decode met S_b > max_seq_tokens: tokens past the bound were ignored */
};

typedef struct {
  int32_t batch;          /* B, sequences in this cache: 1 .. 1024                         */
  int32_t num_q_heads;    /* H_q                                                          */
  int32_t num_kv_heads;   /* H_kv; H_q % H_kv == 0; query head h' reads kv head h'/(H_q/H_kv) */
  int32_t head_dim;       /* d: 64 or 128                                                  */
  int32_t k_bits;         /* 2 or 4                                                       */
  int32_t v_bits;         /* 2 or 4                                                       */
  int32_t k_group;        /* G: tokens per key group = tokens per block (16, 32 or 64)    */
  int32_t v_group;        /* G_V: channels per value group (16, 32 or 64; divides d)      */
  int32_t residual;       /* R >= 0: tokens kept in full precision                         */
  int32_t res_capacity;   /* ring slots per (sequence, kv head); >= R + G                 */
  int32_t max_blocks;     /* dense: blocks per (sequence, kv head); paged: block_table width */
  int32_t num_pages;      /* 0: dense store; > 0: paged store with this many pages         */
  int32_t dtype;          /* KVQ_F16 or KVQ_BF16: K, V, q and the ring                     */
  int32_t sink;           /* P >= 0: leading tokens of every sequence kept in full precision */
  int32_t fp8_blocks;     /* W >= 0: most recent quantized blocks also kept, and read, in FP8 */
  int32_t rotate;         /* Walsh-Hadamard pre-rotation: 0 none, | KVQ_ROTATE_KEYS, | KVQ_ROTATE_VALUES */
} kvq_config;

typedef struct {
  size_t record;          /* bytes of one block of one kv head                              */
  size_t blocks;          /* bytes of the block store (dense records or page pool)           */
  size_t block_table;     /* bytes of the page table (int32 [B][max_blocks]); 0 if dense     */
  size_t ring;            /* bytes of EACH of k_ring and v_ring: [B][H_kv][res_capacity][d]  */
  size_t state;           /* bytes of the state words; must be zeroed before first use       */
  size_t sink;            /* bytes of EACH of k_sink and v_sink: [B][H_kv][P][d]; 0 if P = 0 */
  size_t fp8_record;      /* bytes of one FP8 record: 2*G*d + 4*G; 0 if W = 0               */
  size_t fp8;             /* bytes of the FP8 store: [B][H_kv][W] records; 0 if W = 0        */
} kvq_layout;

typedef struct {
  void* blocks;                /* block store, 16-byte aligned                                */
  const int32_t* block_table;  /* paged: [B][max_blocks] page of each block; NULL if dense    */
  void* k_ring;                /* [B][H_kv][res_capacity][d] of dtype                          */
  void* v_ring;
  int32_t* state;              /* [B][4] {Q_b, S_b, internal, internal}, then the error word
                                  and internal decode counters (kvq_layout.state bytes in all);
                                  zero-filled by the caller for an empty cache                 */
  void* k_sink;                /* [B][H_kv][P][d] of dtype, 16-byte aligned; NULL if P = 0     */
  void* v_sink;
  void* fp8;                   /* FP8 store, 16-byte aligned; NULL if W = 0                    */
} kvq_cache;

/* Host only. Validates cfg and fills the byte sizes of every cache buffer.
 * [P4] section "Le problème" gives the dense cache as 2*L*H*d*S*bytes (per
 * layer and sequence: 2*H_kv*d*S*bytes); here each quantized token costs
 * `record / G` bytes per kv head instead of 2*d*bytes (96 B against 512 B for
 * INT2, G = 32, d = 128), and only the sink and the ring keep 2*d*bytes per
 * token. Returns KVQ_ERR_INVALID_ARG / KVQ_ERR_UNSUPPORTED for a rejected
 * config. */
kvq_status kvq_layout_bytes(const kvq_config* cfg, kvq_layout* out);

/* Host only. Bytes of the decode workspace for sequences of at most
 * max_seq_tokens tokens (partial softmax states of the sequence splits, and
 * of the sink when P > 0). */
kvq_status kvq_workspace_size(const kvq_config* cfg, int32_t max_seq_tokens, size_t* bytes);

/* Append new key/value rows to the full-precision ring ([P4] KIVI: recent
 * tokens stay in full precision); rows whose position is below P go to the
 * sink instead.
 *   k_new, v_new: [B][H_kv][n_max][d] of dtype (device);
 *   n_new: device int32 [B], tokens to take from each sequence's first rows
 *          (0 <= n_new[b] <= n_max), or NULL to take n_max from every sequence.
 * S_b grows by n_new[b]. A sequence whose ring would overflow (its ring tokens
 * after the call, max(S_b + n_new[b] - P, 0) - Q_b, exceed res_capacity) takes
 * nothing and sets KVQ_DEV_RESIDUAL_FULL; call kvq_flush_residual between
 * large chunks. n_max > P + res_capacity can never fit and returns
 * KVQ_ERR_CAPACITY before any launch. */
kvq_status kvq_append(const kvq_config* cfg, const kvq_cache* cache,
                      const void* k_new, const void* v_new,
                      const int32_t* n_new, int32_t n_max, void* stream);

/* Quantize and pack the oldest complete G-token blocks of every ring so that
 * R <= S_b - P - Q_b < R + G afterwards ([P4] KIVI per-channel keys / per-token
 * values; [P4] innovation 3 dense packing; innovation 4 residual window).
 * With W > 0, the blocks of the call that end up among the W most recent also
 * get their FP8 record. Does nothing for sequences whose ring holds fewer than
 * R + G tokens. */
kvq_status kvq_flush_residual(const kvq_config* cfg, const kvq_cache* cache, void* stream);

/* kvq_append followed by kvq_flush_residual, as one launch when n_max <= 64
 * (one workgroup per (sequence, kv head) appends its rows and quantizes the
 * blocks that leave the window): the decode-step path. Same arguments, result
 * and device errors as the two calls in sequence. */
kvq_status kvq_append_flush(const kvq_config* cfg, const kvq_cache* cache,
                            const void* k_new, const void* v_new,
                            const int32_t* n_new, int32_t n_max, void* stream);

/* One decode step of attention for every (sequence, query head): the quantized
 * blocks are dequantized on the fly and the ring tokens read as they are;
 * sequence splits are merged by an online softmax ([P1] Minima-KV).
 *   q:   [B][H_q][d] of dtype (device), one query token per sequence;
 *   out: [B][H_q][d] fp32 (device);
 *   softmax_scale: multiplies q.k; <= 0 selects 1/sqrt(d);
 *   max_seq_tokens: an upper bound on every S_b (sizes the grid; the exact
 *                   lengths are read on the device); above P + max_blocks*G +
 *                   res_capacity, which no sequence can reach, it returns
 *                   KVQ_ERR_CAPACITY;
 *   workspace: device scratch of at least kvq_workspace_size(cfg, max_seq_tokens)
 *              bytes; its contents need no initialisation.
 * A sequence with S_b == 0 gets a zero output. The sink tokens of a sequence
 * (P > 0) and its FP8 blocks (W > 0) each enter as one more partial state per
 * (sequence, query head). The
 * launch hands out its work
 * through counters in the cache's state words (and re-arms them when it ends),
 * so decode calls on one cache, like calls that share a workspace, must be
 * ordered on one stream. */
kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache,
                                const void* q, float* out, float softmax_scale,
                                int32_t max_seq_tokens, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Attention of the T newest tokens of every sequence, causal within the
 * block: block-wise prefill, or checking T drafted tokens ([P3] EpiCache
 * section; [P4] introduction). The caller has appended the T tokens (S_b
 * counts them, and a flush may have run); query t of sequence b
 * (0 <= t < T) is token S_b - T + t and attends to tokens 0 .. S_b - T + t.
 *   q:   [B][H_q][T][d] of dtype (device);
 *   out: [B][H_q][T][d] fp32 (device); a query that sees no token (S_b < T)
 *        gets a zero row;
 *   T:   1 <= T, and T <= R when T > 1 (the T tokens are then all in the
 *        ring, so every quantized block is seen by every query), else
 *        KVQ_ERR_INVALID_ARG; (H_q / H_kv) * T <= 8, else KVQ_ERR_UNSUPPORTED;
 *   workspace: at least kvq_workspace_size_multi(cfg, max_seq_tokens, T)
 *        bytes.
 * Other arguments, errors and ordering as kvq_decode_attention, which is the
 * case T = 1. */
kvq_status kvq_decode_attention_multi(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t T,
                                      float* out, float softmax_scale, int32_t max_seq_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Host only. Workspace bytes of kvq_decode_attention_multi with T queries per
 * sequence (T = 1: kvq_workspace_size). Rejects T as that call does. */
kvq_status kvq_workspace_size_multi(const kvq_config* cfg, int32_t max_seq_tokens, int32_t T, size_t* bytes);

/* The two launches of kvq_decode_attention, callable separately (same
 * arguments and errors; the workspace carries the split states from the first
 * call to the second, which must follow it on the same stream with the same
 * cache, configuration and max_seq_tokens, nothing touching the cache or the
 * workspace in between). kvq_decode_partials computes the partial softmax
 * state (running maximum, sum and unnormalised output, [P1] Minima-KV) of
 * every work unit -- a run of quantized blocks or of ring tokens of one
 * (sequence, kv head) -- into the workspace, and the side states of every
 * output row: its sink tokens (P > 0) and its FP8 tier (W > 0, one state per
 * 64 of the tier's tokens), each from a launch of its own before the units';
 * kvq_decode_combine merges them all into out. Useful to time or overlap the
 * two phases. */
kvq_status kvq_decode_partials(const kvq_config* cfg, const kvq_cache* cache,
                               const void* q, float softmax_scale, int32_t max_seq_tokens,
                               void* workspace, size_t workspace_bytes, void* stream);
kvq_status kvq_decode_combine(const kvq_config* cfg, const kvq_cache* cache, float* out,
                              int32_t max_seq_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kvq_decode_attention with the decode workspace taken from a device array the
 * library holds per GPU, KVQ_NOALLOC_WORKSPACE_BYTES (64 MiB) on each GPU it
 * runs on, kept until the process ends. The caller still passes the cache, q
 * and out. Configurations whose kvq_workspace_size(cfg, max_seq_tokens)
 * exceeds that size get KVQ_ERR_WORKSPACE before any device call. Every call on
 * one GPU uses that GPU's array, whose contents need no initialisation and are
 * left as the last call wrote them: calls that overlap on one GPU (several
 * streams or threads, or a graph replayed while another call runs) race and
 * must be ordered by the caller. Arguments, errors and results otherwise as
 * kvq_decode_attention. No allocation, free or allocating library routine is
 * called; the first call on a GPU looks the array's address up once. */
#define KVQ_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache, const void* q, float* out,
                                        float softmax_scale, int32_t max_seq_tokens, void* stream);

/* Copies the cache's sticky error word (an OR of KVQ_DEV_* bits; 0 = nothing
 * so far) into *err after the stream's earlier work, waiting for the stream.
 * cfg locates the word (it follows the B per-sequence state words). */
kvq_status kvq_get_device_error(const kvq_config* cfg, const kvq_cache* cache, void* stream,
                                int32_t* err);

/* Static string naming a status code. */
const char* kvq_status_string(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
