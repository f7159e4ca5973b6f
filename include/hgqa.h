/*
 * hgqa.h - hybrid sliding/full grouped-query attention for MI355X (gfx950).
 *
 * The C ABI of libhgqa.so. One attention layer of a hybrid stack in which
 * most layers attend through a sliding window and one layer in four attends
 * to the whole causal context:
 *
 *   y[b,i,h] = sigmoid(gate[b,i,h]) * sum_j P[i,j] * V[b,j,h/G]
 *   P[i,:]   = softmax over visible j of scale * <rope(q_i, i), rope(k_j, j)>
 *   visible  : j <= i, and for a sliding layer also i - j < W
 *
 * Sources, cited by page and section:
 *   "Step-3.7-Flash-oQ3e" walkthrough, section 2: layer_types selects full or
 *   sliding attention per layer (2.1, 2.2); both masks are built once and each
 *   layer picks its own (2.2); a sliding layer's cache keeps W = 512 tokens
 *   (2.2); rope_theta is per layer and full layers rotate only half of
 *   head_dim (2.3); every head has its own sigmoid gate (2.3).
 *   "Step-3.7-Flash" model card, table "config.json: all 49 fields": 64 heads
 *   in 8 KV groups (GQA), head_dim 128, sliding_window 512, sink false.
 *   "Muse-Glimmer-30B-6bit" walkthrough, sections "GQA 16:1" (32 Q / 2 KV
 *   heads), "sliding window attention: 39 + 13" (W = 2048, one full layer in
 *   four), "the RoPE zero value" (base 0 means no rotation), and "each layer:
 *   double LayerNorm + gated attention" (gate_proj: sigmoid gate on the
 *   attention output).
 *
 * Readings where the pages are silent: W counts keys including the query;
 * RoPE pairs dim i with dim i + r/2 inside the first r = round(f * D) dims at
 * frequency theta^(-2i/r); Q head h reads KV head h / G (contiguous groups);
 * positions are 0-based; one gate logit per (token, head).
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless marked [host]. The caller owns every
 *     buffer. Buffers are dense row-major in the layouts given, 16-byte
 *     aligned, and outputs do not alias inputs.
 *   - Arguments are checked on the host before anything is enqueued; an
 *     invalid call returns a negative HGQA_E* code, enqueues nothing and
 *     leaves a message for hgqa_last_error().
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the legacy default
 *     stream) and the call returns without waiting for it.
 *   - The library allocates no device memory and keeps no state between calls
 *     besides a per-thread error message and the process-wide tuning
 *     overrides of hgqa_set_tuning. Scratch memory is passed in by the caller
 *     as `workspace`, sized by the matching *_workspace_bytes query: prefill
 *     keeps each key rotated once there (and the cos/sin rows the queries
 *     are rotated with), decode keeps its per-split partial results.
 *   - Device-side integers (start_pos, seq_lens) are trusted within the
 *     host-side bounds passed with them; values outside are clamped so that
 *     no access leaves the buffers, and the result for them is unspecified.
 */
#ifndef HGQA_H
#define HGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer kinds ("Step-3.7-Flash-oQ3e" walkthrough 2.1: layer_types). */
enum { HGQA_FULL = 0, HGQA_SLIDING = 1 };

/* Element type of Q, K, V, gate, output and caches (all the same). */
enum { HGQA_BF16 = 0, HGQA_FP32 = 1 };

/* Return codes. */
enum {
  HGQA_OK = 0,
  HGQA_EINVAL = -1,       /* malformed argument                          */
  HGQA_EUNSUPPORTED = -2, /* well formed but not implemented (shape/type)  */
  HGQA_ENOSPACE = -3,     /* workspace or cache too small                  */
  HGQA_EHIP = -4          /* the HIP runtime reported an error on launch   */
};

/*
 * One layer's attention settings, as the model config gives them.
 *   layer_type      HGQA_FULL or HGQA_SLIDING
 *   window          W >= 1 keys visible to a query, itself included
 *                   (sliding only; ignored for full layers)
 *   num_q_heads     Hq >= 1
 *   gqa_ratio       G >= 1 query heads per KV head; Hkv = Hq / G, Hq % G == 0
 *   head_dim        D: 64 or 128
 *   rope_theta      RoPE base >= 0; 0 means no rotation
 *   rotary_fraction f in [0, 1]; r = round(f * D) leading dims rotate.
 *                   r must be even; bf16 layers need r % 16 == 0.
 *                   r == 0 means no rotation.
 *   softmax_scale   > 0 to set the scale; <= 0 selects 1 / sqrt(D)
 *   dtype           HGQA_BF16 or HGQA_FP32
 *   rope_scaling_factor, rope_low_freq_factor, rope_high_freq_factor,
 *   rope_original_max_positions
 *                   long-context RoPE frequency scaling ("rope_type llama3"),
 *                   which "Step-3.7-Flash-oQ3e" walkthrough 2.3 mounts on full
 *                   layers only: it is ignored on sliding layers. A factor
 *                   <= 1 means none (so does a zero-initialised descriptor).
 *                   With a factor > 1, a frequency w whose wavelength 2 pi / w
 *                   is below N / high keeps w, one above N / low becomes
 *                   w / factor, and one in between is blended linearly:
 *                   s = (N * w / (2 pi) - low) / (high - low),
 *                   w' = (1 - s) w / factor + s w, N the original context.
 *                   Fields <= 0 take the defaults low 1, high 4,
 *                   N 131072; high must exceed low.
 */
typedef struct {
  int32_t layer_type;
  int32_t window;
  int32_t num_q_heads;
  int32_t gqa_ratio;
  int32_t head_dim;
  float rope_theta;
  float rotary_fraction;
  float softmax_scale;
  int32_t dtype;
  float rope_scaling_factor;
  float rope_low_freq_factor;
  float rope_high_freq_factor;
  int32_t rope_original_max_positions;
} hgqa_layer;

/*
 * Scratch bytes attn_prefill needs for this layer and shape: the rotated K,
 * [B, Hkv, T, D] in the layer dtype, a cos/sin table [T, r/2] of float pairs
 * and, for a full bf16 layer with D = 128, V transposed, [B, Hkv, D, T'] bf16
 * with T' = T rounded up to 64; each part rounded up to 256 bytes. Returns 0
 * for an invalid layer.
 */
size_t attn_prefill_workspace_bytes(const hgqa_layer* layer, int32_t batch,
                                    int32_t seq_len);

/*
 * Prefill: attention of a whole prompt at positions 0..T-1 over itself.
 *   q     [B, T, Hq, D]   queries, not rotated
 *   k, v  [B, T, Hkv, D]  keys (not rotated) and values
 *   gate  [B, T, Hq]      gate logits
 *   out   [B, T, Hq, D]   gated attention output
 *   workspace            >= attn_prefill_workspace_bytes(layer, B, T) bytes
 * batch == 0 or seq_len == 0 is a valid call that does nothing. A full bf16
 * layer with D = 128 takes seq_len < 2^23 (HGQA_EUNSUPPORTED otherwise: its
 * V^T rows must stay within 32-bit byte offsets).
 * The masks follow "Step-3.7-Flash-oQ3e" walkthrough 2.2; RoPE and the gate
 * follow 2.3 of the same page.
 */
int attn_prefill(const hgqa_layer* layer, int32_t batch, int32_t seq_len,
                 const void* q, const void* k, const void* v, const void* gate,
                 void* out, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Scratch bytes attn_prefill_chunk needs for a call whose sequences end at
 * most at max_end_pos: the rotated new keys [B, Hkv, n_new, D] in the layer
 * dtype, one cos/sin table per sequence [B, n_new, r/2] of float pairs (the
 * sequences start at different positions), and, when the call is split over
 * keys (few rows over long caches: a multi-token step), per-split partial
 * results [B, n_new, Hq, splits, D + 4] float32; each part rounded up to 256
 * bytes. Returns 0 for an invalid layer or max_end_pos < n_new.
 */
size_t attn_prefill_chunk_workspace_bytes(const hgqa_layer* layer, int32_t batch,
                                          int32_t n_new, int32_t max_end_pos);

/*
 * Chunked prefill: the n_new new tokens of sequence b, at absolute positions
 * start_pos[b] .. start_pos[b] + n_new - 1, attend over the layer's cache (the
 * positions before start_pos[b]) and over themselves; then they are appended
 * to the cache. The result is what attn_prefill over the whole sequence gives
 * for these rows. This is the cache-backed prefill that the model pages leave
 * to the full implementation ("Step-3.7-Flash-oQ3e" walkthrough, section 6,
 * where the model class takes over KV-cache prefill control) over the
 * sliding cache of section 2.2 of the same page. A multi-token decode step
 * (one token plus draft tokens, each seeing the cache and the earlier new
 * tokens; the "Step-3.7-Flash" model card lists num_nextn_predict_layers 3)
 * is this call with a small n_new; every sequence may sit at its own
 * position.
 *   start_pos [B] int32   position of the first new token of each sequence
 *   max_end_pos [host]    >= start_pos[b] + n_new for every b, >= n_new
 *   q     [B, n, Hq, D]   queries, not rotated
 *   k, v  [B, n, Hkv, D]  new keys (not rotated) and values
 *   gate  [B, n, Hq]      gate logits
 *   k_cache, v_cache [B, Hkv, cap, D]  as kv_append fills them: rotated keys
 *         and values of positions < start_pos[b]. Full layer: slot p holds
 *         position p, and cap >= max_end_pos. Sliding layer: cap == W and
 *         slot p mod W holds position p for the last W positions before
 *         start_pos[b] (every earlier position the new rows can see).
 *   out   [B, n, Hq, D]   gated attention output
 *   workspace            >= attn_prefill_chunk_workspace_bytes(layer, B, n)
 * On a sliding layer the attention reads the ring before the append writes
 * it (in stream order), so a ring may be overwritten by its own chunk; on a
 * full layer (bf16, D = 128) the chunk is appended first and every key is
 * read from the cache, which gives the same result. The caches must not alias any
 * other argument. n_new == 0 or batch == 0 does nothing. Errors: as
 * attn_prefill, plus HGQA_ENOSPACE when a full cache is smaller than
 * max_end_pos and HGQA_EINVAL when a ring's capacity differs from W. A
 * start_pos[b] outside [0, max_end_pos - n_new] is clamped into it (no access
 * leaves the buffers; that sequence's result is unspecified).
 */
int attn_prefill_chunk(const hgqa_layer* layer, int32_t batch, int32_t n_new,
                       const int32_t* start_pos, int32_t max_end_pos, const void* q,
                       const void* k, const void* v, const void* gate, void* k_cache,
                       void* v_cache, int32_t cache_capacity, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Append new tokens to a layer's KV cache.
 *   start_pos    [B] int32  absolute position of k_new[b, 0]; >= 0
 *   max_end_pos  [host]     >= start_pos[b] + n_new for every b
 *   k_new, v_new [B, n_new, Hkv, D]  new keys (not rotated) and values
 *   k_cache, v_cache [B, Hkv, cache_capacity, D]
 * Token n of sequence b sits at p = start_pos[b] + n. Its key, rotated at p,
 * and its value are written to slot p of a full layer's cache (which needs
 * cache_capacity >= max_end_pos), or to slot p mod W of a sliding layer's
 * ring, whose cache_capacity must equal W ("Step-3.7-Flash-oQ3e" walkthrough
 * 2.2: a sliding layer's cache keeps only W tokens). When one call writes
 * more than W tokens to a ring, only the last W positions are written, so
 * each slot ends with the highest position that maps to it.
 */
int kv_append(const hgqa_layer* layer, int32_t batch, int32_t n_new,
              const int32_t* start_pos, int32_t max_end_pos,
              const void* k_new, const void* v_new, void* k_cache,
              void* v_cache, int32_t cache_capacity, void* stream);

/*
 * Scratch bytes attn_decode needs: per-split partial results (running max,
 * running sum and unnormalised output, float32) for the split count the
 * library picks for this layer, batch and longest context. May be 0 when no
 * split is needed. Returns 0 for an invalid layer.
 */
size_t attn_decode_workspace_bytes(const hgqa_layer* layer, int32_t batch,
                                   int32_t max_seq_len);

/*
 * Decode: one new query token per sequence against its cache. This is the
 * cached form of the layer that "Step-3.7-Flash-oQ3e" walkthrough 2.2
 * describes: a sliding layer's cache keeps only the last W tokens and the
 * query attends to them, a full layer's cache keeps every token (2.3 of the
 * same page: full layers see the whole context). RoPE and the per-head
 * sigmoid gate follow 2.3.
 *   q        [B, Hq, D]  queries, not rotated; the query of sequence b sits
 *                        at position seq_lens[b] - 1
 *   gate     [B, Hq]     gate logits
 *   k_cache, v_cache [B, Hkv, cache_capacity, D] as written by kv_append
 *                        (K rotated), already holding the new token
 *   seq_lens [B] int32   tokens in the cache including the new one, >= 1
 *   max_seq_len [host]   >= every seq_lens[b]; full layers need
 *                        cache_capacity >= max_seq_len
 *   workspace            >= attn_decode_workspace_bytes(layer, B,
 *                        max_seq_len) bytes (may be NULL when that is 0)
 *   out      [B, Hq, D]
 * A full layer attends to slots 0..L-1; a sliding layer's ring holds the
 * last min(L, W) positions and the query attends to all of them. bf16
 * layers support gqa_ratio <= 16 (HGQA_EUNSUPPORTED above). A seq_lens[b]
 * outside [1, max_seq_len] is clamped into it.
 */
int attn_decode(const hgqa_layer* layer, int32_t batch, const void* q,
                const void* gate, const void* k_cache, const void* v_cache,
                int32_t cache_capacity, const int32_t* seq_lens,
                int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                void* out, void* stream);

/*
 * attn_decode for callers that cannot allocate: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc. The same
 * arguments without the workspace; the per-split partials go to a static
 * device array of the library (16 MiB, one copy per GPU, held until the
 * process ends), whose address on each GPU is looked up on that GPU's first
 * call. Nothing is allocated. A plan that needs more than 16 MiB of partials
 * (attn_decode_workspace_bytes above it) returns HGQA_ENOSPACE before
 * anything is enqueued. Calls on one GPU share the array: calls that overlap
 * on one GPU (other streams, other threads) race, and the caller must order
 * them. The output equals attn_decode's for the same inputs.
 */
int attn_decode_noalloc(const hgqa_layer* layer, int32_t batch, const void* q,
                        const void* gate, const void* k_cache, const void* v_cache,
                        int32_t cache_capacity, const int32_t* seq_lens,
                        int32_t max_seq_len, void* out, void* stream);

/*
 * Tuning overrides, for tests and measurements only: process-wide settings
 * that later calls read when they plan their launches. value 0 restores the
 * library's own choice.
 *   HGQA_TUNE_PREFILL_WAVES      4 or 8 waves per bf16 prefill workgroup
 *                                (head_dim 128 only; other layers ignore it)
 *   HGQA_TUNE_DECODE_SPLIT_KEYS  keys per decode split (rounded up to 32)
 *   HGQA_TUNE_CHUNK_SPLIT_TILES  64-key tiles per key split of a bf16
 *                                attn_prefill_chunk (a value at or above the
 *                                longest key range means no split)
 * Returns HGQA_EINVAL for an unknown knob or value. Changing a knob while
 * another thread is inside a call gives that call either setting.
 */
enum { HGQA_TUNE_PREFILL_WAVES = 1, HGQA_TUNE_DECODE_SPLIT_KEYS = 2, HGQA_TUNE_CHUNK_SPLIT_TILES = 3 };
int hgqa_set_tuning(int32_t knob, int32_t value);

/* Text of the last error returned on the calling thread ("" if none). */
const char* hgqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HGQA_H */
