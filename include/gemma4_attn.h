/*
 * gemma4_attn.h -- C ABI of the MI355X (gfx950) hybrid sliding/global
 * attention library (libgemma4_attn.so).
 *
 * The layer this library computes is the attention core of a Gemma-4-style
 * decoder stack.  Citations below name the page and its section:
 *
 *   [FR] onnxruntime-genai feature request "Support for Google Gemma 4 model
 *        family (PLE architecture, variable head dims, KV cache sharing)":
 *        "Three Architectural Blockers" (2. Variable Attention Head
 *        Dimensions, 3. KV Cache Sharing), "Gemma 4 Model Details", "What
 *        Would Need to Change" (items 1 Builder, 2 Runtime, 3 Config);
 *   [HF] Hugging Face forum post "Contributing Gemma 4 support and ONNX
 *        export optimizations", "Key Technical Contributions", item "ONNX
 *        Tracing Compatibility (GQA & MoE Attention)" (sdpa_attention_forward
 *        handing an attention operator its dual-RoPE and KV-cache
 *        parameters);
 *   [LD] Gemma-4 weight loader source page (spark_model/weight_loader/
 *        gemma4.rs): module comment, supports_tp comment, load_layers
 *        (layer_kv_dtypes), kv_layer_dims;
 *   [SG] SGLang pull request "[Model] Support encoder-free unified
 *        Text/Vision/Audio model": description (attention_k_eq_v shard
 *        duplication; sliding/global head-dim and kv-head remap; hybrid
 *        SWA).
 *
 * Semantics (the readings taken where the pages are silent):
 *   - RoPE is rotate-half: pair (k, k + D/2) turns by pos * theta^(-2k/D);
 *     it is applied to queries and keys, never to values;
 *   - caches hold RAW (un-rotated) keys; the library rotates them itself, so
 *     one buffer serves an aliased layer as both key and value;
 *   - query head h reads kv head h / (Hq / Hkv);
 *   - key j is visible from a query at position p iff j <= p and, for a
 *     window W > 0, p - j < W (W keys including the query's own position);
 *   - scores are scale * <q', k'>, scale = 1/sqrt(head_dim) when the
 *     descriptor's scale is 0; softmax over visible keys; output is the
 *     weighted sum of value rows, in fp32.
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers owned by the caller; tensors
 *     are dense, row-major, with the shapes given below; the library never
 *     allocates, frees or synchronises device memory;
 *   - compute calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream); 0 = enqueued;
 *   - arguments are validated on the host before anything is enqueued; a
 *     negative return value is one of the G4_ERR_* codes and nothing was
 *     launched; gemma4_status_string() names it and gemma4_last_error()
 *     gives the detail for the calling thread;
 *   - calls are thread-safe as long as concurrent calls use distinct
 *     workspaces and outputs;
 *   - tuning and test switches, environment variables read by every call
 *     and every workspace query (query with the settings the call will
 *     see): G4_PREFILL_ROWS=64|128 (query-tile height of head size 256),
 *     G4_PREFILL_SPLIT_PV=0|1 (head-size-512 tile schedule),
 *     G4_PREFILL_PRODUCER=0|1 (copy-issuing waves of 64-row tiles),
 *     G4_PREFILL_KPIECES=k (pieces per work unit's key range),
 *     G4_DECODE_PIECES=n (decode split, n <= 512); unset, or out of range,
 *     = the library's own choice.  They change how the work is split and
 *     scheduled, not what is computed: results agree up to fp32 rounding
 *     order.
 */
#ifndef GEMMA4_ATTN_H
#define GEMMA4_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define G4_ABI_VERSION 3

/* Status codes (library plumbing; no passage of the pages defines them). */
#define G4_OK 0
#define G4_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad index            */
#define G4_ERR_UNSUPPORTED (-2) /* head_dim not 256/512, Hq % Hkv != 0, kind    */
#define G4_ERR_BAD_SOURCE (-3)  /* kv_source_layer inconsistent (see below)     */
#define G4_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required   */
#define G4_ERR_HIP (-5)         /* the HIP runtime rejected a launch            */

/* Layer kinds: the attention_pattern values of [FR] Blocker 2 (0 = sliding,
 * 1 = full; full attention on every fifth layer, indices 4, 9, ..., 34). */
#define G4_SLIDING 0
#define G4_FULL 1

/*
 * Per-layer descriptor.  A stack of layers is an array of these; layer
 * indices below refer to positions in that array.  [FR] "What Would Need to
 * Change" item 3 asks for exactly this per-layer configuration (per-layer
 * head size, a KV sharing map); [HF] asks for an attention operator that
 * receives the RoPE and KV-cache parameters directly.
 *
 *   kind            G4_SLIDING or G4_FULL -- [FR] Blocker 2 (attention_pattern);
 *                   [LD] module comment ("Sliding + full attention pattern").
 *   head_dim        256 or 512 (anything else -> G4_ERR_UNSUPPORTED) --
 *                   [FR] Blocker 2 (head_dim 256 sliding, global_head_dim 512
 *                   full) and "What Would Need to Change" item 3.
 *   num_q_heads     Hq >= 1 -- [SG] description (the sliding/global kv-head
 *                   remap: head counts differ by layer kind).
 *   num_kv_heads    Hkv >= 1 with Hq % Hkv == 0 -- [SG] as above; [LD]
 *                   kv_layer_dims (per-layer KV dimensions).
 *   window          sliding: W > 0 keys visible including self; full: 0 --
 *                   [FR] Blocker 2 (sliding attention); [SG] "hybrid SWA".
 *                   The width convention (W keys including the query's own
 *                   position) is a reading: the pages give none.
 *   kv_alias        1: values are read from the key buffer (raw keys) --
 *                   [LD] supports_tp comment (K=V aliasing in sliding layers,
 *                   one slice serving K and V); [SG] attention_k_eq_v.
 *   kv_source_layer -1: the layer owns its cache; otherwise the index of an
 *                   EARLIER layer that owns a cache (its own source is -1)
 *                   with equal head_dim, num_kv_heads and kv_alias; the layer
 *                   then reads that layer's buffers -- [FR] Blocker 3 (35
 *                   layers, 15 unique KV caches, num_kv_shared_layers 20) and
 *                   "What Would Need to Change" items 2 (N layers -> M unique
 *                   caches) and 3 (a KV sharing map).
 *   scale           softmax scale; 0 means 1/sqrt(head_dim) -- the pages are
 *                   silent; the scale of scaled dot-product attention
 *                   ([HF], sdpa_attention_forward) is taken.
 *   rope_theta      RoPE base (> 0), e.g. 1e4 sliding, 1e6 full -- [FR]
 *                   "Gemma 4 Model Details" (separate theta values for
 *                   sliding and full attention); [LD] module comment (dual
 *                   RoPE theta).
 *   kv_dtype        element type of the layer's cache: G4_KV_BF16 (0) or
 *                   G4_KV_FP8_E4M3 (1, one byte per element in the OCP E4M3
 *                   encoding: the element's value is code * k_scale for keys,
 *                   code * v_scale for values) -- [LD] load_layers
 *                   (layer_kv_dtypes: a KV cache dtype per layer).  Must
 *                   equal the source layer's.
 *   kv_ring         0: the cache holds row j for position j ([batch, Hkv,
 *                   max_len, head_dim]); C > 0: a window-sized ring of C rows
 *                   per (batch, kv head), position j in row j mod C (sliding
 *                   layers only, C >= window; decode only) -- [FR] "What
 *                   Would Need to Change" item 2 (variable-size KV cache
 *                   buffers per layer).  Must equal the source layer's.
 *   k_scale,        G4_KV_FP8_E4M3: the per-tensor scales of the cached
 *   v_scale         keys and values (> 0; an aliased layer's values use
 *                   k_scale); a shared layer must give its source's.  Ignored
 *                   for G4_KV_BF16 -- [LD] load_layers (layer_kv_dtypes).
 */
typedef struct {
  int32_t kind;
  int32_t head_dim;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t window;
  int32_t kv_alias;
  int32_t kv_source_layer;
  float scale;
  double rope_theta;
  int32_t kv_dtype;
  int32_t kv_ring;
  float k_scale;
  float v_scale;
} g4_layer_desc;

/* Cache element types (kv_dtype). */
#define G4_KV_BF16 0
#define G4_KV_FP8_E4M3 1

/* ABI version of the loaded library (G4_ABI_VERSION at build time).  Library
 * plumbing; no passage of the pages defines it. */
int gemma4_abi_version(void);

/* Static name of a status code ("G4_OK", "G4_ERR_WORKSPACE", ...).  Library
 * plumbing. */
const char* gemma4_status_string(int status);

/* Detail message of the last failing call on this thread ("" if none).
 * Library plumbing. */
const char* gemma4_last_error(void);

/*
 * Validate a whole stack of descriptors (host only; touches no GPU state):
 * the per-layer head sizes and the KV sharing map of [FR] "What Would Need
 * to Change" item 3, checked so that every shared layer reads an earlier
 * owner of matching shape (the shape mismatch of [FR] Blocker 2 becomes an
 * error code instead of a fault).  Returns G4_OK or the first error found;
 * every entry point below runs the same checks for the layers it reads.
 */
int gemma4_validate_layers(const g4_layer_desc* layers, int32_t n_layers);

/*
 * Cache bytes a layer owns for a batch of `batch` sequences of capacity
 * `max_len` -- [FR] "What Would Need to Change" item 2 (variable-size KV
 * cache buffers per layer; N layers -> M unique caches):
 * k = batch*Hkv*max_len*head_dim*2 (bf16, layout [batch, Hkv, max_len,
 * head_dim] of raw keys), v = the same unless the layer is aliased (v = 0,
 * [LD] supports_tp).  A shared layer owns nothing (both 0).  Host only.
 */
int gemma4_kv_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch, int32_t max_len,
                    size_t* k_bytes, size_t* v_bytes);

/* Device workspace bytes gemma4_attn_prefill needs for this layer and shape
 * (rotated key and value operand tiles, arrival counters, partial results of
 * query tiles split across work-groups).  Host only.  The operation it
 * serves is cited at gemma4_attn_prefill. */
int gemma4_prefill_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                                   int32_t seq_len, size_t* bytes);

/* Device workspace bytes gemma4_attn_decode needs (split-K partial outputs
 * and log-sum-exps); max_kv_len bounds kv_len[].  Host only.  The operation
 * it serves is cited at gemma4_attn_decode. */
int gemma4_decode_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                                  int32_t max_kv_len, size_t* bytes);

/*
 * Prefill: queries at positions 0..seq_len-1 attend to cache rows
 * 0..seq_len-1 of the layer's (or its source layer's) cache.  The attention
 * operator of [HF] (sdpa_attention_forward intercepted so that the operator
 * receives positional dual-RoPE and KV-cache parameters), for the
 * per-layer head sizes of [FR] Blocker 2 and the shared caches of [FR]
 * Blocker 3.
 *   q          bf16 [batch, seq_len, Hq, head_dim], raw (pre-RoPE)
 *   k_cache    host array of n_layers device pointers; entry src(layer) is
 *              bf16 [batch, Hkv, max_len, head_dim] of raw keys whose rows
 *              0..seq_len-1 the caller has written; entries of shared layers
 *              are not read
 *   v_cache    same layout for values; not read for aliased layers (may be
 *              NULL then)
 *   out        fp32 [batch, seq_len, Hq, head_dim]
 *   workspace  device scratch of at least gemma4_prefill_workspace_bytes()
 * Requires 1 <= seq_len <= max_len.
 */
int gemma4_attn_prefill(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                        void* const* k_cache, void* const* v_cache, int32_t batch, int32_t seq_len, int32_t max_len,
                        float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode: one query per sequence at position kv_len[b]-1 attends to cache
 * rows 0..kv_len[b]-1 (only the last `window` of them for a sliding layer).
 * The current token's key/value must already be in the cache.  The same
 * attention operator as prefill ([HF]), reading the per-layer KV caches of
 * [FR] "What Would Need to Change" item 2.
 *   q          bf16 [batch, Hq, head_dim], raw (pre-RoPE)
 *   k_cache    as for prefill; rows >= kv_len[b] are never read
 *   v_cache    as for prefill
 *   kv_len     device int32 [batch], 1 <= kv_len[b] <= max_kv_len <= max_len
 *              (values outside that range give undefined results but no
 *              out-of-bounds access: they are clamped)
 *   max_kv_len host bound on kv_len[] (checked against max_len; the split
 *              of the keys over work-groups is derived from kv_len on the
 *              device, so it needs no host copy of the lengths)
 *   out        fp32 [batch, Hq, head_dim]
 *   workspace  device scratch of at least gemma4_decode_workspace_bytes()
 */
int gemma4_attn_decode(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                       void* const* k_cache, void* const* v_cache, const int32_t* kv_len, int32_t batch,
                       int32_t max_len, int32_t max_kv_len, float* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Bytes of the device scratch gemma4_attn_decode_noalloc uses in place of a
 * workspace: a static array the library holds on every GPU it runs on.
 */
#define G4_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * Decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc); no passage of the pages defines it.  Same
 * arguments, semantics and results as gemma4_attn_decode, except that the
 * split-K partials go to G4_STATIC_SCRATCH_BYTES of static device scratch
 * instead of a caller workspace.  The library allocates nothing: the
 * scratch is a file-scope device array (one per GPU, held until the process
 * ends) whose address is looked up once per device on the first call.
 *   - G4_ERR_WORKSPACE if the call needs more scratch than that
 *     (gemma4_decode_workspace_bytes() > G4_STATIC_SCRATCH_BYTES);
 *   - G4_ERR_HIP if `stream` belongs to another device than the calling
 *     thread's current device;
 *   - every call on one GPU shares that GPU's scratch and leaves the last
 *     call's partials in it: calls that may overlap on one GPU (different
 *     streams, or threads) race and must be serialised by the caller.
 */
int gemma4_attn_decode_noalloc(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                               void* const* k_cache, void* const* v_cache, const int32_t* kv_len, int32_t batch,
                               int32_t max_len, int32_t max_kv_len, float* out, void* stream);

/*
 * Options of gemma4_attn_prefill_ext: queries against a cache that already
 * holds earlier positions.  [SG] MTP paragraph (a draft reading the
 * target's frozen KV cache, FROZEN_KV_MTP) and [FR] "What Would Need to
 * Change" item 2 (the runtime's KV cache management) ask for attention
 * over an existing cache; a prompt processed in chunks is the same call.
 *   start_pos  position of query 0: the call's seq_len queries sit at
 *              positions start_pos .. start_pos + seq_len - 1 and see cache
 *              rows 0 .. start_pos + seq_len - 1 (all written by the
 *              caller); 0 is a whole prompt
 *   span_end   NULL (causal), or device int32 [batch, seq_len]: for query s
 *              the last position of its bidirectional span -- queries inside
 *              a span of image tokens also see the span's later keys ([SG]
 *              "Config note": bidirectional image attention) -- i.e. key j
 *              passes the causal test iff j <= span_end[b][s]; outside
 *              spans span_end[b][s] = start_pos + s.  Spans are disjoint
 *              intervals inside the chunk: start_pos + s <= span_end[b][s] <
 *              start_pos + seq_len (values outside are clamped into that
 *              range).  The window test is unchanged.
 *   images_ready  0, or nonzero when the workspace already holds the key and
 *              value operand images this call would build, written by an
 *              earlier prefill call into the same workspace from the same
 *              cache buffers, with the same head size, query and kv heads,
 *              kv_alias, kv_dtype, rope_theta, batch, seq_len and start_pos,
 *              under the same G4_PREFILL_* settings (the workspace layout
 *              follows the work split): the key pass is then skipped.  This serves the layers that read a cache
 *              written by an earlier layer ([FR] Blocker 3, "KV Cache
 *              Sharing": 20 of the 35 layers share the caches of layers 13
 *              and 14, and a shared layer of the same kind rotates the same
 *              raw keys with the same rope_theta), called after that layer
 *              with its workspace.  The library cannot check the claim:
 *              images of another cache give wrong results, not an error.
 */
typedef struct {
  int32_t start_pos;
  int32_t images_ready;
  const int32_t* span_end;
} g4_prefill_opts;

/*
 * Options of gemma4_attn_decode_ext.
 *   n_tokens   T >= 1 queries per sequence at positions kv_len[b] - T ..
 *              kv_len[b] - 1, each seeing the cache up to its own position
 *              (T > 1: the verify step of speculative decoding over a
 *              frozen cache, [SG] MTP paragraph, FROZEN_KV_MTP); their keys
 *              and values must already be in the cache
 *   k_new      NULL, or device bf16 [batch, n_tokens, Hkv, head_dim]: the raw
 *              keys of the T tokens; the call writes them into the cache
 *              (row of position kv_len[b] - T + t, modulo kv_ring for a
 *              ring) and attends to them as if they had been there -- the
 *              fused append a window-sized cache needs ([FR] "What Would
 *              Need to Change" item 2).  An E4M3 cache stores the code of
 *              x / scale (binary32 quotient, nearest E4M3 value with ties to
 *              even, saturating at +-448) and the attention reads those
 *              codes back
 *   v_new      likewise the values; NULL for an aliased layer (the keys are
 *              the values), required otherwise when k_new is given
 */
typedef struct {
  int32_t n_tokens;
  const void* k_new;
  const void* v_new;
} g4_decode_opts;

/* Workspace bytes of gemma4_attn_prefill_ext (opts NULL: as
 * gemma4_prefill_workspace_bytes).  The operation it serves is cited at
 * gemma4_attn_prefill_ext. */
int gemma4_prefill_ext_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                                       int32_t seq_len, const g4_prefill_opts* opts, size_t* bytes);

/*
 * Prefill of a chunk of queries against a cache holding the earlier
 * positions -- [SG] MTP paragraph (attention over a frozen cache), [FR]
 * "What Would Need to Change" item 2; otherwise as gemma4_attn_prefill.
 *   q          bf16 [batch, seq_len, Hq, head_dim], raw (pre-RoPE), query s
 *              at position start_pos + s
 *   k_cache    rows 0 .. start_pos + seq_len - 1 written by the caller
 *   out        fp32 [batch, seq_len, Hq, head_dim]
 * Requires start_pos + seq_len <= max_len.  opts NULL = start_pos 0.
 */
int gemma4_attn_prefill_ext(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                            void* const* k_cache, void* const* v_cache, int32_t batch, int32_t seq_len,
                            int32_t max_len, const g4_prefill_opts* opts, float* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Workspace bytes of gemma4_attn_decode_ext (opts NULL: as
 * gemma4_decode_workspace_bytes).  The operation it serves is cited at
 * gemma4_attn_decode_ext. */
int gemma4_decode_ext_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                                      int32_t max_kv_len, const g4_decode_opts* opts, size_t* bytes);

/*
 * Decode of n_tokens queries per sequence over its cache -- [SG] MTP
 * paragraph (the verify step over a frozen KV cache) -- optionally writing
 * their keys and values into the cache first (opts->k_new), and reading a
 * ring cache (kv_ring > 0: max_len = kv_ring, kv_len unbounded, kv_ring >=
 * window + n_tokens - 1); otherwise as gemma4_attn_decode.
 *   q          bf16 [batch, n_tokens, Hq, head_dim], raw; token t of
 *              sequence b at position kv_len[b] - n_tokens + t
 *   kv_len     device int32 [batch], n_tokens <= kv_len[b] <= max_kv_len
 *              (values outside are clamped: undefined results, no
 *              out-of-bounds access)
 *   out        fp32 [batch, n_tokens, Hq, head_dim]
 * Requires n_tokens <= max_kv_len <= max_len.  opts NULL = one token.
 */
int gemma4_attn_decode_ext(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                           void* const* k_cache, void* const* v_cache, const int32_t* kv_len, int32_t batch,
                           int32_t max_len, int32_t max_kv_len, const g4_decode_opts* opts, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Profiling aid (not part of the attention computation; no passage of the
 * pages defines it).  After this call, each compute call made on the
 * calling thread records `before` on its stream immediately before
 * launching its main attention kernel (prefill: the kernel after the
 * key-rotation pass; decode: the split-K kernel before the merge) and
 * `after` immediately after it.  The events are caller-owned hipEvent_t
 * handles passed as void*; NULL, NULL turns recording off.
 * Returns G4_OK, or G4_ERR_INVALID_ARG if exactly one of the two is NULL.
 */
int gemma4_set_profile_events(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA4_ATTN_H */
