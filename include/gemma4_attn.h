/*
 * gemma4_attn.h -- C ABI of the MI355X (gfx950) hybrid sliding/global
 * attention library (libgemma4_attn.so).
 *
 * The layer this library computes is the attention core of a Gemma-4-style
 * decoder stack:
 *   - sliding-window layers with head size 256 and full-attention layers
 *     with head size 512 on every fifth layer, each with its own RoPE theta
 *     (1e4 sliding, 1e6 full), and 35 layers that read only 15 distinct KV
 *     caches -- onnxruntime-genai feature request "Support for Google Gemma 4
 *     model family (PLE architecture, variable head dims, KV cache sharing)",
 *     sections "Variable Attention Head Dimensions", "KV Cache Sharing",
 *     "Gemma 4 Model Details" and "What Would Need to Change" (per-layer head
 *     size, a KV sharing map, per-layer cache buffers);
 *   - K=V aliasing in sliding layers, where one projection serves as both
 *     key and value -- Gemma-4 weight loader page
 *     (spark_model/weight_loader/gemma4.rs), comment in supports_tp; SGLang
 *     PR "Support encoder-free unified Text/Vision/Audio model",
 *     attention_k_eq_v;
 *   - an attention operator that receives the RoPE and KV-cache parameters
 *     directly -- Hugging Face forum post "Contributing Gemma 4 support and
 *     ONNX export optimizations", ONNX tracing item on sdpa_attention_forward.
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
 *     workspaces and outputs.
 */
#ifndef GEMMA4_ATTN_H
#define GEMMA4_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define G4_ABI_VERSION 1

/* Status codes. */
#define G4_OK 0
#define G4_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad index            */
#define G4_ERR_UNSUPPORTED (-2) /* head_dim not 256/512, Hq % Hkv != 0, kind    */
#define G4_ERR_BAD_SOURCE (-3)  /* kv_source_layer inconsistent (see below)     */
#define G4_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required   */
#define G4_ERR_HIP (-5)         /* the HIP runtime rejected a launch            */

/* Layer kinds (attention_pattern: 0 = sliding, 1 = full). */
#define G4_SLIDING 0
#define G4_FULL 1

/*
 * Per-layer descriptor.  A stack of layers is an array of these; layer
 * indices below refer to positions in that array.
 *   kind            G4_SLIDING or G4_FULL
 *   head_dim        256 or 512 (anything else -> G4_ERR_UNSUPPORTED)
 *   num_q_heads     Hq >= 1
 *   num_kv_heads    Hkv >= 1 with Hq % Hkv == 0
 *   window          sliding: W > 0 keys visible including self; full: 0
 *   kv_alias        1: values are read from the key buffer (raw keys)
 *   kv_source_layer -1: the layer owns its cache; otherwise the index of an
 *                   EARLIER layer that owns a cache (its own source is -1)
 *                   with equal head_dim, num_kv_heads and kv_alias; the layer
 *                   then reads that layer's buffers
 *   scale           softmax scale; 0 means 1/sqrt(head_dim)
 *   rope_theta      RoPE base (> 0), e.g. 1e4 sliding, 1e6 full
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
} g4_layer_desc;

/* ABI version of the loaded library (G4_ABI_VERSION at build time). */
int gemma4_abi_version(void);

/* Static name of a status code ("G4_OK", "G4_ERR_WORKSPACE", ...). */
const char* gemma4_status_string(int status);

/* Detail message of the last failing call on this thread ("" if none). */
const char* gemma4_last_error(void);

/*
 * Validate a whole stack of descriptors (host only; touches no GPU state).
 * Returns G4_OK or the first error found; every entry point below runs the
 * same checks for the layers it reads.
 */
int gemma4_validate_layers(const g4_layer_desc* layers, int32_t n_layers);

/*
 * Cache bytes a layer owns for a batch of `batch` sequences of capacity
 * `max_len`: k = batch*Hkv*max_len*head_dim*2 (bf16), v = the same unless the
 * layer is aliased (v = 0).  A shared layer owns nothing (both 0).
 */
int gemma4_kv_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch, int32_t max_len,
                    size_t* k_bytes, size_t* v_bytes);

/* Device workspace bytes gemma4_attn_prefill needs for this layer and shape. */
int gemma4_prefill_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                                   int32_t seq_len, size_t* bytes);

/* Device workspace bytes gemma4_attn_decode needs; max_kv_len bounds kv_len[]. */
int gemma4_decode_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                                  int32_t max_kv_len, size_t* bytes);

/*
 * Prefill: queries at positions 0..seq_len-1 attend to cache rows
 * 0..seq_len-1 of the layer's (or its source layer's) cache.
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
 * The current token's key/value must already be in the cache.
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
 * Profiling aid (not part of the attention computation).  After this call,
 * each compute call made on the calling thread records `before` on its
 * stream immediately before launching its main attention kernel (prefill:
 * the kernel after the key-rotation pass; decode: the split-K kernel before
 * the merge) and `after` immediately after it.  The events are caller-owned
 * hipEvent_t handles passed as void*; NULL, NULL turns recording off.
 * Returns G4_OK, or G4_ERR_INVALID_ARG if exactly one of the two is NULL.
 */
int gemma4_set_profile_events(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA4_ATTN_H */
