// C-ABI entry points of libgemma4_attn.so (declared in include/gemma4_attn.h).
//
// Host-side work only: descriptor validation, resolution of the KV-cache
// source layer (N layers reading M < N caches, the sharing map the
// onnxruntime-genai Gemma 4 feature request asks for under "What Would Need
// to Change"), workspace sizing and dispatch to the kernel launchers.  The
// validation and sizing functions never call the HIP runtime, so they can
// be exercised on a machine without a GPU.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/gemma4_attn.h"
#include "g4_internal.h"

#define G4_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";
thread_local g4::ProfileEvents g_profile;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return G4_OK;
}

// Checks of one descriptor on its own.
int check_desc(const g4_layer_desc& d, int idx) {
  if (d.kind != G4_SLIDING && d.kind != G4_FULL) return fail(G4_ERR_UNSUPPORTED, "layer %d: kind %d", idx, d.kind);
  if (d.head_dim != 256 && d.head_dim != 512)
    return fail(G4_ERR_UNSUPPORTED, "layer %d: head_dim %d (supported: 256, 512)", idx, d.head_dim);
  if (d.num_q_heads < 1 || d.num_kv_heads < 1)
    return fail(G4_ERR_INVALID_ARG, "layer %d: head counts %d/%d", idx, d.num_q_heads, d.num_kv_heads);
  if (d.num_q_heads % d.num_kv_heads != 0)
    return fail(G4_ERR_UNSUPPORTED, "layer %d: num_q_heads %d not a multiple of num_kv_heads %d", idx,
                d.num_q_heads, d.num_kv_heads);
  if (d.kind == G4_SLIDING && d.window <= 0)
    return fail(G4_ERR_INVALID_ARG, "layer %d: sliding layer needs window > 0 (got %d)", idx, d.window);
  if (d.kind == G4_FULL && d.window != 0)
    return fail(G4_ERR_INVALID_ARG, "layer %d: full layer must have window 0 (got %d)", idx, d.window);
  if (d.kv_alias != 0 && d.kv_alias != 1) return fail(G4_ERR_INVALID_ARG, "layer %d: kv_alias %d", idx, d.kv_alias);
  if (!(d.rope_theta > 0.0) || !std::isfinite(d.rope_theta))
    return fail(G4_ERR_INVALID_ARG, "layer %d: rope_theta %g", idx, d.rope_theta);
  if (!(d.scale >= 0.f) || !std::isfinite(d.scale)) return fail(G4_ERR_INVALID_ARG, "layer %d: scale %g", idx, d.scale);
  if (d.kv_dtype != G4_KV_BF16 && d.kv_dtype != G4_KV_FP8_E4M3)
    return fail(G4_ERR_UNSUPPORTED, "layer %d: kv_dtype %d", idx, d.kv_dtype);
  if (d.kv_dtype == G4_KV_FP8_E4M3 &&
      (!(d.k_scale > 0.f) || !std::isfinite(d.k_scale) || !(d.v_scale > 0.f) || !std::isfinite(d.v_scale)))
    return fail(G4_ERR_INVALID_ARG, "layer %d: E4M3 scales %g / %g", idx, d.k_scale, d.v_scale);
  if (d.kv_ring < 0) return fail(G4_ERR_INVALID_ARG, "layer %d: kv_ring %d", idx, d.kv_ring);
  if (d.kv_ring > 0 && (d.kind != G4_SLIDING || d.kv_ring < d.window))
    return fail(G4_ERR_INVALID_ARG, "layer %d: a ring cache (kv_ring %d) needs a sliding layer with window <= kv_ring",
                idx, d.kv_ring);
  return G4_OK;
}

// Full check of layer `idx` within its stack, including its cache source.
int check_layer(const g4_layer_desc* layers, int32_t n_layers, int32_t idx) {
  if (!layers) return fail(G4_ERR_INVALID_ARG, "layers is NULL");
  if (n_layers < 1) return fail(G4_ERR_INVALID_ARG, "n_layers %d", n_layers);
  if (idx < 0 || idx >= n_layers) return fail(G4_ERR_INVALID_ARG, "layer %d out of range [0, %d)", idx, n_layers);
  const g4_layer_desc& d = layers[idx];
  int rc = check_desc(d, idx);
  if (rc) return rc;
  const int s = d.kv_source_layer;
  if (s == -1) return G4_OK;
  if (s < 0 || s >= idx)
    return fail(G4_ERR_BAD_SOURCE, "layer %d: kv_source_layer %d must be -1 or an earlier layer", idx, s);
  const g4_layer_desc& src = layers[s];
  rc = check_desc(src, s);
  if (rc) return rc;
  if (src.kv_source_layer != -1)
    return fail(G4_ERR_BAD_SOURCE, "layer %d: source layer %d does not own a cache", idx, s);
  if (src.head_dim != d.head_dim || src.num_kv_heads != d.num_kv_heads || src.kv_alias != d.kv_alias)
    return fail(G4_ERR_BAD_SOURCE, "layer %d: source layer %d has head_dim/num_kv_heads/kv_alias %d/%d/%d, needs %d/%d/%d",
                idx, s, src.head_dim, src.num_kv_heads, src.kv_alias, d.head_dim, d.num_kv_heads, d.kv_alias);
  if (src.kv_dtype != d.kv_dtype || src.kv_ring != d.kv_ring)
    return fail(G4_ERR_BAD_SOURCE, "layer %d: source layer %d has kv_dtype/kv_ring %d/%d, needs %d/%d", idx, s,
                src.kv_dtype, src.kv_ring, d.kv_dtype, d.kv_ring);
  if (d.kv_dtype == G4_KV_FP8_E4M3 && (src.k_scale != d.k_scale || src.v_scale != d.v_scale))
    return fail(G4_ERR_BAD_SOURCE, "layer %d: source layer %d stores its cache with scales %g / %g, not %g / %g", idx,
                s, src.k_scale, src.v_scale, d.k_scale, d.v_scale);
  return G4_OK;
}

int source_of(const g4_layer_desc* layers, int32_t idx) {
  return layers[idx].kv_source_layer < 0 ? idx : layers[idx].kv_source_layer;
}

float resolved_scale(const g4_layer_desc& d) {
  return d.scale > 0.f ? d.scale : (float)(1.0 / std::sqrt((double)d.head_dim));
}


}  // namespace

G4_EXPORT int gemma4_abi_version(void) { return G4_ABI_VERSION; }

G4_EXPORT const char* gemma4_status_string(int status) {
  switch (status) {
    case G4_OK: return "G4_OK";
    case G4_ERR_INVALID_ARG: return "G4_ERR_INVALID_ARG";
    case G4_ERR_UNSUPPORTED: return "G4_ERR_UNSUPPORTED";
    case G4_ERR_BAD_SOURCE: return "G4_ERR_BAD_SOURCE";
    case G4_ERR_WORKSPACE: return "G4_ERR_WORKSPACE";
    case G4_ERR_HIP: return "G4_ERR_HIP";
    default: return "G4_ERR_UNKNOWN";
  }
}

G4_EXPORT const char* gemma4_last_error(void) { return g_last_error; }

G4_EXPORT int gemma4_validate_layers(const g4_layer_desc* layers, int32_t n_layers) {
  if (!layers) return fail(G4_ERR_INVALID_ARG, "layers is NULL");
  if (n_layers < 1) return fail(G4_ERR_INVALID_ARG, "n_layers %d", n_layers);
  for (int32_t i = 0; i < n_layers; ++i) {
    const int rc = check_layer(layers, n_layers, i);
    if (rc) return rc;
  }
  return ok();
}

G4_EXPORT int gemma4_kv_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch,
                              int32_t max_len, size_t* k_bytes, size_t* v_bytes) {
  int rc = check_layer(layers, n_layers, layer);
  if (rc) return rc;
  if (!k_bytes || !v_bytes) return fail(G4_ERR_INVALID_ARG, "output pointer is NULL");
  if (batch < 1 || max_len < 1) return fail(G4_ERR_INVALID_ARG, "batch %d, max_len %d", batch, max_len);
  const g4_layer_desc& d = layers[layer];
  if (d.kv_source_layer >= 0) {
    *k_bytes = *v_bytes = 0;
    return ok();
  }
  const size_t rows = d.kv_ring > 0 ? (size_t)d.kv_ring : (size_t)max_len;  // a ring holds kv_ring rows
  const size_t elem = d.kv_dtype == G4_KV_FP8_E4M3 ? 1 : 2;
  const size_t bytes = (size_t)batch * d.num_kv_heads * rows * d.head_dim * elem;
  *k_bytes = bytes;
  *v_bytes = d.kv_alias ? 0 : bytes;
  return ok();
}

namespace {

const g4_prefill_opts kPrefillDefaults = {0, 0, nullptr};
const g4_decode_opts kDecodeDefaults = {1, nullptr, nullptr};

int check_prefill_opts(const g4_prefill_opts& o) {
  if (o.start_pos < 0) return fail(G4_ERR_INVALID_ARG, "start_pos %d", o.start_pos);
  return G4_OK;
}

int check_decode_opts(const g4_decode_opts& o) {
  if (o.n_tokens < 1) return fail(G4_ERR_INVALID_ARG, "n_tokens %d", o.n_tokens);
  if (!o.k_new && o.v_new) return fail(G4_ERR_INVALID_ARG, "v_new given without k_new");
  return G4_OK;
}

int prefill_ws(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch, int32_t seq_len,
               const g4_prefill_opts& o, size_t* bytes) {
  int rc = check_layer(layers, n_layers, layer);
  if (rc) return rc;
  if (!bytes) return fail(G4_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || seq_len < 1) return fail(G4_ERR_INVALID_ARG, "batch %d, seq_len %d", batch, seq_len);
  if ((rc = check_prefill_opts(o))) return rc;
  const g4_layer_desc& d = layers[layer];
  *bytes = g4::prefill_workspace(batch, seq_len, d.num_q_heads, d.num_kv_heads, d.head_dim,
                                 d.kind == G4_SLIDING ? d.window : 0, o.start_pos);
  return ok();
}

int decode_ws(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, int32_t batch, int32_t max_kv_len,
              const g4_decode_opts& o, size_t* bytes) {
  int rc = check_layer(layers, n_layers, layer);
  if (rc) return rc;
  if (!bytes) return fail(G4_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || max_kv_len < 1) return fail(G4_ERR_INVALID_ARG, "batch %d, max_kv_len %d", batch, max_kv_len);
  if ((rc = check_decode_opts(o))) return rc;
  const g4_layer_desc& d = layers[layer];
  const g4::DecodePlan plan = g4::plan_decode(batch, d.num_kv_heads, d.window, max_kv_len);
  *bytes = g4::decode_workspace(batch, d.num_q_heads, d.num_kv_heads, d.head_dim, o.n_tokens, plan);
  return ok();
}

}  // namespace

G4_EXPORT int gemma4_prefill_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer,
                                             int32_t batch, int32_t seq_len, size_t* bytes) {
  return prefill_ws(layers, n_layers, layer, batch, seq_len, kPrefillDefaults, bytes);
}

G4_EXPORT int gemma4_prefill_ext_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer,
                                                 int32_t batch, int32_t seq_len, const g4_prefill_opts* opts,
                                                 size_t* bytes) {
  return prefill_ws(layers, n_layers, layer, batch, seq_len, opts ? *opts : kPrefillDefaults, bytes);
}

G4_EXPORT int gemma4_decode_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer,
                                            int32_t batch, int32_t max_kv_len, size_t* bytes) {
  return decode_ws(layers, n_layers, layer, batch, max_kv_len, kDecodeDefaults, bytes);
}

G4_EXPORT int gemma4_decode_ext_workspace_bytes(const g4_layer_desc* layers, int32_t n_layers, int32_t layer,
                                                int32_t batch, int32_t max_kv_len, const g4_decode_opts* opts,
                                                size_t* bytes) {
  return decode_ws(layers, n_layers, layer, batch, max_kv_len, opts ? *opts : kDecodeDefaults, bytes);
}

namespace {

int prefill_call(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q, void* const* k_cache,
                 void* const* v_cache, int32_t batch, int32_t seq_len, int32_t max_len, const g4_prefill_opts& o,
                 float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layer(layers, n_layers, layer);
  if (rc) return rc;
  if ((rc = check_prefill_opts(o))) return rc;
  const g4_layer_desc& d = layers[layer];
  if (d.kv_ring > 0)
    return fail(G4_ERR_UNSUPPORTED, "layer %d: prefill reads a cache of one row per position, not a ring", layer);
  if (batch < 1 || seq_len < 1 || (long long)o.start_pos + seq_len > max_len)
    return fail(G4_ERR_INVALID_ARG, "batch %d, seq_len %d, start_pos %d, max_len %d", batch, seq_len, o.start_pos,
                max_len);
  if ((long long)seq_len * (d.num_q_heads / d.num_kv_heads) > 0x7fffffffLL)
    return fail(G4_ERR_INVALID_ARG, "seq_len %d too large", seq_len);
  if (!q || !out || !k_cache) return fail(G4_ERR_INVALID_ARG, "q/out/k_cache is NULL");
  const int src = source_of(layers, layer);
  const void* k = k_cache[src];
  const void* v = d.kv_alias ? k : (v_cache ? v_cache[src] : nullptr);
  if (!k) return fail(G4_ERR_INVALID_ARG, "k_cache[%d] is NULL", src);
  if (!v) return fail(G4_ERR_INVALID_ARG, "v_cache[%d] is NULL for a layer without K=V aliasing", src);
  const size_t need = g4::prefill_workspace(batch, seq_len, d.num_q_heads, d.num_kv_heads, d.head_dim,
                                            d.kind == G4_SLIDING ? d.window : 0, o.start_pos);
  if (!workspace || workspace_bytes < need)
    return fail(G4_ERR_WORKSPACE, "prefill workspace %zu bytes, needs %zu", workspace ? workspace_bytes : 0, need);
  g4::PrefillLaunch p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.kimg = workspace;
  p.B = batch;
  p.S = seq_len;
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.D = d.head_dim;
  p.Lmax = max_len;
  p.W = d.kind == G4_SLIDING ? d.window : 0;
  p.P0 = o.start_pos;
  p.span_end = o.span_end;
  p.images_ready = o.images_ready != 0;
  p.fp8 = d.kv_dtype == G4_KV_FP8_E4M3;
  p.k_scale = p.fp8 ? d.k_scale : 1.f;
  p.v_scale = p.fp8 ? (d.kv_alias ? d.k_scale : d.v_scale) : 1.f;
  p.scale = resolved_scale(d);
  p.theta = d.rope_theta;
  const hipError_t e = g4::launch_prefill(p, static_cast<hipStream_t>(stream), g_profile);
  if (e != hipSuccess) return fail(G4_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

G4_EXPORT int gemma4_attn_prefill(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                                  void* const* k_cache, void* const* v_cache, int32_t batch, int32_t seq_len,
                                  int32_t max_len, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_call(layers, n_layers, layer, q, k_cache, v_cache, batch, seq_len, max_len, kPrefillDefaults, out,
                      workspace, workspace_bytes, stream);
}

G4_EXPORT int gemma4_attn_prefill_ext(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                                      void* const* k_cache, void* const* v_cache, int32_t batch, int32_t seq_len,
                                      int32_t max_len, const g4_prefill_opts* opts, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return prefill_call(layers, n_layers, layer, q, k_cache, v_cache, batch, seq_len, max_len,
                      opts ? *opts : kPrefillDefaults, out, workspace, workspace_bytes, stream);
}

namespace {

// Checks and launch of one decode call; `workspace` NULL means the static
// device scratch (checked against its size before anything touches the GPU).
int decode_call(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q, void* const* k_cache,
                void* const* v_cache, const int32_t* kv_len, int32_t batch, int32_t max_len, int32_t max_kv_len,
                const g4_decode_opts& o, float* out, void* workspace, size_t workspace_bytes, void* stream,
                bool use_static) {
  int rc = check_layer(layers, n_layers, layer);
  if (rc) return rc;
  if ((rc = check_decode_opts(o))) return rc;
  const g4_layer_desc& d = layers[layer];
  if (batch < 1 || max_kv_len < o.n_tokens || (d.kv_ring == 0 && max_len < max_kv_len))
    return fail(G4_ERR_INVALID_ARG, "batch %d, max_len %d, max_kv_len %d, n_tokens %d", batch, max_len, max_kv_len,
                o.n_tokens);
  if (d.kv_ring > 0 && max_len != d.kv_ring)
    return fail(G4_ERR_INVALID_ARG, "layer %d: a ring cache of %d rows, max_len %d", layer, d.kv_ring, max_len);
  if (d.kv_ring > 0 && (long long)d.window + o.n_tokens - 1 > d.kv_ring)
    return fail(G4_ERR_INVALID_ARG, "layer %d: %d tokens with window %d need a ring of %d rows (has %d)", layer,
                o.n_tokens, d.window, d.window + o.n_tokens - 1, d.kv_ring);
  if (o.k_new && d.kv_alias && o.v_new)
    return fail(G4_ERR_INVALID_ARG, "layer %d: v_new given for a K=V layer", layer);
  if (o.k_new && !d.kv_alias && !o.v_new) return fail(G4_ERR_INVALID_ARG, "layer %d: v_new missing", layer);
  if (!q || !out || !k_cache || !kv_len) return fail(G4_ERR_INVALID_ARG, "q/out/k_cache/kv_len is NULL");
  const int src = source_of(layers, layer);
  void* k = k_cache[src];
  void* v = d.kv_alias ? k : (v_cache ? v_cache[src] : nullptr);
  if (!k) return fail(G4_ERR_INVALID_ARG, "k_cache[%d] is NULL", src);
  if (!v) return fail(G4_ERR_INVALID_ARG, "v_cache[%d] is NULL for a layer without K=V aliasing", src);
  const int W = d.kind == G4_SLIDING ? d.window : 0;
  const g4::DecodePlan plan = g4::plan_decode(batch, d.num_kv_heads, W, max_kv_len);
  const size_t need = g4::decode_workspace(batch, d.num_q_heads, d.num_kv_heads, d.head_dim, o.n_tokens, plan);
  if (use_static) {
    if (need > g4::kStaticScratchBytes)
      return fail(G4_ERR_WORKSPACE, "decode needs %zu bytes of scratch, the static scratch holds %zu", need,
                  g4::kStaticScratchBytes);
    const hipError_t e = g4::static_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess) return fail(G4_ERR_HIP, "static scratch: %s", hipGetErrorString(e));
  } else if (!workspace || workspace_bytes < need) {
    return fail(G4_ERR_WORKSPACE, "decode workspace %zu bytes, needs %zu", workspace ? workspace_bytes : 0, need);
  }
  g4::DecodeLaunch p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.kv_len = kv_len;
  p.out = out;
  p.ws = workspace;
  p.B = batch;
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.D = d.head_dim;
  p.Lmax = max_len;
  p.W = W;
  p.alias = d.kv_alias;
  p.T = o.n_tokens;
  p.ring = d.kv_ring;
  p.fp8 = d.kv_dtype == G4_KV_FP8_E4M3;
  p.k_scale = p.fp8 ? d.k_scale : 1.f;
  p.v_scale = p.fp8 ? (d.kv_alias ? d.k_scale : d.v_scale) : 1.f;
  p.k_new = o.k_new;
  p.v_new = d.kv_alias ? o.k_new : o.v_new;
  p.scale = resolved_scale(d);
  p.theta = d.rope_theta;
  p.plan = plan;
  const hipError_t e = g4::launch_decode(p, static_cast<hipStream_t>(stream), g_profile);
  if (e != hipSuccess) return fail(G4_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

G4_EXPORT int gemma4_attn_decode(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                                 void* const* k_cache, void* const* v_cache, const int32_t* kv_len, int32_t batch,
                                 int32_t max_len, int32_t max_kv_len, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return decode_call(layers, n_layers, layer, q, k_cache, v_cache, kv_len, batch, max_len, max_kv_len,
                     kDecodeDefaults, out, workspace, workspace_bytes, stream, false);
}

G4_EXPORT int gemma4_attn_decode_ext(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                                     void* const* k_cache, void* const* v_cache, const int32_t* kv_len, int32_t batch,
                                     int32_t max_len, int32_t max_kv_len, const g4_decode_opts* opts, float* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(layers, n_layers, layer, q, k_cache, v_cache, kv_len, batch, max_len, max_kv_len,
                     opts ? *opts : kDecodeDefaults, out, workspace, workspace_bytes, stream, false);
}

G4_EXPORT int gemma4_attn_decode_noalloc(const g4_layer_desc* layers, int32_t n_layers, int32_t layer, const void* q,
                                         void* const* k_cache, void* const* v_cache, const int32_t* kv_len,
                                         int32_t batch, int32_t max_len, int32_t max_kv_len, float* out,
                                         void* stream) {
  return decode_call(layers, n_layers, layer, q, k_cache, v_cache, kv_len, batch, max_len, max_kv_len,
                     kDecodeDefaults, out, nullptr, 0, stream, true);
}

G4_EXPORT int gemma4_set_profile_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(G4_ERR_INVALID_ARG, "profile events must both be set or both be NULL");
  g_profile.before = static_cast<hipEvent_t>(before);
  g_profile.after = static_cast<hipEvent_t>(after);
  return ok();
}
