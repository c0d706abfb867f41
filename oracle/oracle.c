/*
 * Reference oracle for the Gemma-4-style hybrid sliding/global attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes is plain softmax attention written out from its
 * definition, in IEEE double precision, one query row at a time:
 *
 *   - inputs arrive as bfloat16 bit patterns and are widened exactly;
 *   - rotary position embedding (RoPE) in the rotate-half convention, pair
 *     (k, k + D/2) rotated by angle pos * theta^(-2k/D); the two theta values
 *     (1e4 for sliding layers, 1e6 for full layers) and the two head sizes
 *     (256 sliding, 512 full, full on every fifth layer) are the ones the
 *     onnxruntime-genai Gemma 4 feature request lists under "Variable
 *     Attention Head Dimensions" and "Gemma 4 Model Details";
 *   - RoPE is applied to queries and keys, never to values;
 *   - grouped-query attention: query head h reads kv head floor(h / (Hq/Hkv));
 *   - K=V aliasing (the Gemma-4 weight loader page, TP note in
 *     supports_tp: K and V share one projection slice) means the value
 *     vectors ARE the raw, un-rotated key vectors;
 *   - key j is visible from a query at position p iff j <= p, j < L and,
 *     for a sliding layer with window W > 0, p - j < W (W keys including
 *     the query's own position);
 *   - scores are scale * <RoPE(q, p), RoPE(k_j, j)>, scale = 1/sqrt(D)
 *     unless given; weights are the softmax over the visible keys; the
 *     output is the weighted sum of the value rows.
 *
 * The same definition with the extensions the pages point to next:
 *
 *   - queries at any positions of a sequence whose earlier keys are already
 *     in the cache (a chunk of a longer prompt starting at position P0, or
 *     the T > 1 tokens of a speculative-decoding verify step that reads a
 *     frozen cache: SGLang PR "Support encoder-free unified
 *     Text/Vision/Audio model", the MTP paragraph, FROZEN_KV_MTP);
 *   - a window-sized cache for sliding layers, kept as a ring: the key of
 *     position j lives in row j mod C (onnxruntime-genai feature request,
 *     "What Would Need to Change", item 2: variable-size KV cache buffers
 *     per layer);
 *   - a per-layer KV element type (Gemma-4 weight loader page,
 *     load_layers(..., layer_kv_dtypes)): bfloat16, or 8-bit floats in the
 *     OCP E4M3 encoding (bias 7, no infinities, S.1111.111 = NaN) times one
 *     scale per tensor;
 *   - bidirectional spans (image tokens; the same SGLang PR, "Config note":
 *     bidirectional image attention): a query inside a span also sees the
 *     later keys of its span, i.e. key j passes the causal test iff
 *     j <= e(p), where e(p) is the last position of p's span (p if none).
 *
 * Where the pages are silent (window boundary, scale, RoPE pairing, what
 * the cache stores, query positions) this file takes the plainest reading:
 * the design notes list each one.  No blocking, fusion or reordering is
 * done beyond the definition; OpenMP only runs independent rows in
 * parallel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL -1

#define ORC_KV_BF16 0
#define ORC_KV_FP8 1

/* Exact widening of a bfloat16 bit pattern (the top half of an IEEE binary32). */
static double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Exact value of an OCP E4M3 byte: sign, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN and
 * there are no infinities (largest finite 1.75 * 2^8 = 448). */
double orc_fp8_e4m3_to_f64(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* E4M3 code of x / scale, the element an 8-bit cache stores for the value x:
 * the quotient is taken in binary32 (the precision the library computes it
 * in), then rounded to the nearest E4M3 value (ties to the even code, i.e.
 * mantissa LSB 0); magnitudes beyond the largest finite value 448 saturate
 * to +-448.  Found by scanning the 127 finite non-negative codes. */
uint8_t orc_fp8_e4m3_quantize(float x, float scale) {
  const float qf = x / scale;
  const double q = (double)qf;
  const int neg = signbit(qf) ? 1 : 0;
  const double a = fabs(q);
  if (isnan(q)) return 0x7F;
  int best = 0;
  for (int c = 1; c < 127; ++c) {
    const double dc = fabs(orc_fp8_e4m3_to_f64((uint8_t)c) - a);
    const double db = fabs(orc_fp8_e4m3_to_f64((uint8_t)best) - a);
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)(best | (neg << 7));
}

/* RoPE inverse frequencies theta^(-2k/D), k = 0 .. D/2-1 (dual theta: the
 * caller passes the layer's own theta). */
void orc_rope_inv_freq(int32_t D, double theta, double* out) {
  for (int32_t k = 0; k < D / 2; ++k) out[k] = pow(theta, -2.0 * (double)k / (double)D);
}

/* Rotate-half RoPE of one D-vector x at position pos, given the inverse
 * frequencies f[k]:
 *   y_k       = x_k cos(a_k) - x_{k+D/2} sin(a_k)
 *   y_{k+D/2} = x_{k+D/2} cos(a_k) + x_k sin(a_k),   a_k = pos * f[k]. */
static void orc_rope_freq(const double* x, int32_t D, const double* f, double pos, double* y) {
  const int32_t half = D / 2;
  for (int32_t k = 0; k < half; ++k) {
    double a = pos * f[k];
    double c = cos(a), s = sin(a);
    double x0 = x[k], x1 = x[k + half];
    y[k] = x0 * c - x1 * s;
    y[k + half] = x1 * c + x0 * s;
  }
}

/* Public single-vector form (theta given directly). */
void orc_rope(const double* x, int32_t D, double theta, double pos, double* y) {
  double* f = (double*)malloc(sizeof(double) * (size_t)(D / 2));
  if (!f) return;
  orc_rope_inv_freq(D, theta, f);
  orc_rope_freq(x, D, f, pos, y);
  free(f);
}

/* Rotate one bfloat16 row (widened exactly) at position pos. */
static void orc_rope_row_bf16(const uint16_t* x, int32_t D, const double* f, double pos, double* tmp, double* y) {
  for (int32_t d = 0; d < D; ++d) tmp[d] = orc_bf16_to_f64(x[d]);
  orc_rope_freq(tmp, D, f, pos, y);
}

/*
 * Rows of one (batch, kv-head) cache slice: where the row of key position j
 * lives and how its elements are stored.
 *   base  : row 0 of the slice (row stride D elements)
 *   fmt   : ORC_KV_BF16 (bf16 bits) or ORC_KV_FP8 (E4M3 bytes)
 *   scale : multiplies every E4M3 element (1 for bf16)
 *   ring  : 0 = position j in row j; C > 0 = position j in row j mod C
 */
typedef struct {
  const void* base;
  int32_t fmt;
  double scale;
  int64_t ring;
} orc_rows;

/* The D elements of key/value position j, widened exactly (times the scale). */
static void orc_row(const orc_rows* c, int64_t j, int32_t D, double* out) {
  const int64_t r = c->ring > 0 ? j % c->ring : j;
  if (c->fmt == ORC_KV_FP8) {
    const uint8_t* x = (const uint8_t*)c->base + (size_t)r * D;
    for (int32_t d = 0; d < D; ++d) out[d] = orc_fp8_e4m3_to_f64(x[d]) * c->scale;
  } else {
    const uint16_t* x = (const uint16_t*)c->base + (size_t)r * D;
    for (int32_t d = 0; d < D; ++d) out[d] = orc_bf16_to_f64(x[d]);
  }
}

/* Is key j visible from a query at position p whose causal limit is e
 * (e = p, or the end of p's bidirectional span), with valid length L and
 * window W? */
static int orc_visible(int64_t j, int64_t p, int64_t e, int64_t L, int32_t W) {
  if (j < 0 || j > e || j >= L) return 0;
  if (W > 0 && p - j >= W) return 0;
  return 1;
}

/* Rotate key positions [lo, hi) of one cache slice at their own positions
 * into krot (position j at krot + j*D). */
static void orc_rotate_keys(const orc_rows* kr, int64_t lo, int64_t hi, int32_t D, const double* f, double* krot) {
#pragma omp parallel
  {
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
    for (int64_t j = lo; j < hi; ++j) {
      orc_row(kr, j, D, tmp);
      orc_rope_freq(tmp, D, f, (double)j, krot + (size_t)j * D);
    }
    free(tmp);
  }
}

/* Scores s[j] = scale*<qr, k'_j> of the visible keys j < L (-INFINITY for the
 * others); returns their maximum. */
static double orc_scores(const double* qr, const double* krot, int32_t D, int64_t p, int64_t e, int64_t L, int32_t W,
                         double scale, double* s) {
  double m = -INFINITY;
  for (int64_t j = 0; j < L; ++j) {
    if (!orc_visible(j, p, e, L, W)) { s[j] = -INFINITY; continue; }
    const double* kr = krot + (size_t)j * D;
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += qr[d] * kr[d];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  return m;
}

/*
 * Softmax attention of one rotated query qr (position p, causal limit e) over
 * the rotated keys krot (positions 0..L-1; only visible ones are read) and
 * the value rows vr: scores scale*<qr, k'_j> over visible j, softmax,
 * weighted sum of values.  weights (optional, L doubles) receives every
 * key's weight.
 */
static int orc_attend(const double* qr, const double* krot, const orc_rows* vr, int32_t D, int64_t p, int64_t e,
                      int64_t L, int32_t W, double scale, double* weights, double* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  double* v = (double*)malloc(sizeof(double) * (size_t)D);
  if (!s || !v) { free(s); free(v); return ORC_EINVAL; }
  const double m = orc_scores(qr, krot, D, p, e, L, W, scale, s);
  double denom = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
    denom += s[j];
  }
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (weights)
    for (int64_t j = 0; j < L; ++j) weights[j] = 0.0;
  if (denom > 0.0) {
    for (int64_t j = 0; j < L; ++j) {
      double w = s[j] / denom;
      if (weights) weights[j] = w;
      if (w == 0.0) continue;
      orc_row(vr, j, D, v);
      for (int32_t d = 0; d < D; ++d) out[d] += w * v[d];
    }
  }
  free(s);
  free(v);
  return denom > 0.0 ? ORC_OK : ORC_EINVAL;
}

static orc_rows orc_bf16_rows(const uint16_t* base) {
  orc_rows r = {base, ORC_KV_BF16, 1.0, 0};
  return r;
}

/*
 * One attention row (bf16 cache, one row per position).
 *   q      : D raw (pre-RoPE) query values, bf16 bits
 *   kbase  : row 0 of this (batch, kv-head) cache slice, raw keys, row stride D
 *   vbase  : row 0 of the value slice; equal to kbase for an aliased layer
 *   p      : query position;  L: valid cache length;  W: window (0 = none)
 *   weights: optional, L doubles, receives the softmax weight of every key
 *            (0 for masked keys)
 *   out    : D doubles
 */
int orc_attention_row(const uint16_t* q, const uint16_t* kbase, const uint16_t* vbase, int32_t D, int64_t p, int64_t L,
                      int32_t W, double theta, double scale, double* weights, double* out) {
  if (!q || !kbase || !vbase || !out || D <= 0 || (D & 1) || L <= 0 || p < 0) return ORC_EINVAL;
  if (scale == 0.0) scale = 1.0 / sqrt((double)D);
  const orc_rows kr = orc_bf16_rows(kbase), vr = orc_bf16_rows(vbase);
  double* f = (double*)malloc(sizeof(double) * (size_t)(D / 2));
  double* qr = (double*)malloc(sizeof(double) * (size_t)D);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  double* krot = (double*)malloc(sizeof(double) * (size_t)D * (size_t)L);
  int rc = ORC_EINVAL;
  if (f && qr && tmp && krot) {
    orc_rope_inv_freq(D, theta, f);
    orc_rope_row_bf16(q, D, f, (double)p, tmp, qr);
    for (int64_t j = 0; j < L; ++j)
      if (orc_visible(j, p, p, L, W)) {
        orc_row(&kr, j, D, tmp);
        orc_rope_freq(tmp, D, f, (double)j, krot + (size_t)j * D);
      }
    rc = orc_attend(qr, krot, &vr, D, p, p, L, W, scale, weights, out);
  }
  free(f); free(qr); free(tmp); free(krot);
  return rc;
}

/*
 * Scores of one query row (the logits softmax turns into weights): for each
 * cache row j < L, scale * <RoPE(q, p), RoPE(k_j, j)> in natural units if
 * key j is visible from position p, -INFINITY otherwise.  Arguments as for
 * orc_attention_row; scores receives L doubles.
 */
int orc_scores_row(const uint16_t* q, const uint16_t* kbase, int32_t D, int64_t p, int64_t L, int32_t W, double theta,
                   double scale, double* scores) {
  if (!q || !kbase || !scores || D <= 0 || (D & 1) || L <= 0 || p < 0) return ORC_EINVAL;
  if (scale == 0.0) scale = 1.0 / sqrt((double)D);
  const orc_rows kr = orc_bf16_rows(kbase);
  double* f = (double*)malloc(sizeof(double) * (size_t)(D / 2));
  double* qr = (double*)malloc(sizeof(double) * (size_t)D);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  double* krot = (double*)malloc(sizeof(double) * (size_t)D * (size_t)L);
  int rc = ORC_EINVAL;
  if (f && qr && tmp && krot) {
    orc_rope_inv_freq(D, theta, f);
    orc_rope_row_bf16(q, D, f, (double)p, tmp, qr);
    for (int64_t j = 0; j < L; ++j)
      if (orc_visible(j, p, p, L, W)) {
        orc_row(&kr, j, D, tmp);
        orc_rope_freq(tmp, D, f, (double)j, krot + (size_t)j * D);
      }
    orc_scores(qr, krot, D, p, p, L, W, scale, scores);
    rc = ORC_OK;
  }
  free(f); free(qr); free(tmp); free(krot);
  return rc;
}

static void orc_set_threads(int32_t nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Rows of one (batch, kv-head) cache slice: key positions [klo, khi) are
 * rotated once (each at its own position), then every listed query row
 * attends to them.
 *   qrows[i]  : pointer to the raw query row i;  qpos[i]: its position;
 *   qlim[i]   : its causal limit (qpos[i], or the end of its span);
 *   outs[i]   : its D outputs
 */
static int orc_slice(const orc_rows* kr, const orc_rows* vr, int64_t klo, int64_t khi, int64_t L, int32_t D,
                     int32_t W, double theta, double scale, int64_t nq, const uint16_t* const* qrows,
                     const int64_t* qpos, const int64_t* qlim, double* const* outs) {
  double* f = (double*)malloc(sizeof(double) * (size_t)(D / 2));
  double* krot = (double*)malloc(sizeof(double) * (size_t)D * (size_t)(khi > 0 ? khi : 1));
  if (!f || !krot) { free(f); free(krot); return ORC_EINVAL; }
  orc_rope_inv_freq(D, theta, f);
  orc_rotate_keys(kr, klo, khi, D, f, krot);
  int err = 0;
#pragma omp parallel reduction(| : err)
  {
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nq; ++i) {
      orc_rope_row_bf16(qrows[i], D, f, (double)qpos[i], tmp, qr);
      err |= orc_attend(qr, krot, vr, D, qpos[i], qlim[i], L, W, scale, NULL, outs[i]) != ORC_OK;
    }
    free(qr); free(tmp);
  }
  free(f); free(krot);
  return err ? ORC_EINVAL : ORC_OK;
}

static size_t orc_elem_bytes(int32_t fmt) { return fmt == ORC_KV_FP8 ? 1 : 2; }

/*
 * Prefill of a chunk: S query tokens at positions P0..P0+S-1 over cache
 * positions 0..P0+S-1 (keys of the earlier positions already in the cache).
 *   q        : [B, S, Hq, D] bf16 bits (raw)
 *   k        : [B, Hkv, Lmax, D] raw keys (bf16 bits, or E4M3 bytes times k_scale)
 *   v        : same shape, or NULL for an aliased layer (values = raw keys,
 *              at the key scale); E4M3 values are multiplied by v_scale
 *   span_end : NULL (causal), or [B, S]: the last position of each query's
 *              bidirectional span (its own position outside spans), with
 *              P0+s <= span_end[b][s] < P0+S
 *   out      : [B, S, Hq, D] doubles
 * Only the rows listed in `rows` (flattened b*S*Hq + s*Hq + h) are computed
 * when n_rows >= 0; then `out` holds n_rows x D values in list order.
 */
int orc_prefill_ext(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t W, double theta,
                    double scale, const uint16_t* q, const void* k, const void* v, int32_t fmt, double k_scale,
                    double v_scale, int32_t start_pos, const int32_t* span_end, const int64_t* rows, int64_t n_rows,
                    double* out, int32_t nthreads) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || start_pos < 0 || (int64_t)start_pos + S > Lmax ||
      D <= 0 || (D & 1) || !q || !k || !out || (fmt != ORC_KV_BF16 && fmt != ORC_KV_FP8))
    return ORC_EINVAL;
  if (scale == 0.0) scale = 1.0 / sqrt((double)D);
  const void* vv = v ? v : k;
  const double vs = v ? v_scale : k_scale;
  const int32_t g = Hq / Hkv;
  const int64_t L = (int64_t)start_pos + S;
  const int64_t total = (int64_t)B * S * Hq;
  const int64_t n = n_rows >= 0 ? n_rows : total;
  const size_t eb = orc_elem_bytes(fmt);
  orc_set_threads(nthreads);
  const uint16_t** qrows = (const uint16_t**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int64_t* qpos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  int64_t* qlim = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  double** outs = (double**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int err = !qrows || !qpos || !qlim || !outs;
  for (int64_t b = 0; b < B && !err; ++b)
    for (int64_t kvh = 0; kvh < Hkv && !err; ++kvh) {
      int64_t nq = 0;
      for (int64_t i = 0; i < n; ++i) {
        int64_t r = n_rows >= 0 ? rows[i] : i;
        if (r < 0 || r >= total) { err = 1; break; }
        int64_t rb = r / ((int64_t)S * Hq), s = (r / Hq) % S, h = r % Hq;
        if (rb != b || h / g != kvh) continue;
        qrows[nq] = q + (size_t)r * D;
        qpos[nq] = start_pos + s;
        qlim[nq] = span_end ? span_end[rb * S + s] : start_pos + s;
        if (qlim[nq] < qpos[nq] || qlim[nq] >= L) { err = 1; break; }
        outs[nq] = out + (size_t)i * D;
        ++nq;
      }
      if (err || nq == 0) continue;
      size_t off = ((size_t)b * Hkv + kvh) * (size_t)Lmax * D;
      const orc_rows kr = {(const char*)k + off * eb, fmt, fmt == ORC_KV_FP8 ? k_scale : 1.0, 0};
      const orc_rows vr = {(const char*)vv + off * eb, fmt, fmt == ORC_KV_FP8 ? vs : 1.0, 0};
      err |= orc_slice(&kr, &vr, 0, L, L, D, W, theta, scale, nq, qrows, qpos, qlim, outs) != ORC_OK;
    }
  free(qrows); free(qpos); free(qlim); free(outs);
  return err ? ORC_EINVAL : ORC_OK;
}

/* Prefill of a whole prompt: positions 0..S-1, bf16 cache, causal. */
int orc_prefill(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t W, double theta,
                double scale, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int64_t* rows,
                int64_t n_rows, double* out, int32_t nthreads) {
  return orc_prefill_ext(B, S, Hq, Hkv, D, Lmax, W, theta, scale, q, k, v, ORC_KV_BF16, 1.0, 1.0, 0, NULL, rows,
                         n_rows, out, nthreads);
}

/*
 * Decode of T tokens per sequence over a cache that already holds them: the
 * T queries of sequence b sit at positions kv_len[b]-T .. kv_len[b]-1 and see
 * cache positions up to their own (T = 1: one new token; T > 1: the verify
 * step of speculative decoding over a frozen cache).
 *   q    : [B, T, Hq, D] bf16 bits;  kv_len: [B] (host), T <= kv_len[b]
 *   k, v : as for orc_prefill_ext ([B, Hkv, Lmax, D], kv_len[b] <= Lmax);
 *          with ring = C > 0 the cache holds C rows per slice (Lmax = C)
 *          and position j sits in row j mod C: every visible key must still
 *          be there (kv_len[b] - C <= the first visible position)
 *   out  : [B, T, Hq, D] doubles, or n_rows x D for the listed rows
 *          (b*T + t)*Hq + h
 */
int orc_decode_ext(int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t W, double theta,
                   double scale, const uint16_t* q, const void* k, const void* v, int32_t fmt, double k_scale,
                   double v_scale, const int32_t* kv_len, int64_t ring, const int64_t* rows, int64_t n_rows,
                   double* out, int32_t nthreads) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || (D & 1) || !q || !k || !kv_len || !out ||
      ring < 0 || (ring > 0 && ring != Lmax) || (fmt != ORC_KV_BF16 && fmt != ORC_KV_FP8))
    return ORC_EINVAL;
  if (scale == 0.0) scale = 1.0 / sqrt((double)D);
  const void* vv = v ? v : k;
  const double vs = v ? v_scale : k_scale;
  const int32_t g = Hq / Hkv;
  const int64_t total = (int64_t)B * T * Hq;
  const int64_t n = n_rows >= 0 ? n_rows : total;
  const size_t eb = orc_elem_bytes(fmt);
  orc_set_threads(nthreads);
  const uint16_t** qrows = (const uint16_t**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int64_t* qpos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  double** outs = (double**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int err = !qrows || !qpos || !outs;
  for (int64_t b = 0; b < B && !err; ++b) {
    int64_t L = kv_len[b];
    if (L < T || (ring == 0 && L > Lmax)) { err = 1; break; }
    /* first position any of the T queries sees */
    int64_t lo = (W > 0 && L - T + 1 - W > 0) ? L - T + 1 - W : 0;
    if (ring > 0 && lo < L - ring) { err = 1; break; }
    for (int64_t kvh = 0; kvh < Hkv && !err; ++kvh) {
      int64_t nq = 0;
      for (int64_t i = 0; i < n; ++i) {
        int64_t r = n_rows >= 0 ? rows[i] : i;
        if (r < 0 || r >= total) { err = 1; break; }
        int64_t rb = r / ((int64_t)T * Hq), t = (r / Hq) % T, h = r % Hq;
        if (rb != b || h / g != kvh) continue;
        qrows[nq] = q + (size_t)r * D;
        qpos[nq] = L - T + t;
        outs[nq] = out + (size_t)i * D;
        ++nq;
      }
      if (err || nq == 0) continue;
      size_t off = ((size_t)b * Hkv + kvh) * (size_t)Lmax * D;
      const orc_rows kr = {(const char*)k + off * eb, fmt, fmt == ORC_KV_FP8 ? k_scale : 1.0, ring};
      const orc_rows vr = {(const char*)vv + off * eb, fmt, fmt == ORC_KV_FP8 ? vs : 1.0, ring};
      err |= orc_slice(&kr, &vr, lo, L, L, D, W, theta, scale, nq, qrows, qpos, qpos, outs) != ORC_OK;
    }
  }
  free(qrows); free(qpos); free(outs);
  return err ? ORC_EINVAL : ORC_OK;
}

/* Decode of one new token per sequence at position kv_len[b]-1, bf16 cache. */
int orc_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t W, double theta, double scale,
               const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* kv_len, const int64_t* rows,
               int64_t n_rows, double* out, int32_t nthreads) {
  return orc_decode_ext(B, 1, Hq, Hkv, D, Lmax, W, theta, scale, q, k, v, ORC_KV_BF16, 1.0, 1.0, kv_len, 0, rows,
                        n_rows, out, nthreads);
}
