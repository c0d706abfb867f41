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

/* Exact widening of a bfloat16 bit pattern (the top half of an IEEE binary32). */
static double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
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

/* Is key j visible from a query at position p with valid length L and window W? */
static int orc_visible(int64_t j, int64_t p, int64_t L, int32_t W) {
  if (j < 0 || j > p || j >= L) return 0;
  if (W > 0 && p - j >= W) return 0;
  return 1;
}

/* Rotate key rows [lo, hi) of one cache slice (raw keys, row stride D) at
 * their own positions into krot (row j at krot + j*D). */
static void orc_rotate_keys(const uint16_t* kbase, int64_t lo, int64_t hi, int32_t D, const double* f,
                            double* krot) {
#pragma omp parallel
  {
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
    for (int64_t j = lo; j < hi; ++j)
      orc_rope_row_bf16(kbase + (size_t)j * D, D, f, (double)j, tmp, krot + (size_t)j * D);
    free(tmp);
  }
}

/*
 * Softmax attention of one rotated query qr (position p) over the rotated
 * keys krot (rows 0..L-1; only visible rows are read) and the raw value rows
 * vbase: scores scale*<qr, k'_j> over visible j, softmax, weighted sum of
 * values.  weights (optional, L doubles) receives every key's weight.
 */
static int orc_attend(const double* qr, const double* krot, const uint16_t* vbase, int32_t D, int64_t p, int64_t L,
                      int32_t W, double scale, double* weights, double* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  if (!s) return ORC_EINVAL;
  double m = -INFINITY;
  for (int64_t j = 0; j < L; ++j) {
    if (!orc_visible(j, p, L, W)) { s[j] = -INFINITY; continue; }
    const double* kr = krot + (size_t)j * D;
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += qr[d] * kr[d];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
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
      const uint16_t* v = vbase + (size_t)j * (size_t)D;
      for (int32_t d = 0; d < D; ++d) out[d] += w * orc_bf16_to_f64(v[d]);
    }
  }
  free(s);
  return denom > 0.0 ? ORC_OK : ORC_EINVAL;
}

/*
 * One attention row.
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
  double* f = (double*)malloc(sizeof(double) * (size_t)(D / 2));
  double* qr = (double*)malloc(sizeof(double) * (size_t)D);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  double* krot = (double*)malloc(sizeof(double) * (size_t)D * (size_t)L);
  int rc = ORC_EINVAL;
  if (f && qr && tmp && krot) {
    orc_rope_inv_freq(D, theta, f);
    orc_rope_row_bf16(q, D, f, (double)p, tmp, qr);
    for (int64_t j = 0; j < L; ++j)
      if (orc_visible(j, p, L, W)) orc_rope_row_bf16(kbase + (size_t)j * D, D, f, (double)j, tmp, krot + (size_t)j * D);
    rc = orc_attend(qr, krot, vbase, D, p, L, W, scale, weights, out);
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
 * Rows of one (batch, kv-head) cache slice: keys [klo, khi) are rotated once
 * (each at its own position), then every listed query row attends to them.
 *   qrows[i]  : pointer to the raw query row i;  qpos[i]: its position
 *   outs[i]   : its D outputs
 */
static int orc_slice(const uint16_t* kbase, const uint16_t* vbase, int64_t klo, int64_t khi, int64_t L, int32_t D,
                     int32_t W, double theta, double scale, int64_t nq, const uint16_t* const* qrows,
                     const int64_t* qpos, double* const* outs) {
  double* f = (double*)malloc(sizeof(double) * (size_t)(D / 2));
  double* krot = (double*)malloc(sizeof(double) * (size_t)D * (size_t)(khi > 0 ? khi : 1));
  if (!f || !krot) { free(f); free(krot); return ORC_EINVAL; }
  orc_rope_inv_freq(D, theta, f);
  orc_rotate_keys(kbase, klo, khi, D, f, krot);
  int err = 0;
#pragma omp parallel reduction(| : err)
  {
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nq; ++i) {
      orc_rope_row_bf16(qrows[i], D, f, (double)qpos[i], tmp, qr);
      err |= orc_attend(qr, krot, vbase, D, qpos[i], L, W, scale, NULL, outs[i]) != ORC_OK;
    }
    free(qr); free(tmp);
  }
  free(f); free(krot);
  return err ? ORC_EINVAL : ORC_OK;
}

/*
 * Prefill: query positions 0..S-1 over cache rows 0..S-1.
 *   q   : [B, S, Hq, D] bf16 bits (raw)
 *   k   : [B, Hkv, Lmax, D] bf16 bits (raw keys)
 *   v   : same shape, or NULL for an aliased layer (values = raw keys)
 *   out : [B, S, Hq, D] doubles
 * Only the rows listed in `rows` (flattened b*S*Hq + s*Hq + h) are computed
 * when n_rows >= 0; then `out` holds n_rows x D values in list order.
 */
int orc_prefill(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t W, double theta,
                double scale, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int64_t* rows,
                int64_t n_rows, double* out, int32_t nthreads) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || S > Lmax || D <= 0 || (D & 1) || !q || !k || !out)
    return ORC_EINVAL;
  if (scale == 0.0) scale = 1.0 / sqrt((double)D);
  const uint16_t* vv = v ? v : k;
  const int32_t g = Hq / Hkv;
  const int64_t total = (int64_t)B * S * Hq;
  const int64_t n = n_rows >= 0 ? n_rows : total;
  orc_set_threads(nthreads);
  const uint16_t** qrows = (const uint16_t**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int64_t* qpos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  double** outs = (double**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int err = !qrows || !qpos || !outs;
  for (int64_t b = 0; b < B && !err; ++b)
    for (int64_t kvh = 0; kvh < Hkv && !err; ++kvh) {
      int64_t nq = 0;
      for (int64_t i = 0; i < n; ++i) {
        int64_t r = n_rows >= 0 ? rows[i] : i;
        if (r < 0 || r >= total) { err = 1; break; }
        int64_t rb = r / ((int64_t)S * Hq), s = (r / Hq) % S, h = r % Hq;
        if (rb != b || h / g != kvh) continue;
        qrows[nq] = q + (size_t)r * D;
        qpos[nq] = s;
        outs[nq] = out + (size_t)i * D;
        ++nq;
      }
      if (err || nq == 0) continue;
      size_t off = ((size_t)b * Hkv + kvh) * (size_t)Lmax * D;
      err |= orc_slice(k + off, vv + off, 0, S, S, D, W, theta, scale, nq, qrows, qpos, outs) != ORC_OK;
    }
  free(qrows); free(qpos); free(outs);
  return err ? ORC_EINVAL : ORC_OK;
}

/*
 * Decode: one query per sequence at position kv_len[b]-1 over cache rows
 * 0..kv_len[b]-1 (the current token's key/value already in the cache).
 *   q   : [B, Hq, D] bf16 bits;  kv_len: [B] (host)
 *   out : [B, Hq, D] doubles, or n_rows x D for the listed rows b*Hq + h
 */
int orc_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t W, double theta, double scale,
               const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* kv_len, const int64_t* rows,
               int64_t n_rows, double* out, int32_t nthreads) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || (D & 1) || !q || !k || !kv_len || !out)
    return ORC_EINVAL;
  if (scale == 0.0) scale = 1.0 / sqrt((double)D);
  const uint16_t* vv = v ? v : k;
  const int32_t g = Hq / Hkv;
  const int64_t total = (int64_t)B * Hq;
  const int64_t n = n_rows >= 0 ? n_rows : total;
  orc_set_threads(nthreads);
  const uint16_t** qrows = (const uint16_t**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int64_t* qpos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  double** outs = (double**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
  int err = !qrows || !qpos || !outs;
  for (int64_t b = 0; b < B && !err; ++b) {
    int64_t L = kv_len[b];
    if (L < 1 || L > Lmax) { err = 1; break; }
    int64_t lo = (W > 0 && L - W > 0) ? L - W : 0;
    for (int64_t kvh = 0; kvh < Hkv && !err; ++kvh) {
      int64_t nq = 0;
      for (int64_t i = 0; i < n; ++i) {
        int64_t r = n_rows >= 0 ? rows[i] : i;
        if (r < 0 || r >= total) { err = 1; break; }
        int64_t rb = r / Hq, h = r % Hq;
        if (rb != b || h / g != kvh) continue;
        qrows[nq] = q + (size_t)r * D;
        qpos[nq] = L - 1;
        outs[nq] = out + (size_t)i * D;
        ++nq;
      }
      if (err || nq == 0) continue;
      size_t off = ((size_t)b * Hkv + kvh) * (size_t)Lmax * D;
      err |= orc_slice(k + off, vv + off, lo, L, L, D, W, theta, scale, nq, qrows, qpos, outs) != ORC_OK;
    }
  }
  free(qrows); free(qpos); free(outs);
  return err ? ORC_EINVAL : ORC_OK;
}
