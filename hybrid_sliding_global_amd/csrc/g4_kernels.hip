// HIP kernels for gfx950 (CDNA4): Gemma-4-style hybrid sliding/global attention.
//
// Prefill = two launches on the caller's stream:
//   1. k_rope_keys  : rotates the raw cached keys once (RoPE, the layer's own
//                     theta) into a workspace image laid out exactly as the
//                     attention kernel's LDS tiles (row-swizzled 16 B chunks);
//   2. k_prefill    : flash-style causal / sliding-window attention on bf16
//                     MFMA.  Each work-group owns 128 (position, head) query
//                     rows of one (batch, kv-head) pair -- the GQA group shares
//                     every key/value tile -- and walks the visible key tiles.
//                     Scores are computed transposed, S^T = K' Q'^T, and the
//                     output as O^T += V^T P^T, so every per-query softmax
//                     quantity lives in one lane (plus its partner 32 lanes
//                     away).  V is read straight from the cache through the
//                     LDS transpose read (ds_read_b64_tr_b16); for an aliased
//                     layer that buffer is the raw key cache.
// Decode = split-K over chunks of the visible key range:
//   1. k_decode     : one work-group per (batch, kv-head, chunk); the four
//                     waves split the head dimension, rotate keys on load,
//                     use MFMA for S^T = K' Q'^T (the GQA group is the N
//                     dimension) and for O^T += V^T P^T, and write a partial
//                     (normalised output, log-sum-exp) per chunk;
//   2. k_decode_combine : log-sum-exp merge of the chunk partials.
//
// The method follows the attention definition: softmax(scale * <RoPE(q),
// RoPE(k)>) over the visible keys, weighted sum of (un-rotated) values;
// the tiling, split-K and online softmax only reorder that computation.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "g4_internal.h"

namespace g4 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) short i16x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr int kFragBatch = 4;         // LDS operand fragments in flight per MFMA batch

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// sin/cos of 2*pi*(pos*rev): the product and its reduction to [-1/2, 1/2]
// revolutions are exact enough in fp64 for positions up to 2^31; the
// hardware sin/cos (input in revolutions) then runs on a small argument.
__device__ __forceinline__ void sincos_rev(double pos, double rev, float& s, float& c) {
  double x = pos * rev;
  x -= rint(x);
  const float xf = static_cast<float>(x);
  s = __builtin_amdgcn_sinf(xf);
  c = __builtin_amdgcn_cosf(xf);
}

// Rotate-half RoPE of 8 pairs held as two packed bf16 quads: element e of `x`
// pairs with element e of `y` (head-dim offsets d and d + D/2), frequency
// index f0 + e.  Results are scaled by `mul` and rounded back to bf16.
__device__ __forceinline__ void rope8(u32x4& x, u32x4& y, const double* rev, int f0, double pos, float mul) {
  u32x4 xo, yo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s0, c0, s1, c1;
    sincos_rev(pos, rev[f0 + 2 * e], s0, c0);
    sincos_rev(pos, rev[f0 + 2 * e + 1], s1, c1);
    const float a0 = bf_lo(x[e]), a1 = bf_hi(x[e]);
    const float b0 = bf_lo(y[e]), b1 = bf_hi(y[e]);
    xo[e] = pack_bf16((a0 * c0 - b0 * s0) * mul, (a1 * c1 - b1 * s1) * mul);
    yo[e] = pack_bf16((b0 * c0 + a0 * s0) * mul, (b1 * c1 + a1 * s1) * mul);
  }
  x = xo;
  y = yo;
}

// Swizzle of the 16-byte chunks of one LDS tile row.  It is a bijection on
// the low four chunk-index bits, so 16 consecutive rows read at one chunk
// (ds_read_b128, MFMA A/B operand) hit 16 distinct bank groups, and the four
// rows of a transpose-read group touch four disjoint chunk pairs.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8); }

__device__ __forceinline__ void g2l16(const void* gsrc, void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)ldst, 16, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Work-group barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would drain the prefetch of
// the next tile; here the direct-to-LDS loads are waited for explicitly with
// wait_vm<> by each wave before it reaches the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Batched LDS reads of MFMA operand fragments.  Each batch is one asm block
// that also waits for its own results (lgkmcnt(0)), so no output register is
// ever handed back while its load is still in flight, and the outputs are
// early-clobber so they never share a register with an address.  Written as
// asm because the compiler otherwise drains every outstanding direct-to-LDS
// prefetch (vmcnt(0)) before the first LDS read of a tile.
__device__ __forceinline__ void lds_read_b128x4(u32x4 (&r)[4], const unsigned (&ad)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
}

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Eight transpose reads (ds_read_b64_tr_b16): lane i of each 16-lane group
// receives column (i % 4) of the 4x16-bit rows addressed by lanes
// i/4, i/4 + 4, i/4 + 8, i/4 + 12 of its group.
__device__ __forceinline__ void lds_read_tr_x8(u32x2 (&r)[8], const unsigned (&ad)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]));
}

__device__ __forceinline__ bf16x8 cat2(u32x2 a, u32x2 b) { return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]}); }

// The stored values come straight from MFMA accumulators.  The compiler does
// not insert the MFMA-result -> LDS-store wait states in front of inline asm,
// so each store block starts with 24 of its own (three s_nop 7).
#define G4_MFMA_STORE_WAIT "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"

__device__ __forceinline__ void lds_write_f32x4(unsigned ad, const f32x4& v) {
  asm volatile(G4_MFMA_STORE_WAIT "ds_write_b128 %0, %1" ::"v"(ad), "v"(v));
}

// 64-byte LDS store / load of one lane's 16 floats (partial-score exchange).
__device__ __forceinline__ void lds_write_f32x16(unsigned ad, const f32x16& v) {
  const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  const f32x4 c = {v[8], v[9], v[10], v[11]}, d = {v[12], v[13], v[14], v[15]};
  asm volatile(
      G4_MFMA_STORE_WAIT
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %0, %2 offset:16\n\t"
      "ds_write_b128 %0, %3 offset:32\n\t"
      "ds_write_b128 %0, %4 offset:48" ::"v"(ad),
      "v"(a), "v"(b), "v"(c), "v"(d));
}
__device__ __forceinline__ f32x16 lds_read_f32x16(unsigned ad) {
  f32x4 a, b, c, d;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b128 %2, %4 offset:32\n\t"
      "ds_read_b128 %3, %4 offset:48\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(ad));
  return f32x16{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], c[0], c[1], c[2], c[3], d[0], d[1], d[2], d[3]};
}

__device__ __forceinline__ i16x4 ds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// --------------------------------------------------------- prefill: keys --

// Rotate raw keys rows [0, S) of one (batch, kv-head) slice into the tile
// image: tile t holds rows t*BN .. t*BN+BN-1, each row's 16-byte chunks at
// swizzled positions; rows >= S are zero.
template <int D, int BN>
__global__ __launch_bounds__(256) void k_rope_keys(const uint16_t* __restrict__ k, uint16_t* __restrict__ img, int S,
                                                   int Hkv, int Lmax, int ntiles, RopeRev rope) {
  const int t = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const uint16_t* src = k + ((size_t)b * Hkv + kvh) * (size_t)Lmax * D;
  uint16_t* dst = img + (((size_t)b * Hkv + kvh) * ntiles + t) * (size_t)(BN * D);
  constexpr int CH = D / 16;  // chunk c pairs with chunk c + CH
  for (int it = threadIdx.x; it < BN * CH; it += 256) {
    const int row = it / CH, c = it % CH, p = t * BN + row;
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (p < S) {
      const uint16_t* r = src + (size_t)p * D;
      x = *reinterpret_cast<const u32x4*>(r + 8 * c);
      y = *reinterpret_cast<const u32x4*>(r + D / 2 + 8 * c);
      rope8(x, y, rope.rev, 8 * c, (double)p, 1.0f);
    }
    const int sw = swz(row);
    *reinterpret_cast<u32x4*>(dst + row * D + 8 * (c ^ sw)) = x;
    *reinterpret_cast<u32x4*>(dst + row * D + 8 * ((c + CH) ^ sw)) = y;
  }
}

// ------------------------------------------------------ prefill: attention --

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* kimg;
  const uint16_t* v;
  float* out;
  int B, S, Hq, Hkv, g, Lmax, W, ntiles, nqt;
  float qscale;  // softmax scale * log2(e): scores come out in log2 units
  RopeRev rope;
};

// DS = number of waves sharing one 32-row query group, each owning 1/DS of
// the head dimension (DS = 2 for head size 512 keeps the 32 x 512 fp32
// output block of a row group in two waves' accumulators).  The work-group
// is 4 * DS waves and covers 128 query rows.
template <int D, int BN, int DS>
__global__ __attribute__((amdgpu_flat_work_group_size(256 * DS, 256 * DS), amdgpu_waves_per_eu(DS, DS))) void
k_prefill(PrefillArgs a) {
  constexpr int NT = 256 * DS;                // threads
  constexpr int KSTEPS = D / 16;              // 32x32x16 steps over the head dim
  constexpr int KSW = KSTEPS / DS;            // steps owned by one wave
  constexpr int MB = BN / 32;                 // 32-key blocks per tile
  constexpr int DB = D / 32;                  // 32-wide output blocks
  constexpr int DBW = DB / DS;                // output blocks owned by one wave
  constexpr int LPT = BN * D * 2 / (NT * 16); // 16-byte loads per thread per tile and tensor
  constexpr int ROWB = D * 2;
  static_assert(LPT * NT * 16 == BN * D * 2, "tile must split evenly over the threads");

  // Double-buffered key / value tiles.  The two buffers are distinct objects
  // and the tile loop is unrolled by two, so the compiler can tell that the
  // direct-to-LDS prefetch of the next tile never aliases the tile being read
  // and does not drain it before the first LDS read.
  __shared__ __attribute__((aligned(16))) uint16_t sk0[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[BN * D];
  __shared__ f32x16 sx[DS > 1 ? 4 * DS : 1][MB][64];  // partial S^T exchange

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lives in SGPRs
  const int rg = wave / DS, dp = wave % DS;
  const int nbh = a.B * a.Hkv;
  const int bh = blockIdx.x % nbh;
  const int qt = a.nqt - 1 - (int)(blockIdx.x / nbh);  // longest query tiles first
  const int kvh = bh % a.Hkv, b = bh / a.Hkv;
  const int rows_total = a.S * a.g;
  const int r0 = qt * 128;
  const int r = r0 + rg * 32 + n;
  const bool valid = r < rows_total;
  const int rc = valid ? r : rows_total - 1;
  const int pos = rc / a.g, head = kvh * a.g + rc % a.g;
  const int pos_min = r0 / a.g;
  const int pos_max = min(r0 + 127, rows_total - 1) / a.g;

  // Q' = RoPE(q) * scale * log2(e), as the B operand of S^T = K' Q'^T:
  // lane (n, h) holds head-dim elements 16*ks + 8*h + [0, 8) of its query
  // row for the k-steps this wave owns.  Rotation partners (d, d + D/2) sit
  // in k-steps ks and ks + KSTEPS/2: with DS = 2 the first half of each
  // wave's steps pairs with the second.
  bf16x8 qf[KSW];
  {
    const uint16_t* qrow = a.q + (((size_t)b * a.S + pos) * a.Hq + head) * D;
#pragma unroll
    for (int i = 0; i < KSW / 2; ++i) {
      const int ks = dp * (KSW / 2) + i;  // first-half step, partner ks + KSTEPS/2
      const int d0 = 16 * ks + 8 * h;
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + d0);
      u32x4 y = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
      rope8(x, y, a.rope.rev, d0, (double)pos, a.qscale);
      qf[i] = as_bf16x8(x);
      qf[i + KSW / 2] = as_bf16x8(y);
    }
  }

  const uint16_t* kimg = a.kimg + (size_t)(b * a.Hkv + kvh) * a.ntiles * (size_t)(BN * D);
  const uint16_t* vsl = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * D;
  const int key_lo = a.W > 0 ? max(0, pos_min - a.W + 1) : 0;
  const int j_lo = key_lo / BN, j_hi = pos_max / BN;

  auto issue = [&](int j, uint16_t* dk, uint16_t* dv) {
    int ln = lane;  // opaque: keep the per-lane address math inside the loop (see below)
    asm volatile("" : "+v"(ln));
    const char* ksrc = reinterpret_cast<const char*>(kimg + (size_t)j * (BN * D));
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int blk = i * (NT / 64) + wave;
      g2l16(ksrc + blk * 1024 + ln * 16, reinterpret_cast<char*>(dk) + blk * 1024);
    }
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int blk = i * (NT / 64) + wave;
      const int byte = blk * 1024 + ln * 16;
      const int row = byte / ROWB, slot = (byte % ROWB) >> 4;
      const int src_row = min(j * BN + row, a.S - 1);  // rows past the sequence: any valid row, weight 0
      g2l16(vsl + (size_t)src_row * D + ((slot ^ swz(row)) << 3), reinterpret_cast<char*>(dv) + blk * 1024);
    }
  };

  f32x16 acc[DBW];
#pragma unroll
  for (int i = 0; i < DBW; ++i) acc[i] = f32x16{};
  float m_i = kNegInf, l_i = 0.f;

  const bool windowed = a.W > 0;

  auto step = [&](int j, const uint16_t* ck, const uint16_t* cv, uint16_t* nk, uint16_t* nv) {
    if (j < j_hi) {
      issue(j + 1, nk, nv);
      wait_vm<2 * LPT>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();

    // Per-lane LDS offsets are recomputed every tile from an opaque copy of
    // the lane index instead of being hoisted out of the loop, which would pin
    // a few dozen registers for the whole kernel.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int on = ln & 31, oh = ln >> 5, oG = ln >> 4, oi16 = ln & 15;

    // S^T = K' Q'^T for this tile: s[mb] holds keys 32*mb + 8*i + 4*h + jj (reg 4*i + jj) of query n.
    f32x16 s[MB];
    const char* kb = reinterpret_cast<const char*>(ck);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[mb] = f32x16{};
      const int row = 32 * mb + on;
      const char* kr = kb + row * ROWB;
      const int sw = swz(row);
      const unsigned kra = lds_addr(kr);
#pragma unroll
      for (int i0 = 0; i0 < KSW; i0 += 4) {
        unsigned ad[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u;
          const int ks = i < KSW / 2 ? dp * (KSW / 2) + i : KSTEPS / 2 + dp * (KSW / 2) + (i - KSW / 2);
          ad[u] = kra + (((2 * ks + oh) ^ sw) << 4);
        }
        u32x4 kf[4];
        lds_read_b128x4(kf, ad);
#pragma unroll
        for (int u = 0; u < 4; ++u) s[mb] = mfma32(as_bf16x8(kf[u]), qf[i0 + u], s[mb]);
      }
    }
    if constexpr (DS > 1) {
      // exchange the two halves of the head-dim sum within the wave pair;
      // float addition is commutative, so both waves get identical scores
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) lds_write_f32x16(lds_addr(&sx[wave][mb][ln]), s[mb]);
      lds_barrier();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) s[mb] += lds_read_f32x16(lds_addr(&sx[wave ^ 1][mb][ln]));
    }

    const int kbase = j * BN;
    const bool need_mask = (kbase + BN - 1 > pos_min) || (windowed && kbase <= pos_max - a.W);
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = kbase + 32 * mb + 8 * (rr >> 2) + 4 * h + (rr & 3);
          const bool vis = (key <= pos) & (!windowed | (pos - key < a.W));
          s[mb][rr] = vis ? s[mb][rr] : kNegInf;
        }
    }

    // Online softmax in the log2 domain; lanes n and n+32 share query n.  The
    // reference maximum m_i only moves when a score exceeds it by more than
    // kRescaleSlack, so P = 2^(s - m_i) <= 2^kRescaleSlack and the MFMA
    // accumulators are rescaled only on those (rare) tiles.
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[mb][rr]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool grow = mx > m_i + kRescaleSlack;
    // lanes with m_i = -inf have nothing accumulated yet: they just adopt mx
    const float alpha = (grow & (m_i != kNegInf)) ? fast_exp2(m_i - mx) : 1.f;
    m_i = grow ? mx : m_i;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
      l_i *= alpha;
#pragma unroll
      for (int i = 0; i < DBW; ++i) acc[i] *= alpha;
    }
    const float m_use = (m_i == kNegInf) ? 0.f : m_i;
    float rs = 0.f;
    unsigned pk[MB * 8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const float p0 = fast_exp2(s[mb][rr] - m_use), p1 = fast_exp2(s[mb][rr + 1] - m_use);
        rs += p0 + p1;
        pk[mb * 8 + rr / 2] = pack_bf16(p0, p1);
      }
    l_i += rs;

    // O^T += V^T P^T.  P^T slot t of key-step ks is key 16*ks + 4*hh + t (t < 4)
    // or 16*ks + 8 + 4*hh + (t - 4); the transpose reads fetch V in that order.
    const char* vb = reinterpret_cast<const char*>(cv);
    const int ohh = oG >> 1, odsub = 16 * (oG & 1);
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const bf16x8 pf = as_bf16x8(u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
      const int row1 = 16 * ks + 4 * ohh + (oi16 >> 2), row2 = row1 + 8;
      const unsigned v1 = lds_addr(vb + row1 * ROWB), v2 = lds_addr(vb + row2 * ROWB);
      const int sw1 = swz(row1), sw2 = swz(row2);
#pragma unroll
      for (int i0 = 0; i0 < DBW; i0 += 4) {
        unsigned ad[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int dcol = 32 * (dp * DBW + i0 + u) + odsub + 4 * (oi16 & 3);
          const int chunk = dcol >> 3, half = (dcol & 7) << 1;
          ad[2 * u] = v1 + ((chunk ^ sw1) << 4) + half;
          ad[2 * u + 1] = v2 + ((chunk ^ sw2) << 4) + half;
        }
        u32x2 t[8];
        lds_read_tr_x8(t, ad);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[i0 + u] = mfma32(cat2(t[2 * u], t[2 * u + 1]), pf, acc[i0 + u]);
      }
    }
    lds_barrier();
  };

  issue(j_lo, sk0, sv0);
  for (int j = j_lo;;) {
    step(j, sk0, sv0, sk1, sv1);
    if (++j > j_hi) break;
    step(j, sk1, sv1, sk0, sv0);
    if (++j > j_hi) break;
  }

  const float l = l_i + __shfl_xor(l_i, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (valid) {
    float* orow = a.out + (((size_t)b * a.S + pos) * a.Hq + head) * D + 32 * dp * DBW;
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o = {acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i + 4 * h) = o;
      }
  }
}

// ---------------------------------------------------------------- decode --

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  float* part_o;    // [B, Hq, nchunks, D]
  float* part_lse;  // [B, Hq, nchunks], log2 units
  int B, Hq, Hkv, g, Lmax, W, nchunks, chunk;
  float qscale;
  RopeRev rope;
};

template <int D, bool ALIAS, int NSTAGE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void k_decode(DecodeArgs a) {
  constexpr int KPS = 32;            // keys per step
  constexpr int FQ = D / 8;          // rotation pairs per wave
  constexpr int KSTEPS = FQ / 16;    // 16x16x32 steps per key block (both halves of each pair)
  constexpr int DQ = D / 4;          // output head-dim slice per wave
  constexpr int DBLK = DQ / 16;
  constexpr int NT = ALIAS ? 1 : 2;  // tensors staged per step
  constexpr int ROWB = D * 2;
  constexpr int LPS1 = KPS * ROWB / 4096;
  constexpr int LPS = NT * LPS1;

  __shared__ __attribute__((aligned(16))) uint16_t sbuf[NSTAGE][NT][KPS * D];
  __shared__ f32x4 red[4][2][64];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x % a.nchunks;
  const int bh = blockIdx.x / a.nchunks;
  const int kvh = bh % a.Hkv, b = bh / a.Hkv;
  const int L = min(max(a.kv_len[b], 1), a.Lmax);
  const int lo = a.W > 0 ? max(0, L - a.W) : 0;
  const int k_start = lo + c * a.chunk;
  const int k_end = min(L, k_start + a.chunk);
  const bool qvalid = n < a.g;
  const int head = kvh * a.g + (qvalid ? n : 0);
  const size_t part = ((size_t)b * a.Hq + head) * a.nchunks + c;

  if (k_start >= k_end) {
    if (wave == 0 && G == 0 && qvalid) a.part_lse[part] = kNegInf;
    return;
  }

  // Q' of this wave's rotation pairs, as the B operand (N = query heads).
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS / 2; ++kk) {
      const int d0 = wave * FQ + 32 * kk + 8 * G;
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + d0);
      u32x4 y = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
      rope8(x, y, a.rope.rev, d0, (double)(L - 1), a.qscale);
      if (!qvalid) x = y = u32x4{0, 0, 0, 0};
      qf[kk] = as_bf16x8(x);
      qf[kk + KSTEPS / 2] = as_bf16x8(y);
    }
  }

  const size_t slice = ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * D;
  auto issue = [&](int step, int stg) {
    const int k0 = k_start + step * KPS;
#pragma unroll
    for (int tsr = 0; tsr < NT; ++tsr) {
      const uint16_t* base = (tsr == 0 ? a.k : a.v) + slice;
#pragma unroll
      for (int i = 0; i < LPS1; ++i) {
        const int blk = i * 4 + wave;
        const int byte = blk * 1024 + lane * 16;
        const int row = byte / ROWB, slot = (byte % ROWB) >> 4;
        const int src_row = min(k0 + row, k_end - 1);
        g2l16(base + (size_t)src_row * D + ((slot ^ swz(row)) << 3),
              reinterpret_cast<char*>(sbuf[stg][tsr]) + blk * 1024);
      }
    }
  };

  f32x4 acc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) acc[i] = f32x4{};
  float m_i = kNegInf, l_i = 0.f;

  const int nsteps = (k_end - k_start + KPS - 1) / KPS;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nsteps) issue(s, s);

  for (int s = 0; s < nsteps; ++s) {
    const int stg = s % NSTAGE;
    if (nsteps - s - 1 >= NSTAGE - 2)
      wait_vm<(NSTAGE - 2) * LPS>();
    else
      wait_vm<0>();
    lds_barrier();
    if (s + NSTAGE - 1 < nsteps) issue(s + NSTAGE - 1, (s + NSTAGE - 1) % NSTAGE);

    int ln = lane;  // opaque lane index: per-lane LDS offsets are recomputed each step
    asm volatile("" : "+v"(ln));
    const int on = ln & 15, oG = ln >> 4;
    const int k0 = k_start + s * KPS;
    const char* kb = reinterpret_cast<const char*>(sbuf[stg][0]);
    // Partial S^T over this wave's rotation pairs; keys rotated on the fly.
    // Fragment e of the batch: key block mb = e / (KSTEPS) ..., x/y halves.
    constexpr int NFR = 2 * KSTEPS;  // 16-byte fragments per step and lane (x and y, both key blocks)
    static_assert(NFR % 4 == 0, "fragment batches of four");
    f32x4 sp[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int e0 = 0; e0 < NFR; e0 += 4) {
      unsigned ad[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u, mb = e / KSTEPS, kk = (e % KSTEPS) / 2, hi = e & 1;
        const int row = 16 * mb + on;
        const int d = wave * FQ + 32 * kk + 8 * oG + (hi ? D / 2 : 0);
        ad[u] = lds_addr(kb + row * ROWB) + (((d >> 3) ^ swz(row)) << 4);
      }
      u32x4 fr[4];
      lds_read_b128x4(fr, ad);
#pragma unroll
      for (int u = 0; u < 4; u += 2) {
        const int e = e0 + u, mb = e / KSTEPS, kk = (e % KSTEPS) / 2;
        const int d0 = wave * FQ + 32 * kk + 8 * G;
        u32x4 x = fr[u], y = fr[u + 1];
        rope8(x, y, a.rope.rev, d0, (double)(k0 + 16 * mb + n), 1.0f);
        sp[mb] = mfma16(as_bf16x8(x), qf[kk], sp[mb]);
        sp[mb] = mfma16(as_bf16x8(y), qf[kk + KSTEPS / 2], sp[mb]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) lds_write_f32x4(lds_addr(&red[wave][mb][ln]), sp[mb]);
    lds_barrier();
    f32x4 sc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      u32x4 t[4];
      const unsigned ad[4] = {lds_addr(&red[0][mb][ln]), lds_addr(&red[1][mb][ln]), lds_addr(&red[2][mb][ln]),
                              lds_addr(&red[3][mb][ln])};
      lds_read_b128x4(t, ad);
      sc[mb] = __builtin_bit_cast(f32x4, t[0]) + __builtin_bit_cast(f32x4, t[1]) + __builtin_bit_cast(f32x4, t[2]) +
               __builtin_bit_cast(f32x4, t[3]);
    }

    // keys k0 + 16*mb + 4*G + jj for query n
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = k0 + 16 * mb + 4 * G + jj;
        if (key >= k_end) sc[mb][jj] = kNegInf;
        mx = fmaxf(mx, sc[mb][jj]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_i - m_use);
    float p[2][4];
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        p[mb][jj] = fast_exp2(sc[mb][jj] - m_use);
        rs += p[mb][jj];
      }
    l_i = l_i * alpha + rs;
    m_i = m_new;
    const bf16x8 pf = as_bf16x8(u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                                      pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])});

    const char* vb = reinterpret_cast<const char*>(sbuf[stg][NT - 1]);
    const int row1 = 4 * oG + (on >> 2), row2 = row1 + 16;
    const unsigned v1 = lds_addr(vb + row1 * ROWB), v2 = lds_addr(vb + row2 * ROWB);
    const int sw1 = swz(row1), sw2 = swz(row2);
#pragma unroll
    for (int b0 = 0; b0 < DBLK; b0 += 4) {
      unsigned ad[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dcol = wave * DQ + 16 * (b0 + u) + 4 * (on & 3);
        const int chunk = dcol >> 3, half = (dcol & 7) << 1;
        ad[2 * u] = v1 + ((chunk ^ sw1) << 4) + half;
        ad[2 * u + 1] = v2 + ((chunk ^ sw2) << 4) + half;
      }
      u32x2 t[8];
      lds_read_tr_x8(t, ad);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[b0 + u] = mfma16(cat2(t[2 * u], t[2 * u + 1]), pf, acc[b0 + u] * alpha);
    }
  }

  float l = l_i + __shfl_xor(l_i, 16);
  l += __shfl_xor(l, 32);
  const float inv = 1.f / l;
  if (qvalid) {
    float* o = a.part_o + part * D + wave * DQ + 4 * G;
#pragma unroll
    for (int bi = 0; bi < DBLK; ++bi) *reinterpret_cast<f32x4*>(o + 16 * bi) = acc[bi] * inv;
    if (wave == 0 && G == 0) a.part_lse[part] = m_i + __builtin_amdgcn_logf(l);
  }
}

// Log-sum-exp merge of the chunk partials of one (batch, head).
template <int D>
__global__ __launch_bounds__(256) void k_decode_combine(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse, float* __restrict__ out,
                                                        int nchunks) {
  const int bh = blockIdx.x;
  const float* lse = part_lse + (size_t)bh * nchunks;
  float M = kNegInf;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, lse[c]);
  for (int d = threadIdx.x; d < D; d += 256) {
    float num = 0.f, den = 0.f;
    for (int c = 0; c < nchunks; ++c) {
      const float e = lse[c];
      if (e == kNegInf) continue;
      const float w = fast_exp2(e - M);
      num += w * part_o[((size_t)bh * nchunks + c) * D + d];
      den += w;
    }
    out[(size_t)bh * D + d] = num / den;
  }
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace

// ------------------------------------------------------------- launchers --

void fill_rope_rev(RopeRev* r, int head_dim, double theta) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int f = 0; f < 256; ++f)
    r->rev[f] = f < head_dim / 2 ? std::pow(theta, -2.0 * (double)f / (double)head_dim) / two_pi : 0.0;
}

size_t prefill_workspace(int B, int S, int Hkv, int D) {
  const int BN = prefill_key_tile(D);
  const size_t ntiles = (size_t)ceil_div(S, BN);
  return (size_t)B * Hkv * ntiles * BN * D * 2;
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream, const ProfileEvents& ev) {
  const int BN = prefill_key_tile(p.D);
  const int ntiles = ceil_div(p.S, BN);
  const int g = p.Hq / p.Hkv;
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kimg = static_cast<const uint16_t*>(p.kimg);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = p.out;
  a.B = p.B;
  a.S = p.S;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.g = g;
  a.Lmax = p.Lmax;
  a.W = p.W;
  a.ntiles = ntiles;
  a.nqt = ceil_div(p.S * g, kPrefillRows);
  a.qscale = p.scale * kLog2e;
  fill_rope_rev(&a.rope, p.D, p.theta);
  const dim3 grid_k(ntiles, p.Hkv, p.B);
  const dim3 grid_a(a.nqt * p.B * p.Hkv);
  if (p.D == 512) {
    hipLaunchKernelGGL((k_rope_keys<512, 32>), grid_k, dim3(256), 0, stream, static_cast<const uint16_t*>(p.k),
                       static_cast<uint16_t*>(p.kimg), p.S, p.Hkv, p.Lmax, ntiles, a.rope);
    if (ev.before) (void)hipEventRecord(ev.before, stream);
    hipLaunchKernelGGL((k_prefill<512, 32, 2>), grid_a, dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL((k_rope_keys<256, 64>), grid_k, dim3(256), 0, stream, static_cast<const uint16_t*>(p.k),
                       static_cast<uint16_t*>(p.kimg), p.S, p.Hkv, p.Lmax, ntiles, a.rope);
    if (ev.before) (void)hipEventRecord(ev.before, stream);
    hipLaunchKernelGGL((k_prefill<256, 64, 1>), grid_a, dim3(256), 0, stream, a);
  }
  if (ev.after) (void)hipEventRecord(ev.after, stream);
  return hipGetLastError();
}

DecodePlan plan_decode(int B, int Hkv, int W, int max_kv_len) {
  const long span = W > 0 ? std::min<long>(W, max_kv_len) : max_kv_len;
  const long streams = (long)B * Hkv;
  const long target_groups = 2048;
  long per = (streams * span + target_groups - 1) / target_groups;
  per = std::max<long>(per, 64);
  per = std::min<long>(per, 4096);
  per = (per + 31) / 32 * 32;
  DecodePlan plan;
  plan.chunk = (int)per;
  plan.nchunks = (int)((span + per - 1) / per);
  return plan;
}

size_t decode_workspace(int B, int Hq, int D, const DecodePlan& plan) {
  const size_t parts = (size_t)B * Hq * plan.nchunks;
  return parts * D * sizeof(float) + parts * sizeof(float);
}

hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream, const ProfileEvents& ev) {
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.alias ? p.k : p.v);
  a.kv_len = p.kv_len;
  const size_t parts = (size_t)p.B * p.Hq * p.plan.nchunks;
  a.part_o = static_cast<float*>(p.ws);
  a.part_lse = a.part_o + parts * p.D;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.g = p.Hq / p.Hkv;
  a.Lmax = p.Lmax;
  a.W = p.W;
  a.nchunks = p.plan.nchunks;
  a.chunk = p.plan.chunk;
  a.qscale = p.scale * kLog2e;
  fill_rope_rev(&a.rope, p.D, p.theta);
  const dim3 grid((unsigned)(p.plan.nchunks * p.B * p.Hkv));
  if (ev.before) (void)hipEventRecord(ev.before, stream);
  if (p.D == 512) {
    if (p.alias)
      hipLaunchKernelGGL((k_decode<512, true, 4>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_decode<512, false, 2>), grid, dim3(256), 0, stream, a);
  } else {
    if (p.alias)
      hipLaunchKernelGGL((k_decode<256, true, 4>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_decode<256, false, 4>), grid, dim3(256), 0, stream, a);
  }
  if (ev.after) (void)hipEventRecord(ev.after, stream);
  if (p.D == 512)
    hipLaunchKernelGGL((k_decode_combine<512>), dim3(p.B * p.Hq), dim3(256), 0, stream, a.part_o, a.part_lse, p.out,
                       a.nchunks);
  else
    hipLaunchKernelGGL((k_decode_combine<256>), dim3(p.B * p.Hq), dim3(256), 0, stream, a.part_o, a.part_lse, p.out,
                       a.nchunks);
  return hipGetLastError();
}

}  // namespace g4
