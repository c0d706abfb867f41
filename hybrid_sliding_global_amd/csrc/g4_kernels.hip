// HIP kernels for gfx950 (CDNA4): Gemma-4-style hybrid sliding/global attention.
//
// Prefill = two launches on the caller's stream:
//   1. k_prefill_prep : rotates the raw cached keys once (RoPE, the layer's
//                     own theta) and writes key and value operand images in
//                     exactly the order the attention kernel's MFMA operands
//                     are read from LDS (values transposed, not rotated);
//   2. k_prefill    : flash-style causal / sliding-window attention on bf16
//                     MFMA.  Each work-group owns 128 (position, head) query
//                     rows of one (batch, kv-head) pair -- the GQA group shares
//                     every key/value tile -- and walks the visible key tiles.
//                     Scores are computed transposed, S^T = K' Q'^T, and the
//                     output as O^T += V^T P^T, so every per-query softmax
//                     quantity lives in one lane (plus its partner 32 lanes
//                     away).  For an aliased layer the value image is built
//                     from the raw key cache.  Head size 512 runs the
//                     eight-wave k_prefill, head size 256 the four-wave
//                     k_prefill4 (scores by row block, output by head-dim
//                     block, P exchanged in bf16).
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
#include <cstdlib>
#include <cstdint>
#include <mutex>
#include <type_traits>

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
constexpr float kMaxGrowth = 64.f;     // log2 units: largest P = 2^(s - reference) the four-wave prefill allows
#ifndef G4_PIPE_DEPTH
#define G4_PIPE_DEPTH 4
#endif
constexpr int kDecodePieces = 512;   // decode work-groups: two per CU of an MI355X
constexpr int kReanchorSteps = 64;     // decode: query rotation recomputed from the fp64 angle every 64 key steps
constexpr int kDecodeStages = 4;      // 16-row key/value stages in the decode LDS ring (2 when K and V
                                      // are both staged at head size 512, so two work-groups share a CU)

// ---------------------------------------------------------------- helpers --

// Division by a divisor d >= 1 fixed for a launch (set up on the host), for
// dividends n in [0, 2^31): q = (n * m) >> s with s = 31 + ceil(log2 d) and
// m = ceil(2^s / d), which is below 2^32.  Exact: n * m / 2^s exceeds n / d
// by less than n / 2^s < 2^-ceil(log2 d) <= 1 / d, too little to reach the
// next integer.  Three scalar instructions instead of the ~25 of a division
// by a run-time value (the work-group prologues hold a dozen of them).
struct FastDiv {
  unsigned m, s;
};
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  return (int)(((unsigned long long)(unsigned)n * f.m) >> f.s);
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Eight E4M3 bytes (OCP encoding, what gfx950's conversions read) -> eight
// packed bf16: exact, since every E4M3 value is a bf16 value.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 w) {
  // one instruction per pair (scale 1: every E4M3 value, subnormals included,
  // is exactly a bf16 value; checked bit for bit against the E4M3 -> fp32 ->
  // bf16 route on all 256 codes)
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
  }
  return r;
}

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

// Direct-to-LDS 16-byte load with the non-temporal cache policy, for data
// read exactly once (the decode cache stream): it then neither evicts nor
// competes with what L2 and the MALL hold, which lifts the streaming rate by
// about a tenth.
__device__ __forceinline__ void g2l16_nt(const void* gsrc, void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)ldst, 16, 0, 2);
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

// Scheduling hint for a block of N MFMAs, each fed by one LDS read: keep P
// reads in flight ahead of the MFMAs (P reads, then N - P (MFMA, read)
// pairs, then the last P MFMAs).  Without it the scheduler keeps only two
// reads ahead and every MFMA waits out the LDS latency.
template <int N, int P>
__device__ __forceinline__ void lds_mfma_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, P, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
}

// --------------------------------------------------------- prefill: keys --

// Direct-to-LDS copy of one 1 KiB block: lane l moves 16 bytes from
// gbase + voff (gbase: the tile, in SGPRs; voff = 16 * l + the block's
// offset in the tile) to LDS lds + 16 * l.  Written
// as asm on purpose: the compiler then does not see an LDS store, so it
// schedules the plain LDS reads of the other buffer freely instead of
// draining every outstanding copy (vmcnt(0)) in front of them.  The caller
// waits for its own copies (wait_vm) before the barrier that publishes them.
// M0 is clobbered here; no other code in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_block(const void* gbase, unsigned voff, unsigned lds) {
  // (both operands are wave-uniform; readfirstlane says so where the
  // compiler cannot prove it, and folds away where it can)
  const unsigned long long g = reinterpret_cast<unsigned long long>(gbase);
  const unsigned long long gu =
      ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(g >> 32)) << 32) |
      (unsigned)__builtin_amdgcn_readfirstlane((unsigned)g);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(reinterpret_cast<const void*>(gu)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Operand images of one key tile, written once per prefill call so that the
// attention kernel copies each tile into LDS linearly and reads every MFMA
// operand as one conflict-free 1 KiB row of 16-byte lane slots:
//
//   key image, block (mb, ks) of 64 lane slots (block index mb * D/16 + ks):
//     lane l holds RoPE(k)[32 mb + l % 32][16 ks + 8 (l / 32) + e], e < 8
//     (the A operand of S^T = K' Q'^T for key block mb, head-dim step ks);
//   value image, block (kv, db) (block index kv * D/32 + db):
//     lane l holds v[16 kv + 4 (l / 32) + (e & 3) + 8 (e >> 2)][32 db + l % 32]
//     (the A operand of O^T += V^T P^T for the 16-key step kv; this key order
//     matches where the score layout leaves each probability).
//
// Values are not rotated (for an aliased layer `v` is the raw key buffer).
// Keys 0 .. nkeys-1 are imaged (a chunk at start position P0 of S queries
// sees nkeys = P0 + S); rows at or beyond nkeys are written as zeros.  Also clears the attention
// kernel's arrival counters (this launch precedes it on the same stream).
//
// Grid (2 * ntiles, Hkv, B): even work-groups write a tile's key image, odd
// ones its value image.  Every thread issues all of its global loads before
// it uses any of them, so a work-group costs one memory round trip rather
// than one per loop step.
// FP8: the cache holds E4M3 bytes; their codes are imaged exactly (the
// scales are applied to the queries and to the output instead).
template <int D, int BN, bool FP8>
__global__ __launch_bounds__(256) void k_prefill_prep(const void* __restrict__ k, const void* __restrict__ v,
                                                      uint16_t* __restrict__ kimg, uint16_t* __restrict__ vimg,
                                                      int nkeys, int Hkv, int Lmax, int ntiles, RopeRev rope,
                                                      int* counters, int ncounters) {
  constexpr int EB = FP8 ? 1 : 2;  // bytes per cache element
  // 8 consecutive elements of a cache row, as packed bf16
  auto load8 = [](const char* p) -> u32x4 {
    if constexpr (FP8)
      return fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(p));
    else
      return *reinterpret_cast<const u32x4*>(p);
  };
  constexpr int KSTEPS = D / 16, DB = D / 32, KV = BN / 16;
  constexpr int PITCH = D + 8;  // staged value row, bf16 elements (16-byte skew per row)
  constexpr int CH = D / 16;    // 16-byte chunks per half key row
  constexpr int NK = BN * CH / 256, NV = BN * (D / 8) / 256, NG = KV * DB * 64 / 256;
  static_assert(NK * 256 == BN * CH && NV * 256 == BN * (D / 8) && NG * 256 == KV * DB * 64, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t sv[BN * PITCH];
  const int t = blockIdx.x >> 1, kvh = blockIdx.y, b = blockIdx.z;
  const int flat = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  for (int i = flat * 256 + threadIdx.x; i < ncounters; i += gridDim.x * gridDim.y * gridDim.z * 256) counters[i] = 0;
  const size_t slice = ((size_t)b * Hkv + kvh) * (size_t)Lmax * D * EB;  // bytes
  const size_t tile = (((size_t)b * Hkv + kvh) * ntiles + t) * (size_t)(BN * D);

  if ((blockIdx.x & 1) == 0) {
    // keys: chunk c (8 elements at 8c) of the first half pairs with chunk c of
    // the second half; a thread keeps one chunk index c for all its rows
    static_assert(256 % CH == 0, "chunk index fixed per thread");
    const char* ksrc = static_cast<const char*>(k) + slice;
    uint16_t* kdst = kimg + tile;
    const int c = threadIdx.x % CH, row0 = threadIdx.x / CH;
    u32x4 x[NK], y[NK];
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int p = t * BN + row0 + j * (256 / CH);
      const char* r = ksrc + (size_t)min(p, nkeys - 1) * D * EB;  // rows past the keys load the last, then become zeros
      x[j] = load8(r + 8 * c * EB);
      y[j] = load8(r + (D / 2 + 8 * c) * EB);
    }
    double rev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rev[e] = rope.rev[8 * c + e];
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int row = row0 + j * (256 / CH), p = t * BN + row;
      rope8(x[j], y[j], rev, 0, (double)p, 1.0f);
      if (p >= nkeys) {
        x[j] = u32x4{0, 0, 0, 0};
        y[j] = u32x4{0, 0, 0, 0};
      }
      const int lane = (row & 31) + 32 * (c & 1), mb = row >> 5;
      *reinterpret_cast<u32x4*>(kdst + ((mb * KSTEPS + (c >> 1)) * 64 + lane) * 8) = x[j];
      *reinterpret_cast<u32x4*>(kdst + ((mb * KSTEPS + KSTEPS / 2 + (c >> 1)) * 64 + lane) * 8) = y[j];
    }
    return;
  }

  // values: stage the tile's rows, then gather the transposed lane slots
  const char* vsrc = static_cast<const char*>(v) + slice;
  uint16_t* vdst = vimg + tile;
  u32x4 x[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int it = threadIdx.x + 256 * j, row = it / (D / 8), c = it % (D / 8), p = t * BN + row;
    x[j] = load8(vsrc + ((size_t)min(p, nkeys - 1) * D + 8 * c) * EB);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int it = threadIdx.x + 256 * j, row = it / (D / 8), c = it % (D / 8), p = t * BN + row;
    *reinterpret_cast<u32x4*>(sv + row * PITCH + 8 * c) = p < nkeys ? x[j] : u32x4{0, 0, 0, 0};
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int it = threadIdx.x + 256 * j;
    const int lane = it & 63, blk = it >> 6, kv = blk / DB, db = blk % DB;
    const int d = 32 * db + (lane & 31), k0 = 16 * kv + 4 * (lane >> 5);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ka = k0 + ((2 * e) & 3) + 8 * ((2 * e) >> 2), kb = k0 + ((2 * e + 1) & 3) + 8 * ((2 * e + 1) >> 2);
      o[e] = (unsigned)sv[ka * PITCH + d] | ((unsigned)sv[kb * PITCH + d] << 16);
    }
    *reinterpret_cast<u32x4*>(vdst + (blk * 64 + lane) * 8) = o;
  }
}

// ------------------------------------------------------ prefill: attention --

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* kimg;  // key operand image (see k_prefill_prep)
  const uint16_t* vimg;  // value operand image
  float* out;
  int* counters;  // [B * Hkv * nqt] arrival counts (zeroed by the key pass)
  float* part;    // partial-result slots
  int B, S, Hq, Hkv, g, Lmax, W, ntiles, nqt, npair, kpieces;
  int P0;      // position of query 0 (keys 0 .. P0 + S - 1 are visible to the chunk)
  const int32_t* span_end;  // null (causal), or [B, S]: the last position of each query's bidirectional span
  int paired;  // 1: work unit = query tiles t and nqt-1-t; 0: one query tile
  FastDiv fd_g, fd_kp, fd_pbh, fd_hkv;  // division by g, kpieces, npair * kpieces, Hkv
  float qscale;  // softmax scale * log2(e) (times the key scale of an E4M3 cache): scores in log2 units
  float vscale;  // the value scale of an E4M3 cache (1 otherwise): multiplies every output
  RopeRev rope;
};

// Loads every scalar field of the prefill arguments in one batch at kernel
// entry.  Left to itself the compiler fetches them where they are first
// used, behind branches, as a chain of dependent kernel-argument round trips
// (about 800 cycles of the sliding-layer kernel's start); the empty asm
// takes all of them as inputs, so they are issued together up front.
#define G4_PREFETCH_PREFILL_ARGS(a)                                                                                 \
  asm volatile("" ::"s"((a).q), "s"((a).kimg), "s"((a).vimg), "s"((a).out), "s"((a).counters), "s"((a).part),    \
               "s"((a).B), "s"((a).S), "s"((a).Hq), "s"((a).Hkv), "s"((a).g), "s"((a).Lmax), "s"((a).W),            \
               "s"((a).ntiles), "s"((a).nqt), "s"((a).npair), "s"((a).kpieces), "s"((a).P0), "s"((a).paired),      \
               "s"((a).qscale), "s"((a).vscale), "s"(gridDim.x))

// Causal limit of query sq (at position pos) of batch entry b: the last key
// it sees -- its own position, or the end of its bidirectional span, clamped
// to [pos, P0 + S - 1] so that no image row beyond the chunk is ever read.
// The limit never decreases along the positions (spans are disjoint
// intervals), so over a query tile it is smallest at the tile's first
// position and largest at its last.
// Kernels instantiated without spans (SPAN = false) ignore span_end.
template <bool SPAN>
__device__ __forceinline__ int causal_limit(const PrefillArgs& a, int b, int sq, int pos) {
  if constexpr (!SPAN) return pos;
  return min(max(a.span_end[(size_t)b * a.S + sq], pos), a.P0 + a.S - 1);
}

__device__ __forceinline__ float max_lane_pair(float x) {  // max over lanes l and l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Flash-style prefill.  DS = number of waves sharing one 32-row query group,
// each owning 1/DS of the head dimension (DS = 2 for head size 512 keeps
// the 32 x 512 fp32 output block of a row group in two waves'
// accumulators).  SPV (DS = 2) picks the tile schedule: PV of a tile in its
// softmax phase (false), or split between that phase and the next score
// phase (true: shorter critical path, longer pipeline start; for long
// segments).  A work-group is 4 * DS waves and covers one 128-row query
// tile of one (batch, kv-head) at a time.
//
// Work split: the query tiles of a (batch, kv-head) are paired long with
// short (t with nqt-1-t), so a pair's key-tile count is nearly the same for
// every pair, and each pair's concatenated key work is cut into kpieces
// equal ranges, one per work-group.  A query tile cut across work-groups is
// finished by whichever of its pieces arrives last: every piece stores its
// partial (O, running max, running sum) and bumps the tile's counter; the
// last one merges the others into its own registers and writes the output.
// Nobody waits for anybody.
template <int D, int BN, int DS, bool SPV, bool SPAN>
__global__ __attribute__((amdgpu_flat_work_group_size(256 * DS, 256 * DS), amdgpu_waves_per_eu(DS, DS))) void
k_prefill(PrefillArgs a) {
  G4_PREFETCH_PREFILL_ARGS(a);
  constexpr int NT = 256 * DS;                // threads
  constexpr int NW = 4 * DS;                  // waves
  constexpr int KSTEPS = D / 16;              // 32x32x16 steps over the head dim
  constexpr int KSW = KSTEPS / DS;            // steps owned by one wave
  constexpr int MB = BN / 32;                 // 32-key blocks per tile
  constexpr int KV = BN / 16;                 // 16-key steps per tile
  constexpr int DB = D / 32;                  // 32-wide output blocks
  constexpr int DBW = DB / DS;                // output blocks owned by one wave
  constexpr int TILE_BLKS = BN * D * 2 / 1024;  // 1 KiB blocks per operand tile
  constexpr int LPT = TILE_BLKS / NW;         // blocks each wave copies per tile and operand
  constexpr int ACC_F4 = NW * DBW * 4 * 64;   // f32x4 per partial slot (accumulators)
  static_assert(LPT * NW == TILE_BLKS, "tile must split evenly over the waves");
  constexpr int kPipeDepth = G4_PIPE_DEPTH;  // LDS operand reads kept in flight ahead of the MFMAs

  // Double-buffered key / value operand tiles (layouts of k_prefill_prep).
  __shared__ __attribute__((aligned(1024))) uint16_t sk0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sk1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv1[BN * D];
  // Partial S^T exchange between the DS waves of a row group: [wave][mb][quad][lane].
  __shared__ f32x4 sx[DS > 1 ? NW : 1][MB][4][64];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lives in SGPRs
  const int rg = wave / DS, dp = wave % DS;

  // Work id: consecutive ids (same batch / kv-head) go to the same XCD, whose
  // L2 then serves their shared key/value tiles.
  const int nblk = gridDim.x;
  const int wid = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int per_bh = a.npair * a.kpieces;
  const int bh = fdiv(wid, a.fd_pbh), rem = wid - bh * per_bh;
  const int pair = fdiv(rem, a.fd_kp), piece = rem - pair * a.kpieces;
  const int b = fdiv(bh, a.fd_hkv), kvh = bh - b * a.Hkv;
  const int rows_total = a.S * a.g;
  const bool windowed = a.W > 0;

  auto tile_keys = [&](int qt, int& jlo, int& jhi) {
    const int r0 = qt * 128;
    const int pmin = a.P0 + fdiv(r0, a.fd_g), pmax = a.P0 + fdiv(min(r0 + 127, rows_total - 1), a.fd_g);
    jlo = (windowed ? max(0, pmin - a.W + 1) : 0) / BN;
    jhi = causal_limit<SPAN>(a, b, pmax - a.P0, pmax) / BN;
  };
  const int tl = a.paired ? a.nqt - 1 - pair : pair;   // long tile of the pair
  const int ts = a.paired && pair < tl ? pair : -1;   // short tile (none for the middle of an odd count)
  int jlo_l, jhi_l, jlo_s = 0, jhi_s = -1;
  tile_keys(tl, jlo_l, jhi_l);
  if (ts >= 0) tile_keys(ts, jlo_s, jhi_s);
  const int nL = jhi_l - jlo_l + 1, nS = ts >= 0 ? jhi_s - jlo_s + 1 : 0, U = nL + nS;
  auto ubound = [&](int j) { return fdiv(j * U, a.fd_kp); };  // j * U < 2^31 (the planner caps kpieces)
  const int u0 = ubound(piece), u1 = ubound(piece + 1);

  const size_t slice_off = (size_t)(b * a.Hkv + kvh) * a.ntiles * (size_t)(BN * D);
  const uint16_t* kimg = a.kimg + slice_off;
  const uint16_t* vimg = a.vimg + slice_off;
  const unsigned voff = (unsigned)(wave * 1024 + lane * 16);  // this lane's slot in the wave's first block

  // Copy key tile j into dk / value tile j into dv: this wave's blocks are i * NW + wave.
  auto issue_k = [&](int j, uint16_t* dk) {
    const char* kt = reinterpret_cast<const char*>(kimg + (size_t)j * (BN * D));
    const unsigned lk = lds_addr(dk) + wave * 1024;
#pragma unroll
    for (int i = 0; i < LPT; ++i) dma_block(kt, voff + i * NW * 1024, lk + i * NW * 1024);
  };
  auto issue_v = [&](int j, uint16_t* dv) {
    const char* vt = reinterpret_cast<const char*>(vimg + (size_t)j * (BN * D));
    const unsigned lv = lds_addr(dv) + wave * 1024;
#pragma unroll
    for (int i = 0; i < LPT; ++i) dma_block(vt, voff + i * NW * 1024, lv + i * NW * 1024);
  };
  auto issue = [&](int j, uint16_t* dk, uint16_t* dv) {
    issue_k(j, dk);
    issue_v(j, dv);
  };

  // One segment: query tile qt against key tiles [jb, je]; seg = 0 (long) or 1 (short).
  auto process = [&](int qt, int seg, int jb, int je, int jlo_t, int jhi_t, int us, int ue) {
    issue(jb, sk0, sv0);  // the first tile streams in while the queries are rotated

    const int r0 = qt * 128;
    const int r = r0 + rg * 32 + n;
    const bool valid = r < rows_total;
    const int rc = valid ? r : rows_total - 1;
    const int sq = fdiv(rc, a.fd_g), head = kvh * a.g + (rc - sq * a.g);  // query index within the chunk
    const int pos = a.P0 + sq;                               // its position in the sequence
    const int pos_min = a.P0 + fdiv(r0, a.fd_g);
    const int pos_max = a.P0 + fdiv(min(r0 + 127, rows_total - 1), a.fd_g);
    const int lim = causal_limit<SPAN>(a, b, sq, pos);                      // this row's last visible key
    const int lim_min = causal_limit<SPAN>(a, b, pos_min - a.P0, pos_min);  // the smallest limit of the tile

    // Q' = RoPE(q) * scale * log2(e), as the B operand of S^T = K' Q'^T:
    // lane (n, h) holds head-dim elements 16*ks + 8*h + [0, 8) of its query
    // row for the k-steps this wave owns.  Rotation partners (d, d + D/2)
    // sit in k-steps ks and ks + KSTEPS/2.
    bf16x8 qf[KSW];
    {
      const uint16_t* qrow = a.q + (((size_t)b * a.S + sq) * a.Hq + head) * D;
      // The g query heads of a position share its rotation.  When the
      // tile's positions fit, each (position, frequency) pair's cos / sin is
      // computed once by the work-group into the second key and value
      // buffers (idle until the first phase barrier of the tile schedule:
      // the segment's first tile goes to the first buffers) and read back by
      // every row of that position: the values per-row computation gives,
      // at 1/g of its double-precision and transcendental work.
      // Table row pp (position pos_min + pp) holds HF (cos, sin) pairs, two
      // frequencies per 16-byte slot; the slot index is XOR-swizzled by the
      // row so that the 16 (position, lane half) combinations one read
      // instruction touches fall in 16 distinct bank groups.
      constexpr int HF = D / 2;
      constexpr int kRowBytes = HF * 8;
      constexpr int kRowsPerBuf = (int)(sizeof(sk1) / kRowBytes);
      const int npos = pos_max - pos_min + 1;
      auto tab_slot = [&](int pp, int col) -> unsigned {  // LDS byte address of (row pp, 16-byte slot col)
        const int sw = col ^ ((pp & 3) | ((pp & 4) << 1));
        return (pp < kRowsPerBuf ? lds_addr(sk1) + pp * kRowBytes : lds_addr(sv1) + (pp - kRowsPerBuf) * kRowBytes) +
               sw * 16;
      };
      if (npos <= 2 * kRowsPerBuf) {
        // this wave's query chunks are loaded first; their latency hides
        // behind the table fill (rotated in place afterwards)
        u32x4 xq[KSW / 2], yq[KSW / 2];
#pragma unroll
        for (int i = 0; i < KSW / 2; ++i) {
          const int d0 = 16 * (dp * (KSW / 2) + i) + 8 * h;
          xq[i] = *reinterpret_cast<const u32x4*>(qrow + d0);
          yq[i] = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
        }
        static_assert(NT % HF == 0, "frequencies must tile the work-group");
        const int f = tid % HF;
        const double rev = a.rope.rev[f];
        for (int pp = tid / HF; pp < npos; pp += NT / HF) {
          float sn, cs;
          sincos_rev((double)(pos_min + pp), rev, sn, cs);
          *reinterpret_cast<__attribute__((address_space(3))) f32x2*>(tab_slot(pp, f / 2) + (f & 1) * 8) =
              f32x2{cs, sn};
        }
        lds_barrier();
        const int pp = pos - pos_min;
#pragma unroll
        for (int i = 0; i < KSW / 2; ++i) {
          const int d0 = 16 * (dp * (KSW / 2) + i) + 8 * h;  // frequencies d0 .. d0 + 7
          const u32x4 x = xq[i], y = yq[i];
          u32x4 xo, yo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (cos, sin) of frequencies d0 + 2e and d0 + 2e + 1
            const f32x4 t = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(tab_slot(pp, d0 / 2 + e));
            const float a0 = bf_lo(x[e]), a1 = bf_hi(x[e]), b0 = bf_lo(y[e]), b1 = bf_hi(y[e]);
            xo[e] = pack_bf16((a0 * t[0] - b0 * t[1]) * a.qscale, (a1 * t[2] - b1 * t[3]) * a.qscale);
            yo[e] = pack_bf16((b0 * t[0] + a0 * t[1]) * a.qscale, (b1 * t[2] + a1 * t[3]) * a.qscale);
          }
          qf[i] = as_bf16x8(xo);
          qf[i + KSW / 2] = as_bf16x8(yo);
        }
      } else {
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
    }

    f32x16 acc[DBW];
#pragma unroll
    for (int i = 0; i < DBW; ++i) acc[i] = f32x16{};
    float m_i = kNegInf, l_i = 0.f;

    // S^T = K' Q'^T for one tile (this wave's head-dim steps): s[mb] holds
    // keys 32*mb + 8*i + 4*h + jj (reg 4*i + jj) of query n.
    auto scores = [&](const uint16_t* ck, f32x16 (&s)[MB]) {
      const u32x4* kb = reinterpret_cast<const u32x4*>(ck) + lane;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int i = 0; i < KSW; ++i) {
          const int ks = i < KSW / 2 ? dp * (KSW / 2) + i : KSTEPS / 2 + dp * (KSW / 2) + (i - KSW / 2);
          s[mb] = mfma32(as_bf16x8(kb[(mb * KSTEPS + ks) * 64]), qf[i], s[mb]);
        }
      }
      lds_mfma_pipeline<MB * KSW, kPipeDepth>();
    };
    // The two halves of a head-dim sum meet in LDS: each wave of a pair
    // publishes its partial scores, and after a barrier adds the partner's
    // (float addition is commutative, so both waves get identical scores).
    auto publish = [&](const f32x16 (&s)[MB]) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          sx[wave][mb][qd][lane] = f32x4{s[mb][4 * qd], s[mb][4 * qd + 1], s[mb][4 * qd + 2], s[mb][4 * qd + 3]};
    };
    auto add_partner = [&](f32x16 (&s)[MB]) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 o = sx[wave ^ 1][mb][qd][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) s[mb][4 * qd + e] += o[e];
        }
    };

    // Mask and online softmax of key tile j: P^T (bf16, MFMA B-operand order) into pk.
    auto softmax = [&](int j, f32x16 (&s)[MB], unsigned (&pk)[MB * 8]) __attribute__((always_inline)) {
      const int kbase = j * BN;
      const bool need_mask = (kbase + BN - 1 > lim_min) || (windowed && kbase <= pos_max - a.W);
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = kbase + 32 * mb + 8 * (rr >> 2) + 4 * h + (rr & 3);
            const bool vis = (key <= lim) & (!windowed | (pos - key < a.W));
            s[mb][rr] = vis ? s[mb][rr] : kNegInf;
          }
      }

      // Online softmax in the log2 domain; lanes n and n+32 share query n.
      // The reference maximum m_i only moves when a score exceeds it by more
      // than kRescaleSlack, so P = 2^(s - m_i) <= 2^kRescaleSlack and the
      // MFMA accumulators are rescaled only on those (rare) tiles.
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[mb][rr]);
      mx = max_lane_pair(mx);
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
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2) {
          const float p0 = fast_exp2(s[mb][rr] - m_use), p1 = fast_exp2(s[mb][rr + 1] - m_use);
          rs += p0 + p1;
          pk[mb * 8 + rr / 2] = pack_bf16(p0, p1);
        }
      l_i += rs;
    };
    // O^T += V^T P^T.  P^T slot t of key-step kv is key 16*kv + 4*h + t (t < 4)
    // or 16*kv + 8 + 4*h + (t - 4): the value image stores V in that order.
    auto pv = [&](const unsigned (&pk)[MB * 8], const uint16_t* cv) {
      const u32x4* vb = reinterpret_cast<const u32x4*>(cv) + lane;
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        const bf16x8 pf = as_bf16x8(u32x4{pk[4 * kv], pk[4 * kv + 1], pk[4 * kv + 2], pk[4 * kv + 3]});
#pragma unroll
        for (int db = 0; db < DBW; ++db)
          acc[db] = mfma32(as_bf16x8(vb[(kv * DB + dp * DBW + db) * 64]), pf, acc[db]);
      }
      lds_mfma_pipeline<KV * DBW, kPipeDepth>();
    };
    auto softmax_pv = [&](int j, f32x16 (&s)[MB], const uint16_t* cv) {
      unsigned pk[MB * 8];
      softmax(j, s, pk);
      pv(pk, cv);
    };

    // The same two steps with the operand reads pipelined by hand (a ring of
    // kPipeDepth reads in flight, the order pinned step by step) and a hook
    // after every MFMA, which the two-group schedule uses to spread its tile
    // copies over the MFMAs: issued back to back they hold the wave, and so
    // its share of the MFMA pipe, until the memory pipeline takes them.
    auto scores_h = [&](const uint16_t* ck, f32x16 (&s)[MB], auto&& hook) __attribute__((always_inline)) {
      const u32x4* kb = reinterpret_cast<const u32x4*>(ck) + lane;
      constexpr int N = MB * KSW;
      auto kaddr = [&](int t) {
        const int mb = t / KSW, i = t % KSW;
        const int ks = i < KSW / 2 ? dp * (KSW / 2) + i : KSTEPS / 2 + dp * (KSW / 2) + (i - KSW / 2);
        return (mb * KSTEPS + ks) * 64;
      };
      u32x4 kr[kPipeDepth];
#pragma unroll
      for (int t = 0; t < kPipeDepth; ++t) kr[t] = kb[kaddr(t)];
#pragma unroll
      for (int t = 0; t < N; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 kf = as_bf16x8(kr[t % kPipeDepth]);
        if (t + kPipeDepth < N) kr[t % kPipeDepth] = kb[kaddr(t + kPipeDepth)];
        const int mb = t / KSW, i = t % KSW;
        s[mb] = mfma32(kf, qf[i], i == 0 ? f32x16{} : s[mb]);
        hook(t);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // O^T += V^T P^T for the 16-key step kv only (DBW MFMAs).
    auto pv_kv = [&](auto kv_c, const u32x4& pf, const uint16_t* cv, auto&& hook) __attribute__((always_inline)) {
      constexpr int kv = decltype(kv_c)::value;
      const u32x4* vb = reinterpret_cast<const u32x4*>(cv) + lane + (kv * DB + dp * DBW) * 64;
      u32x4 vr[kPipeDepth];
#pragma unroll
      for (int u = 0; u < kPipeDepth; ++u) vr[u] = vb[u * 64];
#pragma unroll
      for (int t = 0; t < DBW; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 vf = as_bf16x8(vr[t % kPipeDepth]);
        if (t + kPipeDepth < DBW) vr[t % kPipeDepth] = vb[(t + kPipeDepth) * 64];
        acc[t] = mfma32(vf, as_bf16x8(pf), acc[t]);
        hook(t);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto pv_hd = [&](const unsigned (&pk)[MB * 8], const uint16_t* cv, auto&& hook) __attribute__((always_inline)) {
      const u32x4* vb = reinterpret_cast<const u32x4*>(cv) + lane;
      constexpr int N = KV * DBW;
      u32x4 vr[kPipeDepth];
#pragma unroll
      for (int u = 0; u < kPipeDepth; ++u) vr[u] = vb[((u / DBW) * DB + dp * DBW + u % DBW) * 64];
#pragma unroll
      for (int t = 0; t < N; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 vf = as_bf16x8(vr[t % kPipeDepth]);
        if (t + kPipeDepth < N) {
          const int u = t + kPipeDepth;
          vr[t % kPipeDepth] = vb[((u / DBW) * DB + dp * DBW + u % DBW) * 64];
        }
        const int kv = t / DBW, db = t % DBW;
        const bf16x8 pf = as_bf16x8(u32x4{pk[4 * kv], pk[4 * kv + 1], pk[4 * kv + 2], pk[4 * kv + 3]});
        acc[db] = mfma32(vf, pf, acc[db]);
        hook(t);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (DS == 1) {
      auto step = [&](int j, const uint16_t* ck, const uint16_t* cv, uint16_t* nk, uint16_t* nv) {
        wait_vm<0>();  // this wave's share of tile j has landed
        lds_barrier();  // everybody's share has, and tile j-1 is no longer being read
        if (j < je) issue(j + 1, nk, nv);
        f32x16 s[MB];
        scores(ck, s);
        softmax_pv(j, s, cv);
      };
      for (int j = jb;;) {
        step(j, sk0, sv0, sk1, sv1);
        if (++j > je) break;
        step(j, sk1, sv1, sk0, sv0);
        if (++j > je) break;
      }
    } else {
      if constexpr (SPV) {
      // Two wave groups (waves 0-3 and 4-7, one of each per SIMD) run the
      // same tile sequence half a step apart.  A group's step on tile i has
      // two phases: (A) O^T += V^T P^T for tile i-1, then the partial scores
      // of tile i; (B) the partner's half of the scores and the softmax of
      // tile i for this wave's 16 keys.  Phase t: group g works on u = t - g
      // (even u: phase A of tile jb + u/2, odd u: phase B of tile
      // jb + (u-1)/2); after the last tile one more phase A holds only its
      // PV.  In every phase one wave of each SIMD runs 32 MFMAs while the
      // other adds its partner's scores and runs the softmax.
      //
      // LDS exchange slot sx[w] of wave w: its partial scores of tile i
      // (written in phase A of tile i, read by the partner in phase B), then
      // the partner's probabilities of tile i (written by the partner in
      // phase B after reading the scores, read by w in the next phase A
      // before it writes its next scores there).
      //
      // Copies: at every even phase t < 2 nt each wave copies its share of
      // key tile t/2 + 1 and value tile max(t/2, 1) (relative to jb) into
      // the buffers their predecessors two tiles back have left (key tile j
      // is read in phases 2j .. 2j+1, value tile j in 2j+2 .. 2j+3), so every
      // copy has two phases to land.  A tile past the segment's end is
      // replaced by its last tile (its buffer is free and never read again
      // in the segment), so every even phase issues the same 2 * LPT copies.
      // Phase-A waves spread them over their MFMAs; phase-B waves issue them
      // at the start of the phase.
      static_assert(MB == 1 && KV == 2, "one 32-key block per tile");
      const int grp = wave >> 2;
      const int nt = je - jb + 1;
      // Copies of phase t: even t, key tile t/2 + 1 (LPT blocks) and the
      // second 16-key half of value tile t/2 (LPT/2 blocks); odd t, the
      // first half of value tile (t+1)/2 (LPT/2 blocks); none from 2 nt on.
      // A value tile's first half is read in phase B of its tile, its
      // second half in the next phase A, so each half has its own two-phase
      // window and every copy has two phases to land.
      auto ncopies = [&](int t) { return (t < 0 || t >= 2 * nt) ? 0 : ((t & 1) ? LPT / 2 : LPT + LPT / 2); };
      auto phase_begin = [&](int t) {
        // Copies issued during phase t - 1 are first read in phase t + 1 and
        // may stay in flight; everything older must have landed.
        const int n = ncopies(t - 1);
        if (n == LPT + LPT / 2)
          wait_vm<LPT + LPT / 2>();
        else if (n == LPT / 2)
          wait_vm<LPT / 2>();
        else
          wait_vm<0>();
        lds_barrier();
      };
      // Block c (< ncopies(t)) of this wave's copies of phase t.
      auto copy_blk = [&](int t, int c) {
        bool isv;
        int jr, u;
        if (t & 1) {
          isv = true, jr = (t + 1) / 2, u = c;  // value blocks wave + u NW, u < LPT/2: first half
        } else if (c < LPT) {
          isv = false, jr = t / 2 + 1, u = c;
        } else {
          isv = true, jr = t / 2, u = LPT / 2 + (c - LPT);  // second half
        }
        const char* src = reinterpret_cast<const char*>((isv ? vimg : kimg) + (size_t)min(jb + jr, je) * (BN * D));
        uint16_t* dst = isv ? ((jr & 1) ? sv1 : sv0) : ((jr & 1) ? sk1 : sk0);
        dma_block(src, voff + u * NW * 1024, lds_addr(dst) + wave * 1024 + u * NW * 1024);
      };
      auto copy_all = [&](int t) {
#pragma unroll
        for (int c = 0; c < LPT + LPT / 2; ++c) copy_blk(t, c);
      };
      static_assert(LPT == 4 && DBW == 8 && KSW == 16, "copy hooks below assume this tile split");
      using K0 = std::integral_constant<int, 0>;
      using K1 = std::integral_constant<int, 1>;
      auto run = [&](auto g_c) __attribute__((always_inline)) {
        constexpr int G = decltype(g_c)::value;
        unsigned pk[MB * 8];
        f32x16 s[MB];
        if (G == 1) {
          phase_begin(0);
          copy_all(0);
        }
        phase_begin(G);  // phase A of tile 0: scores only
        if (G == 0)
          scores_h(sk0, s, [&](int st) { if (st % 2 == 1 && st / 2 < 6) copy_blk(0, st / 2); });
        else
          scores_h(sk0, s, [&](int st) { if (st % 4 == 1 && st / 4 < 2) copy_blk(1, st / 4); });
        publish(s);
        // Phase B of tile i: the partner's scores, the softmax, the PV of the
        // first 16-key step; then the barrier that opens phase A of tile i + 1.
        auto phase_b = [&](int i, auto copies_c) __attribute__((always_inline)) {
          const int tb = 2 * i + 1 + G;
          phase_begin(tb);
          add_partner(s);
          softmax(jb + i, s, pk);
          const u32x4 pf0{pk[0], pk[1], pk[2], pk[3]};
          if constexpr (!decltype(copies_c)::value)
            pv_kv(K0{}, pf0, (i & 1) ? sv1 : sv0, [](int) {});
          else if constexpr (G == 1)  // even phase: six copies
            pv_kv(K0{}, pf0, (i & 1) ? sv1 : sv0, [&](int st) { if (st < 6) copy_blk(tb, st); });
          else  // odd phase: two copies
            pv_kv(K0{}, pf0, (i & 1) ? sv1 : sv0, [&](int st) { if (st % 4 == 1) copy_blk(tb, st / 4); });
          phase_begin(tb + 1);
        };
        for (int i = 0; i + 1 < nt; ++i) {
          phase_b(i, std::true_type{});
          const int ta = 2 * i + 2 + G;
          const u32x4 pf1{pk[4], pk[5], pk[6], pk[7]};
          const uint16_t* cv = (i & 1) ? sv1 : sv0;
          if (G == 0) {  // even phase: six copies
            pv_kv(K1{}, pf1, cv, [&](int st) { if (st % 4 == 1) copy_blk(ta, st / 4); });
            scores_h(((i + 1) & 1) ? sk1 : sk0, s, [&](int st) { if (st % 4 == 1) copy_blk(ta, 2 + st / 4); });
          } else {  // odd phase: two copies
            pv_kv(K1{}, pf1, cv, [&](int st) { if (st % 4 == 1) copy_blk(ta, st / 4); });
            scores_h(((i + 1) & 1) ? sk1 : sk0, s, [](int) {});
          }
          publish(s);
        }
        if (G == 0)
          phase_b(nt - 1, std::true_type{});  // phase 2 nt - 1: two copies (past the end)
        else
          phase_b(nt - 1, std::false_type{});
        pv_kv(K1{}, u32x4{pk[4], pk[5], pk[6], pk[7]}, ((nt - 1) & 1) ? sv1 : sv0, [](int) {});
        if (G == 0) phase_begin(2 * nt + 1);
      };
      if (grp == 0)
        run(std::integral_constant<int, 0>{});
      else
        run(std::integral_constant<int, 1>{});
      wait_vm<0>();
      } else {
      // Two wave groups (waves 0-3 and 4-7, one of each per SIMD) run the
      // same tile sequence half a step apart: in every phase one group
      // computes scores for tile i while the other finishes tile i-1
      // (partner scores, softmax, PV), so each SIMD always has MFMA work
      // from one wave while the other waits on LDS or runs the softmax.
      // Phase t: group g works on u = t - g; even u = scores of tile jb + u/2,
      // odd u = softmax and PV of tile jb + (u-1)/2.  Key tile j lives in
      // buffer (j - jb) & 1 during phases 2(j-jb) .. 2(j-jb)+1 and value tile
      // j during phases 2(j-jb)+1 .. 2(j-jb)+2; the next key tile is copied
      // during even phases and the next value tile during odd ones, each
      // into the buffer its predecessor has just left, spread over the
      // phase's MFMAs (scores or PV, whichever the wave is running).
      const int grp = wave >> 2;
      const int nt = je - jb + 1;
      auto phase_begin = [&](int t) {
        // Copies issued during phase t - 1 are first read in phase t + 1 and
        // may stay in flight; everything older must have landed.
        if (t > 0 && jb + (t - 1) / 2 + 1 <= je)
          wait_vm<LPT>();
        else
          wait_vm<0>();
        lds_barrier();
      };
      // The copies of phase t (key tile jn for even t, value tile jn for odd
      // t, jn = jb + t/2 + 1), one block after every fourth MFMA of the phase.
      // Past the segment's last tile the copy repeats that tile into the
      // buffer it would fill (no wave reads it again in this segment), so
      // every phase issues the same number of copies and the MFMA chains
      // carry no branches.
      auto copy_hook = [&](int t) {
        const int jn = jb + t / 2 + 1;  // decides the buffer, which is free either way
        const char* src = reinterpret_cast<const char*>(((t & 1) ? vimg : kimg) + (size_t)min(jn, je) * (BN * D));
        uint16_t* dst = (t & 1) ? (((jn - jb) & 1) ? sv1 : sv0) : (((jn - jb) & 1) ? sk1 : sk0);
        const unsigned ld = lds_addr(dst) + wave * 1024;
        return [=](int st) {
          if (st % 4 == 1) dma_block(src, voff + (st / 4) * NW * 1024, ld + (st / 4) * NW * 1024);
        };
      };

      static_assert(MB * KSW >= 4 * LPT && KV * DBW >= 4 * LPT, "each phase's MFMAs must carry its copies");
      if (grp == 1) {
        phase_begin(0);
        const int jn = jb + 1;
        if (jn <= je) issue_k(jn, sk1);
      }
      for (int i = 0; i < nt; ++i) {
        f32x16 s[MB];
        const int ta = 2 * i + grp, tb = ta + 1;
        phase_begin(ta);
        scores_h((i & 1) ? sk1 : sk0, s, copy_hook(ta));
        publish(s);
        phase_begin(tb);
        const uint16_t* cv = (i & 1) ? sv1 : sv0;
        add_partner(s);
        unsigned pk[MB * 8];
        softmax(jb + i, s, pk);
        pv_hd(pk, cv, copy_hook(tb));
      }
      if (grp == 0) phase_begin(2 * nt);
      wait_vm<0>();  // the repeated copies of the last phases
      }
    }

    if (jb != jlo_t || je != jhi_t) {
      // Partial: store (O, m, l), then count this piece in.
      const size_t slot_f4 = (size_t)ACC_F4 + NW * 64 / 2;  // f32x4 units per slot (m and l: NW*64 floats each)
      auto slot_ptr = [&](int pc) {
        return reinterpret_cast<f32x4*>(a.part) + (((size_t)bh * a.npair + pair) * a.kpieces + pc) * 2 * slot_f4 +
               (size_t)seg * slot_f4;
      };
      // Partials go through the device-coherent path (sc1: stores write
      // through the XCD's L2 and loads do not trust it), so publishing them
      // needs no L2-wide write-back or invalidation: wait for this
      // work-group's stores, then bump the tile's counter.  Slot layout
      // (bytes): accumulator quad (w * DBW + db, qd) of lane l at
      // ((((w * DBW + db) * 4 + qd) * 64 + l) * 16), then m and l per (w, l).
      constexpr unsigned kSlotBytes = (unsigned)(ACC_F4 * 16 + NW * 64 * 2 * 4);
      constexpr int kSC1 = 16;  // cache-policy bit sc1 of the buffer instructions
      auto slot_rsrc = [&](int pc) {
        return __builtin_amdgcn_make_buffer_rsrc(slot_ptr(pc), 0, (int)kSlotBytes, 0x00020000);
      };
      const unsigned acc_off = (unsigned)((wave * DBW * 4 * 64 + lane) * 16);
      const unsigned ml_off = (unsigned)(ACC_F4 * 16 + (wave * 64 + lane) * 4);
      {
        const auto r = slot_rsrc(piece);
#pragma unroll
        for (int db = 0; db < DBW; ++db)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, f32x4{acc[db][4 * qd], acc[db][4 * qd + 1], acc[db][4 * qd + 2],
                                                acc[db][4 * qd + 3]}),
                r, acc_off + (db * 4 + qd) * 1024, 0, kSC1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_i), r, ml_off, 0, kSC1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_i), r, ml_off + NW * 64 * 4, 0, kSC1);
      }
      wait_vm<0>();  // the stores above have landed
      __syncthreads();
      auto is_piece = [&](int pc) {
        const int x0 = ubound(pc), x1 = ubound(pc + 1);
        return x0 < x1 && x0 < ue && x1 > us;
      };
      int npieces = 0;
      for (int pc = 0; pc < a.kpieces; ++pc) npieces += is_piece(pc) ? 1 : 0;
      // The arrival flag lives in the first word of a key buffer: no tile is
      // in flight when it is written and read.
      int* s_last = reinterpret_cast<int*>(sk0);
      if (tid == 0) {
        // The last piece also resets the counter (every other piece has
        // counted in already), so a finished launch leaves all counters zero
        // for the next call on this workspace, which may skip the key pass
        // that zeroes them (images_ready).
        int* ctr = &a.counters[(size_t)bh * a.nqt + qt];
        const bool is_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == npieces - 1;
        if (is_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = is_last;
      }
      __syncthreads();
      const bool last = *s_last != 0;
      __syncthreads();  // the buffer is refilled by the next segment
      if (!last) return;
      // Deterministic merge: the result must not depend on which piece came
      // last, so every piece (this one re-read from its own slot) is added in
      // ascending piece order against the common maximum of all pieces:
      // t = O_0 f_0, t = fma(O_k, f_k, t).  A tile cut into at most four
      // pieces is merged by straight-line code (one batch of (m, l) loads,
      // then the accumulator chunks streamed with the next chunk's loads in
      // flight); the pieces' indices need not be consecutive (empty pieces
      // are skipped).
      int pcs[4] = {0, 0, 0, 0}, nfound = 0;
      for (int pc = 0; pc < a.kpieces; ++pc)
        if (is_piece(pc)) {
          if (nfound < 4) pcs[nfound] = pc;
          ++nfound;
        }
      auto merge_np = [&](auto np_c) __attribute__((always_inline)) {
        constexpr int NP = decltype(np_c)::value;
        float f[NP];
        {
          float mp[NP], lp[NP];
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            const auto r = slot_rsrc(pcs[k]);
            mp[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ml_off, 0, kSC1));
            lp[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ml_off + NW * 64 * 4, 0, kSC1));
          }
          float M = mp[0];
#pragma unroll
          for (int k = 1; k < NP; ++k) M = fmaxf(M, mp[k]);
          float lsum = 0.f;
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            f[k] = mp[k] == kNegInf ? 0.f : fast_exp2(mp[k] - M);
            lsum = k == 0 ? lp[0] * f[0] : __builtin_fmaf(lp[k], f[k], lsum);
          }
          l_i = lsum;
          m_i = M;
        }
        constexpr int NG = DBW * 2;  // (head-dim block, half of its quads)
        f32x4 chunk[2][NP][2];
        auto load_group = [&](int g, int sl) {
          const int db = g / 2, q0 = 2 * (g % 2);
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            const auto r = slot_rsrc(pcs[k]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
              chunk[sl][k][j] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, acc_off + (db * 4 + q0 + j) * 1024, 0, kSC1));
          }
        };
        load_group(0, 0);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g + 1 < NG) load_group(g + 1, (g + 1) & 1);
          const int db = g / 2, q0 = 2 * (g % 2);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float t = 0.f;
#pragma unroll
              for (int k = 0; k < NP; ++k) {
                const float v = chunk[g & 1][k][j][e];
                t = k == 0 ? v * f[0] : __builtin_fmaf(v, f[k], t);
              }
              acc[db][4 * (q0 + j) + e] = t;
            }
        }
      };
      if (npieces == 2) {
        merge_np(std::integral_constant<int, 2>{});
      } else if (npieces == 3) {
        merge_np(std::integral_constant<int, 3>{});
      } else if (npieces == 4) {
        merge_np(std::integral_constant<int, 4>{});
      } else {
      // the pieces' maxima, eight loads per round trip
      float M = kNegInf;
      for (int pc0 = 0; pc0 < a.kpieces; pc0 += 8) {
        float mv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int pc = pc0 + k;
          mv[k] = (pc < a.kpieces && is_piece(pc))
                      ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(slot_rsrc(pc), ml_off, 0, kSC1))
                      : kNegInf;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) M = fmaxf(M, mv[k]);
      }
#pragma unroll
      for (int db = 0; db < DBW; ++db) acc[db] = f32x16{};
      l_i = 0.f;
      for (int pc = 0; pc < a.kpieces; ++pc) {
        if (!is_piece(pc)) continue;
        const auto r = slot_rsrc(pc);
        const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ml_off, 0, kSC1));
        const float lp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ml_off + NW * 64 * 4, 0, kSC1));
        const float f = mp == kNegInf ? 0.f : fast_exp2(mp - M);
        l_i += lp * f;
#pragma unroll
        for (int db = 0; db < DBW; ++db)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x4 v = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, acc_off + (db * 4 + qd) * 1024, 0, kSC1));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[db][4 * qd + e] += v[e] * f;
          }
      }
      m_i = M;
      }
    }

    const float l = l_i + __shfl_xor(l_i, 32);
    const float inv = l > 0.f ? a.vscale / l : 0.f;
    // (the row's coordinates are recomputed here rather than kept live
    // through the tile loop, where every register is taken)
    const int r_o = __builtin_amdgcn_readfirstlane(r0) + rg * 32 + n;
    if (r_o < rows_total) {
      const int sq_o = fdiv(r_o, a.fd_g), head_o = kvh * a.g + (r_o - sq_o * a.g);
      float* orow = a.out + (((size_t)b * a.S + sq_o) * a.Hq + head_o) * D + 32 * dp * DBW;
#pragma unroll
      for (int db = 0; db < DBW; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 o = {acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv,
                     acc[db][4 * i + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i + 4 * h) = o;
        }
    }
  };

  if (u0 < u1) {
    if (u0 < nL) process(tl, 0, jlo_l + u0, jlo_l + min(u1, nL) - 1, jlo_l, jhi_l, 0, nL);
    if (u1 > nL) {
      if (u0 < nL) lds_barrier();  // the first segment's last tile may still be in use
      process(ts, 1, jlo_s + max(u0, nL) - nL, jlo_s + u1 - nL - 1, jlo_s, jhi_s, nL, U);
    }
  }
}

// Score MFMAs of the four-wave prefill, written as asm so that their
// accumulators stay in VGPRs: the compiler would otherwise put every MFMA
// result of the kernel in AGPRs, where the output accumulators already take
// all 256.  The first MFMA of a chain starts from zero; consecutive MFMAs
// accumulating into the same registers need no wait states between them,
// and the last one of a chain is followed by 24 wait states so that no
// later instruction reads its result early (the compiler does not know
// these are MFMAs and cannot insert them).
__device__ __forceinline__ void mfma32v_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32v_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d) : "v"(a), "v"(b));
}
// The same for the 16x16x32 score chains of 64-row tiles (two chains,
// interleaved; the wait states after the last MFMA cover both).
__device__ __forceinline__ void mfma16v_first(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16v(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16v_last(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d) : "v"(a), "v"(b));
}

// Four-wave prefill, one wave per SIMD (register budget 512 per lane), for
// one 128-row query tile of one (batch, kv-head) at a time; BN-key tiles.
//
//   scores : wave w owns query rows 32w .. 32w+31 over the whole head dim
//            (queries rotated once into registers), so its S^T = K' Q'^T
//            needs no exchange and its softmax statistics stay in the wave;
//   output : wave w owns head-dim blocks [w*DBW, (w+1)*DBW) of all 128 rows,
//            O^T += V^T P^T, with the four row blocks' P^T (bf16) and
//            rescale factors exchanged through LDS.  Each value operand read
//            from LDS then feeds four MFMAs.
//
// Software pipeline, one barrier per key tile: iteration i (key tile
// jb + i) waits for the copies issued in iteration i-1, passes the barrier,
// issues key tile i+1 and value tile i, computes S(i), then runs PV(i-1)
// (whose P and rescale factors were published in iteration i-1) while the
// softmax of S(i) runs, and publishes P(i).  Key tile i lives in key buffer
// i&1 during iterations i-1 .. i, value tile i in value buffer i&1 during
// iterations i .. i+1, P(i) in exchange buffer i&1 during i .. i+1.
// The work split over work-groups (pairs of query tiles, pieces of their
// key work) and the partial-result merge follow k_prefill.
//
// PROD (64-row tiles): four more waves, one per SIMD beside each compute
// wave, issue every tile copy in place of the compute waves.  A
// direct-to-LDS copy holds its issuing wave until the memory pipeline takes
// it (about 35 cycles each, eight per wave and tile), time the compute
// waves otherwise lose inside their score chains.  A producer wave runs a
// code path of its own with exactly the compute waves' sequence of
// barriers, and no compute.
template <int D, int BN, int ROWS, bool SPAN, bool PROD>
__global__ __attribute__((amdgpu_flat_work_group_size(PROD ? 512 : 256, PROD ? 512 : 256),
                          amdgpu_waves_per_eu(PROD ? 2 : 1, PROD ? 2 : 1))) void
k_prefill4(PrefillArgs a) {
  G4_PREFETCH_PREFILL_ARGS(a);
  static_assert(ROWS == 128 || ROWS == 64, "query tile of 128 or 64 rows");
  static_assert(!PROD || ROWS == 64, "producer waves fit beside the registers of 64-row tiles only");
  static_assert(D == 256, "one wave per SIMD holds the queries and output block of head size 256 only");
  constexpr bool R64 = ROWS == 64;   // 16 score rows per wave (16x16x32 MFMAs), no split pieces
  constexpr int KSTEPS = D / 16;     // 32x32x16 steps over the head dim
  constexpr int MB = BN / 32;        // 32-key blocks per tile
  constexpr int KV = BN / 16;        // 16-key steps per tile
  constexpr int DB = D / 32;         // 32-wide output blocks
  constexpr int DBW = DB / 4;        // output blocks owned by one wave
  constexpr int RB = ROWS / 32;      // 32-row blocks of the output MFMAs
  constexpr int SR = ROWS / 4;       // query rows whose scores one wave computes
  constexpr int NQ = R64 ? D / 64 : D / 32;  // (d, d + D/2) query chunk pairs per lane
  static_assert(!R64 || BN == 32, "64-row tiles use 32-key tiles");
  constexpr int TILE_BLKS = BN * D * 2 / 1024;
  constexpr int LPT = TILE_BLKS / 4;  // 1 KiB blocks each wave copies per tile and operand
  constexpr int ACC_F4 = 4 * RB * DBW * 4 * 64;  // f32x4 per partial slot (accumulators)
  constexpr int kPipeDepth = G4_PIPE_DEPTH;
  static_assert(LPT * 4 == TILE_BLKS, "tile must split evenly over the waves");

  // Key tiles kvb[0..1], value tiles kvb[2..3].
  __shared__ __attribute__((aligned(1024))) uint16_t kvb[4][BN * D];
  uint16_t (*const sk)[BN * D] = kvb;
  uint16_t (*const sv)[BN * D] = kvb + 2;
  __shared__ u32x4 sp[2][RB][KV][64];  // P^T operand of each row block, per 16-key step
  // Query-rotation table (cos, sin) per (position, frequency) of a segment;
  // a region of its own, so that a segment's first tile copies are already
  // in flight while its queries are rotated.
  __shared__ __attribute__((aligned(16))) f32x2 rtab[65536 / sizeof(f32x2)];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int j16 = lane & 15, grp = lane >> 4;  // 64-row tiles: score lane = (row j16, key group grp)
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = PROD && wave_id >= 4;  // wave-uniform
  // a compute wave, or the compute wave whose share of the copies a producer issues
  const int wave = PROD ? (wave_id & 3) : wave_id;
  constexpr int NTH = PROD ? 512 : 256;  // threads

  const int nblk = gridDim.x;
  const int wid = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int per_bh = a.npair * a.kpieces;
  // (the 128-row instantiation keeps plain divisions: with the multiplier
  // form its compiler output demotes the query fragments to scratch)
  const int bh = R64 ? fdiv(wid, a.fd_pbh) : wid / per_bh, rem = wid - bh * per_bh;
  const int pair = R64 ? fdiv(rem, a.fd_kp) : rem / a.kpieces, piece = rem - pair * a.kpieces;
  const int b = R64 ? fdiv(bh, a.fd_hkv) : bh / a.Hkv, kvh = bh - b * a.Hkv;
  const int rows_total = a.S * a.g;
  const bool windowed = a.W > 0;

  auto tile_keys = [&](int qt, int& jlo, int& jhi) {
    const int r0 = qt * ROWS;
    const int rl = min(r0 + ROWS - 1, rows_total - 1);
    const int pmin = a.P0 + (R64 ? fdiv(r0, a.fd_g) : r0 / a.g), pmax = a.P0 + (R64 ? fdiv(rl, a.fd_g) : rl / a.g);
    jlo = (windowed ? max(0, pmin - a.W + 1) : 0) / BN;
    jhi = causal_limit<SPAN>(a, b, pmax - a.P0, pmax) / BN;
  };
  const int tl = a.paired ? a.nqt - 1 - pair : pair;
  const int ts = a.paired && pair < tl ? pair : -1;
  int jlo_l, jhi_l, jlo_s = 0, jhi_s = -1;
  tile_keys(tl, jlo_l, jhi_l);
  if (ts >= 0) tile_keys(ts, jlo_s, jhi_s);
  const int nL = jhi_l - jlo_l + 1, nS = ts >= 0 ? jhi_s - jlo_s + 1 : 0, U = nL + nS;
  auto ubound = [&](int j) { return R64 ? fdiv(j * U, a.fd_kp) : (int)(((long long)j * U) / a.kpieces); };
  const int u0 = ubound(piece), u1 = ubound(piece + 1);

  const size_t slice_off = (size_t)(b * a.Hkv + kvh) * a.ntiles * (size_t)(BN * D);
  const uint16_t* kimg = a.kimg + slice_off;
  const uint16_t* vimg = a.vimg + slice_off;
  const unsigned voff = (unsigned)(wave * 1024 + lane * 16);

  auto copy_block = [&](const void* g, unsigned vo, unsigned l) { dma_block(g, vo, l); };
  auto issue_k = [&](int j, uint16_t* dk) {
    const char* kt = reinterpret_cast<const char*>(kimg + (size_t)j * (BN * D));
    const unsigned lk = lds_addr(dk) + wave * 1024;
#pragma unroll
    for (int i = 0; i < LPT; ++i) copy_block(kt, voff + i * 4 * 1024, lk + i * 4 * 1024);
  };
  auto issue_v = [&](int j, uint16_t* dv) {
    const char* vt = reinterpret_cast<const char*>(vimg + (size_t)j * (BN * D));
    const unsigned lv = lds_addr(dv) + wave * 1024;
#pragma unroll
    for (int i = 0; i < LPT; ++i) copy_block(vt, voff + i * 4 * 1024, lv + i * 4 * 1024);
  };
  // Block u (< LPT) of this wave's share of one operand tile.
  auto issue_blk = [&](const uint16_t* img, int j, uint16_t* dst, int u) {
    const char* src = reinterpret_cast<const char*>(img + (size_t)j * (BN * D));
    copy_block(src, voff + u * 4 * 1024, lds_addr(dst) + wave * 1024 + u * 4 * 1024);
  };

  auto process = [&](int qt, int seg, int jb, int je, int jlo_t, int jhi_t, int us, int ue) __attribute__((always_inline)) {

    const int r0 = qt * ROWS;
    const int r = r0 + wave * SR + (R64 ? j16 : n);  // this lane's score row
    const int rc = r < rows_total ? r : rows_total - 1;
    const int sq = rc / a.g;     // query index within the chunk
    const int pos = a.P0 + sq;   // its position in the sequence
    const int rl = min(r0 + ROWS - 1, rows_total - 1);
    const int pos_min = a.P0 + (R64 ? fdiv(r0, a.fd_g) : r0 / a.g);
    const int pos_max = a.P0 + (R64 ? fdiv(rl, a.fd_g) : rl / a.g);
    const int lim = causal_limit<SPAN>(a, b, sq, pos);                      // this lane's row's last visible key
    const int lim_min = causal_limit<SPAN>(a, b, pos_min - a.P0, pos_min);  // the smallest limit of the tile
    const int nt = je - jb + 1;

    // The first two key tiles and the first value tile of a pass, issued
    // together: one memory round trip instead of two.
    auto issue_head = [&]() __attribute__((always_inline)) {
      if (PROD && !producer) return;
      issue_k(jb, sk[0]);
      issue_v(jb, sv[0]);
      if (1 < nt) issue_k(jb + 1, sk[1]);
    };
    issue_head();  // lands while the queries are loaded and rotated

    // Rotation table of the segment (see below): its positions fit when ...
    constexpr int HF = D / 2;
    const int npos = pos_max - pos_min + 1;
    const bool shared_table = (size_t)npos * HF * sizeof(f32x2) <= sizeof(rtab);
    auto fill_table = [&]() __attribute__((always_inline)) {
      // thread t fills frequency t % HF for every (NTH / HF)-th position
      static_assert(NTH % HF == 0, "frequencies must tile the work-group");
      const int f = tid % HF;
      const double rev = a.rope.rev[f];
#pragma unroll 4
      for (int pp = tid / HF; pp < npos; pp += NTH / HF) {
        float sn, cs;
        sincos_rev((double)(pos_min + pp), rev, sn, cs);
        rtab[pp * HF + f] = f32x2{cs, sn};
      }
    };

    if constexpr (PROD) {
      if (producer) {
        // The compute waves' barriers, in order: table fill (when shared),
        // then per pass: first tile, one per further tile, after the last
        // tile, two around the vote; then the output's.  Copies go out right
        // after the barrier that frees their buffers and are waited for
        // before the next one, as the compute waves did.
        if (shared_table) {
          fill_table();
          lds_barrier();
        }
        for (bool first = true;; first = false) {
          if (!first) issue_head();
          if (1 < nt)  // key tile jb has landed (copies complete in issue order)
            wait_vm<2 * LPT>();
          else
            wait_vm<LPT>();
          lds_barrier();
          for (int i = 1; i < nt; ++i) {
            wait_vm<0>();
            lds_barrier();
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
              if (i + 1 < nt) issue_blk(kimg, jb + i + 1, sk[(i + 1) & 1], u);
              issue_blk(vimg, jb + i, sv[i & 1], u);
            }
          }
          wait_vm<0>();
          lds_barrier();
          lds_barrier();  // the compute waves' votes are written
          const int* vote = reinterpret_cast<const int*>(&sk[1][0]);
          const bool any = __builtin_amdgcn_readfirstlane(vote[0] | vote[1] | vote[2] | vote[3]) != 0;
          lds_barrier();
          if (!any) break;
        }
        lds_barrier();  // the row sums of the output
        return;
      }
    }

    // Q' = RoPE(q) * scale * log2(e) for this wave's rows, whole head dim:
    // qf[ks] is the B operand of head-dim step ks.  128-row tiles (32x32x16
    // steps): lane (n, h) holds elements 16 ks + 8 h + [0, 8).  64-row tiles
    // (16x16x32 steps): lane (j16, grp) holds elements 32 ks + 8 grp + [0, 8).
    // Rotation partners sit in steps ks and ks + NQ.
    bf16x8 qf[2 * NQ];
    auto qchunk = [&](int i) { return R64 ? 32 * i + 8 * grp : 16 * i + 8 * h; };
    {
      const int head = kvh * a.g + rc % a.g;
      const uint16_t* qrow = a.q + (((size_t)b * a.S + sq) * a.Hq + head) * D;
      // The g query heads of a position share its rotation, so when the
      // tile's positions fit, each (position, frequency) pair's cos / sin is
      // computed once by the work-group into LDS (the idle tile buffers) and
      // read back by every row of that position: the same values as
      // computing them per row, at 1/g of the transcendental work.
      if (shared_table) {
        // this wave's query chunks are loaded first; their latency hides
        // behind the table fill (rotated in place afterwards)
        u32x4 xq[NQ], yq[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int d0 = qchunk(i);
          xq[i] = *reinterpret_cast<const u32x4*>(qrow + d0);
          yq[i] = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
        }
        f32x2* tab = rtab;
        fill_table();
        lds_barrier();
        const f32x4* trow = reinterpret_cast<const f32x4*>(tab + (size_t)(pos - pos_min) * HF);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int d0 = qchunk(i);
          const u32x4 x = xq[i], y = yq[i];
          u32x4 xo, yo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4 t = trow[d0 / 2 + e];  // (cos, sin) of frequencies d0 + 2e and d0 + 2e + 1
            const float a0 = bf_lo(x[e]), a1 = bf_hi(x[e]), b0 = bf_lo(y[e]), b1 = bf_hi(y[e]);
            xo[e] = pack_bf16((a0 * t[0] - b0 * t[1]) * a.qscale, (a1 * t[2] - b1 * t[3]) * a.qscale);
            yo[e] = pack_bf16((b0 * t[0] + a0 * t[1]) * a.qscale, (b1 * t[2] + a1 * t[3]) * a.qscale);
          }
          qf[i] = as_bf16x8(xo);
          qf[i + NQ] = as_bf16x8(yo);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int d0 = qchunk(i);
          u32x4 x = *reinterpret_cast<const u32x4*>(qrow + d0);
          u32x4 y = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
          rope8(x, y, a.rope.rev, d0, (double)pos, a.qscale);
          qf[i] = as_bf16x8(x);
          qf[i + NQ] = as_bf16x8(y);
        }
      }
    }

    f32x16 acc[RB][DBW];
    // Scores of one key tile for this wave's rows (layout: see scores()).
    using SArr = std::conditional_t<R64, f32x4[2], f32x16[MB]>;
    float m_i, l_i;
    float m_seen = kNegInf;  // largest score of this lane's row seen so far (log2 units)
    float m_init = kNegInf;  // reference maximum a (re)started pass begins with
    bool outgrown;           // some tile's maximum exceeded m_i + kMaxGrowth in this pass

    // S^T for this wave's rows.  128-row tiles: s[mb] holds keys
    // 32 mb + 8 i + 4 h + jj (register 4 i + jj) of query n.  64-row tiles:
    // s[mb] holds keys 16 mb + 4 grp + ii (register ii) of query j16.
    // Operand reads run kPipeDepth MFMAs ahead; sched_barrier pins that order.
    // step_hook(t) runs after MFMA t is issued (the tile copies ride there).
    auto scores = [&](const uint16_t* ck, SArr& s, auto&& after_first_reads, auto&& step_hook) {
      if constexpr (R64) {
        // 16x16x32 steps: lane (j16, grp) takes key 16 mb + j16, head dims
        // 32 ks + 8 grp + [0, 8): half (grp & 1) of lane slot 16 mb + j16 in
        // key-image block 2 ks + (grp >> 1).
        const u32x4* kb = reinterpret_cast<const u32x4*>(ck) + ((grp >> 1) * 64 + j16 + 32 * (grp & 1));
        constexpr int N = 2 * (D / 32);  // step t: key block t % 2, head-dim step t / 2
        auto kaddr = [](int t) { return 2 * (t / 2) * 64 + 16 * (t % 2); };
        u32x4 kr[kPipeDepth];
#pragma unroll
        for (int t = 0; t < kPipeDepth; ++t) kr[t] = kb[kaddr(t)];
        after_first_reads();
#pragma unroll
        for (int t = 0; t < N; ++t) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 kf = as_bf16x8(kr[t % kPipeDepth]);
          if (t + kPipeDepth < N) kr[t % kPipeDepth] = kb[kaddr(t + kPipeDepth)];
          if (t < 2)
            mfma16v_first(s[t % 2], kf, qf[t / 2]);
          else if (t == N - 1)
            mfma16v_last(s[t % 2], kf, qf[t / 2]);
          else
            mfma16v(s[t % 2], kf, qf[t / 2]);
          step_hook(t);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const u32x4* kb = reinterpret_cast<const u32x4*>(ck) + lane;
        constexpr int N = MB * KSTEPS;  // step t: key block t % MB, head-dim step t / MB
        u32x4 kr[kPipeDepth];
#pragma unroll
        for (int t = 0; t < kPipeDepth; ++t) kr[t] = kb[((t % MB) * KSTEPS + t / MB) * 64];
        after_first_reads();
#pragma unroll
        for (int t = 0; t < N; ++t) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 kf = as_bf16x8(kr[t % kPipeDepth]);
          if (t + kPipeDepth < N) {
            const int u = t + kPipeDepth;
            kr[t % kPipeDepth] = kb[((u % MB) * KSTEPS + u / MB) * 64];
          }
          const int mb = t % MB, ks = t / MB;
          if (ks == 0)
            mfma32v_first(s[mb], kf, qf[ks]);
          else if (t >= N - MB && mb == MB - 1)
            mfma32v_last(s[mb], kf, qf[ks]);
          else
            mfma32v(s[mb], kf, qf[ks]);
          step_hook(t);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Causal / window mask of key tile j; only tiles on the diagonal or at
    // the window's lower edge need one.
    auto needs_mask = [&](int j) {
      const int kbase = j * BN;
      return (kbase + BN - 1 > lim_min) || (windowed && kbase <= pos_max - a.W);
    };
    auto mask = [&](int j, SArr& s) {
      const int kbase = j * BN;
      if constexpr (R64) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int key = kbase + 16 * mb + 4 * grp + ii;
            const bool vis = (key <= lim) & (!windowed | (pos - key < a.W));
            s[mb][ii] = vis ? s[mb][ii] : kNegInf;
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = kbase + 32 * mb + 8 * (rr >> 2) + 4 * h + (rr & 3);
            const bool vis = (key <= lim) & (!windowed | (pos - key < a.W));
            s[mb][rr] = vis ? s[mb][rr] : kNegInf;
          }
      }
    };

    // Online softmax of one (masked) tile for this wave's rows.  Each row
    // keeps one reference maximum m_i: the maximum of its first tile with a
    // visible key.  Later tiles may exceed it by up to kMaxGrowth (P stays
    // below 2^kMaxGrowth, far inside fp32 / bf16 range), so the accumulators
    // are never rescaled inside the loop; a row that would exceed it marks
    // the pass as outgrown and the work-group repeats the segment from a
    // higher reference (see below).  P^T (bf16) goes to exchange buffer
    // `buf`.  Branch-free, so it shares a scheduling region with the PV MFMAs.
    // 64-row tiles: P^T of this lane's 4 + 4 keys goes to half (grp >> 1) of
    // slot 16 (wave & 1) + j16 + 32 (grp & 1) of row block wave >> 1.
    auto publish64 = [&](const unsigned (&pk)[4], int buf) {
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
        reinterpret_cast<u32x2*>(&sp[buf][wave >> 1][kv][16 * (wave & 1) + j16 + 32 * (grp & 1)])[grp >> 1] =
            u32x2{pk[2 * kv], pk[2 * kv + 1]};
    };
    auto softmax = [&](SArr& s, int buf) {
      if constexpr (R64) {
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) mx = fmaxf(mx, s[mb][ii]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = max_lane_pair(mx);
        m_seen = fmaxf(m_seen, mx);
        m_i = (m_i == kNegInf) ? mx : m_i;
        outgrown |= mx > m_i + kMaxGrowth;
        const float m_use = (m_i == kNegInf) ? 0.f : m_i;
        float rs = 0.f;
        unsigned pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float p0 = fast_exp2(s[k / 2][2 * (k % 2)] - m_use), p1 = fast_exp2(s[k / 2][2 * (k % 2) + 1] - m_use);
          rs += p0 + p1;
          pk[k] = pack_bf16(p0, p1);
        }
        l_i += rs;
        publish64(pk, buf);
      } else {
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[mb][rr]);
        mx = max_lane_pair(mx);
        m_seen = fmaxf(m_seen, mx);
        m_i = (m_i == kNegInf) ? mx : m_i;  // nothing accumulated yet: adopt
        outgrown |= mx > m_i + kMaxGrowth;
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
        // P^T slot t of key-step kv is key 16 kv + 4 h + t (t < 4) or
        // 16 kv + 8 + 4 h + (t - 4): the order the value image stores V in.
#pragma unroll
        for (int kv = 0; kv < KV; ++kv)
          sp[buf][wave][kv][lane] = u32x4{pk[4 * kv], pk[4 * kv + 1], pk[4 * kv + 2], pk[4 * kv + 3]};
      }
    };

    // O^T += V^T P^T for one key tile over all four row blocks and this
    // wave's head-dim blocks.  Operand blocks of key step kv: V (DBW blocks)
    // and P^T (one per row block).
    struct PvOps {
      u32x4 v[DBW];
      u32x4 p[RB];
    };
    auto load_ops = [&](const uint16_t* cv, int buf, int kv, PvOps& o) {
      const u32x4* vb = reinterpret_cast<const u32x4*>(cv) + lane;
#pragma unroll
      for (int db = 0; db < DBW; ++db) o.v[db] = vb[(kv * DB + wave * DBW + db) * 64];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o.p[rb] = sp[buf][rb][kv][lane];
    };
    auto pv = [&](const uint16_t* cv, int buf) {
      PvOps o;
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        load_ops(cv, buf, kv, o);
#pragma unroll
        for (int db = 0; db < DBW; ++db)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb][db] = mfma32(as_bf16x8(o.v[db]), as_bf16x8(o.p[rb]), acc[rb][db]);
      }
    };

    // PV(i-1) with the softmax of S(i) woven in: PV MFMA t is followed by
    // softmax stage t (row maximum; reference update; one pair of
    // exponentials per stage; sum and P^T publication at the end), so the
    // VALU work issues while the MFMAs run.  sched_barrier pins the order for
    // the machine scheduler, and an empty asm that takes each stage's result
    // keeps the IR optimisers from sinking the stage to its first use.  The operands of key step 0 arrive in `o0` (loaded during the
    // score chain); those of step kv+1 are read at the start of step kv.
    auto pv_softmax = [&](const uint16_t* cv, int pbuf, PvOps& o0, SArr& s, int sbuf) {
      constexpr int PER_KV = DBW * RB;
      constexpr int NM = KV * PER_KV;
      constexpr int NPAIR = R64 ? 4 : MB * 8;  // exponential pairs per lane
      // score pair k of this lane (first element's block and register)
      auto pmb = [](int k) { return R64 ? k / 2 : k / 8; };
      auto prr = [](int k) { return R64 ? 2 * (k % 2) : 2 * (k % 8); };
      PvOps o1;
      float mx = kNegInf, m_use = 0.f, rs = 0.f;
      unsigned pk[NPAIR];
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int kv = t / PER_KV, db = (t / RB) % DBW, rb = t % RB;
        PvOps& cur = (kv & 1) ? o1 : o0;
        PvOps& nxt = (kv & 1) ? o0 : o1;
        if (t % PER_KV == 0 && kv + 1 < KV) load_ops(cv, pbuf, kv + 1, nxt);
        acc[rb][db] = mfma32(as_bf16x8(cur.v[db]), as_bf16x8(cur.p[rb]), acc[rb][db]);
        __builtin_amdgcn_sched_barrier(0);
        if (t == 0) {
          if constexpr (R64) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) mx = fmaxf(mx, s[mb][ii]);
          } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[mb][rr]);
          }
          asm volatile("" : "+v"(mx));
        } else if (t == 1) {
          if constexpr (R64) mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = max_lane_pair(mx);
          m_seen = fmaxf(m_seen, mx);
          m_i = (m_i == kNegInf) ? mx : m_i;  // nothing accumulated yet: adopt
          outgrown |= mx > m_i + kMaxGrowth;
          m_use = (m_i == kNegInf) ? 0.f : m_i;
          asm volatile("" : "+v"(m_use));
        } else if (t - 2 < NPAIR) {
          const int k = t - 2, mb = pmb(k), rr = prr(k);
          const float p0 = fast_exp2(s[mb][rr] - m_use), p1 = fast_exp2(s[mb][rr + 1] - m_use);
          rs += p0 + p1;
          pk[k] = pack_bf16(p0, p1);
          asm volatile("" : "+v"(pk[k]), "+v"(rs));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = NM - 2; k < NPAIR; ++k) {  // pairs left over when there are few MFMAs
        const int mb = pmb(k), rr = prr(k);
        const float p0 = fast_exp2(s[mb][rr] - m_use), p1 = fast_exp2(s[mb][rr + 1] - m_use);
        rs += p0 + p1;
        pk[k] = pack_bf16(p0, p1);
      }
      l_i += rs;
      if constexpr (R64) {
        publish64(pk, sbuf);
      } else {
#pragma unroll
        for (int kv = 0; kv < KV; ++kv)
          sp[sbuf][wave][kv][lane] = u32x4{pk[4 * kv], pk[4 * kv + 1], pk[4 * kv + 2], pk[4 * kv + 3]};
      }
    };

    // One pass over key tiles jb..je.  Returns false when a row of the
    // work-group outgrew its reference maximum (the accumulated values are
    // then unusable); the caller repeats the pass from the largest scores
    // seen.  The pass always runs to its end, so the loop has a single exit.
    auto pass = [&](bool first) __attribute__((always_inline)) -> bool {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < DBW; ++i) acc[rb][i] = f32x16{};
      m_i = m_init;
      l_i = 0.f;
      outgrown = false;
      if (!first) issue_head();
      // key tile jb has landed (copies complete in issue order)
      if (1 < nt)
        wait_vm<2 * LPT>();
      else
        wait_vm<LPT>();
      lds_barrier();
      {
        SArr s;
        scores(sk[0], s, [] {}, [](int) {});
        if (needs_mask(jb)) mask(jb, s);
        softmax(s, 0);
      }
      for (int i = 1; i < nt; ++i) {
        wait_vm<0>();   // key tile i and value tile i-1 (issued one iteration ago) have landed
        lds_barrier();  // ... for every wave; P(i-1) is published; buffers (i+1)&1 are free
        const int pb = (i - 1) & 1;
        SArr s;
        PvOps o0;
        // The copies of key tile i+1 and value tile i are spread over the
        // score chain, one per two MFMAs: issued back to back they would hold
        // the wave (and with it the MFMA pipe) for hundreds of cycles.
        const bool more = i + 1 < nt;
        scores(sk[i & 1], s, [&] { load_ops(sv[pb], pb, 0, o0); }, [&](int t) {
          if (!PROD && t % 2 == 1 && t / 2 < 2 * LPT) {
            const int u = t / 2;
            if (u < LPT) {
              if (more) issue_blk(kimg, jb + i + 1, sk[(i + 1) & 1], u);
            } else {
              issue_blk(vimg, jb + i, sv[i & 1], u - LPT);
            }
          }
        });
        static_assert(MB * KSTEPS >= 4 * LPT, "the score chain must be long enough to carry the copies");
        if (needs_mask(jb + i)) mask(jb + i, s);
        pv_softmax(sv[pb], pb, o0, s, i & 1);
      }
      wait_vm<0>();
      lds_barrier();
      const int pb = (nt - 1) & 1;
      pv(sv[pb], pb);
      // Work-group vote on `outgrown` (the flag words live in a key buffer,
      // idle now that the last PV has read its operands).
      int* vote = reinterpret_cast<int*>(&sk[1][0]);
      const bool wave_outgrown = __builtin_amdgcn_ballot_w64(outgrown) != 0;  // all 64 lanes vote
      if (lane == 0) vote[wave] = wave_outgrown;
      lds_barrier();
      // (readfirstlane: the compiler cannot tell that an LDS read of one
      // address is uniform, and a divergent loop exit would push the copy
      // addresses out of scalar registers)
      const bool any = __builtin_amdgcn_readfirstlane(vote[0] | vote[1] | vote[2] | vote[3]) != 0;
      lds_barrier();  // the words are read before anybody refills the buffer
      return !any;
    };
    bool first = true;
    while (!pass(first)) {
      // Nothing is in flight and every wave has passed the last barrier.
      m_init = m_seen;
      first = false;
    }

    const size_t slot_f4 = (size_t)ACC_F4 + 4 * 64 / 2;
    constexpr unsigned kSlotBytes = (unsigned)(ACC_F4 * 16 + 4 * 64 * 2 * 4);
    constexpr int kSC1 = 16;
    const unsigned acc_off = (unsigned)((wave * RB * DBW * 4 * 64 + lane) * 16);  // + ((rb * DBW + db) * 4 + qd) * 1024
    auto ml_off = [&](int rb) { return (unsigned)(ACC_F4 * 16 + (rb * 64 + lane) * 4); };
    // Output row of row block rb (query n of this lane), or null past the end.
    auto out_row = [&](int rb) -> float* {
      const int rr = r0 + 32 * rb + n;
      if (rr >= rows_total) return nullptr;
      const int p = rr / a.g, hd = kvh * a.g + rr % a.g;
      return a.out + (((size_t)b * a.S + p) * a.Hq + hd) * D + 32 * wave * DBW;
    };
    if (!R64 && (jb != jlo_t || je != jhi_t)) {  // (64-row tiles are never cut into pieces)
      // Partial: store (O, m, l), then count this piece in (see k_prefill).
      auto slot_rsrc = [&](int pc) {
        f32x4* p = reinterpret_cast<f32x4*>(a.part) + (((size_t)bh * a.npair + pair) * a.kpieces + pc) * 2 * slot_f4 +
                   (size_t)seg * slot_f4;
        return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)kSlotBytes, 0x00020000);
      };
      {
        const auto rs = slot_rsrc(piece);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < DBW; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
              __builtin_amdgcn_raw_buffer_store_b128(
                  __builtin_bit_cast(u32x4, f32x4{acc[rb][db][4 * qd], acc[rb][db][4 * qd + 1], acc[rb][db][4 * qd + 2],
                                                  acc[rb][db][4 * qd + 3]}),
                  rs, acc_off + ((rb * DBW + db) * 4 + qd) * 1024, 0, kSC1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_i), rs, ml_off(wave), 0, kSC1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_i), rs, ml_off(wave) + 4 * 64 * 4, 0, kSC1);
      }
      wait_vm<0>();
      __syncthreads();
      auto is_piece = [&](int pc) {
        const int x0 = ubound(pc), x1 = ubound(pc + 1);
        return x0 < x1 && x0 < ue && x1 > us;
      };
      // The pieces covering this tile in ascending order (empty pieces, which
      // exist when there are more pieces than key tiles, are skipped, so the
      // indices need not be consecutive); the first four are kept.
      int npieces = 0, pcs[4] = {0, 0, 0, 0};
      for (int pc = 0; pc < a.kpieces; ++pc)
        if (is_piece(pc)) {
          if (npieces < 4) pcs[npieces] = pc;
          ++npieces;
        }
      const int p0 = pcs[0];
      int* s_last = reinterpret_cast<int*>(&sk[0][0]);
      if (tid == 0) {  // (the last piece resets the counter, see k_prefill)
        int* ctr = &a.counters[(size_t)bh * a.nqt + qt];
        const bool is_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == npieces - 1;
        if (is_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = is_last;
      }
      __syncthreads();
      const bool last = __builtin_amdgcn_readfirstlane(*s_last) != 0;
      __syncthreads();
      if (!last) return;
      // Deterministic merge in ascending piece order against the common
      // maximum, written straight to the output: O = sum_k f_k O_k with
      // f_k = 2^(m_k - M), accumulated as t = O_0 f_0, t = fma(O_k, f_k, t),
      // whichever piece merges (every O_k, its own included, is read back
      // from the slots).  A tile cut into NP <= 4 pieces is merged by
      // straight-line code: one
      // batch of (m, l) loads, then the accumulator chunks streamed a group
      // (row block, head-dim block, half of its quads) at a time with the
      // next group's loads in flight.
      auto merge_np = [&](auto np_c) __attribute__((always_inline)) {
        constexpr int NP = decltype(np_c)::value;
        float f[NP][RB], inv[RB];
        {
          float mp[NP][RB], lp[NP][RB];
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            const auto rs = slot_rsrc(pcs[k]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              mp[k][rb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ml_off(rb), 0, kSC1));
              lp[k][rb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ml_off(rb) + 4 * 64 * 4, 0, kSC1));
            }
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            float M = mp[0][rb];
#pragma unroll
            for (int k = 1; k < NP; ++k) M = fmaxf(M, mp[k][rb]);
            float lsum = 0.f;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
              f[k][rb] = mp[k][rb] == kNegInf ? 0.f : fast_exp2(mp[k][rb] - M);
              lsum = k == 0 ? lp[0][rb] * f[0][rb] : __builtin_fmaf(lp[k][rb], f[k][rb], lsum);
            }
            const float lt = lsum + __shfl_xor(lsum, 32);
            inv[rb] = lt > 0.f ? a.vscale / lt : 0.f;
          }
        }
        constexpr int NG = RB * DBW * 2;
        f32x4 chunk[2][NP][2];
        auto load_group = [&](int g, int sl) {
          const int rb = g / (2 * DBW), db = (g / 2) % DBW, q0 = 2 * (g % 2);
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            const auto rs = slot_rsrc(pcs[k]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
              chunk[sl][k][j] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, acc_off + ((rb * DBW + db) * 4 + q0 + j) * 1024, 0, kSC1));
          }
        };
        load_group(0, 0);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g + 1 < NG) load_group(g + 1, (g + 1) & 1);
          const int rb = g / (2 * DBW), db = (g / 2) % DBW, q0 = 2 * (g % 2);
          float* orow = out_row(rb);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int qd = q0 + j;
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float t = 0.f;
#pragma unroll
              for (int k = 0; k < NP; ++k) {
                const float v = chunk[g & 1][k][j][e];
                t = k == 0 ? v * f[0][rb] : __builtin_fmaf(v, f[k][rb], t);
              }
              o[e] = t * inv[rb];
            }
            if (orow) *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * qd + 4 * h) = o;
          }
        }
      };
      if (npieces == 2) {
        merge_np(std::integral_constant<int, 2>{});
      } else if (npieces == 3) {
        merge_np(std::integral_constant<int, 3>{});
      } else if (npieces == 4) {
        merge_np(std::integral_constant<int, 4>{});
      } else {
        float M[RB], lsum[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) M[rb] = kNegInf, lsum[rb] = 0.f;
        for (int pc = p0; pc < a.kpieces; ++pc)
          if (is_piece(pc)) {
            const auto rs = slot_rsrc(pc);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              M[rb] = fmaxf(M[rb], __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ml_off(rb), 0, kSC1)));
          }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < DBW; ++db) acc[rb][db] = f32x16{};
        for (int pc = p0; pc < a.kpieces; ++pc) {
          if (!is_piece(pc)) continue;
          const auto rs = slot_rsrc(pc);
          float f[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ml_off(rb), 0, kSC1));
            const float lp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ml_off(rb) + 4 * 64 * 4, 0, kSC1));
            f[rb] = mp == kNegInf ? 0.f : fast_exp2(mp - M[rb]);
            lsum[rb] = __builtin_fmaf(lp, f[rb], lsum[rb]);
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int db = 0; db < DBW; ++db)
#pragma unroll
              for (int qd = 0; qd < 4; ++qd) {
                const f32x4 v = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, acc_off + ((rb * DBW + db) * 4 + qd) * 1024, 0, kSC1));
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[rb][db][4 * qd + e] = __builtin_fmaf(v[e], f[rb], acc[rb][db][4 * qd + e]);
              }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float lt = lsum[rb] + __shfl_xor(lsum[rb], 32);
          const float inv = lt > 0.f ? a.vscale / lt : 0.f;
          float* orow = out_row(rb);
          if (orow) {
#pragma unroll
            for (int db = 0; db < DBW; ++db)
#pragma unroll
              for (int qd = 0; qd < 4; ++qd) {
                f32x4 o = {acc[rb][db][4 * qd] * inv, acc[rb][db][4 * qd + 1] * inv, acc[rb][db][4 * qd + 2] * inv,
                           acc[rb][db][4 * qd + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * qd + 4 * h) = o;
              }
          }
        }
      }
      return;
    }

    // Whole tile here: the row blocks' denominators meet in LDS (the key
    // buffers are idle once the last PV has started).
    float* sl = reinterpret_cast<float*>(&sk[0][0]);
    if constexpr (R64) {
      float lt = l_i + __shfl_xor(l_i, 16);
      lt += __shfl_xor(lt, 32);
      if (grp == 0) sl[wave * 16 + j16] = lt;
    } else {
      sl[wave * 64 + lane] = l_i + __shfl_xor(l_i, 32);
    }
    lds_barrier();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lt = R64 ? sl[32 * rb + n] : sl[rb * 64 + lane];
      const float inv = lt > 0.f ? a.vscale / lt : 0.f;
      float* orow = out_row(rb);
      if (orow) {
#pragma unroll
        for (int db = 0; db < DBW; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 o = {acc[rb][db][4 * i] * inv, acc[rb][db][4 * i + 1] * inv, acc[rb][db][4 * i + 2] * inv,
                       acc[rb][db][4 * i + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i + 4 * h) = o;
          }
      }
    }
  };

  if (u0 < u1) {
    if (u0 < nL) process(tl, 0, jlo_l + u0, jlo_l + min(u1, nL) - 1, jlo_l, jhi_l, 0, nL);
    if (u1 > nL) {
      if (u0 < nL) lds_barrier();  // the first segment's buffers may still be in use
      process(ts, 1, jlo_s + max(u0, nL) - nL, jlo_s + u1 - nL - 1, jlo_s, jhi_s, nL, U);
    }
  }
}

// ---------------------------------------------------------------- decode --

struct DecodeArgs {
  const uint16_t* q;  // [B, T, Hq, D]
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  float* part_o;    // [slots][cols][D]: slot = stream + piece (see k_decode)
  float* part_lse;  // [slots][cols], log2 units
  int B, Hq, Hkv, g, Lmax, W;
  int T;            // query tokens per sequence, at positions kv_len - T .. kv_len - 1
  int ncg;          // column groups per (batch, kv head): the T*g queries in groups of 16
  int cols;         // query columns per partial slot (T*g if one group, else 16)
  int npieces;      // work-groups of the split (pieces of the total key work)
  int ring;         // 0: cache row j holds position j; C > 0: row j % C (a window-sized ring, Lmax = C)
  const uint16_t* knew;  // null, or [B, T, Hkv, D]: keys of the T tokens, read in place of their cache rows
  const uint16_t* vnew;  // their values (== knew when aliased)
  uint16_t* kc;          // the cache, written by k_decode_combine when appending
  uint16_t* vc;
  float qscale;          // softmax scale * log2(e) (times the key scale of an E4M3 cache)
  float vscale;          // the value scale of an E4M3 cache (1 otherwise): multiplies the output
  float kstore, vstore;  // E4M3 append: the scales new keys / values are divided by
  RopeRev rope;
};

// Rotate 8 (x, y) pairs held as packed bf16 quads by per-pair (cos, sin)
// constants cs[2e], cs[2e+1] for e = 0..7 (pair e = element e of x and y).
__device__ __forceinline__ void rot8_const(u32x4& x, u32x4& y, const float* cs) {
  u32x4 xo, yo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float c0 = cs[4 * e], s0 = cs[4 * e + 1], c1 = cs[4 * e + 2], s1 = cs[4 * e + 3];
    const float a0 = bf_lo(x[e]), a1 = bf_hi(x[e]);
    const float b0 = bf_lo(y[e]), b1 = bf_hi(y[e]);
    xo[e] = pack_bf16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
    yo[e] = pack_bf16(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
  }
  x = xo;
  y = yo;
}

__device__ __forceinline__ void lds_read_b128x2(u32x4 (&r)[2], const unsigned (&ad)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(ad[0]), "v"(ad[1]));
}

__device__ __forceinline__ void lds_read_b64x2(u32x2 (&r)[2], const unsigned (&ad)[2]) {
  asm volatile(
      "ds_read_b64 %0, %2\n\t"
      "ds_read_b64 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(ad[0]), "v"(ad[1]));
}

__device__ __forceinline__ void lds_read_tr_x4(u32x2 (&r)[4], const unsigned (&ad)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
}

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c, 0,
                                                   0, 0);
}

// The same rotation for 8 (x, y) pairs held as E4M3 bytes: each byte pair
// goes straight to fp32 (exact) and the rotated pair to packed bf16, the
// values rot8_const gives on the bf16 form of the same bytes.
__device__ __forceinline__ void rot8_const_e4m3(u32x2 x8, u32x2 y8, const float* cs, u32x4& xo, u32x4& yo) {
  f32x2 a[4], b[4];  // element pairs 2e, 2e + 1: bytes of word e / 2, its low or high half
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    a[2 * w] = __builtin_amdgcn_cvt_pk_f32_fp8((int)x8[w], false);
    a[2 * w + 1] = __builtin_amdgcn_cvt_pk_f32_fp8((int)x8[w], true);
    b[2 * w] = __builtin_amdgcn_cvt_pk_f32_fp8((int)y8[w], false);
    b[2 * w + 1] = __builtin_amdgcn_cvt_pk_f32_fp8((int)y8[w], true);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float c0 = cs[4 * e], s0 = cs[4 * e + 1], c1 = cs[4 * e + 2], s1 = cs[4 * e + 3];
    xo[e] = pack_bf16(a[e][0] * c0 - b[e][0] * s0, a[e][1] * c1 - b[e][1] * s1);
    yo[e] = pack_bf16(b[e][0] * c0 + a[e][0] * s0, b[e][1] * c1 + a[e][1] * s1);
  }
}

// max over the four 16-lane groups that share a query column
__device__ __forceinline__ float max_over_groups(float x) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Sequence length of batch entry b, clamped to [T, Lmax] for a cache of one
// row per position (a ring maps any position into its rows), so that no
// access goes out of bounds whatever kv_len holds.
__device__ __forceinline__ int decode_len(const DecodeArgs& a, int b) {
  const int L = max(a.kv_len[b], a.T);
  return a.ring > 0 ? L : min(L, a.Lmax);
}
// Cache row of key position j.
__device__ __forceinline__ int decode_row(const DecodeArgs& a, int j) { return a.ring > 0 ? j % a.ring : j; }
// First key any of the T queries of a length-L sequence sees.
__device__ __forceinline__ int decode_lo(const DecodeArgs& a, int L) {
  return a.W > 0 ? max(0, L - a.T + 1 - a.W) : 0;
}
// Visible key count of batch entry b's streams (all its kv heads and column groups).
__device__ __forceinline__ long long decode_batch_keys(const DecodeArgs& a, int b) {
  const int L = decode_len(a, b);
  return (long long)a.Hkv * a.ncg * (L - decode_lo(a, L));
}

// Sum over the work-group (256 threads) of one value per thread.
__device__ __forceinline__ long long block_sum_ll(long long x, long long* red4) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = x;
  __syncthreads();
  const long long t = red4[0] + red4[1] + red4[2] + red4[3];
  __syncthreads();  // red4 is read before anybody reuses it
  return t;
}

// The split of the decode work: T visible keys over all streams, np pieces
// (at most a.npieces, at least 64 keys each); for work-group blockIdx.x <
// np, the batch entry whose streams hold its first key and where they start.
__device__ void decode_split(const DecodeArgs& a, long long& T, int& np, int& b_lo, long long& base_lo) {
  __shared__ long long s_red[4];
  __shared__ long long s_carry, s_base;
  __shared__ int s_blo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long t = 0;
  for (int b = tid; b < a.B; b += 256) t += decode_batch_keys(a, b);
  T = block_sum_ll(t, s_red);
  np = (int)min((long long)a.npieces, max(1LL, T / 64));
  b_lo = 0;
  base_lo = 0;
  if ((int)blockIdx.x >= np) return;  // (the whole work-group)
  const long long r0 = (long long)blockIdx.x * T / np;
  if (tid == 0) {
    s_carry = 0;
    s_blo = 0;  // (exactly one batch entry's range holds r0 and overwrites these)
    s_base = 0;
  }
  __syncthreads();
  for (int b0 = 0; b0 < a.B; b0 += 256) {
    const int b = b0 + tid;
    const long long sz = b < a.B ? decode_batch_keys(a, b) : 0;
    long long x = sz;  // inclusive scan over the work-group
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_red[wave] = x;
    __syncthreads();
    long long pre = s_carry;
    for (int w = 0; w < wave; ++w) pre += s_red[w];
    const long long incl = pre + x, excl = incl - sz;
    if (b < a.B && excl <= r0 && r0 < incl) {
      s_blo = b;
      s_base = excl;
    }
    __syncthreads();
    if (tid == 255) s_carry = incl;
    __syncthreads();
  }
  b_lo = s_blo;
  base_lo = s_base;
}

// Split-K decode.  Scores need <R_P q, R_j k> (P = kv_len - 1, j = key
// position); RoPE rotations are orthogonal and commute, so this equals
// <R_{P - j0} q, R_{j - j0} k> for any j0.  With j0 = the first key of the
// current 16-key step, every lane's key offset j - j0 (its MFMA row) and its
// rotation pairs are fixed for the whole work-group: their (cos, sin) are
// computed once, and the query is advanced by R_{-16} once per step (fp32
// recurrence).  The four waves split the rotation pairs for S^T = K' Q'^T
// (partial sums exchanged through LDS) and the head dim for O^T += V^T P^T.
// Key/value rows stream through NSTAGE LDS stages of 16 rows each.
// GEN = false is the one-token path over a cache of one row per position
// with nothing appended (T = 1, ring = 0, knew = null): the per-column
// positions, masks, ring rows and appended rows compile away.  RA = false
// (with GEN) is T > 1 tokens over such a cache: only the ring rows and
// appended rows compile away, whose per-load row arithmetic costs a
// verify step over a frozen cache about 5 % of its time.  FP8: the
// cache holds E4M3 bytes; a lane converts its key elements in registers
// before rotating them, and each stage's values are converted once into a
// bf16 tile laid out like a bf16 stage, which the value reads then use (the
// key scale is in qscale, the value scale in the output).
template <int D, bool ALIAS, int NSTAGE, bool GEN, bool FP8, bool RA>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void k_decode(DecodeArgs a) {
  static_assert(GEN || !RA, "ring rows and appended rows belong to the general path");
  constexpr int KPS = 16;            // keys per step
  constexpr int FQ = D / 8;          // rotation pairs per wave
  constexpr int KH = FQ / 32;        // groups of 8 pairs per lane (x and y halves each)
  constexpr int KSTEPS = 2 * KH;     // 16x16x32 steps per key block
  constexpr int DQ = D / 4;          // output head-dim slice per wave
  constexpr int DBLK = DQ / 16;
  constexpr int NT = ALIAS ? 1 : 2;  // tensors staged per step
  constexpr int EB = FP8 ? 1 : 2;    // bytes per cache element
  constexpr int ROWB = D * EB;       // bytes per staged cache row
  constexpr int VROWB = D * 2;       // bytes per bf16 value row read by the output MFMAs
  constexpr int LPS1 = KPS * ROWB / 4096;
  constexpr int LPS = NT * LPS1;
  static_assert(LPS1 >= 1 && LPS1 * 4096 == KPS * ROWB, "stage must split over 256 threads");

  __shared__ __attribute__((aligned(16))) unsigned char sbuf[NSTAGE][NT][KPS * ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char vconv[FP8 ? KPS * VROWB : 16];
  __shared__ f32x4 red[4][64];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // The visible keys of all (batch, kv-head) streams, laid end to end
  // (batch-major, kv heads of a batch entry adjacent, each stream its window
  // [lo_b, L_b)), are cut into np equal pieces, one per work-group; a
  // piece's part of each stream it overlaps is one segment, whose partial
  // goes to slot (stream + piece) -- unique, as streams and pieces are both
  // ordered.  k_decode_combine finds the same pieces from kv_len.
  long long T;
  int np, b_lo;
  long long base_lo;
  decode_split(a, T, np, b_lo, base_lo);
  const int piece = blockIdx.x;
  if (piece >= np) return;
  const long long r0 = (long long)piece * T / np, r1 = (long long)(piece + 1) * T / np;

  auto segment = [&](int b, int kvh, int cg, int k_start, int k_end, int slot) __attribute__((always_inline)) {
  const int L = decode_len(a, b);
  // MFMA column n is query column c = 16 cg + n of this (batch, kv head):
  // token t = c / g at position L - T + t, head kvh * g + c % g.
  const int c = cg * 16 + n;
  const bool qvalid = GEN ? (n < a.cols && c < a.T * a.g) : n < a.g;
  const int ct = GEN && qvalid ? c / a.g : 0, hh = qvalid ? (GEN ? c % a.g : n) : 0;
  const int head = kvh * a.g + hh;
  const int P = GEN ? L - a.T + ct : L - 1;  // this column's query position
  const size_t part = (size_t)slot * a.cols + (qvalid ? n : 0);
  const size_t slice = ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * D;
  // Keys of the T current tokens come from the appended rows when the call
  // writes them (k_decode_combine stores them into the cache afterwards).
  const int new0 = RA && !FP8 && a.knew != nullptr ? L - a.T : 0x7fffffff;
  // Cache row of key position pos of this segment: row0 + (pos - k_start),
  // wrapped once for a ring (a segment spans at most the ring's length).
  const int wrap = RA && a.ring > 0 ? a.ring : 0x7fffffff;
  const int row0 = RA && a.ring > 0 ? k_start % a.ring : k_start;
  auto issue = [&](int step, int stg) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int k0 = k_start + step * KPS;
#pragma unroll
    for (int tsr = 0; tsr < NT; ++tsr) {
      const char* base = reinterpret_cast<const char*>(tsr == 0 ? a.k : a.v) + slice * EB;
      const char* nbase =
          reinterpret_cast<const char*>((tsr == 0 ? a.knew : a.vnew) + ((size_t)b * a.T * a.Hkv + kvh) * D);
#pragma unroll
      for (int i = 0; i < LPS1; ++i) {
        const int blk = i * 4 + wave;
        const int byte = blk * 1024 + ln * 16;
        const int row = byte / ROWB, slot = (byte % ROWB) >> 4;
        const int pos = min(k0 + row, k_end - 1);  // key position
        const char* src;
        if constexpr (RA) {
          int crow = row0 + (pos - k_start);
          crow = crow >= wrap ? crow - wrap : crow;
          // (appended rows are bf16 and read here only for a bf16 cache; an
          // E4M3 cache has them quantised and stored before this kernel)
          src = pos >= new0 ? nbase + (size_t)(pos - new0) * a.Hkv * D * 2 : base + (size_t)crow * ROWB;
        } else {
          src = base + (size_t)pos * ROWB;
        }
        g2l16_nt(src + ((slot ^ swz(row)) << 4), reinterpret_cast<char*>(sbuf[stg][tsr]) + blk * 1024);
      }
    }
  };

  // Start streaming before the per-lane set-up below.
  const int nsteps = (k_end - k_start + KPS - 1) / KPS;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nsteps) issue(s, s);

  // This lane's rotation pairs: f = wave*FQ + 32*kk + 8*G + t (kk < KH, t < 8).
  // Key side: (cos, sin)(n * w_f) for its key offset n < 16 (fp32 is exact
  // enough for angles below 16 rad).
  float kcs[KH][16];
#pragma unroll
  for (int kk = 0; kk < KH; ++kk)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int f = wave * FQ + 32 * kk + 8 * G + t;
      float x = (float)n * (float)a.rope.rev[f];
      x -= __builtin_rintf(x);
      kcs[kk][2 * t] = __builtin_amdgcn_cosf(x);
      kcs[kk][2 * t + 1] = __builtin_amdgcn_sinf(x);
    }
  // Query side: u = RoPE(q, P - k_start) * scale * log2(e) in fp32 (fp64
  // angle), and the per-step rotation R_{-16}.  The recurrence u <- R_{-16} u
  // is re-anchored from the fp64 angle every kReanchorSteps steps, so its
  // fp32 drift (angle and length) is bounded whatever the segment length.
  float ux[KH][8], uy[KH][8], stc[KH][8], sts[KH][8];
  const uint16_t* qrow = a.q + (((size_t)b * a.T + ct) * a.Hq + head) * D;
#pragma unroll
  for (int kk = 0; kk < KH; ++kk) {
    const int d0 = wave * FQ + 32 * kk + 8 * G;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float st = (float)KPS * (float)a.rope.rev[d0 + t];
      st -= __builtin_rintf(st);
      stc[kk][t] = __builtin_amdgcn_cosf(st);
      sts[kk][t] = -__builtin_amdgcn_sinf(st);  // rotation by -KPS positions
    }
  }
  // (the raw query pairs are re-read at each anchor -- from L2, once per
  // kReanchorSteps steps -- rather than held in registers)
  auto anchor = [&](double rel) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const int d0 = wave * FQ + 32 * kk + 8 * G;
      const u32x4 qx = *reinterpret_cast<const u32x4*>(qrow + d0);
      const u32x4 qy = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float sn, cn;
        sincos_rev(rel, a.rope.rev[d0 + t], sn, cn);
        const float xa = (t & 1) ? bf_hi(qx[t >> 1]) : bf_lo(qx[t >> 1]);
        const float ya = (t & 1) ? bf_hi(qy[t >> 1]) : bf_lo(qy[t >> 1]);
        ux[kk][t] = qvalid ? (xa * cn - ya * sn) * a.qscale : 0.f;
        uy[kk][t] = qvalid ? (ya * cn + xa * sn) * a.qscale : 0.f;
      }
    }
  };
  anchor((double)(P - k_start));

  f32x4 acc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) acc[i] = f32x4{};
  float m_i = kNegInf, l_i = 0.f;

  for (int s = 0; s < nsteps; ++s) {
    const int stg = s % NSTAGE;
    if (s > 0 && s % kReanchorSteps == 0) anchor((double)(P - k_start - s * KPS));
    // Q' for this step (bf16), then advance u by R_{-16} for the next one.
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      u32x4 x, y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = pack_bf16(ux[kk][2 * e], ux[kk][2 * e + 1]);
        y[e] = pack_bf16(uy[kk][2 * e], uy[kk][2 * e + 1]);
      }
      qf[kk] = as_bf16x8(x);
      qf[kk + KH] = as_bf16x8(y);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xa = ux[kk][t], ya = uy[kk][t];
        ux[kk][t] = xa * stc[kk][t] - ya * sts[kk][t];
        uy[kk][t] = ya * stc[kk][t] + xa * sts[kk][t];
      }
    }

    if (nsteps - s - 1 >= NSTAGE - 2)
      wait_vm<(NSTAGE - 2) * LPS>();
    else
      wait_vm<0>();
    lds_barrier();
    if (s + NSTAGE - 1 < nsteps) issue(s + NSTAGE - 1, (s + NSTAGE - 1) % NSTAGE);
    if constexpr (FP8) {
      // This stage's values (the keys of an aliased layer) as bf16 rows in
      // the bf16 stage layout: E4M3 chunk cf (16 elements) of row r sits at
      // 16-byte slot cf ^ swz(r); its halves are bf16 chunks 2 cf and
      // 2 cf + 1, stored at slots (2 cf) ^ swz(r) and (2 cf + 1) ^ swz(r).
      // Written before, and read after, the score-exchange barrier below.
      const unsigned char* vs8 = sbuf[stg][NT - 1];
#pragma unroll
      for (int i = 0; i < D / 256; ++i) {
        const int ci = tid + 256 * i, r = ci / (D / 16), cf = ci % (D / 16);
        const u32x4 w = *reinterpret_cast<const u32x4*>(vs8 + r * ROWB + ((cf ^ swz(r)) << 4));
        unsigned char* vrow = vconv + r * VROWB;
        *reinterpret_cast<u32x4*>(vrow + (((2 * cf) ^ swz(r)) << 4)) = fp8x8_to_bf16(u32x2{w[0], w[1]});
        *reinterpret_cast<u32x4*>(vrow + (((2 * cf + 1) ^ swz(r)) << 4)) = fp8x8_to_bf16(u32x2{w[2], w[3]});
      }
    }

    int ln = lane;  // opaque lane index: per-lane LDS offsets are recomputed each step
    asm volatile("" : "+v"(ln));
    const int on = ln & 15, oG = ln >> 4;
    const int k0 = k_start + s * KPS;
    const char* kb = reinterpret_cast<const char*>(sbuf[stg][0]);
    // Partial S^T over this wave's rotation pairs; lane (n, G) supplies key
    // row n, rotated by its offset n within the step.
    f32x4 sp = f32x4{};
    const unsigned kra = lds_addr(kb + on * ROWB);
    const int ksw = swz(on);
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const int d = wave * FQ + 32 * kk + 8 * oG;
      u32x4 fr[2];
      if constexpr (FP8) {
        // 8 E4M3 bytes at element d (16-byte chunk d / 16, half (d / 8) & 1)
        const unsigned ad[2] = {kra + (((d >> 4) ^ ksw) << 4) + (d & 8),
                                kra + ((((d + D / 2) >> 4) ^ ksw) << 4) + ((d + D / 2) & 8)};
        u32x2 f8[2];
        lds_read_b64x2(f8, ad);
        rot8_const_e4m3(f8[0], f8[1], kcs[kk], fr[0], fr[1]);
      } else {
        const unsigned ad[2] = {kra + (((d >> 3) ^ ksw) << 4), kra + ((((d + D / 2) >> 3) ^ ksw) << 4)};
        lds_read_b128x2(fr, ad);
        rot8_const(fr[0], fr[1], kcs[kk]);
      }
      sp = mfma16(as_bf16x8(fr[0]), qf[kk], sp);
      sp = mfma16(as_bf16x8(fr[1]), qf[kk + KH], sp);
    }
    lds_write_f32x4(lds_addr(&red[wave][ln]), sp);
    lds_barrier();
    f32x4 sc;
    {
      u32x4 t[4];
      const unsigned ad[4] = {lds_addr(&red[0][ln]), lds_addr(&red[1][ln]), lds_addr(&red[2][ln]),
                              lds_addr(&red[3][ln])};
      lds_read_b128x4(t, ad);
      sc = __builtin_bit_cast(f32x4, t[0]) + __builtin_bit_cast(f32x4, t[1]) + __builtin_bit_cast(f32x4, t[2]) +
           __builtin_bit_cast(f32x4, t[3]);
    }

    // keys k0 + 4*G + jj for query column n: visible up to its own position
    // and, for a window, back to P - W + 1 (the segment lies inside the
    // union of the T queries' key ranges)
    float mx = kNegInf;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int key = k0 + 4 * G + jj;
      const bool vis = GEN ? key < k_end && key <= P && (a.W == 0 || P - key < a.W) : key < k_end;
      sc[jj] = vis ? sc[jj] : kNegInf;
      mx = fmaxf(mx, sc[jj]);
    }
    mx = max_over_groups(mx);
    const bool grow = mx > m_i + kRescaleSlack;
    const float alpha = (grow & (m_i != kNegInf)) ? fast_exp2(m_i - mx) : 1.f;
    m_i = grow ? mx : m_i;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
      l_i *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) acc[i] *= alpha;
    }
    const float m_use = (m_i == kNegInf) ? 0.f : m_i;
    float p[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p[jj] = fast_exp2(sc[jj] - m_use);
      l_i += p[jj];
    }
    const u32x2 pf = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};

    // O^T += V^T P^T with 16x16x16 MFMAs: P^T slot t of lane group G is key
    // 4*G + t, which one transpose read per output block fetches.
    const char* vb = FP8 ? reinterpret_cast<const char*>(vconv) : reinterpret_cast<const char*>(sbuf[stg][NT - 1]);
    const int vrow = 4 * oG + (on >> 2);
    const unsigned va = lds_addr(vb + vrow * VROWB);
    const int vsw = swz(vrow);
#pragma unroll
    for (int b0 = 0; b0 < DBLK; b0 += 4) {
      unsigned ad[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dcol = wave * DQ + 16 * (b0 + u) + 4 * (on & 3);
        ad[u] = va + (((dcol >> 3) ^ vsw) << 4) + ((dcol & 7) << 1);
      }
      u32x2 t[4];
      lds_read_tr_x4(t, ad);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[b0 + u] = mfma16k16(t[u], pf, acc[b0 + u]);
    }
  }

  // (a column can see no key of a segment: with T > 1 the keys after its
  // position, or before its window; its partial is then 0 with weight 0)
  const float l = sum_over_groups(l_i);
  const float inv = l > 0.f ? a.vscale / l : 0.f;
  if (qvalid) {
    float* o = a.part_o + part * D + wave * DQ + 4 * G;
#pragma unroll
    for (int bi = 0; bi < DBLK; ++bi) *reinterpret_cast<f32x4*>(o + 16 * bi) = acc[bi] * inv;
    if (wave == 0 && G == 0) a.part_lse[part] = l > 0.f ? m_i + __builtin_amdgcn_logf(l) : kNegInf;
  }
  lds_barrier();  // the stages are refilled by the next segment
  };

  // Segments of this piece: streams (batch, kv head, column group) from the
  // one holding key r0 on.
  long long base = base_lo;
  for (int b = b_lo; b < a.B && base < r1; ++b) {
    const int L = decode_len(a, b);
    const int lo = decode_lo(a, L);
    const int span = L - lo;
    for (int st = 0; st < a.Hkv * a.ncg; ++st) {
      const long long s0 = base + (long long)st * span, s1 = s0 + span;
      const long long x0 = max(s0, r0), x1 = min(s1, r1);
      if (x0 < x1)
        segment(b, st / a.ncg, st % a.ncg, lo + (int)(x0 - s0), lo + (int)(x1 - s0),
                (b * a.Hkv) * a.ncg + st + piece);
    }
    base += (long long)a.Hkv * a.ncg * span;
  }
}

// Append to an E4M3 cache: the T tokens' keys (and values) of one (batch,
// token, kv head) per work-group, stored as E4M3 codes of x / scale (the
// quotient in fp32, rounded to nearest with ties to even by the hardware
// conversion, clamped to +-448 first so that it saturates) into their rows.
// Runs before the split-K kernel, which then reads them from the cache.
template <int D>
__global__ __launch_bounds__(64) void k_append_fp8(DecodeArgs a) {
  const int kvh = blockIdx.x % a.Hkv, bt = blockIdx.x / a.Hkv, tok = bt % a.T, b = bt / a.T;
  const int P = decode_len(a, b) - a.T + tok;
  const size_t dst = ((size_t)(b * a.Hkv + kvh) * a.Lmax + decode_row(a, P)) * D;  // E4M3 bytes
  const size_t src = (((size_t)b * a.T + tok) * a.Hkv + kvh) * D;                   // bf16 elements
  auto quant8 = [](const uint16_t* x, float scale) -> u32x2 {
    const u32x4 w = *reinterpret_cast<const u32x4*>(x);
    u32x2 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned wv = w[2 * i + e / 2];
        const float f = (e & 1) ? bf_hi(wv) : bf_lo(wv);
        q[e] = fminf(fmaxf(f / scale, -448.f), 448.f);
      }
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], pk, true);
      r[i] = (unsigned)pk;
    }
    return r;
  };
  for (int i = threadIdx.x; i < D / 8; i += 64) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(a.kc) + dst + 8 * i) = quant8(a.knew + src + 8 * i,
                                                                                             a.kstore);
    if (a.vnew != a.knew)
      *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(a.vc) + dst + 8 * i) =
          quant8(a.vnew + src + 8 * i, a.vstore);
  }
}

// Log-sum-exp merge of the segment partials of one (batch, head) and one
// slice of NQ head-dim quads (blockIdx.y; NQ = D/4: the whole head).  The
// pieces overlapping the head's stream follow from kv_len exactly as
// k_decode cut them; their partials sit in slots stream + piece.  256
// threads: thread t owns quad t % NQ and every (256/NQ)-th partial from
// t / NQ on; its first four partials load together with the log-sum-exps,
// the rest four at a time, and the groups are summed through LDS in a
// fixed order.  Wide slices suit streams of few pieces (one work-group per
// head, one memory round trip), narrow ones streams of many (more
// partials in flight).
template <int D, int NQ>
__global__ __launch_bounds__(256) void k_decode_combine(DecodeArgs a, float* __restrict__ out) {
  constexpr int NGRP = 256 / NQ;    // partial groups
  constexpr int U = 4;              // partials per thread loaded before the maximum is known
  static_assert(NGRP * NQ == 256, "one thread per (partial group, quad)");
  __shared__ f32x4 snum[NGRP][NQ];
  __shared__ float sden[NGRP][NQ];
  __shared__ float smax[4];
  __shared__ long long s_red[4];
  const int bh = blockIdx.x;  // (batch, token, head)
  const int head = bh % a.Hq, bt = bh / a.Hq, tok = bt % a.T, b = bt / a.T;
  const int kvh = head / a.g;
  const int c = tok * a.g + head % a.g;        // query column of this (batch, kv head)
  const int cg = c / 16, n = c - 16 * cg;      // its column group and slot column (one group: cg 0, n = c)
  const int qd = threadIdx.x % NQ, grp = threadIdx.x / NQ;
  if (a.knew != nullptr && head % a.g == 0 && blockIdx.y == 0) {
    // Append: the first head of each kv head stores its token's key (and
    // value) row into the cache; k_decode, which read them from the new rows,
    // has finished (same stream), so no reader sees a half-written row.
    const int P = decode_len(a, b) - a.T + tok;
    const size_t dst = ((size_t)(b * a.Hkv + kvh) * a.Lmax + decode_row(a, P)) * D;
    const size_t src = (((size_t)b * a.T + tok) * a.Hkv + kvh) * D;
    for (int i = threadIdx.x; i < D / 8; i += 256) {
      reinterpret_cast<u32x4*>(a.kc + dst)[i] = reinterpret_cast<const u32x4*>(a.knew + src)[i];
      if (a.vnew != a.knew) reinterpret_cast<u32x4*>(a.vc + dst)[i] = reinterpret_cast<const u32x4*>(a.vnew + src)[i];
    }
  }
  // total keys, and the keys of the streams before this batch entry's
  long long t = 0, tb = 0;
  for (int bb = threadIdx.x; bb < a.B; bb += 256) {
    const long long k = decode_batch_keys(a, bb);
    t += k;
    tb += bb < b ? k : 0;
  }
  const long long T = block_sum_ll(t, s_red);
  const long long base_b = block_sum_ll(tb, s_red);
  const int np = (int)min((long long)a.npieces, max(1LL, T / 64));
  const long long span = decode_batch_keys(a, b) / (a.Hkv * a.ncg);
  const int stream = (b * a.Hkv + kvh) * a.ncg + cg;
  const long long x0 = base_b + (long long)(kvh * a.ncg + cg) * span, x1 = x0 + span;  // this stream's keys
  const int p0 = (int)(((x0 + 1) * np - 1) / T), p1 = (int)((x1 * np - 1) / T);  // pieces holding x0, x1 - 1
  const int npart = p1 - p0 + 1;
  const size_t first = (size_t)(stream + p0) * a.cols + n;  // partial k at first + k * cols
  auto pidx = [&](int k) { return first + (size_t)k * a.cols; };
  const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o) + blockIdx.y * NQ + qd;
  // This thread's first U partials (grp, grp + NGRP, ...) are loaded before
  // the largest log-sum-exp is known, so both take one memory round trip.
  f32x4 o[U];
  float e[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = grp + u * NGRP;
    const bool in = k < npart;
    e[u] = in ? a.part_lse[pidx(k)] : kNegInf;
    o[u] = in ? po[pidx(k) * (D / 4)] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float M = kNegInf;
  for (int k = threadIdx.x; k < npart; k += 256) M = fmaxf(M, a.part_lse[pidx(k)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float w = e[u] == kNegInf ? 0.f : fast_exp2(e[u] - M);
    num += w * o[u];
    den += w;
  }
  int k = grp + U * NGRP;  // streams cut into more pieces: four loads in flight per round trip
  for (; k + (U - 1) * NGRP < npart; k += U * NGRP) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      e[u] = a.part_lse[pidx(k + u * NGRP)];
      o[u] = po[pidx(k + u * NGRP) * (D / 4)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = fast_exp2(e[u] - M);
      num += w * o[u];
      den += w;
    }
  }
  for (; k < npart; k += NGRP) {
    const float w = fast_exp2(a.part_lse[pidx(k)] - M);
    num += w * po[pidx(k) * (D / 4)];
    den += w;
  }
  // (partials of segments the query sees no key of have log-sum-exp -inf:
  // weight 0, value 0)
  snum[grp][qd] = num;
  sden[grp][qd] = den;
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int g2 = 1; g2 < NGRP; ++g2) {
      num += snum[g2][qd];
      den += sden[g2][qd];
    }
    reinterpret_cast<f32x4*>(out + (size_t)bh * D)[blockIdx.y * NQ + qd] = num * (1.f / den);
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

// FastDiv constants of divisor d >= 1 (see fdiv).
static FastDiv make_fastdiv(int d) {
  unsigned L = 0;
  while ((1ull << L) < (unsigned long long)d) ++L;
  const unsigned s = 31 + L;
  const unsigned long long m = ((1ull << s) + (unsigned long long)d - 1) / (unsigned long long)d;
  return FastDiv{(unsigned)m, s};
}

// Key tiles a query tile visits (same rule as the kernel; P0 = position of query 0).
static void prefill_tile_keys(int qt, int S, int g, int W, int BN, int rows, int P0, int& jlo, int& jhi) {
  const int rows_total = S * g, r0 = qt * rows;
  const int pmin = P0 + r0 / g, pmax = P0 + std::min(r0 + rows - 1, rows_total - 1) / g;
  jlo = (W > 0 ? std::max(0, pmin - W + 1) : 0) / BN;
  jhi = pmax / BN;
}

// Work split.  A work unit is either a pair of query tiles (t, nqt-1-t),
// which evens out causal tiles, or a single query tile, which suits
// windowed layers whose tiles all visit about the same number of key tiles;
// each unit's key work is cut into kpieces ranges, one per work-group.
// Head size 256 may also run 64-row query tiles (twice the work-groups, no
// pieces), which fills the GPU when 128-row tiles are too few.
// The choice minimises an estimate of the slowest work-group's time: key
// tiles times the per-tile cost, plus a fixed cost per query-tile segment
// (query load and rotation, first tile copy, output) and, when a tile is
// split, the partial-result store and merge; the constants are per-kernel
// cycle counts measured on MI355X.
constexpr int kSplitPvMinTiles = 32;
struct PrefillCosts {
  double tile, segment, split;
};
static PrefillCosts prefill_costs(int D, int rows) {
  if (D == 512) return {4700.0, 12000.0, 40000.0};
  if (rows == 64) return {1400.0, 12000.0, 0.0};
  return {2400.0, 15000.0, 30000.0};
}

// G4_PREFILL_ROWS=128 or 64 pins the query-tile height of head size 256
// (tests use it to reach both kernels at small sizes); unset = cost model.
static int prefill_rows_override() {
  const char* e = std::getenv("G4_PREFILL_ROWS");
  if (!e) return 0;
  const int v = std::atoi(e);
  return (v == 64 || v == 128) ? v : 0;
}

// G4_PREFILL_SPLIT_PV=0 or 1 pins the head-size-512 schedule (tests use it
// to reach both at small sizes); unset = by key tiles per work-group.
static int prefill_split_pv_override() {
  const char* e = std::getenv("G4_PREFILL_SPLIT_PV");
  if (!e) return -1;
  const int v = std::atoi(e);
  return (v == 0 || v == 1) ? v : -1;
}

// G4_PREFILL_PRODUCER=0 or 1 turns the producer waves of the 64-row
// head-size-256 kernel off or on (tests reach both; unset = on).
static int prefill_producer_override() {
  const char* e = std::getenv("G4_PREFILL_PRODUCER");
  if (!e) return -1;
  const int v = std::atoi(e);
  return (v == 0 || v == 1) ? v : -1;
}

// G4_PREFILL_KPIECES=k pins the number of pieces a work unit's key range is
// cut into (tests and tuning; unset = cost model).
static int prefill_kpieces_override() {
  const char* e = std::getenv("G4_PREFILL_KPIECES");
  if (!e) return 0;
  const int v = std::atoi(e);
  return (v >= 1 && v <= 64) ? v : 0;
}

PrefillPlan plan_prefill(int B, int S, int Hq, int Hkv, int D, int W, int P0) {
  PrefillPlan p;
  p.BN = prefill_key_tile(D);
  p.ntiles = ceil_div(P0 + S, p.BN);
  p.g = Hq / Hkv;
  const int forced = D == 256 ? prefill_rows_override() : 0;
  double best = 0.0;
  int best_tiles = 0;
  for (int rows : {128, 64}) {
    if (rows == 64 && D != 256) continue;
    if (forced && rows != forced) continue;
    const int nqt = ceil_div(S * p.g, rows);
    const PrefillCosts c = prefill_costs(D, rows);
    for (int paired = 1; paired >= 0; --paired) {
      const int nunits = paired ? (nqt + 1) / 2 : nqt;
      // largest key work of a unit bounds the useful number of pieces
      int umax = 1;
      for (int i = 0; i < nunits; ++i) {
        int a0, a1, b0 = 0, b1 = -1;
        if (paired) {
          prefill_tile_keys(nqt - 1 - i, S, p.g, W, p.BN, rows, P0, a0, a1);
          if (i < nqt - 1 - i) prefill_tile_keys(i, S, p.g, W, p.BN, rows, P0, b0, b1);
        } else {
          prefill_tile_keys(i, S, p.g, W, p.BN, rows, P0, a0, a1);
        }
        umax = std::max(umax, (a1 - a0 + 1) + (b1 - b0 + 1));
      }
      const long groups = (long)B * Hkv * nunits;
      int kmax =
          rows == 64 ? 1 : (int)std::max<long>(1, std::min<long>(std::min<long>(kPrefillSlots / groups, umax), 64));
      if (rows != 64 && prefill_kpieces_override()) kmax = std::min(prefill_kpieces_override(), umax);
      // the kernels cut a unit's key tiles at j * U / kpieces (j <= kpieces,
      // U <= 2 * ntiles) in 31-bit arithmetic
      kmax = (int)std::min<long long>(kmax, std::max<long long>(1, ((1LL << 31) - 1) / (2LL * p.ntiles + 2)));
      const int kforced = rows == 64 ? 0 : std::min(prefill_kpieces_override(), kmax);
      for (int k = 1; k <= kmax; ++k) {
        if (kforced && k != std::min(kforced, umax)) continue;
        const double rounds = std::ceil((double)groups * k / kPrefillSlots);
        const double segs = paired ? (k <= 2 ? 2.0 : 1.5) : 1.0;
        const double t = rounds * (std::ceil((double)umax / k) * c.tile + segs * c.segment + (k > 1 ? c.split : 0.0));
        if (best == 0.0 || t < best) {
          best = t;
          p.rows = rows;
          p.nqt = nqt;
          p.paired = paired;
          p.npair = nunits;
          p.kpieces = k;
          best_tiles = (int)std::ceil((double)umax / k);
        }
      }
    }
  }
  // The split-PV schedule of the head-size-512 kernel costs one more phase
  // and a longer pipeline start per segment and saves about 5 % per key
  // tile; it pays from about 32 key tiles per work-group on (measured:
  // faster at 65 tiles, slower at 16).
  const int spv = prefill_split_pv_override();
  p.split_pv = D == 512 && (spv >= 0 ? spv == 1 : best_tiles >= kSplitPvMinTiles) ? 1 : 0;
  const long groups = (long)B * Hkv * p.npair;
  p.kimg_bytes = (size_t)B * Hkv * p.ntiles * p.BN * D * 2;
  p.vimg_off = (p.kimg_bytes + 255) / 256 * 256;
  p.counters_off = p.vimg_off + (p.kimg_bytes + 255) / 256 * 256;
  p.ncounters = (size_t)B * Hkv * p.nqt;
  p.part_off = (p.counters_off + p.ncounters * 4 + 255) / 256 * 256;
  const int nw = prefill_waves(D);
  p.slot_bytes = (size_t)32 * D * 16 + (size_t)nw * 64 * 2 * 4;  // accumulators + (m, l) per wave and lane
  p.nslots = p.kpieces > 1 ? (size_t)groups * p.kpieces * 2 : 0;
  p.total = p.part_off + p.nslots * p.slot_bytes;
  return p;
}

size_t prefill_workspace(int B, int S, int Hq, int Hkv, int D, int W, int P0) {
  return plan_prefill(B, S, Hq, Hkv, D, W, P0).total;
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream, const ProfileEvents& ev) {
  const PrefillPlan pl = plan_prefill(p.B, p.S, p.Hq, p.Hkv, p.D, p.W, p.P0);
  char* ws = static_cast<char*>(p.kimg);
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kimg = reinterpret_cast<const uint16_t*>(ws);
  a.vimg = reinterpret_cast<const uint16_t*>(ws + pl.vimg_off);
  a.out = p.out;
  a.counters = reinterpret_cast<int*>(ws + pl.counters_off);
  a.part = reinterpret_cast<float*>(ws + pl.part_off);
  a.B = p.B;
  a.S = p.S;
  a.P0 = p.P0;
  a.span_end = p.span_end;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.g = pl.g;
  a.Lmax = p.Lmax;
  a.W = p.W;
  a.ntiles = pl.ntiles;
  a.nqt = pl.nqt;
  a.npair = pl.npair;
  a.paired = pl.paired;
  a.kpieces = pl.kpieces;
  a.qscale = p.scale * kLog2e * p.k_scale;
  a.vscale = p.v_scale;
  a.fd_g = make_fastdiv(pl.g);
  a.fd_kp = make_fastdiv(pl.kpieces);
  a.fd_pbh = make_fastdiv(pl.npair * pl.kpieces);
  a.fd_hkv = make_fastdiv(p.Hkv);
  fill_rope_rev(&a.rope, p.D, p.theta);
  const dim3 grid_k(2 * pl.ntiles, p.Hkv, p.B);
  const dim3 grid_a((unsigned)((long)p.B * p.Hkv * pl.npair * pl.kpieces));
  const void* kraw = p.k;
  const void* vraw = p.v;
  uint16_t* kimg = reinterpret_cast<uint16_t*>(ws);
  uint16_t* vimg = reinterpret_cast<uint16_t*>(ws + pl.vimg_off);
  if (p.images_ready) {
    // the operand images are the workspace's already, and the split tiles'
    // counters are zero: the key pass zeroed them, and every merge since
    // reset the ones it used
  } else if (p.D == 512) {
    if (p.fp8)
      hipLaunchKernelGGL((k_prefill_prep<512, 32, true>), grid_k, dim3(256), 0, stream, kraw, vraw, kimg, vimg,
                         p.P0 + p.S, p.Hkv, p.Lmax, pl.ntiles, a.rope, a.counters, (int)pl.ncounters);
    else
      hipLaunchKernelGGL((k_prefill_prep<512, 32, false>), grid_k, dim3(256), 0, stream, kraw, vraw, kimg, vimg,
                         p.P0 + p.S, p.Hkv, p.Lmax, pl.ntiles, a.rope, a.counters, (int)pl.ncounters);
  } else {
    if (p.fp8)
      hipLaunchKernelGGL((k_prefill_prep<256, 32, true>), grid_k, dim3(256), 0, stream, kraw, vraw, kimg, vimg,
                         p.P0 + p.S, p.Hkv, p.Lmax, pl.ntiles, a.rope, a.counters, (int)pl.ncounters);
    else
      hipLaunchKernelGGL((k_prefill_prep<256, 32, false>), grid_k, dim3(256), 0, stream, kraw, vraw, kimg, vimg,
                         p.P0 + p.S, p.Hkv, p.Lmax, pl.ntiles, a.rope, a.counters, (int)pl.ncounters);
  }
  if (p.D == 512) {
    if (ev.before) (void)hipEventRecord(ev.before, stream);
    if (a.span_end != nullptr) {
      // (spans run the split-PV schedule at every length: the other one's
      // register allocation spills with the per-row limit added)
      hipLaunchKernelGGL((k_prefill<512, 32, 2, true, true>), grid_a, dim3(512), 0, stream, a);
    } else {
      if (pl.split_pv)
        hipLaunchKernelGGL((k_prefill<512, 32, 2, true, false>), grid_a, dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL((k_prefill<512, 32, 2, false, false>), grid_a, dim3(512), 0, stream, a);
    }
  } else {
    if (ev.before) (void)hipEventRecord(ev.before, stream);
    const bool prod = prefill_producer_override() != 0;  // 64-row tiles: copies from producer waves
    if (a.span_end != nullptr) {
      if (pl.rows == 64 && prod)
        hipLaunchKernelGGL((k_prefill4<256, 32, 64, true, true>), grid_a, dim3(512), 0, stream, a);
      else if (pl.rows == 64)
        hipLaunchKernelGGL((k_prefill4<256, 32, 64, true, false>), grid_a, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((k_prefill4<256, 32, 128, true, false>), grid_a, dim3(256), 0, stream, a);
    } else {
      if (pl.rows == 64 && prod)
        hipLaunchKernelGGL((k_prefill4<256, 32, 64, false, true>), grid_a, dim3(512), 0, stream, a);
      else if (pl.rows == 64)
        hipLaunchKernelGGL((k_prefill4<256, 32, 64, false, false>), grid_a, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((k_prefill4<256, 32, 128, false, false>), grid_a, dim3(256), 0, stream, a);
    }
  }
  if (ev.after) (void)hipEventRecord(ev.after, stream);
  return hipGetLastError();
}

// Average partials per stream up to which the merge takes a whole head per
// work-group (its threads then hold 2 (head size 512) or 4 (256) groups
// of four partials in flight).  Measured on the batched decode's sliding
// layer (about nine partials per stream): the whole-head merge takes 3 us
// less than the 64-wide slices.
constexpr int kCombineWideMaxParts = 12;

// G4_DECODE_PIECES=n (1..512) caps the decode split at n work-groups
// (tuning; unset = 512, two per CU).
static int decode_pieces_override() {
  const char* e = std::getenv("G4_DECODE_PIECES");
  if (!e) return 0;
  const int v = std::atoi(e);
  return (v >= 1 && v <= kDecodePieces) ? v : 0;
}

DecodePlan plan_decode(int /*B*/, int /*Hkv*/, int /*W*/, int /*max_kv_len*/) {
  DecodePlan plan;
  const int o = decode_pieces_override();
  plan.npieces = o ? o : kDecodePieces;
  return plan;
}

// Query columns of one (batch, kv head): T tokens x g heads, in groups of 16
// (the N dimension of the decode MFMAs); each group is a stream of its own.
static void decode_columns(int T, int g, int& ncg, int& cols) {
  ncg = ceil_div(T * g, 16);
  cols = ncg == 1 ? T * g : 16;
}

size_t decode_workspace(int B, int Hq, int Hkv, int D, int T, const DecodePlan& plan) {
  // one partial per (stream + piece) slot and query column of the stream
  int ncg, cols;
  decode_columns(T, Hq / Hkv, ncg, cols);
  const size_t parts = ((size_t)B * Hkv * ncg + plan.npieces) * (size_t)cols;
  return parts * D * sizeof(float) + parts * sizeof(float);
}

hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream, const ProfileEvents& ev) {
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.alias ? p.k : p.v);
  a.kc = static_cast<uint16_t*>(p.k);
  a.vc = static_cast<uint16_t*>(p.alias ? p.k : p.v);
  a.ring = p.ring;
  a.knew = static_cast<const uint16_t*>(p.k_new);
  a.vnew = static_cast<const uint16_t*>(p.alias ? p.k_new : p.v_new);
  a.kv_len = p.kv_len;
  a.T = p.T;
  decode_columns(p.T, p.Hq / p.Hkv, a.ncg, a.cols);
  const size_t parts = ((size_t)p.B * p.Hkv * a.ncg + p.plan.npieces) * (size_t)a.cols;
  a.part_o = static_cast<float*>(p.ws);
  a.part_lse = a.part_o + parts * p.D;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.g = p.Hq / p.Hkv;
  a.Lmax = p.Lmax;
  a.W = p.W;
  a.npieces = p.plan.npieces;
  a.qscale = p.scale * kLog2e * p.k_scale;
  a.vscale = p.v_scale;
  a.kstore = p.k_scale;
  a.vstore = p.alias ? p.k_scale : p.v_scale;
  fill_rope_rev(&a.rope, p.D, p.theta);
  const dim3 grid((unsigned)p.plan.npieces);
  if (p.fp8 && a.knew != nullptr) {
    // an E4M3 cache takes the new rows quantised before the attention reads it
    const dim3 ga((unsigned)(p.B * p.T * p.Hkv));
    if (p.D == 512)
      hipLaunchKernelGGL((k_append_fp8<512>), ga, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((k_append_fp8<256>), ga, dim3(64), 0, stream, a);
    a.knew = a.vnew = nullptr;
  }
  if (ev.before) (void)hipEventRecord(ev.before, stream);
  const bool gen = p.T > 1 || p.ring > 0 || a.knew != nullptr;
  const bool ring_or_append = p.ring > 0 || a.knew != nullptr;
  auto run = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a); };
  // LDS stages: 4 of 16 rows, except head size 512 with separate K and V
  // (2 of bf16, 3 of E4M3 beside the converted value tile), so that two
  // work-groups share a CU
  auto pick = [&](auto d_c, auto alias_c, auto fp8_c) {
    constexpr int D = decltype(d_c)::value;
    constexpr bool AL = decltype(alias_c)::value, F8 = decltype(fp8_c)::value;
    constexpr int NS = (D == 512 && !AL) ? (F8 ? 3 : 2) : kDecodeStages;
    if (!gen)
      run(k_decode<D, AL, NS, false, F8, false>);
    else if (ring_or_append)
      run(k_decode<D, AL, NS, true, F8, true>);
    else
      run(k_decode<D, AL, NS, true, F8, false>);
  };
  using D512 = std::integral_constant<int, 512>;
  using D256 = std::integral_constant<int, 256>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (p.D == 512) {
    if (p.alias)
      p.fp8 ? pick(D512{}, T_{}, T_{}) : pick(D512{}, T_{}, F_{});
    else
      p.fp8 ? pick(D512{}, F_{}, T_{}) : pick(D512{}, F_{}, F_{});
  } else {
    if (p.alias)
      p.fp8 ? pick(D256{}, T_{}, T_{}) : pick(D256{}, T_{}, F_{});
    else
      p.fp8 ? pick(D256{}, F_{}, T_{}) : pick(D256{}, F_{}, F_{});
  }
  if (ev.after) (void)hipEventRecord(ev.after, stream);
  // Streams of few pieces: one work-group per head; of many: 64-wide slices.
  const int nstreams = p.B * p.Hkv * a.ncg;
  const bool wide = p.plan.npieces / nstreams + 1 <= kCombineWideMaxParts;
  const unsigned nq = (unsigned)(p.B * p.T * p.Hq);
  if (p.D == 512) {
    if (wide)
      hipLaunchKernelGGL((k_decode_combine<512, 128>), dim3(nq), dim3(256), 0, stream, a, p.out);
    else
      hipLaunchKernelGGL((k_decode_combine<512, 16>), dim3(nq, 512 / 64), dim3(256), 0, stream, a, p.out);
  } else {
    if (wide)
      hipLaunchKernelGGL((k_decode_combine<256, 64>), dim3(nq), dim3(256), 0, stream, a, p.out);
    else
      hipLaunchKernelGGL((k_decode_combine<256, 16>), dim3(nq, 256 / 64), dim3(256), 0, stream, a, p.out);
  }
  return hipGetLastError();
}

// ------------------------------------------------- static device scratch --
// Decode scratch for callers that cannot allocate device memory: a
// file-scope device array, one copy per GPU the library runs on (it lives
// until the process ends).  Host code never passes the array's name to a
// kernel: that is a host-side stand-in, not a device address.  Its device
// address is looked up once per device, with that device current, and kept.

namespace {
static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(hipStream_t stream, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if ((int)sdev != cur) return hipErrorInvalidDevice;  // the lookup needs the stream's device current
  }
  if (cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[cur] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[cur] = p;
  }
  *ptr = g_scratch_ptr[cur];
  return hipSuccess;
}

}  // namespace g4
