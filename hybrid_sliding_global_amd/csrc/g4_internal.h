// Internal host-side interface between the C-ABI layer (g4_api.cpp) and the
// kernel launchers (g4_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace g4 {

// RoPE frequencies of one layer in revolutions per position:
// rev[f] = theta^(-2f/D) / (2*pi), f < D/2 (rotate-half pairs (f, f + D/2)).
struct RopeRev {
  double rev[256];
};

void fill_rope_rev(RopeRev* r, int head_dim, double theta);

// Prefill tiling: 32-key tiles and 128 query rows per work-group for both
// head sizes (head size 256 may instead run 64-row tiles).  Head size 512 runs eight waves (two per SIMD, each pair of
// waves splitting the head dimension of one 32-row group); head size 256
// runs four waves (one per SIMD: scores by row block, output by head-dim
// block).
constexpr int kPrefillRows = 128;
inline int prefill_key_tile(int /*head_dim*/) { return 32; }
inline int prefill_waves(int head_dim) { return head_dim == 512 ? 8 : 4; }
// Work-groups one prefill launch aims to keep busy: the CU count of an
// MI355X (one resident prefill work-group per CU).  Fixed so that workspace
// sizes can be computed without touching the device.
constexpr int kPrefillSlots = 256;

// How a prefill call is cut into work-groups and how its workspace is laid
// out: [key operand image][value operand image][arrival counters]
// [partial-result slots]; each image is [B, Hkv, ntiles, BN * D] bf16.
struct PrefillPlan {
  int BN = 0, ntiles = 0, g = 0, nqt = 0, npair = 0, kpieces = 0;
  int rows = kPrefillRows;  // query rows per tile: 128, or 64 (head size 256, never cut into pieces)
  int paired = 1;  // work unit: 1 = query tiles t and nqt-1-t, 0 = one query tile
  int split_pv = 0;  // head size 512: PV of a tile split over two phases (long segments)
  size_t kimg_bytes = 0, vimg_off = 0, counters_off = 0, ncounters = 0, part_off = 0, slot_bytes = 0, nslots = 0,
         total = 0;
};
PrefillPlan plan_prefill(int B, int S, int Hq, int Hkv, int D, int W, int P0);

struct PrefillLaunch {
  const void* q;      // bf16 [B, S, Hq, D]
  const void* k;      // bf16 raw keys [B, Hkv, Lmax, D]
  const void* v;      // bf16 values (== k for an aliased layer)
  float* out;         // fp32 [B, S, Hq, D]
  void* kimg;         // workspace (operand images, counters, partial slots)
  int B, S, Hq, Hkv, D, Lmax, W;
  int P0;             // position of query 0: queries P0 .. P0+S-1 over keys 0 .. P0+S-1
  const int32_t* span_end;  // null, or device [B, S]: last position of each query's bidirectional span
  bool images_ready;  // the workspace already holds this call's key/value operand images: no key pass
  bool fp8;           // the cache holds E4M3 bytes: key element = code * k_scale, value = code * v_scale
  float k_scale, v_scale;  // (v_scale is k_scale for an aliased layer; both 1 for bf16)
  float scale;        // softmax scale (already resolved, > 0)
  double theta;
};

// Optional events recorded around the main attention kernel (may be null).
struct ProfileEvents {
  hipEvent_t before = nullptr;
  hipEvent_t after = nullptr;
};

size_t prefill_workspace(int B, int S, int Hq, int Hkv, int D, int W, int P0);
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream, const ProfileEvents& ev);

// Decode split: the visible keys of all (batch, kv-head) streams are cut
// into equal pieces on the device (from kv_len), one per work-group.
struct DecodePlan {
  int npieces;  // work-groups (pieces of at least 64 keys; fewer when the keys are few)
};
DecodePlan plan_decode(int B, int Hkv, int W, int max_kv_len);
size_t decode_workspace(int B, int Hq, int Hkv, int D, int T, const DecodePlan& plan);

struct DecodeLaunch {
  const void* q;        // bf16 [B, T, Hq, D]
  void* k;              // bf16 raw keys [B, Hkv, Lmax, D] (written only when appending)
  void* v;              // bf16 values (== k when aliased)
  const int32_t* kv_len;  // device [B]
  float* out;           // fp32 [B, T, Hq, D]
  void* ws;
  int B, Hq, Hkv, D, Lmax, W, alias;
  int T;                // query tokens per sequence (positions kv_len - T .. kv_len - 1)
  int ring;             // 0: row j holds position j; C > 0: row j % C (Lmax == C)
  const void* k_new;    // null, or bf16 [B, T, Hkv, D]: keys of the T tokens, written into the cache
  const void* v_new;    // values of the T tokens (== k_new when aliased)
  bool fp8;             // the cache holds E4M3 bytes: key element = code * k_scale, value = code * v_scale
  float k_scale, v_scale;
  float scale;
  double theta;
  DecodePlan plan;
};

hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream, const ProfileEvents& ev);

// Device scratch of kStaticScratchBytes (a file-scope device array, one per
// GPU) for the decode entry point that allocates nothing: its device address
// on the current device, looked up on first use.  Fails with
// hipErrorInvalidDevice if `stream` belongs to another device than the
// current one.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(hipStream_t stream, void** ptr);

}  // namespace g4
