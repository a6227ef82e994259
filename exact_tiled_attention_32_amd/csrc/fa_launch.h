// Internal interface between the C-ABI layer (fa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// Forward arguments, already validated by the host layer.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_len;  // nullptr: every key valid
  const uint8_t* mask;    // nullptr: dense
  int B, H, N;
  int mb;                 // mask block side (multiple of 128) when mask != nullptr
  int nb;                 // mask blocks per side
  int ntq;                // query tiles per (b, h)
  int causal;
  float c2;               // |scale| * log2(e), or log2(e) when scale == 0 (exp2 domain)
  float sc_abs;           // |scale|: lse = m * |scale| + ln l
  float qmul;             // +1, -1 (negative scale) or 0 (zero scale), applied to Q exactly
  // Sliding window: key j allowed for query i iff i - wl <= j <= i + wr; a negative extent
  // is unbounded. The host sets wr = 0 for causal attention.
  int wl, wr;
  // Packed variable-length sequences (cu != nullptr): B counts sequences, tensors are
  // [total, H, d] (row stride rs = H d), sequence s owns tokens cu[s] .. cu[s+1] - 1, lse
  // is [H, total]; N is then the longest sequence. Dense: cu == nullptr, rs == d.
  const int32_t* cu;
  int rs;
  int total;
  // Dropout on the probabilities (used by the dropout instantiations only).
  uint32_t drop_thr, seed_lo, seed_hi;
  float drop_scale;
};

// Backward arguments, already validated by the host layer.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;            // workspace: D = rowsum(dO * O), [B,H,N]
  uint32_t* order;        // workspace: dK/dV key tiles, most mask blocks first (block-sparse)
  const int32_t* kv_len;
  const uint8_t* mask;
  int B, H, N, mb, nb;
  int causal;
  float scale;            // signed softmax scale
  float c2s;              // scale * log2(e)
  int wl, wr;             // sliding window, as in FwdArgs
  const int32_t* cu;      // packed sequences, as in FwdArgs (dsum then [H, total] too)
  int rs;
  int total;
  uint32_t drop_thr, seed_lo, seed_hi;  // dropout, as in FwdArgs
  float drop_scale;
  int dropout;            // nonzero: launch the dropout instantiations
};

// Key/value-cache forward arguments, already validated by the host layer.
struct DecArgs {
  const void* q;          // [B, H, Nq, d]
  const void* k;          // [B, H, Nk, d]
  const void* v;
  void* o;                // [B, H, Nq, d]
  float* lse;             // [B, H, Nq]
  const int32_t* kv_len;  // nullptr: every cached key valid
  float* part_u;          // workspace: [slots, Nq, d] unnormalised partial outputs
  float* part_m;          // workspace: [slots, Nq] partial maxima (raw q.k units)
  float* part_l;          // workspace: [slots, Nq] partial sums
  int B, H, Nq, Nk;
  int waves;              // key-split waves launched (those past the tile count stay idle)
  int causal;
  float c2, sc_abs, qmul; // as in FwdArgs
};

constexpr int kDecMaxQueries = 32;

// Longest sequence the kernels take (dense N, packed max_seqlen): row indices plus a tile
// or a window extent below it stay far from the int range.
constexpr int kMaxSeqLen = 1 << 30;

// Most key-split waves of one call; partial-result slots of a call number
// kvcache_max_waves(B, H, Nk) + B H - 1.
constexpr int kDecMaxWaves = 2048;
// Waves a call may launch: min(kDecMaxWaves, the 32-key tiles of a full cache), at least 1.
int kvcache_max_waves(int B, int H, int Nk);

constexpr int kFwdRowsPerWG = 128;       // fp32 forward; also the mask-block granularity
constexpr int kFwdRowsPerWGBF16 = 128;   // bf16 forward: 4 waves x 32 query rows
// Keys per tile of the bf16 forward (its block-sparse tile list holds N / that).
constexpr int fwd_tile_keys_bf16(int) { return 64; }
constexpr int kFwdTileKeysF32 = 32;
constexpr int kMaxTileList = 4096;
// Smallest tile of the backward kernels (32 query rows per dK/dV step at d = 128); their
// block-sparse tile lists hold at most N / 32 entries.
constexpr int kBwdMinTile = 32;
// Keys per dK/dV workgroup, and the capacity of the block-sparse key-tile order.
constexpr int kBwdKeyTile = 128;
constexpr int kMaxKeyTiles = kMaxTileList * kBwdMinTile / kBwdKeyTile;

// Optional measurement events of a call: ev[0] is recorded before its first kernel and
// ev[i] after its i-th kernel, as far as the caller supplied events (n of them).
struct KernelTimer {
  static constexpr int kMax = 8;
  hipEvent_t ev[kMax] = {};
  int n = 0;
  int next = 0;
  void mark(hipStream_t stream) {
    if (next < n) (void)hipEventRecord(ev[next++], stream);
  }
};

hipError_t launch_fwd(const FwdArgs& a, fa_dtype dt, int d, hipStream_t stream, KernelTimer& tm,
                      bool dropout = false);
hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t stream, KernelTimer& tm);
hipError_t launch_kvcache(const DecArgs& a, int d, hipStream_t stream, KernelTimer& tm);

}  // namespace fa
