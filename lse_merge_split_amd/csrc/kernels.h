// kernels.h -- internal launch interface between the C-ABI host code and the
// HIP kernels of libcpdec.  Not installed; the public API is include/cpdec.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpdec {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

constexpr int kMaxShards = 64;     // equals CPDEC_MAX_SHARDS
constexpr int kTileTokens = 32;    // tokens one wave consumes per loop step
constexpr int kMaxChunks = 256;    // split-KV chunks per (shard, seq, kv head)
constexpr int kGroupRows = 16;     // query heads per MFMA column block

struct AttnParams {
  const void* q;
  const void* k[kMaxShards];
  const void* v[kMaxShards];
  const int32_t* lens;
  void* o_part;
  float* lse_part;
  float* ws_o;        // [units][nchunks][Gb][D] chunk partials (normalised)
  float* ws_lse;      // [units][nchunks][Gb]    chunk lse (natural log)
  int64_t sb, sh, st; // K/V element strides: batch, head, token
  int32_t B, Hq, Hkv, G, Gb, gblocks, R, chunk, nchunks, units, odt;
  int32_t cap;        // K/V capacity per (shard, sequence, kv head), tokens
  float scale_log2;   // sm_scale * log2(e)
  // the whole step (cpdec_cp_decode) only:
  void* out;          // [B][Hq][D] merged output, dtype out_dt
  float* lse_out;     // [B][Hq] merged lse, may be null
  int32_t out_dt;
  int32_t* counters;  // [B * Hkv * gblocks] arrival counters, zero between calls
  // longest-first launch order (unsplit shards only): [R * B] OrderEntry, filled
  // by the order kernel before the attention launch; null: index order
  void* order;
};

// One (shard, sequence) pair of the longest-first launch order.
struct OrderEntry {
  const void* k;  // the pair's shard K and V base pointers
  const void* v;
  int32_t r, b;   // shard, sequence
  int32_t len;    // lens[r][b] as given
  int32_t pad;
};
static_assert(sizeof(OrderEntry) == 32, "order entry layout");

// Longest-first launch order: when shards are not split and the grid is large,
// a one-workgroup pre-pass sorts the (shard, sequence) pairs by length,
// longest first, so that the longest units start first and the short ones
// fill the end of the launch (longest-processing-time-first scheduling).
// The pre-pass costs about 10 us (a launch and a sort), so it is used only
// where the attention is long enough for the schedule to matter.
constexpr int kOrderMaxPairs = 4096;      // R * B that the one-workgroup sort takes
constexpr int64_t kOrderMinUnits = 2048;  // smaller grids keep index order
constexpr double kOrderMinKvBytes = 4294967296.0;  // K+V bytes at capacity, at least

// How a launch treats the cross-shard merge.
enum StepMode : int {
  kPartialsOnly = 0,   // cpdec_attn_partial: o_part/lse_part only
  kStepLaunches = 1,   // whole step as attention, chunk combine and merge launches
  kStepOneShards = 2,  // whole step in one launch, shards not split: the last
                       // shard workgroup of a (sequence, kv head) merges
  kStepOneChunks = 3,  // whole step in one launch, shards split into chunks:
                       // the last chunk workgroup combines chunks and merges
  kStepTwoLevel = 4,   // whole step in one launch, shards split, group too big
                       // for one merging workgroup: the last chunk workgroup of
                       // a unit combines its chunks, the last unit of a group
                       // merges the shards
  kPartialsCombine = 5,  // cpdec_attn_partial, shards split: the last chunk
                         // workgroup of a unit combines its chunks in the launch
};

// Limits of the one-launch step.  The workgroup that merges a group fetches
// everything it needs in one round of loads, so the group must fit it: at
// most one (shard, head) pair and one (shard, head, float4) item per thread,
// at most 16 chunks per shard (16 loads per thread), at most 8 shards when
// shards are not split.  Larger groups take separate launches, where the
// merge work spreads over many workgroups.
constexpr size_t kStepCounterBytes = 65536; // counters at the start of the workspace
constexpr int kStepCounterStride = 16;      // ints: one 64-byte line per counter (atomics
                                            // on one line serialise across groups)
constexpr int kStepCounters = (int)(kStepCounterBytes / 4 / kStepCounterStride);  // groups
constexpr int kStepMaxChunks = 16;          // chunks per shard, split shards
constexpr int kStepMaxShardsUnsplit = 8;    // shards, unsplit
constexpr int kStepSlots = 2048;            // shards * chunks * heads of one group
constexpr int kStepVecs = 512;              // shards * heads * D/4 of one group (<= threads)
constexpr int64_t kStepUnsplitBlocks = 1024; // unsplit shards: one launch up to this grid
constexpr int kStepTwoLevelMaxChunks = 64;   // chunks per shard in the two-level form (lanes
                                             // of one wave per head in the chunk statistics)

// Separate-launch step with split shards: when a query head's (shard, chunk)
// pairs fit one wave (R * chunks rounded up to a power of two <= 64), one
// kernel with a workgroup per (sequence, query head) combines the chunks and
// merges the shards (instead of a chunk-combine and a merge launch).  Its
// waves: threads >= max(R * D/4, D) (one (shard, float4) item per thread, and
// every live chunk within the 16 loads per thread group).  The kernel uses
// 32-bit buffer offsets: the chunk partials (ws_o_bytes) and o_part
// (opart_bytes) must stay below 2 GiB.  0: not eligible.
inline int row_merge_waves(int R, int nchunks, int D, int64_t ws_o_bytes, int64_t opart_bytes) {
  int nchp = 1;
  while (nchp < nchunks) nchp <<= 1;
  if (nchunks < 2 || R * nchp > 64) return 0;
  if (ws_o_bytes >= (int64_t(1) << 31) || opart_bytes >= (int64_t(1) << 31)) return 0;
  const int need = R * (D / 4) > D ? R * (D / 4) : D;
  int w = 2;
  while (w < 8 && 64 * w < need) w *= 2;
  return 64 * w >= need ? w : 0;
}

// Launch the partial-attention kernel over (units / R) x nchunks x R workgroups and
// whatever else `mode` needs (chunk combine and merge kernels for
// kPartialsOnly/kStepLaunches; nothing for the one-launch modes).
hipError_t launch_attn_partial(const AttnParams& p, int qkv_dt, int D, int waves,
                               int64_t units, StepMode mode, hipStream_t s);
// the same for one element type (the per-type halves of the build)
hipError_t launch_attn_partial_bf16(const AttnParams& p, int D, int waves, int64_t units,
                                    StepMode mode, hipStream_t s);
hipError_t launch_attn_partial_f16(const AttnParams& p, int D, int waves, int64_t units,
                                   StepMode mode, hipStream_t s);

hipError_t launch_lse_merge(const void* o, const float* lse, int R, int64_t rows, int D,
                            int in_dt, int out_dt, void* out, float* lse_out, hipStream_t s);
int64_t lse_merge_max_blocks(int64_t rows, int D, int in_dt);

hipError_t launch_clear(void* p, size_t bytes, hipStream_t s);

}  // namespace cpdec
