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
  float scale_log2;   // sm_scale * log2(e)
};

// Where the whole step (cpdec_cp_decode) writes the merged result.
struct StepOut {
  void* out;
  float* lse_out;  // may be null
  int out_dt;
};

// Launch the partial-attention kernel over units x nchunks workgroups, then
// (when a unit can span several chunks) the chunk-combine kernel over units.
// With `so` the cross-shard merge follows: fused into the chunk merge when
// shards are split, else the plain merge kernel (two launches either way).
hipError_t launch_attn_partial(const AttnParams& p, int qkv_dt, int D, int waves,
                               int64_t units, const StepOut* so, hipStream_t s);

hipError_t launch_lse_merge(const void* o, const float* lse, int R, int64_t rows, int D,
                            int in_dt, int out_dt, void* out, float* lse_out, hipStream_t s);
int64_t lse_merge_max_blocks(int64_t rows, int D, int in_dt);

hipError_t launch_clear(void* p, size_t bytes, hipStream_t s);

}  // namespace cpdec
