// cpdec_api.hip -- the C ABI of libcpdec (include/cpdec.h): argument checks,
// launch planning and kernel dispatch.  Every check runs before any HIP call.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "cpdec.h"
#include "kernels.h"

static_assert(cpdec::kStepCounterBytes == CPDEC_STEP_COUNTER_BYTES, "counter region size");

// Scratch of cpdec_cp_decode_noalloc: one copy per GPU, held until the
// process ends, shared by every call on that GPU.  In host code this name is
// only a stand-in for the symbol; the device address of each GPU's copy comes
// from hipGetSymbolAddress (scratch_for_stream below) and is the only
// thing host code passes on.
static __device__ __align__(256) unsigned char scratch[CPDEC_NOALLOC_SCRATCH_BYTES];
static_assert(CPDEC_NOALLOC_SCRATCH_BYTES >= CPDEC_STEP_COUNTER_BYTES, "scratch holds the counters");

namespace {

using namespace cpdec;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int dt) { return dt == CPDEC_F32 || dt == CPDEC_F16 || dt == CPDEC_BF16; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Experiment overrides, read once at first use (never inside a timed loop).
struct Overrides {
  int waves = 0;   // CPDEC_WAVES: 1, 2, 4 or 8
  int chunk = 0;   // CPDEC_CHUNK: tokens, multiple of 32
  bool step_launches = false;  // CPDEC_STEP_LAUNCHES=1: the whole step as separate launches
  bool no_order = false;       // CPDEC_ORDER=0: index launch order always
  Overrides() {
    if (const char* s = getenv("CPDEC_ORDER")) no_order = atoi(s) == 0;
    if (const char* s = getenv("CPDEC_STEP_LAUNCHES")) step_launches = atoi(s) != 0;
    if (const char* s = getenv("CPDEC_WAVES")) {
      int w = atoi(s);
      if (w == 1 || w == 2 || w == 4 || w == 8) waves = w;
    }
    if (const char* s = getenv("CPDEC_CHUNK")) {
      int c = atoi(s);
      if (c >= 32 && c % 32 == 0) chunk = c;
    }
  }
};
const Overrides& overrides() {
  static const Overrides o;
  return o;
}

constexpr int kDefaultWaves = 4;        // waves per workgroup when shards are not split
constexpr int kSplitWaves = 2;          // waves per workgroup when shards are split
constexpr int64_t kSplitBlocks = 512;   // fewer units than this: split shards into chunks,
                                        // aiming at this many workgroups
constexpr int64_t kMinSplitBlocks = 256;  // one workgroup per CU at least
constexpr int kMinWaveTiles = 8;          // tiles a wave should see after a wave raise
constexpr int kSplitMinTiles = 4;         // tiles a wave should see in a split launch
// Longest chunk the library picks.  A wave accumulates its p.V sums in FP32
// (MFMA accumulators), one rounding per tile; when one early token dominates
// and the rest add nearly constant small terms, that rounding is biased, so
// the error grows with the tiles per wave (measured on such input: ~1e-3 of
// the output at 65536 tiles per wave, just past the output tolerance).  No
// chunk is longer than 2^18 tokens, whoever picks it: a wave then sees at
// most 2048 tiles in a 4-wave workgroup (4096 in a 2-wave one).  Longer
// shards are split into chunks and merged with the LSE weighting.
constexpr int kMaxChunkTokens = 1 << 18;

struct AttnPlan {
  int waves = 0;
  int chunk = 0;
  int nchunks = 0;
  int G = 0, Gb = 0, gblocks = 0;
  int64_t units = 0;
  size_t ws_bytes = 0;       // what cpdec_attn_partial needs (0: no workspace)
  size_t step_ws_bytes = 0;  // what cpdec_cp_decode needs (counters + partials)
  size_t off_lse = 0, off_o = 0;
  size_t off_order = 0;      // longest-first launch order entries (when ordered)
  bool ordered = false;      // launch (shard, sequence) pairs longest first
  bool partials_combine = false;  // cpdec_attn_partial combines chunks in its one launch
  StepMode step = kStepLaunches;  // how cpdec_cp_decode runs
};

// Validate a descriptor (no pointers) and plan the launch.
cpdec_status plan_attn(const cpdec_attn_desc* d, AttnPlan* pl) {
  if (d == nullptr) return CPDEC_ERR_INVALID_ARG;
  if (d->batch <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->num_shards <= 0 || d->kv_capacity < 0)
    return CPDEC_ERR_INVALID_ARG;
  if (d->num_shards > CPDEC_MAX_SHARDS) return CPDEC_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return CPDEC_ERR_INVALID_ARG;
  if (!(d->sm_scale >= 0.f) || isinf(d->sm_scale)) return CPDEC_ERR_INVALID_ARG;
  if (d->chunk_tokens < 0 || (d->chunk_tokens > 0 && d->chunk_tokens % kTileTokens != 0))
    return CPDEC_ERR_INVALID_ARG;
  const int D = d->head_dim;
  if (D != 64 && D != 128 && D != 256) return CPDEC_ERR_UNSUPPORTED;
  if (d->qkv_dtype != CPDEC_F16 && d->qkv_dtype != CPDEC_BF16) return CPDEC_ERR_UNSUPPORTED;
  if (!valid_dtype(d->opart_dtype)) return CPDEC_ERR_UNSUPPORTED;
  if (d->kv_stride_token < D || d->kv_stride_head < 0 || d->kv_stride_batch < 0)
    return CPDEC_ERR_INVALID_ARG;
  // 16-byte rows: every stride, in bytes, a multiple of 16 (2-byte elements).
  if ((d->kv_stride_token | d->kv_stride_head | d->kv_stride_batch) % 8 != 0)
    return CPDEC_ERR_ALIGNMENT;

  // K/V of one (shard, sequence, kv head) are addressed with 32-bit offsets.
  if ((int64_t)(d->kv_capacity > 0 ? d->kv_capacity : 1) * d->kv_stride_token * 2 >= (1ll << 31))
    return CPDEC_ERR_UNSUPPORTED;

  AttnPlan p;
  p.G = d->num_q_heads / d->num_kv_heads;
  p.Gb = p.G < kGroupRows ? p.G : kGroupRows;
  p.gblocks = (int)ceil_div(p.G, kGroupRows);
  p.units = (int64_t)d->num_shards * d->batch * d->num_kv_heads * p.gblocks;
  const int64_t cap = d->kv_capacity > 0 ? d->kv_capacity : 1;
  // Shards are split into chunks only when the units alone cannot fill the
  // GPU (every chunk costs a partial write and a merge).  Split problems are
  // latency-bound: fewer, smaller workgroups with two tiles per wave in
  // flight measured fastest (c2: 23 vs 27 us).  Exactly kMinSplitBlocks units
  // (one workgroup per CU) stay whole: over two samples of random shapes
  // (100 in all) that put 6 more within 8% of the best plan measured and
  // none more than 5% slower (4 shards x 8 sequences x 8 kv heads over 512
  // tokens: 18.6 vs 23.2 us).
  const bool split = d->chunk_tokens == 0 && overrides().chunk == 0 && p.units < kSplitBlocks &&
                     p.units != kMinSplitBlocks && cap > (int64_t)kTileTokens * kDefaultWaves;
  p.waves = overrides().waves ? overrides().waves : (split ? kSplitWaves : kDefaultWaves);
  const int span = kTileTokens * p.waves;  // tokens one pass of all waves covers

  int chunk = d->chunk_tokens ? d->chunk_tokens : overrides().chunk;
  if (chunk == 0) {
    int64_t want = split ? ceil_div(kSplitBlocks, p.units) : 1;
    const int64_t most = ceil_div(cap, span);      // chunks of one pass of all waves
    if (want > most) want = most;
    // More than kStepTwoLevelMaxChunks chunks leave only the three-launch step
    // (batch 1, 16 heads on one kv head, 8192 tokens at D = 256: 64.3 us with
    // 128 chunks, 16.1 us with 64).
    if (want > kStepTwoLevelMaxChunks) want = kStepTwoLevelMaxChunks;
    chunk = (int)(ceil_div(ceil_div(cap, want), span) * span);
    // At least kSplitMinTiles tiles per wave while kMinSplitBlocks workgroups
    // remain (8 shards x 4 heads x 2048 tokens at D = 64: 15.0 us over 128-token
    // chunks, 11.6 us over 256).
    if (split) {
      const int64_t c_min = (int64_t)kSplitMinTiles * span;
      if (chunk < c_min && p.units * ceil_div(cap, c_min) >= kMinSplitBlocks) chunk = (int)c_min;
    }
  }
  if (chunk > kMaxChunkTokens) chunk = kMaxChunkTokens;  // a multiple of every span
  if (ceil_div(cap, chunk) > kMaxChunks)
    chunk = (int)ceil_div(ceil_div(cap, kMaxChunks), kTileTokens) * kTileTokens;
  p.chunk = chunk;
  p.nchunks = (int)ceil_div(cap, chunk);
  // Split shards: the workgroup that merges a group in the one-launch step
  // needs a thread per (shard, head, float4) item; give it more waves when
  // that lets the group fit (a wave past the chunk's end simply sees no tile).
  // When the library picked the chunks, it also doubles their length while a
  // wave would see fewer than kMinWaveTiles tiles and at least
  // kMinSplitBlocks workgroups remain: more waves over the same short chunks
  // measured 9-50% slower (batch 1, MHA, 16 x 2048 tokens at D = 64: 22.0 us
  // with 4 waves over 256-token chunks, 14.7 us over 512-token chunks).
  // Where the waves as they are would merge through the row-merge launch, the
  // raise needs each wave to keep at least 2 tiles of library-picked chunks
  // (2 shards x 64 heads over 512 tokens: 14.5 us with 8 waves over a quarter
  // tile each, 10.2 us with 2 waves and the row merge); where they would take
  // the two-level merge, the one-level merge of the raise wins even over
  // short chunks (16 shards x 2 heads over 1024 tokens at D = 64: 14.5 vs
  // 17.9 us).  The raise stops at 4 waves for D = 256, whose 8-wave kernels
  // spill registers to scratch (2.3-2.5x slower).
  bool raised = false;
  if (!overrides().waves && p.nchunks > 1) {
    const int64_t items = (int64_t)d->num_shards * p.Gb * (D / 4);
    const int w_max = D >= 256 ? 4 : 8;
    int w = p.waves;
    while (w < w_max && items > 64 * w) w *= 2;
    if (items <= 64 * w && w != p.waves) {
      int64_t c = p.chunk;
      if (split) {
        while (c < (int64_t)kMinWaveTiles * kTileTokens * w && 2 * c <= kMaxChunkTokens &&
               p.units * ceil_div(cap, 2 * c) >= kMinSplitBlocks)
          c *= 2;
      }
      const bool two_level_as_is = (int64_t)p.Gb * (D / 4) <= 64LL * p.waves;
      if (!split || two_level_as_is || c >= 2LL * kTileTokens * w) {
        p.waves = w;
        raised = true;
        p.chunk = (int)c;
        p.nchunks = (int)ceil_div(cap, c);
      }
    }
  }
  // Split launches whose merger did not set the waves, with at least one full
  // round of workgroups and long chunks: 2 or 4 waves, whichever fills the
  // last round of resident workgroups better (these kernels hold one wave per
  // SIMD, so kSplitBlocks x kSplitWaves / w workgroups at a time).  Batch 6,
  // GQA 4, 8 x 8192 tokens (768 workgroups): 288 us with 2 waves (1.5
  // rounds), 253 us with 4 (3 rounds).
  if (split && !raised && !overrides().waves && p.nchunks > 1 &&
      p.units * p.nchunks >= kSplitBlocks && p.chunk >= kMinWaveTiles * kTileTokens * 4) {
    auto fill = [&](int w) {
      const int64_t resident = kSplitBlocks * kSplitWaves / w;
      const int64_t nblocks = p.units * p.nchunks;
      return (double)nblocks / (double)(ceil_div(nblocks, resident) * resident);
    };
    if (fill(4) > fill(p.waves) + 1e-9) p.waves = 4;
  }
  // Split groups that no one-launch merge fits at the final waves (neither
  // the shards' vectors nor one unit's vectors fit the workgroup's threads):
  // the step takes the row merge when shards x chunks (rounded up to a power
  // of two) fit one wave and its workgroup fits the shards' vectors, else a
  // chunk-combine and a merge launch.  Library-picked chunks are made longer
  // to fit the row merge where it can run (4 shards x 3 sequences x 16 heads
  // over 4096 tokens at D = 256: 41.6 us with 32 chunks and three launches,
  // 22.7 us with 16 and two).
  // Where that would cut the chunks by more than half, 4 waves that let the
  // two-level merge fit are taken instead, over chunks of at least
  // kSplitMinTiles tiles per wave while kMinSplitBlocks workgroups remain (16
  // shards x 8 heads over 8192 tokens: 43.4 us over 4 chunks and the row
  // merge, 28.8 us with 4 waves over 16 chunks in one launch).
  if (split && p.nchunks > 1) {
    const int64_t threads = 64LL * p.waves;
    const int64_t items = (int64_t)d->num_shards * p.Gb * (D / 4);
    const int R = d->num_shards;
    int fit = 1;
    while (fit * 2 * R <= 64) fit *= 2;            // chunks whose power of two fits with R
    if (items > threads && (int64_t)p.Gb * (D / 4) > threads && fit >= 2 && p.nchunks > fit) {
      const int span_w = kTileTokens * p.waves;
      const int64_t c = ceil_div(ceil_div(cap, fit), span_w) * span_w;
      if (p.nchunks <= 2 * fit && row_merge_waves(R, fit, D, 0, 0) > 0 && c <= kMaxChunkTokens) {
        p.chunk = (int)c;
        p.nchunks = (int)ceil_div(cap, c);
      } else if (!overrides().waves && p.waves < 4 && (int64_t)p.Gb * (D / 4) <= 64 * 4 &&
                 p.nchunks <= kStepTwoLevelMaxChunks) {
        p.waves = 4;
        const int64_t c_min = (int64_t)kSplitMinTiles * kTileTokens * 4;
        if (p.chunk < c_min && c_min <= kMaxChunkTokens &&
            p.units * ceil_div(cap, c_min) >= kMinSplitBlocks) {
          p.chunk = (int)c_min;
          p.nchunks = (int)ceil_div(cap, c_min);
        }
      }
    }
  }

  const int64_t blocks = p.units * p.nchunks;
  if (blocks > INT32_MAX || p.units > INT32_MAX ||
      (int64_t)d->num_shards * d->batch * d->num_q_heads > INT32_MAX)
    return CPDEC_ERR_INVALID_ARG;

  // Workspace: the whole step's arrival counters first (at a fixed offset, so
  // calls of any shape that share a workspace never overwrite them), then the
  // chunk partials.
  const size_t slots = (size_t)p.units * p.nchunks * p.Gb;
  if (p.nchunks > 1) {
    p.off_lse = kStepCounterBytes;
    p.off_o = p.off_lse + round256(slots * sizeof(float));
    p.ws_bytes = p.off_o + slots * (size_t)D * sizeof(float);
  }
  p.step_ws_bytes = p.ws_bytes > kStepCounterBytes ? p.ws_bytes : kStepCounterBytes;

  // The whole step in one launch when the counters, the merging workgroup's
  // LDS and 32-bit buffer offsets allow it.
  const int64_t groups = (int64_t)d->batch * d->num_kv_heads * p.gblocks;
  const uint64_t opart_bytes = (uint64_t)d->num_shards * d->batch * d->num_q_heads * D *
                               (d->opart_dtype == CPDEC_F32 ? 4u : 2u);
  const int64_t threads = 64 * p.waves;
  const int64_t R = d->num_shards;
  bool one = !overrides().step_launches && groups <= kStepCounters && opart_bytes < (1ull << 31);
  if (p.nchunks > 1) {
    const int64_t items = R * p.Gb * (D / 4);
    one = one && items <= threads && items <= kStepVecs && R * p.Gb <= threads &&
          p.nchunks <= kStepMaxChunks && R * p.nchunks * p.Gb <= kStepSlots &&
          slots * (size_t)D * sizeof(float) < (1ull << 31);
  } else {  // large unsplit grids: a merge launch costs less than write-through o_part stores
    one = one && p.units <= kStepUnsplitBlocks && R <= kStepMaxShardsUnsplit &&
          (int64_t)p.Gb * (D / 4) <= threads;
  }
  // Split groups too big for one merging workgroup: two levels in the same
  // launch (chunk combine per unit, then the shard merge per group), with one
  // counter line per unit and one per group, when each level's output vectors
  // (min(G,16) x D/4) fit the workgroup's threads -- with a second pass per
  // level the separate launches measured faster (GQA 8 at D=128: 57 vs 54 us).
  const bool two = !one && p.nchunks > 1 && !overrides().step_launches &&
                   p.units + groups <= kStepCounters && p.nchunks <= kStepTwoLevelMaxChunks &&
                   (int64_t)p.Gb * (D / 4) <= threads && opart_bytes < (1ull << 31) &&
                   slots * (size_t)D * sizeof(float) < (1ull << 31);
  p.step = one ? (p.nchunks > 1 ? kStepOneChunks : kStepOneShards)
               : (two ? kStepTwoLevel : kStepLaunches);

  // cpdec_attn_partial with split shards: the unit's last chunk workgroup
  // combines the chunks in the attention launch (one counter line per unit).
  p.partials_combine = p.nchunks > 1 && !overrides().step_launches && p.units <= kStepCounters &&
                       p.nchunks <= kStepTwoLevelMaxChunks && opart_bytes < (1ull << 31) &&
                       slots * (size_t)D * sizeof(float) < (1ull << 31);

  // Longest-first launch order for large grids of unsplit shards when the
  // library picks the schedule: the order entries follow the counter region.
  // (Such grids never take the one-launch step: kOrderMinUnits > kStepUnsplitBlocks.)
  const double kv_cap_bytes =
      (double)R * d->batch * d->num_kv_heads * (double)cap * D * 2.0 * 2.0;  // K and V, 16-bit
  p.ordered = d->chunk_tokens == 0 && !overrides().no_order && p.nchunks == 1 &&
              p.units >= kOrderMinUnits && R * d->batch <= kOrderMaxPairs &&
              kv_cap_bytes >= kOrderMinKvBytes;
  if (p.ordered) {
    p.off_order = kStepCounterBytes;
    p.ws_bytes = p.off_order + (size_t)R * d->batch * sizeof(OrderEntry);
    p.step_ws_bytes = p.ws_bytes;
  }
  *pl = p;
  return CPDEC_OK;
}

size_t dtype_size(int dt) { return dt == CPDEC_F32 ? 4 : 2; }

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream), looked up once per device with that
// device current and kept.  The first lookup on a device also clears the
// arrival counters at the start of the scratch on `stream`, ahead of the
// kernels that use them; every completed call leaves them zero.
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kScratchDevices] = {};

cpdec_status scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return CPDEC_ERR_HIP;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return CPDEC_ERR_HIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kScratchDevices) return CPDEC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return CPDEC_ERR_HIP;
    void* ptr = nullptr;
    const bool found = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr != nullptr;
    const bool cleared = found && launch_clear(ptr, kStepCounterBytes, stream) == hipSuccess;
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return CPDEC_ERR_HIP;
    if (!cleared) return CPDEC_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return CPDEC_OK;
}

}  // namespace

extern "C" {

size_t cpdec_attn_workspace_bytes(const cpdec_attn_desc* d) {
  AttnPlan pl;
  if (plan_attn(d, &pl) != CPDEC_OK) return 0;
  return pl.ws_bytes;
}

size_t cpdec_step_workspace_bytes(const cpdec_attn_desc* d) {
  AttnPlan pl;
  if (plan_attn(d, &pl) != CPDEC_OK) return 0;
  return pl.step_ws_bytes;
}

cpdec_status cpdec_step_plan(const cpdec_attn_desc* d, int32_t* launches) {
  AttnPlan pl;
  const cpdec_status st = plan_attn(d, &pl);
  if (st != CPDEC_OK) return st;
  if (launches) {
    int n = 1;
    if (pl.step == kStepLaunches) {
      const int64_t ws_o_bytes = pl.units * pl.nchunks * pl.Gb * (int64_t)d->head_dim * 4;
      const int64_t opart_bytes = (int64_t)d->num_shards * d->batch * d->num_q_heads *
                                  d->head_dim * (d->opart_dtype == CPDEC_F32 ? 4 : 2);
      const bool row = row_merge_waves(d->num_shards, pl.nchunks, d->head_dim, ws_o_bytes,
                                       opart_bytes) > 0;
      n = (pl.nchunks > 1 && !row ? 3 : 2) + (pl.ordered ? 1 : 0);
    }
    *launches = n;
  }
  return CPDEC_OK;
}

cpdec_status cpdec_attn_launches(const cpdec_attn_desc* d, int32_t* launches) {
  AttnPlan pl;
  const cpdec_status st = plan_attn(d, &pl);
  if (st != CPDEC_OK) return st;
  if (launches)
    *launches = 1 + (pl.ordered ? 1 : 0) + (pl.nchunks > 1 && !pl.partials_combine ? 1 : 0);
  return CPDEC_OK;
}

cpdec_status cpdec_attn_order(const cpdec_attn_desc* d, int32_t* longest_first) {
  AttnPlan pl;
  const cpdec_status st = plan_attn(d, &pl);
  if (st != CPDEC_OK) return st;
  if (longest_first) *longest_first = pl.ordered ? 1 : 0;
  return CPDEC_OK;
}

cpdec_status cpdec_attn_plan(const cpdec_attn_desc* d, int32_t* chunk_tokens, int32_t* num_chunks,
                             int32_t* waves) {
  AttnPlan pl;
  const cpdec_status st = plan_attn(d, &pl);
  if (st != CPDEC_OK) return st;
  if (chunk_tokens) *chunk_tokens = pl.chunk;
  if (num_chunks) *num_chunks = pl.nchunks;
  if (waves) *waves = pl.waves;
  return CPDEC_OK;
}

struct StepOut {
  void* out;
  float* lse_out;
  int out_dt;
};

static cpdec_status attn_launch(const cpdec_attn_desc* d, const void* q,
                                const void* const* k_shards, const void* const* v_shards,
                                const int32_t* lens, void* o_part, float* lse_part,
                                void* workspace, size_t workspace_bytes, const StepOut* so,
                                void* stream, bool use_scratch = false);

cpdec_status cpdec_attn_partial(const cpdec_attn_desc* d, const void* q,
                                const void* const* k_shards, const void* const* v_shards,
                                const int32_t* lens, void* o_part, float* lse_part,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return attn_launch(d, q, k_shards, v_shards, lens, o_part, lse_part, workspace,
                     workspace_bytes, nullptr, stream);
}

cpdec_status cpdec_cp_decode(const cpdec_attn_desc* d, const void* q,
                             const void* const* k_shards, const void* const* v_shards,
                             const int32_t* lens, void* o_part, float* lse_part, void* out,
                             float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (out == nullptr) return CPDEC_ERR_INVALID_ARG;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(lse_out) & 3u)) return CPDEC_ERR_ALIGNMENT;
  StepOut so{out, lse_out, d != nullptr ? (int)d->qkv_dtype : 0};
  return attn_launch(d, q, k_shards, v_shards, lens, o_part, lse_part, workspace,
                     workspace_bytes, &so, stream);
}

cpdec_status cpdec_cp_decode_noalloc(const cpdec_attn_desc* d, const void* q,
                                     const void* const* k_shards, const void* const* v_shards,
                                     const int32_t* lens, void* o_part, float* lse_part,
                                     void* out, float* lse_out, void* stream) {
  if (out == nullptr) return CPDEC_ERR_INVALID_ARG;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(lse_out) & 3u)) return CPDEC_ERR_ALIGNMENT;
  StepOut so{out, lse_out, d != nullptr ? (int)d->qkv_dtype : 0};
  return attn_launch(d, q, k_shards, v_shards, lens, o_part, lse_part, nullptr, 0, &so, stream,
                     true);
}

static cpdec_status attn_launch(const cpdec_attn_desc* d, const void* q,
                                const void* const* k_shards, const void* const* v_shards,
                                const int32_t* lens, void* o_part, float* lse_part,
                                void* workspace, size_t workspace_bytes, const StepOut* so,
                                void* stream, bool use_scratch) {
  AttnPlan pl;
  cpdec_status st = plan_attn(d, &pl);
  if (st != CPDEC_OK) return st;
  if (q == nullptr || k_shards == nullptr || v_shards == nullptr || lens == nullptr ||
      o_part == nullptr || lse_part == nullptr)
    return CPDEC_ERR_INVALID_ARG;
  for (int r = 0; r < d->num_shards; ++r)
    if (k_shards[r] == nullptr || v_shards[r] == nullptr) return CPDEC_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u) ||
      (reinterpret_cast<uintptr_t>(lens) & 3u))
    return CPDEC_ERR_ALIGNMENT;
  for (int r = 0; r < d->num_shards; ++r)
    if (!aligned16(k_shards[r]) || !aligned16(v_shards[r])) return CPDEC_ERR_ALIGNMENT;
  // The separate-launch step runs the merge kernel, which addresses each
  // shard's o_part rows and the lse array with 32-bit offsets.
  if (so != nullptr && pl.step == kStepLaunches) {
    const uint64_t rows = (uint64_t)d->batch * d->num_q_heads;
    if (rows * (uint64_t)d->head_dim * dtype_size(d->opart_dtype) >= (1ull << 31) ||
        rows * (uint64_t)d->num_shards * 4 >= (1ull << 31))
      return CPDEC_ERR_UNSUPPORTED;
  }
  const size_t need = so != nullptr ? pl.step_ws_bytes : pl.ws_bytes;
  if (use_scratch) {
    // the library's own scratch: every check above ran without a HIP call
    if (need > CPDEC_NOALLOC_SCRATCH_BYTES) return CPDEC_ERR_WORKSPACE;
    const cpdec_status sst = scratch_for_stream(static_cast<hipStream_t>(stream), &workspace);
    if (sst != CPDEC_OK) return sst;
    workspace_bytes = CPDEC_NOALLOC_SCRATCH_BYTES;
  } else if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return CPDEC_ERR_WORKSPACE;
  }

  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  for (int r = 0; r < d->num_shards; ++r) {
    p.k[r] = k_shards[r];
    p.v[r] = v_shards[r];
  }
  p.lens = lens;
  p.o_part = o_part;
  p.lse_part = lse_part;
  if (pl.nchunks > 1) {
    char* ws = static_cast<char*>(workspace);
    p.ws_lse = reinterpret_cast<float*>(ws + pl.off_lse);
    p.ws_o = reinterpret_cast<float*>(ws + pl.off_o);
  }
  if (pl.ordered) p.order = static_cast<char*>(workspace) + pl.off_order;
  StepMode mode = kPartialsOnly;
  if (so == nullptr && pl.partials_combine) {
    mode = kPartialsCombine;
    p.counters = static_cast<int32_t*>(workspace);
  }
  if (so != nullptr) {
    mode = pl.step;
    p.out = so->out;
    p.lse_out = so->lse_out;
    p.out_dt = so->out_dt;
    p.counters = static_cast<int32_t*>(workspace);
  }
  p.sb = d->kv_stride_batch;
  p.sh = d->kv_stride_head;
  p.st = d->kv_stride_token;
  p.B = d->batch;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.G = pl.G;
  p.Gb = pl.Gb;
  p.gblocks = pl.gblocks;
  p.R = d->num_shards;
  p.chunk = pl.chunk;
  p.nchunks = pl.nchunks;
  p.units = (int32_t)pl.units;
  p.cap = d->kv_capacity;
  p.odt = d->opart_dtype;
  const double scale = d->sm_scale > 0.f ? (double)d->sm_scale : 1.0 / sqrt((double)d->head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634);

  hipError_t e = launch_attn_partial(p, d->qkv_dtype, d->head_dim, pl.waves, pl.units, mode,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CPDEC_OK : CPDEC_ERR_HIP;
}

cpdec_status cpdec_lse_merge(const void* o_part, const float* lse_part, int32_t num_shards,
                             int64_t rows, int32_t head_dim, cpdec_dtype in_dtype,
                             cpdec_dtype out_dtype, void* out, float* lse_out, void* stream) {
  if (o_part == nullptr || lse_part == nullptr || out == nullptr) return CPDEC_ERR_INVALID_ARG;
  if (num_shards < 1 || num_shards > CPDEC_MAX_SHARDS || rows < 0) return CPDEC_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return CPDEC_ERR_UNSUPPORTED;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return CPDEC_ERR_UNSUPPORTED;
  if (!aligned16(o_part) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lse_part) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_out) & 3u))
    return CPDEC_ERR_ALIGNMENT;
  // Element counts must stay addressable and the grid within 2^31 blocks.
  if (rows > 0 && (uint64_t)rows * (uint64_t)num_shards > (uint64_t)INT64_MAX / 4096)
    return CPDEC_ERR_INVALID_ARG;
  // Each shard's partial rows, and the lse array, are addressed with 32-bit offsets.
  {
    const uint64_t esz = in_dtype == CPDEC_F32 ? 4 : 2;
    if ((uint64_t)rows * (uint64_t)head_dim * esz >= (1ull << 31) ||
        (uint64_t)rows * (uint64_t)num_shards * 4 >= (1ull << 31))
      return CPDEC_ERR_UNSUPPORTED;
  }
  if (lse_merge_max_blocks(rows, head_dim, in_dtype) > INT32_MAX) return CPDEC_ERR_INVALID_ARG;
  (void)dtype_size;
  if (rows == 0) return CPDEC_OK;
  hipError_t e = launch_lse_merge(o_part, lse_part, num_shards, rows, head_dim, in_dtype,
                                  out_dtype, out, lse_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CPDEC_OK : CPDEC_ERR_HIP;
}

cpdec_status cpdec_workspace_clear(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return CPDEC_OK;
  if (workspace == nullptr) return CPDEC_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return CPDEC_ERR_ALIGNMENT;
  hipError_t e = launch_clear(workspace, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CPDEC_OK : CPDEC_ERR_HIP;
}

const char* cpdec_status_string(cpdec_status s) {
  switch (s) {
    case CPDEC_OK: return "CPDEC_OK";
    case CPDEC_ERR_INVALID_ARG: return "CPDEC_ERR_INVALID_ARG";
    case CPDEC_ERR_UNSUPPORTED: return "CPDEC_ERR_UNSUPPORTED";
    case CPDEC_ERR_ALIGNMENT: return "CPDEC_ERR_ALIGNMENT";
    case CPDEC_ERR_WORKSPACE: return "CPDEC_ERR_WORKSPACE";
    case CPDEC_ERR_HIP: return "CPDEC_ERR_HIP";
  }
  return "CPDEC_ERR_UNKNOWN";
}

const char* cpdec_version(void) { return "cpdec 0.1.0 gfx950"; }

}  // extern "C"
