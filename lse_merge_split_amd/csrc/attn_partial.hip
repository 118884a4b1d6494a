// attn_partial.hip -- split-KV decode attention per KV shard (gfx950).
//
// Method: page "FlashInfer's Context-Parallel Decode optimisation: Fused A2A
// + LSE Reduce" (flashinfer PR #4929), section "Introduction": every KV shard
// r of a sequence gets decode attention over its local tokens, giving a
// partial output o_r and lse_r for the later LSE merge.
//
// Work decomposition
//   unit  = (shard r, sequence b, kv head h, block of <= 16 query heads of h)
//   chunk = `chunk` consecutive tokens of a unit; one workgroup per
//           (unit, chunk) in chunk-major order, chunks at or past L exit at
//           once.
//   A workgroup has NW waves; wave w takes the 32-token tiles w, w+NW, ... of
//   its chunk and keeps an online-softmax state (running max m, exp-sum l,
//   un-normalised accumulator) per query head, loading tile i+1 while it
//   computes tile i (split shards: the first two tiles are requested before
//   the length is known).  The waves' states are merged through LDS.  A unit
//   whose tokens fit one chunk is written straight to o_part/lse_part;
//   otherwise each chunk writes a normalised partial to the workspace.  Every
//   merge -- chunks of a shard, shards of a sequence -- uses the LSE weighting
//   of the page's merge formula, which makes it exact.  Large ragged grids of
//   unsplit shards may take their units longest first (order_kernel).
//
// Who merges:
//   * partials only (cpdec_attn_partial): a second, small kernel merges the
//     chunks of every unit.
//   * the whole step in one launch (cpdec_cp_decode): workgroups hand their
//     results over with device-scope stores and an arrival counter per
//     (sequence, kv head, head block); the workgroup that arrives last merges
//     that group's chunks and shards -- or, for split groups too big for one
//     workgroup, in two levels: the last chunk of a unit combines the unit's
//     chunks, the last unit of the group merges the shards.  No workgroup
//     ever waits for another, and no device-scope fence is used: on gfx950
//     such a fence writes back and invalidates the XCD's L2, which costs
//     microseconds per workgroup.
//   * the whole step as separate launches (groups beyond the one-launch
//     limits): the attention, then one workgroup per (sequence, query head)
//     combines and merges (row_merge_kernel), or the chunk-combine kernel and
//     the merge kernel.
//
// Per 32-token tile, with G <= 16 query heads of one kv head as MFMA columns:
//   S^T[t][g] = K[t][:] . Q[g][:]       4 (D/32) MFMA 16x16x32 per 16 tokens;
//                                       K rows are loaded straight into the A
//                                       operand (lane = token row, 8 contiguous
//                                       d per lane), no LDS.
//   online softmax in base 2 on the S^T accumulator layout: each lane holds
//   8 tokens of one head g, so the max/sum need only a 4-lane (xor 16, 32)
//   exchange.
//   O^T[d][g] += V^T[d][t] . P^T[t][g]  8 MFMA per 16-row block of d; the P
//                                       operand is exactly the lane's own 8
//                                       probabilities (token order within the
//                                       tile is permuted consistently for P and
//                                       V), and V^T comes from an in-register
//                                       8x8 transpose of 16-byte row loads
//                                       (one v_perm_b32 per dword).
//   P is fed to the MFMA as hi + lo 16-bit parts (two MFMAs), keeping its
//   relative error near 2^-16 instead of 2^-8 at negligible MFMA cost.
//
// Roofline: reading K and V once (2*D*2 bytes per token per kv head) is the
// bound; the GQA group shares every K/V byte across its G heads.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace cpdec {
namespace {

// Token of the 32-token tile that lane quarter q4 owns in P/V slot j: slots
// 0..3 are tokens 4*q4 + j of the first 16-token block, slots 4..7 the same
// positions of the second block (matching the S^T accumulator layout).
__device__ __forceinline__ int tile_token(int q4, int j) {
  return (j < 4) ? 4 * q4 + j : 16 + 4 * q4 + (j - 4);
}

// Store 32 consecutive fp32 values starting at element `idx` of a row-major
// output of dtype `odt`.
__device__ __forceinline__ void store32(void* base, int64_t idx, const float* x, int odt) {
  if (odt == kF32) {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
  } else if (odt == kBF16) {
    u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = u32x4{pack2<bf16_t>(x[8 * i], x[8 * i + 1]), pack2<bf16_t>(x[8 * i + 2], x[8 * i + 3]),
                   pack2<bf16_t>(x[8 * i + 4], x[8 * i + 5]), pack2<bf16_t>(x[8 * i + 6], x[8 * i + 7])};
  } else {
    u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = u32x4{pack2<f16_t>(x[8 * i], x[8 * i + 1]), pack2<f16_t>(x[8 * i + 2], x[8 * i + 3]),
                   pack2<f16_t>(x[8 * i + 4], x[8 * i + 5]), pack2<f16_t>(x[8 * i + 6], x[8 * i + 7])};
  }
}

// Store 4 consecutive fp32 values.
__device__ __forceinline__ void store4(void* base, int64_t idx, f32x4 x, int odt) {
  if (odt == kF32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = x;
  } else if (odt == kBF16) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) =
        u32x2{pack2<bf16_t>(x[0], x[1]), pack2<bf16_t>(x[2], x[3])};
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) =
        u32x2{pack2<f16_t>(x[0], x[1]), pack2<f16_t>(x[2], x[3])};
  }
}

template <int D, int NW>
struct Smem {
  static constexpr int NB = (D / 8 + 15) / 16;
  f32x4 acc[NW > 1 ? NW - 1 : 1][NB * 8][64];
  float m[NW][16];
  float l[NW][16];
};

// LDS of the workgroup that merges a group in a one-launch step (shares the
// attention's LDS: it is used only after the workgroup's own chunk is done).
template <int NW, int MODE>
struct MergeSmem {
  static constexpr bool kChunks =
      MODE == kStepOneChunks || MODE == kStepTwoLevel || MODE == kPartialsCombine;
  float w[kChunks ? kStepSlots : 1];    // chunk weights, [(r * ng + g) * nchunks + c]
  f32x4 y[kChunks ? kStepVecs : 1];     // shard partials as stored, [r * E + e]
  f32x4 part[kChunks ? NW * 64 : 1];    // partition sums
  float lse[kMaxShards * kGroupRows];   // shard lse, [r * ng + g]
  double ew[kMaxShards * kGroupRows];   // cross-shard weights e^(lse - M), [r * ng + g]
  float M[kGroupRows];                  // max shard lse per head
};

template <typename T, int D, int NW, int MODE>
union KernelSmem {
  Smem<D, NW> a;
  MergeSmem<NW, MODE> m;
};

// 32 consecutive fp32 values, converted to dtype `odt`, written with
// device-scope stores at byte offset `off` of resource `r`.
__device__ __forceinline__ void store32_dev(rsrc_t r, uint32_t off, const float* x, int odt) {
  if (odt == kF32) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st16_dev(r, off + 16u * i,
               __builtin_bit_cast(u32x4, f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]}));
  } else if (odt == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st16_dev(r, off + 16u * i,
               u32x4{pack2<bf16_t>(x[8 * i], x[8 * i + 1]), pack2<bf16_t>(x[8 * i + 2], x[8 * i + 3]),
                     pack2<bf16_t>(x[8 * i + 4], x[8 * i + 5]), pack2<bf16_t>(x[8 * i + 6], x[8 * i + 7])});
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st16_dev(r, off + 16u * i,
               u32x4{pack2<f16_t>(x[8 * i], x[8 * i + 1]), pack2<f16_t>(x[8 * i + 2], x[8 * i + 3]),
                     pack2<f16_t>(x[8 * i + 4], x[8 * i + 5]), pack2<f16_t>(x[8 * i + 6], x[8 * i + 7])});
  }
}

// 4 consecutive values of dtype `odt` at byte offset `off`, device-scope load.
__device__ __forceinline__ f32x4 load4_dev(rsrc_t r, uint32_t off, int odt) {
  if (odt == kF32) return __builtin_bit_cast(f32x4, ld16_dev(r, off));
  const u32x2 w = ld8_dev(r, off);
  if (odt == kBF16) return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  return f32x4{f16_lo(w[0]), f16_hi(w[0]), f16_lo(w[1]), f16_hi(w[1])};
}

// load4_dev in two halves with no branch between the load and the loads
// issued before it: both widths are requested, the one `odt` does not use at
// an out-of-range offset (no memory traffic), and raw4_f32 converts where the
// value is used.  (A branch around a load makes the compiler wait for every
// outstanding load where the paths join.)
struct Raw4 {
  u32x4 w4;
  u32x2 w2;
};
__device__ __forceinline__ Raw4 load4_dev_raw(rsrc_t r, uint32_t off, int odt) {
  const bool f32 = odt == kF32;
  return Raw4{ld16_dev(r, f32 ? off : kOutOfRange), ld8_dev(r, f32 ? kOutOfRange : off)};
}
__device__ __forceinline__ f32x4 raw4_f32(const Raw4& x, int odt) {
  if (odt == kF32) return __builtin_bit_cast(f32x4, x.w4);
  if (odt == kBF16) return f32x4{bf16_lo(x.w2[0]), bf16_hi(x.w2[0]), bf16_lo(x.w2[1]), bf16_hi(x.w2[1])};
  return f32x4{f16_lo(x.w2[0]), f16_hi(x.w2[0]), f16_lo(x.w2[1]), f16_hi(x.w2[1])};
}

// The values x takes once stored as dtype `odt`.
__device__ __forceinline__ f32x4 round4(f32x4 x, int odt) {
  if (odt == kBF16) {
    const uint32_t a = pack2<bf16_t>(x[0], x[1]), b = pack2<bf16_t>(x[2], x[3]);
    return f32x4{bf16_lo(a), bf16_hi(a), bf16_lo(b), bf16_hi(b)};
  }
  if (odt == kF16) {
    const uint32_t a = pack2<f16_t>(x[0], x[1]), b = pack2<f16_t>(x[2], x[3]);
    return f32x4{f16_lo(a), f16_hi(a), f16_lo(b), f16_hi(b)};
  }
  return x;
}

__device__ __forceinline__ uint32_t esize(int dt) { return dt == kF32 ? 4u : 2u; }

// Scalar launch parameters, read once at kernel start.  Each value passes
// through an empty asm statement that makes it opaque to the compiler, so it
// stays in a register (or a VGPR lane when registers run short) instead of
// being fetched again from the kernel arguments later: the argument buffer is
// not cached, and each such re-fetch would cost a memory round trip in the
// latency-bound tail of a workgroup (its stores, the arrival, the merge).
struct Args {
  const void* q;
  const int32_t* lens;
  void* o_part;
  float* lse_part;
  float* ws_o;
  float* ws_lse;
  void* out;
  float* lse_out;
  int32_t* counters;
  int64_t sb, sh, st;
  int32_t B, Hq, Hkv, G, Gb, gblocks, R, chunk, nchunks, units, odt, out_dt, cap;
  float scale_log2;
  const void* order;  // longest-first launch order (ordered kernels only, else null)
};

// (readfirstlane afterwards: the compiler takes an asm result for a per-lane
// value, and a buffer resource built from one would need a waterfall loop.)
// All fields pass through ONE asm statement, so every argument load is issued
// before the first wait (one memory round trip instead of one per field).
__device__ __forceinline__ uint32_t rfl(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename V>
__device__ __forceinline__ V rfl_v(V x) {
  if constexpr (sizeof(V) == 4) {
    return __builtin_bit_cast(V, rfl(__builtin_bit_cast(uint32_t, x)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    return __builtin_bit_cast(V, (uint64_t)rfl((uint32_t)u) | ((uint64_t)rfl((uint32_t)(u >> 32)) << 32));
  }
}

template <bool ORDERED = false>
__device__ __forceinline__ Args load_args(const AttnParams& p, const void*& kshard,
                                          const void*& vshard) {
  Args a;
  a.order = nullptr;
  a.q = p.q; a.lens = p.lens; a.o_part = p.o_part; a.lse_part = p.lse_part; a.ws_o = p.ws_o;
  a.ws_lse = p.ws_lse; a.out = p.out; a.lse_out = p.lse_out; a.counters = p.counters;
  a.sb = p.sb; a.sh = p.sh; a.st = p.st;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.Gb = p.Gb; a.gblocks = p.gblocks; a.R = p.R;
  a.chunk = p.chunk; a.nchunks = p.nchunks; a.units = p.units; a.odt = p.odt; a.out_dt = p.out_dt;
  a.cap = p.cap; a.scale_log2 = p.scale_log2;
  if constexpr (ORDERED) {  // the shard pointers come from the order entry instead
    // (unsplit partials only: no workspace partials, no merge outputs, no counters)
    a.order = p.order;
    a.ws_o = nullptr;
    a.ws_lse = nullptr;
    a.out = nullptr;
    a.lse_out = nullptr;
    a.counters = nullptr;
    a.out_dt = 0;
    kshard = nullptr;
    vshard = nullptr;
    asm volatile(""
                 : "+s"(a.q), "+s"(a.lens), "+s"(a.o_part), "+s"(a.lse_part), "+s"(a.order),
                   "+s"(a.sb), "+s"(a.sh), "+s"(a.st), "+s"(a.B), "+s"(a.Hq), "+s"(a.Hkv),
                   "+s"(a.G), "+s"(a.Gb), "+s"(a.gblocks), "+s"(a.R), "+s"(a.chunk),
                   "+s"(a.nchunks), "+s"(a.units), "+s"(a.odt), "+s"(a.cap), "+s"(a.scale_log2));
    a.q = rfl_v(a.q); a.lens = rfl_v(a.lens); a.o_part = rfl_v(a.o_part);
    a.lse_part = rfl_v(a.lse_part); a.order = rfl_v(a.order);
    a.sb = rfl_v(a.sb); a.sh = rfl_v(a.sh); a.st = rfl_v(a.st);
    a.B = rfl_v(a.B); a.Hq = rfl_v(a.Hq); a.Hkv = rfl_v(a.Hkv); a.G = rfl_v(a.G); a.Gb = rfl_v(a.Gb);
    a.gblocks = rfl_v(a.gblocks); a.R = rfl_v(a.R); a.chunk = rfl_v(a.chunk);
    a.nchunks = rfl_v(a.nchunks); a.units = rfl_v(a.units); a.odt = rfl_v(a.odt);
    a.cap = rfl_v(a.cap); a.scale_log2 = rfl_v(a.scale_log2);
    return a;
  }
  kshard = p.k[blockIdx.y];
  vshard = p.v[blockIdx.y];
  asm volatile(""
               : "+s"(a.q), "+s"(a.lens), "+s"(a.o_part), "+s"(a.lse_part), "+s"(a.ws_o),
                 "+s"(a.ws_lse), "+s"(a.out), "+s"(a.lse_out), "+s"(a.counters), "+s"(a.sb),
                 "+s"(a.sh), "+s"(a.st), "+s"(kshard), "+s"(vshard), "+s"(a.B), "+s"(a.Hq),
                 "+s"(a.Hkv), "+s"(a.G), "+s"(a.Gb), "+s"(a.gblocks), "+s"(a.R), "+s"(a.chunk),
                 "+s"(a.nchunks), "+s"(a.units), "+s"(a.odt), "+s"(a.out_dt), "+s"(a.cap),
                 "+s"(a.scale_log2));
  a.q = rfl_v(a.q); a.lens = rfl_v(a.lens); a.o_part = rfl_v(a.o_part);
  a.lse_part = rfl_v(a.lse_part); a.ws_o = rfl_v(a.ws_o); a.ws_lse = rfl_v(a.ws_lse);
  a.out = rfl_v(a.out); a.lse_out = rfl_v(a.lse_out); a.counters = rfl_v(a.counters);
  a.sb = rfl_v(a.sb); a.sh = rfl_v(a.sh); a.st = rfl_v(a.st);
  kshard = rfl_v(kshard); vshard = rfl_v(vshard);
  a.B = rfl_v(a.B); a.Hq = rfl_v(a.Hq); a.Hkv = rfl_v(a.Hkv); a.G = rfl_v(a.G); a.Gb = rfl_v(a.Gb);
  a.gblocks = rfl_v(a.gblocks); a.R = rfl_v(a.R); a.chunk = rfl_v(a.chunk);
  a.nchunks = rfl_v(a.nchunks); a.units = rfl_v(a.units); a.odt = rfl_v(a.odt);
  a.out_dt = rfl_v(a.out_dt); a.cap = rfl_v(a.cap); a.scale_log2 = rfl_v(a.scale_log2);
  return a;
}

// Attention of one workgroup over chunk c of `unit` (t_begin < L): the
// normalised chunk result goes to o_part/lse_part when the unit has one live
// chunk, else to the workspace.  In the one-launch step modes these stores are
// device-scope, for the workgroup that merges the group.
template <typename T, int D, int NW, int MODE, bool SPEC2>
__device__ __forceinline__ bool attend_chunk(const Args& p, const void* kshard, const void* vshard,
                                             Smem<D, NW>& sm, int c, int unit, int r, int b, int h,
                                             int gb, int len_raw, int& len_t) {
  constexpr int NCH = D / 8;           // 16-byte chunks per token row
  constexpr int NB = (NCH + 15) / 16;  // 16-chunk row blocks of the PV product
  constexpr int KS = D / 32;           // k-steps of the QK product
  constexpr bool kDev = MODE >= kStepOneShards;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  const int t_begin = c * p.chunk;
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int hq0 = h * p.G + g0;
  const int64_t orow0 = ((int64_t)r * p.B + b) * p.Hq + hq0;  // o_part/lse_part row of head g0

  // Q operand (B of S^T = K Q^T): lane (q4, g = l16) holds Q[g][32 s + 8 q4 .. +8].
  u32x4 qop[KS];
  {
    const rsrc_t qrs = make_rsrc(static_cast<const T*>(p.q) + ((int64_t)b * p.Hq + hq0) * D,
                                 (uint32_t)(ng * D * sizeof(T)));  // the group's heads
    const uint32_t qoff = (uint32_t)((l16 * D + 8 * q4) * sizeof(T));
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[s] = buf16(qrs, l16 < ng ? qoff + 64u * s : kOutOfRange);
  }

  const T* kb = static_cast<const T*>(kshard) + b * p.sb + h * p.sh;
  const T* vb = static_cast<const T*>(vshard) + b * p.sb + h * p.sh;
  const int64_t st = p.st;

  float m = neg_inf();  // running max (base-2 units), uniform over q4
  // This lane's share of the exp-sum, accumulated in FP64: after a dominant
  // token the running sum sits near 1 while each tile adds a nearly constant
  // small term, and FP32 round-to-nearest would then drop the same fraction of
  // every term (an lse bias growing with the chunk length).
  double lsum_d = 0.0;
  f32x4 acc[NB][8];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[nb][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K rows go straight into the A operand (lane = token row l16, 8 contiguous
  // d per k-step); V rows are loaded for the in-register transpose.
  // K/V of this unit through buffer resources ending at the chunk's last
  // token: rows past it read as zeros without memory traffic, so the tail and
  // the prefetch beyond the end need neither clamping nor a branch (a branch
  // around loads makes the compiler drain every outstanding load at the join).
  // The wave's first tile is requested before the length is known, through a
  // resource that ends at the chunk's end within the capacity; a tile that
  // crosses the end zeroes its V rows past it before they are used.
  const uint32_t rowb = (uint32_t)(st * sizeof(T));  // bytes per token row
  auto rows_span = [&](int rows) {
    return rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * st + D) * sizeof(T)) : 0u;
  };
  auto load_tile = [&](int t0, rsrc_t krs, rsrc_t vrs, u32x4 (&kr)[2][KS], u32x4 (&vr)[NB][8]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint32_t off = (uint32_t)(t0 + 16 * blk + l16) * rowb + 16u * q4;
#pragma unroll
      for (int s = 0; s < KS; ++s) kr[blk][s] = buf16_stream(krs, off + 64u * s);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = (uint32_t)(t0 + tile_token(q4, j)) * rowb;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int ch = 16 * nb + l16;
        vr[nb][j] = buf16_stream(vrs, (ch < NCH) ? off + 16u * ch : kOutOfRange);
      }
    }
  };

  // Tile registers: kt0/vt0 hold the tile being computed; kt1/vt1 are the prefetch
  // buffer (one tile ahead), or with SPEC2 the second slot of a two-tile ring.
  u32x4 kt0[2][KS], vt0[NB][8], kt1[2][KS], vt1[NB][8];
  int t0 = t_begin + wave * kTileTokens;
  {
    const uint32_t span0 = rows_span(min(p.cap, t_begin + p.chunk));
    const rsrc_t k0 = make_rsrc(kb, span0), v0 = make_rsrc(vb, span0);
    load_tile(t0, k0, v0, kt0, vt0);
    // SPEC2 (split shards with two or more tiles per wave): the second tile too
    // is requested before the length is known, one memory round trip earlier.
    if constexpr (SPEC2) load_tile(t0 + NW * kTileTokens, k0, v0, kt1, vt1);
  }
  if constexpr (kDev) {  // every shard's length of this sequence, for the merge (used at the end)
    const rsrc_t lens_rs = make_rsrc(p.lens, (uint32_t)(p.R * p.B * 4));
    len_t = (int)__builtin_amdgcn_raw_buffer_load_b32(
        lens_rs, threadIdx.x < (unsigned)p.R ? (int)((threadIdx.x * p.B + b) * 4) : (int)kOutOfRange, 0,
        0);
  }
  // lengths outside [0, cap] are taken as the nearest bound (reads stay inside the shard)
  const int L = min(max(__builtin_amdgcn_readfirstlane(len_raw), 0), p.cap);
  const int t_end = min(L, t_begin + p.chunk);  // <= t_begin for an empty chunk
  const int nlive = (L + p.chunk - 1) / p.chunk;
  const uint32_t span = rows_span(t_end);
  const rsrc_t krs = make_rsrc(kb, span);
  const rsrc_t vrs = make_rsrc(vb, span);

  // One tile at t0: scores, online softmax, p.V into the accumulators.
  auto tile_step = [&](u32x4 (&kr)[2][KS], u32x4 (&vr)[NB][8]) {
      // ---- scores S^T (16 tokens x 16 heads per block), base-2 scaled, masked ----
      float x[2][4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc = mfma16x16x32<T>(kr[blk][s], qop[s], sacc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * blk + 4 * q4 + i;
          x[blk][i] = (t < t_end) ? sacc[i] * p.scale_log2 : neg_inf();
        }
      }

      // ---- online softmax for head g = l16 ----
      float mt = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      {  // over the 4 lane rows (q4) holding head g's tokens
        const f32x2 a = rows16(mt);
        mt = fmaxf(a[0], a[1]);
        const f32x2 c = rows32(mt);
        mt = fmaxf(c[0], c[1]);
      }
      const float m_new = fmaxf(m, mt);  // -inf only while every token so far was masked
      const float m_ref = m_new == neg_inf() ? 0.f : m_new;  // keeps -inf - -inf out
      const float alpha = exp2f(m - m_ref);
      // rescale the accumulators only when some head's running max grew
      // (rare after the first tiles); the branch is wave-uniform and holds no loads
      const bool grew = __any(m_new > m);
      m = m_new;
      // fp16 operands: the probabilities are taken relative to this tile's own
      // max (its largest is then 1) and the tile's p.V is scaled by
      // beta = 2^(tile max - running max) on its way into the accumulator.
      // Relative to the running max, a tile far below an earlier dominant
      // token would hold probabilities in fp16's subnormal range, where the
      // hi + lo split keeps only an absolute step of 2^-24.  (bf16 has fp32's
      // exponent range and takes the probabilities as they are, beta = 1.)
      constexpr bool kTileRef = std::is_same<T, f16_t>::value;
      const float p_ref = (kTileRef && mt != neg_inf()) ? mt : m_ref;
      const float beta = kTileRef ? exp2f(p_ref - m_ref) : 1.f;
      float pr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] = exp2f(x[j >> 2][j & 3] - p_ref);
      float ps = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      lsum_d = __builtin_fma(lsum_d, (double)alpha, (double)ps * (double)beta);

      // A tile crossing the end: V rows past it (padding read by the first,
      // speculative load) become zeros, since 0 * NaN would poison the sums.
      if (t0 + kTileTokens > t_end) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool dead = t0 + tile_token(q4, j) >= t_end;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            if (dead) vr[nb][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }

      // P operand (B of O^T = V^T P^T), split into hi + lo 16-bit parts.
      u32x4 phi, plo;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t hw = pack2<T>(pr[2 * k], pr[2 * k + 1]);
        phi[k] = hw;
        plo[k] = pack2<T>(pr[2 * k] - lo_of<T>(hw), pr[2 * k + 1] - hi_of<T>(hw));
      }

#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          // V^T operand row (d = 8*(16 nb + l16) + n), tokens tile_token(q4, 0..7).
          const int w = n >> 1;
          const uint32_t sel = (n & 1) ? kSelHiHalves : kSelLoHalves;
          u32x4 va;
#pragma unroll
          for (int k = 0; k < 4; ++k) va[k] = perm_b32(vr[nb][2 * k + 1][w], vr[nb][2 * k][w], sel);
          const f32x4 a = grew ? acc[nb][n] * alpha : acc[nb][n];
          if constexpr (kTileRef) {
            f32x4 t = mfma16x16x32<T>(va, phi, f32x4{0.f, 0.f, 0.f, 0.f});
            t = mfma16x16x32<T>(va, plo, t);
            acc[nb][n] = a + t * beta;
          } else {
            acc[nb][n] = mfma16x16x32<T>(va, plo, mfma16x16x32<T>(va, phi, a));
          }
        }
      }
  };

  // The first tile is always processed (fully masked when the wave's part of
  // the chunk is empty): no branch may separate its loads from their use, or
  // the compiler moves the loads behind the length check.
  if constexpr (SPEC2) {
    // Two slots with fixed roles (no register copies of tiles in flight): a
    // slot is refilled with the tile two steps ahead as soon as it is consumed.
    do {
      tile_step(kt0, vt0);
      load_tile(t0 + 2 * NW * kTileTokens, krs, vrs, kt0, vt0);
      t0 += NW * kTileTokens;
      if (t0 >= t_end) break;
      tile_step(kt1, vt1);
      load_tile(t0 + 2 * NW * kTileTokens, krs, vrs, kt1, vt1);
      t0 += NW * kTileTokens;
    } while (t0 < t_end);
  } else {
    do {
      load_tile(t0 + NW * kTileTokens, krs, vrs, kt1, vt1);  // prefetch the wave's next tile
      tile_step(kt0, vt0);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int s = 0; s < KS; ++s) kt0[blk][s] = kt1[blk][s];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 8; ++j) vt0[nb][j] = vt1[nb][j];
      t0 += NW * kTileTokens;
    } while (t0 < t_end);
  }
  if (t_begin >= L) return false;  // empty chunk: nothing is written

  float lsum = (float)lsum_d;
  {
    const f32x2 a = rows16(lsum);
    lsum = a[0] + a[1];
    const f32x2 c = rows32(lsum);
    lsum = c[0] + c[1];
  }

  // ---- merge the waves' states (wave 0 ends up holding the chunk result) ----
  if constexpr (NW > 1) {
    if (wave > 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int n = 0; n < 8; ++n) sm.acc[wave - 1][nb * 8 + n][lane] = acc[nb][n];
      if (q4 == 0) {
        sm.m[wave][l16] = m;
        sm.l[wave][l16] = lsum;
      }
    }
    __syncthreads();
    if (wave == 0) {
      float mw[NW];
      float M = m;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        mw[w] = sm.m[w][l16];
        M = fmaxf(M, mw[w]);
      }
      const float a0 = exp2f(m - M);  // M finite: wave 0 saw the chunk's first tile
      lsum *= a0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[nb][n] *= a0;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float aw = exp2f(mw[w] - M);  // 0 for a wave that saw no tile
        lsum += aw * sm.l[w][l16];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int n = 0; n < 8; ++n) acc[nb][n] += aw * sm.acc[w - 1][nb * 8 + n][lane];
      }
      m = M;
    }
  }

  // Normalised chunk result of head g = l16 for wave 0: lane (q4, g) owns
  // d = 8*(16 nb + 4 q4) + 8 i + n for i = 0..3, n = 0..7 (32 consecutive d).
  const float inv_l = 1.0f / lsum;
  const float lse_nat = (m + log2f(lsum)) * kLn2;

  if (nlive == 1) {
    if (wave == 0 && l16 < ng) {
      const rsrc_t o_rs =
          make_rsrc(p.o_part, (uint32_t)((int64_t)p.R * p.B * p.Hq * D * esize(p.odt)));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int d0 = 8 * (16 * nb + 4 * q4);
        if (d0 >= D) continue;
        float y[32];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int n = 0; n < 8; ++n) y[8 * i + n] = acc[nb][n][i] * inv_l;
        if constexpr (kDev)
          store32_dev(o_rs, (uint32_t)(((orow0 + l16) * D + d0) * esize(p.odt)), y, p.odt);
        else
          store32(p.o_part, (orow0 + l16) * D + d0, y, p.odt);
      }
      if (q4 == 0) {
        if constexpr (kDev)
          st4_dev(make_rsrc(p.lse_part, (uint32_t)((int64_t)p.R * p.B * p.Hq * 4)),
                  (uint32_t)((orow0 + l16) * 4), lse_nat);
        else
          p.lse_part[orow0 + l16] = lse_nat;
      }
    }
    return true;
  }

  // ---- several live chunks: this chunk's normalised partial to the workspace ----
  const int64_t slot = (int64_t)unit * p.nchunks + c;
  if (wave == 0 && l16 < ng) {
    const int64_t nslots = (int64_t)p.units * p.nchunks * p.Gb;
    const rsrc_t wo_rs = make_rsrc(p.ws_o, (uint32_t)(nslots * D * 4));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int d0 = 8 * (16 * nb + 4 * q4);
      if (d0 >= D) continue;
      float y[32];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 8; ++n) y[8 * i + n] = acc[nb][n][i] * inv_l;
      if constexpr (kDev)
        store32_dev(wo_rs, (uint32_t)(((slot * p.Gb + l16) * D + d0) * 4), y, kF32);
      else
        store32(p.ws_o, (slot * p.Gb + l16) * D + d0, y, kF32);
    }
    if (q4 == 0) {
      if constexpr (kDev)
        st4_dev(make_rsrc(p.ws_lse, (uint32_t)(nslots * 4)), (uint32_t)((slot * p.Gb + l16) * 4),
                lse_nat);
      else
        p.ws_lse[slot * p.Gb + l16] = lse_nat;
    }
  }
  return true;
}

// Cross-shard weights of one group, one thread per (shard r, head g) pair:
// ew = e^(lse_r - M_g) in FP64 with M_g the head's largest shard lse (0 for an
// empty shard), and M_g itself.  Needs ms.lse; a barrier must follow.
template <int NW, int MODE>
__device__ __forceinline__ void shard_weights(int R, int ng, MergeSmem<NW, MODE>& ms) {
  for (int pi = threadIdx.x; pi < R * ng; pi += NW * 64) {
    const int g = pi % ng;
    float M = neg_inf();
    for (int r0 = 0; r0 < R; r0 += 8) {  // 8 LDS reads in flight (no read inside a branch)
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ms.lse[min(r0 + j, R - 1) * ng + g];
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, r0 + j < R ? v[j] : neg_inf());
    }
    const float l = ms.lse[pi];
    ms.ew[pi] = l == neg_inf() ? 0.0 : exp((double)l - (double)M);
    if (pi < ng) ms.M[pi] = M;
  }
}

// The cross-shard merge of output vector e (head g = e / (D/4)) from the
// shard vectors y(r) (shard order, FP32 sums, FP64 weights and lse; every
// shard empty: 0 and -inf).  Same arithmetic as the merge kernel.
template <int D, typename YF, int NW, int MODE>
__device__ __forceinline__ void merge_vector(const Args& p, int64_t row0, int e, int R, int ng,
                                             const MergeSmem<NW, MODE>& ms, YF y) {
  constexpr int Q = D / 4;
  const int g = e / Q, qd = e % Q;
  const int64_t row = row0 + g;
  // Reads are issued 8 at a time outside branches; an empty shard has weight
  // 0 and a zero vector (never read from memory), so it adds exactly nothing.
  double S = 0.0;
  for (int r0 = 0; r0 < R; r0 += 8) {
    double w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = ms.ew[min(r0 + j, R - 1) * ng + g];
#pragma unroll
    for (int j = 0; j < 8; ++j) S += r0 + j < R ? w[j] : 0.0;
  }
  if (S == 0.0) {
    store4(p.out, row * D + 4 * qd, f32x4{0.f, 0.f, 0.f, 0.f}, p.out_dt);
    if (p.lse_out != nullptr && qd == 0) p.lse_out[row] = neg_inf();
    return;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < R; r0 += 8) {
    float w[8];
    f32x4 yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = min(r0 + j, R - 1);
      w[j] = r0 + j < R ? (float)ms.ew[r * ng + g] : 0.f;
      yv[j] = y(r);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += w[j] * yv[j];
  }
  store4(p.out, row * D + 4 * qd, acc * (float)(1.0 / S), p.out_dt);
  if (p.lse_out != nullptr && qd == 0) p.lse_out[row] = (float)((double)ms.M[g] + log(S));
}

// Merge of one (sequence, kv head, head block) group over its R shards when
// shards are not split: every shard's o_part/lse_part rows were written by
// the other workgroups of this launch with device-scope stores; empty shards
// (no tokens) are never read.  s_nl[r] = live chunks (0 or 1) of shard r.
// The shard vectors of this thread's first output vector are loaded together
// with the lse values (one memory round trip).
template <int D, int NW, int MODE>
__device__ void merge_shards(const Args& p, int b, int h, int gb, const int* s_nl,
                             MergeSmem<NW, MODE>& ms) {
  constexpr int NT = NW * 64;
  constexpr int Q = D / 4;  // float4 outputs per head
  constexpr int RB = 8;     // shard vectors loaded per batch
  const int t = threadIdx.x;
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int R = p.R;
  const int E = ng * Q;
  const uint32_t es = esize(p.odt);
  const rsrc_t o_rs = make_rsrc(p.o_part, (uint32_t)((int64_t)R * p.B * p.Hq * D * es));
  const rsrc_t l_rs = make_rsrc(p.lse_part, (uint32_t)((int64_t)R * p.B * p.Hq * 4));
  const int64_t row0 = (int64_t)b * p.Hq + h * p.G + g0;  // out row of head 0
  const int64_t rstride = (int64_t)p.B * p.Hq;             // o_part rows from shard to shard
  auto vec_off = [&](int r, int e) {  // shard r's float4 e, out of range for an empty shard
    return (e < E && r < R && s_nl[min(r, R - 1)] > 0)
               ? (uint32_t)(((r * rstride + row0 + e / Q) * D + 4 * (e % Q)) * es)
               : kOutOfRange;
  };

  float l_first = neg_inf();
  if (t < R * ng) {
    const int r = t / ng;
    l_first = ld4f_dev(l_rs, s_nl[r] > 0 ? (uint32_t)((r * rstride + row0 + t % ng) * 4) : kOutOfRange);
  }
  Raw4 pre[RB];  // shards 0..RB-1 of output vector e = t
#pragma unroll
  for (int j = 0; j < RB; ++j) pre[j] = load4_dev_raw(o_rs, vec_off(j, t), p.odt);

  if (t < R * ng) ms.lse[t] = s_nl[t / ng] > 0 ? l_first : neg_inf();
  for (int i = t + NT; i < R * ng; i += NT) {
    const int r = i / ng;
    const float v = ld4f_dev(l_rs, s_nl[r] > 0 ? (uint32_t)((r * rstride + row0 + i % ng) * 4) : kOutOfRange);
    ms.lse[i] = s_nl[r] > 0 ? v : neg_inf();
  }
  __syncthreads();
  shard_weights(R, ng, ms);
  __syncthreads();

  for (int e = t; e < E; e += NT) {
    if (e == t && R <= RB) {  // the prefetched vectors, shard order (static indices)
      const int g = e / Q, qd = e % Q;
      const int64_t row = row0 + g;
      double S = 0.0;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const double w = ms.ew[min(j, R - 1) * ng + g];
        S += j < R ? w : 0.0;
      }
      if (S == 0.0) {
        store4(p.out, row * D + 4 * qd, f32x4{0.f, 0.f, 0.f, 0.f}, p.out_dt);
        if (p.lse_out != nullptr && qd == 0) p.lse_out[row] = neg_inf();
        continue;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};  // shards j >= R: weight 0, vector 0 (out of range)
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const float w = j < R ? (float)ms.ew[min(j, R - 1) * ng + g] : 0.f;
        acc += w * raw4_f32(pre[j], p.odt);
      }
      store4(p.out, row * D + 4 * qd, acc * (float)(1.0 / S), p.out_dt);
      if (p.lse_out != nullptr && qd == 0) p.lse_out[row] = (float)((double)ms.M[g] + log(S));
    } else {
      merge_vector<D>(p, row0, e, R, ng, ms,
                      [&](int r) { return load4_dev(o_rs, vec_off(r, e), p.odt); });
    }
  }
}

// Merge of one group when shards are split into chunks.  (1) One thread per
// (shard, head) pair: the chunk lse of its live chunks, their max, weights
// and sum (the chunk-combine arithmetic) and the shard lse.  (2) The FP64
// cross-shard weights.  (3) Per (shard, output vector) the chunk sum, split
// over P thread groups added in a fixed order, written to o_part.  (4) The
// cross-shard merge of the stored shard vectors.  The first batch of (3)'s
// loads is issued with (1)'s.  s_nl[r] = live chunks of shard r.
template <int D, int NW>
__device__ void merge_chunks(const Args& p, int b, int h, int gb, const int* s_nl,
                             MergeSmem<NW, kStepOneChunks>& ms) {
  constexpr int NT = NW * 64;
  constexpr int Q = D / 4;
  constexpr int KB = 16;  // loads per batch
  const int t = threadIdx.x;
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int R = p.R;
  const int nch = p.nchunks;
  const uint32_t es = esize(p.odt);
  const int64_t nslots = (int64_t)p.units * nch * p.Gb;
  const rsrc_t o_rs = make_rsrc(p.o_part, (uint32_t)((int64_t)R * p.B * p.Hq * D * es));
  const rsrc_t l_rs = make_rsrc(p.lse_part, (uint32_t)((int64_t)R * p.B * p.Hq * 4));
  const rsrc_t wo_rs = make_rsrc(p.ws_o, (uint32_t)(nslots * D * 4));
  const rsrc_t wl_rs = make_rsrc(p.ws_lse, (uint32_t)(nslots * 4));
  const int64_t row0 = (int64_t)b * p.Hq + h * p.G + g0;  // out row of head 0
  const int64_t rstride = (int64_t)p.B * p.Hq;
  const int64_t ustride = (int64_t)p.B * p.Hkv * p.gblocks;  // units from shard to shard
  const int64_t slot00 = (int64_t)((b * p.Hkv + h) * p.gblocks + gb) * nch;  // shard 0, chunk 0
  const uint32_t cstride = (uint32_t)(p.Gb * D * 4);  // workspace bytes from chunk to chunk

  // (3)'s work split: items = (shard, float4) pairs, P chunk partitions each
  const int E = ng * Q;
  const int items = R * E;
  int P = 1;
  while (P < 8 && items * P * 2 <= NT) P *= 2;
  const int per = NT / P;
  const int part_id = t / per;
  auto vec_base = [&](int r, int e) {  // chunk 0 of shard r's float4 e in the workspace
    return (uint32_t)(((slot00 + r * ustride * nch) * p.Gb + e / Q) * D * 4) + 16u * (e % Q);
  };

  // ---- one round of loads: the chunk lse of this thread's (shard, head) pair
  //      first (phase (1) waits only for those), then the first batch of its
  //      first item's chunk vectors ----
  constexpr int LB = 16;  // chunk lse values held in registers
  const int pi0 = t;      // this thread's (shard, head) pair, if any
  const int r0p = min(pi0 / ng, R - 1), g0p = pi0 - (pi0 / ng) * ng;
  const int nl0p = pi0 < R * ng ? s_nl[r0p] : 0;
  const uint32_t lstride = (uint32_t)(p.Gb * 4);
  const uint32_t lbase0 = (uint32_t)(((slot00 + r0p * ustride * nch) * p.Gb + g0p) * 4);
  float v0[LB];
#pragma unroll
  for (int j = 0; j < LB; ++j)
    v0[j] = ld4f_dev(wl_rs, (nl0p >= 2 && j < nl0p) ? lbase0 + j * lstride : kOutOfRange);
  const float l_one0 =
      ld4f_dev(l_rs, nl0p == 1 ? (uint32_t)((r0p * rstride + row0 + g0p) * 4) : kOutOfRange);

  // ---- prefetch the first batch of this thread's first item ----
  const int it_first = t % per;
  const int r_first = min(it_first / E, R - 1), e_first = it_first % E;
  const int nl_first = it_first < items ? s_nl[r_first] : 0;
  f32x4 pre[KB];
  {
    const uint32_t base = vec_base(r_first, e_first);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int cc = part_id + j * P;
      pre[j] = __builtin_bit_cast(
          f32x4, ld16_dev(wo_rs, (nl_first >= 2 && cc < nl_first) ? base + cc * cstride : kOutOfRange));
    }
  }
  const Raw4 pre_one = load4_dev_raw(
      o_rs,
      (nl_first == 1 && part_id == 0)
          ? (uint32_t)(((r_first * rstride + row0 + e_first / Q) * D + 4 * (e_first % Q)) * es)
          : kOutOfRange,
      p.odt);

  // (1) per (shard, head): chunk weights and shard lse
  for (int pi = t; pi < R * ng; pi += NT) {
    const int r = pi / ng, g = pi - r * ng;
    const int nl = s_nl[r];
    const bool first = pi == pi0;
    float l = neg_inf();
    if (nl == 1) {
      l = first ? l_one0 : ld4f_dev(l_rs, (uint32_t)((r * rstride + row0 + g) * 4));
    } else if (nl >= 2) {
      float* wr = ms.w + pi * nch;
      const uint32_t lbase = (uint32_t)(((slot00 + r * ustride * nch) * p.Gb + g) * 4);
      float v[LB];
      if (first) {
#pragma unroll
        for (int j = 0; j < LB; ++j) v[j] = v0[j];
      } else {
#pragma unroll
        for (int j = 0; j < LB; ++j) v[j] = ld4f_dev(wl_rs, j < nl ? lbase + j * lstride : kOutOfRange);
      }
      float M = neg_inf();
      float S = 0.f;
      if (nl <= LB) {  // all in registers
#pragma unroll
        for (int j = 0; j < LB; ++j)
          if (j < nl) M = fmaxf(M, v[j]);
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          v[j] = j < nl ? expf(v[j] - M) : 0.f;
          S += v[j];
        }
        const float invS = 1.0f / S;
#pragma unroll
        for (int j = 0; j < LB; ++j)
          if (j < nl) wr[j] = v[j] * invS;
      } else {  // through LDS, in chunk order
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          wr[j] = v[j];
          M = fmaxf(M, v[j]);
        }
        for (int c = LB; c < nl; ++c) {
          wr[c] = ld4f_dev(wl_rs, lbase + c * lstride);
          M = fmaxf(M, wr[c]);
        }
        for (int c = 0; c < nl; ++c) {
          const float e = expf(wr[c] - M);
          wr[c] = e;
          S += e;
        }
        const float invS = 1.0f / S;
        for (int c = 0; c < nl; ++c) wr[c] *= invS;
      }
      l = M + logf(S);
      p.lse_part[r * rstride + row0 + g] = l;
    }
    ms.lse[pi] = l;
  }
  __syncthreads();
  shard_weights(R, ng, ms);  // (2); read only after the next barrier

  // (3) every shard's partial vectors
  for (int i0 = 0; i0 < items; i0 += per) {
    const int it = i0 + t % per;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    int r = 0, e = 0, nl = 0;
    if (it < items) {
      r = it / E;
      e = it - r * E;
      nl = s_nl[r];
      if (nl >= 2) {
        const float* wr = ms.w + (r * ng + e / Q) * nch;
        const uint32_t base = vec_base(r, e);
        int c0 = part_id;
        if (i0 == 0) {  // the prefetched first batch (weights read first, no branch per chunk)
          float wv[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) wv[j] = wr[min(c0 + j * P, nch - 1)];
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            const f32x4 yj = y + wv[j] * pre[j];
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = c0 + j * P < nl ? yj[k] : y[k];
          }
          c0 += KB * P;
        }
        for (; c0 < nl; c0 += KB * P) {
          f32x4 v[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            const int cc = c0 + j * P;
            v[j] = __builtin_bit_cast(f32x4, ld16_dev(wo_rs, cc < nl ? base + cc * cstride : kOutOfRange));
          }
          float wv[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) wv[j] = wr[min(c0 + j * P, nch - 1)];
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            const f32x4 yj = y + wv[j] * v[j];
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = c0 + j * P < nl ? yj[k] : y[k];
          }
        }
      } else if (nl == 1 && part_id == 0) {
        y = i0 == 0 ? raw4_f32(pre_one, p.odt)
                    : load4_dev(o_rs, (uint32_t)(((r * rstride + row0 + e / Q) * D + 4 * (e % Q)) * es),
                                p.odt);
      }
    }
    if (P > 1) {
      ms.part[t] = y;
      __syncthreads();
      if (part_id == 0 && it < items)
        for (int q = 1; q < P; ++q) y += ms.part[t + q * per];
      __syncthreads();
    }
    if (part_id == 0 && it < items) {
      if (nl >= 2) {
        store4(p.o_part, (r * rstride + row0 + e / Q) * D + 4 * (e % Q), y, p.odt);
        y = round4(y, p.odt);
      }
      ms.y[it] = y;
    }
  }
  __syncthreads();

  // (4) cross-shard merge
  for (int e = t; e < E; e += NT)
    merge_vector<D>(p, row0, e, R, ng, ms, [&](int r) { return ms.y[r * E + e]; });
}

// Chunk combine and cross-shard merge of ONE query head (head g of head block
// gb of kv head h, sequence b) whose (shard, chunk) pairs fit one wave: lanes
// of wave 0 hold one chunk lse each (shard r in lanes [r * nchp, (r + 1) *
// nchp), nchp = chunks rounded up to a power of two), so every statistic is
// an xor-shuffle reduction; threads (partition, shard, float4) sum their
// chunk vectors from registers.  Same formulas as merge_chunks (chunk max,
// weights, shard lse; cross-shard weights; merged lse in FP64), with the
// shuffle trees' summation order, except that the cross-shard weights that
// scale the output are FP32 here (the output moves by ~1e-7 of itself, far
// inside its tolerance) so that the FP64 merged lse can be formed beside the
// output instead of ahead of it, and that the FP32 statistics take exp, log
// and 1/x from the hardware instructions (about 1 ulp each).  KB chunk
// vectors are loaded per thread group.  Needs R * Q <= threads and every live
// chunk among the KB * P a thread group loads (both hold where it is called).
template <int D, int NW, int MODE, int KB = 16>
__device__ void merge_row_chunks(const Args& p, int b, int h, int gb, int g, const int* s_nl,
                                 MergeSmem<NW, MODE>& ms, int lg_nchp) {
  constexpr int NT = NW * 64;
  constexpr int Q = D / 4;
  constexpr int LGQ = __builtin_ctz(Q);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int R = p.R;
  const int nch = p.nchunks;
  const int nchp = 1 << lg_nchp;
  const uint32_t es = esize(p.odt);
  const int Gb = p.Gb;
  const int64_t nslots = (int64_t)p.units * nch * Gb;
  const rsrc_t o_rs = make_rsrc(p.o_part, (uint32_t)((int64_t)R * p.B * p.Hq * D * es));
  const rsrc_t l_rs = make_rsrc(p.lse_part, (uint32_t)((int64_t)R * p.B * p.Hq * 4));
  const rsrc_t wo_rs = make_rsrc(p.ws_o, (uint32_t)(nslots * D * 4));
  const rsrc_t wl_rs = make_rsrc(p.ws_lse, (uint32_t)(nslots * 4));
  const int row0 = b * p.Hq + h * p.G + gb * kGroupRows + g;    // the query head's row
  const int rstride = p.B * p.Hq;                                // o_part rows, shard to shard
  const int sstride = p.B * p.Hkv * p.gblocks * nch;             // slots, shard to shard
  const int slot00 = ((b * p.Hkv + h) * p.gblocks + gb) * nch;   // shard 0, chunk 0

  // items (shard, float4): per = power of two >= R * Q threads, P partitions
  int lg_per = LGQ;
  while ((1 << lg_per) < R * Q) ++lg_per;
  const int per = 1 << lg_per;
  const int P = NT >> lg_per;
  const int it = t & (per - 1), part = t >> lg_per;
  const int ri = it >> LGQ, qi = it & (Q - 1);
  const int nli = ri < R ? s_nl[ri] : 0;

  // ---- one round of loads: wave 0's chunk lse first, then the chunk vectors ----
  const int rl = lane >> lg_nchp, cl = lane & (nchp - 1);
  const int nll = rl < R ? s_nl[rl] : 0;
  const bool chunk_l = t < 64 && nll >= 2 && cl < nll;  // a live chunk of a split shard
  const bool shard_l = t < 64 && nll == 1 && cl == 0;   // a shard with one live chunk
  const float lc =
      ld4f_dev(wl_rs, chunk_l ? (uint32_t)(((slot00 + rl * sstride + cl) * Gb + g) * 4) : kOutOfRange);
  const float ls1 = ld4f_dev(l_rs, shard_l ? (uint32_t)((rl * rstride + row0) * 4) : kOutOfRange);
  f32x4 v[KB];
  {
    const uint32_t base = (uint32_t)(((slot00 + ri * sstride) * Gb + g) * D * 4) + 16u * qi;
    const uint32_t cstride = (uint32_t)(Gb * D * 4);  // chunk to chunk
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int cc = part + j * P;
      v[j] = __builtin_bit_cast(
          f32x4, ld16_dev(wo_rs, (nli >= 2 && cc < nli) ? base + (uint32_t)cc * cstride : kOutOfRange));
    }
  }
  const Raw4 v_one = load4_dev_raw(
      o_rs, (nli == 1 && part == 0) ? (uint32_t)(((ri * rstride + row0) * D + 4 * qi) * es) : kOutOfRange,
      p.odt);

  // ---- (1)+(2) wave 0: chunk weights, shard lse, cross-shard weights ----
  // The global stores (split shards' lse_part and o_part) are issued after the
  // last barrier: a workgroup barrier waits for this wave's outstanding
  // stores too, which would put a store round trip on the path to the output.
  float ls_split = 0.f;  // lse_part of a split shard, stored by lane cl == 0
  if (t < 64) {
    const float lv = chunk_l ? lc : shard_l ? ls1 : neg_inf();
    // This chain is the merge's critical path, a few hundred dependent
    // instructions: exp, log and reciprocal use the hardware's base-2
    // exponential, logarithm and reciprocal (about 1 ulp each, against the
    // library calls' dozen instructions apiece).
    const float M = lane_reduce(lv, lg_nchp, OpMax{});       // over the shard's lanes
    const float e = M == neg_inf() ? 0.f : __expf(lv - M);  // -inf chunks give 0
    const float S = lane_reduce(e, lg_nchp, OpSum{});
    if (nll >= 2 && cl < nll) ms.w[rl * nch + cl] = e * __builtin_amdgcn_rcpf(S);
    // shard lse (nl == 1: the stored one, S = 1)
    const float ls = S > 0.f ? M + __builtin_amdgcn_logf(S) * kLn2 : neg_inf();
    ls_split = ls;
    const float Mx = wave_max(cl == 0 ? ls : neg_inf());  // max over shards
    // FP32 cross-shard weights for the output; the merged lse is formed in
    // FP64 at the end, off the path to the output.
    const float ew = (cl == 0 && rl < R && ls != neg_inf()) ? __expf(ls - Mx) : 0.f;
    const float St = wave_sum(ew);
    if (cl == 0 && rl < R) {
      ms.lse[rl] = ew;               // shard weight (unnormalised)
      ms.lse[kMaxShards + rl] = ls;  // shard lse, for the merged lse
    }
    if (lane == 0) {
      ms.M[0] = St > 0.f ? __builtin_amdgcn_rcpf(St) : 0.f;
      ms.M[1] = Mx;
    }
  }
  __syncthreads();

  // ---- (3) shard vectors ----
  // All weights are read first and the sum is branch-free: a read inside a
  // per-chunk branch would wait for the LDS on its own, 16 times in a row.
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
  if (ri < R) {
    const float* wr = ms.w + ri * nch;
    float wv[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) wv[j] = wr[min(part + j * P, nch - 1)];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const bool live = nli >= 2 && part + j * P < nli;  // else wv[j] may be stale
      const f32x4 yj = y + wv[j] * v[j];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = live ? yj[k] : y[k];
    }
    if (nli == 1) y = raw4_f32(v_one, p.odt);
  }
  if (P > 1) {
    ms.part[t] = y;
    __syncthreads();
    if (part == 0)
      for (int q = 1; q < P; ++q) y += ms.part[t + q * per];
  }
  const f32x4 y_split = y;  // o_part of a split shard, stored at the end
  if (part == 0 && ri < R) ms.y[it] = nli >= 2 ? round4(y, p.odt) : y;
  __syncthreads();

  // ---- (4) cross-shard merge, shard order ----
  // An empty shard has weight 0 and vector 0, so it adds exactly nothing; the
  // sum needs no branch and its reads can be issued together.
  if (t < Q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int r = 0; r < R; ++r) acc += ms.lse[r] * ms.y[r * Q + t];
    store4(p.out, (int64_t)row0 * D + 4 * t, acc * ms.M[0], p.out_dt);
  }
  // ---- (5) merged lse, FP64 (the merge kernel's formula) ----
  // Lane r of the last wave takes shard r (R <= 64 here), so with two or more
  // waves this runs beside the output above instead of ahead of it.
  if (p.lse_out != nullptr && (t >> 6) == NW - 1) {
    const int r = t & 63;
    const float Mx = ms.M[1];
    const float ls = r < R ? ms.lse[kMaxShards + r] : neg_inf();
    const double e = ls != neg_inf() ? exp((double)ls - (double)Mx) : 0.0;
    const double St = wave_sum_f64(e);
    if (r == 0) p.lse_out[row0] = St > 0.0 ? (float)((double)Mx + log(St)) : neg_inf();
  }
  // ---- split shards' partials (no barrier follows) ----
  if (part == 0 && ri < R && nli >= 2)
    store4(p.o_part, (int64_t)(ri * rstride + row0) * D + 4 * qi, y_split, p.odt);
  if (t < 64 && nll >= 2 && cl == 0) p.lse_part[rl * rstride + row0] = ls_split;
}


// One arrival at a counter of `members` arrivals (relaxed, agent scope; the
// caller's device-scope stores have completed).  Returns whether this was the
// last arrival, and then resets the counter to zero for the next call.
__device__ __forceinline__ int arrive(int32_t* counter, int members) {
  const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int last = old == members - 1;
  if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// The 4 values x as stored in dtype `odt`, written with a device-scope store at
// byte offset `off`.
__device__ __forceinline__ void store4_dev(rsrc_t r, uint32_t off, f32x4 x, int odt) {
  if (odt == kF32) {
    st16_dev(r, off, __builtin_bit_cast(u32x4, x));
  } else if (odt == kBF16) {
    st8_dev(r, off, u32x2{pack2<bf16_t>(x[0], x[1]), pack2<bf16_t>(x[2], x[3])});
  } else {
    st8_dev(r, off, u32x2{pack2<f16_t>(x[0], x[1]), pack2<f16_t>(x[2], x[3])});
  }
}

// First level of the two-level one-launch step: the chunk combine of one unit
// (shard r, sequence b, kv head h, head block gb) with nl >= 2 live chunks,
// done by the unit's last-arriving chunk workgroup.  Same arithmetic as the
// chunk-combine launch (per head: chunk max, weights e^(lse_c - M) / sum,
// shard lse M + ln sum; the weighted sum of the normalised chunk partials),
// written to o_part/lse_part with device-scope stores for the second level.
// Chunk statistics: lanes (head g, chunk c) with nlp = nl rounded up to a
// power of two lanes per head (xor-shuffle reductions within a wave); the
// weighted sums: threads (partition, head, float4), chunks split over P
// partitions added in a fixed order.
template <int D, int NW, int MODE>
__device__ void combine_unit(const Args& p, int unit, int r, int b, int h, int gb, int nl,
                             MergeSmem<NW, MODE>& ms) {
  if (nl < 2) return;  // one live chunk went straight to o_part; none: the shard is empty
  constexpr int NT = NW * 64;
  constexpr int Q = D / 4;
  constexpr int KB = 16;  // chunk vectors in flight per thread
  const int t = threadIdx.x;
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int nch = p.nchunks;
  const uint32_t es = esize(p.odt);
  const int64_t nslots = (int64_t)p.units * nch * p.Gb;
  const rsrc_t wo_rs = make_rsrc(p.ws_o, (uint32_t)(nslots * D * 4));
  const rsrc_t wl_rs = make_rsrc(p.ws_lse, (uint32_t)(nslots * 4));
  const rsrc_t o_rs = make_rsrc(p.o_part, (uint32_t)((int64_t)p.R * p.B * p.Hq * D * es));
  const rsrc_t l_rs = make_rsrc(p.lse_part, (uint32_t)((int64_t)p.R * p.B * p.Hq * 4));
  const int64_t orow0 = ((int64_t)r * p.B + b) * p.Hq + h * p.G + g0;  // o_part row of head g0
  const int64_t slot0 = (int64_t)unit * nch;                          // chunk 0 of this unit

  // (1) chunk weights and shard lse per head
  int lg = 0;
  while ((1 << lg) < nl) ++lg;  // nl <= 64: one wave holds a head's chunks
  const int nlp = 1 << lg;
  const int hpp = NT / nlp;  // heads per pass
  for (int gp = 0; gp < ng; gp += hpp) {
    const int g = gp + t / nlp, c = t % nlp;
    const bool on = g < ng && c < nl;
    float lv = ld4f_dev(wl_rs, on ? (uint32_t)(((slot0 + c) * p.Gb + g) * 4) : kOutOfRange);
    lv = on ? lv : neg_inf();
    const float M = lane_reduce(lv, lg, OpMax{});  // finite: a live chunk has tokens
    const float e = on ? expf(lv - M) : 0.f;
    const float S = lane_reduce(e, lg, OpSum{});
    if (on) ms.w[g * nch + c] = e * (1.0f / S);
    if (c == 0 && g < ng) st4_dev(l_rs, (uint32_t)((orow0 + g) * 4), M + logf(S));
  }
  __syncthreads();

  // (2) weighted sums of the chunk partials
  const int E = ng * Q;
  int P = 1;
  while (P < 8 && E * P * 2 <= NT) P *= 2;
  const int per = NT / P;
  const int part = t / per;
  for (int e0 = 0; e0 < E; e0 += per) {
    const int e = e0 + t % per;
    const int g = min(e / Q, ng - 1), q = e % Q;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (e < E) {
      const float* wr = ms.w + g * nch;
      const uint32_t base = (uint32_t)((slot0 * p.Gb + g) * D * 4) + 16u * q;
      const uint32_t cstride = (uint32_t)(p.Gb * D * 4);
      for (int c0 = part; c0 < nl; c0 += KB * P) {
        f32x4 v[KB];
        float wv[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const int cc = c0 + j * P;
          v[j] = __builtin_bit_cast(f32x4, ld16_dev(wo_rs, cc < nl ? base + cc * cstride : kOutOfRange));
          wv[j] = wr[min(cc, nch - 1)];
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const f32x4 yj = y + wv[j] * v[j];
#pragma unroll
          for (int k = 0; k < 4; ++k) y[k] = c0 + j * P < nl ? yj[k] : y[k];
        }
      }
    }
    if (P > 1) {
      ms.part[t] = y;
      __syncthreads();
      if (part == 0)
        for (int k = 1; k < P; ++k) y += ms.part[t + k * per];
      __syncthreads();
    }
    if (part == 0 && e < E) store4_dev(o_rs, (uint32_t)(((orow0 + g) * D + 4 * q) * es), y, p.odt);
  }
}

// SMALL_MERGE: the one-launch single-head merge loads 2 chunk vectors per
// thread group instead of 16 (the launch checks that 2 cover every chunk).
template <typename T, int D, int NW, int MODE, bool ORDERED = false, bool SPEC2 = false,
          bool SMALL_MERGE = false>
__global__ __launch_bounds__(NW * 64) void attn_partial_kernel(const AttnParams kp) {
  const void* kshard;
  const void* vshard;
  const Args p = load_args<ORDERED>(kp, kshard, vshard);
  __shared__ KernelSmem<T, D, NW, MODE> sh;
  __shared__ int s_last;
  __shared__ int s_nl[MODE >= kStepOneShards ? kMaxShards : 1];  // live chunks per shard

  // Grid: x = (chunk, unit within the shard), chunk-major; y = shard.  The
  // shard's K/V pointers are then fetched with the other arguments at once.
  // Workgroups are dealt to the 8 XCDs round-robin by linear block index, so
  // block % 8 must not correlate with the chunk index (the later chunks of
  // ragged shards are mostly empty); here it follows the unit.
  const int upr = p.B * p.Hkv * p.gblocks;  // units per shard
  int r, c, uis, gb, h, b, len_raw;
  if constexpr (ORDERED) {
    // Longest-first order (shards not split): consecutive blocks are the
    // (kv head, head block) units of one (shard, sequence) pair, and the
    // pairs come longest first, as the order pre-pass listed them.
    const int per_pair = p.Hkv * p.gblocks;
    const int lin = blockIdx.x + blockIdx.y * gridDim.x;
    const int pair = lin / per_pair;
    const int hu = lin - pair * per_pair;
    const rsrc_t ors = make_rsrc(p.order, (uint32_t)(p.R * p.B * sizeof(OrderEntry)));
    const u32x4 e0 = buf16(ors, (uint32_t)pair * sizeof(OrderEntry));
    const u32x4 e1 = buf16(ors, (uint32_t)pair * sizeof(OrderEntry) + 16u);
    kshard = reinterpret_cast<const void*>((uint64_t)rfl(e0[0]) | ((uint64_t)rfl(e0[1]) << 32));
    vshard = reinterpret_cast<const void*>((uint64_t)rfl(e0[2]) | ((uint64_t)rfl(e0[3]) << 32));
    r = (int)rfl(e1[0]);
    b = (int)rfl(e1[1]);
    len_raw = (int)rfl(e1[2]);
    c = 0;
    gb = hu % p.gblocks;
    h = hu / p.gblocks;
    uis = b * per_pair + hu;
  } else {
    r = blockIdx.y;
    c = blockIdx.x / upr;
    uis = blockIdx.x - c * upr;
    int u = uis;
    gb = u % p.gblocks; u /= p.gblocks;
    h = u % p.Hkv;
    b = u / p.Hkv;
    // this shard's length (waited for inside, after the first tile is requested)
    len_raw = (int)__builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(p.lens, (uint32_t)(p.R * p.B * 4)), (r * p.B + b) * 4, 0, 0);
  }
  const int unit = r * upr + uis;
  // One-launch step: every shard's length of this sequence, for whichever
  // workgroup ends up merging (requested early inside, used after the attention).
  int len_t = 0;
  if (!attend_chunk<T, D, NW, MODE, SPEC2>(p, kshard, vshard, sh.a, c, unit, r, b, h, gb, len_raw,
                                           len_t) &&
      c == 0) {  // empty shard: o_r = 0, lse_r = -inf (the merge never reads them)
    const int g0 = gb * kGroupRows;
    const int ng = min(kGroupRows, p.G - g0);
    const int64_t orow0 = ((int64_t)r * p.B + b) * p.Hq + h * p.G + g0;
    for (int e = threadIdx.x; e < ng * (D / 4); e += NW * 64)
      store4(p.o_part, orow0 * D + 4 * e, f32x4{0.f, 0.f, 0.f, 0.f}, p.odt);
    if ((int)threadIdx.x < ng) p.lse_part[orow0 + threadIdx.x] = neg_inf();
  }
  if constexpr (MODE >= kStepOneShards) {
    // Arrival: this workgroup's device-scope stores are complete before the
    // counter moves; the workgroup that takes the group's counter to its
    // member count (R shards x chunks) merges the group and resets it.
    if (threadIdx.x < (unsigned)p.R)
      s_nl[threadIdx.x] = (min(max(len_t, 0), p.cap) + p.chunk - 1) / p.chunk;
    wait_vm_all();
    __syncthreads();
    const int grp = (b * p.Hkv + h) * p.gblocks + gb;
    if constexpr (MODE == kPartialsCombine) {
      // Partials only: the unit's last chunk workgroup combines its chunks.
      if (threadIdx.x == 0) s_last = arrive(p.counters + unit * kStepCounterStride, p.nchunks);
      __syncthreads();
      if (!s_last) return;
      combine_unit<D, NW>(p, unit, r, b, h, gb, s_nl[r], sh.m);
    } else if constexpr (MODE == kStepTwoLevel) {
      // Level 1: the unit's chunk workgroups (counter line `unit`); the last
      // one combines the unit's chunks into o_part/lse_part.
      if (threadIdx.x == 0) s_last = arrive(p.counters + unit * kStepCounterStride, p.nchunks);
      __syncthreads();
      if (!s_last) return;
      combine_unit<D, NW>(p, unit, r, b, h, gb, s_nl[r], sh.m);
      wait_vm_all();
      __syncthreads();
      // Level 2: the group's units, one per shard (counter lines after the
      // units'); the last one merges the shards.
      if (threadIdx.x == 0)
        s_last = arrive(p.counters + (p.units + grp) * kStepCounterStride, p.R);
      __syncthreads();
      if (!s_last) return;
      merge_shards<D, NW>(p, b, h, gb, s_nl, sh.m);
    } else {
      if (threadIdx.x == 0) s_last = arrive(p.counters + grp * kStepCounterStride, p.R * p.nchunks);
      __syncthreads();
      if (!s_last) return;
      if constexpr (MODE == kStepOneShards) {
        merge_shards<D, NW>(p, b, h, gb, s_nl, sh.m);
      } else {
        int lg_nchp = 0;
        while ((1 << lg_nchp) < p.nchunks) ++lg_nchp;
        if (p.G == 1 && (p.R << lg_nchp) <= 64)
          merge_row_chunks<D, NW, MODE, SMALL_MERGE ? 2 : 16>(p, b, h, 0, 0, s_nl, sh.m, lg_nchp);
        else
          merge_chunks<D, NW>(p, b, h, gb, s_nl, sh.m);
      }
    }
  }
}

// The separate-launch step's chunk combine and cross-shard merge in one
// kernel: one workgroup per (sequence b, query head), reading the chunk
// partials and single-chunk shard results the attention launch wrote, and
// writing o_part/lse_part of split shards and out/lse_out (merge_row_chunks).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void row_merge_kernel(const AttnParams kp) {
  const void* ks_unused;
  const void* vs_unused;
  const Args p = load_args(kp, ks_unused, vs_unused);
  __shared__ MergeSmem<NW, kStepOneChunks> ms;
  __shared__ int s_nl[kMaxShards];
  const int row = blockIdx.x;  // b * Hq + query head
  const int b = row / p.Hq, hq = row - b * p.Hq;
  const int h = hq / p.G, gl = hq - h * p.G;
  const int gb = gl / kGroupRows, g = gl - gb * kGroupRows;
  if (threadIdx.x < (unsigned)p.R) {
    const int L = min(max(p.lens[threadIdx.x * p.B + b], 0), p.cap);
    s_nl[threadIdx.x] = (L + p.chunk - 1) / p.chunk;
  }
  __syncthreads();
  int lg_nchp = 0;
  while ((1 << lg_nchp) < p.nchunks) ++lg_nchp;
  merge_row_chunks<D, NW>(p, b, h, gb, g, s_nl, ms, lg_nchp);
}

// Merge the chunk partials of every unit that has more than one live chunk
// (one 256-thread workgroup per unit), with the LSE weighting of the
// cross-shard merge.  Per-head statistics use wave reductions over chunks;
// the weighted sum splits the chunks over P thread groups when the unit has
// fewer than 256 float4 outputs, and the groups are added in a fixed order
// (results do not depend on timing).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnParams kp) {
  const void* ks_unused;
  const void* vs_unused;
  const Args p = load_args(kp, ks_unused, vs_unused);
  __shared__ float w[kMaxChunks][16];
  __shared__ f32x4 part[256];
  const int unit = blockIdx.x;
  int u = unit;
  const int gb = u % p.gblocks; u /= p.gblocks;
  const int h = u % p.Hkv; u /= p.Hkv;
  const int b = u % p.B;
  const int r = u / p.B;
  const int L = min(max(__builtin_amdgcn_readfirstlane(p.lens[r * p.B + b]), 0), p.cap);
  const int nlive = (L + p.chunk - 1) / p.chunk;
  if (nlive < 2) return;  // written directly by the attention kernel
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int64_t orow0 = ((int64_t)r * p.B + b) * p.Hq + h * p.G + g0;
  const int64_t slot0 = (int64_t)unit * p.nchunks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // per-head max, weight sum and normalised weights (wave per head)
  for (int g = wave; g < ng; g += 4) {
    float M = neg_inf();
    for (int cc = lane; cc < nlive; cc += 64) M = fmaxf(M, p.ws_lse[(slot0 + cc) * p.Gb + g]);
    M = wave_max(M);
    float S = 0.f;
    for (int cc = lane; cc < nlive; cc += 64) {
      const float e = expf(p.ws_lse[(slot0 + cc) * p.Gb + g] - M);
      w[cc][g] = e;
      S += e;
    }
    S = wave_sum(S);
    const float invS = 1.0f / S;
    for (int cc = lane; cc < nlive; cc += 64) w[cc][g] *= invS;
    if (lane == 0) p.lse_part[orow0 + g] = M + logf(S);
  }
  __syncthreads();

  constexpr int Q = D / 4;               // float4 outputs per head
  const int E = ng * Q;                  // float4 outputs of this unit
  int P = 1;                             // chunk partitions
  while (P < 8 && E * P * 2 <= 256) P *= 2;
  const int t = threadIdx.x;
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
  for (int e0 = 0; e0 < E; e0 += 256 / P) {
    const int e = e0 + t % (256 / P);
    const int part_id = t / (256 / P);
    y = f32x4{0.f, 0.f, 0.f, 0.f};
    if (e < E) {
      const int g = e / Q;
      const float* src = p.ws_o + (slot0 * p.Gb + g) * D + 4 * (e % Q);
      const int64_t cstride = (int64_t)p.Gb * D;
#pragma unroll 4
      for (int cc = part_id; cc < nlive; cc += P)
        y += w[cc][g] * *reinterpret_cast<const f32x4*>(src + cc * cstride);
    }
    if (P > 1) {
      part[t] = y;
      __syncthreads();
      if (part_id == 0 && e < E) {
        for (int q = 1; q < P; ++q) y += part[t + q * (256 / P)];
      }
      __syncthreads();
    }
    if (part_id == 0 && e < E) store4(p.o_part, (orow0 + e / Q) * D + 4 * (e % Q), y, p.odt);
  }
}

// Longest-first launch order: one workgroup sorts the R*B (shard, sequence)
// pairs by length, longest first (ties in index order, so the order is
// deterministic), with a bitonic sort of 64-bit keys in LDS, and writes one
// OrderEntry per pair.  Lengths are clamped to [0, cap] for the key only.
// npad = R*B rounded up to a power of two; threads = npad/2 within [64, 1024],
// so each thread does one compare-exchange per stage (two for npad = 4096).
constexpr int kOrderMaxThreads = 1024;
__global__ __launch_bounds__(kOrderMaxThreads) void order_kernel(const AttnParams p, int npad) {
  __shared__ uint64_t key[kOrderMaxPairs];
  __shared__ const void* kp[kMaxShards];
  __shared__ const void* vp[kMaxShards];
  const int t = threadIdx.x;
  const int nt = blockDim.x;
  const int n = p.R * p.B;
  if (t < p.R) {
    kp[t] = p.k[t];
    vp[t] = p.v[t];
  }
  for (int i = t; i < npad; i += nt) {
    uint64_t k = ~0ull;  // padding sorts last
    if (i < n) {
      const int L = min(max(p.lens[i], 0), p.cap);
      k = ((uint64_t)(uint32_t)(0x7fffffff - L) << 32) | (uint32_t)i;
    }
    key[i] = k;
  }
  // Stage (size, stride): pair i compares positions lo = 2i - (i mod stride)
  // and lo + stride, ascending where lo & size == 0.  For stride <= 64 the 64
  // pairs of a wave (i = 64w + j, in each pass of nt pairs) stay inside the
  // wave's own 128 positions, so a run of such stages needs no workgroup
  // barrier, only the wave's own program order; a wider stage, and the first
  // stage after one, synchronise the workgroup.
  bool prev_wide = true;
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const bool wide = stride > 64;
      if (wide || prev_wide) {
        __syncthreads();
      } else {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
      prev_wide = wide;
      for (int i = t; i < npad / 2; i += nt) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool ascending = (lo & size) == 0;
        const uint64_t a = key[lo], c = key[hi];
        if ((a > c) == ascending) {
          key[lo] = c;
          key[hi] = a;
        }
      }
    }
  }
  __syncthreads();
  for (int i = t; i < n; i += nt) {
    const int idx = (int)(uint32_t)key[i];
    const int r = idx / p.B;
    const int b = idx - r * p.B;
    const uint64_t kk = reinterpret_cast<uint64_t>(kp[r]), vv = reinterpret_cast<uint64_t>(vp[r]);
    u32x4* e = reinterpret_cast<u32x4*>(static_cast<char*>(p.order) + (size_t)i * sizeof(OrderEntry));
    e[0] = u32x4{(uint32_t)kk, (uint32_t)(kk >> 32), (uint32_t)vv, (uint32_t)(vv >> 32)};
    e[1] = u32x4{(uint32_t)r, (uint32_t)b, (uint32_t)p.lens[idx], 0u};
  }
}

hipError_t launch_order(const AttnParams& p, hipStream_t s) {
  const int n = p.R * p.B;  // <= kOrderMaxPairs (the planner's limit)
  int npad = 2;
  while (npad < n) npad <<= 1;
  const int threads = min(kOrderMaxThreads, max(64, npad / 2));
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(threads), 0, s, p, npad);
  return hipGetLastError();
}

// Whether the one-launch step's merge takes the single-head merger with 2
// chunk vectors per thread group: one query head per group (G = 1), shards x
// chunks (rounded up to a power of two) within one wave, and ceil(chunks /
// partitions) <= 2, where partitions = threads / (R * D/4 rounded up to a
// power of two, at least D/4) -- as merge_row_chunks lays them out.
inline bool small_row_merge(const AttnParams& p, int D, int NW) {
  if (p.G != 1) return false;
  int lg_nchp = 0;
  while ((1 << lg_nchp) < p.nchunks) ++lg_nchp;
  if ((p.R << lg_nchp) > 64) return false;
  const int q = D / 4;
  int per = q;
  while (per < p.R * q) per <<= 1;
  const int parts = NW * 64 / per;
  return parts >= 1 && (p.nchunks + parts - 1) / parts <= 2;
}

template <typename T, int D, int NW>
hipError_t launch_typed(const AttnParams& p, int64_t units, StepMode mode, hipStream_t s) {
  const dim3 grid((unsigned)(units / p.R * p.nchunks), (unsigned)p.R), block(NW * 64);
  if (p.order != nullptr) {  // shards not split, separate launches
    hipError_t e = launch_order(p, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kPartialsOnly, true>), grid, block, 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess || mode != kStepLaunches) return e;
    return launch_lse_merge(p.o_part, p.lse_part, p.R, (int64_t)p.B * p.Hq, D, p.odt, p.out_dt,
                            p.out, p.lse_out, s);
  }
  if (mode == kStepOneShards) {
    hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepOneShards>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  if (mode == kStepOneChunks) {
    // Single-head groups whose chunks 2 loads per merging thread group cover
    // take the kernel with the short merge (c1: 7.80 -> 7.48 us); a second
    // merge inside one kernel made the longer splits slower (c2 +0.25 us).
    if constexpr (NW == 2 || NW == 4) {
      if (small_row_merge(p, D, NW)) {
        if (p.chunk >= 2 * NW * kTileTokens)
          hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepOneChunks, false, true, true>), grid,
                             block, 0, s, p);
        else
          hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepOneChunks, false, false, true>), grid,
                             block, 0, s, p);
        return hipGetLastError();
      }
    }
    // two or more tiles per wave: request the second tile with the first
    if (p.chunk >= 2 * NW * kTileTokens)
      hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepOneChunks, false, true>), grid, block, 0,
                         s, p);
    else
      hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepOneChunks>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  if (mode == kPartialsCombine) {
    if (p.chunk >= 2 * NW * kTileTokens)
      hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kPartialsCombine, false, true>), grid, block,
                         0, s, p);
    else
      hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kPartialsCombine>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  if (mode == kStepTwoLevel) {
    if (p.chunk >= 2 * NW * kTileTokens)
      hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepTwoLevel, false, true>), grid, block, 0,
                         s, p);
    else
      hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kStepTwoLevel>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  if (p.nchunks >= 2 && p.chunk >= 2 * NW * kTileTokens)  // split, two or more tiles per wave
    hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kPartialsOnly, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_kernel<T, D, NW, kPartialsOnly>), grid, block, 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mode == kStepLaunches && p.nchunks >= 2) {  // chunk combine and merge in one launch
    const dim3 rgrid((unsigned)((int64_t)p.B * p.Hq));
    const int64_t ws_o_bytes = (int64_t)p.units * p.nchunks * p.Gb * D * 4;
    const int64_t opart_bytes = (int64_t)p.R * p.B * p.Hq * D * (p.odt == kF32 ? 4 : 2);
    switch (row_merge_waves(p.R, p.nchunks, D, ws_o_bytes, opart_bytes)) {
      case 2: hipLaunchKernelGGL((row_merge_kernel<D, 2>), rgrid, dim3(128), 0, s, p); return hipGetLastError();
      case 4: hipLaunchKernelGGL((row_merge_kernel<D, 4>), rgrid, dim3(256), 0, s, p); return hipGetLastError();
      case 8: hipLaunchKernelGGL((row_merge_kernel<D, 8>), rgrid, dim3(512), 0, s, p); return hipGetLastError();
      default: break;
    }
  }
  if (p.nchunks >= 2) {
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)units), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mode == kStepLaunches)  // the cross-shard merge reads o_part
    return launch_lse_merge(p.o_part, p.lse_part, p.R, (int64_t)p.B * p.Hq, D, p.odt, p.out_dt,
                            p.out, p.lse_out, s);
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_w(const AttnParams& p, int waves, int64_t units, StepMode mode, hipStream_t s) {
  switch (waves) {
    case 1: return launch_typed<T, D, 1>(p, units, mode, s);
    case 2: return launch_typed<T, D, 2>(p, units, mode, s);
    case 4: return launch_typed<T, D, 4>(p, units, mode, s);
    case 8: return launch_typed<T, D, 8>(p, units, mode, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const AttnParams& p, int D, int waves, int64_t units, StepMode mode,
                    hipStream_t s) {
  switch (D) {
    case 64: return launch_w<T, 64>(p, waves, units, mode, s);
    case 128: return launch_w<T, 128>(p, waves, units, mode, s);
    case 256: return launch_w<T, 256>(p, waves, units, mode, s);
  }
  return hipErrorInvalidValue;
}

#if !defined(CPDEC_ATTN_TYPE) || CPDEC_ATTN_TYPE == 2
__global__ void clear_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ void clear_tail_kernel(unsigned char* q, size_t n) {
  if (threadIdx.x < n) q[threadIdx.x] = 0;
}
#endif

}  // namespace

// The build compiles this file once per element type (CPDEC_ATTN_TYPE = 2:
// bf16 with the type dispatch and the clear kernels, 1: fp16) into separate
// objects, in parallel; without the macro the file holds everything.
#if !defined(CPDEC_ATTN_TYPE) || CPDEC_ATTN_TYPE == 2
hipError_t launch_attn_partial_bf16(const AttnParams& p, int D, int waves, int64_t units,
                                    StepMode mode, hipStream_t s) {
  return launch_d<bf16_t>(p, D, waves, units, mode, s);
}
#endif
#if !defined(CPDEC_ATTN_TYPE) || CPDEC_ATTN_TYPE == 1
hipError_t launch_attn_partial_f16(const AttnParams& p, int D, int waves, int64_t units,
                                   StepMode mode, hipStream_t s) {
  return launch_d<f16_t>(p, D, waves, units, mode, s);
}
#endif
#if !defined(CPDEC_ATTN_TYPE) || CPDEC_ATTN_TYPE == 2
hipError_t launch_attn_partial(const AttnParams& p, int qkv_dt, int D, int waves, int64_t units,
                               StepMode mode, hipStream_t s) {
  if (qkv_dt == kBF16) return launch_attn_partial_bf16(p, D, waves, units, mode, s);
  if (qkv_dt == kF16) return launch_attn_partial_f16(p, D, waves, units, mode, s);
  return hipErrorInvalidValue;
}

hipError_t launch_clear(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 > 0) {
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<u32x4*>(ptr), n16);
  }
  const size_t tail = bytes - n16 * 16;
  if (tail > 0)  // < 16 trailing bytes; a kernel, so nothing here records a memset node
    hipLaunchKernelGGL(clear_tail_kernel, dim3(1), dim3(64), 0, s,
                       static_cast<unsigned char*>(ptr) + n16 * 16, tail);
  return hipGetLastError();
}
#endif

}  // namespace cpdec
