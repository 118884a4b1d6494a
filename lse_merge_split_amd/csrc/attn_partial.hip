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
//   computes tile i.  The waves' states are merged through LDS.  A unit whose
//   tokens fit one chunk is written straight to o_part/lse_part; otherwise each
//   chunk writes a normalised partial to the workspace and a second, small
//   kernel merges the chunks of every unit -- both merges use the same LSE
//   weighting as the cross-shard merge, which the page's merge formula makes
//   exact.  No workgroup waits on another inside a kernel: on gfx950 a
//   device-scope release/acquire pair writes back and invalidates the L2 of
//   the XCD, which costs more than a second launch.
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

// Load 4 consecutive values of dtype `odt` as fp32.
__device__ __forceinline__ f32x4 load4(const void* base, int64_t idx, int odt) {
  if (odt == kF32) return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + idx);
  if (odt == kBF16) return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  return f32x4{f16_lo(w[0]), f16_hi(w[0]), f16_lo(w[1]), f16_hi(w[1])};
}

template <int D, int NW>
struct Smem {
  static constexpr int NB = (D / 8 + 15) / 16;
  f32x4 acc[NW > 1 ? NW - 1 : 1][NB * 8][64];
  float m[NW][16];
  float l[NW][16];
};

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_partial_kernel(const AttnParams p) {
  constexpr int NCH = D / 8;           // 16-byte chunks per token row
  constexpr int NB = (NCH + 15) / 16;  // 16-chunk row blocks of the PV product
  constexpr int KS = D / 32;           // k-steps of the QK product
  __shared__ Smem<D, NW> sm;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  // Chunk-major order: workgroups are dealt to the 8 XCDs round-robin by
  // block index, so block % 8 must not correlate with the chunk index (the
  // later chunks of ragged shards are mostly empty); here it follows the unit.
  const int c = blockIdx.x / p.units;
  const int unit = blockIdx.x % p.units;
  int u = unit;
  const int gb = u % p.gblocks; u /= p.gblocks;
  const int h = u % p.Hkv; u /= p.Hkv;
  const int b = u % p.B;
  const int r = u / p.B;

  const int L = p.lens[r * p.B + b];
  const int t_begin = c * p.chunk;
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int hq0 = h * p.G + g0;
  const int64_t orow0 = ((int64_t)r * p.B + b) * p.Hq + hq0;  // o_part/lse_part row of head g0

  if (t_begin >= L) {
    if (c == 0) {  // empty shard: o_r = 0, lse_r = -inf
      for (int e = threadIdx.x; e < ng * (D / 4); e += NW * 64)
        store4(p.o_part, orow0 * D + 4 * e, f32x4{0.f, 0.f, 0.f, 0.f}, p.odt);
      if (threadIdx.x < ng) p.lse_part[orow0 + threadIdx.x] = neg_inf();
    }
    return;
  }
  const int t_end = min(L, t_begin + p.chunk);
  const int nlive = (L + p.chunk - 1) / p.chunk;

  // Q operand (B of S^T = K Q^T): lane (q4, g = l16) holds Q[g][32 s + 8 q4 .. +8].
  u32x4 qop[KS];
  {
    const T* qrow = static_cast<const T*>(p.q) + ((int64_t)b * p.Hq + hq0 + l16) * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[s] = (l16 < ng) ? ld16(qrow + 32 * s) : u32x4{0u, 0u, 0u, 0u};
  }

  const T* kb = static_cast<const T*>(p.k[r]) + b * p.sb + h * p.sh;
  const T* vb = static_cast<const T*>(p.v[r]) + b * p.sb + h * p.sh;
  const int64_t st = p.st;

  float m = neg_inf();  // running max (base-2 units), uniform over q4
  float lsum = 0.f;     // this lane's share of the exp-sum
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
  const uint32_t span = (uint32_t)(((int64_t)(t_end - 1) * st + D) * sizeof(T));
  const rsrc_t krs = make_rsrc(kb, span);
  const rsrc_t vrs = make_rsrc(vb, span);
  const uint32_t rowb = (uint32_t)(st * sizeof(T));  // bytes per token row
  auto load_tile = [&](int t0, u32x4 (&kr)[2][KS], u32x4 (&vr)[NB][8]) {
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

  u32x4 kr[2][KS], vr[NB][8];
  int t0 = t_begin + wave * kTileTokens;
  load_tile(t0, kr, vr);
  for (; t0 < t_end; t0 += NW * kTileTokens) {
    // prefetch the wave's next tile while this one is computed
    u32x4 krn[2][KS], vrn[NB][8];
    load_tile(t0 + NW * kTileTokens, krn, vrn);

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
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);  // finite: the tile holds >= 1 live token
    const float alpha = exp2f(m - m_new);
    // rescale the accumulators only when some head's running max grew
    // (rare after the first tiles); the branch is wave-uniform and holds no loads
    const bool grew = __any(m_new > m);
    m = m_new;
    float pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pr[j] = exp2f(x[j >> 2][j & 3] - m_new);
    float ps = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    lsum = lsum * alpha + ps;

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
        f32x4 a = grew ? acc[nb][n] * alpha : acc[nb][n];
        a = mfma16x16x32<T>(va, phi, a);
        acc[nb][n] = mfma16x16x32<T>(va, plo, a);
      }
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s = 0; s < KS; ++s) kr[blk][s] = krn[blk][s];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[nb][j] = vrn[nb][j];
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

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
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int d0 = 8 * (16 * nb + 4 * q4);
        if (d0 >= D) continue;
        float y[32];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int n = 0; n < 8; ++n) y[8 * i + n] = acc[nb][n][i] * inv_l;
        store32(p.o_part, (orow0 + l16) * D + d0, y, p.odt);
      }
      if (q4 == 0) p.lse_part[orow0 + l16] = lse_nat;
    }
    return;
  }

  // ---- several live chunks: this chunk's normalised partial to the workspace ----
  const int64_t slot = (int64_t)unit * p.nchunks + c;
  if (wave == 0 && l16 < ng) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int d0 = 8 * (16 * nb + 4 * q4);
      if (d0 >= D) continue;
      float y[32];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 8; ++n) y[8 * i + n] = acc[nb][n][i] * inv_l;
      store32(p.ws_o, (slot * p.Gb + l16) * D + d0, y, kF32);
    }
    if (q4 == 0) p.ws_lse[slot * p.Gb + l16] = lse_nat;
  }
}

// Merge the chunk partials of every unit that has more than one live chunk
// (one 256-thread workgroup per unit), with the LSE weighting of the
// cross-shard merge.  Per-head statistics use wave reductions over chunks;
// the weighted sum splits the chunks over P thread groups when the unit has
// fewer than 256 float4 outputs, and the groups are added in a fixed order
// (results do not depend on timing).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnParams p) {
  __shared__ float w[kMaxChunks][16];
  __shared__ f32x4 part[256];
  const int unit = blockIdx.x;
  int u = unit;
  const int gb = u % p.gblocks; u /= p.gblocks;
  const int h = u % p.Hkv; u /= p.Hkv;
  const int b = u % p.B;
  const int r = u / p.B;
  const int L = p.lens[r * p.B + b];
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
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float S = 0.f;
    for (int cc = lane; cc < nlive; cc += 64) {
      const float e = expf(p.ws_lse[(slot0 + cc) * p.Gb + g] - M);
      w[cc][g] = e;
      S += e;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) S += __shfl_xor(S, off);
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

// The whole step's second launch, for one (sequence, kv head, head block)
// and all R shards at once: (1) per (shard, head) the chunk weights (wave
// reductions), (2) per (shard, output vector) the shard's partial -- merged
// from its chunks and written to o_part, or read back when the attention
// kernel wrote it (0 or 1 live chunk) -- kept in LDS, (3) the cross-shard
// merge in shard order (FP64 weights and lse, FP32 sums, -inf shards
// skipped) into out/lse_out.  Used when the per-shard state fits LDS
// (kFusedChunkSlots, kFusedVecs); otherwise the separate kernels run.
constexpr int kFusedChunkSlots = 512;  // R * chunks
constexpr int kFusedVecs = 1024;       // R * (heads * D / 4)

template <int D>
__global__ __launch_bounds__(256) void attn_combine_merge_kernel(const AttnParams p, void* out,
                                                                 float* lse_out, int out_dt) {
  __shared__ float w[kFusedChunkSlots][16];
  __shared__ f32x4 ybuf[kFusedVecs];
  __shared__ f32x4 part[256];
  __shared__ float s_lse[kMaxShards][16];
  __shared__ int s_nlive[kMaxShards];
  const int bh = blockIdx.x;  // ((b * Hkv) + h) * gblocks + gb
  const int gb = bh % p.gblocks;
  const int h = (bh / p.gblocks) % p.Hkv;
  const int b = bh / (p.gblocks * p.Hkv);
  const int g0 = gb * kGroupRows;
  const int ng = min(kGroupRows, p.G - g0);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int t = threadIdx.x;
  const int R = p.R;
  auto unit_of = [&](int r) { return ((r * p.B + b) * p.Hkv + h) * p.gblocks + gb; };
  auto orow_of = [&](int r) { return ((int64_t)r * p.B + b) * p.Hq + h * p.G + g0; };

  if (t < R) {
    const int L = p.lens[t * p.B + b];
    s_nlive[t] = (L + p.chunk - 1) / p.chunk;
  }
  __syncthreads();

  // (1) chunk weights and shard lse, one (shard, head) pair per wave in turn
  for (int pi = wave; pi < R * ng; pi += 4) {
    const int r = pi / ng, g = pi % ng;
    const int nlive = s_nlive[r];
    if (nlive < 2) {  // 0 or 1 live chunk: the attention kernel wrote lse_part
      if (lane == 0) s_lse[r][g] = p.lse_part[orow_of(r) + g];
      continue;
    }
    const int64_t slot0 = (int64_t)unit_of(r) * p.nchunks;
    float M = neg_inf();
    for (int cc = lane; cc < nlive; cc += 64) M = fmaxf(M, p.ws_lse[(slot0 + cc) * p.Gb + g]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float S = 0.f;
    for (int cc = lane; cc < nlive; cc += 64) {
      const float e = expf(p.ws_lse[(slot0 + cc) * p.Gb + g] - M);
      w[r * p.nchunks + cc][g] = e;
      S += e;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) S += __shfl_xor(S, off);
    const float invS = 1.0f / S;
    for (int cc = lane; cc < nlive; cc += 64) w[r * p.nchunks + cc][g] *= invS;
    if (lane == 0) {
      const float l = M + logf(S);
      p.lse_part[orow_of(r) + g] = l;
      s_lse[r][g] = l;
    }
  }
  __syncthreads();

  // (2) every shard's partial vectors (chunks split over P thread groups)
  constexpr int Q = D / 4;               // float4 outputs per head
  const int E = ng * Q;                  // float4 outputs per shard
  const int items = R * E;
  int P = 1;
  while (P < 8 && items * P * 2 <= 256) P *= 2;
  const int per = 256 / P;
  const int part_id = t / per;
  for (int i0 = 0; i0 < items; i0 += per) {
    const int it = i0 + t % per;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    int r = 0, e = 0, nlive = 0;
    if (it < items) {
      r = it / E;
      e = it % E;
      nlive = s_nlive[r];
      const int g = e / Q;
      if (nlive >= 2) {
        const int64_t slot0 = (int64_t)unit_of(r) * p.nchunks;
        const float* src = p.ws_o + (slot0 * p.Gb + g) * D + 4 * (e % Q);
        const int64_t cstride = (int64_t)p.Gb * D;
#pragma unroll 4
        for (int cc = part_id; cc < nlive; cc += P)
          y += w[r * p.nchunks + cc][g] * *reinterpret_cast<const f32x4*>(src + cc * cstride);
      } else if (nlive == 1 && part_id == 0) {
        y = load4(p.o_part, (orow_of(r) + g) * D + 4 * (e % Q), p.odt);
      }
    }
    if (P > 1) {
      part[t] = y;
      __syncthreads();
      if (part_id == 0 && it < items)
        for (int q = 1; q < P; ++q) y += part[t + q * per];
      __syncthreads();
    }
    if (part_id == 0 && it < items) {
      if (nlive >= 2) store4(p.o_part, (orow_of(r) + e / Q) * D + 4 * (e % Q), y, p.odt);
      ybuf[it] = y;
    }
  }
  __syncthreads();

  // (3) cross-shard merge in shard order
  for (int e = t; e < E; e += 256) {
    const int g = e / Q;
    float M = neg_inf();
    for (int r = 0; r < R; ++r) M = fmaxf(M, s_lse[r][g]);
    const int64_t row = (int64_t)b * p.Hq + h * p.G + g0 + g;
    if (M == neg_inf()) {
      store4(out, row * D + 4 * (e % Q), f32x4{0.f, 0.f, 0.f, 0.f}, out_dt);
      if (lse_out != nullptr && e % Q == 0) lse_out[row] = neg_inf();
      continue;
    }
    double S = 0.0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < R; ++r) {
      const float l = s_lse[r][g];
      if (l == neg_inf()) continue;  // empty shard: never used
      const double ew = exp((double)l - (double)M);
      S += ew;
      acc += (float)ew * ybuf[r * E + e];
    }
    store4(out, row * D + 4 * (e % Q), acc * (float)(1.0 / S), out_dt);
    if (lse_out != nullptr && e % Q == 0) lse_out[row] = (float)((double)M + log(S));
  }
}

template <typename T, int D, int NW>
hipError_t launch_typed(const AttnParams& p, int64_t units, const StepOut* so, hipStream_t s) {
  const int64_t blocks = units * p.nchunks;
  hipLaunchKernelGGL((attn_partial_kernel<T, D, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, s,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t fused_vecs = (int64_t)p.R * p.Gb * (D / 4);
  if (so != nullptr && p.nchunks >= 2 && (int64_t)p.R * p.nchunks <= kFusedChunkSlots &&
      fused_vecs <= kFusedVecs) {  // the whole step: chunk merge + shard merge fused
    hipLaunchKernelGGL((attn_combine_merge_kernel<D>), dim3((unsigned)(units / p.R)), dim3(256), 0,
                       s, p, so->out, so->lse_out, so->out_dt);
    return hipGetLastError();
  }
  if (p.nchunks >= 2) {
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)units), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (so != nullptr)  // the whole step, unsplit: the cross-shard merge reads o_part
    return launch_lse_merge(p.o_part, p.lse_part, p.R, (int64_t)p.B * p.Hq, D, p.odt, so->out_dt,
                            so->out, so->lse_out, s);
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_w(const AttnParams& p, int waves, int64_t units, const StepOut* so,
                    hipStream_t s) {
  switch (waves) {
    case 1: return launch_typed<T, D, 1>(p, units, so, s);
    case 2: return launch_typed<T, D, 2>(p, units, so, s);
    case 4: return launch_typed<T, D, 4>(p, units, so, s);
    case 8: return launch_typed<T, D, 8>(p, units, so, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const AttnParams& p, int D, int waves, int64_t units, const StepOut* so,
                    hipStream_t s) {
  switch (D) {
    case 64: return launch_w<T, 64>(p, waves, units, so, s);
    case 128: return launch_w<T, 128>(p, waves, units, so, s);
    case 256: return launch_w<T, 256>(p, waves, units, so, s);
  }
  return hipErrorInvalidValue;
}

__global__ void clear_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ void clear_tail_kernel(unsigned char* q, size_t n) {
  if (threadIdx.x < n) q[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_attn_partial(const AttnParams& p, int qkv_dt, int D, int waves, int64_t units,
                               const StepOut* so, hipStream_t s) {
  if (qkv_dt == kBF16) return launch_d<bf16_t>(p, D, waves, units, so, s);
  if (qkv_dt == kF16) return launch_d<f16_t>(p, D, waves, units, so, s);
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

}  // namespace cpdec
