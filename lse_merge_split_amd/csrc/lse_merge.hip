// lse_merge.hip -- fused LSE merge of R partial outputs (gfx950).
//
// Method: page "FlashInfer's Context-Parallel Decode optimisation: Fused A2A
// + LSE Reduce" (flashinfer PR #4929), section "Code analysis, 1. Fused
// kernel": each output row is the sum over shards of o_r weighted by
// e^{lse_r - max lse}, divided by the sum of the weights, accumulated in FP32
// and converted to FP16/BF16; the merged lse is max lse + ln(sum of weights).
//
// Design (HBM-streaming, ~0.5 flop/byte, no MFMA):
//   * One row group of GS lanes per output row, one output row per group and
//     no persistence: a wave lives for one lse round trip and one round trip
//     for the partial rows, so many waves fit on a CU and hide the latency
//     (persistent, software-pipelined forms measured no faster: this access
//     pattern runs at the memory system's limit for 8 strided read streams
//     plus a write stream).  Each lane owns 16-byte vectors of the row (D=512
//     16-bit: one wave per row, one 16-byte load per lane per shard).
//   * Weights are formed in FP64 so the merged lse keeps ~1e-7 relative
//     accuracy even when it cancels towards 0.  Lane j computes the one exp of
//     shard j while the partial rows load; shuffles (or readlane when a wave
//     holds one row) hand the weights to the other lanes.  The weight sum
//     (FP64) and the o sum (FP32) run in shard order, and the division by the
//     weight sum is applied once at the end.
//   * Shards with lse = -inf are skipped before their row is loaded: the load
//     is given an offset outside its buffer resource, which returns zeros
//     without touching memory, so their bytes are never read and garbage/NaN
//     in them cannot leak.
//   * Partial rows are read through buffer loads with the non-temporal
//     (streaming) policy, in batches of shards whose 16-byte loads are in
//     flight together (8 shards per batch for a row per wave or R > 32; 2 or
//     4 for rows of several per wave, where a smaller register set lets more
//     waves share a SIMD).
#include "device_common.h"
#include "kernels.h"

namespace cpdec {
namespace {

template <typename T> struct InVec;
template <> struct InVec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void cvt(u32x4 w, float* x) {
    x[0] = __uint_as_float(w[0]); x[1] = __uint_as_float(w[1]);
    x[2] = __uint_as_float(w[2]); x[3] = __uint_as_float(w[3]);
  }
};
template <typename T16> struct InVec16 {
  static constexpr int N = 8;
  static __device__ __forceinline__ void cvt(u32x4 w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = lo_of<T16>(w[i]); x[2 * i + 1] = hi_of<T16>(w[i]); }
  }
};
template <> struct InVec<bf16_t> : InVec16<bf16_t> {};
template <> struct InVec<f16_t> : InVec16<f16_t> {};

// Store N floats (N = 4 or 8) as Tout.
template <typename Tout, int N> __device__ __forceinline__ void store_vec(Tout* p, const float* x);
template <> __device__ __forceinline__ void store_vec<float, 4>(float* p, const float* x) {
  f32x4 v = {x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p) = v;
}
template <> __device__ __forceinline__ void store_vec<float, 8>(float* p, const float* x) {
  store_vec<float, 4>(p, x);
  store_vec<float, 4>(p + 4, x + 4);
}
template <typename T16, int N> __device__ __forceinline__ void store_vec16(T16* p, const float* x) {
  if constexpr (N == 8) {
    u32x4 v = {pack2<T16>(x[0], x[1]), pack2<T16>(x[2], x[3]), pack2<T16>(x[4], x[5]),
               pack2<T16>(x[6], x[7])};
    st16(p, v);
  } else {
    u32x2 v = {pack2<T16>(x[0], x[1]), pack2<T16>(x[2], x[3])};
    *reinterpret_cast<u32x2*>(p) = v;
  }
}
template <> __device__ __forceinline__ void store_vec<bf16_t, 4>(bf16_t* p, const float* x) { store_vec16<bf16_t, 4>(p, x); }
template <> __device__ __forceinline__ void store_vec<bf16_t, 8>(bf16_t* p, const float* x) { store_vec16<bf16_t, 8>(p, x); }
template <> __device__ __forceinline__ void store_vec<f16_t, 4>(f16_t* p, const float* x) { store_vec16<f16_t, 4>(p, x); }
template <> __device__ __forceinline__ void store_vec<f16_t, 8>(f16_t* p, const float* x) { store_vec16<f16_t, 8>(p, x); }

constexpr int kMergeWaves = 8;  // 512-thread workgroups (measured faster than 4 or 16 waves)
constexpr int kBatch = 8;  // shards whose loads are in flight together

// One row per row group, non-persistent (a wave's whole life is one memory
// round trip for the lse values and one for the partial rows, so many waves
// fit on a CU).  Lane li of a row group owns shards li, li + GS, ...: it
// loads their lse, the group takes the max, then every live shard's row is
// requested before the FP64 exps are computed, so the arithmetic overlaps the
// loads.  Batches of KB shards keep KB x 16 bytes per lane in flight: KB = 2
// for R <= 2, 4 for R <= 32, else 8.  The smaller register sets let more waves
// share a SIMD (8 at KB = 2, 4 at KB = 8), which is what hides the latency
// when each wave carries little data (65,536 rows, D = 128: R = 2 19.9 ->
// 12.8 us, R = 8 33.3 -> 30.3 us; R = 64 measured 2% slower with KB = 4).
template <typename Tin, typename Tout, int D, int KB>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_kernel(
    const Tin* __restrict__ o, const float* __restrict__ lse, int R, int64_t rows,
    Tout* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int VEC = InVec<Tin>::N;       // elements per 16-byte load
  constexpr int NV = D / VEC;              // 16-byte vectors per row
  constexpr int GS = NV < 64 ? NV : 64;    // lanes per row
  constexpr int RPW = 64 / GS;             // rows per wave
  constexpr int VPL = NV / GS;             // vectors per lane
  static_assert(NV % GS == 0 && 64 % GS == 0 && GS >= KB, "row split");

  const int lane = threadIdx.x & 63;
  const int64_t row_raw = ((int64_t)blockIdx.x * kMergeWaves + wave_id()) * RPW + lane / GS;
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;  // idle lanes shadow a real row
  const int li = lane % GS;
  const int base = lane - li;
  const rsrc_t lrs = make_rsrc(lse, (uint32_t)((int64_t)R * rows * sizeof(float)));
  const uint32_t roff = (uint32_t)(row * D * sizeof(Tin)) + (uint32_t)(li * 16);

  // Row max over shards: lane li reads shards li, li+GS, ..., then the group
  // reduces.  The first block's value is kept for the weights (one load).
  const float l_first = (li < R) ? buf4f(lrs, (uint32_t)(((int64_t)li * rows + row) * 4)) : neg_inf();
  float M = l_first;
  for (int r = li + GS; r < R; r += GS) M = fmaxf(M, buf4f(lrs, (uint32_t)(((int64_t)r * rows + row) * 4)));
#pragma unroll
  for (int off = GS / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, GS));

  Tout* orow = out + row * D;
  if (M == neg_inf()) {  // every shard empty: out = 0, lse = -inf
    if (valid) {
      float z[VEC] = {};
#pragma unroll
      for (int v = 0; v < VPL; ++v) store_vec<Tout, VEC>(orow + (v * GS + li) * VEC, z);
      if (lse_out != nullptr && li == 0) lse_out[row] = neg_inf();
    }
    return;
  }

  const double Md = (double)M;
  double S = 0.0;  // weight sum, accumulated in shard order
  float acc[VPL][VEC];
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[v][e] = 0.f;

  for (int rb = 0; rb < R; rb += GS) {
    // lane li owns shard rb + li of this block (its lse is cached from above)
    const int rl = rb + li;
    const float lme = rb == 0 ? l_first
                              : (rl < R) ? buf4f(lrs, (uint32_t)(((int64_t)rl * rows + row) * 4)) : neg_inf();
    const int nb = min(GS, R - rb);
    for (int j0 = 0; j0 < nb; j0 += KB) {
      float lj[KB];
      u32x4 raw[KB][VPL];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const float l = __shfl(lme, base + min(j0 + j, nb - 1));
        lj[j] = (j0 + j < nb) ? l : neg_inf();
        // an empty shard's row is never read: its offset is out of range (zeros)
        const rsrc_t ors = make_rsrc(o + (int64_t)(rb + min(j0 + j, nb - 1)) * rows * D,
                                     (uint32_t)(rows * D * sizeof(Tin)));
        const uint32_t off = (lj[j] != neg_inf()) ? roff : kOutOfRange;
#pragma unroll
        for (int v = 0; v < VPL; ++v) raw[j][v] = buf16_stream(ors, off + (uint32_t)(v * GS * 16));
      }
      // the exps of this batch's shards, computed while the rows load
      const double e_own = (lme != neg_inf()) ? exp((double)lme - Md) : 0.0;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const double ej = __shfl(e_own, base + min(j0 + j, nb - 1));
        if (lj[j] == neg_inf() || ej == 0.0) continue;  // never read, never used
        S += ej;
        const float wj = (float)ej;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          float x[VEC];
          InVec<Tin>::cvt(raw[j][v], x);
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[v][k] = fmaf(wj, x[k], acc[v][k]);
        }
      }
    }
  }

  if (!valid) return;
  const float inv = (float)(1.0 / S);
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    float y[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) y[k] = acc[v][k] * inv;
    store_vec<Tout, VEC>(orow + (v * GS + li) * VEC, y);
  }
  if (lse_out != nullptr && li == 0) lse_out[row] = (float)(Md + log(S));
}

// R <= kBatch and a whole wave per row (e.g. D = 512 in 16-bit types): the
// row index is wave-uniform, so the lse values arrive through scalar loads
// (scalar cache; the vector memory pipe carries only the partial rows), lane
// j computes shard j's FP64 exp and readlane makes every weight uniform.
template <typename Tin, typename Tout, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_wave_row_kernel(
    const Tin* __restrict__ o, const float* __restrict__ lse, int R, int64_t rows,
    Tout* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int VEC = InVec<Tin>::N;
  constexpr int NV = D / VEC;
  constexpr int VPL = NV / 64;
  static_assert(NV % 64 == 0, "one wave per row");
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + wave_id();  // wave-uniform
  if (row >= rows) return;

  float lj[kBatch];
  float M = neg_inf();
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    lj[j] = (j < R) ? lse[(int64_t)j * rows + row] : neg_inf();  // scalar loads
    M = fmaxf(M, lj[j]);
  }
  Tout* orow = out + row * D;
  if (M == neg_inf()) {  // every shard empty
    float z[VEC] = {};
#pragma unroll
    for (int v = 0; v < VPL; ++v) store_vec<Tout, VEC>(orow + (v * 64 + lane) * VEC, z);
    if (lse_out != nullptr && lane == 0) lse_out[row] = neg_inf();
    return;
  }
  const uint32_t roff = (uint32_t)(row * D * sizeof(Tin)) + (uint32_t)(lane * 16);
  u32x4 raw[kBatch][VPL];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const rsrc_t ors = make_rsrc(o + (int64_t)(j < R ? j : 0) * rows * D, (uint32_t)(rows * D * sizeof(Tin)));
    // an empty shard's row is never read: its offset is out of range (zeros)
    const uint32_t off = (lj[j] != neg_inf()) ? roff : kOutOfRange;
#pragma unroll
    for (int v = 0; v < VPL; ++v) raw[j][v] = buf16_stream(ors, off + (uint32_t)(v * 64 * 16));
  }
  // lane j: shard j's weight in FP64, while the rows load
  float lmine = neg_inf();
#pragma unroll
  for (int j = 0; j < kBatch; ++j) lmine = (lane == j) ? lj[j] : lmine;
  const double Md = (double)M;
  const double e_mine = (lmine != neg_inf()) ? exp((double)lmine - Md) : 0.0;
  double S = 0.0;
  float acc[VPL][VEC];
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[v][k] = 0.f;
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const double ej = __builtin_bit_cast(
        double, ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane(
                     (int)(__builtin_bit_cast(unsigned long long, e_mine) >> 32), j) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane(
                        (int)__builtin_bit_cast(unsigned long long, e_mine), j));
    if (lj[j] == neg_inf() || ej == 0.0) continue;  // uniform branch
    S += ej;
    const float wj = (float)ej;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      float x[VEC];
      InVec<Tin>::cvt(raw[j][v], x);
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[v][k] = fmaf(wj, x[k], acc[v][k]);
    }
  }
  const float inv = (float)(1.0 / S);
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    float y[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) y[k] = acc[v][k] * inv;
    store_vec<Tout, VEC>(orow + (v * 64 + lane) * VEC, y);
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = (float)(Md + log(S));
}

template <typename Tin, typename Tout, int D>
hipError_t launch_typed(const void* o, const float* lse, int R, int64_t rows, void* out,
                        float* lse_out, hipStream_t s) {
  constexpr int VEC = InVec<Tin>::N;
  constexpr int NV = D / VEC;
  if constexpr (NV % 64 == 0) {
    if (R <= kBatch) {  // a whole wave per row: scalar lse loads
      const int64_t blocks = (rows + kMergeWaves - 1) / kMergeWaves;
      hipLaunchKernelGGL((lse_merge_wave_row_kernel<Tin, Tout, D>), dim3((unsigned)blocks),
                         dim3(kMergeWaves * 64), 0, s, static_cast<const Tin*>(o), lse, R, rows,
                         static_cast<Tout*>(out), lse_out);
      return hipGetLastError();
    }
  }
  constexpr int GS = NV < 64 ? NV : 64;
  constexpr int rows_per_block = kMergeWaves * (64 / GS);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (R <= 2)
    hipLaunchKernelGGL((lse_merge_kernel<Tin, Tout, D, 2>), dim3((unsigned)blocks),
                       dim3(kMergeWaves * 64), 0, s, static_cast<const Tin*>(o), lse, R, rows,
                       static_cast<Tout*>(out), lse_out);
  else if (R <= 32)
    hipLaunchKernelGGL((lse_merge_kernel<Tin, Tout, D, 4>), dim3((unsigned)blocks),
                       dim3(kMergeWaves * 64), 0, s, static_cast<const Tin*>(o), lse, R, rows,
                       static_cast<Tout*>(out), lse_out);
  else
    hipLaunchKernelGGL((lse_merge_kernel<Tin, Tout, D, kBatch>), dim3((unsigned)blocks),
                       dim3(kMergeWaves * 64), 0, s, static_cast<const Tin*>(o), lse, R, rows,
                       static_cast<Tout*>(out), lse_out);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_d(const void* o, const float* lse, int R, int64_t rows, int D, void* out,
                    float* lse_out, hipStream_t s) {
  switch (D) {
    case 64: return launch_typed<Tin, Tout, 64>(o, lse, R, rows, out, lse_out, s);
    case 128: return launch_typed<Tin, Tout, 128>(o, lse, R, rows, out, lse_out, s);
    case 256: return launch_typed<Tin, Tout, 256>(o, lse, R, rows, out, lse_out, s);
    case 512: return launch_typed<Tin, Tout, 512>(o, lse, R, rows, out, lse_out, s);
  }
  return hipErrorInvalidValue;
}

template <typename Tin>
hipError_t launch_out(const void* o, const float* lse, int R, int64_t rows, int D, int out_dt,
                      void* out, float* lse_out, hipStream_t s) {
  switch (out_dt) {
    case kF32: return launch_d<Tin, float>(o, lse, R, rows, D, out, lse_out, s);
    case kF16: return launch_d<Tin, f16_t>(o, lse, R, rows, D, out, lse_out, s);
    case kBF16: return launch_d<Tin, bf16_t>(o, lse, R, rows, D, out, lse_out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int64_t lse_merge_max_blocks(int64_t rows, int D, int in_dt) {
  const int vec = in_dt == kF32 ? 4 : 8;
  const int nv = D / vec;
  const int gs = nv < 64 ? nv : 64;
  const int rows_per_block = kMergeWaves * (64 / gs);
  return (rows + rows_per_block - 1) / rows_per_block;
}

hipError_t launch_lse_merge(const void* o, const float* lse, int R, int64_t rows, int D,
                            int in_dt, int out_dt, void* out, float* lse_out, hipStream_t s) {
  switch (in_dt) {
    case kF32: return launch_out<float>(o, lse, R, rows, D, out_dt, out, lse_out, s);
    case kF16: return launch_out<f16_t>(o, lse, R, rows, D, out_dt, out, lse_out, s);
    case kBF16: return launch_out<bf16_t>(o, lse, R, rows, D, out_dt, out, lse_out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace cpdec
