// lse_merge.hip -- fused LSE merge of R partial outputs (gfx950).
//
// Method: page "FlashInfer's Context-Parallel Decode optimisation: Fused A2A
// + LSE Reduce" (flashinfer PR #4929), section "Code analysis, 1. Fused
// kernel": each output row is the sum over shards of o_r weighted by
// e^{lse_r - max lse}, divided by the sum of the weights, accumulated in FP32
// and converted to FP16/BF16; the merged lse is max lse + ln(sum of weights).
//
// Design (HBM-streaming, ~0.5 flop/byte, no MFMA):
//   * One row group of GS lanes per output row; each lane owns 16-byte
//     vectors of the row (D=512 bf16: one wave per row, one 16-byte load per
//     lane per shard; D=128 fp32: two rows per wave).
//   * Weights are formed in FP64 so the merged lse keeps ~1e-7 relative
//     accuracy even when it cancels towards 0.  Lane j of a row group computes
//     the one exp of shard j and the weights reach the other lanes by shuffles;
//     the weight sum (FP64) and the o sum (FP32) run in shard order, and the
//     division by the weight sum is applied once at the end.
//   * Shards with lse = -inf are skipped before their row is loaded: their
//     bytes are never read and any garbage/NaN in them cannot leak.
//   * Loads of a batch of 8 shards are issued back to back before any use so
//     8 x 16 bytes per lane are in flight.  For R <= 8 a persistent,
//     software-pipelined form overlaps the next row's lse fetch with this
//     row's partial loads; larger R uses one wave per row and batches of 8.
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

constexpr int kMergeWaves = 4;
constexpr int kBatch = 8;  // shards whose loads are in flight together

template <typename Tin, typename Tout, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_kernel(
    const Tin* __restrict__ o, const float* __restrict__ lse, int R, int64_t rows,
    Tout* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int VEC = InVec<Tin>::N;       // elements per 16-byte load
  constexpr int NV = D / VEC;              // 16-byte vectors per row
  constexpr int GS = NV < 64 ? NV : 64;    // lanes per row
  constexpr int RPW = 64 / GS;             // rows per wave
  constexpr int VPL = NV / GS;             // vectors per lane
  static_assert(NV % GS == 0 && 64 % GS == 0 && GS >= kBatch, "row split");

  const int lane = threadIdx.x & 63;
  const int64_t row_raw = ((int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6)) * RPW + lane / GS;
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;  // idle lanes shadow a real row
  const int li = lane % GS;
  const int base = lane - li;                      // first lane of this row group
  const float* lrow = lse + row;

  // Row max over shards: lane li reads shards li, li+GS, ..., then the group reduces.
  float M = neg_inf();
  for (int r = li; r < R; r += GS) M = fmaxf(M, lrow[(int64_t)r * rows]);
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

  const Tin* obase = o + row * D + li * VEC;
  for (int rb = 0; rb < R; rb += GS) {
    // one FP64 exp per lane: lane li owns shard rb + li of this block
    const int rl = rb + li;
    const float lme = (rl < R) ? lrow[(int64_t)rl * rows] : neg_inf();
    const double eme = (lme != neg_inf()) ? exp((double)lme - Md) : 0.0;
    const int nb = min(GS, R - rb);
    for (int j0 = 0; j0 < nb; j0 += kBatch) {
      double e[kBatch];
      u32x4 raw[kBatch][VPL];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int src = base + ((j0 + j) < nb ? (j0 + j) : 0);
        e[j] = (j0 + j < nb) ? __shfl(eme, src) : 0.0;
        if (e[j] != 0.0) {  // empty shards (and weights below FP64 range) are never read
          const Tin* sp = obase + (int64_t)(rb + j0 + j) * rows * D;
#pragma unroll
          for (int v = 0; v < VPL; ++v) raw[j][v] = ld16(sp + v * GS * VEC);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (e[j] == 0.0) continue;
        S += e[j];
        const float wj = (float)e[j];
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

// Pipelined form for R <= kBatch (every shard's 16-byte vectors in flight
// together): persistent waves walk rows with a stride; while the partial rows
// of row k are loading, the lse values of row k+1 are already requested, so a
// row costs one memory round trip.  Lane li of a row group owns shard li's lse
// and its FP64 exp; shuffles hand the values to the other lanes.
template <typename Tin, typename Tout, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_pipelined_kernel(
    const Tin* __restrict__ o, const float* __restrict__ lse, int R, int64_t rows,
    Tout* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int VEC = InVec<Tin>::N;
  constexpr int NV = D / VEC;
  constexpr int GS = NV < 64 ? NV : 64;
  constexpr int RPW = 64 / GS;
  constexpr int VPL = NV / GS;
  static_assert(GS >= kBatch, "a row group must hold one lane per shard");

  const int lane = threadIdx.x & 63;
  const int li = lane % GS;
  const int base = lane - li;
  const int64_t step = (int64_t)gridDim.x * kMergeWaves * RPW;
  int64_t wrow = ((int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6)) * RPW;

  float l_next = neg_inf();
  {
    const int64_t row = wrow + lane / GS;
    if (row < rows && li < R) l_next = lse[(int64_t)li * rows + row];
  }
  for (; wrow < rows; wrow += step) {
    const int64_t row = wrow + lane / GS;
    const bool valid = row < rows;
    const float l_own = l_next;

    // every shard's lse in every lane of the group; issue the live rows' loads
    float lj[kBatch];
    u32x4 raw[kBatch][VPL];
    const Tin* obase = o + (valid ? row : 0) * D + li * VEC;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      lj[j] = __shfl(l_own, base + j);
      if (j >= R) lj[j] = neg_inf();
      if (valid && lj[j] != neg_inf()) {
        const Tin* sp = obase + (int64_t)j * rows * D;
#pragma unroll
        for (int v = 0; v < VPL; ++v) raw[j][v] = ld16(sp + v * GS * VEC);
      }
    }
    // request the next row's lse while these loads are in flight
    {
      const int64_t nrow = row + step;
      l_next = (nrow < rows && li < R) ? lse[(int64_t)li * rows + nrow] : neg_inf();
    }

    float M = lj[0];
#pragma unroll
    for (int j = 1; j < kBatch; ++j) M = fmaxf(M, lj[j]);
    Tout* orow = out + (valid ? row : 0) * D;
    if (M == neg_inf()) {  // every shard empty
      if (valid) {
        float z[VEC] = {};
#pragma unroll
        for (int v = 0; v < VPL; ++v) store_vec<Tout, VEC>(orow + (v * GS + li) * VEC, z);
        if (lse_out != nullptr && li == 0) lse_out[row] = neg_inf();
      }
      continue;
    }
    const double Md = (double)M;
    const double e_own = (l_own != neg_inf() && li < R) ? exp((double)l_own - Md) : 0.0;
    double S = 0.0;
    float acc[VPL][VEC];
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[v][k] = 0.f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const double ej = __shfl(e_own, base + j);
      if (lj[j] == neg_inf() || ej == 0.0) continue;
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
    if (!valid) continue;
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
}

// Resident workgroups per CU x CUs for a kernel on the current device
// (queried once per device and kernel; a benign race recomputes the same value).
template <typename K>
int64_t resident_blocks(K kernel, int threads) {
  static int64_t cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
      return 1024;
    cache[dev] = (int64_t)cus * per_cu;
  }
  return cache[dev];
}

template <typename Tin, typename Tout, int D>
hipError_t launch_typed(const void* o, const float* lse, int R, int64_t rows, void* out,
                        float* lse_out, hipStream_t s) {
  constexpr int VEC = InVec<Tin>::N;
  constexpr int NV = D / VEC;
  constexpr int GS = NV < 64 ? NV : 64;
  constexpr int rows_per_block = kMergeWaves * (64 / GS);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks == 0) return hipSuccess;
  if (R <= kBatch) {
    auto kern = lse_merge_pipelined_kernel<Tin, Tout, D>;
    int64_t grid = resident_blocks(kern, kMergeWaves * 64);
    if (grid > blocks) grid = blocks;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMergeWaves * 64), 0, s,
                       static_cast<const Tin*>(o), lse, R, rows, static_cast<Tout*>(out), lse_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((lse_merge_kernel<Tin, Tout, D>), dim3((unsigned)blocks),
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
