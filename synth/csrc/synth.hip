// synth.hip -- GPU twin of synth/philox.py: fills device tensors from the
// seeded counter-based streams.  Holds no attention or merge arithmetic.
//
// Definition (identical to the CPU side): Philox4x32-10 (Salmon, Moraes,
// Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) with key
// (seed, tag) and counter (block lo, block hi, 0, 0); element i is word i%4 of
// block i/4; normals by Box-Muller in float64 on word pairs (0,1) and (2,3),
// rounded to float32, optionally scaled in float32, then rounded to the
// storage type (round to nearest even).  Built with -ffp-contract=off so every
// operation rounds exactly as the numpy twin does.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0;
    const uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void fill_normal_kernel(void* dst, int dtype, uint64_t count, uint64_t start,
                                   uint32_t seed, uint32_t tag, float scale) {
  const uint64_t fb = start / 4;
  const uint64_t nblocks = (start + count + 3) / 4 - fb;
  const double kInv232 = 2.3283064365386963e-10;  // 2^-32
  const double kTwoPi = 6.283185307179586;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblocks;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t blk = fb + i;
    uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
    philox4x32_10(c, seed, tag);
    float z[4];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const double u1 = ((double)c[2 * pr] + 1.0) * kInv232;
      const double u2 = (double)c[2 * pr + 1] * kInv232;
      const double rad = sqrt(-2.0 * log(u1));
      const double ang = kTwoPi * u2;
      z[2 * pr] = (float)(rad * cos(ang));
      z[2 * pr + 1] = (float)(rad * sin(ang));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t e = 4 * blk + j;
      if (e < start || e >= start + count) continue;
      const float v = (scale != 1.0f) ? z[j] * scale : z[j];
      const uint64_t o = e - start;
      if (dtype == 0) static_cast<float*>(dst)[o] = v;
      else if (dtype == 1) static_cast<_Float16*>(dst)[o] = (_Float16)v;
      else static_cast<uint16_t*>(dst)[o] = f32_to_bf16_rne(v);
    }
  }
}

}  // namespace

extern "C" {

// dst: device buffer of `count` elements of dtype (0 f32, 1 f16, 2 bf16);
// element o receives stream element (start + o).  Returns a hipError_t code.
int synth_fill_normal(void* dst, int dtype, uint64_t count, uint64_t start, uint32_t seed,
                      uint32_t tag, float scale, void* stream) {
  if (count == 0) return 0;
  if (dst == nullptr || dtype < 0 || dtype > 2) return (int)hipErrorInvalidValue;
  const uint64_t nblocks = (start + count + 3) / 4 - start / 4;
  uint64_t grid = (nblocks + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(fill_normal_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dst, dtype, count, start, seed, tag, scale);
  return (int)hipGetLastError();
}

}  // extern "C"
