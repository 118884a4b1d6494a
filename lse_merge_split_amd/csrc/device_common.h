// device_common.h -- small device helpers shared by the cpdec kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpdec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Storage tags: 16-bit element types are handled as raw bits.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Index of the calling wave in its workgroup, as a value the compiler knows
// to be wave-uniform (loops over it compile to scalar branches, not exec masks).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---- 16-bit <-> fp32 conversions ------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <typename T> __device__ __forceinline__ float lo_of(uint32_t w);
template <typename T> __device__ __forceinline__ float hi_of(uint32_t w);
template <> __device__ __forceinline__ float lo_of<bf16_t>(uint32_t w) { return bf16_lo(w); }
template <> __device__ __forceinline__ float hi_of<bf16_t>(uint32_t w) { return bf16_hi(w); }
template <> __device__ __forceinline__ float lo_of<f16_t>(uint32_t w) { return f16_lo(w); }
template <> __device__ __forceinline__ float hi_of<f16_t>(uint32_t w) { return f16_hi(w); }

// Two fp32 values -> one dword holding two 16-bit values (round to nearest
// even), element a in the low half.
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// ---- MFMA: D(16x16 f32) += A(16x32) * B(32x16) -----------------------------
// Operand layout (64 lanes): lane l supplies A[l % 16][8*(l/16) + j] and
// B[8*(l/16) + j][l % 16] for j = 0..7 (8 packed 16-bit values, j = 0 in the
// low half of the first dword); it receives D[4*(l/16) + i][l % 16], i = 0..3.
template <typename T> __device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma16x16x32<bf16_t>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16x16x32<f16_t>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Byte permute of the 8-byte value {hi:lo}: selector byte i picks result byte i.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
constexpr uint32_t kSelLoHalves = 0x05040100u;  // {lo16(hi), lo16(lo)}
constexpr uint32_t kSelHiHalves = 0x07060302u;  // {hi16(hi), hi16(lo)}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---- raw buffer loads ---------------------------------------------------
// A buffer resource covers [base, base + bytes); a load whose offset falls
// outside returns zeros without touching memory.  Streaming loads go through
// these intrinsics rather than plain pointer loads: the IR optimiser merges
// plain loads that feed a loop-carried phi into one load after the phi, which
// turns a software prefetch back into a load-then-wait; it leaves these alone.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kSrdConfig = 0x00020000;  // gfx9 raw buffer: 32-bit format, no swizzle
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past any range we build

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kSrdConfig);
}
// Cache-policy bits of a buffer load on gfx950: bit 1 = nt (non-temporal).
constexpr int kPolicyStream = 2;  // data read once: stream it through the caches
__device__ __forceinline__ u32x4 buf16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x4 buf16_stream(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyStream));
}
__device__ __forceinline__ float buf4f(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---- lane exchanges in VALU (no LDS crossbar) ------------------------------
// DPP within a 16-lane row: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at
// distance 1 and 2, the half-row mirror pairs lane i with 7-i and the row
// mirror lane i with 15-i; gfx950's permlane16/32 swaps exchange rows.  A
// butterfly of these over a commutative operation leaves the identical
// result in every lane of the group (each step pairs lanes symmetrically).
// Every lane of the wave must be active.
enum LaneStep : int { kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140 };
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// The two values that rows r and r ^ 1 (xor 16) or halves (xor 32) hold.
__device__ __forceinline__ f32x2 rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return f32x2{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
__device__ __forceinline__ f32x2 rows32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return f32x2{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpSum { __device__ float operator()(float a, float b) const { return a + b; } };
// Reduce over aligned groups of 2^levels lanes (levels 0..6).
template <typename Op>
__device__ __forceinline__ float lane_reduce(float x, int levels, Op op) {
  if (levels > 0) x = op(x, dpp<kXor1>(x));
  if (levels > 1) x = op(x, dpp<kXor2>(x));
  if (levels > 2) x = op(x, dpp<kHalfMirror>(x));
  if (levels > 3) x = op(x, dpp<kMirror>(x));
  if (levels > 4) { const f32x2 r = rows16(x); x = op(r[0], r[1]); }
  if (levels > 5) { const f32x2 r = rows32(x); x = op(r[0], r[1]); }
  return x;
}
__device__ __forceinline__ float wave_max(float x) { return lane_reduce(x, 6, OpMax{}); }
__device__ __forceinline__ float wave_sum(float x) { return lane_reduce(x, 6, OpSum{}); }
// FP64 sum over the wave (halves exchanged separately).
__device__ __forceinline__ double wave_sum_f64(double x) {
  auto ex = [](double v, auto f) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const float lo = f(__builtin_bit_cast(float, (uint32_t)u));
    const float hi = f(__builtin_bit_cast(float, (uint32_t)(u >> 32)));
    return __builtin_bit_cast(double, (uint64_t)__builtin_bit_cast(uint32_t, lo) |
                                          ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32));
  };
  x += ex(x, [](float v) { return dpp<kXor1>(v); });
  x += ex(x, [](float v) { return dpp<kXor2>(v); });
  x += ex(x, [](float v) { return dpp<kHalfMirror>(v); });
  x += ex(x, [](float v) { return dpp<kMirror>(v); });
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const f32x2 lo = rows16(__builtin_bit_cast(float, (uint32_t)u));
    const f32x2 hi = rows16(__builtin_bit_cast(float, (uint32_t)(u >> 32)));
    auto mk = [](float l, float h) {
      return __builtin_bit_cast(double, (uint64_t)__builtin_bit_cast(uint32_t, l) |
                                            ((uint64_t)__builtin_bit_cast(uint32_t, h) << 32));
    };
    x = mk(lo[0], hi[0]) + mk(lo[1], hi[1]);
  }
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const f32x2 lo = rows32(__builtin_bit_cast(float, (uint32_t)u));
    const f32x2 hi = rows32(__builtin_bit_cast(float, (uint32_t)(u >> 32)));
    auto mk = [](float l, float h) {
      return __builtin_bit_cast(double, (uint64_t)__builtin_bit_cast(uint32_t, l) |
                                            ((uint64_t)__builtin_bit_cast(uint32_t, h) << 32));
    };
    x = mk(lo[0], hi[0]) + mk(lo[1], hi[1]);
  }
  return x;
}

// ---- hand-off between workgroups of one launch ---------------------------
// Cache-policy bit sc1 (device scope).  A device-scope store is written
// through to the level that every XCD's device-scope loads read, and a
// device-scope load is served from there; the compiler emits exactly these
// accesses for relaxed agent-scope atomic loads and stores.  A workgroup that
// writes its result this way, waits for the stores to complete and then bumps
// an agent-scope atomic counter has made the result visible to the workgroup
// that sees the counter's last increment, without the L2 writeback and
// invalidate of a device-scope fence (which costs microseconds per workgroup).
constexpr int kPolicyDevice = 16;
__device__ __forceinline__ void st16_dev(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ void st8_dev(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ void st4_dev(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ u32x4 ld16_dev(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyDevice));
}
__device__ __forceinline__ u32x2 ld8_dev(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyDevice));
}
__device__ __forceinline__ float ld4f_dev(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyDevice));
}
// Wait until every memory access this wave issued has completed: s_waitcnt
// vmcnt(0) expcnt(7) lgkmcnt(15) in the gfx9 encoding.  (A workgroup barrier
// alone does not wait for outstanding global stores.)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace cpdec
