// Device-side helpers for the gfx950 kernels (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// BF16 is carried as its raw 16 bits; widening to fp32 is a shift.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16-byte vector of raw data.
struct alignas(16) vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ vec16 load16(const void *p) {
  return *reinterpret_cast<const vec16 *>(p);
}

// Widen the 16 bytes at `v` holding elements of type KV into fp32 values.
template <typename KV>
struct Widen;
template <>
struct Widen<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void apply(const vec16 &v, float *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v.w[i]);
  }
};
template <>
struct Widen<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void apply(const vec16 &v, float *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf16_lo(v.w[i]);
      o[2 * i + 1] = bf16_hi(v.w[i]);
    }
  }
};

// E4M3FN code (one byte) of an FP8 cache.
struct fp8_t {
  uint8_t bits;
};

// Four E4M3FN codes (bytes of w, lowest first) as fp32 values. gfx950's
// conversion implements the OCP E4M3FN format exactly (every code, NaN
// codes included, decodes to its value; checked against the format's
// definition).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *o) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0];
  o[1] = lo[1];
  o[2] = hi[0];
  o[3] = hi[1];
}

// A lane's piece of one K or V row, widened to fp32: 16 bytes of fp32 or
// BF16, or 8 bytes of E4M3 codes (so that the lane count per row matches a
// BF16 query's). Q is the query's element type.
template <typename KV>
struct KvPiece;
template <>
struct KvPiece<float> {
  static constexpr int N = 4;
  using Q = float;
  __device__ __forceinline__ static void load(const float *p, float *o) {
    Widen<float>::apply(load16(p), o);
  }
};
template <>
struct KvPiece<bf16_t> {
  static constexpr int N = 8;
  using Q = bf16_t;
  __device__ __forceinline__ static void load(const bf16_t *p, float *o) {
    Widen<bf16_t>::apply(load16(p), o);
  }
};
template <>
struct KvPiece<fp8_t> {
  static constexpr int N = 8;
  using Q = bf16_t;
  __device__ __forceinline__ static void load(const fp8_t *p, float *o) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    e4m3x4_to_f32(x.x, o);
    e4m3x4_to_f32(x.y, o + 4);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Store one output element as fp32 or bf16.
__device__ __forceinline__ void store_out(void *out, int64_t idx, float v, bool bf16) {
  if (bf16)
    reinterpret_cast<uint16_t *>(out)[idx] = f32_to_bf16(v);
  else
    reinterpret_cast<float *>(out)[idx] = v;
}

// Cache policy of the K/V tile loads: non-temporal (the nt bit of the
// buffer instruction). Decode reads every cached K/V byte once per step, so
// keeping it in L2 and the Infinity Cache only evicts useful lines; on
// MI355X random 8 KiB gathers run measurably faster this way.
constexpr int kStreamLoad = 2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no logit seen yet": exp2(kNoMax - m) is 0 for any
// finite m, and exp2(kNoMax - kNoMax) = 1 keeps empty merges well defined.
constexpr float kNoMax = -1.0e30f;

}  // namespace pa
