// Slot-mapped write of each new token's K and V rows into the paged pools.
//
// "vLLM Architecture, Memory and Benchmarks Deep Dive", section 1 (K/V of
// past tokens are cached) and section 2 (fixed-size physical blocks handed
// out on demand): token i's rows go to block slot/bs, offset slot%bs.
//
// One thread moves one 16-byte piece (or 4/2 bytes when a row is not a
// multiple of 16 bytes). Consecutive threads cover consecutive bytes of a
// source row, so both the read of key/value and the write into the block
// are fully coalesced; K and V are handled by the same thread to share the
// slot lookup. Pure bit copy: the pools receive the exact input bits.
#include "launch.h"
#include "pa_device.h"

namespace pa {

template <int UNIT>
struct Unit;
template <>
struct Unit<16> {
  using T = vec16;
};
template <>
struct Unit<4> {
  using T = uint32_t;
};
template <>
struct Unit<2> {
  using T = uint16_t;
};

template <int UNIT>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint8_t *__restrict__ key, const uint8_t *__restrict__ value,
    uint8_t *__restrict__ key_cache, uint8_t *__restrict__ value_cache,
    const int64_t *__restrict__ slot_mapping, int64_t units_per_token, int64_t units_per_row,
    int64_t total_units, int64_t row_bytes, int32_t num_kv_heads, int32_t block_size,
    int64_t num_slots) {
  using T = typename Unit<UNIT>::T;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total_units; u += stride) {
    const int64_t tok = u / units_per_token;
    const int64_t in_tok = u - tok * units_per_token;
    const int64_t head = in_tok / units_per_row;
    const int64_t piece = in_tok - head * units_per_row;
    // The rows are read before the slot is checked (they are always in
    // bounds), so the three loads are in flight together.
    const int64_t src = u * UNIT;
    const T kx = *reinterpret_cast<const T *>(key + src);
    const T vx = *reinterpret_cast<const T *>(value + src);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int64_t dst = ((blk * num_kv_heads + head) * block_size + off) * row_bytes + piece * UNIT;
    *reinterpret_cast<T *>(key_cache + dst) = kx;
    *reinterpret_cast<T *>(value_cache + dst) = vx;
  }
}

pa_status launch_cache_write(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int elem_bytes, hipStream_t stream) {
  const int64_t row_bytes = (int64_t)head_dim * elem_bytes;
  const int unit = (row_bytes % 16 == 0) ? 16 : (row_bytes % 4 == 0) ? 4 : 2;
  const int64_t units_per_row = row_bytes / unit;
  const int64_t units_per_token = units_per_row * num_kv_heads;
  const int64_t total = units_per_token * num_tokens;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  auto k = (const uint8_t *)key;
  auto v = (const uint8_t *)value;
  auto kc = (uint8_t *)key_cache;
  auto vc = (uint8_t *)value_cache;
  if (unit == 16)
    cache_write_kernel<16><<<(unsigned)blocks, threads, 0, stream>>>(
        k, v, kc, vc, slot_mapping, units_per_token, units_per_row, total, row_bytes,
        num_kv_heads, block_size, num_slots);
  else if (unit == 4)
    cache_write_kernel<4><<<(unsigned)blocks, threads, 0, stream>>>(
        k, v, kc, vc, slot_mapping, units_per_token, units_per_row, total, row_bytes,
        num_kv_heads, block_size, num_slots);
  else
    cache_write_kernel<2><<<(unsigned)blocks, threads, 0, stream>>>(
        k, v, kc, vc, slot_mapping, units_per_token, units_per_row, total, row_bytes,
        num_kv_heads, block_size, num_slots);
  return check_launch("pa_reshape_and_cache");
}

// ---------------------------------------------------------------- FP8 cache
//
// Quantising write into E4M3FN code pools (one byte per element: sign, 4
// exponent bits with bias 7, 3 mantissa bits; no infinities, 0x7F / 0xFF are
// NaN). A cache in a one-byte format halves the bytes decode must stream
// ("Optimizing LLM Inference", KV-cache section: the cache size is linear in
// the bytes per element). The code of x is the E4M3 value nearest to the
// fp32 quotient x / scale (ties to even), magnitudes of 448 and beyond
// saturate to +-448, and NaN becomes 0x7F. The quotient is an IEEE division
// (correctly rounded), so the code is a function of the two fp32 inputs.

namespace {

// E4M3FN code of an fp32 value, by integer rounding of its bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448 (and inf): saturate
  if (a < 0x3c800000u) {
    // |x| < 2^-6: subnormal codes, steps of 2^-9. The product is exact and
    // v_rndne rounds ties to even; 8 lands on the smallest normal, 0x08.
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  }
  // Normal: round the 23-bit mantissa to 3 bits, ties to even; a carry moves
  // into the exponent. Re-bias the exponent from 127 to 7.
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  const uint32_t code = (r >> 20) - (120u << 3);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

template <typename IN, int VEC>
__device__ __forceinline__ void load_vals(const IN *p, float *o);
template <>
__device__ __forceinline__ void load_vals<bf16_t, 8>(const bf16_t *p, float *o) {
  Widen<bf16_t>::apply(load16(p), o);
}
template <>
__device__ __forceinline__ void load_vals<float, 8>(const float *p, float *o) {
  Widen<float>::apply(load16(p), o);
  Widen<float>::apply(load16(p + 4), o + 4);
}
template <>
__device__ __forceinline__ void load_vals<bf16_t, 1>(const bf16_t *p, float *o) {
  o[0] = __uint_as_float((uint32_t)p->bits << 16);
}
template <>
__device__ __forceinline__ void load_vals<float, 1>(const float *p, float *o) {
  o[0] = *p;
}

template <int VEC>
__device__ __forceinline__ void store_codes(uint8_t *dst, const float *x, float scale);
// Value pools store each block transposed: consecutive channels are
// block_size bytes apart.
template <int VEC>
__device__ __forceinline__ void store_codes_strided(uint8_t *dst, const float *x, float scale,
                                                    int stride) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) dst[(int64_t)v * stride] = (uint8_t)f32_to_e4m3(x[v] / scale);
}
template <>
__device__ __forceinline__ void store_codes<8>(uint8_t *dst, const float *x, float scale) {
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    w[h] = f32_to_e4m3(x[4 * h] / scale) | (f32_to_e4m3(x[4 * h + 1] / scale) << 8) |
           (f32_to_e4m3(x[4 * h + 2] / scale) << 16) | (f32_to_e4m3(x[4 * h + 3] / scale) << 24);
  }
  *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
}
template <>
__device__ __forceinline__ void store_codes<1>(uint8_t *dst, const float *x, float scale) {
  *dst = (uint8_t)f32_to_e4m3(x[0] / scale);
}

}  // namespace

// One thread quantises VEC consecutive elements of one K row and the same
// elements of the V row (8 when head_dim is a multiple of 8: a 16- or
// 32-byte coalesced read and an 8-byte write; else 1).
template <typename IN, int VEC>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const IN *__restrict__ key, const IN *__restrict__ value, uint8_t *__restrict__ key_cache,
    uint8_t *__restrict__ value_cache, const int64_t *__restrict__ slot_mapping,
    int64_t units_per_token, int64_t units_per_row, int64_t total_units, int32_t head_dim,
    int32_t num_kv_heads, int32_t block_size, int64_t num_slots, float k_scale, float v_scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total_units; u += stride) {
    const int64_t tok = u / units_per_token;
    const int64_t in_tok = u - tok * units_per_token;
    const int64_t head = in_tok / units_per_row;
    const int64_t piece = in_tok - head * units_per_row;
    float kx[VEC], vx[VEC];
    load_vals<IN, VEC>(key + u * VEC, kx);
    load_vals<IN, VEC>(value + u * VEC, vx);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int64_t dst = ((blk * num_kv_heads + head) * block_size + off) * head_dim + piece * VEC;
    const int64_t vdst = ((blk * num_kv_heads + head) * head_dim + piece * VEC) * block_size + off;
    store_codes<VEC>(key_cache + dst, kx, k_scale);
    store_codes_strided<VEC>(value_cache + vdst, vx, v_scale, block_size);
  }
}

template <typename IN>
static void launch_fp8_write(const void *key, const void *value, uint8_t *kc, uint8_t *vc,
                             const int64_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_slots, float k_scale, float v_scale,
                             hipStream_t stream) {
  const int vec = head_dim % 8 == 0 ? 8 : 1;
  const int64_t units_per_row = head_dim / vec;
  const int64_t units_per_token = units_per_row * num_kv_heads;
  const int64_t total = units_per_token * num_tokens;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  auto k = (const IN *)key;
  auto v = (const IN *)value;
  if (vec == 8)
    cache_write_fp8_kernel<IN, 8><<<(unsigned)blocks, threads, 0, stream>>>(
        k, v, kc, vc, slot_mapping, units_per_token, units_per_row, total, head_dim,
        num_kv_heads, block_size, num_slots, k_scale, v_scale);
  else
    cache_write_fp8_kernel<IN, 1><<<(unsigned)blocks, threads, 0, stream>>>(
        k, v, kc, vc, slot_mapping, units_per_token, units_per_row, total, head_dim,
        num_kv_heads, block_size, num_slots, k_scale, v_scale);
}

pa_status launch_cache_write_fp8(const void *key, const void *value, uint8_t *key_cache,
                                 uint8_t *value_cache, const int64_t *slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, bool in_bf16,
                                 float k_scale, float v_scale, hipStream_t stream) {
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (in_bf16)
    launch_fp8_write<bf16_t>(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                             num_kv_heads, head_dim, block_size, num_slots, k_scale, v_scale,
                             stream);
  else
    launch_fp8_write<float>(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                            num_kv_heads, head_dim, block_size, num_slots, k_scale, v_scale,
                            stream);
  return check_launch("pa_reshape_and_cache_fp8");
}

}  // namespace pa
