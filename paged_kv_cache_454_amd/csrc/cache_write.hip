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

}  // namespace pa
