// Whole-block copies, for copy-on-write sharing inside the two pools ("vLLM
// Architecture, Memory and Benchmarks Deep Dive", section 2, "Copy-on-Write
// (CoW) Branching": a shared block is cloned when the sequences holding it
// diverge) and for swapping blocks between device pools and pools in pinned
// host memory ("Inside vLLM: Anatomy of a High-Throughput LLM Inference
// System", "Memory-Efficient KV Cache Storage": blocks are paged out to host
// memory and back).
//
// A block is contiguous in each pool ([num_kv_heads][block_size][head_dim]),
// so a copy is a straight memcpy of block_bytes. Grid: x = 16 KiB slices of
// a block, y = pairs. Each thread issues all of its K and V loads of a slice
// before the stores, so a workgroup keeps 32 KiB in flight (for a host-side
// pool these are PCIe reads or writes; many workgroups in flight hide their
// latency). The pair is read once per workgroup (the same address in every
// lane); pairs with an id outside its pool do nothing, and so do pairs with
// source equal to destination when both sides are the same pools.
#include "launch.h"
#include "pa_device.h"

namespace pa {

typedef uint32_t copy_u32x4 __attribute__((ext_vector_type(4)));

template <int UNIT>
struct CopyUnit;
template <>
struct CopyUnit<16> {
  using T = copy_u32x4;
};
template <>
struct CopyUnit<4> {
  using T = uint32_t;
};
template <>
struct CopyUnit<2> {
  using T = uint16_t;
};

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// Source and destination pools may be the same buffers (copy-on-write):
// destinations are never sources, so no byte is both read and written and the
// restrict qualifiers still hold.
template <int UNIT>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const uint8_t *__restrict__ src_key, const uint8_t *__restrict__ src_value,
    uint8_t *__restrict__ dst_key, uint8_t *__restrict__ dst_value,
    const int32_t *__restrict__ pairs, int32_t num_pairs, int32_t src_blocks, int32_t dst_blocks,
    int64_t block_bytes, int32_t skip_same) {
  using T = typename CopyUnit<UNIT>::T;
  const int64_t units = block_bytes / UNIT;
  for (int32_t pr = blockIdx.y; pr < num_pairs; pr += gridDim.y) {
    const int32_t src = pairs[2 * pr], dst = pairs[2 * pr + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
    if (skip_same && src == dst) continue;
    const T *ks = reinterpret_cast<const T *>(src_key + (int64_t)src * block_bytes);
    const T *vs = reinterpret_cast<const T *>(src_value + (int64_t)src * block_bytes);
    T *kd = reinterpret_cast<T *>(dst_key + (int64_t)dst * block_bytes);
    T *vd = reinterpret_cast<T *>(dst_value + (int64_t)dst * block_bytes);
    for (int64_t base = (int64_t)blockIdx.x * kCopyThreads * kCopyUnroll; base < units;
         base += (int64_t)gridDim.x * kCopyThreads * kCopyUnroll) {
      T k[kCopyUnroll], v[kCopyUnroll];
#pragma unroll
      for (int i = 0; i < kCopyUnroll; ++i) {
        const int64_t u = base + i * kCopyThreads + threadIdx.x;
        if (u < units) {
          k[i] = ks[u];
          v[i] = vs[u];
        }
      }
#pragma unroll
      for (int i = 0; i < kCopyUnroll; ++i) {
        const int64_t u = base + i * kCopyThreads + threadIdx.x;
        if (u < units) {
          kd[u] = k[i];
          vd[u] = v[i];
        }
      }
    }
  }
}

pa_status launch_move_blocks(const void *src_key, const void *src_value, void *dst_key,
                             void *dst_value, const int32_t *pairs, int32_t num_pairs,
                             int64_t block_bytes, int32_t src_blocks, int32_t dst_blocks,
                             bool skip_same, const char *fn, hipStream_t stream) {
  const int unit = (block_bytes % 16 == 0) ? 16 : (block_bytes % 4 == 0) ? 4 : 2;
  const int64_t units = block_bytes / unit;
  int64_t gx = (units + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll);
  if (gx > 1024) gx = 1024;  // the slice loop covers the rest
  const unsigned gy = (unsigned)(num_pairs < 65535 ? num_pairs : 65535);
  const dim3 grid((unsigned)gx, gy);
  auto sk = (const uint8_t *)src_key;
  auto sv = (const uint8_t *)src_value;
  auto dk = (uint8_t *)dst_key;
  auto dv = (uint8_t *)dst_value;
  const int32_t same = skip_same ? 1 : 0;
  if (unit == 16)
    copy_blocks_kernel<16><<<grid, kCopyThreads, 0, stream>>>(
        sk, sv, dk, dv, pairs, num_pairs, src_blocks, dst_blocks, block_bytes, same);
  else if (unit == 4)
    copy_blocks_kernel<4><<<grid, kCopyThreads, 0, stream>>>(
        sk, sv, dk, dv, pairs, num_pairs, src_blocks, dst_blocks, block_bytes, same);
  else
    copy_blocks_kernel<2><<<grid, kCopyThreads, 0, stream>>>(
        sk, sv, dk, dv, pairs, num_pairs, src_blocks, dst_blocks, block_bytes, same);
  return check_launch(fn);
}

pa_status launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream) {
  return launch_move_blocks(key_cache, value_cache, key_cache, value_cache, pairs, num_pairs,
                            block_bytes, num_blocks, num_blocks, true, "pa_copy_blocks", stream);
}

}  // namespace pa
