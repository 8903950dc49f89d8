// C entry points: host-side argument checks, then the kernel launchers.
#include <math.h>

#include "launch.h"
#include "pa_internal.h"
#include "persistent_plan.h"

namespace {

bool dtype_ok(pa_dtype t) { return t == PA_F32 || t == PA_BF16; }
int dtype_bytes(pa_dtype t) { return t == PA_FP8_E4M3 ? 1 : t == PA_BF16 ? 2 : 4; }

pa_status check_fp8_scales(const char *fn, float k_scale, float v_scale) {
  if (!(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
    return pa::fail(PA_EINVAL, "%s: k_scale=%g v_scale=%g must be finite and > 0", fn,
                    (double)k_scale, (double)v_scale);
  return PA_OK;
}

// Shared checks of the paged-attention shapes.
pa_status check_attention_shape(const char *fn, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                                pa_dtype kv_dtype) {
  if (num_seqs < 0) return pa::fail(PA_EINVAL, "%s: num_seqs=%d < 0", fn, num_seqs);
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return pa::fail(PA_EINVAL, "%s: head counts must be > 0 (q=%d kv=%d)", fn, num_q_heads,
                    num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return pa::fail(PA_EINVAL, "%s: num_q_heads=%d not a multiple of num_kv_heads=%d", fn,
                    num_q_heads, num_kv_heads);
  if (head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return pa::fail(PA_EINVAL,
                    "%s: head_dim=%d block_size=%d max_blocks_per_seq=%d num_blocks=%d must be > 0",
                    fn, head_dim, block_size, max_blocks_per_seq, num_blocks);
  if (!isfinite(scale)) return pa::fail(PA_EINVAL, "%s: scale is not finite", fn);
  if (!dtype_ok(kv_dtype)) return pa::fail(PA_EINVAL, "%s: bad kv_dtype %d", fn, (int)kv_dtype);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return pa::fail(PA_EUNSUPPORTED, "%s: head_dim=%d (supported: 64, 128, 256)", fn, head_dim);
  if (num_q_heads / num_kv_heads > 8)
    return pa::fail(PA_EUNSUPPORTED, "%s: query heads per KV head = %d > 8", fn,
                    num_q_heads / num_kv_heads);
  if ((int64_t)max_blocks_per_seq * block_size > 0x7fffffff)
    return pa::fail(PA_EUNSUPPORTED, "%s: max_blocks_per_seq * block_size exceeds 2^31", fn);
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_reshape_and_cache(const void *key, const void *value, void *key_cache,
                                          void *value_cache, const int64_t *slot_mapping,
                                          int32_t num_tokens, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t num_blocks, pa_dtype kv_dtype,
                                          hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_reshape_and_cache";
  if (num_tokens < 0) return pa::fail(PA_EINVAL, "%s: num_tokens=%d < 0", fn, num_tokens);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa::fail(PA_EINVAL, "%s: num_kv_heads=%d head_dim=%d block_size=%d num_blocks=%d", fn,
                    num_kv_heads, head_dim, block_size, num_blocks);
  if (head_dim > 1024) return pa::fail(PA_EUNSUPPORTED, "%s: head_dim=%d > 1024", fn, head_dim);
  if (!dtype_ok(kv_dtype)) return pa::fail(PA_EINVAL, "%s: bad kv_dtype %d", fn, (int)kv_dtype);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  return pa::launch_cache_write(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                num_kv_heads, head_dim, block_size, num_blocks,
                                dtype_bytes(kv_dtype), stream);
}

extern "C" pa_status pa_reshape_and_cache_fp8(const void *key, const void *value,
                                              uint8_t *key_cache, uint8_t *value_cache,
                                              const int64_t *slot_mapping, int32_t num_tokens,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t block_size, int32_t num_blocks,
                                              pa_dtype in_dtype, float k_scale, float v_scale,
                                              hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_reshape_and_cache_fp8";
  if (num_tokens < 0) return pa::fail(PA_EINVAL, "%s: num_tokens=%d < 0", fn, num_tokens);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa::fail(PA_EINVAL, "%s: num_kv_heads=%d head_dim=%d block_size=%d num_blocks=%d", fn,
                    num_kv_heads, head_dim, block_size, num_blocks);
  if (head_dim > 1024) return pa::fail(PA_EUNSUPPORTED, "%s: head_dim=%d > 1024", fn, head_dim);
  if (!dtype_ok(in_dtype)) return pa::fail(PA_EINVAL, "%s: bad in_dtype %d", fn, (int)in_dtype);
  pa_status st = check_fp8_scales(fn, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  return pa::launch_cache_write_fp8(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                    num_kv_heads, head_dim, block_size, num_blocks,
                                    in_dtype == PA_BF16, k_scale, v_scale, stream);
}

extern "C" pa_status pa_copy_blocks(void *key_cache, void *value_cache, const int32_t *block_pairs,
                                    int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, pa_dtype kv_dtype,
                                    hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_copy_blocks";
  if (num_pairs < 0) return pa::fail(PA_EINVAL, "%s: num_pairs=%d < 0", fn, num_pairs);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa::fail(PA_EINVAL, "%s: num_kv_heads=%d head_dim=%d block_size=%d num_blocks=%d", fn,
                    num_kv_heads, head_dim, block_size, num_blocks);
  if (!dtype_ok(kv_dtype) && kv_dtype != PA_FP8_E4M3)
    return pa::fail(PA_EINVAL, "%s: bad kv_dtype %d", fn, (int)kv_dtype);
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_pairs)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  const int64_t block_bytes =
      (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(kv_dtype);
  return pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs, block_bytes,
                                num_blocks, stream);
}

// True when the bytes [ptr, ptr + bytes) start and end in memory a kernel on
// the current device may address at these same pointers: device memory of
// this device, or pinned host memory mapped into the device's address space.
// Anything else (pageable host memory, another device's memory) is refused
// before a launch could fault on it.
static pa_status check_reachable(const char *fn, const char *what, const void *ptr,
                                 int64_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return pa::fail(PA_EHIP, "%s: hipGetDevice failed", fn);
  }
  for (int end = 0; end < 2; ++end) {
    const char *p = (const char *)ptr + (end ? bytes - 1 : 0);
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
      (void)hipGetLastError();
      return pa::fail(PA_EINVAL, "%s: %s is neither device memory nor pinned host memory", fn,
                      what);
    }
    const bool on_device = attr.type == hipMemoryTypeDevice && attr.device == dev;
    const bool pinned_host = attr.type == hipMemoryTypeHost && attr.devicePointer == (void *)p;
    if (!on_device && !pinned_host)
      return pa::fail(PA_EINVAL,
                      "%s: %s (%s byte) is not device memory of device %d nor pinned host "
                      "memory mapped at the same address", fn, what, end ? "last" : "first",
                      dev);
  }
  return PA_OK;
}

extern "C" pa_status pa_swap_blocks(const void *src_key_cache, const void *src_value_cache,
                                    int32_t src_num_blocks, void *dst_key_cache,
                                    void *dst_value_cache, int32_t dst_num_blocks,
                                    const int32_t *block_pairs, int32_t num_pairs,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    pa_dtype kv_dtype, hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_swap_blocks";
  if (num_pairs < 0) return pa::fail(PA_EINVAL, "%s: num_pairs=%d < 0", fn, num_pairs);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || src_num_blocks <= 0 ||
      dst_num_blocks <= 0)
    return pa::fail(PA_EINVAL,
                    "%s: num_kv_heads=%d head_dim=%d block_size=%d src_num_blocks=%d "
                    "dst_num_blocks=%d", fn, num_kv_heads, head_dim, block_size, src_num_blocks,
                    dst_num_blocks);
  if (!dtype_ok(kv_dtype) && kv_dtype != PA_FP8_E4M3)
    return pa::fail(PA_EINVAL, "%s: bad kv_dtype %d", fn, (int)kv_dtype);
  if (num_pairs == 0) return PA_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_pairs)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  const int64_t block_bytes =
      (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(kv_dtype);
  const struct { const char *what; const void *p; int64_t bytes; } spans[] = {
      {"src_key_cache", src_key_cache, block_bytes * src_num_blocks},
      {"src_value_cache", src_value_cache, block_bytes * src_num_blocks},
      {"dst_key_cache", dst_key_cache, block_bytes * dst_num_blocks},
      {"dst_value_cache", dst_value_cache, block_bytes * dst_num_blocks},
      {"block_pairs", block_pairs, (int64_t)num_pairs * 2 * (int64_t)sizeof(int32_t)}};
  for (const auto &sp : spans) {
    const pa_status st = check_reachable(fn, sp.what, sp.p, sp.bytes);
    if (st != PA_OK) return st;
  }
  return pa::launch_move_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache,
                                block_pairs, num_pairs, block_bytes, src_num_blocks,
                                dst_num_blocks, src_key_cache == dst_key_cache, fn, stream);
}

extern "C" int64_t pa_read_probe_sink_words(void) { return pa::read_probe_sink_words(); }

extern "C" pa_status pa_read_probe(const void *pool, int64_t pool_bytes, const int32_t *order,
                                   int32_t num_blocks, uint32_t *sink, int64_t sink_words,
                                   hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_read_probe";
  if (num_blocks < 0 || pool_bytes < 0 || sink_words < 0)
    return pa::fail(PA_EINVAL, "%s: num_blocks=%d pool_bytes=%lld sink_words=%lld", fn,
                    num_blocks, (long long)pool_bytes, (long long)sink_words);
  if (!sink) return pa::fail(PA_EINVAL, "%s: sink is NULL", fn);
  const int64_t need = pa::read_probe_sink_words();
  if (sink_words < need)
    return pa::fail(PA_EINVAL, "%s: sink has %lld words, needs %lld", fn, (long long)sink_words,
                    (long long)need);
  if (num_blocks > 0 && (!pool || !order)) return pa::fail(PA_EINVAL, "%s: null pointer", fn);
  return pa::launch_read_probe(pool, pool_bytes, order, num_blocks, sink, stream);
}

extern "C" pa_status pa_decode(void *out, const void *query, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                               pa_dtype kv_dtype, pa_dtype out_dtype, hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_decode";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = 0;
  p.max_parts = 1;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.out_bf16 = out_dtype == PA_BF16;
  return pa::launch_decode(p, stream);
}

extern "C" pa_status pa_decode_fp8(void *out, const void *query, const uint8_t *key_cache,
                                   const uint8_t *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, float scale, float k_scale, float v_scale,
                                   pa_dtype out_dtype, hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_decode_fp8";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale, PA_BF16);
  if (st != PA_OK) return st;
  st = check_fp8_scales(fn, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = 0;
  p.max_parts = 1;
  p.kv_bf16 = 0;
  p.kv_fp8 = 1;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.out_bf16 = out_dtype == PA_BF16;
  return pa::launch_decode(p, stream);
}

extern "C" size_t pa_partition_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_dim, int32_t max_parts) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_parts <= 0) return 0;
  const size_t n = (size_t)num_seqs * num_q_heads * max_parts;
  return n * (size_t)head_dim * sizeof(float) + 2 * n * sizeof(float);
}

static pa_status decode_partitioned(const char *fn, void *plan, uint32_t plan_epoch,
                                   float *part_out, float *part_max, float *part_sum,
                                   const void *query, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, float scale, int32_t partition_size,
                                   int32_t max_parts, pa_dtype kv_dtype, hipStream_t stream) {
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (partition_size < 16 || partition_size % block_size != 0)
    return pa::fail(PA_EINVAL, "%s: partition_size=%d must be >= 16 and a multiple of block_size=%d",
                    fn, partition_size, block_size);
  if (max_parts <= 0) return pa::fail(PA_EINVAL, "%s: max_parts=%d must be > 0", fn, max_parts);
  if (num_seqs == 0) return PA_OK;
  if (!part_out || !part_max || !part_sum || !query || !key_cache || !value_cache ||
      !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.part_out = part_out;
  p.part_max = part_max;
  p.part_sum = part_sum;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = partition_size;
  p.max_parts = max_parts;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.plan = plan;
  p.plan_epoch = plan_epoch;
  return pa::launch_decode(p, stream);
}

extern "C" pa_status pa_decode_partitioned(float *part_out, float *part_max, float *part_sum,
                                           const void *query, const void *key_cache,
                                           const void *value_cache, const int32_t *block_tables,
                                           const int32_t *context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int32_t num_blocks,
                                           float scale, int32_t partition_size,
                                           int32_t max_parts, pa_dtype kv_dtype,
                                           hipStream_t stream) {
  pa::clear_error();
  return decode_partitioned("pa_decode_partitioned", nullptr, 0, part_out, part_max, part_sum,
                            query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                            num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            num_blocks, scale, partition_size, max_parts, kv_dtype, stream);
}

static pa_status decode_partitioned_fp8(
    const char *fn, void *plan, uint32_t plan_epoch, float *part_out, float *part_max, float *part_sum, const void *query,
    const uint8_t *key_cache, const uint8_t *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    float scale, float k_scale, float v_scale, int32_t partition_size, int32_t max_parts,
    hipStream_t stream) {
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale, PA_BF16);
  if (st != PA_OK) return st;
  st = check_fp8_scales(fn, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (partition_size < 16 || partition_size % block_size != 0)
    return pa::fail(PA_EINVAL, "%s: partition_size=%d must be >= 16 and a multiple of block_size=%d",
                    fn, partition_size, block_size);
  if (max_parts <= 0) return pa::fail(PA_EINVAL, "%s: max_parts=%d must be > 0", fn, max_parts);
  if (num_seqs == 0) return PA_OK;
  if (!part_out || !part_max || !part_sum || !query || !key_cache || !value_cache ||
      !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.part_out = part_out;
  p.part_max = part_max;
  p.part_sum = part_sum;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = partition_size;
  p.max_parts = max_parts;
  p.kv_bf16 = 0;
  p.kv_fp8 = 1;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.plan = plan;
  p.plan_epoch = plan_epoch;
  return pa::launch_decode(p, stream);
}

extern "C" pa_status pa_decode_partitioned_fp8(
    float *part_out, float *part_max, float *part_sum, const void *query,
    const uint8_t *key_cache, const uint8_t *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    float scale, float k_scale, float v_scale, int32_t partition_size, int32_t max_parts,
    hipStream_t stream) {
  pa::clear_error();
  return decode_partitioned_fp8("pa_decode_partitioned_fp8", nullptr, 0, part_out, part_max,
                                part_sum, query, key_cache, value_cache, block_tables,
                                context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                block_size, max_blocks_per_seq, num_blocks, scale, k_scale,
                                v_scale, partition_size, max_parts, stream);
}

extern "C" pa_status pa_decode_partitioned_fp8_planned(
    float *part_out, float *part_max, float *part_sum, const void *query,
    const uint8_t *key_cache, const uint8_t *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    float scale, float k_scale, float v_scale, int32_t partition_size, int32_t max_parts,
    void *plan, uint32_t plan_epoch, hipStream_t stream) {
  pa::clear_error();
  return decode_partitioned_fp8("pa_decode_partitioned_fp8_planned", plan, plan_epoch, part_out,
                                part_max, part_sum, query, key_cache, value_cache, block_tables,
                                context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                block_size, max_blocks_per_seq, num_blocks, scale, k_scale,
                                v_scale, partition_size, max_parts, stream);
}

// Checks of a balanced call's scratch (caller-owned device memory, zero
// before the first call; the kernels leave the counters at zero).
static pa_status check_scratch(const char *fn, const void *scratch, size_t scratch_bytes) {
  const int64_t need = pa::bal_scratch_bytes_current();
  if (!scratch) return pa::fail(PA_EINVAL, "%s: scratch is NULL", fn);
  if ((int64_t)scratch_bytes < need)
    return pa::fail(PA_EINVAL, "%s: scratch_bytes=%zu < %lld (pa_decode_scratch_bytes)", fn,
                    scratch_bytes, (long long)need);
  if ((uintptr_t)scratch % 16 != 0)
    return pa::fail(PA_EINVAL, "%s: scratch must be 16-byte aligned", fn);
  return PA_OK;
}

extern "C" size_t pa_decode_scratch_bytes(void) {
  return (size_t)pa::bal_scratch_bytes_current();
}

extern "C" pa_status pa_decode_balanced(void *out, const void *query, const void *key_cache,
                                        const void *value_cache, const int32_t *block_tables,
                                        const int32_t *context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t max_blocks_per_seq, int32_t num_blocks,
                                        float scale, pa_dtype kv_dtype, pa_dtype out_dtype,
                                        void *scratch, size_t scratch_bytes,
                                        hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_decode_balanced";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  st = check_scratch(fn, scratch, scratch_bytes);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = 0;
  p.max_parts = 1;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.out_bf16 = out_dtype == PA_BF16;
  p.scratch = scratch;
  p.scratch_bytes = (int64_t)scratch_bytes;
  if (pa::launch_decode_balanced(p, stream)) return pa::check_launch("decode");
  p.scratch = nullptr;  // a shape the balanced kernel does not cover
  return pa::launch_decode(p, stream);
}

extern "C" pa_status pa_decode_balanced_static(void *out, const void *query,
                                               const void *key_cache, const void *value_cache,
                                               const int32_t *block_tables,
                                               const int32_t *context_lens, int32_t num_seqs,
                                               int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size,
                                               int32_t max_blocks_per_seq, int32_t num_blocks,
                                               float scale, pa_dtype kv_dtype,
                                               pa_dtype out_dtype, hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_decode_balanced_static";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  const int64_t need = pa::bal_scratch_bytes_current();
  if (need > pa::bal_static_scratch_limit())
    return pa::fail(PA_EUNSUPPORTED,
                    "%s: this device needs %lld bytes of scratch, more than the static %lld", fn,
                    (long long)need, (long long)pa::bal_static_scratch_limit());
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  const char *why = "";
  void *scratch = pa::bal_static_scratch(&why);
  if (!scratch) return pa::fail(PA_EHIP, "%s: %s", fn, why);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = 0;
  p.max_parts = 1;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.out_bf16 = out_dtype == PA_BF16;
  p.scratch = scratch;
  p.scratch_bytes = pa::bal_static_scratch_limit();
  if (pa::launch_decode_balanced(p, stream)) return pa::check_launch("decode");
  p.scratch = nullptr;  // a shape the balanced kernel does not cover
  return pa::launch_decode(p, stream);
}

extern "C" pa_status pa_decode_partitioned_balanced(
    float *part_out, float *part_max, float *part_sum, const void *query, const void *key_cache,
    const void *value_cache, const int32_t *block_tables, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
    int32_t partition_size, int32_t max_parts, pa_dtype kv_dtype, void *scratch,
    size_t scratch_bytes, hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_decode_partitioned_balanced";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (partition_size < 16 || partition_size % block_size != 0)
    return pa::fail(PA_EINVAL, "%s: partition_size=%d must be >= 16 and a multiple of block_size=%d",
                    fn, partition_size, block_size);
  if (max_parts <= 0) return pa::fail(PA_EINVAL, "%s: max_parts=%d must be > 0", fn, max_parts);
  st = check_scratch(fn, scratch, scratch_bytes);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!part_out || !part_max || !part_sum || !query || !key_cache || !value_cache ||
      !block_tables || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.part_out = part_out;
  p.part_max = part_max;
  p.part_sum = part_sum;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = partition_size;
  p.max_parts = max_parts;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.scratch = scratch;
  p.scratch_bytes = (int64_t)scratch_bytes;
  if (pa::launch_decode_balanced(p, stream)) return pa::check_launch("decode");
  p.scratch = nullptr;
  return pa::launch_decode(p, stream);
}

extern "C" pa_status pa_reduce(void *out, const float *part_out, const float *part_max,
                               const float *part_sum, const int32_t *context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                               int32_t partition_size, int32_t max_parts, pa_dtype out_dtype,
                               hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_reduce";
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || partition_size <= 0 || max_parts <= 0)
    return pa::fail(PA_EINVAL,
                    "%s: num_seqs=%d num_q_heads=%d head_dim=%d partition_size=%d max_parts=%d",
                    fn, num_seqs, num_q_heads, head_dim, partition_size, max_parts);
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  if (num_seqs == 0) return PA_OK;
  if (!out || !part_out || !part_max || !part_sum || !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  return pa::launch_reduce(out, part_out, part_max, part_sum, context_lens, num_seqs, num_q_heads,
                           head_dim, partition_size, max_parts, out_dtype == PA_BF16, stream);
}

extern "C" pa_status pa_decode_step(void *out, float *part_out, float *part_max,
                                    float *part_sum, const void *query, const void *key,
                                    const void *value, void *key_cache, void *value_cache,
                                    const int32_t *block_tables, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                                    int32_t partition_size, int32_t max_parts, pa_dtype kv_dtype,
                                    pa_dtype out_dtype, void *plan, uint32_t plan_epoch,
                                    hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_decode_step";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  const bool split = partition_size != 0;
  if (split) {
    if (partition_size < 16 || partition_size % block_size != 0)
      return pa::fail(PA_EINVAL,
                      "%s: partition_size=%d must be 0 or >= 16 and a multiple of block_size=%d",
                      fn, partition_size, block_size);
    if (max_parts <= 0) return pa::fail(PA_EINVAL, "%s: max_parts=%d must be > 0", fn, max_parts);
  }
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key || !value || !key_cache || !value_cache || !block_tables ||
      !context_lens || (split && (!part_out || !part_max || !part_sum)))
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);

  pa::AppendArgs a{};
  a.new_key = key;
  a.new_value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.row_bytes = head_dim * (kv_dtype == PA_BF16 ? 2 : 4);

  pa::DecodeParams p{};
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.part_out = part_out;
  p.part_max = part_max;
  p.part_sum = part_sum;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.partition_size = split ? partition_size : 0;
  p.max_parts = split ? max_parts : 1;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.out_bf16 = out_dtype == PA_BF16;

  // The matrix-core kernel reads the step's token from key/value, so the
  // slot write can follow it (inside the merge launch when there is one).
  // Other kernels read it from the pool: the write goes first.
  p.new_key = key;
  p.new_value = value;
  p.step = 1;
  p.plan = plan;
  p.plan_epoch = plan_epoch;
  const bool fused = pa::launch_decode_mfma(p, stream);
  if (fused) {
    st = pa::check_launch(fn);
  } else {
    p.new_key = p.new_value = nullptr;
    p.step = 0;
    p.plan = nullptr;
    st = pa::launch_append(a, context_lens, num_seqs, stream);
    if (st == PA_OK) st = pa::launch_decode(p, stream);
  }
  if (st != PA_OK) return st;
  if (split)
    return pa::launch_reduce(out, part_out, part_max, part_sum, context_lens, num_seqs,
                             num_q_heads, head_dim, partition_size, max_parts,
                             out_dtype == PA_BF16, stream, fused ? &a : nullptr);
  return fused ? pa::launch_append(a, context_lens, num_seqs, stream) : PA_OK;
}

extern "C" size_t pa_decode_plan_bytes(void) {
  return (size_t)pa::persist::num_cus() * pa::kPlanWgBytes;
}

extern "C" pa_status pa_decode_partitioned_planned(
    float *part_out, float *part_max, float *part_sum, const void *query, const void *key_cache,
    const void *value_cache, const int32_t *block_tables, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
    int32_t partition_size, int32_t max_parts, pa_dtype kv_dtype, void *plan,
    uint32_t plan_epoch, hipStream_t stream) {
  pa::clear_error();
  return decode_partitioned("pa_decode_partitioned_planned", plan, plan_epoch, part_out,
                            part_max, part_sum, query, key_cache, value_cache, block_tables,
                            context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, num_blocks, scale, partition_size,
                            max_parts, kv_dtype, stream);
}

extern "C" pa_status pa_prefill_chunk(void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const int32_t *block_tables,
                                      const int32_t *query_start_loc, const int32_t *context_lens,
                                      int32_t num_seqs, int32_t num_q_tokens,
                                      int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t num_blocks, float scale, pa_dtype kv_dtype,
                                      pa_dtype out_dtype, hipStream_t stream) {
  pa::clear_error();
  const char *fn = "pa_prefill_chunk";
  pa_status st = check_attention_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, scale,
                                       kv_dtype);
  if (st != PA_OK) return st;
  if (kv_dtype != PA_BF16) return pa::fail(PA_EUNSUPPORTED, "%s: kv_dtype must be BF16", fn);
  if (!dtype_ok(out_dtype)) return pa::fail(PA_EINVAL, "%s: bad out_dtype", fn);
  if (max_query_len < 0 || num_q_tokens < 0)
    return pa::fail(PA_EINVAL, "%s: max_query_len=%d num_q_tokens=%d", fn, max_query_len,
                    num_q_tokens);
  if (num_seqs == 0 || max_query_len == 0 || num_q_tokens == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !query_start_loc ||
      !context_lens)
    return pa::fail(PA_EINVAL, "%s: null pointer argument", fn);
  pa::PrefillParams p{};
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.query_start_loc = query_start_loc;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_q_tokens = num_q_tokens;
  p.max_query_len = max_query_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.out_bf16 = out_dtype == PA_BF16;
  return pa::launch_prefill(p, stream);
}
