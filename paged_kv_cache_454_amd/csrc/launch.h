// Internal launchers called by the C entry points after argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

pa_status launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream);

// Block copies from one pair of pools to another (device memory or pinned,
// device-mapped host memory); pairs are (source, destination) block ids.
pa_status launch_move_blocks(const void *src_key, const void *src_value, void *dst_key,
                             void *dst_value, const int32_t *pairs, int32_t num_pairs,
                             int64_t block_bytes, int32_t src_blocks, int32_t dst_blocks,
                             bool skip_same, const char *fn, hipStream_t stream);

pa_status launch_cache_write(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int elem_bytes, hipStream_t stream);

pa_status launch_cache_write_fp8(const void *key, const void *value, uint8_t *key_cache,
                                 uint8_t *value_cache, const int64_t *slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, bool in_bf16,
                                 float k_scale, float v_scale, hipStream_t stream);

// Arguments of the decode kernels (single pass when partition_size == 0).
struct DecodeParams {
  const void *query;
  const void *key_cache;
  const void *value_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;  // non-null: causal prefill rows (generic kernel only)
  int32_t max_query_len;           // prefill: bound on rows per sequence
  int32_t num_q_tokens;            // prefill: rows of query / out
  void *out;          // single pass: [num_seqs][num_q_heads][head_dim], out dtype
  float *part_out;    // partitioned: [num_seqs][num_q_heads][max_parts][head_dim]
  float *part_max;    // partitioned: [num_seqs][num_q_heads][max_parts]
  float *part_sum;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  float scale;
  int32_t partition_size;  // 0 = single pass
  int32_t max_parts;       // 1 for single pass
  int32_t kv_bf16;
  int32_t out_bf16;
  int32_t kv_fp8;   // E4M3FN code pools, BF16 queries; logits scale by k_scale,
  float k_scale;    // outputs by v_scale (used only when kv_fp8)
  float v_scale;
  void *scratch;          // balanced kernels: merge entries + piece slots
  int64_t scratch_bytes;
  // Decode step: non-null means position T_s - 1 of every sequence is this
  // step's token and its K/V rows are read from here ([num_seqs][num_kv_heads]
  // [head_dim], the pools' dtype) instead of from the pools. Only the
  // matrix-core BF16 kernel accepts it; the others decline such a launch.
  const void *new_key;
  const void *new_value;
  int32_t step;  // 1: a decode step (new_key/new_value set)
  // Plan cache (matrix-core kernel only): a launch whose plan_epoch matches
  // the slot it finds reads its units from there, else plans and stores them.
  void *plan;
  uint32_t plan_epoch;
};

// Plan buffer: per workgroup of the persistent decode grid kPlanWgBytes
// bytes: the 64 unit slots (int4 sequence, KV head, first token, end of its
// pool tokens), their int partition * 4 + 2 * step token + bad (-1: no
// unit), each wave's first two block ids, and a header (mode word, grid,
// batch size, partition size, epoch) naming the launch that wrote it.
constexpr int kPlanWgBytes = 1536;
constexpr int kPlanUnits = 0, kPlanBp = 1024, kPlanIds = 1280, kPlanHdr = 1408;
constexpr int kPlanIdBytes = 16;  // per wave: up to four block ids
constexpr int kPlanMagic = 0x504c0000;

// The step's K/V rows written to position T_s - 1 of each sequence (the slot
// its block table gives; a block id outside the pool, T_s = 0 or T_s past the
// table's capacity writes nothing). Null new_key = no write.
struct AppendArgs {
  const void *new_key;
  const void *new_value;
  void *key_cache;
  void *value_cache;
  const int32_t *block_tables;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t row_bytes;  // head_dim x element bytes
};

// The append write on its own: one wavefront per (sequence, KV head).
pa_status launch_append(const AppendArgs &a, const int32_t *context_lens, int32_t num_seqs,
                        hipStream_t stream);

// Balanced decode (every workgroup an equal share of the rounds). A unit
// that crosses workgroup boundaries is computed in pieces; each piece's
// softmax state goes to a scratch slot, and a second, small kernel merges
// the pieces of every such unit. Scratch layout: one merge entry per
// workgroup, int4 (sequence, KV head, partition, piece count; count 0 = no
// unit to merge) - written by the decode kernel for the cut unit that
// starts in that workgroup - padded to 256 bytes; then two piece slots per
// workgroup of BAL_SLOT_FLOATS floats: the unnormalised output
// [BAL_GMAX][256], the running maxima [BAL_GMAX] (log2 domain), the sums
// [BAL_GMAX], a poison flag, padding. Every byte the merge reads was
// written by the decode launch before it, so scratch needs no initial
// contents.
constexpr int BAL_MAX_SEQS = 1024;
constexpr int BAL_GMAX = 8;
constexpr int BAL_SLOT_FLOATS = BAL_GMAX * 256 + 4 * BAL_GMAX;
__host__ __device__ inline int64_t bal_entry_bytes(int grid) {
  return ((int64_t)grid * 16 + 255) & ~(int64_t)255;
}
int64_t bal_scratch_bytes(int grid);
// Scratch bytes the balanced kernels need on the current device.
int64_t bal_scratch_bytes_current();
// The static scratch of pa_decode_balanced_static on the current device
// (null, with *why set, when its address cannot be obtained), and its size.
void *bal_static_scratch(const char **why);
int64_t bal_static_scratch_limit();
// False when the shape is not covered (the caller then uses launch_decode).
bool launch_decode_balanced(const DecodeParams &p, hipStream_t stream);

pa_status launch_decode(const DecodeParams &p, hipStream_t stream);

// Specialised decode for BF16, head_dim 256, block_size % 16 == 0 (decode
// rows only). Returns false when the shape is not covered.
bool launch_decode_tiled(const DecodeParams &p, unsigned grid, hipStream_t stream);

// Matrix-core decode for BF16, head_dim 256, block_size % 16 == 0 (decode
// rows only). Returns false when the shape is not covered.
bool launch_decode_mfma(const DecodeParams &p, hipStream_t stream);
// Persistent grid of the matrix-core kernel for p, or 0 when that kernel does
// not take p (then neither a plan nor a planned launch applies).
int64_t decode_mfma_grid(const DecodeParams &p);


// Matrix-core decode over FP8 pools (head_dim 256, block_size % 16 == 0,
// partitions of a multiple of 32 tokens). Returns false when the shape is
// not covered.
bool launch_decode_fp8(const DecodeParams &p, hipStream_t stream);

// HBM read probe: 8 KiB blocks of a pool in the given order (see read_probe.hip).
int64_t read_probe_sink_words();
pa_status launch_read_probe(const void *pool, int64_t pool_bytes, const int32_t *order,
                            int32_t num_blocks, uint32_t *sink, hipStream_t stream);

pa_status launch_reduce(void *out, const float *part_out, const float *part_max,
                        const float *part_sum, const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_parts, int32_t out_bf16, hipStream_t stream,
                        const AppendArgs *append = nullptr);

struct PrefillParams {
  void *out;
  const void *query;
  const void *key_cache;
  const void *value_cache;
  const int32_t *block_tables;
  const int32_t *query_start_loc;
  const int32_t *context_lens;
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t max_query_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  float scale;
  int32_t out_bf16;
};

pa_status launch_prefill(const PrefillParams &p, hipStream_t stream);

// Matrix-core prefill for BF16, head_dim 256; false when the shape is not
// covered.
bool launch_prefill_mfma(const PrefillParams &p, hipStream_t stream);

}  // namespace pa
