/*
 * pa.h - C ABI of libpa.so: paged KV cache writes, paged decode attention
 * (single pass, and split-context partitions with a log-sum-exp reduce),
 * chunked paged prefill, and a host-side block allocator, for AMD MI355X
 * (gfx950).
 *
 * Sources the operations follow (cited by page title and section):
 *  [P1] "High-Throughput LLM Inference & Training: A Deep Dive into vLLM"
 *       (wpnews.pro), Fig. 1 and Fig. 2.
 *  [P2] "vLLM Architecture, Memory and Benchmarks Deep Dive" (wpnews.pro),
 *       sections 1-4.
 *  [P3] "Optimizing LLM Inference: A Deep Dive into vLLM's PagedAttention and
 *       Continuous Batching" (voronkin.com), KV-cache and PagedAttention
 *       sections.
 *  [P4] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
 *       (syntaxis blog), "Memory-Efficient KV Cache Storage", "Garbage
 *       Collection & Reuse", "FlashAttention-2 Integration".
 *
 * Conventions shared by every device entry point
 * ----------------------------------------------
 *  - Every tensor argument is a caller-owned, contiguous buffer; "[device]"
 *    marks device memory on the current HIP device, "[host]" host memory.
 *    The library never allocates, frees or keeps a pointer after returning.
 *  - KV pools (one for keys, one for values), [P2] s.2 "fixed-size physical
 *    blocks", [P3] "logical block ID mapped to a physical block ID":
 *        key_cache, value_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *    Logical position t of sequence s lives in physical block
 *    block_tables[s][t / block_size] at offset t % block_size.
 *  - block_tables : int32 [num_seqs][max_blocks_per_seq] ([P2] s.2 block
 *    table); entries past a sequence's last block are never read.
 *  - context_lens : int32 [num_seqs], tokens cached for each sequence,
 *    counting the token written this step ([P2] s.1: the new token attends
 *    over the cached K/V of the tokens before it and of itself).
 *  - Grouped-query heads ([P2] s.1): query head h reads KV head
 *    h / (num_q_heads / num_kv_heads).
 *  - Calls are asynchronous and ordered on `stream` (0 = null stream).
 *  - Host-checkable arguments are validated before anything is launched:
 *    PA_EINVAL for bad sizes/pointers, PA_EUNSUPPORTED for shapes or dtypes
 *    the kernels do not cover. pa_last_error() then describes the problem.
 *  - Device-side contents are checked only as far as memory safety needs:
 *    a block id outside [0, num_blocks) or a context longer than
 *    max_blocks_per_seq * block_size never causes an out-of-range access; the
 *    affected (sequence, head) outputs are set to NaN instead. A slot outside
 *    [0, num_blocks * block_size) is not written.
 *  - Nothing throws or aborts across the ABI.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_EINVAL = 1,        /* invalid argument (null pointer, bad size, ...)    */
  PA_EUNSUPPORTED = 2,  /* valid, but a shape/dtype the kernels do not cover */
  PA_ENOMEM = 3,        /* allocator: not enough free blocks                 */
  PA_EHIP = 4,          /* a HIP runtime call failed (launch error, ...)     */
  PA_ENOTFOUND = 5      /* allocator: unknown sequence id                    */
} pa_status;

/* PA_FP8_E4M3: one-byte OCP E4M3FN codes (pools of the *_fp8 entry points,
 * pa_copy_blocks and pa_swap_blocks only; see pa_reshape_and_cache_fp8). */
typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Message describing the last non-OK status returned on this thread
 * ("" if none). The string stays valid until the next call on the thread. */
const char *pa_last_error(void);

/* Library version string, e.g. "0.1.0". */
const char *pa_version(void);

/*
 * pa_reshape_and_cache - slot-mapped write of this step's new K/V rows into
 * the pools ([P2] s.1 KV caching; [P2] s.2 on-demand blocks: each new token
 * goes to its sequence's last block).
 *
 *  key, value   [device] kv_dtype [num_tokens][num_kv_heads][head_dim]
 *  key_cache,
 *  value_cache  [device] kv_dtype pools (layout above), updated in place
 *  slot_mapping [device] int64 [num_tokens]; slot = block * block_size +
 *               offset. A negative slot skips the token.
 * A bit copy: the pools receive the exact bits of key/value.
 * num_tokens == 0 is a no-op. head_dim in [1, 1024].
 */
pa_status pa_reshape_and_cache(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, pa_dtype kv_dtype,
                               hipStream_t stream);

/*
 * pa_copy_blocks - apply copy-on-write clones ([P2] s.2 "Copy-on-Write (CoW)
 * Branching": a block shared by forked sequences is duplicated when they
 * diverge; pa_alloc_take_copies lists the pairs). For each pair, all
 * num_kv_heads x block_size rows of block src are copied to block dst, in
 * both pools.
 *  key_cache,
 *  value_cache  [device] kv_dtype pools (layout above), updated in place;
 *               kv_dtype PA_F32, PA_BF16 or PA_FP8_E4M3
 *  block_pairs  [device] int32 [num_pairs][2] = (src, dst)
 * A pair with an id outside [0, num_blocks), or with src == dst, is skipped.
 * Destinations must be distinct and never the source of another pair (the
 * allocator's pairs are); otherwise the result is unspecified. A bit copy.
 * num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void *key_cache, void *value_cache, const int32_t *block_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype kv_dtype,
                         hipStream_t stream);

/*
 * pa_swap_blocks - move whole blocks between two pairs of pools, one of which
 * is usually in pinned host memory ([P4] "Memory-Efficient KV Cache Storage":
 * blocks move between GPU and CPU memory; when GPU memory runs short they are
 * paged out to host memory; pa_alloc_swap_out / pa_alloc_swap_in list the
 * pairs). For each pair, block src of the source pools (all num_kv_heads x
 * block_size rows, both pools) is copied to block dst of the destination
 * pools; the copy runs in one kernel that reads or writes the host side over
 * the bus.
 *  src_key_cache,
 *  src_value_cache  [device or pinned host] kv_dtype [src_num_blocks][...]
 *  dst_key_cache,
 *  dst_value_cache  [device or pinned host] kv_dtype [dst_num_blocks][...],
 *                   updated in place
 *  block_pairs      [device or pinned host] int32 [num_pairs][2] = (src, dst)
 * Pool layouts as above (FP8 pools included: a block is copied whole, so the
 * transposed value layout needs nothing special). "Pinned host" means memory
 * from hipHostMalloc (torch's pin_memory=True), which the device addresses
 * at the same pointer; every buffer's first and last byte are checked and
 * anything else (pageable memory, another device's memory) gives PA_EINVAL
 * before any launch. A pair with an id outside its pool is skipped; when
 * source and destination are the same pools a pair with src == dst is too.
 * Destinations must be distinct and, for the same pools, never a source.
 * A bit copy, asynchronous on stream: the host side must stay allocated and
 * untouched by the host until the stream has passed the copy.
 * num_pairs == 0 is a no-op.
 */
pa_status pa_swap_blocks(const void *src_key_cache, const void *src_value_cache,
                         int32_t src_num_blocks, void *dst_key_cache, void *dst_value_cache,
                         int32_t dst_num_blocks, const int32_t *block_pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype kv_dtype, hipStream_t stream);

/*
 * pa_read_probe - a measurement helper, not a step of the attention path: the
 * HBM read bandwidth of decode's access pattern. Decode streams its K/V as
 * 8 KiB (block, head) tiles gathered through the block table ([P2] s.1-2);
 * this call reads the 8 KiB blocks order[0..num_blocks) of pool with the
 * same non-temporal 16-byte loads, two blocks in flight per wavefront, and
 * folds every word into a per-lane XOR. The identity order gives a plain
 * streaming read, a random permutation the gather pattern.
 *  pool        [device] pool_bytes bytes; block b is bytes [8192 b, 8192 b + 8192)
 *  order       [device] int32 [num_blocks]; ids outside [0, pool_bytes / 8192)
 *              are skipped (read as zeros, no access)
 *  sink        [device] uint32 [sink_words], sink_words >= pa_read_probe_sink_words();
 *              the first pa_read_probe_sink_words() words are overwritten, and
 *              their XOR equals the XOR of all 32-bit words of the blocks read
 * PA_EINVAL for negative sizes, null pointers or a short sink.
 */
int64_t pa_read_probe_sink_words(void);
pa_status pa_read_probe(const void *pool, int64_t pool_bytes, const int32_t *order,
                        int32_t num_blocks, uint32_t *sink, int64_t sink_words,
                        hipStream_t stream);

/*
 * pa_decode - single-pass paged decode attention: one query token per
 * sequence attends over its whole paged context ([P3] PagedAttention section:
 * the scattered blocks "appear contiguous to the attention mechanism").
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_s[t][g]) V_s[t][g],
 *   t < context_lens[s], g = h / (num_q_heads / num_kv_heads).
 *
 *  out          [device] out_dtype [num_seqs][num_q_heads][head_dim]
 *  query        [device] kv_dtype  [num_seqs][num_q_heads][head_dim]
 *  key_cache,
 *  value_cache  [device] kv_dtype pools
 *  block_tables [device] int32 [num_seqs][max_blocks_per_seq]
 *  context_lens [device] int32 [num_seqs]; 0 gives an all-zero output row.
 * One workgroup per (sequence, KV head); best when num_seqs * num_kv_heads
 * is in the hundreds. For few long sequences use pa_decode_partitioned.
 * Supported: head_dim in {64, 128, 256}; num_q_heads / num_kv_heads <= 8;
 * kv_dtype F32 or BF16; out_dtype F32 or BF16; any block_size >= 1.
 */
pa_status pa_decode(void *out, const void *query, const void *key_cache,
                    const void *value_cache, const int32_t *block_tables,
                    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                    pa_dtype kv_dtype, pa_dtype out_dtype, hipStream_t stream);

/*
 * Bytes of fp32 workspace the split-context path needs:
 * part_out [num_seqs][num_q_heads][max_parts][head_dim] plus
 * part_max and part_sum [num_seqs][num_q_heads][max_parts] each.
 * Returns 0 for non-positive arguments.
 */
size_t pa_partition_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_parts);

/*
 * pa_decode_partitioned - split-context decode. Partition p of sequence s
 * covers positions [p*partition_size, min(T_s, (p+1)*partition_size)), where
 * T_s = context_lens[s]; partitions p >= ceil(T_s / partition_size) are not
 * written. For each (s, h, p) it writes
 *   part_out[s][h][p][:] = softmax-weighted V over the partition (normalised
 *                          within it),
 *   part_max[s][h][p]    = m_p, the reference logit the partition's
 *                          exponentials were taken against (close to its
 *                          largest scaled logit),
 *   part_sum[s][h][p]    = l_p = sum_t exp(logit_t - m_p) over the partition,
 * so m_p + ln(l_p) is the partition's log-sum-exp (only that sum is unique).
 *
 *  part_out, part_max, part_sum [device] fp32, shapes above (see
 *               pa_partition_workspace_bytes)
 *  other arguments as pa_decode.
 *  partition_size: multiple of block_size, >= 16.
 *  max_parts >= ceil(max_s T_s / partition_size) (the caller's bound; a
 *               longer context makes that sequence's outputs NaN).
 */
pa_status pa_decode_partitioned(float *part_out, float *part_max, float *part_sum,
                                const void *query, const void *key_cache,
                                const void *value_cache, const int32_t *block_tables,
                                const int32_t *context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t num_blocks, float scale, int32_t partition_size,
                                int32_t max_parts, pa_dtype kv_dtype, hipStream_t stream);

/*
 * pa_reduce - log-sum-exp merge of the partitions written by
 * pa_decode_partitioned:
 *   w_p = part_sum_p * exp(part_max_p - max_q part_max_q),
 *   out[s][h] = sum_p w_p * part_out_p / sum_p w_p, p < ceil(T_s/partition_size).
 *
 *  out          [device] out_dtype [num_seqs][num_q_heads][head_dim]
 *  part_*       [device] as written by pa_decode_partitioned
 *  context_lens [device] int32 [num_seqs]; 0 gives an all-zero row.
 * A sequence whose context needs more than max_parts partitions gets a NaN
 * row. max_parts <= 1024 (PA_EUNSUPPORTED otherwise).
 */
pa_status pa_reduce(void *out, const float *part_out, const float *part_max,
                    const float *part_sum, const int32_t *context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                    int32_t max_parts, pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_decode_step - one decode step of one layer in one call: the step's K/V
 * rows join the cache and every sequence's query attends over its whole
 * context, this step's token included ("vLLM Architecture, Memory and
 * Benchmarks Deep Dive", s.1 and s.2; "Optimizing LLM Inference ...
 * PagedAttention" (voronkin.com): blocks reached through the table appear
 * contiguous to attention).
 *
 * The step's token of sequence s is position T_s - 1 (T_s = context_lens[s]
 * counts it). Its rows key[s], value[s] are written to the slot its block
 * table gives, table[s][(T_s - 1) / block_size] * block_size +
 * (T_s - 1) % block_size; T_s = 0, T_s past the table's capacity or a block
 * id outside the pool writes nothing (and decode then poisons that sequence's
 * outputs as usual). The results equal pa_reshape_and_cache with those slots
 * followed by pa_decode (partition_size == 0) or by pa_decode_partitioned and
 * pa_reduce (partition_size > 0), within the same tolerance: the matrix-core
 * kernel reads the step's token from key/value in a tile of its own, so its
 * sums run in another order than the separate calls'.
 *
 * Where the matrix-core kernel covers the shape (BF16, head_dim 256, block
 * size a multiple of 16, and in split mode more units than compute units
 * with partitions of at least 256 tokens) this is two launches: the decode,
 * then the merge (or, in single pass, the write) with the slot write inside
 * it. Otherwise it is the write, the decode and the merge.
 *
 *  out            [device] out_dtype [num_seqs][num_q_heads][head_dim]
 *  part_out, part_max, part_sum  [device] fp32 workspace as for
 *                 pa_decode_partitioned (may be NULL when partition_size == 0)
 *  query          [device] kv_dtype [num_seqs][num_q_heads][head_dim]
 *  key, value     [device] kv_dtype [num_seqs][num_kv_heads][head_dim]: the
 *                 step's rows (read only)
 *  key_cache, value_cache  [device] pools as for pa_reshape_and_cache
 *                 (written at the step's slots only)
 *  block_tables, context_lens, sizes, scale  as pa_decode
 *  partition_size 0 (single pass) or as pa_decode_partitioned; max_parts as
 *                 there
 *  kv_dtype       PA_F32 or PA_BF16
 *  plan, plan_epoch  [device] NULL (each launch plans for itself), or a
 *                 plan buffer and its epoch (see pa_decode_plan_bytes)
 * Errors as pa_decode_partitioned and pa_reduce; every check is made before
 * anything is launched, except that a failing later launch can leave the
 * earlier ones queued.
 */
pa_status pa_decode_step(void *out, float *part_out, float *part_max, float *part_sum,
                         const void *query, const void *key, const void *value, void *key_cache,
                         void *value_cache, const int32_t *block_tables,
                         const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                         int32_t partition_size, int32_t max_parts, pa_dtype kv_dtype,
                         pa_dtype out_dtype, void *plan, uint32_t plan_epoch,
                         hipStream_t stream);

/*
 * Decode plans. The persistent matrix-core decode kernel starts by reading
 * the context lengths, dealing the (sequence, KV head, partition) units to
 * its workgroups and looking up each wave's first block ids: three dependent
 * memory round trips before its first K/V load. Every layer of a decode step
 * has the same lengths and tables ("vLLM Architecture, Memory and Benchmarks
 * Deep Dive", s.2: one block table per sequence serves its whole cache), so
 * the deal can be made once per step and read by each later layer's launch
 * in one round trip.
 *
 * A plan buffer ([device], pa_decode_plan_bytes() bytes on the current
 * device, any initial contents) is a cache of that deal, one slot per
 * workgroup, each tagged with the launch that wrote it: entry point kind,
 * grid, num_seqs, partition_size and the caller's plan_epoch. A launch given
 * a buffer and an epoch reads its slot when the tag matches, and otherwise
 * plans as usual and writes the slot. An epoch with bit 31 set always plans
 * and stores the slots under the epoch without that bit: a step's first
 * layer can pass E | 0x80000000 and the later layers E, the same values every
 * step (so a captured graph replays correctly). The caller's contract: a
 * launch that reads (bit 31 clear) finds slots written for the same
 * context_lens, block_tables and sizes (take a new epoch whenever they
 * change, or refresh with bit 31); with a stale plan the outputs are wrong
 * (the kernel still never accesses memory outside the caller's buffers).
 * Launches that share a buffer must run in order (one stream). Where the
 * matrix-core kernel does not take the shape the buffer is not used. Results
 * are bit for bit those of the calls without a plan.
 *
 * A launch that plans and stores its slots deals the units longest-first by
 * work (each, largest first, to the workgroup with the least work so far)
 * where that can beat the plain deal of launches without a buffer, for
 * batches of up to 64 sequences. That deal takes longer to make (about 11 us
 * against 2 us on a 64-sequence batch with 420 units) and is repaid by the
 * launches that read it: pass a buffer when later layers will read the plan.
 */
size_t pa_decode_plan_bytes(void);

/* pa_decode_partitioned with a plan buffer and epoch (above): same
 * arguments otherwise, results bit for bit equal to pa_decode_partitioned's. */
pa_status pa_decode_partitioned_planned(float *part_out, float *part_max, float *part_sum,
                                        const void *query, const void *key_cache,
                                        const void *value_cache, const int32_t *block_tables,
                                        const int32_t *context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t max_blocks_per_seq, int32_t num_blocks,
                                        float scale, int32_t partition_size, int32_t max_parts,
                                        pa_dtype kv_dtype, void *plan, uint32_t plan_epoch,
                                        hipStream_t stream);

/*
 * Balanced decode: the same operations as pa_decode and
 * pa_decode_partitioned (same arguments, outputs and error behaviour), with
 * the batch's work cut into equal shares, one per compute unit, whatever the
 * mix of context lengths ([P2] s.3: a continuous batch mixes short and long
 * requests). Work is counted in rounds of 128 tokens of one KV head; a
 * unit (one output record: a (sequence, KV head), or a (sequence, KV head,
 * partition)) that straddles two shares is computed in pieces whose softmax
 * states (running max, sum, unnormalised output) go to `scratch`; a second,
 * small kernel launched by the same call merges each such unit's pieces in a
 * fixed order with the log-sum-exp rule of pa_reduce and writes its record.
 * Results are deterministic and do not depend on physical block ids. In
 * single-pass mode no separate reduce is needed.
 *
 *  scratch        [device] caller-owned, 16-byte aligned, at least
 *                 pa_decode_scratch_bytes() bytes; no initial contents are
 *                 needed (every byte the merge reads is written earlier in
 *                 the same call). One buffer serves any number of calls
 *                 issued in order on one stream; calls that may run at the
 *                 same time (other streams) must not share one.
 *  scratch_bytes  its size in bytes (PA_EINVAL when smaller than needed).
 * Covered on the matrix cores: BF16 pools, head_dim 256, block_size a
 * multiple of 16, num_seqs <= 1024, query heads per KV head <= 8, partition
 * sizes that are multiples of 16; other supported shapes run the kernels of
 * pa_decode / pa_decode_partitioned and leave scratch untouched.
 */
size_t pa_decode_scratch_bytes(void); /* for the current device: a 16-byte
                                         merge entry and two piece slots of
                                         8,320 bytes per compute unit */
pa_status pa_decode_balanced(void *out, const void *query, const void *key_cache,
                             const void *value_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                             pa_dtype kv_dtype, pa_dtype out_dtype, void *scratch,
                             size_t scratch_bytes, hipStream_t stream);
/*
 * pa_decode_balanced_static - pa_decode_balanced for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without
 * scratch, the same results. Its scratch is a static array inside the
 * library, 8 MiB per GPU it runs on, held until the process ends; no call
 * allocates or frees anything. Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (other streams) race;
 * nothing in it needs to start at zero. PA_EUNSUPPORTED when the device
 * would need more than 8 MiB (pa_decode_scratch_bytes() above it, i.e. more
 * than 503 compute units); PA_EHIP when the array's device address cannot
 * be obtained.
 */
pa_status pa_decode_balanced_static(void *out, const void *query, const void *key_cache,
                                    const void *value_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, float scale, pa_dtype kv_dtype,
                                    pa_dtype out_dtype, hipStream_t stream);
pa_status pa_decode_partitioned_balanced(float *part_out, float *part_max, float *part_sum,
                                         const void *query, const void *key_cache,
                                         const void *value_cache, const int32_t *block_tables,
                                         const int32_t *context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int32_t num_blocks,
                                         float scale, int32_t partition_size, int32_t max_parts,
                                         pa_dtype kv_dtype, void *scratch, size_t scratch_bytes,
                                         hipStream_t stream);

/*
 * pa_prefill_chunk - chunked paged prefill ([P2] s.4 chunked prefill; [P4]
 * "FlashAttention-2 Integration": causal attention over packed, unpadded
 * queries). The chunk's own K/V must already be in the pools
 * (pa_reshape_and_cache). Queries of sequence s are the packed rows
 * query_start_loc[s] .. query_start_loc[s+1]-1; with n_s rows they sit at
 * positions T_s - n_s .. T_s - 1 (T_s = context_lens[s]) and query j attends
 * causally to positions 0 .. T_s - n_s + j.
 *
 *  out             [device] out_dtype [num_q_tokens][num_q_heads][head_dim]
 *  query           [device] kv_dtype  [num_q_tokens][num_q_heads][head_dim]
 *  query_start_loc [device] int32 [num_seqs + 1], non-decreasing, starting at 0
 *  context_lens    [device] int32 [num_seqs], T_s >= n_s (else NaN rows)
 *  num_q_tokens    rows of query/out; rows at or past it are never touched
 *  max_query_len   host bound on n_s (sizes the launch grid); queries past
 *                  it are not computed
 * Supported: kv_dtype BF16, head_dim 256 or 128 or 64, num_q_heads /
 * num_kv_heads <= 8. With head_dim 256, an even block_size and
 * max_blocks_per_seq <= 2048, Q.K^T and P.V run on the matrix cores (MFMA,
 * BF16 operands, fp32 accumulation, P rounded to BF16); other supported
 * shapes run on the vector units with fp32 arithmetic.
 */
pa_status pa_prefill_chunk(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *query_start_loc, const int32_t *context_lens,
                           int32_t num_seqs, int32_t num_q_tokens, int32_t max_query_len,
                           int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                           pa_dtype kv_dtype, pa_dtype out_dtype, hipStream_t stream);

/*
 * FP8 KV cache. The pools hold one-byte E4M3FN codes (OCP 8-bit floating
 * point: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, values
 * down to 2^-9, largest finite magnitude 448, no infinities, 0x7F / 0xFF
 * NaN), with one scale per pool: a code c with scale s stands for
 * value(c) * s. Halving the bytes per element halves both the cache's size
 * and the bytes decode streams ([P3] KV-cache section: the cache size is
 * linear in the bytes per element; [P2] s.1: decode is bound by memory
 * traffic). The pages fix no quantised format; this one is the library's
 * choice. The block table and slots mean what they mean above. Layouts
 * (element size 1):
 *  key_cache    uint8 [num_blocks][num_kv_heads][block_size][head_dim]  (as above)
 *  value_cache  uint8 [num_blocks][num_kv_heads][head_dim][block_size]  (each block
 *               transposed, token index fastest: the tokens of one channel are
 *               adjacent, so the P.V contraction loads 16 tokens of a channel at once)
 * pa_copy_blocks copies whole blocks, so it serves these pools unchanged.
 *
 * pa_reshape_and_cache_fp8 - the slot-mapped write of pa_reshape_and_cache,
 * quantising on the way: the code stored for element x of key (value) is
 * the E4M3 value nearest to the fp32 quotient x / k_scale (x / v_scale),
 * computed as a correctly rounded fp32 division; ties round to even,
 * magnitudes of 448 and above (and infinities) become +-448, NaN becomes
 * 0x7F.
 *  key, value   [device] in_dtype (PA_F32 or PA_BF16) [num_tokens][num_kv_heads][head_dim]
 *  key_cache,
 *  value_cache  [device] uint8 code pools, updated in place
 *  slot_mapping [device] int64 [num_tokens] (negative: token skipped)
 *  k_scale, v_scale  finite, > 0 (PA_EINVAL otherwise)
 * num_tokens == 0 is a no-op. head_dim in [1, 1024].
 */
pa_status pa_reshape_and_cache_fp8(const void *key, const void *value, uint8_t *key_cache,
                                   uint8_t *value_cache, const int64_t *slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, pa_dtype in_dtype,
                                   float k_scale, float v_scale, hipStream_t stream);

/*
 * pa_decode_fp8 / pa_decode_partitioned_fp8 - pa_decode and
 * pa_decode_partitioned over FP8 pools: attention over the dequantised
 * cache, K_t = value(code) * k_scale and V_t = value(code) * v_scale.
 * query is BF16 [num_seqs][num_q_heads][head_dim]; the other arguments,
 * outputs, workspace layout and error behaviour are those of the BF16 entry
 * points (pa_reduce merges the partitions). Codes widen to BF16 exactly;
 * the K scale is applied to the logits and the V scale to the outputs, in
 * fp32. Supported shapes as pa_decode (head_dim 64/128/256, groups <= 8);
 * head_dim 256 with block_size a multiple of 16 takes the persistent matrix-core kernel.
 */
pa_status pa_decode_fp8(void *out, const void *query, const uint8_t *key_cache,
                        const uint8_t *value_cache, const int32_t *block_tables,
                        const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                        float k_scale, float v_scale, pa_dtype out_dtype, hipStream_t stream);

pa_status pa_decode_partitioned_fp8(float *part_out, float *part_max, float *part_sum,
                                    const void *query, const uint8_t *key_cache,
                                    const uint8_t *value_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, float scale, float k_scale,
                                    float v_scale, int32_t partition_size, int32_t max_parts,
                                    hipStream_t stream);

/* pa_decode_partitioned_fp8 with a plan buffer and epoch (see
 * pa_decode_plan_bytes); a BF16 launch's slots are not read here, nor the
 * other way round. Results bit for bit pa_decode_partitioned_fp8's. */
pa_status pa_decode_partitioned_fp8_planned(float *part_out, float *part_max, float *part_sum,
                                            const void *query, const uint8_t *key_cache,
                                            const uint8_t *value_cache,
                                            const int32_t *block_tables,
                                            const int32_t *context_lens, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size,
                                            int32_t max_blocks_per_seq, int32_t num_blocks,
                                            float scale, float k_scale, float v_scale,
                                            int32_t partition_size, int32_t max_parts,
                                            void *plan, uint32_t plan_epoch, hipStream_t stream);

/*
 * Host block allocator ([P2] s.2 "On-Demand Allocation": blocks are handed
 * out only as tokens arrive, so only a sequence's last block has unused
 * slots; [P2] s.3: a finished sequence's blocks return to the pool at once;
 * [P4] "Garbage Collection & Reuse": free blocks form a first-in first-out
 * queue). Host memory only; not thread-safe (one allocator per thread or
 * external locking). No device memory is touched.
 */
typedef struct pa_alloc pa_alloc;

/* Create a pool of num_blocks blocks of block_size tokens. initial_order
 * [host] int32 [num_blocks] is the initial free-queue order (a permutation of
 * 0..num_blocks-1; NULL = 0, 1, 2, ...). On success *out owns the allocator. */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t *initial_order,
                          pa_alloc **out);
void pa_alloc_destroy(pa_alloc *a);

/* Grow sequence seq_id (created on first use) by num_tokens tokens, taking
 * blocks from the front of the free queue only when its last block is full.
 * slots_out [host] int64 [num_tokens] or NULL receives each new token's slot.
 * All or nothing: on PA_ENOMEM nothing changes. */
pa_status pa_alloc_append(pa_alloc *a, int64_t seq_id, int32_t num_tokens, int64_t *slots_out);

/* Release seq_id and forget it: each of its blocks loses one holder, and
 * the blocks no other sequence holds go to the back of the free queue (in the
 * sequence's logical order). PA_ENOTFOUND if unknown. */
pa_status pa_alloc_free(pa_alloc *a, int64_t seq_id);

/* Copy-on-write branching ([P2] s.2 "Copy-on-Write (CoW) Branching": forked
 * rollouts share the prompt's physical blocks, cloned only when they
 * diverge). Start child_id as a sharer of every block of parent_id (same
 * table, same length); nothing is copied now. PA_ENOTFOUND if parent_id is
 * unknown, PA_EINVAL if child_id exists.
 * Appends then copy on write: an append to a sequence whose last block is
 * shared and has free slots first takes a fresh block from the front of the
 * free queue and queues the copy (old block -> fresh block); the last holder
 * of a block writes in place. The queued copies must be applied to both pools
 * (pa_copy_blocks) before the step's new K/V are written. */
pa_status pa_alloc_fork(pa_alloc *a, int64_t parent_id, int64_t child_id);

/* Take the queued copies: pairs_out [host] int32 [max_pairs][2] receives
 * (source, destination) block ids in the order they were queued and the
 * queue is emptied. Returns the number of queued pairs; if that exceeds
 * max_pairs nothing is taken (call again with room for that many). -1 for a
 * NULL allocator or bad arguments. */
int32_t pa_alloc_take_copies(pa_alloc *a, int32_t *pairs_out, int32_t max_pairs);

/* Number of sequences holding block (0 = free), or -1 if out of range. */
int32_t pa_alloc_block_refs(const pa_alloc *a, int32_t block);

/* One step of an iteration-level decode loop ([P2] s.3 "Continuous
 * Batching": every iteration each running sequence gets its next token, and
 * finished ones leave at once), in one call: append num_tokens[i] tokens to
 * seq_ids[i] for i < n (as pa_alloc_append, copy on write included), then
 * write the block-table rows and context lengths of the n sequences (as
 * pa_alloc_block_table).
 *  seq_ids    [host] int64 [n], distinct
 *  num_tokens [host] int32 [n], >= 0
 *  slots_out  [host] int64 [sum num_tokens]: the new tokens' slots, sequence
 *             by sequence in the order of seq_ids (NULL allowed if the sum is 0)
 *  table_out  [host] int32 [n][max_blocks], unused entries -1
 *  lens_out   [host] int32 [n] or NULL
 * All or nothing: PA_ENOMEM if the step needs more blocks (growth plus
 * copy-on-write replacements) than are free, PA_EINVAL for a sequence listed
 * twice or one that would hold more than max_blocks blocks; nothing changes
 * then. Copies are queued as by pa_alloc_append. */
pa_status pa_alloc_step(pa_alloc *a, const int64_t *seq_ids, const int32_t *num_tokens, int32_t n,
                        int64_t *slots_out, int32_t max_blocks, int32_t *table_out,
                        int32_t *lens_out);

/* Swapping to host memory ([P4] "Memory-Efficient KV Cache Storage": when
 * GPU memory runs short, blocks are paged out to host memory; "The
 * Scheduler": requests are suspended under memory pressure). The unit is a
 * whole sequence.
 *
 * pa_alloc_set_host_pool - give the allocator a host pool of num_host_blocks
 * blocks (ids 0..num_host_blocks-1) with its own first-in first-out free
 * queue in initial_order ([host] int32 [num_host_blocks], a permutation, or
 * NULL = 0, 1, 2, ...). Replaces any earlier host pool; PA_EINVAL while a
 * sequence is swapped out. Without a call the host pool is empty. */
pa_status pa_alloc_set_host_pool(pa_alloc *a, int32_t num_host_blocks,
                                 const int32_t *initial_order);

/* Free blocks of the host pool; -1 if a is NULL. */
int32_t pa_alloc_num_free_host(const pa_alloc *a);

/* 1 if seq_id is swapped out, 0 if it is on device blocks, -1 if unknown. */
int32_t pa_alloc_is_swapped(const pa_alloc *a, int64_t seq_id);

/* pa_alloc_swap_out - move seq_id to host blocks: one host block per device
 * block, from the front of the host queue, in logical order; then the device
 * blocks are released as by pa_alloc_free (a block another table holds stays
 * with it). pairs_out [host] int32 [max_pairs][2] receives the (device block,
 * host block) moves in logical order, *num_pairs their count (the sequence's
 * block count, ceil(len / block_size)). Apply them with pa_swap_blocks
 * (device pools -> host pools) after any copy-on-write pairs taken before the
 * call and before the freed device blocks are written again.
 * pa_alloc_swap_in - the reverse: one device block per host block from the
 * front of the device queue; pairs_out receives (host block, device block);
 * the host blocks go to the back of the host queue. Blocks shared before a
 * swap-out come back as the sequence's own.
 * Both are all or nothing: PA_ENOMEM if the receiving side has too few free
 * blocks, PA_EINVAL if max_pairs is too small or the sequence is already on
 * that side, PA_ENOTFOUND for an unknown id; nothing changes then. A
 * swapped-out sequence keeps its length; pa_alloc_append, pa_alloc_fork,
 * pa_alloc_step and pa_alloc_block_table refuse it (PA_EINVAL) and
 * pa_alloc_free returns its host blocks to the back of the host queue. */
pa_status pa_alloc_swap_out(pa_alloc *a, int64_t seq_id, int32_t max_pairs, int32_t *pairs_out,
                            int32_t *num_pairs);
pa_status pa_alloc_swap_in(pa_alloc *a, int64_t seq_id, int32_t max_pairs, int32_t *pairs_out,
                           int32_t *num_pairs);

/* Free blocks in the pool; -1 if a is NULL. */
int32_t pa_alloc_num_free(const pa_alloc *a);

/* Tokens held by seq_id, or -1 if unknown. */
int32_t pa_alloc_seq_len(const pa_alloc *a, int64_t seq_id);

/* Write block-table rows and context lengths for n sequences.
 *  seq_ids   [host] int64 [n]
 *  table_out [host] int32 [n][max_blocks], unused entries set to -1
 *  lens_out  [host] int32 [n] or NULL
 * PA_EINVAL if a sequence holds more than max_blocks blocks,
 * PA_ENOTFOUND for an unknown id (outputs then unspecified). */
pa_status pa_alloc_block_table(const pa_alloc *a, const int64_t *seq_ids, int32_t n,
                               int32_t max_blocks, int32_t *table_out, int32_t *lens_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
