// Chunked paged prefill launcher.
//
// BF16 caches with head_dim 256 run on the matrix-core kernel
// (prefill_mfma.hip). Other shapes take the general path: each packed query
// row of a sequence's chunk is a decode over the prefix of that sequence up
// to and including the row's own position (causal), run by the generic
// paged decode kernel.
#include "launch.h"
#include "pa_device.h"

namespace pa {

pa_status launch_prefill(const PrefillParams &p, hipStream_t stream) {
  if (launch_prefill_mfma(p, stream)) return check_launch("pa_prefill_chunk");
  DecodeParams d{};
  d.query = p.query;
  d.key_cache = p.key_cache;
  d.value_cache = p.value_cache;
  d.block_tables = p.block_tables;
  d.context_lens = p.context_lens;
  d.query_start_loc = p.query_start_loc;
  d.max_query_len = p.max_query_len;
  d.num_q_tokens = p.num_q_tokens;
  d.out = p.out;
  d.num_seqs = p.num_seqs;
  d.num_q_heads = p.num_q_heads;
  d.num_kv_heads = p.num_kv_heads;
  d.head_dim = p.head_dim;
  d.block_size = p.block_size;
  d.max_blocks_per_seq = p.max_blocks_per_seq;
  d.num_blocks = p.num_blocks;
  d.scale = p.scale;
  d.partition_size = 0;
  d.max_parts = 1;
  d.kv_bf16 = 1;
  d.out_bf16 = p.out_bf16;
  return launch_decode(d, stream);
}

}  // namespace pa
