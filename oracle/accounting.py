"""KV-cache size and reservation accounting (oracle; test infrastructure only).

Sources:
* "Optimizing LLM Inference: A Deep Dive into vLLM's PagedAttention and
  Continuous Batching" (voronkin.com), section "Understanding the KV Cache
  Bottleneck", equation M_KV: two tensors (keys and values) times layers times
  KV heads times head dimension times tokens times bytes per element.
* "vLLM Architecture, Memory and Benchmarks Deep Dive", section 1 (the same
  variables, defined in prose) and section 2 (the allocation-policy widget).
* "High-Throughput LLM Inference & Training: A Deep Dive into vLLM",
  Fig. 1 (contiguous worst-case reservation) and Fig. 2 (paged blocks).
"""


def kv_cache_bytes(num_layers, num_kv_heads, head_dim, num_tokens, bytes_per_elem):
    """M_KV = 2 * L * H_KV * d_head * T * b (voronkin.com, eq. M_KV).

    The leading 2 counts keys and values. Integer arithmetic: exact.
    """
    return 2 * num_layers * num_kv_heads * head_dim * num_tokens * bytes_per_elem


def contiguous_reservation(token_counts, max_len):
    """Slots under the fixed worst-case policy of Fig. 1: every request
    reserves ``max_len`` slots regardless of how many tokens it holds.

    Returns (reserved, used, unused) in token slots.
    """
    reserved = len(token_counts) * max_len
    used = sum(token_counts)
    return reserved, used, reserved - used


def blocks_needed(num_tokens, block_size):
    """Whole blocks a sequence of ``num_tokens`` tokens occupies when blocks are
    handed out only as tokens arrive (vLLM Architecture Deep Dive, section 2,
    "On-Demand Allocation"): the ceiling of tokens over block size."""
    return -(-num_tokens // block_size)


def paged_reservation(token_counts, block_size):
    """Slots under the paged policy of Fig. 2: each request holds
    ceil(tokens / block_size) whole blocks.

    Returns (reserved, used, unused) in token slots.
    """
    reserved = sum(blocks_needed(t, block_size) * block_size for t in token_counts)
    used = sum(token_counts)
    return reserved, used, reserved - used
