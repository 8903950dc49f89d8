"""Paged attention in float64 (oracle; test infrastructure only).

The pages describe paging as a pure re-indexing: logical block IDs map to
physical block IDs so that a sequence's cache may sit anywhere in memory yet
"appear contiguous to the attention mechanism" ("Optimizing LLM Inference"
(voronkin.com), section "PagedAttention: Borrowing a 50-Year-Old OS
Masterpiece"; "vLLM Architecture, Memory and Benchmarks Deep Dive", section 2,
block table). So the oracle first reassembles each sequence's logical cache
through its block table and then applies textbook softmax attention to it; no
blocking, fusion or online rescaling.

Conventions (readings where the pages are silent; listed in the design notes):
* Pools are laid out [num_blocks][num_kv_heads][block_size][head_dim]; logical
  position t of a sequence lives in physical block table[t // block_size] at
  offset t % block_size.
* Grouped-query attention ("vLLM Architecture ... Deep Dive", section 1:
  fewer KV heads than query heads): query head h reads KV head
  h // (num_q_heads // num_kv_heads).
* ``context_lens`` counts the cached tokens including the one written this
  step, so a decode query attends to every cached token, itself included
  (section 1 of the same page: the new token attends over the tokens before
  it, whose K and V are cached).
* A sequence with zero context yields an all-zero output and no partitions.
* Prefill ("vLLM Architecture ... Deep Dive", section 4, chunked prefill;
  "Inside vLLM", "FlashAttention-2 Integration": causal attention over
  unpadded, packed queries): the n queries of a sequence's chunk are its last
  n positions; query j attends to positions 0 .. context_len - n + j.

All arithmetic is float64; inputs are upcast first (BF16 inputs arrive already
rounded, as float32 values that BF16 represents exactly).
"""

import numpy as np


def cache_write(key_cache, value_cache, key, value, slot_mapping, block_size):
    """Slot-mapped write of new K/V rows into copies of the two pools.

    key/value: [num_tokens][num_kv_heads][head_dim]. For token i with
    slot = slot_mapping[i] >= 0, block = slot // block_size and
    offset = slot % block_size receive the row; negative slots are skipped.
    A pure copy in the pools' own dtype, so the result is bit-exact.
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = slot // block_size, slot % block_size
        kc[blk, :, off, :] = key[i]
        vc[blk, :, off, :] = value[i]
    return kc, vc


def copy_blocks(key_cache, value_cache, block_pairs):
    """Copy-on-write duplication ("vLLM Architecture, Memory and Benchmarks
    Deep Dive", section 2, "Copy-on-Write (CoW) Branching": a shared block is
    cloned when the sequences holding it diverge) applied to copies of both
    pools: for each (src, dst) pair, every KV head and token row of block src
    is written to block dst. Pairs whose ids fall outside the pool are
    skipped. The destinations are distinct and never a source of another
    pair, so the pairs are independent. A bit copy."""
    kc = key_cache.copy()
    vc = value_cache.copy()
    nb = kc.shape[0]
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2).tolist():
        if not (0 <= src < nb and 0 <= dst < nb):
            continue
        kc[dst] = key_cache[src]
        vc[dst] = value_cache[src]
    return kc, vc


def swap_blocks(src_key, src_value, dst_key, dst_value, block_pairs):
    """Block moves between two pools of the same block shape ("Inside vLLM:
    Anatomy of a High-Throughput LLM Inference System", "Memory-Efficient KV
    Cache Storage": blocks are paged out to host memory and back): for each
    (src, dst) pair, every KV head and token row of block src of the source
    pools is written to block dst of copies of the destination pools. Pairs
    whose ids fall outside their pool are skipped. A bit copy."""
    kd = dst_key.copy()
    vd = dst_value.copy()
    ns, nd = src_key.shape[0], dst_key.shape[0]
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2).tolist():
        if not (0 <= src < ns and 0 <= dst < nd):
            continue
        kd[dst] = src_key[src]
        vd[dst] = src_value[src]
    return kd, vd


def gather_context(cache, block_table_row, context_len, block_size):
    """Logical [context_len][num_kv_heads][head_dim] view of one sequence's
    cache, rebuilt position by position through its block table."""
    num_kv_heads, head_dim = cache.shape[1], cache.shape[3]
    out = np.empty((context_len, num_kv_heads, head_dim), dtype=np.float64)
    for t in range(context_len):
        phys = int(block_table_row[t // block_size])
        out[t] = cache[phys, :, t % block_size, :]
    return out


def kv_head_of(h, num_q_heads, num_kv_heads):
    """KV head read by query head h: the query heads form num_kv_heads
    contiguous groups of num_q_heads // num_kv_heads heads each."""
    return h // (num_q_heads // num_kv_heads)


def _softmax_attend(q, K, V, scale):
    """softmax(scale * K q) weighted sum of V rows, plus log-sum-exp of the
    scaled logits. q: [d], K/V: [T][d], T >= 1."""
    z = scale * (K @ q)
    zmax = z.max()
    w = np.exp(z - zmax)
    total = w.sum()
    return (w @ V) / total, zmax + np.log(total)


def decode(query, key_cache, value_cache, block_tables, context_lens, block_size, scale):
    """One query token per sequence over its paged cache.

    query: [num_seqs][num_q_heads][head_dim]. Returns float64 of that shape.
    """
    q = np.asarray(query, dtype=np.float64)
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = key_cache.shape[1]
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        T = int(context_lens[s])
        if T == 0:
            continue
        K = gather_context(key_cache, block_tables[s], T, block_size)
        V = gather_context(value_cache, block_tables[s], T, block_size)
        for h in range(num_q_heads):
            g = kv_head_of(h, num_q_heads, num_kv_heads)
            out[s, h], _ = _softmax_attend(q[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def decode_partitions(query, key_cache, value_cache, block_tables, context_lens,
                      block_size, scale, partition_size, seqs=None, heads=None):
    """Split-context decode: partition p of sequence s covers positions
    [p * partition_size, min(T_s, (p + 1) * partition_size)).

    Returns (o, lse, num_parts): o[s][h][p] is softmax-weighted V within the
    partition (normalised inside it), lse[s][h][p] the log-sum-exp of its
    scaled logits, num_parts[s] = ceil(T_s / partition_size). Entries of
    absent partitions are NaN. ``seqs``/``heads`` restrict the work to a
    sample (other entries stay NaN).
    """
    q = np.asarray(query, dtype=np.float64)
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = key_cache.shape[1]
    num_parts = [-(-int(t) // partition_size) for t in context_lens]
    max_parts = max(num_parts) if num_parts else 0
    o = np.full((num_seqs, num_q_heads, max_parts, head_dim), np.nan)
    lse = np.full((num_seqs, num_q_heads, max_parts), np.nan)
    for s in (range(num_seqs) if seqs is None else seqs):
        T = int(context_lens[s])
        if T == 0:
            continue
        K = gather_context(key_cache, block_tables[s], T, block_size)
        V = gather_context(value_cache, block_tables[s], T, block_size)
        for h in (range(num_q_heads) if heads is None else heads):
            g = kv_head_of(h, num_q_heads, num_kv_heads)
            for p in range(num_parts[s]):
                lo, hi = p * partition_size, min(T, (p + 1) * partition_size)
                o[s, h, p], lse[s, h, p] = _softmax_attend(
                    q[s, h], K[lo:hi, g, :], V[lo:hi, g, :], scale)
    return o, lse, np.asarray(num_parts)


def merge_partitions(o, lse, num_parts):
    """Log-sum-exp merge of partition results into the full softmax result.

    With L = log-sum-exp over partitions of lse[p], the merged output is
    sum_p exp(lse[p] - L) * o[p]: each partition's normalised output weighted
    by its share of the total softmax mass.
    """
    num_seqs, num_q_heads, _, head_dim = o.shape
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        n = int(num_parts[s])
        if n == 0:
            continue
        for h in range(num_q_heads):
            l = lse[s, h, :n]
            top = l.max()
            total = top + np.log(np.exp(l - top).sum())
            out[s, h] = (np.exp(l - total)[:, None] * o[s, h, :n]).sum(axis=0)
    return out


def prefill(query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
            block_size, scale, seqs=None, rows=None):
    """Causal chunked prefill over the paged cache (chunk K/V already written).

    query: packed [num_q_tokens][num_q_heads][head_dim]; the queries of
    sequence s are rows query_start_loc[s] .. query_start_loc[s+1]-1 and sit
    at positions context_lens[s] - n_s .. context_lens[s] - 1.
    ``seqs`` restricts the work to some sequences and ``rows`` (a set of
    packed row indices) to some queries; skipped rows stay NaN.
    """
    q = np.asarray(query, dtype=np.float64)
    num_tokens, num_q_heads, head_dim = q.shape
    num_kv_heads = key_cache.shape[1]
    out = np.full((num_tokens, num_q_heads, head_dim), np.nan)
    num_seqs = len(query_start_loc) - 1
    for s in (range(num_seqs) if seqs is None else seqs):
        lo, hi = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n = hi - lo
        if n == 0:
            continue
        T = int(context_lens[s])
        K = gather_context(key_cache, block_tables[s], T, block_size)
        V = gather_context(value_cache, block_tables[s], T, block_size)
        for j in range(n):
            if rows is not None and lo + j not in rows:
                continue
            visible = T - n + j + 1
            for h in range(num_q_heads):
                g = kv_head_of(h, num_q_heads, num_kv_heads)
                out[lo + j, h], _ = _softmax_attend(
                    q[lo + j, h], K[:visible, g, :], V[:visible, g, :], scale)
    return out
