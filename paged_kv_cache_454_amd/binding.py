"""Python binding of libpa.so with the C ABI's names.

Marshalling only: each function reads shapes, dtypes and device pointers off
torch tensors, checks that they are consistent (so the C side is handed the
true sizes of every buffer), passes the current HIP stream, calls the C entry
point and raises ``PAError`` on a non-OK status. Every step of the path runs
in the library's kernels; nothing here computes.
"""

import ctypes

import numpy as np
import torch

from ._lib import PA_BF16, PA_F32, PA_FP8_E4M3, PAError, check, lib  # noqa: F401

_DT = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}
# FP8 pools: E4M3FN codes, as uint8 or as torch's float8_e4m3fn.
_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _dtype(t, what):
    if t.dtype not in _DT:
        raise ValueError(f"{what}: dtype {t.dtype} (supported: float32, bfloat16)")
    return _DT[t.dtype]


def _dev(t, what, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{what}: {t.dim()} dims, expected {ndim}")
    if t.data_ptr() % 16 != 0 and t.numel() > 0:
        raise ValueError(f"{what}: data pointer must be 16-byte aligned")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _pool_shape(key_cache, value_cache):
    if key_cache.shape != value_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("key_cache and value_cache must match in shape and dtype")
    if key_cache.dim() != 4:
        raise ValueError("pools are [num_blocks][num_kv_heads][block_size][head_dim]")
    return key_cache.shape


def _fp8_pool_shape(key_cache, value_cache):
    """FP8 pools: keys [num_blocks][H_KV][block_size][d], values with each
    block transposed, [num_blocks][H_KV][d][block_size]; uint8 codes (or
    float8_e4m3fn)."""
    if key_cache.dtype not in _FP8 or value_cache.dtype not in _FP8:
        raise ValueError("FP8 pools must be uint8 or float8_e4m3fn")
    if key_cache.dim() != 4 or value_cache.dim() != 4:
        raise ValueError("pools are 4-d: keys [nb][H][bs][d], values [nb][H][d][bs]")
    nb, hkv, bs, d = key_cache.shape
    if tuple(value_cache.shape) != (nb, hkv, d, bs):
        raise ValueError("the FP8 value pool must be [num_blocks][num_kv_heads][head_dim][block_size]")
    return key_cache.shape


def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, stream=None):
    """Write key/value [num_tokens][H_KV][d] into the pools at slot_mapping."""
    num_blocks, hkv, bs, d = _pool_shape(key_cache, value_cache)
    if key.shape != value.shape or key.dim() != 3 or tuple(key.shape[1:]) != (hkv, d):
        raise ValueError("key/value must be [num_tokens][num_kv_heads][head_dim] matching the pools")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise ValueError("key/value dtype must match the pools")
    n = key.shape[0]
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != n:
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    args = [_dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
            _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping", torch.int64)]
    check(lib().pa_reshape_and_cache(*args, n, hkv, d, bs, num_blocks,
                                     _dtype(key_cache, "pools"), _stream(stream)))


def pa_copy_blocks(key_cache, value_cache, block_pairs, stream=None):
    """Copy whole blocks inside both pools: block_pairs is int32 [n][2] of
    (source, destination) ids (the allocator's copy-on-write pairs)."""
    fp8 = key_cache.dtype in _FP8
    num_blocks, hkv, bs, d = (_fp8_pool_shape if fp8 else _pool_shape)(key_cache, value_cache)
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int32 [num_pairs][2]")
    n = block_pairs.shape[0]
    dt = PA_FP8_E4M3 if fp8 else _dtype(key_cache, "pools")
    check(lib().pa_copy_blocks(_dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                               _dev(block_pairs, "block_pairs", torch.int32), n, hkv, d, bs,
                               num_blocks, dt, _stream(stream)))


def _reachable(t, what, dtype=None):
    """Pointer of a contiguous tensor in device memory or pinned host memory
    (the library checks that the device can address it)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{what}: must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if t.data_ptr() % 16 != 0 and t.numel() > 0:
        raise ValueError(f"{what}: data pointer must be 16-byte aligned")
    return t.data_ptr()


def pa_swap_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache, block_pairs,
                   stream=None):
    """Copy whole blocks from the source pools to the destination pools, one
    side usually pinned host memory (swap-out: device -> host; swap-in: host
    -> device). block_pairs: int32 [n][2] (source id, destination id), on the
    device or pinned."""
    fp8 = src_key_cache.dtype in _FP8
    shape = _fp8_pool_shape if fp8 else _pool_shape
    snb, hkv, bs, d = shape(src_key_cache, src_value_cache)
    dnb, hkv2, bs2, d2 = shape(dst_key_cache, dst_value_cache)
    if (hkv, bs, d) != (hkv2, bs2, d2) or src_key_cache.dtype != dst_key_cache.dtype:
        raise ValueError("source and destination pools must have the same block shape and dtype")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int32 [num_pairs][2]")
    dt = PA_FP8_E4M3 if fp8 else _dtype(src_key_cache, "pools")
    check(lib().pa_swap_blocks(
        _reachable(src_key_cache, "src_key_cache"), _reachable(src_value_cache, "src_value_cache"),
        snb, _reachable(dst_key_cache, "dst_key_cache"),
        _reachable(dst_value_cache, "dst_value_cache"), dnb,
        _reachable(block_pairs, "block_pairs", torch.int32), block_pairs.shape[0], hkv, d, bs,
        dt, _stream(stream)))


def pa_read_probe(pool, order, sink=None, stream=None):
    """Read the 8 KiB blocks ``order`` (int32, device) of ``pool`` (any device
    tensor, its bytes taken as the pool) with decode's loads; returns the
    uint32 sink whose XOR is the XOR of every word read. A measurement helper."""
    n = int(lib().pa_read_probe_sink_words())
    if sink is None:
        sink = torch.empty(n, dtype=torch.int32, device=pool.device)
    if order.dim() != 1:
        raise ValueError("order must be int32 [num_blocks]")
    check(lib().pa_read_probe(_dev(pool, "pool"), pool.numel() * pool.element_size(),
                              _dev(order, "order", torch.int32), order.shape[0],
                              _dev(sink, "sink"), sink.numel() * sink.element_size() // 4,
                              _stream(stream)))
    return sink


def pa_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                             stream=None):
    """Quantising write: the E4M3 codes of key / k_scale and value / v_scale
    (key/value float32 or bfloat16 [num_tokens][H_KV][d]) go into the uint8
    (or float8_e4m3fn) pools at slot_mapping."""
    num_blocks, hkv, bs, d = _fp8_pool_shape(key_cache, value_cache)
    if key.shape != value.shape or key.dim() != 3 or tuple(key.shape[1:]) != (hkv, d):
        raise ValueError("key/value must be [num_tokens][num_kv_heads][head_dim] matching the pools")
    if key.dtype != value.dtype:
        raise ValueError("key and value must share a dtype")
    n = key.shape[0]
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != n:
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    args = [_dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
            _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping", torch.int64)]
    check(lib().pa_reshape_and_cache_fp8(*args, n, hkv, d, bs, num_blocks, _dtype(key, "key"),
                                         float(k_scale), float(v_scale), _stream(stream)))


def _attn_common(query, key_cache, value_cache, block_tables, context_lens, rows_name,
                 fp8=False):
    num_blocks, hkv, bs, d = (_fp8_pool_shape if fp8 else _pool_shape)(key_cache, value_cache)
    if query.dim() != 3 or query.shape[2] != d:
        raise ValueError(f"query must be [{rows_name}][num_q_heads][{d}]")
    if fp8:
        if key_cache.dtype not in _FP8 or query.dtype != torch.bfloat16:
            raise ValueError("FP8 decode takes uint8 / float8_e4m3fn pools and a bfloat16 query")
    elif query.dtype != key_cache.dtype:
        raise ValueError("query dtype must match the pools")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be int32 [num_seqs][max_blocks_per_seq]")
    num_seqs = block_tables.shape[0]
    if context_lens.dim() != 1 or context_lens.shape[0] != num_seqs:
        raise ValueError("context_lens must be int32 [num_seqs]")
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    return num_blocks, hkv, bs, d, num_seqs


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
              stream=None):
    """Single-pass paged decode; out [num_seqs][H_q][d] (float32 or bfloat16)."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    if query.shape[0] != num_seqs or tuple(out.shape) != tuple(query.shape):
        raise ValueError("query/out must be [num_seqs][num_q_heads][head_dim]")
    hq = query.shape[1]
    check(lib().pa_decode(_dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
                          _dev(value_cache, "value_cache"), block_tables.data_ptr(),
                          context_lens.data_ptr(), num_seqs, hq, hkv, d, bs,
                          block_tables.shape[1], num_blocks, float(scale),
                          _dtype(key_cache, "pools"), _dtype(out, "out"), _stream(stream)))


def pa_partition_workspace_bytes(num_seqs, num_q_heads, head_dim, max_parts):
    return int(lib().pa_partition_workspace_bytes(num_seqs, num_q_heads, head_dim, max_parts))


def pa_decode_partitioned(part_out, part_max, part_sum, query, key_cache, value_cache,
                          block_tables, context_lens, scale, partition_size, stream=None):
    """Split-context decode into part_out [S][H_q][P][d], part_max/part_sum [S][H_q][P]."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    hq = query.shape[1]
    if query.shape[0] != num_seqs:
        raise ValueError("query must be [num_seqs][num_q_heads][head_dim]")
    if part_out.dim() != 4 or tuple(part_out.shape[:2]) != (num_seqs, hq) or part_out.shape[3] != d:
        raise ValueError("part_out must be float32 [num_seqs][num_q_heads][max_parts][head_dim]")
    max_parts = part_out.shape[2]
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (num_seqs, hq, max_parts):
            raise ValueError(f"{nm} must be float32 [num_seqs][num_q_heads][max_parts]")
    check(lib().pa_decode_partitioned(
        _dev(part_out, "part_out", torch.float32), _dev(part_max, "part_max", torch.float32),
        _dev(part_sum, "part_sum", torch.float32), _dev(query, "query"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), block_tables.data_ptr(),
        context_lens.data_ptr(), num_seqs, hq, hkv, d, bs, block_tables.shape[1], num_blocks,
        float(scale), int(partition_size), max_parts, _dtype(key_cache, "pools"),
        _stream(stream)))


def pa_decode_scratch_bytes():
    """Scratch bytes a balanced decode call needs on the current device."""
    return int(lib().pa_decode_scratch_bytes())


def decode_scratch(device=None):
    """A scratch buffer for the balanced decode calls (no initial contents
    needed; one buffer serves any number of calls issued in order on one
    stream)."""
    return torch.empty(pa_decode_scratch_bytes(), dtype=torch.uint8,
                       device=device if device is not None else torch.cuda.current_device())


def _scratch(scratch):
    return _dev(scratch, "scratch", torch.uint8, 1), scratch.numel()


def pa_decode_balanced(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                       scratch, stream=None):
    """Single-pass paged decode with every workgroup given an equal share of
    the batch; out [num_seqs][H_q][d]. scratch: decode_scratch()."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    if query.shape[0] != num_seqs or tuple(out.shape) != tuple(query.shape):
        raise ValueError("query/out must be [num_seqs][num_q_heads][head_dim]")
    hq = query.shape[1]
    sp, sn = _scratch(scratch)
    check(lib().pa_decode_balanced(_dev(out, "out"), _dev(query, "query"),
                                   _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                                   block_tables.data_ptr(), context_lens.data_ptr(), num_seqs, hq,
                                   hkv, d, bs, block_tables.shape[1], num_blocks, float(scale),
                                   _dtype(key_cache, "pools"), _dtype(out, "out"), sp, sn,
                                   _stream(stream)))


def pa_decode_balanced_static(out, query, key_cache, value_cache, block_tables, context_lens,
                              scale, stream=None):
    """pa_decode_balanced with the library's static scratch: allocates
    nothing (calls that overlap in time on one GPU race)."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    if query.shape[0] != num_seqs or tuple(out.shape) != tuple(query.shape):
        raise ValueError("query/out must be [num_seqs][num_q_heads][head_dim]")
    hq = query.shape[1]
    check(lib().pa_decode_balanced_static(
        _dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), block_tables.data_ptr(), context_lens.data_ptr(),
        num_seqs, hq, hkv, d, bs, block_tables.shape[1], num_blocks, float(scale),
        _dtype(key_cache, "pools"), _dtype(out, "out"), _stream(stream)))


def pa_decode_partitioned_balanced(part_out, part_max, part_sum, query, key_cache, value_cache,
                                   block_tables, context_lens, scale, partition_size, scratch,
                                   stream=None):
    """pa_decode_partitioned with every workgroup given an equal share of the
    batch (same records). scratch: decode_scratch()."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    hq = query.shape[1]
    if query.shape[0] != num_seqs:
        raise ValueError("query must be [num_seqs][num_q_heads][head_dim]")
    if part_out.dim() != 4 or tuple(part_out.shape[:2]) != (num_seqs, hq) or part_out.shape[3] != d:
        raise ValueError("part_out must be float32 [num_seqs][num_q_heads][max_parts][head_dim]")
    max_parts = part_out.shape[2]
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (num_seqs, hq, max_parts):
            raise ValueError(f"{nm} must be float32 [num_seqs][num_q_heads][max_parts]")
    sp, sn = _scratch(scratch)
    check(lib().pa_decode_partitioned_balanced(
        _dev(part_out, "part_out", torch.float32), _dev(part_max, "part_max", torch.float32),
        _dev(part_sum, "part_sum", torch.float32), _dev(query, "query"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), block_tables.data_ptr(),
        context_lens.data_ptr(), num_seqs, hq, hkv, d, bs, block_tables.shape[1], num_blocks,
        float(scale), int(partition_size), max_parts, _dtype(key_cache, "pools"), sp, sn,
        _stream(stream)))


def pa_decode_fp8(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                  k_scale, v_scale, stream=None):
    """pa_decode over FP8 pools (codes times k_scale / v_scale); bfloat16 query."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs", fp8=True)
    if query.shape[0] != num_seqs or tuple(out.shape) != tuple(query.shape):
        raise ValueError("query/out must be [num_seqs][num_q_heads][head_dim]")
    hq = query.shape[1]
    check(lib().pa_decode_fp8(_dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
                              _dev(value_cache, "value_cache"), block_tables.data_ptr(),
                              context_lens.data_ptr(), num_seqs, hq, hkv, d, bs,
                              block_tables.shape[1], num_blocks, float(scale), float(k_scale),
                              float(v_scale), _dtype(out, "out"), _stream(stream)))


def pa_decode_partitioned_fp8(part_out, part_max, part_sum, query, key_cache, value_cache,
                              block_tables, context_lens, scale, k_scale, v_scale,
                              partition_size, stream=None, plan=None, plan_epoch=0):
    """pa_decode_partitioned over FP8 pools; pa_reduce merges the partitions.
    With plan (a decode_plan_buffer()) and plan_epoch: the planned call."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs", fp8=True)
    hq = query.shape[1]
    if query.shape[0] != num_seqs:
        raise ValueError("query must be [num_seqs][num_q_heads][head_dim]")
    if part_out.dim() != 4 or tuple(part_out.shape[:2]) != (num_seqs, hq) or part_out.shape[3] != d:
        raise ValueError("part_out must be float32 [num_seqs][num_q_heads][max_parts][head_dim]")
    max_parts = part_out.shape[2]
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (num_seqs, hq, max_parts):
            raise ValueError(f"{nm} must be float32 [num_seqs][num_q_heads][max_parts]")
    args = [_dev(part_out, "part_out", torch.float32), _dev(part_max, "part_max", torch.float32),
            _dev(part_sum, "part_sum", torch.float32), _dev(query, "query"),
            _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            block_tables.data_ptr(), context_lens.data_ptr(), num_seqs, hq, hkv, d, bs,
            block_tables.shape[1], num_blocks, float(scale), float(k_scale), float(v_scale),
            int(partition_size), max_parts]
    if plan is None:
        check(lib().pa_decode_partitioned_fp8(*args, _stream(stream)))
    else:
        check(lib().pa_decode_partitioned_fp8_planned(*args, _plan(plan),
                                                      int(plan_epoch) & 0xffffffff,
                                                      _stream(stream)))


def pa_reduce(out, part_out, part_max, part_sum, context_lens, partition_size, stream=None):
    """Log-sum-exp merge of partitions into out [num_seqs][H_q][d]."""
    if part_out.dim() != 4:
        raise ValueError("part_out must be [num_seqs][num_q_heads][max_parts][head_dim]")
    num_seqs, hq, max_parts, d = part_out.shape
    if tuple(out.shape) != (num_seqs, hq, d):
        raise ValueError("out must be [num_seqs][num_q_heads][head_dim]")
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (num_seqs, hq, max_parts):
            raise ValueError(f"{nm} must be [num_seqs][num_q_heads][max_parts]")
    if context_lens.dim() != 1 or context_lens.shape[0] != num_seqs:
        raise ValueError("context_lens must be int32 [num_seqs]")
    check(lib().pa_reduce(_dev(out, "out"), _dev(part_out, "part_out", torch.float32),
                          _dev(part_max, "part_max", torch.float32),
                          _dev(part_sum, "part_sum", torch.float32),
                          _dev(context_lens, "context_lens", torch.int32), num_seqs, hq, d,
                          int(partition_size), max_parts, _dtype(out, "out"), _stream(stream)))


def pa_decode_step(out, query, key, value, key_cache, value_cache, block_tables, context_lens,
                   scale, partition_size=0, part_out=None, part_max=None, part_sum=None,
                   plan=None, plan_epoch=0, stream=None):
    """One decode step: key/value [num_seqs][H_KV][d] (the step's token, at
    position context_lens[s] - 1) join the pools at the slot the block table
    gives, then out [num_seqs][H_q][d] = attention over the whole context.
    partition_size > 0 splits the context (part_* as for
    pa_decode_partitioned); 0 is a single pass. plan: None or a
    decode_plan_buffer(), with plan_epoch naming this step's lengths and
    tables (a launch whose epoch matches reads the plan, otherwise writes it)."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    hq = query.shape[1]
    if query.shape[0] != num_seqs or tuple(out.shape) != tuple(query.shape):
        raise ValueError("query/out must be [num_seqs][num_q_heads][head_dim]")
    for t, nm in ((key, "key"), (value, "value")):
        if tuple(t.shape) != (num_seqs, hkv, d) or t.dtype != key_cache.dtype:
            raise ValueError(f"{nm} must be [num_seqs][num_kv_heads][head_dim] in the pools' dtype")
    if partition_size:
        if part_out is None or part_max is None or part_sum is None:
            raise ValueError("a split step needs part_out, part_max and part_sum")
        if part_out.dim() != 4 or tuple(part_out.shape[:2]) != (num_seqs, hq) or \
                part_out.shape[3] != d:
            raise ValueError("part_out must be float32 [num_seqs][num_q_heads][max_parts][head_dim]")
        max_parts = part_out.shape[2]
        for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
            if tuple(t.shape) != (num_seqs, hq, max_parts):
                raise ValueError(f"{nm} must be float32 [num_seqs][num_q_heads][max_parts]")
        parts = [_dev(part_out, "part_out", torch.float32),
                 _dev(part_max, "part_max", torch.float32),
                 _dev(part_sum, "part_sum", torch.float32)]
    else:
        max_parts = 1
        parts = [None, None, None]
    check(lib().pa_decode_step(
        _dev(out, "out"), *parts, _dev(query, "query"), _dev(key, "key"), _dev(value, "value"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), block_tables.data_ptr(),
        context_lens.data_ptr(), num_seqs, hq, hkv, d, bs, block_tables.shape[1], num_blocks,
        float(scale), int(partition_size), max_parts, _dtype(key_cache, "pools"),
        _dtype(out, "out"), _plan(plan), int(plan_epoch) & 0xffffffff, _stream(stream)))


def _plan(plan):
    return None if plan is None else _dev(plan, "plan", torch.uint8, 1)


def pa_decode_plan_bytes():
    """Bytes of a decode plan buffer on the current device."""
    return int(lib().pa_decode_plan_bytes())


def decode_plan_buffer(device=None):
    """A plan buffer for the planned decode calls (any initial contents)."""
    return torch.empty(pa_decode_plan_bytes(), dtype=torch.uint8,
                       device=device if device is not None else torch.cuda.current_device())


def pa_decode_partitioned_planned(part_out, part_max, part_sum, query, key_cache, value_cache,
                                  block_tables, context_lens, scale, partition_size, plan,
                                  plan_epoch, stream=None):
    """pa_decode_partitioned with a plan buffer and epoch (see pa_decode_step)."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_seqs")
    hq = query.shape[1]
    if query.shape[0] != num_seqs:
        raise ValueError("query must be [num_seqs][num_q_heads][head_dim]")
    if part_out.dim() != 4 or tuple(part_out.shape[:2]) != (num_seqs, hq) or part_out.shape[3] != d:
        raise ValueError("part_out must be float32 [num_seqs][num_q_heads][max_parts][head_dim]")
    max_parts = part_out.shape[2]
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (num_seqs, hq, max_parts):
            raise ValueError(f"{nm} must be float32 [num_seqs][num_q_heads][max_parts]")
    check(lib().pa_decode_partitioned_planned(
        _dev(part_out, "part_out", torch.float32), _dev(part_max, "part_max", torch.float32),
        _dev(part_sum, "part_sum", torch.float32), _dev(query, "query"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), block_tables.data_ptr(),
        context_lens.data_ptr(), num_seqs, hq, hkv, d, bs, block_tables.shape[1], num_blocks,
        float(scale), int(partition_size), max_parts, _dtype(key_cache, "pools"), _plan(plan),
        int(plan_epoch) & 0xffffffff, _stream(stream)))


def pa_prefill_chunk(out, query, key_cache, value_cache, block_tables, query_start_loc,
                     context_lens, max_query_len, scale, stream=None):
    """Causal chunked prefill; query/out packed [num_q_tokens][H_q][d]."""
    num_blocks, hkv, bs, d, num_seqs = _attn_common(query, key_cache, value_cache, block_tables,
                                                    context_lens, "num_q_tokens")
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must match query's shape")
    if query_start_loc.dim() != 1 or query_start_loc.shape[0] != num_seqs + 1:
        raise ValueError("query_start_loc must be int32 [num_seqs + 1]")
    hq = query.shape[1]
    check(lib().pa_prefill_chunk(
        _dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), block_tables.data_ptr(),
        _dev(query_start_loc, "query_start_loc", torch.int32), context_lens.data_ptr(),
        num_seqs, query.shape[0], int(max_query_len), hq, hkv, d, bs, block_tables.shape[1],
        num_blocks, float(scale), _dtype(key_cache, "pools"), _dtype(out, "out"),
        _stream(stream)))


class BlockAllocator:
    """Owner of a host ``pa_alloc``: on-demand blocks from a FIFO free queue."""

    def __init__(self, num_blocks, block_size, initial_order=None):
        h = ctypes.c_void_p()
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("initial_order must have num_blocks entries")
        check(lib().pa_alloc_create(num_blocks, block_size,
                                    None if order is None else order.ctypes.data,
                                    ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            lib().pa_alloc_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, seq_id, num_tokens):
        """Grow a sequence; returns the new tokens' slots (int64 numpy array)."""
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        check(lib().pa_alloc_append(self._h, int(seq_id), int(num_tokens),
                                    slots.ctypes.data if num_tokens > 0 else None))
        return slots

    def free(self, seq_id):
        check(lib().pa_alloc_free(self._h, int(seq_id)))

    def num_free(self):
        return int(lib().pa_alloc_num_free(self._h))

    def seq_len(self, seq_id):
        return int(lib().pa_alloc_seq_len(self._h, int(seq_id)))

    def fork(self, parent_id, child_id):
        """Start child_id as a sharer of all of parent_id's blocks (copy on write)."""
        check(lib().pa_alloc_fork(self._h, int(parent_id), int(child_id)))

    def take_copies(self):
        """Queued copy-on-write pairs as int32 [n][2] (source, destination);
        the queue is emptied."""
        n = int(lib().pa_alloc_take_copies(self._h, None, 0))
        if n < 0:
            raise PAError(-1, "pa_alloc_take_copies failed")
        pairs = np.empty((n, 2), dtype=np.int32)
        if n:
            got = int(lib().pa_alloc_take_copies(self._h, pairs.ctypes.data, n))
            if got != n:
                raise PAError(-1, "pa_alloc_take_copies: queue changed")
        return pairs

    def block_refs(self, block):
        return int(lib().pa_alloc_block_refs(self._h, int(block)))

    def set_host_pool(self, num_host_blocks, initial_order=None):
        """Give the allocator a host pool with its own FIFO free queue."""
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.shape != (num_host_blocks,):
                raise ValueError("initial_order must have num_host_blocks entries")
        check(lib().pa_alloc_set_host_pool(self._h, int(num_host_blocks),
                                           None if order is None else order.ctypes.data))

    def num_free_host(self):
        return int(lib().pa_alloc_num_free_host(self._h))

    def is_swapped(self, seq_id):
        return int(lib().pa_alloc_is_swapped(self._h, int(seq_id)))

    def _swap(self, fn, seq_id):
        n_blocks = -(-max(self.seq_len(seq_id), 0) // self.block_size)
        pairs = np.empty((max(n_blocks, 1), 2), dtype=np.int32)
        n = ctypes.c_int32(0)
        check(fn(self._h, int(seq_id), n_blocks, pairs.ctypes.data, ctypes.byref(n)))
        return pairs[:n.value]

    def swap_out(self, seq_id):
        """Move a sequence to host blocks; returns int32 [n][2] (device block,
        host block) moves for pa_swap_blocks."""
        return self._swap(lib().pa_alloc_swap_out, seq_id)

    def swap_in(self, seq_id):
        """Bring a sequence back to device blocks; returns int32 [n][2] (host
        block, device block) moves for pa_swap_blocks."""
        return self._swap(lib().pa_alloc_swap_in, seq_id)

    def step(self, seq_ids, num_tokens, max_blocks, slots_out=None, table_out=None,
             lens_out=None):
        """Append num_tokens[i] tokens to seq_ids[i] and export the table rows
        in one native call; returns (slots, table, lens). Output arrays may be
        passed in (e.g. pinned host buffers) to avoid allocations."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        nt = np.ascontiguousarray(num_tokens, dtype=np.int32)
        n = len(ids)
        total = int(nt.sum()) if n else 0
        slots = slots_out if slots_out is not None else np.empty(total, dtype=np.int64)
        table = table_out if table_out is not None else np.empty((n, max_blocks), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        check(lib().pa_alloc_step(self._h, ids.ctypes.data if n else None,
                                  nt.ctypes.data if n else None, n,
                                  slots.ctypes.data if total else None, int(max_blocks),
                                  table.ctypes.data if n else None,
                                  lens.ctypes.data if n else None))
        return slots[:total], table[:n], lens[:n]

    def block_table(self, seq_ids, max_blocks):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        table = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        check(lib().pa_alloc_block_table(self._h, ids.ctypes.data if len(ids) else None, len(ids),
                                         max_blocks, table.ctypes.data, lens.ctypes.data))
        return table, lens
