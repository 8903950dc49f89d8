"""Seeded synthetic workloads for the paged decode and prefill path.

This module is the one piece shared by the product's tests/bench and the CPU
oracle. It holds none of the method's arithmetic: it only draws random
numbers, rounds them to BF16 where a workload is BF16 (torch's
round-to-nearest-even conversion), scatters each sequence's blocks over a
physical pool in a seeded order, and marks the slots that hold no token.

Workloads (all draws come from one ``numpy.random.default_rng(seed)`` per
case, in the order written in :func:`decode_case` / :func:`prefill_case`):

* ``tiny``    fp32, 3 sequences of 3, 5 and 2 tokens (after this step's write),
              4 query heads / 1 KV head, head_dim 64, block_size 4, a pool of 8
              physical blocks handed out in a seeded random order, scale 1/8.
              These are the request sizes of the worked example on "High-
              Throughput LLM Inference & Training" (Fig. 1 / Fig. 2).
* ``uniform`` bf16, 8 sequences x 2048 tokens, 24/4 heads, head_dim 256,
              block_size 16, pool exactly the blocks needed, seeded order.
              One layer; timed over 8 independent pool sets in turn (8 x 64
              MiB), so that repeated steps cannot be served from the caches.
* ``mixed``   bf16, 64 sequences, lengths floor(exp(U(ln 16, ln 8192))),
              24/4/256, block_size 16, pool 1.5x the blocks needed with the
              sequences' blocks scattered at random; unused blocks are garbage.
              Run as 16 independent layers back to back.
* ``long``    bf16, 4 sequences of 8192/16384/32768/32768 tokens, 24/4/256,
              block_size 32, 512-token partitions; K and V are N(0,1) plus a
              per-(KV head, channel) bias drawn N(0, 3^2). One layer;
              timed over 3 independent pool sets in turn (3 x 352 MiB).
* ``prefill`` bf16, 16 sequences with an existing context drawn uniformly
              from 0..6000 tokens plus a 512-token query chunk, 24/4/256,
              block_size 16.

Head dimensions, head counts and shapes follow "vLLM Architecture, Memory and
Benchmarks Deep Dive", section 1 (4 KV heads, head dimension 256, BF16) and
section 2 (blocks of 16 or 32 tokens); chunked prefill's 512-token chunk is
from section 4 of the same page.
"""

import math
from dataclasses import dataclass, field

import numpy as np

PRESETS = {
    "tiny": dict(kind="decode", dtype="f32", context_lens=[3, 5, 2], num_q_heads=4,
                 num_kv_heads=1, head_dim=64, block_size=4, num_blocks=8, scale=1.0 / 8.0),
    "uniform": dict(kind="decode", dtype="bf16", context_lens=[2048] * 8, num_q_heads=24,
                    num_kv_heads=4, head_dim=256, block_size=16, pool_factor=1.0, pool_sets=8),
    "mixed": dict(kind="decode", dtype="bf16", num_seqs=64, min_len=16, max_len=8192,
                  num_q_heads=24, num_kv_heads=4, head_dim=256, block_size=16,
                  pool_factor=1.5, layers=16),
    "long": dict(kind="decode", dtype="bf16", context_lens=[8192, 16384, 32768, 32768],
                 num_q_heads=24, num_kv_heads=4, head_dim=256, block_size=32,
                 pool_factor=1.0, kv_bias_scale=3.0, partition_size=512, pool_sets=3),
    "prefill": dict(kind="prefill", dtype="bf16", num_seqs=16, max_existing=6000, chunk=512,
                    num_q_heads=24, num_kv_heads=4, head_dim=256, block_size=16),
}

NAN_F32 = np.float32(np.nan)


def round_to_bf16(x):
    """float32 array -> float32 array of the nearest BF16 values (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def log_uniform_lengths(rng, n, lo, hi):
    """floor(exp(U(ln lo, ln hi))), clamped to [lo, hi]."""
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int64)


def _ceil_div(a, b):
    return -(-int(a) // int(b))


@dataclass
class PagedCase:
    """Host arrays of one paged workload. Floating arrays are float32 holding
    values exactly representable in ``dtype`` (NaN marks garbage)."""
    name: str
    seed: int
    dtype: str                 # "f32" | "bf16": storage type of q, K, V
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray   # int32 [num_seqs], tokens held after this step's write
    block_tables: np.ndarray   # int32 [num_seqs][max_blocks_per_seq], pad -1
    slot_mapping: np.ndarray   # int64 [num_new_tokens]
    key: np.ndarray            # float32 [num_new_tokens][num_kv_heads][head_dim]
    value: np.ndarray
    key_cache: np.ndarray      # float32 [num_blocks][num_kv_heads][block_size][head_dim]
    value_cache: np.ndarray    # (pool before this step's write)
    query: np.ndarray          # decode: [num_seqs][H_q][d]; prefill: [num_q_tokens][H_q][d]
    query_start_loc: np.ndarray = None   # prefill only: int32 [num_seqs + 1]
    partition_size: int = 512
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self):
        return int(self.block_tables.shape[1])


def _scatter_tables(rng, blocks_per_seq, num_blocks):
    """Each sequence takes the next run of a seeded permutation of the pool."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    maxb = max(1, max(blocks_per_seq) if len(blocks_per_seq) else 1)
    tables = np.full((len(blocks_per_seq), maxb), -1, dtype=np.int32)
    off = 0
    for s, nb in enumerate(blocks_per_seq):
        tables[s, :nb] = perm[off:off + nb]
        off += nb
    if off > num_blocks:
        raise ValueError("pool too small for the requested contexts")
    return tables


def _layout(rng, lens, block_size, pool_factor, num_blocks):
    """Block tables (seeded scatter) and the slot of each sequence's newest
    token, position T_s - 1 (the token this decode step writes)."""
    bps = [_ceil_div(t, block_size) for t in lens]
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * sum(bps))))
    tables = _scatter_tables(rng, bps, num_blocks)
    slots = np.full(len(lens), -1, dtype=np.int64)
    for s in range(len(lens)):
        if lens[s] > 0:
            pos = int(lens[s]) - 1
            slots[s] = int(tables[s, pos // block_size]) * block_size + pos % block_size
    return tables, slots, num_blocks


def decode_layout(context_lens, block_size, pool_factor=1.0, num_blocks=None, seed=0):
    """Only the integer layout of :func:`decode_case` (same seed -> same
    tables and slots): (block_tables, slot_mapping, num_blocks)."""
    rng = np.random.default_rng(seed)
    return _layout(rng, np.asarray(context_lens, dtype=np.int64), block_size, pool_factor,
                   num_blocks)


def _mark_garbage(pool, tables, filled, block_size, garbage):
    """Slots that hold no token (unused blocks, tails, this step's targets)
    become NaN ('nan') or keep their random draw ('random')."""
    if garbage == "random":
        return
    if garbage != "nan":
        raise ValueError(garbage)
    used = np.zeros(pool.shape[0], dtype=bool)
    for s in range(tables.shape[0]):
        n_tok = int(filled[s])
        nb = int((tables[s] >= 0).sum())
        for j in range(nb):
            phys = int(tables[s, j])
            used[phys] = True
            valid = min(block_size, max(0, n_tok - j * block_size))
            pool[phys, :, valid:, :] = NAN_F32
    pool[~used] = NAN_F32


def _draw_pools(rng, num_blocks, hkv, bs, d, bias_scale):
    kc = rng.standard_normal((num_blocks, hkv, bs, d), dtype=np.float32)
    vc = rng.standard_normal((num_blocks, hkv, bs, d), dtype=np.float32)
    if bias_scale:
        bk = (bias_scale * rng.standard_normal((hkv, d))).astype(np.float32)
        bv = (bias_scale * rng.standard_normal((hkv, d))).astype(np.float32)
        kc += bk[None, :, None, :]
        vc += bv[None, :, None, :]
    else:
        bk = bv = None
    return kc, vc, bk, bv


def decode_case(context_lens, num_q_heads, num_kv_heads, head_dim, block_size, dtype="bf16",
                num_blocks=None, pool_factor=1.0, scale=None, seed=0, garbage="nan",
                kv_bias_scale=0.0, partition_size=512, name="custom", max_blocks_per_seq=None):
    """One decode step: each sequence gets one new token (its last position),
    written through ``slot_mapping`` and then used as the query's own key.

    Draw order: block permutation, K pool, V pool, [K bias, V bias], new K,
    new V, query.
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    tables, slots, num_blocks = _layout(rng, lens, block_size, pool_factor, num_blocks)
    if max_blocks_per_seq is not None and max_blocks_per_seq > tables.shape[1]:
        pad = np.full((tables.shape[0], max_blocks_per_seq - tables.shape[1]), -1, np.int32)
        tables = np.concatenate([tables, pad], axis=1)
    kc, vc, bk, bv = _draw_pools(rng, num_blocks, num_kv_heads, block_size, head_dim,
                                 kv_bias_scale)
    B = len(lens)
    new_k = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32)
    new_v = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32)
    if bk is not None:
        new_k += bk[None]
        new_v += bv[None]
    q = rng.standard_normal((B, num_q_heads, head_dim), dtype=np.float32)
    if dtype == "bf16":
        kc, vc, new_k, new_v, q = (round_to_bf16(a) for a in (kc, vc, new_k, new_v, q))
    elif dtype != "f32":
        raise ValueError(dtype)
    # Before the write each sequence holds all but its newest token.
    _mark_garbage(kc, tables, lens - 1, block_size, garbage)
    _mark_garbage(vc, tables, lens - 1, block_size, garbage)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PagedCase(name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                     num_blocks=num_blocks, scale=float(scale),
                     context_lens=lens.astype(np.int32), block_tables=tables,
                     slot_mapping=slots, key=new_k, value=new_v, key_cache=kc,
                     value_cache=vc, query=q, partition_size=partition_size,
                     extra={"kv_bias_k": bk, "kv_bias_v": bv})


def prefill_case(existing_lens, chunk_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                 dtype="bf16", pool_factor=1.0, scale=None, seed=0, garbage="nan",
                 name="custom"):
    """One chunked-prefill step: sequence s holds existing_lens[s] cached tokens
    and appends chunk_lens[s] new ones, whose K/V are written through
    ``slot_mapping`` and whose queries attend causally.

    Draw order: block permutation, K pool, V pool, new K, new V, query.
    """
    rng = np.random.default_rng(seed)
    ex = np.asarray(existing_lens, dtype=np.int64)
    ch = np.asarray(chunk_lens, dtype=np.int64)
    lens = ex + ch
    bps = [_ceil_div(t, block_size) for t in lens]
    num_blocks = max(1, int(math.ceil(pool_factor * sum(bps))))
    tables = _scatter_tables(rng, bps, num_blocks)
    kc, vc, _, _ = _draw_pools(rng, num_blocks, num_kv_heads, block_size, head_dim, 0.0)
    n_new = int(ch.sum())
    new_k = rng.standard_normal((n_new, num_kv_heads, head_dim), dtype=np.float32)
    new_v = rng.standard_normal((n_new, num_kv_heads, head_dim), dtype=np.float32)
    q = rng.standard_normal((n_new, num_q_heads, head_dim), dtype=np.float32)
    if dtype == "bf16":
        kc, vc, new_k, new_v, q = (round_to_bf16(a) for a in (kc, vc, new_k, new_v, q))
    _mark_garbage(kc, tables, ex, block_size, garbage)
    _mark_garbage(vc, tables, ex, block_size, garbage)
    qsl = np.zeros(len(lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ch)
    slots = np.empty(n_new, dtype=np.int64)
    i = 0
    for s in range(len(lens)):
        for pos in range(int(ex[s]), int(lens[s])):
            slots[i] = int(tables[s, pos // block_size]) * block_size + pos % block_size
            i += 1
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PagedCase(name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                     num_blocks=num_blocks, scale=float(scale),
                     context_lens=lens.astype(np.int32), block_tables=tables,
                     slot_mapping=slots, key=new_k, value=new_v, key_cache=kc,
                     value_cache=vc, query=q, query_start_loc=qsl,
                     extra={"existing_lens": ex.astype(np.int32)})


def preset_lengths(name, seed):
    """Context lengths (after this step's write) of a preset, without drawing
    the tensors; uses its own generator stream so it is cheap."""
    p = PRESETS[name]
    if "context_lens" in p:
        return np.asarray(p["context_lens"], dtype=np.int64)
    rng = np.random.default_rng(seed + 1_000_003)
    if name == "mixed":
        return log_uniform_lengths(rng, p["num_seqs"], p["min_len"], p["max_len"])
    if name == "prefill":
        return rng.integers(0, p["max_existing"], size=p["num_seqs"], endpoint=True) + p["chunk"]
    raise KeyError(name)


def preset_case(name, seed=0, garbage="nan"):
    """The named workload at its full size (one layer)."""
    p = PRESETS[name]
    if p["kind"] == "decode":
        lens = preset_lengths(name, seed)
        return decode_case(lens, p["num_q_heads"], p["num_kv_heads"], p["head_dim"],
                           p["block_size"], dtype=p["dtype"], num_blocks=p.get("num_blocks"),
                           pool_factor=p.get("pool_factor", 1.0), scale=p.get("scale"),
                           seed=seed, garbage=garbage,
                           kv_bias_scale=p.get("kv_bias_scale", 0.0),
                           partition_size=p.get("partition_size", 512), name=name)
    lens = preset_lengths(name, seed)
    chunk = p["chunk"]
    ex = lens - chunk
    return prefill_case(ex, [chunk] * len(ex), p["num_q_heads"], p["num_kv_heads"],
                        p["head_dim"], p["block_size"], dtype=p["dtype"], seed=seed,
                        garbage=garbage, name=name)


def device_decode_layers(name, seed, layers, device, dtype=None):
    """Full-size decode workload generated on the device for timing: one
    shared block table / slot mapping (a block table per sequence, as for a
    real model's layers) and, per layer, its own K/V pools, query and new
    K/V drawn N(0,1) (plus the preset's per-head bias) with a seeded torch
    generator, rounded to BF16. Garbage slots keep their random draws."""
    import torch
    p = PRESETS[name]
    lens = preset_lengths(name, seed)
    tables, slots, num_blocks = decode_layout(lens, p["block_size"],
                                              pool_factor=p.get("pool_factor", 1.0),
                                              num_blocks=p.get("num_blocks"), seed=seed)
    dt = dtype or (torch.bfloat16 if p["dtype"] == "bf16" else torch.float32)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    hq, hkv, d, bs = p["num_q_heads"], p["num_kv_heads"], p["head_dim"], p["block_size"]
    B = len(lens)
    bias = p.get("kv_bias_scale", 0.0)
    out = []
    for _ in range(layers):
        layer = {}
        for nm, shape in (("key_cache", (num_blocks, hkv, bs, d)),
                          ("value_cache", (num_blocks, hkv, bs, d)),
                          ("key", (B, hkv, d)), ("value", (B, hkv, d)), ("query", (B, hq, d))):
            x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            layer[nm] = x
        if bias:
            bk = bias * torch.randn((hkv, d), generator=g, device=device)
            bv = bias * torch.randn((hkv, d), generator=g, device=device)
            layer["key_cache"] += bk[None, :, None, :]
            layer["value_cache"] += bv[None, :, None, :]
            layer["key"] += bk[None]
            layer["value"] += bv[None]
        out.append({k: v.to(dt) for k, v in layer.items()})
        del layer
    meta = dict(
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        block_tables=torch.from_numpy(tables).to(device),
        slot_mapping=torch.from_numpy(slots).to(device),
        lens=lens, num_blocks=num_blocks, scale=p.get("scale") or 1.0 / math.sqrt(d),
        partition_size=p.get("partition_size", 512))
    return out, meta


def device_prefill_case(seed, device):
    """The full-size chunked-prefill workload generated on the device for
    timing: the integer layout (seeded scatter of each sequence's blocks, the
    slots of the chunk's positions c_s .. c_s + 511, the packed query offsets)
    on the host, and the K/V pools, the chunk's new K/V and its queries drawn
    N(0,1) on the device with a seeded torch generator and rounded to BF16."""
    import torch
    p = PRESETS["prefill"]
    lens = preset_lengths("prefill", seed)
    chunk, bs = p["chunk"], p["block_size"]
    ex = lens - chunk
    rng = np.random.default_rng(seed)
    bps = [_ceil_div(int(t), bs) for t in lens]
    num_blocks = max(1, sum(bps))
    tables = _scatter_tables(rng, bps, num_blocks)
    n_new = int(chunk * len(lens))
    slots = np.empty(n_new, dtype=np.int64)
    i = 0
    for s in range(len(lens)):
        pos = np.arange(int(ex[s]), int(lens[s]))
        slots[i:i + len(pos)] = tables[s, pos // bs].astype(np.int64) * bs + pos % bs
        i += len(pos)
    qsl = np.arange(len(lens) + 1, dtype=np.int32) * chunk
    hq, hkv, d = p["num_q_heads"], p["num_kv_heads"], p["head_dim"]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = {}
    for nm, shape in (("key_cache", (num_blocks, hkv, bs, d)),
                      ("value_cache", (num_blocks, hkv, bs, d)),
                      ("key", (n_new, hkv, d)), ("value", (n_new, hkv, d)),
                      ("query", (n_new, hq, d))):
        t[nm] = torch.randn(shape, generator=g, device=device,
                            dtype=torch.float32).to(torch.bfloat16)
    t.update(context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
             block_tables=torch.from_numpy(tables).to(device),
             slot_mapping=torch.from_numpy(slots).to(device),
             query_start_loc=torch.from_numpy(qsl).to(device))
    meta = dict(lens=lens, existing=ex, chunk=chunk, num_blocks=num_blocks,
                scale=1.0 / math.sqrt(d), max_query_len=chunk)
    return t, meta
