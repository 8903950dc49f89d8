"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes the oracle modules it checks as arguments (so a
deliberately broken copy can be passed in by the mutation tests) and raises
AssertionError when the oracle disagrees with:

* numbers the pages print (golden fixtures under tests/golden/, each cited),
* closed forms and invariants the pages state,
* a pure-Python brute force that walks the physical blocks in logical order
  (forward mapping block j, offset o -> position j*bs + o; no NumPy),
* a library attention routine (torch scaled_dot_product_attention in float64
  on the CPU, with its own grouped-query head mapping), and
* mathematical special cases (one token, constant values, zero query, ...).
"""

import json
import math
import os
import random

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- helpers

def _tiny_case(rng, num_seqs, max_len, hq, hkv, d, bs, pool_extra=2, zero_len=False):
    """Random tiny paged case built without the oracle: dense per-sequence K/V,
    scattered into a pool by walking blocks forward. Returns the pool, tables,
    lens and the dense tensors for brute force / library checks."""
    lens = [rng.randint(1, max_len) for _ in range(num_seqs)]
    if zero_len:
        lens[0] = 0
    nblk = [(t + bs - 1) // bs for t in lens]
    num_blocks = sum(nblk) + pool_extra
    ids = list(range(num_blocks))
    rng.shuffle(ids)
    kc = np.full((num_blocks, hkv, bs, d), np.nan)
    vc = np.full((num_blocks, hkv, bs, d), np.nan)
    tables = np.full((num_seqs, max(1, max(nblk))), -1, dtype=np.int64)
    dense_k, dense_v = [], []
    nxt = 0
    for s in range(num_seqs):
        K = [[[rng.gauss(0, 1) for _ in range(d)] for _ in range(hkv)] for _ in range(lens[s])]
        V = [[[rng.gauss(0, 1) for _ in range(d)] for _ in range(hkv)] for _ in range(lens[s])]
        dense_k.append(K)
        dense_v.append(V)
        for j in range(nblk[s]):
            phys = ids[nxt]
            nxt += 1
            tables[s, j] = phys
            for o in range(bs):
                pos = j * bs + o
                if pos < lens[s]:
                    kc[phys, :, o, :] = K[pos]
                    vc[phys, :, o, :] = V[pos]
    q = [[[rng.gauss(0, 1) for _ in range(d)] for _ in range(hq)] for _ in range(num_seqs)]
    return dict(kc=kc, vc=vc, tables=tables, lens=lens, q=np.array(q), K=dense_k, V=dense_v,
                bs=bs, hq=hq, hkv=hkv, d=d)


def _brute_attend(q, keys, vals, scale):
    logits = [scale * sum(a * b for a, b in zip(q, k)) for k in keys]
    top = max(logits)
    e = [math.exp(z - top) for z in logits]
    tot = sum(e)
    d = len(vals[0])
    return [sum(e[t] * vals[t][c] for t in range(len(vals))) / tot for c in range(d)]


def _brute_decode(case, scale):
    """Pure-Python paged decode: visit table entries in order, each block's
    offsets in order, and stop at the context length."""
    bs, hq, hkv = case["bs"], case["hq"], case["hkv"]
    out = []
    for s, T in enumerate(case["lens"]):
        keys = [[] for _ in range(hkv)]
        vals = [[] for _ in range(hkv)]
        j = 0
        while j * bs < T:
            phys = int(case["tables"][s, j])
            for o in range(bs):
                if j * bs + o >= T:
                    break
                for g in range(hkv):
                    keys[g].append(case["kc"][phys, g, o].tolist())
                    vals[g].append(case["vc"][phys, g, o].tolist())
            j += 1
        row = []
        for h in range(hq):
            g = h * hkv // hq
            if T == 0:
                row.append([0.0] * case["d"])
            else:
                row.append(_brute_attend(case["q"][s, h].tolist(), keys[g], vals[g], scale))
        out.append(row)
    return np.array(out)


def _sdpa(q, K, V, scale, causal=False):
    """torch SDPA, float64, CPU, grouped-query heads by the library's own rule.
    q: [Hq][Lq][d], K/V: [Hkv][Lk][d]."""
    qt = torch.tensor(q, dtype=torch.float64)[None]
    kt = torch.tensor(K, dtype=torch.float64)[None]
    vt = torch.tensor(V, dtype=torch.float64)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=causal,
                                       enable_gqa=True)
    return o[0].numpy()


# ------------------------------------------------------------- accounting

def pin_kv_size(acct):
    g = _golden("kv_cache_size.json")
    m = acct.kv_cache_bytes(**g["inputs"])
    assert round(m / 1e9, 2) == g["printed_approx"], m
    assert m / 2 ** 30 == g["printed_half_gigabyte_binary"], m
    # Linear in every factor (doubling any one doubles M), zero with no tokens.
    base = g["inputs"]
    for key in base:
        twice = dict(base)
        twice[key] = 2 * base[key]
        assert acct.kv_cache_bytes(**twice) == 2 * m
    assert acct.kv_cache_bytes(16, 4, 256, 0, 2) == 0


def pin_worked_example_accounting(acct):
    g = _golden("worked_example.json")
    r, u, w = acct.contiguous_reservation(g["requests_tokens"], g["max_len"])
    c = g["contiguous"]
    assert (r, u, w) == (c["reserved"], c["used"], c["unused"])
    assert round(100 * w / r) == c["waste_percent_printed"]
    r2, u2, w2 = acct.paged_reservation(g["requests_tokens"], g["block_size"])
    p = g["paged"]
    assert (r2, u2, w2) == (p["reserved"], p["used"], p["unused"])
    assert [acct.blocks_needed(t, g["block_size"]) * g["block_size"]
            for t in g["requests_tokens"]] == p["per_request_slots"]
    assert r - r2 == p["freed_vs_contiguous"]


# -------------------------------------------------------------- allocator

def pin_worked_example_allocator(alloc):
    g = _golden("worked_example.json")
    bs = g["block_size"]
    pool = g["contiguous"]["reserved"] // bs
    a = alloc.BlockAllocatorModel(pool, bs)
    # Tokens arrive one at a time; blocks are handed out only when needed.
    for step in range(max(g["requests_tokens"])):
        for sid, n in enumerate(g["requests_tokens"]):
            if step < n:
                a.append(sid, 1)
    held = [len(a.tables[s]) * bs for s in range(3)]
    assert held == g["paged"]["per_request_slots"]
    assert sum(held) == g["paged"]["reserved"]
    assert a.num_free() * bs == g["paged"]["freed_vs_contiguous"]


def _check_allocator_state(a, bs):
    seen = set()
    for sid, table in a.tables.items():
        n = a.lengths[sid]
        assert len(table) == (n + bs - 1) // bs          # on demand: no spare blocks
        assert len(table) * bs - n < bs                   # only the last block has holes
        for b in table:
            assert b not in seen
            seen.add(b)
    assert not seen & set(a.free_blocks)
    assert len(seen) + a.num_free() == a.num_blocks


def pin_allocator_invariants(alloc):
    rng = random.Random(7)
    bs, nb = 4, 40
    order = list(range(nb))
    rng.shuffle(order)
    a = alloc.BlockAllocatorModel(nb, bs, initial_order=order)
    # The first blocks handed out follow the given free order.
    s0 = a.append(100, 9)
    assert a.tables[100] == order[:3]
    assert s0 == [order[p // bs] * bs + p % bs for p in range(9)]
    a.free(100)
    assert list(a.free_blocks)[-3:] == order[:3]          # released to the back (FIFO)
    live = {}
    for step in range(400):
        op = rng.random()
        if op < 0.6 or not live:
            sid = rng.randrange(12)
            n = rng.randint(1, 9)
            before = (list(a.free_blocks), {k: list(v) for k, v in a.tables.items()},
                      dict(a.lengths))
            try:
                slots = a.append(sid, n)
            except alloc.OutOfBlocks:
                # atomic: nothing changed
                assert before == (list(a.free_blocks),
                                  {k: list(v) for k, v in a.tables.items()}, dict(a.lengths))
                continue
            start = a.lengths[sid] - n
            table = a.tables[sid]
            for i, slot in enumerate(slots):
                pos = start + i
                assert slot // bs == table[pos // bs] and slot % bs == pos % bs
            live[sid] = True
        else:
            sid = rng.choice(sorted(live))
            freed = list(a.tables[sid])
            head = list(a.free_blocks)
            a.free(sid)
            del live[sid]
            assert list(a.free_blocks) == head + freed
        _check_allocator_state(a, bs)
    # exhausting the pool raises and leaves the state intact
    b = alloc.BlockAllocatorModel(3, 4)
    b.append(1, 12)
    try:
        b.append(2, 1)
        raise AssertionError("expected OutOfBlocks")
    except alloc.OutOfBlocks:
        pass
    assert b.num_free() == 0 and 2 not in b.tables


def pin_block_table_rows(alloc):
    """The exported block-table rows against fixed ids: a partly filled last
    block, padding with -1 past the table ("vLLM Architecture, Memory and
    Benchmarks Deep Dive", s.2: a block table maps each sequence's logical
    blocks to physical ones; unused entries hold no block), and the lengths
    are the tokens held, not whole blocks."""
    order = [5, 2, 7, 0, 3, 6, 1, 4]
    a = alloc.BlockAllocatorModel(8, 4, initial_order=order)
    a.append(10, 6)          # blocks 5, 2: the second holds 2 of 4 slots
    a.append(11, 1)          # block 7, 1 of 4 slots
    a.append(12, 8)          # blocks 0, 3: both full
    rows, lens = a.block_table([11, 10, 12], 4)
    assert rows == [[7, -1, -1, -1], [5, 2, -1, -1], [0, 3, -1, -1]], rows
    assert lens == [1, 6, 8], lens
    a.append(10, 3)          # fills block 2 and takes block 6 for the ninth token
    rows, lens = a.block_table([10], 3)
    assert rows == [[5, 2, 6]] and lens == [9], (rows, lens)
    try:
        a.block_table([10], 2)   # three blocks do not fit a two-entry row
    except ValueError:
        pass
    else:
        raise AssertionError("a row shorter than the table must be refused")


def _cow_state_ok(a):
    held = {}
    for table in a.tables.values():
        for b in table:
            held[b] = held.get(b, 0) + 1
    assert held == a.refs                                 # counts = tables holding each block
    assert not set(held) & set(a.free_blocks)
    assert len(held) + a.num_free() == a.num_blocks


def pin_cow_contents(alloc):
    """Copy-on-write judged by what each sequence reads back: a token marker
    is written at every appended slot of a simulated pool, recorded copies
    duplicate whole blocks before the writes, and every live sequence must
    then read, through its table, exactly its own history (its ancestors'
    tokens up to the fork, then its own), whatever its siblings wrote."""
    rng = random.Random(11)
    for bs, nb in ((4, 48), (1, 30), (5, 40)):
        a = alloc.BlockAllocatorModel(nb, bs)
        pool = [[None] * bs for _ in range(nb)]
        history = {}
        mark = 0
        for _ in range(600):
            op = rng.random()
            live = sorted(history)
            if op < 0.5 or not live:
                sid = rng.choice(live) if live and rng.random() < 0.8 else rng.randrange(1000)
                n = rng.randint(0, 2 * bs + 1)
                try:
                    slots = a.append(sid, n)
                except alloc.OutOfBlocks:
                    assert a.take_copies() == []
                    continue
                for src, dst in a.take_copies():
                    pool[dst] = list(pool[src])
                for slot in slots:
                    mark += 1
                    pool[slot // bs][slot % bs] = mark
                    history.setdefault(sid, []).append(mark)
                history.setdefault(sid, [])
            elif op < 0.75:
                parent = rng.choice(live)
                child = 1000 + rng.randrange(1000)
                if child in history:
                    continue
                a.fork(parent, child)
                history[child] = list(history[parent])
            else:
                sid = rng.choice(live)
                a.free(sid)
                del history[sid]
            for sid, hist in history.items():
                t = a.tables[sid]
                assert a.lengths[sid] == len(hist)
                assert [pool[t[p // bs]][p % bs] for p in range(len(hist))] == hist, sid
            _cow_state_ok(a)


def pin_cow_counts(alloc):
    """A prompt whose last block is partly filled, forked k times: nothing is
    copied at fork time; when each of the k+1 holders appends a token, the
    first k copy the shared block and the last writes in place. With a full
    last block no append copies anything."""
    for k in (1, 3, 7):
        a = alloc.BlockAllocatorModel(64, 4)
        a.append(0, 10)                                   # blocks 0, 1, 2 (2 slots free)
        for c in range(1, k + 1):
            a.fork(0, c)
        assert a.take_copies() == [] and a.num_free() == 61
        for c in range(k + 1):
            a.append(c, 1)
        cp = a.take_copies()
        assert len(cp) == k and all(src == 2 for src, _ in cp)
        assert [dst for _, dst in cp] == list(range(3, 3 + k))  # from the front, in order
        assert a.num_free() == 61 - k
        b = alloc.BlockAllocatorModel(64, 4)
        b.append(0, 8)                                    # two full blocks
        for c in range(1, k + 1):
            b.fork(0, c)
        for c in range(k + 1):
            b.append(c, 3)
        assert b.take_copies() == [] and b.num_free() == 62 - (k + 1)
        # the shared blocks survive until their last holder is released
        for c in range(k + 1):
            before = b.num_free()
            b.free(c)
            assert b.num_free() - before == 1 + (2 if c == k else 0)


def _swap_state_ok(a):
    _cow_state_ok(a)
    host_held = [b for t in a.host_tables.values() for b in t]
    assert len(host_held) == len(set(host_held))          # a host block has one owner
    assert not set(host_held) & set(a.host_free)
    assert len(host_held) + a.num_free_host() == a.num_host_blocks
    assert not set(a.host_tables) & set(a.tables)


def pin_swap_contents(alloc):
    """Swapping judged by what each sequence reads back: the copy-on-write
    simulation above with a host pool beside the device pool. Swap-out pairs
    move device blocks to host blocks and swap-in pairs move them back (after
    the step's copy-on-write copies); every resident sequence reads its own
    history through its table from the device pool, every swapped-out one
    through its host blocks from the host pool."""
    rng = random.Random(23)
    for bs, nb, nh in ((4, 40, 24), (1, 24, 30), (3, 36, 12)):
        a = alloc.BlockAllocatorModel(nb, bs, num_host_blocks=nh)
        dev = [[None] * bs for _ in range(nb)]
        host = [[None] * bs for _ in range(nh)]
        history, swapped = {}, set()
        mark = 0
        for _ in range(700):
            op = rng.random()
            live = sorted(s for s in history if s not in swapped)
            out = sorted(swapped)
            if op < 0.4 or not history:
                sid = rng.choice(live) if live and rng.random() < 0.8 else rng.randrange(1000)
                if sid in history and sid in swapped:
                    continue
                n = rng.randint(0, 2 * bs + 1)
                try:
                    slots = a.append(sid, n)
                except alloc.OutOfBlocks:
                    assert a.take_copies() == []
                    continue
                for src, dst in a.take_copies():
                    dev[dst] = list(dev[src])
                for slot in slots:
                    mark += 1
                    dev[slot // bs][slot % bs] = mark
                    history.setdefault(sid, []).append(mark)
                history.setdefault(sid, [])
            elif op < 0.55 and live:
                parent = rng.choice(live)
                child = 1000 + rng.randrange(1000)
                if child in history:
                    continue
                a.fork(parent, child)
                history[child] = list(history[parent])
            elif op < 0.7 and live:
                sid = rng.choice(live)
                free_before = (a.num_free(), a.num_free_host())
                table = list(a.tables[sid])
                try:
                    pairs = a.swap_out(sid)
                except alloc.OutOfBlocks:
                    assert (a.num_free(), a.num_free_host()) == free_before
                    continue
                assert [d for d, _ in pairs] == table        # every block, logical order
                for d, h in pairs:
                    host[h] = list(dev[d])
                swapped.add(sid)
            elif op < 0.85 and out:
                sid = rng.choice(out)
                free_before = (a.num_free(), a.num_free_host())
                try:
                    pairs = a.swap_in(sid)
                except alloc.OutOfBlocks:
                    assert (a.num_free(), a.num_free_host()) == free_before
                    continue
                for h, d in pairs:
                    dev[d] = list(host[h])
                swapped.discard(sid)
            else:
                sid = rng.choice(sorted(history))
                a.free(sid)
                del history[sid]
                swapped.discard(sid)
            for sid, hist in history.items():
                assert a.lengths[sid] == len(hist)
                if sid in swapped:
                    t = a.host_tables[sid]
                    assert [host[t[p // bs]][p % bs] for p in range(len(hist))] == hist, sid
                else:
                    t = a.tables[sid]
                    assert [dev[t[p // bs]][p % bs] for p in range(len(hist))] == hist, sid
            _swap_state_ok(a)


def pin_swap_counts(alloc):
    """Swap order and atomicity on a small pool, every block id fixed by the
    first-in first-out queues: swap-out takes host blocks from the front in
    logical order and frees the device blocks no one else holds to the back;
    swap-in does the reverse; a side without room raises and changes nothing;
    a swapped-out sequence cannot grow or be forked and keeps its length."""
    a = alloc.BlockAllocatorModel(16, 4, num_host_blocks=6)
    a.append(0, 10)                                      # device 0, 1, 2
    a.append(1, 5)                                       # device 3, 4
    assert a.swap_out(0) == [(0, 0), (1, 1), (2, 2)]
    assert list(a.free_blocks) == list(range(5, 16)) + [0, 1, 2]
    assert a.num_free_host() == 3 and a.lengths[0] == 10
    assert a.swap_out(1) == [(3, 3), (4, 4)]
    assert list(a.free_blocks)[-2:] == [3, 4] and list(a.host_free) == [5]
    for bad in (lambda: a.append(0, 1), lambda: a.fork(0, 9), lambda: a.block_table([0], 4)):
        try:
            bad()
        except (ValueError, KeyError):
            pass
        else:
            raise AssertionError("a swapped-out sequence was used")
    a.append(2, 6)                                       # device 5, 6 (6 half full)
    a.fork(2, 3)
    snap = (list(a.free_blocks), list(a.host_free), dict(a.refs), dict(a.host_tables))
    try:
        a.swap_out(3)                                    # needs 2 host blocks, 1 free
    except alloc.OutOfBlocks:
        pass
    else:
        raise AssertionError("swap-out beyond the host pool")
    assert snap == (list(a.free_blocks), list(a.host_free), dict(a.refs), dict(a.host_tables))
    a.free(1)                                            # host 3, 4 back at the end
    assert list(a.host_free) == [5, 3, 4]
    assert a.swap_out(3) == [(5, 5), (6, 3)]             # shared blocks stay for 2
    assert a.refs == {5: 1, 6: 1} and 5 not in a.free_blocks
    assert a.swap_in(0) == [(0, 7), (1, 8), (2, 9)]
    assert list(a.host_free) == [4, 0, 1, 2] and a.tables[0] == [7, 8, 9]
    assert a.append(0, 2) == [9 * 4 + 2, 9 * 4 + 3]        # grows in its new last block
    b = alloc.BlockAllocatorModel(4, 2, num_host_blocks=8)
    b.append(0, 6)                                       # device 0, 1, 2
    b.swap_out(0)
    b.append(1, 4)                                       # device 3, 0
    snap = (list(b.free_blocks), list(b.host_free), dict(b.refs))
    try:
        b.swap_in(0)                                     # needs 3, 2 free
    except alloc.OutOfBlocks:
        pass
    else:
        raise AssertionError("swap-in beyond the device pool")
    assert snap == (list(b.free_blocks), list(b.host_free), dict(b.refs))
    b.free(1)
    assert b.swap_in(0) == [(0, 1), (1, 2), (2, 3)]
    assert b.block_table([0], 3) == ([[1, 2, 3]], [6])
    b.free(0)
    assert list(b.host_free) == [3, 4, 5, 6, 7, 0, 1, 2] and b.num_free() == 4


# -------------------------------------------------------------- attention

def pin_cache_write(attn):
    rng = np.random.default_rng(3)
    nb, hkv, bs, d = 6, 2, 4, 8
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    kc[4] = np.nan
    slots = np.array([0, 7, 22, -1, 13], dtype=np.int64)
    key = rng.standard_normal((5, hkv, d)).astype(np.float32)
    val = rng.standard_normal((5, hkv, d)).astype(np.float32)
    k2, v2 = attn.cache_write(kc, vc, key, val, slots, bs)
    flat_k = k2.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
    flat_v = v2.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
    touched = set()
    for i, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        assert np.array_equal(flat_k[s], key[i]) and np.array_equal(flat_v[s], val[i])
        touched.add(s)
    ok = np.transpose(kc, (0, 2, 1, 3)).reshape(nb * bs, hkv, d)
    for s in range(nb * bs):
        if s not in touched:
            assert np.array_equal(flat_k[s].view(np.uint32), ok[s].view(np.uint32))
    assert np.isnan(k2[4]).all()


def pin_decode_bruteforce(attn):
    rng = random.Random(11)
    for trial in range(12):
        hkv = rng.choice([1, 2, 3])
        hq = hkv * rng.choice([1, 2, 3])
        bs = rng.choice([1, 2, 4])
        d = rng.choice([2, 3, 5, 8])
        case = _tiny_case(rng, rng.randint(1, 3), 9, hq, hkv, d, bs, zero_len=(trial == 5))
        scale = rng.uniform(0.2, 1.5)
        want = _brute_decode(case, scale)
        got = attn.decode(case["q"], case["kc"], case["vc"], case["tables"], case["lens"], bs,
                          scale)
        assert np.abs(got - want).max() <= 1e-12, (trial, np.abs(got - want).max())


def pin_decode_vs_library(attn):
    """One block per sequence at a random physical ID reduces paged decode to
    textbook attention, which torch computes with its own GQA rule."""
    rng = np.random.default_rng(5)
    for hq, hkv, d, T in [(4, 1, 16, 7), (6, 2, 8, 12), (24, 4, 32, 16), (3, 3, 4, 1)]:
        bs = 16
        nb = 5
        phys = int(rng.integers(nb))
        K = rng.standard_normal((hkv, T, d))
        V = rng.standard_normal((hkv, T, d))
        q = rng.standard_normal((hq, d))
        kc = np.full((nb, hkv, bs, d), np.nan)
        vc = np.full((nb, hkv, bs, d), np.nan)
        kc[phys, :, :T] = K
        vc[phys, :, :T] = V
        scale = 1 / math.sqrt(d)
        got = attn.decode(q[None], kc, vc, np.array([[phys]]), [T], bs, scale)[0]
        want = _sdpa(q[:, None, :], K, V, scale)[:, 0, :]
        assert np.abs(got - want).max() < 1e-12


def pin_decode_special_cases(attn):
    rng = np.random.default_rng(9)
    hq, hkv, d, bs = 6, 2, 8, 4
    nb = 8
    kc = rng.standard_normal((nb, hkv, bs, d))
    vc = rng.standard_normal((nb, hkv, bs, d))
    tables = np.array([[3, 1, 6], [0, 5, 2]])
    q = rng.standard_normal((2, hq, d))
    # one token: the output is that token's V exactly
    out = attn.decode(q, kc, vc, tables, [1, 1], bs, 0.7)
    for s in range(2):
        for h in range(hq):
            assert np.array_equal(out[s, h], vc[tables[s, 0], h // 3, 0])
    # zero query: uniform weights -> mean of the V rows in context
    out = attn.decode(np.zeros_like(q), kc, vc, tables, [10, 7], bs, 0.7)
    for s, T in enumerate([10, 7]):
        rows = [vc[tables[s, t // bs], :, t % bs] for t in range(T)]
        assert np.abs(out[s, 0] - np.mean(rows, axis=0)[0]).max() < 1e-12
        assert np.abs(out[s, 5] - np.mean(rows, axis=0)[1]).max() < 1e-12
    # identical keys: uniform weights again, whatever q is
    kc2 = np.broadcast_to(kc[0:1, :, 0:1, :], kc.shape).copy()
    out = attn.decode(q, kc2, vc, tables, [9, 12], bs, 0.7)
    rows = [vc[tables[1, t // bs], 1, t % bs] for t in range(12)]
    assert np.abs(out[1, 4] - np.mean(rows, axis=0)).max() < 1e-12
    # constant V: output equals the constant
    vc3 = np.full_like(vc, 2.5)
    out = attn.decode(q, kc, vc3, tables, [11, 5], bs, 0.7)
    assert np.abs(out - 2.5).max() < 1e-12
    # a huge scale turns softmax into a hard argmax over the keys
    out = attn.decode(q, kc, vc, tables, [12, 12], bs, 1e4)
    for s in range(2):
        for h in range(hq):
            g = h // 3
            keys = [kc[tables[s, t // bs], g, t % bs] for t in range(12)]
            best = int(np.argmax([k @ q[s, h] for k in keys]))
            assert np.abs(out[s, h] - vc[tables[s, best // bs], g, best % bs]).max() < 1e-9


def pin_permutation_invariance(attn):
    rng = random.Random(21)
    case = _tiny_case(rng, 3, 11, 4, 2, 5, 2, pool_extra=5)
    base = attn.decode(case["q"], case["kc"], case["vc"], case["tables"], case["lens"], 2, 0.5)
    nb = case["kc"].shape[0]
    perm = list(range(nb))
    rng.shuffle(perm)
    kc = np.empty_like(case["kc"])
    vc = np.empty_like(case["vc"])
    for old, new in enumerate(perm):
        kc[new] = case["kc"][old]
        vc[new] = case["vc"][old]
    tables = np.where(case["tables"] >= 0, np.array(perm)[case["tables"]], -1)
    again = attn.decode(case["q"], kc, vc, tables, case["lens"], 2, 0.5)
    assert np.array_equal(base, again)


def pin_partitions(attn):
    rng = random.Random(4)
    case = _tiny_case(rng, 3, 23, 6, 3, 4, 2)
    scale = 0.9
    full = attn.decode(case["q"], case["kc"], case["vc"], case["tables"], case["lens"], 2, scale)
    for P in [2, 4, 6, 8, 64]:
        o, lse, n = attn.decode_partitions(case["q"], case["kc"], case["vc"], case["tables"],
                                           case["lens"], 2, scale, P)
        assert list(n) == [(t + P - 1) // P for t in case["lens"]]
        merged = attn.merge_partitions(o, lse, n)
        assert np.abs(merged - full).max() < 1e-12
        # each partition's lse is log(sum(exp(logits))) over its own tokens
        for s, T in enumerate(case["lens"]):
            for h in range(6):
                g = h // 2
                for p in range(n[s]):
                    logits = [scale * sum(a * b for a, b in
                                          zip(case["q"][s, h].tolist(), case["K"][s][t][g]))
                              for t in range(p * P, min(T, (p + 1) * P))]
                    assert abs(lse[s, h, p] - math.log(sum(math.exp(z) for z in logits))) < 1e-12
        if P == 64:   # one partition: o is the decode output itself
            assert np.abs(o[:, :, 0, :] - full).max() < 1e-12
    # very different partition scales: merge must not underflow
    q = np.array(case["q"]) * 60.0
    full = attn.decode(q, case["kc"], case["vc"], case["tables"], case["lens"], 2, scale)
    o, lse, n = attn.decode_partitions(q, case["kc"], case["vc"], case["tables"], case["lens"],
                                       2, scale, 4)
    assert np.isfinite(full).all()
    assert np.abs(attn.merge_partitions(o, lse, n) - full).max() < 1e-9


def pin_prefill(attn):
    rng = random.Random(8)
    # no earlier context: causal textbook attention over the chunk (library)
    case = _tiny_case(rng, 2, 10, 4, 2, 8, 4)
    lens = case["lens"]
    qsl = [0, lens[0], lens[0] + lens[1]]
    nprng = np.random.default_rng(1)
    q = nprng.standard_normal((qsl[-1], 4, 8))
    out = attn.prefill(q, case["kc"], case["vc"], case["tables"], qsl, lens, 4, 0.35)
    for s in range(2):
        K = np.array(case["K"][s]).transpose(1, 0, 2)
        V = np.array(case["V"][s]).transpose(1, 0, 2)
        qs = q[qsl[s]:qsl[s + 1]].transpose(1, 0, 2)
        want = _sdpa(qs, K, V, 0.35, causal=True).transpose(1, 0, 2)
        assert np.abs(out[qsl[s]:qsl[s + 1]] - want).max() < 1e-12
    # with earlier context: query j of a chunk of n sees the first T-n+j+1
    # tokens, i.e. it equals decode over that prefix (brute force)
    case = _tiny_case(rng, 3, 14, 6, 2, 4, 4)
    chunks = [min(t, c) for t, c in zip(case["lens"], [3, 1, 5])]
    qsl = np.concatenate([[0], np.cumsum(chunks)]).tolist()
    q = nprng.standard_normal((qsl[-1], 6, 4))
    out = attn.prefill(q, case["kc"], case["vc"], case["tables"], qsl, case["lens"], 4, 0.6)
    for s, T in enumerate(case["lens"]):
        n = chunks[s]
        for j in range(n):
            sub = dict(case)
            sub["lens"] = [T - n + j + 1]
            sub["tables"] = case["tables"][s:s + 1]
            sub["q"] = q[qsl[s] + j][None]
            want = _brute_decode(sub, 0.6)[0]
            assert np.abs(out[qsl[s] + j] - want).max() < 1e-12


def pin_swap_blocks(attn):
    """Block moves between two pools of different sizes against element-wise
    loops: each destination block equals its source block in all heads and
    rows, the source pools and all other destination blocks are untouched,
    and pairs out of either pool's range change nothing."""
    rng = np.random.default_rng(6)
    sk, sv = rng.standard_normal((5, 2, 3, 4)), rng.standard_normal((5, 2, 3, 4))
    dk, dv = rng.standard_normal((8, 2, 3, 4)), rng.standard_normal((8, 2, 3, 4))
    sk0, sv0 = sk.copy(), sv.copy()
    pairs = [(4, 0), (0, 7), (2, 3), (5, 1), (1, 8), (-1, 2)]
    k2, v2 = attn.swap_blocks(sk, sv, dk, dv, pairs)
    src_of = {0: 4, 7: 0, 3: 2}
    for b in range(8):
        for h in range(2):
            for r in range(3):
                for c in range(4):
                    if b in src_of:
                        assert k2[b, h, r, c] == sk[src_of[b], h, r, c]
                        assert v2[b, h, r, c] == sv[src_of[b], h, r, c]
                    else:
                        assert k2[b, h, r, c] == dk[b, h, r, c]
                        assert v2[b, h, r, c] == dv[b, h, r, c]
    assert np.array_equal(sk, sk0) and np.array_equal(sv, sv0)


def pin_copy_blocks(attn):
    """Block copies against element-wise loops over a pool of distinct
    values: every destination block equals its source in all heads and rows,
    other blocks are untouched, and out-of-range pairs change nothing."""
    rng = np.random.default_rng(5)
    kc = rng.standard_normal((9, 2, 3, 4))
    vc = rng.standard_normal((9, 2, 3, 4))
    pairs = [(1, 4), (7, 0), (2, 8), (-1, 3), (5, 9)]
    k2, v2 = attn.copy_blocks(kc, vc, pairs)
    for b in range(9):
        src = {4: 1, 0: 7, 8: 2}.get(b, b)
        for h in range(2):
            for r in range(3):
                for c in range(4):
                    assert k2[b, h, r, c] == kc[src, h, r, c]
                    assert v2[b, h, r, c] == vc[src, h, r, c]


# -------------------------------------------------------------- fp8

def pin_fp8_codes(fp8):
    """E4M3FN codes from the format's definition, independent of the
    encoder's search: known values, every code back to itself, torch's
    float8_e4m3fn conversion on in-range values, ties to even, saturation."""
    import torch
    known = [(0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-2.0, 0xC0), (0.5, 0x30), (448.0, 0x7E),
             (-448.0, 0xFE), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07),
             (1.75, 0x3E), (240.0, 0x77), (0.015625 * 1.875, 0x0F)]   # pairs: 0.0 == -0.0
    for x, c in known:
        assert int(fp8.encode_e4m3([x])[0]) == c, (x, c)
        assert fp8.decode_e4m3([c])[0] == x or (x == 0 and fp8.decode_e4m3([c])[0] == 0)
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = fp8.decode_e4m3(codes)
    assert list(fp8.encode_e4m3(vals)) == codes                 # every code maps back
    assert np.isnan(fp8.decode_e4m3([0x7F, 0xFF])).all()
    assert int(fp8.encode_e4m3([np.nan])[0]) == 0x7F
    pos = np.sort(vals[vals > 0])
    assert pos[-1] == 448.0 and pos[0] == 2.0 ** -9 and len(pos) == 126
    # torch's conversion (round to nearest even) on finite in-range values
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.1, 3.0, 100.0)])
    x = x[np.abs(x) < 448.0].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode_e4m3(x.astype(np.float64)), ref)
    # ties between neighbouring codes go to the even code
    for lo in (0x38, 0x39, 0x01, 0x10, 0x7C):
        a, b = fp8.decode_e4m3([lo, lo + 1])
        want = lo if lo % 2 == 0 else lo + 1
        assert int(fp8.encode_e4m3([(a + b) / 2])[0]) == want
    # saturation (a stated choice): beyond 448 stays at the largest finite code
    assert list(fp8.encode_e4m3([460.0, 500.0, 1e9, -1e9])) == [0x7E, 0x7E, 0x7E, 0xFE]


def pin_fp8_cache(fp8):
    """The quantising cache write stores torch's codes of the fp32 quotients
    at the written slots (and nothing else); decode over a cache whose values
    are all exactly representable equals the unquantised decode."""
    import torch
    rng = np.random.default_rng(29)
    nb, hkv, bs, d = 6, 2, 4, 8
    kc = np.zeros((nb, hkv, bs, d), np.uint8)
    vc = np.zeros((nb, hkv, d, bs), np.uint8)       # value blocks: token index fastest
    key = rng.standard_normal((5, hkv, d)).astype(np.float32)
    val = rng.standard_normal((5, hkv, d)).astype(np.float32)
    slots = np.array([3, 9, -1, 22, 0])
    ks, vs = 0.05, 0.02
    k2, v2 = fp8.cache_write(kc, vc, key, val, slots, bs, ks, vs)
    for i, sl in enumerate(slots.tolist()):
        if sl < 0:
            continue
        qk = (torch.from_numpy(key[i]) / torch.tensor(ks, dtype=torch.float32))
        qv = (torch.from_numpy(val[i]) / torch.tensor(vs, dtype=torch.float32))
        assert np.array_equal(k2[sl // bs, :, sl % bs], qk.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        assert np.array_equal(v2[sl // bs, :, :, sl % bs], qv.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert int((k2 != 0).sum()) <= 4 * hkv * d and np.array_equal(k2[1], kc[1])  # block 1 unwritten
    assert int((v2 != 0).sum()) <= 4 * hkv * d and np.array_equal(v2[1], vc[1])
    # values on the E4M3 grid times the scale survive exactly: fp8 decode = plain decode
    codes_k = rng.integers(0, 0x7E, size=(nb, hkv, bs, d)).astype(np.uint8)
    codes_v = rng.integers(0, 0x7E, size=(nb, hkv, d, bs)).astype(np.uint8)
    q = rng.standard_normal((2, 4, d))
    tables = np.array([[0, 3, -1], [5, 1, 2]])
    lens = np.array([7, 12])
    got = fp8.decode(q, codes_k, codes_v, tables, lens, bs, 0.3, 0.25, 2.0)
    want = attention_decode_ref(q, fp8.decode_e4m3(codes_k) * 0.25, fp8.decode_e4m3(codes_v) * 2.0,
                                tables, lens, bs, 0.3, v_tokens_last=True)
    assert np.abs(got - want).max() < 1e-12


def pin_fp8_partitions(fp8):
    """Per-partition FP8 records against a brute-force loop: every code is
    dequantised on its own through torch's float8_e4m3fn (a library
    conversion), keys read from the row layout [nb][H][bs][d] and values from
    the transposed block layout [nb][H][d][bs]; unequal key and value scales,
    so a swap of the two changes the logits and the outputs."""
    import torch
    rng = np.random.default_rng(37)
    nb, hkv, hq, bs, d, P = 10, 2, 6, 4, 6, 4   # d != bs: the value layout matters
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes_k = rng.choice(finite, size=(nb, hkv, bs, d))
    codes_v = rng.choice(finite, size=(nb, hkv, d, bs))
    q = rng.standard_normal((3, hq, d)) * 0.05
    tables = np.array([[4, 9, 1], [7, -1, -1], [0, 5, 8]])
    lens = np.array([9, 3, 12])
    scale, ks, vs = 0.4, 0.03, 1.7

    def deq(c, sc):
        t = torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn)
        return float(t.to(torch.float64)[0]) * float(np.float32(sc))

    o, lse, n = fp8.decode_partitions(q, codes_k, codes_v, tables, lens, bs, scale, ks, vs, P)
    assert list(n) == [3, 1, 3]
    for s in range(3):
        T = int(lens[s])
        for h in range(hq):
            g = h // (hq // hkv)
            for p in range(-(-T // P)):
                toks = range(p * P, min(T, (p + 1) * P))
                z = []
                for t in toks:
                    blk, off = int(tables[s][t // bs]), t % bs
                    z.append(scale * sum(float(q[s, h, c]) * deq(codes_k[blk, g, off, c], ks)
                                         for c in range(d)))
                top = max(z)
                tot = sum(math.exp(v - top) for v in z)
                assert abs(lse[s, h, p] - (top + math.log(tot))) < 1e-12
                for c in range(d):
                    acc = 0.0
                    for t, v in zip(toks, z):
                        blk, off = int(tables[s][t // bs]), t % bs
                        acc += math.exp(v - top) * deq(codes_v[blk, g, c, off], vs)
                    assert abs(o[s, h, p, c] - acc / tot) < 1e-12 * max(1.0, abs(acc / tot))


def attention_decode_ref(q, kc, vc, tables, lens, bs, scale, v_tokens_last=False):
    """Brute-force decode (loops), for the fp8 pin; v_tokens_last: the value
    pool is [nb][H][d][bs]."""
    out = np.zeros(q.shape)
    hq, hkv = q.shape[1], kc.shape[1]
    for s in range(q.shape[0]):
        for h in range(hq):
            g = h // (hq // hkv)
            z = []
            for t in range(int(lens[s])):
                blk = int(tables[s][t // bs])
                z.append(scale * float(np.dot(q[s, h], kc[blk, g, t % bs])))
            zmax = max(z)
            w = [np.exp(v - zmax) for v in z]
            acc = np.zeros(q.shape[2])
            for t, wt in enumerate(w):
                blk = int(tables[s][t // bs])
                acc += wt * (vc[blk, g, :, t % bs] if v_tokens_last else vc[blk, g, t % bs])
            out[s, h] = acc / sum(w)
    return out


ATTENTION_PINS = [pin_cache_write, pin_decode_bruteforce, pin_decode_vs_library,
                  pin_decode_special_cases, pin_permutation_invariance, pin_partitions,
                  pin_prefill, pin_copy_blocks, pin_swap_blocks]
ACCOUNTING_PINS = [pin_kv_size, pin_worked_example_accounting]
FP8_PINS = [pin_fp8_codes, pin_fp8_cache, pin_fp8_partitions]
ALLOCATOR_PINS = [pin_worked_example_allocator, pin_allocator_invariants, pin_cow_contents,
                  pin_cow_counts, pin_swap_contents, pin_swap_counts, pin_block_table_rows]
