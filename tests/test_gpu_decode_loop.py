"""The iteration-level decode loop (DecodeLoop) against an oracle loop run on
the same request stream: the oracle's allocator model, cache write and
decode, step by step. Requests of random prompt and generation lengths join
as slots free up; every step's new K/V and queries are seeded BF16 values.
Checked every step: the allocator's slots (bit-exact, through the device
pools) and the attention outputs of sampled running slots in every layer
(2e-2 max abs). Eager launches, and HIP graph replay of the device part
(the graph is captured once and replayed with each step's batch)."""

import numpy as np
import pytest
import torch

from oracle import allocator as model
from oracle import attention as oracle
from paged_kv_cache_454_amd import inputs
from paged_kv_cache_454_amd.decode_loop import DecodeLoop
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("use_graph", [False, True], ids=["eager", "graph"])
def test_decode_loop_matches_oracle(use_graph):
    print(f"[loop] graph={use_graph}", flush=True)
    slots, layers, hq, hkv, d, bs, P, maxc = 32, 2, 24, 4, 256, 16, 256, 2048
    nb = slots * (maxc // bs)
    rng = np.random.default_rng(17 + use_graph)
    loop = DecodeLoop(slots=slots, num_blocks=nb, block_size=bs, layers=layers, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, partition_size=P, max_context=maxc,
                      device=G.DEV, use_graph=use_graph)
    m = model.BlockAllocatorModel(nb, bs)
    pools = [(np.zeros((nb, hkv, bs, d), np.float32), np.zeros((nb, hkv, bs, d), np.float32))
             for _ in range(layers)]
    bf = lambda shape: inputs.round_to_bf16(rng.standard_normal(shape).astype(np.float32))
    dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(G.DEV)
    next_id = 0
    slot_seq = {}

    def admit(slot):
        nonlocal next_id
        n = int(rng.integers(1, 1900))
        g = int(rng.integers(2, 7))
        pk, pv = bf((layers, n, hkv, d)), bf((layers, n, hkv, d))
        got = loop.admit(slot, next_id, n, g, dev(pk), dev(pv))
        want = m.append(next_id, n)
        assert list(got) == want
        for l in range(layers):
            pools[l] = oracle.cache_write(pools[l][0], pools[l][1], pk[l], pv[l], np.array(want), bs)
        slot_seq[slot] = next_id
        next_id += 1

    for s in range(slots):
        if rng.random() < 0.8:
            admit(s)
    checked = 0
    for step in range(12):
        q, nk, nv = bf((layers, slots, hq, d)), bf((layers, slots, hkv, d)), bf((layers, slots, hkv, d))
        loop.query.copy_(dev(q))
        loop.new_k.copy_(dev(nk))
        loop.new_v.copy_(dev(nv))
        act = loop.step()
        # oracle: the same appends in slot order, the same writes, then decode
        rows = [s for s, _ in act]
        new_slots = []
        for s, sid in act:
            assert slot_seq[s] == sid
            new_slots += m.append(sid, 1)
        for l in range(layers):
            pools[l] = oracle.cache_write(pools[l][0], pools[l][1], nk[l][rows], nv[l][rows],
                                          np.array(new_slots), bs)
        sample = rows if step in (0, 7) else list(rng.choice(rows, size=min(4, len(rows)),
                                                                replace=False))
        table, lens = m.block_table([slot_seq[s] for s in sample], loop.max_blocks)
        out = G.host(loop.out)
        for l in range(layers):
            want = oracle.decode(q[l][sample], pools[l][0], pools[l][1], np.array(table),
                                 np.array(lens), bs, loop.scale)
            assert G.max_err(out[l][sample], want) <= G.BF16_TOL, (step, l)
            checked += len(sample)
        for s, sid in loop.finish_done():
            m.free(sid)
            del slot_seq[s]
            if rng.random() < 0.9:
                admit(s)
        assert loop.alloc.num_free() == m.num_free()
    # the device pools equal the oracle's bit for bit
    for l in range(layers):
        assert np.array_equal(G.bits(loop.pools[l][0]), G.bits(pools[l][0], torch.bfloat16))
        assert np.array_equal(G.bits(loop.pools[l][1]), G.bits(pools[l][1], torch.bfloat16))
    assert checked > 100
    loop.close()
