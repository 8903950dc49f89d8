"""Swapping blocks to pinned host memory on the GPU: pa_swap_blocks against
the oracle's block move between pools (bit-exact, both directions, BF16,
fp32 and FP8 pools), and whole sequences swapped out and back in through
the native allocator while other sequences reuse their device blocks, then
decoded, against the oracle's allocator model, block moves, cache write and
decode on the same seeded inputs. Pools bit-exact; attention within the BF16
tolerance (2e-2 max abs, fp32 accumulation)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_454_amd as pa
from oracle import allocator as model
from oracle import attention as oracle
from paged_kv_cache_454_amd import BlockAllocator, PAError, inputs
from paged_kv_cache_454_amd._lib import PA_BF16, PA_EINVAL, lib
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _pairs(rng, ns, nd, n):
    """n pairs with distinct destinations, plus pairs out of either range."""
    src = rng.choice(ns, size=n, replace=n > ns)
    dst = rng.permutation(nd)[:n]
    pairs = [(int(s), int(d)) for s, d in zip(src, dst)]
    pairs += [(-1, int(rng.integers(nd))), (int(rng.integers(ns)), nd), (ns, 0)]
    return np.array(pairs, dtype=np.int32)


def _pinned(a, dtype):
    t = torch.empty(a.shape, dtype=dtype, pin_memory=True)
    t.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(dtype))
    return t


def _pools(rng, nb, hkv, bs, d, dtype):
    if dtype == "fp8":
        k = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
        v = rng.integers(0, 256, size=(nb, hkv, d, bs), dtype=np.uint8)
        return k, v
    k = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    v = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    if dtype == "bf16":
        k, v = inputs.round_to_bf16(k), inputs.round_to_bf16(v)
    return k, v


_TDT = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}


def _host(a, dtype):
    if dtype == "fp8":
        t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
        t.copy_(torch.from_numpy(a))
        return t
    return _pinned(a, _TDT[dtype])


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_TDT[dtype]).to(G.DEV)


def _bits(x, dtype):
    if dtype == "fp8":
        return x.cpu().numpy() if isinstance(x, torch.Tensor) else x
    return G.bits(x, _TDT[dtype])


@pytest.mark.parametrize("dtype,hkv,bs,d,nb,nh", [("bf16", 4, 16, 256, 200, 120),
                                                ("f32", 1, 4, 64, 40, 60),
                                                ("fp8", 4, 16, 256, 90, 70),
                                                ("bf16", 1, 3, 5, 20, 16)])
def test_swap_blocks_bitexact(dtype, hkv, bs, d, nb, nh):
    """Device -> pinned host (swap-out), then pinned host -> another device
    pool (swap-in), each against the oracle's block move; once with the
    pairs themselves in pinned host memory."""
    print(f"[swap] {dtype} hkv={hkv} bs={bs} d={d} nb={nb} nh={nh}", flush=True)
    rng = np.random.default_rng(nb * 7 + nh + d)
    dk, dv = _pools(rng, nb, hkv, bs, d, dtype)
    hk, hv = _pools(rng, nh, hkv, bs, d, dtype)
    ek, ev = _pools(rng, nb, hkv, bs, d, dtype)        # the pools swapped back into
    out_pairs = _pairs(rng, nb, nh, min(nb, nh) // 2)
    in_pairs = _pairs(rng, nh, nb, min(nb, nh) // 3)
    t_dk, t_dv, t_ek, t_ev = _dev(dk, dtype), _dev(dv, dtype), _dev(ek, dtype), _dev(ev, dtype)
    t_hk, t_hv = _host(hk, dtype), _host(hv, dtype)
    pa.pa_swap_blocks(t_dk, t_dv, t_hk, t_hv, torch.from_numpy(out_pairs).to(G.DEV))
    host_pairs = torch.from_numpy(in_pairs).pin_memory()
    pa.pa_swap_blocks(t_hk, t_hv, t_ek, t_ev, host_pairs)
    torch.cuda.synchronize()
    want_hk, want_hv = oracle.swap_blocks(dk, dv, hk, hv, out_pairs)
    want_ek, want_ev = oracle.swap_blocks(want_hk, want_hv, ek, ev, in_pairs)
    assert np.array_equal(_bits(t_hk, dtype), _bits(want_hk, dtype))
    assert np.array_equal(_bits(t_hv, dtype), _bits(want_hv, dtype))
    assert np.array_equal(_bits(t_ek, dtype), _bits(want_ek, dtype))
    assert np.array_equal(_bits(t_ev, dtype), _bits(want_ev, dtype))
    assert np.array_equal(_bits(t_dk, dtype), _bits(dk, dtype))   # sources untouched
    # no pairs: nothing happens
    pa.pa_swap_blocks(t_dk, t_dv, t_hk, t_hv, torch.empty((0, 2), dtype=torch.int32,
                                                          device=G.DEV))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(t_hk, dtype), _bits(want_hk, dtype))


def test_swap_blocks_rejects_unreachable_memory():
    """Pageable host memory is refused before any launch (the device could
    not address it); so is a size that runs past a pinned buffer's end."""
    print("[swap] unreachable memory", flush=True)
    nb, hkv, bs, d = 8, 2, 16, 64
    dk = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=G.DEV)
    dv = torch.zeros_like(dk)
    pageable = np.zeros((nb, hkv, bs, d), dtype=np.uint16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device=G.DEV)
    st = lib().pa_swap_blocks(dk.data_ptr(), dv.data_ptr(), nb, pageable.ctypes.data,
                              pageable.ctypes.data, nb, pairs.data_ptr(), 1, hkv, d, bs, PA_BF16,
                              None)
    assert st == PA_EINVAL, lib().pa_last_error()
    with pytest.raises(ValueError):
        pa.pa_swap_blocks(dk, dv, torch.zeros_like(dk, device="cpu"),
                          torch.zeros_like(dv, device="cpu"), pairs)
    torch.cuda.synchronize()
    assert float(dk.abs().sum()) == 0.0


def test_swapped_sequences_decode():
    """Four sequences are written; two are swapped out to pinned host pools,
    a new sequence grows into the device blocks they freed (overwriting
    them), one swapped sequence comes back into fresh blocks, and every
    resident sequence takes one more token and is decoded. The allocator's
    pairs, both pools on both sides and the outputs match the oracle's."""
    print("[swap] swapped sequences decode", flush=True)
    hq, hkv, d, bs, nb, nh = 24, 4, 256, 16, 40, 32
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(17)
    a = BlockAllocator(nb, bs)
    a.set_host_pool(nh)
    m = model.BlockAllocatorModel(nb, bs, num_host_blocks=nh)
    ok, ov = _pools(rng, nb, hkv, bs, d, "bf16")
    ohk, ohv = _pools(rng, nh, hkv, bs, d, "bf16")
    dk, dv = _dev(ok, "bf16"), _dev(ov, "bf16")
    hk, hv = _pinned(ohk, torch.bfloat16), _pinned(ohv, torch.bfloat16)

    def write(seq_ids, counts):
        nonlocal ok, ov
        slots = []
        for s, n in zip(seq_ids, counts):
            got = list(a.append(s, n))
            assert got == m.append(s, n)
            slots += got
        key = inputs.round_to_bf16(rng.standard_normal((len(slots), hkv, d)).astype(np.float32))
        val = inputs.round_to_bf16(rng.standard_normal((len(slots), hkv, d)).astype(np.float32))
        sm = np.array(slots, dtype=np.int64)
        pa.pa_reshape_and_cache(_dev(key, "bf16"), _dev(val, "bf16"), dk, dv,
                                torch.from_numpy(sm).to(G.DEV))
        ok, ov = oracle.cache_write(ok, ov, key, val, sm, bs)

    def swap(seq, out):
        nonlocal ok, ov, ohk, ohv
        pairs = a.swap_out(seq) if out else a.swap_in(seq)
        want = m.swap_out(seq) if out else m.swap_in(seq)
        assert [tuple(p) for p in pairs.tolist()] == want
        p_dev = torch.from_numpy(pairs).to(G.DEV)
        if out:
            pa.pa_swap_blocks(dk, dv, hk, hv, p_dev)
            ohk, ohv = oracle.swap_blocks(ok, ov, ohk, ohv, pairs)
        else:
            pa.pa_swap_blocks(hk, hv, dk, dv, p_dev)
            ok, ov = oracle.swap_blocks(ohk, ohv, ok, ov, pairs)

    write([0, 1, 2, 3], [40, 100, 17, 64])
    swap(1, True)
    swap(3, True)
    assert a.num_free_host() == nh - 7 - 4
    write([4], [150])                                    # reuses the freed blocks
    swap(1, False)
    resident = [0, 1, 2, 4]
    write(resident, [1, 1, 1, 1])
    maxb = 12
    table, lens = a.block_table(resident, maxb)
    t_m, l_m = m.block_table(resident, maxb)
    assert np.array_equal(table, np.array(t_m, dtype=np.int32)) and list(lens) == l_m
    q = inputs.round_to_bf16(rng.standard_normal((len(resident), hq, d)).astype(np.float32))
    out = torch.empty((len(resident), hq, d), dtype=torch.float32, device=G.DEV)
    pa.pa_decode(out, _dev(q, "bf16"), dk, dv, torch.from_numpy(table).to(G.DEV),
                 torch.from_numpy(lens).to(G.DEV), scale)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits(dk), G.bits(ok, torch.bfloat16))
    assert np.array_equal(G.bits(dv), G.bits(ov, torch.bfloat16))
    assert np.array_equal(G.bits(hk), G.bits(ohk, torch.bfloat16))
    assert np.array_equal(G.bits(hv), G.bits(ohv, torch.bfloat16))
    want = oracle.decode(q, ok, ov, table, lens, bs, scale)
    err = np.abs(out.cpu().numpy() - want).max()
    assert err <= G.BF16_TOL, err
    with pytest.raises(PAError):
        a.append(3, 1)                                   # still on the host
