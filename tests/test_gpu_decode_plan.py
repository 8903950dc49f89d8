"""Decode plan buffers: the first launch of an epoch plans and stores its
deal of units, later launches of the same epoch read it. Either way a launch
deals the same units to the same workgroups as one without a buffer, so its
outputs must be bit for bit the unplanned call's; slots tagged for another
launch (mode, partition size) or holding zeros must be detected and replanned
(again the same bits). The step's outputs are also compared with the oracle
directly."""

import numpy as np
import pytest
import torch

import paged_kv_cache_454_amd as pa
from oracle import attention as oracle
from paged_kv_cache_454_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _parts(case, P):
    S, H, D = case.query.shape
    mp = G.max_parts_for(case, P)
    return (torch.full((S, H, mp, D), float("nan"), device=G.DEV),
            torch.full((S, H, mp), float("nan"), device=G.DEV),
            torch.full((S, H, mp), float("nan"), device=G.DEV))


def _partitioned(t, case, P, plan=None, epoch=0):
    po, pm, ps = _parts(case, P)
    args = (po, pm, ps, t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
            t["context_lens"], case.scale, P)
    if plan is None:
        pa.pa_decode_partitioned(*args)
    else:
        pa.pa_decode_partitioned_planned(*args, plan, epoch)
    return [G.bits(x) for x in (po, pm, ps)]


def _step(case, P, plan=None, epoch=0, t=None):
    t = G.to_dev(case) if t is None else t
    S, H, D = case.query.shape
    out = torch.full((S, H, D), float("nan"), device=G.DEV)
    po, pm, ps = _parts(case, P) if P else (None, None, None)
    pa.pa_decode_step(out, t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"],
                      t["block_tables"], t["context_lens"], case.scale, P, po, pm, ps,
                      plan=plan, plan_epoch=epoch)
    return out, t


def _oracle_step(case):
    kc, vc = oracle.cache_write(case.key_cache, case.value_cache, case.key, case.value,
                                case.slot_mapping, case.block_size)
    return oracle.decode(case.query, kc, vc, case.block_tables, case.context_lens,
                         case.block_size, case.scale)


@pytest.mark.parametrize("preset", ["mixed", "long"])
def test_planned_partitioned_bitexact(preset):
    """First launch with a fresh epoch plans and writes the buffer, the next
    ones read it; all give the unplanned bits."""
    print(f"[plan] partitioned preset={preset}", flush=True)
    case = inputs.preset_case(preset, seed=0)
    t = G.to_dev(case)
    G.write(t)
    P = G.bench_partitions()[0][preset]
    plan = pa.decode_plan_buffer()
    want = _partitioned(t, case, P)
    for _ in range(3):
        for a, b in zip(want, _partitioned(t, case, P, plan, 11)):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("preset", ["mixed", "long"])
def test_planned_step_bitexact_and_oracle(preset):
    print(f"[plan] step preset={preset}", flush=True)
    case = inputs.preset_case(preset, seed=0)
    P = G.bench_partitions()[0][preset]
    base, tb = _step(case, P)
    plan = pa.decode_plan_buffer()
    want = _oracle_step(case)
    for _ in range(2):           # writes the plan, then reads it
        got, t = _step(case, P, plan, 5)
        assert np.array_equal(G.bits(base), G.bits(got))
        assert np.array_equal(G.bits(tb["key_cache"]), G.bits(t["key_cache"]))
        assert np.array_equal(G.bits(tb["value_cache"]), G.bits(t["value_cache"]))
        assert G.max_err(G.host(got), want) <= G.BF16_TOL


EDGE_LENS = ([1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1025, 2049, 4097]
             + [int(x) for x in np.random.default_rng(3).integers(1, 3000, 83)])


@pytest.mark.parametrize("P", [0, 256, 1024])
def test_planned_step_edges(P):
    print(f"[plan] step edges P={P}", flush=True)
    case = inputs.decode_case(EDGE_LENS, 24, 4, 256, 16, dtype="bf16", pool_factor=1.2,
                              seed=P + 1, kv_bias_scale=3.0)
    base, _ = _step(case, P)
    plan = pa.decode_plan_buffer()
    want = _oracle_step(case)
    for _ in range(2):
        got, _ = _step(case, P, plan, 3)
        assert np.array_equal(G.bits(base), G.bits(got))
        assert G.max_err(G.host(got), want) <= G.BF16_TOL


def test_epochs_across_steps():
    """Three steps of one growing batch (every sequence one token longer each
    step, new tables and pools each time) through one plan buffer, a new
    epoch per step: every step matches the oracle and its unplanned bits."""
    plan = pa.decode_plan_buffer()
    lens = np.array(EDGE_LENS)
    for k in range(3):
        case = inputs.decode_case(lens + k, 24, 4, 256, 16, dtype="bf16", pool_factor=1.2,
                                  seed=40 + k)
        base, _ = _step(case, 512)
        for _ in range(2):
            got, _ = _step(case, 512, plan, 100 + k)
            assert np.array_equal(G.bits(base), G.bits(got)), k
        assert G.max_err(G.host(got), _oracle_step(case)) <= G.BF16_TOL


def test_mismatched_plans_are_replanned():
    """Slots written by a step launch, by a launch at another partition
    size, or zeros, under the same epoch: the tags differ, so each launch
    plans for itself (and rewrites the slots)."""
    case = inputs.decode_case(EDGE_LENS, 24, 4, 256, 16, dtype="bf16", pool_factor=1.2, seed=8)
    P = 512
    t = G.to_dev(case)
    G.write(t)
    want = _partitioned(t, case, P)
    plan = pa.decode_plan_buffer()
    _step(case, P, plan, 9)                          # slots tagged for the step
    for a, b in zip(want, _partitioned(t, case, P, plan, 9)):
        assert np.array_equal(a, b)
    _partitioned(t, case, 1024, plan, 9)             # tagged for P = 1024
    for a, b in zip(want, _partitioned(t, case, P, plan, 9)):
        assert np.array_equal(a, b)
    plan.zero_()
    for a, b in zip(want, _partitioned(t, case, P, plan, 0)):
        assert np.array_equal(a, b)
    base, _ = _step(case, P)
    got, _ = _step(case, P, plan, 9)                 # slots tagged for partitioned
    assert np.array_equal(G.bits(base), G.bits(got))


def test_plan_not_applicable_shapes():
    """Where the matrix-core kernel does not take the batch (one unit per
    compute unit; another head size) the buffer is left alone and the planned
    calls give the unplanned results."""
    for lens, d, P in (([2048] * 8, 256, 256), ([300, 40], 128, 256)):
        case = inputs.decode_case(lens, 24, 4, d, 16, dtype="bf16", seed=2)
        t = G.to_dev(case)
        G.write(t)
        buf = torch.zeros(pa.pa_decode_plan_bytes(), dtype=torch.uint8, device=G.DEV)
        want = _partitioned(t, case, P)
        for a, b in zip(want, _partitioned(t, case, P, buf, 1)):
            assert np.array_equal(a, b)
        torch.cuda.synchronize()
        assert int(buf.sum()) == 0


def _fp8_records(t, case, P, ks, vs, plan=None, epoch=0):
    po, pm, ps = _parts(case, P)
    pa.pa_decode_partitioned_fp8(po, pm, ps, t["query"], t["key_cache"], t["value_cache"],
                                 t["block_tables"], t["context_lens"], case.scale, ks, vs, P,
                                 plan=plan, plan_epoch=epoch)
    return [G.bits(x) for x in (po, pm, ps)]


@pytest.mark.parametrize("preset", ["mixed", "long"])
def test_planned_fp8_bitexact(preset):
    """The FP8 kernel with a plan buffer: the same bits as without (the first
    launch of the epoch plans, the next read); slots a BF16 launch wrote under
    the same epoch are replanned, not read."""
    print(f"[plan] fp8 preset={preset}", flush=True)
    from tests.test_gpu_fp8 import _fp8_case, _write
    import bench
    ks, vs = bench.FP8_SCALES[preset]
    case = inputs.preset_case(preset, seed=0)
    t, _, _ = _fp8_case(case, ks, vs)
    _write(t, ks, vs)
    P = G.bench_partitions()[1][preset]
    want = _fp8_records(t, case, P, ks, vs)
    plan = pa.decode_plan_buffer()
    for _ in range(2):
        for a, b in zip(want, _fp8_records(t, case, P, ks, vs, plan, 4)):
            assert np.array_equal(a, b)
    tb = G.to_dev(case)
    G.write(tb)
    _partitioned(tb, case, G.bench_partitions()[0][preset], plan, 4)    # BF16 slots
    for a, b in zip(want, _fp8_records(t, case, P, ks, vs, plan, 4)):
        assert np.array_equal(a, b)


def test_refresh_bit_replans_under_a_fixed_epoch():
    """Bit 31 of the epoch plans afresh and stores the slots under the epoch
    without it: three growing batches through one buffer with the same two
    epoch values every step (refresh on the first call, read on the next)."""
    plan = pa.decode_plan_buffer()
    lens = np.array(EDGE_LENS)
    for k in range(3):
        case = inputs.decode_case(lens + 7 * k, 24, 4, 256, 16, dtype="bf16", pool_factor=1.2,
                                  seed=60 + k)
        base, _ = _step(case, 512)
        got0, _ = _step(case, 512, plan, 5 | 0x80000000)
        got1, _ = _step(case, 512, plan, 5)
        assert np.array_equal(G.bits(base), G.bits(got0)), k
        assert np.array_equal(G.bits(base), G.bits(got1)), k


def test_plan_buffer_across_random_batches():
    """One plan buffer driven through 12 random batches (sizes, lengths,
    partition sizes, step or plain calls), each decoded three times: a fresh
    epoch, the same epoch again, and a refresh under it; every output is
    bit for bit the unplanned call's."""
    rng = np.random.default_rng(23)
    plan = pa.decode_plan_buffer()
    epoch = 1000
    for k in range(12):
        S = int(rng.integers(70, 200))
        lens = [int(x) for x in rng.integers(1, 4000, S)]
        P = int(rng.choice([256, 512, 1024]))
        step = bool(rng.integers(0, 2))
        case = inputs.decode_case(lens, 24, 4, 256, 16, dtype="bf16", pool_factor=1.1,
                                  seed=100 + k)
        print(f"[plan] random batch {k}: S={S} P={P} step={step}", flush=True)
        epoch += 1
        if step:
            base, _ = _step(case, P)
            for e in (epoch, epoch, epoch | 0x80000000):
                got, _ = _step(case, P, plan, e)
                assert np.array_equal(G.bits(base), G.bits(got)), (k, e)
        else:
            t = G.to_dev(case)
            G.write(t)
            want = _partitioned(t, case, P)
            for e in (epoch, epoch, epoch | 0x80000000):
                for a, b in zip(want, _partitioned(t, case, P, plan, e)):
                    assert np.array_equal(a, b), (k, e)


@pytest.mark.parametrize("k", range(10))
def test_longest_first_deal_random_batches(k):
    """Batches of at most 64 sequences with partitions of several sizes (the
    launches that store a plan deal them longest-first): the planning call
    and a call that reads the stored plan give the unplanned bits, as a step
    and as a plain partitioned call, and the step matches the oracle."""
    rng = np.random.default_rng(500 + k)
    S = int(rng.integers(2, 65))
    lens = [int(x) for x in np.exp(rng.uniform(np.log(16), np.log(9000), S))]
    P = int(rng.choice([256, 512, 1024, 1792, 2048]))
    hq, hkv = [(24, 4), (16, 8), (8, 1), (24, 3)][k % 4]
    print(f"[plan] longest-first batch {k}: S={S} P={P} heads {hq}/{hkv}", flush=True)
    case = inputs.decode_case(lens, hq, hkv, 256, 16, dtype="bf16", pool_factor=1.2, seed=700 + k)
    plan = pa.decode_plan_buffer()
    base, _ = _step(case, P)
    for e in (31 + k, 31 + k):
        got, _ = _step(case, P, plan, e)
        assert np.array_equal(G.bits(base), G.bits(got)), e
    assert G.max_err(G.host(got), _oracle_step(case)) <= G.BF16_TOL
    t = G.to_dev(case)
    G.write(t)
    want = _partitioned(t, case, P)
    for e in (900 + k, 900 + k):
        for a, b in zip(want, _partitioned(t, case, P, plan, e)):
            assert np.array_equal(a, b), e


def test_longest_first_deal_fp8():
    """The FP8 kernel's longest-first deal (mixed batch, its 2048-token
    partitions and a 1024-token one): planning and reading calls give the
    unplanned bits."""
    from tests.test_gpu_fp8 import _fp8_case, _write
    import bench
    ks, vs = bench.FP8_SCALES["mixed"]
    case = inputs.preset_case("mixed", seed=3)
    t, _, _ = _fp8_case(case, ks, vs)
    _write(t, ks, vs)
    for P in (G.bench_partitions()[1]["mixed"], 1024):
        want = _fp8_records(t, case, P, ks, vs)
        plan = pa.decode_plan_buffer()
        for _ in range(2):
            for a, b in zip(want, _fp8_records(t, case, P, ks, vs, plan, 77)):
                assert np.array_equal(a, b), P
