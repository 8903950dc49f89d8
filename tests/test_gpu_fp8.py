"""FP8 (E4M3FN) KV cache on the GPU against the oracle's fp8 module.

* The quantising write is bit-exact: the pools hold the oracle's codes of the
  fp32 quotients (special values, ties, saturation, NaN, skipped slots).
* Decode over code pools (single pass, and partitions + the log-sum-exp
  reduce) matches the oracle's decode over the dequantised cache within the
  BF16 tolerance (2e-2 max abs: codes widen to BF16 exactly, weights are
  BF16, accumulation fp32), on ragged shapes that take the persistent kernel
  (head_dim 256, blocks of 16 or 32) and the generic one, and at the mixed
  batch's full size on sampled sequences.
* Degenerate cases: empty contexts give zeros, bad block ids and lengths
  poison only their rows, results are deterministic.

FP8 pools: keys [nb][H][bs][d], values transposed per block [nb][H][d][bs].

Input codes of the pools are made by torch's float8_e4m3fn conversion of
seeded values (an input generator; every expected value is the oracle's)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_454_amd as pa
from oracle import attention as oracle_attn
from oracle import fp8 as oracle
from paged_kv_cache_454_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

KS, VS = 0.0375, 0.021   # pool scales: N(0,1) values use codes up to ~200


def _codes(x, scale):
    """E4M3 codes of x / scale as uint8 (torch's conversion; NaN stays NaN)."""
    q = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / torch.tensor(
        scale, dtype=torch.float32)
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _fp8_case(case, ks=KS, vs=VS):
    """Device tensors of a BF16 decode case with the pools as codes (the
    value pool in its transposed block layout [nb][H][d][bs])."""
    kc, vc = _codes(case.key_cache, ks), _codes(np.swapaxes(case.value_cache, 2, 3), vs)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(G.DEV)
    t = dict(key_cache=torch.from_numpy(kc).to(G.DEV), value_cache=torch.from_numpy(vc).to(G.DEV),
             key=bf(case.key), value=bf(case.value), query=bf(case.query),
             block_tables=torch.from_numpy(case.block_tables).to(G.DEV),
             context_lens=torch.from_numpy(case.context_lens).to(G.DEV),
             slot_mapping=torch.from_numpy(case.slot_mapping).to(G.DEV))
    return t, kc, vc


def _write(t, ks=KS, vs=VS):
    pa.pa_reshape_and_cache_fp8(t["key"], t["value"], t["key_cache"], t["value_cache"],
                                t["slot_mapping"], ks, vs)


def _oracle_pools(case, kc, vc, ks=KS, vs=VS):
    return oracle.cache_write(kc, vc, case.key, case.value, case.slot_mapping, case.block_size,
                              ks, vs)


def _decode(t, case, out_dtype=torch.float32, ks=KS, vs=VS):
    out = torch.empty(tuple(t["query"].shape), dtype=out_dtype, device=G.DEV)
    pa.pa_decode_fp8(out, t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                     t["context_lens"], case.scale, ks, vs)
    return out


def _partitioned(t, case, P, max_parts=None, ks=KS, vs=VS):
    S, H, D = t["query"].shape
    n = max_parts or G.max_parts_for(case, P)
    po = torch.full((S, H, n, D), float("nan"), dtype=torch.float32, device=G.DEV)
    pm = torch.full((S, H, n), float("nan"), dtype=torch.float32, device=G.DEV)
    ps = torch.full((S, H, n), float("nan"), dtype=torch.float32, device=G.DEV)
    pa.pa_decode_partitioned_fp8(po, pm, ps, t["query"], t["key_cache"], t["value_cache"],
                                 t["block_tables"], t["context_lens"], case.scale, ks, vs, P)
    out = torch.empty((S, H, D), dtype=torch.float32, device=G.DEV)
    pa.pa_reduce(out, po, pm, ps, t["context_lens"], P)
    return out, po, pm, ps


# ------------------------------------------------------------------- write

SPECIAL = [0.0, -0.0, 1.0, -1.0, 448.0, -448.0, 449.0, 464.0, 465.0, 1e6, -1e30,
           float("inf"), float("-inf"), float("nan"), 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10,
           2.0 ** -6, 1.0625, 1.1875, 2.0 ** -20, 240.0, 0.0146484375]


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hkv,bs,d", [(4, 16, 256), (2, 3, 40), (1, 5, 7), (3, 8, 64)])
def test_cache_write_fp8_bitexact(in_dtype, hkv, bs, d):
    print(f"[fp8] write {in_dtype} hkv={hkv} bs={bs} d={d}", flush=True)
    rng = np.random.default_rng(hkv * 100 + bs * 10 + d)
    nb, n = 9, 23
    key = (rng.standard_normal((n, hkv, d)) * rng.choice([1e-4, 0.01, 1.0, 30.0],
                                                         size=(n, hkv, 1))).astype(np.float32)
    val = (rng.standard_normal((n, hkv, d)) * 3.0).astype(np.float32)
    flat = key.reshape(-1)
    flat[:len(SPECIAL)] = np.array(SPECIAL, dtype=np.float32) * np.float32(KS)
    flat[len(SPECIAL):2 * len(SPECIAL)] = np.array(SPECIAL, dtype=np.float32)
    if in_dtype == "bf16":
        key, val = inputs.round_to_bf16(key), inputs.round_to_bf16(val)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[3] = -1                       # skipped
    slots[7] = nb * bs + 2              # outside the pool: skipped
    kc0 = np.full((nb, hkv, bs, d), 0xA5, np.uint8)
    vc0 = np.full((nb, hkv, d, bs), 0x5A, np.uint8)     # value blocks transposed
    tdt = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    dk, dv = torch.from_numpy(kc0).to(G.DEV), torch.from_numpy(vc0).to(G.DEV)
    pa.pa_reshape_and_cache_fp8(torch.from_numpy(key).to(tdt).to(G.DEV),
                                torch.from_numpy(val).to(tdt).to(G.DEV), dk, dv,
                                torch.from_numpy(slots).to(G.DEV), KS, VS)
    # a slot outside the pool is skipped like a negative one
    wk, wv = oracle.cache_write(kc0, vc0, key, val, np.where(slots < nb * bs, slots, -1), bs, KS,
                                VS)
    assert np.array_equal(dk.cpu().numpy(), wk)
    assert np.array_equal(dv.cpu().numpy(), wv)
    # float8_e4m3fn views of the pools are accepted too; no tokens is a no-op
    pa.pa_reshape_and_cache_fp8(torch.empty((0, hkv, d), dtype=tdt, device=G.DEV),
                                torch.empty((0, hkv, d), dtype=tdt, device=G.DEV),
                                dk.view(torch.float8_e4m3fn), dv.view(torch.float8_e4m3fn),
                                torch.empty((0,), dtype=torch.int64, device=G.DEV), KS, VS)
    assert np.array_equal(dk.cpu().numpy(), wk)


def test_copy_blocks_fp8_pools():
    rng = np.random.default_rng(4)
    nb, hkv, bs, d = 40, 4, 16, 256
    kc = rng.integers(0, 256, size=(nb, hkv, bs, d)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(nb, hkv, d, bs)).astype(np.uint8)
    ids = rng.permutation(nb)
    pairs = np.array([(int(ids[i]), int(ids[10 + i])) for i in range(10)], dtype=np.int32)
    dk, dv = torch.from_numpy(kc).to(G.DEV), torch.from_numpy(vc).to(G.DEV)
    pa.pa_copy_blocks(dk, dv, torch.from_numpy(pairs).to(G.DEV))
    wk, wv = oracle_attn.copy_blocks(kc, vc, pairs)
    assert np.array_equal(dk.cpu().numpy(), wk) and np.array_equal(dv.cpu().numpy(), wv)


# ------------------------------------------------------------------ decode

SHAPES = [
    # (head_dim, block_size, num_q_heads, num_kv_heads, lens); d 256 with
    # blocks of 16/32 take the persistent kernel, the rest the generic one
    (256, 16, 24, 4, [1, 15, 16, 17, 300, 511, 513, 1100, 0]),
    (256, 32, 8, 1, [33, 64, 1000, 2]),
    (256, 16, 12, 4, [700, 20]),
    (128, 16, 8, 8, [5, 250]),
    (64, 8, 16, 2, [1, 2, 70]),
    (256, 5, 8, 2, [3, 99]),
    (256, 16, 32, 4, [2047, 31, 32, 33]),
    (256, 64, 4, 2, [200, 64]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"d{s[0]}-bs{s[1]}-g{s[2]//s[3]}" for s in SHAPES])
def test_decode_fp8_matches_oracle(shape):
    d, bs, hq, hkv, lens = shape
    print(f"[fp8] decode shape={shape}", flush=True)
    case = inputs.decode_case(lens, hq, hkv, d, bs, dtype="bf16", pool_factor=1.3,
                              seed=len(lens) + d)
    t, kc, vc = _fp8_case(case)
    _write(t)
    okc, ovc = _oracle_pools(case, kc, vc)
    # the write also went through the device pools, bit for bit
    assert np.array_equal(t["key_cache"].cpu().numpy(), okc)
    assert np.array_equal(t["value_cache"].cpu().numpy(), ovc)
    want = oracle.decode(case.query, okc, ovc, case.block_tables, case.context_lens, bs,
                         case.scale, KS, VS)
    assert G.max_err(G.host(_decode(t, case)), want) <= G.BF16_TOL
    p1 = -(-16 // bs) * bs
    for P in (p1, 4 * p1, -(-512 // bs) * bs):
        got, *_ = _partitioned(t, case, P)
        assert G.max_err(G.host(got), want) <= G.BF16_TOL, P


def test_partition_records_fp8():
    """Per-partition outputs and log-sum-exps against the oracle's."""
    case = inputs.decode_case([2000, 700, 1300], 24, 4, 256, 16, dtype="bf16", seed=12)
    t, kc, vc = _fp8_case(case)
    _write(t)
    okc, ovc = _oracle_pools(case, kc, vc)
    P = 256
    got, po, pm, ps = _partitioned(t, case, P)
    o_w, lse_w, n = oracle.decode_partitions(case.query, okc, ovc, case.block_tables,
                                             case.context_lens, 16, case.scale, KS, VS, P,
                                             seqs=[0, 2], heads=[0, 5, 23])
    po, pm, ps = G.host(po), G.host(pm), G.host(ps)
    for s in [0, 2]:
        for h in [0, 5, 23]:
            k = int(n[s])
            lse_g = pm[s, h, :k] + np.log(ps[s, h, :k])
            assert np.abs(lse_g - lse_w[s, h, :k]).max() <= G.LSE_TOL
            assert np.abs(po[s, h, :k] - o_w[s, h, :k]).max() <= G.BF16_TOL


def test_mixed_full_size_fp8():
    """The mixed batch (64 sequences, 16..8192 tokens, 24/4 heads, d 256,
    blocks of 16) with FP8 pools, every sequence against the oracle: single
    pass, and partitions at the size the benchmark's FP8 leg times, with
    every partition record compared."""
    print("[fp8] preset=mixed", flush=True)
    case = inputs.preset_case("mixed", seed=0)
    t, kc, vc = _fp8_case(case)
    _write(t)
    okc, ovc = _oracle_pools(case, kc, vc)
    want = oracle.decode(case.query, okc, ovc, case.block_tables, case.context_lens,
                         case.block_size, case.scale, KS, VS)
    assert G.max_err(G.host(_decode(t, case)), want) <= G.BF16_TOL
    P = G.bench_partitions()[1]["mixed"]
    got_p, po, pm, ps = _partitioned(t, case, P)
    assert G.max_err(G.host(got_p), want) <= G.BF16_TOL
    o_w, lse_w, n = oracle.decode_partitions(case.query, okc, ovc, case.block_tables,
                                             case.context_lens, case.block_size, case.scale,
                                             KS, VS, P)
    G.check_records(po, pm, ps, o_w, lse_w, n)
    again, *_ = _partitioned(t, case, P)
    assert np.array_equal(G.bits(got_p), G.bits(again))


# The long batch's keys and values carry a per-head bias of scale 3 (|x| up
# to about 16), so its pools take scales that keep every code finite.
KS_LONG, VS_LONG = 0.05, 0.05


def test_long_full_size_fp8():
    """The long-context batch (4 sequences, 8192..32768 tokens, blocks of 32)
    with FP8 pools at full size: partitions at the size the benchmark's FP8
    leg times, every record and the merged output against the oracle, and
    the single pass."""
    print("[fp8] preset=long", flush=True)
    case = inputs.preset_case("long", seed=0)
    t, kc, vc = _fp8_case(case, KS_LONG, VS_LONG)
    _write(t, KS_LONG, VS_LONG)
    okc, ovc = _oracle_pools(case, kc, vc, KS_LONG, VS_LONG)
    want = oracle.decode(case.query, okc, ovc, case.block_tables, case.context_lens,
                         case.block_size, case.scale, KS_LONG, VS_LONG)
    P = G.bench_partitions()[1]["long"]
    got_p, po, pm, ps = _partitioned(t, case, P, ks=KS_LONG, vs=VS_LONG)
    assert G.max_err(G.host(got_p), want) <= G.BF16_TOL
    o_w, lse_w, n = oracle.decode_partitions(case.query, okc, ovc, case.block_tables,
                                             case.context_lens, case.block_size, case.scale,
                                             KS_LONG, VS_LONG, P)
    G.check_records(po, pm, ps, o_w, lse_w, n)
    assert G.max_err(G.host(_decode(t, case, ks=KS_LONG, vs=VS_LONG)), want) <= G.BF16_TOL


def test_bf16_output_fp8():
    case = inputs.decode_case([700, 20, 1], 24, 4, 256, 16, dtype="bf16", seed=9)
    t, kc, vc = _fp8_case(case)
    _write(t)
    okc, ovc = _oracle_pools(case, kc, vc)
    want = oracle.decode(case.query, okc, ovc, case.block_tables, case.context_lens, 16,
                         case.scale, KS, VS)
    got = G.host(_decode(t, case, out_dtype=torch.bfloat16))
    assert (np.abs(got - want) <= G.BF16_TOL + np.abs(want) * 2.0 ** -8).all()


def test_degenerate_and_poisoned_fp8():
    case = inputs.decode_case([40, 50, 60, 3], 8, 2, 256, 16, dtype="bf16", seed=8)
    t, kc, vc = _fp8_case(case)
    _write(t)
    good = G.host(_decode(t, case))
    again = G.host(_decode(t, case))
    assert np.array_equal(good, again)                       # deterministic
    bt = t["block_tables"].clone()
    bt[0, 1] = case.num_blocks + 5                             # out of the pool
    lens = t["context_lens"].clone()
    lens[2] = 10 ** 6                                          # beyond the table
    lens[3] = 0                                                # empty context
    t2 = dict(t, block_tables=bt, context_lens=lens)
    out = G.host(_decode(t2, case))
    assert np.isnan(out[0]).all() and np.isnan(out[2]).all()
    assert np.array_equal(out[1], good[1])
    assert np.all(out[3] == 0)
    out_p, *_ = _partitioned(t2, case, 32, max_parts=4)
    out_p = G.host(out_p)
    assert np.isnan(out_p[0]).all() and np.isnan(out_p[2]).all()
    assert G.max_err(out_p[1], good[1]) <= G.BF16_TOL
    assert np.all(out_p[3] == 0)


@pytest.mark.parametrize("group", [1, 2, 4, 5, 7])
def test_fp8_matrix_core_groups(group):
    """The FP8 matrix-core kernel at the group sizes the shapes above do not
    reach (its MFMA columns beyond the group repeat real heads): single pass
    and 256-token partitions, ragged contexts over many tiles, block size 16."""
    print(f"[fp8] matrix-core group={group}", flush=True)
    rng = np.random.default_rng(70 + group)
    lens = [int(x) for x in rng.integers(1, 2048, size=12)]
    lens[0] = 2048
    case = inputs.decode_case(lens, 2 * group, 2, 256, 16, dtype="bf16", pool_factor=1.2,
                              seed=group)
    t, kc, vc = _fp8_case(case)
    _write(t)
    okc, ovc = _oracle_pools(case, kc, vc)
    want = oracle.decode(case.query, okc, ovc, case.block_tables, case.context_lens, 16,
                         case.scale, KS, VS)
    assert G.max_err(G.host(_decode(t, case)), want) <= G.BF16_TOL
    got, *_ = _partitioned(t, case, 256)
    assert G.max_err(G.host(got), want) <= G.BF16_TOL
