"""Benchmark: paged decode attention on one MI355X.

Workload (default): the mixed-length multi-tenant decode batch - 64 sequences
with context lengths drawn log-uniform in [16, 8192], 24 query heads / 4 KV
heads, head_dim 256, BF16, block_size 16, blocks scattered over a pool 1.5x
the needed size - run as 16 independent layers back to back.

One step = for each of the 16 layers: the slot-mapped write of the step's
new K/V (pa_reshape_and_cache), split-context decode (pa_decode_partitioned,
1792-token partitions) and the log-sum-exp merge (pa_reduce). Block tables and
slot mappings come from the host allocator's layout before timing starts;
every input is resident in HBM when the timed region begins.

Printed JSON (one line): value = effective KV read bandwidth of the whole
step (exact context tokens x 4096 B per token per layer / step time); also
tokens/s (64 new tokens per step), the decode kernel's roofline against
8 TB/s HBM (its own launches timed with HIP events on the launch stream) and
the CPU oracle timed on a bounded sample of the same workload.

The FP8 leg ("fp8") repeats the decode step over E4M3FN code pools (the
same workload's values divided by fixed pool scales; the value pool in its
transposed block layout): per layer the quantising write, the matrix-core
FP8 decode and the merge. It reports its own step time and the FP8 kernel's
roofline (one byte per cached element) and does not enter `value`.

After the decode measurement, a separate leg times the chunked-prefill
workload (16 sequences with 0-6000 cached tokens, a 512-token causal chunk
each, 24/4 heads, head_dim 256, BF16, block_size 16): the slot write of the
chunk's K/V and pa_prefill_chunk, the latter against the BF16 matrix-core
peak. It reports under "prefill" and does not enter `value`. Two more side
legs time block moves: "cow" (copy-on-write clones of a 16-rollout fan-out,
pa_copy_blocks, against HBM) and "swap" (8 sequences preempted to pinned
host memory and brought back, pa_swap_blocks, against the PCIe link).
"""

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense BF16 matrix cores, vendor figure
HERE = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch, measured with FETCH_SIZE / WRITE_SIZE counters and
# scaled by the same counters' reading for a plain copy of known size: one
# record per (kernel leg, workload), each keyed to the sha256 of the sources
# of the kernel it measured (a changed kernel reports null).
_CSRC = os.path.join(HERE, "paged_kv_cache_454_amd", "csrc")
_DECODE_SRC = [os.path.join(_CSRC, f) for f in ("decode_mfma.hip", "pa_device.h",
                                                "persistent_plan.h")]
_TILED_SRC = [os.path.join(_CSRC, f) for f in ("decode_tiled.hip", "pa_device.h")]
_FP8_SRC = [os.path.join(_CSRC, f) for f in ("decode_fp8.hip", "pa_device.h",
                                             "persistent_plan.h")]
TRAFFIC_RECORDS = {
    ("bf16-split", "mixed"): ("decode_mfma_mixed_64seq_hbm_counters.md", _DECODE_SRC),
    ("bf16-split", "long"): ("decode_mfma_long_4seq_hbm_counters.md", _DECODE_SRC),
    ("bf16-split", "uniform"): ("decode_tiled_uniform_8x2048_hbm_counters.md", _TILED_SRC),
    ("fp8", "mixed"): ("decode_fp8_mixed_64seq_16layer.md", _FP8_SRC),
    ("fp8", "long"): ("decode_fp8_long_4seq_hbm_counters.md", _FP8_SRC),
}
PREFILL_TRAFFIC_RECORD = os.path.join(HERE, "profiles", "prefill_mfma_chunked_16x512.md")
PREFILL_TRAFFIC_SOURCES = [os.path.join(_CSRC, f) for f in ("prefill_mfma.hip", "pa_device.h")]
# Partition size per workload: the long-context configuration fixes 512
# tokens; for the others it is the fastest measured on MI355X (mixed
# 16-layer step with the matrix-core decode: 1.335 ms at 1536, 1.281-1.284
# ms at 1792, 1.297-1.303 ms at 2048, 1.822 ms at 4096, where too few units
# are left to balance the CUs). The FP8 leg: 1.005 ms at 512, 0.928 ms at
# 1024, 0.931 ms at 1792, 0.915 ms at 2048; on the long-context batch its
# decode takes 44.5 us at 512, 38.1 us at 1536 and 39.7-39.9 us at 2048.
# Bit 31 of a plan epoch: the launch plans afresh and stores its slots under
# the epoch without the bit. A step's first layer sets it, so that launch plans
# whatever an earlier user of the buffer's memory left there; the later layers
# read its slots.
PLAN_REFRESH = 0x80000000
DEFAULT_PARTITION = {"mixed": 1792, "long": 512, "uniform": 256}
FP8_DEFAULT_PARTITION = {"mixed": 2048, "long": 1536, "uniform": 256}
WORKLOAD_NAMES = {
    "mixed": "mixed-length multi-tenant decode, 64 seqs log-uniform [16, 8192], 16 layers",
    "long": "long-context split decode, 4 seqs {8192, 16384, 32768, 32768}, bs 32",
    "uniform": "uniform decode, 8 seqs x 2048, bs 16",
}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-context partition in tokens (default: 1792 for the mixed "
                         "workload, 512 for the long one as its configuration states, 256 "
                         "for the uniform one)")
    ap.add_argument("--workload", default="mixed", choices=["mixed", "long", "uniform"],
                    help="decode workload (default: the mixed-length 16-layer batch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 256 MiB device copy three times: its "
                         "FETCH_SIZE/WRITE_SIZE under a counter profiler give the scale "
                         "between those counters and bytes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle sample (0 disables it)")
    ap.add_argument("--fp8", type=int, default=1,
                    help="also time the step over FP8 (E4M3FN) pools (0: skip)")
    ap.add_argument("--fp8-partition-size", type=int, default=None,
                    help="partition size of the FP8 leg (default: 2048 for the mixed workload, "
                         "512 for the long one, 256 for the uniform one)")
    ap.add_argument("--mode", default=None, choices=["split", "balanced", "single", "whole"],
                    help="how the step runs attention: split (pa_decode_partitioned + "
                         "pa_reduce, the default), balanced (pa_decode_partitioned_balanced + "
                         "pa_reduce), single (pa_decode_balanced) or whole (pa_decode)")
    ap.add_argument("--step", default=None, choices=["fused", "calls"],
                    help="fused: each layer's step is one pa_decode_step call (the step's K/V "
                         "write inside the decode and merge launches); calls: "
                         "pa_reshape_and_cache, then the decode and pa_reduce (default: per "
                         "workload, the faster measured). Split and whole modes only; the other "
                         "form is timed too, as ms_per_step_other")
    ap.add_argument("--compare-step", type=int, default=1,
                    help="also time the other step form (0: only the chosen one, e.g. for "
                         "counter runs that should see one form's launches)")
    ap.add_argument("--side-decode", type=int, default=1,
                    help="with the mixed workload, also time the long-context and uniform "
                         "decode workloads, each in a process of its own (0: skip)")
    ap.add_argument("--leg-json", type=int, default=0,
                    help="print only this workload's decode leg as one JSON line (how the "
                         "mixed run times its long-context and uniform legs)")
    ap.add_argument("--loop-steps", type=int, default=50,
                    help="timed iterations of the continuous-batching loop leg (0 skips it)")
    ap.add_argument("--prefill-reps", type=int, default=10,
                    help="timed repetitions of the side legs, chunked prefill and "
                         "copy-on-write block copies (0 skips them)")
    return ap.parse_args(argv)


def cpu_baseline(seed, budget_s, single_core_s=6.0):
    """Time the fp64 oracle (write + decode) on whole passes over one layer of
    the same workload until the budget is spent; GB/s over the same
    algorithmic KV bytes as the GPU figure. Runs with the BLAS thread pool as
    the process gets it (``cores`` = its size, the threads actually used),
    then once more limited to one thread."""
    from oracle import attention as oracle
    from paged_kv_cache_454_amd import inputs
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    case = inputs.preset_case("mixed", seed=seed, garbage="random")

    def run(budget):
        t0 = time.perf_counter()
        done_tokens, done_seqs, passes = 0, 0, 0
        while True:   # whole passes over the layer (write + decode of every sequence)
            kc, vc = oracle.cache_write(case.key_cache, case.value_cache, case.key, case.value,
                                        case.slot_mapping, case.block_size)
            oracle.decode(case.query, kc, vc, case.block_tables, case.context_lens,
                          case.block_size, case.scale)
            done_tokens += int(case.context_lens.sum())
            done_seqs += case.num_seqs
            passes += 1
            if time.perf_counter() - t0 > budget:
                break
        dt = time.perf_counter() - t0
        return done_tokens * 4096 / dt / 1e9, passes, done_tokens, done_seqs, dt

    gbs, passes, done_tokens, done_seqs, dt = run(budget_s)
    res = {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{passes} pass(es) over 1 layer of the mixed workload (slot write + "
                     f"fp64 decode of all {case.num_seqs} sequences, {done_tokens} context "
                     f"tokens in total) in {dt:.1f} s; decode tokens/s for a 16-layer step "
                     f"{done_seqs / dt / 16:.3f}",
           "host_cpus": os.cpu_count(),
           "cpu_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
           else None}
    if threadpool_limits is not None and single_core_s > 0:
        with threadpool_limits(limits=1):
            g1, p1, _, s1, d1 = run(single_core_s)
        res["single_core"] = {"value": round(g1, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{p1} pass(es) of the same layer in {d1:.1f} s"}
    return res


def counted_traffic(workload, partition_size, seed, record, sources):
    """A counter record's HBM bytes per launch, or None when the record is
    missing, was taken on another workload, or the kernel's source has
    changed since."""
    try:
        text = open(record).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        h = hashlib.sha256()
        for f in sources:
            with open(f, "rb") as fh:
                h.update(fh.read())
    except (OSError, AttributeError, ValueError):
        return None
    if (rec.get("source_sha256") != h.hexdigest() or rec.get("workload") != workload
            or rec.get("partition_size") != partition_size or rec.get("seed") != seed):
        return None
    return int(rec["traffic_bytes"])


def decode_traffic(kind, workload, partition_size, seed):
    if (kind, workload) not in TRAFFIC_RECORDS:
        return None
    name, sources = TRAFFIC_RECORDS[(kind, workload)]
    return counted_traffic(workload, partition_size, seed, os.path.join(HERE, "profiles", name),
                           sources)


def timed_launches(fn, reps, stream):
    """Mean duration (ms) of fn's launch, each bracketed by HIP events on the
    stream it runs on."""
    import torch
    pairs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)


def decode_launch_ms(launch, nlayers, reps, stream, min_launches=48):
    """Mean duration (ms) of one decode launch: each repetition runs the
    layers' decodes back to back, cycling through the layers for at least
    min_launches launches, between two HIP events on the stream the kernels
    are launched on. The host enqueues a launch much faster than the GPU
    runs it, so the queue stays ahead and the events see the kernels (and
    the gaps between them), not the host's submission time. In a kernel
    trace the GPU idles up to 10 us where one event pair ends and the next
    begins, against about 0.5 us between launches inside a pair; with three
    launches per pair that added about 3 us to each."""
    import torch
    n = nlayers * max(1, -(-min_launches // nlayers))
    pairs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            launch(i % nlayers)
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) / n


def prefill_leg(seed, reps, dev):
    """Chunked prefill at full size: the chunk's slot write and the causal
    paged attention of its 8,192 query rows."""
    import torch

    import paged_kv_cache_454_amd as pa
    from paged_kv_cache_454_amd import inputs
    t, m = inputs.device_prefill_case(seed, dev)
    stream = torch.cuda.current_stream()
    out = torch.empty(tuple(t["query"].shape), dtype=torch.float32, device=dev)

    def write():
        pa.pa_reshape_and_cache(t["key"], t["value"], t["key_cache"], t["value_cache"],
                                t["slot_mapping"], stream=stream)

    def prefill():
        pa.pa_prefill_chunk(out, t["query"], t["key_cache"], t["value_cache"],
                            t["block_tables"], t["query_start_loc"], t["context_lens"],
                            m["max_query_len"], m["scale"], stream=stream)

    # Untimed launches first: the matrix cores' clock ramps over the first
    # tens of ms of this load (measured: one warm-up launch, then 10 timed
    # ones averaged 770-790 us; the next 10 took 702-706 us, the 10 after
    # those 679-687 us).
    write()
    for _ in range(max(20, 3 * reps)):
        prefill()
    torch.cuda.synchronize()
    w_ms = timed_launches(write, reps, stream)
    p_ms = timed_launches(prefill, reps, stream)
    hq, d = t["query"].shape[1], t["query"].shape[2]
    hkv = t["key"].shape[1]
    n = m["chunk"]
    # Q.K^T and P.V over the causal span: query j of sequence s sees c_s + j + 1 keys.
    flops = sum(4 * d * hq * (n * int(c) + n * (n + 1) // 2) for c in m["existing"])
    kv_bytes = int(m["lens"].sum()) * hkv * d * 2 * 2
    w_bytes = 2 * 2 * t["key"].numel() * 2   # K and V rows, read and written, BF16
    tf = flops / (p_ms * 1e-3) / 1e12
    return {
        "workload": "chunked prefill, 16 seqs x (0-6000 cached + 512-token causal chunk), "
                    "24/4 heads, d 256, bs 16, 1 layer",
        "query_rows": int(t["query"].shape[0]), "flops": flops,
        "prefill_us": round(p_ms * 1e3, 2), "tflops": round(tf, 1),
        "roofline": {"bound": "mfma", "kernel": "pa_prefill_chunk", "achieved": round(tf, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": counted_traffic("prefill", None, seed, PREFILL_TRAFFIC_RECORD,
                                                PREFILL_TRAFFIC_SOURCES)},
        "kv_context_bytes": kv_bytes,
        "write_us": round(w_ms * 1e3, 2),
        "write_gbs": round(w_bytes / (w_ms * 1e-3) / 1e9, 1),
        "reps": reps,
    }


def cow_leg(seed, reps, dev):
    """Copy-on-write fan-out: the 64 prompts of the mixed workload each
    forked into 16 rollouts with the native allocator; the first decode step
    of every rollout appends one token, which queues one block copy per
    rollout that shares a partly filled last block. The step applies those
    copies to the pools of all 16 layers (4 KV heads x 16 tokens x 256,
    BF16): 16 pa_copy_blocks launches over 16 separate pool pairs, about
    1.9 GB read and written per step, far more than the 256 MB Infinity
    Cache holds."""
    import torch

    import paged_kv_cache_454_amd as pa
    from paged_kv_cache_454_amd import BlockAllocator, inputs
    lens = [int(x) for x in inputs.preset_lengths("mixed", seed)]
    bs, rollouts, hkv, d, nlayers = 16, 16, 4, 256, 16
    nb = sum(-(-n // bs) for n in lens) + len(lens) * rollouts + 16
    a = BlockAllocator(nb, bs)
    for s, n in enumerate(lens):
        a.append(s * rollouts, n)
        for r in range(1, rollouts):
            a.fork(s * rollouts, s * rollouts + r)
    for s in range(len(lens)):
        for r in range(rollouts):
            a.append(s * rollouts + r, 1)
    pairs = a.take_copies()
    pools = [(torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev),
              torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev))
             for _ in range(nlayers)]
    pd = torch.from_numpy(pairs).to(dev)
    stream = torch.cuda.current_stream()

    def step():
        for kc, vc in pools:
            pa.pa_copy_blocks(kc, vc, pd, stream=stream)

    step()
    torch.cuda.synchronize()
    ms = timed_launches(step, reps, stream) / nlayers
    nbytes = 2 * 2 * len(pairs) * hkv * bs * d * 2   # K and V blocks, read and written
    gbs = nbytes / (ms * 1e-3) / 1e9
    del pools
    return {
        "workload": "copy-on-write fan-out: 64 mixed-length prompts x 16 rollouts, first "
                    "divergent step, blocks of 4 x 16 x 256 BF16, 16 layers",
        "pairs": int(len(pairs)), "bytes_per_launch": nbytes,
        "copy_us_per_launch": round(ms * 1e3, 2),
        "roofline": {"bound": "hbm", "kernel": "pa_copy_blocks", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "steps": reps,
    }


PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16 host link, per direction, nominal


def swap_leg(seed, reps, dev):
    """Swapping to host memory: 8 of the mixed workload's 64 sequences
    (seeded choice) are preempted - the native allocator moves their blocks
    to a pinned host pool - and brought back into fresh device blocks. Each
    direction applies its block moves to the pools of all 16 layers (4 KV
    heads x 16 tokens x 256, BF16) with one pa_swap_blocks launch per layer:
    the kernel reads HBM and writes host memory over the bus (swap-out), or
    the reverse (swap-in)."""
    import numpy as np
    import torch

    import paged_kv_cache_454_amd as pa
    from paged_kv_cache_454_amd import BlockAllocator, inputs
    lens = [int(x) for x in inputs.preset_lengths("mixed", seed)]
    bs, hkv, d, nlayers = 16, 4, 256, 16
    victims = sorted(int(v) for v in np.random.default_rng(seed + 2).choice(len(lens), 8,
                                                                           replace=False))
    nb = sum(-(-n // bs) for n in lens) + 16
    nh = sum(-(-lens[v] // bs) for v in victims)
    a = BlockAllocator(nb, bs)
    a.set_host_pool(nh)
    for s, n in enumerate(lens):
        a.append(s, n)
    out_pairs = np.concatenate([a.swap_out(v) for v in victims])
    in_pairs = np.concatenate([a.swap_in(v) for v in victims])
    dev_pools = [(torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev),
                  torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev))
                 for _ in range(nlayers)]
    host_pools = [(torch.zeros((nh, hkv, bs, d), dtype=torch.bfloat16, pin_memory=True),
                   torch.zeros((nh, hkv, bs, d), dtype=torch.bfloat16, pin_memory=True))
                  for _ in range(nlayers)]
    po, pi = torch.from_numpy(out_pairs).to(dev), torch.from_numpy(in_pairs).to(dev)
    stream = torch.cuda.current_stream()

    def swap_out():
        for (dk, dv), (hk, hv) in zip(dev_pools, host_pools):
            pa.pa_swap_blocks(dk, dv, hk, hv, po, stream=stream)

    def swap_in():
        for (dk, dv), (hk, hv) in zip(dev_pools, host_pools):
            pa.pa_swap_blocks(hk, hv, dk, dv, pi, stream=stream)

    swap_out()
    swap_in()
    torch.cuda.synchronize()
    block_bytes = hkv * bs * d * 2
    res = {"workload": f"preempt 8 of the 64 mixed-length sequences ({nh} blocks of 4 x 16 x "
                       f"256 BF16) to pinned host memory and back, 16 layers",
           "sequences": victims, "pairs": int(len(out_pairs)), "steps": reps}
    for name, fn in (("out", swap_out), ("in", swap_in)):
        ms = timed_launches(fn, reps, stream) / nlayers
        nbytes = 2 * len(out_pairs) * block_bytes        # K and V blocks crossing the link
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"bytes_per_launch": nbytes, "us_per_launch": round(ms * 1e3, 2),
                     "roofline": {"bound": "pcie", "kernel": "pa_swap_blocks",
                                  "achieved": round(gbs, 2), "peak": PCIE_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / PCIE_PEAK_GBS, 4),
                                  "traffic": None}}
    del dev_pools, host_pools
    return res


def read_ceiling(dev, seed, reps=5):
    """Measured HBM read ceilings to set beside the 8 TB/s vendor peak: the
    library's read probe (pa_read_probe: 8 KiB blocks, decode's non-temporal
    16-byte loads) over a 4 GiB pool, once in address order (a streaming
    read) and once in a seeded random block order (decode's gather pattern
    without its arithmetic). Best of `reps`, HIP events on the launch stream."""
    import numpy as np
    import torch

    import paged_kv_cache_454_amd as pa
    pool = torch.ones(1 << 30, dtype=torch.int32, device=dev)   # 4 GiB
    nblocks = pool.numel() * 4 // 8192
    sink = torch.empty(int(pa.binding.lib().pa_read_probe_sink_words()), dtype=torch.int32,
                       device=dev)
    stream = torch.cuda.current_stream()
    res = {"kernel": "pa_read_probe", "pool_bytes": pool.numel() * 4, "unit": "GB/s"}
    orders = {"sequential": torch.arange(nblocks, dtype=torch.int32, device=dev),
              "random_8k_blocks": torch.from_numpy(
                  np.random.default_rng(seed + 3).permutation(nblocks).astype(np.int32)).to(dev)}
    for name, order in orders.items():
        pa.pa_read_probe(pool, order, sink, stream=stream)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            pa.pa_read_probe(pool, order, sink, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        gbs = nblocks * 8192 / (best * 1e-3) / 1e9
        res[name] = {"value": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del pool, orders, sink
    torch.cuda.empty_cache()
    return res


def loop_leg(seed, steps, dev):
    """Continuous-batching decode loop (``DecodeLoop``): 64 batch slots, 16
    layers of the mixed workload's shape (24/4 heads, d 256, block 16, the
    mixed workload's partition size), each layer one pa_decode_step call
    sharing the step's plan. Prompts are drawn log-uniform in [16, 8192] like
    the mixed workload, generation lengths uniform in [16, 128]; a finished
    request's slot is refilled at once (its prompt K/V written into all 16
    layers). Times `steps` whole iterations (native allocator step, batch
    upload, write + split decode + merge for 16 layers, releases and
    admissions) after a warm-up, with eager launches and with the device part
    replayed as a HIP graph."""
    import time

    import numpy as np
    import torch

    from paged_kv_cache_454_amd import inputs
    from paged_kv_cache_454_amd.decode_loop import DecodeLoop
    slots, layers, hq, hkv, d, bs = 64, 16, 24, 4, 256, 16
    P = DEFAULT_PARTITION["mixed"]
    maxc = 8192 + 512
    nb = slots * (maxc // bs) + 64
    rng = np.random.default_rng(seed + 1)
    prompt = torch.randn((layers, 8192, hkv, d), dtype=torch.bfloat16, device=dev)
    res = {}
    for mode in ("eager", "graph"):
        loop = DecodeLoop(slots=slots, num_blocks=nb, block_size=bs, layers=layers,
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, partition_size=P,
                          max_context=maxc, device=dev, use_graph=(mode == "graph"))
        loop.query.normal_()
        loop.new_k.normal_()
        loop.new_v.normal_()
        nid = [0]
        admitted = [0]

        def admit(slot):
            n = int(inputs.log_uniform_lengths(rng, 1, 16, 8192)[0])
            loop.admit(slot, nid[0], n, int(rng.integers(16, 129)), prompt[:, :n], prompt[:, :n])
            nid[0] += 1
            admitted[0] += 1

        for s in range(slots):
            admit(s)

        def iteration():
            act = loop.step()
            for s, _ in loop.finish_done():
                admit(s)
            return len(act)

        for _ in range(5):
            iteration()
        torch.cuda.synchronize()
        admitted[0] = 0
        t0 = time.perf_counter()
        tokens = sum(iteration() for _ in range(steps))
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        res[mode] = {"tokens_per_s": round(tokens / dt, 1), "ms_per_step": round(dt / steps * 1e3, 4),
                     "admissions": admitted[0]}
        loop.close()
        del loop
        torch.cuda.empty_cache()
    return {
        "workload": f"continuous-batching decode loop: 64 slots, 16 layers, 24/4 heads, d 256, "
                    f"bs 16, P {P}, prompts log-uniform [16, 8192], generation uniform [16, 128]",
        "steps": steps, **res,
    }


# k_scale, v_scale of the FP8 pools: N(0,1) data uses codes up to ~200; the
# long-context batch adds a per-head bias of scale 3 (|x| up to ~16).
FP8_SCALES = {"mixed": (0.0375, 0.021), "uniform": (0.0375, 0.021), "long": (0.05, 0.05)}


def fp8_leg(layers, meta, P, steps, warmup, dev, workload, seed):
    """The same decode step over FP8 (E4M3FN) pools: each layer's BF16 pools
    are converted to codes of value / scale before timing (input
    preparation); one step = per layer the quantising write of the step's new
    K/V (pa_reshape_and_cache_fp8), pa_decode_partitioned_fp8 (planned: the
    step's first layer plans, the others read its plan) and pa_reduce."""
    import numpy as np
    import torch

    import paged_kv_cache_454_amd as pa
    from paged_kv_cache_454_amd import inputs
    ks, vs = FP8_SCALES[workload]
    # new tokens per step: one per sequence per independent copy of the layer
    sets = len(layers) // inputs.PRESETS[workload].get("layers", 1)

    def codes(x, sc):
        return (x.float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)

    # value pools store each block transposed ([H][d][bs] per block)
    pools = [(codes(L["key_cache"], ks), codes(L["value_cache"].transpose(2, 3), vs).contiguous())
             for L in layers]
    torch.cuda.synchronize()
    lens = meta["lens"]
    S = len(lens)
    hq, d = layers[0]["query"].shape[1], layers[0]["query"].shape[2]
    hkv = pools[0][0].shape[1]
    max_parts = max(1, math.ceil(int(lens.max()) / P))
    po = torch.empty((S, hq, max_parts, d), dtype=torch.float32, device=dev)
    pm = torch.empty((S, hq, max_parts), dtype=torch.float32, device=dev)
    ps = torch.empty((S, hq, max_parts), dtype=torch.float32, device=dev)
    outs = [torch.empty((S, hq, d), dtype=torch.float32, device=dev) for _ in layers]
    bt, cl, sm = meta["block_tables"], meta["context_lens"], meta["slot_mapping"]
    scale = meta["scale"]
    stream = torch.cuda.current_stream()

    # One-layer workloads: every launch plans for itself (see decode_leg).
    plan = None if "layers" not in inputs.PRESETS[workload] else pa.decode_plan_buffer(dev)
    epoch = [0]

    def decode(li):
        kc, vc = pools[li]
        if li == 0:
            epoch[0] += 1
        pa.pa_decode_partitioned_fp8(po, pm, ps, layers[li]["query"], kc, vc, bt, cl, scale, ks,
                                     vs, P, stream=stream, plan=plan,
                                     plan_epoch=epoch[0] | (PLAN_REFRESH if li == 0 else 0))

    def step():
        for li, L in enumerate(layers):
            kc, vc = pools[li]
            pa.pa_reshape_and_cache_fp8(L["key"], L["value"], kc, vc, sm, ks, vs, stream=stream)
            decode(li)
            pa.pa_reduce(outs[li], po, pm, ps, cl, P, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps
    kern_ms = decode_launch_ms(decode, len(layers), max(3, min(steps, 20)), stream)
    kv_bytes_layer = int(lens.sum()) * hkv * d * 2      # one byte per element, K and V
    k_gbs = kv_bytes_layer / (kern_ms * 1e-3) / 1e9
    del pools, po, pm, ps, outs
    torch.cuda.empty_cache()
    return {
        "what": f"the decode step over FP8 E4M3FN pools (scales k {ks}, v {vs}): per pool set "
                "pa_reshape_and_cache_fp8 + pa_decode_partitioned_fp8_planned + pa_reduce",
        "ms_per_step": round(ms_step, 5),
        "tokens_per_s": round(S * sets / (ms_step * 1e-3), 1),
        "kv_gbs_effective": round(kv_bytes_layer * len(layers) / (ms_step * 1e-3) / 1e9, 2),
        "partition_size": P,
        "roofline": {"bound": "hbm", "kernel": "pa_decode_partitioned_fp8_planned",
                     "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": decode_traffic("fp8", workload, P, seed),
                     "avg_launch_us": round(kern_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": kv_bytes_layer},
    }


# How a decode step runs the attention:
#  "split"    pa_decode_partitioned + pa_reduce (whole units per workgroup)
#  "balanced" pa_decode_partitioned_balanced + pa_reduce (equal shares per
#             compute unit; cut units merged by the call's second kernel)
#  "single"   pa_decode_balanced (single pass, equal shares; no reduce)
#  "whole"    pa_decode (single pass, one (sequence, KV head) per workgroup)
# The split path is the fastest measured on every decode workload here
# (mixed 71.5 us against 82.9 balanced and 84.7 single; long 63.1 against
# 71.2 and 79.8; uniform 16.2 against 27.4 single): with the memory system
# saturated, a piece end costs more than the round that balancing saves.
DEFAULT_MODE = {"mixed": "split", "long": "split", "uniform": "split"}
MODE_KERNEL = {"split": "pa_decode_partitioned_planned",
               "balanced": "pa_decode_partitioned_balanced",
               "single": "pa_decode_balanced", "whole": "pa_decode"}
# Step form: one pa_decode_step call per layer, or the write, the decode and
# the merge as three calls. Timed alternately in one run (median of three
# each): mixed 1.2183 ms fused against 1.2447 ms, long 0.2120 against 0.2170,
# uniform 0.1798 against 0.1799 (there the tiled kernel reads the step's
# token from the pool, so both forms launch the same three kernels).
DEFAULT_STEP = {"mixed": "fused", "long": "fused", "uniform": "fused"}


def decode_leg(W, P, steps, warmup, dev, seed, fp8_P=None, mode="split", step_form="fused",
               compare=True):
    """One decode workload at full size: K timed steps (per pool set: the
    slot write of the step's new K/V, pa_decode_partitioned at partition
    size P, pa_reduce; as one pa_decode_step call when step_form is "fused")
    after W warm-up steps, then the decode kernel's own launches timed back
    to back on the launch stream. Pool sets are the
    mixed batch's 16 layers, or independent copies of a one-layer workload
    decoded in turn so that no step re-reads K/V the last one left in the
    caches. Returns the leg's figures (and the FP8 leg's, given fp8_P)."""
    import torch

    import paged_kv_cache_454_amd as pa
    from paged_kv_cache_454_amd import inputs

    pre = inputs.PRESETS[W]
    layers_n = pre.get("layers", pre.get("pool_sets", 1))
    layers, meta = inputs.device_decode_layers(W, seed, layers_n, dev)
    lens = meta["lens"]
    S = len(lens)
    hq, d = layers[0]["query"].shape[1], layers[0]["query"].shape[2]
    hkv = pre["num_kv_heads"]
    max_parts = max(1, math.ceil(int(lens.max()) / P))
    po = torch.empty((S, hq, max_parts, d), dtype=torch.float32, device=dev)
    pm = torch.empty((S, hq, max_parts), dtype=torch.float32, device=dev)
    ps = torch.empty((S, hq, max_parts), dtype=torch.float32, device=dev)
    outs = [torch.empty((S, hq, d), dtype=torch.float32, device=dev) for _ in layers]
    bt, cl, sm = meta["block_tables"], meta["context_lens"], meta["slot_mapping"]
    scale = meta["scale"]
    stream = torch.cuda.current_stream()

    scratch = pa.decode_scratch(dev)
    # Plan buffers: the layers of a step share context lengths and block
    # tables, so the first launch of a step plans and the others read its
    # plan. Each step takes a new epoch (the lengths and tables of a real step
    # change every step), so every step plans once, in its first layer's
    # launch (refresh bit set). plan_step serves the fused step, plan_dec the
    # planned partitioned decode. The pool sets of a one-layer workload are
    # successive steps of that layer, not layers of one step: there every
    # launch plans for itself (no buffer).
    one_layer = "layers" not in pre
    plan_step = None if one_layer else pa.decode_plan_buffer(dev)
    plan_dec = None if one_layer else pa.decode_plan_buffer(dev)
    epoch = [0]

    def decode(li):
        L = layers[li]
        if li == 0:
            epoch[0] += 1
        if mode == "single":
            pa.pa_decode_balanced(outs[li], L["query"], L["key_cache"], L["value_cache"], bt, cl,
                                  scale, scratch, stream=stream)
        elif mode == "whole":
            pa.pa_decode(outs[li], L["query"], L["key_cache"], L["value_cache"], bt, cl, scale,
                         stream=stream)
        elif mode == "balanced":
            pa.pa_decode_partitioned_balanced(po, pm, ps, L["query"], L["key_cache"],
                                              L["value_cache"], bt, cl, scale, P, scratch,
                                              stream=stream)
        else:
            pa.pa_decode_partitioned_planned(po, pm, ps, L["query"], L["key_cache"],
                                             L["value_cache"], bt, cl, scale, P, plan_dec,
                                             epoch[0] | (PLAN_REFRESH if li == 0 else 0),
                                             stream=stream)

    def step_calls():
        for li, L in enumerate(layers):
            pa.pa_reshape_and_cache(L["key"], L["value"], L["key_cache"], L["value_cache"], sm,
                                    stream=stream)
            decode(li)
            if mode in ("split", "balanced"):
                pa.pa_reduce(outs[li], po, pm, ps, cl, P, stream=stream)

    def step_fused():
        split = mode == "split"
        epoch[0] += 1
        for li, L in enumerate(layers):
            pa.pa_decode_step(outs[li], L["query"], L["key"], L["value"], L["key_cache"],
                              L["value_cache"], bt, cl, scale, P if split else 0,
                              po if split else None, pm if split else None,
                              ps if split else None, plan=plan_step,
                              plan_epoch=epoch[0] | (PLAN_REFRESH if li == 0 else 0),
                              stream=stream)

    def time_steps(step):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for _ in range(steps):
            step()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / steps

    fusable = mode in ("split", "whole")
    if not fusable:
        step_form = "calls"
    compare = compare and fusable
    main = step_fused if step_form == "fused" else step_calls
    other = step_calls if step_form == "fused" else step_fused
    if compare:
        # The two forms alternate, three timings each, medians reported: the
        # clocks settle over the first timings, so back-to-back single
        # timings would favour whichever form runs second.
        a, b = [], []
        for _ in range(3):
            a.append(time_steps(main))
            b.append(time_steps(other))
        ms_step, ms_other = statistics.median(a), statistics.median(b)
    else:
        ms_step, ms_other = time_steps(main), None

    # The decode kernel's own launches, timed in a separate pass (so the step
    # timing above carries no event overhead) on the stream they run on.
    kern_ms = decode_launch_ms(decode, len(layers), max(3, min(steps, 20)), stream)

    kv_bytes_layer = int(lens.sum()) * hkv * d * 2 * 2
    step_bytes = kv_bytes_layer * layers_n
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    k_gbs = kv_bytes_layer / (kern_ms * 1e-3) / 1e9
    res = {
        "workload": WORKLOAD_NAMES[W],
        "ms_per_step": round(ms_step, 5),
        "tokens_per_s": round(S * (layers_n // pre.get("layers", 1)) / (ms_step * 1e-3), 1),
        "kv_gbs_effective": round(gbs, 2),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "mode": mode,
        "step": step_form,
        "ms_per_step_other": round(ms_other, 5) if ms_other else None,
        "config": {"num_seqs": S, "context_tokens_per_layer": int(lens.sum()),
                   "context_len_range": [int(lens.min()), int(lens.max())],
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                   "block_size": pre["block_size"], "pool_blocks": int(meta["num_blocks"]),
                   "layers": pre.get("layers", 1), "pool_sets_per_step": layers_n,
                   "partition_size": P if mode in ("split", "balanced") else None,
                   "seed": seed},
        "roofline": {"bound": "hbm", "kernel": MODE_KERNEL[mode],
                     "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": decode_traffic("bf16-" + mode, W,
                                               P if mode in ("split", "balanced") else None, seed),
                     "avg_launch_us": round(kern_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": kv_bytes_layer},
    }
    if fp8_P:
        del po, pm, ps, outs, scratch
        res["fp8"] = fp8_leg(layers, meta, fp8_P, steps, warmup, dev, W, seed)
    del layers
    torch.cuda.empty_cache()
    return res


def side_leg(w2, args):
    """One of the other two decode workloads, timed by a child bench.py of its
    own. Pools that a process allocates after earlier allocations went back
    to the driver gather more slowly: the long-context leg took 63.8-64.6 us
    as a second leg of one process (or after a 10 GiB allocate / free
    cycle) against 61.4-61.9 us as the first, same kernel and data. A serving
    process allocates its cache once at start-up, so each workload is timed
    on the memory a fresh process gets. The children run before this process
    touches the GPU."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", w2,
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--seed", str(args.seed),
           "--fp8", str(args.fp8 if w2 == "long" else 0),
           "--compare-step", str(args.compare_step), "--leg-json", "1", "--side-decode", "0",
           "--prefill-reps", "0", "--loop-steps", "0", "--cpu-seconds", "0"]
    if args.step:
        cmd += ["--step", args.step]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        sys.stderr.write(r.stderr[-4000:])
        raise RuntimeError(f"bench.py: the {w2} decode leg failed (exit {r.returncode})")
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)
    side = {}
    if args.side_decode and args.workload == "mixed" and not args.leg_json:
        for w2 in ("long", "uniform"):
            side[w2] = side_leg(w2, args)
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = args.workload
    P = args.partition_size or DEFAULT_PARTITION[W]
    fp8_P = (args.fp8_partition_size or FP8_DEFAULT_PARTITION[W]) if args.fp8 else None
    mode = args.mode or DEFAULT_MODE[W]
    main_leg = decode_leg(W, P, args.steps, args.warmup, dev, args.seed, fp8_P, mode,
                          args.step or DEFAULT_STEP[W], bool(args.compare_step))
    if args.leg_json:
        print(json.dumps(main_leg), flush=True)
        return

    result = {
        "metric": "paged decode attention: effective KV GB/s (% of HBM peak) + tokens/s, 1 GPU",
        "value": main_leg["kv_gbs_effective"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), rounded to BF16)",
        "config": {"workload": main_leg["workload"], "mode": main_leg["mode"],
                   "step": main_leg["step"], **main_leg["config"]},
        "ms_per_step_other": main_leg["ms_per_step_other"],
        "tokens_per_s": main_leg["tokens_per_s"],
        "pct_of_hbm_peak": main_leg["pct_of_hbm_peak"],
        "roofline": main_leg["roofline"],
    }
    if "fp8" in main_leg:
        result["fp8"] = main_leg["fp8"]
    # The other two decode configurations of the target (long-context split
    # decode at its stated 512-token partitions; uniform batch), each with its
    # own step time and kernel roofline, timed first in processes of their own
    # (side_leg); they do not enter `value`.
    result.update(side)
    if args.prefill_reps > 0:
        torch.cuda.empty_cache()
        result["prefill"] = prefill_leg(args.seed, args.prefill_reps, dev)
        result["cow"] = cow_leg(args.seed, args.prefill_reps, dev)
        result["swap"] = swap_leg(args.seed, args.prefill_reps, dev)
        result["hbm_read_ceiling"] = read_ceiling(dev, args.seed)
    if args.loop_steps > 0:
        result["loop"] = loop_leg(args.seed, args.loop_steps, dev)
    if args.cpu_seconds > 0 and W == "mixed":
        result["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_seconds)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
