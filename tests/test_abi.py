"""The C-ABI library loads and exports every symbol include/pa.h declares;
host-side argument checks reject bad calls before anything is launched
(no GPU needed: every call here fails validation)."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_454_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["pa_reshape_and_cache", "pa_decode", "pa_decode_partitioned", "pa_reduce",
              "pa_prefill_chunk", "pa_alloc_create", "pa_alloc_append", "pa_alloc_free",
              "pa_alloc_block_table", "pa_last_error", "pa_reshape_and_cache_fp8",
              "pa_decode_fp8", "pa_decode_partitioned_fp8", "pa_swap_blocks",
              "pa_alloc_swap_out", "pa_alloc_swap_in", "pa_alloc_set_host_pool",
              "pa_decode_step", "pa_decode_plan_bytes", "pa_decode_partitioned_planned",
              "pa_decode_partitioned_fp8_planned", "pa_decode_balanced"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"


def test_version_and_empty_error():
    lib = _lib.lib()
    assert lib.pa_version().decode().count(".") == 2
    assert lib.pa_last_error() is not None


NULL = None


def test_cache_write_rejects_bad_sizes():
    lib = _lib.lib()
    st = lib.pa_reshape_and_cache(NULL, NULL, NULL, NULL, NULL, -1, 4, 256, 16, 10, 1, NULL)
    assert st == _lib.PA_EINVAL and b"num_tokens" in lib.pa_last_error()
    st = lib.pa_reshape_and_cache(NULL, NULL, NULL, NULL, NULL, 5, 4, 256, 16, 10, 1, NULL)
    assert st == _lib.PA_EINVAL and b"null" in lib.pa_last_error()
    st = lib.pa_reshape_and_cache(NULL, NULL, NULL, NULL, NULL, 5, 4, 2048, 16, 10, 1, NULL)
    assert st == _lib.PA_EUNSUPPORTED
    st = lib.pa_reshape_and_cache(NULL, NULL, NULL, NULL, NULL, 5, 4, 256, 16, 10, 7, NULL)
    assert st == _lib.PA_EINVAL
    # zero tokens is a no-op that touches nothing
    assert lib.pa_reshape_and_cache(NULL, NULL, NULL, NULL, NULL, 0, 4, 256, 16, 10, 1,
                                    NULL) == _lib.PA_OK


def _decode(lib, **kw):
    a = dict(out=NULL, q=NULL, kc=NULL, vc=NULL, bt=NULL, cl=NULL, num_seqs=2, hq=24, hkv=4,
             d=256, bs=16, maxb=8, nb=100, scale=0.0625, kv=1, od=0)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["num_seqs"],
                         a["hq"], a["hkv"], a["d"], a["bs"], a["maxb"], a["nb"], a["scale"],
                         a["kv"], a["od"], NULL)


def test_decode_rejects_bad_shapes():
    lib = _lib.lib()
    assert _decode(lib, hq=25) == _lib.PA_EINVAL                  # not a multiple of hkv
    assert _decode(lib, hkv=0) == _lib.PA_EINVAL
    assert _decode(lib, d=96) == _lib.PA_EUNSUPPORTED
    assert _decode(lib, hq=40, hkv=4) == _lib.PA_EUNSUPPORTED     # group 10 > 8
    assert _decode(lib, scale=float("nan")) == _lib.PA_EINVAL
    assert _decode(lib, bs=0) == _lib.PA_EINVAL
    assert _decode(lib, kv=3) == _lib.PA_EINVAL
    assert _decode(lib) == _lib.PA_EINVAL                          # null pointers
    assert _decode(lib, num_seqs=0) == _lib.PA_OK                  # nothing to do


def test_partitioned_and_reduce_reject_bad_partitions():
    lib = _lib.lib()
    st = lib.pa_decode_partitioned(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, 24, 4, 256,
                                   32, 8, 100, 0.0625, 48, 4, 1, NULL)
    assert st == _lib.PA_EINVAL and b"partition_size" in lib.pa_last_error()
    st = lib.pa_decode_partitioned(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, 24, 4, 256,
                                   16, 8, 100, 0.0625, 512, 0, 1, NULL)
    assert st == _lib.PA_EINVAL
    st = lib.pa_reduce(NULL, NULL, NULL, NULL, NULL, 2, 24, 256, 0, 4, 0, NULL)
    assert st == _lib.PA_EINVAL
    st = lib.pa_reduce(NULL, NULL, NULL, NULL, NULL, 2, 24, 256, 512, 4, 0, NULL)
    assert st == _lib.PA_EINVAL
    assert lib.pa_partition_workspace_bytes(4, 24, 256, 64) == 4 * 24 * 64 * (256 + 2) * 4
    assert lib.pa_partition_workspace_bytes(0, 24, 256, 64) == 0


def _step(lib, **kw):
    a = dict(out=NULL, po=NULL, pm=NULL, ps=NULL, q=NULL, k=NULL, v=NULL, kc=NULL, vc=NULL,
             bt=NULL, cl=NULL, num_seqs=2, hq=24, hkv=4, d=256, bs=16, maxb=8, nb=100,
             scale=0.0625, P=512, mp=4, kv=1, od=0, plan=NULL, epoch=0)
    a.update(kw)
    return lib.pa_decode_step(a["out"], a["po"], a["pm"], a["ps"], a["q"], a["k"], a["v"],
                              a["kc"], a["vc"], a["bt"], a["cl"], a["num_seqs"], a["hq"],
                              a["hkv"], a["d"], a["bs"], a["maxb"], a["nb"], a["scale"], a["P"],
                              a["mp"], a["kv"], a["od"], a["plan"], a["epoch"], NULL)


def test_decode_step_rejects_bad_arguments():
    lib = _lib.lib()
    assert _step(lib, P=48, bs=32) == _lib.PA_EINVAL               # not a multiple of bs
    assert b"partition_size" in lib.pa_last_error()
    assert _step(lib, P=8) == _lib.PA_EINVAL                       # under 16
    assert _step(lib, mp=0) == _lib.PA_EINVAL
    assert _step(lib, hq=25) == _lib.PA_EINVAL
    assert _step(lib, d=96) == _lib.PA_EUNSUPPORTED
    assert _step(lib, od=5) == _lib.PA_EINVAL
    assert _step(lib) == _lib.PA_EINVAL and b"null" in lib.pa_last_error()
    assert _step(lib, P=0, mp=0) == _lib.PA_EINVAL                 # single pass, null pointers
    assert _step(lib, num_seqs=0) == _lib.PA_OK                    # nothing to do


def test_planned_calls_reject_bad_arguments():
    lib = _lib.lib()
    st = lib.pa_decode_partitioned_planned(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, 24,
                                           4, 256, 32, 8, 100, 0.0625, 48, 4, 1, NULL, 1, NULL)
    assert st == _lib.PA_EINVAL and b"pa_decode_partitioned_planned" in lib.pa_last_error()
    st = lib.pa_decode_partitioned_fp8_planned(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2,
                                               24, 4, 256, 16, 8, 100, 0.0625, 0.0, 1.0, 512, 4,
                                               NULL, 1, NULL)
    assert st == _lib.PA_EINVAL                                     # zero k_scale
    assert b"pa_decode_partitioned_fp8_planned" in lib.pa_last_error()


def test_prefill_rejects_bad_arguments():
    lib = _lib.lib()
    st = lib.pa_prefill_chunk(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 16, 8192, 512, 24, 4,
                              256, 16, 400, 4000, 0.0625, 0, 0, NULL)
    assert st == _lib.PA_EUNSUPPORTED                              # fp32 KV not covered
    st = lib.pa_prefill_chunk(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 16, 8192, -1, 24, 4,
                              256, 16, 400, 4000, 0.0625, 1, 0, NULL)
    assert st == _lib.PA_EINVAL
    st = lib.pa_prefill_chunk(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 16, 8192, 512, 24, 4,
                              256, 16, 400, 4000, 0.0625, 1, 0, NULL)
    assert st == _lib.PA_EINVAL


def test_fp8_entry_points_reject_bad_arguments():
    lib = _lib.lib()
    w = lambda n, d, dt, ks, vs: lib.pa_reshape_and_cache_fp8(NULL, NULL, NULL, NULL, NULL, n, 4,
                                                              d, 16, 10, dt, ks, vs, NULL)
    assert w(5, 256, 1, 0.0, 1.0) == _lib.PA_EINVAL                # zero scale
    assert w(5, 256, 1, 1.0, float("inf")) == _lib.PA_EINVAL
    assert w(5, 256, 1, -2.0, 1.0) == _lib.PA_EINVAL
    assert w(5, 256, _lib.PA_FP8_E4M3, 1.0, 1.0) == _lib.PA_EINVAL  # inputs are f32/bf16
    assert w(5, 2048, 1, 1.0, 1.0) == _lib.PA_EUNSUPPORTED
    assert w(5, 256, 1, 1.0, 1.0) == _lib.PA_EINVAL                # null pointers
    assert w(0, 256, 1, 1.0, 1.0) == _lib.PA_OK                    # no tokens: no-op

    def dec(hq=24, d=256, ks=1.0, vs=1.0, n=2, od=0):
        return lib.pa_decode_fp8(NULL, NULL, NULL, NULL, NULL, NULL, n, hq, 4, d, 16, 8, 100,
                                 0.0625, ks, vs, od, NULL)
    assert dec(ks=float("nan")) == _lib.PA_EINVAL
    assert dec(vs=0.0) == _lib.PA_EINVAL
    assert dec(d=96) == _lib.PA_EUNSUPPORTED
    assert dec(hq=25) == _lib.PA_EINVAL
    assert dec(od=_lib.PA_FP8_E4M3) == _lib.PA_EINVAL
    assert dec() == _lib.PA_EINVAL                                  # null pointers
    assert dec(n=0) == _lib.PA_OK

    def part(P=512, maxp=4, ks=1.0):
        return lib.pa_decode_partitioned_fp8(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, 24,
                                             4, 256, 16, 8, 100, 0.0625, ks, 1.0, P, maxp, NULL)
    assert part(P=24) == _lib.PA_EINVAL
    assert part(maxp=0) == _lib.PA_EINVAL
    assert part(ks=-1.0) == _lib.PA_EINVAL
    assert part() == _lib.PA_EINVAL                                 # null pointers
    # FP8 pools are accepted by the block copy (no pairs: nothing launched)
    assert lib.pa_copy_blocks(NULL, NULL, NULL, 0, 4, 256, 16, 10, _lib.PA_FP8_E4M3,
                              NULL) == _lib.PA_OK
    assert lib.pa_copy_blocks(NULL, NULL, NULL, 0, 4, 256, 16, 10, 3, NULL) == _lib.PA_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libpa.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.lib()


def test_swap_blocks_rejects_bad_arguments():
    lib = _lib.lib()

    def sw(n=4, hkv=4, d=256, bs=16, snb=10, dnb=10, dt=1):
        return lib.pa_swap_blocks(NULL, NULL, snb, NULL, NULL, dnb, NULL, n, hkv, d, bs, dt, NULL)
    assert sw(n=-1) == _lib.PA_EINVAL and b"num_pairs" in lib.pa_last_error()
    assert sw(snb=0) == _lib.PA_EINVAL
    assert sw(dnb=-3) == _lib.PA_EINVAL
    assert sw(bs=0) == _lib.PA_EINVAL
    assert sw(dt=7) == _lib.PA_EINVAL
    assert sw() == _lib.PA_EINVAL and b"null" in lib.pa_last_error()
    assert sw(n=0) == _lib.PA_OK                                    # no pairs: no-op
    assert sw(n=0, dt=_lib.PA_FP8_E4M3) == _lib.PA_OK


def test_read_probe_rejects_bad_arguments():
    lib = _lib.lib()
    fake = ctypes.c_void_p(16)          # never dereferenced: validation fails first
    assert lib.pa_read_probe(NULL, 0, NULL, -1, fake, 1 << 20, NULL) == _lib.PA_EINVAL
    assert lib.pa_read_probe(NULL, -5, NULL, 0, fake, 1 << 20, NULL) == _lib.PA_EINVAL
    assert lib.pa_read_probe(NULL, 0, NULL, 0, NULL, 1 << 20, NULL) == _lib.PA_EINVAL
    assert lib.pa_read_probe(fake, 8192, NULL, 4, fake, 1 << 20, NULL) == _lib.PA_EINVAL
    st = lib.pa_read_probe(fake, 8192, fake, 4, fake, 10, NULL)
    assert st == _lib.PA_EINVAL and b"sink" in lib.pa_last_error()


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; --gpus N > 1 exits with a message (checked
    before anything touches a GPU)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_side_legs_run_in_child_processes(monkeypatch):
    """The mixed run times the long-context and uniform legs by child
    bench.py processes (each on the memory a fresh process gets): each child
    gets its workload, the step settings, FP8 only for the long-context leg
    and no nested side legs; its last stdout line is the leg's JSON; a failed
    child raises. The children start before the parent touches a GPU."""
    import json
    import subprocess
    import sys
    sys.path.insert(0, ROOT)
    import bench
    calls = []

    def fake_run(cmd, capture_output, text, timeout):
        calls.append(cmd)
        w = cmd[cmd.index("--workload") + 1]
        return subprocess.CompletedProcess(cmd, 0, stdout="noise\n" + json.dumps({"leg": w}) + "\n",
                                           stderr="")

    monkeypatch.setattr(subprocess, "run", fake_run)
    args = bench.parse(["--steps", "7", "--warmup", "2", "--step", "calls"])
    for w2 in ("long", "uniform"):
        assert bench.side_leg(w2, args) == {"leg": w2}
    (c_long, c_uni) = calls
    opt = lambda c, k: c[c.index(k) + 1]
    for c, w in ((c_long, "long"), (c_uni, "uniform")):
        assert c[0] == sys.executable and c[1].endswith("bench.py")
        assert opt(c, "--workload") == w and opt(c, "--leg-json") == "1"
        assert opt(c, "--side-decode") == "0" and opt(c, "--prefill-reps") == "0"
        assert opt(c, "--steps") == "7" and opt(c, "--warmup") == "2"
        assert opt(c, "--step") == "calls"
        assert "--partition-size" not in c and "--mode" not in c
    assert opt(c_long, "--fp8") == "1" and opt(c_uni, "--fp8") == "0"

    def failing_run(cmd, capture_output, text, timeout):
        return subprocess.CompletedProcess(cmd, 3, stdout="", stderr="boom")

    monkeypatch.setattr(subprocess, "run", failing_run)
    with pytest.raises(RuntimeError, match="long decode leg failed"):
        bench.side_leg("long", args)
    # The side legs are started in main() before torch is imported there.
    src = open(os.path.join(ROOT, "bench.py")).read()
    body = src[src.index("\ndef main():"):]
    assert body.index("side_leg(w2, args)") < body.index("import torch")
