"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that at least one pin catches each. This shows the pins constrain every part
of the oracle: a dropped term, a wrong sign or index, a swapped operand."""

import importlib.util
import os
import types

import pytest

from tests import oracle_pins as P

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTATIONS = [
    # (module, original text, planted mistake)
    ("attention", "return h // (num_q_heads // num_kv_heads)", "return h % num_kv_heads"),
    ("attention", "phys = int(block_table_row[t // block_size])",
     "phys = int(block_table_row[t % block_size])"),
    ("attention", "out[t] = cache[phys, :, t % block_size, :]",
     "out[t] = cache[phys, :, t // block_size % cache.shape[2], :]"),
    ("attention", "z = scale * (K @ q)", "z = K @ q"),
    ("attention", "return (w @ V) / total, zmax + np.log(total)",
     "return (w @ V), zmax + np.log(total)"),
    ("attention", "return (w @ V) / total, zmax + np.log(total)",
     "return (w @ V) / total, np.log(total)"),
    ("attention", "w = np.exp(z - zmax)", "w = np.exp(zmax - z)"),
    ("attention", "T = int(context_lens[s])\n        if T == 0:\n            continue\n        K = gather_context(key_cache, block_tables[s], T, block_size)\n        V = gather_context(value_cache, block_tables[s], T, block_size)\n        for h in range(num_q_heads):",
     "T = int(context_lens[s]) - 1\n        if T <= 0:\n            continue\n        K = gather_context(key_cache, block_tables[s], T, block_size)\n        V = gather_context(value_cache, block_tables[s], T, block_size)\n        for h in range(num_q_heads):"),
    ("attention", "lo, hi = p * partition_size, min(T, (p + 1) * partition_size)",
     "lo, hi = p * partition_size, min(T, (p + 1) * partition_size - 1)"),
    ("attention", "out[s, h] = (np.exp(l - total)[:, None] * o[s, h, :n]).sum(axis=0)",
     "out[s, h] = (np.exp(l - top)[:, None] * o[s, h, :n]).sum(axis=0)"),
    ("attention", "visible = T - n + j + 1", "visible = T - n + j"),
    ("attention", "visible = T - n + j + 1", "visible = T"),
    ("attention", "blk, off = slot // block_size, slot % block_size",
     "off, blk = slot // block_size, slot % block_size"),
    ("attention", "kc[blk, :, off, :] = key[i]", "kc[blk, :, off, :] = value[i]"),
    ("accounting", "return 2 * num_layers * num_kv_heads", "return num_layers * num_kv_heads"),
    ("accounting", "return -(-num_tokens // block_size)", "return num_tokens // block_size"),
    ("accounting", "reserved = len(token_counts) * max_len", "reserved = sum(token_counts)"),
    ("allocator", "            b = self.free_blocks.popleft()",
     "            b = self.free_blocks.pop()"),
    ("allocator", "            fresh = self.free_blocks.popleft()",
     "            fresh = self.free_blocks.pop()"),
    ("allocator", "                self.free_blocks.append(b)",
     "                self.free_blocks.appendleft(b)"),
    ("allocator", "self.refs[table[-1]] > 1", "self.refs[table[-1]] > 0"),
    ("allocator", "self.refs[table[-1]] > 1", "self.refs[table[-1]] > 2"),
    ("allocator", "self.copies.append((table[-1], fresh))", "self.copies.append((fresh, table[-1]))"),
    ("allocator", "            self.refs[table[-1]] -= 1\n", "\n"),
    ("allocator", "            if self.refs[b] == 0:", "            if self.refs[b] <= 1:"),
    ("allocator", "            self.refs[b] += 1", "            self.refs[b] += 0"),
    ("allocator", "cow = num_tokens > 0 and held % self.block_size != 0",
     "cow = num_tokens > 0"),
    ("attention", "        kc[dst] = key_cache[src]", "        kc[src] = key_cache[dst]"),
    ("attention", "        vc[dst] = value_cache[src]", "        vc[dst] = key_cache[src]"),
    ("allocator", "if want - have + cow > len(self.free_blocks):",
     "if want - have + cow > len(self.free_blocks) + 1:"),
    ("allocator", "if want - have + cow > len(self.free_blocks):",
     "if want - have > len(self.free_blocks):"),
    ("allocator", "want = -(-(held + num_tokens) // self.block_size)",
     "want = (held + num_tokens) // self.block_size + 1"),
]

MUTATIONS += [
    ("fp8", "val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))",
     "val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 8))"),
    ("fp8", "            m = int(np.rint(a / 2.0 ** -9))     # exact quotient, ties to even",
     "            m = int(np.floor(a / 2.0 ** -9))"),
    ("fp8", "        m = int(np.rint((a / 2.0 ** e - 1.0) * 8.0))",
     "        m = int(np.floor((a / 2.0 ** e - 1.0) * 8.0 + 0.5))"),
    ("fp8", "        if a >= E4M3_MAX:\n            flat_o[i] = s | 0x7E",
     "        if a >= E4M3_MAX:\n            flat_o[i] = s | 0x7F"),
    ("fp8", "        flat_o[i] = s | ((e + 7) << 3) | m", "        flat_o[i] = s | ((e + 7) << 3) | (m ^ 1)"),
    ("fp8", "    q = np.asarray(x, dtype=np.float32) / np.float32(scale)",
     "    q = np.asarray(x, dtype=np.float32) * np.float32(scale)"),
    ("fp8", "    return decode_e4m3(codes) * float(np.float32(scale))",
     "    return decode_e4m3(codes)"),
    ("fp8", "        s = 0x80 if np.signbit(x) else 0", "        s = 0x80 if x < 0 else 0"),
    ("fp8", "    return np.ascontiguousarray(np.swapaxes(value_codes, 2, 3))",
     "    return np.ascontiguousarray(value_codes)"),
    ("fp8", "    return kc, value_pool(vr)", "    return kc, vr"),
]

MUTATIONS += [
    ("allocator", "        host = [self.host_free.popleft() for _ in table]",
     "        host = [self.host_free.pop() for _ in table]"),
    ("allocator", "        table = [self.free_blocks.popleft() for _ in host]",
     "        table = [self.free_blocks.pop() for _ in host]"),
    ("allocator", "        pairs = list(zip(table, host))", "        pairs = list(zip(host, table))"),
    ("allocator", "        pairs = list(zip(host, table))", "        pairs = list(zip(table, host))"),
    ("allocator", "        if len(table) > len(self.host_free):",
     "        if len(table) > len(self.host_free) + 1:"),
    ("allocator", "        if len(host) > len(self.free_blocks):",
     "        if len(host) - 1 > len(self.free_blocks):"),
    ("allocator", "        self.host_free.extend(self.host_tables.pop(seq_id))\n        self.tables[seq_id] = table",
     "        self.host_tables.pop(seq_id)\n        self.tables[seq_id] = table"),
    ("allocator", "        self._release(self.tables.pop(seq_id))\n        self.host_tables[seq_id] = host",
     "        self.free_blocks.extend(self.tables.pop(seq_id))\n        self.host_tables[seq_id] = host"),
    ("attention", "        kd[dst] = src_key[src]", "        kd[dst] = src_key[dst % ns]"),
    ("attention", "        vd[dst] = src_value[src]", "        vd[dst] = src_key[src]"),
    ("attention", "        if not (0 <= src < ns and 0 <= dst < nd):\n            continue\n        kd[dst]",
     "        if not (0 <= src < nd and 0 <= dst < ns):\n            continue\n        kd[dst]"),
]

MUTATIONS += [
    # split-context decode over FP8 pools: the value pool read untransposed,
    # and the key and value scales exchanged
    ("fp8", "dequantize(key_codes, k_scale),\n                                       dequantize(value_rows(value_codes), v_scale), block_tables,\n                                       context_lens, block_size, scale, partition_size,",
     "dequantize(key_codes, k_scale),\n                                       dequantize(value_codes, v_scale), block_tables,\n                                       context_lens, block_size, scale, partition_size,"),
    ("fp8", "dequantize(key_codes, k_scale),\n                                       dequantize(value_rows(value_codes), v_scale), block_tables,\n                                       context_lens, block_size, scale, partition_size,",
     "dequantize(key_codes, v_scale),\n                                       dequantize(value_rows(value_codes), k_scale), block_tables,\n                                       context_lens, block_size, scale, partition_size,"),
    # exported block-table rows: padding and lengths
    ("allocator", "def block_table(self, seq_ids, max_blocks, pad=-1):",
     "def block_table(self, seq_ids, max_blocks, pad=0):"),
    ("allocator", "            lens.append(self.lengths[sid])",
     "            lens.append(len(t) * self.block_size)"),
]

PINS = {"attention": P.ATTENTION_PINS, "accounting": P.ACCOUNTING_PINS,
        "allocator": P.ALLOCATOR_PINS, "fp8": P.FP8_PINS}


def _mutant(modname, old, new):
    path = os.path.join(ORACLE_DIR, modname + ".py")
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique in {modname}: {old!r}"
    mod = types.ModuleType("mutant_" + modname)
    mod.__package__ = "oracle"   # relative imports resolve to the real oracle modules
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("modname,old,new", MUTATIONS,
                         ids=[f"{m}:{n[:40]}" for m, _, n in MUTATIONS])
def test_some_pin_catches_planted_mistake(modname, old, new):
    mod = _mutant(modname, old, new)
    caught = []
    for pin in PINS[modname]:
        try:
            pin(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {new!r}"


def test_unmutated_copies_pass_every_pin():
    for modname, pins in PINS.items():
        mod = importlib.import_module("oracle." + modname)
        for pin in pins:
            pin(mod)
