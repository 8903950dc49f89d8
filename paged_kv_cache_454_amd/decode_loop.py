"""Iteration-level decode loop over the library ("vLLM Architecture, Memory
and Benchmarks Deep Dive", section 3 "Continuous Batching": every iteration
each running sequence produces its next token; a finished sequence leaves at
once and a waiting request takes its place, instead of the batch waiting for
its slowest member; section 2: blocks are handed out as tokens arrive).

A fixed number of batch slots each hold one running request or nothing.
One step:
  * host: one native call (``BlockAllocator.step``) appends a token to every
    running request and exports their block-table rows and context lengths;
    idle slots get length 0 (the new token's slot is the last position's,
    which the device call reads from the table);
  * device, for every layer: one ``pa_decode_step`` call, which writes the
    step's new K/V rows at each request's newest position and runs the split
    decode and the log-sum-exp merge (two launches). The first layer's call
    deals the batch's work to the compute units and stores that plan; the
    other layers read it (the same lengths and tables serve every layer);
  * host: requests that reached their length release their blocks.
Admitting a request allocates its prompt and writes the prompt's K/V rows
for every layer (eager launches).

All device buffers of a step (queries, new K/V rows, tables, lengths,
partition workspace, plan, outputs) live at fixed addresses, and the kernels take
the batch composition from device memory (idle rows are empty contexts and
skipped slots), so the device part of a step can be captured once as a HIP
graph and replayed: each step then costs one native allocator call, two
host-to-device copies and one graph launch. The plan is refreshed by the
first layer of every step, eager or replayed, so it never outlives the batch
it was made for.

This is host orchestration only; every step of the attention path runs in
the library's kernels.
"""

import math

import numpy as np
import torch

from .binding import BlockAllocator, decode_plan_buffer, pa_decode_step, pa_reshape_and_cache

# Plan epoch of the loop's launches; the first layer of a step adds bit 31
# (plan afresh and store), the others read that plan.
_EPOCH = 1
_REFRESH = 0x80000000


class DecodeLoop:
    def __init__(self, *, slots, num_blocks, block_size, layers, num_q_heads, num_kv_heads,
                 head_dim, partition_size, max_context, device, use_graph=False):
        self.slots = int(slots)
        self.block_size = int(block_size)
        self.layers = int(layers)
        self.hq, self.hkv, self.d = int(num_q_heads), int(num_kv_heads), int(head_dim)
        self.partition_size = int(partition_size)
        self.max_context = int(max_context)
        self.max_blocks = -(-self.max_context // self.block_size)
        self.max_parts = max(1, -(-self.max_context // self.partition_size))
        self.dev = torch.device(device)
        self.use_graph = bool(use_graph)
        self.alloc = BlockAllocator(num_blocks, block_size)
        bf = torch.bfloat16
        shape = (num_blocks, self.hkv, self.block_size, self.d)
        self.pools = [(torch.zeros(shape, dtype=bf, device=self.dev),
                       torch.zeros(shape, dtype=bf, device=self.dev)) for _ in range(self.layers)]
        S, L = self.slots, self.layers
        # Inputs of a step (written by the caller, or left as they are).
        self.query = torch.zeros((L, S, self.hq, self.d), dtype=bf, device=self.dev)
        self.new_k = torch.zeros((L, S, self.hkv, self.d), dtype=bf, device=self.dev)
        self.new_v = torch.zeros((L, S, self.hkv, self.d), dtype=bf, device=self.dev)
        # Batch description, host (pinned) and device.
        self.h_table = torch.full((S, self.max_blocks), -1, dtype=torch.int32).pin_memory()
        self.h_lens = torch.zeros((S,), dtype=torch.int32).pin_memory()
        self.d_table = torch.full((S, self.max_blocks), -1, dtype=torch.int32, device=self.dev)
        self.d_lens = torch.zeros((S,), dtype=torch.int32, device=self.dev)
        # Partition workspace (shared by the layers, which run in order) and outputs.
        self.part_out = torch.empty((S, self.hq, self.max_parts, self.d), dtype=torch.float32,
                                    device=self.dev)
        self.part_max = torch.empty((S, self.hq, self.max_parts), dtype=torch.float32,
                                    device=self.dev)
        self.part_sum = torch.empty_like(self.part_max)
        self.out = torch.empty((L, S, self.hq, self.d), dtype=torch.float32, device=self.dev)
        self.plan = decode_plan_buffer(self.dev)
        self.scale = 1.0 / math.sqrt(self.d)
        # slot -> [seq_id, tokens still to generate]
        self.running = [None] * S
        self._graph = None
        self._copied = None   # event after the last host-to-device copies
        self.generated = 0

    # ---------------------------------------------------------------- requests
    def free_slots(self):
        return [i for i, r in enumerate(self.running) if r is None]

    def admit(self, slot, seq_id, prompt_len, gen_len, prompt_k=None, prompt_v=None):
        """Start request seq_id in an idle slot: allocate its prompt and write
        the prompt's K/V rows into every layer's pools (prompt_k/v: device
        BF16 [layers][prompt_len][H_KV][d]; zeros of that shape when None).
        Returns the prompt's slots (host int64)."""
        if self.running[slot] is not None:
            raise ValueError(f"slot {slot} is busy")
        if prompt_len + gen_len > self.max_context:
            raise ValueError("request longer than max_context")
        slots = self.alloc.append(seq_id, prompt_len)
        if prompt_len > 0:
            sm = torch.from_numpy(slots).to(self.dev)
            if prompt_k is None:
                prompt_k = torch.zeros((self.layers, prompt_len, self.hkv, self.d),
                                       dtype=torch.bfloat16, device=self.dev)
                prompt_v = prompt_k
            for l, (kc, vc) in enumerate(self.pools):
                pa_reshape_and_cache(prompt_k[l], prompt_v[l], kc, vc, sm)
        self.running[slot] = [seq_id, int(gen_len)]
        return slots

    # -------------------------------------------------------------------- step
    def _device_step(self):
        for l, (kc, vc) in enumerate(self.pools):
            pa_decode_step(self.out[l], self.query[l], self.new_k[l], self.new_v[l], kc, vc,
                           self.d_table, self.d_lens, self.scale, self.partition_size,
                           self.part_out, self.part_max, self.part_sum, plan=self.plan,
                           plan_epoch=_EPOCH | (_REFRESH if l == 0 else 0))

    def step(self):
        """One iteration. Returns the (slot, seq_id) pairs that ran; their
        attention outputs are in self.out[:, slot] until the next step."""
        act = [(i, r[0]) for i, r in enumerate(self.running) if r is not None]
        ids = [sid for _, sid in act]
        _, table, lens = self.alloc.step(ids, np.ones(len(ids), dtype=np.int32),
                                             self.max_blocks)
        if self._copied is not None:
            self._copied.synchronize()   # the pinned buffers are free again
        ht, hl = self.h_table.numpy(), self.h_lens.numpy()
        ht.fill(-1)
        hl.fill(0)
        rows = [i for i, _ in act]
        ht[rows] = table
        hl[rows] = lens
        self.d_table.copy_(self.h_table, non_blocking=True)
        self.d_lens.copy_(self.h_lens, non_blocking=True)
        self._copied = torch.cuda.Event()
        self._copied.record()
        if self.use_graph and self._graph is not None:
            self._graph.replay()
        else:
            self._device_step()
            if self.use_graph:
                # Capture the device part once (the capture runs nothing);
                # later steps replay it with their own batch in the buffers.
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self._device_step()
                self._graph = g
        self.generated += len(act)
        for i, sid in act:
            r = self.running[i]
            r[1] -= 1
        return act

    def finish_done(self):
        """Release the requests that have produced all their tokens; returns
        their (slot, seq_id). Call after the step's outputs are consumed."""
        done = []
        for i, r in enumerate(self.running):
            if r is not None and r[1] <= 0:
                self.alloc.free(r[0])
                self.running[i] = None
                done.append((i, r[0]))
        return done

    def close(self):
        self._graph = None
        self.alloc.close()
