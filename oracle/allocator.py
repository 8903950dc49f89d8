"""Model of the on-demand block allocator (oracle; test infrastructure only).

What it follows:
* "vLLM Architecture, Memory and Benchmarks Deep Dive", section 2: the cache
  is cut into fixed-size physical blocks, a block table maps each sequence's
  logical positions to physical blocks, and blocks are handed out only when
  tokens arrive, so only a sequence's last block can hold unused slots.
* Same page, section 3: when a sequence finishes, its blocks go straight back
  to the pool for a waiting request.
* "Inside vLLM: Anatomy of a High-Throughput LLM Inference System", section
  "Garbage Collection & Reuse": free blocks sit in a double-ended queue, are
  taken from its front, and released blocks are appended at its back (first
  in, first out). The same page's "Memory-Efficient KV Cache Storage" snippet
  raises an error when a request does not fit instead of returning partial
  space; the model does the same and leaves its state untouched.

Readings where the pages leave a step open (also listed in the design notes):
* The page's snippet replaces a sequence's table when it asks for more blocks;
  here a sequence's table only grows (its earlier tokens stay where they are).
* The page's snippet calls an undefined helper when the queue is empty; here an
  empty queue is an out-of-blocks error.
* The initial order of the free queue is an input (identity by default), so a
  seeded scatter of physical blocks is passed in, never drawn here.
"""

from collections import deque


class OutOfBlocks(Exception):
    """Raised when a request needs more free blocks than the pool holds."""


class BlockAllocatorModel:
    """Free-block queue plus one growing block table per sequence."""

    def __init__(self, num_blocks, block_size, initial_order=None):
        if initial_order is None:
            initial_order = range(num_blocks)
        order = [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of 0..num_blocks-1")
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        self.free_blocks = deque(order)
        self.tables = {}   # seq_id -> list of physical block ids, logical order
        self.lengths = {}  # seq_id -> tokens held

    def num_free(self):
        return len(self.free_blocks)

    def append(self, seq_id, num_tokens):
        """Grow ``seq_id`` by ``num_tokens`` tokens and return their slots.

        A slot is (physical block) * block_size + (offset inside the block),
        the position in the flattened pool where the token's K and V rows live.
        New blocks are taken only when the current last block is full.
        """
        held = self.lengths.get(seq_id, 0)
        table = self.tables.get(seq_id, [])
        have = len(table)
        want = -(-(held + num_tokens) // self.block_size)
        if want - have > len(self.free_blocks):
            raise OutOfBlocks(
                f"sequence {seq_id}: needs {want - have} blocks, {len(self.free_blocks)} free")
        table = list(table)
        for _ in range(want - have):
            table.append(self.free_blocks.popleft())
        self.tables[seq_id] = table
        self.lengths[seq_id] = held + num_tokens
        slots = []
        for pos in range(held, held + num_tokens):
            slots.append(table[pos // self.block_size] * self.block_size + pos % self.block_size)
        return slots

    def free(self, seq_id):
        """Return every block of ``seq_id`` to the back of the free queue."""
        if seq_id not in self.tables:
            raise KeyError(seq_id)
        self.free_blocks.extend(self.tables.pop(seq_id))
        del self.lengths[seq_id]

    def block_table(self, seq_ids, max_blocks, pad=-1):
        """Rows of the block table for ``seq_ids``, padded with ``pad``, and
        the matching context lengths."""
        rows, lens = [], []
        for sid in seq_ids:
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise ValueError(f"sequence {sid} holds {len(t)} blocks > {max_blocks}")
            rows.append(list(t) + [pad] * (max_blocks - len(t)))
            lens.append(self.lengths[sid])
        return rows, lens
