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

Copy-on-write sharing ("vLLM Architecture, Memory and Benchmarks Deep Dive",
section 2, the "Copy-on-Write (CoW) Branching" item: rollouts forked from one
prompt share its physical blocks, and a block is duplicated only when the
rollouts diverge). Readings where the page leaves the mechanics open:
* Every physical block carries a count of the block tables that hold it. A
  fork gives the child a copy of the parent's table and length and raises the
  count of each of those blocks; nothing is copied at fork time.
* Sequences only grow, so a shared block that is full is never written again
  and stays shared. The one block a sequence writes into is its last one while
  it has free slots: an append into a last block that is shared and not full
  first takes a fresh block (from the front of the free queue, before any
  blocks for the growth), records the copy (old block -> fresh block), drops
  one count from the old block and puts the fresh block in its place. The last
  holder of a block (count 1) writes in place.
* Releasing a sequence drops one count from each of its blocks; blocks whose
  count reaches zero go to the back of the free queue, in the sequence's
  logical order.
* The recorded copies are taken by the caller once per step and applied to the
  cache pools before that step's writes; the copy itself is the bitwise block
  copy in ``attention.copy_blocks``.

Swapping to host memory ("Inside vLLM: Anatomy of a High-Throughput LLM
Inference System", section "Memory-Efficient KV Cache Storage": blocks move
between GPU and CPU memory, and when GPU memory runs short some blocks are
paged out to host memory; its "How It Works" list: paged attention swaps
blocks in and out as needed; "The Scheduler: Dynamic Batching & Resource
Allocation": under memory pressure low-priority requests are suspended).
Readings where the page leaves the mechanics open:
* A second, host-side pool of blocks with its own first-in first-out free
  queue (identity order unless given).
* The unit of a swap is a whole sequence (a suspended request). Swapping out
  takes one host block per device block of the sequence, from the front of
  the host queue, in logical order, and returns the (device block, host
  block) copies to make; then each device block drops one holder count and
  the blocks no one else holds go to the back of the device queue in logical
  order, exactly as in a release. A block shared with another sequence stays
  on the device for that sequence; the swapped sequence takes its own copy.
* Swapping in takes one device block per host block from the front of the
  device queue, in logical order, returns the (host block, device block)
  copies, and puts the host blocks at the back of the host queue in logical
  order. Sharing lost at swap-out is not restored.
* Either direction is all or nothing: too few free blocks on the receiving
  side raises the out-of-blocks error and changes nothing.
* A swapped-out sequence keeps its length; it cannot be appended to, forked
  or exported to a block table until it is swapped back in; releasing it
  returns its host blocks to the back of the host queue.
* Copies are applied by the caller: the copy-on-write copies taken before a
  swap-out are applied before its copies (they may fill the blocks it
  reads); the swap copies are the bitwise block copy between pools in
  ``attention.swap_blocks``.
"""

from collections import deque


class OutOfBlocks(Exception):
    """Raised when a request needs more free blocks than the pool holds."""


class BlockAllocatorModel:
    """Free-block queue plus one growing block table per sequence."""

    def __init__(self, num_blocks, block_size, initial_order=None, num_host_blocks=0,
                 host_initial_order=None):
        if initial_order is None:
            initial_order = range(num_blocks)
        order = [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of 0..num_blocks-1")
        if host_initial_order is None:
            host_initial_order = range(num_host_blocks)
        host_order = [int(b) for b in host_initial_order]
        if sorted(host_order) != list(range(num_host_blocks)):
            raise ValueError("host_initial_order must be a permutation of 0..num_host_blocks-1")
        self.num_host_blocks = int(num_host_blocks)
        self.host_free = deque(host_order)
        self.host_tables = {}  # swapped-out seq_id -> host block ids, logical order
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        self.free_blocks = deque(order)
        self.tables = {}   # seq_id -> list of physical block ids, logical order
        self.lengths = {}  # seq_id -> tokens held
        self.refs = {}     # physical block -> number of tables holding it
        self.copies = []   # (source block, destination block) not yet taken

    def num_free(self):
        return len(self.free_blocks)

    def fork(self, parent_id, child_id):
        """Start ``child_id`` as a sharer of every block of ``parent_id``."""
        if parent_id not in self.tables:
            raise KeyError(parent_id)
        if child_id in self.tables or child_id in self.host_tables:
            raise ValueError(f"sequence {child_id} already exists")
        self.tables[child_id] = list(self.tables[parent_id])
        self.lengths[child_id] = self.lengths[parent_id]
        for b in self.tables[child_id]:
            self.refs[b] += 1

    def take_copies(self):
        """The block copies recorded since the last call, in order."""
        out, self.copies = self.copies, []
        return out

    def append(self, seq_id, num_tokens):
        """Grow ``seq_id`` by ``num_tokens`` tokens and return their slots.

        A slot is (physical block) * block_size + (offset inside the block),
        the position in the flattened pool where the token's K and V rows live.
        New blocks are taken only when the current last block is full.
        """
        if seq_id in self.host_tables:
            raise ValueError(f"sequence {seq_id} is swapped out")
        held = self.lengths.get(seq_id, 0)
        table = self.tables.get(seq_id, [])
        have = len(table)
        want = -(-(held + num_tokens) // self.block_size)
        # Writing into a shared last block that still has room needs a copy.
        cow = num_tokens > 0 and held % self.block_size != 0 and self.refs[table[-1]] > 1
        if want - have + cow > len(self.free_blocks):
            raise OutOfBlocks(
                f"sequence {seq_id}: needs {want - have + cow} blocks, "
                f"{len(self.free_blocks)} free")
        table = list(table)
        if cow:
            fresh = self.free_blocks.popleft()
            self.copies.append((table[-1], fresh))
            self.refs[table[-1]] -= 1
            self.refs[fresh] = 1
            table[-1] = fresh
        for _ in range(want - have):
            b = self.free_blocks.popleft()
            self.refs[b] = 1
            table.append(b)
        self.tables[seq_id] = table
        self.lengths[seq_id] = held + num_tokens
        slots = []
        for pos in range(held, held + num_tokens):
            slots.append(table[pos // self.block_size] * self.block_size + pos % self.block_size)
        return slots

    def free(self, seq_id):
        """Release ``seq_id``: its blocks that no other table holds go to the
        back of the free queue (in logical order); a swapped-out sequence's
        host blocks go to the back of the host queue."""
        if seq_id in self.host_tables:
            self.host_free.extend(self.host_tables.pop(seq_id))
            del self.lengths[seq_id]
            return
        if seq_id not in self.tables:
            raise KeyError(seq_id)
        self._release(self.tables.pop(seq_id))
        del self.lengths[seq_id]

    def _release(self, table):
        """Drop one holder count from each block of ``table``; blocks no
        table holds any more go to the back of the free queue, in order."""
        for b in table:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                del self.refs[b]
                self.free_blocks.append(b)

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

    def num_free_host(self):
        return len(self.host_free)

    def swap_out(self, seq_id):
        """Move ``seq_id`` to host blocks; returns the (device block, host
        block) copies to make, in logical order."""
        if seq_id not in self.tables:
            raise KeyError(seq_id)
        table = self.tables[seq_id]
        if len(table) > len(self.host_free):
            raise OutOfBlocks(f"sequence {seq_id}: needs {len(table)} host blocks, "
                              f"{len(self.host_free)} free")
        host = [self.host_free.popleft() for _ in table]
        pairs = list(zip(table, host))
        self._release(self.tables.pop(seq_id))
        self.host_tables[seq_id] = host
        return pairs

    def swap_in(self, seq_id):
        """Bring ``seq_id`` back to device blocks; returns the (host block,
        device block) copies to make, in logical order."""
        if seq_id not in self.host_tables:
            raise KeyError(seq_id)
        host = self.host_tables[seq_id]
        if len(host) > len(self.free_blocks):
            raise OutOfBlocks(f"sequence {seq_id}: needs {len(host)} blocks, "
                              f"{len(self.free_blocks)} free")
        table = [self.free_blocks.popleft() for _ in host]
        for b in table:
            self.refs[b] = 1
        pairs = list(zip(host, table))
        self.host_free.extend(self.host_tables.pop(seq_id))
        self.tables[seq_id] = table
        return pairs
