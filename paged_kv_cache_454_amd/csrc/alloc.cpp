// Host block allocator: on-demand blocks from a first-in first-out free
// queue, one growing block table per sequence.
//
// "vLLM Architecture, Memory and Benchmarks Deep Dive", section 2: blocks are
// handed out only when tokens arrive, so only a sequence's last block holds
// unused slots; section 3: a finished sequence's blocks return to the pool
// at once. "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
// "Garbage Collection & Reuse": free blocks are taken from the front of a
// double-ended queue and released blocks go to its back.
//
// The queue is a ring buffer of block ids (capacity = pool size), so taking
// and returning blocks is O(1) per block with no allocation on the hot path;
// sequences live in a hash map keyed by their 64-bit id.
//
// Copy-on-write sharing ("vLLM Architecture, Memory and Benchmarks Deep
// Dive", section 2, "Copy-on-Write (CoW) Branching": forked rollouts share
// the prompt's blocks, which are cloned only when the rollouts diverge).
// Every block carries the number of tables that hold it. A fork copies the
// parent's table and raises those counts; an append into a last block that is
// shared and not yet full first takes a fresh block from the front of the
// queue, records the pending copy (old -> fresh) and swaps it in; a release
// returns only the blocks whose count drops to zero. Full shared blocks are
// never written again (sequences only grow), so they stay shared.
//
// Swapping to host memory ("Inside vLLM: Anatomy of a High-Throughput LLM
// Inference System", "Memory-Efficient KV Cache Storage": when GPU memory runs
// short, blocks are paged out to host memory and later brought back). A
// second ring holds the free blocks of a host pool. A swap moves a whole
// sequence: swap-out takes one host block per device block from the front of
// the host queue and releases the device blocks as a free would (blocks
// another table holds stay); swap-in takes one device block per host block
// from the front of the device queue and returns the host blocks to the back
// of theirs. Both are all or nothing and hand back the block moves the
// caller applies with pa_swap_blocks. While swapped out a sequence keeps its
// length but cannot grow, fork or be exported to a block table.
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

// A first-in first-out queue of block ids in a ring of fixed capacity.
struct BlockRing {
  std::vector<int32_t> ring;
  int64_t head = 0;   // index of the front element
  int64_t count = 0;  // elements in the queue

  int32_t pop_front() {
    int32_t b = ring[head];
    head = (head + 1) % (int64_t)ring.size();
    --count;
    return b;
  }
  void push_back(int32_t b) {
    ring[(head + count) % (int64_t)ring.size()] = b;
    ++count;
  }
};

struct pa_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  BlockRing free;             // device blocks, capacity num_blocks
  std::vector<int32_t> refs;  // tables holding each block (0 = free)
  std::vector<int32_t> copies;  // pending (source, destination) pairs, flattened
  int32_t num_host_blocks = 0;
  BlockRing host_free;        // host pool blocks, capacity num_host_blocks
  int64_t num_swapped = 0;    // sequences currently on host blocks
  struct Seq {
    std::vector<int32_t> blocks;  // device block ids, or host block ids while swapped
    int64_t len = 0;
    bool swapped = false;
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop_front() { return free.pop_front(); }
  void push_back(int32_t b) { free.push_back(b); }
  int64_t count() const { return free.count; }
};

extern "C" pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                                     const int32_t *initial_order, pa_alloc **out) {
  pa::clear_error();
  if (!out) return pa::fail(PA_EINVAL, "pa_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_EINVAL, "pa_alloc_create: num_blocks=%d block_size=%d must be > 0",
                    num_blocks, block_size);
  pa_alloc *a = new (std::nothrow) pa_alloc();
  if (!a) return pa::fail(PA_ENOMEM, "pa_alloc_create: host allocation failed");
  try {
    a->free.ring.resize(num_blocks);
    a->refs.assign(num_blocks, 0);
  } catch (...) {
    delete a;
    return pa::fail(PA_ENOMEM, "pa_alloc_create: host allocation failed");
  }
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  if (initial_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return pa::fail(PA_EINVAL,
                        "pa_alloc_create: initial_order is not a permutation (entry %d = %d)",
                        i, b);
      }
      seen[b] = 1;
      a->free.ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free.ring[i] = i;
  }
  a->free.head = 0;
  a->free.count = num_blocks;
  *out = a;
  return PA_OK;
}

extern "C" void pa_alloc_destroy(pa_alloc *a) { delete a; }

extern "C" pa_status pa_alloc_append(pa_alloc *a, int64_t seq_id, int32_t num_tokens,
                                     int64_t *slots_out) {
  pa::clear_error();
  if (!a) return pa::fail(PA_EINVAL, "pa_alloc_append: allocator is NULL");
  if (num_tokens < 0) return pa::fail(PA_EINVAL, "pa_alloc_append: num_tokens=%d", num_tokens);
  auto it = a->seqs.find(seq_id);
  if (it != a->seqs.end() && it->second.swapped)
    return pa::fail(PA_EINVAL, "pa_alloc_append: sequence %lld is swapped out", (long long)seq_id);
  const int64_t held = it == a->seqs.end() ? 0 : it->second.len;
  const int64_t have = it == a->seqs.end() ? 0 : (int64_t)it->second.blocks.size();
  const int64_t want = (held + num_tokens + a->block_size - 1) / a->block_size;
  // Writing into a shared last block that still has room needs a copy.
  const bool cow = num_tokens > 0 && held % a->block_size != 0 &&
                   a->refs[it->second.blocks.back()] > 1;
  if (want - have + cow > a->count())
    return pa::fail(PA_ENOMEM, "pa_alloc_append: sequence %lld needs %lld blocks, %lld free",
                    (long long)seq_id, (long long)(want - have + cow), (long long)a->count());
  pa_alloc::Seq *s;
  try {
    s = &a->seqs[seq_id];
    s->blocks.reserve(want);
    if (cow) a->copies.reserve(a->copies.size() + 2);
  } catch (...) {
    if (it == a->seqs.end()) a->seqs.erase(seq_id);
    return pa::fail(PA_ENOMEM, "pa_alloc_append: host allocation failed");
  }
  if (cow) {
    const int32_t old = s->blocks.back(), fresh = a->pop_front();
    a->copies.push_back(old);
    a->copies.push_back(fresh);
    --a->refs[old];
    a->refs[fresh] = 1;
    s->blocks.back() = fresh;
  }
  for (int64_t i = have; i < want; ++i) {
    const int32_t b = a->pop_front();
    a->refs[b] = 1;
    s->blocks.push_back(b);
  }
  if (slots_out) {
    for (int32_t i = 0; i < num_tokens; ++i) {
      const int64_t pos = held + i;
      slots_out[i] = (int64_t)s->blocks[pos / a->block_size] * a->block_size + pos % a->block_size;
    }
  }
  s->len = held + num_tokens;
  return PA_OK;
}

extern "C" pa_status pa_alloc_free(pa_alloc *a, int64_t seq_id) {
  pa::clear_error();
  if (!a) return pa::fail(PA_EINVAL, "pa_alloc_free: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ENOTFOUND, "pa_alloc_free: unknown sequence %lld", (long long)seq_id);
  if (it->second.swapped) {
    for (int32_t h : it->second.blocks) a->host_free.push_back(h);
    --a->num_swapped;
  } else {
    for (int32_t b : it->second.blocks)
      if (--a->refs[b] == 0) a->push_back(b);
  }
  a->seqs.erase(it);
  return PA_OK;
}

extern "C" pa_status pa_alloc_fork(pa_alloc *a, int64_t parent_id, int64_t child_id) {
  pa::clear_error();
  if (!a) return pa::fail(PA_EINVAL, "pa_alloc_fork: allocator is NULL");
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ENOTFOUND, "pa_alloc_fork: unknown sequence %lld", (long long)parent_id);
  if (it->second.swapped)
    return pa::fail(PA_EINVAL, "pa_alloc_fork: sequence %lld is swapped out",
                    (long long)parent_id);
  if (a->seqs.count(child_id))
    return pa::fail(PA_EINVAL, "pa_alloc_fork: sequence %lld already exists",
                    (long long)child_id);
  try {
    pa_alloc::Seq child = it->second;  // copy before the map may rehash
    a->seqs.emplace(child_id, std::move(child));
  } catch (...) {
    return pa::fail(PA_ENOMEM, "pa_alloc_fork: host allocation failed");
  }
  for (int32_t b : a->seqs[child_id].blocks) ++a->refs[b];
  return PA_OK;
}

extern "C" int32_t pa_alloc_take_copies(pa_alloc *a, int32_t *pairs_out, int32_t max_pairs) {
  if (!a || max_pairs < 0 || (max_pairs > 0 && !pairs_out)) return -1;
  const int64_t n = (int64_t)a->copies.size() / 2;
  if (n > max_pairs) return (int32_t)n;  // nothing taken; ask again with room for n
  for (int64_t i = 0; i < 2 * n; ++i) pairs_out[i] = a->copies[i];
  a->copies.clear();
  return (int32_t)n;
}

extern "C" int32_t pa_alloc_block_refs(const pa_alloc *a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refs[block];
}

extern "C" int32_t pa_alloc_num_free(const pa_alloc *a) { return a ? (int32_t)a->count() : -1; }

extern "C" int32_t pa_alloc_seq_len(const pa_alloc *a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : (int32_t)it->second.len;
}

extern "C" pa_status pa_alloc_block_table(const pa_alloc *a, const int64_t *seq_ids, int32_t n,
                                          int32_t max_blocks, int32_t *table_out,
                                          int32_t *lens_out) {
  pa::clear_error();
  if (!a || (n > 0 && (!seq_ids || !table_out)) || n < 0 || max_blocks < 0)
    return pa::fail(PA_EINVAL, "pa_alloc_block_table: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return pa::fail(PA_ENOTFOUND, "pa_alloc_block_table: unknown sequence %lld",
                      (long long)seq_ids[i]);
    if (it->second.swapped)
      return pa::fail(PA_EINVAL, "pa_alloc_block_table: sequence %lld is swapped out",
                      (long long)seq_ids[i]);
    const auto &blocks = it->second.blocks;
    if ((int64_t)blocks.size() > max_blocks)
      return pa::fail(PA_EINVAL, "pa_alloc_block_table: sequence %lld holds %zu blocks > %d",
                      (long long)seq_ids[i], blocks.size(), max_blocks);
    int32_t *row = table_out + (int64_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)blocks.size() ? blocks[j] : -1;
    if (lens_out) lens_out[i] = (int32_t)it->second.len;
  }
  return PA_OK;
}

extern "C" pa_status pa_alloc_step(pa_alloc *a, const int64_t *seq_ids, const int32_t *num_tokens,
                                   int32_t n, int64_t *slots_out, int32_t max_blocks,
                                   int32_t *table_out, int32_t *lens_out) {
  pa::clear_error();
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !num_tokens || !table_out)))
    return pa::fail(PA_EINVAL, "pa_alloc_step: bad arguments");
  // Check the whole step first so that it is all or nothing: blocks needed
  // (growth plus copy-on-write replacements) against the free queue, table
  // widths, and no sequence listed twice.
  int64_t need = 0, total = 0;
  try {
    std::unordered_map<int64_t, int> seen;
    std::unordered_map<int32_t, int> left;  // holders a shared last block loses this step
    seen.reserve((size_t)n * 2);
    for (int32_t i = 0; i < n; ++i) {
      if (num_tokens[i] < 0)
        return pa::fail(PA_EINVAL, "pa_alloc_step: num_tokens[%d]=%d", i, num_tokens[i]);
      if (seen[seq_ids[i]]++)
        return pa::fail(PA_EINVAL, "pa_alloc_step: sequence %lld listed twice",
                        (long long)seq_ids[i]);
      auto it = a->seqs.find(seq_ids[i]);
      if (it != a->seqs.end() && it->second.swapped)
        return pa::fail(PA_EINVAL, "pa_alloc_step: sequence %lld is swapped out",
                        (long long)seq_ids[i]);
      const int64_t held = it == a->seqs.end() ? 0 : it->second.len;
      const int64_t have = it == a->seqs.end() ? 0 : (int64_t)it->second.blocks.size();
      const int64_t want = (held + num_tokens[i] + a->block_size - 1) / a->block_size;
      if (want > max_blocks)
        return pa::fail(PA_EINVAL, "pa_alloc_step: sequence %lld would hold %lld blocks > %d",
                        (long long)seq_ids[i], (long long)want, max_blocks);
      bool cow = false;
      if (num_tokens[i] > 0 && held % a->block_size != 0) {
        const int32_t last = it->second.blocks.back();
        // Earlier sequences of this step that copied away from the same
        // block leave fewer holders; the last one writes in place.
        cow = a->refs[last] - left[last] > 1;
        if (cow) ++left[last];
      }
      need += want - have + cow;
      total += num_tokens[i];
    }
  } catch (...) {
    return pa::fail(PA_ENOMEM, "pa_alloc_step: host allocation failed");
  }
  if (need > a->count())
    return pa::fail(PA_ENOMEM, "pa_alloc_step: the step needs %lld blocks, %lld free",
                    (long long)need, (long long)a->count());
  if (total > 0 && !slots_out) return pa::fail(PA_EINVAL, "pa_alloc_step: slots_out is NULL");
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pa_status st = pa_alloc_append(a, seq_ids[i], num_tokens[i],
                                         num_tokens[i] > 0 ? slots_out + off : nullptr);
    if (st != PA_OK) return st;  // host allocation failure only (capacity was checked)
    off += num_tokens[i];
  }
  return pa_alloc_block_table(a, seq_ids, n, max_blocks, table_out, lens_out);
}

extern "C" pa_status pa_alloc_set_host_pool(pa_alloc *a, int32_t num_host_blocks,
                                            const int32_t *initial_order) {
  pa::clear_error();
  if (!a) return pa::fail(PA_EINVAL, "pa_alloc_set_host_pool: allocator is NULL");
  if (num_host_blocks < 0)
    return pa::fail(PA_EINVAL, "pa_alloc_set_host_pool: num_host_blocks=%d", num_host_blocks);
  if (a->num_swapped > 0)
    return pa::fail(PA_EINVAL, "pa_alloc_set_host_pool: %lld sequences are swapped out",
                    (long long)a->num_swapped);
  BlockRing ring;
  try {
    ring.ring.resize(num_host_blocks);
  } catch (...) {
    return pa::fail(PA_ENOMEM, "pa_alloc_set_host_pool: host allocation failed");
  }
  if (initial_order) {
    std::vector<char> seen;
    try {
      seen.assign(num_host_blocks, 0);
    } catch (...) {
      return pa::fail(PA_ENOMEM, "pa_alloc_set_host_pool: host allocation failed");
    }
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t b = initial_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b])
        return pa::fail(PA_EINVAL,
                        "pa_alloc_set_host_pool: initial_order is not a permutation "
                        "(entry %d = %d)", i, b);
      seen[b] = 1;
      ring.ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_host_blocks; ++i) ring.ring[i] = i;
  }
  ring.count = num_host_blocks;
  a->host_free = std::move(ring);
  a->num_host_blocks = num_host_blocks;
  return PA_OK;
}

extern "C" int32_t pa_alloc_num_free_host(const pa_alloc *a) {
  return a ? (int32_t)a->host_free.count : -1;
}

extern "C" int32_t pa_alloc_is_swapped(const pa_alloc *a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

// Shared checks of the two swap directions: the sequence exists and is on
// the expected side, and pairs_out has room for one pair per block.
static pa_status swap_lookup(pa_alloc *a, const char *fn, int64_t seq_id, bool want_swapped,
                             int32_t max_pairs, int32_t *pairs_out, int32_t *num_pairs,
                             pa_alloc::Seq **seq) {
  if (!a || !num_pairs || max_pairs < 0 || (max_pairs > 0 && !pairs_out))
    return pa::fail(PA_EINVAL, "%s: bad arguments", fn);
  *num_pairs = 0;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ENOTFOUND, "%s: unknown sequence %lld", fn, (long long)seq_id);
  if (it->second.swapped != want_swapped)
    return pa::fail(PA_EINVAL, "%s: sequence %lld is %s", fn, (long long)seq_id,
                    want_swapped ? "not swapped out" : "already swapped out");
  if ((int64_t)it->second.blocks.size() > max_pairs)
    return pa::fail(PA_EINVAL, "%s: sequence %lld holds %zu blocks > max_pairs %d", fn,
                    (long long)seq_id, it->second.blocks.size(), max_pairs);
  *seq = &it->second;
  return PA_OK;
}

extern "C" pa_status pa_alloc_swap_out(pa_alloc *a, int64_t seq_id, int32_t max_pairs,
                                       int32_t *pairs_out, int32_t *num_pairs) {
  pa::clear_error();
  const char *fn = "pa_alloc_swap_out";
  pa_alloc::Seq *s = nullptr;
  pa_status st = swap_lookup(a, fn, seq_id, false, max_pairs, pairs_out, num_pairs, &s);
  if (st != PA_OK) return st;
  const int64_t n = (int64_t)s->blocks.size();
  if (n > a->host_free.count)
    return pa::fail(PA_ENOMEM, "%s: sequence %lld needs %lld host blocks, %lld free", fn,
                    (long long)seq_id, (long long)n, (long long)a->host_free.count);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t dev = s->blocks[i], host = a->host_free.pop_front();
    pairs_out[2 * i] = dev;
    pairs_out[2 * i + 1] = host;
    s->blocks[i] = host;
    if (--a->refs[dev] == 0) a->push_back(dev);
  }
  s->swapped = true;
  ++a->num_swapped;
  *num_pairs = (int32_t)n;
  return PA_OK;
}

extern "C" pa_status pa_alloc_swap_in(pa_alloc *a, int64_t seq_id, int32_t max_pairs,
                                      int32_t *pairs_out, int32_t *num_pairs) {
  pa::clear_error();
  const char *fn = "pa_alloc_swap_in";
  pa_alloc::Seq *s = nullptr;
  pa_status st = swap_lookup(a, fn, seq_id, true, max_pairs, pairs_out, num_pairs, &s);
  if (st != PA_OK) return st;
  const int64_t n = (int64_t)s->blocks.size();
  if (n > a->count())
    return pa::fail(PA_ENOMEM, "%s: sequence %lld needs %lld blocks, %lld free", fn,
                    (long long)seq_id, (long long)n, (long long)a->count());
  for (int64_t i = 0; i < n; ++i) {
    const int32_t host = s->blocks[i], dev = a->pop_front();
    pairs_out[2 * i] = host;
    pairs_out[2 * i + 1] = dev;
    s->blocks[i] = dev;
    a->refs[dev] = 1;
    a->host_free.push_back(host);
  }
  s->swapped = false;
  --a->num_swapped;
  *num_pairs = (int32_t)n;
  return PA_OK;
}
