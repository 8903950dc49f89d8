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
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // free queue storage, capacity num_blocks
  int64_t head = 0;           // index of the front element
  int64_t count = 0;          // elements in the queue
  std::vector<int32_t> refs;  // tables holding each block (0 = free)
  std::vector<int32_t> copies;  // pending (source, destination) pairs, flattened
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop_front() {
    int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --count;
    return b;
  }
  void push_back(int32_t b) {
    ring[(head + count) % num_blocks] = b;
    ++count;
  }
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
    a->ring.resize(num_blocks);
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
      a->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
  }
  a->head = 0;
  a->count = num_blocks;
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
  const int64_t held = it == a->seqs.end() ? 0 : it->second.len;
  const int64_t have = it == a->seqs.end() ? 0 : (int64_t)it->second.blocks.size();
  const int64_t want = (held + num_tokens + a->block_size - 1) / a->block_size;
  // Writing into a shared last block that still has room needs a copy.
  const bool cow = num_tokens > 0 && held % a->block_size != 0 &&
                   a->refs[it->second.blocks.back()] > 1;
  if (want - have + cow > a->count)
    return pa::fail(PA_ENOMEM, "pa_alloc_append: sequence %lld needs %lld blocks, %lld free",
                    (long long)seq_id, (long long)(want - have + cow), (long long)a->count);
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
  for (int32_t b : it->second.blocks)
    if (--a->refs[b] == 0) a->push_back(b);
  a->seqs.erase(it);
  return PA_OK;
}

extern "C" pa_status pa_alloc_fork(pa_alloc *a, int64_t parent_id, int64_t child_id) {
  pa::clear_error();
  if (!a) return pa::fail(PA_EINVAL, "pa_alloc_fork: allocator is NULL");
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ENOTFOUND, "pa_alloc_fork: unknown sequence %lld", (long long)parent_id);
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

extern "C" int32_t pa_alloc_num_free(const pa_alloc *a) { return a ? (int32_t)a->count : -1; }

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
  if (need > a->count)
    return pa::fail(PA_ENOMEM, "pa_alloc_step: the step needs %lld blocks, %lld free",
                    (long long)need, (long long)a->count);
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
