// The decode step's own K/V write (device code, not installed): the step's
// token of sequence s is position T_s - 1 ("vLLM Architecture, Memory and
// Benchmarks Deep Dive", s.1: the new token's K/V join the cache before it
// attends), so its rows go to slot table[s][(T_s - 1) / bs] * bs +
// (T_s - 1) % bs. One wavefront moves one (sequence, KV head): the K row's
// 16-byte pieces, then the V row's, over the 64 lanes. A block id outside
// the pool, T_s = 0 or T_s past the table's capacity writes nothing, as the
// slot write skips a slot outside the pool.
#pragma once

#include "launch.h"

namespace pa {

// Rows of up to 1 KiB each (head_dim 256 in fp32): at most two pieces per
// lane.
constexpr int kAppendPieces = 2;

struct AppendLoad {
  uint4 v[kAppendPieces];
  int blk;    // block id (VGPR, pending load)
  int T;      // context length, uniform
  int pieces; // 16-byte pieces per row
};

// Issue the loads of (s, h)'s rows and of the block id holding T - 1.
__device__ inline AppendLoad append_issue(const AppendArgs &a, int s, int h, int T, int lane) {
  AppendLoad r;
  r.T = T;
  r.pieces = a.row_bytes / 16;
  const int cap = a.max_blocks_per_seq * a.block_size;
  const bool ok = T > 0 && T <= cap;
  r.blk = ok ? a.block_tables[(int64_t)s * a.max_blocks_per_seq + (T - 1) / a.block_size] : -1;
  const int64_t row = ((int64_t)s * a.num_kv_heads + h) * a.row_bytes;
#pragma unroll
  for (int i = 0; i < kAppendPieces; ++i) {
    const int q = lane + 64 * i;  // piece q of [K row | V row]
    r.v[i] = make_uint4(0, 0, 0, 0);
    if (ok && q < 2 * r.pieces) {
      const uint8_t *src = reinterpret_cast<const uint8_t *>(q < r.pieces ? a.new_key : a.new_value);
      r.v[i] = *reinterpret_cast<const uint4 *>(src + row + 16 * (q % r.pieces));
    }
  }
  return r;
}

// Store the rows loaded by append_issue into their slot.
__device__ inline void append_commit(const AppendArgs &a, const AppendLoad &r, int h, int lane) {
  const int blk = r.blk;
  if (r.T <= 0 || blk < 0 || blk >= a.num_blocks) return;
  const int t = r.T - 1;
  const int64_t dst = (((int64_t)blk * a.num_kv_heads + h) * a.block_size + t % a.block_size) *
                      a.row_bytes;
#pragma unroll
  for (int i = 0; i < kAppendPieces; ++i) {
    const int q = lane + 64 * i;
    if (q < 2 * r.pieces) {
      uint8_t *pool = reinterpret_cast<uint8_t *>(q < r.pieces ? a.key_cache : a.value_cache);
      *reinterpret_cast<uint4 *>(pool + dst + 16 * (q % r.pieces)) = r.v[i];
    }
  }
}

}  // namespace pa
