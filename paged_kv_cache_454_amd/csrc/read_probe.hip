// HBM read probe: the bandwidth ceiling of the access pattern paged decode
// uses. Decode streams its K/V as 8 KiB (block, head) tiles gathered through
// the block table ("vLLM Architecture, Memory and Benchmarks Deep Dive",
// s.1-2: fixed-size blocks, decode bound by memory traffic), so this kernel
// reads whole 8 KiB blocks of a pool in a caller-given order with the same
// loads: non-temporal 16-byte vector loads, 1 KiB per wavefront instruction.
// With the identity order it is a plain streaming read; with a random
// permutation it is the gather pattern of decode without its arithmetic.
//
// Eight wavefronts per workgroup, one workgroup per CU; global wave w reads
// blocks order[w], order[w + W], ... (W = all waves), each through a ring of
// two blocks in flight. Measured on MI355X over random 8 KiB blocks, eight
// waves per CU read 13 % faster than four (with the same or twice the bytes
// in flight), and four blocks in flight per wave are slower than two. Every word read is folded into a per-lane XOR, which
// is stored at the end (the data must be consumed, and the XOR of all sinks
// equals the XOR of all words read, which the tests check).
#include "launch.h"
#include "pa_device.h"
#include "persistent_plan.h"

namespace pa {
namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeBlock = 8192;
typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeWaves * 64) void read_probe_kernel(
    const uint8_t *__restrict__ pool, int64_t pool_blocks, const int32_t *__restrict__ order,
    int32_t num_blocks, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kProbeWaves;
  const int mine = gw < num_blocks ? (num_blocks - gw + nw - 1) / nw : 0;
  probe_u32x4 a[8], b[8];
  uint32_t acc = 0;
  // Block k of this wave, or nothing (zeros) past the end or outside the pool.
  auto issue = [&](probe_u32x4(&r)[8], int k) {
    int64_t blk = -1;
    if (k < mine) blk = order[gw + (int64_t)k * nw];
    const bool ok = blk >= 0 && blk < pool_blocks;
    const probe_u32x4 *src =
        reinterpret_cast<const probe_u32x4 *>(pool + (ok ? blk : 0) * kProbeBlock) + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = ok ? __builtin_nontemporal_load(src + i * 64) : probe_u32x4{0u, 0u, 0u, 0u};
  };
  auto fold = [&](const probe_u32x4(&r)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= r[i][0] ^ r[i][1] ^ r[i][2] ^ r[i][3];
  };
  issue(a, 0);
  issue(b, 1);
  for (int k = 0; k < mine; k += 2) {
    fold(a);
    issue(a, k + 2);
    fold(b);
    issue(b, k + 3);
  }
  sink[(int64_t)gw * 64 + lane] = acc;
}

}  // namespace

int64_t read_probe_sink_words() { return (int64_t)persist::num_cus() * kProbeWaves * 64; }

pa_status launch_read_probe(const void *pool, int64_t pool_bytes, const int32_t *order,
                            int32_t num_blocks, uint32_t *sink, hipStream_t stream) {
  const int grid = persist::num_cus();
  read_probe_kernel<<<grid, kProbeWaves * 64, 0, stream>>>(
      reinterpret_cast<const uint8_t *>(pool), pool_bytes / kProbeBlock, order, num_blocks, sink);
  return check_launch("pa_read_probe");
}

}  // namespace pa
