// The decode step's K/V write as a launch of its own: used when the step's
// decode kernel reads the step's token from the pool (shapes the matrix-core
// kernel does not cover, where this runs before the decode) or when no merge
// kernel follows (single pass, where it runs after).
#include "append_rows.h"
#include "pa_device.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, const int32_t *context_lens,
                                                     int rows) {
  const int lane = threadIdx.x & 63;
  const int sh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (sh >= rows) return;
  const int s = sh / a.num_kv_heads, h = sh - s * a.num_kv_heads;
  const int T = __builtin_amdgcn_readfirstlane(context_lens[s]);
  const AppendLoad r = append_issue(a, s, h, T, lane);
  append_commit(a, r, h, lane);
}

}  // namespace

pa_status launch_append(const AppendArgs &a, const int32_t *context_lens, int32_t num_seqs,
                        hipStream_t stream) {
  const int64_t rows = (int64_t)num_seqs * a.num_kv_heads;
  if (rows == 0) return PA_OK;
  if (a.row_bytes % 16 != 0 || a.row_bytes / 16 * 2 > 64 * kAppendPieces)
    return fail(PA_EUNSUPPORTED, "decode step: %d-byte rows", a.row_bytes);
  if (rows > INT32_MAX - 3)
    return fail(PA_EUNSUPPORTED, "decode step: %lld rows", (long long)rows);
  append_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(a, context_lens, (int)rows);
  return check_launch("decode step write");
}

}  // namespace pa
