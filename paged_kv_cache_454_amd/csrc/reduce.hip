// Log-sum-exp merge of split-context partitions.
//
// Partition p of (sequence, query head) carries its normalised output o_p,
// its logit bound m_p and l_p = sum exp(logit - m_p). With M = max_p m_p the
// merged result is sum_p (l_p e^(m_p - M)) o_p / sum_p l_p e^(m_p - M): the
// weights are each partition's share of the total softmax mass, so the merge
// is exact up to rounding and never evaluates exp of a large positive value.
//
// One wavefront per (sequence, query head). The work is two dependent memory
// round trips: (1) the context length together with the (m, l) records of the
// first 64 partitions, one per lane, read before the count is known (the
// records lie inside the caller's [max_parts] rows either way); (2) the
// partition outputs, 16 partitions per batch, through a buffer resource that
// ends at the last valid partition, so loads past it return zeros without a
// memory access and need no branch. Each lane owns VEC channels of a row (a
// lane past head_dim reads the next partition's channels and discards them).
//
// In a decode step the same launch also writes the step's K/V rows to their
// slots (the decode kernel before it read them from the step's rows, not
// from the pool): the wavefront of each KV head's first query head issues
// those loads beside its round trip 2 and stores them at the end.
#include <math.h>

#include "append_rows.h"
#include "launch.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kReduceMaxParts = 1024;
constexpr int kBatch = 16;  // partition outputs in flight per lane

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int VEC>
struct Chan;
template <>
struct Chan<4> {
  float v[4];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(x[i]);
  }
};
template <>
struct Chan<1> {
  float v[1];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
};

template <int VEC>
__global__ __launch_bounds__(256) void reduce_kernel(void *out, const float *__restrict__ part_out,
                                                     const float *__restrict__ part_max,
                                                     const float *__restrict__ part_sum,
                                                     const int32_t *__restrict__ context_lens,
                                                     int rows, int num_q_heads, int head_dim,
                                                     int partition_size, int max_parts,
                                                     int out_bf16, AppendArgs app) {
  const int lane = threadIdx.x & 63;
  // sequence * num_q_heads + head, uniform per wavefront
  const int sh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (sh >= rows) return;
  const int seq = sh / num_q_heads;
  const float *pm = part_max + (int64_t)sh * max_parts;
  const float *ps = part_sum + (int64_t)sh * max_parts;

  // Round trip 1.
  const bool in_row = lane < max_parts;
  const float m0 = in_row ? pm[lane] : 0.f;
  const float l0 = in_row ? ps[lane] : 0.f;
  int T = __builtin_amdgcn_readfirstlane(context_lens[seq]);
  T = T < 0 ? 0 : T;
  const int64_t n64 = ((int64_t)T + partition_size - 1) / partition_size;
  const bool bad = n64 > max_parts;
  const int n = bad ? 0 : (int)n64;

  const int group = app.new_key ? num_q_heads / app.num_kv_heads : 1;
  const int qh = sh - seq * num_q_heads;
  const bool writer = app.new_key != nullptr && qh % group == 0;  // uniform
  AppendLoad al{};
  if (writer) al = append_issue(app, seq, qh / group, T, lane);

  // M over the valid partitions (fmaxf skips a NaN record; its NaN weight
  // still poisons the row below).
  float M = lane < n ? m0 : kNoMax;
  for (int i = 64 + lane; i < n; i += 64) M = fmaxf(M, pm[i]);
  M = wave_max(M);

  // Round trip 2: sum_p w_p o_p, 64 partitions' weights per chunk (lane j
  // holds w of partition j0 + j), outputs in batches of kBatch.
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(part_out + (int64_t)sh * max_parts * head_dim), (short)0,
      n * head_dim * 4, 0x00020000);
  float wsum = 0.f;
  // Every lane runs every channel group (lane j holds partition j's weight,
  // read by all lanes); lanes past head_dim only skip the store.
  for (int cb = 0; cb < head_dim; cb += 64 * VEC) {
    const int c0 = cb + lane * VEC;
    float a[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) a[e] = 0.f;
    wsum = 0.f;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      float mj = m0, lj = l0;
      if (j0 > 0) {
        mj = j < n ? pm[j] : 0.f;
        lj = j < n ? ps[j] : 0.f;
      }
      const float w = j < n ? lj * fast_exp2((mj - M) * kLog2e) : 0.f;
      wsum += w;
      const int cnt = min(64, n - j0);
      for (int b = 0; b < cnt; b += kBatch) {
        Chan<VEC> x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) x[u].load(orsrc, ((j0 + b + u) * head_dim + c0) * 4);
        __builtin_amdgcn_sched_barrier(0);  // keep the whole batch in flight
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), b + u));
#pragma unroll
          for (int e = 0; e < VEC; ++e) a[e] = fmaf(wu, x[u].v[e], a[e]);
        }
      }
    }
    const float tot = wave_sum(wsum);
    const float inv = n > 0 ? 1.f / tot : 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (c0 + e < head_dim)
        store_out(out, (int64_t)sh * head_dim + c0 + e, bad ? __builtin_nanf("") : a[e] * inv,
                  out_bf16);
    }
  }
  if (writer) append_commit(app, al, qh / group, lane);
}

}  // namespace

pa_status launch_reduce(void *out, const float *part_out, const float *part_max,
                        const float *part_sum, const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_parts, int32_t out_bf16, hipStream_t stream,
                        const AppendArgs *append) {
  AppendArgs app{};
  if (append) {
    app = *append;
    if (app.row_bytes % 16 != 0 || app.row_bytes / 16 * 2 > 64 * kAppendPieces ||
        app.num_kv_heads <= 0 || num_q_heads % app.num_kv_heads != 0)
      return fail(PA_EUNSUPPORTED, "decode step: %d-byte rows", app.row_bytes);
  }
  if (max_parts > kReduceMaxParts)
    return fail(PA_EUNSUPPORTED, "pa_reduce: max_parts=%d > %d", max_parts, kReduceMaxParts);
  const int64_t rows = (int64_t)num_seqs * num_q_heads;
  if (rows == 0) return PA_OK;
  if (rows > INT32_MAX - 3 || (int64_t)max_parts * head_dim * 4 > INT32_MAX)
    return fail(PA_EUNSUPPORTED, "pa_reduce: %lld rows of %d x %d partitions too large",
                (long long)rows, max_parts, head_dim);
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (head_dim % 4 == 0)
    reduce_kernel<4><<<grid, 256, 0, stream>>>(out, part_out, part_max, part_sum, context_lens,
                                               (int)rows, num_q_heads, head_dim, partition_size,
                                               max_parts, out_bf16, app);
  else
    reduce_kernel<1><<<grid, 256, 0, stream>>>(out, part_out, part_max, part_sum, context_lens,
                                               (int)rows, num_q_heads, head_dim, partition_size,
                                               max_parts, out_bf16, app);
  return check_launch("pa_reduce");
}

}  // namespace pa
