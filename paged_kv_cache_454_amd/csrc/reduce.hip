// Log-sum-exp merge of split-context partitions.
//
// Partition p of (sequence, query head) carries its normalised output o_p,
// its logit bound m_p and l_p = sum exp(logit - m_p). With M = max_p m_p the
// merged result is sum_p (l_p e^(m_p - M)) o_p / sum_p l_p e^(m_p - M): the
// weights are each partition's share of the total softmax mass, so the merge
// is exact up to rounding and never evaluates exp of a large positive value.
//
// One workgroup per (sequence, query head). The partition weights are
// computed once into LDS by the first wavefront; then every thread owns
// head_dim / blockDim channels and streams the partitions' outputs, which
// are contiguous per (sequence, head), so the reads are coalesced.
#include <math.h>

#include "launch.h"
#include "pa_device.h"

namespace pa {

constexpr int kReduceMaxParts = 1024;  // weights held in LDS

__global__ __launch_bounds__(256) void reduce_kernel(void *out, const float *__restrict__ part_out,
                                                     const float *__restrict__ part_max,
                                                     const float *__restrict__ part_sum,
                                                     const int32_t *__restrict__ context_lens,
                                                     int num_q_heads, int head_dim,
                                                     int partition_size, int max_parts,
                                                     int out_bf16) {
  __shared__ float sm_w[kReduceMaxParts];
  __shared__ float sm_total;
  const int sh = blockIdx.x;  // sequence * num_q_heads + head
  const int seq = sh / num_q_heads;
  int T = context_lens[seq];
  T = T < 0 ? 0 : T;
  const int64_t n64 = ((int64_t)T + partition_size - 1) / partition_size;
  const bool bad = n64 > max_parts;
  const int n = bad ? 0 : (int)n64;
  const float *pm = part_max + (int64_t)sh * max_parts;
  const float *ps = part_sum + (int64_t)sh * max_parts;

  if (threadIdx.x < 64) {
    float M = kNoMax;
    for (int i = threadIdx.x; i < n; i += 64) M = fmaxf(M, pm[i]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float tot = 0.f;
    for (int i = threadIdx.x; i < n; i += 64) {
      const float wgt = ps[i] * fast_exp2((pm[i] - M) * kLog2e);
      sm_w[i] = wgt;
      tot += wgt;
    }
    for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
    if (threadIdx.x == 0) sm_total = tot;
  }
  __syncthreads();
  const float inv = n > 0 ? 1.f / sm_total : 0.f;
  const float *po = part_out + (int64_t)sh * max_parts * head_dim;
  for (int ch = threadIdx.x; ch < head_dim; ch += blockDim.x) {
    float a = 0.f;
    for (int i = 0; i < n; ++i) a = fmaf(sm_w[i], po[(int64_t)i * head_dim + ch], a);
    const float o = bad ? __builtin_nanf("") : a * inv;
    store_out(out, (int64_t)sh * head_dim + ch, o, out_bf16);
  }
}

pa_status launch_reduce(void *out, const float *part_out, const float *part_max,
                        const float *part_sum, const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_parts, int32_t out_bf16, hipStream_t stream) {
  if (max_parts > kReduceMaxParts)
    return fail(PA_EUNSUPPORTED, "pa_reduce: max_parts=%d > %d", max_parts, kReduceMaxParts);
  const int64_t grid = (int64_t)num_seqs * num_q_heads;
  if (grid == 0) return PA_OK;
  const int threads = head_dim >= 256 ? 256 : 64;
  reduce_kernel<<<(unsigned)grid, threads, 0, stream>>>(out, part_out, part_max, part_sum,
                                                        context_lens, num_q_heads, head_dim,
                                                        partition_size, max_parts, out_bf16);
  return check_launch("pa_reduce");
}

}  // namespace pa
