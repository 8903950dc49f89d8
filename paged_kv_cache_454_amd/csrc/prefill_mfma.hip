// Chunked paged prefill on the matrix cores (BF16 in, fp32 accumulation),
// head_dim 256: "vLLM Architecture, Memory and Benchmarks Deep Dive", s.4
// (a long prompt is processed in chunks, e.g. 512 tokens, against the paged
// cache) and "Inside vLLM", "FlashAttention-2 Integration" (one fused causal
// pass over packed, unpadded queries, no n x n score matrix in memory).
//
// Rows. The query rows of one KV head are the (position j, query head hh)
// pairs of a sequence's chunk, flattened as r = j * G + hh, so the G query
// heads that share a KV head sit in the same tile and every K/V byte staged
// in LDS serves all of them. A workgroup owns 128 rows (4 wavefronts x 32).
//
// Per 32-token K/V tile (K and V gathered through the block table into LDS,
// double-buffered, the next tile's global loads in flight during compute):
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (M = 32 tokens, N = 32
//    rows, K = 16 channels; 16 steps over head_dim). In the accumulator
//    layout each lane holds one query row (lane % 32) and 16 of the tile's
//    tokens, so the causal/length mask, the row max and the exponentials are
//    per-lane work plus one v_permlane32_swap to meet the other 16 tokens.
//  * Online softmax in the exp2 domain with a lazy running max (the output
//    is rescaled only when a tile raises the max by more than 2^8), weights
//    rounded to BF16.
//  * O^T += V^T . P^T with the same instruction (M = 32 channels, N = 32
//    rows, K = 16 tokens): the weights are already in B-operand order in the
//    lane that computed them; V is staged transposed in LDS ([channel][token])
//    so the A operand is two 8-byte LDS reads. The k order of the tokens in
//    both operands is the same permutation, which a sum over tokens ignores.
// Causality: query j of a chunk of n sits at position T - n + j and sees
// tokens [0, T - n + j]; a workgroup stops at the last tile its rows can see.
#include <math.h>

#include "launch.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int D = 256;
constexpr int WAVES = 4;
constexpr int ROWS = WAVES * 32;        // query rows per workgroup
constexpr int KT = 32;                  // tokens per K/V tile
constexpr int KPITCH = D * 2 + 16;      // bytes per token row of the K tile (+16: bank spread)
constexpr int VPITCH = KT * 2 + 8;      // bytes per channel row of the transposed V tile
constexpr int KBYTES = KT * KPITCH;     // 16,896
constexpr int VBYTES = D * VPITCH;      // 18,432
constexpr int MAX_TABLE = 2048;         // block ids staged in LDS
constexpr float kLazy = 8.f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma(const uint4 &a, const uint4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int G>
__global__ __launch_bounds__(WAVES * 64) void prefill_mfma_kernel(PrefillParams p, int row_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][KBYTES + VBYTES];
  __shared__ int tab[MAX_TABLE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 8 of a 16-wide k step this lane supplies
  const int l32 = lane & 31;

  // Later row blocks see more tokens: launch them first.
  const int rb = row_blocks - 1 - (int)(blockIdx.x % row_blocks);
  const int sk = blockIdx.x / row_blocks;
  const int kvh = sk % p.num_kv_heads;
  const int s = sk / p.num_kv_heads;

  const int q0 = p.query_start_loc[s];
  const int n = p.query_start_loc[s + 1] - q0;
  const int T = p.context_lens[s];
  const int nrows = n * G;
  if (n <= 0 || rb * ROWS >= nrows) return;
  const bool bad = T < n || (int64_t)T > (int64_t)p.max_blocks_per_seq * p.block_size;
  const int ctx0 = T - n;  // position of the chunk's first query

  // This lane's query row.
  const int r = rb * ROWS + wave * 32 + l32;
  const bool row_ok = r < nrows && q0 + r / G < p.num_q_tokens;
  const int j = row_ok ? r / G : 0;
  const int hh = row_ok ? r - j * G : 0;
  const int limit = row_ok && !bad ? ctx0 + j + 1 : 0;  // tokens [0, limit) are visible
  // Tokens the workgroup needs: up to the last valid row's limit.
  const int last_row = min(rb * ROWS + ROWS, nrows) - 1;
  const int wg_limit = bad ? 0 : ctx0 + last_row / G + 1;
  const int ntiles = (wg_limit + KT - 1) / KT;

  // Block ids of the tokens the workgroup reads, and the first invalid one:
  // a row that would read it gets NaN outputs (its reads become zeros).
  __shared__ int first_bad;
  const int bs = p.block_size;
  const int nb = p.num_blocks;
  const int nblk = (wg_limit + bs - 1) / bs;
  const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
  if (tid == 0) first_bad = 0x7fffffff;
  __syncthreads();
  for (int i = tid; i < nblk; i += WAVES * 64) {
    const int b = table[i];
    tab[i] = b;
    if (b < 0 || b >= nb) atomicMin(&first_bad, i);
  }

  // Q^T fragments (B operand of S^T): row l32, channels 16k + 8*half .. +7.
  uint4 qf[16];
  {
    const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.query) +
                         ((int64_t)(q0 + j) * p.num_q_heads + (int64_t)kvh * G + hh) * D +
                         8 * half;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const vec16 v = row_ok ? load16(qp + 16 * k) : vec16{{0, 0, 0, 0}};
      qf[k] = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
    }
  }
  __syncthreads();  // block ids visible

  const int64_t head_stride = (int64_t)bs * D;
  const int64_t block_stride = head_stride * p.num_kv_heads;
  const uint16_t *kpool = reinterpret_cast<const uint16_t *>(p.key_cache) + kvh * head_stride;
  const uint16_t *vpool = reinterpret_cast<const uint16_t *>(p.value_cache) + kvh * head_stride;

  // Global -> register staging of one tile: K as 4 pieces of 16 B per thread
  // (32 threads per token row), V as 2 token pairs x 16 B per thread.
  // Tokens past the context, or in a block with an invalid id, read as zero.
  vec16 kreg[4], vreg[2][2];
  auto tok_ptr = [&](const uint16_t *pool, int tok) -> const uint16_t * {
    if (tok >= wg_limit) return nullptr;
    const int blk = tab[tok / bs];
    if (blk < 0 || blk >= nb) return nullptr;
    return pool + (int64_t)blk * block_stride + (int64_t)(tok % bs) * D;
  };
  auto fetch = [&](int it) {
    const int t0 = it * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + i * WAVES * 64;  // 32 tokens x 32 chunks
      const int tok = piece >> 5, ch = piece & 31;
      const uint16_t *src = tok_ptr(kpool, t0 + tok);
      kreg[i] = src ? load16(src + ch * 8) : vec16{{0, 0, 0, 0}};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + i * WAVES * 64;  // 16 token pairs x 32 chunks
      const int pr = q >> 5, ch = q & 31;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint16_t *src = tok_ptr(vpool, t0 + 2 * pr + u);
        vreg[i][u] = src ? load16(src + ch * 8) : vec16{{0, 0, 0, 0}};
      }
    }
  };
  auto stash = [&](int buf) {
    uint8_t *kl = kv_lds[buf];
    uint8_t *vl = kv_lds[buf] + KBYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + i * WAVES * 64;
      const int tok = piece >> 5, ch = piece & 31;
      *reinterpret_cast<uint4 *>(kl + tok * KPITCH + ch * 16) =
          make_uint4(kreg[i].w[0], kreg[i].w[1], kreg[i].w[2], kreg[i].w[3]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + i * WAVES * 64;
      const int pr = q >> 5, ch = q & 31;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = vreg[i][0].w[w], b = vreg[i][1].w[w];
        // channels 8ch + 2w and 8ch + 2w + 1, tokens 2pr and 2pr + 1
        const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07060302u);
        *reinterpret_cast<uint32_t *>(vl + (8 * ch + 2 * w) * VPITCH + pr * 4) = lo;
        *reinterpret_cast<uint32_t *>(vl + (8 * ch + 2 * w + 1) * VPITCH + pr * 4) = hi;
      }
    }
  };

  f32x16 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = kNoMax, l = 0.f;
  const float sl2 = p.scale * kLog2e;

  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) fetch(it + 1);  // in flight during this tile's math
    const uint8_t *kl = kv_lds[buf];
    const uint8_t *vl = kv_lds[buf] + KBYTES;
    const int t0 = it * KT;

    // S^T (32 tokens x 32 rows), two independent accumulation chains.
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      const uint4 ka = *reinterpret_cast<const uint4 *>(kl + l32 * KPITCH + (16 * k + 8 * half) * 2);
      const uint4 kb =
          *reinterpret_cast<const uint4 *>(kl + l32 * KPITCH + (16 * (k + 1) + 8 * half) * 2);
      s0 = mfma(ka, qf[k], s0);
      s1 = mfma(kb, qf[k + 1], s1);
    }
    // Element e of the accumulator is token 8*(e/4) + 4*half + e%4.
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tok = t0 + 8 * (e >> 2) + 4 * half + (e & 3);
      const float v = (s0[e] + s1[e]) * sl2;
      z[e] = tok < limit ? v : -INFINITY;
      mx = fmaxf(mx, z[e]);
    }
    mx = other_half_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
      const float mn = fmaxf(m, mx);
      const float a = fast_exp2(m - mn);
      l *= a;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= a;
      m = mn;
    }
    // Weights as the B operand of O^T: chunk c takes elements 8c .. 8c+7.
    uint4 pw[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float pa = fast_exp2(z[8 * c + 2 * u] - m);
        const float pb = fast_exp2(z[8 * c + 2 * u + 1] - m);
        w4[u] = bf16_pair(pa, pb);
        l += __uint_as_float(w4[u] << 16) + __uint_as_float(w4[u] & 0xffff0000u);
      }
      pw[c] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    // O^T (32 channels x 32 rows per dt) += V^T . P^T; the A operand's token
    // order matches the weights': 16c + 8*(e/4) + 4*half + e%4.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint8_t *vrow = vl + (32 * dt + l32) * VPITCH;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + (16 * c + 4 * half) * 2);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + (16 * c + 8 + 4 * half) * 2);
        o[dt] = mfma(make_uint4(lo.x, lo.y, hi.x, hi.y), pw[c], o[dt]);
      }
    }
    if (it + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }

  const float lt = other_half_sum(l);  // both halves of a row share row_ok
  if (!row_ok) return;
  const bool row_bad = bad || (int64_t)first_bad * bs < limit;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float nan = __builtin_nanf("");
  const int64_t orow = ((int64_t)(q0 + j) * p.num_q_heads + (int64_t)kvh * G + hh) * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * dt + 8 * i + 4 * half;
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = row_bad ? nan : o[dt][4 * i + u] * inv;
      if (p.out_bf16) {
        uint16_t *op = reinterpret_cast<uint16_t *>(p.out) + orow + d0;
        *reinterpret_cast<uint2 *>(op) =
            make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
      } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.out) + orow + d0) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
}

}  // namespace

// The MFMA path covers BF16, head_dim 256 and tables of up to 2048 blocks
// per sequence; false otherwise.
bool launch_prefill_mfma(const PrefillParams &p, hipStream_t stream) {
  if (p.head_dim != D || p.max_blocks_per_seq > MAX_TABLE) return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  const int64_t row_blocks = ((int64_t)p.max_query_len * group + ROWS - 1) / ROWS;
  const int64_t grid = row_blocks * p.num_seqs * p.num_kv_heads;
  if (grid <= 0 || grid > 0x7fffffff) return false;
  switch (group) {
#define PA_CASE(g)                                                                  \
  case g:                                                                           \
    prefill_mfma_kernel<g><<<(unsigned)grid, WAVES * 64, 0, stream>>>(p, (int)row_blocks); \
    return true;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default: return false;
  }
}

}  // namespace pa
