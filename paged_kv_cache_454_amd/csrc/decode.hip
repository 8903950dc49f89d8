// Paged decode attention: generic kernel (any supported head_dim, dtype,
// block size and group), single pass or split into context partitions.
//
// What is computed ("Optimizing LLM Inference" (voronkin.com), PagedAttention
// section: blocks scattered in memory "appear contiguous to the attention
// mechanism"; "vLLM Architecture, Memory and Benchmarks Deep Dive", s.1-2):
// for query head h of row s, softmax over the scaled logits q.K_t of the
// row's cached tokens t, applied to their V rows, with K_t/V_t fetched from
// physical block block_tables[s][t / block_size] at offset t % block_size.
//
// Work decomposition (one workgroup = NW wavefronts of 64 lanes per
// (row, KV head, partition)):
//  * A token's K (or V) row for one KV head is head_dim contiguous elements.
//    Each lane loads one 16-byte piece of a row, so one wavefront load covers
//    64 * 16 = 1 KiB = whole rows (two rows at head_dim 256 BF16), fully
//    coalesced, straight from the physical block into registers.
//  * All query heads of the group sharing the KV head are handled by the
//    same lanes: each K/V byte is read from HBM once per group, not once per
//    query head.
//  * Partial dot products are summed across the lanes of a row with
//    butterfly shuffles; each row group keeps its own running max / sum /
//    accumulator (online softmax, log2 domain), merged at the end first
//    across row groups (shuffles) and then across wavefronts (LDS).
// Masking uses selects, never multiplication by zero, so NaN garbage in
// unused slots cannot leak.
//
// The same kernel also serves as the plain correctness path for causal
// prefill rows (query_start_loc != nullptr): a prefill query row is a decode
// over the prefix of its sequence up to and including its own position.
#include <math.h>

#include "launch.h"
#include "pa_device.h"

namespace pa {

namespace {

struct RowWork {
  int seq;     // sequence whose block table / cache the row reads
  int row;     // output row (== seq for decode); -1: no such prefill row
  int T;       // tokens visible to the row
  bool bad;    // inconsistent lengths: poison the outputs
};

// Decode: virtual row = sequence. Prefill: virtual row = seq * max_query_len
// + j, the j-th query of the sequence's chunk (absent when j >= chunk length).
__device__ __forceinline__ RowWork row_work(const DecodeParams &p, int vrow) {
  RowWork w;
  w.bad = false;
  if (p.query_start_loc == nullptr) {
    w.seq = vrow;
    w.row = vrow;
    w.T = p.context_lens[vrow];
  } else {
    w.seq = vrow / p.max_query_len;
    const int j = vrow - w.seq * p.max_query_len;
    const int start = p.query_start_loc[w.seq];
    const int n = p.query_start_loc[w.seq + 1] - start;
    const int total = p.context_lens[w.seq];
    w.row = (j < n && start + j < p.num_q_tokens) ? start + j : -1;
    if (total < n) w.bad = true;
    w.T = total - n + j + 1;
  }
  if (w.T < 0) w.T = 0;
  return w;
}

}  // namespace

template <typename KV, int HEAD_DIM, int MAXG, int NW>
__global__ __launch_bounds__(NW * 64) void decode_generic_kernel(DecodeParams p) {
  using Piece = KvPiece<KV>;
  using QT = typename Piece::Q;
  constexpr int VEC = Piece::N;
  static_assert(Widen<QT>::N == VEC, "query and K/V pieces must cover the same channels");
  constexpr bool F8 = sizeof(KV) == 1;
  constexpr int LPR = HEAD_DIM / VEC;  // lanes per token row
  constexpr int RPL = 64 / LPR;        // token rows per wavefront load
  static_assert(HEAD_DIM % VEC == 0 && LPR <= 64 && 64 % LPR == 0, "unsupported shape");

  __shared__ float sm_m[NW][MAXG];
  __shared__ float sm_l[NW][MAXG];
  __shared__ float sm_acc[NW][MAXG][HEAD_DIM];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;

  const int num_rows = p.query_start_loc ? p.num_seqs * p.max_query_len : p.num_seqs;
  const int bid = blockIdx.x;  // (part * num_rows + row) * num_kv_heads + kvh
  const int kvh = bid % p.num_kv_heads;
  const int rest = bid / p.num_kv_heads;
  const int part = rest / num_rows;
  RowWork w = row_work(p, rest % num_rows);
  if (w.row < 0) return;  // uniform for the workgroup
  const int group = p.num_q_heads / p.num_kv_heads;

  int T = w.T;
  bool bad = w.bad;
  const int64_t cap = (int64_t)p.max_blocks_per_seq * p.block_size;
  if ((int64_t)T > cap) {
    bad = true;
    T = (int)cap;
  }
  int lo = 0, hi = T;
  if (p.partition_size > 0) {
    if ((int64_t)T > (int64_t)p.max_parts * p.partition_size) bad = true;
    lo = part * p.partition_size;
    if (lo >= T) return;  // absent partition: uniform exit of the workgroup
    hi = min(T, lo + p.partition_size);
  }

  const int64_t qrow = (int64_t)w.row * p.num_q_heads + (int64_t)kvh * group;
  float q[MAXG][VEC];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < group) {
      const QT *qp = reinterpret_cast<const QT *>(p.query) + (qrow + h) * HEAD_DIM + c * VEC;
      Widen<QT>::apply(load16(qp), q[h]);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) q[h][v] = 0.f;
    }
  }

  float m[MAXG], l[MAXG], acc[MAXG][VEC];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    m[h] = kNoMax;
    l[h] = 0.f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[h][v] = 0.f;
  }

  // An FP8 cache holds K / k_scale: the K scale folds into the logit scale,
  // the V scale into the final outputs.
  const float sl2 = p.scale * kLog2e * (F8 ? p.k_scale : 1.f);
  const float vsc = F8 ? p.v_scale : 1.f;
  const int bs = p.block_size;
  const int32_t *table = p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq;
  const int64_t head_stride = (int64_t)bs * HEAD_DIM;
  const int64_t block_stride = head_stride * p.num_kv_heads;
  const KV *kbase = reinterpret_cast<const KV *>(p.key_cache) + kvh * head_stride + c * VEC;
  // An FP8 value pool stores each block transposed ([head_dim][block_size]):
  // channel ch of token offset o sits at ch * bs + o.
  const KV *vbase = reinterpret_cast<const KV *>(p.value_cache) + kvh * head_stride +
                    (F8 ? (int64_t)c * VEC * bs : (int64_t)c * VEC);

  for (int t0 = lo + wave * RPL; t0 < hi; t0 += NW * RPL) {
    const int t = t0 + r;
    bool valid = t < hi;
    int64_t off = 0, voff = 0;
    if (valid) {
      const int blk = table[t / bs];
      if (blk < 0 || blk >= p.num_blocks) {
        bad = true;
        valid = false;
      } else {
        off = (int64_t)blk * block_stride + (int64_t)(t % bs) * HEAD_DIM;
        voff = F8 ? (int64_t)blk * block_stride + t % bs : off;
      }
    }
    float kf[VEC], vf[VEC];
    if (valid) {
      Piece::load(kbase + off, kf);
      if constexpr (F8) {
        const uint8_t *vp = reinterpret_cast<const uint8_t *>(vbase + voff);
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int v = 0; v < VEC; ++v) w[v / 4] |= (uint32_t)vp[(int64_t)v * bs] << (8 * (v % 4));
        e4m3x4_to_f32(w[0], vf);
        e4m3x4_to_f32(w[1], vf + 4);
      } else {
        Piece::load(vbase + voff, vf);
      }
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) kf[v] = vf[v] = 0.f;
    }
    float s[MAXG];
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      float d = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) d = fmaf(q[h][v], kf[v], d);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o);
      s[h] = valid ? d * sl2 : -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      if (h < group) {
        const float mn = fmaxf(m[h], s[h]);
        const float alpha = fast_exp2(m[h] - mn);
        const float pr = fast_exp2(s[h] - mn);
        l[h] = fmaf(l[h], alpha, pr);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[h][v] = fmaf(acc[h][v], alpha, pr * vf[v]);
        m[h] = mn;
      }
    }
  }

  // Merge row groups of the wavefront (they saw different tokens).
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      const float m2 = __shfl_xor(m[h], o);
      const float l2 = __shfl_xor(l[h], o);
      const float mn = fmaxf(m[h], m2);
      const float f1 = fast_exp2(m[h] - mn), f2 = fast_exp2(m2 - mn);
      l[h] = l[h] * f1 + l2 * f2;
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[h][v] = acc[h][v] * f1 + __shfl_xor(acc[h][v], o) * f2;
      m[h] = mn;
    }
  }

  if (r == 0) {
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) sm_acc[wave][h][c * VEC + v] = acc[h][v];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  bad = __syncthreads_or(bad);

  const float nan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < group * HEAD_DIM; idx += NW * 64) {
    const int h = idx / HEAD_DIM;
    const int ch = idx - h * HEAD_DIM;
    float M = kNoMax;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float f = fast_exp2(sm_m[i][h] - M);
      L += sm_l[i][h] * f;
      A += sm_acc[i][h][ch] * f;
    }
    if (p.partition_size == 0) {
      const float o = bad ? nan : (L > 0.f ? A / L * vsc : 0.f);
      store_out(p.out, (qrow + h) * HEAD_DIM + ch, o, p.out_bf16);
    } else {
      const int64_t pidx = (qrow + h) * p.max_parts + part;
      p.part_out[pidx * HEAD_DIM + ch] = bad ? nan : A / L * vsc;
      if (ch == 0) {
        p.part_max[pidx] = bad ? nan : M * kLn2;
        p.part_sum[pidx] = bad ? nan : L;
      }
    }
  }
}

template <typename KV, int HEAD_DIM, int MAXG>
static void launch_generic(const DecodeParams &p, unsigned grid, hipStream_t stream) {
  constexpr int NW = 4;
  decode_generic_kernel<KV, HEAD_DIM, MAXG, NW><<<grid, NW * 64, 0, stream>>>(p);
}

template <typename KV, int HEAD_DIM>
static void launch_generic_g(const DecodeParams &p, int group, unsigned grid,
                             hipStream_t stream) {
  if (group <= 1)
    launch_generic<KV, HEAD_DIM, 1>(p, grid, stream);
  else if (group <= 2)
    launch_generic<KV, HEAD_DIM, 2>(p, grid, stream);
  else if (group <= 4)
    launch_generic<KV, HEAD_DIM, 4>(p, grid, stream);
  else
    launch_generic<KV, HEAD_DIM, 8>(p, grid, stream);
}

template <typename KV>
static void launch_generic_d(const DecodeParams &p, int group, unsigned grid,
                             hipStream_t stream) {
  switch (p.head_dim) {
    case 64: launch_generic_g<KV, 64>(p, group, grid, stream); break;
    case 128: launch_generic_g<KV, 128>(p, group, grid, stream); break;
    default: launch_generic_g<KV, 256>(p, group, grid, stream); break;
  }
}

pa_status launch_decode(const DecodeParams &p, hipStream_t stream) {
  const int group = p.num_q_heads / p.num_kv_heads;
  const int64_t rows =
      p.query_start_loc ? (int64_t)p.num_seqs * p.max_query_len : (int64_t)p.num_seqs;
  const int64_t parts = p.partition_size > 0 ? p.max_parts : 1;
  const int64_t grid = rows * p.num_kv_heads * parts;
  if (grid == 0) return PA_OK;
  if (grid > 0x7fffffff) return fail(PA_EUNSUPPORTED, "decode: grid of %lld workgroups", (long long)grid);
  if (launch_decode_fp8(p, stream)) return check_launch("decode");
  if (launch_decode_mfma(p, stream)) return check_launch("decode");
  // Only the matrix-core kernel reads a step's token from new_key/new_value.
  if (p.new_key) return fail(PA_EUNSUPPORTED, "decode: step rows need the matrix-core kernel");
  if (launch_decode_tiled(p, (unsigned)grid, stream)) return check_launch("decode");
  if (p.kv_fp8)
    launch_generic_d<fp8_t>(p, group, (unsigned)grid, stream);
  else if (p.kv_bf16)
    launch_generic_d<bf16_t>(p, group, (unsigned)grid, stream);
  else
    launch_generic_d<float>(p, group, (unsigned)grid, stream);
  return check_launch("decode");
}

}  // namespace pa
