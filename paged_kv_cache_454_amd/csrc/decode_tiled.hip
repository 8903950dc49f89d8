// Paged decode attention for BF16 caches with head_dim 256 and block sizes
// that are multiples of 16 - the shape of the pages' workloads ("vLLM
// Architecture, Memory and Benchmarks Deep Dive", s.1: 4 KV heads, head
// dimension 256, BF16; s.2: blocks of 16 or 32 tokens). Same result and ABI
// as the generic kernel; this one is organised for gfx950's memory system
// and VALU.
//
// One workgroup = NW wavefronts per (sequence, KV head, context partition).
// A wavefront walks 16-token tiles of its partition (tile k -> wave k % NW):
//
//  * Loads. A tile's K (and V) rows for one KV head are 16 x 512 B = 8 KiB
//    contiguous inside one physical block. Each of 8 wavefront loads moves
//    1 KiB (16 B per lane, lanes in address order): lane l gets the 8
//    channels 8*(l%32).. of token 2*i + l/32. Loads are buffer loads off a
//    per-tile resource (tile base in SGPRs). The next tile's K is requested
//    before the current tile's Q.K and its V right after, so 8-16 KiB per
//    wavefront stay in flight; block ids are scalar loads issued one tile
//    ahead.
//  * Q.K. The group's G query heads are staged in LDS as BF16 pairs; per
//    head, the lane's 8 channels come back in one 16-byte read and 4
//    v_dot2_f32_bf16 per (token, head) give a partial
//    dot product. Partials are summed over the 32 lanes of a token: one
//    v_permlane16_swap + add halves them (32 -> 16 lanes, two values at a
//    time), then the 16 lanes of each row go through LDS and come back
//    transposed, one (head, token) logit per lane.
//  * Softmax. Logits live one per lane with each DPP row (16 lanes) holding
//    one head's 16 tokens, so the tile max is a 4-step DPP all-reduce. The
//    running max is only moved when a tile exceeds it by more than 2^8
//    (exp2 domain); otherwise exponentials are taken against the stale max,
//    which keeps every weight <= 256 and skips the accumulator rescale on
//    almost every tile. Weights are rounded to BF16; the running sum adds
//    the rounded weights, so numerator and denominator use the same numbers.
//  * P.V. Weights go to LDS as BF16 pairs of two tokens; each lane reads its
//    token half's pairs, packs the matching V channels of the two tokens
//    with v_perm_b32, and accumulates with v_dot2_f32_bf16 into G x 8 fp32
//    accumulators.
//  * The two token halves of the wavefront are merged with
//    v_permlane32_swap, the NW wavefronts through LDS.
// Out-of-range tokens of a partial tile (their slots may hold NaN garbage)
// never reach the arithmetic: their logits are set to -inf with selects, and
// their K/V rows lie past the tile resource's num_records, so the buffer
// loads return zeros for them (the whole byte offset is a vector offset,
// which the range check covers).
#include <math.h>

#include "launch.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int D = 256;         // head_dim
constexpr int TILE = 16;       // tokens per wavefront iteration
constexpr int LOADS = 8;       // 1 KiB wavefront loads per 8 KiB K (or V) tile
constexpr int RSTRIDE = 20;    // floats per LDS reduction row (16 + pad)
constexpr float kLazy = 8.f;   // rescale when the max grows by more than 2^8

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// All-reduce over the 16 lanes of a DPP row by rotations 8, 4, 2, 1.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x122>(x));
  x = fmaxf(x, dpp<0x121>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x128>(x);
  x += dpp<0x124>(x);
  x += dpp<0x122>(x);
  x += dpp<0x121>(x);
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16(float a) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)0.f;
  return __builtin_bit_cast(uint32_t, v) & 0xffffu;
}

template <int G, int NW>
struct Tiled {
  static constexpr int NV = 4 * G;            // partials per lane after the row-pair step
  static constexpr int NOUT = TILE * G;       // logits per tile
  static constexpr int ROUNDS = (NOUT + 63) / 64;
  static constexpr int RED = 4 * NV * RSTRIDE;  // floats of LDS per wave (>= G * D)
  static_assert(RED >= G * D, "merge buffer must fit in the reduction buffer");
};

template <int G, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_tiled_kernel(DecodeParams p) {
  using C = Tiled<G, NW>;
  __shared__ __attribute__((aligned(16))) float red_all[NW][C::RED];
  __shared__ __attribute__((aligned(16))) uint32_t pl_all[NW][2][4][8];  // [parity][pair][head]
  __shared__ float alpha_all[NW][8];
  __shared__ float mg_m[NW][8], mg_l[NW][8];

  const int lane = threadIdx.x & 63;
  // Uniform per wavefront; readfirstlane lets the compiler keep it (and all
  // tile addressing derived from it) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tau = lane >> 5;     // which token of a 1 KiB load (token parity)
  const int rrow = lane >> 4;    // DPP row
  const int k16 = lane & 15;
  float *red = red_all[wave];
  uint32_t(*pl)[4][8] = pl_all[wave];
  uint16_t *pl16 = reinterpret_cast<uint16_t *>(pl_all[wave]);

  const int bid = blockIdx.x;  // (part * num_seqs + seq) * num_kv_heads + kvh
  const int kvh = bid % p.num_kv_heads;
  const int rest = bid / p.num_kv_heads;
  const int seq = rest % p.num_seqs;
  const int part = rest / p.num_seqs;

  // Everything the first tiles need is requested at once, before any of it
  // is waited for: the context length, the block ids of this wave's first
  // three tiles and the group's query rows. The ids are looked up before the
  // length is known (a table index past the row is clamped into it; ids of
  // tiles past the context are never used), and the queries go to registers
  // and reach LDS after the first tile's loads have been issued.
  const int bs = p.block_size;
  typedef __attribute__((address_space(4))) const int32_t cint32;
  cint32 *tab = (cint32 *)(p.block_tables + (int64_t)seq * p.max_blocks_per_seq);
  const int64_t lo0 = p.partition_size > 0 ? (int64_t)part * p.partition_size : 0;
  auto early_id = [&](int j) -> int {
    const int64_t e = (lo0 + (int64_t)(wave + j * NW) * TILE) / bs;
    return tab[e < p.max_blocks_per_seq ? e : p.max_blocks_per_seq - 1];
  };
  const int eid0 = early_id(0), eid1 = early_id(1), eid2 = early_id(2);
  static_assert(G * 32 <= NW * 64, "one 16-byte query piece per thread");
  const int64_t qrow = (int64_t)seq * p.num_q_heads + (int64_t)kvh * G;
  uint4 qpiece = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < G * 32) {
    const vec16 v = load16(reinterpret_cast<const uint16_t *>(p.query) +
                           (qrow + threadIdx.x / 32) * D + (threadIdx.x % 32) * 8);
    qpiece = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
  }

  int T = p.context_lens[seq];
  T = T < 0 ? 0 : T;
  bool bad = false;
  const int64_t cap = (int64_t)p.max_blocks_per_seq * p.block_size;
  if ((int64_t)T > cap) {
    bad = true;
    T = (int)cap;
  }
  int lo = 0, hi = T;
  if (p.partition_size > 0) {
    if ((int64_t)T > (int64_t)p.max_parts * p.partition_size) bad = true;
    lo = part * p.partition_size;
    if (lo >= T) return;  // absent partition (uniform for the workgroup)
    hi = min(T, lo + p.partition_size);
  }
  const int ntiles = (hi - lo + TILE - 1) / TILE;

  // Query heads of the group as BF16 pairs, staged once in LDS: Q.K reads
  // the lane's 8 channels of one head at a time, which keeps 4*G registers
  // free for the K/V pipeline.
  __shared__ uint4 qs[G][32];

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m_r[C::ROUNDS], l_r[C::ROUNDS];
#pragma unroll
  for (int r = 0; r < C::ROUNDS; ++r) {
    m_r[r] = kNoMax;
    l_r[r] = 0.f;
  }

  const float sl2 = p.scale * kLog2e;
  const int64_t head_stride = (int64_t)bs * D;
  const int64_t block_stride = head_stride * p.num_kv_heads;
  const uint16_t *kpool = reinterpret_cast<const uint16_t *>(p.key_cache) + kvh * head_stride;
  const uint16_t *vpool = reinterpret_cast<const uint16_t *>(p.value_cache) + kvh * head_stride;

  // This wave's tiles are kk = wave + j * NW, j < nj. Block ids come through
  // the scalar cache (uniform per wavefront) one iteration ahead of the
  // loads that need them, so no vector-memory wait is spent on the table.
  const int nj = wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0;
  auto block_of = [&](int j) -> int {
    const int kk = wave + j * NW;
    return kk < ntiles ? tab[(lo + kk * TILE) / bs] : 0;
  };
  // Buffer resource over the valid rows of one tile of a pool: the base sits
  // in SGPRs, lanes add 16-byte offsets and loads add 1 KiB steps. Rows past
  // the context (and every row of a tile past the wave's last) lie outside
  // num_records, so the hardware returns zeros for them without touching
  // memory: V rows of out-of-range tokens arrive as 0 and need no masking.
  auto tile_rsrc = [&](int j, int blk, const uint16_t *pool) {
    const int kk = wave + j * NW;
    const int tok0 = lo + kk * TILE;
    int bytes = 0;
    if (kk < ntiles) {
      if (blk < 0 || blk >= p.num_blocks) {
        bad = true;
        blk = 0;
      }
      bytes = min(TILE, hi - tok0) * D * 2;
    } else {
      blk = 0;
    }
    const uint16_t *base = pool + (int64_t)blk * block_stride + (int64_t)(tok0 % bs) * D;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, bytes,
                                             0x00020000);
  };

  // Q.K for one tile: partial dot products over this lane's 8 channels,
  // summed over lanes c and c+16 of each token with one swap + add for two
  // values at a time, then parked in LDS for the transposed read-back.
  auto qk = [&](const vec16(&kt)[LOADS]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 qv = qs[h][lane & 31];
      const uint32_t qh[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s0 = dot2(qh[0], kt[2 * j].w[0], 0.f);
        float s1 = dot2(qh[0], kt[2 * j + 1].w[0], 0.f);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          s0 = dot2(qh[w], kt[2 * j].w[w], s0);
          s1 = dot2(qh[w], kt[2 * j + 1].w[w], s1);
        }
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s1),
                                                        false, false);
        red[((rrow * C::NV) + j * G + h) * RSTRIDE + k16] =
            __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    }
  };

  // Softmax and P.V for one tile whose partial logits are in LDS.
  auto softmax_pv = [&](int j, const vec16(&vt)[LOADS]) {
    const int nvalid = min(TILE, hi - (lo + (wave + j * NW) * TILE));
    // Transposed read-back: lane -> (head, token) logit.
    float z[C::ROUNDS];
#pragma unroll
    for (int rd = 0; rd < C::ROUNDS; ++rd) {
      const int o = rd * 64 + lane;
      const int h = o >> 4, t = o & 15;
      float sum = -INFINITY;
      if (o < C::NOUT) {
        const int R = 2 * (t & 1) + ((t >> 1) & 1);
        const float4 *src = reinterpret_cast<const float4 *>(
            red + ((R * C::NV) + (t >> 2) * G + h) * RSTRIDE);
        const float4 a = src[0], b = src[1], c4 = src[2], d4 = src[3];
        sum = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)) +
              ((c4.x + c4.y) + (c4.z + c4.w)) + ((d4.x + d4.y) + (d4.z + d4.w));
        sum = t < nvalid ? sum * sl2 : -INFINITY;
      }
      z[rd] = sum;
    }
    // Tile max per head (DPP row = one head) and the lazy running-max update.
    float tmax[C::ROUNDS];
    bool need = false;
#pragma unroll
    for (int rd = 0; rd < C::ROUNDS; ++rd) {
      tmax[rd] = row_max16(z[rd]);
      need |= tmax[rd] > m_r[rd] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int rd = 0; rd < C::ROUNDS; ++rd) {
        const float mn = fmaxf(m_r[rd], tmax[rd]);
        const float a = fast_exp2(m_r[rd] - mn);
        l_r[rd] *= a;
        m_r[rd] = mn;
        const int o = rd * 64 + lane;
        if (o < C::NOUT && (o & 15) == 0) alpha_all[wave][o >> 4] = a;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float a = alpha_all[wave][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= a;
      }
    }
    // Weights (BF16-rounded), running sums, and the pair layout for P.V.
#pragma unroll
    for (int rd = 0; rd < C::ROUNDS; ++rd) {
      const int o = rd * 64 + lane;
      if (o < C::NOUT) {
        const int h = o >> 4, t = o & 15;
        const uint32_t pb = pack_bf16(fast_exp2(z[rd] - m_r[rd]));
        l_r[rd] += __uint_as_float(pb << 16);
        const int i = t >> 1;  // load index of token t
        pl16[(((t & 1) * 4 + (i >> 1)) * 8 + h) * 2 + (i & 1)] = (uint16_t)pb;
      }
    }
    // P.V on BF16 pairs of two tokens (loads 2j and 2j+1 of this lane).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pp[8];
      const uint4 p0 = *reinterpret_cast<const uint4 *>(&pl[tau][j][0]);
      const uint4 p1 = *reinterpret_cast<const uint4 *>(&pl[tau][j][4]);
      pp[0] = p0.x; pp[1] = p0.y; pp[2] = p0.z; pp[3] = p0.w;
      pp[4] = p1.x; pp[5] = p1.y; pp[6] = p1.z; pp[7] = p1.w;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t va = vt[2 * j].w[w], vb = vt[2 * j + 1].w[w];
        const uint32_t lo2 = __builtin_amdgcn_perm(vb, va, 0x05040100u);
        const uint32_t hi2 = __builtin_amdgcn_perm(vb, va, 0x07060302u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * w] = dot2(pp[h], lo2, acc[h][2 * w]);
          acc[h][2 * w + 1] = dot2(pp[h], hi2, acc[h][2 * w + 1]);
        }
      }
    }
  };

  auto load8 = [&](vec16(&kt)[LOADS], __amdgpu_buffer_rsrc_t r) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      // The whole byte offset goes in the vector offset: only the vector and
      // instruction offsets are range-checked against num_records, the
      // scalar offset is not.
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16 + i * 1024, 0, kStreamLoad);
      kt[i].w[0] = x[0];
      kt[i].w[1] = x[1];
      kt[i].w[2] = x[2];
      kt[i].w[3] = x[3];
    }
  };

  // Software pipeline over this wave's tiles with two register sets A/B and
  // a straight-line body (tiles past the last are empty resources and
  // process as no-ops): the next tile's K is requested before this tile's
  // Q.K and its V right after (reusing the registers this tile's K just
  // freed), so 8-16 KiB per wavefront are always in flight.
  vec16 ka[LOADS], va[LOADS], kb[LOADS], vb[LOADS];
  int blk1 = wave + NW < ntiles ? eid1 : 0, blk2 = wave + 2 * NW < ntiles ? eid2 : 0;
  {
    const int blk0 = wave < ntiles ? eid0 : 0;
    load8(ka, tile_rsrc(0, blk0, kpool));
    load8(va, tile_rsrc(0, blk0, vpool));
  }
  // The queries reach LDS behind the first tile's loads (their wait leaves
  // those in flight) and must be there before the first Q.K.
  if (threadIdx.x < G * 32) qs[threadIdx.x / 32][threadIdx.x % 32] = qpiece;
  __syncthreads();
  for (int j = 0; j < nj; j += 2) {
    const int blk3 = block_of(j + 3), blk4 = block_of(j + 4);
    load8(kb, tile_rsrc(j + 1, blk1, kpool));
    qk(ka);
    load8(vb, tile_rsrc(j + 1, blk1, vpool));
    softmax_pv(j, va);
    load8(ka, tile_rsrc(j + 2, blk2, kpool));
    qk(kb);
    load8(va, tile_rsrc(j + 2, blk2, vpool));
    softmax_pv(j + 1, vb);
    blk1 = blk3;
    blk2 = blk4;
  }

  // Per-head sums: each DPP row of round rd holds head rd*4 + row.
#pragma unroll
  for (int rd = 0; rd < C::ROUNDS; ++rd) l_r[rd] = row_sum16(l_r[rd]);

  // Merge the two token halves: lanes 0-31 end with channel 8c+e, lanes
  // 32-63 with channel 8c+e+1 (e even).
  float *mg = red;  // this wave's reduction buffer, reused as [G][D]
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[h][e]),
                                                      __float_as_uint(acc[h][e + 1]), false,
                                                      false);
      mg[h * D + (lane & 31) * 8 + e + tau] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
  for (int rd = 0; rd < C::ROUNDS; ++rd) {
    const int o = rd * 64 + lane;
    if (o < C::NOUT && (o & 15) == 0) {
      mg_m[wave][o >> 4] = m_r[rd];
      mg_l[wave][o >> 4] = l_r[rd];
    }
  }
  bad = __syncthreads_or(bad);

  const float nan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int ch = idx - h * D;
    float M = kNoMax;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mg_m[w][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(mg_m[w][h] - M);
      L += mg_l[w][h] * f;
      A += red_all[w][h * D + ch] * f;
    }
    if (p.partition_size == 0) {
      const float o = bad ? nan : (L > 0.f ? A / L : 0.f);
      store_out(p.out, (qrow + h) * D + ch, o, p.out_bf16);
    } else {
      const int64_t pidx = (qrow + h) * p.max_parts + part;
      p.part_out[pidx * D + ch] = bad ? nan : A / L;
      if (ch == 0) {
        p.part_max[pidx] = bad ? nan : M * kLn2;
        p.part_sum[pidx] = bad ? nan : L;
      }
    }
  }
}

template <int NW>
bool launch_tiled_nw(const DecodeParams &p, int group, unsigned grid, hipStream_t stream) {
  switch (group) {
#define PA_CASE(g) \
  case g: decode_tiled_kernel<g, NW><<<grid, NW * 64, 0, stream>>>(p); return true;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default: return false;
  }
}

}  // namespace

// Launch the tiled kernel when the shape is one it covers; false otherwise.
bool launch_decode_tiled(const DecodeParams &p, unsigned grid, hipStream_t stream) {
  if (!p.kv_bf16 || p.head_dim != D || p.block_size % TILE != 0 || p.query_start_loc)
    return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  return launch_tiled_nw<4>(p, group, grid, stream);
}

}  // namespace pa
