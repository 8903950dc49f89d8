// Paged decode attention for BF16 caches with head_dim 256 and block sizes
// that are multiples of 16 (the pages' shape: "vLLM Architecture, Memory and
// Benchmarks Deep Dive", s.1: 4 KV heads, head dimension 256, BF16; s.2:
// blocks of 16 or 32 tokens), single pass or split into context partitions.
// Same results and ABI as the generic kernel; this one is organised for
// gfx950's memory system.
//
// Work decomposition. A unit is one (sequence, KV head, partition) - or one
// (sequence, KV head) in single-pass mode - and produces one output record.
// Workgroups are persistent: one per compute unit, 8 wavefronts (two per
// SIMD). Workgroup b owns units b, b + grid, b + 2*grid, ... (at most 64);
// within a unit, 16-token tiles are dealt round-robin to the 8 wavefronts,
// whose partial softmax states are merged through LDS at the unit's end.
// With 8 wavefronts per unit and one workgroup per CU, work is spread over
// 256 slots instead of 512, which halves the imbalance of the last round.
//
// Each wavefront streams its tiles of all the workgroup's units as one
// sequence through a two-deep register ring (tile A is consumed while tile B
// is in flight; a consumed K or V set is refilled at once with the tile two
// ahead), and the stream runs across unit boundaries: the first tiles of the
// next unit are already in flight while the current unit is merged. The
// queries of the workgroup's units are staged in LDS up front, so a new unit
// starts without a dependent global load.
//
// Per tile (16 tokens of one KV head, 8 KiB of K and 8 KiB of V):
//  * Loads: eight 1 KiB wavefront buffer loads per K (or V) tile, lane l
//    getting the 8 channels 8*(l%32).. of token 2*i + l/32. The resource's
//    num_records covers only the tile's valid tokens, and the whole byte
//    offset is a vector offset (range-checked), so rows past the context
//    read as zeros without touching memory.
//  * Q.K: v_dot2_f32_bf16 on BF16 pairs; partial dot products of a token's
//    32 lanes are halved with one v_permlane16_swap + add (two values at a
//    time), then transposed through LDS so each lane ends with one
//    (head, token) logit and each 16-lane DPP row holds one head's 16 tokens.
//  * Online softmax in the exp2 domain; the running max is moved only when a
//    tile exceeds it by more than 2^8, which bounds every weight by 256 and
//    skips the accumulator rescale on almost every tile. Weights are rounded
//    to BF16 and the running sum adds the rounded weights, so numerator and
//    denominator use the same numbers.
//  * P.V: weights go through LDS as BF16 pairs of two tokens; V channels of
//    the two tokens are paired with v_perm_b32 and accumulated with
//    v_dot2_f32_bf16 into G x 8 fp32 accumulators per lane.
// Out-of-range logits are set to -inf with selects; NaN garbage in unused
// slots never reaches the arithmetic.
#include <math.h>

#include "launch.h"
#include "pa_device.h"
#include "persistent_plan.h"

namespace pa {
namespace {
using namespace persist;

constexpr int D = 256;       // head_dim
constexpr int TILE = 16;     // tokens per tile
constexpr int LOADS = 8;     // 1 KiB wavefront loads per 8 KiB K (or V) tile
constexpr int RSTRIDE = 20;  // floats per LDS reduction row (16 + pad)
constexpr int NW = 8;        // wavefronts per workgroup (two per SIMD)
constexpr float kLazy = 8.f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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


template <int G>
struct Cfg {
  static constexpr int NV = 4 * G;              // partials per lane after the row-pair step
  static constexpr int NOUT = TILE * G;         // logits per tile
  static constexpr int ROUNDS = (NOUT + 63) / 64;
  static constexpr int RED = 4 * NV * RSTRIDE;  // floats of LDS per wave (>= G * D)
  static_assert(RED >= G * D, "merge buffer must fit in the reduction buffer");
  static constexpr int FIXED = NW * RED * 4 + NW * 2 * 4 * 8 * 4 + 3 * NW * 8 * 4;
  static constexpr int NQ_FIT = (150 * 1024 - FIXED) / (G * 32 * 16);
  static constexpr int NQ = NQ_FIT > 32 ? 32 : NQ_FIT;  // query slots in LDS
  static_assert(NQ >= 4, "too little LDS left for the query slots");
};

// One tile of a wavefront's stream, as decided by the cursor. Its block id
// comes from a vector load issued when the descriptor is made (all lanes
// read the same entry) and is first used two stream positions later, when
// the tile's own loads are issued. Vector loads return in order, so waiting
// for it never waits for LDS traffic (a scalar load would: it shares the
// LDS counter and returns out of order).
struct Desc {
  int blk;      // physical block id (VGPR, pending load)
  int head;     // KV head
  int tok_off;  // token offset of the tile inside its block
  int nvalid;   // valid tokens of the tile (0: empty, loads return zeros)
};

template <int G, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_persistent_kernel(DecodeParams p) {
  using C = Cfg<G>;
  __shared__ __attribute__((aligned(16))) float red_all[NW][C::RED];
  __shared__ __attribute__((aligned(16))) uint32_t pl_all[NW][2][4][8];  // [parity][pair][head]
  __shared__ float alpha_all[NW][8];
  __shared__ float mg_m[NW][8], mg_l[NW][8];
  __shared__ int mg_bad[NW];
  __shared__ __attribute__((aligned(16))) uint4 qs[C::NQ][G][32];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tau = lane >> 5;   // token parity within a 1 KiB load
  const int rrow = lane >> 4;  // DPP row
  const int k16 = lane & 15;
  float *red = red_all[wave];
  uint32_t(*pl)[4][8] = pl_all[wave];
  uint16_t *pl16 = reinterpret_cast<uint16_t *>(pl_all[wave]);

  // ---- The workgroup's units, planned by wave 0 and shared through LDS.
  __shared__ int4 uinfo[MAXU];  // (s, h, lo, hi)
  __shared__ int ubadpart[MAXU];  // part * 2 + bad
  __shared__ uint32_t act_lds[2];
  const int S = p.num_seqs, H = p.num_kv_heads, HQ = p.num_q_heads;
  constexpr bool split = SPLIT;
  if (wave == 0) {
    int4 my{0, 0, 0, 0};
    int my_bp = 0, my_act = 0;
    plan_units<SPLIT>(p, lane, reinterpret_cast<int *>(red), my, my_bp, my_act);
    uinfo[lane] = my;
    ubadpart[lane] = my_bp;
    const uint64_t m = __builtin_amdgcn_ballot_w64(my_act != 0);
    if (lane == 0) {
      act_lds[0] = (uint32_t)m;
      act_lds[1] = (uint32_t)(m >> 32);
    }
  }
  __syncthreads();  // the plan is visible to every wave
  const uint64_t act_mask =
      (uint64_t)__builtin_amdgcn_readfirstlane(act_lds[0]) |
      ((uint64_t)__builtin_amdgcn_readfirstlane(act_lds[1]) << 32);
  if (act_mask == 0) return;  // uniform for the workgroup

  const int bs = p.block_size;
  const int64_t head_stride = (int64_t)bs * D;
  const int64_t block_stride = head_stride * H;
  const uint16_t *kpool = reinterpret_cast<const uint16_t *>(p.key_cache);
  const uint16_t *vpool = reinterpret_cast<const uint16_t *>(p.value_cache);
  // The whole block table as one buffer (the host checks it fits 2^31 bytes).
  const __amdgpu_buffer_rsrc_t tab_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(p.block_tables), (short)0,
      (int)((int64_t)S * p.max_blocks_per_seq * 4), 0x00020000);
  // Output buffers (the host checks each fits 2^31 bytes).
  const int64_t rows = (int64_t)S * HQ * (SPLIT ? p.max_parts : 1);
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      SPLIT ? (void *)p.part_out : p.out, (short)0,
      (int)(rows * D * (SPLIT ? 4 : (p.out_bf16 ? 2 : 4))), 0x00020000);
  const __amdgpu_buffer_rsrc_t max_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.part_max, (short)0, SPLIT ? (int)(rows * 4) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t sum_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.part_sum, (short)0, SPLIT ? (int)(rows * 4) : 0, 0x00020000);

  // Unit j's (s, h, lo, hi).
  auto info = [&](int j) -> int4 {
    const int4 v = uinfo[j];
    return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                     __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
  };
  // A wave's tiles of a unit of nt tiles: kk = wave, wave + NW, ...; the
  // count is padded to even with empty tiles so that stream positions
  // alternate between the A and B register sets inside every unit.
  auto padded_count = [&](int nt) {
    const int c = wave < nt ? (nt - wave + NW - 1) / NW : 0;
    return c + (c & 1);
  };

  // ---- Cursor over this wave's tile stream (uniform state).
  uint64_t cur_mask = act_mask;  // active units not yet entered
  int cur_j = -1, cur_i = 0, cur_c = 0;
  int4 cur_u{0, 0, 0, 0};
  auto advance = [&]() {
    ++cur_i;
    while (cur_i >= cur_c) {
      if (cur_mask == 0) {
        cur_j = -1;
        cur_i = 0;
        cur_c = 1 << 30;  // end of stream: stays here
        return;
      }
      cur_j = __builtin_ctzll(cur_mask);
      cur_mask &= cur_mask - 1;
      cur_u = info(cur_j);
      cur_c = padded_count((cur_u.w - cur_u.z + TILE - 1) / TILE);
      cur_i = 0;
    }
  };
  auto make_desc = [&]() -> Desc {
    Desc d{0, 0, 0, 0};
    const int tok0 = cur_u.z + (wave + cur_i * NW) * TILE;
    // The id load is issued on every path (an empty tile reads past the
    // table's num_records, which returns 0 without an access): the same
    // number of vector loads on every path keeps the compiler's wait
    // counts exact across the loop.
    int entry_off = 0x7ffffff0;
    if (cur_j >= 0 && tok0 < cur_u.w) {
      entry_off = (cur_u.x * p.max_blocks_per_seq + tok0 / bs) * 4;
      d.head = cur_u.y;
      d.tok_off = tok0 % bs;
      d.nvalid = min(TILE, cur_u.w - tok0);
    }
    d.blk = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, entry_off, 0, 0);
    return d;
  };
  // Buffer resources over the valid rows of one tile of a pool, one per
  // 4 KiB half (tokens 0-7 and 8-15), so that the per-load offsets fit the
  // instruction's immediate field and one VGPR holds the lane offset. Rows
  // past the context lie outside num_records and read as zeros. An invalid
  // block id gives empty resources (zeros, no access) and marks the tile.
  struct TileRsrc {
    __amdgpu_buffer_rsrc_t lo, hi;
  };
  auto tile_rsrc = [&](const Desc &d, const uint16_t *pool, int &nvalid, int &bad) {
    int blk = __builtin_amdgcn_readfirstlane(d.blk), n = d.nvalid;
    bad = 0;
    if (n > 0 && (blk < 0 || blk >= p.num_blocks)) {
      bad = 1;
      n = 0;
    }
    if (n <= 0) blk = 0;
    nvalid = n;
    const uint16_t *base =
        pool + (int64_t)blk * block_stride + (int64_t)d.head * head_stride + (int64_t)d.tok_off * D;
    const int n_lo = n < 8 ? n : 8, n_hi = n > 8 ? n - 8 : 0;
    TileRsrc r;
    r.lo = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0,
                                             n_lo * D * 2, 0x00020000);
    r.hi = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base + 8 * D), (short)0,
                                             n_hi * D * 2, 0x00020000);
    return r;
  };
  const int lane_off = lane * 16;
  auto load8 = [&](vec16(&kt)[LOADS], const TileRsrc &r) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      // Vector offset + immediate offset: both are range-checked against
      // num_records (the scalar offset would not be).
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
          i < 4 ? r.lo : r.hi, lane_off + (i & 3) * 1024, 0, kStreamLoad);
      kt[i].w[0] = x[0];
      kt[i].w[1] = x[1];
      kt[i].w[2] = x[2];
      kt[i].w[3] = x[3];
    }
  };

  // Prime the ring with the stream's first two tiles, and load the block ids
  // of the next two, in the same order as the loop body issues them (tile,
  // id two ahead, tile, id two ahead), so the compiler's wait counts inside
  // the loop are the steady-state ones from the first iteration on.
  vec16 ka[LOADS], va[LOADS], kb[LOADS], vb[LOADS];
  int nv_a, nv_b, bad_a, bad_b;
  Desc dn, dn2;  // descriptors of the tiles two and three positions ahead
  {
    cur_i = -1;
    advance();
    const Desc d0 = make_desc();
    advance();
    const Desc d1 = make_desc();
    load8(ka, tile_rsrc(d0, kpool, nv_a, bad_a));
    load8(va, tile_rsrc(d0, vpool, nv_a, bad_a));
    advance();
    dn = make_desc();
    load8(kb, tile_rsrc(d1, kpool, nv_b, bad_b));
    load8(vb, tile_rsrc(d1, vpool, nv_b, bad_b));
    advance();
    dn2 = make_desc();
  }

  // Stage the queries of the first NQ active units in LDS.
  auto stage_queries = [&](uint64_t mask) {
    for (int k = 0; k < C::NQ && mask != 0; ++k) {
      const int j = __builtin_ctzll(mask);
      mask &= mask - 1;
      const int4 uj = info(j);
      const int64_t qrow = (int64_t)uj.x * HQ + (int64_t)uj.y * G;
      for (int i = threadIdx.x; i < G * 32; i += NW * 64) {
        const vec16 v =
            load16(reinterpret_cast<const uint16_t *>(p.query) + (qrow + i / 32) * D + (i % 32) * 8);
        qs[k][i / 32][i % 32] = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
      }
    }
  };
  stage_queries(act_mask);
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  float acc[G][8];
  float m_r[C::ROUNDS], l_r[C::ROUNDS];

  // Q.K for one tile: partial dot products over this lane's 8 channels,
  // summed over lanes c and c+16 of each token with one swap + add for two
  // values at a time, then parked in LDS for the transposed read-back.
  auto qk = [&](const vec16(&kt)[LOADS], int qslot) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 qv = qs[qslot][h][lane & 31];
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
  auto softmax_pv = [&](int nvalid, const vec16(&vt)[LOADS]) {
    float z[C::ROUNDS];
#pragma unroll
    for (int rd = 0; rd < C::ROUNDS; ++rd) {
      const int o = rd * 64 + lane;
      const int h = o >> 4, t = o & 15;
      float sum = -INFINITY;
      if (o < C::NOUT) {
        const int R = 2 * (t & 1) + ((t >> 1) & 1);
        const float4 *src =
            reinterpret_cast<const float4 *>(red + ((R * C::NV) + (t >> 2) * G + h) * RSTRIDE);
        const float4 a = src[0], b = src[1], c4 = src[2], d4 = src[3];
        sum = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)) +
              ((c4.x + c4.y) + (c4.z + c4.w)) + ((d4.x + d4.y) + (d4.z + d4.w));
        sum = t < nvalid ? sum * sl2 : -INFINITY;
      }
      z[rd] = sum;
    }
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
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pp[8];
      const uint4 p0 = *reinterpret_cast<const uint4 *>(&pl[tau][j][0]);
      const uint4 p1 = *reinterpret_cast<const uint4 *>(&pl[tau][j][4]);
      pp[0] = p0.x; pp[1] = p0.y; pp[2] = p0.z; pp[3] = p0.w;
      pp[4] = p1.x; pp[5] = p1.y; pp[6] = p1.z; pp[7] = p1.w;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t va_ = vt[2 * j].w[w], vb_ = vt[2 * j + 1].w[w];
        const uint32_t lo2 = __builtin_amdgcn_perm(vb_, va_, 0x05040100u);
        const uint32_t hi2 = __builtin_amdgcn_perm(vb_, va_, 0x07060302u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * w] = dot2(pp[h], lo2, acc[h][2 * w]);
          acc[h][2 * w + 1] = dot2(pp[h], hi2, acc[h][2 * w + 1]);
        }
      }
    }
  };

  const float nan = __builtin_nanf("");
  int kq = 0;  // ordinal of the unit among the active ones (query slot)
  uint64_t todo = act_mask;
  while (todo != 0) {
    const int j = __builtin_ctzll(todo);
    todo &= todo - 1;
    if (__builtin_expect(kq == C::NQ, 0)) {
      // More units than query slots: every wave is between units (after the
      // merge barriers below), so the slots can be refilled.
      stage_queries(todo | (1ull << j));
      __syncthreads();
      kq = 0;
    }
    const int qslot = kq++;
    const int4 uj = info(j);
    const int cpad = padded_count((uj.w - uj.z + TILE - 1) / TILE);
    int ubad = __builtin_amdgcn_readfirstlane(ubadpart[j]) & 1;

#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int r = 0; r < C::ROUNDS; ++r) {
      m_r[r] = kNoMax;
      l_r[r] = 0.f;
    }

    // Two stream positions per iteration: A, then B. Empty tiles (padding or
    // past a short unit) skip the arithmetic but keep the ring moving.
    for (int i = 0; i < cpad; i += 2) {
      int nvn, badn;
      if (nv_a > 0) qk(ka, qslot);
      load8(ka, tile_rsrc(dn, kpool, nvn, badn));
      if (nv_a > 0) softmax_pv(nv_a, va);
      ubad |= bad_a;
      load8(va, tile_rsrc(dn, vpool, nv_a, bad_a));
      dn = dn2;
      advance();
      dn2 = make_desc();

      if (nv_b > 0) qk(kb, qslot);
      load8(kb, tile_rsrc(dn, kpool, nvn, badn));
      if (nv_b > 0) softmax_pv(nv_b, vb);
      ubad |= bad_b;
      load8(vb, tile_rsrc(dn, vpool, nv_b, bad_b));
      dn = dn2;
      advance();
      dn2 = make_desc();
    }

    // Merge this wave's two token halves and park the state in LDS.
#pragma unroll
    for (int rd = 0; rd < C::ROUNDS; ++rd) l_r[rd] = row_sum16(l_r[rd]);
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
    if (lane == 0) mg_bad[wave] = ubad;
    __syncthreads();
    int anybad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) anybad |= mg_bad[w];
    const bool bad = anybad != 0;

    // All waves together merge the unit's 8 partial states and store it.
    // Every thread issues the same, fixed number of buffer stores; stores
    // that must not happen get an offset past num_records and are dropped.
    // A fixed store count keeps the compiler's wait counts exact for the
    // loads already in flight for the next unit.
    const int64_t qrow = (int64_t)uj.x * HQ + (int64_t)uj.y * G;
    const int part = __builtin_amdgcn_readfirstlane(ubadpart[j]) >> 1;
    constexpr int ITER = (G * D + NW * 64 - 1) / (NW * 64);
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = threadIdx.x + it * NW * 64;
      const bool live = idx < G * D;
      const int h = live ? idx / D : 0;
      const int ch = idx - h * D;
      float M = kNoMax;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mg_m[w][h]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(mg_m[w][h] - M);
        L += mg_l[w][h] * f;
        A += red_all[w][(live ? idx : 0)] * f;
      }
      constexpr int kDrop = 0x7ffffff0;
      if constexpr (!split) {
        const float o = bad ? nan : (L > 0.f ? A / L : 0.f);
        const int64_t e = (qrow + h) * D + ch;
        if (p.out_bf16)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(o), out_rsrc, live ? (int)(e * 2) : kDrop,
                                                0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), out_rsrc,
                                                live ? (int)(e * 4) : kDrop, 0, 0);
      } else {
        const int64_t pidx = (qrow + h) * p.max_parts + part;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : A / L), out_rsrc,
                                              live ? (int)((pidx * D + ch) * 4) : kDrop, 0, 0);
        const int moff = (live && ch == 0) ? (int)(pidx * 4) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : M * kLn2), max_rsrc, moff,
                                              0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : L), sum_rsrc, moff, 0, 0);
      }
    }
    __syncthreads();  // the reduction buffers are reused by the next unit
  }
}


}  // namespace

// Launch the persistent kernel when the shape is one it covers; false
// otherwise (the caller then uses the generic kernel).
bool launch_decode_persistent(const DecodeParams &p, hipStream_t stream) {
  if (!p.kv_bf16 || p.head_dim != D || p.block_size % TILE != 0 || p.query_start_loc)
    return false;
  if (p.partition_size > 0 && p.partition_size % TILE != 0) return false;
  if ((int64_t)p.num_seqs * p.max_blocks_per_seq * 4 > 0x7fffffff) return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  const int64_t parts = p.partition_size > 0 ? p.max_parts : 1;
  const int64_t units = parts * p.num_seqs * p.num_kv_heads;
  if (units <= 0 || units > 0x7fffffff) return false;
  int64_t grid = num_cus();
  // Split mode takes the tiled kernel (a workgroup per unit, two per CU,
  // balanced by the hardware dispatcher) when the persistent one cannot pay
  // for its planner and ring: with at most one unit per CU, or with
  // partitions under 2 tiles per wavefront, where padding every wavefront's
  // share of a unit to an even count would leave half the ring empty.
  if (p.partition_size > 0 && (units <= grid || p.partition_size < 2 * NW * TILE)) return false;
  if (grid > units) grid = units;
  if (grid * MAXU < units) return false;  // more than 64 units per workgroup
  const int64_t out_bytes = (int64_t)p.num_seqs * p.num_q_heads * parts * D *
                            (p.partition_size > 0 ? 4 : (p.out_bf16 ? 2 : 4));
  if (out_bytes > 0x7fff0000) return false;
  const bool split = p.partition_size > 0;
  switch (group) {
#define PA_CASE(g)                                                                        \
  case g:                                                                                 \
    if (split)                                                                            \
      decode_persistent_kernel<g, true><<<(unsigned)grid, NW * 64, 0, stream>>>(p); \
    else                                                                                  \
      decode_persistent_kernel<g, false><<<(unsigned)grid, NW * 64, 0, stream>>>(p); \
    return true;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default: return false;
  }
}

}  // namespace pa
