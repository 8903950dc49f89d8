// Paged decode attention over FP8 (E4M3FN) pools on the matrix cores,
// head_dim 256, block sizes that are multiples of 16, single pass or split
// into context partitions (multiples of 32 tokens). Same results and ABI as
// the generic kernel's FP8 path.
//
// Why matrix cores here: a one-byte cache halves the bytes decode streams
// ("Optimizing LLM Inference", KV-cache section: the cache size is linear in
// the bytes per element; "vLLM Architecture, Memory and Benchmarks Deep
// Dive", s.1: decode is bound by memory traffic), and with half the bytes
// the vector-unit arithmetic of the BF16 kernel (one v_dot2 per channel pair
// per query head, plus the cross-lane sums) would take longer than the
// loads. Q.K and P.V of a 32-token tile are two small contractions (16
// padded query heads x 256 channels x 32 tokens), which v_mfma_f32_16x16x32
// _bf16 does in 32 instructions.
//
// Work decomposition and streaming are those of the BF16 matrix-core kernel:
// one 8-wave workgroup per compute unit owns up to 64 units (planned on the
// device from the context lengths), each wave streams its tiles of all of
// them through a two-deep register ring, and the 8 waves' partial softmax
// states of a unit are merged through LDS.
//
// Per tile (32 tokens of one KV head: two 16-token halves, each inside one
// block, 8 KiB of K codes and 8 KiB of V codes):
//  * K (rows [token][256]) is the A operand of S^T = K . Q^T: lane (m, g)
//    (m = lane % 16, g = lane / 16) needs, for j = 0..3, the 16 bytes of
//    token row m at byte 16g + 64j. Loaded that way, one wavefront load
//    would read 64-byte halves of 16 different 128-byte lines; instead each
//    load reads whole lines of 8 rows (lane (m, g): row 8i + m % 8, byte
//    128p + 16g + 64 (m / 8)), and a DPP rotation by 8 lanes within each
//    16-lane row exchanges the halves so that every lane holds its own row's
//    pieces. Rows past the context lie outside the load's range and read as
//    zeros. Each 16-byte piece feeds two MFMA steps of 8 channels; the query
//    fragment of a step (B operand, lane (head n, g)) takes the same
//    channels 64j + 16g + 8h .. +7, so the contraction pairs every channel
//    once. Columns beyond the group repeat real heads and are never stored.
//  * The accumulator gives lane (n, g) the logits of head n for tokens
//    4g .. 4g+3 of each half: softmax is per-lane work plus two lane swaps
//    (v_permlane16_swap, v_permlane32_swap) for the max and the sum. Online
//    softmax in the exp2 domain with a lazy running max (rescale only when
//    a tile raises it by more than 2^8); weights rounded to BF16, and the
//    running sum adds the rounded weights.
//  * O^T = V^T . P^T. The value pool stores each block transposed
//    ([head_dim][block_size]), so the 16 tokens of one half at one channel
//    are 16 adjacent codes: lane (c, g) loads them for channel 16 X + c of
//    half g & 1, X = 2L + (g >> 1), L = 0..7 (eight 16-byte loads per tile,
//    with per-lane addresses since the halves sit in different blocks). One
//    v_permlane32_swap per dword pair then leaves every lane with 8 tokens
//    of one channel for block 2L and 8 for block 2L+1: group g holds tile
//    tokens 8 * (2 (g & 1) + (g >> 1)) .. +7. One v_permlane16_swap gives
//    the weights the same token order (B operand). Codes of tokens past the
//    context are masked to zero before widening (0 x NaN garbage would
//    poison the sum).
//  * Codes widen to BF16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1); the
//    K scale folds into the logit scale and the V scale into the outputs.
#include <math.h>

#include "launch.h"
#include "pa_device.h"
#include "persistent_plan.h"

namespace pa {
namespace {
using namespace persist;

constexpr int D = 256;     // head_dim
constexpr int TILE = 32;   // tokens per tile
constexpr int HALF = 16;   // tokens per half tile (inside one block)
constexpr int NW = 8;      // wavefronts per workgroup (two per SIMD)
static_assert(NW == persist::kPlanWaves, "the planner's unit costs count 8 waves");
constexpr int KL = 8;      // 16-byte K loads per lane per tile
constexpr int VL = 8;      // 16-byte V loads per lane per tile (two channel blocks each)
// LDS row strides padded by 16 bytes so that the rows of different query
// heads start on different banks: a query row of 32 x 16 bytes (read 16
// lanes at a time, one head per lane, the same channels) and a parked merge
// row of D floats (written one head per lane).
constexpr int QROW = 33;      // uint4 per query row
constexpr int RSTR = D + 4;   // floats per parked merge row
constexpr float kLazy = 8.f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two E4M3 codes (bytes 2*HI, 2*HI+1 of w) as a BF16 pair, lower byte in the
// lower half.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight codes (four in lo, four in hi) as an 8-element BF16 operand.
__device__ __forceinline__ u32x4 widen8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = cvt2<false>(lo);
  r[1] = cvt2<true>(lo);
  r[2] = cvt2<false>(hi);
  r[3] = cvt2<true>(hi);
  return r;
}

__device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Reductions over the four lanes n, n+16, n+32, n+48 (the groups g of one
// head column): a swap of 16-lane rows, then of 32-lane halves.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Byte mask of the codes of tokens 4g .. 4g+3 of a half holding n valid
// tokens.
__device__ __forceinline__ uint32_t half_mask(int n, int g) {
  const int c = n - 4 * g;
  return c >= 4 ? 0xffffffffu : (c <= 0 ? 0u : (1u << (8 * c)) - 1u);
}

template <int G>
struct Cfg8 {
  static constexpr int MERGE = NW * G * RSTR * 4;  // bytes of the merge buffers
  static constexpr int FIXED = MERGE + 4096;
  static constexpr int NQ_FIT = (150 * 1024 - FIXED) / (G * QROW * 16);
  static constexpr int NQ = NQ_FIT > 32 ? 32 : NQ_FIT;  // query slots in LDS
  static_assert(NQ >= 4, "too little LDS left for the query slots");
  static_assert(G * D >= 192, "the planner needs 192 ints of scratch");
};

// One tile of a wave's stream (see the BF16 kernel's Desc): the block ids
// of its two halves come from vector loads issued when the descriptor is
// made and first used two stream positions later.
struct Desc8 {
  int blk0, blk1;  // physical block ids (VGPRs, pending loads)
  int head;        // KV head
  int off0, off1;  // token offsets of the halves inside their blocks
  int nvalid;      // valid tokens of the tile (0: empty, loads return zeros)
};

// Plan-cache kind of this kernel's slots (the two halves' block ids of each
// wave's first two tiles).
constexpr uint32_t kPlanKindFp8 = 0x200;

template <int G, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_fp8_kernel(DecodeParams p) {
  using C = Cfg8<G>;
  __shared__ __attribute__((aligned(16))) float red_all[NW][G * RSTR];
  __shared__ float mg_m[NW][8], mg_l[NW][8];
  __shared__ int mg_bad[NW];
  __shared__ __attribute__((aligned(16))) uint4 qs[C::NQ][G][QROW];
  __shared__ int4 uinfo[MAXU];     // (s, h, lo, hi)
  __shared__ int ubadpart[MAXU];   // part * 4 + bad (no step tokens here)
  __shared__ uint32_t act_lds[3];  // active-unit mask, and whether the plan slot is used

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;  // A row / B column / accumulator column
  const int grp = lane >> 4;  // k group / accumulator row group
  float *red = red_all[wave];

  const int S = p.num_seqs, H = p.num_kv_heads, HQ = p.num_q_heads;
  // With a plan buffer: the slot, this wave's first four block ids and (wave
  // 0) the units, loaded together when the slot's tag names this launch.
  const PlanSlot ps = plan_slot<SPLIT>(p, kPlanKindFp8, wave, wave == 0);
  int pre_id[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pre_id[k] = (int)ps.ids[k];
  if (wave == 0) {
    int4 my{0, 0, 0, 0};
    int my_bp = 0, my_act = 0;
    plan_or_load_units<SPLIT, TILE>(p, ps, lane, reinterpret_cast<int *>(red), my, my_bp, my_act);
    uinfo[lane] = my;
    ubadpart[lane] = my_bp;
    const uint64_t m = __builtin_amdgcn_ballot_w64(my_act != 0);
    if (lane == 0) {
      act_lds[0] = (uint32_t)m;
      act_lds[1] = (uint32_t)(m >> 32);
      act_lds[2] = ps.use ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint64_t act_mask =
      (uint64_t)__builtin_amdgcn_readfirstlane(act_lds[0]) |
      ((uint64_t)__builtin_amdgcn_readfirstlane(act_lds[1]) << 32);
  // Wave 0's reading of the slot decides for the workgroup: it may rewrite
  // the slot's tag before a later wave reads it, and each wave's own ids in
  // the slot are as the launch that wrote the tag left them.
  const bool use_plan = __builtin_amdgcn_readfirstlane(act_lds[2]) != 0;
  if (act_mask == 0) return;  // uniform for the workgroup

  const int bs = p.block_size;
  const int64_t head_stride = (int64_t)bs * D;  // bytes, both pools
  const int64_t block_stride = head_stride * H;
  const uint8_t *kpool = reinterpret_cast<const uint8_t *>(p.key_cache);
  const uint8_t *vpool = reinterpret_cast<const uint8_t *>(p.value_cache);
  const __amdgpu_buffer_rsrc_t tab_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(p.block_tables), (short)0,
      (int)((int64_t)S * p.max_blocks_per_seq * 4), 0x00020000);
  const int64_t rows = (int64_t)S * HQ * (SPLIT ? p.max_parts : 1);
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      SPLIT ? (void *)p.part_out : p.out, (short)0,
      (int)(rows * D * (SPLIT ? 4 : (p.out_bf16 ? 2 : 4))), 0x00020000);
  const __amdgpu_buffer_rsrc_t max_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.part_max, (short)0, SPLIT ? (int)(rows * 4) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t sum_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.part_sum, (short)0, SPLIT ? (int)(rows * 4) : 0, 0x00020000);

  auto info = [&](int j) -> int4 {
    const int4 v = uinfo[j];
    return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                     __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
  };
  auto padded_count = [&](int nt) {
    const int c = wave < nt ? (nt - wave + NW - 1) / NW : 0;
    return c + (c & 1);
  };

  // ---- Cursor over this wave's tile stream (uniform state).
  uint64_t cur_mask = act_mask;
  int cur_j = -1, cur_i = 0, cur_c = 0;
  int4 cur_u{0, 0, 0, 0};
  auto advance = [&]() {
    ++cur_i;
    while (cur_i >= cur_c) {
      if (cur_mask == 0) {
        cur_j = -1;
        cur_i = 0;
        cur_c = 1 << 30;
        return;
      }
      cur_j = __builtin_ctzll(cur_mask);
      cur_mask &= cur_mask - 1;
      cur_u = info(cur_j);
      cur_c = padded_count((cur_u.w - cur_u.z + TILE - 1) / TILE);
      cur_i = 0;
    }
  };
  // pre >= 0: the ids were preloaded from the plan (stream position pre).
  auto make_desc = [&](int pre = -1) -> Desc8 {
    Desc8 d{0, 0, 0, 0, 0, 0};
    const int tok0 = cur_u.z + (wave + cur_i * NW) * TILE;
    // Both id loads are issued on every path (an absent half reads past the
    // table's num_records, which returns 0 without an access).
    int e0 = 0x7ffffff0, e1 = 0x7ffffff0;
    if (cur_j >= 0 && tok0 < cur_u.w) {
      const int row = cur_u.x * p.max_blocks_per_seq;
      d.head = cur_u.y;
      d.nvalid = min(TILE, cur_u.w - tok0);
      e0 = (row + tok0 / bs) * 4;
      d.off0 = tok0 % bs;
      if (d.nvalid > HALF) {
        e1 = (row + (tok0 + HALF) / bs) * 4;
        d.off1 = (tok0 + HALF) % bs;
      }
    }
    if (pre >= 0) {
      d.blk0 = pre ? pre_id[2] : pre_id[0];
      d.blk1 = pre ? pre_id[3] : pre_id[1];
    } else {
      d.blk0 = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, e0, 0, 0);
      d.blk1 = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, e1, 0, 0);
    }
    return d;
  };
  // Valid tokens and block ids of the two halves; an invalid id empties its
  // half (zeros, no access) and marks the tile.
  struct Halves {
    int b0, b1, n0, n1, bad;
  };
  auto halves = [&](const Desc8 &d) {
    Halves r;
    r.b0 = __builtin_amdgcn_readfirstlane(d.blk0);
    r.b1 = __builtin_amdgcn_readfirstlane(d.blk1);
    r.n0 = min(d.nvalid, HALF);
    r.n1 = d.nvalid > HALF ? d.nvalid - HALF : 0;
    r.bad = 0;
    if (r.n0 > 0 && (r.b0 < 0 || r.b0 >= p.num_blocks)) {
      r.bad = 1;
      r.n0 = 0;
    }
    if (r.n1 > 0 && (r.b1 < 0 || r.b1 >= p.num_blocks)) {
      r.bad = 1;
      r.n1 = 0;
    }
    if (r.n0 <= 0) r.b0 = 0;
    if (r.n1 <= 0) r.b1 = 0;
    return r;
  };
  // lane's byte offset in a K half: row m % 8 (+ 8 for the second load of a
  // pair), byte 16g + 64 (m / 8) (+ 128 for the second pair)
  const int koff = (n16 & 7) * D + 16 * grp + 64 * (n16 >> 3);
  // lane's byte offset from its V half's base: channel 16 (g >> 1) + c
  const int64_t voff = (int64_t)(16 * (grp >> 1) + n16) * bs;
  auto load_k = [&](u32x4(&kt)[KL], const Desc8 &d) {
    const Halves hv = halves(d);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int blk = h ? hv.b1 : hv.b0, off = h ? d.off1 : d.off0, n = h ? hv.n1 : hv.n0;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t *>(kpool + (int64_t)blk * block_stride +
                                (int64_t)d.head * head_stride + (int64_t)off * D),
          (short)0, n * D, 0x00020000);
#pragma unroll
      for (int j = 0; j < 4; ++j)  // load 2p + i: bytes 128p.. of rows 8i..8i+7
        kt[4 * h + j] = __builtin_amdgcn_raw_buffer_load_b128(
            r, koff + (j & 1) * 8 * D + (j >> 1) * 128, 0, kStreamLoad);
    }
  };
  // V codes: vt[L] holds tokens 0..15 of half g & 1 at channel
  // 16 (2L + (g >> 1)) + c. Every address lies in the head's slab of a
  // block: an empty or invalid half reads block 0 instead, and its codes
  // are masked to zero before use.
  auto load_v = [&](u32x4(&vt)[VL], const Desc8 &d, int &nvalid, int &bad) {
    const Halves hv = halves(d);
    nvalid = hv.n0 + hv.n1 > 0 ? d.nvalid : 0;
    bad = hv.bad;
    const bool h1 = (grp & 1) != 0;
    const int blk = h1 ? hv.b1 : hv.b0;
    const int off = h1 ? (hv.n1 > 0 ? d.off1 : 0) : (hv.n0 > 0 ? d.off0 : 0);
    const uint8_t *base =
        vpool + (int64_t)blk * block_stride + (int64_t)d.head * head_stride + off + voff;
#pragma unroll
    for (int L = 0; L < VL; ++L)
      vt[L] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + (int64_t)L * 32 * bs));
  };

  // Prime the ring (same issue order as the loop body).
  u32x4 ka[KL], kb[KL];
  u32x4 va[VL], vb[VL];
  int nv_a, nv_b, bad_a, bad_b;
  Desc8 dn, dn2;
  {
    cur_i = -1;
    advance();
    const Desc8 d0 = make_desc(use_plan ? 0 : -1);
    advance();
    const Desc8 d1 = make_desc(use_plan ? 1 : -1);
    load_k(ka, d0);
    load_v(va, d0, nv_a, bad_a);
    advance();
    dn = make_desc();
    load_k(kb, d1);
    load_v(vb, d1, nv_b, bad_b);
    advance();
    dn2 = make_desc();
    plan_store_id(ps, use_plan, wave, 0, lane, d0.blk0);
    plan_store_id(ps, use_plan, wave, 1, lane, d0.blk1);
    plan_store_id(ps, use_plan, wave, 2, lane, d1.blk0);
    plan_store_id(ps, use_plan, wave, 3, lane, d1.blk1);
  }

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

  const float sl2 = p.scale * kLog2e * p.k_scale;
  const float vsc = p.v_scale;
  f32x4 o[16];
  float m_run, l_run;
  // Columns n >= G repeat query head n % G: MFMA columns do not mix, those
  // columns are never stored, and their maxima equal a real head's, so they
  // trigger no extra rescales.
  const bool live_head = n16 < G;
  const int qh = n16 % G;

  // S^T, softmax and the weights (B operand of P.V) for one tile.
  auto qk_softmax = [&](const u32x4(&kraw)[KL], int qslot, int nvalid) -> u32x4 {
    // Loads 2p, 2p+1 of a half give lane m < 8 row m's piece j = 2p and lane
    // m >= 8 row m's piece j = 2p+1; each lane takes the piece it lacks from
    // its partner m ^ 8 (row rotation by 8) and keeps its own. The rotation
    // writes only the receiving half of each 16-lane row (DPP bank mask:
    // lanes 8-15 = banks 2, 3; lanes 0-7 = banks 0, 1), so the other half
    // keeps the old value, its own piece, and no selects are needed.
    u32x4 kt[KL];
#pragma unroll
    for (int hp = 0; hp < 4; ++hp) {
      const u32x4 v0 = kraw[2 * hp], v1 = kraw[2 * hp + 1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kt[2 * hp][w] =
            (uint32_t)__builtin_amdgcn_update_dpp((int)v0[w], (int)v1[w], 0x128, 0xf, 0xc, false);
        kt[2 * hp + 1][w] =
            (uint32_t)__builtin_amdgcn_update_dpp((int)v1[w], (int)v0[w], 0x128, 0xf, 0x3, false);
      }
    }
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 q4 = qs[qslot][qh][8 * j + 2 * grp + h];
        u32x4 qb;
        qb[0] = q4.x;
        qb[1] = q4.y;
        qb[2] = q4.z;
        qb[3] = q4.w;
        s0 = mfma(widen8(kt[j][2 * h], kt[j][2 * h + 1]), qb, s0);
        s1 = mfma(widen8(kt[4 + j][2 * h], kt[4 + j][2 * h + 1]), qb, s1);
      }
    }
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = 4 * grp + r < nvalid ? s0[r] * sl2 : -INFINITY;
      z[4 + r] = HALF + 4 * grp + r < nvalid ? s1[r] * sl2 : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = group_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
      const float mn = fmaxf(m_run, mx);
      const float a = fast_exp2(m_run - mn);
      l_run *= a;
      m_run = mn;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[cb][r] *= a;
    }
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = bf16_pair(fast_exp2(z[2 * u] - m_run), fast_exp2(z[2 * u + 1] - m_run));
      l_run += __uint_as_float(w[u] << 16) + __uint_as_float(w[u] & 0xffff0000u);
    }
    // w[0..1]: tokens 4g..4g+3 of half 0, w[2..3]: of half 1. Row swap to the
    // value operand's order: group g gets tokens 8 (2 (g & 1) + (g >> 1)) .. +7.
    const auto x = __builtin_amdgcn_permlane16_swap(w[0], w[2], false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(w[1], w[3], false, false);
    u32x4 pb;
    pb[0] = x[0];
    pb[1] = y[0];
    pb[2] = x[1];
    pb[3] = y[1];
    return pb;
  };
  // O^T += V^T . P^T for one tile.
  auto pv = [&](const u32x4(&vt)[VL], const u32x4 &pb, int nvalid) {
    const int n = (grp & 1) ? nvalid - HALF : min(nvalid, HALF);  // valid tokens of my half
    uint32_t mk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) mk[k] = half_mask(n, k);
#pragma unroll
    for (int L = 0; L < VL; ++L) {
      // Rows 0,1 hold block 2L, rows 2,3 block 2L+1 (halves 0,1); the swap
      // of the upper dword pair of rows 0,1 with the lower of rows 2,3 gives
      // each lane 8 tokens of both blocks.
      const auto x = __builtin_amdgcn_permlane32_swap(vt[L][0] & mk[0], vt[L][2] & mk[2], false,
                                                      false);
      const auto y = __builtin_amdgcn_permlane32_swap(vt[L][1] & mk[1], vt[L][3] & mk[3], false,
                                                      false);
      o[2 * L] = mfma(widen8(x[0], y[0]), pb, o[2 * L]);
      o[2 * L + 1] = mfma(widen8(x[1], y[1]), pb, o[2 * L + 1]);
    }
  };

  const float nan = __builtin_nanf("");
  int kq = 0;
  uint64_t todo = act_mask;
  while (todo != 0) {
    const int j = __builtin_ctzll(todo);
    todo &= todo - 1;
    if (__builtin_expect(kq == C::NQ, 0)) {
      stage_queries(todo | (1ull << j));
      __syncthreads();
      kq = 0;
    }
    const int qslot = kq++;
    const int4 uj = info(j);
    const int cpad = padded_count((uj.w - uj.z + TILE - 1) / TILE);
    int ubad = __builtin_amdgcn_readfirstlane(ubadpart[j]) & 1;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNoMax;
    l_run = 0.f;

    for (int i = 0; i < cpad; i += 2) {
      int nvn, badn;
      u32x4 pb{0u, 0u, 0u, 0u};
      if (nv_a > 0) pb = qk_softmax(ka, qslot, nv_a);
      load_k(ka, dn);
      if (nv_a > 0) pv(va, pb, nv_a);
      ubad |= bad_a;
      load_v(va, dn, nv_a, bad_a);
      dn = dn2;
      advance();
      dn2 = make_desc();

      if (nv_b > 0) pb = qk_softmax(kb, qslot, nv_b);
      load_k(kb, dn);
      if (nv_b > 0) pv(vb, pb, nv_b);
      ubad |= bad_b;
      load_v(vb, dn, nv_b, bad_b);
      dn = dn2;
      advance();
      dn2 = make_desc();
      (void)nvn;
      (void)badn;
    }

    // Park this wave's state: sum of the weights over the four groups,
    // accumulator rows 4g + r of channel block cb -> channel 16 cb + 4g + r.
    const float l_tot = group_sum(l_run);
    if (live_head) {
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
        *reinterpret_cast<float4 *>(&red[n16 * RSTR + 16 * cb + 4 * grp]) =
            make_float4(o[cb][0], o[cb][1], o[cb][2], o[cb][3]);
      if (grp == 0) {
        mg_m[wave][n16] = m_run;
        mg_l[wave][n16] = l_tot;
      }
    }
    if (lane == 0) mg_bad[wave] = ubad;
    __syncthreads();
    int anybad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) anybad |= mg_bad[w];
    const bool bad = anybad != 0;

    // All waves merge the unit's 8 partial states and store it (fixed store
    // count; stores that must not happen fall past num_records).
    const int64_t qrow = (int64_t)uj.x * HQ + (int64_t)uj.y * G;
    const int part = __builtin_amdgcn_readfirstlane(ubadpart[j]) >> 2;
    constexpr int ITER = (G * D + NW * 64 - 1) / (NW * 64);
#pragma unroll 1
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
        A += red_all[w][live ? h * RSTR + ch : 0] * f;
      }
      constexpr int kDrop = 0x7ffffff0;
      if constexpr (!SPLIT) {
        const float ov = bad ? nan : (L > 0.f ? A / L * vsc : 0.f);
        const int64_t e = (qrow + h) * D + ch;
        if (p.out_bf16)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(ov), out_rsrc,
                                                live ? (int)(e * 2) : kDrop, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), out_rsrc,
                                                live ? (int)(e * 4) : kDrop, 0, 0);
      } else {
        const int64_t pidx = (qrow + h) * p.max_parts + part;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : A / L * vsc), out_rsrc,
                                              live ? (int)((pidx * D + ch) * 4) : kDrop, 0, 0);
        const int moff = (live && ch == 0) ? (int)(pidx * 4) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : M * kLn2), max_rsrc,
                                              moff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : L), sum_rsrc, moff, 0,
                                              0);
      }
    }
    __syncthreads();  // the merge buffers are reused by the next unit
  }
}

}  // namespace

// Launch the FP8 matrix-core kernel when the shape is one it covers; false
// otherwise (the caller then uses the generic kernel).
bool launch_decode_fp8(const DecodeParams &p, hipStream_t stream) {
  if (!p.kv_fp8 || p.head_dim != D || p.block_size % HALF != 0 || p.query_start_loc || p.new_key)
    return false;
  if (p.partition_size > 0 && p.partition_size % TILE != 0) return false;
  if ((int64_t)p.num_seqs * p.max_blocks_per_seq * 4 > 0x7fffffff) return false;
  if ((int64_t)p.block_size * D * p.num_kv_heads * p.num_blocks > ((int64_t)1 << 47)) return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  const int64_t parts = p.partition_size > 0 ? p.max_parts : 1;
  const int64_t units = parts * p.num_seqs * p.num_kv_heads;
  if (units <= 0 || units > 0x7fffffff) return false;
  int64_t grid = num_cus();
  if (grid > units) grid = units;
  if (grid * MAXU < units) return false;  // more than 64 units per workgroup
  const int64_t out_bytes = (int64_t)p.num_seqs * p.num_q_heads * parts * D *
                            (p.partition_size > 0 ? 4 : (p.out_bf16 ? 2 : 4));
  if (out_bytes > 0x7fff0000) return false;
  const bool split = p.partition_size > 0;
  switch (group) {
#define PA_CASE(g)                                                                \
  case g:                                                                         \
    if (split)                                                                    \
      decode_fp8_kernel<g, true><<<(unsigned)grid, NW * 64, 0, stream>>>(p);      \
    else                                                                          \
      decode_fp8_kernel<g, false><<<(unsigned)grid, NW * 64, 0, stream>>>(p);     \
    return true;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default: return false;
  }
}

}  // namespace pa
