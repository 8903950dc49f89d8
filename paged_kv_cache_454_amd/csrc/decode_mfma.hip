// Paged decode attention for BF16 caches with head_dim 256 and block sizes
// that are multiples of 16, on the matrix cores; single pass or split into
// context partitions. Same results and ABI as the generic kernel.
//
// Why matrix cores in a bandwidth-bound kernel: decode moves 4 KiB of K/V
// per token and KV head ("vLLM Architecture, Memory and Benchmarks Deep
// Dive", s.1: 4 KV heads, head dimension 256, BF16; decode is bound by
// memory traffic), and the vector-unit form of Q.K and P.V (one v_dot2 per
// channel pair and query head) costs about 600 VALU instructions per
// 16-token tile. Those delay each wave's next loads and stretch the tail of
// the launch. On the matrix cores the two contractions of a tile are 8 + 16
// MFMA instructions.
//
// Work decomposition and streaming are the persistent kernel's: one 8-wave
// workgroup per compute unit owns up to 64 units (one (sequence, KV head,
// partition) each, planned on the device from the context lengths); within a
// unit the 16-token tiles go round-robin to the waves, each of which streams
// its tiles of all the workgroup's units through a two-deep register ring;
// at a unit's end the 8 waves' softmax states are merged through LDS.
//
// Per tile (16 tokens of one KV head inside one block: 8 KiB of K and 8 KiB
// of V):
//  * S^T = K . Q^T with v_mfma_f32_16x16x32_bf16 (M = 16 tokens, N = 16
//    columns, the group's G query heads and repeats of them, K = 256
//    channels in 8 steps). Lane (m, g) (m = lane % 16, g = lane / 16) needs
//    16-byte pieces of token row m. Eight wavefront loads each read whole
//    128-byte lines of 8 rows (lane (m, g): row m % 8 + 8 (i & 1), byte
//    128 (i >> 1) + 16 g + 64 (m / 8)), and a DPP rotation by 8 lanes inside
//    each 16-lane row swaps the halves, so every lane ends with the pieces
//    of its own row: bytes 128 p + 64 h + 16 g, channels 64 p + 32 h + 8 g
//    .. +7 in step 2 p + h. The query operand takes the same channels.
//  * The accumulator gives lane (n, g) the logits of head n for tokens
//    4g .. 4g+3; the row maximum and the sum need two lane swaps. Online
//    softmax in the exp2 domain with a lazy running max (rescale only when a
//    tile raises it by more than 2^8); weights rounded to BF16, and the
//    running sum adds the rounded weights. The four weights of a lane are
//    already the B operand of P.V (tokens 4g .. 4g+3 of head n).
//  * O^T = V^T . P^T with v_mfma_f32_16x16x16_bf16 (M = 16 channels per
//    step, 16 steps; K = the 16 tokens). The pool is token-major, so each
//    wave writes its V tile to its own LDS buffer (rows padded to 544 bytes,
//    so the four rows one transpose read touches fall on distinct banks) and
//    reads the A operands back transposed with ds_read_b64_tr_b16: lane m of
//    group g gets channel 16 cb + m of tokens 4g .. 4g+3.
//  * Rows past the context lie outside the loads' num_records and read as
//    zeros; their logits are -inf. An out-of-pool block id gives an empty
//    tile and poisons only that unit's outputs with NaN.
//  * Decode step (new_key set): the last unit of each sequence streams its
//    pool tokens up to T - 2 and then one more tile whose only row is the
//    step's token, read from the step's K/V rows (same row layout, so the
//    same loads; the other rows lie past num_records). Nothing this launch
//    reads comes from that token's slot, so the slot write may run later on
//    the stream (the merge kernel does it).
#include <math.h>

#include "launch.h"
#include "pa_device.h"
#include "persistent_plan.h"

namespace pa {
namespace {
using namespace persist;

constexpr int D = 256;      // head_dim
constexpr int TILE = 16;    // tokens per tile
constexpr int NW = 8;       // wavefronts per workgroup (two per SIMD)
static_assert(NW == persist::kPlanWaves, "the planner's unit costs count 8 waves");
constexpr int KL = 8;       // 16-byte K loads per lane per tile
constexpr int VL = 8;       // 16-byte V loads per lane per tile
constexpr int VROW = 544;   // bytes per token row of a wave's LDS V buffer
constexpr int VBUF = TILE * VROW;
// LDS row strides padded by 16 bytes so that the rows of different query
// heads start on different banks: a query row of 32 x 16 bytes (read 16
// lanes at a time, one head per lane, the same channels) and a parked merge
// row of D floats (written one head per lane).
constexpr int QROW = 33;      // uint4 per query row
constexpr int RSTR = D + 4;   // floats per parked merge row
constexpr float kLazy = 8.f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma32(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8 bytes addressed by lane 4e + i / 4, for e = 0..3.
__device__ __forceinline__ u32x2 tr_read(const uint8_t *lds_byte_ptr) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) bf16x4 lds_v4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_v4 *)((__attribute__((address_space(3))) uint8_t *)lds_byte_ptr));
  return __builtin_bit_cast(u32x2, v);
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

template <int G>
struct CfgM {
  static constexpr int FIXED = NW * VBUF + 4096;
  static constexpr int NQ_FIT = (150 * 1024 - FIXED) / (G * QROW * 16);
  static constexpr int NQ = NQ_FIT > 32 ? 32 : NQ_FIT;  // query slots in LDS
  static_assert(NQ >= 4, "too little LDS left for the query slots");
  static_assert(G * RSTR * 4 <= VBUF, "a wave's merge state must fit its V buffer");
  static_assert(VBUF >= 192 * 4, "the planner needs 192 ints of scratch");
};

// One tile of a wave's stream: its block id comes from a vector load issued
// when the descriptor is made and first used two stream positions later.
struct DescM {
  int blk;      // physical block id (VGPR, pending load)
  int head;     // KV head
  int tok_off;  // token offset of the tile inside its block
  int nvalid;   // valid tokens of the tile (0: empty, loads return zeros)
  int newrow;   // -1: a pool tile; else the tile is the step's token alone,
                // read from row newrow (sequence x KV heads + head) of the
                // step's K/V rows
};

// Plan-cache kind of this kernel's slots (first two block ids per wave).
constexpr uint32_t kPlanKindMfma = 0x100;

template <int G, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mfma_kernel(DecodeParams p) {
  using C = CfgM<G>;
  // Per wave: the V tile being consumed, then (at a unit's end) the wave's
  // merge state [G][RSTR] floats.
  __shared__ __attribute__((aligned(16))) uint8_t vbuf_all[NW][VBUF];
  __shared__ float mg_m[NW][8], mg_l[NW][8];
  __shared__ int mg_bad[NW];
  __shared__ __attribute__((aligned(16))) uint4 qs[C::NQ][G][QROW];
  __shared__ int4 uinfo[MAXU];     // (s, h, lo, hi)
  __shared__ int ubadpart[MAXU];   // part * 4 + 2 * append + bad
  __shared__ uint32_t act_lds[3];  // active-unit mask, and whether the plan slot is used

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;  // A row / B column / accumulator column
  const int grp = lane >> 4;  // k group / accumulator row group
  uint8_t *vbuf = vbuf_all[wave];
  float *red = reinterpret_cast<float *>(vbuf);

  const int S = p.num_seqs, H = p.num_kv_heads, HQ = p.num_q_heads;
  // With a plan buffer: this workgroup's slot, this wave's first two block
  // ids and (wave 0) the units, loaded together when the slot's tag names
  // this launch; otherwise planned here and stored.
  const PlanSlot ps = plan_slot<SPLIT>(p, kPlanKindMfma, wave, wave == 0);
  const int pre_id0 = (int)ps.ids[0], pre_id1 = (int)ps.ids[1];
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
  const int64_t head_stride = (int64_t)bs * D * 2;  // bytes
  const int64_t block_stride = head_stride * H;
  const uint8_t *kpool = reinterpret_cast<const uint8_t *>(p.key_cache);
  const uint8_t *vpool = reinterpret_cast<const uint8_t *>(p.value_cache);
  const uint8_t *knew = reinterpret_cast<const uint8_t *>(p.new_key);
  const uint8_t *vnew = reinterpret_cast<const uint8_t *>(p.new_value);
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
  // A wave's tiles of a unit of nt tiles, padded to even with empty tiles so
  // that stream positions alternate between the A and B register sets
  // inside every unit.
  auto padded_count = [&](int nt) {
    const int c = wave < nt ? (nt - wave + NW - 1) / NW : 0;
    return c + (c & 1);
  };

  // ---- Cursor over this wave's tile stream (uniform state). A unit is
  // cur_np pool tiles, then (cur_app) one tile holding the step's token.
  uint64_t cur_mask = act_mask;
  int cur_j = -1, cur_i = 0, cur_c = 0, cur_np = 0, cur_app = 0;
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
      cur_app = (__builtin_amdgcn_readfirstlane(ubadpart[cur_j]) >> 1) & 1;
      cur_np = (cur_u.w - cur_u.z + TILE - 1) / TILE;
      cur_c = padded_count(cur_np + cur_app);
      cur_i = 0;
    }
  };
  // pre >= 0: the id was preloaded from the plan (stream position pre of
  // this wave); the step's-token tile still looks its id up.
  auto make_desc = [&](int pre = -1) -> DescM {
    DescM d{0, 0, 0, 0, -1};
    const int k = wave + cur_i * NW;
    const int tok0 = cur_u.z + k * TILE;
    // The id load is issued on every path (an empty tile reads past the
    // table's num_records, which returns 0 without an access).
    int entry_off = 0x7ffffff0;
    if (cur_j >= 0 && tok0 < cur_u.w) {
      entry_off = (cur_u.x * p.max_blocks_per_seq + tok0 / bs) * 4;
      d.head = cur_u.y;
      d.tok_off = tok0 % bs;
      d.nvalid = min(TILE, cur_u.w - tok0);
    } else if (cur_j >= 0 && cur_app && k == cur_np) {
      // The step's token (position cur_u.w = T - 1): its block id is still
      // looked up, so a bad table entry poisons the unit as a pool read would.
      entry_off = (cur_u.x * p.max_blocks_per_seq + cur_u.w / bs) * 4;
      d.head = cur_u.y;
      d.nvalid = 1;
      d.newrow = cur_u.x * H + cur_u.y;
    }
    if (pre >= 0 && d.newrow < 0)
      d.blk = pre == 0 ? pre_id0 : pre_id1;
    else
      d.blk = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, entry_off, 0, 0);
    return d;
  };
  // Buffer resource over the valid rows of one tile of a pool; an invalid
  // block id gives an empty resource (zeros, no access) and marks the tile.
  auto tile_rsrc = [&](const DescM &d, const uint8_t *pool, const uint8_t *step_rows,
                       int &nvalid, int &bad) {
    int blk = __builtin_amdgcn_readfirstlane(d.blk), n = d.nvalid;
    bad = 0;
    if (n > 0 && (blk < 0 || blk >= p.num_blocks)) {
      bad = 1;
      n = 0;
    }
    if (n <= 0) blk = 0;
    nvalid = n;
    const uint8_t *base = d.newrow >= 0
                              ? step_rows + (int64_t)d.newrow * (D * 2)
                              : pool + (int64_t)blk * block_stride +
                                    (int64_t)d.head * head_stride + (int64_t)d.tok_off * D * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, n * D * 2,
                                             0x00020000);
  };
  // K: load i reads bytes 128 (i >> 1) .. of rows 8 (i & 1) .. +7.
  const int koff = (n16 & 7) * (2 * D) + 16 * grp + 64 * (n16 >> 3);
  auto load_k = [&](u32x4(&kt)[KL], const DescM &d) {
    int nv, bad;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(d, kpool, knew, nv, bad);
#pragma unroll
    for (int i = 0; i < KL; ++i)
      kt[i] = __builtin_amdgcn_raw_buffer_load_b128(
          r, koff + (i & 1) * 8 * (2 * D) + (i >> 1) * 128, 0, kStreamLoad);
  };
  // V: load i gives lane l the 8 channels 8 (l % 32) .. of token 2i + l / 32.
  const int voff = lane * 16;
  auto load_v = [&](u32x4(&vt)[VL], const DescM &d, int &nvalid, int &bad) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(d, vpool, vnew, nvalid, bad);
#pragma unroll
    for (int i = 0; i < VL; ++i)
      vt[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + i * 1024, 0, kStreamLoad);
  };

  // Prime the ring with the stream's first two tiles, and load the block ids
  // of the next two, in the order the loop body issues them.
  u32x4 ka[KL], va[VL], kb[KL], vb[VL];
  int nv_a, nv_b, bad_a, bad_b;
  DescM dn, dn2;
  {
    cur_i = -1;
    advance();
    const DescM d0 = make_desc(use_plan ? 0 : -1);
    advance();
    const DescM d1 = make_desc(use_plan ? 1 : -1);
    load_k(ka, d0);
    load_v(va, d0, nv_a, bad_a);
    advance();
    dn = make_desc();
    load_k(kb, d1);
    load_v(vb, d1, nv_b, bad_b);
    advance();
    dn2 = make_desc();
    // The wave's first two ids, stored for the launches after this one
    // unless they came from the slot (dropped stores otherwise).
    plan_store_id(ps, use_plan, wave, 0, lane, d0.blk);
    plan_store_id(ps, use_plan, wave, 1, lane, d1.blk);
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

  const float sl2 = p.scale * kLog2e;
  f32x4 o[16];
  float m_run, l_run;
  // Columns n >= G repeat query head n % G: MFMA columns do not mix, those
  // columns are never stored, and their maxima equal a real head's, so they
  // trigger no extra rescales.
  const bool live_head = n16 < G;
  const int qh = n16 % G;

  // S^T, softmax and the weights (B operand of P.V) for one tile.
  auto qk_softmax = [&](const u32x4(&kraw)[KL], int qslot, int nvalid) -> u32x2 {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const bool lo8 = n16 < 8;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      // Loads 2p, 2p+1 give lane m < 8 row m's piece at byte 128p + 16g and
      // lane m >= 8 row m's piece at 128p + 64 + 16g; each lane passes the
      // piece its partner m ^ 8 needs and keeps its own.
      const u32x4 v0 = kraw[2 * pp], v1 = kraw[2 * pp + 1];
      u32x4 k0, k1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t send = lo8 ? v1[w] : v0[w];
        const uint32_t recv =
            (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x128, 0xf, 0xf, false);
        k0[w] = lo8 ? v0[w] : recv;
        k1[w] = lo8 ? recv : v1[w];
      }
      // Channels 64p + 8g .. (k0) and 64p + 32 + 8g .. (k1).
      const uint4 q0 = qs[qslot][qh][8 * pp + grp];
      const uint4 q1 = qs[qslot][qh][8 * pp + 4 + grp];
      u32x4 b0, b1;
      b0[0] = q0.x;
      b0[1] = q0.y;
      b0[2] = q0.z;
      b0[3] = q0.w;
      b1[0] = q1.x;
      b1[1] = q1.y;
      b1[2] = q1.z;
      b1[3] = q1.w;
      s0 = mfma32(k0, b0, s0);
      s1 = mfma32(k1, b1, s1);
    }
    float z[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = 4 * grp + r < nvalid ? (s0[r] + s1[r]) * sl2 : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
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
    u32x2 pb;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[u] = bf16_pair(fast_exp2(z[2 * u] - m_run), fast_exp2(z[2 * u + 1] - m_run));
      l_run += __uint_as_float(pb[u] << 16) + __uint_as_float(pb[u] & 0xffff0000u);
    }
    return pb;
  };
  // O^T += V^T . P^T for one tile: the V tile goes through this wave's LDS
  // buffer and comes back transposed.
  const int vrow_w = (2 * 0 + (lane >> 5)) * VROW + 16 * (lane & 31);  // row of load 0
  const int vrd = (4 * grp + (n16 >> 2)) * VROW + 8 * (n16 & 3);       // transpose read base
  auto pv = [&](const u32x4(&vt)[VL], const u32x2 &pb) {
#pragma unroll
    for (int i = 0; i < VL; ++i)
      *reinterpret_cast<u32x4 *>(vbuf + vrow_w + 2 * i * VROW) = vt[i];
    // LDS operations of a wave complete in order; keep the compiler from
    // moving the transpose reads above the writes.
    asm volatile("" ::: "memory");
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = mfma16(tr_read(vbuf + vrd + 32 * cb), pb, o[cb]);
    asm volatile("" ::: "memory");
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
    const int ubp = __builtin_amdgcn_readfirstlane(ubadpart[j]);
    const int cpad = padded_count((uj.w - uj.z + TILE - 1) / TILE + ((ubp >> 1) & 1));
    int ubad = ubp & 1;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNoMax;
    l_run = 0.f;

    // Two stream positions per iteration: A, then B. Empty tiles (padding or
    // past a short unit) skip the arithmetic but keep the ring moving.
    for (int i = 0; i < cpad; i += 2) {
      int nvn, badn;
      u32x2 pb{0u, 0u};
      if (nv_a > 0) pb = qk_softmax(ka, qslot, nv_a);
      load_k(ka, dn);
      if (nv_a > 0) pv(va, pb);
      ubad |= bad_a;
      load_v(va, dn, nv_a, bad_a);
      dn = dn2;
      advance();
      dn2 = make_desc();

      if (nv_b > 0) pb = qk_softmax(kb, qslot, nv_b);
      load_k(kb, dn);
      if (nv_b > 0) pv(vb, pb);
      ubad |= bad_b;
      load_v(vb, dn, nv_b, bad_b);
      dn = dn2;
      advance();
      dn2 = make_desc();
      (void)nvn;
      (void)badn;
    }

    // Park this wave's state in its LDS buffer: accumulator rows 4g + r of
    // channel block cb -> channel 16 cb + 4g + r of head n.
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

    // All waves merge the unit's 8 partial states and store it: thread t
    // takes channels 4t .. 4t+3 of the unit's G x 256 outputs (float4 LDS
    // reads and 16-byte stores). Every thread issues the same, fixed number
    // of buffer stores (stores that must not happen get an offset past
    // num_records and are dropped), which keeps the compiler's wait counts
    // exact for the loads in flight.
    static_assert(G * D / 4 <= NW * 64, "one channel quad per thread");
    const int64_t qrow = (int64_t)uj.x * HQ + (int64_t)uj.y * G;
    const int part = ubp >> 2;
    {
      const int idx = 4 * threadIdx.x;
      const bool live = idx < G * D;
      const int h = live ? idx / D : 0;
      const int ch = idx - h * D;
      float M = kNoMax;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mg_m[w][h]);
      float L = 0.f;
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(mg_m[w][h] - M);
        L += mg_l[w][h] * f;
        const float4 a = *reinterpret_cast<const float4 *>(
            reinterpret_cast<const float *>(vbuf_all[w]) + (live ? h * RSTR + ch : 0));
        A.x += a.x * f;
        A.y += a.y * f;
        A.z += a.z * f;
        A.w += a.w * f;
      }
      const float inv = SPLIT ? 1.f / L : (L > 0.f ? 1.f / L : 0.f);
      const float4 ov = bad ? make_float4(nan, nan, nan, nan)
                            : make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
      u32x4 ob;
      ob[0] = __float_as_uint(ov.x);
      ob[1] = __float_as_uint(ov.y);
      ob[2] = __float_as_uint(ov.z);
      ob[3] = __float_as_uint(ov.w);
      constexpr int kDrop = 0x7ffffff0;
      if constexpr (!SPLIT) {
        const int64_t e = (qrow + h) * D + ch;
        if (p.out_bf16) {
          u32x2 b2;
          b2[0] = (uint32_t)f32_to_bf16(ov.x) | ((uint32_t)f32_to_bf16(ov.y) << 16);
          b2[1] = (uint32_t)f32_to_bf16(ov.z) | ((uint32_t)f32_to_bf16(ov.w) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(b2, out_rsrc, live ? (int)(e * 2) : kDrop, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(ob, out_rsrc, live ? (int)(e * 4) : kDrop, 0, 0);
        }
      } else {
        const int64_t pidx = (qrow + h) * p.max_parts + part;
        __builtin_amdgcn_raw_buffer_store_b128(ob, out_rsrc,
                                               live ? (int)((pidx * D + ch) * 4) : kDrop, 0, 0);
        const int moff = (live && ch == 0) ? (int)(pidx * 4) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : M * kLn2), max_rsrc,
                                              moff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : L), sum_rsrc, moff, 0,
                                              0);
      }
    }
    __syncthreads();  // the buffers are reused by the next unit's V tiles
  }
}

}  // namespace

int64_t decode_mfma_grid(const DecodeParams &p) {
  if (!p.kv_bf16 || p.kv_fp8 || p.head_dim != D || p.block_size % TILE != 0 || p.query_start_loc)
    return 0;
  if (p.partition_size > 0 && p.partition_size % TILE != 0) return 0;
  if ((int64_t)p.num_seqs * p.max_blocks_per_seq * 4 > 0x7fffffff) return 0;
  const int group = p.num_q_heads / p.num_kv_heads;
  if (group < 1 || group > 8) return 0;
  const int64_t parts = p.partition_size > 0 ? p.max_parts : 1;
  const int64_t units = parts * p.num_seqs * p.num_kv_heads;
  if (units <= 0 || units > 0x7fffffff) return 0;
  int64_t grid = num_cus();
  // Split mode takes the tiled kernel (a workgroup per unit) when the
  // persistent form cannot pay for its planner and ring: at most one unit
  // per CU, or partitions under 2 tiles per wavefront.
  if (p.partition_size > 0 && (units <= grid || p.partition_size < 2 * NW * TILE)) return 0;
  if (grid > units) grid = units;
  if (grid * MAXU < units) return 0;  // more than 64 units per workgroup
  const int64_t out_bytes = (int64_t)p.num_seqs * p.num_q_heads * parts * D *
                            (p.partition_size > 0 ? 4 : (p.out_bf16 ? 2 : 4));
  if (out_bytes > 0x7fff0000) return 0;
  return grid;
}

// Launch the matrix-core kernel when the shape is one it covers; false
// otherwise (the caller then uses another kernel).
bool launch_decode_mfma(const DecodeParams &p, hipStream_t stream) {
  const int64_t grid = decode_mfma_grid(p);
  if (grid == 0) return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  const bool split = p.partition_size > 0;
  switch (group) {
#define PA_CASE(g)                                                                \
  case g:                                                                         \
    if (split)                                                                    \
      decode_mfma_kernel<g, true><<<(unsigned)grid, NW * 64, 0, stream>>>(p);     \
    else                                                                          \
      decode_mfma_kernel<g, false><<<(unsigned)grid, NW * 64, 0, stream>>>(p);    \
    return true;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default: return false;
  }
}

}  // namespace pa
