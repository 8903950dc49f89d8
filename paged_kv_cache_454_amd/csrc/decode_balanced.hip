// Paged decode attention for BF16 caches (head_dim 256, block sizes that are
// multiples of 16) on the matrix cores, with every workgroup given an equal
// share of the batch's work. Single pass, or split into context partitions;
// same results as the other decode kernels.
//
// Work is counted in rounds: a round is one 16-token tile for each of the 8
// wavefronts of a workgroup, 128 tokens of one KV head. A unit - one
// (sequence, KV head) in single-pass mode, one (sequence, KV head,
// partition) in split mode, i.e. one output record - takes ceil(tokens /
// 128) rounds. Units are laid end to end in a fixed order and workgroup b of
// NB takes rounds [b R / NB, (b + 1) R / NB) of the R in total, so the
// busiest workgroup has at most one round more than any other, whatever the
// mix of context lengths ("vLLM Architecture, Memory and Benchmarks Deep
// Dive", s.3: a continuous batch mixes requests of very different lengths).
// A unit that crosses a workgroup boundary is computed in pieces: each piece
// leaves its softmax state (running max, sum, unnormalised output) in a
// scratch slot, without waiting for the stores, and a second, small kernel
// launched behind the decode kernel merges the pieces of each such unit in
// their fixed order (so the result does not depend on timing) and writes
// the unit's output. The merge is the same log-sum-exp combination as the
// partition merge; in single-pass mode it makes a separate reduction over
// partitions unnecessary. (Under a saturated memory system a dependent
// round trip - waiting for stores, then an arrival counter - costs a wave
// several microseconds, so the pieces never wait on one another inside the
// decode kernel; the kernel boundary orders the slot writes before the
// merge reads them.)
//
// Unit order: sequences longest, shortest, second longest, second shortest,
// ... (batches of up to 64 sequences; larger batches keep their order), so
// that short sequences are spread over many workgroups and no workgroup
// collects many unit ends; inside a sequence, KV heads, then partitions.
//
// Inside a workgroup a piece's tiles go round-robin to the 8 wavefronts, each
// streaming its tiles through a two-deep register ring that runs across
// piece boundaries, and the wavefronts' states merge through LDS at the
// piece's end. The per-tile arithmetic (S^T = K.Q^T and O^T = V^T.P^T with
// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x16_bf16, online softmax in
// the exp2 domain with a lazy running max, BF16 weights, V transposed
// through LDS with ds_read_b64_tr_b16) is that of the persistent matrix-core
// kernel; see decode_mfma.hip for the lane layouts.
#include <math.h>

#include <mutex>

#include "launch.h"
#include "pa_device.h"
#include "persistent_plan.h"

namespace pa {
namespace {

constexpr int D = 256;      // head_dim
constexpr int TILE = 16;    // tokens per tile
constexpr int NW = 8;       // wavefronts per workgroup (two per SIMD)
constexpr int KL = 8;       // 16-byte K loads per lane per tile
constexpr int VL = 8;       // 16-byte V loads per lane per tile
constexpr int VROW = 544;   // bytes per token row of a wave's LDS V buffer
constexpr int VBUF = TILE * VROW;
constexpr int QROW = 33;    // uint4 per staged query row (16 bytes of padding)
constexpr int RSTR = D + 4; // floats per parked merge row
constexpr int ROUND_SHIFT = 7;   // 128 tokens per round
constexpr float kLazy = 8.f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ f32x4 mfma32(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 tr_read(const uint8_t *lds_byte_ptr) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) bf16x4 lds_v4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_v4 *)((__attribute__((address_space(3))) uint8_t *)lds_byte_ptr));
  return __builtin_bit_cast(u32x2, v);
}

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
struct CfgB {
  static constexpr int TABLES = 4 * BAL_MAX_SEQS * 4 + 16;
  static constexpr int FIXED = NW * VBUF + TABLES + 2048;
  static constexpr int NQ_FIT = (150 * 1024 - FIXED) / (G * QROW * 16);
  static constexpr int NQ = NQ_FIT > 16 ? 16 : NQ_FIT;  // staged query slots
  static_assert(NQ >= 2, "too little LDS left for the query slots");
  static_assert(G * RSTR * 4 <= VBUF, "a wave's merge state must fit its V buffer");
  static_assert(VBUF >= 192 * 4, "the planner needs 192 ints of scratch");
};

// Rounds of one (sequence, KV head) and its unit count, from the clamped
// context T: single pass, one unit of max(1, ceil(T/128)) rounds (an empty
// context still writes its zero output); split, ceil(T/P) partitions
// (clamped to max_parts), each ceil(tokens/128) rounds.
template <bool SPLIT>
__device__ __forceinline__ void seq_rounds(int T, int P, int max_parts, int &np, int &rh,
                                           int &over) {
  over = 0;
  if (!SPLIT) {
    np = 1;
    rh = max(1, (T + 127) >> ROUND_SHIFT);
    return;
  }
  unsigned n = ((unsigned)T + (unsigned)P - 1u) / (unsigned)P;
  if (n > (unsigned)max_parts) {
    over = 1;
    n = (unsigned)max_parts;
  }
  np = (int)n;
  if (n == 0) {
    rh = 0;
    return;
  }
  const int rf = (P + 127) >> ROUND_SHIFT;
  const int last = (int)(min((int64_t)T, (int64_t)n * P) - ((int64_t)n - 1) * P);
  rh = ((int)n - 1) * rf + ((last + 127) >> ROUND_SHIFT);
}

// Plan tables (one wavefront): for each position si of the unit order, the
// sequence (bit 30: outputs poisoned), its clamped context length, its
// units per KV head and the first global round of its units; sequences
// without units (split mode, empty context) are left out. Returns (in
// tab_r0[BAL_MAX_SEQS]) the number of positions; tab_r0[that] = R, the total.
template <bool SPLIT>
__device__ void plan_tables(const DecodeParams &p, int lane, int *tab_s, int *tab_T, int *tab_np,
                            int *tab_r0, int *scr) {
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int P = SPLIT ? p.partition_size : 1;
  const int cap = p.max_blocks_per_seq * p.block_size;
  auto info = [&](int s, int &T, int &bad, int &np, int &rs) __attribute__((always_inline)) {
    T = 0;
    bad = 0;
    np = 0;
    rs = 0;
    if (s >= S) return;
    int t = p.context_lens[s];
    t = t < 0 ? 0 : t;
    if (t > cap) {
      bad = 1;
      t = cap;
    }
    int rh, over;
    seq_rounds<SPLIT>(t, P, p.max_parts, np, rh, over);
    bad |= over;
    T = t;
    rs = rh * H;
  };
  if (S <= 64) {
    int T, bad, np, rs;
    info(lane, T, bad, np, rs);
    const bool has = rs > 0;
    const int n = __popcll(__builtin_amdgcn_ballot_w64(has));
    // Rank by decreasing length (ties: lower index first), then interleave:
    // rank k < ceil(n/2) goes to position 2k, the others fill the odd
    // positions from the shortest up.
    const int key = has ? (min(T, (1 << 24) - 1) << 6) | (63 - lane) : -1;
    persist::lane_exchange_fence();
    scr[lane] = key;
    persist::lane_exchange_fence();
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
      const int4 k4 = *reinterpret_cast<const int4 *>(&scr[j]);
      rank += (k4.x > key) + (k4.y > key) + (k4.z > key) + (k4.w > key);
    }
    const int half = (n + 1) >> 1;
    const int pos = rank < half ? 2 * rank : 2 * (n - 1 - rank) + 1;
    persist::lane_exchange_fence();
    if (has) {
      tab_s[pos] = lane | (bad << 30);
      tab_T[pos] = T;
      tab_np[pos] = np;
      scr[64 + pos] = rs;
    }
    persist::lane_exchange_fence();
    const int x = lane < n ? scr[64 + lane] : 0;
    const int incl = persist::wave_incl_scan(x, lane);
    if (lane < n) tab_r0[lane] = incl - x;
    if (lane == 63) {
      tab_r0[n] = incl;
      tab_r0[BAL_MAX_SEQS] = n;
    }
  } else {
    int carry = 0, cnt = 0;
    for (int c = 0; c < S; c += 64) {
      const int s = c + lane;
      int T, bad, np, rs;
      info(s, T, bad, np, rs);
      const int has = rs > 0;
      const int incl = persist::wave_incl_scan(rs, lane);
      const int pos = cnt + persist::wave_incl_scan(has, lane) - has;
      if (has) {
        tab_s[pos] = s | (bad << 30);
        tab_T[pos] = T;
        tab_np[pos] = np;
        tab_r0[pos] = carry + incl - rs;
      }
      carry += __shfl(incl, 63, 64);
      cnt += __popcll(__builtin_amdgcn_ballot_w64(has != 0));
    }
    if (lane == 0) {
      tab_r0[cnt] = carry;
      tab_r0[BAL_MAX_SEQS] = cnt;
    }
  }
}

// Position in a wavefront's stream (uniform across the wavefront): the unit
// (sequence s at order position si, KV head g, partition pt) with its token
// range [ulo, uhi), its ur rounds starting at global round u0; the piece of
// it this workgroup computes, global rounds [ps, pe); and the stream
// position k of the piece's npos. npos is the piece's round count rounded up
// to even - an odd piece ends with one empty position - so that every piece
// starts on the same half of the two-deep register ring.
struct Cursor {
  int si, s, T, bad, np, g, pt, ulo, uhi, ur, u0, ps, pe, k, npos;
};

template <bool SPLIT>
__device__ __forceinline__ Cursor cur_unit(Cursor c, int P) {
  c.ulo = SPLIT ? c.pt * P : 0;
  c.uhi = SPLIT ? (int)min((int64_t)c.T, (int64_t)c.ulo + P) : c.T;
  c.ur = max(1, (c.uhi - c.ulo + 127) >> ROUND_SHIFT);
  return c;
}

// Store channels ch .. ch+3 of query head h of a unit from its merged state
// (M in the log2 domain, L the sum, A the unnormalised output): single
// pass, out = A / L (zeros for an empty context); split, the partition
// record o_p = A / L, m_p = M ln 2, l_p = L. A poisoned unit stores NaN.
// Every thread issues the same, fixed number of buffer stores (stores that
// must not happen get an offset past num_records and are dropped), which
// keeps the compiler's wait counts exact for the loads in flight.
template <bool SPLIT>
__device__ __forceinline__ void store_unit(const DecodeParams &p, int G, int s_id, int g_id,
                                           int part, int h, int ch, bool live, bool bad, float M,
                                           float L, float4 A) {
  constexpr int kDrop = 0x7ffffff0;
  const float nan = __builtin_nanf("");
  const int HQ = p.num_q_heads;
  const int64_t qrow = (int64_t)s_id * HQ + (int64_t)g_id * G;
  const int64_t rows = (int64_t)p.num_seqs * HQ * (SPLIT ? p.max_parts : 1);
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      SPLIT ? (void *)p.part_out : p.out, (short)0,
      (int)(rows * D * (SPLIT ? 4 : (p.out_bf16 ? 2 : 4))), 0x00020000);
  const float inv = SPLIT ? 1.f / L : (L > 0.f ? 1.f / L : 0.f);
  const float4 ov = bad ? make_float4(nan, nan, nan, nan)
                        : make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
  u32x4 ob;
  ob[0] = __float_as_uint(ov.x);
  ob[1] = __float_as_uint(ov.y);
  ob[2] = __float_as_uint(ov.z);
  ob[3] = __float_as_uint(ov.w);
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
    const __amdgpu_buffer_rsrc_t max_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(p.part_max, (short)0, (int)(rows * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t sum_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(p.part_sum, (short)0, (int)(rows * 4), 0x00020000);
    const int64_t pidx = (qrow + h) * p.max_parts + part;
    __builtin_amdgcn_raw_buffer_store_b128(ob, out_rsrc,
                                           live ? (int)((pidx * D + ch) * 4) : kDrop, 0, 0);
    const int moff = (live && ch == 0) ? (int)(pidx * 4) : kDrop;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : M * kLn2), max_rsrc, moff,
                                          0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bad ? nan : L), sum_rsrc, moff, 0, 0);
  }
}

template <int G, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_bal_kernel(DecodeParams p) {
  using C = CfgB<G>;
  __shared__ __attribute__((aligned(16))) uint8_t vbuf_all[NW][VBUF];
  __shared__ float mg_m[NW][8], mg_l[NW][8];
  __shared__ int mg_bad[NW];
  __shared__ __attribute__((aligned(16))) uint4 qs[C::NQ][G][QROW];
  __shared__ int tab_s[BAL_MAX_SEQS], tab_T[BAL_MAX_SEQS], tab_np[BAL_MAX_SEQS];
  __shared__ int tab_r0[BAL_MAX_SEQS + 1];

  const int lane = threadIdx.x & 63;
  const int wave = rfl(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int grp = lane >> 4;
  uint8_t *vbuf = vbuf_all[wave];
  float *red = reinterpret_cast<float *>(vbuf);

  const int S = p.num_seqs, H = p.num_kv_heads, HQ = p.num_q_heads;
  const int P = SPLIT ? p.partition_size : 1;
  if (wave == 0)
    plan_tables<SPLIT>(p, lane, tab_s, tab_T, tab_np, tab_r0, reinterpret_cast<int *>(red));
  __syncthreads();
  const int nseq = rfl(tab_r0[BAL_MAX_SEQS]);  // order positions with units
  const int R = rfl(tab_r0[nseq]);
  // With fewer rounds than workgroups only the first R take part, so every
  // taking part holds at least one round (the piece count of a unit is the
  // number of consecutive workgroups it spans).
  int4 *entries = reinterpret_cast<int4 *>(p.scratch);
  const int NB = min((int)gridDim.x, R), b = blockIdx.x;
  if (b >= NB) {  // uniform for the workgroup: nothing to compute or merge
    if (threadIdx.x == 0) entries[b] = make_int4(0, 0, 0, 0);
    return;
  }
  const int lo = (int)((int64_t)b * R / NB), hi = (int)((int64_t)(b + 1) * R / NB);

  // ---- the stream cursor (the tables are read straight from LDS)
  // The first unit of the sequence at order position c.si.
  auto cur_seq = [&](Cursor c) __attribute__((always_inline)) -> Cursor {
    const int sb = rfl(tab_s[c.si]);
    c.s = sb & 0x3fffffff;
    c.bad = sb >> 30;
    c.T = rfl(tab_T[c.si]);
    c.np = rfl(tab_np[c.si]);
    c.g = 0;
    c.pt = 0;
    return cur_unit<SPLIT>(c, P);
  };
  // The piece of the current unit that starts at round ps.
  auto set_piece = [&](Cursor c, int ps) __attribute__((always_inline)) -> Cursor {
    c.ps = ps;
    c.pe = min(c.u0 + c.ur, hi);
    c.npos = (c.pe - c.ps + 1) & ~1;
    c.k = 0;
    return c;
  };
  // The next piece: the start of the next unit, or the end of the range
  // (ps == pe == hi; every later position is empty).
  auto next_piece = [&](Cursor c) __attribute__((always_inline)) -> Cursor {
    if (c.pe >= hi) {
      c.ps = c.pe = hi;
      c.npos = 1 << 30;
      c.k = 0;
      return c;
    }
    c.u0 += c.ur;
    ++c.pt;
    if (c.pt >= c.np) {
      c.pt = 0;
      ++c.g;
      if (c.g >= H) {
        c.g = 0;
        ++c.si;  // below nseq: the range ends inside the units
        c = cur_seq(c);
      }
    }
    c = cur_unit<SPLIT>(c, P);
    return set_piece(c, c.u0);
  };
  auto advance = [&](Cursor c) __attribute__((always_inline)) -> Cursor {
    if (++c.k < c.npos) return c;
    return next_piece(c);
  };
  Cursor start{};
  {
    // The order position holding round lo: the last si with tab_r0[si] <= lo
    // (every position has at least one round).
    int a = 0, z = nseq - 1;
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (rfl(tab_r0[mid]) <= lo)
        a = mid;
      else
        z = mid - 1;
    }
    start.si = a;
    start = cur_seq(start);
    const int off = lo - rfl(tab_r0[a]);
    int np, rh, over;
    seq_rounds<SPLIT>(start.T, P, p.max_parts, np, rh, over);
    start.g = off / rh;
    const int offh = off - start.g * rh;
    const int rf = SPLIT ? (P + 127) >> ROUND_SHIFT : rh;
    start.pt = SPLIT ? min(offh / rf, start.np - 1) : 0;
    start = cur_unit<SPLIT>(start, P);
    start.u0 = lo - (offh - start.pt * rf);
    start = set_piece(start, lo);
  }

  const int bs = p.block_size;
  const int64_t head_stride = (int64_t)bs * D * 2;  // bytes
  const int64_t block_stride = head_stride * H;
  const uint8_t *kpool = reinterpret_cast<const uint8_t *>(p.key_cache);
  const uint8_t *vpool = reinterpret_cast<const uint8_t *>(p.value_cache);
  const __amdgpu_buffer_rsrc_t tab_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(p.block_tables), (short)0,
      (int)((int64_t)S * p.max_blocks_per_seq * 4), 0x00020000);
  float *slots = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(p.scratch) +
                                           bal_entry_bytes((int)gridDim.x));
  int4 my_entry = make_int4(0, 0, 0, 0);  // the cut unit that starts here

  // ---- tile descriptors along this wave's stream
  struct Desc {
    int blk, head, tok_off, nvalid;
  };
  auto make_desc = [&](const Cursor &c) __attribute__((always_inline)) -> Desc {
    Desc d{0, 0, 0, 0};
    int entry_off = 0x7ffffff0;  // an empty tile still issues the id load (returns 0)
    if (c.k < c.pe - c.ps) {
      const int r = c.ps + c.k - c.u0;  // round inside the unit
      const int tok0 = c.ulo + (r * NW + wave) * TILE;
      if (tok0 < c.uhi) {
        entry_off = (c.s * p.max_blocks_per_seq + tok0 / bs) * 4;
        d.head = c.g;
        d.tok_off = tok0 % bs;
        d.nvalid = min(TILE, c.uhi - tok0);
      }
    }
    d.blk = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, entry_off, 0, 0);
    return d;
  };
  auto tile_rsrc = [&](const Desc &d, const uint8_t *pool, int &nvalid, int &bad) __attribute__((always_inline)) {
    int blk = rfl(d.blk), n = d.nvalid;
    bad = 0;
    if (n > 0 && (blk < 0 || blk >= p.num_blocks)) {
      bad = 1;
      n = 0;
    }
    if (n <= 0) blk = 0;
    nvalid = n;
    const uint8_t *base = pool + (int64_t)blk * block_stride + (int64_t)d.head * head_stride +
                          (int64_t)d.tok_off * D * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, n * D * 2,
                                             0x00020000);
  };
  const int koff = (n16 & 7) * (2 * D) + 16 * grp + 64 * (n16 >> 3);
  auto load_k = [&](u32x4(&kt)[KL], const Desc &d) {
    int nv, bad;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(d, kpool, nv, bad);
#pragma unroll
    for (int i = 0; i < KL; ++i)
      kt[i] = __builtin_amdgcn_raw_buffer_load_b128(
          r, koff + (i & 1) * 8 * (2 * D) + (i >> 1) * 128, 0, kStreamLoad);
  };
  const int voff = lane * 16;
  auto load_v = [&](u32x4(&vt)[VL], const Desc &d, int &nvalid, int &bad) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(d, vpool, nvalid, bad);
#pragma unroll
    for (int i = 0; i < VL; ++i)
      vt[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + i * 1024, 0, kStreamLoad);
  };

  // Prime the ring with the stream's first two tiles, and the block ids of
  // the next two. Each half of the ring (A: even positions, B: odd) has its
  // own descriptor, refilled in place: the block id of position x + 4 is
  // requested while position x is computed and used two positions later, and
  // no register with a load in flight is ever copied (a copy would make the
  // compiler wait for every load issued before it).
  Cursor dc = start;
  u32x4 ka[KL], va[VL], kb[KL], vb[VL];
  int nv_a, nv_b, bad_a, bad_b;
  Desc da, db;
  {
    const Desc d0 = make_desc(dc);
    dc = advance(dc);
    const Desc d1 = make_desc(dc);
    dc = advance(dc);
    load_k(ka, d0);
    load_v(va, d0, nv_a, bad_a);
    da = make_desc(dc);
    dc = advance(dc);
    load_k(kb, d1);
    load_v(vb, d1, nv_b, bad_b);
    db = make_desc(dc);
    dc = advance(dc);
  }

  // Query rows of the next pieces, NQ at a time (qc walks unit by unit).
  Cursor qc = start;
  auto stage_queries = [&]() __attribute__((always_inline)) {
    for (int k = 0; k < C::NQ && qc.ps < hi; ++k) {
      const int64_t qrow = (int64_t)qc.s * HQ + (int64_t)qc.g * G;
      for (int i = threadIdx.x; i < G * 32; i += NW * 64) {
        const vec16 v =
            load16(reinterpret_cast<const uint16_t *>(p.query) + (qrow + i / 32) * D + (i % 32) * 8);
        qs[k][i / 32][i % 32] = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
      }
      qc = next_piece(qc);
    }
  };
  stage_queries();
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  f32x4 o[16];
  float m_run, l_run;
  const bool live_head = n16 < G;
  const int qh = n16 % G;

  auto qk_softmax = [&](const u32x4(&kraw)[KL], int qslot, int nvalid) -> u32x2 {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const bool lo8 = n16 < 8;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
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
  const int vrow_w = (lane >> 5) * VROW + 16 * (lane & 31);
  const int vrd = (4 * grp + (n16 >> 2)) * VROW + 8 * (n16 & 3);
  auto pv = [&](const u32x4(&vt)[VL], const u32x2 &pb) {
#pragma unroll
    for (int i = 0; i < VL; ++i)
      *reinterpret_cast<u32x4 *>(vbuf + vrow_w + 2 * i * VROW) = vt[i];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = mfma16(tr_read(vbuf + vrd + 32 * cb), pb, o[cb]);
    asm volatile("" ::: "memory");
  };

  // One stream position on each half of the ring: the tile in the registers
  // is computed, its registers are refilled with the tile two positions
  // ahead, and the block id four positions ahead is requested.
  auto step_a = [&](int qslot, int &ubad) __attribute__((always_inline)) {
    u32x2 pb{0u, 0u};
    if (nv_a > 0) pb = qk_softmax(ka, qslot, nv_a);
    load_k(ka, da);
    if (nv_a > 0) pv(va, pb);
    ubad |= bad_a;
    load_v(va, da, nv_a, bad_a);
    da = make_desc(dc);
    dc = advance(dc);
  };
  auto step_b = [&](int qslot, int &ubad) __attribute__((always_inline)) {
    u32x2 pb{0u, 0u};
    if (nv_b > 0) pb = qk_softmax(kb, qslot, nv_b);
    load_k(kb, db);
    if (nv_b > 0) pv(vb, pb);
    ubad |= bad_b;
    load_v(vb, db, nv_b, bad_b);
    db = make_desc(dc);
    dc = advance(dc);
  };

  Cursor cc = start;   // compute side: the current piece
  int kq = 0;          // query slots used
  // The current piece of unit (s_id, g_id, part), which spans global rounds
  // [u0, uend).
  int qslot = 0, u0 = 0, uend = 0, s_id = 0, g_id = 0, part = 0, ubad = 0;
  bool split = false;
  auto begin_piece = [&]() __attribute__((always_inline)) {
    if (__builtin_expect(kq == C::NQ, 0)) {
      // Every wave is between pieces (after the merge barriers).
      stage_queries();
      __syncthreads();
      kq = 0;
    }
    qslot = kq++;
    u0 = cc.u0;
    uend = u0 + cc.ur;
    split = u0 < lo || uend > hi;
    s_id = cc.s;
    g_id = cc.g;
    part = cc.pt;
    ubad = cc.bad;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNoMax;
    l_run = 0.f;
  };
  auto end_piece = [&]() __attribute__((always_inline)) {
    cc = next_piece(cc);

    // Park this wave's state; merge the 8 waves.
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

    static_assert(G * D / 4 <= NW * 64, "one channel quad per thread");
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
    bool write = true;
    if (split) {
      // Leave this piece's state in its slot; the merge kernel combines the
      // unit's pieces. Piece k of a unit that starts in workgroup b0 comes
      // from workgroup b0 + k; a workgroup holds at most one piece that
      // starts a unit (its last) and one that continues one (its first), in
      // slots 2b + 1 and 2b. The workgroup where the unit starts records it.
      const int b0 = (int)(((int64_t)(u0 + 1) * NB - 1) / R);
      const int b1 = (int)(((int64_t)uend * NB - 1) / R);
      float *slot = slots + (int64_t)(2 * b + (b == b0 ? 1 : 0)) * BAL_SLOT_FLOATS;
      if (live) {
        *reinterpret_cast<float4 *>(slot + h * D + ch) = A;
        if (ch == 0) {
          slot[BAL_GMAX * D + h] = M;
          slot[BAL_GMAX * D + BAL_GMAX + h] = L;
        }
      }
      if (threadIdx.x == 0) slot[BAL_GMAX * D + 2 * BAL_GMAX] = anybad ? 1.f : 0.f;
      if (b == b0) my_entry = make_int4(s_id, g_id, part, b1 - b0 + 1);
      write = false;
    }
    if (write) store_unit<SPLIT>(p, G, s_id, g_id, part, h, ch, live, anybad != 0, M, L, A);
    __syncthreads();  // the buffers are reused by the next piece's V tiles
  };

  // Every piece has an even number of stream positions, so the inner loop
  // is the straight pair A, B and each piece starts on the A half; the
  // piece's end (with its barriers and branches) stays outside it.
  while (cc.ps < hi) {
    begin_piece();
    const int npos = cc.npos;
    for (int i = 0; i < npos; i += 2) {
      step_a(qslot, ubad);
      step_b(qslot, ubad);
    }
    end_piece();
  }
  if (threadIdx.x == 0) entries[b] = my_entry;
}

// The pieces of every unit the decode kernel cut: workgroup b0 merges the
// unit recorded in entry b0 (pieces k = 0 .. n-1 in slots 2 (b0 + k) + (k
// == 0), in that order) and stores its output like the decode kernel. One
// thread per channel quad of the G heads.
template <int G, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void bal_merge_kernel(DecodeParams p) {
  const int4 e = reinterpret_cast<const int4 *>(p.scratch)[blockIdx.x];
  const int n = __builtin_amdgcn_readfirstlane(e.w);
  if (n <= 0) return;
  const float *slots = reinterpret_cast<const float *>(
      reinterpret_cast<const uint8_t *>(p.scratch) + bal_entry_bytes((int)gridDim.x));
  const int b0 = blockIdx.x;
  const int idx = 4 * threadIdx.x;
  const bool live = idx < G * D;
  const int h = live ? idx / D : 0;
  const int ch = idx - h * D;
  auto slot = [&](int k) { return slots + (int64_t)(2 * (b0 + k) + (k == 0 ? 1 : 0)) * BAL_SLOT_FLOATS; };
  float M = kNoMax;
  for (int k = 0; k < n; ++k) M = fmaxf(M, slot(k)[BAL_GMAX * D + h]);
  float L = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  int bad = 0;
  for (int k = 0; k < n; ++k) {
    const float *sk = slot(k);
    const float f = fast_exp2(sk[BAL_GMAX * D + h] - M);
    L += sk[BAL_GMAX * D + BAL_GMAX + h] * f;
    const float4 a = *reinterpret_cast<const float4 *>(sk + h * D + ch);
    A.x += a.x * f;
    A.y += a.y * f;
    A.z += a.z * f;
    A.w += a.w * f;
    bad |= sk[BAL_GMAX * D + 2 * BAL_GMAX] != 0.f;
  }
  store_unit<SPLIT>(p, G, __builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                    __builtin_amdgcn_readfirstlane(e.z), h, ch, live, bad != 0, M, L, A);
}

}  // namespace

int64_t bal_scratch_bytes(int grid) {
  return bal_entry_bytes(grid) + (int64_t)2 * grid * BAL_SLOT_FLOATS * 4;
}

int64_t bal_scratch_bytes_current() { return bal_scratch_bytes(persist::num_cus()); }

// Scratch for pa_decode_balanced_static, for callers that cannot allocate:
// one array per GPU the library runs on, held until the process ends, shared
// by every call on that GPU (calls that overlap in time race; nothing in it
// needs to start at zero). Host code never uses the array's name as an
// address: its device address is looked up once per device.
constexpr int64_t kStaticScratchBytes = 8 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
std::mutex g_static_mu;
void *g_static_ptr[64] = {nullptr};
}  // namespace

int64_t bal_static_scratch_limit() { return kStaticScratchBytes; }

// The current device's copy of the static scratch (looked up on the first
// call with that device current); null with a message on failure.
void *bal_static_scratch(const char **why) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    *why = "no current HIP device (or device index >= 64)";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      *why = "hipGetSymbolAddress of the static scratch failed";
      return nullptr;
    }
    g_static_ptr[dev] = ptr;
  }
  return g_static_ptr[dev];
}

// Launch the balanced matrix-core kernel when the shape is one it covers
// and p.scratch holds bal_scratch_bytes(#CUs); false otherwise.
bool launch_decode_balanced(const DecodeParams &p, hipStream_t stream) {
  if (!p.scratch || !p.kv_bf16 || p.kv_fp8 || p.head_dim != D || p.block_size % TILE != 0 ||
      p.query_start_loc)
    return false;
  if (p.partition_size > 0 && p.partition_size % TILE != 0) return false;
  if (p.num_seqs <= 0 || p.num_seqs > BAL_MAX_SEQS) return false;
  if ((int64_t)p.num_seqs * p.max_blocks_per_seq * 4 > 0x7fffffff) return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  if (group < 1 || group > BAL_GMAX) return false;
  const int grid = persist::num_cus();
  if (p.scratch_bytes < bal_scratch_bytes(grid)) return false;
  // Total rounds must fit 32 bits: per (sequence, KV head) at most
  // ceil(capacity / 128) + 1 rounds.
  const int64_t cap = (int64_t)p.max_blocks_per_seq * p.block_size;
  const int64_t parts = p.partition_size > 0 ? p.max_parts : 1;
  const int64_t per_head = (cap >> ROUND_SHIFT) + parts + 1;
  if ((int64_t)p.num_seqs * p.num_kv_heads * per_head > 0x3fffffff) return false;
  const int64_t out_bytes = (int64_t)p.num_seqs * p.num_q_heads * parts * D *
                            (p.partition_size > 0 ? 4 : (p.out_bf16 ? 2 : 4));
  if (out_bytes > 0x7fff0000) return false;
  const bool split = p.partition_size > 0;
  switch (group) {
#define PA_CASE(g)                                                                  \
  case g:                                                                           \
    if (split) {                                                                    \
      decode_bal_kernel<g, true><<<(unsigned)grid, NW * 64, 0, stream>>>(p);        \
      bal_merge_kernel<g, true><<<(unsigned)grid, NW * 64, 0, stream>>>(p);         \
    } else {                                                                        \
      decode_bal_kernel<g, false><<<(unsigned)grid, NW * 64, 0, stream>>>(p);       \
      bal_merge_kernel<g, false><<<(unsigned)grid, NW * 64, 0, stream>>>(p);        \
    }                                                                               \
    return true;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default: return false;
  }
}

}  // namespace pa
