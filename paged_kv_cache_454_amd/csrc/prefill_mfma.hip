// Chunked paged prefill on the matrix cores (BF16 in, fp32 accumulation),
// head_dim 256: "vLLM Architecture, Memory and Benchmarks Deep Dive", s.4
// (a long prompt is processed in chunks, e.g. 512 tokens, against the paged
// cache) and "Inside vLLM", "FlashAttention-2 Integration" (one fused causal
// pass over packed, unpadded queries, no n x n score matrix in memory).
//
// Rows. The query rows of one KV head are the (position j, query head hh)
// pairs of a sequence's chunk, flattened as r = j * G + hh, so the G query
// heads that share a KV head sit in the same tile and every K/V byte staged
// in LDS serves all of them. A workgroup owns 256 rows (8 wavefronts x 32,
// two per SIMD).
//
// Per 32-token K/V tile (K and V gathered through the block table straight
// into an LDS ring of 4 tiles by buffer-to-LDS loads, 3 tiles in flight,
// token pairs 1 KiB + 16 B (K) or + 32 B (V) apart; one barrier per tile,
// after each wave's own wait for its loads of that tile):
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
//    lane that computed them; the A operand is read from the row-major V
//    tile with two ds_read_b64_tr_b16 (transposing 4x4 blocks of 16-bit
//    elements across lanes). The k order of the tokens in both operands is
//    the same permutation, which a sum over tokens ignores.
// Causality: query j of a chunk of n sits at position T - n + j and sees
// tokens [0, T - n + j]; a workgroup stops at the last tile its rows can see.
#include <math.h>

#include "launch.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int D = 256;
constexpr int WAVES = 8;                // two per SIMD
constexpr int ROWS = WAVES * 32;        // query rows per workgroup
constexpr int KT = 32;                  // tokens per K/V tile
constexpr int STAGES = 4;               // K/V tiles in the LDS ring (3 in flight)
constexpr int PAIR = 1040;              // K tile: bytes per token pair in LDS, 2 x 512 + 16
constexpr int PAIR_V = 1056;            // V tile: bytes per token pair in LDS, 2 x 512 + 32
constexpr int TILE_K = (KT / 2) * PAIR;    // one K tile
constexpr int TILE_V = (KT / 2) * PAIR_V;  // one V tile
constexpr int MAX_TABLE = 2048;         // block ids staged in LDS
constexpr int NXCD = 8;                 // XCDs (dies) the workgroups are dealt to
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

// l + lo + hi of a pair of BF16 weights in one instruction (a dot product
// with (1, 1)): the row sum uses exactly the rounded weights the matrix
// products use.
__device__ __forceinline__ float row_sum_add(uint32_t pair, float l) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, l, false);
}

// s_waitcnt immediates: vmcnt(n) with the other counters left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kVmcnt8 = waitcnt_vm(8);

// LDS byte offset of channel ch of token row t in a K tile: token pairs are
// 1 KiB apart plus 16 bytes, so the 16 lanes a 16-byte read serves per cycle
// (64 banks of 4 bytes) address 16 different 16-byte bank slots, and every
// fragment address is a lane base plus an immediate. V tiles use the same
// layout with pairs 1 KiB + 32 bytes apart: the transposed 8-byte reads serve
// 32 lanes per cycle, whose addresses step by two pairs, and two pairs must
// then be 64 bytes of banks apart for the 32 to cover all 64 banks once
// (with 16 bytes, lanes two pairs apart met on the same banks).
__device__ __forceinline__ int tile_off(int t, int ch) { return (t >> 1) * PAIR + (t & 1) * 512 + ch * 2; }

// Token of the tile in slot m (0..31) of the S^T rows and of the P.V sums.
// Any permutation is correct as long as K, V and the mask agree (the
// products sum over tokens); this one spreads LDS reads over the banks: the
// 8 K rows read together by lanes m..m+7 lie in 8 different 16-byte slots
// of a 128-byte bank line, and the 4 V rows of a transpose read lie in 4
// disjoint 32-byte spans (rows of a pair are 512 bytes apart, i.e. on the
// same banks, so neighbouring slots take tokens from different pairs).
__device__ __forceinline__ int tok_of(int m) {
  return 16 * ((m >> 3) & 1) + 4 * (m & 3) + 2 * ((m >> 2) & 1) + (m >> 4);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8 bytes addressed by lane 4e + i / 4, for e = 0..3.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint64_t tr_read(const lds_u8 *p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) bf16x4 lds_v4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4 *)p);
  return __builtin_bit_cast(uint64_t, v);
}

// One buffer-to-LDS load: each lane's 16 bytes at `voffset` of the buffer
// go to LDS address lds_addr + 16 * lane. Issued through inline assembly so
// that the compiler's wait-count pass does not track it: that pass cannot
// tell the ring's stages apart and would wait for every outstanding load
// before each LDS read. The kernel waits for these loads itself (vmcnt, then
// a barrier) before any wave reads the stage they fill; vector memory
// operations complete in order, so the compiler's own waits for other loads
// stay correct (they only become stricter).
// M0 (the LDS address of the load) is declared clobbered, so the compiler
// sets it again wherever it needs it; the one wait state between writing
// M0 and the load that reads it is an explicit s_nop.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_load16(u32x4v rsrc, uint32_t lds_addr, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

// 16 bytes from LDS.
__device__ __forceinline__ uint4 lds_read16(const lds_u8 *p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(__attribute__((address_space(3))) const u32x4 *)p;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Buffer resource over [base, base + bytes): raw buffer, no stride, the
// same dword 3 as the rest of the library's resources.
__device__ __forceinline__ u32x4v raw_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4v r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
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
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_kernel(PrefillParams p, int row_blocks) {
  // The ring's stages are separate arrays and the loop below is unrolled by
  // STAGES, so every buffer-to-LDS load and every LDS read names its stage
  // statically: the compiler can then tell that the loads issued for tile
  // it+3 do not write the stage being read, and does not wait for them.
  typedef uint8_t Stage[TILE_K + TILE_V];  // K tile, then V tile
  __shared__ __attribute__((aligned(16))) Stage stage0, stage1, stage2, stage3;
  // The stages by LDS address (constants), so that no generic pointer has
  // to be converted in the loop.
  lds_u8 *const st0 = (lds_u8 *)&stage0[0];
  lds_u8 *const st1 = (lds_u8 *)&stage1[0];
  lds_u8 *const st2 = (lds_u8 *)&stage2[0];
  lds_u8 *const st3 = (lds_u8 *)&stage3[0];
  static_assert(STAGES == 4, "the ring is four named stages");
  __shared__ int tab[MAX_TABLE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform (LDS DMA addresses)
  const int half = lane >> 5;  // which 8 of a 16-wide k step this lane supplies
  const int l32 = lane & 31;

  // Workgroup id -> (sequence, KV head, row block). Ids are dealt to the 8
  // XCDs round-robin (id % 8), and each XCD has its own L2: the (sequence,
  // KV head) pairs are dealt to the XCDs and each keeps all its row blocks on
  // its XCD, so they read the sequence's K/V through one L2. Later row
  // blocks see more tokens: launch them first.
  const int SK = p.num_seqs * p.num_kv_heads;
  const int xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD;
  const int q_round = slot / row_blocks;  // the XCD's q_round-th pair
  int sk;
  if (SK <= 64) {
    // Pairs are dealt by cost: every wave ranks the pairs by their K/V tiles
    // summed over the row blocks (largest first, ties by index) and deals
    // them to the XCDs in snake order (round q goes 0..7 when even, 7..0
    // when odd), so each XCD gets an equal count and nearly equal work, and
    // each XCD starts its largest pairs first.
    int cost = -1;
    if (lane < SK) {
      const int si = lane / p.num_kv_heads;
      const int ni = p.query_start_loc[si + 1] - p.query_start_loc[si];
      const int Ti = p.context_lens[si];
      const int nr = ni * G;
      cost = 0;
      if (ni > 0 && Ti >= ni && (int64_t)Ti <= (int64_t)p.max_blocks_per_seq * p.block_size)
        for (int b = 0; b * ROWS < nr; ++b) {
          const int lim = Ti - ni + (min(b * ROWS + ROWS, nr) - 1) / G + 1;
          cost += (lim + KT - 1) / KT;
        }
    }
    int rank = 0;
    for (int k = 0; k < 64; ++k) {
      const int ck = __builtin_amdgcn_readlane(cost, k);
      rank += ck > cost || (ck == cost && k < lane);
    }
    const int want = NXCD * q_round + ((q_round & 1) ? NXCD - 1 - xcd : xcd);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < SK && rank == want);
    if (hit == 0) return;
    sk = __builtin_ctzll(hit);
  } else {
    sk = xcd + NXCD * q_round;
    if (sk >= SK) return;
  }
  const int rb = row_blocks - 1 - slot % row_blocks;
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
  // Tiles that every row of this wave sees entirely need no mask.
  const int wave_first_row = min(rb * ROWS + wave * 32, nrows - 1);
  const int wave_min_lim = bad ? 0 : ctx0 + wave_first_row / G + 1;

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

  // Tile staging: buffer-to-LDS loads, 1 KiB (two token rows) per wavefront
  // instruction, two K and two V instructions per wavefront per tile. The
  // resource of each instruction covers just the valid rows of its token pair
  // (zero bytes past the context or for an invalid block id), so the LDS
  // receives zeros there without a memory access.
  // Tiles are issued in order, so each of the wave's two token pairs keeps a
  // cursor (table index, token within the block) that moves on by one tile
  // per issue: no division per load.
  const int q_kt = KT / bs, r_kt = KT % bs;
  int cur_b[KT / 2 / WAVES], cur_r[KT / 2 / WAVES];
#pragma unroll
  for (int i = 0; i < KT / 2 / WAVES; ++i) {
    const int tok0 = 2 * (wave * (KT / 2 / WAVES) + i);
    cur_b[i] = tok0 / bs;
    cur_r[i] = tok0 - cur_b[i] * bs;
  }
  auto issue_tile = [&](int it, lds_u8 *dst) {
    const int t_base = it * KT;
#pragma unroll
    for (int i = 0; i < KT / 2 / WAVES; ++i) {
      const int pi = wave * (KT / 2 / WAVES) + i;  // token pair of the tile, 0..15
      const int tok0 = t_base + 2 * pi;
      int nv = wg_limit - tok0;
      nv = __builtin_amdgcn_readfirstlane(nv < 0 ? 0 : (nv > 2 ? 2 : nv));
      // The table index stays inside the staged table; past the context the
      // id read is not used (nv = 0).
      int blk = __builtin_amdgcn_readfirstlane(tab[cur_b[i] < MAX_TABLE ? cur_b[i] : MAX_TABLE - 1]);
      if (nv == 0 || (uint32_t)blk >= (uint32_t)nb) {  // also blk < 0
        nv = 0;
        blk = 0;
      }
      const int64_t off = (int64_t)blk * block_stride + (int64_t)cur_r[i] * D;
      cur_r[i] += r_kt;
      cur_b[i] += q_kt;
      if (cur_r[i] >= bs) {
        cur_r[i] -= bs;
        cur_b[i] += 1;
      }
      const uint32_t kdst = (uint32_t)(uintptr_t)(dst + pi * PAIR);
      const uint32_t vdst = (uint32_t)(uintptr_t)(dst + TILE_K + pi * PAIR_V);
      lds_load16(raw_rsrc(kpool + off, nv * D * 2), kdst, lane * 16);
      lds_load16(raw_rsrc(vpool + off, nv * D * 2), vdst, lane * 16);
    }
  };

  f32x16 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = kNoMax, l = 0.f;
  const float sl2 = p.scale * kLog2e;
  const bool pos_scale = sl2 > 0.f;
  const float zscale = pos_scale ? sl2 : 1.f;  // what the kept scores still need

  // Lane roles in the transpose reads of V (A operand of O^T): the lane is
  // k = lane % 16 of a 16-lane group; it supplies the address of token
  // row tok(k / 4) at channels 4 * (k % 4) of the group's 16-channel slice.
  // For the chunk c of 16 slots, the lane addresses slot 16c + 4*half +
  // kq/4 (first read) and 16c + 8 + 4*half + kq/4 (second read), i.e.
  // tokens 4*(kq/4) + 2*half + c and 16 + the same: pairs 2*(kq/4) + half
  // and 8 + that, row c.
  const int grp = lane >> 4, kq = lane & 15;
  const int vd0 = 16 * (grp & 1) + 4 * (kq & 3);  // channel within the 32-channel tile
  const int vpair = 2 * (kq >> 2) + half;

  // Tiles are issued unconditionally: one past the last needed token has an
  // empty resource, so it reads nothing and fills a stage no one reads with
  // zeros. Every step then issues the same 4 instructions per wave and the
  // compiler's wait counts stay exact (a conditional issue would make it
  // wait for every load before each LDS read).
  // The query fragments must be in registers before the first tile loads
  // leave: a wait for them inside the loop would also wait for every tile
  // load in flight.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  issue_tile(0, st0);
  issue_tile(1, st1);
  issue_tile(2, st2);

  // One tile: `cur` holds tile it, `nxt` (the stage tile it-1 used) receives
  // tile it+3.
  auto step = [&](int it, const lds_u8 *cur, lds_u8 *nxt) {
    // This wave's loads for tile it are complete once only the two later
    // tiles' are outstanding (4 instructions per tile per wave).
    __builtin_amdgcn_s_waitcnt(kVmcnt8);
    __syncthreads();  // every wave's loads for tile it are in LDS; stage it-1 is free
    const lds_u8 *kl = cur;
    const lds_u8 *vl = cur + TILE_K;
    const int t0 = it * KT;

    // S^T (32 tokens x 32 rows). The K fragments are read three steps
    // ahead of their products, in a fixed order.
    f32x16 s0;
    const lds_u8 *krow = kl + tile_off(tok_of(l32), 8 * half);
    uint4 kf[4];
#pragma unroll
    for (int k = 0; k < 3; ++k) kf[k] = lds_read16(krow + 32 * k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k + 3 < 16) kf[(k + 3) & 3] = lds_read16(krow + 32 * (k + 3));
      s0 = k == 0 ? mfma(kf[0], qf[0], f32x16{}) : mfma(kf[k & 3], qf[k], s0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The loads of tile it+3 (into the stage tile it-1 left) go out here,
    // after the S products, and not right after the barrier, where every
    // wave of the workgroup would queue its address work on the compute
    // unit's one scalar unit while the matrix cores wait.
    issue_tile(it + STAGES - 1, nxt);
    // Element e of the accumulator is slot 8*(e/4) + 4*half + e%4. The
    // scores stay unscaled here (for a positive scale the max commutes with
    // the scaling, and rounding is monotone, so the scaled max is exactly
    // the max of the scaled scores); the scale enters the exponent's fma.
    float z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = s0[e];
    if (!pos_scale) {
      asm volatile("");
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] *= sl2;
    }
    if (t0 + KT > wave_min_lim) {  // uniform: some token of the tile is masked for this wave
      // Only the tiles on the causal diagonal (and past short contexts)
      // take this branch; the empty statement keeps it a branch instead of
      // selects that every tile would pay for.
      asm volatile("");
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = t0 + tok_of(8 * (e >> 2) + 4 * half + (e & 3));
        z[e] = tok < limit ? z[e] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, z[e]);
    mx = other_half_max(mx) * zscale;
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
    // Weights as the B operand of O^T: chunk c takes elements 8c .. 8c+7,
    // i.e. slots 16c + 4*half + (0..3) and 16c + 8 + 4*half + (0..3).
    uint4 pw[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float pa = fast_exp2(__builtin_fmaf(z[8 * c + 2 * u], zscale, -m));
        const float pb = fast_exp2(__builtin_fmaf(z[8 * c + 2 * u + 1], zscale, -m));
        w4[u] = bf16_pair(pa, pb);
        l = row_sum_add(w4[u], l);
      }
      pw[c] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    // O^T (32 channels x 32 rows per dt) += V^T . P^T. The A operand comes
    // from the row-major V tile through two transpose reads whose token
    // order matches the weights'.
    const lds_u8 *vbase = vl + vpair * PAIR_V + 2 * vd0;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // row c of pair vpair, and of pair vpair + 8
        const uint64_t va = tr_read(vbase + c * 512 + dt * 64);
        const uint64_t vb = tr_read(vbase + c * 512 + 8 * PAIR_V + dt * 64);
        const uint4 a = make_uint4((uint32_t)va, (uint32_t)(va >> 32), (uint32_t)vb,
                                   (uint32_t)(vb >> 32));
        o[dt] = mfma(a, pw[c], o[dt]);
      }
    }
  };

  for (int it = 0; it < ntiles; it += STAGES) {
    step(it, st0, st3);
    if (it + 1 >= ntiles) break;
    step(it + 1, st1, st0);
    if (it + 2 >= ntiles) break;
    step(it + 2, st2, st1);
    if (it + 3 >= ntiles) break;
    step(it + 3, st3, st2);
  }
  // The loads issued for the three tiles past the end (empty, but they still
  // write LDS) finish before any wave of the workgroup ends.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

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

// The MFMA path covers BF16, head_dim 256, even block sizes (a token pair
// never straddles two blocks) and tables of up to 2048 blocks per sequence;
// false otherwise.
bool launch_prefill_mfma(const PrefillParams &p, hipStream_t stream) {
  if (p.head_dim != D || p.block_size % 2 != 0 || p.max_blocks_per_seq > MAX_TABLE) return false;
  const int group = p.num_q_heads / p.num_kv_heads;
  const int64_t row_blocks = ((int64_t)p.max_query_len * group + ROWS - 1) / ROWS;
  const int64_t sk = (int64_t)p.num_seqs * p.num_kv_heads;
  const int64_t grid = NXCD * row_blocks * ((sk + NXCD - 1) / NXCD);
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
