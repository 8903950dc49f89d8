// Unit planning shared by the persistent decode kernels (device code, not
// installed). A unit is one (sequence, KV head, partition) - or one
// (sequence, KV head) in single-pass mode - and produces one output record;
// each persistent workgroup owns up to MAXU units, planned by one wavefront
// at kernel start from the device-side context lengths.
#pragma once

#include "launch.h"
#include "pa_device.h"

namespace pa {
namespace persist {

constexpr int MAXU = 64;  // candidate units per workgroup (one per lane)

// Partitions of one sequence: T (context clamped to the table's capacity),
// full partitions, whether a last, partial one follows, and whether the
// sequence's outputs must be poisoned (context longer than the table or, in
// split mode, than max_parts partitions).
struct SeqParts {
  int T, nfull, partial, bad;
};

// 32-bit arithmetic throughout: the host guarantees max_blocks_per_seq *
// block_size < 2^31, so the clamped T fits.
template <bool SPLIT>
__device__ __forceinline__ SeqParts seq_parts(const DecodeParams &p, int s) {
  SeqParts r{0, 0, 0, 0};
  if (s >= p.num_seqs) return r;
  int T = p.context_lens[s];
  T = T < 0 ? 0 : T;
  const int cap = p.max_blocks_per_seq * p.block_size;
  if (T > cap) {
    r.bad = 1;
    T = cap;
  }
  r.T = T;
  if (SPLIT) {
    const unsigned P = (unsigned)p.partition_size;
    unsigned nf = (unsigned)T / P;
    unsigned np = nf + ((unsigned)T != nf * P);  // ceil(T / P)
    if (np > (unsigned)p.max_parts) {
      r.bad = 1;  // T > max_parts * P
      np = (unsigned)p.max_parts;
    }
    if (nf > np) nf = np;
    r.nfull = (int)nf;
    r.partial = np > nf;
  } else {
    r.partial = 1;  // one unit per sequence (an empty one still writes zeros)
  }
  return r;
}

// The planner's lanes exchange values through LDS. A wavefront's LDS
// operations execute in program order, but the compiler treats each lane as
// a thread of its own and may move one lane's store past loads that only the
// other lanes make (it has merged such a store into a later one). This
// compiler barrier keeps every memory operation on its side.
__device__ __forceinline__ void lane_exchange_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(x, d, 64);
    if (lane >= d) x += t;
  }
  return x;
}

// First index i in [0, 64) with incl[i] > off (incl non-decreasing).
__device__ __forceinline__ int upper_index(const int *incl, int off) {
  int lo = 0, hi = 63;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > off)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// The workgroup's units, one per lane: lane k holds the unit assigned in
// round k, as (sequence, KV head, first token, end of its pool tokens) and
// partition * 4 + 2 * (takes the step's token from new_key/new_value) + bad. Units are enumerated as all full partitions (sequence-major)
// followed by the last, partial partitions ordered by decreasing size (for
// up to 64 sequences; in sequence order beyond that), and dealt to the
// workgroups in snake order (round k goes 0..grid-1 when k is even,
// grid-1..0 when odd). Big units go first and the round-by-round reversal
// evens out the loads; in single-pass mode every sequence is one partial
// unit, so the longest contexts start first. Run by one wavefront.
// scr: 192 ints of this wave's LDS (prologue scratch).
template <bool SPLIT>
__device__ inline void plan_units(const DecodeParams &p, int lane, int *scr, int4 &unit, int &bad_part,
                           int &active) {
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int NB = gridDim.x, b = blockIdx.x;
  const int a = lane * NB + ((lane & 1) ? NB - 1 - b : b);
  const int P = SPLIT ? p.partition_size : 0;
  int c_s = -1, c_h = 0, c_p = 0, c_T = 0, c_bad = 0;

  // Full partitions, sequence-major. The first 64 sequences' counts are
  // loaded once and serve the partial partitions below as well.
  const SeqParts sp_first = seq_parts<SPLIT>(p, lane);
  int F = 0;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const SeqParts sp = s0 == 0 ? sp_first : seq_parts<SPLIT>(p, s0 + lane);
    const int incl = wave_incl_scan(sp.nfull * H, lane);
    const int tot = __shfl(incl, 63, 64);
    lane_exchange_fence();
    scr[lane] = incl;
    lane_exchange_fence();
    const int off = a - F;
    const bool hit = off >= 0 && off < tot;
    const int i = hit ? upper_index(scr, off) : lane;
    const int T_i = __shfl(sp.T, i, 64), bad_i = __shfl(sp.bad, i, 64);
    if (hit) {
      const int r = off - (i ? scr[i - 1] : 0);
      c_s = s0 + i;
      c_p = r / H;
      c_h = r - c_p * H;
      c_T = T_i;
      c_bad = bad_i;
    }
    F += tot;
  }

  // Last, partial partitions.
  int NPH = 0;  // partial units
  if (S <= 64) {
    const SeqParts sp = sp_first;
    // A unique key per sequence that orders by decreasing size, then by
    // increasing sequence index; the rank is the count of larger keys.
    // Every lane reads all 64 keys from LDS (broadcast reads, no serial
    // dependency); lanes past S hold -1.
    const int sz = sp.T - sp.nfull * P;
    const int key = sp.partial ? (min(sz, (1 << 25) - 1) << 6) | (63 - lane) : -1;
    scr[128 + lane] = key;
    lane_exchange_fence();
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
      const int4 k4 = *reinterpret_cast<const int4 *>(&scr[128 + j]);
      rank += (k4.x > key) + (k4.y > key) + (k4.z > key) + (k4.w > key);
    }
    lane_exchange_fence();
    if (sp.partial) scr[64 + rank] = lane;
    lane_exchange_fence();
    const int nps = __popcll(__builtin_amdgcn_ballot_w64(sp.partial != 0));
    NPH = nps * H;
    const int off = a - F;
    const bool hit = off >= 0 && off < NPH;
    const int q = hit ? off / H : 0;
    const int sel = hit ? scr[64 + q] : lane;
    const int T_i = __shfl(sp.T, sel, 64), bad_i = __shfl(sp.bad, sel, 64);
    const int nf_i = __shfl(sp.nfull, sel, 64);
    if (hit) {
      c_s = sel;
      c_h = off - q * H;
      c_p = nf_i;
      c_T = T_i;
      c_bad = bad_i;
    }
  } else {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const SeqParts sp = seq_parts<SPLIT>(p, s0 + lane);
      const int incl = wave_incl_scan(sp.partial * H, lane);
      const int tot = __shfl(incl, 63, 64);
      lane_exchange_fence();
      scr[lane] = incl;
      lane_exchange_fence();
      const int off = a - F - NPH;
      const bool hit = off >= 0 && off < tot;
      const int i = hit ? upper_index(scr, off) : lane;
      const int T_i = __shfl(sp.T, i, 64), bad_i = __shfl(sp.bad, i, 64);
      const int nf_i = __shfl(sp.nfull, i, 64);
      if (hit) {
        c_s = s0 + i;
        c_h = off - (i ? scr[i - 1] : 0);
        c_p = nf_i;
        c_T = T_i;
        c_bad = bad_i;
      }
      NPH += tot;
    }
  }

  // Only a unit inside the batch is ever entered.
  active = c_s >= 0 && c_s < S && c_h >= 0 && c_h < H && c_T >= 0;
  if (!active) {
    unit = make_int4(0, 0, 0, 0);
    bad_part = 0;
    return;
  }
  int lo = 0, hi = c_T;
  if (SPLIT) {
    lo = c_p * P;
    hi = c_T < lo + P ? c_T : lo + P;
  }
  // A decode step's last unit of a sequence takes its final token from the
  // step's K/V rows: the pool part of the unit ends one token earlier.
  const int app = p.step && c_T > 0 && hi == c_T && !c_bad;
  unit = make_int4(c_s, c_h, lo, hi - app);
  bad_part = c_p * 4 + app * 2 + c_bad;
}

// ---- Longest-first deal.
//
// The snake deal above balances unit counts, not work: on a batch whose
// full partitions all cost the same and whose last partitions vary, its
// second round lands small units on workgroups that already hold a full
// one. plan_units_lpt deals the same units longest-first instead: each unit,
// largest first, goes to the workgroup with the least work so far (ties to
// the lowest index). A unit's cost is the stream positions it gives wave 0
// (the most of any wave): ceil(tiles / kPlanWaves), padded to even. The result
// does not depend on the deal (a unit's arithmetic is the same on every
// workgroup); only the balance does. It is made by launches that store
// their plan (a step's later layers read it) and only where it can beat
// the snake deal.
//
// Units of equal cost are dealt at once: with costs c, the greedy choice is
// the least (load + i c, workgroup) "slot" among all workgroups' free slots,
// so n units of cost c take the n least slots in that order. A binary search
// on the slot value finds the level of the n-th slot: every slot below it is
// taken, and of the slots at it, those of the lowest-indexed workgroups
// make up the rest. Within a cost class the
// units are numbered by sequence, then partition, then head, and a
// workgroup's slots map to those numbers by their rank among all slots.
constexpr int kPlanWaves = 8;       // wavefronts of the persistent kernels
constexpr int kLptMaxGroups = 256;  // workgroups one wavefront tracks (4 per lane)

// Wave-wide reductions (every lane receives the result; all 64 lanes must
// be active): rotations by 8, 4, 2 and 1 inside each 16-lane row, then the
// four rows combined with two lane swaps. Integer DPP and swaps, no LDS.
template <int CTRL>
__device__ __forceinline__ int lpt_dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
template <typename Op>
__device__ __forceinline__ int wave_reduce(int x, Op op) {
  x = op(x, lpt_dpp<0x128>(x));
  x = op(x, lpt_dpp<0x124>(x));
  x = op(x, lpt_dpp<0x122>(x));
  x = op(x, lpt_dpp<0x121>(x));
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = op((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  // The same in every lane: readfirstlane lets the compiler keep it, and the
  // control flow that depends on it, scalar.
  return __builtin_amdgcn_readfirstlane(op((int)b[0], (int)b[1]));
}
__device__ __forceinline__ int wave_sum(int x) {
  return wave_reduce(x, [](int u, int v) { return u + v; });
}
__device__ __forceinline__ int wave_max(int x) {
  return wave_reduce(x, [](int u, int v) { return u > v ? u : v; });
}
__device__ __forceinline__ int wave_min(int x) {
  return wave_reduce(x, [](int u, int v) { return u < v ? u : v; });
}

// Inclusive prefix sum over the wave's lanes (all 64 active): shifts by 1,
// 2, 4 and 8 inside each 16-lane row, then the totals of the rows below
// added on.
__device__ __forceinline__ int wave_incl_scan_dpp(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Stream positions of wave 0 for a unit of nt tiles, halved (costs are even).
__device__ __forceinline__ int lpt_half_cost(int nt) {
  const int c = (nt + kPlanWaves - 1) / kPlanWaves;
  const int pc = c + (c & 1);
  return pc > 2 ? pc / 2 : 1;  // an empty unit still merges and stores
}

// Division by a class's cost c (uniform) through a multiply-high by
// m = ceil(2^32 / c) (c > 1): exact for t * c < 2^32, which the planner's
// bounds guarantee.
struct LptDiv {
  int c;
  uint32_t m;
  __device__ __forceinline__ int floor_div(int t) const {
    return c == 1 ? t : (int)__umulhi((uint32_t)t, m);
  }
};
__device__ __forceinline__ LptDiv lpt_div(int c) {
  return LptDiv{c, c > 1 ? 0xffffffffu / (uint32_t)c + 1u : 0u};
}
// Slots of one workgroup with load L below level v: ceil((v - L) / c)
// (selects, no branches).
__device__ __forceinline__ int lpt_slots_below(int v, int L, const LptDiv &d) {
  const int t = v - L;
  const int q = d.floor_div(t > 0 ? t - 1 : 0) + 1;
  return t > 0 ? q : 0;
}
// Whether the workgroup has a slot exactly at level v.
__device__ __forceinline__ int lpt_slot_at(int v, int L, const LptDiv &d) {
  const int t = v - L;
  const int tt = t > 0 ? t : 0;
  return (t >= 0) & (d.floor_div(tt) * d.c == tt);
}

// Deals this workgroup's units longest-first (one per lane, as plan_units).
// Returns false, leaving the outputs alone, where it does not apply: more
// than 64 sequences, more than kLptMaxGroups workgroups, or a deal that
// would give a workgroup more than MAXU units. Run by one wavefront, with
// the same inputs and so the same deal on every workgroup.
// scr: 192 ints of this wave's LDS (prologue scratch).
template <bool SPLIT, int TILE_TOKENS>
__device__ inline bool plan_units_lpt(const DecodeParams &p, int lane, int *scr, int4 &unit,
                                      int &bad_part, int &active) {
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int NB = gridDim.x, b0 = blockIdx.x;
  if (S > 64 || NB > kLptMaxGroups) return false;
  const int P = SPLIT ? p.partition_size : 0;
  const SeqParts sp = seq_parts<SPLIT>(p, lane);
  const int live_seq = lane < S;

  // This lane's sequence: its partitions fall into at most three cost
  // classes: full ones, the last full one when it holds the step's token,
  // and the last partial one (single pass: the whole context).
  int nfa = 0, lastapp = 0, cf = 0, cfa = 0, cp = 0;
  if (live_seq) {
    if (SPLIT) {
      lastapp = p.step && !sp.partial && sp.nfull > 0 && sp.T > 0 && !sp.bad;
      nfa = sp.nfull - lastapp;
      if (nfa > 0) cf = lpt_half_cost(P / TILE_TOKENS);
      if (lastapp) cfa = lpt_half_cost((P - 1 + TILE_TOKENS - 1) / TILE_TOKENS + 1);
      if (sp.partial) {
        const int z = sp.T - sp.nfull * P;
        const int app = p.step && sp.T > 0 && !sp.bad;
        cp = lpt_half_cost((z - app + TILE_TOKENS - 1) / TILE_TOKENS + app);
      }
    } else {
      const int app = p.step && sp.T > 0 && !sp.bad;
      cp = lpt_half_cost((sp.T - app + TILE_TOKENS - 1) / TILE_TOKENS + app);
    }
  }

  // Where the snake deal is already optimal, keep it (it costs less to
  // make): every unit costs the same (equal unit counts, which the snake
  // deal gives, are then optimal), or no workgroup gets a second unit.
  const int cmax = wave_max(max(cf, max(cfa, cp)));
  const int big = 1 << 30;
  const int cmin = wave_min(min(cf > 0 ? cf : big, min(cfa > 0 ? cfa : big, cp > 0 ? cp : big)));
  const int nunits = wave_sum(live_seq ? H * (nfa + lastapp + (cp > 0 ? 1 : 0)) : 0);
  if (cmin == cmax || nunits <= NB) return false;
  // Multiply-high division stays exact while every level times every cost
  // is below 2^32: levels stay below twice the total work, so bound both.
  const int64_t mywork = (int64_t)H * ((int64_t)nfa * cf + cfa + cp);
  const int work = wave_sum((int)(mywork < (1 << 21) ? mywork : (1 << 21)));
  if (cmax > (1 << 10) || work > (1 << 20)) return false;

  // Loads (halved costs) of workgroups 4 lane + k; absent ones never take a slot.
  constexpr int kAbsent = 0x3fffffff;
  int L[4], U[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    L[k] = 4 * lane + k < NB ? 0 : kAbsent;
    U[k] = 0;
  }
  int nown = 0;         // this workgroup's units so far (uniform)
  int floor_level = 0;  // every load is at least this
  int lmax = 0;         // no load is above this
  int *own = scr + 64;  // [64][2] this workgroup's units: sequence, partition * H + head
  for (;;) {
    const int c = wave_max(max(cf, max(cfa, cp)));
    if (c == 0) break;
    const int A = cf == c ? nfa : 0, B = cfa == c ? 1 : 0, C1 = cp == c ? 1 : 0;
    if (cf == c) cf = 0;
    if (cfa == c) cfa = 0;
    if (cp == c) cp = 0;
    const int incl = wave_incl_scan_dpp(H * (A + B + C1), lane);
    const int n = __builtin_amdgcn_readlane(incl, 63);
    const LptDiv dc = lpt_div(c);

    // Level v* of the n-th least slot: the largest v with fewer than n slots
    // below it. After a class every load is at least that class's level
    // (the workgroups below it took every slot up to it), so the search
    // starts there with no slot below; the highest load is at most the
    // previous highest or the last level plus its cost.
    auto below = [&](int v) {
      int t = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) t += lpt_slots_below(v, L[k], dc);
      return wave_sum(t);
    };
    int lo = floor_level, hi = lmax + ((n + NB - 1) / NB) * c, below_lo = 0;
    while (hi - lo > 1) {
      const int mid = lo + ((hi - lo) >> 1);
      const int bm = below(mid);
      if (bm < n) {
        lo = mid;
        below_lo = bm;
      } else {
        hi = mid;
      }
    }
    const int vstar = lo;
    const int rest = n - below_lo;  // slots at v* taken, lowest workgroups first
    // Workgroups with a slot at v* in lower-indexed lanes: one ballot per
    // workgroup of a lane, counted below this lane with mbcnt.
    int ex[4], before = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ex[k] = lpt_slot_at(vstar, L[k], dc);
      const uint64_t m = __builtin_amdgcn_ballot_w64(ex[k] != 0);
      before += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    }
    int take[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      take[k] = lpt_slots_below(vstar, L[k], dc) + (ex[k] && before < rest ? 1 : 0);
      before += ex[k];
    }

    // This workgroup's slots of the class, each mapped to a unit by its rank.
    const int src = b0 >> 2, kk = b0 & 3;
    const int myL = __builtin_amdgcn_readlane(kk == 0 ? L[0] : kk == 1 ? L[1] : kk == 2 ? L[2] : L[3], src);
    const int myk =
        __builtin_amdgcn_readlane(kk == 0 ? take[0] : kk == 1 ? take[1] : kk == 2 ? take[2] : take[3], src);
    for (int i = 0; i < myk; ++i) {
      const int v = myL + i * c;
      int t = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int b = 4 * lane + k;
        t += lpt_slots_below(v, L[k], dc) * 512 + ((b < b0) & lpt_slot_at(v, L[k], dc));
      }
      t = wave_sum(t);  // slots below v (x 512) and workgroups before this one at v
      const int rank = (t >> 9) + (t & 511);
      // The unit's sequence: the first whose inclusive count exceeds rank.
      const int s = __popcll(__builtin_amdgcn_ballot_w64(incl <= rank));
      const int r = rank - (s ? __builtin_amdgcn_readlane(incl, s - 1) : 0);
      const int q = r / H, h = r - (r / H) * H;
      const int As = __builtin_amdgcn_readlane(A, s), Bs = __builtin_amdgcn_readlane(B, s);
      const int nfs = __builtin_amdgcn_readlane(sp.nfull, s);
      const int part = q < As ? q : (q < As + Bs ? nfs - 1 : nfs);
      if (nown < MAXU && lane == 0) {
        own[2 * nown] = s;
        own[2 * nown + 1] = part * H + h;
      }
      ++nown;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (L[k] != kAbsent) L[k] += take[k] * c;
      U[k] += take[k];
    }
    floor_level = vstar;
    lmax = max(lmax, vstar + c);
  }
  if (wave_max(max(max(U[0], U[1]), max(U[2], U[3]))) > MAXU) return false;
  lane_exchange_fence();

  active = 0;
  unit = make_int4(0, 0, 0, 0);
  bad_part = 0;
  const int mine_s = lane < nown ? own[2 * lane] : 0;
  const int mine_ph = lane < nown ? own[2 * lane + 1] : 0;
  const int T_i = __shfl(sp.T, mine_s, 64), bad_i = __shfl(sp.bad, mine_s, 64);
  if (lane < nown) {
    const int part = mine_ph / H, h = mine_ph - part * H;
    int lo = 0, hi = T_i;
    if (SPLIT) {
      lo = part * P;
      hi = T_i < lo + P ? T_i : lo + P;
    }
    const int app = p.step && T_i > 0 && hi == T_i && !bad_i;
    active = mine_s < S && h < H && T_i >= 0;
    if (active) {
      unit = make_int4(mine_s, h, lo, hi - app);
      bad_part = part * 4 + app * 2 + bad_i;
    }
  }
  return true;
}

// ---- Plan cache (see DecodeParams::plan). A workgroup's slot is tagged with
// the launch that wrote it; kind distinguishes kernels whose slots differ.
typedef uint32_t plan_u32x4 __attribute__((ext_vector_type(4)));

struct PlanSlot {
  __amdgpu_buffer_rsrc_t r;  // this workgroup's slot (empty without a buffer)
  plan_u32x4 tag;            // kind and mode, grid, batch size, partition size
  bool use;                  // the slot holds this launch's plan
  plan_u32x4 ids;            // the wave's stored block ids (up to four)
  plan_u32x4 unit;           // with_units: the lane's stored unit ...
  uint32_t bp;               // ... and its partition * 4 + flags word
};

// The wave's stored block ids and (with_units, wave 0) the lane's unit
// entry are loaded together with the header, before the tag is checked, so
// that a launch reading its plan waits for one round trip, not two. They
// lie inside the slot, so the loads are harmless when the tag turns out not
// to match (the values are then not used).
template <bool SPLIT>
__device__ inline PlanSlot plan_slot(const DecodeParams &p, uint32_t kind, int wave,
                                     bool with_units) {
  PlanSlot ps;
  ps.r = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<uint8_t *>(p.plan) + (int64_t)blockIdx.x * kPlanWgBytes, (short)0,
      p.plan ? kPlanWgBytes : 0, 0x00020000);
  ps.tag = plan_u32x4{(uint32_t)kPlanMagic | kind | (SPLIT ? 1u : 0u) | (p.step ? 2u : 0u),
                      gridDim.x, (uint32_t)p.num_seqs, (uint32_t)p.partition_size};
  ps.use = false;
  ps.ids = plan_u32x4{0u, 0u, 0u, 0u};
  ps.unit = plan_u32x4{0u, 0u, 0u, 0u};
  ps.bp = 0xffffffffu;
  // Bit 31 of the epoch asks for a fresh plan, stored under the epoch
  // without that bit.
  if (p.plan && !(p.plan_epoch & 0x80000000u)) {
    const plan_u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(ps.r, kPlanHdr, 0, 0);
    const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(ps.r, kPlanHdr + 16, 0, 0);
    ps.ids = __builtin_amdgcn_raw_buffer_load_b128(ps.r, kPlanIds + kPlanIdBytes * wave, 0, 0);
    if (with_units) {
      const int lane = threadIdx.x & 63;
      ps.unit = __builtin_amdgcn_raw_buffer_load_b128(ps.r, kPlanUnits + 16 * lane, 0, 0);
      ps.bp = __builtin_amdgcn_raw_buffer_load_b32(ps.r, kPlanBp + 4 * lane, 0, 0);
    }
    ps.use = __builtin_amdgcn_readfirstlane(h[0]) == ps.tag[0] &&
             __builtin_amdgcn_readfirstlane(h[1]) == ps.tag[1] &&
             __builtin_amdgcn_readfirstlane(h[2]) == ps.tag[2] &&
             __builtin_amdgcn_readfirstlane(h[3]) == ps.tag[3] &&
             __builtin_amdgcn_readfirstlane(e) == p.plan_epoch;
  }
  return ps;
}

// Wave 0: the workgroup's units, from the slot (loaded by plan_slot with
// with_units) when it holds this launch's plan (each checked, so that a plan made for other inputs can give wrong
// numbers but never an access outside the caller's buffers), else planned
// here and, with a buffer, stored with the tag for the launches after this
// one. Every path issues the same stores (the unwanted ones go past
// num_records and are dropped).
template <bool SPLIT, int TILE_TOKENS>
__device__ inline void plan_or_load_units(const DecodeParams &p, const PlanSlot &ps, int lane,
                                          int *scr, int4 &my, int &my_bp, int &my_act) {
  if (ps.use) {
    const plan_u32x4 u = ps.unit;
    const int bp = (int)ps.bp;
    my = make_int4((int)u[0], (int)u[1], (int)u[2], (int)u[3]);
    const int cap = p.max_blocks_per_seq * p.block_size;
    my_act = bp >= 0 && my.x >= 0 && my.x < p.num_seqs && my.y >= 0 && my.y < p.num_kv_heads &&
             my.z >= 0 && my.z <= my.w && my.w <= cap &&
             (bp >> 2) < (SPLIT ? p.max_parts : 1) && (p.step || (bp & 2) == 0);
    my_bp = my_act ? bp : 0;
    if (!my_act) my = make_int4(0, 0, 0, 0);
  } else if (!p.plan || !plan_units_lpt<SPLIT, TILE_TOKENS>(p, lane, scr, my, my_bp, my_act)) {
    // Without a plan buffer every launch deals for itself, and there the
    // snake deal pays: on the mixed batch the longest-first deal takes about
    // 12 us longer to make than it saves in one launch (2.7 us).
    plan_units<SPLIT>(p, lane, scr, my, my_bp, my_act);
  }
  if (p.plan) {
    const int drop = ps.use ? kPlanWgBytes : 0;
    __builtin_amdgcn_raw_buffer_store_b128(
        plan_u32x4{(uint32_t)my.x, (uint32_t)my.y, (uint32_t)my.z, (uint32_t)my.w}, ps.r,
        drop + kPlanUnits + 16 * lane, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(my_act ? (uint32_t)my_bp : 0xffffffffu, ps.r,
                                          drop + kPlanBp + 4 * lane, 0, 0);
    const uint32_t hv = lane < 4 ? ps.tag[lane & 3] : (p.plan_epoch & 0x7fffffffu);
    __builtin_amdgcn_raw_buffer_store_b32(hv, ps.r,
                                          lane < 5 ? drop + kPlanHdr + 4 * lane : kPlanWgBytes,
                                          0, 0);
  }
}

// A wave's k-th stored block id (lane 0 stores; every lane holds the same).
// The store is dropped when the workgroup read its slot (use: wave 0's
// decision, shared through LDS).
__device__ inline void plan_store_id(const PlanSlot &ps, bool use, int wave, int k, int lane,
                                     int id) {
  const int drop = use || lane != 0 ? kPlanWgBytes : 0;
  __builtin_amdgcn_raw_buffer_store_b32((uint32_t)id, ps.r,
                                        drop + kPlanIds + kPlanIdBytes * wave + 4 * k, 0, 0);
}

// Compute units of the current device (cached per device).
inline int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace persist
}  // namespace pa
