// plan.hip — the single-workgroup replica planner of libmoebal.
//
// One workgroup of 256 threads (the per-rank targets come from the host):
//  1. routed pairs per expert c_e (summed over sources by k_scan, or here
//     from d[s][e] or from a small table of block counts);
//  2. wave 0 runs the greedy with lane r = logical rank r (P <= 64): the
//     rank farthest above its target tau_r gives a replica of its heaviest
//     home expert to the rank farthest below its own target that has a free
//     slot and no copy yet, filling that rank up to its target. With equal
//     speeds every target is the water level T, the first rank is the
//     busiest and the second the least loaded;
//  3. all threads write slot quotas, cu_seqlens, loads and the status word.
// The lookup tables that turn a pair's stable rank into its dispatch row are
// built afterwards by k_tables (route.hip), one wave per expert.
//
// Every choice is a full-wave DPP reduction over keys that carry the lane or
// expert index in their low bits (or a ballot that picks the lowest lane, or
// a per-lane scan in index order), so ties resolve to the lowest rank /
// expert index and the result does not depend on timing.
//
// Sources: ISER-MoE, Methodology, HALO-Q Scheduler — Objective 1 (water
// level T = ceil(sum L_r / P)), stage 2 (busiest rank's heaviest home expert
// goes where a slot is free), stage 3 (smallest free helper index), stage 5
// (surplus routes onto the hosts' spare quotas); Zepp summary §4.1 (R replica
// slots per GPU); MoonEP, "What MoonEP enforces and how" (S*K rows per rank,
// planner-made cu_seqlens) and "Implementation details" (home experts, then
// prefetch slots, in one numbering); ViBE summary, Methodology, Variability-
// Informed Expert Placement (token target per GPU in proportion to its
// speed, experts to the GPU farthest below its target).
#include "mb_internal.h"
#include "tables.h"
#include "wave.h"

namespace mb {
namespace {

struct PlanArgs {
  int N, K, E, P, R, cap, Eh, NS, nblk;
  int32_t tau[kMaxRanks];  // target of each rank (all T with equal speeds)
  int tau_max;
  // drift-gated replanning: state buffer (nullptr: run the greedy every call)
  uint8_t* drift_state;
  int delta_num, delta_den, window, check_every;
  int tol_num, tol_den;       // load guard on a replayed placement
  int repair;                 // quota repair after placement
  const int32_t* counts;      // [P][E] pairs per (source rank, expert), from k_scan
  int32_t* counts_out;        // the same buffer, cleared when the routing is invalid
  const int32_t* expert_total;
  const int32_t* blockcnt;    // small table of block counts [nblk][E] (k_scan skipped)
  int nbps;                   // routing blocks per source rank
  const int32_t* blockflags;
  int32_t* load_pre;
  int32_t* load_post;
  int32_t* rep_expert;
  int32_t* slot_quota;
  int32_t* cu_seqlens;
  int32_t* status;
  // k_assign's lookup tables, built here when non-null (few experts)
  PairEntry* pair_tab;
  HostEntry* host_list;
  int2* host_range;
};

constexpr int kPlanThreads = 256;

typedef unsigned __int128 u128;

struct PlanSmem {
  u128* red;        // [64*3] per-lane partial sums of the drift check
  uint64_t* hold;   // [E] ranks holding a replica of expert e
  double* dmisc;    // [2] distance of this call's check
  int32_t* c;       // [E] routed pairs per expert
  int32_t* qh;      // [E] remaining home quota
  int32_t* repE;    // [P*R] expert of replica slot, -1 empty
  int32_t* repM;    // [P*R] quota of replica slot
  int32_t* order;   // [P*R] replica slots in placement order
  int32_t* dRep;    // [P*R] own pairs of the slot's rank for its expert (repair)
  int32_t* dHome;   // [P*R] own pairs of the slot expert's home rank (repair)
  int32_t* homeOf;  // [P*R] home rank of the slot's expert (repair)
  int32_t* xab;     // [P*R] this round's flows of each slot's entry (repair)
  int32_t* xba;
  int32_t* loadv;   // [64] load after planning
  int32_t* lpre;    // [64] load before planning
  int32_t* tau;     // [64] target of each rank
  int32_t* misc;    // [8] moves, unbalanced, guard replan, largest target,
                    //     replan, checked, next countdown, window size
};

__host__ __device__ inline size_t plan_smem_bytes(int E, int P, int R, int NS) {
  return sizeof(u128) * 64 * 3 + sizeof(uint64_t) * (size_t)E + 2 * sizeof(double) +
         sizeof(int32_t) * (2 * (size_t)E + 8 * (size_t)P * R + 64 + 64 + 64 + 8);
}

__device__ inline PlanSmem carve(uint8_t* base, int E, int P, int R, int NS) {
  PlanSmem m;
  m.red = reinterpret_cast<u128*>(base);
  m.hold = reinterpret_cast<uint64_t*>(base + sizeof(u128) * 64 * 3);
  m.dmisc = reinterpret_cast<double*>(m.hold + E);
  int32_t* p = reinterpret_cast<int32_t*>(m.dmisc + 2);
  m.c = p;
  p += E;
  m.qh = p;
  p += E;
  m.repE = p;
  p += P * R;
  m.repM = p;
  p += P * R;
  m.order = p;
  p += P * R;
  m.dRep = p;
  p += P * R;
  m.dHome = p;
  p += P * R;
  m.homeOf = p;
  p += P * R;
  m.xab = p;
  p += P * R;
  m.xba = p;
  p += P * R;
  m.loadv = p;
  p += 64;
  m.lpre = p;
  p += 64;
  m.tau = p;
  p += 64;
  m.misc = p;
  return m;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Greedy placement, run by the 64 lanes of wave 0 (lane = rank).
//
// Each lane works on x = load - tau, its rank's distance above (x > 0) or
// below (x < 0) its target. A move gives its destination min(-x, remaining
// home quota) pairs, so a rank that receives a replica of an expert either
// ends at its target or exhausts that expert's home quota, and a rank at or
// below its target never sheds. Hence, for an expert with home quota left,
// every holder other than its home is at its target: no open rank (x < 0,
// slot free) holds it, and the destination of a move is the open rank with
// the smallest x whatever expert the busiest rank gives. A step is then two
// independent wave reductions over x (largest; smallest among open ranks)
// plus a read of the busiest rank's heaviest expert, which each rank lane
// keeps up to date in registers.
//
// EHM >= Eh: registers per lane for the home quotas of its rank; kLanes =
// 32 when P <= 32 (shorter reductions), else 64; kOneSlot: R == 1.
//
// Packed keys make every choice one max or min: a rank lane enters the
// busiest-rank reduction with x*64 + (63 - lane) and, when open, the
// open-rank reduction with x*64 + lane, and keeps its home quotas as
// q*32 + (31 - j), so the extreme key also names the lowest rank or expert
// index among equal values. The keys are exact while |x| and q stay below
// 2^25, which N*K < 2^25 guarantees (loads, targets and quotas are at most
// N*K); larger plans take greedy_lds.
//
// A single wave issues about one instruction per SIMD turn, so the move is
// written for few instructions. Both reduction results are keys, which give
// the two lanes' x back (x*64 = key with the low six bits cleared): the move
// writes the donor's and the destination's new x, slot count and quota key
// into those lanes alone (v_writelane), and is recorded the same way: in
// the destination's lane with one slot per rank, else in lane (move mod
// 64). With at most 8 home experts a lane keeps its keys in descending
// order, so its heaviest is the first register and the donor's lowered key
// sinks back into place in one compare-exchange pass (lanes other than the
// donor are already in order); with more, the heaviest is a max over the
// registers and the lowered key is written at the uniform expert index.
constexpr long long kPackedPairsLimit = 1LL << 25;

// Descending order of n registers: k[from] sinks past its smaller
// neighbours (compare-exchange; indices fixed at compile time, so the array
// stays in registers).
template <int n, int from>
__device__ __forceinline__ void sink_pass(int (&k)[n]) {
  if constexpr (from + 1 < n) {
    const int hi = max(k[from], k[from + 1]), lo = min(k[from], k[from + 1]);
    k[from] = hi;
    k[from + 1] = lo;
    sink_pass<n, from + 1>(k);
  }
}

// Insertion sort, descending: elements i, i-1, ..., 0 sink in turn.
template <int n, int i>
__device__ __forceinline__ void sort_desc(int (&k)[n]) {
  if constexpr (i >= 0) {
    sink_pass<n, i>(k);
    sort_desc<n, i - 1>(k);
  }
}

template <int EHM, int kLanes, bool kOneSlot>
__device__ __forceinline__ void greedy_regs(const PlanArgs& a, PlanSmem& m) {
  static_assert(EHM <= 32, "five index bits per quota key");
  constexpr bool kSorted = EHM <= 8;
  const int lane = threadIdx.x;
  const int P = a.P, R = a.R, Eh = a.Eh;
  const bool rank_lane = lane < P;
  const int tau = rank_lane ? m.tau[lane] : 0;
  int kq[EHM];  // quota keys; -1 pads ranks with fewer home experts
  int load = 0;
#pragma unroll
  for (int j = 0; j < EHM; ++j) {
    const bool real = rank_lane && j < Eh;
    const int q = real ? m.c[lane * Eh + j] : 0;
    load += q;
    kq[j] = real ? q * 32 + (31 - j) : -1;
  }
  if constexpr (kSorted) sort_desc<EHM, EHM - 2>(kq);
  const int lpre = load;
  // The lane keeps x*64 itself, so both reduction keys are one add away.
  // A lane without a rank sits far below every key (never the busiest)
  // with no free slot (never open).
  int kx = rank_lane ? (load - tau) * 64 : -(1 << 30);
  const int c63 = 63 - lane;
  // Free slots: with one slot per rank a mask that the open key passes
  // through (all ones while the slot is free), else the slot count.
  int om = rank_lane ? -1 : 0x7fffffff;
  int used = rank_lane ? 0 : R;
  auto open_key = [&]() -> int {
    const int kn = kx + lane;  // x*64 + lane: negative exactly when x < 0
    if constexpr (kOneSlot) return (int)max((unsigned)(kn & om), 0x7fffffffu);
    return used < R && kn < 0 ? kn : INT32_MAX;
  };
  auto heaviest = [&]() -> int {
    if constexpr (kSorted) return kq[0];
    int bk = kq[0];
#pragma unroll
    for (int j = 1; j + 1 < EHM; j += 2) bk = max(bk, max(kq[j], kq[j + 1]));
    return max(bk, kq[EHM - 1]);
  };
  int moves = 0;
  int rec_e = 0, rec_m = 0, rec_i = kOneSlot ? -1 : 0;  // the moves recorded in this lane
  int kmax, kmin;
  wave_max_min_i32<kLanes>(kx + c63, open_key(), kmax, kmin);
  int bk = heaviest();
  // Go on while the largest x is positive (kmax >= 64) and a rank is open
  // (kmin < 0; INT32_MAX when none is).
  while (((63 - kmax) & kmin) < 0) {
    const int rs = 63 - (kmax & 63);
    const int d = kmin & 63;
    const int kd = __builtin_amdgcn_readlane(bk, rs);
    const int slot = kOneSlot ? 0 : __builtin_amdgcn_readlane(used, d);  // slots fill in order
    const int mv = min(-(kmin >> 6), kd >> 5);
    const int jb = 31 - (kd & 31);
    if constexpr (kOneSlot) {
      // one replica per rank: the record sits in the destination's lane,
      // rec_i holding the move's place in the placement order
      rec_e = writelane_i32(rs * Eh + jb, d, rec_e);
      rec_m = writelane_i32(mv, d, rec_m);
      rec_i = writelane_i32(moves, d, rec_i);
    } else {
      const int mi = moves & 63;
      rec_e = writelane_i32(rs * Eh + jb, mi, rec_e);
      rec_m = writelane_i32(mv, mi, rec_m);
      rec_i = writelane_i32(d * R + slot, mi, rec_i);
    }
    kx = writelane_i32((kmin & ~63) + mv * 64, d, kx);
    kx = writelane_i32((kmax & ~63) - mv * 64, rs, kx);
    if constexpr (kOneSlot)
      om = writelane_i32(0x7fffffff, d, om);
    else
      used = writelane_i32(slot + 1, d, used);
    if constexpr (kSorted) {
      kq[0] = writelane_i32(kd - mv * 32, rs, kq[0]);
      sink_pass<EHM, 0>(kq);
    } else {
      kq[jb] = writelane_i32(kd - mv * 32, rs, kq[jb]);  // uniform index: relative addressing
    }
    ++moves;
    if (!kOneSlot && (moves & 63) == 0) {
      m.repE[rec_i] = rec_e;
      m.repM[rec_i] = rec_m;
      m.order[moves - 64 + lane] = rec_i;
    }
    wave_max_min_i32<kLanes>(kx + c63, open_key(), kmax, kmin);
    bk = heaviest();
  }
  const int unbalanced = kmax >= 64;  // a rank above target and none open
  load = rank_lane ? (kx >> 6) + tau : 0;
  if constexpr (kOneSlot) {
    if (rec_i >= 0) {  // this rank received move rec_i into its one slot
      m.repE[lane] = rec_e;
      m.repM[lane] = rec_m;
      m.order[rec_i] = lane;
    }
  } else {
    const int done = moves & ~63;
    if (lane < moves - done) {
      m.repE[rec_i] = rec_e;
      m.repM[rec_i] = rec_m;
      m.order[done + lane] = rec_i;
    }
  }
  if (rank_lane) {
#pragma unroll
    for (int j = 0; j < EHM; ++j) {
      if constexpr (kSorted) {
        if (kq[j] >= 0) m.qh[lane * Eh + (31 - (kq[j] & 31))] = kq[j] >> 5;
      } else {
        if (j < Eh) m.qh[lane * Eh + j] = kq[j] >> 5;
      }
    }
    m.loadv[lane] = load;
    m.lpre[lane] = lpre;
  }
  if (lane == 0) {
    m.misc[0] = moves;
    m.misc[1] = unbalanced;
  }
}

template <int kLanes, bool kOneSlot>
__device__ __forceinline__ void greedy_regs_for(const PlanArgs& a, PlanSmem& m) {
  if (a.Eh <= 4)
    greedy_regs<4, kLanes, kOneSlot>(a, m);
  else if (a.Eh <= 8)
    greedy_regs<8, kLanes, kOneSlot>(a, m);
  else if (a.Eh <= 16)
    greedy_regs<16, kLanes, kOneSlot>(a, m);
  else if (a.Eh <= 24)
    greedy_regs<24, kLanes, kOneSlot>(a, m);
  else
    greedy_regs<32, kLanes, kOneSlot>(a, m);
}

template <int kLanes>
__device__ __forceinline__ void greedy_regs_lanes(const PlanArgs& a, PlanSmem& m) {
  if (a.R == 1)
    greedy_regs_for<kLanes, true>(a, m);
  else
    greedy_regs_for<kLanes, false>(a, m);
}

// The same greedy for ranks with more home experts than fit in registers:
// home quotas stay in LDS and the heaviest expert of the busiest rank is a
// wave reduction per step.
__device__ __forceinline__ void greedy_lds(const PlanArgs& a, PlanSmem& m) {
  const int lane = threadIdx.x;
  const int P = a.P, R = a.R, Eh = a.Eh;
  const bool rank_lane = lane < P;
  const int tau = rank_lane ? m.tau[lane] : 0;
  int load = 0;
  if (rank_lane)
    for (int i = 0; i < Eh; ++i) load += m.c[lane * Eh + i];
  const int lpre = load;
  int used = 0, moves = 0, unbalanced = 0;
  for (;;) {
    const int x = load - tau;
    const bool open_lane = rank_lane && used < R && x < 0;
    const int xmax = wave_max_i32(rank_lane ? x : INT32_MIN);
    const int xmin = wave_min_i32(open_lane ? x : INT32_MAX);
    if (xmax <= 0) break;
    if (xmin == INT32_MAX) {
      unbalanced = 1;
      break;
    }
    const int rs = lowest_lane(ballot64(rank_lane && x == xmax));
    const int d = lowest_lane(ballot64(open_lane && x == xmin));
    int myq = 0, myj = INT32_MAX;
    for (int j = lane; j < Eh; j += 64) {
      const int qq = m.qh[rs * Eh + j];
      if (qq > myq) {
        myq = qq;
        myj = j;
      }
    }
    const int qmax = wave_max_i32(myq);
    const int jb = wave_min_i32(myq == qmax ? myj : INT32_MAX);
    const int e = rs * Eh + jb;
    const int slot = __builtin_amdgcn_readlane(used, d);
    const int mv = min(-xmin, qmax);
    if (lane == 0) {
      m.qh[e] = qmax - mv;
      m.repE[d * R + slot] = e;
      m.repM[d * R + slot] = mv;
      m.order[moves] = d * R + slot;
    }
    if (lane == rs) load -= mv;
    if (lane == d) {
      load += mv;
      used += 1;
    }
    ++moves;
    wave_lds_sync();
  }
  if (rank_lane) {
    m.loadv[lane] = load;
    m.lpre[lane] = lpre;
  }
  if (lane == 0) {
    m.misc[0] = moves;
    m.misc[1] = unbalanced;
  }
}

static_assert(sizeof(mb_drift_header) == 64, "drift header layout");

struct DriftView {
  mb_drift_header* hdr;
  int64_t* wsum;   // [E] reference sum
  int32_t* rep;    // [P*R] kept replica experts
  int32_t* order;  // [P*R] kept slots in placement order
};

__device__ inline DriftView drift_view(const PlanArgs& a) {
  DriftView v;
  v.hdr = reinterpret_cast<mb_drift_header*>(a.drift_state);
  v.wsum = reinterpret_cast<int64_t*>(a.drift_state + sizeof(mb_drift_header));
  v.rep = reinterpret_cast<int32_t*>(v.wsum + a.E);
  v.order = v.rep + a.P * a.R;
  return v;
}

// d = 1 - c.r / (|c| |r|) from exact integer sums (ViBE summary, Drift-Aware
// Recalibration); the window's sum r has the direction of its mean.
__device__ __forceinline__ double cosine_distance(u128 dot, u128 n1, u128 n2) {
#pragma clang fp contract(off)
  if (n1 == 0 || n2 == 0) return n1 == n2 ? 0.0 : 1.0;
  return 1.0 - (double)dot / (__builtin_sqrt((double)n1) * __builtin_sqrt((double)n2));
}

// Wave 0: whether this call runs the greedy. The first call does; after
// that a check every check_every calls compares the counts with the
// reference and replans when d exceeds delta_num / delta_den.
__device__ __forceinline__ void drift_decide(const PlanArgs& a, PlanSmem& m) {
  const int lane = threadIdx.x;
  const DriftView v = drift_view(a);
  const int have = v.hdr->have_plan;
  int countdown = v.hdr->countdown;
  const int nwin = v.hdr->nwin;
  double d = v.hdr->last_d;
  int replan = !have, checked = 0;
  if (!replan && --countdown == 0) {
    countdown = a.check_every;
    checked = 1;
    u128 dot = 0, n1 = 0, n2 = 0;
    for (int e = lane; e < a.E; e += 64) {
      const uint64_t c = (uint32_t)m.c[e], w = (uint64_t)v.wsum[e];
      dot += (u128)c * w;
      n1 += (u128)c * c;
      n2 += (u128)w * w;
    }
    m.red[lane] = dot;
    m.red[64 + lane] = n1;
    m.red[128 + lane] = n2;
    wave_lds_sync();
    for (int w = 32; w >= 1; w >>= 1) {  // pairwise tree over the lanes
      if (lane < w) {
        m.red[lane] += m.red[lane + w];
        m.red[64 + lane] += m.red[64 + lane + w];
        m.red[128 + lane] += m.red[128 + lane + w];
      }
      wave_lds_sync();
    }
    if (lane == 0) m.dmisc[0] = cosine_distance(m.red[0], m.red[64], m.red[128]);
    wave_lds_sync();
    d = m.dmisc[0];
    replan = d > (double)a.delta_num / (double)a.delta_den;
  }
  if (replan) countdown = a.check_every;
  if (lane == 0) {
    m.misc[4] = replan;
    m.misc[5] = checked;
    m.misc[6] = countdown;
    m.misc[7] = nwin;
    m.dmisc[0] = d;
  }
  wave_lds_sync();
}

// Wave 0, no replan: the kept replicas, in the order they were placed, each
// take min(target - host load, remaining home quota) pairs while the
// expert's home rank is above its target and the host below its own. Loads
// stay in lane registers (lane = rank); a chunk of up to 64 moves is read
// one move per lane, each lane also holding its move's expert's remaining
// home quota, then stepped through in order (a move lowers the quota on
// every lane of the same expert).
__device__ __forceinline__ void replay_kept(const PlanArgs& a, PlanSmem& m) {
  const int lane = threadIdx.x;
  const int P = a.P, R = a.R, Eh = a.Eh;
  const DriftView v = drift_view(a);
  // (a state written by this kernel for the same sizes always passes these
  // range checks; they only keep a foreign buffer inside the arrays)
  const int n_moves = min(max(v.hdr->n_moves, 0), P * R);
  for (int i = lane; i < P * R; i += 64) {
    const int e = v.rep[i];
    m.repE[i] = (unsigned)e < (unsigned)a.E ? e : -1;
    m.order[i] = v.order[i];
  }
  const bool rank_lane = lane < P;
  const int tau = rank_lane ? m.tau[lane] : 0;
  int load = 0;
  if (rank_lane)
    for (int i = 0; i < Eh; ++i) load += m.c[lane * Eh + i];
  const int lpre = load;
  // x = load - tau per rank lane: a move needs its home above target
  // (x_h > 0) and its host below (x_d < 0), and gives min(-x_d, quota).
  int x = load - tau;
  wave_lds_sync();
  for (int base = 0; base < n_moves; base += 64) {
    const int i = base + lane;
    int slot = 0, e = 0, dst = -1, h = 0;  // dst < 0: no move in this lane
    if (i < n_moves) {
      slot = m.order[i];
      const bool ok_slot = (unsigned)slot < (unsigned)(P * R);
      e = ok_slot ? m.repE[slot] : -1;
      if (ok_slot && (unsigned)e < (unsigned)a.E) {
        dst = slot / R;
        h = e / Eh;
      } else {
        e = 0;
      }
    }
    const bool ok = dst >= 0;
    int q = ok ? m.qh[e] : 0;  // remaining home quota of this lane's expert
    int mine = 0;
    const int cnt = min(64, n_moves - base);
    for (int j = 0; j < cnt; ++j) {
      const int sd = __builtin_amdgcn_readlane(dst, j);
      const int sh = __builtin_amdgcn_readlane(h, j);
      const int se = __builtin_amdgcn_readlane(e, j);
      const int qe = __builtin_amdgcn_readlane(q, j);
      const int xd = __builtin_amdgcn_readlane(x, sd & 63);
      const int xh = __builtin_amdgcn_readlane(x, sh);
      // no move unless the home is above target and the host below (q is
      // 0 in lanes without a move)
      const int mv = min(min(max(-xd, 0), qe), xh > 0 ? INT32_MAX : 0);
      mine = writelane_i32(mv, j, mine);
      q -= (ok && e == se) ? mv : 0;
      // the two changed lanes written alone (a host is never its expert's
      // home; were it, the second write restores the lane)
      x = writelane_i32(xh - mv, sh, x);
      x = writelane_i32((sd & 63) == sh ? xd : xd + mv, sd & 63, x);
    }
    if (ok) {
      m.repM[slot] = mine;
      m.qh[e] = q;  // lanes of one expert hold the same final quota
    }
    wave_lds_sync();
  }
  load = x + tau;
  const int unbalanced = ballot64(rank_lane && load > tau) != 0;
  if (rank_lane) {
    m.loadv[lane] = load;
    m.lpre[lane] = lpre;
  }
  if (lane == 0) {
    m.misc[0] = n_moves;
    m.misc[1] = unbalanced;
  }
}

// Wave 0, after replay_kept: the load guard (ViBE, Incremental placement
// update: a placement is done once every GPU is within the tolerance epsilon
// of the balanced time, i.e. load_r <= (1 + epsilon) tau_r when time is load
// over speed). The replay stands when no rank needs more than cap rows and,
// with tol_den > 0, load * tol_den <= tau * (tol_den + tol_num) on every rank
// (exact in 64-bit integers). Otherwise the placement state is reset for
// the greedy, which then runs in this call as on a replan. Returns whether
// it must run.
__device__ __forceinline__ bool guard_rejects(const PlanArgs& a, PlanSmem& m) {
  const int lane = threadIdx.x;
  bool over = false;
  if (lane < a.P) {
    const long long load = m.loadv[lane], tau = m.tau[lane];
    over = load > a.cap ||
           (a.tol_den > 0 && load * a.tol_den > tau * ((long long)a.tol_den + a.tol_num));
  }
  if (ballot64(over) == 0) return false;
  for (int e = lane; e < a.E; e += 64) m.qh[e] = m.c[e];
  for (int i = lane; i < a.P * a.R; i += 64) {
    m.repE[i] = -1;
    m.repM[i] = 0;
  }
  if (lane == 0) {
    m.misc[2] = 1;
    m.misc[4] = 1;
    m.misc[6] = a.check_every;
  }
  wave_lds_sync();
  return true;
}

// Wave 0, after the placement: ISER-MoE HALO-Q stage 4, quota repair. A
// circle-method tournament (n = P rounded up to even players, n - 1 rounds;
// player 0 stays at position 0, the others rotate one position per round;
// positions k and n-1-k meet) pairs ranks disjointly. For a pair a < b and
// each expert both hold, taken in ascending replica-slot order (a's slots
// whose expert b also holds, then b's slots whose expert is homed on a),
// x_ab = min((d_a - Q_a)^+, (Q_b - d_b)^+) of a's own pairs could come back to
// a, and x_ba likewise; m = min(sum x_ab, sum x_ba) units of quota move
// b -> a over the x_ab experts and a -> b over the x_ba experts, each expert
// taking min(x, what is left of m) in that order. Loads and expert totals do
// not change. Each replica slot is an entry handled by one lane: in every
// round it finds its holder's partner, whether its expert is one the pair
// holds in common, and its two quota cells; the entries of a pair read each
// other's x from LDS for the pair's totals and running sums. Different
// entries have different cells, so the entries of a round act at once.
__device__ __forceinline__ void quota_repair(const PlanArgs& a, PlanSmem& m) {
  const int lane = threadIdx.x;
  const int P = a.P, R = a.R, Eh = a.Eh, E = a.E, PR = P * R;
  // Per slot: home of its expert, own demands of its holder and of that
  // home; per expert: the ranks holding a replica.
  for (int e = lane; e < E; e += 64) m.hold[e] = 0;
  wave_lds_sync();
  for (int i = lane; i < PR; i += 64) {
    const int e = m.repE[i];
    const int h = e >= 0 ? e / Eh : -1;
    m.homeOf[i] = h;
    m.dRep[i] = e >= 0 ? a.counts[(size_t)(i / R) * E + e] : 0;
    m.dHome[i] = e >= 0 ? a.counts[(size_t)h * E + e] : 0;
    if (e >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&m.hold[e]), 1ull << (i / R));
  }
  wave_lds_sync();
  // A quota cell c >= 0 is home quota qh[c]; c < 0 is replica quota
  // repM[-1 - c]. (Indices, not pointers, keep the accesses in LDS.)
  auto qget = [&](int c) { return c >= 0 ? m.qh[c] : m.repM[-1 - c]; };
  auto qadd = [&](int c, int v) {
    if (c >= 0)
      m.qh[c] += v;
    else
      m.repM[-1 - c] += v;
  };
  // Quotas change only where a pair cancels flows in both directions: if no
  // pair of ranks has a flow each way on the experts it shares under the
  // placement's quotas, no round changes anything. fwd[a] / back[a] mark the
  // ranks b > a with which rank a has a flow a -> b / b -> a.
  {
    uint64_t* fwd = reinterpret_cast<uint64_t*>(m.red);  // the drift sums are done
    uint64_t* back = fwd + 64;
    fwd[lane] = back[lane] = 0;
    wave_lds_sync();
    auto mark = [&](int ra, int rb, int xab, int xba) {
      if (xab > 0) atomicOr(reinterpret_cast<unsigned long long*>(&fwd[ra]), 1ull << rb);
      if (xba > 0) atomicOr(reinterpret_cast<unsigned long long*>(&back[ra]), 1ull << rb);
    };
    for (int i = lane; i < PR; i += 64) {
      const int e = m.repE[i];
      if (e < 0) continue;
      const int r = i / R, h = m.homeOf[i];
      const int Qr = m.repM[i], Qh = m.qh[e], dr = m.dRep[i], dh = m.dHome[i];
      const int xr = min(max(dr - Qr, 0), max(Qh - dh, 0));  // holder's pairs home could take
      const int xh = min(max(dh - Qh, 0), max(Qr - dr, 0));  // home's pairs the holder could take
      if (r < h)
        mark(r, h, xr, xh);
      else
        mark(h, r, xh, xr);
      // pairs of holders of the same expert (r below the other holder)
      for (uint64_t o = m.hold[e] & ~((2ull << r) - 1); o; o &= o - 1) {
        const int q = __builtin_ctzll(o);
        for (int j = 0; j < R; ++j)
          if (m.repE[q * R + j] == e) {
            const int Qq = m.repM[q * R + j], dq = m.dRep[q * R + j];
            mark(r, q, min(max(dr - Qr, 0), max(Qq - dq, 0)),
                 min(max(dq - Qq, 0), max(Qr - dr, 0)));
          }
      }
    }
    wave_lds_sync();
    if (ballot64((fwd[lane] & back[lane]) != 0) == 0) return;
  }
  const int n = P + (P & 1);
  // Entry of slot i in a round: cells of ranks a < b, their own demands, the pair.
  auto entry = [&](int i, int round, int& ca, int& cb, int& da, int& db, int& lo,
                   int& hi) -> bool {
    const int e = m.repE[i];
    if (e < 0) return false;
    const int r = i / R, h = m.homeOf[i];
    // position of r this round, then the player at the opposite position
    int pos = 0;
    if (r > 0) {
      pos = r - 1 - round;
      pos += pos < 0 ? n - 1 : 0;
      pos += 1;
    }
    const int ppos = n - 1 - pos;
    int q = 0;
    if (ppos > 0) {
      q = ppos - 1 + round;
      q -= q >= n - 1 ? n - 1 : 0;
      q += 1;
    }
    if (q >= P) return false;  // bye
    if (h == q) {              // the partner is e's home
      if (r < q) {
        ca = -1 - i, cb = e, da = m.dRep[i], db = m.dHome[i], lo = r, hi = q;
      } else {
        ca = e, cb = -1 - i, da = m.dHome[i], db = m.dRep[i], lo = q, hi = r;
      }
      return true;
    }
    if (r < q && ((m.hold[e] >> q) & 1))  // the partner holds e in a slot
      for (int j = 0; j < R; ++j)
        if (m.repE[q * R + j] == e) {
          ca = -1 - i, cb = -1 - (q * R + j), da = m.dRep[i], db = m.dRep[q * R + j];
          lo = r, hi = q;
          return true;
        }
    return false;
  };
  if (PR <= 64) {
    // One slot per lane: everything but the quotas stays in registers.
    const int i = lane;
    const int e = i < PR ? m.repE[i] : -1;
    const int r = i < PR ? i / R : 0, h = i < PR ? m.homeOf[i] : -1;
    const int dr = i < PR ? m.dRep[i] : 0, dh = i < PR ? m.dHome[i] : 0;
    const uint64_t hold = e >= 0 ? m.hold[e] : 0;
    for (int round = 0; round + 1 < n; ++round) {
      int ca = 0, cb = 0, da = 0, db = 0, lo = 0, hi = 0;
      bool on = false;
      if (e >= 0) {
        int pos = 0;
        if (r > 0) {
          pos = r - 1 - round;
          pos += pos < 0 ? n - 1 : 0;
          pos += 1;
        }
        const int ppos = n - 1 - pos;
        int q = 0;
        if (ppos > 0) {
          q = ppos - 1 + round;
          q -= q >= n - 1 ? n - 1 : 0;
          q += 1;
        }
        if (q < P && h == q) {
          on = true;
          if (r < q) {
            ca = -1 - i, cb = e, da = dr, db = dh, lo = r, hi = q;
          } else {
            ca = e, cb = -1 - i, da = dh, db = dr, lo = q, hi = r;
          }
        } else if (q < P && r < q && ((hold >> q) & 1)) {
          for (int j = 0; j < R; ++j)
            if (m.repE[q * R + j] == e) {
              on = true;
              ca = -1 - i, cb = -1 - (q * R + j), da = dr, db = m.dRep[q * R + j];
              lo = r, hi = q;
            }
        }
      }
      if (ballot64(on) == 0) continue;  // no pair of this round holds an expert in common
      int xab = 0, xba = 0;
      if (on) {
        const int Qa = qget(ca), Qb = qget(cb);
        xab = min(max(da - Qa, 0), max(Qb - db, 0));
        xba = min(max(db - Qb, 0), max(Qa - da, 0));
      }
      if (i < PR) {
        m.xab[i] = xab;
        m.xba[i] = xba;
      }
      if (ballot64(xab != 0 || xba != 0) == 0) continue;  // no flow to cancel
      wave_lds_sync();
      if (xab != 0 || xba != 0) {
        int fab = 0, fba = 0, pab = 0, pba = 0;  // pair totals; sums before this slot
        for (int s2 = 0; s2 < 2 * R; ++s2) {
          const int j = s2 < R ? lo * R + s2 : hi * R + (s2 - R);
          const int x1 = m.xab[j], x2 = m.xba[j];
          fab += x1;
          fba += x2;
          pab += j < i ? x1 : 0;
          pba += j < i ? x2 : 0;
        }
        const int mm = min(fab, fba);
        const int t = min(xab, max(mm - pab, 0)) - min(xba, max(mm - pba, 0));
        qadd(ca, t);
        qadd(cb, -t);
      }
      wave_lds_sync();
    }
    return;
  }
  for (int round = 0; round + 1 < n; ++round) {
    int any = 0;
    for (int i = lane; i < PR; i += 64) {
      int ca, cb, da, db, lo, hi, xab = 0, xba = 0;
      if (entry(i, round, ca, cb, da, db, lo, hi)) {
        const int Qa = qget(ca), Qb = qget(cb);
        xab = min(max(da - Qa, 0), max(Qb - db, 0));
        xba = min(max(db - Qb, 0), max(Qa - da, 0));
        any |= (xab | xba) != 0;
      }
      m.xab[i] = xab;
      m.xba[i] = xba;
    }
    if (ballot64(any) == 0) continue;  // no flow to cancel this round
    wave_lds_sync();
    for (int i = lane; i < PR; i += 64) {
      const int xab = m.xab[i], xba = m.xba[i];
      int ca, cb, da, db, lo, hi;
      if ((xab == 0 && xba == 0) || !entry(i, round, ca, cb, da, db, lo, hi)) continue;
      int fab = 0, fba = 0, pab = 0, pba = 0;  // pair totals; sums before this slot
      for (int s2 = 0; s2 < 2 * R; ++s2) {
        const int j = s2 < R ? lo * R + s2 : hi * R + (s2 - R);
        const int x1 = m.xab[j], x2 = m.xba[j];
        fab += x1;
        fba += x2;
        pab += j < i ? x1 : 0;
        pba += j < i ? x2 : 0;
      }
      const int mm = min(fab, fba);
      const int t = min(xab, max(mm - pab, 0)) - min(xba, max(mm - pba, 0));
      qadd(ca, t);
      qadd(cb, -t);
    }
    wave_lds_sync();
  }
}

// All threads, after the placement: the state for the layer's next call.
__device__ __forceinline__ void drift_update(const PlanArgs& a, PlanSmem& m) {
  const int tid = threadIdx.x;
  const DriftView v = drift_view(a);
  const int replan = m.misc[4], moves = m.misc[0], nwin = m.misc[7];
  const int PR = a.P * a.R;
  if (replan) {
    for (int e = tid; e < a.E; e += kPlanThreads) v.wsum[e] = m.c[e];
    for (int i = tid; i < PR; i += kPlanThreads) {
      v.rep[i] = m.repE[i];
      v.order[i] = i < moves ? m.order[i] : -1;
    }
  } else if (nwin < a.window) {
    for (int e = tid; e < a.E; e += kPlanThreads) v.wsum[e] += m.c[e];
  }
  if (tid == 0) {
    mb_drift_header h = *v.hdr;
    h.have_plan = 1;
    h.countdown = m.misc[6];
    h.nwin = replan ? 1 : min(nwin + 1, a.window);
    if (replan) h.n_moves = moves;
    h.calls += 1;
    h.replans += replan;
    h.guarded += m.misc[2];
    h.last_d = m.dmisc[0];
    *v.hdr = h;
  }
}

__global__ __launch_bounds__(kPlanThreads) void k_plan(PlanArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int E = a.E, P = a.P, R = a.R, Eh = a.Eh, NS = a.NS;
  PlanSmem m = carve(smem, E, P, R, NS);

  // The targets, the status bits of the routing decisions and c_e (summed
  // over sources by k_scan, or here when k_scan did not run: from d[s][e],
  // or from the block counts) are loaded before any of them is used, so
  // their latencies overlap.
  static_assert(kMaxExperts <= 4 * kPlanThreads, "c_e takes one batch of loads");
  const int tau_v = a.tau[tid & (kMaxRanks - 1)];
  int f[4], cv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = u * kPlanThreads + tid;
    f[u] = i < a.nblk ? a.blockflags[i] : 0;
  }
  if (a.expert_total) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = u * kPlanThreads + tid;
      cv[u] = e < E ? a.expert_total[e] : 0;
    }
  }
  int fl = f[0] | f[1] | f[2] | f[3];
  for (int i = 4 * kPlanThreads + tid; i < a.nblk; i += kPlanThreads) fl |= a.blockflags[i];
  if (a.expert_total) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = u * kPlanThreads + tid;
      if (e < E) m.c[e] = m.qh[e] = cv[u];
    }
  } else if (a.blockcnt) {
    // A small table of block counts: d[s][e] is the sum of the source's
    // blocks (a plan output, here in place of k_scan's), c_e their sum over
    // sources, accumulated in LDS.
    for (int e = tid; e < E; e += kPlanThreads) m.c[e] = 0;
    __syncthreads();
    for (int i = tid; i < P * E; i += kPlanThreads) {
      const int s = i / E, e = i - s * E;
      const int32_t* col = a.blockcnt + (size_t)s * a.nbps * E + e;
      int d = 0;
      for (int j = 0; j < a.nbps; ++j) d += col[(size_t)j * E];
      a.counts_out[i] = d;
      atomicAdd(&m.c[e], d);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPlanThreads) m.qh[e] = m.c[e];
  } else {
    // Every source's count of the thread's expert in flight at once; the
    // address advances in a vector register (kept there by the empty asm),
    // so the row offsets are not all held in scalar registers.
    for (int e = tid; e < E; e += kPlanThreads) {
      const int32_t* col = a.counts + e;
      int v[kMaxRanks];
#pragma unroll
      for (int q = 0; q < kMaxRanks; ++q) {
        v[q] = q < P ? *col : 0;
        col += E;
        __asm__ volatile("" : "+v"(col));
      }
      int c = 0;
#pragma unroll
      for (int q = 0; q < kMaxRanks; ++q) c += v[q];
      m.c[e] = m.qh[e] = c;
    }
  }
  if (tid < 64) m.tau[tid] = tid < P ? tau_v : 0;
  if (tid == 0) {
    m.misc[2] = 0;
    m.misc[3] = a.tau_max;
  }
  for (int i = tid; i < P * R; i += kPlanThreads) {
    m.repE[i] = -1;
    m.repM[i] = 0;
  }
  if (__syncthreads_or(fl)) {
    // Routing decisions that name no expert or one twice define no plan:
    // every count, load and quota is 0, every replica slot empty, and
    // cu_seqlens all 0 (pos and row_src are left unspecified).
    const int bad = __syncthreads_or(fl & MB_ST_BAD_ID);
    const int dup = __syncthreads_or(fl & MB_ST_DUP_ID);
    for (int i = tid; i < P * E; i += kPlanThreads) a.counts_out[i] = 0;
    for (int r = tid; r < P; r += kPlanThreads) a.load_pre[r] = a.load_post[r] = 0;
    for (int i = tid; i < P * R; i += kPlanThreads) a.rep_expert[i] = -1;
    for (int i = tid; i < P * NS; i += kPlanThreads) a.slot_quota[i] = 0;
    for (int i = tid; i < P * (NS + 1); i += kPlanThreads) a.cu_seqlens[i] = 0;
    if (tid == 0) {
      a.status[0] = (bad ? MB_ST_BAD_ID : 0) | (dup ? MB_ST_DUP_ID : 0);
      a.status[1] = m.misc[3];
      a.status[2] = 0;
      a.status[3] = 0;
    }
    return;
  }

  const bool drift = a.drift_state != nullptr;
  if (tid < 64) {
    if (drift) drift_decide(a, m);
    bool greedy = true;
    if (drift && !m.misc[4]) {
      replay_kept(a, m);
      greedy = guard_rejects(a, m);
    }
    if (greedy) {
      if ((long long)a.N * a.K >= kPackedPairsLimit || Eh > 32)
        greedy_lds(a, m);
      else if (P <= 32)
        greedy_regs_lanes<32>(a, m);
      else
        greedy_regs_lanes<64>(a, m);
    }
    if (a.repair && R > 0) quota_repair(a, m);
  }
  __syncthreads();
  if (drift) {
    drift_update(a, m);
    __syncthreads();
  }

  // Slot quotas, cu_seqlens and loads: one thread per rank, or with many
  // slots per rank one wave per rank (lane = slot, a wave scan per 64).
  auto slot_q = [&](int r, int i) { return i < Eh ? m.qh[r * Eh + i] : m.repM[r * R + (i - Eh)]; };
  if (NS <= 16) {
    for (int r = tid; r < P; r += kPlanThreads) {
      int acc = 0;
      a.cu_seqlens[r * (NS + 1)] = 0;
      for (int i = 0; i < NS; ++i) {
        const int q = slot_q(r, i);
        a.slot_quota[r * NS + i] = q;
        acc += q;
        a.cu_seqlens[r * (NS + 1) + i + 1] = acc;
      }
    }
  } else {
    const int w = tid >> 6, ln = tid & 63;
    for (int r = w; r < P; r += kPlanThreads / 64) {
      int base = 0;
      if (ln == 0) a.cu_seqlens[r * (NS + 1)] = 0;
      for (int i0 = 0; i0 < NS; i0 += 64) {
        const int i = i0 + ln;
        const int q = i < NS ? slot_q(r, i) : 0;
        const int inc = wave_inclusive_sum(q);
        if (i < NS) {
          a.slot_quota[r * NS + i] = q;
          a.cu_seqlens[r * (NS + 1) + i + 1] = base + inc;
        }
        base += __builtin_amdgcn_readlane(inc, 63);
      }
    }
  }
  for (int r = tid; r < P; r += kPlanThreads) {
    a.load_pre[r] = m.lpre[r];
    a.load_post[r] = m.loadv[r];
  }
  for (int i = tid; i < P * R; i += kPlanThreads) a.rep_expert[i] = m.repE[i];
  int mymax = 0;
  for (int r = tid; r < P; r += kPlanThreads) mymax = max(mymax, m.loadv[r]);
  if (tid < 64) {
    const int max_load = wave_max_i32(mymax);
    if (tid == 0) {
      a.status[0] = (m.misc[1] ? MB_ST_UNBALANCED : 0) | (max_load > a.cap ? MB_ST_CAPACITY : 0) |
                    (drift && m.misc[4] ? MB_ST_REPLANNED : 0) |
                    (drift && m.misc[2] ? MB_ST_GUARDED : 0);
      a.status[1] = m.misc[3];
      a.status[2] = max_load;
      a.status[3] = m.misc[0];
    }
  }
  if (a.pair_tab) {
    // With few experts k_assign's lookup tables are built here, one wave
    // per expert in turn, from the plan outputs this workgroup has just
    // stored (nothing is needed under CAPACITY: k_assign then stores no row).
    const int ln = tid & 63;
    const int ml = wave_max_i32(ln < P ? m.loadv[ln] : 0);
    __syncthreads();
    if (ml <= a.cap)
      for (int e = tid >> 6; e < E; e += kPlanThreads / 64)
        tables_for_expert(e, E, P, R, Eh, NS, a.cap, a.counts, a.rep_expert, a.slot_quota,
                          a.cu_seqlens, a.pair_tab, a.host_list, a.host_range);
  }
}

}  // namespace

hipError_t launch_plan(const mb_dims& d, const Geometry& g, const mb_plan_bufs& o,
                       const int32_t* rank_speed, const mb_drift_params* drift,
                       void* drift_state, int repair, const int32_t* blockflags,
                       const int32_t* expert_total, const int32_t* blockcnt, PairEntry* pair_tab,
                       HostEntry* host_list, int2* host_range, hipStream_t st) {
  PlanArgs a;
  a.N = d.n_tokens;
  a.K = d.top_k;
  a.E = d.n_experts;
  a.P = d.n_ranks;
  a.R = d.slots_per_rank;
  a.cap = d.cap;
  a.Eh = g.Eh;
  a.NS = g.NS;
  a.nblk = g.nblk;
  // Targets (ViBE, token target in proportion to speed), exact in integers:
  // tau_r = ceil(N*K * s_r / sum s); equal speeds give T = ceil(N*K / P).
  long long sum = 0;
  for (int r = 0; r < d.n_ranks; ++r) sum += rank_speed[r];
  const long long nk = (long long)d.n_tokens * d.top_k;
  a.tau_max = 0;
  for (int r = 0; r < kMaxRanks; ++r) {
    a.tau[r] = r < d.n_ranks ? (int32_t)((nk * rank_speed[r] + sum - 1) / sum) : 0;
    a.tau_max = a.tau[r] > a.tau_max ? a.tau[r] : a.tau_max;
  }
  a.drift_state = static_cast<uint8_t*>(drift_state);
  a.delta_num = drift ? drift->delta_num : 0;
  a.delta_den = drift ? drift->delta_den : 1;
  a.window = drift ? drift->window : 1;
  a.check_every = drift ? drift->check_every : 1;
  a.tol_num = drift ? drift->tol_num : 0;
  a.tol_den = drift ? drift->tol_den : 0;
  a.repair = repair;
  a.counts = o.counts;
  a.counts_out = o.counts;
  a.expert_total = expert_total;
  a.blockcnt = blockcnt;
  a.nbps = g.nbps;
  a.blockflags = blockflags;
  a.load_pre = o.load_pre;
  a.load_post = o.load_post;
  a.rep_expert = o.rep_expert;
  a.slot_quota = o.slot_quota;
  a.cu_seqlens = o.cu_seqlens;
  a.status = o.status;
  a.pair_tab = pair_tab;
  a.host_list = host_list;
  a.host_range = host_range;
  const size_t shmem = plan_smem_bytes(a.E, a.P, a.R, a.NS);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), shmem, st, a);
  return hipGetLastError();
}

}  // namespace mb
