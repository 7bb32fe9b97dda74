// tables.h — the lookup tables k_assign reads, for one expert: the body of
// k_tables (route.hip), also run inside k_plan (plan.hip) when the experts
// are few.
//
// One wave per expert e, lane = source rank s: pass 1 keeps
// min(d[s][e], quota of s) pairs on each holder s; the remaining (surplus)
// pairs, in token order, fill the holders' spare quota in ascending rank
// order (ISER-MoE, HALO-Q stage 5; Zepp summary, eq. (1)). Prefix sums over
// s are wave scans. Every lane of the wave must be active; e is uniform.
#pragma once

#include "mb_internal.h"
#include "wave.h"

namespace mb {

__device__ __forceinline__ void tables_for_expert(
    int e, int E, int P, int R, int Eh, int NS, int cap, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ rep_expert, const int32_t* __restrict__ slot_quota,
    const int32_t* __restrict__ cu_seqlens, PairEntry* __restrict__ pair_tab,
    HostEntry* __restrict__ host_list, int2* __restrict__ host_range) {
  const int s = threadIdx.x & 63;
  const bool valid = s < P;
  const int home = e / Eh;
  int d = 0, slot = -1, lq = 0, rowbase = 0, reps_below = 0;
  if (valid) {
    d = counts[(size_t)s * E + e];
    for (int q = 0; q < R; ++q) {
      const int re = rep_expert[s * R + q];
      reps_below += (unsigned)re < (unsigned)e ? 1 : 0;
      if (s != home && re == e) slot = Eh + q;
    }
    if (s == home) slot = e - s * Eh;
    if (slot >= 0) {
      lq = slot_quota[s * NS + slot];
      rowbase = s * cap + cu_seqlens[s * (NS + 1) + slot];
    }
  }
  const int lt = min(d, lq);
  const int sur = d - lt, sp = lq - lt;
  const int sur_before = wave_inclusive_sum(sur) - sur;
  const int sp_before = wave_inclusive_sum(sp) - sp;
  if (valid) {
    PairEntry pe;
    pe.local_quota = lq;
    pe.local_base = slot >= 0 ? rowbase + min(max(sur_before - sp_before, 0), sp) : 0;
    pe.surplus_shift = sur_before - lq;
    pe.pad = 0;
    pair_tab[(size_t)s * E + e] = pe;
  }
  // The host list in expert order, 1 + (replicas of e) entries for e: its
  // entries start after those of the experts below it.
  const int off = e + __builtin_amdgcn_readlane(wave_inclusive_sum(reps_below), 63);
  const uint64_t hb = ballot64(valid && sp > 0);
  if (valid && sp > 0) {
    HostEntry h;
    h.end = sp_before + sp;
    h.base = rowbase - sp_before;
    h.rank = s;
    h.lt = lt;
    host_list[off + lanes_below(hb)] = h;
  }
  if (s == 0) host_range[e] = make_int2(off, __popcll(hb));
}

}  // namespace mb
