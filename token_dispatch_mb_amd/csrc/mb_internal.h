// mb_internal.h — declarations shared by libmoebal's own translation units:
// block geometry, workspace layout and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moebal.h"

namespace mb {

// Tokens handled by one routing workgroup: four wave64s, one token per lane.
constexpr int kTokensPerBlock = 256;
constexpr int kWaves = kTokensPerBlock / 64;

constexpr int kMaxRanks = 64;     // one wave lane per logical rank in k_plan
constexpr int kMaxExperts = 1024; // LDS: kWaves * E * 8 bytes of token masks
constexpr int kMaxTopK = 32;
constexpr int kMaxSlots = 16;
// Block-count tables k_plan and k_assign sum directly instead of running
// k_scan: at most this many routing blocks per source and block counts.
constexpr int kSmallTableBlocks = 4;
constexpr int kSmallTableCounts = 4096;
// Experts few enough for k_plan's four waves to build k_assign's lookup
// tables (one wave per expert, at most four in turn) instead of k_tables.
constexpr int kPlanTableExperts = 16;

// One entry per (source rank s, expert e), written by k_tables, read by
// k_assign for every pair (s, e):
//   local_quota   = quota of s for e (0 when s holds no copy of e)
//   local_base    = first row of s's local pairs of e, absolute in the
//                   dispatch buffer
//   surplus_shift = (surplus pairs of e from ranks < s) - local_quota, so
//                   that a surplus pair of stable rank rho has surplus
//                   index u = rho + surplus_shift
struct alignas(16) PairEntry {
  int32_t local_quota;
  int32_t local_base;
  int32_t surplus_shift;
  int32_t pad;
};

// Hosts of expert e that take surplus pairs, ascending rank, stored in a
// compact list: expert e owns entries [host_range[e].x, host_range[e].x +
// host_range[e].y); its capacity is 1 + (replicas of e).
//   end  = surplus index one past this host's share
//   base = dispatch row of surplus index 0 on this host (row - start index)
//   rank = host rank
//   lt   = local pairs this host keeps (they precede surplus from higher
//          source ranks in token order)
struct alignas(16) HostEntry {
  int32_t end;
  int32_t base;
  int32_t rank;
  int32_t lt;
};

struct Geometry {
  int32_t S, Eh, NS;     // tokens per rank, home experts per rank, slots per rank
  int32_t nbps, nblk;    // routing blocks per source rank, in total
};

struct WsLayout {
  size_t blockcnt, blockoff, blockflags, brank, expert_total, pair_tab, host_list, host_range,
      total;
};

// Entries of the compact host list: one home per expert plus one per
// replica slot.
inline int host_list_cap(const mb_dims& d) { return d.n_experts + d.n_ranks * d.slots_per_rank; }

Geometry geometry(const mb_dims& d);
WsLayout ws_layout(const mb_dims& d, const Geometry& g);

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_count(const mb_dims& d, const Geometry& g, const int32_t* ids,
                        int32_t* blockcnt, int32_t* blockflags, uint8_t* brank, hipStream_t st);
hipError_t launch_scan(const mb_dims& d, const Geometry& g, const int32_t* blockcnt,
                       int32_t* blockoff, int32_t* counts, int32_t* expert_total,
                       hipStream_t st);
// rank_speed: P host values (all 1 for the single water level);
// drift/drift_state: drift-gated replanning, or both nullptr; repair: the
// quota repair after placement.
// c_e comes from expert_total (k_scan ran), else from the block counts
// `blockcnt` (a small table: k_plan also writes d[s][e]), else from d[s][e]
// itself (one routing block per source). With pair_tab, host_list and
// host_range non-null k_plan also builds k_assign's lookup tables (few
// experts; k_tables is then not launched).
hipError_t launch_plan(const mb_dims& d, const Geometry& g, const mb_plan_bufs& o,
                       const int32_t* rank_speed, const mb_drift_params* drift,
                       void* drift_state, int repair, const int32_t* blockflags,
                       const int32_t* expert_total, const int32_t* blockcnt, PairEntry* pair_tab,
                       HostEntry* host_list, int2* host_range, hipStream_t st);

// Whether the block counts are few enough for k_plan and k_assign to sum
// them directly, so that k_scan is skipped.
inline bool small_block_table(const mb_dims& d, const Geometry& g) {
  return g.nbps > 1 && g.nbps <= kSmallTableBlocks &&
         (long long)g.nblk * d.n_experts <= kSmallTableCounts;
}

// Bytes of a drift state buffer: header, int64 reference [E], kept replicas
// and their placement order [P*R] each.
size_t drift_state_bytes(const mb_dims& d);
hipError_t launch_tables(const mb_dims& d, const Geometry& g, const mb_plan_bufs& o,
                         PairEntry* pair_tab, HostEntry* host_list, int2* host_range,
                         hipStream_t st);
// A block's offsets come from blockoff (k_scan ran), else from summing the
// earlier blocks of its source in blockcnt (small table), else are 0.
hipError_t launch_assign(const mb_dims& d, const Geometry& g, const int32_t* ids,
                         const uint8_t* brank, const int32_t* blockoff, const int32_t* blockcnt,
                         const PairEntry* pair_tab, const HostEntry* host_list,
                         const int2* host_range, const mb_plan_bufs& o, hipStream_t st);
hipError_t launch_dispatch(const mb_dims& d, const mb_plan_bufs& o, const void* x,
                           const float* x_scale, void* buf, float* buf_scale, hipStream_t st);
hipError_t launch_combine(const mb_dims& d, const mb_plan_bufs& o, const void* y_exp,
                          const float* w, void* y, hipStream_t st);
hipError_t launch_combine_fp8(const mb_dims& d, const mb_plan_bufs& o, const void* y_exp,
                              const float* y_scale, const float* w, void* y, hipStream_t st);

// Launch KERNEL<K> for the top-K values with a specialised kernel, KERNEL<0>
// (runtime K) otherwise.
#define MB_DISPATCH_TOPK(K, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                     \
  do {                                                                                   \
    switch (K) {                                                                         \
      case 1: hipLaunchKernelGGL(KERNEL<1>, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__); break; \
      case 2: hipLaunchKernelGGL(KERNEL<2>, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__); break; \
      case 4: hipLaunchKernelGGL(KERNEL<4>, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__); break; \
      case 8: hipLaunchKernelGGL(KERNEL<8>, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__); break; \
      default: hipLaunchKernelGGL(KERNEL<0>, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__); break; \
    }                                                                                    \
  } while (0)

inline int64_t elt_bytes(int32_t dtype) {
  return dtype == MB_F32 ? 4 : dtype == MB_BF16 ? 2 : dtype == MB_FP8_E4M3 ? 1 : 0;
}

}  // namespace mb
