// route.hip — counting, per-source prefix offsets and the per-pair
// assignment of libmoebal's plan.
//
// Stable ranks without atomics deciding order. A routing workgroup owns 256
// consecutive tokens of one source rank (one token per lane). In k_count each
// wave64 builds, in LDS, one 64-bit mask per expert whose bit l says "lane
// l's token routes to this expert" (ds_or_b64: commutative, so the masks do
// not depend on timing). A pair's rank among the earlier pairs of its (source
// rank, expert) is then
//   rho = (pairs in earlier workgroups of the same source, from k_scan)
//       + popcount of the masks of earlier waves
//       + popcount of its own wave's mask below its lane (mbcnt);
// k_count stores the in-workgroup part (below 256, one byte) for k_assign.
// Tokens list distinct experts, so "earlier pair with the same expert" and
// "earlier token with that expert" coincide.
//
// Sources: ISER-MoE, HALO-Q stage 1 (route counts per rank) and stage 5
// (local-first rewrite of surplus routes onto the hosts' spare quotas);
// Zepp summary §4.1, eq. (1) (demand d_i^e per source GPU, locality-preferred
// routing); MoonEP, "What MoonEP enforces and how" (fixed per-rank regions
// indexed by cu_seqlens).
#include "mb_internal.h"
#include "tables.h"
#include "wave.h"

namespace mb {
namespace {

// Sets this lane's bit in the wave's mask of each of its token's experts and
// returns the token's status bits (bad or repeated ids). With a compile-time
// K the ids are already in registers; otherwise they are read one by one.
template <int KT>
__device__ __forceinline__ int mark_token(const int* ev, const int32_t* __restrict__ row, int K_,
                                          int E, unsigned long long* wmask, int lane) {
  int flags = 0;
  if constexpr (KT > 0) {
#pragma unroll
    for (int k = 1; k < KT; ++k)
#pragma unroll
      for (int k2 = 0; k2 < k; ++k2)
        if (ev[k2] == ev[k]) flags |= MB_ST_DUP_ID;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if ((unsigned)ev[k] >= (unsigned)E)
        flags |= MB_ST_BAD_ID;
      else
        atomicOr(&wmask[ev[k]], 1ull << lane);
    }
  } else {
    for (int k = 0; k < K_; ++k) {
      const int e = row[k];
      for (int k2 = 0; k2 < k; ++k2)
        if (row[k2] == e) flags |= MB_ST_DUP_ID;
      if ((unsigned)e >= (unsigned)E) {
        flags |= MB_ST_BAD_ID;
        continue;
      }
      atomicOr(&wmask[e], 1ull << lane);
    }
  }
  return flags;
}

template <int KT>
__global__ __launch_bounds__(kTokensPerBlock) void k_count(
    const int32_t* __restrict__ ids, int K_, int E, int S, int nbps,
    int32_t* __restrict__ blockcnt, int32_t* __restrict__ blockflags,
    uint8_t* __restrict__ brank) {
  extern __shared__ unsigned long long masks[];  // [kWaves][E], then int32 [kWaves][E]
  const int K = KT ? KT : K_;
  const int b = blockIdx.x;
  const int s = b / nbps, j = b - s * nbps;
  const int tl = threadIdx.x;
  const int nt = min(kTokensPerBlock, S - j * kTokensPerBlock);
  const int w = tl >> 6, lane = tl & 63;
  const size_t t = (size_t)s * S + (size_t)j * kTokensPerBlock + tl;
  const int32_t* row = ids + t * K;
  // The lane's ids are loaded before the masks are cleared, so their
  // latency overlaps the clearing; they stay in registers for the ranks.
  constexpr int KR = KT ? KT : 1;
  int ev[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) ev[k] = KT && tl < nt ? row[k] : 0;
  for (int i = tl; i < kWaves * E; i += kTokensPerBlock) masks[i] = 0ull;
  __syncthreads();
  int flags = 0;
  if (tl < nt) flags = mark_token<KT>(ev, row, K, E, masks + w * E, lane);
  __shared__ int wfl[kWaves];
  const int fl_all = block_or_bits(flags, wfl, kWaves);
  const int bad = fl_all & MB_ST_BAD_ID, dup = fl_all & MB_ST_DUP_ID;
  // before[w][e]: pairs of e in the waves before w
  int32_t* before = reinterpret_cast<int32_t*>(masks + kWaves * E);
  for (int e = tl; e < E; e += kTokensPerBlock) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      before[ww * E + e] = c;
      c += __popcll(masks[ww * E + e]);
    }
    blockcnt[(size_t)b * E + e] = c;
  }
  if (tl == 0) blockflags[b] = (bad ? MB_ST_BAD_ID : 0) | (dup ? MB_ST_DUP_ID : 0);
  __syncthreads();
  if (tl >= nt) return;
  // In-workgroup rank of each of the token's pairs (0 for a bad id).
  auto rank_in_block = [&](int e) -> uint32_t {
    if ((unsigned)e >= (unsigned)E) return 0u;
    return (uint32_t)(before[w * E + e] + lanes_below(masks[w * E + e]));
  };
  if constexpr (KT == 8) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) lo |= rank_in_block(ev[k]) << (8 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) hi |= rank_in_block(ev[4 + k]) << (8 * k);
    reinterpret_cast<uint2*>(brank)[t] = make_uint2(lo, hi);
  } else if constexpr (KT == 4) {
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) v |= rank_in_block(ev[k]) << (8 * k);
    reinterpret_cast<uint32_t*>(brank)[t] = v;
  } else if constexpr (KT > 0) {
#pragma unroll
    for (int k = 0; k < KT; ++k) brank[t * K + k] = (uint8_t)rank_in_block(ev[k]);
  } else {
    for (int k = 0; k < K; ++k) brank[t * K + k] = (uint8_t)rank_in_block(row[k]);
  }
}

// Exclusive scan over the workgroups of each source rank, per expert; the
// per-source totals d[s][e]; and c_e = sum_s d[s][e]. A workgroup covers
// 256 / P experts for all P sources (thread = (source, expert)), so c_e is
// a reduction inside the workgroup.
__global__ __launch_bounds__(256) void k_scan(const int32_t* __restrict__ blockcnt, int E, int P,
                                               int nbps, int32_t* __restrict__ blockoff,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ expert_total) {
  __shared__ int32_t part[256];
  const int epw = 256 / P;
  const int tid = threadIdx.x;
  const int s = tid / epw, el = tid - s * epw;
  const int e = blockIdx.x * epw + el;
  int off = 0;
  if (s < P && e < E) {
    const size_t b0 = (size_t)s * nbps;
    int j = 0;
    for (; j + 16 <= nbps; j += 16) {  // 16 loads in flight per round trip
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = blockcnt[(b0 + j + i) * E + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        blockoff[(b0 + j + i) * E + e] = off;
        off += c[i];
      }
    }
    for (; j < nbps; ++j) {
      const int c = blockcnt[(b0 + j) * E + e];
      blockoff[(b0 + j) * E + e] = off;
      off += c;
    }
    counts[(size_t)s * E + e] = off;
  }
  part[tid] = off;
  __syncthreads();
  if (tid < epw && blockIdx.x * epw + tid < E) {
    int c = 0;
    for (int q = 0; q < P; ++q) c += part[q * epw + tid];
    expert_total[blockIdx.x * epw + tid] = c;
  }
}

// Dispatch row of every pair, and the token of every row (-1 for padding).
// The workgroup stages in LDS its rows of the offset and pair tables and,
// when it fits (kStageHosts), the whole compact host list.
template <int KT, bool kStageHosts>
__global__ __launch_bounds__(kTokensPerBlock) void k_assign(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ brank, int K_, int E, int S,
    int P, int nbps, int nblk, int cap, int nhost, const int32_t* __restrict__ blockoff,
    const PairEntry* __restrict__ pair_tab, const HostEntry* __restrict__ host_list,
    const int2* __restrict__ host_range, const int32_t* __restrict__ status,
    const int32_t* __restrict__ load_post, int32_t* __restrict__ pos,
    int32_t* __restrict__ row_src, const int32_t* __restrict__ blockcnt) {
  // LDS: offsets [E4] | pairs [E] | ranges [E4] | hosts [nhost]
  extern __shared__ int4 lds[];
  __shared__ int32_t lp_s[kMaxRanks];
  // The plan's status is loaded with the tables and checked after staging,
  // before anything is stored.
  const int st = status[0];
  const int K = KT ? KT : K_;
  const int b = blockIdx.x;
  const int tl = threadIdx.x;
  const int s = b / max(nbps, 1), j = b - s * nbps;
  const bool has_tokens = b < nblk;
  const int nt = has_tokens ? min(kTokensPerBlock, S - j * kTokensPerBlock) : 0;
  const int E4 = (E + 3) & ~3;
  int32_t* boff = reinterpret_cast<int32_t*>(lds);
  PairEntry* ptab = reinterpret_cast<PairEntry*>(boff + E4);
  int2* hrange = reinterpret_cast<int2*>(ptab + E);
  HostEntry* hl = reinterpret_cast<HostEntry*>(hrange + E4);

  // The lane's token: expert ids and in-workgroup ranks, fetched first.
  const size_t t = (size_t)s * S + (size_t)j * kTokensPerBlock + tl;
  constexpr int KR = KT ? KT : 1;
  int er[KR], br[KR];
  if (KT && tl < nt) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      er[k] = ids[t * K + k];
      br[k] = brank[t * K + k];
    }
  }
  int pad = 0;
  if (tl < P) {
    lp_s[tl] = load_post[tl];
    pad = cap - lp_s[tl];
  }
  if (has_tokens) {
    for (int i = tl; i < E; i += kTokensPerBlock) {
      // from k_scan; else the sum of the source's earlier blocks (j of
      // them, a small table); with one block per source, 0
      int o = 0;
      if (blockoff) {
        o = blockoff[(size_t)b * E + i];
      } else if (blockcnt) {
        for (int jj = 0; jj < j; ++jj) o += blockcnt[(size_t)(b - j + jj) * E + i];
      }
      boff[i] = o;
      ptab[i] = pair_tab[(size_t)s * E + i];
      hrange[i] = host_range[i];
    }
    if constexpr (kStageHosts)
      for (int i = tl; i < nhost; i += kTokensPerBlock) hl[i] = host_list[i];
  }
  const HostEntry* hosts = kStageHosts ? hl : host_list;
  // Padding rows: region r has rows [r*cap + load_post[r], (r+1)*cap); with
  // every region full (a balanced plan at cap = T) there are none. Global
  // wave gw fills region gw mod P, the waves of one region interleaving in
  // 64-row strides (or, with fewer waves than regions, wave gw fills
  // regions gw, gw + GW, ...).
  __shared__ int wfl[kWaves];
  const bool fill = block_or_bits(pad > 0 ? 1 : 0, wfl, kWaves) != 0;
  if (st & MB_ST_FATAL) return;
  if (fill) {
    const int GW = gridDim.x * kWaves, gw = b * kWaves + (tl >> 6), ln = tl & 63;
    if (GW >= P) {
      const int r = gw % P, k = gw / P, nk = (GW - 1 - r) / P + 1;  // waves r, r + P, ... < GW
      const int lp = lp_s[r];
      for (int i = k * 64 + ln; i < cap - lp; i += nk * 64) row_src[(size_t)r * cap + lp + i] = -1;
    } else {
      for (int r = gw; r < P; r += GW) {
        const int lp = lp_s[r];
        for (int i = ln; i < cap - lp; i += 64) row_src[(size_t)r * cap + lp + i] = -1;
      }
    }
  }
  if (tl >= nt) return;

  const int rows = P * cap;
  // Pass 1 keeps the first local_quota pairs of (s, e) on s; a later pair is
  // surplus number u of e and goes to the host whose share covers u.
  // The hosts' share ends ascend (each host listed has spare quota), so the
  // host of surplus number u is found by bisection.
  auto search = [&](const int2 rg, int u, int q0) {
    int lo = q0, hi = rg.y;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (u < hosts[rg.x + mid].end)
        hi = mid;
      else
        lo = mid + 1;
    }
    if (lo >= rg.y) return -1;
    const HostEntry h = hosts[rg.x + lo];
    return h.base + u + (h.rank < s ? h.lt : 0);
  };
  if constexpr (KT > 0) {
    // All table reads of the K pairs are independent; the first two hosts of
    // each expert are probed unconditionally (clamped indices stay inside
    // the expert's own range), the rest only when a share lies further out.
    PairEntry pe[KT];
    int2 rg[KT];
    HostEntry h0[KT], h1[KT];
    int rho[KT], p[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      rho[k] = boff[er[k]] + br[k];
      pe[k] = ptab[er[k]];
      rg[k] = hrange[er[k]];
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      h0[k] = hosts[rg[k].x];
      h1[k] = hosts[rg[k].x + (rg[k].y > 1 ? 1 : 0)];
    }
    // Every candidate row is computed and the right one selected, so the
    // table reads above stay independent of each other; only a share past
    // the second host needs the bisection.
    unsigned far = 0;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int u = rho[k] + pe[k].surplus_shift;
      const int p0 = h0[k].base + u + (h0[k].rank < s ? h0[k].lt : 0);
      const int p1 = h1[k].base + u + (h1[k].rank < s ? h1[k].lt : 0);
      const bool loc = rho[k] < pe[k].local_quota, in0 = u < h0[k].end;
      const bool in1 = rg[k].y > 1 && u < h1[k].end;
      p[k] = loc ? pe[k].local_base + rho[k] : in0 ? p0 : p1;
      far |= (!loc && !in0 && !in1) ? 1u << k : 0u;
    }
    if (far) {
#pragma unroll
      for (int k = 0; k < KT; ++k)
        if (far >> k & 1) p[k] = search(rg[k], rho[k] + pe[k].surplus_shift, 2);
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) pos[t * K + k] = p[k];
#pragma unroll
    for (int k = 0; k < KT; ++k)
      if ((unsigned)p[k] < (unsigned)rows) row_src[p[k]] = (int32_t)t;
  } else {
    for (int k = 0; k < K; ++k) {
      const int e = ids[t * K + k];
      const int rho = boff[e] + brank[t * K + k];
      const PairEntry pe = ptab[e];
      const int p = rho < pe.local_quota ? pe.local_base + rho
                                         : search(hrange[e], rho + pe.surplus_shift, 0);
      pos[t * K + k] = p;
      if ((unsigned)p < (unsigned)rows) row_src[p] = (int32_t)t;
    }
  }
}

// Lookup tables of k_assign, one wave per expert (tables.h).
__global__ __launch_bounds__(256) void k_tables(
    int E, int P, int R, int Eh, int NS, int cap, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ rep_expert, const int32_t* __restrict__ slot_quota,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ status,
    PairEntry* __restrict__ pair_tab, HostEntry* __restrict__ host_list,
    int2* __restrict__ host_range) {
  if (status[0] & MB_ST_FATAL) return;
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (e >= E) return;
  tables_for_expert(e, E, P, R, Eh, NS, cap, counts, rep_expert, slot_quota, cu_seqlens,
                    pair_tab, host_list, host_range);
}

}  // namespace


hipError_t launch_count(const mb_dims& d, const Geometry& g, const int32_t* ids,
                        int32_t* blockcnt, int32_t* blockflags, uint8_t* brank, hipStream_t st) {
  if (g.nblk == 0) return hipSuccess;
  const size_t shmem = (sizeof(unsigned long long) + sizeof(int32_t)) * kWaves * d.n_experts;
  MB_DISPATCH_TOPK(d.top_k, k_count, dim3(g.nblk), dim3(kTokensPerBlock), shmem, st, ids,
                   d.top_k, d.n_experts, g.S, g.nbps, blockcnt, blockflags, brank);
  return hipGetLastError();
}

hipError_t launch_scan(const mb_dims& d, const Geometry& g, const int32_t* blockcnt,
                       int32_t* blockoff, int32_t* counts, int32_t* expert_total,
                       hipStream_t st) {
  const int epw = 256 / d.n_ranks;
  hipLaunchKernelGGL(k_scan, dim3((d.n_experts + epw - 1) / epw), dim3(256), 0, st, blockcnt,
                     d.n_experts, d.n_ranks, g.nbps, blockoff, counts, expert_total);
  return hipGetLastError();
}

hipError_t launch_tables(const mb_dims& d, const Geometry& g, const mb_plan_bufs& o,
                         PairEntry* pair_tab, HostEntry* host_list, int2* host_range,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_tables, dim3((d.n_experts + 3) / 4), dim3(256), 0, st, d.n_experts,
                     d.n_ranks, d.slots_per_rank, g.Eh, g.NS, d.cap, o.counts, o.rep_expert,
                     o.slot_quota, o.cu_seqlens, o.status, pair_tab, host_list, host_range);
  return hipGetLastError();
}

hipError_t launch_assign(const mb_dims& d, const Geometry& g, const int32_t* ids,
                         const uint8_t* brank, const int32_t* blockoff, const int32_t* blockcnt,
                         const PairEntry* pair_tab, const HostEntry* host_list,
                         const int2* host_range, const mb_plan_bufs& o, hipStream_t st) {
  const int64_t rows = (int64_t)d.n_ranks * d.cap;
  int grid = g.nblk;
  const int64_t pad_blocks = (rows + kTokensPerBlock - 1) / kTokensPerBlock;
  if (grid == 0) grid = (int)(pad_blocks < 1024 ? pad_blocks : 1024);
  if (grid < 1) grid = 1;
  const int E4 = (d.n_experts + 3) & ~3;
  const int nhost = host_list_cap(d);
  const size_t base =
      sizeof(int32_t) * E4 + sizeof(PairEntry) * d.n_experts + sizeof(int2) * E4;
  const size_t with_hosts = base + sizeof(HostEntry) * nhost;
  const bool stage = with_hosts <= 48 * 1024;
  const size_t shmem = stage ? with_hosts : base;
#define MB_A(KT)                                                                             \
  do {                                                                                       \
    if (stage)                                                                               \
      hipLaunchKernelGGL((k_assign<KT, true>), dim3(grid), dim3(kTokensPerBlock), shmem, st, \
                         ids, brank, d.top_k, d.n_experts, g.S, d.n_ranks, g.nbps, g.nblk,   \
                         d.cap, nhost, blockoff, pair_tab, host_list, host_range, o.status,  \
                         o.load_post, o.pos, o.row_src, blockcnt);                           \
    else                                                                                     \
      hipLaunchKernelGGL((k_assign<KT, false>), dim3(grid), dim3(kTokensPerBlock), shmem,    \
                         st, ids, brank, d.top_k, d.n_experts, g.S, d.n_ranks, g.nbps,       \
                         g.nblk, d.cap, nhost, blockoff, pair_tab, host_list, host_range,    \
                         o.status, o.load_post, o.pos, o.row_src, blockcnt);                 \
  } while (0)
  switch (d.top_k) {
    case 1: MB_A(1); break;
    case 2: MB_A(2); break;
    case 4: MB_A(4); break;
    case 8: MB_A(8); break;
    default: MB_A(0); break;
  }
#undef MB_A
  return hipGetLastError();
}

}  // namespace mb
