// wave.h — wave64 primitives for gfx950 used by libmoebal's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mb {

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// v_writelane_b32: `old` with lane `lane` replaced by `value` (lane and value
// wave-uniform). This clang has no builtin for it, so the declaration names
// the LLVM intrinsic.
__device__ int writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// OR over the workgroup of per-thread status bits (the low 8 bits): one
// ballot per bit in each wave, a word per wave in `wfl`, and one barrier,
// which also orders the workgroup's earlier LDS writes as __syncthreads()
// does. Called once per kernel (wfl is not reset).
__device__ __forceinline__ int block_or_bits(int bits, int* wfl, int nwaves) {
  int w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= __ballot((bits >> i) & 1) ? 1 << i : 0;
  if ((threadIdx.x & 63) == 0) wfl[threadIdx.x >> 6] = w;
  __syncthreads();
  int all = 0;
  for (int i = 0; i < nwaves; ++i) all |= wfl[i];
  return all;
}

// DPP row shift / broadcast with `identity` for lanes that receive nothing.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_or_identity(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, kCtrl, kRowMask, 0xf, false);
}

// Full-wave reductions; every lane of the wave must be active. The result is
// uniform (read from lane 63 after an inclusive DPP scan: row_shr 1, 2, 4, 8
// inside 16-lane rows, then row_bcast 15 and row_bcast 31).
__device__ __forceinline__ int wave_max_i32(int v) {
  constexpr int I = INT32_MIN;
  v = max(v, dpp_or_identity<0x111, 0xf>(I, v));
  v = max(v, dpp_or_identity<0x112, 0xf>(I, v));
  v = max(v, dpp_or_identity<0x114, 0xf>(I, v));
  v = max(v, dpp_or_identity<0x118, 0xf>(I, v));
  v = max(v, dpp_or_identity<0x142, 0xa>(I, v));
  v = max(v, dpp_or_identity<0x143, 0xc>(I, v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_min_i32(int v) {
  constexpr int I = INT32_MAX;
  v = min(v, dpp_or_identity<0x111, 0xf>(I, v));
  v = min(v, dpp_or_identity<0x112, 0xf>(I, v));
  v = min(v, dpp_or_identity<0x114, 0xf>(I, v));
  v = min(v, dpp_or_identity<0x118, 0xf>(I, v));
  v = min(v, dpp_or_identity<0x142, 0xa>(I, v));
  v = min(v, dpp_or_identity<0x143, 0xc>(I, v));
  return __builtin_amdgcn_readlane(v, 63);
}

// max of `a` and min of `b` over lanes 0..kLanes-1 (kLanes = 32 or 64; the
// other lanes must hold the identities), the two DPP chains interleaved so
// that each hides the other's latency. With 32 lanes the row_bcast 31 step
// is left out and the result is read from lane 31.
template <int kLanes = 64>
__device__ __forceinline__ void wave_max_min_i32(int a, int b, int& amax, int& bmin) {
  static_assert(kLanes == 32 || kLanes == 64, "lane count");
  constexpr int IA = INT32_MIN, IB = INT32_MAX;
  a = max(a, dpp_or_identity<0x111, 0xf>(IA, a));
  b = min(b, dpp_or_identity<0x111, 0xf>(IB, b));
  a = max(a, dpp_or_identity<0x112, 0xf>(IA, a));
  b = min(b, dpp_or_identity<0x112, 0xf>(IB, b));
  a = max(a, dpp_or_identity<0x114, 0xf>(IA, a));
  b = min(b, dpp_or_identity<0x114, 0xf>(IB, b));
  a = max(a, dpp_or_identity<0x118, 0xf>(IA, a));
  b = min(b, dpp_or_identity<0x118, 0xf>(IB, b));
  a = max(a, dpp_or_identity<0x142, 0xa>(IA, a));
  b = min(b, dpp_or_identity<0x142, 0xa>(IB, b));
  if constexpr (kLanes == 64) {
    a = max(a, dpp_or_identity<0x143, 0xc>(IA, a));
    b = min(b, dpp_or_identity<0x143, 0xc>(IB, b));
  }
  amax = __builtin_amdgcn_readlane(a, kLanes - 1);
  bmin = __builtin_amdgcn_readlane(b, kLanes - 1);
}

// Inclusive prefix sum over the 64 lanes (every lane active).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += dpp_or_identity<0x111, 0xf>(0, v);
  v += dpp_or_identity<0x112, 0xf>(0, v);
  v += dpp_or_identity<0x114, 0xf>(0, v);
  v += dpp_or_identity<0x118, 0xf>(0, v);
  v += dpp_or_identity<0x142, 0xa>(0, v);
  v += dpp_or_identity<0x143, 0xc>(0, v);
  return v;
}

__device__ __forceinline__ int lowest_lane(uint64_t mask) {
  return mask ? __builtin_ctzll(mask) : -1;
}

}  // namespace mb
