// ceiling.hip — libmoebal_ceiling: reference kernels that bound k_dispatch
// (the MoonEP dispatch, "What MoonEP enforces and how": each token row read
// once and written to its K rows of the expert-grouped buffer).
//
// The dispatch moves N row reads and N*K row writes, the writes scattered
// over the buffer by pos. Against it: a contiguous fill and copy (HBM
// streaming), a contiguous read, and the dispatch's own writes with the reads
// taken out — in k_dispatch's shape (one 1 KiB lane span per wave, four waves
// per workgroup, K stores per lane) and in k_dispatch_span's (a workgroup of
// K waves per 2 KiB span, one destination row per wave). And the combine's
// traffic without its arithmetic: K gathered row loads per lane, one store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moebal_ceiling.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__global__ __launch_bounds__(kThreads) void k_fill(u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n16) dst[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
}

__global__ __launch_bounds__(kThreads) void k_copy(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void k_read(const u32x4* __restrict__ src, int64_t n16,
                                                   u32x4 key, u32x4* __restrict__ sink) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n16) {
    const u32x4 v = src[i];
    if (v.x == key.x && v.y == key.y && v.z == key.z && v.w == key.w) *sink = v;
  }
}

// k_dispatch's indexing with a register value in place of the row load.
template <int KT>
__global__ __launch_bounds__(kThreads) void k_scatter_write(const int32_t* __restrict__ pos,
                                                            u32x4* __restrict__ buf, int N, int K_,
                                                            int rb16, int wpt, int rows) {
  const int K = KT ? KT : K_;
  const int lane = threadIdx.x & 63;
  const int gw = uniform(blockIdx.x * kWaves + (threadIdx.x >> 6));
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= N) return;
  const int i = part * 64 + lane;
  if (i >= rb16) return;
  const u32x4 v = u32x4{(unsigned)t, (unsigned)i, 5u, 6u};
  const int32_t* pt = pos + (size_t)t * K;
  auto put = [&](int k) {
    const int p = pt[k];
    if ((unsigned)p < (unsigned)rows) buf[(size_t)p * rb16 + i] = v;
  };
  if constexpr (KT > 0) {
#pragma unroll
    for (int k = 0; k < KT; ++k) put(k);
  } else {
    for (int k = 0; k < K; ++k) put(k);
  }
}

// One destination row per wave: workgroup (t, span) of K waves, wave k
// writes 2 KiB (two 1 KiB lane spans) of row pos[t*K + k].
__global__ __launch_bounds__(1024) void k_row_write(const int32_t* __restrict__ pos,
                                                    u32x4* __restrict__ buf, int N, int K,
                                                    int rb16, int spans, int rows) {
  const int lane = threadIdx.x & 63, k = threadIdx.x >> 6;
  const int t = blockIdx.x / spans, s = blockIdx.x - t * spans;
  if (t >= N || k >= K) return;
  const int p = pos[(size_t)t * K + k];
  if ((unsigned)p >= (unsigned)rows) return;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = (s * 2 + c) * 64 + lane;
    if (i < rb16) buf[(size_t)p * rb16 + i] = u32x4{(unsigned)t, (unsigned)i, 3u, 4u};
  }
}

// The combine's traffic without its arithmetic, in k_combine's shape: one
// wave per 512 B of an output row (8-byte lane chunks), 16 waves per
// workgroup, a lane's K row loads issued before use (nontemporal), their XOR
// stored once (nontemporal).
constexpr int kGatherThreads = 1024;
constexpr int kGatherWaves = kGatherThreads / 64;

template <int KT>
__global__ __launch_bounds__(kGatherThreads) void k_gather_xor(const int32_t* __restrict__ pos,
                                                               const u32x2* __restrict__ ye,
                                                               u32x2* __restrict__ y, int N, int K_,
                                                               int rc, int wpt, int rows) {
  const int K = KT ? KT : K_;
  const int lane = threadIdx.x & 63;
  const int gw = uniform(blockIdx.x * kGatherWaves + (threadIdx.x >> 6));
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= N) return;
  const int ci = part * 64 + lane;
  if (ci >= rc) return;
  const int32_t* pt = pos + (size_t)t * K;
  u32x2 acc = u32x2{0u, 0u};
  if constexpr (KT > 0) {
    u32x2 v[KT];
    bool ok[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {  // as k_combine: every load issued, at row 0 when skipped
      const int p = pt[k];
      ok[k] = (unsigned)p < (unsigned)rows;
      v[k] = __builtin_nontemporal_load(ye + (ok[k] ? (size_t)p : 0) * rc + ci);
    }
#pragma unroll
    for (int k = 0; k < KT; ++k)
      if (ok[k]) acc ^= v[k];
  } else {
    for (int k = 0; k < K; ++k) {
      const int p = pt[k];
      if ((unsigned)p < (unsigned)rows) acc ^= __builtin_nontemporal_load(ye + (size_t)p * rc + ci);
    }
  }
  __builtin_nontemporal_store(acc, y + (size_t)t * rc + ci);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Blocks for n16 lanes of one 16-byte access each, or -1 past the grid limit.
int64_t stream_blocks(int64_t n16) {
  const int64_t b = (n16 + kThreads - 1) / kThreads;
  return b <= 0x7fffffff ? b : -1;
}

bool rows_ok(const int32_t* pos, const void* buf, int32_t N, int32_t K, int32_t row_bytes,
             int32_t rows, int kmax) {
  return pos && buf && aligned16(buf) && N >= 0 && K >= 1 && K <= kmax && row_bytes > 0 &&
         row_bytes % 16 == 0 && rows >= 0;
}

}  // namespace

extern "C" {

int mbc_fill(void* dst, int64_t bytes, hipStream_t st) {
  if (!dst || !aligned16(dst) || bytes < 0 || bytes % 16) return -1;
  const int64_t n16 = bytes / 16, b = stream_blocks(n16);
  if (b < 0) return -1;
  if (b == 0) return 0;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)b), dim3(kThreads), 0, st, static_cast<u32x4*>(dst),
                     n16);
  return hipGetLastError();
}

int mbc_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes < 0 || bytes % 16) return -1;
  const int64_t n16 = bytes / 16, b = stream_blocks(n16);
  if (b < 0) return -1;
  if (b == 0) return 0;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)b), dim3(kThreads), 0, st,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

int mbc_read(const void* src, int64_t bytes, const uint32_t key[4], void* sink, hipStream_t st) {
  if (!src || !sink || !key || !aligned16(src) || !aligned16(sink) || bytes < 0 || bytes % 16)
    return -1;
  const int64_t n16 = bytes / 16, b = stream_blocks(n16);
  if (b < 0) return -1;
  if (b == 0) return 0;
  const u32x4 kv = u32x4{key[0], key[1], key[2], key[3]};
  hipLaunchKernelGGL(k_read, dim3((unsigned)b), dim3(kThreads), 0, st,
                     static_cast<const u32x4*>(src), n16, kv, static_cast<u32x4*>(sink));
  return hipGetLastError();
}

int mbc_scatter_write(const int32_t* pos, void* buf, int32_t N, int32_t K, int32_t row_bytes,
                      int32_t rows, hipStream_t st) {
  if (!rows_ok(pos, buf, N, K, row_bytes, rows, 32)) return -1;
  const int rb16 = row_bytes / 16, wpt = (rb16 + 63) / 64;
  const int64_t waves = (int64_t)N * wpt, blocks = (waves + kWaves - 1) / kWaves;
  if (waves > 0x7fffffff) return -1;
  if (blocks == 0) return 0;
  const dim3 g((unsigned)blocks), b(kThreads);
  auto* out = static_cast<u32x4*>(buf);
  switch (K) {
    case 8: hipLaunchKernelGGL(k_scatter_write<8>, g, b, 0, st, pos, out, N, K, rb16, wpt, rows); break;
    case 4: hipLaunchKernelGGL(k_scatter_write<4>, g, b, 0, st, pos, out, N, K, rb16, wpt, rows); break;
    default: hipLaunchKernelGGL(k_scatter_write<0>, g, b, 0, st, pos, out, N, K, rb16, wpt, rows); break;
  }
  return hipGetLastError();
}

int mbc_row_write(const int32_t* pos, void* buf, int32_t N, int32_t K, int32_t row_bytes,
                  int32_t rows, hipStream_t st) {
  if (!rows_ok(pos, buf, N, K, row_bytes, rows, 16)) return -1;
  const int rb16 = row_bytes / 16, spans = (rb16 + 127) / 128;
  const int64_t blocks = (int64_t)N * spans;
  if (blocks > 0x7fffffff) return -1;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(k_row_write, dim3((unsigned)blocks), dim3(64 * K), 0, st, pos,
                     static_cast<u32x4*>(buf), N, K, rb16, spans, rows);
  return hipGetLastError();
}

int mbc_gather_xor(const int32_t* pos, const void* y_exp, void* y, int32_t N, int32_t K,
                   int32_t row_bytes, int32_t rows, hipStream_t st) {
  if (!rows_ok(pos, y_exp, N, K, row_bytes, rows, 32) || !y || !aligned16(y)) return -1;
  const int rc = row_bytes / 8, wpt = (rc + 63) / 64;
  const int64_t waves = (int64_t)N * wpt, blocks = (waves + kGatherWaves - 1) / kGatherWaves;
  if (waves > 0x7fffffff) return -1;
  if (blocks == 0) return 0;
  const dim3 g((unsigned)blocks), b(kGatherThreads);
  const auto* src = static_cast<const u32x2*>(y_exp);
  auto* out = static_cast<u32x2*>(y);
  switch (K) {
    case 8: hipLaunchKernelGGL(k_gather_xor<8>, g, b, 0, st, pos, src, out, N, K, rc, wpt, rows); break;
    case 2: hipLaunchKernelGGL(k_gather_xor<2>, g, b, 0, st, pos, src, out, N, K, rc, wpt, rows); break;
    default: hipLaunchKernelGGL(k_gather_xor<0>, g, b, 0, st, pos, src, out, N, K, rc, wpt, rows); break;
  }
  return hipGetLastError();
}

}  // extern "C"
