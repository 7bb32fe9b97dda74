// rows.hip — row dispatch (scatter) and combine (weighted gather-reduce).
//
// The kernels are HBM-bound byte movers: one wave64 per part of a token's
// row, a token's parts on consecutive waves; dispatch moves 1 KiB parts in
// 16-byte lane chunks (global_load/store_dwordx4), or, for rows of whole
// 2 KiB spans, one span per workgroup of K waves staged once in LDS; the
// combines move 512-byte parts in 8-byte lane chunks. The part size and the cache hint of each
// access (temporal or nontemporal) are the ones measured fastest on MI355X
// for that kernel's traffic mix; see the comment at each kernel.
//
// Dispatch reads each token row once and stores it to its K rows (the
// one-GPU form of "a token's experts on one node share a transfer" in the
// Zepp summary §4.2, Merge). Combine reads the K expert-output rows of a
// token, accumulates w[t][k] * row in fp32 in k order and stores the result
// once.
//
// Sources: MoonEP, "What MoonEP enforces and how" (tokens written straight
// into fixed-shape expert-grouped buffers, kernels indexing rows through the
// planner's layout); Zepp summary §4.2 (Merge: dispatch shares a token's
// transfer, combine aggregates a token's expert outputs).
#include <type_traits>

#include "mb_internal.h"

namespace mb {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowThreads = 256;
constexpr int kWavesPerRowBlock = kRowThreads / 64;
// The combine kernels launch 16-wave workgroups: for their small waves this
// measured 1.5-2 % faster on MI355X than 4- or 8-wave groups (dispatch is
// fastest with 4).
constexpr int kCombThreads = 1024;
constexpr int kWavesPerCombBlock = kCombThreads / 64;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Dispatch: one wave per 1 KiB chunk of a token row (64 lanes x 16 bytes),
// the chunks of a token on consecutive waves; each wave loads its chunk once
// and stores it to the token's K rows. On MI355X this shape moved the
// 1-read / K-write traffic faster than a wave holding a whole row (many small
// waves keep more independent store streams in flight) and 3 % faster than
// 512-byte chunks, and plain (temporal) loads and stores beat nontemporal
// ones here.
template <int KT>
__global__ __launch_bounds__(kRowThreads) void k_dispatch(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ status, u32x4* __restrict__ buf, int N, int K_, int rb16,
    int wpt, int rows, const float* __restrict__ xs, float* __restrict__ bs, int nsc, int vec4) {
  const int K = KT ? KT : K_;
  const int lane = threadIdx.x & 63;
  const int gw = uniform(blockIdx.x * kWavesPerRowBlock + (threadIdx.x >> 6));
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= N) return;
  if (status[0] & MB_ST_FATAL) return;
  const int i = part * 64 + lane;
  const int32_t* pt = pos + (size_t)t * K;
  if (i < rb16) {
    const u32x4 v = x[(size_t)t * rb16 + i];
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
  // fp8 rows: the token's first wave also copies its scale row to the K
  // rows, one (row, unit) pair per lane: 16-byte units when the scale arrays
  // allow it (vec4), else single floats. This issues ceil(K * units / 64)
  // stores instead of K narrow ones (3 % of the fp8 dispatch at 8192 tokens
  // x 8 x 7168 on MI355X; one extra wave per token for the scales was
  // slower).
  if (part == 0 && nsc > 0) {
    if (vec4) {
      const int cu = nsc >> 2;
      const u32x4* src = reinterpret_cast<const u32x4*>(xs) + (size_t)t * cu;
      u32x4* dst = reinterpret_cast<u32x4*>(bs);
      for (int u = lane; u < K * cu; u += 64) {
        const int k = u / cu, c = u - k * cu;
        const int p = pt[k];
        if ((unsigned)p < (unsigned)rows) dst[(size_t)p * cu + c] = src[c];
      }
    } else {
      for (int u = lane; u < K * nsc; u += 64) {
        const int k = u / nsc, c = u - k * nsc;
        const int p = pt[k];
        if ((unsigned)p < (unsigned)rows) bs[(size_t)p * nsc + c] = xs[(size_t)t * nsc + c];
      }
    }
  }
}

// Dispatch of rows made of whole 2 KiB spans (2 <= K <= 16): a workgroup
// of K waves per (token, span); the span's 128 lane chunks are loaded once
// into LDS, then wave k writes the whole span to row pos[t][k] (two 1 KiB
// stores per lane, 2 KiB contiguous per wave). On MI355X this beat the
// one-wave-per-chunk kernel by 2 % at 131072 tokens x 8 x 14336 B (3.08 vs
// 3.16 ms): the destination rows receive 2 KiB runs instead of 1 KiB ones
// (write-only, those runs alone measured 5.80 against 5.56 TB/s), while the
// load is shared by the K waves. Spans of 1, 3 and 4 KiB were 22, 7 and 11 %
// slower than 2 KiB ones; on fp8 rows of 7168 B (3.5 spans) this kernel lost.
// With its arguments all in preloaded registers (below) the bf16 case runs
// at 2.95 ms, 5.73 TB/s: 99 % of the same writes alone in the same shape.
// For fp8 rows the first span's waves also copy the token's scale row to
// their destination, 16-byte units when the scale arrays allow (vec4).
constexpr int kSpanChunks = 128;  // 16-byte lane chunks per 2 KiB span

// kScales: fp8 rows, whose scale rows travel too. Without it the kernel has
// no scale code at all: its arguments then fit the preloaded kernel-argument
// registers, where the scale arguments had cost every wave a scalar load
// between the barrier and its stores (3.08 against 2.94 ms at 131072 tokens
// x 8 x 14336 B, measured).
template <int KT, bool kScales>
__global__ __launch_bounds__(KT > 0 ? 64 * KT : 1024) void k_dispatch_span(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ status, u32x4* __restrict__ buf, int K_, int rb16, int spans,
    int rows, const float* __restrict__ xs, float* __restrict__ bs, int nsc, int vec4) {
  __shared__ u32x4 span[kSpanChunks];
  const int K = KT ? KT : K_;
  const int lane = threadIdx.x & 63, k = threadIdx.x >> 6;
  const int t = blockIdx.x / spans, h = blockIdx.x - t * spans;
  if (status[0] & MB_ST_FATAL) return;  // the same word for every thread
  const int base = h * kSpanChunks;
  const int p = pos[(size_t)t * K + k];
  if (threadIdx.x < kSpanChunks) span[threadIdx.x] = x[(size_t)t * rb16 + base + threadIdx.x];
  __syncthreads();
  if ((unsigned)p >= (unsigned)rows) return;
  u32x4* dst = buf + (size_t)p * rb16 + base;
  dst[lane] = span[lane];
  dst[64 + lane] = span[64 + lane];
  if constexpr (kScales) {
    if (h == 0) {
      if (vec4) {
        const int cu = nsc >> 2;
        const u32x4* src = reinterpret_cast<const u32x4*>(xs) + (size_t)t * cu;
        u32x4* d4 = reinterpret_cast<u32x4*>(bs) + (size_t)p * cu;
        for (int u = lane; u < cu; u += 64) d4[u] = src[u];
      } else {
        for (int u = lane; u < nsc; u += 64) bs[(size_t)p * nsc + u] = xs[(size_t)t * nsc + u];
      }
    }
  }
}

template <bool kScales>
static void launch_dispatch_span(const mb_dims& d, const mb_plan_bufs& o, const void* x,
                                 const float* xs, void* buf, float* bs, int rb16, int rows,
                                 int nsc, int vec4, hipStream_t st) {
  const int spans = rb16 / kSpanChunks;
  const dim3 grid((unsigned)((int64_t)d.n_tokens * spans)), block(64 * d.top_k);
  const auto* xv = static_cast<const u32x4*>(x);
  auto* bv = static_cast<u32x4*>(buf);
#define MB_S(KT)                                                                                  \
  hipLaunchKernelGGL((k_dispatch_span<KT, kScales>), grid, block, 0, st, xv, o.pos, o.status, bv, \
                     d.top_k, rb16, spans, rows, xs, bs, nsc, vec4)
  switch (d.top_k) {
    case 2: MB_S(2); break;
    case 4: MB_S(4); break;
    case 8: MB_S(8); break;
    default: MB_S(0); break;
  }
#undef MB_S
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;  // quiet NaN
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// A lane chunk of CW dwords (8 or 16 bytes).
template <int CW>
using chunk_t = typename std::conditional<CW == 4, u32x4, u32x2>::type;

// acc[0..2CW) += w * (2 CW bf16 of v), or acc[0..CW) += w * (CW f32 of v).
template <bool kBF16, int CW>
__device__ __forceinline__ void fma_chunk(float* acc, float w, chunk_t<CW> v) {
  if constexpr (kBF16) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      acc[2 * i] = fmaf(w, __uint_as_float(v[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(w, __uint_as_float(v[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CW; ++i) acc[i] = fmaf(w, __uint_as_float(v[i]), acc[i]);
  }
}

// The accumulators of one chunk to bf16 pairs or f32.
template <bool kBF16, int CW>
__device__ __forceinline__ chunk_t<CW> pack_chunk(const float* acc) {
  chunk_t<CW> o;
  if constexpr (kBF16) {
#pragma unroll
    for (int i = 0; i < CW; ++i)
      o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < CW; ++i) o[i] = __float_as_uint(acc[i]);
  }
  return o;
}

// Combine: one wave per part of a token's output row (64 lanes x one chunk
// of CW dwords), the parts of a token on consecutive waves; each lane reads
// its chunk of the token's K expert rows, accumulates w[t][k] * value in
// fp32 in k order and stores the chunk once. With a compile-time K the K
// loads are issued before the first FMA. Measured on MI355X: with K = 8,
// 8-byte chunks (512-byte parts) moved the K-read / 1-write traffic faster
// than 16-byte chunks (2.71-2.89 against 2.99 ms at 131072 tokens x top-8 x
// 7168 bf16; 170 against 183 us at 8192 tokens x 8) and 4-byte chunks; with
// K = 2, 16-byte chunks are faster (20.8 against 22.5 us at 4096 tokens x 2
// x 4096), a wave with only two loads needing the wider chunk. Waves of
// 16-byte chunks had in turn beaten one wave per whole row, and nontemporal
// loads and stores beat temporal ones.
template <int KT, bool kBF16, int CW>
__global__ __launch_bounds__(kCombThreads) void k_combine(
    const chunk_t<CW>* __restrict__ ye, const int32_t* __restrict__ pos,
    const float* __restrict__ w, const int32_t* __restrict__ status, chunk_t<CW>* __restrict__ y,
    int N, int K_, int rc, int wpt, int rows) {
  constexpr int EPC = kBF16 ? 2 * CW : CW;  // elements per chunk
  const int K = KT ? KT : K_;
  const int lane = threadIdx.x & 63;
  const int gw = uniform(blockIdx.x * kWavesPerCombBlock + (threadIdx.x >> 6));
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= N) return;
  if (status[0] & MB_ST_FATAL) return;
  const int ci = part * 64 + lane;  // this lane's chunk of the row
  if (ci >= rc) return;
  const int32_t* pt = pos + (size_t)t * K;
  const float* wt = w + (size_t)t * K;
  float acc[EPC];
#pragma unroll
  for (int i = 0; i < EPC; ++i) acc[i] = 0.0f;
  if constexpr (KT > 0) {
    chunk_t<CW> v[KT];
    bool ok[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int p = pt[k];
      ok[k] = (unsigned)p < (unsigned)rows;  // only a broken plan fails this
      v[k] = __builtin_nontemporal_load(ye + (ok[k] ? (size_t)p : 0) * rc + ci);
    }
#pragma unroll
    for (int k = 0; k < KT; ++k)
      if (ok[k]) fma_chunk<kBF16, CW>(acc, wt[k], v[k]);
  } else {
    for (int k = 0; k < K; ++k) {
      const int p = pt[k];
      if ((unsigned)p >= (unsigned)rows) continue;  // a row outside the buffer adds nothing
      fma_chunk<kBF16, CW>(acc, wt[k], __builtin_nontemporal_load(ye + (size_t)p * rc + ci));
    }
  }
  __builtin_nontemporal_store(pack_chunk<kBF16, CW>(acc), y + (size_t)t * rc + ci);
}

// ---- dequantising combine: fp8 e4m3 expert outputs, fp32 scale per 128 -----

typedef float f32x2 __attribute__((ext_vector_type(2)));

// acc[0..7] += ws * (8 e4m3 values of v), ws = w * the chunk's scale; the
// hardware conversion decodes OCP e4m3fn exactly (two bytes per call).
__device__ __forceinline__ void fma_fp8(float* acc, float ws, u32x2 v) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], true);
    acc[4 * i] = fmaf(ws, lo.x, acc[4 * i]);
    acc[4 * i + 1] = fmaf(ws, lo.y, acc[4 * i + 1]);
    acc[4 * i + 2] = fmaf(ws, hi.x, acc[4 * i + 2]);
    acc[4 * i + 3] = fmaf(ws, hi.y, acc[4 * i + 3]);
  }
}

// 8 accumulators to the output row: one 16-byte chunk of bf16 (chunk ci of
// the row) or two of fp32 (chunks 2 ci, 2 ci + 1).
template <bool kBF16>
__device__ __forceinline__ void store_fp8_piece(const float* acc, u32x4* __restrict__ y, size_t ci) {
  if constexpr (kBF16) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
    __builtin_nontemporal_store(o, y + ci);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[4 * j + i]);
      __builtin_nontemporal_store(o, y + 2 * ci + j);
    }
  }
}

// Dequantising combine: y[t][i] = sum_k w[t][k] * e4m3(y_exp[p][i]) *
// scale[p][i/128], accumulated in fp32 in k order as fma(w * scale, value,
// acc). One wave per 512-element part of a token's fp8 row (64 lanes x 8
// elements, each lane's 8 under one scale: chunk c uses scale c / 16), the
// parts of a token on consecutive waves. On MI355X 8 elements per lane ran
// 23 % faster than 16 (96 against 125 us for 8192 tokens x top-8 x 7168) and
// 10 % faster than 4: small waves with few accumulators keep the most loads
// in flight. With a compile-time K the K loads of a part are issued before
// the first FMA.
template <int KT, bool kBF16>
__global__ __launch_bounds__(kCombThreads) void k_combine_fp8(
    const u32x2* __restrict__ ye, const float* __restrict__ ys, const int32_t* __restrict__ pos,
    const float* __restrict__ w, const int32_t* __restrict__ status, u32x4* __restrict__ y,
    int N, int K_, int rc8, int wpt, int rows) {
  const int K = KT ? KT : K_;
  const int nsc = rc8 / 16;  // scales per row
  const int lane = threadIdx.x & 63;
  const int gw = uniform(blockIdx.x * kWavesPerCombBlock + (threadIdx.x >> 6));
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= N) return;
  if (status[0] & MB_ST_FATAL) return;
  const int ci = part * 64 + lane;  // this lane's chunk of the row
  if (ci >= rc8) return;
  const int32_t* pt = pos + (size_t)t * K;
  const float* wt = w + (size_t)t * K;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if constexpr (KT > 0) {
    u32x2 v[KT];
    float s[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int p = pt[k];
      const bool ok = (unsigned)p < (unsigned)rows;  // only a broken plan fails this
      const size_t row = ok ? (size_t)p : 0;
      v[k] = __builtin_nontemporal_load(ye + row * rc8 + ci);
      s[k] = ok ? ys[row * nsc + (ci >> 4)] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) fma_fp8(acc, wt[k] * s[k], v[k]);
  } else {
    for (int k = 0; k < K; ++k) {
      const int p = pt[k];
      if ((unsigned)p >= (unsigned)rows) continue;
      fma_fp8(acc, wt[k] * ys[(size_t)p * nsc + (ci >> 4)],
              __builtin_nontemporal_load(ye + (size_t)p * rc8 + ci));
    }
  }
  store_fp8_piece<kBF16>(acc, y, (size_t)t * rc8 + ci);
}

}  // namespace

hipError_t launch_dispatch(const mb_dims& d, const mb_plan_bufs& o, const void* x,
                           const float* x_scale, void* buf, float* buf_scale, hipStream_t st) {
  if (d.n_tokens == 0) return hipSuccess;
  const int rb16 = (int)(d.hidden * elt_bytes(d.dtype_in) / 16);
  const int nsc = d.dtype_in == MB_FP8_E4M3 ? d.hidden / 128 : 0;
  const int rows = d.n_ranks * d.cap;
  const int wpt = (rb16 + 63) / 64;  // waves per token
  const int64_t waves = (int64_t)d.n_tokens * wpt;
  const dim3 grid((unsigned)((waves + kWavesPerRowBlock - 1) / kWavesPerRowBlock));
  const int vec4 = nsc % 4 == 0 && ((uintptr_t)x_scale & 15u) == 0 && ((uintptr_t)buf_scale & 15u) == 0;
  if (rb16 % kSpanChunks == 0 && d.top_k >= 2 && d.top_k <= 16) {
    if (nsc > 0)
      launch_dispatch_span<true>(d, o, x, x_scale, buf, buf_scale, rb16, rows, nsc, vec4, st);
    else
      launch_dispatch_span<false>(d, o, x, x_scale, buf, buf_scale, rb16, rows, nsc, vec4, st);
    return hipGetLastError();
  }
  MB_DISPATCH_TOPK(d.top_k, k_dispatch, grid, dim3(kRowThreads), 0, st,
                   static_cast<const u32x4*>(x), o.pos, o.status, static_cast<u32x4*>(buf),
                   d.n_tokens, d.top_k, rb16, wpt, rows, x_scale, buf_scale, nsc, vec4);
  return hipGetLastError();
}

template <bool kBF16, int CW>
static void launch_combine_t(const mb_dims& d, const mb_plan_bufs& o, const void* ye,
                             const float* w, void* yy, int rows, hipStream_t st) {
  const int rc = (int)(d.hidden * elt_bytes(d.dtype_out) / (4 * CW));  // chunks per row
  const int wpt = (rc + 63) / 64;                                      // waves per token
  const int64_t waves = (int64_t)d.n_tokens * wpt;
  const dim3 grid((unsigned)((waves + kWavesPerCombBlock - 1) / kWavesPerCombBlock));
  const auto* src = static_cast<const chunk_t<CW>*>(ye);
  auto* dst = static_cast<chunk_t<CW>*>(yy);
#define MB_C(KT)                                                                                 \
  hipLaunchKernelGGL((k_combine<KT, kBF16, CW>), grid, dim3(kCombThreads), 0, st, src, o.pos, w, \
                     o.status, dst, d.n_tokens, d.top_k, rc, wpt, rows)
  switch (d.top_k) {
    case 1: MB_C(1); break;
    case 2: MB_C(2); break;
    case 4: MB_C(4); break;
    case 8: MB_C(8); break;
    default: MB_C(0); break;
  }
#undef MB_C
}

template <bool kBF16>
static void launch_combine_fp8_t(const mb_dims& d, const mb_plan_bufs& o, const u32x2* ye,
                                 const float* ys, const float* w, u32x4* yy, int rc8, int rows,
                                 hipStream_t st) {
  const int wpt = (rc8 + 63) / 64;  // waves per token
  const int64_t waves = (int64_t)d.n_tokens * wpt;
  const dim3 grid((unsigned)((waves + kWavesPerCombBlock - 1) / kWavesPerCombBlock));
#define MB_C(KT)                                                                             \
  hipLaunchKernelGGL((k_combine_fp8<KT, kBF16>), grid, dim3(kCombThreads), 0, st, ye, ys, o.pos, \
                     w, o.status, yy, d.n_tokens, d.top_k, rc8, wpt, rows)
  switch (d.top_k) {
    case 1: MB_C(1); break;
    case 2: MB_C(2); break;
    case 4: MB_C(4); break;
    case 8: MB_C(8); break;
    default: MB_C(0); break;
  }
#undef MB_C
}

hipError_t launch_combine_fp8(const mb_dims& d, const mb_plan_bufs& o, const void* y_exp,
                              const float* y_scale, const float* w, void* y, hipStream_t st) {
  if (d.n_tokens == 0) return hipSuccess;
  const int rc8 = d.hidden / 8;  // 8 fp8 elements per chunk
  const int rows = d.n_ranks * d.cap;
  const u32x2* ye = static_cast<const u32x2*>(y_exp);
  u32x4* yy = static_cast<u32x4*>(y);
  if (d.dtype_out == MB_BF16)
    launch_combine_fp8_t<true>(d, o, ye, y_scale, w, yy, rc8, rows, st);
  else
    launch_combine_fp8_t<false>(d, o, ye, y_scale, w, yy, rc8, rows, st);
  return hipGetLastError();
}

hipError_t launch_combine(const mb_dims& d, const mb_plan_bufs& o, const void* y_exp,
                          const float* w, void* y, hipStream_t st) {
  if (d.n_tokens == 0) return hipSuccess;
  const int rows = d.n_ranks * d.cap;
  // 16-byte lane chunks for K <= 2, 8-byte chunks for more rows per token
  const bool wide = d.top_k <= 2;
  if (d.dtype_out == MB_BF16) {
    if (wide)
      launch_combine_t<true, 4>(d, o, y_exp, w, y, rows, st);
    else
      launch_combine_t<true, 2>(d, o, y_exp, w, y, rows, st);
  } else {
    if (wide)
      launch_combine_t<false, 4>(d, o, y_exp, w, y, rows, st);
    else
      launch_combine_t<false, 2>(d, o, y_exp, w, y, rows, st);
  }
  return hipGetLastError();
}

}  // namespace mb
