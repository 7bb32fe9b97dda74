// api.hip — libmoebal's C ABI: argument checks, workspace layout, launches.
// The operations and conventions are documented in include/moebal.h.
#include <string.h>

#include <mutex>

#include "mb_internal.h"

namespace mb {

Geometry geometry(const mb_dims& d) {
  Geometry g;
  g.S = d.n_tokens / d.n_ranks;
  g.Eh = d.n_experts / d.n_ranks;
  g.NS = g.Eh + d.slots_per_rank;
  g.nbps = (g.S + kTokensPerBlock - 1) / kTokensPerBlock;
  g.nblk = g.nbps * d.n_ranks;
  return g;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t drift_state_bytes(const mb_dims& d) {
  const size_t PR = (size_t)d.n_ranks * d.slots_per_rank;
  return align256(sizeof(mb_drift_header) + sizeof(int64_t) * d.n_experts +
                  2 * sizeof(int32_t) * PR);
}

WsLayout ws_layout(const mb_dims& d, const Geometry& g) {
  WsLayout L;
  size_t off = 0;
  const size_t per_block = (size_t)g.nblk * d.n_experts * sizeof(int32_t);
  L.blockcnt = off;
  off = align256(off + per_block);
  L.blockoff = off;
  off = align256(off + per_block);
  L.blockflags = off;
  off = align256(off + (size_t)g.nblk * sizeof(int32_t) + sizeof(int32_t));
  L.brank = off;
  off = align256(off + (size_t)d.n_tokens * d.top_k);
  L.expert_total = off;
  off = align256(off + (size_t)d.n_experts * sizeof(int32_t));
  L.pair_tab = off;
  off = align256(off + (size_t)d.n_ranks * d.n_experts * sizeof(PairEntry));
  L.host_list = off;
  off = align256(off + (size_t)host_list_cap(d) * sizeof(HostEntry));
  L.host_range = off;
  off = align256(off + (size_t)d.n_experts * sizeof(int2));
  L.total = off;
  return L;
}

}  // namespace mb

using namespace mb;

static int validate(const mb_dims* d) {
  if (!d) return MB_ERR_INVALID_ARG;
  if (d->n_ranks < 1 || d->n_ranks > kMaxRanks) return MB_ERR_INVALID_ARG;
  if (d->n_tokens < 0 || d->n_tokens % d->n_ranks) return MB_ERR_INVALID_ARG;
  if (d->n_experts < 1 || d->n_experts > kMaxExperts || d->n_experts % d->n_ranks)
    return MB_ERR_INVALID_ARG;
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > kMaxTopK) return MB_ERR_INVALID_ARG;
  if (d->slots_per_rank < 0 || d->slots_per_rank > kMaxSlots) return MB_ERR_INVALID_ARG;
  if (d->hidden < 1 || d->cap < 1) return MB_ERR_INVALID_ARG;
  if ((int64_t)d->n_tokens * d->top_k > INT32_MAX) return MB_ERR_INVALID_ARG;
  if ((int64_t)d->n_ranks * d->cap > INT32_MAX) return MB_ERR_INVALID_ARG;
  const int64_t bin = elt_bytes(d->dtype_in);
  if (!bin) return MB_ERR_INVALID_ARG;
  if (d->dtype_out != MB_F32 && d->dtype_out != MB_BF16) return MB_ERR_INVALID_ARG;
  if ((int64_t)d->hidden * bin % 16 || (int64_t)d->hidden * elt_bytes(d->dtype_out) % 16)
    return MB_ERR_INVALID_ARG;
  if ((int64_t)d->hidden * bin / 16 > INT32_MAX) return MB_ERR_INVALID_ARG;
  // dispatch runs one wave per 1 KiB part of every token row, the combines
  // one per 512 bytes of output row (at least as many as per 512 fp8
  // elements of an expert row, which the fp8 combine uses)
  if ((int64_t)d->n_tokens * (((int64_t)d->hidden * bin / 16 + 63) / 64) > INT32_MAX)
    return MB_ERR_INVALID_ARG;
  if ((int64_t)d->n_tokens * (((int64_t)d->hidden * elt_bytes(d->dtype_out) / 8 + 63) / 64) >
      INT32_MAX)
    return MB_ERR_INVALID_ARG;
  if (d->dtype_in == MB_FP8_E4M3 && d->hidden % 128) return MB_ERR_INVALID_ARG;
  return MB_OK;
}

// pos may be NULL only when there are no pairs (N == 0).
static bool plan_ptrs_ok(const mb_dims* d, const mb_plan_bufs* o) {
  return o && o->counts && o->load_pre && o->load_post && o->slot_quota && o->cu_seqlens &&
         (o->pos || d->n_tokens == 0) && o->row_src && o->status;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" {

int mb_version(void) { return MB_VERSION; }

const char* mb_strerror(int code) {
  switch (code) {
    case MB_OK: return "ok";
    case MB_ERR_INVALID_ARG: return "invalid argument (sizes outside the limits or null pointer)";
    case MB_ERR_WORKSPACE: return "workspace smaller than mb_plan_workspace_bytes()";
    case MB_ERR_HIP: return "HIP runtime error";
    case MB_ST_BAD_ID: return "status: an expert id outside [0, E)";
    case MB_ST_DUP_ID: return "status: a token lists one expert twice";
    case MB_ST_UNBALANCED: return "status: placement stopped with a rank above its target";
    case MB_ST_CAPACITY: return "status: a rank needs more rows than cap";
    default: return "unknown code";
  }
}

size_t mb_plan_workspace_bytes(const mb_dims* dims) {
  if (validate(dims) != MB_OK) return 0;
  const Geometry g = geometry(*dims);
  return ws_layout(*dims, g).total;
}

static int plan_impl(const mb_dims* dims, const int32_t* ids_dev, const int32_t* rank_speed,
                     const mb_drift_params* drift, void* drift_state, int repair, void* ws_dev,
                     size_t ws_bytes, const mb_plan_bufs* out, hipStream_t stream) {
  int rc = validate(dims);
  if (rc != MB_OK) return rc;
  if (!plan_ptrs_ok(dims, out) || !ws_dev || (dims->n_tokens > 0 && !ids_dev) ||
      (dims->slots_per_rank > 0 && !out->rep_expert) || !aligned16(ws_dev))
    return MB_ERR_INVALID_ARG;
  for (int r = 0; r < dims->n_ranks; ++r)
    if (rank_speed[r] < 1 || rank_speed[r] > MB_MAX_SPEED) return MB_ERR_INVALID_ARG;
  const Geometry g = geometry(*dims);
  const WsLayout L = ws_layout(*dims, g);
  if (ws_bytes < L.total) return MB_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  int32_t* blockcnt = reinterpret_cast<int32_t*>(ws + L.blockcnt);
  int32_t* blockoff = reinterpret_cast<int32_t*>(ws + L.blockoff);
  int32_t* blockflags = reinterpret_cast<int32_t*>(ws + L.blockflags);
  PairEntry* pair_tab = reinterpret_cast<PairEntry*>(ws + L.pair_tab);
  HostEntry* host_list = reinterpret_cast<HostEntry*>(ws + L.host_list);
  int2* host_range = reinterpret_cast<int2*>(ws + L.host_range);
  int32_t* expert_total = reinterpret_cast<int32_t*>(ws + L.expert_total);
  uint8_t* brank = ws + L.brank;

  // count -> per-source offsets and totals -> greedy placement -> lookup
  // tables -> per-pair rows, all on `stream`, no host synchronisation.
  // With one routing block per source rank, the block counts are d[s][e]
  // and every block offset is 0: k_count writes d itself, the scan is
  // skipped and k_plan sums c_e. With a few blocks per source and a small
  // table of block counts, the scan is skipped too: k_plan sums the table
  // into d[s][e] and c_e, and each k_assign block sums its source's earlier
  // blocks.
  const bool one_block = g.nbps == 1;
  const bool small = small_block_table(*dims, g);
  const bool scan = !one_block && !small;
  const bool tables_in_plan = dims->n_experts <= kPlanTableExperts;
  if (launch_count(*dims, g, ids_dev, one_block ? out->counts : blockcnt, blockflags, brank,
                   stream) != hipSuccess)
    return MB_ERR_HIP;
  if (scan &&
      launch_scan(*dims, g, blockcnt, blockoff, out->counts, expert_total, stream) != hipSuccess)
    return MB_ERR_HIP;
  if (launch_plan(*dims, g, *out, rank_speed, drift, drift_state, repair, blockflags,
                  scan ? expert_total : nullptr, small ? blockcnt : nullptr,
                  tables_in_plan ? pair_tab : nullptr, tables_in_plan ? host_list : nullptr,
                  tables_in_plan ? host_range : nullptr, stream) != hipSuccess)
    return MB_ERR_HIP;
  if (!tables_in_plan &&
      launch_tables(*dims, g, *out, pair_tab, host_list, host_range, stream) != hipSuccess)
    return MB_ERR_HIP;
  if (launch_assign(*dims, g, ids_dev, brank, scan ? blockoff : nullptr,
                    small ? blockcnt : nullptr, pair_tab, host_list, host_range, *out,
                    stream) != hipSuccess)
    return MB_ERR_HIP;
  return MB_OK;
}

int mb_plan(const mb_dims* dims, const int32_t* ids_dev, void* ws_dev, size_t ws_bytes,
            const mb_plan_bufs* out, hipStream_t stream) {
  // Equal speeds: every target is the water level T = ceil(N*K / P)
  // (ISER-MoE, HALO-Q Objective 1).
  int32_t ones[kMaxRanks];
  for (int r = 0; r < kMaxRanks; ++r) ones[r] = 1;
  return plan_impl(dims, ids_dev, ones, nullptr, nullptr, 0, ws_dev, ws_bytes, out, stream);
}

// ---- mb_plan_noalloc: mb_plan on a workspace the library holds ----------
//
// Every GPU the library runs on holds its own copy of `scratch`, at its own
// address, until the process ends. In host code the array's name is only a
// host-side stand-in: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// handed to kernels.
static __device__ __align__(256) uint8_t scratch[MB_NOALLOC_WS_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[kMaxDevices];

// Device address of `scratch` on the GPU that `stream` belongs to.
static int scratch_for(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MB_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MB_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MB_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MB_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MB_ERR_HIP;
    if (e != hipSuccess || !p) return MB_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MB_OK;
}

int mb_plan_noalloc(const mb_dims* dims, const int32_t* ids_dev, const mb_plan_bufs* out,
                    hipStream_t stream) {
  const int rc = validate(dims);
  if (rc != MB_OK) return rc;
  const size_t need = ws_layout(*dims, geometry(*dims)).total;
  if (need > MB_NOALLOC_WS_BYTES) return MB_ERR_WORKSPACE;
  void* ws = nullptr;
  const int src = scratch_for(stream, &ws);
  if (src != MB_OK) return src;
  int32_t ones[kMaxRanks];
  for (int r = 0; r < kMaxRanks; ++r) ones[r] = 1;
  return plan_impl(dims, ids_dev, ones, nullptr, nullptr, 0, ws, MB_NOALLOC_WS_BYTES, out,
                   stream);
}

int mb_plan_weighted(const mb_dims* dims, const int32_t* ids_dev, const int32_t* rank_speed,
                     void* ws_dev, size_t ws_bytes, const mb_plan_bufs* out,
                     hipStream_t stream) {
  if (!rank_speed) return MB_ERR_INVALID_ARG;
  return plan_impl(dims, ids_dev, rank_speed, nullptr, nullptr, 0, ws_dev, ws_bytes, out,
                   stream);
}

size_t mb_drift_state_bytes(const mb_dims* dims) {
  if (validate(dims) != MB_OK) return 0;
  return drift_state_bytes(*dims);
}

int mb_plan_ex(const mb_dims* dims, const int32_t* ids_dev, const mb_plan_options* opt,
               void* ws_dev, size_t ws_bytes, const mb_plan_bufs* out, hipStream_t stream) {
  if (!opt) return MB_ERR_INVALID_ARG;
  const mb_drift_params* prm = opt->drift;
  if ((prm != nullptr) != (opt->drift_state != nullptr)) return MB_ERR_INVALID_ARG;
  if (prm) {
    if (!aligned16(opt->drift_state)) return MB_ERR_INVALID_ARG;
    if (prm->delta_den < 1 || prm->delta_num < 0 || prm->delta_num > prm->delta_den ||
        prm->window < 1 || prm->window > MB_MAX_WINDOW || prm->check_every < 1 ||
        prm->tol_num < 0 || prm->tol_den < 0)
      return MB_ERR_INVALID_ARG;
  }
  int32_t ones[kMaxRanks];
  for (int r = 0; r < kMaxRanks; ++r) ones[r] = 1;
  return plan_impl(dims, ids_dev, opt->rank_speed ? opt->rank_speed : ones, prm,
                   opt->drift_state, opt->quota_repair != 0, ws_dev, ws_bytes, out, stream);
}

int mb_plan_drift(const mb_dims* dims, const int32_t* ids_dev, const int32_t* rank_speed,
                  const mb_drift_params* params, void* state_dev, void* ws_dev,
                  size_t ws_bytes, const mb_plan_bufs* out, hipStream_t stream) {
  if (!params || !state_dev) return MB_ERR_INVALID_ARG;
  const mb_plan_options opt = {rank_speed, params, state_dev, 0};
  return mb_plan_ex(dims, ids_dev, &opt, ws_dev, ws_bytes, out, stream);
}

int mb_dispatch(const mb_dims* dims, const mb_plan_bufs* plan, const void* x_dev,
                const float* x_scale_dev, void* buf_dev, float* buf_scale_dev,
                hipStream_t stream) {
  int rc = validate(dims);
  if (rc != MB_OK) return rc;
  if (!plan || (dims->n_tokens > 0 && (!plan->pos || !x_dev)) || !plan->status || !buf_dev)
    return MB_ERR_INVALID_ARG;
  if (!aligned16(x_dev) || !aligned16(buf_dev)) return MB_ERR_INVALID_ARG;
  if (dims->dtype_in == MB_FP8_E4M3 && (!x_scale_dev || !buf_scale_dev)) return MB_ERR_INVALID_ARG;
  return launch_dispatch(*dims, *plan, x_dev, x_scale_dev, buf_dev, buf_scale_dev, stream) ==
                 hipSuccess
             ? MB_OK
             : MB_ERR_HIP;
}

int mb_combine(const mb_dims* dims, const mb_plan_bufs* plan, const void* y_exp_dev,
               const float* w_dev, void* y_dev, hipStream_t stream) {
  int rc = validate(dims);
  if (rc != MB_OK) return rc;
  if (!plan || !plan->status || !y_exp_dev ||
      (dims->n_tokens > 0 && (!plan->pos || !w_dev || !y_dev)))
    return MB_ERR_INVALID_ARG;
  if (!aligned16(y_exp_dev) || !aligned16(y_dev)) return MB_ERR_INVALID_ARG;
  return launch_combine(*dims, *plan, y_exp_dev, w_dev, y_dev, stream) == hipSuccess ? MB_OK
                                                                                     : MB_ERR_HIP;
}

int mb_combine_fp8(const mb_dims* dims, const mb_plan_bufs* plan, const uint8_t* y_exp_dev,
                   const float* y_scale_dev, const float* w_dev, void* y_dev,
                   hipStream_t stream) {
  int rc = validate(dims);
  if (rc != MB_OK) return rc;
  if (dims->hidden % 128) return MB_ERR_INVALID_ARG;
  if (!plan || !plan->status || !y_exp_dev || !y_scale_dev ||
      (dims->n_tokens > 0 && (!plan->pos || !w_dev || !y_dev)))
    return MB_ERR_INVALID_ARG;
  if (!aligned16(y_exp_dev) || !aligned16(y_dev) || ((uintptr_t)y_scale_dev & 3u))
    return MB_ERR_INVALID_ARG;
  return launch_combine_fp8(*dims, *plan, y_exp_dev, y_scale_dev, w_dev, y_dev, stream) ==
                 hipSuccess
             ? MB_OK
             : MB_ERR_HIP;
}

int mb_plan_status(const mb_plan_bufs* plan, hipStream_t stream, int32_t host_status[4]) {
  if (!plan || !plan->status || !host_status) return MB_ERR_INVALID_ARG;
  if (hipMemcpyAsync(host_status, plan->status, 4 * sizeof(int32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return MB_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MB_ERR_HIP;
  return MB_OK;
}

}  // extern "C"
