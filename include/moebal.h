/*
 * moebal.h — C ABI of libmoebal: per-invocation hot-expert replication and
 * token dispatch/combine for expert-parallel MoE layers on AMD MI355X
 * (gfx950).
 *
 * One MoE layer call goes through three asynchronous steps on one HIP stream:
 *
 *   mb_plan      count routed pairs, replicate the heaviest experts of the
 *                busiest ranks into free replica slots until every rank is at
 *                or below the water level T, assign pairs to replicas
 *                local-first, and lay out fixed-shape per-rank regions
 *                (cu_seqlens, a dispatch row per pair, the token of each row);
 *   mb_dispatch  copy every token row to its K dispatch rows;
 *   mb_combine   weighted gather-reduce of the K expert-output rows of each
 *                token back into token order.
 *
 * The P logical ranks of the expert-parallel group are partitions of one
 * GPU's memory: rank r owns rows [r*cap, (r+1)*cap) of every [P*cap, ...]
 * buffer.
 *
 * Sources (pages, by title and section):
 *  [ISER]   "ISER-MoE: Dynamic In-Switch Replication of Hot Experts for Load
 *           Balancing in Expert-Parallel", Methodology, HALO-Q Scheduler
 *           (Objectives 1-2, stages 1-3 and 5); Background (imbalance ratio).
 *  [Zepp]   Zepp summary (picx.dev/p/sh48ti), §4.1 (R replica slots per GPU;
 *           eq. (1) locality-preferred routing).
 *  [MoonEP] "MoonEP: Planner-Enforced S×K Token Balance and Zero-Copy Buffers
 *           to Fix MoE Skew", "What MoonEP enforces and how" (S*K per rank,
 *           planner-made cu_seqlens, fixed-shape expert-grouped buffers,
 *           no host synchronisation) and "Implementation details"
 *           (home experts then prefetch slots in one numbering).
 *  [ViBE]   ViBE summary (picx.dev/p/p7vJoN), Methodology, Variability-
 *           Informed Expert Placement (token targets in proportion to GPU
 *           speed; experts go to the GPU farthest below its target).
 *
 * Conventions
 *  - Every buffer is owned by the caller and lives in device memory unless
 *    stated otherwise. The library never allocates or frees memory and keeps
 *    no state between calls; all calls except mb_plan_status only enqueue
 *    work on `stream` and return without waiting. Calls on different streams
 *    with disjoint buffers may run concurrently. Since they neither allocate
 *    nor synchronise, mb_plan*, mb_dispatch and mb_combine* can be captured
 *    in a HIP graph and replayed (a drift state then advances per replay).
 *  - All integers are int32, all arrays row-major and densely packed.
 *  - Host-detectable errors (bad sizes, null pointers, misaligned rows, a
 *    workspace that is too small) return a negative MB_ERR_* code and enqueue
 *    nothing. MB_ERR_HIP means a HIP launch failed.
 *  - Data-dependent problems are reported by mb_plan in status[0] on the
 *    device (MB_ST_* bits). mb_dispatch and mb_combine read that word on the
 *    device and do nothing when a fatal bit (MB_ST_FATAL) is set, so a bad
 *    plan never writes out of bounds. When a fatal bit is set, the plan's
 *    pos and row_src contents are unspecified. With MB_ST_BAD_ID or
 *    MB_ST_DUP_ID there is no plan: counts, load_pre, load_post, slot_quota
 *    and cu_seqlens are all 0, every rep_expert entry is -1, and status is
 *    {flags, T, 0, 0}. With MB_ST_CAPACITY alone every output but pos and
 *    row_src holds the plan that did not fit.
 *
 * Limits: 1 <= P <= 64, E % P == 0, E <= 1024, 1 <= K <= min(E, 32),
 * 0 <= R <= 16, N % P == 0, N*K < 2^31, P*cap < 2^31, row bytes a multiple
 * of 16; fp8 rows need H % 128 == 0. rep_expert may be NULL when R == 0.
 */
#ifndef MOEBAL_H
#define MOEBAL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MB_VERSION 2

/* Element types of rows. */
enum mb_dtype {
  MB_F32 = 0,       /* IEEE binary32 */
  MB_BF16 = 1,      /* bfloat16 */
  MB_FP8_E4M3 = 2   /* OCP fp8 e4m3fn, one fp32 scale per 128 elements */
};

/* Return codes. */
enum mb_error {
  MB_OK = 0,
  MB_ERR_INVALID_ARG = -1, /* sizes outside the limits, null pointer, ... */
  MB_ERR_WORKSPACE = -2,   /* ws_bytes < mb_plan_workspace_bytes(dims) */
  MB_ERR_HIP = -3          /* a HIP runtime call failed */
};

/* status[0] bits written by mb_plan. */
enum mb_status_flag {
  MB_ST_BAD_ID = 1,     /* an id outside [0, E) (fatal) */
  MB_ST_DUP_ID = 2,     /* a token lists one expert twice (fatal) */
  MB_ST_UNBALANCED = 4, /* placement stopped with a rank above its target (not fatal) */
  MB_ST_CAPACITY = 8    /* a rank needs more than cap rows (fatal) */
};
#define MB_ST_FATAL (MB_ST_BAD_ID | MB_ST_DUP_ID | MB_ST_CAPACITY)

/* Largest rank speed accepted by mb_plan_weighted. */
#define MB_MAX_SPEED (1 << 20)

/* status[0] bit of mb_plan_drift: this call ran the greedy placement
 * (informational, never fatal). */
#define MB_ST_REPLANNED 16
/* status[0] bit of mb_plan_drift, set with MB_ST_REPLANNED: the gate kept
 * the placement, but its replay on this call's counts failed the load guard,
 * so the greedy ran in the same call (informational). */
#define MB_ST_GUARDED 32

/* Largest reference window of mb_plan_drift, in calls. */
#define MB_MAX_WINDOW 4096

/* Drift gate of mb_plan_drift [ViBE, Drift-Aware Recalibration]. */
typedef struct mb_drift_params {
  int32_t delta_num;   /* replan when d > delta_num / delta_den, where  */
  int32_t delta_den;   /*   d = 1 - cos(current counts, reference)      */
  int32_t window;      /* reference = count vectors of up to `window` calls
                          since the last replan, in [1, MB_MAX_WINDOW] */
  int32_t check_every; /* calls between two checks (>= 1) */
  int32_t tol_num;     /* load guard: a kept placement stands only if no   */
  int32_t tol_den;     /*   rank needs more than cap rows and, when tol_den
                          > 0, none ends above (1 + tol_num / tol_den) times
                          its target; both >= 0 (0, 0: cap only) */
} mb_drift_params;

/* First bytes of a drift state buffer (device memory, caller-owned); the
 * rest holds the reference sum int64[E], then the kept placement: replica
 * experts int32[P*R] and their slots in placement order int32[P*R]. A
 * zero-filled buffer is a fresh state. */
typedef struct mb_drift_header {
  int32_t have_plan;  /* a placement is kept */
  int32_t countdown;  /* calls until the next check */
  int32_t nwin;       /* count vectors in the reference */
  int32_t n_moves;    /* replicas of the kept placement */
  int64_t calls;      /* calls planned with this state */
  int64_t replans;    /* of which ran the greedy */
  double last_d;      /* distance found at the last check */
  int64_t guarded;    /* replans forced by the load guard */
  int64_t reserved[2];
} mb_drift_header;

/* Problem sizes of one MoE layer call. */
typedef struct mb_dims {
  int32_t n_tokens;       /* N tokens; token t originates on rank t / (N/P) */
  int32_t top_k;          /* K experts per token, distinct within a token */
  int32_t n_experts;      /* E experts; expert e is homed on rank e / (E/P) */
  int32_t n_ranks;        /* P logical ranks */
  int32_t slots_per_rank; /* R replica slots per rank */
  int32_t hidden;         /* H elements per row */
  int32_t cap;            /* rows per rank region; S*K = the water level T */
  int32_t dtype_in;       /* token rows x and dispatch buffer (mb_dtype) */
  int32_t dtype_out;      /* expert outputs and combined rows: F32 or BF16 */
} mb_dims;

/*
 * Caller-owned device outputs of mb_plan (Eh = E/P, NS = Eh + R):
 *   counts[P*E]         d[s][e] = pairs from source rank s to expert e
 *   load_pre[P]         L_r = pairs whose expert is homed on r
 *   load_post[P]        rows rank r serves after planning
 *   rep_expert[P*R]     expert held by replica slot j of rank r, -1 if empty
 *   slot_quota[P*NS]    rows of local slot i of rank r: i < Eh is home expert
 *                       r*Eh + i, i >= Eh is replica slot i - Eh
 *   cu_seqlens[P*(NS+1)] per-rank running row offsets of the local slots,
 *                       relative to the rank's region (cu[r][0] = 0)
 *   pos[N*K]            dispatch row of pair (t, k), in [0, P*cap) (may be
 *                       NULL when N == 0)
 *   row_src[P*cap]      token of each dispatch row, -1 for padding rows
 *   status[4]           {flags (mb_status_flag), T, max_r load_post, moves};
 *                       from mb_plan_weighted, T is the largest target tau_r
 */
typedef struct mb_plan_bufs {
  int32_t* counts;
  int32_t* load_pre;
  int32_t* load_post;
  int32_t* rep_expert;
  int32_t* slot_quota;
  int32_t* cu_seqlens;
  int32_t* pos;
  int32_t* row_src;
  int32_t* status;
} mb_plan_bufs;

/* Library version (MB_VERSION). */
int mb_version(void);

/* Short description of an mb_error code or of one mb_status_flag bit
 * (pass the flag as a positive value). Never NULL; static storage. */
const char* mb_strerror(int code);

/* Bytes of device workspace mb_plan needs for these sizes; 0 for sizes
 * outside the limits. Pure host function. */
size_t mb_plan_workspace_bytes(const mb_dims* dims);

/*
 * Plan one MoE layer call [ISER HALO-Q stages 1-3, 5; Zepp §4.1; MoonEP].
 *  ids_dev   [N*K] int32 expert ids, device.
 *  ws_dev    device workspace of at least mb_plan_workspace_bytes(dims)
 *            bytes, 16-byte aligned; contents need no initialisation and are
 *            scratch after the call.
 *  out       device pointers of the outputs (struct itself is host memory,
 *            read during the call only).
 * The greedy: while the busiest rank (lowest index on ties) is above
 * T = ceil(N*K/P), take its home expert with the largest remaining home
 * quota (lowest id on ties) that has an eligible destination: a rank with a
 * free replica slot, load below T, not yet holding that expert; the least
 * loaded such rank (lowest index on ties) gets a replica in its lowest free
 * slot and min(T - its load, remaining home quota) pairs. Placement stops
 * when every rank is at or below T, or with MB_ST_UNBALANCED when the
 * busiest rank has no expert with a destination. Pairs are then assigned in
 * (t, k) order: to the source rank when it holds the expert and has quota
 * left, otherwise to the lowest-index holder with quota left; rows of a
 * slot are in ascending token order.
 * Returns MB_OK once the work is enqueued.
 */
int mb_plan(const mb_dims* dims, const int32_t* ids_dev, void* ws_dev, size_t ws_bytes,
            const mb_plan_bufs* out, hipStream_t stream);

/* Largest workspace mb_plan_noalloc can use: 4 MiB per GPU. */
#define MB_NOALLOC_WS_BYTES (4u << 20)

/*
 * mb_plan for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plan as mb_plan, with the workspace taken from an array the
 * library holds in device memory, one per GPU (MB_NOALLOC_WS_BYTES bytes,
 * kept until the process ends). The call allocates and frees nothing.
 *  ids_dev, out, stream  as in mb_plan; the GPU is the one `stream` runs on.
 * Returns MB_ERR_WORKSPACE, enqueueing nothing, when these sizes need more
 * than MB_NOALLOC_WS_BYTES (mb_plan_workspace_bytes(dims) tells), and
 * MB_ERR_HIP if the array's device address cannot be obtained (the first
 * call on each GPU looks it up). Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: two calls whose work
 * overlaps in time on one GPU (on different streams, or from different
 * threads without ordering) race and may both produce wrong plans.
 */
int mb_plan_noalloc(const mb_dims* dims, const int32_t* ids_dev, const mb_plan_bufs* out,
                    hipStream_t stream);

/*
 * mb_plan with per-rank targets in place of the single water level [ViBE,
 * Variability-Informed Expert Placement]: rank r of speed s_r aims at
 *   tau_r = ceil(N*K * s_r / sum_h s_h)
 * rows. The busiest rank is the one farthest above its target (largest
 * load - tau), a move's destination the eligible rank farthest below its
 * own (largest tau - load), and a move gives min(tau_dst - load_dst,
 * remaining home quota) pairs; everything else is as in mb_plan, which is
 * this call with equal speeds.
 *  rank_speed  [P] int32 HOST array, each in [1, MB_MAX_SPEED] (relative
 *              throughput, e.g. the inverse of a rank's measured latency at
 *              a reference load, scaled to integers); read during the call
 *              only. NULL or a value out of range -> MB_ERR_INVALID_ARG.
 * Fast ranks' targets exceed N*K/P: size cap to at least the largest
 * target, or the plan reports MB_ST_CAPACITY.
 */
int mb_plan_weighted(const mb_dims* dims, const int32_t* ids_dev, const int32_t* rank_speed,
                     void* ws_dev, size_t ws_bytes, const mb_plan_bufs* out,
                     hipStream_t stream);

/* Bytes of a drift state buffer for these sizes (0 outside the limits).
 * Pure host function. */
size_t mb_drift_state_bytes(const mb_dims* dims);

/*
 * One call of a layer planned with drift-gated replanning [ViBE, Drift-Aware
 * Recalibration], on `state` (mb_drift_state_bytes(dims) bytes of device
 * memory, 16-byte aligned, zero-filled before the layer's first call, then
 * passed to every call of that layer with the same dims and params; calls
 * on one state must be ordered on one stream).
 * On the first call, and when a check finds d > delta (checks run every
 * check_every calls), the greedy of mb_plan (or of mb_plan_weighted when
 * rank_speed, a P-entry host array, is not NULL) places replicas; the
 * placement is kept in the state, the reference restarts from this call's
 * counts, and status[0] gets MB_ST_REPLANNED. Otherwise the kept replicas,
 * in the order they were placed, each take min(target - host load,
 * remaining home quota) pairs while the expert's home rank is above its
 * target and the host below its own (none otherwise), and this call's counts
 * join the reference while it holds fewer than `window` vectors. Load guard
 * [ViBE, Incremental placement update: done once every GPU is within the
 * tolerance epsilon]: when that replay leaves a rank with more than cap
 * rows, or (tol_den > 0) with load * tol_den > target * (tol_den + tol_num),
 * the greedy runs in the same call as on a replan and status[0] gets
 * MB_ST_REPLANNED | MB_ST_GUARDED. A plan with a rank above its target is
 * MB_ST_UNBALANCED either way.
 * d = 1 - r.c / (|r| |c|) over the expert counts c and the reference sum r,
 * with exact integer sums, then one division and two square roots in
 * double. A call with BAD_ID or DUP_ID leaves the state unchanged.
 * Outputs and everything else as mb_plan.
 */
int mb_plan_drift(const mb_dims* dims, const int32_t* ids_dev, const int32_t* rank_speed,
                  const mb_drift_params* params, void* state_dev, void* ws_dev,
                  size_t ws_bytes, const mb_plan_bufs* out, hipStream_t stream);

/* Options of mb_plan_ex; a zero-filled struct gives mb_plan. */
typedef struct mb_plan_options {
  const int32_t* rank_speed;   /* [P] host speeds as in mb_plan_weighted, or NULL (equal) */
  const mb_drift_params* drift; /* drift gate as in mb_plan_drift, or NULL */
  void* drift_state;           /* its device state; NULL exactly when drift is NULL */
  int32_t quota_repair;        /* non-zero: quota repair between placement and routing */
} mb_plan_options;

/*
 * mb_plan with any of rank speeds, the drift gate and the quota repair
 * [ISER HALO-Q stage 4: a circle-method tournament over disjoint rank pairs
 * cancels opposite token flows]. The repair runs after the placement (fresh
 * or kept): n = P rounded up to even players, n - 1 rounds; in round r,
 * player 0 stays at position 0, player 1 + (p - 1 + r) mod (n - 1) sits at
 * position p >= 1, and positions k and n-1-k meet (player P is a bye). For
 * a pair a < b, over the experts both hold (a's replica slots in order whose
 * expert b also holds, then b's replica slots in order whose expert is
 * homed on a), with d the rank's own pairs of the expert and Q its quota,
 * x_ab = min((d_a - Q_a)^+, (Q_b - d_b)^+) and x_ba = min((d_b - Q_b)^+,
 * (Q_a - d_a)^+); m = min(sum x_ab, sum x_ba) units of quota move from b to
 * a over the x_ab experts and from a to b over the x_ba experts, in that
 * order, each taking at most its own x. Rank loads and expert totals are
 * unchanged and 2m more pairs are served where they originate.
 * Error behaviour as mb_plan, mb_plan_weighted and mb_plan_drift; drift and
 * drift_state must be both set or both NULL.
 */
int mb_plan_ex(const mb_dims* dims, const int32_t* ids_dev, const mb_plan_options* opt,
               void* ws_dev, size_t ws_bytes, const mb_plan_bufs* out, hipStream_t stream);

/*
 * Dispatch [MoonEP, "What MoonEP enforces and how": tokens written into
 * fixed-shape expert-grouped buffers]: buf[pos[t][k]] = x[t] for every pair.
 *  x_dev          [N, H] rows of dtype_in.
 *  x_scale_dev    [N, H/128] fp32 scales for MB_FP8_E4M3 rows, else NULL.
 *  buf_dev        [P*cap, H] rows of dtype_in; padding rows are not written.
 *  buf_scale_dev  [P*cap, H/128] fp32 for MB_FP8_E4M3, else NULL.
 * Reads plan->pos and plan->status. Row pointers must be 16-byte aligned.
 */
int mb_dispatch(const mb_dims* dims, const mb_plan_bufs* plan, const void* x_dev,
                const float* x_scale_dev, void* buf_dev, float* buf_scale_dev,
                hipStream_t stream);

/*
 * Combine [Zepp §4.2, Merge: the combine step aggregates a token's expert
 * outputs; MoonEP fixed buffers]:
 *   y[t][i] = sum_{k=0..K-1} w[t][k] * y_exp[pos[t][k]][i]
 * accumulated in fp32 in k order, stored as dtype_out (bf16: round to
 * nearest even).
 *  y_exp_dev  [P*cap, H] expert outputs of dtype_out (the dispatch layout).
 *  w_dev      [N*K] fp32 gate weights.
 *  y_dev      [N, H] of dtype_out.
 * Reads plan->pos and plan->status. Row pointers must be 16-byte aligned.
 */
int mb_combine(const mb_dims* dims, const mb_plan_bufs* plan, const void* y_exp_dev,
               const float* w_dev, void* y_dev, hipStream_t stream);

/*
 * Dequantising combine for fp8 expert outputs [MoonEP fixed buffers; the
 * fp8 payload format of the dispatch]:
 *   y[t][i] = sum_k w[t][k] * e4m3(y_exp[p][i]) * y_scale[p][i / 128],
 *   p = pos[t][k],
 * accumulated in fp32 in k order as fma(w * scale, value, acc), stored as
 * dtype_out (F32, or BF16 by round to nearest even). dtype_in is not used.
 *  y_exp_dev    [P*cap, H] OCP fp8 e4m3fn expert outputs (the dispatch layout).
 *  y_scale_dev  [P*cap, H/128] fp32 scales, one per 128 elements.
 *  w_dev        [N*K] fp32 gate weights.
 *  y_dev        [N, H] of dtype_out.
 * Needs H % 128 == 0; y_exp and y 16-byte aligned, y_scale 4-byte aligned.
 * Reads plan->pos and plan->status; does nothing under a fatal status.
 */
int mb_combine_fp8(const mb_dims* dims, const mb_plan_bufs* plan, const uint8_t* y_exp_dev,
                   const float* y_scale_dev, const float* w_dev, void* y_dev,
                   hipStream_t stream);

/*
 * Copy status[4] to host_status (host memory) after the work enqueued on
 * `stream` so far has finished. The only call that synchronises.
 */
int mb_plan_status(const mb_plan_bufs* plan, hipStream_t stream, int32_t host_status[4]);

#ifdef __cplusplus
}
#endif

#endif /* MOEBAL_H */
