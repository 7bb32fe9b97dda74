/*
 * mbref.h — CPU oracle for per-invocation hot-expert replication and token
 * dispatch/combine.
 *
 * TEST INFRASTRUCTURE. This library defines the expected results that the
 * GPU library is compared against. Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the GPU path never calls it
 * and shares no code, header or table with it.
 *
 * Plain, slow and single threaded on purpose: every step is a loop over the
 * definition, in the order the pages state it. See mbref.c for the steps and
 * their citations.
 *
 * Layouts (all row-major, all int32 unless noted):
 *   ids[N][K], w[N][K] (float)            routing decisions per token
 *   counts[P][E]                          d[s][e], pairs from source rank s to e
 *   load_pre[P], load_post[P]             rank loads before / after planning
 *   rep_expert[P][R]                      expert held by replica slot, -1 empty
 *   slot_quota[P][Eh+R]                   rows planned per local slot
 *   cu_seqlens[P][Eh+R+1]                 per-rank row offsets of the slots
 *   pos[N][K]                             dispatch row of each pair
 *   row_src[P*cap]                        token of each row, -1 for padding
 *   host[N][K]                            rank serving each pair
 *   status[4]                             {flags, T, max load_post, moves}
 *                                         (T = the largest target tau_r when
 *                                         planned with rank speeds)
 */
#ifndef MBREF_H
#define MBREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MBREF_F32 = 0, MBREF_BF16 = 1, MBREF_FP8_E4M3 = 2 };

enum {
  MBREF_OK = 0,
  MBREF_ERR_INVALID_ARG = -1,
  MBREF_ERR_INTERNAL = -2,
  MBREF_ERR_NOMEM = -3
};

/* status[0] bit flags */
enum {
  MBREF_ST_BAD_ID = 1,     /* an id outside [0, E) */
  MBREF_ST_DUP_ID = 2,     /* an expert listed twice for one token */
  MBREF_ST_UNBALANCED = 4, /* placement stopped with a rank above its target */
  MBREF_ST_CAPACITY = 8    /* a rank needs more than cap rows */
};
#define MBREF_ST_FATAL (MBREF_ST_BAD_ID | MBREF_ST_DUP_ID | MBREF_ST_CAPACITY)

/* Move size rule of a placement step (see mbref.c, step O2). */
enum { MBREF_MOVE_FILL_HOST = 0, MBREF_MOVE_EXCESS_ONLY = 1 };

/* Largest rank speed accepted by mbref_plan_weighted. */
#define MBREF_MAX_SPEED (1 << 20)

/* status[0] bit of mbref_plan_drift: this call ran the greedy (no fatal
 * meaning). */
#define MBREF_ST_REPLANNED 16
/* status[0] bit of mbref_plan_drift, set with REPLANNED: the kept placement,
 * replayed on this call's counts, missed the load tolerance or the region
 * size, so the greedy ran in the same call. */
#define MBREF_ST_GUARDED 32

/* Largest reference window of mbref_plan_drift (calls). */
#define MBREF_MAX_WINDOW 4096

/* Drift gate: replan when d = 1 - cos(current counts, reference) exceeds
 * delta_num / delta_den, checked every check_every calls; the reference is
 * the sum of the count vectors of up to `window` calls since the last
 * replan. Load guard: a call that keeps the placement replans after all
 * when the replay leaves a rank above cap rows or, with tol_den > 0, above
 * (1 + tol_num / tol_den) times its target (tol_den = 0: cap only). */
typedef struct mbref_drift_params {
  int32_t delta_num, delta_den, window, check_every, tol_num, tol_den;
} mbref_drift_params;

/* State carried between the calls of one layer; zero-filled (and arrays of
 * E, P*R, P*R entries) before the first call. */
typedef struct mbref_drift_state {
  int32_t have_plan;  /* a placement is kept */
  int32_t countdown;  /* calls until the next check */
  int32_t nwin;       /* count vectors in the reference */
  int32_t n_moves;    /* replicas of the kept placement */
  int64_t calls, replans;
  int64_t guarded;    /* replans the load guard forced */
  double last_d;      /* distance at the last check */
  int64_t* wsum;      /* [E] sum of the reference's count vectors */
  int32_t* rep;       /* [P*R] kept replica experts */
  int32_t* order;     /* [P*R] kept slots in placement order, -1 after */
} mbref_drift_state;

typedef struct mbref_dims {
  int32_t n_tokens;       /* N */
  int32_t top_k;          /* K */
  int32_t n_experts;      /* E */
  int32_t n_ranks;        /* P */
  int32_t slots_per_rank; /* R */
  int32_t hidden;         /* H */
  int32_t cap;            /* rows per rank region of the dispatch buffer */
  int32_t dtype_in;       /* token rows: MBREF_F32 / BF16 / FP8_E4M3 */
  int32_t dtype_out;      /* expert outputs and combined rows: F32 / BF16 */
} mbref_dims;

typedef struct mbref_plan_out {
  int32_t* counts;
  int32_t* load_pre;
  int32_t* load_post;
  int32_t* rep_expert;
  int32_t* slot_quota;
  int32_t* cu_seqlens;
  int32_t* pos;
  int32_t* row_src;
  int32_t* host;
  int32_t* status;
} mbref_plan_out;

typedef struct mbref_report {
  double ir_before;      /* max_r L_r / mean_r L_r */
  double ir_after;       /* max_r load_post / mean */
  double maxvio;         /* max_e c_e / mean_e c_e - 1 */
  double excess_removed; /* (ir_before - ir_after) / (ir_before - 1) */
  int64_t water_level;   /* T */
  int64_t n_moves;
  int64_t slots_used;
  int64_t excess_before; /* sum_r (L_r - T)^+ */
  int64_t offhome_pairs; /* pairs served by a rank other than home(e) */
  int64_t nonlocal_pairs;/* pairs served by a rank other than src(t) */
  double wir_before;     /* max_r L_r / tau*_r, tau*_r = N*K*s_r / sum s */
  double wir_after;      /* max_r load_post / tau*_r */
} mbref_report;

int mbref_version(void);

/* Steps O0-O4 and O7. Outputs must be sized as in the header comment.
 * Returns MBREF_OK (data-dependent problems are status flags) or a
 * negative error for invalid sizes. */
int mbref_plan(const mbref_dims* dims, const int32_t* ids, int32_t move_rule,
               mbref_plan_out* out, mbref_report* report);

/* The same with per-rank targets tau_r = ceil(N*K*s_r / sum_h s_h) in place
 * of the single water level (speed[P], each in [1, MBREF_MAX_SPEED]; NULL
 * means equal speeds, which is mbref_plan). */
int mbref_plan_weighted(const mbref_dims* dims, const int32_t* ids,
                        const int32_t* speed, int32_t move_rule,
                        mbref_plan_out* out, mbref_report* report);

/* Drift-gated planning of one layer's successive calls: the greedy runs on
 * the first call and whenever a check finds the counts drifted; otherwise
 * the kept placement gets new quotas (see mbref.c). */
int mbref_plan_drift(const mbref_dims* dims, const int32_t* ids, const int32_t* speed,
                     const mbref_drift_params* params, mbref_drift_state* state,
                     mbref_plan_out* out, mbref_report* report);

/* Everything at once: rank speeds (NULL = equal), a drift gate (both NULL
 * = none) and the quota repair (non-zero = on, after placement). */
typedef struct mbref_plan_options {
  const int32_t* rank_speed;
  const mbref_drift_params* drift;
  mbref_drift_state* drift_state;
  int32_t quota_repair;
} mbref_plan_options;

int mbref_plan_ex(const mbref_dims* dims, const int32_t* ids, const mbref_plan_options* opt,
                  mbref_plan_out* out, mbref_report* report);

/* The circle-method schedule of the quota repair: for n = P rounded up to
 * even, (n - 1) rounds of n/2 pairs, written as pairs[(round*n/2 + k)*2 + {0,1}];
 * index P is the bye of an odd P. */
void mbref_circle_schedule(int32_t P, int32_t* pairs);

/* Step O5: buf[pos[t][k]] = x[t] (and the fp8 scale row). Rows of buf that
 * no pair maps to are left untouched. Returns 1 if status is fatal (nothing
 * written), 0 otherwise. */
int mbref_dispatch(const mbref_dims* dims, const int32_t* pos,
                   const int32_t* status, const void* x, const float* x_scale,
                   void* buf, float* buf_scale);

/* Step O5 restricted to destination rows [row0, row1): writes row p of the
 * window to buf_win[p - row0]. */
int mbref_dispatch_window(const mbref_dims* dims, const int32_t* pos,
                          const int32_t* status, const void* x,
                          const float* x_scale, int64_t row0, int64_t row1,
                          void* buf_win, float* buf_scale_win);

/* Step O6 for tokens [t0, t1): y[t - t0][i] = sum_k w[t][k] y_exp[pos[t][k]][i]
 * in double; mag receives sum_k |w y| (may be NULL). y_exp is read as
 * dtype_out. Returns 1 if status is fatal, 0 otherwise. */
int mbref_combine(const mbref_dims* dims, const int32_t* pos,
                  const int32_t* status, const float* w, const void* y_exp,
                  int32_t t0, int32_t t1, double* y, double* mag);

/* The value of one OCP fp8 e4m3fn byte (NaN for S.1111.111). */
double mbref_e4m3_value(uint8_t b);

/* Step O6 for fp8 expert outputs with fp32 scales per 128 elements:
 * y[t][i] = sum_k w[t][k] * e4m3(y_exp[pos][i]) * y_scale[pos][i/128] in
 * double; hidden % 128 == 0. Returns 1 if status is fatal, 0 otherwise. */
int mbref_combine_fp8(const mbref_dims* dims, const int32_t* pos, const int32_t* status,
                      const float* w, const uint8_t* y_exp, const float* y_scale, int32_t t0,
                      int32_t t1, double* y, double* mag);

#ifdef __cplusplus
}
#endif

#endif /* MBREF_H */
