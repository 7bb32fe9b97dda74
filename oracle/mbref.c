/*
 * mbref.c — CPU oracle for per-invocation hot-expert replication and token
 * dispatch/combine.
 *
 * TEST INFRASTRUCTURE: the reference the GPU library is checked against.
 * Single threaded, plain loops, no blocking or fusion; built with
 * -ffp-contract=off. It shares no code with the GPU path.
 *
 * Sources (pages, by title and section):
 *  [ISER]   "ISER-MoE: Dynamic In-Switch Replication of Hot Experts for Load
 *           Balancing in Expert-Parallel" — Methodology, HALO-Q Scheduler:
 *           Objective 1 (water level T), Objective 2 (locality), stage 1
 *           (count exchange), stage 2 (busiest rank's heaviest home expert
 *           placed where a slot is free), stage 3 (smallest free helper
 *           index), stage 5 (local-first rewrite of surplus routes onto the
 *           hosts' spare quotas); Background (rank imbalance ratio); E1 table
 *           (excess load removed).
 *  [Zepp]   Zepp summary (picx.dev/p/sh48ti) — §4.1: R replica slots per
 *           GPU given greedily to the experts of highest demand; eq. (1):
 *           locality-preferred routing with demand d_i^e per source GPU.
 *  [MoonEP] "MoonEP: Planner-Enforced S×K Token Balance and Zero-Copy
 *           Buffers to Fix MoE Skew" — "What MoonEP enforces and how": every
 *           rank receives S*K tokens into fixed-shape expert-grouped buffers
 *           indexed by planner-made cu_seqlens; "Variables and core terms":
 *           maxvio; "Implementation details": home experts, then prefetch
 *           rows, in one [E+B, H, H'] numbering.
 *  [ViBE]   ViBE summary (picx.dev/p/p7vJoN) — Methodology, Variability-
 *           Informed Expert Placement: a token target per GPU in proportion
 *           to its speed, and experts go to the GPU farthest below its
 *           target.
 *
 * Readings taken where the pages leave a step open (each one is also listed
 * with its reason in the design notes of the repository):
 *  - token t originates on rank t / S; expert e is homed on rank e / Eh;
 *  - L_r counts (token, expert) pairs whose expert is homed on r, so
 *    T = ceil(N*K / P) = S*K;
 *  - with rank speeds s_r, rank r's target is tau_r = ceil(N*K*s_r / sum s)
 *    (integer speeds, so the targets are exact); the busiest rank is the one
 *    farthest above its target and the destination the one farthest below
 *    its own. With equal speeds every tau_r = T and these are the busiest
 *    and least loaded ranks;
 *  - ties: busiest rank -> lowest index; heaviest expert -> largest remaining
 *    home quota, then lowest id; destination -> least loaded, then lowest
 *    index; replica slot -> lowest free index;
 *  - a move gives the destination min(tau - load[dst], remaining home quota)
 *    pairs (it fills the host's spare quota); MBREF_MOVE_EXCESS_ONLY also
 *    caps it at the busiest rank's excess, for comparison only;
 *  - if the busiest rank's heaviest expert has no eligible destination its
 *    next heaviest is tried; if none has one, placement stops UNBALANCED;
 *  - surplus pairs go to hosts in ascending rank order; rows inside a slot
 *    are in ascending token order; local slots are numbered home experts
 *    first (by id), then replica slots;
 *  - a rank needing more than cap rows sets CAPACITY and nothing is laid out.
 *
 * Pins (tests/test_oracle_pins.py, run without a GPU): numpy bincount for the
 * counts, closed forms (one expert; uniform loads as a stable argsort),
 * brute force and an LP for the locality of the assignment, exhaustive
 * placements of the tiny workload, hand-derived worked examples, the E1
 * table of [ISER], numpy for dispatch and combine, and planted mistakes that
 * must fail them. Parity unpinned: the exact choices of the greedy, the
 * drift gate with its load guard and the quota repair follow the readings
 * above, which no page illustrates with a worked example of its own; they
 * are pinned only by the hand-derived examples, the invariants and the
 * exhaustive bound.
 */
#include "mbref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int mbref_version(void) { return 1; }

static int64_t elt_bytes(int32_t dtype) {
  switch (dtype) {
    case MBREF_F32: return 4;
    case MBREF_BF16: return 2;
    case MBREF_FP8_E4M3: return 1;
    default: return 0;
  }
}

/* O0 — sizes the method is defined for. */
static int valid_dims(const mbref_dims* d) {
  if (d->n_ranks < 1 || d->n_tokens < 0 || d->n_tokens % d->n_ranks) return 0;
  if (d->n_experts < 1 || d->n_experts % d->n_ranks) return 0;
  if (d->top_k < 1 || d->top_k > d->n_experts) return 0;
  if (d->slots_per_rank < 0 || d->cap < 1 || d->hidden < 1) return 0;
  if (!elt_bytes(d->dtype_in)) return 0;
  if (d->dtype_out != MBREF_F32 && d->dtype_out != MBREF_BF16) return 0;
  if (d->dtype_in == MBREF_FP8_E4M3 && d->hidden % 128) return 0;
  if ((int64_t)d->n_tokens * d->top_k > 2147483647LL) return 0;
  if ((int64_t)d->n_ranks * d->cap > 2147483647LL) return 0;
  return 1;
}

/* A placement kept from an earlier call: replica experts per slot and the
 * slots in the order their replicas were placed. */
typedef struct keep_t {
  const int32_t* rep;
  const int32_t* order;
  int64_t n_moves;
} keep_t;

static int plan_core(const mbref_dims* dm, const int32_t* ids, const int32_t* speed,
                     int32_t move_rule, const keep_t* keep, int32_t* order_out, int repair,
                     mbref_plan_out* o, mbref_report* rep);

int mbref_plan(const mbref_dims* dm, const int32_t* ids, int32_t move_rule,
               mbref_plan_out* o, mbref_report* rep) {
  return plan_core(dm, ids, NULL, move_rule, NULL, NULL, 0, o, rep);
}


/* Round `round` of the circle method for n (even) players: player 0 stays,
 * the others rotate one place per round; position k meets position n-1-k. */
static void circle_pair(int64_t n, int64_t round, int64_t k, int64_t* a, int64_t* b) {
  const int64_t pa = k, pb = n - 1 - k;
  *a = pa == 0 ? 0 : 1 + (pa - 1 + round) % (n - 1);
  *b = pb == 0 ? 0 : 1 + (pb - 1 + round) % (n - 1);
}

void mbref_circle_schedule(int32_t P, int32_t* pairs) {
  const int64_t n = P + (P & 1);
  for (int64_t r = 0; r + 1 < n; ++r)
    for (int64_t k = 0; k < n / 2; ++k) {
      int64_t a, b;
      circle_pair(n, r, k, &a, &b);
      pairs[(r * (n / 2) + k) * 2] = (int32_t)a;
      pairs[(r * (n / 2) + k) * 2 + 1] = (int32_t)b;
    }
}

/* Quota of expert e on rank r (home quota or replica slot), or NULL if r
 * does not hold e. */
static int64_t* quota_at(int64_t e, int64_t r, int64_t Eh, int64_t R, const int32_t* rep_expert,
                         int64_t* qh, int64_t* rq) {
  if (e / Eh == r) return &qh[e];
  for (int64_t j = 0; j < R; ++j)
    if (rep_expert[r * R + j] == e) return &rq[r * R + j];
  return NULL;
}

/* [ISER] HALO-Q stage 4, quota repair: a circle-method tournament over
 * disjoint rank pairs cancels opposite token flows. For a pair a < b and an
 * expert e both hold, a sends x_ab(e) = min((d[a][e] - Q[e][a])^+,
 * (Q[e][b] - d[b][e])^+) of its own pairs of e that b's quota could give
 * back to a; likewise x_ba(e). With m = min(sum_e x_ab(e), sum_e x_ba(e)),
 * m units of quota move from b to a over the experts of x_ab (and m from a
 * to b over those of x_ba): both ranks keep their loads, every expert keeps
 * its total, and 2m pairs become local. The experts both hold are taken in
 * the order of a's replica slots (experts homed on b or also replicated on
 * b), then b's replica slots (experts homed on a). One tournament: n - 1
 * rounds of n/2 pairs, n = P rounded up to even (the extra player is a
 * bye). */
static void quota_repair(int64_t P, int64_t E, int64_t R, const int32_t* counts,
                         const int32_t* rep_expert, int64_t* qh, int64_t* rq) {
  const int64_t Eh = E / P, n = P + (P & 1);
  int64_t* common = calloc((size_t)(2 * R + 1), sizeof(int64_t));
  if (!common) return;
  for (int64_t round = 0; round + 1 < n; ++round)
    for (int64_t k = 0; k < n / 2; ++k) {
      int64_t a, b;
      circle_pair(n, round, k, &a, &b);
      if (a >= P || b >= P) continue; /* bye */
      if (a > b) {
        const int64_t t = a;
        a = b;
        b = t;
      }
      int64_t nc = 0;
      for (int64_t j = 0; j < R; ++j) {
        const int64_t e = rep_expert[a * R + j];
        if (e >= 0 && quota_at(e, b, Eh, R, rep_expert, qh, rq)) common[nc++] = e;
      }
      for (int64_t j = 0; j < R; ++j) {
        const int64_t e = rep_expert[b * R + j];
        if (e >= 0 && e / Eh == a) common[nc++] = e;
      }
      int64_t fab = 0, fba = 0;
      for (int64_t i = 0; i < nc; ++i) {
        const int64_t e = common[i];
        const int64_t qa = *quota_at(e, a, Eh, R, rep_expert, qh, rq);
        const int64_t qb = *quota_at(e, b, Eh, R, rep_expert, qh, rq);
        const int64_t da = counts[a * E + e], db = counts[b * E + e];
        const int64_t ua = da > qa ? da - qa : 0, sb = qb > db ? qb - db : 0;
        const int64_t ub = db > qb ? db - qb : 0, sa = qa > da ? qa - da : 0;
        fab += ua < sb ? ua : sb;
        fba += ub < sa ? ub : sa;
      }
      int64_t left_ab = fab < fba ? fab : fba, left_ba = left_ab;
      for (int64_t i = 0; i < nc; ++i) {
        const int64_t e = common[i];
        int64_t* qa = quota_at(e, a, Eh, R, rep_expert, qh, rq);
        int64_t* qb = quota_at(e, b, Eh, R, rep_expert, qh, rq);
        const int64_t da = counts[a * E + e], db = counts[b * E + e];
        const int64_t ua = da > *qa ? da - *qa : 0, sb = *qb > db ? *qb - db : 0;
        const int64_t ub = db > *qb ? db - *qb : 0, sa = *qa > da ? *qa - da : 0;
        int64_t t = ua < sb ? ua : sb;
        if (t > left_ab) t = left_ab;
        *qa += t;
        *qb -= t;
        left_ab -= t;
        t = ub < sa ? ub : sa;
        if (t > left_ba) t = left_ba;
        *qb += t;
        *qa -= t;
        left_ba -= t;
      }
    }
  free(common);
}

/* Steps O0-O4 and O7. With `keep`, step O2 reuses that placement instead of
 * running the greedy; otherwise the greedy's slots are written, in move
 * order, to order_out (if not NULL). With `repair`, the quota repair runs
 * between placement and assignment. */
static int plan_core(const mbref_dims* dm, const int32_t* ids, const int32_t* speed,
                     int32_t move_rule, const keep_t* keep, int32_t* order_out, int repair,
                     mbref_plan_out* o, mbref_report* rep) {
  if (!dm || !o || !valid_dims(dm)) return MBREF_ERR_INVALID_ARG;
  if (move_rule != MBREF_MOVE_FILL_HOST && move_rule != MBREF_MOVE_EXCESS_ONLY)
    return MBREF_ERR_INVALID_ARG;
  const int64_t N = dm->n_tokens, K = dm->top_k, E = dm->n_experts;
  const int64_t P = dm->n_ranks, R = dm->slots_per_rank, cap = dm->cap;
  const int64_t S = N / P, Eh = E / P, NS = Eh + R;
  if (speed)
    for (int64_t r = 0; r < P; ++r)
      if (speed[r] < 1 || speed[r] > MBREF_MAX_SPEED) return MBREF_ERR_INVALID_ARG;
  /* [ISER] Objective 1: T = ceil(sum_r L_r / P); sum_r L_r = N*K.
   * [ViBE] token target tau_r = (total load) * s_r / sum_h s_h, rounded up;
   * equal speeds give tau_r = T. */
  int64_t* tau = calloc((size_t)(P > 0 ? P : 1), sizeof(int64_t)); /* tau_r */
  if (!tau) return MBREF_ERR_NOMEM;
  int64_t sum_s = 0;
  for (int64_t r = 0; r < P; ++r) sum_s += speed ? speed[r] : 1;
  int64_t T = 0; /* the largest target */
  for (int64_t r = 0; r < P; ++r) {
    const int64_t sr = speed ? speed[r] : 1;
    tau[r] = (N * K * sr + sum_s - 1) / sum_s;
    if (tau[r] > T) T = tau[r];
  }

  memset(o->counts, 0, sizeof(int32_t) * P * E);
  memset(o->load_pre, 0, sizeof(int32_t) * P);
  memset(o->load_post, 0, sizeof(int32_t) * P);
  for (int64_t i = 0; i < P * R; ++i) o->rep_expert[i] = -1;
  memset(o->slot_quota, 0, sizeof(int32_t) * P * NS);
  memset(o->cu_seqlens, 0, sizeof(int32_t) * P * (NS + 1));
  for (int64_t i = 0; i < N * K; ++i) o->pos[i] = -1;
  for (int64_t i = 0; i < N * K; ++i) o->host[i] = -1;
  for (int64_t i = 0; i < P * cap; ++i) o->row_src[i] = -1;
  o->status[0] = 0;
  o->status[1] = (int32_t)T;
  o->status[2] = 0;
  o->status[3] = 0;
  if (rep) memset(rep, 0, sizeof(*rep));

  /* O0 — every id names an expert, and no token names one twice. */
  int32_t flags = 0;
  for (int64_t t = 0; t < N; ++t)
    for (int64_t k = 0; k < K; ++k) {
      int32_t e = ids[t * K + k];
      if (e < 0 || e >= E) flags |= MBREF_ST_BAD_ID;
      for (int64_t k2 = 0; k2 < k; ++k2)
        if (ids[t * K + k2] == e) flags |= MBREF_ST_DUP_ID;
    }
  if (flags) {
    o->status[0] = flags;
    free(tau);
    return MBREF_OK;
  }

  int64_t* c = calloc((size_t)E, sizeof(int64_t));     /* c_e */
  int64_t* L = calloc((size_t)P, sizeof(int64_t));     /* L_r */
  int64_t* load = calloc((size_t)P, sizeof(int64_t));  /* running load */
  int64_t* qh = calloc((size_t)E, sizeof(int64_t));    /* home quota */
  int64_t* rq = calloc((size_t)(P * R + 1), sizeof(int64_t)); /* replica quota */
  char* is_host = calloc((size_t)(E * P), 1);          /* [e][r] */
  char* tried = calloc((size_t)(Eh + 1), 1);
  int64_t* Q = calloc((size_t)(E * P), sizeof(int64_t));    /* quota [e][h] */
  int64_t* used = calloc((size_t)(E * P), sizeof(int64_t)); /* [e][h] */
  int64_t* slot_of = calloc((size_t)(E * P), sizeof(int64_t)); /* [h][e] */
  int64_t* rows = calloc((size_t)(P * NS), sizeof(int64_t));
  int64_t* cu = calloc((size_t)(P * (NS + 1)), sizeof(int64_t));
  int64_t* fill = calloc((size_t)(P * NS), sizeof(int64_t));
  int rc = MBREF_OK;
  if (!c || !L || !load || !qh || !rq || !is_host || !tried || !Q || !used ||
      !slot_of || !rows || !cu || !fill) {
    rc = MBREF_ERR_NOMEM;
    goto done;
  }

  /* O1 — count. [ISER] stage 1: routed pairs per (source rank, expert),
   * d_i^e of [Zepp] eq. (1); c_e = sum_s d[s][e]; L_r = sum of c_e over
   * r's home experts. */
  for (int64_t t = 0; t < N; ++t) {
    const int64_t s = t / S;
    for (int64_t k = 0; k < K; ++k) o->counts[s * E + ids[t * K + k]] += 1;
  }
  for (int64_t s = 0; s < P; ++s)
    for (int64_t e = 0; e < E; ++e) c[e] += o->counts[s * E + e];
  for (int64_t e = 0; e < E; ++e) L[e / Eh] += c[e];
  for (int64_t r = 0; r < P; ++r) o->load_pre[r] = (int32_t)L[r];

  /* O2 — greedy placement. [ISER] stage 2 picks the busiest rank's heaviest
   * home expert and places a replica where a slot is free; stage 3 takes the
   * smallest free helper index; [Zepp] §4.1 provides R slots per rank. */
  for (int64_t r = 0; r < P; ++r) load[r] = L[r];
  for (int64_t e = 0; e < E; ++e) {
    qh[e] = c[e];
    is_host[e * P + e / Eh] = 1;
  }
  int64_t moves = 0;
  int unbalanced = 0;
  if (keep) {
    /* [ViBE] Drift-Aware Recalibration keeps the placement while the load
     * has not drifted: the kept replicas, in the order they were placed,
     * each take min(target - load of its host, remaining home quota) pairs
     * while its home rank is above its target and its host below its own,
     * else none. */
    for (int64_t i = 0; i < P * R; ++i) o->rep_expert[i] = keep->rep[i];
    for (int64_t i = 0; i < keep->n_moves; ++i) {
      const int64_t slot = keep->order[i], dst = slot / R;
      const int64_t e = keep->rep[slot], h = e / Eh;
      int64_t m = 0;
      if (load[h] > tau[h] && load[dst] < tau[dst]) {
        m = tau[dst] - load[dst];
        if (qh[e] < m) m = qh[e];
      }
      rq[slot] = m;
      is_host[e * P + dst] = 1;
      qh[e] -= m;
      load[h] -= m;
      load[dst] += m;
    }
    moves = keep->n_moves;
    for (int64_t r = 0; r < P; ++r)
      if (load[r] > tau[r]) unbalanced = 1;
  }
  for (; !keep;) {
    int64_t rs = 0; /* busiest rank (farthest above its target), lowest index on ties */
    for (int64_t r = 1; r < P; ++r)
      if (load[r] - tau[r] > load[rs] - tau[rs]) rs = r;
    if (load[rs] <= tau[rs]) break;
    memset(tried, 0, (size_t)Eh);
    int moved = 0;
    for (;;) {
      int64_t best = -1; /* heaviest untried home expert of rs */
      for (int64_t i = 0; i < Eh; ++i) {
        const int64_t e = rs * Eh + i;
        if (tried[i] || qh[e] == 0) continue;
        if (best < 0 || qh[e] > qh[best]) best = e;
      }
      if (best < 0) break;
      tried[best - rs * Eh] = 1;
      /* eligible rank farthest below its target (the least loaded one when
       * targets are equal), lowest index on ties */
      int64_t dst = -1;
      for (int64_t r = 0; r < P; ++r) {
        int64_t nfree = 0;
        for (int64_t j = 0; j < R; ++j)
          if (o->rep_expert[r * R + j] < 0) ++nfree;
        if (nfree == 0 || load[r] >= tau[r] || is_host[best * P + r]) continue;
        if (dst < 0 || tau[r] - load[r] > tau[dst] - load[dst]) dst = r;
      }
      if (dst < 0) continue;
      int64_t m = tau[dst] - load[dst];
      if (qh[best] < m) m = qh[best];
      if (move_rule == MBREF_MOVE_EXCESS_ONLY && load[rs] - tau[rs] < m) m = load[rs] - tau[rs];
      int64_t j = 0; /* smallest free slot index */
      while (o->rep_expert[dst * R + j] >= 0) ++j;
      o->rep_expert[dst * R + j] = (int32_t)best;
      rq[dst * R + j] = m;
      if (order_out) order_out[moves] = (int32_t)(dst * R + j);
      is_host[best * P + dst] = 1;
      qh[best] -= m;
      load[rs] -= m;
      load[dst] += m;
      ++moves;
      moved = 1;
      break;
    }
    if (!moved) {
      unbalanced = 1;
      break;
    }
  }

  if (repair) quota_repair(P, E, R, o->counts, o->rep_expert, qh, rq);

  /* Quotas per (expert, host) and the local slot of each (host, expert):
   * home experts first by id, then replica slots ([MoonEP] [E+B,H,H']). */
  for (int64_t i = 0; i < E * P; ++i) slot_of[i] = -1;
  for (int64_t e = 0; e < E; ++e) {
    const int64_t h = e / Eh;
    Q[e * P + h] = qh[e];
    slot_of[h * E + e] = e - h * Eh;
    o->slot_quota[h * NS + (e - h * Eh)] = (int32_t)qh[e];
  }
  for (int64_t r = 0; r < P; ++r)
    for (int64_t j = 0; j < R; ++j) {
      const int32_t e = o->rep_expert[r * R + j];
      if (e < 0) continue;
      Q[e * P + r] = rq[r * R + j];
      slot_of[r * E + e] = Eh + j;
      o->slot_quota[r * NS + Eh + j] = (int32_t)rq[r * R + j];
    }

  /* O3 — assignment. [ISER] Objective 2 and stage 5; [Zepp] eq. (1).
   * Pass 1, in (t, k) order: a pair stays on its source rank when that rank
   * hosts the expert and still has quota. */
  for (int64_t t = 0; t < N; ++t) {
    const int64_t s = t / S;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t e = ids[t * K + k];
      if (is_host[e * P + s] && used[e * P + s] < Q[e * P + s]) {
        o->host[t * K + k] = (int32_t)s;
        used[e * P + s] += 1;
      }
    }
  }
  /* Pass 2, same order: every other pair goes to the lowest-index host of
   * its expert that still has spare quota. */
  for (int64_t t = 0; t < N; ++t)
    for (int64_t k = 0; k < K; ++k) {
      if (o->host[t * K + k] >= 0) continue;
      const int64_t e = ids[t * K + k];
      int64_t h = 0;
      while (h < P && !(is_host[e * P + h] && used[e * P + h] < Q[e * P + h])) ++h;
      if (h == P) {
        rc = MBREF_ERR_INTERNAL; /* sum of quotas < c_e: cannot happen */
        goto done;
      }
      o->host[t * K + k] = (int32_t)h;
      used[e * P + h] += 1;
    }

  /* O4 — layout. [MoonEP] fixed [P*cap, H] buffer, rank r's region starting
   * at row r*cap, slots contiguous in local slot order (cu_seqlens), rows of
   * a slot in ascending token order. */
  for (int64_t t = 0; t < N; ++t)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t h = o->host[t * K + k];
      rows[h * NS + slot_of[h * E + ids[t * K + k]]] += 1;
    }
  int64_t max_load = 0;
  int cap_exceeded = 0;
  for (int64_t h = 0; h < P; ++h) {
    for (int64_t i = 0; i < NS; ++i) cu[h * (NS + 1) + i + 1] = cu[h * (NS + 1) + i] + rows[h * NS + i];
    for (int64_t i = 0; i <= NS; ++i) o->cu_seqlens[h * (NS + 1) + i] = (int32_t)cu[h * (NS + 1) + i];
    const int64_t lp = cu[h * (NS + 1) + NS];
    o->load_post[h] = (int32_t)lp;
    if (lp > max_load) max_load = lp;
    if (lp > cap) cap_exceeded = 1;
  }
  if (!cap_exceeded) {
    for (int64_t t = 0; t < N; ++t)
      for (int64_t k = 0; k < K; ++k) {
        const int64_t h = o->host[t * K + k];
        const int64_t sl = slot_of[h * E + ids[t * K + k]];
        const int64_t p = h * cap + cu[h * (NS + 1) + sl] + fill[h * NS + sl];
        fill[h * NS + sl] += 1;
        o->pos[t * K + k] = (int32_t)p;
        o->row_src[p] = (int32_t)t;
      }
  }
  o->status[0] = (unbalanced ? MBREF_ST_UNBALANCED : 0) | (cap_exceeded ? MBREF_ST_CAPACITY : 0);
  o->status[2] = (int32_t)max_load;
  o->status[3] = (int32_t)moves;

  /* O7 — report. IR as in [ISER] Background; maxvio as in [MoonEP]
   * "Variables and core terms"; excess removed as in [ISER] E1. */
  if (rep) {
    const double mean_l = (double)(N * K) / (double)P;
    const double mean_c = (double)(N * K) / (double)E;
    int64_t maxL = 0, maxc = 0;
    for (int64_t r = 0; r < P; ++r) {
      if (L[r] > maxL) maxL = L[r];
      if (L[r] > tau[r]) rep->excess_before += L[r] - tau[r];
    }
    /* the same ratios against each rank's unrounded target
     * tau*_r = N*K*s_r / sum s (no pairs: balanced) */
    rep->wir_before = rep->wir_after = N * K > 0 ? 0.0 : 1.0;
    for (int64_t r = 0; r < P && N * K > 0; ++r) {
      const double ts = (double)(N * K) * (double)(speed ? speed[r] : 1) / (double)sum_s;
      if (L[r] / ts > rep->wir_before) rep->wir_before = L[r] / ts;
      if (o->load_post[r] / ts > rep->wir_after) rep->wir_after = o->load_post[r] / ts;
    }
    for (int64_t e = 0; e < E; ++e)
      if (c[e] > maxc) maxc = c[e];
    rep->ir_before = mean_l > 0 ? (double)maxL / mean_l : 1.0;
    rep->ir_after = mean_l > 0 ? (double)max_load / mean_l : 1.0;
    rep->maxvio = mean_c > 0 ? (double)maxc / mean_c - 1.0 : 0.0;
    rep->excess_removed = rep->ir_before > 1.0
                              ? (rep->ir_before - rep->ir_after) / (rep->ir_before - 1.0)
                              : 1.0;
    rep->water_level = T;
    rep->n_moves = moves;
    rep->slots_used = moves;
    for (int64_t t = 0; t < N; ++t)
      for (int64_t k = 0; k < K; ++k) {
        const int64_t h = o->host[t * K + k];
        if (h != ids[t * K + k] / Eh) rep->offhome_pairs += 1;
        if (h != t / S) rep->nonlocal_pairs += 1;
      }
  }

done:
  free(c); free(L); free(load); free(qh); free(rq); free(is_host); free(tried);
  free(Q); free(used); free(slot_of); free(rows); free(cu); free(fill); free(tau);
  return rc;
}

int mbref_plan_weighted(const mbref_dims* dm, const int32_t* ids, const int32_t* speed,
                        int32_t move_rule, mbref_plan_out* o, mbref_report* rep) {
  return plan_core(dm, ids, speed, move_rule, NULL, NULL, 0, o, rep);
}

/* [ViBE] Drift-Aware Recalibration: d = 1 - w.w^ / (|w| |w^|). The window's
 * sum stands for its mean (same direction); the three sums are exact
 * integers, then one division and two square roots in double. */
static double cosine_distance(const int64_t* c, const int64_t* ws, int64_t E) {
  unsigned __int128 dot = 0, n1 = 0, n2 = 0;
  for (int64_t e = 0; e < E; ++e) {
    dot += (unsigned __int128)(uint64_t)c[e] * (uint64_t)ws[e];
    n1 += (unsigned __int128)(uint64_t)c[e] * (uint64_t)c[e];
    n2 += (unsigned __int128)(uint64_t)ws[e] * (uint64_t)ws[e];
  }
  if (n1 == 0 || n2 == 0) return n1 == n2 ? 0.0 : 1.0;
  return 1.0 - (double)dot / (sqrt((double)n1) * sqrt((double)n2));
}

/* Load guard on a replayed placement ([ViBE] Incremental placement update:
 * a placement is done once every GPU is within the tolerance epsilon of the
 * balanced time; with time proportional to load over speed that is load_r
 * <= (1 + epsilon) tau_r): the replay stands when no rank needs more than
 * cap rows and, with tol_den > 0, load_r * tol_den <= tau_r * (tol_den +
 * tol_num) for every rank, in exact integers. */
static int replay_within_guard(const mbref_dims* dm, const int32_t* speed,
                               const mbref_drift_params* prm, const mbref_plan_out* o) {
  const int64_t P = dm->n_ranks, NK = (int64_t)dm->n_tokens * dm->top_k;
  int64_t sum_s = 0;
  for (int64_t r = 0; r < P; ++r) sum_s += speed ? speed[r] : 1;
  for (int64_t r = 0; r < P; ++r) {
    const int64_t load = o->load_post[r];
    const int64_t tau = (NK * (speed ? speed[r] : 1) + sum_s - 1) / sum_s;
    if (load > dm->cap) return 0;
    if (prm->tol_den > 0 && load * prm->tol_den > tau * ((int64_t)prm->tol_den + prm->tol_num))
      return 0;
  }
  return 1;
}

static int plan_drift_core(const mbref_dims* dm, const int32_t* ids, const int32_t* speed,
                           const mbref_drift_params* prm, mbref_drift_state* st, int repair,
                           mbref_plan_out* o, mbref_report* rep) {
  if (!dm || !o || !prm || !st || !valid_dims(dm)) return MBREF_ERR_INVALID_ARG;
  if (prm->delta_den < 1 || prm->delta_num < 0 || prm->delta_num > prm->delta_den ||
      prm->window < 1 || prm->window > MBREF_MAX_WINDOW || prm->check_every < 1 ||
      prm->tol_num < 0 || prm->tol_den < 0)
    return MBREF_ERR_INVALID_ARG;
  const int64_t N = dm->n_tokens, K = dm->top_k, E = dm->n_experts;
  const int64_t P = dm->n_ranks, R = dm->slots_per_rank;
  /* Routing decisions that are not a valid input leave the state alone. */
  for (int64_t t = 0; t < N; ++t)
    for (int64_t k = 0; k < K; ++k) {
      const int32_t e = ids[t * K + k];
      int bad = e < 0 || e >= E;
      for (int64_t k2 = 0; k2 < k; ++k2) bad |= ids[t * K + k2] == e;
      if (bad) return plan_core(dm, ids, speed, MBREF_MOVE_FILL_HOST, NULL, NULL, 0, o, rep);
    }
  int64_t* c = calloc((size_t)E, sizeof(int64_t));
  int32_t* order = calloc((size_t)(P * R + 1), sizeof(int32_t));
  if (!c || !order) {
    free(c);
    free(order);
    return MBREF_ERR_NOMEM;
  }
  for (int64_t i = 0; i < N * K; ++i) c[ids[i]] += 1;
  /* Replan on the first call, then check every check_every calls. */
  int replan = !st->have_plan, guarded = 0;
  if (!replan && --st->countdown == 0) {
    st->countdown = prm->check_every;
    st->last_d = cosine_distance(c, st->wsum, E);
    if (st->last_d > (double)prm->delta_num / (double)prm->delta_den) replan = 1;
  }
  int rc = MBREF_OK;
  if (!replan) {
    const keep_t keep = {st->rep, st->order, st->n_moves};
    rc = plan_core(dm, ids, speed, MBREF_MOVE_FILL_HOST, &keep, NULL, repair, o, rep);
    if (rc == MBREF_OK && !replay_within_guard(dm, speed, prm, o)) {
      replan = 1;
      guarded = 1;
    } else if (rc == MBREF_OK && st->nwin < prm->window) {
      for (int64_t e = 0; e < E; ++e) st->wsum[e] += c[e];
      st->nwin += 1;
    }
  }
  if (replan) {
    rc = plan_core(dm, ids, speed, MBREF_MOVE_FILL_HOST, NULL, order, repair, o, rep);
    if (rc == MBREF_OK) {
      for (int64_t i = 0; i < P * R; ++i) st->rep[i] = o->rep_expert[i];
      for (int64_t i = 0; i < P * R; ++i) st->order[i] = i < o->status[3] ? order[i] : -1;
      st->n_moves = o->status[3];
      st->have_plan = 1;
      st->countdown = prm->check_every;
      /* the reference restarts from the load seen at the recalibration */
      for (int64_t e = 0; e < E; ++e) st->wsum[e] = c[e];
      st->nwin = 1;
      st->replans += 1;
      st->guarded += guarded;
      o->status[0] |= MBREF_ST_REPLANNED | (guarded ? MBREF_ST_GUARDED : 0);
    }
  }
  if (rc == MBREF_OK) st->calls += 1;
  free(c);
  free(order);
  return rc;
}

int mbref_plan_drift(const mbref_dims* dm, const int32_t* ids, const int32_t* speed,
                     const mbref_drift_params* prm, mbref_drift_state* st,
                     mbref_plan_out* o, mbref_report* rep) {
  return plan_drift_core(dm, ids, speed, prm, st, 0, o, rep);
}

int mbref_plan_ex(const mbref_dims* dm, const int32_t* ids, const mbref_plan_options* opt,
                  mbref_plan_out* o, mbref_report* rep) {
  if (!opt) return MBREF_ERR_INVALID_ARG;
  if (opt->drift || opt->drift_state) {
    if (!opt->drift || !opt->drift_state) return MBREF_ERR_INVALID_ARG;
    return plan_drift_core(dm, ids, opt->rank_speed, opt->drift, opt->drift_state,
                           opt->quota_repair != 0, o, rep);
  }
  return plan_core(dm, ids, opt->rank_speed, MBREF_MOVE_FILL_HOST, NULL, NULL,
                   opt->quota_repair != 0, o, rep);
}

/* O5 — dispatch: the row of token t is copied to every row pos[t][k]
 * ([MoonEP] "What MoonEP enforces and how": tokens written straight into the
 * fixed-shape expert-grouped buffers). */
int mbref_dispatch_window(const mbref_dims* dm, const int32_t* pos,
                          const int32_t* status, const void* x,
                          const float* x_scale, int64_t row0, int64_t row1,
                          void* buf_win, float* buf_scale_win) {
  if (!dm || !valid_dims(dm)) return MBREF_ERR_INVALID_ARG;
  if (status[0] & MBREF_ST_FATAL) return 1;
  const int64_t N = dm->n_tokens, K = dm->top_k;
  const int64_t rb = (int64_t)dm->hidden * elt_bytes(dm->dtype_in);
  const int64_t nsc = dm->dtype_in == MBREF_FP8_E4M3 ? dm->hidden / 128 : 0;
  for (int64_t t = 0; t < N; ++t)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t p = pos[t * K + k];
      if (p < row0 || p >= row1) continue;
      memcpy((char*)buf_win + (p - row0) * rb, (const char*)x + t * rb, (size_t)rb);
      if (nsc && buf_scale_win && x_scale)
        memcpy(buf_scale_win + (p - row0) * nsc, x_scale + t * nsc, sizeof(float) * (size_t)nsc);
    }
  return 0;
}

int mbref_dispatch(const mbref_dims* dm, const int32_t* pos,
                   const int32_t* status, const void* x, const float* x_scale,
                   void* buf, float* buf_scale) {
  if (!dm || !valid_dims(dm)) return MBREF_ERR_INVALID_ARG;
  return mbref_dispatch_window(dm, pos, status, x, x_scale, 0,
                               (int64_t)dm->n_ranks * dm->cap, buf, buf_scale);
}

static double out_elem(int32_t dtype, const void* base, int64_t idx) {
  if (dtype == MBREF_F32) return (double)((const float*)base)[idx];
  uint32_t b = (uint32_t)((const uint16_t*)base)[idx] << 16; /* bf16 */
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

/* O6 — combine: the weighted gather-reduce of the K expert-output rows of
 * each token, in double precision. */
int mbref_combine(const mbref_dims* dm, const int32_t* pos,
                  const int32_t* status, const float* w, const void* y_exp,
                  int32_t t0, int32_t t1, double* y, double* mag) {
  if (!dm || !valid_dims(dm) || t0 < 0 || t1 < t0 || t1 > dm->n_tokens)
    return MBREF_ERR_INVALID_ARG;
  if (status[0] & MBREF_ST_FATAL) return 1;
  const int64_t K = dm->top_k, H = dm->hidden;
  for (int64_t t = t0; t < t1; ++t)
    for (int64_t i = 0; i < H; ++i) {
      double acc = 0.0, a = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double v = out_elem(dm->dtype_out, y_exp, (int64_t)pos[t * K + k] * H + i);
        const double term = (double)w[t * K + k] * v;
        acc += term;
        a += fabs(term);
      }
      y[(t - t0) * H + i] = acc;
      if (mag) mag[(t - t0) * H + i] = a;
    }
  return 0;
}

/* OCP fp8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities. */
double mbref_e4m3_value(uint8_t b) {
  const int sign = b >> 7, ex = (b >> 3) & 15, m = b & 7;
  double v;
  if (ex == 15 && m == 7)
    v = NAN;
  else if (ex == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, ex - 7);
  return sign ? -v : v;
}

/* Step O6 with fp8 expert outputs (the dequantising combine):
 * y[t][i] = sum_k w[t][k] * e4m3(y_exp[pos][i]) * y_scale[pos][i / 128] in
 * double for tokens [t0, t1); mag receives sum_k |term|. */
int mbref_combine_fp8(const mbref_dims* dm, const int32_t* pos, const int32_t* status,
                      const float* w, const uint8_t* y_exp, const float* y_scale, int32_t t0,
                      int32_t t1, double* y, double* mag) {
  if (!dm || !valid_dims(dm) || dm->hidden % 128 || t0 < 0 || t1 < t0 || t1 > dm->n_tokens)
    return MBREF_ERR_INVALID_ARG;
  if (status[0] & MBREF_ST_FATAL) return 1;
  const int64_t K = dm->top_k, H = dm->hidden;
  for (int64_t t = t0; t < t1; ++t)
    for (int64_t i = 0; i < H; ++i) {
      double acc = 0.0, a = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t p = pos[t * K + k];
        const double v = mbref_e4m3_value(y_exp[p * H + i]) * (double)y_scale[p * (H / 128) + i / 128];
        const double term = (double)w[t * K + k] * v;
        acc += term;
        a += fabs(term);
      }
      y[(t - t0) * H + i] = acc;
      if (mag) mag[(t - t0) * H + i] = a;
    }
  return 0;
}
