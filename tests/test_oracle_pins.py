"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test fixes the oracle to something other than itself: library routines
(numpy bincount / stable argsort / fancy indexing, scipy milp), closed forms,
invariants, brute force on tiny inputs, a hand-derived worked example, and
the E1 table of the ISER-MoE page. A plausible slip in the oracle (a wrong
tie-break, a wrong move size, a transposed count, a lost term in combine)
fails at least one of them.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
import workload as W
from tests import plan_checks as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _plan_workload(name, call=0, **kw):
    wl = W.get_workload(name)
    ids, w = W.routing_for(wl, call)
    d = O.dims_for(wl, **kw)
    return wl, ids, w, d, O.plan(d, ids)


# ---- hand-derived worked example ------------------------------------------

def test_hand_example_fill():
    """P=3 ranks, 2 home experts each, R=1, K=1, 12 tokens, T = 4.

    Routed counts c = [4, 1, 3, 2, 2, 0] give L = [5, 5, 2].
    Step 1: ranks 0 and 1 tie at 5 -> rank 0; its heaviest expert is 0
    (quota 4); the only rank below T with a free slot is rank 2 (load 2);
    the move fills it to T: m = min(4 - 2, 4) = 2 -> loads [3, 5, 4].
    Step 2: rank 1 (5); heaviest expert 2 (quota 3); eligible: rank 0
    (load 3, slot free); m = min(1, 3) = 1 -> loads [4, 4, 4]; stop.
    Routing: pass 1 keeps t0, t2 (e0) and t1 (e2 replica) on rank 0, t5, t6
    on rank 1, t8 (e0 replica) and t11 on rank 2; pass 2 sends t3 -> 2,
    t4 -> 2 (rank 0's e0 quota is full), t7 -> 0, t9 -> 1, t10 -> 1.
    Rows follow home slots by id, then the replica slot, ascending token
    order inside each slot, region of rank r at row 4r.
    """
    g = json.load(open(os.path.join(GOLDEN, "hand_example_fill.json")))
    dd = g["dims"]
    d = O.make_dims(**dd)
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    p = O.plan(d, ids)
    f = g["fill_host"]
    for key in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
                "status", "row_src"):
        assert np.array_equal(getattr(p, key), np.array(f[key])), key
    assert np.array_equal(p.host.ravel(), f["host"])
    assert np.array_equal(p.pos.ravel(), f["pos"])
    assert p.report["nonlocal_pairs"] == f["nonlocal_pairs"]
    assert p.report["offhome_pairs"] == f["offhome_pairs"]
    assert p.report["ir_before"] == pytest.approx(f["ir_before"])
    assert p.report["ir_after"] == pytest.approx(f["ir_after"])
    assert p.report["maxvio"] == pytest.approx(f["maxvio"])


def test_hand_example_excess_only_stalls():
    """Same input, moves capped at the busiest rank's excess: step 1 moves
    only 1 pair of expert 0 to rank 2 (loads [4, 5, 3]); then rank 1 is
    busiest, but rank 0 is at T and rank 2's only slot is taken, so no
    expert of rank 1 has a destination: UNBALANCED, and rank 1 needs 5 > cap
    rows (CAPACITY)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example_fill.json")))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    p = O.plan(d, ids, move_rule=O.MOVE_EXCESS_ONLY)
    f = g["excess_only"]
    for key in ("load_post", "rep_expert", "slot_quota", "status"):
        assert np.array_equal(getattr(p, key), np.array(f[key])), key
    assert np.all(p.pos == -1) and np.all(p.row_src == -1)


def test_hand_example_expert_tie():
    """P=2 ranks, 2 home experts each, R=1, K=1, 8 tokens, T = 4.

    c = [3, 3, 2, 0], L = [6, 2]. Rank 0 is above T; its experts 0 and 1 tie
    at quota 3, so expert 0 (the lower id) gets the replica, on rank 1 (the
    only open rank): m = min(4 - 2, 3) = 2, loads [4, 4]. Pass 1 keeps t0
    (e0, quota 1), t1 and t3 (e1) on rank 0 and t4 (replica of e0), t6, t7
    (e2) on rank 1; pass 2 sends t2 (e0: rank 0 full) to rank 1 and t5 (e1)
    to rank 0. Rank 1's replica slot holds t2, t4 in token order.
    """
    g = json.load(open(os.path.join(GOLDEN, "hand_example_expert_tie.json")))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    p = O.plan(d, ids)
    for key in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
                "status", "row_src"):
        assert np.array_equal(getattr(p, key), np.array(g[key])), key
    assert np.array_equal(p.host.ravel(), g["host"])
    assert np.array_equal(p.pos.ravel(), g["pos"])


def _check_golden(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    p = O.plan(d, ids)
    for key in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
                "status", "row_src"):
        assert np.array_equal(getattr(p, key), np.array(g[key])), key
    assert np.array_equal(p.host.ravel(), g["host"])
    assert np.array_equal(p.pos.ravel(), g["pos"])


def test_hand_example_destination_tie():
    """P=3, 2 home experts each, R=1, K=1, 6 tokens, T = 2.

    c = [0, 1, 1, 0, 2, 2], L = [1, 1, 4]. Step 1: rank 2's experts 4 and 5
    tie at 2 -> expert 4; ranks 0 and 1 tie as open ranks at load 1 -> rank
    0 (lower index) gets expert 4, m = min(2 - 1, 2) = 1 -> loads [2, 1, 3].
    Step 2: rank 2's heaviest is now expert 5 (2 > 1); the only open rank is
    1: m = 1 -> loads [2, 2, 2]. Pass 1 keeps t1 (e1) on 0, t3 (e2) on 1, t4
    (e4) and t5 (e5) on 2; pass 2 sends t0 (e5) to its replica on rank 1 and
    t2 (e4) to its replica on rank 0 (lower index than home rank 2).
    """
    _check_golden("hand_example_destination_tie.json")


def test_hand_example_surplus_order():
    """P=3, 1 home expert each, R=1, K=1, 6 tokens, T = 2.

    c = [3, 2, 1], L = [3, 2, 1]. Rank 0 gives expert 0 to rank 2 (the only
    rank below T): m = min(2 - 1, 3) = 1, quotas e0: rank 0 two, rank 2 one.
    Pass 1 keeps only t1 (e0 on its home). Pass 2 in token order: t0 (e2) to
    rank 2; t2 (e0) to the lowest-index holder with quota left, rank 0; t3
    (e0) then finds rank 0 full and goes to rank 2; t4, t5 (e1) to rank 1.
    """
    _check_golden("hand_example_surplus_order.json")


# ---- invariants on every workload -------------------------------------------

def test_hand_example_weighted():
    """P=4 ranks of speeds s = [4, 4, 2, 1], 2 home experts each, R=1, K=1,
    16 tokens (4 per source rank), cap 6.

    Targets tau_r = ceil(16 s_r / 11) = ceil([5.82, 5.82, 2.91, 1.45]) =
    [6, 6, 3, 2]. Counts c = [5, 2, 2, 1, 1, 1, 3, 1] give L = [7, 3, 2, 4],
    i.e. L - tau = [+1, -3, -1, +2].
    Step 1: farthest above its target is rank 3 (+2; rank 0 has the larger
    load but only +1); its heaviest expert is 6 (quota 3); open ranks are
    1 (deficit 3) and 2 (deficit 1; it is the least loaded, but not the
    farthest below target) -> rank 1; m = min(6 - 3, 3) = 3 -> loads
    [7, 6, 2, 1].
    Step 2: rank 0 (+1); heaviest expert 0 (quota 5); rank 1 has no free
    slot, ranks 2 and 3 both lack 1 -> rank 2 (lower index);
    m = min(3 - 2, 5) = 1 -> loads [6, 6, 3, 1]; every rank is at or below
    its target; stop after 2 moves.
    Routing: pass 1 keeps t0-t3 (e0, quota 4), t7 (e2), t10, t11, t15 home;
    pass 2 sends t4 (e0) -> 2 (rank 0 is full), t5, t6 -> 0, t8, t9 -> 1,
    t12-t14 (e6: home quota 0) -> the replica on rank 1.
    Region of rank r at row 6r; home slots by id, then the replica slot.
    Against the unrounded targets 16 s_r / 11 the largest ratio falls from
    4 / 1.4545 = 2.75 to 6 / 5.8182 = 1.03125.
    """
    g = json.load(open(os.path.join(GOLDEN, "hand_example_weighted.json")))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    p = O.plan(d, ids, speeds=np.array(g["speeds"], np.int32))
    for key in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
                "status", "row_src"):
        assert np.array_equal(getattr(p, key), np.array(g[key])), key
    assert np.array_equal(p.host.ravel(), g["host"])
    assert np.array_equal(p.pos.ravel(), g["pos"])
    assert p.report["water_level"] == max(g["targets"])
    assert p.report["nonlocal_pairs"] == g["nonlocal_pairs"]
    assert p.report["offhome_pairs"] == g["offhome_pairs"]
    assert p.report["wir_before"] == pytest.approx(g["wir_before"])
    assert p.report["wir_after"] == pytest.approx(g["wir_after"])
    # the rounding of the targets matters: with cap 5 rank 0 and 1 overflow
    d5 = O.make_dims(**dict(g["dims"], cap=5))
    p5 = O.plan(d5, ids, speeds=np.array(g["speeds"], np.int32))
    assert p5.flags == O.ST_CAPACITY and np.array_equal(p5.load_post, g["load_post"])


def test_equal_speeds_are_the_water_level():
    """Equal speeds (any value) give every rank the target T: the hand-derived
    unweighted example comes out unchanged."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example_fill.json")))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    f = g["fill_host"]
    for v in (1, 7, 1 << 20):
        p = O.plan(d, ids, speeds=np.full(3, v, np.int32))
        for key in ("load_post", "rep_expert", "slot_quota", "cu_seqlens", "status", "row_src"):
            assert np.array_equal(getattr(p, key), np.array(f[key])), key
        assert np.array_equal(p.pos.ravel(), f["pos"])
        assert p.report["wir_after"] == pytest.approx(f["ir_after"])


def test_speeds_rejected_out_of_range():
    g = json.load(open(os.path.join(GOLDEN, "hand_example_weighted.json")))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32)
    for bad in ([0, 4, 2, 1], [4, -1, 2, 1], [4, 4, 2, (1 << 20) + 1]):
        assert O.plan_rc(d, ids, np.array(bad, np.int32)) == O.ERR_INVALID_ARG


def test_hand_example_drift():
    """Drift-gated replanning: P=2 ranks, 2 home experts each, R=1, K=1,
    8 tokens, T = 4; replan when d > 1/2, checked every call, reference of
    up to 2 calls.

    Call 0 (c = [4, 1, 1, 2], L = [5, 3]): the first call runs the greedy:
    expert 0 goes to rank 1 with min(4 - 3, 4) = 1 pair -> loads [4, 4];
    the kept placement is slot 1 (rank 1) holding expert 0; reference
    r = [4, 1, 1, 2].
    Call 1 (c = [2, 0, 3, 3], L = [2, 6]): c.r = 17, |c|^2 = 22, |r|^2 = 22,
    d = 1 - 17/22 = 5/22 < 1/2 -> keep; the kept replica takes nothing (its
    home rank 0 is not above T) -> loads [2, 6], UNBALANCED, where a fresh
    greedy would have reached [4, 4]; r = [6, 1, 4, 5] (2 calls).
    Call 2 (c = [5, 1, 0, 2], L = [6, 2]): c.r = 41, |c|^2 = 30, |r|^2 = 78,
    d = 1 - 41/sqrt(2340) = 0.152 -> keep; the replica takes
    min(4 - 2, 5) = 2 -> [4, 4]; the window is full, r stays.
    Call 3 (all tokens to expert 1): c.r = 8, |c|^2 = 64, d = 1 -
    8/sqrt(4992) = 0.887 -> replan: expert 1 goes to rank 1 with
    min(4 - 0, 8) = 4 pairs; the reference restarts at [0, 8, 0, 0].
    (Had the reference not accumulated call 1, call 2 would have seen
    d = 1 - 25/sqrt(660) = 0.027 against r = [4, 1, 1, 2] as well, and kept;
    had it not restarted at call 3, the window would still hold [6, 1, 4, 5].)
    """
    g = json.load(open(os.path.join(GOLDEN, "hand_example_drift.json")))
    d = O.make_dims(**g["dims"])
    prm = O.DriftParams(**g["params"])
    st = O.DriftState(d.n_experts, d.n_ranks, d.slots_per_rank)
    for i, call in enumerate(g["calls"]):
        ids = np.array(call["ids"], np.int32).reshape(-1, 1)
        p = O.plan(d, ids, drift=(prm, st))
        for key in ("status", "load_post", "rep_expert", "slot_quota"):
            assert np.array_equal(getattr(p, key), np.array(call[key])), (i, key)
        C.check_layout(p, ids, d.n_ranks, d.n_experts, d.slots_per_rank, d.cap)
        exp = call["state"]
        for key in ("have_plan", "countdown", "nwin", "n_moves", "calls", "replans"):
            assert getattr(st, key) == exp[key], (i, key)
        assert np.array_equal(st.wsum, exp["wsum"]), i
        if "last_d" in exp:
            assert st.last_d == pytest.approx(exp["last_d"], rel=1e-14), i
        if "rep" in exp:
            assert np.array_equal(st.rep, exp["rep"]) and np.array_equal(st.order, exp["order"])
        if "fresh_load_post" in call:
            assert np.array_equal(O.plan(d, ids).load_post, call["fresh_load_post"])


def test_drift_replay_needs_home_above_target():
    """A kept replica takes pairs only while its expert's home rank is above
    its target. P=3 ranks of one home expert, R=1, K=1, 12 tokens, T = 4,
    no replan after the first call (delta = 1).

    Call 0 (c = [6, 3, 3]): expert 0 goes to rank 1 (least loaded, lower
    index of the tie) with min(4 - 3, 6) = 1 pair, then to rank 2 with
    min(4 - 3, 5) = 1 -> loads [4, 4, 4]; kept slots in order: 1, 2.
    Call 1 (c = [4, 2, 6]): rank 0 is at T, so neither replica takes
    anything even though rank 1 is below T -> loads [4, 2, 6], UNBALANCED.
    """
    d = O.make_dims(12, 1, 3, 3, 1, 4, cap=12)
    st = O.DriftState(3, 3, 1)
    prm = O.DriftParams(1, 1, 4, 1)
    c0 = np.array([0] * 6 + [1] * 3 + [2] * 3, np.int32).reshape(-1, 1)
    p0 = O.plan(d, c0, drift=(prm, st))
    assert p0.flags == O.ST_REPLANNED and np.array_equal(p0.load_post, [4, 4, 4])
    assert np.array_equal(p0.rep_expert.ravel(), [-1, 0, 0])
    assert np.array_equal(st.order, [1, 2, -1])
    c1 = np.array([0] * 4 + [1] * 2 + [2] * 6, np.int32).reshape(-1, 1)
    p1 = O.plan(d, c1, drift=(prm, st))
    assert p1.flags == O.ST_UNBALANCED
    assert np.array_equal(p1.load_post, [4, 2, 6])
    assert np.array_equal(p1.slot_quota, [[4, 0], [2, 0], [6, 0]])


@pytest.mark.parametrize("cap,tol,kept", [(12, (0, 0), True), (5, (0, 0), False),
                                           (12, (1, 2), True), (12, (1, 3), False)])
def test_drift_load_guard_hand_example(cap, tol, kept):
    """The load guard on the example above (T = 4; call 1 replays to loads
    [4, 2, 6]). Rank 2 ends at 6 rows: within a region of 12, not of 5; with
    tolerance 1/2 the limit is 4 * 3/2 = 6 (6 * 2 <= 4 * 3, kept at the
    boundary), with 1/3 it is 16/3 (6 * 3 > 4 * 4, guarded). Guarded, the
    greedy runs on c = [4, 2, 6]: rank 2 (x = +2) gives its home expert 2 to
    rank 1 (x = -2, the only rank below T) with min(4 - 2, 6) = 2 pairs ->
    loads [4, 4, 4], replica slots [-1, 2, -1]; the reference restarts at
    [4, 2, 6] and the state counts a second replan, one of them guarded."""
    d = O.make_dims(12, 1, 3, 3, 1, 4, cap=cap)
    st = O.DriftState(3, 3, 1)
    prm = O.DriftParams(1, 1, 4, 1, *tol)
    c0 = np.array([0] * 6 + [1] * 3 + [2] * 3, np.int32).reshape(-1, 1)
    assert O.plan(d, c0, drift=(prm, st)).flags == O.ST_REPLANNED
    c1 = np.array([0] * 4 + [1] * 2 + [2] * 6, np.int32).reshape(-1, 1)
    p1 = O.plan(d, c1, drift=(prm, st))
    if kept:
        assert p1.flags == O.ST_UNBALANCED
        assert np.array_equal(p1.load_post, [4, 2, 6])
        assert st.replans == 1 and st.guarded == 0 and st.nwin == 2
        assert np.array_equal(st.wsum, [10, 5, 9])
    else:
        assert p1.flags == O.ST_REPLANNED | O.ST_GUARDED
        assert np.array_equal(p1.load_post, [4, 4, 4])
        assert np.array_equal(p1.rep_expert.ravel(), [-1, 2, -1])
        assert np.array_equal(p1.slot_quota, [[4, 0], [2, 2], [4, 0]])
        assert st.replans == 2 and st.guarded == 1 and st.nwin == 1
        assert np.array_equal(st.wsum, [4, 2, 6])
        assert np.array_equal(st.rep, [-1, 2, -1]) and np.array_equal(st.order, [1, -1, -1])
        assert st.countdown == 1 and st.n_moves == 1
    C.check_layout(p1, c1, 3, 3, 1, cap)


def test_drift_load_guard_uses_each_ranks_own_target():
    """With speeds [1, 1, 2] the targets are ceil(12 s_r / 4) = [3, 3, 6].
    Call 0 (c = [9, 2, 1]): rank 0 gives expert 0 to rank 2 (x = -5) with
    min(6 - 1, 9) = 5, then to rank 1 (x = -1) with min(3 - 2, 4) = 1 ->
    loads [3, 3, 6]; kept slots in order: 2, 1.
    Call 1 (c = [5, 5, 2]): the slot on rank 2 takes min(6 - 2, 5) = 4
    (home 0 at 5 > 3, host at 2 < 6), the slot on rank 1 nothing (home now
    at 1) -> loads [1, 5, 6]. Rank 1 is 5/3 of its own target of 3 (and
    below the largest, 6): tolerance 1/4 guards it (5 * 4 > 3 * 5) and the
    greedy reaches [3, 3, 6] (expert 0 to rank 2 with 4 pairs, then rank 1,
    x = +2, gives expert 1 to rank 0, x = -2, with 2); without a tolerance
    the replay is kept, UNBALANCED."""
    d = O.make_dims(12, 1, 3, 3, 1, 4, cap=12)
    sp = np.array([1, 1, 2], np.int32)
    c0 = np.array([0] * 9 + [1] * 2 + [2], np.int32).reshape(-1, 1)
    c1 = np.array([0] * 5 + [1] * 5 + [2] * 2, np.int32).reshape(-1, 1)
    for tol in ((1, 4), (0, 0)):
        st = O.DriftState(3, 3, 1)
        prm = O.DriftParams(1, 1, 4, 1, *tol)
        p0 = O.plan(d, c0, speeds=sp, drift=(prm, st))
        assert p0.flags == O.ST_REPLANNED and np.array_equal(p0.load_post, [3, 3, 6])
        assert np.array_equal(st.order, [2, 1, -1])
        p1 = O.plan(d, c1, speeds=sp, drift=(prm, st))
        if tol[1]:
            assert p1.flags == O.ST_REPLANNED | O.ST_GUARDED
            assert np.array_equal(p1.load_post, [3, 3, 6])
            assert np.array_equal(p1.rep_expert.ravel(), [1, -1, 0])
        else:
            assert p1.flags == O.ST_UNBALANCED
            assert np.array_equal(p1.load_post, [1, 5, 6])


def test_drift_load_guard_adds_no_fatal_call():
    """drift_decode over its 60 passes with regions of S*K rows: a guarded
    call runs the same greedy as a fresh plan of that call, so the calls the
    gate leaves CAPACITY-fatal are among those a fresh greedy leaves fatal;
    with regions 5/4 S K and tolerance 1/4 no call is fatal. Checked on the
    first 30 passes (one popularity shift)."""
    wl = W.get_workload("drift_decode")
    for cap, tol in ((wl.tokens_per_rank * wl.top_k, (0, 0)),
                     (wl.tokens_per_rank * wl.top_k * 5 // 4, (1, 4))):
        d = O.dims_for(wl, cap=cap)
        st = O.DriftState(wl.n_experts, wl.n_ranks, wl.slots_per_rank)
        prm = O.DriftParams(*wl.drift[:4], *tol)
        for call in range(30):
            ids, _ = W.routing_for(wl, call)
            p = O.plan(d, ids, drift=(prm, st))
            if p.flags & O.ST_FATAL:
                assert tol == (0, 0) and O.plan(d, ids).flags & O.ST_CAPACITY, call
            assert p.status[2] <= cap or p.flags & O.ST_REPLANNED, call
            if tol[1] and not p.flags & O.ST_FATAL:
                assert p.status[2] * 4 <= 5 * p.status[1] or p.flags & O.ST_GUARDED, call


@pytest.mark.parametrize("H", [1, 3, 4])
def test_drift_replans_every_check_when_counts_are_orthogonal(H):
    """Each call sends every token to one expert, a different one each call:
    d = 1 at every check, so the greedy runs on the first call and at every
    H-th call after it; with delta = 1 (d never exceeds it) only the first
    call replans; with delta = 0 every check replans."""
    d = O.make_dims(32, 1, 8, 2, 1, 4, cap=32)
    seq = [np.full((32, 1), e % 8, np.int32) for e in range(13)]
    for num, den, expect in ((1, 20, [i for i in range(13) if i % H == 0]), (1, 1, [0]),
                             (0, 1, [i for i in range(13) if i % H == 0])):
        st = O.DriftState(8, 2, 1)
        prm = O.DriftParams(num, den, 100, H)
        got = [i for i, ids in enumerate(seq)
               if O.plan(d, ids, drift=(prm, st)).flags & O.ST_REPLANNED]
        assert got == expect, (num, den)
        assert st.replans == len(expect) and st.calls == 13


def test_drift_identical_calls_never_replan_and_match_mb_plan():
    """The same routing every call: d = 0 (to rounding) at every check, the
    placement is kept, and replaying it gives exactly the greedy's plan."""
    wl = W.get_workload("decode_drift")
    ids, _ = W.routing_for(wl, 3)
    d = O.dims_for(wl)
    ref = O.plan(d, ids)
    st = O.DriftState(wl.n_experts, wl.n_ranks, wl.slots_per_rank)
    prm = O.DriftParams(1, 1000, 8, 1)
    for i in range(5):
        p = O.plan(d, ids, drift=(prm, st))
        assert (p.flags & ~O.ST_REPLANNED) == ref.flags
        for key in ("load_post", "rep_expert", "slot_quota", "cu_seqlens", "pos", "row_src"):
            assert np.array_equal(getattr(p, key), getattr(ref, key)), (i, key)
        assert abs(st.last_d) <= 1e-15
    assert st.replans == 1 and st.nwin == 5


def test_drift_rejects_bad_params_and_keeps_state_on_bad_ids():
    d = O.make_dims(8, 1, 4, 2, 1, 4, cap=8)
    ids = np.zeros((8, 1), np.int32)
    for prm in ((1, 0, 2, 1), (-1, 2, 2, 1), (3, 2, 2, 1), (1, 2, 0, 1), (1, 2, 2, 0),
                (1, 2, 4097, 1), (1, 2, 2, 1, -1, 4), (1, 2, 2, 1, 1, -4)):
        st = O.DriftState(4, 2, 1)
        assert O.plan_drift_rc(d, ids, O.DriftParams(*prm), st) == O.ERR_INVALID_ARG, prm
    st = O.DriftState(4, 2, 1)
    prm = O.DriftParams(1, 2, 2, 1)
    O.plan(d, ids, drift=(prm, st))
    bad = ids.copy()
    bad[3] = 9
    p = O.plan(d, bad, drift=(prm, st))
    assert p.flags == O.ST_BAD_ID
    assert st.calls == 1 and st.replans == 1 and st.nwin == 1


def test_hand_example_repair():
    """Quota repair: P=2 ranks of 3 home experts, R=2, K=1, 16 tokens, T = 8.

    Sources: rank 0 sends e0 x3, e1, e2 x2, e3, e4; rank 1 sends e0 x2,
    e1 x4, e2 x2, so c = [5, 5, 4, 1, 1, 0] and L = [14, 2].
    Placement: rank 0 gives e0 (quota 5; ties with e1, lower id) to rank 1,
    m = min(8 - 2, 5) = 5 -> loads [9, 7]; then e1 (5) to rank 1's second
    slot, m = min(8 - 7, 5) = 1 -> loads [8, 8]. Quotas: e0 0 at home, 5 on
    rank 1; e1 4 at home, 1 on rank 1.
    Routing without repair: rank 0's 3 pairs of e0 go to rank 1 (rank 1
    keeps its own 2), rank 1's pairs of e1 beyond its quota (3) go to
    rank 0, rank 1's e2 pairs (2) and rank 0's e3, e4 (2) cross too:
    10 non-local pairs.
    Repair, the only pair (0, 1): both hold e0 and e1 (b's slots, homed on
    a). x_01(e0) = min(3 - 0, 5 - 2) = 3, x_10(e1) = min(4 - 1, 4 - 1) = 3,
    m = 3: e0's quota 3 moves to rank 0 (0 -> 3, 5 -> 2), e1's 3 to rank 1
    (4 -> 1, 1 -> 4). Loads stay [8, 8]; 6 pairs become local: 4 remain
    (e2 from rank 1, e3 and e4 from rank 0 have a single host), which is
    the least any routing with these hosts and loads can reach.
    """
    g = json.load(open(os.path.join(GOLDEN, "hand_example_repair.json")))
    d = O.make_dims(**g["dims"])
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    a = O.plan(d, ids)
    b = O.plan(d, ids, repair=True)
    for p, q, nl in ((a, "slot_quota_placed", "nonlocal_placed"),
                     (b, "slot_quota_repaired", "nonlocal_repaired")):
        assert np.array_equal(p.status, g["status"])
        assert np.array_equal(p.rep_expert, g["rep_expert"])
        assert np.array_equal(p.load_post, g["load_post"])
        assert np.array_equal(p.slot_quota, g[q]), q
        assert p.report["nonlocal_pairs"] == g[nl], nl
        C.check_layout(p, ids, d.n_ranks, d.n_experts, d.slots_per_rank, d.cap)
    assert _routing_lp_optimum(b, d) == g["nonlocal_best"]


def _routing_lp_optimum(p, d) -> int:
    """Zepp eq. (1) with a_ij = [i != j] over the plan's hosts, each rank's
    load fixed at the plan's (the quotas free): a transportation problem,
    solved by scipy's LP (its constraint matrix is totally unimodular, so
    the optimum is integral)."""
    from scipy.optimize import linprog

    P, E = d.n_ranks, d.n_experts
    eh = E // P
    hosts = [[e // eh] + [r for r in range(P) for j in range(d.slots_per_rank)
                          if p.rep_expert[r, j] == e] for e in range(E)]
    dm = p.counts
    var = [(i, e, j) for i in range(P) for e in range(E) if dm[i, e] > 0 for j in hosts[e]]
    if not var:
        return 0
    cost = np.array([0.0 if i == j else 1.0 for (i, e, j) in var])
    rows, rhs = [], []
    for i in range(P):
        for e in range(E):
            if dm[i, e] > 0:
                rows.append(np.array([1.0 if (v[0], v[1]) == (i, e) else 0.0 for v in var]))
                rhs.append(dm[i, e])
    for j in range(P):
        rows.append(np.array([1.0 if v[2] == j else 0.0 for v in var]))
        rhs.append(p.load_post[j])
    res = linprog(cost, A_eq=np.array(rows), b_eq=np.array(rhs, float), bounds=(0, None),
                  method="highs")
    assert res.status == 0
    return int(round(res.fun))


@pytest.mark.parametrize("P", list(range(1, 18)))
def test_circle_schedule(P):
    """The repair's tournament: n - 1 rounds (n = P rounded up to even) of
    disjoint pairs in which every two ranks meet exactly once (the round-
    robin of the circle method); an odd P leaves one rank a bye per round."""
    sch = O.circle_schedule(P)
    n = P + (P & 1)
    assert sch.shape == (max(n - 1, 0), n // 2, 2)
    met = set()
    for rnd in sch:
        seen = rnd.ravel().tolist()
        assert len(set(seen)) == len(seen) == n  # disjoint, everyone plays
        for a, b in rnd:
            if a < P and b < P:
                key = (min(a, b), max(a, b))
                assert key not in met
                met.add(key)
    assert len(met) == P * (P - 1) // 2


def _repair_checks(d, ids, speeds=None):
    a = O.plan(d, ids, speeds=speeds)
    b = O.plan(d, ids, speeds=speeds, repair=True)
    assert b.flags == a.flags and np.array_equal(b.rep_expert, a.rep_expert)
    assert np.array_equal(b.load_post, a.load_post)  # loads never change
    Q = C.quotas_matrix(b, d.n_experts, d.n_ranks)
    assert np.array_equal(Q.sum(1), a.counts.sum(0))  # nor expert totals
    assert np.all(Q >= 0)
    if not b.flags & O.ST_CAPACITY:
        C.check_layout(b, ids, d.n_ranks, d.n_experts, d.slots_per_rank, d.cap)
    # routing stays optimal for the repaired quotas, and never gets worse
    assert b.report["nonlocal_pairs"] == C.transport_nonlocal_optimum(b.counts, Q)
    assert b.report["nonlocal_pairs"] <= a.report["nonlocal_pairs"]
    return a, b


@pytest.mark.parametrize("name", ["tiny", "mixtral", "decode_drift"])
def test_repair_on_workloads(name):
    """On the workloads (tokens routed independently of their rank) the
    greedy leaves no opposite flows on experts two ranks share: the repair
    changes nothing, and the routing is already the best these hosts and
    loads allow (tiny, mixtral)."""
    wl, ids, w, d, _ = _plan_workload(name)
    a, b = _repair_checks(d, ids)
    assert np.array_equal(a.slot_quota, b.slot_quota)
    if name != "decode_drift":
        assert a.report["nonlocal_pairs"] == _routing_lp_optimum(a, d)


def test_repair_on_pattern_inputs():
    """Inputs built so that rank pairs hold opposite flows: the repair cancels
    them and never moves a load. Against the routing optimum over the plan's
    hosts and loads (scipy LP, cases up to 8 ranks) it never goes below it,
    and reaches it when a single pattern pair is planted; with several, the
    greedy can interleave their replicas into cycles over three or more
    ranks, which pairwise cancellation cannot undo."""
    from tests.crafted import repair_cases, repair_pattern_ids

    fired = 0
    for P, pairs, R, seed in repair_cases():
        ids = repair_pattern_ids(P, pairs, seed)
        d = O.make_dims(8 * P, 1, 3 * P, P, R, 16, cap=16)
        a, b = _repair_checks(d, ids)
        fired += b.report["nonlocal_pairs"] < a.report["nonlocal_pairs"]
        if P <= 8:
            opt = _routing_lp_optimum(b, d)
            assert b.report["nonlocal_pairs"] >= opt
            if len(pairs) == 1:
                assert b.report["nonlocal_pairs"] == opt
    assert fired >= 20


SMALL = ["tiny", "mixtral", "decode_drift"]


@pytest.mark.parametrize("name", SMALL)
def test_invariants_small_workloads(name):
    wl, ids, w, d, p = _plan_workload(name)
    dmat = C.check_counts(p, ids, wl.n_ranks, wl.n_experts)
    assert p.status[1] == wl.tokens_per_rank * wl.top_k  # pi2: T = S*K
    assert p.flags & O.ST_FATAL == 0
    if not p.flags & O.ST_UNBALANCED:
        assert p.load_post.max() <= p.status[1]  # pi4
    C.check_layout(p, ids, wl.n_ranks, wl.n_experts, wl.slots_per_rank, d.cap)
    Q = C.quotas_matrix(p, wl.n_experts, wl.n_ranks)
    assert p.report["nonlocal_pairs"] == C.transport_nonlocal_optimum(dmat, Q)  # pi7
    T = int(p.status[1])
    assert p.report["offhome_pairs"] >= int(np.maximum(p.load_pre - T, 0).sum())  # pi6
    assert p.report["ir_before"] == pytest.approx(C.rank_imbalance(p.load_pre))
    assert p.report["ir_after"] == pytest.approx(C.rank_imbalance(p.load_post))
    assert p.report["maxvio"] == pytest.approx(C.maxvio(dmat.sum(0)))
    assert p.status[3] <= wl.n_ranks * wl.slots_per_rank


@pytest.mark.parametrize("name", ["dsv3_prefill", "kimi_prefill"] + W.configs.SWEEP_ORDER)
def test_invariants_prefill_plans(name):
    """Full-size plans (0.5-1 M pairs) of the prefill and maxvio-sweep workloads."""
    wl, ids, w, d, p = _plan_workload(name)
    dmat = C.check_counts(p, ids, wl.n_ranks, wl.n_experts)
    assert p.flags == 0
    assert p.load_post.max() <= p.status[1] == wl.cap
    # vectorised conservation (the per-slot loop is too slow at this size)
    pos = p.pos.ravel().astype(np.int64)
    assert np.unique(pos).size == pos.size
    assert np.array_equal(p.row_src[pos], np.repeat(np.arange(wl.n_tokens), wl.top_k))
    assert np.array_equal(np.diff(p.cu_seqlens, axis=1), p.slot_quota)
    Q = C.quotas_matrix(p, wl.n_experts, wl.n_ranks)
    assert np.array_equal(Q.sum(1), dmat.sum(0))
    assert p.report["nonlocal_pairs"] == C.transport_nonlocal_optimum(dmat, Q)


def test_dsv3_prefill_balance_target():
    """Post-plan rank imbalance at most 1.01 on the DeepSeek-V3-like prefill."""
    wl, ids, w, d, p = _plan_workload("dsv3_prefill")
    assert p.report["ir_after"] <= 1.01


@pytest.mark.parametrize("name", W.configs.SWEEP_ORDER)
def test_maxvio_sweep_holds_s_times_k(name):
    """MoonEP's invariant at every skew of its sweep: with two replica slots
    every rank receives exactly S*K rows; the reported maxvio is the routing's
    (pairs per expert over their mean, minus one)."""
    wl, ids, w, d, p = _plan_workload(name)
    c = np.bincount(ids.ravel(), minlength=wl.n_experts)
    assert p.report["maxvio"] == pytest.approx(c.max() / c.mean() - 1.0)
    assert np.all(p.load_post == wl.cap)
    assert p.report["ir_after"] == 1.0


def test_maxvio_sweep_one_slot_breaks_at_high_skew():
    """With one replica slot per rank the S*K regions overflow at maxvio 10
    (UNBALANCED and CAPACITY), which is why the sweep uses two."""
    wl = W.get_workload("moonep_maxvio_10")
    ids, _ = W.routing_for(wl)
    d = O.make_dims(wl.n_tokens, wl.top_k, wl.n_experts, wl.n_ranks, 1, wl.hidden,
                    dtype_in=wl.dtype_in, dtype_out=wl.dtype_out)
    p = O.plan(d, ids)
    assert p.flags == O.ST_UNBALANCED | O.ST_CAPACITY
    assert p.status[2] > wl.cap


def test_decode_drift_sequence_invariants():
    """All 61 layer calls of the decode sequence plan within T, stateless."""
    wl = W.get_workload("decode_drift")
    d = O.dims_for(wl)
    irs = []
    for call in range(wl.calls):
        ids, _ = W.routing_for(wl, call)
        p = O.plan(d, ids)
        assert p.flags == 0
        assert p.load_post.max() <= wl.cap
        C.check_counts(p, ids, wl.n_ranks, wl.n_experts)
        irs.append(p.report["ir_before"])
    assert min(irs) > 1.5  # fresh popularity every call keeps the skew high


# ---- closed forms -------------------------------------------------------------

def _stable_ep_positions(ids, n_ranks, n_experts, cap):
    """Plain expert parallelism: pairs sorted stably by expert id (numpy
    stable argsort), each rank's home experts in its own region."""
    n, k = ids.shape
    flat = ids.ravel().astype(np.int64)
    order = np.argsort(flat, kind="stable")
    rank_in_sorted = np.empty_like(order)
    rank_in_sorted[order] = np.arange(order.size)
    eh = n_experts // n_ranks
    home = flat // eh
    load = np.bincount(home, minlength=n_ranks)
    start = np.concatenate([[0], np.cumsum(load)[:-1]])
    return (home * cap + rank_in_sorted - start[home]).reshape(n, k), load


@pytest.mark.parametrize("name", SMALL)
def test_r0_is_plain_expert_parallelism(name):
    """pi9: with no replica slots the layout is a stable sort by expert."""
    wl = W.get_workload(name)
    ids, _ = W.routing_for(wl)
    cap = wl.n_tokens * wl.top_k  # large enough for any rank
    d = O.make_dims(wl.n_tokens, wl.top_k, wl.n_experts, wl.n_ranks, 0, wl.hidden, cap=cap,
                    dtype_in=wl.dtype_in, dtype_out=wl.dtype_out)
    p = O.plan(d, ids)
    exp_pos, load = _stable_ep_positions(ids, wl.n_ranks, wl.n_experts, cap)
    assert np.array_equal(p.pos, exp_pos)
    assert p.status[3] == 0
    assert np.array_equal(p.load_post, load)
    eh = wl.n_experts // wl.n_ranks
    cnt = np.bincount(ids.ravel(), minlength=wl.n_experts).reshape(wl.n_ranks, eh)
    assert np.array_equal(p.cu_seqlens[:, 1:], np.cumsum(cnt, axis=1))
    assert bool(p.flags & O.ST_UNBALANCED) == bool(load.max() > p.status[1])
    assert not p.flags & O.ST_CAPACITY


def test_r0_default_cap_skewed_is_capacity():
    """R=0 under skew with cap = S*K: UNBALANCED and CAPACITY, nothing laid out."""
    wl = W.get_workload("mixtral")
    ids, _ = W.routing_for(wl)
    d = O.make_dims(wl.n_tokens, wl.top_k, wl.n_experts, wl.n_ranks, 0, wl.hidden)
    p = O.plan(d, ids)
    assert p.flags == O.ST_UNBALANCED | O.ST_CAPACITY
    assert np.all(p.pos == -1)


@pytest.mark.parametrize("P,S,eh,R", [(4, 16, 4, 1), (8, 32, 1, 1), (16, 8, 2, 3), (64, 4, 4, 1)])
def test_all_tokens_one_expert(P, S, eh, R):
    """pi10: K=1, every token routed to expert 0, R >= 1. The busiest rank
    sheds S pairs per move to ranks 1..P-1 in index order (all tie at load
    0): P-1 moves, every rank serves exactly the S tokens originating on it,
    so token t lands on row (t/S)*cap + t%S."""
    N, E = P * S, P * eh
    ids = np.zeros((N, 1), np.int32)
    d = O.make_dims(N, 1, E, P, R, 8)
    p = O.plan(d, ids)
    t = np.arange(N)
    assert p.flags == 0
    assert p.status[3] == P - 1
    assert np.array_equal(p.pos.ravel(), (t // S) * d.cap + t % S)
    assert np.all(p.load_post == S)
    assert np.array_equal(p.rep_expert[1:, 0], np.zeros(P - 1))
    assert p.report["nonlocal_pairs"] == 0


@pytest.mark.parametrize("P,S,eh,K", [(4, 16, 4, 2), (8, 8, 2, 4), (2, 6, 3, 6), (1, 10, 5, 3)])
def test_uniform_loads_need_no_moves(P, S, eh, K):
    """pi11: ids[t][k] = (t*K + k) mod E loads every rank exactly T: no move,
    and the layout is the plain stable sort of pi9."""
    N, E = P * S, P * eh
    t = np.arange(N)[:, None]
    ids = ((t * K + np.arange(K)[None, :]) % E).astype(np.int32)
    assert (N * K) % E == 0
    d = O.make_dims(N, K, E, P, 2, 8)
    p = O.plan(d, ids)
    assert p.flags == 0 and p.status[3] == 0
    exp_pos, _ = _stable_ep_positions(ids, P, E, d.cap)
    assert np.array_equal(p.pos, exp_pos)
    assert p.report["ir_before"] == 1.0 and p.report["ir_after"] == 1.0


def test_k_equals_e_and_single_rank():
    """K = E (every token routes to every expert) and P = 1 are balanced."""
    for (P, E, K, S) in [(4, 8, 8, 4), (1, 6, 2, 10), (3, 3, 1, 5)]:
        N = P * S
        ids, _ = W.routing(N, E, K, 0, 1.0, 1.0, 77)
        d = O.make_dims(N, K, E, P, 1, 8)
        p = O.plan(d, ids)
        C.check_counts(p, ids, P, E)
        C.check_layout(p, ids, P, E, 1, d.cap)
        if K == E or P == 1:
            assert p.status[3] == 0
        assert p.load_post.max() <= p.status[1]


def test_empty_input():
    d = O.make_dims(0, 2, 8, 4, 1, 8, cap=1)
    p = O.plan(d, np.zeros((0, 2), np.int32))
    assert np.array_equal(p.status, [0, 0, 0, 0])
    assert np.all(p.cu_seqlens == 0) and np.all(p.row_src == -1)


# ---- error paths ----------------------------------------------------------------

def test_bad_and_duplicate_ids_flagged():
    d = O.make_dims(8, 2, 4, 2, 1, 8)
    ids = np.array([[0, 1]] * 8, np.int32)
    ids[3, 1] = 4
    assert O.plan(d, ids).flags == O.ST_BAD_ID
    ids[3, 1] = -1
    assert O.plan(d, ids).flags == O.ST_BAD_ID
    ids[3, 1] = 0
    assert O.plan(d, ids).flags == O.ST_DUP_ID
    ids[5, 0] = 9
    assert O.plan(d, ids).flags == O.ST_DUP_ID | O.ST_BAD_ID


@pytest.mark.parametrize("args", [
    (7, 2, 4, 2, 1, 8),    # N % P
    (8, 2, 5, 2, 1, 8),    # E % P
    (8, 5, 4, 2, 1, 8),    # K > E
    (8, 0, 4, 2, 1, 8),    # K = 0
    (8, 2, 4, 2, -1, 8),   # R < 0
    (8, 2, 4, 0, 1, 8),    # P = 0
])
def test_invalid_sizes_rejected(args):
    d = O.make_dims(*args, cap=max(1, args[0]))
    assert O.plan_rc(d, np.zeros(max(args[0] * max(args[1], 1), 1), np.int32)) == O.ERR_INVALID_ARG


def test_capacity_when_cap_below_balanced_load():
    wl = W.get_workload("tiny")
    ids, _ = W.routing_for(wl)
    d = O.dims_for(wl, cap=wl.cap - 1)
    p = O.plan(d, ids)
    assert p.flags & O.ST_CAPACITY
    assert np.all(p.pos == -1)


# ---- locality: brute force over every M and scipy milp ---------------------------

def _compositions(n, parts):
    if parts == 1:
        yield (n,)
        return
    for i in range(n + 1):
        for rest in _compositions(n - i, parts - 1):
            yield (i,) + rest


def _brute_force_nonlocal(d: np.ndarray, Q: np.ndarray) -> int:
    """Zepp eq. (1), a_ij = [i != j], C = 0: enumerate every non-negative
    integer M^e with row sums d_i^e and column sums q_j^e."""
    P, E = d.shape
    total = 0
    for e in range(E):
        best = None
        rows = [list(_compositions(int(d[i, e]), P)) for i in range(P)]
        for M in itertools.product(*rows):
            M = np.array(M)
            if not np.array_equal(M.sum(0), Q[e]):
                continue
            cost = int(M.sum() - np.trace(M))
            best = cost if best is None else min(best, cost)
        assert best is not None
        total += best
    return total


@pytest.mark.parametrize("seed", range(6))
def test_locality_brute_force_micro(seed):
    """pi7 on micro inputs (N <= 8, E <= 4, P <= 2): the oracle's non-local
    count equals the true optimum of the locality ILP for its quotas."""
    rng = np.random.default_rng(seed)
    P, E, K, N, R = 2, 4, 2, 8, 1
    ids = np.stack([rng.choice(E, size=K, replace=False, p=[0.55, 0.25, 0.15, 0.05])
                    for _ in range(N)]).astype(np.int32)
    d = O.make_dims(N, K, E, P, R, 8)
    p = O.plan(d, ids)
    dm = C.check_counts(p, ids, P, E)
    Q = C.quotas_matrix(p, E, P)
    assert p.report["nonlocal_pairs"] == _brute_force_nonlocal(dm, Q)
    assert _brute_force_nonlocal(dm, Q) == C.transport_nonlocal_optimum(dm, Q)


def test_locality_milp_tiny():
    """pi7 on the tiny workload: scipy's MILP solver on Zepp eq. (1)
    (a_ij = [i != j], C = 0, q = the oracle's quotas) finds the oracle's
    non-local count."""
    from scipy.optimize import LinearConstraint, milp

    wl, ids, w, d, p = _plan_workload("tiny")
    P, E = wl.n_ranks, wl.n_experts
    dm = p.counts.astype(np.int64)
    Q = C.quotas_matrix(p, E, P)
    total = 0
    for e in range(E):
        cost = np.array([0.0 if i == j else 1.0 for i in range(P) for j in range(P)])
        A_row = np.zeros((P, P * P))
        A_col = np.zeros((P, P * P))
        for i in range(P):
            for j in range(P):
                A_row[i, i * P + j] = 1
                A_col[j, i * P + j] = 1
        cons = [LinearConstraint(A_row, dm[:, e], dm[:, e]), LinearConstraint(A_col, Q[e], Q[e])]
        res = milp(cost, constraints=cons, integrality=np.ones(P * P))
        assert res.success
        total += int(round(res.fun))
    assert total == p.report["nonlocal_pairs"]


# ---- exhaustive placements on the tiny workload ------------------------------------

def _min_max_load(c: np.ndarray, hosts: list[list[int]], P: int) -> int:
    """Smallest achievable max rank load for a placement: by max-flow/min-cut
    on expert -> host -> sink, it is max over rank sets U of
    ceil(sum of c_e over experts whose hosts all lie in U / |U|)."""
    best = 0
    for mask in range(1, 1 << P):
        size = bin(mask).count("1")
        dem = sum(int(c[e]) for e, hs in enumerate(hosts) if all((mask >> h) & 1 for h in hs))
        best = max(best, -(-dem // size))
    return best


def test_exhaustive_placements_tiny():
    """pi8: over all 13^4 single-slot placements of the tiny workload, the
    best achievable max load is the lower bound the greedy is measured
    against; the greedy's own max load is feasible (>= that bound) and its
    gap is reported."""
    wl, ids, w, d, p = _plan_workload("tiny")
    P, E = wl.n_ranks, wl.n_experts
    eh = E // P
    c = p.counts.sum(0)
    home = [[e // eh] for e in range(E)]
    # vectorised: demand of each rank set for each placement
    options = [[-1] + [e for e in range(E) if e // eh != r] for r in range(P)]
    best = None
    for pl in itertools.product(*options):
        hosts = [list(h) for h in home]
        for r, e in enumerate(pl):
            if e >= 0:
                hosts[e].append(r)
        v = _min_max_load(c, hosts, P)
        best = v if best is None else min(best, v)
        if best == int(p.status[1]):
            break  # cannot beat the water level
    greedy = int(p.load_post.max())
    own = [list(h) for h in home]
    for r in range(P):
        for e in p.rep_expert[r]:
            if e >= 0:
                own[e].append(r)
    assert greedy >= _min_max_load(c, own, P) >= best >= int(p.status[1])
    print(f"tiny: greedy max load {greedy}, best over all placements {best}")


def test_exhaustive_locality_tiny():
    """pi8's locality half: over all 13^4 single-slot placements of the tiny
    workload that can reach max load T, the fewest non-local pairs any
    routing with loads <= T achieves (scipy LP per placement: a
    transportation problem, so integral). The greedy (with or without the
    quota repair) is feasible, so it cannot beat that; the gap is reported."""
    from scipy.optimize import linprog

    wl, ids, w, d, p = _plan_workload("tiny")
    P, E = wl.n_ranks, wl.n_experts
    eh, T, dm = E // P, int(p.status[1]), p.counts
    c = dm.sum(0)
    home = [[e // eh] for e in range(E)]
    best = None
    for pl in itertools.product(*[[-1] + [e for e in range(E) if e // eh != r] for r in range(P)]):
        hosts = [list(h) for h in home]
        for r, e in enumerate(pl):
            if e >= 0:
                hosts[e].append(r)
        if _min_max_load(c, hosts, P) > T:
            continue
        var = [(i, e, j) for i in range(P) for e in range(E) if dm[i, e] > 0 for j in hosts[e]]
        cost = [0.0 if i == j else 1.0 for (i, e, j) in var]
        a_eq = [[1.0 if (v[0], v[1]) == (i, e) else 0.0 for v in var]
                for i in range(P) for e in range(E) if dm[i, e] > 0]
        b_eq = [dm[i, e] for i in range(P) for e in range(E) if dm[i, e] > 0]
        a_ub = [[1.0 if v[2] == j else 0.0 for v in var] for j in range(P)]
        res = linprog(cost, A_ub=a_ub, b_ub=[T] * P, A_eq=a_eq, b_eq=b_eq, bounds=(0, None),
                      method="highs")
        if res.status == 0 and (best is None or res.fun < best):
            best = int(round(res.fun))
    greedy = p.report["nonlocal_pairs"]
    repaired = O.plan(d, ids, repair=True).report["nonlocal_pairs"]
    assert p.flags == 0 and greedy >= best and repaired >= best
    print(f"tiny: non-local pairs greedy {greedy}, repaired {repaired}, best over placements {best}")


# ---- report formulas -------------------------------------------------------------

def test_excess_removed_reproduces_iser_e1_table():
    """pi12: excess removed = (IR_before - IR_after) / (IR_before - 1) gives
    the percentages of ISER-MoE's E1 table from its two IR rows."""
    before = [1.20, 1.44, 1.84, 2.24]
    after = [1.002, 1.006, 1.010, 1.020]
    printed = [99.0, 98.6, 98.8, 98.4]
    for b, a, pct in zip(before, after, printed):
        assert round(100 * (b - a) / (b - 1), 1) == pytest.approx(pct, abs=0.05)


def test_report_by_hand_tiny():
    wl, ids, w, d, p = _plan_workload("tiny")
    c = np.bincount(ids.ravel(), minlength=wl.n_experts)
    L = c.reshape(wl.n_ranks, -1).sum(1)
    mean = wl.n_tokens * wl.top_k / wl.n_ranks
    assert p.report["ir_before"] == pytest.approx(L.max() / mean)
    assert p.report["maxvio"] == pytest.approx(c.max() / c.mean() - 1)
    ira = p.load_post.max() / mean
    assert p.report["excess_removed"] == pytest.approx((L.max() / mean - ira) / (L.max() / mean - 1))
    assert p.report["excess_before"] == int(np.maximum(L - p.status[1], 0).sum())


# ---- dispatch and combine -----------------------------------------------------------

@pytest.mark.parametrize("name", SMALL)
def test_dispatch_is_row_scatter(name):
    """O5 equals numpy fancy assignment buf[pos] = repeat(x, K)."""
    wl, ids, w, d, p = _plan_workload(name)
    x, xs = W.token_rows(wl)
    buf, bs, rc = O.dispatch(d, p, x, xs)
    assert rc == 0
    rb = O.row_bytes_in(d)
    exp = np.zeros((wl.n_ranks * d.cap, rb), np.uint8)
    exp[p.pos.ravel()] = np.repeat(x.view(np.uint8).reshape(wl.n_tokens, rb), wl.top_k, axis=0)
    assert np.array_equal(buf, exp)
    if xs is not None:
        exps = np.zeros((wl.n_ranks * d.cap, wl.hidden // 128), np.float32)
        exps[p.pos.ravel()] = np.repeat(xs, wl.top_k, axis=0)
        assert np.array_equal(bs, exps)
    # a window gives the same rows
    r0, r1 = d.cap, 3 * d.cap
    win, _, _ = O.dispatch(d, p, x, xs, row0=r0, row1=r1)
    assert np.array_equal(win, exp[r0:r1])


def _y_exp_for(wl, d, seed_shift=0):
    rows = wl.n_ranks * d.cap
    if wl.dtype_out == "f32":
        return W.rows_f32(wl.seed + seed_shift, W.TAG_YEXP, wl.hidden, n=rows)
    return W.rows_bf16(wl.seed + seed_shift, W.TAG_YEXP, wl.hidden, n=rows)


@pytest.mark.parametrize("name", ["tiny", "mixtral"])
def test_combine_matches_numpy(name):
    """O6 equals sum_k w[:,k] * y_exp[pos[:,k]] evaluated by numpy in float64."""
    wl, ids, w, d, p = _plan_workload(name)
    ye = _y_exp_for(wl, d)
    yf = ye if wl.dtype_out == "f32" else W.bf16_bits_to_f32(ye)
    y, mag, rc = O.combine(d, p.pos, p.status, w, ye)
    g = yf.astype(np.float64)[p.pos]  # [N, K, H]
    exp = np.einsum("nk,nkh->nh", w.astype(np.float64), g)
    np.testing.assert_allclose(y, exp, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mag, np.einsum("nk,nkh->nh", np.abs(w.astype(np.float64)), np.abs(g)),
                               rtol=1e-12, atol=1e-12)
    # a token sub-range gives the same values
    y2, _, _ = O.combine(d, p.pos, p.status, w, ye, t0=5, t1=9)
    assert np.array_equal(y2, y[5:9])


def test_combine_round_trip_identity_experts():
    """pi14: identity experts (y_exp = dispatched x) and one-hot weights give
    x back exactly; weights summing to 1 give x within the weights' own
    rounding."""
    wl, ids, w, d, p = _plan_workload("tiny")
    x, _ = W.token_rows(wl)
    buf, _, _ = O.dispatch(d, p, x)
    ye = buf.view(np.float32).reshape(-1, wl.hidden)
    onehot = np.zeros_like(w)
    onehot[np.arange(wl.n_tokens), np.arange(wl.n_tokens) % wl.top_k] = 1.0
    y, _, _ = O.combine(d, p.pos, p.status, onehot, ye)
    assert np.array_equal(y, x.astype(np.float64))
    y, _, _ = O.combine(d, p.pos, p.status, w, ye)
    wsum = w.astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(y, x.astype(np.float64) * wsum, rtol=1e-15, atol=1e-15)
    assert np.all(np.abs(wsum - 1) < 1e-6)


def test_e4m3_decode_matches_torch():
    """The oracle's OCP e4m3fn decode equals torch's float8_e4m3fn on all 256
    codes (subnormals, the largest value 448, NaN)."""
    import torch

    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([O.e4m3_value(b) for b in range(256)])
    assert np.array_equal(mine, ref, equal_nan=True)
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


def test_combine_fp8_matches_numpy():
    """The dequantising combine equals numpy in float64: torch's e4m3 decode
    times the row's scale of each 128-element block, weighted and summed."""
    import torch

    wl = W.get_workload("decode_drift")
    P, K, E, H = 8, 3, 16, 384
    N, cap = 64, 64
    ids, w = W.routing(N, E, K, W.NOISE_GUMBEL, 1.1, 1.0, 321)
    d = O.make_dims(N, K, E, P, 1, H, cap=cap, dtype_in="fp8", dtype_out="bf16")
    p = O.plan(d, ids)
    assert p.flags == 0
    rows = P * cap
    q, sc, _ = W.rows_fp8(wl.seed, W.TAG_YEXP, H, n=rows)
    y, mag, rc = O.combine_fp8(d, p.pos, p.status, w, q, sc)
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    deq = deq * np.repeat(sc.astype(np.float64), 128, axis=1)
    terms = w.astype(np.float64)[:, :, None] * deq[p.pos]
    assert rc == 0
    assert np.allclose(y, terms.sum(1), rtol=1e-13, atol=1e-12)
    assert np.allclose(mag, np.abs(terms).sum(1), rtol=1e-13, atol=1e-12)


def test_combine_fp8_round_trip():
    """fp8 rows dispatched with their scales and combined with one-hot
    weights come back as their exact dequantisation q * scale."""
    wl = W.get_workload("decode_drift")
    ids, w = W.routing_for(wl, 5)
    d = O.dims_for(wl)
    d.hidden = 256
    x, xs, _ = W.rows_fp8(wl.seed, W.TAG_X, 256, n=wl.n_tokens)
    p = O.plan(d, ids)
    buf, bs, _ = O.dispatch(d, p, x, xs)
    onehot = np.zeros_like(w)
    onehot[:, 2] = 1.0
    y, _, _ = O.combine_fp8(d, p.pos, p.status, onehot, buf, bs, 0, 512)
    exp = np.array([[O.e4m3_value(b) for b in row] for row in x[:512, :]]) * \
        np.repeat(xs[:512].astype(np.float64), 128, axis=1)
    assert np.array_equal(y, exp)


def test_fatal_status_skips_dispatch_and_combine():
    wl, ids, w, d, p = _plan_workload("tiny")
    x, _ = W.token_rows(wl)
    st = p.status.copy()
    st[0] = O.ST_CAPACITY
    _, _, rc = O.dispatch(d, p._replace(status=st) if hasattr(p, "_replace") else
                          O.Plan(**{**p.__dict__, "status": st}), x)
    assert rc == 1
    _, _, rc = O.combine(d, p.pos, st, w, _y_exp_for(wl, d))
    assert rc == 1
