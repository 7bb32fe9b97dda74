"""Property checks on a plan, shared by the oracle pins and the GPU parity
tests. Each check restates a fact the pages fix (conservation, the water
level, the S*K regions, the slot layout) using numpy library routines, never
the oracle's own loops.

A plan here is any object with numpy attributes counts, load_pre, load_post,
rep_expert, slot_quota, cu_seqlens, pos, row_src and status.
"""
from __future__ import annotations

import numpy as np


def slot_expert_table(rep_expert: np.ndarray, n_experts: int, n_ranks: int) -> np.ndarray:
    """Expert held by local slot i of rank h: home experts by id, then the
    replica slots (MoonEP, "Implementation details": [E+B, H, H'] numbering)."""
    eh = n_experts // n_ranks
    home = np.arange(n_experts, dtype=np.int64).reshape(n_ranks, eh)
    return np.concatenate([home, rep_expert.astype(np.int64)], axis=1)


def check_counts(p, ids: np.ndarray, n_ranks: int, n_experts: int):
    """pi1: d[s][e] equals a bincount of each source rank's ids; totals N*K."""
    n, k = ids.shape
    s = n // n_ranks
    src = np.repeat(np.arange(n) // s, k)
    d = np.bincount(src * n_experts + ids.ravel().astype(np.int64),
                    minlength=n_ranks * n_experts).reshape(n_ranks, n_experts)
    assert np.array_equal(p.counts, d)
    c = d.sum(0)
    eh = n_experts // n_ranks
    assert np.array_equal(p.load_pre, c.reshape(n_ranks, eh).sum(1))
    assert int(p.load_pre.sum()) == n * k
    return d


def check_layout(p, ids: np.ndarray, n_ranks: int, n_experts: int, slots: int, cap: int):
    """pi3, pi5, pi13: every pair has exactly one row, in its rank's region,
    inside a slot holding its own expert; rows of a slot ascend in token
    index; rows per slot equal the slot quota; quotas of an expert add up to
    its routed count; row_src inverts pos and marks the rest -1."""
    n, k = ids.shape
    eh = n_experts // n_ranks
    ns = eh + slots
    pos = p.pos.astype(np.int64).ravel()
    # one row per pair, all distinct, inside [0, P*cap)
    assert pos.min(initial=0) >= 0 and (pos.size == 0 or pos.max() < n_ranks * cap)
    assert np.unique(pos).size == pos.size
    tok = np.repeat(np.arange(n), k)
    rs = p.row_src.astype(np.int64)
    assert np.array_equal(rs[pos], tok)
    mask = np.ones(n_ranks * cap, bool)
    mask[pos] = False
    assert np.all(rs[mask] == -1)
    # cu_seqlens is the running sum of the slot quotas, per rank
    cu = p.cu_seqlens.astype(np.int64)
    assert cu.shape == (n_ranks, ns + 1)
    assert np.all(cu[:, 0] == 0)
    assert np.array_equal(np.diff(cu, axis=1), p.slot_quota)
    assert np.array_equal(cu[:, -1], p.load_post)
    # the slot each row falls in, and its expert
    h = pos // cap
    off = pos - h * cap
    assert np.all(off < cu[h, -1])
    slot = np.array([np.searchsorted(cu[hh], oo, side="right") - 1 for hh, oo in zip(h, off)],
                    dtype=np.int64) if pos.size else np.zeros(0, np.int64)
    table = slot_expert_table(p.rep_expert, n_experts, n_ranks)
    assert np.array_equal(table[h, slot], ids.ravel().astype(np.int64))
    # rows per slot equal the quota
    rows = np.bincount(h * ns + slot, minlength=n_ranks * ns).reshape(n_ranks, ns)
    assert np.array_equal(rows, p.slot_quota)
    # quotas of each expert add up to its routed count
    c = np.bincount(ids.ravel(), minlength=n_experts)
    qsum = np.bincount(table.ravel()[table.ravel() >= 0],
                       weights=p.slot_quota.ravel()[table.ravel() >= 0],
                       minlength=n_experts).astype(np.int64)
    assert np.array_equal(qsum, c)
    # rows inside a slot ascend in token index
    for hh in range(n_ranks):
        for i in range(ns):
            seg = rs[hh * cap + cu[hh, i]: hh * cap + cu[hh, i + 1]]
            assert np.all(np.diff(seg) > 0)
    # a replica is never a second copy on the same rank
    for hh in range(n_ranks):
        held = table[hh][table[hh] >= 0]
        assert np.unique(held).size == held.size
    return h


def quotas_matrix(p, n_experts: int, n_ranks: int) -> np.ndarray:
    """Q[e][h]: rows rank h serves for expert e."""
    table = slot_expert_table(p.rep_expert, n_experts, n_ranks)
    Q = np.zeros((n_experts, n_ranks), np.int64)
    for h in range(n_ranks):
        for i, e in enumerate(table[h]):
            if e >= 0:
                Q[e, h] += p.slot_quota[h, i]
    return Q


def transport_nonlocal_optimum(d: np.ndarray, Q: np.ndarray) -> int:
    """Closed-form optimum of Zepp eq. (1) with a_ij = [i != j], C = 0 and
    q = Q: per expert, the most pairs that can stay local is
    sum_h min(d[h][e], Q[e][h]), the rest must move."""
    c = d.sum(0)
    keep = np.minimum(d.T, Q).sum(1)
    return int((c - keep).sum())


def rank_imbalance(loads: np.ndarray) -> float:
    """ISER-MoE Background: max / mean routed pairs per rank."""
    m = loads.mean()
    return float(loads.max() / m) if m > 0 else 1.0


def maxvio(c: np.ndarray) -> float:
    """MoonEP "Variables and core terms": max_e (T_e / mean T) - 1."""
    m = c.mean()
    return float(c.max() / m - 1.0) if m > 0 else 0.0
