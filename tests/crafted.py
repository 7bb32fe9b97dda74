"""Routing inputs built to a pattern, for tests of the quota repair.

Each listed pair (a, b) of ranks follows the pattern of the hand-derived
repair example (rank a: 3 home experts with 5, 5 and 4 routed pairs, rank b
with 2): the greedy gives b replicas of two of a's experts, one holding all
of its quota and one a single pair, so a's and b's own tokens of those two
experts cross in opposite directions. Every other rank routes its 8 tokens
to one of its own 3 experts. K = 1, 8 tokens per rank, 3 experts per rank.
"""
from __future__ import annotations

import numpy as np


def repair_pattern_ids(n_ranks: int, pairs: list[tuple[int, int]], seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    src = {}
    for a, b in pairs:
        ea = [3 * a + i for i in range(3)]
        eb = [3 * b + i for i in range(3)]
        src[a] = [ea[0]] * 3 + [ea[1]] + [ea[2]] * 2 + [eb[0], eb[1]]
        src[b] = [ea[0]] * 2 + [ea[1]] * 4 + [ea[2]] * 2
    ids = []
    for r in range(n_ranks):
        row = list(src.get(r, [3 * r + int(rng.integers(0, 3))] * 8))
        rng.shuffle(row)
        ids += row
    return np.array(ids, np.int32).reshape(-1, 1)


def repair_cases(n: int = 40):
    """(P, pairs, R, seed) for n pattern inputs over rank counts 2..64."""
    out = []
    for seed in range(n):
        rng = np.random.default_rng(seed)
        P = int(rng.choice([2, 3, 5, 8, 13, 32, 64]))
        perm = rng.permutation(P)
        npairs = int(rng.integers(1, P // 2 + 1))
        pairs = [(int(perm[2 * i]), int(perm[2 * i + 1])) for i in range(npairs)]
        out.append((P, pairs, int(rng.choice([2, 3, 4])), seed))
    return out
