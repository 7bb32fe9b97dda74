"""Seeded random shapes, plan bit-exact against the oracle on the GPU.

240 cases over rank counts 1..64 (both reduction widths of the register
greedy), 1..40 home experts per rank (every register width and the LDS
greedy), top-K up to 32, 0..4 replica slots, 1..700 tokens per rank, skewed
and flat popularity, rank speeds on a third of the cases, and capacities from
generous to too small (CAPACITY). Every fourth case also dispatches and
combines small rows; the same shapes again with the quota repair; and 40
drift-gated sequences with random thresholds, windows and check intervals.
Inputs come from ``workload``; expected values from the oracle only.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle as O
import token_dispatch_mb_amd as mb
import workload as W
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_required():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.synchronize()


def fuzz_cases(n: int | None = None, seed: int | None = None):
    """Seeded random shapes; MB_FUZZ_CASES and MB_FUZZ_SEED widen a run
    (defaults 240 and 4242)."""
    n = int(os.environ.get("MB_FUZZ_CASES", 240)) if n is None else n
    seed = int(os.environ.get("MB_FUZZ_SEED", 4242)) if seed is None else seed
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        P = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 24, 31, 32, 33, 48, 63, 64]))
        eh = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 40]))
        eh = max(1, min(eh, 1024 // P))
        E = P * eh
        K = int(min(E, 32, rng.choice([1, 2, 3, 4, 6, 8, 8, 8, 16, 32])))
        R = int(rng.integers(0, 5))
        S = int(rng.integers(1, 701))
        S = max(1, min(S, (1 << 22) // (P * E)))  # keeps the routing draw small
        noise = int(rng.choice([W.NOISE_NORMAL, W.NOISE_GUMBEL]))
        zipf = float(rng.uniform(0.5, 1.5))
        beta = float(rng.choice([0.0, 0.3, 1.0, 2.0]))
        cap_kind = str(rng.choice(["tight", "double", "quad", "short"]))
        speeds = None
        if rng.random() < 1 / 3:
            speeds = rng.integers(1, 9, P).astype(np.int32)
        out.append((i, P, eh, K, R, S, noise, zipf, beta, cap_kind, speeds))
    return out


def test_random_shapes_plan_bit_exact():
    n_rows = n_span = 0
    for (i, P, eh, K, R, S, noise, zipf, beta, cap_kind, speeds) in fuzz_cases():
        E, N = P * eh, P * S
        cap = {"tight": S * K, "double": 2 * S * K, "quad": 4 * S * K,
               "short": max(1, S * K - 1 - i % 5)}[cap_kind]
        label = (f"fuzz {i}: P={P} Eh={eh} K={K} R={R} S={S} noise={noise} zipf={zipf:.2f} "
                 f"beta={beta} cap={cap} speeds={None if speeds is None else speeds.tolist()}")
        G.log(label)
        ids, w = W.routing(N, E, K, noise, zipf, beta, 50000 + i)
        H = 16
        dg = mb.Dims.make(N, K, E, P, R, H, cap=cap, dtype_in="f32", dtype_out="f32")
        od = O.make_dims(N, K, E, P, R, H, cap=cap, dtype_in="f32", dtype_out="f32")
        sp = None if speeds is None else speeds.tolist()
        gp = G.GpuPlan(dg).run(ids, speeds=sp)
        got = gp.fetch()
        ref = O.plan(od, ids, speeds=sp)
        G.assert_plan_equal(got, ref)
        if i % 4 == 0 and not ref.status[0] & O.ST_FATAL:
            # every other dispatched case moves rows of one 2 KiB span (512
            # f32), the span kernel's shape when 2 <= K <= 16; the rest rows
            # of 64 bytes (one wave per row chunk)
            dr, orr, Hr = dg, od, H
            if (i // 4) % 2 and 2 <= K <= 16 and P * cap * 2048 <= 1 << 28:
                Hr = 512
                dr = mb.Dims.make(N, K, E, P, R, Hr, cap=cap, dtype_in="f32", dtype_out="f32")
                orr = O.make_dims(N, K, E, P, R, Hr, cap=cap, dtype_in="f32", dtype_out="f32")
                n_span += 1
            x = W.rows_f32(60000 + i, W.TAG_X, Hr, n=N)
            ye = W.rows_f32(60000 + i, W.TAG_YEXP, Hr, n=P * cap)
            buf, _, y = G.run_rows(dr, gp, x, None, ye, w)
            ref_buf, _, _ = O.dispatch(orr, ref, x, None)
            used = ref.row_src >= 0
            assert np.array_equal(buf[used], ref_buf[used]), label
            y_ref, mag, _ = O.combine(orr, ref.pos, ref.status, w, ye)
            G.assert_combine_close(y, y_ref, mag, "f32")
            n_rows += 1
    assert n_rows > 20 and n_span > 5


def test_random_shapes_with_quota_repair_bit_exact():
    """The same shapes planned with the pairwise quota repair (mb_plan_ex)."""
    for (i, P, eh, K, R, S, noise, zipf, beta, cap_kind, speeds) in fuzz_cases()[::2]:
        E, N = P * eh, P * S
        cap = {"tight": S * K, "double": 2 * S * K, "quad": 4 * S * K,
               "short": max(1, S * K - 1 - i % 5)}[cap_kind]
        G.log(f"fuzz repair {i}: P={P} Eh={eh} K={K} R={R} S={S} cap={cap}")
        ids, _ = W.routing(N, E, K, noise, zipf, beta, 50000 + i)
        dg = mb.Dims.make(N, K, E, P, R, 16, cap=cap, dtype_in="f32", dtype_out="f32")
        od = O.make_dims(N, K, E, P, R, 16, cap=cap, dtype_in="f32", dtype_out="f32")
        sp = None if speeds is None else speeds.tolist()
        got = G.GpuPlan(dg).run(ids, speeds=sp, repair=True).fetch()
        G.assert_plan_equal(got, O.plan(od, ids, speeds=sp, repair=True))


def test_random_drift_sequences_bit_exact():
    """40 seeded drift-gated sequences of 6-14 calls: random shapes,
    thresholds (including 0 and 1), windows, check intervals, load-guard
    tolerances (cap only, 0, 1/20, 1/4), popularity changes, rank speeds and
    the quota repair on some; every call's plan and the whole drift state
    after it equal the oracle's. MB_FUZZ_DRIFT and MB_FUZZ_SEED widen a run."""
    seed = int(os.environ.get("MB_FUZZ_SEED", 0))
    rng = np.random.default_rng(777 + seed)
    trng = np.random.default_rng(991 + seed)  # tolerances, drawn apart so the shapes stay put
    n_guarded = 0
    for n in range(int(os.environ.get("MB_FUZZ_DRIFT", 40))):
        P = int(rng.choice([1, 2, 5, 16, 31, 32, 33, 64]))
        eh = max(1, min(int(rng.choice([1, 2, 4, 8, 17, 40])), 1024 // P))
        E = P * eh
        K = int(min(E, rng.choice([1, 2, 4, 8])))
        R = int(rng.integers(0, 4))
        S = int(rng.integers(2, 120))
        N = P * S
        cap = 4 * S * K if R > 0 else N * K
        num, den = [(0, 1), (1, 1), (1, 20), (3, 100), (1, 2)][int(rng.integers(0, 5))]
        window, every = int(rng.integers(1, 6)), int(rng.integers(1, 5))
        change = int(rng.integers(2, 6))
        speeds = rng.integers(1, 5, P).tolist() if rng.random() < 0.3 else None
        repair = bool(rng.random() < 0.25)
        calls = int(rng.integers(6, 15))
        tn, td = [(0, 0), (0, 1), (1, 20), (1, 4)][int(trng.integers(0, 4))]
        label = (f"drift fuzz {n}: P={P} Eh={eh} K={K} R={R} S={S} delta={num}/{den} "
                 f"window={window} every={every} tol={tn}/{td} change={change} speeds={speeds} "
                 f"repair={repair}")
        G.log(label)
        dg = mb.Dims.make(N, K, E, P, R, 16, cap=cap, dtype_in="f32", dtype_out="f32")
        od = O.make_dims(N, K, E, P, R, 16, cap=cap, dtype_in="f32", dtype_out="f32")
        state = mb.alloc_drift_state(dg, G.dev())
        st = O.DriftState(E, P, R)
        gprm = mb.DriftParams(num, den, window, every, tn, td)
        oprm = O.DriftParams(num, den, window, every, tn, td)
        gp = G.GpuPlan(dg)
        for call in range(calls):
            ids, _ = W.routing(N, E, K, W.NOISE_GUMBEL, 1.1, 1.0, 70000 + 100 * n + call,
                               pop_seed=80000 + 100 * n + call // change)
            got = gp.run(ids, speeds=speeds, drift=(gprm, state), repair=repair).fetch()
            ref = O.plan(od, ids, speeds=speeds, drift=(oprm, st), repair=repair)
            G.assert_plan_equal(got, ref)
            h = mb.drift_header(state)
            for key in ("have_plan", "countdown", "nwin", "n_moves", "calls", "replans", "guarded"):
                assert h[key] == getattr(st, key), (label, call, key, h[key], getattr(st, key))
            assert h["last_d"] == st.last_d, (label, call, "last_d")
            wsum = state[64:64 + 8 * E].cpu().numpy().view(np.int64)
            assert np.array_equal(wsum, st.wsum), (label, call, "reference")
        n_guarded += st.guarded
    if int(os.environ.get("MB_FUZZ_DRIFT", 40)) >= 40:
        assert n_guarded > 0  # the guard's replan branch ran
