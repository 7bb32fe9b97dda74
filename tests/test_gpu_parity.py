"""Parity of libmoebal on the GPU with the CPU oracle, through the C ABI.

Integers (counts, loads, plan, quotas, cu_seqlens, pos, row_src, status) and
dispatched bytes must be bit-exact; combine must be within the tolerance of
``gpu_harness.TOL`` relative to sum_k |w_k y_k|. Inputs are seeded synthetic
workloads from ``workload``; expected values come from ``oracle`` only.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import token_dispatch_mb_amd as mb
import workload as W
from tests import gpu_harness as G
from tests import plan_checks as C

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_required():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.synchronize()


def _y_exp_rows(wl_seed: int, dims, n_rows: int):
    if dims.dtype_out == O.F32:
        return W.rows_f32(wl_seed, W.TAG_YEXP, dims.hidden, n=n_rows)
    return W.rows_bf16(wl_seed, W.TAG_YEXP, dims.hidden, n=n_rows)


def _full_check(dims_g, od, ids, w, x, xs, y_exp, label="", speeds=None):
    """Plan, dispatch and combine on the GPU; compare everything with the oracle."""
    G.log(f"case {label}: N={od.n_tokens} K={od.top_k} E={od.n_experts} P={od.n_ranks} "
          f"R={od.slots_per_rank} H={od.hidden} cap={od.cap}")
    gp = G.GpuPlan(dims_g).run(ids, speeds=speeds)
    got = gp.fetch()
    ref = O.plan(od, ids, speeds=speeds)
    G.assert_plan_equal(got, ref)
    buf, bs, y = G.run_rows(dims_g, gp, x, xs, y_exp, w)
    fatal = bool(ref.status[0] & O.ST_FATAL)
    if fatal:
        assert np.all(buf == 0xA5), "dispatch wrote despite a fatal status"
        assert np.all(np.isnan(y)), "combine wrote despite a fatal status"
        return ref
    ref_buf, ref_bs, _ = O.dispatch(od, ref, x, xs)
    used = ref.row_src >= 0
    assert np.array_equal(buf[used], ref_buf[used]), "dispatched rows"
    assert np.all(buf[~used] == 0xA5), "padding rows were written"
    if ref_bs is not None:
        assert np.array_equal(bs[used], ref_bs[used]), "dispatched fp8 scales"
    y_ref, mag, _ = O.combine(od, ref.pos, ref.status, w, y_exp)
    G.assert_combine_close(y, y_ref, mag, "f32" if od.dtype_out == O.F32 else "bf16")
    return ref


# ---- the small workloads, end to end -------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "mixtral", "decode_drift"])
def test_workload_end_to_end(name):
    wl = W.get_workload(name)
    ids, w = W.routing_for(wl)
    x, xs = W.token_rows(wl)
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    ye = _y_exp_rows(wl.seed, od, od.n_ranks * od.cap)
    ref = _full_check(dg, od, ids, w, x, xs, ye, name)
    assert ref.status[0] == 0


def test_decode_drift_61_calls_stateless():
    """Every call of the 61-layer decode sequence, planned back to back into
    the same buffers, equals the oracle; calls planned alone into fresh
    buffers equal the same calls inside the sequence."""
    wl = W.get_workload("decode_drift")
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    seq = G.GpuPlan(dg)
    G.log("decode_drift: 61 calls")
    kept = {}
    for call in range(wl.calls):
        ids, _ = W.routing_for(wl, call)
        got = seq.run(ids).fetch()
        G.assert_plan_equal(got, O.plan(od, ids))
        if call in (0, 29, 60):
            kept[call] = got
    for call, got_seq in kept.items():
        ids, _ = W.routing_for(wl, call)
        alone = G.GpuPlan(dg).run(ids).fetch()
        for k in G.PLAN_FIELDS:
            assert np.array_equal(alone[k], got_seq[k]), (call, k)


def test_decode_drift_rows_several_calls():
    wl = W.get_workload("decode_drift")
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    for call in (1, 37):
        ids, w = W.routing_for(wl, call)
        x, xs = W.token_rows(wl, call)
        ye = _y_exp_rows(wl.seed_for(call), od, od.n_ranks * od.cap)
        _full_check(dg, od, ids, w, x, xs, ye, f"decode_drift call {call}")


# ---- shape sweep ------------------------------------------------------------------

def _sweep_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for P in (1, 2, 4, 8, 16, 32, 64):
        for R in (0, 1, 2, 4):
            K = int(rng.choice([1, 2, 8]))
            eh = int(rng.choice([1, 4, 8, 24]))
            if K > P * eh:
                K = P * eh
            S = int(rng.choice([3, 37, 300, 513]))
            cases.append((P, eh, K, R, S))
    return cases


@pytest.mark.parametrize("P,eh,K,R,S", _sweep_cases())
def test_shape_sweep(P, eh, K, R, S):
    E, N = P * eh, P * S
    ids, w = W.routing(N, E, K, W.NOISE_NORMAL, 1.0, 0.8, 7000 + P * 31 + R * 7 + K)
    cap = S * K if R > 0 else N * K  # R = 0: make room for the unbalanced load
    H = 64
    dg = mb.Dims.make(N, K, E, P, R, H, cap=cap, dtype_in="f32", dtype_out="f32")
    od = O.make_dims(N, K, E, P, R, H, cap=cap, dtype_in="f32", dtype_out="f32")
    x = W.rows_f32(P * 1000 + S, W.TAG_X, H, n=N)
    ye = W.rows_f32(P * 1000 + S, W.TAG_YEXP, H, n=P * cap)
    _full_check(dg, od, ids, w, x, xs=None, y_exp=ye, label=f"sweep P{P} Eh{eh} K{K} R{R} S{S}")


# ---- edge cases ---------------------------------------------------------------------

def _edge(N, K, E, P, R, H, ids, cap=None, din="bf16", dout="bf16", seed=11, label="edge"):
    dg = mb.Dims.make(N, K, E, P, R, H, cap=cap, dtype_in=din, dtype_out=dout)
    od = O.make_dims(N, K, E, P, R, H, cap=cap, dtype_in=din, dtype_out=dout)
    w = np.full((N, K), 1.0 / K, np.float32)
    if din == "fp8":
        x, xs, _ = W.rows_fp8(seed, W.TAG_X, H, n=N)
    elif din == "f32":
        x, xs = W.rows_f32(seed, W.TAG_X, H, n=N), None
    else:
        x, xs = W.rows_bf16(seed, W.TAG_X, H, n=N), None
    ye = _y_exp_rows(seed, od, od.n_ranks * od.cap)
    return _full_check(dg, od, np.ascontiguousarray(ids, np.int32), w, x, xs, ye, label)


def test_all_tokens_one_expert():
    P, S = 16, 40
    ref = _edge(P * S, 1, P * 2, P, 1, 32, np.zeros((P * S, 1)), label="all-to-one")
    assert ref.status[3] == P - 1


def test_uniform_loads():
    P, S, K, E = 8, 32, 4, 32
    t = np.arange(P * S)[:, None]
    ids = (t * K + np.arange(K)[None]) % E
    ref = _edge(P * S, K, E, P, 2, 64, ids, label="uniform")
    assert ref.status[3] == 0


def test_r0_unbalanced_with_room_and_capacity():
    wl = W.get_workload("mixtral")
    ids, _ = W.routing_for(wl)
    ref = _edge(wl.n_tokens, 2, 8, 8, 0, 256, ids, cap=wl.n_tokens * 2, label="R0 room")
    assert ref.status[0] == O.ST_UNBALANCED
    ref = _edge(wl.n_tokens, 2, 8, 8, 0, 256, ids, label="R0 capacity")
    assert ref.status[0] == O.ST_UNBALANCED | O.ST_CAPACITY


def test_capacity_below_water_level():
    wl = W.get_workload("tiny")
    ids, _ = W.routing_for(wl)
    ref = _edge(64, 2, 16, 4, 1, 128, ids, cap=wl.cap - 3, din="f32", dout="f32", label="cap<T")
    assert ref.status[0] & O.ST_CAPACITY


def test_bad_and_duplicate_ids():
    ids = np.tile(np.array([[0, 1]], np.int32), (64, 1))
    ids[10, 1] = 16
    ref = _edge(64, 2, 16, 4, 1, 64, ids, label="bad id")
    assert ref.status[0] == O.ST_BAD_ID
    ids[10, 1] = -5
    _edge(64, 2, 16, 4, 1, 64, ids, label="negative id")
    ids[10, 1] = 0
    ref = _edge(64, 2, 16, 4, 1, 64, ids, label="dup id")
    assert ref.status[0] == O.ST_DUP_ID


def test_workspace_reused_across_sizes():
    """One workspace for plans of different sizes in a row (one to 33 routing
    blocks per source rank, several top-K, R = 0 to 3): every plan matches
    the oracle, whatever the previous call left in the workspace."""
    shapes = [(4, 8448, 16, 2, 1), (8, 300, 64, 8, 2), (64, 128, 256, 8, 1), (2, 256, 8, 3, 0),
              (16, 1030, 96, 4, 3), (1, 700, 4, 1, 1), (32, 4096, 256, 8, 1)]
    dev = G.dev()
    dims = [mb.Dims.make(P * S, K, E, P, R, 64, cap=2 * S * K) for P, S, E, K, R in shapes]
    ws = torch.empty(max(mb.workspace_bytes(d) for d in dims), dtype=torch.uint8, device=dev)
    for (P, S, E, K, R), dg in zip(shapes, dims):
        ids, _ = W.routing(P * S, E, K, W.NOISE_GUMBEL, 1.1, 1.0, 7000 + P * S)
        od = O.make_dims(P * S, K, E, P, R, 64, cap=2 * S * K)
        gp = G.GpuPlan(dg)
        gp.ws = ws
        G.assert_plan_equal(gp.run(ids).fetch(), O.plan(od, ids))


def test_bad_ids_clear_the_previous_plan():
    """A plan of bad or repeated ids into buffers that hold a valid plan:
    counts, loads, quotas and cu_seqlens read 0 and every replica slot -1,
    as in the oracle, not the previous call's values."""
    wl = W.get_workload("tiny")
    ids, _ = W.routing_for(wl)
    dg = mb.Dims.for_workload(wl)
    od = O.dims_for(wl)
    gp = G.GpuPlan(dg)
    good = gp.run(ids).fetch()
    G.assert_plan_equal(good, O.plan(od, ids))
    assert good["counts"].any() and (good["rep_expert"] >= 0).any()
    for bad_val, flag in ((wl.n_experts, O.ST_BAD_ID), (-1, O.ST_BAD_ID), (None, O.ST_DUP_ID)):
        gp.run(ids)
        bad = ids.copy()
        bad[37, 1] = bad[37, 0] if bad_val is None else bad_val
        got = gp.run(bad).fetch()
        ref = O.plan(od, bad)
        assert ref.status[0] == flag
        G.assert_plan_equal(got, ref)
        assert not got["counts"].any() and (got["rep_expert"] == -1).all()


@pytest.mark.parametrize("din,dout,H", [("bf16", "f32", 200), ("f32", "bf16", 200),
                                         ("fp8", "f32", 384), ("fp8", "bf16", 384)])
def test_mixed_row_types(din, dout, H):
    """Input rows and expert outputs of different types in one plan: the
    dispatch follows the input type (fp8 with its scale rows), the combine
    the output type; both against the oracle on a skewed routing."""
    P, S, K, eh, R = 8, 300, 8, 8, 2
    ids, _ = W.routing(P * S, P * eh, K, W.NOISE_GUMBEL, 1.1, 1.0, 6100 + H)
    _edge(P * S, K, P * eh, P, R, H, ids, cap=2 * S * K, din=din, dout=dout, seed=H,
          label=f"mixed {din}->{dout} H{H}")


def test_empty_batch():
    dg = mb.Dims.make(0, 2, 16, 4, 1, 64, cap=8, dtype_in="bf16", dtype_out="bf16")
    od = O.make_dims(0, 2, 16, 4, 1, 64, cap=8, dtype_in="bf16", dtype_out="bf16")
    ids = np.zeros((0, 2), np.int32)
    got = G.GpuPlan(dg).run(ids).fetch()
    ref = O.plan(od, ids)
    G.assert_plan_equal(got, ref)


@pytest.mark.parametrize("K", [3, 5, 16, 32])
def test_generic_top_k(K):
    """Top-K values without a specialised kernel use the runtime-K path."""
    P, eh, S = 4, 16, 77
    E = P * eh
    ids, w = W.routing(P * S, E, K, W.NOISE_NORMAL, 1.0, 1.0, 900 + K)
    _edge(P * S, K, E, P, 2, 64, ids, label=f"K={K}")


def test_k_equals_e_and_single_rank_and_e_equals_p():
    ids, _ = W.routing(40, 8, 8, W.NOISE_NORMAL, 1.0, 1.0, 3)
    _edge(40, 8, 8, 4, 1, 64, ids, label="K=E")
    ids, _ = W.routing(300, 24, 4, W.NOISE_NORMAL, 1.0, 1.0, 4)
    _edge(300, 4, 24, 1, 2, 64, ids, label="P=1")
    ids, _ = W.routing(640, 64, 2, W.NOISE_GUMBEL, 1.0, 1.0, 5)
    _edge(640, 2, 64, 64, 1, 64, ids, label="E=P=64")


def test_maximum_sizes():
    """E = 1024 experts, P = 64 ranks, R = 16 slots, K = 32, 16-byte rows."""
    P, eh, S, K, R = 64, 16, 20, 32, 16
    ids, _ = W.routing(P * S, P * eh, K, W.NOISE_GUMBEL, 1.2, 1.0, 12)
    _edge(P * S, K, P * eh, P, R, 8, ids, label="max E/P/R/K")
    ids, _ = W.routing(P * S, P * eh, 8, W.NOISE_GUMBEL, 1.2, 1.0, 13)
    _edge(P * S, 8, P * eh, P, R, 4, ids, din="f32", dout="f32", label="16-byte f32 rows")


def _skewed_ids(N, K, E, seed):
    """Distinct ids per token, (b + k) mod E for k < K, from a skewed first
    choice b = floor(E u^3): cheap to draw at tens of millions of pairs."""
    rng = np.random.default_rng(seed)
    b = np.floor(E * rng.random(N) ** 3).astype(np.int64)
    return ((b[:, None] + np.arange(K)[None]) % E).astype(np.int32)


@pytest.mark.parametrize("N,K,E,P,R,kind", [
    (2 ** 25 - 64, 1, 128, 64, 1, "one"),   # register greedy, loads up to the key limit
    (2 ** 25, 1, 128, 64, 1, "one"),        # N*K = 2^25: the LDS greedy
    (2 ** 22 - 32, 8, 256, 32, 2, "skew"),  # register greedy, 32 lanes
    (2 ** 22, 8, 256, 32, 2, "skew"),       # the LDS greedy
])
def test_plan_around_the_packed_key_limit(N, K, E, P, R, kind):
    """The register greedy packs (value, index) into one int32 key, exact
    while N*K < 2^25; larger plans run the LDS greedy. Both sides of the
    limit, with the busiest rank's excess close to it, are bit-exact."""
    ids = np.zeros((N, 1), np.int32) if kind == "one" else _skewed_ids(N, K, E, 5)
    cap = 2 * (N // P) * K
    G.log(f"case packed-key limit N={N} K={K} E={E} P={P} R={R} {kind}")
    dg = mb.Dims.make(N, K, E, P, R, 8, cap=cap, dtype_in="f32", dtype_out="f32")
    od = O.make_dims(N, K, E, P, R, 8, cap=cap, dtype_in="f32", dtype_out="f32")
    got = G.GpuPlan(dg).run(ids).fetch()
    ref = O.plan(od, ids)
    G.assert_plan_equal(got, ref)
    assert ref.status[0] == 0 and ref.status[3] > 0


@pytest.mark.parametrize("P,eh,R", [
    # home experts per rank: 4 | 8 | 16 | 24 | 32 quota registers per lane (the first two kept in
    # order); 32-lane (P <= 32) and 64-lane reductions; one slot per rank and several
    (16, 4, 1), (16, 4, 2), (64, 4, 1), (64, 4, 3),
    (32, 8, 1), (32, 8, 2), (40, 6, 1), (40, 6, 2),
    (20, 12, 1), (20, 12, 3), (48, 16, 1), (48, 16, 2),
    (16, 24, 1), (16, 24, 2), (40, 20, 1), (40, 20, 4),
    (32, 32, 1), (32, 32, 2), (33, 31, 1), (33, 31, 3),
])
def test_register_greedy_variants(P, eh, R):
    """Every register-greedy variant, bit-exact: once with equal speeds and
    once with rank speeds alternating 8 and 1, whose fast ranks fill all
    their slots (more than 64 moves when the P/2 fast ranks hold more than 64
    slots, so the move records leave registers mid-loop)."""
    E, S, K = P * eh, 96, 8
    N = P * S
    dg = mb.Dims.make(N, K, E, P, R, 16, cap=4 * S * K, dtype_in="f32", dtype_out="f32")
    od = O.make_dims(N, K, E, P, R, 16, cap=4 * S * K, dtype_in="f32", dtype_out="f32")
    for speeds in (None, [8 if r % 2 == 0 else 1 for r in range(P)]):
        G.log(f"case greedy variant P={P} Eh={eh} R={R} speeds={'8/1' if speeds else None}")
        ids, _ = W.routing(N, E, K, W.NOISE_GUMBEL, 1.0, 0.3, 61000 + P * 100 + eh)
        got = G.GpuPlan(dg).run(ids, speeds=speeds).fetch()
        ref = O.plan(od, ids, speeds=speeds)
        G.assert_plan_equal(got, ref)
        assert ref.status[3] > 0
        if speeds and (P // 2) * R > 64:
            assert ref.status[3] > 64, "the mid-loop record flush did not run"


@pytest.mark.parametrize("din,H,K", [
    ("bf16", 1024, 2), ("bf16", 1024, 3), ("bf16", 2048, 16), ("f32", 512, 8), ("fp8", 2048, 4),
    ("fp8", 4096, 8),                       # rows of whole 2 KiB spans: k_dispatch_span
    ("bf16", 1024, 1), ("bf16", 1536, 8), ("bf16", 1024, 17), ("fp8", 1152, 5),  # k_dispatch
])
def test_dispatch_kernels_by_row_shape(din, H, K):
    """Rows made of whole 2 KiB spans with 2 <= K <= 16 go through the
    span kernel (one workgroup of K waves per span, staged in LDS), the rest
    through the one-wave-per-KiB kernel; both bit-exact against the oracle
    on a ragged token count, fp8 scale rows included, padding rows left
    untouched; and with a bad id neither writes anything."""
    P, eh, S, R = 4, 8, 77, 2
    E = P * eh
    ids, _ = W.routing(P * S, E, K, W.NOISE_GUMBEL, 1.1, 1.0, 5300 + H + K)
    _edge(P * S, K, E, P, R, H, ids, cap=2 * S * K, din=din, dout="bf16", seed=H + K,
          label=f"dispatch {din} H{H} K{K}")
    bad = ids.copy()
    bad[S + 3, 0] = E
    ref = _edge(P * S, K, E, P, R, H, bad, cap=2 * S * K, din=din, dout="bf16", seed=H,
                label=f"dispatch {din} H{H} K{K} bad id")
    assert ref.status[0] & O.ST_BAD_ID


def test_fp8_rows_and_scales_small():
    ids, _ = W.routing(512, 32, 4, W.NOISE_GUMBEL, 1.1, 1.0, 21)
    _edge(512, 4, 32, 8, 1, 256, ids, din="fp8", dout="bf16", label="fp8")


def test_repeat_is_bit_identical():
    wl = W.get_workload("decode_drift")
    ids, _ = W.routing_for(wl, 5)
    gp = G.GpuPlan(mb.Dims.for_workload(wl))
    first = gp.run(ids).fetch()
    for _ in range(4):
        again = gp.run(ids).fetch()
        for k in G.PLAN_FIELDS:
            assert np.array_equal(first[k], again[k]), k


def test_round_trip_identity_experts():
    """pi14 on the GPU: with expert outputs equal to the dispatched rows,
    one-hot weights return x bit-exactly."""
    wl = W.get_workload("mixtral")
    ids, _ = W.routing_for(wl)
    dg = mb.Dims.for_workload(wl)
    gp = G.GpuPlan(dg).run(ids)
    x, _ = W.token_rows(wl)
    x_d = G.torch_rows(x, O.BF16)
    buf = torch.empty((dg.rows, dg.hidden), dtype=torch.bfloat16, device=G.dev())
    mb.dispatch(dg, gp.bufs, x_d, buf)
    onehot = np.zeros((wl.n_tokens, wl.top_k), np.float32)
    onehot[np.arange(wl.n_tokens), np.arange(wl.n_tokens) % wl.top_k] = 1.0
    y = torch.empty_like(x_d)
    mb.combine(dg, gp.bufs, buf, torch.from_numpy(onehot).to(G.dev()), y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), x_d.view(torch.int16))


# ---- full-size prefill workloads -----------------------------------------------------

G_ROWS = 4099  # distinct expert-output rows, cycled over the buffer (prime)


@pytest.mark.parametrize("name", ["dsv3_prefill", "kimi_prefill", "vibe_dsv3_prefill"]
                         + W.configs.SWEEP_ORDER)
def test_prefill_full_size(name):
    """The full prefill and maxvio-sweep workloads in the launch configuration
    the benchmark times, nothing sampled: the whole plan bit-exact; every
    dispatch row bit-exact against x gathered through the oracle's row_src,
    and every padding row still holding what was there before; every
    token's combine in tolerance against the oracle. Expert outputs cycle
    through 4099 generated rows (row p holds generated row p mod 4099), so
    the oracle reads those rows at pos mod 4099: the same values."""
    wl = W.get_workload(name)
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    G.log(f"{name}: routing")
    ids, w = W.routing_for(wl)
    speeds = W.rank_speeds(wl)
    ref = O.plan(od, ids, speeds=speeds)
    gp = G.GpuPlan(dg).run(ids, speeds=speeds)
    got = gp.fetch()
    G.assert_plan_equal(got, ref)
    assert ref.status[0] == 0 and ref.report["wir_after"] <= 1.01
    G.log(f"{name}: plan bit-exact (IR {ref.report['ir_before']:.3f} -> {ref.report['ir_after']:.4f}, "
          f"against speed targets {ref.report['wir_before']:.3f} -> {ref.report['wir_after']:.4f})")

    x, _ = W.token_rows(wl)
    d = G.dev()
    x_d = G.torch_rows(x, O.BF16).view(torch.int16)
    del x
    sentinel = 0x7F7F
    buf = torch.empty((dg.rows, dg.hidden), dtype=torch.bfloat16, device=d)
    buf.view(torch.int16).fill_(sentinel)
    mb.dispatch(dg, gp.bufs, x_d.view(torch.bfloat16), buf)
    src = torch.from_numpy(ref.row_src).to(d)
    chunk = 32768
    n_pad = 0
    for r0 in range(0, dg.rows, chunk):
        r1 = min(dg.rows, r0 + chunk)
        s_c = src[r0:r1]
        used = s_c >= 0
        got_c = buf[r0:r1].view(torch.int16)
        assert torch.equal(got_c[used], x_d[s_c[used].long()]), f"rows {r0}..{r1}"
        if not bool(used.all()):
            n_pad += int((~used).sum())
            assert bool((got_c[~used] == sentinel).all()), f"padding rows in {r0}..{r1}"
    G.log(f"{name}: all {int((src >= 0).sum())} dispatch rows bit-exact, {n_pad} padding rows untouched")
    del buf, src

    gen = W.rows_bf16(wl.seed, W.TAG_YEXP, dg.hidden, n=G_ROWS)
    gen_d = torch.from_numpy(gen).view(torch.bfloat16).to(d)
    ye = gen_d[torch.arange(dg.rows, device=d) % G_ROWS]
    w_d = torch.from_numpy(w).to(d)
    y = torch.empty((dg.n_tokens, dg.hidden), dtype=torch.bfloat16, device=d)
    mb.combine(dg, gp.bufs, ye, w_d, y)
    torch.cuda.synchronize()
    del ye
    pos_mod = (ref.pos.astype(np.int64) % G_ROWS).astype(np.int32)
    ct = 4096
    y_ref = np.empty((ct, dg.hidden), np.float64)
    mag = np.empty_like(y_ref)
    for t0 in range(0, dg.n_tokens, ct):
        t1 = min(dg.n_tokens, t0 + ct)
        O.combine(od, pos_mod, ref.status, w, gen, t0, t1,
                  out=(y_ref[: t1 - t0], mag[: t1 - t0]))
        G.assert_combine_close(G.y_to_f64(y[t0:t1]), y_ref[: t1 - t0], mag[: t1 - t0], "bf16")
    G.log(f"{name}: combine of all {dg.n_tokens} tokens in tolerance")
    del y, x_d
    torch.cuda.empty_cache()


# ---- hand-derived examples (tie-breaks, host order) ------------------------------

@pytest.mark.parametrize("golden", ["hand_example_fill.json", "hand_example_expert_tie.json",
                                    "hand_example_destination_tie.json",
                                    "hand_example_surplus_order.json"])
def test_hand_examples_on_gpu(golden):
    """The GPU plan of each hand-derived example equals its stored values
    (and the oracle's)."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", golden)))
    dd = dict(g["dims"])
    dd["hidden"] = 8  # 16-byte bf16 rows; the plan does not depend on H
    ids = np.array(g["ids"], np.int32).reshape(dd["n_tokens"], dd["top_k"])
    dg = mb.Dims.make(**dd, dtype_in="bf16", dtype_out="bf16")
    got = G.GpuPlan(dg).run(ids).fetch()
    exp = g.get("fill_host", g)
    for key in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
                "row_src", "status"):
        assert np.array_equal(got[key].reshape(np.array(exp[key]).shape), np.array(exp[key])), key
    assert np.array_equal(got["pos"].ravel(), exp["pos"])
    G.assert_plan_equal(got, O.plan(O.make_dims(**dd, dtype_in="bf16", dtype_out="bf16"), ids))


def test_hand_example_weighted_on_gpu():
    """The hand-derived example with rank speeds [4, 4, 2, 1] through
    mb_plan_weighted equals its stored values (and the oracle's)."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "hand_example_weighted.json")))
    dd = dict(g["dims"])
    dd["hidden"] = 8
    ids = np.array(g["ids"], np.int32).reshape(dd["n_tokens"], dd["top_k"])
    dg = mb.Dims.make(**dd, dtype_in="bf16", dtype_out="bf16")
    got = G.GpuPlan(dg).run(ids, speeds=g["speeds"]).fetch()
    for key in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
                "row_src", "status"):
        assert np.array_equal(got[key].reshape(np.array(g[key]).shape), np.array(g[key])), key
    assert np.array_equal(got["pos"].ravel(), g["pos"])
    G.assert_plan_equal(got, O.plan(O.make_dims(**dd, dtype_in="bf16", dtype_out="bf16"), ids,
                                    speeds=np.array(g["speeds"], np.int32)))


def _speed_cases():
    rng = np.random.default_rng(77)
    cases = []
    for P in (1, 3, 8, 32, 64):
        for R in (0, 1, 3):
            eh = min(int(rng.choice([1, 5, 24, 40])), 1024 // P)  # E <= 1024
            K = min(int(rng.choice([1, 4, 8])), P * eh)
            S = int(rng.choice([5, 64, 301]))
            kind = str(rng.choice(["narrow", "wide", "extreme"]))
            cases.append((P, eh, K, R, S, kind))
    return cases


@pytest.mark.parametrize("P,eh,K,R,S,kind", _speed_cases())
def test_weighted_shape_sweep(P, eh, K, R, S, kind):
    """mb_plan_weighted against the oracle over shapes and speed spreads:
    narrow (within 15 %), wide (up to 8x) and extreme (1 and 2^20 mixed,
    where slow ranks get targets near zero)."""
    E, N = P * eh, P * S
    ids, w = W.routing(N, E, K, W.NOISE_NORMAL, 1.0, 0.8, 9000 + P * 31 + R * 7 + K)
    rng = np.random.default_rng(P * 100 + R)
    if kind == "narrow":
        speeds = rng.integers(57000, 65537, P)
    elif kind == "wide":
        speeds = rng.integers(1000, 8001, P)
    else:
        speeds = np.where(rng.random(P) < 0.5, 1, mb.MAX_SPEED)
    speeds = speeds.astype(np.int32)
    cap = 2 * S * K if R > 0 else N * K
    H = 64
    dg = mb.Dims.make(N, K, E, P, R, H, cap=cap, dtype_in="f32", dtype_out="f32")
    od = O.make_dims(N, K, E, P, R, H, cap=cap, dtype_in="f32", dtype_out="f32")
    x = W.rows_f32(P * 1000 + S, W.TAG_X, H, n=N)
    ye = W.rows_f32(P * 1000 + S, W.TAG_YEXP, H, n=P * cap)
    _full_check(dg, od, ids, w, x, xs=None, y_exp=ye,
                label=f"weighted P{P} Eh{eh} K{K} R{R} S{S} {kind}", speeds=speeds)


def test_equal_speeds_match_mb_plan():
    """mb_plan_weighted with equal speeds writes exactly what mb_plan writes."""
    wl = W.get_workload("kimi_prefill").scaled(16384)
    ids, _ = W.routing_for(wl)
    dg = mb.Dims.for_workload(wl, cap=2 * wl.cap)
    a = G.GpuPlan(dg).run(ids).fetch()
    b = G.GpuPlan(dg).run(ids, speeds=[977] * wl.n_ranks).fetch()
    for k in G.PLAN_FIELDS:
        assert np.array_equal(a[k], b[k]), k


# ---- drift-gated replanning ------------------------------------------------------

def _gpu_drift_state(dg):
    return mb.alloc_drift_state(dg, G.dev())


def _assert_state_equal(state_d, st, E, label):
    h = mb.drift_header(state_d)
    for key in ("have_plan", "countdown", "nwin", "n_moves", "calls", "replans", "guarded"):
        assert h[key] == getattr(st, key), (label, key, h[key], getattr(st, key))
    # the decision is taken in double on both sides from exact integer sums
    assert h["last_d"] == st.last_d, (label, "last_d", h["last_d"], st.last_d)
    wsum = state_d[64:64 + 8 * E].cpu().numpy().view(np.int64)
    assert np.array_equal(wsum, st.wsum), (label, "reference")


def test_hand_example_drift_on_gpu():
    """The hand-derived drift sequence through mb_plan_drift: every call's
    plan and the state after it equal the stored values and the oracle's."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "hand_example_drift.json")))
    dd = dict(g["dims"])
    dd["hidden"] = 8
    dg = mb.Dims.make(**dd, dtype_in="bf16", dtype_out="bf16")
    od = O.make_dims(**dd, dtype_in="bf16", dtype_out="bf16")
    gprm, oprm = mb.DriftParams(**g["params"]), O.DriftParams(**g["params"])
    state = _gpu_drift_state(dg)
    st = O.DriftState(od.n_experts, od.n_ranks, od.slots_per_rank)
    gp = G.GpuPlan(dg)
    for i, call in enumerate(g["calls"]):
        ids = np.array(call["ids"], np.int32).reshape(-1, 1)
        got = gp.run(ids, drift=(gprm, state)).fetch()
        for key in ("status", "load_post", "rep_expert", "slot_quota"):
            assert np.array_equal(got[key].reshape(np.array(call[key]).shape),
                                  np.array(call[key])), (i, key)
        ref = O.plan(od, ids, drift=(oprm, st))
        G.assert_plan_equal(got, ref)
        _assert_state_equal(state, st, od.n_experts, f"call {i}")


def test_drift_replay_needs_home_above_target_on_gpu():
    dg = mb.Dims.make(12, 1, 3, 3, 1, 8, cap=12, dtype_in="bf16", dtype_out="bf16")
    state = _gpu_drift_state(dg)
    prm = mb.DriftParams(1, 1, 4, 1)
    gp = G.GpuPlan(dg)
    c0 = np.array([0] * 6 + [1] * 3 + [2] * 3, np.int32).reshape(-1, 1)
    c1 = np.array([0] * 4 + [1] * 2 + [2] * 6, np.int32).reshape(-1, 1)
    a = gp.run(c0, drift=(prm, state)).fetch()
    assert a["status"][0] == mb.ST_REPLANNED and np.array_equal(a["load_post"], [4, 4, 4])
    b = gp.run(c1, drift=(prm, state)).fetch()
    assert b["status"][0] == mb.ST_UNBALANCED and np.array_equal(b["load_post"], [4, 2, 6])


@pytest.mark.parametrize("H", [1, 10])
def test_drift_decode_sequence(H):
    """The 60-pass drift workload through mb_plan_drift and the oracle in
    lockstep, with its load guard (5/4 of the targets) and regions of
    5/4 S K rows: every call's plan bit-exact, the state (counters,
    reference, distance) equal after every call, no call fatal; dispatch and
    combine on three kept calls. Rows are 128 wide here (the plan does not
    depend on H)."""
    wl = W.get_workload("drift_decode")
    num, den, win, _, tn, td = wl.drift
    dg = mb.Dims.for_workload(wl)
    dg.hidden = 128
    od = O.dims_for(wl)
    od.hidden = 128
    state = _gpu_drift_state(dg)
    st = O.DriftState(wl.n_experts, wl.n_ranks, wl.slots_per_rank)
    gprm, oprm = mb.DriftParams(num, den, win, H, tn, td), O.DriftParams(num, den, win, H, tn, td)
    gp = G.GpuPlan(dg)
    replans, guarded, rows_at = [], [], [7, 33, 59]
    for call in range(wl.calls):
        ids, w = W.routing_for(wl, call)
        got = gp.run(ids, drift=(gprm, state)).fetch()
        ref = O.plan(od, ids, drift=(oprm, st))
        G.assert_plan_equal(got, ref)
        _assert_state_equal(state, st, wl.n_experts, f"call {call}")
        assert not ref.flags & O.ST_FATAL, call
        if ref.flags & O.ST_REPLANNED:
            replans.append(call)
        if ref.flags & O.ST_GUARDED:
            guarded.append(call)
        if rows_at and call >= rows_at[0] and not ref.flags & O.ST_REPLANNED:
            rows_at.pop(0)
            x, xs, _ = W.rows_fp8(wl.seed_for(call), W.TAG_X, 128, n=wl.n_tokens)
            ye = _y_exp_rows(wl.seed_for(call), od, od.n_ranks * od.cap)
            buf, bs, y = G.run_rows(dg, gp, x, xs, ye, w)
            ref_buf, ref_bs, _ = O.dispatch(od, ref, x, xs)
            used = ref.row_src >= 0
            assert np.array_equal(buf[used], ref_buf[used]) and np.array_equal(bs[used], ref_bs[used])
            y_ref, mag, _ = O.combine(od, ref.pos, ref.status, w, ye)
            G.assert_combine_close(y, y_ref, mag, "bf16")
    G.log(f"drift_decode H={H}: replans at {replans}, guarded {guarded}")
    assert not rows_at
    # the popularity shifts at 25 and 50 are caught in the call itself: by
    # the check when one runs every call, else by the load guard
    assert replans == [0, 25, 50]
    assert guarded == ([] if H == 1 else [25, 50])


@pytest.mark.parametrize("cap_q,tol", [(4, (0, 0)), (5, (1, 4)), (5, (3, 100))])
def test_drift_decode_load_guard_regions(cap_q, tol):
    """drift_decode in lockstep with the oracle at regions of cap_q/4 S K
    rows (S K is the library's default) under the load guard alone (0, 0),
    at 1/4 and at ViBE's 0.03: plans and state bit-exact every call; a call
    is CAPACITY-fatal only where a fresh greedy plan of that call is too
    (the guard falls back to that same greedy), so at 5/4 S K none is."""
    wl = W.get_workload("drift_decode")
    num, den, win, H = wl.drift[:4]
    cap = wl.tokens_per_rank * wl.top_k * cap_q // 4
    dg = mb.Dims.for_workload(wl, cap=cap)
    dg.hidden = 128
    od = O.dims_for(wl, cap=cap)
    od.hidden = 128
    state = _gpu_drift_state(dg)
    st = O.DriftState(wl.n_experts, wl.n_ranks, wl.slots_per_rank)
    gprm, oprm = mb.DriftParams(num, den, win, H, *tol), O.DriftParams(num, den, win, H, *tol)
    gp = G.GpuPlan(dg)
    fatal = []
    for call in range(wl.calls):
        ids, _ = W.routing_for(wl, call)
        got = gp.run(ids, drift=(gprm, state)).fetch()
        ref = O.plan(od, ids, drift=(oprm, st))
        G.assert_plan_equal(got, ref)
        _assert_state_equal(state, st, wl.n_experts, f"call {call}")
        if ref.flags & O.ST_FATAL:
            fatal.append(call)
            assert ref.flags & O.ST_REPLANNED, call  # a kept replay never overflows
            assert O.plan(od, ids).flags & O.ST_CAPACITY, call
    G.log(f"drift_decode cap {cap} tol {tol}: fatal calls {fatal}, guarded {st.guarded}")
    if cap_q == 5:
        assert not fatal


def _drift_cases():
    rng = np.random.default_rng(31)
    cases = []
    for P in (2, 8, 33, 64):
        for R in (0, 1, 2, 5):
            eh = min(int(rng.choice([1, 3, 16, 40])), 1024 // P)
            K = min(int(rng.choice([1, 2, 8])), P * eh)
            S = int(rng.choice([4, 50, 200]))
            H = int(rng.choice([1, 2, 5]))
            delta = (int(rng.choice([0, 1, 3])), 100)
            cases.append((P, eh, K, R, S, H, delta))
    return cases


@pytest.mark.parametrize("P,eh,K,R,S,H,delta", _drift_cases())
def test_drift_sequences_sweep(P, eh, K, R, S, H, delta):
    """Short sequences (12 calls, popularity changing every 4) over shapes,
    check intervals and thresholds; some with rank speeds."""
    E, N = P * eh, P * S
    cap = 2 * S * K if R > 0 else N * K
    dg = mb.Dims.make(N, K, E, P, R, 16, cap=cap, dtype_in="bf16", dtype_out="bf16")
    od = O.make_dims(N, K, E, P, R, 16, cap=cap, dtype_in="bf16", dtype_out="bf16")
    speeds = None
    if (P + R) % 2:
        speeds = np.random.default_rng(P * 7 + R).integers(1000, 3000, P).astype(np.int32)
    state = _gpu_drift_state(dg)
    st = O.DriftState(E, P, R)
    gprm, oprm = mb.DriftParams(delta[0], delta[1], 3, H), O.DriftParams(delta[0], delta[1], 3, H)
    gp = G.GpuPlan(dg)
    for call in range(12):
        ids, _ = W.routing(N, E, K, W.NOISE_GUMBEL, 1.1, 0.9, 12000 + P * 100 + call,
                           pop_seed=13000 + P * 100 + call // 4)
        got = gp.run(ids, speeds=speeds, drift=(gprm, state)).fetch()
        ref = O.plan(od, ids, speeds=speeds, drift=(oprm, st))
        G.assert_plan_equal(got, ref)
        _assert_state_equal(state, st, E, f"P{P} R{R} call {call}")


# ---- quota repair ------------------------------------------------------------------

def test_hand_example_repair_on_gpu():
    """The hand-derived repair example through mb_plan_ex: quotas repaired as
    stored, and the whole plan equal to the oracle's."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "hand_example_repair.json")))
    dd = dict(g["dims"])
    dd["hidden"] = 8
    ids = np.array(g["ids"], np.int32).reshape(-1, 1)
    dg = mb.Dims.make(**dd, dtype_in="bf16", dtype_out="bf16")
    od = O.make_dims(**dd, dtype_in="bf16", dtype_out="bf16")
    got = G.GpuPlan(dg).run(ids, repair=True).fetch()
    assert np.array_equal(got["slot_quota"].reshape(2, 5), g["slot_quota_repaired"])
    G.assert_plan_equal(got, O.plan(od, ids, repair=True))
    plain = G.GpuPlan(dg).run(ids).fetch()
    assert np.array_equal(plain["slot_quota"].reshape(2, 5), g["slot_quota_placed"])


def test_repair_pattern_sweep():
    """40 pattern inputs (2 to 64 ranks, 2 to 4 slots) with the repair: every
    plan bit-exact; rows dispatched and combined on every fifth case."""
    from tests.crafted import repair_cases, repair_pattern_ids

    for n, (P, pairs, R, seed) in enumerate(repair_cases()):
        ids = repair_pattern_ids(P, pairs, seed)
        N, E, H = 8 * P, 3 * P, 64
        dg = mb.Dims.make(N, 1, E, P, R, H, cap=16, dtype_in="f32", dtype_out="f32")
        od = O.make_dims(N, 1, E, P, R, H, cap=16, dtype_in="f32", dtype_out="f32")
        G.log(f"repair pattern P={P} pairs={len(pairs)} R={R} seed={seed}")
        gp = G.GpuPlan(dg).run(ids, repair=True)
        ref = O.plan(od, ids, repair=True)
        G.assert_plan_equal(gp.fetch(), ref)
        if n % 5 == 0:
            w = np.ones((N, 1), np.float32)
            x = W.rows_f32(seed, W.TAG_X, H, n=N)
            ye = W.rows_f32(seed, W.TAG_YEXP, H, n=P * 16)
            buf, _, y = G.run_rows(dg, gp, x, None, ye, w)
            ref_buf, _, _ = O.dispatch(od, ref, x, None)
            used = ref.row_src >= 0
            assert np.array_equal(buf[used], ref_buf[used])
            y_ref, mag, _ = O.combine(od, ref.pos, ref.status, w, ye)
            G.assert_combine_close(y, y_ref, mag, "f32")


@pytest.mark.parametrize("name", ["tiny", "mixtral", "decode_drift", "kimi_prefill"])
def test_repair_on_workloads_gpu(name):
    wl = W.get_workload(name)
    ids, _ = W.routing_for(wl)
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    G.assert_plan_equal(G.GpuPlan(dg).run(ids, repair=True).fetch(), O.plan(od, ids, repair=True))


def test_repair_with_speeds_and_drift():
    """All three options at once over a 10-call sequence of pattern inputs
    whose planted pairs change every 3 calls, in lockstep with the oracle."""
    from tests.crafted import repair_pattern_ids

    P, R = 13, 3
    N, E = 8 * P, 3 * P
    dg = mb.Dims.make(N, 1, E, P, R, 8, cap=24, dtype_in="bf16", dtype_out="bf16")
    od = O.make_dims(N, 1, E, P, R, 8, cap=24, dtype_in="bf16", dtype_out="bf16")
    speeds = np.random.default_rng(3).integers(900, 1100, P).astype(np.int32)
    state = mb.alloc_drift_state(dg, G.dev())
    st = O.DriftState(E, P, R)
    gprm, oprm = mb.DriftParams(1, 10, 4, 2), O.DriftParams(1, 10, 4, 2)
    gp = G.GpuPlan(dg)
    for call in range(10):
        rng = np.random.default_rng(call // 3)
        perm = rng.permutation(P)
        pairs = [(int(perm[2 * i]), int(perm[2 * i + 1])) for i in range(3)]
        ids = repair_pattern_ids(P, pairs, call)
        got = gp.run(ids, speeds=speeds, drift=(gprm, state), repair=True).fetch()
        ref = O.plan(od, ids, speeds=speeds, drift=(oprm, st), repair=True)
        G.assert_plan_equal(got, ref)
        _assert_state_equal(state, st, E, f"call {call}")


# ---- dequantising fp8 combine ------------------------------------------------------

def _combine_fp8_case(N, K, E, P, R, H, dout, seed, label):
    ids, w = W.routing(N, E, K, W.NOISE_GUMBEL, 1.1, 1.0, seed)
    cap = 2 * (N // P) * K
    dg = mb.Dims.make(N, K, E, P, R, H, cap=cap, dtype_in="fp8", dtype_out=dout)
    od = O.make_dims(N, K, E, P, R, H, cap=cap, dtype_in="fp8", dtype_out=dout)
    G.log(f"combine_fp8 {label}: N={N} K={K} H={H} out={dout}")
    gp = G.GpuPlan(dg).run(ids)
    ref = O.plan(od, ids)
    rows = P * cap
    q, sc, _ = W.rows_fp8(seed, W.TAG_YEXP, H, n=rows)
    d = G.dev()
    q_d = torch.from_numpy(q).to(d)
    sc_d = torch.from_numpy(sc).to(d)
    w_d = torch.from_numpy(w).to(d)
    odt = torch.bfloat16 if dout == "bf16" else torch.float32
    y = torch.full((N, H), float("nan"), dtype=odt, device=d)
    mb.combine_fp8(dg, gp.bufs, q_d, sc_d, w_d, y)
    torch.cuda.synchronize()
    y_ref, mag, rc = O.combine_fp8(od, ref.pos, ref.status, w, q, sc)
    if ref.status[0] & O.ST_FATAL:
        assert torch.isnan(y.float()).all()
        return
    G.assert_combine_close(G.y_to_f64(y), y_ref, mag, dout)


@pytest.mark.parametrize("H", [128, 384, 1024, 1152, 7168, 16384, 17408])
@pytest.mark.parametrize("K", [1, 3, 8])
def test_combine_fp8_shapes(H, K):
    """Whole-KiB rows up to 16 KiB take the straight-line path, others the
    checked loop; K = 3 takes the runtime-K kernel."""
    for dout in ("bf16", "f32"):
        _combine_fp8_case(512, K, 32, 8, 1, H, dout, 4000 + H + K, f"H{H} K{K}")


def test_combine_fp8_decode_round_trip():
    """The decode workload's fp8 dispatch buffer (rows and scales) combined
    by mb_combine_fp8 against the oracle, and with one-hot weights the
    exact dequantisation of each token's row (bf16 of the fp32 q * scale)."""
    wl = W.get_workload("decode_drift")
    ids, w = W.routing_for(wl, 3)
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    x, xs = W.token_rows(wl, 3)
    d = G.dev()
    gp = G.GpuPlan(dg).run(ids)
    ref = O.plan(od, ids)
    buf = torch.zeros((dg.rows, wl.hidden), dtype=torch.uint8, device=d)
    bs = torch.zeros((dg.rows, wl.hidden // 128), dtype=torch.float32, device=d)
    x_d, xs_d = torch.from_numpy(x).to(d), torch.from_numpy(xs).to(d)
    mb.dispatch(dg, gp.bufs, x_d, buf, xs_d, bs)
    y = torch.empty((wl.n_tokens, wl.hidden), dtype=torch.bfloat16, device=d)
    mb.combine_fp8(dg, gp.bufs, buf, bs, torch.from_numpy(w).to(d), y)
    torch.cuda.synchronize()
    t0, t1 = 0, 256
    ref_buf, ref_bs, _ = O.dispatch(od, ref, x, xs)
    y_ref, mag, _ = O.combine_fp8(od, ref.pos, ref.status, w, ref_buf, ref_bs, t0, t1)
    G.assert_combine_close(G.y_to_f64(y[t0:t1]), y_ref, mag, "bf16")
    onehot = np.zeros_like(w)
    onehot[:, 0] = 1.0
    mb.combine_fp8(dg, gp.bufs, buf, bs, torch.from_numpy(onehot).to(d), y)
    deq = torch.from_numpy(x).view(torch.float8_e4m3fn).float() * \
        torch.from_numpy(xs).repeat_interleave(128, dim=1)
    # equal values (a -0 code comes back as +0: the accumulator starts at +0)
    assert torch.equal(y.cpu().float(), deq.to(torch.bfloat16).float())


def test_combine_fp8_fatal_status_writes_nothing():
    N, K, E, P = 64, 2, 8, 4
    ids = np.zeros((N, K), np.int32)
    ids[:, 1] = 1
    ids[5, 1] = 0  # duplicate id: fatal
    dg = mb.Dims.make(N, K, E, P, 1, 128, dtype_in="fp8", dtype_out="bf16")
    gp = G.GpuPlan(dg).run(ids)
    d = G.dev()
    q = torch.zeros((dg.rows, 128), dtype=torch.uint8, device=d)
    sc = torch.ones((dg.rows, 1), dtype=torch.float32, device=d)
    y = torch.full((N, 128), float("nan"), dtype=torch.bfloat16, device=d)
    mb.combine_fp8(dg, gp.bufs, q, sc, torch.ones((N, K), device=d), y)
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()


# ---- HIP graph capture ---------------------------------------------------------------

def test_graph_capture_replays():
    """plan + dispatch + combine captured once in a HIP graph (no host
    synchronisation, no allocation, no memset inside the calls) and replayed
    on three different routings copied into the captured inputs, with eager
    library work between the replays: every replay equals the oracle."""
    wl = W.get_workload("mixtral")
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    d = G.dev()
    ids0, w0 = W.routing_for(wl, 0)
    x0, _ = W.token_rows(wl, 0)
    ids_s = torch.from_numpy(ids0).to(d)
    w_s = torch.from_numpy(w0).to(d)
    x_s = G.torch_rows(x0, O.BF16)
    bufs = mb.PlanBuffers.allocate(dg, d)
    ws = mb.alloc_workspace(dg, d)
    buf = torch.zeros((dg.rows, dg.hidden), dtype=torch.bfloat16, device=d)
    y = torch.zeros((dg.n_tokens, dg.hidden), dtype=torch.bfloat16, device=d)

    def layer():
        mb.plan(dg, ids_s, ws, bufs)
        mb.dispatch(dg, bufs, x_s, buf)
        mb.combine(dg, bufs, buf, w_s, y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    other = G.GpuPlan(dg)
    for call in (3, 7, 11):
        ids, w = W.routing_for(wl, call)
        x, _ = W.token_rows(wl, call)
        ids_s.copy_(torch.from_numpy(ids))
        w_s.copy_(torch.from_numpy(w))
        x_s.copy_(G.torch_rows(x, O.BF16))
        graph.replay()
        other.run(W.routing_for(wl, call + 1)[0])  # eager work between replays
        torch.cuda.synchronize()
        ref = O.plan(od, ids)
        got = {k: getattr(bufs, k).cpu().numpy() for k in G.PLAN_FIELDS}
        got["rep_expert"] = got["rep_expert"][:, : dg.slots_per_rank]
        G.assert_plan_equal(got, ref)
        ref_buf, _, _ = O.dispatch(od, ref, x, None)
        used = ref.row_src >= 0
        assert np.array_equal(G.rows_to_bytes(buf)[used], ref_buf[used]), call
        y_ref, mag, _ = O.combine(od, ref.pos, ref.status, w, ref_buf.view(np.uint16).reshape(
            -1, od.hidden))
        G.assert_combine_close(G.y_to_f64(y), y_ref, mag, "bf16")


def test_graph_capture_drift_state_advances():
    """A drift-gated plan captured in a graph: each replay advances the
    caller's state exactly as the oracle's sequence does."""
    wl = W.get_workload("drift_decode")
    dg, od = mb.Dims.for_workload(wl), O.dims_for(wl)
    dg.hidden = od.hidden = 128
    d = G.dev()
    num, den, win, _, tn, td = wl.drift
    gprm, oprm = mb.DriftParams(num, den, win, 2, tn, td), O.DriftParams(num, den, win, 2, tn, td)
    ids_s = torch.from_numpy(W.routing_for(wl, 0)[0]).to(d)
    state = mb.alloc_drift_state(dg, d)
    st = O.DriftState(wl.n_experts, wl.n_ranks, wl.slots_per_rank)
    gp = G.GpuPlan(dg)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mb.plan(dg, ids_s, gp.ws, gp.bufs, drift=(gprm, state))
    torch.cuda.current_stream().wait_stream(side)
    state.zero_()  # the warm-up call above advanced it
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mb.plan(dg, ids_s, gp.ws, gp.bufs, drift=(gprm, state))
    state.zero_()  # capture does not run the kernels; start fresh anyway
    for call in range(0, 30, 3):
        ids, _ = W.routing_for(wl, call)
        ids_s.copy_(torch.from_numpy(ids))
        graph.replay()
        torch.cuda.synchronize()
        ref = O.plan(od, ids, drift=(oprm, st))
        G.assert_plan_equal(gp.fetch(), ref)
        _assert_state_equal(state, st, wl.n_experts, f"replay at call {call}")


def test_graph_capture_weighted_repair_fp8():
    """The fp8 decode path captured in one graph: mb_plan_weighted with the
    quota repair, the fp8 dispatch with its scale rows, and mb_combine_fp8,
    replayed on three routings copied into the captured inputs with eager
    library work between the replays; every replay equals the oracle (plan
    bit-exact, rows and scales byte-exact, combine on two token ranges). The
    repair leaves these plans as placed; the next test captures one that
    changes them."""
    wl = W.get_workload("decode_drift")
    # uneven speeds move rows toward the fast ranks: room for 1.5x the even share
    dg, od = mb.Dims.for_workload(wl, cap=3 * wl.cap // 2), O.dims_for(wl, cap=3 * wl.cap // 2)
    d = G.dev()
    speeds = np.random.default_rng(77).integers(4000, 8001, wl.n_ranks).astype(np.int32)
    ids0, w0 = W.routing_for(wl, 0)
    x0, xs0 = W.token_rows(wl, 0)
    ids_s, w_s = torch.from_numpy(ids0).to(d), torch.from_numpy(w0).to(d)
    x_s, xs_s = torch.from_numpy(x0).to(d), torch.from_numpy(xs0).to(d)
    bufs = mb.PlanBuffers.allocate(dg, d)
    ws = mb.alloc_workspace(dg, d)
    buf = torch.zeros((dg.rows, dg.hidden), dtype=torch.uint8, device=d)
    bs = torch.zeros((dg.rows, dg.hidden // 128), dtype=torch.float32, device=d)
    y = torch.zeros((dg.n_tokens, dg.hidden), dtype=torch.bfloat16, device=d)

    def layer():
        mb.plan(dg, ids_s, ws, bufs, speeds=speeds.tolist(), repair=True)
        mb.dispatch(dg, bufs, x_s, buf, xs_s, bs)
        mb.combine_fp8(dg, bufs, buf, bs, w_s, y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    other = G.GpuPlan(dg)
    for call in (2, 5, 9):
        ids, w = W.routing_for(wl, call)
        x, xs = W.token_rows(wl, call)
        ids_s.copy_(torch.from_numpy(ids))
        w_s.copy_(torch.from_numpy(w))
        x_s.copy_(torch.from_numpy(x))
        xs_s.copy_(torch.from_numpy(xs))
        graph.replay()
        other.run(W.routing_for(wl, call + 1)[0], repair=True)  # eager work between replays
        torch.cuda.synchronize()
        ref = O.plan(od, ids, speeds=speeds, repair=True)
        got = {k: getattr(bufs, k).cpu().numpy() for k in G.PLAN_FIELDS}
        got["rep_expert"] = got["rep_expert"][:, : dg.slots_per_rank]
        G.assert_plan_equal(got, ref)
        ref_buf, ref_bs, _ = O.dispatch(od, ref, x, xs)
        used = ref.row_src >= 0
        assert np.array_equal(buf.cpu().numpy()[used], ref_buf[used]), call
        assert np.array_equal(bs.cpu().numpy().view(np.uint32)[used],
                              ref_bs.view(np.uint32)[used]), call
        for t0, t1 in ((0, 192), (dg.n_tokens - 192, dg.n_tokens)):
            y_ref, mag, _ = O.combine_fp8(od, ref.pos, ref.status, w, ref_buf, ref_bs, t0, t1)
            G.assert_combine_close(G.y_to_f64(y[t0:t1]), y_ref, mag, "bf16")


def test_graph_capture_repair_changes_quotas():
    """mb_plan_ex with the repair, mb_dispatch and mb_combine captured once
    and replayed on repair pattern inputs where the repair moves quota (and
    so positions) away from the placed plan: each replay equals the oracle's
    repaired plan, rows and combine."""
    from tests.crafted import repair_pattern_ids

    P, R, H = 8, 2, 64
    N, E = 8 * P, 3 * P
    dg = mb.Dims.make(N, 1, E, P, R, H, cap=16, dtype_in="f32", dtype_out="f32")
    od = O.make_dims(N, 1, E, P, R, H, cap=16, dtype_in="f32", dtype_out="f32")
    d = G.dev()
    cases = [([(0, 1)], 1), ([(2, 5), (3, 7)], 2), ([(6, 7)], 4)]
    ids_s = torch.from_numpy(repair_pattern_ids(P, *cases[0])).to(d)
    w = np.ones((N, 1), np.float32)
    w_s = torch.from_numpy(w).to(d)
    x_s = torch.zeros((N, H), dtype=torch.float32, device=d)
    ye = W.rows_f32(5, W.TAG_YEXP, H, n=P * 16)
    ye_s = torch.from_numpy(ye).to(d)
    bufs = mb.PlanBuffers.allocate(dg, d)
    ws = mb.alloc_workspace(dg, d)
    buf = torch.zeros((dg.rows, H), dtype=torch.float32, device=d)
    y = torch.zeros((N, H), dtype=torch.float32, device=d)

    def layer():
        mb.plan(dg, ids_s, ws, bufs, repair=True)
        mb.dispatch(dg, bufs, x_s, buf)
        mb.combine(dg, bufs, ye_s, w_s, y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    other = G.GpuPlan(dg)
    for pairs, seed in cases:
        ids = repair_pattern_ids(P, pairs, seed)
        x = W.rows_f32(seed, W.TAG_X, H, n=N)
        ids_s.copy_(torch.from_numpy(ids))
        x_s.copy_(torch.from_numpy(x))
        graph.replay()
        other.run(ids)  # eager, unrepaired, between replays
        torch.cuda.synchronize()
        ref = O.plan(od, ids, repair=True)
        assert not np.array_equal(ref.slot_quota, O.plan(od, ids).slot_quota), seed
        got = {k: getattr(bufs, k).cpu().numpy() for k in G.PLAN_FIELDS}
        got["rep_expert"] = got["rep_expert"][:, : dg.slots_per_rank]
        G.assert_plan_equal(got, ref)
        ref_buf, _, _ = O.dispatch(od, ref, x, None)
        used = ref.row_src >= 0
        assert np.array_equal(G.rows_to_bytes(buf)[used], ref_buf[used]), seed
        y_ref, mag, _ = O.combine(od, ref.pos, ref.status, w, ye)
        G.assert_combine_close(y.cpu().numpy().astype(np.float64), y_ref, mag, "f32")
