"""The seeded input generator: determinism, shapes, encodings.

The generator holds no method arithmetic; these checks make sure the inputs
both sides receive are what the workload recipes say.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workload as W
from workload.tune import routing_stats


def test_routing_shapes_and_properties():
    ids, w = W.routing(512, 16, 4, W.NOISE_NORMAL, 1.2, 1.0, 7)
    assert ids.shape == (512, 4) and w.shape == (512, 4)
    assert ids.min() >= 0 and ids.max() < 16
    for row in ids:
        assert len(set(row.tolist())) == 4  # distinct experts per token
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # listed in descending logit order


def test_routing_deterministic_and_seeded():
    a = W.routing(256, 32, 8, W.NOISE_GUMBEL, 1.1, 1.0, 123)
    b = W.routing(256, 32, 8, W.NOISE_GUMBEL, 1.1, 1.0, 123)
    c = W.routing(256, 32, 8, W.NOISE_GUMBEL, 1.1, 1.0, 124)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])


def test_zipf_popularity_and_permutation():
    perm = W.permutation(9, 50)
    assert sorted(perm.tolist()) == list(range(50))
    lnp = W.log_popularity(9, 50, 1.0)
    p = np.exp(lnp)
    assert p.sum() == pytest.approx(1.0)
    # popularity rank j (1-based) holds p proportional to j^-s
    ranked = p[perm]
    np.testing.assert_allclose(ranked / ranked[0], np.arange(1, 51, dtype=float) ** -1.0, rtol=1e-12)


def test_gumbel_beta1_is_plackett_luce_first_choice():
    """With Gumbel noise and beta = 1 the top-1 expert is drawn with
    probability p(e) (Gumbel-max)."""
    n, E = 40000, 6
    ids, _ = W.routing(n, E, 1, W.NOISE_GUMBEL, 1.0, 1.0, 5)
    p = np.exp(W.log_popularity(5, E, 1.0))
    freq = np.bincount(ids.ravel(), minlength=E) / n
    np.testing.assert_allclose(freq, p, atol=0.01)


def test_rows_are_counter_based():
    full = W.rows_f32(11, W.TAG_X, 64, n=20)
    part = W.rows_f32(11, W.TAG_X, 64, n=5, row0=7)
    sel = W.rows_f32(11, W.TAG_X, 64, rows=[19, 3, 7])
    assert np.array_equal(full[7:12], part)
    assert np.array_equal(sel, full[[19, 3, 7]])
    big = W.rows_f32(11, W.TAG_X, 256, n=400)
    assert abs(big.mean()) < 0.02 and abs(big.std() - 1) < 0.02


def test_bf16_encoding_matches_torch():
    v = np.concatenate([W.rows_f32(3, W.TAG_X, 128, n=64).ravel(),
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -1.0000001, 65504.5], np.float32)])
    ours = np.array([W.lib().mbgen_f32_to_bf16(float(f)) for f in v], np.uint16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    bulk = W.rows_bf16(3, W.TAG_X, 128, n=64)
    assert np.array_equal(bulk.ravel(), ours[: 64 * 128])


def test_e4m3_encoding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 100, 4000), rng.normal(0, 0.01, 2000),
                        [0.0, 448.0, -448.0, 0.001953125, 0.0009765625, 2.0 ** -6, 15.5, 17.0]])
    v = np.clip(v, -448, 448).astype(np.float32)
    ours = np.array([W.lib().mbgen_f32_to_e4m3(float(f)) for f in v], np.uint8)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    back = np.array([W.lib().mbgen_e4m3_to_f32(int(c)) for c in range(256) if (c & 0x7F) != 0x7F],
                    np.float32)
    ref_back = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=torch.uint8) \
        .view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(back, ref_back)


def test_fp8_rows_scales_and_dequant():
    q, sc, deq = W.rows_fp8(5, W.TAG_X, 256, n=8, want_dequant=True)
    x = W.rows_f32(5, W.TAG_X, 256, n=8)
    amax = np.abs(x.reshape(8, 2, 128)).max(-1)
    np.testing.assert_allclose(sc, amax / 448.0, rtol=1e-7)
    dq = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy().reshape(8, 2, 128) * sc[..., None]
    ref = torch.from_numpy(dq.reshape(8, 256).astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(deq, ref)
    assert np.all(np.abs(dq.reshape(8, 256) - x) <= np.repeat(sc, 128, axis=1) * 16.0)


def test_workloads_recipe():
    for name in W.configs.ORDER + W.configs.EXTRA_ORDER:
        wl = W.get_workload(name)
        assert wl.n_tokens % wl.n_ranks == 0 and wl.n_experts % wl.n_ranks == 0
        assert wl.cap == (wl.cap_rows or wl.tokens_per_rank * wl.top_k)
        assert wl.cap >= wl.tokens_per_rank * wl.top_k


@pytest.mark.parametrize("name", ["dsv3_prefill", "kimi_prefill"])
def test_prefill_skew_near_targets(name):
    """Pre-plan statistics of the tuned prefill workloads are near their
    targets (routing statistics only)."""
    wl = W.get_workload(name)
    ids, _ = W.routing_for(wl)
    st = routing_stats(ids, wl.n_experts, wl.n_ranks)
    if name == "dsv3_prefill":
        assert abs(st["group8_max_share"] - 0.24) < 0.03
        assert abs(st["group8_min_share"] - 0.10) < 0.035
    else:
        assert abs(st["top4_share"] - 0.13) < 0.01
        assert abs(st["ir_before"] - 1.45) < 0.05


@pytest.mark.parametrize("name", W.configs.SWEEP_ORDER)
def test_maxvio_sweep_targets(name):
    """The MoonEP-shaped sweep reaches its maxvio target from the routing
    alone (max over mean routed pairs per expert, minus one)."""
    wl = W.get_workload(name)
    ids, _ = W.routing_for(wl)
    c = np.bincount(ids.ravel(), minlength=wl.n_experts)
    maxvio = c.max() / c.mean() - 1.0
    target = wl.targets["maxvio"]
    assert abs(maxvio - target) < 0.01 * target
