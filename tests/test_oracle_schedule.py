"""Pins for the oracle's ForeSpark scheduling ("ForeSpark", sec. 4.2-4.4).

* the printed worked example (Fig. 5: benefits 0.9, 0.7, 0.3 give
  Reward(3, 3) = 1.9), from ``tests/golden/forespark_fig5_reward.json``;
* the concave envelope against scipy's convex hull (upper hull of the reward
  points) and its defining properties; scores non-increasing;
* the directional-drafter special case (sec. 4.2: rows are prefixes of the
  last row, so the reward curve is already concave and the scores are the
  survival benefits themselves);
* the bucket-pair search of eq. (4) against an exhaustive search over every
  (sum d_i, B);
* the prefix property of both selections (sec. 4.3, 4.4);
* the estimators (eqs. (2), (5)) against torch.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.spatial import ConvexHull

from oracle import schedule as osch
from oracle.attention import bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "forespark_fig5_reward.json")


def _logit(p):
    return float(np.log(p / (1 - p)))


def test_fig5_worked_example():
    g = json.load(open(GOLDEN))
    S_target = g["survival_benefits"]
    K = g["draft_length"]
    z = np.zeros(K * (K + 1) // 2)
    prev = 1.0
    for t, s in enumerate(S_target, start=1):
        z[osch.tri_index(K, t)] = _logit(s / prev)    # conditional acceptance
        prev = s
    S = osch.survival_benefits(z, K)
    np.testing.assert_allclose(S[K - 1], S_target, rtol=0, atol=1e-15)
    assert abs(osch.reward(S, K, K) - g["reward_3_3"]) < 1e-15


def _upper_hull(R):
    K = len(R) - 1
    pts = np.stack([np.arange(K + 1), R], 1).astype(np.float64)
    # add a point far below so the hull always has an upper chain over all x
    pts = np.vstack([pts, [[0.0, R.min() - 100.0], [float(K), R.min() - 100.0]]])
    hull = ConvexHull(pts)
    up = sorted({tuple(pts[i]) for i in hull.vertices if pts[i, 1] > R.min() - 50.0})
    xs, ys = zip(*up)
    return np.interp(np.arange(K + 1), xs, ys)


@pytest.mark.parametrize("seed", range(8))
def test_envelope_is_the_upper_hull(seed):
    rng = np.random.default_rng(seed)
    K = 16
    R = np.concatenate([[0.0], np.cumsum(rng.uniform(-0.3, 1.0, K))])
    F = osch.concave_envelope(R)
    np.testing.assert_allclose(F, _upper_hull(R), rtol=0, atol=1e-12)
    assert np.all(F >= R - 1e-15)
    assert np.all(np.diff(F, 2) <= 1e-12)              # concave
    g = osch.survival_scores(R)
    assert np.all(np.diff(g) <= 1e-12)                  # non-increasing


def test_concave_curve_is_unchanged():
    R = np.concatenate([[0.0], np.cumsum(np.linspace(1.0, 0.1, 10))])
    np.testing.assert_allclose(osch.concave_envelope(R), R, rtol=0, atol=1e-15)


def test_directional_drafter_scores_are_the_benefits():
    rng = np.random.default_rng(3)
    K = 12
    row_K = rng.normal(1.0, 1.5, K)
    z = np.zeros(K * (K + 1) // 2)
    for d in range(1, K + 1):
        for t in range(1, d + 1):
            z[osch.tri_index(d, t)] = row_K[t - 1]      # every row a prefix of row K
    S = osch.survival_benefits(z, K)
    R = osch.reward_curve(S, K)
    np.testing.assert_allclose(osch.concave_envelope(R), R, rtol=0, atol=1e-14)
    np.testing.assert_allclose(osch.survival_scores(R), S[K - 1], rtol=0, atol=1e-14)


def _random_problem(rng, n, K):
    g = np.empty((n, K))
    for i in range(n):
        R = np.concatenate([[0.0], np.cumsum(rng.uniform(-0.2, 1.0, K) * rng.uniform(0.2, 1.0))])
        g[i] = osch.survival_scores(R)
    nb_d, nb_v = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    d_caps = np.sort(rng.choice(np.arange(n, n * (K + 1) + 8), nb_d, replace=False))
    v_caps = np.sort(rng.choice(np.arange(n, n * (K + 1) + 8), nb_v, replace=False))
    d_lat = np.sort(rng.uniform(1.0, 5.0, nb_d))
    v_lat = np.sort(rng.uniform(2.0, 9.0, nb_v))
    return g, d_caps, d_lat, v_caps, v_lat


@pytest.mark.parametrize("seed", range(10))
def test_bucket_search_reaches_the_exhaustive_optimum(seed):
    rng = np.random.default_rng(seed)
    n, K = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    g, dc, dl, vc, vl = _random_problem(rng, n, K)
    N = n
    res = osch.joint_schedule(g, N, dc, dl, vc, vl)
    best = osch.joint_schedule_exhaustive(g, N, dc, dl, vc, vl)
    if np.isfinite(best):
        assert abs(res["objective"] - best) < 1e-12
        assert res["budget"] <= res["draft_len"].sum()
        # the schedule is a prefix of every request: its scores are the top k
        vals, _ = osch.sorted_scores(g)
        picked = np.concatenate([g[i, :res["draft_len"][i]] for i in range(n)])
        np.testing.assert_allclose(np.sort(picked)[::-1], vals[:res["k"]], rtol=0, atol=0)
    else:
        assert res["objective"] == -np.inf


def test_budget_distribution_is_a_prefix_of_every_draft():
    rng = np.random.default_rng(9)
    d = np.array([0, 3, 16, 7, 1])
    q_off = np.concatenate([[0], np.cumsum(d)])
    p = rng.uniform(0.05, 1.0, q_off[-1])
    for B in (0, 1, 5, 12, 27, 100):
        S, b = osch.distribute_budget(p, q_off, B)
        assert b.sum() == min(B, q_off[-1])
        assert np.all(b <= d)
        chosen = np.concatenate([S[q_off[i]:q_off[i] + b[i]] for i in range(len(d))])
        rest = np.concatenate([S[q_off[i] + b[i]:q_off[i + 1]] for i in range(len(d))])
        if len(chosen) and len(rest):
            assert chosen.min() >= rest.max()


def _bf16(x):
    return (torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def test_predraft_estimator_matches_torch():
    rng = np.random.default_rng(4)
    n, dh, r, K = 5, 64, 32, 6
    T = K * (K + 1) // 2
    c, e = _bf16(rng.normal(0, 1, (n, dh))), _bf16(rng.normal(0, 1, (n, dh)))
    wc, we = _bf16(rng.normal(0, 0.1, (r, dh))), _bf16(rng.normal(0, 0.1, (r, dh)))
    wo = _bf16(rng.normal(0, 0.1, (T, r)))
    bu, bo = rng.normal(0, 0.1, r), rng.normal(0, 0.1, T)
    sc, bi = rng.uniform(0.5, 1.5, T), rng.normal(0, 0.2, T)
    z = osch.predraft_logits(c, e, wc, we, wo, bu, bo, sc, bi)
    t = lambda a: torch.from_numpy(bf16_bits_to_f64(a))
    u = torch.nn.functional.silu(t(c) @ t(wc).T + t(e) @ t(we).T + torch.from_numpy(bu))
    ref = ((u @ t(wo).T + torch.from_numpy(bo)) * torch.from_numpy(sc) + torch.from_numpy(bi))
    np.testing.assert_allclose(z, ref.numpy(), rtol=0, atol=1e-12)


def test_postdraft_estimator_matches_torch():
    rng = np.random.default_rng(5)
    M, H, m, V = 9, 64, 16, 50
    h = _bf16(rng.normal(0, 1, (M, H)))
    ws = _bf16(rng.normal(0, 0.1, (m, H)))
    ep = _bf16(rng.normal(0, 1, (V, m)))
    w = rng.normal(0, 0.1, H + m)
    prev = rng.integers(0, V, M)
    pos = np.array([1, 2, 3, 1, 1, 2, 3, 4, 5])
    temp = rng.uniform(0.5, 2.0, 5)
    p = osch.postdraft_probs(h, ws, ep, w, prev, pos, 0.25, temp)
    t = lambda a: torch.from_numpy(bf16_bits_to_f64(a))
    s = (t(h) @ t(ws).T) * t(ep)[torch.from_numpy(prev)]
    logit = torch.cat([t(h), s], 1) @ torch.from_numpy(w) + 0.25
    ref = torch.sigmoid(logit / torch.from_numpy(temp)[torch.from_numpy(pos - 1)])
    np.testing.assert_allclose(p, ref.numpy(), rtol=0, atol=1e-14)
