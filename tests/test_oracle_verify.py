"""Pins for the oracle's speculative-sampling verification.

* Exact: the lossless property ("LongSpark", sec. 2.1: accepting a drafts and
  emitting one more token preserves the target distribution).  The oracle's
  ``verify_request`` runs under exhaustive enumeration of every random choice
  it makes, in exact rational arithmetic, across several rounds of a toy
  target / drafter; the law of the first T emitted tokens must equal the
  autoregressive law of the target.
* Exact: the per-position acceptance rate ``alpha_j = sum_v min(P_j, Q_j)``
  ("ForeSpark", sec. 4.5) composes to P(a >= j) = prod_{t<=j} alpha_t.
* Statistical and special cases on the full float64 path with Philox draws.
"""
import itertools
from collections import defaultdict
from fractions import Fraction as Fr

import numpy as np
import pytest
from scipy import special, stats

from oracle import lm_head as ol
from oracle import verify as ov

# ------------------------------------------------------------ enumeration


class _Need(Exception):
    def __init__(self, options):
        self.options = options


def _enumerate(p_rows, q_rows, y, nv, grid):
    """All outcomes of one ``verify_request`` call with their exact
    probabilities.  Acceptance uniforms range over the grid {m / grid} (each
    equally likely); a draw proportional to weights w picks index t with
    probability w_t / sum(w)."""
    out = defaultdict(Fr)
    stack = [[]]
    while stack:
        script = stack.pop()
        cursor = [0]

        def choose(options):
            i = cursor[0]
            if i < len(script):
                cursor[0] += 1
                return script[i][0]
            raise _Need(options)

        def accept_u(j):
            return choose([(Fr(m, grid), Fr(1, grid)) for m in range(grid)])

        def sample(w, j):
            tot = sum(w)
            return choose([(t, Fr(w[t]) / tot) for t in range(len(w)) if w[t] > 0])

        try:
            a, c, _ = ov.verify_request(p_rows, q_rows, y, nv, accept_u, sample)
        except _Need as n:
            for opt in n.options:
                stack.append(script + [opt])
            continue
        pr = Fr(1)
        for _, p in script:
            pr *= p
        out[(a, c)] += pr
    return out


def _row(*xs):
    return np.array([Fr(x) for x in xs], dtype=object)


# target rows: multiples of 1/8 (zeros allowed); drafter rows: entries in
# {0, 1/4, 1/2} so that every ratio p/q is a multiple of 1/4
P_TABLE = [_row(Fr(1, 8), Fr(3, 8), Fr(4, 8)), _row(Fr(5, 8), 0, Fr(3, 8)),
           _row(Fr(2, 8), Fr(2, 8), Fr(4, 8)), _row(0, Fr(7, 8), Fr(1, 8)),
           _row(Fr(6, 8), Fr(1, 8), Fr(1, 8)), _row(Fr(3, 8), Fr(3, 8), Fr(2, 8))]
Q_TABLE = [_row(Fr(1, 2), Fr(1, 4), Fr(1, 4)), _row(Fr(1, 4), Fr(1, 2), Fr(1, 4)),
           _row(Fr(1, 4), Fr(1, 4), Fr(1, 2)), _row(Fr(1, 2), Fr(1, 2), 0),
           _row(0, Fr(1, 2), Fr(1, 2)), _row(Fr(1, 2), 0, Fr(1, 2))]
GRID = 4


def _p(h):
    return P_TABLE[(7 * len(h) + sum((i + 2) * t for i, t in enumerate(h))) % len(P_TABLE)]


def _q(h, j):
    return Q_TABLE[(3 * len(h) + 5 * j + sum(h)) % len(Q_TABLE)]


def _round(h, K, nv, target=_p):
    """Law of the tokens one round emits from history h (tuple -> prob)."""
    q_rows = [_q(h, j) for j in range(1, K + 1)]
    out = defaultdict(Fr)
    supports = [[t for t in range(3) if q[t] > 0] for q in q_rows]
    for y in itertools.product(*supports):
        py = Fr(1)
        for j, t in enumerate(y):
            py *= q_rows[j][t]
        p_rows = [target(h + y[:j]) for j in range(nv + 1)]
        for (a, c), pr in _enumerate(p_rows, q_rows, y, nv, GRID).items():
            out[tuple(y[:a]) + (c,)] += py * pr
    return out


def _first_T(h, T, K, nv, memo):
    key = (h, T)
    if key in memo:
        return memo[key]
    res = defaultdict(Fr)
    for em, pr in _round(h, K, nv).items():
        if len(em) >= T:
            res[em[:T]] += pr
        else:
            for rest, pr2 in _first_T(h + em, T - len(em), K, nv, memo).items():
                res[em + rest] += pr * pr2
    memo[key] = res
    return res


def _ar_law(T):
    law = {}
    for seq in itertools.product(range(3), repeat=T):
        pr = Fr(1)
        for t in range(T):
            pr *= _p(seq[:t])[seq[t]]
        law[seq] = pr
    return law


@pytest.mark.parametrize("K,nv", [(2, 2), (3, 3), (3, 1), (2, 0)])
def test_lossless_exact_enumeration(K, nv):
    T = 3
    got = _first_T((), T, K, nv, {})
    ar = _ar_law(T)
    assert sum(got.values()) == 1
    for seq, pr in ar.items():
        assert got.get(seq, Fr(0)) == pr, (seq, got.get(seq), pr)


def test_enumeration_detects_a_wrong_residual(monkeypatch):
    # The enumeration is sharp: a residual of [q - p]_+ breaks losslessness.
    monkeypatch.setattr(ov, "residual_weights",
                        lambda p, q: np.where(q - p > 0, q - p, 0 * p))
    got = _first_T((), 2, 2, 2, {})
    assert any(got.get(s, Fr(0)) != pr for s, pr in _ar_law(2).items())


def test_acceptance_rate_closed_form():
    # Target rows fixed per position (independent of the drafts): the
    # probability of accepting at least j drafts is prod_{t<=j} alpha_t with
    # alpha_t = sum_v min(p_t(v), q_t(v)).
    K = 3
    fixed = {0: P_TABLE[0], 1: P_TABLE[2], 2: P_TABLE[4], 3: P_TABLE[1]}
    h = ()
    q_rows = [_q(h, j) for j in range(1, K + 1)]
    p_rows = [fixed[j] for j in range(K + 1)]
    dist = defaultdict(Fr)
    supports = [[t for t in range(3) if q[t] > 0] for q in q_rows]
    for y in itertools.product(*supports):
        py = Fr(1)
        for j, t in enumerate(y):
            py *= q_rows[j][t]
        for (a, c), pr in _enumerate(p_rows, q_rows, y, K, GRID).items():
            dist[a] += py * pr
    alpha = [sum(min(p[v], q[v]) for v in range(3)) for p, q in zip(p_rows, q_rows)]
    for j in range(1, K + 1):
        p_ge = sum(pr for a, pr in dist.items() if a >= j)
        expect = Fr(1)
        for t in range(j):
            expect *= alpha[t]
        assert p_ge == expect


# ------------------------------------------------ float64 path with Philox


def _mc_requests(n_req, z_draft, x_target, K, seed=0x5EED):
    """n_req independent requests sharing the same draft and target logits;
    drafts come from the oracle's Gumbel-max sampler."""
    V = z_draft.shape[1]
    q_off = np.arange(n_req + 1) * K
    t_off = np.arange(n_req + 1) * (K + 1)
    req_id = (np.arange(n_req, dtype=np.uint64) * 2246822519 + 7) % (2 ** 32)
    req_id = req_id.astype(np.uint32)
    draft_logits = np.tile(z_draft, (n_req, 1)).astype(np.float32)
    target = np.tile(x_target, (n_req, 1)).astype(np.float32)
    rq, pos = ol.row_owner(q_off)
    tok, _ = ol.draft_tokens(draft_logits.astype(np.float64), rq, pos, req_id, seed)
    res = ov.verify(target, t_off, draft_logits, tok, q_off, req_id, seed)
    return tok.reshape(n_req, K), res


def test_first_token_law_and_acceptance_rate_mc():
    rng = np.random.default_rng(1)
    V, K, n = 8, 3, 6000
    z = (rng.standard_normal((K, V)) * 1.0).astype(np.float32)
    x = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    tok, res = _mc_requests(n, z, x, K)
    a = res["accepted"]
    first = np.where(a >= 1, tok[:, 0], res["next_token"])
    p1 = special.softmax(x[0].astype(np.float64))
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p1 * n).pvalue > 1e-3
    p = special.softmax(x.astype(np.float64), axis=1)
    q = special.softmax(z.astype(np.float64), axis=1)
    alpha = np.minimum(p[:K], q).sum(1)
    for j in range(1, K + 1):
        expect = np.prod(alpha[:j])
        got = np.mean(a >= j)
        se = np.sqrt(expect * (1 - expect) / n)
        assert abs(got - expect) < 5 * se + 1e-9


def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(2)
    V, K, n = 50, 4, 200
    z = rng.standard_normal((K + 1, V)).astype(np.float32)
    tok, res = _mc_requests(n, z[:K], z, K)
    assert np.all(res["accepted"] == K)
    # the bonus is a draw from p_{K+1}
    p = special.softmax(z[K].astype(np.float64))
    assert np.all(p[res["next_token"]] > 0)


def test_one_hot_target_is_deterministic():
    V, K, n = 16, 3, 100
    rng = np.random.default_rng(4)
    z = rng.standard_normal((K, V)).astype(np.float32)
    x = np.zeros((K + 1, V), np.float32)
    hot = [5, 9, 2, 14]
    for j, t in enumerate(hot):
        x[j, :] = -2000.0
        x[j, t] = 0.0
    tok, res = _mc_requests(n, z, x, K)
    for i in range(n):
        a = res["accepted"][i]
        emitted = list(tok[i, :a]) + [res["next_token"][i]]
        assert emitted == hot[:a + 1]


def test_one_hot_draft_on_zero_target_rejects_and_corrects_from_p():
    V, K, n = 8, 2, 4000
    rng = np.random.default_rng(6)
    z = np.full((K, V), -2000.0, np.float32)
    z[0, 3] = 0.0                     # q_1 is one-hot at token 3
    z[1, 1] = 0.0
    x = rng.standard_normal((K + 1, V)).astype(np.float32)
    x[0, 3] = -2000.0                 # p_1(3) = 0
    tok, res = _mc_requests(n, z, x, K)
    assert np.all(tok[:, 0] == 3)
    assert np.all(res["accepted"] == 0)
    p1 = special.softmax(x[0].astype(np.float64))
    counts = np.bincount(res["next_token"], minlength=V)
    assert counts[3] == 0
    keep = p1 > 0
    assert stats.chisquare(counts[keep], p1[keep] / p1[keep].sum() * n).pvalue > 1e-3


def test_zero_verify_budget_is_autoregressive():
    V, n = 8, 3000
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, V)).astype(np.float32)
    q_off = np.zeros(n + 1, np.int64)          # no drafts verified
    t_off = np.arange(n + 1)
    req_id = np.arange(n, dtype=np.uint32) + 11
    res = ov.verify(np.tile(x, (n, 1)), t_off, np.zeros((0, V), np.float32),
                    np.zeros(0, np.int32), q_off, req_id, 77)
    assert np.all(res["accepted"] == 0)
    counts = np.bincount(res["next_token"], minlength=V)
    p = special.softmax(x[0].astype(np.float64))
    assert stats.chisquare(counts, p * n).pvalue > 1e-3


def test_enumeration_detects_an_inverted_ratio(monkeypatch):
    monkeypatch.setattr(ov, "accept_probability",
                        lambda p, q: 1 if p == 0 else min(Fr(1), Fr(q) / Fr(p)))
    got = _first_T((), 2, 2, 2, {})
    assert any(got.get(s, Fr(0)) != pr for s, pr in _ar_law(2).items())
