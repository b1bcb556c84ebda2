"""Pins for the oracle's sequential (Markov) correction ("LongSpark",
sec. 2.3, eqs. (7)-(8)).

* a zero correction reproduces the factorised proposal's draws (eq. (4));
* the corrected logits equal base + W_c e_c(y_{j-1}) computed with torch from
  the previous draw, position by position (the dependence on y_{j-1});
* a correction that adds a huge bonus to one token forces every draw after
  the first (a closed form: y_j = argmax of that bonus), whatever the base.

"DeLS-Spec" fusion (alpha, unigram-prior bias):
* the smoothed prior is a distribution; uniform counts give 1/V and lambda = 0
  the empirical frequencies (closed forms);
* long logits equal to the log prior, minus the prior (beta = 1, alpha = 0),
  leave a flat row: lse = log V exactly (a sign error would double the prior);
* alpha = 2 equals doubling W_M (exact in bf16).

Temperature 0: every draw is torch.argmax of the corrected row, and the next
row's correction follows that argmax.
"""
import numpy as np
import torch

from oracle import lm_head as olm
from oracle import markov as omk
from oracle.attention import bf16_bits_to_f64


def _bf16(x):
    return (torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def _problem(seed=0, V=50, r=8, d=(3, 5, 1)):
    rng = np.random.default_rng(seed)
    q_off = np.concatenate([[0], np.cumsum(d)]).astype(np.int64)
    M = int(q_off[-1])
    base = rng.normal(0, 1.5, (M, V)).astype(np.float32)
    w_c = _bf16(rng.normal(0, 0.5, (V, r)))
    e_c = _bf16(rng.normal(0, 0.5, (V, r)))
    anchor = rng.integers(0, V, len(d))
    req_id = np.array([11, 22, 33], np.uint32)[:len(d)]
    return base, q_off, anchor, w_c, e_c, req_id


def test_zero_correction_is_the_factorised_proposal():
    base, q_off, anchor, w_c, e_c, req_id = _problem()
    zero = np.zeros_like(w_c)
    got = omk.markov_sample(base, q_off, anchor, zero, e_c, req_id, 1234)
    req, pos = olm.row_owner(q_off)
    tok, _ = olm.draft_tokens(base.astype(np.float64), req, pos, req_id, 1234)
    np.testing.assert_array_equal(got["tokens"], tok)
    np.testing.assert_allclose(got["logits"], base, rtol=0, atol=0)


def test_logits_follow_the_previous_draw():
    base, q_off, anchor, w_c, e_c, req_id = _problem(1)
    got = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 99)
    W = torch.from_numpy(bf16_bits_to_f64(w_c))
    E = torch.from_numpy(bf16_bits_to_f64(e_c))
    for b in range(len(q_off) - 1):
        prev = int(anchor[b])
        for m in range(q_off[b], q_off[b + 1]):
            ref = torch.from_numpy(base[m].astype(np.float64)) + W @ E[prev]
            np.testing.assert_allclose(got["logits"][m], ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(got["lse"][m], torch.logsumexp(ref, 0).item(),
                                       rtol=0, atol=1e-12)
            prev = int(got["tokens"][m])


def test_dominant_correction_forces_the_chain():
    # W_c = I and e_c(y) = 60 * onehot((y + 7) mod V): the correction of the
    # successor of the previous token dwarfs the base logits (|base| < ~8), so
    # every draw is that successor, the first one the anchor's
    V = 40
    base, q_off, anchor, _, _, req_id = _problem(2, V=V)
    E = np.zeros((V, V), np.float32)
    for y in range(V):
        E[y, (y + 7) % V] = 60.0
    got = omk.markov_sample(base, q_off, anchor, _bf16(np.eye(V)), _bf16(E), req_id, 5)
    for b in range(len(q_off) - 1):
        prev = int(anchor[b])
        for m in range(q_off[b], q_off[b + 1]):
            assert got["tokens"][m] == (prev + 7) % V
            prev = int(got["tokens"][m])


def test_unigram_prior_closed_forms():
    counts = np.array([0, 3, 10, 0, 7, 1000], np.int64)
    lp = omk.unigram_log_prior(counts)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-15
    np.testing.assert_allclose(np.exp(lp), (counts + 1.0) / (counts.sum() + 6.0), rtol=1e-15)
    np.testing.assert_allclose(omk.unigram_log_prior(np.full(9, 5)), np.full(9, -np.log(9.0)), rtol=0,
                               atol=1e-15)
    nz = counts > 0
    np.testing.assert_allclose(np.exp(omk.unigram_log_prior(counts, lam=0.0))[nz],
                               counts[nz] / counts.sum(), rtol=1e-15)


def test_prior_subtraction_flattens_the_prior():
    V = 37
    rng = np.random.default_rng(4)
    counts = rng.integers(0, 50, V)
    b0 = omk.unigram_log_prior(counts).astype(np.float32)
    base, q_off, anchor, w_c, e_c, req_id = _problem(3, V=V)
    base = np.broadcast_to(b0, base.shape).copy()
    got = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 8, alpha=0.0, vocab_bias=-b0)
    np.testing.assert_array_equal(got["logits"], 0.0)
    np.testing.assert_allclose(got["lse"], np.log(V), rtol=0, atol=1e-15)


def test_alpha_scales_the_correction():
    base, q_off, anchor, w_c, e_c, req_id = _problem(5)
    w2 = _bf16(2.0 * bf16_bits_to_f64(w_c))
    a = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 17, alpha=2.0)
    b = omk.markov_sample(base, q_off, anchor, w2, e_c, req_id, 17)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=0, atol=1e-13)


def test_greedy_draws_follow_the_argmax():
    base, q_off, anchor, w_c, e_c, req_id = _problem(6)
    got = omk.markov_sample(base, q_off, anchor, w_c, e_c, req_id, 3, greedy=True)
    W = torch.from_numpy(bf16_bits_to_f64(w_c))
    E = torch.from_numpy(bf16_bits_to_f64(e_c))
    for b in range(len(q_off) - 1):
        prev = int(anchor[b])
        for m in range(q_off[b], q_off[b + 1]):
            row = torch.from_numpy(base[m].astype(np.float64)) + W @ E[prev]
            assert got["tokens"][m] == int(torch.argmax(row))
            prev = int(got["tokens"][m])
