"""Pins for the oracle's LM head, softmax statistics and Gumbel-max sampler."""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

from oracle import lm_head as ol
from oracle import philox
from oracle.attention import bf16_bits_to_f64
from synth import StepInputs
from synth.configs import C0_TINY


def test_logits_match_pure_python_dot():
    inp = StepInputs(C0_TINY)
    z = ol.lm_head_logits(inp.hidden, inp.w_vocab)
    assert z.shape == (16, 1024)
    h = bf16_bits_to_f64(inp.hidden)
    w = bf16_bits_to_f64(inp.w_vocab)
    for r, v in [(0, 0), (3, 517), (15, 1023), (7, 64)]:
        ref = math.fsum(float(h[r, i]) * float(w[v, i]) for i in range(256))
        assert abs(z[r, v] - ref) < 1e-15


def test_logits_chunking_irrelevant():
    inp = StepInputs(C0_TINY)
    a = ol.lm_head_logits(inp.hidden, inp.w_vocab, v_chunk=8192)
    b = ol.lm_head_logits(inp.hidden, inp.w_vocab, v_chunk=100)
    np.testing.assert_allclose(a, b, atol=1e-15)


def test_logsumexp_against_scipy_and_rows_sum_to_one():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((9, 5000)) * 7
    np.testing.assert_allclose(ol.logsumexp_rows(z), special.logsumexp(z, axis=1),
                               rtol=0, atol=1e-12)
    p = ol.softmax_rows(z)
    assert np.max(np.abs(p.sum(1) - 1)) < 1e-12


def test_logsumexp_constant_and_large():
    z = np.full((2, 151936), 3.25)
    np.testing.assert_allclose(ol.logsumexp_rows(z), 3.25 + math.log(151936), atol=1e-12)
    z = np.array([[1000.0, 1000.0, -1e9]])       # no overflow
    assert abs(ol.logsumexp_rows(z)[0] - (1000 + math.log(2))) < 1e-12


def test_gumbel_argmax_tie_rule_and_gap():
    u = np.full(4, 0.5)
    idx, gap = ol.gumbel_argmax(np.array([0.0, 1.0, 1.0, -np.inf]), u)
    assert idx == 1 and gap == 0.0
    idx, gap = ol.gumbel_argmax(np.array([-np.inf, 2.0, -np.inf, -np.inf]), u)
    assert idx == 1 and gap == np.inf


def test_gumbel_key_is_standard_gumbel():
    # -log(-log u) of the Philox uniforms follows the standard Gumbel law
    u = philox.gumbel_uniforms(99, 5, 2, philox.STREAM_DRAFT, 200000)
    g = -np.log(-np.log(u))
    assert stats.kstest(g, "gumbel_r").pvalue > 1e-3


def test_draft_sampler_chi_square_v8():
    # Gumbel-max over Philox uniforms draws softmax(z) exactly: 200k rows
    # with distinct (request, position) counters, one shared logit row.
    z_row = np.array([0.3, -1.2, 2.0, 0.0, -0.5, 1.1, -3.0, 0.7])
    n_req, n_pos = 12500, 16
    q_off = np.arange(n_req + 1) * n_pos
    req, pos = ol.row_owner(q_off)
    req_id = (np.arange(n_req, dtype=np.uint64) * 2654435761 % (2 ** 32)).astype(np.uint32)
    # vectorised over rows: one Philox call per (row, group of 4 entries)
    k0, k1 = philox.split_seed(0xC0FFEE)
    words = philox.philox4x32_10(np.arange(2)[None, :], pos[:, None],
                                 req_id[req][:, None], philox.STREAM_DRAFT, k0, k1)
    x = np.stack(words, -1).reshape(len(req), 8).astype(np.uint64)
    u = ((x >> np.uint64(9)) * 2 + 1) * 2.0 ** -24
    keys = z_row[None, :] - np.log(-np.log(u))
    tok = np.argmax(keys, 1)
    # the same draws through the oracle's own per-row path on a subset
    sub = np.arange(0, len(req), 997)
    t_sub, _ = ol.draft_tokens(np.tile(z_row, (len(sub), 1)), req[sub], pos[sub],
                               req_id, 0xC0FFEE)
    assert np.array_equal(t_sub, tok[sub])
    p = special.softmax(z_row)
    counts = np.bincount(tok, minlength=8)
    assert stats.chisquare(counts, p * len(tok)).pvalue > 1e-3


def test_torch_log_softmax_cross_check():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((4, 3000)) * 3
    ref = torch.log_softmax(torch.from_numpy(z), dim=1).numpy()
    np.testing.assert_allclose(z - ol.logsumexp_rows(z)[:, None], ref, atol=1e-12)
