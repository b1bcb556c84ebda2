"""Pins for the oracle's variants: attention (causal block, window, summary
rows), the context summary, temperature-0 verification and the pruned
drafter vocabulary.

Attention variants are checked against PyTorch's scaled_dot_product_attention
in float64 on the *logical* keys and values (regenerated from their seeds,
not read from the paged caches) with an explicit boolean mask, or with
``is_causal``; the summary against the same routine (its definition,
"LongSpark" sec. 2.2 eq. (5)), against torch.logsumexp, against the union of
two folded parts (App. A.2 eq. (11) must reproduce eq. (10) over the union)
and against a closed form.  Temperature-0 verification is checked against the
general rules applied to one-hot distributions, greedy drafting against
torch.argmax, and the pruned vocabulary against the full-vocabulary path with
-inf logits outside the subset and against columns of the full head.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import lm_head as olm
from oracle import summary as osum
from oracle import verify as ov
from synth import StepInputs
from synth.configs import C1_32K

F = torch.nn.functional


def _cfg(**kw):
    base = dict(name="variant_pin", batch=4, ctx=("list", (0, 37, 160, 300)),
                draft_k=("list", (3, 16, 5, 8)), verify="full",
                num_heads_q=8, num_heads_kv=2, head_dim=64, hidden=64,
                vocab=64, seed=4242)
    base.update(kw)
    return C1_32K.with_(**base)


def _t(bits):
    return torch.from_numpy(oa.bf16_bits_to_f64(bits))


def _sdpa_ref(inp, window=0, causal=False, u=None, z=None, is_causal_when_empty=False):
    """SDPA (float64) over concat(logical prefix window, block[, U]) with an
    explicit mask."""
    c, bud = inp.cfg, inp.budgets
    out = np.zeros((inp.total_q, c.num_heads_q, c.head_dim))
    for b in range(c.batch):
        r0, r1 = int(bud.q_off[b]), int(bud.q_off[b + 1])
        kb = r1 - r0
        kl, vl = inp.logical_kv(b)
        n = kl.shape[0]
        n0 = max(0, n - window) if window else 0
        for h in range(c.num_heads_q):
            g = h // c.group
            ks = [_t(kl[n0:, g]), _t(inp.k_blk[r0:r1, g])]
            vs = [_t(vl[n0:, g]), _t(inp.v_blk[r0:r1, g])]
            if u is not None:
                ks.append(_t(u[g]))
                # bf16 rounding of the fp32 summary values, by torch
                vs.append(torch.from_numpy(z[b, g]).to(torch.bfloat16).to(torch.float64))
            k = torch.cat(ks)[None, None]
            v = torch.cat(vs)[None, None]
            q = _t(inp.q[r0:r1, h])[None, None]
            if is_causal_when_empty and n == 0 and u is None:
                o = F.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                   scale=inp.softmax_scale)
            else:
                mask = torch.ones(kb, k.shape[2], dtype=torch.bool)
                if causal:
                    mask[:, n - n0:n - n0 + kb] = torch.ones(kb, kb, dtype=torch.bool).tril()
                o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                   scale=inp.softmax_scale)
            out[r0:r1, h] = o[0, 0].numpy()
    return out


def _oracle(inp, **kw):
    b = inp.budgets
    return oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache,
                         inp.page_table, b.ctx_len, b.q_off, inp.cfg.num_heads_kv,
                         inp.softmax_scale, **kw)


def test_causal_block_matches_masked_sdpa():
    inp = StepInputs(_cfg())
    np.testing.assert_allclose(_oracle(inp, block_mask="causal"),
                               _sdpa_ref(inp, causal=True), rtol=0, atol=1e-12)


def test_causal_empty_prefix_is_textbook_causal_attention():
    inp = StepInputs(_cfg(batch=2, ctx=("list", (0, 0)), draft_k=("list", (7, 16))))
    np.testing.assert_allclose(_oracle(inp, block_mask="causal"),
                               _sdpa_ref(inp, causal=True, is_causal_when_empty=True),
                               rtol=0, atol=1e-12)


def test_causal_differs_from_bidirectional():
    inp = StepInputs(_cfg())
    a = _oracle(inp, block_mask="causal")
    b = _oracle(inp)
    # the last row of every request sees the whole block: identical
    last = inp.budgets.q_off[1:] - 1
    np.testing.assert_allclose(a[last], b[last], rtol=0, atol=1e-12)
    assert np.abs(a - b).max() > 1e-3


@pytest.mark.parametrize("window", [1, 16, 50, 256])
def test_window_matches_sdpa_over_last_rows(window):
    inp = StepInputs(_cfg())
    np.testing.assert_allclose(_oracle(inp, window=window), _sdpa_ref(inp, window=window),
                               rtol=0, atol=1e-12)


def test_window_at_least_prefix_is_whole_prefix():
    inp = StepInputs(_cfg())
    np.testing.assert_allclose(_oracle(inp, window=300), _oracle(inp), rtol=0, atol=0)


def test_window_summary_causal_together():
    inp = StepInputs(_cfg())
    u, z = inp.summary_queries(16), inp.summary_values(16)
    got = _oracle(inp, window=50, block_mask="causal", summary_keys=u, summary_values=z)
    ref = _sdpa_ref(inp, window=50, causal=True, u=u, z=z)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ summary

def test_summary_of_rows_is_attention_of_queries():
    inp = StepInputs(_cfg())
    u = inp.summary_queries(16)
    kl, vl = inp.logical_kv(3)
    for g in range(2):
        z, c = osum.summary_of_rows(u[g], kl[:, g], vl[:, g], inp.softmax_scale)
        q, k, v = _t(u[g]), _t(kl[:, g]), _t(vl[:, g])
        ref = F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                             scale=inp.softmax_scale)[0, 0].numpy()
        np.testing.assert_allclose(z, ref, rtol=0, atol=1e-12)
        lse = torch.logsumexp(q @ k.T * inp.softmax_scale, dim=1).numpy()
        np.testing.assert_allclose(c, lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("split", [1, 17, 150, 299])
def test_fold_of_two_parts_equals_summary_of_union(split):
    inp = StepInputs(_cfg())
    u = inp.summary_queries(8)
    kl, vl = inp.logical_kv(3)        # 300 rows
    g = 1
    za, ca = osum.summary_of_rows(u[g], kl[:split, g], vl[:split, g], inp.softmax_scale)
    zb, cb = osum.summary_of_rows(u[g], kl[split:, g], vl[split:, g], inp.softmax_scale)
    z, c = osum.fold(za, ca, zb, cb)
    zr, cr = osum.summary_of_rows(u[g], kl[:, g], vl[:, g], inp.softmax_scale)
    np.testing.assert_allclose(z, zr, rtol=0, atol=1e-12)
    np.testing.assert_allclose(c, cr, rtol=0, atol=1e-12)


def test_fold_empty_sets():
    inp = StepInputs(_cfg())
    u = inp.summary_queries(4)
    kl, vl = inp.logical_kv(2)
    z, c = osum.summary_of_rows(u[0], kl[:, 0], vl[:, 0], inp.softmax_scale)
    ze, ce = osum.summary_of_rows(u[0], kl[:0, 0], vl[:0, 0], inp.softmax_scale)
    assert np.all(ce == -np.inf) and np.all(ze == 0)
    z1, c1 = osum.fold(z, c, ze, ce)          # nothing new: unchanged
    np.testing.assert_array_equal(z1, z)
    np.testing.assert_array_equal(c1, c)
    z2, c2 = osum.fold(ze, ce, z, c)          # empty state takes the new rows
    np.testing.assert_array_equal(z2, z)
    np.testing.assert_array_equal(c2, c)


def test_equal_keys_give_mean_value():
    # all scores equal: Z is the mean of the values, c = s + log n (closed form)
    rng = np.random.default_rng(5)
    D, n = 64, 37
    k = np.tile(rng.integers(0x3C00, 0x3F00, D, dtype=np.uint16), (n, 1))
    v = rng.integers(0x3C00, 0x4000, (n, D), dtype=np.uint16)
    u = rng.integers(0x3C00, 0x3E00, (3, D), dtype=np.uint16)
    z, c = osum.summary_of_rows(u, k, v, 0.125)
    vf, kf, uf = oa.bf16_bits_to_f64(v), oa.bf16_bits_to_f64(k), oa.bf16_bits_to_f64(u)
    np.testing.assert_allclose(z, np.tile(vf.mean(0), (3, 1)), rtol=1e-13, atol=0)
    np.testing.assert_allclose(c, uf @ kf[0] * 0.125 + np.log(n), rtol=1e-13, atol=0)


def test_update_equals_summary_of_all_rows():
    inp = StepInputs(_cfg(batch=3, ctx=("list", (17, 160, 300)), draft_k=("list", (16, 16, 16))))
    b = inp.budgets
    u = inp.summary_queries(16)
    acc = np.array([0, 5, 16], np.int32)
    old = (b.ctx_len - acc - 1).astype(np.int32)
    Z0, C0 = osum.summary_init(u, inp.k_cache, inp.v_cache, inp.page_table, old, 2,
                               inp.softmax_scale)
    Z1, C1 = osum.summary_update(u, inp.k_cache, inp.v_cache, inp.page_table, old, acc,
                                 Z0, C0, 2, inp.softmax_scale)
    for r in range(3):
        kl, vl = inp.logical_kv(r)
        for g in range(2):
            z, c = osum.summary_of_rows(u[g], kl[:, g], vl[:, g], inp.softmax_scale)
            np.testing.assert_allclose(Z1[r, g], z, rtol=0, atol=1e-12)
            np.testing.assert_allclose(C1[r, g], c, rtol=0, atol=1e-12)


# ------------------------------------------------- temperature 0, pruned vocab


def _one_hot(i, V):
    e = np.zeros(V)
    e[i] = 1.0
    return e


@pytest.mark.parametrize("seed", range(6))
def test_greedy_verify_is_the_rules_on_one_hot_distributions(seed):
    rng = np.random.default_rng(seed)
    V, K = 7, 5
    for _ in range(40):
        nv = int(rng.integers(0, K + 1))
        x = rng.integers(-3, 4, (nv + 1, V)).astype(np.float64)   # ties happen
        amax = [int(np.flatnonzero(r == r.max())[0]) for r in x]
        y = [amax[j] if rng.random() < 0.6 else int(rng.integers(0, V)) for j in range(nv)]
        a, c, _ = ov.greedy_request(x, y, nv)
        # the general algorithm with p_j, q_j one-hot at their argmax
        p_rows = [_one_hot(m, V) for m in amax]
        q_rows = [_one_hot(t, V) for t in y]
        a2, c2, _ = ov.verify_request(p_rows, q_rows, y, nv, lambda j: 0.5,
                                      lambda w, j: int(np.flatnonzero(np.asarray(w) > 0)[0]))
        assert (a, c) == (a2, c2)


def test_greedy_draft_tokens_are_torch_argmax():
    rng = np.random.default_rng(1)
    z = rng.integers(-5, 6, (50, 33)).astype(np.float64)       # many ties
    req = np.zeros(50, np.int64)
    pos = np.arange(1, 51)
    tok, _ = olm.draft_tokens(z, req, pos, np.array([3], np.uint32), 11, greedy=True)
    np.testing.assert_array_equal(tok, torch.argmax(torch.from_numpy(z), dim=1).numpy())


def test_pruned_draft_rows_embed_the_subset_softmax():
    rng = np.random.default_rng(2)
    V, Vd = 40, 9
    vmap = np.sort(rng.choice(V, Vd, replace=False))
    inv = np.full(V, -1)
    inv[vmap] = np.arange(Vd)
    z = rng.standard_normal((4, Vd))
    q = ov.draft_rows_full_vocab(z, inv, V)
    np.testing.assert_allclose(q.sum(1), 1.0, rtol=0, atol=1e-15)
    outside = np.setdiff1d(np.arange(V), vmap)
    assert np.all(q[:, outside] == 0)
    np.testing.assert_allclose(q[:, vmap], torch.softmax(torch.from_numpy(z), 1).numpy(),
                               rtol=0, atol=1e-15)


def test_pruned_verify_equals_full_vocab_with_minus_inf_logits():
    inp = StepInputs(_cfg(vocab=96, draft_k=("list", (3, 16, 5, 8))))
    b = inp.budgets
    vmap = inp.pruned_vocab(40)
    inv = np.full(96, -1, np.int32)
    inv[vmap] = np.arange(40)
    rng = np.random.default_rng(3)
    z = rng.standard_normal((inp.total_q, 40)) * 2
    y = vmap[rng.integers(0, 40, inp.total_q)]
    x = inp.target_logits
    got = ov.verify(x, b.t_off, z, y, b.q_off, inp.req_id, inp.philox_seed, draft_vocab_inv=inv)
    z_full = np.full((inp.total_q, 96), -np.inf)
    z_full[:, vmap] = z
    ref = ov.verify(x, b.t_off, z_full, y, b.q_off, inp.req_id, inp.philox_seed)
    np.testing.assert_array_equal(got["accepted"], ref["accepted"])
    np.testing.assert_array_equal(got["next_token"], ref["next_token"])


def test_pruned_lm_head_logits_are_columns_of_the_full_head():
    inp = StepInputs(_cfg(vocab=96))
    vmap = inp.pruned_vocab(40)
    z = olm.lm_head_logits(inp.hidden, inp.w_vocab, vocab_map=vmap)
    h = torch.from_numpy(oa.bf16_bits_to_f64(inp.hidden))
    w = torch.from_numpy(oa.bf16_bits_to_f64(inp.w_vocab))
    np.testing.assert_allclose(z, (h @ w.T).numpy()[:, vmap], rtol=0, atol=1e-12)
