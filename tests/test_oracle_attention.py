"""Pins for the oracle's draft-block attention.

Each check compares the oracle against something it does not share code
with: PyTorch's scaled_dot_product_attention in float64 on the *logical*
keys and values (regenerated from their seeds, not read from the paged
caches), a pure-Python loop, the merge identity of "LongSpark" App. A.2
eq. (11), a planted needle written straight into the documented page layout,
and invariance under a re-permutation of the physical pages.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from synth import StepInputs
from synth.configs import C0_TINY, C1_32K

F = torch.nn.functional


def _cfg(**kw):
    base = dict(name="attn_pin", batch=4, ctx=("list", (0, 1, 37, 160)),
                draft_k=("list", (3, 1, 16, 5)), verify="full",
                num_heads_q=8, num_heads_kv=2, head_dim=64, hidden=64,
                vocab=64, seed=777)
    base.update(kw)
    return C1_32K.with_(**base)


def _oracle_out(inp):
    b = inp.budgets
    return oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, inp.k_cache, inp.v_cache,
                         inp.page_table, b.ctx_len, b.q_off,
                         inp.cfg.num_heads_kv, inp.softmax_scale)


def _sdpa_ref(inp):
    """SDPA (float64, no mask) over concat(logical prefix, block) per head."""
    c = inp.cfg
    bud = inp.budgets
    G = c.group
    out = np.zeros((inp.total_q, c.num_heads_q, c.head_dim))
    for b in range(c.batch):
        r0, r1 = int(bud.q_off[b]), int(bud.q_off[b + 1])
        kl, vl = inp.logical_kv(b)
        for h in range(c.num_heads_q):
            g = h // G
            k = np.concatenate([kl[:, g], inp.k_blk[r0:r1, g]], 0)
            v = np.concatenate([vl[:, g], inp.v_blk[r0:r1, g]], 0)
            qt = torch.from_numpy(oa.bf16_bits_to_f64(inp.q[r0:r1, h]))[None, None]
            kt = torch.from_numpy(oa.bf16_bits_to_f64(k))[None, None]
            vt = torch.from_numpy(oa.bf16_bits_to_f64(v))[None, None]
            o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=None,
                                               scale=inp.softmax_scale)
            out[r0:r1, h] = o[0, 0].numpy()
    return out


def test_matches_sdpa_no_mask_ragged():
    inp = StepInputs(_cfg())
    np.testing.assert_allclose(_oracle_out(inp), _sdpa_ref(inp), rtol=0, atol=1e-12)


def test_k1_is_decode_attention():
    # K = 1: one query row over N prefix keys plus its own key
    inp = StepInputs(_cfg(batch=3, ctx=("list", (1, 16, 333)),
                          draft_k=("list", (1, 1, 1))))
    np.testing.assert_allclose(_oracle_out(inp), _sdpa_ref(inp), rtol=0, atol=1e-12)


def test_mha_group_one():
    inp = StepInputs(_cfg(num_heads_q=2, num_heads_kv=2))
    np.testing.assert_allclose(_oracle_out(inp), _sdpa_ref(inp), rtol=0, atol=1e-12)


def test_empty_prefix_is_block_self_attention():
    inp = StepInputs(_cfg(batch=1, ctx=("list", (0,)), draft_k=("list", (6,))))
    out = _oracle_out(inp)
    c = inp.cfg
    for h in range(c.num_heads_q):
        g = h // c.group
        q = oa.bf16_bits_to_f64(inp.q[:, h])
        k = oa.bf16_bits_to_f64(inp.k_blk[:, g])
        v = oa.bf16_bits_to_f64(inp.v_blk[:, g])
        s = q @ k.T / math.sqrt(c.head_dim)
        w = np.exp(s - s.max(1, keepdims=True))
        np.testing.assert_allclose(out[:, h], (w / w.sum(1, keepdims=True)) @ v,
                                   atol=1e-13)


def test_pure_python_loop_tiny():
    inp = StepInputs(_cfg(batch=1, ctx=("list", (21,)), draft_k=("list", (2,)),
                          num_heads_q=2, num_heads_kv=1, head_dim=16))
    out = _oracle_out(inp)
    kl, vl = inp.logical_kv(0)
    D = 16
    dec = lambda bits: float(oa.bf16_bits_to_f64(np.array([bits]))[0])
    keys = [[dec(kl[t, 0, d]) for d in range(D)] for t in range(21)] + \
           [[dec(inp.k_blk[r, 0, d]) for d in range(D)] for r in range(2)]
    vals = [[dec(vl[t, 0, d]) for d in range(D)] for t in range(21)] + \
           [[dec(inp.v_blk[r, 0, d]) for d in range(D)] for r in range(2)]
    for r in range(2):
        for h in range(2):
            qv = [dec(inp.q[r, h, d]) for d in range(D)]
            sc = [sum(a * b for a, b in zip(qv, k)) / math.sqrt(D) for k in keys]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            ref = [sum(w[i] * vals[i][d] for i in range(len(w))) / tot for d in range(D)]
            np.testing.assert_allclose(out[r, h], ref, atol=1e-14)


def test_lse_merge_equals_union():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((7, 32))
    k = rng.standard_normal((300, 32))
    v = rng.standard_normal((300, 32))
    full, lse_full = oa.attention_lse(q, k, v, 0.3)
    mask = rng.random(300) < 0.37
    za, la = oa.attention_lse(q, k[mask], v[mask], 0.3)
    zb, lb = oa.attention_lse(q, k[~mask], v[~mask], 0.3)
    z, l = oa.lse_merge(za, la, zb, lb)
    np.testing.assert_allclose(z, full, atol=1e-13)
    np.testing.assert_allclose(l, lse_full, atol=1e-12)
    # merging is associative over a three-way split
    parts = np.array_split(rng.permutation(300), 3)
    st = [oa.attention_lse(q, k[p], v[p], 0.3) for p in parts]
    z1, l1 = oa.lse_merge(*oa.lse_merge(*st[0], *st[1]), *st[2])
    np.testing.assert_allclose(z1, full, atol=1e-13)


def test_page_permutation_invariance():
    inp = StepInputs(_cfg())
    base = _oracle_out(inp)
    rng = np.random.default_rng(11)
    pi = rng.permutation(inp.num_pages)
    k2 = np.empty_like(inp.k_cache)
    v2 = np.empty_like(inp.v_cache)
    k2[pi] = inp.k_cache
    v2[pi] = inp.v_cache
    pt2 = pi[inp.page_table].astype(np.int32)
    b = inp.budgets
    out2 = oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, k2, v2, pt2, b.ctx_len,
                         b.q_off, inp.cfg.num_heads_kv, inp.softmax_scale)
    assert np.array_equal(out2, base, equal_nan=True)


def test_planted_needle():
    # A key aligned with one query row, written through the documented layout,
    # dominates that row's softmax: the output is the needle's value row.
    inp = StepInputs(_cfg(batch=2, ctx=("list", (100, 517)),
                          draft_k=("list", (2, 4))))
    c = inp.cfg
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    b, t, g, row, h = 1, 389, 1, 2, 5          # h // G == g
    qrow = oa.bf16_bits_to_f64(inp.q[int(inp.budgets.q_off[b]) + row, h])
    key = qrow * (60.0 / (qrow @ qrow * inp.softmax_scale))
    key_bits = (key.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    val = np.linspace(-1, 1, c.head_dim)
    val_bits = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    page, slot = inp.page_table[b, t // c.page_size], t % c.page_size
    for d in range(c.head_dim):
        kc[page, g, d // 8, slot, d % 8] = key_bits[d]
        vc[page, g, d, slot] = val_bits[d]
    bud = inp.budgets
    out = oa.draft_attn(inp.q, inp.k_blk, inp.v_blk, kc, vc, inp.page_table,
                        bud.ctx_len, bud.q_off, c.num_heads_kv, inp.softmax_scale)
    np.testing.assert_allclose(out[int(bud.q_off[b]) + row, h],
                               oa.bf16_bits_to_f64(val_bits), atol=1e-6)


def test_tiny_workload_shapes():
    inp = StepInputs(C0_TINY)
    out = _oracle_out(inp)
    assert out.shape == (16, 4, 64) and np.isfinite(out).all()
    np.testing.assert_allclose(out, _sdpa_ref(inp), atol=1e-12)
