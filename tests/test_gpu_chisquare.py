"""Distribution of the implemented GPU samplers at vocabulary 8 (chi-square).

Speculative sampling is lossless ("LongSpark", sec. 2.1, eqs. (1)-(2) and the
text after eq. (2)): whatever the draft distributions q_j, the tokens a round
emits follow the target's autoregressive law.  Here 10^6 independent rounds
(one request each, own req_id) run through the library: sd_lm_head_probs draws
the K = 2 drafts of every request from fixed proposals q_1, q_2 (Gumbel-max
on Philox stream 0), the target rows of each request are taken from a toy
table p(. | prefix) at the request's own drafted prefix (as a target model
would score the drafted sequence), and sd_verify accepts, corrects or adds
the bonus token.  Counted per (position j, emitted prefix) cell:

* j = 1: every round's first emitted token ~ p(. | empty);
* j = 2: given the first draft u was accepted, the second emitted token
  ~ p(. | u)  (8 cells);
* j = 3: given both drafts (u, w) were accepted, the bonus token
  ~ p(. | u, w)  (64 cells);
* and the drafts themselves: y_j ~ q_j.

Each cell with at least 500 rounds is tested with Pearson's chi-square (7
degrees of freedom) against the exact conditional law; every p-value must
exceed 1e-4 (about 75 cells, so a correct sampler fails with probability
below 1%; the seeds are fixed, so the test is deterministic).
"""
import numpy as np
import pytest
import torch
from scipy import stats

import block_drafting_sd_amd as sd

from gpu_common import DEV, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

V, K, H = 8, 2, 64
ROUNDS = 1_000_000
MIN_CELL = 500
P_MIN = 1e-4


def _softmax(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def _chi2_p(counts, probs):
    n = counts.sum()
    return stats.chisquare(counts, n * probs).pvalue


def test_verify_emits_the_target_law_v8():
    rng = np.random.default_rng(2024)
    # drafter: two distinct hidden rows (positions 1 and 2) shared by every
    # request, a [V, H] head; logits std ~1.5
    w = (rng.standard_normal((V, H)) * (1.5 / np.sqrt(H))).astype(np.float32)
    h2 = rng.standard_normal((K, H)).astype(np.float32)
    hid = torch.from_numpy(np.tile(h2, (ROUNDS, 1))).to(torch.bfloat16).to(DEV)
    wv = torch.from_numpy(w).to(torch.bfloat16).to(DEV)
    q_off = torch.arange(0, K * ROUNDS + 1, K, dtype=torch.int32, device=DEV)
    req_id = torch.arange(ROUNDS, dtype=torch.int32, device=DEV)
    seed = 0x5EED_C0DE_1234
    log("chi-square: drafting 10^6 rounds")
    z, lse, y = sd.sd_lm_head_probs(hid, wv, q_off, req_id, seed)
    torch.cuda.synchronize()
    zr = z[:K].double().cpu().numpy()                  # the two proposals
    q = _softmax(zr)
    y = y.cpu().numpy().reshape(ROUNDS, K)
    # target: a toy table of conditional logits, std 1.5
    L0 = rng.standard_normal(V) * 1.5
    L1 = rng.standard_normal((V, V)) * 1.5
    L2 = rng.standard_normal((V, V, V)) * 1.5
    rows = np.stack([np.broadcast_to(L0, (ROUNDS, V)), L1[y[:, 0]], L2[y[:, 0], y[:, 1]]], 1)
    tgt = torch.from_numpy(rows.reshape(ROUNDS * (K + 1), V).astype(np.float32)).to(DEV)
    t_off = torch.arange(0, (K + 1) * ROUNDS + 1, K + 1, dtype=torch.int32, device=DEV)
    log("chi-square: verifying 10^6 rounds")
    acc, nxt, _ = sd.sd_verify(tgt, t_off, z, lse, torch.from_numpy(y.reshape(-1)).to(DEV),
                               q_off, req_id, seed + 1, want_ratio=False)
    torch.cuda.synchronize()
    acc = acc.cpu().numpy()
    nxt = nxt.cpu().numpy()
    # the emitted prefix: accepted drafts then next_token
    first = np.where(acc >= 1, y[:, 0], nxt)
    pvals = {}
    for j in range(K):
        pvals[f"draft y{j + 1} ~ q{j + 1}"] = _chi2_p(np.bincount(y[:, j], minlength=V), q[j])
    pvals["x1 ~ p(.|-)"] = _chi2_p(np.bincount(first, minlength=V), _softmax(L0))
    reached2 = acc >= 1
    second = np.where(acc >= 2, y[:, 1], nxt)
    n_cells = 0
    for u in range(V):
        sel = reached2 & (y[:, 0] == u)
        if sel.sum() >= MIN_CELL:
            pvals[f"x2 | x1={u}"] = _chi2_p(np.bincount(second[sel], minlength=V), _softmax(L1[u]))
            n_cells += 1
    reached3 = acc >= 2
    for u in range(V):
        for w_ in range(V):
            sel = reached3 & (y[:, 0] == u) & (y[:, 1] == w_)
            if sel.sum() >= MIN_CELL:
                pvals[f"x3 | x1={u},x2={w_}"] = _chi2_p(np.bincount(nxt[sel], minlength=V),
                                                       _softmax(L2[u, w_]))
                n_cells += 1
    worst = min(pvals, key=pvals.get)
    log(f"chi-square: {len(pvals)} cells, mean accepted {acc.mean():.3f}, "
        f"smallest p-value {pvals[worst]:.3g} ({worst})")
    assert n_cells >= 30, n_cells      # conditional cells with at least MIN_CELL rounds
    assert min(pvals.values()) > P_MIN, (worst, pvals[worst])


def test_chisquare_catches_a_wrong_law():
    """Power check of the statistic used above (host only, no kernel): a
    target law with one probability moved by 1% is rejected at 10^6 draws."""
    rng = np.random.default_rng(7)
    p = _softmax(rng.standard_normal(V) * 1.5)
    bad = p.copy()
    bad[0] += 0.01
    bad[1] -= 0.01
    draws = rng.choice(V, size=ROUNDS, p=bad)
    assert _chi2_p(np.bincount(draws, minlength=V), p) < P_MIN
