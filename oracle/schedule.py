"""Work-conserving draft / verification budget scheduling (fp64).

Test infrastructure (see ``oracle/__init__``): never imported by the product.

"ForeSpark", sec. 4.2-4.4:

* Pre-draft estimator, eq. (2): ``u_i = SiLU(W_c c_i + W_e e_i)`` (r dims),
  ``z_i = W_o u_i`` -- K(K+1)/2 conditional-acceptance logits, one row
  ``z_i^(d)`` of d entries per candidate draft length d (the triangle of
  Fig. 5).  Entry (d, t) is stored at index d(d-1)/2 + t - 1.  Optional
  biases, and the per-entry scale and bias of the calibration (sec. 4.5),
  enter as ``z = scale * (W_o u + b_o) + bias``.
* Survival benefits, eq. (3): ``S_{i,d,j} = prod_{t<=j} sigmoid(z_{i,t}^(d))``;
  verifying the first b tokens of a length-d draft yields
  ``Reward_i(d, b) = sum_{j<=b} S_{i,d,j}`` accepted tokens (Fig. 5:
  benefits 0.9, 0.7, 0.3 give Reward_i(3, 3) = 1.9).
* Per-request reward curve ``R_i(d) = Reward_i(d, d)``, ``R_i(0) = 0``; its
  upper concave envelope ``F_i`` on {0..K} (the smallest concave function
  above it); survival scores ``g_{i,d} = F_i(d) - F_i(d-1)``, non-increasing
  in d (sec. 4.3).
* Global gather: all scores sorted, ``g_(1) >= g_(2) >= ...``; the top k
  entries form a prefix of every request, i.e. a draft schedule D with
  sum_i d_i = k.
* Joint schedule, eq. (4): ``(D, B) = argmax (n + sum_{r<=B} g_(r)) /
  (T_draft(D) + T_verify(N + B))`` over B <= sum_i d_i, with latencies from
  profiled tables that are constant within token-count buckets.  Within a
  pair of buckets the largest feasible schedule is best, so the search checks
  one candidate per pair (sec. 4.3).
* Post-draft estimator, eq. (5): ``p_{i,j} = sigmoid(w . [h_{i,j}; s_{i,j}])``
  with ``s_{i,j} = (W_s h_{i,j}) * E_pred(x_{i,j-1})`` (x_{i,0} the anchor),
  ``S^_{i,j} = prod_{t<=j} p_{i,t}``; a per-position temperature (sec. 4.5)
  divides the logit.  Budget distribution (sec. 4.4): the B positions with
  the highest ``S^`` across the batch are verified -- a prefix of every draft.

Readings where the pages are silent (all in the design notes):
* the drafter's token count is ``n + sum_i d_i`` (each request's anchor plus
  its masks, Fig. 7) and the verifier's ``N + B``; a latency table is a list
  of (token capacity, latency) buckets, a count uses the smallest bucket that
  holds it, and counts above the last bucket are infeasible;
* within a pair of buckets B is the largest feasible count of positive
  scores (a non-positive score cannot raise the numerator);
* order of equal scores: smaller request index first, then smaller d (keeps
  the prefix property); ties of eq. (4) between bucket pairs go to the first
  pair in (draft bucket, verify bucket) order.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64


def tri_index(d: int, t: int) -> int:
    """Index of entry (d, t), 1 <= t <= d <= K, in a triangle row-vector."""
    return d * (d - 1) // 2 + t - 1


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def predraft_logits(c, e, w_c, w_e, w_o, b_u=None, b_o=None, cal_scale=None, cal_bias=None):
    """Eq. (2) (with the optional biases and calibration): ``z [n, T]``."""
    C, E = bf16_bits_to_f64(c), bf16_bits_to_f64(e)
    pre = C @ bf16_bits_to_f64(w_c).T + E @ bf16_bits_to_f64(w_e).T
    if b_u is not None:
        pre = pre + np.asarray(b_u, np.float64)
    u = pre * sigmoid(pre)                            # SiLU
    z = u @ bf16_bits_to_f64(w_o).T
    if b_o is not None:
        z = z + np.asarray(b_o, np.float64)
    if cal_scale is not None:
        z = z * np.asarray(cal_scale, np.float64)
    if cal_bias is not None:
        z = z + np.asarray(cal_bias, np.float64)
    return z


def survival_benefits(z_row, K: int):
    """``S[d-1][j-1] = S_{d,j}`` for one request (eq. (3)); NaN above the
    diagonal."""
    S = np.full((K, K), np.nan)
    for d in range(1, K + 1):
        prod = 1.0
        for t in range(1, d + 1):
            prod *= float(sigmoid(z_row[tri_index(d, t)]))
            S[d - 1, t - 1] = prod
    return S


def reward(S, d: int, b: int) -> float:
    """``Reward(d, b) = sum_{j<=b} S_{d,j}`` (b <= d)."""
    return float(sum(S[d - 1, j - 1] for j in range(1, b + 1)))


def reward_curve(S, K: int):
    """``R(0..K)`` with ``R(d) = Reward(d, d)``."""
    return np.array([0.0] + [reward(S, d, d) for d in range(1, K + 1)])


def concave_envelope(R):
    """Smallest concave function on {0..K} that is >= R: at every d, the best
    value a chord between two points of the curve around d reaches."""
    K = len(R) - 1
    F = np.array(R, np.float64)
    for d in range(K + 1):
        for a in range(0, d + 1):
            for b in range(d, K + 1):
                if a == b:
                    continue
                F[d] = max(F[d], R[a] + (R[b] - R[a]) * (d - a) / (b - a))
    return F


def survival_scores(R):
    """``g_d = F(d) - F(d-1)``.  Concavity makes them non-increasing; a
    running minimum removes rounding noise (~1e-16) that could break that
    order and with it the prefix property of the selection."""
    F = concave_envelope(R)
    return np.minimum.accumulate(F[1:] - F[:-1])


def bucket_latency(tokens: int, caps, lat):
    """Latency of the smallest bucket that holds ``tokens`` (inf if none)."""
    for c, l in zip(caps, lat):
        if tokens <= c:
            return float(l)
    return np.inf


def sorted_scores(g):
    """All scores ``g [n, K]`` sorted descending with the order of equal
    scores fixed (request, then d); returns (values, request of each)."""
    n, K = g.shape
    keys = [(-g[i, d], i, d) for i in range(n) for d in range(K)]
    keys.sort()
    return np.array([-k[0] for k in keys]), np.array([k[1] for k in keys], np.int64)


def pair_candidates(g, n_nonspec: int, d_caps, d_lat, v_caps, v_lat):
    """The candidate of every (draft bucket, verify bucket) pair, in that
    order: a list of (objective, k, B), objective -inf if infeasible."""
    n, K = g.shape
    vals, _ = sorted_scores(g)
    prefix = np.concatenate([[0.0], np.cumsum(vals)])
    n_pos = int((vals > 0).sum())
    out = []
    for dc, dl in zip(d_caps, d_lat):
        k = min(int(dc) - n, n * K)
        for vc, vl in zip(v_caps, v_lat):
            B = min(int(vc) - n_nonspec, k, n_pos)
            if k < 0 or B < 0:
                out.append((-np.inf, 0, 0))
            else:
                out.append(((n + prefix[B]) / (float(dl) + float(vl)), k, B))
    return out


def joint_schedule(g, n_nonspec: int, d_caps, d_lat, v_caps, v_lat):
    """Eq. (4) by the bucket-pair search.  Returns dict(draft_len [n],
    budget B, objective, k = sum d_i)."""
    n, K = g.shape
    vals, owner = sorted_scores(g)
    best = (-np.inf, 0, 0)
    for cand in pair_candidates(g, n_nonspec, d_caps, d_lat, v_caps, v_lat):
        if cand[0] > best[0]:
            best = cand
    obj, k, B = best
    d = np.zeros(n, np.int32)
    for r in range(k):
        d[owner[r]] += 1
    return dict(draft_len=d, budget=B, objective=obj, k=k)


def joint_schedule_exhaustive(g, n_nonspec: int, d_caps, d_lat, v_caps, v_lat):
    """Eq. (4) by trying every total draft count k and budget B <= k."""
    n, K = g.shape
    vals, _ = sorted_scores(g)
    prefix = np.concatenate([[0.0], np.cumsum(vals)])
    best = -np.inf
    for k in range(0, n * K + 1):
        td = bucket_latency(n + k, d_caps, d_lat)
        for B in range(0, k + 1):
            tv = bucket_latency(n_nonspec + B, v_caps, v_lat)
            if np.isfinite(td + tv):
                best = max(best, (n + prefix[B]) / (td + tv))
    return best


def postdraft_probs(hidden, w_s, e_pred, w, prev_tokens, positions, bias=0.0, temperature=None):
    """Eq. (5): ``p [M]`` for packed draft rows; ``prev_tokens[m]`` is the
    token before row m's (the anchor for position 1), ``positions[m]`` its
    1-based position."""
    h = bf16_bits_to_f64(hidden)
    s = (h @ bf16_bits_to_f64(w_s).T) * bf16_bits_to_f64(e_pred[np.asarray(prev_tokens)])
    logit = np.concatenate([h, s], axis=1) @ np.asarray(w, np.float64) + bias
    if temperature is not None:
        logit = logit / np.asarray(temperature, np.float64)[np.asarray(positions) - 1]
    return sigmoid(logit)


def distribute_budget(p, q_off, B: int):
    """``S^`` per row and the verified prefix length b_i of every request: the
    B rows with the highest ``S^`` (equal values: smaller request, then
    smaller position first)."""
    q_off = np.asarray(q_off, np.int64)
    n = len(q_off) - 1
    S = np.empty(len(p))
    keys = []
    for i in range(n):
        prod = 1.0
        for m in range(q_off[i], q_off[i + 1]):
            prod *= float(p[m])
            S[m] = prod
            keys.append((-prod, i, m - q_off[i]))
    keys.sort()
    b = np.zeros(n, np.int32)
    for key in keys[:max(0, B)]:
        b[key[1]] += 1
    return S, b
