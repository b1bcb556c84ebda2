"""Parity rules between the HIP library's outputs and the oracle.

Test infrastructure (see ``oracle/__init__``): never imported by the product.

* attention output: max |gpu - oracle| <= ATTN_TOL (1e-2), relative L2 and
  max error reported;
* probabilities: max |q_gpu - q_oracle| <= PROB_TOL (1e-5), q = exp(z - lse);
* integer decisions (draft tokens, accepted lengths, next tokens) exact,
  except decisions the oracle marks as near-ties: an acceptance test with
  |u - r| < NEAR_TIE or a Gumbel-max draw whose top-2 key gap is < NEAR_TIE.
  A near-tie upstream (a request's draft token) excuses that request's
  verification outcome as well.  Near-ties are counted and reported.
"""
from __future__ import annotations

import numpy as np

from . import attention, lm_head, verify
from .step import NEAR_TIE

ATTN_TOL = 1e-2
PROB_TOL = 1e-5


def bf16_bits_to_f64(x):
    return attention.bf16_bits_to_f64(x)


def attention_report(gpu_out_bits: np.ndarray, ref: np.ndarray, rows=None) -> dict:
    """``gpu_out_bits``: uint16 [total_q, Hq, D]; ``ref``: oracle float64."""
    g = bf16_bits_to_f64(gpu_out_bits)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    mask = np.isfinite(ref)
    err = np.abs(g[mask] - ref[mask])
    denom = np.sqrt(np.sum(ref[mask] ** 2)) or 1.0
    return dict(max_abs=float(err.max()) if err.size else 0.0,
                rel_l2=float(np.sqrt(np.sum((g[mask] - ref[mask]) ** 2)) / denom),
                n=int(mask.sum()), ok=bool(err.size == 0 or err.max() <= ATTN_TOL))


def lm_head_report(gpu_logits, gpu_lse, gpu_tokens, ref: dict) -> dict:
    """``ref`` from ``oracle.step.run_lm_head`` (rows = ref['rows'])."""
    rows = ref["rows"]
    z, lse = ref["logits"], ref["lse"]
    gz = gpu_logits[rows].astype(np.float64)
    gl = gpu_lse[rows].astype(np.float64)
    q_ref = np.exp(z - lse[:, None])
    q_gpu = np.exp(gz - gl[:, None])
    tok = gpu_tokens[rows]
    near = ref["gap"] < NEAR_TIE
    mism = (tok != ref["tokens"]) & ~near
    return dict(logit_max_abs=float(np.abs(gz - z).max()),
                lse_max_abs=float(np.abs(gl - lse).max()),
                prob_max_abs=float(np.abs(q_gpu - q_ref).max()),
                prob_row_sum_err=float(np.abs(q_gpu.sum(1) - 1).max()),
                token_mismatch=int(mism.sum()), token_near_ties=int(near.sum()),
                token_near_tie_mismatch=int(((tok != ref["tokens"]) & near).sum()),
                n_rows=len(rows),
                ok=bool(np.abs(q_gpu - q_ref).max() <= PROB_TOL and mism.sum() == 0))


def verify_report(gpu_acc, gpu_next, ref: dict, requests, excused=None) -> dict:
    """``ref`` from ``oracle.verify.verify``; ``excused`` a boolean array of
    requests whose inputs already hold an upstream near-tie."""
    requests = np.asarray(list(requests))
    near = (ref["accept_margin"][requests] < NEAR_TIE) | (ref["sample_gap"][requests] < NEAR_TIE)
    if excused is not None:
        near |= np.asarray(excused)[requests]
    acc_bad = (gpu_acc[requests] != ref["accepted"][requests]) & ~near
    nxt_bad = (gpu_next[requests] != ref["next_token"][requests]) & ~near
    return dict(n=len(requests), near_ties=int(near.sum()),
                accepted_mismatch=int(acc_bad.sum()), next_mismatch=int(nxt_bad.sum()),
                near_tie_mismatch=int(((gpu_acc[requests] != ref["accepted"][requests]) |
                                       (gpu_next[requests] != ref["next_token"][requests]))[near].sum()),
                mean_accepted=float(np.mean(ref["accepted"][requests])),
                ok=bool(acc_bad.sum() == 0 and nxt_bad.sum() == 0))


def ratio_report(gpu_ratio, ref: dict, q_off, requests) -> dict:
    """Compare min(1, p/q) at every test the oracle made."""
    errs = []
    for b in requests:
        for j, u, r in ref["tests"][b] or []:
            errs.append(abs(float(gpu_ratio[int(q_off[b]) + j - 1]) - float(r)))
    return dict(n=len(errs), max_abs=float(max(errs)) if errs else 0.0)
