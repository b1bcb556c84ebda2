"""Seeded synthetic inputs for the draft / verification scheduler.

Only random draws and their layout; none of the method's arithmetic.  The
estimators' weights stand in for trained ones: scales are chosen so the
pre-activations are O(1), and the logits' bias puts the conditional
acceptance probabilities around sigmoid(1) ~ 0.73 -- in the range the pages
report for parallel drafters.  Latency tables stand in for offline profiles:
bucket capacities in powers of two and latencies growing with the bucket.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .inputs import _normal_bf16, _rng

TAG_SCHED = 31


@dataclass
class ScheduleInputs:
    n: int = 192          # requests in the batch
    K: int = 16           # longest draft
    d_h: int = 4096       # target hidden size (context feature, embedding)
    r: int = 256          # estimator rank
    m: int = 256          # selector feature size
    V: int = 151936       # vocabulary
    seed: int = 0x5C4E

    def _g(self, *tags):
        return _rng(self.seed, TAG_SCHED, *tags)

    @property
    def T(self) -> int:
        return self.K * (self.K + 1) // 2

    def predraft(self):
        """Estimator inputs and weights (eq. (2) of the scheduler)."""
        n, d, r, T = self.n, self.d_h, self.r, self.T
        return dict(
            ctx_feat=_normal_bf16(self._g(1), (n, d), 1.0),
            anchor_emb=_normal_bf16(self._g(2), (n, d), 1.0),
            w_c=_normal_bf16(self._g(3), (r, d), 1.0 / np.sqrt(d)),
            w_e=_normal_bf16(self._g(4), (r, d), 1.0 / np.sqrt(d)),
            b_u=(self._g(5).standard_normal(r) * 0.1).astype(np.float32),
            w_o=_normal_bf16(self._g(6), (T, r), 1.0 / np.sqrt(r)),
            b_o=(1.0 + self._g(7).standard_normal(T) * 0.5).astype(np.float32),
            cal_scale=self._g(8).uniform(0.8, 1.25, T).astype(np.float32),
            cal_bias=(self._g(9).standard_normal(T) * 0.1).astype(np.float32))

    def latency_tables(self):
        """(capacities, latencies) for the drafter and the verifier."""
        n, K = self.n, self.K
        top = n * (K + 1)
        caps = [n]
        while caps[-1] < top:
            caps.append(min(top, caps[-1] * 2 if caps[-1] >= 64 else caps[-1] + 64))
        caps = np.array(caps, np.int32)
        jit = self._g(10).uniform(0.95, 1.05, (2, len(caps)))
        d_lat = ((1.0 + 0.002 * caps) * jit[0]).astype(np.float32)
        v_lat = ((6.0 + 0.004 * caps) * jit[1]).astype(np.float32)
        return caps, d_lat, caps.copy(), v_lat

    def postdraft(self, rows: int):
        """Selector weights and ``rows`` packed draft rows (hidden states and
        tokens), plus the anchors."""
        H, m, V, n, K = self.d_h, self.m, self.V, self.n, self.K
        return dict(
            hidden=_normal_bf16(self._g(11), (rows, H), 1.0),
            w_s=_normal_bf16(self._g(12), (m, H), 1.0 / np.sqrt(H)),
            e_pred=_normal_bf16(self._g(13), (V, m), 1.0),
            w=(self._g(14).standard_normal(H + m) / np.sqrt(H + m)).astype(np.float32),
            bias=1.5,
            temperature=self._g(15).uniform(0.8, 1.25, K).astype(np.float32),
            anchor=self._g(16).integers(0, V, n).astype(np.int32),
            tokens=self._g(17).integers(0, V, rows).astype(np.int32))
