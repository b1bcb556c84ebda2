"""CPU oracle for one block-parallel draft-and-verify step.

TEST INFRASTRUCTURE.  This package is a plain, slow, float64 NumPy statement
of what the step computes, written from the pages' definitions; it exists to
check the HIP library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP path (``block_drafting_sd_amd``) and imports nothing from it; both read
their inputs from the seeded generators in ``synth``.

Modules:
  philox     -- Philox-4x32-10 and the step's uniform draws
  attention  -- draft-block attention over the paged target KV cache (whole
                prefix, or recent window + context summary; causal block)
  summary    -- the fixed-cost drafter's global context summary and its fold
  lm_head    -- LM-head logits, softmax statistics, Gumbel-max draft sampling
  markov     -- the sequential (Markov) correction of the draft distributions
  verify     -- speculative-sampling verification (and its temperature-0 and
                pruned-vocabulary variants)
  schedule   -- ForeSpark's pre-draft estimation, joint draft / verification
                schedule and post-draft budget distribution
  step       -- the three parts run end to end with their near-tie audit

Every function is pinned by ``tests/test_oracle_*.py`` against facts the
pages and the mathematics fix (the lossless theorem by exact enumeration,
closed-form acceptance rates, decode-attention and SDPA special cases,
bit-exact agreement of Philox with rocRAND's implementation, chi-square tests of the samplers).
"""
from . import attention, lm_head, markov, philox, schedule, step, summary, verify  # noqa: F401
