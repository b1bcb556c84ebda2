"""The five synthetic workloads of the block-parallel draft-and-verify step.

Each workload fixes shapes and value distributions only; no arithmetic of the
method lives here.  Shapes follow the pages' serving setups:

* Qwen3-8B attention shapes (32 query heads, 8 KV heads, head dim 128) and
  concurrency 16 at 32K / 128K context: "LongSpark: Efficient speculative
  decoding with a fixed-cost parallel drafter", Fig. 1 and Table 2.
* A block of 16 drafts: "DeLS-Spec: Decoupled long-short contexts for parallel
  speculative drafting" (local head trained with block size 16), and
  "ForeSpark" (K = 15 drafts plus the anchor).
* Ragged per-request draft budgets d_i and verify budgets b_i <= d_i:
  "ForeSpark: Joint draft and verification budget scheduling", sec. 4.3-4.4.

The pages' datasets (LongSpec, CodeSpan, LongSWE-Bench, ShareGPT, SPEED-Bench)
are stood in for by Gaussian tensors of these shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

PAGE_SIZE = 16
QWEN3_VOCAB = 151936


@dataclass(frozen=True)
class StepConfig:
    name: str
    index: int
    batch: int
    # prefix lengths: a fixed length, ("loguniform", lo, hi) or
    # ("list", lengths)
    ctx: object
    # draft budget K_b: a fixed int, a tuple of choices or ("list", budgets)
    draft_k: object
    # verify budget b_b: "full" (b_b = K_b), "uniform" (b_b ~ U{1..K_b}),
    # "zero" or ("list", budgets)
    verify: object
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    hidden: int
    vocab: int
    qkv_std: float = 1.0
    hidden_std: float = 0.02
    w_std: float = 0.02
    # target logits: ("normal", sigma) or ("drafter_plus_noise", lo, hi) with
    # per-request sigma log-spaced in [lo, hi], or ("drafter_plus_noise", s, s)
    target: Tuple = ("normal", 3.0)
    page_size: int = PAGE_SIZE
    q_scale: float = 1.0           # multiplies Q (peaked-softmax variants)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_heads_q // self.num_heads_kv

    def with_(self, **kw) -> "StepConfig":
        return replace(self, **kw)


def _cfg(index, **kw):
    kw.setdefault("seed", 0x5D00 + index)
    return StepConfig(index=index, **kw)


# c0: one request, CPU-checkable in well under a second.
C0_TINY = _cfg(0, name="c0_tiny_n512_k16", batch=1, ctx=512, draft_k=16,
               verify="full", num_heads_q=4, num_heads_kv=1, head_dim=64,
               hidden=256, vocab=1024, target=("normal", 2.0))

# c1: Qwen3-8B-shaped drafting at 32K context, concurrency 16.
C1_32K = _cfg(1, name="c1_qwen3_8b_n32k_b16_k16", batch=16, ctx=32768,
              draft_k=16, verify="full", num_heads_q=32, num_heads_kv=8,
              head_dim=128, hidden=4096, vocab=QWEN3_VOCAB,
              target=("normal", 3.0))

# c2: the same shapes at 128K context (8 GiB of bf16 KV per layer).
C2_128K = C1_32K.with_(index=2, name="c2_qwen3_8b_n128k_b16_k16",
                       ctx=131072, seed=0x5D02)

# c3: verification-heavy large batch; target = drafter logits + noise.
C3_VERIFY = _cfg(3, name="c3_verify_heavy_b64_n4k_k16", batch=64, ctx=4096,
                 draft_k=16, verify="full", num_heads_q=32, num_heads_kv=8,
                 head_dim=128, hidden=4096, vocab=QWEN3_VOCAB,
                 target=("drafter_plus_noise", 0.25, 2.07))

# c4: ragged serving mix with joint draft / verify budgets.
C4_RAGGED = _cfg(4, name="c4_ragged_b128_n1k_128k", batch=128,
                 ctx=("loguniform", 1024, 131072), draft_k=(4, 8, 16),
                 verify="uniform", num_heads_q=32, num_heads_kv=8,
                 head_dim=128, hidden=4096, vocab=QWEN3_VOCAB,
                 target=("normal", 3.0))

CONFIGS = (C0_TINY, C1_32K, C2_128K, C3_VERIFY, C4_RAGGED)


def by_index(i: int) -> StepConfig:
    return CONFIGS[i]


def small(cfg: StepConfig, batch: Optional[int] = None, ctx=None,
          vocab: Optional[int] = None, hidden: Optional[int] = None,
          **kw) -> StepConfig:
    """A shrunken copy of a workload with the same head shapes (for tests)."""
    upd = dict(kw)
    if batch is not None:
        upd["batch"] = batch
    if ctx is not None:
        upd["ctx"] = ctx
    if vocab is not None:
        upd["vocab"] = vocab
    if hidden is not None:
        upd["hidden"] = hidden
    upd.setdefault("name", cfg.name + "_small")
    return cfg.with_(**upd)
