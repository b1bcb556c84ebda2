"""Seeded synthetic inputs for one draft-and-verify step.

This module only draws random tensors and lays them out in memory; it holds
none of the method's arithmetic.  Both the HIP path and the CPU oracle consume
exactly what it returns.  bf16 tensors are returned as ``uint16`` bit patterns
(round-to-nearest-even of float32 normal draws), fp32 tensors as ``float32``.

Memory layouts (the formats the C ABI documents):

* ``k_cache``: ``[num_pages, Hkv, D/8, P, 8]`` -- within one (page, kv head)
  the key rows are stored in 16-byte column chunks: chunk ``c`` of token ``t``
  holds dims ``8c .. 8c+7`` at ``((c * P) + t) * 8``.
* ``v_cache``: ``[num_pages, Hkv, D, P]`` -- within one (page, kv head) the
  values are stored dimension-major, 16 tokens contiguous per dimension.
* ``page_table``: ``int32 [B, max_pages]``; logical page ``i`` of request
  ``b`` lives in physical page ``page_table[b, i]``; unused entries are 0.

Content of every logical page is drawn from its own seeded stream, so any
request's logical keys and values can be regenerated without the rest.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from functools import cached_property
from typing import Dict, Optional, Tuple

import numpy as np

from .configs import StepConfig

# stream tags for the per-tensor seed sequences
TAG_CTX, TAG_KB, TAG_VB, TAG_PERM, TAG_K, TAG_V = 1, 2, 3, 4, 5, 6
TAG_Q, TAG_KBLK, TAG_VBLK, TAG_HID, TAG_W, TAG_TGT = 7, 8, 9, 10, 11, 12
TAG_SIGMA, TAG_REQ, TAG_SEED, TAG_NOISE, TAG_TOK = 13, 14, 15, 16, 17
TAG_SUMQ, TAG_SUMV, TAG_VMAP = 18, 19, 20
TAG_MKW, TAG_MKE, TAG_ANCHOR, TAG_COUNTS = 21, 22, 23, 24

PAGES_PER_CHUNK = 256
W_ROWS_PER_CHUNK = 4096
TGT_ROWS_PER_CHUNK = 16


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(w) & 0xFFFFFFFF for w in words])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Budgets:
    ctx_len: np.ndarray      # int32 [B]
    draft_k: np.ndarray      # int32 [B]  K_b
    verify_b: np.ndarray     # int32 [B]  b_b <= K_b
    q_off: np.ndarray        # int32 [B+1]
    t_off: np.ndarray        # int32 [B+1]


class StepInputs:
    """Lazily generated inputs of one step for a workload ``cfg``."""

    def __init__(self, cfg: StepConfig):
        self.cfg = cfg
        self._cache: Dict[str, np.ndarray] = {}

    # ------------------------------------------------------------------ sizes
    @cached_property
    def budgets(self) -> Budgets:
        c = self.cfg
        B = c.batch
        if isinstance(c.ctx, tuple) and c.ctx[0] == "list":
            ctx = np.asarray(c.ctx[1], np.int32)
            assert len(ctx) == B
        elif isinstance(c.ctx, tuple):
            kind, lo, hi = c.ctx
            assert kind == "loguniform"
            u = _rng(c.seed, TAG_CTX).random(B)
            ctx = np.rint(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
            ctx = ctx.astype(np.int32)
        else:
            ctx = np.full(B, int(c.ctx), np.int32)
        if isinstance(c.draft_k, tuple) and c.draft_k[0] == "list":
            kb = np.asarray(c.draft_k[1], np.int32)
            assert len(kb) == B
        elif isinstance(c.draft_k, tuple):
            kb = _rng(c.seed, TAG_KB).choice(np.array(c.draft_k), size=B)
            kb = kb.astype(np.int32)
        else:
            kb = np.full(B, int(c.draft_k), np.int32)
        if c.verify == "full":
            vb = kb.copy()
        elif c.verify == "uniform":
            r = _rng(c.seed, TAG_VB)
            vb = np.array([r.integers(1, k + 1) for k in kb], np.int32)
        elif c.verify == "zero":
            vb = np.zeros(B, np.int32)
        elif isinstance(c.verify, tuple) and c.verify[0] == "list":
            vb = np.asarray(c.verify[1], np.int32)
            assert len(vb) == B and np.all(vb <= kb) and np.all(vb >= 0)
        else:
            raise ValueError(c.verify)
        q_off = np.zeros(B + 1, np.int32)
        q_off[1:] = np.cumsum(kb)
        t_off = np.zeros(B + 1, np.int32)
        t_off[1:] = np.cumsum(vb + 1)
        return Budgets(ctx, kb, vb, q_off, t_off)

    @property
    def total_q(self) -> int:
        return int(self.budgets.q_off[-1])

    @property
    def total_target_rows(self) -> int:
        return int(self.budgets.t_off[-1])

    @cached_property
    def pages_per_req(self) -> np.ndarray:
        P = self.cfg.page_size
        return ((self.budgets.ctx_len.astype(np.int64) + P - 1) // P)

    @property
    def max_pages(self) -> int:
        return max(1, int(self.pages_per_req.max()))

    @property
    def num_pages(self) -> int:
        return max(1, int(self.pages_per_req.sum()))

    @property
    def max_total_ctx(self) -> int:
        return int(self.budgets.ctx_len.astype(np.int64).sum())

    # ------------------------------------------------------------- page table
    @cached_property
    def page_table(self) -> np.ndarray:
        c = self.cfg
        perm = _rng(c.seed, TAG_PERM).permutation(self.num_pages).astype(np.int32)
        pt = np.zeros((c.batch, self.max_pages), np.int32)
        off = 0
        for b, n in enumerate(self.pages_per_req):
            n = int(n)
            pt[b, :n] = perm[off:off + n]
            off += n
        return pt

    # ------------------------------------------------------- logical KV pages
    def _logical_chunk(self, tag: int, b: int, chunk: int) -> np.ndarray:
        """bf16 bits [n, P, Hkv, D] for logical pages of one chunk."""
        c = self.cfg
        n_pages = int(self.pages_per_req[b])
        first = chunk * PAGES_PER_CHUNK
        n = min(PAGES_PER_CHUNK, n_pages - first)
        rng = _rng(c.seed, tag, b, chunk)
        return _normal_bf16(rng, (n, c.page_size, c.num_heads_kv, c.head_dim),
                            c.qkv_std)

    def logical_kv(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """Request ``b``'s prefix keys and values, ``[N_b, Hkv, D]`` bf16 bits,
        regenerated from their seeds (independent of the physical caches)."""
        c = self.cfg
        N = int(self.budgets.ctx_len[b])
        n_chunks = (int(self.pages_per_req[b]) + PAGES_PER_CHUNK - 1) // PAGES_PER_CHUNK
        out = []
        for tag in (TAG_K, TAG_V):
            parts = [self._logical_chunk(tag, b, ch) for ch in range(n_chunks)]
            if parts:
                x = np.concatenate(parts, 0).reshape(-1, c.num_heads_kv, c.head_dim)
            else:
                x = np.zeros((0, c.num_heads_kv, c.head_dim), np.uint16)
            out.append(np.ascontiguousarray(x[:N]))
        return out[0], out[1]

    def _build_caches(self) -> None:
        c = self.cfg
        P, Hkv, D = c.page_size, c.num_heads_kv, c.head_dim
        kc = np.zeros((self.num_pages, Hkv, D // 8, P, 8), np.uint16)
        vc = np.zeros((self.num_pages, Hkv, D, P), np.uint16)
        pt = self.page_table
        tasks = []
        for b in range(c.batch):
            n_pages = int(self.pages_per_req[b])
            for ch in range((n_pages + PAGES_PER_CHUNK - 1) // PAGES_PER_CHUNK):
                tasks.append((b, ch))

        def work(t):
            b, ch = t
            first = ch * PAGES_PER_CHUNK
            k = self._logical_chunk(TAG_K, b, ch)          # [n, P, Hkv, D]
            v = self._logical_chunk(TAG_V, b, ch)
            n = k.shape[0]
            phys = pt[b, first:first + n]
            kc[phys] = k.reshape(n, P, Hkv, D // 8, 8).transpose(0, 2, 3, 1, 4)
            vc[phys] = v.transpose(0, 2, 3, 1)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, tasks))
        self._cache["k_cache"] = kc
        self._cache["v_cache"] = vc

    @property
    def k_cache(self) -> np.ndarray:
        if "k_cache" not in self._cache:
            self._build_caches()
        return self._cache["k_cache"]

    @property
    def v_cache(self) -> np.ndarray:
        if "v_cache" not in self._cache:
            self._build_caches()
        return self._cache["v_cache"]

    # ---------------------------------------------------------- block tensors
    @cached_property
    def q(self) -> np.ndarray:
        c = self.cfg
        x = _rng(c.seed, TAG_Q).standard_normal(
            (self.total_q, c.num_heads_q, c.head_dim), dtype=np.float32)
        x *= np.float32(c.qkv_std * c.q_scale)
        return f32_to_bf16_bits(x)

    @cached_property
    def k_blk(self) -> np.ndarray:
        c = self.cfg
        return _normal_bf16(_rng(c.seed, TAG_KBLK),
                            (self.total_q, c.num_heads_kv, c.head_dim), c.qkv_std)

    @cached_property
    def v_blk(self) -> np.ndarray:
        c = self.cfg
        return _normal_bf16(_rng(c.seed, TAG_VBLK),
                            (self.total_q, c.num_heads_kv, c.head_dim), c.qkv_std)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.cfg.head_dim)

    # -------------------------------------------------------------- LM head
    @cached_property
    def hidden(self) -> np.ndarray:
        c = self.cfg
        return _normal_bf16(_rng(c.seed, TAG_HID), (self.total_q, c.hidden),
                            c.hidden_std)

    @cached_property
    def w_vocab(self) -> np.ndarray:
        c = self.cfg
        V, H = c.vocab, c.hidden
        out = np.empty((V, H), np.uint16)
        n_chunks = (V + W_ROWS_PER_CHUNK - 1) // W_ROWS_PER_CHUNK

        def work(ch):
            lo = ch * W_ROWS_PER_CHUNK
            hi = min(V, lo + W_ROWS_PER_CHUNK)
            out[lo:hi] = _normal_bf16(_rng(c.seed, TAG_W, ch), (hi - lo, H),
                                      c.w_std)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
        return out

    # ----------------------------------------------------------- randomness
    @cached_property
    def req_id(self) -> np.ndarray:
        c = self.cfg
        r = _rng(c.seed, TAG_REQ)
        return r.choice(np.uint64(1) << np.uint64(32), size=c.batch,
                        replace=False).astype(np.uint32)

    @cached_property
    def philox_seed(self) -> int:
        return int(_rng(self.cfg.seed, TAG_SEED).integers(0, 2**63 - 1)) * 2 + 1

    # --------------------------------------------------------- target logits
    @cached_property
    def target_sigma(self) -> np.ndarray:
        """Per-request noise scale for the drafter-plus-noise target."""
        t = self.cfg.target
        B = self.cfg.batch
        if t[0] == "normal":
            return np.full(B, float(t[1]))
        lo, hi = float(t[1]), float(t[2])
        if B == 1 or lo == hi:
            return np.full(B, lo)
        s = np.exp(np.linspace(math.log(lo), math.log(hi), B))
        return _rng(self.cfg.seed, TAG_SIGMA).permutation(s)

    def target_row_source(self) -> np.ndarray:
        """For each target row, the draft row whose logits it is built from in
        the drafter-plus-noise workload (the bonus row reuses the last draft
        row of its request)."""
        bud = self.budgets
        src = np.empty(self.total_target_rows, np.int64)
        for b in range(self.cfg.batch):
            k = int(bud.draft_k[b])
            for j in range(int(bud.verify_b[b]) + 1):
                src[bud.t_off[b] + j] = bud.q_off[b] + min(j, k - 1)
        return src

    @cached_property
    def target_logits(self) -> np.ndarray:
        """fp32 ``[R, V]`` target logits of the ``("normal", sigma)`` workloads.
        The drafter-plus-noise workload is built by ``target_from_drafter``
        from drafter logits the caller supplies."""
        c = self.cfg
        if c.target[0] != "normal":
            raise ValueError(f"{c.name}: target logits depend on the drafter's; "
                             "build them with target_from_drafter(drafter_logits)")
        R, V = self.total_target_rows, c.vocab
        bud = self.budgets
        out = np.empty((R, V), np.float32)
        row_req = np.repeat(np.arange(c.batch), np.diff(bud.t_off))
        n_chunks = (R + TGT_ROWS_PER_CHUNK - 1) // TGT_ROWS_PER_CHUNK
        sig = self.target_sigma

        def work(ch):
            lo = ch * TGT_ROWS_PER_CHUNK
            hi = min(R, lo + TGT_ROWS_PER_CHUNK)
            x = _rng(c.seed, TAG_TGT, ch).standard_normal((hi - lo, V), dtype=np.float32)
            x *= sig[row_req[lo:hi], None].astype(np.float32)
            out[lo:hi] = x

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
        return out

    def target_from_drafter(self, drafter_logits: np.ndarray) -> np.ndarray:
        """Target logits of the drafter-plus-noise workload: for every target
        row, the drafter logits of the row ``target_row_source`` names plus
        seeded N(0, sigma_b^2) noise, rounded to fp32.  ``drafter_logits``
        ``[total_q, V]`` come from whoever evaluates the drafter's LM head."""
        c = self.cfg
        R, V = self.total_target_rows, c.vocab
        bud = self.budgets
        assert drafter_logits.shape == (self.total_q, V)
        out = np.empty((R, V), np.float32)
        row_req = np.repeat(np.arange(c.batch), np.diff(bud.t_off))
        n_chunks = (R + TGT_ROWS_PER_CHUNK - 1) // TGT_ROWS_PER_CHUNK
        sig = self.target_sigma
        src = self.target_row_source()

        def work(ch):
            lo = ch * TGT_ROWS_PER_CHUNK
            hi = min(R, lo + TGT_ROWS_PER_CHUNK)
            x = _rng(c.seed, TAG_NOISE, ch).standard_normal((hi - lo, V))
            x *= sig[row_req[lo:hi], None]
            x += drafter_logits[src[lo:hi]]
            out[lo:hi] = x.astype(np.float32)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
        return out

    # ----------------------------------------------------------------- misc
    def random_draft_tokens(self) -> np.ndarray:
        """Seeded tokens in [0, V) standing in for drafts in verify-only runs."""
        return _rng(self.cfg.seed, TAG_TOK).integers(
            0, self.cfg.vocab, self.total_q).astype(np.int32)

    def random_draft_logits(self, sigma: float = 1.0) -> np.ndarray:
        """Seeded fp32 draft logits standing in for the LM head in
        verify-only runs."""
        c = self.cfg
        return (_rng(c.seed, TAG_TOK, 1).standard_normal(
            (self.total_q, c.vocab)) * sigma).astype(np.float32)

    # ------------------------------------------------------ context summary
    def summary_queries(self, n_summary: int = 16) -> np.ndarray:
        """Seeded stand-in for the learned summary queries U: bf16 bits
        ``[Hkv, n_summary, D]`` drawn N(0, 1) like the cached keys."""
        c = self.cfg
        return _normal_bf16(_rng(c.seed, TAG_SUMQ, n_summary),
                            (c.num_heads_kv, n_summary, c.head_dim), 1.0)

    def summary_values(self, n_summary: int = 16) -> np.ndarray:
        """Seeded fp32 ``[B, Hkv, n_summary, D]`` standing in for a summary
        state when only the draft attention is exercised (an attention
        output over N(0, 1) values is a convex combination of them, so its
        entries are drawn N(0, 0.1^2))."""
        c = self.cfg
        return (_rng(c.seed, TAG_SUMV, n_summary).standard_normal(
            (c.batch, c.num_heads_kv, n_summary, c.head_dim)) * 0.1).astype(np.float32)

    # ------------------------------------------------------ pruned vocabulary
    def pruned_vocab(self, v_draft: int) -> np.ndarray:
        """Seeded stand-in for a pruned drafter vocabulary: ``v_draft``
        distinct target token ids (int32, ascending), the rows of the target
        LM head the drafter predicts over."""
        c = self.cfg
        ids = _rng(c.seed, TAG_VMAP, v_draft).choice(c.vocab, size=v_draft, replace=False)
        return np.sort(ids).astype(np.int32)

    # ------------------------------------------------- sequential correction
    def markov_tables(self, rank: int = 256):
        """Seeded stand-ins for the correction's output mapping W_c and
        embedding table e_c, bf16 bits ``[V, rank]`` each, entries
        N(0, s^2) with s^2 = 0.5 / sqrt(rank): the correction of one logit
        has standard deviation 0.5 whatever the rank."""
        c = self.cfg
        s = float(np.sqrt(0.5 / np.sqrt(rank)))
        return (_normal_bf16(_rng(c.seed, TAG_MKW, rank), (c.vocab, rank), s),
                _normal_bf16(_rng(c.seed, TAG_MKE, rank), (c.vocab, rank), s))

    def anchor_tokens(self) -> np.ndarray:
        """Seeded committed tokens y_0, one per request, in [0, V)."""
        c = self.cfg
        return _rng(c.seed, TAG_ANCHOR).integers(0, c.vocab, c.batch).astype(np.int32)

    def unigram_counts(self) -> np.ndarray:
        """Seeded stand-in for corpus token counts, int64 ``[V]``: a Zipf-like
        profile (1e9 / rank^1.1) over a random permutation of the vocabulary,
        with a tenth of the entries never seen (count 0)."""
        c = self.cfg
        rng = _rng(c.seed, TAG_COUNTS)
        counts = (1e9 / np.arange(1, c.vocab + 1) ** 1.1).astype(np.int64)
        counts[rng.random(c.vocab) < 0.1] = 0
        return rng.permutation(counts)
