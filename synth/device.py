"""Upload a step's seeded inputs to device memory as torch tensors.

Plumbing only: bit-exact copies of the arrays ``StepInputs`` generates.
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from .inputs import StepInputs


def bf16(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device``."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def i32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def f32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def attention_tensors(inp: StepInputs, device) -> Dict[str, torch.Tensor]:
    b = inp.budgets
    return dict(q=bf16(inp.q, device), k_blk=bf16(inp.k_blk, device),
                v_blk=bf16(inp.v_blk, device), k_cache=bf16(inp.k_cache, device),
                v_cache=bf16(inp.v_cache, device), page_table=i32(inp.page_table, device),
                ctx_len=i32(b.ctx_len, device), q_off=i32(b.q_off, device))


def lm_head_tensors(inp: StepInputs, device) -> Dict[str, torch.Tensor]:
    b = inp.budgets
    return dict(hidden=bf16(inp.hidden, device), w_vocab=bf16(inp.w_vocab, device),
                q_off=i32(b.q_off, device),
                req_id=i32(inp.req_id.view(np.int32), device))


def verify_tensors(inp: StepInputs, device, target: np.ndarray = None) -> Dict[str, torch.Tensor]:
    """Verification inputs; ``target`` overrides the workload's own target
    logits (needed for the drafter-plus-noise workload, whose target is built
    from drafter logits by ``StepInputs.target_from_drafter``)."""
    b = inp.budgets
    tgt = inp.target_logits if target is None else target
    return dict(target_logits=f32(tgt, device), t_off=i32(b.t_off, device),
                q_off=i32(b.q_off, device), req_id=i32(inp.req_id.view(np.int32), device))
