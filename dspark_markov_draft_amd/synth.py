"""Seeded synthetic inputs for the Markov draft walk, shared by the tests, the benchmark and
the smoke check. This module holds no part of the walk's arithmetic: it only draws W1, W2, base
logits, start tokens and request seeds, with the shapes of the workloads measured on the vLLM
pull-request pages (PR #62958, Validation, kernel table: V = 151936 / 129280 / 248320, 5 / 7 / 16
draft tokens, bs 1 / 16 / 64; PR #49969, Results: top-k 512 at 7 tokens).

Recipe (the pages state no input distributions; these stand in for the Qwen3 / DeepSeek-class
drafters, whose weights are not used):
  * every tensor comes from its own ``torch.Generator().manual_seed(S)`` in fp32, then
    ``.to(torch.bfloat16)`` (round to nearest even) where the case says bf16;
  * request seeds come from ``numpy.random.default_rng(S).integers(0, 2**64, dtype=uint64)``;
  * S = 1000 * case.family + 10 * case.sub + tensor id, tensor ids W1 = 0, W2 = 1, base = 2,
    start = 3, seeds = 4.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

RANK = 256


@dataclass(frozen=True)
class Case:
    name: str
    family: int          # workload family (1 tiny, 2 greedy bs1, 3 batched, 4 long/sweep, 5 top-k)
    sub: int             # sub-case within the family (seeds differ per sub-case)
    V: int
    T: int
    bs: int
    wdtype: str          # "f32" or "bf16" (dtype of W1 and W2 as handed to the walk)
    w_std: float
    base_std: float
    k: int = 0           # 0 = full vocabulary, else top-k candidates
    modes: tuple = ("greedy",)
    temperature: float = 1.0


CASES: Dict[str, Case] = {c.name: c for c in [
    Case("tiny_v4096_t4_bs1", 1, 0, 4096, 4, 1, "f32", 0.05, 2.0),
    Case("v151936_t7_bs1", 2, 0, 151936, 7, 1, "bf16", 0.02, 3.0),
    Case("v151936_t7_bs16", 3, 1, 151936, 7, 16, "bf16", 0.02, 3.0, modes=("greedy", "sample")),
    Case("v151936_t7_bs64", 3, 2, 151936, 7, 64, "bf16", 0.02, 3.0, modes=("greedy", "sample")),
    Case("v151936_t16_bs1", 4, 0, 151936, 16, 1, "bf16", 0.02, 3.0, modes=("sample", "greedy")),
    Case("v248320_t16_bs1", 4, 1, 248320, 16, 1, "bf16", 0.02, 3.0, modes=("sample", "greedy")),
    Case("v129280_t5_bs1", 4, 2, 129280, 5, 1, "bf16", 0.02, 3.0, modes=("sample", "greedy")),
    Case("v129280_t5_bs64", 4, 3, 129280, 5, 64, "bf16", 0.02, 3.0, modes=("sample", "greedy")),
    Case("topk512_v151936_t7_bs64", 5, 0, 151936, 7, 64, "bf16", 0.02, 3.0, k=512,
         modes=("greedy", "sample")),
    # the library's largest supported shape (V = 270336, 16 draft steps, 64 requests), same
    # distributions as the V = 151936 workloads: a parity case, not a measured workload
    Case("vmax270336_t16_bs64", 6, 0, 270336, 16, 64, "bf16", 0.02, 3.0,
         modes=("greedy", "sample")),
    Case("vmax270336_t16_bs1", 6, 1, 270336, 16, 1, "bf16", 0.02, 3.0,
         modes=("greedy", "sample")),
]}


def _seed(case: Case, tensor_id: int) -> int:
    return 1000 * case.family + 10 * case.sub + tensor_id


def _normal(shape, std, seed) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


@dataclass
class Inputs:
    case: Case
    w1: torch.Tensor          # [V, 256] fp32 or bf16 (CPU)
    w2: torch.Tensor          # [V, 256] fp32 or bf16 (CPU)
    base: torch.Tensor        # [bs, T, V] fp32 (CPU)
    start: torch.Tensor       # [bs] int32 (CPU)
    seeds: np.ndarray         # [bs] uint64
    temperature: torch.Tensor  # [bs] fp32 (CPU)
    positions: Optional[torch.Tensor] = None  # [bs] int64 or None (offset 0)
    extra: dict = field(default_factory=dict)


def make_inputs(case: Case, bs: Optional[int] = None, V: Optional[int] = None,
                T: Optional[int] = None) -> Inputs:
    """Draw the inputs of ``case``; bs / V / T may be overridden for reduced-size parity runs
    (the distributions stay those of the case)."""
    V = case.V if V is None else V
    T = case.T if T is None else T
    bs = case.bs if bs is None else bs
    dt = torch.bfloat16 if case.wdtype == "bf16" else torch.float32
    w1 = _normal((V, RANK), case.w_std, _seed(case, 0)).to(dt)
    w2 = _normal((V, RANK), case.w_std, _seed(case, 1)).to(dt)
    base = _normal((bs, T, V), case.base_std, _seed(case, 2))
    g = torch.Generator().manual_seed(_seed(case, 3))
    start = torch.randint(0, V, (bs,), generator=g, dtype=torch.int64).to(torch.int32)
    seeds = np.random.default_rng(_seed(case, 4)).integers(0, 2**64, size=bs, dtype=np.uint64,
                                                           endpoint=False)
    temperature = torch.full((bs,), case.temperature, dtype=torch.float32)
    return Inputs(case, w1, w2, base, start, seeds, temperature)


def seeds_as_int64(seeds: np.ndarray) -> torch.Tensor:
    """uint64 request seeds as a same-bits int64 tensor (torch has no uint64 arithmetic)."""
    return torch.from_numpy(np.ascontiguousarray(seeds, dtype=np.uint64).view(np.int64))
