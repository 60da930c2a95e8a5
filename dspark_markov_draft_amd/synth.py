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


def with_heavy_entries(w: torch.Tensor, per_row: int, mult: float, std: float,
                       seed: int) -> torch.Tensor:
    """A copy of ``w`` [V, 256] in which ``per_row`` entries of every row, at seeded random
    columns, are replaced by +-``mult`` * ``std`` (random signs): rows whose largest entries are
    far above the rest, as some trained rows have. Same dtype as ``w``."""
    g = torch.Generator().manual_seed(seed)
    V, K = w.shape
    cols = torch.argsort(torch.rand(V, K, generator=g), dim=1)[:, :per_row]
    signs = torch.where(torch.rand(V, per_row, generator=g) < 0.5, -1.0, 1.0)
    out = w.float().clone()
    out.scatter_(1, cols, signs * (mult * std))
    return out.to(w.dtype)


def seeds_as_int64(seeds: np.ndarray) -> torch.Tensor:
    """uint64 request seeds as a same-bits int64 tensor (torch has no uint64 arithmetic)."""
    return torch.from_numpy(np.ascontiguousarray(seeds, dtype=np.uint64).view(np.int64))


@dataclass
class VerifyInputs:
    draft_lb: torch.Tensor       # [bs, T, V] bf16 (CPU)
    draft_tokens: torch.Tensor   # [bs, T] int32
    target: torch.Tensor         # [bs, T + 1, V] fp32
    temperature: torch.Tensor    # [bs] fp32
    uniforms: torch.Tensor       # [bs, T + 1] fp32 in (0, 1)


def make_verify_inputs(bs: int, T: int, V: int, seed: int, draft_std: float = 3.0,
                       target_noise: float = 1.0, temperature: Optional[float] = 1.0
                       ) -> VerifyInputs:
    """Seeded inputs of a block verification, shaped like a probabilistic walk's output: draft
    logits ~ N(0, draft_std^2) rounded to bf16 (the stored rows); target logits for rows
    0..T-1 = those draft logits + N(0, target_noise^2) (a target model close to the draft),
    row T ~ N(0, draft_std^2); draft tokens uniform on [0, V) (so that steps are both kept and
    rejected); uniforms uniform on [2^-24, 1); temperature fixed, or (None) uniform on
    [0.5, 1.5] per request. Each tensor has its own generator seeded seed * 10 + tensor id."""
    def gen(i):
        return torch.Generator().manual_seed(seed * 10 + i)
    draft = torch.randn(bs, T, V, generator=gen(0)) * draft_std
    lb = draft.to(torch.bfloat16)
    target = torch.empty(bs, T + 1, V)
    target[:, :T] = lb.float() + torch.randn(bs, T, V, generator=gen(1)) * target_noise
    target[:, T] = torch.randn(bs, V, generator=gen(2)) * draft_std
    tokens = torch.randint(0, V, (bs, T), generator=gen(3), dtype=torch.int64).to(torch.int32)
    u = torch.rand(bs, T + 1, generator=gen(4)).clamp_min(2.0 ** -24)
    if temperature is None:
        temps = 0.5 + torch.rand(bs, generator=gen(5))
    else:
        temps = torch.full((bs,), float(temperature))
    return VerifyInputs(lb, tokens, target, temps.float(), u.float())
