"""Helpers of the GPU parity tests: move seeded inputs to the device, run the library's walks,
and compare them with the CPU oracle (teacher-forced, see oracle/check.py)."""
import numpy as np
import torch

import dspark_markov_draft_amd as dm
import oracle
from oracle.check import check_walk

DEV = torch.device("cuda:0")


def lb_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Problem:
    """One walk problem: CPU copies for the oracle, device copies for the library."""

    def __init__(self, w1, w2, base, start, seeds=None, temps=None, positions=None):
        self.w1_cpu, self.w2_cpu = w1, w2                 # torch CPU, fp32/bf16/f16
        self.base_np = np.ascontiguousarray(base.numpy() if torch.is_tensor(base) else base,
                                            dtype=np.float32)
        self.start_np = np.asarray(start.numpy() if torch.is_tensor(start) else start, np.int32)
        bs = self.base_np.shape[0]
        self.seeds_np = (np.asarray(seeds, np.uint64) if seeds is not None else
                         np.arange(1, bs + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15))
        self.temps_np = (np.asarray(temps, np.float32) if temps is not None else
                         np.ones(bs, np.float32))
        self.pos_np = None if positions is None else np.asarray(positions, np.int64)
        # device
        self.w1 = w1.to(DEV)
        self.w2 = w2.to(DEV)
        self.base = torch.from_numpy(self.base_np).to(DEV)
        self.start = torch.from_numpy(self.start_np).to(DEV)
        self.seeds = torch.from_numpy(self.seeds_np.view(np.int64)).to(DEV)
        self.temps = torch.from_numpy(self.temps_np).to(DEV)
        self.pos = None if self.pos_np is None else torch.from_numpy(self.pos_np).to(DEV)
        self._orc = None
        self._w1_np = None

    @property
    def shape(self):
        return self.base_np.shape

    def oracle_q(self):
        if self._orc is None:
            self._orc = oracle.quantize_w2(self.w2_cpu.float().numpy())
        return self._orc

    def w1_np(self):
        if self._w1_np is None:
            self._w1_np = self.w1_cpu.float().numpy()
        return self._w1_np

    def quantize(self):
        return dm.dspark_quantize_w2(self.w2)

    def greedy(self, want_logits=True, ws=None, qs=None):
        bs, T, V = self.shape
        q, s = qs if qs is not None else self.quantize()
        ws = dm.new_workspace(bs, T, V) if ws is None else ws
        logits = torch.empty((bs, T, V), dtype=torch.float32, device=DEV) if want_logits else None
        tok = dm.dspark_walk_greedy(q, s, self.w1, self.base, self.start, ws, out_logits=logits)
        torch.cuda.synchronize()
        return tok.cpu().numpy(), (None if logits is None else logits.cpu().numpy())

    def sample(self, ws=None, qs=None):
        bs, T, V = self.shape
        q, s = qs if qs is not None else self.quantize()
        ws = dm.new_workspace(bs, T, V) if ws is None else ws
        tok, lb = dm.dspark_walk_sample(q, s, self.w1, self.base, self.start, self.seeds,
                                        self.temps, ws, positions=self.pos)
        torch.cuda.synchronize()
        return tok.cpu().numpy(), lb_bits(lb)

    def topk(self, k, sample=False, want_logits=True, ws=None, qs=None):
        """Top-k walk: (tokens, dense fp32 logits or None) greedy; (tokens, bf16 bits) sample."""
        bs, T, V = self.shape
        q, s = qs if qs is not None else self.quantize()
        ws = dm.new_workspace(bs, T, V, k) if ws is None else ws
        if sample:
            tok, lb = dm.dspark_walk_topk(q, s, self.w1, self.base, self.start, k, ws,
                                          sample=True, seeds=self.seeds,
                                          temperature=self.temps, positions=self.pos)
            torch.cuda.synchronize()
            return tok.cpu().numpy(), lb_bits(lb)
        logits = torch.empty((bs, T, V), dtype=torch.float32, device=DEV) if want_logits else None
        tok, _ = dm.dspark_walk_topk(q, s, self.w1, self.base, self.start, k, ws,
                                     draft_logits=logits)
        torch.cuda.synchronize()
        return tok.cpu().numpy(), (None if logits is None else logits.cpu().numpy())

    def check_topk(self, k, tokens, out, sample=False, requests=None):
        q, s = self.oracle_q()
        if sample:
            return check_walk(q, s, self.w1_np(), self.base_np, self.start_np, tokens,
                              sample=True, seeds=self.seeds_np, temps=self.temps_np,
                              positions=self.pos_np, lb=out, k=k, requests=requests)
        return check_walk(q, s, self.w1_np(), self.base_np, self.start_np, tokens, logits=out,
                          k=k, requests=requests)

    def check_greedy(self, tokens, logits, requests=None):
        q, s = self.oracle_q()
        return check_walk(q, s, self.w1_np(), self.base_np, self.start_np, tokens, logits=logits,
                          requests=requests)

    def check_sample(self, tokens, lb, requests=None):
        q, s = self.oracle_q()
        return check_walk(q, s, self.w1_np(), self.base_np, self.start_np, tokens, sample=True,
                          seeds=self.seeds_np, temps=self.temps_np, positions=self.pos_np,
                          lb=lb, requests=requests)


def random_problem(V, T, bs, dtype=torch.bfloat16, w_std=0.02, base_std=3.0, seed=0,
                   temps=None, positions=None):
    g = torch.Generator().manual_seed(seed)
    w1 = (torch.randn(V, 256, generator=g) * w_std).to(dtype)
    w2 = (torch.randn(V, 256, generator=g) * w_std).to(dtype)
    base = torch.randn(bs, T, V, generator=g) * base_std
    start = torch.randint(0, V, (bs,), generator=g, dtype=torch.int64).to(torch.int32)
    rng = np.random.default_rng(seed)
    seeds = rng.integers(0, 2**64, bs, dtype=np.uint64)
    return Problem(w1, w2, base, start, seeds=seeds, temps=temps, positions=positions)
