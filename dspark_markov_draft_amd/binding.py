"""Thin Python binding of libdspark.so, the gfx950 DSpark Markov draft walk.

Every function has the name of the C entry point it calls and only marshals arguments: torch
tensors in (device memory and the current stream come from PyTorch), status codes out as
``DsparkError``. All arithmetic runs in the HIP kernels behind the C ABI (``include/dspark.h``).
There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")

F32, BF16, F16 = 0, 1, 2
RANK = 256
MAX_STEPS, MAX_BS, MAX_V, MAX_TOPK = 16, 64, 270336, 2048
DEBUG_MAX_WORKGROUPS, DEBUG_SPIN_LIMIT, DEBUG_WAIT_UNSET_FLAG, DEBUG_STAMPS = 1, 2, 3, 4
DEBUG_FORCE_PATH = 5
DEBUG_KERNEL_TIMING = 6
DEBUG_MFMA_WAVES = 7
DEBUG_TOPK_SPLIT = 8
PATH_DOT4, PATH_MFMA, PATH_MFMA1 = 1, 2, 3
STAMPS_PER_WG = 210

OK = 0
ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_NO_DEVICE = -1, -2, -3, -4
ERR_LAUNCH, ERR_NONFINITE, ERR_TIMEOUT = -5, -6, -7

_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class DsparkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class WalkPlan(ctypes.Structure):
    _fields_ = [("device_cus", ctypes.c_int32), ("num_workgroups", ctypes.c_int32),
                ("rows_per_workgroup", ctypes.c_int32), ("rows_in_registers", ctypes.c_int32),
                ("rows_in_lds", ctypes.c_int32), ("rows_streamed", ctypes.c_int32),
                ("resident_bytes", ctypes.c_int64), ("streamed_bytes", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int32), ("path", ctypes.c_int32),
                ("reg_units", ctypes.c_int32), ("lds_units", ctypes.c_int32),
                ("total_units", ctypes.c_int32), ("stage_bufs", ctypes.c_int32),
                ("stage_stride", ctypes.c_int32), ("waves_per_workgroup", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib():
    """Load libdspark.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DsparkError(ERR_NO_DEVICE, f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.dspark_status_string.argtypes = [i32]
        L.dspark_status_string.restype = ctypes.c_char_p
        L.dspark_quantize_w2.argtypes = [vp, i32, i64, i64, vp, vp, vp]
        L.dspark_walk_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.dspark_walk_workspace_bytes.restype = ctypes.c_size_t
        L.dspark_walk_plan_query.argtypes = [i64, i64, i64, ctypes.POINTER(WalkPlan)]
        L.dspark_walk_greedy.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        L.dspark_walk_greedy_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, vp,
                                                 vp, vp, vp]
        L.dspark_walk_sample.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, vp, vp, vp,
                                         vp, vp, vp, ctypes.c_size_t, vp]
        L.dspark_walk_sample_icdf.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, vp, vp,
                                              vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dspark_walk_topk.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, i64, i32, vp,
                                       vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dspark_walk_plan_for.argtypes = [ctypes.c_int32, i64, i64, i64, i64,
                                           ctypes.POINTER(WalkPlan)]
        L.dspark_w2_prune_bound.argtypes = [vp, vp, i64, i64, vp, vp]
        L.dspark_walk_greedy_pruned.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, i64,
                                                vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dspark_verify_workspace_bytes.argtypes = [i64, i64, i64]
        L.dspark_verify_workspace_bytes.restype = ctypes.c_size_t
        L.dspark_verify.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp,
                                    ctypes.c_size_t, vp]
        L.dspark_workspace_status.argtypes = [vp, vp]
        L.dspark_philox_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, i64, i64, vp, vp]
        L.dspark_debug_set.argtypes = [i32, i64]
        L.dspark_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_float), i32,
                                          ctypes.POINTER(i32)]
        for name in ["dspark_quantize_w2", "dspark_walk_plan_query", "dspark_walk_plan_for",
                     "dspark_walk_greedy", "dspark_walk_greedy_noalloc",
                     "dspark_walk_sample", "dspark_walk_topk", "dspark_workspace_status",
                     "dspark_philox_words", "dspark_debug_set", "dspark_kernel_times",
                     "dspark_verify", "dspark_w2_prune_bound", "dspark_walk_greedy_pruned",
                     "dspark_walk_sample_icdf"]:
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def dspark_status_string(status: int) -> str:
    return lib().dspark_status_string(int(status)).decode()


def _check(status: int):
    if status != OK:
        raise DsparkError(status, dspark_status_string(status))


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdspark must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


# The C ABI sees pointers only, so the wrappers check what it cannot: every tensor's dtype and
# shape against the sizes the call is made with, and that all of them sit on one CUDA device.
# A mismatch raises ValueError before anything reaches the library (a short or mistyped buffer
# would otherwise be read or written past its end by the kernels).
_W_DTYPES = (torch.float32, torch.bfloat16, torch.float16)


def _expect(t, name: str, dtypes, shape, optional: bool = False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not torch.is_tensor(t):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be {want}, got {str(t.dtype).replace('torch.', '')}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(**tensors):
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a CUDA device, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")


def _check_walk_args(q, s, w1, base, start, workspace, draft_tokens):
    _expect(base, "base", torch.float32, None)
    if base.dim() != 3:
        raise ValueError(f"base must be [bs, T, V], got shape {tuple(base.shape)}")
    bs, T, V = base.shape
    _expect(q, "q", torch.int8, (V, RANK))
    _expect(s, "s", torch.float32, (V,))
    _expect(w1, "w1", _W_DTYPES, (V, RANK))
    _expect(start, "start", torch.int32, (bs,))
    if not torch.is_tensor(workspace) or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D tensor")
    _expect(draft_tokens, "draft_tokens", torch.int32, (bs, T))
    return bs, T, V


def _check_sample_args(bs, seeds, temperature, positions):
    _expect(seeds, "seeds", torch.int64, (bs,))
    _expect(temperature, "temperature", torch.float32, (bs,))
    _expect(positions, "positions", torch.int64, (bs,), optional=True)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE_CODE:
        raise DsparkError(ERR_UNSUPPORTED, f"unsupported dtype {t.dtype}")
    return _DTYPE_CODE[t.dtype]


def dspark_quantize_w2(w2: torch.Tensor, q: Optional[torch.Tensor] = None,
                       s: Optional[torch.Tensor] = None, stream=None):
    """W2 [V, 256] (fp32 / bf16 / fp16, device) -> (q int8 [V, 256], s fp32 [V])."""
    _expect(w2, "w2", _W_DTYPES, None)
    if w2.dim() != 2:
        raise ValueError(f"w2 must be [V, {RANK}], got shape {tuple(w2.shape)}")
    V, R = w2.shape
    if q is None:
        q = torch.empty((V, R), dtype=torch.int8, device=w2.device)
    if s is None:
        s = torch.empty((V,), dtype=torch.float32, device=w2.device)
    _expect(q, "q", torch.int8, (V, R))
    _expect(s, "s", torch.float32, (V,))
    _same_device(w2=w2, q=q, s=s)
    _check(lib().dspark_quantize_w2(_p(w2), _dtype_code(w2), V, R, _p(q), _p(s), _stream(stream)))
    return q, s


def dspark_walk_workspace_bytes(bs: int, T: int, V: int, k: int = 0) -> int:
    return int(lib().dspark_walk_workspace_bytes(bs, T, V, k))


def new_workspace(bs: int, T: int, V: int, k: int = 0, device="cuda") -> torch.Tensor:
    """A zeroed workspace of the size the walk needs (zeroed once; walks leave it zeroed)."""
    n = dspark_walk_workspace_bytes(bs, T, V, k)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def dspark_walk_plan_query(bs: int, T: int, V: int) -> dict:
    plan = WalkPlan()
    _check(lib().dspark_walk_plan_query(bs, T, V, ctypes.byref(plan)))
    return plan.as_dict()


def dspark_walk_plan_for(cus: int, max_lds: int, bs: int, T: int, V: int) -> dict:
    plan = WalkPlan()
    _check(lib().dspark_walk_plan_for(cus, max_lds, bs, T, V, ctypes.byref(plan)))
    return plan.as_dict()


def dspark_walk_greedy(q, s, w1, base, start, workspace, draft_tokens=None, out_logits=None,
                       stream=None):
    """Greedy walk. base [bs, T, V] fp32; start [bs] int32. Returns draft_tokens [bs, T] int32."""
    _expect(base, "base", torch.float32, None)
    bs, T, V = base.shape if base.dim() == 3 else (0, 0, 0)
    if draft_tokens is None and base.dim() == 3:
        draft_tokens = torch.empty((bs, T), dtype=torch.int32, device=base.device)
    bs, T, V = _check_walk_args(q, s, w1, base, start, workspace, draft_tokens)
    _expect(out_logits, "out_logits", torch.float32, (bs, T, V), optional=True)
    _same_device(q=q, s=s, w1=w1, base=base, start=start, workspace=workspace,
                 draft_tokens=draft_tokens, out_logits=out_logits)
    _check(lib().dspark_walk_greedy(_p(q), _p(s), _p(w1), _dtype_code(w1), _p(base), _p(start),
                                    bs, T, V, q.shape[1], _p(draft_tokens), _p(out_logits),
                                    _p(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return draft_tokens


def dspark_walk_greedy_noalloc(q, s, w1, base, start, draft_tokens=None, out_logits=None,
                               error_word=None, stream=None):
    """Greedy walk on the library-held scratch (no workspace argument; allocates nothing when
    draft_tokens is given). error_word: optional int32 [1] device tensor, zeroed by the caller,
    where the walk records -status on an error. Returns draft_tokens [bs, T] int32."""
    _expect(base, "base", torch.float32, None)
    if base.dim() == 3 and draft_tokens is None:
        draft_tokens = torch.empty(base.shape[:2], dtype=torch.int32, device=base.device)
    if base.dim() != 3:
        raise ValueError(f"base must be [bs, T, V], got shape {tuple(base.shape)}")
    bs, T, V = base.shape
    _expect(q, "q", torch.int8, (V, RANK))
    _expect(s, "s", torch.float32, (V,))
    _expect(w1, "w1", _W_DTYPES, (V, RANK))
    _expect(start, "start", torch.int32, (bs,))
    _expect(draft_tokens, "draft_tokens", torch.int32, (bs, T))
    _expect(out_logits, "out_logits", torch.float32, (bs, T, V), optional=True)
    _expect(error_word, "error_word", torch.int32, (1,), optional=True)
    _same_device(q=q, s=s, w1=w1, base=base, start=start, draft_tokens=draft_tokens,
                 out_logits=out_logits, error_word=error_word)
    _check(lib().dspark_walk_greedy_noalloc(_p(q), _p(s), _p(w1), _dtype_code(w1), _p(base),
                                            _p(start), bs, T, V, q.shape[1], _p(draft_tokens),
                                            _p(out_logits), _p(error_word), _stream(stream)))
    return draft_tokens


def dspark_walk_sample(q, s, w1, base, start, seeds, temperature, workspace, positions=None,
                       draft_tokens=None, draft_logits=None, stream=None):
    """Probabilistic walk. seeds [bs] int64 holding the uint64 bits; temperature [bs] fp32;
    positions [bs] int64 or None. Returns (draft_tokens [bs, T] int32, draft_logits [bs, T, V]
    bf16)."""
    _expect(base, "base", torch.float32, None)
    if base.dim() == 3:
        bs, T, V = base.shape
        if draft_tokens is None:
            draft_tokens = torch.empty((bs, T), dtype=torch.int32, device=base.device)
        if draft_logits is None:
            draft_logits = torch.empty((bs, T, V), dtype=torch.bfloat16, device=base.device)
    bs, T, V = _check_walk_args(q, s, w1, base, start, workspace, draft_tokens)
    _check_sample_args(bs, seeds, temperature, positions)
    _expect(draft_logits, "draft_logits", torch.bfloat16, (bs, T, V))
    _same_device(q=q, s=s, w1=w1, base=base, start=start, workspace=workspace,
                 draft_tokens=draft_tokens, draft_logits=draft_logits, seeds=seeds,
                 temperature=temperature, positions=positions)
    _check(lib().dspark_walk_sample(_p(q), _p(s), _p(w1), _dtype_code(w1), _p(base), _p(start),
                                    bs, T, V, q.shape[1], _p(seeds), _p(positions),
                                    _p(temperature), _p(draft_tokens), _p(draft_logits),
                                    _p(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return draft_tokens, draft_logits


def dspark_walk_sample_icdf(q, s, w1, base, start, seeds, temperature, workspace,
                            positions=None, draft_tokens=None, draft_logits=None, stream=None):
    """Probabilistic walk drawing each token by inverse CDF (arguments and outputs as
    dspark_walk_sample). Returns (draft_tokens [bs, T] int32, draft_logits [bs, T, V] bf16)."""
    _expect(base, "base", torch.float32, None)
    if base.dim() == 3:
        bs, T, V = base.shape
        if draft_tokens is None:
            draft_tokens = torch.empty((bs, T), dtype=torch.int32, device=base.device)
        if draft_logits is None:
            draft_logits = torch.empty((bs, T, V), dtype=torch.bfloat16, device=base.device)
    bs, T, V = _check_walk_args(q, s, w1, base, start, workspace, draft_tokens)
    _check_sample_args(bs, seeds, temperature, positions)
    _expect(draft_logits, "draft_logits", torch.bfloat16, (bs, T, V))
    _same_device(q=q, s=s, w1=w1, base=base, start=start, workspace=workspace,
                 draft_tokens=draft_tokens, draft_logits=draft_logits, seeds=seeds,
                 temperature=temperature, positions=positions)
    _check(lib().dspark_walk_sample_icdf(_p(q), _p(s), _p(w1), _dtype_code(w1), _p(base),
                                         _p(start), bs, T, V, q.shape[1], _p(seeds),
                                         _p(positions), _p(temperature), _p(draft_tokens),
                                         _p(draft_logits), _p(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(stream)))
    return draft_tokens, draft_logits


def dspark_walk_topk(q, s, w1, base, start, k, workspace, sample=False, seeds=None,
                     temperature=None, positions=None, draft_tokens=None, draft_logits=None,
                     stream=None):
    """Top-k walk. Returns (draft_tokens, draft_logits): draft_logits is bf16 [bs, T, V] when
    sampling, else the fp32 [bs, T, V] tensor passed in (or None)."""
    _expect(base, "base", torch.float32, None)
    if base.dim() == 3:
        bs, T, V = base.shape
        if draft_tokens is None:
            draft_tokens = torch.empty((bs, T), dtype=torch.int32, device=base.device)
        if sample and draft_logits is None:
            draft_logits = torch.empty((bs, T, V), dtype=torch.bfloat16, device=base.device)
    bs, T, V = _check_walk_args(q, s, w1, base, start, workspace, draft_tokens)
    if sample:
        _check_sample_args(bs, seeds, temperature, positions)
        _expect(draft_logits, "draft_logits", torch.bfloat16, (bs, T, V))
    else:
        _expect(draft_logits, "draft_logits", torch.float32, (bs, T, V), optional=True)
    _same_device(q=q, s=s, w1=w1, base=base, start=start, workspace=workspace,
                 draft_tokens=draft_tokens, draft_logits=draft_logits,
                 seeds=seeds if sample else None, temperature=temperature if sample else None,
                 positions=positions if sample else None)
    _check(lib().dspark_walk_topk(_p(q), _p(s), _p(w1), _dtype_code(w1), _p(base), _p(start), bs,
                                  T, V, q.shape[1], int(k), int(bool(sample)), _p(seeds),
                                  _p(positions), _p(temperature), _p(draft_tokens),
                                  _p(draft_logits), _p(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return draft_tokens, draft_logits


def dspark_w2_prune_bound(q, s, bound=None, stream=None):
    """Load-time bound B = max_v s[v] * sum_k |q[v,k]| of the lossless pruned walk, as a device
    fp32 tensor of one element."""
    _expect(q, "q", torch.int8, None)
    if q.dim() != 2:
        raise ValueError(f"q must be [V, {RANK}], got shape {tuple(q.shape)}")
    V = q.shape[0]
    _expect(s, "s", torch.float32, (V,))
    if bound is None:
        bound = torch.empty(1, dtype=torch.float32, device=q.device)
    _expect(bound, "bound", torch.float32, (1,))
    _same_device(q=q, s=s, bound=bound)
    _check(lib().dspark_w2_prune_bound(_p(q), _p(s), V, q.shape[1], _p(bound), _stream(stream)))
    return bound


def dspark_walk_greedy_pruned(q, s, w1, base, start, k, w2_bound, workspace, draft_tokens=None,
                              out_logits=None, dense_steps=None, stream=None):
    """Lossless top-k pruned greedy walk: the tokens of dspark_walk_greedy, computing only the
    W2 rows of the k best base logits on every step the bound certifies. Returns draft_tokens."""
    _expect(base, "base", torch.float32, None)
    if base.dim() == 3 and draft_tokens is None:
        draft_tokens = torch.empty(base.shape[:2], dtype=torch.int32, device=base.device)
    bs, T, V = _check_walk_args(q, s, w1, base, start, workspace, draft_tokens)
    _expect(w2_bound, "w2_bound", torch.float32, (1,))
    _expect(out_logits, "out_logits", torch.float32, (bs, T, V), optional=True)
    _expect(dense_steps, "dense_steps", torch.int32, (bs,), optional=True)
    _same_device(q=q, s=s, w1=w1, base=base, start=start, workspace=workspace,
                 draft_tokens=draft_tokens, w2_bound=w2_bound, out_logits=out_logits,
                 dense_steps=dense_steps)
    _check(lib().dspark_walk_greedy_pruned(_p(q), _p(s), _p(w1), _dtype_code(w1), _p(base),
                                           _p(start), bs, T, V, q.shape[1], int(k), _p(w2_bound),
                                           _p(draft_tokens), _p(out_logits), _p(dense_steps),
                                           _p(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream)))
    return draft_tokens


VERIFY_TOKEN, VERIFY_BLOCK = 0, 1


def dspark_verify_workspace_bytes(bs: int, T: int, V: int) -> int:
    return int(lib().dspark_verify_workspace_bytes(bs, T, V))


def dspark_verify(draft_logits, draft_tokens, target_logits, temperature, uniforms, workspace,
                  mode=VERIFY_TOKEN, accepted=None, out_tokens=None, accept_prob=None,
                  stream=None):
    """Verification of drafted blocks (token or block verification). draft_logits bf16
    [bs, T, V]; draft_tokens int32 [bs, T]; target_logits fp32 [bs, T + 1, V]; temperature fp32
    [bs]; uniforms fp32 [bs, T + 1]. Returns (accepted int32 [bs], out_tokens int32 [bs, T + 1],
    accept_prob fp32 [bs, T] or None)."""
    _expect(draft_logits, "draft_logits", torch.bfloat16, None)
    if draft_logits.dim() != 3:
        raise ValueError(f"draft_logits must be [bs, T, V], got {tuple(draft_logits.shape)}")
    bs, T, V = draft_logits.shape
    dev = draft_logits.device
    if accepted is None:
        accepted = torch.empty(bs, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((bs, T + 1), dtype=torch.int32, device=dev)
    _expect(draft_tokens, "draft_tokens", torch.int32, (bs, T))
    _expect(target_logits, "target_logits", torch.float32, (bs, T + 1, V))
    _expect(temperature, "temperature", torch.float32, (bs,))
    _expect(uniforms, "uniforms", torch.float32, (bs, T + 1))
    _expect(accepted, "accepted", torch.int32, (bs,))
    _expect(out_tokens, "out_tokens", torch.int32, (bs, T + 1))
    _expect(accept_prob, "accept_prob", torch.float32, (bs, T), optional=True)
    if not torch.is_tensor(workspace) or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D tensor")
    if mode not in (VERIFY_TOKEN, VERIFY_BLOCK):
        raise ValueError("mode must be VERIFY_TOKEN or VERIFY_BLOCK")
    _same_device(draft_logits=draft_logits, draft_tokens=draft_tokens,
                 target_logits=target_logits, temperature=temperature, uniforms=uniforms,
                 accepted=accepted, out_tokens=out_tokens, accept_prob=accept_prob,
                 workspace=workspace)
    _check(lib().dspark_verify(_p(draft_logits), _p(draft_tokens), _p(target_logits),
                               _p(temperature), _p(uniforms), bs, T, V, int(mode), _p(accepted),
                               _p(out_tokens), _p(accept_prob), _p(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)))
    return accepted, out_tokens, accept_prob


def dspark_workspace_status(workspace, stream=None) -> int:
    return int(lib().dspark_workspace_status(_p(workspace), _stream(stream)))


def check_workspace(workspace, stream=None) -> None:
    """Synchronising check of the error a walk recorded in its workspace (for callers that share
    the GPU with other work). On DSPARK_ERR_TIMEOUT the tokens of that walk are invalid and the
    workspace may hold stale keys: it is zeroed again before the error is raised, so the next
    walk can use it. Any recorded error raises DsparkError."""
    st = dspark_workspace_status(workspace, stream)
    if st == ERR_TIMEOUT:
        workspace.zero_()
    _check(st)


def dspark_philox_words(seed: int, position: int, v0: int, n: int, device="cuda",
                        stream=None) -> np.ndarray:
    out = torch.empty(n, dtype=torch.int32, device=device)
    _check(lib().dspark_philox_words(seed, position, v0, n, _p(out), _stream(stream)))
    return out.cpu().numpy().view(np.uint32)


def dspark_debug_set(key: int, value: int):
    _check(lib().dspark_debug_set(key, value))


def dspark_kernel_times(max_count: int = 4096) -> list:
    """Durations (us) of the walk kernels launched since kernel timing was switched on or last
    read, oldest first (see DEBUG_KERNEL_TIMING)."""
    buf = (ctypes.c_float * max_count)()
    n = ctypes.c_int32(0)
    _check(lib().dspark_kernel_times(buf, max_count, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]
