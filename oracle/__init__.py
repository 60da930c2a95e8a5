"""Python access to the plain CPU oracle of the DSpark Markov draft walk (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the HIP library and its Python binding never do, and
the two share no code. Everything here is argument marshalling between numpy arrays and the
C functions; the arithmetic lives in ``oracle.c``, whose header lists the passages of the vLLM
pull-request pages each function follows and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK = 0
ERR_ARG = -1
ERR_NONFINITE = -6


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, u64, u32, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
        vp = ctypes.c_void_p
        L.oracle_quantize_w2.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_quantize_w2.restype = ctypes.c_int
        L.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        L.oracle_philox4x32_10.restype = None
        L.oracle_noise_word.argtypes = [u64, u64, i64]
        L.oracle_noise_word.restype = u32
        L.oracle_uniform.argtypes = [u32]
        L.oracle_uniform.restype = ctypes.c_double
        L.oracle_gumbel.argtypes = [u32]
        L.oracle_gumbel.restype = ctypes.c_double
        L.oracle_bf16_rne.argtypes = [f32]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = f32
        L.oracle_argmax_f32.argtypes = [vp, i64]
        L.oracle_argmax_f32.restype = i64
        L.oracle_topk.argtypes = [vp, i64, i64, vp]
        L.oracle_topk.restype = ctypes.c_int
        L.oracle_step.argtypes = [vp, vp, vp, i64, i64, vp, i64, vp, i64, ctypes.c_int, u64, u64,
                                  f32, vp, vp, vp]
        L.oracle_step.restype = i64
        L.oracle_walk.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, vp,
                                  vp, vp, vp, vp, vp]
        L.oracle_walk.restype = ctypes.c_int
        L.oracle_verify.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp, vp, vp]
        L.oracle_verify.restype = ctypes.c_int
        L.oracle_w2_l1_bound.argtypes = [vp, vp, i64, i64]
        L.oracle_w2_l1_bound.restype = f32
        L.oracle_icdf_uniform.argtypes = [u64, u64]
        L.oracle_icdf_uniform.restype = ctypes.c_double
        L.oracle_icdf_draw.argtypes = [vp, i64, f32, ctypes.c_double]
        L.oracle_icdf_draw.restype = i64
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def quantize_w2(w2: np.ndarray):
    """W2 [V, R] (any float dtype, upcast exactly to fp32) -> (q int8 [V, R], s fp32 [V])."""
    w = _c(w2, np.float32)
    V, R = w.shape
    q = np.empty((V, R), np.int8)
    s = np.empty((V,), np.float32)
    st = lib().oracle_quantize_w2(_ptr(w), V, R, _ptr(q), _ptr(s))
    if st == ERR_NONFINITE:
        raise OracleError("non-finite W2")
    if st != OK:
        raise OracleError(f"oracle_quantize_w2 failed ({st})")
    return q, s


def philox4x32_10(ctr, key) -> np.ndarray:
    c = _c(np.asarray(ctr, dtype=np.uint64).astype(np.uint32), np.uint32)
    k = _c(np.asarray(key, dtype=np.uint64).astype(np.uint32), np.uint32)
    out = np.empty(4, np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def noise_word(seed: int, P: int, v: int) -> int:
    return int(lib().oracle_noise_word(seed, P, v))


def uniform(x: int) -> float:
    return float(lib().oracle_uniform(x))


def gumbel(x: int) -> float:
    return float(lib().oracle_gumbel(x))


def bf16_rne(x: float) -> int:
    return int(lib().oracle_bf16_rne(float(x)))


def bf16_to_f32(h: int) -> float:
    return float(lib().oracle_bf16_to_f32(h))


def argmax_f32(x: np.ndarray) -> int:
    a = _c(x, np.float32)
    return int(lib().oracle_argmax_f32(_ptr(a), a.size))


def topk(row: np.ndarray, k: int) -> np.ndarray:
    r = _c(row, np.float32)
    cand = np.empty(k, np.int32)
    st = lib().oracle_topk(_ptr(r), r.size, k, _ptr(cand))
    if st != OK:
        raise OracleError(f"oracle_topk failed ({st})")
    return cand


def step(q, s, w1, base_row, prev, cand=None, sample=False, seed=0, P=0, temp=1.0):
    """One step of one request. sample: False (greedy), True or 1 (Gumbel), 2 (inverse CDF).
    Returns (token, logits fp32 [V], lb uint16 [V] | None, score fp32 [V] | None)."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    w1 = _c(w1, np.float32)
    base_row = _c(base_row, np.float32)
    V, R = q.shape
    logits = np.empty(V, np.float32)
    lb = np.empty(V, np.uint16) if sample else None
    score = np.empty(V, np.float32) if sample else None
    c = None if cand is None else _c(cand, np.int32)
    tok = lib().oracle_step(_ptr(q), _ptr(s), _ptr(w1), V, R, _ptr(base_row), int(prev), _ptr(c),
                            0 if c is None else c.size, int(sample), int(seed), int(P),
                            float(temp), _ptr(logits), _ptr(lb), _ptr(score))
    if tok < 0:
        raise OracleError(f"oracle_step failed ({tok})")
    return int(tok), logits, lb, score


def walk(q, s, w1, base, start, k=0, sample=False, seeds=None, positions=None, temps=None,
         want_logits=False):
    """Free-running walk. base [bs, T, V]. Returns (tokens int32 [bs, T], logits fp32
    [bs, T, V] | None, lb uint16 [bs, T, V] | None)."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    w1 = _c(w1, np.float32)
    base = _c(base, np.float32)
    start = _c(start, np.int32)
    bs, T, V = base.shape
    R = q.shape[1]
    tokens = np.empty((bs, T), np.int32)
    logits = np.empty((bs, T, V), np.float32) if want_logits else None
    lb = np.empty((bs, T, V), np.uint16) if (want_logits and sample) else None
    sd = None if seeds is None else _c(np.asarray(seeds, dtype=np.uint64), np.uint64)
    ps = None if positions is None else _c(positions, np.int64)
    tp = None if temps is None else _c(temps, np.float32)
    st = lib().oracle_walk(_ptr(q), _ptr(s), _ptr(w1), _ptr(base), _ptr(start), bs, T, V, R, k,
                           int(sample), _ptr(sd), _ptr(ps), _ptr(tp), _ptr(tokens),
                           _ptr(logits), _ptr(lb))
    if st != OK:
        raise OracleError(f"oracle_walk failed ({st})")
    return tokens, logits, lb


VERIFY_TOKEN, VERIFY_BLOCK = 0, 1


def verify(draft_lb, draft_tokens, target_logits, temps, uniforms, mode=VERIFY_TOKEN):
    """Verification of drafted blocks (see oracle_verify in oracle.c).

    draft_lb uint16 [bs, T, V] (bf16 bits), draft_tokens int32 [bs, T], target_logits fp32
    [bs, T + 1, V], temps fp32 [bs], uniforms fp32 [bs, T + 1]. Returns (accepted int32 [bs],
    out_tokens int32 [bs, T + 1] (kept prefix, the next token, then -1), accept_prob fp64 [bs, T]
    (min(1, p/q) per step in token mode, h_i in block mode))."""
    lb = _c(draft_lb, np.uint16)
    X = _c(draft_tokens, np.int32)
    tg = _c(target_logits, np.float32)
    tp = _c(temps, np.float32)
    un = _c(uniforms, np.float32)
    bs, T, V = lb.shape
    if X.shape != (bs, T) or tg.shape != (bs, T + 1, V) or tp.shape != (bs,) or \
            un.shape != (bs, T + 1):
        raise OracleError("verify: inconsistent shapes")
    acc = np.empty(bs, np.int32)
    out = np.empty((bs, T + 1), np.int32)
    prob = np.empty((bs, T), np.float64)
    st = lib().oracle_verify(_ptr(lb), _ptr(X), _ptr(tg), _ptr(tp), _ptr(un), bs, T, V, int(mode),
                             _ptr(acc), _ptr(out), _ptr(prob))
    if st != OK:
        raise OracleError(f"oracle_verify failed ({st})")
    return acc, out, prob


def w2_l1_bound(q, s) -> float:
    """max_v fl32(s[v] * sum_k |q[v,k]|): per unit of max |W1[prev]|, a bound on every row's
    bias (the lossless top-k pruning certificate; see oracle_w2_l1_bound in oracle.c)."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    V, R = q.shape
    return float(lib().oracle_w2_l1_bound(_ptr(q), _ptr(s), V, R))


def icdf_uniform(seed: int, P: int) -> float:
    """The inverse-CDF sampler's uniform for a request seed and draft position."""
    return float(lib().oracle_icdf_uniform(seed, P))


def icdf_draw(lb_row, temp: float, u: float) -> int:
    """Inverse-CDF draw from a stored bf16 row (uint16 bits) with uniform u (-1: invalid row)."""
    r = _c(lb_row, np.uint16)
    return int(lib().oracle_icdf_draw(_ptr(r), r.size, float(temp), float(u)))
