"""Hand-built structured inputs shared by the oracle pins and the GPU parity tests.

These build inputs only (no walk arithmetic): the two-step worked example of
``golden/hand_walk_v4.json`` and the token-feedback cycle, both derived from the step definition
of vLLM PR #62958 (int8 DSpark Markov walk), Overview.
"""
import json
import os

import numpy as np

RANK = 256
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def hand_walk_v4():
    """Inputs and expected outputs of the hand-worked 4-entry, 2-step walk."""
    with open(os.path.join(GOLDEN, "hand_walk_v4.json")) as f:
        g = json.load(f)
    V = g["V"]
    c = [1.0, -2.0, 3.0, -4.0]
    w2 = np.zeros((V, RANK), np.float32)
    w1 = np.zeros((V, RANK), np.float32)
    for v in range(V):
        w2[v, (v - 1) % V] = 15.875
        w2[v, 4] = 0.125 * c[v]
        w1[v, v] = 1.984375
        w1[v, 4] = 0.5
    base = np.asarray(g["base"], np.float32)[None]          # [1, 2, 4]
    start = np.asarray([g["start"]], np.int32)
    return dict(w1=w1, w2=w2, base=base, start=start, golden=g)


def feedback_cycle(V=251, T=16, start=7, seed=5):
    """W1[i, i] = 127/64 and W2[v, (v-1) mod V] = 15.875 make the bias of prev p equal to
    15.875 * 127/64 = 31.501953125 at v = p + 1 (mod V) and 0 elsewhere; with base ~ N(0, 1)
    the walk must emit start+1, start+2, ... (mod V)."""
    assert V <= RANK
    w2 = np.zeros((V, RANK), np.float32)
    w1 = np.zeros((V, RANK), np.float32)
    for v in range(V):
        w2[v, (v - 1) % V] = 15.875
        w1[v, v] = 1.984375
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((1, T, V)).astype(np.float32)
    expected = np.asarray([(start + 1 + t) % V for t in range(T)], np.int32)
    return dict(w1=w1, w2=w2, base=base, start=np.asarray([start], np.int32), expected=expected)
