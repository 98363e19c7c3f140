"""Top-k softmax router -- the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The router sits above the library's boundary: it produces the ``topk_ids`` the
slot manager consumes and the gate weights the MoE layer takes as an input.  What
it computes for one token x with gate matrix Wg [E, H]:

    logits = Wg @ x                       (E values)
    p      = softmax(logits)              over all E experts
    ids    = the K experts of largest p, in descending order of p; equal p go to
             the lower expert id ("Running 125B MoE on Two 32 GB Cards", section
             4.2: on a tie of two logits the lower id wins)
    w      = p[ids]                       (gathered, not renormalised)

Everything is float64.  ``gate_weights`` gives w for ids chosen elsewhere (a
routing trace): the same softmax, gathered at those ids.
"""
from __future__ import annotations

import numpy as np


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, in float64 (shifted by the row maximum)."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def probabilities(Wg: np.ndarray, x: np.ndarray) -> np.ndarray:
    """p[T, E] = softmax(x @ Wg^T) for activations x[T, H] and gate Wg[E, H]."""
    Wg = np.asarray(Wg, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return softmax(x @ Wg.T)


def top_k(p: np.ndarray, k: int) -> np.ndarray:
    """ids[T, k]: per row the k largest entries of p, largest first, equal values
    taken in ascending id order."""
    p = np.atleast_2d(np.asarray(p, dtype=np.float64))
    T, E = p.shape
    if not 1 <= k <= E:
        raise ValueError(f"k={k} outside [1, {E}]")
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # a stable sort on -p keeps equal values in ascending id order
        order = np.argsort(-p[t], kind="stable")
        out[t] = order[:k]
    return out


def route(Wg: np.ndarray, x: np.ndarray, k: int):
    """(ids[T, k] int32, w[T, k] float64) for activations x[T, H]."""
    p = probabilities(Wg, x)
    ids = top_k(p, k)
    return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)


def gate_weights(Wg: np.ndarray, x: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[T, K] = softmax(x @ Wg^T)[ids] for ids chosen by a routing trace."""
    p = probabilities(Wg, x)
    return np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
