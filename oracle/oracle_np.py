"""NumPy fp64 formulation of GQA attention -- TEST INFRASTRUCTURE ONLY.

An independent second statement of the definition the C oracle computes, in
matrix form: for each (sequence, query head) the whole score matrix
scale * Q K^T is formed, keys a query may not see are set to -inf (the
additive causal mask of the ADR-0060 page, sections 3 and 5.4, with the
diagonal included), and softmax(S) V and LSE = ln sum_j exp(S_j) follow.
The KV head of query head h is h // G (ADR-0060 TL;DR, section 5.2: the
G query heads of a KV head form one group).  Meant for small shapes only;
it materialises every score.
"""
from __future__ import annotations

import numpy as np


def _attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
            visible: np.ndarray | None):
    """q [T,d], k/v [S,d] (float64); visible [T,S] bool or None (all)."""
    s = scale * (q @ k.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    lsum = p.sum(axis=1, keepdims=True)
    o = (p @ v) / lsum
    lse = (m + np.log(lsum))[:, 0]
    return o, lse, p / lsum


def prefill(q, k, v, *, causal: bool, q_offset: int = 0, scale: float | None = None,
            return_probs: bool = False, window: int | None = None, sink: int = 0):
    """``window`` (causal only): additionally hide key j from the query at
    position p unless j < sink or j > p - window (the sink + local-window
    policy of the pccx page, section 4, hard-cap ring buffer)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, Hq, d = q.shape
    _, S, Hkv, _ = k.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    vis = None
    if causal:
        pos = q_offset + np.arange(T)[:, None]
        key = np.arange(S)[None, :]
        vis = key <= pos
        if window is not None:
            vis = vis & ((key < sink) | (key > pos - window))
    o = np.empty((B, T, Hq, d))
    lse = np.empty((B, T, Hq))
    probs = np.empty((B, Hq, T, S)) if return_probs else None
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            ob, lb, pb = _attend(q[b, :, h, :], k[b, :, kv, :], v[b, :, kv, :], scale, vis)
            o[b, :, h, :] = ob
            lse[b, :, h] = lb
            if return_probs:
                probs[b, h] = pb
    if return_probs:
        return o, lse, probs
    return o, lse


def decode(q, k, v, kv_len, *, scale: float | None = None):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    starts = np.concatenate([[0], np.cumsum(np.asarray(kv_len, np.int64))])
    o = np.empty((B, Hq, d))
    lse = np.empty((B, Hq))
    for b in range(B):
        ks = k[starts[b]:starts[b + 1]]
        vs = v[starts[b]:starts[b + 1]]
        for h in range(Hq):
            kv = h // G
            ob, lb, _ = _attend(q[b, h][None, :], ks[:, kv, :], vs[:, kv, :], scale, None)
            o[b, h] = ob[0]
            lse[b, h] = lb[0]
    return o, lse
