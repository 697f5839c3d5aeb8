"""Pins for the fp64 oracle: checks against facts fixed by mathematics, not by
the oracle's own formula.

Each ``pin_*`` function takes an object with ``prefill``/``decode`` methods
(the default oracle build, or a build with a planted mistake) and raises
AssertionError when the oracle disagrees with the pinned fact.  The facts:

* closed forms -- zero queries or identical keys give uniform weights, so O is
  a (causal, bottom-right aligned) running mean of V and LSE = s + ln(n);
  V constant per KV head gives O equal to that constant (head mapping
  h -> h // G of the ADR-0060 page, TL;DR and section 5.2); one key gives
  O = v_0; two keys give the logistic weight 1 / (1 + e^(s_1 - s_0));
* identity V exposes the probability row itself: it sums to one, is zero on
  keys the causal rule hides (key j visible iff j <= q_offset + t, section
  5.4 tile classes, diagonal included) and its ratios are e^(s_j - s_k);
* a 50-digit Decimal evaluation of the textbook softmax on tiny shapes;
* torch's scaled_dot_product_attention in float64 (a library routine), for
  multi-head attention and for GQA with its own enable_gqa head grouping;
* split invariance: the FlashDecoding form (per-split partials merged with the
  section 4 formula) equals the unsplit result for any split count;
* the sink + local-window mask: uniform weights over an explicitly built
  visible set, Decimal brute force, and its two limits (the causal mask, the
  diagonal alone).
Scores s_j are formed here with math.fsum over exactly representable products
(float32 x float32 fits in float64), i.e. correctly rounded dot products.
"""
from __future__ import annotations

import decimal
import math

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _randf32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _dot(a, b) -> float:
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max relative error {err:.3e} > {tol:.1e}"


def _pack(kv_len, H_kv, d, rng):
    n = int(np.sum(kv_len))
    return _randf32(rng, (n, H_kv, d)), _randf32(rng, (n, H_kv, d))


# ---------------------------------------------------------------------------
# closed forms


def pin_uniform_scores(lib):
    """Q = 0: every visible key has score 0, so O is the mean of the visible V
    rows and LSE = ln(#visible)."""
    rng = _rng(11)
    B, T, S, Hq, Hkv, d = 2, 7, 11, 6, 3, 5
    G = Hq // Hkv
    q = np.zeros((B, T, Hq, d), np.float32)
    k = _randf32(rng, (B, S, Hkv, d))
    v = _randf32(rng, (B, S, Hkv, d))
    for q_offset in (4, 0):
        Tq = T if q_offset else S      # q_offset = 0 with T = S: square causal
        qq = np.zeros((B, Tq, Hq, d), np.float32)
        o, lse = lib.prefill(qq, k, v, causal=True, q_offset=q_offset)
        csum = np.cumsum(v.astype(np.float64), axis=1)            # [B,S,Hkv,d]
        for t in range(Tq):
            n = q_offset + t + 1
            for h in range(Hq):
                _close(o[:, t, h, :], csum[:, n - 1, h // G, :] / n, what="causal mean")
                _close(lse[:, t, h], np.full(B, math.log(n)), what="causal LSE")
    o, lse = lib.prefill(q, k, v, causal=False)
    for h in range(Hq):
        _close(o[:, :, h, :], np.broadcast_to(v.astype(np.float64).mean(axis=1)[:, None, h // G, :],
                                              (B, T, d)), what="non-causal mean")
    _close(lse, np.full((B, T, Hq), math.log(S)), what="non-causal LSE")
    kv_len = np.array([5, 1, 9], np.int32)
    kd, vd = _pack(kv_len, Hkv, d, rng)
    qd = np.zeros((3, Hq, d), np.float32)
    o, lse = lib.decode(qd, kd, vd, kv_len)
    start = 0
    for b, n in enumerate(kv_len):
        for h in range(Hq):
            _close(o[b, h], vd[start:start + n, h // G, :].astype(np.float64).mean(axis=0),
                   what="decode mean")
            _close(lse[b, h], math.log(n), what="decode LSE")
        start += n


def pin_equal_keys(lib):
    """All keys of a KV head equal u_kv: score s = scale * q.u_kv for every key,
    O = mean of visible V, LSE = s + ln(#visible).  Pins the scale and the q.k
    contraction."""
    rng = _rng(12)
    B, T, S, Hq, Hkv, d = 1, 5, 9, 4, 2, 6
    G = Hq // Hkv
    scale = 0.37
    q = _randf32(rng, (B, T, Hq, d), 2.0)
    u = _randf32(rng, (Hkv, d), 2.0)
    k = np.broadcast_to(u[None, None], (B, S, Hkv, d)).copy()
    v = _randf32(rng, (B, S, Hkv, d))
    q_offset = 3
    o, lse = lib.prefill(q, k, v, causal=True, q_offset=q_offset, scale=scale)
    csum = np.cumsum(v.astype(np.float64), axis=1)
    for t in range(T):
        n = q_offset + t + 1
        for h in range(Hq):
            s = scale * _dot(q[0, t, h], u[h // G])
            _close(o[0, t, h], csum[0, n - 1, h // G] / n, what="equal-key mean")
            _close(lse[0, t, h], s + math.log(n), what="equal-key LSE")
    kv_len = np.array([4, 7], np.int32)
    kd = np.broadcast_to(u[None], (11, Hkv, d)).copy()
    vd = _randf32(rng, (11, Hkv, d))
    qd = _randf32(rng, (2, Hq, d), 2.0)
    o, lse = lib.decode(qd, kd, vd, kv_len, scale=scale)
    start = 0
    for b, n in enumerate(kv_len):
        for h in range(Hq):
            s = scale * _dot(qd[b, h], u[h // G])
            _close(o[b, h], vd[start:start + n, h // G].astype(np.float64).mean(axis=0),
                   what="decode equal-key mean")
            _close(lse[b, h], s + math.log(n), what="decode equal-key LSE")
        start += n


def pin_constant_v(lib):
    """V[:, :, kv, :] = c_kv (distinct per KV head): O = c_(h // G) exactly,
    for any Q and K -- no leakage across KV heads."""
    rng = _rng(13)
    B, T, S, Hq, Hkv, d = 2, 6, 8, 12, 3, 4
    G = Hq // Hkv
    q = _randf32(rng, (B, T, Hq, d))
    k = _randf32(rng, (B, S, Hkv, d))
    c = np.arange(1, Hkv * d + 1, dtype=np.float32).reshape(Hkv, d) * np.float32(0.25)
    v = np.broadcast_to(c[None, None], (B, S, Hkv, d)).copy()
    for causal, q_offset in ((True, 2), (False, 0)):
        o, _ = lib.prefill(q, k, v, causal=causal, q_offset=q_offset)
        for h in range(Hq):
            _close(o[:, :, h, :], np.broadcast_to(c[h // G], (B, T, d)), what="constant V")
    kv_len = np.array([3, 5], np.int32)
    kd = _randf32(rng, (8, Hkv, d))
    vd = np.broadcast_to(c[None], (8, Hkv, d)).copy()
    qd = _randf32(rng, (2, Hq, d))
    o, _ = lib.decode(qd, kd, vd, kv_len)
    for h in range(Hq):
        _close(o[:, h, :], np.broadcast_to(c[h // G], (2, d)), what="decode constant V")


def pin_one_and_two_keys(lib):
    """One visible key: O = v_0 and LSE = s_0.  Two keys: weights
    1/(1 + e^(s_1 - s_0)) and its complement, LSE = s_0 + ln(1 + e^(s_1 - s_0))."""
    rng = _rng(14)
    Hq, Hkv, d = 4, 2, 8
    G = Hq // Hkv
    q = _randf32(rng, (1, 1, Hq, d))
    k = _randf32(rng, (1, 5, Hkv, d))
    v = _randf32(rng, (1, 5, Hkv, d))
    scale = 0.5
    o, lse = lib.prefill(q, k, v, causal=True, q_offset=0, scale=scale)   # sees key 0 only
    for h in range(Hq):
        _close(o[0, 0, h], v[0, 0, h // G], what="one key O")
        _close(lse[0, 0, h], scale * _dot(q[0, 0, h], k[0, 0, h // G]), what="one key LSE")
    o, lse = lib.prefill(q, k, v, causal=True, q_offset=1, scale=scale)   # sees keys 0, 1
    for h in range(Hq):
        s0 = scale * _dot(q[0, 0, h], k[0, 0, h // G])
        s1 = scale * _dot(q[0, 0, h], k[0, 1, h // G])
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        _close(o[0, 0, h], p0 * v[0, 0, h // G].astype(np.float64)
               + (1.0 - p0) * v[0, 1, h // G].astype(np.float64), what="two keys O")
        _close(lse[0, 0, h], s0 + math.log1p(math.exp(s1 - s0)), what="two keys LSE")
    kv_len = np.array([1, 2], np.int32)
    kd = _randf32(rng, (3, Hkv, d))
    vd = _randf32(rng, (3, Hkv, d))
    qd = _randf32(rng, (2, Hq, d))
    o, lse = lib.decode(qd, kd, vd, kv_len, scale=scale)
    for h in range(Hq):
        kv = h // G
        _close(o[0, h], vd[0, kv], what="decode one key")
        _close(lse[0, h], scale * _dot(qd[0, h], kd[0, kv]), what="decode one key LSE")
        s0 = scale * _dot(qd[1, h], kd[1, kv])
        s1 = scale * _dot(qd[1, h], kd[2, kv])
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        _close(o[1, h], p0 * vd[1, kv].astype(np.float64) + (1 - p0) * vd[2, kv].astype(np.float64),
               what="decode two keys")


# ---------------------------------------------------------------------------
# brute force in 50-digit decimal arithmetic


def _dec_attend(qrow, keys, vals, scale):
    """Textbook softmax attention in Decimal: weights e^(s_j) / sum_k e^(s_k),
    no max subtraction; returns (O list, LSE)."""
    D = decimal.Decimal
    sc = D(repr(float(scale)))
    w = []
    for kr in keys:
        s = sum((D(float(a)) * D(float(b)) for a, b in zip(qrow, kr)), D(0)) * sc
        w.append(s.exp())
    tot = sum(w, D(0))
    o = [sum((wj * D(float(vr[x])) for wj, vr in zip(w, vals)), D(0)) / tot
         for x in range(len(vals[0]))]
    return [float(x) for x in o], float(tot.ln())


def pin_decimal_bruteforce(lib):
    rng = _rng(15)
    B, T, S, Hq, Hkv, d = 2, 4, 6, 6, 2, 3
    G = Hq // Hkv
    scale = 0.8
    q = _randf32(rng, (B, T, Hq, d), 1.5)
    k = _randf32(rng, (B, S, Hkv, d))
    v = _randf32(rng, (B, S, Hkv, d))
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        for causal, q_offset in ((True, 2), (False, 0)):
            o, lse = lib.prefill(q, k, v, causal=causal, q_offset=q_offset, scale=scale)
            for b in range(B):
                for t in range(T):
                    n = q_offset + t + 1 if causal else S
                    for h in range(Hq):
                        eo, el = _dec_attend(q[b, t, h], k[b, :n, h // G], v[b, :n, h // G], scale)
                        _close(o[b, t, h], eo, what="decimal O")
                        _close(lse[b, t, h], el, what="decimal LSE")
        kv_len = np.array([3, 1, 6], np.int32)
        kd, vd = _pack(kv_len, Hkv, d, rng)
        qd = _randf32(rng, (3, Hq, d), 1.5)
        o, lse = lib.decode(qd, kd, vd, kv_len, scale=scale)
        start = 0
        for b, n in enumerate(kv_len):
            for h in range(Hq):
                eo, el = _dec_attend(qd[b, h], kd[start:start + n, h // G],
                                     vd[start:start + n, h // G], scale)
                _close(o[b, h], eo, what="decimal decode O")
                _close(lse[b, h], el, what="decimal decode LSE")
            start += n


# ---------------------------------------------------------------------------
# library routine: torch scaled_dot_product_attention in float64


def pin_torch_sdpa(lib):
    import torch
    import torch.nn.functional as F
    rng = _rng(16)
    B, T, Hq, d = 2, 9, 8, 16
    for Hkv in (8, 2):          # G = 1 (multi-head attention), G = 4
        q = _randf32(rng, (B, T, Hq, d))
        k = _randf32(rng, (B, T, Hkv, d))
        v = _randf32(rng, (B, T, Hkv, d))
        tq, tk, tv = (torch.from_numpy(x.astype(np.float64)).transpose(1, 2) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                             enable_gqa=Hkv != Hq).transpose(1, 2).numpy()
        o, _ = lib.prefill(q, k, v, causal=True, q_offset=0)
        _close(o, ref, what=f"sdpa causal Hkv={Hkv}")
        ref = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=Hkv != Hq)
        o, _ = lib.prefill(q, k, v, causal=False)
        _close(o, ref.transpose(1, 2).numpy(), what=f"sdpa full Hkv={Hkv}")
    # chunk of T queries at q_offset against S = q_offset + T keys (bottom-right)
    S, q_offset, Hkv = 13, 4, 2
    q = _randf32(rng, (B, T, Hq, d))
    k = _randf32(rng, (B, S, Hkv, d))
    v = _randf32(rng, (B, S, Hkv, d))
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)).transpose(1, 2) for x in (q, k, v))
    mask = torch.ones(T, S, dtype=torch.bool).tril(diagonal=q_offset)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True)
    o, lse = lib.prefill(q, k, v, causal=True, q_offset=q_offset)
    _close(o, ref.transpose(1, 2).numpy(), what="sdpa chunk")
    scores = torch.matmul(tq, tk.repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2).contiguous())
    scores = scores / math.sqrt(d)
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    _close(lse, ref_lse.transpose(1, 2).numpy(), what="logsumexp chunk")


# ---------------------------------------------------------------------------
# the probability row itself


def pin_identity_v(lib):
    """V rows are unit vectors e_j (d >= S): O[t] is the probability row P[t]."""
    rng = _rng(17)
    B, T, S, Hq, Hkv = 1, 6, 10, 4, 2
    d = 12
    G = Hq // Hkv
    q_offset = 4
    q = _randf32(rng, (B, T, Hq, d), 2.0)
    k = _randf32(rng, (B, S, Hkv, d))
    v = np.zeros((B, S, Hkv, d), np.float32)
    for j in range(S):
        v[0, j, :, j] = 1.0
    o, _ = lib.prefill(q, k, v, causal=True, q_offset=q_offset)
    for t in range(T):
        n = q_offset + t + 1
        for h in range(Hq):
            p = o[0, t, h]
            assert abs(math.fsum(p) - 1.0) <= TOL, "probability row does not sum to 1"
            assert np.all(p >= 0.0), "negative probability"
            assert np.all(p[n:] == 0.0), "weight on a key the causal rule hides"
            s = [_dot(q[0, t, h], k[0, j, h // G]) / math.sqrt(d) for j in range(n)]
            for j in range(1, n):
                _close(p[j] / p[0], math.exp(s[j] - s[0]), what="probability ratio")


def pin_moving_max(lib):
    """K_j = alpha * (j / S) * u, Q = u: scores rise along j in closed form
    s_j = scale * alpha * (j / S) * |u|^2; O and LSE equal scipy's softmax and
    logsumexp of those scores."""
    from scipy.special import logsumexp, softmax
    rng = _rng(18)
    S, d, alpha = 40, 8, 3.0
    u = np.full(d, 0.5, np.float32)
    k = np.stack([u * np.float32(alpha * j / S) for j in range(S)]).astype(np.float32)
    k = k[None, :, None, :]
    v = _randf32(rng, (1, S, 1, d))
    q = u[None, None, None, :]
    scale = 1.0 / math.sqrt(d)
    s = np.array([scale * _dot(u, k[0, j, 0]) for j in range(S)])
    o, lse = lib.prefill(q, k, v, causal=True, q_offset=S - 1)
    _close(o[0, 0, 0], softmax(s) @ v[0, :, 0].astype(np.float64), what="moving max O")
    _close(lse[0, 0, 0], logsumexp(s), what="moving max LSE")


def pin_large_scores(lib):
    """Score gaps of hundreds (far beyond exp's float64 range): the weight of
    every key but the top one underflows to exactly 0 relative to it, so O is
    the top key's V row and LSE its score.  Catches a softmax that does not
    subtract the true row maximum."""
    d = 4
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0] = 40.0
    c = np.array([0.0, 20.0, 10.0, 19.0], np.float32)        # scores 0, 800, 400, 760
    k = np.zeros((1, 4, 1, d), np.float32)
    k[0, :, 0, 0] = c
    v = np.arange(16, dtype=np.float32).reshape(1, 4, 1, d)
    o, lse = lib.prefill(q, k, v, causal=False, scale=1.0)
    _close(o[0, 0, 0], v[0, 1, 0], what="large-score O")
    _close(lse[0, 0, 0], 800.0, what="large-score LSE")
    o, lse = lib.decode(q[0], k[:, :, 0, :].reshape(4, 1, d), v.reshape(4, 1, d),
                        np.array([4], np.int32), scale=1.0)
    _close(o[0, 0], v[0, 1, 0], what="large-score decode O")
    _close(lse[0, 0], 800.0, what="large-score decode LSE")
    o, lse = lib.decode(q[0], k[:, :, 0, :].reshape(4, 1, d), v.reshape(4, 1, d),
                        np.array([4], np.int32), scale=1.0, num_splits=4)
    _close(o[0, 0], v[0, 1, 0], what="large-score split O")
    _close(lse[0, 0], 800.0, what="large-score split LSE")


# ---------------------------------------------------------------------------
# FlashDecoding split form


def pin_split_invariance(lib):
    rng = _rng(19)
    Hq, Hkv, d = 8, 2, 16
    kv_len = np.array([37, 1, 64], np.int32)
    kd, vd = _pack(kv_len, Hkv, d, rng)
    qd = _randf32(rng, (3, Hq, d), 2.0)
    o0, l0 = lib.decode(qd, kd, vd, kv_len)
    for ns in (1, 2, 3, 7, 64, int(kv_len.max())):
        o, lse = lib.decode(qd, kd, vd, kv_len, num_splits=ns)
        _close(o, o0, what=f"split O ns={ns}")
        _close(lse, l0, what=f"split LSE ns={ns}")


# ---------------------------------------------------------------------------
# sink + local-window mask (pccx page, section 4, hard-cap ring buffer policy)
#
# The visible set of a query at position p is built here as an explicit union
# of two integer ranges -- the first `sink` positions and the `window` newest
# positions up to p -- not through the oracle's per-key predicate.


def _window_set(p, window, sink):
    return sorted(set(range(min(sink, p + 1))) | set(range(max(0, p - window + 1), p + 1)))


def pin_window_uniform(lib):
    """Q = 0: uniform weights over the visible set, so O is the mean of V over
    exactly those positions and LSE = ln(count)."""
    rng = _rng(20)
    Hq, Hkv, d = 4, 2, 8
    G = Hq // Hkv
    S = 40
    k = _randf32(rng, (1, S, Hkv, d))
    v = _randf32(rng, (1, S, Hkv, d))
    for T, q_offset, window, sink in ((8, 32, 5, 3), (12, 0, 4, 2), (6, 30, 1, 0), (6, 30, 1, 4),
                                      (10, 20, 64, 0), (7, 10, 3, 30), (9, 31, 8, 8)):
        q = np.zeros((1, T, Hq, d), np.float32)
        o, lse = lib.prefill_window(q, k[:, :q_offset + T], v[:, :q_offset + T],
                                    q_offset=q_offset, window=window, sink=sink)
        for t in range(T):
            vis = _window_set(q_offset + t, window, sink)
            for h in range(Hq):
                mean = np.array([math.fsum(float(v[0, j, h // G, x]) for j in vis) / len(vis)
                                 for x in range(d)])
                _close(o[0, t, h], mean, what=f"window mean w={window} s={sink}")
                _close(lse[0, t, h], math.log(len(vis)), what=f"window LSE w={window} s={sink}")


def pin_window_decimal(lib):
    """Random queries on tiny shapes: 50-digit textbook softmax over the
    explicit visible set."""
    rng = _rng(21)
    B, T, S, Hq, Hkv, d = 2, 5, 9, 4, 2, 3
    G = Hq // Hkv
    q = _randf32(rng, (B, T, Hq, d), 1.5)
    k = _randf32(rng, (B, S, Hkv, d))
    v = _randf32(rng, (B, S, Hkv, d))
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        for window, sink in ((2, 1), (3, 0), (1, 2), (4, 3)):
            o, lse = lib.prefill_window(q, k, v, q_offset=S - T, window=window, sink=sink,
                                        scale=0.7)
            for b in range(B):
                for t in range(T):
                    vis = _window_set(S - T + t, window, sink)
                    for h in range(Hq):
                        eo, el = _dec_attend(q[b, t, h], k[b, vis, h // G], v[b, vis, h // G],
                                             0.7)
                        _close(o[b, t, h], eo, what="window decimal O")
                        _close(lse[b, t, h], el, what="window decimal LSE")


def pin_window_limits(lib):
    """A window covering every earlier key is the causal mask; a window of one
    with no sink sees only the diagonal: O = v_p, LSE = s_pp."""
    rng = _rng(22)
    Hq, Hkv, d = 6, 3, 8
    G = Hq // Hkv
    q = _randf32(rng, (2, 7, Hq, d))
    k = _randf32(rng, (2, 19, Hkv, d))
    v = _randf32(rng, (2, 19, Hkv, d))
    oc, lc = lib.prefill(q, k, v, causal=True, q_offset=12)
    for window, sink in ((19, 0), (1000, 5), (19, 19)):
        o, lse = lib.prefill_window(q, k, v, q_offset=12, window=window, sink=sink)
        _close(o, oc, what="window = causal O")
        _close(lse, lc, what="window = causal LSE")
    o, lse = lib.prefill_window(q, k, v, q_offset=12, window=1, sink=0, scale=0.3)
    for b in range(2):
        for t in range(7):
            for h in range(Hq):
                _close(o[b, t, h], v[b, 12 + t, h // G], what="diagonal-only O")
                _close(lse[b, t, h], 0.3 * _dot(q[b, t, h], k[b, 12 + t, h // G]),
                       what="diagonal-only LSE")


ALL_PINS = [pin_uniform_scores, pin_equal_keys, pin_constant_v, pin_one_and_two_keys,
            pin_decimal_bruteforce, pin_torch_sdpa, pin_identity_v, pin_moving_max,
            pin_large_scores, pin_split_invariance, pin_window_uniform, pin_window_decimal,
            pin_window_limits]
