"""Seeded random shapes through every bf16 entry point, each against the
fp64 oracle element by element: many tile counts, ragged edges, head groups,
offsets and split plans that the hand-picked cases do not enumerate."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu

HEADS = [(8, 1), (16, 2), (12, 4), (64, 8), (5, 5), (24, 3), (32, 1), (48, 6)]


def _prefill_case(i):
    rng = np.random.default_rng(1000 + i)
    Hq, Hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    T = int(rng.integers(1, 400))
    causal = bool(rng.integers(2))
    S = int(rng.integers(T if causal else 1, T + 700))
    q_off = S - T if causal else 0
    if causal and rng.integers(2):      # causal chunk not at the bottom: fewer keys visible
        q_off = int(rng.integers(0, S - T + 1))
    return dict(B=B, T=T, S=S, Hq=Hq, Hkv=Hkv, d=d, causal=causal, q_off=q_off)


@pytest.mark.parametrize("i", range(24))
def test_random_prefill(i):
    import gqa_attention_flashattention_amd as gq
    import torch
    c = _prefill_case(i)
    inp = gin.random_case("prefill", "bf16", B=c["B"], H_q=c["Hq"], H_kv=c["Hkv"], d=c["d"],
                          T_q=c["T"], S_kv=c["S"], seed=2000 + i)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o, lse = gq.prefill(q, k, v, causal=c["causal"], q_offset=c["q_off"])
    torch.cuda.synchronize()
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=c["causal"], q_offset=c["q_off"])
    assert_close(to_f64(o), oref, to_f64(lse), lref, name=f"random prefill {c}")


@pytest.mark.parametrize("i", range(24))
def test_random_decode(i):
    """Plain (T_q = 1) and multi-token decode, automatic or fixed split counts
    (both the one-head and the two-head work-group layouts occur)."""
    import gqa_attention_flashattention_amd as gq
    import torch
    rng = np.random.default_rng(3000 + i)
    Hq, Hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 6))
    T_q = int(rng.choice([1, 1, 2, 3, 4, 8]))
    kv_len = rng.integers(T_q, 3000, size=B).tolist()
    num_splits = int(rng.choice([0, 0, 1, 2, 5, 17]))
    inp = gin.random_case("decode", "bf16", B=B, H_q=Hq, H_kv=Hkv, d=d, T_q=T_q, kv_len=kv_len,
                          seed=4000 + i)
    if inp.q.ndim == 3:                 # one token: an explicit T_q axis
        inp.q, inp.q_store = inp.q[:, None], inp.q_store[:, None]
    q = to_gpu(inp.q_store, "bf16")
    k = to_gpu(inp.k_store, "bf16")
    v = to_gpu(inp.v_store, "bf16")
    o, lse = gq.decode_multi(q, k, v, inp.kv_len, num_splits=num_splits)
    torch.cuda.synchronize()
    # oracle: per sequence, its T_q new tokens against its cache, causal with
    # the new tokens at the end (q_offset = len - T_q)
    oref = np.empty(inp.q.shape)
    lref = np.empty(inp.q.shape[:3])
    off = 0
    for b, n in enumerate(kv_len):
        ob, lb = oracle.prefill(inp.q[b:b + 1], inp.k[None, off:off + n], inp.v[None, off:off + n],
                                causal=True, q_offset=n - T_q)
        oref[b], lref[b] = ob[0], lb[0]
        off += n
    assert_close(to_f64(o), oref, to_f64(lse), lref,
                 name=f"random decode B={B} T_q={T_q} {Hq}/{Hkv} d={d} splits={num_splits}")


def _quant_oracle(inp, ring=None):
    """Per sequence against the dequantised cache; ring = (capacity, window,
    sink) unwraps a ring cache into the logical sequence (zeros where evicted)."""
    k = oracle.dequantize(inp.k_codes, inp.k_scale)
    v = oracle.dequantize(inp.v_codes, inp.v_scale)
    B, T_q, Hq, d = inp.q.shape
    oref = np.empty((B, T_q, Hq, d))
    lref = np.empty((B, T_q, Hq))
    off = 0
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()):
        if ring is None:
            ob, lb = oracle.prefill(inp.q[b:b + 1], k[None, off:off + n], v[None, off:off + n],
                                    causal=True, q_offset=n - T_q)
            off += n
        else:
            cap, window, sink = ring
            wrap = cap - sink
            pos = np.arange(n)
            keep = (pos < sink) | (pos >= n - wrap)
            slot = np.where(pos < sink, pos, sink + (pos - sink) % wrap)
            kl = np.zeros((n,) + k.shape[2:], np.float32)
            vl = np.zeros((n,) + v.shape[2:], np.float32)
            kl[keep] = k[b, slot[keep]]
            vl[keep] = v[b, slot[keep]]
            ob, lb = oracle.prefill_window(inp.q[b:b + 1], kl[None], vl[None], q_offset=n - T_q,
                                           window=window, sink=sink)
        oref[b], lref[b] = ob[0], lb[0]
    return oref, lref


@pytest.mark.parametrize("i", range(12))
def test_random_quant_decode(i):
    """INT8 / INT4 caches with the automatic split plan over assorted batches
    (the int4 plan searches split lengths against rounds of work-groups)."""
    import gqa_attention_flashattention_amd as gq
    import torch
    rng = np.random.default_rng(5000 + i)
    Hq, Hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    bits = int(rng.choice([8, 4]))
    B = int(rng.integers(1, 24))
    T_q = int(rng.choice([1, 1, 2, 4]))
    kv_len = rng.integers(T_q, 12000, size=B).tolist()
    inp = gin.quant_case(B=B, H_q=Hq, H_kv=Hkv, d=d, kv_len=kv_len, kv_bits=bits, T_q=T_q,
                         seed=6000 + i)
    pack = (lambda c: c) if bits == 8 else gin.pack_int4
    o, lse = gq.decode_quant(to_gpu(inp.q_store, "bf16"),
                             torch.from_numpy(pack(inp.k_codes)).cuda(),
                             torch.from_numpy(pack(inp.v_codes)).cuda(),
                             torch.from_numpy(inp.k_scale).cuda(),
                             torch.from_numpy(inp.v_scale).cuda(), kv_len, kv_bits=bits)
    torch.cuda.synchronize()
    oref, lref = _quant_oracle(inp)
    assert_close(to_f64(o), oref, to_f64(lse), lref,
                 name=f"random int{bits} decode B={B} T_q={T_q} {Hq}/{Hkv} d={d}")


@pytest.mark.parametrize("i", range(12))
def test_random_ring_quant_decode(i):
    """Quantised ring caches: random capacities, windows, sinks and token counts
    (wrapped and unwrapped), automatic split plan."""
    import gqa_attention_flashattention_amd as gq
    import torch
    rng = np.random.default_rng(7000 + i)
    Hq, Hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    bits = int(rng.choice([8, 4]))
    B = int(rng.integers(1, 20))
    T_q = int(rng.choice([1, 1, 2, 3]))
    sink = int(rng.integers(0, 8))
    cap = int(rng.integers(sink + T_q + 8, 3000))
    window = int(rng.integers(1, cap - sink - T_q + 2))
    kv_len = rng.integers(T_q, 3 * cap, size=B).tolist()
    inp = gin.quant_case(B=B, H_q=Hq, H_kv=Hkv, d=d, kv_len=kv_len, kv_bits=bits, T_q=T_q,
                         seed=8000 + i, capacity=cap)
    pack = (lambda c: c) if bits == 8 else gin.pack_int4
    o, lse = gq.decode_ring_quant(to_gpu(inp.q_store, "bf16"),
                                  torch.from_numpy(pack(inp.k_codes)).cuda(),
                                  torch.from_numpy(pack(inp.v_codes)).cuda(),
                                  torch.from_numpy(inp.k_scale).cuda(),
                                  torch.from_numpy(inp.v_scale).cuda(), kv_len, kv_bits=bits,
                                  window=window, sink=sink)
    torch.cuda.synchronize()
    oref, lref = _quant_oracle(inp, ring=(cap, window, sink))
    assert_close(to_f64(o), oref, to_f64(lse), lref,
                 name=f"random ring int{bits} B={B} T_q={T_q} cap={cap} w={window} s={sink}")
