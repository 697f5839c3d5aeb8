"""GPU parity of decode over a hard-cap ring-buffer cache with attention sinks
and a local window (C ABI gqa_attn_decode_ring) against the fp64 oracle.

The GPU gets a random ring cache; the oracle gets the logical (unwrapped)
sequence that cache stands for, rebuilt here from the ring rule -- the first
`sink` positions in slots 0.., position j >= sink in slot
sink + (j - sink) mod (capacity - sink) -- with zeros at positions no longer
resident (the validity rule guarantees no new token sees them).  Slots never
written hold 300.0, so a stray read would show."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu

UNUSED = 300.0


def _ring_inputs(B, T_q, Hq, Hkv, d, cap, kv_len, seed):
    """Random q and ring caches (bf16 values as float32 + storage bits)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T_q, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, cap, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, cap, Hkv, d), dtype=np.float32)
    for b, n in enumerate(kv_len):
        k[b, n:] = UNUSED
        v[b, n:] = UNUSED
    bits = [gin.bf16_round_bits(x) for x in (q, k, v)]
    vals = [gin.bf16_bits_to_f32(x) for x in bits]
    return vals, bits


def _logical(cache_b, n, cap, sink):
    """The unwrapped sequence [n, H_kv, d] a ring cache holds (zeros where evicted)."""
    wrap = cap - sink
    out = np.zeros((n,) + cache_b.shape[1:], np.float32)
    for j in range(n):
        if j < sink:
            out[j] = cache_b[j]
        elif j >= n - wrap:
            out[j] = cache_b[sink + (j - sink) % wrap]
    return out


def _oracle_ring(vals, kv_len, cap, window, sink, rows_per_seq=None):
    q, k, v = vals
    B, T_q, Hq, d = q.shape
    o = np.empty((B, T_q, Hq, d))
    lse = np.empty((B, T_q, Hq))
    for b, n in enumerate(kv_len):
        kl = _logical(k[b], n, cap, sink)[None]
        vl = _logical(v[b], n, cap, sink)[None]
        ob, lb = oracle.prefill_window(q[b:b + 1], kl, vl, q_offset=n - T_q, window=window,
                                       sink=sink)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def _gpu_ring(bits, kv_len, window, sink, num_splits=0):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = (to_gpu(x, "bf16") for x in bits)
    o, lse = gq.decode_ring(q, k, v, kv_len, window=window, sink=sink, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("T_q,Hq,Hkv,d,cap,window,sink,kv_len", [
    (1, 16, 2, 128, 64, 60, 4, [1, 3, 4, 5, 63, 64, 65, 200, 1000]),   # ring = window
    (1, 16, 2, 128, 300, 100, 2, [50, 250, 299, 300, 301, 1000]),      # window inside the ring
    (4, 64, 8, 128, 128, 121, 4, [4, 6, 130, 500]),                    # widest window for T_q = 4
    (3, 16, 2, 128, 100, 98, 0, [3, 99, 100, 101, 777]),               # no sinks
    (2, 12, 4, 64, 70, 20, 1, [2, 25, 69, 70, 71, 400]),               # G = 3, d = 64
    (8, 64, 8, 128, 4096, 2048, 4, [8, 3000, 9000]),
    (5, 8, 8, 128, 40, 30, 6, [5, 7, 10, 41, 1234]),                   # G = 1, sinks > T_q
])
def test_ring_decode_parity(T_q, Hq, Hkv, d, cap, window, sink, kv_len):
    vals, bits = _ring_inputs(len(kv_len), T_q, Hq, Hkv, d, cap, kv_len, seed=cap + sum(kv_len))
    og, lg = _gpu_ring(bits, kv_len, window, sink)
    oref, lref = _oracle_ring(vals, kv_len, cap, window, sink)
    assert_close(og, oref, lg, lref, name=f"ring T_q={T_q} cap={cap} w={window} s={sink}")


def test_ring_head_pairs():
    """Long ring splits (>= 512 resident keys each) take two KV heads per work-group."""
    kv_len = [5000, 1300]
    vals, bits = _ring_inputs(2, 1, 64, 8, 128, 2048, kv_len, seed=52)
    og, lg = _gpu_ring(bits, kv_len, 1500, 4, 1)
    oref, lref = _oracle_ring(vals, kv_len, 2048, 1500, 4)
    assert_close(og, oref, lg, lref, name="ring head pairs")


@pytest.mark.parametrize("num_splits", [1, 3, 100])
def test_ring_decode_split_counts(num_splits):
    kv_len = [700, 40, 2500]
    vals, bits = _ring_inputs(3, 2, 64, 8, 128, 512, kv_len, seed=51)
    og, lg = _gpu_ring(bits, kv_len, 300, 4, num_splits)
    oref, lref = _oracle_ring(vals, kv_len, 512, 300, 4)
    assert_close(og, oref, lg, lref, name=f"ring splits={num_splits}")


def test_unwrapped_ring_equals_decode():
    """Before the ring wraps, with a window covering everything, ring decode
    is plain decode over the first kv_len slots (same keys, same plan)."""
    import gqa_attention_flashattention_amd as gq
    import torch
    kv_len = [100, 37, 256]
    vals, bits = _ring_inputs(3, 1, 64, 8, 128, 256, kv_len, seed=52)
    q, k, v = (to_gpu(x, "bf16") for x in bits)
    o1, _ = gq.decode_ring(q, k, v, kv_len, window=252, sink=4)
    packed_k = torch.cat([k[b, :n] for b, n in enumerate(kv_len)])
    packed_v = torch.cat([v[b, :n] for b, n in enumerate(kv_len)])
    o2 = gq.decode(q[:, 0].contiguous(), packed_k, packed_v, kv_len)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2)


def test_full_size_ring_workload():
    """16 sequences of 1k-32k tokens through an 8192-slot ring (4 sinks):
    every output row against the oracle."""
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.make("decode_ring_8k_b16")
    w = inp.workload
    kv_len = inp.kv_len
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o, lse = gq.decode_ring(q, k, v, kv_len, window=w.window, sink=w.sink)
    torch.cuda.synchronize()
    oref, lref = _oracle_ring((inp.q, inp.k, inp.v), kv_len.tolist(), w.capacity,
                              w.window, w.sink)
    assert_close(to_f64(o), oref, to_f64(lse), lref, name="decode_ring_8k_b16")


def test_ring_deterministic_and_many_sequences():
    """70 sequences (two launches), twice: bitwise identical, and against the oracle."""
    import gqa_attention_flashattention_amd as gq
    import torch
    rng = np.random.default_rng(63)
    kv_len = rng.integers(3, 700, size=70).tolist()
    vals, bits = _ring_inputs(70, 3, 16, 2, 128, 256, kv_len, seed=63)
    q, k, v = (to_gpu(x, "bf16") for x in bits)
    o1, l1 = gq.decode_ring(q, k, v, kv_len, window=200, sink=4)
    o2, l2 = gq.decode_ring(q, k, v, kv_len, window=200, sink=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    oref, lref = _oracle_ring(vals, kv_len, 256, 200, 4)
    assert_close(to_f64(o1), oref, to_f64(l1), lref, name="ring B=70")
