"""GPU parity of decode over a quantised (INT8 / INT4, per-channel scales)
hard-cap ring-buffer cache with attention sinks and a local window (C ABI
gqa_attn_decode_ring_quant) against the fp64 oracle.

The oracle sees the dequantised cache (codes x scales) unwrapped into the
logical sequence by the ring rule -- the first `sink` positions in slots
0.., position j >= sink in slot sink + (j - sink) mod (capacity - sink) --
with zeros at positions no longer resident (the validity rule guarantees no
new token sees them), and runs the sink + window oracle on it."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu
from test_gpu_decode_quant import scales_16bit

pytestmark = pytest.mark.gpu


def _logical(cache_b, n, cap, sink):
    """The unwrapped sequence [n, H_kv, d] a ring cache holds (zeros where evicted)."""
    wrap = cap - sink
    out = np.zeros((n,) + cache_b.shape[1:], np.float64)
    for j in range(n):
        if j < sink:
            out[j] = cache_b[j]
        elif j >= n - wrap:
            out[j] = cache_b[sink + (j - sink) % wrap]
    return out


def _oracle(inp, cap, window, sink, seqs=None):
    k = oracle.dequantize(inp.k_codes, inp.k_scale)     # [B, cap, H_kv, d]
    v = oracle.dequantize(inp.v_codes, inp.v_scale)
    B, T_q, Hq, d = inp.q.shape
    o = np.full((B, T_q, Hq, d), np.nan)
    lse = np.full((B, T_q, Hq), np.nan)
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()):
        if seqs is not None and b not in seqs:
            continue
        kl = _logical(k[b], n, cap, sink)[None]
        vl = _logical(v[b], n, cap, sink)[None]
        ob, lb = oracle.prefill_window(inp.q[b:b + 1], kl, vl, q_offset=n - T_q, window=window,
                                       sink=sink)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def _gpu(inp, window, sink, num_splits=0):
    import gqa_attention_flashattention_amd as gq
    import torch
    w = inp.workload
    pack = (lambda c: c) if w.kv_bits == 8 else gin.pack_int4
    kc = torch.from_numpy(pack(inp.k_codes)).cuda()
    vc = torch.from_numpy(pack(inp.v_codes)).cuda()
    ks = torch.from_numpy(inp.k_scale).cuda()
    vs = torch.from_numpy(inp.v_scale).cuda()
    q = to_gpu(inp.q_store, "bf16")
    o, lse = gq.decode_ring_quant(q, kc, vc, ks, vs, inp.kv_len, kv_bits=w.kv_bits,
                                  window=window, sink=sink, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T_q,Hq,Hkv,d,cap,window,sink,kv_len", [
    (1, 16, 2, 128, 64, 60, 4, [1, 3, 4, 5, 63, 64, 65, 200, 1000]),   # ring = window
    (1, 16, 2, 128, 300, 100, 2, [50, 250, 299, 300, 301, 1000]),      # window inside the ring
    (4, 64, 8, 128, 128, 121, 4, [4, 6, 130, 500]),                    # widest window for T_q = 4
    (3, 16, 2, 64, 100, 98, 0, [3, 99, 100, 101, 777]),                # no sinks, d = 64
    (2, 12, 4, 128, 70, 20, 1, [2, 25, 69, 70, 71, 400]),              # G = 3
    (5, 8, 8, 128, 40, 30, 6, [5, 7, 10, 41, 1234]),                   # G = 1, sinks > T_q
])
def test_ring_quant_parity(bits, T_q, Hq, Hkv, d, cap, window, sink, kv_len):
    inp = gin.quant_case(B=len(kv_len), H_q=Hq, H_kv=Hkv, d=d, kv_len=kv_len, kv_bits=bits,
                         T_q=T_q, seed=cap + bits + sum(kv_len), capacity=cap)
    og, lg = _gpu(inp, window, sink)
    oref, lref = _oracle(inp, cap, window, sink)
    assert_close(og, oref, lg, lref, name=f"ring int{bits} T_q={T_q} cap={cap} w={window}")


@pytest.mark.parametrize("num_splits", [1, 3, 100])
def test_ring_quant_split_counts(num_splits):
    kv_len = [700, 40, 2500]
    inp = gin.quant_case(B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, kv_bits=4, T_q=2, seed=71,
                         capacity=512)
    og, lg = _gpu(inp, 300, 4, num_splits)
    oref, lref = _oracle(inp, 512, 300, 4)
    assert_close(og, oref, lg, lref, name=f"ring int4 splits={num_splits}")


@pytest.mark.parametrize("bits", [8, 4])
def test_unwrapped_ring_quant_equals_quant_decode(bits):
    """Before the ring wraps, with a window covering everything, the quantised
    ring decode is the packed quantised decode over the first kv_len slots
    (same keys, same plan): bitwise equal."""
    import gqa_attention_flashattention_amd as gq
    import torch
    kv_len = [100, 37, 256]
    inp = gin.quant_case(B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, kv_bits=bits, T_q=1,
                         seed=72 + bits, capacity=256)
    pack = (lambda c: c) if bits == 8 else gin.pack_int4
    kc = torch.from_numpy(pack(inp.k_codes)).cuda()
    vc = torch.from_numpy(pack(inp.v_codes)).cuda()
    ks = torch.from_numpy(inp.k_scale).cuda()
    vs = torch.from_numpy(inp.v_scale).cuda()
    q = to_gpu(inp.q_store, "bf16")
    o1, l1 = gq.decode_ring_quant(q, kc, vc, ks, vs, kv_len, kv_bits=bits, window=252, sink=4)
    kp = torch.cat([kc[b, :n] for b, n in enumerate(kv_len)]).contiguous()
    vp = torch.cat([vc[b, :n] for b, n in enumerate(kv_len)]).contiguous()
    o2, l2 = gq.decode_quant(q, kp, vp, ks, vs, kv_len, kv_bits=bits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_full_size_ring_int4_workload():
    """The pccx base configuration: 16 sequences of 1k-32k tokens through an
    8192-slot INT4 ring (4 sinks); whole sequences against the oracle."""
    inp = gin.make_quant("decode_ring_int4_b16")
    w = inp.workload
    og, lg = _gpu(inp, w.window, w.sink)
    seqs = [0, 1, 7, 15]
    oref, lref = _oracle(inp, w.capacity, w.window, w.sink, seqs=seqs)
    assert_close(og[seqs], oref[seqs], lg[seqs], lref[seqs], name="decode_ring_int4_b16")


def test_ring_quant_deterministic_and_many_sequences():
    """70 sequences (two launches), twice: bitwise identical, and against the oracle."""
    rng = np.random.default_rng(73)
    kv_len = rng.integers(3, 700, size=70).tolist()
    inp = gin.quant_case(B=70, H_q=16, H_kv=2, d=128, kv_len=kv_len, kv_bits=8, T_q=3, seed=73,
                         capacity=256)
    og1, lg1 = _gpu(inp, 200, 4)
    og2, lg2 = _gpu(inp, 200, 4)
    assert np.array_equal(og1, og2) and np.array_equal(lg1, lg2)
    oref, lref = _oracle(inp, 256, 200, 4)
    assert_close(og1, oref, lg1, lref, name="ring int8 B=70")


@pytest.mark.parametrize("bits", [8, 4])
def test_ring_quant_fp32_scales(bits):
    """Per-channel fp32 scales that are not bf16 values (16 significant bits)
    against the fp64 oracle on those exact scales."""
    rng = np.random.default_rng(90 + bits)
    kv_len = [3, 300, 1000]
    inp = gin.quant_case(B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, kv_bits=bits, T_q=2,
                         seed=91 + bits, capacity=256)
    inp.k_scale = scales_16bit(inp.k_scale, rng)
    inp.v_scale = scales_16bit(inp.v_scale, rng)
    og, lg = _gpu(inp, 200, 4)
    oref, lref = _oracle(inp, 256, 200, 4)
    assert_close(og, oref, lg, lref, name=f"ring int{bits} fp32 scales")
