"""GPU parity of decode over an INT8 / INT4 quantised KV cache with
per-channel scales (C ABI gqa_attn_decode_quant) against the fp64 oracle run
on the dequantised values, element by element."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _gpu(inp, num_splits=0):
    import gqa_attention_flashattention_amd as gq
    import torch
    w = inp.workload
    q = to_gpu(inp.q_store, "bf16")
    if w.kv_bits == 8:
        kc = torch.from_numpy(inp.k_codes).cuda()
        vc = torch.from_numpy(inp.v_codes).cuda()
    else:
        kc = torch.from_numpy(gin.pack_int4(inp.k_codes)).cuda()
        vc = torch.from_numpy(gin.pack_int4(inp.v_codes)).cuda()
    ks = torch.from_numpy(inp.k_scale).cuda()
    vs = torch.from_numpy(inp.v_scale).cuda()
    o, lse = gq.decode_quant(q, kc, vc, ks, vs, inp.kv_len, kv_bits=w.kv_bits,
                             num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def _oracle(inp, seqs=None):
    """Per sequence: the oracle over the dequantised cache, the T_q new tokens
    causal at the end."""
    w = inp.workload
    k = oracle.dequantize(inp.k_codes, inp.k_scale)
    v = oracle.dequantize(inp.v_codes, inp.v_scale)
    B, T_q, Hq, d = inp.q.shape
    o = np.full((B, T_q, Hq, d), np.nan)
    lse = np.full((B, T_q, Hq), np.nan)
    off = 0
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()):
        if seqs is None or b in seqs:
            ob, lb = oracle.prefill(inp.q[b:b + 1], k[None, off:off + n], v[None, off:off + n],
                                    causal=True, q_offset=n - T_q)
            o[b], lse[b] = ob[0], lb[0]
        off += n
    return o, lse


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T_q,kv_len,Hq,Hkv,d", [
    (1, [1, 2, 31, 32, 33, 1000], 64, 8, 128),
    (1, [5, 130, 4097], 64, 8, 64),
    (1, [77, 300], 12, 4, 128),          # G = 3
    (4, [4, 9, 700], 64, 8, 128),        # multi-token, two column blocks
    (3, [3, 250], 20, 1, 64),            # G = 20
    (2, [513, 2], 8, 8, 128),            # G = 1
    (1, [50, 700], 6, 3, 128),           # odd H_kv
    (2, [2, 333, 1500], 32, 8, 128),     # G = 4, two new tokens: 8 rows per KV head
])
def test_quant_decode_parity(bits, T_q, kv_len, Hq, Hkv, d):
    inp = gin.quant_case(B=len(kv_len), H_q=Hq, H_kv=Hkv, d=d, kv_len=kv_len, kv_bits=bits,
                         T_q=T_q, seed=bits * 100 + sum(kv_len))
    og, lg = _gpu(inp)
    oref, lref = _oracle(inp)
    assert_close(og, oref, lg, lref, name=f"int{bits} T_q={T_q} {kv_len} {Hq}/{Hkv} d={d}")


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_extreme_codes(bits):
    """Codes at both ends of the range and large scales (sharp softmax)."""
    inp = gin.quant_case(B=2, H_q=64, H_kv=8, d=128, kv_len=[300, 64], kv_bits=bits, seed=7)
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    inp.k_codes[::3] = hi
    inp.k_codes[1::3] = lo
    inp.v_codes[::2] = lo
    inp.k_scale *= 4
    og, lg = _gpu(inp)
    oref, lref = _oracle(inp)
    assert_close(og, oref, lg, lref, name=f"int{bits} extreme")


@pytest.mark.parametrize("num_splits", [1, 5, 1000])
def test_quant_split_counts(num_splits):
    inp = gin.quant_case(B=2, H_q=64, H_kv=8, d=128, kv_len=[1500, 33], kv_bits=4, seed=8)
    og, lg = _gpu(inp, num_splits)
    oref, lref = _oracle(inp)
    assert_close(og, oref, lg, lref, name=f"int4 splits={num_splits}")


@pytest.mark.parametrize("name", ["decode_int8_varlen_b16", "decode_int4_varlen_b16"])
def test_quant_full_size(name):
    """16 ragged sequences of 1k-32k keys: three whole sequences (first,
    middle, last) against the oracle."""
    inp = gin.make_quant(name)
    og, lg = _gpu(inp)
    seqs = {0, 7, 15}
    oref, lref = _oracle(inp, seqs)
    sel = sorted(seqs)
    assert_close(og[sel], oref[sel], lg[sel], lref[sel], name=name)


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_deterministic(bits):
    """The same call twice gives bitwise identical outputs."""
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.quant_case(B=3, H_q=64, H_kv=8, d=128, kv_len=[3000, 17, 900], kv_bits=bits,
                         T_q=2, seed=61)
    pack = (lambda c: c) if bits == 8 else gin.pack_int4
    q = to_gpu(inp.q_store, "bf16")
    kc = torch.from_numpy(pack(inp.k_codes)).cuda()
    vc = torch.from_numpy(pack(inp.v_codes)).cuda()
    ks = torch.from_numpy(inp.k_scale).cuda()
    vs = torch.from_numpy(inp.v_scale).cuda()
    o1, l1 = gq.decode_quant(q, kc, vc, ks, vs, inp.kv_len, kv_bits=bits)
    o2, l2 = gq.decode_quant(q, kc, vc, ks, vs, inp.kv_len, kv_bits=bits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_quant_many_sequences_two_launches():
    """More sequences than one launch describes (64)."""
    rng = np.random.default_rng(62)
    kv_len = rng.integers(1, 400, size=70).tolist()
    inp = gin.quant_case(B=70, H_q=16, H_kv=2, d=128, kv_len=kv_len, kv_bits=4, seed=62)
    og, lg = _gpu(inp)
    oref, lref = _oracle(inp)
    assert_close(og, oref, lg, lref, name="int4 B=70")


def scales_16bit(scale, rng):
    """fp32 scales with 16 significant bits that are not bf16 values: a
    random perturbation kept to the top 16 bits of the significand, with
    some of bits 8-15 set.  code * scale (at most 8 + 16 bits) is still
    exact in float32, so the oracle runs on the exact dequantised cache,
    while a kernel that rounded a scale to bf16 would drop its low part."""
    s = np.asarray(scale, np.float64) * (1.0 + rng.uniform(2.0**-8, 2.0**-7, size=scale.shape))
    u = s.astype(np.float32).view(np.uint32) & np.uint32(0xFFFFFF00)
    u |= np.uint32(0x100)          # bit 8 set: never a bf16 value
    out = u.view(np.float32)
    assert not np.any(gin.bf16_bits_to_f32(gin.bf16_round_bits(out)) == out)
    return out


def _full_fp32_scales(inp, seed):
    rng = np.random.default_rng(seed)
    inp.k_scale = scales_16bit(inp.k_scale, rng)
    inp.v_scale = scales_16bit(inp.v_scale, rng)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T_q,kv_len", [(1, [1, 40, 2000]), (4, [9, 700])])
def test_quant_fp32_scales(bits, T_q, kv_len):
    """Scales that bf16 cannot hold: K's is folded into Q as a bf16 high and
    low pair and V's multiplies the fp32 partial, so both stay within the
    bf16 parity gate of the fp64 oracle on the exact fp32 scales."""
    inp = gin.quant_case(B=len(kv_len), H_q=64, H_kv=8, d=128, kv_len=kv_len, kv_bits=bits,
                         T_q=T_q, seed=500 + bits + T_q)
    _full_fp32_scales(inp, 501 + bits)
    og, lg = _gpu(inp)
    oref, lref = _oracle(inp)
    assert_close(og, oref, lg, lref, name=f"int{bits} fp32 scales T_q={T_q}")
