"""GPU parity of the split-KV decode path (C ABI gqa_attn_decode and the
split/combine pair) against the fp64 oracle, element by element."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _dev(inp):
    return tuple(to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))


def _decode(inp, num_splits=0):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = _dev(inp)
    o = gq.decode(q, k, v, inp.kv_len, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o)


def _decode_with_lse(inp, num_splits=0):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = _dev(inp)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    nbytes = gq.decode_workspace_bytes(B, Hq, Hkv, d, inp.kv_len, num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gq.decode_split(q, k, v, inp.kv_len, ws, num_splits=num_splits)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    gq.decode_combine(ws, inp.kv_len, H_q=Hq, H_kv=Hkv, d=d, out=o, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("kv_len,Hq,Hkv,d", [
    ([1, 2, 31, 32, 33, 63, 64, 65, 1000], 64, 8, 128),
    ([1, 2, 31, 32, 33, 130, 4097], 64, 8, 64),
    ([77, 300, 5], 12, 4, 128),          # G = 3
    ([129, 17], 32, 1, 128),             # G = 32: two 16-head groups
    ([250], 20, 1, 64),                  # G = 20: partial second head group
    ([513, 1], 8, 8, 128),               # G = 1
    ([300, 1, 65], 64, 1, 128),          # G = 64: four column blocks per KV head
    ([77, 5000], 48, 1, 64),             # G = 48, d = 64
])
def test_decode_parity(kv_len, Hq, Hkv, d):
    inp = gin.random_case("decode", "bf16", B=len(kv_len), H_q=Hq, H_kv=Hkv, d=d, kv_len=kv_len,
                          seed=sum(kv_len))
    og = _decode(inp)
    oref, _ = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(og, oref, name=f"decode {kv_len} {Hq}/{Hkv} d={d}")


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 64, 1000])
def test_split_count_invariance(num_splits):
    kv_len = [1000, 1, 257]
    inp = gin.random_case("decode", "bf16", B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, seed=2)
    og, lg = _decode_with_lse(inp, num_splits)
    oref, lref = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(og, oref, lg, lref, name=f"decode splits={num_splits}")
    o1, l1 = _decode_with_lse(inp, 1)
    assert np.abs(og - o1).max() <= 1e-2 and np.abs(lg - l1).max() <= 1e-3


def test_many_sequences_two_launches():
    """More sequences than one launch describes (64): chunked launches."""
    rng = np.random.default_rng(3)
    kv_len = rng.integers(1, 300, size=70).tolist()
    inp = gin.random_case("decode", "bf16", B=70, H_q=16, H_kv=2, d=128, kv_len=kv_len, seed=6)
    og, lg = _decode_with_lse(inp)
    oref, lref = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(og, oref, lg, lref, name="decode B=70")


def test_uniform_scores_mean_of_v():
    kv_len = [5, 700, 64]
    inp = gin.random_case("decode", "bf16", B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, seed=8)
    inp.q_store[...] = 0
    inp.q[...] = 0
    og, lg = _decode_with_lse(inp)
    oref, lref = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert np.abs(lref - np.log(np.array(kv_len))[:, None]).max() < 1e-12
    assert_close(og, oref, lg, lref, name="decode uniform")


def test_peaky_decode():
    inp = gin.random_case("decode", "bf16", B=2, H_q=64, H_kv=8, d=128, kv_len=[3000, 70], seed=9,
                          q_scale=8.0)
    og, lg = _decode_with_lse(inp)
    oref, lref = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(og, oref, lg, lref, name="decode peaky")


def test_decode_deterministic():
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("decode", "bf16", B=2, H_q=64, H_kv=8, d=128, kv_len=[5000, 333], seed=10)
    q, k, v = _dev(inp)
    o1 = gq.decode(q, k, v, inp.kv_len)
    o2 = gq.decode(q, k, v, inp.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("kv_len,Hq,Hkv,d,num_splits", [
    ([600, 1000, 513], 64, 8, 128, 1),     # every split >= 512 keys: two KV heads per work-group
    ([2049, 512], 16, 2, 128, 1),          # ragged last tiles, one head pair
    ([700, 1500], 32, 4, 64, 1),           # d = 64
    ([900, 3000], 24, 6, 128, 1),          # three head pairs, G = 4
    ([777, 1200], 24, 3, 128, 1),          # odd H_kv: one head per work-group
    ([100, 5000], 64, 8, 128, 1),          # one short split: one head per work-group
])
def test_head_pair_work_groups(kv_len, Hq, Hkv, d, num_splits):
    """Long splits take two KV heads per work-group (waves 0/2 and 1/3);
    every output and LSE against the oracle, and equal to the one-head layout
    of the same plan within rounding."""
    inp = gin.random_case("decode", "bf16", B=len(kv_len), H_q=Hq, H_kv=Hkv, d=d, kv_len=kv_len,
                          seed=sum(kv_len) + Hkv)
    og, lg = _decode_with_lse(inp, num_splits)
    oref, lref = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(og, oref, lg, lref, name=f"decode head pairs {kv_len} {Hq}/{Hkv} d={d}")


@pytest.mark.parametrize("name", ["decode_8k", "decode_varlen_b16", "decode_128k"])
def test_full_size_workloads(name):
    """Full-size decode workloads in the benchmark's launch configuration,
    every output element against the oracle."""
    inp = gin.make(name)
    og, lg = _decode_with_lse(inp)
    oref, lref = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(og, oref, lg, lref, name=name)
    og2 = _decode(inp)
    assert np.array_equal(og2, og)


# ---- multi-token decode: T_q new tokens per sequence, causal among them ----

def _as_multi(inp):
    """Decode inputs with one token per sequence get an explicit T_q = 1 axis."""
    if inp.q.ndim == 3:
        inp.q = inp.q[:, None]
        inp.q_store = inp.q_store[:, None]
    return inp


def _subset(inp, sel):
    """The sequences `sel` of a packed decode case (q rows and their K/V rows)."""
    import dataclasses
    kv_len = np.asarray(inp.kv_len, np.int64)
    off = np.concatenate([[0], np.cumsum(kv_len)])
    k = np.concatenate([inp.k[off[b]:off[b + 1]] for b in sel])
    v = np.concatenate([inp.v[off[b]:off[b + 1]] for b in sel])
    return dataclasses.replace(inp, q=inp.q[sel], k=k, v=v, q_store=inp.q_store[sel],
                               k_store=None, v_store=None,
                               kv_len=np.asarray(inp.kv_len)[sel])


def _oracle_multi(inp):
    """Per sequence: the oracle prefill of its T_q new tokens against its
    cache, causal with the new tokens at the end (q_offset = len - T_q)."""
    B, T_q, Hq, d = inp.q.shape
    o = np.empty((B, T_q, Hq, d))
    lse = np.empty((B, T_q, Hq))
    off = 0
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()):
        ob, lb = oracle.prefill(inp.q[b:b + 1], inp.k[None, off:off + n], inp.v[None, off:off + n],
                                causal=True, q_offset=n - T_q)
        o[b], lse[b] = ob[0], lb[0]
        off += n
    return o, lse


def _decode_multi(inp, num_splits=0):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = _dev(inp)
    o, lse = gq.decode_multi(q, k, v, inp.kv_len, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("T_q,kv_len,Hq,Hkv,d", [
    (1, [1, 33, 700], 64, 8, 128),
    (2, [2, 3, 64, 65, 1000], 64, 8, 128),
    (3, [3, 31, 130], 64, 8, 64),        # G * T_q = 24: partial second column block
    (4, [4, 5, 4097], 64, 8, 128),
    (8, [8, 9, 40, 513], 64, 8, 128),
    (16, [16, 17, 333], 64, 8, 128),      # G * T_q = 128: eight column blocks
    (5, [77, 300, 5], 12, 4, 128),        # G = 3, odd T_q
    (2, [250, 40], 20, 1, 64),            # G = 20
    (7, [129, 7], 8, 8, 128),             # G = 1
    (16, [16, 300, 2000], 64, 8, 64),     # 128 rows, d = 64
    (32, [32, 33, 700], 64, 8, 128),      # 256 rows: two work-groups per KV head
    (3, [3, 100, 4097], 96, 8, 128),      # G = 12, 36 rows: three column blocks
])
def test_decode_multi_parity(T_q, kv_len, Hq, Hkv, d):
    inp = _as_multi(gin.random_case("decode", "bf16", B=len(kv_len), H_q=Hq, H_kv=Hkv, d=d,
                                    T_q=T_q, kv_len=kv_len, seed=T_q * 1000 + sum(kv_len)))
    og, lg = _decode_multi(inp)
    oref, lref = _oracle_multi(inp)
    assert_close(og, oref, lg, lref, name=f"decode_multi T_q={T_q} {kv_len} {Hq}/{Hkv} d={d}")


@pytest.mark.parametrize("T_q,kv_len,num_splits", [
    (4, [600, 2000], 1),                   # two KV heads per work-group, T_q * G = 32
    (2, [1024, 513, 4000], 1),
])
def test_decode_multi_head_pairs(T_q, kv_len, num_splits):
    inp = _as_multi(gin.random_case("decode", "bf16", B=len(kv_len), H_q=64, H_kv=8, d=128,
                                    T_q=T_q, kv_len=kv_len, seed=31 + T_q))
    og, lg = _decode_multi(inp, num_splits)
    oref, lref = _oracle_multi(inp)
    assert_close(og, oref, lg, lref, name=f"decode_multi head pairs T_q={T_q}")


@pytest.mark.parametrize("num_splits", [1, 3, 1000])
def test_decode_multi_split_counts(num_splits):
    """Splits that end inside the new tokens' causal band (some splits are
    wholly in the future for the earlier new tokens)."""
    kv_len = [1000, 9, 257]
    inp = gin.random_case("decode", "bf16", B=3, H_q=64, H_kv=8, d=128, T_q=8, kv_len=kv_len,
                          seed=21)
    og, lg = _decode_multi(inp, num_splits)
    oref, lref = _oracle_multi(inp)
    assert_close(og, oref, lg, lref, name=f"decode_multi splits={num_splits}")


@pytest.mark.parametrize("T_q,kv_len,Hq,Hkv,d,num_splits", [
    (64, [64, 65, 1000], 64, 8, 128, 0),      # 512 rows: two row blocks of 256
    (16, [1000, 16, 257], 64, 8, 128, 1),     # one split: ranges of any length
    (16, [1000, 16, 257], 64, 8, 128, 7),     # splits ending inside the causal band
    (16, [200, 17], 64, 8, 128, 1000),        # one-key splits
    (43, [43, 44, 600], 12, 4, 128, 0),       # G = 3, 129 rows: one live row in the last wave
    (7, [7, 300, 1500], 140, 7, 64, 5),       # G = 20, 140 rows, d = 64
    (128, [128, 129], 16, 8, 128, 3),         # G = 2, 256 rows
    (8, [8, 600, 2000], 48, 3, 128, 0),       # 128 rows, odd H_kv: one head per work-group
    (4, [4, 999], 64, 2, 128, 3),             # 128 rows, G = 32: one pair of heads
])
def test_decode_multi_rows_path(T_q, kv_len, Hq, Hkv, d, num_splits):
    """From 128 query rows per KV head, decode runs the prefill tile loop on
    each split's key range: row blocks, ranges of any length and start,
    ranges wholly in the future of some new tokens, two KV heads per
    work-group at 128 rows (one with an odd number of heads)."""
    inp = _as_multi(gin.random_case("decode", "bf16", B=len(kv_len), H_q=Hq, H_kv=Hkv, d=d,
                                    T_q=T_q, kv_len=kv_len, seed=T_q * 77 + sum(kv_len)))
    og, lg = _decode_multi(inp, num_splits)
    oref, lref = _oracle_multi(inp)
    assert_close(og, oref, lg, lref,
                 name=f"decode_multi rows T_q={T_q} {kv_len} {Hq}/{Hkv} d={d} ns={num_splits}")


@pytest.mark.parametrize("name", ["decode_t16_varlen_b16", "decode_t32_varlen_b16"])
def test_decode_multi_wide_full_size(name):
    """16 ragged sequences of 1k-32k keys with 16 / 32 new tokens: three whole
    sequences (first, middle, last) against the oracle."""
    inp = gin.make(name)
    og, lg = _decode_multi(inp)
    sel = [0, 7, 15]
    sub = _subset(inp, sel)
    oref, lref = _oracle_multi(sub)
    assert_close(og[sel], oref, lg[sel], lref, name=name)


def test_decode_multi_one_token_matches_decode():
    """T_q = 1 is plain decode: same kernels, bitwise equal outputs."""
    import gqa_attention_flashattention_amd as gq
    import torch
    kv_len = [300, 4000, 1]
    inp = gin.random_case("decode", "bf16", B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, seed=22)
    q, k, v = _dev(inp)
    o1 = gq.decode(q, k, v, inp.kv_len)
    om, _ = gq.decode_multi(q[:, None], k, v, inp.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(o1, om[:, 0])


def test_decode_multi_full_size():
    """The multi-token decode workload (16 ragged sequences, 4 new tokens),
    every output element against the oracle."""
    inp = gin.make("decode_t4_varlen_b16")
    og, lg = _decode_multi(inp)
    oref, lref = _oracle_multi(inp)
    assert_close(og, oref, lg, lref, name="decode_t4_varlen_b16")


def test_binding_rejects_mismatched_buffers():
    """Caller-given outputs of the wrong shape/dtype and mixed-dtype inputs are
    refused on the host, before anything is launched."""
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("decode", "bf16", B=2, H_q=16, H_kv=2, d=128, kv_len=[40, 9], seed=60)
    q, k, v = _dev(inp)
    with pytest.raises(gq.GQAError):
        gq.decode(q, k, v, inp.kv_len, out=torch.empty(2, 16, 64, dtype=torch.bfloat16,
                                                      device="cuda"))
    with pytest.raises(gq.GQAError):
        gq.decode(q, k.float(), v, inp.kv_len)
    with pytest.raises(gq.GQAError):
        gq.decode_multi(q[:, None], k, v, inp.kv_len,
                        lse=torch.empty(2, 1, 8, dtype=torch.float32, device="cuda"))
    with pytest.raises(gq.GQAError):
        gq.decode_combine(torch.empty(1 << 20, dtype=torch.uint8, device="cuda"), inp.kv_len,
                          H_q=16, H_kv=2, d=128,
                          out=torch.empty(2, 8, 128, dtype=torch.bfloat16, device="cuda"))
    qp = torch.zeros(1, 4, 16, 128, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gq.GQAError):
        gq.prefill(qp, kp, kp, causal=True, q_offset=4,
                   out=torch.empty(1, 4, 16, 128, dtype=torch.float32, device="cuda"))


def test_decode_multi_deterministic_and_many_sequences():
    import gqa_attention_flashattention_amd as gq
    import torch
    rng = np.random.default_rng(64)
    kv_len = rng.integers(8, 500, size=70).tolist()
    inp = gin.random_case("decode", "bf16", B=70, H_q=64, H_kv=8, d=128, T_q=8, kv_len=kv_len,
                          seed=64)
    q, k, v = _dev(inp)
    o1, l1 = gq.decode_multi(q, k, v, inp.kv_len)
    o2, l2 = gq.decode_multi(q, k, v, inp.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    oref, lref = _oracle_multi(inp)
    assert_close(to_f64(o1), oref, to_f64(l1), lref, name="decode_multi B=70 T_q=8")
