"""GPU parity of the KV-parallel prefill (C ABI gqa_attn_prefill_kvsplit:
key ranges on separate work-groups, merged by log-sum-exp) against the fp64
oracle, element by element."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _dev(inp):
    return tuple(to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))


def _run(inp, causal, q_offset, num_splits):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = _dev(inp)
    o, lse = gq.prefill_kvsplit(q, k, v, causal=causal, q_offset=q_offset, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("B,T,S,Hq,Hkv,d,causal,q_offset,ns", [
    (1, 300, 300, 16, 2, 128, True, 0, 3),       # diagonal inside the splits, ragged
    (1, 300, 300, 16, 2, 128, True, 0, 64),      # more ranges than tiles: empty ranges
    (1, 100, 1457, 16, 2, 128, True, 1357, 5),   # chunk at an offset
    (2, 77, 203, 12, 4, 64, False, 0, 2),        # non-causal, G = 3, d = 64
    (2, 65, 650, 5, 5, 128, True, 585, 4),       # G = 1
    (3, 1, 1300, 8, 2, 128, True, 1299, 7),      # one query token
    (1, 513, 2000, 64, 8, 128, True, 1487, 0),   # automatic range count
    (1, 256, 4352, 64, 8, 128, True, 4096, 0),
])
def test_kvsplit_parity(B, T, S, Hq, Hkv, d, causal, q_offset, ns):
    inp = gin.random_case("prefill", "bf16", B=B, H_q=Hq, H_kv=Hkv, d=d, T_q=T, S_kv=S,
                          seed=T + S + ns)
    og, lg = _run(inp, causal, q_offset, ns)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=causal, q_offset=q_offset)
    assert_close(og, oref, lg, lref, name=f"kvsplit {B},{T},{S},{Hq},{Hkv},{d} ns={ns}")


def test_range_count_invariance():
    """Every range count gives the oracle's result, within rounding of each other."""
    inp = gin.random_case("prefill", "bf16", B=1, H_q=16, H_kv=2, d=128, T_q=200, S_kv=1224,
                          seed=31)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True, q_offset=1024)
    outs = []
    for ns in [1, 2, 3, 8, 19]:
        og, lg = _run(inp, True, 1024, ns)
        assert_close(og, oref, lg, lref, name=f"kvsplit ns={ns}")
        outs.append((og, lg))
    for og, lg in outs[1:]:
        assert np.abs(og - outs[0][0]).max() <= 1e-2 and np.abs(lg - outs[0][1]).max() <= 1e-3


def test_one_range_is_plain_prefill():
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("prefill", "bf16", B=1, H_q=64, H_kv=8, d=128, T_q=130, S_kv=900,
                          seed=32)
    q, k, v = _dev(inp)
    o1, l1 = gq.prefill(q, k, v, causal=True, q_offset=770)
    o2, l2 = gq.prefill_kvsplit(q, k, v, causal=True, q_offset=770, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_kvsplit_deterministic():
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("prefill", "bf16", B=1, H_q=64, H_kv=8, d=128, T_q=64, S_kv=3000,
                          seed=33)
    q, k, v = _dev(inp)
    o1, l1 = gq.prefill_kvsplit(q, k, v, causal=True, q_offset=2936, num_splits=6)
    o2, l2 = gq.prefill_kvsplit(q, k, v, causal=True, q_offset=2936, num_splits=6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_full_size_chunk_over_long_cache():
    """A 256-token chunk over a 64k cache (64 row-block work-groups without the
    split): the automatic range count, every output row of a sample of query
    heads and tokens against the oracle."""
    import gqa_attention_flashattention_amd as gq
    inp = gin.make("prefill_chunk_256_64k")
    w = inp.workload
    assert gq.prefill_kvsplit_count(w.B, w.T_q, w.S_kv, w.H_q, w.H_kv, w.d, causal=True,
                                    q_offset=w.q_offset) > 1
    og, lg = _run(inp, True, w.q_offset, 0)
    rng = np.random.default_rng(7)
    total = w.B * w.T_q * w.H_q
    rows = np.unique(np.concatenate([[0, 1, w.H_q - 1, total // 2, total - 1],
                                     rng.integers(0, total, 250)]))
    rows = np.union1d(rows, gin.rows_per_workgroup(w.B, w.T_q, w.H_q, w.H_kv, seed=8))
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True, q_offset=w.q_offset, rows=rows)
    assert_close(og.reshape(-1, w.d)[rows], oref, lg.reshape(-1)[rows], lref,
                 name="prefill_chunk_256_64k kvsplit")


@pytest.mark.parametrize("window", [0, 90])
def test_kvsplit_many_batch_entries(window):
    """70 batch entries: the combine runs in two launches of at most 64
    sequences; plain causal and sink + window, every element against the oracle."""
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("prefill", "bf16", B=70, H_q=16, H_kv=2, d=64, T_q=9, S_kv=400,
                          seed=77 + window)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    if window:
        o, lse = gq.prefill_window(q, k, v, q_offset=391, window=window, sink=3, kv_split=True,
                                   num_splits=4)
        oref, lref = oracle.prefill_window(inp.q, inp.k, inp.v, q_offset=391, window=window,
                                           sink=3)
    else:
        o, lse = gq.prefill_kvsplit(q, k, v, causal=True, q_offset=391, num_splits=4)
        oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True, q_offset=391)
    torch.cuda.synchronize()
    assert_close(to_f64(o), oref, to_f64(lse), lref, name=f"kvsplit B=70 window={window}")
