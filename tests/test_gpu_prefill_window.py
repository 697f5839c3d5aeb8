"""GPU parity of the sink + local-window prefill (C ABI gqa_attn_prefill_window)
against the fp64 oracle, element by element."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _run(inp, q_offset, window, sink):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o, lse = gq.prefill_window(q, k, v, q_offset=q_offset, window=window, sink=sink)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("B,T,S,Hq,Hkv,d,q_offset,window,sink", [
    (1, 300, 300, 16, 2, 128, 0, 64, 4),        # tile-aligned window, sinks in tile 0
    (1, 700, 700, 16, 2, 128, 0, 100, 0),       # no sink: first tiles fully hidden for some rows
    (1, 700, 700, 16, 2, 128, 0, 37, 70),       # sinks spanning two tiles, skipped gap
    (1, 100, 1457, 16, 2, 128, 1357, 200, 3),   # chunk at an offset, gap of many tiles
    (2, 77, 903, 12, 4, 64, 826, 129, 1),       # G = 3, d = 64
    (2, 65, 650, 5, 5, 128, 585, 1, 0),         # window of one: the diagonal alone
    (1, 513, 2000, 64, 8, 128, 1487, 256, 16),  # Llama3-70B heads
    (1, 200, 260, 8, 1, 64, 60, 5000, 0),       # window wider than the sequence: causal
    (1, 129, 129, 8, 2, 128, 0, 1, 200),        # every key a sink: causal
])
def test_window_parity(B, T, S, Hq, Hkv, d, q_offset, window, sink):
    inp = gin.random_case("prefill", "bf16", B=B, H_q=Hq, H_kv=Hkv, d=d, T_q=T, S_kv=S,
                          seed=T + S + window + sink)
    og, lg = _run(inp, q_offset, window, sink)
    oref, lref = oracle.prefill_window(inp.q, inp.k, inp.v, q_offset=q_offset, window=window,
                                       sink=sink)
    assert_close(og, oref, lg, lref, name=f"window {B},{T},{S},{Hq},{Hkv},{d} w={window} s={sink}")


def test_wide_window_equals_causal_prefill():
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("prefill", "bf16", B=1, H_q=64, H_kv=8, d=128, T_q=300, S_kv=800,
                          seed=41)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o1, l1 = gq.prefill(q, k, v, causal=True, q_offset=500)
    o2, l2 = gq.prefill_window(q, k, v, q_offset=500, window=801, sink=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_window_uniform_scores():
    """Q = 0: O is the mean of V over the sinks and the window."""
    inp = gin.random_case("prefill", "bf16", B=1, H_q=16, H_kv=2, d=128, T_q=400, S_kv=400,
                          seed=42)
    inp.q_store[...] = 0
    inp.q[...] = 0
    og, lg = _run(inp, 0, 70, 5)
    oref, lref = oracle.prefill_window(inp.q, inp.k, inp.v, q_offset=0, window=70, sink=5)
    cnt = np.array([min(5, p + 1) + max(0, p - max(5, p - 69) + 1) for p in range(400)])
    assert np.abs(lref - np.log(cnt)[None, :, None]).max() < 1e-12
    assert_close(og, oref, lg, lref, name="window uniform")


def test_full_size_window_sampled():
    """8k tokens, window 1024 with 4 sinks, Llama3-70B heads: sampled rows."""
    inp = gin.make("prefill_8k_window1k")
    w = inp.workload
    og, lg = _run(inp, w.q_offset, w.window, w.sink)
    rng = np.random.default_rng(7)
    total = w.B * w.T_q * w.H_q
    rows = np.unique(np.concatenate([[0, 1, w.H_q - 1, 1030 * w.H_q, total // 2, total - 1],
                                     rng.integers(0, total, 250)]))
    rows = np.union1d(rows, gin.rows_per_workgroup(w.B, w.T_q, w.H_q, w.H_kv, seed=8))
    oref, lref = oracle.prefill_window(inp.q, inp.k, inp.v, q_offset=w.q_offset, window=w.window,
                                       sink=w.sink, rows=rows)
    assert_close(og.reshape(-1, w.d)[rows], oref, lg.reshape(-1)[rows], lref,
                 name="prefill_8k_window1k")


# ---- KV-parallel form (gqa_attn_prefill_window_kvsplit) ----

def _run_split(inp, q_offset, window, sink, num_splits):
    import gqa_attention_flashattention_amd as gq
    import torch
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o, lse = gq.prefill_window(q, k, v, q_offset=q_offset, window=window, sink=sink,
                               kv_split=True, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("B,T,S,Hq,Hkv,d,q_offset,window,sink,num_splits", [
    (1, 100, 1457, 16, 2, 128, 1357, 200, 3, 0),       # automatic range count
    (1, 100, 1457, 16, 2, 128, 1357, 200, 3, 3),       # sink tile + window tiles in 3 ranges
    (1, 64, 5000, 64, 8, 128, 4936, 3000, 4, 0),       # short chunk under a long window
    (2, 77, 903, 12, 4, 64, 826, 129, 1, 5),           # G = 3, d = 64
    (1, 300, 300, 16, 2, 128, 0, 64, 4, 2),            # ranges with rows that see none of them
    (1, 200, 260, 8, 1, 64, 60, 5000, 0, 4),           # window wider than the sequence
    (1, 129, 129, 8, 2, 128, 0, 1, 200, 3),            # every key a sink
])
def test_window_kvsplit_parity(B, T, S, Hq, Hkv, d, q_offset, window, sink, num_splits):
    inp = gin.random_case("prefill", "bf16", B=B, H_q=Hq, H_kv=Hkv, d=d, T_q=T, S_kv=S,
                          seed=T + S + window + sink + 7)
    og, lg = _run_split(inp, q_offset, window, sink, num_splits)
    oref, lref = oracle.prefill_window(inp.q, inp.k, inp.v, q_offset=q_offset, window=window,
                                       sink=sink)
    assert_close(og, oref, lg, lref,
                 name=f"window kvsplit {B},{T},{S},{Hq},{Hkv},{d} w={window} s={sink} n={num_splits}")


def test_window_kvsplit_one_range_equals_window_prefill():
    """One range is the plain window kernel: bitwise equal outputs."""
    inp = gin.random_case("prefill", "bf16", B=1, H_q=64, H_kv=8, d=128, T_q=256, S_kv=3000,
                          seed=43)
    o1, l1 = _run(inp, 2744, 1000, 4)
    o2, l2 = _run_split(inp, 2744, 1000, 4, 1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
