"""Entry points captured into a HIP graph (torch.cuda.CUDAGraph over the
binding's calls on the capture stream) and replayed: every replay must
rewrite every output element with exactly the eager call's bits, with eager
work and synchronisations between the replays (the outputs are filled with
NaN before each one).  The benchmark times the calls this way.  The eager
call comes first so that the library-owned workspace is already large
enough: a call that would grow it cannot be captured."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_matches_eager(call, outs):
    import torch
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager call"
    del g
    return eager


def test_graph_decode():
    import gqa_attention_flashattention_amd as gq
    import torch
    kv_len = [8192, 1, 700]
    inp = gin.random_case("decode", "bf16", B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, seed=81)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o = torch.empty_like(q)
    (oe,) = _replay_matches_eager(lambda: gq.decode(q, k, v, inp.kv_len, out=o), [o])
    oref, _ = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
    assert_close(to_f64(oe), oref, name="graph decode")


def test_graph_prefill_causal():
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("prefill", "bf16", B=1, H_q=16, H_kv=2, d=128, T_q=333, S_kv=333,
                          seed=82)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    oe, le = _replay_matches_eager(lambda: gq.prefill(q, k, v, causal=True, out=o, lse=lse),
                                   [o, lse])
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True)
    assert_close(to_f64(oe), oref, to_f64(le), lref, name="graph prefill")


def test_graph_prefill_kvsplit():
    """Split kernel and combine kernel, library-owned partials."""
    import gqa_attention_flashattention_amd as gq
    import torch
    T, S = 200, 2000
    inp = gin.random_case("prefill", "bf16", B=1, H_q=16, H_kv=2, d=128, T_q=T, S_kv=S, seed=83)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    oe, le = _replay_matches_eager(
        lambda: gq.prefill_kvsplit(q, k, v, causal=True, q_offset=S - T, num_splits=5, out=o,
                                   lse=lse), [o, lse])
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True, q_offset=S - T)
    assert_close(to_f64(oe), oref, to_f64(le), lref, name="graph prefill kvsplit")


def test_graph_decode_ring_int4():
    import gqa_attention_flashattention_amd as gq
    import torch
    kv_len, cap, window, sink = [700, 40, 2500], 512, 300, 4
    inp = gin.quant_case(B=3, H_q=64, H_kv=8, d=128, kv_len=kv_len, kv_bits=4, T_q=2, seed=84,
                         capacity=cap)
    kc = torch.from_numpy(gin.pack_int4(inp.k_codes)).cuda()
    vc = torch.from_numpy(gin.pack_int4(inp.v_codes)).cuda()
    ks = torch.from_numpy(inp.k_scale).cuda()
    vs = torch.from_numpy(inp.v_scale).cuda()
    q = to_gpu(inp.q_store, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    _replay_matches_eager(
        lambda: gq.decode_ring_quant(q, kc, vc, ks, vs, inp.kv_len, kv_bits=4, window=window,
                                     sink=sink, out=o, lse=lse), [o, lse])


def test_graph_survives_workspace_growth_and_release():
    """A graph captured from a one-call decode keeps a valid workspace when a
    later call grows the library-owned workspace (the old buffer is retired,
    not freed): replays after the growth still give the eager call's bits.
    gqa_attn_release_workspace then frees everything and the next call
    allocates afresh."""
    import gqa_attention_flashattention_amd as gq
    import torch
    gq.release_workspace()
    small = gin.random_case("decode", "bf16", B=2, H_q=64, H_kv=8, d=128, kv_len=[900, 37],
                            seed=86)
    q, k, v = (to_gpu(x, "bf16") for x in (small.q_store, small.k_store, small.v_store))
    o = torch.empty_like(q)
    call = lambda: gq.decode(q, k, v, small.kv_len, out=o)
    call()
    torch.cuda.synchronize()
    eager = o.clone()
    oref, _ = oracle.decode(small.q, small.k, small.v, small.kv_len)
    assert_close(to_f64(eager), oref, name="small decode")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    # 4096 one-key splits of 64 heads: a workspace of about 136 MB
    big = gin.random_case("decode", "bf16", B=1, H_q=64, H_kv=8, d=128, kv_len=[4096], seed=87)
    qb, kb, vb = (to_gpu(x, "bf16") for x in (big.q_store, big.k_store, big.v_store))
    need = gq.decode_workspace_bytes(1, 64, 8, 128, big.kv_len, 4096)
    assert need > (64 << 20)
    ob = gq.decode(qb, kb, vb, big.kv_len, num_splits=4096)
    torch.cuda.synchronize()
    obref, _ = oracle.decode(big.q, big.k, big.v, big.kv_len)
    assert_close(to_f64(ob), obref, name="decode after growth")

    for i in range(REPLAYS):
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager), f"replay {i} after the growth differs from the eager call"
        ob2 = gq.decode(qb, kb, vb, big.kv_len, num_splits=4096)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(ob2, ob)
    del g
    gq.release_workspace()
    o.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    assert torch.equal(o, eager)
    gq.release_workspace()
