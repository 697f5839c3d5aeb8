"""GPU parity of the prefill path (C ABI gqa_attn_prefill) against the fp64
oracle, element by element."""
import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _run(inp, causal, q_offset, scale=None):
    import gqa_attention_flashattention_amd as gq
    w = inp.workload
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q_store, inp.k_store, inp.v_store))
    o, lse = gq.prefill(q, k, v, causal=causal, q_offset=q_offset, scale=scale)
    import torch
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("B,T,S,Hq,Hkv,d,causal,q_offset,dtype", [
    (1, 128, 128, 8, 1, 64, True, 0, "f32"),          # the tiny fp32 workload's shape
    (2, 77, 203, 12, 4, 128, False, 0, "f32"),
    (1, 100, 457, 16, 2, 128, True, 357, "f32"),
    (1, 300, 300, 16, 2, 128, True, 0, "bf16"),       # ragged rows and keys, G = 8
    (1, 100, 457, 16, 2, 128, True, 357, "bf16"),     # chunk at an offset
    (2, 77, 203, 12, 4, 64, False, 0, "bf16"),        # G = 3, d = 64, non-causal ragged
    (2, 65, 65, 5, 5, 128, True, 0, "bf16"),          # G = 1 (multi-head attention)
    (1, 40, 96, 10, 2, 64, True, 56, "bf16"),         # G = 5
    (3, 1, 130, 8, 2, 128, True, 129, "bf16"),        # one query token
    (1, 513, 700, 64, 8, 128, True, 187, "bf16"),     # Llama3-70B heads, several tiles
    (1, 300, 100, 16, 2, 128, False, 0, "bf16"),      # more queries than keys, non-causal
    (2, 40, 300, 64, 1, 128, True, 260, "bf16"),      # G = 64: one KV head for all query heads
    (1, 33, 33, 16, 2, 64, False, 0, "f32"),          # fp32 non-causal, d = 64
])
def test_prefill_parity(B, T, S, Hq, Hkv, d, causal, q_offset, dtype):
    inp = gin.random_case("prefill", dtype, B=B, H_q=Hq, H_kv=Hkv, d=d, T_q=T, S_kv=S, seed=T + S)
    og, lg = _run(inp, causal, q_offset)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=causal, q_offset=q_offset)
    assert_close(og, oref, lg, lref, dtype=dtype, name=f"prefill {B},{T},{S},{Hq},{Hkv},{d}")


def test_tiny_f32_workload():
    inp = gin.make("prefill_tiny_f32")
    og, lg = _run(inp, True, 0)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True)
    assert_close(og, oref, lg, lref, dtype="f32", name="prefill_tiny_f32")


def test_uniform_scores_mean_of_v():
    """Q = 0: O is the causal running mean of V, LSE = ln(position + 1)."""
    inp = gin.random_case("prefill", "bf16", B=1, H_q=16, H_kv=2, d=128, T_q=200, S_kv=200, seed=3)
    inp.q_store[...] = 0
    inp.q[...] = 0
    og, lg = _run(inp, True, 0)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True)
    assert np.abs(lref - np.log(np.arange(1, 201))[None, :, None]).max() < 1e-12
    assert_close(og, oref, lg, lref, name="uniform scores")


def test_constant_v_per_head():
    inp = gin.random_case("prefill", "bf16", B=1, H_q=16, H_kv=4, d=64, T_q=130, S_kv=130, seed=4)
    c = gin.bf16_round_bits(np.arange(4 * 64, dtype=np.float32).reshape(4, 64) / 64.0)
    inp.v_store[...] = c[None, None]
    inp.v[...] = gin.bf16_bits_to_f32(c)[None, None]
    og, _ = _run(inp, True, 0)
    exp = np.repeat(gin.bf16_bits_to_f32(c).astype(np.float64), 4, axis=0)   # head h -> kv h // 4
    assert np.abs(og[0] - exp[None]).max() <= 2e-2


@pytest.mark.parametrize("q_scale", [4.0, 8.0])
def test_peaky_scores(q_scale):
    inp = gin.random_case("prefill", "bf16", B=1, H_q=8, H_kv=1, d=128, T_q=192, S_kv=320, seed=9,
                          q_scale=q_scale)
    og, lg = _run(inp, True, 128)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True, q_offset=128)
    assert_close(og, oref, lg, lref, name=f"peaky x{q_scale}")


def test_moving_max_across_tiles():
    """Scores rise along the keys, so the running max changes on every tile."""
    S, d = 512, 128
    u = np.full(d, 0.25, np.float32)
    k = (np.arange(S, dtype=np.float32)[:, None] / S * 6.0) * u[None, :]
    kb = gin.bf16_round_bits(k.reshape(1, S, 1, d))
    q = gin.bf16_round_bits(np.tile(u, (1, S, 8, 1)).reshape(1, S, 8, d))
    rng = np.random.default_rng(1)
    vb = gin.bf16_round_bits(rng.standard_normal((1, S, 1, d), dtype=np.float32))
    inp = gin.Inputs(None, gin.bf16_bits_to_f32(q), gin.bf16_bits_to_f32(kb), gin.bf16_bits_to_f32(vb),
                     q, kb, vb)
    inp.workload = gin.Workload("moving", "prefill", "bf16", B=1, H_q=8, H_kv=1, d=d, T_q=S, S_kv=S)
    og, lg = _run(inp, True, 0)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=True)
    assert_close(og, oref, lg, lref, name="moving max")


def test_deterministic():
    import gqa_attention_flashattention_amd as gq
    import torch
    inp = gin.random_case("prefill", "bf16", B=1, H_q=64, H_kv=8, d=128, T_q=257, S_kv=400, seed=5)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    o1, l1 = gq.prefill(q, k, v, causal=True, q_offset=143)
    o2, l2 = gq.prefill(q, k, v, causal=True, q_offset=143)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _sampled_rows(B, T, Hq, n, seed):
    rng = np.random.default_rng(seed)
    total = B * T * Hq
    fixed = np.array([0, 1, Hq - 1, Hq, total // 2, total - Hq, total - 1], np.int64)
    return np.unique(np.concatenate([fixed, rng.integers(0, total, n)]))


@pytest.mark.parametrize("name", ["prefill_8k_causal", "prefill_chunk_64k"])
def test_full_size_sampled(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    computes a sample of rows (first, last, head boundaries, random, and one
    row of every work-group's 256-row block)."""
    inp = gin.make(name)
    w = inp.workload
    og, lg = _run(inp, w.causal, w.q_offset)
    rows = np.union1d(_sampled_rows(w.B, w.T_q, w.H_q, 384, 7),
                      gin.rows_per_workgroup(w.B, w.T_q, w.H_q, w.H_kv, seed=8))
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=w.causal, q_offset=w.q_offset,
                                rows=rows)
    assert_close(og.reshape(-1, w.d)[rows], oref, lg.reshape(-1)[rows], lref, name=name)


def _staircase_scores(levels, *, causal, T=192, Hq=16, Hkv=2, d=128, seed=21):
    """Q along one axis and K scaled along it so that every query row sees the
    scores `levels[j]` (base-2 units after the kernel's scale * log2(e)) on key
    tile j (64 keys each): all rows share the same score staircase.  The
    products alpha * beta are exact in fp32, so the oracle and the kernel see
    the same scores."""
    S = 64 * len(levels)
    q_offset = S - T if causal else 0      # causal: the chunk ends at the last key
    inp = gin.random_case("prefill", "bf16", B=1, H_q=Hq, H_kv=Hkv, d=d, T_q=T, S_kv=S, seed=seed)
    c = (1.0 / np.sqrt(d)) * np.log2(np.e)
    alpha = 8.0
    qf = np.zeros(inp.q.shape, np.float32)
    qf[..., 0] = alpha
    beta = np.repeat(np.asarray(levels, np.float64) / (c * alpha), 64).astype(np.float32)
    kf = np.zeros(inp.k.shape, np.float32)
    kf[0, :, :, 0] = beta[:, None]
    for name, arr in (("q", qf), ("k", kf)):
        bits = gin.bf16_round_bits(arr)
        getattr(inp, name + "_store")[...] = bits
        getattr(inp, name)[...] = gin.bf16_bits_to_f32(bits)
    og, lg = _run(inp, causal, q_offset)
    oref, lref = oracle.prefill(inp.q, inp.k, inp.v, causal=causal, q_offset=q_offset)
    return og, lg, oref, lref


@pytest.mark.parametrize("levels", [
    # tile 1: every P = 2^5 against the reference set by tile 0, so each
    # lane's sum of P exceeds 2^8 with no row max grown by more than 8 (the
    # row max is taken and P recomputed unchanged); tile 2 likewise just
    # below the rescale threshold; tile 3 grows by 12 (rescale); tile 4 back
    # under the reference (fast path); tile 5 grows again
    [0.0, 5.0, 7.9, 12.0, 9.0, 24.0, 3.0],
    # falling scores: the first tile sets the reference, every later tile
    # takes the fast path
    [10.0, 6.0, 2.0, -3.0, -8.0, -20.0],
])
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_reference_paths(levels, causal):
    og, lg, oref, lref = _staircase_scores(levels, causal=causal)
    assert_close(og, oref, lg, lref, name=f"score staircase {levels} causal={causal}")
