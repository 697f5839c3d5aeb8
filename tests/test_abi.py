"""C ABI checks that need no GPU: the library loads, exports every function
include/gqa_attn.h declares, validates arguments (returning a status before
anything reaches the GPU) and computes the decode split plan."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import gqa_attention_flashattention_amd as gq
from gqa_attention_flashattention_amd import binding


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "gqa_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["gqa_attn_prefill", "gqa_attn_decode", "gqa_attn_decode_split",
              "gqa_attn_decode_combine", "gqa_attn_decode_plan", "gqa_attn_decode_multi",
              "gqa_attn_prefill_kvsplit", "gqa_attn_prefill_kvsplit_count",
              "gqa_attn_prefill_window", "gqa_attn_decode_ring", "gqa_attn_decode_quant",
              "gqa_attn_decode_ring_quant", "gqa_attn_prefill_window_kvsplit",
              "gqa_attn_decode_noalloc",
              "gqa_attn_status_string", "gqa_attn_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = gq.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings():
    lib = gq.load_library()
    for code in range(6):
        assert lib.gqa_attn_status_string(code)
    assert lib.gqa_attn_status_string(99) == b"unknown status"


P = ctypes.c_void_p(16)   # never dereferenced: validation fails before any device access


def _prefill(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, T=4, S=8, Hq=8, Hkv=2, d=128, scale=0.1,
             causal=1, qoff=0, dtype=0)
    a.update(kw)
    return gq.load_library().gqa_attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                              a["T"], a["S"], a["Hq"], a["Hkv"], a["d"],
                                              a["scale"], a["causal"], a["qoff"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(T=0), 2), (dict(S=0), 2), (dict(Hq=7), 2), (dict(Hkv=0), 2),
    (dict(d=96), 3), (dict(d=256), 3), (dict(dtype=2), 3),
    (dict(qoff=-1), 4), (dict(qoff=5), 4), (dict(scale=0.0), 4), (dict(scale=float("nan")), 4),
    (dict(scale=-1.0), 4),
    (dict(Hq=32768, Hkv=2), 2),          # H_q * d * 514 > 2^31 - 1
])
def test_prefill_rejects(kw, code):
    assert _prefill(**kw) == code


def _decode(kv_len, **kw):
    a = dict(q=P, k=P, v=P, o=P, B=len(kv_len), Hq=8, Hkv=2, d=128, scale=0.1, ns=0, dtype=0)
    a.update(kw)
    arr = np.asarray(kv_len, np.int32)
    return gq.load_library().gqa_attn_decode(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"],
                                             a["Hkv"], a["d"], arr.ctypes.data if kv_len else None,
                                             a["scale"], a["ns"], a["dtype"], None)


@pytest.mark.parametrize("kv_len,kw,code", [
    ([4], dict(q=None), 1), ([4], dict(o=None), 1), ([], dict(B=1), 1),
    ([4, 0], {}, 2), ([4, -3], {}, 2), ([4], dict(B=0), 2), ([4], dict(Hq=9), 2),
    ([4], dict(d=32), 3), ([4], dict(dtype=1), 3), ([4], dict(scale=float("inf")), 4),
])
def test_decode_rejects(kv_len, kw, code):
    assert _decode(kv_len, **kw) == code


def _decode_noalloc(kv_len, **kw):
    a = dict(q=P, k=P, v=P, o=P, B=len(kv_len), Hq=8, Hkv=2, d=128, scale=0.1, ns=0, dtype=0)
    a.update(kw)
    arr = np.asarray(kv_len, np.int32)
    return gq.load_library().gqa_attn_decode_noalloc(
        a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"], a["d"],
        arr.ctypes.data if kv_len else None, a["scale"], a["ns"], a["dtype"], None)


@pytest.mark.parametrize("kv_len,kw,code", [
    ([4], dict(q=None), 1), ([4], dict(o=None), 1), ([], dict(B=1), 1),
    ([4, 0], {}, 2), ([4], dict(Hq=9), 2), ([4], dict(d=32), 3), ([4], dict(dtype=1), 3),
    ([4], dict(scale=0.0), 4),
    # 2 x 4096 one-key splits of 64 query heads: 8192 * 64 * 130 * 4 bytes > 16 MiB
    ([4096, 4096], dict(Hq=64, Hkv=8, ns=4096), 4),
])
def test_decode_noalloc_rejects(kv_len, kw, code):
    assert _decode_noalloc(kv_len, **kw) == code


def _decode_multi(kv_len, **kw):
    a = dict(q=P, k=P, v=P, o=P, B=len(kv_len), T=2, Hq=8, Hkv=2, d=128, scale=0.1, ns=0, dtype=0)
    a.update(kw)
    arr = np.asarray(kv_len, np.int32)
    return gq.load_library().gqa_attn_decode_multi(
        a["q"], a["k"], a["v"], a["o"], None, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"],
        arr.ctypes.data if kv_len else None, a["scale"], a["ns"], a["dtype"], None)


@pytest.mark.parametrize("kv_len,kw,code", [
    ([4], dict(q=None), 1), ([4], dict(o=None), 1), ([], dict(B=1), 1),
    ([4, 1], {}, 2),                     # fewer keys than new tokens
    ([4], dict(T=0), 2), ([400], dict(T=257), 2), ([4], dict(Hq=9), 2),
    ([4], dict(d=32), 3), ([4], dict(dtype=1), 3), ([4], dict(scale=0.0), 4),
])
def test_decode_multi_rejects(kv_len, kw, code):
    assert _decode_multi(kv_len, **kw) == code


def test_kvsplit_rejects_and_counts():
    lib = gq.load_library()
    # f32 is not built for the KV-parallel path; bad offset; NULL output
    assert lib.gqa_attn_prefill_kvsplit(P, P, P, P, None, 1, 4, 8, 8, 2, 128, 0.1, 1, 4, 0, 1,
                                        None) == 3
    assert lib.gqa_attn_prefill_kvsplit(P, P, P, P, None, 1, 4, 8, 8, 2, 128, 0.1, 1, 5, 0, 0,
                                        None) == 4
    assert lib.gqa_attn_prefill_kvsplit(P, P, P, None, None, 1, 4, 8, 8, 2, 128, 0.1, 1, 4, 0, 0,
                                        None) == 1
    with pytest.raises(binding.GQAError):
        gq.prefill_kvsplit_count(1, 4, 8, 8, 2, 100, causal=False)
    # explicit counts are clamped to the key tiles and to 64
    assert gq.prefill_kvsplit_count(1, 64, 200, 8, 2, 128, causal=False, num_splits=16) == 4
    assert gq.prefill_kvsplit_count(1, 64, 100000, 8, 2, 128, causal=False, num_splits=500) == 64
    # a large grid needs no split; a short chunk over a long cache gets several
    assert gq.prefill_kvsplit_count(1, 8192, 8192, 64, 8, 128, causal=True) == 1
    assert gq.prefill_kvsplit_count(1, 256, 65792, 64, 8, 128, causal=True, q_offset=65536) > 1


def test_window_prefill_rejects():
    lib = gq.load_library()
    args = lambda **kw: [kw.get("q", P), P, P, kw.get("o", P), None, 1, 4, 8, 8, 2,
                         kw.get("d", 128), 0.1, kw.get("qoff", 4), kw.get("window", 3),
                         kw.get("sink", 0), kw.get("dtype", 0), None]
    assert lib.gqa_attn_prefill_window(*args(q=None)) == 1
    assert lib.gqa_attn_prefill_window(*args(d=96)) == 3
    assert lib.gqa_attn_prefill_window(*args(dtype=1)) == 3
    assert lib.gqa_attn_prefill_window(*args(qoff=5)) == 4
    assert lib.gqa_attn_prefill_window(*args(window=0)) == 4
    assert lib.gqa_attn_prefill_window(*args(sink=-1)) == 4
    sargs = lambda **kw: args(**kw)[:15] + [kw.get("ns", 0)] + args(**kw)[15:]
    assert lib.gqa_attn_prefill_window_kvsplit(*sargs(q=None)) == 1
    assert lib.gqa_attn_prefill_window_kvsplit(*sargs(d=96)) == 3
    assert lib.gqa_attn_prefill_window_kvsplit(*sargs(dtype=1)) == 3
    assert lib.gqa_attn_prefill_window_kvsplit(*sargs(qoff=5)) == 4
    assert lib.gqa_attn_prefill_window_kvsplit(*sargs(window=0)) == 4
    assert lib.gqa_attn_prefill_window_kvsplit(*sargs(sink=-1)) == 4


def test_ring_decode_rejects():
    lib = gq.load_library()

    def call(kv=(10,), **kw):
        a = dict(q=P, o=P, T=2, cap=16, window=10, sink=4, dtype=0, d=128)
        a.update(kw)
        arr = np.asarray(kv, np.int32)
        return lib.gqa_attn_decode_ring(a["q"], P, P, a["o"], None, len(kv), a["T"], 8, 2, a["d"],
                                        a["cap"], arr.ctypes.data, a["window"], a["sink"], 0.1, 0,
                                        a["dtype"], None)
    assert call(q=None) == 1 and call(o=None) == 1
    assert call(kv=(1,)) == 2                   # fewer tokens than new tokens
    assert call(T=0) == 2 and call(cap=0) == 2
    assert call(d=32) == 3 and call(dtype=1) == 3
    assert call(sink=16) == 4 and call(sink=-1) == 4 and call(window=0) == 4
    assert call(window=13) == 4                 # window + T_q - 1 > capacity - sink


def test_quant_decode_rejects():
    lib = gq.load_library()

    def call(kv=(10,), **kw):
        a = dict(q=P, o=P, ks=P, vs=P, T=1, bits=8, d=128)
        a.update(kw)
        arr = np.asarray(kv, np.int32)
        return lib.gqa_attn_decode_quant(a["q"], P, P, a["ks"], a["vs"], a["o"], None, len(kv),
                                         a["T"], 8, 2, a["d"], arr.ctypes.data, a["bits"], 0.1, 0,
                                         None)
    assert call(q=None) == 1 and call(o=None) == 1 and call(ks=None) == 1 and call(vs=None) == 1
    assert call(bits=2) == 3 and call(bits=16) == 3 and call(d=32) == 3
    assert call(T=0) == 2 and call(kv=(1,), T=2) == 2 and call(kv=(0,)) == 2


def test_ring_quant_decode_rejects():
    lib = gq.load_library()

    def call(kv=(10,), **kw):
        a = dict(q=P, o=P, ks=P, vs=P, T=2, cap=16, window=10, sink=4, bits=4, d=128)
        a.update(kw)
        arr = np.asarray(kv, np.int32)
        return lib.gqa_attn_decode_ring_quant(a["q"], P, P, a["ks"], a["vs"], a["o"], None,
                                              len(kv), a["T"], 8, 2, a["d"], a["cap"],
                                              arr.ctypes.data, a["window"], a["sink"], a["bits"],
                                              0.1, 0, None)
    assert call(q=None) == 1 and call(o=None) == 1 and call(ks=None) == 1 and call(vs=None) == 1
    assert call(bits=2) == 3 and call(bits=16) == 3 and call(d=32) == 3
    assert call(kv=(1,)) == 2 and call(T=0) == 2 and call(cap=0) == 2
    assert call(sink=16) == 4 and call(window=0) == 4 and call(window=13) == 4


def test_split_and_combine_reject_small_workspace():
    lib = gq.load_library()
    kv = np.array([1000], np.int32)
    need = gq.decode_workspace_bytes(1, 64, 8, 128, kv)
    assert lib.gqa_attn_decode_split(P, P, P, P, need - 4, 1, 64, 8, 128, kv.ctypes.data, 0.1, 0,
                                     0, None) == 4
    assert lib.gqa_attn_decode_combine(P, need - 1, P, None, 1, 64, 8, 128, kv.ctypes.data, 0, 0,
                                       None) == 4
    assert lib.gqa_attn_decode_split(P, P, P, None, need, 1, 64, 8, 128, kv.ctypes.data, 0.1, 0,
                                     0, None) == 1


def test_binding_raises():
    with pytest.raises(binding.GQAError):
        gq.decode_plan(2, 64, 8, 128, [5, 0])
    with pytest.raises(binding.GQAError):
        gq.decode_plan(1, 64, 8, 100, [5])


@pytest.mark.parametrize("kv_len,num_splits", [
    ([8192], 0), ([1, 2, 3], 0), ([1024, 32768, 5000], 0), ([131072], 0),
    ([37, 1, 64], 7), ([10], 4), ([10], 6), ([10], 100), ([5, 9], 1),
])
def test_decode_plan_covers_every_key_once(kv_len, num_splits):
    """Every key of every sequence falls in exactly one split; splits are
    contiguous, non-empty, and follow the documented rule."""
    p = gq.decode_plan(len(kv_len), 64, 8, 128, kv_len, num_splits)
    assert p["total_splits"] == int(p["splits"].sum())
    assert p["workspace_bytes"] == p["total_splits"] * 64 * 130 * 4
    for n, ns_b in zip(kv_len, p["splits"]):
        if num_splits > 0:
            L = -(-n // min(num_splits, n))
            assert ns_b <= num_splits
        else:
            L = p["split_len"] if len(set(kv_len)) == 1 else None
        if L is not None:
            assert ns_b == -(-n // L)
            covered = np.zeros(n, np.int32)
            for s in range(ns_b):
                lo, hi = s * L, min((s + 1) * L, n)
                assert hi > lo
                covered[lo:hi] += 1
            assert np.all(covered == 1)


def test_auto_plan_targets_occupancy():
    # decode_8k: 8 KV heads x splits should give several work-groups per CU
    p = gq.decode_plan(1, 64, 8, 128, [8192])
    assert p["split_len"] % 64 == 0 and 128 <= p["split_len"] <= 8192
    assert p["total_splits"] * 8 >= 256


def test_plan_split_len_is_the_longest_split():
    """*split_len is the longest split over the batch, max_b min(L_b, n_b),
    also when a later sequence is shorter than the first (both shorter than
    the automatic L = 128 here)."""
    p = gq.decode_plan(2, 64, 8, 128, [100, 50])
    assert p["splits"].tolist() == [1, 1]
    assert p["split_len"] == 100
    p = gq.decode_plan(3, 64, 8, 128, [50, 100, 70])
    assert p["split_len"] == 100


def _documented_auto_len(kv_len, H_kv, cus=256):
    """The automatic split length of gqa_attn_decode_plan as its header states
    it (bf16 cache, one new token, G <= 16): the candidate in [128, 8192]
    (multiples of 64 up to 1024, of 128 up to 2048, of 256 beyond)
    minimising ceil(W / R) * (L + 256) summed over launches of 64 sequences
    plus 8 x the largest split count of a sequence,
    W = split work-groups (H_kv per split, each counting twice above 128
    keys), R = 2 per compute unit; ties to the longer L."""
    slots = 2 * cus
    hi = min(8192, max(128, -(-max(kv_len) // 64) * 64))
    best, best_cost = None, None
    cands = [L for L in range(128, hi + 1, 64)
             if L <= 1024 or (L <= 2048 and L % 128 == 0) or L % 256 == 0]
    for L in cands:
        per = H_kv * (2 if L > 128 else 1)
        cost = 0
        for b0 in range(0, len(kv_len), 64):
            n = sum(-(-x // L) for x in kv_len[b0:b0 + 64])
            cost += -(-(n * per) // slots) * (L + 256)
        cost += 8 * max(-(-x // L) for x in kv_len)
        if best_cost is None or cost <= best_cost:
            best, best_cost = L, cost
    return best


@pytest.mark.parametrize("seed,B", [(0, 1), (1, 3), (2, 16), (3, 16), (4, 70), (5, 200)])
def test_auto_plan_follows_the_documented_rule(seed, B):
    """Without a device (256 compute units assumed, as on MI355X) the
    automatic split length is the argmin of the documented cost."""
    rng = np.random.default_rng(seed)
    kv_len = rng.integers(1, 40000, size=B).tolist()
    p = gq.decode_plan(B, 64, 8, 128, kv_len)
    assert p["split_len"] == _documented_auto_len(kv_len, 8)


def test_auto_plan_on_the_benchmark_batches():
    """Whole rounds of resident work-groups where that is cheapest: the
    16-sequence ragged batch takes 64 splits of 4864 keys (512 work-groups of
    one KV head, two rounds of one per compute unit), decode_8k 32 splits of
    256 keys (256 work-groups: one round), the 128k sequence 32 splits of
    4096 (one round)."""
    from gqa_attention_flashattention_amd import inputs as gin
    kv_len = gin.kv_lengths(gin.WORKLOADS["decode_varlen_b16"], np.random.default_rng(0))
    p = gq.decode_plan(16, 64, 8, 128, kv_len)
    assert (p["split_len"], p["total_splits"]) == (4864, 64)
    p = gq.decode_plan(1, 64, 8, 128, [8192])
    assert (p["split_len"], p["total_splits"]) == (256, 32)
    p = gq.decode_plan(1, 64, 8, 128, [131072])
    assert (p["split_len"], p["total_splits"]) == (4096, 32)


def _documented_kvsplit_count(B, T_q, S_kv, H_q, H_kv, causal, q_offset, cus=256):
    """gqa_attn_prefill_kvsplit's automatic range count as its header states it
    (d = 128: 256 query rows per row block, partials far below 4 GiB here)."""
    G = H_q // H_kv
    blocks = -(-(T_q * G) // 256) * B * H_kv
    keys = q_offset + T_q if causal else S_kv
    T = -(-keys // 64)
    hi = max(1, min(64, T // 4))
    best, best_n = None, 1
    for n in range(1, hi + 1):
        cost = -(-(blocks * n) // cus) * (-(-T // n) + 4)
        if best is None or cost < best:
            best, best_n = cost, n
    return min(best_n, 64, T)


@pytest.mark.parametrize("B,T_q,S_kv,causal,q_offset", [
    (1, 256, 65792, True, 65536), (1, 2048, 67584, True, 65536), (1, 8192, 8192, True, 0),
    (1, 64, 8192, True, 8128), (2, 32, 4096, False, 0), (1, 1, 100000, True, 99999),
    (4, 512, 20000, True, 19488), (1, 128, 300, False, 0),
])
def test_kvsplit_count_follows_the_documented_rule(B, T_q, S_kv, causal, q_offset):
    n = gq.prefill_kvsplit_count(B, T_q, S_kv, 64, 8, 128, causal=causal, q_offset=q_offset)
    assert n == _documented_kvsplit_count(B, T_q, S_kv, 64, 8, causal, q_offset)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """bench.py runs on one GPU only: --gpus N > 1 (or a multi-rank launch)
    exits with status 2 and a JSON message, before touching any device."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + argv,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_ceilings_library_loads_and_rejects_bad_sizes():
    """The benchmark's ceiling kernels (separate library) export their two
    entry points and refuse invalid sizes before any launch."""
    from gqa_attention_flashattention_amd import ceilings
    lib = ceilings._load()
    assert lib.gqa_ceiling_read(None, 1024, None, 4, None) == 2
    assert lib.gqa_ceiling_read(8, 1000, 8, 4, None) == 2      # not a multiple of 16
    assert lib.gqa_ceiling_read(8, 1024, 8, 0, None) == 2      # no work-groups
    assert lib.gqa_ceiling_mfma(None, 4, 10, None) == 2
    assert lib.gqa_ceiling_mfma(8, 4, 0, None) == 2
