"""Host threads sharing the library-owned decode workspace on one stream.

Several Python threads (ctypes releases the GIL during each C call) issue
gqa_attn_decode on the same device stream with split counts that grow from
call to call, so the library has to replace its workspace (retiring the old
one) while other threads have kernels queued against the old one.  Every output is checked
against the fp64 oracle; a call that launched into a freed or replaced
buffer would show up as a wrong or non-finite result."""
import threading

import numpy as np
import pytest

import oracle
from gqa_attention_flashattention_amd import inputs as gin

from gpu_util import assert_close, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def test_threads_share_workspace_on_one_stream():
    import torch
    import gqa_attention_flashattention_amd as gq

    cases = []
    for i, kv_len in enumerate(([3000, 17, 1200], [4096, 2049], [513, 64, 9, 2500])):
        inp = gin.random_case("decode", "bf16", B=len(kv_len), H_q=64, H_kv=8, d=128,
                              kv_len=kv_len, seed=40 + i)
        oref, _ = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len)
        dev = tuple(to_gpu(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
        cases.append((inp, dev, oref))
    torch.cuda.synchronize()

    # split caps that grow over the calls: the partials workspace grows from
    # well under a megabyte to about 136 MB (4096 one-key splits of 64 heads)
    caps = [4, 32, 128, 512, 1024, 2048, 4096]
    n_threads = 4
    results = [[] for _ in range(n_threads)]
    errors = []
    start = threading.Barrier(n_threads)

    def worker(t):
        try:
            start.wait()
            for j, cap in enumerate(caps):
                c = (t + j) % len(cases)
                inp, (q, k, v), _ = cases[c]
                o = gq.decode(q, k, v, inp.kv_len, num_splits=cap + t)
                results[t].append((c, cap + t, o))
        except Exception as e:   # reported in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(n_threads):
        assert len(results[t]) == len(caps)
        for c, cap, o in results[t]:
            assert_close(to_f64(o), cases[c][2], name=f"thread {t} case {c} num_splits={cap}")
