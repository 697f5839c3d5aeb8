"""Measured ceilings of HBM reads and bf16 MFMA throughput on the current
GPU (libgqa_ceilings.so, built from csrc/ceilings.hip), which the benchmark
prints beside the spec-sheet peaks.  Measurement only: nothing on the
attention path uses this module."""
from __future__ import annotations

import ctypes
import os
import time

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.CEIL_LIB):
            raise RuntimeError(f"{_build.CEIL_LIB} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(_build.CEIL_LIB)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.gqa_ceiling_read.argtypes = [vp, sz, vp, i, vp]
        lib.gqa_ceiling_read.restype = i
        lib.gqa_ceiling_mfma.argtypes = [vp, i, i, vp]
        lib.gqa_ceiling_mfma.restype = i
        _lib = lib
    return _lib


def _timed(fn, reps: int, warm_s: float = 0.2) -> float:
    """ms per call of fn after warm_s seconds of back-to-back calls (the
    shader clock ramps up under sustained load)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"{name} returned {rc}")


def hbm_read_gbps(nbytes: int = 4 << 30, blocks: int = 1024, reps: int = 10) -> float:
    """GB/s (1e9 B) of a streaming read of nbytes with 16-byte non-temporal
    loads (the decode kernels' K/V load form), each of `blocks` work-groups
    reading a contiguous range (1024 measured fastest of 1024-8192 on
    MI355X: 7.05 vs 6.70 TB/s)."""
    import torch
    lib = _load()
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call():
        _check(lib.gqa_ceiling_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream),
               "gqa_ceiling_read")
    ms = _timed(call, reps)
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9


def mfma_bf16_tflops(blocks: int = 1024, iters: int = 10000, reps: int = 5) -> float:
    """TFLOP/s of back-to-back v_mfma_f32_32x32x16_bf16 on register operands
    that change at every issue, blocks work-groups of four waves (1024: two
    waves per SIMD; one wave per SIMD measures the same)."""
    import torch
    lib = _load()
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call():
        _check(lib.gqa_ceiling_mfma(sink.data_ptr(), blocks, iters, stream), "gqa_ceiling_mfma")
    ms = _timed(call, reps)
    flops = blocks * 4 * iters * 4 * 32768
    return flops / (ms * 1e-3) / 1e12
