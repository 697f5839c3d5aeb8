"""fp64 CPU oracle for grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it
imports nothing from the product package.

Two independent implementations live here:

* ``prefill`` / ``decode`` -- ctypes wrappers over ``gqa_oracle.c`` (plain
  C, double precision, OpenMP over output rows), the definition
  softmax(scale * Q K^T + causal mask) V written out per row;
* ``oracle_np`` -- a NumPy fp64 formulation (whole score matrix per head,
  explicit mask), used to cross-check the C code on small shapes.

Citations refer to the ADR-0060 page ("AHBM GQA Fused Attention kernel
(Llama3-70B)"): the per-tile op sequence of section 3, the merge of section 4
and the causal tile classes of section 5.4 all reduce, in exact arithmetic,
to the definition computed here (its "Algorithm lineage" paragraph: no new
mathematics).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgqa_oracle.so")


_i64 = ctypes.c_int64


class OracleLib:
    """ctypes view of one build of gqa_oracle.c (the default build, or a
    test-only variant compiled elsewhere)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.gqa_oracle_prefill.restype = ctypes.c_int
        lib.gqa_oracle_prefill.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, _i64, ctypes.c_int]
        lib.gqa_oracle_prefill_window.restype = ctypes.c_int
        lib.gqa_oracle_prefill_window.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, _i64,
            ctypes.c_int]
        lib.gqa_oracle_decode.restype = ctypes.c_int
        lib.gqa_oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, _i64, ctypes.c_int]
        lib.gqa_oracle_num_threads.restype = ctypes.c_int
        lib.gqa_oracle_num_threads.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = path

    def num_threads(self, n: int = 0) -> int:
        """Set (n > 0) and return the OpenMP thread count the oracle uses."""
        return self.lib.gqa_oracle_num_threads(int(n))

    def prefill(self, q, k, v, *, causal: bool, q_offset: int = 0,
                scale: float | None = None, rows=None, threads: int = 0):
        """Oracle prefill.  q [B,T_q,H_q,d]; k, v [B,S_kv,H_kv,d].

        Returns (O, LSE) in float64: O [B,T_q,H_q,d] and LSE [B,T_q,H_q], or,
        when ``rows`` (flat indices (b*T_q+t)*H_q+h) is given, O [n,d], LSE [n].
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, T_q, H_q, d = q.shape
        Bk, S_kv, H_kv, dk = k.shape
        if Bk != B or dk != d or v.shape != k.shape:
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        if rows is None:
            o = np.empty((B, T_q, H_q, d), np.float64)
            lse = np.empty((B, T_q, H_q), np.float64)
            rp, nr = None, 0
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            o = np.empty((rows.size, d), np.float64)
            lse = np.empty((rows.size,), np.float64)
            rp, nr = rows.ctypes.data, rows.size
        rc = self.lib.gqa_oracle_prefill(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         o.ctypes.data, lse.ctypes.data, B, T_q, S_kv, H_q,
                                         H_kv, d, float(scale), int(bool(causal)),
                                         int(q_offset), rp, nr, int(threads))
        if rc != 0:
            raise ValueError(f"gqa_oracle_prefill failed with code {rc}")
        return o, lse

    def prefill_window(self, q, k, v, *, q_offset: int, window: int, sink: int = 0,
                       scale: float | None = None, rows=None, threads: int = 0):
        """Oracle sink + local-window prefill (always causal): query t at
        position p = q_offset + t sees key j iff j <= p and (j < sink or
        j > p - window).  Shapes and return values as ``prefill``."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, T_q, H_q, d = q.shape
        Bk, S_kv, H_kv, dk = k.shape
        if Bk != B or dk != d or v.shape != k.shape:
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        if rows is None:
            o = np.empty((B, T_q, H_q, d), np.float64)
            lse = np.empty((B, T_q, H_q), np.float64)
            rp, nr = None, 0
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            o = np.empty((rows.size, d), np.float64)
            lse = np.empty((rows.size,), np.float64)
            rp, nr = rows.ctypes.data, rows.size
        rc = self.lib.gqa_oracle_prefill_window(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                                o.ctypes.data, lse.ctypes.data, B, T_q, S_kv,
                                                H_q, H_kv, d, float(scale), int(q_offset),
                                                int(window), int(sink), rp, nr, int(threads))
        if rc != 0:
            raise ValueError(f"gqa_oracle_prefill_window failed with code {rc}")
        return o, lse

    def decode(self, q, k, v, kv_len, *, scale: float | None = None, num_splits: int = 0,
               rows=None, threads: int = 0):
        """Oracle decode.  q [B,H_q,d]; k, v packed [sum(kv_len),H_kv,d].

        ``num_splits`` = 0 computes the unsplit definition; > 0 computes
        per-shard partials and merges them (the FlashDecoding form).  Returns
        (O, LSE) in float64: O [B,H_q,d], LSE [B,H_q] (or [n,d], [n] for
        ``rows``, flat b*H_q+h).
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, H_q, d = q.shape
        kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
        if kv_len.shape != (B,):
            raise ValueError("kv_len must have shape [B]")
        N, H_kv, dk = k.shape
        if dk != d or v.shape != k.shape or N != int(kv_len.astype(np.int64).sum()):
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        if rows is None:
            o = np.empty((B, H_q, d), np.float64)
            lse = np.empty((B, H_q), np.float64)
            rp, nr = None, 0
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            o = np.empty((rows.size, d), np.float64)
            lse = np.empty((rows.size,), np.float64)
            rp, nr = rows.ctypes.data, rows.size
        rc = self.lib.gqa_oracle_decode(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                        o.ctypes.data, lse.ctypes.data, B, H_q, H_kv, d,
                                        kv_len.ctypes.data, float(scale), int(num_splits),
                                        rp, nr, int(threads))
        if rc != 0:
            raise ValueError(f"gqa_oracle_decode failed with code {rc}")
        return o, lse


_default: OracleLib | None = None


def _lib() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _default = OracleLib(_LIB_PATH)
    return _default


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        # every test input is exactly representable in float32 (bf16 values
        # or small integers); refuse anything that would be rounded here
        b = a.astype(np.float32)
        if not np.array_equal(b.astype(a.dtype), a):
            raise ValueError("oracle inputs must be exactly representable in float32")
        a = b
    return np.ascontiguousarray(a)


def num_threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle uses."""
    return _lib().num_threads(n)


def prefill(q, k, v, **kw):
    """See OracleLib.prefill."""
    return _lib().prefill(q, k, v, **kw)


def decode(q, k, v, kv_len, **kw):
    """See OracleLib.decode."""
    return _lib().decode(q, k, v, kv_len, **kw)


def prefill_window(q, k, v, **kw):
    """See OracleLib.prefill_window."""
    return _lib().prefill_window(q, k, v, **kw)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Two's-complement int4 codes stored two per byte, channel 2i in the low
    nibble of byte i (pccx page, section 4 item 3: optional INT4 KV cache),
    -> int8 codes with the channel axis doubled."""
    b = np.asarray(packed, np.uint8).astype(np.int16)
    lo = b & 0x0F
    hi = b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Symmetric per-channel dequantisation: value[j, kv, x] = code[j, kv, x] *
    scale[kv, x] (codes int8 [N, H_kv, d], scale [H_kv, d]).  Returned as
    float32, which must hold every product exactly (the oracle's inputs are
    exact float32 values); raises otherwise."""
    prod = np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[None]
    out = prod.astype(np.float32)
    if not np.array_equal(out.astype(np.float64), prod):
        raise ValueError("dequantised values are not exactly representable in float32")
    return out
