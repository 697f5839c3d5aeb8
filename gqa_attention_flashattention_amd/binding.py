"""ctypes binding of libgqa_attn.so (C ABI in include/gqa_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Tensors are torch tensors that live on the GPU;
torch supplies device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, GQAError is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgqa_attn.so"

GQA_BF16 = 0
GQA_F32 = 1

_lib = None


class GQAError(RuntimeError):
    """Raised when the library is missing or returns a nonzero gqa_status."""

    def __init__(self, msg: str, status: int | None = None):
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library():
    """Load libgqa_attn.so (once).  Raises GQAError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise GQAError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
                       f"g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i, f, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_size_t
    lib.gqa_attn_status_string.restype = ctypes.c_char_p
    lib.gqa_attn_status_string.argtypes = [i]
    lib.gqa_attn_version.restype = i
    lib.gqa_attn_version.argtypes = []
    lib.gqa_attn_prefill.restype = i
    lib.gqa_attn_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
    lib.gqa_attn_decode.restype = i
    lib.gqa_attn_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, f, i, i, vp]
    lib.gqa_attn_decode_noalloc.restype = i
    lib.gqa_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, f, i, i, vp]
    lib.gqa_attn_release_workspace.restype = i
    lib.gqa_attn_release_workspace.argtypes = []
    lib.gqa_attn_decode_plan.restype = i
    lib.gqa_attn_decode_plan.argtypes = [i, i, i, i, vp, i, vp, vp, vp, vp, vp]
    lib.gqa_attn_decode_split.restype = i
    lib.gqa_attn_decode_split.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, vp, f, i, i, vp]
    lib.gqa_attn_prefill_kvsplit.restype = i
    lib.gqa_attn_prefill_kvsplit.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, i,
                                             vp]
    lib.gqa_attn_prefill_window.restype = i
    lib.gqa_attn_prefill_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, i, vp]
    lib.gqa_attn_prefill_window_kvsplit.restype = i
    lib.gqa_attn_prefill_window_kvsplit.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i,
                                                    i, i, i, vp]
    lib.gqa_attn_prefill_kvsplit_count.restype = i
    lib.gqa_attn_prefill_kvsplit_count.argtypes = [i] * 9
    lib.gqa_attn_decode_quant.restype = i
    lib.gqa_attn_decode_quant.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, f, i,
                                          vp]
    lib.gqa_attn_decode_ring.restype = i
    lib.gqa_attn_decode_ring.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, i, f, i, i,
                                         vp]
    lib.gqa_attn_decode_ring_quant.restype = i
    lib.gqa_attn_decode_ring_quant.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp,
                                               i, i, i, f, i, vp]
    lib.gqa_attn_decode_multi.restype = i
    lib.gqa_attn_decode_multi.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, f, i, i, vp]
    lib.gqa_attn_decode_combine.restype = i
    lib.gqa_attn_decode_combine.argtypes = [vp, sz, vp, vp, i, i, i, i, vp, i, i, vp]
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().gqa_attn_status_string(rc).decode()
        raise GQAError(f"{what} failed: {msg} (status {rc})", rc)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_F32
    raise GQAError(f"unsupported dtype {t.dtype}", 3)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name: str, ndim: int):
    if t.dim() != ndim:
        raise GQAError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}", 2)
    if not t.is_cuda:
        raise GQAError(f"{name} must be a GPU tensor", 1)
    if not t.is_contiguous():
        raise GQAError(f"{name} must be contiguous", 2)


def _same(ref, *ts):
    """Every tensor in ts on ref's device and of ref's dtype (None entries skipped)."""
    for t in ts:
        if t is None:
            continue
        if t.device != ref.device:
            raise GQAError(f"tensors must be on {ref.device}, got {t.device}", 2)
        if t.dtype != ref.dtype:
            raise GQAError(f"tensors must share dtype {ref.dtype}, got {t.dtype}", 3)


def _out_like(out, ref, shape, name="out"):
    """A caller-given output must be a contiguous GPU tensor of exactly the shape
    and dtype the kernels write (the library trusts the sizes it is given)."""
    import torch
    if out is None:
        return torch.empty(shape, dtype=ref.dtype, device=ref.device)
    _require(out, name, len(shape))
    if tuple(out.shape) != tuple(shape) or out.dtype != ref.dtype or out.device != ref.device:
        raise GQAError(f"{name} must be {ref.dtype} {tuple(shape)} on {ref.device}, got "
                       f"{out.dtype} {tuple(out.shape)} on {out.device}", 2)
    return out


def _lse_buf(lse, ref, shape, wanted: bool):
    import torch
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=ref.device) if wanted else None
    _require(lse, "lse", len(shape))
    if tuple(lse.shape) != tuple(shape) or lse.dtype != torch.float32 or lse.device != ref.device:
        raise GQAError(f"lse must be float32 {tuple(shape)} on {ref.device}", 2)
    return lse


def _kv_len_array(kv_len, B: int) -> np.ndarray:
    try:
        import torch
        if isinstance(kv_len, torch.Tensor):
            kv_len = kv_len.detach().cpu().numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(np.asarray(kv_len), dtype=np.int32)
    if a.shape != (B,):
        raise GQAError(f"kv_len must have shape [{B}]", 2)
    return a


def prefill(q, k, v, *, causal: bool, q_offset: int = 0, scale: float | None = None,
            out=None, lse=None, return_lse: bool = True):
    """Fused GQA prefill.  q [B,T_q,H_q,d], k/v [B,S_kv,H_kv,d] (bf16 or fp32).

    Returns (o, lse): o like q, lse fp32 [B,T_q,H_q] (None if return_lse is
    False and no lse buffer was given)."""
    import torch
    _require(q, "q", 4)
    _require(k, "k", 4)
    _require(v, "v", 4)
    B, T_q, H_q, d = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise GQAError("k and v must be [B, S_kv, H_kv, d] matching q", 2)
    _same(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    rc = load_library().gqa_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T_q,
                                         S_kv, H_q, H_kv, d, float(scale), int(bool(causal)),
                                         int(q_offset), _dtype_code(q), _stream(q.device))
    _check(rc, "gqa_attn_prefill")
    return out, lse


def prefill_kvsplit(q, k, v, *, causal: bool, q_offset: int = 0, scale: float | None = None,
                    num_splits: int = 0, out=None, lse=None, return_lse: bool = True):
    """KV-parallel prefill: as prefill (bf16), with each row block's key tiles
    cut into ranges on separate work-groups and merged by log-sum-exp."""
    import torch
    _require(q, "q", 4)
    _require(k, "k", 4)
    _require(v, "v", 4)
    B, T_q, H_q, d = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise GQAError("k and v must be [B, S_kv, H_kv, d] matching q", 2)
    _same(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    rc = load_library().gqa_attn_prefill_kvsplit(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T_q, S_kv, H_q, H_kv, d,
        float(scale), int(bool(causal)), int(q_offset), int(num_splits), _dtype_code(q),
        _stream(q.device))
    _check(rc, "gqa_attn_prefill_kvsplit")
    return out, lse


def prefill_window(q, k, v, *, window: int, sink: int = 0, q_offset: int = 0,
                   scale: float | None = None, out=None, lse=None, return_lse: bool = True,
                   kv_split: bool = False, num_splits: int = 0):
    """Causal prefill with `sink` attention-sink keys and a local window of
    `window` keys (bf16): the query at position p sees key j iff j <= p and
    (j < sink or j > p - window).  kv_split=True runs the KV-parallel form
    (gqa_attn_prefill_window_kvsplit; num_splits <= 0: automatic)."""
    import torch
    _require(q, "q", 4)
    _require(k, "k", 4)
    _require(v, "v", 4)
    B, T_q, H_q, d = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise GQAError("k and v must be [B, S_kv, H_kv, d] matching q", 2)
    _same(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    if kv_split:
        rc = load_library().gqa_attn_prefill_window_kvsplit(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T_q, S_kv, H_q, H_kv, d,
            float(scale), int(q_offset), int(window), int(sink), int(num_splits),
            _dtype_code(q), _stream(q.device))
        _check(rc, "gqa_attn_prefill_window_kvsplit")
        return out, lse
    rc = load_library().gqa_attn_prefill_window(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T_q, S_kv, H_q, H_kv, d,
        float(scale), int(q_offset), int(window), int(sink), _dtype_code(q), _stream(q.device))
    _check(rc, "gqa_attn_prefill_window")
    return out, lse


def prefill_kvsplit_count(B: int, T_q: int, S_kv: int, H_q: int, H_kv: int, d: int, *,
                          causal: bool, q_offset: int = 0, num_splits: int = 0) -> int:
    """Host-only: the key-range count prefill_kvsplit uses."""
    n = load_library().gqa_attn_prefill_kvsplit_count(B, T_q, S_kv, H_q, H_kv, d,
                                                      int(bool(causal)), int(q_offset),
                                                      int(num_splits))
    if n < 1:
        _check(-n, "gqa_attn_prefill_kvsplit_count")
    return n


def decode_plan(B: int, H_q: int, H_kv: int, d: int, kv_len, num_splits: int = 0) -> dict:
    """Host-only split plan (no GPU needed)."""
    a = _kv_len_array(kv_len, B)
    splits = np.zeros(B, np.int32)
    split_len = ctypes.c_int(0)
    total = ctypes.c_int64(0)
    mx = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    rc = load_library().gqa_attn_decode_plan(B, H_q, H_kv, d, a.ctypes.data, int(num_splits),
                                             splits.ctypes.data, ctypes.addressof(split_len),
                                             ctypes.addressof(total), ctypes.addressof(mx),
                                             ctypes.addressof(ws))
    _check(rc, "gqa_attn_decode_plan")
    return {"splits": splits, "split_len": split_len.value, "total_splits": total.value,
            "max_splits": mx.value, "workspace_bytes": ws.value}


def decode_workspace_bytes(B, H_q, H_kv, d, kv_len, num_splits: int = 0) -> int:
    return decode_plan(B, H_q, H_kv, d, kv_len, num_splits)["workspace_bytes"]


def _decode_shapes(q, k, v, kv_len):
    _require(q, "q", 3)
    _require(k, "k", 3)
    _require(v, "v", 3)
    B, H_q, d = q.shape
    if k.shape != v.shape or k.shape[2] != d:
        raise GQAError("k and v must be [sum(kv_len), H_kv, d] matching q", 2)
    _same(q, k, v)
    a = _kv_len_array(kv_len, B)
    if int(a.astype(np.int64).sum()) != k.shape[0]:
        raise GQAError("k/v rows must equal sum(kv_len)", 2)
    return B, H_q, k.shape[1], d, a


def decode(q, k, v, kv_len, *, scale: float | None = None, num_splits: int = 0, out=None):
    """Split-KV GQA decode.  q [B,H_q,d] bf16, k/v packed [sum(kv_len),H_kv,d]."""
    import torch
    B, H_q, H_kv, d, a = _decode_shapes(q, k, v, kv_len)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, H_q, d))
    rc = load_library().gqa_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H_q, H_kv, d,
                                        a.ctypes.data, float(scale), int(num_splits),
                                        _dtype_code(q), _stream(q.device))
    _check(rc, "gqa_attn_decode")
    return out


def decode_noalloc(q, k, v, kv_len, *, scale: float | None = None, num_splits: int = 0,
                   out=None):
    """gqa_attn_decode_noalloc: decode whose partials live in the library's
    fixed per-device scratch (no device allocation by the library; pass
    ``out`` to avoid torch's).  Raises GQAError (status 4) when the split
    plan's partials exceed the scratch."""
    B, H_q, H_kv, d, a = _decode_shapes(q, k, v, kv_len)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, H_q, d))
    rc = load_library().gqa_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H_q,
                                                H_kv, d, a.ctypes.data, float(scale),
                                                int(num_splits), _dtype_code(q),
                                                _stream(q.device))
    _check(rc, "gqa_attn_decode_noalloc")
    return out


def release_workspace():
    """gqa_attn_release_workspace: wait for the current device and free the
    library-owned workspace buffers (the current one and those retired by
    growth).  Graphs captured from calls that used them must not be replayed
    afterwards."""
    _check(load_library().gqa_attn_release_workspace(), "gqa_attn_release_workspace")


def decode_multi(q, k, v, kv_len, *, scale: float | None = None, num_splits: int = 0,
                 out=None, lse=None, return_lse: bool = True):
    """Multi-token decode.  q [B,T_q,H_q,d] bf16 (T_q new tokens per sequence,
    already appended to the cache), k/v packed [sum(kv_len),H_kv,d].
    Returns (o [B,T_q,H_q,d], lse [B,T_q,H_q] fp32 or None)."""
    import torch
    _require(q, "q", 4)
    _require(k, "k", 3)
    _require(v, "v", 3)
    B, T_q, H_q, d = q.shape
    if k.shape != v.shape or k.shape[2] != d:
        raise GQAError("k and v must be [sum(kv_len), H_kv, d] matching q", 2)
    _same(q, k, v)
    a = _kv_len_array(kv_len, B)
    if int(a.astype(np.int64).sum()) != k.shape[0]:
        raise GQAError("k/v rows must equal sum(kv_len)", 2)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    rc = load_library().gqa_attn_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                              B, T_q, H_q, k.shape[1], d, a.ctypes.data,
                                              float(scale), int(num_splits), _dtype_code(q),
                                              _stream(q.device))
    _check(rc, "gqa_attn_decode_multi")
    return out, lse


def decode_quant(q, k_codes, v_codes, k_scale, v_scale, kv_len, *, kv_bits: int,
                 scale: float | None = None, num_splits: int = 0, out=None, lse=None,
                 return_lse: bool = True):
    """Decode over a quantised cache.  q [B,T_q,H_q,d] bf16; k_codes/v_codes
    int8 tensors [sum(kv_len), H_kv, d] (kv_bits=8) or uint8 [.., d/2] holding
    two int4 codes per byte (kv_bits=4, even channel in the low nibble);
    k_scale/v_scale fp32 [H_kv, d].  Returns (o, lse)."""
    import torch
    _require(q, "q", 4)
    _require(k_codes, "k_codes", 3)
    _require(v_codes, "v_codes", 3)
    B, T_q, H_q, d = q.shape
    width = d if kv_bits == 8 else d // 2
    if k_codes.shape != v_codes.shape or k_codes.shape[2] != width:
        raise GQAError(f"k/v codes must be [sum(kv_len), H_kv, {width}] bytes", 2)
    if k_codes.element_size() != 1 or v_codes.element_size() != 1:
        raise GQAError("k/v codes must be 1-byte tensors", 3)
    if q.dtype != torch.bfloat16:
        raise GQAError("q must be bf16", 3)
    H_kv = k_codes.shape[1]
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _require(t, name, 2)
        if t.dtype != torch.float32 or tuple(t.shape) != (H_kv, d) or t.device != q.device:
            raise GQAError(f"{name} must be fp32 [{H_kv}, {d}] on {q.device}", 2)
    a = _kv_len_array(kv_len, B)
    if int(a.astype(np.int64).sum()) != k_codes.shape[0]:
        raise GQAError("k/v rows must equal sum(kv_len)", 2)
    if k_codes.device != q.device or v_codes.device != q.device:
        raise GQAError(f"k/v codes must be on {q.device}", 2)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    rc = load_library().gqa_attn_decode_quant(
        _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        _ptr(lse), B, T_q, H_q, H_kv, d, a.ctypes.data, int(kv_bits), float(scale),
        int(num_splits), _stream(q.device))
    _check(rc, "gqa_attn_decode_quant")
    return out, lse


def decode_ring(q, k_cache, v_cache, kv_len, *, window: int, sink: int = 0,
                scale: float | None = None, num_splits: int = 0, out=None, lse=None,
                return_lse: bool = True):
    """Decode over a ring-buffer cache.  q [B,T_q,H_q,d] bf16 (T_q new tokens,
    already written); k_cache/v_cache [B,capacity,H_kv,d]; kv_len = tokens
    written per sequence.  Returns (o [B,T_q,H_q,d], lse [B,T_q,H_q] or None)."""
    import torch
    _require(q, "q", 4)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    B, T_q, H_q, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise GQAError("k_cache and v_cache must be [B, capacity, H_kv, d] matching q", 2)
    _same(q, k_cache, v_cache)
    a = _kv_len_array(kv_len, B)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    rc = load_library().gqa_attn_decode_ring(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, T_q, H_q,
        k_cache.shape[2], d, k_cache.shape[1], a.ctypes.data, int(window), int(sink),
        float(scale), int(num_splits), _dtype_code(q), _stream(q.device))
    _check(rc, "gqa_attn_decode_ring")
    return out, lse


def decode_ring_quant(q, k_codes, v_codes, k_scale, v_scale, kv_len, *, kv_bits: int,
                      window: int, sink: int = 0, scale: float | None = None,
                      num_splits: int = 0, out=None, lse=None, return_lse: bool = True):
    """Decode over a quantised ring-buffer cache.  q [B,T_q,H_q,d] bf16;
    k_codes/v_codes 1-byte tensors [B,capacity,H_kv,d] (int8, kv_bits=8) or
    [B,capacity,H_kv,d/2] (two int4 codes per byte, kv_bits=4); k_scale/v_scale
    fp32 [H_kv,d]; kv_len = tokens written per sequence.  Returns (o, lse)."""
    import torch
    _require(q, "q", 4)
    _require(k_codes, "k_codes", 4)
    _require(v_codes, "v_codes", 4)
    B, T_q, H_q, d = q.shape
    width = d if kv_bits == 8 else d // 2
    if (k_codes.shape != v_codes.shape or k_codes.shape[0] != B
            or k_codes.shape[3] != width):
        raise GQAError(f"k/v codes must be [B, capacity, H_kv, {width}] bytes", 2)
    if k_codes.element_size() != 1 or v_codes.element_size() != 1:
        raise GQAError("k/v codes must be 1-byte tensors", 3)
    if q.dtype != torch.bfloat16:
        raise GQAError("q must be bf16", 3)
    if k_codes.device != q.device or v_codes.device != q.device:
        raise GQAError(f"k/v codes must be on {q.device}", 2)
    H_kv = k_codes.shape[2]
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _require(t, name, 2)
        if t.dtype != torch.float32 or tuple(t.shape) != (H_kv, d) or t.device != q.device:
            raise GQAError(f"{name} must be fp32 [{H_kv}, {d}] on {q.device}", 2)
    a = _kv_len_array(kv_len, B)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(out, q, (B, T_q, H_q, d))
    lse = _lse_buf(lse, q, (B, T_q, H_q), return_lse)
    rc = load_library().gqa_attn_decode_ring_quant(
        _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        _ptr(lse), B, T_q, H_q, H_kv, d, k_codes.shape[1], a.ctypes.data, int(window),
        int(sink), int(kv_bits), float(scale), int(num_splits), _stream(q.device))
    _check(rc, "gqa_attn_decode_ring_quant")
    return out, lse


def decode_split(q, k, v, kv_len, workspace, *, scale: float | None = None, num_splits: int = 0):
    """Decode step 1: partials (m, l, O) into ``workspace`` (a uint8/float GPU tensor)."""
    B, H_q, H_kv, d, a = _decode_shapes(q, k, v, kv_len)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _require(workspace, "workspace", workspace.dim())
    if workspace.device != q.device:
        raise GQAError(f"workspace must be on {q.device}", 2)
    nbytes = workspace.numel() * workspace.element_size()
    rc = load_library().gqa_attn_decode_split(_ptr(q), _ptr(k), _ptr(v), _ptr(workspace), nbytes,
                                              B, H_q, H_kv, d, a.ctypes.data, float(scale),
                                              int(num_splits), _dtype_code(q), _stream(q.device))
    _check(rc, "gqa_attn_decode_split")


def decode_combine(workspace, kv_len, *, H_q: int, H_kv: int, d: int, out, lse=None,
                   num_splits: int = 0):
    """Decode step 2: merge the partials, normalise, write ``out`` [B,H_q,d]
    (and ``lse`` [B,H_q] fp32 if given)."""
    _require(out, "out", 3)
    B = out.shape[0]
    if tuple(out.shape[1:]) != (H_q, d):
        raise GQAError(f"out must be [B, {H_q}, {d}]", 2)
    a = _kv_len_array(kv_len, B)
    _require(workspace, "workspace", workspace.dim())
    if workspace.device != out.device:
        raise GQAError(f"workspace must be on {out.device}", 2)
    nbytes = workspace.numel() * workspace.element_size()
    lse = _lse_buf(lse, out, (B, H_q), False)
    rc = load_library().gqa_attn_decode_combine(_ptr(workspace), nbytes, _ptr(out), _ptr(lse), B,
                                                H_q, H_kv, d, a.ctypes.data, int(num_splits),
                                                _dtype_code(out), _stream(out.device))
    _check(rc, "gqa_attn_decode_combine")
