"""Seeded synthetic inputs for the GQA attention workloads.

This module holds no attention arithmetic: it only draws random tensors and
rounds them to the storage type, so that the HIP path and the CPU oracle can
be fed the very same bytes.  It imports nothing else from this package.

Recipe (identical for every workload):
  rng = numpy.random.default_rng(seed)          # PCG64, default seed 0
  kv_len   (varlen decode only) rng.integers(lo, hi, endpoint=True, size=B)
  Q, K, V  rng.standard_normal(shape, dtype=float32), drawn in that order
  bf16 workloads: each value rounded to bfloat16, round-to-nearest-even.
The shapes are the Llama3-70B attention geometry the ADR-0060 page uses
(section 0, reference dimensions: H_q = 64, H_kv = 8, d = 128), plus one tiny
fp32 case.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str               # "prefill" or "decode"
    dtype: str              # "bf16" or "f32"
    B: int
    H_q: int
    H_kv: int
    d: int
    T_q: int = 1            # prefill query rows, or new tokens per sequence in decode
    S_kv: int = 0           # prefill keys, or fixed decode length
    causal: bool = False
    q_offset: int = 0
    kv_len_range: tuple | None = None   # varlen decode: (lo, hi) inclusive
    window: int = 0         # > 0: sink + local-window mask (keys j < sink or j > p - window)
    sink: int = 0
    capacity: int = 0       # > 0: decode over a ring-buffer cache of this many slots
    kv_bits: int = 16       # 8 / 4: quantised K/V codes with per-channel scales

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))


WORKLOADS = {
    w.name: w for w in [
        Workload("prefill_tiny_f32", "prefill", "f32", B=1, H_q=8, H_kv=1, d=64,
                 T_q=128, S_kv=128, causal=True),
        Workload("decode_8k", "decode", "bf16", B=1, H_q=64, H_kv=8, d=128, S_kv=8192),
        Workload("decode_varlen_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 kv_len_range=(1024, 32768)),
        Workload("prefill_8k_causal", "prefill", "bf16", B=1, H_q=64, H_kv=8, d=128,
                 T_q=8192, S_kv=8192, causal=True),
        Workload("decode_128k", "decode", "bf16", B=1, H_q=64, H_kv=8, d=128, S_kv=131072),
        Workload("prefill_chunk_64k", "prefill", "bf16", B=1, H_q=64, H_kv=8, d=128,
                 T_q=2048, S_kv=67584, causal=True, q_offset=65536),
        Workload("prefill_chunk_256_64k", "prefill", "bf16", B=1, H_q=64, H_kv=8, d=128,
                 T_q=256, S_kv=65792, causal=True, q_offset=65536),
        Workload("prefill_8k_window1k", "prefill", "bf16", B=1, H_q=64, H_kv=8, d=128,
                 T_q=8192, S_kv=8192, causal=True, window=1024, sink=4),
        Workload("decode_ring_8k_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 kv_len_range=(1024, 32768), capacity=8192, window=8188, sink=4),
        Workload("decode_int8_varlen_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 kv_len_range=(1024, 32768), kv_bits=8),
        Workload("decode_int4_varlen_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 kv_len_range=(1024, 32768), kv_bits=4),
        Workload("decode_t4_varlen_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 T_q=4, kv_len_range=(1024, 32768)),
        Workload("decode_t16_varlen_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 T_q=16, kv_len_range=(1024, 32768)),
        Workload("decode_t32_varlen_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 T_q=32, kv_len_range=(1024, 32768)),
        # the pccx base configuration: INT4 KV in an 8192-token hard-cap ring
        Workload("decode_ring_int4_b16", "decode", "bf16", B=16, H_q=64, H_kv=8, d=128,
                 kv_len_range=(1024, 32768), capacity=8192, window=8188, sink=4, kv_bits=4),
    ]
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exactly equal float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """q, k, v as float32 arrays holding exactly the stored values, plus the
    raw storage bits (uint16 for bf16, the float32 arrays themselves for f32)."""
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_store: np.ndarray
    k_store: np.ndarray
    v_store: np.ndarray
    kv_len: np.ndarray | None = None    # int32 [B], decode only


def kv_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.kind != "decode":
        return None
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        return rng.integers(lo, hi, endpoint=True, size=w.B).astype(np.int32)
    return np.full((w.B,), w.S_kv, np.int32)


def shapes(w: Workload, kv_len: np.ndarray | None):
    if w.kind == "prefill":
        return ((w.B, w.T_q, w.H_q, w.d), (w.B, w.S_kv, w.H_kv, w.d))
    total = int(np.asarray(kv_len, np.int64).sum())
    if w.capacity > 0:     # ring-buffer cache [B, capacity, H_kv, d], kv_len = tokens written
        return ((w.B, w.T_q, w.H_q, w.d), (w.B, w.capacity, w.H_kv, w.d))
    if w.T_q > 1:   # multi-token decode: T_q new tokens per sequence
        return ((w.B, w.T_q, w.H_q, w.d), (total, w.H_kv, w.d))
    return ((w.B, w.H_q, w.d), (total, w.H_kv, w.d))


def make(w: Workload | str, seed: int = 0) -> Inputs:
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(seed)
    kv_len = kv_lengths(w, rng)
    qs, ks = shapes(w, kv_len)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    if w.dtype == "bf16":
        qb, kb, vb = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
        return Inputs(w, bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                      qb, kb, vb, kv_len)
    return Inputs(w, q, k, v, q, k, v, kv_len)


def random_case(kind: str, dtype: str, *, B: int, H_q: int, H_kv: int, d: int, T_q: int = 1,
                S_kv: int = 0, kv_len=None, seed: int = 0, q_scale: float = 1.0) -> Inputs:
    """A seeded case of arbitrary shape (tests).  ``q_scale`` multiplies Q
    before rounding (peaky softmax inputs)."""
    w = Workload("custom", kind, dtype, B=B, H_q=H_q, H_kv=H_kv, d=d, T_q=T_q, S_kv=S_kv)
    rng = np.random.default_rng(seed)
    if kind == "decode":
        kv_len = np.asarray(kv_len if kv_len is not None else [S_kv] * B, np.int32)
    qs, ks = shapes(w, kv_len)
    q = rng.standard_normal(qs, dtype=np.float32) * np.float32(q_scale)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    if dtype == "bf16":
        qb, kb, vb = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
        return Inputs(w, bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                      qb, kb, vb, kv_len)
    return Inputs(w, q, k, v, q, k, v, kv_len)


@dataclasses.dataclass
class QuantInputs:
    """A quantised-cache decode case: bf16 queries, integer K/V codes and
    per-(KV head, channel) scales.  Codes are int8 [N, H_kv, d] (kv_bits 8)
    or unpacked int4 values in int8 [N, H_kv, d] (kv_bits 4; ``pack_int4``
    gives the two-per-byte storage).  Scales are bfloat16-representable fp32,
    so that code * scale is exact in float32."""
    workload: Workload
    q: np.ndarray
    q_store: np.ndarray
    k_codes: np.ndarray
    v_codes: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray
    kv_len: np.ndarray


def quant_case(*, B: int, H_q: int, H_kv: int, d: int, kv_len, kv_bits: int, T_q: int = 1,
               seed: int = 0, name: str = "custom", capacity: int = 0) -> QuantInputs:
    """Seeded quantised-cache case.  Draw order: kv_len (if a range workload
    drew it), Q, K codes, V codes, K scales, V scales.  Codes are rounded
    normals clipped to the code range (sigma = 127/4 for int8, 7/3 for int4);
    scales are bf16(uniform(0.5, 1.5) * 4/127) or bf16(uniform(0.5, 1.5) * 3/7),
    so values are roughly standard normal."""
    rng = np.random.default_rng(seed)
    return _quant_draw(rng, Workload(name, "decode", "bf16", B=B, H_q=H_q, H_kv=H_kv, d=d,
                                     T_q=T_q, kv_bits=kv_bits, capacity=capacity),
                       np.asarray(kv_len, np.int32))


def _quant_draw(rng, w: Workload, kv_len: np.ndarray) -> QuantInputs:
    total = int(kv_len.astype(np.int64).sum())
    # packed cache [sum kv_len, H_kv, d]; ring cache [B, capacity, H_kv, d]
    rows = (w.B, w.capacity) if w.capacity > 0 else (total,)
    qs = (w.B, w.T_q, w.H_q, w.d)
    q = rng.standard_normal(qs, dtype=np.float32)
    lo, hi, sigma, unit = (-128, 127, 127 / 4, 4 / 127) if w.kv_bits == 8 else (-8, 7, 7 / 3, 3 / 7)
    codes = []
    for _ in range(2):
        c = np.rint(rng.standard_normal(rows + (w.H_kv, w.d)) * sigma)
        codes.append(np.clip(c, lo, hi).astype(np.int8))
    scales = []
    for _ in range(2):
        sc = (rng.uniform(0.5, 1.5, size=(w.H_kv, w.d)) * unit).astype(np.float32)
        scales.append(bf16_bits_to_f32(bf16_round_bits(sc)))
    qb = bf16_round_bits(q)
    return QuantInputs(w, bf16_bits_to_f32(qb), qb, codes[0], codes[1], scales[0], scales[1],
                       kv_len)


def make_quant(name: str, seed: int = 0) -> QuantInputs:
    w = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    return _quant_draw(rng, w, kv_lengths(w, rng))


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int4 codes int8 [..., d] in [-8, 7] -> uint8 [..., d/2], channel 2i in
    the low nibble of byte i (two's complement nibbles)."""
    u = codes.astype(np.uint8) & np.uint8(0x0F)
    return (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)


def rows_per_workgroup(B: int, T_q: int, H_q: int, H_kv: int, seed: int = 0,
                       block_rows: int = 256) -> np.ndarray:
    """Flat output-row indices ((b * T_q + t) * H_q + h) for sampled parity
    checks of a full-size prefill: one random row from every (batch entry, KV
    head, block of `block_rows` folded rows), where the G query heads of a KV
    head are folded t-major (folded row t * G + g, query head kv * G + g), so
    every prefill work-group contributes a row, plus the first and last rows."""
    G = H_q // H_kv
    rng = np.random.default_rng(seed)
    n_fold = T_q * G
    n_blk = -(-n_fold // block_rows)
    out = [0, B * T_q * H_q - 1]
    for b in range(B):
        for kv in range(H_kv):
            lo = np.arange(n_blk, dtype=np.int64) * block_rows
            hi = np.minimum(lo + block_rows, n_fold)
            i = lo + (rng.random(n_blk) * (hi - lo)).astype(np.int64)
            t, g = i // G, i % G
            out.extend(((b * T_q + t) * H_q + kv * G + g).tolist())
    return np.unique(np.asarray(out, np.int64))

