"""MI355X-native grouped-query fused attention (gfx950 HIP kernels).

The compute lives in ``libgqa_attn.so`` (hand-written HIP kernels behind a
C ABI, declared in include/gqa_attn.h).  ``binding`` is the thin ctypes layer
over it; importing this package does not load the library, the first call
does, and it raises if the library is missing -- there is no fallback path.
"""
from .binding import (GQAError, decode, decode_combine, decode_multi, decode_noalloc,  # noqa: F401
                      decode_plan,
                      decode_quant, decode_ring, decode_ring_quant,
                      decode_split,
                      decode_workspace_bytes, library_path, load_library, prefill,
                      prefill_kvsplit, prefill_kvsplit_count, prefill_window,
                      release_workspace)

__all__ = ["GQAError", "prefill", "prefill_window", "prefill_kvsplit", "prefill_kvsplit_count", "decode", "decode_noalloc", "decode_multi", "decode_quant", "decode_ring", "decode_ring_quant", "decode_split", "decode_combine",
           "decode_plan",
           "decode_workspace_bytes", "release_workspace", "load_library", "library_path"]
