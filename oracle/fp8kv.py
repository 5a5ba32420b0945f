"""Decode attention over an FP8 main K/V cache (E4M3FN bytes, per-tensor
scales): fp64, literal definition, numpy.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may use this module; the product path never
does.

What it computes (TensorRT-LLM "MiniMaxM3SparseAttentionConfig",
fuse_qkv_index_projection: the MiniMax-M3 MSA path runs with an FP8 main KV
cache).  The page does not give the cache's scaling; this reads it as the
per-tensor scheme: K = e4m3(byte) * k_scale, V = e4m3(byte) * v_scale.  The
attention is the decode step of the bf16 cache (query at position L-1, keys
of the selected document-local blocks up to L-1, softmax of scale * q.k) on
those dequantised values.
"""
from __future__ import annotations

import numpy as np

from .mxfp8 import e4m3fn_value


def dequantize(cache_bytes: np.ndarray, scale: float) -> np.ndarray:
    """fp64 values of an E4M3FN cache with one scale."""
    return e4m3fn_value(cache_bytes) * float(scale)


def decode_attend(q_f64, k_f64, v_f64, page_table, context_lens, q2k_rows, scale) -> np.ndarray:
    """out [B,64,128] fp64 for queries q_f64 [B,64,128] over dequantised caches
    k_f64, v_f64 [slots,4,128]; q2k_rows [B,4,topk] document-local block ids
    (ids outside 0..c and -1 select nothing; repeats count once)."""
    B = len(context_lens)
    out = np.zeros((B, 64, 128), dtype=np.float64)
    for r in range(B):
        L = int(context_lens[r])
        c = (L - 1) // 128
        j = np.arange(L)
        for g in range(4):
            sel = {int(b) for b in q2k_rows[r, g] if 0 <= b <= c}
            keys = j[np.isin(j // 128, sorted(sel))]
            if len(keys) == 0:
                continue
            slots = page_table[r, keys // 128].astype(np.int64) * 128 + keys % 128
            K, V = k_f64[slots, g], v_f64[slots, g]             # [n, 128]
            s = scale * (K @ q_f64[r, 16 * g:16 * g + 16].T)    # [n, 16]
            p = np.exp(s - s.max(axis=0, keepdims=True))
            p /= p.sum(axis=0, keepdims=True)
            out[r, 16 * g:16 * g + 16] = p.T @ V
    return out
