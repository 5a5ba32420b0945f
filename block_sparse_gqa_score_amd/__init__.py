"""MiniMax-M3 two-step block-sparse GQA attention on MI355X (gfx950).

Thin ctypes binding over libmsa.so (C ABI in include/msa.h).  This module
only checks tensors, allocates outputs and workspaces with torch and passes
raw device pointers plus torch's current HIP stream; every step of the path
runs in the HIP kernels.  There is no fallback: if the library is missing
or no GPU is present the calls raise.

Entry points (names follow the C ABI):
  select_blocks(index_q, index_k, cu_seqlens, max_seqlen, topk=16,
                init_blocks=0, local_blocks=1, scores=False) -> q2k [4,T,topk]
  sparse_attend_prefill(q, k, v, q2k, cu_seqlens, max_seqlen, softmax_scale)
                -> out [T,64,128] bf16
  sparse_attend_decode_paged(q, index_q, k_cache, v_cache, index_k_cache,
                page_table, context_lens, max_context_len, topk=16,
                init_blocks=0, local_blocks=1, softmax_scale=None,
                return_q2k=False) -> out [B,64,128] (, q2k [4,B,topk])
  sparse_attend_decode_paged_mxfp8(same arguments)
                -> (out_q uint8 [B,8192] E4M3, out_scale uint8 [B,256] E8M0)
  mxfp8_quantize(x bf16 [rows, cols]) -> (q uint8 [rows, cols], scale uint8 [rows, cols/32])
  sparse_attend_decode_paged_fp8kv(q, index_q, k_cache, v_cache, k_scale, v_scale, index_k_cache,
                page_table, context_lens, max_context_len, ...) -> out [B,64,128]
                (K/V caches as E4M3 bytes with per-tensor scales)
  cache_insert(k, v, index_k, slot_mapping, k_cache, v_cache, index_k_cache) -> None (in place)
  validate_prefill_inputs(cu_seqlens, total_tokens, max_seqlen) -> (bits, first)
  validate_decode_inputs(page_table, context_lens, max_context_len, num_pages) -> (bits, first)
                (debug checks of the device-side data contract; bits 0 = valid)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "select_blocks", "sparse_attend_prefill", "sparse_attend_decode_paged",
    "sparse_attend_prefill_backward", "prefill_backward_workspace_bytes",
    "sparse_attend_decode_paged_mxfp8", "sparse_attend_decode_paged_fp8kv", "mxfp8_quantize",
    "cache_insert", "validate_prefill_inputs", "validate_decode_inputs", "INVALID_BITS",
    "unsupported_reason", "library_path", "MsaError",
    "select_blocks_workspace_bytes", "prefill_workspace_bytes", "decode_workspace_bytes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmsa.so")
_lib = None

MSA_INDEX_BF16, MSA_INDEX_FP8_E4M3 = 0, 1
_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED",
           3: "MSA_ERR_WORKSPACE", 4: "MSA_ERR_HIP"}


# msa_invalid_bits of the debug validators
INVALID_BITS = {1: "cu_seqlens[0] != 0", 2: "cu_seqlens[num_docs] != total_tokens",
                4: "empty document", 8: "document longer than max_seqlen",
                16: "offset outside [0, total_tokens]", 32: "context length outside [0, max_context_len]",
                64: "page id outside [0, num_pages)"}


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run `python -m block_sparse_gqa_score_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.msa_unsupported_reason.restype = ctypes.c_char_p
        L.msa_unsupported_reason.argtypes = [i] * 7
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_version.restype = i
        L.msa_select_blocks_workspace_bytes.restype = sz
        L.msa_select_blocks_workspace_bytes.argtypes = [i, i, i]
        L.msa_prefill_workspace_bytes.restype = sz
        L.msa_prefill_workspace_bytes.argtypes = [i, i, i]
        L.msa_decode_workspace_bytes.restype = sz
        L.msa_decode_workspace_bytes.argtypes = [i, i, i]
        L.msa_select_blocks.restype = i
        L.msa_select_blocks.argtypes = [P, P, i, P, i, i, i, i, i, i, P, P, P, sz, P]
        L.msa_sparse_attend_prefill.restype = i
        L.msa_sparse_attend_prefill.argtypes = [P, P, P, P, i, P, i, i, i, f, P, P, sz, P]
        L.msa_sparse_attend_prefill_lse.restype = i
        L.msa_sparse_attend_prefill_lse.argtypes = [P, P, P, P, i, P, i, i, i, f, P, P, P, sz, P]
        L.msa_prefill_backward_workspace_bytes.restype = sz
        L.msa_prefill_backward_workspace_bytes.argtypes = [i, i, i, i]
        L.msa_sparse_attend_prefill_backward.restype = i
        L.msa_sparse_attend_prefill_backward.argtypes = [P, P, P, P, P, P, P, i, P, i, i, i, f, P, P, P,
                                                         P, sz, P]
        L.msa_set_timing_events.restype = None
        L.msa_set_timing_events.argtypes = [P, i]
        L.msa_timing_kernel_count.restype = i
        L.msa_timing_kernel_count.argtypes = []
        L.msa_timing_kernel_name.restype = ctypes.c_char_p
        L.msa_timing_kernel_name.argtypes = [i]
        L.msa_sparse_attend_decode_paged.restype = i
        L.msa_sparse_attend_decode_paged.argtypes = [P, P, P, P, P, i, P, i, P, i, i, i, i, i, f,
                                                     P, P, P, sz, P]
        L.msa_sparse_attend_decode_paged_mxfp8.restype = i
        L.msa_sparse_attend_decode_paged_mxfp8.argtypes = [P, P, P, P, P, i, P, i, P, i, i, i, i, i, f,
                                                           P, P, P, P, sz, P]
        L.msa_mxfp8_quantize.restype = i
        L.msa_mxfp8_quantize.argtypes = [P, i, i, P, P, P]
        L.msa_sparse_attend_decode_paged_fp8kv.restype = i
        L.msa_sparse_attend_decode_paged_fp8kv.argtypes = [P, P, P, P, f, f, P, i, P, i, P, i, i, i, i, i,
                                                           f, P, P, P, sz, P]
        L.msa_cache_insert.restype = i
        L.msa_cache_insert.argtypes = [P, P, P, P, i, i, P, P, P, i, P]
        L.msa_sparse_attend_decode_paged_noalloc.restype = i
        L.msa_sparse_attend_decode_paged_noalloc.argtypes = [P, P, P, P, P, i, P, i, P, i, i, i, i, i, f,
                                                             P, P, P]
        L.msa_validate_prefill_inputs.restype = i
        L.msa_validate_prefill_inputs.argtypes = [P, i, i, i, P, P]
        L.msa_validate_decode_inputs.restype = i
        L.msa_validate_decode_inputs.argtypes = [P, i, P, i, i, i, P, P]
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MsaError(status, lib().msa_last_error().decode())


def unsupported_reason(num_heads=64, num_kv_heads=4, head_dim=128, num_index_heads=4,
                       index_dim=128, topk=16, block_size=128):
    r = lib().msa_unsupported_reason(num_heads, num_kv_heads, head_dim, num_index_heads,
                                     index_dim, topk, block_size)
    return None if r is None else r.decode()


def select_blocks_workspace_bytes(total_tokens, num_docs, max_seqlen) -> int:
    return int(lib().msa_select_blocks_workspace_bytes(total_tokens, num_docs, max_seqlen))


def prefill_workspace_bytes(total_tokens, num_docs, max_seqlen) -> int:
    return int(lib().msa_prefill_workspace_bytes(total_tokens, num_docs, max_seqlen))


def prefill_backward_workspace_bytes(total_tokens, num_docs, max_seqlen, topk) -> int:
    return int(lib().msa_prefill_backward_workspace_bytes(total_tokens, num_docs, max_seqlen, topk))


def decode_workspace_bytes(batch, max_context_len, topk) -> int:
    return int(lib().msa_decode_workspace_bytes(batch, max_context_len, topk))


# ---------------------------------------------------------------- helpers
def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(name, t, shape, dtypes, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype in {[str(d) for d in dtypes]} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_INDEX_DTYPES = (torch.bfloat16, torch.float8_e4m3fn, torch.uint8)


def _index_code(t):
    return MSA_INDEX_BF16 if t.dtype == torch.bfloat16 else MSA_INDEX_FP8_E4M3


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- API
def select_blocks(index_q, index_k, cu_seqlens, max_seqlen, topk=16, init_blocks=0,
                  local_blocks=1, scores=False, workspace=None):
    """Index-branch block selection -> int32 q2k [4, T, topk] (see msa.h).

    ``index_q`` [T,4,128] and ``index_k`` [T,1,128] are bf16, or E4M3
    (torch.float8_e4m3fn or raw uint8 bytes).  With ``scores=True`` also
    returns the fp32 block scores [4, ceil(max_seqlen/128), T]."""
    device = index_q.device
    T = int(index_q.shape[0])
    _dev_tensor("index_q", index_q, (T, 4, 128), _INDEX_DTYPES)
    _dev_tensor("index_k", index_k, (T, 1, 128), (index_q.dtype,), device)
    _dev_tensor("cu_seqlens", cu_seqlens, None, (torch.int32,), device)
    ndocs = int(cu_seqlens.numel()) - 1
    q2k = torch.empty((4, T, topk), dtype=torch.int32, device=device)
    S = None
    if scores:
        S = torch.empty((4, math.ceil(max_seqlen / 128), T), dtype=torch.float32, device=device)
    need = select_blocks_workspace_bytes(T, max(ndocs, 1), int(max_seqlen)) if ndocs >= 1 else 0
    if workspace is None:
        workspace = _workspace(need, device)
    _check(lib().msa_select_blocks(_ptr(index_q), _ptr(index_k), _index_code(index_q),
                                   _ptr(cu_seqlens), ndocs, T, int(max_seqlen), int(topk),
                                   int(init_blocks), int(local_blocks), _ptr(q2k), _ptr(S),
                                   _ptr(workspace), workspace.numel(), _stream(device)))
    return (q2k, S) if scores else q2k


def _check_attention_args(q, k, v, q2k, cu_seqlens):
    device = q.device
    T = int(q.shape[0])
    _dev_tensor("q", q, (T, 64, 128), (torch.bfloat16,))
    _dev_tensor("k", k, (T, 4, 128), (torch.bfloat16,), device)
    _dev_tensor("v", v, (T, 4, 128), (torch.bfloat16,), device)
    if q2k.dim() != 3 or q2k.shape[0] != 4 or q2k.shape[1] != T:
        raise ValueError(f"q2k must have shape [4, {T}, topk] (got {tuple(q2k.shape)})")
    _dev_tensor("q2k", q2k, None, (torch.int32,), device)
    _dev_tensor("cu_seqlens", cu_seqlens, None, (torch.int32,), device)
    return device, T, int(cu_seqlens.numel()) - 1


def sparse_attend_prefill(q, k, v, q2k, cu_seqlens, max_seqlen, softmax_scale=None,
                          workspace=None, return_lse=False):
    """Sparse GQA attention over the selected blocks -> bf16 out [T,64,128]
    (with ``return_lse``: (out, fp32 lse [T,64]) for the backward)."""
    device, T, ndocs = _check_attention_args(q, k, v, q2k, cu_seqlens)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128.0)
    out = torch.empty((T, 64, 128), dtype=torch.bfloat16, device=device)
    need = prefill_workspace_bytes(T, max(ndocs, 1), int(max_seqlen)) if ndocs >= 1 else 0
    if workspace is None:
        workspace = _workspace(need, device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(q2k), int(q2k.shape[2]), _ptr(cu_seqlens), ndocs, T,
            int(max_seqlen), float(softmax_scale), _ptr(out))
    tail = (_ptr(workspace), workspace.numel(), _stream(device))
    if return_lse:
        lse = torch.empty((T, 64), dtype=torch.float32, device=device)
        _check(lib().msa_sparse_attend_prefill_lse(*args, _ptr(lse), *tail))
        return out, lse
    _check(lib().msa_sparse_attend_prefill(*args, *tail))
    return out


def sparse_attend_prefill_backward(q, k, v, out, lse, dout, q2k, cu_seqlens, max_seqlen,
                                   softmax_scale=None, workspace=None):
    """Gradients of the sparse prefill attention for a fixed q2k -> (dq [T,64,128],
    dk [T,4,128], dv [T,4,128]) bf16.  ``out`` and ``lse`` come from
    ``sparse_attend_prefill(..., return_lse=True)``; ``dout`` is d(loss)/d(out)."""
    device, T, ndocs = _check_attention_args(q, k, v, q2k, cu_seqlens)
    _dev_tensor("out", out, (T, 64, 128), (torch.bfloat16,), device)
    _dev_tensor("lse", lse, (T, 64), (torch.float32,), device)
    _dev_tensor("dout", dout, (T, 64, 128), (torch.bfloat16,), device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128.0)
    topk = int(q2k.shape[2])
    dq = torch.empty((T, 64, 128), dtype=torch.bfloat16, device=device)
    dk = torch.empty((T, 4, 128), dtype=torch.bfloat16, device=device)
    dv = torch.empty((T, 4, 128), dtype=torch.bfloat16, device=device)
    need = (prefill_backward_workspace_bytes(T, max(ndocs, 1), int(max_seqlen), topk)
            if ndocs >= 1 else 0)
    if workspace is None:
        workspace = _workspace(need, device)
    _check(lib().msa_sparse_attend_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(q2k), topk,
        _ptr(cu_seqlens), ndocs, T, int(max_seqlen), float(softmax_scale), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), workspace.numel(), _stream(device)))
    return dq, dk, dv


def sparse_attend_decode_paged(q, index_q, k_cache, v_cache, index_k_cache, page_table,
                               context_lens, max_context_len, topk=16, init_blocks=0,
                               local_blocks=1, softmax_scale=None, return_q2k=False,
                               workspace=None):
    """One decode step over the paged caches -> bf16 out [B,64,128] (, q2k [4,B,topk])."""
    return _decode(q, index_q, k_cache, v_cache, index_k_cache, page_table, context_lens,
                   max_context_len, topk, init_blocks, local_blocks, softmax_scale, return_q2k,
                   workspace, mxfp8=False)


def sparse_attend_decode_paged_mxfp8(q, index_q, k_cache, v_cache, index_k_cache, page_table,
                                     context_lens, max_context_len, topk=16, init_blocks=0,
                                     local_blocks=1, softmax_scale=None, return_q2k=False,
                                     workspace=None):
    """One decode step with the output as MXFP8 -> (out_q uint8 [B, 8192] E4M3,
    out_scale uint8 [B, 256] E8M0) (, q2k [4,B,topk])."""
    return _decode(q, index_q, k_cache, v_cache, index_k_cache, page_table, context_lens,
                   max_context_len, topk, init_blocks, local_blocks, softmax_scale, return_q2k,
                   workspace, mxfp8=True)


def sparse_attend_decode_paged_fp8kv(q, index_q, k_cache, v_cache, k_scale, v_scale, index_k_cache,
                                     page_table, context_lens, max_context_len, topk=16, init_blocks=0,
                                     local_blocks=1, softmax_scale=None, return_q2k=False,
                                     workspace=None):
    """One decode step over E4M3 K/V caches [slots,4,128] (torch.float8_e4m3fn or uint8) with
    per-tensor scales (K = e4m3 * k_scale, V = e4m3 * v_scale) -> bf16 out [B,64,128]."""
    return _decode(q, index_q, k_cache, v_cache, index_k_cache, page_table, context_lens,
                   max_context_len, topk, init_blocks, local_blocks, softmax_scale, return_q2k,
                   workspace, mxfp8=False, kv_scales=(float(k_scale), float(v_scale)))


def mxfp8_quantize(x):
    """MXFP8 of a bf16 matrix [rows, cols] (cols % 32 == 0) -> (q uint8 [rows, cols] E4M3,
    scale uint8 [rows, cols/32] E8M0)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = int(x.shape[0]), int(x.shape[1])
    _dev_tensor("x", x, (rows, cols), (torch.bfloat16,))
    if cols % 32 or cols == 0:
        raise ValueError(f"cols must be a positive multiple of 32 (got {cols})")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scale = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check(lib().msa_mxfp8_quantize(_ptr(x), rows, cols, _ptr(q), _ptr(scale), _stream(x.device)))
    return q, scale


def cache_insert(k, v, index_k, slot_mapping, k_cache, v_cache, index_k_cache):
    """Write tokens' K/V [N,4,128] and index-K [N,1,128] rows (bf16, normed and RoPE'd) into
    the paged caches at slot_mapping[n] (negative = skip).  index_k_cache is bf16, or
    E4M3 (torch.float8_e4m3fn / uint8) to store unscaled E4M3.  In place."""
    device = k.device
    N = int(k.shape[0])
    _dev_tensor("k", k, (N, 4, 128), (torch.bfloat16,))
    _dev_tensor("v", v, (N, 4, 128), (torch.bfloat16,), device)
    _dev_tensor("index_k", index_k, (N, 1, 128), (torch.bfloat16,), device)
    _dev_tensor("slot_mapping", slot_mapping, (N,), (torch.int32,), device)
    slots = int(k_cache.shape[0])
    _dev_tensor("k_cache", k_cache, (slots, 4, 128), (torch.bfloat16,), device)
    _dev_tensor("v_cache", v_cache, (slots, 4, 128), (torch.bfloat16,), device)
    _dev_tensor("index_k_cache", index_k_cache, (slots, 1, 128), _INDEX_DTYPES, device)
    _check(lib().msa_cache_insert(_ptr(k), _ptr(v), _ptr(index_k), _ptr(slot_mapping), N,
                                  _index_code(index_k_cache), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(index_k_cache), slots, _stream(device)))


def validate_prefill_inputs(cu_seqlens, total_tokens, max_seqlen):
    """Debug check of a document map on the device -> (bits, first): the OR of
    the violated rules (INVALID_BITS; 0 = valid) and the lowest offending
    document (-1 when valid).  Synchronises to read the result back."""
    _dev_tensor("cu_seqlens", cu_seqlens, None, (torch.int32,))
    status = torch.empty(2, dtype=torch.int32, device=cu_seqlens.device)
    _check(lib().msa_validate_prefill_inputs(_ptr(cu_seqlens), int(cu_seqlens.numel()) - 1,
                                             int(total_tokens), int(max_seqlen), _ptr(status),
                                             _stream(cu_seqlens.device)))
    bits, first = status.tolist()
    return int(bits), int(first)


def validate_decode_inputs(page_table, context_lens, max_context_len, num_pages):
    """Debug check of a decode batch's page table and context lengths on the
    device -> (bits, first): INVALID_BITS (0 = valid) and the lowest offending
    request (-1 when valid).  Synchronises to read the result back."""
    device = page_table.device
    if page_table.dim() != 2:
        raise ValueError("page_table must be 2-D [B, max_pages]")
    B = int(page_table.shape[0])
    _dev_tensor("page_table", page_table, None, (torch.int32,))
    _dev_tensor("context_lens", context_lens, (B,), (torch.int32,), device)
    status = torch.empty(2, dtype=torch.int32, device=device)
    _check(lib().msa_validate_decode_inputs(_ptr(page_table), int(page_table.shape[1]),
                                            _ptr(context_lens), B, int(max_context_len),
                                            int(num_pages), _ptr(status), _stream(device)))
    bits, first = status.tolist()
    return int(bits), int(first)


def _decode(q, index_q, k_cache, v_cache, index_k_cache, page_table, context_lens, max_context_len,
            topk, init_blocks, local_blocks, softmax_scale, return_q2k, workspace, mxfp8,
            kv_scales=None):
    device = q.device
    B = int(q.shape[0])
    _dev_tensor("q", q, (B, 64, 128), (torch.bfloat16,))
    _dev_tensor("index_q", index_q, (B, 4, 128), _INDEX_DTYPES, device)
    slots = int(k_cache.shape[0])
    kv_types = (torch.bfloat16,) if kv_scales is None else (torch.float8_e4m3fn, torch.uint8)
    _dev_tensor("k_cache", k_cache, (slots, 4, 128), kv_types, device)
    _dev_tensor("v_cache", v_cache, (slots, 4, 128), kv_types, device)
    _dev_tensor("index_k_cache", index_k_cache, (slots, 1, 128), (index_q.dtype,), device)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError(f"page_table must have shape [{B}, max_pages]")
    _dev_tensor("page_table", page_table, None, (torch.int32,), device)
    _dev_tensor("context_lens", context_lens, (B,), (torch.int32,), device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128.0)
    q2k = torch.empty((4, B, topk), dtype=torch.int32, device=device) if return_q2k else None
    need = decode_workspace_bytes(B, int(max_context_len), int(topk))
    if workspace is None:
        workspace = _workspace(need, device)
    rest = (_ptr(index_k_cache), _index_code(index_q), _ptr(page_table), int(page_table.shape[1]),
            _ptr(context_lens), B, int(max_context_len), int(topk), int(init_blocks), int(local_blocks),
            float(softmax_scale))
    head = (_ptr(q), _ptr(index_q), _ptr(k_cache), _ptr(v_cache)) + rest
    tail = (_ptr(q2k), _ptr(workspace), workspace.numel(), _stream(device))
    if kv_scales is not None:
        out = torch.empty((B, 64, 128), dtype=torch.bfloat16, device=device)
        _check(lib().msa_sparse_attend_decode_paged_fp8kv(_ptr(q), _ptr(index_q), _ptr(k_cache),
                                                          _ptr(v_cache), *kv_scales, *rest, _ptr(out),
                                                          *tail))
    elif mxfp8:
        out_q = torch.empty((B, 64 * 128), dtype=torch.uint8, device=device)
        out_scale = torch.empty((B, 64 * 128 // 32), dtype=torch.uint8, device=device)
        _check(lib().msa_sparse_attend_decode_paged_mxfp8(*head, _ptr(out_q), _ptr(out_scale), *tail))
        out = (out_q, out_scale)
    else:
        out = torch.empty((B, 64, 128), dtype=torch.bfloat16, device=device)
        _check(lib().msa_sparse_attend_decode_paged(*head, _ptr(out), *tail))
    return (out, q2k) if return_q2k else out
