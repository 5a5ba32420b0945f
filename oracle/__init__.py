"""CPU oracle for the MiniMax-M3 two-step block-sparse GQA attention.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path
(``block_sparse_gqa_score_amd``) never does.  The arithmetic lives in
``msa_oracle.c`` (fp64, OpenMP over rows, no code shared with the HIP
library); this module builds it with gcc and marshals numpy arrays.

Layouts returned here are token-major, ``[n, 4, ...]``; the tests transpose
to the library's head-major ``[4, T, ...]`` where they compare.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None

BF16, E4M3 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict fp64: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra", "-Werror",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_query_blocks.argtypes = [P, i, P, i, P]
        L.oracle_scores.argtypes = [P, P, i, P, i, P, i, i, P]
        L.oracle_select.argtypes = [P, P, i, i, i, i, i, P, P]
        L.oracle_attend.argtypes = [P, P, P, P, i, P, i, P, i, ctypes.c_double, P]
        L.oracle_attend_backward_rows.argtypes = [P, P, P, P, P, i, P, i, P, i, ctypes.c_double,
                                                  P, P, P]
        L.oracle_attend_backward_keys.argtypes = [P, P, P, P, P, i, P, i, P, P, ctypes.c_double,
                                                  P, i, P, P]
        L.oracle_decode_query_blocks.argtypes = [P, i, P]
        L.oracle_decode_scores.argtypes = [P, P, i, P, i, P, i, i, P]
        L.oracle_decode_attend.argtypes = [P, P, P, P, i, P, i, P, i, ctypes.c_double, P]
        L.oracle_num_threads.restype = i
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(index_dtype: str) -> int:
    return {"bf16": BF16, "fp8": E4M3}[index_dtype]


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (code {rc})")


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---- prefill -----------------------------------------------------------------
def query_blocks(cu, tokens) -> np.ndarray:
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    c = np.empty(len(tokens), dtype=np.int32)
    _check(lib().oracle_query_blocks(_p(cu), len(cu) - 1, _p(tokens), len(tokens), _p(c)),
           "query_blocks")
    return c


def scores(iq, ik, cu, tokens, nb_max, index_dtype="bf16") -> np.ndarray:
    """fp64 [n, 4, nb_max] block scores of the listed tokens (-inf = not a candidate)."""
    iq = np.ascontiguousarray(iq)
    ik = np.ascontiguousarray(ik)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    S = np.empty((len(tokens), 4, nb_max), dtype=np.float64)
    _check(lib().oracle_scores(_p(iq), _p(ik), _dtype_code(index_dtype), _p(cu), len(cu) - 1,
                               _p(tokens), len(tokens), int(nb_max), _p(S)), "scores")
    return S


def select(S, c, topk, init_blocks, local_blocks):
    """(q2k int32 [n,4,topk], margin fp64 [n,4]) from scores and query blocks."""
    S = np.ascontiguousarray(S, dtype=np.float64)
    c = np.ascontiguousarray(c, dtype=np.int32)
    n, _, nb_max = S.shape
    q2k = np.empty((n, 4, topk), dtype=np.int32)
    margin = np.empty((n, 4), dtype=np.float64)
    _check(lib().oracle_select(_p(S), _p(c), n, nb_max, int(topk), int(init_blocks),
                               int(local_blocks), _p(q2k), _p(margin)), "select")
    return q2k, margin


def attend(q, k, v, q2k_rows, cu, tokens, scale) -> np.ndarray:
    """fp64 [n, 64, 128] attention of the listed tokens; ``q2k_rows`` is [n,4,topk]."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    q2k_rows = np.ascontiguousarray(q2k_rows, dtype=np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.empty((len(tokens), 64, 128), dtype=np.float64)
    _check(lib().oracle_attend(_p(q), _p(k), _p(v), _p(q2k_rows), q2k_rows.shape[2], _p(cu),
                               len(cu) - 1, _p(tokens), len(tokens), float(scale), _p(out)),
           "attend")
    return out


def attend_backward_rows(q, k, v, dout, q2k_full, cu, tokens, scale):
    """Backward phase 1 for the listed tokens: (lse, D) fp64 [n,64] and dq
    fp64 [n,64,128].  ``q2k_full`` is token-major [T,4,topk] (every token)."""
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    q2k_full = np.ascontiguousarray(q2k_full, dtype=np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(tokens)
    lse = np.empty((n, 64), dtype=np.float64)
    D = np.empty((n, 64), dtype=np.float64)
    dq = np.empty((n, 64, 128), dtype=np.float64)
    _check(lib().oracle_attend_backward_rows(_p(q), _p(k), _p(v), _p(dout), _p(q2k_full),
                                             q2k_full.shape[2], _p(cu), len(cu) - 1, _p(tokens), n,
                                             float(scale), _p(lse), _p(D), _p(dq)), "backward rows")
    return lse, D, dq


def attend_backward_keys(q, k, v, dout, q2k_full, cu, lse_full, D_full, keys, scale):
    """Backward phase 2 for the listed keys: dk, dv fp64 [n,4,128].  ``lse_full``
    and ``D_full`` are [T,64]; only rows of tokens that attend to the keys are read."""
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    q2k_full = np.ascontiguousarray(q2k_full, dtype=np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    lse_full = np.ascontiguousarray(lse_full, dtype=np.float64)
    D_full = np.ascontiguousarray(D_full, dtype=np.float64)
    keys = np.ascontiguousarray(keys, dtype=np.int32)
    n = len(keys)
    dk = np.empty((n, 4, 128), dtype=np.float64)
    dv = np.empty((n, 4, 128), dtype=np.float64)
    _check(lib().oracle_attend_backward_keys(_p(q), _p(k), _p(v), _p(dout), _p(q2k_full),
                                             q2k_full.shape[2], _p(cu), len(cu) - 1, _p(lse_full),
                                             _p(D_full), float(scale), _p(keys), n, _p(dk), _p(dv)),
           "backward keys")
    return dk, dv


def attend_backward(q, k, v, dout, q2k_full, cu, scale, keys=None):
    """Whole backward over every token: dict(lse, D [T,64], dq [T,64,128],
    dk, dv [T,4,128] (or [len(keys),4,128] for the listed keys))."""
    T = int(np.asarray(cu)[-1])
    tokens = np.arange(T, dtype=np.int32)
    lse, D, dq = attend_backward_rows(q, k, v, dout, q2k_full, cu, tokens, scale)
    if keys is None:
        keys = tokens
    dk, dv = attend_backward_keys(q, k, v, dout, q2k_full, cu, lse, D, keys, scale)
    return dict(lse=lse, D=D, dq=dq, dk=dk, dv=dv)


def prefill(w, tokens=None, q2k_override=None):
    """Whole prefill path on a ``workloads.Prefill`` for the listed tokens.

    Returns dict(S, c, q2k [n,4,topk], margin, out [n,64,128]).  With
    ``q2k_override`` ([n,4,topk]) attention uses those rows instead."""
    r = prefill_select(w, tokens)
    rows = r["q2k"] if q2k_override is None else q2k_override
    r["out"] = attend(w.q, w.k, w.v, rows, w.cu_seqlens, r["tokens"], w.scale)
    return r


def prefill_select(w, tokens=None):
    """Scores and selection only: dict(S, c, q2k [n,4,topk], margin, tokens)."""
    if tokens is None:
        tokens = np.arange(w.T, dtype=np.int32)
    tokens = np.asarray(tokens, dtype=np.int32)
    nb_max = (w.max_seqlen + 127) // 128
    S = scores(w.iq, w.ik, w.cu_seqlens, tokens, nb_max, w.index_dtype)
    c = query_blocks(w.cu_seqlens, tokens)
    q2k, margin = select(S, c, w.topk, w.init_blocks, w.local_blocks)
    return dict(S=S, c=c, q2k=q2k, margin=margin, tokens=tokens)


# ---- decode ------------------------------------------------------------------
def decode_scores(iq, ik_cache, page_table, context_lens, nb_max, index_dtype="bf16"):
    iq = np.ascontiguousarray(iq)
    ik_cache = np.ascontiguousarray(ik_cache)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    B = len(ctx)
    S = np.empty((B, 4, nb_max), dtype=np.float64)
    _check(lib().oracle_decode_scores(_p(iq), _p(ik_cache), _dtype_code(index_dtype), _p(pt),
                                      pt.shape[1], _p(ctx), B, int(nb_max), _p(S)),
           "decode_scores")
    return S


def decode_query_blocks(context_lens):
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    c = np.empty(len(ctx), dtype=np.int32)
    _check(lib().oracle_decode_query_blocks(_p(ctx), len(ctx), _p(c)), "decode_query_blocks")
    return c


def decode_attend(q, k_cache, v_cache, page_table, context_lens, q2k_rows, scale):
    q, k_cache, v_cache = (np.ascontiguousarray(a) for a in (q, k_cache, v_cache))
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    q2k_rows = np.ascontiguousarray(q2k_rows, dtype=np.int32)
    B = len(ctx)
    out = np.empty((B, 64, 128), dtype=np.float64)
    _check(lib().oracle_decode_attend(_p(q), _p(k_cache), _p(v_cache), _p(pt), pt.shape[1],
                                      _p(ctx), B, _p(q2k_rows), q2k_rows.shape[2],
                                      float(scale), _p(out)), "decode_attend")
    return out


def decode(w, requests=None, q2k_override=None):
    """Whole decode path on a ``workloads.Decode`` (optionally a subset of requests)."""
    if requests is None:
        d = w
    else:
        d = subset_decode(w, requests)
    nb_max = (d.max_context_len + 127) // 128
    S = decode_scores(d.iq, d.ik_cache, d.page_table, d.context_lens, nb_max, d.index_dtype)
    c = decode_query_blocks(d.context_lens)
    q2k, margin = select(S, c, d.topk, d.init_blocks, d.local_blocks)
    rows = q2k if q2k_override is None else q2k_override
    out = decode_attend(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, rows, d.scale)
    return dict(S=S, c=c, q2k=q2k, margin=margin, out=out)


def subset_decode(w, requests):
    """A view of decode workload ``w`` restricted to the listed requests (caches shared)."""
    import copy
    requests = np.asarray(requests, dtype=np.int64)
    d = copy.copy(w)
    d.q = np.ascontiguousarray(w.q[requests])
    d.iq = np.ascontiguousarray(w.iq[requests])
    d.page_table = np.ascontiguousarray(w.page_table[requests])
    d.context_lens = np.ascontiguousarray(w.context_lens[requests])
    return d


def planted_gap(w, tokens):
    """Realised separation of the planted blocks in a planted prefill workload
    (``w.meta['planted_blocks']``), from the oracle's block scores of the
    listed tokens: over every (token, index head) candidate entry, the mean
    block score of planted and of unplanted blocks, their difference, the
    difference in units of the unplanted block scores' standard deviation,
    and the share of the chosen free slots that went to planted blocks."""
    planted = np.asarray(w.meta["planted_blocks"], dtype=np.int64)
    r = prefill_select(w, tokens)
    S = r["S"]                                   # [n,4,nb]
    nb = S.shape[2]
    is_pl = np.zeros(nb, dtype=bool)
    is_pl[planted[planted < nb]] = True
    cand = np.isfinite(S)
    pl = S[cand & is_pl[None, None, :]]
    un = S[cand & ~is_pl[None, None, :]]
    q2k = r["q2k"]
    c = r["c"][:, None, None]
    forced = (q2k >= 0) & ((q2k < w.init_blocks) | (q2k >= c - w.local_blocks + 1))
    free = (q2k >= 0) & ~forced
    chosen_pl = is_pl[np.clip(q2k, 0, nb - 1)] & free
    return dict(tokens=int(len(r["tokens"])), planted_mean=float(pl.mean()), unplanted_mean=float(un.mean()),
                gap=float(pl.mean() - un.mean()), gap_in_unplanted_sd=float((pl.mean() - un.mean()) / un.std()),
                planted_share_of_free_slots=float(chosen_pl.sum() / max(1, free.sum())))
