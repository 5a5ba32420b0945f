"""The allocation-free decode entry point (scratch in a library-held device
array) against the workspace entry point, through the C ABI: identical
outputs and selections, on two calls in a row, the second with a smaller
batch (the array keeps the first call's contents), and a clear error for a
batch whose scratch exceeds the array."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import workloads as W
from parity import dev

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _call_both(d):
    L = msa.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = dict(q=dev(d.q), iq=dev(d.iq), kc=dev(d.k_cache), vc=dev(d.v_cache), ikc=dev(d.ik_cache),
             pt=dev(d.page_table), ctx=dev(d.context_lens))
    idt = 0 if d.index_dtype == "bf16" else 1
    head = (_ptr(a["q"]), _ptr(a["iq"]), _ptr(a["kc"]), _ptr(a["vc"]), _ptr(a["ikc"]), idt, _ptr(a["pt"]),
            d.max_pages, _ptr(a["ctx"]), d.B, d.max_context_len, d.topk, d.init_blocks, d.local_blocks,
            d.scale)
    out_ws = torch.empty((d.B, 64, 128), dtype=torch.bfloat16, device="cuda")
    q2k_ws = torch.empty((4, d.B, d.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(msa.decode_workspace_bytes(d.B, d.max_context_len, d.topk), dtype=torch.uint8,
                     device="cuda")
    assert L.msa_sparse_attend_decode_paged(*head, _ptr(out_ws), _ptr(q2k_ws), _ptr(ws), ws.numel(), s) == 0
    out_na = torch.full((d.B, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    q2k_na = torch.full((4, d.B, d.topk), -7, dtype=torch.int32, device="cuda")
    st = L.msa_sparse_attend_decode_paged_noalloc(*head, _ptr(out_na), _ptr(q2k_na), s)
    assert st == 0, L.msa_last_error().decode()
    torch.cuda.synchronize()
    return out_ws, q2k_ws, out_na, q2k_na


def test_noalloc_decode_equals_workspace_decode_twice():
    print("[noalloc] batch 12 then batch 3", flush=True)
    big = W.make_decode([1, 129, 3000, 20000, 7000, 128, 4097, 300, 9999, 12000, 64, 2500], 601,
                        topk=16, init_blocks=1, local_blocks=1)
    small = W.make_decode([700, 50, 5000], 602, topk=5, init_blocks=0, local_blocks=2,
                          index_dtype="fp8")
    for d in (big, small):
        out_ws, q2k_ws, out_na, q2k_na = _call_both(d)
        assert torch.equal(out_na, out_ws), d.name
        assert torch.equal(q2k_na, q2k_ws), d.name


def test_noalloc_rejects_scratch_beyond_the_array():
    L = msa.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails first
    st = L.msa_sparse_attend_decode_paged_noalloc(fake, fake, fake, fake, fake, 0, fake, 1024, fake, 256,
                                                  131072, 16, 0, 1, 0.088, fake, None, None)
    assert st == 2
    assert "scratch" in L.msa_last_error().decode()
