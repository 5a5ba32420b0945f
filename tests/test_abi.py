"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/msa.h declares, and rejects malformed host arguments before any
GPU work (status code + message)."""
import ctypes
import os
import re

import pytest

import block_sparse_gqa_score_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("msa_select_blocks", "msa_sparse_attend_prefill",
                     "msa_sparse_attend_decode_paged", "msa_unsupported_reason",
                     "msa_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = msa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_unsupported_reason():
    assert msa.unsupported_reason() is None
    assert msa.unsupported_reason(topk=4) is None
    assert "num_heads" in msa.unsupported_reason(num_heads=32)
    assert "num_kv_heads" in msa.unsupported_reason(num_kv_heads=8)
    assert "head_dim" in msa.unsupported_reason(head_dim=64)
    assert "topk" in msa.unsupported_reason(topk=17)
    assert "topk" in msa.unsupported_reason(topk=0)
    assert "block_size" in msa.unsupported_reason(block_size=64)


def test_workspace_sizes():
    T, D, S = 32768, 1, 32768
    ws = msa.select_blocks_workspace_bytes(T, D, S)
    assert ws >= 4 * 256 * T * 4 and ws % 256 == 0
    assert msa.select_blocks_workspace_bytes(0, 1, 1) == 0
    assert msa.select_blocks_workspace_bytes(10, 11, 10) == 0
    assert msa.prefill_workspace_bytes(100, 3, 50) > 0
    assert msa.decode_workspace_bytes(32, 32768, 16) > 32 * 4 * 256 * 4
    assert msa.decode_workspace_bytes(1, 8192 * 128 + 1, 16) == 0
    assert msa.decode_workspace_bytes(1, 100, 17) == 0


def _select(**kw):
    a = dict(index_q=FAKE, index_k=FAKE, index_dtype=0, cu=FAKE, ndocs=1, T=256, max_seqlen=256,
             topk=16, init=0, local=1, q2k=FAKE, scores=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return msa.lib().msa_select_blocks(a["index_q"], a["index_k"], a["index_dtype"], a["cu"],
                                       a["ndocs"], a["T"], a["max_seqlen"], a["topk"], a["init"],
                                       a["local"], a["q2k"], a["scores"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(index_q=None), 1, "non-NULL"),
    (dict(cu=None), 1, "cu_seqlens"),
    (dict(index_dtype=7), 2, "index_dtype"),
    (dict(T=0), 1, "total_tokens"),
    (dict(ndocs=0), 1, "num_docs"),
    (dict(ndocs=300), 1, "num_docs"),
    (dict(max_seqlen=0), 1, "max_seqlen"),
    (dict(max_seqlen=257), 1, "max_seqlen"),
    (dict(topk=0), 2, "topk"),
    (dict(topk=17), 2, "topk"),
    (dict(init=-1), 1, "init_blocks"),
    (dict(init=10, local=7), 1, "exceeds topk"),
    (dict(ws_bytes=16), 3, "workspace"),
    (dict(ws=None), 3, "workspace"),
])
def test_select_blocks_rejects(kw, status, needle):
    assert _select(**kw) == status
    assert needle in msa.lib().msa_last_error().decode()


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, q2k=FAKE, topk=16, cu=FAKE, ndocs=1, T=256, max_seqlen=256,
             scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return msa.lib().msa_sparse_attend_prefill(a["q"], a["k"], a["v"], a["q2k"], a["topk"], a["cu"],
                                               a["ndocs"], a["T"], a["max_seqlen"], a["scale"],
                                               a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(out=None), 1, "non-NULL"),
    (dict(topk=0), 2, "topk"),
    (dict(T=-5), 1, "total_tokens"),
    (dict(scale=0.0), 1, "softmax_scale"),
    (dict(scale=float("nan")), 1, "softmax_scale"),
    (dict(ws_bytes=0), 3, "workspace"),
])
def test_prefill_rejects(kw, status, needle):
    assert _prefill(**kw) == status
    assert needle in msa.lib().msa_last_error().decode()


def _decode(**kw):
    a = dict(q=FAKE, iq=FAKE, kc=FAKE, vc=FAKE, ikc=FAKE, dtype=0, pt=FAKE, max_pages=256, ctx=FAKE,
             B=32, max_ctx=32768, topk=16, init=0, local=1, scale=0.088, out=FAKE, q2k=None,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return msa.lib().msa_sparse_attend_decode_paged(
        a["q"], a["iq"], a["kc"], a["vc"], a["ikc"], a["dtype"], a["pt"], a["max_pages"], a["ctx"],
        a["B"], a["max_ctx"], a["topk"], a["init"], a["local"], a["scale"], a["out"], a["q2k"],
        a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(pt=None), 1, "non-NULL"),
    (dict(dtype=3), 2, "index_dtype"),
    (dict(B=0), 1, "batch"),
    (dict(max_ctx=0), 1, "max_context_len"),
    (dict(max_ctx=8192 * 128 + 1, max_pages=9000), 2, "not supported"),
    (dict(max_pages=10), 1, "max_pages_per_seq"),
    (dict(topk=20), 2, "topk"),
    (dict(init=16, local=1), 1, "exceeds topk"),
    (dict(ws_bytes=100), 3, "workspace"),
])
def test_decode_rejects(kw, status, needle):
    assert _decode(**kw) == status
    assert needle in msa.lib().msa_last_error().decode()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "block_sparse_gqa_score_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                for needle in ("import oracle", "from oracle", "msa_oracle", "libmsa_oracle"):
                    assert needle not in text, (f, needle)


def _decode_mx(**kw):
    a = dict(q=FAKE, iq=FAKE, kc=FAKE, vc=FAKE, ikc=FAKE, dtype=0, pt=FAKE, max_pages=256, ctx=FAKE,
             B=32, max_ctx=32768, topk=16, init=0, local=1, scale=0.088, oq=FAKE, os=FAKE, q2k=None,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return msa.lib().msa_sparse_attend_decode_paged_mxfp8(
        a["q"], a["iq"], a["kc"], a["vc"], a["ikc"], a["dtype"], a["pt"], a["max_pages"], a["ctx"],
        a["B"], a["max_ctx"], a["topk"], a["init"], a["local"], a["scale"], a["oq"], a["os"], a["q2k"],
        a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(oq=None), 1, "out_q"),
    (dict(os=None), 1, "out_scale"),
    (dict(pt=None), 1, "non-NULL"),
    (dict(topk=0), 2, "topk"),
    (dict(ws_bytes=100), 3, "workspace"),
])
def test_decode_mxfp8_rejects(kw, status, needle):
    assert _decode_mx(**kw) == status
    assert needle in msa.lib().msa_last_error().decode()


@pytest.mark.parametrize("args,needle", [
    ((None, 4, 64, FAKE, FAKE), "non-NULL"),
    ((FAKE, 4, 48, FAKE, FAKE), "multiple of 32"),
    ((FAKE, 0, 64, FAKE, FAKE), "rows"),
    ((FAKE, 4, 0, FAKE, FAKE), "multiple of 32"),
])
def test_mxfp8_quantize_rejects(args, needle):
    assert msa.lib().msa_mxfp8_quantize(*args, None) == 1
    assert needle in msa.lib().msa_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(k=None), 1, "non-NULL"),
    (dict(dtype=5), 2, "index_dtype"),
    (dict(n=-1), 1, "num_tokens"),
    (dict(slots=0), 1, "num_slots"),
])
def test_cache_insert_rejects(kw, status, needle):
    a = dict(k=FAKE, v=FAKE, ik=FAKE, sm=FAKE, n=4, dtype=0, kc=FAKE, vc=FAKE, ikc=FAKE, slots=128)
    a.update(kw)
    st = msa.lib().msa_cache_insert(a["k"], a["v"], a["ik"], a["sm"], a["n"], a["dtype"], a["kc"], a["vc"],
                                    a["ikc"], a["slots"], None)
    assert st == status
    assert needle in msa.lib().msa_last_error().decode()


def test_cache_insert_of_nothing_is_a_no_op():
    assert msa.lib().msa_cache_insert(FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, 128, None) == 0


def _decode_fp8kv(**kw):
    a = dict(q=FAKE, iq=FAKE, kc=FAKE, vc=FAKE, ks=0.5, vs=0.25, ikc=FAKE, dtype=0, pt=FAKE,
             max_pages=256, ctx=FAKE, B=32, max_ctx=32768, topk=16, init=0, local=1, scale=0.088,
             out=FAKE, q2k=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return msa.lib().msa_sparse_attend_decode_paged_fp8kv(
        a["q"], a["iq"], a["kc"], a["vc"], a["ks"], a["vs"], a["ikc"], a["dtype"], a["pt"],
        a["max_pages"], a["ctx"], a["B"], a["max_ctx"], a["topk"], a["init"], a["local"], a["scale"],
        a["out"], a["q2k"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(ks=0.0), 1, "k_scale"),
    (dict(vs=-1.0), 1, "v_scale"),
    (dict(ks=float("nan")), 1, "k_scale"),
    (dict(vs=float("inf")), 1, "v_scale"),
    (dict(kc=None), 1, "non-NULL"),
    (dict(topk=17), 2, "topk"),
    (dict(ws_bytes=100), 3, "workspace"),
])
def test_decode_fp8kv_rejects(kw, status, needle):
    assert _decode_fp8kv(**kw) == status
    assert needle in msa.lib().msa_last_error().decode()


def test_prefill_lse_rejects_null_lse():
    st = msa.lib().msa_sparse_attend_prefill_lse(FAKE, FAKE, FAKE, FAKE, 16, FAKE, 1, 256, 256, 0.088, FAKE,
                                                 None, FAKE, 1 << 40, None)
    assert st == 1 and "lse" in msa.lib().msa_last_error().decode()


def _backward(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, q2k=FAKE, topk=16, cu=FAKE, ndocs=1,
             T=256, max_seqlen=256, scale=0.088, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return msa.lib().msa_sparse_attend_prefill_backward(
        a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["q2k"], a["topk"], a["cu"], a["ndocs"],
        a["T"], a["max_seqlen"], a["scale"], a["dq"], a["dk"], a["dv"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lse=None), 1, "non-NULL"),
    (dict(dout=None), 1, "non-NULL"),
    (dict(dv=None), 1, "non-NULL"),
    (dict(topk=17), 2, "topk"),
    (dict(ndocs=0), 1, "num_docs"),
    (dict(T=(1 << 22) + 1, max_seqlen=1000), 2, "total_tokens"),
    (dict(scale=-1.0), 1, "softmax_scale"),
    (dict(ws_bytes=1000), 3, "workspace"),
])
def test_backward_rejects(kw, status, needle):
    assert _backward(**kw) == status
    assert needle in msa.lib().msa_last_error().decode()


def test_backward_workspace_bytes():
    T, D = 32768, 1
    ws = msa.prefill_backward_workspace_bytes(T, D, T, 16)
    # at least: D [T,64] fp32 and the block lists (4*T*topk int32)
    assert ws >= T * 64 * 4 + 4 * T * 16 * 4 and ws % 256 == 0
    assert msa.prefill_backward_workspace_bytes(T, D, T, 17) == 0
    assert msa.prefill_backward_workspace_bytes((1 << 22) + 1, 1, 100, 16) == 0
    assert msa.prefill_backward_workspace_bytes(0, 1, 1, 16) == 0


@pytest.mark.parametrize("args,needle", [
    ((None, 1, 10, 10, FAKE), "cu_seqlens"),
    ((FAKE, 0, 10, 10, FAKE), "num_docs"),
    ((FAKE, 1, 10, 11, FAKE), "max_seqlen"),
    ((FAKE, 1, 10, 10, None), "status"),
])
def test_validate_prefill_rejects_host_errors(args, needle):
    assert msa.lib().msa_validate_prefill_inputs(*args, None) == 1
    assert needle in msa.lib().msa_last_error().decode()


@pytest.mark.parametrize("args,needle", [
    ((None, 1, FAKE, 1, 128, 1, FAKE), "page_table"),
    ((FAKE, 1, FAKE, 0, 128, 1, FAKE), "batch"),
    ((FAKE, 1, FAKE, 1, 0, 1, FAKE), "max_context_len"),
    ((FAKE, 1, FAKE, 1, 128, 0, FAKE), "num_pages"),
    ((FAKE, 1, FAKE, 1, 129, 5, FAKE), "max_pages_per_seq"),
    ((FAKE, 1, FAKE, 1, 128, 1, None), "status"),
])
def test_validate_decode_rejects_host_errors(args, needle):
    assert msa.lib().msa_validate_decode_inputs(*args, None) == 1
    assert needle in msa.lib().msa_last_error().decode()
