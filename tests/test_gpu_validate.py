"""GPU tests of the decode path's robustness rules (empty requests, absent
pages) and of the debug validators of the device-side data contract."""
import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import oracle
import workloads as W
from parity import check_attention, dev

pytestmark = pytest.mark.gpu


def _decode(d, ctx, pt, **kw):
    return msa.sparse_attend_decode_paged(
        dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(pt), dev(ctx),
        d.max_context_len, d.topk, d.init_blocks, d.local_blocks, d.scale, return_q2k=True, **kw)


@pytest.mark.parametrize("idt", ["bf16", "fp8"])
def test_decode_empty_requests_read_nothing(idt):
    """context_lens 0 (and negative) mark padding requests, whose page-table
    rows hold -1: their out rows are zero and their q2k rows -1, and every
    other request gets exactly the output of the batch without them."""
    print(f"[empty requests] {idt}", flush=True)
    lens = [300, 5000, 129, 20000]
    d = W.make_decode(lens, 501, topk=8, init_blocks=1, local_blocks=1, index_dtype=idt)
    out_ref, q2k_ref = _decode(d, d.context_lens, d.page_table)
    # interleave padding requests: rows 1 and 3 of a batch of 6
    keep = [0, 2, 4, 5]
    B = 6
    ctx = np.zeros(B, np.int32)
    ctx[keep] = d.context_lens
    ctx[3] = -5
    pt = np.full((B, d.page_table.shape[1]), -1, np.int32)
    pt[keep] = d.page_table
    q = np.zeros((B,) + d.q.shape[1:], d.q.dtype)
    q[keep] = d.q
    iq = np.zeros((B,) + d.iq.shape[1:], d.iq.dtype)
    iq[keep] = d.iq
    out, q2k = msa.sparse_attend_decode_paged(
        dev(q), dev(iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(pt), dev(ctx),
        d.max_context_len, d.topk, d.init_blocks, d.local_blocks, d.scale, return_q2k=True)
    torch.cuda.synchronize()
    assert torch.equal(out[keep], out_ref)
    assert torch.equal(q2k[:, keep], q2k_ref)
    pad = [1, 3]
    assert torch.count_nonzero(out[pad].float()) == 0
    assert bool((q2k[:, pad] == -1).all())


@pytest.mark.parametrize("nan_page0", [False, True])
def test_decode_absent_page_adds_no_keys(nan_page0):
    """A negative page id inside a request's context: nothing of that page is
    read; the block scores -inf, so it is never chosen over a real block, and
    when forced (here the local block of a 1-page request and the init block)
    it adds no key.  The other requests are unaffected.  With nan_page0 the
    caches gain a physical page 0 that no request owns, all NaN: an absent
    block must not read it (a zero weight times NaN would still be NaN)."""
    print(f"[absent page] nan_page0={nan_page0}", flush=True)
    lens = [1000, 3000, 100, 9000]
    d = W.make_decode(lens, 502, topk=6, init_blocks=1, local_blocks=1)
    if nan_page0:
        nan_bf16 = np.uint16(0x7FC0)
        for name in ("k_cache", "v_cache", "ik_cache"):
            a = getattr(d, name)
            setattr(d, name, np.concatenate([np.full((128,) + a.shape[1:], nan_bf16, a.dtype), a]))
        d.page_table = np.where(d.page_table >= 0, d.page_table + 1, d.page_table).astype(np.int32)
    out_ref, q2k_ref = _decode(d, d.context_lens, d.page_table)
    pt = d.page_table.copy()
    pt[0, 3] = -1          # a free (non-forced) block of request 0: never selected now
    pt[1, 0] = -7          # request 1's forced init block: selected, adds no key
    pt[2, 0] = -1          # request 2's only page: no key at all -> zero row
    out, q2k = _decode(d, d.context_lens, pt)
    torch.cuda.synchronize()
    assert torch.equal(out[3], out_ref[3]) and torch.equal(q2k[:, 3], q2k_ref[:, 3])
    assert not bool((q2k[:, 0] == 3).any())
    assert torch.count_nonzero(out[2].float()) == 0
    assert bool(torch.isfinite(out.float()).all())
    # request 1: its forced init block 0 stays in the row but adds no key, so
    # the output is the oracle's attention over the row without block 0
    rows = q2k.cpu().numpy().transpose(1, 0, 2)[[1]].copy()   # [1,4,topk]
    assert np.all(rows[0, :, 0] == 0)
    rows[rows == 0] = -1
    ref = oracle.decode_attend(d.q[[1]], d.k_cache, d.v_cache, d.page_table[[1]], d.context_lens[[1]],
                               rows, d.scale)
    check_attention(out[1:2].float().cpu().numpy(), ref, what="absent init block")


def test_validate_prefill_inputs():
    cu = torch.tensor([0, 100, 300, 301], dtype=torch.int32, device="cuda")
    assert msa.validate_prefill_inputs(cu, 301, 200) == (0, -1)
    assert msa.validate_prefill_inputs(cu, 301, 150) == (8, 1)       # doc 1 longer than max_seqlen
    assert msa.validate_prefill_inputs(cu, 302, 200) == (2, 2)       # ends short of total_tokens
    bad = torch.tensor([5, 100, 100, 301], dtype=torch.int32, device="cuda")
    bits, first = msa.validate_prefill_inputs(bad, 301, 300)
    assert bits == 1 | 4 and first == 0                              # start != 0, empty doc 1
    big = torch.tensor([0, 100, 400, 301], dtype=torch.int32, device="cuda")
    bits, first = msa.validate_prefill_inputs(big, 301, 300)
    assert bits & 16 and bits & 4 and first == 1                     # offset past T, then a drop
    many = torch.arange(0, 2001, dtype=torch.int32, device="cuda")   # 2000 one-token documents
    assert msa.validate_prefill_inputs(many, 2000, 1) == (0, -1)
    many[1500] = many[1499]
    assert msa.validate_prefill_inputs(many, 2000, 1)[1] == 1499


def test_validate_decode_inputs():
    d = W.make_decode([300, 5000, 129], 503, topk=4)
    P = int(((d.context_lens + 127) // 128).sum())
    pt, ctx = dev(d.page_table), dev(d.context_lens)
    assert msa.validate_decode_inputs(pt, ctx, d.max_context_len, P) == (0, -1)
    assert msa.validate_decode_inputs(pt, ctx, d.max_context_len, P - 1)[0] == 64
    pt2 = pt.clone()
    pt2[2, 1] = -1
    assert msa.validate_decode_inputs(pt2, ctx, d.max_context_len, P) == (64, 2)
    pt2[2, 1] = pt[2, 1]
    pt2[2, 2] = -1            # past request 2's context (2 pages): never used
    assert msa.validate_decode_inputs(pt2, ctx, d.max_context_len, P) == (0, -1)
    ctx2 = ctx.clone()
    ctx2[1] = d.max_context_len + 1
    assert msa.validate_decode_inputs(pt, ctx2, d.max_context_len, P) == (32, 1)
    ctx2[1] = 0               # an empty request is valid
    assert msa.validate_decode_inputs(pt, ctx2, d.max_context_len, P) == (0, -1)
