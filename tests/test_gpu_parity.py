"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
small seeded inputs that still span several tiles and ragged tails."""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import oracle
import workloads as W
from parity import check_attention, check_scores, check_selection, dev
from test_oracle_pins import _golden_cases, closed_form_prefill

pytestmark = pytest.mark.gpu

PREFILL_CASES = [
    # name, doc lengths, topk, init, local, index dtype
    ("one_doc_2k_topk4", [2048], 4, 0, 1, "bf16"),
    ("ragged_docs_topk4_init1", [300, 1000, 77, 1], 4, 1, 1, "bf16"),
    ("docs_topk16_dense", [700, 129, 1500], 16, 0, 1, "bf16"),
    ("long_doc_topk3_local2", [3000], 3, 0, 2, "bf16"),
    ("local0_topk2", [900, 640], 2, 0, 0, "bf16"),
    ("init_local_fill_topk", [1100], 3, 2, 1, "bf16"),
    ("single_token", [1], 16, 0, 1, "bf16"),
    ("block_edges", [127, 128, 129, 255, 256, 257], 2, 1, 1, "bf16"),
    ("fp8_ragged_topk4", [300, 1000, 77], 4, 1, 1, "fp8"),
    ("fp8_long_topk8", [2500], 8, 0, 1, "fp8"),
    # topk 1: the local block alone (R = 0), or the single best block (local 0)
    ("topk1_local1", [700, 300], 1, 0, 1, "bf16"),
    ("topk1_local0_argmax", [900, 200], 1, 0, 0, "bf16"),
    # topk 16 over documents of more than 17 blocks, every token checked: the
    # attention's single-token blocks (one token of a 16-token tile selects
    # them) occur here at small sizes
    ("topk16_init1_doc4096", [4096], 16, 1, 1, "bf16"),
    ("topk16_init1_two_docs", [3000, 2500], 16, 1, 1, "bf16"),
    # many short documents (1..251 tokens): the block scorer's equal work
    # ranges then start and end inside documents and cross dozens of them
    ("many_short_docs", [1 + (37 * i) % 251 for i in range(64)], 4, 1, 1, "bf16"),
    ("fp8_many_short_docs", [1 + (53 * i + 11) % 251 for i in range(64)], 3, 0, 1, "fp8"),
]
E2E_CASES = [c for c in PREFILL_CASES
             if c[0] in ("one_doc_2k_topk4", "ragged_docs_topk4_init1", "docs_topk16_dense",
                         "fp8_ragged_topk4", "fp8_long_topk8", "topk1_local0_argmax",
                         "topk16_init1_two_docs", "many_short_docs")]


def _run_select(w, scores=True):
    cu = dev(w.cu_seqlens)
    return msa.select_blocks(dev(w.iq), dev(w.ik), cu, w.max_seqlen, w.topk, w.init_blocks,
                             w.local_blocks, scores=scores)


def _tok_major(q2k_head_major):
    return q2k_head_major.cpu().numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: c[0])
def test_select_blocks_matches_oracle(case):
    name, docs, topk, init, local, idt = case
    print(f"[select] {name}", flush=True)
    w = W.make_prefill(docs, 100 + len(name), topk=topk, init_blocks=init, local_blocks=local,
                       index_dtype=idt)
    q2k, S = _run_select(w)
    torch.cuda.synchronize()
    ref = oracle.prefill_select(w)
    check_scores(S.cpu().numpy(), ref, ref["tokens"], rel=1e-4 if idt == "bf16" else 1e-4)
    same = check_selection(_tok_major(q2k), ref, topk, init, local)
    assert same.mean() > 0.99


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_select_blocks_closed_forms(case):
    """Hand-derived selections (tests/golden): exact on the GPU, the scores
    are exact integers times 1/8 and every tie must go to the lower id."""
    print(f"[golden] {case['name']}", flush=True)
    w = closed_form_prefill(case["docs"], case["pattern"], case["topk"], case["init"], case["local"])
    q2k, S = _run_select(w)
    ref = oracle.prefill_select(w)
    assert np.array_equal(_tok_major(q2k), ref["q2k"])


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: c[0])
def test_attend_with_oracle_selection(case):
    """Step two alone: the GPU attends over the oracle's q2k."""
    name, docs, topk, init, local, idt = case
    print(f"[attend] {name}", flush=True)
    w = W.make_prefill(docs, 200 + len(name), topk=topk, init_blocks=init, local_blocks=local,
                       index_dtype=idt)
    ref = oracle.prefill(w)
    q2k = dev(ref["q2k"].transpose(1, 0, 2).copy())
    out = msa.sparse_attend_prefill(dev(w.q), dev(w.k), dev(w.v), q2k, dev(w.cu_seqlens),
                                    w.max_seqlen, w.scale)
    check_attention(out.float().cpu().numpy(), ref["out"], what=name)


@pytest.mark.parametrize("case", E2E_CASES, ids=lambda c: c[0])
def test_prefill_end_to_end(case):
    name, docs, topk, init, local, idt = case
    print(f"[e2e] {name}", flush=True)
    w = W.make_prefill(docs, 300 + len(name), topk=topk, init_blocks=init, local_blocks=local,
                       index_dtype=idt)
    q2k = _run_select(w, scores=False)
    out = msa.sparse_attend_prefill(dev(w.q), dev(w.k), dev(w.v), q2k, dev(w.cu_seqlens),
                                    w.max_seqlen, w.scale)
    ref = oracle.prefill(w)
    same = check_selection(_tok_major(q2k), ref, topk, init, local)
    rows = same.all(axis=1)
    assert rows.mean() > 0.9
    tol = 2e-2 if idt == "bf16" else 5e-2
    check_attention(out.float().cpu().numpy()[rows], ref["out"][rows], max_tol=tol, what=name)


def test_attend_arbitrary_row_order_and_repeats():
    """q2k rows are a set: order, repeats and out-of-range ids do not matter."""
    w = W.make_prefill([1000, 400], 17, topk=4, init_blocks=0, local_blocks=1)
    ref = oracle.prefill(w)
    rows = ref["q2k"].transpose(1, 0, 2).copy()          # [4,T,4]
    shuffled = rows[:, :, ::-1].copy()
    mixed = np.concatenate([rows, rows[:, :, :2], np.full(rows.shape[:2] + (2,), 999, np.int32)], 2)
    base = msa.sparse_attend_prefill(dev(w.q), dev(w.k), dev(w.v), dev(rows), dev(w.cu_seqlens),
                                     w.max_seqlen, w.scale)
    for alt in (shuffled, mixed):
        out = msa.sparse_attend_prefill(dev(w.q), dev(w.k), dev(w.v), dev(alt), dev(w.cu_seqlens),
                                        w.max_seqlen, w.scale)
        assert torch.equal(out, base)


DECODE_CASES = [
    ("mixed_lengths_bf16", [1, 127, 128, 129, 1000, 5000, 20000], 16, 0, 1, "bf16"),
    ("topk4_init1_bf16", [300, 2048, 9000], 4, 1, 1, "bf16"),
    ("local2_topk3_bf16", [700, 4097], 3, 0, 2, "bf16"),
    ("mixed_lengths_fp8", [1, 129, 3000, 20000], 16, 0, 1, "fp8"),
    ("topk6_init2_fp8", [5000, 777], 6, 2, 1, "fp8"),
    # larger batches: many requests per launch, mixed and short contexts
    ("batch16_mixed_bf16", [1, 2, 127, 128, 129, 255, 256, 257, 1000, 3000, 5000, 8191, 8192, 8193,
                            12000, 20000], 16, 0, 1, "bf16"),
    ("batch20_topk5_init1_fp8", [64 + 997 * i for i in range(20)], 5, 1, 1, "fp8"),
    ("batch24_short_local2_topk3_bf16", [1 + 37 * i for i in range(24)], 3, 0, 2, "bf16"),
    # no local blocks, several init blocks
    ("init3_local0_topk7_bf16", [1, 300, 5000, 20000], 7, 3, 0, "bf16"),
    ("init2_local0_topk16_fp8", [129, 9000, 30000], 16, 2, 0, "fp8"),
    # more than 64 requests: the bf16 scorer's multi-scan page partition
    ("batch70_short_topk4_bf16", [1 + 53 * i for i in range(70)], 4, 0, 1, "bf16"),
    # every slot forced (R = topk - forced = 0 once c >= init): no free slot
    ("r0_topk2_init1_local1_bf16", [1, 129, 700, 5000, 20000], 2, 1, 1, "bf16"),
    ("r0_topk3_init2_local1_fp8", [1, 200, 300, 9000], 3, 2, 1, "fp8"),
    # topk 1: the local block alone (R = 0), the first block alone (init 1),
    # or the single highest-scoring block (R = 1, no forced block)
    ("topk1_local1_bf16", [1, 128, 129, 3000, 17000], 1, 0, 1, "bf16"),
    ("topk1_init1_local0_fp8", [1, 300, 8000], 1, 1, 0, "fp8"),
    ("topk1_argmax_bf16", [1, 127, 1000, 9000, 30000], 1, 0, 0, "bf16"),
    ("topk1_argmax_fp8", [2, 500, 12000], 1, 0, 0, "fp8"),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: c[0])
def test_decode_matches_oracle(case):
    name, lens, topk, init, local, idt = case
    print(f"[decode] {name}", flush=True)
    d = W.make_decode(lens, 400 + len(name), topk=topk, init_blocks=init, local_blocks=local,
                      index_dtype=idt)
    out, q2k = msa.sparse_attend_decode_paged(
        dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(d.page_table),
        dev(d.context_lens), d.max_context_len, topk, init, local, d.scale, return_q2k=True)
    ref = oracle.decode(d)
    same = check_selection(_tok_major(q2k), ref, topk, init, local)
    # attention on the rows (request, KV head) whose selection equals the
    # oracle's; a row may differ only within the margin rule, and at most a
    # few do
    rows = same.all(axis=1)
    assert rows.mean() > 0.9
    tol = 2e-2 if idt == "bf16" else 5e-2
    check_attention(out.float().cpu().numpy()[rows], ref["out"][rows], max_tol=tol, what=name)
    assert np.all(np.isfinite(out.float().cpu().numpy())), "NaN from poisoned tail slots"


@pytest.mark.parametrize("max_ctx,idt", [(1048576, "bf16"), (1048576, "fp8"), (262145, "bf16"),
                                         (131073, "fp8")])
def test_decode_context_bound_far_above_lengths(max_ctx, idt):
    """max_context_len only bounds the grid and the per-lane candidate count
    of the in-kernel top-k (up to 128 per lane at the largest supported
    bound, 1048576): with the same short requests the outputs must equal,
    bit for bit, those of the call with the tight bound, and the oracle."""
    print(f"[decode bound] max_ctx={max_ctx} {idt}", flush=True)
    lens = [1, 300, 4097, 9000]
    d = W.make_decode(lens, 77, topk=16, init_blocks=1, local_blocks=1, index_dtype=idt)
    wide = np.full((d.B, -(-max_ctx // 128)), -1, dtype=np.int32)
    wide[:, :d.page_table.shape[1]] = d.page_table
    args = (dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache))
    out_w, q2k_w = msa.sparse_attend_decode_paged(*args, dev(wide), dev(d.context_lens), max_ctx, 16, 1,
                                                  1, d.scale, return_q2k=True)
    out_t, q2k_t = msa.sparse_attend_decode_paged(*args, dev(d.page_table), dev(d.context_lens),
                                                  d.max_context_len, 16, 1, 1, d.scale, return_q2k=True)
    assert torch.equal(q2k_w, q2k_t) and torch.equal(out_w, out_t)
    ref = oracle.decode(d)
    rows = check_selection(_tok_major(q2k_w), ref, 16, 1, 1).all(axis=1)
    check_attention(out_w.float().cpu().numpy()[rows], ref["out"][rows],
                    max_tol=2e-2 if idt == "bf16" else 5e-2, what=f"bound {max_ctx}")


@pytest.mark.parametrize("pattern", ["constant", "two_level"])
def test_decode_tied_scores_take_lowest_ids(pattern):
    """Index keys built so that many blocks share the same maximum score:
    every block ("constant") or two groups of blocks ("two_level").  The
    selection must equal the oracle's exactly: ties go to the lower block id,
    which exercises the top-k's bisection past a shared score prefix."""
    print(f"[decode ties] {pattern}", flush=True)
    lens = [130, 2000, 5000, 9000, 4097]
    d = W.make_decode(lens, 303, topk=8, init_blocks=1, local_blocks=1)
    row_a, row_b = d.ik_cache[0].copy(), d.ik_cache[1].copy()  # first slots: never poisoned
    for r, L in enumerate(lens):
        for pg in range(-(-L // 128)):
            slot0 = int(d.page_table[r, pg]) * 128
            row = row_b if (pattern == "two_level" and pg % 3 == 0) else row_a
            d.ik_cache[slot0:slot0 + 128] = row
    out, q2k = msa.sparse_attend_decode_paged(
        dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(d.page_table),
        dev(d.context_lens), d.max_context_len, d.topk, 1, 1, d.scale, return_q2k=True)
    ref = oracle.decode(d)
    assert np.array_equal(_tok_major(q2k), ref["q2k"])
    check_attention(out.float().cpu().numpy(), ref["out"], what=f"ties {pattern}")


@pytest.mark.parametrize("init,local", [(0, 1), (2, 0)])
def test_decode_all_tied_around_64_candidates(init, local):
    """Every block's score tied, with 62 to 66 candidates per row.  The decode
    top-k takes its fast path while at most 64 candidates reach the bound it
    derives from the lane maxima, and its general path beyond that; both must
    give the oracle's selection (the lowest ids) exactly."""
    print(f"[decode ties 64] init={init} local={local}", flush=True)
    lens = [8065, 8192, 8193, 8320, 8321, 8449]
    d = W.make_decode(lens, 304, topk=16, init_blocks=init, local_blocks=local)
    row_a = d.ik_cache[0].copy()  # first slots: never poisoned
    for r, L in enumerate(lens):
        for pg in range(-(-L // 128)):
            slot0 = int(d.page_table[r, pg]) * 128
            d.ik_cache[slot0:slot0 + 128] = row_a
    out, q2k = msa.sparse_attend_decode_paged(
        dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(d.page_table),
        dev(d.context_lens), d.max_context_len, d.topk, init, local, d.scale, return_q2k=True)
    ref = oracle.decode(d)
    assert np.array_equal(_tok_major(q2k), ref["q2k"])
    check_attention(out.float().cpu().numpy(), ref["out"], what=f"ties 64 init={init}")


def test_decode_page_permutation_invariance():
    lens = [700, 1281, 256, 3000]
    a = W.make_decode(lens, 81, topk=5, identity_pages=True)
    b = W.make_decode(lens, 81, topk=5, identity_pages=False)
    for r in range(a.B):
        for p in range((lens[r] + 127) // 128):
            pa, pb = a.page_table[r, p], b.page_table[r, p]
            for cache in ("k_cache", "v_cache", "ik_cache"):
                getattr(b, cache)[pb * 128:(pb + 1) * 128] = getattr(a, cache)[pa * 128:(pa + 1) * 128]
    outs = []
    for d in (a, b):
        outs.append(msa.sparse_attend_decode_paged(
            dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(d.page_table),
            dev(d.context_lens), d.max_context_len, d.topk, 0, 1, d.scale, return_q2k=True))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][0], outs[1][0])


def test_decode_equals_prefill_last_token_on_gpu():
    """Both GPU paths on one logical sequence: the decode row equals the
    prefill's last-token row (same selection; attention within tolerance)."""
    L = 3000
    d = W.make_decode([L], 91, topk=6, init_blocks=1, local_blocks=1, identity_pages=True)
    slots = np.arange(L)
    q = np.zeros((L, 64, 128), np.uint16)
    q[L - 1] = d.q[0]
    iq = np.zeros((L, 4, 128), np.uint16)
    iq[L - 1] = d.iq[0]
    cu = np.array([0, L], np.int32)
    q2k_p = msa.select_blocks(dev(iq), dev(d.ik_cache[slots]), dev(cu), L, 6, 1, 1)
    out_p = msa.sparse_attend_prefill(dev(q), dev(d.k_cache[slots]), dev(d.v_cache[slots]), q2k_p,
                                      dev(cu), L, d.scale)
    out_d, q2k_d = msa.sparse_attend_decode_paged(
        dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(d.page_table),
        dev(d.context_lens), L, 6, 1, 1, d.scale, return_q2k=True)
    assert torch.equal(q2k_p[:, L - 1], q2k_d[:, 0])
    err = (out_p[L - 1].float() - out_d[0].float()).abs().max().item()
    assert err <= 2e-2


def test_outputs_are_deterministic():
    w = W.make_prefill([1500, 600], 5, topk=4, init_blocks=1, local_blocks=1)
    outs = []
    for _ in range(3):
        q2k = _run_select(w, scores=False)
        outs.append((q2k, msa.sparse_attend_prefill(dev(w.q), dev(w.k), dev(w.v), q2k,
                                                    dev(w.cu_seqlens), w.max_seqlen, w.scale)))
    for q2k, out in outs[1:]:
        assert torch.equal(q2k, outs[0][0]) and torch.equal(out, outs[0][1])


def test_graph_capture_replays_match_eager():
    """The calls never allocate or sync, so a HIP graph can hold them; every
    replay must reproduce the eager result."""
    w = W.make_prefill([1200, 333], 8, topk=4, init_blocks=0, local_blocks=1)
    iq, ik, cu = dev(w.iq), dev(w.ik), dev(w.cu_seqlens)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    ws_sel = torch.empty(msa.select_blocks_workspace_bytes(w.T, w.num_docs, w.max_seqlen),
                         dtype=torch.uint8, device="cuda")
    ws_att = torch.empty(max(256, msa.prefill_workspace_bytes(w.T, w.num_docs, w.max_seqlen)),
                         dtype=torch.uint8, device="cuda")
    q2k_e = msa.select_blocks(iq, ik, cu, w.max_seqlen, 4, 0, 1, workspace=ws_sel)
    out_e = msa.sparse_attend_prefill(q, k, v, q2k_e, cu, w.max_seqlen, w.scale, workspace=ws_att)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q2k_g = msa.select_blocks(iq, ik, cu, w.max_seqlen, 4, 0, 1, workspace=ws_sel)
            out_g = msa.sparse_attend_prefill(q, k, v, q2k_g, cu, w.max_seqlen, w.scale,
                                              workspace=ws_att)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        q2k_g.fill_(-7)
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q2k_g, q2k_e) and torch.equal(out_g, out_e)
