"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a library
routine (torch's bf16 / float8_e4m3fn conversions, torch's
scaled_dot_product_attention in float64), brute force on tiny inputs, closed
forms, hand-derived fixtures under tests/golden/ and invariants of the
selection rule.  test_oracle_mutants.py shows that planted mistakes in the
oracle's source fail these pins.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def e4m3_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def index_f64(a, index_dtype):
    return bf16_f64(a) if index_dtype == "bf16" else e4m3_f64(a)


def doc_geometry(cu):
    T = int(cu[-1])
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    pos = np.arange(T) - cu[doc]
    return doc, pos


def brute_scores(iq, ik, cu, index_dtype="bf16"):
    """Dense iq.ik^T, causal + same-document mask, then per-block max (numpy)."""
    q = index_f64(iq, index_dtype)            # [T,4,128]
    k = index_f64(ik, index_dtype)[:, 0, :]   # [T,128]
    T = q.shape[0]
    doc, pos = doc_geometry(cu)
    nb = int(math.ceil(np.max(np.diff(cu)) / 128))
    dots = np.einsum("thx,jx->thj", q, k)     # [T,4,T]
    ok = (doc[:, None] == doc[None, :]) & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    kblk = pos // 128
    S = np.full((T, 4, nb), -np.inf)
    for b in range(nb):
        m = ok & (kblk[None, :] == b)
        masked = np.where(m[:, None, :], dots, -np.inf)
        S[:, :, b] = masked.max(axis=2)
    return S


def selection_mask(q2k, cu):
    """[4,T,T] bool: key j is in query t's key set for KV head g."""
    T = int(cu[-1])
    doc, pos = doc_geometry(cu)
    kblk = pos // 128
    ok = (doc[:, None] == doc[None, :]) & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    sel = np.zeros((4, T, T), dtype=bool)
    for g in range(4):
        for s in range(q2k.shape[2]):
            ids = q2k[:, g, s]
            sel[g] |= (kblk[None, :] == ids[:, None]) & (ids[:, None] >= 0)
    return sel & ok[None]


def sdpa_reference(w, mask4):
    """torch SDPA in float64 (CPU), GQA by contiguous head groups h -> h // 16."""
    q = torch.from_numpy(bf16_f64(w.q)).permute(1, 0, 2)               # [64,T,128]
    k = torch.from_numpy(bf16_f64(w.k)).permute(1, 0, 2)               # [4,T,128]
    v = torch.from_numpy(bf16_f64(w.v)).permute(1, 0, 2)
    k = k.repeat_interleave(16, dim=0)
    v = v.repeat_interleave(16, dim=0)
    m = torch.from_numpy(mask4).repeat_interleave(16, dim=0)           # [64,T,T]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=w.scale)
    return o.permute(1, 0, 2).numpy()                                   # [T,64,128]


def closed_form_prefill(docs, pattern, topk, init, local, alpha=0.125, seed=7):
    cu = np.zeros(len(docs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(docs)

    def index_fn(T):
        doc, pos = doc_geometry(cu)
        b = pos // 128
        nb_doc = np.ceil(np.diff(cu) / 128).astype(int)[doc]
        val = {"increasing": b + 1, "decreasing": nb_doc - b, "constant": np.ones_like(b)}[pattern]
        iq = np.zeros((T, 4, 128), np.float32)
        iq[:, :, 0] = 1.0
        ik = np.zeros((T, 1, 128), np.float32)
        ik[:, 0, 0] = alpha * val
        return iq, ik

    return W.make_prefill(docs, seed, topk=topk, init_blocks=init, local_blocks=local,
                          index_fn=index_fn)


# ------------------------------------------------------------ decoders
def test_bf16_decoder_matches_torch_on_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bf16_f64(codes)
    got = np.array([orc.lib().oracle_bf16_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decoder_matches_torch_on_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = e4m3_f64(codes)
    got = np.array([orc.lib().oracle_e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert nan.sum() == 2                                  # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_generator_encoders_match_torch_rounding():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 40
    assert np.array_equal(W.bf16_bits(x).view(np.int16),
                          torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy())
    inr = x[np.abs(x) < 440]
    assert np.array_equal(W.e4m3_bytes(inr),
                          torch.from_numpy(inr).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.all(W.e4m3_bytes(np.array([1e4, -1e4], np.float32)) == np.array([0x7E, 0xFE]))


# ------------------------------------------------------------ scores
@pytest.mark.parametrize("index_dtype", ["bf16", "fp8"])
def test_scores_equal_dense_brute_force(orc, index_dtype):
    w = W.make_prefill([200, 77, 300], 11, index_dtype=index_dtype)
    nb = (w.max_seqlen + 127) // 128
    S = orc.scores(w.iq, w.ik, w.cu_seqlens, np.arange(w.T), nb, index_dtype)
    ref = brute_scores(w.iq, w.ik, w.cu_seqlens, index_dtype)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(S))
    assert np.allclose(S[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_scores_closed_form_increasing(orc):
    w = closed_form_prefill([677, 130], "increasing", 4, 0, 1)
    nb = 6
    S = orc.scores(w.iq, w.ik, w.cu_seqlens, np.arange(w.T), nb)
    doc, pos = doc_geometry(w.cu_seqlens)
    c = pos // 128
    for t in range(w.T):
        expect = np.full(nb, -np.inf)
        expect[: c[t] + 1] = 0.125 * (np.arange(c[t] + 1) + 1)
        assert np.array_equal(S[t, 0], expect) and np.array_equal(S[t, 3], expect)


# ------------------------------------------------------------ selection
def _golden_cases():
    with open(os.path.join(GOLDEN, "select_closed_form.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_selection_golden(orc, case):
    w = closed_form_prefill(case["docs"], case["pattern"], case["topk"], case["init"], case["local"])
    r = orc.prefill_select(w)
    doc, pos = doc_geometry(w.cu_seqlens)
    c = pos // 128
    if "rows_by_c" in case:
        expect = np.array([case["rows_by_c"][str(x)] for x in c])
    else:
        expect = np.array([case["doc_rows_by_c"][str(d)][str(x)] for d, x in zip(doc, c)])
    for g in range(4):
        assert np.array_equal(r["q2k"][:, g], expect), g


def test_selection_brute_force_subsets(orc):
    """Top-R equals the max-sum R-subset of the non-forced candidates."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        c = int(rng.integers(0, 8))
        topk = int(rng.integers(1, 7))
        init = int(rng.integers(0, topk + 1))
        local = int(rng.integers(0, topk - init + 1))
        nb = 8
        S = np.full((1, 4, nb), -np.inf)
        S[0, :, : c + 1] = rng.standard_normal((4, c + 1))
        q2k, margin = orc.select(S, np.array([c]), topk, init, local)
        for h in range(4):
            forced = {b for b in range(c + 1) if b < init or b >= c - local + 1}
            free = [b for b in range(c + 1) if b not in forced]
            R = max(0, topk - len(forced))
            take = min(R, len(free))
            best = max(itertools.combinations(free, take), key=lambda s: sum(S[0, h, b] for b in s))
            want = sorted(forced | set(best))
            want += [-1] * (topk - len(want))
            assert q2k[0, h].tolist() == want


def test_selection_invariants_and_margin(orc):
    w = W.make_prefill([1000, 1500, 333], 21, topk=5, init_blocks=1, local_blocks=2)
    r = orc.prefill_select(w, tokens=np.arange(0, w.T, 23))
    for i, t in enumerate(r["tokens"]):
        c = r["c"][i]
        for g in range(4):
            row = r["q2k"][i, g]
            ids = row[row >= 0]
            n = min(w.topk, c + 1)
            assert len(ids) == n and np.all(row[n:] == -1)
            assert np.all(np.diff(ids) > 0) and ids.max() <= c
            forced = {b for b in range(c + 1) if b < 1 or b >= c - 1}
            assert forced <= set(ids.tolist())
            # margin: chosen free blocks score >= every unchosen free block
            S = r["S"][i, g, : c + 1]
            free = [b for b in range(c + 1) if b not in forced]
            chosen = [b for b in free if b in ids]
            dropped = [b for b in free if b not in ids]
            if chosen and dropped:
                gap = min(S[chosen]) - max(S[dropped])
                assert gap >= 0 and math.isclose(gap, r["margin"][i, g])
            else:
                assert r["margin"][i, g] == np.inf


# ------------------------------------------------------------ attention
def test_dense_reduction_equals_sdpa(orc):
    """topk >= number of blocks: sparse attention is dense causal
    document-local attention (torch SDPA, float64)."""
    w = W.make_prefill([130, 257, 64], 31, topk=16, init_blocks=0, local_blocks=1)
    r = orc.prefill(w)
    doc, pos = doc_geometry(w.cu_seqlens)
    T = w.T
    ok = (doc[:, None] == doc[None, :]) & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    ref = sdpa_reference(w, np.broadcast_to(ok, (4, T, T)).copy())
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def test_sparse_attention_equals_masked_sdpa(orc):
    w = W.make_prefill([700, 450], 41, topk=3, init_blocks=1, local_blocks=1)
    r = orc.prefill(w)
    mask = selection_mask(r["q2k"], w.cu_seqlens)
    ref = sdpa_reference(w, mask)
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def test_attention_closed_forms(orc):
    w = W.make_prefill([300, 200], 51, topk=2, init_blocks=0, local_blocks=1)
    # the first token of each document sees only itself: out = v[first]
    toks = w.cu_seqlens[:-1]
    r = orc.prefill(w, tokens=toks)
    v = bf16_f64(w.v)
    for i, t in enumerate(toks):
        for h in range(64):
            assert np.allclose(r["out"][i, h], v[t, h // 16], rtol=0, atol=1e-15)
    # constant keys: a uniform average of V over the key set
    w.k[:] = W.bf16_bits(np.full(w.k.shape, 0.5, np.float32))
    t = 299
    r = orc.prefill(w, tokens=[t])
    keys = [j for j in range(0, 300) if (j // 128) in r["q2k"][0, 0] and j <= t]
    assert np.allclose(r["out"][0, 0], v[keys, 0].mean(axis=0), atol=1e-12)
    # GQA: identical q rows within one KV group give identical outputs
    w.q[:, 16:32] = w.q[:, 16:17]
    r = orc.prefill(w, tokens=[5, 250, 420])
    for h in range(16, 32):
        assert np.array_equal(r["out"][:, h], r["out"][:, 16])


def test_q2k_row_order_does_not_matter(orc):
    w = W.make_prefill([900], 61, topk=4, init_blocks=0, local_blocks=1)
    toks = np.arange(0, 900, 37)
    r = orc.prefill(w, tokens=toks)
    rows = r["q2k"][:, :, ::-1].copy()
    out2 = orc.attend(w.q, w.k, w.v, rows, w.cu_seqlens, toks, w.scale)
    assert np.allclose(out2, r["out"], rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------ decode
def _gather_sequence(d, r):
    L = int(d.context_lens[r])
    slots = np.array([d.page_table[r, j // 128] * 128 + j % 128 for j in range(L)])
    return slots


@pytest.mark.parametrize("index_dtype", ["bf16", "fp8"])
def test_decode_equals_prefill_last_token(orc, index_dtype):
    d = W.make_decode([1, 129, 300, 640, 1000], 71, topk=4, init_blocks=1, local_blocks=1,
                      index_dtype=index_dtype)
    rd = orc.decode(d)
    for r in range(d.B):
        slots = _gather_sequence(d, r)
        L = len(slots)
        q = np.zeros((L, 64, 128), np.uint16)
        q[L - 1] = d.q[r]
        iq = np.zeros((L, 4, 128), d.iq.dtype)
        iq[L - 1] = d.iq[r]
        p = W.Prefill(name="g", cu_seqlens=np.array([0, L], np.int32), q=q,
                      k=d.k_cache[slots], v=d.v_cache[slots], iq=iq, ik=d.ik_cache[slots],
                      index_dtype=index_dtype, topk=d.topk, init_blocks=d.init_blocks,
                      local_blocks=d.local_blocks, scale=d.scale)
        rp = orc.prefill(p, tokens=[L - 1])
        nb = rp["S"].shape[2]
        assert np.array_equal(rd["S"][r, :, :nb], rp["S"][0])
        assert np.array_equal(rd["q2k"][r], rp["q2k"][0])
        assert np.array_equal(rd["out"][r], rp["out"][0])
        assert np.all(np.isfinite(rd["out"][r]))


def test_decode_page_permutation_invariance(orc):
    lens = [700, 1281, 256]
    a = W.make_decode(lens, 81, topk=3, identity_pages=True)
    b = W.make_decode(lens, 81, topk=3, identity_pages=False)
    # rebuild b's caches so that its pages hold a's logical content
    for r in range(a.B):
        for p in range((lens[r] + 127) // 128):
            pa, pb = a.page_table[r, p], b.page_table[r, p]
            for cache in ("k_cache", "v_cache", "ik_cache"):
                getattr(b, cache)[pb * 128:(pb + 1) * 128] = getattr(a, cache)[pa * 128:(pa + 1) * 128]
    ra, rb = orc.decode(a), orc.decode(b)
    assert not np.array_equal(a.page_table, b.page_table)
    for key in ("S", "q2k", "out"):
        assert np.array_equal(ra[key], rb[key])


def test_decode_dense_reduction_equals_sdpa(orc):
    d = W.make_decode([200, 513], 91, topk=16)
    rd = orc.decode(d)
    for r in range(d.B):
        slots = _gather_sequence(d, r)
        q = torch.from_numpy(bf16_f64(d.q[r]))[:, None, :]                      # [64,1,128]
        k = torch.from_numpy(bf16_f64(d.k_cache[slots])).permute(1, 0, 2)       # [4,L,128]
        v = torch.from_numpy(bf16_f64(d.v_cache[slots])).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k.repeat_interleave(16, 0), v.repeat_interleave(16, 0), scale=d.scale)
        assert np.allclose(rd["out"][r], o[:, 0].numpy(), rtol=1e-10, atol=1e-12)
