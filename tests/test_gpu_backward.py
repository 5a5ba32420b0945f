"""GPU parity of the sparse prefill attention backward.

The selection q2k comes from the oracle (or from seeded synthetic rows),
never from the GPU.  The GPU forward with log-sum-exp feeds the GPU backward,
as in a training step, and dq, dk, dv are compared with the oracle's fp64
gradients of the same rows.  Also: the forward's lse against the oracle's,
bitwise repeatability of the backward (its sums run in a fixed order), and
keys that no row attends to get zero gradients.

Tolerance, from the arithmetic: the GPU rounds the MFMA operands P and dS
to bf16 (relative error <= 2^-9 per term), accumulates in fp32 and rounds
each gradient to bf16 once (<= 2^-9).  So the mean error is about 2^-9 of
the mean magnitude; the test allows twice that (4e-3 of mean|ref|) and a
largest error of 1e-2 of max|ref|.  lse (fp32, exp2/log2 domain) within 1e-4.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import oracle
import workloads as W
from parity import dev

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 1e-2, 4e-3


def run_gpu(w, rows_tm, dout):
    """rows_tm: token-major [T,4,topk] selection; returns lse, dq, dk, dv (numpy)."""
    q2k = dev(np.ascontiguousarray(rows_tm.transpose(1, 0, 2)))
    q, k, v, cu = dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens)
    out, lse = msa.sparse_attend_prefill(q, k, v, q2k, cu, w.max_seqlen, w.scale, return_lse=True)
    dq, dk, dv = msa.sparse_attend_prefill_backward(q, k, v, out, lse, dev(dout), q2k, cu, w.max_seqlen,
                                                    w.scale)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(lse), f(dq), f(dk), f(dv)


def rel_errors(got, ref):
    err = np.abs(got - ref)
    return err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()


def random_rows(cu, topk, seed):
    """Rows with -1 padding, repeats, ids past the query block and empty key sets."""
    T = int(cu[-1])
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    c = (np.arange(T) - cu[doc]) // 128
    g = np.random.default_rng(seed)
    rows = g.integers(-1, c.max() + 3, size=(T, 4, topk)).astype(np.int32)
    rows[:, :, 1] = rows[:, :, 0]
    rows[:, :, 2] = np.where(g.random((T, 4)) < 0.8, c[:, None], rows[:, :, 2])
    rows[5, 1, :] = -1
    rows[6, 2, :] = c[6] + 1
    return rows


def dense_rows(cu, topk):
    T = int(cu[-1])
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    c = (np.arange(T) - cu[doc]) // 128
    rows = np.full((T, 4, topk), -1, dtype=np.int32)
    for t, ct in enumerate(c):
        rows[t, :, :ct + 1] = np.arange(ct + 1)
    return rows


CASES = [
    ("single_2048_topk4", [2048], 4, 0, 1, "oracle"),
    ("ragged_docs", [1, 127, 129, 300, 700], 3, 1, 1, "oracle"),
    ("dense_topk_ge_nb", [600, 257], 5, 0, 1, "dense"),
    ("random_rows", [130, 300, 1, 517], 6, 0, 1, "random"),
    # 1051 document blocks: the list build's block windows (1024 blocks) come twice
    ("many_docs_two_windows", [300, 1, 2, 129] + [1 + i % 3 for i in range(1040)] + [260, 45], 5, 0, 1,
     "random"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_backward_matches_oracle(case):
    name, lens, topk, init, local, how = case
    print(f"[backward] {name}", flush=True)
    w = W.make_prefill(lens, 700 + len(name), topk=topk, init_blocks=init, local_blocks=local)
    if how == "oracle":
        rows = oracle.prefill_select(w)["q2k"]
    elif how == "dense":
        rows = dense_rows(w.cu_seqlens, topk)
    else:
        rows = random_rows(w.cu_seqlens, topk, 71)
    dout = W.grad_out(800 + len(name), w.T)
    ref = oracle.attend_backward(w.q, w.k, w.v, dout, rows, w.cu_seqlens, w.scale)
    lse, dq, dk, dv = run_gpu(w, rows, dout)
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(lse), fin)
    lse_err = np.abs(lse[fin] - ref["lse"][fin]).max()
    stats = {"lse": lse_err}
    for nm, g, r in (("dq", dq, ref["dq"]), ("dk", dk, ref["dk"]), ("dv", dv, ref["dv"])):
        assert np.all(np.isfinite(g)), nm
        stats[nm] = rel_errors(g, r)
    print(f"[backward] {name} errors {stats}", flush=True)
    assert lse_err <= 1e-4
    for nm in ("dq", "dk", "dv"):
        mx, mean = stats[nm]
        assert mx <= MAX_REL and mean <= MEAN_REL, f"{nm}: max {mx:.3g} mean {mean:.3g} (relative to the reference scale)"


def test_backward_is_repeatable_and_unattended_keys_get_zero():
    print("[backward] repeatable", flush=True)
    w = W.make_prefill([700, 300], 77, topk=2, init_blocks=0, local_blocks=0)
    # every token selects block 0 and its own block, except that the tokens
    # of block 3 of the first document select block 0 only: block 3 there is
    # attended by no row
    T = w.T
    doc = np.searchsorted(w.cu_seqlens, np.arange(T), side="right") - 1
    blk = (np.arange(T) - w.cu_seqlens[doc]) // 128
    rows = np.full((T, 4, 2), -1, dtype=np.int32)
    rows[:, :, 0] = 0
    own = (blk > 0) & ~((doc == 0) & (blk == 3))
    rows[own, :, 1] = blk[own, None]
    dout = W.grad_out(78, T)
    q2k = dev(np.ascontiguousarray(rows.transpose(1, 0, 2)))
    q, k, v, cu = dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens)
    out, lse = msa.sparse_attend_prefill(q, k, v, q2k, cu, w.max_seqlen, w.scale, return_lse=True)
    a = msa.sparse_attend_prefill_backward(q, k, v, out, lse, dev(dout), q2k, cu, w.max_seqlen, w.scale)
    b = msa.sparse_attend_prefill_backward(q, k, v, out, lse, dev(dout), q2k, cu, w.max_seqlen, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    dk, dv = a[1].float().cpu().numpy(), a[2].float().cpu().numpy()
    dead = (doc == 0) & (blk == 3)
    assert dead.sum() == 128
    assert np.all(dk[dead] == 0) and np.all(dv[dead] == 0)
    assert np.all(np.abs(dv[~dead]).sum(axis=-1) > 0)


def test_backward_full_size_32k_sampled():
    """32768-token document, topk 16, on a synthetic selection shaped like the
    planted workload's (hot blocks chosen by most rows).  dq and lse on
    sampled tokens, dk and dv on sampled keys of blocks few rows select (the
    oracle needs lse and D of every row that attends to a key), and over all
    keys the sums sum_j dv_jg = sum of dO over group g and sum_j dk_jg = 0."""
    print("[backward] 32k full size", flush=True)
    w = W.config(2)
    rows = W.synthetic_q2k(2, w.cu_seqlens, 16, 0, 1)
    dout = W.grad_out(2, w.T)
    lse, dq, dk, dv = run_gpu(w, rows, dout)
    T = w.T
    toks = np.unique(np.concatenate([[0, 1, 127, 128, 129, T - 129, T - 128, T - 1],
                                     np.random.default_rng(3).integers(0, T, 16)])).astype(np.int32)
    r_lse, _, r_dq = oracle.attend_backward_rows(w.q, w.k, w.v, dout, rows, w.cu_seqlens, toks, w.scale)
    assert np.abs(lse[toks] - r_lse).max() <= 1e-4
    mx, mean = rel_errors(dq[toks], r_dq)
    print(f"[backward] 32k dq rows: max {mx:.3g} mean {mean:.3g}", flush=True)
    assert mx <= MAX_REL and mean <= MEAN_REL
    # keys of blocks that few rows select (not hot in any KV head)
    blk = np.arange(T) // 128
    counts = np.zeros((4, 256), dtype=np.int64)
    for g in range(4):
        sel = rows[:, g, :]
        counts[g] = np.bincount(sel[sel >= 0], minlength=256)
    quiet = np.nonzero(counts.max(axis=0) <= 400)[0]
    pick_blocks = quiet[np.linspace(0, len(quiet) - 1, 3).astype(int)]
    keys = np.concatenate([b * 128 + np.array([0, 77, 127]) for b in pick_blocks]).astype(np.int32)
    users = np.nonzero(np.isin(rows, pick_blocks).any(axis=(1, 2)))[0].astype(np.int32)
    u_lse, u_D, _ = oracle.attend_backward_rows(w.q, w.k, w.v, dout, rows, w.cu_seqlens, users, w.scale)
    lse_full = np.full((T, 64), np.nan)
    D_full = np.full((T, 64), np.nan)
    lse_full[users], D_full[users] = u_lse, u_D
    r_dk, r_dv = oracle.attend_backward_keys(w.q, w.k, w.v, dout, rows, w.cu_seqlens, lse_full, D_full,
                                             keys, w.scale)
    for nm, g_, r_ in (("dk", dk[keys], r_dk), ("dv", dv[keys], r_dv)):
        mx, mean = rel_errors(g_, r_)
        print(f"[backward] 32k {nm} keys: max {mx:.3g} mean {mean:.3g}", flush=True)
        assert mx <= MAX_REL and mean <= MEAN_REL
    # whole-tensor sums (every row attends to its own block, so every row counts)
    dO = torch.from_numpy(dout.view(np.int16)).view(torch.bfloat16).double().numpy()
    for g in range(4):
        want = dO[:, 16 * g:16 * g + 16].sum(axis=(0, 1))
        got = dv[:, g].sum(axis=0)
        assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(dv[:, g]).sum(axis=0) + 1e-6)
        assert np.all(np.abs(dk[:, g].sum(axis=0)) <= 2.0 ** -7 * np.abs(dk[:, g]).sum(axis=0) + 1e-6)


def test_backward_packed_documents_sampled():
    """The packed microbatch (2 x 16384 rows of log-uniform documents, init 1,
    local 1, topk 16) on a synthetic selection: dq and lse on tokens spread
    over every document, dk and dv on keys of the shortest document (the
    oracle gets lse and D of all its tokens), and the whole-tensor sums."""
    from parity import sample_tokens
    print("[backward] packed documents", flush=True)
    w = W.config(3)
    rows = W.synthetic_q2k(3, w.cu_seqlens, 16, w.init_blocks, w.local_blocks)
    dout = W.grad_out(3, w.T)
    lse, dq, dk, dv = run_gpu(w, rows, dout)
    cu = w.cu_seqlens
    toks = sample_tokens(cu, per_doc=3, seed=4)
    r_lse, _, r_dq = oracle.attend_backward_rows(w.q, w.k, w.v, dout, rows, cu, toks, w.scale)
    assert np.abs(lse[toks] - r_lse).max() <= 1e-4
    mx, mean = rel_errors(dq[toks], r_dq)
    print(f"[backward] packed dq rows ({len(toks)}): max {mx:.3g} mean {mean:.3g}", flush=True)
    assert mx <= MAX_REL and mean <= MEAN_REL
    lens = np.diff(cu)
    d = int(np.argmin(lens))
    s, L = int(cu[d]), int(lens[d])
    keys = (s + np.unique(np.array([0, 1, 127, 128, L // 2, L - 1]).clip(0, L - 1))).astype(np.int32)
    users = np.arange(s, s + L, dtype=np.int32)
    u_lse, u_D, _ = oracle.attend_backward_rows(w.q, w.k, w.v, dout, rows, cu, users, w.scale)
    lse_full = np.full((w.T, 64), np.nan)
    D_full = np.full((w.T, 64), np.nan)
    lse_full[users], D_full[users] = u_lse, u_D
    r_dk, r_dv = oracle.attend_backward_keys(w.q, w.k, w.v, dout, rows, cu, lse_full, D_full, keys, w.scale)
    for nm, g_, r_ in (("dk", dk[keys], r_dk), ("dv", dv[keys], r_dv)):
        mx, mean = rel_errors(g_, r_)
        print(f"[backward] packed {nm} keys: max {mx:.3g} mean {mean:.3g}", flush=True)
        assert mx <= MAX_REL and mean <= MEAN_REL
    dO = torch.from_numpy(dout.view(np.int16)).view(torch.bfloat16).double().numpy()
    for g in range(4):
        want = dO[:, 16 * g:16 * g + 16].sum(axis=(0, 1))
        got = dv[:, g].sum(axis=0)
        assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(dv[:, g]).sum(axis=0) + 1e-6)
        assert np.all(np.abs(dk[:, g].sum(axis=0)) <= 2.0 ** -7 * np.abs(dk[:, g]).sum(axis=0) + 1e-6)
