"""Pins for the backward oracle (oracle_attend_backward_rows / _keys).

The oracle writes out the gradient of softmax attention over each row's
selected keys.  It is pinned against torch autograd (fp64, CPU), which
differentiates a forward written independently:
- topk covering every block reduces the method to dense document-causal
  attention;
- random selection rows (with -1 padding, repeats, ids past the query's
  block, and rows whose key set is empty) use a mask that is first tied to
  the pinned forward oracle (same output to 1e-12).
Closed-form invariants catch a wrong D term or a lost scale on their own:
sum_j dv_jg = sum of dO over group g's non-empty rows, sum_j dk_jg = 0,
and a row with a single key has dq = 0 exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def inputs(lens, seed):
    T = sum(lens)
    ss = np.random.SeedSequence(seed).spawn(3)
    q = W.normal_bf16(ss[0], (T, 64, 128))
    k = W.normal_bf16(ss[1], (T, 4, 128))
    v = W.normal_bf16(ss[2], (T, 4, 128))
    dout = W.grad_out(seed, T)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, dout, cu


def doc_pos(cu):
    T = int(cu[-1])
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    return doc, np.arange(T) - cu[doc]


def allowed_mask(q2k_full, cu):
    """[4, T, T] bool: key j is in row (g, t)'s key set."""
    T = int(cu[-1])
    doc, pos = doc_pos(cu)
    same = (doc[:, None] == doc[None, :]) & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    blk = pos // 128
    m = np.zeros((4, T, T), dtype=bool)
    for g in range(4):
        sel = (q2k_full[:, g, :, None] == blk[None, None, :]).any(axis=1)  # [T(t), T(j)]
        m[g] = same & sel
    return m


def torch_grads(q, k, v, dout, mask, scale):
    Q, K, V = (f64(a).requires_grad_(True) for a in (q, k, v))
    dO = f64(dout)
    Kh, Vh = K.repeat_interleave(16, dim=1), V.repeat_interleave(16, dim=1)
    S = scale * torch.einsum("thd,jhd->htj", Q, Kh)
    m = torch.from_numpy(mask).repeat_interleave(16, dim=0)
    nonempty = m.any(-1, keepdim=True)
    S = S.masked_fill(~m, -torch.inf)
    lse = torch.logsumexp(S, -1, keepdim=True)
    P = torch.where(m, torch.exp(S - torch.where(nonempty, lse, torch.zeros_like(lse))), 0.0)
    O = torch.einsum("htj,jhd->thd", P, Vh)
    (O * dO).sum().backward()
    return dict(out=O.detach().numpy(), lse=lse[..., 0].T.detach().numpy(), dq=Q.grad.numpy(),
                dk=K.grad.numpy(), dv=V.grad.numpy(), nonempty=nonempty[..., 0].T.numpy())


def close(a, b, tol=1e-9):
    a, b = np.asarray(a), np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b[fin]))), err


def dense_rows(cu, topk):
    doc, pos = doc_pos(cu)
    c = pos // 128
    rows = np.full((len(c), 4, topk), -1, dtype=np.int32)
    for t, ct in enumerate(c):
        rows[t, :, :ct + 1] = np.arange(ct + 1)
    return rows


def test_dense_reduction_matches_autograd():
    lens = [200, 257]  # 2 and 3 blocks
    q, k, v, dout, cu = inputs(lens, 41)
    scale = 1 / np.sqrt(128)
    rows = dense_rows(cu, 3)
    ref = torch_grads(q, k, v, dout, allowed_mask(rows, cu), scale)
    got = oracle.attend_backward(q, k, v, dout, rows, cu, scale)
    for name in ("lse", "dq", "dk", "dv"):
        close(got[name], ref[name])


def random_rows(cu, topk, seed):
    doc, pos = doc_pos(cu)
    c = pos // 128
    g = np.random.default_rng(seed)
    rows = g.integers(-1, c.max() + 3, size=(len(c), 4, topk)).astype(np.int32)  # ids past c, -1
    rows[:, :, 1] = rows[:, :, 0]  # repeats
    keep_local = g.random((len(c), 4)) < 0.8
    rows[:, :, 2] = np.where(keep_local, c[:, None], rows[:, :, 2])
    rows[5, 1, :] = -1  # an empty key set
    rows[6, 2, :] = c[6] + 1  # only ids past c: empty too
    return rows


def test_sparse_rows_match_autograd_and_forward():
    lens = [130, 300, 1]
    q, k, v, dout, cu = inputs(lens, 42)
    scale = 0.07
    rows = random_rows(cu, 5, 43)
    mask = allowed_mask(rows, cu)
    ref = torch_grads(q, k, v, dout, mask, scale)
    T = int(cu[-1])
    # the mask is the forward's key set: torch's forward equals the pinned forward oracle
    fwd = oracle.attend(q, k, v, rows, cu, np.arange(T, dtype=np.int32), scale)
    close(ref["out"], fwd, 1e-12)
    got = oracle.attend_backward(q, k, v, dout, rows, cu, scale)
    for name in ("lse", "dq", "dk", "dv"):
        close(got[name], ref[name])
    assert not ref["nonempty"][5, 16] and np.all(got["dq"][5, 16:32] == 0)


def test_invariants_and_single_key_row():
    lens = [129, 383]
    q, k, v, dout, cu = inputs(lens, 44)
    scale = 1 / np.sqrt(128)
    rows = random_rows(cu, 4, 45)
    got = oracle.attend_backward(q, k, v, dout, rows, cu, scale)
    nonempty = np.isfinite(got["lse"])  # [T, 64]
    dO = f64(dout).numpy()
    for g in range(4):
        hs = slice(16 * g, 16 * g + 16)
        want = (dO[:, hs] * nonempty[:, hs, None]).sum(axis=(0, 1))
        np.testing.assert_allclose(got["dv"][:, g].sum(axis=0), want, rtol=0, atol=1e-9 * T_abs(want))
        assert np.max(np.abs(got["dk"][:, g].sum(axis=0))) <= 1e-10 * np.abs(got["dk"]).max() * len(q)
    # the first token of a document attends to itself alone (local block)
    for t in cu[:-1]:
        for g in range(4):
            if (rows[t, g] == 0).any():
                assert np.all(got["dq"][t, 16 * g:16 * g + 16] == 0.0)


def T_abs(x):
    return max(1.0, float(np.max(np.abs(x))))


@pytest.mark.parametrize("which", ["tokens", "keys"])
def test_subsets_equal_the_full_run(which):
    lens = [260, 70]
    q, k, v, dout, cu = inputs(lens, 46)
    rows = random_rows(cu, 3, 47)
    full = oracle.attend_backward(q, k, v, dout, rows, cu, 0.09)
    pick = np.array([0, 1, 129, 259, 260, 329], dtype=np.int32)
    if which == "tokens":
        lse, D, dq = oracle.attend_backward_rows(q, k, v, dout, rows, cu, pick, 0.09)
        assert np.array_equal(dq, full["dq"][pick]) and np.array_equal(D, full["D"][pick])
    else:
        dk, dv = oracle.attend_backward_keys(q, k, v, dout, rows, cu, full["lse"], full["D"], pick, 0.09)
        assert np.array_equal(dk, full["dk"][pick]) and np.array_equal(dv, full["dv"][pick])
