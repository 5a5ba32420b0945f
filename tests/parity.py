"""Helpers for the GPU parity tests: move seeded workloads to the device and
compare GPU results with the CPU oracle under the stated rules.

Selection rule: a GPU row must equal the oracle row whenever the oracle's
margin (R-th minus (R+1)-th non-forced score) exceeds 1e-2.  Otherwise the
rows may differ only by swapping blocks whose oracle scores lie within 1e-2
of the selection boundary; forced blocks and the -1 count always match.
Attention rule: max-abs <= 2e-2 and mean-abs <= 2e-3 against the oracle's
fp64 result (5e-2 max-abs where the indexer is fp8).
"""
import numpy as np
import torch

MARGIN_TOL = 1e-2


def dev(a: np.ndarray, device="cuda:0"):
    """numpy -> torch on the GPU, bf16 for uint16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device).view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def forced_set(c, init, local):
    return {b for b in range(c + 1) if b < init or b >= c - local + 1}


def check_selection(gpu_rows, ref, topk, init, local, tol=MARGIN_TOL):
    """gpu_rows, ref['q2k']: int32 [n,4,topk] (token-major).  Returns the
    [n,4] mask of rows that are identical; raises on any rule violation."""
    ref_rows = ref["q2k"]
    same = np.all(gpu_rows == ref_rows, axis=2)
    bad = np.argwhere(~same)
    for i, h in bad:
        g, o = gpu_rows[i, h], ref_rows[i, h]
        c = int(ref["c"][i])
        S = ref["S"][i, h]
        where = f"row (token #{i}, head {h}, c={c}): gpu {g.tolist()} oracle {o.tolist()}"
        assert ref["margin"][i, h] <= tol, f"margin {ref['margin'][i, h]:.4g} > {tol}: {where}"
        gi = g[g >= 0]
        assert np.all(g[len(gi):] == -1) and len(gi) == len(o[o >= 0]), f"-1 padding differs: {where}"
        assert np.all(np.diff(gi) > 0) and (len(gi) == 0 or gi.max() <= c), f"invalid row: {where}"
        F = forced_set(c, init, local)
        assert F <= set(gi.tolist()), f"forced blocks missing: {where}"
        free = np.array(sorted((b for b in range(c + 1) if b not in F), key=lambda b: (-S[b], b)))
        R = topk - len(F)
        s_R, s_R1 = S[free[R - 1]], S[free[R]]
        for b in set(gi.tolist()) - set(o.tolist()):
            assert S[b] >= s_R - tol, f"gpu chose block {b} (S={S[b]:.5f}) below s_R={s_R:.5f}: {where}"
        for b in set(o.tolist()) - set(gi.tolist()):
            assert S[b] <= s_R1 + tol, f"gpu dropped block {b} (S={S[b]:.5f}) above s_R+1={s_R1:.5f}: {where}"
    return same


def check_scores(gpu_S_head_major, ref, tokens, rel=1e-3):
    """gpu [4, nb, T] fp32 vs oracle [n,4,nb] fp64 on candidate entries b <= c."""
    g = gpu_S_head_major[:, :, tokens].transpose(2, 0, 1)  # [n,4,nb]
    r = ref["S"]
    nb = r.shape[2]
    g = g[:, :, :nb]
    cand = np.isfinite(r)
    scale = max(1.0, float(np.abs(r[cand]).max()))
    err = np.abs(g[cand] - r[cand])
    assert err.max() <= rel * scale, f"score max-abs error {err.max():.3g} > {rel * scale:.3g}"
    return float(err.max())


def check_attention(gpu_out, ref_out, max_tol=2e-2, mean_tol=2e-3, what="attention"):
    gpu_out = np.asarray(gpu_out, dtype=np.float64)
    assert np.all(np.isfinite(gpu_out)), f"{what}: non-finite output"
    err = np.abs(gpu_out - ref_out)
    assert err.max() <= max_tol, f"{what}: max-abs error {err.max():.4g} > {max_tol}"
    assert err.mean() <= mean_tol, f"{what}: mean-abs error {err.mean():.4g} > {mean_tol}"
    return float(err.max()), float(err.mean())


def sample_tokens(cu, per_doc=24, seed=0):
    """Token indices spanning every document: first and last token, tokens
    around the first and last block edges, and a seeded random spread."""
    rng = np.random.default_rng(seed)
    out = set()
    for d in range(len(cu) - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        L = e - s
        out.update({s, e - 1})
        out.update(s + p for p in (127, 128, 255, 256) if p < L)
        last_edge = ((L - 1) // 128) * 128
        out.update(s + p for p in (last_edge - 1, last_edge) if 0 <= p < L)
        if L > 2:
            out.update((s + rng.integers(0, L, size=min(per_doc, L))).tolist())
    return np.array(sorted(out), dtype=np.int32)


def sample_tiles(cu, n_tiles=128, tile=16, seed=0):
    """Tokens of whole document-aligned tiles of ``tile`` consecutive tokens
    (the prefill attention's work unit), about ``n_tiles`` in all, spread over
    every document in proportion to its length: each document's first and
    last tile (the last one may be partial), the tiles holding its block
    edges 127/128 and its last block's start, and seeded random tiles
    elsewhere.  Returns sorted token indices."""
    rng = np.random.default_rng(seed)
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    out = set()
    for d in range(len(cu) - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        L = e - s
        nt = -(-L // tile)
        pick = {0, nt - 1, 127 // tile, 128 // tile, ((L - 1) // 128) * 128 // tile}
        want = max(2, int(round(n_tiles * L / T)))
        extra = rng.choice(nt, size=min(nt, want), replace=False)
        pick.update(int(x) for x in extra)
        for i in pick:
            if 0 <= i < nt:
                out.update(range(s + i * tile, min(e, s + (i + 1) * tile)))
    return np.array(sorted(out), dtype=np.int32)
