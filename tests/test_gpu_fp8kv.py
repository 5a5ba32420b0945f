"""GPU parity of decode over an FP8 (E4M3FN) main K/V cache with per-tensor scales.

- Against the fp64 oracle (oracle/fp8kv.py) on the oracle's own selection,
  with power-of-two and arbitrary scales, bf16 and fp8 indexers, NaN-poisoned
  tails: attention tolerance as for the bf16 cache.
- With power-of-two scales, E4M3 values times the scale are exact in bf16:
  the fp8 path must then equal the bf16 path on the dequantised caches bit
  for bit (same arithmetic after an exact conversion).
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import oracle
import workloads as W
from oracle import fp8kv
from parity import check_attention, dev

pytestmark = pytest.mark.gpu


def bf16(bits):
    return dev(bits).view(torch.bfloat16) if bits.dtype == np.uint16 else dev(bits)


CASES = [
    ("mixed_pow2", [1, 127, 128, 129, 1000, 5000, 20000], 16, 0, 1, "bf16", 0.5, 0.25),
    ("batch20_scales", [64 + 997 * i for i in range(20)], 5, 1, 1, "bf16", 0.37, 1.7),
    ("fp8_indexer", [1, 129, 3000, 9000], 6, 2, 1, "fp8", 0.125, 0.0625),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fp8kv_decode_matches_oracle(case):
    name, lens, topk, init, local, idt, ks, vs = case
    print(f"[decode fp8kv] {name}", flush=True)
    d = W.make_decode(lens, 500 + len(name), topk=topk, init_blocks=init, local_blocks=local,
                      index_dtype=idt, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    out, q2k = msa.sparse_attend_decode_paged_fp8kv(
        bf16(d.q), bf16(d.iq), dev(d.k_cache), dev(d.v_cache), d.k_scale, d.v_scale, bf16(d.ik_cache),
        dev(d.page_table), dev(d.context_lens), d.max_context_len, topk, init, local, d.scale,
        return_q2k=True)
    got_sel = q2k.cpu().numpy().transpose(1, 0, 2)
    # selection only reads the index caches: compare against the oracle's
    nb_max = (d.max_context_len + 127) // 128
    S = oracle.decode_scores(d.iq, d.ik_cache, d.page_table, d.context_lens, nb_max, idt)
    ref_sel, _ = oracle.select(S, oracle.decode_query_blocks(d.context_lens), topk, init, local)
    rows = np.all(got_sel == ref_sel, axis=(1, 2))
    assert rows.sum() >= len(lens) - 1
    qf = torch.from_numpy(d.q.view(np.int16)).view(torch.bfloat16).double().numpy()
    ref = fp8kv.decode_attend(qf, fp8kv.dequantize(d.k_cache, d.k_scale),
                              fp8kv.dequantize(d.v_cache, d.v_scale), d.page_table, d.context_lens,
                              ref_sel, d.scale)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got)), "NaN from poisoned tail slots"
    check_attention(got[rows], ref[rows], max_tol=2e-2 if idt == "bf16" else 5e-2, what=name)


def test_fp8kv_equals_bf16_path_on_exact_dequantisation():
    lens = [1, 300, 4097, 12000]
    d = W.make_decode(lens, 77, topk=8, kv_dtype="fp8", k_scale=0.5, v_scale=0.125, poison_tail=False)
    kf = fp8kv.dequantize(d.k_cache, d.k_scale)
    vf = fp8kv.dequantize(d.v_cache, d.v_scale)
    kb = torch.from_numpy(kf).to(torch.bfloat16)
    vb = torch.from_numpy(vf).to(torch.bfloat16)
    assert torch.equal(kb.double(), torch.from_numpy(kf)) and torch.equal(vb.double(), torch.from_numpy(vf))
    args = (bf16(d.page_table), bf16(d.context_lens), d.max_context_len, 8, 0, 1, d.scale)
    a = msa.sparse_attend_decode_paged_fp8kv(bf16(d.q), bf16(d.iq), dev(d.k_cache), dev(d.v_cache),
                                             d.k_scale, d.v_scale, bf16(d.ik_cache), *args)
    b = msa.sparse_attend_decode_paged(bf16(d.q), bf16(d.iq), kb.cuda(), vb.cuda(), bf16(d.ik_cache), *args)
    # same keys, same MFMA operands; only the score scale is formed differently
    # (scale * log2e * k_scale in one product vs. scores of k*k_scale)
    diff = (a.float() - b.float()).abs().max().item()
    assert diff <= 1e-2, diff
