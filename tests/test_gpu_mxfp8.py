"""GPU parity of the MXFP8 output path (E4M3 elements + E8M0 scale per 32).

- msa_mxfp8_quantize against the oracle's quantiser, bit for bit, on seeded
  bit-level bf16 matrices covering every block kind (random, zero, on-grid,
  half-way, saturating, subnormal, wide span).
- msa_sparse_attend_decode_paged_mxfp8 equals msa_mxfp8_quantize of the bf16
  output that msa_sparse_attend_decode_paged returns for the same inputs (the
  defining property of the MXFP8 decode output), and its dequantised values
  stay within the attention tolerance plus half an E4M3 unit of the oracle.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import oracle
import workloads as W
from oracle import mxfp8 as mx
from parity import dev

pytestmark = pytest.mark.gpu


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("rows,cols,seed", [(1, 32, 1), (3, 96, 2), (64, 256, 3), (17, 8192, 4),
                                            (250, 1024, 5)])
def test_quantize_matches_oracle_bit_exact(rows, cols, seed):
    print(f"[mxfp8 quantize] {rows}x{cols} seed {seed}", flush=True)
    bits = W.mx_matrix(seed, rows, cols)
    q_ref, s_ref = mx.quantize(bf16_f64(bits))
    q, s = msa.mxfp8_quantize(dev(bits))
    q, s = q.cpu().numpy(), s.cpu().numpy()
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, f"{len(bad)} element codes differ, first {bad[:4].tolist()}"
    assert np.array_equal(s, s_ref), "scale codes differ"


DECODE_CASES = [
    ("mixed_bf16", [1, 127, 128, 129, 1000, 5000, 20000], 16, 0, 1, "bf16"),
    ("fp8idx_topk5_init1", [64 + 997 * i for i in range(20)], 5, 1, 1, "fp8"),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: c[0])
def test_decode_mxfp8(case):
    name, lens, topk, init, local, idt = case
    print(f"[decode mxfp8] {name}", flush=True)
    d = W.make_decode(lens, 900 + len(name), topk=topk, init_blocks=init, local_blocks=local,
                      index_dtype=idt)
    args = (dev(d.q), dev(d.iq), dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache), dev(d.page_table),
            dev(d.context_lens), d.max_context_len, topk, init, local, d.scale)
    out = msa.sparse_attend_decode_paged(*args)
    (oq, osc), q2k = msa.sparse_attend_decode_paged_mxfp8(*args, return_q2k=True)
    # the MXFP8 output is the quantisation of the bf16 output
    rq, rs = msa.mxfp8_quantize(out.reshape(d.B, 64 * 128))
    assert torch.equal(oq, rq) and torch.equal(osc, rs)
    # and close to the oracle's attention (on rows where the selection agrees)
    ref = oracle.decode(d)
    got_sel = q2k.cpu().numpy().transpose(1, 0, 2)
    rows = np.all(got_sel == ref["q2k"], axis=(1, 2))
    assert rows.sum() >= len(lens) - 1
    deq = mx.dequantize(oq.cpu().numpy(), osc.cpu().numpy()).reshape(d.B, 64, 128)
    unit = np.exp2(osc.cpu().numpy().astype(np.float64) - 127).repeat(32, axis=1).reshape(d.B, 64, 128)
    att = 2e-2 if idt == "bf16" else 5e-2
    a = np.abs(ref["out"])
    # attention tolerance + half an E4M3 step (2^-4 relative, or 2^-10 of the
    # block unit below the normal range) + the saturation excess of block
    # maxima past 448 units (scale = 2^(floor(log2 amax) - 8) lets them reach 512)
    tol = att + np.maximum(2.0 ** -4 * a, 2.0 ** -10 * unit) + np.maximum(0.0, a + att - 448 * unit)
    err = np.abs(deq - ref["out"])[rows]
    assert np.all(err <= tol[rows]), f"max excess {np.max(err - tol[rows]):.3g}"
