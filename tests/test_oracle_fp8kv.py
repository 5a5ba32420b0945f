"""Pins for the FP8-K/V decode oracle (oracle/fp8kv.py).

- With power-of-two scales the dequantised caches are exactly bf16, so the
  numpy attention must equal the pinned C oracle's decode attention on those
  bf16 bits (catches a wrong slot, block, head group or softmax).
- A one-token context returns that token's dequantised V row (catches a
  dropped or doubled scale).
- NaN-poisoned tail slots never reach the output.
"""
import numpy as np
import torch

import oracle
import workloads as W
from oracle import fp8kv


def bf16_bits_exact(x):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    assert torch.equal(t.double(), torch.from_numpy(np.ascontiguousarray(x))), "not bf16-exact"
    return t.view(torch.int16).numpy().view(np.uint16)


def q_f64(d):
    return torch.from_numpy(d.q.view(np.int16)).view(torch.bfloat16).double().numpy()


def test_matches_c_oracle_on_exact_dequantisation():
    d = W.make_decode([1, 127, 129, 700, 3000], 12, topk=5, init_blocks=1, local_blocks=1,
                      kv_dtype="fp8", k_scale=0.5, v_scale=0.125, poison_tail=False)
    ref = oracle.decode(W.make_decode([1, 127, 129, 700, 3000], 12, topk=5, init_blocks=1,
                                      local_blocks=1))  # same selection inputs (index caches)
    kf, vf = fp8kv.dequantize(d.k_cache, d.k_scale), fp8kv.dequantize(d.v_cache, d.v_scale)
    ours = fp8kv.decode_attend(q_f64(d), kf, vf, d.page_table, d.context_lens, ref["q2k"], d.scale)
    c_out = oracle.decode_attend(d.q, bf16_bits_exact(kf), bf16_bits_exact(vf), d.page_table,
                                 d.context_lens, ref["q2k"], d.scale)
    assert np.allclose(ours, c_out, rtol=1e-12, atol=1e-12)


def test_single_token_context_returns_its_value_row():
    d = W.make_decode([1], 13, topk=2, kv_dtype="fp8", k_scale=0.37, v_scale=0.91)
    kf, vf = fp8kv.dequantize(d.k_cache, d.k_scale), fp8kv.dequantize(d.v_cache, d.v_scale)
    q2k = np.array([[[0, -1]] * 4])
    out = fp8kv.decode_attend(q_f64(d), kf, vf, d.page_table, d.context_lens, q2k, d.scale)
    slot = d.page_table[0, 0] * 128
    for g in range(4):
        assert np.array_equal(out[0, 16 * g:16 * g + 16], np.broadcast_to(vf[slot, g], (16, 128)))


def test_poisoned_tails_stay_out():
    d = W.make_decode([5, 300, 1000], 14, topk=16, kv_dtype="fp8")
    kf, vf = fp8kv.dequantize(d.k_cache, d.k_scale), fp8kv.dequantize(d.v_cache, d.v_scale)
    assert np.isnan(kf).any()
    q2k = np.tile(np.arange(16)[None, None, :], (3, 4, 1))
    out = fp8kv.decode_attend(q_f64(d), kf, vf, d.page_table, d.context_lens, q2k, d.scale)
    assert np.all(np.isfinite(out))
