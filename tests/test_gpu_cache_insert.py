"""GPU parity of the paged-cache insertion (msa_cache_insert).

- Gather-back: every inserted token's K, V and index-K rows read back from
  their slots equal the inputs (bf16 bit for bit; the E4M3 index cache equal
  to the oracle's nearest-E4M3 rounding of the bf16 values); slots not named,
  and tokens with a negative or out-of-range slot, leave the caches untouched.
- End to end: caches rebuilt by the producer from a decode workload's logical
  rows give the same decode output, bit for bit, as the workload's own caches.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_score_amd as msa
import workloads as W
from oracle import mxfp8 as mx
from parity import dev

pytestmark = pytest.mark.gpu


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def to_bf16(bits):
    return dev(bits).view(torch.bfloat16) if bits.dtype == np.uint16 else dev(bits)


@pytest.mark.parametrize("index_dtype", ["bf16", "fp8"])
def test_insert_gather_back(index_dtype):
    print(f"[cache insert] {index_dtype}", flush=True)
    n, num_slots = 300, 1024
    ss = np.random.SeedSequence(77).spawn(6)
    k = W.normal_bf16(ss[0], (n, 4, 128))
    v = W.normal_bf16(ss[1], (n, 4, 128))
    # index rows over a wide range: normed rows, some scaled past E4M3's 448
    z = W.rms_normalise(W.normal_f32(ss[2], (n, 1, 128)))
    z[::7] *= 60.0
    ik = W.bf16_bits(z)
    g = np.random.default_rng(ss[3])
    slots = g.permutation(num_slots)[:n].astype(np.int32)
    slots[::20] = -1
    slots[5::37] = num_slots + 3  # out of range: skipped
    kc0 = g.integers(0, 1 << 16, size=(num_slots, 4, 128), dtype=np.uint16)
    vc0 = g.integers(0, 1 << 16, size=(num_slots, 4, 128), dtype=np.uint16)
    if index_dtype == "bf16":
        ikc0 = g.integers(0, 1 << 16, size=(num_slots, 1, 128), dtype=np.uint16)
    else:
        ikc0 = g.integers(0, 256, size=(num_slots, 1, 128), dtype=np.uint8)
    kc, vc, ikc = to_bf16(kc0.copy()), to_bf16(vc0.copy()), to_bf16(ikc0.copy())
    msa.cache_insert(to_bf16(k), to_bf16(v), to_bf16(ik), dev(slots), kc, vc, ikc)
    kc = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    vc = vc.view(torch.int16).cpu().numpy().view(np.uint16)
    ikc = (ikc.view(torch.int16).cpu().numpy().view(np.uint16) if index_dtype == "bf16"
           else ikc.view(torch.uint8).cpu().numpy())
    ok = (slots >= 0) & (slots < num_slots)
    s = slots[ok]
    assert np.array_equal(kc[s], k[ok]) and np.array_equal(vc[s], v[ok])
    if index_dtype == "bf16":
        assert np.array_equal(ikc[s], ik[ok])
    else:
        assert np.array_equal(ikc[s], mx.e4m3_nearest(bf16_f64(ik[ok])))
    untouched = np.setdiff1d(np.arange(num_slots), s)
    assert np.array_equal(kc[untouched], kc0[untouched]) and np.array_equal(vc[untouched], vc0[untouched])
    assert np.array_equal(ikc[untouched], ikc0[untouched])


def test_decode_over_producer_built_caches():
    print("[cache insert] end to end", flush=True)
    lens = [1, 127, 128, 300, 4097]
    d = W.make_decode(lens, 31, topk=5, init_blocks=0, local_blocks=1)
    # logical rows of every request, then their slots
    slots = np.concatenate([d.page_table[r, np.arange(L) // 128] * 128 + np.arange(L) % 128
                            for r, L in enumerate(lens)]).astype(np.int32)
    k, v, ik = d.k_cache[slots], d.v_cache[slots], d.ik_cache[slots]
    num_slots = d.k_cache.shape[0]
    kc = torch.zeros((num_slots, 4, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ikc = torch.zeros((num_slots, 1, 128), dtype=torch.bfloat16, device="cuda")
    msa.cache_insert(to_bf16(k), to_bf16(v), to_bf16(ik), dev(slots), kc, vc, ikc)
    assert torch.equal(kc[dev(slots).long()].view(torch.int16).cpu(), torch.from_numpy(k.view(np.int16)))
    common = (to_bf16(d.q), to_bf16(d.iq))
    tail = (dev(d.page_table), dev(d.context_lens), d.max_context_len, d.topk, d.init_blocks,
            d.local_blocks, d.scale)
    a = msa.sparse_attend_decode_paged(*common, to_bf16(d.k_cache), to_bf16(d.v_cache),
                                       to_bf16(d.ik_cache), *tail)
    b = msa.sparse_attend_decode_paged(*common, kc, vc, ikc, *tail)
    assert torch.equal(a, b)
