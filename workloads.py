"""Seeded synthetic inputs for the MiniMax-M3 block-sparse attention path.

This module only *draws* inputs: Gaussian tensors, RMS-normalised index
vectors, document maps, context lengths and page tables, and encodes them
to the storage formats the path consumes (bf16 bits, OCP E4M3FN bytes).
It holds none of the method's arithmetic (no scores, no selection, no
softmax) and is imported by both the CPU oracle's tests and the GPU tests
and benchmark, so that both sides read identical bytes.

Shapes follow the tensor contracts of the NeMo AutoModel MSA page
(MSAMicrobatch.select_blocks, sparse_attention): q [T,64,128],
k/v [T,4,128], index q [T,4,128], index k [T,1,128]; and of the
TensorRT-LLM MiniMaxM3SparseAttentionConfig page for the paged side
index-K cache [num_slots,1,128] that sits beside the main K/V cache.

Every random tensor is produced chunk by chunk from
``SeedSequence(seed).spawn`` children with a fixed chunk size, so the
bytes depend only on (seed, shape) and never on the thread count.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

NUM_HEADS = 64
NUM_KV_HEADS = 4
NUM_INDEX_HEADS = 4
HEAD_DIM = 128
BLOCK = 128

_CHUNK = 1 << 22  # values per independent RNG stream


# --------------------------------------------------------------------------
# storage-format encoders (input preparation, written from the formats)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    bf16 is the upper half of an IEEE binary32; rounding adds 0x7FFF plus
    the lowest kept bit before truncation.  NaN inputs map to 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
           >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def _e4m3_positive_table() -> np.ndarray:
    """Values of the 127 finite non-negative OCP E4M3FN codes 0x00..0x7E."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            vals[code] = (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_TABLE = _e4m3_positive_table()


def e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3FN bytes: round to nearest (ties to even code),
    saturating to +-448 (E4M3FN has no infinities)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_TABLE, a, side="left")      # first >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_TABLE[lo]
    dhi = _E4M3_TABLE[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_TABLE[hi], hi, code).astype(np.uint8)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------
def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


def normal_f32(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    """Standard normal float32 of ``shape`` from fixed-size independent chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seed_seq.spawn(nchunks)

    def fill(i):
        g = np.random.default_rng(kids[i])
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def normal_bf16(seed_seq, shape) -> np.ndarray:
    return bf16_bits(normal_f32(seed_seq, shape))


def grad_out(seed: int, T: int) -> np.ndarray:
    """Incoming gradient of the attention output: bf16 bits [T,64,128],
    standard normal (a stand-in for d(loss)/d(out) of a training step)."""
    return normal_bf16(np.random.SeedSequence([seed, 0x6472]), (T, 64, 128))


def synthetic_q2k(seed: int, cu_seqlens, topk: int, init_blocks: int = 0, local_blocks: int = 1,
                  hot_frac: float = 0.05) -> np.ndarray:
    """A seeded stand-in selection, token-major int32 [T,4,topk], shaped like
    the planted long-prefill workload's: every row holds its forced blocks,
    then the document's "hot" blocks (a fixed random hot_frac of its blocks)
    that precede the query block, then distinct random earlier blocks, in
    ascending order with -1 padding.  No scores are computed: it is an input
    for the attention step only."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    g = np.random.default_rng(np.random.SeedSequence([seed, 0x71]))
    rows = np.full((T, 4, topk), -1, dtype=np.int32)
    for d in range(len(cu) - 1):
        L = int(cu[d + 1] - cu[d])
        nb = (L + 127) // 128
        hot = [np.sort(g.choice(nb, size=max(1, int(round(hot_frac * nb))), replace=False))
               for _ in range(4)]
        for p in range(L):
            c = p // 128
            for h in range(4):
                forced = {b for b in range(c + 1) if b < init_blocks or b >= c - local_blocks + 1}
                pick = list(forced)
                for b in hot[h]:
                    if len(pick) >= topk or b > c:
                        break
                    if b not in forced:
                        pick.append(int(b))
                if len(pick) < topk:
                    rest = np.setdiff1d(np.arange(c + 1), pick)
                    pick += g.permutation(rest)[:topk - len(pick)].tolist()
                pick = sorted(pick)[:topk]
                rows[cu[d] + p, h, :len(pick)] = pick
    return rows


def rms_normalise(z: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """z / sqrt(mean(z^2) + eps) along the last axis (index vectors arrive
    post-norm; this stands in for the model's norm)."""
    z = z.astype(np.float32)
    r = np.sqrt(np.mean(z.astype(np.float64) ** 2, axis=-1, keepdims=True) + eps)
    return (z / r).astype(np.float32)


def encode_index(x: np.ndarray, index_dtype: str) -> np.ndarray:
    if index_dtype == "bf16":
        return bf16_bits(x)
    if index_dtype == "fp8":
        return e4m3_bytes(x)
    raise ValueError(index_dtype)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass
class Prefill:
    """Compact packed-token prefill batch (one or more documents)."""
    name: str
    cu_seqlens: np.ndarray           # int32 [D+1]
    q: np.ndarray                    # uint16 [T,64,128]
    k: np.ndarray                    # uint16 [T,4,128]
    v: np.ndarray                    # uint16 [T,4,128]
    iq: np.ndarray                   # uint16 or uint8 [T,4,128]
    ik: np.ndarray                   # uint16 or uint8 [T,1,128]
    index_dtype: str = "bf16"
    topk: int = 16
    init_blocks: int = 0
    local_blocks: int = 1
    scale: float = 1.0 / math.sqrt(128.0)
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_docs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def max_seqlen(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens)))


@dataclass
class Decode:
    """One decode step over a paged K/V cache plus a side index-K cache."""
    name: str
    q: np.ndarray                    # uint16 [B,64,128]
    iq: np.ndarray                   # uint16|uint8 [B,4,128]
    k_cache: np.ndarray              # uint16 [P*128,4,128]
    v_cache: np.ndarray              # uint16 [P*128,4,128]
    ik_cache: np.ndarray             # uint16|uint8 [P*128,1,128]
    page_table: np.ndarray           # int32 [B,max_pages]
    context_lens: np.ndarray         # int32 [B]
    index_dtype: str = "bf16"
    topk: int = 16
    init_blocks: int = 0
    local_blocks: int = 1
    scale: float = 1.0 / math.sqrt(128.0)
    meta: dict = field(default_factory=dict)
    kv_dtype: str = "bf16"           # "fp8": k/v caches hold E4M3FN bytes of x / k_scale, x / v_scale
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def make_prefill(doc_lens, seed: int, *, topk=16, init_blocks=0, local_blocks=1,
                 index_dtype="bf16", planted_frac: float | None = None,
                 index_fn=None, name="prefill") -> Prefill:
    """Compact prefill batch with documents of the given lengths.

    q/k/v ~ N(0,1) in bf16.  Index q/k are RMS-normalised Gaussians.  With
    ``planted_frac`` (single-document use), a fraction of key blocks is
    planted: a unit vector u is drawn, every index query becomes z + mu*u and
    every index key in a planted block z + mu*u (others z), before the RMS
    norm, with mu^2 = 2 + 2*sqrt(1 + d).  ``index_fn(T)`` may instead return
    float32 (iq [T,4,128], ik [T,1,128]) for hand-built cases.
    """
    doc_lens = [int(x) for x in doc_lens]
    if not doc_lens or min(doc_lens) < 1:
        raise ValueError("documents must be non-empty")
    cu = np.zeros(len(doc_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(doc_lens)
    T = int(cu[-1])
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_v, s_iq, s_ik, s_plant = ss.spawn(6)
    q = normal_bf16(s_q, (T, NUM_HEADS, HEAD_DIM))
    k = normal_bf16(s_k, (T, NUM_KV_HEADS, HEAD_DIM))
    v = normal_bf16(s_v, (T, NUM_KV_HEADS, HEAD_DIM))
    meta = {}
    if index_fn is not None:
        iqf, ikf = index_fn(T)
    else:
        iqz = normal_f32(s_iq, (T, NUM_INDEX_HEADS, HEAD_DIM))
        ikz = normal_f32(s_ik, (T, 1, HEAD_DIM))
        if planted_frac:
            g = np.random.default_rng(s_plant)
            nb = (T + BLOCK - 1) // BLOCK
            n_plant = int(round(planted_frac * nb))
            planted = np.sort(g.choice(nb, size=n_plant, replace=False))
            u = g.standard_normal(HEAD_DIM)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            mu = math.sqrt(2.0 + 2.0 * math.sqrt(1.0 + HEAD_DIM))
            iqz = iqz + mu * u
            blk = np.arange(T) // BLOCK
            mask = np.isin(blk, planted)
            ikz[mask, 0, :] += mu * u
            meta.update(planted_blocks=planted.tolist(), mu=mu)
        iqf, ikf = rms_normalise(iqz), rms_normalise(ikz)
    iq = encode_index(iqf, index_dtype)
    ik = encode_index(ikf, index_dtype)
    return Prefill(name=name, cu_seqlens=cu, q=q, k=k, v=v, iq=iq, ik=ik,
                   index_dtype=index_dtype, topk=topk, init_blocks=init_blocks,
                   local_blocks=local_blocks, meta=meta)


def with_e4m3_index(w: Prefill) -> Prefill:
    """The same prefill batch with its bf16 index q/k re-encoded as E4M3FN
    bytes (nearest value, ties to the even code): the fp8 indexer's unscaled
    E4M3 storage of the same index vectors.  The main q/k/v are shared."""
    if w.index_dtype != "bf16":
        raise ValueError("expects bf16 index vectors")

    def dec(bits):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)

    return Prefill(name=w.name + "_e4m3_index", cu_seqlens=w.cu_seqlens, q=w.q, k=w.k, v=w.v,
                   iq=e4m3_bytes(dec(w.iq)), ik=e4m3_bytes(dec(w.ik)), index_dtype="fp8",
                   topk=w.topk, init_blocks=w.init_blocks, local_blocks=w.local_blocks,
                   scale=w.scale, meta=dict(w.meta))


def packed_doc_lengths(seed: int, rows: int = 2, seq: int = 16384,
                       lo: int = 256, hi: int = 8192):
    """Document lengths of a packed BSHD microbatch.

    Per row, lengths round(exp(U(ln lo, ln hi))) are drawn and placed
    contiguously while they fit; the first that does not fit ends the row
    and the rest of the row is padding (document id 0).  Returns the
    per-row length lists and the [rows, seq] int64 document map (ids 1.. per
    row, 0 = padding)."""
    g = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    per_row = []
    doc_map = np.zeros((rows, seq), dtype=np.int64)
    for r in range(rows):
        pos, lens = 0, []
        while True:
            L = int(round(math.exp(g.uniform(math.log(lo), math.log(hi)))))
            if pos + L > seq:
                break
            lens.append(L)
            doc_map[r, pos:pos + L] = len(lens)
            pos += L
        per_row.append(lens)
    return per_row, doc_map


def make_decode(context_lens, seed: int, *, topk=16, init_blocks=0, local_blocks=1,
                index_dtype="bf16", name="decode", identity_pages=False,
                poison_tail=True, kv_dtype="bf16", k_scale=0.5, v_scale=0.25) -> Decode:
    """Paged decode step: pages of 128 slots, physical page ids a random
    permutation of all pages (identity when ``identity_pages``).  Slots past
    each request's context length are filled with NaN when ``poison_tail``.
    With ``kv_dtype="fp8"`` the main K/V caches hold E4M3FN bytes of the same
    N(0,1) values divided by ``k_scale`` / ``v_scale`` (per-tensor scales)."""
    L = np.asarray(context_lens, dtype=np.int32)
    if L.min() < 1:
        raise ValueError("context lengths must be >= 1")
    B = len(L)
    nb = (L + BLOCK - 1) // BLOCK
    P = int(nb.sum())
    ss = np.random.SeedSequence(seed)
    s_q, s_iq, s_k, s_v, s_ik, s_perm = ss.spawn(6)
    q = normal_bf16(s_q, (B, NUM_HEADS, HEAD_DIM))
    iq = encode_index(rms_normalise(normal_f32(s_iq, (B, NUM_INDEX_HEADS, HEAD_DIM))),
                      index_dtype)
    if kv_dtype == "fp8":
        k_cache = e4m3_bytes(normal_f32(s_k, (P * BLOCK, NUM_KV_HEADS, HEAD_DIM)) / np.float32(k_scale))
        v_cache = e4m3_bytes(normal_f32(s_v, (P * BLOCK, NUM_KV_HEADS, HEAD_DIM)) / np.float32(v_scale))
    elif kv_dtype == "bf16":
        k_cache = normal_bf16(s_k, (P * BLOCK, NUM_KV_HEADS, HEAD_DIM))
        v_cache = normal_bf16(s_v, (P * BLOCK, NUM_KV_HEADS, HEAD_DIM))
    else:
        raise ValueError(kv_dtype)
    ik_cache = encode_index(rms_normalise(normal_f32(s_ik, (P * BLOCK, 1, HEAD_DIM))),
                            index_dtype)
    if identity_pages:
        perm = np.arange(P, dtype=np.int32)
    else:
        perm = np.random.default_rng(s_perm).permutation(P).astype(np.int32)
    max_pages = int(nb.max())
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for r in range(B):
        page_table[r, :nb[r]] = perm[off:off + nb[r]]
        off += nb[r]
    if poison_tail:
        nan_bits = 0x7FC0
        fp8_nan = 0x7F
        for r in range(B):
            tail = int(nb[r] * BLOCK - L[r])
            if tail == 0:
                continue
            page = int(page_table[r, nb[r] - 1])
            s0 = page * BLOCK + (BLOCK - tail)
            s1 = (page + 1) * BLOCK
            k_cache[s0:s1] = fp8_nan if kv_dtype == "fp8" else nan_bits
            v_cache[s0:s1] = fp8_nan if kv_dtype == "fp8" else nan_bits
            ik_cache[s0:s1] = fp8_nan if index_dtype == "fp8" else nan_bits
    return Decode(name=name, q=q, iq=iq, k_cache=k_cache, v_cache=v_cache,
                  ik_cache=ik_cache, page_table=page_table, context_lens=L,
                  index_dtype=index_dtype, topk=topk, init_blocks=init_blocks,
                  local_blocks=local_blocks, kv_dtype=kv_dtype,
                  k_scale=float(k_scale) if kv_dtype == "fp8" else 1.0,
                  v_scale=float(v_scale) if kv_dtype == "fp8" else 1.0)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
def mx_matrix(seed: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bit patterns [rows, cols] (cols % 32 == 0) for the MXFP8 quantiser
    tests, built at the bit level in blocks of 32 of mixed kinds: random
    values over a wide exponent range; all zeros (either sign); values with at
    most 3 mantissa bits (on the E4M3 grid after a power-of-two scale); values
    with mantissa pattern 1xxx1000 (half-way points of that grid); a block whose
    largest value has a mantissa of 1.75 or more (the saturation range); bf16
    subnormals; and blocks spanning ~40 binades."""
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    g = np.random.default_rng(np.random.SeedSequence(seed).spawn(9)[8])
    nb = cols // 32
    kind = g.integers(0, 7, size=(rows, nb, 1))
    sign = g.integers(0, 2, size=(rows, nb, 32)).astype(np.uint32) << 15
    base = g.integers(20, 240, size=(rows, nb, 1))  # block's top biased exponent
    span = np.where(kind == 6, 40, 12)
    expo = np.clip(base - g.integers(0, 41, size=(rows, nb, 32)) % (span + 1), 1, 254)
    man = g.integers(0, 128, size=(rows, nb, 32))
    man = np.where(kind == 2, man & 0x70, man)
    man = np.where(kind == 3, (man & 0x70) | 0x08, man)
    # saturation kind: element 0 carries the block's top exponent and a mantissa >= 0x60
    first = np.zeros((1, 1, 32), dtype=bool)
    first[..., 0] = True
    expo = np.where((kind == 4) & first, base, expo)
    man = np.where((kind == 4) & first, 0x60 | (man & 0x1F), man)
    bits = sign | (expo.astype(np.uint32) << 7) | man.astype(np.uint32)
    bits = np.where(kind == 1, sign, bits)
    bits = np.where(kind == 5, sign | man.astype(np.uint32), bits)  # exponent field 0
    return bits.reshape(rows, cols).astype(np.uint16)


CONFIG_NAMES = (
    "prefill_2k_topk4",              # one causal document of 2048 tokens, topk=4
    "decode_b32_ctx8k-32k",          # paged decode, batch 32, L ~ U[8192, 32768]
    "prefill_32k_planted",           # one document of 32768 tokens, planted blocks
    "packed_2x16k",                  # packed documents, 2 rows x 16384, init=1 local=1
    "decode_fp8idx_b8_ctx128k",      # fp8 E4M3 indexer decode, batch 8, L=131072
)


def config(i: int):
    """Build workload ``i`` (seed 1000 + i)."""
    seed = 1000 + i
    if i == 0:
        return make_prefill([2048], seed, topk=4, init_blocks=0, local_blocks=1,
                            name=CONFIG_NAMES[0])
    if i == 1:
        g = np.random.default_rng(np.random.SeedSequence(seed).spawn(8)[7])
        lens = g.integers(8192, 32768, size=32, endpoint=True)
        return make_decode(lens, seed, topk=16, init_blocks=0, local_blocks=1,
                           name=CONFIG_NAMES[1])
    if i == 2:
        return make_prefill([32768], seed, topk=16, init_blocks=0, local_blocks=1,
                            planted_frac=0.05, name=CONFIG_NAMES[2])
    if i == 3:
        per_row, doc_map = packed_doc_lengths(seed)
        lens = [L for row in per_row for L in row]
        p = make_prefill(lens, seed, topk=16, init_blocks=1, local_blocks=1,
                         name=CONFIG_NAMES[3])
        p.meta.update(rows=per_row, bshd_shape=(2, 16384), doc_map=doc_map)
        return p
    if i == 4:
        return make_decode([131072] * 8, seed, topk=16, init_blocks=0, local_blocks=1,
                           index_dtype="fp8", name=CONFIG_NAMES[4])
    raise ValueError(i)


def pack(external: np.ndarray, doc_map: np.ndarray) -> np.ndarray:
    """Gather BSHD ``external[batch, seq, ...]`` to ``[tokens, ...]`` in
    document order (row by row, documents in increasing id), the packed
    layout of the NeMo MSA page (MSAMicrobatch.pack)."""
    rows = []
    for r in range(doc_map.shape[0]):
        ids = doc_map[r]
        for d in range(1, int(ids.max()) + 1 if ids.max() > 0 else 1):
            idx = np.nonzero(ids == d)[0]
            rows.append(external[r, idx])
    return np.concatenate(rows, axis=0)
