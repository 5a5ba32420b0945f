#!/usr/bin/env python3
"""Benchmark of the MiniMax-M3 block-sparse attention hot path on one MI355X.

Default workload: paged decode, batch 32, context lengths ~ U[8192, 32768],
topk 16 (one step = index scoring + selection + sparse attention + combine,
i.e. one msa_sparse_attend_decode_paged call).  A second line of numbers for
the 32768-token planted prefill (select + attend) is attached under
"prefill_32k".  Inputs are seeded synthetic tensors, resident in HBM before
timing; L2 and the 256 MB MALL are flushed before every step (outside the
timed span) by READING a 1 GiB buffer: a write-based flush would leave the
Infinity Cache full of dirty lines whose write-back the next step's reads
would pay for (measured: 2.6 vs 5.5 TB/s on a 168 MB paged read).

Each step is timed with HIP events on the stream the kernels run on.  The
decode step is timed three ways: direct launches with no instrumentation
(the headline value), direct launches with events the library records
around each of its launches (msa_set_timing_events: the per-kernel times),
and replayed from a captured HIP graph (reported beside the headline; a
graph launch costs a fixed ~7 us more than direct launches on this ROCm).

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true", help="skip the 32k prefill numbers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-flush", action="store_true", help="do not flush L2/MALL between steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference dispatch for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward leg")
    ap.add_argument("--no-fp8-decode", action="store_true",
                    help="skip the E4M3-indexer decode leg (8 requests of 131072 tokens)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timings of the decode step (reported beside "
                         "the direct-launch headline)")
    return ap.parse_args()


class Hip:
    """hipEvent_t helpers on the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e)
        return out

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ev, ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def dev(a):
    """numpy -> torch on cuda:0 (uint16 bit patterns become bf16)."""
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def keys_of(L, topk):
    """Keys attended by the query at position L-1 of a length-L sequence when
    all min(topk, nb) chosen blocks are full except the query's own."""
    nb = (L + 127) // 128
    return 128 * (min(topk, nb) - 1) + (L - 128 * (nb - 1))


def timed_steps(run, steps, warmup, hip, stream, flush, n_events):
    """Run warmup + steps; returns (per-step ms list, per-kernel ms lists)."""
    import torch
    import block_sparse_gqa_score_amd as msa
    L = msa.lib()
    ev_arrays = [(ctypes.c_void_p * n_events)(*hip.events(n_events)) for _ in range(steps)]
    starts, ends = hip.events(steps), hip.events(steps)
    for _ in range(warmup):
        if flush is not None:
            flush.sum()
        run(None)
    torch.cuda.synchronize()
    names = None
    for i in range(steps):
        if flush is not None:
            flush.sum()
        hip.record(starts[i], stream)
        run(ev_arrays[i])
        hip.record(ends[i], stream)
        if names is None:
            names = [L.msa_timing_kernel_name(j).decode() for j in range(L.msa_timing_kernel_count())]
    torch.cuda.synchronize()
    step_ms = [hip.elapsed_ms(starts[i], ends[i]) for i in range(steps)]
    return step_ms, ev_arrays, names


def kernel_times(ev_arrays, names_per_call, hip):
    """ev_arrays[i] holds, call after call, (k+1) events per call."""
    out = {}
    for arr in ev_arrays:
        off = 0
        for names in names_per_call:
            for j, nm in enumerate(names):
                out.setdefault(nm, []).append(hip.elapsed_ms(arr[off + j], arr[off + j + 1]))
            off += len(names) + 1
    return out


def stats(xs):
    import numpy as np
    a = np.asarray(xs)
    return dict(mean=float(a.mean()), median=float(np.median(a)), p10=float(np.percentile(a, 10)),
                p90=float(np.percentile(a, 90)))


def graph_replay_ms(issue, s, steps, hip, stream, flush):
    """Capture one call (issue() launches on torch's current stream and returns
    its status) into a HIP graph on side stream s; time `steps` replays on
    `stream` with HIP events."""
    import torch
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            st = issue()
            assert st == 0, st
    torch.cuda.current_stream().wait_stream(s)
    ga, gb = hip.events(steps), hip.events(steps)
    for i in range(steps):
        if flush is not None:
            flush.sum()
        hip.record(ga[i], stream)
        g.replay()
        hip.record(gb[i], stream)
    torch.cuda.synchronize()
    return stats([hip.elapsed_ms(ga[i], gb[i]) for i in range(steps)])


def plain_step_ms(issue, steps, hip, stream, flush, warmup=3):
    """Direct launches with no instrumentation: issue(stream) enqueues one
    call; HIP events bracket it on `stream` (the flush before each step gives
    the host time to enqueue, as a serving loop that runs ahead does)."""
    import torch
    for _ in range(warmup):
        if flush is not None:
            flush.sum()
        assert issue(stream) == 0
    torch.cuda.synchronize()
    ga, gb = hip.events(steps), hip.events(steps)
    for i in range(steps):
        if flush is not None:
            flush.sum()
        hip.record(ga[i], stream)
        assert issue(stream) == 0
        hip.record(gb[i], stream)
    torch.cuda.synchronize()
    return stats([hip.elapsed_ms(ga[i], gb[i]) for i in range(steps)])


def bench_decode(args, hip, flush):
    import numpy as np
    import torch
    import block_sparse_gqa_score_amd as msa
    import workloads as W
    t0 = time.time()
    d = W.config(1)
    gen_s = time.time() - t0
    dq, diq = dev(d.q), dev(d.iq)
    dk, dv, dik = dev(d.k_cache), dev(d.v_cache), dev(d.ik_cache)
    dpt, dctx = dev(d.page_table), dev(d.context_lens)
    ws = torch.empty(msa.decode_workspace_bytes(d.B, d.max_context_len, d.topk), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((d.B, 64, 128), dtype=torch.bfloat16, device="cuda")
    L = msa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def run(events):
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events)), len(events))
        st = L.msa_sparse_attend_decode_paged(
            P(dq), P(diq), P(dk), P(dv), P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B,
            d.max_context_len, d.topk, d.init_blocks, d.local_blocks, d.scale, P(out), None, P(ws),
            ws.numel(), ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(L.msa_last_error().decode())

    step_ms, evs, names = timed_steps(run, args.steps, args.warmup, hip, stream, flush, 5)
    kt = kernel_times(evs, [names], hip)
    plain = plain_step_ms(lambda strm: L.msa_sparse_attend_decode_paged(
        P(dq), P(diq), P(dk), P(dv), P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B, d.max_context_len, d.topk,
        d.init_blocks, d.local_blocks, d.scale, P(out), None, P(ws), ws.numel(), ctypes.c_void_p(strm)),
        args.steps, hip, stream, flush)
    oq = torch.empty((d.B, 64 * 128), dtype=torch.uint8, device="cuda")
    osc = torch.empty((d.B, 64 * 128 // 32), dtype=torch.uint8, device="cuda")
    mx_plain = plain_step_ms(lambda strm: L.msa_sparse_attend_decode_paged_mxfp8(
        P(dq), P(diq), P(dk), P(dv), P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B, d.max_context_len, d.topk,
        d.init_blocks, d.local_blocks, d.scale, P(oq), P(osc), None, P(ws), ws.numel(), ctypes.c_void_p(strm)),
        args.steps, hip, stream, flush)
    graph_ms = mx_graph_ms = None
    if not args.no_graph:
        s = torch.cuda.Stream()

        def gstream():
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        graph_ms = graph_replay_ms(lambda: L.msa_sparse_attend_decode_paged(
            P(dq), P(diq), P(dk), P(dv), P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B,
            d.max_context_len, d.topk, d.init_blocks, d.local_blocks, d.scale, P(out), None,
            P(ws), ws.numel(), gstream()), s, args.steps, hip, stream, flush)
        # the same step with the output emitted as MXFP8 (E4M3 + E8M0 per 32)
        mx_graph_ms = graph_replay_ms(lambda: L.msa_sparse_attend_decode_paged_mxfp8(
            P(dq), P(diq), P(dk), P(dv), P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B,
            d.max_context_len, d.topk, d.init_blocks, d.local_blocks, d.scale, P(oq), P(osc),
            None, P(ws), ws.numel(), gstream()), s, args.steps, hip, stream, flush)

    # the same step over E4M3 K/V caches with per-tensor scales (caches made
    # from the bf16 ones before timing; NaN tails stay NaN)
    ks, vs = 1.0 / 32, 1.0 / 32  # N(0,1) rows: |x|/scale stays far below 448
    fk = (dk.float() / ks).to(torch.float8_e4m3fn).view(torch.uint8)
    fv = (dv.float() / vs).to(torch.float8_e4m3fn).view(torch.uint8)
    out8 = torch.empty_like(out)

    def run8(events):
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events)), len(events))
        st = L.msa_sparse_attend_decode_paged_fp8kv(
            P(dq), P(diq), P(fk), P(fv), ks, vs, P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B,
            d.max_context_len, d.topk, d.init_blocks, d.local_blocks, d.scale, P(out8), None, P(ws),
            ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(L.msa_last_error().decode())

    fp8_step, evs8, names8 = timed_steps(run8, args.steps, args.warmup, hip, stream, flush, 5)
    fp8_kt = {k: stats(v)["mean"] for k, v in kernel_times(evs8, [names8], hip).items()}
    fp8_plain = plain_step_ms(lambda strm: L.msa_sparse_attend_decode_paged_fp8kv(
        P(dq), P(diq), P(fk), P(fv), ks, vs, P(dik), 0, P(dpt), d.max_pages, P(dctx), d.B, d.max_context_len,
        d.topk, d.init_blocks, d.local_blocks, d.scale, P(out8), None, P(ws), ws.numel(), ctypes.c_void_p(strm)),
        args.steps, hip, stream, flush)
    fp8_graph = None
    if not args.no_graph:
        fp8_graph = graph_replay_ms(lambda: run8(None) or 0, s, args.steps, hip, stream, flush)
    fp8kv = dict(step=stats(fp8_step), plain=fp8_plain, graph=fp8_graph, per_kernel_ms=fp8_kt, k_scale=ks,
                 v_scale=vs)

    # algorithmic bytes (per request: index-K rows, selected K/V rows, q/iq/out, page table)
    lens = d.context_lens.astype(np.int64)
    nb = (lens + 127) // 128
    idx_bytes = int((lens * 256).sum() + d.B * 4 * 128 * 2 + (nb * 4).sum())
    kv_bytes = int(sum(4 * 512 * keys_of(int(x), d.topk) for x in lens))
    qo_bytes = d.B * 64 * 128 * 2 * 2
    total_bytes = idx_bytes + kv_bytes + qo_bytes
    per_kernel = {k: stats(v)["mean"] for k, v in kt.items()}
    alg = {"decode_scores": idx_bytes, "decode_attend": kv_bytes + d.B * 64 * 128 * 2}
    fp8kv["attend_alg_bytes"] = kv_bytes // 2 + d.B * 64 * 128 * 2
    dom = max(alg, key=lambda k: per_kernel.get(k, 0.0))
    return dict(d=d, gen_s=gen_s, step=stats(step_ms), per_kernel_ms=per_kernel, alg_bytes=alg,
                dominant=dom, total_bytes=total_bytes, out=out, graph=graph_ms, mx_graph=mx_graph_ms,
                fp8kv=fp8kv, plain=plain, mx_plain=mx_plain)


def prefill_flops(w):
    """Algorithmic flops of one prefill pass over workload w: the causal
    index dots (4 heads x 256 flop per (query, key) pair of a document) and
    the selected-key attention (64 heads x 512 flop per attended key, with
    keys(t) = 128 (min(topk, c+1) - 1) + (p mod 128) + 1: every chosen block
    full except the query's own)."""
    import numpy as np
    lens = np.diff(w.cu_seqlens).astype(np.int64)
    score = float(sum(4 * L * (L + 1) // 2 * 256 for L in lens))
    keys = 0
    for L in lens:
        pos = np.arange(L)
        keys += int((128 * (np.minimum(w.topk, pos // 128 + 1) - 1) + pos % 128 + 1).sum())
    return score, 64.0 * 512 * keys


PREFILL_KERNELS = {"doc_setup(select)": (0, 1), "block_scores": (1, 2), "topk_prefill": (2, 3),
                   "doc_setup(attend)": (4, 5), "kv_units": (5, 6), "attend_prefill": (6, 7)}


def bench_prefill(args, hip, flush, cfg=2, steps=None):
    """One prefill pass (select + attend) of workload cfg, timed with HIP
    events around each kernel on the stream they run on."""
    import numpy as np
    import torch
    import block_sparse_gqa_score_amd as msa
    import workloads as W
    t0 = time.time()
    w = W.config(cfg)
    gen_s = time.time() - t0
    iq, ik, cu = dev(w.iq), dev(w.ik), dev(w.cu_seqlens)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    ws_s = torch.empty(msa.select_blocks_workspace_bytes(w.T, w.num_docs, w.max_seqlen),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(256, msa.prefill_workspace_bytes(w.T, w.num_docs, w.max_seqlen)),
                       dtype=torch.uint8, device="cuda")
    q2k = torch.empty((4, w.T, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((w.T, 64, 128), dtype=torch.bfloat16, device="cuda")
    L = msa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def run(events):
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events)), 4)
        st = L.msa_select_blocks(P(iq), P(ik), 0, P(cu), w.num_docs, w.T, w.max_seqlen, w.topk,
                                 w.init_blocks, w.local_blocks, P(q2k), None, P(ws_s), ws_s.numel(),
                                 ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(L.msa_last_error().decode())
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events) + 4 * 8), 4)
        st = L.msa_sparse_attend_prefill(P(q), P(k), P(v), P(q2k), w.topk, P(cu), w.num_docs, w.T,
                                         w.max_seqlen, w.scale, P(out), P(ws_a), ws_a.numel(),
                                         ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(L.msa_last_error().decode())

    step_ms, evs, _ = timed_steps(run, steps or args.prefill_steps, args.warmup, hip, stream, flush, 8)
    kt = {}
    for arr in evs:
        for nm, (a, b) in PREFILL_KERNELS.items():
            kt.setdefault(nm, []).append(hip.elapsed_ms(arr[a], arr[b]))
    score_flops, attn_flops = prefill_flops(w)
    per_kernel = {kk: stats(vv)["mean"] for kk, vv in kt.items()}
    res = dict(w=w, gen_s=gen_s, step=stats(step_ms), steps=len(step_ms), per_kernel_ms=per_kernel,
               score_flops=score_flops, attn_flops=attn_flops, q2k=q2k, out=out)
    if "planted_blocks" in w.meta:
        res["planted_gap"] = planted_gap_gpu(w, iq, ik, cu)
    return res


def planted_gap_gpu(w, iq, ik, cu):
    """Realised planted-vs-unplanted separation from the GPU's own block
    scores (one extra select call with scores_out, outside any timing): mean
    block score of planted and unplanted candidate entries, and the share of
    the chosen non-forced slots held by planted blocks."""
    import torch
    import block_sparse_gqa_score_amd as msa
    q2k, S = msa.select_blocks(iq, ik, cu, w.max_seqlen, w.topk, w.init_blocks, w.local_blocks,
                               scores=True)
    nb = S.shape[1]
    pos = torch.arange(w.T, device="cuda")  # one document
    c = pos // 128
    cand = torch.arange(nb, device="cuda")[:, None] <= c[None, :]          # [nb, T]
    planted = torch.zeros(nb, dtype=torch.bool, device="cuda")
    planted[torch.tensor(w.meta["planted_blocks"], device="cuda")] = True
    pl = cand & planted[:, None]
    un = cand & ~planted[:, None]
    s_pl = S[:, pl].double()
    s_un = S[:, un].double()
    forced = (q2k < w.init_blocks) | (q2k >= (c[None, :, None] - w.local_blocks + 1))
    free = (q2k >= 0) & ~forced
    chosen_pl = planted[q2k.clamp(min=0).long()] & free
    return {"planted_blocks": len(w.meta["planted_blocks"]),
            "planted_mean_block_score": round(float(s_pl.mean()), 3),
            "unplanted_mean_block_score": round(float(s_un.mean()), 3),
            "gap": round(float(s_pl.mean() - s_un.mean()), 3),
            "gap_in_unplanted_sd": round(float((s_pl.mean() - s_un.mean()) / s_un.std()), 3),
            "planted_share_of_free_slots": round(float(chosen_pl.sum()) / max(1, int(free.sum())), 4)}


# counter entries (profiles/hbm_traffic.json) of each prefill workload's attention kernel
COUNTER_KEYS = {"prefill_32k_planted": "attend_prefill", "packed_2x16k": "attend_prefill_packed"}


def prefill_summary(pres, name):
    """The JSON object of one prefill workload: tok/s over real tokens, the
    path's and each kernel's bf16 MFMA fraction on the algorithmic flops."""
    w = pres["w"]
    p_ms = pres["step"]["mean"]
    a_ms = pres["per_kernel_ms"]["attend_prefill"]
    s_ms = pres["per_kernel_ms"]["block_scores"]
    total_flops = pres["score_flops"] + pres["attn_flops"]
    out = {
        "workload": name, "tokens": w.T, "documents": w.num_docs, "topk": w.topk,
        "init_blocks": w.init_blocks, "local_blocks": w.local_blocks,
        "value": round(w.T / (p_ms * 1e-3), 1), "unit": "tok/s",
        "ms_per_step": round(p_ms, 6), "steps": pres["steps"],
        "per_kernel_us": {k: round(v * 1e3, 3) for k, v in pres["per_kernel_ms"].items()},
        "alg_flops": {"score": pres["score_flops"], "attention": pres["attn_flops"]},
        "path_mfma_frac": round(total_flops / (p_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "attend_prefill",
                     "achieved": round(pres["attn_flops"] / (a_ms * 1e-3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pres["attn_flops"] / (a_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(COUNTER_KEYS.get(name, "")),
                     "alg_flops_per_launch": pres["attn_flops"], "avg_launch_us": round(a_ms * 1e3, 3),
                     "mfma_busy_counter": measured_counter(COUNTER_KEYS.get(name, ""), "mfma_busy_frac")},
        "block_scores": {"achieved_tflops": round(pres["score_flops"] / (s_ms * 1e-3) / 1e12, 2),
                         "frac": round(pres["score_flops"] / (s_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "mfma_busy_counter": (measured_counter("block_scores", "mfma_busy_frac")
                                               if name == "prefill_32k_planted" else None)},
    }
    if "planted_gap" in pres:
        out["planted_gap"] = pres["planted_gap"]
    return out


def bench_select_fp8(args, hip, flush, pres):
    """The 32k planted prefill's selection with the index q/k as E4M3FN bytes
    (unscaled; the RMS-normalised values lie far inside E4M3's range): the
    block scorer's E4M3 MFMA variant, timed like the bf16 one."""
    import torch
    import block_sparse_gqa_score_amd as msa
    w = pres["w"]
    fiq = dev(w.iq).float().to(torch.float8_e4m3fn).view(torch.uint8)
    fik = dev(w.ik).float().to(torch.float8_e4m3fn).view(torch.uint8)
    cu = dev(w.cu_seqlens)
    ws_s = torch.empty(msa.select_blocks_workspace_bytes(w.T, w.num_docs, w.max_seqlen),
                       dtype=torch.uint8, device="cuda")
    q2k = torch.empty((4, w.T, w.topk), dtype=torch.int32, device="cuda")
    L = msa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def run(events):
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events)), 4)
        st = L.msa_select_blocks(P(fiq), P(fik), 1, P(cu), w.num_docs, w.T, w.max_seqlen, w.topk,
                                 w.init_blocks, w.local_blocks, P(q2k), None, P(ws_s), ws_s.numel(),
                                 ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(L.msa_last_error().decode())

    step_ms, evs, names = timed_steps(run, args.prefill_steps, args.warmup, hip, stream, flush, 4)
    kt = {k: stats(v)["mean"] for k, v in kernel_times(evs, [names], hip).items()}
    s_ms = kt["block_scores"]
    return {"index_dtype": "e4m3 (unscaled)", "select_ms": round(stats(step_ms)["mean"], 4),
            "per_kernel_us": {k: round(v * 1e3, 3) for k, v in kt.items()},
            "achieved_tflops": round(pres["score_flops"] / (s_ms * 1e-3) / 1e12, 2),
            "peak": PEAK_FP8_TFLOPS,
            "frac": round(pres["score_flops"] / (s_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "mfma_busy_counter": measured_counter("block_scores_fp8", "mfma_busy_frac")}


def bench_decode_fp8_indexer(args, hip, flush):
    """Decode with the E4M3 indexer at long context: 8 requests of 131072
    tokens (1024 pages each, physical pages a random permutation), bf16 K/V,
    topk 16.  A timing leg: the inputs are drawn on the GPU from a seeded
    torch generator with the distributions of the parity workload (K/V and
    q ~N(0,1) bf16, index q/k RMS-normalised Gaussians as E4M3FN bytes);
    parity at this size is covered by the GPU tests on the numpy inputs."""
    import torch
    import block_sparse_gqa_score_amd as msa
    B, Lc, topk = 8, 131072, 16
    npg = Lc // 128
    P_ = B * npg
    g = torch.Generator(device="cuda")
    g.manual_seed(1004)

    def rms_fp8(shape):
        z = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        z = z / torch.sqrt((z * z).mean(dim=-1, keepdim=True) + 1e-6)
        return z.to(torch.float8_e4m3fn).view(torch.uint8)

    kc = torch.randn((P_ * 128, 4, 128), generator=g, device="cuda", dtype=torch.bfloat16)
    vc = torch.randn((P_ * 128, 4, 128), generator=g, device="cuda", dtype=torch.bfloat16)
    ikc = rms_fp8((P_ * 128, 1, 128))
    q = torch.randn((B, 64, 128), generator=g, device="cuda", dtype=torch.bfloat16)
    iq = rms_fp8((B, 4, 128))
    pt = torch.randperm(P_, generator=g, device="cuda").to(torch.int32).reshape(B, npg).contiguous()
    ctx = torch.full((B,), Lc, dtype=torch.int32, device="cuda")
    out = torch.empty((B, 64, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(msa.decode_workspace_bytes(B, Lc, topk), dtype=torch.uint8, device="cuda")
    L = msa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    scale = 1.0 / 128 ** 0.5

    def call(strm):
        return L.msa_sparse_attend_decode_paged(P(q), P(iq), P(kc), P(vc), P(ikc), 1, P(pt), npg, P(ctx), B,
                                                Lc, topk, 0, 1, scale, P(out), None, P(ws), ws.numel(), strm)

    def run(events):
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events)), len(events))
        if call(ctypes.c_void_p(stream)) != 0:
            raise RuntimeError(L.msa_last_error().decode())

    step_ms, evs, names = timed_steps(run, args.steps, args.warmup, hip, stream, flush, 4)
    kt = {k: stats(v)["mean"] for k, v in kernel_times(evs, [names], hip).items()}
    plain = plain_step_ms(lambda strm: call(ctypes.c_void_p(strm)), args.steps, hip, stream, flush)
    graph = None
    if not args.no_graph:
        graph = graph_replay_ms(lambda: call(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)),
                                torch.cuda.Stream(), args.steps, hip, stream, flush)
    idx_bytes = B * Lc * 128 + B * 4 * 128 + B * npg * 4
    kv_bytes = B * 4 * 512 * keys_of(Lc, topk)
    s_ms = kt["decode_scores"]
    a_ms = kt["decode_attend"]
    return {"workload": "decode_fp8idx_b8_ctx128k", "batch": B, "context": Lc, "topk": topk,
            "index_dtype": "e4m3 (unscaled)", "step_us": round(plain["median"] * 1e3, 3),
            "launch": "direct",
            "graph_replay_step_us": round(graph["median"] * 1e3, 3) if graph is not None else None,
            "instrumented_direct_step_us": round(stats(step_ms)["median"] * 1e3, 3),
            "per_kernel_us": {k: round(v * 1e3, 3) for k, v in kt.items()},
            "path_bytes_per_step": idx_bytes + kv_bytes + 2 * B * 64 * 128 * 2,
            "scores_roofline": {"bound": "hbm", "achieved": round(idx_bytes / (s_ms * 1e-3) / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(idx_bytes / (s_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "alg_bytes_per_launch": idx_bytes,
                                "traffic": measured_traffic("decode_scores_fp8"),
                                "avg_launch_us": round(s_ms * 1e3, 3)},
            "attend_roofline": {"bound": "hbm", "achieved": round(kv_bytes / (a_ms * 1e-3) / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(kv_bytes / (a_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "alg_bytes_per_launch": kv_bytes, "avg_launch_us": round(a_ms * 1e3, 3)},
            "data": "seeded torch generator on the GPU (timing leg)",
            "_host_workload": lambda: host_decode(q, iq, kc, vc, ikc, pt, ctx, topk, "fp8")}


def host_decode(q, iq, kc, vc, ikc, pt, ctx, topk, index_dtype):
    """Host (numpy) copy of a decode batch drawn on the GPU, as a
    workloads.Decode for the oracle's CPU baseline."""
    import torch
    import workloads as W

    def h(t):
        return t.cpu().view(torch.int16).numpy().view("uint16") if t.dtype == torch.bfloat16 \
            else t.cpu().numpy()

    return W.Decode(name="decode_fp8idx_b8_ctx128k", q=h(q), iq=h(iq), k_cache=h(kc), v_cache=h(vc),
                    ik_cache=h(ikc), page_table=h(pt), context_lens=h(ctx), index_dtype=index_dtype,
                    topk=topk, init_blocks=0, local_blocks=1)


def bench_backward(args, hip, flush, pres):
    """Training leg on the 32k planted prefill: the forward with log-sum-exp,
    then the backward (dq, dk, dv) for the selection the GPU made."""
    import torch
    import block_sparse_gqa_score_amd as msa
    import workloads as W
    w, q2k = pres["w"], pres["q2k"]
    q, k, v, cu = dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens)
    dout = dev(W.grad_out(2, w.T))
    out = torch.empty((w.T, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.T, 64), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(out)
    dk = torch.empty((w.T, 4, 128), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    ws_a = torch.empty(max(256, msa.prefill_workspace_bytes(w.T, w.num_docs, w.max_seqlen)),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(msa.prefill_backward_workspace_bytes(w.T, w.num_docs, w.max_seqlen, w.topk),
                       dtype=torch.uint8, device="cuda")
    L = msa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.msa_sparse_attend_prefill_lse(P(q), P(k), P(v), P(q2k), w.topk, P(cu), w.num_docs, w.T,
                                         w.max_seqlen, w.scale, P(out), P(lse), P(ws_a), ws_a.numel(),
                                         ctypes.c_void_p(stream))
    if st != 0:
        raise RuntimeError(L.msa_last_error().decode())

    def run(events):
        if events is not None:
            L.msa_set_timing_events(ctypes.c_void_p(ctypes.addressof(events)), 7)
        st = L.msa_sparse_attend_prefill_backward(
            P(q), P(k), P(v), P(out), P(lse), P(dout), P(q2k), w.topk, P(cu), w.num_docs, w.T,
            w.max_seqlen, w.scale, P(dq), P(dk), P(dv), P(ws_b), ws_b.numel(), ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(L.msa_last_error().decode())

    step_ms, evs, names = timed_steps(run, args.prefill_steps, args.warmup, hip, stream, flush, 7)
    kt = kernel_times(evs, [names], hip)
    per_kernel = {kk: stats(vv)["mean"] for kk, vv in kt.items()}
    return dict(step=stats(step_ms), per_kernel_ms=per_kernel)


def cpu_baseline_decode(d, seconds, reps_max=20):
    import numpy as np
    import oracle
    t0 = time.time()
    reps = 0
    while True:
        oracle.decode(d)
        reps += 1
        if time.time() - t0 >= seconds or reps >= reps_max:
            break
    el = time.time() - t0
    return dict(value=el / reps * 1e6, unit="us/step", cores=oracle.num_threads(), kind="oracle",
                sample=f"{reps} full decode step(s) of the same batch (all {d.B} requests)")


def cpu_baseline_prefill(w, seconds, what):
    """The oracle on a bounded sample of the workload's tokens: uniform
    draws of 16 tokens at a time until ``seconds`` of CPU work (or every
    token) is done; tok/s over the tokens done."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)
    n = 16
    t0 = time.time()
    done = 0
    while time.time() - t0 < seconds and done < min(4096, w.T):
        toks = np.sort(rng.choice(w.T, size=min(n, w.T), replace=False)).astype(np.int32)
        oracle.prefill(w, tokens=toks)
        done += len(toks)
    el = time.time() - t0
    return dict(value=done / el, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{done} tokens drawn uniformly from the {w.T} tokens of {what}")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "block_sparse_gqa_score_amd", "csrc")


def source_digest(filename):
    import hashlib
    with open(os.path.join(CSRC, filename), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when absent or when the kernel's source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        e = t["kernels"][kernel]
        if source_digest(e["source"]) != e["source_sha"]:
            return None
        return int(round(e["fetch_kib"] * t["fetch_scale"] * 1024 + e["write_kib"] * t["write_scale"] * 1024))
    except (OSError, KeyError, ValueError):
        return None


def measured_counter(kernel, field):
    """A per-dispatch counter figure of `kernel` (e.g. mfma_busy_frac) from the
    committed counter summary, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            e = json.load(f)["kernels"][kernel]
        if source_digest(e["source"]) != e["source_sha"]:
            return None
        return e[field]
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy():
    import torch
    n = 1 << 30
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "dispatches": 3}))


def fp8kv_summary(dres):
    f = dres["fp8kv"]
    a_ms = f["per_kernel_ms"]["decode_attend"]
    bw = f["attend_alg_bytes"] / (a_ms * 1e-3) / 1e9
    return {"step_us": round(f["plain"]["median"] * 1e3, 3),
            "launch": "direct",
            "graph_replay_step_us": round(f["graph"]["median"] * 1e3, 3) if f["graph"] is not None else None,
            "per_kernel_us": {k: round(v * 1e3, 3) for k, v in f["per_kernel_ms"].items()},
            "k_scale": f["k_scale"], "v_scale": f["v_scale"],
            "attend_roofline": {"bound": "hbm", "achieved": round(bw, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(bw / PEAK_HBM_GBS, 4),
                                "alg_bytes_per_launch": f["attend_alg_bytes"],
                                "traffic": measured_traffic("decode_attend_fp8kv"),
                                "avg_launch_us": round(a_ms * 1e3, 3)}}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path: run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    hip = Hip()
    flush = None
    if not args.no_flush:
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB, read to flush

    dres = bench_decode(args, hip, flush)
    d = dres["d"]
    # headline: the step from direct launches with no instrumentation.  A
    # HIP graph replay of the same step is reported beside it: on this ROCm a
    # graph launch adds a fixed ~7 us (a one-kernel graph replays in ~13.7 us
    # event to event against ~6.3 us launched directly), while the step's
    # three direct launches enqueue in less host time than the step's GPU time.
    step_ms = dres["plain"]["mean"]
    dom = dres["dominant"]
    dom_ms = dres["per_kernel_ms"][dom]
    achieved = dres["alg_bytes"][dom] / (dom_ms * 1e-3) / 1e9
    line = {
        "metric": "sparse-attn prefill tok/s & decode µs/step at 1 GPU; % MFMA / HBM roofline",
        "value": round(step_ms * 1e3, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; pages shaped like the described decode workload)",
        "config": {"workload": "decode_b32_ctx8k-32k", "batch": d.B, "topk": d.topk,
                   "init_blocks": d.init_blocks, "local_blocks": d.local_blocks,
                   "context_lens": "U[8192,32768] seed 1001",
                   "mean_context": float(d.context_lens.mean()), "index_dtype": "bf16",
                   "heads": "64q/4kv/4idx x 128", "l2_mall_flushed": flush is not None},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(dom), "alg_bytes_per_launch": dres["alg_bytes"][dom],
                     "avg_launch_us": round(dom_ms * 1e3, 3)},
        "launch": "direct",
        "step_stats_ms": {k: round(v, 6) for k, v in dres["plain"].items()},
        "graph_replay_step_ms": ({k: round(v, 6) for k, v in dres["graph"].items()}
                                 if dres["graph"] is not None else None),
        "instrumented_direct_step_ms": {k: round(v, 6) for k, v in dres["step"].items()},
        "mxfp8_output_step_us": round(dres["mx_plain"]["median"] * 1e3, 3),
        "mxfp8_output_graph_replay_step_us": (round(dres["mx_graph"]["median"] * 1e3, 3)
                                              if dres["mx_graph"] is not None else None),
        "fp8_kv_cache": fp8kv_summary(dres),
        "per_kernel_us": {k: round(v * 1e3, 3) for k, v in dres["per_kernel_ms"].items()},
        "path_bytes_per_step": dres["total_bytes"],
        "path_hbm_frac": round(dres["total_bytes"] / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
    }
    if not args.no_prefill:
        pres = bench_prefill(args, hip, flush, cfg=2)
        line["prefill_32k"] = prefill_summary(pres, "prefill_32k_planted")
        line["prefill_32k"]["block_scores_fp8"] = bench_select_fp8(args, hip, flush, pres)
        if not args.no_backward:
            bres = bench_backward(args, hip, flush, pres)
            b_ms = bres["step"]["mean"]
            pk = bres["per_kernel_ms"]
            # algorithmic: S recomputed, dP, dV, dK, dQ = 2.5x the forward's attention flops;
            # the dQ kernel executes S, dP, dQ (1.5x), the dK/dV kernel S, dP, dV, dK (2x)
            alg = 2.5 * pres["attn_flops"]
            line["backward_32k"] = {
                "workload": "prefill_32k_planted", "what": "dq, dk, dv for the GPU's selection",
                "ms_per_step": round(b_ms, 6), "steps": args.prefill_steps,
                "per_kernel_us": {kk: round(vv * 1e3, 3) for kk, vv in pk.items()},
                "roofline": {"bound": "mfma", "achieved": round(alg / (b_ms * 1e-3) / 1e12, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(alg / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "alg_flops_per_step": alg},
                "bwd_dq_tflops": round(1.5 * pres["attn_flops"] / (pk["bwd_dq"] * 1e-3) / 1e12, 2),
                "bwd_dkdv_tflops": round(2.0 * pres["attn_flops"] / (pk["bwd_dkdv"] * 1e-3) / 1e12, 2),
                "train_attention_ms": round(b_ms + pres["per_kernel_ms"]["attend_prefill"], 3),
            }
    small = {}
    if not args.no_prefill:
        # the 2048-token prefill (topk 4) and the packed 2 x 16384 microbatch
        # (documents log-uniform in [256, 8192], init 1, local 1)
        for cfg, name in ((0, "prefill_2k"), (3, "packed_2x16k")):
            small[name] = bench_prefill(args, hip, flush, cfg=cfg, steps=max(args.prefill_steps, 20))
            line[name] = prefill_summary(small[name], small[name]["w"].name)
    fp8 = None
    if not args.no_fp8_decode:
        fp8 = bench_decode_fp8_indexer(args, hip, flush)
        line["decode_fp8_indexer"] = {k: v for k, v in fp8.items() if not k.startswith("_")}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(d, args.cpu_seconds)
        if not args.no_prefill:
            line["prefill_32k"]["cpu_baseline"] = cpu_baseline_prefill(
                pres["w"], args.cpu_seconds, "the 32768-token document")
            for name, res in small.items():
                line[name]["cpu_baseline"] = cpu_baseline_prefill(
                    res["w"], args.cpu_seconds, f"{res['w'].num_docs} document(s)")
        if fp8 is not None:
            line["decode_fp8_indexer"]["cpu_baseline"] = cpu_baseline_decode(
                fp8["_host_workload"](), args.cpu_seconds, reps_max=3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
