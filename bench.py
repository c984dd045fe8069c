"""Benchmark of the sparse-attention hot path on one MI355X.

Default workload (the headline metric): Llama-3-8B-shaped decode layer,
batch 32, 32 query / 8 KV heads, d 128, bf16, 32768 tokens per sequence in
pages of 64 in a shuffled shared pool, sink 1 page + window 8 pages + top-41
pages per KV head (3200 of 32768 tokens, ~90% sparsity).

One step = one decode layer's sparse-attention work for one batch.  For the
default workload it is one sa_select_decode call: the newest page's mean key
is recomputed, every page is scored against the pooled query, the sink /
window / top-k lists are selected and the selected pages are attended, in one
kernel (--two-calls runs it as sa_select_pages + sa_sparse_decode, which the
other decode workloads always do; the FP8 variant selects from the page
summaries without the newest-page refresh).  The timed loop replays one HIP
graph that holds one step per input set, run back to back as consecutive
layers' attention runs inside a captured decode forward pass; every kernel
runs in every step, and exactly --steps steps are timed (whole graphs, then
single-step graphs for the remainder).  The same steps are also replayed one
graph per step (ms_per_step_single_step_graphs) and, one by one between HIP
event pairs, give the per-step median and 10th / 90th percentiles
(step_us_p10_p50_p90).  Inputs are resident in HBM before timing; steps rotate
over 3 independently drawn input sets (4.2 GB each) so no step finds its pages
in the 256 MB last-level cache left warm by the previous one.

Prints one JSON line: value = selected K+V bytes per step / step time (GB/s);
roofline of the dominant kernel from HIP events on the launch stream;
cpu_baseline = the CPU oracle on a bounded sample of the same workload (8 of
the 32 sequences, the full step as the GPU runs it: the newest page's mean
refreshed, the other page means built once beforehand), in the same unit.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

import workloads as W

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_decode_32k",
                    choices=["llama3_8b_decode_32k", "token_head_decode_128k", "mla_tiered_decode_64k",
                             "chunked_prefill_128k", "tiny_decode", "llama3_8b_decode_32k_fp8", "hbm_copy"])
    ap.add_argument("--sets", type=int, default=3, help="independent input sets rotated over")
    ap.add_argument("--splits", type=int, default=-1, help="decode splits (-1: workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-calls", action="store_true",
                    help="run the decode step as sa_select_pages + sa_sparse_decode even where one "
                         "sa_select_decode call can")
    return ap.parse_args()


class Timer:
    """Per-call HIP event pairs on the current (launch) stream."""

    def __init__(self):
        self.pairs = {}

    def start(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append([e, None])

    def stop(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[name][-1][1] = e

    def avg_us(self, name):
        ps = self.pairs.get(name, [])
        return 1000.0 * sum(a.elapsed_time(b) for a, b in ps) / max(1, len(ps))

    def reset(self):
        self.pairs = {}


def fused_path(wl, splits):
    """True when one sa_select_decode call can run the step: per-KV-head lists
    scored from page summaries, untiered, a bf16 cache of d 128 in pages of 64,
    one split (the library's own choice when every CU holds one list, as for
    the Llama-3-8B batch of 32 x 8 lists)."""
    return (wl.mode == "per_kv_head" and wl.scores == "summary" and not wl.tiered and not wl.latent
            and wl.d_qk == 128 and wl.d_v == 128 and wl.page_size == 64 and wl.dtype == "bf16" and splits in (0, 1))


def decode_step_fn(S, wl, inp, mu, splits, fused=False):
    """One decode step as one HIP graph on the current stream: page summary of
    the newest page and selection (one call), split-K decode and LSE merge.  Graph replay
    removes the host launch cost between kernels; every kernel still runs in
    every replay.  With `fused` the step is one sa_select_decode call (same
    lists and outputs, bit for bit, as the two calls).  (Running the newest-page summary update on a second stream
    beside the selection, which the library allows when a local window forces
    that page, measured slower here: the fork and join cost more than the
    overlap saves.)  A captured graph does not own the memory its kernels use,
    so the last value returned holds every buffer the graph touches; keep it
    as long as the graph."""
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"], d_v=wl.d_v,
                   k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))
    mode = S.SA_SEL_PER_KV_HEAD if wl.mode == "per_kv_head" else S.SA_SEL_PER_Q_HEAD
    refresh = mu is not None and wl.dtype != "fp8"   # FP8 pages: summaries kept by sa_page_summary
    stride = max(1, min(wl.max_pages, wl.sink_pages + wl.window_pages + wl.top_k))
    dev = inp["q"].device
    n_sel = wl.n_sel
    lists = torch.full((wl.batch, n_sel, stride), -1, dtype=torch.int32, device=dev)
    counts = torch.zeros((wl.batch, n_sel), dtype=torch.int32, device=dev)
    ccounts = torch.zeros_like(counts) if wl.tiered else None
    sel_ws = torch.empty(max(1, S.sa_select_pages_workspace_size(wl.batch, n_sel, wl.max_pages)),
                         dtype=torch.uint8, device=dev)
    dec_ws = torch.zeros(max(1, S.sa_sparse_decode_workspace_size(kv, wl.q_tokens, wl.n_q_heads, stride, mode,
                                                                   splits)), dtype=torch.uint8, device=dev)
    out = torch.empty((wl.batch, wl.q_tokens, wl.n_q_heads, wl.d_v), dtype=inp["q"].dtype, device=dev)
    lse = torch.empty((wl.batch, wl.q_tokens, wl.n_q_heads), dtype=torch.float32, device=dev)
    def select():
        # the newest page's summary is recomputed inside the selection call
        # (same bits as a separate sa_page_summary(last_pages=1) call)
        S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=mode, sink_pages=wl.sink_pages,
                          window_pages=wl.window_pages, top_k=wl.top_k, q=inp["q"] if mu is not None else None,
                          page_summary=mu, scores=inp["scores"], critical_k=wl.critical_k, list_stride=stride,
                          workspace=sel_ws, out=(lists, counts, ccounts), refresh_newest_page=refresh)

    def decode():
        S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=mode, sm_scale=wl.sm_scale,
                           critical_counts=ccounts, ambient_head_mask=inp["ambient_mask"], num_splits=splits,
                           out=out, out_lse=lse, workspace=dec_ws)

    def select_decode():
        S.sa_select_decode(kv, inp["q"], mu, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                           top_k=wl.top_k, sm_scale=wl.sm_scale, refresh_newest_page=True, list_stride=stride,
                           out=(lists, counts, out, lse))

    def step():
        if fused:
            select_decode()
        else:
            select()
            decode()

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    keep = (kv, inp, mu, lists, counts, ccounts, sel_ws, dec_ws, out, lse)
    return g, (lists, counts, ccounts), (step if fused else decode), decode, keep, step


def recorded_traffic(name):
    """HBM bytes of one call of the kernels a record under profiles/ names,
    from their rocprofv3 FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch,
    scaled by what the same counters read for a copy of known size), or None
    when the kernels' sources have changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(root, src), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(round(sum(k["fetch_size_kib_per_dispatch"] * 1024 * rec["fetch_scale"] +
                         k["write_size_kib_per_dispatch"] * 1024 * rec["write_scale"] for k in rec["kernels"])))


def time_back_to_back(calls, reps):
    """Average duration of one call when `reps` calls (cycling over `calls`,
    one per input set) are captured into one HIP graph and replayed between two
    HIP events on the current stream: the kernels run back to back, so the
    figure is their own duration plus the dispatch gaps between them."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            calls[i % len(calls)]()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / reps


def selected_bytes(wl, inp, lists, counts, ccounts):
    """Algorithmic decode bytes: each selected (page, KV head) K and V once (valid tokens)."""
    P = wl.page_size
    el = {"bf16": 2, "fp32": 4, "fp8": 1}[wl.dtype]
    lens = inp["seq_lens"].cpu().numpy()
    L = lists.cpu().numpy()
    C = counts.cpu().numpy()
    per_tok = (wl.d_qk + (0 if wl.latent else wl.d_v)) * el
    per_page = 8 if wl.dtype == "fp8" else 0          # the page's K and V scales
    total = 0
    uniq = 0
    for b in range(wl.batch):
        for s in range(wl.n_sel):
            for lp in L[b, s, :C[b, s]]:
                total += min(P, int(lens[b]) - int(lp) * P) * per_tok + per_page
        if wl.mode == "per_q_head":
            G = wl.group
            for g in range(wl.n_kv_heads):
                pages = set()
                for s in range(g * G, (g + 1) * G):
                    pages.update(int(x) for x in L[b, s, :C[b, s]])
                uniq += sum(min(P, int(lens[b]) - p * P) for p in pages) * per_tok + per_page * len(pages)
    return total, (uniq if wl.mode == "per_q_head" else total)


def fused_bytes(wl, inp, lists, counts, kv_bytes):
    """Algorithmic bytes of one sa_select_decode call: the selected pages' K and
    V (`kv_bytes`, valid tokens), the fp32 mean-key rows of the pages it scores
    (every page but the forced sink and local-window ones), the newest page's
    keys and its new mean-key row (its summary is recomputed), the query rows,
    and what it writes (o, lse, the lists and their counts)."""
    P, D = wl.page_size, wl.d_qk
    G = wl.n_q_heads // wl.n_kv_heads
    lens = inp["seq_lens"].cpu().numpy()
    C = counts.cpu().numpy()
    total = kv_bytes
    for b in range(wl.batch):
        L = int(lens[b])
        n = (L + P - 1) // P
        if n == 0:
            continue
        sink_hi = min(wl.sink_pages, n)
        win_lo = max(n - wl.window_pages, 0)
        scored = n - (sink_hi + max(0, n - max(win_lo, sink_hi)))
        last_nv = L - (n - 1) * P
        per_list = scored * D * 4 + last_nv * D * 2 + D * 4 + wl.q_tokens * G * (2 * D * 2 + 4) + 4
        total += wl.n_kv_heads * per_list + 4 * int(C[b].sum())
    return int(total)


def tiered_flops(wl, inp, lists, counts, ccounts):
    """Algorithmic MLA decode FLOPs: 2*(d_qk + d_v) per (query row, attended
    token); a row attends its Critical pages and the Ambient pages whose head
    set holds its head."""
    P = wl.page_size
    lens = inp["seq_lens"].cpu().numpy()
    L, C, CC = lists.cpu().numpy(), counts.cpu().numpy(), ccounts.cpu().numpy()
    am = inp["ambient_mask"].cpu().numpy().astype(np.int64) & 0xffffffff
    heads = np.arange(wl.n_q_heads)
    total = 0
    for b in range(wl.batch):
        toks = np.zeros(wl.n_q_heads, dtype=np.int64)
        for e in range(C[b, 0]):
            lp = int(L[b, 0, e])
            nv = max(0, min(P, int(lens[b]) - lp * P))
            if e < CC[b, 0]:
                toks += nv
            else:
                bits = (am[b, lp, heads // 32] >> (heads % 32)) & 1
                toks += nv * bits
        total += int(toks.sum()) * wl.q_tokens
    return 2 * (wl.d_qk + wl.d_v) * total


CPU_BASELINE_SECONDS = 10.0   # the oracle repeats its sample until this much CPU time has passed


def cpu_baseline_decode(wl, inp, n_seq=8):
    """The oracle, as is, on the first n_seq sequences of one input set: the
    full step (page means, router scores, selection, attention) repeated until
    CPU_BASELINE_SECONDS have passed."""
    import oracle.sparse_attn_oracle as O
    from threadpoolctl import threadpool_info
    P = wl.page_size
    lens = inp["seq_lens"].cpu().numpy()[:n_seq]
    bt_full = inp["block_table"].cpu()
    pages = [bt_full[b, :math.ceil(int(lens[b]) / P)].long() for b in range(n_seq)]
    allp = torch.cat(pages)
    if wl.dtype == "fp8":
        kp = O.dequantize_pages(inp["k_pool"][allp].cpu().numpy(), inp["k_scale"][allp].cpu().numpy())
        vp = O.dequantize_pages(inp["v_pool"][allp].cpu().numpy(), inp["v_scale"][allp].cpu().numpy())
    else:
        kp = inp["k_pool"][allp].float().cpu().numpy().astype(np.float64)
        vp = None if inp["v_pool"] is None else inp["v_pool"][allp].float().cpu().numpy().astype(np.float64)
    bt = np.full((n_seq, wl.max_pages), -1, dtype=np.int32)
    off = 0
    for b, pg in enumerate(pages):
        bt[b, :len(pg)] = np.arange(off, off + len(pg))
        off += len(pg)
    q = inp["q"][:n_seq].float().cpu().numpy().astype(np.float64)
    am = None if inp["ambient_mask"] is None else inp["ambient_mask"][:n_seq].cpu().numpy().astype(np.int64) & 0xffffffff
    npg = [O.n_pages_of(L, P) for L in lens]
    # page means of every page are built once beforehand, as on the GPU (once
    # per filled page); a step refreshes each sequence's newest page where the
    # GPU step does (bf16 caches), and reads the built means otherwise
    mu_built = None if wl.scores == "gumbel" else O.page_summary(kp, bt, lens, P)
    refresh = wl.scores != "gumbel" and wl.dtype != "fp8"

    def oracle_step():
        if wl.scores == "gumbel":
            scores = inp["scores"][:n_seq].cpu().numpy()
        else:
            mu = mu_built
            if refresh:
                upd = O.page_summary(kp, bt, lens, P, last_pages=1)
                mu = mu_built.copy()
                fresh = ~np.isnan(upd)
                mu[fresh] = upd[fresh]
            scores = O.page_scores(q, mu, bt, lens, P, wl.n_kv_heads, wl.mode)
        lists, counts, cc = O.select_pages(scores, npg, wl.sink_pages, wl.window_pages, wl.top_k, wl.critical_k)
        O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, wl.n_kv_heads, wl.mode, wl.sm_scale, cc, am,
                        d_v=wl.d_v)
        return lists, counts

    reps = 0
    t0 = time.perf_counter()
    while True:
        lists, counts = oracle_step()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_SECONDS:
            break
    el = {"bf16": 2, "fp32": 4, "fp8": 1}[wl.dtype]
    per_tok = (wl.d_qk + (0 if wl.latent else wl.d_v)) * el
    nbytes = sum(min(P, int(lens[b]) - int(lp) * P) * per_tok
                 for b in range(n_seq) for s in range(wl.n_sel) for lp in lists[b, s, :counts[b, s]])
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    return dict(value=round(reps * nbytes / dt / 1e9, 6), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{n_seq} of {wl.batch} sequences, the full step as on the GPU (newest-page mean refresh "
                       f"where the GPU step refreshes, router scores, selection, attention; the other page means "
                       f"built once beforehand), {reps} repetitions (numpy float64 oracle; {dt:.2f} s)",
                seconds=round(dt, 3))


def run_decode(args):
    import sparse_attention_long_page_amd as S
    wl = W.FULL[args.workload]
    dev = torch.device("cuda:0")
    splits = wl.num_splits if args.splits < 0 else args.splits
    sets = []
    for i in range(args.sets):
        inp = W.make_decode_inputs(wl, dev, seed=1000 + i)
        mu = None
        if wl.scores == "summary":
            kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"], d_v=wl.d_v,
                           k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))
            mu = S.sa_page_summary(kv)       # amortised: built once per filled page
        sets.append((inp, mu))
    torch.cuda.synchronize()
    fused = fused_path(wl, splits) and not args.two_calls
    steps = []
    for inp, mu in sets:
        graphs, res, dom, dec, keep, step_call = decode_step_fn(S, wl, inp, mu, splits, fused)
        steps.append((graphs, res, inp, dom, keep, step_call, dec))
    # one graph with one step per input set, in set order
    chain = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chain):
        for st in steps:
            st[5]()
    torch.cuda.synchronize()

    def run_steps(k, chained):
        """k steps in set order: whole chain replays, then single-step graphs."""
        done = 0
        if chained:
            while k - done >= len(steps):
                chain.replay()
                done += len(steps)
        while done < k:
            steps[done % len(steps)][0].replay()
            done += 1

    def timed(k, chained):
        run_steps(args.warmup, chained)
        torch.cuda.synchronize()
        # one event pair around the whole timed region (a pair per step would
        # add its own records between the graph launches)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        run_steps(k, chained)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return 1000.0 * wall / k, 1000.0 * e0.elapsed_time(e1) / k

    single_ms, _ = timed(args.steps, False)
    ms_per_step, step_gpu_us = timed(args.steps, True)
    # per-step spread: single-step graphs, each between its own event pair
    per_step = []
    for i in range(max(args.steps, 20)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        steps[i % len(steps)][0].replay()
        e1.record()
        per_step.append((e0, e1))
    torch.cuda.synchronize()
    step_us = np.array([1000.0 * a.elapsed_time(b) for a, b in per_step])
    pcts = [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)]

    _, (lists, counts, ccounts), inp, _, _, _, _ = steps[0]
    # the dominant kernel alone (the decode, or the fused selection + decode):
    # its calls back to back, inputs rotating
    dec_b2b_us = time_back_to_back([st[3] for st in steps], 4 * len(steps))
    nbytes, uniq = selected_bytes(wl, inp, lists, counts, ccounts)
    algo_bytes = uniq if wl.mode == "per_q_head" else nbytes
    if fused:
        algo_bytes = fused_bytes(wl, inp, lists, counts, nbytes)
    achieved = algo_bytes / (dec_b2b_us * 1e-6) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    if fused:
        tag, kernel = "select_decode", "sa_select_decode (scoring, selection and decode in one kernel)"
    elif wl.latent:
        tag, kernel = "mla_decode", "sa_sparse_decode (latent tiered + split merge)"
    else:
        tag, kernel = "sparse_decode", "sa_sparse_decode (decode kernel + split merge)"
    res = {
        "metric": "sparse-decode selected-KV GB/s (% of HBM peak) + us/layer at 32K ctx, 90% sparsity",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded; N(0,1) q/K/V, planted pages" + ("; E4M3 pages, per-page scales)" if wl.dtype == "fp8"
                                                                    else ")"),
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.context, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.d_qk, "page_size": wl.page_size,
                   "sink_pages": wl.sink_pages, "window_pages": wl.window_pages, "top_k": wl.top_k,
                   "kept_tokens_per_head": int(counts.float().mean().item() * wl.page_size),
                   "splits": splits, "input_sets": args.sets,
                   "step_calls": ["sa_select_decode"] if fused else ["sa_select_pages", "sa_sparse_decode"]},
        "us_per_layer": round(1000.0 * ms_per_step, 2),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "step_gpu_us": round(step_gpu_us, 2),
        "ms_per_step_single_step_graphs": round(single_ms, 5),
        "step_us_p10_p50_p90": pcts,
        "selected_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"{tag}_{wl.name}_traffic.json"),
                     "kernel": kernel, "algorithmic_bytes": algo_bytes,
                     "launch_us": round(dec_b2b_us, 2)},
    }
    if fused:
        # the decode kernel alone, on the lists the fused calls wrote
        d_us = time_back_to_back([st[6] for st in steps], 4 * len(steps))
        d_gbs = nbytes / (d_us * 1e-6) / 1e9
        res["roofline_decode_only"] = {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                                       "kernel": "sa_sparse_decode on the same lists", "algorithmic_bytes": nbytes,
                                       "launch_us": round(d_us, 2)}
    if wl.mode == "per_q_head":
        res["pair_counted_bytes"] = nbytes
    if wl.latent:
        flops = tiered_flops(wl, inp, lists, counts, ccounts)
        tf = flops / (dec_b2b_us * 1e-6) / 1e12
        res["metric"] = "MLA tiered sparse decode: selected-KV GB/s and TFLOP/s (% of HBM and bf16 MFMA peak)"
        res["algorithmic_flops"] = flops
        res["roofline_mfma"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                "kernel": "sa_sparse_decode (latent tiered + split merge)"}
        res["autotune"] = autotune_leg(S, wl, inp, lists, counts, ccounts)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(wl, steps[0][2])
    return res


def autotune_leg(S, wl, inp, lists, counts, ccounts):
    """The per-layer tier search on one step's inputs: the estimated (head,
    page) mass (algorithmic FLOPs 2*d per (query row, page)), the coverage of
    a grid around the configured tiers under the configured budget
    (alpha*G + beta*h entries), and the Ambient head mask of the step's lists."""
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"], d_v=wl.d_v)
    mu = S.sa_page_summary(kv)
    G = wl.n_q_heads // wl.n_kv_heads
    B, T = wl.batch, wl.q_tokens
    mass = torch.empty((B, wl.n_q_heads, wl.max_pages), dtype=torch.float32, device=mu.device)
    ws_m = torch.empty(S.sa_head_page_mass_workspace_size(kv, T, wl.n_q_heads), dtype=torch.uint8, device=mu.device)
    alphas, heads = [0, 2, 4, 8, 12, 16], [8, 16, 32, 64, 128]
    budget = wl.critical_k * G + (wl.top_k - wl.critical_k) * wl.ambient_heads
    ws_t = torch.empty(S.sa_autotune_tiers_workspace_size(kv, len(heads)), dtype=torch.uint8, device=mu.device)
    cov = torch.empty((len(alphas), len(heads)), dtype=torch.float32, device=mu.device)
    choice = torch.empty((3,), dtype=torch.int32, device=mu.device)
    scores = inp["scores"]
    if scores is None:
        # the router's scores of this step (pooled query against the page means)
        scores = torch.empty((B, wl.n_kv_heads, wl.max_pages), dtype=torch.float32, device=mu.device)
        S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=wl.sink_pages,
                          window_pages=wl.window_pages, top_k=wl.top_k, q=inp["q"], page_summary=mu,
                          scores_out=scores)
    mask = torch.empty((B, wl.max_pages, (wl.n_q_heads + 31) // 32), dtype=torch.int32, device=mu.device)
    m_us = time_back_to_back([lambda: S.sa_head_page_mass(kv, inp["q"], mu, wl.sm_scale, out=mass, workspace=ws_m)],
                             8)
    t_us = time_back_to_back([lambda: S.sa_autotune_tiers(kv, mass, scores, q_tokens=T, sink_pages=wl.sink_pages,
                                                          window_pages=wl.window_pages, budget=budget,
                                                          alphas=alphas, ambient_heads=heads, workspace=ws_t,
                                                          out=(cov, choice))], 8)
    a_us = time_back_to_back([lambda: S.sa_ambient_head_mask(kv, mass, lists, counts, ccounts, wl.ambient_heads,
                                                             out=mask)], 8)
    n_pages = int(((inp["seq_lens"].long() + wl.page_size - 1) // wl.page_size).sum().item())
    flops = 2 * wl.d_qk * T * wl.n_q_heads * n_pages
    c = cov.cpu()
    ia, ih, beta = choice.cpu().tolist()
    cfg = c[alphas.index(wl.critical_k), heads.index(wl.ambient_heads)].item() \
        if wl.critical_k in alphas and wl.ambient_heads in heads else None
    return {"head_mass_us": round(m_us, 1), "head_mass_tflops": round(flops / (m_us * 1e-6) / 1e12, 1),
            "search_us": round(t_us, 1), "ambient_mask_us": round(a_us, 1), "budget": budget,
            "grid": {"alphas": alphas, "ambient_heads": heads},
            "kept": {"alpha": alphas[ia], "h": heads[ih], "beta": beta, "coverage": round(c[ia, ih].item(), 5)},
            "configured_coverage": None if cfg is None else round(cfg, 5)}


def prefill_flops(wl, table, counts):
    """Algorithmic prefill FLOPs: 4*d per (query row, head, visible token), the
    visible tokens of row i being those of its group's table blocks at or
    before position q_start + i (QK^T and PV, 2 flops per MAC each)."""
    P = wl.page_size
    pos = wl.q_start + np.arange(wl.q_len, dtype=np.int64)
    T, C = table.cpu().numpy(), counts.cpu().numpy()
    visible = 0
    for g in range(wl.n_kv_heads):
        starts = T[g, :C[g]].astype(np.int64) * P
        seen = np.clip(pos[:, None] - starts[None, :] + 1, 0, P)     # [q_len][blocks]
        visible += int(seen.sum()) * wl.group
    return 4 * wl.d * visible, visible


def cpu_baseline_prefill(wl, inp, table, counts):
    """The oracle, as is, on the first and last Q-block of every head of KV head 0,
    repeated until CPU_BASELINE_SECONDS have passed."""
    import oracle.sparse_attn_oracle as O
    from threadpoolctl import threadpool_info
    P = wl.page_size
    rows = [(i, h) for i in list(range(0, 64)) + list(range(wl.q_len - 64, wl.q_len)) for h in range(wl.group)]
    T, C = table.cpu().numpy(), counts.cpu().numpy()
    q = inp["q"].float().cpu().numpy().astype(np.float64)
    bt = inp["block_table"].cpu().numpy()[0]
    used = T[0, :C[0]]
    # only KV head 0 of the pages the table names is read; copy just those
    kp = np.zeros((wl.n_phys_pages, 1, P, wl.d))
    vp = np.zeros((wl.n_phys_pages, 1, wl.d, P))
    phys = torch.as_tensor(bt[used].astype(np.int64), device=inp["k_pool"].device)
    kp[bt[used], 0] = inp["k_pool"][phys, 0].float().cpu().numpy()
    vp[bt[used], 0] = inp["v_pool"][phys, 0].float().cpu().numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.block_sparse_prefill(q[:, :wl.group], kp, vp, bt, int(inp["seq_lens"][0]), P, wl.q_start,
                               T[:1], C[:1], 1, wl.sm_scale, rows=rows)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_SECONDS:
            break
    pos = wl.q_start + np.array([i for i, _ in rows], dtype=np.int64)
    starts = used.astype(np.int64) * P
    vis = int(np.clip(pos[:, None] - starts[None, :] + 1, 0, P).sum())
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    return dict(value=round(reps * 4 * wl.d * vis / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{len(rows)} (row, head) pairs: first and last 64-row Q-block, all heads of KV head 0, "
                       f"{reps} repetitions (numpy float64 oracle; {dt:.2f} s)", seconds=round(dt, 3))


def run_prefill(args):
    import sparse_attention_long_page_amd as S
    wl = W.FULL[args.workload]
    dev = torch.device("cuda:0")
    sets = []
    for i in range(args.sets):
        inp = W.make_prefill_inputs(wl, dev, seed=2000 + i)
        kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
        out = torch.empty((wl.q_len, wl.n_q_heads, wl.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((wl.q_len, wl.n_q_heads), dtype=torch.float32, device=dev)
        table = torch.full((wl.n_kv_heads, wl.n_kv_blocks), -1, dtype=torch.int32, device=dev)
        counts = torch.zeros((wl.n_kv_heads,), dtype=torch.int32, device=dev)
        sets.append((inp, kv, out, lse, table, counts))
    timer = Timer()

    def step(i):
        inp, kv, out, lse, table, counts = sets[i % len(sets)]
        timer.start("prefill")
        S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, inp["block_mask"], wl.block_q, wl.sm_scale,
                                  out=out, out_lse=lse, block_table_out=table, block_counts_out=counts)
        timer.stop("prefill")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timer.reset()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1000.0 * wall / args.steps
    inp, kv, out, lse, table, counts = sets[0]
    flops, visible = prefill_flops(wl, table, counts)
    k_us = timer.avg_us("prefill")
    achieved = flops / (k_us * 1e-6) / 1e12
    res = {
        "metric": "block-sparse chunked prefill TFLOP/s (% of bf16 MFMA peak) at 128K ctx",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) q/K/V, random 2D block mask)",
        "config": {"workload": wl.name, "q_len": wl.q_len, "q_start": wl.q_start, "kv_tokens": wl.kv_len,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads, "head_dim": wl.d,
                   "page_size": wl.page_size, "block_q": wl.block_q, "random_fraction": wl.random_fraction,
                   "input_sets": args.sets},
        "union_blocks_per_kv_head": [int(c) for c in counts.cpu().tolist()],
        "mask_density": round(float(inp["block_mask"].float().mean().item()), 5),
        "visible_pairs": visible,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(f"block_sparse_prefill_{wl.name}_traffic.json"),
                     "kernel": "sa_block_sparse_prefill (union + attention)", "algorithmic_flops": flops},
    }
    res["mask_variants"] = prefill_mask_variants(S, wl, sets[0], timer)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(wl, inp, table, counts)
    return res


def prefill_mask_variants(S, wl, st, timer, reps=5):
    """Beside the graded random mask (whose union is effectively dense): the
    mask the library's pattern discovery produces (top 8% of the causal blocks
    per row by pooled-query score, plus sink and diagonal), timed itself, and a
    shared-column mask (one 8% column set per KV-head group) whose union stays
    sparse; for each, the union density and the prefill time over it."""
    inp, kv, out, lse, table, counts = st
    mu = S.sa_page_summary(kv)
    top_k = int(0.08 * wl.n_kv_blocks)
    res = {}

    def run(name, fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        timer.reset()
        for _ in range(reps):
            timer.start(name)
            fn()
            timer.stop(name)
        torch.cuda.synchronize()
        return timer.avg_us(name)

    mask = torch.empty((wl.n_q_heads, wl.n_q_blocks, wl.n_kv_blocks), dtype=torch.uint8, device=out.device)
    mask_us = run("mask", lambda: S.sa_prefill_block_mask(kv, 0, inp["q"], wl.q_start, mu, wl.block_q,
                                                           wl.sm_scale, top_k=top_k, out=mask))
    shared = W.make_block_mask(wl.replace(mask_kind="shared_columns"), out.device, seed=2000)
    for name, m in (("produced_top8pct", mask), ("shared_columns_8pct", shared)):
        pf_us = run(name, lambda m=m: S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, m, wl.block_q,
                                                                 wl.sm_scale, out=out, out_lse=lse,
                                                                 block_table_out=table, block_counts_out=counts))
        flops, _ = prefill_flops(wl, table, counts)
        c = [int(x) for x in counts.cpu().tolist()]
        res[name] = {"mask_density": round(float(m.float().mean().item()), 5),
                     "union_density": round(sum(c) / (len(c) * wl.n_kv_blocks), 4),
                     "prefill_us": round(pf_us, 1), "prefill_tflops": round(flops / (pf_us * 1e-6) / 1e12, 1)}
        if name == "shared_columns_8pct":
            res[name]["mean_correction"] = mean_correction_leg(S, wl, st, mu, run)
    res["produced_top8pct"]["mask_producer_us"] = round(mask_us, 1)
    res["produced_top8pct"]["top_k"] = top_k
    return res


def mean_terms(wl, table, counts, seq_len):
    """(row, head) x skipped-block pairs the mean correction adds: per KV
    head, the causal blocks not in its table whose tokens all lie at or
    before the row's position, times the heads of the group."""
    P = wl.page_size
    n_seq = (seq_len + P - 1) // P
    pos = wl.q_start + np.arange(wl.q_len, dtype=np.int64)
    T, C = table.cpu().numpy(), counts.cpu().numpy()
    pairs = 0
    for g in range(wl.n_kv_heads):
        kept = np.zeros(n_seq, dtype=bool)
        kept[T[g, :C[g]]] = True
        kb = np.flatnonzero(~kept).astype(np.int64)
        last_tok = np.minimum(kb * P + P, seq_len) - 1
        pairs += int((pos[:, None] >= last_tok[None, :]).sum()) * wl.group
    return pairs


def mean_correction_leg(S, wl, st, mu, run):
    """Per-page mean values over the whole pool, then the mean correction of
    the prefill just run (its tables, out and lse); algorithmic FLOPs 4*d per
    (row, head, mean term)."""
    inp, kv, out, lse, table, counts = st
    nu = S.sa_page_value_summary(kv)
    ws = torch.empty(S.sa_prefill_mean_correction_workspace_size(kv, wl.n_kv_blocks), dtype=torch.uint8,
                     device=out.device)
    vs_us = run("value_summary", lambda: S.sa_page_value_summary(kv, out=nu))
    mc_us = run("mean_correction", lambda: S.sa_prefill_mean_correction(kv, 0, inp["q"], wl.q_start, table, counts,
                                                                        mu, nu, wl.sm_scale, out, lse, workspace=ws))
    pairs = mean_terms(wl, table, counts, int(inp["seq_lens"][0].item()))
    return {"value_summary_us": round(vs_us, 1), "correction_us": round(mc_us, 1), "mean_term_pairs": pairs,
            "correction_tflops": round(4 * wl.d * pairs / (mc_us * 1e-6) / 1e12, 1)}


def run_hbm_copy(args):
    """Device-to-device copy of a 1 GiB buffer: the measured streaming ceiling
    of this HBM, and the known-size reference that scales the FETCH_SIZE /
    WRITE_SIZE counters of the library's kernels (1 GiB read + 1 GiB written
    per dispatch)."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"metric": "HBM device-to-device copy GB/s (read + write)", "value": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "hbm_copy", "bytes_read": n, "bytes_written": n}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "chunked_prefill_128k":
        res = run_prefill(args)
    elif args.workload == "hbm_copy":
        res = run_hbm_copy(args)
    else:
        res = run_decode(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
