"""Benchmark: sparse decode steps/s and effective KV GB/s on one MI355X.

Workload: Llama-3.1-8B-shaped single-layer decode step, batch 8, 32 query /
8 KV heads, head_dim 128, 16384 cached tokens per sequence, bf16, thoughts of
64-512 tokens, top-8 thoughts + 128-token window, paged (16-token blocks,
random block table). A step = one zr_sparse_decode_step call (scores, top-k,
block lists, attention, combine) for the whole batch, on layer (step mod L) of L
independent layer caches (L = 32 by default: the 17.2 GB cache of a 32-layer
model), so the bytes come from HBM, not from the 256 MB Infinity Cache.

Prints ONE JSON line (rank 0). Inputs are synthetic and resident in HBM before
the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# Figures of the attention kernel on this workload taken with rocprofv3 on the
# same bench (the summaries under profiles/ name the commands):
# - HBM bytes per launch from hardware counters (--pmc FETCH_SIZE, then
#   WRITE_SIZE, each scaled by the counter's reading for a known-size copy);
# - average kernel durations from the kernel trace (--kernel-trace): the runs
#   of back-to-back launches that the roofline figures time with HIP events.
# Valid only for the kernel sources they were taken with: reported as null as
# soon as any of these files changes.
TRAFFIC_SOURCES = ("zr_internal.h", "zr_pair.hip", "zr_attn.hip")
TRAFFIC = {
    "sources_sha256": "8c1c17eb874d74165d3c41e0dbaa0183944c017887ddf2403b9e14de9de787f2",
    "bytes_per_call": 80649117,  # 79,562,665 fetched + 1,086,452 written
    "bytes_per_call_reuse": 80626932,  # 79,538,318 fetched + 1,088,613 written
    "rocprof_kernel_us": 19.00,  # 200 launches of the sparse attention kernel
    "rocprof_kernel_us_reuse": 18.29,  # 401 launches of the kernel on segment records
}


def sources_sha256():
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "hierarchical_sparse_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled(key):
    """A TRAFFIC figure, or None once the kernel sources have changed."""
    return TRAFFIC[key] if TRAFFIC["sources_sha256"] == sources_sha256() else None


def rocprof_figure(key, bytes_per_launch):
    """The roofline figure on the profiler's average kernel duration (no
    launch gaps), or None once the kernel sources have changed."""
    us = profiled(key)
    if us is None:
        return None
    gbs = bytes_per_launch / (us * 1e-6) / 1e9
    return {"avg_kernel_us": us, "achieved": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "source": "rocprofv3 --kernel-trace"}


METRIC = "decode steps/s and effective KV GB/s (% of HBM peak), 16K tokens, batch 8"


def attended_counts(sel, seq_lens, seq_ptr, th_start, th_len, window):
    """Tokens the sparse attention gathers per (sequence, KV head), counted on
    the host from a selection read back from the GPU, for byte accounting:
    the window [T - W, T) plus each selected thought's span clipped below
    T - W (spans do not overlap; a repeated index counts once). int64 [B][Hkv]."""
    sel = np.asarray(sel)
    B, Hkv = sel.shape[0], sel.shape[1]
    n = np.zeros((B, Hkv), dtype=np.int64)
    for b in range(B):
        T = int(seq_lens[b])
        tw = max(0, T - int(window))
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        st = np.asarray(th_start[lo:hi], np.int64)
        en = st + np.asarray(th_len[lo:hi], np.int64)
        for g in range(Hkv):
            idx = np.unique(sel[b, g][(sel[b, g] >= 0) & (sel[b, g] < hi - lo)])
            clipped = np.minimum(en[idx], tw) - np.maximum(st[idx], 0)
            n[b, g] = (T - tw) + int(np.maximum(0, clipped).sum())
    return n


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s, max_threads=16):
    """The CPU oracle, as it stands, on layer 0 of the same workload: whole
    decode steps (scores, top-k, attention for every (sequence, KV head)
    pair), repeated for about ``budget_s`` seconds in two legs of equal
    budget: one thread, then one Python thread per usable host core (at most
    ``max_threads``, the CPU share of one GPU on the box), each running the
    oracle on a contiguous run of the pairs (numpy releases the interpreter
    lock inside its array loops; each thread's BLAS is held to one thread)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from hierarchical_sparse_kv_amd import synth
    from oracle import zr_oracle as O
    f = synth.to_numpy_f32
    q, kp, vp, kb = f(w.q), f(w.k_pool), f(w.v_pool), f(w.summary_keys)
    pairs = [(b, g) for b in range(w.B) for g in range(w.Hkv)]

    def run(chunk):
        O.sparse_decode_step(q, kp, vp, w.block_table, w.seq_lens, w.seq_ptr, w.th_start,
                             w.th_len, kb, w.k, w.window, w.scale, pairs=chunk)

    def leg(n_threads, budget):
        chunks = [pairs[i * len(pairs) // n_threads:(i + 1) * len(pairs) // n_threads]
                  for i in range(n_threads)]
        n = 0
        with ThreadPoolExecutor(n_threads) as ex:
            t0 = time.perf_counter()
            while True:
                if n_threads == 1:
                    run(pairs)
                else:
                    list(ex.map(run, chunks))
                n += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    return n, el

    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    n_thr = max(1, min(max_threads, usable or 1, len(pairs)))
    with threadpool_limits(limits=1):
        n1, el1 = leg(1, budget_s / 2)
        nn, eln = leg(n_thr, budget_s / 2)
    return {"value": nn / eln, "unit": "steps/s", "cores": n_thr, "kind": "oracle",
            "single_thread_steps_per_s": n1 / el1, "host_cores": os.cpu_count(),
            "usable_cores": usable, "cpu_model": cpu_model(),
            "sample": f"full oracle decode steps of layer 0 (all {len(pairs)} (sequence, KV head) "
                      f"pairs, float64 numpy): {n1} step(s) on 1 thread in {el1:.1f} s, then "
                      f"{nn} step(s) on {n_thr} threads (contiguous runs of pairs) in {eln:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the attention figures on the ragged and 64K-token workloads")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the host-memory (PCIe) figure")
    ap.add_argument("--no-zoom", action="store_true",
                    help="skip the multi-granularity (consensus) figure")
    ap.add_argument("--period", type=int, default=35,
                    help="decode steps per semantic boundary for the selection-reuse figure")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="first run an elementwise copy (negation) of 1 GiB into 1 GiB twice, "
                         "untimed: the known-size kernel that scales hardware byte counters "
                         "(FETCH_SIZE, WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode step is built and timed on a "
              "single MI355X (multi-GPU sharding is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    from hierarchical_sparse_kv_amd import synth, zr
    zr.lib()
    torch.cuda.set_device(0)
    dev = "cuda:0"
    L = args.layers
    if args.copy_calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] generating {L} layer caches (config: llama8b-16k-b8)")
    layers, steps = [], []
    for l in range(L):
        # one structure (lengths, thoughts, block table) shared by all layers, as
        # in a model; every layer has its own K/V pools, summary keys and query
        w = synth.make_workload(1, seed=1, value_seed=1000 + l, device=dev)
        layers.append(w)
        steps.append(zr.step_from_workload(w, meta=steps[0] if steps else None))
    torch.cuda.synchronize()
    w0 = layers[0]
    d, s_bytes = w0.d, synth.ELEM_BYTES[w0.dtype]

    # per-layer gathered tokens (selection is query dependent): run each layer once
    for st in steps:
        st.step()
    torch.cuda.synchronize()
    att = [attended_counts(st.sel.cpu().numpy(), w.seq_lens, w.seq_ptr, w.th_start, w.th_len,
                              w.window) for st, w in zip(steps, layers)]
    kv_bytes = [int(a.sum()) * 2 * d * s_bytes for a in att]
    dense_bytes = int(w0.seq_lens.sum()) * w0.Hkv * 2 * d * s_bytes
    q_out_bytes = w0.B * w0.Hq * d * (s_bytes + 4)

    # Steps are captured into HIP graphs (one node per kernel, no host work
    # between kernels), as a serving loop would run them.
    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(n):
                    fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def timed(g, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us per item

    log(f"[bench] capturing {args.warmup} warmup and {args.steps} timed steps")
    g_warm = capture(lambda i: steps[i % L].step(), max(args.warmup, 1))
    g_step = capture(lambda i: steps[i % L].step(), args.steps)
    g_calls = capture(lambda i: steps[i % L].step_calls(), args.steps)
    g_attn = capture(lambda i: steps[i % L].sparse_attn(), args.steps)
    g_dense = capture(lambda i: steps[i % L].dense_attn(), L)
    if args.warmup > 0:
        g_warm.replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    us_per_step = timed(g_step, args.steps)
    ms_per_step = us_per_step / 1e3
    calls_us = timed(g_calls, args.steps)

    # per-step latency (KV-cache management page, "Measuring a cache design":
    # percentiles, not only the mean): one graph per layer holding one step,
    # replayed n_lat times with layers rotating and an event recorded between
    # consecutive replays. A sleep kernel holds the GPU while the host queues
    # every replay, so the intervals are back-to-back step times on the GPU.
    g_one = [capture(lambda i, l=l: steps[l].step(), 1) for l in range(L)]
    n_lat = max(args.steps, 200)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_lat + 1)]
    torch.cuda.synchronize()
    t_q = time.perf_counter()
    torch.cuda._sleep(int(2.4e9 * 0.2))  # ~0.2 s of GPU cycles
    evs[0].record()
    for i in range(n_lat):
        g_one[i % L].replay()
        evs[i + 1].record()
    queued_ms = (time.perf_counter() - t_q) * 1e3
    torch.cuda.synchronize()
    lat = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_lat)])
    latency = {"steps": n_lat, "mean_us": round(float(lat.mean()), 3),
               "p50_us": round(float(np.percentile(lat, 50)), 3),
               "p90_us": round(float(np.percentile(lat, 90)), 3),
               "p99_us": round(float(np.percentile(lat, 99)), 3),
               "max_us": round(float(lat.max()), 3),
               "host_queue_ms": round(queued_ms, 1),
               "note": "one graph replay per step, events between replays, GPU held by a "
                       "sleep kernel while the host queued them"}
    del g_one

    # the whole sparse attention call (block lists, attention, combine)
    attn_us = timed(g_attn, args.steps)
    bytes_per_launch = float(np.mean([kv_bytes[i % L] for i in range(args.steps)]))

    # attention + combine alone: zr_sparse_decode_attn_cached on the lists
    # zr_sparse_decode_attn leaves in each layer's workspace (same window, so the
    # same attended set), timed with HIP events around a graph of back-to-back
    # calls on the stream they run on
    for st in steps:
        st.sparse_attn()
    steps[0].sparse_attn()
    torch.cuda.synchronize()
    ref_out = steps[0].out.clone()
    steps[0].cached_attn(w0.window)
    torch.cuda.synchronize()
    assert torch.equal(ref_out, steps[0].out), "cached call differs from the full call"
    g_gather = capture(lambda i: steps[i % L].cached_attn(w0.window), args.steps)
    gather_us = timed(g_gather, args.steps)
    call_gbs = bytes_per_launch / (gather_us * 1e-6) / 1e9

    # the dominant kernel alone: zr_sparse_decode_attn_partials launches only the
    # attention kernel (its partials + zr_attn_combine give the same output bit
    # for bit, checked here), timed the same way
    steps[0].out.fill_(float("nan"))
    steps[0].cached_partials(w0.window)
    steps[0].combine()
    torch.cuda.synchronize()
    assert torch.equal(ref_out, steps[0].out), "partials + combine differ from the full call"
    g_part = capture(lambda i: steps[i % L].cached_partials(w0.window), args.steps)
    kernel_us = timed(g_part, args.steps)
    achieved = bytes_per_launch / (kernel_us * 1e-6) / 1e9

    # selection reuse (ZoomR Sec. 3.4, Appendix A.3): the attended set is
    # rebuilt at semantic boundaries, about every 35 tokens. Each layer runs
    # its own period: a full step at T0 = T - period + 1, then attention on
    # the kept selection at T0 + i with the window start kept (window grown by
    # i). Two ways between boundaries: zr_sparse_decode_attn_cached (the
    # attention plans every call), and zr_reuse_plan once after the boundary
    # step followed by zr_sparse_decode_attn_reuse (each workgroup starts from
    # its record). Layers rotate call by call, as in the timed steps above.
    R = max(args.period, 1)
    T_full = int(w0.seq_lens[0])
    lens_i = [torch.full((w0.B,), T_full - R + 1 + i, dtype=torch.int32, device=dev)
              for i in range(R)]

    def period_call(c):
        l, i = c % L, (c // L) % R
        if i == 0:
            steps[l].step(seq_lens=lens_i[0])
        else:
            steps[l].cached_attn(w0.window + i, seq_lens=lens_i[i])

    def period_reuse(c):
        l, i = c % L, (c // L) % R
        if i == 0:
            steps[l].step(seq_lens=lens_i[0])
            steps[l].reuse_plan(R - 1, seq_lens=lens_i[0])
        else:
            steps[l].reuse_attn(seq_lens=lens_i[i])

    g_period = capture(period_call, L * R)
    g_period.replay()
    torch.cuda.synchronize()
    period_us = timed(g_period, L * R)
    g_period_r = capture(period_reuse, L * R)
    g_period_r.replay()
    torch.cuda.synchronize()
    period_reuse_us = timed(g_period_r, L * R)
    # the reuse call at T0 + i equals the cached call with window W + i (same
    # attended set; other work split, so compared within the bf16 tolerance)
    i_chk = R - 1
    steps[0].step(seq_lens=lens_i[0])
    steps[0].reuse_plan(R - 1, seq_lens=lens_i[0])
    steps[0].cached_attn(w0.window + i_chk, seq_lens=lens_i[i_chk])
    torch.cuda.synchronize()
    ref_c = steps[0].out.clone()
    steps[0].reuse_attn(seq_lens=lens_i[i_chk])
    torch.cuda.synchronize()
    reuse_diff = float(torch.max(torch.abs(ref_c - steps[0].out)).item())
    assert reuse_diff <= 2e-3, f"reuse call differs from the cached call: {reuse_diff}"
    # the attention kernel between boundaries alone: records of horizon 0 at
    # the lengths of the timed steps (the attended set of the roofline figure)
    for st in steps:
        st.step()
        st.reuse_plan(0)
    torch.cuda.synchronize()
    g_reuse_part = capture(lambda i: steps[i % L].reuse_attn(partials=True), args.steps)
    g_reuse_part.replay()
    reuse_kernel_us = timed(g_reuse_part, args.steps)
    reuse_achieved = bytes_per_launch / (reuse_kernel_us * 1e-6) / 1e9
    g_reuse_call = capture(lambda i: steps[i % L].reuse_attn(), args.steps)
    g_reuse_call.replay()
    reuse_call_us = timed(g_reuse_call, args.steps)
    g_rplan = capture(lambda i: steps[i % L].reuse_plan(R - 1), L)
    g_rplan.replay()
    rplan_us = timed(g_rplan, L)
    del g_reuse_part, g_reuse_call, g_rplan, g_period_r

    # append path: one token per sequence into a paged cache with on-demand
    # blocks (zr_append_kv), and mean summary keys of one completed thought per
    # sequence (zr_summary_keys), same head shapes
    wa = synth.make_workload(1, seed=1, device=dev, overrides=dict(
        seq_len=("fixed", 1024), extra_tokens=args.steps + 16,
        spare_blocks=w0.B * ((args.steps + 15) // 16 + 2)))
    sa = zr.step_from_workload(wa)
    free_np = wa.extra["free_blocks"]
    free = torch.as_tensor(free_np, device=dev)
    free_count = torch.tensor([len(free_np)], dtype=torch.int32, device=dev)
    app_status = torch.empty(wa.B, dtype=torch.int32, device=dev)
    kn = torch.randn((wa.B, wa.Hkv, wa.d), device=dev).to(wa.k_pool.dtype)
    vn = torch.randn((wa.B, wa.Hkv, wa.d), device=dev).to(wa.k_pool.dtype)
    g_app = capture(lambda i: sa.append(kn, vn, free, free_count, app_status), args.steps)
    append_us = timed(g_app, args.steps)
    assert int((app_status != 0).sum()) == 0, "append failed"
    which_np = np.array([int(w0.seq_ptr[b]) + 10 for b in range(w0.B)], np.int32)
    which = torch.as_tensor(which_np, device=dev)
    kb_out = torch.empty_like(steps[0].summary_keys)
    g_sum = capture(lambda i: steps[i % L].compute_summary_keys(which, out=kb_out), args.steps)
    summary_us = timed(g_sum, args.steps)

    # ZoomR's multi-granularity set (Sec. 3.3): per-layer scores and top-k,
    # votes over all layers and KV heads, the consensus set, and each layer's
    # attention over prompt + window + consensus thoughts + other summaries,
    # on L layer caches with the worked example's layout (Sec. 3.5)
    zoom = None
    if not args.no_zoom:
        zl = [synth.make_workload(5, value_seed=2000 + l, device=dev) for l in range(L)]
        wz = zl[0]
        zs = []
        for w in zl:
            zs.append(zr.step_from_workload(w, meta=zs[0] if zs else None))
        cz, npz = wz.extra["c"], wz.extra["prompt"]
        ss = torch.as_tensor(wz.extra["sum_start"], device=dev)
        sl = torch.as_tensor(wz.extra["sum_len"], device=dev)
        votes = torch.empty(wz.n_total, dtype=torch.int32, device=dev)
        cons = torch.empty((wz.B, cz), dtype=torch.int32, device=dev)
        agree = torch.empty(wz.B, dtype=torch.float32, device=dev)
        sel_stack = torch.empty((L,) + tuple(zs[0].sel.shape), dtype=torch.int32, device=dev)

        def boundary(_):
            for l, st in enumerate(zs):
                st.score_topk(sel=sel_stack[l])  # each layer's top-k straight into the stack
            zs[0].consensus(sel_stack, cz, votes, cons, agree)
            # the set is shared by every layer and head: its block lists are built
            # once (layer 0) and every other layer attends on them
            zs[0].zoom_attn(ss, sl, votes, cons, cz, npz)
            for st in zs[1:]:
                st.cached_attn(wz.window, workspace=zs[0].workspace)
            zs[0].reuse_plan(R - 1)  # records for the steps until the next boundary

        g_bound = capture(boundary, 1)
        g_bound.replay()
        torch.cuda.synchronize()
        bound_us = timed(g_bound, L)
        g_between = capture(lambda i: zs[i % L].reuse_attn(workspace=zs[0].workspace),
                            args.steps)
        between_us = timed(g_between, args.steps)
        v_h, c_h = votes.cpu().numpy(), cons.cpu().numpy()
        n_att = []
        for b in range(wz.B):
            lo, hi = int(wz.seq_ptr[b]), int(wz.seq_ptr[b + 1])
            cset = set(int(x) for x in c_h[b] if x >= 0)
            T = int(wz.seq_lens[b])
            toks = np.zeros(T, bool)
            toks[:min(npz, T)] = True
            toks[max(0, T - wz.window):] = True
            for i in range(hi - lo):
                if v_h[lo + i] > 0:
                    s0 = int(wz.th_start[lo + i] if i in cset else wz.extra["sum_start"][lo + i])
                    ln = int(wz.th_len[lo + i] if i in cset else wz.extra["sum_len"][lo + i])
                    toks[s0:s0 + ln] = True
            n_att.append(int(toks.sum()))
        zbytes = int(sum(n_att)) * wz.Hkv * 2 * d * s_bytes
        zoom = {"workload": "zoomr-16k-b8: batch 8, 32/8 heads, d 128, 16384 tokens = 512 prompt "
                            "+ regular U[100,400] / summary U[10,30] segments, top-8 per head, "
                            "c 2, window 512, bf16",
                "layers": L, "votes_per_thought_max": int(v_h.max()),
                "thoughts_voted": int((v_h > 0).sum()), "thoughts": int(wz.n_total),
                "attended_tokens_per_seq": round(float(np.mean(n_att)), 1),
                "kv_reduction": round(float(wz.seq_lens.sum()) / float(sum(n_att)), 3),
                "agreement_mean": round(float(agree.mean().item()), 4),
                "boundary_us_per_layer": round(bound_us, 3),
                "between_us_per_layer": round(between_us, 3),
                "between_gbs": round(zbytes / (between_us * 1e-6) / 1e9, 1)}

    # the same attention + combine kernels on the other scope workloads, each
    # rotating over enough layer caches that one rotation gathers several times
    # the 256 MB Infinity Cache (ragged batch 32: 4 layers, 2.2 GB; 64K tokens
    # x batch 4: 12 layers, 1.4 GB; the 16K x 8 step with fp32 caches: 8
    # layers, 1.2 GB), so that the tiles come from HBM
    others = None
    if not args.no_others:
        others = {}
        for cid, nlay, ov, label in (
                (3, 4, None, "ragged-b32: batch 32, T ~ U[4096, 32768], thoughts U[32, 1024], "
                             "top-8 + 128 window, interleaved blocks"),
                (4, 12, None, "long-64k-b4: batch 4, 65536 tokens, thoughts log-U[32, 2048], "
                              "top-16 + 256 window"),
                (1, 8, dict(dtype="f32"), "llama8b-16k-b8-f32: the 16K x 8 step with fp32 "
                                          "queries and caches (fp32 matrix-core products)")):
            ws_ = [synth.make_workload(cid, value_seed=3000 + l, device=dev, overrides=ov)
                   for l in range(nlay)]
            ss_ = []
            for w in ws_:
                ss_.append(zr.step_from_workload(w, meta=ss_[0] if ss_ else None))
            byts = []
            for w, st in zip(ws_, ss_):
                st.step()
                torch.cuda.synchronize()
                a_ = attended_counts(st.sel.cpu().numpy(), w.seq_lens, w.seq_ptr, w.th_start,
                                        w.th_len, w.window)
                byts.append(int(a_.sum()) * 2 * w.d * synth.ELEM_BYTES[w.dtype])
            g_o = capture(lambda i: ss_[i % nlay].cached_attn(ws_[i % nlay].window), 48)
            g_o.replay()
            us_o = timed(g_o, 48)
            g_k = capture(lambda i: ss_[i % nlay].cached_partials(ws_[i % nlay].window), 48)
            g_k.replay()
            us_k = timed(g_k, 48)
            g_s = capture(lambda i: ss_[i % nlay].step(), 48)
            g_s.replay()
            us_s = timed(g_s, 48)
            gbs = float(np.mean(byts)) / (us_o * 1e-6) / 1e9
            gbs_k = float(np.mean(byts)) / (us_k * 1e-6) / 1e9
            others[ws_[0].name + ("-f32" if ov else "")] = {"workload": label, "layers_rotated": nlay,
                                   "gathered_bytes": int(np.mean(byts)),
                                   "attn_combine_us": round(us_o, 2), "gbs": round(gbs, 1),
                                   "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "attn_kernel_us": round(us_k, 2),
                                   "attn_kernel_gbs": round(gbs_k, 1),
                                   "attn_kernel_frac": round(gbs_k / HBM_PEAK_GBS, 4),
                                   "step_us": round(us_s, 2)}
            del ws_, ss_, g_o, g_k, g_s
            torch.cuda.empty_cache()

    # host-offloaded cache (ZoomR Sec. 3.4, "Decoding Stage"): pools in pinned
    # host memory, each step bringing only the attended set to the GPU.
    # Direct: the attention kernels read the listed blocks over the host link.
    # Staged: zr_stage_selected copies each layer's listed tiles and window
    # into a device staging pool, then attention runs on it; serially (stage,
    # attend, next layer) and pipelined (layer i + 1 staged on a second
    # stream while layer i attends, two staging buffers). 32 layer steps
    # rotate over 4 layers' host pools, each with its own selection.
    offload = None
    if not args.no_offload:
        log("[bench] host-memory pools")
        n_host = min(4, L)
        hosts, pinned = [], []
        for l in range(n_host):
            w = layers[l]
            kp_h, vp_h = w.k_pool.cpu().pin_memory(), w.v_pool.cpu().pin_memory()
            pinned.append((kp_h, vp_h))
            hosts.append(zr.DeviceStep(w.q, kp_h, vp_h, steps[0].block_table, steps[0].seq_lens,
                                       steps[0].seq_ptr, steps[0].th_start, steps[0].th_len,
                                       w.summary_keys, w0.max_per_seq, w0.k, w0.window,
                                       w0.scale, steps[0].max_attended))
        torch.cuda.synchronize()
        hs0 = hosts[0]
        n_off = 10
        g_off = capture(lambda i: hs0.sparse_attn(sel=steps[0].sel), n_off)
        g_off.replay()
        off_us = timed(g_off, n_off)
        g_offd = capture(lambda i: hs0.dense_attn(), 2)
        g_offd.replay()
        offd_us = timed(g_offd, 2)
        stage_blocks = min(w0.max_blocks + 1, -(-steps[0].max_attended // 16) + 2 * w0.k + 2)
        bufs = [zr.Staging(hs0, stage_blocks) for _ in range(2)]
        n_lay = 32

        def stage_only(i):
            hosts[i % n_host].stage(bufs[i % 2], sel=steps[i % n_host].sel)

        def serial(i):
            hosts[i % n_host].stage(bufs[0], sel=steps[i % n_host].sel)
            hosts[i % n_host].attend_staged(bufs[0])

        g_stage = capture(stage_only, n_lay)
        g_serial = capture(serial, n_lay)
        # pipelined: a second stream (default priority) stages while the
        # capture stream attends; events order stage i before attention i and
        # attention i before staging i + 2 into the same buffer
        g_pipe = torch.cuda.CUDAGraph()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        s1.wait_stream(torch.cuda.current_stream())
        ev_st = [torch.cuda.Event() for _ in range(n_lay)]
        ev_at = [torch.cuda.Event() for _ in range(n_lay)]
        with torch.cuda.stream(s1):
            with torch.cuda.graph(g_pipe, stream=s1):
                s2.wait_stream(s1)
                for i in range(n_lay):
                    with torch.cuda.stream(s2):
                        if i >= 2:
                            s2.wait_event(ev_at[i - 2])
                        hosts[i % n_host].stage(bufs[i % 2], sel=steps[i % n_host].sel)
                        ev_st[i].record(s2)
                    s1.wait_event(ev_st[i])
                    hosts[i % n_host].attend_staged(bufs[i % 2])
                    ev_at[i].record(s1)
                s1.wait_stream(s2)
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.synchronize()
        # the staged output equals the direct one (same lists, bit for bit)
        hs0.sparse_attn(sel=steps[0].sel)
        torch.cuda.synchronize()
        direct_out = hs0.out.clone()
        hs0.stage(bufs[0], sel=steps[0].sel)
        hs0.attend_staged(bufs[0])
        torch.cuda.synchronize()
        assert torch.equal(direct_out, hs0.out), "staged attention differs from direct"
        assert int(bufs[0].dropped.sum().item()) == 0, "staging pool too small"
        for g_ in (g_stage, g_serial, g_pipe):
            g_.replay()
        torch.cuda.synchronize()
        stage_us = timed(g_stage, n_lay)
        serial_us = timed(g_serial, n_lay)
        pipe_us = timed(g_pipe, n_lay)
        # bytes moved per layer step: whole (block, KV head) tiles of keys and
        # values, for each pair's listed span blocks and window blocks
        tile = 16 * d * s_bytes
        moved = []
        for l in range(n_host):
            sel_l = steps[l].sel.cpu().numpy()
            nb = 0
            for b in range(w0.B):
                T = int(w0.seq_lens[b])
                tw = max(0, T - w0.window)
                lo = int(w0.seq_ptr[b])
                for g in range(w0.Hkv):
                    blocks = set()
                    for t_ in sel_l[b, g]:
                        if t_ < 0:
                            continue
                        s0 = int(w0.th_start[lo + t_])
                        e = min(s0 + int(w0.th_len[lo + t_]), tw)
                        if e > s0:
                            blocks |= set(range(s0 // 16, (e - 1) // 16 + 1))
                    nb += len(blocks) + (((T - 1) // 16 - tw // 16 + 1) if T > tw else 0)
            moved.append(nb * 2 * tile)
        moved_b = float(np.mean(moved))
        offload = {"pools": f"pinned host memory ({n_host} layers, {n_lay} layer steps)",
                   "direct_sparse_attn_us": round(off_us, 1),
                   "direct_sparse_h2d_gbs": round(kv_bytes[0] / (off_us * 1e-6) / 1e9, 2),
                   "direct_dense_attn_us": round(offd_us, 1),
                   "direct_dense_h2d_gbs": round(dense_bytes / (offd_us * 1e-6) / 1e9, 2),
                   "stage_blocks_per_seq": stage_blocks,
                   "staged_bytes_per_layer": int(moved_b),
                   "stage_us_per_layer": round(stage_us, 1),
                   "stage_h2d_gbs": round(moved_b / (stage_us * 1e-6) / 1e9, 2),
                   "serial_us_per_layer": round(serial_us, 1),
                   "pipelined_us_per_layer": round(pipe_us, 1),
                   "staging_device_bytes": int(2 * (bufs[0].k_stage.numel() * 2
                                                    * bufs[0].k_stage.element_size())),
                   "full_cache_bytes_per_layer": dense_bytes}
        del hosts, pinned, bufs, g_stage, g_serial, g_pipe, g_off, g_offd

    # dense baseline (same caches, every token) for context
    dense_us = timed(g_dense, L)

    cpu = None
    if not args.no_cpu:
        log(f"[bench] cpu oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(w0, args.cpu_seconds)

    steps_per_s = 1000.0 / ms_per_step
    dense_gbs = dense_bytes / (dense_us * 1e-6) / 1e9
    res = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b-16k-b8: one-layer sparse decode step, batch 8, 32/8 GQA "
                               "heads, head_dim 128, 16384 cached tokens, thoughts 64-512, "
                               "top-8 + 128-token window, 16-token paged blocks, bf16",
                   "global_batch": w0.B, "seq_len": int(w0.seq_lens[0]),
                   "layers_rotated": L, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled("bytes_per_call"),
                     "kernel": "attn_mfma_kernel (one zr_sparse_decode_attn_partials call "
                               "on the block lists of zr_sparse_decode_attn)",
                     "avg_launch_us": round(kernel_us, 3),
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "rocprof": rocprof_figure("rocprof_kernel_us", bytes_per_launch)},
        "roofline_between_boundaries": {
            "bound": "hbm", "achieved": round(reuse_achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(reuse_achieved / HBM_PEAK_GBS, 4),
            "kernel": "attn_mfma_kernel on segment records (zr_sparse_decode_attn_reuse with "
                      "out = NULL, records of zr_reuse_plan at the timed steps' lengths)",
            "avg_launch_us": round(reuse_kernel_us, 3),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "traffic": profiled("bytes_per_call_reuse"),
            "rocprof": rocprof_figure("rocprof_kernel_us_reuse", bytes_per_launch),
            "reuse_call_us": round(reuse_call_us, 3),
            "reuse_plan_us": round(rplan_us, 3)},
        "attn_and_combine": {"call": "zr_sparse_decode_attn_cached (attn_mfma_kernel + "
                                     "attn_combine_kernel)",
                             "avg_launch_us": round(gather_us, 3), "gbs": round(call_gbs, 1),
                             "frac": round(call_gbs / HBM_PEAK_GBS, 4)},
        "sparse_attn_call_us": round(attn_us, 3),
        "sparse_attn_call_gbs": round(bytes_per_launch / (attn_us * 1e-6) / 1e9, 1),
        "step_as_three_calls_us": round(calls_us, 3),
        "tokens_per_s": round(steps_per_s * w0.B, 1),
        "latency": latency,
        "selection_reuse": {"period_steps": R,
                            "us_per_step": round(period_reuse_us, 3),
                            "steps_per_s": round(1e6 / period_reuse_us, 1),
                            "between_boundaries": "zr_reuse_plan + zr_sparse_decode_attn_reuse",
                            "cached_calls_us_per_step": round(period_us, 3),
                            "max_abs_diff_reuse_vs_cached": reuse_diff},
        "speedup_vs_dense_attention": round(dense_us / attn_us, 3),
        "other_workloads": others,
        "zoomr_consensus": zoom,
        "host_offload": offload,
        "append_path": {"append_kv_us": round(append_us, 3),
                        "summary_keys_us": round(summary_us, 3),
                        "summary_thoughts_per_call": int(w0.B),
                        "summary_tokens_per_call": int(w0.th_len[which_np].sum())},
        "effective_kv_gbs": round(call_gbs, 1),
        "kv_tokens_per_step": int(np.mean([a.sum() for a in att])),
        "q_out_bytes_per_step": q_out_bytes,
        "dense_baseline": {"avg_launch_us": round(dense_us, 3), "kv_bytes": dense_bytes,
                           "gbs": round(dense_gbs, 1)},
        "kv_reduction": round(dense_bytes / float(np.mean(kv_bytes)), 3),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
