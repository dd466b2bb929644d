#!/usr/bin/env python3
"""Benchmark of the CSA / HCA / DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b,...] [--no-cpu]

Prints ONE JSON line.  ``value`` is CSA prefill tokens/s (8192-token sequence,
64 heads x 512, top-512 of 2048 pool entries, window 128): one step is every
stage of the path over that batch -- window-row rotation, K=V pool and
indexer-key compression, index scores, top-k, sparse attention -- with the
inputs already resident in HBM (the RoPE table is model set-up: built once,
timed on its own and reported beside the step).  Each stage is timed with HIP events on the
stream its kernels run on; ``roofline`` reports the dominant kernel's
algorithmic FLOP/s or bytes/s against the MI355X peak.  CSA decode (64 x 1
token after 131072 cached tokens) is reported in us/step, and the HCA and DSA
workloads in tokens/s.  ``cpu_baseline`` times the CPU oracle on a stratified
sample of the prefill rows.  ``achievable_peaks`` gives what the device
sustains for the two bounding resources (a bf16 matrix-core loop and a
streaming read, libcsa_probe.so), and every stage and roofline carries
``frac_achievable`` against it beside ``frac`` against the published peak.

HBM traffic of the dominant kernels (``roofline.traffic``) comes from two
rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of one workload each,
with ``--calib-copy`` so that a plain device copy of known size is profiled in
the same run; ``--traffic FETCH_DB WRITE_DB`` (no GPU) turns the two counter
databases into profiles/hbm_traffic.json, tagged with a hash of the kernel
sources so that a stale file is ignored.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA prefill tokens/s + decode µs/step; % of MI355X HBM / MFMA peak"
PEAK = {"mfma": (2500.0, "TFLOP/s"), "hbm": (8000.0, "GB/s")}   # bf16 dense MFMA; HBM3E


# ------------------------------------------------------------------ work counts
def ready(t, m, T):
    return np.clip((t + 1) // m, 0, T)


def visible_window(wl, t):
    if not wl.window:
        return np.zeros_like(t)
    return np.minimum(t + 1, wl.window)


def work_counts(wl):
    """Algorithmic work of each stage (flops or bytes), per launch."""
    t = wl.q_pos0 + np.arange(wl.S, dtype=np.int64)
    R = ready(t, wl.m, wl.T)
    e = 2  # bytes per bf16 element
    B = wl.B
    w = {}
    if not wl.decode:
        # one csa_compress_many call: the window rows (read and written once),
        # the K=V pool (rows and gates read, entries written), the index keys
        c = B * wl.ctx * wl.D * e * 2
        if wl.kind != "dsa":
            c += B * (2 * wl.ctx + wl.T) * wl.D * e
        if wl.n_idx_heads:
            gates = 2 if wl.kind != "dsa" else 1
            c += B * (gates * wl.ctx + wl.T) * wl.idx_dim * e
        w["compress"] = ("hbm", c)
    if wl.decode:
        # the new token into both caches: x and gate read, written to the
        # compressor buffers, and (K=V) rotated into the window; a token that
        # closes an entry also reads the other (1+overlap)m - 1 rows of x and
        # gate from the buffers and writes the pooled entry
        L = (1 + wl.overlap) * wl.m

        def append_bytes(closes):
            rows_kv = 5 + (2 * (L - 1) + 1 if closes else 0)
            rows_idx = 4 + (2 * (L - 1) + 1 if closes else 0)
            return B * wl.S * (wl.D * rows_kv + wl.idx_dim * rows_idx) * e
        w["cache_append"] = ("hbm", append_bytes((wl.q_pos0 + 1) % wl.m == 0))
        # beside the step: the update of the token one position earlier, which
        # closes a pool entry when q_pos0 is one past a window's end
        w["cache_append_closing"] = ("hbm", append_bytes(wl.q_pos0 % wl.m == 0))
    if wl.n_idx_heads:
        pairs = int(R.sum()) * B
        if wl.decode:   # streams the index-key pool once: HBM-bound
            w["index_scores"] = ("hbm", B * wl.T * wl.idx_dim * e + pairs * 4 +
                                 B * wl.S * wl.n_idx_heads * (wl.idx_dim * e + 4))
        else:
            w["index_scores"] = ("mfma", pairs * wl.n_idx_heads * (2 * wl.idx_dim + 2))
        w["topk"] = ("hbm", pairs * 4 + B * wl.S * wl.topk * 4)
        # scores and top-k in one kernel: the scores stay on chip
        w["index_topk"] = ("mfma", pairs * wl.n_idx_heads * (2 * wl.idx_dim + 2))
        keys = (visible_window(wl, t) + np.minimum(R, wl.topk)).sum() * B
    else:
        keys = (visible_window(wl, t) + R).sum() * B
    flops = int(keys) * wl.H * (2 * wl.D + 2 * wl.dv)
    if wl.decode:   # gathers the selected K=V rows once: HBM-bound
        w["attention"] = ("hbm", int(keys) * wl.D * e + B * wl.S * wl.H * (wl.D + wl.dv) * e)
    else:
        w["attention"] = ("mfma", flops)
    return w, int(keys)


# ------------------------------------------------------------------ GPU runs
class Runner:
    def __init__(self, wl, csa, torch):
        self.wl, self.csa, self.torch = wl, csa, torch
        self.stages = []          # (name, launch fn)
        self.extra = []           # (name, launch fn, flushed) timed beside the step

    def add(self, name, fn):
        self.stages.append((name, fn))

    def beside(self, name, fn, flushed=False):
        """A launch timed on its own, after the step (not part of it): back to
        back, or (flushed) one launch after each cache flush, as the step's
        stages are."""
        self.extra.append((name, fn, flushed))

    def _capture(self, fns):
        """A HIP graph of the launches of `fns` (launched once on the capture
        stream first; the C entry points enqueue on torch's current stream)."""
        torch = self.torch
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for fn in fns:
                fn()
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        return graph

    def run(self, steps, warmup, flush=None):
        """The step time (the reported value) comes from a HIP graph holding
        one whole step (every stage's launches, no host work between them):
        `warmup` untimed replays, then `steps` timed ones.  The per-stage
        times (each kernel's roofline) come from `steps` eager steps with an
        event pair around every stage on the stream the kernels run on; the
        GPU first runs a spin kernel (or the cache flush) long enough for the
        host to enqueue ahead, so no stage time holds host launch work.
        `flush` (reads that evict the caches) runs before every timed step,
        outside the events."""
        torch = self.torch
        for _ in range(warmup):
            for _, fn in self.stages:
                fn()
        torch.cuda.synchronize()
        whole = self._capture([fn for _, fn in self.stages])
        for _ in range(warmup):
            whole.replay()
        torch.cuda.synchronize()
        if flush is None:
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record()
            for _ in range(steps):
                whole.replay()
            s1.record()
            torch.cuda.synchronize()
            total_ms = s0.elapsed_time(s1)
        else:
            pairs = []
            for _ in range(steps):
                flush()
                s0 = torch.cuda.Event(enable_timing=True)
                s1 = torch.cuda.Event(enable_timing=True)
                s0.record()
                whole.replay()
                s1.record()
                pairs.append((s0, s1))
            torch.cuda.synchronize()
            total_ms = sum(a.elapsed_time(b) for a, b in pairs)
        del whole
        ev = {n: [] for n, _ in self.stages}
        if flush is None:
            torch.cuda._sleep(1 << 22)   # a few ms of spinning: the host runs ahead
        for _ in range(steps):
            if flush is not None:
                flush()
            for name, fn in self.stages:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                ev[name].append((a, b))
        torch.cuda.synchronize()
        avg = {n: float(np.mean([a.elapsed_time(b) for a, b in v])) for n, v in ev.items()}
        beside = {}
        for name, fn, flushed in self.extra:
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            if flushed and flush is not None:
                pairs = []
                for _ in range(steps):
                    flush()
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn()
                    b.record()
                    pairs.append((a, b))
                torch.cuda.synchronize()
                beside[name] = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
                continue
            torch.cuda._sleep(1 << 22)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            beside[name] = a.elapsed_time(b) / steps
        self.beside_ms = beside
        return total_ms / steps, avg


def setup(wl, csa, torch, synth):
    """Inputs resident on the GPU, outputs preallocated, one closure per stage."""
    dev = "cuda"
    a, B, S = wl.act_scale, wl.B, wl.S
    bf = torch.bfloat16

    def gen(name, n, shape, dtype=bf):
        return synth.normal_torch(0, name, n, shape, scale=a, dtype=dtype).to(dev)

    r = Runner(wl, csa, torch)
    # the RoPE table is model set-up (built once, reused by every step); its
    # build is timed on its own and reported beside the step
    cs = torch.empty((wl.n_pos, wl.rope_dim // 2, 2), dtype=torch.float32, device=dev)
    _rope(csa, cs, wl)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _rope(csa, cs, wl)
    e1.record()
    torch.cuda.synchronize()
    r.setup_ms = {"rope_table": e0.elapsed_time(e1)}
    q_pos = torch.full((B,), wl.q_pos0, dtype=torch.int32, device=dev)
    sink = (torch.from_numpy(synth.normal(0, "sink", wl.H, ())).to(dev) if wl.sink else None)
    q = gen("q", B * S, (wl.H, wl.D)).view(B, S, wl.H, wl.D)
    out = torch.empty((B, S, wl.H, wl.dv), dtype=bf, device=dev)
    if wl.decode:
        # caches after q_pos0 tokens: pool and index keys (T entries), the
        # sliding window as a ring (position p at row p mod W), the compressor
        # buffers (raw rows of the last 2m tokens); the step appends the new
        # token to both caches first (no entry closes at this position, so
        # every step repeats the same update)
        pool = gen("pool", B * wl.T, (wl.D,)).view(B, wl.T, wl.D)
        k_idx = gen("k_idx", B * wl.T, (wl.idx_dim,)).view(B, wl.T, wl.idx_dim)
        kv_win = gen("kv_win", B * wl.window, (wl.D,)).view(B, wl.window, wl.D)
        win_pos0 = None
        L = (1 + wl.overlap) * wl.m
        ring_x = gen("ring_x", B * L, (wl.D,)).view(B, L, wl.D)
        ring_g = gen("ring_g", B * L, (wl.D,)).view(B, L, wl.D)
        ring_xi = gen("ring_xi", B * L, (wl.idx_dim,)).view(B, L, wl.idx_dim)
        ring_gi = gen("ring_gi", B * L, (wl.idx_dim,)).view(B, L, wl.idx_dim)
        x_new = gen("x_new", B, (1, wl.D)).view(B, 1, wl.D)
        g_new = gen("g_new", B, (1, wl.D)).view(B, 1, wl.D)
        xi_new = gen("xi_new", B, (1, wl.idx_dim)).view(B, 1, wl.idx_dim)
        gi_new = gen("gi_new", B, (1, wl.idx_dim)).view(B, 1, wl.idx_dim)
        count = torch.full((B,), wl.q_pos0, dtype=torch.int32, device=dev)

        def append(cnt):
            # both caches (K=V with its window, index keys) in one launch
            csa.csa_cache_append_many([
                dict(x=x_new, gate=g_new, count=cnt, ring_x=ring_x, ring_g=ring_g, pool=pool,
                     win=kv_win, m=wl.m, overlap=wl.overlap, rope_dim=wl.rope_dim, cs=cs),
                dict(x=xi_new, gate=gi_new, count=cnt, ring_x=ring_xi, ring_g=ring_gi,
                     pool=k_idx, m=wl.m, overlap=wl.overlap)])

        r.add("cache_append", lambda: append(count))
        # the update of the previous token (position q_pos0 - 1), which closes
        # pool entry q_pos0 / m - 1 when q_pos0 is a multiple of m: timed beside
        # the step, after a cache flush like the step's stages
        count_prev = torch.full((B,), wl.q_pos0 - 1, dtype=torch.int32, device=dev)
        r.beside("cache_append_closing", lambda: append(count_prev), flushed=True)
    else:
        # the sequence's compression in one call: window rows (m = 1, rotated
        # in place of the K=V rows), the K=V pool, the index keys
        x = gen("x", B * wl.ctx, (wl.D,)).view(B, wl.ctx, wl.D)
        kv_win = torch.empty_like(x)
        win_pos0 = torch.zeros((B,), dtype=torch.int32, device=dev)
        passes = [dict(x=x, m=1, overlap=0, rope_dim=wl.rope_dim, cs=cs, pos0=0, out=kv_win)]
        if wl.kind == "dsa":
            pool = kv_win
        else:
            gate = gen("gate", B * wl.ctx, (wl.D,)).view(B, wl.ctx, wl.D)
            pool = torch.empty((B, wl.T, wl.D), dtype=bf, device=dev)
            passes.append(dict(x=x, gate=gate, m=wl.m, overlap=wl.overlap, rope_dim=wl.rope_dim,
                               cs=cs, pos0=0, out=pool))
        if wl.n_idx_heads:
            xi = gen("x_idx", B * wl.ctx, (wl.idx_dim,)).view(B, wl.ctx, wl.idx_dim)
            gi = (None if wl.kind == "dsa" else
                  gen("gate_idx", B * wl.ctx, (wl.idx_dim,)).view(B, wl.ctx, wl.idx_dim))
            k_idx = torch.empty((B, wl.T, wl.idx_dim), dtype=bf, device=dev)
            passes.append(dict(x=xi, gate=gi, m=wl.m, overlap=wl.overlap, out=k_idx))
        r.add("compress", lambda: csa.csa_compress_many(passes))
    kvw = kv_win if wl.window else None
    if wl.n_idx_heads:
        q_idx = gen("q_idx", B * S, (wl.n_idx_heads, wl.idx_dim)).view(B, S, wl.n_idx_heads,
                                                                       wl.idx_dim)
        w_idx = gen("w_idx", B * S, (wl.n_idx_heads,), torch.float32).view(B, S, wl.n_idx_heads)
        idx = torch.empty((B, S, wl.topk), dtype=torch.int32, device=dev)
        scores = torch.empty((B, S, wl.T), dtype=torch.float32, device=dev)
        r.add("index_scores", lambda: csa.csa_index_scores(q_idx, w_idx, k_idx, q_pos,
                                                           m=wl.m, out=scores))
        r.add("topk", lambda: csa.csa_topk(scores, q_pos, k=wl.topk, m=wl.m, out=idx))
        if csa.lib().csa_index_topk_workspace_size(B, S, wl.T, wl.n_idx_heads, wl.idx_dim,
                                                   wl.topk, wl.m, 1) == 0:
            # the fused call (scores kept on chip) is timed beside the step, on the
            # same inputs, with its own output
            idx_f = torch.empty_like(idx)
            r.beside("index_topk", lambda: csa.csa_index_topk(q_idx, w_idx, k_idx, q_pos,
                                                              k=wl.topk, m=wl.m, out=idx_f))
        need = csa.lib().csa_sparse_attn_workspace_size(B, S, wl.H, wl.D, wl.dv, wl.rope_dim,
                                                        wl.topk, wl.window, 1)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        def attention():
            csa.csa_sparse_attn(q, kvw, win_pos0, pool, idx, sink, q_pos, rope_dim=wl.rope_dim,
                                cs=cs, window=wl.window, scale=wl.scale, dv=wl.dv, out=out,
                                workspace=ws)

        r.add("attention", attention)
    else:
        need = csa.lib().hca_attn_workspace_size(B, S, wl.H, wl.D, wl.dv, wl.rope_dim, wl.T,
                                                 wl.window, 1)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        r.add("attention", lambda: csa.hca_attn(q, kvw, win_pos0, pool, sink, q_pos, m=wl.m,
                                                rope_dim=wl.rope_dim, cs=cs, window=wl.window,
                                                scale=wl.scale, dv=wl.dv, out=out, workspace=ws))
    return r


def _rope(csa, cs, wl):
    import ctypes
    import torch
    st = csa.lib().csa_rope_table(ctypes.c_void_p(cs.data_ptr()), wl.n_pos, wl.rope_dim,
                                  float(wl.theta),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError(csa.lib().csa_last_error().decode())


def kernel_source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "sparse_long_context_pool_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_sources") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch", {}).get(f"{workload}/{stage}")


def stage_report(wl, avg_ms, work):
    rep = {}
    for name, ms in avg_ms.items():
        bound, amount = work[name]
        peak, unit = PEAK[bound]
        scale = 1e12 if bound == "mfma" else 1e9
        achieved = amount / (ms * 1e-3) / scale
        rep[name] = {"ms": round(ms, 5), "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "work": amount}
    return rep


def run_workload(name, steps, warmup, csa, torch, synth, WORKLOADS):
    wl = WORKLOADS[name]
    t0 = time.time()
    r = setup(wl, csa, torch, synth)
    torch.cuda.synchronize()
    flush = None
    if wl.decode:
        # the decode working set is comparable to the 256 MB last-level cache:
        # flush it between steps so every step reads HBM, not the cache.  The
        # flush READS 1 GiB (a write would leave dirty lines whose write-back
        # then competes with the timed kernels) and completes before the step.
        # (fp32: its sum reduces in place; an int32 sum would first widen the
        # whole buffer to int64, a 2 GiB write)
        junk = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

        def flush():
            junk.sum()          # stream-ordered before the step that follows
    ms_step, avg = r.run(steps, warmup, flush)
    work, keys = work_counts(wl)
    stages = stage_report(wl, avg, work)
    beside = stage_report(wl, r.beside_ms, work) if r.beside_ms else {}
    dom = max(stages, key=lambda n: stages[n]["ms"])
    print(f"[bench] {name}: {ms_step:.3f} ms/step (setup {time.time() - t0:.1f}s); "
          + ", ".join(f"{n} {v['ms']*1e3:.1f}us {100*v['frac']:.1f}%" for n, v in stages.items())
          + "".join(f"; beside the step: {n} {v['ms']*1e3:.1f}us {100*v['frac']:.1f}%"
                    for n, v in beside.items()),
          file=sys.stderr, flush=True)
    res = {"workload": name, "ms_per_step": round(ms_step, 5),
           "setup_ms": {k: round(v, 5) for k, v in r.setup_ms.items()},
           "tokens_per_s": round(wl.B * wl.S / (ms_step * 1e-3), 1),
           "us_per_step": round(ms_step * 1e3, 2), "stages": stages, "dominant": dom,
           "attended_keys": keys, "beside_step": beside}
    del r
    torch.cuda.empty_cache()
    return wl, res


def run_out_proj(steps, warmup, csa, torch, synth, S=8192, H=64, dv=512, groups=8, rank=1024,
                 hidden=4096):
    """The grouped low-rank output projection (o_groups 8 -> o_lora_rank 1024
    -> hidden 4096) of the prefill workload's attention output [S, H, dv],
    with synthetic weights; timed on its own (it is the step after the
    attention, not part of the hot-path step): `warmup` untimed launches, then
    `steps` launches between two events."""
    dev = "cuda"
    bf = torch.bfloat16
    Kg = H * dv // groups
    o = synth.normal_torch(0, "attn_out", S, (H * dv,), scale=0.5, dtype=bf).to(dev)
    w_a = synth.normal_torch(0, "o_a_proj", groups * rank, (Kg,), scale=Kg ** -0.5,
                             dtype=bf).to(dev).view(groups, rank, Kg)
    w_b = synth.normal_torch(0, "o_b_proj", hidden, (groups * rank,),
                             scale=(groups * rank) ** -0.5, dtype=bf).to(dev)
    mid = torch.empty((S, groups * rank), dtype=bf, device=dev)
    out = torch.empty((S, hidden), dtype=bf, device=dev)

    def fn():
        csa.csa_grouped_out_proj(o, w_a, w_b, mid=mid, out=out)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    torch.cuda._sleep(1 << 22)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    flops = 2 * S * (groups * rank * Kg + hidden * groups * rank)
    achieved = flops / (ms * 1e-3) / 1e12
    rep = {"workload": f"grouped output projection of csa_prefill_bf16's attention output: "
                       f"[{S}, {H}x{dv}] -> {groups} groups x {rank} -> {hidden}",
           "ms": round(ms, 5), "bound": "mfma", "achieved": round(achieved, 2),
           "peak": PEAK["mfma"][0], "unit": "TFLOP/s",
           "frac": round(achieved / PEAK["mfma"][0], 4), "work": flops}
    print(f"[bench] out_proj: {ms * 1e3:.1f}us {100 * rep['frac']:.1f}%", file=sys.stderr,
          flush=True)
    return rep


def achievable_key(st):
    """Which achievable peak a stage is read against: the matrix-core loop of
    about its length (1 ms or 20 ms) for matrix-core stages, the read else."""
    if st["bound"] == "mfma":
        return "mfma_bf16_long" if st["ms"] >= 5.0 else "mfma_bf16_short"
    return "hbm_read"


def add_achievable(stages, ach):
    for st in stages.values():
        st["frac_achievable"] = round(st["achieved"] / ach[achievable_key(st)]["value"], 4)
    return stages


def roofline_of(wl_name, res, ach=None):
    dom = res["dominant"]
    st = res["stages"][dom]
    r = {"kernel": dom, "bound": st["bound"], "achieved": st["achieved"], "peak": st["peak"],
         "unit": st["unit"], "frac": st["frac"],
         "traffic": measured_traffic(wl_name, dom)}
    if ach:
        # the same kernel against what the device sustains (achievable_peaks)
        key = achievable_key(st)
        r["achievable_peak"] = ach[key]["value"]
        r["frac_achievable"] = round(st["achieved"] / ach[key]["value"], 4)
    return r


# ------------------------------------------------------------------ achievable peaks
def achievable_peaks(torch):
    """What the device sustains for the two bounding resources (libcsa_probe.so):
    a bf16 matrix-core loop (two four-wave workgroups per compute unit, eight
    independent chains per wave, no memory traffic) run for about 1 ms and about
    20 ms -- the sustained clock depends on the length of a matrix-core-heavy
    run -- a streaming read of 4 GiB (16x the last-level cache; non-temporal
    loads, 32 workgroups per compute unit), and the LDS read
    rate of 16-byte reads and of the transposing 8-byte operand reads."""
    from sparse_long_context_pool_amd import probe
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    out = {}
    # (the long run first: it also brings the clock up from idle)
    for key, iters, reps in (("mfma_bf16_long", 50000, 3), ("mfma_bf16_short", 2500, 9)):
        tf, _ = probe.mfma_bf16(2 * cus, iters, reps=reps)
        ms = probe.lib().csa_probe_mfma_flops(2 * cus, iters) / (tf * 1e12) * 1e3
        out[key] = {"value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 3)}
    buf = torch.empty(1 << 32, dtype=torch.uint8, device="cuda")
    gbs, _ = probe.hbm_read(buf, 32 * cus, reps=5)
    del buf
    torch.cuda.empty_cache()
    out["hbm_read"] = {"value": round(gbs, 1), "unit": "GB/s", "bytes": 1 << 32}
    # LDS read rates of the two operand widths (one 8-wave workgroup per CU, as
    # the attention kernel runs)
    for key, mode in (("lds_read_b128", 0), ("lds_read_tr_b64", 1)):
        tbs, per_clk, _ = probe.lds_read(mode, cus, 4096, reps=5)
        out[key] = {"value": round(tbs, 2), "unit": "TB/s",
                    "bytes_per_clock_per_cu": round(per_clk, 1)}
    print("[bench] achievable: " + ", ".join(f"{k} {v['value']} {v['unit']}"
                                             for k, v in out.items()),
          file=sys.stderr, flush=True)
    return out


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(WORKLOADS, synth, n_rows=8192):
    """The oracle on the prefill workload: full-sequence compression plus evenly
    spaced query rows (index scores, top-k, attention), scaled to the whole
    sequence (with n_rows = S every row is computed and nothing is scaled)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from parity import Inputs
    wl = WORKLOADS["csa_prefill_bf16"]
    inp = Inputs(wl)
    rows_all = np.arange(wl.ctx)
    x, gate = inp.get("x", rows=rows_all), inp.get("gate", rows=rows_all)
    xi, gi = inp.get("x_idx", rows=rows_all), inp.get("gate_idx", rows=rows_all)
    rows = np.linspace(0, wl.S - 1, n_rows).astype(np.int64)
    q, qi, wi = inp.get("q", rows=rows), inp.get("q_idx", rows=rows), inp.get("w_idx", rows=rows)
    sink = inp.get("sink")
    oracle.ensure_built()
    t0 = time.perf_counter()
    kv_win = oracle.compress(x, None, None, m=1, overlap=0, rope_dim=wl.rope_dim, theta=wl.theta,
                             round_bf16=True)
    pool = oracle.compress(x, gate, None, m=wl.m, overlap=1, rope_dim=wl.rope_dim,
                           theta=wl.theta, round_bf16=True)
    k_idx = oracle.compress(xi, gi, None, m=wl.m, overlap=1, round_bf16=True)
    t1 = time.perf_counter()
    sc = oracle.index_scores(qi, wi, rows, k_idx, m=wl.m)
    idx = oracle.topk(sc, rows, k=wl.topk, m=wl.m)
    oracle.attention(q, rows, kv_win=kv_win, win_pos0=0, window=wl.window, pool=pool, idx=idx,
                     m=wl.m, sink=sink, rope_dim=wl.rope_dim, theta=wl.theta, scale=wl.scale)
    t2 = time.perf_counter()
    total = (t1 - t0) + (t2 - t1) * wl.S / n_rows
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cpu = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(wl.S / total, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu": cpu,
            "sample": (f"csa_prefill_bf16: compression of all {wl.ctx} tokens "
                       f"({t1 - t0:.2f}s) + {n_rows} of {wl.S} query rows, evenly spaced "
                       f"({t2 - t1:.2f}s), scaled to {wl.S} rows"),
            "seconds_measured": round(t2 - t0, 2)}


# ------------------------------------------------------------------ HBM traffic
CALIB_BYTES = 1 << 30       # the calibration copy reads and writes this many bytes
DOMINANT = {                # stage -> kernels that make it (name prefixes)
    "compress": ("csa::(anonymous namespace)::compress_", "csa::(anonymous namespace)::rope_copy"),
    "attention": ("csa::(anonymous namespace)::attn_mfma_kernel",
                  "csa::(anonymous namespace)::attn_combine_kernel",
                  "csa::(anonymous namespace)::attn_generic_kernel"),
    "index_scores": ("csa::(anonymous namespace)::index_scores",),
    "topk": ("csa::(anonymous namespace)::topk_",),
    "index_topk": ("csa::(anonymous namespace)::index_topk_fused",),
    "out_proj": ("csa::(anonymous namespace)::gemm_nt",),
}


def calib_copy(torch):
    """A plain device-to-device copy of CALIB_BYTES (4x the last-level cache, so
    that it streams from and to HBM), three times, so that a counter run sees
    what FETCH_SIZE / WRITE_SIZE report for known traffic."""
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    evict = torch.empty_like(src)
    for _ in range(3):
        evict.fill_(2)
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_values(db_path, counter):
    """kernel name -> the counter's value (KiB) of every dispatch"""
    import sqlite3
    c = sqlite3.connect(db_path).cursor()
    vals = {}
    for name, value in c.execute("select kernel_name, value from counters_collection "
                                 "where counter_name = ? order by dispatch_id", (counter,)):
        name = name[5:] if name.startswith("void ") else name
        vals.setdefault(name, []).append(value)
    return vals


def write_traffic(fetch_db, write_db, workload, out=None):
    """profiles/hbm_traffic.json from a FETCH_SIZE and a WRITE_SIZE run of one
    workload (both with --calib-copy): bytes per launch of each stage's
    kernels, each counter scaled by (known copy bytes) / (what it read for the
    copy)."""
    fetch = _counter_values(fetch_db, "FETCH_SIZE")
    write = _counter_values(write_db, "WRITE_SIZE")

    def copy_kib(d):
        # the calibration copies: the large dispatches of the copy kernel
        big = sorted(v for n, vs in d.items() if "copyBuffer" in n for v in vs
                     if v > CALIB_BYTES / 1024 / 16)
        if not big:
            raise RuntimeError("no calibration copy in the counter database")
        return big[len(big) // 2]

    def mean(vs):
        return sum(vs) / len(vs)

    f_scale = (CALIB_BYTES / 1024) / copy_kib(fetch)
    w_scale = (CALIB_BYTES / 1024) / copy_kib(write)
    out = out or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        doc = json.load(open(out))
        if doc.get("kernel_sources") != kernel_source_hash():
            doc = {}
    except (OSError, ValueError):
        doc = {}
    doc["kernel_sources"] = kernel_source_hash()
    doc.setdefault("bytes_per_launch", {})
    doc.setdefault("calibration", {})
    doc["calibration"][workload] = {"copy_bytes": CALIB_BYTES, "fetch_scale": round(f_scale, 4),
                                    "write_scale": round(w_scale, 4)}
    for stage, prefixes in DOMINANT.items():
        kib_f = sum(mean(v) for n, v in fetch.items() if n.startswith(prefixes))
        kib_w = sum(mean(v) for n, v in write.items() if n.startswith(prefixes))
        if kib_f or kib_w:
            doc["bytes_per_launch"][f"{workload}/{stage}"] = int(
                round((kib_f * f_scale + kib_w * w_scale) * 1024))
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return doc


# ------------------------------------------------------------------ profile summaries
def _short_kernel(name):
    name = name[5:] if name.startswith("void ") else name
    name = name.replace("csa::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def summarize_trace(csv_path, timed):
    """Markdown table of a rocprofv3 kernel trace (`--kernel-trace -f csv`): per
    kernel the number of dispatches and the average duration over all of them
    and over the last `timed` of them (the benchmark's timed eager steps come
    last for every stage kernel)."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3   # us
        per.setdefault(_short_kernel(r["Kernel_Name"]), []).append((int(r["Start_Timestamp"]), dur))
    rows = ["| kernel | dispatches | average, all (us) | average, last %d (us) |" % timed,
            "|---|---:|---:|---:|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        v.sort()
        last = [d for _, d in v[-timed:]]
        rows.append(f"| `{k}` | {len(v)} | {sum(d for _, d in v) / len(v):.1f} | "
                    f"{sum(last) / len(last):.1f} |")
    return "\n".join(rows)


def summarize_pmc(csv_paths):
    """Markdown table of rocprofv3 counter runs (`--pmc ... -f csv`): per kernel
    the mean over its dispatches of MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE of one XCD times the 1024 SIMDs), LDS busy and bank-conflict
    share, texture-addresser busy (TA_TA_BUSY over one XCD's active cycles times
    the 256 compute units), and the raw means of every counter taken."""
    import csv
    vals = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            k = _short_kernel(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = []
    for k, d in vals.items():
        if k.startswith(("at::", "__amd")):     # the benchmark's own fills, copies, spins
            continue
        mean = {c: sum(v) / len(v) for c, v in d.items()}
        line = f"- `{k}`:"
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            # GRBM_GUI_ACTIVE sums the 8 XCDs: one XCD's active cycles are 1/8
            line += f" MFMA busy {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui / 8 * 1024):.3f};"
        if gui and "SQ_LDS_IDX_ACTIVE" in mean:
            line += f" LDS busy {mean['SQ_LDS_IDX_ACTIVE'] / (gui / 8 * 256):.3f};"
            if "SQ_LDS_BANK_CONFLICT" in mean:
                line += (f" bank-conflict cycles / LDS busy "
                         f"{mean['SQ_LDS_BANK_CONFLICT'] / max(mean['SQ_LDS_IDX_ACTIVE'], 1):.3f};")
        if gui and "TA_TA_BUSY" in mean:
            # one texture addresser per compute unit (the counter sums them)
            line += f" TA busy {mean['TA_TA_BUSY'] / (gui / 8 * 256):.3f};"
        line += " raw means: " + ", ".join(f"{c} {v:.4g}" for c, v in sorted(mean.items()))
        out.append(line)
    return "\n".join(out)


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", default="csa_prefill_bf16,csa_decode_bf16,hca_bf16,dsa_bf16")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the rows measured beside the step (output projection)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain copy of known size (for counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write profiles/hbm_traffic.json from two counter databases of "
                         "one --workloads run, then exit (no GPU)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_TRACE_CSV", "TIMED"),
                    help="print a markdown table of a rocprofv3 kernel trace, then exit (no GPU)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="COUNTER_CSV",
                    help="print per-kernel summaries of rocprofv3 counter runs, then exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace[0], int(args.summarize_trace[1])))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.traffic:
        names = [n for n in args.workloads.split(",") if n]
        if len(names) != 1:
            sys.exit("--traffic takes the one workload the counter runs covered")
        print(json.dumps(write_traffic(args.traffic[0], args.traffic[1], names[0])))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design and multi-GPU scaling is not part of this benchmark",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_long_context_pool_amd import csa, synth
    from sparse_long_context_pool_amd.workloads import WORKLOADS
    csa.lib()
    torch.cuda.set_device(0)
    ach = achievable_peaks(torch)

    names = [n for n in args.workloads.split(",") if n]
    results = {}
    for n in names:
        steps = args.steps if n in ("csa_prefill_bf16", "csa_decode_bf16") else max(3, args.steps // 4)
        results[n] = run_workload(n, steps, args.warmup, csa, torch, synth, WORKLOADS)

    main_name = "csa_prefill_bf16" if "csa_prefill_bf16" in results else names[0]
    wl, res = results[main_name]
    line = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": main_name, "B": wl.B, "S": wl.S, "H": wl.H, "D": wl.D,
                   "rope_dim": wl.rope_dim, "m": wl.m, "T": wl.T, "index_heads": wl.n_idx_heads,
                   "index_dim": wl.idx_dim, "index_topk": wl.topk, "window": wl.window,
                   "parallelism": "single GPU"},
        "roofline": roofline_of(main_name, res, ach),
        "stages": add_achievable(res["stages"], ach), "setup_ms": res["setup_ms"],
        "achievable_peaks": ach,
    }
    for n, (w2, r2) in results.items():
        if n == main_name:
            continue
        key = {"csa_decode_bf16": "decode", "hca_bf16": "hca", "dsa_bf16": "dsa"}.get(n, n)
        entry = {"workload": n, "ms_per_step": r2["ms_per_step"], "setup_ms": r2["setup_ms"],
                 "roofline": roofline_of(n, r2, ach), "stages": add_achievable(r2["stages"], ach)}
        if w2.decode:
            entry["us_per_step"] = r2["us_per_step"]
        else:
            entry["tokens_per_s"] = r2["tokens_per_s"]
        line[key] = entry
    if "csa_prefill_bf16" in names and not args.no_next:
        # the rows after the hot path, each measured on its own
        line["next_rows"] = add_achievable(
            {"out_proj": run_out_proj(args.steps, args.warmup, csa, torch, synth)}, ach)
        for n, v in add_achievable(dict(res.get("beside_step", {})), ach).items():
            line["next_rows"][n] = dict(v, workload=f"{main_name}: scores and top-k in one "
                                                    f"call (replaces index_scores + topk)")
    if args.calib_copy:
        calib_copy(torch)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(WORKLOADS, synth)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
