#!/usr/bin/env python3
"""Benchmark of the gated-delta speculative-decoding hot path on one MI355X.

One step = one speculative round over the whole batch: the verify of a
window (8 lanes x 48 layers x 32 value heads / 16 key heads, d_k = d_v =
128, T = 16 window tokens per lane) and the commit of an accepted prefix
(m_lane ~ Uniform{0..16}, seeded, drawn up front), with the recurrent state
carried from one step to the next.  Two ways of running it are timed:
    fused     gdn_commit_verify: the commit of the previous round's prefix
              and the verify of this round in one launch (the headline)
    two-call  gdn_verify, then gdn_commit
Both do the same work per step in steady state.  Inputs are seeded
synthetic tensors (gdn_synth), resident in HBM before the timed region; four
input sets rotate so that the 256 MB Infinity Cache cannot hold a step's
inputs from the previous use.

Printed: one JSON line (metric, value = head-token updates/s, roofline of
the dominant kernel, cpu_baseline = the fp64 oracle on a bounded sample).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--path fused|two-call|both]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "GDN verify+commit head-token updates/s & % HBM roofline (8 lanes, T=16)"

NL, N, HV, HK, DK, DV, T = 48, 8, 32, 16, 128, 128, 16


def alg_bytes_verify(t_lane):
    """Algorithmic bytes of one verify call: per (layer, lane) the S0 read
    (h_v*d_k*d_v*4) plus, per window token, q and k rows (bf16), v (bf16),
    beta and g (f32), o (f32) and the records (raw k f32 [h_k][d_k], u f32
    [h_v][d_v], a (fold, scale) f32 pair per value head)."""
    s0 = HV * DK * DV * 4
    per_tok = (2 * HK * DK * 2 + HV * DV * 2 + 2 * HV * 4 + HV * DV * 4 +
               HK * DK * 4 + HV * DV * 4 + HV * 8)
    return NL * sum(s0 + per_tok * int(t) for t in t_lane)


def alg_bytes_commit(m_lane):
    """S0 read + S_m write for lanes with m > 0, plus m records each."""
    s = HV * DK * DV * 4
    rec = HK * DK * 4 + HV * DV * 4 + HV * 8
    return NL * sum((2 * s + rec * int(m)) if m > 0 else 0 for m in m_lane)


def alg_bytes_kda_verify(t_lane):
    """KDA verify: the S0 read plus, per window token, q and k (bf16), v
    (bf16), beta (f32 per value head), the per-channel gates g (f32
    [h_v][d_k]), o (f32) and the records (raw k f32 [h_k][d_k], u f32
    [h_v][d_v], the per-channel decays f32 [h_v][d_k])."""
    s0 = HV * DK * DV * 4
    per_tok = (2 * HK * DK * 2 + HV * DV * 2 + HV * 4 + HV * DK * 4 +
               HV * DV * 4 + HK * DK * 4 + HV * DV * 4 + HV * DK * 4)
    return NL * sum(s0 + per_tok * int(t) for t in t_lane)


def alg_bytes_kda_commit(m_lane):
    """S0 read + S_m write for lanes with m > 0, plus m KDA records each."""
    s = HV * DK * DV * 4
    rec = HK * DK * 4 + HV * DV * 4 + HV * DK * 4
    return NL * sum((2 * s + rec * int(m)) if m > 0 else 0 for m in m_lane)


def alg_bytes_fused(t_lane, m_prev):
    """Algorithmic bytes of one gdn_commit_verify: per lane-layer the state
    read, the committed state write when m_prev > 0, m_prev records read,
    and the verify traffic of the window without its own state read."""
    s = HV * DK * DV * 4
    rec = HK * DK * 4 + HV * DV * 4 + HV * 8
    win = alg_bytes_verify(t_lane) - NL * len(t_lane) * s
    return win + NL * sum(s + ((s + rec * int(m)) if m > 0 else 0)
                          for m in m_prev)


def alg_bytes_commit_one(m):
    """Bytes of a commit of one lane-layer with m > 0 records replayed."""
    s = HV * DK * DV * 4
    rec = HK * DK * 4 + HV * DV * 4 + HV * 8
    return (2 * s + rec * int(m)) if m > 0 else 0


WINDOW_SOURCES = ("gdn_window.hip", "gdn_window_mfma.hip",
                  "gdn_window_common.h", "gdn_mfma_util.h", "gdn_step.h")


def kernel_source_hash(files=WINDOW_SOURCES):
    """sha256 of the kernel sources with // comments and blank lines removed
    (a comment edit leaves the recorded counters valid)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "commit_gated_delta_amd", "csrc", f)) as fh:
            for line in fh:
                line = re.sub(r"//.*", "", line).rstrip()
                if line:
                    h.update(line.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(kernel):
    """Calibrated HBM bytes per launch from the committed counter record, or
    None when the record is missing or was taken on other kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    k = rec.get(kernel)
    files = (("gdn_prefill.hip",) if kernel.startswith("prefill")
             else WINDOW_SOURCES)
    if not k or k.get("source_sha256") != kernel_source_hash(files):
        return None
    return float(k["bytes_per_launch"])


def region_ms(fn, reps, warmup, stream, settle_s=0.05):
    """Average time of fn(r) over `reps` calls that run back to back, as a
    serving loop runs them: after `warmup` untimed calls, the `reps` calls
    fn(warmup), ..., fn(warmup + reps - 1) are captured once into a HIP graph
    on `stream` (every entry point only launches kernels, so the calls
    capture as they run; fn must launch on `stream`), the graph is replayed
    untimed for at least `settle_s` seconds (a region that starts after the
    GPU has idled through host-side setup otherwise runs its first
    milliseconds slow), then once between one pair of HIP events.  The
    replay runs
    the same kernels with the same arguments as the calls; it removes the
    host work and the dispatch gaps between them (an event record between
    launches is a queue marker on ROCm and would lengthen the launches it
    sits between, so there is one pair for the whole region)."""
    import torch
    if stream == torch.cuda.default_stream():
        raise RuntimeError("region_ms: the timed stream must be capturable "
                           "(not the default stream)")
    for r in range(warmup):
        fn(r)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for r in range(reps):
            fn(warmup + r)
    t0 = time.perf_counter()
    while True:
        graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= settle_s:
            break
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del graph
    return a.elapsed_time(b) / reps


def stream_launch_ms(fn, reps, warmup, stream, settle_s=0.05):
    """The same region with the calls launched one by one from the host
    (host work and dispatch gaps between the launches included), after the
    warm-up calls and the same settling time, spent on the timed calls
    themselves (the steady-state sequence, as the graph replays it)."""
    import torch
    for r in range(warmup):
        fn(r)
    t0 = time.perf_counter()
    r = 0
    while time.perf_counter() - t0 < settle_s:
        fn(warmup + r % reps)
        r += 1
        if r % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for r in range(reps):
        fn(warmup + r)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


PF_L, PF_H, PF_C = 32768, 32, 64
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def prefill_flops(L=PF_L, H=PF_H, C=PF_C, D=128):
    """(useful, issued) MFMA flops of one chunked prefill.  Useful: the dense
    contractions of the chunk form per (chunk, head) -- K K^T, Q K^T, T X,
    P V_new (2 C^2 D each) and K H, Q H, K^T V' (2 C D^2 each).  Issued adds
    the split-bf16 passes: 2 for K H, Q H, K^T V', 3 for T X and P V_new of
    which a quarter is skipped by triangularity."""
    n = ((L + C - 1) // C) * H
    a, b = 2 * C * C * D, 2 * C * D * D
    useful = n * (4 * a + 3 * b)
    issued = n * (2 * a + 2 * 2 * b + 2 * 3 * 0.75 * a + 2 * b)
    return useful, issued


def bench_prefill(reps=10, warmup=2, h_k=PF_H, segments=True):
    """Chunked prefill of one 32,768-token sequence, 32 value heads (h_k key
    heads), d = 128, bf16 q/k/v, zero initial state, checkpoints every
    8,192 tokens, timed by region_ms; with `segments`, also the same
    head-tokens as four 8,192-token sequences."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    p = gs.prefill_inputs(PF_L, PF_H, h_k, 128, 128, (4, h_k))

    def d16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = d16(p.q[None]), d16(p.k[None]), d16(p.v[None])
    beta = torch.from_numpy(p.beta[None]).to(dev)
    g = torch.from_numpy(p.g[None]).to(dev)
    Sf = torch.empty((1, PF_H, 128, 128), device=dev)
    o = torch.empty((1, PF_L, PF_H, 128), device=dev)
    ck = torch.empty((1, PF_L // 8192, PF_H, 128, 128), device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(1, PF_L, PF_H, h_k, 128, 128),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        gdn.prefill_chunked(1, PF_L, PF_H, h_k, 128, 128, q, k, v, beta, g,
                            None, Sf, o, ck, ws, stream=stream)

    ms = region_ms(lambda r: run(), reps, warmup, stream)
    useful, issued = prefill_flops()
    io_bytes = (PF_L * h_k * 128 * 2 * 2 + PF_L * PF_H * 128 * 2 +
                PF_L * PF_H * 4 * 2 + PF_L * PF_H * 128 * 4 +
                (PF_L // 8192 + 1) * PF_H * 128 * 128 * 4)
    rec = {"workload": "1 sequence x 32768 tokens, 32 value / %d key heads, "
                       "d=128, chunk 64, checkpoints every 8192" % h_k,
           "ms": ms, "head_tokens_per_s": PF_L * PF_H / (ms * 1e-3),
           "useful_tflops": useful / (ms * 1e-3) / 1e12,
           "issued_mfma_tflops": issued / (ms * 1e-3) / 1e12,
           "mfma_frac_issued": issued / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
           "mfma_frac_useful": useful / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
           "io_GBps": io_bytes / (ms * 1e-3) / 1e9}
    if not segments:
        return rec
    # The same head-tokens as 4 independent sequences of 8,192 tokens: four
    # times the workgroups, each a quarter of the chunk chain.  This is the
    # pass that produces the outputs in a sequence-parallel prefill with
    # four segments (each segment's chain run from its start state), before
    # the segments' transition matrices and the scan are counted.
    nseg = 4
    Ls = PF_L // nseg
    Sf4 = torch.empty((nseg, PF_H, 128, 128), device=dev)
    ck4 = torch.empty((nseg, Ls // 8192, PF_H, 128, 128), device=dev)

    def run4():
        gdn.prefill_chunked(nseg, Ls, PF_H, h_k, 128, 128, q.view(nseg, Ls, h_k, 128),
                            k.view(nseg, Ls, h_k, 128), v.view(nseg, Ls, PF_H, 128),
                            beta.view(nseg, Ls, PF_H), g.view(nseg, Ls, PF_H), None,
                            Sf4, o.view(nseg, Ls, PF_H, 128), ck4, ws, stream=stream)

    ms4 = region_ms(lambda r: run4(), reps, warmup, stream)
    rec.update({"as_4_sequences_of_8192_ms": ms4,
                "traffic_p1": measured_traffic("prefill_p1"),
                "traffic_p2": measured_traffic("prefill_p2"),
                "peak_mfma_tflops": BF16_MFMA_PEAK_TFLOPS})
    return rec


def bench_prefill_long(reps=3, warmup=1, L=260096, h_v=4, h_k=2, n_seqs=1):
    """Long prefills with few sequence-heads, in segments of 4,096 tokens
    (the library's choice for batches of at most 8 sequence-heads) and as one
    chain (GDN_FLAG_PREFILL_ONE_CHAIN), checkpoints every 8,192, timed by
    region_ms.  The default is the longest prefill the review reports
    (260,096 tokens) on 4 value / 2 key heads -- one GPU's share of 32 heads
    spread over eight."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    ps = [gs.prefill_inputs(L, h_v, h_k, 128, 128, (5, L) if n_seqs == 1
                            else (5, L, i)) for i in range(n_seqs)]

    def d16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    def stack(nm):
        return np.stack([getattr(x, nm) for x in ps])

    q, k, v = d16(stack("q")), d16(stack("k")), d16(stack("v"))
    beta = torch.from_numpy(stack("beta")).to(dev)
    g = torch.from_numpy(stack("g")).to(dev)
    Sf = torch.empty((n_seqs, h_v, 128, 128), device=dev)
    o = torch.empty((n_seqs, L, h_v, 128), device=dev)
    ck = torch.empty((n_seqs, L // 8192, h_v, 128, 128), device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(n_seqs, L, h_v, h_k, 128, 128),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ms = {}
    for seg in (True, False):
        ms[seg] = region_ms(
            lambda r: gdn.prefill_chunked(n_seqs, L, h_v, h_k, 128, 128, q, k,
                                          v, beta, g, None, Sf, o, ck, ws,
                                          stream=stream, segments=seg),
            reps, warmup, stream)
    return {"workload": "%d sequence%s x %d tokens, %d value / %d key heads, "
                        "d=128, chunk 64, checkpoints every 8192"
                        % (n_seqs, "" if n_seqs == 1 else "s", L, h_v, h_k),
            "segments_ms": ms[True], "one_chain_ms": ms[False],
            "speedup": ms[False] / ms[True],
            "head_tokens_per_s": n_seqs * L * h_v / (ms[True] * 1e-3)}


def bench_t_sweep(ts=(1, 2, 4, 6, 8, 12, 16), reps=20, warmup=3):
    """Window length sweep of the same batch (8 lanes x 48 layers x 32 value /
    16 key heads, d = 128) at T in ts, every lane at T: verify alone, and
    the fused commit + verify with the previous window's m ~ U{0..T}.  Shows
    where the per-head state read stops dominating; event-timed."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def d16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    S0 = torch.from_numpy(gs.initial_state(
        gs.WindowShape(NL, N, HV, HK, DK, DV, 1), (9, 0))).to(dev)
    out = []
    for tt in ts:
        shape = gs.WindowShape(NL, N, HV, HK, DK, DV, tt)
        dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, tt)
        t_lane = np.full(N, tt, dtype=np.int32)
        pool = []
        for p in range(4):
            w = gs.window_inputs(shape, (9, tt, p))
            pool.append((d16(w.q), d16(w.k), d16(w.v),
                         torch.from_numpy(w.beta).to(dev),
                         torch.from_numpy(w.g).to(dev)))
        S = S0.clone()
        o = torch.empty((NL, N, tt, HV, DV), device=dev)
        nrec = gdn.records_bytes(dims)
        recs = [torch.empty(nrec, dtype=torch.uint8, device=dev)
                for _ in range(2)]
        ms_all = [gs.accepted_uniform(t_lane, (9, tt, 100 + r))
                  for r in range(warmup + reps + 1)]

        def timed(fn):
            return region_ms(fn, reps, warmup, stream)

        ms_v = timed(lambda r: gdn.verify(dims, t_lane, *pool[r % 4], S, o,
                                          recs[r % 2], stream=stream))
        ms_f = timed(lambda r: gdn.commit_verify(
            dims, ms_all[r], t_lane, recs[(r + 1) % 2], t_lane, *pool[r % 4],
            S, o, recs[r % 2], stream=stream))
        bv = alg_bytes_verify(t_lane)
        bf = float(np.mean([alg_bytes_fused(t_lane, ms_all[warmup + r])
                            for r in range(reps)]))
        upd = int(t_lane.sum()) * NL * HV
        out.append({"t": tt, "verify_ms": ms_v, "fused_ms": ms_f,
                    "verify_updates_per_s": upd / (ms_v * 1e-3),
                    "fused_updates_per_s": upd / (ms_f * 1e-3),
                    "verify_hbm_frac": bv / (ms_v * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "fused_hbm_frac": bf / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del S, o, recs, pool
    return {"workload": "8 lanes x 48 layers x 32/16 heads, d=128, every lane "
                        "at T; fused with the previous window's m ~ U{0..T}",
            "points": out}


def bench_tree(reps=20, warmup=3):
    """Draft-tree verify of the same batch (8 lanes x 48 layers x 32 value /
    16 key heads, d = 128), 16-node trees per lane in depth-first order
    (each node extends the previous one with probability 0.6), plus the
    commit of a drawn accepted path; timed by region_ms, with the inputs
    rotating over four sets and the records over two buffers."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    shape = gs.WindowShape(NL, N, HV, HK, DK, DV, T)
    dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, T)
    t_lane = np.full(N, T, dtype=np.int32)
    pool = []
    for p in range(4):
        w = gs.window_inputs(shape, (8, p))
        pool.append((_dev_bf16(w.q, dev), _dev_bf16(w.k, dev),
                     _dev_bf16(w.v, dev), torch.from_numpy(w.beta).to(dev),
                     torch.from_numpy(w.g).to(dev)))
    parent = gs.tree_parents(t_lane, T, (8, 0))
    paths = gs.accepted_tree_paths(parent, t_lane, (8, 0))
    rebuilds = int(sum((parent[n, t] != t - 1) for n in range(N)
                       for t in range(1, T)))
    S = torch.from_numpy(gs.initial_state(shape, (8, 0))).to(dev)
    o = torch.empty((NL, N, T, HV, DV), device=dev)
    recs = [torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    stream = torch.cuda.current_stream()
    plist = [list(r) for r in parent]

    ms_v = region_ms(lambda r: gdn.verify_tree(
        dims, t_lane, plist, *pool[r % 4], S, o, recs[r % 2], stream=stream),
        reps, warmup, stream)
    # path commits of the same accepted paths, back to back (each replays
    # the path's records of one of the last two trees on the state the
    # previous one left)
    S_c = S.clone()
    ms_c = region_ms(lambda r: gdn.commit_path(dims, paths, t_lane, plist,
                                               recs[r % 2], S_c, stream=stream),
                     reps, warmup, stream)
    upd = N * T * NL * HV
    # a node has the window traffic of a token; the path commit moves the
    # commit's bytes for the path's length
    bv = alg_bytes_verify(t_lane)
    bc = alg_bytes_commit([len(p) for p in paths])
    return {"workload": "8 lanes x 48 layers x 32/16 heads, d=128, 16-node "
                        "depth-first draft trees, accepted-path commit",
            "rebuilds": rebuilds, "verify_ms": ms_v, "commit_ms": ms_c,
            "node_updates_per_s": upd / ((ms_v + ms_c) * 1e-3),
            "verify_hbm_frac": bv / (ms_v * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "commit_hbm_frac": bc / (ms_c * 1e-3) / (HBM_PEAK_GBS * 1e9)}


def bench_kda(reps=20, warmup=3):
    """KDA (per-channel decay) verify + commit on the same batch shape:
    8 lanes x 48 layers x 32/16 heads, d = 128, T = 16, m ~ U{0..16};
    timed by region_ms, with the inputs (per-channel gates included)
    rotating over four sets and the records over two buffers."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    shape = gs.WindowShape(NL, N, HV, HK, DK, DV, T)
    dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, T)
    t_lane = np.full(N, T, dtype=np.int32)
    pool = []
    for p in range(4):
        w = gs.window_inputs(shape, (10, p))
        pool.append((_dev_bf16(w.q, dev), _dev_bf16(w.k, dev),
                     _dev_bf16(w.v, dev), torch.from_numpy(w.beta).to(dev),
                     torch.from_numpy(gs.kda_gates(shape, (10, p))).to(dev)))
    S = torch.from_numpy(gs.initial_state(shape, (10, 0))).to(dev)
    o = torch.empty((NL, N, T, HV, DV), device=dev)
    recs = [torch.empty(gdn.kda_records_bytes(dims), dtype=torch.uint8,
                        device=dev) for _ in range(2)]
    ms_all = [gs.accepted_uniform(t_lane, (10, 1 + r)) for r in range(reps + warmup)]
    stream = torch.cuda.current_stream()
    ms_v = region_ms(lambda r: gdn.kda_verify(dims, t_lane, *pool[r % 4],
                                              S, o, recs[r % 2], stream=stream),
                     reps, warmup, stream)
    # commits of the drawn prefixes, back to back, from the last two
    # verifies' records (each on the state the previous one left)
    ms_c = region_ms(lambda r: gdn.kda_commit(dims, ms_all[r], t_lane,
                                              recs[r % 2], S, stream=stream),
                     reps, warmup, stream)
    upd = N * T * NL * HV
    bv = alg_bytes_kda_verify(t_lane)
    bc = float(np.mean([alg_bytes_kda_commit(m) for m in ms_all[warmup:]]))
    return {"workload": "KDA verify+commit: 8 lanes x 48 layers x 32/16 heads, "
                        "d=128, T=16, m ~ U{0..16}",
            "verify_ms": ms_v, "commit_ms": ms_c,
            "updates_per_s": upd / ((ms_v + ms_c) * 1e-3),
            "verify_hbm_frac": bv / (ms_v * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "commit_hbm_frac": bc / (ms_c * 1e-3) / (HBM_PEAK_GBS * 1e9)}


def bench_snapshot(reps=5):
    """Snapshot of the whole 8-lane, 48-layer state (768 MiB) to a device
    buffer and to pinned host memory, and the restore from pinned memory:
    gdn_state_snapshot / gdn_state_restore, event-timed."""
    import torch
    import commit_gated_delta_amd as gdn
    dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, T)
    lanes = list(range(N))
    S = torch.randn((NL, N, HV, DK, DV), device="cuda")
    dev_snap = torch.empty((N, NL, HV, DK, DV), device="cuda")
    host_snap = torch.empty((N, NL, HV, DK, DV), pin_memory=True)
    stream = torch.cuda.current_stream()
    nbytes = S.numel() * 4

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

    d2d = timed(lambda: gdn.state_snapshot(dims, lanes, S, dev_snap, stream=stream))
    d2h = timed(lambda: gdn.state_snapshot(dims, lanes, S, host_snap, stream=stream))
    h2d = timed(lambda: gdn.state_restore(dims, lanes, host_snap, S, stream=stream))
    return {"workload": "state of 8 lanes x 48 layers x 32 heads x 128 x 128 "
                        "f32 (768 MiB)",
            "bytes": nbytes,
            "device_ms": d2d, "device_GBps": 2 * nbytes / (d2d * 1e-3) / 1e9,
            "device_hbm_frac": 2 * nbytes / (d2d * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "to_pinned_host_ms": d2h,
            "to_pinned_host_GBps": nbytes / (d2h * 1e-3) / 1e9,
            "from_pinned_host_ms": h2d,
            "from_pinned_host_GBps": nbytes / (h2d * 1e-3) / 1e9}


def _dev_bf16(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)


def bench_token_verify(reps=20, warmup=3):
    """The token-by-token verify at the headline batch (8 lanes x 48 layers x
    32/16 heads, d = 128, T = 16) with GDN_FLAG_TOKENWISE: the kernel that
    evaluates the rule one token at a time and holds every intermediate
    state (the design that the block form replaces at these shapes).
    Timed by region_ms."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    shape = gs.WindowShape(NL, N, HV, HK, DK, DV, T)
    dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, T)
    t_lane = np.full(N, T, dtype=np.int32)
    pool = []
    for p in range(4):
        w = gs.window_inputs(shape, (12, p), t_lane=t_lane)
        pool.append((_dev_bf16(w.q, dev), _dev_bf16(w.k, dev),
                     _dev_bf16(w.v, dev), torch.from_numpy(w.beta).to(dev),
                     torch.from_numpy(w.g).to(dev)))
    S = torch.from_numpy(gs.initial_state(shape, (12, 0))).to(dev)
    o = torch.empty((NL, N, T, HV, DV), device=dev)
    recs = [torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    stream = torch.cuda.current_stream()
    ms = region_ms(lambda r: gdn.verify(dims, t_lane, *pool[r % 4], S, o,
                                        recs[r % 2], stream=stream,
                                        tokenwise=True),
                   reps, warmup, stream)
    bv = alg_bytes_verify(t_lane)
    return {"workload": "verify of 8 lanes x 48 layers x 32/16 heads, d=128, "
                        "T=16 on the token-by-token kernel (GDN_FLAG_TOKENWISE)",
            "verify_ms": ms,
            "updates_per_s": int(t_lane.sum()) * NL * HV / (ms * 1e-3),
            "verify_hbm_frac": bv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_general_shapes(reps=10, warmup=2):
    """Shapes beyond the pages' windows, on the same 8-lane x 48-layer x
    32/16-head batch (d = 128): f32 inputs at T = 16 (block form, f32 rows
    in three bf16 parts), bf16 windows of 32 and 64 tokens (block form in
    blocks of 16) and 32-node draft trees (block form, two blocks of 16).
    Verify, commit and the fused round are timed by
    region_ms; HBM fractions against the same algorithmic byte counts as the
    headline (inputs at their own width)."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn):
        return region_ms(fn, reps, warmup, stream)

    out = []
    for name, tm, bf16, tree in (("f32_T16", 16, False, False),
                                 ("bf16_T32", 32, True, False),
                                 ("bf16_T64", 64, True, False),
                                 ("bf16_tree32", 32, True, True)):
        shape = gs.WindowShape(NL, N, HV, HK, DK, DV, tm)
        dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, tm)
        t_lane = np.full(N, tm, dtype=np.int32)
        # two input sets (each at least 200 MB) in rotation, and two record
        # buffers: no call finds the previous call's inputs or records in
        # the 256 MB Infinity Cache
        sets = []
        for p in range(2):
            w = gs.window_inputs(shape, (13, tm, int(bf16), p), bf16=bf16)
            if bf16:
                ins = (_dev_bf16(w.q, dev), _dev_bf16(w.k, dev),
                       _dev_bf16(w.v, dev))
            else:
                ins = tuple(torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
            sets.append(ins + (torch.from_numpy(w.beta).to(dev),
                               torch.from_numpy(w.g).to(dev)))
        S = torch.from_numpy(gs.initial_state(shape, (13, tm))).to(dev)
        o = torch.empty((NL, N, tm, HV, DV), device=dev)
        nrec = gdn.records_bytes(dims)
        recs = [torch.empty(nrec, dtype=torch.uint8, device=dev)
                for _ in range(2)]
        m_all = [gs.accepted_uniform(t_lane, (13, tm, r))
                 for r in range(warmup + reps)]
        isz = 2 if bf16 else 4
        # inputs at their own width: q, k, v rows of isz bytes per element
        win_extra = (0 if bf16 else
                     (2 * HK * DK * 2 + HV * DV * 2) * NL * N * tm)
        bv = alg_bytes_verify(t_lane) + win_extra
        rec = {"shape": name, "t": tm, "inputs": "bf16" if bf16 else "f32"}
        if tree:
            parent = [list(p) for p in gs.tree_parents(t_lane, tm, (13, tm))]
            paths = gs.accepted_tree_paths(np.array(parent), t_lane, (13, tm))
            ms_v = timed(lambda r: gdn.verify_tree(dims, t_lane, parent,
                                                   *sets[r % 2], S, o,
                                                   recs[r % 2], stream=stream))
            Sc = S.clone()
            ms_c = timed(lambda r: gdn.commit_path(dims, paths, t_lane, parent,
                                                   recs[r % 2], Sc,
                                                   stream=stream))
            bc = alg_bytes_commit([len(p) for p in paths])
            rec.update({"verify_ms": ms_v, "commit_ms": ms_c,
                        "verify_hbm_frac": bv / (ms_v * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "commit_hbm_frac": bc / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "node_updates_per_s": N * tm * NL * HV / (ms_v * 1e-3)})
        else:
            ms_v = timed(lambda r: gdn.verify(dims, t_lane, *sets[r % 2], S,
                                              o, recs[r % 2], stream=stream))
            ms_f = timed(lambda r: gdn.commit_verify(
                dims, m_all[r], t_lane, recs[(r + 1) % 2], t_lane,
                *sets[r % 2], S, o, recs[r % 2], stream=stream))
            bf = float(np.mean([alg_bytes_fused(t_lane, m) for m in m_all]))
            bf += win_extra
            upd = N * tm * NL * HV
            rec.update({"verify_ms": ms_v, "fused_ms": ms_f,
                        "verify_hbm_frac": bv / (ms_v * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "fused_hbm_frac": bf / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "fused_updates_per_s": upd / (ms_f * 1e-3)})
        out.append(rec)
        del S, o, recs, ins, sets
        torch.cuda.empty_cache()
    return {"workload": "8 lanes x 48 layers x 32/16 heads, d=128, every "
                        "lane at T (fused: previous window's m ~ U{0..T}); "
                        "windows and 32-node trees in blocks of 16", "points": out}


# Synthetic workloads of the speculative-decoding round, timed as chains of
# fused rounds (gdn_commit_verify: round r commits the accepted prefix of the
# same state set's previous window and verifies window r).
CHAIN_CONFIGS = {
    "one_lane_100_rounds": dict(
        n_lanes=1, t_max=16, rounds=400, n_sets=4, pool=8, t_kind="fixed",
        m_kind="uniform",
        workload="1 lane x 48 layers x 32 value / 16 key heads, d=128, T=16, "
                 "m ~ U{0..16}; 4 state sets (96 MiB each) rotated so that "
                 "the 256 MB Infinity Cache cannot hold a set between its "
                 "rounds; 100 chained rounds per set"),
    "eight_lanes_ragged": dict(
        n_lanes=8, t_max=16, rounds=64, n_sets=1, pool=4, t_kind="ragged",
        m_kind="uniform",
        workload="8 lanes x 48 layers x 32/16 heads, d=128, per-lane window "
                 "T ~ U{1..16} and m ~ U{0..T} drawn every round, 64 chained "
                 "rounds"),
    "twelve_lanes_t6_256_rounds": dict(
        n_lanes=12, t_max=6, rounds=256, n_sets=1, pool=4, t_kind="fixed",
        m_kind="binomial",
        workload="12 lanes x 48 layers x 32/16 heads, d=128, T=6, "
                 "m ~ Binomial(6, 0.7), 256 chained rounds"),
}


def bench_chain(name, cfg, warmup=4, sample_layer=17):
    """One synthetic workload as a chain of fused rounds, event-timed over
    the whole chain.  Returns the timing record and, for the parity check of
    the CPU leg, the sampled chain (one layer of the state set that ran the
    last round): its inputs, initial state, final state and last outputs.
    Also checks on the GPU that the final commit of that layer is bit for
    bit the state a verify with debug states held after the accepted
    prefix."""
    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    Nl, tm, R, ns, P = (cfg["n_lanes"], cfg["t_max"], cfg["rounds"],
                        cfg["n_sets"], cfg["pool"])
    key = 20 + list(CHAIN_CONFIGS).index(name)
    shape = gs.WindowShape(NL, Nl, HV, HK, DK, DV, tm)
    dims = gdn.Dims.of(NL, Nl, HV, HK, DK, DV, tm)
    full = np.full(Nl, tm, dtype=np.int32)
    pool_np, pool = [], []
    for p in range(P):
        w = gs.window_inputs(shape, (key, p), t_lane=full)
        pool_np.append(w)
        pool.append((_dev_bf16(w.q, dev), _dev_bf16(w.k, dev),
                     _dev_bf16(w.v, dev), torch.from_numpy(w.beta).to(dev),
                     torch.from_numpy(w.g).to(dev)))
    if cfg["t_kind"] == "ragged":
        t_all = [gs.window_lengths(Nl, tm, (key, r)) for r in range(R)]
    else:
        t_all = [full.copy() for _ in range(R)]
    if cfg["m_kind"] == "binomial":
        m_all = [gs.accepted_binomial(t_all[r], 0.7, (key, r)) for r in range(R)]
    else:
        m_all = [gs.accepted_uniform(t_all[r], (key, r)) for r in range(R)]
    S0 = [gs.initial_state(gs.WindowShape(NL, Nl, HV, HK, DK, DV, 1),
                           (key, 1000 + j)) for j in range(ns)]
    S = [torch.from_numpy(x).to(dev) for x in S0]
    nrec = gdn.records_bytes(dims)
    recs = [[torch.empty(nrec, dtype=torch.uint8, device=dev) for _ in range(2)]
            for _ in range(ns)]
    o = torch.empty((NL, Nl, tm, HV, DV), device=dev)
    zero = np.zeros(Nl, dtype=np.int32)

    def run(n_rounds, evs=None, strm=None):
        strm = stream if strm is None else strm
        prev = [None] * ns
        for r in range(n_rounds):
            j = r % ns
            cur = (r // ns) % 2
            t_prev, m_prev = (zero, zero) if prev[j] is None else prev[j]
            if evs is not None and r == 0:
                evs[0].record(stream)
            gdn.commit_verify(dims, m_prev, t_prev, recs[j][1 - cur],
                              t_all[r], *pool[r % P], S[j], o, recs[j][cur],
                              stream=strm)
            prev[j] = (t_all[r], m_all[r])
        if evs is not None:
            evs[1].record(stream)
        return prev

    run(warmup)
    torch.cuda.synchronize()
    for j in range(ns):
        S[j].copy_(torch.from_numpy(S0[j]))
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    prev = run(R, ev)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    # end of every chain: commit the last window's accepted prefix
    js = (R - 1) % ns
    ls = sample_layer
    S_pre = S[js][ls:ls + 1].clone()
    for j in range(ns):
        last = R - 1 - ((R - 1 - j) % ns)
        gdn.commit(dims, prev[j][1], prev[j][0], recs[j][(last // ns) % 2],
                   S[j], stream=stream)
    o_last = o[ls:ls + 1].cpu().numpy()
    S_end = S[js][ls:ls + 1].cpu().numpy()
    # bit-exact replay on the sampled layer: verify the last window of set
    # js with debug states from the state before its final commit
    d1 = gdn.Dims.of(1, Nl, HV, HK, DK, DV, tm)
    inp = [x[ls:ls + 1] for x in pool[(R - 1) % P]]
    dbg = torch.empty((1, Nl, tm, HV, DK, DV), device=dev)
    o1 = torch.empty((1, Nl, tm, HV, DV), device=dev)
    r1 = torch.empty(gdn.records_bytes(d1), dtype=torch.uint8, device=dev)
    gdn.verify(d1, t_all[R - 1], *inp, S_pre, o1, r1, dbg, stream=stream)
    torch.cuda.synchronize()
    dbg_np, pre_np = dbg.cpu().numpy(), S_pre.cpu().numpy()
    bitexact = True
    for n in range(Nl):
        mm = int(m_all[R - 1][n])
        want = pre_np[0, n] if mm == 0 else dbg_np[0, n, mm - 1]
        bitexact &= bool(np.array_equal(S_end[0, n], want))
    # The same chain captured once into a HIP graph and replayed (every entry
    # point only launches kernels, so the rounds capture as they run): the
    # rounds then follow each other with no host work in between.  The
    # replay continues from the states the chain above left.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(R, None, side)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while True:                  # settle, as in region_ms
        graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= 0.05:
            break
    ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ge[0].record(stream)
    graph.replay()
    ge[1].record(stream)
    torch.cuda.synchronize()
    ms_g = ge[0].elapsed_time(ge[1])
    del graph
    upd = sum(int(t.sum()) for t in t_all) * NL * HV
    m_prev_seq = [zero if r < ns else m_all[r - ns] for r in range(R)]
    byts = sum(alg_bytes_fused(t_all[r], m_prev_seq[r]) for r in range(R))
    rec = {"workload": cfg["workload"], "rounds": R, "ms_total": ms,
           "ms_per_round": ms / R, "updates_per_s": upd / (ms * 1e-3),
           "alg_bytes_per_round": byts / R,
           "alg_GBps": byts / (ms * 1e-3) / 1e9,
           "hbm_roofline_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "graph_replay": {
               "ms_per_round": ms_g / R,
               "updates_per_s": upd / (ms_g * 1e-3),
               "hbm_roofline_frac": byts / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS},
           "bitexact_replay_sampled_layer": bitexact,
           "parity": None}
    sample = {"name": name, "layer": ls, "set": js, "rounds": [
        r for r in range(R) if r % ns == js], "pool_np": pool_np, "P": P,
        "t_all": t_all, "m_all": m_all, "S0": S0[js][ls:ls + 1],
        "S_end": S_end, "o_last": o_last}
    del S, recs, pool, o, dbg
    torch.cuda.empty_cache()
    return rec, sample


def _layer_f64(w, ls):
    """fp64 inputs of one layer of a window input set, shapes [1, ...]."""
    q, k, v, b, g = w.as_f64()
    return tuple(a[ls:ls + 1] for a in (q, k, v, b, g))


def oracle_chain_parity(sample):
    """The fp64 oracle over a sampled chain (one layer of one state set,
    every round of that set): the final state and the last round's outputs,
    against the GPU's.  Max block-relative error per (lane, head) block, and
    the oracle's own throughput on this sample."""
    import oracle
    S = sample["S0"].astype(np.float64)
    rounds = sample["rounds"]
    t0 = time.perf_counter()
    upd = 0
    o_ref = None
    for r in rounds:
        q, k, v, b, g = _layer_f64(sample["pool_np"][r % sample["P"]],
                                   sample["layer"])
        t_lane = sample["t_all"][r]
        if r == rounds[-1]:
            o_ref, _ = oracle.verify(q, k, v, b, g, S, t_lane)
        S = oracle.commit(q, k, v, b, g, S, sample["m_all"][r])
        upd += int(t_lane.sum()) * HV
    dt = time.perf_counter() - t0

    def blk(x, ref, axes):
        x = np.moveaxis(np.asarray(x, np.float64), axes, range(len(axes)))
        ref = np.moveaxis(np.asarray(ref, np.float64), axes, range(len(axes)))
        nb = int(np.prod(x.shape[:len(axes)]))
        x, ref = x.reshape(nb, -1), ref.reshape(nb, -1)
        den = np.max(np.abs(ref), axis=1)
        return float(np.max(np.max(np.abs(x - ref), axis=1) /
                            np.where(den > 0, den, 1.0)))

    o_gpu = np.array(sample["o_last"], dtype=np.float64)
    t_last = sample["t_all"][rounds[-1]]
    for n, t in enumerate(t_last):
        o_gpu[:, n, t:] = 0.0
        o_ref[:, n, t:] = 0.0
    return {"sample": "layer %d, state set %d: %d chained rounds"
                      % (sample["layer"], sample["set"], len(rounds)),
            "max_rel_err_S": blk(sample["S_end"], S, (0, 1, 2)),
            "max_rel_err_o": blk(o_gpu, o_ref, (0, 1, 3)),
            "oracle_s": dt, "oracle_updates_per_s": upd / dt}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family / model /
    stepping numbers (a virtualised host may report only the brand) and the
    logical CPUs this process may run on."""
    import os
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" not in line:
                    if info:
                        break       # first processor's block only
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        pass
    import platform
    name = info.get("model name") or platform.processor() or "unknown"
    ids = ", ".join("%s %s" % (k.replace("cpu ", ""), info[k])
                    for k in ("cpu family", "model", "stepping") if k in info)
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return "%s (%s; %s logical CPUs usable of %s)" % (
        name, ids or "ids unknown", usable, os.cpu_count())


def _parse_clocks(text):
    try:
        d = json.loads(text)
    except ValueError:
        return None
    for card in d.values():
        if isinstance(card, dict):
            return {k.strip(" :"): v for k, v in card.items()
                    if any(x in k.lower() for x in ("sclk", "mclk", "fclk"))}
    return None


def gpu_clocks_under_load(busy, seconds=1.5):
    """Engine and memory clocks read by rocm-smi (a child process) while
    `busy()` keeps the GPU running the headline kernel; None if rocm-smi is
    unavailable."""
    import subprocess
    import torch
    try:
        pr = subprocess.Popen(["rocm-smi", "--showclocks", "--json"],
                              stdout=subprocess.PIPE,
                              stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    while pr.poll() is None and time.perf_counter() - t0 < seconds + 30:
        busy()
        torch.cuda.synchronize()
    try:
        out, _ = pr.communicate(timeout=30)
    except subprocess.SubprocessError:
        pr.kill()
        return None
    return _parse_clocks(out)


def cpu_baseline(rounds=16):
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workload: `rounds` chained rounds (verify + commit) of the full
    48-layer x 8-lane batch at T = 16; scaled to head-token updates/s."""
    import gdn_synth as gs
    import oracle
    shape = gs.WindowShape(NL, N, HV, HK, DK, DV, T)
    S = gs.initial_state(shape, (9, 0)).astype(np.float64)
    dt = 0.0
    for r in range(rounds):
        w = gs.window_inputs(shape, (9, r))
        m = gs.accepted_uniform(w.t_lane, (9, r))
        q, k, v, b, g = w.as_f64()
        t0 = time.perf_counter()
        oracle.verify(q, k, v, b, g, S, w.t_lane)
        S = oracle.commit(q, k, v, b, g, S, m)
        dt += time.perf_counter() - t0
    upd = rounds * NL * N * T * HV
    cores = oracle.num_threads()
    # the same round at one thread: a single chained round of the batch
    w = gs.window_inputs(shape, (9, rounds))
    m = gs.accepted_uniform(w.t_lane, (9, rounds))
    q, k, v, b, g = w.as_f64()
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.verify(q, k, v, b, g, S, w.t_lane)
        oracle.commit(q, k, v, b, g, S, m)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    return {"value": upd / dt, "unit": "head-token updates/s",
            "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d chained rounds (verify + commit) of the full "
                      "48-layer x 8-lane batch, T=16, fp64 C oracle with "
                      "OpenMP over chains; %.1f s of oracle time" % (rounds, dt),
            "one_thread": {"value": NL * N * T * HV / dt1, "cores": 1,
                           "sample": "1 round (verify + commit) of the same "
                                     "batch, %.1f s" % dt1}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--pool", type=int, default=4)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--path", choices=("fused", "two-call", "both"),
                    default="both",
                    help="which way of running a round to time (the fused "
                         "one is the headline when timed)")
    ap.add_argument("--no-snapshot", action="store_true")
    ap.add_argument("--no-tree", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the window-length sweep")
    ap.add_argument("--no-kda", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 1-lane, ragged 8-lane and 12-lane chains")
    ap.add_argument("--no-token-verify", action="store_true")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip reading the clocks under load (profiler runs)")
    ap.add_argument("--no-general", action="store_true",
                    help="skip f32 / long-window / 32-node-tree shapes")
    ap.add_argument("--general-only", action="store_true",
                    help="time only the shapes beyond the pages' windows")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the chunked prefill (for profiling)")
    ap.add_argument("--prefill-long-only", action="store_true",
                    help="time only the 260,096-token prefill of 4 heads, in "
                         "segments and as one chain (for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 256 MiB f32 copy kernel (y = x * 1) "
                         "before the timed region, as the reference point "
                         "for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU; --gpus %d is not supported.  The "
              "verify/commit path needs no exchange between GPUs: each GPU "
              "runs its own share of the lanes (or of the value-head pairs) "
              "independently." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gdn_synth as gs
    import commit_gated_delta_amd as gdn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # Everything runs on one stream of default priority other than the
    # default stream, so that timed regions can be captured into HIP graphs.
    torch.cuda.set_stream(torch.cuda.Stream(device=dev))
    if args.calibrate_copy:
        cx = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        cy = torch.empty_like(cx)
        torch.mul(cx, 1.0, out=cy)
        torch.cuda.synchronize()
        del cx, cy
    if args.general_only:
        print(json.dumps({"general_shapes": bench_general_shapes(
            reps=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(reps=args.steps,
                                                   warmup=args.warmup)}),
              flush=True)
        return
    if args.prefill_long_only:
        print(json.dumps({"prefill_long_few_heads": bench_prefill_long(
            reps=args.steps, warmup=args.warmup)}), flush=True)
        return
    shape = gs.WindowShape(NL, N, HV, HK, DK, DV, T)
    dims = gdn.Dims.of(NL, N, HV, HK, DK, DV, T)
    t_lane = np.full(N, T, dtype=np.int32)

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    pool = []
    for p in range(args.pool):
        w = gs.window_inputs(shape, (7, p))
        pool.append((dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                     torch.from_numpy(w.beta).to(dev),
                     torch.from_numpy(w.g).to(dev)))
    S0 = gs.initial_state(shape, (7, 0))
    o = torch.empty((NL, N, T, HV, DV), device=dev)
    nrec = gdn.records_bytes(dims)
    total = args.warmup + args.steps
    m_all = [gs.accepted_uniform(t_lane, (7, 100 + s)) for s in range(total)]
    stream = torch.cuda.current_stream()

    # The K timed steps run back to back as one HIP graph replay between one
    # pair of HIP events (region_ms); per-kernel times come from regions of
    # their own.  The same K steps launched one by one from the host are
    # reported beside it.
    def timed(step):
        return region_ms(step, args.steps, args.warmup, stream)

    upd_per_step = int(t_lane.sum()) * NL * HV
    res = {}
    if args.path in ("two-call", "both"):
        S = torch.from_numpy(S0).to(dev)
        recs = [torch.empty(nrec, dtype=torch.uint8, device=dev)
                for _ in range(2)]

        def step2(s):
            q, k, v, beta, g = pool[s % len(pool)]
            gdn.verify(dims, t_lane, q, k, v, beta, g, S, o, recs[s % 2],
                       stream=stream)
            gdn.commit(dims, m_all[s], t_lane, recs[s % 2], S, stream=stream)

        ms = timed(step2)
        bv = alg_bytes_verify(t_lane)
        bc = float(np.mean([alg_bytes_commit(m_all[args.warmup + s])
                            for s in range(args.steps)]))
        # each kernel back to back in a region of its own: verify leaves S
        # as it is; the commits replay the drawn prefixes of the last two
        # windows' records, each on the state the previous one left.  The
        # records alternate between two buffers (as the inputs rotate over
        # the pool), so that no call rewrites or rereads what the call
        # before it left in the 256 MB Infinity Cache.
        ms_v = region_ms(lambda r: gdn.verify(dims, t_lane, *pool[r % len(pool)],
                                              S, o, recs[r % 2], stream=stream),
                         args.steps, 2, stream)
        ms_c = region_ms(lambda r: gdn.commit(dims, m_all[r % total], t_lane,
                                              recs[r % 2], S, stream=stream),
                         args.steps, 2, stream)
        bc_smp = float(np.mean([alg_bytes_commit(m_all[(2 + r) % total])
                                for r in range(args.steps)]))
        res["two-call"] = {
            "ms_per_step": ms, "updates_per_s": upd_per_step / (ms * 1e-3),
            "hbm_roofline_frac_path": (bv + bc) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "verify_ms": ms_v, "commit_ms": ms_c,
            "verify_alg_GBps": bv / (ms_v * 1e-3) / 1e9,
            "verify_hbm_frac": bv / (ms_v * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "commit_alg_GBps": bc_smp / (ms_c * 1e-3) / 1e9,
            "commit_hbm_frac": bc_smp / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "verify_traffic": measured_traffic("verify_kernel"),
            "commit_traffic": measured_traffic("commit_kernel"),
            "alg_bytes_verify": bv, "alg_bytes_per_step": bv + bc}
        del S, recs
    if args.path in ("fused", "both"):
        S = torch.from_numpy(S0).to(dev)
        recs = [torch.empty(nrec, dtype=torch.uint8, device=dev)
                for _ in range(2)]
        zero = np.zeros(N, dtype=np.int32)

        def m_prev_of(s):
            return zero if s == 0 else m_all[s - 1]

        def stepf(s):
            q, k, v, beta, g = pool[s % len(pool)]
            gdn.commit_verify(dims, m_prev_of(s), t_lane, recs[(s + 1) % 2],
                              t_lane, q, k, v, beta, g, S, o, recs[s % 2],
                              stream=stream)

        ms = timed(stepf)
        ms_f = ms  # one launch per step, back to back
        ms_host = stream_launch_ms(stepf, args.steps, args.warmup, stream)

        def busy():
            for s_ in range(20):
                stepf(args.warmup + s_ % args.steps)
        clocks = None if args.no_clocks else gpu_clocks_under_load(busy)
        mp = [m_prev_of(args.warmup + s) for s in range(args.steps)]
        bf = float(np.mean([alg_bytes_fused(t_lane, m) for m in mp]))

        res["fused"] = {
            "ms_per_step": ms, "updates_per_s": upd_per_step / (ms * 1e-3),
            "hbm_roofline_frac_path": bf / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_ms": ms_f, "kernel_launches_timed": args.steps,
            "alg_GBps": bf / (ms_f * 1e-3) / 1e9,
            "alg_bytes_per_launch_timed": bf,
            "traffic": measured_traffic("fused_kernel"),
            "alg_bytes_per_step": bf, "gpu_clocks_under_load": clocks,
            "host_launched": {
                "ms_per_step": ms_host,
                "updates_per_s": upd_per_step / (ms_host * 1e-3),
                "hbm_roofline_frac_path":
                    bf / (ms_host * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        del S, recs

    head = "fused" if "fused" in res else "two-call"
    h = res[head]
    ms_per_step = h["ms_per_step"]
    if head == "fused":
        roof = {"bound": "hbm",
                "kernel": "gdn_commit_verify (mverify_kernel, replay on)",
                "duration": "timed region / K: the K steps replayed back to "
                            "back from one HIP graph, one launch per step, "
                            "gaps between the launches included",
                "achieved": h["alg_GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": h["alg_GBps"] / HBM_PEAK_GBS,
                "traffic": h["traffic"],
                "alg_bytes_per_launch": h["alg_bytes_per_launch_timed"],
                "avg_launch_ms": h["kernel_ms"],
                "launches_timed": h["kernel_launches_timed"]}
    else:
        roof = {"bound": "hbm", "kernel": "gdn_verify (mverify_kernel)",
                "achieved": h["verify_alg_GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": h["verify_hbm_frac"],
                "traffic": h["verify_traffic"],
                "alg_bytes_per_launch": h["alg_bytes_verify"],
                "avg_launch_ms": h["verify_ms"]}
    out = {
        "metric": METRIC,
        "value": h["updates_per_s"],
        "unit": "head-token updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 state / bf16 q,k,v; state products on bf16 MFMA as "
                 "split-bf16 pairs (hi + lo, ~2^-17 rel.), f32 accumulate",
        "data": "synthetic (seeded gdn_synth inputs; S0 ~ N(0, 0.01))",
        "config": {"workload": "verify+commit round: 8 lanes x 48 layers x "
                               "32 value / 16 key heads, d_k=d_v=128, T=16, "
                               "m ~ U{0..16}, state carried across steps",
                   "n_lanes": N, "n_layers": NL, "h_v": HV, "h_k": HK,
                   "d_k": DK, "d_v": DV, "t": T, "path": head},
        "hbm_roofline_frac_path": h["hbm_roofline_frac_path"],
        "roofline": roof,
        "paths": res,
    }
    samples = []
    if not args.no_configs:
        out["configs"] = {}
        for name, cfg in CHAIN_CONFIGS.items():
            rec, smp = bench_chain(name, cfg)
            out["configs"][name] = rec
            samples.append(smp)
    if not args.no_token_verify:
        out["token_by_token_verify"] = bench_token_verify()
    if not args.no_general:
        out["general_shapes"] = bench_general_shapes()
    if not args.no_prefill:
        out["prefill"] = bench_prefill()
        # the same prefill with 16 key heads (two value heads per key head)
        out["prefill_h_k16"] = bench_prefill(h_k=16, segments=False)
        out["prefill_long_few_heads"] = bench_prefill_long()
        out["prefill_batch_few_heads"] = bench_prefill_long(
            L=131072, n_seqs=2)
    if not args.no_snapshot:
        out["state_snapshot"] = bench_snapshot()
        # context for the roofline: what a plain device copy (read + write,
        # the fused round's own mix of state traffic) reaches on this machine
        cp = out["state_snapshot"]["device_GBps"]
        roof["copy_ceiling"] = {
            "kernel": "gdn_state_snapshot device to device (768 MiB read + "
                      "768 MiB write)",
            "GBps": cp, "frac_of_peak": cp / HBM_PEAK_GBS,
            "achieved_over_copy": roof["achieved"] / cp}
    if not args.no_sweep:
        out["t_sweep"] = bench_t_sweep()
    if not args.no_tree:
        out["draft_tree"] = bench_tree()
    if not args.no_kda:
        out["kda"] = bench_kda()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
        for smp in samples:
            out["configs"][smp["name"]]["parity"] = oracle_chain_parity(smp)
    out["gpu_clocks"] = res.get("fused", {}).get("gpu_clocks_under_load")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
