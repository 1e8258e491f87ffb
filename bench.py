#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--leg all|prefill|varlen|long|verify]

One step = one chunked prefill (gdn_chunk_fwd: intra-chunk preparation,
inter-chunk state recurrence, output) of one GDN layer over T = 4000 tokens,
32 value heads / 16 q-k heads, d = 128, bf16 inputs, fp32 state and output,
zero initial state -- the one-layer, 4000-token workload of the "2080 Ti runs
Qwen3.8-27B: a vLLM plugin" page, section 2.  Inputs are synthetic, seeded
and resident in HBM before timing.

The headline is the COLD step: before each of the K timed steps a 1 GiB fill
(outside the step's event pair) evicts the 256 MB last-level cache and L2, so
every step reads its inputs from HBM; ms_per_step is the mean over the K
steps.  The warm figure (K steps back to back) is reported beside it.

Algorithmic work is the layer's own (per token at these dims): 4,237,995
flop (triangular products at half, the K K^T / Q K^T Grams once per q/k
head) and 33,024 bytes of input and output (q, k, v bf16; g, beta, out fp32),
plus 2 MiB per state read or written.  A kernel's share is the terms it
evaluates and the layer I/O it reads or writes; its intermediates are not
algorithmic bytes (they are reported as measured `traffic`).

Printed as one JSON line:
  value      prefill tokens/s per layer over the K cold steps
  roofline   the dominant prefill kernel: its algorithmic bytes or flops
             (the binding one) per launch / its mean launch time (HIP events
             on the launch stream), vs MI355X peak; traffic = measured HBM
             bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a
             plain copy) while the kernel source matches the profiled one
  prefill    cold and warm step times, %MFMA and %HBM of the layer, stages
  varlen     the 8-sequence packed batch (lengths U{512..4096}, random states)
  long       one 131072-token sequence (slow decay)
  verify     the speculative-verify step (8 requests x 6 tokens, per-token
             state snapshots kept), as a fraction of HBM bandwidth; also over
             an fp16 state pool (verify_fp16_slots) and one-token decode
  prefill_snapshots  the prefill that also writes the state after every chunk
  cpu_baseline  the CPU oracle (fp32 token recurrence) on the host's cores
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2.5e15      # dense fp16/bf16 matrix-core FLOP/s (MI355X)
PEAK_HBM = 8.0e12           # HBM3E bytes/s (MI355X)
PAGES_MS_T4000 = 1.35       # pages' hand-written CUDA kernel, 2x RTX 2080 Ti (context only)
CPU_SHARE_PER_GPU = 16      # host cores one GPU's process may use (the rest serve the node's other GPUs)

H_V, H_QK, D, C = 32, 16, 128, 64
STATE_BYTES = H_V * D * D * 4          # one fp32 state of one sequence (all value heads)


def layer_terms(h_v=H_V, h_qk=H_QK, d=D, c=C):
    """Per-token flops of the layer's terms and per-token bytes of its I/O.

    Flops: the recurrence W H0 and K^T U' (4 d^2 per value head), the output
    Q H0 (2 d^2) and P U' (C d, causal half), W and U (C d each, causal
    half), the triangular solve (C^2 / 3), and per q/k head the Grams K K^T
    and Q K^T (C d each, causal half)."""
    f = {
        "recurrence": h_v * 4 * d * d,
        "out_qh": h_v * 2 * d * d,
        "out_pu": h_v * c * d,
        "w_u": h_v * 2 * c * d,
        "solve": h_v * c * c / 3,
        "gram_kk": h_qk * c * d,
        "gram_qk": h_qk * c * d,
    }
    b = {"q": h_qk * d * 2, "k": h_qk * d * 2, "v": h_v * d * 2, "g": h_v * 4, "beta": h_v * 4,
         "out": h_v * d * 4}
    return f, b


def kernel_work():
    """Which layer terms and which layer I/O each prefill kernel evaluates.

    gdn_chunk_prep: the decay, the Grams K K^T and Q K^T and the UT
    transform (Tm diag(beta)); reads q, k, g, beta.  gdn_chunk_state: W and U
    from Tm diag(beta), the recurrence and the output; reads v, writes the
    output and the final states.  (Prep also pulls v into the last-level
    cache for the state kernel; that read is not counted twice.)"""
    f, b = layer_terms()
    return {
        "gdn_chunk_prep": (f["solve"] + f["gram_kk"] + f["gram_qk"],
                           b["q"] + b["k"] + b["g"] + b["beta"]),
        "gdn_chunk_state": (f["w_u"] + f["recurrence"] + f["out_qh"] + f["out_pu"], b["v"] + b["out"]),
        "layer": (sum(f.values()), sum(b.values())),
    }


# HBM bytes per launch of the prefill kernels at T = 4000, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs of `bench.py --leg prefill` scaled by a plain
# 1 GiB copy; valid only for the kernel sources they were taken with.
CSRC = "hybrid_linear_attention_gdn_amd/csrc/"
MEASURED_TRAFFIC = {
    # FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (KiB per launch, mean over the
    # warm and cold launches of the counter run)
    "gdn_chunk_state": {
        "sources": [CSRC + "gdn_chunk.hip", CSRC + "gdn_device.h", CSRC + "gdn_sizes.h"],
        "sources_sha256_prefix": "3c1739538c3cf403",
        "bytes": (44844 * 2 + 66056) * 1024,
    },
    "gdn_chunk_prep": {
        "sources": [CSRC + "gdn_prep.h", CSRC + "gdn_prep.hip", CSRC + "gdn_device.h", CSRC + "gdn_sizes.h"],
        "sources_sha256_prefix": "e87cb96d2b813a07",
        "bytes": (32679 * 2 + 57456) * 1024,
    },
}


def measured_traffic(kernel: str):
    import hashlib
    rec = MEASURED_TRAFFIC.get(kernel)
    if rec is None:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["sources_sha256_prefix"]:
        return None      # kernel changed since the counters were taken
    return rec["bytes"]


def time_launches(fn, n, torch):
    """Mean time per launch of fn() over n back-to-back launches (events on the current stream)."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(n):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / n


def time_cold(fn, n, flush, torch):
    """Per-step times of n steps, each after a fill of `flush` that evicts the
    last-level cache and L2 (outside its event pair).  Returns a sorted list (s)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        flush.fill_(float(i))
        ev[i][0].record(s)
        fn()
        ev[i][1].record(s)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / 1e3 for a, b in ev)


def time_graph(fn, n_inner, reps, torch):
    """Mean time per call of fn() replayed from a HIP graph of n_inner calls
    (captured once; the calls allocate nothing and launch on the current
    stream), as a serving loop replays its decode step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_inner):
            fn()
    g.replay()
    torch.cuda.synchronize()
    t = time_launches(g.replay, reps, torch) / n_inner
    del g
    return t


def host_cores() -> int:
    """Cores this process may run on, up to one GPU's share of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, CPU_SHARE_PER_GPU))


def cpu_baseline(x, budget_s: float):
    import oracle
    cores = host_cores()
    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while True:
        oracle.forward_inputs(x, precision="f32", n_threads=cores)
        reps += 1
        t = time.perf_counter() - t0
        if t >= budget_s or reps >= 100000:
            break
    # one thread, a shorter sample of the same runs
    reps1, t1 = 0, 0.0
    t10 = time.perf_counter()
    while t1 < min(3.0, budget_s / 4) or reps1 == 0:
        oracle.forward_inputs(x, precision="f32", n_threads=1)
        reps1 += 1
        t1 = time.perf_counter() - t10
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": x.total_tokens * reps / t, "unit": "tokens/s per layer", "cores": cores,
            "kind": "oracle", "cpu_model": model, "host_cpus": os.cpu_count(),
            "single_thread_value": x.total_tokens * reps1 / t1,
            "sample": f"fp32 token recurrence, {x.name}, all {x.h_v} value heads, {reps} run(s), "
                      f"{t:.1f} s wall, threads over (sequence, value head)"}


class Prefill:
    """Device copies of one prefill workload with its outputs and workspace."""

    def __init__(self, x, torch, gdn, dev):
        bf = torch.bfloat16
        self.x = x
        self.gdn = gdn
        self.q = torch.from_numpy(x.q).to(dev, bf)
        self.k = torch.from_numpy(x.k).to(dev, bf)
        self.v = torch.from_numpy(x.v).to(dev, bf)
        self.g = torch.from_numpy(x.g).to(dev)
        self.beta = torch.from_numpy(x.beta).to(dev)
        self.cu = torch.from_numpy(x.cu_seqlens).to(dev)
        self.s0 = None if x.initial_state is None else torch.from_numpy(x.initial_state).to(dev)
        self.out = torch.empty((x.total_tokens, x.h_v, x.d_v), device=dev)
        self.fin = torch.empty((x.n_seqs, x.h_v, x.d_k, x.d_v), device=dev)
        n = gdn.gdn_chunk_fwd_workspace_size(x.n_seqs, x.total_tokens, x.h_qk, x.h_v)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def step(self):
        self.gdn.gdn_chunk_fwd(self.q, self.k, self.v, self.g, self.beta, self.cu, self.s0,
                               self.out, self.fin, self.ws)

    def stage(self, mask):
        self.gdn.gdn_chunk_fwd_stages(self.q, self.k, self.v, self.g, self.beta, self.cu, self.s0,
                                      self.out, self.fin, self.ws, mask)

    def algorithmic(self):
        """Layer flops and bytes of this batch (states read if given, final states written)."""
        f, b = kernel_work()["layer"]
        T, N = self.x.total_tokens, self.x.n_seqs
        states = N * (2 if self.x.initial_state is not None else 1)
        return f * T, b * T + states * STATE_BYTES


def layer_fractions(flops, nbytes, t):
    return {"pct_mfma_peak": 100 * flops / t / PEAK_MFMA_F16, "pct_hbm_peak": 100 * nbytes / t / PEAK_HBM}


def roofline_of(kernel, flops, nbytes, t):
    """Roofline of one kernel from its algorithmic work and mean launch time:
    the binding roof is the one with the longer ideal time."""
    t_mfma, t_hbm = flops / PEAK_MFMA_F16, nbytes / PEAK_HBM
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": PEAK_MFMA_F16 / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    traffic = measured_traffic(kernel)
    roof.update({
        "traffic": traffic,
        "kernel": kernel,
        "mean_launch_us": t * 1e6,
        "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": nbytes,
        "frac_mfma": t_mfma / t,
        "frac_hbm": t_hbm / t,
        "traffic_over_algorithmic_bytes": None if traffic is None else traffic / nbytes,
    })
    return roof


def prefill_leg(args, torch, gi, gdn, dev, flush):
    p = Prefill(gi.prefill_4000(), torch, gdn, dev)
    T = p.x.total_tokens
    for _ in range(args.warmup):
        p.step()
    torch.cuda.synchronize()

    # Timed region: K cold steps (the headline), then K warm steps back to back.
    cold = time_cold(p.step, args.steps, flush, torch)
    t_cold = sum(cold) / len(cold)
    t_warm = time_launches(p.step, args.steps, torch)

    # Per-kernel durations: K warm steps launched stage by stage with HIP
    # events between the kernels, on the launch stream (upper bounds: the
    # events add a few microseconds of gap per kernel).
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(s)
        p.stage(1)
        ev[i][1].record(s)
        p.stage(2)
        ev[i][2].record(s)
    torch.cuda.synchronize()
    stage_t = {
        "gdn_chunk_prep": sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3 / args.steps,
        "gdn_chunk_state": sum(e[1].elapsed_time(e[2]) for e in ev) / 1e3 / args.steps,
    }
    p.step()
    torch.cuda.synchronize()

    work = kernel_work()
    per_launch = {
        "gdn_chunk_prep": (work["gdn_chunk_prep"][0] * T, work["gdn_chunk_prep"][1] * T),
        "gdn_chunk_state": (work["gdn_chunk_state"][0] * T, work["gdn_chunk_state"][1] * T + STATE_BYTES),
    }
    dom = max(stage_t, key=stage_t.get)
    roof = roofline_of(dom, *per_launch[dom], stage_t[dom])
    flops, nbytes = p.algorithmic()
    prefill = {
        "workload": p.x.name,
        "ms_per_layer_cold": t_cold * 1e3,
        "ms_per_layer_cold_p10_p50_p90": [cold[min(len(cold) - 1, int(q * len(cold)))] * 1e3 for q in (0.1, 0.5, 0.9)],
        "ms_per_layer_warm": t_warm * 1e3,
        "tokens_per_s_warm": T / t_warm,
        "algorithmic_flops": flops,
        "algorithmic_bytes": nbytes,
        "cold": layer_fractions(flops, nbytes, t_cold),
        "warm": layer_fractions(flops, nbytes, t_warm),
        "stage_us_warm": {n: t * 1e6 for n, t in stage_t.items()},
        "stage_roofline": {n: {k: v for k, v in roofline_of(n, *per_launch[n], stage_t[n]).items()
                               if k in ("bound", "frac", "frac_mfma", "frac_hbm", "traffic")}
                           for n in stage_t},
    }

    # The same prefill writing the state after every chunk (a prefix cache's
    # snapshots): 63 chunk states of 32 heads x 64 KB at T = 4000.
    n_snap = gdn.gdn_chunk_state_slots(1, T, H_QK, H_V)
    chunk_states = torch.empty((n_snap, H_V, D, D), dtype=torch.float32, device=dev)

    def snap_step():
        gdn.gdn_chunk_fwd_snapshots(p.q, p.k, p.v, p.g, p.beta, p.cu, None, p.out, p.fin, chunk_states, p.ws)

    for _ in range(min(args.warmup, 100)):
        snap_step()
    t_snap = time_launches(snap_step, args.steps, torch)
    del chunk_states
    snap_bytes = ((T + C - 1) // C) * STATE_BYTES
    snapshots = {
        "workload": p.x.name + "_chunk_snapshots",
        "us_per_step_warm": t_snap * 1e6,
        "tokens_per_s": T / t_snap,
        "snapshot_bytes": snap_bytes,
        "pct_hbm_peak": 100 * (nbytes + snap_bytes) / t_snap / PEAK_HBM,
        "us_over_prefill_warm": (t_snap - t_warm) * 1e6,
    }
    return p, t_cold, roof, prefill, snapshots


def batch_leg(x, runs, torch, gdn, dev, flush):
    """A bigger prefill batch, timed cold (median of `runs` steps after a cache flush)."""
    p = Prefill(x, torch, gdn, dev)
    p.step()
    p.step()
    torch.cuda.synchronize()
    cold = time_cold(p.step, runs, flush, torch)
    t = cold[len(cold) // 2]
    flops, nbytes = p.algorithmic()
    res = {"workload": x.name, "n_seqs": x.n_seqs, "tokens": x.total_tokens,
           "lengths": [int(n) for n in x.lengths][:16], "ms_cold_median": t * 1e3,
           "tokens_per_s": x.total_tokens / t, **layer_fractions(flops, nbytes, t),
           "algorithmic_flops": flops, "algorithmic_bytes": nbytes}
    del p
    torch.cuda.empty_cache()
    return res


def verify_legs(args, torch, gi, gdn, dev):
    y = gi.verify_8x6()
    bf = torch.bfloat16
    R, n_tok = 8, 6
    vq = torch.from_numpy(y.q).to(dev, bf)
    vk = torch.from_numpy(y.k).to(dev, bf)
    vv = torch.from_numpy(y.v).to(dev, bf)
    vg = torch.from_numpy(y.g).to(dev)
    vb = torch.from_numpy(y.beta).to(dev)
    s_in = torch.from_numpy(y.initial_state).to(dev)
    vout = torch.empty((R * n_tok, H_V, D), device=dev)
    inter = torch.empty((R, n_tok, H_V, D, D), device=dev)
    tok_b = 2 * H_QK * D * 2 + H_V * D * 2 + 2 * H_V * 4 + H_V * D * 4

    def vstep():
        gdn.gdn_recurrent_step(vq, vk, vv, vg, vb, R, n_tok, s_in, None, vout, inter, True)

    for _ in range(args.warmup):
        vstep()
    t_verify = time_launches(vstep, args.steps, torch)
    t_verify_graph = time_graph(vstep, 20, max(1, args.steps // 20), torch)
    v_bytes = R * STATE_BYTES + R * n_tok * STATE_BYTES + R * n_tok * tok_b
    verify = {
        "workload": y.name,
        "us_per_step": t_verify * 1e6,
        "tokens_per_s": R * n_tok / t_verify,
        "algorithmic_bytes": v_bytes,
        "achieved_GBps": v_bytes / t_verify / 1e9,
        "pct_hbm_peak": 100 * v_bytes / t_verify / PEAK_HBM,
        "us_per_step_graph": t_verify_graph * 1e6,
        "pct_hbm_peak_graph": 100 * v_bytes / t_verify_graph / PEAK_HBM,
    }
    if args.leg == "verify":
        return verify, None, None

    # the same verify over an fp16 slot pool (state slots picked by a
    # device-side table, as a serving loop with rollback runs it)
    pool16 = torch.from_numpy(gi.state_pool(y, R * n_tok, f16=True)).to(dev)
    table = torch.from_numpy(gi.slot_table_contiguous(R, n_tok, R)).to(dev)
    cu_tok = torch.from_numpy(y.cu_seqlens).to(dev)

    def sstep():
        gdn.gdn_recurrent_step_slots(vq, vk, vv, vg, vb, cu_tok, R, n_tok, pool16, table, None, vout)

    for _ in range(args.warmup):
        sstep()
    t_slots = time_launches(sstep, args.steps, torch)
    half = STATE_BYTES // 2
    s_bytes = R * half + R * n_tok * half + R * n_tok * tok_b
    verify_f16 = {
        "workload": y.name + "_fp16_slot_pool",
        "us_per_step": t_slots * 1e6,
        "tokens_per_s": R * n_tok / t_slots,
        "algorithmic_bytes": s_bytes,
        "achieved_GBps": s_bytes / t_slots / 1e9,
        "pct_hbm_peak": 100 * s_bytes / t_slots / PEAK_HBM,
    }

    # decode: the same 8 requests, one token each (the first of each
    # request's verify tokens), state advanced in place
    dq, dk, dv = (t[::n_tok].contiguous() for t in (vq, vk, vv))
    dg, db = vg[::n_tok].contiguous(), vb[::n_tok].contiguous()
    d_state = s_in.clone()
    dout = torch.empty((R, H_V, D), device=dev)

    def dstep():
        gdn.gdn_recurrent_step(dq, dk, dv, dg, db, R, 1, d_state, d_state, dout, None, False)

    for _ in range(args.warmup):
        dstep()
    t_decode = time_launches(dstep, args.steps, torch)
    t_decode_graph = time_graph(dstep, 20, max(1, args.steps // 20), torch)
    # the same step with its arguments checked once (a serving loop that
    # writes each step's tokens into the same buffers)
    dprep = gdn.prepare_recurrent_step(dq, dk, dv, dg, db, R, 1, d_state, d_state, dout, None, False)
    for _ in range(min(args.warmup, 100)):
        dprep()
    t_decode_prep = time_launches(dprep, args.steps, torch)
    d_bytes = 2 * R * STATE_BYTES + R * tok_b
    decode = {
        "workload": "decode_8req_1tok_hv32_hqk16_d128",
        "us_per_step": t_decode * 1e6,
        "tokens_per_s": R / t_decode,
        "algorithmic_bytes": d_bytes,
        "achieved_GBps": d_bytes / t_decode / 1e9,
        "pct_hbm_peak": 100 * d_bytes / t_decode / PEAK_HBM,
        "us_per_step_graph": t_decode_graph * 1e6,
        "pct_hbm_peak_graph": 100 * d_bytes / t_decode_graph / PEAK_HBM,
        "us_per_step_prepared": t_decode_prep * 1e6,
        "pct_hbm_peak_prepared": 100 * d_bytes / t_decode_prep / PEAK_HBM,
    }
    return verify, verify_f16, decode


def long_context(args):
    """The long-context workload (one sequence of 131072 tokens, g = -softplus(N(-2, 1))):
    gdn_chunk_fwd (range by range), the single pass and its two stages, and
    gdn_chunk_fwd_segmented at a few segment lengths, at the configuration's
    32 value / 16 q-k heads and at a two-way head shard (16 / 8)."""
    import torch

    import gdn_inputs as gi
    import hybrid_linear_attention_gdn_amd as gdn

    dev, T = torch.device("cuda:0"), 131072
    reps = max(1, min(args.steps, 5))
    res = {"metric": "long-context prefill ms per layer (T=131072)", "unit": "ms", "shapes": []}
    for hqk, hv in ((16, 32), (8, 16)):
        x = gi.make_inputs([T], hqk, hv, D, D, seed=0, g_mean=-2.0, name=f"long_{T}_hv{hv}_hqk{hqk}")
        p = Prefill(x, torch, gdn, dev)
        row = {"workload": x.name}

        def timed(fn):
            fn()
            fn()
            return time_launches(fn, reps, torch) * 1e3

        # gdn_chunk_fwd runs one long sequence range by range; the stage calls
        # run the single pass (prep over every chunk, then the recurrence)
        row["ms"] = timed(p.step)
        row["single_pass_ms"] = timed(lambda: (p.stage(1), p.stage(2)))
        row["single_pass_prep_ms"] = timed(lambda: p.stage(1))
        row["single_pass_state_ms"] = timed(lambda: p.stage(2))
        del p.ws
        for sc in (1024, 512, 256):
            wss = torch.empty(gdn.gdn_chunk_fwd_segmented_workspace_size(1, T, hqk, hv, sc),
                              dtype=torch.uint8, device=dev)
            row[f"segmented_sc{sc}_ms"] = timed(
                lambda: gdn.gdn_chunk_fwd_segmented(p.q, p.k, p.v, p.g, p.beta, p.cu, None, p.out, p.fin, sc, wss))
            del wss
        row["tokens_per_s"] = T / (row["ms"] * 1e-3)
        res["shapes"].append(row)
        del p
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the CPU-oracle baseline (0 skips it)")
    ap.add_argument("--leg", choices=("all", "prefill", "varlen", "long", "verify"), default="all",
                    help="run one leg only (for counter runs); the JSON line then holds that leg")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device-to-device copies of BYTES bytes (reference for "
                         "the HBM byte counters) and exit")
    ap.add_argument("--long", action="store_true",
                    help="only time the long-context prefill (T=131072): range by range, single pass and segment-parallel "
                         "(gdn_chunk_fwd_segmented) at 32/16 and 16/8 heads, print one JSON line and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X "
              "(heads or sequences would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.long:
        long_context(args)
        return
    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 5}), flush=True)
        return

    import torch

    import gdn_inputs as gi
    import hybrid_linear_attention_gdn_amd as gdn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB

    line = {
        "metric": "GDN prefill tokens/s per layer (T=4000) & %MFMA peak; verify %HBM BW",
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "dtype": "f16",
        "dtype_note": "bf16 inputs widened to fp16 matrix-core operands, fp32 accumulation, state and output",
        "data": "synthetic",
    }
    if args.leg in ("all", "prefill"):
        p, t_cold, roof, prefill, snapshots = prefill_leg(args, torch, gi, gdn, dev, flush)
        T = p.x.total_tokens
        line.update({
            "value": T / t_cold,
            "ms_per_step": t_cold * 1e3,
            "vs_baseline": (T / t_cold) / (4000 / (PAGES_MS_T4000 * 1e-3)),
            "vs_baseline_note": "against the pages' 1.35 ms per 4000-token layer on 2x RTX 2080 Ti "
                                "(TP=2): another machine's figure, context only",
            "config": {"workload": p.x.name, "global_batch": 1, "seq_len": T, "n_heads_v": H_V,
                       "n_heads_qk": H_QK, "d_k": D, "d_v": D, "chunk": C, "initial_state": "zeros (NULL)",
                       "timing": "cold: 1 GiB cache flush before each timed step", "parallelism": "single GPU"},
            "roofline": roof,
            "prefill": prefill,
            "prefill_snapshots": snapshots,
        })
        del p
        torch.cuda.empty_cache()
    if args.leg in ("all", "varlen"):
        line["varlen"] = batch_leg(gi.varlen_8(), max(3, min(args.steps, 20)), torch, gdn, dev, flush)
    if args.leg in ("all", "long"):
        line["long"] = batch_leg(gi.long_131072(), 3, torch, gdn, dev, flush)
    if args.leg in ("all", "verify"):
        verify, verify_f16, decode = verify_legs(args, torch, gi, gdn, dev)
        line["verify"] = verify
        if verify_f16 is not None:
            line["verify_fp16_slots"] = verify_f16
            line["decode"] = decode
    if args.leg == "all" and args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(gi.prefill_4000(), args.cpu_seconds)
    if "value" not in line:      # a single non-prefill leg: its own figure
        leg = next(k for k in ("varlen", "long", "verify") if k in line)
        line["value"] = line[leg]["tokens_per_s"]
        line["ms_per_step"] = line[leg].get("ms_cold_median", line[leg].get("us_per_step", 0) / 1e3)
        line["config"] = {"workload": line[leg]["workload"]}
        line["vs_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
