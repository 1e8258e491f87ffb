#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one chunked prefill (gdn_chunk_fwd: prep, state, out) of one GDN
layer over T = 4000 tokens, 32 value heads / 16 q-k heads, d = 128, bf16
inputs, fp32 state and output, zero initial state -- the one-layer,
4000-token workload of the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page,
section 2.  Inputs are synthetic, seeded and resident in HBM before timing.

Printed as one JSON line:
  value      prefill tokens/s per layer over the K timed steps (warm, back to back)
  roofline   the dominant prefill kernel: algorithmic work per launch / its
             mean launch time (HIP events on the launch stream), vs MI355X peak
  verify     the speculative-verify leg (8 requests x 6 tokens, per-token state
             snapshots kept) timed the same way, as a fraction of HBM bandwidth
  verify_fp16_slots  the same verify over an fp16 state pool addressed through
             a slot table (gdn_recurrent_step_slots)
  decode     the same 8 requests, one token each, state advanced in place
             (verify and decode also replayed from a HIP graph of 20 calls:
             *_graph, the launch cost a serving loop does not pay per step)
  prefill_snapshots  the prefill that also writes the fp32 state after every
             64-token chunk (gdn_chunk_fwd_snapshots, for a prefix cache), as
             a fraction of HBM bandwidth on its bytes
  cpu_baseline  the CPU oracle (fp32 token recurrence) on host cores
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

H_V, H_QK, D, C = 32, 16, 128, 64


def algorithmic_work():
    """Per-token algorithmic flops and bytes of each prefill kernel (config dims).

    Flops count each causal (triangular) product at half and the K K^T / Q K^T
    Grams once per q/k head; they are the layer's terms, each assigned to the
    kernel that evaluates it: prep takes the decay, Grams, UT transform, W and
    U; the state kernel the recurrence (W H, K^T U') and the output (Q S and
    P U').  Bytes count each tensor of a kernel's interface read or written
    once: bf16 inputs, fp32 g / beta / decay vectors / output, fp16
    intermediates (-W, U and the six nonzero 16x32 blocks of P per value head,
    K^T and Q fragments per q/k head)."""
    prep_f = H_V * (C * (D + D) + C * C / 3) + H_QK * (C * D) + H_QK * (C * D)
    state_f = H_V * (4 * D * D) + H_V * (2 * D * D) + H_V * (C * D)
    qk_b = H_QK * D * 2          # one of q or k, bf16
    v_b = H_V * D * 2
    gb_b = H_V * 4               # one of g, beta, or one fp32 value per token and value head
    f16_row = H_V * D * 2        # one of -W, U per token (per value head)
    p_row = H_V * 6 * 16 * 32 * 2 // C   # P's six nonzero blocks per token (per value head)
    qk_row = H_QK * D * 2        # K^T or Q fragments per token (per q/k head)
    out_b = H_V * D * 4
    work = 2 * f16_row + p_row + 2 * qk_row + 2 * gb_b   # the intermediates, each way
    prep_b = 2 * qk_b + v_b + 2 * gb_b + work
    state_b = work + out_b
    return {
        "prep": (prep_f, prep_b),
        "state": (state_f, state_b),
        "layer": (prep_f + state_f, 2 * qk_b + v_b + 2 * gb_b + out_b),
    }


# HBM bytes per launch of the prefill kernels at T = 4000, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs scaled by a plain 1 GiB copy (fetch x 2.0,
# write x 1.0); valid only for the kernel source they were taken with.
MEASURED_TRAFFIC = {
    "gdn_chunk_prep": {"bytes": 181932334, "source_sha256_prefix": "b52136c7a5260ad0",
                       "source": "hybrid_linear_attention_gdn_amd/csrc/gdn_prep.h"},
    "gdn_chunk_state": {"bytes": 180855143, "source_sha256_prefix": "efb32dfe6c1d428a",
                        "source": "hybrid_linear_attention_gdn_amd/csrc/gdn_chunk.hip"},
}


def measured_traffic(kernel: str):
    import hashlib
    rec = MEASURED_TRAFFIC.get(kernel)
    if rec is None:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != rec["source_sha256_prefix"]:
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


def cpu_baseline(x, budget_s: float):
    import oracle
    cores = min(16, os.cpu_count() or 1)
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


def long_context(args):
    """The long-context workload (one sequence of 131072 tokens, g = -softplus(N(-2, 1))):
    gdn_chunk_fwd against gdn_chunk_fwd_segmented at a few segment lengths, at the
    configuration's 32 value / 16 q-k heads and at a two-way head shard (16 / 8)."""
    import torch

    import gdn_inputs as gi
    import hybrid_linear_attention_gdn_amd as gdn

    dev, bf, T = torch.device("cuda:0"), torch.bfloat16, 131072
    reps = max(1, min(args.steps, 5))
    res = {"metric": "long-context prefill ms per layer (T=131072)", "unit": "ms", "shapes": []}
    for hqk, hv in ((16, 32), (8, 16)):
        x = gi.make_inputs([T], hqk, hv, D, D, seed=0, g_mean=-2.0, name=f"long_{T}_hv{hv}_hqk{hqk}")
        q = torch.from_numpy(x.q).to(dev, bf)
        k = torch.from_numpy(x.k).to(dev, bf)
        v = torch.from_numpy(x.v).to(dev, bf)
        g = torch.from_numpy(x.g).to(dev)
        beta = torch.from_numpy(x.beta).to(dev)
        cu = torch.from_numpy(x.cu_seqlens).to(dev)
        out = torch.empty((T, hv, D), device=dev)
        fin = torch.empty((1, hv, D, D), device=dev)
        ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(1, T, hqk, hv), dtype=torch.uint8, device=dev)
        row = {"workload": x.name}

        def timed(fn):
            fn()
            return time_launches(fn, reps, torch) * 1e3

        row["serial_ms"] = timed(lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, cu, None, out, fin, ws))
        row["serial_prep_ms"] = timed(lambda: gdn.gdn_chunk_fwd_stages(q, k, v, g, beta, cu, None, out, fin, ws, 1))
        row["serial_state_ms"] = timed(lambda: gdn.gdn_chunk_fwd_stages(q, k, v, g, beta, cu, None, out, fin, ws, 2))
        del ws
        for sc in (1024, 512, 256):
            wss = torch.empty(gdn.gdn_chunk_fwd_segmented_workspace_size(1, T, hqk, hv, sc),
                              dtype=torch.uint8, device=dev)
            row[f"segmented_sc{sc}_ms"] = timed(
                lambda: gdn.gdn_chunk_fwd_segmented(q, k, v, g, beta, cu, None, out, fin, sc, wss))
            del wss
        row["tokens_per_s_serial"] = T / (row["serial_ms"] * 1e-3)
        res["shapes"].append(row)
        del q, k, v, out
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the CPU-oracle baseline (0 skips it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device-to-device copies of BYTES bytes (reference for "
                         "the HBM byte counters) and exit")
    ap.add_argument("--long", action="store_true",
                    help="only time the long-context prefill (T=131072) serially and segment-parallel "
                         "(gdn_chunk_fwd_segmented) at 32/16 and 16/8 heads, print one JSON line and exit")
    args = ap.parse_args()
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

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer's path runs on a single MI355X "
              "(heads or sequences would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gdn_inputs as gi
    import hybrid_linear_attention_gdn_amd as gdn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16

    # ---------------- prefill workload (resident in HBM)
    x = gi.prefill_4000()
    T = x.total_tokens
    q = torch.from_numpy(x.q).to(dev, bf)
    k = torch.from_numpy(x.k).to(dev, bf)
    v = torch.from_numpy(x.v).to(dev, bf)
    g = torch.from_numpy(x.g).to(dev)
    beta = torch.from_numpy(x.beta).to(dev)
    cu = torch.from_numpy(x.cu_seqlens).to(dev)
    out = torch.empty((T, H_V, D), device=dev)
    fin = torch.empty((1, H_V, D, D), device=dev)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(1, T, H_QK, H_V), dtype=torch.uint8, device=dev)

    def step():
        gdn.gdn_chunk_fwd(q, k, v, g, beta, cu, None, out, fin, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps back to back on the current stream.
    t_step = time_launches(step, args.steps, torch)

    # The same K steps again with HIP events between the two kernels of each
    # step (launched stage by stage), for each kernel's mean duration.  The
    # events add a few microseconds of gap per kernel, so these durations are
    # upper bounds of the kernel times.
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(s)
    for i in range(args.steps):
        ev[i][0].record(s)
        gdn.gdn_chunk_fwd_stages(q, k, v, g, beta, cu, None, out, fin, ws, 1)
        ev[i][1].record(s)
        gdn.gdn_chunk_fwd_stages(q, k, v, g, beta, cu, None, out, fin, ws, 2)
        ev[i][2].record(s)
    e_end.record(s)
    torch.cuda.synchronize()
    t_step_evented = e_start.elapsed_time(e_end) / 1e3 / args.steps
    stage_t = {
        "prep": sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3 / args.steps,
        "state": sum(e[1].elapsed_time(e[2]) for e in ev) / 1e3 / args.steps,
    }
    # spread of single steps (the evented pass: event to event, so each
    # includes the gaps the events add)
    per_step = sorted(e[0].elapsed_time(e[2]) * 1e3 for e in ev)
    spread = {f"p{q}": per_step[min(len(per_step) - 1, int(q / 100 * len(per_step)))] for q in (10, 50, 90)}
    step()
    torch.cuda.synchronize()

    # Cold steps: a 1 GiB fill between steps (outside the timed interval)
    # evicts the 256 MB last-level cache and L2, so each timed step reads its
    # inputs and intermediates from HBM.  Reported beside the warm figure.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    n_cold = min(args.steps, 20)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_cold)]
    for i in range(n_cold):
        flush.fill_(float(i))
        cold_ev[i][0].record(s)
        step()
        cold_ev[i][1].record(s)
    torch.cuda.synchronize()
    t_cold = sorted(e[0].elapsed_time(e[1]) for e in cold_ev)[n_cold // 2] / 1e3
    del flush

    # The same prefill writing the state after every chunk (a prefix cache's
    # snapshots): 63 chunk states of 32 heads x 64 KB at T = 4000.
    n_snap = gdn.gdn_chunk_state_slots(1, T, H_QK, H_V)
    chunk_states = torch.empty((n_snap, H_V, D, D), dtype=torch.float32, device=dev)

    def snap_step():
        gdn.gdn_chunk_fwd_snapshots(q, k, v, g, beta, cu, None, out, fin, chunk_states, ws)

    for _ in range(args.warmup):
        snap_step()
    t_snap = time_launches(snap_step, args.steps, torch)
    del chunk_states

    work = algorithmic_work()
    state_bytes = H_V * D * D * 4          # one fp32 state per sequence (final state written)
    per_seq = {"prep": 0, "state": state_bytes, "layer": state_bytes}
    dom = max(stage_t, key=stage_t.get)
    f_tok, b_tok = work[dom]
    flops, nbytes = f_tok * T, b_tok * T + per_seq[dom]
    t_dom = stage_t[dom]
    if flops / PEAK_MFMA_F16 >= nbytes / PEAK_HBM:
        roof = {"bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": PEAK_MFMA_F16 / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / t_dom / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = f"gdn_chunk_{dom}"
    roof["traffic"] = measured_traffic(roof["kernel"])
    roof["mean_launch_us"] = t_dom * 1e6
    roof["algorithmic_flops_per_launch"] = flops
    roof["algorithmic_bytes_per_launch"] = nbytes

    f_layer, b_layer = work["layer"]
    prefill = {
        "ms_per_layer": t_step * 1e3,
        "ms_per_layer_with_events": t_step_evented * 1e3,
        "ms_per_layer_cold_median": t_cold * 1e3,
        "us_per_step_evented_p10_p50_p90": [spread["p10"], spread["p50"], spread["p90"]],
        "pct_mfma_peak": 100 * f_layer * T / t_step / PEAK_MFMA_F16,
        "pct_hbm_peak": 100 * (b_layer * T + per_seq["layer"]) / t_step / PEAK_HBM,
        "algorithmic_flops": f_layer * T,
        "algorithmic_bytes": b_layer * T + per_seq["layer"],
        "stage_us": {n: t * 1e6 for n, t in stage_t.items()},
        "stage_pct_of_roofline": {
            n: 100 * max(work[n][0] * T / PEAK_MFMA_F16, (work[n][1] * T + per_seq[n]) / PEAK_HBM) / stage_t[n]
            for n in stage_t},
    }

    snap_bytes = ((T + C - 1) // C) * state_bytes
    snap_total = work["layer"][1] * T + per_seq["layer"] + snap_bytes
    prefill_snapshots = {
        "workload": x.name + "_chunk_snapshots",
        "us_per_step": t_snap * 1e6,
        "tokens_per_s": T / t_snap,
        "snapshot_bytes": snap_bytes,
        "algorithmic_bytes": snap_total,
        "pct_hbm_peak": 100 * snap_total / t_snap / PEAK_HBM,
        "us_over_prefill": (t_snap - t_step) * 1e6,
    }

    # ---------------- verify workload: 8 requests x (1 + 5) tokens, snapshots kept
    y = gi.verify_8x6()
    R, n_tok = 8, 6
    vq = torch.from_numpy(y.q).to(dev, bf)
    vk = torch.from_numpy(y.k).to(dev, bf)
    vv = torch.from_numpy(y.v).to(dev, bf)
    vg = torch.from_numpy(y.g).to(dev)
    vb = torch.from_numpy(y.beta).to(dev)
    s_in = torch.from_numpy(y.initial_state).to(dev)
    vout = torch.empty((R * n_tok, H_V, D), device=dev)
    inter = torch.empty((R, n_tok, H_V, D, D), device=dev)

    def vstep():
        gdn.gdn_recurrent_step(vq, vk, vv, vg, vb, R, n_tok, s_in, None, vout, inter, True)

    for _ in range(args.warmup):
        vstep()
    t_verify = time_launches(vstep, args.steps, torch)
    t_verify_graph = time_graph(vstep, 20, max(1, args.steps // 20), torch)
    state_b = H_V * D * D * 4
    v_bytes = R * state_b + R * n_tok * state_b + R * n_tok * (2 * H_QK * D * 2 + H_V * D * 2 + 2 * H_V * 4 + H_V * D * 4)
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

    # ---------------- the same verify over an fp16 slot pool (state slots picked by
    #                  a device-side table, as a serving loop with rollback runs it)
    pool16 = torch.from_numpy(gi.state_pool(y, R * n_tok, f16=True)).to(dev)
    table = torch.from_numpy(gi.slot_table_contiguous(R, n_tok, R)).to(dev)
    cu_tok = torch.from_numpy(y.cu_seqlens).to(dev)

    def sstep():
        gdn.gdn_recurrent_step_slots(vq, vk, vv, vg, vb, cu_tok, R, n_tok, pool16, table, None, vout)

    for _ in range(args.warmup):
        sstep()
    t_slots = time_launches(sstep, args.steps, torch)
    state_h = H_V * D * D * 2
    s_bytes = R * state_h + R * n_tok * state_h + R * n_tok * (2 * H_QK * D * 2 + H_V * D * 2 + 2 * H_V * 4 + H_V * D * 4)
    verify_f16 = {
        "workload": y.name + "_fp16_slot_pool",
        "us_per_step": t_slots * 1e6,
        "tokens_per_s": R * n_tok / t_slots,
        "algorithmic_bytes": s_bytes,
        "achieved_GBps": s_bytes / t_slots / 1e9,
        "pct_hbm_peak": 100 * s_bytes / t_slots / PEAK_HBM,
    }

    # ---------------- decode: the same 8 requests, one token each (the first of
    #                  each request's verify tokens), state advanced in place
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
    d_bytes = 2 * R * state_b + R * (2 * H_QK * D * 2 + H_V * D * 2 + 2 * H_V * 4 + H_V * D * 4)
    decode = {
        "workload": "decode_8req_1tok_hv32_hqk16_d128",
        "us_per_step": t_decode * 1e6,
        "tokens_per_s": R / t_decode,
        "algorithmic_bytes": d_bytes,
        "achieved_GBps": d_bytes / t_decode / 1e9,
        "pct_hbm_peak": 100 * d_bytes / t_decode / PEAK_HBM,
        "us_per_step_graph": t_decode_graph * 1e6,
        "pct_hbm_peak_graph": 100 * d_bytes / t_decode_graph / PEAK_HBM,
    }

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(x, args.cpu_seconds)

    value = T / t_step
    line = {
        "metric": "GDN prefill tokens/s per layer (T=4000) & %MFMA peak; verify %HBM BW",
        "value": value,
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": value / (4000 / (PAGES_MS_T4000 * 1e-3)),
        "vs_baseline_note": "pages' 1.35 ms per 4000-token layer on 2x RTX 2080 Ti (TP=2); context, not a target",
        "dtype": "f16",
        "dtype_note": "bf16 inputs widened to fp16 matrix-core operands, fp32 accumulation, state and output",
        "data": "synthetic",
        "config": {"workload": x.name, "global_batch": 1, "seq_len": T, "n_heads_v": H_V,
                   "n_heads_qk": H_QK, "d_k": D, "d_v": D, "chunk": C, "initial_state": "zeros (NULL)",
                   "parallelism": "single GPU"},
        "prefill": prefill,
        "roofline": roof,
        "verify": verify,
        "verify_fp16_slots": verify_f16,
        "decode": decode,
        "prefill_snapshots": prefill_snapshots,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
