#!/usr/bin/env python3
"""Benchmark of the ReplaySSM decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]

Workload (one "step" = one decode token for every slot through every stacked
SSM layer, i.e. one pass of the hot path): 4B-class hybrid-model SSM layers,
batch 256, 4 stacked layers, 96 heads, head dim 64, state dim 128, 8 B/C
groups, fp32 checkpoint, bf16 x/B/C/dt inputs, 16-token interval; inputs for
every timed step are resident in HBM before timing starts; every 16th step
rewrites the checkpoints (fused commit), and those steps are inside the timed
region.

Prints ONE JSON line.  `value` = decode tokens/s (batch * steps / wall time of
the stacked-layer loop, HIP events on the launch stream).  `roofline` rates
the replay step kernel: algorithmic bytes per launch (byte model below) over
its average launch duration, measured with per-launch HIP events in a second
pass.  Extras: the conventional recurrent baseline on the same inputs, a
batch sweep (1, 512), the 120B-class shape, and speculative verify + accept
vs. the per-draft-copy baseline.  `cpu_baseline` times the fp64 oracle on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


# ----------------------------------------------------------------------------
# Algorithmic byte model (per slot per layer per token), see the kernel docs.
# ----------------------------------------------------------------------------
def replay_bytes_per_token(H, G, P=64, N=128, L=16, in_bytes=2, state_bytes=4):
    """Unique HBM bytes one decode token moves through one layer for one slot
    on the replay path, averaged over an interval of L steps:
      checkpoint read every step, rewritten once per interval (1/L);
      current x, B, C, dt read; x, B, dt appended (not on the commit step);
      buffer read: k entries at position k, k = 0..L-1 -> (L-1)/2 on average;
      y written (fp32)."""
    state = H * P * N * state_bytes
    entry = (H * P + G * N + H) * in_bytes          # one buffered token
    cur = (H * P + 2 * G * N + H) * in_bytes
    y = H * P * 4
    return state + state / L + cur + entry * (L - 1) / L + entry * (L - 1) / 2 + y


def replay_step_bytes(H, G, k, L, P=64, N=128, in_bytes=2, state_bytes=4):
    """Bytes one slot moves through one layer in a step taken at buffer
    position k (0..L-1): checkpoint read; the checkpoint rewritten when the
    step closes the interval (k = L-1), else the token appended; current
    x, B, C, dt read; k buffered entries read; y written."""
    state = H * P * N * state_bytes
    entry = (H * P + G * N + H) * in_bytes
    cur = (H * P + 2 * G * N + H) * in_bytes
    return state + (state if k == L - 1 else entry) + cur + k * entry + H * P * 4


def replay_window_bytes(H, G, L, pos0, steps, **kw):
    """Bytes of `steps` consecutive steps of one slot and layer starting at
    buffer position pos0 (lock-step phases: every commit that happens in
    the window is counted, none that does not)."""
    return sum(replay_step_bytes(H, G, (pos0 + i) % L, L, **kw) for i in range(steps))


def split_bytes_per_token(fmt, H, G, P=64, N=128, L=16, in_bytes=2):
    """Replay step with a low-precision state (same buffer/input/output terms
    as the fp32 replay): every step reads the output source; once per
    interval the commit reads the update source and writes it (and the FP4
    copy).  Bytes per element: bf16 2, E4M3 1, FP4 copy 0.5 + 1/32 scale."""
    fp4 = 0.5 + 1.0 / 32
    src = {"split-bf16": (fp4, 2, 2 + fp4), "split-e4m3": (fp4, 1, 1 + fp4),
           "shared-fp4": (fp4, fp4, fp4), "low-bf16": (2, 0, 2), "low-e4m3": (1, 0, 1)}[fmt]
    out_read, upd_read, commit_write = src
    elems = H * P * N
    entry = (H * P + G * N + H) * in_bytes
    cur = (H * P + 2 * G * N + H) * in_bytes
    return (elems * (out_read + (upd_read + commit_write) / L) + cur + entry * (L - 1) / L
            + entry * (L - 1) / 2 + H * P * 4)


def verify_bytes_per_slot(H, G, T, k, P=64, N=128, in_bytes=2, state_bytes=4):
    """One verify of T draft positions for one slot in one layer at buffer
    position k: checkpoint read once; the T drafts' x, B, C, dt read; their
    x, B, dt appended at entries k..k+T-1; the k buffered entries read; T
    outputs written (fp32).  No state is written."""
    entry = (H * P + G * N + H) * in_bytes
    cur = (H * P + 2 * G * N + H) * in_bytes
    return H * P * N * state_bytes + T * (cur + entry + H * P * 4) + k * entry


def recurrent_bytes_per_token(H, G, P=64, N=128, in_bytes=2, state_bytes=4):
    """Conventional step: state read + written every token, inputs read, y written."""
    return 2 * H * P * N * state_bytes + (H * P + 2 * G * N + H) * in_bytes + H * P * 4


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats of the headline window (median)")
    ap.add_argument("--cpu-steps", type=int, default=64)
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="write the counter summary from two rocprofv3 --pmc runs of --probe")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "OUT_MD", "RUN"),
                    help="write the kernel-trace summary of a rocprofv3 --kernel-trace --stats run "
                         "(RUN: 'headline' or 'all')")
    ap.add_argument("--probe-verify", action="store_true",
                    help="short fixed run for profiler counters of the verify kernel: the speculative "
                         "layer (batch 512, 128 heads, 5 positions) after 3 eager rounds, 16 verify "
                         "launches, then 3 plain 1 GiB device copies (calibration)")
    ap.add_argument("--summarize-verify-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="write the verify kernel's counter summary from two --probe-verify runs")
    ap.add_argument("--probe-kernels", action="store_true",
                    help="short fixed run for profiler counters of the other kernels: each precision-split "
                         "format (one 4B-class layer, batch 256, 32 steps), a prompt prefill (batch 256, 256 "
                         "tokens), 8 speculative rounds with deferred and 8 with eager accepts (batch 512, 5 "
                         "positions), then 3 plain 1 GiB device copies (calibration)")
    ap.add_argument("--summarize-kernels", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD", "EXTRA_CSV"),
                    help="write the per-kernel counter summary from two --probe-kernels runs (FETCH_SIZE, "
                         "WRITE_SIZE) and a third run's counters ('-' for none)")
    ap.add_argument("--probe", action="store_true",
                    help="short fixed run for profiler counters: 16 warm-up + 16 replay steps, "
                         "16 recurrent steps, then 3 plain 1 GiB device copies (calibration)")
    args = ap.parse_args()

    if args.summarize_trace:
        stats, out_md, run = args.summarize_trace
        if run == "headline":
            summarize_trace(stats, out_md,
                            command="rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/trace -o trace -- "
                                    "python -u bench.py --steps 64 --no-extras --no-cpu-baseline",
                            title="Kernel trace: replay step vs recurrent step, 4B-class layers, batch 256",
                            workload="batch 256, 4 stacked SSM layers, H=96, G=8, P=64, N=128, L=16, fp32 "
                                     "checkpoint, bf16 inputs; 16 warm-up + 64 timed + 64 per-launch-timed "
                                     "steps per path, x 4 layers (plus the HBM probe launches).")
        else:
            summarize_trace(stats, out_md,
                            command="rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/trace_all -o trace -- "
                                    "python -u bench.py --steps 64 --no-cpu-baseline",
                            title="Kernel trace: every benchmarked path",
                            workload="4B-class layers at batch 256 (64 timed steps), 1 and 512; 120B-class "
                                     "(batch 256, 8 layers, 128 heads); lock-step and staggered interval "
                                     "phases; the interval sweep L = 4..64; speculative verify + accept "
                                     "(batch 512, 4 drafts; eager and deferred commits) and its per-draft-copy "
                                     "baseline; prompt prefill (one 4B-class layer, batch 256, 256 tokens) "
                                     "against token-by-token decode; the precision split formats (batch 256, "
                                     "4 layers; lock-step and staggered phases) and their drift runs.  Kernel names carry <input type, max "
                                     "buffer entries, ...> template arguments; split modes 0..4 = split-bf16, "
                                     "split-e4m3, shared-fp4, low-bf16, low-e4m3.")
        return
    if args.summarize_verify_counters:
        cmd = ("rocprofv3 --pmc COUNTER -f csv -d gpurun_out/pmc_verify_COUNTER -o pmc -- "
               "python -u bench.py --probe-verify")
        summarize_verify_counters(*args.summarize_verify_counters, command=cmd)
        return
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels)
        return
    if args.summarize_counters:
        cmd = ("rocprofv3 --pmc COUNTER -f csv -d gpurun_out/pmc_COUNTER -o pmc -- "
               "python -u bench.py --probe")
        summarize_counters(*args.summarize_counters, command=cmd)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the ReplaySSM decode step "
              "has no cross-GPU exchange; every GPU would run its own slots (or head groups) "
              "independently. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import state_space_recurrence_amd as rs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    L = rs.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    w = synth.WORKLOADS["4b"]

    # ------------------------------------------------------------------ setup
    def make_layers(w, batch, nsteps, max_draft=1, tokens=None):
        layers = []
        for l in range(w.layers):
            A, D = synth.layer_params(w, l, device=dev)
            S0 = synth.init_state(w, l, device=dev, batch=batch)
            ins = synth.token_inputs(w, l, nsteps, device=dev, batch=batch, tokens=tokens)
            ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval,
                               max_draft=max_draft, in_dtype=ins[0].dtype, device=dev, layer_id=l)
            rs.load_checkpoint(ls, S0)
            layers.append({"ls": ls, "S0": S0, "A": ls.A, "D": ls.D, "in": ins,
                           "desc": ls.desc(), "st": ls.cstate()})
        torch.cuda.synchronize()
        return layers

    def replay_loop(layers, t0, n, y, events=None):
        """n decode steps starting at input index t0 (cyclic)."""
        for i in range(n):
            for li, lay in enumerate(layers):
                x, Bm, Cm, dt = lay["in"]
                t = (t0 + i) % x.shape[0]
                if events is not None:
                    events.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                    events[-1][0].record(stream)
                rc = L.replayssm_step(ctypes.byref(lay["desc"]), ctypes.byref(lay["st"]),
                                      x[t].data_ptr(), Bm[t].data_ptr(), Cm[t].data_ptr(),
                                      dt[t].data_ptr(), y[li].data_ptr(), sh)
                if events is not None:
                    events[-1][1].record(stream)
                if rc:
                    raise RuntimeError(L.replayssm_last_error().decode())

    def recurrent_loop(layers, states, t0, n, y, events=None):
        for i in range(n):
            for li, lay in enumerate(layers):
                x, Bm, Cm, dt = lay["in"]
                t = (t0 + i) % x.shape[0]
                if events is not None:
                    events.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                    events[-1][0].record(stream)
                rc = L.replayssm_recurrent_step(ctypes.byref(lay["desc"]), states[li].data_ptr(),
                                                x[t].data_ptr(), Bm[t].data_ptr(), Cm[t].data_ptr(),
                                                dt[t].data_ptr(), lay["A"].data_ptr(), lay["D"].data_ptr(),
                                                y[li].data_ptr(), sh)
                if events is not None:
                    events[-1][1].record(stream)
                if rc:
                    raise RuntimeError(L.replayssm_last_error().decode())

    def timed(fn, *a):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3   # seconds

    def per_launch_us(events):
        torch.cuda.synchronize()
        d = [a.elapsed_time(b) * 1e3 for a, b in events]
        return sum(d) / len(d)

    def graph_timing(layers, w, y, t0, reps=16):
        """Launch-bound small batches: one interval (L steps x layers) captured
        in a HIP graph and replayed, so host launch cost leaves the timing."""
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            with torch.cuda.graph(g, stream=s2):
                for i in range(w.interval):
                    for li, lay in enumerate(layers):
                        x, Bm, Cm, dt = lay["in"]
                        t = (t0 + i) % x.shape[0]
                        rs.step(lay["ls"], x[t], Bm[t], Cm[t], dt[t], y=y[li])
        torch.cuda.current_stream().wait_stream(s2)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * w.interval)
        return {"graph_us_per_step": us, "graph_tokens_per_s": y[0].shape[0] / us * 1e6}

    def median(v):
        v = sorted(v)
        return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])

    def run_standard(w, batch, steps, warmup, with_recurrent=True, per_launch=True, repeats=1):
        """Replay (and recurrent) decode of `steps` steps after `warmup`
        untimed ones, timed `repeats` times back to back (median)."""
        n_in = min(steps + warmup, 64) if batch <= 32 else steps + warmup
        layers = make_layers(w, batch, n_in)
        y = [torch.empty(batch, w.heads, 64, device=dev) for _ in layers]
        replay_loop(layers, 0, warmup, y)
        pos0 = layers[0]["ls"].pos.cpu()
        assert bool((pos0 == pos0[0]).all()), "lock-step phases expected"
        pos0 = int(pos0[0])
        secs = [timed(replay_loop, layers, warmup + r * steps, steps, y) for r in range(repeats)]
        sec = median(secs)
        # bytes of the window from the positions it actually covered (the
        # commits inside it), identical for every repeat when steps % L == 0
        wb = replay_window_bytes(w.heads, w.groups, w.interval, pos0, steps) * batch * w.layers
        out = {"batch": batch, "layers": w.layers, "heads": w.heads, "groups": w.groups,
               "steps": steps, "repeats": repeats, "window_start_pos": pos0,
               "window_commits_per_slot_layer": sum(1 for i in range(steps) if (pos0 + i) % w.interval
                                                    == w.interval - 1),
               "replay_ms_per_step": sec / steps * 1e3,
               # the timed region holds nothing but back-to-back step launches
               "replay_launch_avg_us": sec / (steps * w.layers) * 1e6,
               "replay_ms_per_step_repeats": [round(x / steps * 1e3, 4) for x in secs],
               "replay_tokens_per_s": batch * steps / sec,
               "replay_window_GB": wb / 1e9, "replay_window_GBps": wb / sec / 1e9}
        if per_launch:
            ev = []
            replay_loop(layers, warmup + steps, 4 * w.interval, y, ev)
            out["replay_kernel_avg_us"] = per_launch_us(ev)
        if with_recurrent:
            states = [lay["S0"].clone() for lay in layers]
            recurrent_loop(layers, states, 0, warmup, y)
            rsec = median([timed(recurrent_loop, layers, states, warmup + r * steps, steps, y)
                           for r in range(repeats)])
            out["recurrent_ms_per_step"] = rsec / steps * 1e3
            out["recurrent_tokens_per_s"] = batch * steps / rsec
            out["replay_speedup_vs_recurrent"] = rsec / sec
            if per_launch:
                ev = []
                recurrent_loop(layers, states, warmup + steps, 4 * w.interval, y, ev)
                out["recurrent_kernel_avg_us"] = per_launch_us(ev)
        if batch <= 8:
            out.update(graph_timing(layers, w, y, warmup))
        rb = replay_bytes_per_token(w.heads, w.groups, L=w.interval)
        cb = recurrent_bytes_per_token(w.heads, w.groups)
        out["replay_bytes_per_token_layer"] = rb
        out["recurrent_bytes_per_token_layer"] = cb
        out["replay_GBps_stack"] = out["replay_window_GBps"]
        del layers
        torch.cuda.empty_cache()
        return out

    def run_stagger(w, batch, steps=128):
        """Lock-step phases (every slot commits on the same step) against
        staggered phases (slots admitted one interval position apart, so
        1/L of them commit on each step): tokens/s and the spread of the
        per-step time over the stacked layers."""
        out = {}
        for mode in ("lockstep", "staggered"):
            layers = make_layers(w, batch, steps + w.interval)
            y = [torch.empty(batch, w.heads, 64, device=dev) for _ in layers]
            if mode == "staggered":   # slot b joins at step b % L: pos ends at (L - b % L) % L
                for i in range(w.interval):
                    idx = torch.tensor([b for b in range(batch) if b % w.interval <= i], dtype=torch.int32,
                                       device=dev)
                    n = idx.numel()
                    for li, lay in enumerate(layers):
                        x, Bm, Cm, dt = lay["in"]
                        rs.step(lay["ls"], x[i, :n], Bm[i, :n], Cm[i, :n], dt[i, :n], y=y[li][:n], slots=idx)
            else:
                replay_loop(layers, 0, w.interval, y)
            ev = []
            replay_loop(layers, w.interval, steps, y, ev)
            torch.cuda.synchronize()
            per_launch = [a.elapsed_time(b) * 1e3 for a, b in ev]
            per_step = [sum(per_launch[i:i + w.layers]) for i in range(0, len(per_launch), w.layers)]
            per_step.sort()
            sec = timed(replay_loop, layers, w.interval, steps, y)
            out[mode] = {"tokens_per_s": batch * steps / sec, "step_us_min": per_step[0],
                         "step_us_median": per_step[len(per_step) // 2], "step_us_max": per_step[-1],
                         "pos_distinct": int(layers[0]["ls"].pos.unique().numel())}
            del layers
            torch.cuda.empty_cache()
        log(f"[bench] phases (4b, batch {batch}): lock-step {out['lockstep']['tokens_per_s']:.0f} tok/s, step "
            f"{out['lockstep']['step_us_median']:.0f}/{out['lockstep']['step_us_max']:.0f} us median/max; "
            f"staggered {out['staggered']['tokens_per_s']:.0f} tok/s, step "
            f"{out['staggered']['step_us_median']:.0f}/{out['staggered']['step_us_max']:.0f} us")
        return out

    if args.probe_verify:
        probe_verify(rs, L, torch, synth, dev, stream, sh, log)
        return
    if args.probe_kernels:
        probe_kernels(rs, torch, synth, dev, log)
        return
    if args.probe:
        layers = make_layers(w, args.batch, 32)
        y = [torch.empty(args.batch, w.heads, 64, device=dev) for _ in layers]
        replay_loop(layers, 0, 32, y)
        states = [lay["S0"].clone() for lay in layers]
        recurrent_loop(layers, states, 0, 16, y)
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] probe done: 32 replay steps, 16 recurrent steps, 3 x 1 GiB copies")
        return

    # ------------------------------------------------- practical HBM ceilings
    def hbm_ceilings(nbytes=4 << 30, reps=5):
        """Practical HBM rates: plain read and copy streams (8 loads in flight
        per thread) and a read in the step kernel's shape (one 32 KB block per
        wave, 16 loads in flight per lane); best over grid sizes."""
        src = torch.ones(nbytes // 4, device=dev)
        dst = torch.empty_like(src)
        best = {"read": 0.0, "copy": 0.0, "head_read": 0.0}
        for grid in (1024, 2048, 4096, 8192):
            for mode, name in ((0, "read"), (1, "copy"), (2, "head_read")):
                rs.hbm_probe(mode, src, dst, grid)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    rs.hbm_probe(mode, src, dst, grid)
                e1.record(stream)
                torch.cuda.synchronize()
                gbps = (2 * nbytes if mode == 1 else nbytes) * reps / (e0.elapsed_time(e1) * 1e6)
                best[name] = max(best[name], gbps)
        del src, dst
        torch.cuda.empty_cache()
        return {"read_GBps": round(max(best["read"], best["head_read"]), 1),
                "plain_read_GBps": round(best["read"], 1), "head_read_GBps": round(best["head_read"], 1),
                "copy_GBps": round(best["copy"], 1),
                "probe": "4 GiB streams, 16-byte non-temporal accesses; read/copy: grid-stride, 8 loads in "
                         "flight per thread; head_read: one 32 KB block per wave, 16 loads in flight per lane; "
                         "best of grids 1024-8192"}

    # -------------------------------------------------------------- headline
    # the timed window covers whole intervals and starts at an interval
    # boundary (lock-step phases), whatever --steps / --warmup say: every
    # window then holds exactly steps / L commits per slot and layer
    Lw = w.interval
    steps_t = max(Lw, -(-args.steps // Lw) * Lw)
    warm_t = max(Lw, -(-args.warmup // Lw) * Lw)
    log(f"[bench] {w.describe()} batch={args.batch} steps={steps_t} (asked {args.steps}) "
        f"warmup={warm_t} (asked {args.warmup}) repeats={args.repeats}")
    main_res = run_standard(w, args.batch, steps_t, warm_t, repeats=max(1, args.repeats))
    log(f"[bench] replay {main_res['replay_tokens_per_s']:.0f} tok/s, "
        f"recurrent {main_res.get('recurrent_tokens_per_s', 0):.0f} tok/s")

    rb = main_res["replay_bytes_per_token_layer"]
    # average launch duration over the timed region (HIP events on the launch
    # stream around steps x layers back-to-back launches of this kernel; the
    # window is whole intervals, so commits are in their true proportion);
    # the per-launch event pairs of a separate pass add ~2 us of event
    # overhead to each launch and are reported beside it
    avg_us = main_res["replay_launch_avg_us"]
    achieved = rb * args.batch / (avg_us * 1e-6) / 1e9
    traffic = _load_traffic()
    roofline = {"bound": "hbm", "kernel": "replay_step_kernel<bf16,16>",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "bytes_per_launch": rb * args.batch, "avg_launch_us": round(avg_us, 2),
                "avg_launch_us_event_pairs": round(main_res["replay_kernel_avg_us"], 2)}

    ceil = hbm_ceilings()
    log(f"[bench] practical HBM ceilings: read {ceil['read_GBps']:.0f} GB/s, copy {ceil['copy_GBps']:.0f} GB/s")
    roofline["practical_ceiling"] = ceil
    # the kernel's bytes at the practical rates: read-only steps at the read
    # ceiling, the commit step's extra state write at the copy ceiling
    wl = synth.WORKLOADS["4b"]
    st_bytes = wl.heads * 64 * 128 * 4 * args.batch
    rest = rb * args.batch - st_bytes - st_bytes / wl.interval
    t_ideal = ((wl.interval - 1) * (st_bytes + rest) / (ceil["read_GBps"] * 1e9)
               + (2 * st_bytes + rest) / (ceil["copy_GBps"] * 1e9)) / wl.interval
    roofline["frac_of_practical"] = round(t_ideal / (avg_us * 1e-6), 4)
    extras = {"recurrent_baseline": {k: main_res[k] for k in main_res if k.startswith("recurrent")},
              "replay_speedup_vs_recurrent": main_res.get("replay_speedup_vs_recurrent")}
    if not args.no_extras:
        for b in (1, 512):
            r = run_standard(w, b, 128 if b == 1 else 256, 16)
            extras[f"4b_batch{b}"] = r
            log(f"[bench] batch {b}: replay {r['replay_tokens_per_s']:.0f} tok/s, "
                f"recurrent {r['recurrent_tokens_per_s']:.0f} tok/s")
        w2 = synth.WORKLOADS["120b"]
        r = run_standard(w2, w2.batch, 128, 16)
        extras["120b_batch256"] = r
        log(f"[bench] 120b: replay {r['replay_tokens_per_s']:.0f} tok/s, "
            f"recurrent {r['recurrent_tokens_per_s']:.0f} tok/s")
        import dataclasses
        sweep = {}
        for Li in (4, 8, 16, 32, 64):
            wl_i = dataclasses.replace(w, interval=Li)
            r = run_standard(wl_i, args.batch, 128, Li, with_recurrent=False, per_launch=False)
            sweep[str(Li)] = {k: r[k] for k in ("replay_tokens_per_s", "replay_ms_per_step",
                                                "replay_bytes_per_token_layer", "replay_GBps_stack")}
        extras["interval_sweep_4b_batch256"] = sweep
        extras["phases_4b_batch256"] = run_stagger(w, args.batch)
        log("[bench] interval sweep (4b, batch 256): " + ", ".join(
            f"L={k}: {v['replay_tokens_per_s']:.0f} tok/s ({v['replay_bytes_per_token_layer'] / 1e6:.3f} MB/token/layer)"
            for k, v in sweep.items()))
        extras["spec_batch512"] = run_spec(rs, L, torch, synth, dev, stream, sh, log)
        extras["prefill_4b"] = run_prefill(rs, L, torch, synth, dev, stream, sh, log)
        extras["split_batch256"] = run_split(rs, L, torch, synth, dev, stream, sh, log)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, synth.WORKLOADS["120b"], args.cpu_steps, log)

    res = {
        "metric": "SSM-layer decode tokens/s @B=256,L=16 + achieved HBM GB/s (% of peak)",
        "value": round(main_res["replay_tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_t,
        "warmup": warm_t,
        "ms_per_step": round(main_res["replay_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; bf16 x/B/C/dt ~ the stated distributions, fp32 checkpoint)",
        "config": {"workload": "4B-class hybrid SSM layers: batch 256, 4 stacked layers, 96 heads, "
                               "P=64, N=128, 8 groups, L=16, fp32 checkpoint, bf16 inputs",
                   "batch": args.batch, "layers": w.layers, "heads": w.heads, "groups": w.groups,
                   "interval": w.interval, "parallelism": "single GPU"},
        "timing": {"protocol": "HIP events on the launch stream around the stacked-layer loop; the window "
                              "is rounded up to whole 16-step intervals and starts at an interval boundary; "
                              f"median of {main_res['repeats']} back-to-back repeats",
                   "steps_asked": args.steps, "warmup_asked": args.warmup,
                   "ms_per_step_repeats": main_res["replay_ms_per_step_repeats"],
                   "window_commits_per_slot_layer": main_res["window_commits_per_slot_layer"],
                   "window_GB": round(main_res["replay_window_GB"], 4)},
        "hbm_GBps_stack": round(main_res["replay_GBps_stack"], 1),
        "hbm_frac_stack": round(main_res["replay_GBps_stack"] / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(res), flush=True)


def run_spec(rs, L, torch, synth, dev, stream, sh, log, rounds=64, warm=8):
    """Speculative verify + accept (replay) vs. per-draft-copy recurrent
    verify + accept, 120B-class shape, batch 512, 4 drafts, 4 layers; the
    same seeded accepted lengths drive both paths."""
    w = synth.WORKLOADS["spec"]
    T = w.drafts + 1
    nin = 16
    nk = synth.n_keep(w, nin, device=dev)
    layers = []
    for l in range(w.layers):
        A, D = synth.layer_params(w, l, device=dev)
        S0 = synth.init_state(w, l, device=dev)
        x, Bm, Cm, dt = synth.token_inputs(w, l, nin, device=dev, tokens=T)
        bt = lambda t: t.transpose(1, 2).contiguous()   # [R,T,B,..] -> [R,B,T,..]
        ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T,
                           in_dtype=x.dtype, device=dev, layer_id=l)
        rs.load_checkpoint(ls, S0)
        ddesc = rs.RssmDesc.from_buffer_copy(ls.desc())
        ddesc.deferred_commit = 1      # same layer, declared for deferred accepts
        layers.append({"ls": ls, "desc": ls.desc(), "ddesc": ddesc, "st": ls.cstate(), "S0": S0,
                       "in": (bt(x), bt(Bm), bt(Cm), bt(dt)), "A": ls.A, "D": ls.D})
    y = torch.empty(w.batch, T, w.heads, 64, device=dev)

    def replay_rounds(r0, n, deferred=False):
        accept = L.replayssm_accept_deferred if deferred else L.replayssm_accept
        for i in range(n):
            r = (r0 + i) % nin
            for lay in layers:
                x, Bm, Cm, dt = lay["in"]
                d = lay["ddesc"] if deferred else lay["desc"]
                rc = L.replayssm_verify(ctypes.byref(d), ctypes.byref(lay["st"]), T,
                                        x[r].data_ptr(), Bm[r].data_ptr(), Cm[r].data_ptr(),
                                        dt[r].data_ptr(), y.data_ptr(), sh)
                rc |= accept(ctypes.byref(d), ctypes.byref(lay["st"]), nk[r].data_ptr(), T, sh)
                if rc:
                    raise RuntimeError(L.replayssm_last_error().decode())

    def t(fn, *a):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    replay_rounds(0, warm)
    sec = t(replay_rounds, warm, rounds)
    kept = float(nk.double().mean()) * w.batch * rounds
    # deferred accept: the commit folds into the next round's verify
    replay_rounds(warm + rounds, warm, True)
    dsec = t(replay_rounds, 2 * warm + rounds, rounds, True)
    out = {"batch": w.batch, "layers": w.layers, "heads": w.heads, "drafts": w.drafts,
           "rounds": rounds, "replay_ms_per_round": sec / rounds * 1e3,
           "replay_kept_tokens_per_s": kept / sec,
           "deferred_ms_per_round": dsec / rounds * 1e3,
           "deferred_kept_tokens_per_s": kept / dsec}
    # verify kernel alone, in the state the rounds left (positions 0..L-1 after
    # eager accepts): repeated verifies of one round's drafts change nothing
    # but re-append the same entries.  Algorithmic bytes from the positions.
    lay0 = layers[0]
    for lay in layers:
        rs.commit(lay["ls"])   # flush what the deferred rounds left; eager rounds from here
    replay_rounds(0, 3)
    ksum = int(lay0["ls"].pos.sum())
    x, Bm, Cm, dt = lay0["in"]

    def verifies(n):
        for _ in range(n):
            rc = L.replayssm_verify(ctypes.byref(lay0["desc"]), ctypes.byref(lay0["st"]), T, x[0].data_ptr(),
                                    Bm[0].data_ptr(), Cm[0].data_ptr(), dt[0].data_ptr(), y.data_ptr(), sh)
            if rc:
                raise RuntimeError(L.replayssm_last_error().decode())

    verifies(8)
    vsec = min(t(verifies, 32) for _ in range(3)) / 32
    vbytes = (w.batch * verify_bytes_per_slot(w.heads, w.groups, T, 0)
              + ksum * (64 * w.heads + 128 * w.groups + w.heads) * 2)
    out["verify_kernel"] = {"us_per_launch": vsec * 1e6, "bytes_per_launch": vbytes,
                            "mean_pos": ksum / w.batch, "GBps": vbytes / vsec / 1e9,
                            "frac_of_peak": vbytes / vsec / 1e9 / HBM_PEAK_GBS,
                            "checkpoint_GBps": w.batch * w.heads * 64 * 128 * 4 / vsec / 1e9}
    log(f"[bench] verify kernel (T={T}, batch {w.batch}, mean pos {ksum / w.batch:.1f}): "
        f"{vsec * 1e6:.1f} us, {vbytes / 1e9:.3f} GB algorithmic = {vbytes / vsec / 1e9:.0f} GB/s "
        f"({vbytes / vsec / 1e9 / HBM_PEAK_GBS:.3f} of peak)")
    # conventional: a pool of T+1 states per slot, one copy written per draft
    pools, sels = [], []
    for lay in layers:
        lay["ls"].ckpt = None
        p = torch.empty(w.batch, T + 1, w.heads, 64, 128, device=dev)
        p[:, 0] = lay["S0"]
        pools.append(p)
        sels.append(torch.zeros(w.batch, dtype=torch.int32, device=dev))
    torch.cuda.empty_cache()

    def rec_rounds(r0, n):
        for i in range(n):
            r = (r0 + i) % nin
            for li, lay in enumerate(layers):
                x, Bm, Cm, dt = lay["in"]
                d = lay["desc"]
                dd = rs.RssmDesc(d.batch, d.n_heads, 64, 128, d.n_groups, 1, T, d.in_dtype, 0, 4, 0, 0, 0)
                rc = L.replayssm_recurrent_verify(ctypes.byref(dd), pools[li].data_ptr(), sels[li].data_ptr(),
                                                  T, x[r].data_ptr(), Bm[r].data_ptr(), Cm[r].data_ptr(),
                                                  dt[r].data_ptr(), lay["A"].data_ptr(), lay["D"].data_ptr(),
                                                  y.data_ptr(), sh)
                rc |= L.replayssm_recurrent_accept(ctypes.byref(dd), sels[li].data_ptr(), nk[r].data_ptr(), T, sh)
                if rc:
                    raise RuntimeError(L.replayssm_last_error().decode())

    rec_rounds(0, warm)
    rsec = t(rec_rounds, warm, rounds)
    out["recurrent_ms_per_round"] = rsec / rounds * 1e3
    out["recurrent_kept_tokens_per_s"] = kept / rsec
    out["replay_speedup_vs_recurrent"] = rsec / sec
    out["deferred_speedup_vs_recurrent"] = rsec / dsec
    log(f"[bench] spec: replay {out['replay_kept_tokens_per_s']:.0f} kept tok/s (deferred commit "
        f"{out['deferred_kept_tokens_per_s']:.0f}), recurrent {out['recurrent_kept_tokens_per_s']:.0f} "
        f"({out['replay_speedup_vs_recurrent']:.2f}x / {out['deferred_speedup_vs_recurrent']:.2f}x)")
    del pools
    torch.cuda.empty_cache()
    # the same rounds on low-precision states (verify reads the output copy,
    # accepts list the committing slots for the commit pass)
    out["split"] = {}
    for fmt in ("split-bf16", "split-e4m3", "shared-fp4"):
        for l, lay in enumerate(layers):
            lay["ls"] = None
            torch.cuda.empty_cache()
            ls = rs.LayerState(w.batch, w.heads, w.groups, lay["A"], lay["D"], interval=w.interval, max_draft=T,
                               in_dtype=lay["in"][0].dtype, device=dev, state_format=fmt, seed=w.seed,
                               layer_id=l)
            rs.load_checkpoint(ls, lay["S0"])
            lay["ls"], lay["desc"], lay["st"] = ls, ls.desc(), ls.cstate()
        replay_rounds(0, warm)
        ssec = t(replay_rounds, warm, rounds)
        for lay in layers:
            rs.check_device_errors(lay["ls"])
        out["split"][fmt] = {"ms_per_round": ssec / rounds * 1e3, "kept_tokens_per_s": kept / ssec,
                             "speedup_vs_fp32_replay": sec / ssec}
        log(f"[bench] spec {fmt}: {kept / ssec:.0f} kept tok/s ({sec / ssec:.2f}x the fp32 state)")
    del layers
    torch.cuda.empty_cache()
    return out


# fp32 FMA throughput of the vector ALUs without packed-fp32 instructions
# (256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz); the kernels are built
# without v_pk_*_f32, whose 2x is therefore out of reach.
VALU_FP32_TFLOPS = 78.6


def run_prefill(rs, L, torch, synth, dev, stream, sh, log, batch=256, Tp=256, reps=3):
    """Prompt prefill on the 4B-class layer shape (one layer): prompt tokens/s
    of replayssm_prefill (outputs of every prompt token + final checkpoint)
    against decoding the same prompt token by token with the replay step and
    with the recurrent step.  Algorithmic flops per token and head: the
    replayed outputs 2PN (S . C_t) and the state update 2PN."""
    w = synth.WORKLOADS["4b"]
    A, D = synth.layer_params(w, 0, device=dev)
    S0 = synth.init_state(w, 0, device=dev, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, Tp, device=dev, batch=batch)
    bt = lambda t: t.transpose(0, 1).contiguous()
    px, pB, pC, pdt = bt(x), bt(Bm), bt(Cm), bt(dt)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=16, in_dtype=x.dtype, device=dev)
    y = torch.empty(batch, Tp, w.heads, 64, device=dev)

    def t_of(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    pf = lambda: rs.prefill(ls, px, pB, pC, pdt, from_zero=True, y=y)
    pf()
    sec = t_of(pf, reps)
    pso = lambda: rs.prefill(ls, px, pB, None, pdt, from_zero=True, outputs=False)
    pso()
    sec_state = t_of(pso, reps)
    yd = torch.empty(batch, w.heads, 64, device=dev)

    def decode():
        rs.load_checkpoint(ls, S0)
        for t in range(Tp):
            rs.step(ls, x[t], Bm[t], Cm[t], dt[t], y=yd)
    decode()
    sec_dec = t_of(decode, 1)
    st = S0.clone()

    def rec():
        for t in range(Tp):
            rs.recurrent_step(st, x[t], Bm[t], Cm[t], dt[t], ls.A, ls.D, groups=w.groups, y=yd)
    rec()
    sec_rec = t_of(rec, 1)
    tok = batch * Tp
    flops = tok * w.heads * 4.0 * 64 * 128
    out = {"batch": batch, "prompt_tokens": Tp, "heads": w.heads, "groups": w.groups,
           "prefill_ms": sec * 1e3, "prefill_tokens_per_s": tok / sec,
           "prefill_state_only_ms": sec_state * 1e3,
           "prefill_TFLOPs": flops / sec / 1e12, "valu_fp32_peak_TFLOPs": VALU_FP32_TFLOPS,
           "prefill_frac_of_valu_peak": flops / sec / 1e12 / VALU_FP32_TFLOPS,
           "decode_replay_ms": sec_dec * 1e3, "decode_recurrent_ms": sec_rec * 1e3,
           "prefill_speedup_vs_replay_decode": sec_dec / sec,
           "prefill_speedup_vs_recurrent_decode": sec_rec / sec}
    log(f"[bench] prefill (4b layer, batch {batch}, {Tp} tokens): {tok / sec:.0f} tok/s, "
        f"{out['prefill_TFLOPs']:.1f} TFLOP/s ({out['prefill_frac_of_valu_peak']:.2f} of fp32 VALU), "
        f"{sec_dec / sec:.1f}x token-by-token replay, {sec_rec / sec:.1f}x recurrent")
    del ls, x, Bm, Cm, dt, px, pB, pC, pdt, y
    torch.cuda.empty_cache()
    return out


def run_split(rs, L, torch, synth, dev, stream, sh, log, steps=256, warm=16, drift_steps=512):
    """Precision split on the 4B-class shape (batch 256, 4 layers, L=16):
    decode tokens/s per state format, and the output drift of each format
    against the fp32-state trajectory on identical inputs (relative L2 norm
    of y over all slots/heads/rows of all layers, per step)."""
    w = synth.WORKLOADS["split"]
    fmts = ["split-bf16", "split-e4m3", "shared-fp4", "low-bf16", "low-e4m3"]
    nin = 64
    ins = [synth.token_inputs(w, l, nin, device=dev) for l in range(w.layers)]
    params = [synth.layer_params(w, l, device=dev) for l in range(w.layers)]
    S0 = [synth.init_state(w, l, device=dev) for l in range(w.layers)]
    seed = 0x5EED

    def make(fmt):
        out = []
        for l in range(w.layers):
            ls = rs.LayerState(w.batch, w.heads, w.groups, *params[l], interval=w.interval,
                               in_dtype=ins[l][0].dtype, device=dev, layer_id=l, seed=seed,
                               state_format=fmt)
            rs.load_checkpoint(ls, S0[l])
            out.append((ls, ls.desc(), ls.cstate()))
        return out

    def loop(layers, t0, n, y):
        for i in range(n):
            t = (t0 + i) % nin
            for li, (ls, d, st) in enumerate(layers):
                x, Bm, Cm, dt = ins[li]
                rc = L.replayssm_step(ctypes.byref(d), ctypes.byref(st), x[t].data_ptr(), Bm[t].data_ptr(),
                                      Cm[t].data_ptr(), dt[t].data_ptr(), y[li].data_ptr(), sh)
                if rc:
                    raise RuntimeError(L.replayssm_last_error().decode())

    out = {"batch": w.batch, "layers": w.layers, "heads": w.heads, "steps": steps}
    ys = [torch.empty(w.batch, w.heads, 64, device=dev) for _ in range(w.layers)]
    for fmt in fmts:
        layers = make(fmt)
        loop(layers, 0, warm, ys)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        loop(layers, warm, steps, ys)
        e1.record(stream)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3
        bpt = split_bytes_per_token(fmt, w.heads, w.groups, L=w.interval)
        out[fmt] = {"tokens_per_s": w.batch * steps / sec, "ms_per_step": sec / steps * 1e3,
                    "bytes_per_token_layer": bpt,
                    "GBps_stack": bpt * w.batch * w.layers * steps / sec / 1e9}
        del layers
        # staggered phases: slot b joins at step b % L (through the slot map),
        # so 1/L of the slots commit on every step instead of all on one
        layers = make(fmt)
        for i in range(w.interval):
            idx = torch.tensor([b for b in range(w.batch) if b % w.interval <= i], dtype=torch.int32, device=dev)
            n = idx.numel()
            for li, (ls, d, st) in enumerate(layers):
                x, Bm, Cm, dt = ins[li]
                rs.step(ls, x[i, :n], Bm[i, :n], Cm[i, :n], dt[i, :n], y=ys[li][:n], slots=idx)
        loop(layers, w.interval, warm, ys)
        torch.cuda.synchronize()
        e0.record(stream)
        loop(layers, w.interval + warm, steps, ys)
        e1.record(stream)
        torch.cuda.synchronize()
        ssec = e0.elapsed_time(e1) / 1e3
        out[fmt]["staggered_tokens_per_s"] = w.batch * steps / ssec
        out[fmt]["staggered_pos_distinct"] = int(layers[0][0].pos.unique().numel())
        log(f"[bench] {fmt}: {out[fmt]['tokens_per_s']:.0f} tok/s ({out[fmt]['GBps_stack']:.0f} GB/s); "
            f"staggered phases {out[fmt]['staggered_tokens_per_s']:.0f} tok/s")
        del layers
    # drift vs the fp32 trajectory, all formats stepped together on the same inputs
    def drift(tag):
        runs = {f: make(f) for f in ["f32"] + fmts}
        yb = {f: [torch.empty(w.batch, w.heads, 64, device=dev) for _ in range(w.layers)] for f in runs}
        curve = {f: [] for f in fmts}
        for t in range(drift_steps):
            for f, layers in runs.items():
                loop(layers, t, 1, yb[f])
            ref = torch.stack(yb["f32"])
            rn = float(ref.norm())
            for f in curve:
                curve[f].append(float((torch.stack(yb[f]) - ref).norm()) / rn)
        out[f"drift_{tag}_last64_mean"] = {f: sum(c[-64:]) / 64 for f, c in curve.items()}
        out[f"drift_{tag}_every64"] = {f: [round(sum(c[i:i + 64]) / 64, 6) for i in range(0, len(c), 64)]
                                      for f, c in curve.items()}
        log(f"[bench] drift {tag} (last 64 steps): "
            + ", ".join(f"{f} {v:.5f}" for f, v in out[f"drift_{tag}_last64_mean"].items()))
        del runs
        torch.cuda.empty_cache()

    drift("workload")
    # Long-memory variant: the same inputs with every A scaled by 1/100, so the
    # state remembers ~30-500 tokens instead of ~1-5 and rounding errors that
    # feed back into updates have time to accumulate.
    params[:] = [(A * 0.01, D) for A, D in params]
    drift("long_memory")
    return out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(w, steps, slots, log, tag):
    """Decode tokens/s of the fp64 oracle over `slots` slots of workload w,
    all its layers, `steps` steps (each layer's inputs generated outside the
    timed region)."""
    import oracle
    import synth
    total = 0.0
    for l in range(w.layers):
        A, D = (oracle._f64(t) for t in synth.layer_params(w, l))
        S = oracle._f64(synth.init_state(w, l, batch=slots))
        ins = [oracle._f64(t) for t in synth.token_inputs(w, l, steps, batch=slots)]
        # the call's fixed cost (copying the state) is timed on zero steps and
        # taken out, so the rate is the per-step work
        t0 = time.perf_counter()
        oracle.recurrent(S, *(t[:0] for t in ins), A, D, w.groups)
        t1 = time.perf_counter()
        oracle.recurrent(S, *ins, A, D, w.groups)
        total += (time.perf_counter() - t1) - (t1 - t0)
        del S, ins
    tok = slots * steps / total
    log(f"[bench] cpu oracle {tag}: {tok:.1f} tok/s on {oracle.num_threads()} threads "
        f"({slots} slots x {w.layers} layers x {steps} steps, {total:.1f}s)")
    return {"tokens_per_s": round(tok, 2), "ms_per_step": round(total / steps * 1e3, 2),
            "threads": oracle.num_threads(), "slots": slots, "layers": w.layers, "heads": w.heads,
            "steps": steps, "seconds": round(total, 2)}


def cpu_baseline(w, w2, steps, log):
    """fp64 oracle (the plain per-token recurrence, OpenMP over slot x head)
    on the host: the full 4B-class and 120B-class batches on all the cores
    the process may use, and a 16-slot sample of each on one core (the cost
    per slot is the same for every slot).  `steps` decode steps per layer."""
    import oracle
    import synth
    # warm the library and its thread pool on a tiny call
    S, x, Bm, Cm, dt = (oracle._f64(t) for t in (synth.init_state(w, 0, batch=1),
                                                 *synth.token_inputs(w, 0, 1, batch=1)))
    A, D = (oracle._f64(t) for t in synth.layer_params(w, 0))
    oracle.recurrent(S, x, Bm, Cm, dt, A, D, w.groups)
    allc = oracle.num_threads()
    res = {"all_cores": {}, "one_core": {}}
    res["all_cores"]["4b"] = _oracle_rate(w, steps, w.batch, log, "4b, all cores")
    res["all_cores"]["120b"] = _oracle_rate(w2, steps, w2.batch, log, "120b, all cores")
    oracle.set_num_threads(1)
    try:
        res["one_core"]["4b"] = _oracle_rate(w, steps, 16, log, "4b, 1 core")
        res["one_core"]["120b"] = _oracle_rate(w2, steps, 16, log, "120b, 1 core")
    finally:
        oracle.set_num_threads(allc)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    head = res["all_cores"]["4b"]
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": head["threads"], "kind": "oracle",
            "sample": f"4B-class workload, all {w.batch} slots x {w.layers} layers x {steps} decode steps "
                      f"(per-step cost is constant), fp64 per-token recurrence, OpenMP over slot x head; "
                      f"1-core figures on 16 slots",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "omp_threads": allc, **res}


TRAFFIC_MD = os.path.join(ROOT, "profiles", "replay_step_4b_b256_counters.md")
KERNEL_SOURCES = ("replay_kernels.hip", "replay_common.h", "device_common.h", "kernels.h")


def _kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "state_space_recurrence_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _load_traffic():
    """HBM bytes per launch of the replay step kernel from the committed
    rocprofv3 counter summary -- only if it was taken on the current kernel
    source (else null)."""
    if not os.path.exists(TRAFFIC_MD):
        return None
    kv = {}
    for line in open(TRAFFIC_MD):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            kv[k.strip("`")] = v.strip().strip("`")
    if kv.get("kernel_source_sha256_16") != _kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_trace(stats_csv: str, out_md: str, command: str, title: str, workload: str) -> None:
    """Kernel-trace summary (rocprofv3 --kernel-trace --stats) of the library's kernels."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (from the repository root):", "", f"    {command}", "",
             f"Workload: {workload}", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        if "rssm" not in n:
            continue
        short = n.split("(anonymous namespace)::")[-1].split("(rssm")[0]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                     f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines.append("")
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


PROBE_VERIFY_ROUNDS = 3


def probe_verify_positions(synth, w):
    """Positions the probe's eager rounds leave (every slot starts at 0; an
    accept that brings the count to L or more commits and resets it)."""
    nk = synth.n_keep(w, PROBE_VERIFY_ROUNDS)
    pos = [0] * w.batch
    for r in range(PROBE_VERIFY_ROUNDS):
        for b in range(w.batch):
            k = pos[b] + int(nk[r, b])
            pos[b] = 0 if k >= w.interval else k
    return pos


def probe_verify(rs, L, torch, synth, dev, stream, sh, log, launches=16):
    """Counter probe of the verify kernel: layer 0 of the speculative
    workload, PROBE_VERIFY_ROUNDS eager rounds (verify + accept), then
    `launches` verifies of one round's drafts on that state (verify writes no
    state, so every launch sees the same positions), then the calibration
    copies."""
    w = synth.WORKLOADS["spec"]
    T = w.drafts + 1
    A, D = synth.layer_params(w, 0, device=dev)
    S0 = synth.init_state(w, 0, device=dev)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, PROBE_VERIFY_ROUNDS, device=dev, tokens=T)
    bt = lambda t: t.transpose(1, 2).contiguous()
    x, Bm, Cm, dt = bt(x), bt(Bm), bt(Cm), bt(dt)
    # drawn on the host (the summary recomputes the positions from the same draws)
    nk = synth.n_keep(w, PROBE_VERIFY_ROUNDS).to(dev)
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T,
                       in_dtype=x.dtype, device=dev)
    rs.load_checkpoint(ls, S0)
    y = torch.empty(w.batch, T, w.heads, 64, device=dev)
    for r in range(PROBE_VERIFY_ROUNDS):
        rs.verify(ls, x[r], Bm[r], Cm[r], dt[r], y=y)
        rs.accept(ls, nk[r], T)
    torch.cuda.synchronize()
    assert ls.pos.cpu().tolist() == probe_verify_positions(synth, w)
    for _ in range(launches):
        rs.verify(ls, x[0], Bm[0], Cm[0], dt[0], y=y)
    rs.check_device_errors(ls)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] verify probe done: {PROBE_VERIFY_ROUNDS} eager rounds, {launches} verifies, 3 x 1 GiB copies")


PROBE_SPLIT_FORMATS = ("split-bf16", "split-e4m3", "shared-fp4", "low-bf16", "low-e4m3")
PROBE_SPLIT_STEPS = 32
PROBE_PREFILL = (256, 256)   # batch, prompt tokens
PROBE_SPEC_ROUNDS = 8


def probe_kernels(rs, torch, synth, dev, log):
    """Counter probe of the kernels other than the fp32 step and verify, each
    in its benchmark shape (see --probe-kernels)."""
    w = synth.WORKLOADS["split"]
    A, D = synth.layer_params(w, 0, device=dev)
    S0 = synth.init_state(w, 0, device=dev)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, PROBE_SPLIT_STEPS, device=dev)
    for fmt in PROBE_SPLIT_FORMATS:
        ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval, in_dtype=x.dtype, device=dev,
                           state_format=fmt, seed=0x5EED)
        rs.load_checkpoint(ls, S0)
        y = torch.empty(w.batch, w.heads, 64, device=dev)
        for t in range(PROBE_SPLIT_STEPS):
            rs.step(ls, x[t], Bm[t], Cm[t], dt[t], y=y)
        rs.check_device_errors(ls)
        del ls
    del x, Bm, Cm, dt
    batch, Tp = PROBE_PREFILL
    w4 = synth.WORKLOADS["4b"]
    A4, D4 = synth.layer_params(w4, 0, device=dev)
    px, pB, pC, pdt = (t.transpose(0, 1).contiguous() for t in synth.token_inputs(w4, 0, Tp, device=dev, batch=batch))
    ls = rs.LayerState(batch, w4.heads, w4.groups, A4, D4, interval=16, in_dtype=px.dtype, device=dev)
    rs.prefill(ls, px, pB, pC, pdt, from_zero=True, y=torch.empty(batch, Tp, w4.heads, 64, device=dev))
    rs.check_device_errors(ls)
    del ls, px, pB, pC, pdt
    ws = synth.WORKLOADS["spec"]
    T = ws.drafts + 1
    A, D = synth.layer_params(ws, 0, device=dev)
    S0 = synth.init_state(ws, 0, device=dev)
    x, Bm, Cm, dt = (t.transpose(1, 2).contiguous()
                     for t in synth.token_inputs(ws, 0, PROBE_SPEC_ROUNDS, device=dev, tokens=T))
    nk = synth.n_keep(ws, PROBE_SPEC_ROUNDS).to(dev)
    y = torch.empty(ws.batch, T, ws.heads, 64, device=dev)
    for deferred in (True, False):
        ls = rs.LayerState(ws.batch, ws.heads, ws.groups, A, D, interval=ws.interval, max_draft=T,
                           in_dtype=x.dtype, device=dev, deferred_commit=deferred)
        rs.load_checkpoint(ls, S0)
        for r in range(PROBE_SPEC_ROUNDS):
            rs.verify(ls, x[r], Bm[r], Cm[r], dt[r], y=y)
            (rs.accept_deferred if deferred else rs.accept)(ls, nk[r], T)
        rs.check_device_errors(ls)
        del ls
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] kernel probe done: {len(PROBE_SPLIT_FORMATS)} split formats x {PROBE_SPLIT_STEPS} steps, "
        f"a prefill, {PROBE_SPEC_ROUNDS} deferred + {PROBE_SPEC_ROUNDS} eager speculative rounds, 3 x 1 GiB copies")


def _kernel_label(name: str) -> str:
    """Short kernel label: the function name with its template arguments."""
    base = name.replace("rssm::(anonymous namespace)::", "").replace("rssm::", "").replace("void ", "")
    return base.split("(")[0].strip()


def summarize_kernels(fetch_csv: str, write_csv: str, out_md: str, extra_csv: str) -> None:
    """Per-kernel counter summary of `bench.py --probe-kernels`: FETCH_SIZE /
    WRITE_SIZE per dispatch scaled by the probe's 1 GiB copies, against the
    algorithmic bytes where the byte model covers the launch; split-step
    launches are split into the interval-closing (commit) launches and the
    others.  A third run's counters (EXTRA_CSV, e.g. VALU activity) are
    averaged per kernel as read."""
    import csv
    import synth
    copy_bytes = float(1 << 30)

    def load(path):
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        return rows

    def calib(rows, counter):
        cp = [r for r in rows if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        big = max(int(r["Grid_Size"]) for r in cp)
        vals = [float(r["Counter_Value"]) for r in cp if int(r["Grid_Size"]) == big][-3:]
        return copy_bytes / (sum(vals) / len(vals) * 1024)

    fr, wr = load(fetch_csv), load(write_csv)
    fcal, wcal = calib(fr, "FETCH_SIZE"), calib(wr, "WRITE_SIZE")
    ours = lambda r: "rssm::" in r["Kernel_Name"]
    fseq = [(_kernel_label(r["Kernel_Name"]), float(r["Counter_Value"]) * 1024 * fcal)
            for r in fr if ours(r) and r["Counter_Name"] == "FETCH_SIZE"]
    wseq = [(_kernel_label(r["Kernel_Name"]), float(r["Counter_Value"]) * 1024 * wcal)
            for r in wr if ours(r) and r["Counter_Name"] == "WRITE_SIZE"]
    assert [k for k, _ in fseq] == [k for k, _ in wseq], "the two runs dispatched different kernel sequences"
    ws = synth.WORKLOADS["split"]
    E = ws.heads * 64 * 128
    groups = {}
    split_i = {}
    for (k, f), (_, wv) in zip(fseq, wseq):
        key = k
        if k.startswith("split_commit_list_kernel"):
            i = split_i.get(k, 0)
            split_i[k] = i + 1
            key = k + (" [commit launches]" if i % ws.interval == ws.interval - 1 else " [empty launches]")
        groups.setdefault(key, []).append((f, wv))
    extra = {}
    if extra_csv != "-":
        by_dispatch = {}
        for r in load(extra_csv):
            if ours(r):
                by_dispatch.setdefault(int(r["Dispatch_Id"]), []).append(r)
        extra_i = {}
        for d in sorted(by_dispatch):
            rs_ = by_dispatch[d]
            k = _kernel_label(rs_[0]["Kernel_Name"])
            if k.startswith("split_commit_list_kernel"):
                i = extra_i.get(k, 0)
                extra_i[k] = i + 1
                k = k + (" [commit launches]" if i % ws.interval == ws.interval - 1 else " [empty launches]")
            for r in rs_:
                extra.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    modes = {0: "split-bf16", 1: "split-e4m3", 2: "shared-fp4", 3: "low-bf16", 4: "low-e4m3"}
    fp4 = 0.5 + 1.0 / 32

    def model(key):
        """Algorithmic bytes of one launch (None where the model does not
        cover it)."""
        if key.startswith("split_step_kernel") or key.startswith("split_commit_list_kernel"):
            mode = int(key.split("<")[1].split(">")[0].split(",")[2])   # <input type, entries, mode, ...>
            fmt = modes[mode]
            # bytes per element: output source read, update source read, state written
            out_r, upd_r, cw = {"split-bf16": (fp4, 2, 2 + fp4), "split-e4m3": (fp4, 1, 1 + fp4),
                                "shared-fp4": (fp4, fp4, fp4), "low-bf16": (2, 2, 2),
                                "low-e4m3": (1, 1, 1)}[fmt]
            L = ws.interval
            entry = (ws.heads * 64 + ws.groups * 128 + ws.heads) * 2
            cur = (ws.heads * 64 + 2 * ws.groups * 128 + ws.heads) * 2
            if key.startswith("split_step_kernel"):   # positions 0..L-1 averaged: read k entries, append one
                b = E * out_r + cur + entry + (L - 1) / 2 * entry + ws.heads * 64 * 4
            elif "[commit launches]" in key:          # every slot: read U and the L entries, write the state
                b = E * (upd_r + cw) + L * entry
            else:
                return None
            return b * ws.batch
        if key.startswith("prefill_kernel"):
            batch, Tp = PROBE_PREFILL
            w4 = synth.WORKLOADS["4b"]
            return batch * (Tp * (w4.heads * 64 + 2 * w4.groups * 128 + w4.heads) * 2 + Tp * w4.heads * 64 * 4
                            + w4.heads * 64 * 128 * 4)
        return None

    lines = ["# HBM traffic counters: precision-split, prefill, fold and commit kernels",
             "",
             "Commands (from the repository root; one counter set per run):",
             "",
             "    rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_k_FETCH_SIZE -o pmc -- python -u bench.py --probe-kernels",
             "    rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_k_WRITE_SIZE -o pmc -- python -u bench.py --probe-kernels",
             ]
    if extra_csv != "-":
        names = sorted({c for _, c in extra})
        lines.append(f"    rocprofv3 --pmc {' '.join(names)} -f csv -d gpurun_out/pmc_k_extra -o pmc -- "
                     "python -u bench.py --probe-kernels")
    lines += ["",
              f"`bench.py --probe-kernels`: each precision-split format on one 4B-class layer (batch {ws.batch}, "
              f"H={ws.heads}, G={ws.groups}, L={ws.interval}, lock-step phases, {PROBE_SPLIT_STEPS} steps: "
              f"{PROBE_SPLIT_STEPS // ws.interval} commit launches each); a prompt prefill (batch {PROBE_PREFILL[0]}, "
              f"{PROBE_PREFILL[1]} tokens, 4B-class heads, from zero, with outputs); {PROBE_SPEC_ROUNDS} speculative "
              "rounds with deferred accepts, then as many with eager accepts (batch 512, H=128, 5 positions); "
              "three 1 GiB copies calibrate the counters.",
              "",
              f"Calibration: FETCH_SIZE x {fcal:.4f}, WRITE_SIZE x {wcal:.4f} (known bytes / counter bytes "
              "of the 1 GiB copy).", "",
              "| kernel | launches | FETCH MB / launch | WRITE MB / launch | algorithmic MB / launch | ratio |",
              "|---|---|---|---|---|---|"]
    for key, v in groups.items():
        f = sum(a for a, _ in v) / len(v)
        wv = sum(b for _, b in v) / len(v)
        m = model(key)
        ms = f"{m / 1e6:.1f}" if m else "-"
        rt = f"{(f + wv) / m:.3f}" if m else "-"
        lines.append(f"| `{key}` | {len(v)} | {f / 1e6:.1f} | {wv / 1e6:.1f} | {ms} | {rt} |")
    if extra:
        names = sorted({c for _, c in extra})
        per_wave = "SQ_WAVES" in names
        lines += ["", "Third run, averaged per launch" + (" (SQ_ counters other than SQ_WAVES per wave)" if per_wave else "")
                  + ":", "", "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
        for k in dict.fromkeys(k for k, _ in extra):
            waves = extra.get((k, "SQ_WAVES"))
            nw = sum(waves) / len(waves) if waves else 0
            cells = []
            for c in names:
                x = extra.get((k, c))
                if not x:
                    cells.append("-")
                    continue
                v = sum(x) / len(x)
                if per_wave and c.startswith("SQ_") and c != "SQ_WAVES" and nw > 0:
                    v /= nw
                cells.append(f"{v:.4g}")
            lines.append(f"| `{k}` | " + " | ".join(cells) + " |")
    lines.append("")
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


def summarize_verify_counters(fetch_csv: str, write_csv: str, out_md: str, command: str,
                              launches: int = 16) -> None:
    """Counter summary of the verify kernel from two `bench.py --probe-verify`
    runs (FETCH_SIZE, then WRITE_SIZE): the last `launches` verify dispatches,
    calibrated by the probe's 1 GiB copies, against the algorithmic bytes of
    those launches (positions recomputed from the seeded accepted lengths)."""
    import csv
    import synth
    copy_bytes = float(1 << 30)

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        cp = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max(int(r["Grid_Size"]) for r in cp)      # the 1 GiB calibration copies (not small runtime copies)
        copies = [float(r["Counter_Value"]) for r in cp if int(r["Grid_Size"]) == big]
        ver = [float(r["Counter_Value"]) for r in rows if "replay_verify_kernel" in r["Kernel_Name"]]
        return copies, ver[-launches:]

    fc, fv = per_kernel(fetch_csv, "FETCH_SIZE")
    wc, wv = per_kernel(write_csv, "WRITE_SIZE")
    avg = lambda v: sum(v) / len(v)
    fcal = copy_bytes / (avg(fc[-3:]) * 1024)
    wcal = copy_bytes / (avg(wc[-3:]) * 1024)
    f_v, w_v = avg(fv) * 1024 * fcal, avg(wv) * 1024 * wcal
    w = synth.WORKLOADS["spec"]
    T = w.drafts + 1
    pos = probe_verify_positions(synth, w)
    entry = (64 * w.heads + 128 * w.groups + w.heads) * 2
    algo = w.batch * verify_bytes_per_slot(w.heads, w.groups, T, 0) + sum(pos) * entry
    algo_w = w.batch * T * ((64 * w.heads + 128 * w.groups + w.heads) * 2 + w.heads * 64 * 4)
    lines = [
        "# HBM traffic counters: speculative verify kernel, 120B-class heads, batch 512, 5 positions",
        "",
        "Commands (from the repository root; one counter per run):",
        "",
        f"    {command.replace('COUNTER', 'FETCH_SIZE')}",
        f"    {command.replace('COUNTER', 'WRITE_SIZE')}",
        "",
        f"`bench.py --probe-verify` runs {PROBE_VERIFY_ROUNDS} eager speculative rounds (verify + accept) on one",
        "layer (batch 512, H=128, G=8, P=64, N=128, L=16, T=5, fp32 checkpoint, bf16 inputs), then",
        f"{launches} verifies of one round's drafts on that state (mean buffer position "
        f"{sum(pos) / w.batch:.2f}), then three plain 1 GiB device copies used as calibration.",
        "",
        "| quantity | FETCH_SIZE | WRITE_SIZE |",
        "|---|---|---|",
        f"| 1 GiB copy, counter KiB per dispatch | {avg(fc[-3:]):.0f} | {avg(wc[-3:]):.0f} |",
        f"| calibration scale (known bytes / counter bytes) | {fcal:.4f} | {wcal:.4f} |",
        f"| verify, scaled MB per launch (avg of {len(fv)}) | {f_v/1e6:.1f} | {w_v/1e6:.1f} |",
        f"| verify, algorithmic MB per launch | {(algo - algo_w)/1e6:.1f} | {algo_w/1e6:.1f} |",
        "",
        f"Verify: measured {(f_v + w_v)/1e6:.1f} MB per launch vs algorithmic {algo/1e6:.1f} MB "
        f"(ratio {(f_v + w_v)/algo:.3f}); no checkpoint bytes are written (WRITE = outputs and buffer "
        "appends).",
        "",
    ]
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


def summarize_counters(fetch_csv: str, write_csv: str, out_md: str, command: str) -> None:
    """Turn two rocprofv3 --pmc runs of `bench.py --probe` (FETCH_SIZE, then
    WRITE_SIZE) into the counter summary: per-dispatch KiB of the replay step
    and recurrent kernels, calibrated by the 1 GiB device copies of the probe
    (scale = known bytes / counter bytes of the copy)."""
    import csv
    copy_bytes = float(1 << 30)

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        rep = [float(r["Counter_Value"]) for r in rows if "replay_step_kernel" in r["Kernel_Name"]]
        rec = [float(r["Counter_Value"]) for r in rows if "recurrent_kernel" in r["Kernel_Name"]]
        return copies, rep, rec

    fc, frep, frec = per_kernel(fetch_csv, "FETCH_SIZE")
    wc, wrep, wrec = per_kernel(write_csv, "WRITE_SIZE")
    # the probe's last three copies are the 1 GiB calibration copies
    fcal = copy_bytes / (sum(fc[-3:]) / 3 * 1024)
    wcal = copy_bytes / (sum(wc[-3:]) / 3 * 1024)
    avg = lambda v: sum(v) / len(v)
    f_rep, w_rep = avg(frep) * 1024 * fcal, avg(wrep) * 1024 * wcal
    f_rec, w_rec = avg(frec) * 1024 * fcal, avg(wrec) * 1024 * wcal
    import synth
    w = synth.WORKLOADS["4b"]
    algo = replay_bytes_per_token(w.heads, w.groups, L=w.interval) * w.batch
    algo_rec = recurrent_bytes_per_token(w.heads, w.groups) * w.batch
    lines = [
        "# HBM traffic counters: replay step vs recurrent step, 4B-class layers, batch 256",
        "",
        "Commands (from the repository root; one counter per run):",
        "",
        f"    {command.replace('COUNTER', 'FETCH_SIZE')}",
        f"    {command.replace('COUNTER', 'WRITE_SIZE')}",
        "",
        "`bench.py --probe` runs 32 replay steps (2 whole intervals, 2 fused commits per layer) and",
        "16 recurrent steps on the 4 stacked layers (batch 256, H=96, G=8, P=64, N=128, L=16, fp32",
        "checkpoint, bf16 inputs), then three plain 1 GiB device copies used as calibration.",
        "",
        "| quantity | FETCH_SIZE | WRITE_SIZE |",
        "|---|---|---|",
        f"| 1 GiB copy, counter KiB per dispatch | {avg(fc[-3:]):.0f} | {avg(wc[-3:]):.0f} |",
        f"| calibration scale (known bytes / counter bytes) | {fcal:.4f} | {wcal:.4f} |",
        f"| replay step, scaled MB per launch (avg of {len(frep)}) | {f_rep/1e6:.1f} | {w_rep/1e6:.1f} |",
        f"| recurrent step, scaled MB per launch (avg of {len(frec)}) | {f_rec/1e6:.1f} | {w_rec/1e6:.1f} |",
        "",
        f"Replay step: measured {(f_rep + w_rep)/1e6:.1f} MB per launch vs algorithmic {algo/1e6:.1f} MB "
        f"(ratio {(f_rep + w_rep)/algo:.3f}).",
        f"Recurrent step: measured {(f_rec + w_rec)/1e6:.1f} MB per launch vs algorithmic {algo_rec/1e6:.1f} MB "
        f"(ratio {(f_rec + w_rec)/algo_rec:.3f}).",
        f"State-transfer bytes per token, recurrent / replay (measured): {(f_rec + w_rec)/(f_rep + w_rep):.3f}.",
        "",
        f"- kernel_source_sha256_16: `{_kernel_source_hash()}`",
        f"- traffic_bytes_per_launch: `{f_rep + w_rep:.0f}`",
        f"- fetch_scale: `{fcal:.4f}`",
        f"- write_scale: `{wcal:.4f}`",
        "",
    ]
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
