#!/usr/bin/env python
"""Benchmark of the Gated DeltaNet mixer core on one MI355X (gfx950).

One step = one pass of the whole hot path over one batch of synthetic
input:
  * a chunked prefill of one sequence, T = 4096 tokens, H_k = 16, H_v = 32,
    d_k = d_v = 128, K = 4, C = 64, bf16 activations and output, zero
    initial state;
  * 100 consecutive decode steps for B = 64 sequences (same heads), bf16
    activations and output, fp32 states updated in place, a distinct input
    set per step.
All inputs are resident in HBM before timing starts.  The prefill call and
the block of decode steps are bracketed with HIP events on the stream they
run on, so the line reports prefill tokens/s (``value``) and the decode-step
latency separately; a second decode measurement rotates four state sets so
that the states do not stay in the 256 MB Infinity Cache.

Beside the step, ``workloads`` reports the other workloads on their own:
the tiny recurrent case (64 single-token steps, H=2, d=32, fp32: us/step),
the packed varlen prefill (8 sequences of U{512..8192} tokens: tokens/s and
its MFMA and HBM fractions) and the long-context hand-off (T=65536 prefill,
then 256 decode steps at B=1: tokens/s and us/step).  ``cpu_baseline``
times the oracle on the step's prefill and decode workloads, on one thread
and on all host threads given to the run.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this build is a
one-GPU build (the sharding design is written up, not launched).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CALIB_BYTES = 1 << 30          # the calibration copy reads and writes 1 GiB
# (the kernels of the measured launches and the local headers they include:
# device helpers, and the constants the kernels are compiled with)
KERNEL_SOURCES = ["gated_deltanet_linear_causal_amd/csrc/decode.hip",
                  "gated_deltanet_linear_causal_amd/csrc/decode_multi.hip",
                  "gated_deltanet_linear_causal_amd/csrc/prefill.hip",
                  "gated_deltanet_linear_causal_amd/csrc/gdn_device.h",
                  "gated_deltanet_linear_causal_amd/csrc/gdn_internal.h"]
DECODE_KERNELS = ("decode_multi_kernel", "decode_kernel")


def decode_bytes(d, batch):
    """Algorithmic HBM bytes of one decode step (per launch): fp32 state and
    conv history read + written, bf16 inputs read, bf16 output written, and
    the fp32 parameters read once."""
    state = batch * d.h_v * d.d_k * d.d_v * 4 * 2
    conv = batch * (d.conv_k - 1) * d.conv_dim * 4 * 2
    inp = batch * (d.conv_dim + d.value_dim + 2 * d.h_v) * 2
    out = batch * d.value_dim * 2
    params = (d.conv_dim * d.conv_k + 2 * d.h_v + d.d_v) * 4
    return state + conv + inp + out + params


def decode_multi_bytes(d, batch, t_new):
    """Algorithmic HBM bytes of one multi-token decode call: the state and
    conv history cross HBM once (read + write) whatever t_new is; inputs and
    outputs scale with the tokens.  With one decay per key channel the gate
    input a and dt_bias carry d_k values per value head."""
    gw = d.gate_width
    state = batch * d.h_v * d.d_k * d.d_v * 4 * 2
    conv = batch * (d.conv_k - 1) * d.conv_dim * 4 * 2
    inp = batch * t_new * (d.conv_dim + d.value_dim + d.h_v + d.h_v * gw) * 2
    out = batch * t_new * d.value_dim * 2
    params = (d.conv_dim * d.conv_k + d.h_v + d.h_v * gw + d.d_v) * 4
    return state + conv + inp + out + params


def prefill_flops(d, T, C=64):
    """Algorithmic flops of the chunked (W/U) form as computed, per call: per
    token and key head the K K^T and Q K^T rows (4 C d_k); per token and
    value head W = T diag(b e^G) K (2 C d_k), U = T diag(b) V and P D
    (2 C d_v each), and W S, Q S and the state update (6 d_k d_v)."""
    per_tok = d.h_k * 4 * C * d.d_k + d.h_v * (2 * C * (2 * d.d_v + d.d_k) + 6 * d.d_k * d.d_v)
    return T * per_tok


def prefill_bytes(d, T, n_seq=1, state_in=False):
    """Algorithmic HBM bytes of one prefill call: bf16 inputs and output,
    each sequence's final fp32 state and conv history written, and its
    initial ones read when the call is given them."""
    io = T * ((d.conv_dim + d.value_dim + 2 * d.h_v) * 2 + d.value_dim * 2)
    states = n_seq * (d.h_v * d.d_k * d.d_v + (d.conv_k - 1) * d.conv_dim) * 4
    return io + states * (2 if state_in else 1)


def sources_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


PREFILL_KERNELS = ("qknorm_kernel", "tri_kernel", "scan_kernel", "norm_kernel")


def _counter_rows(directory):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4   # MI355X


def write_traffic(fetch_dir, write_dir, mfma_dir=None):
    """Summarise two rocprofv3 --pmc runs of `bench.py --calib-copy` (one
    with FETCH_SIZE, one with WRITE_SIZE) into per-launch HBM bytes.  Each
    counter is scaled by what it counts for the calibration copy (the largest
    non-GDN dispatch, 1 GiB read + 1 GiB written; FETCH_SIZE counts half of
    the bytes read on gfx950, WRITE_SIZE all of the bytes written)."""
    out = {"sources_sha": sources_hash(), "kernels": {}, "calibration": {}}
    per = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        sums, counts, calib = {}, {}, 0.0
        for r in _counter_rows(directory):
            if r["Counter_Name"] != counter:
                continue
            name, val = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
            key = next((k for k in PREFILL_KERNELS + DECODE_KERNELS if k in name), None)
            if key is None:
                calib = max(calib, val)
                continue
            sums[key] = sums.get(key, 0.0) + val
            counts[key] = counts.get(key, 0) + 1
        if not 0.25 * CALIB_BYTES < calib < 4.0 * CALIB_BYTES:
            raise SystemExit(f"{counter}: calibration copy counted {calib:.3e} B for {CALIB_BYTES} B")
        scale = CALIB_BYTES / calib
        out["calibration"][counter] = {"copy_bytes": CALIB_BYTES, "counter_bytes": calib, "scale": scale}
        per[counter] = {k: sums[k] / counts[k] * scale for k in sums}
    for k in per["FETCH_SIZE"]:
        f, w = per["FETCH_SIZE"][k], per["WRITE_SIZE"].get(k, 0.0)
        out["kernels"][k] = {"fetch_bytes": round(f), "write_bytes": round(w), "bytes_per_launch": round(f + w)}
    pre = [out["kernels"][k] for k in PREFILL_KERNELS if k in out["kernels"]]
    out["kernels"]["prefill_call"] = {"bytes_per_launch": sum(e["bytes_per_launch"] for e in pre)}
    if mfma_dir:
        # MFMA-busy fraction: SQ_VALU_MFMA_BUSY_CYCLES over every matrix pipe
        # (CUs x SIMDs) for the kernel's duration (GRBM_GUI_ACTIVE sums the
        # XCDs).
        acc = {}
        for r in _counter_rows(mfma_dir):
            key = next((k for k in PREFILL_KERNELS + DECODE_KERNELS if k in r["Kernel_Name"]), None)
            if key is None:
                continue
            e = acc.setdefault(key, {})
            e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        busy_all = gui_all = 0.0
        for k, e in acc.items():
            busy = sum(e.get("SQ_VALU_MFMA_BUSY_CYCLES", [0.0])) / max(1, len(e.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])))
            gui = sum(e.get("GRBM_GUI_ACTIVE", [0.0])) / max(1, len(e.get("GRBM_GUI_ACTIVE", [0])))
            pipes = gui / N_XCD * N_CU * SIMD_PER_CU
            if k in out["kernels"] and pipes > 0:
                out["kernels"][k]["mfma_busy"] = round(busy / pipes, 4)
            if k in PREFILL_KERNELS:
                busy_all += busy
                gui_all += gui
        if gui_all > 0:
            out["kernels"]["prefill_call"]["mfma_busy"] = round(busy_all / (gui_all / N_XCD * N_CU * SIMD_PER_CU), 4)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def load_counter(kernel, field):
    """A per-kernel field of profiles/traffic_counters.json, or None if the
    counters were taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha") != sources_hash():
        return None
    return rec.get("kernels", {}).get(kernel, {}).get(field)


def load_traffic(kernel):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counter
    runs (scaled by a plain-copy calibration), or None if they were taken on
    other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha") != sources_hash():
        return None
    ent = rec.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pf_case, dc_case, threads, reps=3):
    """The oracle, untuned, on the host cores, on the two workloads of the
    step: the T=4096 prefill over every head, and the B=64 x 100 decode
    steps (run as 64 sequences of 100 tokens: the oracle steps token by
    token either way).  Each is timed on one thread (one run) and on
    `threads` threads (median of `reps`), after an untimed warm-up call."""
    import statistics

    import oracle
    shape = oracle.Shape(pf_case.dims.h_k, pf_case.dims.h_v, pf_case.dims.d_k, pf_case.dims.d_v,
                         pf_case.dims.conv_k, pf_case.dims.gate)
    B, steps = dc_case.dec["qkv"].shape[1], dc_case.dec["qkv"].shape[0]

    def pack(x):
        return x.transpose(0, 1).reshape(B * steps, -1)
    dcu = [i * steps for i in range(B + 1)]
    runs = {
        "prefill": (lambda nt: oracle.mixer(shape, pf_case.cu_seqlens, pf_case.params, pf_case.qkv,
                                            pf_case.z, pf_case.a, pf_case.b, pf_case.S0,
                                            pf_case.conv0, nthreads=nt), pf_case.t_total),
        "decode": (lambda nt: oracle.mixer(shape, dcu, dc_case.params, pack(dc_case.dec["qkv"]),
                                           pack(dc_case.dec["z"]), pack(dc_case.dec["a"]),
                                           pack(dc_case.dec["b"]), dc_case.S0, dc_case.conv0,
                                           nthreads=nt), B * steps),
    }
    oracle.mixer(shape, [0, 1], pf_case.params, pf_case.qkv[:1], pf_case.z[:1], pf_case.a[:1],
                 pf_case.b[:1], pf_case.S0, pf_case.conv0, nthreads=threads)
    legs = {}
    for name, (fn, tokens) in runs.items():
        for nt, n in ((1, 1), (threads, reps)):
            times = []
            for _ in range(n):
                t = time.perf_counter()
                fn(nt)
                times.append(time.perf_counter() - t)
            dt = statistics.median(times)
            legs[f"{name}_{nt}t"] = {"tokens_per_s": round(tokens / dt, 1), "seconds": round(dt, 3),
                                     "threads": nt, "runs": n}
    dec_all = legs[f"decode_{threads}t"]
    return {"value": legs[f"prefill_{threads}t"]["tokens_per_s"], "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the full T={pf_case.t_total} prefill (all {pf_case.dims.h_v} value heads) "
                      f"and the B={B} x {steps}-step decode, float64 token-by-token C oracle; "
                      f"value = prefill on {threads} threads (median of {reps}); decode on "
                      f"{threads} threads: {dec_all['tokens_per_s']} tokens/s = "
                      f"{round(dec_all['seconds'] / steps * 1e6, 1)} us per B={B} step",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(), "legs": legs}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the multi-token decode legs (profiling runs: every "
                         "decode_multi_kernel launch is then a gdn_decode_step)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the tiny-recurrent, varlen and T=65536 hand-off legs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs into "
                         "profiles/traffic_counters.json and exit")
    ap.add_argument("--mfma-dir", help="with --write-traffic: a rocprofv3 run with "
                    "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, mfma_dir=args.mfma_dir)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_deltanet_linear_causal_amd as gdn
    from gdn_inputs import BIG, chunked_prefill, decode_batch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    d = BIG
    cfg = gdn.Config(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k, torch.bfloat16, torch.bfloat16)

    # ---- inputs, resident in HBM ----------------------------------------
    pf = chunked_prefill()
    dc = decode_batch(steps=100)
    bf = torch.bfloat16
    params = {k: v.to(dev) for k, v in pf.params.items()}
    dparams = {k: v.to(dev) for k, v in dc.params.items()}
    seq = gdn.SeqLens(pf.cu_seqlens, dev)
    x_pf = [getattr(pf, k).to(bf).to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
    T = pf.t_total
    out_pf = torch.empty((T, d.value_dim), dtype=bf, device=dev)
    S_pf = torch.empty((1, d.h_v, d.d_k, d.d_v), dtype=torch.float32, device=dev)
    c_pf = torch.empty((1, d.conv_k - 1, d.conv_dim), dtype=torch.float32, device=dev)
    ws = gdn.alloc_workspace(cfg, 1, T, dev)
    B = dc.dec["qkv"].shape[1]
    x_dc = [dc.dec[k].to(bf).to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
    S_dc = dc.S0.to(dev)
    c_dc = dc.conv0.to(dev)
    out_dc = torch.empty((B, d.value_dim), dtype=bf, device=dev)
    n_sets = x_dc[0].shape[0]

    def step(i, evs=None):
        if evs is not None:
            evs[0].record(stream)
        gdn.prefill_chunked(cfg, params, seq, *x_pf, state_in=None, state_out=S_pf,
                            conv_in=None, conv_out=c_pf, out=out_pf, workspace=ws,
                            stream=stream)
        if evs is not None:
            evs[1].record(stream)
        for j in range(n_sets):
            gdn.decode_step(cfg, dparams, x_dc[0][j], x_dc[1][j], x_dc[2][j], x_dc[3][j], c_dc,
                            S_dc, out=out_dc, stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(args.warmup):
        step(i)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pf_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    dc_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps / n_sets
    ms_step = wall * 1e3 / args.steps

    # Decode with the Infinity Cache cold for the states: four state sets
    # (4 x 134 MiB, more than the 256 MB cache) used in rotation, as in a
    # model whose other layers evict a layer's state between its steps.  Timed
    # with the state cache hint for that case (streamed: non-temporal state
    # loads and stores) and, for comparison, with the default (cached).
    rot = 4
    S_rot = [S_dc.clone() for _ in range(rot)]
    c_rot = [c_dc.clone() for _ in range(rot)]
    cold_steps = 2 * n_sets

    def cold_leg(c):
        for j in range(rot):
            gdn.decode_step(c, dparams, x_dc[0][j], x_dc[1][j], x_dc[2][j], x_dc[3][j], c_rot[j],
                            S_rot[j], out=out_dc, stream=stream)
        ev_c = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev_c[0].record(stream)
        for j in range(cold_steps):
            k = j % n_sets
            gdn.decode_step(c, dparams, x_dc[0][k], x_dc[1][k], x_dc[2][k], x_dc[3][k],
                            c_rot[j % rot], S_rot[j % rot], out=out_dc, stream=stream)
        ev_c[1].record(stream)
        torch.cuda.synchronize()
        return ev_c[0].elapsed_time(ev_c[1]) / cold_steps

    cfg_stream = dataclasses.replace(cfg, state_cache="streamed")
    dc_cold_ms = cold_leg(cfg_stream)
    dc_cold_cached_ms = cold_leg(cfg)
    del S_rot, c_rot

    def time_calls(fn, calls, warm=2):
        for _ in range(warm):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(calls):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / calls

    def time_graph(fn, replays=5):
        """Device time of fn's launches: fn captured once into a HIP graph
        (its launches go to the capture stream), then replayed; ms per
        replay.  Launch-bound steps measured eagerly include the host's
        launch overhead, which this leaves out."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(replays):
            g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / replays

    work = {}
    if not args.no_workloads:
        from gdn_inputs import long_handoff, tiny_recurrent, varlen_prefill
        # Tiny recurrent workload: 1 sequence, 64 tokens one at a time
        # through gdn_decode_step, H=2, d=32, fp32 (launch-latency bound).
        tc = tiny_recurrent()
        td = tc.dims
        tcfg = gdn.Config(td.h_k, td.h_v, td.d_k, td.d_v, td.conv_k, torch.float32,
                          torch.float32)
        tp = {k: v.to(dev) for k, v in tc.params.items()}
        tx = [tc.dec[k].to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
        tS, tC = tc.S0.to(dev), tc.conv0.to(dev)
        tout = torch.empty((1, td.value_dim), dtype=torch.float32, device=dev)
        nst = tx[0].shape[0]

        def tiny_run(st=None):
            for j in range(nst):
                gdn.decode_step(tcfg, tp, tx[0][j], tx[1][j], tx[2][j], tx[3][j], tC, tS,
                                out=tout, stream=st)
        work["tiny"] = (time_calls(lambda: tiny_run(stream), 20) / nst,
                        time_graph(tiny_run) / nst, nst, td)

        # Varlen packed prefill: 8 sequences of U{512..8192} tokens, random
        # initial states and histories.
        vc = varlen_prefill()
        vx = [getattr(vc, k).to(bf).to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
        vseq = gdn.SeqLens(vc.cu_seqlens, dev)
        vS0, vC0 = vc.S0.to(dev), vc.conv0.to(dev)
        vS, vC = torch.empty_like(vS0), torch.empty_like(vC0)
        vout = torch.empty((vc.t_total, d.value_dim), dtype=bf, device=dev)
        vws = gdn.alloc_workspace(cfg, vc.n_seq, vc.t_total, dev)
        vp = {k: v.to(dev) for k, v in vc.params.items()}
        work["varlen"] = (time_calls(lambda: gdn.prefill_chunked(
            cfg, vp, vseq, *vx, state_in=vS0, state_out=vS, conv_in=vC0, conv_out=vC, out=vout,
            workspace=vws, stream=stream), 5), vc)
        del vx, vws, vout

        # Long-context hand-off: B=1 prefill of T=65536 (sigmoid gate), then
        # 256 decode steps from the returned state and history.
        lc = long_handoff()
        ld = lc.dims
        lcfg = gdn.Config(ld.h_k, ld.h_v, ld.d_k, ld.d_v, ld.conv_k, bf, bf, ld.gate)
        lp = {k: v.to(dev) for k, v in lc.params.items()}
        lx = [getattr(lc, k).to(bf).to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
        lseq = gdn.SeqLens(lc.cu_seqlens, dev)
        lS = torch.empty((1, ld.h_v, ld.d_k, ld.d_v), dtype=torch.float32, device=dev)
        lC = torch.empty((1, ld.conv_k - 1, ld.conv_dim), dtype=torch.float32, device=dev)
        lout = torch.empty((lc.t_total, ld.value_dim), dtype=bf, device=dev)
        lws = gdn.alloc_workspace(lcfg, 1, lc.t_total, dev)
        lpf_ms = time_calls(lambda: gdn.prefill_chunked(lcfg, lp, lseq, *lx, state_out=lS,
                                                        conv_out=lC, out=lout, workspace=lws,
                                                        stream=stream), 3, warm=1)
        del lx, lws, lout
        ldx = [lc.dec[k].to(bf).to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
        ldo = torch.empty((1, ld.value_dim), dtype=bf, device=dev)
        nld = ldx[0].shape[0]

        def long_decode(st=None):
            for j in range(nld):
                gdn.decode_step(lcfg, lp, ldx[0][j], ldx[1][j], ldx[2][j], ldx[3][j], lC, lS,
                                out=ldo, stream=st)
        work["long"] = (lpf_ms, time_calls(lambda: long_decode(stream), 2, warm=1) / nld,
                        time_graph(long_decode, 2) / nld, nld, lc)
        del ldx

    # Multi-token decode (speculative verification of t_new drafted tokens per
    # sequence, gdn_decode_multi), same batch, states updated in place.
    multi = {}
    for t_new in (() if args.no_multi else (1, 2, 4, 8)):
        xm = [x_dc[k][:t_new].transpose(0, 1).contiguous() for k in range(4)]
        out_m = torch.empty((B, t_new, d.value_dim), dtype=bf, device=dev)
        calls = 50
        for _ in range(3):
            gdn.decode_multi(cfg, dparams, *xm, c_dc, S_dc, out=out_m, stream=stream)
        ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev_m[0].record(stream)
        for _ in range(calls):
            gdn.decode_multi(cfg, dparams, *xm, c_dc, S_dc, out=out_m, stream=stream)
        ev_m[1].record(stream)
        torch.cuda.synchronize()
        multi[t_new] = (ev_m[0].elapsed_time(ev_m[1]) / calls, calls)

    # The per-channel-decay variant (Kimi Delta Attention) on the same batch:
    # one, four and eight tokens per sequence.
    from gdn_inputs import make_case
    kd = BIG.__class__(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k, "sigmoid", decay="channel")
    kcase = None if args.no_multi else make_case(kd, [0] * B, act_dtype="bf16", seed=5,
                                                  s0_std=0.02, conv0_std=1.0, decode_steps=8)
    kda = {}
    kda_pf = None
    if kcase is not None:
        kcfg = gdn.Config(kd.h_k, kd.h_v, kd.d_k, kd.d_v, kd.conv_k, bf, bf, "sigmoid",
                          decay="channel")
        kparams = {k: v.to(dev) for k, v in kcase.params.items()}
        S_k, c_k = kcase.S0.to(dev), kcase.conv0.to(dev)
        for t_new in (1, 4, 8):
            xm = [kcase.dec[k][:t_new].transpose(0, 1).to(bf).to(dev).contiguous()
                  for k in ("qkv", "z", "a", "b")]
            out_m = torch.empty((B, t_new, d.value_dim), dtype=bf, device=dev)
            calls = 50
            for _ in range(3):
                gdn.decode_multi(kcfg, kparams, *xm, c_k, S_k, out=out_m, stream=stream)
            ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev_m[0].record(stream)
            for _ in range(calls):
                gdn.decode_multi(kcfg, kparams, *xm, c_k, S_k, out=out_m, stream=stream)
            ev_m[1].record(stream)
            torch.cuda.synchronize()
            kda[t_new] = (ev_m[0].elapsed_time(ev_m[1]) / calls, calls)
        del S_k, c_k
        # chunked prefill with one decay per key channel, T=4096, zero state
        kpf = make_case(kd, [T], act_dtype="bf16", seed=6)
        kx = [getattr(kpf, k).to(bf).to(dev).contiguous() for k in ("qkv", "z", "a", "b")]
        kpp = {k: v.to(dev) for k, v in kpf.params.items()}
        kws = gdn.alloc_workspace(kcfg, 1, T, dev)
        for _ in range(3):
            gdn.prefill_chunked(kcfg, kpp, seq, *kx, state_out=S_pf, conv_out=c_pf, out=out_pf,
                                workspace=kws, stream=stream)
        ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        calls = 20
        ev_m[0].record(stream)
        for _ in range(calls):
            gdn.prefill_chunked(kcfg, kpp, seq, *kx, state_out=S_pf, conv_out=c_pf, out=out_pf,
                                workspace=kws, stream=stream)
        ev_m[1].record(stream)
        torch.cuda.synchronize()
        kda_pf = (ev_m[0].elapsed_time(ev_m[1]) / calls, calls)
        del kws

    # The mixer with its projections (hidden 2048): one decode step for the
    # B=64 batch and the T=4096 prefill, same core inputs' shapes.
    mix = {}
    if not args.no_multi:
        from gdn_inputs import make_hidden, make_projections
        Hd = 2048
        proj = make_projections(d, Hd, seed=7)
        pj = {k: (v if k == "hidden" else v.to(bf).to(dev).contiguous()) for k, v in proj.items()}
        xd = make_hidden(B, Hd, seed=8).to(bf).to(dev)
        xp = make_hidden(T, Hd, seed=9).to(bf).to(dev)
        mws = torch.empty(gdn.mixer_workspace_bytes(cfg, Hd, 1, T), dtype=torch.uint8, device=dev)
        yd = torch.empty((B, Hd), dtype=bf, device=dev)
        yp = torch.empty((T, Hd), dtype=bf, device=dev)
        for name, fn, calls in (
                ("decode", lambda: gdn.mixer_decode(cfg, dparams, pj, xd, c_dc, S_dc, y=yd,
                                                    workspace=mws, stream=stream), 50),
                ("prefill", lambda: gdn.mixer_prefill(cfg, params, pj, seq, xp, state_out=S_pf,
                                                      conv_out=c_pf, y=yp, workspace=mws,
                                                      stream=stream), 10)):
            for _ in range(3):
                fn()
            ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev_m[0].record(stream)
            for _ in range(calls):
                fn()
            ev_m[1].record(stream)
            torch.cuda.synchronize()
            mix[name] = (ev_m[0].elapsed_time(ev_m[1]) / calls, calls, Hd)
        # A few sequences (launch-latency bound): 10 steps replayed as one
        # HIP graph, on the first Bs sequences of the decode batch.
        for Bs in (1, 8):
            xs, ys = xd[:Bs], yd[:Bs]
            Ss, cs = S_dc[:Bs], c_dc[:Bs]

            def small_steps(st=None):
                for _ in range(10):
                    gdn.mixer_decode(cfg, dparams, pj, xs, cs, Ss, y=ys, workspace=mws, stream=st)
            mix[f"decode_b{Bs}"] = (time_graph(small_steps, 5) / 10, 50, Hd)
        del mws

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    dbytes = decode_bytes(d, B)
    pflops = prefill_flops(d, T)
    pbytes = prefill_bytes(d, T)
    dec_gbs = dbytes / (dc_ms * 1e-3) / 1e9
    dec_cold_gbs = dbytes / (dc_cold_ms * 1e-3) / 1e9
    pf_tflops = pflops / (pf_ms * 1e-3) / 1e12
    roof_dec = {"kernel": "gdn::decode_multi_kernel (gdn_decode_step: 1 token per sequence, "
                          "1 launch)", "bound": "hbm",
                "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                "traffic": load_traffic("decode_multi_kernel"),
                "algorithmic_bytes_per_launch": dbytes,
                "duration_us": round(dc_ms * 1e3, 2),
                "launches_timed": args.steps * n_sets}
    roof_dec_cold = dict(roof_dec, achieved=round(dec_cold_gbs, 1),
                         frac=round(dec_cold_gbs / PEAK_HBM_GBS, 4),
                         duration_us=round(dc_cold_ms * 1e3, 2), launches_timed=cold_steps,
                         traffic=None,
                         note="4 state sets in rotation (Infinity Cache cold for the state), "
                              "state_cache=streamed (non-temporal state loads and stores); "
                              "with the default cached hint: %.2f us"
                              % (dc_cold_cached_ms * 1e3))
    roof_pf = {"kernel": "gdn_prefill_chunked (qknorm, tri, scan, norm launches)",
               "bound": "mfma", "achieved": round(pf_tflops, 2), "peak": PEAK_BF16_TFLOPS,
               "unit": "TFLOP/s", "frac": round(pf_tflops / PEAK_BF16_TFLOPS, 4),
               "traffic": load_traffic("prefill_call"),
               "algorithmic_flops_per_launch": pflops,
               "duration_us": round(pf_ms * 1e3, 2), "launches_timed": args.steps,
               "mfma_busy": load_counter("prefill_call", "mfma_busy"),
               "hbm_frac": round(pbytes / (pf_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    roof_multi = {}
    for t_new, (ms, calls) in kda.items():
        mb = decode_multi_bytes(kd, B, t_new)
        gbs = mb / (ms * 1e-3) / 1e9
        roof_multi[f"kda_decode_t{t_new}"] = {
            "kernel": f"gdn::decode_multi_kernel, one decay per key channel "
                      f"(gdn_decode_multi, {t_new} tokens/sequence)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": mb, "duration_us": round(ms * 1e3, 2),
            "launches_timed": calls, "tokens_per_s": round(B * t_new / (ms * 1e-3), 1)}
    if kda_pf is not None:
        ms, calls = kda_pf
        tf = pflops / (ms * 1e-3) / 1e12
        roof_multi["kda_prefill"] = {
            "kernel": "gdn_prefill_chunked, one decay per key channel (kda_intra, tri, scan, "
                      "norm launches)",
            "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": pflops, "duration_us": round(ms * 1e3, 2),
            "launches_timed": calls, "tokens_per_s": round(T / (ms * 1e-3), 1)}
    if "decode" in mix:
        ms, calls, Hd = mix["decode"]
        nproj = d.conv_dim + d.value_dim + 2 * d.h_v
        mb = dbytes + (nproj + d.value_dim) * Hd * 2 + 2 * B * Hd * 2
        gbs = mb / (ms * 1e-3) / 1e9
        roof_multi["mixer_decode"] = {
            "kernel": "gdn_mixer_decode (in_proj product + conv epilogue, decode kernel, "
                      "out_proj product over hi/lo parts + slice sum), hidden 2048",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": mb, "duration_us": round(ms * 1e3, 2),
            "launches_timed": calls, "tokens_per_s": round(B / (ms * 1e-3), 1)}
    for Bs in (1, 8):
        if f"decode_b{Bs}" not in mix:
            continue
        ms, calls, Hd = mix[f"decode_b{Bs}"]
        nproj = d.conv_dim + d.value_dim + 2 * d.h_v
        mb = decode_bytes(d, Bs) + (nproj + d.value_dim) * Hd * 2 + 2 * Bs * Hd * 2
        gbs = mb / (ms * 1e-3) / 1e9
        roof_multi[f"mixer_decode_b{Bs}"] = {
            "kernel": "gdn_mixer_decode at B=%d (in_proj product with the conv in its epilogue, "
                      "decode kernel, out_proj product over hi/lo parts + slice sum), "
                      "hidden 2048" % Bs,
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": mb, "duration_us": round(ms * 1e3, 2),
            "duration_note": "device time, 10 steps replayed as one HIP graph",
            "launches_timed": calls, "tokens_per_s": round(Bs / (ms * 1e-3), 1)}
    if "prefill" in mix:
        ms, calls, Hd = mix["prefill"]
        nproj = d.conv_dim + d.value_dim + 2 * d.h_v
        mf = pflops + 2 * T * Hd * (nproj + d.value_dim)
        tf = mf / (ms * 1e-3) / 1e12
        roof_multi["mixer_prefill"] = {
            "kernel": "gdn_mixer_prefill (in_proj GEMMs, chunked prefill, out_proj GEMMs), "
                      "hidden 2048",
            "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": mf, "duration_us": round(ms * 1e3, 2),
            "launches_timed": calls, "tokens_per_s": round(T / (ms * 1e-3), 1)}
    for t_new, (ms, calls) in multi.items():
        mb = decode_multi_bytes(d, B, t_new)
        gbs = mb / (ms * 1e-3) / 1e9
        roof_multi[f"decode_multi_t{t_new}"] = {
            "kernel": f"gdn::decode_multi_kernel (gdn_decode_multi, {t_new} tokens/sequence)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": mb, "duration_us": round(ms * 1e3, 2),
            "launches_timed": calls, "tokens_per_s": round(B * t_new / (ms * 1e-3), 1)}
    workloads = {}
    if "tiny" in work:
        us, gus, nst, td = work["tiny"]
        tb = decode_bytes(td, 1)
        workloads["tiny_recurrent"] = {
            "config": "1 sequence, 64 tokens one at a time (gdn_decode_step), H_k=H_v=2, "
                      "d_k=d_v=32, K=4, fp32 in/out",
            "us_per_step": round(gus * 1e3, 2),
            "us_per_step_note": "device time, the 64 steps replayed as one HIP graph",
            "us_per_step_eager": round(us * 1e3, 2), "steps_timed": 20 * nst,
            "bound": "launch latency", "algorithmic_bytes_per_step": tb,
            "hbm_frac": round(tb / (gus * 1e-3) / 1e9 / PEAK_HBM_GBS, 6)}
    if "varlen" in work:
        ms, vc = work["varlen"]
        vflops = prefill_flops(d, vc.t_total)
        vbytes = prefill_bytes(d, vc.t_total, vc.n_seq, state_in=True)
        lens = [vc.cu_seqlens[i + 1] - vc.cu_seqlens[i] for i in range(vc.n_seq)]
        workloads["varlen_prefill"] = {
            "config": f"{vc.n_seq} packed sequences, lengths {lens} ({vc.t_total} tokens), "
                      "random initial states, bf16",
            "tokens_per_s": round(vc.t_total / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
            "calls_timed": 5, "algorithmic_flops_per_call": vflops,
            "mfma_frac": round(vflops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_bytes_per_call": vbytes,
            "hbm_frac": round(vbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if "long" in work:
        pms, dms_eager, dms, nld, lc = work["long"]
        lflops = prefill_flops(lc.dims, lc.t_total)
        lbytes = prefill_bytes(lc.dims, lc.t_total)
        db1 = decode_bytes(lc.dims, 1)
        workloads["long_handoff"] = {
            "config": f"B=1 prefill T={lc.t_total} (sigmoid gate), then {nld} decode steps "
                      "from its state, B=1",
            "prefill_tokens_per_s": round(lc.t_total / (pms * 1e-3), 1),
            "prefill_ms": round(pms, 4), "prefill_calls_timed": 3,
            "prefill_mfma_frac": round(lflops / (pms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "prefill_hbm_frac": round(lbytes / (pms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "decode_us_per_step": round(dms * 1e3, 2),
            "decode_us_per_step_note": "device time, the 256 steps replayed as one HIP graph",
            "decode_us_per_step_eager": round(dms_eager * 1e3, 2), "decode_steps_timed": 2 * nld,
            "decode_algorithmic_bytes_per_step": db1,
            "decode_hbm_frac": round(db1 / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # the kernel that takes most of a step's time
    dominant = roof_pf if pf_ms >= dc_ms * n_sets else roof_dec

    line = {
        "metric": "GDN prefill tokens/s (T=4096) + decode step us at B=64; % HBM/MFMA peak",
        "value": round(T / (pf_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32+bf16x3",
        "dtype_note": "decode: fp32 vector FMA; prefill contractions: fp32 operands split into "
                      "bf16 hi + lo parts, three MFMAs (hi.hi + hi.lo + lo.hi; lo.lo dropped), "
                      "fp32 accumulation; conv, norms and gates fp32; activations bf16 in and out",
        "data": "synthetic",
        "config": {"workload": "GDN mixer: prefill B=1 T=4096 + 100 consecutive decode "
                               "steps B=64; H_k=16 H_v=32 d_k=d_v=128 K=4 C=64; bf16 "
                               "activations/output, fp32 state", "global_batch": 64, "seq_len": T,
                   "parallelism": "single GPU"},
        "prefill_ms": round(pf_ms, 4),
        "decode_us_per_step": round(dc_ms * 1e3, 2),
        "decode_cold_us_per_step": round(dc_cold_ms * 1e3, 2),
        "decode_cold_note": "four state sets in rotation, state_cache=streamed",
        "decode_cold_cached_hint_us_per_step": round(dc_cold_cached_ms * 1e3, 2),
        "decode_tokens_per_s": round(B / (dc_ms * 1e-3), 1),
        "roofline": dominant,
        "roofline_note": "roofline is the kernel that takes most of the step's time (the 100 "
                         "decode steps); the prefill's own roofline is rooflines.prefill. The "
                         "100 decode steps (28 GB of state traffic) evict the prefill's data "
                         "from the 256 MB Infinity Cache between prefills, in place of an "
                         "explicit flush",
        "workloads": workloads,
        "rooflines": {"decode": roof_dec, "decode_cold": roof_dec_cold, "prefill": roof_pf,
                      **roof_multi},
        "note": "the pages quote no throughput for this path on any hardware",
    }
    if not args.no_cpu_baseline:
        threads = max(1, min(16, os.cpu_count() or 1))
        line["cpu_baseline"] = cpu_baseline(pf, dc, threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
