#!/usr/bin/env python3
"""Benchmark of the chunkwise gated delta-rule backward on one MI355X.

Workload: GDN (scalar gate) at (B, T, H) = (1, 8192, 16), chunk 64,
d_k = d_v = 128, bf16 inputs with fp32 gates and state, seeded synthetic
inputs (delta_rule_linear_gdr_amd.inputs). One step = one complete low-level
backward under the recompute policy: gate cumsum and chunk preparation, the
forward state scan that rebuilds the per-chunk states, the reverse state
scan, and the chunk-local ReWY backward with Gram elimination. Inputs are
resident in device memory before the timed region.

Prints one JSON line. Besides the headline value it reports the per-stage
durations (HIP events recorded by the library on the launch stream over a
second timed pass), the roofline of the dominant kernel, the whole-path
roofline, the forward, the full-save policy, the seven-product ablation, the
KDA backward at the same shape (and the KDA forward + backward end to end),
and the fp64 CPU oracle on the same workload.

--profile-pass runs a known-size elementwise copy and a few headline steps
only; it is the command the hardware-counter summaries under profiles/ are
taken with (the copy calibrates FETCH_SIZE / WRITE_SIZE to bytes).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
CH = 64
T16, T32, T8, GN = 16384, 32768, 8192, 512   # bf16 64x128, 128x128, 64x64 tiles; exp(G_n)
M = 1048576                                   # 2 * 64 * 64 * 128 FLOPs
SOLVE = CH ** 3 // 3                          # inverse of a 64 x 64 unit lower-triangular matrix

# Whole-path algorithmic bytes per token-head of the operator's inputs and
# outputs at bf16: forward reads q, k, v, g, beta and writes o; backward
# reads q, k, v, dO, g, beta and writes dq, dk, dv, dg, dbeta; the full-save
# forward writes, and its backward reads, the 1152-byte saved area (A, W,
# per-chunk state, R). The gate is 4 bytes (scalar) or 512 (vector) per
# token-head, its gradient the same. GDN2 takes a per-key erase gate and a
# per-value write gate (bf16, 256 bytes each) in place of beta, and returns
# their gradients.
PATH_BYTES_PER_TOKEN_HEAD = {
    ("scalar", "fwd_R"): 1030, ("scalar", "fwd_A"): 2182,
    ("scalar", "bwd_R"): 1804, ("scalar", "bwd_A"): 2956,
    ("vector", "fwd_R"): 1538, ("vector", "fwd_A"): 2690,
    ("vector", "bwd_R"): 2820, ("vector", "bwd_A"): 3972,
    ("gdn2", "fwd_R"): 2048, ("gdn2", "bwd_R"): 3840,
}
# 128 x 128 fp32 state tensors a call touches per head: h0 and ht (forward);
# h0 and dh0 (recompute backward, dht absent); dh0 (full-save backward)
PATH_STATES = {"fwd_R": 2, "fwd_A": 2, "bwd_R": 2, "bwd_A": 1}
# Algorithmic FLOPs per (chunk, head): the dense products of each call
# (2mnk, in units of M) plus the triangular solve, the same for both gates at
# d_k = d_v = 128. Forward: L and H (1 each), W and U (2), the state walk
# W S and K~^T R (4), the output Q_g S and H R (3). Backward, recompute:
# prep's L, H, W, U, X = H^T dO (1) and Y = Q_g^T dO (2), both walks (8) and
# the local kernel (13). Backward, full save: X and Y (3), the reverse walk
# K~ dS and W^T dR (4) and the local kernel (13).
PATH_FLOPS_PER_CHUNK_HEAD = {"fwd_R": 11 * M + SOLVE, "fwd_A": 11 * M + SOLVE,
                             "bwd_R": 28 * M + SOLVE, "bwd_A": 20 * M}


def path_figures(gate: str, kind: str, B: int, T: int, H: int, ms: float) -> dict:
    """Whole-call throughput against both rooflines: achieved TFLOP/s as a
    fraction of the bf16 MFMA peak, algorithmic GB/s as a fraction of the
    HBM peak, and the fraction of the binding one, max(t_MFMA, t_HBM) / t."""
    flops = PATH_FLOPS_PER_CHUNK_HEAD[kind] * B * H * ((T + CH - 1) // CH)
    nbytes = PATH_BYTES_PER_TOKEN_HEAD[(gate, kind)] * B * T * H + PATH_STATES[kind] * 65536 * B * H
    t = ms * 1e-3
    tfs, gbs = flops / t / 1e12, nbytes / t / 1e9
    return {"TFLOP/s": round(tfs, 2), "frac_mfma": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "bytes": nbytes, "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "frac_roofline": round(max(tfs / MFMA_BF16_PEAK_TFS, gbs / HBM_PEAK_GBS), 4)}


def kernel_work(gate: str) -> dict:
    """(algorithmic bytes, algorithmic FLOPs) per (chunk, head) of each kernel,
    as tabulated in the design notes: every operand read once and every result
    written once at its stored type; FLOPs of the method's dense products."""
    g_bytes = CH * 4 if gate == "scalar" else CH * 128 * 4
    # beta, or GDN2's erase (per key) and write (per value) gates; the same
    # again for the gradient
    beta = 2 * T16 if gate == "gdn2" else CH * 2
    inputs4 = 4 * T16
    return {
        # recompute backward: reads q, k, v, dO, g, beta; writes -W, Kt, U, X,
        # Y, A^T, gn (and A, 8 KiB more, for the seven-product backward)
        "prep": (inputs4 + g_bytes + beta + 4 * T16 + T32 + T8 + GN,
                 1 * M + 1 * M + SOLVE + 2 * M + 1 * M + 2 * M),
        # reads -W, Kt (read transposed), U, gn; writes h, R.
        # R = U - W S; S' = gn S + Kt^T R
        "scan_fwd": (3 * T16 + GN + T32 + T16, 4 * M),
        # reads Kt, -W (read transposed), X, Y, gn; writes dh, Rb
        "scan_bwd": (3 * T16 + T32 + GN + T32 + T16, 4 * M),
        # both scans in one launch: the -W, Kt and gn they share count once
        "scan_pair": (4 * T16 + T32 + GN + T32 + T16 + T32 + T16, 8 * M),
        # reads q, k, v, dO, g, beta, R, Rb, h, dh, A^T; writes dq, dk, dv, dg, dbeta
        "bwd_local": (inputs4 + g_bytes + beta + 2 * T16 + 2 * T32 + T8 + 3 * T16 + g_bytes + beta,
                      13 * M),
        "bwd_local_wy7": (inputs4 + g_bytes + beta + 2 * T16 + 2 * T32 + 2 * T8 + 3 * T16 + g_bytes
                          + beta, 16 * M),
        # reads Hm^T, Qg^T, dO; writes X, Y
        "xy": (T8 + T16 + T16 + T16 + T32, 3 * M),
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline only")
    ap.add_argument("--no-sweep", action="store_true", help="skip the six-shape sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="calibration copy + a few headline steps, for rocprofv3 counter runs")
    ap.add_argument("--with-wy7", action="store_true",
                    help="profile pass: after the ReWY steps, as many seven-product backward steps")
    ap.add_argument("--workload", default="gdn_1x8192x16",
                    choices=["gdn_1x8192x16", "kda_1x8192x16", "gdn2_1x8192x16"],
                    help="the backward the profile pass steps (the timed bench is always GDN)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the HIP sources; counter summaries record it so a stale
    summary (kernels changed since the counters were taken) is not used."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "delta_rule_linear_gdr_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, units: int):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None if there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "gdn_bwd_R_1x8192x16_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel sources sha256\[:16\]: `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    row = re.search(r"^\| %s \| ([0-9.]+) \| ([0-9.]+) \|" % re.escape(kernel), text, re.M)
    if not row:
        return None
    return round(float(row.group(1)) + float(row.group(2)), 0)


def shape_sweep(gdr, to_dev, make_runner, time_steps, graph_ms, args):
    """The six shapes of the pages' evaluation, scalar and vector gate (gate
    means 4 and 3, the distributions of the (1,2048,16) and (2,2048,16)
    workloads), backward under both policies and the recompute forward:
    ms per call and backward tokens/s. Each figure is the second of two timed
    passes: calls of a few tens of microseconds right after a change of shape
    otherwise catch the device below its working clock (the first pass of
    the (1,512,4) forward has read 0.042 against 0.022 ms)."""
    import torch
    from delta_rule_linear_gdr_amd.inputs import SHAPES6, make_inputs

    def time2(run):
        time_steps(run, args.steps, args.warmup)
        return time_steps(run, args.steps, args.warmup)

    rows = []
    for Bs, Ts, Hs in SHAPES6:
        for gate in ("scalar", "vector"):
            xs = make_inputs(Bs, Ts, Hs, gate=gate, dtype="bf16", seed=0,
                             gate_mean=4.0 if gate == "scalar" else 3.0)
            ds = to_dev(xs)
            row = {"B": Bs, "T": Ts, "H": Hs, "gate": gate}
            runR = make_runner(ds, gdr.gdr_bwd, "recompute")
            msR = time2(runR)
            msRg = graph_ms(runR, args.steps, args.warmup)
            _, _, saved = gdr.gdr_fwd(ds["q"], ds["k"], ds["v"], ds["g"], ds["beta"], ds["h0"],
                                      policy="full_save")
            msA = time2(make_runner(ds, gdr.gdr_bwd, "full_save", saved))
            _, sc = gdr.workspace_size(Bs, Ts, Hs, gate, "bf16", "recompute")
            scr = torch.empty(sc, dtype=torch.uint8, device=ds["q"].device)
            msF = time2(lambda: gdr.gdr_fwd(ds["q"], ds["k"], ds["v"], ds["g"], ds["beta"],
                                            ds["h0"], policy="recompute", scratch=scr))
            row.update(bwd_R_ms=round(msR, 4), bwd_R_graph_ms=round(msRg, 4), bwd_A_ms=round(msA, 4),
                       fwd_R_ms=round(msF, 4),
                       bwd_R_tokens_per_s=round(Bs * Ts / (msR * 1e-3), 1),
                       bwd_A_tokens_per_s=round(Bs * Ts / (msA * 1e-3), 1),
                       fwd_R_tokens_per_s=round(Bs * Ts / (msF * 1e-3), 1),
                       bwd_R_roofline=path_figures(gate, "bwd_R", Bs, Ts, Hs, msR),
                       bwd_A_roofline=path_figures(gate, "bwd_A", Bs, Ts, Hs, msA),
                       fwd_R_roofline=path_figures(gate, "fwd_R", Bs, Ts, Hs, msF))
            rows.append(row)
            print(f"[bench] sweep {row}", file=sys.stderr, flush=True)
            del ds, xs, saved, scr
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the operator runs on one GPU (it has no multi-GPU path); --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import delta_rule_linear_gdr_amd as gdr
    from delta_rule_linear_gdr_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        bf = torch.bfloat16
        d = {n: torch.from_numpy(x[n]).to(dev, bf) for n in ("q", "k", "v", "beta", "dO")}
        d["g"] = torch.from_numpy(x["g"]).to(dev, torch.float32)
        d["h0"] = torch.from_numpy(x["h0"]).to(dev, torch.float32)
        return d

    if args.workload != "gdn_1x8192x16" and not args.profile_pass:
        print("bench.py: --workload selects the profile pass's backward only", file=sys.stderr)
        sys.exit(2)
    wl = WORKLOADS[args.workload]
    x = wl.make()
    d = to_dev(x)
    B, T, H = wl.B, wl.T, wl.H
    units = B * H * (T // CH)

    def make_runner(dd, fn, policy, saved=None):
        Bq, Tq, Hq = dd["q"].shape[:3]
        _, sc = gdr.workspace_size(Bq, Tq, Hq, "vector" if dd["g"].dim() == 4 else "scalar",
                                   "bf16", policy)
        scratch = torch.empty(sc, dtype=torch.uint8, device=dev)
        out = dict(dq=torch.empty_like(dd["q"]), dk=torch.empty_like(dd["k"]),
                   dv=torch.empty_like(dd["v"]), dg=torch.empty_like(dd["g"]),
                   dbeta=torch.empty_like(dd["beta"]),
                   dh0=torch.empty((Bq, Hq, 128, 128), dtype=torch.float32, device=dev))

        def run():
            fn(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], dd["dO"], None,
               saved=saved, policy=policy, scratch=scratch, out=out)
        return run

    def time_steps(run, steps, warmup):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per step

    def capture(run):
        """A HIP graph of one call of `run` (static buffers), after one warm call
        on the capture stream."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        return graph

    def graph_ms(run, steps, warmup):
        """ms per call of `run` replayed from a HIP graph (the pages time the
        backward as warmed device-graph replays); run uses static buffers."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        ms_g = time_steps(graph.replay, steps, warmup)
        del graph
        return ms_g

    def graph_median_ms(run, n_obs=60, warm_s=2.0):
        """The pages' protocol: at least 2 s of warm-up, then 60 observations
        of one HIP-graph replay each (events around the replay), median."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            for _ in range(20):
                graph.replay()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        obs = []
        for _ in range(n_obs):
            e0.record()
            graph.replay()
            e1.record()
            e1.synchronize()
            obs.append(e0.elapsed_time(e1))
        del graph
        obs.sort()
        return 0.5 * (obs[(n_obs - 1) // 2] + obs[n_obs // 2])

    def profiled(run, steps):
        gdr.profile_begin(8 * steps + 16)
        for _ in range(steps):
            run()
        st = gdr.profile_end()
        return {k: v[1] / v[0] for k, v in st.items()}  # avg ms per launch

    run = make_runner(d, gdr.gdr_bwd, "recompute")
    if wl.gate == "gdn2":
        # (profile pass only) the GDN2 backward on the same tensors plus both gates
        ers2 = torch.from_numpy(x["ers"]).to(dev, torch.bfloat16)
        wrt2 = torch.from_numpy(x["wrt"]).to(dev, torch.bfloat16)
        _, sc2 = gdr.workspace_size(B, T, H, "gdn2", "bf16", "recompute")
        scr2 = torch.empty(sc2, dtype=torch.uint8, device=dev)
        out2 = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
                    dg=torch.empty_like(d["g"]), derase=torch.empty_like(ers2), dwrite=torch.empty_like(wrt2),
                    dh0=torch.empty((B, H, 128, 128), dtype=torch.float32, device=dev))

        def run():
            gdr.gdr_bwd_gdn2(d["q"], d["k"], d["v"], d["g"], ers2, wrt2, d["h0"], d["dO"], None,
                             scratch=scr2, out=out2)

    if args.profile_pass:
        # calibration: an elementwise kernel that reads and writes exactly
        # 256 MiB each (torch.mul over fp32), then the headline steps
        n = 64 * 1024 * 1024
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        if args.with_wy7:
            run7 = make_runner(d, gdr.gdr_bwd_wy7, "recompute")
            for _ in range(args.steps):
                run7()
            torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "workload": wl.name, "copy_bytes_each_way": 4 * n,
                          "steps": args.steps, "with_wy7": args.with_wy7,
                          "kernel_sources": kernel_source_hash()}),
              flush=True)
        return

    # ---- headline: GDN backward, recompute policy ----
    # The device is first warmed for at least 2 s, as in the pages' protocol,
    # followed by one untimed pass of the timing loop itself: measured on an
    # MI355X, the first timed pass after warm-up runs about 10% slow whatever is
    # timed, the later ones agree to 1%. A step is one eager call (its three
    # kernels); the same call replayed from a HIP graph is reported beside it.
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 2.0:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
    time_steps(run, args.steps, 0)
    ms = time_steps(run, args.steps, args.warmup)
    step_graph = capture(run)
    ms_graph = time_steps(step_graph.replay, args.steps, args.warmup)
    del step_graph
    print(f"[bench] gdn bwd-R (1,8192,16): {ms:.4f} ms/step, {ms_graph:.4f} as graph replays",
          file=sys.stderr, flush=True)
    stage_ms = profiled(run, args.steps)
    print(f"[bench] stages (ms): {stage_ms}", file=sys.stderr, flush=True)
    work = kernel_work("scalar")
    dom = max(stage_ms, key=stage_ms.get)
    t_s = stage_ms[dom] * 1e-3
    traffic = measured_traffic(dom, units)
    # The roofline of the dominant kernel as the method's work defines it:
    # the whole backward's algorithmic bytes (the operator's own inputs and
    # outputs, once each: 1,804 B per token-head plus h0 read and dh0
    # written) over that kernel's average launch time. Against the same
    # kernel time the method's dense FLOPs give a far smaller fraction of the
    # MFMA peak, so the HBM roofline is the binding one.
    path = path_figures("scalar", "bwd_R", B, T, H, ms)
    path_bytes = path["bytes"]
    path_flops = PATH_FLOPS_PER_CHUNK_HEAD["bwd_R"] * units
    achieved = path_bytes / t_s / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": dom, "kernel_ms": round(stage_ms[dom], 4),
            "algorithmic_bytes_per_launch": path_bytes,
            "algorithmic_bytes_basis": "whole recompute backward: 1804 B per token-head "
                                       "x 131072 token-heads + h0 and dh0 (64 KiB per head each)",
            "mfma_frac_same_time": round(path_flops / t_s / 1e12 / MFMA_BF16_PEAK_TFS, 4),
            "path_frac": path["frac_hbm"], "path_ms": round(ms, 4)}
    steps_bwd = ("prep", "scan_pair", "bwd_local")
    bwd_flops = sum(work[k][1] for k in steps_bwd) * units
    tok_s = B * T / (ms * 1e-3)
    detail = {
        "bwd_R_ms": round(ms, 4),
        "bwd_R_graph_loop_ms": round(ms_graph, 4),
        "bwd_R_tflops": round(bwd_flops / (ms * 1e-3) / 1e12, 2),
        "path_roofline": path,
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        # each kernel against its own read/write set in this design (the
        # intermediates it exchanges with the other kernels included): a
        # measure of how close a kernel runs to the bandwidth its own traffic
        # needs, not of the method's work
        "per_stage_implementation_roofline": {},
    }
    for k, v in stage_ms.items():
        by_k, fl_k = work[k]
        detail["per_stage_implementation_roofline"][k] = {
            "implementation_bytes_per_launch": by_k * units,
            "GB/s": round(by_k * units / (v * 1e-3) / 1e9, 1),
            "frac_hbm": round(by_k * units / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(fl_k * units / (v * 1e-3) / 1e12, 2)}

    if not args.no_extra:
        # the same step replayed from a HIP graph: mean over the timed steps,
        # and the pages' protocol (median of 60 single replays after >= 2 s)
        detail["bwd_R_graph_ms"] = round(graph_ms(run, args.steps, args.warmup), 4)
        detail["bwd_R_graph_median60_ms"] = round(graph_median_ms(run), 4)
        # forward, recompute policy (output + final state)
        _, sc = gdr.workspace_size(B, T, H, "scalar", "bf16", "recompute")
        scr = torch.empty(sc, dtype=torch.uint8, device=dev)

        def fwd():
            gdr.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], policy="recompute",
                        scratch=scr)
        fms = time_steps(fwd, args.steps, args.warmup)
        detail["fwd_R_ms"] = round(fms, 4)
        detail["fwd_R_tokens_per_s"] = round(B * T / (fms * 1e-3), 1)
        detail["fwd_R_roofline"] = path_figures("scalar", "fwd_R", B, T, H, fms)
        del scr
        # full-save policy: forward saves, backward reuses
        _, _, saved = gdr.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                  policy="full_save")
        runA = make_runner(d, gdr.gdr_bwd, "full_save", saved)
        msA = time_steps(runA, args.steps, args.warmup)
        detail["bwd_A_ms"] = round(msA, 4)
        detail["bwd_A_graph_median60_ms"] = round(graph_median_ms(runA), 4)
        detail["bwd_A_tokens_per_s"] = round(B * T / (msA * 1e-3), 1)
        detail["bwd_A_roofline"] = path_figures("scalar", "bwd_A", B, T, H, msA)
        # seven-product ablation, both policies
        run7 = make_runner(d, gdr.gdr_bwd_wy7, "recompute")
        ms7 = time_steps(run7, args.steps, args.warmup)
        run7A = make_runner(d, gdr.gdr_bwd_wy7, "full_save", saved)
        ms7A = time_steps(run7A, args.steps, args.warmup)
        detail["wy7_R_ms"] = round(ms7, 4)
        detail["wy7_A_ms"] = round(ms7A, 4)
        detail["rewy_speedup_R"] = round(ms7 / ms, 4)
        detail["rewy_speedup_A"] = round(ms7A / msA, 4)
        st7 = profiled(run7, max(4, args.steps // 4))
        stl = stage_ms.get("bwd_local")
        if stl and "bwd_local_wy7" in st7:
            detail["bwd_local_wy7_ms"] = round(st7["bwd_local_wy7"], 4)
            detail["rewy_local_kernel_speedup"] = round(st7["bwd_local_wy7"] / stl, 4)
        # like for like: the three-product local kernel in the seven-product
        # kernel's launch form (one workgroup per chunk and head)
        prev = gdr.set_local_form("per_chunk")
        try:
            msPC = time_steps(run, args.steps, args.warmup)
            msPCA = time_steps(runA, args.steps, args.warmup)
            stPC = profiled(run, max(4, args.steps // 4))
        finally:
            gdr.set_local_form(prev)
        detail["per_chunk_bwd_R_ms"] = round(msPC, 4)
        detail["per_chunk_bwd_A_ms"] = round(msPCA, 4)
        detail["rewy_speedup_R_equal_form"] = round(ms7 / msPC, 4)
        detail["rewy_speedup_A_equal_form"] = round(ms7A / msPCA, 4)
        if "bwd_local" in stPC and "bwd_local_wy7" in st7:
            detail["bwd_local_per_chunk_ms"] = round(stPC["bwd_local"], 4)
            detail["rewy_local_kernel_speedup_equal_form"] = round(
                st7["bwd_local_wy7"] / stPC["bwd_local"], 4)
        del runA, run7A
        del saved
        # KDA at the same shape, recompute policy, h0 ~ 0.1 N(0,1)
        xk = WORKLOADS["kda_1x8192x16"].make()
        dk_ = to_dev(xk)
        runK = make_runner(dk_, gdr.gdr_bwd, "recompute")
        msK = time_steps(runK, args.steps, args.warmup)
        detail["kda_bwd_R_ms"] = round(msK, 4)
        detail["kda_bwd_R_graph_median60_ms"] = round(graph_median_ms(runK), 4)
        detail["kda_bwd_R_tokens_per_s"] = round(B * T / (msK * 1e-3), 1)
        detail["kda_bwd_R_roofline"] = path_figures("vector", "bwd_R", B, T, H, msK)
        detail["kda_stage_ms"] = {k: round(v, 4) for k, v in profiled(runK, args.steps).items()}
        # the same workload end to end: recompute forward (output and final
        # state) followed by the recompute backward, one step per call pair
        _, scK = gdr.workspace_size(B, T, H, "vector", "bf16", "recompute")
        scrK = torch.empty(scK, dtype=torch.uint8, device=dev)

        def runKFB():
            gdr.gdr_fwd(dk_["q"], dk_["k"], dk_["v"], dk_["g"], dk_["beta"], dk_["h0"],
                        policy="recompute", scratch=scrK)
            runK()
        msKFB = time_steps(runKFB, args.steps, args.warmup)
        detail["kda_fwd_bwd_R_ms"] = round(msKFB, 4)
        detail["kda_fwd_bwd_R_tokens_per_s"] = round(B * T / (msKFB * 1e-3), 1)
        del dk_, xk, scrK
        # GDN2 at the same shape (per-channel gate, independent erase and write
        # gates), recompute policy
        xg = make_inputs(B, T, H, gate="gdn2", dtype="bf16", seed=0, gate_mean=3.0, h0_std=0.1)
        dg_ = to_dev(xg)
        ers = torch.from_numpy(xg["ers"]).to(dev, torch.bfloat16)
        wrt = torch.from_numpy(xg["wrt"]).to(dev, torch.bfloat16)
        _, scG = gdr.workspace_size(B, T, H, "gdn2", "bf16", "recompute")
        scrG = torch.empty(scG, dtype=torch.uint8, device=dev)
        outG = dict(dq=torch.empty_like(dg_["q"]), dk=torch.empty_like(dg_["k"]),
                    dv=torch.empty_like(dg_["v"]), dg=torch.empty_like(dg_["g"]),
                    derase=torch.empty_like(ers), dwrite=torch.empty_like(wrt),
                    dh0=torch.empty((B, H, 128, 128), dtype=torch.float32, device=dev))

        def runG():
            gdr.gdr_bwd_gdn2(dg_["q"], dg_["k"], dg_["v"], dg_["g"], ers, wrt, dg_["h0"], dg_["dO"],
                             None, scratch=scrG, out=outG)
        msG = time_steps(runG, args.steps, args.warmup)
        detail["gdn2_bwd_R_ms"] = round(msG, 4)
        detail["gdn2_bwd_R_tokens_per_s"] = round(B * T / (msG * 1e-3), 1)
        detail["gdn2_bwd_R_roofline"] = path_figures("gdn2", "bwd_R", B, T, H, msG)
        detail["gdn2_bwd_R_graph_median60_ms"] = round(graph_median_ms(runG), 4)
        detail["gdn2_stage_ms"] = {k: round(v, 4) for k, v in profiled(runG, args.steps).items()}
        del dg_, xg, scrG, outG, ers, wrt
        if not args.no_sweep:
            detail["shape_sweep"] = shape_sweep(gdr, to_dev, make_runner, time_steps, graph_ms, args)

    cpu = None
    if not args.no_cpu_baseline:
        # the fp64 oracle, one whole-workload call each (it threads over
        # (sequence, head, value-row block)), on the five workloads; the
        # headline workload's call is the CPU baseline
        import oracle
        threads = oracle.default_threads()
        rows = []
        for name, wl_ in WORKLOADS.items():
            xw = x if name == wl.name else wl_.make()
            t0 = time.perf_counter()
            oracle.token_bwd(xw["q"], xw["k"], xw["v"], xw["g"], xw["beta"], xw["h0"], xw["dO"], None,
                             threads=threads)
            tw = time.perf_counter() - t0
            rows.append({"workload": name, "B": wl_.B, "T": wl_.T, "H": wl_.H, "gate": wl_.gate,
                         "seconds": round(tw, 3), "tokens_per_s": round(wl_.B * wl_.T / tw, 1)})
            print(f"[bench] oracle {name}: {tw:.2f} s", file=sys.stderr, flush=True)
            if name == wl.name:
                cpu = {"value": round(B * T / tw, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                       "sample": f"the whole GDN (1,8192,16) workload, one call: fp64 token-recurrence "
                                 f"backward incl. its forward recompute, {tw:.2f} s on {threads} threads"}
        detail["cpu_oracle_workloads"] = {"threads": threads, "rows": rows}

    line = {
        "metric": "GDN/KDA backward tokens/s + TFLOP/s (% roofline) at (1,8192,16), C=64, d=128",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GDN backward, recompute policy, (B,T,H)=(1,8192,16), C=64, "
                               "d_k=d_v=128, bf16 q/k/v/beta/dO, fp32 gates and state",
                   "B": B, "T": T, "H": H, "chunk": CH, "policy": "recompute"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ablation": {k: detail[k] for k in (
            "rewy_speedup_R", "rewy_speedup_A", "rewy_local_kernel_speedup",
            "rewy_speedup_R_equal_form", "rewy_speedup_A_equal_form",
            "rewy_local_kernel_speedup_equal_form") if k in detail} or None,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
