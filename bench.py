#!/usr/bin/env python3
"""Throughput of the selective scan on one MI355X.

One step = one call of the full hot path (softplus discretisation, the
recurrence in every direction, the D skip, the direction merge and the gate)
over one batch of synthetic inputs already resident in HBM. The default
workload is the Vim-S 1024x1024 bidirectional scan (batch 8, L 4,097,
d_inner 768, d_state 16, bf16 activations, fp32 state).

Prints one JSON line: Gtoken*channel/s over the whole job, the achieved
HBM GB/s on the algorithmic bytes, the roofline of the scan kernel (timed
with HIP events on the stream it runs on), and the fp64 CPU oracle's rate on
the host for comparison.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

#: MI355X published peaks and unit counts
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3          # published fp32 vector peak (packed FMA)
CU = 256
SIMDS_PER_CU = 4
LANES_PER_SIMD = 16               # a wave64 VALU instruction issues over 4 cycles
CLOCK_HZ = 2.4e9
#: VALU issue slots per second with non-packed fp32 instructions (the build
#: keeps packed fp32 forms out): 256 x 4 x 16 x 2.4 GHz = 39.3e12. The
#: published 157.3 TFLOP/s is this rate x 2 (FMA) x 2 (packed).
LANE_SLOTS = CU * SIMDS_PER_CU * LANES_PER_SIMD * CLOCK_HZ
#: arithmetic of one state update of the forward scan: delta*A (1 flop),
#: (delta u)*B (1), the state FMA (2) and C*h (1) plus its share of the sum
#: over the 16 states (1); the exp is not a flop
FLOPS_PER_UPDATE = 6
#: issue slots one forward state update needs at least: exp (a transcendental
#: issues in 2 slots, by the counters), delta*A, (delta u)*B, the state FMA,
#: C*h (1 each), and 15 adds per 16 states for the read-out sum
SLOTS_PER_UPDATE = 2 + 4 + 15 / 16
UPDATE_PEAK = LANE_SLOTS / SLOTS_PER_UPDATE      # 5.67e12 state updates / s
#: the gradient per state update: the recomputed forward (delta*A, (delta u)*B,
#: state FMA: 4 flops + exp), the adjoint lam = gs*C + e*lam (3), q = lam*h*e
#: (2), the dA FMA (2), lam*B and q*A with their sums over states (4), and the
#: dB, dC products (2) with the pair sum (1)
GRAD_FLOPS_PER_UPDATE = 18
#: its issue slots: exp (2) plus one slot per multiply, FMA and add above
#: (16 operations; the two state sums are 15 adds per 16 states)
GRAD_SLOTS_PER_UPDATE = 2 + 16

#: dense bf16 matrix-core peak (no sparsity)
MFMA_BF16_PEAK_TFLOPS = 2500.0

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "vision_mamba_selective_amd", "csrc", "vimscan.hip")
PROJ_SRC = os.path.join(ROOT, "vision_mamba_selective_amd", "csrc", "proj.hip")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    # the defaults keep the timed region near 0.1 s after about 30 ms of
    # warmup: with fewer steps the shader clock is still ramping up and the
    # Vim-S 1024^2 step reads about 10 % slower
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", type=int, default=None,
                   help="index into vision_mamba_selective_amd.workloads.WORKLOADS")
    p.add_argument("--sets", type=int, default=0,
                   help="input sets rotated over the steps (0: enough to exceed 768 MB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="the CPU baseline repeats its sample until this many seconds have passed")
    p.add_argument("--cpu-channels", type=int, default=0,
                   help="channels per batch row in the CPU sample (0: whole workload)")
    p.add_argument("--conv", action="store_true",
                   help="time vim_scan_bidir_conv: the same scan with the Vim block's conv1d + "
                        "SiLU front end fused into its token loads (u is then the conv input x)")
    p.add_argument("--grad", action="store_true",
                   help="time vim_scan_bidir_grad: the reverse-mode gradient of the scan for a "
                        "synthetic upstream gradient (forward recompute + adjoint pass)")
    p.add_argument("--train", action="store_true",
                   help="time one training step of the scan: vim_scan_bidir_fwd_saved (y and the "
                        "states the gradient needs) then vim_scan_bidir_grad_saved (the gradient "
                        "from them) for a synthetic upstream gradient")
    p.add_argument("--zoh", action="store_true",
                   help="exact zero-order-hold B_bar = (exp(delta A) - 1) / A B (VS_FLAG_ZOH) "
                        "instead of delta B")
    p.add_argument("--dirs", action="store_true",
                   help="time vim_scan_bidir_dirs: per-direction u, delta, B and C (a second "
                        "seeded draw feeds the backward direction)")
    p.add_argument("--proj", action="store_true",
                   help="time the projections around the scan at the workload's shape: one step is "
                        "out_proj (dim -> dim, bias + residual) on the matrix cores; x_proj and "
                        "dt_proj are timed beside it")
    p.add_argument("--chunks", type=int, default=None,
                   help="time vim_scan_bidir_chunked with this many chunks per sequence (0: the "
                        "library's choice, which is what the default line runs)")
    p.add_argument("--eager", action="store_true",
                   help="launch the timed steps one by one instead of replaying them as one HIP graph")
    p.add_argument("--copy-probe", action="store_true",
                   help="instead of the scan, run torch copies of known size (counter scale)")
    return p.parse_args()


def kernel_hash(path=KERNEL_SRC):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. Every "
              "(batch, channel) scan is independent, so splitting batch x channels across "
              "GPUs would need no communication. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from vision_mamba_selective_amd import workloads as wlm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)

    if args.copy_probe:
        return copy_probe(torch, dev)
    if args.proj:
        return proj_bench(args, torch, dev)

    import vision_mamba_selective_amd as vms

    idx = wlm.HEADLINE if args.workload is None else args.workload
    wl = wlm.WORKLOADS[idx]
    if (args.conv or args.grad or args.dirs or args.train) and wl.kind != "vim":
        print("--conv, --grad, --train and --dirs apply to the Vim workloads only", file=sys.stderr)
        sys.exit(2)
    if args.conv + args.grad + args.dirs + args.train > 1:
        print("--conv, --grad, --train and --dirs are separate measurements", file=sys.stderr)
        sys.exit(2)
    if args.chunks is not None and (wl.kind != "vim" or args.conv or args.grad or args.dirs
                                    or args.zoh or args.train):
        print("--chunks applies to the plain Vim scan", file=sys.stderr)
        sys.exit(2)
    if args.zoh and (args.grad or args.train):
        print("the gradient uses the delta B form; --zoh is a forward option", file=sys.stderr)
        sys.exit(2)
    backward = args.grad or args.train
    tdt = torch.bfloat16 if wl.dtype == wlm.BF16 else torch.float32
    print("bench: workload %s" % wl.name, file=sys.stderr, flush=True)

    inp = wlm.make_inputs(wl)

    def up(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)

    set_bytes = wl.algorithmic_bytes() + (wl.tokens_channels * 4 if wl.dtype == wlm.BF16 else 0)
    nsets = args.sets or max(1, int(np.ceil(768e6 / set_bytes)))
    sets = []
    base = dict(u=up(inp.u, tdt), delta=up(inp.delta, tdt), z=up(inp.z, tdt), B=up(inp.B, tdt),
                C=up(inp.C, tdt), A=up(inp.A, torch.float32), D=up(inp.D, torch.float32),
                bias=up(inp.dt_bias, torch.float32))
    if backward:
        grng = np.random.default_rng(wl.seed + 600)
        gy = grng.standard_normal(inp.u.shape).astype(np.float32)
        base["dy"] = up(wlm.round_bf16(gy) if wl.dtype == wlm.BF16 else gy, tdt)
    if args.dirs:
        # the backward direction's copies from a second draw of the recipe
        other = wlm.make_inputs(wl, seed=wl.seed + 1)
        base["u"] = torch.stack([base["u"], up(other.u, tdt)]).contiguous()
        base["delta"] = torch.stack([base["delta"], up(other.delta, tdt)]).contiguous()
        base["B"] = torch.stack([base["B"], up(other.B, tdt)], 1).contiguous()
        base["C"] = torch.stack([base["C"], up(other.C, tdt)], 1).contiguous()
    if args.conv:
        crng = np.random.default_rng(wl.seed + 500)
        base["cw"] = up((0.6 * crng.standard_normal((2, wl.dim, 3))).astype(np.float32),
                        torch.float32)
        base["cb"] = up((0.2 * crng.standard_normal((2, wl.dim))).astype(np.float32),
                        torch.float32)
    for s in range(nsets):
        t = {k: (None if v is None else (v if s == 0 else v.clone())) for k, v in base.items()}
        t["y"] = torch.empty(wl.batch, wl.dim, wl.seqlen, dtype=tdt, device=dev)
        t["ws"] = None
        op = 3 if args.grad else (5 if args.train else (0 if wl.kind == "vim" else 1))
        need = vms.workspace_bytes(op, wl.batch, wl.dim, wl.seqlen, tdt)
        if need:
            t["ws"] = torch.empty(need, dtype=torch.uint8, device=dev)
        if args.train:
            t["saved"] = torch.empty(vms.workspace_bytes(4, wl.batch, wl.dim, wl.seqlen, tdt),
                                     dtype=torch.uint8, device=dev)
        sets.append(t)

    if backward:
        for t in sets:
            t["g"] = dict(du=torch.empty_like(t["u"]), ddelta=torch.empty_like(t["u"]),
                          dz=None if t["z"] is None else torch.empty_like(t["u"]),
                          dB=torch.empty(wl.batch, wl.dstate, wl.seqlen, device=dev),
                          dC=torch.empty(wl.batch, wl.dstate, wl.seqlen, device=dev),
                          dA=torch.empty(2, wl.dim, wl.dstate, device=dev),
                          dD=torch.empty(2, wl.dim, device=dev),
                          db=torch.empty(2, wl.dim, device=dev))
        from vision_mamba_selective_amd import _native as nat

        def grad_call(t):
            g = t["g"]
            p = lambda x: None if x is None else x.data_ptr()
            rc = nat.lib.vim_scan_bidir_grad(
                wl.batch, wl.dim, wl.dstate, wl.seqlen, nat.VS_BF16 if wl.dtype == wlm.BF16
                else nat.VS_F32, p(t["u"]), p(t["delta"]), p(t["z"]), p(t["B"]), p(t["C"]),
                p(t["A"]), p(t["D"]), p(t["bias"]), 1, p(t["dy"]), p(g["du"]), p(g["ddelta"]),
                p(g["dz"]), p(g["dB"]), p(g["dC"]), p(g["dA"]), p(g["dD"]), p(g["db"]),
                p(t["ws"]), t["ws"].numel(), torch.cuda.current_stream(dev).cuda_stream)
            nat.check("vim_scan_bidir_grad", rc)

        def train_call(t):
            g = t["g"]
            p = lambda x: None if x is None else x.data_ptr()
            dtc = nat.VS_BF16 if wl.dtype == wlm.BF16 else nat.VS_F32
            st = torch.cuda.current_stream(dev).cuda_stream
            ins = (p(t["u"]), p(t["delta"]), p(t["z"]), p(t["B"]), p(t["C"]), p(t["A"]), p(t["D"]),
                   p(t["bias"]), 1)
            rc = nat.lib.vim_scan_bidir_fwd_saved(wl.batch, wl.dim, wl.dstate, wl.seqlen, dtc, *ins,
                                                  p(t["y"]), p(t["saved"]), t["saved"].numel(), st)
            nat.check("vim_scan_bidir_fwd_saved", rc)
            rc = nat.lib.vim_scan_bidir_grad_saved(
                wl.batch, wl.dim, wl.dstate, wl.seqlen, dtc, *ins, p(t["saved"]), t["saved"].numel(),
                p(t["dy"]), p(g["du"]), p(g["ddelta"]), p(g["dz"]), p(g["dB"]), p(g["dC"]), p(g["dA"]),
                p(g["dD"]), p(g["db"]), p(t["ws"]), t["ws"].numel(), st)
            nat.check("vim_scan_bidir_grad_saved", rc)

    def step(t):
        if args.grad:
            grad_call(t)
        elif args.train:
            train_call(t)
        elif args.conv:
            vms.vim_scan_bidir_conv(t["u"], t["cw"], t["cb"], t["delta"], t["z"], t["B"], t["C"],
                                    t["A"], t["D"], t["bias"], out=t["y"], workspace=t["ws"],
                                    zoh=args.zoh)
        elif args.dirs:
            vms.vim_scan_bidir_dirs(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["D"],
                                    t["bias"], out=t["y"], workspace=t["ws"], zoh=args.zoh)
        elif wl.kind == "vim" and args.chunks is not None:
            vms.vim_scan_bidir_chunked(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["D"],
                                       t["bias"], chunks=args.chunks, out=t["y"],
                                       workspace=t["ws"])
        elif wl.kind == "vim":
            vms.vim_scan_bidir(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["D"],
                               t["bias"], out=t["y"], workspace=t["ws"], zoh=args.zoh)
        else:
            vms.vmamba_cross_scan4(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], wl.H, wl.W,
                                   t["D"], t["bias"], out=t["y"], workspace=t["ws"], zoh=args.zoh)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    print("bench: warmup done, timing %d steps over %d input sets" % (args.steps, nsets),
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def eager_steps():
        """K steps launched one by one, each between two HIP events."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(sets[i % nsets])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, [a.elapsed_time(b) for a, b in ev]

    if args.eager:
        wall, kern_ms = eager_steps()
        kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    else:
        # The K timed steps are captured once in a HIP graph (the entry points
        # allocate nothing and launch only kernels) and replayed in one launch
        # between two synchronizations; one untimed replay comes first.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(sets[i % nsets])
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del graph
        # each launch's own duration (for the roofline and the spread), from
        # K more steps launched one by one between event pairs: the replay's
        # duration over K is slightly shorter, since consecutive kernels of
        # the graph overlap a little
        _, kern_ms = eager_steps()
        kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    ms_per_step = wall * 1e3 / args.steps
    copy_gbs = copy_ceiling(torch, dev)

    tc = wl.tokens_channels
    value = tc / (ms_per_step * 1e-3) / 1e9
    alg_bytes = wl.grad_algorithmic_bytes() if args.grad else wl.algorithmic_bytes()
    if args.train:
        alg_bytes = wl.algorithmic_bytes() + wl.grad_algorithmic_bytes()
    if args.dirs:   # the second copies of u, delta, B and C
        alg_bytes += 2 * tc * wl.act_bytes + 2 * wl.batch * wl.dstate * wl.seqlen * wl.act_bytes
    hbm_gbs = alg_bytes / kern_avg_s / 1e9
    updates = wl.state_updates
    upd_rate = updates / kern_avg_s
    flops_per_update = GRAD_FLOPS_PER_UPDATE if args.grad else FLOPS_PER_UPDATE
    slots_per_update = GRAD_SLOTS_PER_UPDATE if args.grad else SLOTS_PER_UPDATE
    if args.train:      # the forward's arithmetic and the gradient's, per update
        flops_per_update = FLOPS_PER_UPDATE + GRAD_FLOPS_PER_UPDATE
        slots_per_update = SLOTS_PER_UPDATE + GRAD_SLOTS_PER_UPDATE
    tflops = flops_per_update * upd_rate / 1e12
    upd_peak = LANE_SLOTS / slots_per_update

    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        try:
            with open(PROFILE_TRAFFIC) as f:
                tr = json.load(f)
            rec = tr.get(wl.name + ("+conv" if args.conv else "") + ("+grad" if args.grad else "")
                         + ("+train" if args.train else "")
                         + ("+dirs" if args.dirs else "") + ("+zoh" if args.zoh else ""))
            if rec and rec.get("kernel_sha") == kernel_hash():
                traffic = rec.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    out = {
        "metric": "selective-scan Gtoken*ch/s + achieved HBM GB/s (Vim-S, 1024^2, bidir)",
        "value": round(value, 3),
        "unit": "Gtoken*ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == wlm.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "kind": wl.kind, "batch": wl.batch, "d_inner": wl.dim,
                   "d_state": wl.dstate, "seq_len": wl.seqlen, "directions": wl.ndir,
                   "state_dtype": "f32", "input_sets_rotated": nsets,
                   "front_end": "conv1d k3 + silu, fused" if args.conv else "none",
                   "pass": ("gradient (forward recompute + adjoint)" if args.grad else
                            ("training step (saving forward + gradient from the saved states)"
                             if args.train else "forward")),
                   "discretization": "exact zero-order hold" if args.zoh else "delta B",
                   "inputs": "per-direction u, delta, B, C" if args.dirs else "shared",
                   "chunks": "library's choice" if args.chunks in (None, 0) else args.chunks,
                   "launch": "one by one" if args.eager else "one HIP graph of the timed steps"},
        "hbm_GBps": round(hbm_gbs, 1),
        "kernel_ms": round(kern_avg_s * 1e3, 5),
        # the arithmetic rate against the published fp32 vector peak
        "roofline": {
            "bound": "alu",
            "achieved": round(tflops, 3),
            "peak": FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / FP32_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_update": flops_per_update,
        },
        # the same rate against the issue-slot ceiling derived from the unit
        # counts for non-packed fp32 VALU code (exp in 2 slots)
        "roofline_issue": {
            "achieved": round(upd_rate / 1e12, 4),
            "peak": round(upd_peak / 1e12, 4),
            "unit": "Tupdate/s",
            "frac": round(upd_rate / upd_peak, 4),
            "slots_per_update": round(slots_per_update, 4),
            "lane_slots_per_s": LANE_SLOTS,
            "clock_hz": CLOCK_HZ,
        },
        "kernel_ms_p10_p50_p90": [round(float(v), 5) for v in np.percentile(kern_ms, [10, 50, 90])],
        "roofline_hbm": {
            "bound": "hbm",
            "achieved": round(hbm_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": alg_bytes,
            "copy_ceiling": round(copy_gbs, 1),
            "frac_of_copy": round(hbm_gbs / copy_gbs, 4),
        },
    }
    if not args.no_cpu_baseline:
        conv = None
        if args.conv:
            conv = (base["cw"].cpu().numpy(), base["cb"].cpu().numpy())
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_channels, conv,
                                           base["dy"].float().cpu().numpy() if backward else None,
                                           zoh=args.zoh, dirs=args.dirs, train=args.train,
                                           min_seconds=args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, inp, nch, conv=None, dy=None, zoh=False, dirs=False, train=False,
                 min_seconds=10.0):
    """The fp64 oracle, as it stands, on the host cores of this machine: the
    sample is run again until min_seconds have passed (at least once), and
    the rate is the work of all runs over their total time."""
    import numpy as np
    import oracle
    from vision_mamba_selective_amd import workloads as wlm

    sample = inp
    desc = "whole workload (%d x %d x %d)" % (wl.batch, wl.dim, wl.seqlen)
    if nch:
        sample = wlm.channel_subset(inp, list(range(wl.batch)), list(range(min(nch, wl.dim))))
        desc = "%d of %d channels of every batch row" % (sample.wl.dim, wl.dim)
    threads = oracle.default_threads()
    print("bench: cpu baseline on %s with %d threads" % (desc, threads), file=sys.stderr,
          flush=True)
    oracle.load()
    if train:
        desc += ", forward then gradient"
    runs = 0
    t0 = time.perf_counter()
    while True:
        run_oracle_once(wl, sample, nch, conv, dy, zoh, dirs, train, threads)
        runs += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(runs * sample.wl.tokens_channels / dt / 1e9, 5), "unit": "Gtoken*ch/s",
            "cores": threads, "kind": "oracle", "seconds": round(dt, 3), "runs": runs,
            "sample": "%s, %d run%s, fp64, %s, %s" % (desc, runs, "" if runs == 1 else "s", cpu,
                                                      platform.machine())}


def run_oracle_once(wl, sample, nch, conv, dy, zoh, dirs, train, threads):
    """One pass of the oracle over the sample (the call the bench times)."""
    import numpy as np
    import oracle
    from vision_mamba_selective_amd import workloads as wlm
    if train:       # the forward, then the gradient
        oracle.run_inputs(sample, nthreads=threads)
    if dy is not None:
        gy = dy[:sample.wl.batch, :sample.wl.dim]
        oracle.vim_bidir_grad(sample.u, sample.delta, sample.z, sample.B, sample.C, sample.A,
                              sample.D, sample.dt_bias, np.ascontiguousarray(gy),
                              nthreads=threads)
    elif dirs:
        other = wlm.make_inputs(wl, seed=wl.seed + 1)
        if nch:
            other = wlm.channel_subset(other, list(range(wl.batch)), list(range(sample.wl.dim)))
        oracle.vim_dirs(np.stack([sample.u, other.u]), np.stack([sample.delta, other.delta]),
                        sample.z, np.stack([sample.B, other.B], 1),
                        np.stack([sample.C, other.C], 1), sample.A, sample.D, sample.dt_bias,
                        nthreads=threads, zoh=zoh)
    elif conv is None:
        oracle.run_inputs(sample, nthreads=threads, zoh=zoh)
    else:
        w, b = conv
        ch = list(range(sample.wl.dim))
        oracle.vim_conv(sample.u, w[:, ch], b[:, ch], sample.delta, sample.z, sample.B, sample.C,
                        sample.A, sample.D, sample.dt_bias, nthreads=threads, zoh=zoh)


def proj_bench(args, torch, dev):
    """The projections at the workload's shape. One step is out_proj: y
    [batch, dim, L] -> W [dim, dim] y + bias + residual (bf16, matrix cores);
    x_proj (dim -> 2 dstate + 1) and dt_proj are timed beside it."""
    import numpy as np
    import vision_mamba_selective_amd as vms
    from vision_mamba_selective_amd import workloads as wlm

    idx = wlm.HEADLINE if args.workload is None else args.workload
    wl = wlm.WORKLOADS[idx]
    if wl.kind != "vim" or wl.dtype != wlm.BF16:
        print("--proj applies to the bf16 Vim workloads", file=sys.stderr)
        sys.exit(2)
    print("bench: projections at %s" % wl.name, file=sys.stderr, flush=True)
    rng = np.random.default_rng(wl.seed + 700)
    bf = torch.bfloat16
    dim, L, batch, N = wl.dim, wl.seqlen, wl.batch, wl.dstate

    def w(shape, scale):
        return torch.from_numpy(wlm.round_bf16(scale * rng.standard_normal(shape))).to(dev).to(bf)

    Wo, Wx = w((dim, dim), dim ** -0.5), w((2 * N + 1, dim), dim ** -0.5)
    bias = torch.from_numpy(rng.standard_normal(dim).astype(np.float32)).to(dev)
    wdt = torch.from_numpy(rng.standard_normal(dim).astype(np.float32)).to(dev)
    y0 = w((batch, dim, L), 1.0)
    r0 = w((batch, dim, L), 1.0)
    per_set = 3 * y0.numel() * 2
    nsets = args.sets or max(1, int(np.ceil(768e6 / per_set)))
    sets = [dict(y=y0 if s == 0 else y0.clone(), r=r0 if s == 0 else r0.clone(),
                 o=torch.empty_like(y0)) for s in range(nsets)]

    def step(t):
        vms.vim_out_proj(t["y"], Wo, bias, t["r"], out=t["o"])

    stream = torch.cuda.current_stream(dev)

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    print("bench: warmup done, timing %d steps over %d input sets" % (args.steps, nsets),
          file=sys.stderr, flush=True)
    if args.eager:
        t0 = time.perf_counter()
        kern_ms = timed(lambda i: step(sets[i % nsets]), args.steps)
        wall = time.perf_counter() - t0
    else:
        # the timed out_proj steps replay as one HIP graph (see main())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(sets[i % nsets])
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del graph
        # each launch's own duration, from one-by-one launches (see main())
        kern_ms = timed(lambda i: step(sets[i % nsets]), args.steps)
    ms_per_step = wall * 1e3 / args.steps
    # x_proj and dt_proj, each timed on its own
    x_ms = timed(lambda i: vms.vim_x_proj(sets[i % nsets]["y"], Wx, N), args.steps)
    _, _, dt = vms.vim_x_proj(y0, Wx, N)
    d_ms = timed(lambda i: vms.vim_dt_proj(dt, wdt), args.steps)

    copy_gbs = copy_ceiling(torch, dev)
    flops = 2.0 * batch * dim * dim * L
    tflops = flops / (kern_ms * 1e-3) / 1e12
    alg_bytes = 3 * batch * dim * L * 2 + dim * dim * 2 + dim * 4   # y, residual, out, W, bias
    hbm_gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
    tc = batch * dim * L
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        try:
            with open(PROFILE_TRAFFIC) as f:
                rec = json.load(f).get(wl.name + "+proj")
            if rec and rec.get("kernel_sha") == kernel_hash(PROJ_SRC):
                traffic = rec.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    out = {
        "metric": "selective-scan Gtoken*ch/s + achieved HBM GB/s (Vim-S, 1024^2, bidir)",
        "value": round(tc / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gtoken*ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "kind": "vim", "batch": batch, "d_inner": dim,
                   "d_state": N, "seq_len": L,
                   "pass": "out_proj %d->%d + bias + residual (matrix cores)" % (dim, dim),
                   "launch": "one by one" if args.eager else "one HIP graph of the timed steps"},
        "kernel_ms": round(kern_ms, 5),
        "x_proj_ms": round(x_ms, 5),
        "dt_proj_ms": round(d_ms, 5),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic},
        "roofline_hbm": {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": alg_bytes, "copy_ceiling": round(copy_gbs, 1),
                         "frac_of_copy": round(hbm_gbs / copy_gbs, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = proj_cpu_baseline(sets[0]["y"], Wo, bias, sets[0]["r"])
    print(json.dumps(out), flush=True)


def proj_cpu_baseline(y, W, bias, r, tokens=256):
    """The fp64 oracle's linear map (single-threaded loops) on every batch row
    and the first `tokens` tokens of out_proj."""
    import oracle
    ys = y[:, :, :tokens].float().cpu().numpy()
    rs = r[:, :, :tokens].float().cpu().numpy()
    Wn, bn = W.float().cpu().numpy(), bias.cpu().numpy()
    oracle.load()
    t0 = time.perf_counter()
    oracle.linear(Wn, ys, bn, rs)
    dt = time.perf_counter() - t0
    tc = ys.shape[0] * W.shape[0] * ys.shape[2]
    return {"value": round(tc / dt / 1e9, 6), "unit": "Gtoken*ch/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "out_proj on %d batch rows x %d tokens, fp64, %s" % (
                ys.shape[0], ys.shape[2], platform.machine())}


def copy_ceiling(torch, dev, nbytes=512 << 20, reps=10):
    """Measured HBM ceiling: GB/s (bytes read + written) of a plain device
    copy of nbytes, timed with HIP events after one untimed copy."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    e1.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return gbs


def copy_probe(torch, dev):
    """Plain copies of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters (a copy of N bytes reads N and writes N)."""
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


if __name__ == "__main__":
    main()
