#!/usr/bin/env python
"""Throughput of one DSpark decode cycle (draft -> schedule -> verify) on one MI355X.

A step is one whole cycle of the hot path on the headline workload (R=256 requests, gamma=8
draft positions, V=151936, r=256, d=4096, bf16 operands with fp32 softmax):
  dspark_draft_markov  (gamma vocabulary sweeps + combines)
  dspark_schedule      (Algorithm 1 with the early-stop break)
  dspark_verify        (rejection sampling of the scheduled prefixes, c*; it also writes
                        each request's last emitted token, the next cycle's anchor, into
                        the x0 the next draft call reads)
All inputs are seeded synthetic tensors already resident in device memory.  Cycle t uses
random-counter cycle t and the anchors cycle t-1 emitted, so the drafted tokens and the
scheduled lengths change from cycle to cycle.  The target logits that verification reads are
a synthetic stand-in for the target model (the drafted logits plus noise, plus a fresh bonus
row), built for every cycle on an untimed first pass over the same chain of cycles; the
timed pass reproduces that chain token for token (checked).

Printed: one JSON line with the metric, the roofline of the dominant kernel (the draft
sweep, timed live with HIP events attached to its launches), the read rate a kernel that only
reads sustains on the same bytes (dspark_read_probe, the practical ceiling beside the
published peak), and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
METRIC = "draft+verify tokens/s at R=256 γ=8 V=151936; % of HBM roofline"
SEED = 0
CYCLE = 1


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3", help="workload: c3 (headline) or c2")
    ap.add_argument("--workload", default="cycle",
                    choices=("cycle", "train", "sts", "decode", "rnn"),
                    help="cycle: the decode cycle (default); train: the training-objective "
                         "forward on teacher-forced blocks; sts: the STS calibration fit; "
                         "decode: the multi-cycle driver on a toy chain; rnn: the RNN-head "
                         "draft at R=256, gamma=16, V=129280")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run a 512 MiB device copy (byte-counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="reduce two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE; taken with --copy-probe) to the sweep's HBM bytes per "
                         "launch, write them under profiles/ and exit")
    return ap.parse_args()


def hip_events(n):
    hip = C.CDLL("libamdhip64.so.7")  # the runtime PyTorch already loaded
    hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    arr = (C.c_void_p * n)()
    for i in range(n):
        ev = C.c_void_p()
        if hip.hipEventCreate(C.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        arr[i] = ev
    return hip, arr


def elapsed_ms(hip, a, b) -> float:
    ms = C.c_float()
    if hip.hipEventElapsedTime(C.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


def make_target(torch, cfg, U, W2t, d, gen):
    """Synthetic target-model stand-in: drafted logits + N(0, s^2) noise for rows 1..gamma,
    a fresh Zipf-ranked row + noise for the bonus row (built on the device, untimed)."""
    R, G, V = cfg.R, cfg.gamma, cfg.V
    noise = cfg.target_noise
    tgt = torch.empty((R, G + 1, V), dtype=torch.bfloat16, device=U.device)
    W2f = W2t.float().t().contiguous()  # [r][V]
    base = -1.1 * torch.log(torch.arange(1, V + 1, device=U.device, dtype=torch.float32))
    for q0 in range(0, R, 32):
        q1 = min(R, q0 + 32)
        br = d["bias_rows"][q0:q1].float()                          # [n, G, r]
        logits = U[q0:q1].float() + torch.matmul(br, W2f)           # [n, G, V]
        logits += noise * torch.randn(logits.shape, device=U.device, generator=gen)
        tgt[q0:q1, :G] = logits.to(torch.bfloat16)
        fresh = torch.stack([base[torch.randperm(V, device=U.device, generator=gen)]
                             for _ in range(q1 - q0)])
        fresh += torch.randn(fresh.shape, device=U.device, generator=gen)
        fresh += noise * torch.randn(fresh.shape, device=U.device, generator=gen)
        tgt[q0:q1, G] = fresh.to(torch.bfloat16)
    return tgt


def cpu_baseline(cfg, I, target_seconds):
    """The oracle, untuned, on the host cores: draft + schedule + verify of a sample of the
    workload's requests (the first S, same inputs), timed wall-clock."""
    import numpy as np

    import oracle
    from draft_sampling_scheduling_amd import synth

    oracle.lib()
    threads = oracle.num_threads()
    W2 = I["W2"]

    targets = {}

    def run(S):
        reqs = np.arange(S)
        U = I["U"][:S]
        h = I["h"][:S]
        t0 = time.perf_counter()
        d = oracle.draft_markov(U, h, I["W1"], W2, I["w"], I["x0"][:S], SEED, CYCLE,
                                req_ids=reqs)
        t_draft = time.perf_counter() - t0
        sps = (1.0 / (1.0 + cfg.sps_alpha * np.arange(S, S * (cfg.gamma + 1) + 1))).astype(np.float32)
        t0 = time.perf_counter()
        s = oracle.schedule(d["c"].astype(np.float32), sps, S, oracle.SYNC_BREAK)
        t_sched = time.perf_counter() - t0
        # target stand-in for the sample (untimed; the same drafted tokens on every repeat)
        if S not in targets:
            logits = synth.decode(cfg, U).astype(np.float64)
            logits += np.einsum("qkr,rv->qkv", d["bias_rows"],
                                synth.decode(cfg, W2).astype(np.float64))
            noise, fresh = synth.target_parts(cfg, range(S), CYCLE)
            targets.clear()
            targets[S] = synth.encode(cfg, (np.concatenate([logits, fresh[:, None, :]], axis=1)
                                            + noise).astype(np.float32))
            del logits, noise
        tgt = targets[S]
        t0 = time.perf_counter()
        oracle.verify(tgt, U, W2, d["bias_rows"], d["x"], s["ell"], SEED, CYCLE, req_ids=reqs)
        t_verify = time.perf_counter() - t0
        return t_draft + t_sched + t_verify, int(s["ell"].sum())

    # calibrate on one request per thread, then size the sample for the target wall time;
    # when the whole workload takes less, repeat it (same inputs) until the target is met
    t1, _ = run(threads)
    S = int(threads * max(1.0, target_seconds / max(t1, 1e-3)))
    S = max(threads, min(cfg.R, (S // threads) * threads))
    t, reps = 0.0, 0
    while reps == 0 or (S == cfg.R and t < target_seconds):
        dt, _ = run(S)
        t += dt
        reps += 1
    # the same oracle on one thread: single requests, repeated for a few seconds
    oracle.set_num_threads(1)
    t1, reps1 = 0.0, 0
    try:
        while reps1 == 0 or t1 < min(3.0, target_seconds / 4):
            dt, _ = run(1)
            t1 += dt
            reps1 += 1
    finally:
        oracle.set_num_threads(threads)
    return dict(value=reps * S * cfg.gamma / t, unit="drafted tokens/s", cores=threads,
                kind="oracle",
                sample=f"{reps} x the first {S} of {cfg.R} requests of the same workload: draft "
                       f"(gamma={cfg.gamma}, V={cfg.V}, fp64), schedule (early stop) and verify; "
                       f"{t:.1f} s wall (target stand-in built untimed)",
                value_1thread=reps1 * cfg.gamma / t1,
                sample_1thread=f"{reps1} x request 0 on one thread, {t1:.1f} s wall",
                cpu_model=cpu_model(), nproc=len(os.sched_getaffinity(0)))


def read_probe_rate(torch, ds, dev, nbytes: int):
    """(GB/s, grid, bytes) of dspark_read_probe: the best median over grid sizes of reads of
    nbytes from four rotated buffers (4 x nbytes above the 256 MB last-level cache, so every
    read finds its bytes in HBM only)."""
    import numpy as np

    n16 = (nbytes + 15) // 16 * 16
    bufs = [torch.zeros(n16 // 4, dtype=torch.int32, device=dev) for _ in range(4)]
    hip, ev = hip_events(2)  # attached to the probe's dispatch, as for the sweep
    best, k = (0.0, 0, n16), 0
    for grid in (1024, 2048, 4096):
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        rates = []
        for _ in range(7):
            ds.read_probe(bufs[k % 4], grid, sink=sink, events=(ev[0], ev[1]))
            torch.cuda.synchronize()
            k += 1
            rates.append(n16 / (elapsed_ms(hip, ev[0], ev[1]) * 1e-3) / 1e9)
        med = float(np.median(rates))
        if med > best[0]:
            best = (med, grid, n16)
    del bufs
    return best


def sweep_bytes_of(R: int, V: int, r: int) -> int:
    """Algorithmic bytes of one draft sweep: U_k rows, all of W2, the gathered W1 rows."""
    return R * V * 2 + V * r * 2 + R * r * 2


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


COPY_PROBE_BYTES = 1 << 29
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "draft_sweep_c3_traffic.json")


def traffic_from(fetch_csv: str, write_csv: str) -> None:
    """HBM bytes per draft-sweep launch from the FETCH_SIZE and WRITE_SIZE counters (KiB
    per dispatch), each scaled so that the 512 MiB copy of the same run reads its true
    size (the copy reads and writes COPY_PROBE_BYTES)."""
    import csv

    def per_kernel(path, counter):
        sweep, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "DraftEpi<false, true>" in r["Kernel_Name"]:
                sweep.append(v)
            elif "copyBuffer" in r["Kernel_Name"] and v > COPY_PROBE_BYTES / 1024 / 8:
                copy.append(v)
        if not sweep or not copy:
            raise SystemExit(f"{path}: no {counter} rows for the draft sweep and the copy probe")
        copy = [v for v in copy if v >= 0.9 * max(copy)]  # the probe copies are the largest
        return sum(sweep) / len(sweep), sum(copy) / len(copy), len(sweep)

    f_sweep, f_copy, n = per_kernel(fetch_csv, "FETCH_SIZE")
    w_sweep, w_copy, _ = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = COPY_PROBE_BYTES / 1024 / f_copy
    w_scale = COPY_PROBE_BYTES / 1024 / w_copy
    out = {
        "kernel": "draft sweep (sweep_kernel<16, false, 2, DraftEpi<false, true>>), R=256 V=151936 r=256",
        "kernel_source_sha": kernel_sha(),
        "dispatches": n,
        "fetch_kib_per_dispatch": f_sweep, "write_kib_per_dispatch": w_sweep,
        "copy_probe_bytes": COPY_PROBE_BYTES,
        "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "bytes_per_launch": (f_sweep * f_scale + w_sweep * w_scale) * 1024,
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the path as one GPU runs its share of a batch); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.workload == "train":
        return bench_train(args)
    if args.workload == "sts":
        return bench_sts(args)
    if args.workload == "decode":
        return bench_decode(args)
    if args.workload == "rnn":
        return bench_rnn(args)
    return bench_cycle(args)


def bench_cycle(args):
    """The decode cycle, advanced as the method runs it: cycle t drafts from the anchors
    that cycle t-1 emitted (its last token per request), with random-counter cycle t; the
    target stand-in of every cycle is built beforehand (untimed) on a first pass over the
    same cycles, and the timed pass must reproduce that pass's emitted tokens exactly."""
    import numpy as np
    import torch

    import draft_sampling_scheduling_amd as ds
    from draft_sampling_scheduling_amd import synth

    ds.lib()  # fails loudly if the HIP library is missing
    cfg = synth.CONFIGS[args.config]
    if cfg.head != "markov" or cfg.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 Markov-head workloads (c2, c3)")
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    I = synth.inputs(cfg)

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    U, h, W1, w, x0_first = T(I["U"]), T(I["h"]), T(I["W1"]), T(I["w"]), T(I["x0"])
    W2t = ds.w2_relayout(T(I["W2"]))  # the pages' [r][V] -> [V][r]
    sps = T(synth.sps_table(cfg))
    R, G, V, r, d = cfg.R, cfg.gamma, cfg.V, cfg.r, cfg.d
    gen_s = time.perf_counter() - t_gen
    log(f"inputs of {cfg.name} resident on the device ({gen_s:.1f} s)")

    # outputs and workspaces allocated once
    dout = dict(x=torch.empty((R, G), dtype=torch.int32, device=dev),
                c=torch.empty((R, G), dtype=torch.float32, device=dev),
                lse=torch.empty((R, G), dtype=torch.float32, device=dev),
                logit_x=torch.empty((R, G), dtype=torch.float32, device=dev),
                bias_rows=torch.empty((R, G, r), dtype=torch.bfloat16, device=dev))
    sout = dict(ell=torch.empty(R, dtype=torch.int32, device=dev),
                a=torch.empty((R, G), dtype=torch.float32, device=dev),
                stats=torch.empty(4, dtype=torch.float64, device=dev))
    vout = dict(n_acc=torch.empty(R, dtype=torch.int32, device=dev),
                y=torch.empty((R, G + 1), dtype=torch.int32, device=dev),
                c_star=torch.empty((R, G), dtype=torch.float32, device=dev))
    dws = torch.empty(ds.draft_workspace_bytes(R, G, V, r, d), dtype=torch.uint8, device=dev)
    vws = torch.empty(ds.verify_workspace_bytes(R, G, V, r), dtype=torch.uint8, device=dev)
    sws = torch.empty(ds.schedule_workspace_bytes(R, G), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    x0 = torch.empty_like(x0_first)
    # verification writes every request's last emitted token, the next cycle's anchor,
    # straight into the draft's x0
    vout["x_next"] = x0

    nsteps = args.warmup + args.steps
    # one sweep launch per cycle is bracketed by events (draft position k = cycle mod gamma,
    # so every position is sampled); the other positions run unbracketed
    hip, evs = hip_events(2 * nsteps)

    # one sweep launch per cycle is bracketed by events (draft position k = cycle mod gamma,
    # so every position is sampled); the other positions run unbracketed
    def ev_arrays(i):
        k = i % G
        evb, eve = (C.c_void_p * G)(), (C.c_void_p * G)()
        evb[k], eve[k] = evs[2 * i], evs[2 * i + 1]
        return evb, eve

    ev_args = [ev_arrays(i) for i in range(nsteps)]

    # first pass (untimed): the chain of cycles, each cycle's target stand-in built for the
    # tokens it drafted; the emitted tokens are kept to check the timed pass
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    targets, emitted_ref, ells = [], [], []
    x0.copy_(x0_first)
    for t in range(nsteps):
        ds.draft_markov(U, h, W1, W2t, w, x0, SEED, t, out=dout, ws=dws, status=status)
        targets.append(make_target(torch, cfg, U, W2t, dout, gen))
        ds.schedule(dout["c"], sps, cfg.sps_B0, ds.SYNC_BREAK, out=sout, ws=sws, status=status)
        ds.verify(targets[t], U, W2t, dout["bias_rows"], dout["x"], dout["lse"],
                  dout["logit_x"], sout["ell"], SEED, t, out=vout, ws=vws, status=status)
        emitted_ref.append(vout["y"].clone())
        ells.append(sout["ell"].clone())
    torch.cuda.synchronize()
    log(f"{nsteps} cycles drafted once and their target stand-ins built")

    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nsteps)]

    def cycle(t):
        e = sev[t]
        e[0].record()
        ds.draft_markov(U, h, W1, W2t, w, x0, SEED, t, out=dout, ws=dws, status=status,
                        events=ev_args[t])
        e[1].record()
        ds.schedule(dout["c"], sps, cfg.sps_B0, ds.SYNC_BREAK, out=sout, ws=sws, status=status)
        e[2].record()
        ds.verify(targets[t], U, W2t, dout["bias_rows"], dout["x"], dout["lse"],
                  dout["logit_x"], sout["ell"], SEED, t, out=vout, ws=vws, status=status)
        e[3].record()

    x0.copy_(x0_first)
    for t in range(args.warmup):
        cycle(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, nsteps):
        cycle(t)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"{args.steps} timed cycles: {wall * 1e3 / args.steps:.3f} ms each")
    if int(status.item()) != 0:
        raise SystemExit(f"device fault bits set: {int(status.item())}")
    # the last timed cycle reproduces the first pass (same anchors, seeds and counters)
    if not torch.equal(vout["y"], emitted_ref[-1]):
        raise SystemExit("the timed cycles did not reproduce the first pass's tokens")
    timed = range(args.warmup, nsteps)
    kern_ms = float(np.mean([elapsed_ms(hip, evs[2 * i], evs[2 * i + 1]) for i in timed]))

    # the cost of the sequential head: the same draft without it (the parallel block's own
    # sampling from U_k), timed on the same inputs after the cycles
    def draft_time(fn, n=10):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(n):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n
    x0.copy_(x0_first)
    t_markov = draft_time(lambda: ds.draft_markov(U, h, W1, W2t, w, x0, SEED, 0, out=dout,
                                                  ws=dws, status=status))
    t_parallel = draft_time(lambda: ds.draft_parallel(U, h, W1, w, x0, SEED, 0, out=dout,
                                                      ws=dws, status=status))
    t_draft = float(np.mean([sev[t][0].elapsed_time(sev[t][1]) for t in timed]))
    t_sched = float(np.mean([sev[t][1].elapsed_time(sev[t][2]) for t in timed]))
    t_ver = float(np.mean([sev[t][2].elapsed_time(sev[t][3]) for t in timed]))
    cycle_median = float(np.median([sev[t][0].elapsed_time(sev[t][3]) for t in timed]))
    ell_all = torch.stack([ells[t] for t in timed]).cpu().numpy()

    # a plain device copy of the sweep's byte count (read + write), the practical HBM rate
    # beside the spec peak; outside the timed region (not in counter runs, whose copies are
    # the scaling probe)
    copy_gbs = None
    if not args.copy_probe:
        cbuf = torch.empty(sweep_bytes_of(R, V, r) // 2, dtype=torch.bfloat16, device=dev)
        cdst = torch.empty_like(cbuf)
        cdst.copy_(cbuf)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ce[0].record()
        for _ in range(10):
            cdst.copy_(cbuf)
        ce[1].record()
        torch.cuda.synchronize()
        copy_gbs = 2 * cbuf.numel() * 2 * 10 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
        del cbuf, cdst
    # the rate of a kernel that only reads (dspark_read_probe) on the sweep's byte count:
    # the practical ceiling for a read-bound kernel beside the published peak
    read_probe = None
    if not args.copy_probe:
        read_probe = read_probe_rate(torch, ds, dev, sweep_bytes_of(R, V, r))
    if args.copy_probe:
        # a plain device copy of known size, for scaling the HBM byte counters
        a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 3 device copies of 512 MiB")
    ms_per_step = wall * 1000.0 / args.steps
    n_acc_sum = sum(int((emitted_ref[t] >= 0).sum()) for t in timed)  # emitted tokens

    # the Markov step (gather, bias contraction, logits, normaliser, sample, confidence) per
    # position: U_k, W2, h_k and the gathered W1 rows; gamma positions per cycle
    step_bytes = R * V * 2 + V * r * 2 + R * d * 2 + R * r * 2
    draft_bytes = G * step_bytes
    # the timed kernel: one vocabulary sweep, U_k rows, all of W2, the gathered W1 rows
    kern_bytes = sweep_bytes_of(R, V, r)
    kern_name = f"draft sweep (sweep_kernel<{r // 16}, false, 2, DraftEpi<false, true>>)"
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    n_b = float(ell_all.sum(axis=1).mean())
    n_a = n_b + R
    cycle_bytes = draft_bytes + (n_a * V * 2 + n_b * V * 2 + V * r * 2)
    # the stricter view of the draft: W2 counted once per cycle (the last-level cache can
    # hold it), so only U_k, the W1 rows and h count per step
    draft_bytes_w2_once = G * (R * V * 2 + R * r * 2) + V * r * 2 + R * G * d * 2
    traffic = None
    if args.config == "c3" and os.path.exists(TRAFFIC_JSON):
        try:
            tr = json.load(open(TRAFFIC_JSON))
            if tr.get("kernel_source_sha") == kernel_sha():
                traffic = tr.get("bytes_per_launch")
        except Exception:
            traffic = None

    res = {
        "metric": METRIC,
        "value": R * G / (ms_per_step * 1e-3),
        "unit": "drafted tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Markov head R={R} gamma={G} V={V} r={r} d={d}, "
                               "bf16 operands, fp32 softmax; draft + schedule (early stop) + "
                               "verify, anchors from the previous cycle's last emitted tokens",
                   "R": R, "gamma": G, "V": V, "r": r, "d": d},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kern_name, "bytes_per_launch": kern_bytes,
                     "launch_us": kern_ms * 1e3},
        "sequential_head_cost": {
            "draft_markov_us": t_markov * 1e3, "draft_parallel_us": t_parallel * 1e3,
            "ratio": t_markov / t_parallel,
            "what": "the draft call with the Markov head against the parallel block's own "
                    "sampling from U_k (dspark_draft_parallel), same inputs, 10 calls each"},
        "markov_step_roofline": {
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "achieved": draft_bytes / (t_draft * 1e-3) / 1e9,
            "frac": draft_bytes / (t_draft * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_cycle": draft_bytes, "draft_us_per_cycle": t_draft * 1e3,
            "us_per_step": t_draft * 1e3 / G,
            "what": "the whole draft call (gamma positions: gather, bias contraction, logits, "
                    "normaliser, two-level sample, confidence) against U_k + W2 + h_k + W1 rows "
                    "per position"},
        "emitted_tokens_per_s": n_acc_sum / len(timed) / (ms_per_step * 1e-3),
        "stage_ms": {"draft": t_draft, "schedule": t_sched, "verify": t_ver},
        "cycle_ms_median": cycle_median,
        "hbm_copy_gbs": copy_gbs,
        "hbm_read_probe": None if read_probe is None else {
            "gbs": read_probe[0], "grid": read_probe[1], "bytes": read_probe[2],
            "frac_of_peak": read_probe[0] / HBM_PEAK_GBS,
            "sweep_frac_of_probe": achieved / read_probe[0],
            "what": "dspark_read_probe (a kernel that only reads, each workgroup streaming its "
                    "own slice) on the sweep's byte count, bytes no cache holds, timed by its "
                    "dispatch as the sweep is; best median of 7 reads over grids of 1024, 2048 "
                    "and 4096 workgroups"},
        "draft_hbm_frac_w2_once": draft_bytes_w2_once / (t_draft * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "cycle_hbm_frac": cycle_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "mean_verified_rows": n_b, "mean_ell": float(ell_all.mean()),
        "ell_per_cycle": [int(v) for v in ell_all.sum(axis=1)],
        "input_gen_s": gen_s,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(cfg, I, args.cpu_seconds)
    print(json.dumps(res))


def _timed_calls(torch, fn, warmup, steps):
    """Mean device time of fn() over `steps` calls on torch's current stream (events around
    each call) and the wall time of the whole timed loop."""
    import numpy as np
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return float(np.mean([a.elapsed_time(b) for a, b in ev])), wall * 1e3 / steps


def bench_train(args):
    """Training-objective forward (teacher-forced blocks, Module F) on the headline sizes:
    R=256 blocks of gamma=8 positions, V=151936, r=256, d=4096, bf16."""
    import numpy as np
    import torch

    import draft_sampling_scheduling_amd as ds
    from draft_sampling_scheduling_amd import synth

    ds.lib()
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    I = synth.inputs(cfg)
    B = synth.train_batch(cfg)

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    U, h, W1, w, x0 = T(I["U"]), T(I["h"]), T(I["W1"]), T(I["w"]), T(I["x0"])
    W2t = ds.w2_relayout(T(I["W2"]))  # the pages' [r][V] -> [V][r]
    target, xstar = T(B["target"]), T(B["xstar"])
    R, G, V, r, d = cfg.R, cfg.gamma, cfg.V, cfg.r, cfg.d
    gen_s = time.perf_counter() - t_gen
    log(f"teacher-forced batch of {cfg.name} resident on the device ({gen_s:.1f} s)")
    out = {k: torch.empty((R, G), dtype=torch.float32, device=dev)
           for k in ("c_star", "c", "logq", "tv")}
    out["loss"] = torch.empty((R, 4), dtype=torch.float32, device=dev)
    ws = torch.empty(ds.train_forward_workspace_bytes(R, G, V, r, d), dtype=torch.uint8,
                     device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        ds.train_forward(U, h, W1, W2t, w, target, x0, xstar, out=out, ws=ws, status=status)

    call_ms, ms_per_step = _timed_calls(torch, call, args.warmup, args.steps)
    if int(status.item()) != 0:
        raise SystemExit(f"device fault bits set: {int(status.item())}")
    rows = R * G
    # algorithmic bytes of one call: each sweep reads U, the target and W2t once (the W1
    # rows are gathered per row); the merge reads the hidden states
    sweep_bytes = 2 * rows * V * 2 + V * r * 2 + rows * r * 2
    call_bytes = 2 * sweep_bytes + rows * d * 2
    achieved = call_bytes / (call_ms * 1e-3) / 1e9
    res = {
        "metric": "training-objective forward rows/s (teacher-forced, R=256 gamma=8 "
                  "V=151936); % of HBM roofline",
        "value": rows / (ms_per_step * 1e-3),
        "unit": "teacher-forced rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} teacher-forced blocks: Markov head R={R} gamma={G} "
                               f"V={V} r={r} d={d}, bf16 operands; c*, L_ce, L_tv, L_conf",
                   "R": R, "gamma": G, "V": V, "r": r, "d": d},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "dspark_train_forward (two sweeps, merge, final), whole call",
                     "bytes_per_launch": call_bytes, "launch_us": call_ms * 1e3},
        "mean_loss": float(out["loss"][:, 3].mean().item()),
        "input_gen_s": gen_s,
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        threads = oracle.num_threads()

        def run(S):
            t0 = time.perf_counter()
            oracle.train_forward(I["U"][:S], I["h"][:S], I["W1"], I["W2"], I["w"],
                                 B["target"][:S], I["x0"][:S], B["xstar"][:S])
            return time.perf_counter() - t0

        t1 = run(threads)
        S = int(threads * max(1.0, args.cpu_seconds / max(t1, 1e-3)))
        S = max(threads, min(R, (S // threads) * threads))
        t = run(S)
        res["cpu_baseline"] = dict(
            value=S * G / t, unit="teacher-forced rows/s", cores=threads, kind="oracle",
            sample=f"the first {S} of {R} blocks of the same batch, fp64; {t:.1f} s wall")
    print(json.dumps(res))


STS_N = 1 << 20  # held-out samples: 4096 cycles of 256 requests
STS_GRID = [round(0.2 + 0.1 * i, 2) for i in range(39)]  # 0.2 .. 4.0
STS_BINS = 15


def bench_sts(args):
    """STS calibration fit (Module D) on 2^20 held-out samples of gamma=8 positions, 39
    candidate temperatures, 15 bins."""
    import numpy as np
    import torch

    import draft_sampling_scheduling_amd as ds
    from draft_sampling_scheduling_amd import synth

    ds.lib()
    dev = torch.device("cuda:0")
    temps = [1.6, 0.7, 1.0, 2.5, 1.2, 0.9, 1.4, 2.0]
    z, n_acc = synth.sts_heldout(STS_N, temps, seed=1)
    zt, nt = torch.from_numpy(z).to(dev), torch.from_numpy(n_acc).to(dev)
    G = len(temps)
    out = dict(T=torch.empty(G, dtype=torch.float32, device=dev),
               ece=torch.empty(G, dtype=torch.float64, device=dev))
    ws = torch.empty(ds.sts_workspace_bytes(STS_N, len(STS_GRID), STS_BINS), dtype=torch.uint8,
                     device=dev)

    def call():
        ds.sts_fit(zt, nt, STS_GRID, STS_BINS, out=out, ws=ws)

    call_ms, ms_per_step = _timed_calls(torch, call, args.warmup, args.steps)
    # the definition's fp64 operations per (sample, candidate, position): z/T, exp, 1 + e,
    # the reciprocal division, the running-product multiply, the bin scale, o - P and the
    # fixed-point scale (divide and exp counted as one each)
    evals = STS_N * len(STS_GRID) * G
    achieved = evals * 8 / (call_ms * 1e-3) / 1e12
    res = {
        "metric": "STS calibration held-out samples/s (gamma=8, 39 temperatures, 15 bins)",
        "value": STS_N / (ms_per_step * 1e-3),
        "unit": "held-out samples/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"STS fit: N={STS_N} held-out samples, gamma={G}, "
                               f"{len(STS_GRID)} candidate temperatures, {STS_BINS} bins",
                   "N": STS_N, "gamma": G, "grid": len(STS_GRID), "nbins": STS_BINS},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": 78.6, "unit": "TFLOP/s",
                     "frac": achieved / 78.6, "traffic": None,
                     "kernel": "dspark_sts_fit (per position: bins, reduce, pick), whole call",
                     "flops_per_eval": 8, "launch_us": call_ms * 1e3},
        "T": [float(x) for x in out["T"].cpu().numpy()],
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        n = 1 << 14
        t0 = time.perf_counter()
        oracle.sts_fit(z[:n], n_acc[:n], np.asarray(STS_GRID, np.float32), STS_BINS)
        t1 = time.perf_counter() - t0
        n = int(min(STS_N, max(n, n * args.cpu_seconds / max(t1, 1e-3))))
        t0 = time.perf_counter()
        oracle.sts_fit(z[:n], n_acc[:n], np.asarray(STS_GRID, np.float32), STS_BINS)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=n / t, unit="held-out samples/s", cores=1,
                                   kind="oracle",
                                   sample=f"the first {n} of {STS_N} samples; {t:.1f} s wall")
    print(json.dumps(res))


DEC = dict(R=256, gamma=8, V=32000, r=256, d=512, ncycles=16, alpha=0.0005)


def bench_decode(args):
    """Multi-cycle driver on a toy chain: R=256 requests, gamma=8, V=32000, r=256, d=512,
    bf16, 16 cycles per step under Algorithm 1 with the break.  The chain's tables follow
    the toy-chain law (Zipf-ranked bigram target + N(0, 1); backbone rows = the anchor's
    target row + N(0, (0.3 + 0.2k)^2)) drawn on the device with a seeded torch generator."""
    import math

    import numpy as np
    import torch

    import draft_sampling_scheduling_amd as ds

    ds.lib()
    R, G, V, r, d, nc = (DEC[k] for k in ("R", "gamma", "V", "r", "d", "ncycles"))
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    t_gen = time.perf_counter()
    base = -1.1 * torch.log(torch.arange(1, V + 1, device=dev, dtype=torch.float32))
    base = base[torch.randperm(V, device=dev, generator=gen)]
    Tb = (base[None, :] + torch.randn((V, V), device=dev, generator=gen)).to(torch.bfloat16)
    Ub = torch.empty((V, G, V), dtype=torch.bfloat16, device=dev)
    for a0 in range(0, V, 1024):
        a1 = min(V, a0 + 1024)
        for k in range(G):
            Ub[a0:a1, k] = (Tb[a0:a1].float() + (0.3 + 0.2 * (k + 1)) *
                            torch.randn((a1 - a0, V), device=dev, generator=gen)).to(torch.bfloat16)
    Hb = torch.randn((V, G, d), device=dev, generator=gen).to(torch.bfloat16)
    s = 1.0 / math.sqrt(r)
    W1 = (s * torch.randn((V, r), device=dev, generator=gen)).to(torch.bfloat16)
    W2t = (s * torch.randn((V, r), device=dev, generator=gen)).to(torch.bfloat16)
    w = math.sqrt(1.0 / (d + r)) * torch.randn(d + r, device=dev, generator=gen)
    x0 = torch.randint(0, V, (R,), device=dev, generator=gen, dtype=torch.int32)
    B = torch.arange(1, R * (G + 1) + 1, device=dev, dtype=torch.float64)
    sps = (1.0 / (1.0 + DEC["alpha"] * B)).float()
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    log(f"toy chain tables on the device ({gen_s:.1f} s)")
    out = dict(tokens=torch.empty((R, nc * (G + 1)), dtype=torch.int32, device=dev),
               n_emitted=torch.empty(R, dtype=torch.int32, device=dev),
               stats=torch.empty(2 * G + 3, dtype=torch.int64, device=dev))
    ws = torch.empty(ds.decode_workspace_bytes(R, G, V, r, d, ds.BF16), dtype=torch.uint8,
                     device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        ds.decode_run(Ub, Hb, W1, W2t, w, Tb, x0, nc, ds.SYNC_BREAK, sps=sps, sps_B0=1,
                      seed=5, out=out, ws=ws, status=status)

    call_ms, ms_per_step = _timed_calls(torch, call, args.warmup, args.steps)
    if int(status.item()) != 0:
        raise SystemExit(f"device fault bits set: {int(status.item())}")
    st = out["stats"].cpu().numpy()
    tested, acc = st[:G], st[G:2 * G]
    sum_ell, emitted, rc = int(st[2 * G]), int(st[2 * G + 1]), int(st[2 * G + 2])
    mean_ell = sum_ell / rc
    # algorithmic bytes of one call (per cycle: the table gathers read and write their rows,
    # gamma draft sweeps read U_k and W2, verification reads the scheduled target rows, the
    # bonus rows and the U rows it re-forms q from, plus W2)
    per_cycle = (2 * R * G * V * 2 + 2 * R * (G + 1) * V * 2 + G * (R * V * 2 + V * r * 2)
                 + (R * mean_ell + R) * V * 2 + 2 * R * mean_ell * V * 2 + V * r * 2)
    achieved = nc * per_cycle / (call_ms * 1e-3) / 1e9
    res = {
        "metric": "toy-chain decode emitted tokens/s (R=256 gamma=8 V=32000, 16 cycles per "
                  "step, Algorithm 1 with the break)",
        "value": emitted / (ms_per_step * 1e-3),
        "unit": "emitted tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"toy chain decode: R={R} gamma={G} V={V} r={r} d={d}, "
                               f"{nc} cycles, SYNC_BREAK, SPS(B)=1/(1+{DEC['alpha']}B)",
                   "R": R, "gamma": G, "V": V, "r": r, "d": d, "cycles": nc},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "dspark_decode_run, whole call (all kernels of 16 cycles)",
                     "bytes_per_launch": nc * per_cycle, "launch_us": call_ms * 1e3},
        "cycles_per_s": nc / (ms_per_step * 1e-3),
        "mean_ell": mean_ell,
        "tokens_per_request_cycle": emitted / rc,
        "conditional_acceptance": [float(a / t) if t else None for a, t in zip(acc, tested)],
        "input_gen_s": gen_s,
    }
    print(json.dumps(res))


def bench_rnn(args):
    """RNN-head draft (eq. (6)) on its workload: R=256 requests, gamma=16, V=129280, r=256,
    d=4096, bf16 operands (float bias rows, entered as hi + lo bf16 terms).  Random operands
    drawn on the device (the timing does not depend on their values)."""
    import math

    import torch

    import draft_sampling_scheduling_amd as ds
    from draft_sampling_scheduling_amd import synth

    ds.lib()
    cfg = synth.CONFIGS["c5"]
    R, G, V, r, d = cfg.R, cfg.gamma, cfg.V, cfg.r, cfg.d
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(55)
    t_gen = time.perf_counter()

    def rnd(shape, std):
        return (std * torch.randn(shape, device=dev, generator=gen)).to(torch.bfloat16)

    U = rnd((R, G, V), 1.0)
    h = rnd((R, G, d), 1.0)
    W1 = rnd((V, r), 1.0 / math.sqrt(r))
    W2t = rnd((V, r), 1.0 / math.sqrt(r))
    Wg = rnd((3 * r, 2 * r + d), 1.0 / math.sqrt(2 * r + d))
    w = math.sqrt(1.0 / (d + r)) * torch.randn(d + r, device=dev, generator=gen)
    x0 = torch.randint(0, V, (R,), device=dev, generator=gen, dtype=torch.int32)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    out = dict(x=torch.empty((R, G), dtype=torch.int32, device=dev),
               c=torch.empty((R, G), dtype=torch.float32, device=dev),
               lse=torch.empty((R, G), dtype=torch.float32, device=dev),
               logit_x=torch.empty((R, G), dtype=torch.float32, device=dev),
               bias_rows=torch.empty((R, G, r), dtype=torch.float32, device=dev))
    ws = torch.empty(ds.draft_rnn_workspace_bytes(R, G, V, r, d), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        ds.draft_rnn(U, h, W1, W2t, Wg, w, x0, SEED, CYCLE, out=out, ws=ws, status=status)

    call_ms, ms_per_step = _timed_calls(torch, call, args.warmup, args.steps)
    if int(status.item()) != 0:
        raise SystemExit(f"device fault bits set: {int(status.item())}")
    # algorithmic bytes of one draft: per position the sweep reads U_k, W2 and the float bias
    # rows; the h-part projection reads h and W_gco's h columns once; the per-step RNN update
    # reads W_gco's [s; e] columns and W1 rows
    sweep = R * V * 2 + V * r * 2 + R * r * 4
    call_bytes = (G * sweep + R * G * d * 2 + 3 * r * d * 2
                  + G * (3 * r * 2 * r * 2 + R * r * 2))
    achieved = call_bytes / (call_ms * 1e-3) / 1e9
    res = {
        "metric": "RNN-head draft tokens/s (R=256 gamma=16 V=129280); % of HBM roofline",
        "value": R * G / (ms_per_step * 1e-3),
        "unit": "drafted tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"c5 RNN head: R={R} gamma={G} V={V} r={r} d={d}, bf16 operands, "
                               "float bias rows; draft only",
                   "R": R, "gamma": G, "V": V, "r": r, "d": d},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "dspark_draft_rnn, whole call (h projection, 16 x (RNN step, "
                               "sweep, combine))",
                     "bytes_per_launch": call_bytes, "launch_us": call_ms * 1e3},
        "input_gen_s": gen_s,
    }
    print(json.dumps(res))


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    # the draft sweep kernel's whole source: the sweep template, its epilogue, the helpers
    for f in ("dev.h", "sweep.h", "draft_epi.h"):
        h.update(open(os.path.join(ROOT, "draft_sampling_scheduling_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
