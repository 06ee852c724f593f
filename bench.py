"""SSD chunked-scan forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one full forward (every kernel of the path) over the Mamba-2 2.7B layer
shape (b8 T4096 H80 P64 N128 G1 Q256, bf16 x/B/C, fp32 dt/A/D/h0, nonzero h0), with
seeded synthetic inputs already resident in HBM.  Prints one JSON line with
tokens/s, TFLOP/s (causal flop count) against the bf16 matrix-core peak, the
roofline of the dominant kernel (timed live with HIP events on the launch stream
through the library's per-stage mask), per-kernel times, the decode step and the
backward pass at the same shape, and the fp64 oracle timed on a bounded sample of the
same workload on this host's cores.
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, published
FP32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix cores, published
COPY_BYTES = 512 << 20      # size of the calibration copy (bytes read = bytes written)
def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    from ssd_chunked_scan_03_amd.metrics import kernel_source_hash
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, budget_s=12.0):
    """The fp64 oracle (step-by-step recurrence) over the whole workload, repeated until
    about `budget_s` of wall time has passed; whole-layer tokens/s on this host's cores."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = max(1, min(threads, len(os.sched_getaffinity(0))))
    reps, total = 0, 0.0
    while total < budget_s:
        t0 = time.perf_counter()
        oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], diag=w.diag,
                          nthreads=threads)
        total += time.perf_counter() - t0
        reps += 1
    tokens = w.batch * w.seqlen * reps
    return {"value": round(tokens / total, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload ({w.batch} x {w.seqlen} tokens, {w.nheads} heads), {reps} pass(es) "
                      f"in {total:.2f} s; fp64 step-by-step recurrence, OpenMP over (batch, head, headdim block)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed forwards first (about 40 ms at the default workload: the GPU clock settles)")
    ap.add_argument("--workload", default=None, help="workload name (default: the 2.7B layer shape)")
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--seqlen", type=int, default=None, help="override the workload's sequence length (scaling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--kernel-steps", type=int, default=None, help="launches per kernel timing")
    ap.add_argument("--schedule", choices=["auto", "split", "fused"], default="auto",
                    help="kernel schedule (auto: the library's choice for the shape)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed work, stream 512 MiB through a plain elementwise kernel "
                         "(calibrates the byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not an implementation", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import ssd_chunked_scan_03_amd as ssd
    from ssd_chunked_scan_03_amd import configs, metrics
    from ssd_chunked_scan_03_amd.synth import make_grads, make_inputs

    w = configs.HEADLINE
    if args.workload:
        w = {x.name: x for x in configs.WORKLOADS}[args.workload]
    if args.chunk:
        w = w.with_(chunk=args.chunk)
    if args.seqlen:
        w = w.with_(seqlen=args.seqlen, name=f"{w.name}_T{args.seqlen}")
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = make_inputs(w)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.from_numpy(inp["x"]).to(dev).to(td).contiguous()
    B = torch.from_numpy(inp["B"]).to(dev).to(td).contiguous()
    C = torch.from_numpy(inp["C"]).to(dev).to(td).contiguous()
    dt = torch.from_numpy(inp["dt"]).to(dev)
    A = torch.from_numpy(inp["A"]).to(dev)
    D = torch.from_numpy(inp["D"]).to(dev)
    h0 = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).to(dev)
    b, T, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    dcode = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
    sched_flag = {"auto": 0, "split": ssd.SCHEDULE_SPLIT, "fused": ssd.SCHEDULE_FUSED}[args.schedule]
    prob = ssd.make_problem(b, T, H, P, N, G, Q, dcode, flags=sched_flag)
    y = torch.empty_like(x)
    hT = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(ssd.workspace_bytes(prob, w.diag), dtype=torch.uint8, device=dev)
    print(f"[bench] {w.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(p=prob):
        ssd.scan_fwd_into(p, w.diag, x, dt, A, B, C, D, h0, y, hT, ws, stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps: {ms:.4f} ms/step (host wall {wall * 1e3 / args.steps:.4f})",
          file=sys.stderr, flush=True)

    # per-kernel average launch duration, HIP events on the same stream: a staged forward
    # launches the forward's kernels in the forward's order, one stage per library call,
    # with an event between stages, so each kernel runs on the cache state it meets in the
    # forward itself
    kb = metrics.kernel_bytes(b, T, H, P, N, G, Q, 2 if w.dtype == "bf16" else 4, w.diag, h0 is not None)
    ksteps = args.kernel_steps or max(10, args.steps)
    schedule = ssd.schedule_of(prob, w.diag)
    plan = ssd.schedule_kernels(schedule, w.diag)
    names = [k for k, _ in plan]
    staged = [ssd.make_problem(b, T, H, P, N, G, Q, dcode, flags=m | sched_flag) for _, m in plan]
    kb["k_prep"] = kb["k_cumsum"] + kb["k_cb"] + (kb["k_bt"] if schedule == "fused" else 0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(ksteps)]
    for _ in range(2):
        for pk in staged:
            step(pk)
    torch.cuda.synchronize()
    for ev in evs:
        for i, pk in enumerate(staged):
            ev[i].record(stream)
            step(pk)
        ev[-1].record(stream)
    torch.cuda.synchronize()
    kernels = {}
    for i, name in enumerate(names):
        kms = sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / ksteps
        kernels[name] = {"ms": round(kms, 5), "bytes": kb[name],
                         "GBps": round(kb[name] / (kms * 1e-3) / 1e9, 1)}
    step()  # leave y/hT from a full forward
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)  # one streaming kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    traffic = measured_traffic(dom, w.name)
    roof = {"kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dk["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": dk["bytes"], "avg_launch_ms": dk["ms"]}

    # one decode step (ssd_step, seqlen 1) at the same batch, heads and state size: the
    # state is read and written once, so it is timed against HBM bandwidth
    es = 2 if w.dtype == "bf16" else 4
    hstate = (h0.clone() if h0 is not None else torch.zeros((b, H, P, N), dtype=torch.float32, device=dev))
    xs, dts, Bs, Cs = x[:, :1].contiguous(), dt[:, :1].contiguous(), B[:, :1].contiguous(), C[:, :1].contiguous()
    ys = torch.empty_like(xs)
    sprob = ssd.make_problem(b, 1, H, P, N, G, Q, dcode)
    for _ in range(3):
        ssd.step_into(sprob, w.diag, xs, dts, A, Bs, Cs, D, hstate, ys, stream.cuda_stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(ksteps):
        ssd.step_into(sprob, w.diag, xs, dts, A, Bs, Cs, D, hstate, ys, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    sms = e0.elapsed_time(e1) / ksteps
    sbytes = 2 * 4 * b * H * P * N + 2 * es * b * H * P + 2 * es * b * G * N + 4 * b * H
    decode = {"us": round(sms * 1e3, 2), "bytes": sbytes, "GBps": round(sbytes / (sms * 1e-3) / 1e9, 1),
              "hbm_frac": round(sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
              "tokens_per_s": round(b / (sms * 1e-3), 1)}

    # the backward pass (either decay) at the same workload: gradients of every input for
    # seeded output gradients dy, dhT, timed as a whole with HIP events on the launch stream
    backward = None
    if not args.no_bwd:
        print("[bench] timing the backward pass", file=sys.stderr, flush=True)
        gr = make_grads(b, T, H, P, N, w.seed, dtype=w.dtype)
        dy = torch.from_numpy(gr["dy"]).to(dev).to(td).contiguous()
        dhT = torch.from_numpy(gr["dhT"]).to(dev)
        bprob = ssd.make_problem(b, T, H, P, N, G, Q, dcode)
        bws = torch.empty(max(ssd.bwd_workspace_bytes(bprob, w.diag), 1), dtype=torch.uint8, device=dev)
        g = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dA=torch.empty_like(A), dB=torch.empty_like(B),
                 dC=torch.empty_like(C), dD=torch.empty_like(D),
                 dh0=torch.empty((b, H, P, N), dtype=torch.float32, device=dev))

        def bstep():
            ssd.scan_bwd_into(bprob, x, dt, A, B, C, D, h0, dy, dhT, g["dx"], g["ddt"], g["dA"], g["dB"], g["dC"],
                              g["dD"], g["dh0"], bws, stream.cuda_stream, diag=w.diag)

        for _ in range(3):
            bstep()
        torch.cuda.synchronize()
        bsteps = max(5, ksteps // 2)
        e0.record(stream)
        for _ in range(bsteps):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / bsteps
        es_ = 2 if w.dtype == "bf16" else 4
        bmin = metrics.bwd_path_min_bytes(b, T, H, P, N, G, es_, h0 is not None, True)
        backward = {"ms": round(bms, 5), "tokens_per_s": round(b * T / (bms * 1e-3), 1), "steps": bsteps,
                    "inputs": "x, dt, A, B, C, D, h0, dy, dhT (y is recomputed, not stored)",
                    "path_min_bytes": bmin,
                    "path_hbm_frac": round(bmin / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "workspace_bytes": int(bws.numel())}
        del bws, g, dy, dhT
        print(f"[bench] backward: {bms:.4f} ms", file=sys.stderr, flush=True)

    fl = metrics.flops(b, T, H, P, N, G, Q, w.diag)
    tokens = b * T
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    min_bytes = metrics.path_min_bytes(b, T, H, P, N, G, 2 if w.dtype == "bf16" else 4, h0 is not None)
    out = {
        "metric": "SSD fwd tokens/s + TFLOP/s (% bf16 MFMA peak), Mamba-2 2.7B layer shape",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; Mamba-2 layer-shaped value distributions)",
        "config": {"workload": w.name, "batch": b, "seqlen": T, "nheads": H, "headdim": P, "dstate": N,
                   "ngroups": G, "chunk": Q, "decay": "diagonal" if w.diag else "scalar",
                   "h0": h0 is not None, "schedule": schedule},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "path_min_bytes": min_bytes,
        "path_hbm_frac": round(min_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roof,
        "kernels": kernels,
        "decode_step": decode,
        "backward": backward,
        "kernel_source_hash": metrics.kernel_source_hash(),
    }
    if not args.no_cpu:
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
