"""SSD chunked-scan forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one full forward (every kernel of the path) over the Mamba-2 2.7B layer
shape (b8 T4096 H80 P64 N128 G1 Q256, bf16 x/B/C, fp32 dt/A/D/h0, nonzero h0), with
seeded synthetic inputs already resident in HBM.  After W untimed forwards, K forwards
are timed one by one with HIP events on the launch stream, each after a 1 GiB scratch
read that flushes the caches (cold: the headline `value`); K back-to-back forwards are
timed the same way (warm, reported beside it).  The JSON line also carries the roofline
of the dominant kernel (timed live inside a staged forward), its matrix-core rate, the
HBM and matrix-core peaks measured on this GPU (a streaming copy and a dense matrix-core
loop), per-kernel times, the other workloads timed briefly (with the long workload's
cost against sequence length over the first 8K..64K tokens of its inputs), the decode
step and the backward pass at the same shape, and the fp64 oracle timed on this host's
cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, published
FP32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix cores, published
COPY_BYTES = 512 << 20      # size of the counter-calibration copy (bytes read = bytes written)
FLUSH_BYTES = 1 << 30       # scratch read before each cold step (> the 256 MB last-level cache)
PEAK_COPY_BYTES = 1 << 30   # streaming-copy measurement: bytes read (= bytes written)


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


def stats(ts):
    """mean / median / min of per-step milliseconds."""
    return {"mean_ms": round(sum(ts) / len(ts), 5), "median_ms": round(statistics.median(ts), 5),
            "min_ms": round(min(ts), 5), "reps": len(ts)}


def time_each(torch, stream, fn, reps, before=None):
    """Per-step milliseconds: an event pair on `stream` around each call of fn; `before`
    (untimed) runs ahead of each step."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        if before is not None:
            before()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def measure_peaks(torch, stream, dev):
    """HBM bandwidth of a plain streaming copy (the best of a few grid sizes and cache
    policies, median of 5 each) and the sustained bf16 matrix-core rate of a dense loop of
    independent 16x16x32 steps (best of 5), both on this GPU."""
    from ssd_chunked_scan_03_amd import build
    if not os.path.exists(build.PEAK_LIB):
        return None
    lib = ctypes.CDLL(build.PEAK_LIB)
    lib.peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                              ctypes.c_void_p]
    lib.peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                              ctypes.c_void_p]
    src = torch.ones(PEAK_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sp = ctypes.c_void_p(stream.cuda_stream)
    best, how = 0.0, ""
    for blocks in (1024, 2048, 4096, 8192):
        for nt in (1, 0):
            def copy():
                assert lib.peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                     PEAK_COPY_BYTES, blocks, nt, sp) == 0
            copy()
            gbs = 2 * PEAK_COPY_BYTES / (statistics.median(time_each(torch, stream, copy, 5)) * 1e-3) / 1e9
            if gbs > best:
                best, how = gbs, f"{blocks} work-groups, {'non-temporal' if nt else 'default'} accesses"
    assert torch.equal(dst[:1024], src[:1024])
    del src, dst
    blocks, iters = 256 * 8, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    fl = ctypes.c_double(0.0)

    def mfma():
        assert lib.peak_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, ctypes.byref(fl), sp) == 0
    mfma()
    ts = time_each(torch, stream, mfma, 5)
    mfma_tflops = fl.value / (min(ts) * 1e-3) / 1e12
    return {"hbm_copy_GBps": round(best, 1), "bf16_mfma_TFLOPs": round(mfma_tflops, 1),
            "copy": f"{PEAK_COPY_BYTES >> 20} MiB read + written by a streaming copy kernel (four 16-byte loads "
                    f"in flight per thread); best setting: {how}; median of 5",
            "mfma": f"{blocks} work-groups x 4 waves x {iters} rounds of 8 independent 16x16x32 bf16 steps, best of 5"}


def upload_inputs(torch, inp, dtype, dev):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {k: torch.from_numpy(inp[k]).to(dev).to(td).contiguous() for k in ("x", "B", "C")}
    for k in ("dt", "A", "D"):
        d[k] = torch.from_numpy(inp[k]).to(dev)
    d["h0"] = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).to(dev)
    return d


def other_workloads(torch, ssd, stream, dev, headline, reps=10):
    """The remaining workloads (every chunk size of the long one), each timed briefly: 3
    untimed forwards, then `reps` forwards one by one (warm), on the library's default
    schedule."""
    from ssd_chunked_scan_03_amd import configs, metrics
    from ssd_chunked_scan_03_amd.synth import make_inputs
    out = {}
    for w0 in configs.WORKLOADS:
        if w0.name == headline.name:
            continue
        chunks = configs.LONG_CHUNKS if w0.name == configs.LONG.name else (w0.chunk,)
        inp = make_inputs(w0)
        d = upload_inputs(torch, inp, w0.dtype, dev)
        del inp
        for Q in chunks:
            w = w0.with_(chunk=Q)
            b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
            dcode = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
            prob = ssd.make_problem(b, T, H, P, N, G, Q, dcode)
            y = torch.empty_like(d["x"])
            hT = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
            ws = torch.empty(max(ssd.workspace_bytes(prob, w.diag), 1), dtype=torch.uint8, device=dev)

            def step():
                ssd.scan_fwd_into(prob, w.diag, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], y, hT, ws,
                                  stream.cuda_stream)
            for _ in range(3):
                step()
            torch.cuda.synchronize()
            st = stats(time_each(torch, stream, step, reps))
            ms = st["median_ms"]
            es = 2 if w.dtype == "bf16" else 4
            mb = metrics.path_min_bytes(b, T, H, P, N, G, es, d["h0"] is not None)
            fl = metrics.flops(b, T, H, P, N, G, Q, w.diag)["total"]
            key = w.name if len(chunks) == 1 else f"{w.name}_Q{Q}"
            out[key] = {"ms_per_step": ms, "min_ms": st["min_ms"], "tokens_per_s": round(b * T / (ms * 1e-3), 1),
                        "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "path_min_bytes": mb,
                        "path_hbm_frac": round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "schedule": ssd.schedule_of(prob, w.diag), "chunk": Q, "dtype": w.dtype,
                        "decay": "diagonal" if w.diag else "scalar"}
            print(f"[bench] {key}: {ms:.4f} ms/step", file=sys.stderr, flush=True)
            del y, hT, ws
        if w0.name == configs.LONG.name:
            out[f"{w0.name}_seqlen_scaling"] = seqlen_scaling(torch, ssd, stream, dev, w0, d, reps)
        del d
    return out


def seqlen_scaling(torch, ssd, stream, dev, w, d, reps):
    """The long workload (batch 1) at its own chunk size over the first T tokens of the same
    resident inputs, T = 8K .. the whole sequence: the forward's cost against T ("still
    linear in T").  Each point: 3 untimed forwards, then `reps` timed one by one (warm)."""
    b, H, P, N, G, Q = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    dcode = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
    pts = {}
    T = 8192
    while T <= w.seqlen:
        sl = {k: (d[k][:, :T] if d[k] is not None and k in ("x", "dt", "B", "C") else d[k]) for k in d}
        assert all(v is None or v.is_contiguous() for v in sl.values())  # batch 1: leading slices
        prob = ssd.make_problem(b, T, H, P, N, G, Q, dcode)
        y = torch.empty_like(sl["x"])
        hT = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(ssd.workspace_bytes(prob, w.diag), 1), dtype=torch.uint8, device=dev)

        def step():
            ssd.scan_fwd_into(prob, w.diag, sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"], sl["h0"], y, hT,
                              ws, stream.cuda_stream)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        ms = stats(time_each(torch, stream, step, reps))["median_ms"]
        pts[str(T)] = {"ms_per_step": ms, "tokens_per_s": round(b * T / (ms * 1e-3), 1)}
        print(f"[bench] {w.name} T={T}: {ms:.4f} ms/step", file=sys.stderr, flush=True)
        del y, hT, ws
        T *= 2
    ts = sorted(int(t) for t in pts)
    lo, hi = ts[0], ts[-1]
    return {"chunk": Q, "schedule": ssd.schedule_of(ssd.make_problem(b, hi, H, P, N, G, Q, dcode), w.diag),
            "points": pts,
            "time_ratio_last_over_first": round(pts[str(hi)]["ms_per_step"] / pts[str(lo)]["ms_per_step"], 3),
            "token_ratio_last_over_first": hi // lo}


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
    ap.add_argument("--no-workloads", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the copy and matrix-core peaks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed work, stream 512 MiB through a plain elementwise kernel "
                         "(calibrates the byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not an implementation", file=sys.stderr)
        sys.exit(2)

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
    d = upload_inputs(torch, inp, w.dtype, dev)
    x, B, C, dt, A, D, h0 = d["x"], d["B"], d["C"], d["dt"], d["A"], d["D"], d["h0"]
    b, T, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    dcode = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
    sched_flag = {"auto": 0, "split": ssd.SCHEDULE_SPLIT, "fused": ssd.SCHEDULE_FUSED}[args.schedule]
    prob = ssd.make_problem(b, T, H, P, N, G, Q, dcode, flags=sched_flag)
    y = torch.empty_like(x)
    hT = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ssd.workspace_bytes(prob, w.diag), 1), dtype=torch.uint8, device=dev)
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    print(f"[bench] {w.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(p=prob):
        ssd.scan_fwd_into(p, w.diag, x, dt, A, B, C, D, h0, y, hT, ws, stream.cuda_stream)

    def flush():
        # 1 GiB read: no input or table of the previous step stays cached.  A read leaves
        # clean lines; a write would leave dirty ones that the timed step then writes back.
        flush_buf.sum()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    cold = time_each(torch, stream, step, args.steps, before=flush)
    wall = time.perf_counter() - wall0
    warm = time_each(torch, stream, step, args.steps)
    cs, wsm = stats(cold), stats(warm)
    ms = cs["mean_ms"]
    print(f"[bench] {args.steps} steps: cold {ms:.4f} ms/step (median {cs['median_ms']:.4f}), "
          f"warm {wsm['mean_ms']:.4f} (host wall {wall * 1e3 / args.steps:.4f} with the flushes)",
          file=sys.stderr, flush=True)
    del flush_buf

    # per-kernel average launch duration, HIP events on the same stream: a staged forward
    # launches the forward's kernels in the forward's order, one stage per library call,
    # with an event between stages, so each kernel runs on the cache state it meets in the
    # forward itself
    kb = metrics.kernel_bytes(b, T, H, P, N, G, Q, 2 if w.dtype == "bf16" else 4, w.diag, h0 is not None)
    ksteps = args.kernel_steps or max(10, args.steps)
    schedule = ssd.schedule_of(prob, w.diag)
    plan = ssd.schedule_kernels(schedule, w.diag, prob)
    names = [k for k, _ in plan]
    staged = [ssd.make_problem(b, T, H, P, N, G, Q, dcode, flags=m | sched_flag) for _, m in plan]
    kb["k_prep"] = kb["k_cumsum"] + kb["k_cb"] + (kb["k_bt"] if schedule == "fused" else 0)
    kb["k_gtab"] = metrics.gtab_bytes(b, T, H, G, N, Q, 2 if w.dtype == "bf16" else 4)
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
        del src, dst

    peaks = None if args.no_peaks else measure_peaks(torch, stream, dev)
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    traffic = measured_traffic(dom, w.name)
    roof = {"kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dk["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": dk["bytes"], "avg_launch_ms": dk["ms"]}
    if peaks:
        roof["peak_measured"] = peaks["hbm_copy_GBps"]
        roof["frac_measured"] = round(dk["GBps"] / peaks["hbm_copy_GBps"], 4)
    # matrix-core rate of the fused kernel (the diagonal-block work runs inside it): the
    # flops of the 16x16x32 steps it issues over its measured launch duration
    mfma = None
    if dom == "k_fused":
        fl_issued = metrics.fused_mfma_flops(b, T, H, N, Q)
        rate = fl_issued / (dk["ms"] * 1e-3) / 1e12
        mfma = {"kernel": dom, "issued_gflop": round(fl_issued / 1e9, 2), "tflops": round(rate, 1),
                "frac_spec": round(rate / BF16_PEAK_TFLOPS, 4)}
        if peaks:
            mfma["frac_measured"] = round(rate / peaks["bf16_mfma_TFLOPs"], 4)

    # one decode step (ssd_step, seqlen 1) at the same batch, heads and state size: the
    # state is read and written once, so it is timed against HBM bandwidth
    es = 2 if w.dtype == "bf16" else 4
    hstate = (h0.clone() if h0 is not None else torch.zeros((b, H, P, N), dtype=torch.float32, device=dev))
    xs, dts, Bs, Cs = x[:, :1].contiguous(), dt[:, :1].contiguous(), B[:, :1].contiguous(), C[:, :1].contiguous()
    ys = torch.empty_like(xs)
    sprob = ssd.make_problem(b, 1, H, P, N, G, Q, dcode)

    def dstep():
        ssd.step_into(sprob, w.diag, xs, dts, A, Bs, Cs, D, hstate, ys, stream.cuda_stream)
    for _ in range(3):
        dstep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(ksteps):
        dstep()
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
        td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
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

        for _ in range(10):  # untimed: the first passes over a fresh workspace run slower
            bstep()
        torch.cuda.synchronize()
        bsteps = max(5, ksteps // 2)
        bst = stats(time_each(torch, stream, bstep, bsteps))
        bms = bst["mean_ms"]
        bmin = metrics.bwd_path_min_bytes(b, T, H, P, N, G, es, h0 is not None, True)
        backward = {"ms": bms, "median_ms": bst["median_ms"], "min_ms": bst["min_ms"],
                    "tokens_per_s": round(b * T / (bms * 1e-3), 1), "steps": bsteps,
                    "inputs": "x, dt, A, B, C, D, h0, dy, dhT (y is recomputed, not stored)",
                    "path_min_bytes": bmin,
                    "path_hbm_frac": round(bmin / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "workspace_bytes": int(bws.numel())}
        del bws, g, dy, dhT
        print(f"[bench] backward: {bms:.4f} ms", file=sys.stderr, flush=True)

    workloads = None
    if not args.no_workloads and not args.workload and not args.seqlen and not args.chunk:
        print("[bench] timing the other workloads", file=sys.stderr, flush=True)
        workloads = other_workloads(torch, ssd, stream, dev, w)

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
        "timing": {"cold": cs, "warm": wsm, "value_from": "cold mean",
                   "cold_protocol": f"{FLUSH_BYTES >> 20} MiB scratch read before each timed step"},
        "warm_tokens_per_s": round(tokens / (wsm["mean_ms"] * 1e-3), 1),
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "path_min_bytes": min_bytes,
        "path_hbm_frac": round(min_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roof,
        "mfma": mfma,
        "peaks_measured": peaks,
        "kernels": kernels,
        "decode_step": decode,
        "backward": backward,
        "workloads": workloads,
        "kernel_source_hash": metrics.kernel_source_hash(),
    }
    if peaks:
        out["path_hbm_frac_measured"] = round(min_bytes / (ms * 1e-3) / 1e9 / peaks["hbm_copy_GBps"], 4)
    if not args.no_cpu:
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
