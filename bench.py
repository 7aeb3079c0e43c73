#!/usr/bin/env python3
"""Throughput of causal linear attention (phi = elu + 1) on one MI355X.

One step = one la_causal_fwd call on the headline workload (B=4, H=8,
N=4096, d=64, bf16 inputs, fp32 state and outputs, chunk 64, eps 1e-6), with
inputs resident in HBM.  Eight input/output sets (about 670 MB, more than
twice the 256 MB Infinity Cache) are rotated so every step reads HBM.

Prints ONE JSON line: value = B*H*N head-tokens per second over the timed
steps; `roofline` = algorithmic bytes of one call / its average duration
(HIP events on the launch stream) against 8 TB/s; `cpu_baseline` = the fp64
oracle on the host cores; `workloads` = the segment-carried, decode,
non-causal and compressive-memory workloads and the unnormalised causal form
of the headline workload, timed the same way.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal linear-attn fwd tokens/sec (B·H·N/s) at d=64/128 + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes_causal(w, with_state_io=False):
    """inputs once, fp32 outputs once (+ fp32 state in and out per head)."""
    b = w.B * w.H * w.N * (3 * w.d * w.dtype.itemsize + 4 * w.d)
    if with_state_io:
        b += 2 * w.B * w.H * (w.d * w.d + w.d) * 4
    return b


def time_steps(fn, steps, warmup, n_rot):
    """Run fn(i) warmup times untimed, then exactly `steps` times back to back
    between two HIP events on the current stream (a device synchronize on both
    sides); return the elapsed ms.  No event is recorded between the steps:
    per-step events cost several microseconds of host time each and would
    leave the GPU idle between launches."""
    import torch
    for i in range(warmup):
        fn(i % n_rot)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        fn((warmup + i) % n_rot)
    t_end.record()
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end)


def measured_traffic(name):
    """HBM bytes per call from the FETCH_SIZE / WRITE_SIZE summary kept in
    profiles/, or None when that summary was taken on another version of the
    HIP source (its recorded sha256 no longer matches)."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", f"{name}_hbm_bytes.txt")).read()
        src = open(os.path.join(ROOT, "segment_wise_compressive_amd", "csrc", "linattn.hip"), "rb").read()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines() if l.startswith(("traffic_bytes_per_call:", "source_sha256:")))
    if fields.get("source_sha256", "").strip() != hashlib.sha256(src).hexdigest():
        return None
    return int(fields["traffic_bytes_per_call"])


def roofline(bytes_per_call, ms_per_call, traffic=None):
    achieved = bytes_per_call / (ms_per_call * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}


def prewarm(fn, n_rot, seconds, batch=100):
    """Untimed calls for about `seconds` of wall time before the warm-up
    steps, so that the GPU clocks have ramped up when the timed region starts
    (a fresh process reaches steady clocks only after some tens of ms of
    work).  Runs in batches of `batch` calls with a synchronize after each."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn(i % n_rot)
            i += 1
        torch.cuda.synchronize()


def leg_counts(args, steps, warmup):
    """Timed and warm-up repetitions of a non-headline workload: fixed
    counts (the headline's --steps / --warmup do not shrink them), or the
    --leg-steps / --leg-warmup overrides (short profiled runs)."""
    return (args.leg_steps if args.leg_steps is not None else steps,
            args.leg_warmup if args.leg_warmup is not None else warmup)


def step_spread(fn, steps, n_rot, blocks=10):
    """Per-call time over `blocks` consecutive blocks of steps (HIP events
    around each block): median, p10 and p90 in ms.  Runs after the timed
    region, as a second look at the same calls."""
    import torch
    per = max(1, steps // blocks)
    times = []
    for b in range(blocks):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(per):
            fn((b * per + i) % n_rot)
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) / per)
    times.sort()
    pick = lambda f: times[min(len(times) - 1, int(round(f * (len(times) - 1))))]
    return {"blocks": blocks, "calls_per_block": per, "median_ms": round(pick(0.5), 5),
            "p10_ms": round(pick(0.1), 5), "p90_ms": round(pick(0.9), 5)}


def copy_bandwidth(torch, reps=5):
    """Achievable HBM bandwidth of a plain 1 GiB device copy (read + write),
    GB/s: the second denominator beside the 8 TB/s peak."""
    n = 256 * 1024 * 1024
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del src, dst
    return round(2 * 4 * n / (ms * 1e-3) / 1e9, 1)


def bench_headline(args, torch, la, inp):
    w = inp.WORKLOADS[inp.HEADLINE]
    dev = torch.device("cuda:0")
    q, k, v = inp.workload_inputs(w)
    n_rot = args.rotate
    sets = []
    for _ in range(n_rot):
        sets.append((q.to(dev), k.to(dev), v.to(dev),
                     torch.empty(w.B, w.H, w.N, w.d, dtype=torch.float32, device=dev)))
    ws = torch.empty(max(1, la.la_causal_fwd_workspace(w.B, w.H, w.N, w.d, w.chunk)),
                     dtype=torch.uint8, device=dev)

    calls = [la.prepare_causal_fwd(a[0], a[1], a[2], a[3], chunk=w.chunk, eps=w.eps, workspace=ws) for a in sets]

    def step(i):
        calls[i]()

    prewarm(step, n_rot, args.prewarm_s)
    total_ms = time_steps(step, args.steps, args.warmup, n_rot)
    spread = step_spread(step, args.steps, n_rot)
    return w, total_ms, total_ms / args.steps, (q, k, v), spread


def bench_unnormalized(args, torch, la, inp):
    """The headline workload through la_causal_fwd_unnormalized (numerators
    only), timed the same way with the same rotated input sets."""
    w = inp.WORKLOADS[inp.HEADLINE]
    dev = torch.device("cuda:0")
    q, k, v = inp.workload_inputs(w)
    n_rot = args.rotate
    sets = [(q.to(dev), k.to(dev), v.to(dev), torch.empty(w.B, w.H, w.N, w.d, dtype=torch.float32, device=dev))
            for _ in range(n_rot)]
    ws = torch.empty(max(1, la.la_causal_fwd_workspace(w.B, w.H, w.N, w.d, w.chunk)),
                     dtype=torch.uint8, device=dev)
    calls = [la.prepare_causal_fwd(a[0], a[1], a[2], a[3], chunk=w.chunk, eps=w.eps, workspace=ws, normalize=False)
             for a in sets]

    def step(i):
        calls[i]()

    prewarm(step, n_rot, args.prewarm_s)
    total_ms = time_steps(step, args.steps, args.warmup, n_rot)
    per_call = total_ms / args.steps
    return {"workload": w.name + "_unnormalized", "value": round(w.head_tokens / (per_call * 1e-3), 1),
            "unit": "head-tokens/s", "ms_per_step": round(per_call, 5),
            "roofline": roofline(alg_bytes_causal(w), per_call, None)}


def bench_segmented(args, torch, la, inp):
    w = inp.WORKLOADS[inp.SEGMENTED]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inp.workload_inputs(w))
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    zs = [torch.zeros(B, H, d, d, device=dev) for _ in range(2)]
    ss = [torch.zeros(B, H, d, device=dev) for _ in range(2)]
    ws = torch.empty(max(1, la.la_causal_fwd_workspace(B, H, w.segment, d)), dtype=torch.uint8,
                     device=dev)
    nseg = N // w.segment

    calls = []
    for i in range(nseg):
        sl = slice(i * w.segment, (i + 1) * w.segment)
        calls.append(la.prepare_causal_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], out[:, :, sl], eps=w.eps,
                                           z_in=zs[i & 1] if i else None, s_in=ss[i & 1] if i else None,
                                           z_out=zs[(i + 1) & 1], s_out=ss[(i + 1) & 1], workspace=ws))

    def step(_):
        for c in calls:
            c()

    steps, warm = leg_counts(args, 20, 5)
    prewarm(step, 1, args.prewarm_s, batch=4)
    total_ms = time_steps(step, steps, warm, 1)
    ms = total_ms / steps
    seg_w = inp.Workload("segment", "causal", w.dtype, w.B, w.H, w.segment, w.d, 0, 1.0)
    b_call = alg_bytes_causal(seg_w, with_state_io=True)
    return {"workload": w.name, "value": round(w.head_tokens / (ms * 1e-3), 1), "unit": "head-tokens/s",
            "ms_per_step": round(ms, 4), "calls_per_step": nseg,
            "roofline": roofline(b_call, ms / nseg, measured_traffic(w.name))}


def bench_decode(args, torch, la, inp):
    w = inp.WORKLOADS[inp.DECODE]
    dev = torch.device("cuda:0")
    (pq, pk, pv), (sq, sk, sv) = inp.workload_inputs(w)
    B, H, d, T = w.B, w.H, w.d, w.N
    sqd, skd, svd = sq.to(dev), sk.to(dev), sv.to(dev)
    res = {}
    for label, nstate in (("hot_state", 1), ("cold_state_x4", 4)):
        zs, ss = [], []
        for _ in range(nstate):
            z = torch.empty(B, H, d, d, device=dev)
            s = torch.empty(B, H, d, device=dev)
            la.la_causal_fwd(None, pk.to(dev), pv.to(dev), None, eps=w.eps, z_out=z, s_out=s)
            zs.append(z)
            ss.append(s)
        out = torch.empty(B, H, d, device=dev)

        nst = min(T, 256)
        calls = [la.prepare_decode_step(sqd[t], skd[t], svd[t], zs[t % nstate], ss[t % nstate], out, eps=w.eps)
                 for t in range(nst)]

        def step(i):
            calls[i % nst]()

        prewarm(step, 10 ** 9, args.prewarm_s)
        total_ms = time_steps(step, nst, 16, 10 ** 9)
        ms = total_ms / nst
        bpc = B * H * (2 * (d * d + d) * 4 + 3 * d * w.dtype.itemsize + d * 4)
        res[label] = {"ms_per_step": round(ms, 5), "value": round(B * H / (ms * 1e-3), 1),
                      "roofline": roofline(bpc, ms, measured_traffic(w.name))}
    # the prefix as a full causal call with outputs: a large B*H data point
    # (not the decode target; the prefix state itself comes from a state-only
    # call, timed in the prefill workload)
    pw = inp.Workload("decode_prefix", "causal", w.dtype, B, H, int(pq.shape[2]), d, 0, 1.0)
    pqd, pkd, pvd = pq.to(dev), pk.to(dev), pv.to(dev)
    pout = torch.empty(B, H, pq.shape[2], d, dtype=torch.float32, device=dev)
    pws = torch.empty(max(1, la.la_causal_fwd_workspace(B, H, pq.shape[2], d)), dtype=torch.uint8,
                      device=dev)
    pcall = la.prepare_causal_fwd(pqd, pkd, pvd, pout, eps=w.eps, workspace=pws)
    psteps, pwarm = leg_counts(args, 10, 2)
    pms = time_steps(lambda _: pcall(), psteps, pwarm, 1) / psteps
    res["prefix_causal_with_outputs"] = {"shape": [B, H, int(pq.shape[2]), d], "ms_per_call": round(pms, 4),
                                         "value": round(B * H * pq.shape[2] / (pms * 1e-3), 1),
                                         "roofline": roofline(alg_bytes_causal(pw), pms)}
    return {"workload": w.name, "unit": "head-tokens/s", **res}


def bench_noncausal(args, torch, la, inp):
    w = inp.WORKLOADS[inp.NONCAUSAL]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inp.workload_inputs(w))
    out = torch.empty(w.B, w.H, w.N, w.d, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, la.la_noncausal_workspace(w.B, w.H, w.N, w.d)), dtype=torch.uint8, device=dev)

    call = la.prepare_noncausal_fwd(q, k, v, out, eps=w.eps, workspace=ws)

    def step(_):
        call()

    steps, warm = leg_counts(args, 20, 5)
    prewarm(step, 1, args.prewarm_s, batch=2)
    total_ms = time_steps(step, steps, warm, 1)
    per_call = total_ms / steps
    return {"workload": w.name, "value": round(w.head_tokens / (per_call * 1e-3), 1), "unit": "head-tokens/s",
            "ms_per_step": round(per_call, 4),
            "roofline": roofline(alg_bytes_causal(w), per_call, measured_traffic(w.name))}


def bench_memory(args, torch, la, inp):
    """The compressive-memory loop: 32 la_memory_fwd calls of 2048 tokens,
    each reading the memory of the earlier segments and adding its own."""
    w = inp.WORKLOADS[inp.MEMORY]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inp.workload_inputs(w))
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    zs = [torch.zeros(B, H, d, d, device=dev) for _ in range(2)]
    ss = [torch.zeros(B, H, d, device=dev) for _ in range(2)]
    ws = torch.empty(max(1, la.la_memory_workspace(B, H, w.segment, d)), dtype=torch.uint8, device=dev)
    nseg = N // w.segment
    calls = []
    for i in range(nseg):
        sl = slice(i * w.segment, (i + 1) * w.segment)
        calls.append(la.prepare_memory_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], out[:, :, sl], eps=w.eps,
                                           z_in=zs[i & 1] if i else None, s_in=ss[i & 1] if i else None,
                                           z_out=zs[(i + 1) & 1], s_out=ss[(i + 1) & 1], workspace=ws))

    def step(_):
        for c in calls:
            c()

    steps, warm = leg_counts(args, 20, 5)
    prewarm(step, 1, args.prewarm_s, batch=4)
    total_ms = time_steps(step, steps, warm, 1)
    ms = total_ms / steps
    seg_w = inp.Workload("segment", "memory", w.dtype, w.B, w.H, w.segment, w.d, 0, 1.0)
    b_call = alg_bytes_causal(seg_w, with_state_io=True)
    return {"workload": w.name, "value": round(w.head_tokens / (ms * 1e-3), 1), "unit": "head-tokens/s",
            "ms_per_step": round(ms, 4), "calls_per_step": nseg,
            "roofline": roofline(b_call, ms / nseg, measured_traffic(w.name))}


def bench_prefill(args, torch, la, inp):
    """State-only calls (out = NULL, no q): the prefill, which needs only the
    state after the prompt.  On the headline shape (B4 H8 N4096 d64) and on
    the decode workload's prefix (B64 H32 N1024 d128).  Algorithmic bytes:
    k and v once (bf16) plus the fp32 state written."""
    dev = torch.device("cuda:0")
    res = {}
    for label, w in (("headline_shape", inp.WORKLOADS[inp.HEADLINE]), ("decode_prefix", inp.WORKLOADS[inp.DECODE])):
        N = w.prefix if w.kind == "decode" else w.N
        g = inp.make_generator(w.seed + 100)
        k, v = (inp.draw((w.B, w.H, N, w.d), g, w.dtype, w.scale).to(dev) for _ in range(2))
        z = torch.empty(w.B, w.H, w.d, w.d, device=dev)
        s = torch.empty(w.B, w.H, w.d, device=dev)
        ws = torch.empty(max(1, la.la_causal_fwd_workspace(w.B, w.H, N, w.d)), dtype=torch.uint8, device=dev)
        call = la.prepare_causal_fwd(None, k, v, None, eps=w.eps, z_out=z, s_out=s, workspace=ws)
        steps, warm = leg_counts(args, 50, 10)
        prewarm(lambda _: call(), 1, args.prewarm_s)
        ms = time_steps(lambda _: call(), steps, warm, 1) / steps
        b = w.B * w.H * (N * 2 * w.d * w.dtype.itemsize + (w.d * w.d + w.d) * 4)
        traffic = measured_traffic("prefill_bf16_b4h8n4096d64") if label == "headline_shape" else None
        res[label] = {"shape": [w.B, w.H, N, w.d], "ms_per_call": round(ms, 5),
                      "value": round(w.B * w.H * N / (ms * 1e-3), 1), "unit": "head-tokens/s",
                      "alg_bytes_per_call": b, "roofline": roofline(b, ms, traffic)}
    return res


def bench_backward(args, torch, la, inp):
    """la_causal_bwd on the headline shape (B4 H8 N4096 d64, bf16 q, k, v;
    fp32 out from the forward call and fp32 dout): dq, dk, dv.  Algorithmic
    bytes: q, k, v (bf16), out and dout (fp32) read once, dq, dk, dv (fp32)
    written once: 26 d bytes per head-token."""
    w = inp.WORKLOADS[inp.HEADLINE]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inp.workload_inputs(w))
    dout = torch.randn(w.B, w.H, w.N, w.d, generator=torch.Generator().manual_seed(w.seed + 7)).to(dev)
    out = torch.empty(w.B, w.H, w.N, w.d, device=dev)
    la.la_causal_fwd(q, k, v, out, eps=w.eps)
    dq, dk, dv = (torch.empty(w.B, w.H, w.N, w.d, device=dev) for _ in range(3))
    ws = torch.empty(max(1, la.la_causal_bwd_workspace(w.B, w.H, w.N, w.d)), dtype=torch.uint8, device=dev)
    call = la.prepare_causal_bwd(q, k, v, out, dout, dq, dk, dv, eps=w.eps, workspace=ws)
    steps, warm = leg_counts(args, 50, 10)
    prewarm(lambda _: call(), 1, args.prewarm_s, batch=10)
    ms = time_steps(lambda _: call(), steps, warm, 1) / steps
    b = w.head_tokens * (3 * w.d * w.dtype.itemsize + 2 * 4 * w.d + 3 * 4 * w.d)
    return {"workload": w.name + "_backward", "value": round(w.head_tokens / (ms * 1e-3), 1),
            "unit": "head-tokens/s", "ms_per_step": round(ms, 5), "alg_bytes_per_call": b,
            "roofline": roofline(b, ms, measured_traffic("backward_bf16_b4h8n4096d64"))}


def cpu_baseline(w, qkv, seconds):
    """The fp64 oracle, as it is, on the host cores: whole steps of the same
    workload repeated until `seconds` of wall time have passed (at least 2)."""
    import oracle
    q, k, v = qkv
    reps = 0
    t0 = time.perf_counter()
    while reps < 2 or time.perf_counter() - t0 < seconds:
        oracle.causal(q, k, v, w.eps)
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": round(reps * w.head_tokens / dt, 1), "unit": "head-tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{reps} whole steps of {w.name} (all {w.B * w.H} heads x {w.N} tokens each), "
                      f"fp64 recurrent form, run back to back for about {seconds:g} s"}


LEGS = ("headline", "segmented", "decode", "noncausal", "memory", "unnormalized", "prefill", "backward")
LEG_FNS = {"segmented": bench_segmented, "decode": bench_decode, "noncausal": bench_noncausal,
           "memory": bench_memory, "unnormalized": bench_unnormalized, "prefill": bench_prefill,
           "backward": bench_backward}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=8, help="input/output sets rotated over the steps")
    ap.add_argument("--prewarm-s", type=float, default=0.25,
                    help="seconds of untimed headline calls before the warm-up steps (GPU clock ramp)")
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--only", default=None,
                    help="comma-separated workloads to run, of " + ",".join(LEGS) + " (profiling runs; "
                         "without 'headline' the line carries only the workloads object)")
    ap.add_argument("--leg-steps", type=int, default=None, help="timed repetitions of each non-headline workload")
    ap.add_argument("--leg-warmup", type=int, default=None, help="warm-up repetitions of each non-headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall time given to the oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (the reference kernel for scaling "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import segment_wise_compressive_amd as la
    from segment_wise_compressive_amd import inputs as inp
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = 256 * 1024 * 1024  # float32 elements = 1 GiB
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n, "launches": 3}))
        return
    la.load_library()
    legs = LEGS if args.only is None else tuple(x.strip() for x in args.only.split(","))
    unknown = [x for x in legs if x not in LEGS]
    if unknown:
        print(f"unknown workloads {unknown}; choose from {LEGS}", file=sys.stderr)
        sys.exit(2)
    if args.headline_only:
        legs = ("headline",)
    if "headline" not in legs:
        line = {"workloads": {}}
        for name in legs:
            log(f"{name} workload ...")
            line["workloads"][name] = LEG_FNS[name](args, torch, la, inp)
        print(json.dumps(line), flush=True)
        return

    log("headline workload ...")
    w, total_ms, per_call, qkv, spread = bench_headline(args, torch, la, inp)
    ms_step = total_ms / args.steps
    line = {
        "metric": METRIC,
        "value": round(w.head_tokens * args.steps / (total_ms * 1e-3), 1),
        "unit": "head-tokens/s (B*H*N per second)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "chunk": w.chunk,
                   "input_dtype": "bf16", "state_and_output_dtype": "fp32", "eps": w.eps, "seed": w.seed,
                   "rotated_sets": args.rotate},
        "roofline": roofline(alg_bytes_causal(w), per_call, measured_traffic(w.name)),
    }
    line["roofline"]["kernels"] = ("k_cs_fwd (one launch per la_causal_fwd call); duration = HIP-event time "
                                   "of the timed back-to-back calls / calls")
    line["step_spread"] = spread
    copy_gbs = copy_bandwidth(torch)
    line["roofline"]["copy_1gib_gbs"] = copy_gbs
    line["roofline"]["frac_of_copy"] = round(line["roofline"]["achieved"] / copy_gbs, 4)
    for name in legs:
        if name != "headline":
            log(f"{name} workload ...")
            line.setdefault("workloads", {})[name] = LEG_FNS[name](args, torch, la, inp)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(w, qkv, args.cpu_seconds)
        line["cpu_baseline"]["gpu_over_cpu"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
