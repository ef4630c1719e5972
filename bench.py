"""Throughput of the H3 attention node on one MI355X.

Forward (default): one step = one h3attn_fwd call (segment plan, Q and K norm + fp16 V staging,
attention) over the full workload, inputs resident in HBM; by default the step is captured once in
a HIP graph and replayed (--launch eager: one library call per step), and its output is checked bit
for bit against an eager step.  Before the W warmup steps, untimed steps run for --prewarm-s seconds
so the clocks reach steady state.  Prints ONE JSON line:
  value     whole-step attention TFLOP/s (nominal 4 * sum(L^2) * H * 128 FLOPs per step)
  roofline  the attention kernel alone (h3attn_attend), timed per launch with HIP events on the
            launch stream, against the bf16/fp16 dense MFMA peak (2516.6 TFLOP/s)
  config.hbm  algorithmic bytes per step over the step time, warm (the previous step's data in the
            256 MB MALL) and cold (a 512 MiB write before each step, untimed), against 8 TB/s
  cpu_baseline  the FP64 CPU oracle on a bounded sample of query rows of the same workload (with
            the host's CPU model and the time of each growing probe)
  parity    the benched output on those same rows against the oracle (relative L2 and max abs,
            with the bounds 2e-3 / 2e-2): the accuracy of the timed output itself
Backward (--pass bwd, default workload batch2): one step = one h3attn_bwd_ex call (plan, operand
staging with D = dO . O, dq, dk/dv, weight-gradient reduction) given dO and the forward's LSE and
fp32 output (--d-from recompute: D recomputed by the dq kernel instead, h3attn_bwd); TFLOP/s on
the nominal 2.5 x forward FLOPs; the CPU baseline is the FP64 oracle's gradients on a subset of
heads.
--order position: the tokens of every segment are shuffled (seeded) and the step calls the
position-ordered entry points (h3attn_fwd_pos / h3attn_bwd_pos) with their position ids.
--rope grid|random: the step calls h3attn_fwd_ex / h3attn_bwd_ex with MM-RoPE tables (the node
between the q/k norm and the attention), and the CPU baseline and parity take the oracle with the
same tables.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long] [--pass fwd|bwd]
                       [--order packed|position] [--rope none|grid|random] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak @8349 tok; bitwise batch-invariant"
METRIC_BWD = "attention bwd TFLOP/s (nominal 2.5x fwd FLOPs) + % bf16 MFMA peak @2x4253 tok; bitwise batch-invariant"
PEAK_MFMA_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_bytes(workload):
    """HBM bytes per launch of the attention kernel, from the counter summary committed under
    profiles/ (FETCH_SIZE + WRITE_SIZE of one dispatch, each scaled by the same counter's reading for
    the calibration kernel), or None when there is none for this workload or the kernel source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"k_attn_fwd_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return int(rec["traffic_bytes"])


FWD_KERNEL_SOURCES = ("k_attn_fwd.hip", "h3_tiles.h", "h3_common.h")


def kernel_source_sha256():
    """sha256 over the attention kernel's source and the headers it includes, in that order."""
    import hashlib
    h = hashlib.sha256()
    for name in FWD_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "deterministic_invariant_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="default: long (fwd), batch2 (bwd)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd")
    ap.add_argument("--order", choices=("packed", "position"), default="packed",
                    help="position: shuffle each segment's tokens and pass their position ids")
    ap.add_argument("--rope", choices=("none", "grid", "random"), default="none",
                    help="MM-RoPE tables for the normed q and k (workloads.rope_tables of this kind)")
    ap.add_argument("--d-from", dest="d_from", choices=("o32", "recompute"), default="o32",
                    help="backward: D = dO . O from the forward's fp32 output (h3attn_bwd_ex), or recomputed "
                         "from P and dP by the dq kernel (h3attn_bwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time of the CPU sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (the reference kernel for HBM byte counters)")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="graph: the step is captured once in a HIP graph and replayed (its outputs are checked "
                         "bit for bit against an eager step); eager: one library call per step")
    ap.add_argument("--prewarm-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warmup steps, so the clocks reach steady state")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the attention node shards by head or packed row with no exchange",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import deterministic_invariant_attention_amd as h3
    import workloads

    if args.which == "bwd":
        return bench_bwd(args, workloads.WORKLOADS[args.workload or "batch2"])
    wl = workloads.WORKLOADS[args.workload or "long"]
    dev = torch.device("cuda:0")
    x, pos = ordered_inputs(workloads.make_inputs(wl), wl, args.order, dev)
    rope = rope_inputs(wl, args, dev)
    g = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    T, H = wl.tokens, wl.heads
    flops = wl.flops()
    out = torch.empty_like(g["q"])
    ws = h3.workspace(T, H, dev)
    stream = torch.cuda.current_stream(dev)
    log(f"workload {wl.name}: {wl.description}; nominal {flops:.4e} FLOP/step")

    if args.copy_calibration:
        copy_calibration(dev)

    def eager_step(st):
        if rope is not None:
            h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], pos, g["wq"], g["wk"], eps=wl.eps, scale=wl.scale,
                             out=out, workspace_buf=ws, stream=st, rope_cos=rope[0], rope_sin=rope[1])
        elif pos is None:
            h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=wl.eps, scale=wl.scale, out=out,
                          workspace_buf=ws, stream=st)
        else:
            h3.h3attn_fwd_pos(g["q"], g["k"], g["v"], g["seg"], pos, g["wq"], g["wk"], eps=wl.eps, scale=wl.scale,
                              out=out, workspace_buf=ws, stream=st)

    # the reference bits: one eager step
    eager_step(stream)
    torch.cuda.synchronize()
    ref_bits = out.view(torch.int16).clone()
    step = lambda: eager_step(stream)  # noqa: E731
    if args.launch == "graph":
        # The library allocates nothing and clears its counters with its own kernels (no memset), so a
        # step is capturable as it stands; each replay enqueues the same three kernels.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step(torch.cuda.current_stream(dev))
        step = graph.replay
    # untimed steps until the clocks have settled (they ramp during the first ~0.1 s of load), then the
    # warmup steps proper
    t_end = time.perf_counter() + args.prewarm_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = e0.elapsed_time(e1) / args.steps
    repeat_bitwise = bool(torch.equal(out.view(torch.int16), ref_bits))
    status = h3.h3attn_status_read(ws, stream)
    value = flops / (ms_per_step * 1e-3) / 1e12
    log(f"step: {ms_per_step:.4f} ms (wall {wall_ms:.4f} ms) -> {value:.1f} TFLOP/s; repeat bitwise {repeat_bitwise}; "
        f"status {status}")

    # ---- the dominant kernel alone: attention launches, one event pair each, on the launch stream
    h3.h3attn_plan(g["seg"], H, ws, stream=stream)
    h3.h3attn_prep_qkv(g["q"], g["k"], g["v"], g["wq"], g["wk"], ws, eps=wl.eps, stream=stream)
    for _ in range(2):
        h3.h3attn_attend(g["q"], g["wq"], ws, out, eps=wl.eps, scale=wl.scale, stream=stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        h3.h3attn_attend(g["q"], g["wq"], ws, out, eps=wl.eps, scale=wl.scale, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in evs]
    attn_ms = float(np.mean(kms))
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    log(f"attention kernel: mean {attn_ms:.4f} ms, median {np.median(kms):.4f} ms -> {attn_tflops:.1f} TFLOP/s "
        f"({100 * attn_tflops / PEAK_MFMA_TFLOPS:.1f}% of bf16 MFMA peak)")

    # ---- algorithmic HBM rate of the whole step, warm (inputs left in the 256 MB MALL by the previous
    # step) and cold (a 512 MiB write evicts them before each step; the scrub is not timed)
    alg_bytes = wl.algorithmic_bytes()
    scrub = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(max(5, min(args.steps, 20))):
        scrub.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del scrub
    cold_ms = float(np.median(cold))
    hbm = {"algorithmic_bytes": alg_bytes, "warm_GBps": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 1),
           "cold_GBps": round(alg_bytes / (cold_ms * 1e-3) / 1e9, 1), "cold_ms_per_step": round(cold_ms, 4),
           "peak_GBps": PEAK_HBM_GBS}
    log(f"HBM (algorithmic bytes / step time): warm {hbm['warm_GBps']} GB/s, cold {hbm['cold_GBps']} GB/s "
        f"({cold_ms:.4f} ms per cold step)")

    # ---- CPU baseline: the FP64 oracle on a bounded sample of query rows (rank 0, N = 1); the same
    # rows of the benched output are then checked against it (the accuracy of the timed output)
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        import oracle
        seg_np = x["seg"].numpy()
        rng = np.random.default_rng(0)
        L = max(wl.seg_lens)

        def run_rows(n):
            rows = np.arange(T) if n == T else np.sort(rng.choice(T, size=n, replace=False))
            t1 = time.perf_counter()
            if rope is None:
                ref = oracle.fwd_rows(x["q"], x["k"], x["v"], seg_np, rows, x["wq"], x["wk"], wl.eps, wl.scale)[0]
            else:
                ref = oracle.fwd_ex(x["q"], x["k"], x["v"], seg_np, x["wq"], x["wk"], wl.eps, wl.scale,
                                    cos=rope[0].cpu(), sin=rope[1].cpu(), rows=rows)[0]
            return rows, ref, time.perf_counter() - t1

        # grow the sample until it takes at least half the target time (or is the whole workload)
        n, probes = min(32, T), []
        while True:
            rows, ref, dt = run_rows(n)
            probes.append([int(n), round(dt, 3)])
            if dt >= 0.5 * args.cpu_seconds or n == T:
                break
            n = int(min(T, max(2 * n, n * args.cpu_seconds / max(dt, 1e-3))))
        starts, lens = oracle.segments(seg_np)
        seg_len = np.repeat(lens, lens)
        sample_flops = float(4.0 * np.sum(seg_len[rows]) * H * 128)
        cpu = {"value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{len(rows)} of {T} query rows x {H} heads of the {wl.name} workload "
                         f"(segment length {L}); {dt:.1f} s FP64",
               "cpu_model": cpu_model(), "probes_rows_seconds": probes}
        log(f"cpu baseline: {cpu}")
        # (with --order position both the benched output and the oracle's rows are in the shuffled
        # packing order of x)
        got = out.float().cpu().double().numpy()[rows]
        diff = got - ref
        parity = {"rows": int(len(rows)), "of_rows": T, "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref)),
                  "max_abs": float(np.max(np.abs(diff))), "bound_rel_l2": 2e-3, "bound_max_abs": 2e-2}
        parity["ok"] = bool(parity["rel_l2"] <= 2e-3 and parity["max_abs"] <= 2e-2)
        log(f"benched output vs oracle: {parity}")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "heads": H, "head_dim": 128, "segments": list(wl.seg_lens),
                   "qk_draw_scale": wl.qk_scale, "pv_operands": "fp16", "accumulate": "fp32",
                   "key_order": args.order, "rope": args.rope, "launch": args.launch,
                   "pct_bf16_mfma_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
                   "algorithmic_GBps": round(wl.algorithmic_bytes() / (ms_per_step * 1e-3) / 1e9, 1),
                   "hbm": hbm, "repeat_bitwise": repeat_bitwise, "device_status": status},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_MFMA_TFLOPS, 4),
                     "traffic": traffic_bytes(wl.name), "kernel": "k_attn_fwd", "kernel_ms": round(attn_ms, 4)},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_calibration(dev):
    """A plain elementwise kernel of known traffic (256 MiB read, 256 MiB written), the reference
    that scales the FETCH_SIZE / WRITE_SIZE counters of a --pmc run into bytes.  Its grid (64 Mi
    elements) tells it apart from every other dispatch of the run."""
    import torch
    src = torch.full((64 << 20,), 1.0, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    scrub = torch.full((128 << 20,), 0.0, dtype=torch.float32, device=dev)  # 512 MiB: evicts the 256 MB MALL
    torch.cuda.synchronize()
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    log("copy calibration: torch.mul over 67108864 fp32 (268435456 bytes read + 268435456 bytes written)")
    del src, dst, scrub


def ordered_inputs(x, wl, order, dev):
    """packed: the inputs as drawn, no position ids.  position: every segment's tokens shuffled
    (seed 11) and the matching position ids on the device."""
    if order == "packed":
        return x, None
    import workloads
    p = workloads.shuffle_within_segments(wl.seg_lens, 11)
    x = {n: (t[p].contiguous() if n in ("q", "k", "v", "dout") else t) for n, t in x.items()}
    return x, workloads.position_ids(wl.seg_lens)[p].contiguous().to(dev)


def rope_inputs(wl, args, dev):
    """--rope: float32 [T, 48] cosine and sine tables on the device (token order of the inputs: with
    --order position they follow the same shuffle as the tokens), else None."""
    if args.rope == "none":
        return None
    import workloads
    c, s = workloads.rope_tables(wl.seg_lens, args.rope)
    if args.order == "position":
        p = workloads.shuffle_within_segments(wl.seg_lens, 11)
        c, s = c[p].contiguous(), s[p].contiguous()
    return c.to(dev), s.to(dev)


def bench_bwd(args, wl):
    import numpy as np
    import torch

    import deterministic_invariant_attention_amd as h3
    import workloads

    dev = torch.device("cuda:0")
    x, pos = ordered_inputs(workloads.make_inputs(wl, with_grad=True), wl, args.order, dev)
    rope = rope_inputs(wl, args, dev)
    rc, rs = (None, None) if rope is None else rope
    g = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    T, H = wl.tokens, wl.heads
    flops = 2.5 * wl.flops()
    stream = torch.cuda.current_stream(dev)
    log(f"workload {wl.name} backward: {wl.description}; nominal {flops:.4e} FLOP/step (2.5 x forward)")
    if args.copy_calibration:
        copy_calibration(dev)
    # the forward that precedes the backward (not timed): LSE, and the fp32 output when D comes from it
    _, lse, o32 = h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], pos, g["wq"], g["wk"], eps=wl.eps,
                                   scale=wl.scale, want_lse=True, want_o32=args.d_from == "o32", stream=stream,
                                   rope_cos=rc, rope_sin=rs)
    ws = h3.bwd_workspace(T, H, dev)
    outs = [torch.empty_like(g["q"]) for _ in range(3)]
    dw = [torch.empty(128, dtype=torch.float32, device=dev) for _ in range(2)]

    def step():
        h3.h3attn_bwd_ex(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], pos, o32, g["wq"], g["wk"], eps=wl.eps,
                         scale=wl.scale, dq=outs[0], dk=outs[1], dv=outs[2], dwq=dw[0], dwk=dw[1], workspace_buf=ws,
                         stream=stream, rope_cos=rc, rope_sin=rs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs + dw]

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = float(np.mean(ms))
    repeat_bitwise = all(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                                     b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
                         for a, b in zip(outs + dw, ref))
    status = h3.h3attn_status_read(ws, stream)
    value = flops / (ms_per_step * 1e-3) / 1e12
    log(f"bwd step: mean {ms_per_step:.4f} ms, median {np.median(ms):.4f} ms (wall {wall_ms:.4f} ms) -> "
        f"{value:.1f} TFLOP/s ({100 * value / PEAK_MFMA_TFLOPS:.1f}% of peak); repeat bitwise {repeat_bitwise}; "
        f"status {status}")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        seg_np = x["seg"].numpy()

        def run_heads(nh):
            sub = {n: x[n][:, :nh].contiguous() for n in ("q", "k", "v", "dout")}
            t1 = time.perf_counter()
            oracle.bwd(sub["q"], sub["k"], sub["v"], seg_np, sub["dout"], x["wq"], x["wk"], wl.eps, wl.scale,
                       cos=None if rope is None else rc.cpu(), sin=None if rope is None else rs.cpu())
            return time.perf_counter() - t1

        nh = 1
        while True:
            dt = run_heads(nh)
            if dt >= 0.5 * args.cpu_seconds or nh == H:
                break
            nh = int(min(H, max(2 * nh, nh * args.cpu_seconds / max(dt, 1e-3))))
        cpu = {"value": round(flops * nh / H / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"gradients of {nh} of {H} heads, all {T} tokens of the {wl.name} workload; {dt:.1f} s FP64"}
        log(f"cpu baseline: {cpu}")

    line = {
        "metric": METRIC_BWD,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + "-bwd", "tokens": T, "heads": H, "head_dim": 128,
                   "segments": list(wl.seg_lens), "products": "fp16 P, dS, dO, q/k hat; fp32 accumulate",
                   "key_order": args.order, "rope": args.rope, "d_from": args.d_from,
                   "pct_bf16_mfma_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
                   "repeat_bitwise": repeat_bitwise, "device_status": status},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_MFMA_TFLOPS, 4), "traffic": None,
                     "kernel": "h3attn_bwd (all launches of one call)", "kernel_ms": round(ms_per_step, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
