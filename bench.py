"""Benchmark of the MI355X M2RNN scan: head-tokens/s for forward + backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole scan path over one batch of seeded synthetic
inputs already resident in HBM: the forward with state checkpoints every 64
steps, then the backward (recompute from the checkpoints, reverse sweep, head
and batch reductions).  `--pass fwd` times the forward alone.  Prints ONE JSON
line.  The roofline object prices the dominant kernel's algorithmic work
(2*K*V^2 MFMA flop per head-token per state contraction) against MI355X's
published dense fp32 matrix peak; its duration is measured with HIP events
recorded on the stream the kernel runs on.  The CPU baseline is the fp64
oracle, timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
HBM_PEAK_GBS = 8000.0
K_DIM, V_DIM = 64, 16
FLOP_PER_CONTRACTION = 2 * K_DIM * V_DIM * V_DIM   # H W per head-token


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--pass", dest="which", choices=["fwdbwd", "fwd", "epilogue", "prologue", "decode"],
                    default="fwdbwd",
                    help="epilogue: the output gate and RMSNorm after the readout; prologue: the causal Conv1D "
                         "and SiLU of q, k and v (each forward + backward); decode: one token per call. "
                         "--workload picks a scan workload and with it the pass")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the oracle CPU-baseline sample")
    ap.add_argument("--copy-calibration-bytes", type=int, default=0,
                    help="also run one plain device-to-device copy of this many bytes (for scaling the "
                         "HBM byte counters of a profiler run)")
    return ap.parse_args()


def algorithmic_bytes_fwd(w):
    """HBM bytes the forward must move: inputs once, y and H_T (fp32) once,
    checkpoints once."""
    s = 2 if w.dtype == "bf16" else 4
    B, T, N = w.B, w.T, w.N
    ins = (2 * B * T * K_DIM + B * T * N * V_DIM + B * T * N + N * V_DIM * V_DIM + N * V_DIM) * s
    outs = (B * T * N * V_DIM + B * N * K_DIM * V_DIM) * 4
    ck = B * N * ((T + 63) // 64) * K_DIM * V_DIM * 4 if w.ckpt_every else 0
    return ins + outs + ck


# the sources each profiled workload's kernels are built from
KERNEL_SOURCES = {
    "scan": ("m2rnn_fwd.hip", "m2rnn_bwd.hip"),
    "gate_rmsnorm": ("m2rnn_norm.hip", "m2rnn_colsum.hip"),
    "conv_silu": ("m2rnn_conv.hip", "m2rnn_colsum.hip"),
}


def kernel_source_sha256(kind):
    """sha256 over the kernel sources of `kind` and the shared device headers,
    with comments and blank space taken out: an edit to comments alone leaves
    the kernels, and the counters taken of them, as they were."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in (*KERNEL_SOURCES[kind], "m2rnn_device.h", "m2rnn_internal.h"):
        with open(os.path.join(ROOT, "non_linear_matrix_amd", "csrc", name), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
        h.update(text.encode("utf-8"))
    return h.hexdigest()


def workload_kind(workload):
    for kind in ("gate_rmsnorm", "conv_silu"):
        if workload.startswith(kind):
            return kind
    return "scan"


def profiled_traffic(workload, which):
    """HBM bytes per launch from the committed profiler summary for this
    workload (two rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by
    a plain copy of known size), or None when there is none or the kernel
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"m2rnn_{workload}_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch_backward",
                                                       "traffic_bytes_per_launch_forward", "source_sha256"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("source_sha256") != kernel_source_sha256(workload_kind(workload)):
        return None
    key = "traffic_bytes_per_launch_backward" if which == "bwd" else "traffic_bytes_per_launch_forward"
    return float(vals[key]) if key in vals else None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, x, which, threads, seconds):
    """The fp64 oracle timed on a bounded sample of the same inputs: the first
    batch rows and heads at the full length, on every host core (one thread
    per core the OS reports), sized from a short calibration run so that each
    of three timed runs takes about a quarter of `seconds`; the value is the
    median of the three.  A run on one thread over a smaller sample gives the
    per-core rate."""
    import statistics
    import oracle
    nthreads = threads or (os.cpu_count() or 1)
    T = w.T

    def run(Bs, Ns, nth):
        sl = dict(q=x["q"][:Bs], k=x["k"][:Bs], v=x["v"][:Bs, :, :Ns], f=x["f"][:Bs, :, :Ns],
                  W=x["W"][:Ns], wr=x["wr"][:Ns])
        ins = [sl[n].double().numpy() for n in ("q", "k", "v", "f", "W", "wr")]
        dy = x["dy"][:Bs, :, :Ns].double().numpy() if which == "fwdbwd" else None
        t0 = time.perf_counter()
        oracle.forward(*ins, nthreads=nth)
        if which == "fwdbwd":
            oracle.backward(*ins, dy, nthreads=nth)
        return time.perf_counter() - t0

    def shape_for(chains):   # the first `chains` (b, n) chains, whole batch rows first
        chains = max(1, min(w.B * w.N, chains))
        Ns = min(w.N, chains)
        return max(1, min(w.B, chains // Ns)), Ns

    # calibration: as many chains as threads (at least one batch row's worth)
    Bc, Nc = shape_for(nthreads)
    rate = Bc * Nc * T / max(run(Bc, Nc, nthreads), 1e-6)          # head-tokens/s on all threads
    Bs, Ns = shape_for(max(nthreads, int(seconds / 4 * rate / T)))
    times = [run(Bs, Ns, nthreads) for _ in range(3)]
    dt = statistics.median(times)
    htok = Bs * T * Ns
    cores = min(nthreads, Bs * Ns)
    # one thread: a sample about 1/8 of the budget
    B1, N1 = shape_for(int(seconds / 8 * rate / max(cores, 1) / T))
    t1 = run(B1, N1, 1)
    return {"value": htok / dt, "unit": "head-tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{'forward+backward' if which == 'fwdbwd' else 'forward'} of the fp64 oracle on the first "
                      f"B={Bs} batch rows x N={Ns} heads at T={T} of the same inputs ({htok} head-tokens): median "
                      f"of 3 runs ({', '.join(f'{t:.2f}' for t in times)} s) on {cores} threads",
            "cpu_model": cpu_model(), "host_cores": os.cpu_count(),
            "per_core_value": B1 * N1 * T / t1,
            "per_core_sample": f"B={B1} x N={N1} heads at T={T} on 1 thread, {t1:.2f} s"}


def bench_epilogue(args):
    """Output gate and RMSNorm over the B=32, T=4096, N=64 readout (d = 1024
    features per token, bf16 gate and weight): forward then backward per step.
    HBM-bound, so the roofline object prices the backward launch's algorithmic
    bytes (y, g, dout read; dy, dg written) against MI355X's 8 TB/s."""
    import torch
    import m2rnn_inputs
    import non_linear_matrix_amd as m2
    B, T, N, dtype = 32, 4096, 64, "bf16"
    name = f"gate_rmsnorm_{dtype}_B{B}_T{T}_N{N}"
    d = N * V_DIM
    x_cpu = m2rnn_inputs.make_epilogue(B, T, N, dtype, seed=args.seed)
    x = {k: v.cuda() for k, v in x_cpu.items()}
    dev = x["y"].device
    out = torch.empty_like(x["y"])
    rstd = torch.empty((B, T), device=dev)
    grads = (torch.empty_like(x["y"]), torch.empty_like(x["y"]), torch.empty((d,), device=dev))
    ws = torch.empty((m2.m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, V_DIM),), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration_bytes > 0:
        src = torch.empty(args.copy_calibration_bytes // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        m2.gate_rmsnorm_forward(x["y"], x["g"], x["w"], out=out, rstd=rstd)
        if ev is not None:
            ev[1].record(stream)
        m2.gate_rmsnorm_backward(x["y"], x["g"], x["w"], x["dout"], out=grads, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(events[i])
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    ntok = B * T
    es = 2 if dtype == "bf16" else 4
    fwd_bytes = ntok * d * (4 + es + 4) + ntok * 4            # y, g read; out, rstd written
    bwd_bytes = ntok * d * (4 + es + 4 + 4 + 4)               # y, g, dout read; dy, dg written
    achieved = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    htok = ntok * N
    res = {
        "metric": "M2RNN output gate + RMSNorm head-tokens/s (N*V = 1024 features per token) fwd & bwd; "
                  "% of HBM roofline",
        "value": htok * args.steps / (total_ms * 1e-3),
        "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in (g, w), fp32 y and arithmetic",
        "data": "synthetic (seeded; y = 3 N(0,1), g = sigmoid(N(0,1)), w = 1 + N(0,1/100), dout = N(0,1))",
        "config": {"workload": name, "pass": "forward+backward", "B": B, "T": T, "N": N, "V": V_DIM,
                   "input_dtype": dtype, "eps": 0.0},
        "copy_calibration_bytes": args.copy_calibration_bytes,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "fwd_GBs": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(name, "bwd"),
                     "kernel": "m2rnn_gate_rmsnorm_backward (norm_bwd_kernel + two dw reduction launches)",
                     "kernel_ms": bwd_ms,
                     "algorithmic": f"{bwd_bytes // ntok} B/token x {ntok} tokens per launch"},
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = max(1, min(ntok, int(args.cpu_seconds * 2.0e5)))   # ~5 us per token row fwd + bwd
        yy = x_cpu["y"].reshape(-1, d)[:rows].double().numpy()
        gg = x_cpu["g"].reshape(-1, d)[:rows].double().numpy()
        ww = x_cpu["w"].reshape(d).double().numpy()
        dd = x_cpu["dout"].reshape(-1, d)[:rows].double().numpy()
        c0 = time.perf_counter()
        oracle.gate_rmsnorm_forward(yy, gg, ww)
        oracle.gate_rmsnorm_backward(yy, gg, ww, dd)
        dt = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": rows * N / dt, "unit": "head-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"forward+backward of the fp64 oracle on the first {rows} token rows "
                                         f"(d = {d}) of the same inputs, {dt:.1f} s on 1 thread"}
    print(json.dumps(res), flush=True)
    return 0


def bench_prologue(args):
    """Causal Conv1D (width 4) and SiLU of q, k (C = 64 each) and v (C = N V
    = 1024) at B=32, T=4096, N=64, bf16: the three forward calls, then the
    three backward calls, per step.  HBM-bound: the roofline object prices the
    v backward launch's algorithmic bytes (u and dz read, du written) against
    MI355X's 8 TB/s."""
    import torch
    import m2rnn_inputs
    import non_linear_matrix_amd as m2
    B, T, N, dtype = 32, 4096, 64, "bf16"
    name = f"conv_silu_{dtype}_B{B}_T{T}_N{N}"
    chans = {"q": K_DIM, "k": K_DIM, "v": N * V_DIM}
    xs = {n: {k: t.cuda() for k, t in m2rnn_inputs.make_conv(B, T, C, dtype, seed=args.seed + i).items()}
          for i, (n, C) in enumerate(chans.items())}
    dev = xs["q"]["u"].device
    zs = {n: torch.empty_like(x["u"]) for n, x in xs.items()}
    gs = {n: (torch.empty(x["u"].shape, device=dev), torch.empty((chans[n], 4), device=dev),
              torch.empty((chans[n],), device=dev)) for n, x in xs.items()}
    wss = {n: torch.empty((max(1, m2.m2rnn_conv_silu_backward_workspace_bytes(B, T, chans[n])),), device=dev,
                          dtype=torch.uint8) for n in xs}
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration_bytes > 0:
        src = torch.empty(args.copy_calibration_bytes // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for n, x in xs.items():
            m2.conv_silu_forward(x["u"], x["w"], x["bias"], out=zs[n])
        if ev is not None:
            ev[1].record(stream)
        for n in ("q", "k"):
            x = xs[n]
            m2.conv_silu_backward(x["u"], x["w"], x["bias"], x["dz"], out=gs[n], workspace=wss[n])
        if ev is not None:
            ev[2].record(stream)
        x = xs["v"]
        m2.conv_silu_backward(x["u"], x["w"], x["bias"], x["dz"], out=gs["v"], workspace=wss["v"])
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(events[i])
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    bwd_qk_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    bwd_v_ms = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    es = 2 if dtype == "bf16" else 4
    elems = B * T * sum(chans.values())
    fwd_bytes = elems * 2 * es                                  # u read, z written
    v_elems = B * T * chans["v"]
    bwd_v_bytes = v_elems * (es + 4 + 4)                        # u, dz read; du written
    achieved = bwd_v_bytes / (bwd_v_ms * 1e-3) / 1e9
    htok = B * T * N
    res = {
        "metric": "M2RNN causal Conv1D(4) + SiLU of q, k, v head-tokens/s fwd & bwd; % of HBM roofline",
        "value": htok * args.steps / (total_ms * 1e-3),
        "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in and out (u, w, bias, z), fp32 arithmetic and gradients",
        "data": "synthetic (seeded; u = N(0,1), w and bias U(-1/2,1/2), dz = N(0,1))",
        "config": {"workload": name, "pass": "forward+backward", "B": B, "T": T, "N": N,
                   "channels": chans, "input_dtype": dtype},
        "copy_calibration_bytes": args.copy_calibration_bytes,
        "fwd_ms": fwd_ms, "bwd_qk_ms": bwd_qk_ms, "bwd_v_ms": bwd_v_ms,
        "fwd_GBs": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(name, "bwd"),
                     "kernel": "m2rnn_conv_silu_backward of v (conv_bwd_kernel + two column-sum launches)",
                     "kernel_ms": bwd_v_ms,
                     "algorithmic": f"{es + 8} B/element x {v_elems} elements per launch"},
    }
    if not args.no_cpu_baseline:
        import oracle
        x = m2rnn_inputs.make_conv(B, T, chans["v"], dtype, seed=args.seed + 2)
        rows = max(1, min(B, int(args.cpu_seconds / 1.5)))       # batch rows of v, about 1.5 s each
        c0 = time.perf_counter()
        u = x["u"][:rows].double().numpy()
        w, bb = x["w"].double().numpy(), x["bias"].double().numpy()
        oracle.conv_silu_forward(u, w, bb)
        oracle.conv_silu_backward(u, w, bb, x["dz"][:rows].double().numpy())
        dt = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": rows * T * N / dt, "unit": "head-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"forward+backward of the fp64 oracle on v's channels (C = {chans['v']}) "
                                         f"for the first {rows} batch rows, {dt:.1f} s on 1 thread"}
    print(json.dumps(res), flush=True)
    return 0


def sq_counters(workload):
    """Matrix-core busy and VALU busy shares per kernel from the committed
    SQ-counter summary of this workload, while the kernel sources still hash
    to the value recorded there (else None)."""
    path = os.path.join(ROOT, "profiles", f"m2rnn_{workload}_sq_counters.md")
    if not os.path.exists(path):
        return None
    out, sha = {}, None
    with open(path) as fh:
        for line in fh:
            if line.startswith("source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            cells = [c.strip() for c in line.split("|")]
            if len(cells) > 9 and cells[1].startswith("`m2rnn_") and cells[8].endswith("%"):
                out[cells[1].strip("`")] = {"mfma_busy": cells[8], "valu_busy": cells[9]}
    if sha != kernel_source_sha256(workload_kind(workload)):
        return None
    return out or None


CLOCK_GHZ = 2.4   # MI355X peak engine clock


def bench_decode(args):
    """One token per call for every (b, n) at B=32, N=64 (bf16 inputs, fp32
    state): m2rnn_decode timed per call, back to back through the C ABI (the
    value), and through the Python binding (us_per_call_python).  Each call
    reads and rewrites the whole state, 4 KB per head, so the roofline object
    prices those bytes (plus the token's inputs and y) against MI355X's 8 TB/s."""
    import torch
    import m2rnn_inputs
    import non_linear_matrix_amd as m2
    B, N, dtype = 32, 64, "bf16"
    steps = max(args.steps, 100)
    x = {k: v.cuda() for k, v in m2rnn_inputs.make_inputs(B, steps, N, dtype=dtype, seed=args.seed).items()}
    dev = x["q"].device
    H = torch.zeros((B, N, K_DIM, V_DIM), device=dev)
    y = torch.empty((B, N, V_DIM), device=dev)
    toks = [{n: x[n][:, t].contiguous() for n in ("q", "k", "v", "f")} for t in range(steps)]
    stream = torch.cuda.current_stream(dev)
    for t in range(min(args.warmup + 1, steps)):
        m2.decode(toks[t]["q"], toks[t]["k"], toks[t]["v"], toks[t]["f"], x["W"], x["wr"], H, y=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # through the Python binding (argument checks on every call)
    e0.record(stream)
    for t in range(steps):
        m2.decode(toks[t]["q"], toks[t]["k"], toks[t]["v"], toks[t]["f"], x["W"], x["wr"], H, y=y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_python = e0.elapsed_time(e1) / steps
    # back to back through the C ABI with the arguments prepared beforehand, as
    # a native or captured caller would issue them: the launches queue up and
    # the events time the kernels
    import ctypes
    vp = ctypes.c_void_p
    common = (vp(x["W"].data_ptr()), vp(x["wr"].data_ptr()), vp(H.data_ptr()), vp(y.data_ptr()),
              vp(stream.cuda_stream))
    calls = [(B, N, K_DIM, V_DIM, m2.M2RNN_BF16, vp(tk["q"].data_ptr()), vp(tk["k"].data_ptr()),
              vp(tk["v"].data_ptr()), vp(tk["f"].data_ptr())) + common for tk in toks]
    fn = m2.lib.m2rnn_decode
    for c in calls[:min(args.warmup + 1, steps)]:
        assert fn(*c) == m2.M2RNN_OK, m2.m2rnn_last_error()
    torch.cuda.synchronize()
    e0.record(stream)
    status = [fn(*c) for c in calls]
    e1.record(stream)
    torch.cuda.synchronize()
    assert all(st == m2.M2RNN_OK for st in status), m2.m2rnn_last_error()
    ms = e0.elapsed_time(e1) / steps
    es = 2
    nbytes = B * N * K_DIM * V_DIM * 4 * 2 + B * (2 * K_DIM * es + N * (V_DIM + 1) * es + N * V_DIM * 4) \
        + N * (V_DIM * V_DIM + V_DIM) * es
    achieved = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "M2RNN decode head-tokens/s (K=64,V=16), one token per call for every (b, n); % of HBM roofline",
        "value": B * N / (ms * 1e-3), "unit": "head-tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, fp32 state; fp16-pair MFMA, fp32 VALU and accumulation",
        "data": "synthetic (seeded; as the scan workloads)",
        "config": {"workload": f"decode_{dtype}_B{B}_N{N}", "pass": "decode", "B": B, "N": N, "K": K_DIM, "V": V_DIM,
                   "input_dtype": dtype},
        "us_per_token": ms * 1e3,
        "us_per_call_python": ms_python * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "m2rnn_decode (one launch)",
                     "kernel_ms": ms, "algorithmic": f"{nbytes} B per call (state read and written, token inputs, y)"},
    }
    print(json.dumps(res), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the scan shards over batch rows/heads with no communication, "
                                   "but no multi-GPU path is built)"}))
        return 2
    if args.which == "epilogue":
        return bench_epilogue(args)
    if args.which == "prologue":
        return bench_prologue(args)
    if args.which == "decode":
        return bench_decode(args)

    import torch
    import m2rnn_inputs
    import non_linear_matrix_amd as m2

    if args.workload:
        name = args.workload
        w = m2rnn_inputs.WORKLOADS[name]
        which = "fwdbwd" if w.backward else "fwd"
    else:
        which = args.which
        name = "fwdbwd_bf16_B32_T4096_N64" if which == "fwdbwd" else "fwd_bf16_B32_T4096_N64"
        w = m2rnn_inputs.WORKLOADS[name]
    ck = 64
    x_cpu = m2rnn_inputs.make_workload(w, seed=args.seed, with_dy=(which == "fwdbwd"))
    x = {k: v.cuda() for k, v in x_cpu.items()}
    dev = x["q"].device
    B, T, N = w.B, w.T, w.N
    y = torch.empty((B, T, N, V_DIM), device=dev)
    HT = torch.empty((B, N, K_DIM, V_DIM), device=dev)
    Hck = torch.empty((B, N, (T + ck - 1) // ck, K_DIM, V_DIM), device=dev)
    fwd_out = (y, HT, Hck) if which == "fwdbwd" else (y, HT)
    fwd_ws_bytes = m2.m2rnn_forward_workspace_bytes(B, T, N)
    fwd_ws = torch.empty((fwd_ws_bytes,), device=dev, dtype=torch.uint8) if fwd_ws_bytes else None
    grads = ws = None
    if which == "fwdbwd":
        grads = dict(dq=torch.empty((B, T, K_DIM), device=dev), dk=torch.empty((B, T, K_DIM), device=dev),
                     dv=torch.empty((B, T, N, V_DIM), device=dev), df=torch.empty((B, T, N), device=dev),
                     dW=torch.empty((N, V_DIM, V_DIM), device=dev), dw_r=torch.empty((N, V_DIM), device=dev))
        nbytes = m2.m2rnn_backward_workspace_bytes(B, T, N, K_DIM, V_DIM, ck)
        ws = torch.empty((max(nbytes, 1),), device=dev, dtype=torch.uint8)

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        m2.forward(x["q"], x["k"], x["v"], x["f"], x["W"], x["wr"],
                   ckpt_every=ck if which == "fwdbwd" else 0, out=fwd_out, workspace=fwd_ws)
        if ev is not None:
            ev[1].record(stream)
        if which == "fwdbwd":
            m2.backward(x["q"], x["k"], x["v"], x["f"], x["W"], x["wr"], Hck, ck, x["dy"],
                        out=grads, workspace=ws)
            if ev is not None:
                ev[2].record(stream)

    if args.copy_calibration_bytes > 0:
        # a plain copy of known size: its profiler byte counters give the scale
        # factor for the kernels' FETCH_SIZE / WRITE_SIZE readings
        src = torch.empty(args.copy_calibration_bytes // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(events[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps if which == "fwdbwd" else 0.0

    htok = w.head_tokens
    value = htok * args.steps / (total_ms * 1e-3)

    def frac(flop_per_htok, ms):
        return flop_per_htok * htok / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS

    # dominant kernel and its algorithmic MFMA work per launch
    if which == "fwdbwd" and bwd_ms > fwd_ms:
        # the backward call: replay, reverse-sweep and reduction launches on one stream
        dom = ("m2rnn_backward (m2rnn_fwd_kernel<...,true> replay + m2rnn_bwd_kernel + "
               "m2rnn_bwd_reduce_qk_kernel + m2rnn_bwd_reduce_head_kernel)")
        dom_ms, flops = bwd_ms, 3 * FLOP_PER_CONTRACTION * htok
        traffic = profiled_traffic(name, "bwd")
    else:
        dom = ("m2rnn_forward (m2rnn_fwd_rows_kernel + m2rnn_fwd_rows_reduce_kernel)" if fwd_ws_bytes
               else "m2rnn_fwd_kernel")
        dom_ms, flops = fwd_ms, FLOP_PER_CONTRACTION * htok
        traffic = profiled_traffic(name, "fwd")
    achieved = flops / (dom_ms * 1e-3) / 1e12
    passes = {"forward": {"ms": fwd_ms, "flop_per_head_token": FLOP_PER_CONTRACTION,
                          "frac": frac(FLOP_PER_CONTRACTION, fwd_ms),
                          "clocks_per_time_step": fwd_ms * 1e-3 * CLOCK_GHZ * 1e9 / T}}
    if which == "fwdbwd":
        passes["backward"] = {"ms": bwd_ms, "flop_per_head_token": 3 * FLOP_PER_CONTRACTION,
                              "frac": frac(3 * FLOP_PER_CONTRACTION, bwd_ms),
                              "clocks_per_time_step": bwd_ms * 1e-3 * CLOCK_GHZ * 1e9 / T}
        passes["step"] = {"ms": ms_step, "flop_per_head_token": 4 * FLOP_PER_CONTRACTION,
                          "frac": frac(4 * FLOP_PER_CONTRACTION, ms_step)}
    res = {
        "metric": "M2RNN scan head-tokens/s (K=64,V=16) fwd & bwd; % of HBM/MFMA roofline",
        "value": value,
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{w.dtype} in, fp32 state; " + ("exact fp32 MFMA" if w.dtype == "f32" else
                  "fp16-pair MFMA (forward, replay), fp16 MFMA (sweep)") + ", fp32 VALU and accumulation"),
        "data": "synthetic (seeded; SiLU(N(0,1)) q,k,v; sigmoid(N(%g,1)) f; N(0,1/16) W; N(0,1) w_r, dy)" % w.f_mu,
        "config": {"workload": name, "pass": "forward+backward" if which == "fwdbwd" else "forward",
                   "B": B, "T": T, "N": N, "K": K_DIM, "V": V_DIM, "input_dtype": w.dtype,
                   "ckpt_every": ck if which == "fwdbwd" else 0},
        "copy_calibration_bytes": args.copy_calibration_bytes,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "fwd_head_tokens_per_s": htok / (fwd_ms * 1e-3),
        "bwd_head_tokens_per_s": htok / (bwd_ms * 1e-3) if bwd_ms else None,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_MFMA_PEAK_TFLOPS, "traffic": traffic, "kernel": dom,
                     "kernel_ms": dom_ms,
                     "algorithmic": f"{flops / htok:.0f} flop/head-token x {htok} head-tokens per launch",
                     "pricing": "fp32-equivalent: the algorithmic 2KV^2 flop of each state contraction at the fp32 "
                                "matrix peak (the state is fp32 to the pages); the kernels issue fp16 MFMA and fp32 "
                                "VALU instructions, and the VALU work (tanh as exp2 + rcp, the gate, the rank-1 term) "
                                "occupies most of each SIMD's cycles (counters below)"},
        "passes": passes,
        "counters": sq_counters(name),
        "hbm": {"fwd_algorithmic_bytes": algorithmic_bytes_fwd(w),
                "fwd_achieved_GBs": algorithmic_bytes_fwd(w) / (fwd_ms * 1e-3) / 1e9, "peak_GBs": HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x_cpu, which, args.cpu_threads, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
