"""Benchmark of the KDA hot path on one MI355X (gfx950).

    python bench.py [--steps K] [--warmup W] [--workload N] [--side 1,2] [--gpus 1]

One step = one kda_chunk_fwd over the headline prefill workload with the
library's default plan: gate prep, WY/UT transform, intra-chunk outputs and
the inter-chunk state pass, plus the segment passes and prefix scan when the
plan splits the sequence.  The headline workload is the largest one that fits
one GPU, the single 1,048,576-token sequence: B=1, T=1,048,576, H=32,
dk=dv=128, chunk 64, bf16 q/k/v/o with float32 gates and state (default plan:
the lead form of 9 segments: segment 0 beside segment pass 1 over segments 1-7
in one launch, the prefix scan from segment 1, and pass 2 over segments 1-8).  Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

The same JSON line carries side figures, each timed the same way:
  * the other prefill workloads (B=1 T=4096 H=16 with 16 segments; the B=8
    T=8192 H=32 floor-stress batch in one pass), with their per-launch times
    and whole-step rooflines;
  * the headline step with state checkpoints every 512 tokens, with raw gate
    logits (KDA_GATE_LOGITS) and with q / k normalised in the kernels;
  * decode: 256 sequences x 32 heads, 128x128 float32 state, 64 consecutive
    in-place steps, plus the speculative verify of 4 drafts and their commit,
    and the 64 steps of its first 1, 8 and 64 sequences as eager calls and as one
    replay of a HIP graph that captured them (small batches are launch-bound).
Rooflines: `roofline` is the dominant launch of the headline step (its
algorithmic bytes over its mean duration, from HIP events the library records
around each launch on the stream the kernels run on) with the whole step's
beside it; executed MFMA figures come from the committed rocprofv3 counter
table of the workload while the library sources match the ones it was taken
on.  `cpu_baseline` is the float64 oracle timed on the host cores on a
bounded sample of the headline workload.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kda_synth as ks  # noqa: E402

METRIC = "KDA prefill tokens/s (+% bf16 MFMA peak); decode steps/s (+% HBM GB/s)"
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
PEAK_BF16_TFLOPS = 2516.6        # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 MFMA
DECODE_WORKLOAD = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic work

def prefill_flops_per_token_head(dk, dv, C):
    """K~S, Q~S, K^T U (3 x 2 dk dv); causal A and M (~2 C dk); T V' and M U (2 (C+1) dv);
    the triangular inverse (C^2 / 3).  Elementwise exps are not counted."""
    return 6 * dk * dv + 2 * C * dk + 2 * (C + 1) * dv + C * C / 3.0


def prefill_bytes_per_token_head(dk, dv, es):
    """q, k, v, o in the storage dtype; log_alpha per channel and beta in float32."""
    return 2 * dk * es + dv * es + 4 * dk + 4 + dv * es


def launch_bytes(r, plan, es):
    """Algorithmic HBM bytes of each kernel launch of one kda_chunk_fwd call, in launch order."""
    B, T, H, dk, dv = r.B, r.T, r.H, r.dk, r.dv
    st = B * H * dk * dv * 4
    s0 = st if r.s0_std > 0 else 0
    if plan.n_segments <= 1:
        return [("chunk_kernel (one pass)", B * T * H * prefill_bytes_per_token_head(dk, dv, es) + s0 + st)]
    P = plan.n_segments
    pair = B * H * (dk * dv + dk * dk) * 4
    summ = dk * es + dv * es + 4 * dk + 4                               # k, v, log_alpha, beta
    full = prefill_bytes_per_token_head(dk, dv, es)
    if plan.seg0_len > 0:
        # lead form: segment 0 in pass-2 form (its end state to the start states) beside pass 1
        # over segments 1 .. P-2; the scan from segment 1; pass 2 over segments 1 .. P-1
        seg0 = plan.seg0_len
        lc = -(-(-(-T // r.chunk) - seg0 // r.chunk) // (P - 1))
        t1 = min(T - seg0, (P - 2) * lc * r.chunk)
        out = [("chunk_lead_kernel (segment 0 beside segment pass 1)",
                B * seg0 * H * full + s0 + st + B * t1 * H * summ + (P - 2) * pair)]
        if P > 2:
            out.append(("scan_kernel", (P - 2) * pair + st + (P - 2) * st))
        out.append(("chunk_kernel (pass 2)", B * (T - seg0) * H * full + (P - 1) * st + st))
        return out
    seg_len = -(-(-(-T // r.chunk)) // P) * r.chunk
    t1 = min(T, (P - 1) * seg_len)                                       # tokens pass 1 summarises
    pass1 = B * t1 * H * summ + (P - 1) * pair
    scan = (P - 1) * pair + s0 + P * st
    pass2 = B * T * H * prefill_bytes_per_token_head(dk, dv, es) + P * st + st
    return [("chunk_kernel (segment pass 1)", pass1), ("scan_kernel", scan), ("chunk_kernel (pass 2)", pass2)]


def decode_bytes_per_step(N, H, dk, dv, es):
    """State read + write (float32), q, k, v, o in the storage dtype, log_alpha and beta float32."""
    return N * H * (2 * dk * dv * 4 + 2 * dk * es + dv * es + 4 * dk + 4 + dv * es)


def verify_bytes(N, n, H, dk, dv, es):
    """Speculative verify of n drafts: state read once (float32), per draft q, k, v, o in the
    storage dtype and log_alpha, beta float32."""
    return N * H * (dk * dv * 4 + n * (2 * dk * es + dv * es + 4 * dk + 4 + dv * es))


def commit_bytes(N, n, H, dk, dv, es):
    """Commit of all n drafts: state read + write, per draft k, v (storage dtype), log_alpha,
    beta; n_accept."""
    return N * H * (2 * dk * dv * 4 + n * (dk * es + dv * es + 4 * dk + 4)) + 4 * N


# ----------------------------------------------------------------------------- CPU baseline (oracle)

_CPU = {}


def _oracle_prefill_head(h):
    import oracle
    x = _CPU["x"]
    sl = lambda a: a[:, :, h:h + 1]  # noqa: E731
    oracle.kda_chunked(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["log_alpha"]), x["beta"][:, :, h:h + 1],
                       None if x["S0"] is None else x["S0"][:, h:h + 1], chunk=_CPU["chunk"])
    return h


def _oracle_decode_slice(i):
    import oracle
    d, sel = _CPU["d"], _CPU["slices"][i]
    S = d["state"][sel].astype(np.float64)
    for s in range(d["q"].shape[0]):
        _, S = oracle.kda_decode_step(S, d["q"][s][sel], d["k"][s][sel], d["v"][s][sel],
                                      d["log_alpha"][s][sel], d["beta"][s][sel])
    return i


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _run_pool(fn, items, workers):
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        t = time.perf_counter()
        list(pool.imap_unordered(fn, items))
        return time.perf_counter() - t


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


CPU_SHARE = 16                        # host cores one GPU's share of the box provides


def cpu_workers():
    """Worker processes for the oracle: every core this process may run on, up to the
    16-core share of the host that goes with one GPU."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(CPU_SHARE, avail))


def host_cores():
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"host_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "cpu_share_per_gpu": CPU_SHARE,
            "cpu_model": cpu_model()}


HOST_GEN_LIMIT = 1 << 23              # token-heads above which inputs are drawn on the device
CKPT_STRIDE = 512                     # state checkpoint stride of the side figure (the hash block)
SPEC_DRAFTS = 4                       # draft tokens per sequence of the speculative-decoding side figure


def cpu_baseline_prefill(r, x):
    """The oracle's chunked form over every head of the workload, repeated until about
    10 s of CPU work; one process per core, BLAS single-threaded.  Workloads drawn on the
    device (x is None) are sampled: the first 4096 tokens of every head."""
    sampled = x is None
    if sampled:
        r = r.with_shape(T=min(r.T, 4096))
        x = ks.make_prefill(r)
    _CPU.update(x=x, chunk=r.chunk)
    workers = cpu_workers()
    reps = 1
    while True:
        wall = _run_pool(_oracle_prefill_head, list(range(r.H)) * reps, workers)
        if wall * workers >= 10.0 or reps >= 512:
            break
        reps = int(min(512, max(2 * reps, np.ceil(reps * 12.0 / max(wall * workers, 1e-3)))))
    tok = r.B * r.T * reps
    out = {"value": tok / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
           "sample": (f"first {r.T} tokens of every head" if sampled else "whole workload")
                     + f" (B={r.B} T={r.T} H={r.H}) x{reps}, float64 chunked form "
                     f"(chunk {r.chunk}), one (b, h) per task; tokens/s of the sample",
           "seconds": wall}
    out.update(host_cores())
    return out


def cpu_baseline_decode(rd, d, n_seq):
    """The oracle's recurrent step over n_seq of the 256 sequences (all heads, all steps)."""
    workers = cpu_workers()
    seqs = np.arange(n_seq)
    slices = [s for s in np.array_split(seqs, min(workers, n_seq)) if len(s)]
    _CPU.update(d=d, slices=slices)
    wall = _run_pool(_oracle_decode_slice, list(range(len(slices))), workers)
    steps = d["q"].shape[0]
    return {"value": steps * (n_seq / rd.B) / wall, "unit": "steps/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_seq} of {rd.B} sequences x {rd.H} heads x {steps} steps, scaled to the full batch",
            "seconds": wall}


# ----------------------------------------------------------------------------- GPU

def make_events(torch, n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()          # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    return evs


def prefill_inputs(torch, r, x, dev):
    """Device tensors of a prefill workload: uploaded from host arrays ``x``, or drawn on the
    device when the workload is too large for host copies (x is None)."""
    dt = torch.bfloat16 if r.dtype == "bf16" else torch.float32
    if x is None:
        t = time.perf_counter()
        xd = ks.make_prefill_device(r, dev)
        torch.cuda.synchronize()
        log(f"generated {r.name} inputs on the device in {time.perf_counter() - t:.1f}s")
        return xd
    T_ = lambda a, t: torch.from_numpy(np.ascontiguousarray(a)).to(dev, t)  # noqa: E731
    return {"q": T_(x["q"], dt), "k": T_(x["k"], dt), "v": T_(x["v"], dt),
            "log_alpha": T_(x["log_alpha"], torch.float32), "beta": T_(x["beta"], torch.float32),
            "S0": None if x["S0"] is None else T_(x["S0"], torch.float32)}


def time_prefill(g, torch, r, xd, steps, warmup, options=False):
    """Times `steps` default-plan kda_chunk_fwd calls (after `warmup`), then the same number with
    the library recording HIP events around every launch; returns the figures as a dict.  With
    ``options`` also the step with state checkpoints, gate logits and q / k normalisation."""
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if r.dtype == "bf16" else torch.float32
    es = 2 if r.dtype == "bf16" else 4
    q, k, v, la, beta, S0 = xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], xd["S0"]
    plan = g.default_plan(r.B, r.T, r.H, r.dk, r.dv, r.chunk, dt)
    nws = g.workspace_bytes(r.B, r.T, r.H, r.dk, r.dv, r.chunk, dt, plan)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    o = torch.empty((r.B, r.T, r.H, r.dv), dtype=dt, device=dev)
    S_T = torch.empty((r.B, r.H, r.dk, r.dv), dtype=torch.float32, device=dev)
    log(f"prefill {r.name}: plan {plan}, workspace {nws} B")

    def run(n, p=None, **kw):
        for _ in range(n):
            g.chunk_fwd(q, k, v, la, beta, S0, chunk=r.chunk, plan=plan if p is None else p, o=o, S_T=S_T,
                        workspace=ws, **kw)

    def timed(**kw):
        run(warmup, **kw)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        run(steps, **kw)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms = timed()

    # per-launch durations from events the library records around each launch
    lb = launch_bytes(r, plan, es)
    nl = len(lb)
    evs = make_events(torch, 2 * nl * steps)
    arrs = [(ctypes.c_void_p * (2 * nl))(*[evs[2 * nl * i + j].cuda_event for j in range(2 * nl)])
            for i in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        p = g.Plan(plan.n_segments, plan.dv_block, ctypes.cast(arrs[i], ctypes.POINTER(ctypes.c_void_p)), 2 * nl)
        p.seg0_len = plan.seg0_len
        run(1, p=p)
    torch.cuda.synchronize()
    per_launch = []
    for j, (name, nbytes) in enumerate(lb):
        d = [evs[2 * nl * i + 2 * j].elapsed_time(evs[2 * nl * i + 2 * j + 1]) for i in range(steps)]
        per_launch.append({"kernel": name, "ms": float(np.mean(d)), "bytes": int(nbytes),
                           "GBps": nbytes / (np.mean(d) * 1e-3) / 1e9})
    log(f"prefill {r.name} per launch:", json.dumps(per_launch))

    token_heads = r.B * r.T * r.H
    flops = token_heads * prefill_flops_per_token_head(r.dk, r.dv, r.chunk)
    nbytes = token_heads * prefill_bytes_per_token_head(r.dk, r.dv, es)
    sec = ms * 1e-3
    peak_mf = PEAK_BF16_TFLOPS if r.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    step_bytes = sum(b for _, b in lb)
    dom = max(per_launch, key=lambda e: e["ms"])
    res = {
        "workload": r.name, "B": r.B, "T": r.T, "H": r.H, "dk": r.dk, "dv": r.dv, "chunk": r.chunk,
        "plan": {"n_segments": plan.n_segments, "dv_block": plan.dv_block, "seg0_len": plan.seg0_len},
        "ms_per_step": round(ms, 5), "tokens_per_s": round(r.B * r.T / sec, 1),
        "roofline": {"bound": "hbm", "kernel": dom["kernel"], "achieved": round(dom["GBps"], 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(dom["GBps"] / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(r.name, dom["kernel"]), "launch_ms": round(dom["ms"], 5),
                     "launch_bytes": dom["bytes"]},
        "whole_step": {"bound": "hbm", "alg_bytes": int(step_bytes),
                       "achieved": round(step_bytes / sec / 1e9, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                       "frac": round(step_bytes / sec / 1e9 / PEAK_HBM_GBPS, 4),
                       "single_pass_bytes": int(nbytes),
                       "single_pass_frac": round(nbytes / sec / (PEAK_HBM_GBPS * 1e9), 4)},
        "mfma_frac_alg": round(flops / sec / (peak_mf * 1e12), 4),
        "hbm_frac_alg": round(nbytes / sec / (PEAK_HBM_GBPS * 1e9), 4),
        "roofline_frac": round(max(flops / (peak_mf * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9)) / sec, 4),
        "alg_gflop": round(flops / 1e9, 3), "alg_mb": round(nbytes / 1e6, 2),
        "launches": per_launch,
    }
    ex = executed_mfma(r.name, per_launch, sec, peak_mf)
    if ex is not None:
        res["mfma_executed"] = ex
    if not options:
        return res

    # the same step with state checkpoints every CKPT_STRIDE tokens (prefix reuse)
    if r.T >= CKPT_STRIDE and CKPT_STRIDE % r.chunk == 0:
        nck = r.T // CKPT_STRIDE
        sck = torch.empty((r.B, nck, r.H, r.dk, r.dv), dtype=torch.float32, device=dev)
        ms_ck = timed(ckpt_stride=CKPT_STRIDE, state_ckpt=sck)
        res["with_state_checkpoints"] = {"stride": CKPT_STRIDE, "checkpoints": nck, "ms_per_step": round(ms_ck, 5),
                                         "overhead": round(ms_ck / ms - 1.0, 4), "extra_bytes": int(sck.numel() * 4)}
        del sck
        log("prefill with state checkpoints:", json.dumps(res["with_state_checkpoints"]))
    # reading log_alpha as raw gate logits (-5 sigmoid formed in gate prep), then also
    # normalising q and k inside the kernels
    ms_gate = timed(gate=g.GATE_LOGITS)
    ms_norm = timed(qk_norm=True)
    res["from_gate_logits"] = {"ms_per_step": round(ms_gate, 5), "overhead": round(ms_gate / ms - 1.0, 4)}
    res["with_qk_norm"] = {"ms_per_step": round(ms_norm, 5), "overhead": round(ms_norm / ms - 1.0, 4)}
    log("prefill options:", json.dumps({k: res[k] for k in ("from_gate_logits", "with_qk_norm")}))
    return res


def bench_speculative(g, torch, rd, d, n, reps):
    """Verify of n drafts per sequence and commit of all of them, on the decode workload's
    state and its first n steps' inputs laid out [N, n, H, .]."""
    dev = torch.device("cuda:0")
    dt = torch.bfloat16
    T_ = lambda a, t: torch.from_numpy(np.ascontiguousarray(np.swapaxes(a[:n], 0, 1))).to(dev, t)  # noqa: E731
    q, k, v = T_(d["q"], dt), T_(d["k"], dt), T_(d["v"], dt)
    la, beta = T_(d["log_alpha"], torch.float32), T_(d["beta"], torch.float32)
    pristine = torch.from_numpy(d["state"]).to(dev)
    state = pristine.clone()
    o = torch.empty((rd.B, n, rd.H, rd.dv), dtype=dt, device=dev)
    acc = torch.full((rd.B,), n, dtype=torch.int32, device=dev)
    out = {}
    for name in ("verify", "commit"):
        times = []
        for i in range(reps + 1):
            state.copy_(pristine)           # restore (not timed)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            if name == "verify":
                g.decode_verify(state, q, k, v, la, beta, o=o)
            else:
                g.decode_commit(state, q, k, v, la, beta, acc)
            t1.record()
            torch.cuda.synchronize()
            if i:                           # the first call is a warm-up
                times.append(t0.elapsed_time(t1))
        ms = float(np.median(times))
        nb = (verify_bytes if name == "verify" else commit_bytes)(rd.B, n, rd.H, rd.dk, rd.dv, 2)
        gbps = nb / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "bytes": nb, "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    out["n_draft"] = n
    return out


def bench_decode(g, torch, rd, d, reps):
    dev = torch.device("cuda:0")
    dt = torch.bfloat16
    T_ = lambda a, t: torch.from_numpy(np.ascontiguousarray(a)).to(dev, t)  # noqa: E731
    pristine = T_(d["state"], torch.float32)
    state = pristine.clone()
    qs, ks_, vs = T_(d["q"], dt), T_(d["k"], dt), T_(d["v"], dt)
    las, bs = T_(d["log_alpha"], torch.float32), T_(d["beta"], torch.float32)
    o = torch.empty((rd.B, rd.H, rd.dv), dtype=dt, device=dev)
    nsteps = qs.shape[0]

    def run():
        for s in range(nsteps):
            g.decode_step(state, qs[s], ks_[s], vs[s], las[s], bs[s], o=o)

    run()                                   # warm-up
    times = []
    for _ in range(reps):
        state.copy_(pristine)               # restore (not timed)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        run()
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) / nsteps)
    ms = float(np.median(times))
    return ms, nsteps


def bench_decode_graph(g, torch, rd, d, sizes=(1, 8, 64), reps=10):
    """Small batches: the decode workload's 64 steps for its first N sequences (all heads),
    as eager binding calls and as one replay of the same steps captured in a HIP graph;
    median microseconds per step of each (the state restored, untimed, between repetitions)."""
    dev = torch.device("cuda:0")
    dt = torch.bfloat16
    out = []
    for N in sizes:
        T_ = lambda a, t: torch.from_numpy(np.ascontiguousarray(a[:, :N])).to(dev, t)  # noqa: E731
        pristine = torch.from_numpy(np.ascontiguousarray(d["state"][:N])).to(dev)
        state = pristine.clone()
        qs, ks_, vs = T_(d["q"], dt), T_(d["k"], dt), T_(d["v"], dt)
        las, bs = T_(d["log_alpha"], torch.float32), T_(d["beta"], torch.float32)
        nsteps = qs.shape[0]
        o = torch.empty((nsteps, N, rd.H, rd.dv), dtype=dt, device=dev)

        def run():
            for s in range(nsteps):
                g.decode_step(state, qs[s], ks_[s], vs[s], las[s], bs[s], o=o[s])

        def timed(fn):
            fn()                                            # warm-up
            times = []
            for _ in range(reps):
                state.copy_(pristine)                       # restore (not timed)
                torch.cuda.synchronize()
                t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t0.record()
                fn()
                t1.record()
                torch.cuda.synchronize()
                times.append(t0.elapsed_time(t1) * 1e3 / nsteps)
            return float(np.median(times))

        eager_us = timed(run)
        side = torch.cuda.Stream()                          # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        graph_us = timed(graph.replay)
        nb = decode_bytes_per_step(N, rd.H, rd.dk, rd.dv, 2)
        out.append({"sequences": N, "heads": rd.H, "eager_us_per_step": round(eager_us, 2),
                    "graph_us_per_step": round(graph_us, 2), "graph_GBps": round(nb / (graph_us * 1e-6) / 1e9, 1)})
        del graph
    return {"steps": int(d["q"].shape[0]), "by_batch": out}


# ----------------------------------------------------------------------------- measured HBM traffic

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_delta_rule_107_amd", "csrc")


def library_source_digest():
    """sha256 over the library's kernel and ABI sources: a counter table measured on other
    sources no longer describes the kernels that run."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))
    for f in files + ["../../include/kda.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter table of
    ``workload`` (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the same counter
    reads for a 1 GiB device copy), or None when there is no table for it or the library
    sources changed since it was taken."""
    path = os.path.join(PROFILES, f"hbm_traffic__{workload}.md")
    if not os.path.exists(path):
        return None
    digest, fetch_f, write_f, rows = None, None, None, {}
    for line in open(path):
        line = line.strip()
        if line.startswith("source digest:"):
            digest = line.split(":", 1)[1].strip().strip("`")
        elif line.startswith("| scale |"):
            cells = [c.strip() for c in line.strip("|").split("|")]
            fetch_f, write_f = float(cells[1]), float(cells[2])
        elif line.startswith("| ") and line.count("|") >= 6 and not line.startswith(("| kernel", "| scale")):
            cells = [c.strip() for c in line.strip("|").split("|")]
            try:
                rows[cells[0]] = (float(cells[2].replace(",", "")), float(cells[3].replace(",", "")))
            except ValueError:
                pass
    if digest != library_source_digest() or fetch_f is None or kernel not in rows:
        return None
    fk, wk = rows[kernel]
    return int(round((fk * fetch_f + wk * write_f) * 1024))


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy of 1 GiB: the box's achievable-bandwidth reference (read + write)."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def executed_mfma(workload, per_launch, step_sec, peak_tflops):
    """Executed MFMA work of one step from the committed rocprofv3 counter table of
    ``workload`` (SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F32 per dispatch, x 512 flops), over the
    live step time; None when there is no table or the library sources changed since."""
    path = os.path.join(PROFILES, f"mfma__{workload}.md")
    if not os.path.exists(path):
        return None
    digest, rows = None, {}
    for line in open(path):
        line = line.strip()
        if line.startswith("source digest:"):
            digest = line.split(":", 1)[1].strip().strip("`")
        elif line.startswith("| ") and not line.startswith(("| kernel", "|---")):
            cells = [c.strip() for c in line.strip("|").split("|")]
            try:
                col = 2 if peak_tflops == PEAK_BF16_TFLOPS else 3            # bf16 or f32 MFMA flops
                rows[cells[0]] = (float(cells[col].replace(",", "")), float(cells[4].rstrip(" %")))
            except (ValueError, IndexError):
                pass
    if digest != library_source_digest():
        return None
    flops, busy = 0.0, {}
    for e in per_launch:
        if e["kernel"] not in rows:
            return None
        flops += rows[e["kernel"]][0]
        busy[e["kernel"]] = rows[e["kernel"]][1]
    return {"label": "executed (rocprofv3 counters: MFMA ops incl. masked halves and recompute)",
            "tflop_per_step": round(flops / 1e12, 4),
            "frac": round(flops / step_sec / (peak_tflops * 1e12), 4),
            "mfma_busy_pct_per_kernel": busy, "table": os.path.relpath(path, ROOT)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[0, 1, 2, 3],
                    help="headline prefill workload (0 tiny fp32, 1 B1 T4096 H16, 2 B8 T8192 H32, 3 B1 T1M H32)")
    ap.add_argument("--side", default="1,2", help="other prefill workloads timed as side figures ('' for none)")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the checkpoint / gate-logit / q-k norm figures of the headline step")
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: every workload runs on a single MI355X and no "
              f"multi-GPU path is built (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    r = ks.WORKLOADS[args.workload]
    rd = ks.WORKLOADS[DECODE_WORKLOAD]
    side = [int(w) for w in args.side.split(",") if w.strip() and int(w) != args.workload]
    hosts = {}
    for w in [args.workload] + side:
        rw = ks.WORKLOADS[w]
        if rw.B * rw.T * rw.H <= HOST_GEN_LIMIT:
            t = time.perf_counter()
            hosts[w] = ks.make_prefill(rw)
            log(f"generated {rw.name} inputs in {time.perf_counter() - t:.1f}s")
        else:
            hosts[w] = None
    d = None
    if not args.no_decode:
        t = time.perf_counter()
        d = ks.make_decode(rd)
        log(f"generated decode inputs in {time.perf_counter() - t:.1f}s")

    # CPU baseline first: the worker processes fork before the GPU is touched
    cpu_pre = cpu_dec = None
    if not args.no_cpu_baseline:
        cpu_pre = cpu_baseline_prefill(r, hosts[args.workload])
        log("cpu baseline prefill:", json.dumps(cpu_pre))
        if d is not None:
            cpu_dec = cpu_baseline_decode(rd, d, 128)
            log("cpu baseline decode:", json.dumps(cpu_dec))

    import torch
    import gated_delta_rule_107_amd as g
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    xd = prefill_inputs(torch, r, hosts.pop(args.workload), dev)
    head = time_prefill(g, torch, r, xd, args.steps, args.warmup, options=not args.no_options)
    del xd
    torch.cuda.empty_cache()
    sides = {}
    for w in side:
        rw = ks.WORKLOADS[w]
        xw = prefill_inputs(torch, rw, hosts.pop(w), dev)
        sides[rw.name] = time_prefill(g, torch, rw, xw, max(args.steps, 10), args.warmup)
        del xw
        torch.cuda.empty_cache()

    dec = None
    if d is not None:
        dms, nsteps = bench_decode(g, torch, rd, d, args.decode_reps)
        dbytes = decode_bytes_per_step(rd.B, rd.H, rd.dk, rd.dv, 2)
        dgbps = dbytes / (dms * 1e-3) / 1e9
        dec = {"workload": rd.name, "value": round(1e3 / dms, 2), "unit": "steps/s", "ms_per_step": round(dms, 5),
               "steps_per_interval": nsteps,
               "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": round(dgbps, 1),
                            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(dgbps / PEAK_HBM_GBPS, 4),
                            "traffic": measured_traffic(rd.name, "decode_kernel"), "launch_bytes": dbytes},
               "cpu_baseline": cpu_dec,
               "speculative": bench_speculative(g, torch, rd, d, SPEC_DRAFTS, 2 * args.decode_reps),
               "small_batch_hip_graph": bench_decode_graph(g, torch, rd, d)}
        log("decode:", json.dumps(dec))
    copy_gbps = copy_bandwidth(torch)

    prefill = {k: head[k] for k in ("mfma_frac_alg", "hbm_frac_alg", "roofline_frac", "alg_gflop", "alg_mb",
                                     "whole_step", "launches")}
    for k in ("mfma_executed", "with_state_checkpoints", "from_gate_logits", "with_qk_norm"):
        if k in head:
            prefill[k] = head[k]
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r.dtype,
        "data": "synthetic",
        "config": {"workload": r.name, "B": r.B, "T": r.T, "H": r.H, "dk": r.dk, "dv": r.dv,
                   "chunk": r.chunk, "plan": head["plan"]},
        "roofline": head["roofline"],
        "cpu_baseline": cpu_pre,
        "prefill": prefill,
        "side_prefill": sides,
        "decode": dec,
        "hbm_copy_GBps": round(copy_gbps, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
