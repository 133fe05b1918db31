#!/usr/bin/env python3
"""Benchmark of the delta-rule / Kalman-Delta scan library on one MI355X.

Prints ONE JSON line. The headline value is the forward-scan throughput of the
gated delta workload (B=4, H=16, L=4096, d_k=d_v=128, chunk 64, bf16 q/k/v,
float32 alpha/beta, float32 output and state), in tokens/s (a token is one
position of one batch row, all H heads). One step = one kdn_scan_fwd call:
the parallel (I + A)^-1 kernel plus the sequential state kernel. Inputs are
resident in HBM before timing starts.

Extra fields: the roofline of the dominant (state) kernel, its time being the
step time less the prepare phase timed back to back (HIP events created without
the system-scope fence, on the stream the kernels run on), and both phases also
timed with events between them inside the step sequence; the same step with the
last-level cache flushed (cold);
the tiny float32 workload's latency; the fp64 oracle timed on a bounded sample
on the host cores, which also gives each workload's max|o - o_oracle| / RMS;
and (unless --quick) the decode + HOLA cache step, the HOLA prompt cache after
a scan with write scores, the backward pass, the diagonal and isotropic Kalman
scans and the long-context scan.
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

METRIC = "scan tokens/sec (fwd, H=16, d=128) + % MFMA peak; decode % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, published


def scan_flops_per_token_head(C, dk, dv):
    """Algorithmic flops of the chunk form per token and head (lower triangles
    counted once): Grams K B^T and Q B^T, T = (I + A)^-1, T X, P U and the three
    state products K S, Q S and the state update."""
    return C * (3 * dk + 2 * dv) + C * C / 3 + 6 * dk * dv


def scan_bytes(B, H, L, dk, dv, in_bytes=2, out_bytes=2, extra_per_token=0, state_out=True):
    """Algorithmic HBM bytes of one scan: q, k, v read once, alpha/beta (+extra)
    read once, o written once, the final state written once. The default is the
    roofline's unit: bf16 q, k, v and o, float32 alpha and beta,
    1032 B per token and head at d = 128; out_bytes=4 gives the float32 output
    the library writes by default (1288 B)."""
    per_tok = (2 * dk + dv) * in_bytes + 8 + extra_per_token + dv * out_bytes
    return B * H * L * per_tok + (B * H * dk * dv * 4 if state_out else 0)


DECODE_BYTES_PER_HEAD = (
    2 * 128 * 128 * 4      # state read + write
    + 2 * 64 * 128 * 4     # cache keys and values read
    + 64 * 8               # cache scores and positions read
    + 3 * 128 * 4 + 8      # q, k, v, alpha, beta
    + 2 * 128 * 4 + 4 + 4  # o, o_cache, m written; m read back
    + 2 * 128 * 4 + 8 + 8  # inserted key/value, score/position, count read + write
)


def code_digest(path):
    """sha256 of a C/HIP source with its // comments and all whitespace removed,
    so that edits to comments alone keep a counter record valid."""
    import hashlib
    import re
    code = "".join(re.sub(r"//.*", "", line) for line in open(path, encoding="utf-8"))
    return hashlib.sha256(re.sub(r"\s+", "", code).encode()).hexdigest()


def counter_record():
    """The state kernel's committed counter record (profiles/*_traffic.json:
    HBM bytes per launch, executed matrix-core flops, matrix-core busy
    fraction), or None when the kernel code changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "scan_gated_B4H16L4096_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if code_digest(os.path.join(ROOT, rec["source"])) != rec["code_sha256"]:
        return None
    return rec


def measured_traffic(kernel_ms):
    """HBM bytes per launch of the state kernel from the committed counter runs,
    or None when the kernel code changed since."""
    rec = counter_record()
    return None if rec is None else rec["hbm_read_bytes"] + rec["hbm_write_bytes"]


def copy_bandwidth(torch, mib=1024, reps=10):
    """On-box attainable HBM rate: a device-to-device copy of `mib` MiB, bytes
    read plus bytes written over the time."""
    x = torch.empty(mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * x.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return round(gbs, 1)


# The GPU runs at its idle clock until it has been busy for a few tens of
# milliseconds (measured: the gated step takes 0.176 ms after 3 warm-up steps
# and 0.154 ms from 300 on), so warm-up always lasts at least this long on top
# of the requested steps. It is untimed.
MIN_WARMUP_S = 0.25


def _warm(torch, step, warmup):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < MIN_WARMUP_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


class HipTimer:
    """HIP events created with hipEventDisableSystemFence, recorded on a given
    stream: timing-only events that skip the system-scope cache writeback and
    invalidate of a default event, which would otherwise land between the two
    kernels of a step and cool the caches the second one reads. Uses the HIP
    runtime already loaded in this process (torch's, which libkdn.so binds to)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        self.ct = ctypes
        torch.cuda.init()
        paths = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln]
        if not paths:
            raise RuntimeError("no HIP runtime loaded in this process")
        self.hip = ctypes.CDLL(paths[0])
        self.events = []

    def event(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.ct.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")
        self.events.append(e)
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: {rc}")

    def ms(self, a, b):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return out.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def bench_scan(kdn, torch, name, steps, warmup, mode="delta", per_phase=True, cold=False,
               keep=False, resid="gated"):
    import workloads
    cfg = workloads.WORKLOADS[name]
    B, H, L, dk, dv, C = cfg["B"], cfg["H"], cfg["L"], cfg["dk"], cfg["dv"], cfg["chunk"]
    inp = workloads.named_scan_inputs(name)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v")}
    for n in t:
        t[n] = t[n].to(torch.bfloat16)
    alpha = torch.from_numpy(inp["alpha"]).to(dev)
    beta = torch.from_numpy(inp["beta"]).to(dev)
    r = torch.from_numpy(inp["r"]).to(dev) if inp["r"] is not None else None
    del inp
    cov_in = cov_out = None
    if mode in ("diag", "iso"):
        cov_in = torch.full((B, H, dk) if mode == "diag" else (B, H), cfg["cov_init"], device=dev)
        cov_out = torch.empty_like(cov_in)
    o = torch.empty((B, H, L, dv), dtype=torch.float32, device=dev)
    s_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    need = kdn.kdn_scan_workspace_size(B, H, L, dk, dv, C, mode, kdn.BF16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    qvar = cfg.get("q_noise_var", 0.0)

    def step(phase="all"):
        kdn.kdn_scan_fwd(t["q"], t["k"], t["v"], alpha=alpha, beta=beta, r=r, cov_in=cov_in,
                         cov_out=cov_out, q_noise_var=qvar, state_out=s_out, o=o, chunk=C,
                         mode=mode, resid=resid, workspace=ws, phase=phase)

    _warm(torch, step, warmup)
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res = dict(ms_per_step=ms, tokens_per_s=B * L / (ms * 1e-3), B=B, H=H, L=L, dk=dk, dv=dv, C=C)
    if cold:
        # a 512 MiB write between steps evicts the 256 MB last-level cache, so
        # every step reads its inputs from HBM; only the scan is timed
        flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        ev = _events(torch, 2 * steps)
        for i in range(steps):
            flush.fill_(float(i))
            ev[2 * i].record()
            step()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        cms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
        res["cold_ms_per_step"] = cms
        del flush
    if per_phase:
        # the step as above, split into its two phases with a fence-less event
        # before, between and after them on the stream the kernels run on: the
        # state kernel is timed in its own context (right after the prepare
        # kernel that writes what it reads), and the events do not flush the
        # caches between the two
        tm = HipTimer(torch)
        stream = torch.cuda.current_stream()
        ev = [tm.event() for _ in range(3 * steps)]
        for i in range(steps):
            tm.record(ev[3 * i], stream)
            step("prepare")
            tm.record(ev[3 * i + 1], stream)
            step("state")
            tm.record(ev[3 * i + 2], stream)
        torch.cuda.synchronize()
        res["prepare_ms"] = sum(tm.ms(ev[3 * i], ev[3 * i + 1]) for i in range(steps)) / steps
        res["state_ms"] = sum(tm.ms(ev[3 * i + 1], ev[3 * i + 2]) for i in range(steps)) / steps
        # An event between the phases delays the dispatch of the kernel after
        # it by a few microseconds, which the phase times above include. The
        # state kernel's share of the step without that: the step time (no
        # event inside a step) minus the prepare phase launched back to back
        # with one event pair around all launches.
        b0, b1 = tm.event(), tm.event()
        tm.record(b0, stream)
        for _ in range(steps):
            step("prepare")
        tm.record(b1, stream)
        torch.cuda.synchronize()
        res["prepare_b2b_ms"] = tm.ms(b0, b1) / steps
        res["state_kernel_ms"] = ms - res["prepare_b2b_ms"]
        tm.close()
    if keep:
        step()
        torch.cuda.synchronize()
        res["o"] = o.cpu().numpy()
        res["S"] = s_out.cpu().numpy()
        if cov_out is not None:
            res["cov"] = cov_out.cpu().numpy()
    return res


def bench_prefill(kdn, torch, steps, warmup, block=256, w=64):
    """The gated workload as a prompt with the HOLA cache: the scan with write
    scores, then the block-by-block cache (blocks of 256, w = 64)."""
    import workloads
    cfg = workloads.WORKLOADS["gated"]
    B, H, L, dk, dv, C = cfg["B"], cfg["H"], cfg["L"], cfg["dk"], cfg["dv"], cfg["chunk"]
    inp = workloads.named_scan_inputs("gated")
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(inp[n]).to(dev).to(torch.bfloat16) for n in ("q", "k", "v")}
    alpha = torch.from_numpy(inp["alpha"]).to(dev)
    beta = torch.from_numpy(inp["beta"]).to(dev)
    del inp
    o = torch.empty((B, H, L, dv), dtype=torch.float32, device=dev)
    m = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    oc = torch.empty_like(o)
    ws = torch.empty(kdn.kdn_scan_workspace_size(B, H, L, dk, dv, C, "delta", kdn.BF16, True),
                     dtype=torch.uint8, device=dev)
    pws = torch.empty(kdn.hola_prefill_workspace_size(B, H, L, dk, dv, w, block), dtype=torch.uint8,
                      device=dev)
    cache = kdn.HolaCache(B, H, dk, dv, w)

    def scan():
        kdn.kdn_scan_fwd(t["q"], t["k"], t["v"], alpha=alpha, beta=beta, o=o, chunk=C,
                         workspace=ws, m=m)

    def prefill():
        cache.count.zero_()
        kdn.hola_prefill(t["q"], t["k"], t["v"], m, 0, cache, block=block, o_cache=oc,
                         workspace=pws)

    _warm(torch, lambda: (scan(), prefill()), warmup)
    ev = _events(torch, 3 * steps)
    for i in range(steps):
        ev[3 * i].record()
        scan()
        ev[3 * i + 1].record()
        prefill()
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    s_ms = sum(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps)) / steps
    p_ms = sum(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps)) / steps
    # the read's algorithmic work: each query against w cached keys plus the causal
    # part of its block, 2 (d_k + d_v) flops per key
    keys = L * w + sum(min(block, L - j) * (min(block, L - j) + 1) // 2 for j in range(0, L, block))
    flops = B * H * keys * 2 * (dk + dv)
    return dict(scan_with_scores_ms=round(s_ms, 5), prefill_ms=round(p_ms, 5),
                tokens_per_s=round(B * L / ((s_ms + p_ms) * 1e-3), 1), block=block, w=w,
                read_gflop=round(flops / 1e9, 2),
                read_tflops=round(flops / (p_ms * 1e-3) / 1e12, 2),
                config="gated delta scan with write scores, then the HOLA prompt cache "
                       f"(blocks of {block}, w = {w}), B=4 H=16 L=4096 d=128")


def bench_backward(kdn, torch, steps, warmup):
    """Gradients of the gated delta scan at the headline shape (float32 inputs)."""
    import workloads
    cfg = workloads.WORKLOADS["gated"]
    B, H, L, dk, dv = cfg["B"], cfg["H"], cfg["L"], cfg["dk"], cfg["dv"]
    inp = workloads.named_scan_inputs("gated")
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v", "alpha", "beta")}
    del inp
    d_o = torch.randn((B, H, L, dv), device=dev)
    ws = torch.empty(int(kdn.lib.kdn_scan_bwd_workspace_size(B, H, L, dk, dv)), dtype=torch.uint8,
                     device=dev)

    def step():
        kdn.kdn_scan_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], d_o, workspace=ws)

    _warm(torch, step, warmup)
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return dict(ms_per_step=round(ms, 5), tokens_per_s=round(B * L / (ms * 1e-3), 1),
                config="gradients of the gated delta scan, B=4 H=16 L=4096 d=128, float32, "
                       "chunked (64 tokens)")


# heads of the decode workload whose outputs the oracle leg re-derives
DECODE_PARITY_HEADS = [(b, h) for b in (0, 37, 128, 255) for h in (0, 9, 20, 31)]


def bench_decode(kdn, torch, steps, warmup, keep=None):
    """Decode + HOLA cache at B=256, H=32, d=128, w=64, timed after the cache is full."""
    import workloads
    cfg = workloads.WORKLOADS["decode"]
    B, H, d, w = cfg["B"], cfg["H"], cfg["dk"], cfg["w"]
    dev = torch.device("cuda:0")
    warmup = max(warmup, w)          # steady state: every step reads a full cache
    total = warmup + steps
    inputs = []
    for s in range(total):
        st = workloads.decode_step_inputs(s, B, H, d, d)
        inputs.append({n: torch.from_numpy(x).to(dev) for n, x in st.items()})
    state = torch.zeros((B, H, d, d), device=dev)
    cache = kdn.HolaCache(B, H, d, d, w, device=dev)
    o = torch.empty((B, H, d), device=dev)
    oc = torch.empty((B, H, d), device=dev)
    m = torch.empty((B, H), device=dev)

    def step(i):
        x = inputs[i]
        kdn.kdn_step_decode(x["q"], x["k"], x["v"], x["alpha"], x["beta"], state, o=o, m=m)
        kdn.hola_cache_update(x["q"], x["k"], x["v"], m, i, cache, o_cache=oc)

    def timed(fn):
        e0, e1 = _events(torch, 2)
        e0.record()
        for i in range(warmup, total):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms = timed(step)
    gbs = B * H * DECODE_BYTES_PER_HEAD / (ms * 1e-3) / 1e9
    if keep is not None:
        # after all `total` steps once: the state, and the last step's outputs, of a few heads
        bs = [b for b, _ in DECODE_PARITY_HEADS]
        hs = [h for _, h in DECODE_PARITY_HEADS]
        keep["decode"] = dict(steps=total, S=state[bs, hs].cpu().numpy(), o=o[bs, hs].cpu().numpy(),
                              o_cache=oc[bs, hs].cpu().numpy(), m=m[bs, hs].cpu().numpy())
    # the same steps captured once into a HIP graph and replayed (the state and
    # the cache keep evolving, so every replay does a full step's work)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(warmup, total):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / (reps * steps)
    frac = lambda t: round(B * H * DECODE_BYTES_PER_HEAD / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)  # noqa: E731
    return dict(ms_per_step=round(ms, 5), tokens_per_s=round(B / (ms * 1e-3), 1),
                bytes_per_step=B * H * DECODE_BYTES_PER_HEAD, achieved_gbs=round(gbs, 1),
                hbm_frac=frac(ms), steps=steps, warmup=warmup,
                graph_ms_per_step=round(gms, 5), graph_hbm_frac=frac(gms),
                config="decode + HOLA cache, B=256 H=32 d=128 fp32, w=64, cache full; "
                       "kdn_step_decode + hola_cache_update per step")


def bench_tiny(kdn, torch, reps=200, keep=None):
    """The tiny float32 workload (1 head, d = 16, L = 64, alpha = 1): the delta
    write (chunk 16) and recursive least squares (full covariance, eps = 1e-2).
    Latency per call: GPU time from events around `reps` back-to-back calls,
    and host wall time of one call followed by a synchronisation."""
    import numpy as np
    import workloads
    inp = workloads.named_scan_inputs("tiny")
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v", "alpha", "beta")}
    d, eps = 16, 1e-2
    P0 = torch.from_numpy((np.eye(d) / eps).astype(np.float32))[None, None].to(dev)
    S = torch.empty((1, 1, d, d), device=dev)
    P = torch.empty_like(P0)
    o = torch.empty((1, 1, 64, d), device=dev)
    calls = {
        "delta": lambda: kdn.kdn_scan_fwd(t["q"], t["k"], t["v"], alpha=t["alpha"],
                                          beta=t["beta"], state_out=S, o=o, chunk=16),
        "rls": lambda: kdn.kdn_scan_fwd(t["q"], t["k"], t["v"], cov_in=P0, cov_out=P,
                                        state_out=S, o=o, chunk=16, mode="full"),
    }
    out = {}
    for name, fn in calls.items():
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(torch, 2)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        gpu_us = e0.elapsed_time(e1) * 1e3 / reps
        walls = []
        for _ in range(50):
            w0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - w0)
        walls.sort()
        # the call captured 20 times into one HIP graph and replayed: GPU time
        # per call without the host's per-call cost (Python, argument checks,
        # launch), which back-to-back eager calls of this size are bound by
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(20):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = _events(torch, 2)
        g0.record()
        for _ in range(10):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        out[name] = dict(gpu_us_per_call=round(gpu_us, 2),
                         graph_gpu_us_per_call=round(g0.elapsed_time(g1) * 1e3 / 200, 2),
                         host_us_per_synchronous_call=round(walls[len(walls) // 2] * 1e6, 1))
        if keep is not None:
            fn()
            torch.cuda.synchronize()
            keep[f"tiny/{name}"] = dict(o=o.cpu().numpy(), S=S.cpu().numpy(),
                                        cov=P.cpu().numpy() if name == "rls" else None)
    out["config"] = "1 head, d_k = d_v = 16, L = 64, float32, alpha = 1; delta write (chunk 16), " \
                    "RLS (full covariance, eps = 1e-2)"
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _rel(got, ref):
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))


def oracle_leg(kept, name="gated", seconds_target=15.0):
    """The CPU baseline and the parity of the benchmark's own outputs, both from
    the fp64 oracle as it stands. Baseline: the whole gated workload (every
    (batch, head) sequence at full length), repeated until about
    `seconds_target` seconds of host time, on all host threads. Parity: each
    workload the benchmark ran is recomputed by the oracle from the same seeded
    inputs and compared with the output the GPU produced in this run:
    max|x - x_oracle| / RMS(x_oracle) for o, the final state and the final
    covariance (decode: a sample of heads after all its steps)."""
    import numpy as np
    import oracle
    import workloads
    cfg = workloads.WORKLOADS[name]
    B, H, L = cfg["B"], cfg["H"], cfg["L"]
    inp = workloads.named_scan_inputs(name)
    q, k, v = (inp[n].reshape(1, B * H, L, -1) for n in ("q", "k", "v"))
    a, b = inp["alpha"].reshape(1, B * H, L), inp["beta"].reshape(1, B * H, L)
    threads = oracle.num_threads()

    def run():
        return oracle.scan(q, k, v, alpha=a, beta=b, want_m=False)

    t0 = time.perf_counter()
    first = run()
    t1 = time.perf_counter() - t0
    reps = max(1, int(round(seconds_target / max(t1, 1e-3))) - 1)
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    dt = time.perf_counter() - t0 + t1
    token_heads_per_s = (reps + 1) * B * H * L / dt
    baseline = dict(value=round(token_heads_per_s / H, 1), unit="tokens/s", cores=threads,
                    cpu_model=_cpu_model(), kind="oracle",
                    sample=f"the whole gated workload ({B * H} (batch, head) sequences of length "
                           f"{L}) {reps + 1} times, fp64 sequential recurrence, {dt:.1f} s; "
                           f"tokens/s = token-heads/s / H")
    parity = {}
    g = kept.get("gated/delta")
    if g is not None:
        parity["gated"] = dict(o=_rel(g["o"].reshape(first["o"].shape), first["o"]),
                               S=_rel(g["S"].reshape(first["S"].shape), first["S"]), tol=2e-2)
    del first
    for key, (wl, mode, resid) in {"kdn_diag/diag": ("kdn_diag", "diag", "gated"),
                                   "kdn_diag/iso": ("kdn_diag", "iso", "gated"),
                                   "long/delta": ("long", "delta", "gated"),
                                   "gated/noerase": ("gated", "delta", "noerase")}.items():
        got = kept.get(key)
        if got is None:
            continue
        c = workloads.WORKLOADS[wl]
        x = workloads.named_scan_inputs(wl)
        cshape = {"diag": (c["B"], c["H"], c["dk"]), "iso": (c["B"], c["H"])}.get(mode)
        cov0 = np.full(cshape, c.get("cov_init", 1.0), np.float32) if cshape else None
        ref = oracle.scan(x["q"], x["k"], x["v"], alpha=x["alpha"], beta=x["beta"], r=x["r"],
                          cov0=cov0, q_noise_var=c.get("q_noise_var", 0.0), mode=mode,
                          resid=resid, want_m=False)
        del x
        e = dict(o=_rel(got["o"], ref["o"]), S=_rel(got["S"], ref["S"]), tol=2e-2)
        if cov0 is not None:
            e["cov"] = _rel(got["cov"], ref["cov"])
            e["cov_tol"] = 1e-4
        parity[key.replace("kdn_diag/", "kdn_")] = e
        del ref
    tiny = workloads.named_scan_inputs("tiny")
    for nm in ("delta", "rls"):
        got = kept.get(f"tiny/{nm}")
        if got is None:
            continue
        if nm == "delta":
            ref = oracle.scan(tiny["q"], tiny["k"], tiny["v"], alpha=tiny["alpha"], beta=tiny["beta"])
        else:
            P0 = (np.eye(16) / 1e-2)[None, None]
            ref = oracle.scan(tiny["q"], tiny["k"], tiny["v"], cov0=P0, mode="full")
        e = dict(o=_rel(got["o"], ref["o"]), S=_rel(got["S"], ref["S"]), tol=1e-4)
        if got["cov"] is not None:
            e["cov"] = _rel(got["cov"], ref["cov"])
        parity[f"tiny_{nm}"] = e
    dec = kept.get("decode")
    if dec is not None:
        c = workloads.WORKLOADS["decode"]
        bs = np.array([x for x, _ in DECODE_PARITY_HEADS])
        hs = np.array([x for _, x in DECODE_PARITY_HEADS])
        steps = []
        for i in range(dec["steps"]):
            st = workloads.decode_step_inputs(i, c["B"], c["H"], c["dk"], c["dv"])
            steps.append({n: np.ascontiguousarray(x[bs, hs][None]) for n, x in st.items()})
        o_ref, oc_ref, m_ref, S_ref, _, _ = oracle.decode_run(steps, 1, len(bs), c["dk"], c["dv"], c["w"])
        parity["decode"] = dict(o=_rel(dec["o"], o_ref[-1][0]), o_cache=_rel(dec["o_cache"], oc_ref[-1][0]),
                                m=_rel(dec["m"], m_ref[-1][0]), S=_rel(dec["S"], S_ref[0]), tol=1e-4,
                                heads=len(bs), steps=dec["steps"])
    for v_ in parity.values():
        for kk in list(v_):
            if isinstance(v_[kk], float) and kk not in ("tol", "cov_tol"):
                v_[kk] = float(f"{v_[kk]:.3e}")
    return baseline, parity


def _extra_scan(name, mode, resid="gated"):
    def run(kdn, torch, args, keep=None):
        r = bench_scan(kdn, torch, name, max(2, args.steps // 4), 1, mode=mode, per_phase=True,
                       keep=keep is not None, resid=resid)
        nb = scan_bytes(r["B"], r["H"], r["L"], r["dk"], r["dv"],
                        extra_per_token=4 if mode in ("diag", "iso") else 0)
        if keep is not None:
            keep[f"{name}/{mode if resid == 'gated' else resid}"] = {
                k: r[k] for k in ("o", "S", "cov") if k in r}
        flops = r["B"] * r["H"] * r["L"] * scan_flops_per_token_head(r["C"], r["dk"], r["dv"])
        return dict(ms_per_step=round(r["ms_per_step"], 5), tokens_per_s=round(r["tokens_per_s"], 1),
                    prepare_ms=round(r["prepare_ms"], 5), state_ms=round(r["state_ms"], 5),
                    state_kernel_ms=round(r["state_kernel_ms"], 5),
                    algorithmic_bytes=nb,
                    hbm_frac_step=round(nb / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    hbm_frac_state_kernel=round(nb / (r["state_kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    mfma_frac_step=round(flops / (r["ms_per_step"] * 1e-3) / 1e12
                                         / MFMA_F16_PEAK_TFLOPS, 4))
    return run


# the extra workloads, in the order the full run reports them
EXTRAS = {
    "decode": lambda kdn, torch, args, keep=None: bench_decode(kdn, torch, steps=max(8, args.steps),
                                                               warmup=args.warmup, keep=keep),
    "prompt_cache": lambda kdn, torch, args, keep=None: bench_prefill(
        kdn, torch, steps=max(2, args.steps // 4), warmup=1),
    "backward": lambda kdn, torch, args, keep=None: bench_backward(kdn, torch, steps=2, warmup=1),
    "kdn_diag": _extra_scan("kdn_diag", "diag"),
    "kdn_iso": _extra_scan("kdn_diag", "iso"),
    "long": _extra_scan("long", "delta"),
    # the gated workload's inputs, write without its erase term (decayed linear attention)
    "noerase": _extra_scan("gated", "delta", resid="noerase"),
}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this size (counter calibration)")
    ap.add_argument("--only", choices=list(EXTRAS), default=None,
                    help="run one of the extra workloads alone and print its result "
                         "(for profiling; not the benchmark line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the scan shards over heads with no communication, see the design notes",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import delta_rule_scans_amd as kdn
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        x = torch.ones(n, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    if args.only:
        res = EXTRAS[args.only](kdn, torch, args)
        print(json.dumps({"only": args.only, args.only: res}), flush=True)
        return

    want_parity = not args.no_cpu_baseline
    kept = {}
    main_res = bench_scan(kdn, torch, "gated", args.steps, args.warmup, cold=not args.quick,
                          keep=want_parity)
    if want_parity:
        kept["gated/delta"] = {k: main_res.pop(k) for k in ("o", "S")}
    B, H, L, dk, dv, C = (main_res[k] for k in ("B", "H", "L", "dk", "dv", "C"))
    token_heads = B * H * L
    nbytes = scan_bytes(B, H, L, dk, dv)            # bf16 o: 1032 B per token-head
    nbytes_f32o = scan_bytes(B, H, L, dk, dv, out_bytes=4)
    flops = token_heads * scan_flops_per_token_head(C, dk, dv)
    state_s = main_res["state_kernel_ms"] * 1e-3
    achieved = nbytes / state_s / 1e9
    rec = counter_record()
    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": MIN_WARMUP_S,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 matrix products, f32 accumulation and state",
        "data": "synthetic",
        "config": {"workload": "gated delta scan B=4 H=16 L=4096 d_k=d_v=128 chunk 64, "
                               "bf16 q/k/v, f32 alpha/beta/o/state",
                   "global_batch": B, "seq_len": L, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(main_res["state_kernel_ms"]),
                     "kernel": "state_kernel (sequential chunk-state scan)",
                     "kernel_ms": round(main_res["state_kernel_ms"], 5),
                     "kernel_ms_note": "ms_per_step minus the prepare phase timed back to back "
                                       "(HIP events around the launches, none inside a step)",
                     "algorithmic_bytes": nbytes,
                     "bytes_per_token_head": scan_bytes(B, H, L, dk, dv, state_out=False) // token_heads,
                     "algorithmic_bytes_note": "1032 B per token-head (bf16 q, k, v, o; float32 "
                                               "alpha, beta) x 262144 token-heads + the float32 "
                                               "final state (65536 B per head)",
                     # the library writes float32 o by default: 256 B more per token-head
                     "algorithmic_bytes_f32_output": nbytes_f32o,
                     "frac_f32_output": round(nbytes_f32o / state_s / 1e9 / HBM_PEAK_GBS, 4),
                     "step_frac": round(nbytes / (main_res["ms_per_step"] * 1e-3) / 1e9
                                        / HBM_PEAK_GBS, 4)},
        "mfma": {"algorithmic_tflops_per_step": round(flops / 1e12, 3),
                 "frac_of_peak_step": round(flops / (main_res["ms_per_step"] * 1e-3) / 1e12
                                            / MFMA_F16_PEAK_TFLOPS, 4),
                 "frac_of_peak_state_kernel": round(flops / state_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                 "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                 # from the committed counter run (null once the kernel changed):
                 # executed matrix-core flops of the state kernel over its time
                 # here, and its matrix-core busy fraction under the profiler
                 "executed_frac_state_kernel": (
                     None if rec is None else
                     round(rec["mfma_executed_flops"] / state_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)),
                 "busy_frac_state_kernel": None if rec is None else rec["mfma_busy_frac"]},
        "phases_ms": {"prepare": round(main_res["prepare_ms"], 5),
                      "state": round(main_res["state_ms"], 5),
                      "prepare_back_to_back": round(main_res["prepare_b2b_ms"], 5),
                      "note": "each phase bracketed by fence-less HIP events inside the step "
                              "sequence, on the stream the kernels run on"},
    }
    line["tiny"] = bench_tiny(kdn, torch, keep=kept if want_parity else None)
    if not args.quick:
        cms = main_res["cold_ms_per_step"]
        line["cold"] = {"ms_per_step": round(cms, 5),
                        "tokens_per_s": round(B * L / (cms * 1e-3), 1),
                        "roofline_frac_step": round(nbytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma_frac_step": round(flops / (cms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                        "note": "256 MB last-level cache flushed by a 512 MiB write before each "
                                "step; fractions over the whole step (both kernels)"}
        line["roofline"]["attainable_copy_gbs"] = copy_bandwidth(torch)
        extra = {}
        for key, fn in EXTRAS.items():
            extra[key] = fn(kdn, torch, args, keep=kept if want_parity else None)
            torch.cuda.empty_cache()
        line["extra"] = extra
    if want_parity:
        line["cpu_baseline"], line["parity"] = oracle_leg(kept)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
