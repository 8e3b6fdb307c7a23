"""Throughput of the LR-AttnRes depth-mix read on one MI355X (gfx950).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-rows]
                    [--rows NAME,...] [--fixed-reps K] [--no-streams]

One step is the depth mix of one forward pass of the full-routing model shape of the
LR-AttnRes paper's 0.5B runs (§4.1: d = 1024, 24 layers = 48 sub-layer writes, so 49
sources and 49 read sites, site t reading sources 0..t-1) over 8 x 2048 tokens, with the
routing key the last r = 64 coordinates (§3.3). Every read site is one lrar_forward call
(bf16 sources and output, fp32 query) on torch's current stream.

Timing. Each launch is bracketed by HIP events recorded on the stream the library launches
on. Before every launch a 512 MiB device copy evicts the 256 MiB Infinity Cache and the L2s,
so every source byte comes from HBM, as it would after the sub-layers that run between two
reads in a real model. The step time is the sum of the read launches' durations; the
eviction copies are outside it (their cost is shown separately as wall time).

Output: ONE JSON line on stdout. `value` is tokens/s per read site averaged over the 49
sites (tokens x sites / total read time); `roofline` prices the read kernel's algorithmic
bytes, e (n + 1) d per token at a site with n sources, against MI355X's 8 TB/s HBM peak;
`rows` reports the other hot-path steps (block routing at d = 2048, production width
d = 7168 single-pass and two-phase, and the backward) on their own workloads, each timed
until two consecutive windows of six launches agree (the LR-AttnRes paper's App. I timing
rule: coefficient of variation <= 1 % in each window, medians within 0.5 %, at most 30
windows); `rooflines_wide` prices the bf16 forward at d >= 2048 the same way as `roofline`;
`ceilings` holds a plain streaming read and copy measured the same way, and the write rate
and per-read mix ceilings derived from them, and `ceilings.streams` the same-traffic streams
(lrar_mix_stream: a kernel's rows in and out per token with next to no arithmetic, in the
fastest of a sweep of launch shapes) that each d >= 2048 read, the headline's sites, Phase 1,
the merges and the backward are also priced against (`frac_of_stream_ceiling`); `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
WINDOW = 6                      # launches per timing window (the pages' stop rule)
MAX_WINDOWS = 30
CV_MAX = 0.01
DRIFT_MAX = 0.005
HOST_THREADS_MAX = 16           # the host CPU share of one GPU on the measurement boxes
EVICT_BYTES = 256 << 20         # copied per eviction: 256 MiB read + 256 MiB written
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "transformer_depth_wise_lrar_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(text: str) -> str:
    """A HIP source without its comments and blank lines, each line stripped: what compiles."""
    def keep(m):
        t = m.group(0)
        return "" if t.startswith("/") else t
    lines = (ln.strip() for ln in _TOKENS.sub(keep, text).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def source_digest() -> str:
    """sha256 over the code of the HIP sources (comments and layout left out): counter figures
    taken on other code are stale."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


class Evictor:
    """A device copy big enough to push every earlier line out of L2 and the MALL."""

    def __init__(self, torch, lrar):
        self.a = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
        self.b = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
        self.a.fill_(1)
        self.copy = lrar.lrar_copy(self.b, self.a, prepare=True)

    def __call__(self):
        self.copy()


class Timer:
    """Per-launch durations from HIP events on torch's current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def run(self, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def collect_ms(self):
        self.torch.cuda.synchronize()
        out = [s.elapsed_time(e) for s, e in self.pairs]
        self.pairs = []
        return out


def gen_sources(torch, n, T, d, scale, seed, dtype):
    """n [T, d] sources N(0,1) x U[scale] drawn on the device (seeded)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sc = torch.empty(n, dtype=torch.float64).uniform_(
        scale[0], scale[1], generator=torch.Generator().manual_seed(seed + 1))
    out = []
    for i in range(n):
        x = torch.randn((T, d), generator=g, device="cuda", dtype=torch.float32)
        x.mul_(float(sc[i]))
        out.append(x.to(dtype))
        del x
    return out


def gen_queries(torch, nq, r, seed, std=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((nq, r), generator=g, device="cuda", dtype=torch.float32) * std


# ---- the headline workload ----------------------------------------------------------------------

FULL = dict(T=8 * 2048, d=1024, r=64, eps=1e-6, n_sources=49, scale=(0.5, 2.0))
DEEP_MIN_SOURCES = 20  # headline reads of this many sources or more take the deeper ring


def fwd_bytes(T, d, n, e):
    return e * (n + 1) * d * T


def headline(torch, lrar, args, ev):
    c = FULL
    T, d, r, eps, S = c["T"], c["d"], c["r"], c["eps"], c["n_sources"]
    srcs = gen_sources(torch, S, T, d, c["scale"], seed=1000, dtype=torch.bfloat16)
    qs = gen_queries(torch, S, r, seed=1001)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    tm = Timer(torch)
    # Arguments marshalled once per site: the timed region holds only the library call.
    calls = [lrar.lrar_forward(srcs[:n], qs[n - 1], r, eps, out=out, prepare=True)
             for n in range(1, S + 1)]

    def step(timed):
        for n in range(1, S + 1):
            ev()
            call = calls[n - 1]
            if timed:
                tm.run(call)
            else:
                call()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = tm.collect_ms()
    per_site = [[ms[k * S + (n - 1)] for k in range(args.steps)] for n in range(1, S + 1)]
    site_ms = [sorted(v)[len(v) // 2] for v in per_site]          # median per site
    site_mean_ms = [sum(v) / len(v) for v in per_site]
    step_ms = sum(ms) / args.steps                                   # mean read time per step
    steps_ms = [sum(ms[k * S:(k + 1) * S]) for k in range(args.steps)]
    step_cv = (sum((x - step_ms) ** 2 for x in steps_ms) / args.steps) ** 0.5 / step_ms
    bytes_step = sum(fwd_bytes(T, d, n, 2) for n in range(1, S + 1))
    gbps = bytes_step / (step_ms * 1e-3) / 1e9
    sites = {str(n): dict(ms=round(site_ms[n - 1], 5),
                          GBps=round(fwd_bytes(T, d, n, 2) / (site_ms[n - 1] * 1e-3) / 1e9, 1))
             for n in SAMPLED_SITES}
    del srcs, calls
    return dict(step_ms=step_ms, step_cv=step_cv, wall_ms=wall * 1e3 / args.steps, gbps=gbps,
                T=T, S=S,
                bytes_step=bytes_step, launches=S, sites=sites, site_mean_ms=site_mean_ms)


# ---- the other hot-path steps on their own workloads --------------------------------------------

class Timing(float):
    """A launch time in ms (the median of the last two timing windows) that also carries the
    coefficient of variation of those launches, the mean, how many windows were run and
    whether the stop rule was met."""
    cv = None
    mean = None
    windows = None
    converged = None


def _cv(xs):
    m = sum(xs) / len(xs)
    return (sum((x - m) ** 2 for x in xs) / len(xs)) ** 0.5 / m


def _median(xs):
    v = sorted(xs)
    k = len(v) // 2
    return v[k] if len(v) % 2 else 0.5 * (v[k - 1] + v[k])


FIXED_REPS = None  # set by --fixed-reps: time exactly that many launches (profiling runs)


def time_calls(torch, ev, fn, reps=None, warm=3):
    """Times fn launch by launch (an eviction before each) in windows of WINDOW launches until
    two consecutive windows each have CV <= 1 % and their medians differ by <= 0.5 %, or
    MAX_WINDOWS windows have run."""
    tm = Timer(torch)
    for _ in range(warm):
        ev()
        fn()
    if FIXED_REPS is not None:
        for _ in range(FIXED_REPS):
            ev()
            tm.run(fn)
        ms = tm.collect_ms()
        t = Timing(_median(ms))
        t.cv, t.mean, t.windows, t.converged = _cv(ms), sum(ms) / len(ms), 0, False
        return t
    wins = []
    converged = False
    for _ in range(MAX_WINDOWS):
        for _ in range(WINDOW):
            ev()
            tm.run(fn)
        wins.append(tm.collect_ms())
        if len(wins) >= 2:
            a, b = wins[-2], wins[-1]
            ma, mb = _median(a), _median(b)
            if _cv(a) <= CV_MAX and _cv(b) <= CV_MAX and abs(mb - ma) <= DRIFT_MAX * ma:
                converged = True
                break
    last = wins[-2] + wins[-1] if len(wins) >= 2 else wins[-1]
    t = Timing(_median(last))
    t.cv, t.mean, t.windows, t.converged = _cv(last), sum(last) / len(last), len(wins), converged
    return t


def row_entry(ms, nbytes, tokens=None):
    """Median time, effective GB/s and fraction of peak of a timed call; with tokens, also
    the call's tokens/s (tokens = the token rows one call processes, for Phase 1 times its
    site queries)."""
    g = nbytes / (ms * 1e-3) / 1e9
    e = dict(ms=round(float(ms), 5), GBps=round(g, 1), frac=round(g / HBM_PEAK_GBPS, 4))
    if tokens is not None:
        e["tokens_per_s"] = round(tokens / (ms * 1e-3), 1)
    if getattr(ms, "cv", None) is not None:
        e["cv"] = round(ms.cv, 4)
    if getattr(ms, "windows", None):
        e["windows"] = ms.windows
        e["converged"] = ms.converged
    if getattr(ms, "mean", None) is not None:
        e["mean_ms"] = round(float(ms.mean), 5)
    return e


def rows_block_routing(torch, lrar, ev, reps):
    """Block routing, d = 2048, T = 16 x 4096: the widest site (n = 9) and the capacity
    site (n = 10), r in {16, 64, 512, 2048 = d}, both read variants."""
    T, d = 16 * 4096, 2048
    srcs = gen_sources(torch, 10, T, d, (0.5, 4.0), seed=2000, dtype=torch.bfloat16)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    res = {}
    for r in (16, 64, 512, 2048):
        q = gen_queries(torch, 1, r, seed=2001 + r)[0]
        for n in (9, 10):
            for var in ("two_pass", "online"):
                ms = time_calls(torch, ev, lrar.lrar_forward(
                    srcs[:n], q, r, 1e-6, out=out, variant=var, prepare=True))
                res[f"r{r}_n{n}_{var}"] = row_entry(ms, fwd_bytes(T, d, n, 2), T)
    del srcs, out
    return res


def rows_production(torch, lrar, ev, reps):
    """Production width d = 7168, T = 32768, 93 writes in 8 blocks (n <= 9): single-pass
    reads at r in {64, 1792, 7168}; the two-phase schedule of the largest block (Phase 1:
    8 cached sources x 12 site queries; Phase 2: one merge per site with the partial sum, and
    the same merge with the partial-sum update b' = b + o fused in)."""
    T, d, nq = 32768, 7168, 12
    srcs = gen_sources(torch, 9, T, d, (0.5, 4.0), seed=3000, dtype=torch.bfloat16)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    res = {}
    for r in (64, 1792, 7168):
        q = gen_queries(torch, 1, r, seed=3001 + r)[0]
        for var in ("two_pass", "online"):
            ms = time_calls(torch, ev, lrar.lrar_forward(
                srcs, q, r, 1e-6, out=out, variant=var, prepare=True))
            res[f"single_pass_r{r}_n9_{var}"] = row_entry(ms, fwd_bytes(T, d, 9, 2), T)
    r = 1792
    qs = gen_queries(torch, nq, r, seed=3100)
    for acc_name, acc_dt, ae in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        m = torch.empty((nq, T), dtype=torch.float32, device="cuda")
        l = torch.empty((nq, T), dtype=torch.float32, device="cuda")
        acc = torch.empty((nq, T, d), dtype=acc_dt, device="cuda")
        ms1 = time_calls(torch, ev, lrar.lrar_forward_stats(
            srcs[:8], qs, r, 1e-6, m=m, l=l, acc=acc, prepare=True))
        b1 = 2 * 8 * d * T + nq * (ae * d + 8) * T
        res[f"phase1_r{r}_ninter8_q{nq}_acc{acc_name}"] = row_entry(ms1, b1, T * nq)
        ms2 = time_calls(torch, ev, lrar.lrar_merge(
            m[0], l[0], acc[0], srcs[8:9], qs[0], r, 1e-6, out=out, prepare=True))
        b2 = (ae * d + 8 + 2 * d + 2 * d) * T
        res[f"phase2_r{r}_acc{acc_name}"] = row_entry(ms2, b2, T)
        # the same site with the partial-sum update fused in: b' = b + o is written and merged
        bnew = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        ms3 = time_calls(torch, ev, lrar.lrar_merge_accumulate(
            m[0], l[0], acc[0], srcs[8], srcs[7], qs[0], r, 1e-6, out=out, b_out=bnew,
            prepare=True))
        b3 = (ae * d + 8 + 2 * d + 2 * d + 2 * d + 2 * d) * T
        res[f"phase2_fused_update_r{r}_acc{acc_name}"] = row_entry(ms3, b3, T)
        del m, l, acc, bnew
    del srcs, out
    return res


def rows_backward(torch, lrar, ev, reps):
    """Backward of block routing: d = 4096, r = 1024, n = 10, T = 16384, with fp32 gradients
    and with bf16 gradients."""
    T, d, r, n = 16384, 4096, 1024, 10
    srcs = gen_sources(torch, n, T, d, (0.5, 4.0), seed=4000, dtype=torch.bfloat16)
    q = gen_queries(torch, 1, r, seed=4001)[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(4002)
    dout = torch.randn((T, d), generator=g, device="cuda", dtype=torch.float32)
    dsrc = [torch.empty((T, d), dtype=torch.float32, device="cuda") for _ in range(n)]
    dq = torch.empty((r,), dtype=torch.float32, device="cuda")
    ws = torch.empty((lrar.lrar_backward_workspace_size(T, d, r, n),), dtype=torch.uint8,
                     device="cuda")
    ms = time_calls(torch, ev, lrar.lrar_backward(
        srcs, q, dout, r, 1e-6, dsrc=dsrc, dq=dq, workspace=ws, prepare=True))
    nbytes = (2 * n * d + 4 * d + 4 * n * d) * T + 4 * r
    res = {f"backward_r{r}_n{n}": row_entry(ms, nbytes, T)}
    del dsrc
    # bf16 gradients (dout and dsrc bf16), as the pages' own kernel writes them
    dout16 = dout.to(torch.bfloat16)
    dsrc16 = [torch.empty((T, d), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    ms16 = time_calls(torch, ev, lrar.lrar_backward_grad(
        srcs, q, dout16, r, 1e-6, dsrc=dsrc16, dq=dq, workspace=ws, prepare=True))
    res[f"backward_bf16_grads_r{r}_n{n}"] = row_entry(
        ms16, (2 * n * d + 2 * d + 2 * n * d) * T + 4 * r, T)
    # the same from the forward's saved statistics (z_i, 1 / rho_i per row: 16 n more bytes
    # read per row), with fp32 and bf16 gradients
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    _, saved = lrar.lrar_forward_save(srcs, q, r, 1e-6, out=out)
    dsrc = [torch.empty((T, d), dtype=torch.float32, device="cuda") for _ in range(n)]
    mss = time_calls(torch, ev, lrar.lrar_backward_saved(
        srcs, q, saved, dout, r, dsrc=dsrc, dq=dq, workspace=ws, prepare=True))
    res[f"backward_saved_r{r}_n{n}"] = row_entry(mss, nbytes + 16 * n * T, T)
    del dsrc
    mss16 = time_calls(torch, ev, lrar.lrar_backward_saved(
        srcs, q, saved, dout16, r, dsrc=dsrc16, dq=dq, workspace=ws, prepare=True))
    res[f"backward_saved_bf16_grads_r{r}_n{n}"] = row_entry(
        mss16, (2 * n * d + 2 * d + 2 * n * d) * T + 4 * r + 16 * n * T, T)
    del srcs, dsrc16, dout, dout16, saved, out
    return res


def rows_read_variants(torch, lrar, ev, reps):
    """The full-width-RMS control read and the separate-key read on the full-routing shape
    (T = 16384, d = 1024, bf16), at the widest site (n = 49) and a middle one (n = 13): the
    control at r = 64, the separate keys at r = 32 (the pages' projected rank) and r = 64.
    The separate-key read also reads n keys of r elements per token."""
    T, d, r = 8 * 2048, 1024, 64
    srcs = gen_sources(torch, 49, T, d, (0.5, 2.0), seed=5000, dtype=torch.bfloat16)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    res = {}
    q = gen_queries(torch, 1, r, seed=5001)[0]
    for n in (13, 49):
        ms = time_calls(torch, ev, lrar.lrar_forward_fullrms(
            srcs[:n], q, r, 1e-6, out=out, prepare=True))
        res[f"fullrms_r{r}_n{n}"] = row_entry(ms, fwd_bytes(T, d, n, 2), T)
    for rk in (32, 64):
        keys = gen_sources(torch, 49, T, rk, (0.5, 2.0), seed=5100 + rk, dtype=torch.bfloat16)
        qk = gen_queries(torch, 1, rk, seed=5002 + rk)[0]
        for n in (13, 49):
            ms = time_calls(torch, ev, lrar.lrar_forward_keys(
                srcs[:n], keys[:n], qk, rk, 1e-6, out=out, prepare=True))
            res[f"keys_r{rk}_n{n}"] = row_entry(ms, fwd_bytes(T, d, n, 2) + 2 * n * rk * T, T)
        del keys
    del srcs, out
    return res


# ---- the CPU baseline: the oracle on a bounded sample -------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, budget_s=15.0):
    """The fp64 oracle on the first R rows of the headline workload, all 49 sites, run on the
    host cores this process may use (the oracle itself is single-threaded), at most the host
    CPU share of one GPU."""
    import oracle
    from transformer_depth_wise_lrar_amd import synth

    c = FULL
    d, r, eps, S = c["d"], c["r"], c["eps"], c["n_sources"]
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(HOST_THREADS_MAX, avail))
    srcs_dev = gen_sources(torch, S, 4096, d, c["scale"], seed=1000, dtype=torch.bfloat16)
    qs = synth.to_f64(gen_queries(torch, S, r, seed=1001))
    srcs = [synth.to_f64(s) for s in srcs_dev]
    del srcs_dev

    def run(R):
        chunk = (R + threads - 1) // threads

        def work(lo):
            hi = min(R, lo + chunk)
            for n in range(1, S + 1):
                oracle.forward([s[lo:hi] for s in srcs[:n]], qs[n - 1], r, eps)

        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(0, R, chunk)))
        return time.perf_counter() - t0

    R = threads * 4
    dt = run(R)
    R = int(min(4096, max(R, R * budget_s / 3 / max(dt, 1e-3))))
    R -= R % threads or 0
    # Whole passes over the sample until the budget is spent.
    passes, dt = 0, 0.0
    while dt < budget_s:
        dt += run(R)
        passes += 1
    rate = passes * R * S / dt
    return dict(value=round(rate, 1), unit="tokens/s per read site", cores=threads,
                kind="oracle", cpu_model=cpu_model(), host_logical_cpus=os.cpu_count(),
                affinity_cpus=avail,
                sample=f"full routing d=1024 r=64: rows 0..{R - 1} of T=16384, all 49 sites, "
                       f"{passes} passes, fp64 oracle (C++, -O2) on {threads} host threads "
                       f"({dt:.1f} s); threads capped at the {HOST_THREADS_MAX}-core host share "
                       f"of one GPU")


def ceilings(torch, lrar, ev):
    """Plain streams over 1 GiB, timed like the rows: a read (lrar_read_stream) and a copy
    (lrar_copy, 1 GiB read + 1 GiB written). The write rate follows from the copy's time less
    the read time of its read half: W = B / (t_copy - B / R)."""
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(3)
    ms_r = time_calls(torch, ev, lrar.lrar_read_stream(a, prepare=True))
    ms_c = time_calls(torch, ev, lrar.lrar_copy(b, a, prepare=True))
    del a, b
    read = row_entry(ms_r, nbytes)
    copy = row_entry(ms_c, 2 * nbytes)
    R = read["GBps"]
    t_write = ms_c * 1e-3 - nbytes / (R * 1e9)
    W = nbytes / t_write / 1e9 if t_write > 0 else None
    return dict(read=read, copy=copy, write_GBps_derived=round(W, 1) if W else None)


# Shapes of the same-traffic streams: the headline's sampled sites and the bf16 forward at
# d >= 2048 (T, d, n), one bf16 row out per n read.
SAMPLED_SITES = (1, 2, 5, 9, 13, 25, 37, 49)
STREAM_SHAPES = tuple((16 * 1024, 1024, n) for n in SAMPLED_SITES) + (
    (16 * 4096, 2048, 10), (16 * 4096, 2048, 9), (32768, 7168, 9))
STREAM_LAUNCHES = [(w, p, c) for w in (4, 8, 12) for p in (1, 2) for c in (0, 2, 4, 8)]
# The other kernels' traffic as streams: name -> (T, d, bf16 rows in, rows out, out dtype, the
# rows it prices). A float32 row read counts as two bf16 rows (Phase 2's fp32 accumulator, the
# backward's fp32 upstream gradient); Phase 1's m and l (8 bytes per query and row) and the
# backward's dq are left out (under 0.03 % of the bytes).
KERNEL_STREAMS = {
    "phase1_d7168_8in_12f32out": (32768, 7168, 8, 12, "f32", [
        ("production_d7168", "phase1_r1792_ninter8_q12_accf32")]),
    "phase1_d7168_8in_12bf16out": (32768, 7168, 8, 12, "bf16", [
        ("production_d7168", "phase1_r1792_ninter8_q12_accbf16")]),
    "merge_d7168_3in_1out": (32768, 7168, 3, 1, "bf16", [
        ("production_d7168", "phase2_r1792_accf32")]),
    "merge_d7168_2in_1out": (32768, 7168, 2, 1, "bf16", [
        ("production_d7168", "phase2_r1792_accbf16")]),
    "fused_update_d7168_4in_2out": (32768, 7168, 4, 2, "bf16", [
        ("production_d7168", "phase2_fused_update_r1792_accf32")]),
    "fused_update_d7168_3in_2out": (32768, 7168, 3, 2, "bf16", [
        ("production_d7168", "phase2_fused_update_r1792_accbf16")]),
    "backward_d4096_12in_10f32out": (16384, 4096, 12, 10, "f32", [
        ("backward_d4096", "backward_r1024_n10"), ("backward_d4096", "backward_saved_r1024_n10")]),
    "backward_d4096_11in_10bf16out": (16384, 4096, 11, 10, "bf16", [
        ("backward_d4096", "backward_bf16_grads_r1024_n10"),
        ("backward_d4096", "backward_saved_bf16_grads_r1024_n10")]),
}
# The streams' waves kept apart (0), or meeting at a workgroup barrier once per row (1) or
# once per group of sources loaded together (2), as the reads keep theirs in lockstep.
STREAM_LOCKSTEP = (0, 1, 2)
KERNEL_STREAM_LAUNCHES = [(w, p, c) for w in (4, 8, 12, 16, 24, 32) for p in (1, 2) for c in (0, 2, 4)]


def stream_slots(d):
    """Units a lane for the same-traffic stream of width d: whole rows in one group up to 16 units
    a lane (d <= 8192), else groups of 4."""
    nur = d // 8
    for u in (2, 4, 8, 16):
        if nur <= 64 * u:
            return (u,) if u <= 4 else (4, u)
    return (4,)


def stream_row_waves(d):
    """Waves sharing a row in the same-traffic stream of width d: from d = 4096 (512 units) a
    row also goes to 2 or 4 waves of a workgroup, as the reads of such rows share theirs."""
    return (1, 2, 4) if d >= 4096 else (1,)


def best_stream(torch, lrar, ev, srcs, outs, launches, slots):
    """Times lrar_mix_stream over every launch shape (waves per CU, sources loaded together,
    rows per row group per launch), units a lane, lockstep (none, per row, per source group)
    and waves per row (stream_row_waves; a shared row takes 4 units a lane), 4 launches each,
    then the fastest like the rows: (its timing, its launch shape)."""
    d = srcs[0].shape[1]
    shapes = [(u, 1) for u in slots] + [(4, g) for g in stream_row_waves(d) if g > 1]
    best = None
    for w, pdep, c in launches:
        for u, g in shapes:
            if pdep * u > 16:
                continue
            for lk in STREAM_LOCKSTEP:
                call = lrar.lrar_mix_stream(srcs, out=outs, waves_per_cu=w, depth=pdep, slots=u,
                                            rows_per_wave=c, lockstep=lk, waves_per_row=g,
                                            prepare=True)
                tm = Timer(torch)
                ev()
                call()
                for _ in range(4):
                    ev()
                    tm.run(call)
                ms = _median(tm.collect_ms())
                if best is None or ms < best[0]:
                    best = (ms, w, pdep, u, c, lk, g)
    _, w, pdep, u, c, lk, g = best
    ms = time_calls(torch, ev, lrar.lrar_mix_stream(srcs, out=outs, waves_per_cu=w, depth=pdep,
                                                    slots=u, rows_per_wave=c, lockstep=lk,
                                                    waves_per_row=g, prepare=True))
    return ms, dict(waves_per_cu=w, depth=pdep, slots=u, rows_per_wave=c, lockstep=lk,
                    waves_per_row=g)


def stream_ceilings(torch, lrar, ev):
    """Each kernel's traffic as a plain stream (lrar_mix_stream: n bf16 rows in and one or more
    rows out per token, next to no arithmetic), in the fastest of a sweep of launch shapes:
    what HBM gives that mix of reads and writes, measured rather than derived. The read's
    mixes (STREAM_SHAPES: n rows in, one bf16 row out) sweep STREAM_LAUNCHES; Phase 1's, the
    merges' and the backward's (KERNEL_STREAMS) sweep KERNEL_STREAM_LAUNCHES."""
    out = {}
    for T, d, n in STREAM_SHAPES:
        srcs = gen_sources(torch, n, T, d, (0.5, 4.0), seed=9000 + d + n, dtype=torch.bfloat16)
        dst = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        ms, launch = best_stream(torch, lrar, ev, srcs, dst, STREAM_LAUNCHES, stream_slots(d))
        e = row_entry(ms, fwd_bytes(T, d, n, 2))
        e["launch"] = launch
        out[f"d{d}_n{n}"] = e
        del srcs, dst
        torch.cuda.empty_cache()
    for name, (T, d, n, nout, odt, _) in KERNEL_STREAMS.items():
        srcs = gen_sources(torch, n, T, d, (0.5, 4.0), seed=9100 + d + n, dtype=torch.bfloat16)
        tdt, oe = (torch.float32, 4) if odt == "f32" else (torch.bfloat16, 2)
        outs = [torch.empty((T, d), dtype=tdt, device="cuda") for _ in range(nout)]
        ms, launch = best_stream(torch, lrar, ev, srcs, outs, KERNEL_STREAM_LAUNCHES,
                                 stream_slots(d))
        e = row_entry(ms, (2 * n + oe * nout) * d * T)
        e["launch"] = launch
        out[name] = e
        del srcs, outs
        torch.cuda.empty_cache()
    return out


def kernel_stream_fractions(rows, ceil):
    """Each priced row's GB/s as a share of its kernel stream's."""
    streams = (ceil or {}).get("streams", {})
    for name, (_, _, _, _, _, priced) in KERNEL_STREAMS.items():
        st = streams.get(name)
        if not st:
            continue
        for group, key in priced:
            e = rows.get(group, {}).get(key)
            if e is not None:
                e["stream"] = name
                e["stream_ceiling_GBps"] = st["GBps"]
                e["frac_of_stream_ceiling"] = round(e["GBps"] / st["GBps"], 4)


def mix_ceiling(ceil, n):
    """Streaming ceiling of a read of n sources that writes one row per n rows read."""
    if not ceil:
        return None
    R, W = ceil["read"]["GBps"], ceil.get("write_GBps_derived")
    if not W:
        return None
    return 1.0 / ((n / (n + 1)) / R + (1.0 / (n + 1)) / W)


# ---- main ------------------------------------------------------------------------------------------

def traffic_entry(digest, key):
    """HBM bytes per launch of one measured kernel from rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by what they read for a copy of known size), if taken on these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != digest:
        return None
    e = t.get("kernels", {}).get(key)
    return None if e is None else e.get("bytes_per_launch")


ROW_GROUPS = (("block_routing_d2048", rows_block_routing),
              ("production_d7168", rows_production),
              ("backward_d4096", rows_backward),
              ("read_variants_d1024", rows_read_variants))

# The bf16 forward at d >= 2048 (block routing and production width, online variant): each row
# is priced like `roofline`, algorithmic bytes per launch over the mean launch time.
WIDE_ROOFLINES = (
    [("block_routing_d2048", f"r{r}_n{n}_online", 16 * 4096, 2048, n, r)
     for n in (10, 9) for r in (16, 64, 512, 2048)]
    + [("production_d7168", f"single_pass_r{r}_n9_online", 32768, 7168, 9, r)
       for r in (64, 1792, 7168)])


def wide_rooflines(rows, ceil, digest):
    out = []
    for group, key, T, d, n, r in WIDE_ROOFLINES:
        e = rows.get(group, {}).get(key)
        if e is None:
            continue
        nbytes = fwd_bytes(T, d, n, 2)
        ms = e.get("mean_ms", e["ms"])
        achieved = nbytes / (ms * 1e-3) / 1e9
        mix = mix_ceiling(ceil, n) if ceil else None
        st = (ceil or {}).get("streams", {}).get(f"d{d}_n{n}")
        sg = st["GBps"] if st else None
        out.append(dict(workload=f"{group.replace('_', ' ')}: T={T} d={d} r={r} n={n}, bf16",
                        row=f"{group}/{key}", bound="hbm", achieved=round(achieved, 1),
                        peak=HBM_PEAK_GBPS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4),
                        traffic=traffic_entry(digest, f"{group}/{key}"),
                        algorithmic_bytes_per_launch=nbytes, avg_launch_us=round(ms * 1e3, 3),
                        mix_ceiling_GBps=round(mix, 1) if mix else None,
                        frac_of_mix_ceiling=round(achieved / mix, 4) if mix else None,
                        stream_ceiling_GBps=sg,
                        frac_of_stream_ceiling=round(achieved / sg, 4) if sg else None))
    return out


def block_schedules(rows):
    """The largest block of the production-width shape (d = 7168, 12 read sites, each reading the
    8 cached sources and the intra-block partial sum) under both schedules, from the measured
    rows: single-pass, 12 reads of 9 sources; two-phase, one Phase 1 of the 12 site queries
    against the 8 cached sources, then 12 Phase-2 merges with the partial sum (fp32 or bf16
    accumulators). Bytes are algorithmic; times the rows' medians."""
    pr = rows.get("production_d7168")
    if not pr:
        return None
    T, d, S = 32768, 7168, 12
    out = {}
    for r in (1792,):
        sp = pr.get(f"single_pass_r{r}_n9_online")
        if sp is None:
            continue
        e = {"single_pass": dict(ms=round(S * sp["ms"], 4),
                                 GB=round(S * fwd_bytes(T, d, 9, 2) / 1e9, 2))}
        for acc, ae in (("f32", 4), ("bf16", 2)):
            p1 = pr.get(f"phase1_r{r}_ninter8_q{S}_acc{acc}")
            p2 = pr.get(f"phase2_r{r}_acc{acc}")
            if p1 is None or p2 is None:
                continue
            b1 = 2 * 8 * d * T + S * (ae * d + 8) * T
            b2 = (ae * d + 8 + 2 * d + 2 * d) * T
            e[f"two_phase_acc{acc}"] = dict(ms=round(p1["ms"] + S * p2["ms"], 4),
                                            GB=round((b1 + S * b2) / 1e9, 2))
        out[f"d{d}_r{r}_block_of_{S}_sites"] = e
    return out


def main():
    global FIXED_REPS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the headline step (profiling runs of single rows)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming ceilings (profiling runs of single rows)")
    ap.add_argument("--no-streams", action="store_true",
                    help="skip the sweep of same-traffic streams (profiling runs)")
    ap.add_argument("--rows", default=None,
                    help="comma-separated row groups to run (default: all): "
                         + ", ".join(n for n, _ in ROW_GROUPS))
    ap.add_argument("--fixed-reps", type=int, default=None,
                    help="time exactly this many launches per row instead of the stop rule "
                         "(profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the depth-mix read shards by token rows with no "
              "exchange in the forward, so there is no multi-GPU run here (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    FIXED_REPS = args.fixed_reps

    import torch

    import transformer_depth_wise_lrar_amd as lrar

    lrar.lib()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    ev = Evictor(torch, lrar)
    h = None
    if not args.no_headline:
        log(f"bench: headline full routing, steps={args.steps} warmup={args.warmup}")
        h = headline(torch, lrar, args, ev)
        log(f"bench: headline {h['step_ms']:.3f} ms/step, {h['gbps']:.0f} GB/s")
    ceil = None
    if not args.no_ceilings:
        ceil = ceilings(torch, lrar, ev)
        log(f"bench: ceilings read {ceil['read']['GBps']:.0f} GB/s, copy "
            f"{ceil['copy']['GBps']:.0f} GB/s, write (derived) {ceil['write_GBps_derived']} GB/s")
        if not args.no_streams:
            ceil["streams"] = stream_ceilings(torch, lrar, ev)
            log("bench: same-traffic streams " + ", ".join(
                f"{k} {v['GBps']:.0f} GB/s" for k, v in ceil["streams"].items()))
    rows = {}
    want = None if args.rows is None else set(args.rows.split(","))
    if not args.no_rows:
        for name, fn in ROW_GROUPS:
            if want is not None and name not in want:
                continue
            log(f"bench: row {name}")
            rows[name] = fn(torch, lrar, ev, None)
            torch.cuda.empty_cache()
    digest = source_digest()
    roofline = None
    if h is not None:
        # The dominant kernel: at d = 1024 the library reads 20 or more sources with its
        # deeper-ring tile instantiation (three sources in flight), which serves sites n = 20..49
        # and moves 84 % of the step's bytes; sites n = 2..19 run the two-deep instantiation.
        deep = range(DEEP_MIN_SOURCES, h["S"] + 1)
        bytes_launch = sum(fwd_bytes(h["T"], FULL["d"], n, 2) for n in deep) / len(deep)
        avg_launch_s = sum(h["site_mean_ms"][n - 1] for n in deep) * 1e-3 / len(deep)
        achieved = bytes_launch / avg_launch_s / 1e9
        roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS,
                        unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4),
                        traffic=traffic_entry(digest, "headline"),
                        kernel="k_read_tile<bf16, 8, 2, 1, 2, true, 2, 3, 1, online> "
                               "(d=1024, r=64; sites n=20..49)",
                        algorithmic_bytes_per_launch=round(bytes_launch),
                        avg_launch_us=round(avg_launch_s * 1e6, 3),
                        launches_per_step=len(deep))
        st49 = (ceil or {}).get("streams", {}).get(f"d{FULL['d']}_n{h['S']}")
        if st49:
            site49 = h["sites"].get(str(h["S"]), {}).get("GBps")
            roofline["stream_ceiling_n49_GBps"] = st49["GBps"]
            roofline["site_n49_frac_of_stream_ceiling"] = (
                round(site49 / st49["GBps"], 4) if site49 else None)
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(torch)
    line = {
        "metric": "depth-mix tokens/sec and effective HBM GB/s (% of MI355X peak), bf16, per site",
        "value": None, "unit": "tokens/s per read site (mean over 49 sites)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full routing d=1024 r=64, 49 sources / 49 read sites, "
                               "T=8x2048 tokens, bf16 sources, fp32 queries",
                   "global_batch": 8, "seq_len": 2048, "parallelism": "none (1 GPU)"},
    }
    if h is not None:
        line.update({
            "value": round(h["T"] * h["S"] / (h["step_ms"] * 1e-3), 1),
            "ms_per_step": round(h["step_ms"], 4),
            "step_cv": round(h["step_cv"], 4),
            "effective_GBps": round(h["gbps"], 1),
            "wall_ms_per_step_with_eviction": round(h["wall_ms"], 3),
            "sites": h["sites"],
            "mix_ceiling_n49_GBps": round(mix_ceiling(ceil, 49), 1) if ceil else None,
        })
    if h is not None and ceil is not None:
        for n, e in h["sites"].items():
            st = ceil.get("streams", {}).get(f"d{FULL['d']}_n{n}")
            if st:
                e["stream_ceiling_GBps"] = st["GBps"]
                e["frac_of_stream_ceiling"] = round(e["GBps"] / st["GBps"], 4)
    kernel_stream_fractions(rows, ceil)
    line.update({"schedules": block_schedules(rows)})
    line.update({
        "roofline": roofline,
        "rooflines_wide": wide_rooflines(rows, ceil, digest),
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "rows": rows,
        "timing": dict(window=WINDOW, max_windows=MAX_WINDOWS, cv_max=CV_MAX,
                       drift_max=DRIFT_MAX, fixed_reps=FIXED_REPS),
        "source_digest": digest,
    })
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
