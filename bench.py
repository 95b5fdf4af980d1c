"""Benchmark of causal streaming attention on one MI355X.

One step = one sattn_fwd call over the T=4096, Hq=32, Hkv=8, d=64 workload
(seeded synthetic fp16 inputs, already resident in HBM).  Prints one JSON
line: causal TFLOP/s (4*T^2*64*Hq/2 flop per call), the roofline of the
kernel against the fp16 dense MFMA peak, and the float64 CPU oracle timed on
a bounded sample of the same workload.

Warm-up: the --warmup calls, continued until at least --min-warmup-s seconds
of back-to-back calls have run (the card takes some load to reach its working
clock); the line gives the warm-up's own call count and duration.  Then
exactly --steps calls are timed.

After the timed region the kernel runs back-to-back for about two seconds
while a host thread reads the shader clock and socket power through amdsmi;
the line's "clock" object gives them and the fraction of the fp16 peak
scaled to that clock (the card is held below 2.4 GHz by board power under
matrix work on random data).

With --backward, one step is one sattn_bwd call (query launch, key launch,
grouped reduction) on the same workload, with dO seeded and O and L from the
forward; its line counts the five products S, dP, dQ, dK, dV once each
(2.5 x the forward's flop) and gives each launch's own time.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6  # MI355X dense fp16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk ("2.5 PF")
WORKLOAD_INDEX = 3
KERNEL_SRC = os.path.join(ROOT, "causal_attention_forward_amd", "csrc", "sattn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sattn_fwd_T4096_Hq32_Hkv8.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_sattn_fwd_T4096_Hq32_Hkv8.txt")
BWD_KERNEL_SRC = os.path.join(ROOT, "causal_attention_forward_amd", "csrc", "sattn_bwd.hip")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sattn_bwd_T4096_Hq32_Hkv8.txt")
BWD_COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_sattn_bwd_T4096_Hq32_Hkv8.txt")


def causal_flops(T, Hq, d=64):
    return 4.0 * T * T * d * Hq / 2.0


def kernel_sha(src=KERNEL_SRC):
    """Hash of a kernel source's code: comments and whitespace are removed
    first, so an edit of comments alone keeps the counters that were taken."""
    with open(src, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def counter_summary(path, src):
    """The key: value lines of a committed rocprofv3 counter summary, or None
    when it is missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sha") != kernel_sha(src):
        return None
    return kv


def measured_traffic(path=TRAFFIC_FILE, src=KERNEL_SRC):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    kv = counter_summary(path, src)
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def measured_utilisation(path=COUNTERS_FILE, src=KERNEL_SRC):
    """Matrix-core and VALU utilisation of the kernel from a committed
    rocprofv3 SQ-counter summary (fractions of the SIMD-cycles of a
    dispatch), or None when missing or taken on a different kernel source."""
    kv = counter_summary(path, src)
    if not kv:
        return None
    try:
        return {"mfma_busy": float(kv["mfma_busy"]), "valu_active": float(kv["valu_active"]),
                "mfma_valu_coexec": float(kv["mfma_valu_coexec"]),
                "wait_any": float(kv["wait_any"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


def measured_utilisation_backward(path=BWD_COUNTERS_FILE, src=BWD_KERNEL_SRC):
    """The backward key launch's matrix-core and VALU utilisation from the
    committed rocprofv3 SQ-counter summary (fractions of the SIMD-cycles of a
    dispatch), or None when missing or taken on a different kernel source."""
    kv = counter_summary(path, src)
    if not kv:
        return None
    try:
        return {"mfma_busy": float(kv["key_mfma_busy"]), "valu_active": float(kv["key_valu_active"]),
                "mfma_valu_coexec": float(kv["key_mfma_valu_coexec"]),
                "wait_any": float(kv["key_wait_any"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    """Threads for the oracle's BLAS calls: the CPUs this process may run on
    (its affinity mask), capped by OMP_NUM_THREADS where the host sets one
    (the share of a shared host this process is meant to use)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return (min(n, cap) if cap > 0 else n), n


def timed_oracle(run_one, units, budget_s):
    """Run `run_one(u)` for u = 0, 1, ... until `units` or about budget_s
    seconds, with BLAS limited to blas_threads(); returns (done, seconds,
    host facts)."""
    threads, affinity = blas_threads()
    facts = {"cores": threads, "affinity_cpus": affinity, "cpu_model": cpu_model(),
             "threads_note": "BLAS products on `cores` threads; NumPy's exp2, max and "
                             "sums run on one thread"}
    import contextlib
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limits = threadpool_limits(limits=threads)
    except Exception:
        threadpool_info, limits = None, contextlib.nullcontext()
    with limits:
        t0 = time.perf_counter()
        done = 0
        while done < units:
            run_one(done)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        if threadpool_info is not None:
            used = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
            if used:
                facts["cores"] = int(max(used))
    return done, dt, facts


def cpu_baseline(x, budget_s=20.0):
    """The float64 oracle on whole heads of the same workload, as many as fit
    in about budget_s seconds (at least one), scaled to TFLOP/s."""
    from oracle import attention_ref
    heads, dt, facts = timed_oracle(
        lambda h: attention_ref(x.Q, x.K, x.Vt, x.c, heads=[h]), x.Hq, budget_s)
    flops = causal_flops(x.T, 1) * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "kind": "oracle", **facts,
            "sample": f"{heads} of {x.Hq} query heads of T={x.T} Hq={x.Hq} Hkv={x.Hkv} "
                      f"({dt:.1f} s, float64 NumPy)"}


def gfx_clock_window(torch, fn, settle=1.0, seconds=1.0):
    """The shader clock while ``fn`` runs back-to-back (after the timed
    region, so the timing is undisturbed): amdsmi's current GFX clock of each
    XCD and the socket power, read every 20 ms from a host thread.  The
    driver refreshes these readings only every few hundred ms, so the first
    ``settle`` seconds (which can still show the idle clock) are discarded
    and the readings of the next ``seconds`` averaged.  None when amdsmi
    cannot read them."""
    try:
        import threading
        import amdsmi
        amdsmi.amdsmi_init()
        bus = torch.cuda.get_device_properties(0).pci_bus_id
        handle = None
        for h in amdsmi.amdsmi_get_processor_handles():
            if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                handle = h
        if handle is None:
            return None
    except Exception:
        return None
    clocks, powers = [], []
    stop = threading.Event()

    def sample():
        stop.wait(settle)
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clks = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float))]
                if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
                    clks = [m["current_gfxclk"]]
                if clks:
                    clocks.append(sum(clks) / len(clks))
                if isinstance(m.get("current_socket_power"), (int, float)):
                    powers.append(m["current_socket_power"])
            except Exception:
                pass
            stop.wait(0.02)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle + seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not clocks:
        return None
    out = {"gfx_mhz": round(sum(clocks) / len(clocks), 1), "gfx_mhz_min": round(min(clocks), 1),
           "gfx_mhz_max": round(max(clocks), 1), "samples": len(clocks),
           "source": "amdsmi current GFX clock (mean of the XCDs), averaged over "
                     f"{seconds:g} s of back-to-back launches after {settle:g} s of settling, "
                     "after the timed region"}
    if powers:
        out["socket_power_w"] = round(sum(powers) / len(powers), 1)
    return out


def clock_fields(clock, achieved):
    """The fraction of the fp16 dense peak scaled to the measured clock."""
    if clock is None:
        return None
    peak = PEAK_FP16_TFLOPS * clock["gfx_mhz"] / 2400.0
    return {**clock, "peak_at_clock": round(peak, 1), "frac_at_clock": round(achieved / peak, 4)}


def warm_up(torch, step, calls, min_seconds):
    """`calls` untimed calls, continued (in groups of ten) until at least
    `min_seconds` of back-to-back work has run: the card raises its shader
    clock over the first milliseconds of load, so a few calls alone leave the
    timed region partly at a lower clock.  Returns the warm-up's calls and
    seconds."""
    t0 = time.perf_counter()
    n = 0
    for _ in range(calls):
        step()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(10):
            step()
            n += 1
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def backward_flops(T, Hq, d=64):
    """S, dP, dQ, dK and dV, each 2*64 flop per causal (query, key) pair."""
    return 2.5 * causal_flops(T, Hq, d)


def cpu_baseline_backward(x, dO, O, L, s, budget_s=20.0):
    """The float64 backward oracle on whole query heads (each with its own
    K/V head), as many as fit in about budget_s seconds, scaled to TFLOP/s."""
    from oracle import attention_backward_ref
    G = x.Hq // x.Hkv

    def one(h):
        kv = h // G
        cols = slice(h * 64, (h + 1) * 64)
        attention_backward_ref(x.Q[h:h + 1], x.K[kv:kv + 1], x.Vt[kv:kv + 1], O[:, cols],
                               dO[:, cols], L[h:h + 1], x.c, s)

    heads, dt, facts = timed_oracle(one, x.Hq, budget_s)
    flops = backward_flops(x.T, 1) * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "kind": "oracle", **facts,
            "sample": f"backward of {heads} of {x.Hq} query heads of T={x.T} Hq={x.Hq} "
                      f"Hkv={x.Hkv} ({dt:.1f} s, float64 NumPy)"}


def bench_backward(args, torch, sattn, x, w):
    """The --backward line (see the module docstring)."""
    import numpy as np
    from causal_attention_forward_amd.inputs import make_output_gradient
    dev = torch.device("cuda:0")
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    dO_np = make_output_gradient(x.T, x.Hq, WORKLOAD_INDEX)
    do = torch.from_numpy(dO_np).to(dev)
    O, L = sattn.fwd(q, k, vt, x.c)
    T, Hq, Hkv = x.T, x.Hq, x.Hkv
    s = 0.125
    f32 = dict(dtype=torch.float32, device=dev)
    dQ, D = torch.empty((Hq, T, 64), **f32), torch.empty((Hq, T), **f32)
    dK, dVt = torch.empty((Hkv, T, 64), **f32), torch.empty((Hkv, 64, T), **f32)
    need = sattn.sattn_bwd_workspace_bytes(T, Hq, Hkv)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptr = lambda t: t.data_ptr()  # noqa: E731

    def query():
        st = sattn.sattn_bwd_query(ptr(q), ptr(k), ptr(vt), ptr(O), ptr(do), ptr(L), ptr(dQ),
                                   ptr(D), x.c, s, T, Hq, Hkv, sp)
        assert st == sattn.SATTN_OK, st

    def key():
        st = sattn.sattn_bwd_key(ptr(q), ptr(k), ptr(vt), ptr(do), ptr(L), ptr(D), ptr(dK),
                                 ptr(dVt), ptr(ws), need, x.c, s, T, Hq, Hkv, sp)
        assert st == sattn.SATTN_OK, st

    def step():
        st = sattn.sattn_bwd(ptr(q), ptr(k), ptr(vt), ptr(O), ptr(do), ptr(L), ptr(dQ), ptr(dK),
                             ptr(dVt), ptr(D), ptr(ws), need, x.c, s, T, Hq, Hkv, sp)
        assert st == sattn.SATTN_OK, st

    def timed(fn, n):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    warm_calls, warm_s = warm_up(torch, step, args.warmup, args.min_warmup_s)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_each = max(args.steps // 2, 1)
    query_ms = timed(query, n_each)
    key_ms = timed(key, n_each)

    flops = backward_flops(T, Hq)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    key_flops = 2.0 * causal_flops(T, Hq)      # S, dP, dV, dK
    query_flops = 1.5 * causal_flops(T, Hq)    # S, dP, dQ
    key_tf = key_flops / (key_ms * 1e-3) / 1e12
    out = {
        "metric": "causal attn bwd TFLOP/s (S, dP, dQ, dK, dV = 2.5x fwd flop), "
                  f"T={T} Hq={Hq} Hkv={Hkv} d=64",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": warm_calls,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name + " backward", "T": T, "Hq": Hq, "Hkv": Hkv,
                   "head_dim": 64, "causal": True, "flop_per_call": flops,
                   "query_launch_ms": round(query_ms, 5),
                   "query_launch_tflops": round(query_flops / (query_ms * 1e-3) / 1e12, 2),
                   "key_launch_and_reduction_ms": round(key_ms, 5)},
        "roofline": {"bound": "mfma", "achieved": round(key_tf, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(key_tf / PEAK_FP16_TFLOPS, 4),
                     "traffic": (measured_traffic(BWD_TRAFFIC_FILE, BWD_KERNEL_SRC)
                                 if args.workload == WORKLOAD_INDEX else None),
                     "kernel": "key launch + reduction (4 products)",
                     "kernel_ms": round(key_ms, 5),
                     "counters": (measured_utilisation_backward()
                                  if args.workload == WORKLOAD_INDEX else None)},
    }
    if not args.no_clock:
        out["clock"] = clock_fields(gfx_clock_window(torch, step), value)
    if not args.no_cpu_baseline:
        O_np = O.cpu().numpy()
        L_np = L.cpu().numpy()
        out["cpu_baseline"] = cpu_baseline_backward(x, dO_np, O_np, L_np, s, args.cpu_budget)
    print(json.dumps(out), flush=True)


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E


def bench_materialized(args, torch, sattn, x, w):
    """The --materialized line: the whole path per step, each launch alone
    (HIP events on the stream), and the streaming forward on the same inputs."""
    dev = torch.device("cuda:0")
    T, Hq, Hkv = x.T, x.Hq, x.Hkv
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    S = torch.empty((Hq, T, T), dtype=torch.float32, device=dev)
    P = torch.empty((Hq, T, T), dtype=torch.float16, device=dev)
    O = torch.empty((T, Hq * 64), dtype=torch.float16, device=dev)
    L = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    c = float(x.c)
    ptr = lambda t: t.data_ptr()  # noqa: E731

    def check(st):
        assert st == sattn.SATTN_OK, sattn.sattn_status_string(st)

    def step():
        check(sattn.sattn_mat_fwd(ptr(q), ptr(k), ptr(vt), ptr(O), ptr(L), ptr(S), ptr(P), c, T,
                                  Hq, Hkv, sp))

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    warm_calls, warm_s = warm_up(torch, step, args.warmup, args.min_warmup_s)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = max(args.steps // 2, 1)
    ms = {
        "scores_ms": timed(lambda: check(sattn.sattn_mat_scores(ptr(q), ptr(k), ptr(S), c, T, Hq,
                                                                 Hkv, sp)), n),
        "softmax_ms": timed(lambda: check(sattn.sattn_mat_softmax(ptr(S), ptr(P), ptr(L), T, Hq,
                                                                   sp)), n),
        "pv_ms": timed(lambda: check(sattn.sattn_mat_pv(ptr(P), ptr(vt), ptr(O), T, Hq, Hkv,
                                                         sp)), n),
    }

    def streaming():
        check(sattn.sattn_fwd(ptr(q), ptr(k), ptr(vt), ptr(O), ptr(L), c, T, Hq, Hkv, sp))

    timed(streaming, max(args.warmup, 100))   # its own warmup after the plane-bound launches
    ms["streaming_fwd_ms"] = timed(streaming, max(args.steps, 200))
    tri = Hq * T * (T + 1) // 2            # plane elements with j <= i
    bytes_ = {                             # algorithmic HBM bytes per launch
        "scores_ms": 4 * tri + 2 * 64 * T * (Hq + Hkv),
        "softmax_ms": 4 * tri + 2 * tri + 4 * Hq * T,
        "pv_ms": 2 * tri + 2 * 64 * T * (Hq + Hkv),
    }
    dom = max(bytes_, key=lambda k_: ms[k_])
    gbs = bytes_[dom] / (ms[dom] * 1e-3) / 1e9
    flops = causal_flops(T, Hq)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": f"causal attn fwd TFLOP/s, materialised path (scores plane, softmax, P V), "
                  f"T={T} Hq={Hq} Hkv={Hkv} d=64",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": warm_calls,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name + " materialised", "T": T, "Hq": Hq, "Hkv": Hkv,
                   "head_dim": 64, "causal": True, "flop_per_call": flops,
                   "plane_bytes": 6 * Hq * T * T,
                   **{k_: round(v_, 5) for k_, v_ in ms.items()},
                   "streaming_speedup": round(ms_per_step / ms["streaming_fwd_ms"], 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": dom.replace("_ms", ""), "algorithmic_bytes": bytes_[dom],
                     "kernel_ms": round(ms[dom], 5)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(out), flush=True)


def compulsory_bytes(T, Hq, Hkv, d=64):
    """Q, K and V^T read once, O and L written once."""
    return 2 * d * T * (Hq + 2 * Hkv) + 2 * d * T * Hq + 4 * T * Hq


def graph_time(torch, call, calls, reps, outputs):
    """Median per-call time of `calls` launches captured once in a HIP graph
    and replayed (the device's own back-to-back time, without the host's
    per-call launch cost), and whether the tensors in `outputs` hold, after
    the replays, exactly what they held before the capture (the same
    deterministic result as the eager calls).  The captured work is the
    library's kernel launches only.  (None, None) if the capture fails."""
    import statistics
    before = [t.clone() for t in outputs]
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sp = torch.cuda.current_stream().cuda_stream
            for i in range(calls):
                call(i, sp)
    except Exception:
        return None, None
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / calls)
    same = all(torch.equal(a, b) for a, b in zip(before, outputs))
    del g
    return statistics.median(times), same


def sweep(torch, sattn, workloads, make_workload, reps=5, calls=50):
    """Every synthetic workload: median over `reps` runs of `calls` back-to-back
    launches, cycling through enough input/output sets (at least 4, about
    300 MB in all, at most 64) that a small workload is not timed from cache."""
    import math
    import statistics
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for idx, w in enumerate(workloads):
        x = make_workload(idx)
        nbytes = compulsory_bytes(x.T, x.Hq, x.Hkv)
        nsets = min(64, max(4, math.ceil(300e6 / nbytes)))
        sets = []
        for _ in range(nsets):
            sets.append((torch.from_numpy(x.Q).to(dev), torch.from_numpy(x.K).to(dev),
                         torch.from_numpy(x.Vt).to(dev),
                         torch.empty((x.T, x.Hq * 64), dtype=torch.float16, device=dev),
                         torch.empty((x.Hq, x.T), dtype=torch.float32, device=dev)))

        def call(i, sp=stream.cuda_stream):
            q, k, vt, O, L = sets[i % nsets]
            st = sattn.sattn_fwd(q.data_ptr(), k.data_ptr(), vt.data_ptr(), O.data_ptr(),
                                 L.data_ptr(), x.c, x.T, x.Hq, x.Hkv, sp)
            assert st == sattn.SATTN_OK, st

        for i in range(max(200, 2 * nsets)):
            call(i)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(calls):
                call(i)
            ev1.record(stream)
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1) / calls)
        ms = statistics.median(times)
        gms, same = graph_time(torch, call, calls, reps, sets[0][3:5])
        tflops = causal_flops(x.T, x.Hq) / (ms * 1e-3) / 1e12
        out = {"sweep": w.name, "T": x.T, "Hq": x.Hq, "Hkv": x.Hkv,
               "us_per_call": round(ms * 1e3, 2), "tflops": round(tflops, 2),
               "pct_fp16_peak": round(100 * tflops / PEAK_FP16_TFLOPS, 2),
               "compulsory_bytes": nbytes, "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "input_sets": nsets}
        if gms is not None:
            gtf = causal_flops(x.T, x.Hq) / (gms * 1e-3) / 1e12
            out.update({"graph_us_per_call": round(gms * 1e3, 2), "graph_tflops": round(gtf, 2),
                        "graph_gbps": round(nbytes / (gms * 1e-3) / 1e9, 1),
                        "graph_matches_eager": same})
        print(json.dumps(out), flush=True)
        del sets
        torch.cuda.empty_cache()


def sweep_backward(torch, sattn, workloads, make_workload, reps=5, calls=20):
    """The backward on every synthetic workload (O and L from the forward on
    the same inputs, dO seeded): median over `reps` runs of `calls` launches,
    input sets rotated as in `sweep`."""
    import math
    import statistics
    from causal_attention_forward_amd.inputs import make_output_gradient
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    for idx, w in enumerate(workloads):
        x = make_workload(idx)
        T, Hq, Hkv = x.T, x.Hq, x.Hkv
        dO = make_output_gradient(T, Hq, idx)
        # read Q, K, V^T, O, dO (binary16), L; write dQ, dK, dV^T, D (binary32)
        nbytes = 2 * 64 * T * (3 * Hq + 2 * Hkv) + 4 * T * Hq + 4 * 64 * T * (Hq + 2 * Hkv) + 4 * T * Hq
        nsets = min(32, max(2, math.ceil(300e6 / nbytes)))
        need = sattn.sattn_bwd_workspace_bytes(T, Hq, Hkv)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        sets = []
        for _ in range(nsets):
            q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
            O, L = sattn.fwd(q, k, vt, x.c)
            f32 = dict(dtype=torch.float32, device=dev)
            sets.append((q, k, vt, O, torch.from_numpy(dO).to(dev), L,
                         torch.empty((Hq, T, 64), **f32), torch.empty((Hkv, T, 64), **f32),
                         torch.empty((Hkv, 64, T), **f32), torch.empty((Hq, T), **f32)))

        def call(i, sp=sp):
            q, k, vt, O, g, L, dQ, dK, dVt, D = sets[i % nsets]
            st = sattn.sattn_bwd(q.data_ptr(), k.data_ptr(), vt.data_ptr(), O.data_ptr(),
                                 g.data_ptr(), L.data_ptr(), dQ.data_ptr(), dK.data_ptr(),
                                 dVt.data_ptr(), D.data_ptr(), ws.data_ptr(), need, x.c, 0.125,
                                 T, Hq, Hkv, sp)
            assert st == sattn.SATTN_OK, st

        for i in range(max(40, 2 * nsets)):
            call(i)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(calls):
                call(i)
            ev1.record(stream)
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1) / calls)
        ms = statistics.median(times)
        # with GQA the grouped planes live in the shared workspace, so the
        # replay check covers one set's dQ, dK, dV^T and D
        gms, same = graph_time(torch, call, calls, reps, sets[0][6:10] if nsets > 1 else ())
        tflops = backward_flops(T, Hq) / (ms * 1e-3) / 1e12
        out = {"sweep_backward": w.name, "T": T, "Hq": Hq, "Hkv": Hkv,
               "us_per_call": round(ms * 1e3, 2), "tflops_algorithmic": round(tflops, 2),
               "pct_fp16_peak": round(100 * tflops / PEAK_FP16_TFLOPS, 2),
               "compulsory_bytes": nbytes, "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "input_sets": nsets}
        if gms is not None:
            gtf = backward_flops(T, Hq) / (gms * 1e-3) / 1e12
            out.update({"graph_us_per_call": round(gms * 1e3, 2),
                        "graph_tflops_algorithmic": round(gtf, 2),
                        "graph_matches_eager": same if nsets > 1 else None})
        print(json.dumps(out), flush=True)
        del sets, ws
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed calls first (continued up to --min-warmup-s)")
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="the warm-up runs at least this long: the GPU needs some load to reach "
                         "its working clock")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock window (amdsmi) after the timed region")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line, one JSON line per synthetic workload "
                         "(median of 5 timed runs, input sets rotated so small ones are not cache figures)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (sattn_bwd) instead of the forward")
    ap.add_argument("--materialized", action="store_true",
                    help="time the materialised path (scores plane, causal softmax, P V) instead")
    ap.add_argument("--workload", type=int, default=WORKLOAD_INDEX,
                    help="index of the synthetic workload (default: the T=4096 Hq=32 Hkv=8 one)")
    ap.add_argument("--vrows", action="store_true",
                    help="time the forward taking V as rows (sattn_fwd_vrows) instead of V^T")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the attention, run device-to-device copies of MIB MiB "
                         "(the reference transfer for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": args.warmup + args.steps}), flush=True)
        return

    from causal_attention_forward_amd import sattn
    from causal_attention_forward_amd.inputs import WORKLOADS, make_workload

    if args.sweep:
        if args.backward:
            sweep_backward(torch, sattn, WORKLOADS, make_workload)
        else:
            sweep(torch, sattn, WORKLOADS, make_workload)
        return

    w = WORKLOADS[args.workload]
    x = make_workload(args.workload)
    if args.materialized:
        bench_materialized(args, torch, sattn, x, w)
        return
    if args.backward:
        bench_backward(args, torch, sattn, x, w)
        return
    dev = torch.device("cuda:0")
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    O = torch.empty((x.T, x.Hq * 64), dtype=torch.float16, device=dev)
    L = torch.empty((x.Hq, x.T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    extra = {}
    if args.vrows:
        v = vt.transpose(1, 2).contiguous()   # V as rows [Hkv][T][64]

        def step():
            sattn.fwd_vrows(q, k, v, x.c, out=O, lse=L, stream=stream)

        # what V rows replace: the V^T kernel on the same values, plus the
        # V -> V^T transpose it needs first (torch's copy kernel, for scale)
        def vt_step():
            sattn.fwd(q, k, vt, x.c, out=O, lse=L, stream=stream)

        def transpose():
            vt.copy_(v.transpose(1, 2))

        def extras():  # after the timed region, on a warm GPU
            for fn, key in ((vt_step, "vt_path_kernel_ms"), (transpose, "v_transpose_ms")):
                for _ in range(50):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(200):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                extra[key] = round(e0.elapsed_time(e1) / 200, 5)
    else:
        extras = None
        def step():
            sattn.fwd(q, k, vt, x.c, out=O, lse=L, stream=stream)

    warm_calls, warm_s = warm_up(torch, step, args.warmup, args.min_warmup_s)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps  # average launch duration on the stream
    if extras is not None:
        extras()

    flops = causal_flops(x.T, x.Hq)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    # the counter summary covers the default workload only
    traffic = None if args.vrows or args.workload != WORKLOAD_INDEX else measured_traffic()
    utilisation = None if args.vrows or args.workload != WORKLOAD_INDEX else measured_utilisation()
    shape = f"T={x.T} Hq={x.Hq} Hkv={x.Hkv} d=64"
    out = {
        "metric": (f"causal attn fwd (V as rows) TFLOP/s, {shape}" if args.vrows else
                   f"causal attn fwd TFLOP/s and % fp16 MFMA peak, {shape}"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": warm_calls,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name + (" V rows" if args.vrows else ""), "T": x.T, "Hq": x.Hq,
                   "Hkv": x.Hkv, "head_dim": 64, "causal": True, "flop_per_call": flops,
                   "pct_fp16_peak": round(100 * value / PEAK_FP16_TFLOPS, 2), **extra},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(kernel_ms, 5),
                     "counters": utilisation},
    }
    if not args.no_clock:
        out["clock"] = clock_fields(gfx_clock_window(torch, step), achieved)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
