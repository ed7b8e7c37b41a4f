"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the causal prefill forward, B=1, H=32, Nq=Nk=8192, d=128,
bf16, one K row per head scaled by 30 (the largest workload; one step = one
fa_fwd over the whole batch, inputs resident in HBM).  It prints ONE JSON line
whose ``value`` is that forward's throughput in TFLOP/s (4*B*H*Nq*Nk*d per
step, halved under causal).  ``parts`` holds the other workloads measured the
same way: the non-causal d=64 prefill forward, the causal backward
(10*B*H*N^2*d/2 per step) and split-KV decoding (GB/s of K, V, Q, O and L).

Every workload, the primary one and each part, carries
  roofline      its dominant kernel against the published peak: achieved
                work per launch / launch time (HIP events on the launch
                stream), HBM traffic from the committed counter profile while
                the kernel source is unchanged, the sustained shader clock,
                and the median and minimum over repeated timed regions;
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of the
                same inputs, in the workload's unit (forward: the dense
                definition and the online recurrence with 64-key blocks;
                backward: the dense Jacobian backward; decode: the dense
                definition and split-and-merge), with the thread count used;
  parity        the largest errors of the GPU result against the oracle on
                that sample, beside the tolerances.

After each workload is timed it keeps running back to back for --clock-s
seconds while a thread reads the shader clock the driver reports
(``sclk_mhz``, the median of the samples; ``sustained_ms``, the time per step
over the same interval): under these loads the clock stays below the 2.4 GHz
the published matrix peak assumes, and ``frac_at_sclk`` is the sustained rate
over the peak scaled to the clock measured.

--sweep times the bf16 forward (d = 64 and 128, with and without the causal
mask) and the causal backward over sequence lengths 512 .. 16384 at a fixed
2^18 tokens per call (B = 1, H = 2^18 / N), one JSON line per shape.

--workload selects another workload as the primary one.  --copy-calibration
runs a plain device copy of known size (for scaling rocprofv3 FETCH_SIZE and
WRITE_SIZE counters to bytes).  Only one GPU is used; --gpus N > 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_SCLK_MHZ = 2400.0      # the engine clock that peak is quoted at
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill_d64": "fwd_bf16.hip", "prefill_causal_d128": "fwd_bf16.hip",
    "bwd_causal_d64": "bwd.hip", "decode_d128": "decode.hip",
}


def source_hash(name: str) -> str:
    """Hash of a kernel source, the device headers and the generated code it includes, with
    comments and white space removed: measured traffic stays valid across
    changes to comments and layout, and lapses with any change to the code."""
    import re
    csrc = os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "csrc")
    with open(os.path.join(csrc, name)) as fh:
        src = fh.read()
    # generated code it includes (the d = 128 forward step) counts as its code
    incs = re.findall(r'#include "([\w.]+\.inc)"', src)
    text = ""
    for f in [name, "fa_device.h", "fa_internal.h"] + incs:
        with open(os.path.join(csrc, f)) as fh:
            text += fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle", type=float, default=0.3,
                   help="keep warming up (untimed) until this many seconds have passed")
    p.add_argument("--workload", default="prefill_causal_d128",
                   choices=["prefill_d64", "prefill_causal_d128", "bwd_causal_d64",
                            "decode_d128"])
    p.add_argument("--n-split", type=int, default=None, help="decode: splits (default best)")
    p.add_argument("--no-parts", action="store_true", help="time only the primary workload")
    p.add_argument("--no-cpu", action="store_true",
                   help="skip the oracle baseline and the parity sample")
    p.add_argument("--cpu-budget", type=float, default=6.0,
                   help="seconds of oracle work per routine and workload (bounded sample)")
    p.add_argument("--repeats", type=int, default=5,
                   help="timed regions of K steps per workload for the median and minimum")
    p.add_argument("--clock-s", type=float, default=1.5,
                   help="seconds of extra steps per workload while the clock is sampled (0: off)")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--sweep", action="store_true",
                   help="forward and backward over sequence lengths; one JSON line per shape")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Workload runners: each returns (callable step, work units per step, unit info)
# ---------------------------------------------------------------------------
def setup(name, fa, torch, n_split=None):
    from fa_inputs import WORKLOADS, workload_inputs
    w = WORKLOADS[name]
    x = workload_inputs(name, device="cuda")
    B, H, Nq, d = x.q.shape
    Nk = x.k.shape[2]
    scale = 1.0 / math.sqrt(d)
    causal = w["causal"][0]
    cfg = {"workload": name, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "causal": causal,
           "dtype": "bf16"}
    if name.startswith("prefill"):
        o = torch.empty_like(x.q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")

        def step():
            fa.fa_fwd(x.q, x.k, x.v, o, lse, scale, causal)
        flops = 4.0 * B * H * Nq * Nk * d * (0.5 if causal else 1.0)
        return dict(step=step, work=flops, unit="TFLOP/s", bound="mfma", cfg=cfg, x=x,
                    scale=scale, causal=causal, kernel="fwd_bf16_kernel", out=dict(o=o, lse=lse))
    if name.startswith("bwd"):
        o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
        ws = torch.empty(fa.fa_bwd_workspace_size(x.q.dtype, B, H, Nq, d), dtype=torch.uint8,
                         device="cuda")
        dq, dk, dv = torch.empty_like(x.q), torch.empty_like(x.k), torch.empty_like(x.v)

        def step():
            fa.fa_bwd(x.q, x.k, x.v, o, lse, x.do, dq, dk, dv, ws, scale, causal)
        flops = 10.0 * B * H * Nq * Nk * d * (0.5 if causal else 1.0)
        return dict(step=step, work=flops, unit="TFLOP/s", bound="mfma", cfg=cfg, x=x,
                    scale=scale, causal=causal,
                    kernel="bwd_dkdv_pipe_kernel" if d == 64 else "bwd_dkdv_kernel",
                    out=dict(dq=dq, dk=dk, dv=dv),
                    extra={"flops_no_recompute": 8.0 * B * H * Nq * Nk * d * 0.5})
    # decode
    splits = [n_split] if n_split else list(w["n_split"])
    pm = {n: torch.empty((B, H, Nq, n), dtype=torch.float32, device="cuda") for n in splits}
    pl = {n: torch.empty_like(pm[n]) for n in splits}
    po = {n: torch.empty((B, H, Nq, n, d), dtype=torch.float32, device="cuda") for n in splits}
    o = torch.empty_like(x.q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    state = {"n": splits[0]}

    def step():
        n = state["n"]
        fa.fa_decode_split(x.q, x.k, x.v, pm[n], pl[n], po[n], n, scale)
        fa.fa_merge_states(pm[n], pl[n], po[n], o, lse)
    bytes_ = 2.0 * (2 * B * H * Nk * d + 2 * B * H * Nq * d) + 4.0 * B * H * Nq
    return dict(step=step, work=bytes_, unit="GB/s", bound="hbm", cfg=cfg, x=x, scale=scale,
                causal=False, kernel="decode_split_kernel", splits=splits, state=state,
                out=dict(o=o, lse=lse),
                partial_bytes={n: 4.0 * B * H * Nq * n * (d + 2) * 2 for n in splits})


def timed(torch, step, steps, warmup, settle_s):
    """ms per step over exactly `steps` timed steps, after `warmup` untimed
    steps and then more untimed steps until `settle_s` seconds of warm-up have
    passed: the GPU clock climbs over the first tens of milliseconds of load,
    and a short warm-up would time the climb instead of the steady state."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps  # ms per step


def measure(run, torch, steps, warmup, settle_s):
    """Time one workload; for decode pick the fastest split count."""
    if "splits" in run:
        best = None
        for n in run["splits"]:
            run["state"]["n"] = n
            ms = timed(torch, run["step"], steps, warmup, settle_s)
            if best is None or ms < best[0]:
                best = (ms, n)
        run["state"]["n"] = best[1]
        run["cfg"]["n_split"] = best[1]
        return best[0]
    return timed(torch, run["step"], steps, warmup, settle_s)


def sclk_path(torch):
    """The amdgpu pp_dpm_sclk file of cuda:0's PCI function, or None."""
    try:
        p = torch.cuda.get_device_properties(0)
        path = (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
                f"{p.pci_device_id:02x}.0/pp_dpm_sclk")
    except (AttributeError, RuntimeError):
        return None
    return path if os.path.exists(path) else None


def read_sclk(path):
    """Current shader clock in MHz: the pp_dpm_sclk line marked '*'."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0])
    except (OSError, ValueError, IndexError):
        pass
    return None


def sample_clock(torch, step, seconds):
    """Run `step` back to back for `seconds` while a second thread reads the
    shader clock every 20 ms (after the first 0.3 s).  Returns (median clock
    in MHz, ms per step over the same interval), or None when the driver file
    is not readable or sampling is off."""
    import threading
    path = sclk_path(torch)
    if path is None or seconds <= 0:
        return None
    samples, stop = [], threading.Event()

    def poll():
        t0 = time.perf_counter()
        while not stop.wait(0.02):
            if time.perf_counter() - t0 > 0.3:
                v = read_sclk(path)
                if v:
                    samples.append(v)
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    a.record(stream)
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            step()
        n += 16
        torch.cuda.synchronize()
    b.record(stream)
    torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    samples.sort()
    return samples[len(samples) // 2], a.elapsed_time(b) / n


def add_clock(rf, run, sampled):
    """Clock fields of a roofline entry: the median shader clock while the
    workload ran back to back, the rate over that interval, and for a
    matrix-bound kernel the peak scaled to that clock and the fraction of it."""
    if sampled is None:
        rf["sclk_mhz"] = None
        return
    sclk, ms = sampled
    rf["sclk_mhz"] = sclk
    rf["sustained_ms"] = round(ms, 5)
    if rf["bound"] == "mfma":
        p = rf["peak"] * sclk / PEAK_SCLK_MHZ
        rf["peak_at_sclk"] = round(p, 1)
        rf["frac_at_sclk"] = round(rate(run, ms) / p, 4)


def rate(run, ms):
    scale = 1e9 if run["unit"] == "TFLOP/s" else 1e6  # work per ms -> T or G per s
    return run["work"] / ms / scale


def roofline(run, ms, name):
    achieved = rate(run, ms)
    peak = PEAK_BF16_TFLOPS if run["bound"] == "mfma" else PEAK_HBM_GBS
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(name)
        if t and t.get("source_hash") == source_hash(KERNEL_SOURCES[name]):
            traffic = t["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    return {"bound": run["bound"], "achieved": round(achieved, 2), "peak": peak,
            "unit": run["unit"] if run["bound"] == "mfma" else "GB/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": run["kernel"], "launch_ms": round(ms, 5)}


def io_model(run, fa_mod):
    """HBM bytes of one forward call under the page's io_flash model
    (flash_forward's IO count in attention_kernels.py: Q read once, O and L
    written once, K and V read once per query tile, or once in total when they
    stay in cache), in bytes for bf16 tensors and an fp32 L, next to the
    measured traffic.  The query tile is the workgroup's rows."""
    cfg = run["cfg"]
    B, H, Nq, Nk, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"]
    rows = None
    try:
        from flashattention_online_softmax_fa_amd import stats
        rows = stats.load().tile(3, d, cfg["causal"])[0]
    except (ImportError, OSError):
        pass
    once = B * H * (2 * Nq * d * 2 + Nq * 4)         # Q read, O written, L written
    kv = B * H * 2 * Nk * d * 2                      # K and V read once
    out = {"kv_cached_bytes": float(once + kv), "query_tile_rows": rows,
           "kv_per_query_tile_bytes": None}
    if rows:
        out["kv_per_query_tile_bytes"] = float(once + kv * math.ceil(Nq / rows))
    return out


def _timed_oracle(fn):
    t0 = time.perf_counter()
    out = fn()
    return out, time.perf_counter() - t0


def _grow(n, total, dt, budget_s):
    """Sample size for the next try: aim at the budget, at least double."""
    return int(min(total, n * max(2.0, budget_s / max(dt, 1e-3))))


def oracle_leg(run, budget_s):
    """The fp64 oracle on a bounded sample of the same inputs: its speed on
    this host in the workload's unit (``cpu_baseline``) and the largest errors
    of the GPU result against it on that sample (``parity``).  The sample
    grows until one routine takes about a quarter of ``budget_s``."""
    import numpy as np
    import oracle
    from fa_inputs import to_f64_numpy
    threads = oracle.default_threads()
    x, out = run["x"], run["out"]
    B, H, Nq, d = x.q.shape
    Nk = x.k.shape[2]
    scale, causal = run["scale"], run["causal"]
    rng = np.random.default_rng(0)
    routines = {}

    def entry(name, work, dt, unit_scale):
        routines[name] = {"value": round(work / dt / unit_scale, 6), "seconds": round(dt, 3)}

    if run["cfg"]["workload"].startswith("prefill"):
        Q, K, V = (to_f64_numpy(t) for t in (x.q, x.k, x.v))
        total = B * H * Nq
        n = min(total, 64)
        while True:
            rows = np.sort(rng.choice(total, size=n, replace=False))
            (O1, L1), dt1 = _timed_oracle(lambda: oracle.dense_fwd(
                Q, K, V, scale, causal, rows=rows, nthreads=threads))
            if dt1 > budget_s / 4 or n == total:
                break
            n = _grow(n, total, dt1, budget_s)
        (O2, L2), dt2 = _timed_oracle(lambda: oracle.online_fwd(
            Q, K, V, scale, causal, block=64, rows=rows, nthreads=threads))
        vis = np.minimum(rows % Nq + 1, Nk) if causal else np.full(rows.shape, Nk)
        work = float(4.0 * d * vis.sum())
        entry("dense_definition", work, dt1, 1e12)
        entry("online_block64", work, dt2, 1e12)
        go = to_f64_numpy(out["o"]).reshape(-1, d)[rows]
        gl = to_f64_numpy(out["lse"]).reshape(-1)[rows]
        parity = {"sample": f"{rows.size} of {total} query rows",
                  "o_max_abs": float(np.abs(go - O1).max()), "o_tol": 2e-2,
                  "l_max_abs": float(np.abs(gl - L1).max()), "l_tol": 1e-3,
                  "online_vs_dense_max_abs": float(max(np.abs(O2 - O1).max(),
                                                       np.abs(L2 - L1).max()))}
        parity["ok"] = parity["o_max_abs"] <= 2e-2 and parity["l_max_abs"] <= 1e-3
        sample = f"{rows.size} of {total} query rows"
        unit = "TFLOP/s"
    elif run["cfg"]["workload"].startswith("bwd"):
        heads_all = rng.permutation(B * H)
        nh = min(B * H, threads)
        while True:
            heads = np.sort(heads_all[:nh])
            sl = lambda t: to_f64_numpy(t.reshape(B * H, -1, d)[heads])[None]
            Q, K, V, dO = (sl(t) for t in (x.q, x.k, x.v, x.do))
            g, dt = _timed_oracle(lambda: oracle.dense_bwd(Q, K, V, dO, scale, causal,
                                                           nthreads=threads))
            if dt > budget_s / 4 or nh == B * H:
                break
            nh = min(B * H, nh * 2)
        work = 10.0 * nh * Nq * Nk * d * (0.5 if causal else 1.0)
        entry("dense_jacobian_backward", work, dt, 1e12)
        parity = {"sample": f"{nh} of {B * H} heads, every element"}
        ok = True
        for key, t in (("dQ", out["dq"]), ("dK", out["dk"]), ("dV", out["dv"])):
            got = to_f64_numpy(t.reshape(B * H, -1, d)[heads])
            ref = g[key][0]
            rel = float(np.abs(got - ref).max() / np.abs(ref).max())
            parity[f"{key}_max_rel"] = rel
            ok = ok and rel <= 5e-2
        parity["tol_max_rel"] = 5e-2
        parity["ok"] = ok
        sample = f"{nh} of {B * H} heads (whole heads)"
        unit = "TFLOP/s"
    else:
        n_split = run["state"]["n"]
        total = B * H * Nq
        cap = min(total, 64)  # rows whose whole K/V cache (64 MiB fp64 each) comes to the host
        n = min(cap, 16)
        while True:
            heads = np.sort(rng.choice(B * H, size=n, replace=False))
            sl = lambda t: to_f64_numpy(t.reshape(B * H, -1, d)[heads])[None]
            Q, K, V = (sl(t) for t in (x.q, x.k, x.v))
            (O1, L1), dt1 = _timed_oracle(lambda: oracle.dense_fwd(Q, K, V, scale,
                                                                   nthreads=threads))
            if dt1 > budget_s / 4 or n == cap:
                break
            n = _grow(n, cap, dt1, budget_s)
        (O6, L6, _, _, _), dt6 = _timed_oracle(lambda: oracle.split_decode(
            Q, K, V, n_split, scale, nthreads=threads))
        per_row = 2.0 * (2 * Nk * d + 2 * d) + 4.0
        entry("dense_definition", per_row * n, dt1, 1e9)
        entry(f"split_merge_{n_split}", per_row * n, dt6, 1e9)
        go = to_f64_numpy(out["o"]).reshape(B * H, d)[heads]
        gl = to_f64_numpy(out["lse"]).reshape(B * H)[heads]
        parity = {"sample": f"{n} of {B * H} heads, n_split {n_split}",
                  "o_max_abs": float(np.abs(go - O1.reshape(n, d)).max()), "o_tol": 2e-2,
                  "l_max_abs": float(np.abs(gl - L1.reshape(n)).max()), "l_tol": 1e-3,
                  "split_vs_dense_max_abs": float(max(np.abs(O6 - O1.reshape(O6.shape)).max(),
                                                      np.abs(L6 - L1.reshape(L6.shape)).max()))}
        parity["ok"] = parity["o_max_abs"] <= 2e-2 and parity["l_max_abs"] <= 1e-3
        sample = f"{n} of {total} query rows (whole K/V cache of each)"
        unit = "GB/s"
    first = next(iter(routines.values()))
    cpu = {"value": first["value"], "unit": unit, "cores": threads, "kind": "oracle",
           "sample": sample + f"; {next(iter(routines))}, {first['seconds']:.2f} s",
           "routines": routines}
    return cpu, parity


def copy_calibration(torch):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    n = 1 << 28  # 256 Mi fp32 = 1 GiB read + 1 GiB written
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def sweep(torch, fa, steps, warmup, settle_s):
    """TFLOP/s of the forward and the causal backward over sequence lengths at
    a fixed number of tokens (one JSON line per shape)."""
    from fa_inputs import make_inputs
    for d in (64, 128):
        for n in (512, 1024, 2048, 4096, 8192, 16384):
            h = (1 << 18) // n
            x = make_inputs(1, h, n, n, d, "bf16", seed=n + d, device="cuda", backward=True)
            scale = 1.0 / math.sqrt(d)
            o = torch.empty_like(x.q)
            lse = torch.empty((1, h, n), dtype=torch.float32, device="cuda")
            ws = torch.empty(fa.fa_bwd_workspace_size(x.q.dtype, 1, h, n, d), dtype=torch.uint8,
                             device="cuda")
            g = [torch.empty_like(x.q) for _ in range(3)]
            for what, causal in (("fwd", False), ("fwd", True), ("bwd", True)):
                if what == "fwd":
                    def step():
                        fa.fa_fwd(x.q, x.k, x.v, o, lse, scale, causal)
                    flops = 4.0 * h * n * n * d
                else:
                    fa.fa_fwd(x.q, x.k, x.v, o, lse, scale, causal)
                    def step():
                        fa.fa_bwd(x.q, x.k, x.v, o, lse, x.do, g[0], g[1], g[2], ws, scale, causal)
                    flops = 10.0 * h * n * n * d
                flops *= 0.5 if causal else 1.0
                ms = timed(torch, step, steps, warmup, settle_s)
                tf = flops / ms / 1e9
                print(json.dumps({"pass": what, "B": 1, "H": h, "N": n, "d": d, "causal": causal,
                                  "ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                                  "frac": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
            del x, o, lse, ws, g
            torch.cuda.empty_cache()


def repeated(torch, step, steps, repeats):
    """Median and minimum ms per step over `repeats` further timed regions of
    `steps` steps each (the clock has settled by then)."""
    if repeats <= 0:
        return None
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(repeats):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / steps)
    ms.sort()
    return {"regions": repeats, "steps": steps, "median_ms": round(ms[len(ms) // 2], 5),
            "min_ms": round(ms[0], 5)}


def measure_workload(name, fa, torch, args, steps, warmup, n_split=None):
    """Time one workload and gather its roofline, oracle baseline and parity
    sample.  Returns (ms per step of the first timed region, entry dict)."""
    run = setup(name, fa, torch, n_split)
    ms = measure(run, torch, steps, warmup, args.settle)
    rf = roofline(run, ms, name)
    rep = repeated(torch, run["step"], steps, args.repeats)
    if rep:
        rf["repeats"] = rep
        rf["frac_median"] = round(run["work"] / rep["median_ms"] /
                                  (1e9 if run["unit"] == "TFLOP/s" else 1e6) / rf["peak"], 4)
    add_clock(rf, run, sample_clock(torch, run["step"], args.clock_s))
    if run["kernel"] == "fwd_bf16_kernel":
        rf["io_flash"] = io_model(run, fa)
    cfg = dict(run["cfg"])
    if "partial_bytes" in run:
        cfg["partial_state_bytes"] = run["partial_bytes"][run["state"]["n"]]
    if "extra" in run:
        cfg.update(run["extra"])
    entry = {"ms": round(ms, 5), "value": round(rate(run, ms), 3),
             "unit": run["unit"] if run["unit"] == "TFLOP/s" else "GB/s", "config": cfg,
             "roofline": rf}
    if not args.no_cpu:
        torch.cuda.synchronize()
        entry["cpu_baseline"], entry["parity"] = oracle_leg(run, args.cpu_budget)
    del run
    torch.cuda.empty_cache()
    return ms, entry


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported (every "
              "(batch, head) is independent, so B*H would split over GPUs with no communication)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import flashattention_online_softmax_fa_amd as fa
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.sweep:
        sweep(torch, fa, args.steps, args.warmup, args.settle)
        return
    ms, prim = measure_workload(args.workload, fa, torch, args, args.steps, args.warmup,
                                args.n_split)
    line = {
        "metric": "attention TFLOP/s and % of bf16 MFMA peak (fwd/bwd); decode GB/s % HBM peak",
        "value": prim["value"],
        "unit": prim["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "warmup_settle_s": args.settle,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": prim["config"],
        "roofline": prim["roofline"],
    }
    if not args.no_cpu:
        line["cpu_baseline"] = prim["cpu_baseline"]
        line["parity"] = prim["parity"]
    if not args.no_parts:
        parts = {}
        for name in ("prefill_causal_d128", "prefill_d64", "bwd_causal_d64", "decode_d128"):
            if name == args.workload:
                continue
            steps = max(3, args.steps // 2) if name == "decode_d128" else args.steps
            _, parts[name] = measure_workload(name, fa, torch, args, steps, min(args.warmup, 3))
        line["parts"] = parts
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
