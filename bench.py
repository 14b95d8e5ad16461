"""Throughput of one Hybrid Linear-Softmax Attention group on one MI355X.

A step is one hybrid group -- three gated linear layers and one gated softmax
anchor, all on their own seeded synthetic inputs resident in HBM -- run through
hybrid_attn_group_timed, which records HIP events between the layers on the
stream the kernels run on.  The headline workload is the 720p/5s latent shape
(B=1, H=24, N=75,600 tokens, d=128, bf16).

Prints ONE JSON line: tokens/s over the timed steps, the roofline of the
dominant kernel (the softmax anchor, MFMA-bound) measured live from those
events, and the float64 CPU oracle timed on a bounded sample of the same
workload.  Extra fields: per-layer milliseconds and the all-softmax group
(four anchors) for the hybrid-vs-softmax speedup.

--anchor lvsa runs the long-video form instead: the anchor is the block-sparse
kernel over the LVSA frame pattern of the workload's latent grid (a window of
frames plus periodic global frames), the three linear layers unchanged; the
extra field then compares against one dense anchor on the same inputs.

--mode train measures one training step of the group: the forward pass (three
linear layers, the anchor with its log-sum-exp) and the backward pass of all
four layers for a synthetic upstream gradient, inputs resident in HBM.

--mode stack measures --blocks attention blocks with block attention residuals
(AttnRes): the linear sub-layers of block k project a per-token softmax mixture
of the outputs of blocks 0 .. k-1 and the current stream.

--mode block measures the attention block around the group instead: a step is
hybrid_attn_block on a residual stream x [B, N, H*d] with synthetic weights
(four sub-layers, each Q/K/V/G projection, the layer, output projection and
residual); one extra untimed-for-value pass times each stage on its own.

Every line also carries `achievable` -- what this part sustains, measured after
the timed steps with the library's probe kernels (an MFMA loop and HBM read and
copy streams, include/ha_probe.h) -- with the roofline's rate against it as
`roofline.frac_of_achievable` (for an MFMA-bound kernel also against the MFMA
loop on random operands, `roofline.frac_of_achievable_random_operands`), and
`telemetry`: the GPU clock and socket power
sampled through amdsmi while the step repeats, untimed, for about 2.5 s after
the timed steps (the device refreshes those metrics about once a second; null
where that interface is unavailable).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
ANCHOR_SOURCES = ("hybrid_linear_softmax_amd/csrc/anchor.hip", "hybrid_linear_softmax_amd/csrc/ha_device.h")


def pmc_summary_path(label: str) -> str:
    return os.path.join(ROOT, "profiles", f"anchor_{label}_pmc.txt")


def anchor_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ANCHOR_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Telemetry:
    """GPU clock (MHz) and socket power (W) sampled through amdsmi on a host
    thread.  The device refreshes these metrics about once a second, so samples
    are told apart by the metrics' own timestamp and only fresh ones count.
    summary() is None when amdsmi cannot be used (no driver, no permission, or
    the device is not found)."""

    def __init__(self, device=0, period_s=0.1):
        self.period_s = period_s
        self.samples = []          # (metrics timestamp or None, clock MHz, power W)
        self.power_limit_w = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self._smi = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._handle = self._find_handle(amdsmi, device)
            limit = amdsmi.amdsmi_get_power_info(self._handle).get("power_limit")
            if isinstance(limit, (int, float)) and limit > 0:
                self.power_limit_w = round(limit / 1e6, 1) if limit > 1e5 else float(limit)   # reported in uW
        except Exception:
            self._handle = None

    @property
    def available(self):
        return self._handle is not None

    @staticmethod
    def _find_handle(amdsmi, device):
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) == 1:
            return handles[0]
        import torch
        bus = getattr(torch.cuda.get_device_properties(device), "pci_bus_id", None)
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)      # "dddd:bb:dd.f"
            if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                return h
        return None

    def _sample(self):
        smi, h = self._smi, self._handle
        num = lambda v: v if isinstance(v, (int, float)) else None   # noqa: E731
        try:
            m = smi.amdsmi_get_gpu_metrics_info(h)
            return (num(m.get("system_clock_counter")), num(m.get("current_gfxclk")),
                    num(m.get("current_socket_power")))
        except Exception:
            clk = smi.amdsmi_get_clock_info(h, smi.AmdSmiClkType.GFX).get("clk")
            return (None, num(clk), num(smi.amdsmi_get_power_info(h).get("current_socket_power")))

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._sample())
            except Exception:
                pass
            self._stop.wait(self.period_s)

    def __enter__(self):
        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self):
        s = summarize_telemetry(self.samples)
        if s is not None and self.power_limit_w is not None:
            s["power_limit_w"] = self.power_limit_w
        return s


def summarize_telemetry(samples):
    """Median / min / max over the fresh (timestamp, clock MHz, power W) samples:
    the first one (it may predate the window) and repeats of a timestamp are
    dropped.  None when nothing fresh was seen."""
    fresh, last = [], object()
    for i, (ts, clk, pw) in enumerate(samples):
        if i == 0 or (ts is not None and ts == last):
            last = ts
            continue
        last = ts
        fresh.append((clk, pw))
    out = {}
    for i, key in ((0, "gfx_clock_mhz"), (1, "socket_power_w")):
        vals = [f[i] for f in fresh if f[i] is not None]
        if vals:
            out[key] = {"median": round(statistics.median(vals), 1), "min": round(min(vals), 1),
                        "max": round(max(vals), 1)}
    if not out:
        return None
    out["fresh_samples"] = len(fresh)
    return out


def sample_telemetry(step, dev, seconds=2.5):
    """Clock and power while `step` repeats (untimed) for at least `seconds`
    and at least once, after the timed steps; None without amdsmi."""
    import torch

    tele = Telemetry(dev.index)
    if not tele.available:
        return None
    n = 0
    with tele:
        t_end = time.time() + seconds
        while n == 0 or time.time() < t_end:
            step()
            torch.cuda.synchronize()
            n += 1
    s = tele.summary()
    if s is not None:
        s["window"] = f"{n} untimed steps over >= {seconds} s after the timed steps"
    return s


def achievable_peaks(dev, reps=3):
    """What this part sustains, from the library's probe kernels: the bf16 MFMA
    loop (TFLOP/s) and HBM streams over 1 GiB buffers (GB/s, read + written);
    the best of `reps` event-timed runs (each of `launches` back-to-back calls,
    so that launch gaps do not count) after one warm-up each.  The MFMA loop is
    also run back to back for about 2 s and timed over the second half, once the
    power management has settled (`mfma_bf16_tflops_sustained`, with the clock
    and power of that half), and so is the loop on operands that change every
    instruction (`mfma_bf16_tflops_random_operands_sustained`): constant
    operands leave the matrix cores' inputs still, which keeps their power, and
    so the power limit's hold on the clock, below what real data costs."""
    import torch

    import hybrid_linear_softmax_amd as ha

    sink = torch.empty(1, dtype=torch.float32, device=dev)

    def best(fn, launches=1):
        fn()
        torch.cuda.synchronize()
        rates = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            work = sum(fn() for _ in range(launches))
            e1.record()
            torch.cuda.synchronize()
            rates.append(work / (e0.elapsed_time(e1) / 1e3))
        return max(rates)

    blocks, iters = 1024, 131072
    out = {"mfma_bf16_tflops": round(best(lambda: ha.probe_mfma(blocks, iters, sink)) / 1e12, 1)}
    half = 40
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    flops = sum(ha.probe_mfma(blocks, iters, sink) for _ in range(half))
    ev[1].record()
    torch.cuda.synchronize()
    tele = Telemetry(dev.index)
    with tele:
        for _ in range(half):
            ha.probe_mfma(blocks, iters, sink)
        ev[2].record()
        torch.cuda.synchronize()
    out["mfma_bf16_tflops_sustained"] = round(flops / (ev[1].elapsed_time(ev[2]) / 1e3) / 1e12, 1)
    out["mfma_sustained_telemetry"] = tele.summary()
    # the same on operands that change every instruction (random bf16): the
    # matrix cores' power, and with it the clock the power limit allows, depends
    # on their inputs toggling
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    flops = sum(ha.probe_mfma_data(blocks, iters, sink) for _ in range(half))
    ev[1].record()
    torch.cuda.synchronize()
    tele = Telemetry(dev.index)
    with tele:
        for _ in range(half):
            ha.probe_mfma_data(blocks, iters, sink)
        ev[2].record()
        torch.cuda.synchronize()
    out["mfma_bf16_tflops_random_operands_sustained"] = round(flops / (ev[1].elapsed_time(ev[2]) / 1e3) / 1e12, 1)
    out["mfma_random_operands_telemetry"] = tele.summary()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ov_iters = 20000
    def launch_ms(mode, wps):
        def one():
            ha.probe_overlap(mode, wps, cus, ov_iters, sink)
            return 1.0                          # one launch: best() then gives launches per second
        return 1e3 / best(one)

    times = {(mode, wps): launch_ms(mode, wps)
             for mode, wps in (("mfma", 1), ("valu", 1), ("both", 1), ("mfma", 2), ("valu", 2), ("both", 2),
                               ("split", 2))}
    out["issue_overlap"] = overlap_summary(times)
    out["issue_overlap"]["how"] = (f"overlap probe: {cus} blocks (one per CU) of 256 or 512 threads, {ov_iters} "
                                   "rounds; per round 4 MFMAs and/or the VALU work of 8 probabilities; best of 3")
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    out["hbm_read_gbs"] = round(best(lambda: ha.probe_read(src, sink), 10) / 1e9, 1)
    out["hbm_copy_gbs"] = round(best(lambda: ha.probe_copy(src, dst), 10) / 1e9, 1)
    out["hbm_copy_nontemporal_gbs"] = round(best(lambda: ha.probe_copy(src, dst, nontemporal=True), 10) / 1e9, 1)
    del src, dst
    out["how"] = (f"probe kernels: {blocks} x 256-thread blocks of 32x32x16 bf16 MFMA chains ({iters} rounds), "
                  f"best of 3 single launches, and sustained over launches {half + 1}-{2 * half} of {2 * half} "
                  "back to back; 1 GiB read, copy and non-temporal copy, 10 back-to-back launches, best of 3; "
                  "each after a warm-up")
    return out


def overlap_summary(times):
    """Issue overlap of VALU and MFMA work on one SIMD from the overlap probe's
    launch times (ms) keyed (mode, waves per SIMD).  valu_hidden: the share of
    the VALU-only time that a mixed run hides under the MFMAs, (t_m + t_v - t_mixed)
    / t_v -- 1 with full overlap, 0 when the two run one after the other.  The
    split run puts one MFMA wave and one VALU wave on each SIMD, so it is read
    against the one-wave-per-SIMD times."""
    out = {}
    for wps in (1, 2):
        tm, tv, tb = times[("mfma", wps)], times[("valu", wps)], times[("both", wps)]
        out[f"waves_per_simd_{wps}"] = {"mfma_ms": round(tm, 4), "valu_ms": round(tv, 4), "both_ms": round(tb, 4),
                                        "valu_hidden": round((tm + tv - tb) / tv, 3)}
    tm1, tv1, ts = times[("mfma", 1)], times[("valu", 1)], times[("split", 2)]
    out["split_ms"] = round(ts, 4)
    out["split_valu_hidden"] = round((tm1 + tv1 - ts) / tv1, 3)
    return out


def annotate(line, peaks, telemetry):
    """Add the achievable peaks, the roofline's fraction of them and the telemetry
    to a bench line (in place)."""
    line["achievable"] = peaks
    line["telemetry"] = telemetry
    r = line.get("roofline")
    if peaks and r:
        if r.get("bound") == "mfma":
            ach = peaks.get("mfma_bf16_tflops_sustained") or peaks.get("mfma_bf16_tflops")
        else:
            ach = max(peaks.get("hbm_read_gbs", 0), peaks.get("hbm_copy_gbs", 0),
                      peaks.get("hbm_copy_nontemporal_gbs", 0)) or None
        if ach:
            r["achievable_peak"] = ach
            r["frac_of_achievable"] = round(r["achieved"] / ach, 4)
        rnd = peaks.get("mfma_bf16_tflops_random_operands_sustained") if r.get("bound") == "mfma" else None
        if rnd:
            r["achievable_peak_random_operands"] = rnd
            r["frac_of_achievable_random_operands"] = round(r["achieved"] / rnd, 4)
    return line


def measured_traffic(label: str):
    """HBM bytes per anchor launch from the committed rocprofv3 PMC summary,
    or None when it is missing, for another workload, or the kernel has changed
    since the counters were taken."""
    path = pmc_summary_path(label)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("workload") != label or vals.get("anchor_source_sha256") != anchor_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, x, rows_sampled: int, pattern=None, lin_heads: int = 4):
    """The oracle as it stands, timed on this host on a sample of the workload:
    the full linear layer of `lin_heads` (b, h) heads, and `rows_sampled` query
    rows of the softmax anchor of one head (rows are independent, each costs the
    same), extrapolated to one whole group.  With a block-sparse pattern the rows
    are whole query blocks and the extrapolation is by query-key pairs."""
    import numpy as np

    import oracle
    from workloads import to_f64

    threads = _blas_threads()
    lin_heads = max(1, min(lin_heads, w.H))
    t_lin = 0.0
    for hh in range(lin_heads):
        q, k, v, g = (to_f64(x[n][0, 0, hh]) for n in "QKVG")
        t0 = time.perf_counter()
        oracle.linear_attention(q, k, v, g)
        t_lin += time.perf_counter() - t0
    t_lin /= lin_heads
    q, k, v, g = (to_f64(x[n][3, 0, 0]) for n in "QKVG")
    if pattern is None:
        rows = np.random.default_rng(0).choice(w.N, size=min(rows_sampled, w.N), replace=False)
        t0 = time.perf_counter()
        oracle.softmax_attention(q, k, v, g, rows=rows)
        t_rows = time.perf_counter() - t0
        scale = w.N / rows.size
    else:
        offsets, indices = pattern
        nqb = len(offsets) - 1
        qbs = np.linspace(0, nqb - 1, num=max(1, min(nqb, rows_sampled // 256))).astype(np.int64)
        rows = np.concatenate([np.arange(qb * 256, min(w.N, (qb + 1) * 256)) for qb in np.unique(qbs)])
        t0 = time.perf_counter()
        oracle.softmax_attention_blocksparse(q, k, v, g, offsets, indices, rows=rows)
        t_rows = time.perf_counter() - t0
        pairs = pattern_pairs(w.N, offsets, indices)
        sampled = sum(pattern_pairs(w.N, offsets, indices, only=int(qb)) for qb in np.unique(qbs))
        scale = pairs / sampled
    heads = w.B * w.H
    t_group = 3 * heads * t_lin + heads * scale * t_rows
    return {
        "value": w.B * w.N / t_group,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "host": host_info(),
        "sample": (f"float64 numpy oracle: full linear layer of {lin_heads} of {heads} heads "
                   f"({t_lin:.2f} s each) and "
                   f"{rows.size} of {w.N} {'block-sparse ' if pattern else ''}softmax query rows of 1 head "
                   f"({t_rows:.2f} s), extrapolated "
                   f"to 3 linear + 1 softmax layers over {heads} heads ({t_group:.0f} s per group)"),
    }


def linear_kernel_split(B, H, N, d, r1_ms, reduce_ms, apply_ms):
    """Per-kernel figures of one linear layer from in-stream HIP events around
    each of its kernels (hybrid_attn_linear_timed): R1 pass 1 (the state
    reduction over tokens), pass 2 (the fixed-order sum of its partials) and R2
    (the apply).  Algorithmic bytes and flops per (token, head): R1 reads K and
    V (4d bytes) for 2d^2 + d flops, R2 reads Q and G and writes O (6d bytes)
    for 2d^2 + 6d flops (bf16 I/O)."""
    th = B * H * N
    r1_bytes, r2_bytes = th * 4 * d, th * 6 * d
    r1_flop, r2_flop = th * (2 * d * d + d), th * (2 * d * d + 6 * d)
    gbs = lambda b, ms: b / (max(ms, 1e-9) / 1e3) / 1e9   # noqa: E731
    tfs = lambda f, ms: f / (max(ms, 1e-9) / 1e3) / 1e12  # noqa: E731
    return {
        "r1_state_ms": round(r1_ms, 4),
        "r1_hbm_gbs": round(gbs(r1_bytes, r1_ms), 1),
        "r1_hbm_frac": round(gbs(r1_bytes, r1_ms) / HBM_PEAK_GBS, 4),
        "r1_mfma_frac": round(tfs(r1_flop, r1_ms) / MFMA_BF16_PEAK_TFLOPS, 4),
        "r1_reduce_ms": round(reduce_ms, 4),
        "r2_apply_ms": round(apply_ms, 4),
        "r2_hbm_gbs": round(gbs(r2_bytes, apply_ms), 1),
        "r2_hbm_frac": round(gbs(r2_bytes, apply_ms) / HBM_PEAK_GBS, 4),
        "r2_mfma_frac": round(tfs(r2_flop, apply_ms) / MFMA_BF16_PEAK_TFLOPS, 4),
        "how": "HIP events recorded in the stream between the layer's three kernels, mean of 10 calls",
    }


def pattern_pairs(N, offsets, indices, only=None):
    """Query-key pairs a block pattern keeps (valid keys only, set semantics)."""
    nkb = -(-N // 64)
    total = 0
    for qb in (range(len(offsets) - 1) if only is None else [only]):
        rows = min(N, (qb + 1) * 256) - qb * 256
        blocks = {int(b) for b in indices[offsets[qb]:offsets[qb + 1]] if 0 <= b < nkb}
        total += rows * sum(min(64, N - 64 * b) for b in blocks)
    return total


def _blas_threads():
    import numpy  # noqa: F401  (loads the BLAS library threadpoolctl inspects)
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"], default=1)


def host_info():
    """What the CPU baseline ran on: the CPU model (/proc/cpuinfo), the cores
    this process may use (its affinity mask), and the BLAS library numpy calls
    with its thread count (the threads the oracle's products actually use)."""
    import platform

    import numpy  # noqa: F401
    from threadpoolctl import threadpool_info

    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    return {
        "cpu_model": model,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "blas": ", ".join(sorted({f"{p.get('internal_api')} {p.get('version') or ''} ({p.get('prefix')})".strip()
                                  for p in blas})) or "none found",
        "blas_threads": _blas_threads(),
    }


def single_thread_baselines(tiny=None, lin=None, lin_heads: int = 2):
    """The oracle on one thread: the whole tiny group (fp32 workload, 4 layers)
    and the 480p linear layer (`lin_heads` whole heads timed, extrapolated to
    all heads: each head costs the same).  `tiny` / `lin` override the
    workloads (for tests)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import get, layer_inputs_host, to_f64

    tiny = tiny or get("tiny")
    lin = lin or get("480p")
    res = {}
    with threadpool_limits(limits=1, user_api="blas"):
        layers = [layer_inputs_host(tiny, l) for l in range(4)]
        x = {k: np.stack([to_f64(L[k]) for L in layers]) for k in "QKVG"}
        t0 = time.perf_counter()
        oracle.group(x["Q"], x["K"], x["V"], x["G"])
        t = time.perf_counter() - t0
        res["tiny_group"] = {"seconds": round(t, 4), "tokens_per_s": round(tiny.B * tiny.N / t, 1),
                             "shape": f"B={tiny.B} H={tiny.H} N={tiny.N} d={tiny.d} fp32, 4 layers"}
        heads = max(1, min(lin_heads, lin.H))
        L = layer_inputs_host(lin, 0, B=1, H=heads)
        q, k, v, g = (to_f64(L[n][0]) for n in "QKVG")
        t0 = time.perf_counter()
        for hh in range(heads):
            oracle.linear_attention(q[hh], k[hh], v[hh], g[hh])
        t_head = (time.perf_counter() - t0) / heads
        t_layer = t_head * lin.B * lin.H
        res["linear_layer_480p"] = {"seconds": round(t_layer, 3), "tokens_per_s": round(lin.B * lin.N / t_layer, 1),
                                    "sample": f"{heads} of {lin.B * lin.H} heads timed ({t_head:.3f} s each), "
                                              "extrapolated to the layer"}
    return res


def _block_oracle_seconds(w, blk, rows_sampled: int):
    """Oracle seconds for one block, extrapolated from a sample: the two
    projections of `rows_sampled` token rows (rows are independent), the linear
    layer of one head and `rows_sampled` anchor rows of one head.  Returns
    (seconds per block, projection s, linear s, anchor-rows s, rows)."""
    import numpy as np

    import oracle
    from workloads import layer_inputs_host, to_f64

    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(w.N, size=min(rows_sampled, w.N), replace=False))
    x = to_f64(blk["x"][:1, rows])
    Wi, Wo = to_f64(blk["W_in"][0]), to_f64(blk["W_out"][0])
    t0 = time.perf_counter()
    Q, K, V, G = oracle.project_in(x, Wi, w.H)
    oracle.project_out(Q, Wo, x)
    t_proj = time.perf_counter() - t0
    # attention on the projected rows of head 0, scaled to the full sequence
    att = layer_inputs_host(w, 3, B=1, H=1, N=w.N)
    q, k, v, g = (to_f64(att[n][0, 0]) for n in "QKVG")
    t0 = time.perf_counter()
    oracle.linear_attention(q, k, v, g)
    t_lin = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.softmax_attention(q, k, v, g, rows=rows)
    t_rows = time.perf_counter() - t0
    heads = w.B * w.H
    t_block = 4 * t_proj * (w.B * w.N / rows.size) + 3 * heads * t_lin + heads * (w.N / rows.size) * t_rows
    return t_block, t_proj, t_lin, t_rows, rows


def block_cpu_baseline(w, blk, rows_sampled: int):
    """The oracle timed on a sample of one block (see _block_oracle_seconds),
    extrapolated to the block."""
    t_block, t_proj, t_lin, t_rows, rows = _block_oracle_seconds(w, blk, rows_sampled)
    heads = w.B * w.H
    return {
        "value": w.B * w.N / t_block,
        "unit": "tokens/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: projections of {rows.size} token rows ({t_proj:.2f} s), the linear "
                   f"layer of 1 of {heads} heads ({t_lin:.2f} s) and {rows.size} anchor rows of 1 head "
                   f"({t_rows:.2f} s), extrapolated to 4 sub-layers ({t_block:.0f} s per block)"),
    }


def train_cpu_baseline(w, x, dO4, rows_sampled: int, lin_heads: int = 2):
    """The oracle timed on a sample of one training step: the linear layer's
    forward and backward on `lin_heads` whole heads, and the anchor's forward
    and backward over `rows_sampled` query rows of one head -- the oracle's
    anchor backward walks query rows against all keys, so each row's share of
    dQ, dK, dV and dG costs the same -- extrapolated to the step (forward and
    backward of 3 linear layers and the anchor over every head)."""
    import numpy as np

    import oracle
    from workloads import to_f64

    lin_heads = max(1, min(lin_heads, w.H))
    t_lin = 0.0
    for hh in range(lin_heads):
        q, k, v, g = (to_f64(x[n][0, 0, hh]) for n in "QKVG")
        do = to_f64(dO4[0, 0, hh])
        t0 = time.perf_counter()
        oracle.linear_attention(q, k, v, g)
        oracle.linear_attention_backward(q, k, v, g, do)
        t_lin += time.perf_counter() - t0
    t_lin /= lin_heads
    q, k, v, g = (to_f64(x[n][3, 0, 0]) for n in "QKVG")
    do = to_f64(dO4[3, 0, 0])
    rows = np.sort(np.random.default_rng(0).choice(w.N, size=min(rows_sampled, w.N), replace=False))
    t0 = time.perf_counter()
    oracle.softmax_attention(q, k, v, g, rows=rows)
    oracle.softmax_attention_backward(q[rows], k, v, g[rows], do[rows])
    t_rows = time.perf_counter() - t0
    heads = w.B * w.H
    t_step = 3 * heads * t_lin + heads * (w.N / rows.size) * t_rows
    return {
        "value": w.B * w.N / t_step,
        "unit": "tokens/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: linear forward + backward of {lin_heads} of {heads} heads "
                   f"({t_lin:.2f} s each) and anchor forward + backward over {rows.size} of {w.N} query rows "
                   f"of 1 head ({t_rows:.2f} s), extrapolated to 3 linear + 1 softmax layers over {heads} heads "
                   f"({t_step:.0f} s per training step)"),
    }


def stack_cpu_baseline(w, nb, blk, summaries, w_route, rows_sampled: int):
    """The oracle timed on a sample of the AttnRes stack: one block as in
    block_cpu_baseline, and the routing mixture of each block (k summaries and
    the stream, three linear sub-layers each) on `rows_sampled` token rows,
    extrapolated to `nb` blocks."""
    import numpy as np

    import oracle
    from workloads import to_f64

    t_block, _, _, _, rows = _block_oracle_seconds(w, blk, rows_sampled)
    xr = to_f64(blk["x"][:1, rows])
    t_mix = 0.0
    for k in range(nb):
        cand = np.stack([to_f64(summaries[j][:1, rows]) for j in range(k)] + [xr])
        wr = to_f64(w_route[k, 0])
        t0 = time.perf_counter()
        oracle.attnres_mix(cand, wr)
        t_mix += 3 * (time.perf_counter() - t0) * (w.B * w.N / rows.size)
    t_stack = nb * t_block + t_mix
    return {
        "value": w.B * w.N / t_stack,
        "unit": "tokens/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: one block sampled as in the block mode ({t_block:.0f} s extrapolated) "
                   f"and the routing mixtures of {nb} blocks on {rows.size} token rows ({t_mix:.1f} s "
                   f"extrapolated), {t_stack:.0f} s per stack of {nb} blocks"),
    }


def run_block(args, w):
    import torch

    import hybrid_linear_softmax_amd as ha
    from workloads import block_inputs_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    C = w.H * w.d
    M = w.B * w.N
    print(f"[bench] block {w.name}: B={w.B} N={w.N} C={C} (H={w.H} x d={w.d}); generating inputs",
          file=sys.stderr, flush=True)
    blk = block_inputs_device(w, dev)
    x, Wi, Wo = blk["x"], blk["W_in"], blk["W_out"]
    x_out = torch.empty_like(x)
    ws = torch.empty(ha.block_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        ha.hybrid_attn_block(x, Wi, Wo, w.H, x_out=x_out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} block steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-stage breakdown: the same kernels called one stage at a time
    Q, K, V, G = (torch.empty((w.B, w.H, w.N, w.d), dtype=x.dtype, device=dev) for _ in range(4))
    O = torch.empty_like(Q)
    lin_ws = torch.empty(ha.workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    y = x.clone()
    stage = {"proj_in": 0.0, "linear": 0.0, "softmax": 0.0, "proj_out": 0.0}
    reps = max(1, min(args.steps, 3))
    for _ in range(reps):
        y.copy_(x)
        for l, kind in enumerate(ha.hybrid_attn_group_schedule()):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
            ha.hybrid_attn_proj_in(y, Wi[l], w.H, Q, K, V, G)
            ev[1].record()
            if kind == "linear":
                ha.hybrid_attn_linear(Q, K, V, G, O, workspace=lin_ws)
            else:
                ha.hybrid_attn_softmax(Q, K, V, G, O)
            ev[2].record()
            ha.hybrid_attn_proj_out(O, Wo[l], y, x_out=y)
            ev[3].record()
            torch.cuda.synchronize()
            stage["proj_in"] += ev[0].elapsed_time(ev[1]) / reps / 4
            stage[kind] += ev[1].elapsed_time(ev[2]) / reps / (3 if kind == "linear" else 1)
            stage["proj_out"] += ev[2].elapsed_time(ev[3]) / reps / 4
    fl_in, fl_out = 2.0 * M * C * 4 * C, 2.0 * M * C * C
    anchor_flop = 4.0 * w.B * w.H * w.N * w.N * w.d
    anchor_tf = anchor_flop / (stage["softmax"] / 1e3) / 1e12
    roofline = {
        "kernel": "anchor_bf16 (gated softmax anchor, the block's dominant kernel)",
        "bound": "mfma",
        "achieved": round(anchor_tf, 1),
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(anchor_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic": None,
    }
    gemm = {
        "proj_in_ms": round(stage["proj_in"], 3),
        "proj_in_tflops": round(fl_in / (stage["proj_in"] / 1e3) / 1e12, 1),
        "proj_out_ms": round(stage["proj_out"], 3),
        "proj_out_tflops": round(fl_out / (stage["proj_out"] / 1e3) / 1e12, 1),
    }
    gemm["proj_in_frac"] = round(gemm["proj_in_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    gemm["proj_out_frac"] = round(gemm["proj_out_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = block_cpu_baseline(w, blk, args.cpu_rows or 16384)
    line = {
        "metric": "attention block (4 projected sub-layers around the 3:1 group) tokens/s",
        "value": round(M / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}_block", "B": w.B, "N": w.N, "H": w.H, "d": w.d, "C": C,
                   "sublayers": "linear,linear,linear,softmax", "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stage_ms": {k: round(v, 3) for k, v in stage.items()},
        "projections": gemm,
    }
    tele = None if args.no_telemetry else sample_telemetry(step, dev)
    peaks = None if args.no_peaks else achievable_peaks(dev)
    if peaks:
        rnd = peaks.get("mfma_bf16_tflops_random_operands_sustained")
        for k in ("proj_in", "proj_out"):
            gemm[f"{k}_frac_of_achievable"] = round(gemm[f"{k}_tflops"] / peaks["mfma_bf16_tflops"], 4)
            if rnd:
                gemm[f"{k}_frac_of_random_operand_mfma"] = round(gemm[f"{k}_tflops"] / rnd, 4)
    print(json.dumps(annotate(line, peaks, tele)), flush=True)


def run_train(args, w):
    import torch

    import hybrid_linear_softmax_amd as ha
    from workloads import group_inputs_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] train step {w.name}: B={w.B} H={w.H} N={w.N} d={w.d}; generating inputs", file=sys.stderr,
          flush=True)
    x = group_inputs_device(w, dev)
    gen = torch.Generator(device=dev).manual_seed(123)
    dO4 = torch.randn(x["Q"].shape, generator=gen, device=dev, dtype=torch.float32).to(x["Q"].dtype)
    O4 = torch.empty_like(x["Q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    grads = [[torch.empty_like(x["Q"][0]) for _ in range(4)] for _ in range(4)]
    ws_f = torch.empty(ha.workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    ws_l = torch.empty(ha.linear_backward_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(ha.softmax_backward_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    kinds = ha.hybrid_attn_group_schedule()
    evs = {}

    def step(timed=False):
        def mark(name):
            if timed:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                evs.setdefault(name, []).append(e)
        mark("start")
        for l, kind in enumerate(kinds):
            a = [x[k][l] for k in "QKVG"]
            if kind == "linear":
                ha.hybrid_attn_linear(*a, O4[l], workspace=ws_f)
            else:
                ha.hybrid_attn_softmax_lse(*a, O4[l], lse)
        mark("fwd")
        for l, kind in enumerate(kinds):
            a = [x[k][l] for k in "QKVG"]
            if kind == "linear":
                ha.hybrid_attn_linear_backward(*a, dO4[l], grads=grads[l], workspace=ws_l)
                mark(f"bwd_linear{l}")
            else:
                ha.hybrid_attn_softmax_backward(*a, O4[l], dO4[l], lse, grads=grads[l], workspace=ws_s)
                mark("bwd_softmax")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} training steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(timed=True)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    n = args.steps
    fwd_ms = sum(evs["start"][i].elapsed_time(evs["fwd"][i]) for i in range(n)) / n
    prev = "fwd"
    bwd = {}
    for l, kind in enumerate(kinds):
        name = f"bwd_linear{l}" if kind == "linear" else "bwd_softmax"
        bwd[name] = sum(evs[prev][i].elapsed_time(evs[name][i]) for i in range(n)) / n
        prev = name
    BH = w.B * w.H
    flop = 14.0 * BH * w.N * w.N * w.d      # 7 products of 2 N^2 d: S, dP in each kernel, dQ, dK, dV
    tf = flop / (bwd["bwd_softmax"] / 1e3) / 1e12
    roofline = {
        "kernel": "anchor backward (sm_bwd_dq_bf16 + sm_bwd_dkv_bf16, the step's dominant work)",
        "bound": "mfma",
        "achieved": round(tf, 1),
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic": None,
    }
    lin_bwd_ms = sum(v for k, v in bwd.items() if k.startswith("bwd_linear")) / 3
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = train_cpu_baseline(w, x, dO4, args.cpu_rows or 16384)
    line = {
        "metric": "hybrid 3:1 group training step (forward + backward) tokens/s",
        "value": round(w.B * w.N / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}_train", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "layers": "linear,linear,linear,softmax", "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "forward_ms": round(fwd_ms, 3),
        "backward_ms": {k: round(v, 3) for k, v in bwd.items()},
        "linear_backward_hbm_gbs_min_bytes": round(9 * BH * w.N * w.d * 2 / (lin_bwd_ms / 1e3) / 1e9, 1),
    }
    tele = None if args.no_telemetry else sample_telemetry(step, dev)
    peaks = None if args.no_peaks else achievable_peaks(dev)
    print(json.dumps(annotate(line, peaks, tele)), flush=True)


def run_stack(args, w):
    import dataclasses

    import torch

    import hybrid_linear_softmax_amd as ha
    from workloads import block_inputs_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    C = w.H * w.d
    M = w.B * w.N
    nb = args.blocks
    print(f"[bench] AttnRes stack {w.name}: {nb} blocks, B={w.B} N={w.N} C={C}; generating inputs",
          file=sys.stderr, flush=True)
    ins = [block_inputs_device(dataclasses.replace(w, seed=k), dev) for k in range(nb)]
    x = ins[0]["x"]
    W_in = [t["W_in"] for t in ins]
    W_out = [t["W_out"] for t in ins]
    for t in ins[1:]:
        del t["x"]
    gen = torch.Generator(device=dev).manual_seed(5)
    w_route = torch.randn((nb, 4, C), generator=gen, device=dev, dtype=torch.float32)
    summaries = torch.empty((nb, w.B, w.N, C), dtype=x.dtype, device=dev)
    ws = torch.empty(ha.block_routed_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        for k in range(nb):
            ha.hybrid_attn_block_routed(x if k == 0 else summaries[k - 1], summaries[:k] if k else None,
                                        w_route[k], W_in[k], W_out[k], w.H, x_out=summaries[k], workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} stack steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # the routing alone, as block nb-1 runs it (nb - 1 summaries + the stream)
    h = torch.empty_like(x)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    S = summaries[:nb - 1] if nb > 1 else None
    ha.hybrid_attn_attnres_mix(S, summaries[nb - 1], w_route[0, 0], h)
    e0.record()
    for _ in range(5):
        ha.hybrid_attn_attnres_mix(S, summaries[nb - 1], w_route[0, 0], h)
    e1.record()
    torch.cuda.synchronize()
    mix_ms = e0.elapsed_time(e1) / 5
    mix_bytes = (nb + 1) * M * C * 2   # nb candidates read once, h written
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = stack_cpu_baseline(w, nb, {"x": x, "W_in": W_in[0], "W_out": W_out[0]}, summaries, w_route,
                                 args.cpu_rows or 16384)
    line = {
        "metric": "stack of AttnRes-routed attention blocks tokens/s",
        "value": round(M / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}_attnres_stack", "blocks": nb, "B": w.B, "N": w.N, "H": w.H, "d": w.d,
                   "parallelism": "single-gpu"},
        "roofline": {
            "kernel": f"attnres_mix_bf16_1pass ({nb} candidates, single pass)",
            "bound": "hbm",
            "achieved": round(mix_bytes / (mix_ms / 1e3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(mix_bytes / (mix_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
        "cpu_baseline": cpu,
        "block_ms": round(ms_per_step / nb, 3),
        "mix_ms": round(mix_ms, 3),
    }
    tele = None if args.no_telemetry else sample_telemetry(step, dev)
    peaks = None if args.no_peaks else achievable_peaks(dev)
    print(json.dumps(annotate(line, peaks, tele)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="720p5s", help="workload name (default: the 720p/5s shape)")
    ap.add_argument("--allsoftmax-steps", type=int, default=3,
                    help="steps of the all-softmax group (4 anchors) for the speedup ratio; 0 skips")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="query or token rows the oracle baseline samples (default: 32768 for the group, "
                         "16384 for --mode train, block and stack: about 5-15 s of host work each)")
    ap.add_argument("--anchor", choices=("dense", "lvsa"), default="dense",
                    help="dense softmax anchor (default) or the block-sparse LVSA anchor")
    ap.add_argument("--mode", choices=("group", "block", "train", "stack"), default="group",
                    help="the hybrid group (default), the attention block around it, one training "
                         "step of the group (forward and backward), or a stack of AttnRes-routed blocks")
    ap.add_argument("--blocks", type=int, default=4, help="blocks in --mode stack")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the clock and power sampling (about 2.5 s of untimed steps after the timed ones)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (MFMA loop, HBM streams) after the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(every (b, h) is independent; see the multi-GPU design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import hybrid_linear_softmax_amd as ha
    from workloads import get, group_inputs_device

    w = get(args.config)
    if w.dtype != "bf16":
        raise SystemExit("bench workloads are the bf16 shapes; the fp32 tiny shape is a test case")
    if args.mode == "block":
        return run_block(args, w)
    if args.mode == "train":
        return run_train(args, w)
    if args.mode == "stack":
        return run_stack(args, w)
    sparse = args.anchor == "lvsa"
    label = f"{w.name}_lvsa" if sparse else w.name
    pattern = None
    if sparse:
        from workloads.sparsity import lvsa_pattern, pattern_density
        pattern = lvsa_pattern(w.frames, w.grid[0] * w.grid[1])
        print(f"[bench] LVSA pattern: {pattern[1].size} key blocks, density "
              f"{pattern_density(pattern[0], w.N):.4f}", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}; generating inputs", file=sys.stderr,
          flush=True)
    x = group_inputs_device(w, dev)
    O4 = torch.empty_like(x["Q"])
    ws = torch.empty(ha.workspace_bytes(w.B, w.H, w.N, w.d, torch.bfloat16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(max(args.steps, 1))]

    if not sparse:
        def step(i=None):
            ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"], O4, workspace=ws,
                                 events=None if i is None else evs[i])
    else:
        off_d = torch.from_numpy(pattern[0]).to(dev)
        idx_d = torch.from_numpy(pattern[1]).to(dev)

        def step(i=None):
            # the same group with the anchor swapped for the block-sparse kernel;
            # events are recorded on the stream the kernels run on
            e = None if i is None else evs[i]
            if e is not None:
                e[0].record()
            for l in range(3):
                ha.hybrid_attn_linear(x["Q"][l], x["K"][l], x["V"][l], x["G"][l], O4[l], workspace=ws)
                if e is not None:
                    e[l + 1].record()
            ha.hybrid_attn_softmax_blocksparse(x["Q"][3], x["K"][3], x["V"][3], x["G"][3], off_d, idx_d, O=O4[3])
            if e is not None:
                e[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    layer_ms = [sum(evs[i][l].elapsed_time(evs[i][l + 1]) for i in range(args.steps)) / args.steps
                for l in range(4)]
    tokens_per_s = w.B * w.N * args.steps / (total_ms / 1e3)

    BH = w.B * w.H
    anchor_ms = layer_ms[3]
    pairs = pattern_pairs(w.N, *pattern) if sparse else w.N * w.N
    anchor_flop = 4.0 * BH * pairs * w.d              # QK^T and PV, 2 flops per multiply-add
    achieved = anchor_flop / (anchor_ms / 1e3) / 1e12
    roofline = {
        "kernel": ("anchor_bf16<SPARSE> (block-sparse gated softmax anchor)" if sparse
                   else "anchor_bf16 (gated softmax anchor)"),
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic": measured_traffic(label),
    }
    lin_ms = sum(layer_ms[:3]) / 3
    lin_bytes = BH * w.N * w.d * 2 * 5                 # Q, K, V, G read + O written, bf16
    extra = {
        "layers_ms": [round(t, 3) for t in layer_ms],
        "linear_layer_hbm_gbs": round(lin_bytes / (lin_ms / 1e3) / 1e9, 1),
    }

    # per-kernel split of one linear layer (untimed for value): events in the
    # stream between its three kernels
    lin_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(10)]
    ha.hybrid_attn_linear(x["Q"][0], x["K"][0], x["V"][0], x["G"][0], O4[0], workspace=ws)
    for e in lin_evs:
        ha.hybrid_attn_linear(x["Q"][0], x["K"][0], x["V"][0], x["G"][0], O4[0], workspace=ws, events=e)
    torch.cuda.synchronize()
    seg = [sum(e[i].elapsed_time(e[i + 1]) for e in lin_evs) / len(lin_evs) for i in range(3)]
    extra["linear_kernels"] = linear_kernel_split(w.B, w.H, w.N, w.d, *seg)
    if sparse:
        extra["pattern_density"] = round(pairs / (w.N * w.N), 5)
        extra["anchor_pairs"] = pairs
    if sparse and args.allsoftmax_steps > 0:
        # one dense anchor on the same inputs: what the pattern saves
        ha.hybrid_attn_softmax(x["Q"][3], x["K"][3], x["V"][3], x["G"][3], O4[3])
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record()
        ha.hybrid_attn_softmax(x["Q"][3], x["K"][3], x["V"][3], x["G"][3], O4[3])
        a1.record()
        torch.cuda.synchronize()
        extra["dense_anchor_ms"] = round(a0.elapsed_time(a1), 3)
        extra["sparse_anchor_speedup_vs_dense"] = round(a0.elapsed_time(a1) / anchor_ms, 3)
    elif args.allsoftmax_steps > 0:
        def soft4():
            for l in range(4):
                ha.hybrid_attn_softmax(x["Q"][l], x["K"][l], x["V"][l], x["G"][l], O4[l])
        soft4()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.allsoftmax_steps):
            soft4()
        a1.record()
        torch.cuda.synchronize()
        soft_ms = a0.elapsed_time(a1) / args.allsoftmax_steps
        extra["allsoftmax_group_ms"] = round(soft_ms, 3)
        extra["hybrid_speedup_vs_allsoftmax"] = round(soft_ms / ms_per_step, 3)

    tele = None if args.no_telemetry else sample_telemetry(step, dev)
    peaks = None if args.no_peaks else achievable_peaks(dev)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, x, args.cpu_rows or 32768, pattern)
        cpu["single_thread"] = single_thread_baselines()

    line = {
        "metric": ("hybrid 3:1 attention group (block-sparse LVSA anchor) tokens/s; % of bf16 MFMA peak"
                   if sparse else "hybrid 3:1 attention group tokens/s at 720p/5s shape; % of bf16 MFMA/HBM peak"),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "layers": "linear,linear,linear," + ("softmax_blocksparse_lvsa" if sparse else "softmax"),
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(annotate(line, peaks, tele)), flush=True)


if __name__ == "__main__":
    main()
