"""Benchmark: ms per denoising step over a whole sparse-attention schedule.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one denoising step of the workload's schedule, run through the
library's schedule driver (C ABI): dense warm-up steps, the pattern
selection step, then sparse steps reusing the pattern (refreshes where the
schedule has them).  K steps form one schedule: with K equal to the
workload's step count it is exactly that schedule; otherwise the schedule is
rescaled to K steps with the same warm-up fraction (rounded to the nearest
step) and refresh spacing.  The step actions come from the library's own
driver (sdattn_schedule_action).  Beside the measured K-step schedule, the
line gives the workload's full schedule modelled from the per-action median
step times (modelled_native_schedule_ms_per_step).

By default the 64K headline is followed by the metric's other contexts, the
8K, 16K and 32K workloads, each run as its own whole schedule (256, 192 and
128 steps; the same K steps instead when --steps is given) and reported under
"configs" (--no-sweep skips them).

Inputs are the seeded synthetic tensors of the workload (planted per-head
structure), resident in HBM before timing starts: the step-0 tensors serve
the dense steps and the selection step's tensors serve the selection and
sparse steps (kernel time does not depend on the drift between steps; the
pattern does, and it is computed from the real selection-step inputs).  With
--probe-interval the probes' decisions do depend on it, so each step after
the selection gets its own inputs: the workload's random-walk drift continued
on the device from the selection step's tensors, generated before timing.

The block-wise workload (--workload losa_sdar8b_32k) is timed the same way
over blocks of iterations on top of a cached prefix: the first iteration of a
block dense, the others LoSA-style (Active tokens, page selection, page union,
partial attention); see run_losa.

The JSON line reports the whole-schedule ms per step (value), per-phase
medians, effective TFLOP/s of the sparse steps on kept-block FLOPs, the dense
schedule on the same GPU, a roofline object for the kernel that takes most
of the timed time, and the oracle timed on the host on a bounded sample.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/denoise step + effective TFLOP/s (MFMA %) of sparse attn at 8K–64K vs dense"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MAX_GFX_CLOCK_MHZ = 2400.0  # the clock the MFMA peak is quoted at
WALK_BYTES_MAX = 64 << 30   # device memory for per-step inputs of a probed schedule


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def rescaled(w, K):
    """The workload's schedule stretched or shrunk to K steps."""
    from workloads.configs import scaled
    if K == w.total_steps:
        return w
    f = K / w.total_steps

    def nearest(x):  # round half up: keeps the warm-up share (205 of 1024 -> 4 of 20)
        return int(math.floor(x + 0.5))

    dense = min(K, nearest(w.dense_steps * f))
    if w.dense_steps > 0:
        dense = max(dense, 1)
    sel = min(dense, nearest(w.select_step * f)) if w.select_step else 0
    sel = min(sel, K - 1)
    if w.refresh_dense and w.selector != "blocks" and dense > 0:
        sel = min(sel, dense - 1)  # these selectors read a dense pass's lse: the selection step is dense
    interval = max(1, nearest(w.refresh_interval * f)) if w.refresh_interval else 0
    refresh = tuple(sorted({min(K - 1, nearest(t * f)) for t in w.refresh_steps} - {sel}))
    return scaled(w, total_steps=K, dense_steps=dense, select_step=sel, refresh_interval=interval,
                  refresh_steps=refresh)


class GpuMonitor:
    """Samples the GPU's socket power and graphics clocks with amd-smi from a
    host thread while the timed region runs.  Under sustained MFMA load the
    chip may run below its 2.4 GHz maximum (power management); the samples
    show at which clock the timed steps actually ran.  Reports nothing when
    amd-smi is absent or fails."""

    def __init__(self, period_s=0.5):
        import shutil
        import threading
        self.period = period_s
        self.samples = []
        self.error = None
        self.exe = shutil.which("amd-smi")
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def read(self):
        import subprocess
        r = subprocess.run([self.exe, "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=20)
        if r.returncode != 0:
            raise RuntimeError(f"amd-smi exited {r.returncode}: {r.stderr.strip()[:200]}")
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        power = float(g["power"]["socket_power"]["value"])
        clocks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                  if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        return power, (sum(clocks) / len(clocks) if clocks else None)

    def _run(self):
        while not self._stop.is_set():
            t0 = time.perf_counter()
            try:
                power, clock = self.read()
            except Exception as e:  # noqa: BLE001 - monitoring must never break the bench
                self.error = str(e)
                return
            self.samples.append((t0, time.perf_counter(), power, clock))
            self._stop.wait(max(0.0, self.period - (time.perf_counter() - t0)))

    def start(self):
        self.t_begin = time.perf_counter()
        if self.exe:
            self._thread.start()
        return self

    def stop(self):
        self.t_end = time.perf_counter()
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join(timeout=30)

    MIN_REGION_S = 2.0    # shorter timed regions report no clock/power statistics
    MIN_SAMPLES = 3
    SETTLE_S = 0.5        # readings that start this early in the region may describe the idle GPU before it

    def summary(self):
        """Statistics of the samples taken wholly inside the timed region,
        after its first SETTLE_S seconds; none unless the region lasts at least
        MIN_REGION_S and at least MIN_SAMPLES readings qualify (amd-smi reports
        averages over its own sampling window, so a lone reading in a short
        region can describe the idle GPU before the work)."""
        import numpy as np
        if not self._thread.ident:
            return {"samples": 0, "error": self.error or ("amd-smi not found" if not self.exe
                                                          else "not sampled (--no-gpu-monitor)")}
        region = self.t_end - self.t_begin
        inside = [s for s in self.samples if s[0] >= self.t_begin + self.SETTLE_S and s[1] <= self.t_end]
        if region < self.MIN_REGION_S or len(inside) < self.MIN_SAMPLES:
            return {"samples": 0, "error": self.error or (
                f"timed region {region:.2f} s with {len(inside)} settled amd-smi readings: at least "
                f"{self.MIN_REGION_S:g} s and {self.MIN_SAMPLES} readings are needed")}
        pw = np.array([s[2] for s in inside])
        ck = np.array([s[3] for s in inside if s[3] is not None])
        out = {"samples": len(inside), "tool": "amd-smi metric -p -c",
               "socket_power_w": {"median": round(float(np.median(pw)), 1), "min": round(float(pw.min()), 1),
                                  "max": round(float(pw.max()), 1)}}
        if len(ck):
            out["gfx_clock_mhz"] = {"median": round(float(np.median(ck)), 1), "min": round(float(ck.min()), 1),
                                    "max": round(float(ck.max()), 1)}
        return out


def schedule_desc(sd, w):
    sel = sd.SEL_KINDS[w.selector]
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    return sd.schedule_desc(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval, list(w.refresh_steps),
                            w.refresh_dense, sel, w.block, w.block, budget, w.column_keep_frac,
                            w.probe_interval, w.min_overlap)


def to_dev(x):
    import numpy as np
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def kernel_source_hash():
    """Hash of the sources the flash-forward kernel and its dispatch order
    are built from (the kernel whose counters the traffic files hold)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_bidirectional_attention_amd", "csrc")
    for f in ("flash_bf16.hip", "common.h", "launch.h", "block_plan.hip"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None if there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, acts, base_step, sel_step_inputs):
    """The oracle (fp64 numpy) on a bounded sample of the same work, scaled
    to ms per denoising step of the same schedule."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                                 if i.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover
        blas = None
    L, H, d = w.seq_len, w.q_heads, w.head_dim
    G = w.q_heads // w.kv_heads
    x0 = base_step
    xs = sel_step_inputs
    samples = {}
    # dense step: a few query rows of one head, scaled to all rows and heads
    rows = np.arange(0, L, max(1, L // 64))[:64]
    t0 = time.perf_counter()
    oracle.dense_attention(x0["q"][:, :1], x0["k"][:, :1], x0["v"][:, :1], rows=rows)
    t_dense = (time.perf_counter() - t0) * (L / len(rows)) * H
    samples["dense"] = f"{len(rows)} query rows of 1 head, x{L / len(rows) * H:.0f}"
    # selection: pooling + pooled mass + budget for one kv group, scaled to all groups
    t0 = time.perf_counter()
    if w.selector != "columns":
        if w.selector == "blocks_exact":
            # exact block mass of 4 query blocks of one head (with their lse), scaled to every block and head
            nqb = -(-L // w.block)
            nb = min(4, nqb)
            qs = xs["q"][:, :1, :nb * w.block]
            _, lse_s = oracle.dense_attention(qs, xs["k"][:, :1], xs["v"][:, :1])
            t0 = time.perf_counter()
            A = oracle.exact_block_mass(qs, xs["k"][:, :1], lse_s, w.block, w.block)
            if w.budget == "topk":
                oracle.select_topk(A, w.keep_frac)
            t_sel = (time.perf_counter() - t0) * (nqb / nb) * H
            samples["select"] = f"exact mass of {nb} query blocks of 1 head, x{nqb / nb * H:.0f}"
        else:
            A = oracle.pooled_mass(xs["q"][:, :G], xs["k"][:, :1], w.block, w.block)
            if w.budget == "topk":
                oracle.select_topk(A, w.keep_frac)
            else:
                oracle.select_mass_cap(A, w.mass, w.max_mean_density)
            t_sel = (time.perf_counter() - t0) * w.kv_heads
            samples["select"] = f"1 of {w.kv_heads} kv groups, x{w.kv_heads}"
        # sparse step: a few query blocks of one head, gather form
        nqb = -(-L // w.block)
        A1 = oracle.pooled_mass(xs["q"][:, :1], xs["k"][:, :1], w.block, w.block)
        if w.budget == "topk":
            rp, ci = oracle.select_topk(A1, w.keep_frac)
        else:
            rp, ci, _ = oracle.select_mass_cap(A1, w.mass, w.max_mean_density)
        qb = np.arange(0, nqb, max(1, nqb // 16))[:16]
        t0 = time.perf_counter()
        oracle.block_sparse_attention(xs["q"][:, :1], xs["k"][:, :1], xs["v"][:, :1], rp, ci, w.block, w.block,
                                      qblocks=qb)
        t_sparse = (time.perf_counter() - t0) * (nqb / len(qb)) * H
        samples["sparse"] = f"{len(qb)} query blocks of 1 head, x{nqb / len(qb) * H:.0f}"
        t_ov = 0.0
        if "PROBE_SPARSE" in acts:
            t0 = time.perf_counter()
            oracle.mask_overlap(rp, ci, rp, ci)
            t_ov = (time.perf_counter() - t0) * H
            samples["overlap"] = f"pattern overlap of 1 head's rows, x{H}"
    else:
        kcol = oracle.count_from_fraction(w.column_keep_frac, L)
        qrows = np.arange(0, L, max(1, L // 16))[:16]
        _, lse = oracle.dense_attention(xs["q"][:, :1], xs["k"][:, :1], xs["v"][:, :1], rows=qrows)
        t0 = time.perf_counter()
        s = (oracle.attention.as_f64(xs["q"][0, 0, qrows]) @ oracle.attention.as_f64(xs["k"][0, 0]).T) / np.sqrt(d)
        np.exp(s - lse[0, 0][:, None]).sum(axis=0)
        t_sel = (time.perf_counter() - t0) * (L / len(qrows)) * H
        samples["select"] = f"column scores of {len(qrows)} query rows of 1 head, x{L / len(qrows) * H:.0f}"
        cols = np.sort(np.random.default_rng(0).choice(L, kcol, replace=False))[None, None].repeat(w.kv_heads, 1)
        t0 = time.perf_counter()
        oracle.column_sparse_attention(xs["q"][:, :1], xs["k"][:, :1], xs["v"][:, :1], cols[:, :1], rows=qrows)
        t_sparse = (time.perf_counter() - t0) * (L / len(qrows)) * H
        samples["sparse"] = f"{len(qrows)} query rows of 1 head, x{L / len(qrows) * H:.0f}"
        t_ov = 0.0
    n = {a: acts.count(a) for a in ("DENSE", "DENSE_SELECT", "SELECT_SPARSE", "SPARSE", "PROBE_SPARSE")}
    total = (n["DENSE"] * t_dense + n["DENSE_SELECT"] * (t_dense + t_sel) + n["SELECT_SPARSE"] * (t_sel + t_sparse)
             + n["SPARSE"] * t_sparse + n["PROBE_SPARSE"] * (t_sel + t_ov + t_sparse))
    ms = 1e3 * total / len(acts)
    return {"value": round(ms, 3), "unit": "ms/denoise step", "cores": threads, "host_cores": cores,
            "cpu_model": cpu_model, "blas": blas, "kind": "oracle",
            "sample": ("fp64 numpy oracle, extrapolated from timed samples: " + "; ".join(
                f"{k}: {v}" for k, v in samples.items()) + "; weighted by the schedule's action counts"),
            "per_step_ms": {"dense": round(1e3 * t_dense, 1), "select": round(1e3 * t_sel, 1),
                            "sparse": round(1e3 * t_sparse, 1)}}


def sdpa_dense_baseline(x, w, dense_ms):
    """PyTorch-ROCm's own fused attention (scaled_dot_product_attention with
    only the flash backend enabled: it raises instead of falling back to the
    unfused path) on the dense step's tensors, for context beside this
    library's dense forward.  GQA heads are expanded to Hq first."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    G = w.q_heads // w.kv_heads
    try:
        k = x["k"].repeat_interleave(G, dim=1).contiguous() if G > 1 else x["k"]
        v = x["v"].repeat_interleave(G, dim=1).contiguous() if G > 1 else x["v"]
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(x["q"], k, v)
            torch.cuda.synchronize()
            n = 3 if w.seq_len >= 32768 else 10
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                torch.nn.functional.scaled_dot_product_attention(x["q"], k, v)
            e1.record()
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
    except Exception as e:  # noqa: BLE001 - context only; never fails the bench
        return {"kind": "torch SDPA (flash backend)", "error": str(e)[:200]}
    flops = 4.0 * w.batch * w.q_heads * w.seq_len ** 2 * w.head_dim
    return {"kind": "torch SDPA (flash backend), PyTorch-ROCm, same GPU and tensors", "ms_per_step": round(ms, 3),
            "tflops": round(flops / (ms * 1e9), 1), "this_library_speedup": round(ms / dense_ms, 3)}


def compare_masks(sd, p, w, x, o, lse):
    """The exact and the pooled pattern of the selection step's tensors: their
    overlap |A n B| / |A u B| (sdattn_mask_overlap) and the share of the exact
    attention mass each keeps (mean over rows of the kept blocks' exact mass)."""
    import numpy as np
    import torch
    L = w.seq_len
    nqb, nkb = -(-L // w.block), -(-L // w.block)
    rows = w.batch * w.q_heads * nqb
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    out = {}
    masks = {}
    A = torch.empty(rows * nkb, dtype=torch.float32, device="cuda")
    for kind in ("exact", "pooled"):
        if kind == "exact":
            wsb, cap = sd.sdattn_select_blocks_exact_workspace(p, w.block, w.block, budget)
        else:
            wsb, cap = sd.sdattn_select_blocks_workspace(p, w.block, w.block, budget)
        rp = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
        ci = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        if kind == "exact":
            sd.sdattn_select_blocks_exact(p, x["q"], x["k"], lse, w.block, w.block, budget, rp, ci, cap, A, ws, wsb)
        else:
            sd.sdattn_select_blocks(p, x["q"], x["k"], w.block, w.block, budget, rp, ci, cap, None, ws, wsb)
        masks[kind] = (rp, ci)
    counts = torch.empty(3, dtype=torch.int64, device="cuda")
    sd.sdattn_mask_overlap(rows, masks["exact"][0], masks["exact"][1], masks["pooled"][0], masks["pooled"][1], counts)
    torch.cuda.synchronize()
    inter, na, nb = (int(v) for v in counts.cpu())
    out["overlap_exact_vs_pooled"] = round(inter / max(1, na + nb - inter), 4)
    Ah = A.cpu().numpy().reshape(rows, nkb).astype(np.float64)
    for kind, (rp, ci) in masks.items():
        rph = rp.cpu().numpy()
        cih = ci.cpu().numpy()[:rph[-1]]
        rid = np.repeat(np.arange(rows), np.diff(rph))
        out[f"captured_mass_{kind}"] = round(float(Ah[rid, cih].sum() / rows), 4)
        out[f"nnz_{kind}"] = int(rph[-1])
    return out


def run_losa(args, w):
    """Block-wise workload: a block of block_len tokens over a cached prefix.
    A step is one denoising iteration of a block; the schedule repeats blocks
    of steps_per_block iterations: iteration 0 computes the page means of the
    prefix and runs the dense form, iterations 1.. run the LoSA-style step
    (locality, Active set, page selection, union, partial attention)."""
    import numpy as np
    import torch

    import sparse_bidirectional_attention_amd as sd
    from workloads.generate import make_losa_base, make_losa_cache, make_losa_iteration

    T = w.steps_per_block
    K = args.steps if args.steps is not None else 64 * T
    B, Hq, Hkv, Lp, Bs, d = w.batch, w.q_heads, w.kv_heads, w.prefix_len, w.block_len, w.head_dim
    n_pages = Lp // w.page
    torch.cuda.set_device(0)
    log(f"workload {w.name}: prefix {Lp}, block {Bs}, Hq={Hq} Hkv={Hkv} d={d} {w.dtype}, page {w.page}, "
        f"{w.n_active} Active tokens, {w.pages_per_query} pages per query; {K} steps in blocks of {T}")
    t0 = time.time()
    base = make_losa_base(w)
    cache = make_losa_cache(w, base)
    iters_h = [make_losa_iteration(w, t, base) for t in range(T)]
    del base
    log(f"inputs generated in {time.time() - t0:.1f} s")
    kc, vc = to_dev(cache["k_cache"]), to_dev(cache["v_cache"])
    its = [{n: to_dev(a) for n, a in x.items()} for x in iters_h]
    p = sd.losa_problem(B, Hq, Hkv, Lp, Bs, d, w.page, w.n_active, w.pages_per_query)
    ws_bytes, cap = sd.sdattn_losa_workspace(p)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    kp = torch.empty(B, Hkv, n_pages, d, dtype=torch.float32, device="cuda")
    o = torch.empty(B, Hq, Bs, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, Bs, dtype=torch.float32, device="cuda")
    active = torch.empty(B, w.n_active, dtype=torch.int32, device="cuda")
    upages = torch.empty(B, Hkv, cap, dtype=torch.int32, device="cuda")
    ucount = torch.empty(B, Hkv, dtype=torch.int32, device="cuda")

    pool_ev = {}

    def step(t, evs=None):
        it = t % T
        if it == 0:
            sd.sdattn_losa_pool_pages(p, kc, kp)
            if evs is not None:  # the dense call alone, for the roofline
                pool_ev[t] = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                pool_ev[t][0].record()
            x = its[0]
            sd.sdattn_losa_dense(p, x["q"], kc, vc, x["k_blk"], x["v_blk"], o, lse, ws)
            if evs is not None:
                pool_ev[t][1].record()
        else:
            x, xp = its[it], its[it - 1]
            sd.sdattn_losa_step(p, x["q"], xp["q"], kc, vc, kp, x["k_blk"], x["v_blk"], o, lse, active, upages,
                                ucount, ws)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    monitor = GpuMonitor()
    if not args.no_gpu_monitor:
        monitor.start()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for t in range(K):
        ev[t][0].record()
        step(t, ev)
        ev[t][1].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    monitor.stop()
    total_ms = start.elapsed_time(end)
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    dense_call_ms = float(np.mean([a.elapsed_time(b) for a, b in pool_ev.values()])) if pool_ev else None
    dense_idx = [t for t in range(K) if t % T == 0]
    losa_idx = [t for t in range(K) if t % T != 0]
    dense_ms = float(np.mean(step_ms[dense_idx])) if dense_idx else None
    losa_ms = float(np.mean(step_ms[losa_idx])) if losa_idx else None

    # The same block replayed from HIP graphs: the page means and the dense
    # iteration in one graph, the T - 1 LoSA iterations in another.  A LoSA
    # iteration is six short launches on one stream; a graph replays them
    # without the host's per-launch work between kernels.
    graph = None
    if T > 1:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            for t in range(T):  # warm the captured calls once outside capture
                step(t)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        g_dense, g_losa = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_dense):
            step(0)
        with torch.cuda.graph(g_losa):
            for t in range(1, T):
                step(t)
        torch.cuda.synchronize()
        reps = max(8, K // T)
        gtimes = {}
        for name, g in (("dense", g_dense), ("losa", g_losa)):
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            gtimes[name] = e0.elapsed_time(e1) / reps
        graph = {"replays": reps, "dense_iteration_ms": round(gtimes["dense"], 4),
                 "losa_step_ms": round(gtimes["losa"] / (T - 1), 4),
                 "ms_per_step": round((gtimes["dense"] + gtimes["losa"]) / T, 4),
                 "note": "one block replayed from two HIP graphs (dense iteration with the page means; the "
                         "T - 1 LoSA iterations); value stays the stream-launched schedule"}
        del g_dense, g_losa

    # union sizes of every iteration of one block (they repeat block after block)
    unions = []
    for it in range(1, T):
        step(it)
        torch.cuda.synchronize()
        unions.append(ucount.cpu().numpy().astype(np.int64))
    u_mean = float(np.mean([u.sum() for u in unions])) if unions else 0.0
    # algorithmic work
    G = Hq // Hkv
    dense_flops = 4.0 * B * Hq * Bs * (Lp + Bs) * d
    dense_bytes = 2.0 * B * Hkv * (Lp + Bs) * d * 2 + B * Hq * Bs * (d * 2 * 2 + 4)
    losa_bytes = (u_mean * w.page * d * 2 * 2 + 2.0 * B * Hkv * Bs * d * 2 + 2.0 * B * Hq * Bs * d * 2
                  + B * Hkv * n_pages * d * 4 + B * Hq * w.n_active * (d * 2 + 4))
    losa_flops = 4.0 * G * w.n_active * d * (u_mean * w.page + B * Hkv * Bs) + 2.0 * B * Hq * w.n_active * n_pages * d
    kernels = {}
    if dense_call_ms:
        # bf16 MFMA at ~128 FLOP per byte of K/V, below the MFMA ridge (~312): bound by the K/V stream
        a = dense_bytes / (dense_call_ms * 1e6)
        tf = dense_flops / (dense_call_ms * 1e9)
        kernels["losa_dense_iteration"] = {
            "bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4), "launch_ms": round(dense_call_ms, 4), "bytes_per_launch": dense_bytes,
            "flops_per_launch": dense_flops, "tflops": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "kernels": "losa_attend_kernel (dense) + losa_merge_kernel; the page means (losa_pool_kernel) run "
                       "once per block before it", "traffic": losa_traffic(w.name)}
        tr = kernels["losa_dense_iteration"]["traffic"]
        if tr:
            kernels["losa_dense_iteration"]["traffic_gbs"] = round(tr / (dense_call_ms * 1e6), 1)
            kernels["losa_dense_iteration"]["traffic_frac_of_hbm_peak"] = round(tr / (dense_call_ms * 1e6) / PEAK_HBM_GBS, 4)
    if losa_ms:
        a = losa_bytes / (losa_ms * 1e6)
        kernels["losa_step"] = {
            "bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4), "launch_ms": round(losa_ms, 4), "bytes_per_launch": losa_bytes,
            "flops_per_launch": losa_flops,
            "kernels": "delta, scores (with the Active ranking), topk, union, attend, merge (six launches)",
            "traffic": None}
    # The roofline names the heaviest single kernel: the dense iteration's
    # attention (one C call = that kernel plus its merge, ~10% of the call).  A
    # LoSA iteration is seven short launches and stays under "kernels".
    dom = "losa_dense_iteration" if "losa_dense_iteration" in kernels else "losa_step"
    roof = {k: v for k, v in kernels[dom].items() if k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dom
    ms_per_step = total_ms / K
    out = {
        "metric": METRIC, "value": round(ms_per_step, 4), "unit": "ms/denoise step", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "prefix_len": Lp,
                   "block_len": Bs, "head_dim": d, "page": w.page, "n_active": w.n_active,
                   "pages_per_query": w.pages_per_query, "steps_per_block": T},
        "roofline": roof,
        "phases": {"dense_iteration_ms": round(dense_ms, 4) if dense_ms else None,
                   "dense_call_ms": round(dense_call_ms, 4) if dense_call_ms else None,
                   "losa_step_ms": round(losa_ms, 4) if losa_ms else None,
                   "losa_step_speedup_vs_dense_iteration": round(dense_ms / losa_ms, 2) if dense_ms and losa_ms
                   else None,
                   "union_pages_per_step": round(u_mean, 1),
                   "union_density": round(u_mean / (B * Hkv * n_pages), 5),
                   "union_pages_by_iteration": [u.ravel().tolist() for u in unions]},
        "dense_baseline": {"ms_per_step": round(dense_ms, 4) if dense_ms else None,
                           "schedule_speedup": round(dense_ms / ms_per_step, 3) if dense_ms else None},
        "kernels": kernels,
        "graph_replay": graph,
        "step_times": {a: {"n": len(v), "median_ms": round(float(np.median(step_ms[v])), 4),
                           "p10_ms": round(float(np.percentile(step_ms[v], 10)), 4),
                           "p90_ms": round(float(np.percentile(step_ms[v], 90)), 4)}
                       for a, v in (("DENSE", dense_idx), ("LOSA", losa_idx)) if v},
        "wall_s": round(wall, 2),
        "gpu_state": monitor.summary(),
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline_losa(w, cache, iters_h)
    print(json.dumps(out), flush=True)


def losa_traffic(workload):
    """Calibrated L2-to-fabric bytes per dense-iteration call from the profile
    counters, if they were taken on the current block-wise kernel sources."""
    f = os.path.join(ROOT, "profiles", f"traffic_losa_dense_{workload}.json")
    if not os.path.exists(f):
        return None
    t = json.load(open(f))
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_bidirectional_attention_amd", "csrc")
    for name in ("losa.hip", "common.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return t["hbm_bytes_per_launch"] if t.get("kernel_source_hash") == h.hexdigest()[:16] else None


def cpu_baseline_losa(w, cache, iters):
    """The oracle on one block's dense iteration and two later iterations,
    weighted by the block schedule."""
    import oracle.losa as ol
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    T = w.steps_per_block
    t0 = time.perf_counter()
    o, lse = ol.losa_dense(iters[0]["q"], cache["k_cache"], cache["v_cache"], iters[0]["k_blk"], iters[0]["v_blk"])
    t_dense = time.perf_counter() - t0
    n = min(2, T - 1)
    t0 = time.perf_counter()
    for it in range(1, n + 1):
        r = ol.losa_step(iters[it]["q"], iters[it - 1]["q"], cache["k_cache"], cache["v_cache"], iters[it]["k_blk"],
                         iters[it]["v_blk"], o, lse, w.page, w.n_active, w.pages_per_query)
        o, lse = r["o"], r["lse"]
    t_step = (time.perf_counter() - t0) / max(1, n)
    ms = 1e3 * (t_dense + (T - 1) * t_step) / T
    return {"value": round(ms, 3), "unit": "ms/denoise step", "cores": threads,
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"fp64 numpy oracle: the dense iteration and {n} later iterations of one block, "
                      f"weighted 1:{T - 1}",
            "per_step_ms": {"dense": round(1e3 * t_dense, 1), "losa": round(1e3 * t_step, 1)}}


def schedule_actions(sd, p, w):
    """The action of every step of workload w's schedule, from the library's
    own driver (sdattn_schedule_action on a handle of that schedule)."""
    h = sd.sdattn_schedule_create(p, schedule_desc(sd, w))
    try:
        return [sd.sdattn_schedule_action(h, t) for t in range(w.total_steps)]
    finally:
        sd.sdattn_schedule_destroy(h)


def d2h_int32(ptr, n):
    """n int32 values from a device pointer (a borrowed schedule buffer)."""
    import ctypes
    import numpy as np
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    out = np.zeros(n, np.int32)
    rc = hip.hipMemcpy(out.ctypes.data, ptr, 4 * n, 2)  # hipMemcpyDeviceToHost
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
    return out


def run_schedule(args, w0, K, warmup, with_gpu_state=True):
    """One workload's schedule of K steps through the C-ABI driver, timed with
    HIP events per step and over the whole schedule.  Returns the JSON record
    (without the oracle leg) and the host inputs (for the oracle leg)."""
    import numpy as np
    import torch

    import sparse_bidirectional_attention_amd as sd
    from workloads import make_base, make_step

    w = rescaled(w0, K)
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    acts = schedule_actions(sd, p, w)
    native_acts = schedule_actions(sd, p, w0)
    log(f"workload {w.name}: L={w.seq_len} Hq={w.q_heads} Hkv={w.kv_heads} d={w.head_dim} {w.dtype} "
        f"block={w.block}; schedule of {K} steps: " + ", ".join(f"{a} x{acts.count(a)}" for a in sorted(set(acts))))
    t0 = time.time()
    base = make_base(w0)
    x0h = make_step(w0, 0, base)
    xsh = make_step(w0, w0.select_step, base) if w0.select_step else x0h
    del base
    log(f"inputs generated in {time.time() - t0:.1f} s")
    x0 = {n: to_dev(a) for n, a in x0h.items()}
    xs = {n: to_dev(a) for n, a in xsh.items()}
    o = torch.empty_like(x0["q"])
    lse = torch.empty(x0["q"].shape[:3], dtype=torch.float32, device="cuda")

    # With probes (adaptive anchors), every step after the selection gets its
    # own inputs: the random walk of the workload's step drift continued on
    # the device from the selection step's tensors, X_t = X_{t-1} + sigma N_t
    # for Q and K (V fixed), rounded to the input dtype, all generated before
    # the timed region.  Otherwise kernel time does not depend on the drift:
    # the dense steps take the step-0 tensors and the rest the selection
    # step's.
    walk = {}
    walk_note = None
    if w.probe_interval and w.selector == "blocks" and w.step_noise == "walk":
        n_walk = K - 1 - w.select_step
        need = n_walk * (xs["q"].numel() + xs["k"].numel()) * xs["q"].element_size()
        if need <= WALK_BYTES_MAX:
            gen = torch.Generator(device="cuda")
            gen.manual_seed(1_000_003 * w.wid + 7)
            qf, kf = xs["q"].float(), xs["k"].float()
            for t in range(w.select_step + 1, K):
                qf.add_(torch.randn(qf.shape, generator=gen, device="cuda"), alpha=w.step_sigma)
                kf.add_(torch.randn(kf.shape, generator=gen, device="cuda"), alpha=w.step_sigma)
                walk[t] = {"q": qf.to(xs["q"].dtype), "k": kf.to(xs["k"].dtype), "v": xs["v"]}
            del qf, kf
            torch.cuda.synchronize()
            walk_note = (f"steps {w.select_step + 1}..{K - 1}: own inputs, a random walk (sigma {w.step_sigma:g} per "
                         f"step) on the device from the selection step's tensors ({need / 2**30:.1f} GiB)")
        else:
            walk_note = f"the per-step inputs would need {need / 2**30:.0f} GiB; selection-step tensors reused"

    def inputs_for(a, t=-1):
        if t in walk:
            return walk[t]
        return x0 if a == "DENSE" else xs

    # warm-up: W untimed steps of a schedule of the same shape
    if warmup > 0:
        ww = rescaled(w0, max(2, warmup))
        hw = sd.sdattn_schedule_create(p, schedule_desc(sd, ww))
        for t in range(warmup):
            x = inputs_for(sd.sdattn_schedule_action(hw, t % ww.total_steps))
            sd.sdattn_schedule_step(hw, t % ww.total_steps, x["q"], x["k"], x["v"], o, lse)
        torch.cuda.synchronize()
        sd.sdattn_schedule_destroy(hw)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    h = sd.sdattn_schedule_create(p, schedule_desc(sd, w))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    monitor = GpuMonitor()
    if with_gpu_state and not args.no_gpu_monitor:
        monitor.start()
    t_wall = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for t in range(K):
        x = inputs_for(acts[t], t)
        ev[t][0].record()
        sd.sdattn_schedule_step(h, t, x["q"], x["k"], x["v"], o, lse)
        ev[t][1].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    monitor.stop()
    total_ms = start.elapsed_time(end)
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    stats, last_sel = sd.sdattn_schedule_stats(h)
    n_probes, n_adopted, last_overlap = sd.sdattn_schedule_probe_stats(h)

    # pattern size for the kept-FLOP count, read back from the driver's buffers
    L, H, Hkv, d = w.seq_len, w.q_heads, w.kv_heads, w.head_dim
    rp_ptr, ci_ptr, cap = sd.sdattn_schedule_mask(h)
    if w.selector != "columns":
        rows = w.batch * H * (-(-L // w.block))
        nnz = int(d2h_int32(rp_ptr + 4 * rows, 1)[0])
        kept_flops = 4.0 * d * w.block * w.block * nnz
        density = nnz / (rows * (-(-L // w.block)))
    else:
        kcol = cap // (w.batch * Hkv)  # the column list holds [B][Hkv][kcol]
        kept_flops = 4.0 * d * L * kcol * H * w.batch
        nnz = kcol * Hkv
        density = kcol / L
    sd.sdattn_schedule_destroy(h)
    dense_flops = 4.0 * w.batch * H * L * L * d
    mask_cmp = compare_masks(sd, p, w, xs, o, lse) if w.selector == "blocks_exact" else None

    def med(a):
        return float(np.median(a)) if len(a) else None

    idx = {a: [t for t in range(K) if acts[t] == a] for a in set(acts)}
    sparse_ms = med(step_ms[idx["SPARSE"]]) if idx.get("SPARSE") else None
    dense_ms = med(step_ms[idx["DENSE"]]) if idx.get("DENSE") else None
    # dense baseline on the same GPU: the dense forward for every step
    nd = 3 if L >= 32768 else 10
    sd.sdattn_forward_dense(p, x0["q"], x0["k"], x0["v"], o, lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nd):
        sd.sdattn_forward_dense(p, x0["q"], x0["k"], x0["v"], o, lse)
    e1.record()
    torch.cuda.synchronize()
    dense_base_ms = e0.elapsed_time(e1) / nd

    if dense_ms is None:
        dense_ms = dense_base_ms
    # selection time: a selecting step minus the attention it also runs
    select_ms = None
    if idx.get("SELECT_SPARSE") and sparse_ms is not None:
        select_ms = med(step_ms[idx["SELECT_SPARSE"]]) - sparse_ms
    elif idx.get("DENSE_SELECT"):
        select_ms = med(step_ms[idx["DENSE_SELECT"]]) - dense_ms

    probe_ms = med(step_ms[idx["PROBE_SPARSE"]]) if idx.get("PROBE_SPARSE") else None
    ms_per_step = total_ms / K
    # per action: median and p10/p90 of the step times; the K-step schedule
    # modelled from the medians (beside the measured one), and the workload's
    # own full schedule modelled from the same medians
    step_stats = {a: {"n": len(v), "median_ms": round(float(np.median(step_ms[v])), 4),
                      "p10_ms": round(float(np.percentile(step_ms[v], 10)), 4),
                      "p90_ms": round(float(np.percentile(step_ms[v], 90)), 4)} for a, v in sorted(idx.items())}
    medians = {a: float(np.median(step_ms[v])) for a, v in idx.items()}
    modelled_ms = sum(len(v) * medians[a] for a, v in idx.items()) / K
    native_counts = {a: native_acts.count(a) for a in sorted(set(native_acts))}
    if all(a in medians for a in native_counts):
        native_ms = sum(n * medians[a] for a, n in native_counts.items()) / len(native_acts)
    else:  # an action of the full schedule did not occur in the K steps
        native_ms = None
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # Roofline figures use each kernel's average launch inside the timed region:
    # a SPARSE step is one sparse forward, a DENSE step one dense forward.
    def mean(a):
        return float(np.mean(a)) if len(a) else None

    sparse_launch_ms = mean(step_ms[idx["SPARSE"]]) if idx.get("SPARSE") else sparse_ms
    dense_launch_ms = mean(step_ms[idx["DENSE"]]) if idx.get("DENSE") else dense_base_ms
    sparse_tflops = kept_flops / (sparse_launch_ms * 1e9) if sparse_launch_ms else None
    dense_tflops = dense_flops / (dense_launch_ms * 1e9)
    dense_base_tflops = dense_flops / (dense_base_ms * 1e9)
    # kernel with the largest share of the timed region
    n_sparse = len(idx.get("SPARSE", [])) + len(idx.get("SELECT_SPARSE", [])) + len(idx.get("PROBE_SPARSE", []))
    n_dense = len(idx.get("DENSE", [])) + len(idx.get("DENSE_SELECT", []))
    share_sparse = n_sparse * (sparse_launch_ms or 0)
    share_dense = n_dense * dense_launch_ms
    kernels = {
        "flash_fwd_bf16_sparse" if w.selector != "columns" else "flash_fwd_bf16_column": {
            "bound": "mfma", "achieved": round(sparse_tflops, 1) if sparse_tflops else None, "peak": peak,
            "unit": "TFLOP/s", "frac": round(sparse_tflops / peak, 4) if sparse_tflops else None,
            "launch_ms": round(sparse_launch_ms, 4) if sparse_launch_ms else None,
            "flops_per_launch": kept_flops,
            "traffic": load_traffic("flash_sparse", w0.name)},
        "flash_fwd_bf16_dense": {
            "bound": "mfma", "achieved": round(dense_tflops, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(dense_tflops / peak, 4), "launch_ms": round(dense_launch_ms, 3),
            "flops_per_launch": dense_flops, "traffic": load_traffic("flash_dense", w0.name)},
    }
    # the calibrated L2-to-fabric bytes per launch (FETCH_SIZE also counts
    # Infinity Cache hits, so this bounds HBM traffic from above) as a rate
    for kv in kernels.values():
        if kv["traffic"] and kv["launch_ms"]:
            gbs = kv["traffic"] / (kv["launch_ms"] * 1e6)
            kv["traffic_gbs"] = round(gbs, 1)
            kv["traffic_frac_of_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
    dom = max(kernels, key=lambda k: share_sparse if "dense" not in k else share_dense)
    roof = {k: v for k, v in kernels[dom].items() if k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dom

    # the MFMA peak scales with the graphics clock: the published peak is at 2.4 GHz
    gpu_state = monitor.summary() if with_gpu_state else None
    if gpu_state and "gfx_clock_mhz" in gpu_state:
        clk = gpu_state["gfx_clock_mhz"]["median"]
        scaled_peak = peak * clk / MAX_GFX_CLOCK_MHZ
        fr = {k: v["achieved"] / scaled_peak for k, v in kernels.items() if v["achieved"]}
        if any(f > 1.0 for f in fr.values()):
            # a kernel above the clock-scaled peak: the clock readings do not describe the timed work
            gpu_state["peak_at_median_clock_tflops"] = None
            gpu_state["frac_of_peak_at_median_clock"] = None
            gpu_state["note"] = "clock readings inconsistent with the measured throughput; not used"
        else:
            gpu_state["peak_at_median_clock_tflops"] = round(scaled_peak, 1)
            gpu_state["frac_of_peak_at_median_clock"] = {k: round(f, 4) for k, f in fr.items()}
    budget = (f"top-{w.keep_frac:g}" if w.budget == "topk" and w.selector != "columns"
              else f"mass {w.mass:g} cap {w.max_mean_density:g}" if w.selector != "columns"
              else f"columns {w.column_keep_frac:g}")
    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms/denoise step",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w0.name, "batch": w.batch, "q_heads": H, "kv_heads": Hkv, "seq_len": L,
                   "head_dim": d, "block": w.block, "selector": w.selector, "budget": budget,
                   "schedule": {a: acts.count(a) for a in sorted(set(acts))},
                   "native_schedule": native_counts},
        "roofline": roof,
        "phases": {"dense_step_ms": round(dense_ms, 3) if dense_ms else None,
                   "select_ms": round(select_ms, 3) if select_ms else None,
                   "sparse_step_ms": round(sparse_ms, 4) if sparse_ms else None,
                   "sparse_effective_tflops": round(sparse_tflops, 1) if sparse_tflops else None,
                   "sparse_mfma_frac": round(sparse_tflops / peak, 4) if sparse_tflops else None,
                   "kept_density": round(density, 5), "kept_nnz": nnz},
        "mask_comparison": mask_cmp,
        "probes": ({"probe_step_ms": round(probe_ms, 4), "probe_overhead_ms": round(probe_ms - sparse_ms, 4)
                    if sparse_ms else None, "n_probes": n_probes, "n_adopted": n_adopted,
                    "last_overlap": round(last_overlap, 6), "min_overlap": w.min_overlap,
                    "probe_interval": w.probe_interval, "inputs": walk_note} if probe_ms is not None else None),
        "dense_baseline": {"ms_per_step": round(dense_base_ms, 3), "tflops": round(dense_base_tflops, 1),
                           "mfma_frac": round(dense_base_tflops / peak, 4),
                           "schedule_speedup": round(dense_base_ms / ms_per_step, 3),
                           "native_schedule_speedup": round(dense_base_ms / native_ms, 3) if native_ms else None,
                           "sparse_step_speedup": round(dense_base_ms / sparse_ms, 3) if sparse_ms else None},
        "kernels": kernels,
        "step_times": step_stats,
        "modelled_ms_per_step": round(modelled_ms, 4),
        "modelled_native_schedule_ms_per_step": round(native_ms, 4) if native_ms else None,
        "wall_s": round(wall, 2),
        "gpu_state": gpu_state,
        "schedule_stats": stats,
    }
    if not args.no_sdpa_baseline and w.dtype == "bf16":
        out["sdpa_dense_baseline"] = sdpa_dense_baseline(x0, w, dense_launch_ms)
    del x0, xs, o, lse, walk
    torch.cuda.empty_cache()
    return out, (acts, x0h, xsh)


# The other contexts of the metric (8K-64K), run after the 64K headline with
# the same step count: one compact record each.
SWEEP = ("llada8b_8k", "pulsecol_dream7b_16k", "sparsed_32k")


def compact(rec):
    ph = rec["phases"]
    return {"ms_per_step": rec["value"], "steps": rec["steps"], "schedule": rec["config"]["schedule"],
            "modelled_native_schedule_ms_per_step": rec["modelled_native_schedule_ms_per_step"],
            "native_schedule": rec["config"]["native_schedule"],
            "dense_step_ms": ph["dense_step_ms"], "select_ms": ph["select_ms"], "sparse_step_ms": ph["sparse_step_ms"],
            "sparse_effective_tflops": ph["sparse_effective_tflops"], "sparse_mfma_frac": ph["sparse_mfma_frac"],
            "kept_density": ph["kept_density"],
            "dense_tflops": rec["kernels"]["flash_fwd_bf16_dense"]["achieved"],
            "dense_mfma_frac": rec["kernels"]["flash_fwd_bf16_dense"]["frac"],
            "sparse_traffic": next(iter(rec["kernels"].values()))["traffic"],
            "dense_baseline_ms_per_step": rec["dense_baseline"]["ms_per_step"],
            "native_schedule_speedup_vs_dense": rec["dense_baseline"]["native_schedule_speedup"],
            "sparse_step_speedup_vs_dense": rec["dense_baseline"]["sparse_step_speedup"],
            "sdpa_dense_ms": (rec.get("sdpa_dense_baseline") or {}).get("ms_per_step")}


def operand_study(args, w0):
    """The dense forward and the block-sparse forward (on the pattern the
    pooled selection makes from the workload's inputs), each one instruction
    stream, on three operand sets: the workload's inputs, all zeros and all
    ones (K and V; Q as given), each for a few seconds while amd-smi samples
    the socket power and graphics clock.  The chip runs at its package power
    limit under sustained MFMA load, so what an MFMA costs depends on its
    operands' switching activity: the same kernel that is power-limited on
    real data runs faster on constant data.  Reports each set's launch time,
    TFLOP/s, fraction of the 2.5 PF peak, the median clock and power, and the
    fraction of the peak scaled to that clock."""
    import numpy as np
    import torch

    import sparse_bidirectional_attention_amd as sd
    from workloads import make_base, make_step

    w = w0
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    base = make_base(w)
    xh = make_step(w, 0, base)
    del base
    x = {n: to_dev(a) for n, a in xh.items()}
    del xh
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    dense_flops = 4.0 * w.batch * w.q_heads * w.seq_len ** 2 * w.head_dim
    sets = {"workload": (x["q"], x["k"], x["v"]),
            "zeros": (x["q"], torch.zeros_like(x["k"]), torch.zeros_like(x["v"])),
            "ones": (x["q"], torch.ones_like(x["k"]), torch.ones_like(x["v"]))}
    if w.selector == "columns":
        raise SystemExit("--operand-study takes a block workload (its pooled block pattern)")
    # the pooled selection's pattern of the workload's own inputs, kept fixed
    # across the operand sets
    nqb = -(-w.seq_len // w.block)
    rows = w.batch * w.q_heads * nqb
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    wsb, cap = sd.sdattn_select_blocks_workspace(p, w.block, w.block, budget)
    rp = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
    ci = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    sd.sdattn_select_blocks(p, x["q"], x["k"], w.block, w.block, budget, rp, ci, cap, None, ws, wsb)
    torch.cuda.synchronize()
    del ws
    kept_flops = 4.0 * w.head_dim * w.block * w.block * int(rp[rows].item())
    forwards = {
        "dense": (dense_flops, lambda q, k, v: sd.sdattn_forward_dense(p, q, k, v, o, lse)),
        "block_sparse": (kept_flops, lambda q, k, v: sd.sdattn_forward_block_sparse(p, q, k, v, w.block, w.block,
                                                                                    rp, ci, o, lse)),
    }
    out = {"kind": "dense and block-sparse forwards on three operand sets, same kernels, same pattern",
           "workload": w.name, "forwards": {}}
    for fname, (flops, fwd) in forwards.items():
        recs = {}
        for name, (q, k, v) in sets.items():
            fwd(q, k, v)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fwd(q, k, v)
            torch.cuda.synchronize()
            one_ms = max(1e-3, (time.perf_counter() - t0) * 1e3)
            n = max(8, int(math.ceil(args.operand_seconds * 1e3 / one_ms)))
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            mon = GpuMonitor()
            if not args.no_gpu_monitor:
                mon.start()
            for e0, e1 in evs:
                e0.record()
                fwd(q, k, v)
                e1.record()
            torch.cuda.synchronize()
            mon.stop()
            ms = np.array([a.elapsed_time(b) for a, b in evs])
            med = float(np.median(ms))
            tf = flops / (med * 1e9)
            rec = {"launches": n, "median_ms": round(med, 3), "tflops": round(tf, 1),
                   "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "gpu_state": mon.summary()}
            gs = rec["gpu_state"]
            if "gfx_clock_mhz" in gs:
                sp = PEAK_BF16_TFLOPS * gs["gfx_clock_mhz"]["median"] / MAX_GFX_CLOCK_MHZ
                rec["peak_at_median_clock_tflops"] = round(sp, 1)
                rec["frac_of_peak_at_median_clock"] = round(tf / sp, 4) if tf <= sp else None
            recs[name] = rec
            log(f"{fname} operand set {name}: {med:.3f} ms, {tf:.1f} TFLOP/s")
        out["forwards"][fname] = {"flops_per_launch": flops, "sets": recs}
    print(json.dumps(out), flush=True)


def split_study(args, w0):
    """Split rows against the dispatch plan alone, on the workload's inputs and
    block size with head-skewed patterns: n heads keep every key block, the
    others a few (seeded random kept blocks, ascending), n = 0, 1, 2, 4; and
    the pooled selection's own pattern.  A near-dense head beside sparse ones
    is what a head-adaptive budget without a cap can produce (Step-dLLM,
    Abstract); no schedule of the five workloads makes one, so this is a
    study, not the headline.  Reports per pattern the kept blocks, the rows
    the split plan cuts and its chunk length, both forwards' launch times
    (HIP events, median of three rounds) and TFLOP/s on the kept blocks, and
    the split output's largest difference from the planned one."""
    import numpy as np
    import torch

    import sparse_bidirectional_attention_amd as sd
    from workloads import make_base, make_step

    w = w0
    if w.selector == "columns":
        raise SystemExit("--split-study takes a block workload")
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    base = make_base(w)
    xh = make_step(w, w.select_step, base)
    del base
    x = {n: to_dev(a) for n, a in xh.items()}
    del xh
    bq = w.block
    nqb = -(-w.seq_len // bq)
    pairs = w.batch * w.q_heads
    rows = pairs * nqb
    slots = 256 * (4 if bq == 64 else 2)
    o1 = torch.empty_like(x["q"])
    o2 = torch.empty_like(x["q"])
    l1 = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    rng = np.random.default_rng(12345)
    few = 4 if nqb <= 128 else max(4, int(round(0.05 * nqb)))

    def skewed(n_dense):
        rp, kept = [0], []
        for pr in range(pairs):
            k = nqb if pr % w.q_heads < n_dense else few
            for _ in range(nqb):
                kept.append(np.sort(rng.choice(nqb, size=k, replace=False)).astype(np.int32))
                rp.append(rp[-1] + k)
        return (torch.from_numpy(np.array(rp, np.int32)).cuda(),
                torch.from_numpy(np.concatenate(kept)).cuda())

    def timed(fn, n):
        for _ in range(3):
            fn()
        meds = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            meds.append(e0.elapsed_time(e1) / n)
        return float(np.median(meds))

    patterns = {}
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    wsb, cap = sd.sdattn_select_blocks_workspace(p, bq, bq, budget)
    rp = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
    ci = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    sd.sdattn_select_blocks(p, x["q"], x["k"], bq, bq, budget, rp, ci, cap, None, ws, wsb)
    del ws
    patterns["pooled selection"] = (rp, ci)
    for n in (1, 2, 4):
        patterns[f"{n} dense head{'s' if n > 1 else ''}, others {few} blocks"] = skewed(n)
    swsb = sd.sdattn_block_split_workspace(p, bq, bq)
    sws = torch.empty(swsb, dtype=torch.uint8, device="cuda")
    plan = torch.empty(rows, dtype=torch.int32, device="cuda")
    out = {"kind": "block-sparse forward: dispatch plan vs split rows (online-softmax merge)",
           "workload": w.name, "block": bq, "patterns": {}}
    for name, (rpp, cip) in patterns.items():
        torch.cuda.synchronize()
        nnz = int(rpp[rows].item())
        flops = 4.0 * w.head_dim * bq * bq * nnz
        sd.sdattn_block_plan(p, bq, bq, rpp, plan)
        sd.sdattn_block_split_plan(p, bq, bq, rpp, sws, swsb)
        torch.cuda.synchronize()
        w32 = sws.view(torch.int32)
        cnt = rows + 2 * slots + rows
        cut, T = int(w32[cnt].item()), int(w32[cnt + 1].item())
        n = max(5, min(200, int(2000.0 / max(0.05, flops / 1e12))))
        t_plan = timed(lambda: sd.sdattn_forward_block_sparse_planned(p, x["q"], x["k"], x["v"], bq, bq, rpp, cip,
                                                                      plan, o1, l1), n)
        t_split = timed(lambda: sd.sdattn_forward_block_sparse_split(p, x["q"], x["k"], x["v"], bq, bq, rpp, cip,
                                                                     sws, o2, l2, ws_bytes=swsb), n)
        torch.cuda.synchronize()
        diff = float((o1.float() - o2.float()).abs().max().item())
        rec = {"kept_blocks": nnz, "rows_cut": cut, "chunk_blocks": T,
               "planned_ms": round(t_plan, 4), "split_ms": round(t_split, 4),
               "speedup": round(t_plan / t_split, 3),
               "planned_tflops": round(flops / t_plan / 1e9, 1), "split_tflops": round(flops / t_split / 1e9, 1),
               "max_abs_diff_vs_planned": diff}
        out["patterns"][name] = rec
        log(f"split study {name}: {rec}")
    print(json.dumps(out), flush=True)


def mfma_ceiling(args):
    """The MFMA-only ceiling: a probe kernel (libsdattn_probe.so) that keeps
    its operands in registers and issues nothing but bf16 32x32x16 MFMAs,
    run for a few seconds per operand set (random N(0, 1) values, all zeros,
    all ones) while amd-smi samples power and clock.  Under the package power
    limit the MFMA rate with random operands is what the attention kernels'
    own MFMA work can reach at best; the zeros show the clock-limited peak."""
    import ctypes

    import numpy as np
    import torch

    path = os.path.join(ROOT, "sparse_bidirectional_attention_amd", "libsdattn_probe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run `python -m sparse_bidirectional_attention_amd.build`")
    lib = ctypes.CDLL(path)
    fn = lib.sdattn_probe_mfma_ceiling
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    grid = 768            # three waves per SIMD on 256 CUs
    n_vals = grid * 4 * 8 * 2 * 64 * 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12345)
    sets = {"random": torch.randn(n_vals, generator=gen, device="cuda").to(torch.bfloat16),
            "zeros": torch.zeros(n_vals, dtype=torch.bfloat16, device="cuda"),
            "ones": torch.ones(n_vals, dtype=torch.bfloat16, device="cuda")}
    sink = torch.empty(grid * 4 * 64, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    iters = 4096
    flops = float(grid) * 4 * iters * 8 * 32 * 32 * 16 * 2

    def launch(ops):
        rc = fn(ops.data_ptr(), grid, iters, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    out = {"kind": "MFMA-only probe: v_mfma_f32_32x32x16_bf16 back to back from registers",
           "grid": grid, "iters": iters, "flops_per_launch": flops, "sets": {}}
    for name, ops in sets.items():
        launch(ops)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        launch(ops)
        torch.cuda.synchronize()
        one_ms = max(1e-3, (time.perf_counter() - t0) * 1e3)
        n = max(8, int(math.ceil(args.operand_seconds * 1e3 / one_ms)))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        mon = GpuMonitor()
        if not args.no_gpu_monitor:
            mon.start()
        for e0, e1 in evs:
            e0.record()
            launch(ops)
            e1.record()
        torch.cuda.synchronize()
        mon.stop()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        med = float(np.median(ms))
        tf = flops / (med * 1e9)
        rec = {"launches": n, "median_ms": round(med, 3), "tflops": round(tf, 1),
               "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "gpu_state": mon.summary()}
        gs = rec["gpu_state"]
        if "gfx_clock_mhz" in gs:
            sp = PEAK_BF16_TFLOPS * gs["gfx_clock_mhz"]["median"] / MAX_GFX_CLOCK_MHZ
            rec["peak_at_median_clock_tflops"] = round(sp, 1)
            rec["frac_of_peak_at_median_clock"] = round(tf / sp, 4) if tf <= sp else None
        out["sets"][name] = rec
        log(f"MFMA-only probe, {name} operands: {med:.3f} ms, {tf:.1f} TFLOP/s")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="sparsed_64k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--selector", choices=["pooled", "exact"], default="pooled",
                    help="block workloads: pattern from pooled scores (default) or from the exact block mass of "
                         "the last dense step")
    ap.add_argument("--no-gpu-monitor", action="store_true",
                    help="do not sample power and clocks with amd-smi (e.g. under a profiler)")
    ap.add_argument("--no-sdpa-baseline", action="store_true",
                    help="skip timing torch's own SDPA (flash backend) on the dense step for context")
    ap.add_argument("--no-sweep", action="store_true",
                    help="time only the named workload (by default the 64K headline is followed by the 8K, 16K "
                         "and 32K workloads, reported under 'configs')")
    ap.add_argument("--probe-interval", type=int, default=None,
                    help="adaptive anchors (block workloads): probe the pattern every N steps after the selection")
    ap.add_argument("--min-overlap", type=float, default=0.9,
                    help="with --probe-interval: adopt a probe whose overlap with the cached pattern is below this")
    ap.add_argument("--operand-study", action="store_true",
                    help="instead of the schedule: the dense forward on the workload's inputs, all-zero and all-one "
                         "K/V, each for --operand-seconds, with clock and power (how far operand data moves a "
                         "power-limited kernel)")
    ap.add_argument("--operand-seconds", type=float, default=4.0)
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="run only the MFMA-only probe on three operand sets (random, zeros, ones) and print "
                         "its throughput, clock and power")
    ap.add_argument("--split-study", action="store_true",
                    help="instead of the schedule: the block-sparse forward over the dispatch plan against split "
                         "rows, on head-skewed patterns (dense heads beside sparse ones) and the pooled pattern")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a known-size "
                         "kernel that scales the profiler's HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(sharding the heads across GPUs is not implemented); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    from workloads.configs import LOSA_WORKLOADS
    if args.workload in LOSA_WORKLOADS:
        run_losa(args, LOSA_WORKLOADS[args.workload])
        return

    import torch

    from workloads import get_workload
    from workloads.configs import scaled

    w0 = get_workload(args.workload)
    if args.selector == "exact":
        if w0.selector != "blocks" or w0.dense_steps < 1:
            print("--selector exact needs a block workload with at least one dense step", file=sys.stderr)
            sys.exit(2)
        # the exact mass reads the lse of a dense pass: select on the last dense step at the latest
        w0 = scaled(w0, selector="blocks_exact", refresh_dense=True, select_step=min(w0.select_step, w0.dense_steps - 1))
    if args.probe_interval is not None:
        w0 = scaled(w0, probe_interval=args.probe_interval, min_overlap=args.min_overlap)
    K = args.steps if args.steps is not None else w0.total_steps
    torch.cuda.set_device(0)
    if args.operand_study:
        operand_study(args, w0)
        return
    if args.mfma_ceiling:
        mfma_ceiling(args)
        return
    if args.split_study:
        split_study(args, w0)
        return
    out, (acts, x0h, xsh) = run_schedule(args, w0, K, args.warmup)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(w0, acts, x0h, xsh)
    del x0h, xsh
    sweep = (args.workload == "sparsed_64k" and args.selector == "pooled" and args.probe_interval is None
             and not args.no_sweep and args.copy_calibration_mib == 0)
    if sweep:
        cfgs = {}
        for name in SWEEP:
            wc = get_workload(name)
            # each context runs its own schedule unless --steps fixes K for all
            Kc = args.steps if args.steps is not None else wc.total_steps
            rec, _ = run_schedule(args, wc, Kc, args.warmup, with_gpu_state=False)
            cfgs[name] = compact(rec)
        out["configs"] = cfgs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
