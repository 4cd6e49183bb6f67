"""Benchmark of the R-KV compression step on one MI355X.

A step is one compression event over a whole decode batch: every (sequence,
layer, KV head) unit of a Llama3-8B-shaped cache (batch 64 x 32 layers x 8 KV
heads = 16384 units, N = 1152 candidates = kv_budget 1024 + divide_length
128, window 8, lambda 0.1, GQA group 4, head_dim 128, bf16) is scored,
selected and compacted by rkv_compress. Inputs are synthetic (repeated-segment
keys covering 40% of each sequence, i.i.d. values and queries) and resident in
HBM before timing starts. The line printed reports compressed KV-heads/s, the
roofline of the kernel that takes the most time (measured live with HIP
events around each of its launches in the timed region), and the CPU oracle's
rate on a bounded sample.

python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload llama-event|qwen|llama-layer|decode-loop]
                [--symmetric] [--no-causal] [--pool mean] [--select-group G] [--graph]

The last four select the reading variants (symmetric redundancy, no causal
window, mean pooling over the GQA heads) and head-shared selection over runs
of G consecutive units (G = 8: the KV heads of one layer of one sequence); the
workload name then carries them as a suffix. --graph captures one
compression call in a HIP graph (torch.cuda.CUDAGraph) and times its replays.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressed KV-heads/sec (budget 1024, N=1152, d=128) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

WORKLOADS = {
    "llama-event": dict(cfg=2, name="llama3-8b-decode-event"),
    "qwen": dict(cfg=3, name="qwen-14b"),
    "llama-layer": dict(cfg=1, name="llama3-8b-1layer"),
    "decode-loop": dict(cfg=2, name="llama3-8b-decode-loop"),
    "paged": dict(cfg=4, name="paged-ragged"),
}


# launch labels of the kernels that run the whole dense step in one launch
# (register-resident keys for short units, the LDS tile ring otherwise)
WHOLE_STEP = ("rkv_k2_resident", "rkv_k2_resident2", "rkv_k2_compress")


def whole_step_label(times):
    """The whole-step kernel among the timed launches (None if neither ran)."""
    return next((k for k in WHOLE_STEP if k in times), None)


def kernel_work(name, units, n, b, g, w, esize=2, symmetric=False, group=1):
    """Algorithmic work of one launch of `name`: (bound, amount, unit).

    bytes: K read once for scoring, the window queries, the kept K and V rows
    read, K' and V' written, the indices; flops: the cosine contraction over
    unique pairs, N(N-1)*d per unit (2N(N-1)*d for the symmetric R, which
    needs every ordered pair). The dense redundancy kernel also selects and
    gathers, so it carries both; its bound is the one whose time at peak is
    longer. Under head-shared selection (group > 1) it only scores: K and Q
    read, Z written; selection and gather are launches of their own. The
    statistics kernel is charged its own read of K and Q.
    """
    d = 128
    row = d * esize
    nk = min(n, b)
    flops = units * n * (n - 1) * d * (2 if symmetric else 1)
    if name in WHOLE_STEP:
        if group > 1:
            nbytes = units * (n * row + g * w * row + 4 * n)
        else:
            nbytes = units * bytes_per_unit(n, b, g, w, esize)
        if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
            return "mfma", flops, "flop"
        return "hbm", nbytes, "byte"
    if name == "rkv_k2_redundancy":
        return "mfma", flops, "flop"
    if name == "rkv_k5_gather":
        return "hbm", units * (4 * nk * row + 4 * nk), "byte"
    if name == "rkv_k1_stats":
        return "hbm", units * (n * row + g * w * row), "byte"
    if name == "rkv_k4_select":
        return "hbm", units * (4 * n + 4 * b), "byte"
    if name == "rkv_k4_group_select":
        return "hbm", units * (4 * (n - w) + 4 * b), "byte"
    return None, 0, None


def bytes_per_unit(n, b, g, w, esize=2):
    """Algorithmic HBM bytes of the whole step per unit: K read once for
    scoring, Q_win read, kept K and V rows read, K' and V' written, indices."""
    row = 128 * esize
    nk = min(n, b)
    return n * row + g * w * row + 2 * nk * row + 2 * nk * row + 4 * nk


def add_moved_rate(roof, avg_s):
    """Beside the algorithmic figure: the HBM rate of the bytes the kernel
    actually moved (rocprofv3 counter traffic per launch / the same launch
    time), as GB/s and as a fraction of the HBM peak; absent without traffic."""
    if roof.get("traffic"):
        gbs = roof["traffic"] / avg_s / 1e9
        roof["moved_gbs"] = gbs
        roof["moved_frac"] = gbs / HBM_PEAK_GBS


def source_hash(files):
    """Hash of the sources a kernel is compiled from (its .hip file and headers)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "decode_kv_cache_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_HEADERS = ["rkv_device.hpp", "rkv_problem.hpp", "rkv_launch.hpp"]
KERNEL_SOURCES = {
    "rkv_k2_resident": ["k2_resident.hip", "rkv_resident.hpp", "rkv_frag16.hpp", "rkv_select.hpp",
                        "rkv_stream.hpp"] + _HEADERS,
    "rkv_k2_resident2": ["k2_resident2.hip", "rkv_resident.hpp", "rkv_frag16.hpp", "rkv_select.hpp",
                         "rkv_stream.hpp"] + _HEADERS,
    "rkv_k2_compress": ["k2_wide.hip", "k2_redundancy.hip", "rkv_select.hpp", "rkv_stream.hpp"] + _HEADERS,
    "rkv_k2_redundancy": ["k2_redundancy.hip", "rkv_select.hpp"] + _HEADERS,
    "rkv_k2_long": ["k2_long.hip", "rkv_frag16.hpp", "rkv_stream.hpp"] + _HEADERS,
    "rkv_k1_stats": ["k1_importance.hip"] + _HEADERS,
    "rkv_k1_combine": ["k1_importance.hip"] + _HEADERS,
    "rkv_k4_select": ["k4_select.hip", "rkv_select.hpp"] + _HEADERS,
    "rkv_k4_group_select": ["k4_select.hip", "rkv_select.hpp"] + _HEADERS,
    "rkv_k4_paged_shared": ["k4_shared.hip", "rkv_select.hpp"] + _HEADERS,
    "rkv_k5_gather": ["k5_compact.hip"] + _HEADERS,
    "rkv_k5_paged_compact": ["k5_compact.hip"] + _HEADERS,
    "rkv_free_pages": ["k5_compact.hip"] + _HEADERS,
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on a different version of the kernel's source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
        e = data[workload][kernel]
    except (KeyError, ValueError, OSError):
        return None
    if kernel not in KERNEL_SOURCES or e.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return e.get("bytes_per_launch")


_POOL = {}


def _pool_init(folder, threads_env):
    """Pool worker set-up (fresh interpreter): one BLAS thread, the oracle
    imported, the folder of sampled units noted."""
    os.environ.update(threads_env)
    import numpy  # noqa: F401
    from oracle import rkv_oracle  # noqa: F401
    _POOL["folder"] = folder


def _pool_work(job):
    """The oracle on one worker's share of the sampled units, cycling through
    it until the deadline (wall clock). Returns (units done, seconds busy)."""
    import numpy as np
    from oracle import rkv_oracle as orc
    share, deadline, budgets, window, lam, variant, shared = job
    done, busy, k = 0, 0.0, 0
    while share and time.time() < deadline:
        i = share[k % len(share)]
        k += 1
        Ki, Vi, Qi = (np.load(os.path.join(_POOL["folder"], f"{t}{i}.npy")) for t in "KVQ")
        s = time.perf_counter()
        if shared:
            orc.compress_shared(Ki, Vi, Qi, budgets[i], window, lam, **variant)
        else:
            orc.compress_head(Ki[0], Vi[0], Qi[0], budgets[i], window, lam, **variant)
        busy += time.perf_counter() - s
        done += Ki.shape[0]
    return done, busy


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def pool_workers() -> int:
    """One worker per core this process may run on, at most 16 (the host cores
    that one GPU of a shared node gets)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def run_oracle_pool(units, budgets, window, lam, variant, seconds, shared=False):
    """Time the oracle, as it stands, over a multiprocessing pool.

    units: list of (K, V, Q) float32 host arrays, K and V [h, N, d] and Q
    [h, G, w, d] (h = 1, or the heads of one head-shared group); budgets: the
    budget of each. The pool has one single-BLAS-thread worker per core
    (spawned interpreters, so no GPU state is inherited); after start-up,
    each worker cycles through its share of the units until `seconds` of
    wall clock have passed. Returns (units per second over the pool's wall
    time, workers, units done, distinct units)."""
    import multiprocessing
    import shutil
    import tempfile
    import numpy as np
    folder = tempfile.mkdtemp(prefix="rkv_oracle_")
    try:
        for i, u in enumerate(units):
            for t, arr in zip("KVQ", u):
                np.save(os.path.join(folder, f"{t}{i}.npy"), np.ascontiguousarray(arr, np.float32))
        workers = pool_workers()
        threads_env = {k: "1" for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                        "MKL_NUM_THREADS", "BLIS_NUM_THREADS")}
        saved = {k: os.environ.get(k) for k in threads_env}
        os.environ.update(threads_env)      # inherited by the spawned workers
        try:
            ctx = multiprocessing.get_context("spawn")
            with ctx.Pool(workers, initializer=_pool_init, initargs=(folder, threads_env)) as pool:
                pool.map(abs, range(workers))          # every worker started
                shares = [list(range(w, len(units), workers)) for w in range(workers)]
                t0 = time.perf_counter()
                deadline = time.time() + seconds
                out = pool.map(_pool_work, [(sh, deadline, list(budgets), window, lam, variant,
                                             shared) for sh in shares], chunksize=1)
                wall = time.perf_counter() - t0
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    done = sum(d for d, _ in out)
    return done / wall, workers, done, len(units)


def cpu_baseline(case, seconds=12.0, distinct=256, variant=None, group=1):
    """The oracle as it stands on units drawn from the same cache (copied to
    the host), timed over a pool of single-threaded workers."""
    import numpy as np
    variant = variant or {}
    rng = np.random.default_rng(0)
    order = rng.permutation(case.num_heads // group)[:max(1, distinct // group)]
    units = []
    for gi in order:
        sl = slice(int(gi) * group, (int(gi) + 1) * group)
        units.append((case.K[sl].float().cpu().numpy(), case.V[sl].float().cpu().numpy(),
                      case.Q[sl].float().cpu().numpy()))
    rate, workers, done, m = run_oracle_pool(units, [case.budget] * len(units), case.window,
                                             case.lam, variant, seconds, shared=group > 1)
    what = f"{m} groups of {group} units" if group > 1 else f"{m} units"
    return {"value": rate, "unit": "KV-heads/s", "cores": workers, "kind": "oracle",
            "sample": f"{what} drawn at random from the same {case.num_heads}-unit cache "
                      f"(N={case.n}), float64 numpy oracle, one process per core with one BLAS "
                      f"thread each, cycling through the sample for {seconds:.0f} s of wall "
                      f"clock ({done} units done); CPU: {cpu_model()}"}


def run_decode_loop(args, wl, c, rkv):
    """The whole decode loop of the Llama3-8B-shaped batch: 16,384 steps, each
    appending one row per unit, and a compression event whenever a unit holds
    kv_budget + divide_length rows (120 events). Rows come from the seeded
    counter-based generator, so the loop's inputs are synthetic like the
    others. Reports compressed KV-heads/s of the median event (library HIP
    events around each compression launch) and the loop's wall time."""
    import torch
    from decode_kv_cache_03_amd.decode_loop import DecodeLoop
    from synth.decode_gen import DecodeStream
    steps = c["steps"]
    stream = DecodeStream(wl["cfg"], c["batch"], c["layers"], c["kv_heads"], c["gqa"], steps,
                          coverage=c["coverage"], sigma=c["sigma"], max_back=c["budget"])
    loop = DecodeLoop(stream.units, c["gqa"], kv_budget=c["budget"], window_size=c["window"],
                      divide_length=c["divide_length"], mix_lambda=c["lam"])
    torch.cuda.synchronize()
    rkv.timing_enable(True)
    ev_pairs = []
    t0 = time.perf_counter()
    for t in range(steps):
        k, v, q = stream.rows(t)
        if loop.active and loop.length + 1 == loop.capacity:   # this append compresses
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            loop.append(k, v, q)
            e1.record()
            ev_pairs.append((e0, e1))
        else:
            loop.append(k, v, q)
        if (t + 1) % 2048 == 0:
            print(f"decode loop: step {t + 1}/{steps}, events {loop.events}", file=sys.stderr,
                  flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = rkv.timing_read()
    rkv.timing_enable(False)
    launches, total_ms = times[whole_step_label(times)]
    kern_ms = total_ms / launches
    ev = sorted(a.elapsed_time(b) for a, b in ev_pairs)
    out = {
        "metric": METRIC, "value": stream.units / (kern_ms * 1e-3), "unit": "KV-heads/s",
        "n_gpus": 1, "steps": steps, "warmup": 0, "ms_per_step": kern_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "units": stream.units, "decode_steps": steps,
                   "kv_budget": c["budget"], "divide_length": c["divide_length"],
                   "window_size": c["window"], "mix_lambda": c["lam"], "gqa_group": c["gqa"],
                   "head_dim": 128, "batch": c["batch"], "layers": c["layers"],
                   "kv_heads": c["kv_heads"], "key_repeat_coverage": round(stream.coverage, 4)},
        "events": loop.events, "event_kernel_ms_mean": kern_ms,
        "event_step_ms": {"median": ev[len(ev) // 2], "min": ev[0], "max": ev[-1]},
        "loop_wall_s": wall,
        "note": "ms_per_step is the mean compression kernel time per event; event_step_ms "
                "times a whole compressing decode step (row append, window query reorder, "
                "compression); row generation is outside both",
    }
    print(json.dumps(out))


def run_paged(args, wl, c, rkv, variant):
    """The paged ragged workload: 128 sequences of 2K..32K tokens x 8 KV heads
    in 16-token shuffled pages, compressed in place with page return. The call
    mutates the page pools, the page table and the free list, so all three
    are restored from copies before every step, outside the timed region
    (every step then does the same work); each step is timed with HIP events
    on the call's stream (the host-side planning and the metadata upload it
    enqueues are inside)."""
    import numpy as np
    import torch
    from synth import paged_case_device
    case = paged_case_device(4, c["seqs"], c["kv_heads"], c["gqa"], c["n_min"], c["n_max"],
                             c["frac_min"], c["frac_max"], c["window"], c["lam"], c["dtype"],
                             c["coverage"], c["sigma"], c["page_size"], c["spare_pages"])
    H, ps, w = case.kv_heads, case.page_size, case.window
    table0 = torch.from_numpy(case.page_table).cuda()
    table = table0.clone()
    K0, V0 = case.K_pages.clone(), case.V_pages.clone()
    freed = int(sum(-(-int(n) // ps) - int(b) // ps for n, b in zip(case.seq_len, case.budget)
                    if n > b))
    fl0 = torch.full((len(case.free_list) + freed,), -1, dtype=torch.int32, device="cuda")
    fl0[:len(case.free_list)] = torch.from_numpy(case.free_list.astype(np.int32)).cuda()
    fl = fl0.clone()
    units = case.num_seqs * H
    total_kept = H * int(sum(min(int(a), int(b)) for a, b in zip(case.seq_len, case.budget)))
    kept = torch.empty(total_kept, dtype=torch.int32, device="cuda")

    def step():
        return rkv.compress_paged(case.K_pages, case.V_pages, table, case.seq_len, case.budget,
                                  case.Q, fl, len(case.free_list), w, case.lam, kept_idx=kept,
                                  **variant)

    def restore():
        table.copy_(table0)
        fl.copy_(fl0)
        case.K_pages.copy_(K0)
        case.V_pages.copy_(V0)

    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()
    rkv.timing_enable(True)
    evs = []
    for _ in range(args.steps):
        restore()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    times = rkv.timing_read()
    rkv.timing_enable(False)
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    ms_per_step = sum(ms) / len(ms)
    kernels = {k: {"launches": v[0], "avg_ms": v[1] / max(v[0], 1)} for k, v in times.items()}
    scored = [(int(n), int(b)) for n, b in zip(case.seq_len, case.budget) if n > b]
    pairs = sum(n * (n - 1) for n, _ in scored) * H * (2 if variant.get("symmetric") else 1)
    flops = pairs * 128
    dom = max(times, key=lambda k: times[k][1])
    roof = None
    if dom in ("rkv_k2_redundancy", "rkv_k2_long"):
        achieved = flops / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "kernel": dom,
                "traffic": measured_traffic(dom, wl["name"])}
        add_moved_rate(roof, kernels[dom]["avg_ms"] * 1e-3)
    for k in ("rkv_k2_redundancy", "rkv_k2_long"):
        if k in kernels:
            kernels[k]["tflops"] = flops / (kernels[k]["avg_ms"] * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        # (sequence, head) units of the shorter sequences, read through the
        # page table: the oracle's N^2 loop makes a 32K-token unit minutes long;
        # under head-shared selection, whole sequences (all heads)
        shared = bool(variant.get("shared_heads"))
        ovar = {k: v for k, v in variant.items() if k != "shared_heads"}
        rng = np.random.default_rng(0)
        short = [int(s_) for s_ in rng.permutation(case.num_seqs) if case.seq_len[s_] <= 4096]
        sample, budgets = [], []
        for s_ in short[:(8 if shared else 64)]:
            n = int(case.seq_len[s_])
            t = torch.arange(n, device="cuda")
            pg = table0[s_][t // ps].long()
            hs = list(range(H)) if shared else [int(rng.integers(0, H))]
            sample.append((np.stack([K0[pg, h, t % ps].float().cpu().numpy() for h in hs]),
                           np.stack([V0[pg, h, t % ps].float().cpu().numpy() for h in hs]),
                           np.stack([case.Q[s_, h].float().cpu().numpy() for h in hs])))
            budgets.append(int(case.budget[s_]))
        if sample:
            rate, workers, done, m = run_oracle_pool(sample, budgets, w, case.lam, ovar,
                                                     args.cpu_seconds, shared=shared)
            what = (f"{m} whole sequences ({H} heads each, head-shared selection)" if shared
                    else f"{m} (sequence, head) units")
            cpu = {"value": rate, "unit": "KV-heads/s", "cores": workers, "kind": "oracle",
                   "sample": f"{what} of the sequences with N_s <= 4096, "
                             f"one process per core with one BLAS thread each, cycling for "
                             f"{args.cpu_seconds:.0f} s ({done} units done); the rate "
                             f"overstates the oracle on the whole workload, whose units reach "
                             f"32K tokens; CPU: {cpu_model()}"}
    out = {
        "metric": METRIC, "value": units / (ms_per_step * 1e-3), "unit": "KV-heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["name"], "units": units, "seqs": case.num_seqs, "kv_heads": H,
                   "page_size": ps, "n_min": int(case.seq_len.min()),
                   "n_max": int(case.seq_len.max()), "tokens": int(case.seq_len.sum()),
                   "window_size": w, "mix_lambda": case.lam, "gqa_group": c["gqa"],
                   "head_dim": 128, "pool_pages": int(case.meta["pool"])},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
        "step_ms": {"median": ms[len(ms) // 2], "min": ms[0], "max": ms[-1]},
        "note": "page pools, page table and free list restored before every step, outside the "
                "timed region",
    }
    print(json.dumps(out))


def memory_ceilings():
    """What plain torch operations reach on this part, as a yardstick for the
    kernels' rates: device copy (read + write), fill (write only) and a
    random gather of 256-byte rows (read + write), at 0.5, 2 and 8 GiB, each
    timed with HIP events over 10 calls after 3 untimed ones. One JSON line."""
    import torch
    out = []

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    for gib in (0.5, 2, 8):
        n = int(gib * 2**30) // 2
        a = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
        b = torch.empty_like(a)
        idx = torch.randperm(n // 128, device="cuda")
        rows_a, rows_b = a.view(-1, 128), b.view(-1, 128)
        out.append({"gib": gib,
                    "copy_tbs": 2 * n * 2 / timed(lambda: b.copy_(a)) / 1e12,
                    "fill_tbs": n * 2 / timed(lambda: b.fill_(1.0)) / 1e12,
                    "row_gather_tbs": 2 * n * 2 / timed(
                        lambda: torch.index_select(rows_a, 0, idx, out=rows_b)) / 1e12})
        del a, b, idx, rows_a, rows_b
    print(json.dumps({"memory_ceilings": out, "unit": "TB/s (bytes read + written / time)"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama-event", choices=sorted(WORKLOADS))
    ap.add_argument("--lam", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock seconds of the oracle pool behind cpu_baseline")
    ap.add_argument("--symmetric", action="store_true", help="R over every other candidate")
    ap.add_argument("--no-causal", action="store_true", help="window queries see all candidates")
    ap.add_argument("--pool", default="max", choices=["max", "mean"], help="GQA pooling of I")
    ap.add_argument("--select-group", type=int, default=1,
                    help="head-shared selection over runs of this many consecutive units")
    ap.add_argument("--graph", action="store_true",
                    help="capture the compression call in a HIP graph and time its replays")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure plain copy, fill and random row-gather rates of this part")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy kernel three times, so "
                         "memory counters can be scaled against a known byte count")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the compression step is per-unit independent and "
              f"the library has no multi-GPU path); got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_kv_cache_03_amd as rkv
    from synth import CONFIGS, dense_case_device

    if args.ceilings:
        memory_ceilings()
        return
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 2,
                          "copy_calibration_bytes_written": dst.numel() * 2}), file=sys.stderr)
        del src, dst

    wl = dict(WORKLOADS[args.workload])
    c = CONFIGS[wl["cfg"]]
    variant = dict(symmetric=args.symmetric, causal=not args.no_causal, pool=args.pool)
    group = max(1, args.select_group)
    suffix = "".join(s for s, on in (("+symmetric", args.symmetric), ("+no-causal", args.no_causal),
                                     ("+pool-mean", args.pool == "mean"),
                                     (f"+shared{group}", group > 1)) if on)
    if suffix and args.workload == "decode-loop":
        print("the decode-loop workload runs the default readings only", file=sys.stderr)
        sys.exit(2)
    wl["name"] += suffix
    if args.workload == "decode-loop":
        run_decode_loop(args, wl, c, rkv)
        return
    if args.workload == "paged":
        if group > 1:
            # on pages the group is a sequence's KV heads (they share its pages)
            if group != c["kv_heads"]:
                print(f"on pages, head-shared selection groups the {c['kv_heads']} KV heads of a "
                      f"sequence (--select-group {c['kv_heads']})", file=sys.stderr)
                sys.exit(2)
            variant = dict(variant, shared_heads=True)
        run_paged(args, wl, c, rkv, variant)
        return
    lam = args.lam if args.lam is not None else c.get("lam", 0.1)
    torch.cuda.set_device(0)
    case = dense_case_device(wl["cfg"], c["batch"], c["layers"], c["kv_heads"], c["gqa"], c["n"],
                             c["budget"], c["window"], lam, c["dtype"], c["coverage"], c["sigma"])
    units, n, b, g, w = case.num_heads, case.n, case.budget, case.gqa, case.window
    K_out = torch.empty((units, b, 128), dtype=case.K.dtype, device="cuda")
    V_out = torch.empty_like(K_out)
    kept = torch.empty((units, b), dtype=torch.int32, device="cuda")
    ws = torch.empty(rkv.workspace_size(units, n, g, w, b, select_group=group), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()

    def call():
        rkv.compress(case.K, case.V, case.Q, b, w, lam, K_out=K_out, V_out=V_out, kept_idx=kept,
                     workspace=ws, select_group=group, **variant)

    step = call
    graph_label = "graph_replay"
    if args.graph:
        # the label of the one launch a single-unit-selection call makes on
        # the dense bf16 path, from an eager call (replays carry no events)
        rkv.timing_enable(True)
        call()
        torch.cuda.synchronize()
        eager = rkv.timing_read()
        rkv.timing_enable(False)
        if len(eager) == 1 and whole_step_label(eager) is not None:
            graph_label = whole_step_label(eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        step = graph.replay
        wl["name"] += "+graph"

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rkv.timing_enable(True)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if args.graph:
            # replays carry no library events: time each on the stream it runs on
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            evs.append((e0, e1))
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    times = rkv.timing_read()
    rkv.timing_enable(False)
    if args.graph:
        times = {graph_label: (len(evs), sum(a.elapsed_time(b_) for a, b_ in evs))}

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = units / (ms_per_step * 1e-3)
    kernels = {k: {"launches": v[0], "avg_ms": v[1] / max(v[0], 1)} for k, v in times.items()}
    dom = max(times, key=lambda k: times[k][1])
    bound, amount, _ = kernel_work(dom, units, n, b, g, w, symmetric=args.symmetric, group=group)
    avg_s = kernels[dom]["avg_ms"] * 1e-3
    if bound == "mfma":
        achieved = amount / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
    else:
        achieved = amount / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(dom, wl["name"])
    add_moved_rate(roof, avg_s)
    for k, v in kernels.items():
        kb, amt, _ = kernel_work(k, units, n, b, g, w, symmetric=args.symmetric, group=group)
        if kb == "mfma":
            v["tflops"] = amt / (v["avg_ms"] * 1e-3) / 1e12
        elif kb == "hbm":
            v["gbs"] = amt / (v["avg_ms"] * 1e-3) / 1e9
        if k in WHOLE_STEP:   # the contraction it also carries
            pairs = n * (n - 1) * (2 if args.symmetric else 1)
            v["tflops"] = units * pairs * 128 / (v["avg_ms"] * 1e-3) / 1e12
            v["mfma_frac"] = v["tflops"] / MFMA_BF16_PEAK_TFLOPS

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, seconds=args.cpu_seconds, variant=variant, group=group)

    step_bytes = units * bytes_per_unit(n, b, g, w)
    out = {
        "metric": METRIC, "value": value, "unit": "KV-heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "units": units, "n_cand": n, "kv_budget": b,
                   "window_size": w, "mix_lambda": lam, "gqa_group": g, "head_dim": 128,
                   "batch": c["batch"], "layers": c["layers"], "kv_heads": c["kv_heads"],
                   "key_repeat_coverage": round(case.meta["coverage"], 4),
                   "symmetric": args.symmetric, "causal_window": not args.no_causal,
                   "gqa_pool": args.pool, "select_group": group},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "step_algorithmic_gb": step_bytes / 1e9,
        "step_effective_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
