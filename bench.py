"""Benchmark of one rank's FlatParameter shard step on one MI355X.

Workload: the Llama-7B-shaped block unit (q/k/v/o 4096x4096, gate/up
11008x4096, down 4096x11008, two 4096 norms; 202,383,360 params) as one
FlatParameter, sharding factor F=8, rank 0 (shard of 25,297,920 params),
8 bf16 gradient rows ~N(0, 1e-3), fp32 master ~N(0, 0.02), AdamW lr 1e-4,
betas 0.9/0.999, eps 1e-8, wd 0.01. Inputs are synthetic (datagen) and
resident in HBM before the timed region.

One step = the whole per-unit hot path of the rank:
  1. fsdp_reduce_adamw_shard: fp32 reduce of the 8 bf16 rows into the shard,
     AdamW on fp32 master/m/v in place, bf16 emission of the new parameter;
  2. fsdp_cast_unflatten: the all-gather arithmetic, F bf16 shards (this
     rank's just emitted) -> the 9 per-tensor bf16 parameters.
(The indexer and the flatten/pad of the master weights run once at init.)

Prints one JSON line. value = shard params/s (shard_valid per step / step
time, the wall clock over the --steps headline steps); roofline = the fused
kernel's algorithmic bytes / its average duration over a sample of at least
64 further in-step launches, each bracketed by HIP events on its stream (the
same sample is taken on rank F-1); stream_mix_ceiling = the same loads and
stores without the AdamW arithmetic (a reference kernel under tests/probes),
timed the same way; cpu_baseline = the CPU oracle on a bounded sample of the
same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_reduce_adamw_blk7_f8_traffic.md")
KERNEL_SRC = os.path.join(ROOT, "sharded_flatparameter_flatten_amd", "csrc", "kernels.hip")
METRIC = "shard step params/s + HBM GB/s (% of peak), 7B-block unit at F=8"


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per fused launch from the committed counter summary, if current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernels_hip_sha256_16") != kernel_source_hash():
        return None           # kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def device_record():
    """Marketing name, ISA, CU count and peak engine clock of GPU agent 0, from rocminfo.

    Runs before this process touches the GPU."""
    import subprocess
    rec = {}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError) as e:
        return {"error": f"rocminfo: {e}"}
    for block in re.split(r"^\s*Agent \d+\s*$", out, flags=re.M)[1:]:
        if not re.search(r"^\s*Device Type:\s*GPU\s*$", block, re.M):
            continue
        for key, name in (("Marketing Name", "marketing_name"), ("Name", "isa"),
                          ("Compute Unit", "compute_units"),
                          ("Max Clock Freq. (MHz)", "max_clock_mhz")):
            m = re.search(r"^[ \t]*" + re.escape(key) + r":[ \t]*(.*?)[ \t]*$", block, re.M)
            if m:
                rec[name] = m.group(1)
        break
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers() -> int:
    """Host cores to use: the process's CPU set, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_worker(F: int, rank: int, first: int, n: int, budget_s: float):
    """One worker of the all-cores oracle run: the fused oracle step on shard
    elements [first, first + n), repeated for budget_s; prints its rate."""
    import numpy as np

    import datagen
    from datagen import workloads as W
    from oracle import fsdp_oracle as O

    L = O.unit_layout(W.shapes(W.BLK7), F, rank)
    g = L.shard_begin + first + np.arange(n, dtype=np.int64)
    grads = [datagen.bf16_bits_host(datagen.seed_for(1, 1, 1), k, g, W.GRAD_SIGMA)
             for k in range(F)]
    p = datagen.normal_f32_host(datagen.seed_for(1, 0), 0, g, W.MASTER_SIGMA)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    one = O.unit_layout([(n,)], 1, 0)
    hp = O.AdamW(**W.ADAMW)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.reduce_adamw_shard(grads, one, p, m, v, hp, 1, grad_scale=1.0 / F, emit_bf16=True)
        reps += 1
        el = time.perf_counter() - t0
        if reps >= 2 and el >= budget_s:
            break
    print(json.dumps({"elements": n * reps, "seconds": el}), flush=True)


def cpu_all_cores(F: int, rank: int, per_worker: int, budget_s: float):
    """The oracle on every host core: one single-threaded worker process per
    core, each on its own stretch of the shard, started together."""
    import subprocess
    from oracle import fsdp_oracle as O
    from datagen import workloads as W

    valid = O.unit_layout(W.shapes(W.BLK7), F, rank).shard_valid
    k = cpu_workers()
    n = max(1, min(per_worker, valid // k))
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker",
                               str(F), str(rank), str(j * n), str(n), str(budget_s)],
                              stdout=subprocess.PIPE, text=True, env=env) for j in range(k)]
    rate = 0.0
    for pr in procs:
        out, _ = pr.communicate(timeout=budget_s * 10 + 120)
        if pr.returncode != 0:
            return None
        r = json.loads(out.strip().splitlines()[-1])
        rate += r["elements"] / r["seconds"]
    return {"value": rate, "cores": k, "elements_per_worker": n}


def cpu_baseline(F: int, rank: int, sample: int, budget_s: float):
    """The CPU oracle (as it stands) on the first `sample` elements of the shard."""
    import numpy as np

    import datagen
    from datagen import workloads as W
    from oracle import fsdp_oracle as O

    L = O.unit_layout(W.shapes(W.BLK7), F, rank)
    n = min(sample, L.shard_valid)
    g = L.shard_begin + np.arange(n, dtype=np.int64)
    grads = [datagen.bf16_bits_host(datagen.seed_for(1, 1, 1), k, g, W.GRAD_SIGMA)
             for k in range(F)]
    p = datagen.normal_f32_host(datagen.seed_for(1, 0), 0, g, W.MASTER_SIGMA)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    one = O.unit_layout([(n,)], 1, 0)
    hp = O.AdamW(**W.ADAMW)

    def rate(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if reps >= 3 and el >= budget:
                return n * reps / el, reps, el

    value, reps, el = rate(lambda: O.reduce_adamw_shard(grads, one, p, m, v, hp, 1,
                                                        grad_scale=1.0 / F, emit_bf16=True),
                           budget_s)
    g = O.reduce_shard(grads, one, grad_scale=1.0 / F)
    rows = {
        "a3_reduce_shard": rate(lambda: O.reduce_shard(grads, one, grad_scale=1.0 / F), 2.0)[0],
        "a4_adamw_shard_emit": rate(lambda: O.adamw_step(g, p, m, v, hp, 1, emit_bf16=True),
                                    2.0)[0],
        "a6_bf16_round": rate(lambda: O.bf16_round_nearest_even(p), 2.0)[0],
    }
    allc = cpu_all_cores(F, rank, 1 << 20, budget_s)
    per_param = 2 * F + 26
    res = {
        "value": value, "unit": "params/s", "cores": 1, "kind": "oracle",
        "sample": (f"fused reduce+AdamW+bf16 emit of the CPU oracle (numpy, one thread) on the "
                   f"first {n:,} elements of rank {rank}'s shard of the 7B block at F={F}, "
                   f"{reps} repetitions, {el:.1f} s"),
        "GBps": value * per_param / 1e9,
        "cpu_model": cpu_model(),
        "rows_params_per_s": rows,
    }
    if allc is not None:
        res["all_cores"] = {
            "value": allc["value"], "unit": "params/s", "cores": allc["cores"],
            "GBps": allc["value"] * per_param / 1e9,
            "sample": (f"the same oracle step in {allc['cores']} single-threaded processes at "
                       f"once, each on its own {allc['elements_per_worker']:,} shard elements, "
                       f"about {budget_s:.0f} s each"),
        }
    return res


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence, with the
    record / elapsed_time interface of torch.cuda.Event.

    torch's events record with a system-scope fence (cache write-back and
    invalidation when the event completes); HIP documents disabling it for
    events used only to measure time, as it improves the accuracy of the
    measurement on AMD GPUs and costs the stream less. Measured on the 7B-block
    step: the fused kernel's event interval is 166.0 us with these events and
    167.3 us with torch's, against 163.5 us of kernel time in a rocprofv3 trace
    of the same loop."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")     # the runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        st = self._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream=None):
        import torch
        s = (stream or torch.cuda.current_stream()).cuda_stream
        st = self._hip.hipEventRecord(self.h, self._ct.c_void_p(s))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._ct.c_float()
        st = self._hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)
            self.h = None


def spread(ms):
    """Average, median, 10th and 90th percentile and minimum of event intervals, in us."""
    xs = sorted(x * 1e3 for x in ms)

    def pct(q):
        i = q * (len(xs) - 1)
        lo = int(i)
        hi = min(lo + 1, len(xs) - 1)
        return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)

    return {"avg": sum(xs) / len(xs), "median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9),
            "min": xs[0]}


def rotating_rows(torch, datagen, W, unit, n_rows, n_sets, dev, seed, outlier_seed=None,
                  separate=False):
    """n_sets sets of n_rows gradient rows whose rank windows are all disjoint.

    The kernels read only [shard_begin, shard_begin + shard_valid) of a row.
    separate=True: every row is its own U-element allocation (one buffer per
    contributing rank, as the ranks' gradients are), only its window filled.
    Otherwise each row is a U-long view into one arena, placed so that its
    window lands on its own stretch of the arena: R*n_rows*S elements are
    filled and allocated instead of R*n_rows*U allocated.
    """
    S, U, r0 = unit.S, unit.U, unit.shard_begin
    if separate:
        out = []
        for j in range(n_sets):
            rows = []
            for k in range(n_rows):
                row = torch.empty(U, dtype=torch.bfloat16, device=dev)
                datagen.fill_bf16_(row[r0:r0 + unit.shard_valid], seed, 64 * j + k,
                                   W.GRAD_SIGMA, start=r0, outlier_seed=outlier_seed)
                rows.append(row)
            out.append(rows)
        return out
    S8 = (S + 7) // 8 * 8          # window spacing that keeps every row base 16-byte aligned
    arena = torch.empty(r0 + n_sets * n_rows * S8 + U, dtype=torch.bfloat16, device=dev)
    out = []
    for j in range(n_sets):
        rows = []
        for k in range(n_rows):
            w0 = r0 + (j * n_rows + k) * S8           # window start in the arena
            row = arena[w0 - r0:w0 - r0 + U]
            datagen.fill_bf16_(row[r0:r0 + unit.shard_valid], seed, 64 * j + k, W.GRAD_SIGMA,
                               start=r0, outlier_seed=outlier_seed)
            rows.append(row)
        out.append(rows)
    return out


def make_sets(fsdp, torch, datagen, W, units, rank, R, dev, separate=True, keep_masters=True):
    """R independent buffer sets of the 7B-block step for `rank`: gradient rows
    (that rank's window filled), fp32 master (flattened from per-tensor draws),
    m, v, every rank's bf16 shard, and the 9 bf16 outputs of the gather."""
    u = units[rank]
    F, S = u.F, u.S
    shapes = u.shapes
    row_sets = rotating_rows(torch, datagen, W, u, F, R, dev, datagen.seed_for(1, 1, 1),
                             separate=separate)
    sets, set_masters = [], []
    for j in range(R):
        masters = []
        for i, nel in enumerate(u.numels):
            t = torch.empty(nel, dtype=torch.float32, device=dev)
            datagen.fill_normal_f32_(t, datagen.seed_for(1, 0), 256 * j + i, W.MASTER_SIGMA)
            masters.append(t)
        p = torch.empty(S, dtype=torch.float32, device=dev)
        fsdp.flatten_pad(u, masters, p)                   # init: flatten + pad (once)
        masters_bf16 = [t.to(torch.bfloat16) for t in masters]
        shards = []
        for r in range(F):                                # every rank's bf16 parameter shard
            sh = torch.empty(S, dtype=torch.bfloat16, device=dev)
            fsdp.flatten_pad(units[r], masters_bf16, sh)
            shards.append(sh)
        del masters_bf16
        m = torch.zeros(S, dtype=torch.float32, device=dev)
        v = torch.zeros(S, dtype=torch.float32, device=dev)
        outs = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in shapes]
        sets.append((row_sets[j], p, m, v, shards, outs))
        set_masters.append(masters if keep_masters else None)
    return sets, set_masters


def bracketed_steps(torch, stream, fused, gather, first, L):
    """L steps (fused, then gather) with each kernel bracketed by HIP events on
    `stream`; returns the fused and gather intervals in ms."""
    ev = [[TimingEvent() for _ in range(3)] for _ in range(L)]
    torch.cuda.synchronize()
    for i in range(L):
        ev[i][0].record(stream)
        fused(first + i)
        ev[i][1].record(stream)
        gather(first + i)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    return ([e[0].elapsed_time(e[1]) for e in ev], [e[1].elapsed_time(e[2]) for e in ev])


STREAM_MIX_LIB = os.path.join(ROOT, "tests", "probes", "libstreammix.so")


def stream_mix_leg(torch, stream, sets, u, rank, F, gather, first, L):
    """The stream-mix reference kernel in the step loop (see stream_mix_probe.hip),
    or None when it is not built or the workload is not 8 rows on a 4-aligned shard."""
    import ctypes
    n = u.shard_valid
    if F != 8 or n % 4 or (2 * u.shard_begin) % 8 or not os.path.exists(STREAM_MIX_LIB):
        return None
    lib = ctypes.CDLL(STREAM_MIX_LIB)
    lib.probe_stream_mix.restype = ctypes.c_int
    lib.probe_stream_mix.argtypes = [ctypes.POINTER(ctypes.c_void_p)] + [ctypes.c_void_p] * 4 + \
        [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    # the library's shape for this launch: one-wave workgroups, 10 per CU (the
    # staged fused step's count)
    threads, wg_per_cu = 64, 10
    R = len(sets)
    rows = []
    for grads, p, m, v, shards, outs in sets:
        arr = (ctypes.c_void_p * 8)(*[g.data_ptr() + 2 * u.shard_begin for g in grads])
        rows.append((arr, p.data_ptr(), m.data_ptr(), v.data_ptr(), shards[rank].data_ptr()))

    def mix(i):
        arr, p, m, v, w = rows[i % R]
        st = lib.probe_stream_mix(arr, p, m, v, w, n, threads, wg_per_cu, stream.cuda_stream)
        if st:
            raise RuntimeError(f"probe_stream_mix returned {st}")

    for i in range(R):
        mix(first + i)
        gather(first + i)
    f, _ = bracketed_steps(torch, stream, mix, gather, first, L)
    return {"kernel": "stream-mix reference (8 bf16 row reads, 3 fp32 reads, 3 fp32 + 1 bf16 "
                      "writes per element; no AdamW arithmetic)",
            "threads": threads, "wg_per_cu": wg_per_cu, "launches_timed": len(f),
            "us": spread(f)}


CALIB_ELEMS = 1 << 28          # fp32 elements of the calibration copy (1 GiB)


def copy_reference(fsdp, torch, dev, stream, reps=10):
    cu = fsdp.Unit([(CALIB_ELEMS,)], 1, 0)
    src = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        fsdp.flatten_pad(cu, [src], dst, stream=stream)
    c0, c1 = TimingEvent(), TimingEvent()
    c0.record(stream)
    for _ in range(reps):
        fsdp.flatten_pad(cu, [src], dst, stream=stream)
    c1.record(stream)
    torch.cuda.synchronize()
    return 2 * 4 * CALIB_ELEMS * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9


def torch_copy_reference(torch, dev, reps=2):
    """torch's own device copy of 1 GiB of fp32 (a known-size transfer that
    shares no code with the library); returns GB/s."""
    src = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = TimingEvent(), TimingEvent()
    c0.record()
    for _ in range(reps):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    return 2 * 4 * CALIB_ELEMS * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9


def model_sequence(args):
    """Whole-model rank shard: one step = fused reduce+AdamW+bf16 emit for every unit in order."""
    import torch

    import datagen
    import sharded_flatparameter_flatten_amd as fsdp
    from datagen import workloads as W

    wl = W.WORKLOADS[args.workload]
    F, rank = wl["F"], wl["rank"]
    dev = torch.device("cuda:0")
    units = [fsdp.Unit(W.shapes(u), F, rank) for u in wl["units"]]
    starts = [0]
    for u in units:
        starts.append(starts[-1] + u.S)
    total = starts[-1]
    print(f"# workload {args.workload}: {len(units)} units, shard {total:,} params", file=sys.stderr,
          flush=True)
    # Optimizer state: by default every unit's fp32 master / m / v and bf16
    # parameter shard are windows side by side in one allocation per array (one
    # flat state buffer per rank); --state-layout per-unit gives each unit's
    # arrays their own allocations instead.
    mseed = datagen.seed_for(wl["config"], 0)
    if args.state_layout == "packed":
        p = torch.empty(total, dtype=torch.float32, device=dev)
        datagen.fill_normal_f32_(p, mseed, 0, W.MASTER_SIGMA)
        m = torch.zeros(total, dtype=torch.float32, device=dev)
        v = torch.zeros(total, dtype=torch.float32, device=dev)
        w = torch.empty(total, dtype=torch.bfloat16, device=dev)
        win = [(p[a:a + u.S], m[a:a + u.S], v[a:a + u.S], w[a:a + u.S])
               for u, a in zip(units, starts)]
    else:
        win = []
        for i, u in enumerate(units):
            pu = torch.empty(u.S, dtype=torch.float32, device=dev)
            datagen.fill_normal_f32_(pu, mseed, i, W.MASTER_SIGMA)
            win.append((pu, torch.zeros_like(pu), torch.zeros_like(pu),
                        torch.empty(u.S, dtype=torch.bfloat16, device=dev)))
    gseed = datagen.seed_for(wl["config"], 1, 1)
    # Gradient rows: `row_sets` sets of F rows per distinct unit size, unit i of
    # that size using set i % row_sets, so that consecutive units never read the
    # same rows (a unit's rows are re-read only after other units' traffic has
    # gone through the memory-side cache). Only the rank windows are filled.
    arenas = {}
    for u in units:
        if u.U not in arenas:
            sets = []
            for j in range(args.row_sets):
                rows = [torch.empty(u.U, dtype=torch.bfloat16, device=dev) for _ in range(F)]
                for k in range(F):
                    datagen.fill_bf16_(rows[k][u.shard_begin:u.shard_begin + u.shard_valid],
                                       gseed, 100 * len(arenas) + 16 * j + k, W.GRAD_SIGMA,
                                       start=u.shard_begin)
                sets.append(rows)
            arenas[u.U] = sets
    seen = {}
    unit_rows = []
    for u in units:
        j = seen.get(u.U, 0)
        seen[u.U] = j + 1
        unit_rows.append(arenas[u.U][j % args.row_sets])
    hp = fsdp.AdamWHparams(**W.ADAMW)
    stream = torch.cuda.current_stream(dev)

    batch = [(u, rows) + tuple(wn) for u, rows, wn in zip(units, unit_rows, win)]

    def step(t):
        if args.per_unit:
            for u, rows, (pp, mm, vv, ww) in zip(units, unit_rows, win):
                fsdp.reduce_adamw_shard(u, rows, pp, mm, vv, ww, hp, t, stream=stream)
        else:
            fsdp.reduce_adamw_units(batch, hp, t, stream=stream)

    for i in range(args.warmup):
        step(i + 1)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = TimingEvent(), TimingEvent()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(args.warmup + i + 1)
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / K
    valid = sum(u.shard_valid for u in units)
    nbytes = sum((2 * F + 26) * u.shard_valid for u in units)
    res = {
        "metric": "model shard step params/s + HBM GB/s", "workload": args.workload,
        "value": valid / (ms_step * 1e-3), "unit": "params/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_step, "wall_ms_per_step": elapsed * 1e3 / K,
        "units": len(units), "shard_params": valid, "row_sets": args.row_sets,
        "state_layout": args.state_layout,
        "entry_point": "fsdp_reduce_adamw_shard per unit" if args.per_unit
        else "fsdp_reduce_adamw_units (batched launches)",
        "persistent_bytes": sum(u.persistent_bytes for u in units),
        "algorithmic_bytes_per_step": nbytes, "GBps": nbytes / (ms_step * 1e-3) / 1e9,
        "frac_of_8TBps": nbytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "dtype": "f32", "data": "synthetic",
    }
    print(json.dumps(res), flush=True)


def sharding_sweep(args):
    """Fused reduce+AdamW+emit on ranks 0 and F-1 of the 7B block for each F of the sweep,
    visiting `--rotate` independent buffer sets in turn (gradient rows laid out as
    --row-layout says; "both": each rank in the separate layout, then in the arena)."""
    import torch

    import datagen
    import sharded_flatparameter_flatten_amd as fsdp
    from datagen import workloads as W

    wl = W.WORKLOADS["sweep"]
    dev = torch.device("cuda:0")
    shapes = W.shapes(W.BLK7)
    Fs = wl["Fs"] + wl["padded_Fs"]
    R = args.rotate
    gseed, oseed = datagen.seed_for(wl["config"], 1, 1), datagen.seed_for(wl["config"], 2, 1)
    hp = fsdp.AdamWHparams(**W.ADAMW)
    stream = torch.cuda.current_stream(dev)
    out = []
    layouts = ["separate", "arena"] if args.row_layout == "both" else [args.row_layout]
    for F, rank, layout in ((F, rank, layout) for F in Fs for rank in sorted({0, F - 1})
                            for layout in layouts):
            u = fsdp.Unit(shapes, F, rank)
            rows = rotating_rows(torch, datagen, W, u, F, R, dev, gseed, outlier_seed=oseed,
                                 separate=layout == "separate")
            state = []
            for j in range(R):
                p = torch.empty(u.S, dtype=torch.float32, device=dev)
                datagen.fill_normal_f32_(p, datagen.seed_for(wl["config"], 0), j, W.MASTER_SIGMA)
                state.append((p, torch.zeros_like(p), torch.zeros_like(p),
                              torch.empty(u.S, dtype=torch.bfloat16, device=dev)))

            def fused(i):
                p, m, v, w = state[i % R]
                fsdp.reduce_adamw_shard(u, rows[i % R], p, m, v, w, hp, i // R + 1,
                                        stream=stream)

            W0 = max(args.warmup, R)
            for i in range(W0):
                fused(i)
            K = max(args.steps, 2 * R)
            ev = [TimingEvent() for _ in range(K + 1)]
            ev[0].record(stream)
            for i in range(K):
                fused(W0 + i)
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(K))
            avg = sum(us) / len(us)
            nbytes = (2 * F + 26) * u.shard_valid
            out.append({"F": F, "rank": rank, "S": u.S, "valid": u.shard_valid,
                        "row_path": "vector" if (2 * u.shard_begin) % 8 == 0 else "shifted",
                        "row_layout": layout,
                        "rotating_sets": R,
                        "fused_us_avg": avg, "fused_us_median": us[len(us) // 2],
                        "bytes": nbytes, "GBps": nbytes / (avg * 1e-6) / 1e9,
                        "frac_of_8TBps": nbytes / (avg * 1e-6) / 1e9 / PEAK_HBM_GBPS})
            print(json.dumps(out[-1]), file=sys.stderr, flush=True)
            del rows, state
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "fused shard step per sharding factor", "workload": "sweep",
                      "rows": out}), flush=True)


def hybrid_bench(args):
    """Hybrid sharding on the 7B block: R = 2 replica groups of F = 8, rank 0, fused step."""
    import torch

    import datagen
    import sharded_flatparameter_flatten_amd as fsdp
    from datagen import workloads as W

    dev = torch.device("cuda:0")
    shapes, F, Rg, rank = W.shapes(W.BLK7), 8, 2, 0
    u = fsdp.Unit(shapes, F, rank)
    R = args.rotate
    rows = rotating_rows(torch, datagen, W, u, Rg * F, R, dev, datagen.seed_for(17, 1, 1))
    state = []
    for j in range(R):
        p = torch.empty(u.S, dtype=torch.float32, device=dev)
        datagen.fill_normal_f32_(p, datagen.seed_for(17, 0), j, W.MASTER_SIGMA)
        state.append((p, torch.zeros_like(p), torch.zeros_like(p),
                      torch.empty(u.S, dtype=torch.bfloat16, device=dev)))
    hp = fsdp.AdamWHparams(**W.ADAMW)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, fn in (("hybrid", lambda i: fsdp.reduce_adamw_shard_hybrid(
                          u, Rg, rows[i % R], *state[i % R], hp, 2, stream=stream)),
                     ("flat_16_rows", lambda i: fsdp.reduce_adamw_shard(
                          u, rows[i % R], *state[i % R], hp, 2, stream=stream)),
                     ("flat_16_rows_bf16_partials", lambda i: fsdp.reduce_adamw_shard_bf16acc(
                          u, rows[i % R], *state[i % R], hp, 2, stream=stream))):
        for i in range(max(args.warmup, R)):
            fn(i)
        K = max(args.steps, 2 * R)
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        for i in range(K):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        nbytes = (2 * Rg * F + 26) * u.shard_valid
        res[name] = {"us": us, "bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                     "frac_of_8TBps": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    print(json.dumps({"metric": "hybrid-sharding and bf16-partials fused shard step (16 rows)",
                      "workload": "7B block unit, F=8, 2 replica groups, rank 0",
                      "rotating_sets": R, **res}), flush=True)


def state_dict_bench(args):
    """Full-state-dict export (F fp32 shards -> whole fp32 tensors, for master, m and v)
    and resume (whole tensors -> this rank's fp32 shard) on the 7B block at F=8."""
    import torch

    import datagen
    import sharded_flatparameter_flatten_amd as fsdp
    from datagen import workloads as W

    dev = torch.device("cuda:0")
    shapes, F = W.shapes(W.BLK7), 8
    units = [fsdp.Unit(shapes, F, r) for r in range(F)]
    U, S = units[0].U, units[0].S
    R = args.rotate
    sets = []
    for j in range(R):
        shards = []
        for kind in range(3):
            row = []
            for r in range(F):
                t = torch.empty(S, dtype=torch.float32, device=dev)
                datagen.fill_normal_f32_(t, datagen.seed_for(16, 0), 100 * j + 10 * kind + r, 0.02)
                row.append(t)
            shards.append(row)
        whole = [[torch.empty(sh, dtype=torch.float32, device=dev) for sh in shapes]
                 for _ in range(3)]
        back = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(3)]
        sets.append((shards, whole, back))
    stream = torch.cuda.current_stream(dev)

    def export(i):
        shards, whole, _ = sets[i % R]
        for kind in range(3):
            fsdp.unflatten(units[0], shards[kind], whole[kind], stream=stream)

    def resume(i):
        _, whole, back = sets[i % R]
        for kind in range(3):
            fsdp.flatten_pad(units[0], whole[kind], back[kind], stream=stream)

    res = {}
    for name, fn, nbytes in (("export", export, 3 * 8 * U), ("resume", resume, 3 * 8 * S)):
        for i in range(max(args.warmup, R)):
            fn(i)
        K = max(args.steps, 2 * R)
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        for i in range(K):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        res[name] = {"us": us, "bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                     "frac_of_8TBps": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    print(json.dumps({"metric": "full-state-dict export/resume (fp32 master, m, v)",
                      "workload": "7B block unit, F=8, rank 0", "rotating_sets": R, **res}),
          flush=True)


def _counter_rows(path):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {path}")
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum",
                 "TCC_EA0_RDREQ_DRAM_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum")
READ_REQUEST_BYTES = 128     # gfx950 L2 -> memory read request (see pmc_summary)


def _dispatch_counters(rows, match):
    """{dispatch id: {counter: value summed over instances}} for kernels matching `match`."""
    acc = {}
    for r in rows:
        if not match(r.get("Kernel_Name", "")):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        d = acc.setdefault(key, {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return acc


def _request_bytes(rd, wr):
    """HBM bytes of one dispatch from the raw L2 <-> memory request counts:
    reads are 128-byte requests (TCC_EA0_RDREQ, none of them 32-byte), writes
    64-byte (TCC_EA0_WRREQ_64B) or 32-byte (the rest of TCC_EA0_WRREQ)."""
    r32 = rd.get("TCC_EA0_RDREQ_32B_sum", 0.0)
    read = READ_REQUEST_BYTES * (rd["TCC_EA0_RDREQ_sum"] - r32) + 32 * r32
    w64 = wr["TCC_EA0_WRREQ_64B_sum"]
    write = 64 * w64 + 32 * (wr["TCC_EA0_WRREQ_sum"] - w64)
    return read, write


def fused_kernel_re(F: int):
    """The fused reduce+AdamW+bf16 emit kernel of an F-row flat fold, by its
    demangled name in rocprofv3 output: the one-tile kernel of the staged fused
    step (8 or 16 rows), or the general vector kernel (other counts)."""
    return re.compile(r"k_step_one<%d, true(, 0, false)?>|"
                      r"k_step_vec<\(\(anonymous namespace\)::Op\)2, %d, true(, 0, false)?>" % (F, F))


def pmc_summary(read_dir: str, write_dir: str, F: int = 8):
    """Prints the traffic summary (markdown + JSON block) from two rocprofv3
    --pmc runs of `bench.py --quick`: one with READ_COUNTERS, one with
    WRITE_COUNTERS.

    On gfx950 an L2 -> memory read request moves a 128-byte line. The derived
    FETCH_SIZE metric counts a request as 128 bytes only through TCC_BUBBLE,
    which stays 0 for these kernels, so it reports half the bytes read. The
    128-byte size is checked here on two 1 GiB copies of known size: the HIP
    runtime's own device copy (torch's copy_) and the library's fp32 copy;
    both must come out within 0.1% of 2^30 bytes read and written."""
    import datagen.workloads as W

    fused = fused_kernel_re(F)
    rr, wr = _counter_rows(read_dir), _counter_rows(write_dir)
    kinds = {
        "fused": lambda n: bool(fused.search(n)),
        "gather": lambda n: "k_segcopy<1>" in n,
        "library_copy": lambda n: "k_segcopy<0>" in n,
        "runtime_copy": lambda n: "copyBuffer" in n,
    }
    avg = lambda x: sum(x) / len(x)
    per = {}
    for kind, match in kinds.items():
        dr, dw = _dispatch_counters(rr, match), _dispatch_counters(wr, match)
        pairs = [_request_bytes(dr[k], dw_k) for k, dw_k in
                 zip(sorted(dr, key=int), [dw[k] for k in sorted(dw, key=int)])]
        if not pairs:
            raise SystemExit(f"no {kind} dispatches in the counter runs")
        tot = [a + b for a, b in pairs]
        # the gathers and the 1 GiB copies are the largest launches of their kernel
        keep = [i for i, t in enumerate(tot) if t >= 0.5 * max(tot)]
        per[kind] = {
            "dispatches": len(keep),
            "read_bytes": avg([pairs[i][0] for i in keep]),
            "write_bytes": avg([pairs[i][1] for i in keep]),
            "raw": {c: avg([dr[k][c] for k in [sorted(dr, key=int)[i] for i in keep]])
                    for c in READ_COUNTERS},
            "raw_write": {c: avg([dw[k][c] for k in [sorted(dw, key=int)[i] for i in keep]])
                          for c in WRITE_COUNTERS},
        }
    gib = float(1 << 30)
    for kind in ("runtime_copy", "library_copy"):
        c = per[kind]
        c["read_over_known"] = c["read_bytes"] / gib
        c["write_over_known"] = c["write_bytes"] / gib
        if not (abs(c["read_over_known"] - 1) < 1e-3 and abs(c["write_over_known"] - 1) < 1e-3):
            raise SystemExit(f"{kind}: counted bytes do not match its 1 GiB: {c}")
    U = sum(math.prod(sh) for sh in W.shapes(W.BLK7))
    valid = min(-(-U // F), U)                    # rank 0's shard: ceil(U / F) elements
    alg_r, alg_w = (2 * F + 12) * valid, 14 * valid
    f, g = per["fused"], per["gather"]
    rec = {
        "kernel": "k_step_one<%d, emit> (fused reduce+AdamW+bf16 emit)" % F,
        "workload": "7B block unit, F=%d, rank 0, shard %d" % (F, valid),
        "kernels_hip_sha256_16": kernel_source_hash(),
        "read_request_bytes": READ_REQUEST_BYTES,
        "fused": f, "hbm_read_bytes_per_launch": f["read_bytes"],
        "hbm_write_bytes_per_launch": f["write_bytes"],
        "hbm_bytes_per_launch": f["read_bytes"] + f["write_bytes"],
        "algorithmic_read_bytes": alg_r, "algorithmic_write_bytes": alg_w,
        "traffic_over_algorithmic": (f["read_bytes"] + f["write_bytes"]) / (alg_r + alg_w),
        "gather": dict(g, algorithmic_bytes=4 * U,
                       traffic_over_algorithmic=(g["read_bytes"] + g["write_bytes"]) / (4 * U)),
        "known_size_checks": {k: per[k] for k in ("runtime_copy", "library_copy")},
    }
    print("```json\n" + json.dumps(rec, indent=1) + "\n```")


def trace_gaps(trace_csv: str, units: int, steps: int, warmup: int):
    """Per-step span, kernel time and launch gaps of a whole-model sequence, from a
    rocprofv3 kernel trace of `bench.py --workload full7b|full70b` (one launch per
    unit per step; the library's step kernels only). Prints a markdown table."""
    import csv
    import statistics

    rows = [r for r in csv.DictReader(open(trace_csv)) if "k_step" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    if len(rows) != units * (steps + warmup):
        raise SystemExit(f"expected {units * (steps + warmup)} step launches, found {len(rows)}")
    print("| step | first start → last end (ms) | sum of kernel durations (ms) | idle share | "
          "median gap between launches (us) | largest gap (us) |")
    print("|---|---|---|---|---|---|")
    spans, busys = [], []
    for s in range(warmup, warmup + steps):
        rr = rows[s * units:(s + 1) * units]
        st = [int(r["Start_Timestamp"]) for r in rr]
        en = [int(r["End_Timestamp"]) for r in rr]
        busy = sum(e - b for b, e in zip(st, en))
        span = en[-1] - st[0]
        gaps = [st[i + 1] - en[i] for i in range(len(rr) - 1)] or [0]
        spans.append(span)
        busys.append(busy)
        print(f"| {s - warmup + 1} | {span / 1e6:.3f} | {busy / 1e6:.3f} | "
              f"{max(0.0, 100 * (1 - busy / span)):.2f}% | {statistics.median(gaps) / 1e3:.1f} | "
              f"{max(gaps) / 1e3:.1f} |")
    span, busy = sum(spans) / len(spans), sum(busys) / len(busys)
    print(f"\nmean over the timed steps: span {span / 1e6:.3f} ms, kernels {busy / 1e6:.3f} ms, "
          f"idle {max(0.0, 100 * (1 - busy / span)):.2f}%")


def trace_steps(trace_csv: str, warmup: int, steps: int, F: int = 8):
    """Durations of the timed steps' launches in a rocprofv3 kernel trace of the
    default (blk7) bench: a step is a fused launch followed by a gather launch;
    the first `warmup` steps are skipped, the next `steps` are the timed ones.
    Prints one JSON line with avg/median/p10/p90/min in us per kernel."""
    import csv

    fused = fused_kernel_re(F)
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    lib = [r for r in rows if "k_step" in r["Kernel_Name"] or "k_segcopy" in r["Kernel_Name"]]
    pairs = []
    for a, b in zip(lib, lib[1:]):
        if fused.search(a["Kernel_Name"]) and "k_segcopy<1>" in b["Kernel_Name"]:
            pairs.append((a, b))
    if len(pairs) < warmup + steps:
        raise SystemExit(f"found {len(pairs)} fused+gather steps, expected {warmup + steps}")
    timed = pairs[warmup:warmup + steps]
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6   # ms
    print(json.dumps({"steps": len(timed),
                      "fused_us": spread([dur(a) for a, _ in timed]),
                      "gather_us": spread([dur(b) for _, b in timed])}))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-steps":
        trace_steps(sys.argv[2], int(sys.argv[3]), int(sys.argv[4]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-gaps":
        trace_gaps(sys.argv[2], *(int(x) for x in sys.argv[3:6]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        pmc_summary(sys.argv[2], sys.argv[3])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--cpu-worker":
        F, rank, first, n = (int(x) for x in sys.argv[2:6])
        cpu_worker(F, rank, first, n, float(sys.argv[6]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--F", type=int, default=8)
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--event-every", type=int, default=4,
                    help="blk7: bracket every N-th timed step with timing events")
    ap.add_argument("--roofline-steps", type=int, default=64,
                    help="blk7: steps of the roofline sample (every fused launch bracketed; "
                         "at least 64)")
    ap.add_argument("--rotate", type=int, default=4,
                    help="independent buffer sets visited in turn (1 = repeat one set)")
    ap.add_argument("--workload", default="blk7", choices=["blk7", "full7b", "full70b", "sweep", "state_dict", "hybrid"])
    ap.add_argument("--row-sets", type=int, default=2,
                    help="whole-model workloads: gradient row sets per unit size, used in turn")
    ap.add_argument("--state-layout", default="packed", choices=["packed", "per-unit"],
                    help="whole-model workloads: all units' master/m/v/param windows packed into "
                         "one allocation per array, or each unit's arrays allocated on their own")
    ap.add_argument("--per-unit", action="store_true",
                    help="whole-model workloads: one launch per unit instead of batched")
    ap.add_argument("--row-layout", default="separate", choices=["separate", "arena", "both"],
                    help="blk7, sweep: one allocation per gradient row (each rank's gradient "
                         "its own buffer), or all rows' windows in one arena; sweep only: "
                         "both, one after the other")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="blk7: only the headline steps and the two 1 GiB reference copies "
                         "(for profiler runs)")
    ap.add_argument("--cpu-sample", type=int, default=1 << 22)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()
    if args.row_layout == "both" and args.workload != "sweep":
        ap.error("--row-layout both applies to --workload sweep only")

    if args.gpus != 1:
        print(f"bench.py measures one rank's shard step on one GPU; --gpus {args.gpus} is not "
              "supported (the cross-GPU exchange steps on either side of the shard step are "
              "not implemented here)", file=sys.stderr)
        sys.exit(2)

    device = device_record() if args.workload == "blk7" else None

    import torch

    import datagen
    import sharded_flatparameter_flatten_amd as fsdp
    from datagen import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "sweep":
        sharding_sweep(args)
        return
    if args.workload == "state_dict":
        state_dict_bench(args)
        return
    if args.workload == "hybrid":
        hybrid_bench(args)
        return
    if args.workload != "blk7":
        model_sequence(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = W.shapes(W.BLK7)
    F, rank, R = args.F, args.rank, args.rotate
    units = [fsdp.Unit(shapes, F, r) for r in range(F)]
    u = units[rank]
    S, n = u.S, u.shard_valid
    print(f"# workload blk7 U={u.U} F={F} rank={rank} S={S} valid={n} sets={R}", file=sys.stderr,
          flush=True)

    # ---- inputs resident in HBM: R independent sets, visited in turn -------
    # (every set has its own gradient windows, optimizer state, bf16 shards and
    # outputs, so no step finds the previous step's data in a cache)
    sets, set_masters = make_sets(fsdp, torch, datagen, W, units, rank, R, dev,
                                  separate=args.row_layout == "separate")
    hp = fsdp.AdamWHparams(**W.ADAMW)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def fused(i):
        grads, p, m, v, shards, outs = sets[i % R]
        fsdp.reduce_adamw_shard(u, grads, p, m, v, shards[rank], hp, i // R + 1, stream=stream)

    def gather(i):
        grads, p, m, v, shards, outs = sets[i % R]
        fsdp.cast_unflatten(u, shards, outs, stream=stream)

    W0 = max(args.warmup, R)
    for i in range(W0):
        fused(i)
        gather(i)
    torch.cuda.synchronize()

    # Headline: K steps timed by the wall clock (value, ms_per_step). Timing
    # events cost the stream a few microseconds each, so only every
    # `event_every`-th of these steps is bracketed (start, between the fused
    # kernel and the gather, end); timing_us reports those steps.
    K = args.steps
    N = max(1, args.event_every)
    sampled = [i for i in range(K) if i % N == 0]
    ev = {i: [TimingEvent() for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev.get(i)
        if e:
            e[0].record(stream)
        fused(W0 + i)
        if e:
            e[1].record(stream)
        gather(W0 + i)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fused_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in sampled]
    gather_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in sampled]
    step_ev_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in sampled]
    ms_per_step = elapsed * 1e3 / K

    if args.quick:
        # profiler runs: the headline steps, then the two known-size copies
        # (the library's 1 GiB fp32 copy and torch's copy of the same size)
        copy_reference(fsdp, torch, dev, stream, reps=2)
        torch_copy_reference(torch, dev, reps=2)
        print(json.dumps({"workload": "blk7", "quick": True, "steps": K,
                          "ms_per_step": elapsed * 1e3 / K}), flush=True)
        return

    # Roofline sample: the same step loop run for `roofline_steps` more steps
    # (at least 64, whatever --steps is) with every fused launch bracketed, so
    # the kernel's average duration rests on that many launches.
    Lr = max(args.roofline_steps, 64)
    roof_f, roof_g = bracketed_steps(torch, stream, fused, gather, W0 + K, Lr)
    fused_avg = sum(roof_f) / len(roof_f)
    gather_avg = sum(roof_g) / len(roof_g)

    # The same sample on rank F-1 (its own rotating sets: the last window of
    # every gradient row).
    last = None
    if F > 1 and rank != F - 1:
        ul = units[F - 1]
        sets_l, _ = make_sets(fsdp, torch, datagen, W, units, F - 1, R, dev,
                              separate=args.row_layout == "separate", keep_masters=False)

        def fused_l(i):
            grads, p, m, v, shards, outs = sets_l[i % R]
            fsdp.reduce_adamw_shard(ul, grads, p, m, v, shards[F - 1], hp, i // R + 1,
                                    stream=stream)

        def gather_l(i):
            grads, p, m, v, shards, outs = sets_l[i % R]
            fsdp.cast_unflatten(ul, shards, outs, stream=stream)

        for i in range(W0):
            fused_l(i)
            gather_l(i)
        lf, lg = bracketed_steps(torch, stream, fused_l, gather_l, W0, Lr)
        nl = ul.shard_valid
        last = {"rank": F - 1, "shard_params": nl, "launches_timed": len(lf),
                "algorithmic_bytes_per_launch": (2 * F + 26) * nl,
                "fused_us": spread(lf), "gather_us": spread(lg),
                "achieved": (2 * F + 26) * nl / (sum(lf) / len(lf) * 1e-3) / 1e9,
                "frac": (2 * F + 26) * nl / (sum(lf) / len(lf) * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        del sets_l
        torch.cuda.empty_cache()

    # Stream-mix ceiling: the fused kernel's loads and stores without the
    # AdamW arithmetic (tests/probes/stream_mix_probe.hip), in the same step
    # loop over the same sets, in the workgroup shape the library picks for
    # this launch.
    mix = stream_mix_leg(torch, stream, sets, u, rank, F, gather, W0, Lr)

    # ---- every row of the path on its own (same rotation) -----------------
    g32 = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(R)]
    flat_dst = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(R)]

    def timed(fn, reps):
        for i in range(R):
            fn(i)
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def row(name, us, nbytes):
        return {"us": us, "bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                "frac_of_8TBps": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS}

    reps = max(2 * R, min(args.steps // 2, 48))
    rows = {
        "a2_flatten_pad_fp32": row("flatten", timed(lambda i: fsdp.flatten_pad(
            u, set_masters[i % R], flat_dst[i % R], stream=stream), reps), 8 * S),
        "a3_reduce_shard": row("reduce", timed(lambda i: fsdp.reduce_shard(
            u, sets[i % R][0], g32[i % R], stream=stream), reps), (2 * F + 4) * n),
        "a4_adamw_shard_emit": row("adamw", timed(lambda i: fsdp.adamw_shard(
            u, g32[i % R], sets[i % R][1], sets[i % R][2], sets[i % R][3], sets[i % R][4][rank],
            hp, 2, stream=stream), reps), 30 * n),
        "a5_fused_no_emit": row("fused", timed(lambda i: fsdp.reduce_adamw_shard(
            u, sets[i % R][0], sets[i % R][1], sets[i % R][2], sets[i % R][3], None, hp, 2,
            stream=stream), reps), (2 * F + 24) * n),
        "a5_fused_emit": row("fused", timed(lambda i: fsdp.reduce_adamw_shard(
            u, sets[i % R][0], sets[i % R][1], sets[i % R][2], sets[i % R][3],
            sets[i % R][4][rank], hp, 2, stream=stream), reps), (2 * F + 26) * n),
        "a6_cast_unflatten_bf16": row("gather", timed(lambda i: fsdp.cast_unflatten(
            u, sets[i % R][4], sets[i % R][5], stream=stream), reps), 4 * u.U),
    }
    del g32, flat_dst, set_masters

    # ---- secondary, "warm": one buffer set repeated, so the memory-side cache
    # may still hold part of the previous launch's data (not a training step's
    # situation; reported beside the rotating figures only)
    warm_us = timed(lambda i: fsdp.reduce_adamw_shard(
        u, sets[0][0], sets[0][1], sets[0][2], sets[0][3], sets[0][4][rank], hp, 2,
        stream=stream), reps)

    # ---- reference: the library's plain 4-byte copy of 1 GiB (same run) ----
    # (one tensor, F = 1: fsdp_flatten_pad is then a straight copy; its
    # counters also calibrate the HBM traffic figures)
    copy_gbps = copy_reference(fsdp, torch, dev, stream)

    props = torch.cuda.get_device_properties(dev)
    fused_bytes = (2 * F + 26) * n                # bf16 rows + fp32 p/m/v in/out + bf16 out
    gather_bytes = 4 * u.U                        # bf16 in (F*S valid) + bf16 out
    achieved = fused_bytes / (fused_avg * 1e-3) / 1e9
    if mix is not None:
        mix["GBps"] = fused_bytes / (mix["us"]["avg"] * 1e-6) / 1e9
        mix["fused_us_over_ceiling_us"] = fused_avg * 1e3 / mix["us"]["avg"]
    traffic = read_traffic()
    result = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator; bf16 grads, fp32 master)",
        "config": {
            "workload": (f"Llama-7B-shaped block unit (202,383,360 params, 9 tensors) as one "
                         f"FlatParameter, F={F}, rank {rank}: fused reduce+AdamW+bf16 emit on "
                         f"the {n:,}-param shard, then cast/unflatten of the {F} bf16 shards"),
            "F": F, "rank": rank, "n_grads": F, "unit_params": u.U, "shard_params": n,
            "param_dtype": "bf16", "reduce_dtype": "f32", "rotating_sets": R,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "fused reduce+AdamW+bf16 emit (k_step_one<8, emit>)",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": fused_bytes,
            "avg_launch_us": fused_avg * 1e3,
            "median_launch_us": spread(roof_f)["median"],
            "p90_launch_us": spread(roof_f)["p90"],
            "launches_timed": len(roof_f),
            "protocol": (f"{len(roof_f)} in-step launches after the headline loop, each "
                         "bracketed by HIP events on the launch stream; rotating sets"),
        },
        "roofline_rank_last": last,
        "stream_mix_ceiling": mix,
        "fused_us": fused_avg * 1e3,
        "fused_us_min": min(roof_f) * 1e3,
        "gather_us": gather_avg * 1e3,
        "gather_GBps": gather_bytes / (gather_avg * 1e-3) / 1e9,
        "step_GBps": (fused_bytes + gather_bytes) / (ms_per_step * 1e-3) / 1e9,
        "unit_params_per_s": u.U / (ms_per_step * 1e-3),
        "copy_GBps": copy_gbps,
        "timing_us": {"event_every": N, "fused": spread(fused_ms), "gather": spread(gather_ms),
                      "step": spread(step_ev_ms), "roofline_fused": spread(roof_f),
                      "roofline_gather": spread(roof_g)},
        "rows_alone": rows,
        "warm_secondary": {"fused_us": warm_us,
                           "GBps": (2 * F + 26) * n / (warm_us * 1e-6) / 1e9,
                           "frac_of_8TBps": (2 * F + 26) * n / (warm_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                           "protocol": "one buffer set repeated back to back"},
        "device": dict(device or {}, torch_name=props.name, arch=props.gcnArchName,
                       multiprocessors=props.multi_processor_count,
                       hbm_bytes=props.total_memory),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(F, rank, args.cpu_sample, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
