"""Benchmark of the fused ragged GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one call of the operator through the C ABI on one batch of
seeded synthetic input already resident in HBM.  The default workload is
the packed/packed ragged causal GQA prefill (B=16, lengths ~ U[64, 2048],
H_q=32, H_kv=8, D=128, bf16, lower_right).  W untimed steps, then K steps
bracketed by stream synchronisation and timed with HIP events recorded on
the stream the kernels run on.  The JSON line reports

  value     algorithmic TFLOP/s (prefill: 4*D*allowed pairs; the extra
            statistics pass of the quantized op is not counted) or GB/s
            (decode: valid K/V bytes + Q + Y);
  roofline  that rate against the MI355X peak of the bounding unit;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
            workload on this host's cores (a reported baseline only);
  secondary the other workload shapes measured the same way (decode
            GB/s, chunked context, quantized fp8), unless --no-secondary.

--profile-pass runs one copy of known size plus one step, untimed, for the
rocprofv3 counter runs that calibrate and measure HBM traffic.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}  # dense MFMA TFLOP/s
HBM_PEAK = 8000.0  # GB/s
WORKLOADS = ("2", "3", "4a", "4b", "4p", "5a", "5b", "tree", "kvu", "1")
KERNEL_SOURCES = {
    "prefill": ["gqa_attention_ragged_amd/csrc/prefill.hip",
                "gqa_attention_ragged_amd/csrc/prefill_impl.h",
                "gqa_attention_ragged_amd/csrc/tile_common.h",
                "gqa_attention_ragged_amd/csrc/device_common.h"],
    "decode": ["gqa_attention_ragged_amd/csrc/decode.hip",
               "gqa_attention_ragged_amd/csrc/device_common.h"],
}


def kernel_sha(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def work_of(case) -> dict:
    """Algorithmic work of one step: FLOP (prefill kernel) or bytes (decode)."""
    D = case.q.shape[-1]
    ql = np.asarray(case.q_lens, dtype=np.int64)
    kl = np.asarray(case.kv_lens, dtype=np.int64)
    if case.query_form == "padded_bhnd" and case.q.shape[2] == 1 and case.mask is None:
        kv_b = case.k.element_size()
        q_b = case.q.element_size()
        byts = int(np.sum(kl)) * case.kv_num_heads * D * 2 * kv_b + \
            case.batch * case.num_heads * D * (q_b + 2)
        return {"kind": "decode", "bytes": byts}
    pairs = 0
    tree = None if case.tree_parents is None else case.tree_parents.cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(ql)])
    for b in range(case.batch):
        i = np.arange(ql[b])
        if case.causal_kind == "none":
            n = np.full(ql[b], kl[b])
        else:
            diag = 0 if case.causal_kind == "upper_left" else kl[b] - ql[b]
            n = np.clip(i + diag + 1, 0, kl[b])
        if tree is not None:
            # tree decoding (causal none): the context plus the draft's own
            # ancestor chain, itself included
            row0 = int(starts[b]) if case.query_form == "packed_nhd" else b * case.q.shape[2]
            par = tree[row0:row0 + ql[b]]
            depth = np.zeros(ql[b], dtype=np.int64)
            for t in range(int(ql[b])):
                u, d = t, 0
                while 0 <= par[u] < u:
                    u, d = int(par[u]), d + 1
                depth[t] = d
            n = np.minimum(n, kl[b] - ql[b] + depth + 1)
        pairs += int(n.sum())
    pairs *= case.num_heads
    return {"kind": "prefill", "flop": 4 * D * pairs, "pairs": pairs}


def kernel_name(case, kind: str) -> str:
    """The kernel that dominates a step."""
    return "gqa::decode_split_kernel" if kind == "decode" else "gqa::prefill_kernel"


def dtype_name(case) -> str:
    import torch
    return {torch.bfloat16: "bf16", torch.float16: "f16", torch.float8_e4m3fn: "fp8"}[case.q.dtype]


def make_step(case):
    import torch
    from gqa_attention_ragged_amd import capi, synth
    out = synth.sentinel_like(case.q.shape, case.out_dtype, case.q.device)
    args = capi.make_args(case.q, case.k, case.v, case.mask, out, **case.kwargs())
    n = capi.gqa_attn_workspace_size(args)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=case.q.device)
    stream = torch.cuda.current_stream().cuda_stream
    lib = capi.load()
    import ctypes
    pargs = ctypes.byref(args)
    ws_ptr, ws_n = ws.data_ptr(), ws.numel()

    def step():
        st = lib.gqa_attn_forward(pargs, ws_ptr, ws_n, stream)
        if st != 0:
            raise capi.GqaError(st, capi.last_error())

    step.keep = (out, ws, args)  # keep buffers alive
    return step


# The GPU raises its clocks over the first tens of milliseconds of
# back-to-back work (measured on the prefill workload: 0.37 -> 0.28 ms per
# step over ~100 steps); warming up for at least this long, whatever the
# requested step count, makes the timed steps steady state.
MIN_WARMUP_MS = 400.0
_warmup_log: dict = {}
# Average duration of the main attention kernel over the timed steps (ms),
# from the library's own event pairs around that kernel (gqa_attn_timer_*).
_kernel_ms: dict = {}


def time_steps(step, steps: int, warmup: int, tag: str = "", kernel_timer: bool = False,
               min_warmup_ms: float = MIN_WARMUP_MS) -> float:
    """Average ms per step over `steps` timed launches (HIP events on the
    stream the kernels run on), after `warmup` steps and as many more as it
    takes to reach min_warmup_ms of warm-up (recorded in _warmup_log).  With
    kernel_timer, the library also times its main kernel in each timed step
    (an event pair on the same stream around that kernel alone): the average
    goes to _kernel_ms[tag].  The event records add a few microseconds per
    step, so whole-step rates come from runs without them."""
    import torch
    from gqa_attention_ragged_amd import capi
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    while (time.perf_counter() - t0) * 1e3 < min_warmup_ms:
        for _ in range(10):
            step()
        extra += 10
        torch.cuda.synchronize()
    _warmup_log[tag] = {"extra_steps": extra, "ms": round((time.perf_counter() - t0) * 1e3, 1)}
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if kernel_timer and capi.timer_start(steps) != capi.GQA_OK:
        raise RuntimeError(f"gqa_attn_timer_start: {capi.last_error()}")
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    if kernel_timer:
        st, kms, n = capi.timer_stop()
        if st != capi.GQA_OK or n != steps:
            raise RuntimeError(f"gqa_attn_timer_stop: status {st}, {n} of {steps} steps timed: "
                               f"{capi.last_error()}")
        _kernel_ms[tag] = kms / n
    return start.elapsed_time(end) / steps


def measure_kv_update(steps: int, warmup: int) -> dict:
    """The KV-cache update workload: bytes = update rows read + cache rows
    written (all rows land inside the cache)."""
    import torch
    from gqa_attention_ragged_amd import capi, synth
    c = synth.make_kv_update_workload(device="cuda")
    args = capi.make_kv_update_args(c.past_cache, c.update, **c.kwargs())
    stream = torch.cuda.current_stream().cuda_stream
    lib = capi.load()
    import ctypes
    pargs = ctypes.byref(args)

    def step():
        st = lib.gqa_kv_cache_update(pargs, stream)
        if st != 0:
            raise capi.GqaError(st, capi.last_error())

    ms = time_steps(step, steps, warmup, "kvu")
    H, D = c.past_cache.shape[1], c.past_cache.shape[3]
    byts = 2 * int(np.sum(c.counts)) * H * D * c.past_cache.element_size()
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": "kvu", "description": synth.KV_UPDATE_DESCRIPTION, "ms_per_step": round(ms, 4),
            "dtype": "bf16", "metric": "KV-cache update GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "bytes": byts, "roofline_frac": round(gbs / HBM_PEAK, 4), "bound": "hbm",
            "peak": HBM_PEAK, "_case": c}


def measure(cfg: str, steps: int, warmup: int) -> dict:
    import torch
    from gqa_attention_ragged_amd import synth
    if cfg == "kvu":
        return measure_kv_update(steps, warmup)
    case = synth.make_config(cfg, device="cuda")
    torch.cuda.synchronize()
    w = work_of(case)
    step = make_step(case)
    ms = time_steps(step, steps, warmup, cfg)
    # the main kernel's own duration: the same number of steps again, right
    # after the timed ones (clocks warm), with the library's event pair
    # around that kernel in each step
    time_steps(step, steps, 0, cfg + ":kernel", kernel_timer=True, min_warmup_ms=0.0)
    kms = _kernel_ms[cfg + ":kernel"]
    dt = dtype_name(case)
    r = {"workload": cfg, "description": synth.DESCRIPTIONS[cfg], "ms_per_step": round(ms, 4),
         "kernel_ms": round(kms, 4), "dtype": dt}
    if cfg == "1":
        r["latency_us"] = round(ms * 1e3, 2)  # one call, latency-bound
    if w["kind"] == "decode":
        gbs = w["bytes"] / (ms * 1e-3) / 1e9
        r.update(metric="KV GB/s", value=round(gbs, 1), unit="GB/s", bytes=w["bytes"],
                 roofline_frac=round(gbs / HBM_PEAK, 4), bound="hbm", peak=HBM_PEAK,
                 kernel_value=round(w["bytes"] / (kms * 1e-3) / 1e9, 1))
    else:
        tf = w["flop"] / (ms * 1e-3) / 1e12
        r.update(metric="attention TFLOP/s", value=round(tf, 1), unit="TFLOP/s", flop=w["flop"],
                 roofline_frac=round(tf / PEAK[dt], 4), bound="mfma", peak=PEAK[dt],
                 kernel_value=round(w["flop"] / (kms * 1e-3) / 1e12, 1))
    r["_case"] = case
    return r


def traffic_for(cfg: str, kind: str):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_cfg{cfg}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha(kind):
        return None
    return int(t["hbm_bytes_per_launch"])


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads(n: int) -> None:
    """Set the OpenMP thread count of the oracle's parallel regions."""
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def oracle_cfg1_ms() -> dict:
    """The oracle on the whole tiny workload (every row), on one thread and
    on all the process's cores: ms per call (best of 3)."""
    import oracle
    from gqa_attention_ragged_amd import synth
    c = synth.make_config("1", device="cpu")
    out = {}
    for tag, n in (("1thread", 1), ("all_cores", int(os.environ["OMP_NUM_THREADS"]))):
        _omp_threads(n)
        best = 1e30
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
            best = min(best, time.perf_counter() - t0)
        out[f"ms_{tag}"] = round(best * 1e3, 3)
    _omp_threads(int(os.environ["OMP_NUM_THREADS"]))
    return out


def cpu_baseline(case, seconds: float) -> dict:
    """The CPU oracle on a bounded sample of rows of the same workload."""
    import oracle
    from tests import parity
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    w = work_of(case)
    # pick whole rows, last rows of each sequence first (the longest), until
    # the estimated work fills the time budget at ~1 GFLOP/s per core
    budget = seconds * cores * 1.0e9
    rows, work = [], 0
    rng = np.random.default_rng(0)
    per_b = []
    for b in range(case.batch):
        L = int(case.q_lens[b])
        if L:
            per_b.append((b, L))
    D = case.q.shape[-1]
    while work < budget and len(rows) < 200000:
        b, L = per_b[int(rng.integers(0, len(per_b)))]
        i = int(rng.integers(0, L))
        h = int(rng.integers(0, case.num_heads))
        rows.append((b, h, i))
        kvl = int(case.kv_lens[b])
        if case.causal_kind == "none":
            n = kvl
        else:
            diag = 0 if case.causal_kind == "upper_left" else kvl - L
            n = max(0, min(kvl, i + diag + 1))
        work += 4 * D * max(n, 1)
    rows = np.asarray(rows, dtype=np.int32)
    # host copies of the sequences involved (outside the timed region)
    done_work = 0
    t_all = 0.0
    for b in np.unique(rows[:, 0]):
        sel = rows[:, 0] == b
        sub = parity.subcase(case, [int(b)])
        r = rows[sel].copy()
        r[:, 0] = 0
        t0 = time.perf_counter()
        res = oracle.attention(sub.q, sub.k, sub.v, sub.mask, rows=r, **sub.kwargs())
        t_all += time.perf_counter() - t0
        if w["kind"] == "prefill":
            done_work += int(res.nallowed.sum()) * 4 * D
        else:
            kvl = int(case.kv_lens[b])
            done_work += int(sel.sum()) * kvl * D * 2 * case.k.element_size()
    if w["kind"] == "prefill":
        val = done_work / t_all / 1e12
        unit = "TFLOP/s"
        desc = f"{len(rows)} sampled query rows (all their allowed keys), {done_work:.3e} FLOP"
    else:
        val = done_work / t_all / 1e9
        unit = "GB/s"
        desc = f"{len(rows)} sampled (b, head) rows, {done_work:.3e} KV bytes"
    # the same oracle on one thread, over the first rows of the sample
    # (about a tenth of the time budget)
    r1 = rows[: max(1, len(rows) // (10 * max(1, int(os.environ["OMP_NUM_THREADS"]))))]
    _omp_threads(1)
    t1, w1 = 0.0, 0
    for b in np.unique(r1[:, 0]):
        sel = r1[:, 0] == b
        sub = parity.subcase(case, [int(b)])
        r = r1[sel].copy()
        r[:, 0] = 0
        t0 = time.perf_counter()
        res = oracle.attention(sub.q, sub.k, sub.v, sub.mask, rows=r, **sub.kwargs())
        t1 += time.perf_counter() - t0
        if w["kind"] == "prefill":
            w1 += int(res.nallowed.sum()) * 4 * D
        else:
            w1 += int(sel.sum()) * int(case.kv_lens[b]) * D * 2 * case.k.element_size()
    _omp_threads(int(os.environ["OMP_NUM_THREADS"]))
    v1 = w1 / t1 / (1e12 if w["kind"] == "prefill" else 1e9)
    return {"value": float(f"{val:.6g}"), "unit": unit, "cores": int(os.environ["OMP_NUM_THREADS"]),
            "kind": "oracle", "sample": desc, "seconds": round(t_all, 2),
            "host_cpu": host_cpu_model(),
            "value_1thread": float(f"{v1:.6g}"),
            "sample_1thread": f"{len(r1)} of those rows on one thread, {t1:.2f} s",
            "tiny_workload_oracle": oracle_cfg1_ms()}


def profile_pass(cfg: str) -> None:
    """One 256 MiB device copy (counter calibration) and one step."""
    import torch
    from gqa_attention_ragged_amd import synth
    case = synth.make_config(cfg, device="cuda")
    step = make_step(case)
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": cfg, "copy_bytes": n}), flush=True)


def write_traffic(cfg: str, fetch_dir: str, write_dir: str) -> dict:
    """profiles/traffic_cfg<cfg>.json from two rocprofv3 --pmc runs of
    --profile-pass (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each
    counter is scaled by what it reads for the 256 MiB device copy of the same
    run, so that the figure is HBM bytes."""
    import csv
    import glob
    from gqa_attention_ragged_amd import synth

    def per_dispatch(d: str, counter: str) -> dict:
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    case = synth.make_config(cfg, device="cpu")
    kind = work_of(case)["kind"]
    want = kernel_name(case, kind).split("::")[1]
    out = {"workload": cfg}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        v = per_dispatch(d, counter)
        ker = [(k, x) for k, x in v.items() if want in k[0]]
        copy = [x for k, x in v.items() if "copyBuffer" in k[0] or "copy" in k[0].lower()]
        if not ker or not copy:
            raise SystemExit(f"{counter}: kernel or copy dispatch not found in {d}")
        kib = sum(x for _, x in ker) / len(ker)
        copy_kib = max(copy)
        expect = (256 << 20) / 1024.0  # the copy reads and writes 256 MiB
        scale = expect / copy_kib
        tag = counter.split("_")[0].lower()
        out["kernel"] = ker[0][0][0]
        out[f"{tag}_kib_per_dispatch"] = kib
        out[f"copy_256MiB_{tag}_kib"] = copy_kib
        out[f"{tag}_scale"] = scale
        out[f"{tag}_bytes"] = kib * 1024.0 * scale
    out["kernel_sha"] = kernel_sha(kind)
    out["hbm_bytes_per_launch"] = int(out["fetch_bytes"] + out["write_bytes"])
    out["commands"] = [
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
        f"python3 bench.py --profile-pass --workload {cfg}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- "
        f"python3 bench.py --profile-pass --workload {cfg}",
        f"python3 bench.py --write-traffic {fetch_dir} {write_dir} --workload {cfg}",
    ]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", f"traffic_cfg{cfg}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


# Two counter passes per prefill workload (at most 8 SQ counters each).
COUNTER_PASSES = (
    ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU",
     "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_CMD_FIFO_FULL",
     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_SALU", "SQ_WAIT_INST_LDS"],
)
SIMDS = 256 * 4


def write_trace(cfg: str, trace_dir: str, steps: int = 50) -> dict:
    """profiles/<kernel>_cfg<cfg>.md from a rocprofv3 --kernel-trace --stats run
    of `bench.py --workload <cfg> --no-secondary --no-cpu`: the per-kernel
    statistics (kernels above 0.5% of GPU time), the dominant kernel's average
    over its last `steps` dispatches (the timed steps) and the algorithmic rate
    that average gives, beside the rate bench.py reported in the same run."""
    import csv
    import glob
    from gqa_attention_ragged_amd import synth
    case = synth.make_config(cfg, device="cpu")
    w = work_of(case)
    want = kernel_name(case, w["kind"]).split("::")[1]
    stats = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        stats += list(csv.DictReader(open(f)))
    trace = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        trace += list(csv.DictReader(open(f)))
    if not stats or not trace:
        raise SystemExit(f"no kernel statistics or trace under {trace_dir}")
    mine = [r for r in trace if want in r["Kernel_Name"]]
    mine.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = mine[-steps:]
    avg_ns = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in last) / len(last)
    kernel = last[0]["Kernel_Name"]
    if w["kind"] == "decode":
        rate, unit, peak = w["bytes"] / avg_ns, "GB/s", HBM_PEAK
        work = f"{w['bytes'] / 1e9:.3f} GB of K/V, Q and Y per step"
    else:
        rate, unit = w["flop"] / avg_ns / 1e3, "TFLOP/s"
        peak = PEAK[dtype_name(case)]
        work = f"{w['flop'] / 1e9:.2f} GFLOP per step"
    # bench.py's own line, printed by the traced run
    bench_line = None
    for f in glob.glob(os.path.join(trace_dir, "..", f"trace_{cfg}.log")):
        for line in open(f):
            if line.startswith("{"):
                bench_line = json.loads(line)
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- "
           f"python3 bench.py --workload {cfg} --no-secondary --no-cpu")
    short = want.replace("_kernel", "")
    path = os.path.join(ROOT, "profiles", f"{short}_kernel_cfg{cfg}.md")
    lines = [f"# {want}, workload {cfg}", "", f"Workload: {synth.DESCRIPTIONS[cfg]}.", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", f"    {cmd}",
             f"    python3 bench.py --write-trace {trace_dir} --workload {cfg}", "",
             f"Kernel sources sha {kernel_sha(w['kind'])}.  Kernel statistics (every dispatch of the run: "
             "warm-up and timed steps; rows below 0.5% of GPU time omitted):", "",
             "| kernel | calls | average ns | min ns | max ns | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["Percentage"])):
        if float(r["Percentage"]) < 0.5:
            continue
        name = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['Percentage']):.2f} |")
    lines += ["", f"Average of the dominant kernel's last {len(last)} dispatches (the timed steps): "
              f"{avg_ns:.0f} ns.", f"Algorithmic work {work} / {avg_ns / 1e3:.1f} us = {rate:.1f} {unit} "
              f"({rate / peak:.3f} of the {peak:g} {unit} peak)."]
    # the library's other kernels of each step (tile-map plan, split-KV merge)
    others = {}
    for r in trace:
        n = r["Kernel_Name"]
        if "gqa" in n and want not in n:
            others.setdefault(n, []).append(r)
    for n, rs in sorted(others.items()):
        rs.sort(key=lambda r: int(r["Start_Timestamp"]))
        tail = rs[-steps:]
        ns = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tail) / len(tail)
        lines.append(f"Also launched in each step: `{n}`, {ns:.0f} ns on average over its last "
                     f"{len(tail)} dispatches (included in the whole-step rate below).")
    if bench_line:
        lines.append(f"bench.py in the same run (HIP events over the timed steps, whole step): "
                     f"{bench_line['value']} {bench_line['unit']}, {bench_line['ms_per_step']} ms/step.")
        roof = bench_line.get("roofline") or {}
        if roof.get("kernel_ms") is not None:
            kns = roof["kernel_ms"] * 1e6
            lines.append(f"bench.py's own timing of this kernel (the library's event pair around it, "
                         f"in a second pass of the timed steps): {kns:.0f} ns on average, {roof['achieved']} "
                         f"{roof['unit']} (roofline.achieved); the trace's average above: "
                         f"{avg_ns:.0f} ns ({(kns / avg_ns - 1) * 100:+.1f}%).")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return {"workload": cfg, "kernel": kernel, "avg_ns": avg_ns, "rate": rate, "unit": unit, "path": path}


def write_counters(cfg: str, dirs: list) -> dict:
    """profiles/counters_<kernel>_cfg<cfg>.md from the rocprofv3 --pmc runs of
    --profile-pass in `dirs` (one per COUNTER_PASSES entry): the counters of
    the dominant kernel's dispatch, per wave and per 64-key wave-tile."""
    import csv
    import glob
    from gqa_attention_ragged_amd import synth
    case = synth.make_config(cfg, device="cpu")
    w = work_of(case)
    want = kernel_name(case, w["kind"]).split("::")[1]
    vals = {}
    kernel = None
    dur_ns = None
    for d in dirs:
        per = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if want not in r["Kernel_Name"]:
                    continue
                kernel = r["Kernel_Name"]
                key = (r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                dur_ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for (name, _), v in per.items():
            vals[name] = v  # one dispatch of the kernel per profile pass
    D = case.q.shape[-1]
    # wave-tiles: 32 query rows x 64 keys per wave, over the allowed pairs
    # rounded to whole tiles is not known here: report per allowed 32x64 block
    blocks = w.get("pairs", 0) / (32 * 64)
    out = {"workload": cfg, "kernel": kernel, "counters": vals, "dispatch_ns": dur_ns}
    # GRBM_GUI_ACTIVE as collected is the sum over the 8 XCDs
    g = vals.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
    if g:
        out["mfma_busy_frac"] = vals.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (g * SIMDS)
        if dur_ns:
            out["clock_ghz"] = g / dur_ns
    if vals.get("SQ_WAVE_CYCLES"):
        out["wait_frac"] = vals.get("SQ_WAIT_INST_ANY", 0.0) / vals["SQ_WAVE_CYCLES"]
        out["valu_active_frac"] = vals.get("SQ_ACTIVE_INST_VALU", 0.0) / vals["SQ_WAVE_CYCLES"]
    if blocks:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS",
                  "SQ_INSTS_SALU"):
            if k in vals:
                out[f"{k}_per_32x64_block"] = vals[k] / blocks
    cmds = [f"rocprofv3 --pmc {' '.join(p)} --output-format csv -d <dir{i}> -o run -- "
            f"python3 bench.py --profile-pass --workload {cfg}" for i, p in enumerate(COUNTER_PASSES)]
    short = want.split("_kernel")[0]
    path = os.path.join(ROOT, "profiles", f"counters_{short}_cfg{cfg}.md")
    lines = [f"# {want} counters, workload {cfg}", "",
             f"Workload: {synth.DESCRIPTIONS[cfg]}.", "",
             "Commands (one rocprofv3 --pmc pass each, from the repository root):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += [f"    python3 bench.py --write-counters <dir0> <dir1> --workload {cfg}", "",
              f"Kernel: `{kernel}` (one dispatch per pass); kernel sources sha {kernel_sha(w['kind'])}.",
              "", "| Counter | Value |", "|---|---|"]
    for k in sorted(vals):
        lines.append(f"| {k} | {vals[k]:.6g} |")
    lines += ["", "Derived:", ""]
    if dur_ns:
        lines.append(f"- dispatch duration under the counters: {dur_ns / 1e3:.1f} us")
    if "mfma_busy_frac" in out:
        lines.append(f"- MFMA busy: {out['mfma_busy_frac']:.3f} of the kernel's cycles per SIMD "
                     "(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs))")
    if "clock_ghz" in out:
        lines.append(f"- shader clock during the dispatch: {out['clock_ghz']:.2f} GHz "
                     "(GRBM_GUI_ACTIVE / 8 over the dispatch duration)")
    if "wait_frac" in out:
        lines.append(f"- waves waiting on s_waitcnt: {out['wait_frac']:.3f} of wave cycles; "
                     f"issuing VALU: {out['valu_active_frac']:.3f}")
    if blocks:
        lines.append(f"- per 32-row x 64-key block of allowed pairs ({blocks:.0f} blocks):")
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                  "SQ_INSTS_SALU"):
            if f"{k}_per_32x64_block" in out:
                lines.append(f"  - {k}: {out[k + '_per_32x64_block']:.1f}")
    if vals.get("SQ_LDS_IDX_ACTIVE"):
        lines.append(f"- LDS bank conflicts: {vals.get('SQ_LDS_BANK_CONFLICT', 0) / vals['SQ_LDS_IDX_ACTIVE']:.3f}"
                     " of LDS-active cycles; command FIFO full: "
                     f"{vals.get('SQ_LDS_CMD_FIFO_FULL', 0):.4g} cycles")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    out["path"] = path
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU ramps its clocks up over the first ~30 ms of back-to-back steps
    # (measured: workload 2 goes 0.37 -> 0.28 ms per step over ~100 steps);
    # the default warm-up covers that, so the timed steps are steady state.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--workload", default="2", choices=[w for w in WORKLOADS if w != "kvu"])
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--write-counters", nargs="+", metavar="PASS_DIR")
    ap.add_argument("--write-trace", metavar="TRACE_DIR")
    a = ap.parse_args()
    if a.write_traffic:
        print(json.dumps(write_traffic(a.workload, *a.write_traffic)))
        return 0
    if a.write_counters:
        print(json.dumps(write_counters(a.workload, a.write_counters), default=str))
        return 0
    if a.write_trace:
        print(json.dumps(write_trace(a.workload, a.write_trace), default=str))
        return 0
    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {a.gpus} requested); the "
              "operator shards by KV-head group or by sequence with no exchange, but no "
              "multi-GPU path is built", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from gqa_attention_ragged_amd import capi
    capi.load()  # fails loudly if the HIP library is missing
    if a.profile_pass:
        profile_pass(a.workload)
        return 0

    main_r = measure(a.workload, a.steps, a.warmup)
    case = main_r.pop("_case")
    kind = "decode" if main_r["bound"] == "hbm" else "prefill"
    per_launch = main_r["bytes"] if kind == "decode" else main_r["flop"]
    traffic = traffic_for(a.workload, kind)
    # the main kernel's own rate: algorithmic work per launch over its
    # average duration (the library's event pairs, in a second pass of the
    # timed steps)
    ach = main_r["kernel_value"]
    roof = {"bound": main_r["bound"], "achieved": ach, "peak": main_r["peak"],
            "unit": main_r["unit"], "frac": round(ach / main_r["peak"], 4), "traffic": traffic,
            "kernel": kernel_name(case, kind),
            "per_launch": per_launch, "kernel_ms": main_r["kernel_ms"]}
    secondary = {}
    if not a.no_secondary:
        for cfg in WORKLOADS:
            if cfg == a.workload:
                continue
            # the same warm-up as the headline workload: the clocks need
            # about 150 launches to settle
            r = measure(cfg, max(5, a.steps // 2), a.warmup)
            r.pop("_case")
            secondary[cfg] = r
            torch.cuda.empty_cache()
    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(case, a.cpu_seconds)
    line = {
        "metric": "attention TFLOP/s (prefill) + KV GB/s (decode), % of MI355X roofline",
        "value": main_r["value"],
        "unit": main_r["unit"],
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        # warm-up steps added beyond --warmup to reach MIN_WARMUP_MS (clocks)
        "warmup_extra": _warmup_log.get(a.workload),
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_r["dtype"],
        "data": "synthetic (seeded; lengths, masks and values drawn as the workload specifies)",
        "config": {"workload": main_r["description"], "global_batch": int(case.batch),
                   "seq_len": int(max(case.q_lens)), "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
