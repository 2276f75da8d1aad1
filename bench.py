"""Benchmark: valid-work TFLOP/s of padded varlen sigmoid attention, forward
plus backward, on one MI355X.

One step = the whole hot path over one synthetic single-cell-shaped batch
(B32 H8 d64, log-normal lengths with median 800 clipped to [200, 2048], padded
to the batch maximum, block 128, bias -ln n):
  blockmask_build (block mask and work schedule from seq_lens)
    -> sigattn_fwd -> sigattn_bwd (dK/dV and dQ, one launch)
Inputs are resident in HBM before the timed region.  Valid FLOPs count only
attended (query, key) pairs: 4 d per pair per head forward, 10 d backward.

Prints ONE JSON line on stdout; progress goes to stderr.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "valid-work TFLOP/s + % bf16 MFMA peak, padded varlen sigmoid attn fwd/bwd"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# The sources each measured kernel is built from (the benchmark's sigmoid
# instantiations), for the digest that ties a counter summary to the code.
KERNEL_SOURCES = {
    "fwd": ["varlen_attention_amd/csrc/fwd_kernel.h", "varlen_attention_amd/csrc/fwd_sigmoid.hip"],
    "bwd": ["varlen_attention_amd/csrc/bwd_kernel.h", "varlen_attention_amd/csrc/bwd_sigmoid.hip"],
    "blockmask": ["varlen_attention_amd/csrc/blockmask.hip"],
    "schedule": ["varlen_attention_amd/csrc/schedule.hip"],
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without // comments and blank lines: what the compiler sees."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code.strip():
            lines.append(code)
    return "\n".join(lines)


def source_digest(kernel: str) -> str:
    """Digest of the code (not the comments) a kernel is built from."""
    paths = KERNEL_SOURCES[kernel] + ["varlen_attention_amd/csrc/device_common.h",
                                      "varlen_attention_amd/csrc/kernels.h"]
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it still
    describes the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != source_digest(kernel):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(kernel: str, w) -> float:
    """Minimum HBM bytes of one launch on workload w: every valid row of each
    input read once, every row of each output written once (bf16)."""
    valid = float(np.clip(w.seq_lens, 0, w.L).sum()) * w.H
    every = float(w.B) * w.L * w.H
    row = 2.0 * w.d
    reads, writes = {"fwd": (3, 1), "bwd": (4, 3)}[kernel]
    return (reads * valid + writes * every) * row


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirname}")


KERNEL_SYMBOLS = {"fwd": "::fwd_kernel<", "bwd": "::bwd_kernel<", "blockmask": "blockmask_",
                  "schedule": "schedule_kernel"}


def summarize_stats(dirname: str, skip: int = 0) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats run: the profiler's
    own statistics over all calls, and per-dispatch durations from the kernel
    trace without each kernel's first `skip` dispatches (the warmup steps,
    which run before the clocks settle)."""
    rows = _csv_rows(_find(dirname, "kernel_stats.csv"))
    out = ["All dispatches (rocprofv3 --stats):", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    trace = _csv_rows(_find(dirname, "kernel_trace.csv"))
    by_kernel = {}
    for r in trace:
        by_kernel.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out += ["", f"Timed dispatches (kernel trace, first {skip} dispatches of each kernel "
                "skipped):", "",
            "| kernel | dispatches | average (us) | min (us) | max (us) |",
            "|---|---|---|---|---|"]
    for name, v in by_kernel.items():
        v.sort()
        d = np.array([x[1] for x in v[skip:]], dtype=np.float64) / 1e3
        if d.size:
            out.append(f"| `{name[:90]}` | {d.size} | {d.mean():.2f} | {d.min():.2f} | "
                       f"{d.max():.2f} |")
    return "\n".join(out)


def _counter_per_dispatch(dirname: str, symbol: str, counter: str) -> float:
    rows = _csv_rows(_find(dirname, "counter_collection.csv"))
    vals = [float(r["Counter_Value"]) for r in rows
            if symbol in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise ValueError(f"{counter} for {symbol} not found in {dirname}")
    return float(np.mean(vals))


def _copy_counter(dirname: str, counter: str) -> float:
    rows = _csv_rows(_find(dirname, "counter_collection.csv"))
    vals = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter]
    return max(vals)


def summarize_traffic(kernel: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                      copy_write_dir: str, copy_mib: int, workload, workload_name: str) -> str:
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE counters
    (KiB per dispatch), each scaled by what the same counter reads for a
    plain device copy of copy_mib MiB."""
    sym = KERNEL_SYMBOLS[kernel]
    fetch = _counter_per_dispatch(fetch_dir, sym, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, sym, "WRITE_SIZE")
    true_kib = copy_mib * 1024.0
    fscale = true_kib / _copy_counter(copy_fetch_dir, "FETCH_SIZE")
    wscale = true_kib / _copy_counter(copy_write_dir, "WRITE_SIZE")
    hbm = (fetch * fscale + write * wscale) * 1024.0
    algo = algorithmic_bytes(kernel, workload)
    lines = [
        f"# HBM traffic of {kernel} on {workload_name}",
        f"kernel: {kernel}",
        f"workload: {workload_name}",
        f"source_sha256_16: {source_digest(kernel)}",
        f"fetch_kib_per_launch_raw: {fetch:.1f}",
        f"write_kib_per_launch_raw: {write:.1f}",
        f"copy_reference_mib: {copy_mib}",
        f"fetch_scale: {fscale:.4f}",
        f"write_scale: {wscale:.4f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
        f"algorithmic_bytes_per_launch: {algo:.0f}",
        f"traffic_over_algorithmic: {hbm / algo:.3f}",
    ]
    return "\n".join(lines)


def summarize_counters(kernel: str, dirs) -> str:
    """Markdown table of rocprofv3 --pmc runs (one or more output directories)
    for one kernel: each counter's average per dispatch, and the ratios the
    kernel's bound is read from, with their formulas."""
    sym = KERNEL_SYMBOLS[kernel]
    vals = {}
    for d in dirs:
        for r in _csv_rows(_find(d, "counter_collection.csv")):
            if sym in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: float(np.mean(v)) for k, v in vals.items()}
    out = [f"Counters of `{kernel}` (source digest {source_digest(kernel)}), average per "
           "dispatch:", "", "| counter | dispatches | average |", "|---|---|---|"]
    for k in sorted(avg):
        out.append(f"| {k} | {len(vals[k])} | {avg[k]:.6g} |")
    # GRBM_GUI_ACTIVE counts GPU-busy cycles summed over the 8 XCDs, so one
    # XCD's cycles are a eighth of it; the SQ cycle counters sum over all
    # 1024 SIMDs (256 CUs x 4).
    simds = 256 * 4
    xcds = 8
    derived = []

    def have(*names):
        return all(n in avg for n in names)
    if have("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"):
        derived.append(("MFMA busy, SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 "
                        "SIMDs)",
                        avg["SQ_VALU_MFMA_BUSY_CYCLES"] * xcds / (avg["GRBM_GUI_ACTIVE"] * simds)))
    if have("SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"):
        derived.append(("VALU active, 4 x SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 "
                        "SIMDs)",
                        4 * avg["SQ_ACTIVE_INST_VALU"] * xcds / (avg["GRBM_GUI_ACTIVE"] * simds)))
    if have("SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES"):
        derived.append(("MFMA cycles with VALU issuing beside them, "
                        "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES",
                        avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"]))
    if have("SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"):
        # Summed over every CU's LDS, as rocprofv3's LdsUtil takes it.
        derived.append(("LDS active, SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs)",
                        avg["SQ_LDS_IDX_ACTIVE"] * xcds / (avg["GRBM_GUI_ACTIVE"] * 256)))
    if have("SQ_INSTS_LDS_LOAD_BANDWIDTH", "GRBM_GUI_ACTIVE"):
        derived.append(("LDS bytes loaded per CU and cycle, 64 x SQ_INSTS_LDS_LOAD_BANDWIDTH / "
                        "(GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs)",
                        64 * avg["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * xcds / (avg["GRBM_GUI_ACTIVE"] * 256)))
    # Wave states, all in quad-cycles summed over the waves: waiting for
    # anything (a dependency, a barrier), ready but not picked for issue, and
    # issuing any instruction.
    for num, what in (("SQ_WAIT_ANY", "waiting for anything"),
                      ("SQ_WAIT_INST_ANY", "waiting for instruction issue"),
                      ("SQ_ACTIVE_INST_ANY", "issuing an instruction")):
        if have(num, "SQ_WAVE_CYCLES"):
            derived.append((f"wave-cycles {what}, {num} / SQ_WAVE_CYCLES",
                            avg[num] / avg["SQ_WAVE_CYCLES"]))
    for num in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_CVT",
                "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_ADD_F32",
                "SQ_INSTS_VALU_INT32", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
        if have(num, "SQ_INSTS_MFMA"):
            derived.append((f"{num} per MFMA instruction", avg[num] / avg["SQ_INSTS_MFMA"]))
    if have("GRBM_GUI_ACTIVE"):
        derived.append(("one XCD's busy cycles, GRBM_GUI_ACTIVE / 8", avg["GRBM_GUI_ACTIVE"] / xcds))
    if derived:
        out += ["", "| derived | value |", "|---|---|"]
        out += [f"| {name} | {value:.4g} |" for name, value in derived]
    return "\n".join(out)


def copy_reference(mib: int) -> None:
    """A plain device-to-device copy of `mib` MiB, for counter calibration."""
    import torch
    src = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB three times")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def host_threads() -> int:
    """Threads the host may use: every CPU the process sees, capped by
    OMP_NUM_THREADS when it is set (the share of a machine's cores given to
    one GPU)."""
    cap = os.environ.get("OMP_NUM_THREADS", "")
    n = os.cpu_count() or 1
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


def _oracle_step(w, pairs, threads):
    """Forward + backward of the fp32 oracle over the given (batch entry,
    head) pairs; returns (seconds, valid FLOPs at 14 d per attended pair)."""
    import oracle
    t0 = time.perf_counter()
    oracle.fwd(w.q, w.k, w.v, w.seq_lens, heads=pairs, precision="f32", threads=threads)
    oracle.bwd(w.q, w.k, w.v, w.do, w.seq_lens, heads=pairs, precision="f32", threads=threads)
    dt = time.perf_counter() - t0
    return dt, sum(14.0 * w.d * float(w.seq_lens[b]) ** 2 for b, _ in pairs)


def _pairs_within(w, per_pair_s: float, budget_s: float, threads: int, seed: int = 0):
    """(batch entry, head) pairs drawn at random until the estimated CPU time
    (per_pair_s per n^2, spread over `threads`) fills budget_s."""
    rng = np.random.default_rng(seed)
    all_pairs = [(int(b), h) for b in range(w.B) for h in range(w.H)]
    pairs, est = [], 0.0
    for idx in rng.permutation(len(all_pairs)):
        b, h = all_pairs[idx]
        cost = per_pair_s * float(w.seq_lens[b]) ** 2 / threads
        if est + cost > budget_s and pairs:
            break
        pairs.append((b, h))
        est += cost
    return pairs


def cpu_baseline(w, budget_all_s: float = 10.0, budget_one_s: float = 8.0):
    """The oracle (fp32 statement, as it stands) timed on the host: forward +
    backward in valid TFLOP/s, once on every host thread (the reported value)
    and once on a single thread, each over a bounded sample of (batch entry,
    head) pairs of the same workload."""
    threads = host_threads()
    b_med = int(np.argsort(w.seq_lens)[len(w.seq_lens) // 2])
    dt, _ = _oracle_step(w, [(b_med, 0)], 1)  # calibration: seconds per n^2 on one thread
    per_pair = max(dt, 1e-3) / float(w.seq_lens[b_med]) ** 2
    pairs_all = _pairs_within(w, per_pair, budget_all_s, threads, seed=0)
    dt_all, fl_all = _oracle_step(w, pairs_all, threads)
    pairs_one = _pairs_within(w, per_pair, budget_one_s, 1, seed=1)
    dt_one, fl_one = _oracle_step(w, pairs_one, 1)
    total = w.B * w.H
    return {"value": fl_all / dt_all / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(pairs_all)} of {total} (batch entry, head) pairs of the same "
                      f"workload, forward + backward, fp32 oracle, {dt_all:.1f} s on "
                      f"{threads} threads",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": fl_one / dt_one / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": f"{len(pairs_one)} of {total} pairs, {dt_one:.1f} s"}}


class HipTimer:
    """Timing events recorded on a HIP stream without the system-scope fence.

    A default event record writes the caches back and invalidates them; between
    kernels of one step that perturbs the next kernel and inflates both.  These
    events only order timestamps on the stream (hipEventDisableSystemFence), so
    the per-kernel durations add up to the step.  They come from the HIP
    runtime that torch itself loaded.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream_handle: int):
        import ctypes
        self._c = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                      ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._stream = ctypes.c_void_p(stream_handle)
        self._events = []

    def event(self):
        e = self._c.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(self._c.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self._events.append(e)
        return e

    def record(self, e) -> None:
        rc = self._hip.hipEventRecord(e, self._stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        f = self._c.c_float()
        rc = self._hip.hipEventElapsedTime(self._c.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def close(self) -> None:
        for e in self._events:
            self._hip.hipEventDestroy(e)
        self._events = []


# --------------------------------------------------------------------------
# Measurement suite (--suite): warm and cold kernel times, valid-work and
# tile-work TFLOP/s and algorithmic HBM GB/s for the benchmark shapes, the
# softmax variants at the single-cell shapes, a padding sweep and the
# long packed-document case.  Markdown on stdout; the default JSON line above
# is unaffected.
# --------------------------------------------------------------------------

SUITE_WARMUP = 20
SUITE_REPS = 50
SUITE_SETTLE_S = 0.3
FLUSH_BYTES = 1 << 30  # larger than the last-level cache, so each cold rep starts empty


def suite_bytes(kernel: str, w, variant: int, masked, ranges: bool = False) -> float:
    """Algorithmic HBM bytes of one launch: valid rows of the inputs read once,
    every row of the outputs written once; the softmax variants add O and the
    log-sum-exp rows; the block-mask builder reads the element mask once (or
    the key ranges, 8 bytes per row)."""
    valid = float(np.clip(w.seq_lens, 0, w.L).sum()) * w.H
    every = float(w.B) * w.L * w.H
    row = 2.0 * w.d
    if kernel == "blockmask":
        tiles = float(w.B) * (-(-w.L // w.block_q)) * (-(-w.L // w.block_k))
        if ranges:
            return 8.0 * w.B * w.L + tiles
        return (float(w.B) * w.L * w.L if masked else 4.0 * w.B) + tiles
    soft = variant != 0
    if kernel == "fwd":
        return (3 * valid + every) * row + (every * 4.0 if soft else 0.0)
    reads = 5 if soft else 4
    writes = {"bwd": 3, "dkdv": 2, "dq": 1}[kernel]
    return (reads * valid + writes * every) * row + (valid * 4.0 if soft else 0.0)


class SuiteTimer:
    """Per-launch durations from fence-free HIP events on one stream."""

    def __init__(self, stream):
        self.stream = stream
        self.timer = HipTimer(stream.cuda_stream)

    def steps(self, fns, reps=SUITE_REPS, settle_s=SUITE_SETTLE_S):
        """Repeats the sequence fns (one step) and returns per-launch times in
        us, shape [reps, len(fns)].  Untimed steps run first until the clocks
        have settled: at least SUITE_WARMUP steps and settle_s seconds."""
        import torch
        t0, done = time.perf_counter(), 0
        while done < SUITE_WARMUP or time.perf_counter() - t0 < settle_s:
            for fn in fns:
                fn()
            done += 1
            if done % 10 == 0:
                torch.cuda.synchronize()
        ev = [self.timer.event() for _ in range(reps * len(fns) + 1)]
        torch.cuda.synchronize()
        self.timer.record(ev[0])
        for i in range(reps):
            for j, fn in enumerate(fns):
                fn()
                self.timer.record(ev[i * len(fns) + j + 1])
        torch.cuda.synchronize()
        t = [self.timer.elapsed_ms(ev[i], ev[i + 1]) for i in range(reps * len(fns))]
        return np.array(t).reshape(reps, len(fns)) * 1e3

    def cold(self, fn, flush, reps=SUITE_REPS):
        """Per-launch times in us of fn run right after a fill of `flush`."""
        import torch
        fn()
        ev = [self.timer.event() for _ in range(2 * reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            flush.fill_(float(i))
            self.timer.record(ev[2 * i])
            fn()
            self.timer.record(ev[2 * i + 1])
        torch.cuda.synchronize()
        return np.array([self.timer.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(reps)]) * 1e3

    def close(self):
        self.timer.close()


# Which outputs a suite row's kernel writes (for its parity errors).
SUITE_OUTPUTS = {"fwd": ("O",), "bwd": ("dQ", "dK", "dV"), "dkdv": ("dK", "dV"), "dq": ("dQ",)}


def attach_parity(rows, path) -> None:
    """Adds max_abs / rel_l2 (worst over the row's outputs) to the suite rows
    whose workload, variant, block and mask form the full-size parity tests
    compared against the oracle; `path` is the JSON-lines log those tests
    write (SIGATTN_PARITY_LOG).  Rows without a record keep no error fields."""
    if not path or not os.path.exists(path):
        return
    with open(path) as f:
        recs = [json.loads(line) for line in f if line.strip()]
    for r in rows:
        outs = SUITE_OUTPUTS.get(r.get("kernel"))
        if outs is None:
            continue
        hit = [x for x in recs
               if (x["B"], x["H"], x["L"], x["d"]) == (r["B"], r["H"], r["L"], r["d"])
               and x["variant"] == r["variant"] and x.get("block") == r["block"]
               and x.get("mask", "none") == r["mask"] and x["output"] in outs]
        if hit:
            r["max_abs"] = max(x["max_abs"] for x in hit)
            r["rel_l2"] = max(x["rel_l2"] for x in hit)
            r["parity_outputs"] = sorted({x["output"] for x in hit})


def run_suite(args) -> int:
    import torch

    import synthetic as syn
    import varlen_attention_amd as va

    assert torch.cuda.is_available(), "the suite needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    timer = SuiteTimer(stream)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    rows = []
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name}: {props.multi_processor_count} compute units")

    def gpu(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def workload(w, variant, mask_form, block, tiles):
        return {"seed": args.seed, "B": w.B, "H": w.H, "L": w.L, "d": w.d,
                "sum_n": int(w.seq_lens.sum()), "valid_pairs": int(w.valid_pairs) * w.H,
                "kept_tiles": tiles, "block": block, "mask": mask_form,
                "variant": ("sigmoid", "softmax", "softmax_1", "differential")[int(variant)]}

    def case(label, w, variant=syn.SIGMOID, bias=syn.BIAS_LOG_SEQLEN, block=128, kernels=("fwd", "bwd"),
             cold=True, ranges=False):
        """Times blockmask_build, fwd and bwd of workload w; one table row each.
        ranges: the element mask as key ranges instead of the dense mask."""
        log(f"case {label}: B={w.B} H={w.H} L={w.L} d={w.d} block={block} variant={variant}")
        q, k, v = gpu(w.q), gpu(w.k), gpu(w.v)
        do = gpu(w.do) if w.do is not None else None
        n = torch.from_numpy(w.seq_lens).to(dev)
        mask = torch.from_numpy(w.mask).to(dev) if w.mask is not None and not ranges else None
        kr = torch.from_numpy(w.key_range).to(dev) if ranges else None
        form = {"key_range": kr} if ranges else {"mask": mask}
        w.block_q = w.block_k = block
        bm, sched = va.blockmask_build(n, w.L, block, block, heads=w.H, **form)
        tiles = int((bm != 0).sum().item()) * w.H  # kept tiles (entries are 0, 1 or 3)
        pairs = w.valid_pairs * w.H
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev) if variant else None
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        fns = {
            "blockmask": lambda: va.blockmask_build(n, w.L, block, block, out=bm, heads=w.H,
                                                    schedule=sched, **form),
            "fwd": lambda: va.sigattn_fwd(q, k, v, n, block_mask=bm, schedule=sched, bias=bias,
                                          variant=variant, block_q=block, block_k=block, out=o,
                                          lse=lse, **form),
            "bwd": lambda: va.sigattn_bwd(q, k, v, do, n, block_mask=bm, schedule=sched,
                                          bias=bias, variant=variant, block_q=block,
                                          block_k=block, dq=dq, dk=dk, dv=dv,
                                          o=o if variant else None, lse=lse, **form),
            "dkdv": lambda: va.sigattn_bwd_dkdv(q, k, v, do, n, block_mask=bm, schedule=sched,
                                                bias=bias, variant=variant, block_q=block,
                                                block_k=block, dk=dk, dv=dv,
                                                o=o if variant else None, lse=lse, **form),
            "dq": lambda: va.sigattn_bwd_dq(q, k, v, do, n, block_mask=bm, schedule=sched,
                                            bias=bias, variant=variant, block_q=block,
                                            block_k=block, dq=dq, o=o if variant else None,
                                            lse=lse, **form),
        }
        fns["fwd"]()
        torch.cuda.synchronize()
        # The halves alone count the products they execute: S, dP, dV, dK
        # (8d) and S, dP, dQ (6d).
        per_pair = {"fwd": 4.0 * w.d, "bwd": 10.0 * w.d, "dkdv": 8.0 * w.d, "dq": 6.0 * w.d}
        names = ("blockmask",) + tuple(kernels)
        warm = timer.steps([fns[kern] for kern in names])
        tot = warm.sum(axis=1)
        for j, kern in enumerate(names):
            cold_t = timer.cold(fns[kern], flush) if cold else None
            med = float(np.median(warm[:, j]))
            r = {"case": label, "kernel": kern, "warm_med_us": med,
                 "warm_min_us": float(warm[:, j].min()),
                 "cold_med_us": float(np.median(cold_t)) if cold else None,
                 "gbs": suite_bytes(kern, w, variant, mask is not None, ranges) / (med * 1e-6) / 1e9}
            if kern in per_pair:
                r["valid_tf"] = per_pair[kern] * pairs / (med * 1e-6) / 1e12
                r["tile_tf"] = per_pair[kern] * tiles * block * block / (med * 1e-6) / 1e12
            r.update(workload(w, variant, "key ranges" if ranges else
                              ("dense" if mask is not None else "none"), block, tiles))
            rows.append(r)
            log(f"  {kern}: warm median {med:.2f} us, min {warm[:, j].min():.2f} us"
                + (f", cold median {np.median(cold_t):.2f} us" if cold else ""))
        flops = sum(per_pair[kern] for kern in kernels) * pairs
        rows.append({**workload(w, variant, "key ranges" if ranges else
                                ("dense" if mask is not None else "none"), block, tiles),
                     "case": label, "kernel": "step", "warm_med_us": float(np.median(tot)),
                     "warm_min_us": float(tot.min()), "cold_med_us": None,
                     "valid_tf": flops / (np.median(tot) * 1e-6) / 1e12,
                     "tile_tf": flops / pairs * tiles * block * block / (np.median(tot) * 1e-6) / 1e12,
                     "gbs": None})
        del q, k, v, do, o, dq, dk, dv, mask, kr, bm, sched
        torch.cuda.empty_cache()
        return rows[-1]

    # Single cell, sigmoid with bias -ln n, block 128 and 64.
    w = syn.single_cell(args.seed, tensors=("q", "k", "v", "do"))
    case("single cell, sigmoid, block 128", w)
    case("single cell, sigmoid, block 64", w, block=64)
    # The softmax variants at the same shapes (no bias).
    case("single cell, softmax", w, variant=syn.SOFTMAX, bias=syn.BIAS_NONE)
    case("single cell, softmax_1", w, variant=syn.SOFTMAX1, bias=syn.BIAS_NONE)
    # Backward workload: lengths clipped to [200, 4096] (the same draw).
    wb = syn.single_cell_backward(args.seed)
    case("single cell bwd (clip 4096)", wb, kernels=("bwd",))
    case("single cell bwd halves, two launches", wb, kernels=("dkdv", "dq"))
    # Padding sweep: the same lengths padded to 1x, 2x and 4x the longest.
    maxn = int(w.seq_lens.max())
    for f in (1, 2, 4):
        ws = syn.make_workload(f"pad{f}", seed=args.seed, B=w.B, H=w.H, d=w.d, lengths="lognormal",
                               lo=200, hi=2048, seq_lens=w.seq_lens, L=f * maxn,
                               tensors=("q", "k", "v", "do"))
        case(f"padding sweep, L = {f} x max n", ws, cold=False)
    # Equal valid tokens with no padding and with 25% padding.
    flat = np.full(32, 768, dtype=np.int32)
    ramp = np.rint(np.linspace(512, 1024, 32)).astype(np.int32)
    for label, lens in (("0% padding (n = 768 for all 32)", flat),
                        ("25% padding (n = 512..1024, L = 1024)", ramp)):
        wp = syn.make_workload("pad_pair", seed=args.seed, B=32, H=8, d=64, lengths="uniform",
                               lo=0, hi=0, seq_lens=lens, tensors=("q", "k", "v", "do"))
        case(label, wp, cold=False)
    sc_B, sc_H, sc_L, sc_lens = w.B, w.H, w.L, w.seq_lens.copy()
    del w, wb
    # Differential attention at the single-cell lengths, d = 64 (both maps in
    # one forward launch) and d = 128 (a softmax pass for map 1, then map 2
    # combined at its store), against two softmax forward launches (4 d flops
    # per pair and map).
    for dd in (64, 128):
        if dd == 64:
            wd = syn.single_cell(args.seed, tensors=("q", "k", "v", "do"))
        else:
            wd = syn.make_workload(f"single_cell_d{dd}", seed=args.seed, B=sc_B, H=sc_H, d=dd,
                                   lengths="lognormal", lo=0, hi=0, seq_lens=sc_lens, L=sc_L,
                                   tensors=("q", "k", "v", "do"))
        rng = np.random.default_rng(args.seed + 1)
        q1, k1, v = gpu(wd.q), gpu(wd.k), gpu(wd.v)
        q2, k2 = gpu(syn.random_tensor(rng, wd.q.shape)), gpu(syn.random_tensor(rng, wd.k.shape))
        n = torch.from_numpy(wd.seq_lens).to(dev)
        bm, sched = va.blockmask_build(n, wd.L, 128, 128, heads=wd.H)
        dout = gpu(wd.do)
        o, o2 = torch.empty_like(q1), torch.empty_like(q1)
        label = f"single cell{'' if dd == 64 else f', d = {dd}'}, differential (lambda 0.8)"
        log(f"case {label}")
        _, l1, l2, m1, m2 = va.sigattn_diff_fwd(q1, k1, q2, k2, v, n, 0.8, block_mask=bm,
                                                schedule=sched, return_maps=True)
        grads = [torch.empty_like(q1) for _ in range(5)]
        fns = [lambda: va.sigattn_diff_fwd(q1, k1, q2, k2, v, n, 0.8, block_mask=bm,
                                           schedule=sched, out=o),
               lambda: va.sigattn_fwd(q1, k1, v, n, block_mask=bm, schedule=sched,
                                      variant=syn.SOFTMAX, bias=0, out=o),
               lambda: va.sigattn_fwd(q2, k2, v, n, block_mask=bm, schedule=sched,
                                      variant=syn.SOFTMAX, bias=0, out=o2),
               lambda: va.sigattn_diff_bwd(q1, k1, q2, k2, v, dout, m1, m2, l1, l2, n, 0.8,
                                           block_mask=bm, schedule=sched, grads=grads)]
        warm = timer.steps(fns)
        cold = timer.cold(fns[0], flush)
        tiles = int((bm != 0).sum().item()) * wd.H
        pairs = wd.valid_pairs * wd.H
        valid_rows = float(np.clip(wd.seq_lens, 0, wd.L).sum()) * wd.H
        all_rows = float(wd.B) * wd.L * wd.H
        # (name, maps, flops per pair and map, rows read, rows written)
        kinds = (("diff fwd", 2, 4, 5, 1), ("softmax fwd (map 1)", 1, 4, 3, 1),
                 ("softmax fwd (map 2)", 1, 4, 3, 1), ("diff bwd", 2, 10, 10, 5))
        for j, (kern, maps, fpp, rd, wr) in enumerate(kinds):
            med = float(np.median(warm[:, j]))
            algo = (rd * valid_rows + wr * all_rows) * 2.0 * wd.d
            rows.append({**workload(wd, 3 if j in (0, 3) else syn.SOFTMAX, "none", 128, tiles),
                         "case": label, "kernel": kern, "warm_med_us": med,
                         "warm_min_us": float(warm[:, j].min()),
                         "cold_med_us": float(np.median(cold)) if j == 0 else None,
                         "valid_tf": fpp * wd.d * maps * pairs / (med * 1e-6) / 1e12,
                         "tile_tf": fpp * wd.d * maps * tiles * 128 * 128 / (med * 1e-6) / 1e12,
                         "gbs": algo / (med * 1e-6) / 1e9})
            log(f"  {kern}: warm median {med:.2f} us")
        del wd, q1, k1, q2, k2, v, dout, o, o2, bm, sched, grads, l1, l2, m1, m2, fns
        torch.cuda.empty_cache()
    # Long packed documents: causal mask within documents, d = 128.
    wl = syn.long_packed_docs(args.seed, tensors=("q", "k", "v", "do"))
    case("long packed documents, causal mask", wl)
    case("long packed documents, causal key ranges", wl, ranges=True)
    timer.close()

    print(f"Measurement suite on {props.name} ({props.multi_processor_count} CUs), seed {args.seed}.")
    print(f"Warm: steps (block mask, forward, backward) repeated until the clocks settle "
          f"(at least {SUITE_WARMUP} steps and {SUITE_SETTLE_S} s), then {SUITE_REPS} timed steps; "
          f"cold: a {FLUSH_BYTES >> 20} MiB fill before each of {SUITE_REPS} timed launches of "
          "one kernel.  Times are HIP-event durations per launch; rates use the warm median; "
          "'step' is the sum of the step's kernels.")
    print("Valid TF counts attended (query, key) pairs (4d per pair forward, 10d backward; the "
          "backward halves alone 8d and 6d, the products they execute); tile TF "
          "counts every pair of the tiles the block mask keeps; GB/s is algorithmic bytes "
          "(valid input rows read once, every output row written once).")
    print()
    attach_parity(rows, args.parity_log)
    if args.suite_jsonl:
        with open(args.suite_jsonl, "w") as f:
            for r in rows:
                f.write(json.dumps({**r, "peak_bf16_tflops": PEAK_BF16_TFLOPS,
                                    "frac_peak_valid": (r["valid_tf"] / PEAK_BF16_TFLOPS
                                                        if r.get("valid_tf") else None),
                                    "frac_hbm": (r["gbs"] / PEAK_HBM_GBS if r.get("gbs") else None)})
                        + "\n")
    print("| case | kernel | warm median (us) | warm min (us) | cold median (us) | valid TFLOP/s | "
          "tile TFLOP/s | algorithmic GB/s |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        f = lambda key, fmt: (fmt.format(r[key]) if r.get(key) is not None else "-")
        print(f"| {r['case']} | {r['kernel']} | {r['warm_med_us']:.2f} | {r['warm_min_us']:.2f} | "
              f"{f('cold_med_us', '{:.2f}')} | {f('valid_tf', '{:.1f}')} | {f('tile_tf', '{:.1f}')} | "
              f"{f('gbs', '{:.0f}')} |")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="single_cell",
                    choices=("single_cell", "long_docs_ranges", "long_docs_mask"),
                    help="the step's workload: the single-cell benchmark (default), or, for "
                         "profiling, the long packed documents (B8 H16 d128, causal within "
                         "documents) with the mask as key ranges or as the dense array")
    ap.add_argument("--copy-reference-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="print a markdown table of a rocprofv3 --stats output directory")
    ap.add_argument("--skip-dispatches", type=int, default=0,
                    help="with --summarize-stats: dispatches of each kernel to leave out")
    ap.add_argument("--summarize-traffic", nargs=5,
                    metavar=("KERNEL", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="print the HBM traffic summary of KERNEL from FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--summarize-counters", nargs="+", metavar=("KERNEL", "DIR"),
                    help="print the counter summary of KERNEL from rocprofv3 --pmc output DIRs")
    ap.add_argument("--suite", action="store_true",
                    help="run the measurement suite (markdown on stdout) instead of the step")
    ap.add_argument("--suite-jsonl", metavar="PATH",
                    help="with --suite: also write one JSON line per measured row to PATH")
    ap.add_argument("--parity-log", metavar="PATH",
                    help="with --suite: the JSON-lines log of the full-size parity tests "
                         "(SIGATTN_PARITY_LOG); their errors are attached to matching rows")
    args = ap.parse_args()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, args.skip_dispatches))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters[0], args.summarize_counters[1:]))
        return 0
    if args.summarize_traffic:
        import synthetic as syn
        w = syn.single_cell(args.seed, tensors=())
        print(summarize_traffic(*args.summarize_traffic, args.copy_mib, w,
                                "single_cell_b32h8d64_lognormal800"))
        return 0
    if args.copy_reference_mib:
        copy_reference(args.copy_reference_mib)
        return 0
    if args.suite:
        return run_suite(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by batch entry and head without any exchange).", file=sys.stderr)
        return 2

    import torch

    import synthetic as syn
    import varlen_attention_amd as va

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    form = {}  # the element mask, for the long-document workloads
    if args.workload == "single_cell":
        w = syn.single_cell(args.seed, tensors=("q", "k", "v", "do"))
        workload = "single_cell_b32h8d64_lognormal800"
    else:
        w = syn.long_packed_docs(args.seed, tensors=("q", "k", "v", "do"))
        if args.workload == "long_docs_ranges":
            workload = "long_docs_b8h16d128_causal_ranges"
            form = {"key_range": torch.from_numpy(w.key_range).to(dev)}
        else:
            workload = "long_docs_b8h16d128_causal_mask"
            form = {"mask": torch.from_numpy(w.mask).to(dev)}
    B, H, L, d = w.B, w.H, w.L, w.d
    pairs = w.valid_pairs  # summed over the batch, per head
    log(f"workload {workload}: B={B} H={H} L={L} d={d} sum_n={int(w.seq_lens.sum())} "
        f"valid pairs/head={pairs}")

    def gpu(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (gpu(t) for t in (w.q, w.k, w.v, w.do))
    n = torch.from_numpy(w.seq_lens).to(dev)
    bq = bk = 128
    bm = torch.empty((B, va.num_tiles(L, bq), va.num_tiles(L, bk)), dtype=torch.uint8, device=dev)
    sched = torch.empty(va.schedule_bytes(B, H, L, bq, bk, dense_mask="mask" in form),
                        dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()

    names = ["blockmask", "fwd", "bwd"]

    timer = HipTimer(stream.cuda_stream)

    def step(events=None):
        def mark(i):
            if events is not None:
                timer.record(events[i])
        mark(0)
        va.blockmask_build(n, L, bq, bk, out=bm, heads=H, schedule=sched, **form)
        mark(1)
        va.sigattn_fwd(q, k, v, n, block_mask=bm, schedule=sched, out=o, block_q=bq, block_k=bk,
                       **form)
        mark(2)
        va.sigattn_bwd(q, k, v, do, n, block_mask=bm, schedule=sched, dq=dq, dk=dk, dv=dv,
                       block_q=bq, block_k=bk, **form)
        mark(3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    ev = [[timer.event() for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per_kernel = {nm: float(np.mean([timer.elapsed_ms(ev[s][i], ev[s][i + 1])
                                     for s in range(args.steps)]))
                  for i, nm in enumerate(names)}
    timer.close()
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step; per kernel (ms): "
        + ", ".join(f"{k_}={v_:.4f}" for k_, v_ in per_kernel.items()))

    flops_fwd = 4.0 * d * H * pairs
    flops_bwd = 10.0 * d * H * pairs
    value = (flops_fwd + flops_bwd) / (ms_step * 1e-3) / 1e12
    # Per-kernel algorithmic FLOPs per launch: valid work, 4 d per attended
    # pair forward and 10 d backward (its five products).  The backward
    # recomputes S and dP for dQ, so it executes 14 d per pair; that rate is
    # reported beside it as `executed_tflops`, never as the roofline figure.
    algo = {"fwd": flops_fwd, "bwd": flops_bwd}
    executed = {"fwd": flops_fwd, "bwd": 14.0 * d * H * pairs}
    dominant = max(algo, key=lambda k_: per_kernel[k_])
    achieved = algo[dominant] / (per_kernel[dominant] * 1e-3) / 1e12
    traffic = read_traffic(dominant, workload)
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    kernels = {}
    for nm in names:
        ent = {"ms": round(per_kernel[nm], 4)}
        if nm in algo:
            tf = algo[nm] / (per_kernel[nm] * 1e-3) / 1e12
            ent.update(tflops=round(tf, 2), frac_peak=round(tf / PEAK_BF16_TFLOPS, 4),
                       executed_tflops=round(executed[nm] / (per_kernel[nm] * 1e-3) / 1e12, 2))
        kernels[nm] = ent

    cpu = None
    if not args.no_cpu_baseline and not form:
        log("timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(w)
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "B": B, "H": H, "L": L, "d": d,
                   "sum_n": int(w.seq_lens.sum()), "valid_pairs_per_head": int(pairs),
                   "block": bq, "variant": "sigmoid", "bias": "-ln n", "seed": args.seed,
                   "mask": next(iter(form), "padding only"),
                   "step": "blockmask_build (block mask + schedule) + fwd + bwd (dK/dV and dQ "
                           "in one launch)",
                   "parallelism": "single GPU"},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
