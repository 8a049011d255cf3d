#!/usr/bin/env python3
"""Attention throughput on one MI355X: forward + backward, bf16.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
fa_fwd (O and LSE) followed by fa_bwd (the query-outer dQ kernel, which also
forms D_i and L_i log2 e, then the key-outer dK/dV kernel), all on torch's
current stream, with the inputs
already resident in device memory. W untimed steps, then exactly K timed steps
between two device synchronisations. One JSON line is printed.

FLOPs follow the attention convention: 4 B H N^2 d for the forward (two
N x N x d products), 2.5x that for the backward (five products), halved when
causal. ``value`` is fwd+bwd TFLOP/s over the wall time of the timed steps.

The ``roofline`` object is for the dominant kernel, the backward's dK/dV
kernel: its algorithmic FLOPs per launch (four of the backward's five
N x N x d products: S, dP, dV, dK; 8 B H N^2 d, halved when causal) divided
by its average duration, measured with HIP events recorded on the launch
stream immediately before and after it (fa_bwd_timed), against the bf16 dense
matrix-core peak. ``traffic``
is read from the committed rocprofv3 counter summary for this kernel and
workload when that summary was taken from the current kernel source, else
null.

``cpu_baseline`` times the fp64 CPU oracle (materialised S and P, NumPy/BLAS)
on a bounded sample of the same workload -- whole heads, fwd+bwd, until about
10 s of CPU work -- and scales it to the same TFLOP/s convention.

    python bench.py --sweep [--out FILE] [--only PREFIX ...]
    python bench.py --fp8 [--out FILE] [--only PREFIX ...]

times fa_fwd and fa_bwd separately on every parity workload with a backward
(the BERT- and GPT-2-shaped ones, the grouped-head one, the 18-point
(N, d, causal) sweep and the packed variable-length batches, which use
fa_fwd_varlen / fa_bwd_varlen):
10 warm-up iterations, then at least 50 timed iterations and 200 ms, HIP
events around each call; median and minimum. Per point it reports TFLOP/s,
the fraction of the bf16 matrix-core peak and of the binding roof
(min(peak, arithmetic intensity x 8 TB/s) over compulsory HBM bytes), and the
compulsory bytes per second. Points whose working set is at most 256 MB are
also timed cold: a 512 MB buffer is written between calls.

    python bench.py --fp8 [--out FILE] [--only PREFIX ...] [--calibrate-copy MIB]

times the FP8 forward on every padded workload (d = 64, 128, 256) without a
window or block mask: the three block encodings (fa_fp8_quantize for Q and K with the
Hadamard rotation, for V in the transposed layout), fa_fwd_fp8 on the codes,
and the bf16 fa_fwd on the same inputs, with the same iteration rule; it
reports TFLOP/s against the fp8 dense peak (5.0 PFLOP/s) and the speed-up
over bf16.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E bandwidth (published)
# The headline dK/dV kernel, the dispatch that picks it and their shared helpers.
KERNEL_SOURCES = ("exact_io_aware_fa_amd/csrc/kernels/fa_bwd_dkdv_wide.hip",
                  "exact_io_aware_fa_amd/csrc/kernels/fa_bwd_bf16.hip",
                  "exact_io_aware_fa_amd/csrc/kernels/fa_device.h")
TRAFFIC_WORKLOAD = "long_causal_b1_h32_n16384_d128"
def dkdv_kernel_name(d: int, n: int) -> str:
    """The dK/dV kernel a bf16 backward of head dimension d and n rows runs."""
    if d == 64:
        return "bwd_dkdv_d64_kernel" if n <= 1024 else "bwd_dkdv_kernel"
    if d == 128:
        return "bwd_dkdv_wide_kernel" if n >= 4096 else "bwd_dkdv_kernel"
    return "bwd_dkdv_d256_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_dkdv_%s_traffic.json" % TRAFFIC_WORKLOAD)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw HIP events through the HIP runtime torch already loaded."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.rt.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def record(self, ev: int, stream: int) -> None:
        rc = self.rt.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a: int, b: int) -> float:
        self.rt.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, ev: int) -> None:
        self.rt.hipEventDestroy(ev)


def host_info() -> dict:
    """The host the CPU oracle runs on: CPU model, the cores this process may
    use, and the BLAS library NumPy calls with its thread count."""
    import numpy  # noqa: F401  (loads the BLAS threadpoolctl reports)
    from threadpoolctl import threadpool_info

    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    vendor = ", ".join(sorted({"%s %s" % (i.get("internal_api", "?"), i.get("version", "?"))
                               for i in blas})) or "none found"
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "blas": vendor, "blas_threads": int(threads)}


class SclkSampler:
    """Samples the GPU's current shader clock from sysfs (pp_dpm_sclk, the
    level marked '*') in a background thread while the timed steps run; the
    main thread waits in a device synchronisation meanwhile. Reports the
    median, minimum and maximum in MHz and the number of samples, and, where
    the device's hwmon node exposes them, the board power read alongside
    (power1_average or power1_input, microwatts) and its cap (power1_cap)."""

    def __init__(self, period_s: float = 0.004):
        import glob
        import threading

        cands = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = cands[0] if len(cands) == 1 else None
        self.note = ("pp_dpm_sclk of %s" % self.path if self.path else
                     "no unique pp_dpm_sclk (%d found)" % len(cands))
        self.period = period_s
        self.samples = []
        self.power = []
        self.power_path = self.power_cap = None
        if self.path:
            dev = os.path.dirname(self.path)
            for name in ("power1_average", "power1_input"):
                found = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", name)))
                if found:
                    self.power_path = found[0]
                    break
            if self.power_path:
                try:
                    with open(os.path.join(os.path.dirname(self.power_path), "power1_cap")) as f:
                        self.power_cap = float(f.read().strip()) / 1e6
                except (OSError, ValueError):
                    self.power_cap = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().lower().split("mhz")[0])
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except (OSError, ValueError, IndexError):
                v = None
            if v is not None:
                self.samples.append(v)
            if self.power_path:
                try:
                    with open(self.power_path) as f:
                        self.power.append(float(f.read().strip()) / 1e6)
                except (OSError, ValueError):
                    pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def result(self) -> dict:
        import statistics

        if not self.samples:
            return {"source": self.note, "samples": 0}
        out = {"median_mhz": statistics.median(self.samples), "min_mhz": min(self.samples),
               "max_mhz": max(self.samples), "samples": len(self.samples),
               "source": self.note + ", sampled during the timed steps"}
        if self.power:
            out.update(power_median_w=round(statistics.median(self.power), 1),
                       power_max_w=round(max(self.power), 1), power_cap_w=self.power_cap,
                       power_source=os.path.basename(self.power_path))
        return out


def cpu_baseline(w, inp, budget_s: float = 10.0) -> dict:
    """Time the fp64 oracle on whole heads (fwd+bwd) until ~budget_s."""
    import oracle

    heads = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    kv = inp["kv_len"]
    group = w.heads // w.kv_heads
    spent, done = 0.0, 0
    for b, h in heads:
        args = [inp[x][b, h if x in ("q", "do") else h // group].float().double().numpy()
                for x in ("q", "k", "v", "do")]
        t0 = time.perf_counter()
        oracle.head_backward(*args, w.softmax_scale, w.causal,
                             None if kv is None else int(kv[b]))
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    per_head = spent / done
    flops_per_head = (w.flops_fwd() + w.flops_bwd()) / (w.batch * w.heads)
    host = host_info()
    return {
        "value": flops_per_head / per_head / 1e12,
        "unit": "TFLOP/s",
        "cores": host["blas_threads"],
        "kind": "oracle",
        "sample": (f"{done} of {w.batch * w.heads} heads, fwd+bwd, fp64 NumPy "
                   f"(materialised S, P, dP, dS; no causal skipping), "
                   f"{per_head:.2f} s per head; FLOPs counted as for the GPU"),
        "cpu_model": host["cpu_model"],
        "affinity_cores": host["affinity_cores"],
        "blas": host["blas"],
    }


def cpu_baseline_fp8(w, inp, signs, budget_s: float = 10.0, rows: int = 1024) -> dict:
    """Time the FP8 oracle (fp64 NumPy) on one head after another until
    ~budget_s: the encoding of the head's Q, K, V, then the forward on codes
    for `rows` evenly spaced query rows (the oracle's row subset). FLOPs:
    4 d per visible (query, key) pair of the sampled rows, as for the GPU."""
    import numpy as np

    from oracle import fp8 as of
    from oracle.attention import visible_mask

    group = w.heads // w.kv_heads
    spent, flops, done = 0.0, 0.0, 0
    sg = signs.cpu().numpy().astype(np.float64)
    sel = np.linspace(0, w.n - 1, min(rows, w.n)).astype(np.int64)
    for b in range(w.batch):
        for h in range(w.heads):
            q = inp["q"][b:b + 1, h:h + 1].float().double().numpy()
            k = inp["k"][b:b + 1, h // group:h // group + 1].float().double().numpy()
            v = inp["v"][b:b + 1, h // group:h // group + 1].float().double().numpy()
            kv = None if inp["kv_len"] is None else int(inp["kv_len"][b])
            t0 = time.perf_counter()
            qc, qs = of.quantize(q, sg)
            kc, ks = of.quantize(k, sg)
            vc, vs = of.quantize(v)
            of.fp8_head_forward(qc[0, 0], qs[0, 0], kc[0, 0], ks[0, 0], vc[0, 0], vs[0, 0], w.n,
                                w.softmax_scale, w.causal, kv, rows=sel)
            spent += time.perf_counter() - t0
            flops += 4.0 * w.d * visible_mask(w.n, w.causal, kv, sel).sum()
            done += 1
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    host = host_info()
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": host["blas_threads"],
            "kind": "oracle",
            "sample": f"{done} head(s): encode Q, K, V of the head, then the forward of "
                      f"{len(sel)} evenly spaced query rows against all keys, fp64 NumPy, "
                      f"{spent / done:.2f} s per head",
            "cpu_model": host["cpu_model"], "affinity_cores": host["affinity_cores"],
            "blas": host["blas"]}


def load_traffic(src_hash: str, workload: str):
    """HBM bytes per dK/dV launch from the committed counter summary, or None
    when that summary is for another workload or an older kernel source."""
    if workload != TRAFFIC_WORKLOAD:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def _short(name: str) -> str:
    for key in ("fwd_bf16_kernel", "fwd_bf16_d64_kernel",
                "bwd_dkdv_kernel", "bwd_dkdv_d64_kernel", "bwd_dkdv_d256_kernel", "bwd_dkdv_wide_kernel",
                "bwd_dq_kernel", "bwd_dq_d256_kernel", "bwd_prep_kernel", "fwd_fp32_kernel",
                "bwd_fp32_kernel", "fwd_fp8_kernel", "fp8_quant_kernel", "copyBuffer"):
        if key in name:
            if key == "copyBuffer":
                return name
            rest = name[name.find(key) + len(key):]
            return key + rest.split("(")[0] if rest.startswith("<") else key
    return name[:60]


XCDS = 8                # MI355X: 8 accelerator dies (GRBM counters add over them)
SIMDS = 256 * 4         # 256 compute units x 4 SIMDs
MFMA_FLOP_PER_CLK = 1024  # bf16 32x32x16 product: 32768 FLOP in 32 cycles per SIMD


def summarize_sq(sq_db) -> list:
    """Markdown lines for an SQ counter pass: per kernel, the shader clock
    the kernel ran at (GRBM_GUI_ACTIVE per die over the dispatch duration),
    the matrix-core FLOPs counted by the hardware (SQ_INSTS_VALU_MFMA_MOPS_BF16,
    512 FLOP each) and their rate, matrix-core busy time as a fraction of all
    SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES), vector instructions per matrix
    instruction, and LDS bank conflicts (SQ_LDS_BANK_CONFLICT cycles over
    SQ_LDS_IDX_ACTIVE cycles)."""
    import sqlite3

    per = {}
    for kn, ctr, val, dur, did in sqlite3.connect(sq_db).execute(
            "select kernel_name, counter_name, value, duration, dispatch_id from counters_collection"):
        d = per.setdefault(_short(kn), {}).setdefault(did, {"dur": dur})
        d[ctr] = d.get(ctr, 0.0) + val
    lines = ["", "## Clock, matrix cores and LDS (`--pmc` SQ pass)", "",
             "Per dispatch, averaged: clock = GRBM_GUI_ACTIVE / %d dies / duration; FLOP = "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x "
             "cycles); peak at clock = %d SIMDs x %d FLOP/cycle x clock; LDS conflicts = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. Durations are those of the counter pass "
             "(dispatches serialised by the profiler)." % (XCDS, SIMDS, SIMDS, MFMA_FLOP_PER_CLK), "",
             "| kernel | dispatches | us | clock GHz | MFMA TFLOP | TFLOP/s | peak at clock TFLOP/s | "
             "MFMA busy | VALU instr per MFMA instr | LDS bank-conflict cycles / LDS active |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for k, ds in per.items():
        if k.startswith("__amd") or k.startswith("void at::"):
            continue
        n = len(ds)

        def avg(c):
            return sum(d.get(c, 0.0) for d in ds.values()) / n
        dur = sum(d["dur"] for d in ds.values()) / n
        cyc = avg("GRBM_GUI_ACTIVE") / XCDS
        if dur <= 0 or cyc <= 0:
            continue
        clk = cyc / dur
        flop = avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        mfma_instr = flop / 32768.0
        busy = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (SIMDS * cyc)
        valu = (avg("SQ_INSTS_VALU") - mfma_instr) / mfma_instr if mfma_instr else float("nan")
        lds_act = avg("SQ_LDS_IDX_ACTIVE")
        conf = avg("SQ_LDS_BANK_CONFLICT") / lds_act if lds_act else 0.0
        lines.append("| `%s` | %d | %.1f | %.2f | %.3f | %.0f | %.0f | %.3f | %.2f | %.4f |" % (
            k, n, dur / 1e3, clk, flop / 1e12, flop / dur / 1e3,
            SIMDS * MFMA_FLOP_PER_CLK * clk / 1e3, busy, valu, conf))
    return lines


def summarize_tcc(tcc_db) -> list:
    """Markdown lines for an L2 pass (TCC_HIT_sum, TCC_MISS_sum): per kernel,
    the L2 requests per dispatch and the fraction that hit. A miss goes on
    to the Infinity Cache (MALL) or HBM; FETCH_SIZE counts the bytes those
    misses read."""
    import sqlite3

    per = {}
    for kn, ctr, val, did in sqlite3.connect(tcc_db).execute(
            "select kernel_name, counter_name, value, dispatch_id from counters_collection"):
        d = per.setdefault(_short(kn), {}).setdefault(did, {})
        d[ctr] = d.get(ctr, 0.0) + val
    lines = ["", "## L2 hit rate (`--pmc TCC_HIT_sum TCC_MISS_sum` pass)", "",
             "Per dispatch, averaged: hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum).", "",
             "| kernel | dispatches | L2 requests (M) | hits (M) | misses (M) | hit rate |",
             "|---|---|---|---|---|---|"]
    for k, ds in per.items():
        if k.startswith("__amd") or k.startswith("void at::"):
            continue
        n = len(ds)
        hit = sum(d.get("TCC_HIT_sum", 0.0) for d in ds.values()) / n
        miss = sum(d.get("TCC_MISS_sum", 0.0) for d in ds.values()) / n
        tot = hit + miss
        if tot <= 0:
            continue
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.4f |" % (
            k, n, tot / 1e6, hit / 1e6, miss / 1e6, hit / tot))
    return lines


def summarize_launch_gaps(trace_db) -> list:
    """Markdown lines splitting each backward call of a kernel trace into
    kernel time and the gaps between its kernels. A call is a maximal run of
    consecutive backward kernels (an optional prep kernel, the dQ and the
    dK/dV kernel, launched back to back on one stream); span = end of its
    last kernel - start of its first; gaps = span - the sum of its kernel
    durations. Forward calls are single kernels (no gap inside a call).
    Calls are grouped by their dK/dV and dQ kernels' template arguments."""
    import sqlite3

    rows = sqlite3.connect(trace_db).execute(
        "select name, start, end from kernels order by start").fetchall()
    runs, cur = [], []
    for name, start, end in rows:
        short = _short(name)
        if short.startswith("bwd_"):
            cur.append((short, start, end))
        elif cur:
            runs.append(cur)
            cur = []
    if cur:
        runs.append(cur)
    seqs = {}
    for run in runs:
        kinds = {k: (e - s_) for k, s_, e in run}
        dk = [k for k in kinds if k.startswith("bwd_dkdv")]
        dq = [k for k in kinds if k.startswith("bwd_dq")]
        if len(dk) != 1 or len(dq) != 1 or len(run) > 3:
            continue
        prep = sum(v for k, v in kinds.items() if k.startswith("bwd_prep"))
        durs = (prep, kinds[dk[0]], kinds[dq[0]])
        span = run[-1][2] - run[0][1]
        seqs.setdefault(dk[0] + " + " + dq[0], []).append((span, sum(durs), durs, len(run)))
    lines = ["", "## Backward calls: kernel time and launch gaps (kernel trace)", "",
             "Per call (its kernels in order on one stream): span = end of the last kernel - "
             "start of the first; gaps = span - sum of the kernel durations. Averages over "
             "the traced calls.", "",
             "| dK/dV + dQ kernels | calls | kernels per call | prep us | dK/dV us | dQ us | "
             "kernels us | span us | gaps us |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, v in seqs.items():
        n = len(v)
        avg = lambda f: sum(f(x) for x in v) / n / 1e3  # noqa: E731
        lines.append("| `%s` | %d | %d | %.1f | %.1f | %.1f | %.1f | %.1f | %.1f |" % (
            k, n, v[0][3], avg(lambda x: x[2][0]), avg(lambda x: x[2][1]),
            avg(lambda x: x[2][2]), avg(lambda x: x[1]), avg(lambda x: x[0]),
            avg(lambda x: x[0] - x[1])))
    return lines


def summarize_trace(trace_db, command, out_md) -> None:
    """A kernel-trace-only summary: per-kernel durations and the launch-gap
    split of the backward calls."""
    import sqlite3

    rows = sqlite3.connect(trace_db).execute(
        "select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows)
    lines = ["# rocprofv3 summary: %s" % os.path.basename(out_md).rsplit(".", 1)[0], "",
             "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "## Kernel trace (`--kernel-trace --stats`)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, tot in rows:
        lines.append("| `%s` | %d | %.1f | %.1f | %.1f | %.1f |" % (_short(name), calls, avg / 1e3,
                                                                   mn / 1e3, mx / 1e3, 100 * tot / total))
    lines += summarize_launch_gaps(trace_db)
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_rocprof(trace_db, fetch_db, write_db, copy_mib, command, out_md, out_json, sq_db=None,
                      tcc_db=None):
    """Summarise rocprofv3 databases (kernel trace + FETCH_SIZE + WRITE_SIZE
    passes, optionally an SQ counter pass) into a short markdown file and the
    traffic JSON this bench reads."""
    import sqlite3

    rows = sqlite3.connect(trace_db).execute(
        "select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows)
    lines = ["# rocprofv3 summary: %s" % os.path.basename(out_md).rsplit(".", 1)[0], "",
             "Commands (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "## Kernel trace (`--kernel-trace --stats`)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, tot in rows:
        lines.append("| `%s` | %d | %.1f | %.1f | %.1f | %.1f |" % (_short(name), calls, avg / 1e3,
                                                                   mn / 1e3, mx / 1e3, 100 * tot / total))
    per = {}
    for db, ctr in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        for kn, val in sqlite3.connect(db).execute(
                "select kernel_name, value from counters_collection where counter_name = ?", (ctr,)):
            per.setdefault(_short(kn), {}).setdefault(ctr, []).append(val)
    copy = per.get("__amd_rocclr_copyBuffer", {})
    copy_kib = copy_mib * 1024.0

    def big(vals):
        # The calibration copies only: other copies (small host uploads) read
        # and write far fewer bytes.
        top = max(vals)
        vals = [x for x in vals if x >= 0.9 * top]
        return sum(vals) / len(vals)
    f_fac = copy_kib / big(copy["FETCH_SIZE"])
    w_fac = copy_kib / big(copy["WRITE_SIZE"])
    lines += ["", "## HBM bytes per dispatch (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`)", "",
              "Calibration: a %d MiB device-to-device copy reads FETCH_SIZE %.0f KiB and WRITE_SIZE "
              "%.0f KiB per dispatch, so FETCH_SIZE is scaled by %.3f and WRITE_SIZE by %.3f." % (
                  copy_mib, copy_kib / f_fac, copy_kib / w_fac, f_fac, w_fac), "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | write GB (scaled) |",
              "|---|---|---|---|---|---|"]
    traffic = {}
    for k, v in per.items():
        if "FETCH_SIZE" not in v or "WRITE_SIZE" not in v or k.startswith("__amd") or k.startswith("void at::"):
            continue
        fk = sum(v["FETCH_SIZE"]) / len(v["FETCH_SIZE"])
        wk = sum(v["WRITE_SIZE"]) / len(v["WRITE_SIZE"])
        rd, wr = fk * 1024 * f_fac, wk * 1024 * w_fac
        traffic[k] = {"read_bytes": rd, "write_bytes": wr}
        lines.append("| `%s` | %d | %.0f | %.0f | %.3f | %.3f |" % (k, len(v["FETCH_SIZE"]), fk, wk,
                                                                   rd / 1e9, wr / 1e9))
    if sq_db:
        lines += summarize_sq(sq_db)
    if tcc_db:
        lines += summarize_tcc(tcc_db)
    open(out_md, "w").write("\n".join(lines) + "\n")
    bwd = [k for k in traffic if k.startswith(dkdv_kernel_name(128, 16384))]
    if bwd and out_json:
        t = traffic[bwd[0]]
        json.dump({"kernel": bwd[0], "kernel_source_hash": kernel_source_hash(),
                   "hbm_bytes_per_launch": round(t["read_bytes"] + t["write_bytes"]),
                   "read_bytes": round(t["read_bytes"]), "write_bytes": round(t["write_bytes"]),
                   "calibration": {"copy_mib": copy_mib, "fetch_factor": f_fac, "write_factor": w_fac},
                   "summary": os.path.basename(out_md)}, open(out_json, "w"), indent=1)


def comp_bytes(w) -> tuple[float, float]:
    """Compulsory HBM bytes of the forward and the backward of a workload:
    forward reads Q, K, V and writes O and LSE; backward reads Q, K, V, O,
    dO and LSE, writes and reads back the D vector, writes dQ, dK, dV. K, V,
    dK and dV have the K/V heads' size."""
    e = 2 if w.dtype == "bf16" else 4
    bhn = w.batch * w.heads * w.n
    bkn = w.batch * w.kv_heads * w.n
    fwd = (2.0 * bhn + 2.0 * bkn) * w.d * e + 4 * bhn
    bwd = (4.0 * bhn + 4.0 * bkn) * w.d * e + 4 * bhn + 8 * bhn
    return fwd, bwd


def _gpu_clocks() -> str:
    import subprocess
    # Under a profiler that preloads its library into every process, the
    # rocm-smi child (a script started through env) would initialise the GPU
    # and then exec its interpreter; clocks are not needed there.
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(
            k.startswith("ROCPROF") for k in os.environ):
        return "not queried under the profiler"
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError) as exc:
        return "rocm-smi unavailable (%s)" % exc
    keep = [l.strip() for l in r.stdout.splitlines() if "sclk" in l or "mclk" in l]
    return "; ".join(keep) if keep else "rocm-smi printed no clock lines"


def visible_pairs(w) -> float:
    """(query, key) pairs a masked workload computes, per (batch, head): the
    exact count under its causal, window and block masks (FLOP accounting)."""
    import numpy as np

    from exact_io_aware_fa_amd.inputs import block_mask

    n = w.n
    i = np.arange(n)
    lo = np.zeros(n, dtype=np.int64) if w.window[0] < 0 else np.maximum(i - w.window[0], 0)
    hi = np.full(n, n, dtype=np.int64)
    if w.causal:
        hi = np.minimum(hi, i + 1)
    if w.window[1] >= 0:
        hi = np.minimum(hi, i + w.window[1] + 1)
    bm = block_mask(w)
    if bm is None:
        return float(np.maximum(hi - lo, 0).sum())
    total = 0
    for kb in range(bm.shape[1]):
        a, e = kb * 128, min(kb * 128 + 128, n)
        rows = bm[i // 128, kb]
        total += int(np.maximum(np.minimum(hi, e) - np.maximum(lo, a), 0)[rows].sum())
    return float(total)


def masked_flops(w):
    """(fwd, bwd) FLOPs of a workload: 4 d per visible pair forward, 2.5x
    that backward; the unmasked conventions for the others."""
    if w.window == (-1, -1) and w.blocks is None:
        return w.flops_fwd(), w.flops_bwd()
    f = 4.0 * w.batch * w.heads * w.d * visible_pairs(w)
    return f, 2.5 * f


def _sweep_calls(name, dev, stream):
    """(fwd, bwd, tensors, flops_fwd, flops_bwd, bytes_fwd, bytes_bwd) of one
    sweep workload: a padded batch (with grouped heads when k has fewer) or a
    packed variable-length batch."""
    import torch

    from exact_io_aware_fa_amd import binding as B
    from exact_io_aware_fa_amd.inputs import PACKED, WORKLOADS, make_inputs, make_packed_inputs

    if name in PACKED:
        w = PACKED[name]
        inp = make_packed_inputs(w)
        q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
        cu = inp["cu_seqlens"].to(dev)
        hh, total, d = q.shape
        hkv = k.shape[0]
        nseq, mx = cu.numel() - 1, max(w.seqlens())
        dt = B.FA_BF16 if q.dtype == torch.bfloat16 else B.FA_FP32
        o = torch.empty_like(q)
        lse = torch.empty((hh, total), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        wsb = B.fa_bwd_workspace_bytes(nseq, hh, mx, d, dt)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        sc = w.softmax_scale

        def fwd():
            B.check(B.fa_fwd_varlen(nseq, hh, hkv, total, mx, d, cu.data_ptr(), w.causal, sc, dt,
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), None,
                                    o.data_ptr(), lse.data_ptr(), stream))

        def bwd():
            B.check(B.fa_bwd_varlen(nseq, hh, hkv, total, mx, d, cu.data_ptr(), w.causal, sc, dt,
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    do.data_ptr(), lse.data_ptr(), None, dq.data_ptr(),
                                    dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), wsb, stream))
        e = 2 if w.dtype == "bf16" else 4
        bf = (2.0 * hh + 2.0 * hkv) * total * d * e + 4 * hh * total
        bb = (4.0 * hh + 4.0 * hkv) * total * d * e + 12 * hh * total
        tensors = (q, k, v, o, do, dq, dk, dv, lse, ws, cu)
        return fwd, bwd, tensors, w.flops_fwd(), w.flops_bwd(), bf, bb

    from exact_io_aware_fa_amd.inputs import block_mask

    w = WORKLOADS[name]
    inp = make_inputs(w)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    kvl = None if inp["kv_len"] is None else inp["kv_len"].to(dev)
    kv_ptr = None if kvl is None else kvl.data_ptr()
    bsz, hh, n, d = q.shape
    hkv = k.shape[1]
    bm = block_mask(w)
    idx = None
    if bm is not None:
        idx = torch.empty(B.fa_block_index_bytes(n) // 4, dtype=torch.int32, device=dev)
        bmd = torch.from_numpy(bm).to(device=dev, dtype=torch.uint8)
        B.check(B.fa_block_index_build(n, bmd.data_ptr(), idx.data_ptr(), stream))
    mask = B.mask_arg(w.window, None if idx is None else idx.data_ptr())
    dt = B.FA_BF16 if q.dtype == torch.bfloat16 else B.FA_FP32
    scale = w.softmax_scale
    o = torch.empty_like(q)
    lse = torch.empty((bsz, hh, n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = B.fa_bwd_workspace_bytes(bsz, hh, n, d, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def fwd():
        B.check(B.fa_fwd_masked(bsz, hh, hkv, n, d, w.causal, scale, dt, q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), kv_ptr, mask, o.data_ptr(),
                                lse.data_ptr(), stream))

    def bwd():
        B.check(B.fa_bwd_masked(bsz, hh, hkv, n, d, w.causal, scale, dt, q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), kv_ptr, mask, dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), ws.data_ptr(), wsb, stream))
    bf, bb = comp_bytes(w)
    tensors = (q, k, v, o, do, dq, dk, dv, lse, ws) + (() if idx is None else (idx,))
    ff, fb = masked_flops(w)
    return fwd, bwd, tensors, ff, fb, bf, bb


def run_sweep(out_path: str | None, only=None) -> int:
    import statistics

    import torch

    from exact_io_aware_fa_amd import binding as B
    from exact_io_aware_fa_amd.inputs import PACKED, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py --sweep needs a GPU", file=sys.stderr)
        return 1
    B.lib()
    dev = torch.device("cuda:0")
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    names = [n for n, w in WORKLOADS.items()
             if w.backward and n.startswith(("bert", "gpt2", "gqa", "window", "blocksparse",
                                              "sweep"))] + list(PACKED)
    if only:
        names = [n for n in names if any(n.startswith(o) for o in only)]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ev = [hip.create() for _ in range(2)]
    clocks_before = _gpu_clocks()
    rows = []
    sclk = SclkSampler(period_s=0.02)
    sclk.__enter__()
    for name in names:
        fwd, bwd, tensors, ff, fb, bf, bb = _sweep_calls(name, dev, stream)

        def timed(fn, cold):
            if cold:
                flush.fill_(1)
            hip.record(ev[0], stream)
            fn()
            hip.record(ev[1], stream)
            return hip.elapsed_ms(ev[0], ev[1])

        for _ in range(10):
            fwd()
            bwd()
        torch.cuda.synchronize()
        tf, tb, spent = [], [], 0.0
        while len(tf) < 50 or spent < 200.0:
            tf.append(timed(fwd, False))
            tb.append(timed(bwd, False))
            spent += tf[-1] + tb[-1]
        working = sum(t.numel() * t.element_size() for t in tensors)
        cf = cb = None
        if working <= 256 << 20:
            cf = statistics.median(timed(fwd, True) for _ in range(20))
            cb = statistics.median(timed(bwd, True) for _ in range(20))
        mf, mb = statistics.median(tf), statistics.median(tb)
        roof_f = min(PEAK_BF16_TFLOPS, ff / bf * PEAK_HBM_GBS / 1e3)
        roof_b = min(PEAK_BF16_TFLOPS, fb / bb * PEAK_HBM_GBS / 1e3)
        tff, tfb = ff / mf / 1e9, fb / mb / 1e9
        rows.append((name, mf, min(tf), tff, tff / PEAK_BF16_TFLOPS, tff / roof_f, bf / mf / 1e6,
                     mb, min(tb), tfb, tfb / PEAK_BF16_TFLOPS, tfb / roof_b, bb / mb / 1e6,
                     3.5 * ff / (mf + mb) / 1e9, cf, cb))
        print(json.dumps({"workload": name, "fwd_ms_median": round(mf, 4), "bwd_ms_median": round(mb, 4),
                          "fwd_tflops": round(tff, 1), "bwd_tflops": round(tfb, 1)}), flush=True)
        del fwd, bwd, tensors
        torch.cuda.empty_cache()
    sclk.__exit__(None, None, None)
    for e_ in ev:
        hip.destroy(e_)
    sr = sclk.result()
    sclk_line = ("Shader clock sampled during the sweep (%s): median %.0f MHz, min %.0f, max %.0f "
                 "(%d samples)" % (sr["source"], sr["median_mhz"], sr["min_mhz"], sr["max_mhz"],
                                   sr["samples"]) if sr.get("samples") else
                 "Shader clock: not sampled (%s)" % sr["source"])
    if sr.get("power_median_w") is not None:
        sclk_line += "; board power (%s) median %.0f W, max %.0f W, cap %s W" % (
            sr["power_source"], sr["power_median_w"], sr["power_max_w"],
            "?" if sr["power_cap_w"] is None else "%.0f" % sr["power_cap_w"])
    lines = ["# Attention sweep on one MI355X", "",
             "Command: `python bench.py --sweep --out <this file>` (from the repository root).", "",
             "Clocks before the sweep (rocm-smi): " + clocks_before,
             "Clocks after the sweep (rocm-smi): " + _gpu_clocks(), sclk_line, "",
             "Times are medians (min in parentheses) over >= 50 calls and >= 200 ms, warm "
             "cache; `cold` medians write a 512 MB buffer before each call. Peak = bf16 dense "
             "MFMA %.0f TFLOP/s; roof = min(peak, compulsory-byte AI x %.0f GB/s); GB/s = "
             "compulsory bytes / time. FLOPs: 4BHN^2d forward (x2.5 backward), halved when "
             "causal; the padded workload counts nominal FLOPs; packed (varlen) workloads "
             "count 4Hd sum_s L_s^2; window and block-sparse workloads count 4d per visible "
             "(query, key) pair." % (PEAK_BF16_TFLOPS, PEAK_HBM_GBS), "",
             "| workload | fwd ms | fwd TFLOP/s | fwd % peak | fwd % roof | fwd GB/s | bwd ms | "
             "bwd TFLOP/s | bwd % peak | bwd % roof | bwd GB/s | fwd+bwd TFLOP/s | cold fwd / bwd ms |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        cold = "-" if r[14] is None else "%.4f / %.4f" % (r[14], r[15])
        lines.append("| %s | %.4f (%.4f) | %.1f | %.1f | %.1f | %.0f | %.4f (%.4f) | %.1f | %.1f | %.1f | %.0f | %.1f | %s |"
                     % (r[0], r[1], r[2], r[3], 100 * r[4], 100 * r[5], r[6], r[7], r[8], r[9],
                        100 * r[10], 100 * r[11], r[12], r[13], cold))
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    print(text)
    return 0


PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 matrix-core peak (published)


def calibrate_copy(mib: int, dev) -> None:
    """Copy `mib` MiB device-to-device three times: a plain copy kernel of
    known size, against which rocprofv3's HBM byte counters are scaled."""
    if not mib:
        return
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_fp8(out_path: str | None, only=None, copy_mib: int = 0) -> int:
    """FP8 forward timings: the three block encodings (Q, K with the Hadamard
    rotation; V transposed) and the E4M3 attention kernel, next to the bf16
    forward on the same inputs."""
    import statistics

    import torch

    from exact_io_aware_fa_amd import attention as fa
    from exact_io_aware_fa_amd import binding as B
    from exact_io_aware_fa_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py --fp8 needs a GPU", file=sys.stderr)
        return 1
    B.lib()
    dev = torch.device("cuda:0")
    calibrate_copy(copy_mib, dev)
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    names = [n for n, w in WORKLOADS.items()
             if w.window == (-1, -1) and w.blocks is None
             and w.dtype == "bf16"]
    if only:
        names = [n for n in names if any(n.startswith(o) for o in only)]
    ev = [hip.create() for _ in range(4)]
    clocks_before = _gpu_clocks()
    rows = []
    cpu = None  # (workload, CPU oracle timing) for the long causal workload
    for name in names:
        w = WORKLOADS[name]
        inp = make_inputs(w, with_grad_out=False)
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
        kvl = None if inp["kv_len"] is None else inp["kv_len"].to(dev)
        bsz, hh, n, d = q.shape
        hkv = k.shape[1]
        signs = fa.hadamard_signs(d, torch.Generator().manual_seed(w.seed), dev)
        q8, qs = fa.fp8_quantize(q, signs)
        k8, ks = fa.fp8_quantize(k, signs)
        v8, vs = fa.fp8_quantize(v, layout="vt")
        o = torch.empty_like(q)
        lse = torch.empty((bsz, hh, n), dtype=torch.float32, device=dev)
        kp = None if kvl is None else kvl.data_ptr()
        sc = w.softmax_scale

        def quant():
            for x, c, s_, sg, lay in ((q, q8, qs, signs, B.FA_FP8_ROWS),
                                      (k, k8, ks, signs, B.FA_FP8_ROWS),
                                      (v, v8, vs, None, B.FA_FP8_VT)):
                B.check(B.fa_fp8_quantize(bsz, x.shape[1], n, d, lay, x.data_ptr(),
                                          None if sg is None else sg.data_ptr(), c.data_ptr(),
                                          s_.data_ptr(), stream))

        def attn():
            B.check(B.fa_fwd_fp8(bsz, hh, hkv, n, d, w.causal, sc, q8.data_ptr(), qs.data_ptr(),
                                 k8.data_ptr(), ks.data_ptr(), v8.data_ptr(), vs.data_ptr(), kp,
                                 o.data_ptr(), lse.data_ptr(), stream))

        def bf16():
            B.check(B.fa_fwd_gqa(bsz, hh, hkv, n, d, w.causal, sc, B.FA_BF16, q.data_ptr(),
                                 k.data_ptr(), v.data_ptr(), kp, o.data_ptr(), lse.data_ptr(),
                                 stream))

        def timed(fn):
            hip.record(ev[0], stream)
            fn()
            hip.record(ev[1], stream)
            return hip.elapsed_ms(ev[0], ev[1])

        for _ in range(10):
            quant()
            attn()
            bf16()
        torch.cuda.synchronize()
        tq, ta, tb, spent = [], [], [], 0.0
        while len(ta) < 50 or spent < 200.0:
            tq.append(timed(quant))
            ta.append(timed(attn))
            tb.append(timed(bf16))
            spent += tq[-1] + ta[-1] + tb[-1]
        mq, ma, mb = statistics.median(tq), statistics.median(ta), statistics.median(tb)
        ff = w.flops_fwd()
        if cpu is None and name.startswith("long_causal"):
            cpu = (name, cpu_baseline_fp8(w, inp, signs))
        rows.append((name, mq, ma, min(ta), ff / ma / 1e9, ff / (ma + mq) / 1e9, mb,
                     ff / mb / 1e9))
        print(json.dumps({"workload": name, "fp8_quantize_ms": round(mq, 4),
                          "fp8_attn_ms": round(ma, 4), "bf16_fwd_ms": round(mb, 4),
                          "fp8_attn_tflops": round(ff / ma / 1e9, 1)}), flush=True)
        del q, k, v, q8, k8, v8, o, lse
        torch.cuda.empty_cache()
    for e_ in ev:
        hip.destroy(e_)
    lines = ["# FP8 (E4M3) forward on one MI355X", "",
             "Command: `python bench.py --fp8 --out <this file>` (from the repository root).", "",
             "Clocks before (rocm-smi): " + clocks_before,
             "Clocks after (rocm-smi): " + _gpu_clocks(), "",
             "Medians (min in parentheses) over >= 50 calls and >= 200 ms, warm cache. "
             "`encode` = the three block encodings (Q and K rotated by the Hadamard matrix, "
             "V transposed); `attention` = fa_fwd_fp8 on the codes; `bf16` = fa_fwd on the "
             "same bf16 inputs. FLOPs 4BHN^2d, halved when causal (nominal for padded "
             "batches); fp8 peak %.0f TFLOP/s, bf16 peak %.0f." % (PEAK_FP8_TFLOPS,
                                                                   PEAK_BF16_TFLOPS), "",
             "| workload | encode ms | attention ms | attention TFLOP/s | % fp8 peak | "
             "encode+attention TFLOP/s | bf16 fwd ms | bf16 fwd TFLOP/s | speed-up vs bf16 |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %.4f | %.4f (%.4f) | %.1f | %.1f | %.1f | %.4f | %.1f | %.2fx |"
                     % (r[0], r[1], r[2], r[3], r[4], 100 * r[4] / PEAK_FP8_TFLOPS, r[5], r[6],
                        r[7], r[6] / r[2]))
    if cpu is not None:
        lines += ["", "CPU oracle beside it (%s): %.4f TFLOP/s on %d threads; %s." % (
            cpu[0], cpu[1]["value"], cpu[1]["cores"], cpu[1]["sample"])]
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    print(text)
    return 0


def main() -> int:
    if len(sys.argv) > 1 and sys.argv[1] == "summarize-trace":
        sp = argparse.ArgumentParser(prog="bench.py summarize-trace")
        sp.add_argument("trace_db")
        sp.add_argument("--command", required=True)
        sp.add_argument("--out-md", required=True)
        a = sp.parse_args(sys.argv[2:])
        summarize_trace(a.trace_db, a.command, a.out_md)
        return 0
    if len(sys.argv) > 1 and sys.argv[1] == "summarize":
        sp = argparse.ArgumentParser(prog="bench.py summarize")
        sp.add_argument("trace_db")
        sp.add_argument("fetch_db")
        sp.add_argument("write_db")
        sp.add_argument("--copy-mib", type=int, default=1024)
        sp.add_argument("--command", required=True)
        sp.add_argument("--out-md", required=True)
        sp.add_argument("--out-json", default=None)
        sp.add_argument("--sq-db", default=None, help="database of an SQ counter pass")
        sp.add_argument("--tcc-db", default=None, help="database of an L2 hit/miss pass")
        a = sp.parse_args(sys.argv[2:])
        summarize_rocprof(a.trace_db, a.fetch_db, a.write_db, a.copy_mib, a.command, a.out_md, a.out_json,
                          a.sq_db, a.tcc_db)
        return 0
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--sweep", action="store_true",
                    help="time fwd and bwd on every sweep workload and print a table")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward (encode + E4M3 attention) against the bf16 "
                         "forward on the d=64 and d=128 workloads and print a table")
    ap.add_argument("--out", default=None, help="with --sweep / --fp8: also write the table here")
    ap.add_argument("--only", nargs="*", default=None, metavar="PREFIX",
                    help="with --sweep: only the workloads whose names start so")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device three times (a plain copy "
                         "kernel of known size, to scale HBM byte counters)")
    args = ap.parse_args()

    if args.sweep:
        return run_sweep(args.out, args.only)
    if args.fp8:
        return run_fp8(args.out, args.only, args.calibrate_copy)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the work would shard by (batch, head) with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from exact_io_aware_fa_amd import binding as B
    from exact_io_aware_fa_amd.inputs import HEADLINE, WORKLOADS, make_inputs

    w = WORKLOADS[args.workload or HEADLINE]
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    B.lib()  # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    calibrate_copy(args.calibrate_copy, dev)
    inp = make_inputs(w)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    kvl = None if inp["kv_len"] is None else inp["kv_len"].to(dev)
    bsz, hh, n, d = q.shape
    hkv = k.shape[1]
    dt = B.FA_BF16 if q.dtype == torch.bfloat16 else B.FA_FP32
    o = torch.empty_like(q)
    lse = torch.empty((bsz, hh, n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = B.fa_bwd_workspace_bytes(bsz, hh, n, d, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    kv_ptr = None if kvl is None else kvl.data_ptr()
    scale = w.softmax_scale

    hip = HipEvents()
    nev = args.steps
    ev_f0 = [hip.create() for _ in range(nev)]
    ev_f1 = [hip.create() for _ in range(nev)]
    ev_b = [[hip.create() for _ in range(4)] for _ in range(nev)]

    def step(i=None):
        if i is not None:
            hip.record(ev_f0[i], stream)
        B.check(B.fa_fwd_gqa(bsz, hh, hkv, n, d, w.causal, scale, dt, q.data_ptr(),
                             k.data_ptr(), v.data_ptr(), kv_ptr, o.data_ptr(),
                             lse.data_ptr(), stream))
        if i is not None:
            hip.record(ev_f1[i], stream)
        B.check(B.fa_bwd_timed(bsz, hh, hkv, n, d, w.causal, scale, dt, q.data_ptr(),
                               k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), kv_ptr, dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), ws.data_ptr(), ws_bytes, stream,
                               None if i is None else ev_b[i]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    with SclkSampler() as sclk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    fwd_ms = [hip.elapsed_ms(ev_f0[i], ev_f1[i]) for i in range(nev)]
    # bf16: dQ kernel (with D_i, L_i log2 e) between events 0 and 1, the
    # dK/dV kernel between events 1 and 2.
    dq_ms = [hip.elapsed_ms(ev_b[i][0], ev_b[i][1]) for i in range(nev)]
    main_ms = [hip.elapsed_ms(ev_b[i][1], ev_b[i][2]) for i in range(nev)]
    bwd_ms = [hip.elapsed_ms(ev_b[i][0], ev_b[i][3]) for i in range(nev)]
    for e in ev_f0 + ev_f1 + [x for r in ev_b for x in r]:
        hip.destroy(e)

    ff, fb = w.flops_fwd(), w.flops_bwd()
    ms_step = wall / args.steps * 1e3
    value = (ff + fb) / (ms_step / 1e3) / 1e12
    avg = lambda xs: sum(xs) / len(xs)  # noqa: E731
    fwd_tf = ff / (avg(fwd_ms) / 1e3) / 1e12
    bwd_tf = fb / (avg(bwd_ms) / 1e3) / 1e12
    f_dkdv = fb * 4 / 5  # S, dP, dV, dK of the backward's five products
    main_tf = f_dkdv / (avg(main_ms) / 1e3) / 1e12
    src_hash = kernel_source_hash()

    out = {
        "metric": "attention TFLOP/s fwd+bwd (bf16) and % of MI355X MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == B.FA_BF16 else "fp32",
        "data": "synthetic (seeded normal inputs; Q,K std %g, V,dO std 1)" % w.qk_sigma,
        "config": {"workload": w.name, "batch": bsz, "heads": hh, "heads_kv": hkv, "seq_len": n,
                   "head_dim": d, "causal": w.causal, "key_padding": w.padded,
                   "softmax_scale": scale},
        "frac_of_peak_fwd_bwd": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(avg(fwd_ms), 4), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(avg(bwd_ms), 4), "tflops": round(bwd_tf, 2),
                "frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "dkdv_kernel_ms": round(avg(main_ms), 4),
                "dq_kernel_ms": round(avg(dq_ms), 4)},
        "sclk": sclk.result(),
        "roofline": {
            "kernel": "%s (recompute backward, dK and dV, d=%d)" % (dkdv_kernel_name(d, n), d),
            "bound": "mfma",
            "achieved": round(main_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(main_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(src_hash, w.name),
            "kernel_source_hash": src_hash,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
