#!/usr/bin/env python3
"""Throughput of the FP4 compress + decompress hot path on one MI355X.

A step compresses one 32768 x 4096 bf16 tensor (N(0,1), seed 3) and
decompresses one payload of the same shape to fp32, the two halves of what a
tensor-parallel rank does around an AllReduce.  Three buffer sets rotate, and
step i decompresses the payload compressed in step i-1, so no read is served
from the 256 MB last-level cache.  Inputs are resident in HBM before the timed
region.  Prints one JSON line on stdout; progress goes to stderr.

Order of a run: a quarter second of untimed steps, then the other GPU legs
(entry-point variants, cold launches, the receiver kernels, the transform
trade-off, the traffic twins, the copy ceiling, the error report), which also
bring the GPU to a steady state; then W warm-up steps; then
K timed steps by wall clock between two synchronisations, with nothing else
queued in between; then a separate per-kernel pass of KERNEL_PASS steps with
HIP events around each kernel; then the CPU baseline.

value    = bf16 input bytes (2 N per step) / wall time of the K timed steps.
roofline = the dominant kernel's algorithmic bytes per launch / its median
           duration in the per-kernel pass, against 8 TB/s.
cpu_baseline = the CPU oracle on the host's usable cores (the OMP_NUM_THREADS
           share where one is set), compress and decompress timed separately
           on every workload and the k = 8 reduce, median of 3 runs, with a
           single-threaded leg beside it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compress+decompress GB/s of bf16 input and % HBM roofline, 32768x4096"
PEAK_GBPS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "fp4_communication_compression_amd", "csrc", f)
                  for f in ("fp4q.hip", "fp4q_numerics.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_large32768.md")
RECEIVER_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_reduce_k8.md")
COPY_REF_BYTES = 256 << 20
KERNEL_PASS = 60   # steps of the per-kernel pass (HIP events around each kernel)
HEADLINE = "large32768"
#: the step's workloads: what each tensor is (shapes and seeds in inputs.CONFIGS)
WORKLOADS = {
    "large32768": "bf16 32768x4096 N(0,1) seed 3",
    "act2048": "bf16 2048x4096 N(0,1) x exp(N(0,0.5)) per row, seed 1",
    "outlier8192": "bf16 8192x4096 Student-t(3), 4 fixed columns x100, seed 2",
}
ROTATION_BYTES = 512 << 20   # rotating buffer sets span at least twice the last-level cache


class TimingEvent:
    """A HIP event for timing only, recorded on torch's current stream (the stream
    the library launches on).  It is created with hipEventDisableSystemFence: the
    HIP runtime documents that flag for events used only to measure time, since
    recording it then performs no system-scope cache write-back.  torch's events
    do, and read about 2 us more per kernel here.  The same interface as
    torch.cuda.Event: record(), elapsed_time(end) in ms after a synchronisation."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.e = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self):
        import torch
        rc = self._lib().hipEventRecord(self.e, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        rc = self._lib().hipEventElapsedTime(self._ct.byref(ms), self.e, end.e)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        if self._hip is not None and self.e:
            self._hip.hipEventDestroy(self.e)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n: int):
    nb = n // 256
    payload = n // 2 + n // 16 + 4 * nb
    return {"compress": 2 * n + payload, "decompress": payload + 4 * n}


def kernel_source_hash() -> str:
    """Hash of the kernel source with comments and white space removed, so that
    counter summaries stay attached to the code they measured, not its prose."""
    text = "\n".join(open(f).read() for f in KERNEL_SOURCES)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def measured_traffic(path: str = None):
    """HBM bytes per launch, per kernel, from a committed counter summary, if it
    was taken on the current kernel source (else None)."""
    path = path or TRAFFIC_SUMMARY
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic: source=(\w+)((?: \w+=\d+)*)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    return {k: int(v) for k, v in re.findall(r"(\w+)=(\d+)", m.group(2))}


def _short(kernel_name: str) -> str:
    if "twin_" in kernel_name:                       # the traffic twins of the ceilings leg
        return "twin"
    if "requantize_kernel<" in kernel_name:          # with the rank's own slice
        return "requantize_local"
    for fam in ("decompress_mx", "compress_mx", "decompress", "compress", "accumulate_narrow", "accumulate",
                "requantize_narrow"):
        if fam + "_kernel" in kernel_name:
            return fam.replace("_narrow", "")
    if "copyBuffer" in kernel_name:
        return "copy"
    return kernel_name.split("(")[0][:40]


REDUCE_N = 4096 * 11008          # elements per peer of the k = 8 reduce workload
REDUCE_K = 8


def _receiver_bytes():
    n = REDUCE_N
    pay = n // 2 + n // 16 + n // 64
    return {"accumulate": REDUCE_K * pay + 4 * n, "requantize": (REDUCE_K + 1) * pay,
            "requantize_local": REDUCE_K * pay + 2 * n}   # 7 payloads + local bf16 in, 1 out


def _largest_grid(rows, grid_key):
    """Per kernel family, the dispatches of its largest grid (the workload the
    bench times; smaller launches of the same kernel are set-up or other shapes)."""
    by = {}
    for r in rows:
        by.setdefault(_short(r["Kernel_Name"]), []).append(r)
    out = {}
    for fam, rs in by.items():
        g = max(int(r[grid_key]) for r in rs)
        out[fam] = [r for r in rs if int(r[grid_key]) == g]
    return out


def summarize_counters(fetch_dir: str, write_dir: str) -> str:
    """Counter summary (markdown) from two rocprofv3 --pmc runs of this bench with
    --copy-reference: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), scaled by what
    the same counters read for a plain device copy of COPY_REF_BYTES."""
    grids = {}

    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        fams = _largest_grid(rows, "Grid_Size")
        grids.update({k: int(v[0]["Grid_Size"]) for k, v in fams.items()})
        vals = {k: [float(r["Counter_Value"]) for r in v] for k, v in fams.items()}
        # the reference: the COPY_REF_BYTES copies, the largest a --copy-reference run
        # makes (it leaves out the copy ceiling's larger ones).  The runtime's copy
        # kernel is grid-strided, so smaller copies (tensor clones) share their grid
        # and are told apart by their counts; the reference issues three.
        copies = sorted(vals.get("copy", []))
        if copies:
            vals["copy"] = [c for c in copies if c >= 0.9 * copies[-1]]
        if len(vals.get("copy", [])) < 3:
            raise ValueError("%s: fewer than the three reference copies of %d bytes; run the "
                             "bench with --copy-reference" % (counter, COPY_REF_BYTES))
        return {k: float(np.median(v)) for k, v in vals.items()}
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    f_scale = COPY_REF_BYTES / (fetch["copy"] * 1024.0)
    w_scale = COPY_REF_BYTES / (write["copy"] * 1024.0)
    ab = dict(algorithmic_bytes(32768 * 4096))
    ab.update(_receiver_bytes())
    out = ["| kernel | workload | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) | algorithmic bytes | ratio |",
           "|---|---|---|---|---|---|---|"]
    traffic = {}
    for k in ("compress", "decompress", "accumulate", "requantize", "requantize_local"):
        # only launches of the workload each figure is defined for: one thread per
        # 64 elements in the wide layout, per 32 in the narrow one (accumulate and
        # the re-quantise without a local slice), up to a last partial workgroup
        head = k in ("compress", "decompress")
        per_lane = 32 if k in ("accumulate", "requantize") else 64
        want_grid = (32768 * 4096 if head else REDUCE_N) // per_lane
        if k not in fetch or k not in write or not want_grid <= grids[k] < want_grid + 1024:
            continue
        t = fetch[k] * 1024 * f_scale + write[k] * 1024 * w_scale
        traffic[k] = int(round(t))
        wl = "32768x4096" if head else "k=8 x 4096x11008"
        out.append("| %s | %s | %.0f | %.0f | %d | %d | %.3f |" % (k, wl, fetch[k], write[k], traffic[k],
                                                                 ab[k], t / ab[k]))
    out.append("| copy (%d B) | | %.0f | %.0f | scale factors: fetch x%.3f, write x%.3f | | |"
               % (COPY_REF_BYTES, fetch["copy"], write["copy"], f_scale, w_scale))
    out.append("")
    out.append("traffic: source=%s " % kernel_source_hash() +
               " ".join("%s=%d" % (k, v) for k, v in traffic.items()))
    return "\n".join(out)


# The library's kernels as named in a profiler's records (templates with their arguments).
KERNEL_NAME = re.compile(r"\b((?:de)?compress(?:_mx)?_kernel(?:<[^>]*>)?|accumulate(?:_narrow)?_kernel<[^>]*>|"
                         r"requantize_kernel<[^>]*>|requantize_narrow_kernel)")


def summarize_trace(trace_dir: str, timed_steps: int = 0) -> str:
    """Per-dispatch kernel durations from a rocprofv3 --kernel-trace run (markdown):
    each of this library's kernel instantiations at its largest grid.  With
    timed_steps K (the run's --steps), also the headline kernels' launches of the
    per-kernel pass (the last KERNEL_PASS launches at full size) and of the timed
    region (the K launches before them)."""
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))   # dispatch order
    groups = {}
    for r in rows:
        m = KERNEL_NAME.search(r["Kernel_Name"])
        if not m:
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups.setdefault(m.group(1), []).append((grid, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out = ["| kernel | grid (threads) | calls | average us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    passes = []
    for name in sorted(groups, key=lambda n: -len(groups[n])):
        g = max(x[0] for x in groups[name])
        d = np.array([x[1] for x in groups[name] if x[0] == g])
        out.append("| %s | %d | %d | %.2f | %.2f | %.2f | %.2f |" % (
            name, g, len(d), d.mean(), float(np.median(d)), d.min(), d.max()))
        if timed_steps and name in ("compress_kernel<true>", "decompress_kernel<true, false>") \
                and len(d) >= timed_steps + KERNEL_PASS:
            for label, t in (("per-kernel pass", d[-KERNEL_PASS:]),
                             ("timed region", d[-KERNEL_PASS - timed_steps:-KERNEL_PASS])):
                passes.append("| %s | %s | %d | %.2f | %.2f | %.2f | %.2f |" % (
                    name, label, len(t), t.mean(), float(np.median(t)), float(np.percentile(t, 90)),
                    t.min()))
    if passes:
        out += ["", "Headline kernels, per part of the run (%d timed steps, then the %d-step "
                "per-kernel pass):" % (timed_steps, KERNEL_PASS), "",
                "| kernel | part | calls | average us | median us | p90 us | min us |",
                "|---|---|---|---|---|---|---|"] + passes
    return "\n".join(out)


SIMDS, XCDS = 1024, 8   # MI355X: 256 compute units of 4 SIMDs, in 8 XCDs
PMC_KERNELS = ("compress_kernel<true>", "compress_kernel<false>", "decompress_kernel<true, false>",
               "decompress_kernel<true, true>", "accumulate_narrow_kernel<true, false>",
               "requantize_narrow_kernel", "requantize_kernel<true>")


def summarize_pmc(dirs) -> str:
    """Per-kernel counter summary (markdown) from rocprofv3 --pmc runs (one
    directory per pass): for each headline and receiver kernel at its largest
    grid, the median over its dispatches of every counter collected, then the
    per-wavefront instruction mix and the shares of wavefront time."""
    vals, dur, grid_of = {}, {}, {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                m = KERNEL_NAME.search(r["Kernel_Name"])
                if not m or m.group(1) not in PMC_KERNELS:
                    continue
                k, g = m.group(1), int(r["Grid_Size"])
                if g < grid_of.get(k, 0):
                    continue
                if g > grid_of.get(k, 0):
                    grid_of[k] = g
                    vals[k], dur[k] = {}, []
                vals[k].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    med = {k: {c: float(np.median(v)) for c, v in vals[k].items()} for k in vals}
    names = sorted({c for k in med for c in med[k]})
    out = ["| kernel | grid | us (under counters) | " + " | ".join(names) + " |",
           "|---|---|---|" + "---|" * len(names)]
    for k in PMC_KERNELS:
        if k in med:
            out.append("| %s | %d | %.1f | " % (k, grid_of[k], float(np.median(dur[k]))) +
                       " | ".join("%.0f" % med[k].get(c, float("nan")) for c in names) + " |")
    out += ["", "Derived, per wavefront (instructions) and as shares of the wavefronts' resident "
            "time SQ_WAVE_CYCLES (all in the same quad-cycle units); SIMD VALU busy = "
            "SQ_ACTIVE_INST_VALU x 4 cycles / %d SIMDs / (GRBM_GUI_ACTIVE / %d XCDs); clock = "
            "GRBM_GUI_ACTIVE / %d / duration:" % (SIMDS, XCDS, XCDS), "",
            "| kernel | waves | VALU | SALU | LDS | VMEM rd | VMEM wr | VALU active / wave time | "
            "any inst active / wave time | waiting / wave time | SIMD VALU busy | clock GHz |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in PMC_KERNELS:
        c = med.get(k)
        if not c or not c.get("SQ_WAVES"):
            continue
        w = c["SQ_WAVES"]
        per = lambda n: ("%.0f" % (c[n] / w)) if n in c else "-"
        frac = lambda n: ("%.3f" % (c[n] / c["SQ_WAVE_CYCLES"])) if n in c and c.get("SQ_WAVE_CYCLES") else "-"
        gui = c.get("GRBM_GUI_ACTIVE")
        busy = ("%.3f" % (c["SQ_ACTIVE_INST_VALU"] * 4 / SIMDS / (gui / XCDS))) \
            if gui and "SQ_ACTIVE_INST_VALU" in c else "-"
        clock = ("%.2f" % (gui / XCDS / (float(np.median(dur[k])) * 1e3))) if gui else "-"
        out.append("| %s | %.0f | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            k, w, per("SQ_INSTS_VALU"), per("SQ_INSTS_SALU"), per("SQ_INSTS_LDS"), per("SQ_INSTS_VMEM_RD"),
            per("SQ_INSTS_VMEM_WR"), frac("SQ_ACTIVE_INST_VALU"), frac("SQ_ACTIVE_INST_ANY"),
            frac("SQ_WAIT_INST_ANY"), busy, clock))
    return "\n".join(out)


def receiver_timing(fp4q, inputs, torch, dev, iters: int = 40):
    """The receiver's kernels on the reduce workload (k = 8 peers of 4096 x 11008,
    N(0, 1e-3)): fp4q_decompress_accumulate (fp32 out), fp4q_reduce_requantize, and
    fp4q_reduce_requantize with the rank's own slice added uncompressed (7 payloads
    + 1 bf16 tensor).  Three rotating copies of the inputs; HIP events around every
    launch; the rate is taken from the median launch."""
    k, rows, L = 8, 4096, 11008
    n = rows * L
    pay = []
    for xb in reduce_peers(inputs):
        pay.append(fp4q.fp4q_compress(torch.from_numpy(xb.view(np.int16)).to(dev)))
    sets = [pay] + [[tuple(t.clone() for t in q) for q in pay] for _ in range(2)]
    out = [torch.empty((rows, L), dtype=torch.float32, device=dev) for _ in range(3)]
    req = [fp4q.fp4q_reduce_requantize(pay) for _ in range(3)]
    # an 8-rank slice with the rank's own part uncompressed: 7 payloads + the local bf16 tensor
    loc = [torch.from_numpy(reduce_peers(inputs)[k - 1].view(np.int16)).to(dev) for _ in range(3)]
    payload = n // 2 + n // 16 + n // 64
    res = {}
    for name, fn, nbytes in (
            ("decompress_accumulate", lambda i: fp4q.fp4q_decompress_accumulate(sets[i % 3], out=out[i % 3]),
             k * payload + 4 * n),
            ("reduce_requantize", lambda i: fp4q.fp4q_reduce_requantize(sets[i % 3], *req[i % 3]),
             (k + 1) * payload),
            ("reduce_requantize_local", lambda i: fp4q.fp4q_reduce_requantize(
                sets[i % 3][:k - 1], *req[i % 3], local=loc[i % 3]), k * payload + 2 * n)):
        for i in range(6):
            fn(i)
        ev = [(TimingEvent(), TimingEvent()) for _ in range(iters)]
        torch.cuda.synchronize()
        # untimed launches queued right before the timed ones give the host a head
        # start, so no event pair spans time the GPU spent waiting for the host
        for i in range(16):
            fn(i)
        for i in range(iters):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        med = float(np.median(t))
        gbps = nbytes / med / 1e9
        res[name] = {"median_us": round(med * 1e6, 2), "avg_us": round(t.mean() * 1e6, 2),
                     "min_us": round(t.min() * 1e6, 2),
                     "p90_us": round(float(np.percentile(t, 90)) * 1e6, 2),
                     "algorithmic_bytes": nbytes, "achieved_GBps": round(gbps, 1),
                     "frac": round(gbps / PEAK_GBPS, 4),
                     "traffic": (measured_traffic(RECEIVER_TRAFFIC_SUMMARY) or {}).get(
                         name.replace("decompress_", "").replace("reduce_", ""))}
        log("receiver %-22s median %7.1f us (avg %.1f, p90 %.1f)  %7.1f GB/s  %.1f%% of HBM peak" % (
            name, med * 1e6, t.mean() * 1e6, res[name]["p90_us"], gbps, 100 * gbps / PEAK_GBPS))
    # One rank's GPU work in an 8-rank compressed AllReduce (two exchanges): compress
    # its whole partial tensor, re-quantise its 1/8 row-slice from the 7 received
    # payload slices plus its own uncompressed slice, decompress the gathered payload.
    per = rows // k
    Xs = loc
    Ps = [tuple(torch.empty_like(t) for t in pay[0]) for _ in range(3)]
    Rs = [tuple(t[:per].clone() for t in pay[0]) for _ in range(3)]
    Ys = out

    def rank_step(i):
        s = i % 3
        fp4q.fp4q_compress(Xs[s], *Ps[s])
        fp4q.fp4q_reduce_requantize([tuple(t[:per] for t in q) for q in sets[s][:k - 1]], *Rs[s],
                                    local=Xs[s][:per])
        fp4q.fp4q_decompress(*sets[s][k - 1], out=Ys[s])
    for i in range(6):
        rank_step(i)
    torch.cuda.synchronize()
    for i in range(8):
        rank_step(i)
    ev = [(TimingEvent(), TimingEvent()) for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        rank_step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    nbytes = (2 * n + payload) + ((k - 1) * payload // k + 2 * n // k + payload // k) + (payload + 4 * n)
    med = float(np.median(t))
    res["allreduce_rank"] = {"median_us": round(med * 1e6, 2), "algorithmic_bytes": nbytes,
                             "achieved_GBps": round(nbytes / med / 1e9, 1),
                             "frac": round(nbytes / med / 1e9 / PEAK_GBPS, 4),
                             "what": "compress 4096x11008 + re-quantise a 512-row slice (7 payload "
                                     "slices + local) + decompress 4096x11008 (fp32)"}
    log("receiver %-22s median %7.1f us  (one rank's kernels of an 8-rank compressed AllReduce)" % (
        "allreduce_rank", med * 1e6))
    res["workload"] = ("k=8 peers of bf16 4096x11008 N(0,1e-3), seeds 4..11; the _local entry sums "
                       "peers 0..6 and adds peer 7's bf16 tensor uncompressed")
    return res


def spin_up(torch, step, seconds: float = 0.25):
    """Untimed steps for a fixed wall time before the first measured leg, so that
    the first leg does not run while the GPU's clocks are still rising."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()
    return i


def variant_timing(fp4q, torch, X, P, Y, iters: int = 40):
    """The other entry points on the same 32768 x 4096 buffers (three rotating
    sets, HIP events around every launch, a queued head start): median launch
    time, algorithmic bytes and the HBM roofline fraction."""
    n = X[0].numel()
    S = len(X)
    nf = fp4q.FP4Q_FLAG_NO_FWHT
    Yb = [torch.empty(X[0].shape, dtype=torch.bfloat16, device=X[0].device) for _ in range(S)]
    MX = [fp4q.fp4q_compress_mx(X[s]) for s in range(S)]
    pay = n // 2 + n // 16 + n // 64
    mx_pay = n // 2 + n // 32
    cases = (
        ("decompress_bf16_out", lambda s: fp4q.fp4q_decompress(*P[s], out=Yb[s]), pay + 2 * n),
        ("compress_no_fwht", lambda s: fp4q.fp4q_compress(X[s], *P[s], flags=nf), 2 * n + pay),
        ("decompress_no_fwht", lambda s: fp4q.fp4q_decompress(*P[s], out=Y[s], flags=nf), pay + 4 * n),
        ("compress_mx", lambda s: fp4q.fp4q_compress_mx(X[s], *MX[s]), 2 * n + mx_pay),
        ("decompress_mx", lambda s: fp4q.fp4q_decompress_mx(*MX[s], out=Y[s]), mx_pay + 4 * n),
        ("decompress_mx_bf16_out", lambda s: fp4q.fp4q_decompress_mx(*MX[s], out=Yb[s]), mx_pay + 2 * n),
    )
    res = {}
    for name, fn, nbytes in cases:
        for i in range(6):
            fn(i % S)
        torch.cuda.synchronize()
        for i in range(16):
            fn(i % S)
        ev = [(TimingEvent(), TimingEvent()) for _ in range(iters)]
        for i in range(iters):
            ev[i][0].record()
            fn(i % S)
            ev[i][1].record()
        torch.cuda.synchronize()
        med = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
        gbps = nbytes / med / 1e9
        res[name] = {"median_us": round(med * 1e6, 2), "algorithmic_bytes": nbytes,
                     "achieved_GBps": round(gbps, 1), "frac": round(gbps / PEAK_GBPS, 4)}
        log("variant %-20s median %7.1f us  %7.1f GB/s  %.1f%% of HBM peak" % (
            name, med * 1e6, gbps, 100 * gbps / PEAK_GBPS))
    # restore the payloads the step uses (the no-transform compress overwrote them)
    for s in range(S):
        fp4q.fp4q_compress(X[s], *P[s])
    torch.cuda.synchronize()
    return res


TWINS_LIB = os.path.join(ROOT, "tests", "hip", "libfp4q_twins.so")


def ceilings(fp4q, inputs, torch, dev, X, P, Y, iters: int = 40):
    """Compute-free traffic twins of the kernels (tests/hip/fp4q_twins.hip: the
    same launch shape and the same memory instructions, calling the kernels' own
    load and store functions, with the arithmetic left out), timed like the
    variants on the same buffers: what each kernel's exact traffic pattern costs
    the memory system.  Plus plain read and write streams of 512 MiB (1 KiB per
    instruction, the library's load and store policies).  None if the twins
    library has not been built."""
    if not os.path.exists(TWINS_LIB):   # built by __graft_entry__.build(); else try now
        try:
            import importlib.util
            spec = importlib.util.spec_from_file_location("hip_build", os.path.join(
                os.path.dirname(TWINS_LIB), "build.py"))
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.build()
        except Exception as e:  # noqa: BLE001 - the ceilings are context, not the metric
            log("ceilings: %s not built (%s), skipped" % (TWINS_LIB, e))
            return None
    import ctypes
    L = ctypes.CDLL(TWINS_LIB)
    Pp, I64 = ctypes.c_void_p, ctypes.c_int64
    L.twin_compress.argtypes = [Pp, I64, I64, Pp, Pp, Pp, Pp]
    L.twin_decompress.argtypes = [Pp, Pp, Pp, I64, I64, Pp, ctypes.c_int, Pp]
    L.twin_accumulate.argtypes = [ctypes.c_int, Pp, Pp, Pp, I64, I64, Pp, Pp]
    L.twin_read.argtypes = [Pp, I64, Pp, Pp]
    L.twin_write.argtypes = [Pp, I64, Pp]
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows, Lr = X[0].shape
    n = rows * Lr
    S = len(X)
    ab = algorithmic_bytes(n)
    k, rr, rl = REDUCE_K, 4096, 11008
    pays = [fp4q.fp4q_compress(torch.from_numpy(q.view(np.int16)).to(dev)) for q in reduce_peers(inputs)]
    # three rotating copies of the peers and outputs, as the receiver leg times the kernels
    psets = [pays] + [[tuple(t.clone() for t in q) for q in pays] for _ in range(2)]
    PA = ctypes.c_void_p * k
    ptrs = [tuple(PA(*[ptr(q[i]) for q in ps]) for i in range(3)) for ps in psets]
    raccs = [torch.empty((rr, rl), dtype=torch.float32, device=dev) for _ in range(3)]
    nbig = 512 << 20
    big = [torch.empty(nbig, dtype=torch.uint8, device=dev) for _ in range(2)]
    sink = torch.empty(nbig // 1024, dtype=torch.uint8, device=dev)

    def ok(rc):
        if rc != 0:
            raise RuntimeError("twin launch failed: %d" % rc)

    cases = (
        ("compress", lambda i: ok(L.twin_compress(ptr(X[i % S]), rows, Lr, *[ptr(t) for t in P[i % S]], stream())),
         ab["compress"]),
        ("decompress", lambda i: ok(L.twin_decompress(*[ptr(t) for t in P[i % S]], rows, Lr, ptr(Y[i % S]), 0,
                                                      stream())), ab["decompress"]),
        ("decompress_bf16_out", lambda i: ok(L.twin_decompress(*[ptr(t) for t in P[i % S]], rows, Lr,
                                                               ptr(Y[i % S]), 1, stream())),
         ab["decompress"] - 2 * n),
        ("accumulate_k8", lambda i: ok(L.twin_accumulate(k, *ptrs[i % 3], rr, rl, ptr(raccs[i % 3]), stream())),
         _receiver_bytes()["accumulate"]),
        # written first: reads of never-written pages were served at an impossible 22 TB/s
        ("write_512MiB", lambda i: ok(L.twin_write(ptr(big[i % 2]), nbig, stream())), nbig),
        ("read_512MiB", lambda i: ok(L.twin_read(ptr(big[i % 2]), nbig, ptr(sink), stream())), nbig),
    )
    res = {}
    for name, fn, nbytes in cases:
        for i in range(6):
            fn(i)
        torch.cuda.synchronize()
        for i in range(16):
            fn(i)
        ev = [(TimingEvent(), TimingEvent()) for _ in range(iters)]
        for i in range(iters):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        med = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
        gbps = nbytes / med / 1e9
        res[name] = {"median_us": round(med * 1e6, 2), "bytes": nbytes, "achieved_GBps": round(gbps, 1),
                     "frac": round(gbps / PEAK_GBPS, 4)}
        log("ceiling %-14s median %7.1f us  %7.1f GB/s  %.1f%% of HBM peak" % (
            name, med * 1e6, gbps, 100 * gbps / PEAK_GBPS))
    # the twins of the step itself, in the step's context: compress twin and
    # decompress twin alternated over the same rotation (decompress reading the
    # previous step's payload), first 20 steps by wall clock, then 60 steps with
    # events around each launch, as the headline kernels are timed
    def twin_step(i, e=None):
        s_ = i % S
        if e:
            e[0].record()
        cases[0][1](s_)
        if e:
            e[1].record()
            e[2].record()
        ok(L.twin_decompress(*[ptr(t) for t in P[(s_ - 1) % S]], rows, Lr, ptr(Y[s_]), 0, stream()))
        if e:
            e[3].record()
    for i in range(10):
        twin_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(20):
        twin_step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / 20
    ev = [[TimingEvent() for _ in range(4)] for _ in range(KERNEL_PASS)]
    for i in range(KERNEL_PASS):
        twin_step(i, ev[i])
    torch.cuda.synchronize()
    tc = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    td = float(np.median([e[2].elapsed_time(e[3]) for e in ev])) * 1e-3
    res["step"] = {"ms_per_step": round(wall * 1e3, 4), "compress_median_us": round(tc * 1e6, 2),
                   "decompress_median_us": round(td * 1e6, 2)}
    log("ceiling step (twins alternated as the step): %.4f ms/step; per-kernel medians: compress %.1f us, "
        "decompress %.1f us" % (wall * 1e3, tc * 1e6, td * 1e6))
    del pays, psets, raccs, big, sink
    # the twins wrote the step's payloads and outputs: restore the payloads
    for s_ in range(S):
        fp4q.fp4q_compress(X[s_], *P[s_])
    torch.cuda.synchronize()
    res["what"] = ("compute-free kernels with each kernel's launch shape and memory instructions "
                   "(tests/hip/fp4q_twins.hip), each timed alone; step: the compress and decompress "
                   "twins alternated as the step alternates the kernels; read/write: plain 512 MiB "
                   "streams")
    return res


def fwht_tradeoff(fp4q, inputs, torch, dev, iters: int = 50):
    """Throughput and relative RMSE with and without the transform on the activation
    (2048x4096) and outlier (8192x4096) workloads.  These tensors fit in the 256 MB
    last-level cache, so their rates are cache-resident, not HBM roofline figures.
    Times are GPU time per compress + decompress, from a HIP graph of `iters`
    steps replayed 5 times."""
    rows_out = []
    for name in ("act2048", "outlier8192"):
        xb = inputs.make_config(name)
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        xf = x.double()
        for fmt, flags, label in (("dual", 0, "fwht"), ("dual", fp4q.FP4Q_FLAG_NO_FWHT, "no_fwht"),
                                  ("mx", 0, "mx_fwht"), ("mx", fp4q.FP4Q_FLAG_NO_FWHT, "mx_no_fwht")):
            if fmt == "dual":
                P = fp4q.fp4q_compress(x, flags=flags)
                Y = fp4q.fp4q_decompress(*P, flags=flags)

                def once(P=P, Y=Y, flags=flags):
                    fp4q.fp4q_compress(x, *P, flags=flags)
                    fp4q.fp4q_decompress(*P, out=Y, flags=flags)
            else:
                P = fp4q.fp4q_compress_mx(x, flags=flags)
                Y = fp4q.fp4q_decompress_mx(*P, flags=flags)

                def once(P=P, Y=Y, flags=flags):
                    fp4q.fp4q_compress_mx(x, *P, flags=flags)
                    fp4q.fp4q_decompress_mx(*P, out=Y, flags=flags)
            for _ in range(5):
                once()
            torch.cuda.synchronize()
            # GPU time per step: `iters` steps captured in one HIP graph, replayed
            # (on tensors this small the Python calls would otherwise dominate)
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for _ in range(iters):
                        once()
            torch.cuda.current_stream().wait_stream(side)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = TimingEvent(), TimingEvent()
            reps = 5
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            dt = e0.elapsed_time(e1) * 1e-3 / (reps * iters)
            del g
            rmse = float(torch.linalg.vector_norm(Y.double() - xf) / torch.linalg.vector_norm(xf))
            rows_out.append({"workload": name, "transform": label, "us_per_step": round(dt * 1e6, 1),
                             "GBps_bf16_in": round(2 * x.numel() / dt / 1e9, 1),
                             "rel_rmse": round(rmse, 6), "cache_resident": True})
            log("tradeoff %-12s %-8s %7.1f us  %7.1f GB/s  rel RMSE %.6f" % (
                name, label, dt * 1e6, 2 * x.numel() / dt / 1e9, rmse))
    return rows_out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_REDUCE_PEERS = []


def reduce_peers(inputs):
    """The k = 8 reduce workload's peers (bf16 bits, host), generated once and
    shared by the receiver leg and the CPU baseline."""
    if not _REDUCE_PEERS:
        _REDUCE_PEERS.extend(inputs.make_reduce_peer(p) for p in range(REDUCE_K))
    return _REDUCE_PEERS


def _host_cpus():
    """(nproc, CPUs this process may run on, the OMP_NUM_THREADS share or None)."""
    nproc = os.cpu_count() or 1
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    omp = os.environ.get("OMP_NUM_THREADS", "")
    share = int(omp) if omp.isdigit() and int(omp) > 0 else None
    return nproc, affinity, share


def cpu_baseline(xb: np.ndarray, wl: str, runs: int = 3, single_rows: int = 1024):
    """The oracle on the host, as it stands: compress and decompress timed
    separately (median of `runs` runs each) on every workload, and the k = 8
    receiver reduce (fp64 accumulate of 8 payloads), once on all usable cores
    (the CPUs this process may run on, capped by OMP_NUM_THREADS where the host
    sets that share) and once on one thread.  Single-threaded legs take the first
    `single_rows` rows (512 for the reduce); rates are GB/s of bf16 input (the
    reduce: of the 8 peers' bf16 tensors)."""
    import oracle
    from fp4_communication_compression_amd import inputs
    nproc, affinity, share = _host_cpus()
    threads = max(1, min(affinity, share) if share else affinity)

    def med(fn):
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def codec(x, th):
        oracle.set_threads(th)
        p = oracle.compress(x)
        tc = med(lambda: oracle.compress(x))
        td = med(lambda: oracle.decompress(p["codes"], p["micro"], p["block"]))
        gb = 2 * x.size / 1e9
        return {"threads": th, "rows": int(x.shape[0]), "compress_s": round(tc, 4),
                "decompress_s": round(td, 4), "compress_GBps": round(gb / tc, 4),
                "decompress_GBps": round(gb / td, 4), "GBps": round(gb / (tc + td), 4)}

    per = {}
    for name in ("tiny", "act2048", "outlier8192", HEADLINE):
        x = xb if name == wl else inputs.make_config(name)
        per[name] = {"all_cores": codec(x, threads), "single_thread": codec(x[:single_rows], 1)}
        log("cpu oracle %-12s all cores (%d) %.4f GB/s (compress %.4f, decompress %.4f); one thread %.4f" % (
            name, threads, per[name]["all_cores"]["GBps"], per[name]["all_cores"]["compress_GBps"],
            per[name]["all_cores"]["decompress_GBps"], per[name]["single_thread"]["GBps"]))

    def reduce_leg(peers, th):
        oracle.set_threads(th)
        pay = [oracle.compress(q) for q in peers]
        trip = [(r["codes"], r["micro"], r["block"]) for r in pay]
        t = med(lambda: oracle.accumulate_f64(trip))
        gb = 2 * sum(q.size for q in peers) / 1e9
        return {"threads": th, "rows": int(peers[0].shape[0]), "k": len(peers),
                "accumulate_s": round(t, 4), "GBps": round(gb / t, 4)}

    red = reduce_peers(inputs)
    tiny_peers = [inputs.make_normal(4, 256, seed=100 + p) for p in range(REDUCE_K)]
    per["reduce_k8"] = {"all_cores": reduce_leg(red, threads),
                        "single_thread": reduce_leg([q[:512] for q in red], 1)}
    per["tiny_reduce_k8"] = {"all_cores": reduce_leg(tiny_peers, threads),
                             "single_thread": reduce_leg(tiny_peers, 1)}
    for name in ("reduce_k8", "tiny_reduce_k8"):
        log("cpu oracle %-14s accumulate: all cores %.4f GB/s, one thread %.4f GB/s" % (
            name, per[name]["all_cores"]["GBps"], per[name]["single_thread"]["GBps"]))
    oracle.set_threads(threads)
    a = per[wl]["all_cores"]
    return {"value": a["GBps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the whole %d x %d tensor: compress and decompress timed separately, median "
                      "of %d runs each (%.2f s + %.2f s)" % (xb.shape[0], xb.shape[1], runs,
                                                             a["compress_s"], a["decompress_s"]),
            "cpu_model": _cpu_model(), "nproc": nproc, "affinity_cpus": affinity,
            "omp_num_threads": share, "threads": threads, "workloads": per}


def copy_reference(torch, dev):
    """Three plain device-to-device copies of COPY_REF_BYTES (the runtime's blit
    kernel): the scale reference for the HBM byte counters."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    src = torch.empty(COPY_REF_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        rc = hip.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                COPY_REF_BYTES, 3, stream)  # 3 = device to device
        if rc != 0:
            raise RuntimeError("hipMemcpyAsync failed: %d" % rc)
    torch.cuda.synchronize()
    del src, dst


def cold_timing(fp4q, torch, X, P, Y, reps: int = 10, flush_bytes: int = 2 << 30):
    """Single launches from a cold cache: before each one, a read of flush_bytes
    (a reduction over a buffer eight times the last-level cache) evicts what the
    previous launch left and drains its write-back.  The kernel and its event
    pair are queued right behind that read, so the host's launch latency never
    falls inside the events.  Medians of `reps` launches."""
    flush = torch.ones(flush_bytes // 8, dtype=torch.int64, device=X[0].device)
    n = X[0].numel()
    ab = algorithmic_bytes(n)
    res = {}
    for name, fn in (("compress", lambda: fp4q.fp4q_compress(X[0], *P[0])),
                     ("decompress", lambda: fp4q.fp4q_decompress(*P[1], out=Y[0]))):
        ev = [(TimingEvent(), TimingEvent())
              for _ in range(reps)]
        for a, b in ev:
            flush.max()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        med = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
        gbps = ab[name] / med / 1e9
        res[name] = {"median_us": round(med * 1e6, 2), "achieved_GBps": round(gbps, 1),
                     "frac": round(gbps / PEAK_GBPS, 4)}
        log("cold %-10s median %7.1f us  %7.1f GB/s  %.1f%% of HBM peak" % (
            name, med * 1e6, gbps, 100 * gbps / PEAK_GBPS))
    del flush
    res["flush"] = "%d MiB read before each launch" % (flush_bytes >> 20)
    return res


def copy_ceiling(torch, dev, nbytes: int = 512 << 20, iters: int = 20):
    """A plain device-to-device copy (the runtime's copy kernel) between two
    buffers of nbytes, timed with HIP events: the GB/s (bytes read + written)
    a copy reaches on this GPU, as context for the roofline fractions."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(3)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def copy(i):
        src, dst = bufs[i % 3], bufs[(i + 1) % 3]
        rc = hip.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                nbytes, 3, stream)  # 3 = device to device
        if rc != 0:
            raise RuntimeError("hipMemcpyAsync failed: %d" % rc)
    for i in range(4):
        copy(i)
    torch.cuda.synchronize()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        copy(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    med = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    del bufs
    gbps = 2 * nbytes / med / 1e9
    log("copy ceiling: %d MiB device copy %.1f us, %.0f GB/s (read + write)" % (nbytes >> 20, med * 1e6, gbps))
    return {"bytes_per_copy": nbytes, "median_us": round(med * 1e6, 1), "GBps_read_plus_write": round(gbps, 1),
            "frac": round(gbps / PEAK_GBPS, 4)}


def graph_timed_steps(torch, fp4q, step, X, P, Y, S, args, min_steps: int = 40):
    """The timed steps as replays of a HIP graph of m steps (m a multiple of the
    S buffer sets, at least min_steps), then one replay of a graph of the
    remaining K mod m steps, so exactly K steps are timed: on tensors this small,
    launching from Python would take longer than the kernels.  Per-kernel
    durations: HIP events around replays of graphs of m compress launches and of
    m decompress launches on the same rotation, divided by m."""
    m = S * -(-min_steps // S)

    def capture(fn, count=m):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(count):
                    fn(i)
        torch.cuda.current_stream().wait_stream(side)
        return g

    g_step = capture(step)
    reps, rest = divmod(args.steps, m)
    g_rest = capture(step, rest) if rest else None   # continues the rotation: m % S == 0
    g_c = capture(lambda i: fp4q.fp4q_compress(X[i % S], *P[i % S]))
    g_d = capture(lambda i: fp4q.fp4q_decompress(*P[(i % S - 1) % S], out=Y[i % S]))
    torch.cuda.synchronize()
    log("graph of %d steps; warmup %d" % (m, args.warmup))
    for _ in range(-(-args.warmup // m)):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g_step.replay()
    if g_rest is not None:
        g_rest.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {}
    for name, g in (("compress", g_c), ("decompress", g_d)):
        g.replay()
        ev = [(TimingEvent(), TimingEvent())
              for _ in range(10)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        per[name] = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3 / m
    timing = ("HIP graph replays of %d steps (and one of the remaining %d); per-kernel: HIP events "
              "around replays of graphs of %d launches of each kernel, divided by %d" % (m, rest, m, m))
    return args.steps, wall, per["compress"], per["decompress"], timing


SWEEP_ROWS = (64, 512, 1024, 2048, 4096, 8192)


def size_sweep(fp4q, torch, dev, launches: int = 40, replays: int = 7):
    """Launch time against tensor size (rows of 4096, N(0,1), seed 5): for each
    size a HIP graph of `launches` compress (then decompress) calls on the same
    buffers, replayed `replays` times with events around each replay; the median
    replay divided by `launches`.  The small tensors stay in the caches: this
    measures the fixed cost of a launch and its ramp, not HBM rates."""
    out = []
    for rows in SWEEP_ROWS:
        x = torch.from_numpy(np.random.default_rng(5).standard_normal((rows, 4096), dtype=np.float32)).to(dev)
        x = x.to(torch.bfloat16)
        P = fp4q.fp4q_compress(x)
        y = torch.empty((rows, 4096), dtype=torch.float32, device=dev)
        calls = {"compress": lambda: fp4q.fp4q_compress(x, *P),
                 "decompress": lambda: fp4q.fp4q_decompress(*P, out=y)}
        row = {"rows": rows, "wavefronts": rows * 4096 // 256 // 16}
        for name, call in calls.items():
            s = torch.cuda.Stream()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                for _ in range(3):
                    call()
                s.synchronize()
                with torch.cuda.graph(g, stream=s):
                    for _ in range(launches):
                        call()
            torch.cuda.synchronize()
            ts = []
            for _ in range(replays):
                a, b = TimingEvent(), TimingEvent()
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / launches)
            row[name + "_us"] = round(float(np.median(ts)), 2)
        log("size %5d rows (%5d wavefronts): compress %6.2f us, decompress %6.2f us" % (
            rows, row["wavefronts"], row["compress_us"], row["decompress_us"]))
        out.append(row)
    return out


def kernel_pass(fp4q, torch, X, P, Y, S, first_step: int, steps: int = KERNEL_PASS):
    """Per-kernel durations, in a pass of its own after the timed region: `steps`
    more steps of the same rotation, each kernel bracketed by its own pair of
    HIP events on the launch stream.  Returns the compress and decompress
    durations (seconds), one per launch."""
    ev = [[TimingEvent() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for j in range(steps):
        s = (first_step + j) % S
        e = ev[j]
        e[0].record()
        fp4q.fp4q_compress(X[s], *P[s])
        e[1].record()
        e[2].record()
        fp4q.fp4q_decompress(*P[(s - 1) % S], out=Y[s])
        e[3].record()
    torch.cuda.synchronize()
    t_c = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    t_d = np.array([e[2].elapsed_time(e[3]) for e in ev]) * 1e-3
    return t_c, t_d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1, help="number of GPUs (only 1 is supported)")
    ap.add_argument("--steps", type=int, default=400, help="timed compress + decompress steps")
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps before them")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=HEADLINE,
                    help="the tensor each step compresses and decompresses (default: the "
                         "32768x4096 headline workload)")
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="time the steps as HIP graph replays (auto: for every workload but the "
                         "headline, where the eager launches keep ahead of the GPU)")
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating buffer sets (default: enough to span %d MiB, at least 3, "
                         "which keeps reads out of the last-level cache)" % (ROTATION_BYTES >> 20))
    ap.add_argument("--no-receiver", action="store_true",
                    help="skip the receiver-kernel timings on the k=8 reduce workload")
    ap.add_argument("--receiver-only", action="store_true",
                    help="time only the receiver kernels on the k=8 reduce workload (for profiling) "
                         "and print their JSON")
    ap.add_argument("--no-tradeoff", action="store_true",
                    help="skip the throughput and error report with and without the transform "
                         "on the 2048x4096 and 8192x4096 workloads (cache-resident)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip timing the compute-free traffic twins of the kernels")
    ap.add_argument("--copy-reference", action="store_true",
                    help="also run a plain %d-byte device copy (counter scale reference)" % COPY_REF_BYTES)
    ap.add_argument("--size-sweep", action="store_true",
                    help="only time compress and decompress launches against tensor size (rows of 4096)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--timed-steps", type=int, default=0,
                    help="with --summarize-trace: the traced run's --steps, to report its timed "
                         "region's launches of the headline kernels on their own")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="PMC_DIR",
                    help="print the per-kernel summary of rocprofv3 --pmc runs (one directory per "
                         "pass) and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the kernel durations of a rocprofv3 --kernel-trace --stats run and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.timed_steps))
        return
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU; the library has no multi-GPU exchange "
              "(the method shards by block range with no halo, so a GPU's share is measured "
              "as is); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp4_communication_compression_amd as fp4q
    from fp4_communication_compression_amd import inputs

    fp4q.lib()
    dev = torch.device("cuda:0")
    if args.receiver_only:
        if args.copy_reference:
            copy_reference(torch, dev)
        print(json.dumps({"receiver": receiver_timing(fp4q, inputs, torch, dev)}), flush=True)
        return
    if args.size_sweep:
        print(json.dumps({"size_sweep": size_sweep(fp4q, torch, dev)}), flush=True)
        return
    wl = args.workload
    rows, L = inputs.CONFIGS[wl][:2]
    n = rows * L
    log("generating %s (%dx%d) ..." % (wl, rows, L))
    xb = inputs.make_config(wl)
    x0 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    per_set = sum(algorithmic_bytes(n).values()) - (n // 2 + n // 16 + n // 64)  # in + payload + out
    S = max(2, args.sets) if args.sets else max(3, -(-ROTATION_BYTES // per_set))
    X = [x0] + [x0.clone() for _ in range(S - 1)]
    P = [fp4q.fp4q_compress(X[s]) for s in range(S)]
    Y = [torch.empty((rows, L), dtype=torch.float32, device=dev) for _ in range(S)]
    torch.cuda.synchronize()

    def step(i):
        s = i % S
        fp4q.fp4q_compress(X[s], *P[s])
        fp4q.fp4q_decompress(*P[(s - 1) % S], out=Y[s])

    if args.copy_reference:
        copy_reference(torch, dev)

    # The other GPU legs run first: besides their own figures they bring the GPU
    # to a steady state (clocks, memory pools) before the timed region, whatever
    # --warmup is.
    result = {}
    if wl == HEADLINE:
        spin_up(torch, step)
        result["variants"] = variant_timing(fp4q, torch, X, P, Y)
        result["cold"] = cold_timing(fp4q, torch, X, P, Y)
        if not args.no_receiver:
            result["receiver"] = receiver_timing(fp4q, inputs, torch, dev)
        if not args.no_tradeoff:
            result["tradeoff"] = fwht_tradeoff(fp4q, inputs, torch, dev)
        if not args.no_ceilings:
            result["ceilings"] = ceilings(fp4q, inputs, torch, dev, X, P, Y)
        # the copy ceiling's 512 MiB copies would join the counter-scale reference's
        # 256 MiB copies in a --copy-reference run (the summary takes the largest copies)
        if not args.copy_reference:
            result["copy_ceiling"] = copy_ceiling(torch, dev)

    # RMSE with and without the transform (GPU path), reported only
    out = fp4q.fp4q_decompress(*fp4q.fp4q_compress(X[0]))
    out_nf = fp4q.fp4q_decompress(*fp4q.fp4q_compress(X[0], flags=fp4q.FP4Q_FLAG_NO_FWHT),
                                  flags=fp4q.FP4Q_FLAG_NO_FWHT)
    torch.cuda.synchronize()
    xf = x0.double()
    rmse = float(torch.linalg.vector_norm(out.double() - xf) / torch.linalg.vector_norm(xf))
    rmse_nf = float(torch.linalg.vector_norm(out_nf.double() - xf) / torch.linalg.vector_norm(xf))
    del out, out_nf, xf
    for s in range(S):   # the step's payloads, from the transform (the legs above reused them)
        fp4q.fp4q_compress(X[s], *P[s])
    torch.cuda.synchronize()

    use_graph = args.graph == "on" or (args.graph == "auto" and wl != HEADLINE)
    if use_graph:
        K, wall, t_c, t_d, timing = graph_timed_steps(torch, fp4q, step, X, P, Y, S, args)
    else:
        log("warmup %d" % args.warmup)
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        K = args.steps
        t0 = time.perf_counter()
        for i in range(K):
            step(args.warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        t_c, t_d = kernel_pass(fp4q, torch, X, P, Y, S, args.warmup + K)
        timing = ("order: 0.25 s of untimed steps, then the variant, cold, receiver, trade-off, "
                  "copy and error legs (steady state), then %d warm-up steps, then %d timed steps by wall clock (eager launches, "
                  "nothing else queued), then a separate pass of %d steps with HIP events around "
                  "each kernel; per-kernel figures are that pass's medians" % (args.warmup, K, KERNEL_PASS))
    log("timed %d steps: %.4f ms/step; per-kernel medians: compress %.1f us, decompress %.1f us "
        "(%d launches each)" % (K, wall / K * 1e3, np.median(t_c) * 1e6, np.median(t_d) * 1e6, len(t_c)))

    ab = algorithmic_bytes(n)
    kern = {}
    for name, t in (("compress", t_c), ("decompress", t_d)):
        med = float(np.median(t))
        gbps = ab[name] / med / 1e9
        kern[name] = {"median_us": round(med * 1e6, 2), "avg_us": round(t.mean() * 1e6, 2),
                      "min_us": round(t.min() * 1e6, 2),
                      "p90_us": round(float(np.percentile(t, 90)) * 1e6, 2), "launches": int(len(t)),
                      "algorithmic_bytes": ab[name], "achieved_GBps": round(gbps, 1),
                      "frac": round(gbps / PEAK_GBPS, 4)}
    dom = max(kern, key=lambda k: kern[k]["median_us"])

    result = dict({
        "metric": METRIC if wl == HEADLINE else METRIC.replace("32768x4096", "%dx%d" % (rows, L)),
        "value": round(2 * n * K / wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "timing": timing,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s; compress + decompress (fp32 out) per step, %d rotating "
                               "buffer sets" % (wl, WORKLOADS[wl], S),
                   "rows": rows, "row_len": L, "block": 256, "micro_group": 16},
        "roofline": {"bound": "hbm", "achieved": kern[dom]["achieved_GBps"], "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": kern[dom]["frac"],
                     # the counter summary is the headline workload's
                     "traffic": (measured_traffic() or {}).get(dom) if wl == HEADLINE else None,
                     "kernel": dom,
                     "per_kernel_frac": {k: v["frac"] for k, v in kern.items()}},
        "kernels": kern,
        # the whole step (compress + decompress) against the HBM roofline, by wall clock
        "step_roofline_frac": round((ab["compress"] + ab["decompress"]) * K / wall / 1e9 / PEAK_GBPS, 4),
        "combined_roofline_frac": round((ab["compress"] + ab["decompress"]) /
                                        (float(np.median(t_c)) + float(np.median(t_d))) / 1e9 / PEAK_GBPS, 4),
        "rel_rmse": {"fwht": round(rmse, 6), "no_fwht": round(rmse_nf, 6)},
    }, **result)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(xb, wl)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
