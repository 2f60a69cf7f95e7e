#!/usr/bin/env python3
"""Decode QMV benchmark on one MI355X.

Workload (one step): the decode QMV of one hidden=5120 decoder layer -- the
seven projection shapes (q 6144x5120, k/v 1024x5120, o 5120x6144, gate/up
17408x5120, down 5120x17408) -- at M = 1..5 activation rows, for 2-bit
affine weights (stored biases, bq_qmv_wide), 2-bit symmetric weights (bias
-1.5*scale implied and never read, bq_qmv_sym) and t5 ternary weights (bias
-scale implied, bq_t5_qmv_wide), each at group sizes 64 and 128: 210 calls.
Inputs are seeded synthetic tensors already resident in HBM.  The calls run
M by M, and within one M through all 42 weight sets (about 550 MB), so no
weight set is read again before every other one has been: the 256 MB
last-level cache never serves weights from one launch to the next.

value = algorithmic bytes of a step (packed W + scales + biases [0 when
        implied] + x + y) / measured step time, in GB/s.

Each step is one HIP graph replay (the graph holds the 210 launches), so
launch overhead from Python is not in the timed region.

Extra objects on the JSON line:
  roofline      the dominant kernel family by time share of the step (one
                format, group size, bias kind and M over the seven shapes):
                algorithmic bytes per launch / average launch duration from
                HIP events around graph replays of just those launches,
                rotating input copies (>= 512 MB).  traffic: HBM bytes per
                launch from FETCH_SIZE + WRITE_SIZE counters, calibrated on a
                copy kernel, when they were taken on the current kernel
                sources (profiles/traffic.json).
  cpu_baseline  the fp64 CPU oracle on the dominant family's seven shapes,
                timed on the host cores.  The same leg checks sampled rows
                of every timed call (outputs written by the timed buffers
                before timing) against the oracle: "parity".
  breakdown     per (format-variant, gs, M, shape) microseconds and GB/s,
                each call timed alone over rotating input copies.
  families      per (format-variant, gs, M): microseconds over the seven
                shapes and share of the step.

Other modes:
  python3 bench.py --suite full            also 1-bit, per-row calls, qmm, dequant,
                                           repack and verify; CSV table
  python3 bench.py --launch-set NAME       eager launches for rocprofv3 --pmc runs:
                                           one calibration copy, then each call of the
                                           set once after a pass that evicts the cache
  python3 bench.py --traffic-from F.csv W.csv --family KEY
                                           writes profiles/traffic.json from two
                                           --launch-set family:KEY counter runs
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

METRIC = "QMV achieved HBM GB/s (W+scales+biases+x) at M=1..5; % of MI355X peak"
PEAK_HBM_GBS = 8000.0
SHAPES = ("q", "k", "v", "o", "gate", "up", "down")
MS = (1, 2, 3, 4, 5)
GROUP_SIZES = (64, 128)
# (format, variant, entry point): the three decode families of the step
FAMILIES = (("u2", "asym", "bq_qmv_wide"), ("u2", "sym", "bq_qmv_sym"), ("t5", "t5", "bq_t5_qmv_wide"))
COLD_BYTES = 512 << 20  # rotation set: twice the last-level cache
CAL_BYTES = 256 << 20   # calibration copy: bytes read and bytes written
ENTRY_OF = {("u1", "asym"): "bq_qmv_wide", ("u1", "sym"): "bq_qmv_sym", ("u2", "asym"): "bq_qmv_wide",
            ("u2", "sym"): "bq_qmv_sym", ("t5", "t5"): "bq_t5_qmv_wide", ("t5", "asym"): "bq_t5_qmv_wide"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (oracle timing and the parity check of the timed calls)")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-call breakdown")
    ap.add_argument("--suite", default="", help="'full': also time 1-bit, per-row, qmm, dequant, repack and "
                    "verify configurations and write them to --detail-csv")
    ap.add_argument("--detail-csv", default=os.path.join(ROOT, "results", "bench_detail.csv"),
                    help="where --suite full writes its per-call table")
    ap.add_argument("--launch-set", default="",
                    help="eager launches for rocprofv3 --pmc runs: 'family:KEY' (KEY like u2-asym/gs64/M5: the "
                         "seven shapes), 'decode' (gate and down, M 1..5, 2-bit affine and t5, gs 64), 't5' (t5 "
                         "gs 64 and 128, seven shapes, M 1 and 5), 'qmm' (t5 qmm gs 128 on gate and down, M 32, "
                         "512, 2048), 'dequant' (bits 1, 2, t5 on gate and down), 'next' (2-bit qmm on gate and "
                         "down at M 32 and 512, K-split at M 32; t5 repack of 2-bit gate weights; draft "
                         "verification B1 L4 and B8 L7)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="rocprofv3 counter_collection.csv files of two --launch-set family:KEY runs with "
                         "FETCH_SIZE and WRITE_SIZE; writes profiles/traffic.json")
    ap.add_argument("--family", default="", help="family key for --traffic-from")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + steps only (for rocprofv3), skip the extra measurements")
    return ap.parse_args()


def algorithmic_bytes(fmt, M, N, K, gs, bias_stored):
    G = K // gs
    if fmt == "t5":
        w = N * G * ((gs + 4) // 5)
    else:
        w = N * K * (1 if fmt == "u1" else 2) // 8
    return w + N * G * 2 * (2 if bias_stored else 1) + M * K * 2 + M * N * 2


def family_key(fmt, variant, gs, M):
    return f"{fmt}-{variant}/gs{gs}/M{M}"


class WeightSet:
    """Host and device copies of one (format, variant, gs, shape) input set
    drawn at M = 5; a call at M uses the first M rows of x."""

    def __init__(self, torch, dev, fmt, variant, gs, shape):
        import synth
        self.fmt, self.variant, self.gs, self.shape = fmt, variant, gs, shape
        self.N, self.K = synth.PROJECTION_SHAPES[shape]
        self.host = synth.make_inputs(fmt, 5, self.N, self.K, gs, variant, seed=0)
        h = self.host
        self.dev = [upload(torch, a, dev) for a in (h.x, h.w, h.scales, h.biases)]


class Call:
    """One C ABI call on device-resident inputs (x rows 0..M-1 of its set)."""

    def __init__(self, torch, entry, fmt, variant, M, N, K, gs, tensors, label):
        self.entry, self.fmt, self.variant, self.M, self.N, self.K, self.gs = entry, fmt, variant, M, N, K, gs
        self.label = label
        x, w, s, b = tensors
        x = x[:M] if x.shape[0] != M else x
        y = torch.empty((M, N), dtype=torch.float16, device=w.device)
        self.t = (x, w, s, b, y)  # keep alive
        self.ptrs = (x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr() if b is not None else None,
                     y.data_ptr())
        self.bits = {"u1": 1, "u2": 2, "t5": 0}[fmt]
        self.bytes = algorithmic_bytes(fmt, M, N, K, gs, b is not None and entry != "bq_qmv_sym")
        self.ws = None
        if entry.endswith("_ws"):
            # the K-split prefill products: a zero-filled workspace of the
            # size the library asks for (shared by this call's copies)
            import bit_quantized_decode_qmv_amd as bq
            need = bq.bq_qmm_workspace(M, N, K, self.bits, gs)
            self.ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=w.device)

    @property
    def y(self):
        return self.t[4]

    def launch(self, lib, stream):
        x, w, s, b, y = self.ptrs
        if self.ws is not None:
            st = getattr(lib, self.entry)(x, w, s, b, y, self.M, self.N, self.K, self.bits, self.gs,
                                          self.ws.data_ptr(), self.ws.numel(), stream)
        else:
            st = getattr(lib, self.entry)(x, w, s, b, y, self.M, self.N, self.K, self.bits, self.gs, stream)
        if st != 0:
            raise RuntimeError(f"{self.entry} {self.label}: status {st}")

    def copies(self, torch, n):
        """n calls on distinct copies of this call's inputs (copy 0 = self)."""
        out = [self]
        x, w, s, b, _ = self.t
        for _ in range(n - 1):
            ts = [t.clone() if t is not None else None for t in (x, w, s, b)]
            out.append(Call(torch, self.entry, self.fmt, self.variant, self.M, self.N, self.K, self.gs, ts,
                            self.label))
            if self.ws is not None:
                out[-1].ws = self.ws
        return out


class CopyRef:
    """Reference launch for the roofline: torch's elementwise add of a
    constant over nbytes/4 fp16 values (reads nbytes/2, writes nbytes/2)."""

    def __init__(self, torch, dev, nbytes):
        n = max(64, nbytes // 4)
        self.src = torch.ones(n, dtype=torch.float16, device=dev)
        self.dst = torch.empty_like(self.src)
        self.bytes = 4 * n
        self.torch = torch

    def launch(self, lib, stream):
        # on the current stream (the capturing one inside capture())
        self.torch.add(self.src, 1.0, out=self.dst)


def upload(torch, a, dev):
    import numpy as np
    if a is None:
        return None
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def n_copies(bytes_per_copy, cap=400):
    return min(cap, max(2, -(-COLD_BYTES // max(1, bytes_per_copy))))


def capture(torch, lib, calls, reps=1):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for _ in range(reps):
            for c in calls:
                c.launch(lib, h)
    return g


def time_graphs(torch, graphs, replays):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(replays):
        graphs[i % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3  # seconds


def rotation_seconds(torch, lib, seq, replays=3):
    """Average launch period of a sequence of calls on distinct buffers:
    graph of the sequence, replayed `replays` times after one warm replay."""
    g = capture(torch, lib, seq)
    g.replay()
    t = time_graphs(torch, [g], replays)
    del g
    return t / (len(seq) * replays)


def per_call_seconds(torch, lib, call, launches=40, replays=3):
    """Average duration of one call, launched back to back on copies of its
    inputs whose total exceeds the last-level cache (at least `launches`)."""
    cps = call.copies(torch, n_copies(call.bytes))
    seq = [cps[i % len(cps)] for i in range(max(launches, len(cps)))]
    t = rotation_seconds(torch, lib, seq, replays)
    del cps, seq
    return t


# --------------------------------------------------------------------------
# The step
# --------------------------------------------------------------------------
def build_step(torch, dev):
    sets = {}
    for fmt, variant, _ in FAMILIES:
        for gs in GROUP_SIZES:
            for shape in SHAPES:
                sets[(fmt, variant, gs, shape)] = WeightSet(torch, dev, fmt, variant, gs, shape)
    calls = []
    for M in MS:
        for fmt, variant, entry in FAMILIES:
            for gs in GROUP_SIZES:
                for shape in SHAPES:
                    ws = sets[(fmt, variant, gs, shape)]
                    calls.append(Call(torch, entry, fmt, variant, M, ws.N, ws.K, gs, ws.dev,
                                      f"{fmt}-{variant}/gs{gs}/M{M}/{shape}"))
                    calls[-1].set = ws
    return sets, calls


def sample_rows(N, label):
    import numpy as np
    import synth
    rng = np.random.default_rng(synth.seed_for("bench-rows", label))
    return np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 3)]))


def outputs_for_parity(torch, lib, calls):
    """Runs every call once (eager) and keeps sampled rows of its output."""
    h = torch.cuda.current_stream().cuda_stream
    for c in calls:
        c.launch(lib, h)
    torch.cuda.synchronize()
    out = []
    for c in calls:
        rows = sample_rows(c.N, c.label)
        out.append((rows, c.y[:, torch.as_tensor(rows, device=c.y.device)].float().cpu().numpy()))
    return out


def cpu_baseline_leg(calls, gpu_rows, family):
    """The CPU leg: (1) the oracle on sampled rows of every timed call,
    compared with the outputs the same device buffers gave; (2) the oracle
    timed on the dominant family's seven shapes (full weight matrices)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    worst, worst_label, bad = 0.0, "", []
    for c, (rows, y) in zip(calls, gpu_rows):
        h = c.set.host
        y_ref, mass = oracle.qmv_reference(c.fmt, h.x[:c.M], h.w, h.scales, h.biases, c.K, c.gs, rows)
        ok, r = oracle.check_close(y.astype(np.float64), y_ref, mass)
        if r > worst:
            worst, worst_label = r, c.label
        if not ok:
            bad.append(c.label)
    parity = {"calls": len(calls), "rows_checked": int(sum(len(r) for r, _ in gpu_rows)),
              "worst_err_over_tol": round(worst, 4), "worst_call": worst_label, "failed": bad,
              "rule": "|y - y_ref| <= 1e-3*sum_k|x_k w_k| + 1e-3*|y_ref| (fp64 oracle)"}
    fmt, variant, gs, M = family
    total_bytes, total_t = 0, 0.0
    for c in calls:
        if (c.fmt, c.variant, c.gs, c.M) != family:
            continue
        h = c.set.host
        t0 = time.perf_counter()
        y, _ = oracle.qmv_reference(fmt, h.x[:M], h.w, h.scales, h.biases, c.K, gs)
        total_t += time.perf_counter() - t0
        total_bytes += c.bytes
        del y
    base = {
        "value": round(total_bytes / total_t / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle (unpack, dequantize, x@W^T) on {family_key(*family[:2], gs, M)}, "
                  f"shapes {','.join(SHAPES)}: {total_bytes / 1e6:.1f} MB in {total_t:.2f} s; host cores "
                  f"visible {len(os.sched_getaffinity(0))}, BLAS threads {blas_threads}",
    }
    return base, parity


def kernel_source_hash():
    """Hash of the decode kernel's own sources: qmv_kernels.hpp and its host
    launch configuration (qmv_launch.hpp).  Counter results are tied to it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_decode_qmv_amd", "csrc")
    for name in ("qmv_kernels.hpp", "qmv_launch.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM traffic per launch from committed counter runs, if they were taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(key)
        if rec and rec.get("source_hash") == kernel_source_hash():
            return rec.get("bytes_per_launch")
    except Exception:  # noqa: BLE001
        return None
    return None


# --------------------------------------------------------------------------
# Eager launch sets for counter runs
# --------------------------------------------------------------------------
def parse_family(key):
    fv, g, m = key.split("/")
    fmt, variant = fv.split("-")
    return fmt, variant, int(g[2:]), int(m[1:])


def launch_set_specs(name):
    """(entry, fmt, variant, M, shape, gs) of a named eager launch set."""
    if name.startswith("family:"):
        fmt, variant, gs, M = parse_family(name.split(":", 1)[1])
        return [(ENTRY_OF[(fmt, variant)], fmt, variant, M, s, gs) for s in SHAPES]
    if name == "decode":
        return [(ENTRY_OF[(f, v)], f, v, M, s, 64) for f, v in (("u2", "asym"), ("t5", "t5"))
                for s in ("gate", "down") for M in MS]
    if name == "t5":
        return [("bq_t5_qmv_wide", "t5", "t5", M, s, gs) for gs in GROUP_SIZES for M in (1, 5) for s in SHAPES]
    if name == "qmm":
        return ([("bq_t5_qmm", "t5", "t5", M, s, 128) for s in ("gate", "down") for M in (32, 512, 2048)]
                + [("bq_t5_qmm_ws", "t5", "t5", 32, s, 128) for s in ("gate", "down")])
    if name == "dequant":
        return [("bq_dequant", f, "asym" if f != "t5" else "t5", 0, s, 64) for f in ("u1", "u2", "t5")
                for s in ("gate", "down")]
    if name == "next":
        # the 1/2-bit prefill product (whole and K-split), the t5 repack of
        # 2-bit gate weights, and draft verification over the Qwen
        # vocabulary (B sequences of L draft tokens, fp16 logits)
        return ([("bq_qmm", "u2", "asym", M, s, 64) for s in ("gate", "down") for M in (32, 512)]
                + [("bq_qmm_ws", "u2", "asym", 32, s, 64) for s in ("gate", "down")]
                + [("bq_t5_repack", "u2", "asym", 0, "gate", 128)]
                + [("bq_spec_decode_verify", "f16", f"B{B}L{L}", 0, "vocab", 0) for B, L in ((1, 4), (8, 7))])
    raise SystemExit(f"unknown launch set {name!r}")


def next_row_launch(torch, lib, dev, entry, fmt, variant, shape, gs, h, dst, src):
    """One eager bq_t5_repack or bq_spec_decode_verify call of the "next"
    launch set, after the cache-evicting pass; returns the bytes it must
    read and write."""
    import ctypes

    import numpy as np
    import synth
    if entry == "bq_t5_repack":
        N, K = synth.PROJECTION_SHAPES[shape]
        inp = synth.make_inputs(fmt, 1, N, K, gs, variant, seed=0)
        w = upload(torch, inp.w, dev)
        o = torch.empty((N, (K // gs) * (gs * 13 // 64)), dtype=torch.uint8, device=dev)
        flag = torch.empty(1, dtype=torch.int32, device=dev)
        torch.add(dst, 1.0, out=src)
        torch.cuda.synchronize()
        st = lib.bq_t5_repack(w.data_ptr(), o.data_ptr(), N, K, inp.bits, gs, flag.data_ptr(), h)
        nb = w.numel() * 4 + o.numel()
    else:
        B, L = (int(v) for v in variant[1:].split("L"))
        V = synth.QWEN_VOCAB
        sp = synth.make_spec_inputs(B, L, V, dtype=np.float16, seed=0)
        lg, dr = upload(torch, sp.logits, dev), upload(torch, sp.draft, dev)
        n = ctypes.c_size_t(0)
        lib.bq_spec_verify_workspace(B, L, V, ctypes.byref(n))
        ws = torch.zeros(n.value, dtype=torch.uint8, device=dev)
        a = torch.empty(B, dtype=torch.int32, device=dev)
        nx = torch.empty(B, dtype=torch.int32, device=dev)
        torch.add(dst, 1.0, out=src)
        torch.cuda.synchronize()
        st = lib.bq_spec_decode_verify(lg.data_ptr(), 1, dr.data_ptr(), B, L, V, a.data_ptr(), nx.data_ptr(), None,
                                       ws.data_ptr(), n.value, h)
        nb = lg.numel() * 2
    if st != 0:
        raise RuntimeError(f"{entry}: status {st}")
    torch.cuda.synchronize()
    return nb


def launch_set_run(torch, lib, dev, name):
    """One calibration copy kernel of CAL_BYTES read and CAL_BYTES written,
    then each call of the set once, each after a pass over CAL_BYTES that
    evicts the last-level cache, so its inputs come from HBM."""
    import synth
    src = torch.ones(CAL_BYTES // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    torch.add(src, 1.0, out=dst)  # calibration: reads and writes CAL_BYTES
    torch.cuda.synchronize()
    h = torch.cuda.current_stream().cuda_stream
    labels, nbytes = [], []
    for entry, fmt, variant, M, shape, gs in launch_set_specs(name):
        if entry in ("bq_t5_repack", "bq_spec_decode_verify"):
            nb = next_row_launch(torch, lib, dev, entry, fmt, variant, shape, gs, h, dst, src)
            labels.append(f"{entry}/{fmt}-{variant}/gs{gs}/M{M}/{shape}")
            nbytes.append(nb)
            continue
        N, K = synth.PROJECTION_SHAPES[shape]
        inp = synth.make_inputs(fmt, max(M, 1), N, K, gs, variant, seed=0)
        x, w, s, b = [upload(torch, a, dev) for a in (inp.x, inp.w, inp.scales, inp.biases)]
        torch.add(dst, 1.0, out=src)  # evicts the last-level cache
        torch.cuda.synchronize()
        if entry == "bq_dequant":
            y = torch.empty((N, K), dtype=torch.float16, device=dev)
            st = lib.bq_dequant(None, w.data_ptr(), s.data_ptr(), b.data_ptr() if b is not None else None,
                                y.data_ptr(), 0, N, K, inp.bits, gs, h)
            nb = w.numel() * w.element_size() + s.numel() * 2 * (2 if b is not None else 1) + N * K * 2
        else:
            c = Call(torch, entry, fmt, variant, M, N, K, gs, (x, w, s, b), "")
            st = 0
            c.launch(lib, h)
            nb = c.bytes
        if st != 0:
            raise RuntimeError(f"{entry}: status {st}")
        torch.cuda.synchronize()
        labels.append(f"{entry}/{fmt}-{variant}/gs{gs}/M{M}/{shape}")
        nbytes.append(nb)
        del x, w, s, b
    if name == "dequant":
        # reference for the write-bound dequant: a plain fill of the same
        # fp16 [N][K] output (gate), after the same cache-evicting pass
        N, K = synth.PROJECTION_SHAPES["gate"]
        y = torch.empty((N, K), dtype=torch.float16, device=dev)
        torch.add(dst, 1.0, out=src)
        torch.cuda.synchronize()
        y.fill_(1.0)
        torch.cuda.synchronize()
        labels.append("fill/gate")
        nbytes.append(N * K * 2)
        del y
    print(json.dumps({"launch_set": name, "calls": labels, "bytes": nbytes}), flush=True)


def traffic_from(fetch_csv, write_csv, key):
    """profiles/traffic.json entry for family KEY from the counter_collection
    CSVs of two --launch-set family:KEY runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch)."""
    import csv

    import synth
    fmt, variant, gs, M = parse_family(key)

    def read(path, counter):
        rows = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        return rows

    out, per = {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = read(path, counter)
        cal = [v for (_, name, v) in rows if "elementwise" in name and "_add" in name]
        qmv = [v for (_, name, v) in rows if "qmv_kernel" in name]
        if not cal or len(qmv) != len(SHAPES):
            raise SystemExit(f"{path}: expected a calibration copy and {len(SHAPES)} qmv dispatches, "
                             f"found {len(cal)} and {len(qmv)}")
        factor = cal[0] * 1024.0 / CAL_BYTES  # counter KiB per true KiB
        per[counter] = [v * 1024.0 / factor for v in qmv]
        out[counter] = {"calibration_kib": cal[0], "factor": round(factor, 4),
                        "kib_per_dispatch": [round(v, 1) for v in qmv]}
    per_launch = [f + w for f, w in zip(per["FETCH_SIZE"], per["WRITE_SIZE"])]
    stored = variant == "asym"
    alg = [algorithmic_bytes(fmt, M, *synth.PROJECTION_SHAPES[s], gs, stored) for s in SHAPES]
    rec = {
        "source_hash": kernel_source_hash(),
        "shapes": list(SHAPES),
        "bytes_per_launch": int(sum(per_launch) / len(per_launch)),
        "algorithmic_bytes_per_launch": int(sum(alg) / len(alg)),
        "per_shape_bytes": [int(v) for v in per_launch],
        "per_shape_algorithmic_bytes": alg,
        "counters": out,
        "method": "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, on python3 bench.py --launch-set family:"
                  f"{key}; each divided by what it reads for a copy of {CAL_BYTES >> 20} MiB read + "
                  f"{CAL_BYTES >> 20} MiB written",
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[key] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)


# --------------------------------------------------------------------------
# Full suite (CSV)
# --------------------------------------------------------------------------
def full_suite(torch, lib, dev, path):
    import synth
    specs = []
    for M in MS:
        for fmt in ("u1", "u2"):
            for gs in GROUP_SIZES:
                for variant in ("asym", "sym"):
                    for shape in SHAPES:
                        specs.append((ENTRY_OF[(fmt, variant)], fmt, variant, M, shape, gs))
                for shape in ("gate", "down"):  # W read M times
                    specs.append(("bq_qmv", fmt, "asym", M, shape, gs))
        for gs in GROUP_SIZES:
            for shape in SHAPES:
                specs.append(("bq_t5_qmv_wide", "t5", "t5", M, shape, gs))
    for M in (32, 512, 2048):
        for shape in ("gate", "down"):
            specs.append(("bq_t5_qmm", "t5", "t5", M, shape, 128))
            for fmt in ("u1", "u2"):
                specs.append(("bq_qmm", fmt, "asym", M, shape, 128))
    for M in (17, 32):  # the K-split products
        for shape in SHAPES:
            specs.append(("bq_t5_qmm_ws", "t5", "t5", M, shape, 128))
            specs.append(("bq_qmm_ws", "u2", "asym", M, shape, 128))
    rows = []
    with open(path, "w") as f:
        f.write("entry,fmt,variant,M,shape,N,K,gs,us,GBps,frac_hbm,TFLOPs\n")
        for entry, fmt, variant, M, shape, gs in specs:
            N, K = synth.PROJECTION_SHAPES[shape]
            inp = synth.make_inputs(fmt, M, N, K, gs, variant, seed=0)
            c = Call(torch, entry, fmt, variant, M, N, K, gs,
                     [upload(torch, a, dev) for a in (inp.x, inp.w, inp.scales, inp.biases)], "")
            mm = entry in ("bq_t5_qmm", "bq_qmm", "bq_t5_qmm_ws", "bq_qmm_ws")
            t = per_call_seconds(torch, lib, c, launches=8 if mm and M >= 512 else 40, replays=3)
            gbs = c.bytes / t / 1e9
            tflops = (2.0 * M * N * K / t / 1e12) if mm else 0.0
            line = (f"{entry},{fmt},{variant},{M},{shape},{N},{K},{gs},{t * 1e6:.3f},{gbs:.1f},"
                    f"{gbs / PEAK_HBM_GBS:.4f},{tflops:.1f}")
            f.write(line + "\n")
            f.flush()
            print(line, file=sys.stderr, flush=True)
            rows.append(line)
            del c
            torch.cuda.empty_cache()
        for line in dequant_rows(torch, lib, dev) + spec_and_repack_rows(torch, lib, dev):
            f.write(line + "\n")
            f.flush()
            print(line, file=sys.stderr, flush=True)
            rows.append(line)
    return rows


def dequant_rows(torch, lib, dev):
    """bq_dequant for bits 1, 2 and t5 (gs 64 and 128, stored and implied
    biases) on gate and down: bytes = packed W + scales (+ biases) read +
    N*K*2 written; graph of back-to-back launches over rotating inputs and
    two outputs."""
    import synth
    out = []
    h = torch.cuda.current_stream().cuda_stream
    for fmt in ("u1", "u2", "t5"):
        for gs in GROUP_SIZES:
            for variant in (("asym", "sym") if fmt != "t5" else ("t5", "asym")):
                for shape in ("gate", "down"):
                    N, K = synth.PROJECTION_SHAPES[shape]
                    inp = synth.make_inputs(fmt, 1, N, K, gs, variant, seed=0)
                    ins = [[upload(torch, a, dev) for a in (inp.w, inp.scales, inp.biases)]]
                    ins += [[t.clone() if t is not None else None for t in ins[0]] for _ in range(3)]
                    ys = [torch.empty((N, K), dtype=torch.float16, device=dev) for _ in range(2)]
                    bits = inp.bits
                    g = torch.cuda.CUDAGraph()
                    n = 8
                    with torch.cuda.graph(g):
                        hs = torch.cuda.current_stream().cuda_stream
                        for i in range(n):
                            w, s, b = ins[i % len(ins)]
                            st = lib.bq_dequant(None, w.data_ptr(), s.data_ptr(), b.data_ptr() if b is not None
                                                else None, ys[i % 2].data_ptr(), 0, N, K, bits, gs, hs)
                            if st != 0:
                                raise RuntimeError(f"bq_dequant: status {st}")
                    g.replay()
                    t = time_graphs(torch, [g], 3) / (3 * n)
                    w, s, b = ins[0]
                    nb = w.numel() * w.element_size() + s.numel() * 2 * (2 if b is not None else 1) + N * K * 2
                    gbs = nb / t / 1e9
                    out.append(f"bq_dequant,{fmt},{variant},0,{shape},{N},{K},{gs},{t * 1e6:.3f},{gbs:.1f},"
                               f"{gbs / PEAK_HBM_GBS:.4f},0.0")
                    del g, ins, ys
                    torch.cuda.empty_cache()
    del h
    return out


def spec_and_repack_rows(torch, lib, dev):
    """Timing of bq_spec_decode_verify (Qwen vocabulary, fp16 logits) and of
    bq_t5_repack (2-bit gate weights), as CSV rows; GB/s of the bytes each
    call must read and write."""
    import ctypes

    import numpy as np
    import synth
    out = []
    for B, L in ((1, 4), (8, 4), (8, 7)):
        V = synth.QWEN_VOCAB
        s = synth.make_spec_inputs(B, L, V, dtype=np.float16, seed=0)
        lg = upload(torch, s.logits, dev)
        dr = upload(torch, s.draft, dev)
        n = ctypes.c_size_t(0)
        lib.bq_spec_verify_workspace(B, L, V, ctypes.byref(n))
        ws = torch.zeros(n.value, dtype=torch.uint8, device=dev)
        a = torch.empty(B, dtype=torch.int32, device=dev)
        nx = torch.empty(B, dtype=torch.int32, device=dev)

        def one(h):
            st = lib.bq_spec_decode_verify(lg.data_ptr(), 1, dr.data_ptr(), B, L, V, a.data_ptr(), nx.data_ptr(),
                                           None, ws.data_ptr(), n.value, h)
            if st != 0:
                raise RuntimeError(f"bq_spec_decode_verify: status {st}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            # the capturing stream (the graph context makes it current)
            hs = torch.cuda.current_stream().cuda_stream
            for _ in range(20):
                one(hs)
        g.replay()
        t = time_graphs(torch, [g], 5) / 100
        nbytes = B * (L + 1) * V * 2
        gbs = nbytes / t / 1e9
        out.append(f"bq_spec_decode_verify,f16,B{B},{L},vocab,{B * (L + 1)},{V},0,{t * 1e6:.3f},{gbs:.1f},"
                   f"{gbs / PEAK_HBM_GBS:.4f},0.0")
    N, K = synth.PROJECTION_SHAPES["gate"]
    inp = synth.make_inputs("u2", 1, N, K, 128, "asym", seed=0)
    w = upload(torch, inp.w, dev)
    o = torch.empty((N, (K // 128) * 26), dtype=torch.uint8, device=dev)
    flag = torch.empty(1, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hs = torch.cuda.current_stream().cuda_stream
        for _ in range(10):
            st = lib.bq_t5_repack(w.data_ptr(), o.data_ptr(), N, K, 2, 128, flag.data_ptr(), hs)
            if st != 0:
                raise RuntimeError(f"bq_t5_repack: status {st}")
    g.replay()
    t = time_graphs(torch, [g], 3) / 30
    nbytes = w.numel() * 4 + o.numel()
    gbs = nbytes / t / 1e9
    out.append(f"bq_t5_repack,u2,asym,0,gate,{N},{K},128,{t * 1e6:.3f},{gbs:.1f},{gbs / PEAK_HBM_GBS:.4f},0.0")
    return out


# --------------------------------------------------------------------------
def main():
    args = parse()
    if args.traffic_from:
        if not args.family:
            raise SystemExit("--traffic-from needs --family KEY")
        traffic_from(*args.traffic_from, args.family)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the QMV path has no multi-GPU mode (it would shard W "
              "along N with no communication); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_decode_qmv_amd as bq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = bq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.launch_set:
        launch_set_run(torch, lib, dev, args.launch_set)
        return

    sets, calls = build_step(torch, dev)
    step_bytes = sum(c.bytes for c in calls)
    print(f"bench: {len(calls)} calls per step, {step_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)

    # eager pass: loads the code objects before any capture, and leaves the
    # outputs whose sampled rows the CPU leg checks against the oracle
    gpu_rows = outputs_for_parity(torch, lib, calls)

    graph = capture(torch, lib, calls)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    elapsed = time_graphs(torch, [graph], args.steps)
    ms_per_step = elapsed / args.steps * 1e3
    value = step_bytes * args.steps / elapsed / 1e9
    del graph

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode QMV of one hidden=5120 decoder layer: 7 projection shapes x M=1..5 x {2-bit "
                        "affine (bq_qmv_wide), 2-bit symmetric (bq_qmv_sym), t5 ternary (bq_t5_qmv_wide)} x "
                        "group_size {64,128}",
            "M": list(MS),
            "calls_per_step": len(calls),
            "bytes_per_step": step_bytes,
            "parallelism": "single GPU",
        },
    }

    if not args.profile_only:
        # per-call durations, each call alone over rotating copies of its inputs
        per = {}
        if not args.no_breakdown:
            print("bench: per-call breakdown", file=sys.stderr, flush=True)
            for c in calls:
                per[c.label] = per_call_seconds(torch, lib, c, launches=20, replays=3)
                torch.cuda.empty_cache()
            result["breakdown"] = {k: {"us": round(v * 1e6, 2),
                                       "GBps": round(next(c.bytes for c in calls if c.label == k) / v / 1e9, 1)}
                                   for k, v in per.items()}
        fam_t = {}
        for c in calls:
            k = (c.fmt, c.variant, c.gs, c.M)
            fam_t[k] = fam_t.get(k, 0.0) + per.get(c.label, 0.0)
        tot = sum(fam_t.values()) or 1.0
        if per:
            result["families"] = {family_key(*k[:2], k[2], k[3]): {"us": round(v * 1e6, 2),
                                                                    "share": round(v / tot, 4)}
                                  for k, v in sorted(fam_t.items(), key=lambda kv: -kv[1])}
            dom = max(fam_t, key=fam_t.get)
        else:
            dom = ("t5", "t5", 64, 5)
        fmt, variant, gs, M = dom
        key = family_key(fmt, variant, gs, M)
        # roofline of the dominant family: its seven launches, rotating copies
        fam_calls = [c for c in calls if (c.fmt, c.variant, c.gs, c.M) == dom]
        per_copy = sum(c.bytes for c in fam_calls)
        ncp = n_copies(per_copy, cap=64)
        copies = [c.copies(torch, ncp) for c in fam_calls]
        seq = [copies[i][j] for j in range(ncp) for i in range(len(fam_calls))]
        avg_launch = rotation_seconds(torch, lib, seq, replays=5)
        bytes_per_launch = per_copy / len(fam_calls)
        achieved = bytes_per_launch / avg_launch / 1e9
        del copies, seq
        torch.cuda.empty_cache()
        # in-run streaming reference at the same bytes per launch: a plain
        # elementwise pass (half read, half written) over the same number
        # of rotating buffers of each shape's size
        refs = [[CopyRef(torch, dev, c.bytes) for _ in range(ncp)] for c in fam_calls]
        rseq = [refs[i][j] for j in range(ncp) for i in range(len(fam_calls))]
        ref_launch = rotation_seconds(torch, lib, rseq, replays=5)
        ref_bytes = sum(r[0].bytes for r in refs) / len(fam_calls)
        del refs, rseq
        torch.cuda.empty_cache()
        result["roofline"] = {
            "bound": "hbm",
            "kernel": f"qmv_kernel family {key} (format-variant / group size / M) over its 7 shapes",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(key),
            "avg_launch_us": round(avg_launch * 1e6, 3),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "share_of_step": round(fam_t.get(dom, 0.0) / tot, 4) if per else None,
            "stream_ref": {"kind": "torch elementwise add over rotating fp16 buffers of the family's per-shape "
                                   "bytes (half read, half written), same launch sequence",
                           "avg_launch_us": round(ref_launch * 1e6, 3),
                           "GBps": round(ref_bytes / ref_launch / 1e9, 1),
                           "frac": round(ref_bytes / ref_launch / 1e9 / PEAK_HBM_GBS, 4)},
        }
        if args.suite == "full":
            os.makedirs(os.path.dirname(args.detail_csv), exist_ok=True)
            full_suite(torch, lib, dev, args.detail_csv)
        if not args.no_cpu_baseline:
            print(f"bench: cpu leg (parity of {len(calls)} calls, oracle timing on {key})", file=sys.stderr,
                  flush=True)
            base, parity = cpu_baseline_leg(calls, gpu_rows, dom)
            result["cpu_baseline"] = base
            result["parity"] = parity
    print(json.dumps(result), flush=True)
    if "parity" in result and result["parity"]["failed"]:
        print(f"bench: parity failed for {result['parity']['failed']}", file=sys.stderr, flush=True)
        sys.exit(3)


if __name__ == "__main__":
    main()
