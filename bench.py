#!/usr/bin/env python3
"""Decode QMV benchmark on one MI355X.

Workload (one step): the decode QMV of one hidden=5120 decoder layer at M=1
-- the seven projection shapes (q 6144x5120, k/v 1024x5120, o 5120x6144,
gate/up 17408x5120, down 5120x17408) -- for bits 1 and 2 and group sizes 64
and 128 (28 calls, affine weights with stored biases).  Inputs are seeded
synthetic tensors already resident in HBM.  Every timed sequence rotates
through enough distinct copies of its inputs (at least 512 MB) that the
256 MB last-level cache cannot serve the weights from one launch to the
next.

value = algorithmic bytes of a step (packed W + scales + biases + x + y)
        / measured step time, in GB/s.

Each step is one HIP graph replay (the graph holds the 28 launches), so
launch overhead from Python is not in the timed region.

Extra objects on the JSON line:
  roofline      the dominant kernel (2-bit, gs=64, M=1) over its seven shapes:
                algorithmic bytes per launch / average launch duration from
                HIP events around graph replays of just those launches (the
                duration is the launch period in the graph: kernel time plus
                the gap to the next launch).  traffic: HBM bytes per launch
                from FETCH_SIZE + WRITE_SIZE counters, calibrated on a copy
                kernel, when taken on the current kernel sources.

  cpu_baseline  the fp64 CPU oracle on the dominant kernel's seven shapes
                (see --cpu-sample), timed on the host.
  breakdown     per (bits, gs, shape) microseconds and GB/s.

Other modes:
  python3 bench.py --suite full            also M = 1..5 (affine, symmetric, per-row),
                                           t5, qmm, repack and verify; CSV table
  python3 bench.py --counters              calibration copy + cold decode launches
                                           (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)
  python3 bench.py --traffic-from F.csv W.csv   writes profiles/traffic.json
  python3 bench.py --qmm-counters          cold t5_qmm launches on the prefill
                                           configurations (matrix-core counters)
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
COLD_BYTES = 512 << 20  # rotation set: twice the last-level cache
CAL_BYTES = 256 << 20   # calibration copy: bytes read and bytes written
DOMINANT = "qmv_u2_gs64_m1"


def n_copies(bytes_per_copy):
    return max(2, -(-COLD_BYTES // max(1, bytes_per_copy)))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", default="q,k,v,o,gate,up,down",
                    help="shapes (2-bit, gs=64, M=1) timed with the CPU oracle")
    ap.add_argument("--suite", default="", help="'full': also time M=1..5 wide/sym, t5 and qmm "
                    "configurations and write them to --detail-csv")
    ap.add_argument("--detail-csv", default=os.path.join(ROOT, "results", "bench_detail.csv"),
                    help="where --suite full writes its per-call table")
    ap.add_argument("--counters", action="store_true",
                    help="eager calibration copy and one cold launch per shape of the dominant kernel, for "
                         "rocprofv3 --pmc runs")
    ap.add_argument("--qmm-counters", action="store_true",
                    help="one cold t5_qmm launch per prefill configuration (gs 128, gate and down, M 32, 512, "
                         "2048), for rocprofv3 --pmc runs of the matrix-core counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="rocprofv3 counter_collection.csv files of --counters runs with FETCH_SIZE and "
                         "WRITE_SIZE; writes profiles/traffic.json")
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


class Call:
    """One C ABI call on device-resident inputs."""

    def __init__(self, entry, fmt, M, N, K, gs, tensors, label):
        self.entry, self.fmt, self.M, self.N, self.K, self.gs = entry, fmt, M, N, K, gs
        self.t = tensors  # keep alive
        self.label = label
        x, w, s, b, y = tensors
        self.ptrs = (x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr() if b is not None else None,
                     y.data_ptr())
        self.bits = {"u1": 1, "u2": 2, "t5": 0}[fmt]
        self.bytes = algorithmic_bytes(fmt, M, N, K, gs, b is not None and entry != "bq_qmv_sym")

    def launch(self, lib, stream):
        x, w, s, b, y = self.ptrs
        st = getattr(lib, self.entry)(x, w, s, b, y, self.M, self.N, self.K, self.bits, self.gs, stream)
        if st != 0:
            raise RuntimeError(f"{self.entry} {self.label}: status {st}")


def upload(torch, a, dev):
    import numpy as np
    if a is None:
        return None
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def make_calls(torch, dev, specs, copies=None):
    """specs: list of (entry, fmt, M, N, K, gs, variant, label).  Returns
    calls[copy][i] with distinct device buffers per copy; by default as many
    copies as it takes for all of them to fill COLD_BYTES."""
    import synth
    base = []
    for (entry, fmt, M, N, K, gs, variant, label) in specs:
        inp = synth.make_inputs(fmt, M, N, K, gs, variant, seed=0)
        base.append([upload(torch, a, dev) for a in (inp.x, inp.w, inp.scales, inp.biases)])
    if copies is None:
        per_copy = sum(sum(t.numel() * t.element_size() for t in ts if t is not None) for ts in base)
        copies = n_copies(per_copy)
    out = [[] for _ in range(copies)]
    for (entry, fmt, M, N, K, gs, variant, label), ts in zip(specs, base):
        for c in range(copies):
            x, w, s, b = [t if (c == 0 or t is None) else t.clone() for t in ts]
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            out[c].append(Call(entry, fmt, M, N, K, gs, (x, w, s, b, y), label))
    return out


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


def per_call_seconds(torch, lib, call_copies, launches=40, replays=5):
    """Average duration of one call: graph of back-to-back launches rotating
    through the buffer copies (at least `launches`, at least one pass over
    the copies), replayed `replays` times."""
    launches = max(launches, len(call_copies))
    seq = [call_copies[i % len(call_copies)] for i in range(launches)]
    g = capture(torch, lib, seq)
    g.replay()
    t = time_graphs(torch, [g], replays)
    return t / (launches * replays)


def cpu_baseline(shapes):
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    total_bytes, total_t = 0, 0.0
    for shape in shapes:
        N, K = synth.PROJECTION_SHAPES[shape]
        inp = synth.make_inputs("u2", 1, N, K, 64, "asym", seed=0)
        t0 = time.perf_counter()
        y, _ = oracle.qmv_reference("u2", inp.x, inp.w, inp.scales, inp.biases, K, 64)
        total_t += time.perf_counter() - t0
        total_bytes += algorithmic_bytes("u2", 1, N, K, 64, True)
        del y
    return {
        "value": round(total_bytes / total_t / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle (unpack, dequantize, x@W^T), 2-bit gs=64 M=1, shapes {','.join(shapes)}: "
                  f"{total_bytes / 1e6:.1f} MB in {total_t:.2f} s; host cores visible "
                  f"{len(os.sched_getaffinity(0))}, BLAS threads {blas_threads}",
    }


def kernel_source_hash():
    """Hash of the decode kernel's own sources: qmv_kernels.hpp and its host
    launch configuration (qmv_launch.hpp).  Counter results are tied to it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_decode_qmv_amd", "csrc")
    for name in ("qmv_kernels.hpp", "qmv_launch.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM traffic per launch from committed counter runs, if they were taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        rec = data.get(kernel_key)
        if rec and rec.get("source_hash") == kernel_source_hash():
            return rec.get("bytes_per_launch")
    except Exception:  # noqa: BLE001
        return None
    return None


def full_suite(torch, lib, dev, path):
    import synth
    rows = []
    specs = []
    for fmt in ("u1", "u2"):
        for gs in (64, 128):
            for M in (1, 2, 3, 4, 5):
                for variant, entry in (("asym", "bq_qmv_wide"), ("sym", "bq_qmv_sym")):
                    for shape in SHAPES:
                        N, K = synth.PROJECTION_SHAPES[shape]
                        specs.append((entry, fmt, M, N, K, gs, variant, shape))
                for shape in ("gate", "down"):  # W read M times
                    N, K = synth.PROJECTION_SHAPES[shape]
                    specs.append(("bq_qmv", fmt, M, N, K, gs, "asym", shape))
    for gs in (64, 128):
        for M in (1, 2, 3, 4, 5):
            for shape in SHAPES:
                N, K = synth.PROJECTION_SHAPES[shape]
                specs.append(("bq_t5_qmv_wide", "t5", M, N, K, gs, "t5", shape))
    qmm_specs = []
    for M in (32, 512, 2048):
        for shape in ("gate", "down"):
            N, K = synth.PROJECTION_SHAPES[shape]
            qmm_specs.append(("bq_t5_qmm", "t5", M, N, K, 128, "t5", shape))
            for fmt in ("u1", "u2"):
                qmm_specs.append(("bq_qmm", fmt, M, N, K, 128, "asym", shape))
    with open(path, "w") as f:
        f.write("entry,fmt,variant,M,shape,N,K,gs,us,GBps,frac_hbm,TFLOPs\n")
        for spec in specs + qmm_specs:
            copies = make_calls(torch, dev, [spec])
            pair = [cs[0] for cs in copies]
            mm = spec[0] in ("bq_t5_qmm", "bq_qmm")
            launches = 8 if mm and spec[2] >= 512 else 40
            t = per_call_seconds(torch, lib, pair, launches=launches, replays=3)
            c = pair[0]
            gbs = c.bytes / t / 1e9
            tflops = (2.0 * c.M * c.N * c.K / t / 1e12) if mm else 0.0
            line = (f"{spec[0]},{spec[1]},{spec[6]},{spec[2]},{spec[7]},{spec[3]},{spec[4]},{spec[5]},"
                    f"{t * 1e6:.3f},{gbs:.1f},{gbs / PEAK_HBM_GBS:.4f},{tflops:.1f}")
            f.write(line + "\n")
            f.flush()
            print(line, file=sys.stderr, flush=True)
            rows.append(line)
            del copies, pair
            torch.cuda.empty_cache()
        for line in spec_and_repack_rows(torch, lib, dev):
            f.write(line + "\n")
            f.flush()
            print(line, file=sys.stderr, flush=True)
            rows.append(line)
    return rows


def spec_and_repack_rows(torch, lib, dev):
    """Timing of bq_spec_decode_verify (Qwen vocabulary, fp16 logits) and of
    bq_t5_repack (2-bit gate weights), as CSV rows; GB/s of the bytes each
    call must read and write."""
    import ctypes

    import numpy as np
    import synth
    out = []
    stream = torch.cuda.current_stream().cuda_stream
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

        def one():
            st = lib.bq_spec_decode_verify(lg.data_ptr(), 1, dr.data_ptr(), B, L, V, a.data_ptr(), nx.data_ptr(),
                                           None, ws.data_ptr(), n.value, stream)
            if st != 0:
                raise RuntimeError(f"bq_spec_decode_verify: status {st}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                one()
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
        for _ in range(10):
            lib.bq_t5_repack(w.data_ptr(), o.data_ptr(), N, K, 2, 128, flag.data_ptr(), stream)
    g.replay()
    t = time_graphs(torch, [g], 3) / 30
    nbytes = w.numel() * 4 + o.numel()
    gbs = nbytes / t / 1e9
    out.append(f"bq_t5_repack,u2,asym,0,gate,{N},{K},128,{t * 1e6:.3f},{gbs:.1f},{gbs / PEAK_HBM_GBS:.4f},0.0")
    return out


def counter_run(torch, lib, dev):
    """Eager launches for counter runs: one calibration copy kernel of
    CAL_BYTES read and CAL_BYTES written, then each shape of the dominant
    kernel once, each after a fresh pass of the calibration copy so that its
    inputs come from HBM."""
    import synth
    src = torch.ones(CAL_BYTES // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    torch.add(src, 1.0, out=dst)  # calibration: reads and writes CAL_BYTES
    torch.cuda.synchronize()
    specs = []
    for shape in SHAPES:
        N, K = synth.PROJECTION_SHAPES[shape]
        specs.append(("bq_qmv", "u2", 1, N, K, 64, "asym", f"u2/gs64/{shape}"))
    calls = make_calls(torch, dev, specs, copies=1)[0]
    h = torch.cuda.current_stream().cuda_stream
    for c in calls:
        torch.add(dst, 1.0, out=src)  # evicts the last-level cache
        torch.cuda.synchronize()
        c.launch(lib, h)
        torch.cuda.synchronize()
    print(json.dumps({"counter_run": [c.label for c in calls], "bytes": [c.bytes for c in calls]}), flush=True)


def qmm_counter_run(torch, lib, dev):
    """Eager launches for matrix-core counter runs: t5_qmm (gs 128) on the
    gate and down shapes at M = 32, 512, 2048, each after a pass over
    CAL_BYTES that evicts the last-level cache."""
    import synth
    src = torch.ones(CAL_BYTES // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    specs = []
    for shape in ("gate", "down"):
        N, K = synth.PROJECTION_SHAPES[shape]
        for M in (32, 512, 2048):
            specs.append(("bq_t5_qmm", "t5", M, N, K, 128, "t5", f"t5_qmm/gs128/{shape}/M{M}"))
    calls = make_calls(torch, dev, specs, copies=1)[0]
    h = torch.cuda.current_stream().cuda_stream
    for c in calls:
        torch.add(src, 1.0, out=dst)  # evicts the last-level cache
        torch.cuda.synchronize()
        c.launch(lib, h)
        torch.cuda.synchronize()
    print(json.dumps({"qmm_counter_run": [c.label for c in calls],
                      "flops": [2 * c.M * c.N * c.K for c in calls]}), flush=True)


def traffic_from(fetch_csv, write_csv):
    """profiles/traffic.json from the counter_collection.csv files of two
    --counters runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)."""
    import csv

    def read(path, counter):
        rows = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        return rows

    out = {}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = read(path, counter)
        # the calibration copy: the first elementwise add (not the fill that made its input)
        cal = [v for (_, name, v) in rows if "elementwise" in name and "_add" in name]
        qmv = [v for (_, name, v) in rows if "qmv_kernel<2, 64, 1, false" in name]
        if not cal or len(qmv) != len(SHAPES):
            raise SystemExit(f"{path}: expected a calibration copy and {len(SHAPES)} qmv dispatches, "
                             f"found {len(cal)} and {len(qmv)}")
        factor = cal[0] * 1024.0 / CAL_BYTES  # counter KiB per true KiB
        per[counter] = [v * 1024.0 / factor for v in qmv]
        out[counter] = {"calibration_kib": cal[0], "factor": round(factor, 4),
                        "kib_per_dispatch": [round(v, 1) for v in qmv]}
    per_launch = [f + w for f, w in zip(per["FETCH_SIZE"], per["WRITE_SIZE"])]
    import synth
    alg = [algorithmic_bytes("u2", 1, *synth.PROJECTION_SHAPES[s], 64, True) for s in SHAPES]
    rec = {
        "source_hash": kernel_source_hash(),
        "shapes": list(SHAPES),
        "bytes_per_launch": int(sum(per_launch) / len(per_launch)),
        "algorithmic_bytes_per_launch": int(sum(alg) / len(alg)),
        "per_shape_bytes": [int(v) for v in per_launch],
        "per_shape_algorithmic_bytes": alg,
        "counters": out,
        "method": "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, on python3 bench.py --counters; each divided "
                  f"by what it reads for a copy of {CAL_BYTES >> 20} MiB read + {CAL_BYTES >> 20} MiB written",
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[DOMINANT] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the QMV path has no multi-GPU mode (it would shard W "
              "along N with no communication); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_decode_qmv_amd as bq
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = bq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.counters:
        counter_run(torch, lib, dev)
        return
    if args.qmm_counters:
        qmm_counter_run(torch, lib, dev)
        return

    specs = []
    for bits in (1, 2):
        fmt = "u1" if bits == 1 else "u2"
        for gs in (64, 128):
            for shape in SHAPES:
                N, K = synth.PROJECTION_SHAPES[shape]
                specs.append(("bq_qmv", fmt, 1, N, K, gs, "asym", f"{fmt}/gs{gs}/{shape}"))
    copies = make_calls(torch, dev, specs)
    print(f"bench: {len(specs)} calls x {len(copies)} copies", file=sys.stderr, flush=True)
    step_bytes = sum(c.bytes for c in copies[0])

    # eager warm-up (loads the code object before any capture)
    h = torch.cuda.current_stream().cuda_stream
    for cs in copies:
        for c in cs:
            c.launch(lib, h)
    torch.cuda.synchronize()

    graphs = [capture(torch, lib, cs) for cs in copies]
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    elapsed = time_graphs(torch, graphs, args.steps)
    ms_per_step = elapsed / args.steps * 1e3
    value = step_bytes * args.steps / elapsed / 1e9

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
            "workload": "decode QMV M=1, 7 projection shapes of a hidden=5120 decoder, bits {1,2} x "
                        "group_size {64,128}, affine (stored biases)",
            "M": 1,
            "calls_per_step": len(specs),
            "bytes_per_step": step_bytes,
            "parallelism": "single GPU",
        },
    }

    if not args.profile_only:
        # dominant kernel: 2-bit, gs=64, M=1 affine, over its seven shapes
        dom_specs = [sp for sp in specs if sp[1] == "u2" and sp[5] == 64]
        dom_copies = make_calls(torch, dev, dom_specs)
        seq = [c for cs in dom_copies for c in cs]
        gd = capture(torch, lib, seq)
        gd.replay()
        reps = 5
        t = time_graphs(torch, [gd], reps)
        avg_launch = t / (reps * len(seq))
        bytes_per_launch = sum(c.bytes for c in dom_copies[0]) / len(dom_copies[0])
        achieved = bytes_per_launch / avg_launch / 1e9
        del gd, dom_copies, seq
        result["roofline"] = {
            "bound": "hbm",
            "kernel": "qmv_kernel<2-bit, gs=64, M=1, stored bias>",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(DOMINANT),
            "avg_launch_us": round(avg_launch * 1e6, 3),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
        }
        bd = {}
        for spec in specs:
            cc = make_calls(torch, dev, [spec])
            ts = per_call_seconds(torch, lib, [cs[0] for cs in cc], launches=20, replays=3)
            c = cc[0][0]
            bd[c.label] = {"us": round(ts * 1e6, 2), "GBps": round(c.bytes / ts / 1e9, 1)}
            del cc
        result["breakdown"] = bd
        if args.suite == "full":
            os.makedirs(os.path.dirname(args.detail_csv), exist_ok=True)
            del graphs
            torch.cuda.empty_cache()
            full_suite(torch, lib, dev, args.detail_csv)
        if not args.no_cpu_baseline:
            shapes = [s for s in args.cpu_sample.split(",") if s]
            print(f"bench: cpu oracle on {shapes}", file=sys.stderr, flush=True)
            result["cpu_baseline"] = cpu_baseline(shapes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
