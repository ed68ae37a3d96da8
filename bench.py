"""Benchmark: one decode step of the paged-KV hot path on one MI355X.

A step is one pass of the whole path over one batch: the paged KV append of every sequence's newest row, then
paged decode attention (single pass, or split-K phase 1 + combine, as the workload's dispatch mode says).  By default
the step is the library's fused decode step (pkv_paged_decode_step: append and attention in one launch); --unfused
times the two separate entry points (pkv_paged_kv_append, then pkv_paged_decode_attention).  The varlen workloads
(v1, v2: several new rows per sequence) time the varlen step (pkv_paged_varlen_step, one launch; --unfused:
pkv_paged_kv_append, then pkv_paged_varlen_attention), w1 the windowed decode step (pkv_paged_decode_step_window).  The r workloads start
one step earlier, from the QKV projection rows: r1 is the decode step from those rows in one launch
(pkv_paged_decode_step_qkv: q/k RMS norm, RoPE, the new K/V rows written, attention; --unfused: the QKV-to-cache
kernel, then attention); r2 times the QKV-to-cache kernel alone on a chunked-prefill batch.  Inputs
are seeded synthetic data already resident in HBM; R independent copies rotate between steps so that the ~256 MB
Infinity Cache cannot hold a step's working set (R=4 for c2).

    python bench.py [--steps K] [--warmup W] [--config c2] [--splits S] [--rotations R] [--no-cpu-baseline]
    python bench.py --copy-calibration-mib 512 ...     also runs a plain copy kernel (torch.neg, out=) of known size
    python bench.py --summarize-pmc FETCH.csv WRITE.csv --config c2   writes profiles/traffic_<config>_s<S>.json
    python bench.py --summarize-counters COUNTERS.csv                  mean per dispatch of each counter, per kernel

Prints ONE JSON line on stdout (progress goes to stderr):
  value        algorithmic HBM bytes of a step / measured step time, in GB/s (whole job, one GPU)
  roofline     the dominant kernel: algorithmic bytes / its average duration from HIP events on its stream (a fused
               single-pass step is one launch: step region / K; otherwise a second region of K back-to-back
               attention calls), against the 8 TB/s HBM peak; `traffic` is the measured HBM bytes per launch from the committed
               rocprofv3 counter summary when it was taken on the current kernel source, else null
  cpu_baseline the CPU oracle (f64, threads = the host cores it used) on a bounded sample of the same workload
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

import numpy as np  # noqa: E402

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + calls/s, 1 MI355X"
PEAK_GBS = 8000.0

WORKLOADS = {
    "c1": ("tiny paged decode: B=1, Hq=4, Hkv=2, D=64, BS=16, L=37, pool of 8 blocks", 0, 1),
    "c2": ("Llama-3-8B-shaped layer: B=32, Hq=32, Hkv=8, D=128, BS=16, L~U[512,2048], single pass", 1, 4),
    "c3": ("long-context split-K: B=4, Hq=32, Hkv=8, D=128, BS=16, L=32768, q~2N(0,1)", 8, 2),
    "c4": ("mixed serving (70B-layer-shaped, one GPU's share): B=256, Hq=64, Hkv=8, D=128, BS=16, "
           "L=lognormal(median 1024, sigma 1) clipped to [1,16384], auto dispatch", 0, 1),
    "c5": ("MHA wide head: B=128, Hq=Hkv=16, D=256, BS=32, L=4096, K/V~U(-1,1), scale 1/16", 0, 1),
    "v1": ("speculative verification, varlen (Llama-3-8B-shaped batch): B=32, Hq=32, Hkv=8, D=128, BS=16, 4 new rows "
           "per sequence, final L~U[512,2048]", 0, 4),
    "v2": ("speculative verification of 8 draft tokens, varlen (Llama-3-8B-shaped batch): B=32, Hq=32, Hkv=8, D=128, "
           "BS=16, 8 new rows per sequence, final L~U[512,2048]", 0, 4),
    "v3": ("speculative verification on the mixed serving batch: B=256, Hq=64, Hkv=8, D=128, BS=16, 4 new rows per "
           "sequence, final L lognormal (median 1024, sigma 1) clipped to [4,16384]", 0, 1),
    "w1": ("sliding-window decode on the Llama-3-8B-shaped batch: B=32, Hq=32, Hkv=8, D=128, BS=16, L~U[512,2048], "
           "window 512", 0, 8),
    "r1": ("Qwen3-8B-shaped decode step from the QKV projection: split QKV + q/k RMSNorm + RoPE + paged-cache write, "
           "then single-pass attention; B=32, Hq=32, Hkv=8, D=128, BS=16, final L~U[512,2048]", 1, 4),
    "r2": ("chunked-prefill QKV-to-cache step of the same layer: 4 sequences x 512 new rows after cached prefixes "
           "U[0,1024], split QKV + q/k RMSNorm + RoPE + paged-cache write (2048 tokens)", 1, 6),
}
WINDOWS = {"w1": 512}  # workloads run with pkv_paged_decode_attention_window, and their window


QKV_ONLY = {"r2"}  # QKV-step workloads whose step is that kernel alone (a 512-row prefill chunk's attention is not
#                    decode work)


def step_is_fused(config: str, unfused: bool) -> bool:
    """Whether bench.py times the workload's step through the library's step entry point (pkv_paged_decode_step,
    pkv_paged_decode_step_window, pkv_paged_varlen_step, or pkv_paged_decode_step_qkv for a decode step from QKV
    rows), one launch where the grid allows; QKV-only workloads time that kernel alone."""
    return not unfused and config not in QKV_ONLY


def step_launch_count(c, plan, splits: int, varlen: bool, cu: int) -> int:
    """Launches of the library's step entry point for this workload (the routing rule of pkv_paged_decode_step,
    pkv_paged_decode_step_window, pkv_paged_decode_step_qkv and pkv_paged_varlen_step): 1 when it takes its
    single-launch form, 2 or more otherwise."""
    if varlen:
        G = c.Hq // c.Hkv
        R = 16 // G
        qmax = int(c.q_lens.max())
        QT = 2 if qmax > R else 1
        grid = c.B * ((qmax + QT * R - 1) // (QT * R)) * c.Hkv
        one_pass = splits == 1 or (splits == 0 and 2 * grid >= cu)
        return 1 if one_pass and qmax <= 32 and grid <= cu and (QT == 1 or c.D <= 128) else 2
    return 1 if plan["num_splits"] == 1 and c.B * c.Hkv <= cu else 2


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of every source of the library (any change retires the traffic summaries taken before it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_04_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(config: str, splits: int, fused: bool) -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s_s%d%s.json" % (config, splits, "_fused" if fused else ""))


def measured_traffic(config: str, splits: int, fused: bool):
    """HBM bytes per launch of the dominant kernel from its traffic summary under profiles/, if taken on this
    source."""
    path = traffic_path(config, splits, fused)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_step")


def _pmc_per_dispatch(path: str, counter: str) -> dict:
    """{dispatch id: (kernel name, counter value)} from a rocprofv3 --pmc CSV (values summed over the counter's
    instances)."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name", counter) != counter:
                continue
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            name, val = rows.get(key, (r.get("Kernel_Name", ""), 0.0))
            rows[key] = (name, val + float(r["Counter_Value"]))
    return rows


def _kernel_kind(short: str):
    """(base name, fused, split) of a pkv kernel name as the profiler prints it, e.g.
    'pkv::decode_kernel<128, 16, 8, false, true, false, false>' (template arguments D, BS, NW, SPLIT, FUSED, ...;
    varlen_kernel: D, BS, NW, SPLIT, QT[, FUSED])."""
    base, _, rest = short.partition("<")
    args = [a.strip() for a in rest.rstrip(">").split(",")] if rest else []
    base = base.split("::")[-1]
    if base == "decode_kernel" and len(args) >= 5:
        return base, args[4] == "true", args[3] == "true"
    if base == "varlen_kernel" and len(args) >= 5:
        return base, len(args) >= 6 and args[5] == "true", args[3] == "true"
    return base, False, False


def dominant_kernels(config: str, names) -> list:
    """The kernels of the launch (or call) `roofline` reports: the QKV kernel for QKV-only workloads; the step
    kernel when the step is one launch (a fused single-pass kernel); otherwise the attention call's kernels
    (unfused attention, the dispatch order, the combine)."""
    if config in QKV_ONLY:
        return [n for n in names if "qkv" in n]
    kinds = {n: _kernel_kind(n) for n in names}
    step = [n for n, (_, fused, split) in kinds.items() if fused and not split]
    if step:
        return step
    return [n for n, (base, fused, _) in kinds.items()
            if (base in ("decode_kernel", "varlen_kernel") and not fused) or base in ("combine_kernel", "order_kernel", "order_varlen_kernel")]


def summarize_pmc(fetch_csv: str, write_csv: str, config: str, splits: int, copy_mib: float) -> dict:
    """HBM traffic per decode step from two counter passes (FETCH_SIZE then WRITE_SIZE, KiB per dispatch), each
    scaled by what the same counter reads for the plain copy kernel (reads and writes copy_mib MiB)."""
    out = {"config": config, "num_splits": splits, "kernel_source_hash": kernel_source_hash()}
    factors = {}
    per_kernel = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_per_dispatch(path, counter)
        copy = [v for n, v in rows.values() if "neg" in n.lower()]
        if not copy:
            raise SystemExit("no copy-calibration dispatches (torch.neg) in %s" % path)
        measured_kib = sum(copy) / len(copy)
        factors[counter] = copy_mib * 1024.0 / measured_kib
        for n, v in rows.values():
            if "pkv::" in n:
                short = n.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
                per_kernel.setdefault(short, {}).setdefault(counter, []).append(v)
    step_bytes = 0.0
    kern = {}
    dom = dominant_kernels(config, list(per_kernel))
    for short, cnt in per_kernel.items():
        f = sum(cnt.get("FETCH_SIZE", [0])) / max(1, len(cnt.get("FETCH_SIZE", [0])))
        w = sum(cnt.get("WRITE_SIZE", [0])) / max(1, len(cnt.get("WRITE_SIZE", [0])))
        fb = f * 1024 * factors["FETCH_SIZE"]
        wb = w * 1024 * factors["WRITE_SIZE"]
        kern[short] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": len(cnt.get("FETCH_SIZE", []))}
        if short in dom:
            step_bytes += fb + wb
    out.update({"copy_calibration_mib": copy_mib, "scale_factors": factors, "kernels": kern,
                "dominant_kernels": dom,
                "hbm_bytes_per_step": round(step_bytes),
                "note": "Counters are KiB per dispatch; each is scaled by its reading for the calibration copy kernel "
                        "(torch.neg over %g MiB, which reads and writes %g MiB). hbm_bytes_per_step sums, per "
                        "dispatch, the kernels of the launch or call that roofline reports (dominant_kernels: the "
                        "step kernel when a step is one launch, else the attention call's kernels; a separate append "
                        "or QKV launch excluded)." % (copy_mib, copy_mib)})
    return out


def summarize_counters(path: str) -> dict:
    """Mean value per dispatch of every counter in a rocprofv3 --pmc CSV, per kernel (pkv kernels by their short
    name, others by the start of theirs), with the dispatch count."""
    import csv
    with open(path) as f:
        counters = sorted({r["Counter_Name"] for r in csv.DictReader(f)})
    out = {}
    for counter in counters:
        for name, val in _pmc_per_dispatch(path, counter).values():
            short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            short = short if "pkv::" in short else short[:60]
            rec = out.setdefault(short, {})
            rec.setdefault(counter, []).append(val)
    return {k: dict({c: sum(v) / len(v) for c, v in cs.items()}, dispatches=max(len(v) for v in cs.values()))
            for k, cs in out.items()}


def _host_cpu() -> dict:
    """The host's logical CPU count and model name (from /proc/cpuinfo, where readable)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline_qkv(case, seconds: float, with_attention: bool):
    """The oracle's QKV step (and, for a decode step, its decode attention on the step's outputs) on the host."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    from paged_kv_decode_04_amd import workloads as W
    vc = case.varlen
    nbytes = W.algorithmic_bytes_qkv(case) + (W.algorithmic_bytes_varlen(vc)["attention"] if with_attention else 0)
    reps, t0 = 0, time.perf_counter()
    while True:
        vp = vc.v_pool.copy()
        q, k, slots = oracle.qkv_norm_rope_paged(case.qkv, case.q_norm_w, case.k_norm_w, case.cos, case.sin,
                                                 vc.cu_seqlens_q, vc.pos_offsets, vc.pos_offsets, vc.block_tables,
                                                 vc.k_pool, vp, case.eps, case.qk_mode)
        if with_attention:
            kp = vc.k_pool.copy()
            k16 = k.astype(np.float16)
            for t, slot in enumerate(slots):
                W.set_k_row(kp, int(slot) // vc.BS, slice(None), int(slot) % vc.BS, k16[t])
            oracle.decode_attention(q.astype(np.float16), kp, vp, vc.block_tables, vc.final_lens, vc.scale,
                                    threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            **_host_cpu(),
            "sample": "%d full step(s) of the workload (QKV step of %d tokens%s, f64) in %.1f s; %.3f steps/s; the "
                      "QKV step is single-threaded" % (reps, vc.T, ", then decode attention of all %d sequences x %d "
                      "heads" % (vc.B, vc.Hq) if with_attention else "", el, reps / el)}


def cpu_baseline(case, seconds: float, window: int = 0):
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    from paged_kv_decode_04_amd import workloads as W
    varlen = isinstance(case, W.VarlenCase)
    nbytes = (W.algorithmic_bytes_varlen(case) if varlen else W.algorithmic_bytes(case, window))["attention"]
    reps, t0 = 0, time.perf_counter()
    while True:
        if varlen:
            oracle.varlen_attention(case.q, case.k_pool, case.v_pool, case.block_tables, case.cu_seqlens_q,
                                    case.pos_offsets, case.scale, threads=threads)
        else:
            oracle.decode_attention(case.q, case.k_pool, case.v_pool, case.block_tables, case.context_lens,
                                    case.scale, threads=threads, window=window)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            **_host_cpu(),
            "sample": "%d full %s call(s) of the workload (all %d sequences x %d heads, f64) in %.1f s; "
                      "%.3f calls/s" % (reps, "varlen-attention" if varlen else "decode-attention", case.B, case.Hq,
                                        el, reps / el)}


def floor_tiles(case, window: int, splits: int, varlen: bool, cus: int):
    """The decode launch's tiles for the stream-read floor: (bytes read, bytes written) per workgroup in the order the
    launch dispatches them -- one per (sequence, kv head) (times the splits of a fixed split count), the sequences
    longest first when the grid has more workgroups than CUs, and then the longest split into pieces by the library's
    rule (at least 1024 rows, else all rows x kv heads / CUs rounded up to 64; rows per piece rounded up to 64)."""
    D, Hkv, G = case.D, case.Hkv, case.Hq // case.Hkv
    if varlen:
        rows = np.asarray(case.pos_offsets, np.int64) + np.diff(np.asarray(case.cu_seqlens_q, np.int64))
        outs = np.diff(np.asarray(case.cu_seqlens_q, np.int64)) * G * D * 2
    else:
        rows = np.asarray(case.context_lens, np.int64)
        rows = np.minimum(rows, window) if window > 0 else rows
        outs = np.full(len(rows), G * D * 2, np.int64)
    tiles = []  # (rows, out bytes) per (sequence or piece, kv head) in dispatch order
    seqs = list(range(len(rows)))
    multi = len(rows) * Hkv * max(1, splits) > cus
    if multi:
        seqs.sort(key=lambda i: (-rows[i], i))
    C = None
    if multi and splits <= 1 and window <= 0 and not varlen:
        fair = (int(rows.sum()) * Hkv + cus - 1) // cus
        C = max(1024, (fair + 63) // 64 * 64)
    for i in seqs:
        parts = [int(rows[i])]
        if C is not None and rows[i] > C:
            n = -(-int(rows[i]) // C)
            pr = (-(-int(rows[i]) // n) + 63) // 64 * 64
            k = -(-int(rows[i]) // pr)
            parts = [pr] * (k - 1) + [int(rows[i]) - pr * (k - 1)]
        elif splits > 1:
            ch = -(-int(rows[i]) // splits)
            parts = [max(0, min(ch, int(rows[i]) - j * ch)) for j in range(splits)]
        for part in parts:
            tiles.extend([(part * D * 4, int(outs[i]))] * Hkv)
    return tiles


def run_floor(args) -> int:
    """bench.py --floor: time the stream-read probe (libpkvprobe.so) on the workload's exact tiles."""
    import ctypes
    import torch
    from paged_kv_decode_04_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_decode_04_amd", "libpkvprobe.so"))
    lib.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    desc, default_splits, default_rot = WORKLOADS[args.config]
    splits = default_splits if args.splits is None else args.splits
    R = default_rot if args.rotations is None else args.rotations
    varlen = args.config in W.VARLEN_CONFIGS
    window = WINDOWS.get(args.config, 0)
    if args.config in W.QKV_CONFIGS:
        print("--floor covers the decode and varlen workloads", file=sys.stderr)
        return 2
    sets, total_read, total_written = [], 0, 0
    for r in range(R):
        if varlen:
            c = W.VARLEN_CONFIGS[args.config](rotation=r)
        elif window:
            c = W.config_c2(rotation=r, with_pools=False)
        else:
            c = W.CONFIGS[args.config](rotation=r, with_pools=False)
        tiles = floor_tiles(c, window, splits, varlen, cus)
        len16 = np.array([(b + 15) // 16 for b, _ in tiles], np.int64)
        off16 = np.concatenate([[0], np.cumsum(len16)[:-1]]).astype(np.int64)
        wb = (max(o for _, o in tiles) + 15) // 16 * 16
        x = torch.empty(int(len16.sum()) * 8 + 8, dtype=torch.float16, device=dev).normal_()
        y = torch.empty(len(tiles) * wb // 2 + 8, dtype=torch.float16, device=dev)
        sets.append((x, torch.from_numpy(off16).to(dev), torch.from_numpy(len16.astype(np.int32)).to(dev), y,
                     len(tiles), wb))
        total_read += int(len16.sum()) * 16
        total_written += sum(o for _, o in tiles)
        del c
    st = torch.cuda.current_stream().cuda_stream
    call = lambda k: lib.pkv_probe_stream_read(sets[k % R][0].data_ptr(), sets[k % R][0].numel() * 2,
                                               sets[k % R][1].data_ptr(), sets[k % R][2].data_ptr(),
                                               sets[k % R][3].data_ptr(), sets[k % R][4], sets[k % R][5], st)
    for k in range(args.warmup):
        if call(k) != 0:
            print("probe launch failed", file=sys.stderr)
            return 1
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(args.steps):
        call(k)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    mb = total_read / R / 1e6
    print(json.dumps({"floor": {"config": args.config, "probe": "pkv_probe_stream_read: one 512-thread workgroup "
                                "per tile in dispatch order, contiguous non-temporal reads of the tile's K/V bytes, "
                                "then its output bytes written", "workgroups": sets[0][4], "rotations": R,
                                "us_per_launch": round(us, 2), "read_MB": round(mb, 2),
                                "written_MB": round(total_written / R / 1e6, 3),
                                "GBs": round(mb * 1e3 / us, 1), "frac_of_8TBs": round(mb / us / 8e6 * 1e6, 4)}}))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--splits", type=int, default=None, help="num_splits (default: the workload's mode)")
    ap.add_argument("--rotations", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=float, default=0.0,
                    help="also run a plain copy kernel over this many MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="print the mean per dispatch of every counter in a rocprofv3 --pmc CSV, per kernel")
    ap.add_argument("--pmc-steps", type=int, nargs=2, default=(50, 10), metavar=("STEPS", "WARMUP"),
                    help="with --summarize-pmc: the --steps/--warmup of the counter runs, for the recorded commands")
    ap.add_argument("--unfused", action="store_true",
                    help="append and attention as two launches instead of the library's step entry point")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph holding 32 consecutive steps instead of eager launches")
    ap.add_argument("--floor", action="store_true",
                    help="time the stream-read probe on the workload's exact tiles instead (the plainest kernel "
                         "with one workgroup per tile: a reference for the decode launch)")
    args = ap.parse_args(argv)

    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return 0

    if args.summarize_pmc:
        splits = WORKLOADS[args.config][1] if args.splits is None else args.splits
        rec = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.config, splits,
                            args.copy_calibration_mib or 512.0)
        extra = " --unfused" if args.unfused and step_is_fused(args.config, False) else ""
        # the commands that produced the two counter files (their directories as given here)
        fetch_csv, write_csv = args.summarize_pmc
        rec["commands"] = [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o %s -- python3 bench.py --config %s "
            "--steps %d --warmup %d --no-cpu-baseline --copy-calibration-mib %g%s"
            % (os.path.dirname(fetch_csv), args.config, args.config, args.pmc_steps[0], args.pmc_steps[1],
               rec["copy_calibration_mib"], extra),
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o %s -- python3 bench.py --config %s "
            "--steps %d --warmup %d --no-cpu-baseline --copy-calibration-mib %g%s"
            % (os.path.dirname(write_csv), args.config, args.config, args.pmc_steps[0], args.pmc_steps[1],
               rec["copy_calibration_mib"], extra),
            "python bench.py --summarize-pmc %s %s --config %s%s" % (fetch_csv, write_csv, args.config, extra),
        ]
        path = traffic_path(args.config, splits, step_is_fused(args.config, args.unfused))
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only (the decode-attention hot path has no cross-GPU "
              "exchange); run with --gpus 1", file=sys.stderr)
        return 2
    if args.floor:
        return run_floor(args)

    import torch
    from paged_kv_decode_04_amd import pkv
    from paged_kv_decode_04_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    desc, default_splits, default_rot = WORKLOADS[args.config]
    splits = default_splits if args.splits is None else args.splits
    R = default_rot if args.rotations is None else args.rotations
    varlen = args.config in W.VARLEN_CONFIGS
    qkv = args.config in W.QKV_CONFIGS
    qkv_only = args.config in QKV_ONLY
    window = WINDOWS.get(args.config, 0)
    make = (W.VARLEN_CONFIGS[args.config] if varlen else W.QKV_CONFIGS[args.config] if qkv else
            (lambda rotation: W.config_c2(rotation=rotation)) if window else W.CONFIGS[args.config])

    log("building %d rotation set(s) of %s" % (R, args.config))
    sets = []
    host0 = None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    for r in range(R):
        c = make(rotation=r)
        if qkv:
            vc = c.varlen
            d = dict(qkv=t(c.qkv), qw=t(c.q_norm_w), kw=t(c.k_norm_w), cos=t(c.cos), sin=t(c.sin),
                     k_pool=t(vc.k_pool), v_pool=t(vc.v_pool), bt=t(vc.block_tables), cu=t(vc.cu_seqlens_q),
                     pos=t(vc.pos_offsets), cl=t(vc.final_lens), case=vc, qkv_case=c)
            d["q"] = torch.empty((vc.T, vc.Hq, vc.D), dtype=torch.float16, device=dev)
            d["qkv_bytes"] = W.algorithmic_bytes_qkv(c)
            d["bytes"] = {"attention": 0 if qkv_only else W.algorithmic_bytes_varlen(vc)["attention"],
                          "append": d["qkv_bytes"]}
        else:
            d = dict(q=t(c.q), k_pool=t(c.k_pool), v_pool=t(c.v_pool), bt=t(c.block_tables), k_new=t(c.k_new),
                     v_new=t(c.v_new), slots=t(c.slot_mapping), case=c)
        if varlen:
            d["cu"], d["pos"] = t(c.cu_seqlens_q), t(c.pos_offsets)
            d["bytes"] = W.algorithmic_bytes_varlen(c)
        elif not qkv:
            d["cl"] = t(c.context_lens)
            # one new row per sequence for the fused step (rows of empty sequences are never written)
            kn = np.zeros((c.B, c.Hkv, c.D), np.float16)
            vn = np.zeros_like(kn)
            nz = np.nonzero(c.context_lens > 0)[0]
            kn[nz], vn[nz] = c.k_new, c.v_new
            d["k_new_all"], d["v_new_all"] = t(kn), t(vn)
            d["bytes"] = W.algorithmic_bytes(c, window)
        d["out"] = torch.empty_like(d["q"])
        if r == 0:
            host0 = c
        elif qkv:
            c.varlen.k_pool = c.varlen.v_pool = None
        else:
            c.k_pool = c.v_pool = None  # only set 0 stays on the host (for the CPU baseline)
        sets.append(d)
    torch.cuda.synchronize()
    c0 = sets[0]["case"]
    if varlen or qkv_only:
        plan = {"num_splits": splits, "note": "varlen: 0 = the library chooses from the grid size"}
    else:
        plan = pkv.plan_decode(c0.B, c0.Hq, c0.Hkv, c0.D, c0.BS, c0.M, num_splits=splits,
                               max_context_hint=window)  # a window bounds the rows a sequence attends
    log("plan: %s, %s" % (plan, pkv.version()))

    fused = step_is_fused(args.config, args.unfused)  # varlen / window steps: the append, then attention
    if args.graph:
        # prepared calls are bound to the stream current when they are made: make it the capture stream
        torch.cuda.set_stream(torch.cuda.Stream())
    # arguments marshalled once per rotation set (the binding's prepared calls): per-step Python marshalling would
    # otherwise outlast the kernel and leave the GPU idle between steps
    for d in sets:
        if not qkv:
            # the append alone, timed for the record (the fused step does it inside its launch)
            d["append_only"] = pkv.prepare_paged_kv_append(d["k_new"], d["v_new"], d["slots"], d["k_pool"],
                                                           d["v_pool"])
        if qkv:
            qc = d["qkv_case"]
            d["append"] = pkv.prepare_split_qkv_norm_rope_into_paged_cache_varlen(
                d["qkv"], d["qw"], d["kw"], d["cos"], d["sin"], d["k_pool"], d["v_pool"], d["bt"], d["cu"], d["pos"],
                qc.varlen.Hq, qc.eps, qc.qk_mode, d["q"])
            if qkv_only:
                d["call"] = d["append"]
            elif fused:  # one launch: q and the new K/V rows formed in the attention kernel's prologue
                d["call"] = pkv.prepare_decode_step_qkv(d["qkv"], d["qw"], d["kw"], d["cos"], d["sin"], d["k_pool"],
                                                        d["v_pool"], d["bt"], d["cl"], qc.varlen.Hq, qc.varlen.scale,
                                                        qc.eps, qc.qk_mode, d["q"], d["out"], num_splits=splits)
            else:
                d["call"] = pkv.prepare_paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cl"],
                                                               qc.varlen.scale, d["out"], num_splits=splits)
        elif fused and varlen:  # one launch: the attention workgroups write the new rows themselves
            d["call"] = pkv.prepare_paged_varlen_step(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                                      d["bt"], d["cu"], d["pos"], d["case"].scale,
                                                      int(d["case"].q_lens.max()), d["out"], num_splits=splits)
        elif fused and window:
            d["call"] = pkv.prepare_decode_step_window(d["q"], d["k_new_all"], d["v_new_all"], d["k_pool"],
                                                       d["v_pool"], d["bt"], d["cl"], d["case"].scale, window,
                                                       d["out"], num_splits=splits)
        elif fused:
            d["call"] = pkv.prepare_decode_step(d["q"], d["k_new_all"], d["v_new_all"], d["k_pool"], d["v_pool"],
                                                d["bt"], d["cl"], d["case"].scale, d["out"], num_splits=splits)
        elif window:
            d["append"] = pkv.prepare_paged_kv_append(d["k_new"], d["v_new"], d["slots"], d["k_pool"], d["v_pool"])
            d["call"] = pkv.prepare_paged_decode_attention_window(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cl"],
                                                                  d["case"].scale, d["out"], window,
                                                                  num_splits=splits)
        elif varlen:
            d["append"] = pkv.prepare_paged_kv_append(d["k_new"], d["v_new"], d["slots"], d["k_pool"], d["v_pool"])
            d["call"] = pkv.prepare_paged_varlen_attention(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cu"],
                                                           d["pos"], d["case"].scale, d["out"], num_splits=splits,
                                                           max_q_len=int(d["case"].q_lens.max()))
        else:
            d["append"] = pkv.prepare_paged_kv_append(d["k_new"], d["v_new"], d["slots"], d["k_pool"], d["v_pool"])
            d["call"] = pkv.prepare_paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cl"],
                                                           d["case"].scale, d["out"], num_splits=splits)

        # attention alone (the dominant launch when a step takes more than one)
        if varlen:
            d["attn"] = pkv.prepare_paged_varlen_attention(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cu"],
                                                           d["pos"], d["case"].scale, d["out"], num_splits=splits,
                                                           max_q_len=int(d["case"].q_lens.max()))
        elif window:
            d["attn"] = pkv.prepare_paged_decode_attention_window(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cl"],
                                                                  d["case"].scale, d["out"], window,
                                                                  num_splits=splits)
        elif not qkv_only:
            d["attn"] = pkv.prepare_paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["cl"],
                                                           d["case"].scale, d["out"], num_splits=splits)

    def step(d):
        if not fused and not qkv_only:
            d["append"]()
        d["call"]()

    if args.copy_calibration_mib > 0:
        n = int(args.copy_calibration_mib * (1 << 20)) // 2
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("ran the copy calibration kernel (%.0f MiB read + written) 10 times" % args.copy_calibration_mib)

    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    K = args.steps

    def timed_n(fn, n):
        """Milliseconds per iteration of n back-to-back calls of fn(i), between two events on the current stream."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    def timed(fn):
        return timed_n(fn, K)

    # No event inside a timed region: an event pair costs ~7 us of stream time here, more than a kernel's launch gap.
    # The step region gives value; when a step is one launch (the fused single-pass step) that launch's average
    # duration is the same region / K, otherwise a second region of K back-to-back attention calls gives it.
    one_launch = qkv_only or (fused and step_launch_count(c0, plan, splits, varlen, pkv.device_cu_count()) == 1)
    if args.graph:
        # 32 consecutive steps over the rotation sets captured once (the capture stream's workspace is sized by an
        # eager step on it first) and replayed; every replay rewrites the same new rows, so the state is stable.
        G = 32
        cap = torch.cuda.current_stream()
        for i in range(R):
            step(sets[i])
        cap.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(G):
                step(sets[i % R])
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        K = (K + G - 1) // G * G
        ms_per_step = timed(lambda i: graph.replay() if i % G == 0 else None)
        attn_ms = np.array([ms_per_step if one_launch else timed(lambda i: sets[i % R]["attn"]())])
        log("graph of %d steps, %d replays" % (G, K // G))
    else:
        ms_per_step = timed(lambda i: step(sets[i % R]))
        attn_ms = np.array([ms_per_step if one_launch else timed(lambda i: sets[i % R]["attn"]())])

    # Per-step spread: REPS regions of C back-to-back steps each (an event pair per region), median and p90 of
    # the per-step times.
    REPS = 20
    C = max(1, min(100, K // REPS))
    per_step = []
    if not args.graph:
        for rr in range(REPS):
            per_step.append(timed_n(lambda i: step(sets[(rr * C + i) % R]), C))
    spread = None
    if per_step:
        spread = {"median_ms": round(float(np.median(per_step)), 5),
                  "p90_ms": round(float(np.percentile(per_step, 90)), 5),
                  "regions": REPS, "steps_per_region": C}

    append_info = None
    if not qkv:
        ab = float(np.mean([d["bytes"]["append"] for d in sets]))
        app_ms = timed(lambda i: sets[i % R]["append_only"]())
        append_info = {"kernel": "append_kernel (pkv_paged_kv_append)", "ms": round(float(app_ms), 5),
                       "algorithmic_bytes": int(ab), "achieved_GBs": round(ab / (app_ms * 1e-3) / 1e9, 2),
                       "calls_per_s": round(1e3 / app_ms, 1),
                       "timing": "region of back-to-back append calls / calls"}
        log("append alone: %s" % append_info)

    qkv_info = None
    if qkv:
        # the QKV kernel on its own (for a fused step: what the step's prologue replaces)
        qkv_ms = ms_per_step if qkv_only else timed(lambda i: sets[i % R]["append"]())
        qb = float(np.mean([d["qkv_bytes"] for d in sets]))
        qkv_info = {"kernel": "qkv_cache_kernel (pkv_split_qkv_norm_rope_into_paged_cache_varlen)",
                    "ms": round(float(qkv_ms), 5), "algorithmic_bytes": int(qb),
                    "achieved_GBs": round(qb / (qkv_ms * 1e-3) / 1e9, 2),
                    "frac": round(qb / (qkv_ms * 1e-3) / 1e9 / PEAK_GBS, 4),
                    "timing": "step region / steps" if qkv_only else "region of back-to-back QKV-step calls / calls"}
        log("qkv step kernel: %s" % qkv_info)

    # bytes per step, averaged over the rotation sets
    step_bytes = np.mean([d["bytes"]["attention"] + d["bytes"]["append"] for d in sets])
    attn_bytes = np.mean([d["bytes"]["attention"] for d in sets])
    kernel_bytes = step_bytes if one_launch else attn_bytes  # algorithmic bytes of one dominant launch
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    attn_avg_ms = float(attn_ms.mean())
    achieved = kernel_bytes / (attn_avg_ms * 1e-3) / 1e9
    calls_per_s = 1e3 / attn_avg_ms
    log("step %.4f ms (%.1f GB/s); %s avg %.4f ms -> %.1f GB/s, %.0f calls/s"
        % (ms_per_step, value, "step launch" if one_launch else "attention call", attn_avg_ms, achieved, calls_per_s))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same workload for ~%.0f s" % args.cpu_seconds)
        cpu = (cpu_baseline_qkv(host0, args.cpu_seconds, not qkv_only) if qkv else
               cpu_baseline(host0, args.cpu_seconds, window))
        log("cpu baseline: %s" % cpu)

    result = {
        "metric": METRIC,
        "value": round(float(value), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(float(ms_per_step), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "%s: %s" % (args.config, desc),
            "num_seqs": c0.B, "num_q_heads": c0.Hq, "num_kv_heads": c0.Hkv, "head_dim": c0.D,
            "block_size": c0.BS, "num_splits": splits, "plan": plan, "rotations": R,
            "step": ("pkv_split_qkv_norm_rope_into_paged_cache_varlen" if qkv_only else
                     "fused (pkv_paged_decode_step_qkv)" if qkv and fused else
                     "pkv_split_qkv_norm_rope_into_paged_cache_varlen + pkv_paged_decode_attention" if qkv else
                     "fused (pkv_paged_varlen_step)" if fused and varlen else
                     "fused (pkv_paged_decode_step_window, window %d)" % window if fused and window else
                     "fused (pkv_paged_decode_step)" if fused else
                     "pkv_paged_kv_append + pkv_paged_varlen_attention" if varlen else
                     "pkv_paged_kv_append + pkv_paged_decode_attention_window (window %d)" % window if window else
                     "pkv_paged_kv_append + pkv_paged_decode_attention"),
            "parallelism": "single GPU",
            "launch": "HIP graph replay (32 steps per graph)" if args.graph else "eager launches",
        },
        "pct_of_peak": round(100.0 * float(value) / PEAK_GBS, 2),
        "calls_per_s": round(calls_per_s, 1),
        "tokens_per_s": round(calls_per_s * (c0.T if varlen or qkv else c0.B), 1),
        "kernel_ms": {"mean": round(attn_avg_ms, 5),
                      "timing": ("step region / steps (one launch per step)" if one_launch or qkv_only else
                                 "region of back-to-back attention calls / calls")},
        "bytes_per_step": {"attention": int(attn_bytes),
                           ("qkv_step" if qkv else "append"): int(np.mean([d["bytes"]["append"] for d in sets]))},
        "qkv_kernel": qkv_info,
        "append_kernel": append_info,
        "step_spread": spread,
        "roofline": {
            "bound": "hbm",
            "achieved": round(float(achieved), 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(float(achieved) / PEAK_GBS, 4),
            "traffic": measured_traffic(args.config, splits, fused),
        },
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
