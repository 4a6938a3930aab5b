#!/usr/bin/env python3
"""Benchmark of the exact EDT hot path on one MI355X.

One step = one complete transform (every pass of the path) of one synthetic
workload already resident in HBM.  The default workload is the 512^3 volume
with spacing (2.5, 1, 1) and distances + indices: the one configuration that
runs all three passes (axis-0 scan, middle-axis envelope, last-axis envelope
with the epilogue).  Prints ONE JSON line:

  value        whole-job throughput, Gpixel/s (elements per second / 1e9)
  roofline     the dominant kernel's algorithmic HBM bytes per launch / its mean
               duration (HIP events on the launch stream), against 8 TB/s; the
               measured HBM traffic of that kernel comes from the committed
               rocprofv3 counter summary (profiles/traffic_<config>.json) and is
               null when the kernel sources changed since it was taken
  cpu_baseline the CPU oracle (single thread) on a bounded sample of the same
               workload, same unit

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5]
                       [--no-cpu-baseline] [--check]
       python bench.py --probe-copy           (copy kernel for counter calibration)
       python bench.py --summarize-traffic FETCH WRITE COPY_FETCH COPY_WRITE --config c5
                       (rocprofv3 --pmc output directories -> profiles/traffic_<config>.json)
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EDT Gpixel/s at 1 GPU + achieved HBM GB/s fraction of peak"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s
DEFAULT_CONFIG = "c5"
SECOND_CONFIG = "c3"   # the other workload with an HBM target, timed beside the default
COPY_PROBE_BYTES = 1 << 30   # float32 elements read (and as many written) by the copy probe
# the sources of the EDT kernels and their launches (the counter summaries in
# profiles/ are keyed by their hash)
KERNEL_SOURCES = ("exact_euclidean_distance_amd/csrc/kernels.hip",
                  "exact_euclidean_distance_amd/csrc/envelope.h",
                  "exact_euclidean_distance_amd/csrc/kernels.h")

WORKLOADS = {
    "c1": "2D 512x512 uint8, background i.i.d. Bernoulli(0.01), isotropic; "
          "outputs int32 sqdist + float32 dist + int32 index",
    "c2a": "2D 4096x4096 uint8, foreground = union of 300 disks (r ~ U[8,400]); "
           "outputs sqdist + dist + index",
    "c2b": "2D 4096x4096 uint8, single background pixel; outputs sqdist + dist + index",
    "c3": "2D 16384x16384 uint8, background i.i.d. Bernoulli(1e-4), isotropic; "
          "outputs int32 sqdist + float32 dist",
    "c4": "3D batch 16 x 128^3 uint8, foreground = union of 5-20 ellipsoids per volume, "
          "isotropic; output float32 dist",
    "c5": "3D 512^3 uint8, background Bernoulli(1e-3) + 64-voxel background slab, "
          "sampling (2.5,1,1); outputs float32 dist + int32 index",
    "b2d": "batched 2D: 32 images of 1024x1024 uint8, background i.i.d. Bernoulli(0.01) "
           "per image, isotropic; outputs sqdist + dist + index (flat per image)",
}
WORKLOADS["nd4"] = ("4D 80^4 uint8 (any-rank path), background i.i.d. Bernoulli(1e-3), "
                    "sampling (2.5,1,1,1); outputs float32 dist + int32 index")
WORKLOADS["w40k"] = ("2D 256x40000 uint8 (rows past the LDS kernels, any-rank path), background "
                     "i.i.d. Bernoulli(1e-3), isotropic; outputs sqdist + dist + int32 index")
WORKLOADS["l4m"] = ("1D signal of 2^22 uint8 samples (one line longer than 65535, any-rank path), "
                    "background i.i.d. Bernoulli(1e-4); outputs float32 dist + int32 index")
WORKLOADS["v2048"] = ("3D 64x2048x2048 uint8 (a stack of 2048^2 slices), background i.i.d. "
                      "Bernoulli(1e-3), isotropic; output float32 dist")
for _n in (1024, 2048, 4096, 8192):
    for _pct in (1, 99):
        WORKLOADS[f"p1_{_n}_{_pct}"] = (
            f"2D {_n}x{_n} uint8, background i.i.d. Bernoulli({_pct / 100:g}) (PR-EDT's "
            f"workload, its Table 1), isotropic; output float32 dist")
OUTPUTS = {
    "c1": ("sqdist", "dist", "indices"),
    "c2a": ("sqdist", "dist", "indices"),
    "c2b": ("sqdist", "dist", "indices"),
    "c3": ("sqdist", "dist"),
    "c4": ("dist",),
    "c5": ("dist", "indices"),
    "b2d": ("sqdist", "dist", "indices"),
}
OUTPUTS.update({k: ("dist",) for k in WORKLOADS if k.startswith("p1_")})
OUTPUTS["v2048"] = ("dist",)
OUTPUTS["nd4"] = ("dist", "indices")
OUTPUTS["w40k"] = ("sqdist", "dist", "indices")
OUTPUTS["l4m"] = ("dist", "indices")
ND_CONFIGS = ("nd4", "w40k", "l4m")   # timed through edt_nd_u8 (any-rank entry point)


def algorithmic_bytes(kernel: str, shape, n_out: int) -> int:
    """Bytes a kernel must move through HBM by the per-element byte model:
    every input it needs read once and every output written once, at the
    narrowest exact width (mask 1 B, axis-0 coordinate 2 B, packed coordinate
    pair 4 B, each requested output 4 B; segment summaries 2 B each, and the
    64-bit background-row mask of each 64-row segment, 1 bit per element)."""
    n = int(np.prod(shape))
    if len(shape) == 2:
        n0, M, B = shape[0], shape[1], 1
    elif len(shape) == 3:             # a batch of 2-D images
        B, n0, M = shape
    else:
        B, n0, M = shape[0], shape[1], shape[2] * shape[3]
    nseg = (n0 + 63) // 64
    summ = B * nseg * M * 2 * 2          # first + last, uint16 each
    rows = B * nseg * M * 8              # background-row masks
    if kernel == "axis0_summary":
        return n + summ + rows
    if kernel == "axis0_scan":
        return 2 * summ
    if kernel == "axis0_resolve":
        return rows + summ + 2 * n
    if kernel == "envelope_rows_2d":
        return 2 * n + 4 * n * n_out
    if kernel == "envelope_cols_3d":
        return 2 * n + 4 * n
    if kernel == "envelope_rows_3d":
        return 4 * n + 4 * n * n_out
    if kernel == "proximate_rows_2d":
        # summaries and row bits read, outputs written, and each pixel's
        # upper answer (float64 + int32) written and read back
        return summ // 2 + rows + 4 * n * n_out + 2 * 12 * n
    raise KeyError(kernel)


def sources_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# rocprofv3 kernel names -> the names the timed entry points report
KERNEL_KEYS = (("k_axis0_summary", "axis0_summary"), ("k_axis0_scan", "axis0_scan"),
               ("k_axis0_resolve", "axis0_resolve"), ("k_envelope_cols", "envelope_cols_3d"),
               ("Geo3D", "envelope_rows_3d"), ("Geo2D", "envelope_rows_2d"))


def _kernel_key(name: str):
    for pat, key in KERNEL_KEYS:
        if pat in name:
            return key
    return None


def _pmc_per_dispatch(run_dir: str, counter: str):
    """Mean value of one counter per dispatch, per kernel, from a rocprofv3
    --pmc --output-format csv directory."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: float(np.mean(v)) for k, v in acc.items()}


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, config, check=None):
    """Write profiles/traffic_<config>.json: per-kernel HBM bytes per dispatch
    from FETCH_SIZE / WRITE_SIZE (KiB), each scaled by the same counter's
    reading for the copy probe divided by the bytes it is known to move.
    check: (fetch dir, write dir, bytes) of a second copy probe of another
    size, whose scale factors are recorded beside the first ones."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    cf = _pmc_per_dispatch(copy_fetch_dir, "FETCH_SIZE")
    cw = _pmc_per_dispatch(copy_write_dir, "WRITE_SIZE")
    # the copy probe is the largest dispatch of its run
    copy_fetch_kib = max(cf.values())
    copy_write_kib = max(cw.values())
    f_fetch = copy_fetch_kib * 1024.0 / COPY_PROBE_BYTES
    f_write = copy_write_kib * 1024.0 / COPY_PROBE_BYTES
    kernels = {}
    for name, kib in fetch.items():
        key = _kernel_key(name)
        if key is None:
            continue
        wkib = write.get(name, 0.0)
        kernels[key] = {
            "rocprof_name": name,
            "FETCH_SIZE_KiB": round(kib, 1), "WRITE_SIZE_KiB": round(wkib, 1),
            "hbm_bytes": int(kib * 1024.0 / f_fetch + wkib * 1024.0 / f_write),
        }
    out = {"config": config, "sources_sha256_16": sources_hash(),
           "copy_probe_bytes_each_way": COPY_PROBE_BYTES,
           "copy_probe_FETCH_SIZE_KiB": round(copy_fetch_kib, 1),
           "copy_probe_WRITE_SIZE_KiB": round(copy_write_kib, 1),
           "scale_fetch": round(f_fetch, 5), "scale_write": round(f_write, 5),
           "kernels": kernels}
    if check:
        nb = int(check[2])
        out["copy_probe_check"] = {
            "bytes_each_way": nb,
            "scale_fetch": round(max(_pmc_per_dispatch(check[0], "FETCH_SIZE").values()) * 1024.0 / nb, 5),
            "scale_write": round(max(_pmc_per_dispatch(check[1], "WRITE_SIZE").values()) * 1024.0 / nb, 5)}
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))
    return 0


COUNTER_PASSES = (
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR "
    "SQ_INSTS_VALU_CVT SQ_INSTS_VALU_FMA_F64",
    "SQ_ACTIVE_INST_LDS SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_WAVE_CYCLES "
    "SQ_BUSY_CYCLES SQ_INSTS_VALU_MUL_F64 SQ_INSTS_VALU_INT32",
    "VALUBusy VALUUtilization LDSBankConflict OccupancyPercent",
    "MeanOccupancyPerCU",
)


def summarize_counters(dirs, config):
    """Markdown table of rocprofv3 --pmc counters (one directory per pass of
    COUNTER_PASSES), per envelope kernel, averaged over its dispatches, with
    per-element figures (instructions per element are wave instructions x 64
    lanes / elements of the dispatch)."""
    from workloads import make_config
    mask, _, _ = make_config(config)
    n = int(np.prod(mask.shape))
    acc = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter_collection.csv under {d}")
        for path in files:
            with open(path) as fh:
                for r in csv.DictReader(fh):
                    key = _kernel_key(r["Kernel_Name"])
                    if key is None:
                        continue
                    acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    lines = [f"kernel | VALU/elem | SALU/elem | LDS/elem | VMEM rd+wr/elem | cvt/elem | "
             f"f64 fma+mul/elem | int32/elem | VALUBusy % | VALUUtil % | LDSBankConflict % | "
             f"LDS-issue wait / wave cycles | any wait / wave cycles | Occupancy % | "
             f"MeanOccupancyPerCU (waves)"]
    lines.append(" | ".join(["---"] * 15))
    for key in ("axis0_summary", "axis0_scan", "axis0_resolve", "envelope_cols_3d",
                "envelope_rows_3d", "envelope_rows_2d"):
        c = acc.get(key)
        if not c:
            continue
        m = {k: float(np.mean(v)) for k, v in c.items()}
        g = lambda k: m.get(k, float("nan"))  # noqa: E731
        per = lambda k: 64.0 * g(k) / n  # noqa: E731
        wc = g("SQ_WAVE_CYCLES")
        lines.append(" | ".join([
            key, f"{per('SQ_INSTS_VALU'):.1f}", f"{per('SQ_INSTS_SALU'):.1f}", f"{per('SQ_INSTS_LDS'):.1f}",
            f"{per('SQ_INSTS_VMEM_RD') + per('SQ_INSTS_VMEM_WR'):.2f}", f"{per('SQ_INSTS_VALU_CVT'):.1f}",
            f"{per('SQ_INSTS_VALU_FMA_F64') + per('SQ_INSTS_VALU_MUL_F64'):.1f}",
            f"{per('SQ_INSTS_VALU_INT32'):.1f}", f"{g('VALUBusy'):.1f}", f"{g('VALUUtilization'):.1f}",
            f"{g('LDSBankConflict'):.2f}", f"{g('SQ_WAIT_INST_LDS') / wc:.3f}", f"{g('SQ_WAIT_ANY') / wc:.3f}",
            f"{g('OccupancyPercent'):.1f}", f"{g('MeanOccupancyPerCU'):.2f}"]))
    print("\n".join(lines))
    return 0


def measured_traffic(config: str, kernel: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256_16") != sources_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes")


def probe_copy(nbytes: int = COPY_PROBE_BYTES):
    """A plain elementwise kernel of known size (reads and writes nbytes
    each) for calibrating FETCH_SIZE / WRITE_SIZE."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print("copy probe done", flush=True)
    return 0


def cpu_baseline(name, mask, sampling, budget_s=15.0):
    """Time the oracle (single thread, as written) on a bounded sample of the
    same workload: whole volumes for batched 3-D, whole 3-D volumes split into
    slabs of axis-0 planes otherwise, leading rows for 2-D; grown until about
    budget_s seconds of oracle time."""
    import oracle
    want_idx = "indices" in OUTPUTS[name]
    if mask.ndim == 2:
        rows = mask.shape[0]
        take = max(1, min(rows, 2_000_000 // mask.shape[1]))
        while True:
            sample = np.ascontiguousarray(mask[:take])
            if not (sample == 0).any():
                sample[0, 0] = 0
            t0 = time.perf_counter()
            oracle.edt(sample, sampling, features=want_idx)
            dt = time.perf_counter() - t0
            if dt >= budget_s / 4 or take == rows:
                break
            take = min(rows, int(take * max(2.0, budget_s / max(dt, 1e-3) * 0.8)))
        desc = f"oracle on rows [0,{take}) of the {mask.shape[0]}x{mask.shape[1]} mask"
    else:
        vols, D = mask.shape[0], mask.shape[1]
        if vols > 1:
            take = 1
            while True:
                sample = mask[:take]
                t0 = time.perf_counter()
                oracle.edt_batch(sample, sampling, features=want_idx)
                dt = time.perf_counter() - t0
                if dt >= budget_s / 4 or take == vols:
                    break
                take = min(vols, int(take * max(2.0, budget_s / max(dt, 1e-3) * 0.8)))
            desc = f"oracle on {take} of {vols} images of {mask.shape[1:]}"
        else:
            take = max(1, min(D, 8))
            while True:
                sample = np.ascontiguousarray(mask[0, :take])
                if not (sample == 0).any():
                    sample.reshape(-1)[0] = 0
                t0 = time.perf_counter()
                oracle.edt(sample, sampling, features=want_idx)
                dt = time.perf_counter() - t0
                if dt >= budget_s / 4 or take == D:
                    break
                take = min(D, int(take * max(2.0, budget_s / max(dt, 1e-3) * 0.8)))
            desc = (f"oracle on axis-0 planes [0,{take}) of the {mask.shape[1:]} volume "
                    f"(as its own volume)")
    n = sample.size
    return {"value": n / dt / 1e9, "unit": "Gpixel/s", "cores": 1, "kind": "oracle",
            "sample": desc + (", with indices" if want_idx else ""), "seconds": round(dt, 3),
            "cpu": host_info()["cpu_model"], "host_cpus": host_info()["usable_cpus"]}


FP64_PEAK_TFLOPS = 78.6   # MI355X vector fp64


# 32-bit integer VALU operations per second: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz (a wave64 instruction takes four cycles on a 16-lane SIMD)
INT32_VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def bench_brute(args):
    """Time the device brute force (every element against every background
    element of its image) on a workload; ALU-bound.  At unit spacing the
    integer kernel runs: per pair 2 integer operations per axis (|difference|,
    multiply-add) and 3 for the running minimum (compare, two selects),
    against the int32 VALU peak; otherwise 3 fp64 flops per axis and pair,
    against the fp64 vector peak."""
    import torch
    from exact_euclidean_distance_amd import edt_brute
    from workloads import make_config
    name = args.config
    mask_np, sampling, _ = make_config(name)
    batched = mask_np.ndim >= 3          # batches of images (and the volume workloads)
    imgs = mask_np if batched else mask_np[None]
    ndim = imgs.ndim - 1
    pairs = int(sum(int(m.size) * int((m == 0).sum()) for m in imgs))
    dev = torch.device("cuda:0")
    mask = torch.from_numpy(mask_np).to(dev)
    want = OUTPUTS[name]
    kw = dict(batched=batched, return_sqdist="sqdist" in want, return_indices="indices" in want,
              return_distances="dist" in want)
    for _ in range(args.warmup):
        edt_brute(mask, sampling, **kw)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(args.steps):
        edt_brute(mask, sampling, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(1, args.steps)
    integer = sampling is None or all(float(x) == 1.0 for x in sampling)
    if integer:
        rate = pairs * (2 * ndim + 3) / (ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(rate, 3), "peak": round(INT32_VALU_PEAK_TOPS, 2),
                "unit": "TOP/s (int32 VALU)", "frac": round(rate / INT32_VALU_PEAK_TOPS, 4), "traffic": None}
    else:
        rate = pairs * 3 * ndim / (ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(rate, 3), "peak": FP64_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(rate / FP64_PEAK_TFLOPS, 4), "traffic": None}
    line = {
        "metric": METRIC + " (device brute-force check, not the transform's path)",
        "value": round(mask_np.size / (ms * 1e-3) / 1e9, 4), "unit": "Gpixel/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32" if integer else "f64", "data": "synthetic",
        "config": {"workload": f"{name}: {WORKLOADS[name]}", "shape": list(mask_np.shape),
                   "path": "brute force", "pairs": pairs},
        "roofline": roof,
        "Gpairs_per_s": round(pairs / (ms * 1e-3) / 1e9, 2),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_nd(args):
    """Time the any-rank entry point (edt_nd_u8, Python ``edt``) on a shape
    that takes its workspace path.  Bytes: model A (mask in, outputs out) and
    the path's own model (per spatial axis the float64 distance and int64
    feature read and written once, 32 bytes per element, plus the mask and
    the outputs)."""
    import torch
    from exact_euclidean_distance_amd import alloc_workspace, edt
    from exact_euclidean_distance_amd import _lib
    from workloads import make_config
    name = args.config
    mask_np, sampling, _ = make_config(name)
    dev = torch.device("cuda:0")
    mask = torch.from_numpy(mask_np).to(dev)
    shape = tuple(mask.shape)
    n = int(np.prod(shape))
    want = OUTPUTS[name]
    idx_dt = torch.int32
    sq = torch.empty(shape, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.empty(shape, dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.empty(shape, dtype=idx_dt, device=dev) if "indices" in want else None
    import ctypes
    shp = (ctypes.c_int64 * len(shape))(*shape)
    strd = (ctypes.c_int64 * len(shape))(*mask.stride())
    ib = 8 if idx_dt == torch.int64 else 4
    ws = alloc_workspace(int(_lib.load().edt_nd_workspace_size(0, len(shape), shp, strd, ib)), dev)

    def step():
        edt(mask, sampling, sqdist=sq, dist=ds, indices=ix, return_distances=ds is not None,
            index_dtype=idx_dt, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    stream = torch.cuda.current_stream()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = ev[0].elapsed_time(ev[-1]) / max(1, args.steps)
    out_bytes = sum(4 if k != "indices" else ib for k in want)
    model_a = n * (1 + out_bytes)
    model_path = n * (1 + 32 * len(shape) + out_bytes)
    if args.check:
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from gpu_check import compare
        print(f"[bench] {name}: parity check against the oracle", file=sys.stderr, flush=True)
        ref, _ = oracle.edt(mask_np, sampling, features=False)
        compare(mask_np, sampling, ref, None if sq is None else sq.cpu().numpy(),
                None if ds is None else ds.cpu().numpy(),
                None if ix is None else ix.cpu().numpy())
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the oracle on leading slabs of the array (each its own image)
        take = 1
        while True:
            sample = np.ascontiguousarray(mask_np[:take])
            if not (sample == 0).any():
                sample.reshape(-1)[0] = 0
            t0 = time.perf_counter()
            oracle.edt(sample, sampling, features="indices" in want)
            dt = time.perf_counter() - t0
            if dt > 10.0 or take >= shape[0]:
                break
            take = min(shape[0], take * 2)
        cpu = {"value": sample.size / dt / 1e9, "unit": "Gpixel/s", "cores": 1, "kind": "oracle",
               "sample": f"oracle on the leading {take} of {shape[0]} slabs along axis 0 (as its own array)",
               "seconds": round(dt, 2), "cpu": host_info()["cpu_model"], "host_cpus": host_info()["usable_cpus"]}
    line = {
        "metric": METRIC + " (any-rank path)", "value": round(n / (ms * 1e-3) / 1e9, 3), "unit": "Gpixel/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"{name}: {WORKLOADS[name]}", "shape": list(shape),
                   "sampling": list(sampling) if sampling else None, "outputs": list(want), "path": "edt_nd_u8"},
        "gpu_ms": {"mean": round(ms, 4), "median": round(float(np.median(per_step)), 4),
                   "min": round(float(np.min(per_step)), 4)},
        "roofline": {"bound": "hbm", "kernel": "whole path", "achieved": round(model_path / (ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(model_path / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None},
        "path": {"model_A_bytes": model_a, "model_A_GBps": round(model_a / (ms * 1e-3) / 1e9, 1),
                 "path_model_bytes": model_path},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_chamfer(args, metric):
    """Time a chamfer transform, city-block ("taxicab") or chessboard (int32
    distances, plus indices when the workload times them), on a 2-D, batched
    2-D or 3-D workload.  Bytes of the path per element: mask 1 B, axis-0
    coordinate written and read 2 + 2 B, 4 B per output; 3-D adds the middle
    pass: taxicab reads the coordinate twice and writes, reads back and
    rewrites its packed owners, which the row pass reads (2 + 2 + 4 + 4 + 4 B,
    as counted here), chessboard writes the owners once and the row pass reads
    them (4 + 4 B)."""
    import torch
    import exact_euclidean_distance_amd as pkg
    from workloads import make_config
    fn = getattr(pkg, metric)
    name = args.config
    mask_np, _, _ = make_config(name)
    dev = torch.device("cuda:0")
    mask = torch.from_numpy(mask_np).to(dev)
    want_idx = "indices" in OUTPUTS[name]
    r = fn(mask, return_indices=want_idx)
    for _ in range(args.warmup):
        fn(mask, return_indices=want_idx, dist=r.dist, indices=r.indices)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(args.steps):
        fn(mask, return_indices=want_idx, dist=r.dist, indices=r.indices)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(1, args.steps)
    n = mask_np.size
    mid = (16 if metric == "taxicab" else 8) if mask_np.ndim == 4 else 0
    per = 1 + 4 + mid + 4 * (2 if want_idx else 1)
    gbs = n * per / (ms * 1e-3) / 1e9
    title = {"taxicab": "city-block (taxicab)", "chessboard": "chessboard (L-infinity)"}[metric]
    line = {
        "metric": f"{title} transform Gpixel/s at 1 GPU (adjacent operator, not the EDT)",
        "value": round(n / (ms * 1e-3) / 1e9, 3), "unit": "Gpixel/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": f"{name}: {WORKLOADS[name]}", "shape": list(mask_np.shape),
                   "outputs": ["dist"] + (["indices"] if want_idx else [])},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "note": "whole path, bytes per element as in the docstring"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second", action="store_true",
                    help="with the default workload, skip the 16384^2 sub-record")
    ap.add_argument("--check", action="store_true", help="also compare with the oracle")
    ap.add_argument("--brute", action="store_true",
                    help="time the device brute-force transform (the exactness check) instead")
    ap.add_argument("--taxicab", action="store_true",
                    help="time the city-block (L1) transform on the workload instead")
    ap.add_argument("--chessboard", action="store_true",
                    help="time the chessboard (L-infinity) transform on the workload instead")
    ap.add_argument("--method", default="separable", choices=("separable", "proximate"),
                    help="2-D row pass: the separable envelope (default) or PR-EDT's "
                         "row-recursive proximate-point sets")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph holding one transform (launch gaps removed)")
    ap.add_argument("--probe-copy", action="store_true")
    ap.add_argument("--probe-bytes", type=int, default=COPY_PROBE_BYTES,
                    help="bytes read (and written) by --probe-copy")
    ap.add_argument("--summarize-traffic", nargs=4, metavar="DIR")
    ap.add_argument("--copy-check", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BYTES"),
                    help="with --summarize-traffic: a second copy probe of another size")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc directories (the COUNTER_PASSES) -> markdown table")
    args = ap.parse_args(argv)

    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, args.config, args.copy_check)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.config)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the transform of one workload runs "
              "on a single MI355X); run with --gpus 1", file=sys.stderr)
        return 2

    if args.probe_copy:
        return probe_copy(args.probe_bytes)

    import torch

    if args.brute:
        return bench_brute(args)
    if args.config in ND_CONFIGS:
        return bench_nd(args)
    if args.taxicab:
        return bench_chamfer(args, "taxicab")
    if args.chessboard:
        return bench_chamfer(args, "chessboard")

    if not torch.cuda.is_available():
        print("bench.py: no HIP device", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    copy_gbs = measure_copy_bandwidth(dev)
    rec = bench_workload(args.config, args, dev, copy_gbs)
    line = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "Gpixel/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "gpu_ms": rec["gpu_ms"],
        "path": rec["path"],
        "kernels": rec["kernels"],
        "cpu_baseline": rec["cpu_baseline"],
        "copy_GBps": round(copy_gbs, 1),
        "host": host_info(),
    }
    # the other configuration the HBM target is set on, timed in the same run
    if args.config == DEFAULT_CONFIG and not args.no_second:
        sub = bench_workload(SECOND_CONFIG, args, dev, copy_gbs)
        line[SECOND_CONFIG] = {k: sub[k] for k in ("value", "ms_per_step", "gpu_ms", "config",
                                                   "roofline", "path", "kernels", "cpu_baseline",
                                                   "dtype")}
    print(json.dumps(line), flush=True)
    return 0


def host_info():
    """CPU model and core counts of the host the oracle baseline ran on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def measure_copy_bandwidth(dev, nbytes=1 << 31, reps=10):
    """Device-to-device copy rate (GB/s, bytes read + written) of a plain
    elementwise copy of `nbytes`: the practical ceiling the HBM fraction is
    also reported against."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def bench_workload(name, args, dev, copy_gbs):
    """Time K transforms of one workload resident in HBM (after W warm-ups):
    the whole-path rate, per-step median and minimum, per-kernel durations
    from HIP events on the launch stream, the dominant kernel's roofline, and
    the oracle baseline on the host."""
    import torch
    from exact_euclidean_distance_amd import alloc_workspace, edt2d, edt3d, workspace_size_2d_batched, \
        workspace_size_3d
    from workloads import make_config

    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    mask_np, sampling, _ = make_config(name)
    shape = mask_np.shape
    n = int(np.prod(shape))
    want = OUTPUTS[name]
    mask = torch.from_numpy(mask_np).to(dev)
    sq = torch.empty(shape, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.empty(shape, dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.empty(shape, dtype=torch.int32, device=dev) if "indices" in want else None
    method = getattr(args, "method", "separable")
    if len(shape) in (2, 3):
        if method == "proximate":
            from exact_euclidean_distance_amd import _lib
            ws = alloc_workspace(int(_lib.load().edt2d_proximate_workspace_size(*((1,) + shape)[-3:])), dev)
            fn = lambda *a, **k: edt2d(*a, method="proximate", **k)   # noqa: E731
        else:
            ws = alloc_workspace(workspace_size_2d_batched(*((1,) + shape)[-3:]), dev)
            fn = edt2d
    else:
        ws = alloc_workspace(workspace_size_3d(*shape), dev)
        fn = edt3d
    stream = torch.cuda.current_stream()

    def step(timed=False, s=stream):
        return fn(mask, sampling, sqdist=sq, dist=ds, indices=ix, return_distances=ds is not None,
                  workspace=ws, stream=s, timed=timed)

    print(f"[bench] {name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graph = None
    if args.graph:   # one transform captured once; each timed step is one replay
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(s=torch.cuda.current_stream())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    print(f"[bench] {name}: timing {args.steps} steps", file=sys.stderr, flush=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = ev[0].elapsed_time(ev[-1]) / max(1, args.steps)

    # per-kernel durations: HIP events recorded by the library around each
    # launch, on the stream the kernels run on
    per = {}
    for _ in range(max(3, args.steps)):
        _, times = step(timed=True)
        for k, t in times:
            per.setdefault(k, []).append(t)
    kernels = []
    n_out = len(want)
    for k, ts in per.items():
        avg = float(np.mean(ts))
        b = algorithmic_bytes(k, shape, n_out)
        kernels.append({"name": k, "ms": round(avg, 4), "ms_min": round(float(np.min(ts)), 4),
                        "alg_bytes": b, "GBps": round(b / (avg * 1e-3) / 1e9, 1)})
    dom = max(kernels, key=lambda r: r["ms"])
    achieved = dom["alg_bytes"] / (dom["ms"] * 1e-3) / 1e9

    if args.check:
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from gpu_check import compare
        print(f"[bench] {name}: parity check against the oracle", file=sys.stderr, flush=True)
        if len(shape) == 2:
            ref, _ = oracle.edt(mask_np, sampling, features=False)
        else:
            ref, _ = oracle.edt_batch(mask_np, sampling, features=False)
        compare(mask_np, sampling, ref,
                None if sq is None else sq.cpu().numpy(),
                None if ds is None else ds.cpu().numpy(),
                None if ix is None else ix.cpu().numpy(), batch=(len(shape) > 2))

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] {name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(name, mask_np, sampling)

    model_b = sum(k["alg_bytes"] for k in kernels)
    model_a = n * (1 + 4 * n_out)
    path_b = model_b / (ms * 1e-3) / 1e9
    path_a = model_a / (ms * 1e-3) / 1e9
    traffic = measured_traffic(name, dom["name"])
    del mask, sq, ds, ix, ws
    torch.cuda.empty_cache()
    return {
        "value": round(n / (ms * 1e-3) / 1e9, 3),
        "ms_per_step": round(ms, 4),
        "gpu_ms": {"mean": round(ms, 4), "median": round(float(np.median(per_step)), 4),
                   "min": round(float(np.min(per_step)), 4)},
        "dtype": "f64",
        "config": {"workload": f"{name}: {WORKLOADS[name]}", "shape": list(shape),
                   "sampling": list(sampling) if sampling else None, "outputs": list(want),
                   "launch": "graph" if graph is not None else "stream",
                   "row_pass": method if len(shape) in (2, 3) else "separable"},
        "roofline": {"bound": "hbm", "kernel": dom["name"], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "path": {"model_B_bytes": model_b, "model_B_GBps": round(path_b, 1),
                 "model_B_frac": round(path_b / HBM_PEAK_GBS, 4),
                 "model_B_frac_of_copy": round(path_b / copy_gbs, 4),
                 "model_A_bytes": model_a, "model_A_GBps": round(path_a, 1),
                 "model_A_frac": round(path_a / HBM_PEAK_GBS, 4)},
        "kernels": kernels,
        "cpu_baseline": cpu,
    }


if __name__ == "__main__":
    sys.exit(main())
