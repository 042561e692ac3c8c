#!/usr/bin/env python
"""Benchmark of the transform-coded KV-cache hot path on one MI355X.

Headline workload (batched decode): B=64 sequences, H=8 KV heads, D=128, 8192
rows already stored per (b, h) through a frozen per-(b, h) basis (rank 96, DP
bit allocation at 320 bits/token from widths {0, 2, 4, 8}).  One step = append
one new K row and one new V row per (b, h) (fp64-MFMA project + quantise +
pack, one launch for both tensors) and fetch every stored K and V row back to
fp16 [B, H, S, D] (unpack + dequantise + fp16-MFMA reconstruct, one launch for
both tensors).  Inputs are resident in HBM
before the timed region.  ``value`` is fetched positions per second
(B * H * S per step, K and V of one position counted once).

Prints one JSON line.  ``roofline`` reports the fetch kernel (the dominant
launch, K and V together): algorithmic bytes per launch / mean launch time measured with HIP
events on the launch stream, against 8 TB/s.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same units.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fetch_batched_decode_pmc.txt")
# the sources that decide the fetch kernel's code and launch shape
FETCH_SRC = [os.path.join(ROOT, "kv_cache_compression_kvtc_amd", "csrc", f)
             for f in ("kvtc_device.h", "kvtc_fetch_kernel.h", "kvtc_fetch_ks.hip", "kvtc_device.hip")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # (about 25 ms of untimed steps: after the host-side set-up the first ~20 ms of
    # launches run up to 7% slower than the steady state)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads (long context, "
                   "group-head, Llama layer), which the default run also times")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a device copy of known size (for HBM counter scaling)")
    p.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                   help="write the HBM counter summary of the fetch kernel from four rocprofv3 --pmc "
                        "csv directories (FETCH_SIZE and WRITE_SIZE of this bench, then of --copy-calibration)")
    p.add_argument("--trace-summary", nargs=3, metavar=("STATS_CSV", "TITLE", "COMMAND"),
                   help="print a per-kernel table from a rocprofv3 --kernel-trace --stats kernel_stats.csv")
    p.add_argument("--counter-summary", nargs="+", metavar="ARG",
                   help="TITLE COMMAND DIR [DIR ...]: print a per-kernel table of the counters in the "
                        "counter_collection.csv of each rocprofv3 --pmc output directory")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the fetch kernel's sources: counters taken on other sources are not reported."""
    h = hashlib.sha256()
    for f in FETCH_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic():
    """HBM bytes per fetch launch from the committed counter summary, if it was
    taken on the current kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_fetch_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != source_hash():
        return None
    return float(m_val.group(1))


# ------------------------------------------------------------------ copy calibration
def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(3)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 5}))


def copy_ceiling_gbps(dev, reps=10):
    """Bytes moved per second (read + write) by a 1 GiB device-to-device copy in
    this process: the practical HBM ceiling the fetch is compared with."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(3)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbps


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {len(files)}")
    return list(csv.DictReader(open(files[0])))


def pmc_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """HBM bytes per fetch launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled so that the device copy of --copy-calibration reads and writes
    exactly its known size."""
    def per_kernel(rows, counter, match):
        return [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    is_fetch = lambda n: "fetch_kernel" in n
    is_copy = lambda n: "copyBuffer" in n or "copy" in n.lower()
    copy_kib = (1 << 30) / 1024
    cal_f = per_kernel(_counter_rows(cal_fetch_dir), "FETCH_SIZE", is_copy)
    cal_w = per_kernel(_counter_rows(cal_write_dir), "WRITE_SIZE", is_copy)
    f = per_kernel(_counter_rows(fetch_dir), "FETCH_SIZE", is_fetch)
    w = per_kernel(_counter_rows(write_dir), "WRITE_SIZE", is_fetch)
    if not (cal_f and cal_w and f and w):
        raise SystemExit("missing counter rows")
    sf = copy_kib / float(np.mean(cal_f))
    sw = copy_kib / float(np.mean(cal_w))
    read_b = float(np.mean(f)) * sf * 1024
    write_b = float(np.mean(w)) * sw * 1024
    lines = [
        "# HBM traffic of the fetch kernel, batched-decode workload (B=64, H=8, D=128, S~8195, r=96, 320 bits/token)",
        "commands (from /tmp with TMPDIR=/tmp; R is the repository root; each in a run of its own, csv output):",
        "  rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -o bd --output-format csv -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extra",
        "  rocprofv3 --pmc WRITE_SIZE -d <write_dir> -o bd --output-format csv -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extra",
        "  rocprofv3 --pmc FETCH_SIZE -d <cal_fetch_dir> -o cal --output-format csv -- python3 $R/bench.py --copy-calibration",
        "  rocprofv3 --pmc WRITE_SIZE -d <cal_write_dir> -o cal --output-format csv -- python3 $R/bench.py --copy-calibration",
        "  python3 $R/bench.py --pmc-summary <fetch_dir> <write_dir> <cal_fetch_dir> <cal_write_dir>",
        f"copy calibration (1 GiB device copy): FETCH_SIZE {np.mean(cal_f):.0f} KiB -> scale {sf:.4f}; "
        f"WRITE_SIZE {np.mean(cal_w):.0f} KiB -> scale {sw:.4f}",
        f"fetch dispatches: {len(f)} (FETCH_SIZE), {len(w)} (WRITE_SIZE); each covers the K and the V tensor",
        f"FETCH_SIZE mean {np.mean(f):.1f} KiB -> {read_b / 1e6:.2f} MB read per launch",
        f"WRITE_SIZE mean {np.mean(w):.1f} KiB -> {write_b / 1e6:.2f} MB written per launch",
        f"hbm_bytes_per_fetch_launch: {read_b + write_b:.6e}",
        f"kernel_source_sha256_16: {source_hash()}",
    ]
    return "\n".join(lines) + "\n"


def short_kernel(name):
    """A kernel's name without namespaces, argument lists or return type, template arguments kept."""
    m = re.match(r"_ZN4kvtc(?:12_GLOBAL__N_1)?(\d+)", name)
    if m:
        # rocprofv3 leaves some names mangled (binutils does not know the _Float16 code DF16_):
        # render kvtc::name<template arguments> from the mangled form
        n0 = int(m.group(1))
        base = name[m.end():m.end() + n0]
        rest = name[m.end() + n0:]
        args = []
        if rest.startswith("I"):
            for t in re.findall(r"Lb[01]|DF16_|Li-?\d+E|L[a-z]\d+E", rest[1:rest.find("EE") + 1]):
                args.append({"Lb0": "false", "Lb1": "true", "DF16_": "f16"}.get(t, re.sub(r"^L[a-z]|E$", "", t)))
        name = base + (f"<{', '.join(args)}>" if args else "")
    n = name.replace("(anonymous namespace)::", "")
    n = re.sub(r"\(.*$", "", n)
    n = n.replace("void ", "").replace("kvtc::", "")
    n = n.replace("_Float16", "f16")
    if "copyBuffer" in n or "copy" in n.lower():
        return "device copy (ceiling)"
    return n[:70]


def trace_summary(csv_path, title, command):
    """Per-kernel call count and durations from rocprofv3's kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    out = [title, "command (from /tmp with TMPDIR=/tmp; R is the repository root):", "  " + command,
           f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share_%':>8s}"]
    for r in rows:
        out.append(f"{short_kernel(r['Name']):70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                   f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):8.2f}")
    return "\n".join(out) + "\n"


def counter_summary(title, command, dirs):
    """Mean per dispatch of every counter, per kernel, over rocprofv3 --pmc output directories."""
    import collections
    agg = collections.defaultdict(list)
    counters = []
    for d in dirs:
        for r in _counter_rows(d):
            k = short_kernel(r["Kernel_Name"])
            agg[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
            if r["Counter_Name"] not in counters:
                counters.append(r["Counter_Name"])
    kernels = sorted({k for k, _ in agg})
    out = [title, "commands (from /tmp with TMPDIR=/tmp; R is the repository root; one pass per directory):",
           "  " + command, "mean per dispatch over the run's dispatches of each kernel", ""]
    for k in kernels:
        vals = [(c, agg.get((k, c))) for c in counters]
        out.append(k)
        for c, v in vals:
            if v:
                out.append(f"    {c:28s} {sum(v) / len(v):14.6g}   ({len(v)} dispatches)")
    return "\n".join(out) + "\n"


# ------------------------------------------------------------------ workloads
class TensorPath:
    """One tensor (K or V) of a workload on the device: blob, store, rows, output."""

    def __init__(self, K, w, tensor, s_fit, s_total, capacity, dev, x_host=None):
        import torch
        from kv_cache_compression_kvtc_amd import synth
        X = x_host if x_host is not None else synth.generate(w, tensor, 0, s_total)
        cfg = K.make_config(w.mode, w.D, w.heads_per_unit, w.rank, w.energy, w.budget, w.choices,
                            w.beta, w.hi_bits, w.lo_bits, w.group_size, w.hi_fraction)
        self.x = torch.from_numpy(X).to(dev)
        # the prefill fit runs on the device rows (kvtc_fit_device), timed from
        # the call to the returned host blob
        K.kvtc_fit_device(cfg, self.x[:1, :, :s_fit])       # first call: kernel set-up
        torch.cuda.synchronize()
        t = time.perf_counter()
        self.blob = K.kvtc_fit_device(cfg, self.x[:, :, :s_fit])
        self.fit_s = time.perf_counter() - t
        self.h = K.header(self.blob)
        self.K = K
        self.cap = capacity
        self.blob_dev = torch.from_numpy(self.blob).to(dev)
        cb, pb = K.kvtc_store_bytes(self.blob, capacity)
        self.codes = torch.zeros(max(cb, 4), dtype=torch.uint8, device=dev)
        self.params = torch.zeros(max(pb // 4, 1), dtype=torch.int32, device=dev) if pb else None
        self.out = torch.empty((w.B, w.H, capacity, w.D), dtype=torch.float16, device=dev)
        del X

    def append_ref(self):
        return (self.blob, self.blob_dev, self.x, self.codes, self.params)

    def fetch_ref(self):
        return (self.blob, self.blob_dev, self.codes, self.params, self.out)

    # algorithmic bytes: what the method has to move (inputs, codes, outputs, frozen state)
    def fetch_bytes(self, S):
        h = self.h
        per_pos = h.row_stride / h.heads_per_unit + 4 * h.n_qgroups / h.heads_per_unit + 2 * h.head_dim
        state = h.units * (h.dg * h.kslots * 2 + h.dg * 4 + h.kslots * 4)
        return h.batch * h.heads * S * per_pos + state

    def append_bytes(self, n, in_bytes=2):
        h = self.h
        per_pos = in_bytes * h.head_dim + h.row_stride / h.heads_per_unit + 4 * h.n_qgroups / h.heads_per_unit
        state = h.units * (h.kslots * h.dg * 4 + h.dg * 4 + h.kslots * 20)
        return h.batch * h.heads * n * per_pos + state


class KVLayer:
    """The key and value tensors of a workload, appended and fetched with the
    paired calls (one launch for both where their shapes allow); buffers are
    checked once and each timed call passes only its row range."""

    def __init__(self, K, w, s_fit, s_total, capacity, dev):
        from kv_cache_compression_kvtc_amd import synth
        self.paths = []
        for tensor in (synth.KEY, synth.VALUE):
            t = time.time()
            self.paths.append(TensorPath(K, w, tensor, s_fit, s_total, capacity, dev))
            log(f"setup tensor {tensor}: {time.time() - t:.1f}s (device fit {self.paths[-1].fit_s * 1e3:.1f} ms)")
        k, v = self.paths
        self.append = K.PreparedAppendKV(k.append_ref(), v.append_ref(), capacity)
        self.fetch = K.PreparedFetchKV(k.fetch_ref(), v.fetch_ref(), capacity)

    def fetch_bytes(self, S):
        return sum(p.fetch_bytes(S) for p in self.paths)

    def append_bytes(self, n):
        return sum(p.append_bytes(n) for p in self.paths)


def time_batched_decode(K, args, dev):
    import torch
    from kv_cache_compression_kvtc_amd import synth
    w = synth.WORKLOADS[4]
    S0 = w.s_prefill
    s_total = S0 + args.warmup + args.steps
    layer = KVLayer(K, w, S0, s_total, s_total, dev)
    layer.append(0, S0)                                    # rows already stored (untimed)
    torch.cuda.synchronize()

    def step(k, evs=None):
        s = S0 + k
        layer.append(s, s + 1)                             # one launch: K and V rows
        if evs is not None:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            layer.fetch(0, s + 1)                          # one launch: all K and V rows
            b.record()
            evs.append((a, b))
        else:
            layer.fetch(0, s + 1)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    evs = []
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for k in range(args.warmup, args.warmup + args.steps):
        step(k, evs)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    fetch_ms = [a.elapsed_time(b) for a, b in evs]
    sizes = [S0 + k + 1 for k in range(args.warmup, args.warmup + args.steps)]
    positions = sum(w.B * w.H * s for s in sizes)
    fetch_bytes = [layer.fetch_bytes(s) for s in sizes]
    append_bytes = layer.append_bytes(1) * args.steps
    h = layer.paths[0].h
    # the traffic-only probe on the last step's rows: same launch plan and bytes
    # as the fetch, no arithmetic (its output is placeholder values)
    S_last = sizes[-1]
    layer.fetch.probe(0, S_last)
    torch.cuda.synchronize()
    probe_ms = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        layer.fetch.probe(0, S_last)
        b.record()
        probe_ms.append((a, b))
    torch.cuda.synchronize()
    probe_ms = [a.elapsed_time(b) for a, b in probe_ms]
    probe = {"ms": float(np.mean(probe_ms)), "bytes": layer.fetch_bytes(S_last)}
    att = time_attend(K, layer, sizes[-1], dev)
    return dict(w=w, total_ms=total_ms, fetch_ms=fetch_ms, positions=positions,
                fetch_bytes=fetch_bytes, append_bytes=append_bytes, sizes=sizes, header=h, attend=att,
                probe=probe, fit_ms=[p.fit_s * 1e3 for p in layer.paths])


def time_attend(K, layer, S, dev, reps=20):
    """Decode attention from the codes (one query per (b, h)) over the same
    stored rows [0, S): what a decode step needs instead of the full fetch.
    Algorithmic bytes: both code stores' rows plus both fp32 bases once."""
    import torch
    k, v = layer.paths
    att = K.Attend((k.blob, k.blob_dev, k.codes, k.params), (v.blob, v.blob_dev, v.codes, v.params), k.cap)
    h = k.h
    q = torch.randn((h.batch, h.heads, h.head_dim), device=dev, dtype=torch.float16)
    out = att(q, S)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        att(q, S, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = sum(p.h.batch * p.h.heads * S * p.h.row_stride + p.h.units * p.h.kslots * p.h.dg * 4 for p in (k, v))
    return {"ms_per_call": round(ms, 4), "positions_per_s": round(h.batch * h.heads * S / (ms / 1e3), 1),
            "algorithmic_bytes": nbytes, "GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
            "launches": "one partial launch (one segment per unit; longer caches add a merge launch)"}


def time_one_shot(K, wid, dev, reps=10):
    """Other workloads: one-shot append of the rows after the fit prefix + full
    fetch, each kernel timed in a loop of its own (appending the same rows again
    stores the same codes), then the fetch's traffic-only probe."""
    import torch
    from kv_cache_compression_kvtc_amd import synth
    w = synth.WORKLOADS[wid]
    S = w.s_total
    layer = KVLayer(K, w, w.s_prefill, S, S, dev)
    a0 = 0 if w.s_prefill == S else w.s_prefill
    if a0:
        layer.append(0, a0)
    layer.append(a0, S)
    torch.cuda.synchronize()

    def med_ms(fn):
        fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            fn()
            e[1].record()
            evs.append(e)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in evs]))

    ap = med_ms(lambda: layer.append(a0, S))
    fe = med_ms(lambda: layer.fetch(0, S))
    pm = med_ms(lambda: layer.fetch.probe(0, S))
    fb = layer.fetch_bytes(S)
    ab = layer.append_bytes(S - a0)
    return {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "S": S, "append_rows": S - a0,
            "append_ms": round(ap, 4), "fetch_ms": round(fe, 4),
            "tokens_per_s": round(w.B * w.H * S / ((ap + fe) / 1e3), 1),
            "fetch_GBps": round(fb / fe / 1e6, 1), "append_GBps": round(ab / ap / 1e6, 1),
            "fetch_frac_hbm": round(fb / fe / 1e6 / PEAK_HBM_GBPS, 4),
            "probe_ms": round(pm, 4), "fetch_frac_of_probe": round(pm / fe, 4),
            "prefill_fit_ms": [round(p.fit_s * 1e3, 1) for p in layer.paths]}


def time_modes(K, dev, reps=5):
    """The other storage modes at the batched-decode shape (key tensor, 512 units,
    8192 stored rows): a refit-mode decode step (kvtc_append_refit of one row,
    which refits every range and re-packs all 8193 rows, then kvtc_fetch_refit
    of all rows) and the entropy-coded storage of the 8193 rows
    (kvtc_entropy_encode: device counts, host code tables, device encode; then
    kvtc_entropy_decode back into a code store).  Medians of reps calls."""
    import torch
    from kv_cache_compression_kvtc_amd import synth
    w = synth.WORKLOADS[4]
    S0, cap = w.s_prefill, w.s_prefill + 1
    p = TensorPath(K, w, synth.KEY, S0, cap, cap, dev)
    K.kvtc_append(p.blob, p.blob_dev, p.x, 0, p.codes, p.params, cap)
    rs = K.RefitStore(p.blob, p.blob_dev, cap)
    rs.append(p.x[:, :, :S0], 0)
    torch.cuda.synchronize()

    def med_ms(fn, sync=False):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            if sync:
                t = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t) * 1e3)
            else:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
                fn()
                e[1].record()
                torch.cuda.synchronize()
                ts.append(e[0].elapsed_time(e[1]))
        return float(np.median(ts))

    out = p.out[:, :, :cap]
    step = med_ms(lambda: rs.append(p.x[:, :, S0:cap], S0))
    fetch = med_ms(lambda: rs.fetch(0, cap, out))
    frozen_fetch = med_ms(lambda: K.kvtc_fetch(p.blob, p.blob_dev, p.codes, p.params, cap, 0, cap, out))
    arch = K.EntropyArchive(p.blob, p.blob_dev, p.codes, cap, cap)
    enc = med_ms(lambda: K.EntropyArchive(p.blob, p.blob_dev, p.codes, cap, cap), sync=True)
    codes2 = torch.zeros_like(p.codes)
    dec = med_ms(lambda: arch.decode(codes2, cap))
    same = bool(torch.equal(codes2, p.codes))
    h = p.h
    return {"workload": "batched-decode, key tensor: refit mode and entropy-coded storage",
            "units": h.units, "rows": cap,
            "refit_append_1_row_ms": round(step, 4),
            "refit_fetch_ms": round(fetch, 4), "frozen_fetch_ms": round(frozen_fetch, 4),
            "refit_latent_store_bytes": h.units * cap * h.kslots * 8,
            "entropy_encode_ms": round(enc, 3), "entropy_decode_ms": round(dec, 4),
            "entropy_archive_bytes": int(arch.header.archive_bytes),
            "fixed_width_bytes": int(h.units * cap * h.row_stride),
            "units_entropy_coded": int(arch.header.units_coded),
            "decode_round_trip_exact": same}


def time_decode_steps(K, dev, steps=64):
    """Llama-3-8B-like layer: prefill 4096, then per step append 1 + fetch all."""
    import torch
    from kv_cache_compression_kvtc_amd import synth
    w = synth.WORKLOADS[2]
    S0 = w.s_prefill
    cap = S0 + steps + 1
    layer = KVLayer(K, w, S0, cap, cap, dev)
    layer.append(0, S0)
    torch.cuda.synchronize()
    times = []
    for k in range(steps):
        s = S0 + k
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.append(s, s + 1)
        layer.fetch(0, s + 1)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    med = float(np.median(times[4:]))
    S = S0 + steps // 2
    return {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "S_mid": S, "steps": steps,
            "median_step_ms": round(med, 4),
            "tokens_per_s": round(w.B * w.H * S / (med / 1e3), 1),
            "note": "launch-latency bound: ~20 MB moved per step"}


# ------------------------------------------------------------------ CPU oracle baseline
def cpu_baseline(seconds):
    """The oracle, as it stands, on whole (b, h) units of the batched-decode workload:
    per unit and tensor, append the new row and fetch all rows.  Units are independent,
    so positions/s extrapolate linearly to the full batch."""
    from oracle import kvtc_oracle as O
    from kv_cache_compression_kvtc_amd import synth
    w = synth.WORKLOADS[4]
    S0 = w.s_prefill
    cfg = O.Config(mode="dp", head_dim=w.D, rank=w.rank, budget=w.budget, choices=w.choices)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rng = np.random.default_rng(7)
    order = rng.permutation(w.B * w.H)
    elapsed = 0.0
    positions = 0
    units = 0
    for unit in order:
        b, hh = divmod(int(unit), w.H)
        per_unit = 0.0
        for tensor in (synth.KEY, synth.VALUE):
            X = synth.unit_rows(w, tensor, b, hh, 0, S0 + 1).astype(np.float16)[None, None]
            st = O.fit(cfg, X[:, :, :S0])
            rows, _ = O.append(st, X[:, :, :S0])               # stored rows (setup)
            t = time.perf_counter()
            new, _ = O.append(st, X[:, :, S0:])
            allrows = np.concatenate([rows, new], axis=1)
            out = O.to_f16(O.fetch(st, allrows))
            per_unit += time.perf_counter() - t
        elapsed += per_unit
        positions += S0 + 1
        units += 1
        if elapsed >= seconds and units >= 4:
            break
    return {"value": round(positions / elapsed, 1), "unit": "tokens/s", "cores": int(threads),
            "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model,
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "kind": "oracle",
            "sample": f"{units} of {w.B * w.H} (b,h) units of the batched-decode workload, K and V: "
                      f"append 1 row + fetch {S0 + 1} rows each, numpy float64; "
                      f"{elapsed:.1f}s of CPU time, extrapolates linearly (units independent)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no "
              "cross-GPU exchange, see the sharding notes in the design document", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.pmc_summary:
        text = pmc_summary(*args.pmc_summary)
        with open(PMC_SUMMARY, "w") as fh:
            fh.write(text)
        print(text, end="")
        return
    if args.trace_summary:
        print(trace_summary(*args.trace_summary), end="")
        return
    if args.counter_summary:
        if len(args.counter_summary) < 3:
            raise SystemExit("--counter-summary TITLE COMMAND DIR [DIR ...]")
        print(counter_summary(args.counter_summary[0], args.counter_summary[1], args.counter_summary[2:]), end="")
        return
    from kv_cache_compression_kvtc_amd.build import ensure_current
    ensure_current(log=log)                                # never time a library built from other sources
    import torch
    from kv_cache_compression_kvtc_amd import kvtc as K
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")

    r = time_batched_decode(K, args, dev)
    w, h = r["w"], r["header"]
    torch.cuda.empty_cache()
    copy_gbps = copy_ceiling_gbps(dev)
    ms_per_step = r["total_ms"] / args.steps
    value = r["positions"] / (r["total_ms"] / 1e3)
    total_bytes = sum(r["fetch_bytes"]) + r["append_bytes"]
    fetch_mean_ms = float(np.mean(r["fetch_ms"]))
    fetch_bytes_mean = float(np.mean(r["fetch_bytes"]))
    achieved = fetch_bytes_mean / (fetch_mean_ms / 1e3) / 1e9
    out = {
        "metric": "fetch+append tokens/s and achieved HBM GB/s (% of peak) at B*H*S tokens",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "batched-decode", "B": w.B, "H": w.H, "D": w.D,
                   "S_stored": w.s_prefill, "S_fetched": [r["sizes"][0], r["sizes"][-1]],
                   "rank": w.rank, "bit_budget": w.budget, "bit_choices": list(w.choices),
                   "row_stride_bytes": h.row_stride, "step": "append 1 row/seq (K,V) + fetch all rows (K,V)",
                   "arithmetic": "fetch fp16 MFMA with fp32 accumulate; append fp64 MFMA",
                   "parallelism": "single GPU"},
        "hbm_GBps_step": round(total_bytes / (r["total_ms"] / 1e3) / 1e9, 1),
        "hbm_frac_step": round(total_bytes / (r["total_ms"] / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"kernel": "fetch_kernel<dp, 128 columns>, K and V in one launch", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": pmc_traffic(),
                     "copy_ceiling_GBps": round(copy_gbps, 1),
                     "frac_of_copy_ceiling": round(achieved / copy_gbps, 4),
                     "algorithmic_bytes_per_launch": round(fetch_bytes_mean),
                     "mean_launch_ms": round(fetch_mean_ms, 4),
                     "launches": len(r["fetch_ms"])},
    }
    a = r["attend"]
    out["attend_from_codes"] = dict(a, S=r["sizes"][-1], note="one query per (b, h); softmax attention over all "
                                    "stored K and V rows computed from the codes, no fp16 K/V written",
                                    fetch_ms_same_rows=round(float(np.mean(r["fetch_ms"][-2:])), 4))
    pr = r["probe"]
    probe_gbps = pr["bytes"] / (pr["ms"] / 1e3) / 1e9
    out["roofline"]["probe_ceiling_GBps"] = round(probe_gbps, 1)
    out["roofline"]["frac_of_probe_ceiling"] = round(achieved / probe_gbps, 4)
    out["roofline"]["probe"] = ("kvtc_fetch_kv_probe: the fetch's launch plan and bytes (W slices, code rows, "
                                f"whole output rows, NT stores), no arithmetic; {pr['ms']:.4f} ms at S={r['sizes'][-1]}")
    out["prefill_fit_ms"] = {"K": round(r["fit_ms"][0], 1), "V": round(r["fit_ms"][1], 1),
                             "call": "kvtc_fit_device, 512 units x 8192 rows, device moments and ranges, "
                                     "host eigensolve and DP"}
    if not args.no_extra:
        extra = []
        for fn in (lambda: time_one_shot(K, 5, dev), lambda: time_one_shot(K, 3, dev),
                   lambda: time_decode_steps(K, dev), lambda: time_modes(K, dev)):
            torch.cuda.empty_cache()
            extra.append(fn())
            log(json.dumps(extra[-1]))
        out["other_workloads"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
