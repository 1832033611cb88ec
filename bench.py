#!/usr/bin/env python3
"""Benchmark of the paged decode hot path (KV slot write + paged attention) on
one MI355X.

A step is one pass of the whole path over one batch: write every sequence's
new token into the paged KV cache through its slot (pa_cache_write), run
attention over every partition (pa_decode_partitions) and merge the
partitions (pa_decode_merge).  Inputs are seeded synthetic tensors already
resident in HBM; the timed region holds exactly K steps bracketed by
synchronisation.  Prints one JSON line:

  value          KV bytes the step's attention must read (each context element
                 once) / wall time per step, in GB/s
  roofline       the partitioned attention kernel: algorithmic KV bytes per
                 launch / its mean launch time (HIP events on the launch
                 stream) against the 8 TB/s HBM3E peak; `traffic` is the HBM
                 bytes per launch from the committed rocprofv3 counter summary
                 when it was taken on the current kernel source, else null
  cpu_baseline   the fp64 CPU oracle timed on this host on the same step

Usage: python bench.py [--steps K] [--warmup W] [--workload N]
Only one GPU is used; --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published
KERNEL_SOURCES = ["decode_valu.hip", "decode_mfma.hip", "decode_order.hip", "work_list.hpp",
                  "pa_device.hpp", "pa_launch.hpp", "pa_api.cpp", "../build.py"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{workload}.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        p = os.path.join(ROOT, "pagedattention_kv_cache_amd", "csrc", name)
        if os.path.exists(p):
            h.update(name.encode())
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed counter summary of this
    workload, or None where there is none or it was taken on other kernel sources."""
    tf = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(tf):
        return None
    with open(tf) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes")


def side_bytes(wl, queries: int = 1) -> dict:
    """Bytes a decode step moves besides the KV stream, which alone is the
    algorithmic figure: the queries, the fp32 outputs, the block-table entries and
    context lengths the decode reads, and the cache write of one new token per
    sequence (its rows read, the cache bytes written)."""
    import numpy as np

    from pagedattention_kv_cache_amd.workloads import DTYPE_BYTES
    c = wl.cfg
    lens = np.asarray(wl.context_lens(0), dtype=np.int64)
    rows = c.num_seqs * queries * c.num_q_heads
    new = c.num_seqs * c.num_kv_heads * c.head_dim * 2
    return {"q": rows * c.head_dim * DTYPE_BYTES[c.dtype],
            "out_f32": rows * c.head_dim * 4,
            "block_tables": int(((lens + c.block_size - 1) // c.block_size).sum()) * 4,
            "context_lens": 4 * c.num_seqs,
            "cache_write_read": new * DTYPE_BYTES[c.dtype],
            "cache_write_written": new * DTYPE_BYTES[c.kv_dtype]}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="decode workload 1..5 (default 4)")
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="-1: the workload's setting (0 = library picks)")
    ap.add_argument("--flags", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--waves", type=int, choices=[0, 1, 2, 4], default=0,
                    help="waves per decode work item (0: library picks)")
    ap.add_argument("--kv-cache", choices=["native", "fp8"], default="native",
                    help="fp8: the workload's E4M3-cache variant (workloads 4 and 5)")
    ap.add_argument("--queries", type=int, default=1,
                    help="query tokens per sequence (several: multi-query decode, as when draft "
                         "tokens are verified; the oracle baseline is then skipped)")
    ap.add_argument("--separate-write", action="store_true",
                    help="a step as pa_cache_write, then pa_decode_partitions (which orders the "
                         "items itself on the sorted grid), then the merge; default: "
                         "pa_decode_order (the write and the item order in one launch), then "
                         "pa_decode_partitions with PA_DECODE_ORDERED (the decode kernel alone), "
                         "then the merge")
    ap.add_argument("--fused-step", action="store_true",
                    help="one pa_decode_step call for write + decode partitions (its cache write "
                         "shares the launch that orders the decode's items); default: separate "
                         "pa_cache_write and pa_decode_partitions calls, timed one by one")
    ap.add_argument("--grid", choices=["auto", "grid", "sorted", "work_list"], default="auto",
                    help="how workgroups find their items (default: the library's choice)")
    ap.add_argument("--no-work-list", action="store_true",
                    help="one workgroup per possible decode item instead of the persistent grid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0, help="0: min(16, host cores)")
    ap.add_argument("--layers", type=int, default=4,
                    help="KV-cache copies the steps rotate over, so no step re-reads what the "
                         "previous one left in the 256 MB Infinity Cache")
    ap.add_argument("--no-stream-probe", action="store_true")
    ap.add_argument("--no-size-probe", action="store_true",
                    help="skip the streaming read of one launch's KV bytes")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step(s) captured in HIP graphs (multi-step "
                         "workloads: state advanced on the device by pa_advance_step)")
    ap.add_argument("--one-pass-ratio", action="store_true",
                    help="also time the whole decode (partitions + merge) of the same steps in "
                         "one pass per (sequence, kv head) -- the partition as long as the "
                         "longest context -- against the partitioned launch, interleaved, and "
                         "report the ratio")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="post-process two rocprofv3 --pmc counter CSVs into profiles/ (no GPU)")
    ap.add_argument("--pmc-copy-mib", type=int, default=1024)
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="post-process a rocprofv3 kernel trace of this workload into profiles/ "
                         "(no GPU)")
    ap.add_argument("--bench-json", metavar="FILE",
                    help="with --summarize-trace: a file whose last line is a bench JSON line")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------- counters

def _read_counter_rows(path):
    """rocprofv3 counter CSV -> [(kernel name, grid size, counter, value)], one row per
    (dispatch, counter)."""
    import csv
    out = []
    for r in csv.DictReader(open(path)):
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("KernelName") or ""
        cname = r.get("Counter_Name") or r.get("Counter-Name") or ""
        val = float(r.get("Counter_Value") or r.get("Counter-Value") or 0.0)
        grid = int(float(r.get("Grid_Size") or r.get("Grid_Size_X") or 0))
        out.append((name, grid, cname, val, int(r.get("Dispatch_Id") or 0)))
    return out


def _probe_copy_value(rows, counter):
    """The counter of the calibration copy: the run's first device-to-device copy
    dispatch (bench.py --copy-probe issues it before anything else)."""
    copies = sorted((d, v) for (k, g, c, v, d) in rows
                    if c == counter and "copyBuffer" in k)
    return copies[0][1]


def _is_decode(k):
    return "decode_valu_kernel" in k or "decode_mfma_kernel" in k


def _is_write(k):
    return "cache_write_kernel" in k or "cache_write_fp8_kernel" in k


def _is_prologue(k):
    return "decode_prologue" in k


def _step_values(rows, counter, pred):
    """Counter values of the dispatches of kernels matching pred at their most
    frequent grid size: the per-step launches (the set-up's bulk writes of the
    prior context use other grid sizes)."""
    import collections
    sel = [(g, v) for (k, g, c, v, _) in rows if c == counter and pred(k)]
    if not sel:
        return []
    grid = collections.Counter(g for g, _ in sel).most_common(1)[0][0]
    return [v for g, v in sel if g == grid]


def _workload_cfg(args):
    from pagedattention_kv_cache_amd.workloads import WORKLOADS, FP8_WORKLOADS
    return FP8_WORKLOADS[args.workload] if args.kv_cache == "fp8" else WORKLOADS[args.workload]


def summarize_pmc(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the decode kernel and of the
    per-step cache write, scaled by what the same counters read for a plain
    device copy of known size."""
    from pagedattention_kv_cache_amd.workloads import DTYPE_BYTES, Workload
    fetch = _read_counter_rows(args.summarize_pmc[0])
    write = _read_counter_rows(args.summarize_pmc[1])
    copy_bytes = args.pmc_copy_mib * 2**20
    copy_f = _probe_copy_value(fetch, "FETCH_SIZE")
    copy_w = _probe_copy_value(write, "WRITE_SIZE")
    f_scale = copy_bytes / (copy_f * 1024.0)
    w_scale = copy_bytes / (copy_w * 1024.0)
    dec_f = statistics.median(_step_values(fetch, "FETCH_SIZE", _is_decode))
    dec_w = statistics.median(_step_values(write, "WRITE_SIZE", _is_decode))
    cfg = _workload_cfg(args)
    wl = Workload(cfg)
    res = {
        "workload": cfg.name,
        "kernel_source_hash": kernel_source_hash(),
        "copy_probe_bytes": copy_bytes,
        "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "decode_fetch_kib": dec_f, "decode_write_kib": dec_w,
        "decode_fetch_bytes": dec_f * 1024.0 * f_scale,
        "decode_write_bytes": dec_w * 1024.0 * w_scale,
        "algorithmic_kv_bytes": wl.kv_bytes(0),
    }
    res["traffic_bytes"] = res["decode_fetch_bytes"] + res["decode_write_bytes"]
    res["fetch_over_algorithmic"] = res["decode_fetch_bytes"] / res["algorithmic_kv_bytes"]
    # the step's cache write: its own kernel where it launches every step (the
    # separate-write form, E4M3), else the launch that writes and orders the
    # items (the default step form; its order traffic is a few KiB)
    n_dec = len(_step_values(fetch, "FETCH_SIZE", _is_decode))
    write_kernel = _is_write
    if len(_step_values(fetch, "FETCH_SIZE", _is_write)) < n_dec:
        write_kernel = _is_prologue
    wf = _step_values(fetch, "FETCH_SIZE", write_kernel)
    ww = _step_values(write, "WRITE_SIZE", write_kernel)
    if wf and ww:
        # the step's new K and V rows, read once and written once
        new_kv = cfg.num_seqs * cfg.num_kv_heads * cfg.head_dim * 2
        res["cache_write"] = {
            "source_bytes": new_kv * DTYPE_BYTES[cfg.dtype],
            "cache_bytes": new_kv * DTYPE_BYTES[cfg.kv_dtype],
            "fetch_bytes": statistics.median(wf) * 1024.0 * f_scale,
            "write_bytes": statistics.median(ww) * 1024.0 * w_scale,
        }
        cw = res["cache_write"]
        cw["kernel"] = "decode_prologue (write + order)" if write_kernel is _is_prologue else \
            "cache_write_kernel"
        cw["write_over_cache_bytes"] = cw["write_bytes"] / cw["cache_bytes"]
    path = TRAFFIC_FILE.format(workload=cfg.name)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))
    return res


def summarize_trace(args):
    """profiles/<decode kernel>_<workload>.md from a rocprofv3 kernel trace of
    `bench.py --workload N [--kv-cache fp8]`, the counter summary of the same
    workload (profiles/traffic_<workload>.json, when taken on the current kernel
    sources) and the JSON line of a plain benchmark run (--bench-json)."""
    import collections
    import csv

    from pagedattention_kv_cache_amd.workloads import Workload
    cfg = _workload_cfg(args)
    wl = Workload(cfg)
    disp = collections.defaultdict(list)
    for r in csv.DictReader(open(args.summarize_trace)):
        name = r["Kernel_Name"]
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0) * \
            int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        disp[name].append((grid, dur))
    rows = []
    for name, ds in disp.items():
        if not any(tag in name for tag in ("decode_", "cache_write", "advance_step")):
            continue
        grid = collections.Counter(g for g, _ in ds).most_common(1)[0][0]
        d = [x for g, x in ds if g == grid]
        rows.append((name, len(d), statistics.mean(d), statistics.median(d), min(d), max(d)))
    rows.sort(key=lambda r: -r[1] * r[2])
    dec = [r for r in rows if _is_decode(r[0])]
    kname = dec[0][0].split("<")[0].split("::")[-1].replace("void ", "") if dec else "decode"
    kv = wl.kv_bytes(0) if cfg.steps == 1 else statistics.mean(wl.kv_bytes(s)
                                                             for s in range(cfg.steps))
    lines = [f"# {kname} -- {cfg.name}", ""]
    d = wl.describe()
    lines.append(f"Workload: {cfg.num_seqs} sequences, {cfg.num_q_heads}/{cfg.num_kv_heads} q/kv "
                 f"heads, head_dim {cfg.head_dim}, {cfg.kv_dtype} KV, block_size {cfg.block_size}, "
                 f"mean context {d['ctx_mean']:.0f} (max {d['ctx_max']}), {cfg.steps} step(s); "
                 f"{kv:.0f} algorithmic KV bytes per decode launch.")
    flags = f" --kv-cache {args.kv_cache}" if args.kv_cache != "native" else ""
    lines += ["", "## Kernel trace", "", "```",
              f"rocprofv3 --kernel-trace --stats -d <out>/trace -o trace --output-format csv -- \\",
              f"    python3 bench.py --workload {args.workload}{flags} --steps 20 --warmup 2 "
              f"--no-cpu-baseline --no-stream-probe",
              f"python3 bench.py --workload {args.workload}{flags} --summarize-trace "
              f"<out>/trace/trace_kernel_trace.csv --bench-json <bench line file>", "```", "",
              "Per-step launches only (each kernel's most frequent grid size; the set-up's bulk "
              "prefix writes are left out):", "",
              "| kernel | launches | mean (us) | median (us) | min (us) | max (us) |",
              "|---|---|---|---|---|---|"]
    for name, n, mean, med, lo, hi in rows:
        lines.append(f"| `{name.replace('void ', '').replace('(anonymous namespace)::', '')}` "
                     f"| {n} | {mean:.1f} | {med:.1f} | {lo:.1f} | {hi:.1f} |")
    if dec:
        mean = dec[0][2]
        lines += ["", f"Decode kernel: {kv:.0f} B / {mean:.1f} us = **{kv / mean / 1e3:.0f} GB/s, "
                  f"{kv / mean / 1e3 / HBM_PEAK_GBPS:.1%} of 8 TB/s** (rocprofv3 mean)."]
        probe = [(name, ds) for name, ds in disp.items() if "stream_read_kernel" in name]
        if probe:
            # the bench's size-matched probe: one plain streaming read of the
            # decode launch's bytes per launch, at a few grid sizes
            by_grid = collections.defaultdict(list)
            for g, x in probe[0][1]:
                by_grid[g].append(x)
            best_g, best = min(((g, statistics.mean(x)) for g, x in by_grid.items()),
                               key=lambda t: t[1])
            lines.append(
                f"The same run's size-matched streaming read (a plain read of the same bytes in "
                f"one launch, rotating over the cache copies; {len(probe[0][1])} launches over "
                f"{len(by_grid)} grid sizes): best mean {best:.1f} us at {best_g // 256} "
                f"workgroups = {kv / best / 1e3:.0f} GB/s ({kv / best / 1e3 / HBM_PEAK_GBPS:.1%} "
                f"of 8 TB/s); the decode kernel runs at {best / mean:.1%} of its rate.")
    tf = TRAFFIC_FILE.format(workload=cfg.name)
    if os.path.exists(tf):
        t = json.load(open(tf))
        t.setdefault("algorithmic_kv_bytes", wl.kv_bytes(0))
        stamp = "matches" if t.get("kernel_source_hash") == kernel_source_hash() else \
            "does NOT match"
        lines += ["", "## HBM traffic (rocprofv3 --pmc)", "", "```"]
        for ctr, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            lines.append(f"rocprofv3 --pmc {ctr} -d <out>/pmc_{tag} -o {tag} --output-format csv -- "
                         f"\\")
            lines.append(f"    python3 bench.py --workload {args.workload}{flags} --steps 4 "
                         f"--warmup 1 --no-cpu-baseline --no-stream-probe --copy-probe 1024")
        lines.append(f"python3 bench.py --workload {args.workload}{flags} --summarize-pmc "
                     f"<out>/pmc_fetch/fetch_counter_collection.csv "
                     f"<out>/pmc_write/write_counter_collection.csv")
        lines += ["```", "",
                  f"Calibration: a 1 GiB device copy reads FETCH_SIZE = {t['copy_fetch_kib']:.0f} "
                  f"KiB and WRITE_SIZE = {t['copy_write_kib']:.0f} KiB: fetched bytes = FETCH_SIZE "
                  f"x {t['fetch_scale']:.3f} KiB, written = WRITE_SIZE x {t['write_scale']:.3f} KiB.",
                  "", "| per launch | bytes | vs algorithmic |", "|---|---|---|",
                  f"| decode fetched | {t['decode_fetch_bytes']:.4e} | "
                  f"{t['decode_fetch_bytes'] / t['algorithmic_kv_bytes']:.4f} x KV bytes |",
                  f"| decode written | {t['decode_write_bytes']:.4e} | partition results and "
                  f"outputs |"]
        cw = t.get("cache_write")
        if cw:
            lines += [f"| cache write fetched | {cw['fetch_bytes']:.4e} | "
                      f"{cw['fetch_bytes'] / cw['source_bytes']:.2f} x the new rows "
                      f"({cw['source_bytes']} B) |",
                      f"| cache write written | {cw['write_bytes']:.4e} | "
                      f"{cw['write_over_cache_bytes']:.2f} x the cache bytes of the new rows "
                      f"({cw['cache_bytes']} B) |"]
        lines += ["", f"Kernel source hash of the counted build: `{t['kernel_source_hash']}` "
                  f"({stamp} the current sources)."]
    if args.bench_json:
        b = json.loads(open(args.bench_json).read().strip().splitlines()[-1])
        r = b["roofline"]
        lines += ["", "## Benchmark line (`python3 bench.py --workload "
                  f"{args.workload}{flags}`, no profiler)", "",
                  f"- step {b['ms_per_step'] * 1e3:.1f} us = {b['value']:.0f} GB/s "
                  f"({b['pct_hbm_peak']:.1f}% of 8 TB/s), {b['tokens_per_s']:.3g} tokens/s;",
                  f"- decode launch (HIP events around pa_decode_partitions"
                  + (": the ordering kernel and the decode kernel" if b["config"]["grid"] ==
                     "sorted" and not b.get("step_form", "").startswith("write+order,")
                     else ": the decode kernel") + f") {b['decode_partitions_ms'] * 1e3:.1f} us "
                  f"= {r['achieved']:.0f} GB/s ({r['frac']:.1%} of 8 TB/s"
                  + (f", {r['frac_of_attainable']:.1%} of the streaming-read probe"
                     if r.get("frac_of_attainable") else "") + ");",
                  f"- {'write + item order' if b.get('step_form', '').startswith('write+order,') else 'write'} "
                  f"{b['write_ms'] * 1e3:.1f} us, merge {b['decode_merge_ms'] * 1e3:.1f} us "
                  f"between events; partition {b['config']['partition_size']}, grid "
                  f"{b['config']['grid']}, {b['config']['waves_per_item']} waves per item."]
        if b.get("size_matched_read"):
            m = b["size_matched_read"]
            lines.append(f"- a plain streaming read of the same {m['bytes']:.4g} bytes in one "
                         f"launch (probe, same event timing, {m['copies']} copies, "
                         f"{m['blocks']} workgroups): {m['us']:.1f} us = {m['gbps']:.0f} GB/s "
                         f"({m['gbps'] / 8000:.1%} of 8 TB/s); the decode launch takes "
                         f"{r['frac_of_size_matched_read']:.1%} of its rate.")
        if b.get("one_pass_vs_partitioned"):
            o = b["one_pass_vs_partitioned"]
            lines.append(f"- one pass per (sequence, kv head) {o['one_pass_us']:.1f} us against "
                         f"partitioned {o['partitioned_us']:.1f} us: {o['speedup']:.2f}x.")
    out = os.path.join(ROOT, "profiles", f"{kname}_{cfg.name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


# ----------------------------------------------------------------------------- benchmark

def write_kv(c, k, v, slots, kc, vc):
    """The library's cache write for the workload's cache dtype."""
    import pagedattention_kv_cache_amd as pa
    if c.kv_dtype == "fp8":
        pa.cache_write_fp8(k, v, slots, kc, vc, *c.fp8_scales)
    else:
        pa.cache_write(k, v, slots, kc, vc)


def decode_partitions_kv(c, out, q, kc, vc, bt, lens, part, ws, flags):
    """Phase 1 of the library's decode for the workload's cache dtype."""
    import pagedattention_kv_cache_amd as pa
    if c.kv_dtype == "fp8":
        pa.decode_fp8_partitions(out, q, kc, vc, bt, lens, c.attn_scale(), *c.fp8_scales,
                                 c.block_size, part, ws, flags)
    else:
        pa.decode_partitions(out, q, kc, vc, bt, lens, c.attn_scale(), c.block_size, part, ws,
                             flags)


def oracle_write(c, k, v, slots, okc, ovc):
    import oracle
    if c.kv_dtype == "fp8":
        oracle.cache_write_fp8(k, v, slots, okc, ovc, c.dtype, *c.fp8_scales)
    else:
        oracle.cache_write(k, v, slots, okc, ovc, c.dtype)


def fill_caches(wl, dev, kc, vc, oracle_caches=None):
    import torch

    import pagedattention_kv_cache_amd as pa
    from pagedattention_kv_cache_amd.workloads import raw_bits
    c = wl.cfg
    for b in range(c.num_seqs):
        k, v = wl.prior_kv(b)
        if k.shape[0] == 0:
            continue
        slots = wl.prior_slots(b)
        write_kv(c, k.to(dev), v.to(dev), torch.from_numpy(slots).to(dev), kc, vc)
        if oracle_caches is not None:
            oracle_write(c, raw_bits(k), raw_bits(v), slots, oracle_caches[0], oracle_caches[1])


def cpu_baseline(wl, okc, ovc, threads):
    """The oracle on the same step: ORC-W of the step's new tokens, then ORC-D
    of every (sequence, q head) row; median of repetitions."""
    import numpy as np

    import oracle
    from pagedattention_kv_cache_amd.workloads import raw_bits
    c = wl.cfg
    sk, sv = wl.step_kv()
    q = raw_bits(wl.queries()[0])
    slots = wl.step_slots(0)
    times = []
    t_start = time.perf_counter()
    while len(times) < 2 or (time.perf_counter() - t_start < 10.0 and len(times) < 10):
        t0 = time.perf_counter()
        oracle_write(c, raw_bits(sk[0]), raw_bits(sv[0]), slots, okc, ovc)
        ks, vs = c.fp8_scales if c.kv_dtype == "fp8" else (1.0, 1.0)
        oracle.decode(q, c.dtype, okc, ovc, c.kv_dtype, wl.block_tables, wl.context_lens(0),
                      c.attn_scale(), threads=threads, k_scale=ks, v_scale=vs)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    kv = wl.kv_bytes(0)
    # one more repetition on a single thread, for the per-core rate
    t1 = time.perf_counter()
    oracle_write(c, raw_bits(sk[0]), raw_bits(sv[0]), slots, okc, ovc)
    oracle.decode(q, c.dtype, okc, ovc, c.kv_dtype, wl.block_tables, wl.context_lens(0),
                  c.attn_scale(), threads=1, k_scale=ks, v_scale=vs)
    t1 = time.perf_counter() - t1
    return {
        "value": kv / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"one full step of {c.name} (write of {c.num_seqs} new tokens + all "
                   f"{c.num_seqs * c.num_q_heads} attention rows), fp64, median of {len(times)} "
                   f"repetitions"),
        "seconds_per_step": t,
        "tokens_per_s": c.num_seqs / t,
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
        "host_cpus_usable": len(os.sched_getaffinity(0)),
        "single_thread": {"seconds_per_step": t1, "value": kv / t1 / 1e9, "unit": "GB/s"},
    }


def graph_steps(args, wl, kcs, vcs, sk, sv, qs, bt, out, ws, part, flags) -> dict:
    """The workload's consecutive decode steps (write -> partitions -> merge ->
    device advance step) captured once per KV-cache layer in a HIP graph;
    each timed replay restores the initial per-sequence state first (four
    small device copies, as a scheduler would upload it) and runs all steps.
    A one-step workload captures write -> partitions -> merge only and
    replays it as is, like the eager timed loop: the same step's inputs each
    time, nothing to restore."""
    import torch

    import pagedattention_kv_cache_amd as pa
    c = wl.cfg
    dev = out.device
    init = {k: torch.from_numpy(v.copy()).to(dev) for k, v in wl.initial_state().items()}
    state = {k: v.clone() for k, v in init.items()}
    sampled = torch.from_numpy(wl.sampled_tokens()).to(dev)
    scale = c.attn_scale()

    multi = c.steps > 1

    def steps(k_l, v_l):
        for s in range(c.steps):
            write_kv(c, sk[s], sv[s], state["slot_mapping"], k_l, v_l)
            decode_partitions_kv(c, out, qs[s], k_l, v_l, bt, state["seq_lens"], part, ws, flags)
            pa.decode_merge(out, qs[s], k_l, v_l, bt, state["seq_lens"], scale, c.block_size,
                            part, ws, flags)
            if multi:
                pa.advance_step(c.num_seqs, c.block_size, state["input_tokens"], sampled[s],
                                state["input_positions"], state["seq_lens"],
                                state["slot_mapping"], bt)

    def reset():
        if multi:
            for k in state:
                state[k].copy_(init[k])

    graphs = []
    for k_l, v_l in zip(kcs, vcs):
        reset()
        steps(k_l, v_l)  # eager pass before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            steps(k_l, v_l)
        graphs.append(g)
    for g in graphs:
        reset()
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // c.steps) * len(graphs)
    t0 = time.perf_counter()
    for i in range(reps):
        reset()
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / (reps * c.steps)
    kv = statistics.mean(wl.kv_bytes(s) for s in range(c.steps))
    return {"steps_per_graph": c.steps, "replays": reps, "ms_per_step": round(ms_step, 5),
            "value": round(kv / (ms_step * 1e-3) / 1e9, 2),
            "tokens_per_s": round(c.num_seqs / (ms_step * 1e-3), 1)}


def one_pass_ratio(args, wl, kcs, vcs, qs, bt, ctx, out, ws, part_eff, flags) -> dict:
    """Whole decode (partitions + merge) per step, one pass per (sequence, kv
    head) against the partitioned launch: the first is one workgroup per
    (sequence, kv head) walking its whole context, the second the workload's
    partitions.  Rounds alternate between the two, each round timing every
    step of the rotation with HIP events on the launch stream."""
    import torch

    import pagedattention_kv_cache_amd as pa
    c = wl.cfg
    full = wl.max_blocks_per_seq * c.block_size
    stream = torch.cuda.current_stream()
    n_layers = len(kcs)

    def decode(i, p):
        s = (i // n_layers) % c.steps
        k_l, v_l = kcs[i % n_layers], vcs[i % n_layers]
        decode_partitions_kv(c, out, qs[s], k_l, v_l, bt, ctx[s], p, ws, flags)
        pa.decode_merge(out, qs[s], k_l, v_l, bt, ctx[s], c.attn_scale(), c.block_size, p, ws,
                        flags)

    times = {full: [], part_eff: []}
    for rnd in range(4):
        for p in ((full, part_eff) if rnd % 2 == 0 else (part_eff, full)):
            for i in range(2):
                decode(i, p)  # warm-up of this launch shape
            for i in range(args.steps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                decode(i, p)
                e1.record(stream)
                times[p].append((e0, e1))
    torch.cuda.synchronize()
    ms = {p: statistics.median(a.elapsed_time(b) for a, b in ev) for p, ev in times.items()}
    waves = {p: pa.decode_waves(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                c.block_size, wl.max_blocks_per_seq, p, qs.dtype, kcs[0].dtype,
                                flags) for p in (full, part_eff)}
    return {
        "one_pass_us": round(ms[full] * 1e3, 2),
        "one_pass_partition_tokens": int(full),
        "one_pass_waves_per_item": int(waves[full]),
        "partitioned_us": round(ms[part_eff] * 1e3, 2),
        "partition_tokens": int(part_eff),
        "partitioned_waves_per_item": int(waves[part_eff]),
        "speedup": round(ms[full] / ms[part_eff], 3),
        "timing": f"median over 4 alternating rounds of {args.steps} steps, decode + merge",
    }


def stream_probe(dev, gib: int = 4, reps: int = 10) -> float:
    """Attainable HBM read bandwidth: best of several grid sizes of a plain
    non-temporal streaming read over `gib` GiB (libpa_probe.so)."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "pagedattention_kv_cache_amd", "libpa_probe.so"))
    fn = lib.pa_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p]
    nbytes = gib * 2**30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for blocks in (4096, 8192, 16384):
        for _ in range(2):
            assert fn(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream) == 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream)
        e1.record(stream)
        e1.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def size_matched_probe(dev, nbytes: int, copies: int, launches: int = 24) -> dict:
    """A plain streaming read of the bytes one decode launch streams, in one
    launch, timed like the decode: HIP events around each launch, rotating over
    `copies` buffers as the decode rotates over its cache copies; best mean
    over a few grid sizes.  What one launch of this size can reach (dispatch,
    ramp and drain included), beside the large probe's steady rate."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "pagedattention_kv_cache_amd", "libpa_probe.so"))
    fn = lib.pa_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p]
    n = (int(nbytes) + 255) // 256 * 256
    buf = torch.ones(copies * n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best_us, best_blocks = None, None
    for blocks in (1024, 2048, 4096, 8192):
        def launch(i):
            assert fn(buf.data_ptr() + (i % copies) * n, n, sink.data_ptr(), blocks,
                      stream.cuda_stream) == 0
        for i in range(copies):
            launch(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            launch(i)
            e1.record(stream)
        torch.cuda.synchronize()
        us = statistics.mean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
        if best_us is None or us < best_us:
            best_us, best_blocks = us, blocks
    del buf
    torch.cuda.empty_cache()
    return {"bytes": n, "us": round(best_us, 2), "gbps": round(n / (best_us * 1e-6) / 1e9, 1),
            "blocks": best_blocks, "copies": copies}


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, then family / model /
    stepping (a virtualised host may report only a short model name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key = key.strip()
            if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                fields[key] = val.strip()
            if not line.strip() and fields:
                break
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    ident = "/".join(fields.get(k, "?") for k in ("cpu family", "model", "stepping"))
    return f"{name} (family/model/stepping {ident})"


def run(args):
    import numpy as np
    import torch

    import pagedattention_kv_cache_amd as pa
    from pagedattention_kv_cache_amd.workloads import (WORKLOADS, DTYPE_TORCH, FP8_WORKLOADS,
                                                       Workload)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the paged decode "
                          "path has no multi-GPU mode here (it would shard by sequences or by "
                          "kv heads, with no exchange inside the path)", "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    pa.lib()
    dev = torch.device("cuda:0")
    if args.kv_cache == "fp8":
        if args.workload not in FP8_WORKLOADS:
            print(json.dumps({"error": f"no E4M3-cache variant of workload {args.workload}; "
                              f"have {sorted(FP8_WORKLOADS)}"}))
            sys.exit(2)
        cfg = FP8_WORKLOADS[args.workload]
    else:
        cfg = WORKLOADS[args.workload]
    wl = Workload(cfg)
    c = cfg
    flags = {"auto": pa.AUTO, "valu": pa.FORCE_VALU, "mfma": pa.FORCE_MFMA}[args.flags]
    if args.waves:
        flags |= pa.WAVES_FLAG[args.waves]
    if args.no_work_list:
        flags |= pa.NO_WORK_LIST
    flags |= {"auto": 0, "grid": pa.NO_WORK_LIST, "sorted": pa.SORTED_GRID,
              "work_list": pa.WORK_LIST}[args.grid]
    part = cfg.partition_size if args.partition_size < 0 else args.partition_size

    if args.copy_probe:
        n = args.copy_probe * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    qdt = DTYPE_TORCH[c.dtype]
    kdt = DTYPE_TORCH[c.kv_dtype]
    kc = torch.empty(pa.key_cache_shape(wl.num_blocks, c.num_kv_heads, c.head_dim, c.block_size,
                                        kdt), dtype=kdt, device=dev)
    vc = torch.empty(pa.value_cache_shape(wl.num_blocks, c.num_kv_heads, c.head_dim,
                                          c.block_size), dtype=kdt, device=dev)
    Q = args.queries
    want_cpu = not args.no_cpu_baseline and Q == 1
    okc = ovc = None
    if want_cpu:
        import oracle
        from pagedattention_kv_cache_amd.workloads import POISON_BITS
        oracle.build(force=False)
        bits = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}[c.kv_dtype]
        okc = np.full(tuple(kc.shape), POISON_BITS[c.kv_dtype], bits)
        ovc = np.full(tuple(vc.shape), POISON_BITS[c.kv_dtype], bits)
    t_fill = time.perf_counter()
    fill_caches(wl, dev, kc, vc, (okc, ovc) if want_cpu else None)
    # further layers: device copies of the first one (same values, own memory)
    kcs, vcs = [kc], [vc]
    for _ in range(1, max(1, args.layers)):
        kcs.append(kc.clone())
        vcs.append(vc.clone())
    torch.cuda.synchronize()
    t_fill = time.perf_counter() - t_fill

    bt = torch.from_numpy(wl.block_tables).to(dev)
    qs = wl.queries().to(dev)
    sk, sv = wl.step_kv()
    sk, sv = sk.to(dev), sv.to(dev)
    slots = [torch.from_numpy(wl.step_slots(s)).to(dev) for s in range(c.steps)]
    ctx = [torch.from_numpy(wl.context_lens(s)).to(dev) for s in range(c.steps)]
    MB = wl.max_blocks_per_seq
    p_eff = part if part else pa.decode_partition_size(c.num_seqs * Q, c.num_q_heads,
                                                       c.num_kv_heads,
                                                       c.head_dim, c.block_size, MB, kdt, flags)
    ws_bytes = pa.decode_workspace_size(c.num_seqs * Q, c.num_q_heads, c.num_kv_heads,
                                        c.head_dim, c.block_size, MB, part, kdt, flags)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)  # zeroed once
    if Q > 1:
        qs = wl.multi_queries(Q).to(dev).unsqueeze(0).expand(c.steps, -1, -1, -1, -1)
    out = torch.empty(qs.shape[1:], dtype=torch.float32, device=dev)
    scale = c.attn_scale()
    stream = torch.cuda.current_stream(dev)

    n_layers = len(kcs)
    fused = args.fused_step and Q == 1 and c.kv_dtype != "fp8"
    # default step form: the write and the item order in one launch before the
    # decode kernel, which the events then bracket alone
    split = not fused and not args.separate_write and Q == 1

    def step(i, ev=None):
        # step i: decode step (i // n_layers) % steps of layer i % n_layers
        s = (i // n_layers) % c.steps
        k_l, v_l = kcs[i % n_layers], vcs[i % n_layers]
        if ev is not None and ev[0] is not None:
            ev[0].record(stream)
        if fused:
            if ev is not None:
                ev[1].record(stream)
            pa.decode_step_partitions(sk[s], sv[s], slots[s], out, qs[s], k_l, v_l, bt, ctx[s],
                                      scale, c.block_size, part, ws, flags)
        elif split:
            if c.kv_dtype == "fp8":  # the quantizing write and the order
                pa.decode_order_fp8(out, qs[s], k_l, v_l, bt, ctx[s], scale, *c.fp8_scales,
                                    c.block_size, part, ws, flags, sk[s], sv[s], slots[s])
            else:
                pa.decode_order(out, qs[s], k_l, v_l, bt, ctx[s], scale, c.block_size, part, ws,
                                flags, k=sk[s], v=sv[s], slot_mapping=slots[s])
            if ev is not None:
                ev[1].record(stream)
        else:
            write_kv(c, sk[s], sv[s], slots[s], k_l, v_l)
            if ev is not None:
                ev[1].record(stream)
        if fused:
            pass
        elif split:
            decode_partitions_kv(c, out, qs[s], k_l, v_l, bt, ctx[s], part, ws,
                                 flags | pa.ORDERED)
        elif Q > 1:
            ks, vs = c.fp8_scales if c.kv_dtype == "fp8" else (1.0, 1.0)
            pa.decode_mq_partitions(out, qs[s], k_l, v_l, bt, ctx[s], scale, c.block_size, part,
                                    ws, flags, ks, vs)
        else:
            decode_partitions_kv(c, out, qs[s], k_l, v_l, bt, ctx[s], part, ws, flags)
        if ev is not None:
            ev[2].record(stream)
        if Q > 1:
            pa.decode_mq_merge(out, qs[s], k_l, v_l, bt, ctx[s], scale, c.block_size, part, ws,
                               flags)
        else:
            pa.decode_merge(out, qs[s], k_l, v_l, bt, ctx[s], scale, c.block_size, part, ws,
                            flags)
        if ev is not None and ev[3] is not None:
            ev[3].record(stream)

    def events():
        return [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                for _ in range(args.steps)]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: only the decode launches are bracketed by events (each
    # event record is one more packet between the kernels of a step).
    evs = events()
    for e in evs:
        e[0] = e[3] = None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dec_times = [e[1].elapsed_time(e[2]) for e in evs]
    dec_ms = statistics.mean(dec_times)
    # Breakdown pass (after the timed region, same steps): events around every launch.
    evs = events()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    write_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    merge_ms = statistics.mean(e[2].elapsed_time(e[3]) for e in evs)
    dec_ms_breakdown = statistics.mean(e[1].elapsed_time(e[2]) for e in evs)

    kv = statistics.mean(wl.kv_bytes((i // n_layers) % c.steps) for i in range(args.steps))
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = kv / (dec_ms * 1e-3) / 1e9

    # the partition the timed launches used: the library's pick, or its
    # refinement on the device from the actual lengths (partition_size 0)
    p_used = int(p_eff)
    if not part and Q == 1:
        p_used = pa.decode_partition_used(ws, c.num_seqs, c.num_q_heads, c.num_kv_heads,
                                          c.head_dim, c.block_size, wl.max_blocks_per_seq, kdt,
                                          flags)

    graph = None
    if args.graph and Q == 1:
        graph = graph_steps(args, wl, kcs, vcs, sk, sv, qs, bt, out, ws, part, flags)
    ratio = None
    if args.one_pass_ratio and Q == 1:
        ratio = one_pass_ratio(args, wl, kcs, vcs, qs, bt, ctx, out, ws, p_used, flags)
    attainable = None if args.no_stream_probe else stream_probe(dev)
    same_bytes = None if args.no_size_probe else size_matched_probe(dev, kv, len(kcs))
    traffic = measured_traffic(c.name)

    family = pa.decode_mq_kernel(Q, c.num_q_heads, c.num_kv_heads, qdt, kdt, flags)
    kname = f"decode_{family}_kernel"
    result = {
        "metric": "paged decode attention: achieved KV HBM GB/s (% peak) + tokens/s, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block pool; no dataset)",
        "config": {"workload": c.name, **{k: v for k, v in wl.describe().items() if k != "workload"},
                   "partition_size": p_used, "partition_size_host_pick": int(p_eff),
                   "kernel_flags": args.flags,
                   "queries_per_seq": Q,
                   "grid": pa.decode_grid(c.num_seqs * Q, c.num_q_heads, c.num_kv_heads,
                                          c.head_dim, c.block_size, wl.max_blocks_per_seq,
                                          int(p_eff), qdt, kdt,
                                          flags | (pa.ORDERED if split else 0)),
                   "waves_per_item": pa.decode_waves(c.num_seqs, c.num_q_heads, c.num_kv_heads,
                                                     c.head_dim, c.block_size,
                                                     wl.max_blocks_per_seq, int(p_eff), qdt, kdt,
                                                     flags)},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(c.num_seqs * Q / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": int(kv),
        "other_bytes_per_step": side_bytes(wl, Q),
        "write_ms": None if fused else round(write_ms, 5),
        "fused_write": fused,
        "step_form": ("write+order, decode kernel, merge" if split else
                      "write+order+decode, merge" if fused else "write, order+decode, merge"),
        "decode_partitions_ms": round(dec_ms, 5),
        "decode_partitions_ms_median_min_max": [round(statistics.median(dec_times), 5),
                                                round(min(dec_times), 5),
                                                round(max(dec_times), 5)],
        "decode_merge_ms": round(merge_ms, 5),
        "decode_partitions_ms_breakdown_pass": round(dec_ms_breakdown, 5),
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(kv),
        },
        "fill_seconds": round(t_fill, 2),
        "kv_cache_layers": n_layers,
    }
    if graph:
        result["graph"] = graph
    if ratio:
        result["one_pass_vs_partitioned"] = ratio
    if attainable:
        result["attainable_read_gbps"] = round(attainable, 1)
        result["roofline"]["frac_of_attainable"] = round(achieved / attainable, 4)
    if same_bytes:
        result["size_matched_read"] = same_bytes
        result["roofline"]["frac_of_size_matched_read"] = round(achieved / same_bytes["gbps"], 4)
    if want_cpu:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        result["cpu_baseline"] = cpu_baseline(wl, okc, ovc, threads)
    print(json.dumps(result), flush=True)


def main(argv=None):
    args = parse_args(argv)
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    run(args)


if __name__ == "__main__":
    main()
