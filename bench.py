"""Benchmark of the ternary linear layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  decode  for b = 1, 4, 8 and 16 tokens: block rotation fused with the GEMV
          activation prep (one kernel) -> the GEMV weight stream of DEC_LAYERS
          qkv-shaped layers (K=5120 -> N=10240, each a different weight copy);
  prefill (512-token chunk): for gate_up (5120 -> 34816) and down (17408 -> 5120),
          block rotation fused with per-token int8 quantisation (one kernel) ->
          int8 GEMM + rescale of PRE_LAYERS layers each.
Weights are packed once (load time, not timed) and cloned into rotating copies
(>= 1 GiB per layer type) so that successive launches read weights that are not
resident in the 256 MB Infinity Cache.

Reported: decode GEMV GB/s (algorithmic bytes / kernel time, aggregated over the
four batch sizes) as `value`, its fraction of the 8 TB/s HBM peak, prefill int8
TOP/s against the 5.0 POP/s dense int8 peak, and the CPU oracle timed on a
bounded sample.  Kernel durations come from HIP events recorded on the stream
the kernels run on (torch's current stream) around each back-to-back run of
GEMV (or GEMM) launches inside the timed steps, divided by the launch count;
bracketing runs rather than single launches keeps the event overhead out of the
per-launch figure, which then matches the rocprofv3 kernel durations.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402  (seeded input recipes; no arithmetic of the method)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
MALL_BYTES = 256 * 2 ** 20
ROTATE_BYTES = 2 ** 30

CALIB_BYTES = 64 * 2 ** 20    # the PMC calibration kernel reads and writes this many bytes
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "gemv": ("quantized_gemv_gemm_amd/csrc/k_gemv.hip", "quantized_gemv_gemm_amd/csrc/tl_device.h"),
    "gemm": ("quantized_gemv_gemm_amd/csrc/k_gemm.hip", "quantized_gemv_gemm_amd/csrc/tl_device.h"),
}

DECODE_BS = (1, 4, 8, 16)
PREFILL_M = 512
MFMA_PROBE_GRID = 512        # workgroups of tl_mfma_probe (four waves each)
DEC_LAYERS = 8     # qkv-shaped layers per decode pass (distinct weight copies)
PRE_LAYERS = 2     # layers of each MLP type per prefill pass
# random-stream numbers of the synthetic workloads
S_DEC, S_MLP, S_PRE = (synth.WORKLOADS[w]["stream"] for w in ("decode_qkv", "decode_mlp", "prefill_mlp"))


def gemv_bytes(b, K, N):
    """Algorithmic bytes of one GEMV weight-stream launch: packed codes, scales,
    the two int8 activation limbs, and the bf16 output."""
    return N * K // 4 + N * (K // 128) * 2 + 2 * b * K + 2 * b * N


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-stack", action="store_true", help="skip the 64-block whole-stack pass")
    p.add_argument("--stack-steps", type=int, default=5)
    p.add_argument("--bsweep", action="store_true",
                   help="token-count sweep of the two layer paths (GEMV vs int8 GEMM) instead of the bench")
    p.add_argument("--library-reference", action="store_true",
                   help="time torch._int_mm (the vendor int8 GEMM the pages' prefill calls) at the prefill "
                        "shapes, with int8 weights already expanded, beside this library's GEMM")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a 64 MiB device copy 20 times (the PMC byte-counter calibration)")
    p.add_argument("--warm", action="store_true",
                   help="with --phase-stamps: one weight copy (Infinity-Cache resident) instead of rotating copies")
    p.add_argument("--phase-stamps", action="store_true",
                   help="load the instrumented library (python -m quantized_gemv_gemm_amd._build --phase-stamps) "
                        "and print the decode GEMV's per-wave phase times at qkv and gate_up, b = 1, 4, 8, 16")
    p.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                   help="print the per-launch median of every counter in rocprofv3 --pmc CSVs of this bench "
                        "(--steps S --warmup W), one row per decode b and prefill shape, then exit")
    p.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="write the HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                        "counter CSVs of this bench (--steps S --warmup W) and of --calib-copy, then exit")
    p.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "STATS_CSV"),
                   help="print the per-launch device time of the GEMV and GEMM launches from a rocprofv3 "
                        "--kernel-trace --stats run of this bench, and the library's kernel statistics, then exit")
    return p.parse_args()


def source_hash(kind):
    """sha256 of the sources a kernel family is built from (counters go stale when it changes)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _pmc_rows(path):
    import csv
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]


def _short_name(name):
    """`gemv_lds_kernel<1, 1, 5>` out of a demangled kernel signature."""
    import re
    m = re.search(r"(\w+_kernel(?:<[^()]*>)?)\(", name)
    return m.group(1) if m else name[:80]


def _attribute(rows):
    """(launch, kernel, value) for the GEMV and GEMM launches of the bench steps, in order.

    Launches are attributed by their order inside a step: DEC_LAYERS GEMV launches
    for each b in DECODE_BS, then PRE_LAYERS GEMM launches for gate_up and for down.
    The GEMV launches of the read-floor comparison follow the steps and are dropped."""
    gemv = [(n, v) for n, v in rows if "gemv_stream_kernel" in n or "gemv_ring_kernel" in n]
    gemm = [(n, v) for n, v in rows if "gemm_i8_kernel" in n]
    gemv = gemv[:len(gemm) // (2 * PRE_LAYERS) * DEC_LAYERS * len(DECODE_BS)]
    if not gemv or len(gemv) % (DEC_LAYERS * len(DECODE_BS)) or not gemm or len(gemm) % (2 * PRE_LAYERS):
        raise SystemExit(f"unexpected launch counts: {len(gemv)} GEMV, {len(gemm)} GEMM")
    out = []
    for i, (name, v) in enumerate(gemv):
        out.append(("gemv", str(DECODE_BS[(i // DEC_LAYERS) % len(DECODE_BS)]), _short_name(name), v))
    for i, (name, v) in enumerate(gemm):
        out.append(("gemm", ("gate_up", "down")[(i // PRE_LAYERS) % 2], _short_name(name), v))
    return out


def summarize_counters(paths):
    """Median per launch of each counter, as a markdown table (counters summed over the chip)."""
    import csv
    table, counters = {}, []
    for path in paths:
        with open(path, newline="") as f:
            rows = list(csv.DictReader(f))
        for cname in sorted({r["Counter_Name"] for r in rows}):
            sel = sorted((r for r in rows if r["Counter_Name"] == cname), key=lambda r: int(r["Dispatch_Id"]))
            counters.append(cname)
            for fam, key, kname, v in _attribute([(r["Kernel_Name"], float(r["Counter_Value"])) for r in sel]):
                e = table.setdefault((fam, key), {"kernel": kname})
                e.setdefault(cname, []).append(v)
    print("| launch | kernel | launches | " + " | ".join(counters) + " |")
    print("|---|---|---|" + "---|" * len(counters))
    for (fam, key), e in table.items():
        label = f"decode GEMV qkv b={key}" if fam == "gemv" else f"prefill GEMM {key}"
        vals = " | ".join(f"{float(np.median(e[c])):.4g}" if c in e else "-" for c in counters)
        print(f"| {label} | `{e['kernel']}` | {len(e[counters[0]])} | {vals} |")


def summarize_trace(trace_csv, stats_csv):
    """Per-launch device time (kernel trace) of the bench's GEMV and GEMM launches, as
    markdown: count, mean, median, p10, p90 in µs; then the library's rows of the
    --stats table."""
    import csv
    with open(trace_csv, newline="") as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    durs = [(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]
    groups = {}
    for fam, key, kname, v in _attribute(durs):
        groups.setdefault((fam, key), (kname, []))[1].append(v)
    print("| launch | kernel | launches | mean µs | median µs | p10 µs | p90 µs |")
    print("|---|---|---|---|---|---|---|")
    labels = {"gate_up": "gate_up 5120→34816", "down": "down 17408→5120"}
    for (fam, key), (kname, v) in groups.items():
        d = np.sort(np.asarray(v))
        name = (f"decode GEMV qkv 5120→10240 b={key}" if fam == "gemv" else f"prefill GEMM M={PREFILL_M} {labels[key]}")
        print(f"| {name} | `{kname}` | {len(d)} | {d.mean():.2f} | {np.median(d):.2f} | "
              f"{np.percentile(d, 10):.2f} | {np.percentile(d, 90):.2f} |")
    print()
    with open(stats_csv, newline="") as f:
        stats = list(csv.DictReader(f))
    print("| kernel | calls | avg µs | min µs | max µs | % |")
    print("|---|---|---|---|---|---|")
    for r in stats:
        name = _short_name(r["Name"] + "(")
        if not any(k in name for k in ("gemv_", "gemm_", "spin_kernel", "read_probe", "mfma_probe")):
            continue
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")


def summarize_pmc(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per launch of the GEMV and GEMM kernels from rocprofv3 FETCH_SIZE / WRITE_SIZE runs.

    The counters read KiB per dispatch.  Each is scaled by the factor that makes
    it read exactly CALIB_BYTES for the calibration kernel (an elementwise
    negation of CALIB_BYTES of float32: CALIB_BYTES read, CALIB_BYTES written).
    Launches are attributed as _attribute says.
    """
    def calib(path):
        vals = [v for name, v in _pmc_rows(path) if "neg" in name]
        if not vals:
            raise SystemExit(f"no calibration dispatch in {path}")
        return (CALIB_BYTES / 1024.0) / float(np.median(vals))

    f_fac, w_fac = calib(copy_fetch_csv), calib(copy_write_csv)
    out = {"copy_factor": {"fetch": round(f_fac, 4), "write": round(w_fac, 4)},
           "sources": {k: source_hash(k) for k in KERNEL_SOURCES}, "gemv": {}, "gemm": {}}
    for counter, path, fac in (("fetch", fetch_csv, f_fac), ("write", write_csv, w_fac)):
        for fam, key, kname, v in _attribute(_pmc_rows(path)):
            e = out[fam].setdefault(key, {"kernel": kname, "fetch": [], "write": []})
            e[counter].append(v * 1024.0 * fac)
    for fam in ("gemv", "gemm"):
        for e in out[fam].values():
            e["launches"] = len(e["fetch"])
            e["fetch_bytes"] = round(float(np.mean(e.pop("fetch"))))
            e["write_bytes"] = round(float(np.mean(e.pop("write"))))
            e["traffic_bytes"] = e["fetch_bytes"] + e["write_bytes"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def spread(samples_ms, run_medians_ms):
    """p10 / p50 / p90 (us) of the per-step samples of one arm, and the median of each run."""
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    return {"us_p10": round(float(np.percentile(a, 10)), 3), "us_p50": round(float(np.percentile(a, 50)), 3),
            "us_p90": round(float(np.percentile(a, 90)), 3),
            "us_run_medians": [round(m * 1e3, 3) for m in run_medians_ms]}


def roofline_gate(out):
    """Any rate above the chip's peak means a measurement artefact (a launch that did
    not do its work, or data served from a cache): such a line is not valid."""
    bad = []
    for b, v in out["decode_gemv_by_b"].items():
        if v["GBps"] > HBM_PEAK_GBS:
            bad.append(f"decode_gemv b={b} {v['GBps']} GB/s")
    for b, v in out.get("decode_layer", {}).items():
        if v["GBps"] > HBM_PEAK_GBS:
            bad.append(f"decode_layer b={b} {v['GBps']} GB/s")
    for k, v in out["prefill_gemm"].items():
        if v["TOPs"] > INT8_PEAK_TOPS:
            bad.append(f"prefill_gemm {k} {v['TOPs']} TOP/s")
    rc = out["launch_floor"].get("read_codes")
    if rc and rc["GBps"] > HBM_PEAK_GBS:
        bad.append(f"read floor {rc['GBps']} GB/s")
    for b, rows in out.get("gemv_vs_read_floor", {}).items():
        for r in rows:
            for key in ("gemv_GBps", "read_GBps"):
                if r[key] > HBM_PEAK_GBS:
                    bad.append(f"gemv_vs_read_floor {b} {r['shape']} {key} {r[key]}")
    st = out.get("stack64")
    if st:
        if st["decode_b16"]["gemv_GBps"] > HBM_PEAK_GBS:
            bad.append("stack64 decode")
        if st["prefill_m2048"]["gemm_TOPs"] > INT8_PEAK_TOPS:
            bad.append("stack64 prefill")
    return {"rule": f"every GB/s <= {HBM_PEAK_GBS:.0f} and every TOP/s <= {INT8_PEAK_TOPS:.0f}",
            "valid": not bad, "violations": bad}


def load_traffic():
    """Per-launch HBM traffic measured for the current kernel sources, or {} if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    return {fam: t[fam] for fam in KERNEL_SOURCES if t.get("sources", {}).get(fam) == source_hash(fam)}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): it measures the "
              "single-GPU kernels; sharding across GPUs is described, not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_gemv_gemm_amd as tl
    import synth

    if args.phase_stamps:
        from quantized_gemv_gemm_amd import _build
        if not os.path.exists(_build.STAMPS_LIB):
            raise SystemExit(f"{_build.STAMPS_LIB} is not built: python -m quantized_gemv_gemm_amd._build --phase-stamps")
        tl.LIB_PATH = _build.STAMPS_LIB
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tl.lib()

    if args.calib_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calib_kernel": "neg float32", "bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES,
                          "launches": 20}))
        return

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.bsweep:
        bsweep(tl, torch, dev, log)
        return
    if args.library_reference:
        library_reference(tl, torch, dev)
        return

    # ---------------- weights (packed once, cloned into rotating copies) ----------------
    def make_layer(stream, li, K, N):
        L = synth.LayerInputs(0, stream, li, K, N)
        codes = L.codes_torch(dev)
        scales = torch.from_numpy(L.scales()).to(dev)
        packed, q, rs = tl.pack_weights(codes, scales)
        del codes
        per = packed.numel() * 4 + scales.numel() * 2 + q.numel() + rs.numel() * 4
        R = max(2, math.ceil(ROTATE_BYTES / per))
        copies = [(packed, scales, q, rs)] + [(packed.clone(), scales.clone(), q.clone(), rs.clone())
                                              for _ in range(R - 1)]
        return copies

    log("packing the decode qkv layer and the prefill MLP layers")
    qkv = make_layer(S_DEC, 0, 5120, 10240)
    gate_up = make_layer(S_PRE, 0, 5120, 34816)
    down = make_layer(S_PRE, 1, 17408, 5120)
    torch.cuda.synchronize()
    log(f"rotating copies: qkv {len(qkv)}, gate_up {len(gate_up)}, down {len(down)}")

    # ---------------- activations ----------------
    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.phase_stamps:
        if args.warm:   # a diagnostic: the weights served from the Infinity Cache, not HBM
            phase_stamps(tl, torch, dev, {"qkv_warm": (qkv[:1], 5120, 10240), "gate_up_warm": (gate_up[:1], 5120, 34816)},
                         bf16, synth)
        else:
            phase_stamps(tl, torch, dev, {"qkv": (qkv, 5120, 10240), "gate_up": (gate_up, 5120, 34816)}, bf16, synth)
        return

    Kq, Nq = 5120, 10240
    x_dec = {b: bf16(synth.activations(0, S_DEC, 0, b, Kq)) for b in DECODE_BS}
    ws_dec = {b: torch.empty((tl.gemv_workspace_size(b, Kq, Nq),), dtype=torch.uint8, device=dev)
              for b in DECODE_BS}
    y_dec = {b: torch.empty((b, Nq), dtype=torch.bfloat16, device=dev) for b in DECODE_BS}

    pre = {}
    for name, copies, li, K, N in (("gate_up", gate_up, 0, 5120, 34816), ("down", down, 1, 17408, 5120)):
        pre[name] = dict(copies=copies, K=K, N=N,
                         x=bf16(synth.activations(0, S_PRE, li, PREFILL_M, K)),
                         xq=torch.empty((PREFILL_M, K), dtype=torch.int8, device=dev),
                         sx=torch.empty((PREFILL_M,), dtype=torch.float32, device=dev),
                         y=torch.empty((PREFILL_M, N), dtype=torch.bfloat16, device=dev))

    stream = torch.cuda.current_stream(dev)
    rot = {"qkv": 0, "gate_up": 0, "down": 0}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    kernel_names = {}

    def step(rec, spin=False):
        """One pass of the hot path; appends (kind, key, n_launches, start, end) when rec is a list.
        spin: queue a device-side spin before each timed group, so that the group's
        launches reach the GPU back to back and the events measure device time
        rather than the pace of the launching Python thread."""
        for b in DECODE_BS:
            tl.gemv_prepare_x(x_dec[b], ws_dec[b])          # rotation fused into the GEMV prep
            if rec is not None:
                e0, e1 = ev(), ev()
                if spin:
                    torch.cuda._sleep(200_000)
                e0.record(stream)
            for _ in range(DEC_LAYERS):
                packed, scales, _, _ = qkv[rot["qkv"] % len(qkv)]
                rot["qkv"] += 1
                tl.gemv_prepared(ws_dec[b], b, Kq, packed, scales, y_dec[b])
            kernel_names[("gemv", b)] = tl.last_kernel_name()
            if rec is not None:
                e1.record(stream)
                rec.append(("gemv", b, DEC_LAYERS, e0, e1))
        for name in ("gate_up", "down"):
            P = pre[name]
            tl.quant_act_int8_x(P["x"], xq=P["xq"], tok_scale=P["sx"])   # rotation fused into the quantisation
            if rec is not None:
                e0, e1 = ev(), ev()
                if spin:
                    torch.cuda._sleep(200_000)
                e0.record(stream)
            for _ in range(PRE_LAYERS):
                packed, _, q, rs = P["copies"][rot[name] % len(P["copies"])]
                rot[name] += 1
                tl.gemm_int8_rescale(P["xq"], P["sx"], packed, q, rs, out=P["y"])
            kernel_names[("gemm", name)] = tl.last_kernel_name()
            if rec is not None:
                e1.record(stream)
                rec.append(("gemm", name, PRE_LAYERS, e0, e1))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    # the timed region runs with Python's garbage collector off: a collection
    # pause stalls the launch thread and shows up as idle GPU time in the events
    import gc
    gc.collect()
    gc.disable()
    log(f"timing {args.steps} steps")
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step(None)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # per-kernel device times: the same steps again, each timed group queued
    # behind a spin (the step time above is the plain, spin-free pass); two such
    # runs, so that every arm has two medians from the same session
    gemv_ms = {b: [] for b in DECODE_BS}
    gemm_ms = {"gate_up": [], "down": []}
    gemv_runs = {b: [] for b in DECODE_BS}
    gemm_runs = {"gate_up": [], "down": []}
    for _run in range(2):
        rec = []
        for _ in range(args.steps):
            step(rec, spin=True)
        torch.cuda.synchronize()
        sink = {"gemv": gemv_ms, "gemm": gemm_ms}
        runs = {"gemv": gemv_runs, "gemm": gemm_runs}
        this = {"gemv": {b: [] for b in DECODE_BS}, "gemm": {"gate_up": [], "down": []}}
        for kind, key, n, e0, e1 in rec:
            sink[kind][key].append(e0.elapsed_time(e1) / n)
            this[kind][key].append(e0.elapsed_time(e1) / n)
        for kind in ("gemv", "gemm"):
            for key, v in this[kind].items():
                runs[kind][key].append(float(np.median(v)))

    # the fused input kernels: n back-to-back launches between two events, all
    # queued behind a device-side spin so that the GPU never waits for the host
    # (small launches issued from Python would otherwise measure the host's pace)
    def run_time(fn, n=20):
        fn()
        e0, e1 = ev(), ev()
        torch.cuda._sleep(2_000_000)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    prep_ms = {b: [run_time(lambda: tl.gemv_prepare_x(x_dec[b], ws_dec[b]))] for b in DECODE_BS}
    quant_ms = {k: [run_time(lambda: tl.quant_act_int8_x(P["x"], xq=P["xq"], tok_scale=P["sx"]))]
                for k, P in pre.items()}
    # The GEMV weight stream against the streaming floor, per layer shape (qkv,
    # down, gate_up: 14 to 48 MB) at b = 1 and 16: the GEMV's time and that of a
    # launch that only reads the same layer's packed codes (read_probe), each the
    # mean of back-to-back launches over rotating weight copies behind a spin.
    # excess_us = what the GEMV adds on top of moving its codes at all.
    sink_f = torch.zeros((4,), dtype=torch.int32, device=dev)
    vs_floor = {}
    floor_shapes = (("qkv", qkv, 5120, 10240), ("down", pre["down"]["copies"], 17408, 5120),
                    ("gate_up", pre["gate_up"]["copies"], 5120, 34816))
    read_us = {}
    for name, copies, K, N in floor_shapes:
        kr = [0]

        def read_one():
            tl.read_probe(copies[kr[0] % len(copies)][0], sink_f)
            kr[0] += 1
        read_us[name] = run_time(read_one, n=DEC_LAYERS * 4) * 1e3
    for b in (1, 16):
        rows = []
        for name, copies, K, N in floor_shapes:
            xr = tl.hadamard_blk(bf16(synth.activations(0, S_MLP, 7, b, K)))
            ws = torch.empty((tl.gemv_workspace_size(b, K, N),), dtype=torch.uint8, device=dev)
            yb = torch.empty((b, N), dtype=torch.bfloat16, device=dev)
            tl.gemv_prepare(xr, ws)
            k = [0]

            def one():
                packed, scales = copies[k[0] % len(copies)][:2]
                k[0] += 1
                tl.gemv_prepared(ws, b, K, packed, scales, yb)
            t_us = run_time(one, n=DEC_LAYERS * 4) * 1e3
            code_bytes = copies[0][0].numel() * 4
            rows.append({"shape": name, "kernel": tl.last_kernel_name(), "gemv_us": round(t_us, 2),
                         "gemv_bytes": int(gemv_bytes(b, K, N)),
                         "gemv_GBps": round(gemv_bytes(b, K, N) / (t_us * 1e-6) / 1e9, 1),
                         "read_codes_us": round(read_us[name], 2), "code_bytes": int(code_bytes),
                         "read_GBps": round(code_bytes / (read_us[name] * 1e-6) / 1e9, 1),
                         "ratio": round(t_us / read_us[name], 3), "excess_us": round(t_us - read_us[name], 2)})
        vs_floor[f"b{b}"] = rows
    # the rotation alone (tl_hadamard_blk: bf16 in, f32 out), at the decode and prefill sizes
    rot_only = {}
    for label, xs in (("decode_b16_k5120", x_dec[16]), ("prefill_m512_k17408", pre["down"]["x"])):
        xr_o = torch.empty(xs.shape, dtype=torch.float32, device=dev)
        t_ms = run_time(lambda: tl.hadamard_blk(xs, out=xr_o))
        nb = xs.numel() * 6
        rot_only[label] = {"us": round(t_ms * 1e3, 2), "GBps": round(nb / (t_ms * 1e-3) / 1e9, 1)}
    # split-block rotation stages of a TP=2 shard boundary (down_proj's block 8):
    # the half stage on a column slice of the raw input, the join into the rank's columns
    split_us = {}
    for T, xs in ((16, x_dec[16]), (PREFILL_M, pre["down"]["x"])):
        u = torch.empty((T, 512), dtype=torch.float64, device=dev)
        xr_half = torch.empty((T, 512), dtype=torch.float32, device=dev)
        split_us[f"half_T{T}"] = round(run_time(lambda: tl.hadamard_half(xs[:, 512:1024], u=u)) * 1e3, 2)
        split_us[f"join_T{T}"] = round(run_time(lambda: tl.hadamard_join(u, u, 1, out=xr_half)) * 1e3, 2)
    # Context for the per-launch floor, timed the same way: a one-element launch
    # (dispatch and completion only), and the vendor library copying the qkv
    # layer's packed codes (N K / 4 bytes read and written), over the same
    # rotating copies.
    one = torch.zeros((1,), dtype=torch.float32, device=dev)
    codes_dst = torch.empty_like(qkv[0][0])
    kq = [0]

    def copy_codes():
        codes_dst.copy_(qkv[kq[0] % len(qkv)][0])
        kq[0] += 1
    floor = {"empty_launch_us": round(run_time(lambda: one.add_(1.0)) * 1e3, 2)}
    t_copy = run_time(copy_codes, n=DEC_LAYERS * 4) * 1e-3
    nb = 2 * codes_dst.numel() * 4
    floor["library_copy_codes"] = {"bytes_moved": int(nb), "us": round(t_copy * 1e6, 2),
                                   "GBps": round(nb / t_copy / 1e9, 1)}
    del codes_dst
    # the streaming floor: one launch that only reads the qkv layer's packed codes
    # (13.1 MB, rotating copies), shaped like the GEMV's weight stream
    sink_t = torch.zeros((4,), dtype=torch.int32, device=dev)

    def read_codes():
        tl.read_probe(qkv[kq[0] % len(qkv)][0], sink_t)
        kq[0] += 1
    t_read = run_time(read_codes, n=DEC_LAYERS * 4) * 1e-3
    nb = qkv[0][0].numel() * 4
    floor["read_codes"] = {"bytes": int(nb), "us": round(t_read * 1e6, 2), "GBps": round(nb / t_read / 1e9, 1),
                           "kernel": "read_probe"}
    # Diagnostic only, never a headline figure: the same launches over ONE weight
    # copy, so that after the first launch the 13.9 MB are served by the 256 MB
    # Infinity Cache (MALL) instead of HBM.  If the warm time is close to the cold
    # one, the launch is held back by its own latency and issue, not by HBM.
    warm = {"note": "diagnostic: qkv GEMV and read probe re-reading one weight copy (MALL-resident), "
                    "not HBM-bound; never the headline"}
    packed0, scales0 = qkv[0][0], qkv[0][1]
    for b in DECODE_BS:
        warm[f"gemv_b{b}_us"] = round(run_time(lambda: tl.gemv_prepared(ws_dec[b], b, Kq, packed0, scales0,
                                                                         y_dec[b]), n=DEC_LAYERS * 4) * 1e3, 2)
    warm["read_codes_us"] = round(run_time(lambda: tl.read_probe(packed0, sink_t), n=DEC_LAYERS * 4) * 1e3, 2)
    # the matrix-core floor: one launch of back-to-back int8 32x32x32 MFMAs on every
    # SIMD (two waves each, eight independent chains per wave), no memory traffic,
    # with constant operands and with random ones; the GEMM's own rate compares
    # with the random figure, since its operands are random int8 too
    mf_iters = 2000
    mf_ops = MFMA_PROBE_GRID * 4 * mf_iters * 8 * 2 * 32 * 32 * 32
    mfma_ceiling = {"ops_per_launch": int(mf_ops)}
    for name, rnd in (("constant", False), ("random", True)):
        t_m = run_time(lambda: tl.mfma_probe(rnd, mf_iters, sink_t), n=5) * 1e-3
        mfma_ceiling[name] = {"us": round(t_m * 1e6, 1), "TOPs": round(mf_ops / t_m / 1e12, 1),
                              "frac_of_peak": round(mf_ops / t_m / 1e12 / INT8_PEAK_TOPS, 4),
                              "kernel": "mfma_probe_" + name}
    # the whole decode layer from the raw bf16 input (rotation, limbs, GEMV): one
    # launch for b <= 2 at this shape, else the fused rotation + limb prep and the GEMV
    layer = {}
    for b in DECODE_BS:
        kl = [0]

        def one_layer():
            packed, scales, _, _ = qkv[kl[0] % len(qkv)]
            kl[0] += 1
            tl.gemv_ternary_x(x_dec[b], packed, scales, out=y_dec[b], workspace=ws_dec[b])
        t_l = run_time(one_layer, n=DEC_LAYERS * 4) * 1e-3
        nbytes = gemv_bytes(b, Kq, Nq)   # bf16 input: 2 b K bytes, as many as the limbs
        layer[str(b)] = {"us": round(t_l * 1e6, 2), "GBps": round(nbytes / t_l / 1e9, 1),
                         "frac": round(nbytes / t_l / 1e9 / HBM_PEAK_GBS, 4),
                         "path": tl.last_kernel_name() if tl.last_kernel_name().startswith("gemv_rot")
                         else "gemv_prep_x + " + tl.last_kernel_name()}
    gc.enable()

    if os.environ.get("BENCH_DEBUG"):
        for k, v in gemm_ms.items():
            log(f"per-step ms {k}: {[round(x, 4) for x in v]}")
    by_b = {}
    tot_bytes = tot_s = 0.0
    for b in DECODE_BS:
        t = float(np.mean(gemv_ms[b])) * 1e-3
        nbytes = gemv_bytes(b, Kq, Nq)
        by_b[str(b)] = {"us": round(t * 1e6, 3), "GBps": round(nbytes / t / 1e9, 1),
                        "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "kernel": kernel_names[("gemv", b)],
                        "bytes": nbytes, **spread(gemv_ms[b], gemv_runs[b])}
        tot_bytes += nbytes
        tot_s += t
    dec_gbs = tot_bytes / tot_s / 1e9

    pre_out = {}
    ops_tot = t_tot = 0.0
    for name in ("gate_up", "down"):
        t = float(np.mean(gemm_ms[name])) * 1e-3
        ops = 2.0 * PREFILL_M * pre[name]["K"] * pre[name]["N"]
        pre_out[name] = {"us": round(t * 1e6, 2), "TOPs": round(ops / t / 1e12, 1),
                         "frac": round(ops / t / 1e12 / INT8_PEAK_TOPS, 4), "kernel": kernel_names[("gemm", name)],
                         **spread(gemm_ms[name], gemm_runs[name])}
        ops_tot += ops
        t_tot += t
    pre_tops = ops_tot / t_tot / 1e12

    traffic = load_traffic()
    gemv_traffic = gemm_traffic = None
    if "gemv" in traffic and all(str(b) in traffic["gemv"] for b in DECODE_BS):
        for b in DECODE_BS:
            by_b[str(b)]["traffic_bytes"] = traffic["gemv"][str(b)]["traffic_bytes"]
        gemv_traffic = round(float(np.mean([traffic["gemv"][str(b)]["traffic_bytes"] for b in DECODE_BS])))
    if "gemm" in traffic and all(k in traffic["gemm"] for k in pre_out):
        for k in pre_out:
            pre_out[k]["traffic_bytes"] = traffic["gemm"][k]["traffic_bytes"]
        gemm_traffic = round(float(np.mean([traffic["gemm"][k]["traffic_bytes"] for k in pre_out])))

    pre_k = {k: P["K"] for k, P in pre.items()}
    stack = None
    if not args.no_stack:
        del qkv, gate_up, down, pre
        torch.cuda.empty_cache()
        log("stack64: packing 256 layers")
        stack = stack_pass(tl, torch, dev, args.stack_steps, log)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle decode qkv b=16, prefill gate_up and down M=512")
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "decode GEMV HBM GB/s (% of peak) at 5120→10240 b=1..16; prefill int8 TOPS",
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"ternary linear layer: decode qkv K=5120 N=10240 at b=1,4,8,16 "
                               f"({DEC_LAYERS} layers per pass) + prefill M=512 gate_up 5120->34816 and "
                               f"down 17408->5120 ({PRE_LAYERS} layers each)",
                   "decode_b": list(DECODE_BS), "prefill_tokens": PREFILL_M,
                   "rotating_weight_bytes": ROTATE_BYTES},
        "decode_gemv_by_b": by_b,
        "gemv_vs_read_floor": vs_floor,
        "rotation_only": rot_only,
        "input_kernels_GBps": {
            "decode_rotate_prep": {str(b): round((2 * b * Kq + 2 * b * Kq + 4 * b) / (float(np.mean(prep_ms[b])) * 1e-3) / 1e9, 1)
                                   for b in DECODE_BS},
            "prefill_rotate_quant_m512": {k: round((3 * PREFILL_M * pre_k[k] + 4 * PREFILL_M) /
                                                   (float(np.mean(v)) * 1e-3) / 1e9, 1)
                                          for k, v in quant_ms.items()}},
        "launch_floor": floor,
        "warm_mall_diagnostic": warm,
        "mfma_ceiling": mfma_ceiling,
        "input_kernels_us": {
            "decode_rotate_prep": {str(b): round(float(np.mean(prep_ms[b])) * 1e3, 2) for b in DECODE_BS},
            "prefill_rotate_quant_m512": {k: round(float(np.mean(v)) * 1e3, 2) for k, v in quant_ms.items()},
            "split_block_stages": split_us},
        "prefill_tops": round(pre_tops, 1),
        "prefill_gemm": pre_out,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": gemv_traffic,
                     "algorithmic_bytes_per_launch": round(float(np.mean([gemv_bytes(b, Kq, Nq) for b in DECODE_BS]))),
                     "kernel": "GEMV weight stream (" + ", ".join(sorted({v["kernel"] for v in by_b.values()})) + ")"},
        "roofline_prefill": {"bound": "mfma", "achieved": round(pre_tops, 1), "peak": INT8_PEAK_TOPS,
                             "unit": "TOP/s", "frac": round(pre_tops / INT8_PEAK_TOPS, 4), "traffic": gemm_traffic},
        "stack64": stack,
        "cpu_baseline": cpu,
    }
    out["decode_layer"] = layer
    out["gate"] = roofline_gate(out)
    print(json.dumps(out), flush=True)


def library_reference(tl, torch, dev, n=20):
    """torch._int_mm (int8 x int8 -> int32 on the vendor GEMM library; the call [P1] §4
    makes after expanding the weights to int8 each step) against tl_gemm_int8_rescale
    (2-bit weights expanded in registers, rescale fused) at the same shapes.  Weights
    rotate over copies beyond the Infinity Cache; n launches behind a device spin
    between two HIP events.  _int_mm gets its int8 weight matrix ready-made (its
    expansion is not timed) and writes int32; ours writes bf16 after the rescale."""
    import synth
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        torch.cuda._sleep(3_000_000)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3
    for (M, K, N) in ((512, 5120, 34816), (512, 17408, 5120), (2048, 5120, 34816), (4096, 8192, 8192)):
        L = synth.LayerInputs(0, S_PRE, 1, K, N)
        codes = L.codes_torch(dev)
        scales = torch.from_numpy(L.scales()).to(dev)
        packed, q, rs = tl.pack_weights(codes, scales)
        del codes
        R = max(2, min(12, math.ceil(ROTATE_BYTES / (N * K))))
        w8 = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev).t() for _ in range(R)]
        ours = [(packed, q, rs)] + [(packed.clone(), q.clone(), rs.clone()) for _ in range(R - 1)]
        xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        sx = torch.rand(M, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_lib = timed(lambda i: torch._int_mm(xq, w8[i % R]))
        t_tl = timed(lambda i: tl.gemm_int8_rescale(xq, sx, *ours[i % R], out=y))
        ops = 2.0 * M * N * K
        print(json.dumps({"M": M, "K": K, "N": N, "torch_int_mm_us": round(t_lib, 1),
                          "torch_int_mm_TOPs": round(ops / t_lib / 1e6, 1), "tl_gemm_us": round(t_tl, 1),
                          "tl_gemm_TOPs": round(ops / t_tl / 1e6, 1), "tl_kernel": tl.last_kernel_name()}), flush=True)
        del w8, ours, packed, q, rs
        torch.cuda.empty_cache()


SWEEP_BS = (1, 2, 4, 8, 12, 16, 20, 24, 32, 40, 48, 64, 96, 128, 192, 256, 384, 512)
SWEEP_SHAPES = (("qkv", "decode_qkv", 0, 5120, 10240), ("gate_up", "decode_mlp", 0, 5120, 34816),
                ("down", "decode_mlp", 1, 17408, 5120))


def bsweep(tl, torch, dev, log, n=20):
    """Whole-layer time from the raw bf16 input, per token count T, for the two paths:
    'gemv' = rotation fused into the limb prep, then the two-limb GEMV (T <= 64);
    'int8' = rotation fused into the per-token int8 quantisation, then the int8 GEMM
    + rescale.  Each point: n back-to-back layers over rotating weight copies,
    queued behind a device-side spin, between two HIP events on the launch stream.
    Prints one JSON line per (shape, T) and one per shape with the crossover."""
    import gc

    import synth
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    bf16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    # the spin must outlast the host's issue of n layers (two binding calls each)
    e0, e1 = ev(), ev()
    e0.record(stream)
    torch.cuda._sleep(1_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    spin_ms_per_m = e0.elapsed_time(e1)
    spin = int(1_000_000 * (n * 0.2) / spin_ms_per_m)      # about 200 us of device spin per layer
    print(json.dumps({"spin_cycles": spin, "spin_ms": round(spin * spin_ms_per_m / 1e6, 2)}), flush=True)
    for name, wl, li, K, N in SWEEP_SHAPES:
        stream = synth.WORKLOADS[wl]["stream"]
        L = synth.LayerInputs(0, stream, li, K, N)
        codes = L.codes_torch(dev)
        scales = torch.from_numpy(L.scales()).to(dev)
        packed, q, rs = tl.pack_weights(codes, scales)
        del codes
        per = packed.numel() * 4 + scales.numel() * 2 + q.numel() + rs.numel() * 4
        R = max(2, math.ceil(ROTATE_BYTES / per))
        copies = [(packed, scales, q, rs)] + [(packed.clone(), scales.clone(), q.clone(), rs.clone())
                                              for _ in range(R - 1)]
        x_all = bf16(synth.activations(0, stream, 100 + li, max(SWEEP_BS), K))
        rows = []
        for T in SWEEP_BS:
            x = x_all[:T]
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            xq = torch.empty((T, K), dtype=torch.int8, device=dev)
            sx = torch.empty((T,), dtype=torch.float32, device=dev)
            ws = (torch.empty((tl.gemv_workspace_size(T, K, N),), dtype=torch.uint8, device=dev)
                  if T <= 64 else None)
            rot = [0]

            def nxt():
                c = copies[rot[0] % len(copies)]
                rot[0] += 1
                return c

            def gemv():
                pk, sc, _, _ = nxt()
                tl.gemv_ternary_x(x, pk, sc, out=y, workspace=ws)

            def int8():
                pk, _, qq, r = nxt()
                tl.quant_act_int8_x(x, xq=xq, tok_scale=sx)
                tl.gemm_int8_rescale(xq, sx, pk, qq, r, out=y)

            lws = torch.zeros((tl.linear_workspace_size(T, K, N),), dtype=torch.uint8, device=dev)

            def linear():
                pk, sc, qq, r = nxt()
                tl.linear_apply(x, pk, sc, qq, r, out=y, workspace=lws)

            row = {"shape": name, "K": K, "N": N, "T": T,
                   "path": "gemv" if tl.linear_path(T, K, N) == tl.PATH_GEMV else "int8"}
            for pname, fn in (("gemv", gemv), ("int8", int8), ("linear", linear)):
                if pname == "gemv" and ws is None:
                    continue
                fn()
                torch.cuda.synchronize()
                gc.disable()
                e0, e1 = ev(), ev()
                torch.cuda._sleep(spin)
                e0.record(stream)
                h0 = time.perf_counter()
                for _ in range(n):
                    fn()
                host_us = (time.perf_counter() - h0) / n * 1e6
                e1.record(stream)
                torch.cuda.synchronize()
                gc.enable()
                row[pname + "_us"] = round(e0.elapsed_time(e1) / n * 1e3, 2)
                row[pname + "_host_us"] = round(host_us, 1)   # issue pace; the spin covers it
            row["faster"] = "gemv" if row.get("gemv_us", 1e30) <= row["int8_us"] else "int8"
            del lws
            rows.append(row)
            print(json.dumps(row), flush=True)
        gemv_wins = [r["T"] for r in rows if r["faster"] == "gemv"]
        print(json.dumps({"shape": name, "K": K, "N": N,
                          "gemv_faster_up_to": max(gemv_wins) if gemv_wins else 0,
                          "gemv_faster_at": gemv_wins}), flush=True)
        log(f"bsweep {name} done")
        del copies, packed, scales, q, rs
        torch.cuda.empty_cache()


def stack_pass(tl, torch, dev, steps, log):
    """64 synthetic decoder blocks x (qkv, o, gate_up, down), weights resident in HBM.

    One activation tensor per layer type is shared by the 64 blocks (the layers do
    not chain).  Decode pass: per type, rotation + GEMV prep once, then the 64
    GEMVs (b = 16).  Prefill pass: per type, rotation + quantisation of a
    2048-token chunk once, then the 64 GEMMs.  Reported: GB/s of the GEMV launches
    and TOP/s of the GEMM launches (events around each type's 64 launches), and
    the whole-pass times.
    """
    import synth
    types = [(name, K, N) for name, K, N in synth.WORKLOADS["stack64"]["layers"]]
    blocks = synth.WORKLOADS["stack64"]["blocks"]
    s_stack = synth.WORKLOADS["stack64"]["stream"]
    layers = []
    packed_bytes = 0
    for blk in range(blocks):
        for ti, (name, K, N) in enumerate(types):
            L = synth.LayerInputs(0, s_stack, 4 * blk + ti, K, N)
            codes = L.codes_torch(dev)
            scales = torch.from_numpy(L.scales()).to(dev)
            packed, q, rs = tl.pack_weights(codes, scales)
            del codes
            layers.append((ti, packed, scales, q, rs))
            packed_bytes += packed.numel() * 4 + scales.numel() * 2 + q.numel() + rs.numel() * 4
    torch.cuda.synchronize()
    bf16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    B, M = 16, 2048
    io = []
    for ti, (name, K, N) in enumerate(types):
        io.append(dict(K=K, N=N, xd=bf16(synth.activations(0, s_stack, ti, B, K)),
                       xp=bf16(synth.activations(0, s_stack, len(types) + ti, M, K)),
                       ws=torch.empty((tl.gemv_workspace_size(B, K, N),), dtype=torch.uint8, device=dev),
                       yd=torch.empty((B, N), dtype=torch.bfloat16, device=dev),
                       xq=torch.empty((M, K), dtype=torch.int8, device=dev),
                       sx=torch.empty((M,), dtype=torch.float32, device=dev),
                       yp=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def decode(rec):
        for ti, P in enumerate(io):
            tl.gemv_prepare_x(P["xd"], P["ws"])
            e0, e1 = ev(), ev()
            e0.record(stream)
            for lt, packed, scales, q, rs in layers:
                if lt == ti:
                    tl.gemv_prepared(P["ws"], B, P["K"], packed, scales, P["yd"])
            e1.record(stream)
            rec.append((e0, e1))

    def prefill(rec):
        for ti, P in enumerate(io):
            tl.quant_act_int8_x(P["xp"], xq=P["xq"], tok_scale=P["sx"])
            e0, e1 = ev(), ev()
            e0.record(stream)
            for lt, packed, scales, q, rs in layers:
                if lt == ti:
                    tl.gemm_int8_rescale(P["xq"], P["sx"], packed, q, rs, out=P["yp"])
            e1.record(stream)
            rec.append((e0, e1))

    out = {"blocks": blocks, "layers": len(layers), "weight_bytes": packed_bytes}
    import gc
    gc.collect()
    gc.disable()
    for name, fn in (("decode_b16", decode), ("prefill_m2048", prefill)):
        fn([])
        torch.cuda.synchronize()
        rec = []
        t0, t1 = ev(), ev()
        t0.record(stream)
        for _ in range(steps):
            fn(rec)
        t1.record(stream)
        torch.cuda.synchronize()
        kern_s = sum(a.elapsed_time(b) for a, b in rec) / steps * 1e-3
        pass_ms = t0.elapsed_time(t1) / steps
        if name == "decode_b16":
            nbytes = sum(P["N"] * P["K"] // 4 + P["N"] * (P["K"] // 128) * 2 + 2 * B * P["K"] + 2 * B * P["N"]
                         for ti, P in enumerate(io) for lt, *_ in layers if lt == ti)
            out[name] = {"gemv_GBps": round(nbytes / kern_s / 1e9, 1), "gemv_ms": round(kern_s * 1e3, 3),
                         "pass_ms": round(pass_ms, 3), "bytes": nbytes,
                         "frac": round(nbytes / kern_s / 1e9 / HBM_PEAK_GBS, 4)}
        else:
            ops = sum(2.0 * M * P["K"] * P["N"] for ti, P in enumerate(io) for lt, *_ in layers if lt == ti)
            out[name] = {"gemm_TOPs": round(ops / kern_s / 1e12, 1), "gemm_ms": round(kern_s * 1e3, 3),
                         "pass_ms": round(pass_ms, 3), "ops": ops,
                         "frac": round(ops / kern_s / 1e12 / INT8_PEAK_TOPS, 4)}
        log(f"stack64 {name}: {out[name]}")
    gc.enable()
    return out


PHASES = ("issue", "direct_wait", "barrier", "first_pair", "other_pairs", "to_reduction")


def phase_stamps(tl, torch, dev, layers, bf16, synth):
    """Per-wave phase times of the decode GEMV from the instrumented library.

    Each launch group is DEC_LAYERS back-to-back launches over rotating weight
    copies behind a device spin; every launch writes its waves' records (8 words
    each, see the kernel) and those of the last launch remain and are read.  Phases per wave, in µs:
    entry -> every load issued -> direct loads waited for -> barrier passed ->
    first pair computed -> last pair computed -> stamps stored (the reduction
    follows); plus the spread of entries and of the waves' output stores (each
    wave adds and stores its share of the workgroup's outputs) across the grid.  The clock is the 100 MHz constant-rate counter."""
    import ctypes
    L = tl.lib()
    L.tl_phase_stamps_set.argtypes = [ctypes.c_void_p]
    L.tl_phase_stamps_set.restype = ctypes.c_int
    buf = torch.zeros((4 * 4096 * 16 * 8,), dtype=torch.int64, device=dev)
    out = {}
    for name, (copies, K, N) in layers.items():
        for b in DECODE_BS:
            x = bf16(synth.activations(0, S_DEC, 0, b, K))
            ws = torch.empty((tl.gemv_workspace_size(b, K, N),), dtype=torch.uint8, device=dev)
            y = torch.empty((b, N), dtype=torch.bfloat16, device=dev)
            tl.gemv_prepare_x(x, ws)
            times, recs = [], []
            for rep in range(5):
                buf.zero_()
                torch.cuda.synchronize()
                assert L.tl_phase_stamps_set(ctypes.c_void_p(buf.data_ptr())) == 0
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(2_000_000)
                e0.record()
                for i in range(DEC_LAYERS):   # every launch writes the records; the last one's remain
                    p, s = copies[(rep * DEC_LAYERS + i) % len(copies)][:2]
                    tl.gemv_prepared(ws, b, K, p, s, y)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3 / DEC_LAYERS)
                a = buf.view(-1, 8).cpu().numpy()
                recs.append(a[a[:, 0] > 0])
            kname = tl.last_kernel_name()
            a = recs[-1]
            t0 = a[:, 0].min()
            t = (a[:, :7].astype(np.float64) - t0) / 100.0           # µs from the first wave's entry
            dur = np.diff(t[:, :6], axis=1)                             # five phases per wave
            tail = t[:, 5]                                              # stamps stored: reduction starts
            w0 = t[:, 6][a[:, 6] > 0]                                   # each wave: its outputs stored
            xcc = ((a[:, 7] >> 32) & 0xF).astype(np.int64)
            out[f"{name}_b{b}"] = {
                "kernel": kname, "event_us": round(float(np.median(times)), 2), "waves": int(len(a)),
                "phase_median_us": {ph: round(float(np.median(dur[:, k])), 2) for k, ph in enumerate(PHASES[:5])},
                "entry_p10_p50_p90": [round(float(np.percentile(t[:, 0], q)), 2) for q in (10, 50, 90)],
                "reduction_start_p10_p50_p90": [round(float(np.percentile(tail, q)), 2) for q in (10, 50, 90)],
                "outputs_stored_p50_p90_max": [round(float(np.percentile(w0, q)), 2) for q in (50, 90)] +
                                              [round(float(w0.max()), 2)],
                "waves_per_xcd": np.bincount(xcc, minlength=8).tolist()}
            print(f"[stamps] {name} b={b} {kname}: {out[f'{name}_b{b}']}", file=sys.stderr, flush=True)
    assert L.tl_phase_stamps_set(ctypes.c_void_p(0)) == 0
    print(json.dumps({"phase_stamps": out}))


def host_info():
    """CPU model and the cores this process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": int(avail), "os_cpu_count": os.cpu_count()}


def _timed(fn, seconds, max_reps=1000):
    """Mean wall time of fn over repeats filling about `seconds` (at least one)."""
    reps, t = 0, 0.0
    while reps == 0 or (t < seconds and reps < max_reps):
        s = time.perf_counter()
        fn()
        t += time.perf_counter() - s
        reps += 1
    return t / reps, reps


def cpu_baseline(seconds):
    """The oracle (numpy binary64, as it stands) on the bench's workloads, on the host:
    decode qkv at b = 16 (rotation + GEMV) and the 512-token prefill of gate_up and
    down (rotation, per-token int8, int GEMM, rescale; the scale decomposition is
    load-time work, not timed, as on the GPU), with every BLAS thread and with one.
    The one-thread prefill runs on the first 64 tokens of the chunk (a bounded
    sample; rates are per token and so comparable)."""
    import threadpoolctl

    import oracle
    import synth
    blas = [i for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas"]
    threads = max(i["num_threads"] for i in blas) if blas else (os.cpu_count() or 1)
    L = synth.LayerInputs(0, S_DEC, 0, 5120, 10240)
    codes, scales = L.codes(), L.scales()
    x = synth.bf16_bits_to_f32(L.x(16))

    def dec():
        oracle.gemv_ternary(oracle.rotate_exact(x), codes, scales)
    dec_all, reps_all = _timed(dec, seconds * 0.3)
    with threadpoolctl.threadpool_limits(1):
        dec_one, reps_one = _timed(dec, seconds * 0.1)
    del codes, scales
    db = gemv_bytes(16, 5120, 10240)
    prefill = {}
    for name, li, K, N in (("gate_up", 0, 5120, 34816), ("down", 1, 17408, 5120)):
        Lp = synth.LayerInputs(0, S_PRE, li, K, N)
        pc, ps = Lp.codes(), Lp.scales()
        q, rs, _ = oracle.decompose_scales(ps)
        xp = synth.bf16_bits_to_f32(synth.activations(0, S_PRE, li, PREFILL_M, K))

        def pre(xs):
            xq, sx = oracle.quant_act_int8(oracle.rotate_f32(xs))
            oracle.rescale(oracle.gemm_int8_acc(xq, pc, q), rs, sx)
        t_all, _ = _timed(lambda: pre(xp), 0.0)
        with threadpoolctl.threadpool_limits(1):
            t_one, _ = _timed(lambda: pre(xp[:64]), 0.0)
        prefill[name] = {"all_threads_s": round(t_all, 3),
                         "all_threads_TOPs": round(2.0 * PREFILL_M * N * K / t_all / 1e12, 4),
                         "one_thread_s_64_tokens": round(t_one, 3),
                         "one_thread_TOPs": round(2.0 * 64 * N * K / t_one / 1e12, 4)}
        del pc, ps, q, rs, xp
    return {"value": round(db / dec_all / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"decode qkv K=5120 N=10240 b=16 (rotation + GEMV), {reps_all} reps, "
                      f"{dec_all * 1e3:.1f} ms each, on {threads} BLAS threads; prefill M=512 gate_up and "
                      f"down once each (one thread: 64 tokens)",
            "one_thread": {"value": round(db / dec_one / 1e9, 3), "unit": "GB/s", "cores": 1, "reps": reps_one,
                           "ms": round(dec_one * 1e3, 1)},
            "prefill_m512": prefill, "host": host_info()}


if __name__ == "__main__":
    main()
