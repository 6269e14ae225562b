"""Benchmark: fused attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole hot path over one batch of synthetic input already in
HBM: forward (O, LSE), backward preparation (segment metadata when present,
Delta), dK/dV and dQ.  Prints one JSON line:

  value      algorithmic fwd+bwd TFLOP/s, F = 2 n (4 Dqk + 3 Dv) with n the
             number of allowed (query, key) pairs over batch rows and query
             heads (masked pairs are not counted)
  roofline   the slowest kernel of the step against the bf16 dense MFMA peak
             (2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096 FLOP/clk); its time is
             the average of HIP events recorded around its launch on the
             stream it runs on
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
             (a few query heads), timed on the host cores

The workload is the 8K causal GQA configuration unless --workload says
otherwise; the others are parity-test cases.  Only one GPU is used.
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
sys.path.insert(0, ROOT)

from bwd_packed_segments_amd import inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_BYTES = 8.0e12
PEAK_FP32_TFLOPS = 157.3
METRIC = "fwd+bwd attention TFLOP/s (bf16) and % of MI355X MFMA peak, 1 GPU"
DEFAULT_WORKLOAD = "gqa_causal_8k"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["bps_common.hpp", "lds_tile.hpp", "attn_kernels.hpp", "dkdv_gs.hpp", "fwd_pp.hpp", "dq_hp.hpp", "attn_inst.hip"]


# ------------------------------------------------------------------ counting

def allowed_pairs(w, segments) -> int:
    """Number of allowed (query, key) pairs summed over batch rows and query
    heads, counted from the metadata directly."""
    if segments is None:
        if w.causal:
            per_row = w.Sq * (w.Sq + 1) // 2
        else:
            per_row = w.Sq * w.Skv
        return w.B * w.Hq * per_row
    ids_q = np.asarray(segments["ids_q"])
    pos_q = segments.get("pos_q")
    ids_kv = segments.get("ids_kv")
    if ids_kv is None:
        ids_kv, pos_kv = ids_q, pos_q
    else:
        ids_kv = np.asarray(ids_kv)
        pos_kv = segments.get("pos_kv")
    total = 0
    for b in range(w.B):
        for s in np.unique(ids_q[b]):
            if s == 0:
                continue
            qi = np.nonzero(ids_q[b] == s)[0]
            kj = np.nonzero(ids_kv[b] == s)[0]
            if not w.causal:
                total += qi.size * kj.size
            else:
                kp = np.sort(np.asarray(pos_kv)[b, kj])
                qp = np.asarray(pos_q)[b, qi]
                total += int(np.searchsorted(kp, qp, side="right").sum())
    return total * w.Hq


def flops(w, n):
    return {
        "fwd": 2.0 * n * (w.Dqk + w.Dv),
        "bwd": 2.0 * n * (3 * w.Dqk + 2 * w.Dv),
        # per kernel: the contractions each one must do over allowed pairs
        "k_fwd": 2.0 * n * (w.Dqk + w.Dv),
        "k_dkdv": 2.0 * n * (2 * w.Dqk + 2 * w.Dv),
        "k_dq": 2.0 * n * (2 * w.Dqk + w.Dv),
    }


def kernel_core_bytes(w):
    """Algorithmic HBM bytes per launch of each kernel without variants:
    every tensor it must read or write, once."""
    es = 2 if w.dtype == "bf16" else 4
    q = w.B * w.Sq * w.Hq * w.Dqk * es
    o = w.B * w.Sq * w.Hq * w.Dv * es
    k = w.B * w.Skv * w.Hkv * w.Dqk * es
    v = w.B * w.Skv * w.Hkv * w.Dv * es
    row = w.B * w.Hq * w.Sq * 4
    return {"attn_fwd": q + k + v + o + row,
            "attn_bwd_dkdv": q + o + k + v + 2 * row + k + v,
            "attn_bwd_dq": q + o + k + v + 2 * row + q}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bwd_packed_segments_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(f"{kernel}:{workload}")
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


# ------------------------------------------------------------------ GPU timing

VARIANT_SOFTCAP = 50.0


def variant_tensors(w, variant, seed=0):
    """Device inputs of the requested variants (bias [B, Hq, Sq, Skv] of the
    workload's dtype, soft-cap value, sink logits [Hq]); seeded like the
    rest of the inputs."""
    import torch
    if not variant:
        return {}
    if "bias" in variant and w.B * w.Hq * w.Sq * w.Skv > (1 << 30):
        raise SystemExit(f"--variant bias: a [B, Hq, Sq, Skv] bias of {w.name} has more than 2^30 elements; "
                         "use a smaller workload (e.g. bshd_causal_2k)")
    vi = inputs.variant_inputs(w, seed, bias_batch=w.B if "bias" in variant else None, sink="sink" in variant)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {"softcap": VARIANT_SOFTCAP if "softcap" in variant else 0.0, "max_logit": "max_logit" in variant}
    out["bias"] = torch.from_numpy(vi["bias"]).to("cuda").to(dt) if vi["bias"] is not None else None
    out["sink"] = torch.from_numpy(vi["sink"]).to("cuda") if vi["sink"] is not None else None
    return out


def run_gpu(w, steps, warmup, seed=0, variant=(), flags=0, serial_bwd=False):
    import torch
    import bwd_packed_segments_amd as bps

    case = inputs.make_case(w, seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {k: torch.from_numpy(case[k]).to("cuda").to(dt) for k in ("q", "k", "v", "do")}
    vt = variant_tensors(w, variant, seed)
    fwd_var = {k: vt[k] for k in ("bias", "softcap", "sink", "max_logit")} if vt else {}
    bwd_var = {k: vt[k] for k in ("bias", "softcap", "sink")} if vt else {}
    seg = None
    if case["segments"] is not None:
        sg = case["segments"]

        def t(x):
            return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")
        seg = bps.Segments(t(sg["ids_q"]), t(sg.get("pos_q")), t(sg.get("ids_kv")), t(sg.get("pos_kv")))
    fwd = bps.FwdPlan(dev["q"], dev["k"], dev["v"], causal=w.causal, segments=seg, flags=flags & ~bps.ATTN_FUSED_BWD,
                      **fwd_var)
    bwd = bps.BwdPlan(dev["q"], dev["k"], dev["v"], fwd.o, fwd.lse, dev["do"], causal=w.causal, segments=seg,
                      flags=flags, **bwd_var)
    stream = torch.cuda.current_stream()
    # dK/dV and dQ read the prepared workspace and write different outputs,
    # so they may run at the same time (not under ATTN_FUSED_BWD, where dQ
    # sums the partials dK/dV writes): dQ on a second stream of default
    # priority, joined before the step ends.  Each fills the CUs the other's
    # last workgroups leave idle.
    can_overlap = not serial_bwd and not (flags & bps.ATTN_FUSED_BWD)
    side = torch.cuda.Stream() if can_overlap else None
    forked = torch.cuda.Event() if can_overlap else None
    joined = torch.cuda.Event() if can_overlap else None
    concurrent = False

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fwd.run()
        if ev is not None:
            ev[1].record(stream)
        bwd.run(bps.ATTN_BWD_PREPARE)
        if ev is not None:
            ev[2].record(stream)
        if concurrent:
            forked.record(stream)
            side.wait_event(forked)
            with torch.cuda.stream(side):
                if ev is not None:
                    ev[5].record(side)
                bwd.run(bps.ATTN_BWD_DQ)
                if ev is not None:
                    ev[6].record(side)
                joined.record(side)
            bwd.run(bps.ATTN_BWD_DKDV)
            if ev is not None:
                ev[3].record(stream)
            stream.wait_event(joined)
            if ev is not None:
                ev[4].record(stream)
            return
        bwd.run(bps.ATTN_BWD_DKDV)
        if ev is not None:
            ev[3].record(stream)
        bwd.run(bps.ATTN_BWD_DQ)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(warmup):
        step()
    # Two legal schedules of the backward phases: one stream, or dQ beside
    # dK/dV.  Where the grids fill the GPU they take the same time and the
    # overlap only blurs each kernel's own launch time (the roofline), so
    # the second stream is used only when it is clearly faster here.
    schedule = None
    if can_overlap and warmup > 0:
        def timed(conc, n=4):
            nonlocal concurrent
            concurrent = conc
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            step()
            a.record(stream)
            for _ in range(n):
                step()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n
        t_ser = min(timed(False), timed(False))
        t_con = min(timed(True), timed(True))
        concurrent = t_con < 0.97 * t_ser
        schedule = {"one_stream_ms": round(t_ser, 4), "two_streams_ms": round(t_con, 4)}
    # The route each batch row took on the device (the metadata check may
    # send a row that the host requested on the fast route to the general
    # one); read once, before the timed region.
    rows = bps.route_counts(bwd.route_rows()) if warmup > 0 else None
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phases = {"fwd": [], "prepare": [], "dkdv": [], "dq": [], "step": []}
    for ev in events:
        phases["fwd"].append(ev[0].elapsed_time(ev[1]))
        phases["prepare"].append(ev[1].elapsed_time(ev[2]))
        phases["dkdv"].append(ev[2].elapsed_time(ev[3]))
        phases["dq"].append(ev[5].elapsed_time(ev[6]) if concurrent else ev[3].elapsed_time(ev[4]))
        phases["step"].append(ev[0].elapsed_time(ev[4]))
    avg = {k: float(np.mean(v)) for k, v in phases.items()}
    med = {k: float(np.median(v)) for k, v in phases.items()}
    if rows is None:
        rows = bps.route_counts(bwd.route_rows())
    return case, wall, avg, med, (fwd.route, rows), (2 if concurrent else 1, schedule)


def ring_bench(w, cp, steps, warmup, seed=0):
    """One JSON line for the ring emulation: algorithmic FLOP of the whole
    sequence over the time of attn_ring_fwd + attn_ring_bwd (cp x cp shard
    steps, the log-sum-exp merge and the gradient sums)."""
    import torch
    import bwd_packed_segments_amd as bps
    case = inputs.make_case(w, seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {k: torch.from_numpy(case[k]).to("cuda").to(dt) for k in ("q", "k", "v", "do")}
    seg = None
    if case["segments"] is not None:
        sg = case["segments"]

        def t(x):
            return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")
        seg = bps.Segments(t(sg["ids_q"]), t(sg.get("pos_q")), t(sg.get("ids_kv")), t(sg.get("pos_kv")))

    def step():
        o, lse = bps.attn_ring_fwd(dev["q"], dev["k"], dev["v"], cp=cp, causal=w.causal, segments=seg)
        bps.attn_ring_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cp=cp, causal=w.causal, segments=seg)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    n = allowed_pairs(w, case["segments"])
    F = flops(w, n)
    f_step = F["fwd"] + F["bwd"]
    value = f_step / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    print(json.dumps({"metric": METRIC + " (one-GPU ring emulation)", "value": round(value, 2), "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
                      "data": f"synthetic (seeded iid N(0,1) tensors, seed {seed})",
                      "config": {"workload": w.name, "ring_shards": cp, "allowed_pairs": n, "flop_per_step": f_step},
                      "pct_peak": round(100.0 * value / peak, 2)}))


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(w, case, n_alg_per_head_flops, budget_s=15.0):
    """The fp64 oracle (test infrastructure) on a sample of query heads of
    the same inputs, forward + backward, until about budget_s seconds.  When
    one head's dense score matrix is too large for the host (the long
    non-causal shard) the sample is also cut to the first query rows, which
    are independent of each other without a causal or segment mask."""
    import oracle
    rows_note = ""
    if w.meta == "none" and not w.causal and w.B * w.Sq * w.Skv > (1 << 26):
        rows = max(64, (1 << 26) // (w.B * w.Skv))
        case = dict(case)
        case["q"] = case["q"][:, :rows]
        case["do"] = case["do"][:, :rows]
        n_alg_per_head_flops = n_alg_per_head_flops * rows / w.Sq
        rows_note = f", first {rows} of {w.Sq} query rows"
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    heads = []
    t_total = 0.0
    h = 0
    while h < w.Hq and (t_total < budget_s or not heads):
        t0 = time.perf_counter()
        oracle.forward(case["q"], case["k"], case["v"], causal=w.causal, segments=case["segments"], heads=[h])
        oracle.backward(case["q"], case["k"], case["v"], case["do"], causal=w.causal, segments=case["segments"],
                        heads=[h])
        t_total += time.perf_counter() - t0
        heads.append(h)
        h += 1
        if t_total / len(heads) * (len(heads) + 1) > 2 * budget_s:
            break
    value = n_alg_per_head_flops * len(heads) / t_total / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{w.name}: forward+backward of {len(heads)} of {w.Hq} query heads "
                      f"(batch rows all{rows_note}), {t_total:.1f} s, fp64 NumPy",
            "cpu": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "seconds": t_total}


def cpu_model() -> str:
    """Model name of the host CPU (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ counter calibration

def copy_calibration(nbytes=1 << 30, reps=3):
    """A device copy of known size: each launch reads and writes nbytes, so
    the counters' per-dispatch readings for it give their scale factors."""
    import torch
    a = torch.ones(nbytes // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": nbytes, "copy_bytes_written_per_launch": nbytes,
                      "launches": reps}))


def ingest_counters(d, workload):
    """Writes the HBM-traffic record bench reports from four rocprofv3
    counter runs in directory d: C (FETCH_SIZE) and D (WRITE_SIZE) over a
    bench run of the workload, copyC / copyD the same counters over
    --copy-calibration.  Readings are KiB per dispatch; each counter's factor
    is the copy's true bytes over what the counter read for it."""
    import csv
    import re

    def per_kernel(tag):
        out = {}
        with open(os.path.join(d, f"{tag}_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                m = re.search(r"(attn_[a-z_]+?)(?:_ws|_gs|_pp|_hp)?_kernel", r["Kernel_Name"])
                name = m.group(1) if m else ("copy" if "copy" in r["Kernel_Name"] else None)
                if name:
                    out.setdefault(name, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in out.items()}

    copy_bytes = 1 << 30
    cf, cw = per_kernel("copyC")["copy"], per_kernel("copyD")["copy"]
    fetch_factor, write_factor = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    rec = {}
    if os.path.exists(TRAFFIC_FILE):   # records of other workloads are kept
        with open(TRAFFIC_FILE) as f:
            rec = {k: v for k, v in json.load(f).items() if not k.endswith(":" + workload)}
    rec.update({"_comment": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), "
                            "each scaled by what it read for a 1 GiB device copy; source_hash is "
                            "kernel_source_hash() of the sources the counters were taken on",
                "calibration": {"copy_bytes": copy_bytes, "fetch_kib_read": round(cf), "write_kib_read": round(cw),
                                "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4)}})
    fetch, write = per_kernel("C"), per_kernel("D")
    h = kernel_source_hash()
    for k in sorted(fetch):
        if k == "copy" or k not in write:
            continue
        fb, wb = fetch[k] * 1024 * fetch_factor, write[k] * 1024 * write_factor
        rec[f"{k}:{workload}"] = {"source_hash": h, "fetch_bytes": int(fb), "write_bytes": int(wb),
                                  "bytes_per_launch": int(fb + wb)}
    rec = {"_comment": rec.pop("_comment"), "calibration": rec.pop("calibration"), **dict(sorted(rec.items()))}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--ring", type=int, default=0, metavar="CP",
                    help="time the one-GPU ring emulation with CP shards (attn_ring_fwd + attn_ring_bwd) "
                         "instead of the plain entry points; same workload and FLOP count")
    ap.add_argument("--variant", default="",
                    help="comma list of attention variants to run through attn_fwd_ex / attn_bwd_ex: bias "
                         "(per-row [B, Hq, Sq, Skv] bias with its gradient), softcap (soft-capping at "
                         f"{VARIANT_SOFTCAP:g}), sink (sink logits with their gradient), max_logit")
    ap.add_argument("--fused-bwd", action="store_true",
                    help="time the single-pass backward (ATTN_FUSED_BWD): the dK/dV kernel also writes dQ "
                         "partials, the dQ phase sums them in key-tile order")
    ap.add_argument("--serial-bwd", action="store_true",
                    help="run the dK/dV and dQ phases one after the other on one stream (default: dQ on a second "
                         "stream beside dK/dV)")
    ap.add_argument("--force-general", action="store_true",
                    help="set ATTN_FORCE_GENERAL: run workloads with segment metadata on the general route even "
                         "where the fast route applies (what the fast path saves)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="no GPU work: read rocprofv3 FETCH_SIZE / WRITE_SIZE runs (C, D, copyC, copyD "
                         "counter_collection.csv in DIR) for --workload and write the traffic record")
    args = ap.parse_args()

    if args.ingest_counters:
        ingest_counters(args.ingest_counters, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration()
        return

    w = inputs.WORKLOADS[args.workload]
    t_setup = time.perf_counter()
    if args.ring:
        ring_bench(w, args.ring, args.steps, args.warmup)
        return
    variant = tuple(x for x in args.variant.split(",") if x)
    unknown = set(variant) - {"bias", "softcap", "sink", "max_logit"}
    if unknown:
        raise SystemExit(f"unknown --variant entries {sorted(unknown)}")
    if args.fused_bwd and set(variant) - {"sink", "max_logit"}:
        raise SystemExit("--fused-bwd takes no bias or soft cap")
    import bwd_packed_segments_amd as bps
    flags = (bps.ATTN_FUSED_BWD if args.fused_bwd else 0) | (bps.ATTN_FORCE_GENERAL if args.force_general else 0)
    case, wall, avg, med, (route_req, route_rows), (bwd_streams, schedule) = run_gpu(
        w, args.steps, args.warmup, variant=variant, flags=flags, serial_bwd=args.serial_bwd)
    route = next(iter(route_rows)) if len(route_rows) == 1 else "mixed"
    n = allowed_pairs(w, case["segments"])
    F = flops(w, n)
    f_step = F["fwd"] + F["bwd"]
    ms_per_step = wall / args.steps * 1e3
    value = f_step / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS

    kernels = {"attn_fwd": (avg["fwd"], F["k_fwd"]), "attn_bwd_dkdv": (avg["dkdv"], F["k_dkdv"]),
               "attn_bwd_dq": (avg["dq"], F["k_dq"])}
    if args.fused_bwd:
        # the dK/dV phase runs all five backward products; the dQ phase only
        # sums partials (bound by HBM, reported as its time in phase_ms)
        kernels = {"attn_fwd": (avg["fwd"], F["k_fwd"]), "attn_bwd_fused": (avg["dkdv"], F["bwd"])}
    dom = max(kernels, key=lambda k: kernels[k][0])
    ms_dom, f_dom = kernels[dom]
    achieved = f_dom / (ms_dom * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_for(dom, w.name) if not variant else None,
                "kernel": dom, "avg_ms": round(ms_dom, 4)}
    if "bias" in variant:
        # A bias adds one element read per allowed pair to the forward and
        # dQ kernels, and a read plus a dbias write to dK/dV: the dominant
        # kernel may then be bound by HBM instead of the matrix cores.
        es = 2 if w.dtype == "bf16" else 4
        core = kernel_core_bytes(w)
        extra = {"attn_fwd": n * es, "attn_bwd_dq": n * es, "attn_bwd_dkdv": 2 * n * es}
        hbm_bytes = core[dom] + extra[dom]
        t_mfma = f_dom / (peak * 1e12)
        t_hbm = hbm_bytes / PEAK_HBM_BYTES
        if t_hbm > t_mfma:
            gbs = hbm_bytes / (ms_dom * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                        "frac": round(gbs * 1e9 / PEAK_HBM_BYTES, 4), "traffic": None, "kernel": dom,
                        "avg_ms": round(ms_dom, 4), "alg_bytes": int(hbm_bytes),
                        "mfma_tflops": round(achieved, 2)}
        else:
            roofline["alg_bytes"] = int(hbm_bytes)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) tensors, seed 0)",
        "config": {"workload": w.name, "B": w.B, "Sq": w.Sq, "Skv": w.Skv, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Dqk": w.Dqk, "Dv": w.Dv, "causal": w.causal, "metadata": w.meta, "route": route,
                   "route_requested": route_req, "route_rows": route_rows,
                   "allowed_pairs": n, "flop_per_step": f_step,
                   "bwd_streams": bwd_streams, "bwd_schedule_probe_ms": schedule},
        "pct_peak": round(100.0 * value / peak, 2),
        "phase_ms": {k: round(v, 4) for k, v in avg.items()},
        "phase_ms_median": {k: round(v, 4) for k, v in med.items()},
        "roofline": roofline,
    }
    if variant:
        out["metric"] = METRIC + " (attention variants)"
        out["config"]["variants"] = {"list": list(variant), "softcap": VARIANT_SOFTCAP if "softcap" in variant else 0,
                                     "bias": "[B, Hq, Sq, Skv] per batch row, N(0,1)" if "bias" in variant else None}
        args.no_cpu_baseline = True      # the baseline line is the plain workload's
    if args.force_general:
        out["metric"] = out["metric"] + " (general route forced)"
        out["config"]["force_general"] = True
        args.no_cpu_baseline = True
    if args.fused_bwd:
        out["metric"] = out["metric"] + " (single-pass backward)"
        out["config"]["backward"] = "single pass: dK/dV kernel with dQ partials, then a key-tile-ordered dQ sum"
        args.no_cpu_baseline = True
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, case, f_step / w.Hq, args.cpu_seconds)
        cb.pop("seconds", None)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(f"# {w.name}: {value:.1f} TFLOP/s ({100 * value / peak:.1f}% of peak), {ms_per_step:.3f} ms/step; "
          f"phases {json.dumps(out['phase_ms'])}; setup+run {time.perf_counter() - t_setup:.1f}s", file=sys.stderr)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
