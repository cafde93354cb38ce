"""Throughput of the H2O chunk step on one MI355X.

A step is one h2o_chunk_step call on a full cache (the evicting regime of the
long bf16 stream: B=1, Hq=32, Hkv=8, D=128, C=32768 slots, chunks of T=2048):
attention with exact summed weights, score update, bottom-T selection with
replay log, and slot overwrite.  Inputs (cache state and a rotation of chunks)
are synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line.  `value` is chunk tokens per second; `roofline` covers
the dominant kernel (attention pass A) from its average launch duration
measured with HIP events on the launch stream over the timed region;
`cpu_baseline` times the fp64 oracle on a bounded sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
       [--no-cpu-baseline] [--calibrate-copy]
       python bench.py --traffic-from FETCH_DIR WRITE_DIR   (no GPU)

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
this script with --calibrate-copy (one collecting FETCH_SIZE, one WRITE_SIZE).
--calibrate-copy appends a plain elementwise copy of known size after the
timed region; the ratio of its known bytes to what each counter reads for it
scales the attention kernel's readings to bytes.  --traffic-from turns the
two counter folders into profiles/attn_a_traffic.json (tagged with a digest
of the kernel sources, so a stale record is ignored) and prints a summary.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
STEP_TARGET_FRAC = 0.60     # target for the whole evicting step, 6*D flops per visible pair
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector / matrix peak
PEAK_HBM_GBS = 8000.0
N_CHUNKS = 4                # distinct chunks rotated through the timed steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_a_traffic.json")
COPY_ELEMS = 64 << 20       # fp32 elements of the calibration copy (256 MiB each way)
COPY_REPS = 3


def dominant_kernel(w):
    """Name of pass A's kernel for a workload, as the profiler reports it."""
    if w.cache_fmt == "native" and w.D == 128 and w.dtype == "bf16":
        return "attn_a_native"
    return "attn_a_mfma"


def kernel_sources_digest():
    """Digest of the sources the measured pass-A kernel (attn_a_native) and
    its dispatch are built from; a stored HBM-traffic measurement is only
    reported while it still matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "h2o_kv_cache_sdpa_amd", "csrc")
    for name in ("attn_native.hip", "attn_mfma.hip", "tile_util.hpp", "device_util.hpp", "h2o_internal.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pairs_visible(B, Hq, T, n_occ):
    """(query head, key) pairs the softmax sees in one step."""
    return B * Hq * (T * n_occ + T * (T + 1) // 2)


def gemm_ceiling(dev, n=8192, reps=10):
    """The matrix rate this GPU sustains on a plain library GEMM (torch.matmul
    in bf16, n x n x n, hipBLASLt), for context beside the nominal peak: under
    a full matrix-core load the clock settles well below its maximum."""
    import torch
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"achieved": tf, "unit": "TFLOP/s", "frac_of_peak": tf / PEAK_BF16_TFLOPS,
            "how": f"torch.matmul bf16 {n}x{n}x{n}, mean of {reps} after 3 warm-up calls"}


def host_description(blas):
    """CPU model, logical CPUs and the BLAS the oracle's products run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {
        "cpu_model": model,
        "logical_cpus": os.cpu_count(),
        "usable_cpus": usable,
        "blas": [{"library": p.get("internal_api"), "version": p.get("version"),
                  "threads": p.get("num_threads"), "arch": p.get("architecture")} for p in blas],
        "threads_note": "matrix products run on the BLAS threads; exp and the other "
                        "elementwise numpy work on one thread",
    }


def cpu_baseline(w, max_groups=8):
    """Time the fp64 oracle on up to `max_groups` KV groups of one evicting
    step (about 10 s of host work for the 32K/2048 step, where 8 groups are
    the whole step) and scale to the whole step (the B*Hkv groups are
    independent)."""
    groups = min(max_groups, w.B * w.Hkv)
    import numpy as np
    from threadpoolctl import threadpool_info

    from h2o_kv_cache_sdpa_amd import workloads as W
    from oracle import h2o_oracle as O

    k, v, scores, _, _ = W.random_cache([w.cfg_id, 777], 1, groups, w.C, w.D, w.C, w.dtype, hh_frac=0.02)
    ch = W.random_chunk([w.cfg_id, 778], 1, groups * w.qg, groups, w.T, w.D, w.dtype, w.hh_new)
    scale = float(np.float32(1.0 / np.sqrt(w.D)))
    t0 = time.perf_counter()
    out, wsum, _ = O.attend_chunk(ch["q"].f64, k.f64, v.f64, w.C, ch["k"].f64, ch["v"].f64, scale)
    phi = O.update_scores(scores.astype(np.float64), wsum, w.C, w.C, w.T)
    O.bottom_t(phi, w.C, w.C, w.T)
    dt = time.perf_counter() - t0
    step_s = dt * (w.B * w.Hkv) / groups
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    return {
        "value": w.B * w.T / step_s,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "host": host_description(blas),
        "sample": f"{groups} of {w.B * w.Hkv} KV groups of one evicting step "
                  f"({w.qg} heads x {w.T} queries x {w.C + w.T} keys each) in {dt:.1f} s"
                  + (f", scaled by {w.B * w.Hkv / groups:g} to the full step" if groups < w.B * w.Hkv else ""),
    }


def _counter_rows(folder, counter):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def _short_kernel_name(name):
    """Kernel name without the argument list and namespaces."""
    base = name.replace("(anonymous namespace)::", "").replace("h2o::", "")
    base = base.split("(")[0].strip()
    if base.startswith("void "):
        base = base[5:]
    return base


def _csv_rows(folder, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    return rows


def trace_summary(folder, skip):
    """Per-kernel durations from a rocprofv3 --kernel-trace folder, leaving
    out the first `skip` dispatches of every kernel (warm-up)."""
    per = {}
    rows = _csv_rows(folder, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        name = _short_kernel_name(r["Kernel_Name"])
        per.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = [f"{'kernel':44s} {'calls':>6s} {'used':>5s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    total = sum(sum(v[skip:]) for v in per.values())
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1][skip:])):
        used = d[skip:]
        if not used:
            continue
        lines.append(f"{name[:44]:44s} {len(d):6d} {len(used):5d} {sum(used) / len(used):9.1f} "
                     f"{min(used):9.1f} {max(used):9.1f}   {100 * sum(used) / total:5.1f}%")
    return "\n".join(lines)


def counters_summary(folders, skip, cus=256, xcds=8):
    """Per-kernel averages of the counters in rocprofv3 --pmc folders (first
    `skip` dispatches of every kernel left out; the library's kernels only),
    with ratios derived from them.  SQ counters are chip totals.
    GRBM_GUI_ACTIVE is summed over the XCDs, so GRBM_GUI_ACTIVE / xcds is the
    kernel's length in GPU cycles (cyc), and a SIMD-cycle share divides by
    cyc * 4 * cus.  SQ_VALU_MFMA_BUSY_CYCLES counts 32 cycles per
    32x32x16 MFMA; SQ_ACTIVE_INST_VALU counts one 4-cycle issue slot per
    vector instruction (MFMAs included) and one more per transcendental, so
    4 * (SQ_ACTIVE_INST_VALU - SQ_INSTS_MFMA) estimates the SIMD cycles the
    vector ALU is busy.  SQ_WAVE_CYCLES and the SQ_WAIT counters are in the
    same (4-cycle) units, so their ratios are shares of wave time."""
    per = {}
    for folder in folders:
        for r in _csv_rows(folder, "counter_collection.csv"):
            name = _short_kernel_name(r["Kernel_Name"])
            if name.startswith("at::"):
                continue
            did = int(r["Dispatch_Id"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append((did, float(r["Counter_Value"]), dur))
    out = []
    for name, cnt in sorted(per.items()):
        avg = {}
        durs = []
        nd = 0
        for c, vals in cnt.items():
            vals.sort()
            used = vals[skip:] or vals
            nd = len(used)
            avg[c] = sum(v for _, v, _ in used) / len(used)
            durs += [d for _, _, d in used]
        out.append(f"## {name}  (dispatches averaged: {nd}, mean duration {sum(durs) / len(durs):.1f} us)")
        for c in sorted(avg):
            out.append(f"  {c:34s} {avg[c]:18.1f}")
        derived = []
        cyc = avg.get("GRBM_GUI_ACTIVE")
        if cyc and sum(durs) / len(durs) < 100.0:
            out.append("  (shorter than 100 us: launch overhead dominates GRBM_GUI_ACTIVE, so no cycle shares)")
            cyc = None
        if cyc:
            cyc /= xcds
            simd = cyc * cus * 4
            derived.append(("GPU clock over the kernel (GHz)", cyc / (sum(durs) / len(durs)) * 1e-3))
            mfma = avg.get("SQ_VALU_MFMA_BUSY_CYCLES")
            if mfma is not None:
                derived.append(("MFMA busy, share of SIMD cycles", mfma / simd))
            valu = None
            if "SQ_ACTIVE_INST_VALU" in avg and "SQ_INSTS_MFMA" in avg:
                valu = 4 * (avg["SQ_ACTIVE_INST_VALU"] - avg["SQ_INSTS_MFMA"]) / simd
                derived.append(("vector ALU busy (estimate), share of SIMD cycles", valu))
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
                co = avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd
                derived.append(("MFMA and vector ALU both busy, share", co))
                if mfma is not None and valu is not None:
                    derived.append(("neither busy, share", 1 - mfma / simd - valu + co))
            if "SQ_LDS_IDX_ACTIVE" in avg:
                derived.append(("LDS active, share of CU cycles", avg["SQ_LDS_IDX_ACTIVE"] / (cyc * cus)))
            if "SQ_LDS_BANK_CONFLICT" in avg:
                derived.append(("LDS bank-conflict cycles, share of CU cycles",
                                avg["SQ_LDS_BANK_CONFLICT"] / (cyc * cus)))
        if "SQ_WAVE_CYCLES" in avg:
            for c, label in (("SQ_WAIT_INST_ANY", "waiting on a dependency, share of wave time"),
                             ("SQ_WAIT_ANY", "waiting (any reason), share of wave time"),
                             ("SQ_WAIT_INST_LDS", "waiting on LDS, share of wave time")):
                if c in avg:
                    derived.append((label, avg[c] / avg["SQ_WAVE_CYCLES"]))
        if "SQ_INSTS_VALU" in avg and avg.get("SQ_INSTS_MFMA"):
            m = avg["SQ_INSTS_MFMA"]
            derived.append(("vector instructions per MFMA", (avg["SQ_INSTS_VALU"] - m) / m))
            for c, label in (("SQ_INSTS_VALU_TRANS_F32", "  of them transcendental"),
                             ("SQ_INSTS_VALU_FMA_F32", "  of them FMA"), ("SQ_INSTS_VALU_ADD_F32", "  of them add"),
                             ("SQ_INSTS_VALU_MUL_F32", "  of them multiply"), ("SQ_INSTS_VALU_CVT", "  of them conversion"),
                             ("SQ_INSTS_LDS", "LDS instructions per MFMA"), ("SQ_INSTS_SALU", "scalar instructions per MFMA")):
                if c in avg:
                    derived.append((label, avg[c] / m))
        for label, v in derived:
            out.append(f"  {label:52s} {v:8.3f}")
        out.append("")
    return "\n".join(out)


def traffic_from(workload, fetch_dir, write_dir):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of pass A by the calibration copy."""
    from h2o_kv_cache_sdpa_amd import workloads as W
    w = W.WORKLOADS[workload]
    kname = dominant_kernel(w)
    out = {"workload": w.name, "kernel": kname, "sources": kernel_sources_digest()}
    known = COPY_ELEMS * 4
    for counter, folder, key in (("FETCH_SIZE", fetch_dir, "read"), ("WRITE_SIZE", write_dir, "write")):
        rows = _counter_rows(folder, counter)
        copy = [v for _, n, v in rows if "neg_kernel" in n][-COPY_REPS:]
        attn = [v for _, n, v in rows if kname in n]
        if len(copy) < COPY_REPS or len(attn) < 2:
            raise SystemExit(f"{counter}: found {len(copy)} copy and {len(attn)} {kname} dispatches in {folder}")
        attn = attn[1:]                          # drop the first (cold) dispatch
        factor = known / (sum(copy) / len(copy) * 1024.0)
        out[f"{key}_kib_counter"] = sum(attn) / len(attn)
        out[f"{key}_factor"] = factor
        out[f"{key}_bytes"] = out[f"{key}_kib_counter"] * 1024.0 * factor
        out[f"{key}_dispatches"] = len(attn)
    out["bytes_per_launch"] = out["read_bytes"] + out["write_bytes"]
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T
    esz = {"native": 2 * D, "int8": D + 2, "int4": D // 2 + 4}[w.cache_fmt]
    algo = 2 * B * Hkv * C * esz + 2 * B * Hq * T * D * 2 + 2 * B * Hkv * T * D * 2 + B * Hq * T * 4
    out["algorithmic_bytes"] = algo
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


class CheckOnce:
    """True the first time a chunk of the rotation is used: the binding checks
    that call's tensors, and the timing loops skip the checks afterwards."""

    def __init__(self):
        self.seen = set()

    def __call__(self, i):
        k = i % N_CHUNKS
        if k in self.seen:
            return False
        self.seen.add(k)
        return True


def step_bytes(w, n_occ):
    """Algorithmic HBM bytes of one chunk step: the cache read once plus Q, the
    chunk's K/V, O, the summed weights, the scores (read and written) and the
    row normalisers; token positions and the replay log row."""
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T
    row = {"native": 2 * D, "int8": D + 2, "int4": D // 2 + 4}[w.cache_fmt]
    esz = 2 if w.dtype == "bf16" else 4
    cache = 2 * B * Hkv * n_occ * row
    qo = 2 * B * Hq * T * D * esz
    chunk = 2 * B * Hkv * T * D * esz
    small = B * Hkv * ((n_occ + T) * 4 + 2 * C * 4 + C * 4 + T * 4) + B * Hq * T * 4
    return cache + qo + chunk + small


def _resident_setup(w, policy, dev):
    """A full cache of workload w with seeded contents and a rotation of
    chunks, all resident on the device."""
    import numpy as np
    import torch

    from h2o_kv_cache_sdpa_amd import workloads as W
    from h2o_kv_cache_sdpa_amd.cache import H2OCache
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T
    gc = H2OCache(B, Hq, Hkv, D, C, T, dtype=w.dtype, cache_fmt=w.cache_fmt, device=dev, policy=policy)
    seed = [w.cfg_id, 777]
    if w.cache_fmt == "native":
        k, v, scores, tp, _ = W.random_cache(seed, B, Hkv, C, D, C, w.dtype, hh_frac=0.02)
        for name, st in (("k", k), ("v", v)):
            getattr(gc, name).copy_(torch.from_numpy(np.ascontiguousarray(st.raw).view(np.int16))
                                    .view(torch.bfloat16))
    else:
        arr = W.random_quant_cache(seed, B, Hkv, C, D, C, w.cache_fmt)
        scores, tp = arr["scores"], arr["token_pos"]
        for key, val in arr.items():
            if key.endswith(("_codes", "_scale", "_zero")):
                name = key.replace("_codes", "")
                getattr(gc, name).copy_(torch.from_numpy(val))
    gc.scores.copy_(torch.from_numpy(scores))
    gc.token_pos.copy_(torch.from_numpy(tp))
    gc.n_occ, gc.pos = C, C
    chunks = []
    to_dev = lambda st: torch.from_numpy(np.ascontiguousarray(st.raw).view(np.int16)).view(torch.bfloat16).to(dev)
    for s in range(N_CHUNKS):
        ch = W.chunk(w, w.n_fill + s)
        chunks.append((to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])))
    return gc, chunks


def sweep_small_t(args):
    """HBM-bound regime: chunk lengths 1..128 on full caches (32K slots unless
    --sweep-slots names other sizes)."""
    import torch

    from h2o_kv_cache_sdpa_amd import api
    from h2o_kv_cache_sdpa_amd import workloads as W
    dev = torch.device("cuda:0")
    base = W.WORKLOADS[3]
    cases = [(fmt, C, T) for fmt in args.sweep_fmts.split(",") for C in (int(c) for c in args.sweep_slots.split(","))
             for T in (int(t) for t in args.sweep_ts.split(","))]
    for fmt, C, T in cases:
        w = base.scaled(T=T, C=C, cache_fmt=fmt, name=f"small_t_{fmt}_{C // 1024}k_t{T}")
        gc, chunks = _resident_setup(w, "h2o", dev)
        out, wsum, slot_log = gc.new_outputs(w.C)
        bufs = gc.bufs()
        stream = torch.cuda.current_stream()
        reps = args.sweep_reps

        first = CheckOnce()

        def step(i):
            q, kn, vn = chunks[i % N_CHUNKS]
            api.h2o_chunk_step(gc.dims, bufs, w.C, gc.pos, q, kn, vn, out, wsum, slot_log, gc.ws, stream,
                           check=first(i))
            gc.pos += T

        for i in range(min(10, reps)):
            step(i)
        torch.cuda.synchronize()
        # step time without per-kernel events
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        t0 = time.perf_counter()
        for i in range(reps):
            step(i)
        host_ms = (time.perf_counter() - t0) * 1e3 / reps
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        # per-kernel breakdown in a second, event-bracketed run
        api.profile_reset()
        api.profile_enable(True)
        for i in range(reps):
            step(i)
        torch.cuda.synchronize()
        api.profile_enable(False)
        prof = api.profile_read()
        nbytes = step_bytes(w, w.C)
        print(json.dumps({
            "sweep": "small_t", "workload": w.name, "cache_fmt": fmt, "chunk": T, "cache_slots": w.C,
            "ms_per_step": ms, "tokens_per_s": w.B * T / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "host_enqueue_ms": host_ms,
            "kernel_ms": {k: (v[0] / v[1] if v[1] else None) for k, v in prof.items()},
        }), flush=True)
        del gc, chunks, out, wsum, slot_log
        torch.cuda.empty_cache()


def replay(args):
    """Replay steps: the chunk's attention and the overwrite of the slots a
    recorded log row names, with no weight sums, scores or selection.  The
    log rows are recorded by chunk steps over the same rotation of chunks;
    the chunk step is timed beside the replay step on the same cache."""
    import torch

    from h2o_kv_cache_sdpa_amd import api
    from h2o_kv_cache_sdpa_amd import workloads as W
    dev = torch.device("cuda:0")
    for wid in (int(x) for x in args.replay_workloads.split(",")):
        w = W.WORKLOADS[wid]
        B, T, C = w.B, w.T, w.C
        gc, chunks = _resident_setup(w, "h2o", dev)
        out, wsum, slot_log = gc.new_outputs(C)
        bufs = gc.bufs()
        stream = torch.cuda.current_stream()
        logs = []

        first, first_replay = CheckOnce(), CheckOnce()

        def chunk_step(i):
            q, kn, vn = chunks[i % N_CHUNKS]
            api.h2o_chunk_step(gc.dims, bufs, C, gc.pos, q, kn, vn, out, wsum, slot_log, gc.ws, stream,
                               check=first(i))
            gc.pos += T

        def replay_step(i):
            q, kn, vn = chunks[i % N_CHUNKS]
            api.h2o_replay_step(gc.dims, bufs, C, gc.pos, q, kn, vn, out, logs[i % N_CHUNKS], gc.ws, stream,
                                check=first_replay(i))
            gc.pos += T

        for i in range(N_CHUNKS):
            chunk_step(i)
            logs.append(slot_log.clone())
        res = {}
        for name, fn in (("chunk_step", chunk_step), ("replay_step", replay_step)):
            for i in range(args.warmup):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            api.profile_reset()
            api.profile_enable(True)
            for i in range(args.steps):
                fn(i)
            torch.cuda.synchronize()
            api.profile_enable(False)
            prof = api.profile_read()
            res[name] = {"ms_per_step": ms, "tokens_per_s": B * T / (ms * 1e-3),
                         "kernel_ms": {k: (v[0] / v[1] if v[1] else None) for k, v in prof.items() if v[1]}}
        print(json.dumps({"mode": "replay", "workload": w.name, "B": B, "cache_slots": C, "chunk": T,
                          "cache_fmt": w.cache_fmt, **res}), flush=True)
        del gc, chunks, out, wsum, slot_log, logs
        torch.cuda.empty_cache()


def prefill(args):
    """First chunk of a sequence on an empty cache: n_occ = 0, T = C, a causal
    square with summed weights (the pages' length-N_C prefill)."""
    import numpy as np
    import torch

    from h2o_kv_cache_sdpa_amd import api
    from h2o_kv_cache_sdpa_amd import workloads as W
    from h2o_kv_cache_sdpa_amd.cache import H2OCache
    dev = torch.device("cuda:0")
    to_dev = lambda st: torch.from_numpy(np.ascontiguousarray(st.raw).view(np.int16)).view(torch.bfloat16).to(dev)
    for C in (int(c) for c in args.prefill_sizes.split(",")):
        w = W.WORKLOADS[3].scaled(C=C, T=C, name=f"prefill_bf16_{C // 1024}k")
        gc = H2OCache(w.B, w.Hq, w.Hkv, w.D, C, C, dtype="bf16", cache_fmt="native", device=dev)
        ch = W.chunk(w, 0)
        q, kn, vn = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])
        del ch
        out, wsum, slot_log = gc.new_outputs(0)
        bufs = gc.bufs()
        stream = torch.cuda.current_stream()
        reps = 5

        def step():
            api.h2o_chunk_step(gc.dims, bufs, 0, 0, q, kn, vn, out, wsum, slot_log, gc.ws, stream)

        for _ in range(2):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        api.profile_reset()
        api.profile_enable(True)
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        api.profile_enable(False)
        prof = api.profile_read()
        kms = {k: (v[0] / v[1] if v[1] else None) for k, v in prof.items()}
        pairs = pairs_visible(w.B, w.Hq, C, 0)
        a_tf = 4 * w.D * pairs / (kms["attn_a"] * 1e-3) / 1e12
        b_tf = 2 * w.D * pairs / (kms["attn_b"] * 1e-3) / 1e12
        print(json.dumps({
            "prefill": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "chunk": C, "cache_slots": C,
            "ms_per_step": ms, "tokens_per_s": w.B * C / (ms * 1e-3),
            "step_mfma_frac_6d": 6 * w.D * pairs / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "attn_a_tflops": a_tf, "attn_b_tflops": b_tf, "kernel_ms": kms,
        }), flush=True)
        del gc, q, kn, vn, out, wsum, slot_log
        torch.cuda.empty_cache()


def backward(args):
    """Gradients of the chunk attention (the fine-tuning pass): the evicting
    step of the 32K cache (n_occ = C = 32768, T = 2048) and a 16K prefill
    square.  Matrix work per visible pair: row terms 4*D flops (S, dP),
    dq 6*D (S, dP, dS K), dk/dv 8*D (S, dP, P^T dO, dS^T Q); the figure of
    merit counts the 14*D of the gradients themselves."""
    import numpy as np
    import torch

    from h2o_kv_cache_sdpa_amd import api
    from h2o_kv_cache_sdpa_amd import workloads as W
    dev = torch.device("cuda:0")
    to_dev = lambda st: torch.from_numpy(np.ascontiguousarray(st.raw).view(np.int16)).view(torch.bfloat16).to(dev)
    for name, C, T, n_occ in (("bwd_bf16_32k_t2048", 32768, 2048, 32768), ("bwd_prefill_bf16_16k", 16384, 16384, 0)):
        w = W.WORKLOADS[3].scaled(C=C, T=T, name=name)
        B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
        dims = api.make_dims(B, Hq, Hkv, D, C, T)
        ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=dev)
        kc = torch.randn(B, Hkv, C, D, device=dev).to(torch.bfloat16)
        vc = torch.randn(B, Hkv, C, D, device=dev).to(torch.bfloat16)
        ch = W.chunk(w, 0)
        q, kn, vn = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])
        del ch
        dout = torch.randn(B, Hq, T, D, device=dev).to(torch.bfloat16)
        bufs = api.cache_struct(kc, vc)
        out = torch.empty_like(q)
        wsum = torch.empty(B, Hkv, n_occ + T, dtype=torch.float32, device=dev)
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
        api.h2o_sdpa_scoresum(dims, bufs, n_occ, q, kn, vn, out, wsum, lse, ws)
        dq = torch.empty(B, Hq, T, D, dtype=torch.float32, device=dev)
        dkc = torch.empty(B, Hkv, C, D, dtype=torch.float32, device=dev)
        dvc = torch.empty_like(dkc)
        dkn = torch.empty(B, Hkv, T, D, dtype=torch.float32, device=dev)
        dvn = torch.empty_like(dkn)
        stream = torch.cuda.current_stream()
        reps = 5

        def step():
            api.h2o_sdpa_backward(dims, bufs, n_occ, q, kn, vn, lse, dout, dq, dkc, dvc, dkn, dvn, ws, stream)

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        api.profile_reset()
        api.profile_enable(True)
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        api.profile_enable(False)
        kms = {k: (v[0] / v[1] if v[1] else None) for k, v in api.profile_read().items() if v[1]}
        pairs = pairs_visible(B, Hq, T, n_occ)
        print(json.dumps({
            "backward": name, "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "chunk": T, "cache_slots": C, "n_occ": n_occ,
            "ms": ms, "tflops_14d": 14 * D * pairs / (ms * 1e-3) / 1e12,
            "mfma_frac_14d": 14 * D * pairs / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "rowterm_tflops": 4 * D * pairs / (kms["bwd_rows"] * 1e-3) / 1e12,
            "dq_tflops": 6 * D * pairs / (kms["bwd_dq"] * 1e-3) / 1e12,
            "dkdv_tflops": 8 * D * pairs / (kms["bwd_dkdv"] * 1e-3) / 1e12,
            "kernel_ms": kms,
        }), flush=True)
        del q, kn, vn, out, dout, dq, dkc, dvc, dkn, dvn, kc, vc, ws, wsum, lse
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--policy", default="h2o", choices=["h2o", "h2o_norm", "h2o_orig"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-ceiling", action="store_true",
                    help="skip the library-GEMM rate printed beside the headline for context")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--trace-from", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace folder (no GPU); --skip-first dispatches "
                         "of every kernel are left out")
    ap.add_argument("--counters-from", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc folders per kernel (no GPU)")
    ap.add_argument("--skip-first", type=int, default=0, help="warm-up dispatches per kernel to leave out")
    ap.add_argument("--sweep-small-t", action="store_true",
                    help="chunk lengths 1, 4, 16, 64, 128 on the 32K-slot cache in bf16, int8 and int4; "
                         "one JSON line each (HBM-bound regime)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the first chunk of a sequence (empty cache, T = C): one JSON line per size")
    ap.add_argument("--backward", action="store_true",
                    help="time h2o_sdpa_backward on the 32K evicting step and a 16K prefill square")
    ap.add_argument("--prefill-sizes", default="16384,32768", help="cache sizes (= chunk lengths) of --prefill")
    ap.add_argument("--replay", action="store_true",
                    help="time h2o_replay_step beside h2o_chunk_step on full caches: one JSON line per workload")
    ap.add_argument("--replay-workloads", default="3,4,5", help="workloads of --replay")
    ap.add_argument("--sweep-fmts", default="native,int8,int4", help="cache formats of --sweep-small-t")
    ap.add_argument("--sweep-ts", default="1,4,16,64,128", help="chunk lengths of --sweep-small-t")
    ap.add_argument("--sweep-reps", type=int, default=200, help="timed steps per --sweep-small-t case")
    ap.add_argument("--sweep-slots", default="32768", help="cache sizes (slots) of --sweep-small-t")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; the chunk step shards "
                          "over (batch, KV head) groups with no exchange, but no multi-GPU "
                          "path is built", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.traffic_from:
        traffic_from(args.workload, *args.traffic_from)
        return
    if args.trace_from:
        print(trace_summary(args.trace_from, args.skip_first))
        return
    if args.counters_from:
        print(counters_summary(args.counters_from, args.skip_first))
        return
    if args.prefill:
        prefill(args)
        return
    if args.backward:
        backward(args)
        return
    if args.replay:
        replay(args)
        return
    if args.sweep_small_t:
        sweep_small_t(args)
        return

    import numpy as np
    import torch

    from h2o_kv_cache_sdpa_amd import api
    from h2o_kv_cache_sdpa_amd import workloads as W
    from h2o_kv_cache_sdpa_amd.cache import H2OCache

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T

    # ---- resident inputs: a full cache and a rotation of chunks ----
    gc, chunks = _resident_setup(w, args.policy, dev)
    out, wsum, slot_log = gc.new_outputs(C)
    bufs = gc.bufs()
    stream = torch.cuda.current_stream()

    first = CheckOnce()

    def step(i):
        q, kn, vn = chunks[i % N_CHUNKS]
        api.h2o_chunk_step(gc.dims, bufs, C, gc.pos, q, kn, vn, out, wsum, slot_log, gc.ws, stream,
                           check=first(i))
        gc.pos += T

    for i in range(args.warmup):
        step(i)
    # timed region: the K steps alone, bracketed by two events on the launch stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # per-kernel durations: a second run of K steps with the library's event
    # timers around every launch (they add a few microseconds per kernel, so
    # they stay out of the timed region above)
    api.profile_reset()
    api.profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    api.profile_enable(False)
    prof = api.profile_read()

    pairs = pairs_visible(B, Hq, T, C)
    flops_a = 4 * D * pairs       # QK^T and PV of pass A
    flops_b = 2 * D * pairs       # QK^T recomputed in pass B
    a_ms = prof["attn_a"][0] / max(prof["attn_a"][1], 1)
    b_ms = prof["attn_b"][0] / max(prof["attn_b"][1], 1)
    achieved_a = flops_a / (a_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("sources") == kernel_sources_digest() and rec.get("workload") == w.name:
            traffic = rec.get("bytes_per_launch")
    if args.calibrate_copy:
        src = torch.randn(COPY_ELEMS, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
    line = {
        "metric": "H2O chunk-step tokens/s (S=32K,T=2048,bf16); % of MFMA/HBM roofline",
        "value": B * T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: evicting chunk step", "B": B, "Hq": Hq, "Hkv": Hkv,
                   "D": D, "cache_slots": C, "chunk": T, "cache_fmt": w.cache_fmt, "policy": args.policy},
        "roofline": {
            "bound": "mfma",
            "kernel": dominant_kernel(w) + " (pass A: output and row normalisers)",
            "achieved": achieved_a,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_a / PEAK_BF16_TFLOPS,
            "traffic": traffic,
        },
        # the whole step against the bf16 peak (the headline fraction), and the
        # step time that STEP_TARGET_FRAC of the peak would take
        "step_mfma_frac_6d": 6 * D * pairs / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "step_target_frac_6d": STEP_TARGET_FRAC,
        "ms_per_step_at_target": 6 * D * pairs / (STEP_TARGET_FRAC * PEAK_BF16_TFLOPS * 1e12) * 1e3,
        "step_mfma_frac_4d": 4 * D * pairs / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_ms": {k: (v[0] / v[1] if v[1] else None) for k, v in prof.items()},
        "attn_b_tflops": flops_b / (b_ms * 1e-3) / 1e12,
        "wall_s_timed": wall,
    }
    if not args.no_gemm_ceiling:
        line["gemm_ceiling"] = gemm_ceiling(dev)
        line["step_frac_of_gemm_ceiling_6d"] = (6 * D * pairs / (ms_step * 1e-3) / 1e12
                                                / line["gemm_ceiling"]["achieved"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
