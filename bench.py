#!/usr/bin/env python3
"""Throughput of one HySparse2 Hybrid Block step on one MI355X.

A step is one hs2_block_forward call: causal GQA full attention, the
head-summed score pass, token top-k selection (1024 + 128-token window) and
every sparse layer reusing the full layer's K/V and index sets, over one
batch of synthetic inputs already resident in HBM. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config 5]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selection+sparse-attn tokens/s at 128K-1M ctx; MFMA util and HBM GB/s vs peak"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
# in the order of the library's pass-timer slots
PASSES = ["full_attention", "score", "select", "sparse_attention", "v_layout",
          "bwd_prep", "bwd_sparse", "bwd_dkdv", "bwd_dq", "kv_stage"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w):
    """Per-step algorithmic work of each pass (flops or bytes)."""
    esz = 2 if w.dtype == "bf16" else 4
    B, nq, nkv, hq, hkv, d = w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.d
    pos = [nkv - nq + i for i in range(nq)]
    pairs = sum(p + 1 for p in pos) * B                         # causal (query, key)
    cand = sum(max(0, p - w.window + 1) for p in pos) * B       # candidate pairs
    sel = sum(min(p + 1, w.top_k + w.window) for p in pos) * B  # selected keys
    L = w.n_sparse
    # selection reads each candidate score once, except on rows of more than
    # 128 * top_k candidates with the bf16 score pass: those read the row's
    # 64-key segment maxima and then top_k whole segments (the keys at or
    # above the top_k-th largest maximum lie in at least that many)
    seg = nq > 1 and w.dtype == "bf16" and d == 128
    sel_read = 0.0
    for p in pos:
        n_c = max(0, p - w.window + 1)
        if seg and n_c >= 128 * w.top_k:
            sel_read += 4.0 * ((n_c + 63) // 64) + 256.0 * w.top_k
        else:
            sel_read += 4.0 * n_c
    sel_read *= B
    if nq == 1:
        # decode: one query per sequence, so pass 1 streams K and V once
        # (8 flop/B) and the score pass reads the stored logits
        full = ("hbm", 2.0 * B * nkv * hkv * d * esz + 2.0 * B * hq * d * esz)
        score = ("hbm", 4.0 * hq * cand + 4.0 * cand)
    else:
        full = ("mfma", 4.0 * hq * d * pairs)
        score = ("mfma", 2.0 * hq * d * cand)
    return {
        "full_attention": full,
        "score": score,
        "select": ("hbm", sel_read + 4.0 * B * nq * (w.top_k + w.window)),
        "sparse_attention": ("hbm", sel * hkv * d * 2.0 * esz + 2.0 * L * B * nq * hq * d * esz),
        # V read once, written once in key-tile-major transposed order
        "v_layout": ("hbm", 2.0 * B * nkv * hkv * d * esz),
    }


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CSRC = "token_level_sparse_pass_amd/csrc/"
_BUILD = "token_level_sparse_pass_amd/build.py"       # compiler flags shape the code too
KERNEL_SOURCES = {
    "full_attention": [_CSRC + "attn_fwd_bf16.hip", _CSRC + "attn_fwd.hip",
                       _CSRC + "attn_decode_bf16.hip", _CSRC + "hs2_device.h", _BUILD],
    # decode's score step (decode_score_kernel) lives in attn_fwd.hip
    "score": [_CSRC + "score_bf16.hip", _CSRC + "score.hip", _CSRC + "attn_fwd.hip",
              _CSRC + "hs2_device.h", _BUILD],
    "select": [_CSRC + "select.hip", _BUILD],
    "sparse_attention": [_CSRC + "sparse_attn_bf16.hip", _CSRC + "sparse_attn.hip",
                         _CSRC + "hs2_device.h", _BUILD],
    "v_layout": [_CSRC + "attn_fwd_bf16.hip", _BUILD],
}


def committed_counters(kind, pass_name, workload):
    """A pass's record from profiles/<kind>.json (kind "traffic": HBM bytes
    from FETCH_SIZE / WRITE_SIZE; kind "mfma": MFMA counters) for this
    workload, or None when there is none or the pass's kernel sources have
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", kind + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("passes", {}).get(pass_name, {}).get(workload)
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[pass_name]):
        return None
    return rec


def measured_traffic(pass_name, workload):
    """HBM bytes per launch of the pass's kernels from the committed counters."""
    rec = committed_counters("traffic", pass_name, workload)
    return None if rec is None else rec["bytes_per_launch"]


def hbm_pass(per_ms, launches, amount, pass_name, workload):
    """Record of an HBM-bound pass: achieved / frac from the committed
    FETCH/WRITE counters for this workload (null without them), and the
    effective rate of its algorithmic bytes, which counts what the caches
    serve too and so can pass the HBM peak."""
    secs = per_ms / 1e3
    eff = amount / secs / 1e9
    tr = committed_counters("traffic", pass_name, workload)
    ach = None if tr is None else tr["bytes_per_step"] / secs / 1e9
    return {"ms": round(per_ms, 4), "launches_per_step": int(launches), "bound": "hbm",
            "achieved": None if ach is None else round(ach, 1), "unit": "GB/s",
            "frac": None if ach is None else round(ach / PEAK_HBM_GBS, 4),
            "effective_GBs": round(eff, 1), "effective_frac": round(eff / PEAK_HBM_GBS, 4)}


# kernels of each pass, by name prefix (as rocprofv3 reports them)
PASS_KERNELS = {
    "full_attention": ("hs2::attn_fwd_bf16_kernel", "hs2::attn_fwd_prefill_kernel",
                       "hs2::attn_decode_bf16_kernel", "hs2::attn_fwd_decode_kernel",
                       "hs2::decode_combine_kernel"),
    "score": ("hs2::score_bf16_kernel", "hs2::score_prefill_kernel", "hs2::decode_score_kernel"),
    "select": ("hs2::select_token_kernel", "hs2::select_block_kernel"),
    "sparse_attention": ("hs2::sparse_bf16_kernel", "hs2::sparse_bf16_split_kernel", "hs2::sparse_attn_kernel"),
    "v_layout": ("hs2::transpose_v_kernel",),
}
COUNTER_REGEX = "attn_fwd|attn_decode|decode_|score|sparse|select|transpose"
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
                 "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
N_CU = 256


def _read_counter_csv(path):
    """{(dispatch id, kernel name): {counter: value}} from a rocprofv3 csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = _kernel_base_name(r["Kernel_Name"])
            key = (int(r["Dispatch_Id"]), name)
            out.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def _kernel_base_name(name):
    """'hs2::name' from a demangled signature or an Itanium-mangled name
    (_ZN<len><part>...: the nested-name prefix, template arguments dropped)."""
    if name.startswith("_ZN"):
        parts, i = [], 3
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            parts.append(name[j:j + n])
            i = j + n
        return "::".join(parts)
    name = name.split("(")[0]
    if name.startswith("void "):
        name = name[5:]
    return name.split("<")[0]


def _pass_of(kernel):
    for name, prefixes in PASS_KERNELS.items():
        if kernel in prefixes:
            return name
    return None


def trace_summary(trace_dir, cid):
    """Summarise a `rocprofv3 --kernel-trace --stats` run of `bench.py
    --config cid --steps 3 --warmup 1 --no-cpu-baseline` (host only) into
    profiles/block_step_<workload>.md: the per-kernel statistics and the
    bench line the same run printed (run.log beside the trace)."""
    import csv
    import glob
    from synth import CONFIGS
    w = CONFIGS[cid]
    stats = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True))
    dbs = sorted(glob.glob(os.path.join(trace_dir, "**", "*results.db"), recursive=True))
    if stats:
        with open(stats[0]) as f:
            rows = list(csv.DictReader(f))
    elif dbs:
        # rocprofv3's database output: its top_kernels view holds the same
        # statistics (durations in microseconds there)
        import sqlite3
        con = sqlite3.connect(dbs[0])
        rows = [{"Name": n, "Calls": c, "TotalDurationNs": t * 1e3, "AverageNs": a * 1e3,
                 "Percentage": pc}
                for n, c, t, a, pc in con.execute(
                    "select name, total_calls, total_duration, average, percentage "
                    "from top_kernels order by total_duration desc")]
        con.close()
    else:
        raise SystemExit(f"no kernel statistics under {trace_dir}")
    bench_line = None
    log_path = trace_dir.rstrip("/") + ".log"
    if os.path.exists(log_path):
        for line in open(log_path):
            if line.startswith("{") and '"metric"' in line:
                bench_line = json.loads(line)
    lines = [f"# Kernel trace: Hybrid Block step, {w.name}", "",
             "Command (from /tmp, with R = the repository root, on one MI355X; summarised by "
             "`python bench.py --trace-summary DIR --config N`):", "", "```",
             f"rocprofv3 --kernel-trace --stats -f csv -d $R/gpurun_out/prof/trace_c{cid} -o run -- "
             f"python3 $R/bench.py --config {cid} --steps 3 --warmup 1 --no-cpu-baseline "
             f"> $R/gpurun_out/prof/trace_c{cid}.log", "```", "",
             "Kernel trace statistics (durations in microseconds; the bench runs 1 warm-up and "
             "3 timed steps, so each launch slot of a step is counted 4 times):", "",
             "| kernel | calls | total (us) | average (us) | % of GPU time |", "|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(float(r.get("Calls", 0)))
        tot = float(r.get("TotalDurationNs", 0)) / 1e3
        avg = float(r.get("AverageNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        lines.append(f"| `{name.split('(')[0][:90]}` | {calls} | {tot:.1f} | {avg:.1f} | {pct:.2f} |")
    if bench_line:
        ps = bench_line.get("passes", {})
        lines += ["", "The same run's bench line (HIP events on the library's stream): "
                  f"{bench_line['ms_per_step']:.3f} ms per step, {bench_line['value']:.1f} tokens/s; "
                  "per pass: " + ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in ps.items()) + "."]
    out = os.path.join(ROOT, "profiles", f"block_step_{w.name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def counters_summary(pmc_dir, steps_profiled=2):
    """Summarise rocprofv3 --pmc runs into profiles/traffic.json,
    profiles/mfma.json and one markdown file per workload (host only).

    pmc_dir holds the runs made by the commands this function writes into
    the markdown (directories mfma_c<N>, fetch_c<N>, write_c<N> for
    workload N, fetch_copy / write_copy for the copy calibration), each with
    rocprofv3's run_counter_collection.csv and run_agent_info.csv. Each
    workload run is `bench.py --steps 1 --warmup 0`: two block_forward
    calls, so per-step figures are totals / 2."""
    import csv
    from synth import CONFIGS

    def csv_of(sub):
        path = os.path.join(pmc_dir, sub, "run_counter_collection.csv")
        return _read_counter_csv(path) if os.path.exists(path) else None

    n_xcc = 8
    agent = os.path.join(pmc_dir, "fetch_copy", "run_agent_info.csv")
    if os.path.exists(agent):
        with open(agent) as f:
            for r in csv.DictReader(f):
                if r.get("Agent_Type") == "GPU" or r.get("Name", "").startswith("gfx"):
                    n_xcc = int(r.get("Num_Xcc", n_xcc))
    # copy calibration: a 2 GiB elementwise copy (2 GiB read, 2 GiB written)
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        d = csv_of(("fetch" if c == "FETCH_SIZE" else "write") + "_copy")
        vals = [v[c] for v in d.values()]
        cal[c] = sum(vals) / len(vals)
    size_kib = 2048 * 1024
    scale = {"fetch": size_kib / cal["FETCH_SIZE"], "write": size_kib / cal["WRITE_SIZE"]}

    traffic, mfma = {}, {}
    md = {}
    cmd_base = ("cd /tmp && export TMPDIR=/tmp  # then, from there, with R = the repository root:\n")
    for cid, w in CONFIGS.items():
        fetch, write, mf = csv_of(f"fetch_c{cid}"), csv_of(f"write_c{cid}"), csv_of(f"mfma_c{cid}")
        if fetch is None and mf is None:
            continue
        run = f"python3 $R/bench.py --config {cid} --steps 1 --warmup 0 --no-cpu-baseline"
        cmds = []
        lines = []
        if fetch is not None and write is not None:
            for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
                cmds.append(f"rocprofv3 --pmc {c} --kernel-include-regex \"{COUNTER_REGEX}\" -f csv "
                            f"-d $R/gpurun_out/pmc/{sub}_c{cid} -o run -- {run}")
            # the two runs launch the same kernels in the same order: pair the
            # n-th dispatch of each kernel in one with the n-th in the other
            per = {}
            for kern in sorted({k[1] for k in fetch if _pass_of(k[1])}):
                fk = sorted(k for k in fetch if k[1] == kern)
                wk = sorted(k for k in write if k[1] == kern)
                assert len(fk) == len(wk), (kern, len(fk), len(wk))
                ps = _pass_of(kern)
                e = per.setdefault(ps, {"kernels": set(), "dispatches": 0, "fetch": 0.0,
                                        "write": 0.0})
                e["kernels"].add(kern)
                e["dispatches"] += len(fk)
                e["fetch"] += sum(fetch[k]["FETCH_SIZE"] for k in fk)
                e["write"] += sum(write[k]["WRITE_SIZE"] for k in wk)
            lines += ["", "HBM traffic (FETCH_SIZE and WRITE_SIZE in KiB, summed over the "
                      f"{steps_profiled} profiled steps; bytes scaled by the copy calibration):", "",
                      "| pass | kernels | dispatches per step | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) "
                      "| HBM bytes per step | per launch |", "|---|---|---|---|---|---|---|"]
            for ps, e in per.items():
                byts = (e["fetch"] * scale["fetch"] + e["write"] * scale["write"]) * 1024
                step = byts / steps_profiled
                launches = e["dispatches"] / steps_profiled
                traffic.setdefault(ps, {})[w.name] = {
                    "kernels": sorted(e["kernels"]), "launches_per_step": launches,
                    "fetch_kib": round(e["fetch"], 1), "write_kib": round(e["write"], 1),
                    "bytes_per_step": round(step), "bytes_per_launch": round(step / launches),
                    "source_sha": source_sha(KERNEL_SOURCES[ps])}
                lines.append(f"| {ps} | {', '.join('`' + k + '`' for k in sorted(e['kernels']))} "
                             f"| {launches:g} | {e['fetch']:.0f} | {e['write']:.0f} "
                             f"| {step / 2**30:.3f} GiB | {step / launches / 2**30:.4f} GiB |")
        if mf is not None:
            cmds.append(f"rocprofv3 --pmc {MFMA_COUNTERS} --kernel-include-regex "
                        f"\"{COUNTER_REGEX}\" -f csv -d $R/gpurun_out/pmc/mfma_c{cid} -o run -- {run}")
            per = {}
            for (disp, kern), v in mf.items():
                ps = _pass_of(kern)
                if ps is None:
                    continue
                e = per.setdefault(ps, {"kernels": set(), "dispatches": 0})
                e["kernels"].add(kern)
                e["dispatches"] += 1
                for c, x in v.items():
                    e[c] = e.get(c, 0.0) + x
            lines += ["", "MFMA counters (summed over the dispatches of the profiled steps; "
                      f"GRBM_GUI_ACTIVE is reported summed over the {n_xcc} XCDs, so one XCD's "
                      f"active cycles are that sum / {n_xcc}):", "",
                      "| pass | dispatches per step | MFMA flops per step (MOPS_BF16 x 512) "
                      "| MFMA busy (BUSY_CYCLES / (GUI_ACTIVE/XCDs x 1024 SIMDs)) "
                      "| active cycles per launch (one XCD) | VALU instr per MFMA "
                      "| LDS instr per MFMA | LDS bank-conflict cycles (share of active, per CU) |",
                      "|---|---|---|---|---|---|---|---|"]
            for ps, e in per.items():
                if e.get("SQ_INSTS_MFMA", 0) == 0:
                    continue
                gui = e["GRBM_GUI_ACTIVE"] / n_xcc
                busy = e["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024)
                flops_step = e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / steps_profiled
                launches = e["dispatches"] / steps_profiled
                rec = {"kernels": sorted(e["kernels"]), "launches_per_step": launches,
                       "mfma_flops_per_step": flops_step, "mfma_busy": round(busy, 4),
                       "active_cycles_per_launch": round(gui / e["dispatches"]),
                       "valu_per_mfma": round(e["SQ_INSTS_VALU"] / e["SQ_INSTS_MFMA"], 3),
                       "lds_per_mfma": round(e["SQ_INSTS_LDS"] / e["SQ_INSTS_MFMA"], 3),
                       "lds_bank_conflict_frac": (round(e["SQ_LDS_BANK_CONFLICT"] / (gui * N_CU), 4)
                                                  if "SQ_LDS_BANK_CONFLICT" in e else None),
                       "source_sha": source_sha(KERNEL_SOURCES[ps])}
                mfma.setdefault(ps, {})[w.name] = rec
                lines.append(f"| {ps} | {launches:g} | {flops_step:.4e} | {100 * busy:.1f} % "
                             f"| {rec['active_cycles_per_launch']:.4e} | {rec['valu_per_mfma']:.2f} "
                             f"| {rec['lds_per_mfma']:.2f} | "
                             + ("n/a" if rec["lds_bank_conflict_frac"] is None
                                else f"{100 * rec['lds_bank_conflict_frac']:.1f} %") + " |")
        md[w.name] = (cmds, lines)
    cal_cmds = [f"rocprofv3 --pmc {c} --kernel-include-regex \"neg\" -f csv -d "
                f"$R/gpurun_out/pmc/{sub}_copy -o run -- python3 $R/bench.py --copy-calibration 2048"
                for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]
    cal_line = (f"Copy calibration: a plain elementwise copy of 2 GiB (2 GiB read, 2 GiB written) "
                f"reads FETCH_SIZE = {cal['FETCH_SIZE']:.0f} KiB and WRITE_SIZE = "
                f"{cal['WRITE_SIZE']:.0f} KiB per dispatch, so fetch counts are scaled by "
                f"{scale['fetch']:.4f} and write counts by {scale['write']:.4f}.")
    prof = os.path.join(ROOT, "profiles")
    note = ("rocprofv3 --pmc counters per pass and workload; bytes are FETCH_SIZE and WRITE_SIZE "
            "scaled by a plain copy's readings; MFMA flops are SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; "
            "records hold for the kernel sources whose hash they carry")
    with open(os.path.join(prof, "traffic.json"), "w") as f:
        json.dump({"_note": note, "scale": scale, "passes": traffic}, f, indent=1)
    with open(os.path.join(prof, "mfma.json"), "w") as f:
        json.dump({"_note": note, "xcds": n_xcc, "passes": mfma}, f, indent=1)
    for wname, (cmds, lines) in md.items():
        with open(os.path.join(prof, f"counters_{wname}.md"), "w") as f:
            f.write(f"# rocprofv3 counters: Hybrid Block step, {wname}\n\n"
                    "Commands (one pass per counter set; each run's program is bench.py of this "
                    "repository; summarised by `python bench.py --counters-summary "
                    "gpurun_out/pmc`):\n\n```\n" + cmd_base + "\n".join(cmds + cal_cmds) +
                    "\n```\n\n" + cal_line + "\n" + "\n".join(lines) + "\n")
    print(json.dumps({"workloads": sorted(md), "scale": scale}))


def host_cpu():
    """CPU model and the number of cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(w, inp, target_s=25.0, max_rows=64):
    """The fp64 oracle on a bounded sample of query rows of the same workload:
    the first and last rows, then up to max_rows - 2 uniformly spaced rows
    as the time budget allows (the oracle runs the rows of one call in
    parallel, one BLAS thread each), and the full workload's oracle time
    extrapolated from the rate."""
    import numpy as np
    from oracle import hs2_oracle as O
    from synth import to_host
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    b = 0
    k, v = to_host(inp["k"][b:b + 1]), to_host(inp["v"][b:b + 1])
    q = to_host(inp["q_full"][b:b + 1])
    qs = to_host(inp["q_sparse"][:, b:b + 1])

    def run(rows):
        t0 = time.perf_counter()
        O.block_rows(q, qs, k, v, 0, rows, top_k=w.top_k, window=w.window)
        return time.perf_counter() - t0

    ends = sorted({0, w.n_q - 1})
    t1 = run(ends)
    workers = max(1, min(cores, len(os.sched_getaffinity(0))))
    rounds = max(1, int(target_s / max(t1, 1e-3)))
    n_more = max(0, min(max_rows - len(ends), rounds * workers, w.n_q - len(ends)))
    more = sorted(set(np.linspace(1, w.n_q - 2, n_more).round().astype(int).tolist())
                  - set(ends)) if n_more > 0 else []
    t2 = run(more) if more else 0.0
    total_rows = len(ends) + len(more)
    total_t = t1 + t2
    rate = total_rows / total_t
    return {"value": rate, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", **host_cpu(),
            "rows": total_rows,
            "extrapolated_full_s": round(w.batch * w.n_q / rate, 1),
            "sample": f"{total_rows} query rows of sequence 0 of {w.name} (the first and last "
                      f"rows and {len(more)} uniformly spaced ones; full-layer LSE and score "
                      f"sweeps over all {w.n_kv} keys, token top-{w.top_k} + "
                      f"{w.window}-token window, {w.n_sparse} sparse layers), "
                      f"{total_t:.1f} s"}


def decode_loop(args):
    """Steps of hs2_decode_step over a growing, ragged cache (decode workload).

    The 64-sequence, 128K-capacity decode workload starts every sequence at
    a seeded length in [cap/2, cap - steps - 1); each step appends one token
    per sequence and runs the whole block for it. Inputs of every step are
    drawn before the timed region; one step = one decode_step call.
    """
    import numpy as np
    import torch
    from synth import CONFIGS, decode_step_inputs, make_inputs
    from token_level_sparse_pass_amd import hs2

    lib = hs2.load()
    w = CONFIGS[3]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_steps = args.warmup + args.steps
    cap = w.n_kv
    rng = np.random.default_rng(2024)
    lens0 = rng.integers(cap // 2, cap - n_steps - 1, size=w.batch).tolist()
    log(f"decode loop on {w.name}: generating the cache and {n_steps} steps of inputs")
    inp = make_inputs(w, device=dev, sparse_layers=0)
    k_cache, v_cache = inp["k"], inp["v"]
    xs = [decode_step_inputs(w, s, device=dev) for s in range(n_steps)]
    kw = dict(top_k=w.top_k, window=w.window)
    p = hs2.problem(k_cache.dtype, w.batch, 1, cap, w.h_q, w.h_kv, w.d, **kw)
    ws = hs2.alloc_workspace(p, dev)
    ps = args.page_size
    if ps:
        # the same memory as a pool of pages, handed out in shuffled order
        n_pages = w.batch * cap // ps
        perm = torch.from_numpy(np.random.default_rng(7).permutation(n_pages).astype(np.int32))
        table = perm.view(w.batch, cap // ps).to(dev)
        k_cache = k_cache.view(w.batch * cap, w.h_kv, w.d)
        v_cache = v_cache.view(w.batch * cap, w.h_kv, w.d)

    def step(x, lens, out):
        if ps:
            return hs2.decode_step_paged(x["q_full"], x["q_sparse"], x["k_new"], x["v_new"],
                                         k_cache, v_cache, table, ps, lens, workspace=ws,
                                         out=out, **kw)
        return hs2.decode_step(x["q_full"], x["q_sparse"], x["k_new"], x["v_new"], k_cache,
                               v_cache, lens, workspace=ws, out=out, **kw)

    lens = list(lens0)
    out = None
    for s in range(args.warmup):
        out = step(xs[s], lens, out)
        lens = [n + 1 for n in lens]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    keys_read = 0
    lib.hs2_profile_enable(1)
    torch.cuda.synchronize()
    ev0.record(stream)
    for s in range(args.warmup, n_steps):
        out = step(xs[s], lens, out)
        keys_read += sum(n + 1 for n in lens)
        lens = [n + 1 for n in lens]
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (ctypes.c_double * len(PASSES))()
    nl = (ctypes.c_int64 * len(PASSES))()
    st = lib.hs2_profile_read(ms, nl)
    lib.hs2_profile_enable(0)
    if st != 0:
        raise RuntimeError(lib.hs2_last_error().decode())
    ms_step = ev0.elapsed_time(ev1) / args.steps
    esz = 2
    kv_bytes = 2.0 * keys_read * w.h_kv * w.d * esz / args.steps      # K + V per step
    passes = {}
    for i, name in enumerate(PASSES):
        if nl[i] == 0:
            continue
        per = ms[i] / args.steps
        passes[name] = {"ms": round(per, 4), "launches_per_step": int(nl[i] // args.steps)}
    fa = passes["full_attention"]["ms"]
    ach = kv_bytes / (fa / 1e3) / 1e9
    rec = {"metric": "decode-loop tokens/s (one Hybrid Block step per new token, ragged batch)",
           "value": round(w.batch / (ms_step / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic (seeded; shapes and structure of the workload, no datasets)",
           "config": {"workload": w.name + "_decode_loop" + (f"_paged{ps}" if ps else ""),
                      "batch": w.batch, "capacity": cap, "page_size": ps or None,
                      "start_lengths": [int(min(lens0)), int(max(lens0))], "h_q": w.h_q,
                      "h_kv": w.h_kv, "head_dim": w.d, "top_k": w.top_k, "window": w.window,
                      "sparse_layers": w.n_sparse, "parallelism": "single GPU"},
           "roofline": {"kernel": "full_attention", "bound": "hbm", "achieved": round(ach, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                        "algorithmic_per_launch": kv_bytes, "traffic": None},
           "passes": passes, "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def kv_bridge_bench(args):
    """The KV Bridging projection for the 1M-token context: K and V of one
    Cross-Decoder full layer (8 KV heads x 128) from 1M hidden states of
    width 4096 (hidden width: a reading; the pages give none)."""
    import torch
    from synth import CONFIGS, bridge_inputs
    from token_level_sparse_pass_amd import hs2

    hs2.load()
    w = CONFIGS[5]
    d_model = 4096
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"KV bridge for {w.name}: generating {w.n_kv} hidden states of width {d_model}")
    x = bridge_inputs(w, d_model, device=dev)
    out = hs2.kv_bridge(x["hidden"], x["w_kv"], w.h_kv)
    for _ in range(args.warmup):
        hs2.kv_bridge(x["hidden"], x["w_kv"], w.h_kv, out=out)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        hs2.kv_bridge(x["hidden"], x["w_kv"], w.h_kv, out=out)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = 2.0 * w.batch * w.n_kv * d_model * 2 * w.h_kv * w.d
    ach = flops / (ms / 1e3) / 1e12
    rec = {"metric": "KV-bridge projection TFLOP/s (K and V of one full layer from hidden states)",
           "value": round(ach, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; shapes of the workload, random weights)",
           "config": {"workload": w.name + "_kv_bridge", "tokens": w.batch * w.n_kv,
                      "d_model": d_model, "h_kv": w.h_kv, "head_dim": w.d,
                      "parallelism": "single GPU"},
           "roofline": {"kernel": "kv_bridge", "bound": "mfma", "achieved": round(ach, 2),
                        "peak": PEAK_MFMA_TFLOPS["bf16"], "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_MFMA_TFLOPS["bf16"], 4),
                        "algorithmic_per_launch": flops, "traffic": None},
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def backward_work(w):
    """Per-step algorithmic work of each backward kernel (flops or bytes).

    Full layer, per causal (query, key) pair and query head: the products
    S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q and dQ += dS K, 2 d
    flops each. The dK/dV kernel performs the first four; the dQ kernel's
    own share is dQ (it recomputes S and dP, which is not counted).
    Preparation: Delta = rowsum(dO * O) (O, dO read, Delta written), the
    sparse layers' fp32 accumulators cleared and, for bf16 at head dim 128,
    K, Q and dO copied into the transposed tile layouts the dQ and dK/dV
    kernels read (each read once and written once, plus lse and Delta read
    and written again per row).
    Sparse layers: the K and V rows each query selects, gathered once per KV
    head; Q, O, dO read and dQ written for every layer; the fp32 K/V
    gradient rows read and written once per selected key.
    """
    esz = 2 if w.dtype == "bf16" else 4
    B, nq, nkv, hq, hkv, d, L = w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.d, w.n_sparse
    pos = [nkv - nq + i for i in range(nq)]
    pairs = sum(p + 1 for p in pos) * B
    sel = sum(min(p + 1, w.top_k + w.window) for p in pos) * B
    prep = 2.0 * B * nq * hq * d * esz + 4.0 * B * hq * nq + (2.0 * B * nkv * hkv * d * 4 if L else 0.0)
    if w.dtype == "bf16" and d == 128:
        # K^T copy, and Q / dO with their row statistics in transposed tiles
        prep += 2.0 * B * nkv * hkv * d * esz + 4.0 * B * nq * hq * d * esz + 16.0 * B * hq * nq
    return {
        "bwd_prep": ("hbm", prep),
        "bwd_sparse": ("hbm", sel * hkv * d * 2.0 * esz + 4.0 * L * B * nq * hq * d * esz +
                       sel * hkv * d * 2.0 * 4 * 2),
        "bwd_dkdv": ("mfma", 8.0 * hq * d * pairs),
        "bwd_dq": ("mfma", 2.0 * hq * d * pairs),
    }


def backward_cpu_baseline(w, inp, grads, idx, n_rows=64):
    """The oracle's backward (block_backward_tail) for the last n_rows
    queries of sequence 0: each query's complete gradient work."""
    from oracle import hs2_oracle as O
    from synth import to_host
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [cores])
    except Exception:
        pass
    n_rows = min(n_rows, w.n_q)
    j_lo = w.n_kv - n_rows
    t0 = time.perf_counter()
    O.block_backward_tail(to_host(inp["q_full"][:1]), to_host(inp["q_sparse"][:, :1]),
                          to_host(inp["k"][:1]), to_host(inp["v"][:1]), to_host(idx[:1]),
                          to_host(grads["do_full"][:1]), to_host(grads["do_sparse"][:, :1]),
                          0, j_lo)
    t = time.perf_counter() - t0
    return {"value": n_rows / t, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            **host_cpu(),
            "sample": f"the last {n_rows} queries of sequence 0 of {w.name}: their dQ (full "
                      f"and {w.n_sparse} sparse layers) and every K/V-gradient contribution "
                      f"they make, over all {w.n_kv} keys, {t:.1f} s"}


def backward_bench(args):
    """Backward pass of the block (fine-tuning) on the 32K-token prefill
    workload by default: the forward runs once, then K timed backward steps
    over its outputs and index sets."""
    import torch
    from synth import CONFIGS, grad_inputs, make_inputs
    from token_level_sparse_pass_amd import hs2

    lib = hs2.load()
    w = CONFIGS[args.bwd_config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"backward on {w.name}: generating inputs")
    inp = make_inputs(w, device=dev)
    grads = grad_inputs(w, device=dev)
    kw = dict(top_k=w.top_k, window=w.window)
    fwd = hs2.block_forward(inp["q_full"], inp["q_sparse"], inp["k"], inp["v"], **kw)
    torch.cuda.synchronize()
    log("forward done")
    p = hs2.problem(inp["q_full"].dtype, w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.d, **kw)
    ws = torch.empty(hs2.backward_workspace_size(p, w.n_sparse), dtype=torch.uint8, device=dev)
    args_ = (inp["q_full"], inp["q_sparse"], inp["k"], inp["v"], fwd["o_full"], fwd["o_sparse"],
             fwd["lse"], fwd["idx"], grads["do_full"], grads["do_sparse"])
    bkw = dict(kw, deterministic=args.deterministic)
    out = None
    for s in range(args.warmup):
        out = hs2.block_backward(*args_, workspace=ws, out=out, **bkw)
        torch.cuda.synchronize()
        log(f"warmup step {s + 1}/{args.warmup} done")
    if out is None:
        out = hs2.block_backward(*args_, workspace=ws, **bkw)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lib.hs2_profile_enable(1)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        hs2.block_backward(*args_, workspace=ws, out=out, **bkw)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (ctypes.c_double * len(PASSES))()
    nl = (ctypes.c_int64 * len(PASSES))()
    st = lib.hs2_profile_read(ms, nl)
    lib.hs2_profile_enable(0)
    if st != 0:
        raise RuntimeError(lib.hs2_last_error().decode())
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step")
    work = backward_work(w)
    peak_mfma = PEAK_MFMA_TFLOPS[w.dtype]
    passes = {}
    workload_name = w.name + ("_backward_deterministic" if args.deterministic else "_backward")
    for i, name in enumerate(PASSES):
        if nl[i] == 0 or name not in work:
            continue
        bound, amount = work[name]
        per = ms[i] / args.steps
        if bound == "mfma":
            ach = amount / (per / 1e3) / 1e12
            passes[name] = {"ms": round(per, 4), "launches_per_step": int(nl[i] // args.steps),
                            "bound": "mfma", "achieved": round(ach, 2), "unit": "TFLOP/s",
                            "frac": round(ach / peak_mfma, 4)}
        else:
            passes[name] = hbm_pass(per, nl[i] // args.steps, amount, name, workload_name)
    dom = max(passes, key=lambda n: passes[n]["ms"])
    d = passes[dom]
    # the roofline counts the dominant kernel's algorithmic work
    hbm = d["bound"] == "hbm"
    roofline = {"kernel": dom, "bound": d["bound"],
                "achieved": d["effective_GBs"] if hbm else d["achieved"],
                "peak": peak_mfma if d["bound"] == "mfma" else PEAK_HBM_GBS, "unit": d["unit"],
                "frac": d["effective_frac"] if hbm else d["frac"],
                "algorithmic_per_launch": work[dom][1] / max(1, d["launches_per_step"]),
                "traffic": None}
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle's backward on a sample of queries")
        cpu = backward_cpu_baseline(w, inp, grads, fwd["idx"])
    tokens = w.batch * w.n_q
    rec = {"metric": "backward tokens/s (Hybrid Block with its index sets held fixed)",
           "value": round(tokens / (ms_step / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic (seeded; shapes and structure of the workload, no datasets)",
           "config": {"workload": w.name + ("_backward_deterministic" if args.deterministic
                                            else "_backward"), "batch": w.batch, "n_q": w.n_q,
                      "n_kv": w.n_kv, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d,
                      "top_k": w.top_k, "window": w.window, "sparse_layers": w.n_sparse,
                      "parallelism": "single GPU"},
           "roofline": roofline, "passes": passes, "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def varlen_bench(args, paged=False):
    """A packed batch of agent turns of different lengths
    (hs2_block_forward_varlen): 8 sequences with contexts of 32K-262K keys,
    each appending a new chunk of 256-4096 tokens (lengths drawn from a
    seeded generator), the 8K-on-262K workload's heads and 5 sparse layers.
    paged: the same turns through hs2_block_forward_paged, the cached
    context in shuffled 256-row pages of a pool; every step appends the
    chunks at the same positions, so each step sees the same cache."""
    import dataclasses
    import numpy as np
    import torch
    from synth import CONFIGS, make_inputs
    from token_level_sparse_pass_amd import hs2

    lib = hs2.load()
    base = CONFIGS[4]
    rng = np.random.default_rng([base.cid, 77])
    n_seq = 8
    nkv = rng.integers(32768, 262144 + 1, size=n_seq)
    nq = np.minimum(rng.integers(256, 4096 + 1, size=n_seq), nkv)
    cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(nkv)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_kv[-1])
    w = dataclasses.replace(base, name=base.name + "_varlen", n_q=tq, n_kv=tk, structure="none")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"varlen: {n_seq} sequences, {tq} queries over {tk} keys")
    inp = make_inputs(w, device=dev)
    q, qs = inp["q_full"][0].contiguous(), inp["q_sparse"][:, 0].contiguous()
    k, v = inp["k"][0].contiguous(), inp["v"][0].contiguous()
    kw = dict(top_k=w.top_k, window=w.window)
    if paged:
        # sequence b's positions 0 .. nkv[b] - 1 live in pages of 256 rows,
        # handed out in a seeded shuffled order; its last nq[b] keys are the
        # chunk the call appends, the rest are already cached
        ps = 256
        mp = int(-(-nkv.max() // ps))
        n_pages = int(sum(-(-n // ps) for n in nkv.tolist())) + 1
        perm = rng.permutation(n_pages)
        table = np.zeros((n_seq, mp), dtype=np.int32)
        pool_idx = np.zeros(tk, dtype=np.int64)
        used = 0
        for b, n in enumerate(nkv.tolist()):
            np_b = -(-n // ps)
            table[b, :np_b] = perm[used:used + np_b]
            used += np_b
            j = np.arange(n)
            pool_idx[cu_kv[b]:cu_kv[b] + n] = table[b, j // ps].astype(np.int64) * ps + j % ps
        k_pool = torch.zeros((n_pages * ps, w.h_kv, w.d), dtype=k.dtype, device=dev)
        v_pool = torch.zeros_like(k_pool)
        pidx = torch.from_numpy(pool_idx).to(dev)
        k_pool[pidx] = k
        v_pool[pidx] = v
        new_rows = torch.from_numpy(np.concatenate(
            [np.arange(cu_kv[b + 1] - nq[b], cu_kv[b + 1]) for b in range(n_seq)])).to(dev)
        k_new, v_new = k[new_rows].contiguous(), v[new_rows].contiguous()
        del k, v, inp
        lens = (nkv - nq).tolist()
        table_d = torch.from_numpy(table).to(dev)
        p, pages = hs2._paged_problem(q, k_pool, table_d, ps, n_seq, kw)
        _, pref = hs2.workspace_size_paged(p, pages, cu_q, lens)
        ws = torch.empty(pref, dtype=torch.uint8, device=dev)

        def run():
            hs2.block_forward_paged(q, qs, k_new, v_new, k_pool, v_pool, table_d, ps, cu_q, lens,
                                    workspace=ws, **kw)
    else:
        p = hs2.problem(q.dtype, n_seq, 1, 1, w.h_q, w.h_kv, w.d, **kw)
        _, pref = hs2.workspace_size_varlen(p, cu_q, cu_kv)
        ws = torch.empty(pref, dtype=torch.uint8, device=dev)

        def run():
            hs2.block_forward_varlen(q, qs, k, v, cu_q, cu_kv, workspace=ws, **kw)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lib.hs2_profile_enable(1)
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (ctypes.c_double * len(PASSES))()
    nl = (ctypes.c_int64 * len(PASSES))()
    st = lib.hs2_profile_read(ms, nl)
    lib.hs2_profile_enable(0)
    if st != 0:
        raise RuntimeError(lib.hs2_last_error().decode())
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # algorithmic work: the sum over sequences, each a batch-1 block
    work = {}
    for a_, b_ in zip(nq.tolist(), nkv.tolist()):
        ws_ = dataclasses.replace(base, batch=1, n_q=int(a_), n_kv=int(b_))
        for name, (bound, amount) in algorithmic_work(ws_).items():
            work[name] = (bound, work.get(name, (bound, 0.0))[1] + amount)
        # staging (paged): K and V rows read once (pool or new rows) and
        # written once to the staging copy, and the new rows to the pool
        row_b = w.h_kv * w.d * (2 if w.dtype == "bf16" else 4)
        stage = 2.0 * row_b * (2 * b_ + a_) if a_ >= 2 else 2.0 * row_b * 2 * a_
        work["kv_stage"] = ("hbm", work.get("kv_stage", ("hbm", 0.0))[1] + stage)
    peak_mfma = PEAK_MFMA_TFLOPS[w.dtype]
    passes = {}
    workload_name = "agent_turns_bf16_" + ("paged256" if paged else "varlen")
    for i, name in enumerate(PASSES):
        if nl[i] == 0 or name not in work:
            continue
        bound, amount = work[name]
        per = ms[i] / args.steps
        if bound == "mfma":
            ach = amount / (per / 1e3) / 1e12
            passes[name] = {"ms": round(per, 4), "launches_per_step": int(nl[i] // args.steps),
                            "bound": "mfma", "achieved": round(ach, 2), "unit": "TFLOP/s",
                            "frac": round(ach / peak_mfma, 4)}
        else:
            passes[name] = hbm_pass(per, nl[i] // args.steps, amount, name, workload_name)
    dom = max(passes, key=lambda n: passes[n]["ms"])
    d = passes[dom]
    metric = "varlen batch tokens/s (packed agent turns of different lengths)"
    if paged:
        metric = "paged chunked-prefill tokens/s (agent turns appended to a paged KV pool)"
    rec = {"metric": metric,
           "value": round(tq / (ms_step / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic (seeded lengths and values; no datasets)",
           "config": {"workload": "agent_turns_bf16_" + ("paged256" if paged else "varlen"),
                      "sequences": n_seq,
                      "n_q": nq.tolist(), "n_kv": nkv.tolist(), "h_q": w.h_q, "h_kv": w.h_kv,
                      "head_dim": w.d, "top_k": w.top_k, "window": w.window,
                      "sparse_layers": w.n_sparse, "parallelism": "single GPU"},
           "roofline": {"kernel": dom, "bound": d["bound"],
                        "achieved": d["effective_GBs"] if d["bound"] == "hbm" else d["achieved"],
                        "peak": peak_mfma if d["bound"] == "mfma" else PEAK_HBM_GBS,
                        "unit": d["unit"],
                        "frac": d["effective_frac"] if d["bound"] == "hbm" else d["frac"],
                        "traffic": None},
           "passes": passes, "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-loop", action="store_true",
                    help="time decode steps over a growing ragged cache (the 64 x 128K decode "
                         "workload) instead of the default workload")
    ap.add_argument("--kv-bridge", action="store_true",
                    help="time the KV Bridging projection for the 1M-token context instead")
    ap.add_argument("--select", choices=["token", "block"], default="token",
                    help="selection of the timed block: token top-k (the method) or the "
                         "64-token block ablation")
    ap.add_argument("--varlen", action="store_true",
                    help="time a packed batch of agent turns of different lengths instead")
    ap.add_argument("--paged", action="store_true",
                    help="the --varlen batch through the paged-pool entry point (chunked "
                         "prefill over 256-row pages) instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (fixed index sets) instead")
    ap.add_argument("--deterministic", action="store_true",
                    help="with --backward: time hs2_block_backward_deterministic")
    ap.add_argument("--bwd-config", type=int, default=2,
                    help="with --backward: the workload (default 2, the 32K-token prefill)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="with --decode-loop: keep the cache in a pool of pages of this many "
                         "rows, handed out in shuffled order (hs2_decode_step_paged)")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="host only: summarise a rocprofv3 --kernel-trace --stats run of "
                         "--config N under DIR into profiles/ and exit")
    ap.add_argument("--counters-summary", metavar="DIR", default=None,
                    help="host only: summarise rocprofv3 --pmc runs under DIR into profiles/ "
                         "and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read MIB, write MIB) "
                         "three times, to scale HBM byte counters, and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Hybrid Block hot path here is a "
              "single-GPU build (no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.counters_summary:
        counters_summary(args.counters_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.config)
        return
    import torch
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)          # one elementwise kernel: n bytes in, n out
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel": "elementwise neg (float32)", "bytes_read": n,
                          "bytes_written": n, "launches": 3}), flush=True)
        return
    if args.decode_loop:
        decode_loop(args)
        return
    if args.kv_bridge:
        kv_bridge_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.varlen or args.paged:
        varlen_bench(args, paged=args.paged)
        return
    from synth import CONFIGS, make_inputs
    from token_level_sparse_pass_amd import hs2

    lib = hs2.load()
    w = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {w.name}: generating inputs")
    inp = make_inputs(w, device=dev)
    kw = dict(top_k=w.top_k, window=w.window)
    if args.select == "block":
        kw.update(select="block", block_size=w.block_size, top_blocks=w.top_blocks)
    p = hs2.problem(inp["q_full"].dtype, w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.d, **kw)
    ws = hs2.alloc_workspace(p, dev)
    out = None
    args_ = (inp["q_full"], inp["q_sparse"], inp["k"], inp["v"])
    for s in range(args.warmup):
        out = hs2.block_forward(*args_, workspace=ws, out=out, **kw)
        torch.cuda.synchronize()
        log(f"warmup step {s + 1}/{args.warmup} done")
    if out is None:
        out = hs2.block_forward(*args_, workspace=ws, **kw)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lib.hs2_profile_enable(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for s in range(args.steps):
        hs2.block_forward(*args_, workspace=ws, out=out, **kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = (ctypes.c_double * len(PASSES))()
    nl = (ctypes.c_int64 * len(PASSES))()
    st = lib.hs2_profile_read(ms, nl)
    lib.hs2_profile_enable(0)
    if st != 0:
        raise RuntimeError(lib.hs2_last_error().decode())
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f})")
    tokens = w.batch * w.n_q
    value = tokens / (ms_step / 1e3)

    work = algorithmic_work(w)
    peak_mfma = PEAK_MFMA_TFLOPS[w.dtype]
    passes = {}
    for i, name in enumerate(PASSES):
        if nl[i] == 0:
            continue                      # pass not taken on this path
        bound, amount = work[name]
        per_step_ms = ms[i] / args.steps
        launches = nl[i] // args.steps
        secs = per_step_ms / 1e3 if per_step_ms > 0 else float("inf")
        if bound == "mfma":
            ach = amount / secs / 1e12
            passes[name] = {"ms": round(per_step_ms, 4), "launches_per_step": int(launches),
                            "bound": "mfma", "achieved": round(ach, 2), "unit": "TFLOP/s",
                            "frac": round(ach / peak_mfma, 4)}
            mc = committed_counters("mfma", name, w.name)
            if mc is not None:
                # rocprof's own count of the MFMA flops this pass executes,
                # over the live time, and its MFMA-busy fraction
                rate = mc["mfma_flops_per_step"] / secs / 1e12
                passes[name]["rocprof"] = {
                    "mfma_tflops": round(rate, 2), "mfma_frac": round(rate / peak_mfma, 4),
                    "mfma_busy": mc["mfma_busy"], "valu_per_mfma": mc["valu_per_mfma"]}
        else:
            # HBM fraction from the committed FETCH/WRITE counters (null without
            # them); "effective" counts every algorithmic byte, including those
            # that the caches serve, so it can exceed the HBM peak
            eff = amount / secs / 1e9
            tr = committed_counters("traffic", name, w.name)
            ach = None if tr is None else tr["bytes_per_step"] / secs / 1e9
            passes[name] = {"ms": round(per_step_ms, 4), "launches_per_step": int(launches),
                            "bound": "hbm",
                            "achieved": None if ach is None else round(ach, 1), "unit": "GB/s",
                            "frac": None if ach is None else round(ach / PEAK_HBM_GBS, 4),
                            "effective_GBs": round(eff, 1),
                            "effective_frac": round(eff / PEAK_HBM_GBS, 4)}
    dom = max(passes, key=lambda n: passes[n]["ms"])
    d = passes[dom]
    per_launch = work[dom][1] / max(1, d["launches_per_step"])
    traffic = measured_traffic(dom, w.name)
    # the dominant kernel: algorithmic work per launch over its live time
    ach = per_launch * d["launches_per_step"] / (d["ms"] / 1e3) / (1e12 if d["bound"] == "mfma"
                                                                  else 1e9)
    peak = peak_mfma if d["bound"] == "mfma" else PEAK_HBM_GBS
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": round(ach, 2),
                "peak": peak, "unit": d["unit"], "frac": round(ach / peak, 4),
                "algorithmic_per_launch": per_launch,
                "traffic": traffic}
    if "rocprof" in d:
        roofline["rocprof"] = d["rocprof"]

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a sample of rows")
        cpu = cpu_baseline(w, inp)

    rec = {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic (seeded; shapes and structure of the workload, no datasets)",
           "config": {"workload": w.name, "batch": w.batch, "n_q": w.n_q, "n_kv": w.n_kv,
                      "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d, "top_k": w.top_k,
                      "window": w.window, "sparse_layers": w.n_sparse, "select": args.select,
                      "structure": w.structure, "parallelism": "single GPU"},
           "roofline": roofline, "passes": passes, "cpu_baseline": cpu,
           "quality": selection_quality(w, inp["meta"], out["idx"])}
    print(json.dumps(rec), flush=True)


def selection_quality(w, meta, idx):
    """How much of the planted structure the selection found (a sanity
    figure, not parity): needle workloads, the fraction of needles their
    target query selects; cluster workloads, the mean over query rows of the
    fraction of the clustered tokens the row selects. None otherwise."""
    import torch
    if meta.get("structure") == "needles":
        hits = 0
        for j, t in zip(meta["needle_pos"].tolist(), meta["needle_target"].tolist()):
            row = idx[0, int(t) - w.q_off]
            hits += int(bool((row == int(j)).any()))
        return {"needle_hits": hits, "needles": len(meta["needle_pos"]),
                "fraction": round(hits / max(1, len(meta["needle_pos"])), 4)}
    if meta.get("structure") == "clusters":
        mark = torch.zeros(w.n_kv + 1, dtype=torch.int32, device=idx.device)
        pos = torch.as_tensor(meta["cluster_pos"], dtype=torch.long, device=idx.device)
        mark[pos] = 1
        got = mark[torch.where(idx >= 0, idx, w.n_kv).long()].sum(-1).float()   # [B, n_q]
        recall = got / float(len(meta["cluster_pos"]))
        return {"cluster_tokens": int(len(meta["cluster_pos"])),
                "mean_recall": round(float(recall.mean()), 4),
                "min_recall": round(float(recall.min()), 4)}
    return None


if __name__ == "__main__":
    main()
