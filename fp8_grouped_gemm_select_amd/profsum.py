"""Summaries of rocprofv3 CSV output for the layer benchmark.

    python -m fp8_grouped_gemm_select_amd.profsum trace  TRACE_CSV --workload W --command CMD --out MD
    python -m fp8_grouped_gemm_select_amd.profsum traffic FETCH_CSV WRITE_CSV --calib-bytes N
                                                  --workload W --command CMD --out-json J --out-md MD
    python -m fp8_grouped_gemm_select_amd.profsum counters CSV [CSV ...] --workload W
                                                  --command CMD [--command CMD] --out MD

`trace` reads a `--kernel-trace` CSV (one row per dispatch) and writes a
markdown table of calls / total / average duration per kernel, with the two
grouped-GEMM launches of a layer pass (w13 first, then w2) split apart.

`counters` summarises any other `--pmc` CSVs per stage (MFMA busy share,
FP8 matrix flop, L2 hit rate).

`traffic` reads two `--pmc` counter CSVs of the same command (FETCH_SIZE, then
WRITE_SIZE, both in KiB per dispatch) and converts them to bytes per launch of
every stage. The counters are scaled by what they read for the plain device
copy of `calib-bytes` bytes that the benchmark issues after its timed steps
(`--calib-copy-mib`): factor = calib_bytes / (counter KiB * 1024). The JSON
records a hash of each stage's kernel source so that the benchmark reports
traffic only for kernels that have not changed since the counters were taken.
"""
import argparse
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

STAGES = ["select", "pre_reorder", "gemm_w13", "act_requant", "gemm_w2", "post_reorder"]
STAGE_SOURCE = {"select": "select_experts.hip", "pre_reorder": "pre_reorder.hip",
                "gemm_w13": "grouped_gemm.hip", "gemm_w2": "grouped_gemm.hip",
                "act_requant": "act_requant.hip", "post_reorder": "post_reorder.hip"}


def source_hash(stage: str) -> str:
    """sha256 over the stage's kernel source and the shared device header."""
    h = hashlib.sha256()
    for name in (STAGE_SOURCE[stage], "common.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(kernel: str) -> str:
    k = kernel
    if k.startswith("void "):
        k = k[5:]
    for prefix in ("moe::(anonymous namespace)::", "moe::", "(anonymous namespace)::"):
        if k.startswith(prefix):
            k = k[len(prefix):]
    return k.split("(")[0]


def stage_of(kernel: str):
    k = short_name(kernel)
    if k.startswith("select_experts") or k.startswith("select_rows"):
        return "select"
    if k.startswith("pr_"):
        return "pre_reorder"
    if k.startswith("grouped_gemm"):
        return "gemm"
    if k.startswith("act_"):
        return "act_requant"
    if k.startswith("post_reorder"):
        return "post_reorder"
    return None


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _assign_gemm(dispatches):
    """Label grouped-GEMM dispatches w13 / w2 by their order within the run."""
    out, n = [], 0
    for d in dispatches:
        st = stage_of(d["name"])
        if st == "gemm":
            st = "gemm_w13" if n % 2 == 0 else "gemm_w2"
            n += 1
        out.append(dict(d, stage=st))
    return out


def load_trace(path):
    ds = []
    for r in _rows(path):
        ds.append(dict(id=int(r["Dispatch_Id"]), name=r["Kernel_Name"],
                       dur_us=(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    ds.sort(key=lambda d: d["id"])
    return _assign_gemm(ds)


def trace_md(path, workload, command):
    ds = load_trace(path)
    total = sum(d["dur_us"] for d in ds)
    per = {}
    for d in ds:
        p = per.setdefault(short_name(d["name"]), [0, 0.0])
        p[0] += 1
        p[1] += d["dur_us"]
    lines = [f"# Kernel trace: whole layer, workload `{workload}`", "",
             "Command (from /tmp on the GPU host, repository at $REPO):", "", f"    {command}", "",
             "Durations are End - Start of each dispatch in the kernel-trace CSV.", "",
             "| kernel | calls | total (us) | average (us) | % of GPU time |", "|---|---|---|---|---|"]
    for k, (n, t) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{k}` | {n} | {t:.1f} | {t / n:.2f} | {100 * t / total:.1f} |")
    lines += ["", "Per stage of the layer pass (grouped-GEMM launches split by position: w13 first, then w2):",
              "", "| stage | launches | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    n_pass = sum(1 for d in ds if d["stage"] == "select")
    for st in STAGES:
        v = [d["dur_us"] for d in ds if d["stage"] == st]
        if st == "pre_reorder" or len(v) > n_pass:  # several kernels per stage: sum per layer pass
            v = _per_pass_sums(ds, st)
        if v:
            lines.append(f"| {st} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines) + "\n"


SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE reads the sum over the 8 XCDs


def load_counters(paths):
    """Every (dispatch, counter) value of one or more `--pmc` CSVs, stages
    assigned per file (the w13 / w2 split by GEMM order within each run), and
    the layer pass each dispatch belongs to (a pass starts at stage 1)."""
    per = {}
    for path in paths:
        names = sorted({r["Counter_Name"] for r in _rows(path)})
        for name in names:
            for d in load_counter(path, name):
                if d["stage"] is None:
                    continue
                key = (path, d["id"])
                e = per.setdefault(key, {"stage": d["stage"]})
                e[name] = d["value"]
        for r in _rows(path):
            key = (path, int(r["Dispatch_Id"]))
            if key in per and "dur_us" not in per[key] and r.get("End_Timestamp"):
                per[key]["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out, npass, cur_path = [], -1, None
    for (path, _), e in sorted(per.items(), key=lambda kv: kv[0]):
        if path != cur_path:
            cur_path, npass = path, -1
        if e["stage"] == "select":
            npass += 1
        out.append(dict(e, run=(path, npass)))
    return out


def counters_md(paths, workload, commands):
    """Per stage: mean counter values per dispatch and the figures derived from
    them (MFMA busy share of SIMD cycles, FP8 matrix flop from the MOPS counter,
    L2 hit rate)."""
    ds = load_counters(paths)
    lines = [f"# Hardware counters per stage, workload `{workload}`", "",
             "Commands (from /tmp on the GPU host, repository at $REPO):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Median over layer passes of each stage's dispatches summed. GRBM_GUI_ACTIVE reads the sum over the "
              f"{XCDS} XCDs, so one XCD's busy cycles are a {XCDS}th of it (it also counts a fixed "
              "few microseconds around each dispatch, which dominates the short kernels). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
              f"(GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs); FP8 flop = SQ_INSTS_VALU_MFMA_MOPS_F8 x "
              "512 (the MFMA work issued, padded tiles included); L2 hit = TCC_HIT / (TCC_HIT + "
              "TCC_MISS).", "",
              "| stage | dispatches | µs | MFMA busy | FP8 GFLOP issued | L2 hit |",
              "|---|---|---|---|---|---|"]
    for st in STAGES:
        rows = [d for d in ds if d["stage"] == st]
        if not rows:
            continue
        # per layer pass: the stage's dispatches summed (stage 2 has three kernels)
        by_pass = {}
        for d in rows:
            acc = by_pass.setdefault(d["run"], {})
            for k, v in d.items():
                if k not in ("stage", "run"):
                    acc[k] = acc.get(k, 0.0) + v

        def mean(name):  # the median over passes (the first pass can stray)
            v = sorted(p[name] for p in by_pass.values() if name in p)
            return v[len(v) // 2] if v else None

        gui, busy = mean("GRBM_GUI_ACTIVE"), mean("SQ_VALU_MFMA_BUSY_CYCLES")
        mops, hit, miss = mean("SQ_INSTS_VALU_MFMA_MOPS_F8"), mean("TCC_HIT_sum"), mean("TCC_MISS_sum")
        dur = mean("dur_us")
        n = max(sum(1 for d in rows if k in d) for k in rows[0] if k not in ("stage", "dur_us", "run"))
        xcd_cycles = gui / XCDS if gui else None
        util = f"{100 * busy / (xcd_cycles * SIMDS):.1f} %" if xcd_cycles and busy is not None else "—"
        gf = f"{mops * 512 / 1e9:.1f}" if mops is not None else "—"
        l2 = f"{100 * hit / (hit + miss):.1f} %" if hit is not None and miss is not None and hit + miss else "—"
        ds_us = f"{dur:.1f}" if dur else "—"
        lines.append(f"| {st} | {n} | {ds_us} | {util} | {gf} | {l2} |")
    return "\n".join(lines) + "\n"


def stats_md(path):
    """The profiler's own per-kernel summary (`--stats`), names shortened."""
    lines = ["", "rocprofv3 `--stats` kernel summary of the same run:", "",
             "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in _rows(path):
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(lines) + "\n"


def bench_md(path):
    """The benchmark line the profiled command printed (its last JSON line):
    headline figures, the roofline object and the on-box ceilings, if any."""
    line = None
    with open(path) as f:
        for raw in f:
            raw = raw.strip()
            if raw.startswith("{") and raw.endswith("}"):
                line = raw
    if line is None:
        return ""
    d = json.loads(line)
    lines = ["", "Benchmark line of the same run (under the profiler, so slower than an unprofiled run):", "",
             f"- {d.get('metric')}: {d.get('value')} {d.get('unit')}, {d.get('ms_per_step')} ms per step",
             f"- roofline: `{json.dumps(d.get('roofline'))}`"]
    if d.get("ceilings"):
        lines.append(f"- on-box ceilings: `{json.dumps(d['ceilings'])}`")
    return "\n".join(lines) + "\n"


def _per_pass_sums(ds, stage, key="dur_us"):
    """Sum `key` over the kernels of a multi-kernel stage within each layer pass
    (a pass starts at every select_experts dispatch)."""
    sums, cur, seen = [], 0.0, False
    for d in ds:
        if d["stage"] == "select":
            if seen:
                sums.append(cur)
            cur, seen = 0.0, True
        elif d["stage"] == stage:
            cur += d[key]
    if seen:
        sums.append(cur)
    return sums


def load_counter(path, counter):
    ds = []
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        ds.append(dict(id=int(r["Dispatch_Id"]), name=r["Kernel_Name"], value=float(r["Counter_Value"])))
    ds.sort(key=lambda d: d["id"])
    return _assign_gemm(ds)


def _calib(ds, calib_bytes):
    """Counter reading (KiB) of the calibration copy: the last copy dispatch."""
    copies = [d for d in ds if "copy" in d["name"].lower() and d["stage"] is None]
    if not copies:
        raise SystemExit("no copy dispatch found for calibration")
    kib = copies[-1]["value"]
    return calib_bytes / (kib * 1024.0), kib


def traffic(fetch_csv, write_csv, calib_bytes, workload, command):
    fd, wd = load_counter(fetch_csv, "FETCH_SIZE"), load_counter(write_csv, "WRITE_SIZE")
    ff, fkib = _calib(fd, calib_bytes)
    wf, wkib = _calib(wd, calib_bytes)
    stages = {}
    for st in STAGES:
        fv = _per_pass(fd, st)
        wv = _per_pass(wd, st)
        if not fv or not wv:
            continue
        f_b = sum(fv) / len(fv) * 1024.0 * ff
        w_b = sum(wv) / len(wv) * 1024.0 * wf
        stages[st] = dict(fetch_bytes=round(f_b), write_bytes=round(w_b), traffic_bytes=round(f_b + w_b),
                          launches=len(fv), source=STAGE_SOURCE[st], source_sha256=source_hash(st))
    return dict(workload=workload, command=command, calib_bytes=calib_bytes,
                calib_fetch_kib=fkib, calib_write_kib=wkib, fetch_factor=ff, write_factor=wf,
                stages=stages)


def _per_pass(ds, stage):
    if stage == "pre_reorder":
        return _per_pass_sums(ds, stage, "value")
    return [d["value"] for d in ds if d["stage"] == stage]


def traffic_md(t):
    lines = [f"# HBM traffic per launch, workload `{t['workload']}`", "",
             "Commands (from /tmp on the GPU host, repository at $REPO):", ""]
    lines += [f"    {c}" for c in t["command"].split(" && ")]
    lines += ["", f"Counters in KiB per dispatch, scaled by the plain copy of {t['calib_bytes']} bytes that "
              f"the benchmark issues after its timed steps: FETCH_SIZE read {t['calib_fetch_kib']:.0f} KiB "
              f"for it (factor {t['fetch_factor']:.4f}), WRITE_SIZE {t['calib_write_kib']:.0f} KiB "
              f"(factor {t['write_factor']:.4f}).", "",
              "| stage | launches | fetch (MB) | write (MB) | traffic (MB) |", "|---|---|---|---|---|"]
    for st, v in t["stages"].items():
        lines.append(f"| {st} | {v['launches']} | {v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} "
                     f"| {v['traffic_bytes'] / 1e6:.2f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("trace")
    a.add_argument("csv")
    a.add_argument("--workload", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--stats", help="the run's --stats kernel summary CSV, appended as a table")
    a.add_argument("--bench-log", help="the profiled benchmark's output; its JSON line is appended")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--calib-bytes", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--out-json", required=True)
    b.add_argument("--out-md", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--out", required=True)
    args = p.parse_args(argv)
    if args.cmd == "counters":
        with open(args.out, "w") as f:
            f.write(counters_md(args.csv, args.workload, args.command))
        return
    if args.cmd == "trace":
        with open(args.out, "w") as f:
            f.write(trace_md(args.csv, args.workload, args.command))
            if args.stats:
                f.write(stats_md(args.stats))
            if args.bench_log:
                f.write(bench_md(args.bench_log))
    else:
        t = traffic(args.fetch_csv, args.write_csv, args.calib_bytes, args.workload, args.command)
        with open(args.out_json, "w") as f:
            json.dump(t, f, indent=1)
        with open(args.out_md, "w") as f:
            f.write(traffic_md(t))


if __name__ == "__main__":
    sys.exit(main())
