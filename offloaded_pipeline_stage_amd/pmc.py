"""HBM traffic of the step's kernels from rocprofv3 counter runs.

Two `rocprofv3 --pmc` passes of the same bench command, one collecting
FETCH_SIZE and one WRITE_SIZE (KiB per dispatch), are reduced here to
bytes per launch for every kernel. Both counters are calibrated against a
plain device-to-device copy of known size (the library's copy16_kernel,
16 bytes per lane like its other kernels) that the bench command runs before
its steps (`--copy-calibration-mib`): the scale factor is the copy's known bytes
divided by what the counter reports for it.

The summary records, for each kernel, a hash of the source file that
defines it and of the library's headers; `traffic_for` returns None when
any of them has changed since the counters were taken, so a stale figure is
never reported for a new kernel.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_KERNEL = "copy16_kernel"


def norm_name(name: str) -> str:
    """rocprofv3's demangled name -> the library's trace name form:
    no return type, namespaces or argument list; bools as 0/1."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):  # cut the argument list (the first '(' outside <>)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            n = n[:i]
            break
    n = n.replace("(anonymous namespace)::", "")
    n = re.sub(r"\brp::", "", n)
    n = re.sub(r"\btrue\b", "1", n)
    n = re.sub(r"\bfalse\b", "0", n)
    return n


def base_name(n: str) -> str:
    return n.split("<", 1)[0]


def kernel_source(base: str) -> str | None:
    """The csrc file that defines __global__ `base`."""
    pat = re.compile(r"__global__[^;{]*?\b" + re.escape(base) + r"\s*\(", re.S)
    for p in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        if pat.search(open(p).read()):
            return p
    return None


def source_hash(path: str) -> str:
    """Hash of the file that defines a kernel together with every header of
    the library (a kernel's code also comes from the helpers it includes)."""
    h = hashlib.sha256(open(path, "rb").read())
    for hp in sorted(glob.glob(os.path.join(CSRC, "*.h"))):
        h.update(open(hp, "rb").read())
    return h.hexdigest()[:16]


def _dispatches(path: str, counter: str):
    """[(dispatch_id, kernel_name, value)] of one counter, in dispatch order."""
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name", counter) != counter:
                continue
            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    out.sort()
    return out


def _find_csv(d: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    return hits[0]


def summarize(fetch_dir: str, write_dir: str, copy_mib: int, title: str, commands: list[str]) -> str:
    """Text summary of the two counter runs (one table + one JSON line)."""
    copy_kib = copy_mib * 1024.0
    per = {}
    factors = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _dispatches(_find_csv(d), counter)
        cal = [v for _, k, v in rows if COPY_KERNEL in k]
        if not cal:
            raise RuntimeError(f"{counter}: the calibration copy is missing from {d}")
        # the calibration copy is the process's first copy16_kernel launch
        factors[counter] = copy_kib / cal[0]
        agg = defaultdict(lambda: [0, 0.0])
        for _, k, v in rows:
            a = agg[norm_name(k)]
            a[0] += 1
            a[1] += v
        per[counter] = agg
    names = sorted(set(per["FETCH_SIZE"]) | set(per["WRITE_SIZE"]))
    table = {}
    for n in names:
        cf, sf = per["FETCH_SIZE"].get(n, [0, 0.0])
        cw, sw = per["WRITE_SIZE"].get(n, [0, 0.0])
        if cf == 0 or cw == 0:
            continue
        src = kernel_source(base_name(n))
        table[n] = {
            "launches": cf,
            "fetch_bytes": sf / cf * 1024.0 * factors["FETCH_SIZE"],
            "write_bytes": sw / cw * 1024.0 * factors["WRITE_SIZE"],
            "fetch_kib_raw": sf / cf, "write_kib_raw": sw / cw,
            "source": os.path.basename(src) if src else None,
            "source_sha": source_hash(src) if src else None,
        }
    lines = [f"# {title}", ""]
    lines += [f"command: {c}" for c in commands]
    lines += ["",
              f"calibration: {COPY_KERNEL} of {copy_mib} MiB; scale FETCH_SIZE x{factors['FETCH_SIZE']:.4f}, "
              f"WRITE_SIZE x{factors['WRITE_SIZE']:.4f} (known bytes / counter)", "",
              f"{'launches':>8} {'fetch_MB':>10} {'write_MB':>10}  kernel (per launch, calibrated)"]
    for n, t in sorted(table.items(), key=lambda kv: -(kv[1]["fetch_bytes"] + kv[1]["write_bytes"]) * kv[1]["launches"]):
        lines.append(f"{t['launches']:8d} {t['fetch_bytes'] / 1e6:10.2f} {t['write_bytes'] / 1e6:10.2f}  {n}")
    lines += ["", "traffic_json: " + json.dumps({"factors": factors, "kernels": table}, sort_keys=True)]
    return "\n".join(lines) + "\n"


def load(path: str) -> dict | None:
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json: "):
            return json.loads(line[len("traffic_json: "):])
    return None


def traffic_for(path: str, kernel: str) -> float | None:
    """Calibrated HBM bytes per launch of `kernel` (trace-name form) from the
    summary at `path`, or None when absent or taken from other source."""
    d = load(path)
    if d is None:
        return None
    t = d["kernels"].get(kernel)
    if t is None:
        # the trace may name a kernel by its base only
        hits = [v for k, v in d["kernels"].items() if base_name(k) == kernel]
        if len(hits) != 1:
            return None
        t = hits[0]
    src = kernel_source(base_name(kernel))
    if src is None or t.get("source_sha") != source_hash(src):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


# ---------------------------------------------------------------------------
# utilisation counters (MFMA, LDS, waits, L2) per kernel and launch shape
# ---------------------------------------------------------------------------

SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE comes summed over the 8 XCDs' instances


def _counter_rows(dirs):
    """{(kernel, grid size): {counter: [value per dispatch]}} and durations (ns)
    over every counter_collection.csv under `dirs` (one pass each)."""
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    meta = {}
    for d in dirs:
        with open(_find_csv(d)) as f:
            for r in csv.DictReader(f):
                key = (norm_name(r["Kernel_Name"]), int(r["Grid_Size"]))
                vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
                durs[key][(d, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                meta[key] = (int(r["VGPR_Count"]), int(r["Accum_VGPR_Count"]), int(r["LDS_Block_Size"]))
    return vals, durs, meta


def derived(c: dict, dur_ns: float) -> dict:
    """Ratios from one kernel's mean counter values per dispatch."""
    g = lambda n: c.get(n)  # noqa: E731
    out = {}
    if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None and g("GRBM_GUI_ACTIVE"):
        out["mfma_busy"] = g("SQ_VALU_MFMA_BUSY_CYCLES") / (g("GRBM_GUI_ACTIVE") / XCDS * SIMDS)
    if g("SQ_INSTS_VALU_MFMA_MOPS_BF16") is not None and dur_ns > 0:
        out["mfma_bf16_tflops"] = g("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / dur_ns / 1e3
    if g("SQ_WAVE_CYCLES"):
        for n, k in (("SQ_WAIT_INST_ANY", "wait_inst_frac"), ("SQ_WAIT_ANY", "wait_any_frac"),
                     ("SQ_ACTIVE_INST_ANY", "active_inst_frac"), ("SQ_ACTIVE_INST_VALU", "valu_frac"),
                     ("SQ_ACTIVE_INST_LDS", "lds_frac"), ("SQ_ACTIVE_INST_VMEM", "vmem_frac"),
                     ("SQ_WAIT_INST_LDS", "wait_lds_frac")):
            if g(n) is not None:
                out[k] = g(n) / g("SQ_WAVE_CYCLES")
    if g("SQ_LDS_BANK_CONFLICT") is not None and g("SQ_LDS_IDX_ACTIVE"):
        out["lds_bank_conflict_frac"] = g("SQ_LDS_BANK_CONFLICT") / g("SQ_LDS_IDX_ACTIVE")
    if g("SQ_LDS_IDX_ACTIVE") is not None and g("GRBM_GUI_ACTIVE"):
        out["lds_busy"] = g("SQ_LDS_IDX_ACTIVE") / (g("GRBM_GUI_ACTIVE") / XCDS * 256)
    h, m = g("TCC_HIT_sum"), g("TCC_MISS_sum")
    if h is not None and m is not None and h + m > 0:
        out["l2_hit"] = h / (h + m)
    return out


def summarize_counters(dirs, title: str, commands, min_us: float = 20.0) -> str:
    """Text summary: per (kernel, grid size) with a mean duration of at least
    min_us, the mean of every counter per dispatch and the derived ratios."""
    vals, durs, meta = _counter_rows(dirs)
    table = {}
    for key, cs in vals.items():
        dur = sum(durs[key].values()) / len(durs[key])
        if dur < min_us * 1e3:
            continue
        mean = {n: sum(v) / len(v) for n, v in cs.items()}
        name, grid = key
        src = kernel_source(base_name(name))
        table[f"{name} grid={grid}"] = {
            "launches": max(len(v) for v in cs.values()), "mean_us": dur / 1e3, "vgpr": meta[key][0],
            "agpr": meta[key][1], "lds_bytes": meta[key][2], "counters": mean, "derived": derived(mean, dur),
            "source": os.path.basename(src) if src else None, "source_sha": source_hash(src) if src else None}
    lines = [f"# {title}", ""]
    lines += [f"command: {c}" for c in commands]
    cols = ("mfma_busy", "mfma_bf16_tflops", "wait_inst_frac", "valu_frac", "lds_frac", "vmem_frac",
            "lds_bank_conflict_frac", "lds_busy", "l2_hit")
    lines += ["", "mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); mfma_bf16_tflops = "
              "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration; *_frac of SQ_WAVE_CYCLES; lds_bank_conflict_frac = "
              "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; lds_busy = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / 8 x 256 CUs); "
              "l2_hit = TCC_HIT / (TCC_HIT + TCC_MISS). Durations are from the counter runs (dispatches serialised).",
              "", f"{'launch':>6} {'us':>8} {'vgpr':>4} {'agpr':>4} " + " ".join(f"{c[:11]:>11}" for c in cols)
              + "  kernel"]
    for n, t in sorted(table.items(), key=lambda kv: -kv[1]["mean_us"] * kv[1]["launches"]):
        dv = t["derived"]
        cells = " ".join(f"{dv[c]:11.3f}" if c in dv else f"{'-':>11}" for c in cols)
        lines.append(f"{t['launches']:6d} {t['mean_us']:8.1f} {t['vgpr']:4d} {t['agpr']:4d} {cells}  {n}")
    return "\n".join(lines) + "\n"


# ---------------------------------------------------------------------------
# kernel + memory-copy timeline (rocprofv3 --kernel-trace --memory-copy-trace)
# ---------------------------------------------------------------------------

BLIT = "__amd_rocclr_copyBuffer"


def _union_ns(ivs):
    total, end = 0, None
    for a, b in sorted(ivs):
        if end is None or a > end:
            total += b - a
            end = b
        elif b > end:
            total += b - end
            end = b
    return total


def _overlap_ns(xs, ys):
    """Time covered by both interval sets."""
    def merged(v):
        out = []
        for a, b in sorted(v):
            if out and a <= out[-1][1]:
                out[-1][1] = max(out[-1][1], b)
            else:
                out.append([a, b])
        return out
    xs, ys = merged(xs), merged(ys)
    i = j = 0
    tot = 0
    while i < len(xs) and j < len(ys):
        a, b = max(xs[i][0], ys[j][0]), min(xs[i][1], ys[j][1])
        if a < b:
            tot += b - a
        if xs[i][1] < ys[j][1]:
            i += 1
        else:
            j += 1
    return tot


def summarize_copies(d: str, title: str, commands, window_ms: float) -> str:
    """Busy time of the compute kernels, the runtime's device-to-host blit
    kernels and the DMA copies per direction over the last `window_ms` of
    the trace (the timed steps), and how much of each overlaps the compute."""
    ks = list(csv.DictReader(open(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0])))
    ms = list(csv.DictReader(open(glob.glob(os.path.join(d, "**", "*memory_copy_trace.csv"), recursive=True)[0])))
    iv = lambda r: (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))  # noqa: E731
    end = max(iv(r)[1] for r in ks + ms)
    lo = end - int(window_ms * 1e6)
    inwin = lambda v: [x for x in v if x[0] >= lo]  # noqa: E731
    comp = inwin([iv(r) for r in ks if BLIT not in r["Kernel_Name"]])
    blit = inwin([iv(r) for r in ks if BLIT in r["Kernel_Name"]])
    up = inwin([iv(r) for r in ms if "HOST_TO_DEVICE" in r["Direction"]])
    dn = inwin([iv(r) for r in ms if "DEVICE_TO_HOST" in r["Direction"]])
    c_busy = _union_ns(comp)
    rows = [("compute kernels", comp), ("device-to-host blit kernels", blit), ("DMA copies host to device", up),
            ("DMA copies device to host", dn)]
    lines = [f"# {title}", ""] + [f"command: {c}" for c in commands]
    lines += ["", f"window: the last {window_ms:.0f} ms of the trace", "",
              f"{'count':>6} {'busy_ms':>9} {'mean_ms':>8} {'with_compute_ms':>15}  what"]
    for name, v in rows:
        if not v:
            lines.append(f"{0:6d} {0.0:9.2f} {0.0:8.3f} {0.0:15.2f}  {name}")
            continue
        busy = _union_ns(v)
        mean = sum(b - a for a, b in v) / len(v)
        ov = _overlap_ns(v, comp) if name != "compute kernels" else busy
        lines.append(f"{len(v):6d} {busy / 1e6:9.2f} {mean / 1e6:8.3f} {ov / 1e6:15.2f}  {name}")
    lines += ["", f"compute busy {c_busy / 1e6:.2f} ms of the {window_ms:.0f} ms window"]
    return "\n".join(lines) + "\n"


def summarize_kernels(d: str, title: str, commands, bench_line: str | None = None) -> str:
    """Text summary of a `rocprofv3 --kernel-trace --stats` run: per kernel
    (the library's name form) calls, total, average, minimum and maximum
    duration and share of kernel time; optionally the bench line's own
    figures for the dominant kernel (its event timing, measured in a run of
    its own) for comparison."""
    path = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not path:
        raise FileNotFoundError(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(path[0])))
    lines = [f"# {title}", ""] + [f"command: {c}" for c in commands] + [
        "", "calls  total_ms    avg_us    min_us    max_us   pct  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):5d} {int(r['TotalDurationNs']) / 1e6:9.2f} {float(r['AverageNs']) / 1e3:9.1f} "
                     f"{int(r['MinNs']) / 1e3:9.1f} {int(r['MaxNs']) / 1e3:9.1f} {float(r['Percentage']):5.1f}  "
                     f"{norm_name(r['Name'])}")
    if bench_line:
        b = json.loads(bench_line)
        rf = b["roofline"]
        lines += ["", f"bench line of the same build (its own run): the dominant kernel {rf['kernel']} averages "
                      f"{rf['avg_launch_ms']:.4f} ms per launch by the library's event timing, {rf['achieved']:.1f} "
                      f"{rf['unit']} = {rf['frac']:.3f} of the {rf['peak']:.0f} {rf['unit']} peak; step "
                      f"{b['ms_per_step']} ms, {b['value']} {b['unit']}."]
    return "\n".join(lines) + "\n"


def summarize_configs(bench_line: str, commands) -> tuple[str, str | None]:
    """Text summaries of a `bench.py --configs [--ablation] [--optimizer]`
    line: the per-configuration table (and the host optimizer and streamed
    figures the line carries), and the transfer-policy ablation table when
    the line has one (else None)."""
    d = json.loads(bench_line)
    cf = d["configs"]
    out = ["# Per-configuration throughput, weights resident (bench.py --configs)", ""] + [
        f"command: {c}" for c in commands] + [
        "", "Each configuration's own call sequence, wall time with the context synced, median of 3 after one warm-up;",
        "tokens/s = T / time; TFLOP/s counts matrix products only (causal attention on its causal pairs, active experts "
        "only,", "no weight-gradient products for the frozen LoRA base).", "",
        "config             call                                      ms     tokens/s  TFLOP/s"]
    notes = []
    for name, c in cf.items():
        for call, v in c.items():
            if not isinstance(v, dict):
                if call == "note":
                    notes.append(f"{name}: {v}")
                continue
            tf = v.get("tflops")
            out.append(f"{name:18s} {call:36s} {v['ms']:8.2f} {v['tokens_per_s']:12.0f} "
                       f"{tf if tf is not None else '-':>8}")
            if "note" in v:
                notes.append(f"{name} {call}: {v['note']}")
    out += [""] + notes
    for key, label in (("optimizer", "host optimizer step (bench.py --optimizer)"),
                       ("streamed", "streamed step, fp32 gradients"),
                       ("streamed_bf16_grads", "streamed step, bf16 gradients")):
        if key in d:
            out.append(f"{label}: " + json.dumps(d[key]))
    out += ["", "raw: " + json.dumps(cf)]
    ab = d.get("ablation")
    rows = None
    if ab:
        rows = ["# Transfer-policy ablation: Llama-3.1-8B-shaped layers on one MI355X", ""] + [
            f"command: {c}" for c in commands] + ["", "workload: " + ab["workload"],
            f"per stage: {ab['weights_GB_per_stage']} GB of bf16 weights up; per backward stage "
            f"{ab['grads_GB_per_bwd_stage']} GB of fp32 gradients down;",
            "activations and activation gradients go through pinned host memory between stages. Throughput = tokens "
            "of one pass / wall time of one pass (mean of 2 after 1 warm-up).", "",
            "| mbs | no_prefetch | prefetch | windowed | windowed / no_prefetch | windowed / prefetch |",
            "|---|---|---|---|---|---|"]
        for i, m in enumerate(ab["mbs"]):
            rows.append(f"| {m} | {ab['no_prefetch'][i]:.0f} | {ab['prefetch'][i]:.0f} | {ab['windowed'][i]:.0f} | "
                        f"{ab['windowed_over_no_prefetch'][i]:.3f} | {ab['windowed_over_prefetch'][i]:.3f} |")
    return "\n".join(out) + "\n", (None if rows is None else "\n".join(rows) + "\n")


if __name__ == "__main__":
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "configs":
        import argparse
        ap = argparse.ArgumentParser(description="summarise a bench.py --configs line")
        ap.add_argument("mode")
        ap.add_argument("bench_log")
        ap.add_argument("--command", action="append", default=[])
        ap.add_argument("--out", required=True)
        ap.add_argument("--ablation-out", default=None)
        a = ap.parse_args()
        line = [l for l in open(a.bench_log) if l.startswith("{")][-1]
        txt, abl = summarize_configs(line, a.command)
        with open(a.out, "w") as f:
            f.write(txt)
        if abl is not None and a.ablation_out:
            with open(a.ablation_out, "w") as f:
                f.write(abl)
        print(txt)
        sys.exit(0)
    if len(sys.argv) > 1 and sys.argv[1] == "kernels":
        import argparse
        ap = argparse.ArgumentParser(description="summarise a kernel trace")
        ap.add_argument("mode")
        ap.add_argument("dir")
        ap.add_argument("--title", required=True)
        ap.add_argument("--command", action="append", default=[])
        ap.add_argument("--bench-log", default=None, help="a bench.py output whose last JSON line to quote")
        ap.add_argument("--out", required=True)
        a = ap.parse_args()
        bl = None
        if a.bench_log:
            bl = [l for l in open(a.bench_log) if l.startswith("{")][-1]
        txt = summarize_kernels(a.dir, a.title, a.command, bl)
        with open(a.out, "w") as f:
            f.write(txt)
        print(txt)
        sys.exit(0)
    if len(sys.argv) > 1 and sys.argv[1] == "copies":
        import argparse
        ap = argparse.ArgumentParser(description="summarise a kernel + memory-copy trace")
        ap.add_argument("mode")
        ap.add_argument("dir")
        ap.add_argument("--title", required=True)
        ap.add_argument("--window-ms", type=float, required=True)
        ap.add_argument("--command", action="append", default=[])
        ap.add_argument("--note", action="append", default=[])
        ap.add_argument("--out", required=True)
        a = ap.parse_args()
        txt = summarize_copies(a.dir, a.title, a.command, a.window_ms)
        if a.note:
            txt += "\n" + "\n".join(a.note) + "\n"
        with open(a.out, "w") as f:
            f.write(txt)
        print(txt)
        sys.exit(0)
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        import argparse
        ap = argparse.ArgumentParser(description="summarise utilisation counter runs")
        ap.add_argument("mode")
        ap.add_argument("dirs", nargs="+")
        ap.add_argument("--title", required=True)
        ap.add_argument("--command", action="append", default=[])
        ap.add_argument("--out", required=True)
        a = ap.parse_args()
        txt = summarize_counters(a.dirs, a.title, a.command)
        with open(a.out, "w") as f:
            f.write(txt)
        print(txt)
        sys.exit(0)
    import argparse
    ap = argparse.ArgumentParser(description="summarise FETCH_SIZE / WRITE_SIZE counter runs")
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    txt = summarize(a.fetch_dir, a.write_dir, a.copy_mib, a.title, a.command)
    with open(a.out, "w") as f:
        f.write(txt)
    print(txt)
