"""Summaries of rocprofv3 runs of the scan, for the roofline figures.

bench.py reads the records this module writes (profiles/*.json) and uses them
only when they were taken on the current kernel sources (kernel_source_hash).

    python -m chunked_linear_attention_packed_amd.profile_summary \\
        --workload W --form one --kernel piece_kernel \\
        --trace DIR [--sq DIR ...] [--fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --copy-mib 256] \\
        --trace-cmd "..." --pmc-cmd "..." --copy-cmd "..." --sq-cmd "..."

Inputs are rocprofv3 output directories (-d DIR -o run, csv): a kernel trace
of one bench.py run, counter collections of the pass's kernels (one counter
set per run), and FETCH_SIZE / WRITE_SIZE of a plain device copy of known
size (bench.py --calibrate-copy-mib), which gives the scale from the
counters' KiB to bytes.  Outputs: profiles/<kernel>_<form>_<workload>.md (the
commands and the figures) and the records traffic_pass_<form>_<workload>.json
and counters_pass_<form>_<workload>.json.
"""
import argparse
import csv
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_linear_attention_packed_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """sha256 over every kernel source and header of the library, in name
    order (None without the sources)."""
    if not os.path.isdir(CSRC):
        return None
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def profile_record(kind, workload, form, src_hash):
    """profiles/<kind>_pass_<form>_<workload>.json if it was taken on the
    sources with hash src_hash, else None."""
    path = os.path.join(PROFILES, f"{kind}_pass_{form}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if src_hash and rec.get("source_sha256") == src_hash else None


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name):
    return name.split("<")[0].split("(")[0].replace("void ", "").strip()


def _bench_line(log):
    with open(log) as f:
        for line in f:
            if line.startswith('{"metric"'):
                return json.loads(line)
    return None


def _agent(d):
    for r in _rows(os.path.join(d, "run_agent_info.csv")):
        if r.get("Agent_Type") == "GPU" and int(r.get("Simd_Count", 0)) > 0:
            return {"cus": int(r["Cu_Count"]), "simds": int(r["Simd_Count"]),
                    "clock_mhz": float(r["Max_Engine_Clk_Fcompute"])}
    return None


def _counter_medians(d, kernel):
    per = {}
    for r in _rows(os.path.join(d, "run_counter_collection.csv")):
        if _short(r["Kernel_Name"]) != kernel:
            continue
        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in per.items()}


def _copy_reading(d, counter):
    """The copy launches' reading (median over the large dispatches; the
    run's small fills share the kernel name)."""
    vals = [float(r["Counter_Value"]) for r in _rows(os.path.join(d, "run_counter_collection.csv"))
            if r["Counter_Name"] == counter and "elementwise" in r["Kernel_Name"]]
    big = [x for x in vals if x >= 0.5 * max(vals)]
    return statistics.median(big)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--form", required=True)
    ap.add_argument("--kernel", required=True, help="kernel name(s) of the pass, comma separated")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--trace-log", default=None)
    ap.add_argument("--trace-cmd", default="")
    ap.add_argument("--sq", nargs="*", default=[])
    ap.add_argument("--sq-cmd", nargs="*", default=[])
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--pmc-cmd", default="")
    ap.add_argument("--copy-cmd", default="")
    a = ap.parse_args(argv)

    kernels = a.kernel.split(",")
    sha = kernel_source_hash()
    trace = _rows(os.path.join(a.trace, "run_kernel_trace.csv"))
    dur = {}
    for r in trace:
        dur.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    bench = _bench_line(a.trace_log or a.trace.rstrip("/") + ".log")
    pass_kernel_us = sum(statistics.mean(dur[k]) for k in kernels if k in dur)

    md = [f"# rocprofv3: {', '.join(kernels)}, {a.form}-launch form, {a.workload}\n",
          "Kernel trace (run from the repository root on one MI355X):",
          f"    {a.trace_cmd}\n", f"Kernel sources sha256 (csrc/*.hip, *.h): {sha}\n",
          "| kernel | dispatches | mean us | median us | min us | max us |",
          "|---|---|---|---|---|---|"]
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        md.append(f"| {k} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                  f"{min(v):.2f} | {max(v):.2f} |")
    md.append("")
    if bench:
        c = bench["config"]
        md.append(f"bench.py in the same run: {c['gpu_us_per_pass']:.2f} us per pass (HIP events "
                  f"over {bench['steps']} graph-replayed passes, rotating inputs), value "
                  f"{bench['value']:.4g} tokens/s, launches per pass {c['launches']}.  The pass's "
                  f"kernels average {pass_kernel_us:.2f} us per dispatch in the trace (all the "
                  f"run's dispatches: warm-up, cold and warm replays).\n")

    sq_rec = None
    if a.sq:
        agent = _agent(a.sq[0])
        med = {}
        for d in a.sq:
            for k in kernels:
                for name, val in _counter_medians(d, k).items():
                    med[name] = med.get(name, 0.0) + val
        md.append("## SQ counters (rocprofv3 --pmc, one counter set per run)\n")
        md.append("Commands:")
        for cmd in a.sq_cmd:
            md.append(f"    {cmd}")
        md.append("")
        md.append("| counter | median per pass |")
        md.append("|---|---|")
        for name in sorted(med):
            md.append(f"| {name} | {med[name]:.4g} |")
        busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES")
        frac = None
        if busy is not None and agent:
            cycles = pass_kernel_us * 1e-6 * agent["clock_mhz"] * 1e6
            frac = busy / (agent["simds"] * cycles)
            md.append("")
            md.append(f"MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x kernel cycles) = "
                      f"{busy:.4g} / ({agent['simds']} x {cycles:.4g}) = {frac:.3f} (kernel cycles: "
                      f"{pass_kernel_us:.2f} us at {agent['clock_mhz']:.0f} MHz; the counter adds "
                      f"16 cycles per 16x16x32 bf16 MFMA).")
        md.append("")
        sq_rec = {"workload": a.workload, "form": a.form, "kernels": kernels, "source_sha256": sha,
                  "medians": med, "mfma_busy_frac": frac, "kernel_us": pass_kernel_us,
                  "agent": agent, "source": f"profiles/{'_'.join(kernels)}_{a.form}_{a.workload}.md"}

    tr_rec = None
    if a.fetch and a.write and a.copy_fetch and a.copy_write:
        fe = sum(_counter_medians(a.fetch, k).get("FETCH_SIZE", 0.0) for k in kernels)
        wr = sum(_counter_medians(a.write, k).get("WRITE_SIZE", 0.0) for k in kernels)
        cf, cw = _copy_reading(a.copy_fetch, "FETCH_SIZE"), _copy_reading(a.copy_write, "WRITE_SIZE")
        fscale, wscale = a.copy_mib * 1024 / cf, a.copy_mib * 1024 / cw
        rb, wb = fe * fscale * 1024, wr * wscale * 1024
        alg = bench["roofline"]["bytes_per_pass"] if bench else None
        md.append("## HBM traffic per pass (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)\n")
        md.append("Commands:")
        md.append(f"    {a.pmc_cmd}")
        md.append("    (the same with --pmc WRITE_SIZE)")
        md.append(f"    {a.copy_cmd}")
        md.append("    (the same with --pmc WRITE_SIZE)\n")
        md.append(f"Calibration: a device copy reading and writing {a.copy_mib} MiB reads "
                  f"FETCH_SIZE = {cf:.0f} KiB and WRITE_SIZE = {cw:.0f} KiB per dispatch, so bytes "
                  f"= FETCH_SIZE x {fscale:.3f} KiB and WRITE_SIZE x {wscale:.3f} KiB.\n")
        md.append(f"Pass (medians per dispatch, summed over its kernels): FETCH_SIZE {fe:.0f} KiB, "
                  f"WRITE_SIZE {wr:.0f} KiB -> read {rb / 1e6:.2f} MB, written {wb / 1e6:.2f} MB, "
                  f"total {(rb + wb) / 1e6:.2f} MB"
                  + (f" against {alg / 1e6:.2f} MB algorithmic ({(rb + wb) / alg:.3f}x)."
                     if alg else "."))
        md.append("")
        tr_rec = {"workload": a.workload, "form": a.form, "kernels": kernels, "source_sha256": sha,
                  "bytes_per_pass": rb + wb, "read_bytes": rb, "write_bytes": wb,
                  "fetch_scale": fscale, "write_scale": wscale, "algorithmic_bytes": alg,
                  "source": f"profiles/{'_'.join(kernels)}_{a.form}_{a.workload}.md"}

    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{'_'.join(kernels)}_{a.form}_{a.workload}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    for kind, rec in (("traffic", tr_rec), ("counters", sq_rec)):
        if rec:
            with open(os.path.join(PROFILES, f"{kind}_pass_{a.form}_{a.workload}.json"), "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
    print("\n".join(md))


if __name__ == "__main__":
    main()
