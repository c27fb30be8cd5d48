"""Summaries of rocprofv3 output (rocpd SQLite databases) for the profiles/ folder.

  python -m activation_residual_compression_amd.profsummary trace <trace_results.db> [--md OUT] [--json OUT]
      per-kernel dispatch count and duration (avg/min/max, microseconds)

  python -m activation_residual_compression_amd.profsummary pmc <fetch.db> <write.db> [--md OUT] [--json OUT]
      per-kernel HBM bytes per dispatch from a FETCH_SIZE run and a WRITE_SIZE run,
      each scaled by the factor that makes the same counter read the true size of a
      plain 1 GiB -> 1 GiB device copy (__amd_rocclr_copyBuffer) captured in the run.
      The JSON records the sha256 of the kernel sources, so a later reader can tell
      whether the kernels changed since the counters were taken.

  python -m activation_residual_compression_amd.profsummary mfma <pmc.db> [--trace trace.json] [--md OUT] [--json OUT]
      per-kernel MFMA work from one run with SQ_INSTS_VALU_MFMA_MOPS_BF16,
      SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: bf16 MFMA flops per dispatch
      (MOPS x 512), MFMA busy share of the SIMD cycles (busy / (GUI_ACTIVE x SIMDs)),
      and, with a kernel-trace summary, achieved TFLOP/s against the dense bf16 peak.

--title and --command (repeatable) put a heading and the commands that made the
databases at the top of the Markdown summary.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
COPY_BYTES_KB = 1 << 20  # 1 GiB copy: 1 GiB read and 1 GiB written
SIMDS = 256 * 4           # MI355X: 256 CUs x 4 SIMDs
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def short_name(name: str) -> str:
    n = name
    if n.startswith("void "):
        n = n[5:]
    n = n.replace("(anonymous namespace)::", "").replace("rc::", "")
    return n.split("(")[0]


def source_hashes() -> dict:
    out = {}
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            out[f] = hashlib.sha256(open(os.path.join(CSRC, f), "rb").read()).hexdigest()
    return out


def trace_table(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    return [(short_name(r[0]), r[1], r[2] / 1e3, r[3] / 1e3, r[4] / 1e3) for r in rows]


def pmc_values(db: str, counter: str, reduce=sum):
    """Per kernel name, one value per dispatch: the counter's instances (per
    shader engine, per XCD, ...) combined with `reduce` (sum for event counts,
    max for GRBM_GUI_ACTIVE, as rocprofv3's own derived metrics do)."""
    con = sqlite3.connect(db)
    per = collections.defaultdict(list)
    names = {}
    for did, name, val in con.execute("select dispatch_id, name, counter_value from pmc_events "
                                      "where counter_name=?", (counter,)):
        per[did].append(float(val))
        names[did] = short_name(name)
    d = collections.defaultdict(list)
    for did in sorted(per):
        d[names[did]].append(reduce(per[did]))
    return d


def calibration(vals) -> float:
    """Factor = true KB / counter KB for the 1 GiB copies in the run: the largest
    __amd_rocclr_copyBuffer dispatches (other copies in the run are smaller)."""
    copies = vals.get("__amd_rocclr_copyBuffer", [])
    if not copies:
        raise SystemExit("no __amd_rocclr_copyBuffer dispatch in the run (bench.py --copy-calibration)")
    top = max(copies)
    cands = sorted(v for v in copies if v > 0.9 * top)
    return COPY_BYTES_KB / cands[len(cands) // 2]


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--md")
    t.add_argument("--json")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_db")
    p.add_argument("write_db")
    p.add_argument("--md")
    p.add_argument("--json")
    mf = sub.add_parser("mfma")
    mf.add_argument("db")
    mf.add_argument("--trace")
    mf.add_argument("--md")
    mf.add_argument("--json")
    for q in (t, p, mf):
        q.add_argument("--title")
        q.add_argument("--command", action="append", default=[])
    args = ap.parse_args(argv)
    head = []
    if args.title:
        head += ["# " + args.title, ""]
    if args.command:
        head += ["Made by:", "", "```"] + args.command + ["```", ""]

    if args.mode == "trace":
        rows = trace_table(args.db)
        if args.json:
            json.dump(dict(kernels={r[0]: dict(dispatches=r[1], avg_us=r[2], min_us=r[3], max_us=r[4])
                                    for r in rows}, sources=source_hashes()),
                      open(args.json, "w"), indent=1, sort_keys=True)
        lines = ["| kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
        lines += ["| `%s` | %d | %.1f | %.1f | %.1f |" % r for r in rows]
        text = "\n".join(lines)
    elif args.mode == "mfma":
        mops = pmc_values(args.db, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        busy = pmc_values(args.db, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = pmc_values(args.db, "GRBM_GUI_ACTIVE", reduce=max)
        dur = json.load(open(args.trace))["kernels"] if args.trace else {}
        avg = lambda v: sum(v) / len(v) if v else 0.0
        kern = {}
        for k in sorted(mops):
            if avg(mops[k]) <= 0:
                continue
            fl = avg(mops[k]) * 512
            ent = dict(dispatches=len(mops[k]), bf16_flops=fl,
                       mfma_busy_frac=avg(busy.get(k, [])) / (avg(gui.get(k, [])) * SIMDS)
                       if gui.get(k) else None)
            if k in dur:
                ent["avg_us"] = dur[k]["avg_us"]
                ent["tflops"] = fl / (dur[k]["avg_us"] * 1e-6) / 1e12
                ent["frac_of_bf16_peak"] = ent["tflops"] / BF16_PEAK_TFLOPS
            kern[k] = ent
        if args.json:
            json.dump(dict(kernels=kern, sources=source_hashes(), simds=SIMDS,
                           bf16_peak_tflops=BF16_PEAK_TFLOPS), open(args.json, "w"), indent=1,
                      sort_keys=True)
        lines = ["| kernel | dispatches | bf16 MFMA GFLOP/dispatch | MFMA busy / SIMD cycles | avg us | TFLOP/s | of 2.5 PFLOP/s |",
                 "|---|---|---|---|---|---|---|"]
        for k, v in sorted(kern.items(), key=lambda kv: -kv[1]["bf16_flops"]):
            lines.append("| `%s` | %d | %.2f | %s | %s | %s | %s |" % (
                k, v["dispatches"], v["bf16_flops"] / 1e9,
                "%.1f %%" % (100 * v["mfma_busy_frac"]) if v["mfma_busy_frac"] is not None else "-",
                "%.1f" % v["avg_us"] if "avg_us" in v else "-",
                "%.1f" % v["tflops"] if "tflops" in v else "-",
                "%.2f %%" % (100 * v["frac_of_bf16_peak"]) if "tflops" in v else "-"))
        text = "\n".join(lines)
    else:
        F, W = pmc_values(args.fetch_db, "FETCH_SIZE"), pmc_values(args.write_db, "WRITE_SIZE")
        ff, fw = calibration(F), calibration(W)
        kern = {}
        for k in sorted(set(F) | set(W)):
            fv, wv = F.get(k, []), W.get(k, [])
            fk = sum(fv) / len(fv) if fv else 0.0
            wk = sum(wv) / len(wv) if wv else 0.0
            kern[k] = dict(dispatches=len(fv), fetch_kb=fk, write_kb=wk,
                           bytes=fk * ff * 1024 + wk * fw * 1024)
        out = dict(calibration=dict(fetch_factor=ff, write_factor=fw,
                                    reference="__amd_rocclr_copyBuffer, 1 GiB -> 1 GiB"),
                   kernels=kern, sources=source_hashes())
        if args.json:
            json.dump(out, open(args.json, "w"), indent=1, sort_keys=True)
        lines = ["calibration: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f (1 GiB device copy)" % (ff, fw), "",
                 "| kernel | dispatches | FETCH_SIZE KB | WRITE_SIZE KB | calibrated MB/dispatch |",
                 "|---|---|---|---|---|"]
        for k, v in sorted(kern.items(), key=lambda kv: -kv[1]["bytes"]):
            lines.append("| `%s` | %d | %.0f | %.0f | %.1f |" % (k, v["dispatches"], v["fetch_kb"],
                                                              v["write_kb"], v["bytes"] / 2 ** 20))
        text = "\n".join(lines)
    text = "\n".join(head) + ("\n" if head else "") + text
    if args.md:
        open(args.md, "w").write(text + "\n")
    print(text)


if __name__ == "__main__":
    main()
