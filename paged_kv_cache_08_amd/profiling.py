"""Summaries of rocprofv3 results for this library's kernels.

    python -m paged_kv_cache_08_amd.profiling stats DB...
        per-kernel dispatch count and duration (avg/min/max, us) from
        rocprofv3 --kernel-trace result databases, as a markdown table.

    python -m paged_kv_cache_08_amd.profiling traffic --fetch-db DB --write-db DB \\
            --kernel NAME --calib-bytes N --key KEY --out profiles/traffic.json
        HBM bytes per dispatch of kernel NAME from one --pmc FETCH_SIZE run and
        one --pmc WRITE_SIZE run. Each counter is scaled by what it reads for a
        plain copy of known size in the same run (the largest
        __amd_rocclr_copyBuffer dispatch, which copies N bytes). The record is
        stored under KEY with the hash of the kernel sources it was taken on.

    python -m paged_kv_cache_08_amd.profiling trace --kernel NAME --key KEY --out profiles/kernel_trace.json DB...
        The average, min and max duration of kernel NAME (and of the merge
        kernel, if it ran) in one --kernel-trace run, stored under KEY with
        the hash of the kernel sources it was taken on (bench.py reports it
        next to its event-timed figure while the sources still match).

    python -m paged_kv_cache_08_amd.profiling counters --kernel NAME DB...
        Shader counters of kernel NAME from one or more --pmc runs (each with
        GRBM_GUI_ACTIVE), averaged over dispatches, and the busy / utilisation
        figures rocprofv3 derives from them (same expressions: SQ counters
        summed over their instances, GRBM_GUI_ACTIVE the maximum over its
        instances; 256 CUs, 1024 SIMDs, 32 wave slots per CU on MI355X).
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    """sha256 over the HIP sources (file names and contents, sorted)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _db(path: str) -> sqlite3.Connection:
    cand = glob.glob(path) or glob.glob(os.path.join(path, "*.db"))
    if not cand:
        raise FileNotFoundError(path)
    return sqlite3.connect(cand[0])


def kernel_durations(path: str) -> dict:
    """{kernel name: [duration_us, ...]} from a kernel-trace database."""
    con = _db(path)
    out = collections.defaultdict(list)
    for name, dur in con.execute("select name, duration from kernels"):
        out[name].append(dur / 1e3)
    return out


def pmc_per_dispatch(path: str, counter: str) -> dict:
    """{kernel name: [per-dispatch value summed over instances, ...]} for one counter."""
    con = _db(path)
    per = collections.defaultdict(float)
    name = {}
    for did, nm, cn, cv in con.execute("select dispatch_id, name, counter_name, counter_value from pmc_events"):
        if cn != counter:
            continue
        per[did] += cv or 0.0
        name[did] = nm
    out = collections.defaultdict(list)
    for did, v in per.items():
        out[name[did]].append(v)
    return out


CU_NUM = 256       # MI355X compute units
SIMD_NUM = 1024    # 4 SIMDs per CU
WAVE_SLOTS = 32    # wave slots per CU in rocprofv3's occupancy expression


def pmc_dispatch_values(path: str, kernel: str) -> dict:
    """{counter: [per-dispatch value, ...]} for dispatches of kernels whose
    name contains `kernel`: SQ_* and other block counters summed over their
    instances, GRBM_GUI_ACTIVE the maximum over its instances."""
    con = _db(path)
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for did, nm, cn, cv in con.execute("select dispatch_id, name, counter_name, counter_value from pmc_events"):
        if kernel in nm:
            per[cn][did].append(cv or 0.0)
    out = {}
    for cn, d in per.items():
        red = max if cn == "GRBM_GUI_ACTIVE" else sum
        out[cn] = [red(v) for v in d.values()]
    return out


def counter_summary(paths, kernel: str) -> dict:
    """Mean per-dispatch counters over the given runs, and the derived figures."""
    vals = {}
    grbm = []
    for p in paths:
        d = pmc_dispatch_values(p, kernel)
        for cn, v in d.items():
            if cn == "GRBM_GUI_ACTIVE":
                grbm.extend(v)
            else:
                vals[cn] = sum(v) / len(v)
    if not grbm:
        raise KeyError(f"no GRBM_GUI_ACTIVE for {kernel}")
    g = sum(grbm) / len(grbm)
    der = {}

    def have(*cs):
        return all(c in vals for c in cs)

    if have("SQ_VALU_MFMA_BUSY_CYCLES"):
        der["MfmaUtil %"] = 100.0 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMD_NUM)
    if have("SQ_ACTIVE_INST_VALU"):
        der["VALUBusy %"] = 100.0 * vals["SQ_ACTIVE_INST_VALU"] / CU_NUM / g
    if have("SQ_LDS_IDX_ACTIVE"):
        der["LdsUtil %"] = 100.0 * vals["SQ_LDS_IDX_ACTIVE"] / (g * CU_NUM)
    if have("SQ_LDS_BANK_CONFLICT"):
        der["LDSBankConflict %"] = 100.0 * vals["SQ_LDS_BANK_CONFLICT"] / g / CU_NUM
    if have("SQ_WAVE_CYCLES"):
        der["OccupancyPercent %"] = 400.0 * vals["SQ_WAVE_CYCLES"] / g / CU_NUM / WAVE_SLOTS
    if have("SQ_BUSY_CU_CYCLES"):
        der["CU busy %"] = 100.0 * vals["SQ_BUSY_CU_CYCLES"] / (g * CU_NUM)
    if have("SQ_WAVES", "SQ_INSTS_VALU"):
        der["VALU instructions per wave"] = vals["SQ_INSTS_VALU"] / vals["SQ_WAVES"]
    if have("SQ_WAVES", "SQ_INSTS_MFMA"):
        der["MFMA instructions per wave"] = vals["SQ_INSTS_MFMA"] / vals["SQ_WAVES"]
    if have("SQ_WAVES", "SQ_INSTS_LDS"):
        der["LDS instructions per wave"] = vals["SQ_INSTS_LDS"] / vals["SQ_WAVES"]
    return {"kernel": kernel, "dispatches": len(grbm), "GRBM_GUI_ACTIVE": g, "counters": vals, "derived": der}


def counter_table(summary: dict) -> str:
    rows = [f"Kernel `{summary['kernel']}`, {summary['dispatches']} dispatches; GRBM_GUI_ACTIVE "
            f"{summary['GRBM_GUI_ACTIVE']:.0f} cycles per dispatch.", "",
            "| counter (sum over instances, mean per dispatch) | value |", "|---|---:|"]
    for cn, v in sorted(summary["counters"].items()):
        rows.append(f"| {cn} | {v:.0f} |")
    rows += ["", "| derived (rocprofv3 expressions) | value |", "|---|---:|"]
    for cn, v in summary["derived"].items():
        rows.append(f"| {cn} | {v:.1f} |")
    return "\n".join(rows)


def short(name: str) -> str:
    n = name.replace("pkv::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0]


def stats_table(paths) -> str:
    rows = ["| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for p in paths:
        for name, d in sorted(kernel_durations(p).items(), key=lambda kv: -sum(kv[1])):
            rows.append(f"| `{short(name)}` | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    return "\n".join(rows)


def trace_record(paths, kernel: str) -> dict:
    """Duration statistics of `kernel` (and of the LSE merge) over kernel-trace runs."""
    durs = collections.defaultdict(list)
    for p in paths:
        for name, d in kernel_durations(p).items():
            durs[name].extend(d)

    def pick(sub):
        ks = [k for k in durs if sub in k]
        if not ks:
            return None
        d = [x for k in ks for x in durs[k]]
        return d

    d = pick(kernel)
    if d is None:
        raise KeyError(f"no dispatches of {kernel}")
    rec = {"kernel": kernel, "calls": len(d), "kernel_us_avg": round(sum(d) / len(d), 2),
           "kernel_us_min": round(min(d), 2), "kernel_us_max": round(max(d), 2),
           "kernel_src_sha256": kernel_source_hash()}
    m = pick("lse_merge")
    if m:
        rec["merge_us_avg"] = round(sum(m) / len(m), 2)
    return rec


def _store(out: str, key: str, rec: dict) -> None:
    data = {}
    if os.path.exists(out):
        with open(out) as fh:
            data = json.load(fh)
    data[key] = rec
    with open(out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)


def traffic(fetch_db: str, write_db: str, kernel: str, calib_bytes: int) -> dict:
    f = pmc_per_dispatch(fetch_db, "FETCH_SIZE")
    w = pmc_per_dispatch(write_db, "WRITE_SIZE")

    def pick(d, what):
        ks = [k for k in d if kernel in k]
        if not ks:
            raise KeyError(f"no {what} dispatches of {kernel}")
        vals = d[ks[0]]
        cal = max(d.get(next(k for k in d if "copyBuffer" in k), [0.0]))
        return sum(vals) / len(vals), cal

    fk, fcal = pick(f, "FETCH_SIZE")
    wk, wcal = pick(w, "WRITE_SIZE")
    f_scale = calib_bytes / (fcal * 1024.0)
    w_scale = calib_bytes / (wcal * 1024.0)
    read_b = fk * 1024.0 * f_scale
    write_b = wk * 1024.0 * w_scale
    return {
        "kernel": kernel,
        "fetch_kib_raw": round(fk, 1),
        "write_kib_raw": round(wk, 1),
        "calib_copy_bytes": calib_bytes,
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "read_bytes_per_launch": int(read_b),
        "write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(read_b + write_b),
        "kernel_src_sha256": kernel_source_hash(),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-db", required=True)
    t.add_argument("--write-db", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--key", required=True)
    t.add_argument("--out", required=True)
    r = sub.add_parser("trace")
    r.add_argument("--kernel", required=True)
    r.add_argument("--key", required=True)
    r.add_argument("--out", required=True)
    r.add_argument("db", nargs="+")
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True)
    c.add_argument("db", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.db))
        return 0
    if a.cmd == "trace":
        paths = [p for pat in a.db for p in (glob.glob(pat) or [pat])]
        rec = trace_record(paths, a.kernel)
        _store(a.out, a.key, rec)
        print(json.dumps(rec, indent=1))
        return 0
    if a.cmd == "counters":
        paths = [p for pat in a.db for p in (glob.glob(pat) or [pat])]
        print(counter_table(counter_summary(paths, a.kernel)))
        return 0
    rec = traffic(a.fetch_db, a.write_db, a.kernel, a.calib_bytes)
    _store(a.out, a.key, rec)
    print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
