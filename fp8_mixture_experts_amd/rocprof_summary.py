"""Turns rocprofv3 result databases into the short text summaries kept under
``profiles/``.

    python -m fp8_mixture_experts_amd.rocprof_summary trace DB OUT "COMMAND"
    python -m fp8_mixture_experts_amd.rocprof_summary traffic FETCH_DB WRITE_DB OUT WORKLOAD "COMMAND" COPY_BYTES
    python -m fp8_mixture_experts_amd.rocprof_summary mfma DB OUT WORKLOAD "COMMAND" FLOPS [CUS XCDS]

``trace`` reads a ``--kernel-trace --stats`` database and writes one line per
kernel (calls, average and total duration, launch shape, registers, LDS).

``mfma`` reads one ``--pmc --kernel-trace`` database of the matrix-core
counters (``SQ_INSTS_VALU_MFMA_MOPS_F16`` / ``_F8`` in units of 512 FLOPs,
``SQ_VALU_MFMA_BUSY_CYCLES``, ``GRBM_GUI_ACTIVE`` ...) and writes the expert
kernel's per-launch averages with what follows from them: FLOPs per matrix
type (checked against the algorithmic FLOPS), the shader clock (GUI-active
cycles per XCD over the traced duration), the matrix-core busy fraction of
the SIMD cycles, and the achieved rate against the FP8 peak.

``traffic`` reads two ``--pmc`` databases of the same bench command, one with
``FETCH_SIZE`` and one with ``WRITE_SIZE`` (KiB per dispatch), taken with
``bench.py --copy-probe-mib N`` so that each run also holds one plain device
copy of N MiB.  The copy calibrates the counters: a factor per counter equal to
the bytes the copy is known to read (or write) divided by what the counter
reported for it.  The expert kernel's calibrated bytes per launch are written
together with a SHA-256 of the library sources; ``bench.py`` reports them as
``roofline.traffic`` only while the sources still hash to that value.
"""

from __future__ import annotations

import glob
import hashlib
import os
import re
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
EXPERT_KERNEL = "moe_expert_ffn"
COPY_KERNELS = ("copyBuffer", "copy_kernel", "CopyKernel")


_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_text(src: str) -> str:
    """C/C++/HIP source without its comments, whitespace runs collapsed."""
    def keep(m):
        t = m.group(0)
        return " " if t.startswith("/") else t
    return " ".join(_TOKENS.sub(keep, src).split())


def sources_sha256() -> str:
    """Hash of the code (comments and layout ignored) of every library source
    and of the public header: a counter reading is stale once it changes."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, n) for n in sorted(os.listdir(CSRC))
             if n.endswith((".hip", ".cpp", ".h"))]
    files += [os.path.join(INCLUDE, n) for n in sorted(os.listdir(INCLUDE)) if n.endswith(".h")]
    for path in files:
        h.update(os.path.basename(path).encode())
        with open(path, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def _db(path):
    if os.path.isdir(path):
        hits = sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))
    else:
        hits = glob.glob(path)
    if not hits:
        raise SystemExit(f"no rocprofv3 database at {path}")
    return sqlite3.connect(hits[0])


def trace(db, out, command):
    con = _db(db)
    rows = list(con.execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels"))
    info = {r[0]: r[1:] for r in con.execute(
        "select name, grid_x, workgroup_x, vgpr_count, accum_vgpr_count, lds_size "
        "from kernels group by name")}
    lines = ["# rocprofv3 --kernel-trace --stats summary",
             f"# command: {command}",
             "# durations in microseconds (the top_kernels view of the database)",
             f"{'kernel':60s} {'calls':>5s} {'avg_us':>10s} {'total_us':>11s} {'pct':>6s}"
             "  grid wg vgpr agpr lds"]
    for name, calls, total, avg, pct in rows:
        g = info.get(name, ("", "", "", "", ""))
        lines.append(f"{name[:60]:60s} {calls:5d} {avg:10.2f} {total:11.1f} "
                     f"{pct:6.2f}  {g[0]} {g[1]} {g[2]} {g[3]} {g[4]}")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def _counter(con, counter):
    """Average value of one counter per kernel name, and the dispatch count."""
    res = {}
    for name, avg, n in con.execute(
            "select kernel_name, avg(value), count(distinct dispatch_id) from counters_collection "
            "where counter_name = ? group by kernel_name", (counter,)):
        res[name] = (float(avg), int(n))
    return res


def _copy_probe(con, counter):
    """The copy probe's reading: the largest single copy dispatch in the run."""
    best = None
    for name, value in con.execute(
            "select kernel_name, value from counters_collection where counter_name = ?",
            (counter,)):
        if any(k in name for k in COPY_KERNELS) and (best is None or value > best[1]):
            best = (name, float(value))
    if best is None:
        raise SystemExit(f"no copy kernel with {counter} in the run")
    return best


def _pick(res, keys, what):
    for name, v in res.items():
        if any(k in name for k in keys):
            return name, v
    raise SystemExit(f"no {what} kernel among {sorted(res)}")


def traffic(fetch_db, write_db, out, workload, command, copy_bytes):
    fcon, wcon = _db(fetch_db), _db(write_db)
    kname, (fetch_kib, nf) = _pick(_counter(fcon, "FETCH_SIZE"), (EXPERT_KERNEL,), "expert")
    _, (write_kib, nw) = _pick(_counter(wcon, "WRITE_SIZE"), (EXPERT_KERNEL,), "expert")
    cname, copy_fetch_kib = _copy_probe(fcon, "FETCH_SIZE")
    _, copy_write_kib = _copy_probe(wcon, "WRITE_SIZE")
    f_fetch = copy_bytes / (copy_fetch_kib * 1024.0)
    f_write = copy_bytes / (copy_write_kib * 1024.0)
    read_b = fetch_kib * 1024.0 * f_fetch
    write_b = write_kib * 1024.0 * f_write
    lines = [
        f"# HBM traffic of {kname} on the {workload} workload (rocprofv3 --pmc, two passes)",
        f"# command: {command}",
        f"# calibration kernel: {cname} copying {copy_bytes} bytes",
        f"copy_fetch_kib: {copy_fetch_kib:.1f}",
        f"copy_write_kib: {copy_write_kib:.1f}",
        f"fetch_factor: {f_fetch:.4f}",
        f"write_factor: {f_write:.4f}",
        f"expert_fetch_kib_per_launch: {fetch_kib:.1f}   (dispatches: {nf})",
        f"expert_write_kib_per_launch: {write_kib:.1f}   (dispatches: {nw})",
        f"read_bytes_per_launch: {read_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {read_b + write_b:.0f}",
        f"workload: {workload}",
        f"sources_sha256: {sources_sha256()}",
    ]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def _durations(con):
    """Mean traced duration (ns) per kernel name, if the run traced kernels."""
    for q in ('select name, avg("end" - start) from kernels group by name',
              "select name, avg(duration) from kernels group by name",
              "select name, average * 1000.0 from top_kernels"):
        try:
            return {n: float(d) for n, d in con.execute(q)}
        except sqlite3.Error:
            continue
    return {}


def mfma(db, out, workload, command, flops, cus=256, xcds=8):
    con = _db(db)
    counters = [r[0] for r in con.execute("select distinct counter_name from counters_collection")]
    vals = {}
    kname = None
    for c in sorted(counters):
        name, (v, n) = _pick(_counter(con, c), (EXPERT_KERNEL,), "expert")
        kname = name
        vals[c] = (v, n)
    dur = _durations(con)
    dur_ns = next((d for n, d in dur.items() if n == kname), None)
    lines = [f"# matrix-core counters of {kname} on the {workload} workload "
             "(rocprofv3 --pmc --kernel-trace, averages per launch)",
             f"# command: {command}"]
    for c in sorted(vals):
        lines.append(f"{c}: {vals[c][0]:.6g}   (dispatches: {vals[c][1]})")
    simds = 4 * cus
    mops16 = vals.get("SQ_INSTS_VALU_MFMA_MOPS_F16", (0.0, 0))[0]
    mops8 = vals.get("SQ_INSTS_VALU_MFMA_MOPS_F8", (0.0, 0))[0]
    mfma_flops = 512.0 * (mops16 + mops8)
    lines += [f"f16_mfma_flops: {512.0 * mops16:.6g}",
              f"f8_mfma_flops: {512.0 * mops8:.6g}",
              f"algorithmic_flops: {flops:.6g}",
              f"mfma_flops_over_algorithmic: {mfma_flops / flops:.4f}"]
    gui = vals.get("GRBM_GUI_ACTIVE", (0.0, 0))[0]
    busy = vals.get("SQ_VALU_MFMA_BUSY_CYCLES", (0.0, 0))[0]
    if gui:
        cycles = gui / xcds
        lines.append(f"kernel_cycles_per_xcd: {cycles:.6g}")
        if busy:
            lines.append(f"mfma_busy_fraction_of_simd_cycles: {busy / (simds * cycles):.4f}")
        if dur_ns:
            lines.append(f"traced_duration_us: {dur_ns / 1e3:.2f}")
            lines.append(f"shader_clock_ghz: {cycles / dur_ns:.3f}")
    if dur_ns:
        rate = flops / (dur_ns * 1e-9)
        lines += [f"achieved_tflops: {rate / 1e12:.1f}",
                  f"fraction_of_fp8_peak_5000_tflops: {rate / 5e15:.4f}",
                  f"fraction_of_exact_path_peak_3000_tflops: {rate / 3e15:.4f}"]
    lines += [f"workload: {workload}", f"sources_sha256: {sources_sha256()}"]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def read_traffic(path, workload):
    """Calibrated traffic per launch from a summary, or None when it is stale."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.split()[0] if v.split() else ""
    if kv.get("workload") != workload or kv.get("sources_sha256") != sources_sha256():
        return None
    return float(kv["traffic_bytes_per_launch"])


def main(argv):
    if len(argv) >= 4 and argv[0] == "trace":
        print(trace(argv[1], argv[2], argv[3]), end="")
    elif len(argv) >= 6 and argv[0] == "mfma":
        extra = [int(v) for v in argv[6:8]]
        print(mfma(argv[1], argv[2], argv[3], argv[4], float(argv[5]), *extra), end="")
    elif len(argv) >= 7 and argv[0] == "traffic":
        print(traffic(argv[1], argv[2], argv[3], argv[4], argv[5], int(argv[6])), end="")
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
