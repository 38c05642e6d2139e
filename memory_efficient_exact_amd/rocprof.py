"""Reduce rocprofv3 output to per-kernel figures: duration, MFMA utilisation,
VALU and LDS activity, and calibrated HBM traffic (bytes and GB/s).

This is the measurement side of the library, pure Python over the CSV files
that ``rocprofv3 --output-format csv`` writes; it runs no GPU code. The
profiling passes it expects are listed in PASSES; ``plan()`` prints the
rocprofv3 commands that produce them (one counter set per run, each under its
own time limit), ``collect()`` reduces their CSV files per kernel and
``render()`` writes the markdown summary kept under ``profiles/``, ending in a
JSON block that ``bench.py`` reads back (``current_figures``).

Derived figures (MI355X: 8 XCDs, 256 CUs, 1024 SIMDs):
  cycles per XCD = GRBM_GUI_ACTIVE / 8
  MFMA busy      = SQ_VALU_MFMA_BUSY_CYCLES / (1024 * cycles per XCD)
  co-issue       = SQ_VALU_MFMA_COEXEC_CYCLES / (1024 * cycles per XCD)
  VALU share     = SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (share of wave time)
  waiting        = SQ_WAIT_ANY / SQ_WAVE_CYCLES; waiting to issue = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES
  HBM bytes      = FETCH_SIZE * f_read + WRITE_SIZE * f_write, where each factor
                   is the copy kernel's true bytes over its reading of the same
                   counter (a plain device copy of known size in the same run)
  HBM GB/s       = HBM bytes per launch / average launch duration (kernel trace)
"""

import csv
import glob
import hashlib
import json
import os
import re
import statistics

XCDS = 8
SIMDS = 1024
CUS = 256

# one rocprofv3 run per pass: the hardware collects these counter sets together
PASSES = {
    "pmcA": ["SQ_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
             "SQ_ACTIVE_INST_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32",
             "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    "pmcB": ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS",
             "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CYCLES"],
    "pmcF": ["FETCH_SIZE"],
    "pmcW": ["WRITE_SIZE"],
}
COPY_KERNEL = "copyBuffer"  # the runtime's device-to-device copy kernel
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


# ------------------------------------------------------------ reading

def _read(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    """Value of the first of `names` present in `row` (rocprofv3 versions name some
    columns differently)."""
    for n in names:
        if n in row:
            return row[n]
    lower = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in lower:
            return lower[n.lower()]
    raise KeyError(names)


def _files(root, suffix):
    return sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True))


_TYPE_CODES = {"f": "float", "d": "double", "i": "int", "b": "bool", "DF16b": "__bf16"}


def _demangle(sym):
    """Name and template arguments of a mangled kernel symbol of this library, e.g.
    `_ZN3mea12_GLOBAL__N_115bwd_rows_kernelILi64EEEv...` -> `bwd_rows_kernel<64>`
    (the profiler leaves some names mangled, and the system demanglers do not read
    the bf16 type code); other symbols are returned unchanged."""
    pos, name = 2, None
    if sym.startswith("_ZN"):
        pos = 3
        while pos < len(sym) and sym[pos].isdigit():  # nested names: <len><id>...
            j = pos
            while sym[j].isdigit():
                j += 1
            ln = int(sym[pos:j])
            name = sym[j:j + ln]
            pos = j + ln
    if name is None:
        return sym
    args = []
    if pos < len(sym) and sym[pos] == "I":
        pos += 1
        while pos < len(sym) and sym[pos] != "E":
            if sym[pos] == "L":  # literal: L<type><value>E
                j = sym.index("E", pos)
                lit = sym[pos + 1:j]
                if lit.startswith("b"):
                    args.append("true" if lit[1:] == "1" else "false")
                else:
                    args.append(re.sub(r"^[a-z]", "", lit).replace("n", "-"))
                pos = j + 1
            else:
                for code, tname in sorted(_TYPE_CODES.items(), key=lambda kv: -len(kv[0])):
                    if sym.startswith(code, pos):
                        args.append(tname)
                        pos += len(code)
                        break
                else:
                    return sym
    return name + (f"<{', '.join(args)}>" if args else "")


def short_name(kernel):
    """`void mea::(anonymous namespace)::bwd_main_kernel<64, 8>(mea::...)` -> `bwd_main_kernel<64, 8>`."""
    k = kernel.strip()
    if k.startswith("_Z"):
        return _demangle(k)
    if k.startswith("void "):
        k = k[5:]
    depth, cut = 0, len(k)
    for i, ch in enumerate(k):  # drop the argument list (the first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not k[i:].startswith("(anonymous namespace)"):
            cut = i
            break
    k = k[:cut]
    k = k.replace("(anonymous namespace)::", "")
    k = re.sub(r"^(\w+::)+", "", k)
    return k.strip()


def kernel_trace(root):
    """{kernel: [(duration ns, grid work-items), ...] per dispatch, in dispatch order}
    from *_kernel_trace.csv."""
    out = {}
    for path in _files(root, "_kernel_trace.csv"):
        rows = _read(path)
        rows.sort(key=lambda r: int(_col(r, "Dispatch_Id", "Correlation_Id")))
        for r in rows:
            name = short_name(_col(r, "Kernel_Name", "Name"))
            dur = int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
            try:
                grid = int(_col(r, "Grid_Size_X", "Grid_Size")) * int(r.get("Grid_Size_Y") or 1) * \
                    int(r.get("Grid_Size_Z") or 1)
            except (KeyError, ValueError):
                grid = 0
            out.setdefault(name, []).append((dur, grid))
    return out


def counters(root):
    """{kernel: {counter: mean value per dispatch}} from *_counter_collection.csv.
    Rows with the same dispatch and counter (per-instance rows) are summed first."""
    per = {}  # (kernel, dispatch) -> {counter: value}
    for path in _files(root, "_counter_collection.csv"):
        for r in _read(path):
            name = short_name(_col(r, "Kernel_Name", "Name"))
            disp = (path, _col(r, "Dispatch_Id", "Correlation_Id"))
            cname = _col(r, "Counter_Name")
            val = float(_col(r, "Counter_Value"))
            d = per.setdefault((name, disp), {})
            d[cname] = d.get(cname, 0.0) + val
    acc = {}
    for (name, _), vals in per.items():
        k = acc.setdefault(name, {})
        for c, v in vals.items():
            k.setdefault(c, []).append(v)
    return {name: {c: statistics.mean(v) for c, v in cs.items()} for name, cs in acc.items()}


# ------------------------------------------------------------ derived figures

def derive(c):
    """Derived figures of one kernel's mean counters (keys present only when their
    counters were collected)."""
    out = {}
    g = lambda n: c.get(n)
    if g("GRBM_GUI_ACTIVE"):
        cyc = g("GRBM_GUI_ACTIVE") / XCDS
        out["cycles_per_xcd"] = cyc
        if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            out["mfma_busy"] = g("SQ_VALU_MFMA_BUSY_CYCLES") / (SIMDS * cyc)
        if g("SQ_VALU_MFMA_COEXEC_CYCLES") is not None:
            out["mfma_valu_coissue"] = g("SQ_VALU_MFMA_COEXEC_CYCLES") / (SIMDS * cyc)
        if g("SQ_LDS_IDX_ACTIVE") is not None:
            # share of cycles each CU's LDS spends on indexed (ds_*) operations
            out["lds_busy"] = g("SQ_LDS_IDX_ACTIVE") / (CUS * cyc)
    if g("SQ_INSTS_MFMA"):
        out["mfma_insts"] = g("SQ_INSTS_MFMA")
        if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            out["busy_cycles_per_mfma"] = g("SQ_VALU_MFMA_BUSY_CYCLES") / g("SQ_INSTS_MFMA")
        if g("SQ_INSTS_LDS") is not None:
            out["lds_insts_per_mfma"] = g("SQ_INSTS_LDS") / g("SQ_INSTS_MFMA")
    for key, num in (("valu_share", "SQ_ACTIVE_INST_VALU"), ("wait_any_share", "SQ_WAIT_ANY"),
                     ("wait_issue_share", "SQ_WAIT_INST_ANY"), ("lds_active_share", "SQ_ACTIVE_INST_LDS")):
        if g(num) is not None and g("SQ_WAVE_CYCLES"):
            out[key] = g(num) / g("SQ_WAVE_CYCLES")
    for key, name in (("valu_insts", "SQ_INSTS_VALU"), ("exp_f32_insts", "SQ_INSTS_VALU_TRANS_F32"),
                      ("lds_insts", "SQ_INSTS_LDS"), ("lds_bank_conflict_cycles", "SQ_LDS_BANK_CONFLICT")):
        if g(name) is not None:
            out[key] = g(name)
    return out


def calibration(cnt, copy_bytes):
    """(read factor, write factor): the copy kernel's true bytes per KiB the counter read."""
    copy = [v for k, v in cnt.items() if COPY_KERNEL in k]
    if not copy:
        return None, None
    c = copy[0]
    fr = copy_bytes / (c["FETCH_SIZE"] * 1024) if c.get("FETCH_SIZE") else None
    fw = copy_bytes / (c["WRITE_SIZE"] * 1024) if c.get("WRITE_SIZE") else None
    return fr, fw


PROBES = os.path.join(HERE, "probes")


def source_files(kernel):
    """Sources a kernel's code comes from (paths relative to the package): the .hip
    file that defines it, and the shared device header for the library's kernels;
    the issue-cost probes are self-contained."""
    base = re.match(r"\w+", kernel).group(0)
    pat = re.compile(r"\b" + re.escape(base) + r"\s*\(")
    for d, extra in ((CSRC, ["csrc/mea_device.h"]), (PROBES, [])):
        if not os.path.isdir(d):
            continue
        found = [os.path.relpath(os.path.join(d, f), HERE) for f in sorted(os.listdir(d))
                 if f.endswith(".hip") and pat.search(open(os.path.join(d, f)).read())]
        if found:
            return found + extra
    return []


def source_hash(kernel):
    files = source_files(kernel)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(os.path.join(HERE, f), "rb").read())
    return h.hexdigest()


def collect(prof_dir, copy_bytes, timed=None):
    """Everything the passes under `prof_dir` hold, per kernel. `timed` = (first,
    count): the dispatch range of each kernel that the timed steps cover."""
    trace = {}
    if os.path.isdir(os.path.join(prof_dir, "kt")):
        trace = kernel_trace(os.path.join(prof_dir, "kt"))
    cnt = {}
    for p in PASSES:
        d = os.path.join(prof_dir, p)
        if os.path.isdir(d):
            for k, v in counters(d).items():
                cnt.setdefault(k, {}).update(v)
    fr, fw = calibration(cnt, copy_bytes)
    kernels = {}
    for name in sorted(set(trace) | set(cnt)):
        if COPY_KERNEL in name or not source_files(name):
            continue  # the calibration copy and kernels outside this library
        e = {"kernel": name}
        disp = trace.get(name)
        if disp:
            durs = [dd for dd, _ in disp]
            grids = {}
            for dd, gr in disp:
                grids.setdefault(gr, []).append(dd)
            if len(grids) > 1:  # the same kernel on several shapes: one entry per grid
                e["by_grid"] = {str(gr): {"calls": len(v), "avg_us": statistics.mean(v) / 1e3}
                                for gr, v in sorted(grids.items())}
            e["calls"] = len(durs)
            e["avg_us"] = statistics.mean(durs) / 1e3
            e["min_us"] = min(durs) / 1e3
            e["max_us"] = max(durs) / 1e3
            if timed is not None and len(durs) >= timed[0] + timed[1]:
                sel = durs[timed[0]:timed[0] + timed[1]]
                e["timed_avg_us"] = statistics.mean(sel) / 1e3
        c = cnt.get(name, {})
        e.update(derive(c))
        if fr is not None and c.get("FETCH_SIZE") is not None:
            e["hbm_read_bytes"] = c["FETCH_SIZE"] * 1024 * fr
        if fw is not None and c.get("WRITE_SIZE") is not None:
            e["hbm_write_bytes"] = c["WRITE_SIZE"] * 1024 * fw
        if "hbm_read_bytes" in e and "hbm_write_bytes" in e:
            e["hbm_bytes"] = e["hbm_read_bytes"] + e["hbm_write_bytes"]
            dur = e.get("timed_avg_us", e.get("avg_us"))
            if dur:
                e["hbm_gbs"] = e["hbm_bytes"] / (dur * 1e-6) / 1e9
        e["source_files"] = source_files(name)
        e["source_sha256"] = source_hash(name)
        kernels[name] = e
    return {"read_factor": fr, "write_factor": fw, "copy_bytes": copy_bytes, "kernels": kernels}


# ------------------------------------------------------------ commands and rendering

def plan(prof_dir, program, kt_program=None):
    """Shell commands for every pass: a kernel trace of `kt_program` (default `program`)
    and one counter run of `program` per entry of PASSES, each bounded by a KILL
    timeout (a counter request the hardware cannot serve hangs instead of failing)."""
    kt = kt_program or program
    cmds = ["cd /tmp && export TMPDIR=/tmp",
            f"timeout -s KILL 300 rocprofv3 --kernel-trace --stats --output-format csv "
            f"-d {prof_dir}/kt -o run -- {kt}"]
    for p, cs in PASSES.items():
        cmds.append(f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(cs)} --output-format csv "
                    f"-d {prof_dir}/{p} -o run -- {program}")
    return cmds


def _fmt(x, kind):
    if x is None:
        return "—"
    if kind == "pct":
        return f"{100 * x:.1f}%"
    if kind == "sci":
        return f"{x:.4e}"
    if kind == "us":
        return f"{x:.1f}"
    if kind == "mib":
        return f"{x / 2 ** 20:.1f}"
    if kind == "f1":
        return f"{x:.1f}"
    if kind == "f2":
        return f"{x:.2f}"
    return str(x)


def render(summary, title, commands, note=""):
    """Markdown: commands, kernel trace, counters, HBM traffic, and a JSON block."""
    ks = summary["kernels"]
    out = [f"# {title}", ""]
    out += ["Commands (on one MI355X; each pass in its own run):", "", "```"] + commands + ["```", ""]
    if note:
        out += [note, ""]
    if any("calls" in e for e in ks.values()):
        out += ["Kernel trace:", "",
                "| kernel | calls | avg µs | avg µs (timed steps) | min µs | max µs |",
                "|---|---|---|---|---|---|"]
        for e in ks.values():
            if "calls" in e:
                out.append(f"| `{e['kernel']}` | {e['calls']} | {_fmt(e['avg_us'], 'us')} | "
                           f"{_fmt(e.get('timed_avg_us'), 'us')} | {_fmt(e['min_us'], 'us')} | "
                           f"{_fmt(e['max_us'], 'us')} |")
        out.append("")
    if any("by_grid" in e for e in ks.values()):
        out += ["The same kernels on several shapes, by grid size (work-items):", "",
                "| kernel | grid | calls | avg µs |", "|---|---|---|---|"]
        for e in ks.values():
            for gr, v in e.get("by_grid", {}).items():
                out.append(f"| `{e['kernel']}` | {gr} | {v['calls']} | {_fmt(v['avg_us'], 'us')} |")
        out.append("")
    if any("mfma_busy" in e or "wait_any_share" in e for e in ks.values()):
        out += ["Counters (mean per dispatch):", "",
                "| kernel | cycles per XCD | MFMA instr. | busy cycles / MFMA | MFMA busy | "
                "MFMA+VALU co-issue | wave time in VALU | VALU instr. | `v_exp_f32` | wave time waiting | "
                "waiting to issue | LDS instr. | LDS / MFMA | LDS busy | LDS bank-conflict cycles |",
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for e in ks.values():
            if "mfma_busy" not in e and "wait_any_share" not in e:
                continue
            out.append("| `{}` | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} |".format(
                e["kernel"], _fmt(e.get("cycles_per_xcd"), "sci"), _fmt(e.get("mfma_insts"), "sci"),
                _fmt(e.get("busy_cycles_per_mfma"), "f1"), _fmt(e.get("mfma_busy"), "pct"),
                _fmt(e.get("mfma_valu_coissue"), "pct"), _fmt(e.get("valu_share"), "pct"),
                _fmt(e.get("valu_insts"), "sci"), _fmt(e.get("exp_f32_insts"), "sci"),
                _fmt(e.get("wait_any_share"), "pct"), _fmt(e.get("wait_issue_share"), "pct"),
                _fmt(e.get("lds_insts"), "sci"), _fmt(e.get("lds_insts_per_mfma"), "f2"),
                _fmt(e.get("lds_busy"), "pct"), _fmt(e.get("lds_bank_conflict_cycles"), "sci")))
        out.append("")
    if summary.get("read_factor") is not None or summary.get("write_factor") is not None:
        out += [f"HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the "
                f"copy kernel's true bytes ({summary['copy_bytes']} each way) over its reading: "
                f"read factor {_fmt(summary.get('read_factor'), 'f2')}, write factor "
                f"{_fmt(summary.get('write_factor'), 'f2')}.", "",
                "| kernel | read MiB | written MiB | HBM bytes per launch | HBM GB/s |",
                "|---|---|---|---|---|"]
        for e in ks.values():
            if "hbm_bytes" in e:
                out.append(f"| `{e['kernel']}` | {_fmt(e['hbm_read_bytes'], 'mib')} | "
                           f"{_fmt(e['hbm_write_bytes'], 'mib')} | {e['hbm_bytes']:.4e} | "
                           f"{_fmt(e.get('hbm_gbs'), 'f1')} |")
        out.append("")
    out += ["Machine-readable (read by `bench.py`; `source_sha256` covers the files that define "
            "each kernel, so a changed kernel stops matching):", "", "```json",
            json.dumps(summary, indent=1, sort_keys=True), "```", ""]
    return "\n".join(out)


def render_probes(probe):
    """Markdown tables of `bench.py --mode probe` output (issue costs, overlap,
    LDS-fed MFMA rate, fp32 atomic throughput, HBM stream bandwidth)."""
    out = ["Issue-cost probes (`bench.py --mode probe`; per-wave core cycles from `s_memtime`, "
           "the clock from `s_memtime` over `s_memrealtime`):", "",
           "| probe | waves per SIMD | clock MHz | cycles per iteration (MFMA wave) | "
           "cycles per iteration (VALU wave) | MFMAs per iteration | VALU instr. per iteration |",
           "|---|---|---|---|---|---|---|"]
    for p in probe["raw"]["probes"]:
        out.append(f"| {p['probe']} | {p['waves_per_simd']} | {p['clock_mhz']:.0f} | "
                   f"{p['mfma_wave_cycles_per_iter']:.1f} | {p['valu_wave_cycles_per_iter']:.1f} | "
                   f"{p['mfma_per_iter']} | {p['valu_per_iter']} |")
    out += ["", "Derived:", "", "| probe | figures |", "|---|---|"]
    for k, v in probe["derived"].items():
        if k in ("atomic_dq", "hbm_stream"):
            continue
        txt = ", ".join(f"{a} {b:.3f}" if isinstance(b, float) else f"{a} {b}" for a, b in v.items())
        out.append(f"| {k} | {txt} |")
    out += ["", "fp32 atomic adds in the single-pass backward's dQ pattern (1 x 16 x 16384 x 64, "
            "256-key workgroups, 4.29 GB added; best of three):", "",
            "| mode | ms | TB/s |", "|---|---|---|"]
    for a in probe["raw"]["atomic_dq"]:
        out.append(f"| {a['mode']} | {a['ms']:.3f} | {a['tb_per_s']:.2f} |")
    if probe["raw"].get("hbm_stream"):
        out += ["", "HBM streams (2 GiB of 16-byte vectors, 8192 workgroups of 256 threads; "
                "strided: consecutive vectors across all threads, blocked: one contiguous "
                "256 KiB chunk per workgroup; x4 / x8 loads in flight per thread; copy counts "
                "read + write; best of three after one warm-up launch):", "",
                "| stream | ms | bytes | TB/s |", "|---|---|---|---|"]
        for a in probe["raw"]["hbm_stream"]:
            out.append(f"| {a['mode']} | {a['ms']:.3f} | {a['bytes']:.0f} | {a['tb_per_s']:.2f} |")
    out.append("")
    return "\n".join(out)


def load_summaries(profiles_dir):
    """Every JSON block of the markdown summaries under `profiles_dir`."""
    found = []
    for path in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        text = open(path).read()
        for m in re.finditer(r"```json\n(.*?)\n```", text, flags=re.S):
            try:
                found.append((path, json.loads(m.group(1))))
            except ValueError:
                continue
    return found


def current_figures(profiles_dir, kernel):
    """The latest committed figures of `kernel` whose sources are unchanged since they
    were taken, merged over summaries (a counter summary and a trace summary may
    each hold part), or {} when none match."""
    merged = {}
    want = source_hash(kernel)
    for path, s in load_summaries(profiles_dir):
        e = s.get("kernels", {}).get(kernel)
        if e and e.get("source_sha256") == want:
            for k, v in e.items():
                merged.setdefault(k, v)
            merged.setdefault("profiles", []).append(os.path.basename(path))
    return merged
