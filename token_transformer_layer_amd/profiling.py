"""rocprofv3 result summaries for the library's kernels.

Two summaries are produced from rocprofv3 CSV output and committed as text:

* kernel statistics (`--kernel-trace --stats`): a markdown table of calls,
  average and total duration per kernel, under the names the library's own
  event trace uses;
* HBM traffic of one kernel: the per-dispatch `FETCH_SIZE` and `WRITE_SIZE`
  counters (KiB, one rocprofv3 run each), scaled by what the same counters
  read for a plain streaming kernel of known size run in the same process
  (`bench.py --copy-mib`), stored as JSON together with a hash of the source
  files that define the kernel, so that a reader can tell when the figure no
  longer describes the code.

    python -m token_transformer_layer_amd.profiling stats STATS_CSV TITLE CMD > out.md
    python -m token_transformer_layer_amd.profiling traffic FETCH_CSV WRITE_CSV KERNEL WORKLOAD COPY_MIB CMD > out.json
"""
import collections
import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# The trace name of a kernel starts with the name of its family; each family
# is defined by these sources (plus the shared helpers).
_FAMILY_SOURCES = {
    "gemm": ["gemm.hip", "gemm_kernels.h", "gemm_nt.hip", "gemm_nn.hip", "gemm_tn.hip", "gemm_mk.hip"],
    "attn": ["attention.hip"],
    "ln": ["norm.hip"],
    "colsum": ["norm.hip"],
    "block": ["norm.hip"],
    "combine": ["norm.hip"],
    "cube": ["norm.hip"],
}
_SHARED = ["common.h", "kernels.h"]

_EPI = {"EpiStoreF32": "store_f32", "EpiAccumF32": "accum_f32", "EpiStore": "store", "EpiBiasGelu": "bias_gelu",
        "EpiGeluGrad": "gelu_grad", "EpiQkv": "qkv", "EpiSplit": "split"}
# ("0", "1"): the input-gradient products of short slices computed transposed
_LAYOUT = {("1", "1"): "nt", ("1", "0"): "nn", ("0", "0"): "tn", ("0", "1"): "mk"}


def kernel_sources(trace_name):
    fam = trace_name.split("_")[0]
    return [os.path.join(CSRC, f) for f in _FAMILY_SOURCES.get(fam, []) + _SHARED]


def source_hash(trace_name):
    """sha256 over the sources that define the kernel family of `trace_name`."""
    h = hashlib.sha256()
    for p in kernel_sources(trace_name):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def _tile_tag(pp, bm, bn, waves=4):
    """The library's name for a tile configuration (see pick_tile in gemm.hip)."""
    if bm == bn == "128":
        return "p128" if pp else "128"
    if (bm, bn, waves) == ("256", "128", 8):
        return "sk256x128"
    tag = bm if bm == bn else "%sx%s" % (bm, bn)
    return tag + ("w%d" % waves if waves != 4 else "")


def trace_name(symbol):
    """The library's trace name for a kernel symbol as rocprofv3 reports it
    (mangled or demangled); symbols it does not know pass through, shortened."""
    s = symbol.strip()
    if "gemm_bf16_dl_kernel" in s or "gemm_bf16_pp_kernel" in s:
        pp = "gemm_bf16_pp_kernel" in s
        mm = re.search(r"DlCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E.*?EEELb(\d)ELb(\d)ENS_\d+([A-Za-z]\w*?)(?:I|E)", s)
        if mm:
            bm, bn, waves = mm.group(1), mm.group(2), int(mm.group(3)) * int(mm.group(4))
            key, epi = (mm.group(5), mm.group(6)), mm.group(7)
        else:
            mm = re.search(r"DlCfg<(\d+), (\d+), (\d+), (\d+),.*?>, (true|false), (true|false), "
                           r"tpk::(?:\(anonymous namespace\)::)?(\w+)[<,>]", s)
            if mm:
                bm, bn, waves, epi = mm.group(1), mm.group(2), int(mm.group(3)) * int(mm.group(4)), mm.group(7)
                key = ("1" if mm.group(5) == "true" else "0", "1" if mm.group(6) == "true" else "0")
        if mm:
            return "gemm_bf16_%s_%s_%s" % (_tile_tag(pp, bm, bn, waves), _LAYOUT[key], _EPI.get(epi, epi))
    mm = re.match(r"_ZN3tpk\d+(splitk_reduce\w*_kernel)INS_\d+([A-Za-z]\w*?)(?:I|E)", s)
    if mm:  # a split reduction, named by the epilogue it applies
        return "%s<%s>" % (mm.group(1), _EPI.get(mm.group(2), mm.group(2)))
    mm = re.match(r"_ZN3tpk(?:12_GLOBAL__N_1)?(\d+)", s)
    if mm:  # mangled name in the library's namespace: the kernel's own name
        n = int(mm.group(1))
        return s[mm.end():mm.end() + n] + ("<bf16>" if "IDF16b" in s else "<f32>" if "Ifv" in s else "")
    s = s.replace("tpk::(anonymous namespace)::", "").replace("tpk::", "")
    return s[:100]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats_markdown(stats_csv, title, cmd):
    rows = _rows(stats_csv)
    out = ["# " + title, "", "Command (run from the repository root on an MI355X):", "", "```", cmd, "```", "",
           "| kernel | calls | avg us | min us | max us | total ms | % of kernel time |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %s | %.1f | %.1f | %.1f | %.3f | %.2f |" % (
            trace_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    return "\n".join(out) + "\n"


def _per_dispatch(counter_csv, counter):
    """{kernel symbol: [per-dispatch counter value, ...]} (values summed over
    the counter's instances within a dispatch)."""
    disp = collections.OrderedDict()
    for r in _rows(counter_csv):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
        disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"])
    out = collections.defaultdict(list)
    for (name, _), v in disp.items():
        out[name].append(v)
    return out


def _copy_kernel(per):
    names = [n for n in per if "bitwise_not" in n]
    if len(names) != 1:
        raise SystemExit("expected one bitwise_not (copy calibration) kernel in the counter CSV, found %d" % len(names))
    return names[0]


def traffic_summary(fetch_csv, write_csv, kernel, workload, copy_mib, cmd):
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    cf = _copy_kernel(fetch)
    cw = _copy_kernel(write)
    f_copy = sum(fetch[cf]) / len(fetch[cf])
    w_copy = sum(write[cw]) / len(write[cw])
    f_factor = copy_kib / f_copy
    w_factor = copy_kib / w_copy
    fk = [v for n, vs in fetch.items() if trace_name(n) == kernel for v in vs]
    wk = [v for n, vs in write.items() if trace_name(n) == kernel for v in vs]
    if not fk or not wk:
        raise SystemExit("kernel %s not found in the counter CSVs" % kernel)
    f_avg = sum(fk) / len(fk)
    w_avg = sum(wk) / len(wk)
    return dict(kernel=kernel, workload=workload, dispatches=len(fk),
                fetch_kib_per_dispatch=round(f_avg, 1), write_kib_per_dispatch=round(w_avg, 1),
                copy_mib=copy_mib, copy_fetch_kib=round(f_copy, 1), copy_write_kib=round(w_copy, 1),
                fetch_factor=round(f_factor, 4), write_factor=round(w_factor, 4),
                bytes_per_launch=round((f_avg * f_factor + w_avg * w_factor) * 1024.0),
                sources=[os.path.basename(p) for p in kernel_sources(kernel)],
                source_sha256=source_hash(kernel), command=cmd)


def _avg_per_kernel(counter_csv, counters):
    """{trace name: {counter: average per dispatch}} over the dispatches of
    each kernel in one counter run."""
    out = {}
    for c in counters:
        for name, vs in _per_dispatch(counter_csv, c).items():
            out.setdefault(trace_name(name), {})[c] = sum(vs) / len(vs)
    return out


# MI355X: compute units and SIMDs per compute unit (the matrix-core
# utilisation divides the busy cycles of all SIMDs by the active cycles of
# the GPU times their number)
# GRBM_GUI_ACTIVE counts busy cycles in each of the 8 accelerator complex
# dies (XCDs) and the per-dispatch value is their sum: one die's busy cycles
# are the sum over 8.
_CUS, _SIMDS, _XCDS = 256, 4, 8


def _clock_mhz(counter_csv):
    """{trace name: average shader clock in MHz over the kernel's dispatches}:
    one die's GRBM_GUI_ACTIVE cycles over the dispatch's own duration (its
    start and end timestamps in the counter run)."""
    cyc, ns = {}, {}
    for r in _rows(counter_csv):
        if r["Counter_Name"] != "GRBM_GUI_ACTIVE":
            continue
        k = trace_name(r["Kernel_Name"])
        cyc[k] = cyc.get(k, 0.0) + float(r["Counter_Value"]) / _XCDS
        ns[k] = ns.get(k, 0.0) + float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return {k: cyc[k] / ns[k] * 1e3 for k in cyc if ns[k] > 0}


def counters_markdown(stats_csv, fetch_csv, write_csv, pass_csvs, copy_mib, kernels, title, cmd):
    """Per kernel: average duration (kernel trace), matrix-core busy share
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs), vector
    instructions per MFMA, waits, LDS bank conflicts, and HBM bytes and GB/s
    from FETCH_SIZE / WRITE_SIZE scaled by a plain copy's counts."""
    dur = {}
    for r in _rows(stats_csv):
        dur[trace_name(r["Name"])] = float(r["AverageNs"])
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_factor = copy_kib / (sum(fetch[_copy_kernel(fetch)]) / len(fetch[_copy_kernel(fetch)]))
    w_factor = copy_kib / (sum(write[_copy_kernel(write)]) / len(write[_copy_kernel(write)]))
    fk, wk = {}, {}
    for n, vs in fetch.items():
        fk.setdefault(trace_name(n), []).extend(vs)
    for n, vs in write.items():
        wk.setdefault(trace_name(n), []).extend(vs)
    cnt, mhz = {}, {}
    for path, names in pass_csvs:
        if "GRBM_GUI_ACTIVE" in names:
            mhz.update(_clock_mhz(path))
        for k, v in _avg_per_kernel(path, names).items():
            cnt.setdefault(k, {}).update(v)
    out = ["# " + title, "", "Commands (run from the repository root on an MI355X):", "", "```", cmd, "```", "",
           "Per dispatch, averaged over the dispatches of each kernel.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
           "(GRBM_GUI_ACTIVE / %d dies x %d SIMDs) (the MFMA counter sums every SIMD's busy cycles, 32 per "
           "32x32x16 instruction; GRBM_GUI_ACTIVE sums the dies' busy cycles); clock = one die's GRBM_GUI_ACTIVE "
           "over the dispatch duration in the counter run, shown only where it is at most the 2400 MHz peak: for short "
           "kernels the GRBM window runs past the dispatch, so their clock is not shown and their MFMA busy is a lower "
           "bound; VALU/MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA (the VALU count includes the "
           "MFMAs); wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; HBM bytes = FETCH_SIZE x %.3f + WRITE_SIZE x %.3f "
           "(the factors that make a plain %d MiB copy read and write %d MiB), GB/s over the kernel's average "
           "duration." % (_XCDS, _CUS * _SIMDS, f_factor, w_factor, copy_mib, copy_mib), "",
           "| kernel | avg us | clock MHz | MFMA busy | VALU / MFMA | wait / wave cycles | "
           "LDS bank conflicts / LDS active | HBM MB | HBM GB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        c = cnt.get(k, {})
        us = dur.get(k, 0.0) / 1e3
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        act = c.get("GRBM_GUI_ACTIVE")
        mf = c.get("SQ_INSTS_MFMA")
        va = c.get("SQ_INSTS_VALU")
        wt, wc = c.get("SQ_WAIT_INST_ANY"), c.get("SQ_WAVE_CYCLES")
        bc, la = c.get("SQ_LDS_BANK_CONFLICT"), c.get("SQ_ACTIVE_INST_LDS")
        fb = sum(fk.get(k, [])) / len(fk[k]) if fk.get(k) else None
        wb = sum(wk.get(k, [])) / len(wk[k]) if wk.get(k) else None
        hbm = (fb * f_factor + wb * w_factor) * 1024.0 if fb is not None and wb is not None else None

        def f(x, fmt):
            return fmt % x if x is not None else "-"
        out.append("| %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            k, f(us, "%.1f"), f(mhz.get(k) if mhz.get(k, 1e9) <= 2400 else None, "%.0f"),
            f(busy / (act / _XCDS * _CUS * _SIMDS) if busy is not None and act else None, "%.3f"),
            f(va / mf if va and mf else None, "%.1f"), f(wt / wc if wt is not None and wc else None, "%.2f"),
            f(bc / la if bc is not None and la else None, "%.3f"), f(hbm / 1e6 if hbm else None, "%.1f"),
            f(hbm / (us * 1e-6) / 1e9 if hbm and us else None, "%.0f")))
    return "\n".join(out) + "\n"


def load_traffic(profiles_dir, kernel, workload):
    """Bytes per launch of `kernel` on `workload` from a committed traffic
    summary, or None when there is none or its sources have changed since."""
    path = os.path.join(profiles_dir, "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel") != kernel or t.get("source_sha256") != source_hash(kernel):
        return None
    return t["bytes_per_launch"]


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        sys.stdout.write(stats_markdown(argv[1], argv[2], argv[3]))
    elif len(argv) >= 9 and argv[0] == "counters":
        # counters STATS FETCH WRITE PASS1 PASS2 COPY_MIB TITLE CMD [KERNEL ...]
        p1 = ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY",
              "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE"]
        p2 = ["SQ_INSTS_VMEM", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
              "SQ_ACTIVE_INST_ANY", "SQ_INSTS_SALU", "SQ_WAVES"]
        sys.stdout.write(counters_markdown(argv[1], argv[2], argv[3], [(argv[4], p1), (argv[5], p2)],
                                           float(argv[6]), argv[9:], argv[7], argv[8]))
    elif len(argv) >= 7 and argv[0] == "traffic":
        s = traffic_summary(argv[1], argv[2], argv[3], argv[4], float(argv[5]), argv[6])
        sys.stdout.write(json.dumps(s, indent=1) + "\n")
    else:
        sys.stderr.write(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
