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
    "gemm": ["gemm.hip"],
    "attn": ["attention.hip"],
    "ln": ["norm.hip"],
    "colsum": ["norm.hip"],
    "block": ["norm.hip"],
    "combine": ["norm.hip"],
    "cube": ["norm.hip"],
}
_SHARED = ["common.h", "kernels.h"]

_EPI = {"EpiStoreF32": "store_f32", "EpiAccumF32": "accum_f32", "EpiStore": "store", "EpiBiasGelu": "bias_gelu",
        "EpiGeluGrad": "gelu_grad", "EpiQkv": "qkv"}
_LAYOUT = {("1", "1"): "nt", ("1", "0"): "nn", ("0", "0"): "tn", ("0", "1"): "tt"}


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
    tag = bm if bm == bn else "%sx%s" % (bm, bn)
    return tag + ("w%d" % waves if waves != 4 else "")


def trace_name(symbol):
    """The library's trace name for a kernel symbol as rocprofv3 reports it
    (mangled or demangled); symbols it does not know pass through, shortened."""
    s = symbol.strip()
    if "gemm_bf16_dl_kernel" in s or "gemm_bf16_pp_kernel" in s:
        pp = "gemm_bf16_pp_kernel" in s
        mm = re.search(r"DlCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E.*?EEELb(\d)ELb(\d)ENS_\d+(\w+?)I", s)
        if mm:
            bm, bn, waves = mm.group(1), mm.group(2), int(mm.group(3)) * int(mm.group(4))
            key, epi = (mm.group(5), mm.group(6)), mm.group(7)
        else:
            mm = re.search(r"DlCfg<(\d+), (\d+), (\d+), (\d+),.*?>, (true|false), (true|false), "
                           r"tpk::(?:\(anonymous namespace\)::)?(\w+)<", s)
            if mm:
                bm, bn, waves, epi = mm.group(1), mm.group(2), int(mm.group(3)) * int(mm.group(4)), mm.group(7)
                key = ("1" if mm.group(5) == "true" else "0", "1" if mm.group(6) == "true" else "0")
        if mm:
            return "gemm_bf16_%s_%s_%s" % (_tile_tag(pp, bm, bn, waves), _LAYOUT[key], _EPI.get(epi, epi))
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
    elif len(argv) >= 7 and argv[0] == "traffic":
        s = traffic_summary(argv[1], argv[2], argv[3], argv[4], float(argv[5]), argv[6])
        sys.stdout.write(json.dumps(s, indent=1) + "\n")
    else:
        sys.stderr.write(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
