"""Turn rocprofv3 CSV output into the short text summaries kept with the project.

    python -m kv_cache_vector_diag_amd.rocprof_summary stats <kernel_stats.csv>
    python -m kv_cache_vector_diag_amd.rocprof_summary counters <counter_collection.csv> [...]
    python -m kv_cache_vector_diag_amd.rocprof_summary traffic --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --out traffic.json
    python -m kv_cache_vector_diag_amd.rocprof_summary busy --csv B.csv --map kernel=key ... --out traffic.json

``traffic`` scales the per-dispatch FETCH_SIZE / WRITE_SIZE readings (KiB) of
each kernel by the factor that makes the same counter read the known byte
count of a plain device copy, and records the hash of the kernel sources the
counters were taken with (a later source change makes the entry stale).  A
map entry "a+b+c=key" records a step of kernels that each run once per step.
``busy`` records the mean VALUBusy and MfmaUtil (percent) of each mapped
kernel's dispatches in the same file, with their own source hash.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

KERNELS = {
    "gram_scores_fast": "gram_scores",
    "gram_scores_generic": "gram_scores_generic",
    "gram_encode": "gram_encode",
    "gram_table": "gram_table",
    "encode128_pair_kernel": "encode_pair",
    "encode128_kernel": "encode",
    "score128_kernel": "score",
    "encode_generic": "encode_generic",
    "scores_generic": "score_generic",
    "decode_generic": "decode_generic",
    "decode_wh_kernel": "decode_values",
    "attend_part": "attend_part",
    "attend_merge": "attend_merge",
    "attend_mfma": "attend_mfma",
    "attend_fused": "attend_fused",
    "attend_qprep": "attend_qprep",
    "attend": "attend",
    "split256_prep": "split256_prep",
    "split256_kernel": "split256",
    "channel_stats": "channel_stats",
    "select_outliers": "select_outliers",
}


# kernels instantiated for keys and values: (short name, index of the KEY template argument)
ROLE_KERNELS = {"encode128_kernel": ("encode", 1), "encode_tiled_kernel": ("tiled", -1),
                "encode_wide_kernel": ("wide", 1), "split256_kernel": ("split256", -1)}

# sources each measured kernel is built from (a change to any makes its counters stale)
_COMMON = ["tq_device.h", "tq_layout.h", "tq_mfma.h", "tq_fast.h", "../../include/tq.h"]
KERNEL_SOURCES = {
    "encode_keys": ["tq_fast128.hip"] + _COMMON,
    "encode_values": ["tq_fast128.hip"] + _COMMON,
    "wide_keys": ["tq_wide.hip", "tq_kernels.h"] + _COMMON,
    "wide_values": ["tq_wide.hip", "tq_kernels.h"] + _COMMON,
    "decode_values": ["tq_decode.hip", "tq_kernels.h"] + _COMMON,
    "score": ["tq_score128.hip", "tq_score_core.h"] + _COMMON,
    "attend_fused": ["tq_attend.hip", "tq_score_core.h", "tq_kernels.h"] + _COMMON,
    "attend_qprep": ["tq_attend.hip", "tq_score_core.h", "tq_kernels.h"] + _COMMON,
    "attend_merge": ["tq_attend.hip", "tq_kernels.h"] + _COMMON,
    "gram_scores": ["tq_gram.hip", "tq_kernels.h"] + _COMMON,
}


def short_name(kernel_name: str) -> str:
    for key, (short, pos) in ROLE_KERNELS.items():
        if key in kernel_name:
            args = kernel_name.split(key, 1)[1]
            if args.startswith("<"):
                arg = args[1:args.index(">")].split(",")[pos].strip()
                return short + ("_keys" if arg == "true" else "_values" if arg == "false" else "")
            return short
    for key, short in KERNELS.items():
        if key in kernel_name:
            return short
    if "copyBuffer" in kernel_name:
        return "copy"
    if "FillFunctor" in kernel_name:
        return "fill"
    return kernel_name[:48]


def kernel_sources_sha(root: str, kernel: str) -> str:
    """Hash of the sources of one measured kernel (short name, e.g. encode_keys),
    or of a step of several ("attend_qprep+attend_fused+attend_merge": the union
    of their sources, each file once)."""
    h = hashlib.sha256()
    csrc = os.path.join(root, "kv_cache_vector_diag_amd", "csrc")
    names = []
    for part in kernel.split("+"):
        names += [n for n in KERNEL_SOURCES[part] if n not in names]
    for name in names:
        h.update(open(os.path.normpath(os.path.join(csrc, name)), "rb").read())
    return h.hexdigest()[:16]


def cmd_stats(path: str) -> None:
    rows = list(csv.DictReader(open(path)))
    print(f"{'kernel':<16} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}")
    for r in rows:
        print(f"{short_name(r['Name']):<16} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
              f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>6.2f}")


def per_kernel_counters(paths):
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for p in paths:
        for r in csv.DictReader(open(p)):
            agg[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return agg


def cmd_counters(paths) -> None:
    for k, d in sorted(per_kernel_counters(paths).items()):
        print(k)
        for c, v in sorted(d.items()):
            print(f"   {c:<28} {sum(v) / len(v):>16.1f}   (mean of {len(v)} dispatches)")


def cmd_traffic(a) -> None:
    fetch = per_kernel_counters([a.fetch])
    write = per_kernel_counters([a.write])
    cf = per_kernel_counters([a.copy_fetch])["copy"]["FETCH_SIZE"]
    cw = per_kernel_counters([a.copy_write])["copy"]["WRITE_SIZE"]
    # the largest dispatches of the copy kernel are the 1 GiB copies
    f_factor = a.copy_bytes / (max(cf) * 1024.0)
    w_factor = a.copy_bytes / (max(cw) * 1024.0)
    out = json.load(open(a.out)) if os.path.exists(a.out) else {}
    for kern, key in (k.split("=") for k in a.map):
        sha = kernel_sources_sha(a.root, kern)
        # a step of several kernels ("a+b"): each runs once per step, so the
        # step's bytes are the sum of the kernels' per-dispatch means
        rd = wr = 0.0
        for part in kern.split("+"):
            fv = fetch[part]["FETCH_SIZE"]
            wv = write[part]["WRITE_SIZE"]
            rd += sum(fv) / len(fv) * 1024.0 * f_factor
            wr += sum(wv) / len(wv) * 1024.0 * w_factor
        out[key] = {"kernel": kern, "hbm_bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                    "fetch_factor": f_factor, "write_factor": w_factor, "source_sha": sha}
        print(f"{key}: read {rd / 1e6:.1f} MB  write {wr / 1e6:.1f} MB  (factors {f_factor:.3f}, {w_factor:.3f})")
    json.dump(out, open(a.out, "w"), indent=1, sort_keys=True)


def cmd_busy(a) -> None:
    agg = per_kernel_counters([a.csv])
    out = json.load(open(a.out)) if os.path.exists(a.out) else {}
    for kern, key in (k.split("=") for k in a.map):
        ent = out.setdefault(key, {"kernel": kern})
        for counter, field in (("VALUBusy", "valu_busy_pct"), ("MfmaUtil", "mfma_util_pct")):
            v = agg[kern][counter]
            ent[field] = sum(v) / len(v)
        ent["busy_kernel"] = kern
        ent["busy_source_sha"] = kernel_sources_sha(a.root, kern)
        print(f"{key}: VALUBusy {ent['valu_busy_pct']:.1f}%  MfmaUtil {ent['mfma_util_pct']:.1f}%")
    json.dump(out, open(a.out, "w"), indent=1, sort_keys=True)


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats"); s.add_argument("csv")
    c = sub.add_parser("counters"); c.add_argument("csv", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True); t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True); t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    t.add_argument("--map", nargs="+", default=["encode_keys=encode_c3", "score=score_c3"],
                   help="kernel=key pairs")
    t.add_argument("--root", default=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    t.add_argument("--out", required=True)
    u = sub.add_parser("busy")
    u.add_argument("--csv", required=True)
    u.add_argument("--map", nargs="+", required=True, help="kernel=key pairs")
    u.add_argument("--root", default=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    u.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        cmd_stats(a.csv)
    elif a.cmd == "counters":
        cmd_counters(a.csv)
    elif a.cmd == "busy":
        cmd_busy(a)
    else:
        cmd_traffic(a)


if __name__ == "__main__":
    main(sys.argv[1:])
