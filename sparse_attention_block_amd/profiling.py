"""Summaries of rocprofv3 CSV output for this library's kernels.

  python -m sparse_attention_block_amd.profiling stats TRACE_kernel_stats.csv --command CMD
      per-kernel call counts and durations (rocprofv3 --kernel-trace --stats)
  python -m sparse_attention_block_amd.profiling counters FETCH.csv WRITE.csv --copy-mib N
      --command CMD [--json-dir DIR]
      HBM bytes per dispatch from a FETCH_SIZE pass and a WRITE_SIZE pass (each a
      rocprofv3 --pmc run), scaled by what the same counters read for the plain
      copy kernel k_copy of N MiB (read N MiB, write N MiB) in the same run; with
      --json-dir, one counters_<tag>.json per library kernel tagged below, holding
      the bytes per launch and a digest of the sources the kernel was built from.
  python -m sparse_attention_block_amd.profiling sweep SWEEP.json --command CMD
      a markdown table of a ``bench.py --sweep`` run (step times, union sizes and
      densities, the sparse prefix kernel's rate on union bytes, latency floors)
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

# tag -> (kernel-name pattern, sources whose digest identifies the build)
KERNEL_TAGS = {
    "dense_prefix": (r"k_prefix_ring_bf16<\d+, \d+, \d+, false, false, false>", ["prefix.hip", "losa_api.hip", "losa_internal.h"]),
    "sparse_prefix": (r"k_prefix_quarter_bf16<\d+, \d+, false, false>", ["prefix.hip", "losa_api.hip", "losa_internal.h"]),
    "page_score": (r"k_score_prep<\d+, false, \d+, false>", ["select.hip", "block_attn.h", "losa_internal.h"]),
    "page_select": (r"k_select<\d+, true, \d+, false>", ["select.hip", "block_attn.h", "losa_internal.h"]),
    "sparse_finish": (r"k_finish_active<unsigned short, \d+>", ["finish.hip", "losa_internal.h"]),
    "dense_finish": (r"k_finish<unsigned short, \d+>", ["finish.hip", "losa_internal.h"]),
    "page_meta": (r"k_page_meta<unsigned short, \d+>", ["page_meta.hip", "losa_internal.h"]),
    # floors: an empty kernel and pure reads of cold buffers (selftest library)
    "probe_empty": (r"(^|\W)k_empty($|\W)", ["selftest.hip"]),
    "probe_read_1MiB": (r"k_probe_read<1>", ["selftest.hip"]),
    "probe_read_8MiB": (r"k_probe_read<8>", ["selftest.hip"]),
    "probe_read_16MiB": (r"k_probe_read<16>", ["selftest.hip"]),
    "probe_read_64MiB": (r"k_probe_read<64>", ["selftest.hip"]),
    "probe_gather": (r"(^|\W)k_probe_gather($|\W)", ["selftest.hip"]),
}
COPY_KERNEL = r"(^|\W)k_copy($|\W)"


def source_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(kernel_name: str) -> str:
    n = kernel_name.replace("void ", "")
    return n.split("(")[0]


def stats_table(path: str) -> list:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return rows


def counter_means(path: str, counter: str) -> dict:
    """Per kernel name: (mean over its dispatches, dispatch count); for the copy
    kernel the largest dispatch only (the calibration copy; any other copy in
    the run is small)."""
    vals = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: ((max(v), 1) if re.search(COPY_KERNEL, k) else (sum(v) / len(v), len(v)))
            for k, v in vals.items()}


def find(means: dict, pattern: str):
    hits = [k for k in means if re.search(pattern, k)]
    if len(hits) != 1:
        raise SystemExit(f"kernel pattern {pattern!r} matches {hits}")
    return hits[0]


def print_sweep(path: str, command: str):
    with open(path) as f:
        rec = json.load(f)
    fl = rec["floors"]
    print(f"# LoSA step sweep on one MI355X\n\ncommand: `{command}`\n")
    print("Times are per (layer, step) from HIP-graph replays over the layer replicas; stage "
          "times are medians of the library's stage events, each including one event pair "
          f"({fl['empty_event_pair_us']:.2f} us for an empty pair).\n")
    print("Latency floors (event-bracketed: the rocprofv3 summary of the bench command has the "
          "kernels' own durations): empty kernel back to back "
          f"{fl['empty_kernel_back_to_back_us']:.2f} us, between two events "
          f"{fl['empty_kernel_between_events_us']:.2f} us; pure read of a cold buffer: " +
          ", ".join(f"{k} {v['us_events']:.1f} us ({v['gbps_events']:.0f} GB/s)"
                    for k, v in fl["read"].items()) +
          (f"; gather of {fl['gather']['pages']} cold 8 KiB pages after a dependent page-list "
           f"read, with partial-sized stores: {fl['gather']['us_events']:.1f} us"
           if "gather" in fl else "") + ".\n")
    if "page_meta" in fl:
        pm = fl["page_meta"]
        print(f"Page metadata of a 64K layer (8 KV heads): full build {pm['full_build_us']:.1f} us "
              f"({pm['full_build_gbps_on_keys']:.0f} GB/s on the keys); update after a committed "
              f"block of 16 tokens {pm['commit_16_tokens_us']:.2f} us.\n")
    print("| workload | case | budget | \\|A\\| | layers | step us | dense step us | block us "
          "| union pages / KV head | density | score | select | prefix | finish "
          "| prefix GB/s on union | frac of 8 TB/s | step GB/s |")
    print("|" + "---|" * 17)
    for r in rec["rows"]:
        st = r["stage_us"]
        sparse = r["mode"] != "dense"
        a = r["n_active"]
        a = f"{a:.2f}" if isinstance(a, float) and not float(a).is_integer() else f"{int(a)}"
        cells = [r["group"], r["case"], str(r["budget"]), a, str(r["layers"]),
                 f"{r['step_us']:.1f}", f"{r['dense_step_us']:.1f}", f"{r['block_us']:.1f}",
                 f"{r['union_pages_per_kv_head']:.1f}" if sparse else "all",
                 f"{r['density']:.4f}" if sparse else "1",
                 f"{st['score']:.1f}" if sparse else "-", f"{st['select']:.1f}" if sparse else "-",
                 f"{st['prefix']:.1f}", f"{st['finish']:.1f}",
                 f"{r['prefix_gbps_on_union']:.0f}" if sparse else "-",
                 f"{r['prefix_frac']:.3f}" if sparse else "-",
                 f"{r['step_gbps']:.0f}" if sparse else "-"]
        print("| " + " | ".join(c.replace("|", "\\|") for c in cells) + " |")
    for r in rec["rows"]:
        if "note" in r:
            print(f"\n{r['group']}: {r['note']}; whole-model attention per denoising step "
                  f"{r['model_step_us']:.0f} us (dense first step {r['model_dense_step_us']:.0f} us).")


def resource_rows() -> list:
    """Per-kernel register, scratch, occupancy and static LDS figures of the
    library's kernels, from the compiler's resource-usage remarks when each
    source is compiled for the device with the library's own flags."""
    import tempfile
    from . import build as B
    remarks = []
    with tempfile.TemporaryDirectory() as td:
        for src in B.SOURCES:
            r = subprocess.run([B.HIPCC, *B.FLAGS, "--cuda-device-only", "-c", os.path.join(B.CSRC, src),
                                "-o", os.path.join(td, src + ".o"), "-Rpass-analysis=kernel-resource-usage"],
                               stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"device compile of {src} failed")
            remarks += r.stdout.splitlines()
    rows, cur = [], None
    for line in remarks:
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"mangled": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|TotalSGPRs|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    names = subprocess.run(["c++filt"], input="\n".join(r["mangled"] for r in rows),
                           stdout=subprocess.PIPE, text=True).stdout.splitlines()
    out = []
    for r, n in zip(rows, names):
        n = re.sub(r"\(.*$", "", n)
        n = n[5:] if n.startswith("void ") else n
        if n.startswith("losa::k_"):
            out.append((n.replace("unsigned short", "bf16"), r.get("VGPRs", 0), r.get("AGPRs", 0),
                        r.get("TotalSGPRs", 0), r.get("ScratchSize", 0), r.get("Occupancy", 0),
                        r.get("LDS", 0)))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s1 = sub.add_parser("stats")
    s1.add_argument("csv")
    s1.add_argument("--command", required=True)
    s1.add_argument("--json", help="also write the tagged kernels' averages (with the digest "
                                   "of their sources) to this file")
    s2 = sub.add_parser("counters")
    s2.add_argument("fetch_csv")
    s2.add_argument("write_csv")
    s2.add_argument("--copy-mib", type=int, required=True)
    s2.add_argument("--command", required=True)
    s2.add_argument("--json-dir")
    s3 = sub.add_parser("sweep")
    s3.add_argument("json")
    s3.add_argument("--command", required=True)
    sub.add_parser("resources")
    a = ap.parse_args(argv)

    if a.cmd == "resources":
        print("# gfx950 resource usage of the library's kernels (compiler remarks)\n"
              "# command: python3 -m sparse_attention_block_amd.profiling resources\n"
              "# waves/SIMD is the compiler's bound from registers and static LDS; the\n"
              "# dynamic LDS a launch asks for (not counted here) can lower it further\n")
        print(f"{'kernel':52s} {'VGPRs':>5s} {'AGPRs':>5s} {'SGPRs':>5s} {'scratch':>7s} "
              f"{'waves/SIMD':>10s} {'static_LDS':>10s}")
        for n, v, ag, sg, sc, oc, lds in resource_rows():
            print(f"{n[:52]:52s} {v:5d} {ag:5d} {sg:5d} {sc:7d} {oc:10d} {lds:10d}")
        return 0

    if a.cmd == "sweep":
        print_sweep(a.json, a.command)
        return 0

    if a.cmd == "stats":
        print(f"# rocprofv3 kernel statistics\n# command: {a.command}\n")
        print(f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'time%':>6s}")
        table = stats_table(a.csv)
        for name, calls, avg, mn, mx, pct in table:
            print(f"{name[:64]:64s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {pct:6.2f}")
        if a.json:
            means = {name: (avg, calls) for name, calls, avg, *_ in table}
            rec = {"command": a.command, "kernels": {}}
            for tag, (pat, srcs) in KERNEL_TAGS.items():
                hits = [k for k in means if re.search(pat, k)]
                if len(hits) == 1:
                    avg, calls = means[hits[0]]
                    rec["kernels"][tag] = {"kernel": hits[0], "avg_us": avg, "calls": calls,
                                           "source_digest": source_digest(srcs)}
            with open(a.json, "w") as f:
                json.dump(rec, f, indent=1)
        return 0

    fetch = counter_means(a.fetch_csv, "FETCH_SIZE")
    write = counter_means(a.write_csv, "WRITE_SIZE")
    copy_bytes = a.copy_mib << 20
    kf = find(fetch, COPY_KERNEL)
    kw = find(write, COPY_KERNEL)
    f_scale = copy_bytes / (fetch[kf][0] * 1024)
    w_scale = copy_bytes / (write[kw][0] * 1024)
    print(f"# HBM traffic per dispatch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch)\n"
          f"# command: {a.command}\n"
          f"# calibration: k_copy of {a.copy_mib} MiB read {fetch[kf][0]:.1f} KiB fetched and "
          f"{write[kw][0]:.1f} KiB written -> scale fetch x{f_scale:.4f}, write x{w_scale:.4f}\n")
    print(f"{'kernel':64s} {'n':>4s} {'fetch_KiB':>11s} {'write_KiB':>11s} {'hbm_MiB':>9s}")
    for name in sorted(fetch, key=lambda k: -fetch[k][0]):
        if "losa::" not in name and not re.search(COPY_KERNEL, name):
            continue
        fk = fetch[name][0]
        wk = write.get(name, (0.0, 0))[0]
        mib = (fk * f_scale + wk * w_scale) * 1024 / 2**20
        print(f"{name[:64]:64s} {fetch[name][1]:4d} {fk:11.1f} {wk:11.1f} {mib:9.2f}")
    if a.json_dir:
        for tag, (pat, srcs) in KERNEL_TAGS.items():
            try:
                name = find(fetch, pat)
            except SystemExit:
                continue
            fk = fetch[name][0]
            wk = write.get(name, (0.0, 0))[0]
            rec = {"kernel": name, "fetch_kib": fk, "write_kib": wk, "fetch_scale": f_scale,
                   "write_scale": w_scale,
                   "hbm_bytes_per_launch": (fk * f_scale + wk * w_scale) * 1024,
                   "source_digest": source_digest(srcs), "command": a.command}
            with open(os.path.join(a.json_dir, f"counters_{tag}.json"), "w") as f:
                json.dump(rec, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
