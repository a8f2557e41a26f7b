"""rocprofv3 runs behind the summaries in profiles/, and the summaries.

    python bench_profiles.py script > run.sh     # the rocprofv3 commands
    python bench_profiles.py summarize DIR       # DIR: their output folder

Each profile set is one bench.py workload.  For every set the script holds
one kernel trace (per-dispatch durations: calls, mean, median, p10, p90,
min, max per kernel and grid) and two HBM counter passes (FETCH_SIZE, then
WRITE_SIZE, each in a run of its own).  The chunked (hybrid) set adds two
passes of shader counters for the matrix-core prefill tile: MFMA operations
and busy cycles, and the instruction mix.

Counter values are turned into bytes with a plain device copy of known
size in the same run (bench.py --calibration-copy: three 1 GiB copies): the
factor is the copy's known bytes over what the counter read for it.

bench.py reads profiles/<set>_pmc.json back for the `traffic` field of its
roofline, and only while the sources of the kernel are the ones the
counters were taken on (a hash of those files is stored per kernel).
"""

import csv
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "paged_kv_cache_mapping_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
OUT = "gpurun_out/prof"
CALIBRATION_BYTES = 3 * (1 << 30)      # bench.py --calibration-copy

# set name: (bench.py arguments, description)
SETS = {
    "decode_llama8b_b64": (
        "--workload llama8b",
        "Llama-3-8B-shaped decode step: 64 sequences of 128..2048 tokens, Hq 32, Hkv 8, D 128, "
        "block 16, bf16; with the bulk-write, T=64-write and streaming-read probe legs"),
    "decode_llama70b_b32": (
        "--workload llama70b",
        "Llama-3-70B-shaped decode step: 32 sequences of 4096 tokens, Hq 64, Hkv 8, D 128, bf16, "
        "rotating over the 80 layers of an 80 GiB cache"),
    "decode_fp8_b128": (
        "--workload fp8",
        "fp8 e4m3 cache decode step: 128 lognormal sequences (median 1024), Hq 32, Hkv 8, D 128"),
    "decode_int4_b64": (
        "--workload int4",
        "INT4 cache decode step: 64 sequences of 128..2048 tokens, Hq 32, Hkv 8, D 128"),
    "decode_prefix_b100": (
        "--workload prefix",
        "shared-prefix decode step: 100 requests over one 2000-token prompt's blocks, 1..64 "
        "private tokens each; with the copy-on-write leg"),
    "multitoken_spec_b64_q4": (
        "--workload spec",
        "multi-token (speculative) step: 64 requests x 4 query tokens, 128..2048 tokens"),
    "hybrid_chunked": (
        "--workload hybrid --no-prefill-part",
        "hybrid-groups chunked step: 4 layers (full, SWA 4096, full, SWA 4096), 96 decode requests "
        "of 1k..16k + 4 prefill chunks of 512 tokens, bf16"),
}

# bench.py --workload -> set
WORKLOAD_SET = {"llama8b": "decode_llama8b_b64", "llama70b": "decode_llama70b_b32",
                "fp8": "decode_fp8_b128", "int4": "decode_int4_b64", "prefix": "decode_prefix_b100",
                "spec": "multitoken_spec_b64_q4", "hybrid": "hybrid_chunked"}

MFMA_PASS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
             "GRBM_GUI_ACTIVE"]
MIX_PASS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
            "SQ_LDS_BANK_CONFLICT", "SQ_WAVES"]

# kernel name fragment -> the source files its code and launch come from
FAMILIES = [
    ("prefill_", ["prefill.hip", "prefill.h", "common.h"]),
    ("cache_write_kernel", ["slot_write.hip", "common.h"]),
    ("slot_mapping_kernel", ["slot_write.hip", "common.h"]),
    ("copy_blocks", ["slot_write.hip"]),
    ("decode_", ["decode_kernels.h", "decode.hip", "common.h"]),
    ("stream_read", [os.path.join("probe", "stream_read.hip")]),
]


def source_hash(kernel):
    """First 16 hex digits of the SHA-256 of the kernel's source files, or
    None for a kernel of no known family."""
    for frag, files in FAMILIES:
        if frag in kernel:
            h = hashlib.sha256()
            for f in files:
                with open(os.path.join(CSRC, f), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()[:16]
    return None


def commands(name):
    """The rocprofv3 command lines of one set (kind -> command)."""
    args = SETS[name][0]
    bench = "python bench.py %s --no-cpu-baseline" % args
    d = "%s/%s" % (OUT, name)
    cmds = {
        "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d %s/trace -o run -- %s"
                 % (d, bench),
        "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/fetch -o run -- "
                 "%s --steps 10 --warmup 2 --calibration-copy" % (d, bench),
        "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s/write -o run -- "
                 "%s --steps 10 --warmup 2 --calibration-copy" % (d, bench),
    }
    if name == "hybrid_chunked":
        cmds["mfma"] = ("rocprofv3 --pmc %s --output-format csv -d %s/mfma -o run -- %s --steps 10 "
                        "--warmup 2" % (" ".join(MFMA_PASS), d, bench))
        cmds["mix"] = ("rocprofv3 --pmc %s --output-format csv -d %s/mix -o run -- %s --steps 10 "
                       "--warmup 2" % (" ".join(MIX_PASS), d, bench))
    return cmds


def script(names):
    """A bash script running the sets' commands one after another, each under
    a time limit, stopping at the first failure."""
    lines = ["set -e", "export TMPDIR=/tmp"]
    for name in names:
        for kind, cmd in commands(name).items():
            lines.append("echo '== %s %s' >&2" % (name, kind))
            lines.append("timeout -k 10 %d %s > %s/%s.%s.log 2>&1"
                         % (420 if kind == "trace" else 300, cmd, OUT, name, kind))
    return "\n".join(lines) + "\n"


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def _grid(row):
    for key in ("Grid_Size", "Grid_Size_X"):
        if key in row:
            return int(float(row[key]))
    return 0


def short_name(kernel):
    name = kernel.strip()
    if name.startswith("void "):
        name = name[5:]
    name = name.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):       # drop the argument list
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _ours(kernel):
    return "pkv::" in kernel or "stream_read_kernel" in kernel


def trace_summary(name, d):
    """profiles/<name>_kernel_trace.txt from the kernel trace under d."""
    path = _find(d, "kernel_trace.csv")
    if path is None:
        return None
    by = {}
    other = []
    for r in csv.DictReader(open(path)):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if _ours(r["Kernel_Name"]):
            by.setdefault((short_name(r["Kernel_Name"]), _grid(r)), []).append(dur)
        else:
            other.append(dur)
    rows = sorted(by.items(), key=lambda kv: -sum(kv[1]))
    lines = ["rocprofv3 kernel trace: " + SETS[name][1],
             "command: " + commands(name)["trace"],
             "durations per dispatch (End - Start), microseconds; grid in work-items", "",
             "%-58s %9s %6s %9s %9s %9s %9s %9s %9s" % ("kernel", "grid", "calls", "mean", "median",
                                                        "p10", "p90", "min", "max")]
    for (k, g), v in rows:
        a = np.array(v)
        lines.append("%-58s %9d %6d %9.2f %9.2f %9.2f %9.2f %9.2f %9.2f"
                     % (k[:58], g, len(a), a.mean(), np.median(a), np.percentile(a, 10),
                        np.percentile(a, 90), a.min(), a.max()))
    if other:
        lines.append("%-58s %9s %6d %9.2f   (harness: inputs, pools, copies, before timing)"
                     % ("other kernels", "-", len(other), float(np.mean(other))))
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, "%s_kernel_trace.txt" % name), "w") as f:
        f.write(text)
    return text


def _counter_rows(d):
    path = _find(d, "counter_collection.csv")
    if path is None:
        return None
    return list(csv.DictReader(open(path)))


def _per_dispatch(rows, counter):
    """{(kernel, grid): [value per dispatch]} for one counter (values of one
    dispatch summed over the rows it was reported in)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], _grid(r))
        disp = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc.setdefault(key, {}).setdefault(disp, 0.0)
        acc[key][disp] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in acc.items()}


def _calibration(per):
    """Bytes per counter unit from the largest copyBuffer dispatches (the
    calibration copies)."""
    copies = [(g, v) for (k, g), v in per.items() if "copyBuffer" in k]
    if not copies:
        return None, None
    g, v = max(copies, key=lambda gv: gv[0])
    per_dispatch = CALIBRATION_BYTES / len(v)
    return per_dispatch / float(np.mean(v)), dict(dispatches=len(v), grid=g,
                                                  bytes_per_dispatch=per_dispatch,
                                                  counter_mean=float(np.mean(v)))


def pmc_summary(name, d):
    """profiles/<name>_pmc.json from the FETCH_SIZE and WRITE_SIZE passes."""
    fetch_rows, write_rows = _counter_rows(os.path.join(d, "fetch")), _counter_rows(os.path.join(d, "write"))
    if fetch_rows is None or write_rows is None:
        return None
    fetch, write = _per_dispatch(fetch_rows, "FETCH_SIZE"), _per_dispatch(write_rows, "WRITE_SIZE")
    ff, fcal = _calibration(fetch)
    wf, wcal = _calibration(write)
    kernels = []
    for key in sorted(set(fetch) & set(write)):
        k, g = key
        if not _ours(k):
            continue
        fk, wk = float(np.mean(fetch[key])), float(np.mean(write[key]))
        kernels.append(dict(kernel=short_name(k), grid=g, launches=[len(fetch[key]), len(write[key])],
                            fetch_counter=fk, write_counter=wk,
                            hbm_bytes_per_launch=int(round(fk * ff + wk * wf)),
                            fetch_bytes_per_launch=int(round(fk * ff)),
                            write_bytes_per_launch=int(round(wk * wf)),
                            source_sha256_16=source_hash(k)))
    rec = dict(set=name, description=SETS[name][1],
               calibration=dict(fetch_bytes_per_unit=ff, write_bytes_per_unit=wf, fetch_copy=fcal,
                                write_copy=wcal, copy_bytes_total=CALIBRATION_BYTES),
               kernels=kernels, commands=[commands(name)["fetch"], commands(name)["write"]])
    with open(os.path.join(PROFILES, "%s_pmc.json" % name), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def shader_summary(name, d):
    """profiles/<name>_prefill_counters.txt from the MFMA and mix passes:
    per prefill-tile dispatch, the counters and the ratios read from them."""
    mf, mx = _counter_rows(os.path.join(d, "mfma")), _counter_rows(os.path.join(d, "mix"))
    if mf is None or mx is None:
        return None
    lines = ["rocprofv3 shader counters: " + SETS[name][1],
             "commands:", "  " + commands(name)["mfma"], "  " + commands(name)["mix"], "",
             "mean per dispatch, by kernel and grid (work-items)", ""]
    vals = {}
    for rows, counters in ((mf, MFMA_PASS), (mx, MIX_PASS)):
        for c in counters:
            for (k, g), v in _per_dispatch(rows, c).items():
                if _ours(k):
                    vals.setdefault((short_name(k), g), {})[c] = (float(np.mean(v)), len(v))
    for (k, g), cs in sorted(vals.items(), key=lambda kv: kv[0]):
        lines.append("%s  grid %d" % (k, g))
        for c in MFMA_PASS + MIX_PASS:
            if c in cs:
                lines.append("  %-32s %16.1f   (%d dispatches)" % (c, cs[c][0], cs[c][1]))
        m = {c: cs[c][0] for c in cs}
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            lines.append("  bf16 MFMA flops per dispatch (MOPS x 512): %.4g"
                         % (m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m and m["GRBM_GUI_ACTIVE"] > 0:
            # GRBM_GUI_ACTIVE adds up the 8 XCDs' busy cycles and the MFMA
            # busy cycles add up the 1024 SIMDs': the share of SIMD cycles
            # with the matrix pipe busy
            lines.append("  GPU-active cycles (GRBM_GUI_ACTIVE / 8 XCDs): %.0f = %.1f us at 2.4 GHz"
                         % (m["GRBM_GUI_ACTIVE"] / 8, m["GRBM_GUI_ACTIVE"] / 8 / 2400.0))
            lines.append("  MFMA busy per SIMD (busy / (1024 SIMDs x GUI_ACTIVE / 8)): %.3f"
                         % (m["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * m["GRBM_GUI_ACTIVE"] / 8)))
            if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
                lines.append("  bf16 MFMA rate over those cycles: %.1f TFLOP/s"
                             % (m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
                                / (m["GRBM_GUI_ACTIVE"] / 8 / 2.4e9) / 1e12))
        if "SQ_INSTS_MFMA" in m and m["SQ_INSTS_MFMA"] > 0 and "SQ_INSTS_VALU" in m:
            lines.append("  VALU (non-MFMA) instructions per MFMA: %.2f; SALU per MFMA: %.2f; "
                         "LDS per MFMA: %.2f"
                         % ((m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]) / m["SQ_INSTS_MFMA"],
                            m.get("SQ_INSTS_SALU", 0) / m["SQ_INSTS_MFMA"],
                            m.get("SQ_INSTS_LDS", 0) / m["SQ_INSTS_MFMA"]))
        lines.append("")
    text = "\n".join(lines)
    with open(os.path.join(PROFILES, "%s_prefill_counters.txt" % name), "w") as f:
        f.write(text)
    return text


def summarize(out_dir):
    done = {}
    for name in SETS:
        d = os.path.join(out_dir, name)
        if not os.path.isdir(d):
            continue
        done[name] = [kind for kind, ok in (("trace", trace_summary(name, os.path.join(d, "trace"))),
                                            ("pmc", pmc_summary(name, d)),
                                            ("shader", shader_summary(name, d))) if ok is not None]
    return done


def traffic(name, fragments):
    """HBM bytes per call from profiles/<name>_pmc.json: the sum, over the
    kernel name fragments, of the most-launched matching kernel's bytes per
    launch; None if the file, a kernel or a source hash does not match."""
    try:
        with open(os.path.join(PROFILES, "%s_pmc.json" % name)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    total = 0
    for frag in fragments:
        cand = [k for k in rec.get("kernels", []) if frag in k["kernel"]]
        if not cand:
            return None
        k = max(cand, key=lambda k: min(k["launches"]))
        if k.get("source_sha256_16") != source_hash(k["kernel"]):
            return None
        total += k["hbm_bytes_per_launch"]
    return total


def main():
    if len(sys.argv) >= 2 and sys.argv[1] == "script":
        names = sys.argv[2:] or list(SETS)
        sys.stdout.write("mkdir -p %s\n" % OUT + script(names))
    elif len(sys.argv) == 3 and sys.argv[1] == "summarize":
        print(json.dumps(summarize(sys.argv[2])))
    else:
        sys.exit(__doc__)


if __name__ == "__main__":
    main()
