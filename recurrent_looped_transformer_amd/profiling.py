"""rocprofv3 passes over bench.py and their summary (kernel table + HBM traffic of the scan).

    python -m recurrent_looped_transformer_amd.profiling run OUT [bench args...]
        (on the MI355X host; starts rocprofv3 as child processes, never touches the GPU itself)
        1. --kernel-trace --stats over `bench.py --steps 3 --warmup 1 --no-cpu ...`
        2. --pmc FETCH_SIZE, 3. --pmc WRITE_SIZE over
           `bench.py --steps 1 --warmup 0 --no-cpu --progress-every 64 ...` (the scan as calls of
           64 positions with a progress line after each: counter collection serialises every
           dispatch; each call adds one 64-row norm kernel)
        4./5. the same two counters over `bench.py --copy-probe 268435456` (a plain 256 MiB
           device copy: the counters' bytes per dispatch for known traffic)
    python -m recurrent_looped_transformer_amd.profiling summarize OUT NAME [bench args...]
        writes profiles/kernels_NAME.md and profiles/traffic_scan_NAME.json
    python -m recurrent_looped_transformer_amd.profiling trace OUT [bench args...]
        (on the MI355X host) only pass 1, over `bench.py --steps 2 --warmup 1 --no-cpu ...`
    python -m recurrent_looped_transformer_amd.profiling summarize-trace OUT NAME [bench args...]
        writes profiles/kernels_NAME.md (kernel table only, no counters)
    python -m recurrent_looped_transformer_amd.profiling run-decode OUT [bench args...]
        (on the MI355X host) the default measurement of bench.py (decoder transitions at the
        prompt's end): --kernel-trace --stats over `bench.py --steps 3 --warmup 1 --no-cpu ...`,
        --pmc FETCH_SIZE and --pmc WRITE_SIZE over `bench.py --steps 1 --warmup 0 --no-cpu ...`
        on the decoder's kernels only (--kernel-include-regex), and the copy probe for both
    python -m recurrent_looped_transformer_amd.profiling summarize-decode OUT NAME [bench args...]
        writes profiles/kernels_NAME.md (kernel table, counters of the decoder's kernels per
        dispatch) and profiles/traffic_memattn_NAME.json (HBM bytes per launch of the memory
        cross-attention kernel, the bench line's roofline.traffic)

Traffic of the scan = the sum of the counters over the scan's dispatches of the single
profiled step: every dispatch from the RMSNorm that precedes the step's first merge GEMM
to the end of the step (the encode that precedes it is excluded). FETCH_SIZE and
WRITE_SIZE are in KiB per dispatch; each is scaled by (copy bytes) / (counter reading of
the copy), so that a plain copy of N bytes reads back N.
"""
from __future__ import annotations

import csv
import collections
import functools
import glob
import hashlib
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 268435456


def _rocprof(out_dir: str, tag: str, prof_args, bench_args, log):
    d = os.path.join(out_dir, tag)
    cmd = ["rocprofv3"] + prof_args + ["--output-format", "csv", "-d", d, "-o", "run", "--",
                                       sys.executable, os.path.join(ROOT, "bench.py")] + bench_args
    print("[profiling] " + " ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    with open(log, "w") as f:
        r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT, timeout=900)
    if r.returncode != 0:
        raise SystemExit(f"rocprofv3 pass {tag} exited with {r.returncode}; see {log}")
    return d


def run(out_dir: str, bench_args):
    out_dir = os.path.abspath(out_dir)   # rocprofv3 runs from /tmp
    os.makedirs(out_dir, exist_ok=True)
    lg = lambda t: os.path.join(out_dir, f"{t}.log")
    _rocprof(out_dir, "trace", ["--kernel-trace", "--stats"],
             ["--steps", "3", "--warmup", "1", "--no-cpu"] + bench_args, lg("trace"))
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        _rocprof(out_dir, c.lower(), ["--pmc", c],
                 ["--steps", "1", "--warmup", "0", "--no-cpu", "--progress-every", "64"] + bench_args, lg(c.lower()))
        _rocprof(out_dir, "copy_" + c.lower(), ["--pmc", c], ["--copy-probe", str(COPY_BYTES)],
                 lg("copy_" + c.lower()))
    # keep only the small CSVs the summary reads (the per-dispatch trace can be hundreds of MB)
    for big in glob.glob(os.path.join(out_dir, "trace", "**", "*kernel_trace.csv"), recursive=True):
        os.remove(big)


@functools.lru_cache(maxsize=None)
def short(name: str) -> str:
    """Kernel name without return type, namespace and argument list (demangled if needed)."""
    if name.startswith("_Z"):
        try:
            # _Float16 mangles as DF16_, which older c++filt builds do not know; half (Dh) reads the same
            name = subprocess.run(["c++filt", name.replace("DF16_", "Dh")], capture_output=True,
                                  text=True).stdout.strip() or name
        except OSError:
            pass
    name = re.sub(r"^void ", "", name).replace("(anonymous namespace)::", "")
    if "<" in name.split("(")[0]:
        depth, end = 0, len(name)
        for i, ch in enumerate(name):
            if ch == "<":
                depth += 1
            elif ch == ">":
                depth -= 1
                if depth == 0:
                    end = i + 1
                    break
        name = name[:end]
    else:
        name = name.split("(")[0]
    return name.replace("rlt::", "").replace("unsigned short", "bf16").replace("_Float16", "f16").replace("half", "f16")


def _one(path_glob: str) -> str:
    hits = glob.glob(path_glob, recursive=True)
    if not hits:
        raise SystemExit(f"no file matches {path_glob}")
    return hits[0]


def _counters(d: str):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def lib_sha() -> str:
    p = os.path.join(ROOT, "recurrent_looped_transformer_amd", "librlt.so")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16] if os.path.exists(p) else ""


def summarize(out_dir: str, name: str, bench_args):
    stats = list(csv.DictReader(open(_one(os.path.join(out_dir, "trace", "**", "*kernel_stats.csv")))))
    copy_f = [float(r["Counter_Value"]) for r in _counters(os.path.join(out_dir, "copy_fetch_size"))
              if "copyBuffer" in r["Kernel_Name"]]
    copy_w = [float(r["Counter_Value"]) for r in _counters(os.path.join(out_dir, "copy_write_size"))
              if "copyBuffer" in r["Kernel_Name"]]
    fs = COPY_BYTES / 1024 / max(copy_f)
    ws = COPY_BYTES / 1024 / max(copy_w)

    def scan_part(rows):
        merge = [i for i, r in enumerate(rows) if "(Ep)7" in short(r["Kernel_Name"])]
        if not merge:
            raise SystemExit("no merge GEMM dispatch found: the scan region is defined by it")
        return rows[merge[0] - 1:]

    fetch = scan_part(_counters(os.path.join(out_dir, "fetch_size")))
    write = scan_part(_counters(os.path.join(out_dir, "write_size")))
    per_k_f, per_k_w = collections.defaultdict(list), collections.defaultdict(list)
    for r in fetch:
        per_k_f[short(r["Kernel_Name"])].append(float(r["Counter_Value"]) * fs * 1024)
    for r in write:
        per_k_w[short(r["Kernel_Name"])].append(float(r["Counter_Value"]) * ws * 1024)
    read_b = sum(sum(v) for v in per_k_f.values())
    write_b = sum(sum(v) for v in per_k_w.values())

    lines = [f"# Kernel summary: {name}", "",
             "Commands (R = repository root on the MI355X host; every file run is committed):", "",
             f"    python -m recurrent_looped_transformer_amd.profiling run OUT {' '.join(bench_args)}",
             "    (rocprofv3 --kernel-trace --stats ... -- python3 R/bench.py --steps 3 --warmup 1 --no-cpu ARGS;",
             "     rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE ... -- python3 R/bench.py --steps 1 --warmup 0 --no-cpu "
             "--progress-every 64 ARGS;",
             f"     the same counters over python3 R/bench.py --copy-probe {COPY_BYTES})",
             f"    python -m recurrent_looped_transformer_amd.profiling summarize OUT {name} {' '.join(bench_args)}", "",
             f"Counter scale: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f} (a {COPY_BYTES >> 20} MiB copy reads "
             f"{max(copy_f):.0f} / writes {max(copy_w):.0f} KiB of counter).", "",
             "rocprofv3 --stats (3 timed + 1 warm-up steps; a step = encode + scan + batched readout):", "",
             "| kernel | calls | total ms | mean us | share | scan HBM read KiB/dispatch | scan HBM write KiB/dispatch |",
             "|---|---|---|---|---|---|---|"]
    for r in stats[:16]:
        k = short(r["Name"])
        f, w = per_k_f.get(k, []), per_k_w.get(k, [])
        mf = f"{sum(f) / len(f) / 1024:.1f}" if f else "-"
        mw = f"{sum(w) / len(w) / 1024:.1f}" if w else "-"
        lines.append(f"| `{k}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% | {mf} | {mw} |")
    lines += ["", f"Scan traffic of one step (dispatches from the first merge's RMSNorm to the end): "
                  f"read {read_b / 1e9:.2f} GB, write {write_b / 1e9:.2f} GB, {len(fetch)} dispatches."]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"kernels_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    sys.path.insert(0, ROOT)
    from recurrent_looped_transformer_amd.synth import CONFIGS
    cfg = dict(zip(bench_args[::2], bench_args[1::2]))
    shape = CONFIGS[cfg.get("--config", "algo_bf16")]
    rec = {"lib_sha": lib_sha(), "scan_mode": int(cfg.get("--scan-mode", 0)),
           "B": int(cfg.get("--batch", shape.batch)), "T": int(cfg.get("--seq-len", shape.seq_len)),
           "bytes_per_launch": read_b + write_b, "read_bytes": read_b, "write_bytes": write_b,
           "fetch_scale": fs, "write_scale": ws, "dispatches": len(fetch),
           "note": f"sum over the scan's dispatches of one step; see kernels_{name}.md"}
    with open(os.path.join(ROOT, "profiles", f"traffic_scan_{name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


def trace(out_dir: str, bench_args):
    out_dir = os.path.abspath(out_dir)
    os.makedirs(out_dir, exist_ok=True)
    _rocprof(out_dir, "trace", ["--kernel-trace", "--stats"], ["--steps", "2", "--warmup", "1", "--no-cpu"] + bench_args,
             os.path.join(out_dir, "trace.log"))
    for big in glob.glob(os.path.join(out_dir, "trace", "**", "*kernel_trace.csv"), recursive=True):
        os.remove(big)


def summarize_trace(out_dir: str, name: str, bench_args):
    stats = list(csv.DictReader(open(_one(os.path.join(out_dir, "trace", "**", "*kernel_stats.csv")))))
    bench_line = ""
    log = os.path.join(out_dir, "trace.log")
    if os.path.exists(log):
        for ln in open(log):
            if ln.startswith("{") and '"metric"' in ln:
                bench_line = ln.strip()
    lines = [f"# Kernel summary: {name}", "",
             "Commands (R = repository root on the MI355X host; every file run is committed):", "",
             f"    python -m recurrent_looped_transformer_amd.profiling trace OUT {' '.join(bench_args)}",
             "    (rocprofv3 --kernel-trace --stats ... -- python3 R/bench.py --steps 2 --warmup 1 --no-cpu ARGS)",
             f"    python -m recurrent_looped_transformer_amd.profiling summarize-trace OUT {name} "
             f"{' '.join(bench_args)}", "",
             f"Library sha256 prefix: {lib_sha()}", "",
             "rocprofv3 --stats (2 timed + 1 warm-up steps):", "",
             "| kernel | calls | total ms | mean us | share |", "|---|---|---|---|---|"]
    for r in stats[:20]:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    if bench_line:
        lines += ["", "bench line of the profiled run (times include the profiler's overhead):", "",
                  "    " + bench_line]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"kernels_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def run_decode(out_dir: str, bench_args):
    out_dir = os.path.abspath(out_dir)
    os.makedirs(out_dir, exist_ok=True)
    lg = lambda t: os.path.join(out_dir, f"{t}.log")
    _rocprof(out_dir, "trace", ["--kernel-trace", "--stats"], ["--steps", "3", "--warmup", "1", "--no-cpu"] + bench_args,
             lg("trace"))
    for big in glob.glob(os.path.join(out_dir, "trace", "**", "*kernel_trace.csv"), recursive=True):
        os.remove(big)
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        # counters on the decoder's kernels only (the transition's GEMMs and attention): the encode
        # that precedes the transitions runs uninstrumented
        _rocprof(out_dir, c.lower(), ["--pmc", c, "--kernel-include-regex", DECODE_KERNELS],
                 ["--steps", "1", "--warmup", "0", "--no-cpu"] + bench_args, lg(c.lower()))
        _rocprof(out_dir, "copy_" + c.lower(), ["--pmc", c], ["--copy-probe", str(COPY_BYTES)], lg("copy_" + c.lower()))


DECODE_KERNELS = "attn_decode_k|gemm_skinny|skinny_reduce"
MEM_ATTN = re.compile(r"attn_decode_k<[^,]+, \d+, false, 1(, false(, (true|false)(, \d+)?)?)?>")   # any NT / block size


def summarize_decode(out_dir: str, name: str, bench_args):
    stats = list(csv.DictReader(open(_one(os.path.join(out_dir, "trace", "**", "*kernel_stats.csv")))))
    copy_f = [float(r["Counter_Value"]) for r in _counters(os.path.join(out_dir, "copy_fetch_size"))
              if "copyBuffer" in r["Kernel_Name"]]
    copy_w = [float(r["Counter_Value"]) for r in _counters(os.path.join(out_dir, "copy_write_size"))
              if "copyBuffer" in r["Kernel_Name"]]
    fs = COPY_BYTES / 1024 / max(copy_f)
    ws = COPY_BYTES / 1024 / max(copy_w)

    def decode_part(rows):
        # the transitions: every dispatch from the first decoder merge GEMM on (the encode precedes it)
        merge = [i for i, r in enumerate(rows) if "(Ep)7" in short(r["Kernel_Name"])]
        if not merge:
            raise SystemExit("no merge GEMM dispatch found")
        return rows[merge[0]:]

    per_k_f, per_k_w = collections.defaultdict(list), collections.defaultdict(list)
    for r in decode_part(_counters(os.path.join(out_dir, "fetch_size"))):
        per_k_f[short(r["Kernel_Name"])].append(float(r["Counter_Value"]) * fs * 1024)
    for r in decode_part(_counters(os.path.join(out_dir, "write_size"))):
        per_k_w[short(r["Kernel_Name"])].append(float(r["Counter_Value"]) * ws * 1024)
    bench_line = ""
    for ln in open(os.path.join(out_dir, "trace.log")):
        if ln.startswith("{") and '"metric"' in ln:
            bench_line = ln.strip()
    cmd = " ".join(bench_args)
    lines = [f"# Kernel summary: {name}", "",
             "Commands (R = repository root on the MI355X host; every file run is committed):", "",
             f"    python -m recurrent_looped_transformer_amd.profiling run-decode OUT {cmd}",
             "    (rocprofv3 --kernel-trace --stats ... -- python3 R/bench.py --steps 3 --warmup 1 --no-cpu ARGS;",
             f"     rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE --kernel-include-regex '{DECODE_KERNELS}' ... -- "
             "python3 R/bench.py --steps 1 --warmup 0 --no-cpu ARGS;",
             f"     the same counters over python3 R/bench.py --copy-probe {COPY_BYTES})",
             f"    python -m recurrent_looped_transformer_amd.profiling summarize-decode OUT {name} {cmd}", "",
             f"Library sha256 prefix: {lib_sha()}", "",
             f"Counter scale: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f} (a {COPY_BYTES >> 20} MiB copy reads "
             f"{max(copy_f):.0f} / writes {max(copy_w):.0f} KiB of counter).", "",
             "rocprofv3 --stats over the whole run (one encode of the prompt, then 1 warm-up + 3 timed decoder "
             "steps + 3 more with bench.py's per-kernel timers; the encoder's kernels carry most of the total):", "",
             "| kernel | calls | total ms | mean us | share | decode HBM read KiB/dispatch | "
             "decode HBM write KiB/dispatch |", "|---|---|---|---|---|---|---|"]
    for r in stats[:24]:
        k = short(r["Name"])
        f, w = per_k_f.get(k, []), per_k_w.get(k, [])
        mf = f"{sum(f) / len(f) / 1024:.1f}" if f else "-"
        mw = f"{sum(w) / len(w) / 1024:.1f}" if w else "-"
        lines.append(f"| `{k}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% | {mf} | {mw} |")
    mem = [k for k in per_k_f if MEM_ATTN.fullmatch(k)]
    if len(mem) != 1:
        raise SystemExit(f"memory cross-attention kernel not found among {sorted(per_k_f)}")
    k = mem[0]
    rd = sum(per_k_f[k]) / len(per_k_f[k])
    wr = sum(per_k_w[k]) / len(per_k_w[k]) if per_k_w.get(k) else 0.0
    st = [r for r in stats if short(r["Name"]) == k][0]
    lines += ["", f"Memory cross-attention `{k}`: {len(per_k_f[k])} counted dispatches, HBM read {rd / 1e9:.3f} GB + "
                  f"write {wr / 1e9:.4f} GB per dispatch; mean duration {float(st['AverageNs']) / 1e3:.1f} us "
                  f"over {st['Calls']} calls (kernel trace)."]
    if bench_line:
        lines += ["", "bench line of the traced run (times include the profiler's overhead):", "", "    " + bench_line]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"kernels_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    sys.path.insert(0, ROOT)
    from recurrent_looped_transformer_amd.synth import CONFIGS
    args = dict(zip(bench_args[::2], bench_args[1::2]))
    shape = CONFIGS[args.get("--config", "paper_shared")]
    rec = {"lib_sha": lib_sha(), "B": int(args.get("--batch", shape.batch)),
           "position": int(args.get("--prompt", shape.seq_len)), "kernel": k,
           "bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr, "fetch_scale": fs, "write_scale": ws,
           "dispatches": len(per_k_f[k]), "mean_us_trace": float(st["AverageNs"]) / 1e3,
           "note": f"counters of the memory cross-attention dispatches of one decoder step; see kernels_{name}.md"}
    with open(os.path.join(ROOT, "profiles", f"traffic_memattn_{name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    cmds = ("run", "summarize", "trace", "summarize-trace", "run-decode", "summarize-decode")
    if len(sys.argv) < 3 or sys.argv[1] not in cmds:
        raise SystemExit(__doc__)
    if sys.argv[1] == "run":
        run(sys.argv[2], sys.argv[3:])
    elif sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3:])
    elif sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3], sys.argv[4:])
    elif sys.argv[1] == "run-decode":
        run_decode(sys.argv[2], sys.argv[3:])
    elif sys.argv[1] == "summarize-decode":
        summarize_decode(sys.argv[2], sys.argv[3], sys.argv[4:])
    else:
        summarize_trace(sys.argv[2], sys.argv[3], sys.argv[4:])
