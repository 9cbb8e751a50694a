"""rocprofv3 runs of the benchmark and the summaries committed under
``profiles/``.

``collect`` runs ``bench.py`` (one workload and recipe, no variants, no CPU
baseline) under rocprofv3 once per pass, each pass a child process with its
own time limit:

  trace   --kernel-trace --stats              kernel durations
  fetch   --pmc FETCH_SIZE                     HBM bytes read (KiB per dispatch)
  write   --pmc WRITE_SIZE                     HBM bytes written
  sq      --pmc SQ_INSTS_VALU SQ_INSTS_LDS SQ_WAVES VALUBusy MeanOccupancyPerCU

and ``summarize`` turns the CSV output into two short text files named for
the kernel, workload and recipe (``<kernel>_<workload>_<recipe>_trace.txt``
and ``..._counters.txt``).  Each starts with the commands that produced it.

Traffic calibration: the benchmark also runs a plain 16-byte copy kernel of
known size (``k_copy`` of libq4probe.so) in the same process.  Its measured
FETCH_SIZE and WRITE_SIZE per dispatch against the bytes it must move give
one factor each, which scale the step kernel's counters to bytes.

The summaries carry a hash of the step kernels' device source (without
comments and blank space); ``bench.py`` reports the counted traffic only while
that hash matches the current source.

Usage (on a machine with the GPU; summaries go to --dest, raw CSV to --out):
  python -m bit_adamw_update_amd.profiling both --workload gpt-2.7b --recipe zip_sr --dest profiles
  python -m bit_adamw_update_amd.profiling both --workload gpt-2.7b --recipe zip_sr --step-before --passes trace
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KERNEL_SRC = [os.path.join(HERE, "csrc", f) for f in ("q4_kernels.hip", "q4_exact.h", "q4_quant.h")]
PASSES = {
    "trace": ["--kernel-trace", "--stats"],
    "fetch": ["--pmc", "FETCH_SIZE"],
    "write": ["--pmc", "WRITE_SIZE"],
    "sq": ["--pmc", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_WAVES", "VALUBusy", "MeanOccupancyPerCU"],
}
COPY_KERNEL = "k_copy"
BYTE_MIX_KERNEL = "k_byte_mix"
BYTE_MIX_QUEUE_KERNEL = "k_byte_mix_queue"


def kernel_hash() -> str:
    """Hash of the step kernels' device source, without // comments and
    blank space (a comment edit does not orphan the profiles)."""
    h = hashlib.sha256()
    for p in KERNEL_SRC:
        with open(p, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(" ".join(code.split()).encode() + b"\n")
    return h.hexdigest()[:16]


def step_kernel(recipe: str) -> str:
    return {"block8": "k_step8", "fp32": "k_fp32_step"}.get(recipe, "k_fused_step")


STEP_BEFORE = False   # set by --step-before: profile bench.py --step-before instead


def bench_args(workload: str, recipe: str, steps: int, warmup: int) -> list:
    """The benchmark command, relative to the repository root."""
    extra = ["--step-before", "--max-grad-norm", "1.0"] if STEP_BEFORE else []
    return ["python3", "bench.py", "--workload", workload, "--recipe", recipe, "--steps", str(steps), "--warmup",
            str(warmup), "--no-variants", "--no-cpu-baseline", *extra]


def pass_command(name: str, out: str, workload: str, recipe: str, steps: int, warmup: int) -> list:
    rel = os.path.relpath(out, ROOT)
    d = os.path.join(out if rel.startswith("..") else rel, name)
    return ["rocprofv3", *PASSES[name], "--output-format", "csv", "-d", d, "-o", name, "--",
            *bench_args(workload, recipe, steps, warmup)]


def collect(workload: str, recipe: str, out: str, steps: int, warmup: int, passes, limit: int) -> int:
    os.makedirs(out, exist_ok=True)
    for name in passes:
        cmd = ["timeout", "-s", "KILL", str(limit)] + pass_command(name, out, workload, recipe, steps, warmup)
        print(f"[profiling] pass {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"{name}.log"), "w") as log:
            rc = subprocess.call(cmd, stdout=log, stderr=subprocess.STDOUT, cwd=ROOT)
        print(f"[profiling] pass {name}: exit {rc}", flush=True)
        tail = open(os.path.join(out, f"{name}.log")).read().strip().splitlines()[-3:]
        # rocprofv3 itself may end with a segmentation fault after the program
        # finished and its files are complete: accept that when the bench's
        # JSON line was printed
        if rc != 0 and not any(l.startswith("{") for l in open(os.path.join(out, f"{name}.log"))):
            print("\n".join(tail), flush=True)
            return rc
    return 0


# ---------------------------------------------------------------------------
# CSV parsing
# ---------------------------------------------------------------------------

def _rows(out: str, name: str, suffix: str) -> list:
    files = sorted(glob.glob(os.path.join(out, name, "**", f"*{suffix}"), recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _get(row: dict, *keys):
    low = {k.lower(): v for k, v in row.items()}
    for k in keys:
        if k.lower() in low:
            return low[k.lower()]
    raise KeyError(keys)


def _short(name: str) -> str:
    """Kernel name without its return type, namespaces, template arguments
    and parameter list ("void q4::k_fused_step<0, 2, 3, false>(...)" ->
    "k_fused_step")."""
    base = name.replace("(anonymous namespace)::", "").strip()
    if base.startswith("void "):
        base = base[5:]
    base = base.split("(", 1)[0].split("<", 1)[0]
    return base.rsplit("::", 1)[-1].strip()


def trace_durations(out: str) -> dict:
    """Kernel name -> durations (ns) in dispatch order."""
    d = {}
    rows = _rows(out, "trace", "kernel_trace.csv")
    rows.sort(key=lambda r: int(_get(r, "Start_Timestamp")))
    for r in rows:
        d.setdefault(_get(r, "Kernel_Name"), []).append(int(_get(r, "End_Timestamp")) - int(_get(r, "Start_Timestamp")))
    return d


def counters(out: str, name: str) -> dict:
    """Kernel name -> counter name -> values per dispatch, in dispatch order."""
    d = {}
    rows = _rows(out, name, "counter_collection.csv")
    rows.sort(key=lambda r: int(_get(r, "Dispatch_Id")))
    for r in rows:
        d.setdefault(_get(r, "Kernel_Name"), {}).setdefault(_get(r, "Counter_Name"), []).append(
            float(_get(r, "Counter_Value")))
    return d


def _pick(d: dict, name: str) -> list:
    """The keys of d (full kernel names) whose short name is `name`: every
    instantiation of that kernel template, and no other kernel."""
    return [k for k in d if _short(k) == name]


# ---------------------------------------------------------------------------
# Summaries
# ---------------------------------------------------------------------------

def summarize(workload: str, recipe: str, out: str, steps: int, warmup: int, dest: str) -> tuple:
    sys.path.insert(0, ROOT)
    from bit_adamw_update_amd import inputs
    import bench
    wl = inputs.WORKLOADS[workload]()
    kern = step_kernel(recipe)
    alg = bench.alg_bytes(wl, recipe)
    what = "the last microbatch's accumulation pass and the clipped step after it" if STEP_BEFORE else "the step"
    head = [f"# rocprofv3 summary: {kern}, {workload}, recipe {recipe} ({what})"]
    src = [f"kernel_source_sha256_16: {kernel_hash()}"]
    # -- trace
    dur = trace_durations(out)
    names = _pick(dur, kern)
    lines = head + ["# command: " + " ".join(pass_command("trace", out, workload, recipe, steps, warmup))] + src + [""]
    lines.append(f"{'kernel':60s} {'launches':>8s} {'mean_us':>10s} {'last_{}_mean_us'.format(steps):>16s}")
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{_short(k)[:60]:60s} {len(v):8d} {sum(v) / len(v) / 1e3:10.2f} "
                     f"{sum(v[-steps:]) / len(v[-steps:]) / 1e3:16.2f}")
    step_ns = [x for k in names for x in dur[k]]
    lines.append("")
    timed = step_ns[-steps:] if step_ns else []
    if timed:
        avg = sum(timed) / len(timed) / 1e9
        lines.append(f"step_kernel: {kern}")
        lines.append(f"step_launches_timed: {len(timed)}")
        lines.append(f"step_avg_ms_timed: {avg * 1e3:.6f}")
        lines.append(f"alg_bytes_per_launch: {alg}")
        lines.append(f"alg_gbs: {alg / avg / 1e9:.1f}")
        lines.append(f"frac_of_8tbs: {alg / avg / 8e12:.4f}")
    for label, probe_kernel in (("byte_mix_probe_avg_ms", BYTE_MIX_QUEUE_KERNEL),
                                ("byte_mix_step_walk_probe_avg_ms", BYTE_MIX_KERNEL)):
        bm = _pick(dur, probe_kernel)
        if bm:
            v = dur[bm[0]]
            lines.append(f"{label}: {sum(v[-steps:]) / len(v[-steps:]) / 1e6:.4f}")
    if _pick(dur, BYTE_MIX_KERNEL) or _pick(dur, BYTE_MIX_QUEUE_KERNEL):
        # bench.py probes the 8-bit step's own byte mix, the 4-bit one otherwise
        lines.append(f"byte_mix_probe_code_bits: {8 if recipe == 'block8' else 4}")
    prefix = f"accumulate_{workload}_{recipe}" if STEP_BEFORE else f"{kern}_{workload}_{recipe}"
    trace_file = os.path.join(dest, f"{prefix}_trace.txt")
    os.makedirs(dest, exist_ok=True)
    with open(trace_file, "w") as f:
        f.write("\n".join(lines) + "\n")
    # -- counters
    cf, cw, cs = counters(out, "fetch"), counters(out, "write"), counters(out, "sq")
    lines = head + ["# commands:"] + ["#   " + " ".join(pass_command(p, out, workload, recipe, steps, warmup))
                                      for p in ("fetch", "write", "sq")] + src + [""]

    def per_dispatch(c, name, counter):
        vals = [x for k in _pick(c, name) for x in c[k].get(counter, [])]
        return vals[-steps:] if vals else []

    copies_f = per_dispatch(cf, COPY_KERNEL, "FETCH_SIZE")
    copies_w = per_dispatch(cw, COPY_KERNEL, "WRITE_SIZE")
    copy_bytes = bench.COPY_PROBE_BYTES
    fac_f = copy_bytes / (sum(copies_f) / len(copies_f) * 1024) if copies_f else None
    fac_w = copy_bytes / (sum(copies_w) / len(copies_w) * 1024) if copies_w else None
    fetch = per_dispatch(cf, kern, "FETCH_SIZE")
    write = per_dispatch(cw, kern, "WRITE_SIZE")
    lines.append(f"copy_probe_bytes_per_dispatch: {copy_bytes}")
    lines.append(f"fetch_calibration: {fac_f}")
    lines.append(f"write_calibration: {fac_w}")
    traffic = None
    if fetch and write and fac_f and fac_w:
        fb = sum(fetch) / len(fetch) * 1024 * fac_f
        wb = sum(write) / len(write) * 1024 * fac_w
        traffic = fb + wb
        lines.append(f"fetch_kib_per_launch_raw: {sum(fetch) / len(fetch):.1f}")
        lines.append(f"write_kib_per_launch_raw: {sum(write) / len(write):.1f}")
        lines.append(f"fetch_bytes_per_launch: {fb:.0f}")
        lines.append(f"write_bytes_per_launch: {wb:.0f}")
        lines.append(f"traffic_bytes_per_launch: {traffic:.0f}")
        lines.append(f"alg_bytes_per_launch: {alg}")
        lines.append(f"traffic_over_alg: {traffic / alg:.4f}")
    for counter in PASSES["sq"][1:]:
        v = per_dispatch(cs, kern, counter)
        if v:
            lines.append(f"{counter}: {sum(v) / len(v):.6g}")
    v = per_dispatch(cs, kern, "SQ_INSTS_VALU")
    if v:
        lines.append(f"valu_insts_per_element: {sum(v) / len(v) * 64 / wl.numel:.3f}")
    v = per_dispatch(cs, kern, "SQ_INSTS_LDS")
    if v:
        lines.append(f"lds_insts_per_element: {sum(v) / len(v) * 64 / wl.numel:.3f}")
    if not (cf or cw or cs):   # a trace-only run: no counter summary
        return trace_file, None
    counters_file = os.path.join(dest, f"{prefix}_counters.txt")
    with open(counters_file, "w") as f:
        f.write("\n".join(lines) + "\n")
    return trace_file, counters_file


def main():
    ap = argparse.ArgumentParser(description="rocprofv3 passes over bench.py and their summaries")
    ap.add_argument("action", choices=["collect", "summarize", "both"])
    ap.add_argument("--workload", default="gpt-2.7b")
    ap.add_argument("--recipe", default="zip_sr")
    ap.add_argument("--out", default="/tmp/q4prof", help="raw rocprofv3 output (large; kept out of the repository)")
    ap.add_argument("--dest", default=os.path.join(ROOT, "gpurun_out", "profiles"),
                    help="where the text summaries go (copied into profiles/ afterwards)")
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--passes", default="trace,fetch,write,sq")
    ap.add_argument("--limit", type=int, default=180, help="seconds per pass")
    ap.add_argument("--step-before", action="store_true",
                    help="profile the accumulation pass and the clipped step after it (bench.py --step-before)")
    a = ap.parse_args()
    global STEP_BEFORE
    STEP_BEFORE = a.step_before
    out = os.path.join(a.out, f"{a.workload}_{a.recipe}" + ("_accumulate" if a.step_before else ""))
    if a.action in ("collect", "both"):
        rc = collect(a.workload, a.recipe, out, a.steps, a.warmup, a.passes.split(","), a.limit)
        if rc != 0:
            sys.exit(rc)
    if a.action in ("summarize", "both"):
        for f in summarize(a.workload, a.recipe, out, a.steps, a.warmup, a.dest):
            if f:
                print(f"[profiling] wrote {f}", flush=True)


if __name__ == "__main__":
    main()
