#!/usr/bin/env python3
"""Benchmark of the fused 4-bit AdamW optimizer step on one MI355X.

Default workload: the GPT-style 2.7B parameter set (tied 50304x2560
embedding, 32 layers of qkv 2560x7680, proj 2560x2560, fc 2560x10240,
fc2 10240x2560 and four 2560 LayerNorm vectors; 2,645,688,320 parameters in
257 tensors), ZIP-SR recipe, all state resident in HBM.  One step = one
q4adamw_step over every tensor (a single fused kernel launch).  Inputs are
synthetic and seeded (masters N(0, 0.02), BF16 Student-t gradients with a
per-tensor log-uniform scale) and already resident in HBM when timing starts.

Prints ONE JSON line: G params updated per second, the fused kernel's
achieved algorithmic HBM bandwidth against the 8 TB/s peak, the CPU oracle
timed on a bounded sample of the same workload, and the other recipes and
parameter sets for context.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "G params updated/sec for fused 4-bit AdamW step; HBM GB/s vs 8 TB/s peak"
HBM_PEAK_GBS = 8000.0
COPY_PROBE_BYTES = 4 << 30     # the hand-written copy probe (also the counters' calibration)
READ_PROBE_BYTES = 8 << 30
PROBE_LAUNCHES = 10


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(workload, recipe: str) -> int:
    """Bytes the fused kernel must move per launch (no re-reads counted):
    FP32 param read + write, BF16 grad read, each packed code buffer read +
    write (4 bits per element), each FP32 block scale read + write; factored
    matrices: one packed moment plus the row/column vectors read once."""
    total = 0
    for t in workload.tensors:
        n = t.numel
        if n == 0:
            continue
        nb = (n + 127) // 128
        codes = (n + 1) // 2
        if recipe == "fp32":
            total += 10 * n + 16 * n
        elif recipe == "block8":
            total += 10 * n + 4 * n + 16 * nb   # one byte per code, read and written, two moments
        elif recipe == "factored" and len(t.shape) >= 2:
            total += 10 * n + 2 * codes + 8 * nb + 4 * (t.shape[0] + n // t.shape[0])
        else:
            total += 10 * n + 4 * codes + 16 * nb
    return total


def kernel_hash() -> str:
    from bit_adamw_update_amd.profiling import kernel_hash as h
    return h()


def step_kernel(recipe: str) -> str:
    """The kernel that dominates a recipe's step."""
    from bit_adamw_update_amd.profiling import step_kernel as k
    return k(recipe)


def read_traffic(workload_name: str, recipe: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{step_kernel(recipe)}_{workload_name}_{recipe}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# After a process starts, the step runs slow for its first ~35 ms of GPU
# work while the clocks settle (GPT-2.7B: 5 launches, Llama-1.1B: 10,
# GPT-162M: ~100), so the untimed warm-up runs the asked-for W steps and
# then more until WARMUP_MIN_S of steps have run.
WARMUP_MIN_S = 0.25
WARMUP_CAP = 4000


def warm_up(run_one, warmup: int) -> int:
    """Runs `warmup` steps, then more until WARMUP_MIN_S have passed on the
    synchronized clock (at most WARMUP_CAP); returns the number run."""
    import torch

    t0 = time.perf_counter()
    for _ in range(warmup):
        run_one()
    torch.cuda.synchronize()
    done = warmup
    while time.perf_counter() - t0 < WARMUP_MIN_S and done < WARMUP_CAP:
        for _ in range(max(warmup, 1)):
            run_one()
        done += max(warmup, 1)
        torch.cuda.synchronize()
    return done


def time_workload(workload, recipe: str, steps: int, warmup: int, lm_head_phase: bool = False):
    import torch

    import bit_adamw_update_amd as q4

    dev = torch.device("cuda")
    params = [p.reshape(-1) for p in workload.init_params(dev)]
    consts = workload._tensor_consts(dev)
    grads = [g.reshape(-1).contiguous() for g in workload.grads(1, dev, consts)]
    del consts
    state = q4.Q4State(recipe, workload.tensors, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    hp = dict(workload.hp)
    step = 0

    def one():
        nonlocal step
        step += 1
        state.step(params, grads, step, lm_head_sr=1 if lm_head_phase else 0, **hp)

    warmup_run = warm_up(one, warmup)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        step += 1
        evs[k][0].record(stream)
        state.step(params, grads, step, lm_head_sr=1 if lm_head_phase else 0, **hp)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    out = {"wall_s": wall, "launch_ms": launch_ms, "state": state, "params": params, "grads": grads,
           "warmup_run": warmup_run}
    return out


def time_step_before(workload, recipe: str, steps: int, warmup: int, max_grad_norm: float = 0.0):
    """The step before on the same tensors: one accumulation pass of a BF16
    microbatch with the statistics (q4adamw_accumulate, Q4_ACC_LAST), then
    the step that reuses them (Q4_HP_GRAD_STATS; clipping when
    max_grad_norm > 0).  Returns the average duration of each, in ms."""
    import torch

    import bit_adamw_update_amd as q4

    dev = torch.device("cuda")
    params = [p.reshape(-1) for p in workload.init_params(dev)]
    consts = workload._tensor_consts(dev)
    grads = [g.reshape(-1).contiguous() for g in workload.grads(1, dev, consts)]
    state = q4.Q4State(recipe, workload.tensors, device=dev)
    _, total = state.flat_offsets()
    micro = torch.empty(total, dtype=torch.bfloat16, device=dev)
    off = 0
    for g in workload.grads(2, dev, consts):
        n = g.numel()
        micro[off:off + n].copy_(g.reshape(-1))
        off += (n + 511) // 512 * 512
    del consts
    hp = dict(workload.hp)
    stream = torch.cuda.current_stream()
    step = 0

    def one():
        nonlocal step
        state.accumulate(params, grads, micro, first=False, last=True)
        step += 1
        state.step(params, grads, step, grad_stats=True, max_grad_norm=max_grad_norm, **hp)

    warm_up(one, warmup)
    # enqueued back to back, as a training loop would: the events then time
    # the GPU work, not the host's launch overhead
    ev = []
    for _ in range(steps):
        a0, a1, s1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a0.record(stream)
        state.accumulate(params, grads, micro, first=False, last=True)
        a1.record(stream)
        step += 1
        state.step(params, grads, step, grad_stats=True, max_grad_norm=max_grad_norm, **hp)
        s1.record(stream)
        ev.append((a0, a1, s1))
    torch.cuda.synchronize()
    acc_ms = [a0.elapsed_time(a1) for a0, a1, _ in ev]
    step_ms = [a1.elapsed_time(s1) for _, a1, s1 in ev]
    return sum(acc_ms) / len(acc_ms), sum(step_ms) / len(step_ms)


def _time_launches(fn, launches: int) -> float:
    """Average ms of `launches` back-to-back calls on the current stream
    (HIP events), after two untimed calls."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(launches):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / launches


def byte_mix_ceiling(n_elems: int, bits: int = 4) -> dict:
    """The step's byte mix (libq4probe.so: 12.125 B per element with 4-bit
    codes, 14.125 B with the 8-bit step's bytes; the step's lane layout,
    trivial arithmetic) over as many elements as the workload has (rounded
    up to 512), on the same buffers with runs taken from a queue and with the
    step's own launch of one work-group per run. The ceiling is the faster:
    the queue on the largest sets, the step's launch on small ones."""
    import torch

    from bit_adamw_update_amd import probe
    n = (n_elems + 511) // 512 * 512
    bm = probe.ByteMix(n, bits=bits)
    nbytes = bm.bytes()
    ms_queue = _time_launches(bm.run_queue, PROBE_LAUNCHES)
    ms_walk = _time_launches(bm.run, PROBE_LAUNCHES)
    ms = min(ms_queue, ms_walk)
    out = {"byte_mix_ceiling_gbs": nbytes / (ms * 1e-3) / 1e9, "byte_mix_elems": n, "byte_mix_ms": ms,
           "byte_mix_code_bits": bits,
           "byte_mix_queue_gbs": nbytes / (ms_queue * 1e-3) / 1e9,
           "byte_mix_step_walk_gbs": nbytes / (ms_walk * 1e-3) / 1e9}
    del bm
    torch.cuda.empty_cache()
    return out


def probe_ceilings(n_elems: int, bits: int = 4) -> dict:
    """The practical ceilings of this machine, from the hand-written probes of
    libq4probe.so: the step's byte mix (byte_mix_ceiling), then a plain copy,
    an in-place update of one buffer and a read."""
    import torch

    from bit_adamw_update_amd import probe
    out = byte_mix_ceiling(n_elems, bits)
    a = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms = _time_launches(lambda: probe.copy(b, a), PROBE_LAUNCHES)
    out["copy_ceiling_gbs"] = 2 * COPY_PROBE_BYTES / (ms * 1e-3) / 1e9
    # the same bytes read and written back in place, as the step's state is
    ms = _time_launches(lambda: probe.update_in_place(a), PROBE_LAUNCHES)
    out["in_place_ceiling_gbs"] = 2 * COPY_PROBE_BYTES / (ms * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    r = torch.ones(READ_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(probe.load_library().q4probe_read_sink_words(), dtype=torch.int32, device="cuda")
    ms = _time_launches(lambda: probe.read(r, sink), PROBE_LAUNCHES)
    out["read_ceiling_gbs"] = READ_PROBE_BYTES / (ms * 1e-3) / 1e9
    del r, sink
    torch.cuda.empty_cache()
    return out


def cpu_baseline(workload, recipe: str, max_elems: int):
    """The CPU oracle (single thread, as written) on the leading tensors of
    the same workload: step 1 from the zero state (untimed), then step 2
    (timed), so the timed step decodes a real state.  The leading tensors
    get exactly the values the full workload gives them (the generators draw
    tensor after tensor)."""
    import dataclasses

    import torch

    from oracle import oracle as O
    orec = {"zip_sr": O.ZIP_SR, "ze_eden": O.ZE_EDEN, "factored": O.FACTORED, "fp32": O.FP32}.get(recipe)
    picked, n = [], 0
    for t in workload.tensors:
        if n + t.numel > max_elems and picked:
            break
        picked.append(t)
        n += t.numel
    sub = dataclasses.replace(workload, tensors=picked)
    params = [p.reshape(-1).numpy().copy() for p in sub.init_params("cpu")]
    consts = sub._tensor_consts("cpu")
    states = [O.TensorState8(t.shape, t.tensor_id, t.flags) if recipe == "block8"
              else O.TensorState(O.Config.of(orec), t.shape, t.tensor_id, t.flags) for t in picked]
    dt = 0.0
    for step in (1, 2):
        grads = [g.reshape(-1).view(torch.uint16).numpy().copy() for g in sub.grads(step, "cpu", consts)]
        hp = O.HParams(step=step, **workload.hp)
        t0 = time.perf_counter()
        for st, p, g in zip(states, params, grads):
            st.step(hp, p, g)
        if step == 2:
            dt = time.perf_counter() - t0
        del grads
    names = ", ".join(f"{t.name} {list(t.shape)}" for t in picked)
    return {"value": n / dt / 1e9, "unit": "G params/s", "cores": 1, "kind": "oracle",
            "sample": f"step 2 (state from an untimed step 1) of {recipe} over the leading {n:,} parameters "
                      f"({names}) of {workload.name}, with the workload's own seeded gradients; "
                      f"single-threaded C oracle, {dt:.1f} s",
            "host_cpu": host_cpu_model(), "host_nproc": os.cpu_count(), "oracle_threads": 1}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt-2.7b")
    ap.add_argument("--recipe", default="zip_sr")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--step-before", action="store_true",
                    help="time only the last microbatch's accumulation pass (with the statistics) and the step "
                         "that reuses them, on this workload and recipe (a profiling aid; prints its own JSON line)")
    ap.add_argument("--max-grad-norm", type=float, default=0.0, help="clipping for --step-before")
    ap.add_argument("--cpu-sample", type=int, default=300_000_000,
                    help="elements in the oracle sample (about 8 s of single-threaded oracle work per step)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_adamw_update_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wl = inputs.WORKLOADS[args.workload]()
    n = wl.numel
    log(f"{wl.name}: {n:,} params in {len(wl.tensors)} tensors, recipe {args.recipe}")
    if args.step_before:
        acc_ms, st_ms = time_step_before(wl, args.recipe, args.steps, args.warmup, max_grad_norm=args.max_grad_norm)
        torch.cuda.empty_cache()
        print(json.dumps({"workload": wl.name, "recipe": args.recipe, "params": n, "steps": args.steps,
                          "accumulate_ms": acc_ms, "accumulate_gbs": 6 * n / (acc_ms * 1e-3) / 1e9,
                          "step_ms": st_ms, "max_grad_norm": args.max_grad_norm,
                          # the same probes as the main run (the copy calibrates the counters)
                          **probe_ceilings(n, 8 if args.recipe == "block8" else 4)}), flush=True)
        return
    r = time_workload(wl, args.recipe, args.steps, args.warmup,
                      lm_head_phase=wl.lm_head_switch)
    ms_step = r["wall_s"] * 1e3 / args.steps
    launch_ms = r["launch_ms"]
    avg_launch = sum(launch_ms) / len(launch_ms)
    ab = alg_bytes(wl, args.recipe)
    achieved = ab / (avg_launch * 1e-3) / 1e9
    traffic = read_traffic(wl.name, args.recipe)
    warmup_run = r["warmup_run"]
    del r
    torch.cuda.empty_cache()
    log(f"step {ms_step:.3f} ms wall, fused launch {avg_launch:.3f} ms avg ({min(launch_ms):.3f} min), "
        f"{achieved:.0f} GB/s algorithmic")

    result = {
        "metric": METRIC,
        "value": n / (ms_step * 1e-3) / 1e9,
        "unit": "G params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": warmup_run,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "params": n, "tensors": len(wl.tensors), "recipe": args.recipe,
                   "block": 128, "state": ("8-bit" if args.recipe == "block8" else "4-bit")
                   + " codes + FP32 block scales per moment",
                   "grads": "bf16", "masters": "fp32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": step_kernel(args.recipe), "alg_bytes_per_launch": ab,
                     "alg_bytes_per_param": ab / n, "avg_launch_ms": avg_launch,
                     "launch_ms": {"mean": avg_launch, "median": statistics.median(launch_ms),
                                   "min": min(launch_ms), "max": max(launch_ms)}},
    }
    # the 8-bit step's own byte mix for it; the 4-bit mix for the others
    ceil = probe_ceilings(n, 8 if args.recipe == "block8" else 4)
    log(f"probes: {ceil}")
    result["roofline"]["byte_mix_ceiling_gbs"] = ceil["byte_mix_ceiling_gbs"]
    result["roofline"]["frac_of_ceiling"] = achieved / ceil["byte_mix_ceiling_gbs"]
    result["ceilings"] = ceil

    if not args.no_variants:
        variants = {}
        # the other recipes and sets; FP32 AdamW (quantization off) on the
        # same set as the reference point the 4-bit state is measured against
        plan = [("gpt-2.7b", "ze_eden"), ("llama-1.1b", "zip_sr"), ("qwen3-0.6b-factored", "factored"),
                ("gpt-162m", "zip_sr"), ("gpt-2.7b", "block8"), ("gpt-2.7b", "fp32")]
        for wname, rec in plan:
            if (wname, rec) == (args.workload, args.recipe):
                continue
            w2 = inputs.WORKLOADS[wname]()
            v = time_workload(w2, rec, args.steps, args.warmup, lm_head_phase=w2.lm_head_switch)
            lm = v["launch_ms"]
            avg = sum(lm) / len(lm)
            b2 = alg_bytes(w2, rec)
            extra = 0
            if rec == "factored":
                # the row/column kernel reads every matrix gradient once more
                extra = sum(2 * t.numel for t in w2.tensors if len(t.shape) >= 2)
            variants[f"{wname}/{rec}"] = {
                "params": w2.numel, "ms_per_step": v["wall_s"] * 1e3 / args.steps,
                "gparams_per_s": w2.numel / (v["wall_s"] / args.steps) / 1e9,
                "step_launch_ms": avg, "alg_gbs": (b2 + extra) / (avg * 1e-3) / 1e9,
                "frac_of_peak": (b2 + extra) / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "alg_bytes_per_param": (b2 + extra) / w2.numel, "warmup_run": v["warmup_run"]}
            del v
            torch.cuda.empty_cache()
            if rec == "block8":
                # the 8-bit step against its own byte mix, over the same elements
                c8 = byte_mix_ceiling(w2.numel, bits=8)
                variants[f"{wname}/{rec}"].update(
                    byte_mix8_ceiling_gbs=c8["byte_mix_ceiling_gbs"], byte_mix8_queue_gbs=c8["byte_mix_queue_gbs"],
                    byte_mix8_step_walk_gbs=c8["byte_mix_step_walk_gbs"],
                    frac_of_ceiling=variants[f"{wname}/{rec}"]["alg_gbs"] / c8["byte_mix_ceiling_gbs"])
            log(f"{wname}/{rec}: {variants[f'{wname}/{rec}']}")
        # the step before ([A] "State representation"): accumulation pass with
        # statistics, then the step that reuses them (no second gradient read)
        for wname, rec, clip in (("qwen3-0.6b-factored", "factored", 0.0), ("gpt-2.7b", "zip_sr", 1.0)):
            w2 = inputs.WORKLOADS[wname]()
            acc_ms, st_ms = time_step_before(w2, rec, args.steps, args.warmup, max_grad_norm=clip)
            b2 = alg_bytes(w2, rec)
            acc_bytes = 6 * w2.numel   # read the BF16 gradient and the microbatch, write the gradient
            key = f"{wname}/{rec}+accumulated-stats" + ("+clip" if clip else "")
            variants[key] = {
                "params": w2.numel, "step_launch_ms": st_ms, "step_alg_gbs": b2 / (st_ms * 1e-3) / 1e9,
                "step_frac_of_peak": b2 / (st_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "step_alg_bytes_per_param": b2 / w2.numel,
                "accumulate_ms": acc_ms, "accumulate_gbs": acc_bytes / (acc_ms * 1e-3) / 1e9,
                "max_grad_norm": clip}
            log(f"{key}: {variants[key]}")
            torch.cuda.empty_cache()
        result["variants"] = variants

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl, args.recipe, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
