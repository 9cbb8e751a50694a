"""Host logic of the profile summaries (no GPU): rocprofv3 CSV output in,
the committed summary lines out.  Synthetic CSV files in rocprofv3's column
layout stand for a run: the step kernel's counters are scaled by the factor
that the copy probe's known bytes give, and the trace summary averages the
last timed launches."""
import os

import bench
from bit_adamw_update_amd import inputs, profiling

HDR_TRACE = ('"Kind","Agent_Id","Queue_Id","Stream_Id","Thread_Id","Dispatch_Id","Kernel_Id","Kernel_Name",'
             '"Correlation_Id","Start_Timestamp","End_Timestamp"')
HDR_PMC = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
           '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count",'
           '"SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
STEP = "void q4::k_fused_step<0, 2, 3, false>(q4::DevTensor const*, long const*, int, long, int, q4::StepScalars)"
MIX = "(anonymous namespace)::k_byte_mix(float*, unsigned short const*, unsigned char*, long, int, float)"
MIX_QUEUE = "(anonymous namespace)::k_byte_mix_queue(float*, unsigned short const*, long, int, unsigned int*, float)"
COPY = "(anonymous namespace)::k_copy(unsigned int __attribute__((ext_vector_type(4)))*, unsigned int const*, long)"


def _write(path, lines):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def test_short_kernel_names():
    assert profiling._short(STEP) == "k_fused_step"
    assert profiling._short(COPY) == "k_copy"
    assert profiling._short("void at::native::vectorized_elementwise_kernel<4, at::native::Mul>(int)") == \
        "vectorized_elementwise_kernel"


def test_summaries_from_synthetic_csv(tmp_path):
    out, dest = str(tmp_path / "raw"), str(tmp_path / "profiles")
    steps = 5
    rows, t = [], 1000
    durs = [7000, 6600, 6500, 6400, 6500, 6600, 6400]          # ns; the last 5 are the timed ones
    for d, dur in enumerate(durs):
        rows.append(f'"KERNEL_DISPATCH","Agent 1",1,0,1,{d + 1},9,"{STEP}",{d + 1},{t},{t + dur}')
        t += dur + 100
    for d in range(12):
        rows.append(f'"KERNEL_DISPATCH","Agent 1",1,0,1,{100 + d},10,"{COPY}",{100 + d},{t},{t + 2000}')
        t += 2100
    # both byte-mix probes: one short name is a prefix of the other's
    for name, dur in ((MIX_QUEUE, 3000), (MIX, 3300)):
        for d in range(steps):
            rows.append(f'"KERNEL_DISPATCH","Agent 1",1,0,1,{200 + d},11,"{name}",{200 + d},{t},{t + dur}')
            t += dur + 100
    _write(os.path.join(out, "trace", "host", "trace_kernel_trace.csv"), [HDR_TRACE] + rows)
    copy_kib = bench.COPY_PROBE_BYTES / 1024 / 2           # a counter that reads half the bytes
    for name, counter, step_val in (("fetch", "FETCH_SIZE", 1000.0), ("write", "WRITE_SIZE", 600.0)):
        rows = []
        for d in range(len(durs)):
            rows.append(f'{d + 1},{d + 1},"Agent 1",1,1,1,256,9,"{STEP}",256,0,0,64,0,90,"{counter}",{step_val},0,1')
        for d in range(12):
            rows.append(f'{100 + d},{100 + d},"Agent 1",1,1,1,256,10,"{COPY}",256,0,0,16,0,20,"{counter}",{copy_kib},0,1')
        _write(os.path.join(out, name, "host", f"{name}_counter_collection.csv"), [HDR_PMC] + rows)
    rows = []
    for d in range(len(durs)):
        for counter, v in (("SQ_INSTS_VALU", 1000.0), ("SQ_INSTS_LDS", 100.0), ("SQ_WAVES", 64.0),
                           ("VALUBusy", 50.0), ("MeanOccupancyPerCU", 20.0)):
            rows.append(f'{d + 1},{d + 1},"Agent 1",1,1,1,256,9,"{STEP}",256,0,0,64,0,90,"{counter}",{v},0,1')
    _write(os.path.join(out, "sq", "host", "sq_counter_collection.csv"), [HDR_PMC] + rows)

    trace_file, counters_file = profiling.summarize("tiny", "zip_sr", out, steps, 3, dest)
    vals = {}
    for f in (trace_file, counters_file):
        assert os.path.basename(f).startswith("k_fused_step_tiny_zip_sr_")
        for line in open(f):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    wl = inputs.tiny()
    assert abs(float(vals["step_avg_ms_timed"]) - sum(durs[-steps:]) / steps / 1e6) < 1e-9
    assert int(vals["alg_bytes_per_launch"]) == bench.alg_bytes(wl, "zip_sr")
    assert float(vals["fetch_calibration"]) == 2.0 and float(vals["write_calibration"]) == 2.0
    assert float(vals["traffic_bytes_per_launch"]) == (1000.0 + 600.0) * 1024 * 2
    assert float(vals["valu_insts_per_element"]) == round(1000.0 * 64 / wl.numel, 3)
    assert vals["kernel_source_sha256_16"] == profiling.kernel_hash()
    assert float(vals["byte_mix_probe_avg_ms"]) == 0.003
    assert float(vals["byte_mix_step_walk_probe_avg_ms"]) == 0.0033
    # the benchmark reads the counted traffic back from the committed file
    assert abs(float(vals["VALUBusy"]) - 50.0) < 1e-9
