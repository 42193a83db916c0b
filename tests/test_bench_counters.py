"""Host logic of bench.py's counter summary (no GPU): rocprofv3
counter_collection.csv files for the FETCH_SIZE and WRITE_SIZE runs and the
copy calibration are turned into per-op bytes per launch. Synthetic CSVs with
known values: every complete step (the step's kernels in order, found by
name) is averaged, other kernels and incomplete steps are ignored, and the
counters are scaled by the copy calibration."""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write_csv(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows, start=1):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": "Agent 1", "Queue_Id": 1, "Process_Id": 1,
                        "Thread_Id": 1, "Grid_Size": 256, "Kernel_Id": 1, "Kernel_Name": name, "Workgroup_Size": 256,
                        "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 8, "Accum_VGPR_Count": 0,
                        "SGPR_Count": 16, "Counter_Name": counter, "Counter_Value": value,
                        "Start_Timestamp": 10 * i, "End_Timestamp": 10 * i + 5})


def step_kernels(bench):
    """The step's dispatches as the library names them, in order."""
    import invariant_bi_mm_amd as bi
    names = []
    for op, k, n in bench.GEMMS:
        names += [(op, f"void bi::(anonymous namespace)::gemm_kernel<{p[0]}, {p[1]}, 2, 4, false>(x)")
                  for p in bi.bi_gemm_plan(bench.M_GEMM, n, k)]
    names += [("lm_head", f"void bi::(anonymous namespace)::gemm_kernel<{p[0]}, {p[1]}, 2, 4, false>(x)")
              for p in bi.bi_gemm_plan(bench.M_LM, bench.VOCAB, bench.HIDDEN)]
    names += [("lm_logsm", "bi::(anonymous namespace)::log_softmax_kernel(x)"),
              ("rmsnorm", "void bi::(anonymous namespace)::rmsnorm_kernel<8, false>(x)"),
              ("mean", "void bi::(anonymous namespace)::mean_kernel<true, 8>(x)"),
              ("logsm", "bi::(anonymous namespace)::log_softmax_kernel(x)"),
              ("decode_attn", "void bi::(anonymous namespace)::decode_split_kernel<false>(x)"),
              ("decode_attn", "bi::(anonymous namespace)::decode_combine_kernel(x)")]
    return names


def test_summarize_counters(bench, tmp_path):
    seq = step_kernels(bench)
    ops = list(dict.fromkeys(op for op, _ in seq))

    def run(counter, base):
        rows = [("void at::native::fill_kernel(x)", 7.0)]            # not ours: ignored
        for step in range(3):
            for j, (op, name) in enumerate(seq):
                rows.append((name, base * (ops.index(op) + 1) * (step + 1) + j))
            rows.append(("__amd_rocclr_copyBuffer", 5.0))             # between steps: ignored
        rows += [(name, 1e6) for _, name in seq[:3]]                 # an incomplete step: ignored
        return rows

    write_csv(str(tmp_path / "fetch" / "run_counter_collection.csv"), "FETCH_SIZE", run("FETCH_SIZE", 100.0))
    write_csv(str(tmp_path / "write" / "run_counter_collection.csv"), "WRITE_SIZE", run("WRITE_SIZE", 10.0))
    write_csv(str(tmp_path / "cal_fetch" / "run_counter_collection.csv"), "FETCH_SIZE",
              [("void at::native::fill_kernel(x)", 16.0)] + [("__amd_rocclr_copyBuffer", 131072.0)] * 5)
    write_csv(str(tmp_path / "cal_write" / "run_counter_collection.csv"), "WRITE_SIZE",
              [("__amd_rocclr_copyBuffer", 262144.0)] * 5)
    out = tmp_path / "traffic.json"
    bench.summarize_counters(str(tmp_path), str(out))
    d = json.loads(out.read_text())
    assert d["calibration"]["fetch_scale"] == pytest.approx(2.0) and d["calibration"]["write_scale"] == pytest.approx(1.0)
    assert d["steps_averaged"] == {"fetch": 3, "write": 3}
    for op in ops:
        idx = [j for j, (o, _) in enumerate(seq) if o == op]
        # mean over the 3 steps of sum over the op's dispatches of base*(i+1)*(s+1) + j, in KiB, then scaled
        def expect(base, scale):
            per_step = [sum(base * (ops.index(op) + 1) * (s + 1) + j for j in idx) for s in range(3)]
            return sum(per_step) / 3 * 1024 * scale
        e = d["kernels"][op]
        assert e["hbm_fetch_bytes_per_launch"] == round(expect(100.0, 2.0)), op
        assert e["hbm_write_bytes_per_launch"] == round(expect(10.0, 1.0)), op
        assert e["source_sha256"] == bench.source_digest(op)


def test_summarize_counters_needs_a_complete_step(bench, tmp_path):
    seq = step_kernels(bench)
    for sub, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        write_csv(str(tmp_path / sub / "run_counter_collection.csv"), counter, [(n, 1.0) for _, n in seq[:-1]])
    for sub, counter in (("cal_fetch", "FETCH_SIZE"), ("cal_write", "WRITE_SIZE")):
        write_csv(str(tmp_path / sub / "run_counter_collection.csv"), counter, [("__amd_rocclr_copyBuffer", 1.0)])
    with pytest.raises(SystemExit, match="no complete step"):
        bench.summarize_counters(str(tmp_path), str(tmp_path / "t.json"))
