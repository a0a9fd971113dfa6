"""Host logic of bench.py that needs no GPU: the --gpus guard, the attribution of kernel-trace
dispatches to benchmark legs by their markers, the kernel labels, and the summaries written from a
trace (checked on a synthetic trace folder, in a temporary profiles directory)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

MARKER = "void (anonymous namespace)::read_probe_kernel<4>(unsigned int __vector(4) const*, unsigned long)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,label", [
    ("void fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>(fp8gemm::KernelArgs)",
     "fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>"),
    ("fp8gemm::(anonymous namespace)::swiglu_quantize_kernel(fp8gemm::(anonymous namespace)::QuantArgs)",
     "fp8gemm::(anonymous namespace)::swiglu_quantize_kernel"),
    ("fp8gemm::fp8gemm_kernel<64, 64, 1, 4, 4, 0, 2112, 7168>", "fp8gemm::fp8gemm_kernel<64, 64, 1, 4, 4, 0, 2112, 7168>"),
    ("__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"),
])
def test_kernel_label_drops_return_type_and_parameters(name, label):
    assert bench._kernel_label(name) == label


def _dispatch(rows, t, name, wgs, dur, wg=256):
    rows.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur,
                 "Workgroup_Size_X": wg, "Grid_Size_X": wgs * wg})
    return t + dur + 100


def _write_trace(folder, rows):
    os.makedirs(os.path.join(folder, "host"), exist_ok=True)
    with open(os.path.join(folder, "host", "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_dispatches_go_to_the_leg_of_the_last_marker(tmp_path):
    rows, t = [], 1000
    dense = "void fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>(fp8gemm::KernelArgs)"
    # library work before any marker belongs to no leg
    t = _dispatch(rows, t, dense, 256, 5000)
    t = _dispatch(rows, t, MARKER, bench.LEGS.index("sweep") + 1, 500)
    t = _dispatch(rows, t, dense, 256, 7000)
    t = _dispatch(rows, t, "void at::native::reduce_kernel<512, 1>(x)", 1024, 3000)    # not the library's
    t = _dispatch(rows, t, MARKER, bench.LEGS.index("read_floor") + 1, 500)
    # the read floor's own probes (8 and 16 deep, 256+ workgroups) are not markers
    t = _dispatch(rows, t, "void (anonymous namespace)::read_probe_kernel<8>(x)", 512, 9000)
    t = _dispatch(rows, t, "void (anonymous namespace)::read_probe_kernel<16>(x)", 2, 9000)
    t = _dispatch(rows, t, MARKER, bench.LEGS.index("masked_cfg4") + 1, 500)
    t = _dispatch(rows, t, "void fp8gemm::fp8gemm_masked_decode_kernel<128, 4, 4, 2, 4, false>(fp8gemm::KernelArgs)",
                  256, 11000)
    # rows out of start order in the file are sorted first
    rows.reverse()
    _write_trace(str(tmp_path), rows)
    legs = bench.legs_of(bench.trace_dispatches(str(tmp_path)))
    assert legs["sweep"] == [("fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>", 7.0)]
    assert legs["read_floor"] == []
    assert legs["masked_cfg4"] == [("fp8gemm::fp8gemm_masked_decode_kernel<128, 4, 4, 2, 4, false>", 11.0)]


def test_grid_sizes_in_workgroups_are_read_too(tmp_path):
    rows = []
    t = _dispatch(rows, 0, MARKER, 1, 500, wg=1)                 # a grid given in workgroups
    rows[-1]["Grid_Size_X"] = bench.LEGS.index("contiguous_cfg2") + 1
    _dispatch(rows, t, "void fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 1, 0, 0>(a)", 256, 2000)
    _write_trace(str(tmp_path), rows)
    legs = bench.legs_of(bench.trace_dispatches(str(tmp_path)))
    assert list(legs) == ["contiguous_cfg2"]
    assert legs["contiguous_cfg2"][0][1] == 2.0


def test_trace_summary_writes_the_three_profiles(tmp_path, monkeypatch):
    rows, t = [], 0
    dense = "void fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>(fp8gemm::KernelArgs)"
    for leg in bench.LEGS:
        t = _dispatch(rows, t, MARKER, bench.LEGS.index(leg) + 1, 100)
        if leg == "sweep_per_shape":
            for us in (170, 180, 190):
                t = _dispatch(rows, t, dense, 256, us * 1000)
    trace = tmp_path / "trace"
    _write_trace(str(trace), rows)
    line = {"roofline": {"kernel": "nt tile=256x256 waves=4x2 stages=2 split=1", "avg_launch_us": 181.0,
                         "launches_per_step": 5, "achieved": 2000.0, "frac": 0.4, "peak": 5000.0},
            "per_shape": [{"M": 4096, "N": 4096, "K": 7168, "us": 103.0, "tflops": 2300.0, "gbs": 900.0,
                           "config": "nt tile=256x256"}],
            "grouped": {"masked_cfg4": {"us": 100.0, "config": "masked"}},
            "moe_expert_chain": {}, "quantize_1x128": {}}
    js = tmp_path / "bench.json"
    js.write_text("log line\n" + json.dumps(line) + "\n")
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    bench.trace_summary(str(trace), str(js))
    dense_txt = (out / "profiles" / "kernel_stats_dense_sweep_bench.txt").read_text()
    assert "rocprofv3, per-shape leg: 3 dispatches, average 180.00 us" in dense_txt
    assert "avg_launch_us 181.00" in dense_txt
    assert "0123456789abcdef" in dense_txt
    grouped_txt = (out / "profiles" / "kernel_stats_grouped_moe_bench.txt").read_text()
    assert "leg masked_cfg4: bench 100.00 us per call (masked)" in grouped_txt
    assert (out / "profiles" / "kernel_stats_quantize_1x128_bench.txt").exists()


def test_trace_summary_refuses_a_trace_without_markers(tmp_path):
    rows = []
    _dispatch(rows, 0, "void fp8gemm::fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>(a)", 256, 1000)
    _write_trace(str(tmp_path / "t"), rows)
    js = tmp_path / "b.json"
    js.write_text(json.dumps({"roofline": {"kernel": "nt tile=256x256"}}) + "\n")
    with pytest.raises(SystemExit):
        bench.trace_summary(str(tmp_path / "t"), str(js))


def test_gpu_state_sample_never_fails(monkeypatch):
    import subprocess

    class R:
        stdout = '{"card0": {"sclk clock speed:": "(2100Mhz)", "Current Socket Graphics Package Power (W)": "900", "unrelated": 1}}'

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R())
    st = bench.sample_gpu_state()
    assert st == {"card0": {"sclk clock speed": "(2100Mhz)", "Current Socket Graphics Package Power (W)": "900"}}

    def boom(*a, **k):
        raise FileNotFoundError("rocm-smi")

    monkeypatch.setattr(subprocess, "run", boom)
    assert "unavailable" in bench.sample_gpu_state()


@pytest.mark.parametrize("label,key", [
    ("dense 64x2112x7168", "dense 64x2112x7168"),
    ("contiguous cfg2 4x8192 N=4096 K=7168", "contiguous cfg2"),
    ("masked cfg4 16x256 N=4096 K=7168", "masked cfg4"),
    ("masked fp8xfp4 cfg4 16x256 N=4096 K=7168", "masked fp8xfp4 cfg4"),
    ("quantize_1x128 32768x7168", "quantize_1x128 32768x7168"),
])
def test_counter_labels_map_to_bench_legs(label, key):
    assert bench.leg_key(label) == key


def test_leg_traffic_only_from_summaries_of_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = ("title\ncommand\nsummary\nkernel_source_sha256_16: %s\n"
            "dense 64x2112x7168  [fp8gemm_kernel<64, 64, 1, 4, 4, 0, 0, 0>]\n"
            "    derived: hbm_MB 26.897  alg_MB 15.886  hbm/alg 1.693\n"
            "    raw: FETCH_SIZE 1\n"
            "masked fp8xfp4 cfg4 16x256 N=4096 K=7168  [fp8gemm_masked_decode_kernel<128, 4, 2, 2, 8, true>]\n"
            "    derived: hbm_MB 273.519  alg_MB 265.426\n")
    (prof / "counters_dense_decode.txt").write_text(body % "0123456789abcdef")
    # a summary of other kernel sources: its numbers must not be used
    (prof / "counters_grouped.txt").write_text((body % "fedcba9876543210").replace("273.519", "999.0")
                                                .replace("dense 64x2112x7168", "dense 128x2112x7168"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    t = bench.read_leg_traffic()
    assert t == {"dense 64x2112x7168": 26897000, "masked fp8xfp4 cfg4": 273519000}
