"""bench.py's command-line contract, checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profile_view_matches_trace_names_and_the_source_hash(tmp_path, monkeypatch):
    """The committed profile is quoted only while it matches the kernel
    sources, and kernel names are found inside the trace's full signatures."""
    import json
    import bench
    rec = {"source_hash": bench.kernel_source_hash(),
           "phases": {"C2b cold gemm": {
               "void w4a4::gemm_int_decode_kernel<1, 2, 1>(w4a4::GemmArgs, int, int*)": {"median_us": 9.0},
               "void at::native::vectorized_elementwise_kernel<4>": {"median_us": 2.0}}}}
    (tmp_path / "phase_kernels.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    got = bench.profile_view("C2b cold gemm", "gemm_int_decode_kernel")
    assert got is not None and got["median_us"] == 9.0 and "gemm_int_decode_kernel" in got["kernel"]
    assert bench.profile_view("C2b cold gemm", "gemm_wide_kernel") is None
    rec["source_hash"] = "0" * 16
    (tmp_path / "phase_kernels.json").write_text(json.dumps(rec))
    assert bench.profile_view("C2b cold gemm", "gemm_int_decode_kernel") is None
