"""Host logic of bench.py, on the CPU: attribution of profiler dispatches to
the step's ops (the order bench.py launches them in) and the one-GPU rule."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _record():
    ops = [{"label": "fused", "kernels": bench.KERNELS["quantize_bgrad"]},
           {"label": "gemm", "kernels": bench.KERNELS["gemm"]}]
    return {"ops": ops, "pre": 1, "warmup": 1, "steps": 2, "attr_launches": [2, 3]}


def _dispatches(first_fused_kernel):
    # 4 passes over the step, then 2 attribution launches of the fused op and 3 of the GEMM
    ns = "void temx::(anonymous namespace)::"
    fused = [(ns + first_fused_kernel + "<3, true>(...)", 10.0), (ns + "bgrad_final_kernel<1>(...)", 1.0)]
    gemm = [(ns + "mx_gemm_kernel<Cfg<256, 256>>(...)", 100.0)]
    d = (fused + gemm) * 4 + fused * 2 + gemm * 3
    # dispatches that are not the library's are skipped
    return [("__amd_rocclr_copyBuffer", 5.0)] + d


@pytest.mark.parametrize("kernel", ["quantize_both128_kernel", "quantize_colwise_kernel"])
def test_per_op_sums_an_ops_kernels_either_fused_kernel(kernel):
    per = bench._per_op(_dispatches(kernel), _record())
    assert per == {"fused": 11.0, "gemm": 100.0}


def test_per_op_rejects_an_unexpected_kernel():
    with pytest.raises(SystemExit):
        bench._per_op(_dispatches("quantize_rowwise_kernel"), _record())


def test_per_op_rejects_a_missing_dispatch():
    with pytest.raises(SystemExit):
        bench._per_op(_dispatches("quantize_colwise_kernel")[:-1], _record())


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_percentile_interpolates_linearly():
    import bench
    v = [1.0, 2.0, 3.0, 4.0, 5.0]
    assert bench.percentile(v, 50) == 3.0
    assert bench.percentile(v, 0) == 1.0 and bench.percentile(v, 100) == 5.0
    assert abs(bench.percentile(v, 10) - 1.4) < 1e-12 and abs(bench.percentile(v, 90) - 4.6) < 1e-12
    assert bench.percentile([7.0], 90) == 7.0
