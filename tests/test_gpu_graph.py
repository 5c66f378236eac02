"""The hot path under HIP graph capture: every entry point only enqueues
kernels on the given stream (no allocation, no host synchronisation, no
memset), so a step can be captured once and replayed.  The test replays a
captured step several times, with the program's own eager work and
synchronisations in between, and checks every replay bit for bit against
the eager results."""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import dev

pytestmark = pytest.mark.gpu


def te():
    import mxfp8_mixed_precision_amd as m
    return m


def test_graph_replays_equal_eager_results():
    m = te()
    M, N, K = 1040, 784, 640
    xa = dev(workloads.normal_bf16(80, 0, (M, K), 1.0, 0.01))
    xb = dev(workloads.normal_bf16(80, 1, (N, K), 0.05))
    bias = dev(workloads.normal_bf16(80, 2, (N,), 0.5))
    counts = [300, 0, 517, 223]
    splits = torch.tensor(counts, dtype=torch.int32, device="cuda")
    G = len(counts)
    total = sum(counts)
    xg = dev(workloads.normal_bf16(80, 3, (total, K), 1.0))
    wg = dev(workloads.normal_bf16(80, 4, (G * N, K), 0.05))
    gbias = dev(workloads.normal_bf16(80, 5, (G * N,), 0.5))
    u8 = dict(dtype=torch.uint8, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {
        "qa": torch.empty((M, K), **u8), "sa": torch.empty((M, K // 32), **u8),
        "qb": torch.empty((N, K), **u8), "sb": torch.empty((N, K // 32), **u8),
        "qat": torch.empty((M, K), **u8), "sat": torch.empty((M, K // 32), **u8),
        "qc": torch.empty((M, K), **u8), "amax": torch.empty(1, **f32), "scale": torch.empty(1, **f32),
        "scale_inv": torch.empty(1, **f32),
        "d": torch.empty((M, N), **bf), "aux": torch.empty((M, N), **bf),
        "qg": torch.empty((total, K), **u8), "sg": torch.empty((total, K // 32), **u8),
        "qw": torch.empty((G * N, K), **u8), "sw": torch.empty((G * N, K // 32), **u8),
        "dg": torch.empty((total, N), **bf), "auxg": torch.empty((total, N), **bf),
    }
    ws = torch.empty(m.te_amax_workspace_size(M * K), **u8)
    xat = xa.t().contiguous()  # [K, M]: its colwise quantization is [M, K], blocks along K

    def step():
        m.te_mxfp8_quantize(xa, "e4m3", "row", out["qa"], out["sa"])
        m.te_mxfp8_quantize(xb, "e4m3", "row", out["qb"], out["sb"])
        m.te_mxfp8_quantize(xat, "e4m3", "col", None, None, out["qat"], out["sat"])
        m.te_fp8_cast_current_scaling(xa, "e4m3", out["qc"], out["amax"], out["scale"], out["scale_inv"], ws)
        m.te_mxfp8_gemm(out["qa"], out["sa"], "e4m3", out["qb"], out["sb"], "e4m3", out["d"], "bias_gelu_aux",
                        bias, out["aux"])
        m.te_mxfp8_quantize(xg, "e4m3", "row", out["qg"], out["sg"])
        m.te_mxfp8_quantize(wg, "e4m3", "row", out["qw"], out["sw"])
        m.te_mxfp8_grouped_gemm(splits, out["qg"], out["sg"], "e4m3", out["qw"], out["sw"], "e4m3", N, out["dg"],
                                "bias_gelu_aux", gbias, out["auxg"])

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(3):
        for v in out.values():
            v.zero_()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), f"replay {replay}: {k} differs"
