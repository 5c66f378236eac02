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
    gbias = dev(workloads.normal_bf16(80, 5, (G, N), 0.5))
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


def test_graph_replays_equal_eager_results_newer_ops():
    """Fused cast-transpose with bias gradient, MXFP8-output GEMM, backward epilogues (dgelu and the fp32
    accumulate, which reads D), delayed-scaling casts and the per-tensor GEMM (both stateful: scale and
    amax history), blockwise quantize, the scale cast and the blockwise GEMM in both modes.  State that a
    step reads and writes is restored before every run."""
    m = te()
    M, N, K = 1056, 800, 640  # multiples of 32 (cast-transpose, MXFP8 output); ragged 128-blocks
    xa = dev(workloads.normal_bf16(81, 0, (M, K), 1.0, 0.01))
    xb = dev(workloads.normal_bf16(81, 1, (N, K), 0.05))
    dy = dev(workloads.normal_bf16(81, 2, (M, N), 1e-3))
    bias = dev(workloads.normal_bf16(81, 3, (N,), 0.5))
    pre = dev(workloads.normal_bf16(81, 4, (M, N), 2.0))
    u8 = dict(dtype=torch.uint8, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {
        "qa": torch.empty((M, K), **u8), "sa": torch.empty((M, K // 32), **u8),
        "qb": torch.empty((N, K), **u8), "sb": torch.empty((N, K // 32), **u8),
        "dq_r": torch.empty((M, N), **u8), "ds_r": torch.empty((M, N // 32), **u8),
        "dq_c": torch.empty((N, M), **u8), "ds_c": torch.empty((N, M // 32), **u8), "db": torch.empty(N, **f32),
        "mx_d": torch.empty((M, N), **u8), "mx_s": torch.empty((M, N // 32), **u8), "mx_aux": torch.empty((M, N), **bf),
        "dgelu": torch.empty((M, N), **bf),
        "pa": torch.empty((M, K), **u8), "pa_inv": torch.empty(1, **f32),
        "pb": torch.empty((N, K), **u8), "pb_inv": torch.empty(1, **f32), "pt_d": torch.empty((M, N), **bf),
        "ba": torch.empty((M, K), **u8), "bsa": torch.empty((M, K // 128), **f32),
        "bb": torch.empty((N, K), **u8), "bsb": torch.empty(((N + 127) // 128, K // 128), **f32),
        "bmx": torch.empty((M, K // 32), **u8),
        "bd_e8m0": torch.empty((M, N), **bf), "bd_fp32": torch.empty((M, N), **bf),
    }
    state0 = {"acc": dev(workloads.normal_bf16(81, 5, (M, N), 10.0)).view(torch.bfloat16).float(),
              "scale_a": torch.tensor([3.0], **f32), "hist_a": torch.tensor([2.0, 5.0, 1.0, 0.0], **f32),
              "scale_b": torch.tensor([0.5], **f32), "hist_b": torch.zeros(16, **f32)}
    state = {k: v.clone() for k, v in state0.items()}
    ws_bgrad = torch.empty(m.te_mxfp8_quantize_bgrad_workspace_size(M, N), **u8)
    ws_a = torch.empty(m.te_amax_workspace_size(M * K), **u8)
    ws_b = torch.empty(m.te_amax_workspace_size(N * K), **u8)
    ws_blk = torch.empty(m.te_fp8_block_gemm_workspace_size(M, N, K, "e8m0"), **u8)

    def step():
        m.te_mxfp8_quantize(xa, "e4m3", "row", out["qa"], out["sa"])
        m.te_mxfp8_quantize(xb, "e4m3", "row", out["qb"], out["sb"])
        m.te_mxfp8_quantize_bgrad(dy, "e5m2", out["dq_r"], out["ds_r"], out["dq_c"], out["ds_c"], out["db"], ws_bgrad)
        m.te_mxfp8_gemm_mxout(out["qa"], out["sa"], "e4m3", out["qb"], out["sb"], "e4m3", out["mx_d"], out["mx_s"],
                              "e4m3", "bias_gelu_aux", bias, out["mx_aux"])
        m.te_mxfp8_gemm(out["qa"], out["sa"], "e4m3", out["qb"], out["sb"], "e4m3", out["dgelu"], "dgelu", None, pre)
        m.te_mxfp8_gemm(out["qa"], out["sa"], "e4m3", out["qb"], out["sb"], "e4m3", state["acc"], "accumulate")
        m.te_fp8_cast_delayed_scaling(xa, "e4m3", out["pa"], out["pa_inv"], state["scale_a"], state["hist_a"], ws_a,
                                      "max", 1)
        m.te_fp8_cast_delayed_scaling(xb, "e4m3", out["pb"], out["pb_inv"], state["scale_b"], state["hist_b"], ws_b,
                                      "most_recent", 0)
        m.te_fp8_gemm(out["pa"], out["pa_inv"], "e4m3", out["pb"], out["pb_inv"], "e4m3", out["pt_d"], "bias", bias)
        m.te_fp8_block_quantize(xa, "e4m3", False, out["ba"], out["bsa"])
        m.te_fp8_block_quantize(xb, "e4m3", True, out["bb"], out["bsb"])
        m.te_fp8_block_scales_to_mx(out["bsa"], M, K, False, out["bmx"])
        m.te_fp8_block_gemm(out["ba"], out["bsa"], "e4m3", out["bb"], out["bsb"], "e4m3", True, out["bd_e8m0"],
                            mode="e8m0", workspace=ws_blk)
        m.te_fp8_block_gemm(out["ba"], out["bsa"], "e4m3", out["bb"], out["bsb"], "e4m3", True, out["bd_fp32"],
                            mode="fp32")

    def restore():
        for k, v in state0.items():
            state[k].copy_(v)

    def snapshot():
        snap = {k: v.clone() for k, v in out.items()}
        snap.update({"state_" + k: v.clone() for k, v in state.items()})
        return snap

    for v in out.values():
        v.zero_()  # every output is written by the step: replays must reproduce all of them
    restore()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    assert not torch.equal(eager["state_hist_a"], state0["hist_a"])  # the step did update its state
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(3):
        for v in out.values():
            v.zero_()          # eager work between replays
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, v in got.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), f"replay {replay}: {k} differs"
