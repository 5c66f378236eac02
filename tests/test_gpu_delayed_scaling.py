"""GPU parity of the delayed-scaling cast (amax history) and the per-tensor
FP8 GEMM against the CPU oracle.

* Delayed scaling: multi-step sequences on tensors whose amax rises and
  falls; after every step the codes, q_scale_inv, the history and the next
  scale equal the oracle's bit for bit (the oracle state is carried along).
* Per-tensor GEMM: bf16 / fp32 D bit-exact against the MFMA model with unit
  block scales and the fp32 alpha applied to the accumulators, GELU outputs
  to bf16 precision, and everything within the oracle's GEMM bound.
"""

import numpy as np
import pytest
import torch

import mfma_model
import oracle
import workloads
from gpu_util import assert_stated_misses, bf16_to_f64, dev, gemm_check, host, model_outputs

pytestmark = pytest.mark.gpu


def te():
    import mxfp8_mixed_precision_amd as m
    return m


SIGMAS = [1.0, 4.0, 0.25, 0.5, 2.0, 0.0, 1.0]   # a 0.0 step: an all-zero tensor


@pytest.mark.parametrize("fmt,algo,margin,L,n", [("e4m3", "max", 0, 4, 4096 * 8 + 5),
                                                  ("e4m3", "most_recent", 1, 3, 1000),
                                                  ("e5m2", "max", 2, 16, 4096 * 4096),
                                                  ("e4m3", "max", 0, 1, 13)])
def test_delayed_scaling_sequence(fmt, algo, margin, L, n):
    f = oracle.format_by_name(fmt)
    state = te().DelayedScaling(fmt, L, algo, margin)
    h = np.zeros(L, np.float32)
    s = np.float32(1.0)
    for step, sigma in enumerate(SIGMAS):
        bits = workloads.normal_bf16(95, step, (n,), sigma, 0.0) if sigma > 0 else np.zeros(n, np.uint16)
        q, q_inv = state.step(dev(bits))
        torch.cuda.synchronize()
        oq, oq_inv, a, h, s = oracle.delayed_scaling_step(bits, f, h, s, algo, margin)
        assert host(q_inv)[0] == oq_inv, f"step {step}: q_scale_inv"
        assert np.array_equal(host(state.history), h), f"step {step}: history"
        assert host(state.scale)[0] == s, f"step {step}: next scale"
        assert np.array_equal(host(q), oq), f"step {step}: codes"


def per_tensor_operands(M, N, K, seed, fa="e4m3", fb="e4m3"):
    """Delayed-scaling casts (one step each, from scale 1 after a warm-up step) of an activation and a weight."""
    out = []
    for t, (rows, sigma, fmt) in enumerate([(M, 1.0, fa), (N, 0.05, fb)]):
        st = te().DelayedScaling(fmt, 16, "max", 0)
        warm = workloads.normal_bf16(seed, 10 + t, (rows, K), sigma, 0.01)
        st.step(dev(warm))   # the warm-up step gives a data-derived scale
        bits = workloads.normal_bf16(seed, t, (rows, K), sigma, 0.01)
        q, q_inv = st.step(dev(bits))
        out += [q, q_inv]
    return out


@pytest.mark.parametrize("epi", ["none", "bias", "bias_gelu_aux"])
@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (272, 400, 256), (1040, 784, 640), (4096 + 48, 4096 + 80, 256),
                                   (272, 400, 2176), (4096 + 48, 4096 + 80, 2048), (4096 - 48, 3072 - 80, 1024)])
def test_per_tensor_gemm(epi, M, N, K):
    qa, ia, qb, ib = per_tensor_operands(M, N, K, 96 + K)
    bias_bits = None if epi == "none" else workloads.normal_bf16(97, N, (N,), 0.5)
    d, aux = te().fp8_gemm(qa, ia, "e4m3", qb, ib, "e4m3", epi, None if bias_bits is None else dev(bias_bits))
    torch.cuda.synchronize()
    big = M > 2048
    rows = np.unique(np.r_[0, M - 1, np.linspace(0, M - 1, 48).astype(int)]) if big else np.arange(M)
    cols = np.unique(np.r_[0, N - 1, np.linspace(0, N - 1, 48).astype(int)]) if big else np.arange(N)
    hqa, hqb = host(qa)[rows], host(qb)[cols]
    a_inv, b_inv = host(ia)[0], host(ib)[0]
    b = None if bias_bits is None else bias_bits[cols]
    # the MFMA model with unit block scales, then the kernel's fp32 alpha
    ones_a = np.full((len(rows), K // 32), 127, np.uint8)
    ones_b = np.full((len(cols), K // 32), 127, np.uint8)
    acc = mfma_model.hw_gemm_fp32(hqa, ones_a, oracle.E4M3, hqb, ones_b, oracle.E4M3)
    alpha = np.float32(a_inv * b_inv)
    acc = (acc * alpha).astype(np.float32)
    want_d, want_aux = model_outputs(acc, b, epi)
    got_bits = host(d)[rows][:, cols]
    if epi == "bias_gelu_aux":
        assert np.array_equal(host(aux)[rows][:, cols], want_aux)
        g = bf16_to_f64(got_bits)
        assert np.all(np.abs(g - want_d) <= 2.0 ** -8 * np.abs(want_d) + 1e-30)
    else:
        assert np.array_equal(got_bits, want_d), "D differs from the MFMA model"
    # the oracle, within the GEMM bound (S already carries |alpha|)
    ref, ref_aux, s = oracle.fp8_gemm_per_tensor(hqa, a_inv, oracle.E4M3, hqb, b_inv, oracle.E4M3, b, epi)

    def h_pairs(ri, ci):
        return float(alpha) * mfma_model.truncation_bound_pairs(hqa, ones_a, oracle.E4M3, hqb, ones_b, oracle.E4M3,
                                                                ri, ci)
    ok, stated = gemm_check(bf16_to_f64(got_bits), ref, s, b, K, h_pairs, through_gelu=epi == "bias_gelu_aux")
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside the bound"
    assert_stated_misses(f"per_tensor:{M}x{N}x{K}:{epi}", int((~stated).sum()), stated.size)


@pytest.mark.parametrize("fa,fb", [("e5m2", "e4m3"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("M,N,K", [(1040, 784, 640), (4096 + 48, 4096 + 80, 256), (4096 + 48, 4096 + 80, 2048)])
def test_per_tensor_gemm_e5m2_operand(fa, fb, M, N, K):
    # HYBRID per-tensor operands (an E5M2 gradient times E4M3, either side) on the small, 8-wave and
    # 4-wave tiles: D bit-exact against the MFMA model with unit block scales and the fp32 alpha
    qa, ia, qb, ib = per_tensor_operands(M, N, K, 131 + K, fa, fb)
    bias_bits = workloads.normal_bf16(132, N, (N,), 0.5)
    d, _ = te().fp8_gemm(qa, ia, fa, qb, ib, fb, "bias", dev(bias_bits))
    torch.cuda.synchronize()
    big = M > 2048
    rows = np.unique(np.r_[0, M - 1, np.linspace(0, M - 1, 48).astype(int)]) if big else np.arange(M)
    cols = np.unique(np.r_[0, N - 1, np.linspace(0, N - 1, 48).astype(int)]) if big else np.arange(N)
    hqa, hqb = host(qa)[rows], host(qb)[cols]
    ones_a = np.full((len(rows), K // 32), 127, np.uint8)
    ones_b = np.full((len(cols), K // 32), 127, np.uint8)
    acc = mfma_model.hw_gemm_fp32(hqa, ones_a, oracle.format_by_name(fa), hqb, ones_b, oracle.format_by_name(fb))
    alpha = np.float32(host(ia)[0] * host(ib)[0])
    want_d, _ = model_outputs((acc * alpha).astype(np.float32), bias_bits[cols], "bias")
    assert np.array_equal(host(d)[rows][:, cols], want_d), "D differs from the MFMA model"


@pytest.mark.parametrize("M,N,K", [(272, 304, 512), (4096 + 48, 4096 + 80, 2048)])
def test_per_tensor_gemm_fp32_output(M, N, K):
    # (4144, 4176, 2048) runs the 4-wave big tile, which applies alpha inside its epilogue
    qa, ia, qb, ib = per_tensor_operands(M, N, K, 98)
    d, _ = te().fp8_gemm(qa, ia, "e4m3", qb, ib, "e4m3", out_dtype=torch.float32)
    torch.cuda.synchronize()
    big = M > 2048
    rows = np.unique(np.r_[0, M - 1, np.linspace(0, M - 1, 40).astype(int)]) if big else np.arange(M)
    cols = np.unique(np.r_[0, N - 1, np.linspace(0, N - 1, 40).astype(int)]) if big else np.arange(N)
    ones_a = np.full((len(rows), K // 32), 127, np.uint8)
    ones_b = np.full((len(cols), K // 32), 127, np.uint8)
    acc = mfma_model.hw_gemm_fp32(host(qa)[rows], ones_a, oracle.E4M3, host(qb)[cols], ones_b, oracle.E4M3)
    alpha = np.float32(host(ia)[0] * host(ib)[0])
    assert np.array_equal(host(d)[rows][:, cols], (acc * alpha).astype(np.float32))
