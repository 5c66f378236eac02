"""Seeded synthetic inputs for the MXFP8 Linear hot path.

This module only draws random inputs; it holds none of the method's
arithmetic.  It is shared by the GPU tests, ``bench.py`` and the oracle
checks (the oracle itself never imports it; tests pass its arrays to both
sides).

Recipe (no dataset is involved: the pages measure nothing on a public
benchmark, so every input is synthetic):
* ``rng = numpy.random.default_rng([cfg_id, tensor_id])``;
* float32 draws ``standard_normal * sigma`` (sigma is the standard
  deviation);
* "1% outlier columns x20": ``round(0.01 * K)`` distinct columns of the K
  axis, chosen by the same rng, multiplied by 20 in float32;
* conversion to bf16 by round-to-nearest-even (torch's CPU cast);
* tensors are returned as uint16 bf16 bit patterns, row-major; weights are
  [N, K] (out x in), activations [tokens, K].
* MoE routing: ``default_rng([5, 0]).multinomial(16384, [1/32] * 32)``.

The shapes follow the transformer layer sizes the pages use (batch 32 x
sequence 128 tokens with hidden 1024 in the ROCm README's Flax example; an
FFN of hidden 4096 in the JAX quickstart) and the large square and MoE
shapes of the benchmark configurations.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def normal_bf16(cfg_id: int, tensor_id: int, shape, sigma: float, outlier_frac: float = 0.0) -> np.ndarray:
    """Seeded N(0, sigma) tensor as bf16 bit patterns (uint16), with optional
    outlier columns along the last axis scaled by 20."""
    rng = np.random.default_rng([cfg_id, tensor_id])
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    x *= np.float32(sigma)
    if outlier_frac > 0:
        k = shape[-1]
        n_out = int(round(outlier_frac * k))
        cols = rng.choice(k, n_out, replace=False)
        x[..., cols] *= np.float32(20.0)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def moe_counts(total: int = 16384, experts: int = 32, seed=(5, 0)) -> np.ndarray:
    rng = np.random.default_rng(list(seed))
    return rng.multinomial(total, [1.0 / experts] * experts).astype(np.int32)


@dataclass(frozen=True)
class TensorSpec:
    cfg_id: int
    tensor_id: int
    shape: tuple
    sigma: float
    outlier_frac: float = 0.0

    def make(self) -> np.ndarray:
        return normal_bf16(self.cfg_id, self.tensor_id, self.shape, self.sigma, self.outlier_frac)


@dataclass(frozen=True)
class GemmSpec:
    """One TN GEMM D[M,N] = A[M,K] . B[N,K]^T with MXFP8 operands.

    ``a_src``/``b_src`` give the bf16 source tensors and how they are
    quantized: "row" quantizes the given [rows, K] tensor along K; "col"
    quantizes a [K, rows] tensor down its columns (the transposed copy).
    """
    name: str
    M: int
    N: int
    K: int
    fmt_a: str
    fmt_b: str
    epilogue: str
    a_src: TensorSpec
    b_src: TensorSpec
    a_dir: str = "row"
    b_dir: str = "row"
    bias: TensorSpec | None = None
    mx_out: bool = False        # D written as a rowwise MXFP8 operand (fmt_a of the consumer) instead of bf16
    # "mx": MXFP8 operands; "delayed": per-tensor FP8 cast with delayed scaling;
    # "block_e8m0" / "block_fp32": blockwise FP8 (A in 1 x 128 blocks, B in
    # 128 x 128 blocks), the GEMM taking the scales cast to E8M0 or as FP32
    scaling: str = "mx"
    a_from: str | None = None   # A is the MXFP8 output of this earlier GEMM (a_src is then unused)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclass(frozen=True)
class GroupedSpec:
    name: str
    experts: int
    total_m: int
    N: int
    K: int
    fmt_a: str
    fmt_b: str
    epilogue: str
    a_src: TensorSpec
    b_src: TensorSpec          # [experts * N, K]
    bias: TensorSpec | None    # [experts, N]


@dataclass
class Workload:
    name: str
    gemms: list = field(default_factory=list)
    grouped: list = field(default_factory=list)
    quantize: list = field(default_factory=list)     # (TensorSpec, fmt, dir) standalone quantizes
    current_scaling: list = field(default_factory=list)  # (TensorSpec, fmt)
    # (TensorSpec, fmt): both MXFP8 copies and the column sums (bias gradient)
    # in one pass; the GEMMs that take this tensor use those copies
    fused_bgrad: list = field(default_factory=list)


def tiny() -> Workload:
    """M = N = K = 256, bf16 N(0,1), E4M3 rowwise, no epilogue."""
    return Workload("tiny_256", gemms=[GemmSpec(
        "tiny", 256, 256, 256, "e4m3", "e4m3", "none",
        TensorSpec(1, 0, (256, 256), 1.0), TensorSpec(1, 1, (256, 256), 1.0))])


def decoder_forward() -> Workload:
    """4096 tokens (batch 32 x seq 128), hidden 1024: QKV, FC1 (+GELU aux), FC2."""
    T, H, F = 4096, 1024, 4096
    return Workload("decoder_fwd_4096x1024", gemms=[
        GemmSpec("qkv", T, 3 * H, H, "e4m3", "e4m3", "bias",
                 TensorSpec(2, 0, (T, H), 1.0, 0.01), TensorSpec(2, 1, (3 * H, H), 0.02),
                 bias=TensorSpec(2, 2, (3 * H,), 0.02)),
        GemmSpec("fc1", T, F, H, "e4m3", "e4m3", "bias_gelu_aux",
                 TensorSpec(2, 3, (T, H), 1.0, 0.01), TensorSpec(2, 4, (F, H), 0.02),
                 bias=TensorSpec(2, 5, (F,), 0.02)),
        GemmSpec("fc2", T, H, F, "e4m3", "e4m3", "bias",
                 TensorSpec(2, 6, (T, F), 1.0, 0.01), TensorSpec(2, 7, (H, F), 0.02),
                 bias=TensorSpec(2, 8, (H,), 0.02)),
    ])


def decoder_forward_mx() -> Workload:
    """The decoder forward with FC1 -> FC2 chained: FC1's GELU output is written
    as FC2's rowwise MXFP8 operand by FC1's epilogue (no bf16 D, no separate
    quantize of FC2's input)."""
    T, H, F = 4096, 1024, 4096
    base = {g.name: g for g in decoder_forward().gemms}
    fc1, fc2 = base["fc1"], base["fc2"]
    return Workload("decoder_fwd_mx_4096x1024", gemms=[
        base["qkv"],
        GemmSpec("fc1", T, F, H, "e4m3", "e4m3", "bias_gelu_aux", fc1.a_src, fc1.b_src, bias=fc1.bias, mx_out=True),
        GemmSpec("fc2", T, H, F, "e4m3", "e4m3", "bias", fc2.a_src, fc2.b_src, bias=fc2.bias, a_from="fc1"),
    ])


def decoder_forward_delayed() -> Workload:
    """The decoder forward with the other recipe: per-tensor FP8 operands cast
    with delayed scaling (amax history 16, "max", margin 0) and per-tensor
    FP8 GEMMs."""
    from dataclasses import replace
    return Workload("decoder_fwd_delayed_4096x1024",
                    gemms=[replace(g, scaling="delayed") for g in decoder_forward().gemms])


def large_square() -> Workload:
    """M = N = K = 8192 fprop, 1% outlier K-columns on both operands, plus
    standalone rowwise and columnwise quantization of both inputs."""
    n = 8192
    a = TensorSpec(3, 0, (n, n), 1.0, 0.01)
    b = TensorSpec(3, 1, (n, n), 1.0, 0.01)
    return Workload("square_8192", gemms=[GemmSpec("fprop", n, n, n, "e4m3", "e4m3", "none", a, b)],
                    quantize=[(a, "e4m3", "row"), (a, "e4m3", "col"), (b, "e4m3", "row"), (b, "e4m3", "col")])


def block_square(mode: str = "e8m0") -> Workload:
    """M = N = K = 8192 with the blockwise FP8 recipe on the operands of
    square_8192: A quantized in 1 x 128 blocks, B in 128 x 128 blocks
    (power-of-two FP32 scales), then the 1-D x 2-D blockwise GEMM with the
    scales cast to E8M0 (mode "e8m0") or applied as FP32 ("fp32")."""
    n = 8192
    g = large_square().gemms[0]
    return Workload(f"block_{mode}_square_8192", gemms=[GemmSpec("fprop", n, n, n, "e4m3", "e4m3", "none",
                                                                 g.a_src, g.b_src, scaling=f"block_{mode}")])


def hybrid_backward() -> Workload:
    """FFN backward, 4096 tokens, hidden 4096, ffn 14336, HYBRID formats.

    dgrad: dY [4096, 14336] (E5M2, rowwise) x W1 [14336, 4096] quantized
    columnwise -> [4096, 14336] (E4M3): M=4096, N=4096, K=14336.
    wgrad: dY^T (dY quantized columnwise -> [14336, 4096], E5M2) x X^T
    (X [4096, 4096] quantized columnwise, E4M3): M=14336, N=4096, K=4096.
    Plus a per-tensor current-scaling E4M3 cast of X.
    """
    T, H, F = 4096, 4096, 14336
    dy = TensorSpec(4, 0, (T, F), 1e-3)
    w1 = TensorSpec(4, 1, (F, H), 0.02)
    x = TensorSpec(4, 2, (T, H), 1.0)
    return Workload("hybrid_bwd_4096x4096x14336", gemms=[
        GemmSpec("dgrad", T, H, F, "e5m2", "e4m3", "none", dy, w1, a_dir="row", b_dir="col"),
        GemmSpec("wgrad", F, H, T, "e5m2", "e4m3", "none", dy, x, a_dir="col", b_dir="col"),
    ], current_scaling=[(x, "e4m3")])


def hybrid_backward_fused() -> Workload:
    """The same FFN backward, with dY's rowwise and columnwise quantization
    done in one cast-transpose pass that also reduces dY into the bias
    gradient db[f] = sum_t dY[t, f] (fp32)."""
    w = hybrid_backward()
    dy = w.gemms[0].a_src
    return Workload("hybrid_bwd_fused_4096x4096x14336", gemms=w.gemms, current_scaling=w.current_scaling,
                    fused_bgrad=[(dy, "e5m2")])


def moe_grouped() -> Workload:
    """32 experts, hidden 4096 -> expert ffn 1536, bias + GELU aux, 16384 routed tokens."""
    E, T, N, K = 32, 16384, 1536, 4096
    return Workload("moe_grouped_32x1536x4096", grouped=[GroupedSpec(
        "moe_fc1", E, T, N, K, "e4m3", "e4m3", "bias_gelu_aux",
        TensorSpec(5, 1, (T, K), 1.0), TensorSpec(5, 2, (E * N, K), 0.02), TensorSpec(5, 3, (E, N), 0.02))])


ALL = {"tiny": tiny, "decoder_fwd": decoder_forward, "decoder_fwd_mx": decoder_forward_mx,
       "decoder_fwd_delayed": decoder_forward_delayed, "square_8192": large_square,
       "block_e8m0_square_8192": lambda: block_square("e8m0"), "block_fp32_square_8192": lambda: block_square("fp32"),
       "hybrid_bwd": hybrid_backward, "hybrid_bwd_fused": hybrid_backward_fused, "moe_grouped": moe_grouped}
