"""GPU parity of the blockwise FP8 GEMM (both scale modes) and of the cast of
FP32 block scales to MXFP8 E8M0 scales, against the CPU oracle.

* Scale cast: bit-exact against oracle.e8m0_of on every kind of FP32 value
  (powers of two, values just above and below them, subnormals, zeros,
  infinities, NaN, negatives), 1-D and 2-D blocks, ragged rows.
* Exact-integer GEMMs (every partial sum and every scaled term is exact in
  fp32, so any order of summation gives the same fp32 result): bit-exact
  against oracle.block_gemm, for 1-D x 1-D and 1-D x 2-D, every format
  pair, both tiles, ragged M and N.  E8M0 mode is checked against the oracle
  on the scales cast to powers of two, FP32 mode on the FP32 scales.
* Recipe data (normal bf16 inputs quantized by the oracle's 1-D / 2-D
  blockwise quantizers; power-of-two scales, and the same codes with
  non-power-of-two FP32 scales): within the GEMM tolerance
  |y - y_ref| <= 2^-8 |y_ref| + 1e-5 S + H + (K'/16) 2^-24 S, where H
  bounds the MFMA's in-group truncation on the E8M0-cast scales (>= the
  FP32 scales, so the bound covers FP32 mode) and K' = 1.25 K in FP32 mode
  (its per-block product and fma add K/64 roundings).
* Epilogues: with power-of-two scales and exact data both modes form the
  same fp32 accumulators, so every epilogue output of FP32 mode equals
  E8M0 mode's bit for bit; bias and GELU-aux outputs of both modes on
  recipe data against the oracle's epilogue within the GEMM bound (GELU
  outputs with the GELU slope), aux bit-identical to the bias epilogue's D.
* The bench workload's GEMM at full size, sampled rows x columns.
* fp16 D: exact-integer data bit-exact against the half rounding of the
  oracle's result (both tiles), overflow to infinity past the half range,
  and the bias / GELU-aux epilogues on recipe data within the GEMM bound.
* beta: the accumulate epilogue D = fl32(beta C + acc), bit-exact against
  the oracle's beta C + Y on exact data for beta = -0.75, 0 and 2, and
  within the GEMM bound on recipe data for beta = 0.3.
"""

import numpy as np
import pytest
import torch

import mfma_model
import oracle
import workloads
from gpu_util import assert_stated_misses, bf16_rne, bf16_to_f64, dev, gemm_check, host

pytestmark = pytest.mark.gpu

MODES = ["e8m0", "fp32"]


def te():
    import mxfp8_mixed_precision_amd as m
    return m


def special_scales(rng, shape):
    """FP32 scales mixing every case of the E8M0 cast."""
    n = int(np.prod(shape))
    k = rng.integers(-149, 128, size=n).astype(np.float64)
    pow2 = np.ldexp(1.0, k.astype(np.int64))
    kinds = rng.integers(0, 6, size=n)
    f32 = np.float32
    v = np.where(kinds == 0, pow2, 0.0)
    v = np.where(kinds == 1, pow2 * rng.uniform(1.0, 2.0, n), v)            # between powers of two
    v = np.where(kinds == 2, pow2 * (1 + 2.0 ** -23), v)                    # just above a power of two
    v = np.where(kinds == 3, pow2 * (1 - 2.0 ** -24), v)                    # just below
    v = np.where(kinds == 4, rng.uniform(0, 1, n) * 2.0 ** -126, v)         # subnormal range
    v = np.where(kinds == 5, rng.choice([0.0, -0.0, np.inf, -np.inf, np.nan, -1.5, 3.4e38, 2.0 ** -149], n), v)
    with np.errstate(over="ignore"):
        return v.astype(f32).reshape(shape)


@pytest.mark.parametrize("block_2d", [False, True])
def test_scale_cast_matches_oracle(block_2d):
    rng = np.random.default_rng(41 + block_2d)
    rows, cols = 300, 1024
    srows = -(-rows // 128) if block_2d else rows
    s = special_scales(rng, (srows, cols // 128))
    got = host(te().fp8_block_scales_to_mx(dev(s), rows, cols, block_2d))
    torch.cuda.synchronize()
    want = np.repeat(oracle.e8m0_of(s), 4, axis=1)
    if block_2d:
        want = np.repeat(want, 128, axis=0)[:rows]
    assert got.shape == (rows, cols // 32)
    assert np.array_equal(got, want)


def exact_codes(rng, shape, fmt):
    """Codes of values in {0, +-0.5, +-1, +-2}."""
    table = {"e4m3": [0x00, 0x30, 0x38, 0x40], "e5m2": [0x00, 0x38, 0x3C, 0x40]}[fmt]
    c = np.array(table, np.uint8)[rng.integers(0, 4, size=shape)]
    return c | (rng.integers(0, 2, size=shape) * 0x80).astype(np.uint8)


def exact_scales(rng, shape):
    """{3, 4, 5, 6} / 4 * 2^{-1, 0, 1}: every product of two is exact, and so is every scaled block sum."""
    m = np.array([0.75, 1.0, 1.25, 1.5])[rng.integers(0, 4, size=shape)]
    return (m * np.ldexp(1.0, rng.integers(-1, 2, size=shape))).astype(np.float32)


def b_scale_shape(N, K, b_2d):
    return (-(-N // 128) if b_2d else N, K // 128)


def run(mode, qa, sa, fa, qb, sb, fb, b_2d, epi="none", bias=None, out_dtype=torch.float32, aux=None, out=None,
        beta=1.0):
    d, aux_out = te().fp8_block_gemm(dev(qa), dev(sa), fa, dev(qb), dev(sb), fb, b_2d, epi,
                                     None if bias is None else dev(bias), out_dtype,
                                     None if aux is None else dev(aux), out, mode, beta=beta)
    torch.cuda.synchronize()
    return d, aux_out


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b_2d", [False, True])
@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (272, 304, 384), (16, 16, 1024), (8192, 4112, 512),
                                   (272, 304, 2176)])
def test_block_gemm_exact_bitexact(mode, b_2d, fa, fb, M, N, K):
    rng = np.random.default_rng([M, N, K, b_2d])
    qa, qb = exact_codes(rng, (M, K), fa), exact_codes(rng, (N, K), fb)
    sa, sb = exact_scales(rng, (M, K // 128)), exact_scales(rng, b_scale_shape(N, K, b_2d))
    d, _ = run(mode, qa, sa, fa, qb, sb, fb, b_2d)
    if mode == "e8m0":
        sa_ref, sb_ref = oracle.pow2_at_least(sa), oracle.pow2_at_least(sb)
    else:
        sa_ref, sb_ref = sa, sb
    rows = np.arange(M)
    if M * N > 1 << 22 and (fa, fb) != ("e4m3", "e4m3"):
        # the big-tile shape with an E5M2 operand: every 256-row tile boundary, the last row and random rows
        # (exact-integer data, so each sampled fp32 output must match bit for bit)
        rows = np.array(sorted({0, M - 1} | {256 * t + o for t in range(M // 256) for o in (0, 255)}
                               | set(rng.choice(M, 16, replace=False).tolist())))
    ref, _, _ = oracle.block_gemm(qa[rows], sa_ref[rows], oracle.format_by_name(fa), qb, sb_ref,
                                  oracle.format_by_name(fb), b_2d)
    assert np.array_equal(host(d[rows]).astype(np.float64), ref)


def test_block_gemm_k_zero_and_empty():
    for mode in MODES:
        e = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
        s = torch.zeros((64, 0), dtype=torch.float32, device="cuda")
        bias = workloads.normal_bf16(6, 2, (48,), 1.0)
        d, _ = te().fp8_block_gemm(e, s, "e4m3", e[:48], s[:1], "e4m3", True, "bias", dev(bias),
                                   torch.float32, mode=mode)
        torch.cuda.synchronize()
        assert np.array_equal(host(d), np.broadcast_to(bf16_to_f64(bias).astype(np.float32), (64, 48)))
        z = torch.zeros((0, 256), dtype=torch.uint8, device="cuda")
        d, _ = te().fp8_block_gemm(z, torch.zeros((0, 2), device="cuda"), "e4m3", z, torch.zeros((0, 2), device="cuda"),
                                   "e4m3", False, mode=mode)
        assert d.shape == (0, 0)


def recipe_operands(M, N, K, b_2d, seed, fa="e4m3", fb="e4m3"):
    x = workloads.normal_bf16(seed, 0, (M, K), 1.0, outlier_frac=0.01)
    w = workloads.normal_bf16(seed, 1, (N, K), 0.02)
    qa, sa = oracle.quantize_1d(x, oracle.format_by_name(fa))
    qb, sb = (oracle.quantize_2d if b_2d else oracle.quantize_1d)(w, oracle.format_by_name(fb))
    return qa, sa, qb, sb


def e8m0_expanded(s, rows, b_2d):
    c = np.repeat(oracle.e8m0_of(s), 4, axis=1)
    return np.repeat(c, 128, axis=0)[:rows] if b_2d else c


def check_recipe(key, mode, qa, sa, fa, qb, sb, fb, b_2d, rows, cols, d, bias=None, epi="none"):
    """Sampled (or full) outputs against the oracle within the GEMM bound."""
    K = qa.shape[1]
    Fa, Fb = oracle.format_by_name(fa), oracle.format_by_name(fb)
    sa_ref = oracle.pow2_at_least(sa) if mode == "e8m0" else sa
    sb_ref = oracle.pow2_at_least(sb) if mode == "e8m0" else sb
    sb_rows = sb_ref if not b_2d else np.repeat(sb_ref, 128, axis=0)[: qb.shape[0]]
    ref, _, s = oracle.block_gemm(qa[rows], sa_ref[rows], Fa, qb[cols], sb_rows[cols], Fb, False,
                                  None if bias is None else bias[cols], epi)
    ea, eb = e8m0_expanded(sa, qa.shape[0], False), e8m0_expanded(sb, qb.shape[0], b_2d)

    def h_pairs(ri, ci):
        return mfma_model.truncation_bound_pairs(qa[rows], ea[rows], Fa, qb[cols], eb[cols], Fb, ri, ci)

    got = host(d[rows][:, cols]).astype(np.float64) if d.dtype == torch.float32 else bf16_to_f64(
        host(d[rows][:, cols]))
    k_eff = K * 1.25 if mode == "fp32" else K
    ok, stated = gemm_check(got, ref, s, None if bias is None else bias[cols], k_eff, h_pairs,
                            through_gelu=epi == "bias_gelu_aux")
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside the bound"
    assert_stated_misses(f"{key}:{mode}:{epi}", int((~stated).sum()), stated.size)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b_2d", [False, True])
def test_block_gemm_recipe_full(mode, b_2d):
    M, N, K = 512, 656, 2048
    qa, sa, qb, sb = recipe_operands(M, N, K, b_2d, seed=51)
    d, _ = run(mode, qa, sa, "e4m3", qb, sb, "e4m3", b_2d, out_dtype=torch.bfloat16)
    check_recipe(f"block_recipe:{'2d' if b_2d else '1d'}", mode, qa, sa, "e4m3", qb, sb, "e4m3", b_2d, np.arange(M),
                 np.arange(N), d)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b_2d", [False, True])
def test_block_gemm_fp32_scales_not_powers_of_two(mode, b_2d):
    """The recipe's codes with scales multiplied by factors in [1, 2): FP32 mode uses them as they are,
    E8M0 mode rounds each up to a power of two."""
    M, N, K = 384, 400, 1536
    qa, sa, qb, sb = recipe_operands(M, N, K, b_2d, seed=52, fa="e5m2", fb="e4m3")
    rng = np.random.default_rng(53)
    sa = (sa * rng.uniform(1.0, 2.0, sa.shape)).astype(np.float32)
    sb = (sb * rng.uniform(1.0, 2.0, sb.shape)).astype(np.float32)
    d, _ = run(mode, qa, sa, "e5m2", qb, sb, "e4m3", b_2d)
    check_recipe(f"block_nonpow2:{'2d' if b_2d else '1d'}", mode, qa, sa, "e5m2", qb, sb, "e4m3", b_2d, np.arange(M),
                 np.arange(N), d)


@pytest.mark.parametrize("b_2d", [False, True])
@pytest.mark.parametrize("epi", ["none", "bias", "bias_gelu_aux", "dgelu", "accumulate"])
def test_fp32_mode_epilogues_equal_e8m0_mode(b_2d, epi):
    M, N, K = 1024, 784, 640
    rng = np.random.default_rng([61, b_2d])
    qa, qb = exact_codes(rng, (M, K), "e4m3"), exact_codes(rng, (N, K), "e5m2")
    sa = np.ldexp(1.0, rng.integers(-2, 3, (M, K // 128))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-2, 3, b_scale_shape(N, K, b_2d))).astype(np.float32)
    bias = workloads.normal_bf16(61, 3, (N,), 2.0) if epi in ("bias", "bias_gelu_aux") else None
    aux = workloads.normal_bf16(61, 4, (M, N), 2.0) if epi == "dgelu" else None
    outs = {}
    for mode in MODES:
        out = None
        out_dtype = torch.bfloat16
        if epi == "accumulate":
            out = dev(workloads.normal_bf16(61, 5, (M, N), 100.0)).view(torch.bfloat16).float()
            out_dtype = torch.float32
        d, aux_out = run(mode, qa, sa, "e4m3", qb, sb, "e5m2", b_2d, epi, bias, out_dtype, aux, out)
        outs[mode] = (host(d), None if aux_out is None else host(aux_out))
    assert np.array_equal(outs["e8m0"][0], outs["fp32"][0])
    if epi == "bias_gelu_aux":
        assert np.array_equal(outs["e8m0"][1], outs["fp32"][1])
    if epi == "none":  # exact accumulators: bf16 of the oracle's exact result
        ref, _, _ = oracle.block_gemm(qa, sa, oracle.E4M3, qb, sb, oracle.E5M2, b_2d)
        assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
        assert np.array_equal(outs["fp32"][0], bf16_rne(ref))


@pytest.mark.parametrize("mode", MODES)
def test_block_square_full_size_sampled(mode):
    """The bench workload (8192^3, A in 1 x 128 blocks, B in 128 x 128 blocks) through the device quantizer
    and the GEMM as bench.py launches them; sampled rows of A and columns in six 128-row blocks of B
    (first, last, across a 256-column tile boundary, random) against the oracle."""
    g = workloads.block_square(mode).gemms[0]
    a_bits, b_bits = g.a_src.make(), g.b_src.make()
    m = te()
    qa, sa = m.fp8_block_quantize(dev(a_bits), g.fmt_a, block_2d=False)
    qb, sb = m.fp8_block_quantize(dev(b_bits), g.fmt_b, block_2d=True)
    ws_bytes = m.te_fp8_block_gemm_workspace_size(g.M, g.N, g.K, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    d = torch.empty((g.M, g.N), dtype=torch.bfloat16, device="cuda")
    m.te_fp8_block_gemm(qa, sa, g.fmt_a, qb, sb, g.fmt_b, True, d, g.epilogue, None, None, mode, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(81)
    rows = np.array(sorted({0, 255, 256, g.M - 1} | set(rng.choice(g.M, 60, replace=False).tolist())))
    slabs = sorted({0, 1, 2, g.N // 128 - 1} | set(rng.choice(g.N // 128, 2, replace=False).tolist()))
    Fa, Fb = oracle.format_by_name(g.fmt_a), oracle.format_by_name(g.fmt_b)
    oqa, osa = oracle.quantize_1d(a_bits[rows], Fa)
    assert np.array_equal(host(qa[rows]), oqa) and np.array_equal(host(sa[rows]), osa)
    cols, oqb, osb = [], [], []
    for sl in slabs:
        q2, s2 = oracle.quantize_2d(b_bits[128 * sl:128 * (sl + 1)], Fb)
        assert np.array_equal(host(qb[128 * sl:128 * (sl + 1)]), q2) and np.array_equal(host(sb[sl:sl + 1]), s2)
        pick = sorted({0, 127} | set(rng.choice(128, 14, replace=False).tolist()))
        cols += [128 * sl + p for p in pick]
        oqb.append(q2[pick])
        osb.append(np.repeat(s2, len(pick), axis=0))
    cols = np.array(cols)
    # B rows sampled as 1-D rows carrying their block's scale row
    sub_qb, sub_sb = np.concatenate(oqb), np.concatenate(osb)
    full_qb = np.zeros((g.N, g.K), np.uint8)
    full_sb = np.ones((g.N, g.K // 128), np.float32)
    full_qb[cols], full_sb[cols] = sub_qb, sub_sb
    full_qa = np.zeros((g.M, g.K), np.uint8)
    full_sa = np.ones((g.M, g.K // 128), np.float32)
    full_qa[rows], full_sa[rows] = oqa, osa
    check_recipe("block_square_8192", mode, full_qa, full_sa, g.fmt_a, full_qb, full_sb, g.fmt_b, False, rows, cols, d)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("epi", ["bias", "bias_gelu_aux"])
def test_block_gemm_forward_epilogues_vs_oracle(mode, epi):
    """Bias and GELU-aux epilogues on recipe data (1-D x 2-D) against the oracle's epilogue of the blockwise
    product: D (through GELU where it applies) and aux within the GEMM bound."""
    M, N, K = 400, 528, 2176
    qa, sa, qb, sb = recipe_operands(M, N, K, True, seed=91)
    bias = workloads.normal_bf16(91, 5, (N,), 0.5)
    d, aux = run(mode, qa, sa, "e4m3", qb, sb, "e4m3", True, epi, bias, torch.bfloat16)
    check_recipe("block_epilogue", mode, qa, sa, "e4m3", qb, sb, "e4m3", True, np.arange(M), np.arange(N), d, bias, epi)
    if epi == "bias_gelu_aux":
        # aux is the bf16 pre-activation: the bias epilogue's D for the same inputs, bit for bit
        d_bias, _ = run(mode, qa, sa, "e4m3", qb, sb, "e4m3", True, "bias", bias, torch.bfloat16)
        assert torch.equal(aux, d_bias)


# ------------------------------------------------------------ fp16 output and beta

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b_2d", [False, True])
@pytest.mark.parametrize("M,N,K", [(272, 304, 384), (8192, 4112, 512)])
def test_block_gemm_fp16_output_exact(mode, b_2d, M, N, K):
    """Exact-integer data: every fp32 accumulator is exact, so the fp16 D must be the round-to-nearest-even
    half of the oracle's result, bit for bit (both tiles; sampled tile-boundary rows on the big one)."""
    rng = np.random.default_rng([M, N, K, b_2d, 16])
    qa, qb = exact_codes(rng, (M, K), "e4m3"), exact_codes(rng, (N, K), "e5m2")
    sa, sb = exact_scales(rng, (M, K // 128)), exact_scales(rng, b_scale_shape(N, K, b_2d))
    d, _ = run(mode, qa, sa, "e4m3", qb, sb, "e5m2", b_2d, out_dtype=torch.float16)
    sa_ref, sb_ref = (oracle.pow2_at_least(sa), oracle.pow2_at_least(sb)) if mode == "e8m0" else (sa, sb)
    rows = np.arange(M)
    if M > 2048:
        rows = np.array(sorted({0, M - 1} | {256 * t + o for t in range(M // 256) for o in (0, 255)}))
    ref, _, _ = oracle.block_gemm(qa[rows], sa_ref[rows], oracle.E4M3, qb, sb_ref, oracle.E5M2, b_2d)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)   # exact in fp32
    got = d[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("mode", MODES)
def test_block_gemm_fp16_output_overflows_to_inf(mode):
    """Outputs beyond the half range become +-inf (scales of 2^9 make |D| reach ~2^17); the rest round as usual."""
    M, N, K = 272, 304, 384
    rng = np.random.default_rng(17)
    # non-negative codes on A, so the sums grow; rows alternate between scales 2^9 (overflow) and 2^-4
    qa, qb = exact_codes(rng, (M, K), "e4m3") & 0x7F, exact_codes(rng, (N, K), "e4m3")
    qb[: N // 2] &= 0x7F
    sa = np.full((M, K // 128), 512.0, np.float32)
    sa[1::2] = 2.0 ** -4
    sb = np.ones((N, K // 128), np.float32)
    d, _ = run(mode, qa, sa, "e4m3", qb, sb, "e4m3", False, out_dtype=torch.float16)
    ref, _, _ = oracle.block_gemm(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, False)
    with np.errstate(over="ignore"):
        want = ref.astype(np.float16)
    assert np.isinf(want).any() and np.isfinite(want).any()
    assert np.array_equal(d.view(torch.int16).cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("epi", ["bias", "bias_gelu_aux"])
def test_block_gemm_fp16_output_recipe(mode, epi):
    """Recipe data through the bias and GELU-aux epilogues with fp16 D, against the oracle within the GEMM bound;
    aux (bf16) equals the bf16-output run's bit for bit."""
    M, N, K = 400, 528, 2176
    qa, sa, qb, sb = recipe_operands(M, N, K, True, seed=92)
    bias = workloads.normal_bf16(92, 5, (N,), 0.5)
    d, aux = run(mode, qa, sa, "e4m3", qb, sb, "e4m3", True, epi, bias, torch.float16)
    check_recipe("block_fp16", mode, qa, sa, "e4m3", qb, sb, "e4m3", True, np.arange(M), np.arange(N),
                 d.float(), bias, epi)
    if epi == "bias_gelu_aux":
        _, aux16 = run(mode, qa, sa, "e4m3", qb, sb, "e4m3", True, epi, bias, torch.bfloat16)
        assert torch.equal(aux, aux16)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b_2d", [False, True])
@pytest.mark.parametrize("beta", [-0.75, 0.0, 2.0])
def test_block_gemm_accumulate_beta_exact(mode, b_2d, beta):
    """D = fl32(beta C + acc) with one rounding: on exact-integer data (exact accumulators) and C holding
    small dyadic values, equal bit for bit to the float32 rounding of the oracle's beta C + Y."""
    M, N, K = 1040, 784, 640
    rng = np.random.default_rng([M, N, K, b_2d, 7])
    qa, qb = exact_codes(rng, (M, K), "e4m3"), exact_codes(rng, (N, K), "e5m2")
    sa, sb = exact_scales(rng, (M, K // 128)), exact_scales(rng, b_scale_shape(N, K, b_2d))
    c = (rng.integers(-64, 65, size=(M, N)) * 0.25).astype(np.float32)
    out = dev(c)
    run(mode, qa, sa, "e4m3", qb, sb, "e5m2", b_2d, "accumulate", out_dtype=torch.float32, out=out, beta=beta)
    sa_ref, sb_ref = (oracle.pow2_at_least(sa), oracle.pow2_at_least(sb)) if mode == "e8m0" else (sa, sb)
    ref, _, _ = oracle.block_gemm(qa, sa_ref, oracle.E4M3, qb, sb_ref, oracle.E5M2, b_2d, epi="accumulate", c_in=c,
                                  beta=beta)
    assert np.array_equal(host(out), ref.astype(np.float32))


@pytest.mark.parametrize("mode", MODES)
def test_block_gemm_accumulate_beta_recipe(mode):
    """Recipe data, beta = 0.3, against the oracle's beta C + Y within the GEMM bound on the product."""
    M, N, K = 512, 656, 2048
    qa, sa, qb, sb = recipe_operands(M, N, K, True, seed=93)
    rng = np.random.default_rng(94)
    c = (rng.standard_normal((M, N)) * 0.5).astype(np.float32)
    out = dev(c)
    run(mode, qa, sa, "e4m3", qb, sb, "e4m3", True, "accumulate", out_dtype=torch.float32, out=out, beta=0.3)
    sa_ref, sb_ref = (oracle.pow2_at_least(sa), oracle.pow2_at_least(sb)) if mode == "e8m0" else (sa, sb)
    sb_rows = np.repeat(sb_ref, 128, axis=0)[:N]
    ref, _, s = oracle.block_gemm(qa, sa_ref, oracle.E4M3, qb, sb_rows, oracle.E4M3, False, epi="accumulate",
                                  c_in=c, beta=0.3)
    got = host(out).astype(np.float64)
    y_ref = ref - 0.3 * c.astype(np.float64)
    ea, eb = e8m0_expanded(sa, M, False), e8m0_expanded(sb, N, True)
    k_eff = K * 1.25 if mode == "fp32" else K
    # the product's bound, plus the fp32 rounding of beta C + acc
    bound = 2.0 ** -8 * np.abs(y_ref) + 1e-5 * s + (k_eff / 16.0) * 2.0 ** -24 * s + 2.0 ** -24 * np.abs(ref)
    err = np.abs(got - ref)
    r, cc = np.nonzero(err > bound)
    if r.size:
        h = mfma_model.truncation_bound_pairs(qa, ea, oracle.E4M3, qb, eb, oracle.E4M3, r, cc)
        assert np.all(err[r, cc] <= bound[r, cc] + h)
    stated = err <= 2.0 ** -8 * np.abs(y_ref) + 1e-5 * s
    assert_stated_misses(f"block_beta:{mode}", int((~stated).sum()), stated.size)
