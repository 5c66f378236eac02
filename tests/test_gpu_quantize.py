"""GPU parity of MXFP8 quantization, amax and the current-scaling cast against
the CPU oracle: bit-exact codes, scales, amax, scale and scale_inv."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, finite_bf16_patterns, host

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2"]


def te():
    import mxfp8_mixed_precision_amd as m
    return m


def check_quantize(bits: np.ndarray, fmt: str, direction: str = "both"):
    f = oracle.format_by_name(fmt)
    x = dev(bits)
    qr, sr, qc, sc = te().mxfp8_quantize(x, fmt, direction)
    torch.cuda.synchronize()
    if qr is not None:
        oq, os_ = oracle.quantize_rowwise(bits, f)
        assert np.array_equal(host(sr), os_), "rowwise scales differ"
        assert np.array_equal(host(qr), oq), "rowwise codes differ"
    if qc is not None:
        oq, os_ = oracle.quantize_colwise(bits, f)
        assert np.array_equal(host(sc), os_), "colwise scales differ"
        assert np.array_equal(host(qc), oq), "colwise codes differ"


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_every_finite_bf16_random_blocks(fmt):
    rng = np.random.default_rng(100)
    p = rng.permutation(finite_bf16_patterns())
    bits = np.zeros(256 * 256, np.uint16)
    bits[:p.size] = p
    check_quantize(bits.reshape(256, 256), fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_every_finite_bf16_magnitude_sorted_blocks(fmt):
    # neighbours in magnitude share a block, so every element is encoded with
    # a scale close to its own exponent (normals, subnormals, ties, saturation)
    p = finite_bf16_patterns()
    order = np.argsort(p & 0x7FFF, kind="stable")
    rng = np.random.default_rng(101)
    bits = np.zeros(256 * 256, np.uint16)
    bits[:p.size] = p[order]
    blocks = bits.reshape(-1, 32)
    blocks = blocks[:, rng.permutation(32)]  # position of the block maximum varies
    check_quantize(blocks.reshape(256, 256), fmt)
    check_quantize(np.ascontiguousarray(blocks.reshape(256, 256).T), fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 32), (33, 64), (96, 160), (160, 72), (32, 8), (4160, 200)])
def test_quantize_ragged_shapes(fmt, shape):
    rows, cols = shape
    bits = workloads.normal_bf16(77, rows * 1000 + cols, shape, 3.0, 0.05)
    if rows % 32 == 0 and cols % 32 == 0:
        check_quantize(bits, fmt, "both")
    if cols % 32 == 0:
        check_quantize(bits, fmt, "row")
    if rows % 32 == 0 and cols % 8 == 0:
        check_quantize(bits, fmt, "col")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_special_blocks(fmt):
    # zero blocks, negative zeros, subnormal-only blocks, huge blocks, single spikes
    rows = []
    rows.append(np.zeros(64, np.uint16))
    rows.append(np.full(64, 0x8000, np.uint16))
    rows.append(np.arange(1, 65, dtype=np.uint16))            # bf16 subnormals
    rows.append((np.arange(64, dtype=np.uint16) | 0x7F00))    # near the top of the range
    spike = np.full(64, 0x3F80, np.uint16)
    spike[5] = 0x4700  # 32768
    rows.append(spike)
    bits = np.stack(rows * 8)[:32]
    check_quantize(bits, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_decoder_activation(fmt):
    # 4096 tokens x 1024 hidden, N(0,1) with 1% outlier columns x20
    bits = workloads.normal_bf16(2, 0, (4096, 1024), 1.0, 0.01)
    check_quantize(bits, fmt)


def sampled_rows(n, k=48, seed=0):
    rng = np.random.default_rng(seed)
    s = set([0, 1, n - 1, n // 2]) | set(rng.choice(n, k, replace=False).tolist())
    return np.array(sorted(s))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_8192_square_sampled(fmt):
    # full-size standalone quantize of an 8192 x 8192 operand (both directions),
    # checked on sampled output rows
    spec = workloads.large_square().quantize[0][0]
    bits = spec.make()
    f = oracle.format_by_name(fmt)
    x = dev(bits)
    qr, sr, qc, sc = te().mxfp8_quantize(x, fmt, "both")
    torch.cuda.synchronize()
    rows = sampled_rows(8192, seed=1)
    oq, os_ = oracle.quantize_rowwise(bits[rows], f)
    assert np.array_equal(host(qr[rows]), oq) and np.array_equal(host(sr[rows]), os_)
    cols = sampled_rows(8192, seed=2)
    oq, os_ = oracle.quantize_colwise(np.ascontiguousarray(bits[:, cols]), f)
    assert np.array_equal(host(qc[cols]), oq) and np.array_equal(host(sc[cols]), os_)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [
    (8288, 8232),    # 8192^2-sized strips (up to 8 chunks of 128 rows) with a 96-row and a 40-column tail
    (4128, 14344),   # last strip chunk a single 32-row block, 8-column tail
    (14336, 4096),   # the HYBRID backward W1 (dgrad B)
    (4096, 14336),   # the HYBRID backward dY (wgrad A)
    (4096, 4096),    # the HYBRID backward X (wgrad B)
])
def test_colwise_equals_rowwise_of_transpose_full_size(fmt, shape):
    # colwise(X) == rowwise(X^T) element for element on the whole tensor (the
    # rowwise kernel is pinned to the oracle above), plus sampled columns
    # against the oracle itself
    rows, cols = shape
    bits = workloads.normal_bf16(90, rows + 7 * cols, shape, 1.0, 0.01)
    x = dev(bits)
    _, _, qc, sc = te().mxfp8_quantize(x, fmt, "col")
    qr, sr, _, _ = te().mxfp8_quantize(x.t().contiguous(), fmt, "row")
    torch.cuda.synchronize()
    assert torch.equal(sc, sr), "colwise scales differ from rowwise of the transpose"
    assert torch.equal(qc, qr), "colwise codes differ from rowwise of the transpose"
    f = oracle.format_by_name(fmt)
    sel = sampled_rows(cols, k=24, seed=3)
    oq, os_ = oracle.quantize_colwise(np.ascontiguousarray(bits[:, sel]), f)
    assert np.array_equal(host(sc[sel]), os_) and np.array_equal(host(qc[sel]), oq)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 4096 * 8 + 3, 1 << 20, 4096 * 4096])
def test_amax(n):
    bits = workloads.normal_bf16(88, n, (n,), 1.5, 0.0) if n else np.zeros(0, np.uint16)
    if n > 10:
        bits[n // 3] = 0xC3A0  # -320.0 planted
    x = dev(bits) if n else torch.zeros(0, dtype=torch.int16, device="cuda")
    a = te().amax(x)
    torch.cuda.synchronize()
    assert host(a)[0] == oracle.amax(bits)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [1, 13, 4096 + 5, 4096 * 4096])
def test_current_scaling_cast(fmt, n):
    bits = workloads.normal_bf16(4, 2, (n,), 1.0, 0.0)
    f = oracle.format_by_name(fmt)
    q, a, s, si = te().fp8_cast_current_scaling(dev(bits), fmt)
    torch.cuda.synchronize()
    oq, oa, os_, osi = oracle.cast_current_scaling(bits, f)
    assert host(a)[0] == oa and host(s)[0] == os_ and host(si)[0] == osi
    assert np.array_equal(host(q), oq)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("where", ["tail", "last_chunk", "first"])
def test_current_scaling_cast_max_at_the_edges(fmt, where):
    # 2^24 + 7 elements (1024 partial maxima, a 7-element tail): the tensor's
    # largest magnitude sits in the tail, in the last full 16-byte chunk, or
    # first; every workgroup of the cast must derive the same scale from it
    n = (1 << 24) + 7
    bits = workloads.normal_bf16(4, 3, (n,), 1.0, 0.0)
    idx = {"tail": n - 2, "last_chunk": (n // 8) * 8 - 3, "first": 0}[where]
    bits[idx] = 0xC4FA  # -2000.0, far above the N(0, 1) values
    f = oracle.format_by_name(fmt)
    q, a, s, si = te().fp8_cast_current_scaling(dev(bits), fmt)
    torch.cuda.synchronize()
    oq, oa, os_, osi = oracle.cast_current_scaling(bits, f)
    assert oa == 2000.0
    assert host(a)[0] == oa and host(s)[0] == os_ and host(si)[0] == osi
    assert np.array_equal(host(q), oq)


def test_current_scaling_zero_and_subnormal_tensors():
    for bits in (np.zeros(64, np.uint16), np.array([0x8000] * 63 + [0x0001], np.uint16)):
        q, a, s, si = te().fp8_cast_current_scaling(dev(bits), "e4m3")
        torch.cuda.synchronize()
        oq, oa, os_, osi = oracle.cast_current_scaling(bits, oracle.E4M3)
        assert host(a)[0] == oa and host(s)[0] == os_ and host(si)[0] == osi
        assert np.array_equal(host(q), oq)


def test_quantize_is_deterministic():
    bits = workloads.normal_bf16(3, 0, (1024, 1024), 1.0, 0.01)
    x = dev(bits)
    r1 = te().mxfp8_quantize(x, "e4m3", "both")
    r2 = te().mxfp8_quantize(x, "e4m3", "both")
    torch.cuda.synchronize()
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


# ---------------------------------------------------------------- fused pass + bias gradient

def bgrad_bound(bits, bgrad_dtype):
    """|got - ref| allowed for the column sums: fp32 accumulation along a path
    of at most 64 per-lane additions (8 rows x 8 blocks in the 128-column
    kernel, 4 x 8 in the colwise kernel), at most 3 butterfly steps (2 and 3),
    1 across row groups and 1 per 256-row tile, i.e. gamma_d * sum |x|
    with d + 1 terms; bf16 output adds its rounding (2^-8 relative)."""
    ref = oracle.column_sums(bits)
    s = oracle.column_abs_sums(bits)
    tiles = -(-bits.shape[0] // 256)
    d = 64 + 3 + 1 + tiles + 1
    b32 = d * 2.0 ** -24 * s
    if bgrad_dtype == torch.bfloat16:
        return ref, 2.0 ** -8 * (np.abs(ref) + b32) + b32
    return ref, b32


def bgrad_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_quantize_bgrad(bits, fmt, bgrad_dtype, full_oracle=True):
    x = dev(bits)
    qr, sr, qc, sc, bg = te().mxfp8_quantize_bgrad(x, fmt, bgrad_dtype)
    torch.cuda.synchronize()
    f = oracle.format_by_name(fmt)
    if full_oracle:
        oq, os_ = oracle.quantize_rowwise(bits, f)
        assert np.array_equal(host(sr), os_) and np.array_equal(host(qr), oq), "rowwise copy differs"
        oq, os_ = oracle.quantize_colwise(bits, f)
        assert np.array_equal(host(sc), os_) and np.array_equal(host(qc), oq), "colwise copy differs"
    ref, bound = bgrad_bound(bits, bgrad_dtype)
    got = bgrad_host(bg)
    assert np.all(np.abs(got - ref) <= bound), f"bgrad off by up to {np.max(np.abs(got - ref) - bound)} beyond the bound"
    return qr, sr, qc, sc, bg


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bgrad_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (288, 224), (4160, 256), (1056, 4128)])
def test_quantize_bgrad_ragged_shapes(fmt, bgrad_dtype, shape):
    rows, cols = shape
    bits = workloads.normal_bf16(78, rows * 1000 + cols, shape, 1e-3, 0.02)
    check_quantize_bgrad(bits, fmt, bgrad_dtype)


def test_quantize_bgrad_integer_columns_exact():
    # small integers: every partial sum is an integer below 2^24, so any fp32 order is exact
    rng = np.random.default_rng(79)
    vals = rng.integers(-64, 65, size=(2048, 320)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    _, _, _, _, bg = te().mxfp8_quantize_bgrad(dev(bits), "e5m2", torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(bgrad_host(bg), vals.astype(np.float64).sum(axis=0))


def test_quantize_bgrad_single_element_lands_in_its_column():
    rows, cols = 512, 288
    bits = np.zeros((rows, cols), np.uint16)
    for r, c in [(0, 0), (511, 287), (257, 33), (300, 255), (31, 256)]:
        bits[r, c] = 0x3FC0  # 1.5
    ref = oracle.column_sums(bits)
    _, _, _, _, bg = te().mxfp8_quantize_bgrad(dev(bits), "e4m3", torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(bgrad_host(bg), ref)


def test_quantize_bgrad_empty_rows_give_zeros():
    x = torch.zeros((0, 96), dtype=torch.int16, device="cuda")
    bg = torch.full((96,), 7.0, dtype=torch.float32, device="cuda")
    te().te_mxfp8_quantize_bgrad(x, "e5m2", None, None, None, None, bg, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(bg).item() == 0


def test_quantize_bgrad_deterministic():
    bits = workloads.normal_bf16(80, 0, (2048, 1536), 1e-3, 0.0)
    x = dev(bits)
    r1 = te().mxfp8_quantize_bgrad(x, "e5m2")
    r2 = te().mxfp8_quantize_bgrad(x, "e5m2")
    torch.cuda.synchronize()
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


@pytest.mark.parametrize("bgrad_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(4096, 14336), (4128, 14368)])
def test_quantize_bgrad_full_size_backward_dy(bgrad_dtype, shape):
    # the backward pass's output gradient dY [4096, 14336] (E5M2, N(0, 1e-3)),
    # and a shape whose last column and row tiles are partial (both run the
    # 128-column kernel, two chunks per wave): both copies equal the separate
    # (oracle-pinned) kernels' outputs on the whole tensor, sampled rows and
    # columns (the last ones included) equal the oracle, bgrad within the bound
    if shape == (4096, 14336):
        bits = workloads.hybrid_backward().gemms[0].a_src.make()
        assert bits.shape == shape
    else:
        bits = workloads.normal_bf16(81, 0, shape, 1e-3, 0.02)
    x = dev(bits)
    qr, sr, qc, sc, bg = te().mxfp8_quantize_bgrad(x, "e5m2", bgrad_dtype)
    q2r, s2r, _, _ = te().mxfp8_quantize(x, "e5m2", "row")
    _, _, q2c, s2c = te().mxfp8_quantize(x, "e5m2", "col")
    torch.cuda.synchronize()
    assert torch.equal(qr, q2r) and torch.equal(sr, s2r), "fused rowwise copy differs from the rowwise kernel"
    assert torch.equal(qc, q2c) and torch.equal(sc, s2c), "fused colwise copy differs from the colwise kernel"
    f = oracle.E5M2
    rows = sampled_rows(shape[0], k=16, seed=5)
    oq, os_ = oracle.quantize_rowwise(bits[rows], f)
    assert np.array_equal(host(qr[rows]), oq) and np.array_equal(host(sr[rows]), os_)
    cols = sampled_rows(shape[1], k=16, seed=6)
    oq, os_ = oracle.quantize_colwise(np.ascontiguousarray(bits[:, cols]), f)
    assert np.array_equal(host(qc[cols]), oq) and np.array_equal(host(sc[cols]), os_)
    ref, bound = bgrad_bound(bits, bgrad_dtype)
    assert np.all(np.abs(bgrad_host(bg) - ref) <= bound)


def special_patch(kind, rng):
    """A 32 x 32 bf16 patch: zeros, negative zeros, subnormals only, values
    near the top of the bf16 range (either sign), or ones with one spike."""
    if kind == 0:
        return np.zeros((32, 32), np.uint16)
    if kind == 1:
        return np.full((32, 32), 0x8000, np.uint16)
    if kind == 2:
        return (np.arange(1024, dtype=np.uint16) % 127 + 1).reshape(32, 32)
    if kind == 3:
        sign = rng.integers(0, 2, (32, 32)).astype(np.uint16) << 15
        return (0x7F00 | (np.arange(1024, dtype=np.uint16) & 0x3F)).reshape(32, 32) | sign
    p = np.full((32, 32), 0x3F80, np.uint16)
    p[rng.integers(0, 32), rng.integers(0, 32)] = 0x4700
    return p


@pytest.mark.parametrize("fmt", FMTS)
def test_both_directions_special_blocks_large(fmt):
    # a grid large enough for the 128-column fused kernel, with special 32 x 32
    # patches at tile edges and in the partial last row and column tiles: the
    # copies equal the separate kernels on the whole tensor and the oracle on
    # the rows and columns through every patch
    rows, cols = 4128, 14368
    rng = np.random.default_rng(93)
    bits = workloads.normal_bf16(92, 0, (rows, cols), 1.0, 0.0)
    spots = [(0, 0), (96, 128), (128, 224), (512, 256), (2048, 8160), (3968, 14208), (4064, 14304), (4096, 14336),
             (4096, 0), (0, 14336)]
    for k, (r, c) in enumerate(spots):
        bits[r:r + 32, c:c + 32] = special_patch(k % 5, rng)
    x = dev(bits)
    qr, sr, qc, sc = te().mxfp8_quantize(x, fmt, "both")
    q2r, s2r, _, _ = te().mxfp8_quantize(x, fmt, "row")
    _, _, q2c, s2c = te().mxfp8_quantize(x, fmt, "col")
    torch.cuda.synchronize()
    assert torch.equal(qr, q2r) and torch.equal(sr, s2r)
    assert torch.equal(qc, q2c) and torch.equal(sc, s2c)
    f = oracle.format_by_name(fmt)
    rsel = np.array(sorted({r + d for r, _ in spots for d in (0, 13, 31)} | {rows - 1}))
    oq, os_ = oracle.quantize_rowwise(bits[rsel], f)
    assert np.array_equal(host(qr[rsel]), oq) and np.array_equal(host(sr[rsel]), os_)
    csel = np.array(sorted({c + d for _, c in spots for d in (0, 17, 31)} | {cols - 1}))
    oq, os_ = oracle.quantize_colwise(np.ascontiguousarray(bits[:, csel]), f)
    assert np.array_equal(host(qc[csel]), oq) and np.array_equal(host(sc[csel]), os_)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(8192, 8192), (8288, 8224), (4096, 4096), (14336, 4096)])
def test_both_directions_fused_equals_separate_full_size(fmt, shape):
    # TE_BOTH runs the fused pass; it must equal the two single-direction kernels bit for bit
    rows, cols = shape
    bits = workloads.normal_bf16(91, rows + 3 * cols, shape, 1.0, 0.01)
    x = dev(bits)
    qr, sr, qc, sc = te().mxfp8_quantize(x, fmt, "both")
    q2r, s2r, _, _ = te().mxfp8_quantize(x, fmt, "row")
    _, _, q2c, s2c = te().mxfp8_quantize(x, fmt, "col")
    torch.cuda.synchronize()
    assert torch.equal(qr, q2r) and torch.equal(sr, s2r)
    assert torch.equal(qc, q2c) and torch.equal(sc, s2c)
