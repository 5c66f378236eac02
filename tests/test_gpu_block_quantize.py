"""GPU parity of the blockwise FP8 quantizer (1 x 128 and 128 x 128 blocks,
power-of-two FP32 scale inverses): codes and scales bit-exact against
oracle.quantize_1d / quantize_2d.

Inputs: seeded normal bf16 tensors with outlier columns, plus blocks that
take every path of the scale rule: all-zero blocks (scale 1), blocks of
tiny values whose scale lies below 2^-127 (the values are rescaled before
the hardware convert), blocks near the bf16 maximum, amaxes on either side
of the rounding threshold 0.875 * 2^k * max, and signed zeros.  Ragged row
counts for the 2-D blocks; the bench shapes at full size with sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def te():
    import mxfp8_mixed_precision_amd as m
    return m


def to_bf16(f32) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def special_tensor(rows, cols, seed):
    """Normal data with per-128-block overrides (block = 1 x 128 along rows; every 128 x 128 block
    also gets a few of them)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, rng.choice(cols, max(1, cols // 100), replace=False)] *= 20
    nb = cols // 128
    kinds = rng.integers(0, 8, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            sl = x[r, 128 * b:128 * (b + 1)]
            k = kinds[r, b]
            if k == 1:
                sl[:] = 0.0
            elif k == 2:
                sl *= np.float32(2.0 ** -128)                  # scale below 2^-127
            elif k == 3:
                sl *= np.float32(2.0 ** 118)                    # near the top of the range
            elif k == 4:                                        # amax on the threshold 0.875 * 2^k * max
                sl /= np.abs(sl).max()
                sl[rng.integers(0, 128)] = np.float32(rng.choice([0.875, 0.87890625, 0.8671875]) * 2.0 ** rng.integers(-20, 20))
            elif k == 5:
                sl[:] = np.where(rng.integers(0, 2, 128) == 1, -0.0, 0.0)
                sl[rng.integers(0, 128)] = np.float32(2.0 ** -133)  # smallest bf16 subnormal
    bits = to_bf16(x)
    bits[0, :128] = 0x7F7F  # bf16 maximum
    return bits


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(64, 1024), (300, 2048), (1, 128)])
def test_quantize_1d_matches_oracle(fmt, rows, cols):
    x = special_tensor(rows, cols, seed=rows + cols)
    q, s = te().fp8_block_quantize(dev(x), fmt, block_2d=False)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_1d(x, oracle.format_by_name(fmt))
    assert np.array_equal(host(s), os_), "scales differ"
    assert np.array_equal(host(q), oq), "codes differ"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(128, 128), (300, 1024), (1000, 512), (5, 256)])
def test_quantize_2d_matches_oracle(fmt, rows, cols):
    x = special_tensor(rows, cols, seed=3 * rows + cols)
    rng = np.random.default_rng(rows)
    # whole 128 x 128 blocks of zeros and of tiny values
    if rows >= 256:
        x[128:256, :128] = 0
        x[:128, 128:256] = to_bf16(rng.standard_normal((128, 128)).astype(np.float32) * np.float32(2.0 ** -140))
    q, s = te().fp8_block_quantize(dev(x), fmt, block_2d=True)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_2d(x, oracle.format_by_name(fmt))
    assert np.array_equal(host(s), os_), "scales differ"
    assert np.array_equal(host(q), oq), "codes differ"


def test_quantize_empty():
    z = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    for b2d in (False, True):
        q, s = te().fp8_block_quantize(z, "e4m3", block_2d=b2d)
        assert q.shape == (0, 256) and s.shape == (0, 2)


@pytest.mark.parametrize("block_2d", [False, True])
def test_quantize_full_size_sampled(block_2d):
    """8192 x 8192 (the bench operands), checked on sampled rows (1-D) or 128-row slabs (2-D)."""
    rows = cols = 8192
    x = workloads.normal_bf16(71, int(block_2d), (rows, cols), 1.0 if not block_2d else 0.02, outlier_frac=0.01)
    q, s = te().fp8_block_quantize(dev(x), "e4m3", block_2d=block_2d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(72)
    if block_2d:
        for br in sorted({0, 63} | set(rng.choice(64, 4, replace=False).tolist())):
            slab = x[128 * br:128 * (br + 1)]
            oq, os_ = oracle.quantize_2d(slab, oracle.E4M3)
            assert np.array_equal(host(s[br:br + 1]), os_)
            assert np.array_equal(host(q[128 * br:128 * (br + 1)]), oq)
    else:
        rs = np.array(sorted({0, rows - 1} | set(rng.choice(rows, 64, replace=False).tolist())))
        oq, os_ = oracle.quantize_1d(x[rs], oracle.E4M3)
        assert np.array_equal(host(s[rs]), os_)
        assert np.array_equal(host(q[rs]), oq)
