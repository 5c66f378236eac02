"""The allocation-free current-scaling cast (te_fp8_cast_current_scaling_noalloc,
for callers that cannot allocate) against the workspace entry point
te_fp8_cast_current_scaling: bit-identical codes, amax, scale and scale_inv
on two calls in a row, the second with a smaller input whose maximum is
smaller, so a stale partial maximum left in the shared static array by the
first call would show; and against the oracle on the smaller input."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def run_both(bits, fmt):
    import mxfp8_mixed_precision_amd as te
    x = dev(bits)
    outs = []
    for noalloc in (False, True):
        q = torch.empty(bits.shape, dtype=torch.uint8, device="cuda")
        a, s, si = (torch.full((1,), -1.0, dtype=torch.float32, device="cuda") for _ in range(3))
        if noalloc:
            te.te_fp8_cast_current_scaling_noalloc(x, fmt, q, a, s, si)
        else:
            ws = torch.empty(max(te.te_amax_workspace_size(x.numel()), 4), dtype=torch.uint8, device="cuda")
            te.te_fp8_cast_current_scaling(x, fmt, q, a, s, si, ws)
        torch.cuda.synchronize()
        outs.append((host(q), host(a), host(s), host(si)))
    return outs


def test_noalloc_cast_matches_workspace_entry_point_on_two_calls():
    # call 1: 4096 x 4096 + 5 elements, its maximum (|x| = 1000) in the tail, handled by the last of the
    # 1024 amax workgroups
    n1 = 4096 * 4096 + 5
    big = workloads.normal_bf16(77, 0, (n1,), 1.0)
    big[-3] = np.uint16(0xC47A)  # -1000.0
    print(f"noalloc call 1: n = {n1}, e4m3", flush=True)
    (q0, a0, s0, i0), (q1, a1, s1, i1) = run_both(big, "e4m3")
    assert a0[0] == 1000.0
    assert np.array_equal(q0, q1) and a0 == a1 and s0 == s1 and i0 == i1
    # call 2: fewer elements (13 amax workgroups), a smaller maximum
    n2 = 100003
    small = workloads.normal_bf16(77, 1, (n2,), 0.5)
    print(f"noalloc call 2: n = {n2}, e5m2", flush=True)
    (q0, a0, s0, i0), (q1, a1, s1, i1) = run_both(small, "e5m2")
    assert np.array_equal(q0, q1) and a0 == a1 and s0 == s1 and i0 == i1
    want_q, want_amax, want_scale, want_inv = oracle.cast_current_scaling(small, oracle.E5M2)
    assert a1[0] == want_amax and s1[0] == want_scale and i1[0] == want_inv
    assert np.array_equal(q1, want_q)


def test_noalloc_cast_empty_input():
    import mxfp8_mixed_precision_amd as te
    x = torch.empty(0, dtype=torch.int16, device="cuda")
    q = torch.empty(0, dtype=torch.uint8, device="cuda")
    a, s, si = (torch.full((1,), -1.0, dtype=torch.float32, device="cuda") for _ in range(3))
    te.te_fp8_cast_current_scaling_noalloc(x, "e4m3", q, a, s, si)
    torch.cuda.synchronize()
    assert host(a)[0] == 0.0 and host(s)[0] == 1.0 and host(si)[0] == 1.0
