"""CPU tests of the C ABI: the library loads, exports every entry point that
include/temx.h declares, and rejects bad arguments on the host before any
HIP call (only calls that fail validation are made here, with fake device
addresses that are never dereferenced)."""

import ctypes
import os
import re

import pytest

import mxfp8_mixed_precision_amd as te

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "temx.h")

P = 0x10000  # fake, 16-byte aligned device address (never dereferenced)
P2 = 0x20000
P3 = 0x30000
BAD = 0x10004  # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:te_status|size_t|const char\*)\s+(te_\w+)\s*\(", text, re.M)))


def test_header_symbols_are_exported():
    names = declared_functions()
    assert set(names) == set(te.EXPORTED)
    lib = ctypes.CDLL(te._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert te.te_status_str(te.TE_OK) == "TE_OK"
    for s in range(1, 9):
        assert te.te_status_str(s).startswith("TE_ERR_")
    assert te.te_status_str(te.TE_ERR_ARCH).startswith("TE_ERR_ARCH")
    assert te.te_status_str(99) == "unknown te_status"


def test_workspace_queries():
    # the rearranged E8M0 scales of the 4-wave path (big-tile grids, K % 1024 == 0, K >= 2048 and 32
    # or more K steps per CU); without a GPU the library takes a 256-CU device
    assert te.te_mxfp8_gemm_workspace_size(8192, 8192, 8192) == 2 * 8192 * 8192 // 32
    assert te.te_mxfp8_gemm_workspace_size(8192, 8192, 1152) == 0
    assert te.te_mxfp8_gemm_workspace_size(-1, 8192, 8192) == 0
    assert te.te_mxfp8_gemm_workspace_size(8192, 8192, 2048) == 2 * 8192 * 2048 // 32
    assert te.te_mxfp8_gemm_workspace_size(4096, 4096, 4096) == 2 * 4096 * 4096 // 32
    assert te.te_mxfp8_gemm_workspace_size(8192, 8192, 1024) == 0
    assert te.te_mxfp8_gemm_workspace_size(4096, 4096, 2048) == 0
    assert te.te_mxfp8_gemm_workspace_size(4096 + 48, 4096 + 80, 2048) == (4144 * 64 + 255) // 256 * 256 + 4176 * 64
    assert te.te_amax_workspace_size(0) == 4
    assert te.te_amax_workspace_size(8192 * 8192) == 4 * 1024
    assert te.te_amax_workspace_size(4096) == 4


L = te._lib


def quant(x=P, rows=64, cols=64, fmt=te.TE_E4M3, d=te.TE_ROWWISE, qr=P2, sr=P3, qc=None, sc=None):
    return L.te_mxfp8_quantize(x, rows, cols, fmt, d, qr, sr, qc, sc, None)


def test_quantize_validation():
    assert quant(d=0) == te.TE_ERR_VALUE
    assert quant(d=4) == te.TE_ERR_VALUE
    assert quant(fmt=te.TE_BF16) == te.TE_ERR_DTYPE
    assert quant(fmt=te.TE_E8M0) == te.TE_ERR_DTYPE
    assert quant(rows=-1) == te.TE_ERR_SHAPE
    assert quant(cols=48) == te.TE_ERR_SHAPE                      # rowwise needs cols % 32
    assert quant(d=te.TE_COLWISE, qr=None, sr=None, qc=P2, sc=P3, rows=48) == te.TE_ERR_SHAPE  # rows % 32
    assert quant(d=te.TE_COLWISE, qr=None, sr=None, qc=P2, sc=P3, cols=36) == te.TE_ERR_SHAPE  # cols % 8
    assert quant(sr=None) == te.TE_ERR_NULL
    assert quant(qc=P2, sc=P3) == te.TE_ERR_NULL                 # colwise outputs given for rowwise
    assert quant(d=te.TE_BOTH) == te.TE_ERR_NULL
    assert quant(x=None) == te.TE_ERR_NULL
    assert quant(x=BAD) == te.TE_ERR_ALIGN
    assert quant(qr=BAD) == te.TE_ERR_ALIGN
    # empty tensors succeed without touching the device
    assert quant(rows=0) == te.TE_OK
    assert quant(x=None, cols=0) == te.TE_OK


def qbgrad(x=P, rows=64, cols=64, fmt=te.TE_E5M2, qr=P2, sr=P3, qc=P2, sc=P3, bgrad=P3, bdt=te.TE_FP32, ws=P,
           ws_bytes=1 << 20):
    return L.te_mxfp8_quantize_bgrad(x, rows, cols, fmt, qr, sr, qc, sc, bgrad, bdt, ws, ws_bytes, None)


def test_quantize_bgrad_workspace_size():
    # fp32 partial sums for each 256-row tile of the input
    assert te.te_mxfp8_quantize_bgrad_workspace_size(0, 64) == 0
    assert te.te_mxfp8_quantize_bgrad_workspace_size(64, 0) == 0
    assert te.te_mxfp8_quantize_bgrad_workspace_size(32, 64) == 1 * 64 * 4
    assert te.te_mxfp8_quantize_bgrad_workspace_size(256, 64) == 1 * 64 * 4
    assert te.te_mxfp8_quantize_bgrad_workspace_size(288, 64) == 2 * 64 * 4
    assert te.te_mxfp8_quantize_bgrad_workspace_size(4096, 14336) == 16 * 14336 * 4


def test_quantize_bgrad_validation():
    assert qbgrad(fmt=te.TE_BF16) == te.TE_ERR_DTYPE
    assert qbgrad(bdt=te.TE_E4M3) == te.TE_ERR_DTYPE
    assert qbgrad(rows=-32) == te.TE_ERR_SHAPE
    assert qbgrad(rows=48) == te.TE_ERR_SHAPE          # rows % 32
    assert qbgrad(cols=40) == te.TE_ERR_SHAPE          # cols % 32
    assert qbgrad(bgrad=None) == te.TE_ERR_NULL
    assert qbgrad(bgrad=P3 + 2) == te.TE_ERR_ALIGN     # fp32 output
    assert qbgrad(x=None) == te.TE_ERR_NULL
    assert qbgrad(qc=None) == te.TE_ERR_NULL
    assert qbgrad(sr=None) == te.TE_ERR_NULL
    assert qbgrad(ws=None) == te.TE_ERR_NULL
    assert qbgrad(x=BAD) == te.TE_ERR_ALIGN
    assert qbgrad(qr=BAD) == te.TE_ERR_ALIGN
    assert qbgrad(ws=P + 2) == te.TE_ERR_ALIGN
    assert qbgrad(ws_bytes=te.te_mxfp8_quantize_bgrad_workspace_size(64, 64) - 4) == te.TE_ERR_WORKSPACE
    # no columns: nothing to compute or write
    assert qbgrad(cols=0, x=None, qr=None, sr=None, qc=None, sc=None, bgrad=None, ws=None) == te.TE_OK


def gemm(a=P, sa=P, fa=te.TE_E4M3, b=P, sb=P, fb=te.TE_E4M3, M=256, N=256, K=256, d=P2, dt=te.TE_BF16,
         epi=te.TE_EPI_NONE, bias=None, aux=None):
    return L.te_mxfp8_gemm(a, sa, fa, b, sb, fb, M, N, K, d, dt, epi, bias, aux, None, 0, None)


def test_gemm_validation():
    assert gemm(K=192) == te.TE_ERR_SHAPE       # K % 128
    assert gemm(K=(1 << 23) + 128) == te.TE_ERR_SHAPE  # beyond the 32-bit copy offsets
    assert gemm(M=72) == te.TE_ERR_SHAPE        # M % 16
    assert gemm(N=40) == te.TE_ERR_SHAPE        # N % 16
    assert gemm(M=-16) == te.TE_ERR_SHAPE
    assert gemm(fa=te.TE_E5M2, fb=te.TE_E5M2) == te.TE_ERR_DTYPE
    assert gemm(fa=te.TE_BF16) == te.TE_ERR_DTYPE
    assert gemm(dt=te.TE_E4M3) == te.TE_ERR_DTYPE
    assert gemm(dt=te.TE_FP16) == te.TE_ERR_DTYPE                          # fp16 D: the blockwise GEMM only
    assert gemm(epi=6) == te.TE_ERR_VALUE
    assert gemm(epi=te.TE_EPI_BIAS) == te.TE_ERR_NULL                       # bias missing
    assert gemm(bias=P3) == te.TE_ERR_NULL                                  # bias without epilogue
    assert gemm(epi=te.TE_EPI_BIAS_GELU_AUX, bias=P3) == te.TE_ERR_NULL     # aux missing
    assert gemm(epi=te.TE_EPI_BIAS, bias=P3, aux=P3) == te.TE_ERR_NULL      # aux without GELU-aux
    assert gemm(a=None) == te.TE_ERR_NULL
    assert gemm(d=None) == te.TE_ERR_NULL
    assert gemm(a=BAD) == te.TE_ERR_ALIGN
    assert gemm(sa=P + 2) == te.TE_ERR_ALIGN
    assert gemm(d=BAD) == te.TE_ERR_ALIGN
    assert gemm(M=0) == te.TE_OK and gemm(N=0, a=None, d=None) == te.TE_OK
    # backward epilogues: dgelu reads aux and takes no bias; accumulate needs fp32 D
    assert gemm(epi=te.TE_EPI_DGELU) == te.TE_ERR_NULL                      # aux missing
    assert gemm(epi=te.TE_EPI_DGELU, aux=P3, bias=P3) == te.TE_ERR_NULL     # bias with dgelu
    assert gemm(epi=te.TE_EPI_DGELU, aux=BAD) == te.TE_ERR_ALIGN
    assert gemm(epi=te.TE_EPI_ACCUMULATE) == te.TE_ERR_DTYPE                 # bf16 D
    assert gemm(epi=te.TE_EPI_ACCUMULATE, dt=te.TE_FP32, aux=P3) == te.TE_ERR_NULL
    assert gemm(epi=te.TE_EPI_ACCUMULATE, dt=te.TE_FP32, bias=P3) == te.TE_ERR_NULL
    assert gemm(epi=te.TE_EPI_ACCUMULATE, dt=te.TE_FP32, M=0) == te.TE_OK
    assert gemm(epi=5) == te.TE_ERR_VALUE


def mxout(a=P, sa=P, fa=te.TE_E4M3, b=P, sb=P, fb=te.TE_E4M3, M=256, N=256, K=256, d=P2, ds=P3,
          df=te.TE_E4M3, epi=te.TE_EPI_NONE, bias=None, aux=None):
    return L.te_mxfp8_gemm_mxout(a, sa, fa, b, sb, fb, M, N, K, d, ds, df, epi, bias, aux, None, 0, None)


def test_gemm_mxout_validation():
    assert mxout(N=48) == te.TE_ERR_SHAPE                 # blocks of 32 along N
    assert mxout(K=192) == te.TE_ERR_SHAPE
    assert mxout(K=(1 << 23) + 128) == te.TE_ERR_SHAPE
    assert mxout(df=te.TE_BF16) == te.TE_ERR_DTYPE
    assert mxout(df=te.TE_E8M0) == te.TE_ERR_DTYPE
    assert mxout(epi=te.TE_EPI_DGELU, aux=P3) == te.TE_ERR_VALUE      # forward epilogues only
    assert mxout(epi=te.TE_EPI_ACCUMULATE) == te.TE_ERR_VALUE
    assert mxout(epi=te.TE_EPI_BIAS) == te.TE_ERR_NULL
    assert mxout(epi=te.TE_EPI_BIAS_GELU_AUX, bias=P3) == te.TE_ERR_NULL
    assert mxout(ds=None) == te.TE_ERR_NULL
    assert mxout(d=None) == te.TE_ERR_NULL
    assert mxout(d=BAD) == te.TE_ERR_ALIGN
    assert mxout(fa=te.TE_E5M2, fb=te.TE_E5M2) == te.TE_ERR_DTYPE
    assert mxout(M=0, d=None, ds=None) == te.TE_OK


def delayed(x=P, n=64, fmt=te.TE_E4M3, q=P2, qinv=P3, scale=P3, hist=P3, L=16, algo=te.TE_AMAX_MAX, margin=0,
            ws=P, ws_bytes=4096):
    return L_.te_fp8_cast_delayed_scaling(x, n, fmt, q, qinv, scale, hist, L, algo, margin, ws, ws_bytes, None)


L_ = L


def test_delayed_scaling_validation():
    assert delayed(fmt=te.TE_BF16) == te.TE_ERR_DTYPE
    assert delayed(algo=2) == te.TE_ERR_VALUE
    assert delayed(margin=-1) == te.TE_ERR_VALUE
    assert delayed(L=0) == te.TE_ERR_SHAPE and delayed(L=1025) == te.TE_ERR_SHAPE
    assert delayed(n=-8) == te.TE_ERR_SHAPE
    assert delayed(scale=None) == te.TE_ERR_NULL
    assert delayed(hist=None) == te.TE_ERR_NULL
    assert delayed(qinv=None) == te.TE_ERR_NULL
    assert delayed(ws=None) == te.TE_ERR_NULL
    assert delayed(q=None) == te.TE_ERR_NULL
    assert delayed(x=BAD) == te.TE_ERR_ALIGN
    assert delayed(scale=P3 + 2) == te.TE_ERR_ALIGN
    assert delayed(ws_bytes=0) == te.TE_ERR_WORKSPACE


def fp8gemm(a=P, sa=P3, fa=te.TE_E4M3, b=P, sb=P3, fb=te.TE_E4M3, M=256, N=256, K=256, d=P2, dt=te.TE_BF16,
            epi=te.TE_EPI_NONE, bias=None, aux=None):
    return L.te_fp8_gemm(a, sa, fa, b, sb, fb, M, N, K, d, dt, epi, bias, aux, None, 0, None)


def test_fp8_gemm_validation():
    assert fp8gemm(K=192) == te.TE_ERR_SHAPE
    assert fp8gemm(K=(1 << 23) + 128) == te.TE_ERR_SHAPE
    assert fp8gemm(epi=te.TE_EPI_DGELU, aux=P3) == te.TE_ERR_VALUE
    assert fp8gemm(fa=te.TE_E5M2, fb=te.TE_E5M2) == te.TE_ERR_DTYPE
    assert fp8gemm(dt=te.TE_E4M3) == te.TE_ERR_DTYPE
    assert fp8gemm(sa=None) == te.TE_ERR_NULL
    assert fp8gemm(sb=P3 + 2) == te.TE_ERR_ALIGN
    assert fp8gemm(epi=te.TE_EPI_BIAS) == te.TE_ERR_NULL
    assert fp8gemm(M=0, d=None) == te.TE_OK


def blockgemm(a=P, sa=P3, fa=te.TE_E4M3, b=P, sb=P3, fb=te.TE_E4M3, b2d=1, M=256, N=256, K=256, d=P2,
              dt=te.TE_BF16, epi=te.TE_EPI_NONE, bias=None, aux=None, mode=te.TE_BLOCK_SCALES_E8M0, ws=None,
              ws_bytes=None, beta=1.0):
    if ws_bytes is None:
        ws_bytes = te.te_fp8_block_gemm_workspace_size(M, N, K, mode)
    return L.te_fp8_block_gemm(a, sa, fa, b, sb, fb, b2d, M, N, K, d, dt, epi, bias, aux, mode, beta, ws, ws_bytes,
                               None)


def test_block_gemm_workspace_and_validation():
    assert te.te_fp8_block_gemm_workspace_size(4096, 1024, 4096, "e8m0") == 0
    assert te.te_fp8_block_gemm_workspace_size(8192, 8192, 8192, "fp32") == 0
    for mode in (te.TE_BLOCK_SCALES_E8M0, te.TE_BLOCK_SCALES_FP32):
        assert blockgemm(mode=mode, K=192) == te.TE_ERR_SHAPE
        assert blockgemm(mode=mode, K=(1 << 23) + 128) == te.TE_ERR_SHAPE
        assert blockgemm(mode=mode, N=40) == te.TE_ERR_SHAPE
        assert blockgemm(mode=mode, b2d=2) == te.TE_ERR_VALUE
        assert blockgemm(mode=mode, fa=te.TE_E5M2, fb=te.TE_E5M2) == te.TE_ERR_DTYPE
        assert blockgemm(mode=mode, dt=te.TE_E4M3) == te.TE_ERR_DTYPE
        assert blockgemm(mode=mode, epi=te.TE_EPI_ACCUMULATE) == te.TE_ERR_DTYPE
        assert blockgemm(mode=mode, epi=te.TE_EPI_ACCUMULATE, dt=te.TE_FP16) == te.TE_ERR_DTYPE   # fp32 D only
        assert blockgemm(mode=mode, dt=te.TE_FP16, a=BAD) == te.TE_ERR_ALIGN   # fp16 D passes the dtype check
        assert blockgemm(mode=mode, epi=te.TE_EPI_BIAS) == te.TE_ERR_NULL
        assert blockgemm(mode=mode, epi=te.TE_EPI_DGELU) == te.TE_ERR_NULL
        assert blockgemm(mode=mode, sa=None) == te.TE_ERR_NULL
        assert blockgemm(mode=mode, sb=P3 + 2) == te.TE_ERR_ALIGN
        assert blockgemm(mode=mode, a=BAD) == te.TE_ERR_ALIGN
        assert blockgemm(mode=mode, M=0, d=None) == te.TE_OK
    assert blockgemm(mode=2) == te.TE_ERR_VALUE
    assert blockgemm(ws=None, ws_bytes=0, sa=None) == te.TE_ERR_NULL
    bq = L.te_fp8_block_quantize
    assert bq(P, 64, 192, te.TE_E4M3, 0, P2, P3, None) == te.TE_ERR_SHAPE
    assert bq(P, -1, 128, te.TE_E4M3, 0, P2, P3, None) == te.TE_ERR_SHAPE
    assert bq(P, 64, 128, te.TE_BF16, 0, P2, P3, None) == te.TE_ERR_DTYPE
    assert bq(P, 64, 128, te.TE_E5M2, 3, P2, P3, None) == te.TE_ERR_VALUE
    assert bq(P, 64, 128, te.TE_E4M3, 1, None, P3, None) == te.TE_ERR_NULL
    assert bq(P, 64, 128, te.TE_E4M3, 1, P2, None, None) == te.TE_ERR_NULL
    assert bq(BAD, 64, 128, te.TE_E4M3, 0, P2, P3, None) == te.TE_ERR_ALIGN
    assert bq(P, 64, 128, te.TE_E4M3, 0, P2 + 8, P3, None) == te.TE_ERR_ALIGN
    assert bq(P, 64, 128, te.TE_E4M3, 0, P2, P3 + 2, None) == te.TE_ERR_ALIGN
    assert bq(None, 0, 128, te.TE_E4M3, 1, None, None, None) == te.TE_OK
    conv = L.te_fp8_block_scales_to_mx
    assert conv(P, 64, 192, 0, P2, None) == te.TE_ERR_SHAPE
    assert conv(P, -1, 128, 0, P2, None) == te.TE_ERR_SHAPE
    assert conv(P, 64, 128, 2, P2, None) == te.TE_ERR_VALUE
    assert conv(None, 64, 128, 1, P2, None) == te.TE_ERR_NULL
    assert conv(P, 64, 128, 1, None, None) == te.TE_ERR_NULL
    assert conv(P + 2, 64, 128, 0, P2, None) == te.TE_ERR_ALIGN
    assert conv(P, 64, 128, 0, P2 + 1, None) == te.TE_ERR_ALIGN
    assert conv(None, 0, 128, 0, None, None) == te.TE_OK


def grouped(G=4, splits=P3, T=1024, a=P, sa=P, fa=te.TE_E4M3, b=P, sb=P, fb=te.TE_E4M3, N=256, K=256, d=P2,
            dt=te.TE_BF16, epi=te.TE_EPI_NONE, bias=None, aux=None):
    return L.te_mxfp8_grouped_gemm(G, splits, T, a, sa, fa, b, sb, fb, N, K, d, dt, epi, bias, aux, None, 0, None)


def test_grouped_validation():
    assert grouped(G=0) == te.TE_ERR_SHAPE
    assert grouped(G=1025) == te.TE_ERR_SHAPE
    assert grouped(T=-1) == te.TE_ERR_SHAPE
    assert grouped(K=192) == te.TE_ERR_SHAPE
    assert grouped(K=(1 << 23) + 128) == te.TE_ERR_SHAPE
    assert grouped(N=40) == te.TE_ERR_SHAPE
    assert grouped(K=0) == te.TE_ERR_SHAPE
    assert grouped(splits=None) == te.TE_ERR_NULL
    assert grouped(splits=P3 + 2) == te.TE_ERR_ALIGN
    assert grouped(fa=te.TE_E5M2, fb=te.TE_E5M2) == te.TE_ERR_DTYPE
    assert grouped(epi=te.TE_EPI_BIAS_GELU_AUX, bias=P3) == te.TE_ERR_NULL
    assert grouped(b=BAD) == te.TE_ERR_ALIGN
    assert grouped(T=0) == te.TE_OK


def test_amax_and_cast_validation():
    ws = te.te_amax_workspace_size(1 << 20)
    assert L.te_amax_reduce(P, -1, P2, P3, ws, None) == te.TE_ERR_SHAPE
    assert L.te_amax_reduce(P, 1 << 20, None, P3, ws, None) == te.TE_ERR_NULL
    assert L.te_amax_reduce(P, 1 << 20, P2, None, ws, None) == te.TE_ERR_NULL
    assert L.te_amax_reduce(BAD, 1 << 20, P2, P3, ws, None) == te.TE_ERR_ALIGN
    assert L.te_amax_reduce(P, 1 << 20, P2, P3, ws - 4, None) == te.TE_ERR_WORKSPACE
    cast = L.te_fp8_cast_current_scaling
    assert cast(P, 1024, te.TE_BF16, P2, P3, P3, P3, P3, 64, None) == te.TE_ERR_DTYPE
    assert cast(P, 1024, te.TE_E4M3, None, P3, P3, P3, P3, 64, None) == te.TE_ERR_NULL
    assert cast(P, 1024, te.TE_E4M3, P2, P3, None, P3, P3, 64, None) == te.TE_ERR_NULL
    assert cast(P, 1024, te.TE_E4M3, BAD, P3, P3, P3, P3, 64, None) == te.TE_ERR_ALIGN
    assert cast(P, 1 << 24, te.TE_E5M2, P2, P3, P3, P3, P3, 4, None) == te.TE_ERR_WORKSPACE


def test_import_fails_loudly_without_library(tmp_path):
    # the package refuses to import when libtemx.so is absent (no CPU fallback)
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "mxfp8_mixed_precision_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "mxfp8_mixed_precision_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import mxfp8_mixed_precision_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "libtemx.so is missing" in r.stderr


def test_binding_refuses_host_and_strided_tensors():
    # every pointer of the ABI is a device pointer into a dense buffer: the binding checks before calling
    import torch
    x = torch.zeros((64, 64), dtype=torch.int16)
    with pytest.raises(ValueError, match="GPU tensor"):
        te.te_mxfp8_quantize(x, "e4m3", "row", torch.zeros((64, 64), dtype=torch.uint8),
                             torch.zeros((64, 2), dtype=torch.uint8))

    class FakeStrided:
        is_cuda = True
        device = "cuda:0"

        def is_contiguous(self):
            return False

        def data_ptr(self):
            raise AssertionError("must not be reached")

    with pytest.raises(ValueError, match="contiguous"):
        te._ptr(FakeStrided())
    assert te._ptr(None) is None


def test_binding_checks_shapes_and_dtypes_before_the_call():
    # host tensors of the right shape and dtype get as far as the device check; each wrong
    # shape or dtype is refused first (the library itself never sees the tensor sizes)
    import torch
    u8, bf, f32, i32 = torch.uint8, torch.bfloat16, torch.float32, torch.int32

    def t(shape, dtype):
        return torch.zeros(shape, dtype=dtype)

    M, N, K = 32, 48, 128
    a, sa, b, sb = t((M, K), u8), t((M, K // 32), u8), t((N, K), u8), t((N, K // 32), u8)
    d, bias, aux = t((M, N), bf), t((N,), bf), t((M, N), bf)

    def refuse(match, fn, *args, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*args, **kw)

    # MXFP8 GEMM: the valid call reaches the device check
    refuse("GPU tensor", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", d, "bias_gelu_aux", bias, aux)
    refuse("d: expected bfloat16 or float32", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", t((M, N), torch.float16))
    refuse("accumulate epilogue needs float32", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", d, "accumulate")
    refuse(r"d: expected shape \(32, 48\)", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", t((M, N - 16), bf))
    refuse(r"b: expected shape \(48, 128\)", te.te_mxfp8_gemm, a, sa, "e4m3", t((N, K + 128), u8), sb, "e4m3", d)
    refuse("a_scale: expected shape", te.te_mxfp8_gemm, a, t((M, K // 16), u8), "e4m3", b, sb, "e4m3", d)
    refuse("b_scale: expected shape", te.te_mxfp8_gemm, a, sa, "e4m3", b, t((N - 16, K // 32), u8), "e4m3", d)
    refuse("a: expected 1-byte codes", te.te_mxfp8_gemm, t((M, K), bf), sa, "e4m3", b, sb, "e4m3", d)
    refuse("bias: expected shape", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", d, "bias", t((N + 16,), bf))
    refuse("bias: expected bf16", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", d, "bias", t((N,), f32))
    refuse("aux: expected shape", te.te_mxfp8_gemm, a, sa, "e4m3", b, sb, "e4m3", d, "bias_gelu_aux", bias,
           t((M, N - 16), bf))
    # MXFP8 output
    refuse("GPU tensor", te.te_mxfp8_gemm_mxout, a, sa, "e4m3", b, sb, "e4m3", t((M, N), u8), t((M, N // 32), u8),
           "e4m3")
    refuse("d_scale: expected shape", te.te_mxfp8_gemm_mxout, a, sa, "e4m3", b, sb, "e4m3", t((M, N), u8),
           t((M, N // 16), u8), "e4m3")
    # grouped
    G = 3
    gb, gsb = t((G * N, K), u8), t((G * N, K // 32), u8)
    splits = t((G,), i32)
    refuse("GPU tensor", te.te_mxfp8_grouped_gemm, splits, a, sa, "e4m3", gb, gsb, "e4m3", N, d, "bias",
           t((G, N), bf))
    refuse("m_splits: expected a 1-D int32", te.te_mxfp8_grouped_gemm, t((G,), torch.int64), a, sa, "e4m3", gb, gsb,
           "e4m3", N, d)
    refuse("b: expected 3 x 48", te.te_mxfp8_grouped_gemm, splits, a, sa, "e4m3", b, sb, "e4m3", N, d)
    refuse("bias: expected shape", te.te_mxfp8_grouped_gemm, splits, a, sa, "e4m3", gb, gsb, "e4m3", N, d, "bias",
           bias)
    refuse("d: expected bfloat16 or float32", te.te_mxfp8_grouped_gemm, splits, a, sa, "e4m3", gb, gsb, "e4m3", N,
           t((M, N), torch.float16))
    # per-tensor FP8 GEMM
    one = t((1,), f32)
    refuse("GPU tensor", te.te_fp8_gemm, a, one, "e4m3", b, one, "e4m3", d)
    refuse("a_scale_inv: expected a float32 scalar", te.te_fp8_gemm, a, t((1,), bf), "e4m3", b, one, "e4m3", d)
    refuse(r"b: expected shape", te.te_fp8_gemm, a, one, "e4m3", t((N, 2 * K), u8), one, "e4m3", d)
    # blockwise GEMM
    bsa, bsb2 = t((M, K // 128), f32), t(((N + 127) // 128, K // 128), f32)
    refuse("GPU tensor", te.te_fp8_block_gemm, a, bsa, "e4m3", b, bsb2, "e4m3", True, d)
    refuse("b_scale_inv: expected shape", te.te_fp8_block_gemm, a, bsa, "e4m3", b, bsb2, "e4m3", False, d)
    refuse("a_scale_inv: expected float32", te.te_fp8_block_gemm, a, t((M, K // 128), bf), "e4m3", b, bsb2, "e4m3",
           True, d)
    # quantize
    x = t((M, K), bf)
    refuse("GPU tensor", te.te_mxfp8_quantize, x, "e4m3", "row", t((M, K), u8), t((M, K // 32), u8))
    refuse("q_row: expected shape", te.te_mxfp8_quantize, x, "e4m3", "row", t((K, M), u8), t((M, K // 32), u8))
    refuse("s_col: expected shape", te.te_mxfp8_quantize, x, "e4m3", "col", None, None, t((K, M), u8),
           t((K, M // 16), u8))
    refuse("x: expected bf16", te.te_mxfp8_quantize, t((M, K), f32), "e4m3", "row", t((M, K), u8),
           t((M, K // 32), u8))
    refuse("bgrad: expected shape", te.te_mxfp8_quantize_bgrad, x, "e5m2", t((M, K), u8), t((M, K // 32), u8),
           t((K, M), u8), t((K, M // 32), u8), t((M,), f32), None)
    refuse("q: expected shape", te.te_fp8_block_quantize, x, "e4m3", True, t((M, K - 32), u8), t((1, 1), f32))
    refuse("scale_inv: expected shape", te.te_fp8_block_quantize, x, "e4m3", False, t((M, K), u8), t((1, 1), f32))
    refuse("mx_scale: expected shape", te.te_fp8_block_scales_to_mx, t((M, 1), f32), M, K, False, t((M, 2), u8))
    # casts
    refuse("q_out: expected shape", te.te_fp8_cast_current_scaling, x, "e4m3", t((M * K - 1,), u8), one, one, one, None)
    refuse("amax_out: expected a float32", te.te_amax_reduce, x, t((1,), bf), None)
    refuse("amax_history: expected a 1-D float32", te.te_fp8_cast_delayed_scaling, x, "e4m3", t((M, K), u8), one, one,
           t((16,), bf), None)


def test_valid_call_without_a_gfx950_returns_arch_error():
    # a call that passes validation checks the device before enqueuing anything; with no GPU
    # (this container) that check fails.  Skipped where a GPU is visible: there the call would
    # launch on the fake addresses.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    assert quant() == te.TE_ERR_ARCH
    assert L.te_mxfp8_gemm(P, P2, te.TE_E4M3, P, P2, te.TE_E4M3, 16, 16, 128, P3, te.TE_BF16, te.TE_EPI_NONE,
                           None, None, None, 0, None) == te.TE_ERR_ARCH
    # the checks before it still come first
    assert quant(x=BAD) == te.TE_ERR_ALIGN


def test_cast_current_noalloc_validation():
    cast = L.te_fp8_cast_current_scaling_noalloc
    assert cast(P, 1024, te.TE_BF16, P2, P3, P3, P3, None) == te.TE_ERR_DTYPE
    assert cast(P, -1, te.TE_E4M3, P2, P3, P3, P3, None) == te.TE_ERR_SHAPE
    assert cast(P, 1024, te.TE_E4M3, P2, None, P3, P3, None) == te.TE_ERR_NULL
    assert cast(None, 1024, te.TE_E4M3, P2, P3, P3, P3, None) == te.TE_ERR_NULL
    assert cast(P, 1024, te.TE_E4M3, None, P3, P3, P3, None) == te.TE_ERR_NULL
    assert cast(BAD, 1024, te.TE_E4M3, P2, P3, P3, P3, None) == te.TE_ERR_ALIGN
    assert cast(P, 1024, te.TE_E4M3, BAD, P3, P3, P3, None) == te.TE_ERR_ALIGN
