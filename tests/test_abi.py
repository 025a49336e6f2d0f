"""The C-ABI library loads on the CPU host and exports every entry point
include/quads.h declares; argument validation happens on the host and returns
the documented status codes without touching a GPU."""
import ctypes
import os
import re

import pytest

from fp4_quantized_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "quads.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(quads_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libquads.so is not built (python -m fp4_quantized_moe_amd.build)")
    return _lib.load()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_version_and_sizes(L):
    assert L.quads_version().startswith(b"quads")
    assert L.quads_rac_nsel(2048, 50) == 1024
    assert L.quads_rac_nsel(256, 33) == 84
    assert L.quads_rac_nsel(10, 101) == -1
    assert L.quads_rac_nsel(-1, 10) == -1
    assert L.quads_rac_kpad(84) == 96 and L.quads_rac_kpad(0) == 0 and L.quads_rac_kpad(-3) == -1
    assert L.quads_quantize_workspace_bytes(1, 4096, 2048) >= 4
    assert L.quads_moe_route_workspace_bytes(16384, 64) >= 64 * 64 * 4


def _nv(rows, cols, batch=1, ptr=16):
    return _lib._NVFP4(ptr, ptr, ptr, batch, rows, cols)


def test_quantize_validation(L):
    dummy = ctypes.c_void_p(16)
    st = L.quads_quantize_nvfp4(dummy, 0, _nv(4, 10), 0, None, dummy, 1 << 20, None)
    assert st == -2 and b"multiple of 16" in L.quads_last_error()
    assert L.quads_quantize_nvfp4(dummy, 7, _nv(4, 16), 0, None, dummy, 1 << 20, None) == -1
    assert L.quads_quantize_nvfp4(None, 0, _nv(4, 16), 0, None, dummy, 1 << 20, None) == -1
    assert L.quads_quantize_nvfp4(dummy, 0, _nv(4, 16), 0, None, None, 0, None) == -3
    # scores need batch == 1
    assert L.quads_quantize_nvfp4(dummy, 0, _nv(4, 16, batch=2), 2, dummy, dummy, 1 << 20, None) == -1
    assert L.quads_quantize_nvfp4(dummy, 0, _nv(4, 16), 1 << 7, None, dummy, 1 << 20, None) == -1
    # zero rows still write the tensor scale (a GPU test checks the values),
    # so a NULL gscale is rejected before anything is enqueued
    assert L.quads_quantize_nvfp4(None, 0, _lib._NVFP4(None, None, None, 1, 0, 16), 0, None, None, 0, None) == -1
    assert b"gscale" in L.quads_last_error()
    # misaligned arrays are rejected before anything is enqueued
    st = L.quads_quantize_nvfp4(ctypes.c_void_p(24), 0, _nv(4, 16), 0, None, dummy, 1 << 20, None)
    assert st == -1 and b"aligned" in L.quads_last_error()
    assert L.quads_quantize_nvfp4(dummy, 0, _nv(4, 16, ptr=8), 0, None, dummy, 1 << 20, None) == -1


def test_rac_select_validation(L):
    dummy = ctypes.c_void_p(16)
    xq = _nv(8, 256)
    assert L.quads_rac_select(dummy, 0, ctypes.byref(xq), dummy, 101, dummy, _nv(8, 0), None, 0, None) == -1
    assert L.quads_rac_select(dummy, 0, ctypes.byref(xq), dummy, 50, dummy, _nv(8, 64), None, 0, None) == -2
    big = _nv(8, 32768)
    assert L.quads_rac_select(dummy, 0, ctypes.byref(big), dummy, 50, dummy, _nv(8, 16384), None, 0, None) == -2
    assert L.quads_rac_select(dummy, 0, None, dummy, 50, dummy, _nv(8, 128), None, 0, None) == -1
    st = L.quads_rac_select(ctypes.c_void_p(40), 0, ctypes.byref(xq), dummy, 50, dummy, _nv(8, 128), None, 0, None)
    assert st == -1 and b"aligned" in L.quads_last_error()
    # channel limit 16384 (a row of FP32 residuals and the mask in one workgroup's LDS), both forms
    wide = _nv(8, 16400)
    assert L.quads_rac_select(dummy, 0, ctypes.byref(wide), dummy, 0, dummy, _nv(8, 0), None, 0, None) == -2
    assert L.quads_rac_select_merged(dummy, 0, ctypes.byref(wide), dummy, 50, dummy, _nv(8, 8208), dummy,
                                     None, 0, None) == -2


def test_quantize_noalloc_validation(L):
    """The no-allocation quantizer checks its arguments like the workspace
    form and rejects calls whose amax partials exceed its fixed 1 MiB scratch
    before enqueueing anything."""
    dummy = ctypes.c_void_p(16)
    assert L.quads_quantize_nvfp4_noalloc(dummy, 0, _nv(4, 10), 0, None, None) == -2
    assert L.quads_quantize_nvfp4_noalloc(dummy, 7, _nv(4, 16), 0, None, None) == -1
    assert L.quads_quantize_nvfp4_noalloc(None, 0, _nv(4, 16), 0, None, None) == -1
    assert L.quads_quantize_nvfp4_noalloc(dummy, 0, _nv(4, 16, batch=2), 2, dummy, None) == -1
    # 300 matrices of 4096 x 4096: 1024 partials each, 1.2 MB > 1 MiB
    assert L.quads_quantize_nvfp4_noalloc(dummy, 1, _nv(4096, 4096, batch=300), 0, None, None) == -3
    assert b"scratch" in L.quads_last_error()
    assert L.quads_quantize_nvfp4_noalloc(None, 1, _lib._NVFP4(None, None, None, 1, 0, 4096), 0, None, None) == -1


def _gemm_args(**kw):
    a = _lib._GemmArgs()
    a.struct_size = ctypes.sizeof(_lib._GemmArgs)
    a.num_experts, a.n_seg, a.num_rows, a.act_rows, a.N, a.K = 1, 1, 64, 64, 128, 256
    for p in ("x_codes", "x_scales", "x_gscale", "w_codes", "w_scales", "w_gscale", "expert_offsets", "y"):
        setattr(a, p, 16)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_gemm_validation(L):
    ok = _gemm_args()
    assert L.quads_moe_gemm_workspace_bytes(ctypes.byref(ok)) > 0
    assert L.quads_moe_w4a4_gemm(ctypes.byref(ok), None) == -3  # no workspace
    cases = [
        (dict(struct_size=8), -1), (dict(operand_mode=5), -1), (dict(epilogue=3), -1),
        (dict(K=100), -2), (dict(N=96), -2), (dict(num_experts=0), -2), (dict(n_seg=3), -2),
        (dict(epilogue=1, n_seg=1), -2), (dict(y=None), -1), (dict(w_codes=None), -1),
        (dict(act_rows=8, row_token=None), -2), (dict(r_codes=16, kpad=40), -2), (dict(N=192), -2),
        (dict(rac_form=3), -1), (dict(rac_form=-1), -1), (dict(rac_form=1, x_merged=16), -1),
    ]
    for kw, want in cases:
        a = _gemm_args(**kw)
        assert L.quads_moe_w4a4_gemm(ctypes.byref(a), None) == want, kw
        assert L.quads_last_error() != b""


def test_gemm_y_gscale_field(L):
    """The output tensor scale is formed only for the W4A4 GEMM's bf16 output
    (SwiGLU or y_dtype BF16) and costs 256 workspace bytes (its two words)."""
    base = L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(y_dtype=1)))
    assert L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(y_dtype=1, y_gscale=16))) == base + 256
    for kw in (dict(y_gscale=16), dict(y_gscale=16, operand_mode=1, x_bf16=16, w_bf16=16, y_dtype=1)):
        a = _gemm_args(**kw)
        assert L.quads_moe_w4a4_gemm(ctypes.byref(a), None) == -1 and b"y_gscale" in L.quads_last_error()
    assert L.quads_moe_w4a4_gemm(ctypes.byref(_gemm_args(epilogue=1, n_seg=2, y_gscale=16)), None) == -3


def test_gemm_rac_form_field(L):
    """The RAC formulation is an explicit argument (no environment or other
    hidden input): the workspace holds the gathered weight columns
    (E*N*kpad fp16) for the exact form and the merged activation
    (act_rows*K fp16) for the merged form, whatever the process environment."""
    res = dict(r_codes=16, r_scales=16, r_gscale=16, sel_idx=16, kpad=128, num_rows=4096, act_rows=4096,
               N=1536, K=2048)
    exact = L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(rac_form=1, **res)))
    merged = L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(rac_form=2, **res)))
    auto = L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(rac_form=0, **res)))
    assert exact >= 1536 * 128 * 2 and exact < 4096 * 2048 * 2
    assert merged >= 4096 * 2048 * 2
    assert auto == exact  # 128x128 DMA-staged tiles: the exact form by default
    given = L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(rac_form=0, x_merged=16, **res)))
    assert given < 4096  # the caller's merged operand: only the tile list
    # the merge step holds a row of K floats and the mask on chip: K = 32768 does
    # not fit, so MERGED without x_merged is rejected and AUTO keeps the exact form
    big = dict(num_rows=64, act_rows=64, N=128, K=32768, r_codes=16, r_scales=16, r_gscale=16, sel_idx=16, kpad=16384)
    a = _gemm_args(rac_form=2, **big)
    assert L.quads_moe_w4a4_gemm(ctypes.byref(a), None) == -2 and b"merge step" in L.quads_last_error()
    assert L.quads_moe_gemm_workspace_bytes(ctypes.byref(_gemm_args(rac_form=0, **big))) >= 128 * 16384 * 2
    assert L.quads_moe_w4a4_gemm(ctypes.byref(_gemm_args(rac_form=2, x_merged=16, **big)), None) == -3


def test_gemm_32bit_offset_limit(L):
    """The register-staged NVFP4 kernels address the activation tensor through
    32-bit byte offsets; a larger W4A4 activation runs on the DMA-staged kernel,
    which needs K % 128 == 0 (and kpad % 64 == 0 with a residual), and is
    rejected as a shape error otherwise."""
    rows = dict(num_rows=65536, act_rows=1 << 21)  # 2^21 rows x K/2 bytes >= 4 GiB
    bad = _gemm_args(K=4112, **rows)
    assert L.quads_moe_gemm_workspace_bytes(ctypes.byref(bad)) == 0
    assert L.quads_moe_w4a4_gemm(ctypes.byref(bad), None) == -2 and b"4 GiB" in L.quads_last_error()
    good = _gemm_args(K=4224, **rows)
    assert L.quads_moe_gemm_workspace_bytes(ctypes.byref(good)) > 0
    assert L.quads_moe_w4a4_gemm(ctypes.byref(good), None) == -3  # accepted; no workspace
    # below the limit any multiple of 16 is accepted
    small = _gemm_args(K=4112, num_rows=65536, act_rows=65536)
    assert L.quads_moe_w4a4_gemm(ctypes.byref(small), None) == -3
    # with a residual the DMA kernel also needs kpad % 64 == 0
    res = dict(r_codes=16, r_scales=16, r_gscale=16, sel_idx=16, rac_form=1, **rows)
    assert L.quads_moe_w4a4_gemm(ctypes.byref(_gemm_args(K=4224, kpad=48, **res)), None) == -2
    assert L.quads_moe_w4a4_gemm(ctypes.byref(_gemm_args(K=4224, kpad=64, **res)), None) == -3


def test_qdq_route_combine_validation(L):
    dummy = ctypes.c_void_p(16)
    assert L.quads_weight_qdq(dummy, 1, 4, 24, dummy, None, 0, dummy, 1 << 20, None) == -2
    assert L.quads_weight_qdq(dummy, 1, 4, 32, dummy, None, 1, dummy, 1 << 20, None) == -1
    assert L.quads_moe_route(dummy, 16, 2000, 8, dummy, dummy, dummy, dummy, dummy, dummy, 1 << 20, None) == -2
    assert L.quads_moe_route(dummy, 16, 64, 17, dummy, dummy, dummy, dummy, dummy, dummy, 1 << 20, None) == -2
    assert L.quads_moe_route(dummy, 16, 64, 8, dummy, dummy, dummy, dummy, dummy, None, 0, None) == -3
    assert L.quads_moe_combine(dummy, 4, 8, 6, dummy, dummy, dummy, None) == -2
