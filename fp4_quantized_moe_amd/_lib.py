"""ctypes binding of libquads (include/quads.h).

Argument marshalling only: every step of the hot path runs in the HIP
library.  PyTorch provides device memory (torch.empty on the GPU) and the
current HIP stream.  If the library is missing or a call fails, an exception
is raised -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libquads.so")

F32, BF16 = 0, 1
GSCALE_GIVEN, WANT_SCORES = 1, 2
OPERANDS_W4A4, OPERANDS_BF16, OPERANDS_BF16_QDQ, OPERANDS_BF16_W4 = 0, 1, 2, 3
SCALES_ONLY = 4
EPI_NONE, EPI_SWIGLU = 0, 1
RAC_FORM_AUTO, RAC_FORM_EXACT, RAC_FORM_MERGED = 0, 1, 2

_c_i64, _c_i32, _c_u32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p


class QuadsError(RuntimeError):
    pass


class _NVFP4(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("gscale", _vp),
                ("batch", _c_i64), ("rows", _c_i64), ("cols", _c_i64)]


class _GemmArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _c_u32), ("flags", _c_u32), ("operand_mode", _c_i32), ("epilogue", _c_i32), ("y_dtype", _c_i32),
        ("num_experts", _c_i32), ("n_seg", _c_i32),
        ("num_rows", _c_i64), ("act_rows", _c_i64), ("N", _c_i64), ("K", _c_i64),
        ("x_codes", _vp), ("x_scales", _vp), ("x_gscale", _vp),
        ("r_codes", _vp), ("r_scales", _vp), ("r_gscale", _vp), ("sel_idx", _vp), ("kpad", _c_i64),
        ("w_codes", _vp), ("w_scales", _vp), ("w_gscale", _vp),
        ("x_bf16", _vp), ("w_bf16", _vp),
        ("row_token", _vp), ("expert_offsets", _vp),
        ("y", _vp), ("ws", _vp), ("ws_bytes", ctypes.c_size_t), ("x_merged", _vp), ("rac_form", _c_i32),
        ("y_gscale", _vp),
    ]


EXPORTS = [
    "quads_last_error", "quads_version", "quads_rac_nsel", "quads_rac_kpad",
    "quads_quantize_workspace_bytes", "quads_quantize_nvfp4", "quads_quantize_nvfp4_noalloc",
    "quads_rac_select_workspace_bytes", "quads_rac_select", "quads_rac_select_merged",
    "quads_moe_gemm_workspace_bytes", "quads_moe_w4a4_gemm", "quads_moe_gemm_prepare",
    "quads_weight_qdq_workspace_bytes", "quads_weight_qdq",
    "quads_moe_route_workspace_bytes", "quads_moe_route", "quads_moe_combine",
    "quads_moe_wgrad_workspace_bytes", "quads_moe_wgrad_bf16", "quads_transpose_bf16",
]

_lib = None


def load(path: str = LIB_PATH):
    """Load libquads.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise QuadsError(f"{path} not found: build it with `python -m fp4_quantized_moe_amd.build`")
    L = ctypes.CDLL(path)
    L.quads_last_error.restype = ctypes.c_char_p
    L.quads_version.restype = ctypes.c_char_p
    L.quads_rac_nsel.restype = _c_i64
    L.quads_rac_nsel.argtypes = [_c_i64, _c_i32]
    L.quads_rac_kpad.restype = _c_i64
    L.quads_rac_kpad.argtypes = [_c_i64]
    L.quads_quantize_workspace_bytes.restype = ctypes.c_size_t
    L.quads_quantize_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64]
    L.quads_quantize_nvfp4.restype = ctypes.c_int
    L.quads_quantize_nvfp4.argtypes = [_vp, ctypes.c_int, _NVFP4, _c_u32, _vp, _vp, ctypes.c_size_t, _vp]
    L.quads_quantize_nvfp4_noalloc.restype = ctypes.c_int
    L.quads_quantize_nvfp4_noalloc.argtypes = [_vp, ctypes.c_int, _NVFP4, _c_u32, _vp, _vp]
    L.quads_rac_select_workspace_bytes.restype = ctypes.c_size_t
    L.quads_rac_select_workspace_bytes.argtypes = [_c_i64, _c_i64]
    L.quads_rac_select.restype = ctypes.c_int
    L.quads_rac_select.argtypes = [_vp, ctypes.c_int, ctypes.POINTER(_NVFP4), _vp, _c_i32, _vp, _NVFP4,
                                   _vp, ctypes.c_size_t, _vp]
    L.quads_rac_select_merged.restype = ctypes.c_int
    L.quads_rac_select_merged.argtypes = [_vp, ctypes.c_int, ctypes.POINTER(_NVFP4), _vp, _c_i32, _vp, _NVFP4, _vp,
                                          _vp, ctypes.c_size_t, _vp]
    L.quads_moe_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.quads_moe_gemm_workspace_bytes.argtypes = [ctypes.POINTER(_GemmArgs)]
    L.quads_moe_w4a4_gemm.restype = ctypes.c_int
    L.quads_moe_w4a4_gemm.argtypes = [ctypes.POINTER(_GemmArgs), _vp]
    L.quads_moe_gemm_prepare.restype = ctypes.c_int
    L.quads_moe_gemm_prepare.argtypes = [ctypes.POINTER(_GemmArgs), _vp]
    L.quads_weight_qdq_workspace_bytes.restype = ctypes.c_size_t
    L.quads_weight_qdq_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64]
    L.quads_weight_qdq.restype = ctypes.c_int
    L.quads_weight_qdq.argtypes = [_vp, _c_i64, _c_i64, _c_i64, _vp, ctypes.POINTER(_NVFP4), _c_u32, _vp,
                                   ctypes.c_size_t, _vp]
    L.quads_moe_route_workspace_bytes.restype = ctypes.c_size_t
    L.quads_moe_route_workspace_bytes.argtypes = [_c_i64, _c_i32]
    L.quads_moe_route.restype = ctypes.c_int
    L.quads_moe_route.argtypes = [_vp, _c_i64, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.quads_moe_combine.restype = ctypes.c_int
    L.quads_moe_combine.argtypes = [_vp, _c_i64, _c_i32, _c_i64, _vp, _vp, _vp, _vp]
    L.quads_moe_wgrad_workspace_bytes.restype = ctypes.c_size_t
    L.quads_moe_wgrad_workspace_bytes.argtypes = [_c_i64, _c_i32, _c_i64, _c_i64]
    L.quads_moe_wgrad_bf16.restype = ctypes.c_int
    L.quads_moe_wgrad_bf16.argtypes = [_vp, _vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp,
                                       ctypes.c_size_t, _vp]
    L.quads_transpose_bf16.restype = ctypes.c_int
    L.quads_transpose_bf16.argtypes = [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp]
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        msg = load().quads_last_error().decode()
        raise QuadsError(f"{what} failed with status {status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise QuadsError(f"unsupported dtype {t.dtype}")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise QuadsError("tensors must be contiguous and on the GPU")


def _check_route_args(logits):
    _require_cuda(logits)
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise QuadsError("moe_route expects float32 logits [T, E]")


def _check_combine_args(y, inverse, topk_w):
    _require_cuda(y, inverse, topk_w)
    if y.dtype != torch.float32 or y.dim() != 2:
        raise QuadsError("moe_combine expects float32 y [T*top, N]")
    if inverse.dtype != torch.int32 or inverse.dim() != 2:
        raise QuadsError("moe_combine expects int32 inverse [T, top]")
    if topk_w.dtype != torch.float32 or tuple(topk_w.shape) != tuple(inverse.shape):
        raise QuadsError("moe_combine expects float32 topk_w of inverse's shape [T, top]")
    if y.shape[0] != inverse.numel():
        raise QuadsError(f"moe_combine: y has {y.shape[0]} rows, expected T*top = {inverse.numel()}")


def _workspace(nbytes: int, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@dataclass
class NVFP4Tensor:
    """Packed codes [batch, rows, cols/2] u8, E4M3 scales [batch, rows, cols/16]
    u8 and FP32 tensor scales [batch] (batch axis omitted when batch == 1)."""
    codes: torch.Tensor
    scales: torch.Tensor
    gscale: torch.Tensor
    batch: int
    rows: int
    cols: int

    def c_struct(self):
        return _NVFP4(self.codes.data_ptr(), self.scales.data_ptr(), self.gscale.data_ptr(),
                      self.batch, self.rows, self.cols)


def empty_nvfp4(batch, rows, cols, device):
    shape = (rows,) if batch == 1 else (batch, rows)
    return NVFP4Tensor(torch.empty(*shape, cols // 2, dtype=torch.uint8, device=device),
                       torch.empty(*shape, cols // 16, dtype=torch.uint8, device=device),
                       torch.empty(batch, dtype=torch.float32, device=device), batch, rows, cols)


def rac_nsel(cols: int, k_percent: int) -> int:
    return int(load().quads_rac_nsel(cols, k_percent))


def rac_kpad(nsel: int) -> int:
    return int(load().quads_rac_kpad(nsel))


class QuantizeCall:
    """quads_quantize_nvfp4 with output buffers and workspace allocated once.
    x: [rows, cols] or [batch, rows, cols] (bf16/fp32).  `gscale` copies given
    tensor scales once; `gscale_given=True` uses whatever self.q.gscale holds
    at each call (e.g. a GEMM's y_gscale written just before)."""

    def __init__(self, x: torch.Tensor, want_scores: bool = False, gscale: torch.Tensor | None = None,
                 out: NVFP4Tensor | None = None, gscale_given: bool = False):
        L = load()
        _require_cuda(x)
        self.x = x
        batch, rows, cols = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
        self.q = out if out is not None else empty_nvfp4(batch, rows, cols, x.device)
        self.flags = 0
        if gscale is not None:
            self.q.gscale.copy_(gscale.reshape(-1))
            self.flags |= GSCALE_GIVEN
        elif gscale_given:  # self.q.gscale is filled by another call (e.g. a GEMM's y_gscale) before each use
            self.flags |= GSCALE_GIVEN
        self.scores = None
        if want_scores:
            self.scores = torch.empty(cols, dtype=torch.float32, device=x.device)
            self.flags |= WANT_SCORES
        self.ws = _workspace(L.quads_quantize_workspace_bytes(batch, rows, cols), x.device)
        self._st = self.q.c_struct()
        self._dt = _dtype_code(x)

    def __call__(self):
        _check(load().quads_quantize_nvfp4(_ptr(self.x), self._dt, self._st, self.flags, _ptr(self.scores),
                                           _ptr(self.ws), self.ws.numel(), _stream()), "quads_quantize_nvfp4")
        return self.q, self.scores


def quantize_nvfp4(x: torch.Tensor, want_scores: bool = False, gscale: torch.Tensor | None = None,
                   out: NVFP4Tensor | None = None):
    """-> (NVFP4Tensor, scores or None)."""
    return QuantizeCall(x, want_scores, gscale, out)()


class SelectCall:
    """quads_rac_select with sel_idx and the residual tensor allocated once;
    with merged=True quads_rac_select_merged, which also writes the
    RAC-merged fp16 activation `self.merged` [rows, cols]."""

    def __init__(self, x: torch.Tensor, xq: NVFP4Tensor, scores: torch.Tensor, k_percent: int,
                 merged: bool = False):
        _require_cuda(x, scores)
        rows, cols = xq.rows, xq.cols
        self.nsel = rac_nsel(cols, k_percent)
        if self.nsel < 0:
            raise QuadsError(f"invalid k_percent {k_percent}")
        kpad = rac_kpad(self.nsel)
        dev = x.device
        self.sel = torch.empty(max(kpad, 1), dtype=torch.int32, device=dev)
        self.res = empty_nvfp4(1, rows, kpad, dev) if kpad else NVFP4Tensor(
            torch.empty(rows, 0, dtype=torch.uint8, device=dev), torch.empty(rows, 0, dtype=torch.uint8, device=dev),
            torch.empty(1, dtype=torch.float32, device=dev), 1, rows, 0)
        self.x, self.xq, self.scores, self.k = x, xq, scores, k_percent
        self._xs = xq.c_struct()
        self._rs = self.res.c_struct()
        self._dt = _dtype_code(x)
        self.kpad = kpad
        self.merged = torch.empty(rows, cols, dtype=torch.float16, device=dev) if merged else None

    def __call__(self):
        if self.merged is not None:
            _check(load().quads_rac_select_merged(_ptr(self.x), self._dt, ctypes.byref(self._xs), _ptr(self.scores),
                                                  self.k, _ptr(self.sel), self._rs, _ptr(self.merged), None, 0,
                                                  _stream()), "quads_rac_select_merged")
        else:
            _check(load().quads_rac_select(_ptr(self.x), self._dt, ctypes.byref(self._xs), _ptr(self.scores), self.k,
                                           _ptr(self.sel), self._rs, None, 0, _stream()), "quads_rac_select")
        return self.sel[:self.kpad], self.res, self.nsel


def rac_select(x: torch.Tensor, xq: NVFP4Tensor, scores: torch.Tensor, k_percent: int):
    """-> (sel_idx int32 [kpad], residual NVFP4Tensor [rows, kpad], nsel)."""
    return SelectCall(x, xq, scores, k_percent)()


class GemmCall:
    """One grouped-GEMM call with its arguments and workspace built once.

    W4A4 mode when `x` is given, bf16-operand (trainer W4A16) mode when
    `x_bf16`/`w_bf16` are given; with `qdq=True` the bf16 weights are the
    masters, fake-quantized inside the GEMM with their tensor scales
    `w_gscale` (QUADS_OPERANDS_BF16_QDQ); with `x_bf16` and NVFP4 weights
    (`w_codes`, `w_scales`, `w_gscale`) the weights are decoded to their QDQ
    bf16 values inside the GEMM (QUADS_OPERANDS_BF16_W4).  `rac_form` (RAC_FORM_AUTO /
    _EXACT / _MERGED) picks the formulation of the RAC correction, see
    quads.h.  ``y_gscale`` (float32 [1], device) receives the NVFP4 tensor
    scale of the bf16 output, formed by the GEMM (hand it to a QuantizeCall
    with ``gscale_given=True``).  ``prepare()`` + ``run()`` is the split form
    (tile list and residual weight-column gather, then the GEMM kernel);
    calling the object does both."""

    def __init__(self, *, w_codes=None, w_scales=None, w_gscale=None, n_seg=1, N, K,
                 expert_offsets, num_rows, x: NVFP4Tensor | None = None, res: NVFP4Tensor | None = None,
                 sel_idx=None, row_token=None, epilogue=EPI_NONE, y_dtype=torch.float32,
                 x_bf16=None, w_bf16=None, y=None, x_merged=None, rac_form=RAC_FORM_AUTO, qdq=False,
                 y_gscale=None):
        L = load()
        E = int(expert_offsets.numel()) - 1
        bf16_mode = x_bf16 is not None and w_bf16 is not None
        w4_mode = x_bf16 is not None and w_bf16 is None
        dev = expert_offsets.device
        if y is None:
            if epilogue == EPI_SWIGLU:
                y = torch.empty(num_rows, N // 2, dtype=torch.bfloat16, device=dev)
            else:
                y = torch.empty(num_rows, N, dtype=y_dtype, device=dev)
        self.y = y
        self._keep = [w_codes, w_scales, w_gscale, expert_offsets, x, res, sel_idx, row_token, x_bf16, w_bf16, x_merged,
                      y_gscale]
        a = _GemmArgs()
        a.struct_size = ctypes.sizeof(_GemmArgs)
        a.operand_mode = ((OPERANDS_BF16_QDQ if qdq else OPERANDS_BF16) if bf16_mode else
                          OPERANDS_BF16_W4 if w4_mode else OPERANDS_W4A4)
        a.epilogue = epilogue
        a.y_dtype = BF16 if y.dtype == torch.bfloat16 else F32
        a.num_experts = E
        a.n_seg = n_seg
        a.num_rows = num_rows
        a.N, a.K = N, K
        a.rac_form = rac_form
        if bf16_mode:
            _require_cuda(x_bf16, w_bf16)
            if x_bf16.dtype != torch.bfloat16 or w_bf16.dtype != torch.bfloat16:
                raise QuadsError("bf16-operand GEMM expects bf16 x_bf16 and w_bf16")
            a.act_rows = x_bf16.shape[0]
            a.x_bf16, a.w_bf16 = x_bf16.data_ptr(), w_bf16.data_ptr()
            if qdq:
                _require_cuda(w_gscale)
                if w_gscale.dtype != torch.float32 or w_gscale.numel() != E * n_seg:
                    raise QuadsError("qdq=True needs float32 w_gscale with one scale per (expert, segment)")
                a.w_gscale = w_gscale.data_ptr()
        elif w4_mode:
            _require_cuda(x_bf16, w_codes, w_scales, w_gscale)
            if x_bf16.dtype != torch.bfloat16 or w_gscale.dtype != torch.float32 or w_gscale.numel() != E * n_seg:
                raise QuadsError("BF16_W4 GEMM expects bf16 x_bf16 and float32 w_gscale [E * n_seg]")
            a.act_rows = x_bf16.shape[0]
            a.x_bf16 = x_bf16.data_ptr()
            a.w_codes, a.w_scales, a.w_gscale = w_codes.data_ptr(), w_scales.data_ptr(), w_gscale.data_ptr()
        else:
            a.act_rows = x.rows
            a.x_codes, a.x_scales, a.x_gscale = x.codes.data_ptr(), x.scales.data_ptr(), x.gscale.data_ptr()
            a.w_codes, a.w_scales, a.w_gscale = w_codes.data_ptr(), w_scales.data_ptr(), w_gscale.data_ptr()
            if res is not None and res.cols > 0:
                a.r_codes, a.r_scales, a.r_gscale = res.codes.data_ptr(), res.scales.data_ptr(), res.gscale.data_ptr()
                a.sel_idx = sel_idx.data_ptr()
                a.kpad = res.cols
                if x_merged is not None:
                    _require_cuda(x_merged)
                    a.x_merged = x_merged.data_ptr()
        if y_gscale is not None:
            _require_cuda(y_gscale)
            if y_gscale.dtype != torch.float32 or y_gscale.numel() < 1:
                raise QuadsError("y_gscale must be a float32 device tensor with at least one element")
            a.y_gscale = y_gscale.data_ptr()
        a.row_token = None if row_token is None else row_token.data_ptr()
        a.expert_offsets = expert_offsets.data_ptr()
        a.y = y.data_ptr()
        nbytes = L.quads_moe_gemm_workspace_bytes(ctypes.byref(a))
        if nbytes == 0:  # invalid arguments: let the library report why
            _check(L.quads_moe_w4a4_gemm(ctypes.byref(a), None), "quads_moe_w4a4_gemm")
        self.ws = _workspace(nbytes, dev)
        a.ws, a.ws_bytes = self.ws.data_ptr(), self.ws.numel()
        self.args = a
        self.flops_k = K + (a.kpad if a.r_codes else 0)

    def prepare(self):
        _check(load().quads_moe_gemm_prepare(ctypes.byref(self.args), _stream()), "quads_moe_gemm_prepare")

    def run(self):
        """Main GEMM kernel only (after prepare())."""
        self.args.flags = 1
        _check(load().quads_moe_w4a4_gemm(ctypes.byref(self.args), _stream()), "quads_moe_w4a4_gemm")

    def __call__(self):
        self.args.flags = 0
        _check(load().quads_moe_w4a4_gemm(ctypes.byref(self.args), _stream()), "quads_moe_w4a4_gemm")
        return self.y


def moe_w4a4_gemm(**kw):
    """Grouped expert GEMM (see quads.h); returns y."""
    return GemmCall(**kw)()


class QdqCall:
    """quads_weight_qdq with its output and workspace allocated once (or the
    output given): w bf16 [rows, cols] or [batch, rows, cols]."""

    def __init__(self, w: torch.Tensor, out: torch.Tensor | None = None, export: bool = False):
        L = load()
        _require_cuda(w, out)
        if w.dtype != torch.bfloat16 or (out is not None and (out.dtype != torch.bfloat16 or out.shape != w.shape)):
            raise QuadsError("weight_qdq expects bf16 master weights and a bf16 output of the same shape")
        self.w = w
        self.batch, self.rows, self.cols = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
        self.out = torch.empty_like(w) if out is None else out
        self.q = empty_nvfp4(self.batch, self.rows, self.cols, w.device) if export else None
        self._qs = self.q.c_struct() if self.q is not None else None
        self.ws = _workspace(L.quads_weight_qdq_workspace_bytes(self.batch, self.rows, self.cols), w.device)

    def __call__(self):
        _check(load().quads_weight_qdq(_ptr(self.w), self.batch, self.rows, self.cols, _ptr(self.out),
                                       ctypes.byref(self._qs) if self._qs is not None else None, 0, _ptr(self.ws),
                                       self.ws.numel(), _stream()), "quads_weight_qdq")
        return self.out, self.q


class ScalesCall:
    """quads_weight_qdq with QUADS_SCALES_ONLY: the FP32 tensor scale of each
    of the bf16 master matrices w ([rows, cols] or [batch, rows, cols]) into
    `self.gscale` [batch] -- the input of the fused-QDQ GEMM."""

    def __init__(self, w: torch.Tensor, gscale: torch.Tensor | None = None):
        L = load()
        _require_cuda(w, gscale)
        if w.dtype != torch.bfloat16:
            raise QuadsError("weight scales expect bf16 master weights")
        self.w = w
        self.batch, self.rows, self.cols = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
        self.gscale = torch.empty(self.batch, dtype=torch.float32, device=w.device) if gscale is None else gscale
        self._qs = _NVFP4(None, None, self.gscale.data_ptr(), self.batch, self.rows, self.cols)
        self.ws = _workspace(L.quads_weight_qdq_workspace_bytes(self.batch, self.rows, self.cols), w.device)

    def __call__(self):
        _check(load().quads_weight_qdq(_ptr(self.w), self.batch, self.rows, self.cols, None, ctypes.byref(self._qs),
                                       SCALES_ONLY, _ptr(self.ws), self.ws.numel(), _stream()), "quads_weight_qdq")
        return self.gscale


def weight_scales(w: torch.Tensor):
    """Tensor scale of each bf16 master matrix (QUADS_SCALES_ONLY)."""
    return ScalesCall(w)()


def weight_qdq(w: torch.Tensor, export: bool = False):
    """w: bf16 [rows, cols] or [batch, rows, cols] -> (bf16 QDQ tensor, NVFP4Tensor or None)."""
    L = load()
    _require_cuda(w)
    if w.dtype != torch.bfloat16:
        raise QuadsError("weight_qdq expects bf16 master weights")
    batch, rows, cols = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    out = torch.empty_like(w)
    q = empty_nvfp4(batch, rows, cols, w.device) if export else None
    qs = q.c_struct() if q is not None else None
    ws = _workspace(L.quads_weight_qdq_workspace_bytes(batch, rows, cols), w.device)
    _check(L.quads_weight_qdq(_ptr(w), batch, rows, cols, _ptr(out), ctypes.byref(qs) if qs is not None else None,
                              0, _ptr(ws), ws.numel(), _stream()), "quads_weight_qdq")
    return out, q


class RouteCall:
    """quads_moe_route with its outputs and workspace allocated once."""

    def __init__(self, logits: torch.Tensor, top: int):
        L = load()
        _check_route_args(logits)
        T, E = logits.shape
        dev = logits.device
        self.logits, self.T, self.E, self.top = logits, T, E, top
        self.ids = torch.empty(T, top, dtype=torch.int32, device=dev)
        self.w = torch.empty(T, top, dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.row_token = torch.empty(max(T * top, 1), dtype=torch.int32, device=dev)
        self.inverse = torch.empty(T, top, dtype=torch.int32, device=dev)
        self.ws = _workspace(L.quads_moe_route_workspace_bytes(T, E), dev)

    def __call__(self):
        _check(load().quads_moe_route(_ptr(self.logits), self.T, self.E, self.top, _ptr(self.ids), _ptr(self.w),
                                      _ptr(self.offsets), _ptr(self.row_token), _ptr(self.inverse), _ptr(self.ws),
                                      self.ws.numel(), _stream()), "quads_moe_route")
        return self.ids, self.w, self.offsets, self.row_token[:self.T * self.top], self.inverse


class CombineCall:
    """quads_moe_combine with its output allocated once."""

    def __init__(self, y: torch.Tensor, inverse: torch.Tensor, topk_w: torch.Tensor):
        _check_combine_args(y, inverse, topk_w)
        self.y, self.inverse, self.w = y, inverse, topk_w
        self.T, self.top = inverse.shape
        self.N = y.shape[1]
        self.out = torch.empty(self.T, self.N, dtype=torch.float32, device=y.device)

    def __call__(self):
        _check(load().quads_moe_combine(_ptr(self.y), self.T, self.top, self.N, _ptr(self.inverse), _ptr(self.w),
                                        _ptr(self.out), _stream()), "quads_moe_combine")
        return self.out


def moe_route(logits: torch.Tensor, top: int):
    """-> (topk_ids [T, top] i32, topk_w [T, top] f32, expert_offsets [E+1] i32,
    row_token [T*top] i32, inverse [T, top] i32)."""
    L = load()
    _check_route_args(logits)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty(T, top, dtype=torch.int32, device=dev)
    w = torch.empty(T, top, dtype=torch.float32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(max(T * top, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(T, top, dtype=torch.int32, device=dev)
    ws = _workspace(L.quads_moe_route_workspace_bytes(T, E), dev)
    _check(L.quads_moe_route(_ptr(logits), T, E, top, _ptr(ids), _ptr(w), _ptr(offs), _ptr(rt), _ptr(inv),
                             _ptr(ws), ws.numel(), _stream()), "quads_moe_route")
    return ids, w, offs, rt[:T * top], inv


def moe_combine(y: torch.Tensor, inverse: torch.Tensor, topk_w: torch.Tensor):
    L = load()
    _check_combine_args(y, inverse, topk_w)
    T, top = inverse.shape
    N = y.shape[1]
    out = torch.empty(T, N, dtype=torch.float32, device=y.device)
    _check(L.quads_moe_combine(_ptr(y), T, top, N, _ptr(inverse), _ptr(topk_w), _ptr(out), _stream()),
           "quads_moe_combine")
    return out


def transpose_bf16(x: torch.Tensor, out: torch.Tensor | None = None):
    """quads_transpose_bf16: bf16 [rows, cols] or [batch, rows, cols] -> the
    transposed matrices [.., cols, rows]."""
    _require_cuda(x)
    if x.dtype != torch.bfloat16:
        raise QuadsError("transpose_bf16 expects bf16")
    batch, rows, cols = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    if out is None:
        out = torch.empty(*x.shape[:-2], cols, rows, dtype=torch.bfloat16, device=x.device)
    _check(load().quads_transpose_bf16(_ptr(x), batch, rows, cols, _ptr(out), _stream()), "quads_transpose_bf16")
    return out


class WgradCall:
    """quads_moe_wgrad_bf16 with dw and the workspace allocated once:
    dw[e] = sum over the expert's routed rows i of dy[i]^T x[t(i)] (FP32)."""

    def __init__(self, dy: torch.Tensor, x: torch.Tensor, expert_offsets: torch.Tensor,
                 row_token: torch.Tensor | None = None, dw: torch.Tensor | None = None):
        L = load()
        _require_cuda(dy, x, expert_offsets, row_token, dw)
        if dy.dtype != torch.bfloat16 or x.dtype != torch.bfloat16:
            raise QuadsError("wgrad expects bf16 dy and x")
        self.R, self.N = dy.shape
        self.A, self.K = x.shape
        self.E = int(expert_offsets.numel()) - 1
        self.dy, self.x, self.offs, self.rt = dy, x, expert_offsets, row_token
        self.dw = torch.empty(self.E, self.N, self.K, dtype=torch.float32, device=dy.device) if dw is None else dw
        self.ws = _workspace(L.quads_moe_wgrad_workspace_bytes(self.R, self.E, self.N, self.K), dy.device)

    def __call__(self):
        _check(load().quads_moe_wgrad_bf16(_ptr(self.dy), _ptr(self.x), _ptr(self.rt), _ptr(self.offs), self.E,
                                           self.R, self.A, self.N, self.K, _ptr(self.dw), _ptr(self.ws),
                                           self.ws.numel(), _stream()), "quads_moe_wgrad_bf16")
        return self.dw


class QatBackward:
    """W4A16 QAT backward of the grouped linear y[i] = W_qdq[e(i)] . x[t(i)]
    (straight-through QDQ), composed of library calls:
      transpose W_qdq [E, N, K] -> [E, K, N];
      dxr = bf16-operand grouped GEMM of dy over W_qdq^T  (FP32 [R, K]);
      dx  = per-token sum of its routed rows (combine with unit weights),
            or dxr itself when rows are not gathered (row_token None);
      dw  = quads_moe_wgrad_bf16 (FP32 [E, N, K]).
    `inverse` [T, top] is the routed row of each (token, slot), needed with
    row_token."""

    def __init__(self, w_qdq: torch.Tensor, dy: torch.Tensor, x: torch.Tensor, expert_offsets: torch.Tensor,
                 row_token: torch.Tensor | None = None, inverse: torch.Tensor | None = None):
        E, N, K = w_qdq.shape
        self.w_qdq = w_qdq
        self.wt = torch.empty(E, K, N, dtype=torch.bfloat16, device=w_qdq.device)
        R = dy.shape[0]
        self.dxr_call = GemmCall(N=K, K=N, expert_offsets=expert_offsets, num_rows=R, x_bf16=dy, w_bf16=self.wt)
        self.combine = None
        if row_token is not None:
            if inverse is None:
                raise QuadsError("QatBackward: inverse is required with row_token")
            ones = torch.ones(inverse.shape, dtype=torch.float32, device=dy.device)
            self.combine = CombineCall(self.dxr_call.y, inverse, ones)
        self.wgrad = WgradCall(dy, x, expert_offsets, row_token)

    def stages(self):
        st = [("transpose_w", lambda: transpose_bf16(self.w_qdq, self.wt)), ("dx_gemm", self.dxr_call)]
        if self.combine is not None:
            st.append(("dx_token_sum", self.combine))
        st.append(("wgrad", self.wgrad))
        return st

    def __call__(self):
        for _, fn in self.stages():
            fn()
        dx = self.combine.out if self.combine is not None else self.dxr_call.y
        return dx, self.dxr_call.y, self.wgrad.dw
