"""MI355X (gfx950) RMSNorm forward/backward: Python binding of librmsnorm.so.

Argument marshalling only: every computation runs in the HIP kernels of the
C ABI declared in ``include/rmsnorm.h``.  The functions named ``rmsnorm_*``
mirror the C entry points one to one (tensors in place of pointers); ``fwd``
and ``bwd`` allocate their outputs like the page's ``forward_op`` and
``backward_rows`` + ``reduce_gamma_gradient`` launchers (page "Check an AI
model calculation before accelerating it", sections "Triton forward: one row,
one program" and "Reducing dgamma without a write race").

There is no fallback: if the library is missing, or an argument is outside
the contract, a ``RuntimeError`` (or ``ValueError`` for tensor checks) is
raised.  Build the library with ``python -m backward_rmsnorm_fwd_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RMSNORM_F32", "RMSNORM_F16", "RMSNORM_BF16", "RMSNORM_FLAG_OFFSET",
    "RMSNORM_FLAG_DGAMMA_IN_DTYPE",
    "RmsnormError", "library_path", "load_library", "rmsnorm_status_string",
    "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_rows", "rmsnorm_bwd_reduce",
    "rmsnorm_bwd_workspace_bytes", "rmsnorm_query_plan", "rmsnorm_fwd_strided",
    "rmsnorm_bwd_strided", "rmsnorm_bwd_noalloc", "NOALLOC_SCRATCH_BYTES", "row_layout", "fwd",
    "bwd", "EXPORTED_SYMBOLS",
    "layernorm_fwd", "layernorm_bwd", "layernorm_bwd_workspace_bytes", "layernorm_query_plan",
    "layernorm_bwd_rows", "layernorm_bwd_reduce", "ln_fwd", "ln_bwd", "LAYERNORM_MAX_N",
    "LAYERNORM_RESIDENT_MAX_N",
    "rmsnorm_add_fwd", "rmsnorm_add_bwd", "rmsnorm_add_bwd_workspace_bytes",
    "rmsnorm_add_query_plan", "rmsnorm_add_bwd_rows", "rmsnorm_add_bwd_reduce", "add_fwd",
    "add_bwd", "RMSNORM_ADD_MAX_N", "RMSNORM_ADD_RESIDENT_MAX_N",
    "rmsnorm_cast_fwd", "rmsnorm_cast_bwd", "rmsnorm_cast_bwd_workspace_bytes",
    "rmsnorm_cast_query_plan", "rmsnorm_cast_bwd_rows", "rmsnorm_cast_bwd_reduce", "cast_fwd",
    "cast_bwd", "RMSNORM_CAST_MAX_N", "RMSNORM_CAST_RESIDENT_MAX_N",
]

RMSNORM_F32, RMSNORM_F16, RMSNORM_BF16 = 0, 1, 2
RMSNORM_FLAG_OFFSET = 1
RMSNORM_FLAG_DGAMMA_IN_DTYPE = 2
PASS_FWD, PASS_BWD_ROWS, PASS_BWD_REDUCE = 0, 1, 2
KERNEL_NAMES = {1: "fwd_wave", 2: "fwd_block", 3: "bwd_wave", 4: "bwd_block",
                5: "bwd_reduce", 6: "fwd_rows", 7: "bwd_rows", 8: "bwd_reduce16",
                9: "fwd_pipe", 10: "bwd_pipe", 11: "bwd_long", 12: "fwd_split",
                13: "bwd_split", 14: "bwd_reduce_wide", 15: "ln_fwd",
                16: "ln_bwd", 17: "add_fwd", 18: "add_bwd", 19: "cast_fwd", 20: "cast_bwd",
                21: "ln_fwd_split", 22: "ln_bwd_split", 23: "add_fwd_split",
                24: "add_bwd_split", 25: "cast_fwd_split", 26: "cast_bwd_split",
                27: "add_fwd_long", 28: "add_bwd_long", 29: "ln_bwd_rows"}
LAYERNORM_MAX_N = 1 << 24
LAYERNORM_RESIDENT_MAX_N = 16384
RMSNORM_ADD_MAX_N = 1 << 24
RMSNORM_ADD_RESIDENT_MAX_N = 16384
RMSNORM_CAST_MAX_N = 1 << 24
RMSNORM_CAST_RESIDENT_MAX_N = 16384
MAX_N = 1 << 24  # RMSNORM_MAX_N: rows longer than 65536 take the split-row plan
NOALLOC_SCRATCH_BYTES = 72 << 20  # RMSNORM_NOALLOC_SCRATCH_BYTES

EXPORTED_SYMBOLS = (
    "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_rows", "rmsnorm_bwd_reduce",
    "rmsnorm_bwd_workspace_bytes", "rmsnorm_status_string", "rmsnorm_query_plan",
    "rmsnorm_fwd_strided", "rmsnorm_bwd_strided", "rmsnorm_bwd_noalloc",
    "layernorm_fwd", "layernorm_bwd", "layernorm_bwd_workspace_bytes", "layernorm_query_plan",
    "layernorm_bwd_rows", "layernorm_bwd_reduce",
    "rmsnorm_add_fwd", "rmsnorm_add_bwd", "rmsnorm_add_bwd_workspace_bytes",
    "rmsnorm_add_query_plan", "rmsnorm_add_bwd_rows", "rmsnorm_add_bwd_reduce",
    "rmsnorm_cast_fwd", "rmsnorm_cast_bwd", "rmsnorm_cast_bwd_workspace_bytes",
    "rmsnorm_cast_query_plan", "rmsnorm_cast_bwd_rows", "rmsnorm_cast_bwd_reduce",
)

_DTYPES = {torch.float32: RMSNORM_F32, torch.float16: RMSNORM_F16,
           torch.bfloat16: RMSNORM_BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class RmsnormError(RuntimeError):
    def __init__(self, func, status, text):
        super().__init__(f"{func}: status {status}: {text}")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("vec", ctypes.c_int32),
                ("threads_per_row", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("chunks", ctypes.c_int32), ("x_in_lds", ctypes.c_int32),
                ("weight_in_regs", ctypes.c_int32), ("dy_in_lds", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("partials", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int64), ("segments", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def as_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["kernel_name"] = KERNEL_NAMES.get(self.kernel, "?")
        return d


def library_path():
    return os.path.join(_HERE, "librmsnorm.so")


def load_library():
    """dlopen librmsnorm.so (once) and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m backward_rmsnorm_fwd_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, u32, f32, sz, i32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_size_t, ctypes.c_int)
    lib.rmsnorm_fwd.argtypes = [vp, vp, f32, i64, i64, i32, u32, vp, vp, vp]
    lib.rmsnorm_fwd.restype = i32
    lib.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, u32, vp, vp, vp, sz, vp]
    lib.rmsnorm_bwd.restype = i32
    lib.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i32, u32, vp, vp, vp]
    lib.rmsnorm_bwd_noalloc.restype = i32
    lib.rmsnorm_bwd_rows.argtypes = [vp, vp, vp, vp, i64, i64, i32, u32, vp, vp, sz, vp]
    lib.rmsnorm_bwd_rows.restype = i32
    lib.rmsnorm_bwd_reduce.argtypes = [vp, sz, i64, i64, i32, u32, vp, vp]
    lib.rmsnorm_bwd_reduce.restype = i32
    lib.rmsnorm_bwd_workspace_bytes.argtypes = [i64, i64, i32, u32]
    lib.rmsnorm_bwd_workspace_bytes.restype = sz
    lib.rmsnorm_status_string.argtypes = [i32]
    lib.rmsnorm_status_string.restype = ctypes.c_char_p
    lib.rmsnorm_query_plan.argtypes = [i64, i64, i32, u32, i32, i32, ctypes.POINTER(Plan)]
    lib.rmsnorm_query_plan.restype = i32
    lib.rmsnorm_fwd_strided.argtypes = [vp, i64, vp, f32, i64, i64, i32, u32, vp, i64, vp, vp]
    lib.rmsnorm_fwd_strided.restype = i32
    lib.rmsnorm_bwd_strided.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i32, u32, vp, i64,
                                        vp, vp, sz, vp]
    lib.rmsnorm_bwd_strided.restype = i32
    lib.layernorm_fwd.argtypes = [vp, i64, vp, vp, f32, i64, i64, i32, u32, vp, i64, vp, vp, vp]
    lib.layernorm_fwd.restype = i32
    lib.layernorm_bwd.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, i64, i32, u32, vp, i64,
                                  vp, vp, vp, sz, vp]
    lib.layernorm_bwd.restype = i32
    lib.layernorm_bwd_workspace_bytes.argtypes = [i64, i64, i32, u32]
    lib.layernorm_bwd_workspace_bytes.restype = sz
    lib.layernorm_query_plan.argtypes = [i64, i64, i32, u32, i32, i32, ctypes.POINTER(Plan)]
    lib.layernorm_query_plan.restype = i32
    lib.layernorm_bwd_rows.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, i64, i32, u32, vp, i64,
                                       vp, sz, vp]
    lib.layernorm_bwd_rows.restype = i32
    lib.layernorm_bwd_reduce.argtypes = [vp, sz, i64, i64, i32, u32, vp, vp, vp]
    lib.layernorm_bwd_reduce.restype = i32
    lib.rmsnorm_add_fwd.argtypes = [vp, i64, vp, i64, vp, f32, i64, i64, i32, u32, vp, i64, vp,
                                    i64, vp, vp]
    lib.rmsnorm_add_fwd.restype = i32
    lib.rmsnorm_add_bwd.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i64, i64, i32, u32, vp,
                                    i64, vp, vp, sz, vp]
    lib.rmsnorm_add_bwd.restype = i32
    lib.rmsnorm_add_bwd_workspace_bytes.argtypes = [i64, i64, i32, u32]
    lib.rmsnorm_add_bwd_workspace_bytes.restype = sz
    lib.rmsnorm_add_query_plan.argtypes = [i64, i64, i32, u32, i32, i32, ctypes.POINTER(Plan)]
    lib.rmsnorm_add_query_plan.restype = i32
    lib.rmsnorm_add_bwd_rows.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i64, i64, i32, u32,
                                         vp, i64, vp, sz, vp]
    lib.rmsnorm_add_bwd_rows.restype = i32
    lib.rmsnorm_add_bwd_reduce.argtypes = [vp, sz, i64, i64, i32, u32, vp, vp]
    lib.rmsnorm_add_bwd_reduce.restype = i32
    lib.rmsnorm_cast_fwd.argtypes = [vp, i64, vp, f32, i64, i64, i32, i32, u32, vp, i64, vp, vp]
    lib.rmsnorm_cast_fwd.restype = i32
    lib.rmsnorm_cast_bwd.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i32, i32, u32, vp, i64,
                                     vp, vp, sz, vp]
    lib.rmsnorm_cast_bwd.restype = i32
    lib.rmsnorm_cast_bwd_workspace_bytes.argtypes = [i64, i64, i32, i32, u32]
    lib.rmsnorm_cast_bwd_workspace_bytes.restype = sz
    lib.rmsnorm_cast_query_plan.argtypes = [i64, i64, i32, i32, u32, i32, i32,
                                            ctypes.POINTER(Plan)]
    lib.rmsnorm_cast_query_plan.restype = i32
    lib.rmsnorm_cast_bwd_rows.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i32, i32, u32, vp,
                                          i64, vp, sz, vp]
    lib.rmsnorm_cast_bwd_rows.restype = i32
    lib.rmsnorm_cast_bwd_reduce.argtypes = [vp, sz, i64, i64, i32, i32, u32, vp, vp]
    lib.rmsnorm_cast_bwd_reduce.restype = i32
    _LIB = lib
    return lib


def rmsnorm_status_string(status):
    return load_library().rmsnorm_status_string(int(status)).decode()


def _check(func, status):
    if status != 0:
        raise RmsnormError(func, status, rmsnorm_status_string(status))


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _rows(x):
    """[M, N] view of a contiguous tensor (leading dims flatten into M)."""
    if x.dim() == 0:
        raise ValueError("expected at least one dimension")
    n = x.shape[-1]
    m = x.numel() // n if n else 0
    return m, n


def row_layout(t):
    """``(M, N, ld)`` when ``t`` is M rows of N unit-stride elements whose
    starts are ``ld`` elements apart (leading dims flatten into M), else None."""
    if t.dim() == 0:
        return None
    n = t.shape[-1]
    if n > 1 and t.stride(-1) != 1:
        return None
    m = t.numel() // n if n else 0
    ld = None
    expect = None
    for size, stride in zip(reversed(t.shape[:-1]), reversed(t.stride()[:-1])):
        if size == 1:
            continue
        if ld is None:
            ld, expect = stride, stride * size
        elif stride != expect:
            return None
        else:
            expect = stride * size
    if ld is None:
        ld = n
    if ld < n:
        return None
    return m, n, ld


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _flags(offset, dgamma_in_dtype=False):
    return ((RMSNORM_FLAG_OFFSET if offset else 0)
            | (RMSNORM_FLAG_DGAMMA_IN_DTYPE if dgamma_in_dtype else 0))


# ---- one-to-one wrappers of the C entry points ------------------------------

def rmsnorm_query_plan(M, N, dtype, offset=False, which=PASS_FWD, align_bytes=16):
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    p = Plan()
    _check("rmsnorm_query_plan", load_library().rmsnorm_query_plan(
        int(M), int(N), code, _flags(offset), int(which), int(align_bytes), ctypes.byref(p)))
    return p.as_dict()


def rmsnorm_bwd_workspace_bytes(M, N, dtype, offset=False):
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().rmsnorm_bwd_workspace_bytes(int(M), int(N), code, _flags(offset)))


def rmsnorm_fwd(x, gamma, eps, y, rstd, offset=False, stream=None):
    """y, rstd <- forward(x, gamma); tensors are [.., N] / [N] / [.., N] / [M]."""
    m, n = _rows(x)
    _check("rmsnorm_fwd", load_library().rmsnorm_fwd(
        _ptr(x), _ptr(gamma), float(eps), m, n, _dtype_code(x), _flags(offset),
        _ptr(y), _ptr(rstd), _stream(x.device, stream)))


def rmsnorm_bwd_rows(dy, x, gamma, rstd, dx, workspace, offset=False, stream=None):
    m, n = _rows(x)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rmsnorm_bwd_rows", load_library().rmsnorm_bwd_rows(
        _ptr(dy), _ptr(x), _ptr(gamma), _ptr(rstd), m, n, _dtype_code(x), _flags(offset),
        _ptr(dx), _ptr(workspace), ws_bytes, _stream(x.device, stream)))


def rmsnorm_bwd_reduce(workspace, M, N, dtype, dgamma, offset=False, stream=None):
    """dgamma float32, or of ``dtype`` (RMSNORM_FLAG_DGAMMA_IN_DTYPE) when the
    dgamma tensor has that dtype."""
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    in_dtype = dgamma.dtype != torch.float32
    _check("rmsnorm_bwd_reduce", load_library().rmsnorm_bwd_reduce(
        _ptr(workspace), ws_bytes, int(M), int(N), code, _flags(offset, in_dtype),
        _ptr(dgamma), _stream(dgamma.device, stream)))


def _layout(t, name):
    lay = row_layout(t)
    _require(lay is not None, f"{name} must be rows of unit-stride elements at one row stride")
    return lay


def rmsnorm_fwd_strided(x, gamma, eps, y, rstd, offset=False, stream=None):
    """rmsnorm_fwd with the row strides of x and y taken from the tensors."""
    m, n, ldx = _layout(x, "x")
    _, _, ldy = _layout(y, "y")
    _check("rmsnorm_fwd_strided", load_library().rmsnorm_fwd_strided(
        _ptr(x), ldx, _ptr(gamma), float(eps), m, n, _dtype_code(x), _flags(offset),
        _ptr(y), ldy, _ptr(rstd), _stream(x.device, stream)))


def rmsnorm_bwd_strided(dy, x, gamma, rstd, dx, dgamma, workspace, offset=False, stream=None):
    """rmsnorm_bwd with the row strides of dy, x and dx taken from the tensors."""
    m, n, ldx = _layout(x, "x")
    _, _, lddy = _layout(dy, "dy")
    _, _, lddx = _layout(dx, "dx")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    in_dtype = dgamma.dtype != torch.float32
    _check("rmsnorm_bwd_strided", load_library().rmsnorm_bwd_strided(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(rstd), m, n, _dtype_code(x),
        _flags(offset, in_dtype), _ptr(dx), lddx, _ptr(dgamma), _ptr(workspace), ws_bytes,
        _stream(x.device, stream)))


def rmsnorm_bwd(dy, x, gamma, rstd, dx, dgamma, workspace, offset=False, stream=None):
    """As rmsnorm_bwd_reduce, dgamma may be float32 or of x's dtype."""
    m, n = _rows(x)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    in_dtype = dgamma.dtype != torch.float32
    _require(not in_dtype or dgamma.dtype == x.dtype, "dgamma must be float32 or x's dtype")
    _check("rmsnorm_bwd", load_library().rmsnorm_bwd(
        _ptr(dy), _ptr(x), _ptr(gamma), _ptr(rstd), m, n, _dtype_code(x),
        _flags(offset, in_dtype), _ptr(dx), _ptr(dgamma), _ptr(workspace), ws_bytes,
        _stream(x.device, stream)))


def rmsnorm_bwd_noalloc(dy, x, gamma, rstd, dx, dgamma, offset=False, stream=None):
    """rmsnorm_bwd with the dgamma partial sums in the library's own device
    buffer (RMSNORM_NOALLOC_SCRATCH_BYTES per device) instead of a workspace."""
    m, n = _rows(x)
    in_dtype = dgamma.dtype != torch.float32
    _require(not in_dtype or dgamma.dtype == x.dtype, "dgamma must be float32 or x's dtype")
    _check("rmsnorm_bwd_noalloc", load_library().rmsnorm_bwd_noalloc(
        _ptr(dy), _ptr(x), _ptr(gamma), _ptr(rstd), m, n, _dtype_code(x),
        _flags(offset, in_dtype), _ptr(dx), _ptr(dgamma), _stream(x.device, stream)))


# ---- allocating front ends ----------------------------------------------------

def _check_inputs(x, gamma):
    _require(x.is_cuda and gamma.is_cuda, "x and gamma must be device tensors")
    _require(x.device == gamma.device, "x and gamma must be on the same device")
    _require(gamma.is_contiguous(), "gamma must be contiguous")
    _require(row_layout(x) is not None,
             "x must be rows of unit-stride elements at one row stride")
    _require(gamma.dim() == 1 and gamma.shape[0] == x.shape[-1],
             "gamma must be 1-D with the length of x's last dimension")
    _require(x.dtype == gamma.dtype, "x and gamma must share a dtype")


def fwd(x, gamma, eps=1e-6, offset=False, stream=None, poison=False):
    """Returns ``(y, rstd)``: y like x, rstd float32 with one value per row.

    ``poison`` fills the outputs with NaN first (tests use it to show every
    element is written)."""
    _check_inputs(x, gamma)
    m, _, _ = row_layout(x)
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    y = fill(x.shape, float("nan"), device=x.device, dtype=x.dtype)  # dense rows
    rstd = fill((m,), float("nan"), device=x.device, dtype=torch.float32)
    rmsnorm_fwd_strided(x, gamma, eps, y, rstd, offset, stream)
    return y, rstd


def bwd(dy, x, gamma, rstd, offset=False, stream=None, poison=False, workspace=None,
        dgamma_dtype=torch.float32):
    """Returns ``(dx, dgamma)``: dx like x, dgamma [N] (a row sum) in
    ``dgamma_dtype``: float32 (default) or x's dtype.

    x and dy may have any row stride; dy in another layout is made
    contiguous (as the page's autograd wrapper does)."""
    _check_inputs(x, gamma)
    _require(dy.shape == x.shape and dy.dtype == x.dtype and dy.device == x.device,
             "dy must match x in shape, dtype and device")
    if row_layout(dy) is None:
        dy = dy.contiguous()
    m, n, _ = row_layout(x)
    _require(rstd.dtype == torch.float32 and rstd.numel() == m and rstd.is_contiguous(),
             "rstd must be a contiguous float32 tensor with one value per row")
    _require(dgamma_dtype in (torch.float32, x.dtype), "dgamma_dtype must be float32 or x's dtype")
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    dx = fill(x.shape, float("nan"), device=x.device, dtype=x.dtype)  # dense rows
    dgamma = fill((n,), float("nan"), device=x.device, dtype=dgamma_dtype)
    if workspace is None:
        nbytes = rmsnorm_bwd_workspace_bytes(m, n, x.dtype, offset)
        workspace = torch.empty((max(nbytes, 4) // 4,), device=x.device, dtype=torch.float32)
    rmsnorm_bwd_strided(dy, x, gamma, rstd, dx, dgamma, workspace, offset, stream)
    return dx, dgamma


# ---- LayerNorm (include/layernorm.h) --------------------------------------------

def _code(dtype):
    return _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)


def layernorm_query_plan(M, N, dtype, which=PASS_FWD, align_bytes=16, dgamma_in_dtype=False):
    p = Plan()
    _check("layernorm_query_plan", load_library().layernorm_query_plan(
        int(M), int(N), _code(dtype), _flags(False, dgamma_in_dtype), int(which),
        int(align_bytes), ctypes.byref(p)))
    return p.as_dict()


def layernorm_bwd_workspace_bytes(M, N, dtype):
    return int(load_library().layernorm_bwd_workspace_bytes(int(M), int(N), _code(dtype), 0))


def layernorm_fwd(x, gamma, beta, eps, y, mean, rstd, stream=None):
    """y, mean, rstd <- LayerNorm forward of x; beta may be None (no bias).
    Row strides of x and y are taken from the tensors."""
    m, n, ldx = _layout(x, "x")
    _, _, ldy = _layout(y, "y")
    _check("layernorm_fwd", load_library().layernorm_fwd(
        _ptr(x), ldx, _ptr(gamma), _ptr(beta), float(eps), m, n, _dtype_code(x), 0,
        _ptr(y), ldy, _ptr(mean), _ptr(rstd), _stream(x.device, stream)))


def layernorm_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace, stream=None):
    """dx, dgamma, dbeta <- LayerNorm backward; dbeta may be None.  dgamma and
    dbeta are float32, or both of x's dtype."""
    m, n, ldx = _layout(x, "x")
    _, _, lddy = _layout(dy, "dy")
    _, _, lddx = _layout(dx, "dx")
    in_dtype = dgamma.dtype != torch.float32
    _require(dbeta is None or dbeta.dtype == dgamma.dtype, "dgamma and dbeta must share a dtype")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("layernorm_bwd", load_library().layernorm_bwd(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(mean), _ptr(rstd), m, n,
        _dtype_code(x), _flags(False, in_dtype), _ptr(dx), lddx, _ptr(dgamma), _ptr(dbeta),
        _ptr(workspace), ws_bytes, _stream(x.device, stream)))


def layernorm_bwd_rows(dy, x, gamma, mean, rstd, dx, workspace, stream=None):
    m, n, ldx = _layout(x, "x")
    _, _, lddy = _layout(dy, "dy")
    _, _, lddx = _layout(dx, "dx")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("layernorm_bwd_rows", load_library().layernorm_bwd_rows(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(mean), _ptr(rstd), m, n,
        _dtype_code(x), 0, _ptr(dx), lddx, _ptr(workspace), ws_bytes, _stream(x.device, stream)))


def layernorm_bwd_reduce(workspace, M, N, dtype, dgamma, dbeta=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    in_dtype = dgamma.dtype != torch.float32
    _check("layernorm_bwd_reduce", load_library().layernorm_bwd_reduce(
        _ptr(workspace), ws_bytes, int(M), int(N), _code(dtype), _flags(False, in_dtype),
        _ptr(dgamma), _ptr(dbeta), _stream(dgamma.device, stream)))


def ln_fwd(x, gamma, beta=None, eps=1e-5, stream=None, poison=False):
    """Returns ``(y, mean, rstd)``: y like x (dense rows), mean and rstd
    float32 with one value per row."""
    _check_inputs(x, gamma)
    if beta is not None:
        _require(beta.shape == gamma.shape and beta.dtype == x.dtype and beta.is_contiguous()
                 and beta.device == x.device, "beta must be like gamma")
    m, _, _ = row_layout(x)
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    y = fill(x.shape, float("nan"), device=x.device, dtype=x.dtype)
    mean = fill((m,), float("nan"), device=x.device, dtype=torch.float32)
    rstd = fill((m,), float("nan"), device=x.device, dtype=torch.float32)
    layernorm_fwd(x, gamma, beta, eps, y, mean, rstd, stream)
    return y, mean, rstd


def ln_bwd(dy, x, gamma, mean, rstd, stream=None, poison=False, workspace=None,
           dgamma_dtype=torch.float32, bias=True):
    """Returns ``(dx, dgamma, dbeta)`` (dbeta None when ``bias`` is False)."""
    _check_inputs(x, gamma)
    _require(dy.shape == x.shape and dy.dtype == x.dtype and dy.device == x.device,
             "dy must match x in shape, dtype and device")
    if row_layout(dy) is None:
        dy = dy.contiguous()
    m, n, _ = row_layout(x)
    for t, name in ((mean, "mean"), (rstd, "rstd")):
        _require(t.dtype == torch.float32 and t.numel() == m and t.is_contiguous(),
                 f"{name} must be a contiguous float32 tensor with one value per row")
    _require(dgamma_dtype in (torch.float32, x.dtype), "dgamma_dtype must be float32 or x's dtype")
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    dx = fill(x.shape, float("nan"), device=x.device, dtype=x.dtype)
    dgamma = fill((n,), float("nan"), device=x.device, dtype=dgamma_dtype)
    dbeta = fill((n,), float("nan"), device=x.device, dtype=dgamma_dtype) if bias else None
    if workspace is None:
        nbytes = layernorm_bwd_workspace_bytes(m, n, x.dtype)
        workspace = torch.empty((max(nbytes, 4) // 4,), device=x.device, dtype=torch.float32)
    layernorm_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace, stream)
    return dx, dgamma, dbeta


# ---- RMSNorm with the residual add fused before it (include/rmsnorm_add.h) -------

def rmsnorm_add_query_plan(M, N, dtype, offset=False, which=PASS_FWD, align_bytes=16):
    p = Plan()
    _check("rmsnorm_add_query_plan", load_library().rmsnorm_add_query_plan(
        int(M), int(N), _code(dtype), _flags(offset), int(which), int(align_bytes),
        ctypes.byref(p)))
    return p.as_dict()


def rmsnorm_add_bwd_workspace_bytes(M, N, dtype, offset=False):
    return int(load_library().rmsnorm_add_bwd_workspace_bytes(int(M), int(N), _code(dtype),
                                                              _flags(offset)))


def rmsnorm_add_fwd(x, res, gamma, eps, y, h, rstd, offset=False, stream=None):
    """y, h, rstd <- RMSNorm(h) with h = x + res; row strides from the tensors."""
    m, n, ldx = _layout(x, "x")
    _, _, ldr = _layout(res, "res")
    _, _, ldy = _layout(y, "y")
    _, _, ldh = _layout(h, "h")
    _check("rmsnorm_add_fwd", load_library().rmsnorm_add_fwd(
        _ptr(x), ldx, _ptr(res), ldr, _ptr(gamma), float(eps), m, n, _dtype_code(x),
        _flags(offset), _ptr(y), ldy, _ptr(h), ldh, _ptr(rstd), _stream(x.device, stream)))


def rmsnorm_add_bwd(dy, dh, h, gamma, rstd, dx, dgamma, workspace, offset=False, stream=None):
    """dx (the gradient of x and of res), dgamma <- backward; dh may be None."""
    m, n, ldh = _layout(h, "h")
    _, _, lddy = _layout(dy, "dy")
    lddh = _layout(dh, "dh")[2] if dh is not None else n
    _, _, lddx = _layout(dx, "dx")
    in_dtype = dgamma.dtype != torch.float32
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rmsnorm_add_bwd", load_library().rmsnorm_add_bwd(
        _ptr(dy), lddy, _ptr(dh), lddh, _ptr(h), ldh, _ptr(gamma), _ptr(rstd), m, n,
        _dtype_code(h), _flags(offset, in_dtype), _ptr(dx), lddx, _ptr(dgamma),
        _ptr(workspace), ws_bytes, _stream(h.device, stream)))


def rmsnorm_add_bwd_rows(dy, dh, h, gamma, rstd, dx, workspace, offset=False, stream=None):
    m, n, ldh = _layout(h, "h")
    _, _, lddy = _layout(dy, "dy")
    lddh = _layout(dh, "dh")[2] if dh is not None else n
    _, _, lddx = _layout(dx, "dx")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rmsnorm_add_bwd_rows", load_library().rmsnorm_add_bwd_rows(
        _ptr(dy), lddy, _ptr(dh), lddh, _ptr(h), ldh, _ptr(gamma), _ptr(rstd), m, n,
        _dtype_code(h), _flags(offset), _ptr(dx), lddx, _ptr(workspace), ws_bytes,
        _stream(h.device, stream)))


def rmsnorm_add_bwd_reduce(workspace, M, N, dtype, dgamma, offset=False, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    in_dtype = dgamma.dtype != torch.float32
    _check("rmsnorm_add_bwd_reduce", load_library().rmsnorm_add_bwd_reduce(
        _ptr(workspace), ws_bytes, int(M), int(N), _code(dtype), _flags(offset, in_dtype),
        _ptr(dgamma), _stream(dgamma.device, stream)))


def add_fwd(x, res, gamma, eps=1e-6, offset=False, stream=None, poison=False):
    """Returns ``(y, h, rstd)``: h = x + res (the new residual stream),
    y = RMSNorm(h), rstd float32 per row."""
    _check_inputs(x, gamma)
    _require(res.shape == x.shape and res.dtype == x.dtype and res.device == x.device
             and row_layout(res) is not None, "res must match x")
    m, _, _ = row_layout(x)
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    y = fill(x.shape, float("nan"), device=x.device, dtype=x.dtype)
    h = fill(x.shape, float("nan"), device=x.device, dtype=x.dtype)
    rstd = fill((m,), float("nan"), device=x.device, dtype=torch.float32)
    rmsnorm_add_fwd(x, res, gamma, eps, y, h, rstd, offset, stream)
    return y, h, rstd


def add_bwd(dy, dh, h, gamma, rstd, offset=False, stream=None, poison=False, workspace=None,
            dgamma_dtype=torch.float32):
    """Returns ``(dx, dgamma)``: dx is the gradient of both x and res."""
    _check_inputs(h, gamma)
    for t, name in ((dy, "dy"), (dh, "dh")):
        if t is not None:
            _require(t.shape == h.shape and t.dtype == h.dtype and t.device == h.device,
                     f"{name} must match h in shape, dtype and device")
    if row_layout(dy) is None:
        dy = dy.contiguous()
    if dh is not None and row_layout(dh) is None:
        dh = dh.contiguous()
    m, n, _ = row_layout(h)
    _require(rstd.dtype == torch.float32 and rstd.numel() == m and rstd.is_contiguous(),
             "rstd must be a contiguous float32 tensor with one value per row")
    _require(dgamma_dtype in (torch.float32, h.dtype), "dgamma_dtype must be float32 or h's dtype")
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    dx = fill(h.shape, float("nan"), device=h.device, dtype=h.dtype)
    dgamma = fill((n,), float("nan"), device=h.device, dtype=dgamma_dtype)
    if workspace is None:
        nbytes = rmsnorm_add_bwd_workspace_bytes(m, n, h.dtype, offset)
        workspace = torch.empty((max(nbytes, 4) // 4,), device=h.device, dtype=torch.float32)
    rmsnorm_add_bwd(dy, dh, h, gamma, rstd, dx, dgamma, workspace, offset, stream)
    return dx, dgamma


# ---- RMSNorm with its output cast to a narrower dtype (include/rmsnorm_cast.h) ----

def rmsnorm_cast_query_plan(M, N, out_dtype, offset=False, which=PASS_FWD, align_bytes=16):
    p = Plan()
    _check("rmsnorm_cast_query_plan", load_library().rmsnorm_cast_query_plan(
        int(M), int(N), RMSNORM_F32, _code(out_dtype), _flags(offset), int(which),
        int(align_bytes), ctypes.byref(p)))
    return p.as_dict()


def rmsnorm_cast_bwd_workspace_bytes(M, N, out_dtype, offset=False):
    return int(load_library().rmsnorm_cast_bwd_workspace_bytes(
        int(M), int(N), RMSNORM_F32, _code(out_dtype), _flags(offset)))


def rmsnorm_cast_fwd(x, gamma, eps, y, rstd, offset=False, stream=None):
    """y (its own dtype), rstd <- RMSNorm(x) cast to y's dtype; row strides
    from the tensors."""
    m, n, ldx = _layout(x, "x")
    _, _, ldy = _layout(y, "y")
    _check("rmsnorm_cast_fwd", load_library().rmsnorm_cast_fwd(
        _ptr(x), ldx, _ptr(gamma), float(eps), m, n, _dtype_code(x), _dtype_code(y),
        _flags(offset), _ptr(y), ldy, _ptr(rstd), _stream(x.device, stream)))


def rmsnorm_cast_bwd(dy, x, gamma, rstd, dx, dgamma, workspace, offset=False, stream=None):
    """dx, dgamma <- backward from dy in the narrow dtype."""
    m, n, ldx = _layout(x, "x")
    _, _, lddy = _layout(dy, "dy")
    _, _, lddx = _layout(dx, "dx")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rmsnorm_cast_bwd", load_library().rmsnorm_cast_bwd(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(rstd), m, n, _dtype_code(x),
        _dtype_code(dy), _flags(offset), _ptr(dx), lddx, _ptr(dgamma), _ptr(workspace),
        ws_bytes, _stream(x.device, stream)))


def rmsnorm_cast_bwd_rows(dy, x, gamma, rstd, dx, workspace, offset=False, stream=None):
    m, n, ldx = _layout(x, "x")
    _, _, lddy = _layout(dy, "dy")
    _, _, lddx = _layout(dx, "dx")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rmsnorm_cast_bwd_rows", load_library().rmsnorm_cast_bwd_rows(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(rstd), m, n, _dtype_code(x),
        _dtype_code(dy), _flags(offset), _ptr(dx), lddx, _ptr(workspace), ws_bytes,
        _stream(x.device, stream)))


def rmsnorm_cast_bwd_reduce(workspace, M, N, out_dtype, dgamma, offset=False, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rmsnorm_cast_bwd_reduce", load_library().rmsnorm_cast_bwd_reduce(
        _ptr(workspace), ws_bytes, int(M), int(N), RMSNORM_F32, _code(out_dtype),
        _flags(offset), _ptr(dgamma), _stream(dgamma.device, stream)))


def cast_fwd(x, gamma, out_dtype=torch.bfloat16, eps=1e-6, offset=False, stream=None,
             poison=False):
    """Returns ``(y, rstd)``: y = RMSNorm(x) in ``out_dtype`` (x and gamma
    float32), rstd float32 per row."""
    _check_inputs(x, gamma)
    _require(x.dtype == torch.float32, "x must be float32")
    _require(out_dtype in (torch.bfloat16, torch.float16), "out_dtype must be bf16 or fp16")
    m, _, _ = row_layout(x)
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    y = fill(x.shape, float("nan"), device=x.device, dtype=out_dtype)
    rstd = fill((m,), float("nan"), device=x.device, dtype=torch.float32)
    rmsnorm_cast_fwd(x, gamma, eps, y, rstd, offset, stream)
    return y, rstd


def cast_bwd(dy, x, gamma, rstd, offset=False, stream=None, poison=False, workspace=None):
    """Returns ``(dx, dgamma)``, both float32, from dy in the narrow dtype."""
    _check_inputs(x, gamma)
    _require(dy.shape == x.shape and dy.device == x.device
             and dy.dtype in (torch.bfloat16, torch.float16),
             "dy must match x in shape and device and be bf16 or fp16")
    if row_layout(dy) is None:
        dy = dy.contiguous()
    m, n, _ = row_layout(x)
    _require(rstd.dtype == torch.float32 and rstd.numel() == m and rstd.is_contiguous(),
             "rstd must be a contiguous float32 tensor with one value per row")
    fill = torch.full if poison else (lambda shape, _v, **kw: torch.empty(shape, **kw))
    dx = fill(x.shape, float("nan"), device=x.device, dtype=torch.float32)
    dgamma = fill((n,), float("nan"), device=x.device, dtype=torch.float32)
    if workspace is None:
        nbytes = rmsnorm_cast_bwd_workspace_bytes(m, n, dy.dtype, offset)
        workspace = torch.empty((max(nbytes, 4) // 4,), device=x.device, dtype=torch.float32)
    rmsnorm_cast_bwd(dy, x, gamma, rstd, dx, dgamma, workspace, offset, stream)
    return dx, dgamma
