"""ctypes binding of libgemm_epilog.so -- argument marshalling only.

The functions carry the C ABI's names (include/gemm_epilog.h) and raise
GemmEpilogError (with the status code) instead of returning one.  Every step
of the computation runs in the library's HIP kernels; torch provides device
memory and streams.  There is no fallback: if the library is missing, import
of this module's loader raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first so the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_epilog.so")

# ---- ABI constants (mirror include/gemm_epilog.h) ----------------------------
GE_OK, GE_ERR_NULL, GE_ERR_SHAPE, GE_ERR_DTYPE, GE_ERR_EPILOG, GE_ERR_ALIGN, \
    GE_ERR_STATE, GE_ERR_WORKSPACE, GE_ERR_HIP, GE_ERR_ALLOC, GE_ERR_STATIC_LIMIT = range(11)
GE_STATIC_WORKSPACE_BYTES = 16 << 20
GE_F32, GE_F16, GE_BF16, GE_F8_E4M3, GE_MXF8_E4M3 = 0, 1, 2, 3, 4
GE_OP_N, GE_OP_T = 0, 1
GE_EPILOG_NONE, GE_EPILOG_BIAS, GE_EPILOG_RELU_BIAS, GE_EPILOG_RELU_AUX_BIAS, \
    GE_EPILOG_GELU_BIAS, GE_EPILOG_GELU_AUX_BIAS, GE_EPILOG_DRELU, GE_EPILOG_DGELU, \
    GE_EPILOG_DRELU_BGRAD, GE_EPILOG_DGELU_BGRAD, GE_EPILOG_TANH_BIAS = range(11)
GE_BIAS_ROW, GE_BIAS_COL = 0, 1

DTYPE_CODE = {"f32": GE_F32, "f16": GE_F16, "bf16": GE_BF16, "e4m3": GE_F8_E4M3, "mxf8": GE_MXF8_E4M3,
              torch.float32: GE_F32, torch.float16: GE_F16, torch.bfloat16: GE_BF16,
              torch.float8_e4m3fn: GE_F8_E4M3}
EPILOG_CODE = {"none": GE_EPILOG_NONE, "bias": GE_EPILOG_BIAS, "relu_bias": GE_EPILOG_RELU_BIAS,
               "relu_aux_bias": GE_EPILOG_RELU_AUX_BIAS, "gelu_bias": GE_EPILOG_GELU_BIAS,
               "gelu_aux_bias": GE_EPILOG_GELU_AUX_BIAS, "drelu": GE_EPILOG_DRELU,
               "dgelu": GE_EPILOG_DGELU, "drelu_bgrad": GE_EPILOG_DRELU_BGRAD,
               "dgelu_bgrad": GE_EPILOG_DGELU_BGRAD, "tanh_bias": GE_EPILOG_TANH_BIAS}
AXIS_CODE = {"row": GE_BIAS_ROW, "col": GE_BIAS_COL}
TORCH_DTYPE = {GE_F32: torch.float32, GE_F16: torch.float16, GE_BF16: torch.bfloat16,
               GE_F8_E4M3: torch.float8_e4m3fn, GE_MXF8_E4M3: torch.float8_e4m3fn}
ELEM_SIZE = {GE_F32: 4, GE_F16: 2, GE_BF16: 2, GE_F8_E4M3: 1, GE_MXF8_E4M3: 1}


def mx_scale_ld(k: int) -> int:
    """Row stride in bytes of the MX block-scale arrays (GE_MX_SCALE_LD)."""
    return ((k + 31) // 32 + 15) // 16 * 16


class ge_desc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32),
                ("d_type", ctypes.c_int32), ("bias_type", ctypes.c_int32),
                ("op_b", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldd", ctypes.c_int64)]


class ge_pref(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("unfused", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("split_k", ctypes.c_int32), ("group_m", ctypes.c_int32)]


class ge_batch_strides(ctypes.Structure):
    """Per-product strides of a batched handle, in elements of each buffer's
    type (aux: 32-bit words for the mask)."""
    _fields_ = [("a", ctypes.c_int64), ("b", ctypes.c_int64), ("bias", ctypes.c_int64),
                ("d", ctypes.c_int64), ("aux", ctypes.c_int64)]


class GemmEpilogError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {gemm_epilog_status_string(status)} ({status})")


_lib = None


def lib():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              f"(hipcc for gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.gemm_epilog_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(ge_desc)]
        L.gemm_epilog_plan.argtypes = [vp, i32, i32, ctypes.POINTER(ge_pref)]
        L.gemm_epilog_workspace_size.argtypes = [vp, ctypes.POINTER(sz)]
        L.gemm_epilog_aux_ld.argtypes = [vp, ctypes.POINTER(ctypes.c_int64)]
        L.gemm_epilog_execute.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gemm_epilog_free.argtypes = [vp]
        L.gemm_epilog_status_string.argtypes = [ctypes.c_int]
        L.gemm_epilog_status_string.restype = ctypes.c_char_p
        L.gemm_epilog_describe.argtypes = [vp, ctypes.c_char_p, sz]
        L.gemm_epilog_autotune.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, vp,
                                           ctypes.POINTER(ctypes.c_float)]
        L.gemm_epilog_execute_c.argtypes = [vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gemm_epilog_execute_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gemm_epilog_execute_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gemm_epilog_execute_m.argtypes = [vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gemm_epilog_set_batch_strides.argtypes = [vp, ctypes.POINTER(ge_batch_strides)]
        L.gemm_epilog_set_fp8_output.argtypes = [vp, vp, vp]
        for f in ("gemm_epilog_create", "gemm_epilog_plan", "gemm_epilog_workspace_size",
                  "gemm_epilog_aux_ld", "gemm_epilog_execute", "gemm_epilog_free",
                  "gemm_epilog_describe", "gemm_epilog_autotune", "gemm_epilog_execute_c",
                  "gemm_epilog_execute_static", "gemm_epilog_execute_mx"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != GE_OK:
        raise GemmEpilogError(status, what)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def make_desc(m, n, k, a_type, d_type, op_b=GE_OP_N, lda=None, ldb=None, ldd=None,
              b_type=None, bias_type=None, batch=0) -> ge_desc:
    a = DTYPE_CODE[a_type] if not isinstance(a_type, int) else a_type
    d = DTYPE_CODE[d_type] if not isinstance(d_type, int) else d_type
    b = a if b_type is None else (DTYPE_CODE[b_type] if not isinstance(b_type, int) else b_type)
    bt = ((DTYPE_CODE["bf16"] if d == DTYPE_CODE["e4m3"] else d) if bias_type is None
          else (DTYPE_CODE[bias_type] if not isinstance(bias_type, int) else bias_type))
    return ge_desc(m, n, k, a, b, d, bt, op_b, batch,
                   k if lda is None else lda,
                   (n if op_b == GE_OP_N else k) if ldb is None else ldb,
                   n if ldd is None else ldd)


# ---- the ABI, same names ---------------------------------------------------------
def gemm_epilog_create(desc: ge_desc) -> int:
    h = ctypes.c_void_p()
    _check(lib().gemm_epilog_create(ctypes.byref(h), ctypes.byref(desc)), "gemm_epilog_create")
    return h.value


def gemm_epilog_plan(h: int, epilog, axis=GE_BIAS_ROW, pref: Optional[ge_pref] = None) -> None:
    e = EPILOG_CODE[epilog] if isinstance(epilog, str) else epilog
    a = AXIS_CODE[axis] if isinstance(axis, str) else axis
    _check(lib().gemm_epilog_plan(h, e, a, ctypes.byref(pref) if pref is not None else None),
           "gemm_epilog_plan")


def gemm_epilog_workspace_size(h: int) -> int:
    s = ctypes.c_size_t()
    _check(lib().gemm_epilog_workspace_size(h, ctypes.byref(s)), "gemm_epilog_workspace_size")
    return s.value


def gemm_epilog_aux_ld(h: int) -> int:
    s = ctypes.c_int64()
    _check(lib().gemm_epilog_aux_ld(h, ctypes.byref(s)), "gemm_epilog_aux_ld")
    return s.value


def gemm_epilog_execute(h: int, A, B, bias, D, aux=None, scale_a=None, scale_b=None,
                        workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if isinstance(workspace, torch.Tensor) else 0)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    _check(lib().gemm_epilog_execute(h, _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux),
                                     _ptr(scale_a), _ptr(scale_b), _ptr(workspace),
                                     workspace_bytes, stream or None),
           "gemm_epilog_execute")


def gemm_epilog_execute_m(h: int, m: int, A, B, bias, D, aux=None, scale_a=None, scale_b=None,
                          workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    """execute with m rows (0 <= m <= the handle's m), the plan unchanged."""
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if isinstance(workspace, torch.Tensor) else 0)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    _check(lib().gemm_epilog_execute_m(h, m, _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux),
                                       _ptr(scale_a), _ptr(scale_b), _ptr(workspace),
                                       workspace_bytes, stream or None),
           "gemm_epilog_execute_m")


def gemm_epilog_set_fp8_output(h: int, scale_d=None, amax_d=None) -> None:
    """fp8 (E4M3) output: D's scale (device fp32, None = 1) and the amax
    output (device fp32 per product, or None)."""
    _check(lib().gemm_epilog_set_fp8_output(h, _ptr(scale_d), _ptr(amax_d)), "gemm_epilog_set_fp8_output")


def gemm_epilog_set_batch_strides(h: int, strides: Optional[ge_batch_strides]) -> None:
    """Per-product strides (elements) of a batched handle; None = packed."""
    _check(lib().gemm_epilog_set_batch_strides(h, ctypes.byref(strides) if strides is not None else None),
           "gemm_epilog_set_batch_strides")


def gemm_epilog_execute_mx(h: int, A, B, a_scales, b_scales, bias, D, aux=None, scale_a=None, scale_b=None,
                           workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    """execute for block-scaled fp8 handles: a_scales (m x mx_scale_ld(k)
    bytes) and b_scales (n x mx_scale_ld(k) bytes) hold one E8M0 scale per 32
    K values of each row of A and each column of B."""
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if isinstance(workspace, torch.Tensor) else 0)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    _check(lib().gemm_epilog_execute_mx(h, _ptr(A), _ptr(B), _ptr(a_scales), _ptr(b_scales), _ptr(bias), _ptr(D),
                                        _ptr(aux), _ptr(scale_a), _ptr(scale_b), _ptr(workspace), workspace_bytes,
                                        stream or None),
           "gemm_epilog_execute_mx")


def gemm_epilog_execute_static(h: int, A, B, bias, D, aux=None, scale_a=None, scale_b=None,
                               stream=None) -> None:
    """execute with the library's own fixed workspace array (no workspace
    argument; nothing is allocated)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    _check(lib().gemm_epilog_execute_static(h, _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux),
                                            _ptr(scale_a), _ptr(scale_b), stream or None),
           "gemm_epilog_execute_static")


def gemm_epilog_free(h: Optional[int]) -> None:
    _check(lib().gemm_epilog_free(h), "gemm_epilog_free")


def gemm_epilog_status_string(status: int) -> str:
    return lib().gemm_epilog_status_string(status).decode()


def gemm_epilog_execute_c(h: int, A, B, C, ldc: int, beta, bias, D, aux=None, scale_a=None,
                          scale_b=None, workspace=None, workspace_bytes=None, stream=None) -> None:
    """execute with the added input term beta*C (C in D's dtype, row stride
    ldc elements; beta a device fp32 scalar)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gemm_epilog_execute_c(h, _ptr(A), _ptr(B), _ptr(C), ldc, _ptr(beta), _ptr(bias), _ptr(D),
                                       _ptr(aux), _ptr(scale_a), _ptr(scale_b), _ptr(workspace),
                                       workspace_bytes, stream),
           "gemm_epilog_execute_c")


def gemm_epilog_autotune(h: int, A, B, bias, D, aux=None, scale_a=None, scale_b=None,
                         workspace=None, workspace_bytes=None, iters: int = 5, stream=None) -> float:
    """Time the candidate kernels on these buffers and keep the fastest in the
    plan; returns its mean milliseconds per call."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    best = ctypes.c_float(0.0)
    _check(lib().gemm_epilog_autotune(h, _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux),
                                      _ptr(scale_a), _ptr(scale_b), _ptr(workspace), workspace_bytes,
                                      iters, stream, ctypes.byref(best)),
           "gemm_epilog_autotune")
    return best.value


def gemm_epilog_describe(h: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(lib().gemm_epilog_describe(h, buf, 512), "gemm_epilog_describe")
    return buf.value.decode()


# ---- convenience object over torch tensors (still marshalling only) ---------------
class GemmEpilog:
    """create -> plan -> execute -> free, on torch device tensors.

    A is m x k; B is k x n (op_b=N) or n x k (op_b=T); D is m x n.  The
    bias holds m (axis 'row') or n (axis 'col') values of D's dtype.
    """

    def __init__(self, m, n, k, a_dtype, d_dtype, op_b=GE_OP_N, lda=None, ldb=None, ldd=None, batch=0):
        self.desc = make_desc(m, n, k, a_dtype, d_dtype, op_b, lda, ldb, ldd, batch=batch)
        self.h = gemm_epilog_create(self.desc)
        self.epilog = None

    def plan(self, epilog="bias", axis="row", path=0, unfused=0, tile=0, split_k=0, group_m=0):
        gemm_epilog_plan(self.h, epilog, axis, ge_pref(path, unfused, tile, split_k, group_m))
        self.epilog = EPILOG_CODE[epilog] if isinstance(epilog, str) else epilog
        self.ws_bytes = gemm_epilog_workspace_size(self.h)
        self.aux_ld_bits = gemm_epilog_aux_ld(self.h)
        return self

    def alloc_outputs(self, device="cuda"):
        """D (and the aux output, workspace) for the planned problem; with
        batch > 1, leading dimension batch, each product packed after the
        previous one as the ABI's batch strides expect."""
        d = self.desc
        lead = (d.batch,) if d.batch > 1 else ()
        D = torch.empty(lead + (d.m, d.ldd), dtype=TORCH_DTYPE[d.d_type], device=device)[..., :d.n]
        aux = None
        if self.epilog == GE_EPILOG_RELU_AUX_BIAS:
            aux = torch.empty(lead + (d.m, self.aux_ld_bits // 32), dtype=torch.int32, device=device)
        elif self.epilog == GE_EPILOG_GELU_AUX_BIAS:
            # the pre-activation matrix, D's dtype, round_up(n, 128) columns
            dt = TORCH_DTYPE[d.d_type]
            aux = torch.empty(lead + (d.m, self.aux_ld_bits // torch.finfo(dt).bits), dtype=dt,
                              device=device)
        ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device) if self.ws_bytes else None
        return D, aux, ws

    def execute(self, A, B, bias=None, D=None, aux=None, scale_a=None, scale_b=None,
                workspace=None, stream=None):
        if D is None:
            D, aux_new, ws_new = self.alloc_outputs(A.device)
            aux = aux if aux is not None else aux_new
            workspace = workspace if workspace is not None else ws_new
        gemm_epilog_execute(self.h, A, B, bias, D, aux, scale_a, scale_b, workspace,
                            None if workspace is None else workspace.numel() * workspace.element_size(),
                            stream)
        return D, aux

    def describe(self) -> str:
        return gemm_epilog_describe(self.h)

    def free(self):
        if self.h:
            gemm_epilog_free(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
