"""CPU oracle for D = epilogue(A*B + bias): a plain, slow, double-precision
reference written from the pages' definitions (see ``oracle.c`` for the
passes and their citations).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library: its dtype and epilogue codes, codecs and arithmetic are its
own, and it never imports the library's binding.

Every function takes *raw codes* (numpy arrays of float32 / uint16 / uint8)
exactly as they sit in device memory, plus an oracle dtype name, and decodes
them exactly to float64 itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Oracle-private codes (independent of the library's enums).
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
EPILOGS = {"none": 0, "bias": 1, "relu_bias": 2, "relu_aux_bias": 3,
           "gelu_bias": 4, "gelu_erf": 5, "gelu_aux_bias": 4,   # O5's Y is O3's GELU
           "tanh_bias": 6}
AXES = {"row": 0, "col": 1}
_NP_CODE_TYPE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16,
                 "e4m3": np.uint8}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE semantics, no FMA
    contraction, OpenMP over independent output rows)."""
    if not force and os.path.exists(_LIB) and \
            os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fno-fast-math",
           "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.orc_dec_f16.restype = dbl
        L.orc_dec_f16.argtypes = [ctypes.c_uint16]
        L.orc_dec_bf16.restype = dbl
        L.orc_dec_bf16.argtypes = [ctypes.c_uint16]
        L.orc_dec_e4m3.restype = dbl
        L.orc_dec_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_enc_f16.restype = ctypes.c_uint16
        L.orc_enc_f16.argtypes = [dbl]
        L.orc_enc_bf16.restype = ctypes.c_uint16
        L.orc_enc_bf16.argtypes = [dbl]
        L.orc_enc_e4m3_sat.restype = ctypes.c_uint8
        L.orc_enc_e4m3_sat.argtypes = [dbl]
        L.orc_act1.restype = dbl
        L.orc_act1.argtypes = [ctypes.c_int, dbl]
        L.orc_decode.argtypes = [ctypes.c_int, vp, i64, vp]
        L.orc_gemm.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64,
                               ctypes.c_int, vp, i64, ctypes.c_int, dbl, dbl, vp]
        L.orc_gemm_entries.argtypes = [i64, ctypes.c_int, vp, i64, ctypes.c_int,
                                       vp, i64, ctypes.c_int, dbl, dbl, i64,
                                       vp, vp, vp]
        L.orc_gemm_abs.argtypes = L.orc_gemm.argtypes
        L.orc_gemm_mx.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, vp, i64,
                                  ctypes.c_int, vp, i64, ctypes.c_int, vp, i64, dbl, dbl, vp]
        L.orc_gemm_mx_abs.argtypes = L.orc_gemm_mx.argtypes
        L.orc_gemm_mx_entries.argtypes = [i64, ctypes.c_int, vp, i64, vp, i64, ctypes.c_int, vp, i64,
                                          ctypes.c_int, vp, i64, dbl, dbl, i64, vp, vp, vp]
        L.orc_gemm_mx_abs_entries.argtypes = L.orc_gemm_mx_entries.argtypes
        L.orc_dec_e8m0.restype = dbl
        L.orc_dec_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_gemm_abs_entries.argtypes = L.orc_gemm_entries.argtypes
        L.orc_bias.argtypes = [i64, i64, vp, ctypes.c_int, ctypes.c_int, vp, vp]
        L.orc_bias_entries.argtypes = [i64, vp, vp, vp, ctypes.c_int,
                                       ctypes.c_int, vp, vp]
        L.orc_act.argtypes = [i64, ctypes.c_int, vp, vp]
        L.orc_mask.argtypes = [i64, i64, vp, i64, vp]
        L.orc_gelu_deriv.restype = dbl
        L.orc_gelu_deriv.argtypes = [dbl]
        L.orc_drelu.argtypes = [i64, i64, vp, i64, vp, vp]
        L.orc_dgelu.argtypes = [i64, i64, vp, ctypes.c_int, vp, i64, vp]
        L.orc_bgrad.argtypes = [i64, i64, vp, ctypes.c_int, vp]
        L.orc_add_beta_c.argtypes = [i64, i64, vp, dbl, ctypes.c_int, vp, i64, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _codes(x: np.ndarray, dtype: str) -> np.ndarray:
    want = _NP_CODE_TYPE[dtype]
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} codes must be {np.dtype(want)}, got {x.dtype}")
    return np.ascontiguousarray(x)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed ({rc})")


# ---- codecs ----------------------------------------------------------------
def decode(codes: np.ndarray, dtype: str) -> np.ndarray:
    """O0: exact decode of raw codes to float64 (same shape)."""
    c = _codes(codes, dtype)
    out = np.empty(c.shape, dtype=np.float64)
    _check(lib().orc_decode(DTYPES[dtype], _ptr(c), c.size, _ptr(out)), "decode")
    return out


def encode(x, dtype: str) -> np.ndarray:
    """Round-to-nearest-even encode of float64 values (fp16/bf16: overflow to
    inf; e4m3: saturate to +-448)."""
    L = lib()
    fn = {"f16": L.orc_enc_f16, "bf16": L.orc_enc_bf16, "e4m3": L.orc_enc_e4m3_sat}[dtype]
    xs = np.asarray(x, dtype=np.float64)
    out = np.array([fn(float(v)) for v in xs.ravel()], dtype=_NP_CODE_TYPE[dtype])
    return out.reshape(xs.shape)


# ---- O1..O4 ------------------------------------------------------------------
def _gemm_call(fn, what, A, ta, B, tb, op_b, sa, sb, m, n, k, lda, ldb):
    A = _codes(A, ta)
    B = _codes(B, tb)
    if A.ndim == 2:
        m, k = A.shape
        lda = A.shape[1]
    if B.ndim == 2:
        if op_b:
            n, kb = B.shape
        else:
            kb, n = B.shape
        if kb != k:
            raise ValueError(f"oracle {what}: inner dimensions differ")
        ldb = B.shape[1]
    C = np.empty((m, n), dtype=np.float64)
    _check(fn(m, n, k, DTYPES[ta], _ptr(A), lda, DTYPES[tb], _ptr(B),
              ldb, int(op_b), float(sa), float(sb), _ptr(C)), what)
    return C


def gemm(A: np.ndarray, ta: str, B: np.ndarray, tb: str, op_b: int = 0,
         sa: float = 1.0, sb: float = 1.0, m=None, n=None, k=None,
         lda=None, ldb=None) -> np.ndarray:
    """O1: C = sa*sb * A @ B in float64 (p ascending).  A: m x k row-major
    codes (2-D array, or 1-D with m, k, lda).  B: k x n (op_b=0) or n x k
    (op_b=1) row-major codes."""
    return _gemm_call(lib().orc_gemm, "gemm", A, ta, B, tb, op_b, sa, sb, m, n, k, lda, ldb)


def gemm_abs(A: np.ndarray, ta: str, B: np.ndarray, tb: str, op_b: int = 0,
             sa: float = 1.0, sb: float = 1.0, m=None, n=None, k=None,
             lda=None, ldb=None) -> np.ndarray:
    """|sa*sb| * |A| @ |B|: the magnitude term of the dot-product rounding
    error bound (Higham, section 3.1), same arguments as gemm."""
    return _gemm_call(lib().orc_gemm_abs, "gemm_abs", A, ta, B, tb, op_b, sa, sb, m, n, k, lda, ldb)


def _gemm_mx_call(fn, what, A, ta, SA, B, tb, SB, op_b, sa, sb):
    A = _codes(A, ta)
    B = _codes(B, tb)
    SA = np.ascontiguousarray(SA, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    m, k = A.shape
    n = B.shape[0] if op_b else B.shape[1]
    kb = (k + 31) // 32
    if SA.shape[0] != m or SB.shape[0] != n or SA.shape[1] < kb or SB.shape[1] < kb:
        raise ValueError(f"oracle {what}: block scales must be m x >=ceil(k/32) and n x >=ceil(k/32)")
    C = np.empty((m, n), dtype=np.float64)
    _check(fn(m, n, k, DTYPES[ta], _ptr(A), A.shape[1], _ptr(SA), SA.shape[1], DTYPES[tb], _ptr(B),
              B.shape[1], int(op_b), _ptr(SB), SB.shape[1], float(sa), float(sb), _ptr(C)), what)
    return C


def gemm_mx(A, ta, SA, B, tb, SB, op_b=0, sa=1.0, sb=1.0) -> np.ndarray:
    """O1x: the product with one E8M0 scale per 32 K values: SA (m x
    >=ceil(k/32) bytes) for the rows of A, SB (n x >=ceil(k/32) bytes) for the
    columns of B (K blocks contiguous per column, whichever layout B has)."""
    return _gemm_mx_call(lib().orc_gemm_mx, "gemm_mx", A, ta, SA, B, tb, SB, op_b, sa, sb)


def gemm_mx_abs(A, ta, SA, B, tb, SB, op_b=0, sa=1.0, sb=1.0) -> np.ndarray:
    """gemm_mx over absolute values (the error bound's magnitude term)."""
    return _gemm_mx_call(lib().orc_gemm_mx_abs, "gemm_mx_abs", A, ta, SA, B, tb, SB, op_b, sa, sb)


def _mx_entries_call(fn, what, A_rows, ta, SA_rows, slot, cols, B, tb, SB, op_b, sa, sb):
    A_rows = _codes(A_rows, ta)
    B = _codes(B, tb)
    SA_rows = np.ascontiguousarray(SA_rows, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    slot = np.ascontiguousarray(slot, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(slot.shape[0], dtype=np.float64)
    _check(fn(A_rows.shape[1], DTYPES[ta], _ptr(A_rows), A_rows.shape[1], _ptr(SA_rows), SA_rows.shape[1],
              DTYPES[tb], _ptr(B), B.shape[1], int(op_b), _ptr(SB), SB.shape[1], float(sa), float(sb),
              slot.shape[0], _ptr(slot), _ptr(cols), _ptr(out)), what)
    return out


def gemm_mx_entries(A_rows, ta, SA_rows, slot, cols, B, tb, SB, op_b=0, sa=1.0, sb=1.0) -> np.ndarray:
    """O1x at selected entries: C[row slot[t] of A_rows][cols[t]], with
    SA_rows the scale rows of A_rows."""
    return _mx_entries_call(lib().orc_gemm_mx_entries, "gemm_mx_entries", A_rows, ta, SA_rows, slot, cols, B,
                            tb, SB, op_b, sa, sb)


def gemm_mx_abs_entries(A_rows, ta, SA_rows, slot, cols, B, tb, SB, op_b=0, sa=1.0, sb=1.0) -> np.ndarray:
    """gemm_mx_abs at selected entries."""
    return _mx_entries_call(lib().orc_gemm_mx_abs_entries, "gemm_mx_abs_entries", A_rows, ta, SA_rows, slot,
                            cols, B, tb, SB, op_b, sa, sb)


def dec_e8m0(e: int) -> float:
    """An E8M0 scale: 2^(e - 127), NaN for 0xFF."""
    return lib().orc_dec_e8m0(int(e))


def _entries_call(fn, what, A_rows, ta, slot, cols, B, tb, op_b, sa, sb):
    A_rows = _codes(A_rows, ta)
    B = _codes(B, tb)
    k = A_rows.shape[1]
    slot = np.ascontiguousarray(slot, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(slot.shape[0], dtype=np.float64)
    _check(fn(k, DTYPES[ta], _ptr(A_rows), A_rows.shape[1], DTYPES[tb], _ptr(B), B.shape[1], int(op_b),
              float(sa), float(sb), slot.shape[0], _ptr(slot), _ptr(cols), _ptr(out)), what)
    return out


def gemm_entries(A_rows: np.ndarray, ta: str, slot: np.ndarray, cols: np.ndarray,
                 B: np.ndarray, tb: str, op_b: int = 0, sa: float = 1.0,
                 sb: float = 1.0) -> np.ndarray:
    """O1 at selected entries: C[row slot[t] of A_rows][cols[t]]."""
    return _entries_call(lib().orc_gemm_entries, "gemm_entries", A_rows, ta, slot, cols, B, tb, op_b, sa, sb)


def gemm_abs_entries(A_rows: np.ndarray, ta: str, slot: np.ndarray, cols: np.ndarray,
                     B: np.ndarray, tb: str, op_b: int = 0, sa: float = 1.0,
                     sb: float = 1.0) -> np.ndarray:
    """gemm_abs at selected entries (arguments as gemm_entries)."""
    return _entries_call(lib().orc_gemm_abs_entries, "gemm_abs_entries", A_rows, ta, slot, cols, B, tb,
                         op_b, sa, sb)


def bias_pass(C: np.ndarray, bias: np.ndarray, tbias: str, axis: str) -> np.ndarray:
    """O2 on a whole m x n matrix."""
    C = np.ascontiguousarray(C, dtype=np.float64)
    b = _codes(bias.reshape(-1), tbias)
    m, n = C.shape
    need = m if axis == "row" else n
    if b.size != need:
        raise ValueError(f"oracle bias: {axis} bias needs {need} values, got {b.size}")
    P = np.empty_like(C)
    _check(lib().orc_bias(m, n, _ptr(C), AXES[axis], DTYPES[tbias], _ptr(b), _ptr(P)), "bias")
    return P


def bias_entries(Cv: np.ndarray, rows: np.ndarray, cols: np.ndarray,
                 bias: np.ndarray, tbias: str, axis: str) -> np.ndarray:
    """O2 at selected entries with output coordinates (rows, cols)."""
    Cv = np.ascontiguousarray(Cv, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    b = _codes(bias.reshape(-1), tbias)
    P = np.empty_like(Cv)
    _check(lib().orc_bias_entries(Cv.size, _ptr(Cv), _ptr(rows), _ptr(cols), AXES[axis],
                                  DTYPES[tbias], _ptr(b), _ptr(P)), "bias_entries")
    return P


def act_pass(P: np.ndarray, epilog: str) -> np.ndarray:
    """O3: elementwise activation of the epilogue (identity/ReLU/GELU)."""
    P = np.ascontiguousarray(P, dtype=np.float64)
    Y = np.empty_like(P)
    _check(lib().orc_act(P.size, EPILOGS[epilog], _ptr(P), _ptr(Y)), "act")
    return Y


def act1(x: float, epilog: str) -> float:
    return lib().orc_act1(EPILOGS[epilog], float(x))


def mask_pass(P: np.ndarray, ldw: int) -> np.ndarray:
    """O4: packed ReLU sign mask, uint32 words, shape (m, ldw)."""
    P = np.ascontiguousarray(P, dtype=np.float64)
    m, n = P.shape
    W = np.empty((m, ldw), dtype=np.uint32)
    _check(lib().orc_mask(m, n, _ptr(P), ldw, _ptr(W)), "mask")
    return W


def gelu_deriv(x: float) -> float:
    """GELU'(x) of the tanh form (the derivative used by O7)."""
    return lib().orc_gelu_deriv(float(x))


def drelu_pass(C: np.ndarray, words: np.ndarray) -> np.ndarray:
    """O6: D = C where the O4 mask bit is set, else 0.  words: uint32 (m, ldw)."""
    C = np.ascontiguousarray(C, dtype=np.float64)
    m, n = C.shape
    W = np.ascontiguousarray(words, dtype=np.uint32)
    if W.shape[0] != m:
        raise ValueError("oracle drelu: mask rows differ from C's")
    D = np.empty_like(C)
    _check(lib().orc_drelu(m, n, _ptr(C), W.shape[1], _ptr(W), _ptr(D)), "drelu")
    return D


def dgelu_pass(C: np.ndarray, P: np.ndarray, tp: str) -> np.ndarray:
    """O7: D = C * GELU'(P), P given as raw codes of dtype tp, shape (m, ldp)."""
    C = np.ascontiguousarray(C, dtype=np.float64)
    m, n = C.shape
    Pc = _codes(P, tp)
    if Pc.shape[0] != m:
        raise ValueError("oracle dgelu: aux rows differ from C's")
    D = np.empty_like(C)
    _check(lib().orc_dgelu(m, n, _ptr(C), DTYPES[tp], _ptr(Pc), Pc.shape[1], _ptr(D)), "dgelu")
    return D


def add_beta_c(C: np.ndarray, beta: float, Cin: np.ndarray, tc: str) -> np.ndarray:
    """O1b: C + beta * Cin, Cin given as raw codes of dtype tc, shape (m, ldc)."""
    C = np.ascontiguousarray(C, dtype=np.float64)
    m, n = C.shape
    Cc = _codes(Cin, tc)
    if Cc.shape[0] != m:
        raise ValueError("oracle add_beta_c: rows differ")
    P0 = np.empty_like(C)
    _check(lib().orc_add_beta_c(m, n, _ptr(C), float(beta), DTYPES[tc], _ptr(Cc), Cc.shape[1], _ptr(P0)),
           "add_beta_c")
    return P0


def bgrad_pass(Y: np.ndarray, axis: str) -> np.ndarray:
    """O8: the bias gradient, Y summed along the axis the bias was not
    broadcast over (row: m values, col: n values)."""
    Y = np.ascontiguousarray(Y, dtype=np.float64)
    m, n = Y.shape
    g = np.empty(m if axis == "row" else n, dtype=np.float64)
    _check(lib().orc_bgrad(m, n, _ptr(Y), AXES[axis], _ptr(g)), "bgrad")
    return g


def reference(A, ta, B, tb, bias, tbias, epilog, axis, op_b=0, sa=1.0, sb=1.0,
              ldw=None):
    """The whole plain sequence O1 -> O2 -> O3 (-> O4).  Returns (Y, P, mask)."""
    C = gemm(A, ta, B, tb, op_b, sa, sb)
    P = C if epilog == "none" else bias_pass(C, bias, tbias, axis)
    Y = act_pass(P, epilog)
    M = mask_pass(P, ldw) if (epilog == "relu_aux_bias" and ldw is not None) else None
    return Y, P, M
