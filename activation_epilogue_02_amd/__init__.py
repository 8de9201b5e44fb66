"""Fused GEMM + bias/activation epilogue for AMD MI355X (gfx950).

D = epilogue(A*B + bias) in one hand-written HIP kernel, behind the C ABI in
include/gemm_epilog.h.  ``binding`` is the thin ctypes layer with the ABI's
names; ``build`` compiles the library in-tree with hipcc.
"""
from .binding import (GE_BIAS_COL, GE_BIAS_ROW, GE_EPILOG_BIAS, GE_EPILOG_DGELU,  # noqa: F401
                      GE_EPILOG_DGELU_BGRAD, GE_EPILOG_DRELU, GE_EPILOG_DRELU_BGRAD,
                      GE_EPILOG_GELU_AUX_BIAS, GE_EPILOG_GELU_BIAS, GE_EPILOG_NONE,
                      GE_EPILOG_RELU_AUX_BIAS, GE_EPILOG_RELU_BIAS, GE_EPILOG_TANH_BIAS, GE_F8_E4M3,
                      GE_F16, GE_F32, GE_BF16, GE_MXF8_E4M3, GE_OP_N, GE_OP_T, GemmEpilog, GemmEpilogError,
                      gemm_epilog_autotune, gemm_epilog_aux_ld, gemm_epilog_create,
                      gemm_epilog_describe, gemm_epilog_execute, gemm_epilog_execute_c,
                      gemm_epilog_execute_static, gemm_epilog_execute_mx, mx_scale_ld,
                      gemm_epilog_execute_m, gemm_epilog_set_batch_strides, ge_batch_strides,
                      gemm_epilog_set_fp8_output,
                      gemm_epilog_free, gemm_epilog_plan,
                      gemm_epilog_status_string, gemm_epilog_workspace_size, ge_desc, ge_pref,
                      make_desc)
