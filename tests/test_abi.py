"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, and every validation path returns its status before any HIP
call.  No call here ever reaches a kernel launch: every execute() below fails
validation (or hits the launch-failure test hook) on purpose, since the
pointers are fake."""
import ctypes
import os
import re

import pytest

import activation_epilogue_02_amd as ge
from activation_epilogue_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000  # 16-byte aligned, never dereferenced (validation fails first)


def header_functions():
    src = open(os.path.join(ROOT, "include", "gemm_epilog.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(gemm_epilog_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 8
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n


def test_single_hip_runtime_loaded():
    import torch  # noqa: F401
    B.lib()
    maps = open("/proc/self/maps").read()
    hips = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hips) == 1, hips


def desc(**kw):
    d = dict(m=64, n=48, k=40, a_type="bf16", d_type="bf16", op_b=0)
    d.update(kw)
    return B.make_desc(**d)


def status_of(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except B.GemmEpilogError as e:
        return e.status
    return B.GE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(m=-1), B.GE_ERR_SHAPE), (dict(n=-1), B.GE_ERR_SHAPE), (dict(k=-1), B.GE_ERR_SHAPE),
    (dict(m=-3), B.GE_ERR_SHAPE), (dict(k=2 ** 31), B.GE_ERR_SHAPE),
    (dict(lda=32), B.GE_ERR_SHAPE), (dict(ldb=40), B.GE_ERR_SHAPE), (dict(ldd=40), B.GE_ERR_SHAPE),
    (dict(op_b=1, ldb=32), B.GE_ERR_SHAPE), (dict(op_b=2), B.GE_ERR_SHAPE),
    (dict(lda=44), B.GE_ERR_ALIGN), (dict(ldd=52), B.GE_ERR_ALIGN), (dict(ldb=52), B.GE_ERR_ALIGN),
    (dict(a_type="f32", d_type="bf16"), B.GE_ERR_DTYPE),
    (dict(a_type="bf16", d_type="f16"), B.GE_ERR_DTYPE),
    (dict(a_type="f16", d_type="bf16"), B.GE_ERR_DTYPE),
    (dict(a_type="e4m3", d_type="e4m3", k=64, bias_type="e4m3"), B.GE_ERR_DTYPE),   # fp8 D takes a bf16 bias
    (dict(a_type="f16", d_type="e4m3", bias_type="f16"), B.GE_ERR_DTYPE),
    (dict(a_type="f32", d_type="e4m3"), B.GE_ERR_DTYPE),
    (dict(d_type="e4m3", ldd=56), B.GE_ERR_ALIGN),   # 56-byte fp8 rows
    (dict(b_type="f16"), B.GE_ERR_DTYPE),
    (dict(bias_type="f32"), B.GE_ERR_DTYPE),
    (dict(a_type="e4m3", d_type="bf16", k=40), B.GE_ERR_ALIGN),   # 40-byte rows
])
def test_create_rejects(kw, code):
    assert status_of(B.gemm_epilog_create, desc(**kw)) == code


@pytest.mark.parametrize("kw", [
    dict(), dict(a_type="f32", d_type="f32"), dict(a_type="f16", d_type="f16"),
    dict(a_type="f16", d_type="f32"), dict(a_type="bf16", d_type="f32"),
    dict(a_type="e4m3", d_type="bf16", k=48), dict(a_type="e4m3", d_type="f16", k=48),
    dict(a_type="e4m3", d_type="f32", k=48), dict(a_type="e4m3", d_type="bf16", k=40, lda=48),
    dict(op_b=1), dict(m=1, n=1, k=1, lda=8, ldb=8, ldd=8),
])
def test_create_accepts(kw):
    h = B.gemm_epilog_create(desc(**kw))
    B.gemm_epilog_free(h)


def test_null_arguments():
    L = B.lib()
    d = desc()
    assert L.gemm_epilog_create(None, ctypes.byref(d)) == B.GE_ERR_NULL
    h = ctypes.c_void_p()
    assert L.gemm_epilog_create(ctypes.byref(h), None) == B.GE_ERR_NULL
    assert L.gemm_epilog_plan(None, 1, 0, None) == B.GE_ERR_NULL
    assert L.gemm_epilog_free(None) == B.GE_OK
    s = ctypes.c_size_t()
    assert L.gemm_epilog_workspace_size(None, ctypes.byref(s)) == B.GE_ERR_NULL
    assert L.gemm_epilog_execute(None, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None) == B.GE_ERR_NULL


def test_plan_validation_and_state():
    h = B.gemm_epilog_create(desc())
    try:
        assert status_of(B.gemm_epilog_workspace_size, h) == B.GE_ERR_STATE
        assert status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_STATE
        assert status_of(B.gemm_epilog_plan, h, 11, 0) == B.GE_ERR_EPILOG
        assert status_of(B.gemm_epilog_plan, h, -1, 0) == B.GE_ERR_EPILOG
        assert status_of(B.gemm_epilog_plan, h, 1, 2) == B.GE_ERR_EPILOG
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(0, 0, 99, 0)) == B.GE_ERR_SHAPE
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(2, 0, 0, 0)) == B.GE_ERR_SHAPE  # small-m: m > 16
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(0, 2, 0, 0)) == B.GE_ERR_SHAPE
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(1, 0, 0, 4)) == B.GE_ERR_SHAPE  # split on tile
        # a failed plan leaves the handle unplanned
        assert status_of(B.gemm_epilog_workspace_size, h) == B.GE_ERR_STATE
        B.gemm_epilog_plan(h, "relu_aux_bias", "row")
        assert B.gemm_epilog_workspace_size(h) == 0
        assert B.gemm_epilog_aux_ld(h) == 128
        assert "path=tile" in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)


def test_execute_validation_paths():
    h = B.gemm_epilog_create(desc())
    try:
        B.gemm_epilog_plan(h, "relu_aux_bias", "row")
        ex = lambda *a, **k: status_of(B.gemm_epilog_execute, h, *a, **k)
        assert ex(None, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_NULL
        assert ex(FAKE, None, FAKE, FAKE, FAKE) == B.GE_ERR_NULL
        assert ex(FAKE, FAKE, FAKE, None, FAKE) == B.GE_ERR_NULL
        assert ex(FAKE, FAKE, None, FAKE, FAKE) == B.GE_ERR_NULL            # bias required
        assert ex(FAKE, FAKE, FAKE, FAKE, None) == B.GE_ERR_EPILOG          # aux required
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, None) == B.GE_ERR_ALIGN  # alpha pointer
        assert ex(FAKE + 2, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_ALIGN
        assert ex(FAKE, FAKE + 8, FAKE, FAKE, FAKE) == B.GE_ERR_ALIGN
        assert ex(FAKE, FAKE, FAKE + 4, FAKE, FAKE) == B.GE_ERR_ALIGN
        assert ex(FAKE, FAKE, FAKE, FAKE + 2, FAKE) == B.GE_ERR_ALIGN
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE + 4) == B.GE_ERR_ALIGN
        B.gemm_epilog_plan(h, "bias", "col")
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_EPILOG          # aux not expected
        B.gemm_epilog_plan(h, "bias", "col", B.ge_pref(0, 1, 0, 0))         # unfused needs workspace
        ws = B.gemm_epilog_workspace_size(h)
        assert ws >= 64 * 48 * 2 and ws % 256 == 0
        assert ex(FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_WORKSPACE
        assert ex(FAKE, FAKE, FAKE, FAKE, workspace=FAKE, workspace_bytes=ws - 1) == B.GE_ERR_WORKSPACE
        assert ex(FAKE, FAKE, FAKE, FAKE, workspace=FAKE + 8, workspace_bytes=ws) == B.GE_ERR_ALIGN
    finally:
        B.gemm_epilog_free(h)


def test_training_epilogues_validation():
    """GELU_AUX_BIAS needs a bias and writes a pre-activation matrix (row
    stride round_up(n,128) elements); DRELU and DGELU read an aux input, take
    no bias (ignored) and keep the mask / matrix strides."""
    for d_type, bits in (("bf16", 16), ("f32", 32)):
        a_type = "bf16" if d_type == "bf16" else "f32"
        h = B.gemm_epilog_create(desc(a_type=a_type, d_type=d_type, n=200, ldb=200, ldd=200))
        try:
            ex = lambda *a, **k: status_of(B.gemm_epilog_execute, h, *a, **k)
            B.gemm_epilog_plan(h, "gelu_aux_bias", "col")
            assert B.gemm_epilog_aux_ld(h) == 256 * bits
            assert ex(FAKE, FAKE, None, FAKE, FAKE) == B.GE_ERR_NULL      # bias required
            assert ex(FAKE, FAKE, FAKE, FAKE, None) == B.GE_ERR_EPILOG    # aux required
            assert ex(FAKE, FAKE, FAKE, FAKE, FAKE + 8) == B.GE_ERR_ALIGN
            B.gemm_epilog_plan(h, "dgelu", "row")
            assert B.gemm_epilog_aux_ld(h) == 256 * bits
            assert ex(FAKE, FAKE, FAKE, FAKE, None) == B.GE_ERR_EPILOG    # aux input required
            B.gemm_epilog_plan(h, "drelu", "row")
            assert B.gemm_epilog_aux_ld(h) == 256                          # the mask's stride
            assert ex(FAKE, FAKE, FAKE, FAKE, None) == B.GE_ERR_EPILOG
            assert ex(FAKE, FAKE, FAKE, FAKE, FAKE + 4) == B.GE_ERR_ALIGN
            B.gemm_epilog_plan(h, "dgelu", "row", B.ge_pref(0, 1, 0, 0))  # unfused pair
            assert B.gemm_epilog_workspace_size(h) >= 64 * 200 * (bits // 8)
        finally:
            B.gemm_epilog_free(h)


def test_bias_gradient_workspace_and_validation():
    """The bias-gradient epilogues write the gradient to the bias pointer
    (required) and need fp32 partials: one per tile row (col axis) or tile
    column (row axis) and gradient entry; the unfused pair one per 256-row or
    -column block."""
    h = B.gemm_epilog_create(B.make_desc(1000, 600, 64, "bf16", "bf16", 0))
    try:
        ex = lambda *a, **k: status_of(B.gemm_epilog_execute, h, *a, **k)
        r256 = lambda x: (x + 255) // 256 * 256
        B.gemm_epilog_plan(h, "dgelu_bgrad", "col", B.ge_pref(1, 0, 11, 0))   # 256 x 256 tiles
        assert B.gemm_epilog_workspace_size(h) == r256(4 * 600 * 4)
        assert ex(FAKE, FAKE, None, FAKE, FAKE, workspace=FAKE, workspace_bytes=1 << 20) == B.GE_ERR_NULL
        assert ex(FAKE, FAKE, FAKE, FAKE, None, workspace=FAKE, workspace_bytes=1 << 20) == B.GE_ERR_EPILOG
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_WORKSPACE
        B.gemm_epilog_plan(h, "drelu_bgrad", "row", B.ge_pref(1, 0, 11, 0))
        assert B.gemm_epilog_workspace_size(h) == r256(3 * 1000 * 4)
        assert B.gemm_epilog_aux_ld(h) == 640                                  # the mask's stride
        B.gemm_epilog_plan(h, "dgelu_bgrad", "col", B.ge_pref(0, 1, 0, 0))    # unfused pair
        assert B.gemm_epilog_workspace_size(h) == r256(1000 * 600 * 2) + r256(4 * 600 * 4)
        assert B.gemm_epilog_aux_ld(h) == 640 * 16
    finally:
        B.gemm_epilog_free(h)


def test_training_epilogues_take_the_tile_path():
    """The small-m kernel serves the inference epilogues only: automatic
    planning of a batch-16 Linear with a training epilogue takes the tile
    kernel, and forcing the small-m path is refused."""
    h = B.gemm_epilog_create(B.make_desc(16, 4096, 4096, "f16", "f16", 1))
    try:
        for ep in ("gelu_aux_bias", "drelu", "dgelu", "drelu_bgrad", "dgelu_bgrad"):
            B.gemm_epilog_plan(h, ep, "col")
            assert "path=tile" in B.gemm_epilog_describe(h)
            assert status_of(B.gemm_epilog_plan, h, ep, "col", B.ge_pref(2, 0, 0, 0)) == B.GE_ERR_EPILOG
        B.gemm_epilog_plan(h, "gelu_bias", "col")
        assert "path=smallm" in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)


def test_autotune_prechecks():
    """Checks that fail before anything runs: no handle, no plan, iters < 1."""
    L = B.lib()
    assert L.gemm_epilog_autotune(None, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, 5, None,
                                  None) == B.GE_ERR_NULL
    h = B.gemm_epilog_create(desc())
    try:
        assert status_of(B.gemm_epilog_autotune, h, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_STATE
        B.gemm_epilog_plan(h, "bias", "row")
        assert status_of(B.gemm_epilog_autotune, h, FAKE, FAKE, FAKE, FAKE, iters=0) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


def test_batch_validation_and_workspace():
    """batch 0 or 1 is one product; up to 65535 products; the workspace of
    the unfused pair and of the small-m split scales with the batch."""
    assert status_of(B.gemm_epilog_create, B.make_desc(64, 48, 40, "bf16", "bf16", batch=-1)) == B.GE_ERR_SHAPE
    assert status_of(B.gemm_epilog_create, B.make_desc(64, 48, 40, "bf16", "bf16", batch=65536)) == B.GE_ERR_SHAPE
    r256 = lambda x: (x + 255) // 256 * 256
    sizes = {}
    for nb in (0, 1, 3):
        h = B.gemm_epilog_create(B.make_desc(64, 48, 40, "bf16", "bf16", batch=nb))
        try:
            B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(0, 1, 0, 0))
            sizes[nb] = B.gemm_epilog_workspace_size(h)
        finally:
            B.gemm_epilog_free(h)
    assert sizes[0] == sizes[1] == r256(64 * 48 * 2) and sizes[3] == r256(3 * 64 * 48 * 2)
    h = B.gemm_epilog_create(B.make_desc(16, 4096, 4096, "f16", "f16", 1, batch=2))
    try:
        B.gemm_epilog_plan(h, "gelu_bias", "col", B.ge_pref(2, 0, 0, 4))
        assert B.gemm_epilog_workspace_size(h) == r256(2 * 4 * 256 * 256 * 4) + r256(2 * 256 * 4)
    finally:
        B.gemm_epilog_free(h)


def test_execute_c_validation():
    """execute_c's own checks fail before anything runs."""
    h = B.gemm_epilog_create(desc())
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        L = B.lib()
        ex = lambda C, ldc, beta: L.gemm_epilog_execute_c(h, FAKE, FAKE, C, ldc, beta, FAKE, FAKE, None, None,
                                                          None, None, 0, None)
        assert ex(FAKE, 48, None) == B.GE_ERR_NULL        # beta
        assert ex(None, 48, FAKE) == B.GE_ERR_NULL        # C
        assert ex(FAKE, 40, FAKE) == B.GE_ERR_SHAPE       # ldc < n
        assert ex(FAKE, 52, FAKE) == B.GE_ERR_ALIGN       # ldc * 2 bytes not a multiple of 16
        assert ex(FAKE + 8, 48, FAKE) == B.GE_ERR_ALIGN   # C
        assert ex(FAKE, 48, FAKE + 2) == B.GE_ERR_ALIGN   # beta
        assert L.gemm_epilog_execute_c(None, FAKE, FAKE, FAKE, 48, FAKE, FAKE, FAKE, None, None, None, None, 0,
                                       None) == B.GE_ERR_NULL
    finally:
        B.gemm_epilog_free(h)


def test_fp8_scales_alignment():
    h = B.gemm_epilog_create(desc(a_type="e4m3", d_type="bf16", k=48))
    try:
        B.gemm_epilog_plan(h, "relu_bias", "row")
        assert status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE, None, FAKE + 2, None) == B.GE_ERR_ALIGN
    finally:
        B.gemm_epilog_free(h)


def test_forced_launch_failure_hook(monkeypatch):
    # the hook returns GE_ERR_HIP after validation and before any launch
    monkeypatch.setenv("GE_TEST_FAIL_LAUNCH", "1")
    h = B.gemm_epilog_create(desc())
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_HIP
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("m,n,k,op_b,a,expect", [
    (16, 4096, 4096, 1, "f16", "path=smallm"),
    (1, 4096, 4096, 1, "bf16", "path=smallm"),
    (16, 4096, 4096, 0, "f16", "path=tile"),       # B given k x n: tile path
    (17, 4096, 4096, 1, "f16", "path=tile"),
    (16, 4096, 4096, 1, "f32", "path=tile"),
    (8192, 8192, 8192, 0, "bf16", "tile=256x256 waves=2x4 tile_id=6 kernel=2 stages=4"),
    (65536, 8192, 16384, 0, "bf16", "tile_id=6 kernel=2 stages=4 grid=8192 group_m=4 "),
    (65536, 8192, 16384, 0, "e4m3", "tile=256x256 waves=2x4 tile_id=16 kernel=6 stages=4 grid=8192 group_m=4 "),
    (4096, 4096, 1024, 0, "e4m3", "tile=256x128 waves=4x2 tile_id=15 kernel=2 stages=3"),
    (4096, 1024, 4096, 1, "f16", "tile_id=8 kernel=2"),
    (1024, 512, 2048, 0, "f16", "tile=64x64 waves=2x2 tile_id=13 kernel=4 stages=4"),
    (256, 256, 65536, 0, "bf16", "tile=64x64 waves=2x2 tile_id=14 kernel=5 stages=4 grid=16 group_m=4 split_k=8 "),
    (128, 64, 256, 0, "f32", "tile=64x64"),
])
def test_planner_choices(m, n, k, op_b, a, expect):
    d_type = "bf16" if a == "e4m3" else a
    h = B.gemm_epilog_create(B.make_desc(m, n, k, a, d_type, op_b))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert expect in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("a,tile,rot", [("bf16", 6, 0), ("e4m3", 16, 1), ("mxf8", 8, 2)])
def test_k_rotation_choice(a, tile, rot, monkeypatch):
    """The planner rotates the K order of the pipelined tiles where it was
    measured to help (the block-scaled 128 x 128 tile by 2 steps, the fp8
    64-byte-step tile by 1); GE_K_STAGGER overrides it, 0 turning it off."""
    monkeypatch.delenv("GE_K_STAGGER", raising=False)
    h = B.gemm_epilog_create(B.make_desc(65536, 8192, 16384, a, "bf16", 0))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        s = B.gemm_epilog_describe(h)
        assert f"tile_id={tile} " in s and s.endswith(f" k_stagger={rot}"), s
        monkeypatch.setenv("GE_K_STAGGER", "3")
        B.gemm_epilog_plan(h, "bias", "row")
        assert B.gemm_epilog_describe(h).endswith(" k_stagger=3")
        monkeypatch.setenv("GE_K_STAGGER", "0")
        B.gemm_epilog_plan(h, "bias", "row")
        assert B.gemm_epilog_describe(h).endswith(" k_stagger=0")
    finally:
        B.gemm_epilog_free(h)
    # the small-m path has no K order to rotate
    monkeypatch.setenv("GE_K_STAGGER", "3")
    h = B.gemm_epilog_create(B.make_desc(16, 4096, 4096, "bf16", "bf16", 1))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert "path=smallm" in B.gemm_epilog_describe(h)
        assert B.gemm_epilog_describe(h).endswith(" k_stagger=0")
    finally:
        B.gemm_epilog_free(h)


def test_group_order_preference():
    """group_m: 0 = the planner's choice, n > 0 = n tile rows per group
    (clamped to the tile rows there are), negative = GE_ERR_SHAPE."""
    h = B.gemm_epilog_create(B.make_desc(4096, 4096, 1024, "bf16", "bf16", 0))
    try:
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(0, 0, 0, 0, -1)) == B.GE_ERR_SHAPE
        B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(0, 0, 6, 0, 3))
        assert " group_m=3 " in B.gemm_epilog_describe(h)
        B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(0, 0, 6, 0, 1000))
        assert " group_m=16 " in B.gemm_epilog_describe(h)   # 4096 / 256 tile rows
        B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(0, 0, 2, 0, 0))
        assert " group_m=8 " in B.gemm_epilog_describe(h)    # register-staged tile
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("a,op_b", [("bf16", 0), ("bf16", 1), ("e4m3", 1)])
def test_pipelined_tiles_need_rows_within_4_gib(a, op_b):
    """The pipelined tiles address a tile's rows as 32-bit offsets from its
    first row: with rows of 128 MiB the automatic
    plan takes the register-staged kernel and a forced pipelined tile is
    refused; a span of exactly 4 GiB keeps the pipelined tile (the 4096 x
    4096 plan takes 128-row tiles for bf16, 256-row ones for fp8)."""
    big = 1 << 26 if a == "bf16" else 1 << 27   # 128 MiB per row
    h = B.gemm_epilog_create(B.make_desc(4096, 4096, 64, a, "bf16", 0, lda=big))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert "kernel=1 " in B.gemm_epilog_describe(h)
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(0, 0, 5, 0)) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)
    if op_b == 1:   # B given n x k: its rows count too
        h = B.gemm_epilog_create(B.make_desc(4096, 4096, 64, a, "bf16", 1, ldb=big))
        try:
            B.gemm_epilog_plan(h, "bias", "row")
            assert "kernel=1 " in B.gemm_epilog_describe(h)
        finally:
            B.gemm_epilog_free(h)
    ok = 1 << 24   # 128 rows of 32 MiB (bf16) or 256 rows of 16 MiB (fp8): 4 GiB
    h = B.gemm_epilog_create(B.make_desc(4096, 4096, 64, a, "bf16", op_b, lda=ok))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert "kernel=1 " not in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)


def test_block_scaled_plan_refuses_rows_beyond_4_gib():
    h = B.gemm_epilog_create(B.make_desc(4096, 4096, 64, "mxf8", "bf16", 1, lda=1 << 26))
    try:
        assert status_of(B.gemm_epilog_plan, h, 1, 0, None) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("tile", [5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16])
def test_pipelined_tiles_reject_fp32_inputs(tile):
    h = B.gemm_epilog_create(B.make_desc(512, 512, 512, "f32", "f32", 0))
    try:
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(1, 0, tile, 0)) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("tile", [16])
def test_fp8_deep_tiles_take_fp8_only(tile):
    """Tile 16 (256 x 256, 8 waves, 64-byte fp8 K steps, four stages) serves
    fp8 inputs only; id 17 does not exist."""
    for a, d, ok in (("e4m3", "bf16", True), ("bf16", "bf16", False), ("f16", "f16", False)):
        h = B.gemm_epilog_create(B.make_desc(512, 512, 512, a, d, 0))
        try:
            st = status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(1, 0, tile, 0))
            assert st == (B.GE_OK if ok else B.GE_ERR_SHAPE), a
            if ok:
                assert f"tile_id={tile} kernel=6 stages=4 " in B.gemm_epilog_describe(h)
        finally:
            B.gemm_epilog_free(h)
    h = B.gemm_epilog_create(B.make_desc(512, 512, 512, "e4m3", "bf16", 0))
    try:
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(1, 0, 17, 0)) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


def test_small_pipelined_tile_rejects_fp8():
    h = B.gemm_epilog_create(B.make_desc(512, 512, 512, "e4m3", "bf16", 0))
    try:
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(1, 0, 13, 0)) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("m,n,k,tile,split", [
    (128, 128, 65536, 14, 16), (256, 256, 4096, 14, 4), (256, 256, 8192, 14, 8), (256, 256, 65536, 14, 8),
    (256, 512, 32768, 14, 8), (512, 512, 4096, 14, 2), (512, 512, 8192, 14, 4), (512, 512, 16384, 14, 4),
    (1024, 512, 8192, 14, 2), (1024, 512, 16384, 14, 2), (1024, 512, 2048, 13, 1), (1024, 1024, 8192, 13, 1),
    (256, 256, 2048, 13, 1),
])
def test_split_k_planner_choice(m, n, k, tile, split):
    """The planner's split-K choice on the shapes it was measured on: the
    split tile for at most 64 tiles with k >= 4096 or at most 128 with
    k >= 8192; slices of 16 or more K steps (32 beyond 128 workgroups), at
    most 256 workgroups, at most 8 slices (16 for at most 4 tiles)."""
    h = B.gemm_epilog_create(B.make_desc(m, n, k, "bf16", "bf16", 0))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        s = B.gemm_epilog_describe(h)
        assert f"tile_id={tile} " in s and f" split_k={split} " in s, s
    finally:
        B.gemm_epilog_free(h)


def test_split_k_tile_plan():
    """Tile 14 (the 64x64 tile with split-K): 16-bit inputs only, no
    bias-gradient epilogues, partials (tiles x split x 64 x 64 fp32) and one
    counter per tile in the workspace; other tiles refuse a split."""
    h = B.gemm_epilog_create(B.make_desc(1024, 512, 2048, "f16", "f16", 0))
    try:
        B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(1, 0, 14, 0))
        assert "tile_id=14" in B.gemm_epilog_describe(h) and "split_k=1 " in B.gemm_epilog_describe(h)
        # 32 K steps over 128 tiles: two slices would pass 128 workgroups
        # with fewer than 32 steps each, so the tile stays unsplit
        assert B.gemm_epilog_workspace_size(h) == 0
        B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(1, 0, 14, 4))
        assert B.gemm_epilog_workspace_size(h) == 128 * 4 * 64 * 64 * 4 + 512
        B.gemm_epilog_plan(h, "bias", "row", B.ge_pref(1, 0, 14, 3))
        assert "split_k=3 " in B.gemm_epilog_describe(h)
        assert status_of(B.gemm_epilog_plan, h, "bias", "row", B.ge_pref(1, 0, 13, 3)) == B.GE_ERR_SHAPE
        assert status_of(B.gemm_epilog_plan, h, "dgelu_bgrad", "col", B.ge_pref(1, 0, 14, 0)) == B.GE_ERR_EPILOG
        B.gemm_epilog_plan(h, "dgelu_bgrad", "col")     # automatic: the unsplit tile
        assert "tile_id=13" in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)
    h = B.gemm_epilog_create(B.make_desc(256, 256, 65536, "bf16", "bf16", 0))
    try:
        B.gemm_epilog_plan(h, "dgelu_bgrad", "col")     # a bias gradient never takes the split tile
        assert "tile_id=13" in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)
    h = B.gemm_epilog_create(B.make_desc(512, 512, 2048, "e4m3", "bf16", 0))
    try:
        assert status_of(B.gemm_epilog_plan, h, 1, 0, B.ge_pref(1, 0, 14, 0)) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


def test_smallm_row_groups_plan():
    """group_m on the small-m path: 1, 2 or 4 row groups per wave (blocks of
    16 * g columns, partials of 256 * g floats per slice and block); other
    values are refused."""
    h = B.gemm_epilog_create(B.make_desc(16, 1000, 4096, "f16", "f16", 1))
    try:
        for g in (1, 2, 4):
            B.gemm_epilog_plan(h, "gelu_bias", "col", B.ge_pref(2, 0, 0, 4, g))
            s = B.gemm_epilog_describe(h)
            tiles = (1000 + 16 * g - 1) // (16 * g)
            assert f"tile=16x{16 * g} " in s and f"grid={tiles * 4} " in s and f"group_m={g} " in s, s
            assert B.gemm_epilog_workspace_size(h) == 4 * tiles * 256 * g * 4 + ((tiles * 4 + 255) // 256) * 256
        for g in (3, 8, -1):
            assert status_of(B.gemm_epilog_plan, h, "gelu_bias", "col", B.ge_pref(2, 0, 0, 0, g)) == B.GE_ERR_SHAPE
    finally:
        B.gemm_epilog_free(h)


def test_smallm_split_workspace():
    h = B.gemm_epilog_create(B.make_desc(16, 4096, 4096, "f16", "f16", 1))
    try:
        B.gemm_epilog_plan(h, "gelu_bias", "col", B.ge_pref(2, 0, 0, 4))
        s = B.gemm_epilog_describe(h)
        assert "split_k=4" in s
        assert B.gemm_epilog_workspace_size(h) == 4 * 256 * 256 * 4 + 1024
    finally:
        B.gemm_epilog_free(h)


@pytest.mark.parametrize("m,n,k,split", [
    (16, 4096, 4096, 1),     # 256 column blocks already fill the 256 CUs
    (16, 2048, 14336, 2),
    (16, 1024, 16384, 4),
    (16, 512, 8192, 8),
    (16, 128, 65536, 32),
    (4, 1024, 1024, 1),      # 32 K steps: 4 per wave leaves no room to split
    (1, 1024, 2048, 2),
    (16, 8192, 4096, 1),     # two 16-row groups per wave: 256 blocks of 32 columns
    (16, 8160, 4096, 1),     # 255 such blocks: one group
    (16, 28672, 4096, 1),
])
def test_smallm_auto_split(m, n, k, split):
    """Without a preference the small-m path splits K while the grid stays
    within one workgroup per CU and each wave keeps >= 2 spans of 64 K values;
    two row groups per wave once 32-column blocks fill the 256 CUs."""
    h = B.gemm_epilog_create(B.make_desc(m, n, k, "bf16", "bf16", 1))
    try:
        B.gemm_epilog_plan(h, "bias", "col")
        s = B.gemm_epilog_describe(h)
        rg = 2 if (n + 31) // 32 >= 256 else 1
        assert "path=smallm" in s and f"split_k={split} " in s and f"group_m={rg} " in s, s
        tiles_n = (n + 16 * rg - 1) // (16 * rg)
        assert f"grid={tiles_n * split} " in s, s
        ws = B.gemm_epilog_workspace_size(h)
        assert ws == (0 if split == 1 else split * tiles_n * rg * 1024 + ((tiles_n * 4 + 255) // 256) * 256)
        # an explicit preference still wins
        B.gemm_epilog_plan(h, "bias", "col", B.ge_pref(2, 0, 0, 1))
        assert "split_k=1 " in B.gemm_epilog_describe(h)
    finally:
        B.gemm_epilog_free(h)


def test_status_strings():
    for s in range(11):
        assert B.gemm_epilog_status_string(s).startswith("GE_")
    assert B.gemm_epilog_status_string(123) == "unknown status"


def test_package_api_names():
    for n in header_functions():
        assert hasattr(ge, n), n


def test_execute_static_validation():
    """The fixed-workspace execute validates like execute and refuses plans
    whose workspace exceeds the library's array, all before any HIP call."""
    h = B.gemm_epilog_create(desc())
    try:
        ex = lambda *a: status_of(B.gemm_epilog_execute_static, h, *a)
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_STATE          # not planned
        B.gemm_epilog_plan(h, "relu_aux_bias", "row")
        assert ex(None, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_NULL
        assert ex(FAKE, FAKE, FAKE, FAKE, None) == B.GE_ERR_EPILOG
        assert ex(FAKE + 2, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_ALIGN
    finally:
        B.gemm_epilog_free(h)
    # an unfused pair whose intermediate (4096 x 4096 bf16 = 32 MiB) exceeds
    # the 16 MiB array
    big = B.gemm_epilog_create(B.make_desc(4096, 4096, 64, "bf16", "bf16"))
    try:
        B.gemm_epilog_plan(big, "bias", "row", B.ge_pref(0, 1, 0, 0))
        assert B.gemm_epilog_workspace_size(big) > B.GE_STATIC_WORKSPACE_BYTES
        assert status_of(B.gemm_epilog_execute_static, big, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_STATIC_LIMIT
    finally:
        B.gemm_epilog_free(big)


def test_batched_column_bias_alignment():
    """A batched COL bias read by the epilogue needs n * element size to be a
    multiple of 16 bytes (product b's bias starts b*n values in); a ROW bias,
    a single product and the gradient outputs do not."""
    def plan_status(n, batch, ep, axis):
        h = B.gemm_epilog_create(B.make_desc(64, n, 40, "bf16", "bf16", ldd=(n + 7) // 8 * 8,
                                             ldb=(n + 7) // 8 * 8, batch=batch))
        try:
            return status_of(B.gemm_epilog_plan, h, ep, axis)
        finally:
            B.gemm_epilog_free(h)
    assert plan_status(201, 3, "bias", "col") == B.GE_ERR_ALIGN
    assert plan_status(201, 3, "gelu_bias", "col") == B.GE_ERR_ALIGN
    assert plan_status(200, 3, "bias", "col") == B.GE_OK
    assert plan_status(201, 1, "bias", "col") == B.GE_OK
    assert plan_status(201, 3, "bias", "row") == B.GE_OK
    assert plan_status(201, 3, "dgelu_bgrad", "col") == B.GE_OK


def test_mx_dtype_validation_and_planner():
    """Block-scaled fp8: bf16/f16/f32/e4m3 outputs, the 128 x 128 tile only;
    the scales come with execute_mx, and only with it."""
    assert status_of(B.gemm_epilog_create, B.make_desc(64, 48, 64, "mxf8", "f16")) == B.GE_OK
    assert status_of(B.gemm_epilog_create, B.make_desc(64, 48, 64, "mxf8", "e4m3", ldd=64)) == B.GE_OK
    assert status_of(B.gemm_epilog_create, B.make_desc(64, 48, 64, "mxf8", "e4m3", bias_type="e4m3")) == \
        B.GE_ERR_DTYPE
    assert status_of(B.gemm_epilog_create, B.make_desc(64, 48, 64, "mxf8", "bf16", b_type="e4m3")) == B.GE_ERR_DTYPE
    h = B.gemm_epilog_create(B.make_desc(4096, 4096, 4096, "mxf8", "bf16"))
    try:
        B.gemm_epilog_plan(h, "relu_bias", "row")
        assert "tile_id=8 " in B.gemm_epilog_describe(h)
        assert status_of(B.gemm_epilog_plan, h, "relu_bias", "row", B.ge_pref(0, 0, 15, 0)) == B.GE_ERR_SHAPE
        assert status_of(B.gemm_epilog_plan, h, "relu_bias", "row", B.ge_pref(2, 0, 0, 0)) == B.GE_ERR_SHAPE
        B.gemm_epilog_plan(h, "relu_bias", "row")
        ex = lambda *a: status_of(B.gemm_epilog_execute_mx, h, *a)
        assert ex(FAKE, FAKE, None, FAKE, FAKE, FAKE) == B.GE_ERR_NULL        # A's scales missing
        assert ex(FAKE, FAKE, FAKE, None, FAKE, FAKE) == B.GE_ERR_NULL        # B's scales missing
        assert ex(FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE) == B.GE_ERR_ALIGN
        assert ex(FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE) == B.GE_ERR_ALIGN
        # the per-tensor entry points have no scales to give
        assert status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_NULL
        assert status_of(B.gemm_epilog_execute_static, h, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_NULL
    finally:
        B.gemm_epilog_free(h)
    h = B.gemm_epilog_create(B.make_desc(64, 48, 64, "e4m3", "bf16"))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert status_of(B.gemm_epilog_execute_mx, h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_DTYPE
    finally:
        B.gemm_epilog_free(h)
    assert B.mx_scale_ld(1) == 16 and B.mx_scale_ld(512) == 16 and B.mx_scale_ld(513) == 32
    assert B.mx_scale_ld(16384) == 512


def test_batch_strides_validation(monkeypatch):
    """set_batch_strides checks signs; execute checks overlap and alignment
    before any launch (the hook stops a call that passed validation)."""
    monkeypatch.setenv("GE_TEST_FAIL_LAUNCH", "1")
    m, n, k, nb = 64, 48, 32, 3
    S = B.ge_batch_strides
    assert B.lib().gemm_epilog_set_batch_strides(None, None) == B.GE_ERR_NULL
    h = B.gemm_epilog_create(B.make_desc(m, n, k, "bf16", "bf16", 0, batch=nb))
    try:
        B.gemm_epilog_plan(h, "relu_aux_bias", "col")
        ldw = B.gemm_epilog_aux_ld(h) // 32
        ex = lambda: status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE, FAKE)
        assert status_of(B.gemm_epilog_set_batch_strides, h, S(-1, 0, 0, m * n, m * ldw)) == B.GE_ERR_SHAPE
        # shared weight and bias, gaps between products: valid
        B.gemm_epilog_set_batch_strides(h, S(m * k + 8, 0, 0, m * n + n, m * ldw + 4))
        assert ex() == B.GE_ERR_HIP
        # D of two products would overlap
        B.gemm_epilog_set_batch_strides(h, S(m * k, 0, 0, m * n - 8, m * ldw))
        assert ex() == B.GE_ERR_SHAPE
        # the mask rows of two products would overlap
        B.gemm_epilog_set_batch_strides(h, S(m * k, 0, 0, m * n, m * ldw - 4))
        assert ex() == B.GE_ERR_SHAPE
        # a product's A, D or mask rows would not start 16-byte aligned
        for s in (S(m * k + 1, 0, 0, m * n, m * ldw), S(m * k, 0, 0, m * n + 4, m * ldw),
                  S(m * k, 0, 0, m * n, m * ldw + 1), S(m * k, 4, 0, m * n, m * ldw)):
            B.gemm_epilog_set_batch_strides(h, s)
            assert ex() == B.GE_ERR_ALIGN, (s.a, s.b, s.d, s.aux)
        # a COL bias is read 16 bytes at a time
        B.gemm_epilog_set_batch_strides(h, S(m * k, 0, n + 1, m * n, m * ldw))
        assert ex() == B.GE_ERR_ALIGN
        # a ROW bias one element at a time: any stride
        B.gemm_epilog_plan(h, "relu_aux_bias", "row")
        B.gemm_epilog_set_batch_strides(h, S(m * k, 0, m + 1, m * n, m * ldw))
        assert ex() == B.GE_ERR_HIP
        # a bias gradient (an output) needs its own n entries per product
        B.gemm_epilog_plan(h, "drelu_bgrad", "col")
        B.gemm_epilog_set_batch_strides(h, S(m * k, 0, n - 8, m * n, m * ldw))
        assert status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=FAKE,
                         workspace_bytes=1 << 30) == B.GE_ERR_SHAPE
        # back to the packed layout
        B.gemm_epilog_set_batch_strides(h, None)
        B.gemm_epilog_plan(h, "relu_aux_bias", "col")
        assert ex() == B.GE_ERR_HIP
    finally:
        B.gemm_epilog_free(h)


def test_execute_m_validation(monkeypatch):
    monkeypatch.setenv("GE_TEST_FAIL_LAUNCH", "1")
    h = B.gemm_epilog_create(B.make_desc(100, 64, 32, "bf16", "bf16", 0))
    try:
        ex = lambda m: status_of(B.gemm_epilog_execute_m, h, m, FAKE, FAKE, FAKE, FAKE)
        assert ex(10) == B.GE_ERR_STATE   # not planned
        B.gemm_epilog_plan(h, "bias", "row")
        assert ex(101) == B.GE_ERR_SHAPE
        assert ex(-1) == B.GE_ERR_SHAPE
        assert ex(100) == B.GE_ERR_HIP and ex(37) == B.GE_ERR_HIP and ex(0) == B.GE_ERR_HIP
        assert status_of(B.gemm_epilog_execute_m, h, 37, FAKE, FAKE, None, FAKE) == B.GE_ERR_NULL   # bias
    finally:
        B.gemm_epilog_free(h)
    h = B.gemm_epilog_create(B.make_desc(100, 64, 32, "mxf8", "bf16", 1))
    try:
        B.gemm_epilog_plan(h, "bias", "row")
        assert status_of(B.gemm_epilog_execute_m, h, 50, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_DTYPE
    finally:
        B.gemm_epilog_free(h)


def test_fp8_output_validation(monkeypatch):
    """E4M3 output: bf16 bias only, inference epilogues in the fused kernel,
    the instantiated tiles, no C input; set_fp8_output on other handles."""
    monkeypatch.setenv("GE_TEST_FAIL_LAUNCH", "1")
    assert B.lib().gemm_epilog_create(ctypes.byref(ctypes.c_void_p()),
                                      ctypes.byref(B.make_desc(64, 64, 64, "bf16", "e4m3", 0,
                                                               bias_type="e4m3"))) == B.GE_ERR_DTYPE
    for a in ("bf16", "f16", "e4m3", "mxf8"):
        h = B.gemm_epilog_create(B.make_desc(256, 256, 64, a, "e4m3", 0))
        try:
            for ep in ("gelu_aux_bias", "drelu", "dgelu", "drelu_bgrad", "dgelu_bgrad"):
                assert status_of(B.gemm_epilog_plan, h, ep, "row") == B.GE_ERR_DTYPE, (a, ep)
            assert status_of(B.gemm_epilog_plan, h, "relu_bias", "row", B.ge_pref(0, 1, 0, 0)) == B.GE_ERR_DTYPE
            assert status_of(B.gemm_epilog_plan, h, "relu_bias", "row", B.ge_pref(1, 0, 11, 0)) == B.GE_ERR_SHAPE
            assert status_of(B.gemm_epilog_plan, h, "relu_bias", "row", B.ge_pref(1, 0, 2, 0)) == B.GE_ERR_SHAPE
            assert status_of(B.gemm_epilog_plan, h, "relu_bias", "row", B.ge_pref(1, 0, 16, 0)) == \
                (B.GE_OK if a == "e4m3" else B.GE_ERR_SHAPE), a
            B.gemm_epilog_plan(h, "relu_aux_bias", "row")
            assert status_of(B.gemm_epilog_set_fp8_output, h, FAKE + 2, None) == B.GE_ERR_ALIGN
            B.gemm_epilog_set_fp8_output(h, FAKE, FAKE + 4)
            if a != "mxf8":
                assert status_of(B.gemm_epilog_execute, h, FAKE, FAKE, FAKE, FAKE, FAKE) == B.GE_ERR_HIP
                assert L_execute_c(h) == B.GE_ERR_DTYPE
        finally:
            B.gemm_epilog_free(h)
    h = B.gemm_epilog_create(B.make_desc(64, 64, 64, "bf16", "bf16", 0))
    try:
        assert status_of(B.gemm_epilog_set_fp8_output, h, None, None) == B.GE_ERR_DTYPE
    finally:
        B.gemm_epilog_free(h)
    assert B.lib().gemm_epilog_set_fp8_output(None, None, None) == B.GE_ERR_NULL


def L_execute_c(h):
    return B.lib().gemm_epilog_execute_c(h, FAKE, FAKE, FAKE, 256, FAKE, FAKE, FAKE, FAKE, None, None, None, 0,
                                         None)
