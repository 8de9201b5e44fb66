"""Pins for the CPU oracle: each checks it against something other than
itself -- hand-worked values, format definitions, closed forms, invariants,
library routines on special cases, and brute force on tiny inputs.

Each pin targets a plausible mistake: a dropped term, a wrong sign or index,
a transposed operand, a swapped bias axis, a wrong rounding rule.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def bf16_codes(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f16_codes(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


# ---- golden: hand-worked example -------------------------------------------
def test_worked_example_by_hand():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    A, B = f32(g["A"]), f32(g["B"])
    C = oracle.gemm(A, "f32", B, "f32")
    assert np.array_equal(C, np.array(g["C"], dtype=np.float64))
    for axis in ("row", "col"):
        e = g[axis]
        bias = f32(e["bias"])
        P = oracle.bias_pass(C, bias, "f32", axis)
        assert np.array_equal(P, np.array(e["P"], dtype=np.float64)), axis
        Y = oracle.act_pass(P, "relu_bias")
        assert np.array_equal(Y, np.array(e["relu"], dtype=np.float64)), axis
        M = oracle.mask_pass(P, 4)
        assert list(M[:, 0]) == e["mask_words"], axis
        assert not M[:, 1:].any()
        # the BIAS epilogue is the identity on P, NONE skips the bias
        assert np.array_equal(oracle.act_pass(P, "bias"), P)


# ---- P1: identity -------------------------------------------------------------
def test_p1_identity_selects_rows_of_b():
    m, n, k = 128, 64, 256
    rng = np.random.default_rng(1)
    A = np.zeros((m, k), np.float32)
    A[np.arange(m), np.arange(m)] = 1.0
    B = f32(rng.standard_normal((k, n)))
    C = oracle.gemm(A, "f32", B, "f32")
    assert np.array_equal(C, B[:m].astype(np.float64))


# ---- P2: permutation -------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_p2_permutation(dt):
    m = k = 37
    n = 23
    rng = np.random.default_rng(2)
    perm = rng.permutation(m)
    Pm = np.zeros((m, k), np.float32)
    Pm[np.arange(m), perm] = 1.0
    Bv = rng.standard_normal((k, n)).astype(np.float32)
    enc = {"bf16": bf16_codes, "f16": f16_codes, "f32": f32}[dt]
    Bc = enc(Bv)
    Ac = enc(Pm)
    C = oracle.gemm(Ac, dt, Bc, dt)
    Bd = oracle.decode(Bc, dt)
    assert np.array_equal(C, Bd[perm])


# ---- P3: bias axis with A = 0 ----------------------------------------------------
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("ep", ["bias", "relu_bias", "gelu_bias"])
def test_p3_zero_product_gives_activated_bias(axis, ep):
    m, n, k = 5, 7, 3
    A = np.zeros((m, k), np.float32)
    B = f32(np.random.default_rng(3).standard_normal((k, n)))
    ramp = np.arange(m if axis == "row" else n, dtype=np.float32) - 2.5  # index ramp
    Y, P, _ = oracle.reference(A, "f32", B, "f32", ramp, "f32", ep, axis)
    want_p = np.broadcast_to(ramp[:, None] if axis == "row" else ramp[None, :], (m, n))
    assert np.array_equal(P, want_p.astype(np.float64))
    for i in range(m):
        for j in range(n):
            x = ramp[i] if axis == "row" else ramp[j]
            if ep == "bias":
                assert Y[i, j] == x
            elif ep == "relu_bias":
                assert Y[i, j] == max(float(x), 0.0)
            else:
                assert Y[i, j] == oracle.act1(x, "gelu_bias")


def test_bias_shape_checked():
    C = np.zeros((3, 4))
    with pytest.raises(ValueError):
        oracle.bias_pass(C, f32([1, 2, 3, 4]), "f32", "row")


# ---- P4: integer-exact inputs ------------------------------------------------------
def test_p4_small_integer_inputs_exact():
    rng = np.random.default_rng(4)
    m, n, k = 33, 41, 300
    A = rng.integers(-16, 17, size=(m, k)).astype(np.float32)
    B = rng.integers(-16, 17, size=(k, n)).astype(np.float32)
    C = oracle.gemm(bf16_codes(A), "bf16", bf16_codes(B), "bf16")
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(C, exact.astype(np.float64))


# ---- P5: rank-1 closed form --------------------------------------------------------
def test_p5_rank_one_closed_form():
    m, n, k = 9, 11, 64
    u = np.arange(1, m + 1, dtype=np.float32) * 0.5
    v = np.arange(1, n + 1, dtype=np.float32) * -0.25
    A = np.repeat(u[:, None], k, axis=1)
    B = np.repeat(v[None, :], k, axis=0)
    C = oracle.gemm(f32(A), "f32", f32(B), "f32")
    assert np.array_equal(C, k * np.outer(u.astype(np.float64), v.astype(np.float64)))


# ---- P6: brute force on tiny shapes, both B layouts --------------------------------
@pytest.mark.parametrize("op_b", [0, 1])
def test_p6_brute_force_tiny(op_b):
    rng = np.random.default_rng(6)
    for m, n, k in itertools.product([1, 2, 3, 5], repeat=3):
        A = f32(rng.standard_normal((m, k)))
        Bkn = f32(rng.standard_normal((k, n)))
        Bstore = np.ascontiguousarray(Bkn.T) if op_b else Bkn
        C = oracle.gemm(A, "f32", Bstore, "f32", op_b=op_b)
        # explicit triple sum in Python
        for i in range(m):
            for j in range(n):
                s = 0.0
                for p in range(k):
                    s += float(A[i, p]) * float(Bkn[p, j])
                assert C[i, j] == s
        # numpy float64 matmul (library routine); equal up to summation order
        np.testing.assert_allclose(C, A.astype(np.float64) @ Bkn.astype(np.float64),
                                   rtol=1e-14, atol=1e-14)


def test_p6_leading_dimensions_and_scales():
    """Padded leading dimensions and the fp8 dequantisation factors."""
    rng = np.random.default_rng(61)
    m, n, k, lda, ldb = 4, 5, 6, 10, 7
    Af = rng.standard_normal((m, lda)).astype(np.float32)
    Bf = rng.standard_normal((k, ldb)).astype(np.float32)
    C = oracle.gemm(Af.ravel(), "f32", Bf.ravel(), "f32", 0, 0.5, 3.0,
                    m=m, n=n, k=k, lda=lda, ldb=ldb)
    want = 1.5 * (Af[:, :k].astype(np.float64) @ Bf[:, :n].astype(np.float64))
    np.testing.assert_allclose(C, want, rtol=1e-14)


def test_gemm_entries_match_brute_force():
    rng = np.random.default_rng(62)
    m, n, k = 6, 9, 17
    A = f16_codes(rng.standard_normal((m, k)))
    W = f16_codes(rng.standard_normal((n, k)))  # op_b = 1
    rows = np.array([5, 0, 3, 3])
    cols = np.array([8, 0, 2, 7])
    slot = np.arange(4)
    got = oracle.gemm_entries(np.ascontiguousarray(A[rows]), "f16", slot, cols, W, "f16", op_b=1,
                              sa=2.0, sb=0.25)
    Ad = A.view(np.float16).astype(np.float64)
    Wd = W.view(np.float16).astype(np.float64)
    for t in range(4):
        s = sum(Ad[rows[t], p] * Wd[cols[t], p] for p in range(k))
        assert got[t] == 0.5 * s
    b = f16_codes(np.arange(n) * 0.5)
    P = oracle.bias_entries(got, rows, cols, b, "f16", "col")
    assert np.array_equal(P, got + cols * 0.5)
    b2 = f16_codes(np.arange(m) * 0.25)
    P2 = oracle.bias_entries(got, rows, cols, b2, "f16", "row")
    assert np.array_equal(P2, got + rows * 0.25)


# ---- P7: ReLU and mask invariants ----------------------------------------------------
def test_p7_relu_mask_invariants():
    rng = np.random.default_rng(7)
    P = rng.standard_normal((31, 77))
    P[0, :5] = [0.0, -0.0, 1e-300, -1e-300, np.nan]
    Y = oracle.act_pass(P, "relu_bias")
    ldw = 4
    M = oracle.mask_pass(P, ldw)
    bits = np.unpackbits(M.view(np.uint8), axis=1, bitorder="little")
    assert (Y[~np.isnan(P)] >= 0).all()
    for i in range(P.shape[0]):
        for j in range(P.shape[1]):
            b = bits[i, j]
            if b:
                assert Y[i, j] == P[i, j] and P[i, j] > 0
            else:
                assert Y[i, j] == 0.0
    assert bits[:, 77:].sum() == 0  # padding bits are zero
    assert bits[0, :5].tolist() == [0, 0, 1, 0, 0]   # P == 0 -> 0, NaN -> 0


# ---- P8: GELU properties --------------------------------------------------------------
@pytest.mark.parametrize("form", ["gelu_bias", "gelu_erf"])
def test_p8_gelu_properties(form):
    g = lambda x: oracle.act1(x, form)
    assert g(0.0) == 0.0
    for x in np.linspace(-6, 6, 241):
        # x*Phi(x) - (-x)*Phi(-x) = x (Phi(x) + Phi(-x)) = x, for both forms
        assert abs((g(x) - g(-x)) - x) <= 4e-15 * max(1.0, abs(x))
    h = 1e-6
    assert abs((g(h) - g(-h)) / (2 * h) - 0.5) < 1e-9       # GELU'(0) = 1/2
    assert abs(g(30.0) - 30.0) < 1e-12 and abs(g(-30.0)) < 1e-12
    assert g(-1.0) < 0 and g(1.0) > 0.8                       # dips below zero


def test_p8_tanh_form_close_to_erf_form():
    xs = np.linspace(-8, 8, 16001)
    d = np.array([oracle.act1(x, "gelu_bias") - 0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in xs])
    mx = np.abs(d).max()
    # the tanh approximation stays within ~5e-4 of the exact form; dropping
    # the cubic term or misplacing sqrt(2/pi) gives errors of order 1e-2
    assert 4.0e-4 < mx < 5.0e-4
    assert 2.4 < abs(xs[np.abs(d).argmax()]) < 3.0


def test_p8_gelu_forms_match_library_routines():
    """Both GELU forms at fixed points against independent library routines:
    the erf form is x * Phi(x) with Phi the standard normal CDF (scipy's
    ndtr), and both forms are PyTorch's float64 GELU (its default is the erf
    form, approximate='tanh' the tanh form the pages' Linear+GELU uses).  A
    wrong argument scale (erf(x/2) for erf(x/sqrt 2)), a wrong cubic
    coefficient or a misplaced sqrt(2/pi) moves values by far more than the
    1e-13 allowed."""
    from scipy.special import ndtr
    xs = np.concatenate([np.linspace(-8.0, 8.0, 641), [-2.7, -1.0, -0.5, 0.25, 1.0, 1.96, 3.0]])
    t = torch.tensor(xs, dtype=torch.float64)
    erf_lib = torch.nn.functional.gelu(t).numpy()
    tanh_lib = torch.nn.functional.gelu(t, approximate="tanh").numpy()
    for x, e, th in zip(xs, erf_lib, tanh_lib):
        ge = oracle.act1(x, "gelu_erf")
        gt = oracle.act1(x, "gelu_bias")
        assert abs(ge - x * ndtr(x)) <= 1e-13 * max(1.0, abs(x)), x
        assert abs(ge - e) <= 1e-13 * max(1.0, abs(x)), x
        assert abs(gt - th) <= 1e-13 * max(1.0, abs(x)), x


def test_p8_gelu_deriv_matches_autograd():
    """GELU' of the tanh form against PyTorch's float64 autograd of its tanh
    GELU (a library derivative, independent of the oracle's product- and
    chain-rule expression)."""
    xs = np.linspace(-8.0, 8.0, 321)
    t = torch.tensor(xs, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(t, approximate="tanh").sum().backward()
    for x, gref in zip(xs, t.grad.numpy()):
        assert abs(oracle.gelu_deriv(x) - gref) <= 1e-13, x


# ---- the magnitude term of the element-wise error bound ---------------------------
def test_gemm_abs_pins():
    """|A|.|B| (the magnitude term of the dot-product error bound): equal to
    the product for non-negative operands, unchanged by flipping the signs of
    rows of A or of B, never below |A.B| (triangle inequality), numpy's
    float64 matmul of the absolute values on a random case, and the scale
    enters as its absolute value."""
    rng = np.random.default_rng(3)
    A = f32(rng.standard_normal((7, 11)))
    B = f32(rng.standard_normal((11, 5)))
    G = oracle.gemm_abs(A, "f32", B, "f32")
    assert np.array_equal(G, np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)))
    Ap, Bp = f32(np.abs(A)), f32(np.abs(B))
    assert np.array_equal(oracle.gemm_abs(Ap, "f32", Bp, "f32"), oracle.gemm(Ap, "f32", Bp, "f32"))
    flipA = f32(A * np.where(np.arange(7) % 2 == 0, -1.0, 1.0)[:, None])
    flipB = f32(B * np.where(np.arange(11) % 3 == 0, -1.0, 1.0)[:, None])
    assert np.array_equal(oracle.gemm_abs(flipA, "f32", flipB, "f32"), G)
    assert (np.abs(oracle.gemm(A, "f32", B, "f32")) <= G).all()
    assert np.allclose(oracle.gemm_abs(A, "f32", B, "f32", sa=-2.0, sb=0.5), G, rtol=0, atol=0)
    # the transposed layout of B and the entry form agree with the whole form
    Bt = f32(B.T)
    assert np.array_equal(oracle.gemm_abs(A, "f32", Bt, "f32", op_b=1), G)
    rows, cols = np.array([0, 3, 6, 6]), np.array([4, 0, 2, 4])
    e = oracle.gemm_abs_entries(A, "f32", rows, cols, B, "f32")
    assert np.array_equal(e, G[rows, cols])


# ---- P9: e4m3 codec ---------------------------------------------------------------------
def test_p9_e4m3_spec_points():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3_spec.json")))
    for code, val in spec["codes"].items():
        got = oracle.decode(np.array([int(code, 16)], np.uint8), "e4m3")[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in spec["nan_codes"]:
        assert math.isnan(oracle.decode(np.array([int(code, 16)], np.uint8), "e4m3")[0])


def test_p9_e4m3_table_vs_torch_and_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle.decode(codes, "e4m3")
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    fin = ~np.isnan(dec)
    assert np.array_equal(dec[fin], ref[fin])
    # encode round trip on all finite codes
    enc = oracle.encode(dec[fin], "e4m3")
    rt = oracle.decode(enc, "e4m3")
    assert np.array_equal(rt, dec[fin])
    # midpoints between neighbours tie to the even code; saturation at 448
    pos = np.sort(np.unique(dec[fin & (dec >= 0)]))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        ca, cb = oracle.encode([a], "e4m3")[0], oracle.encode([b], "e4m3")[0]
        want = ca if ca % 2 == 0 else cb
        assert oracle.encode([mid], "e4m3")[0] == want, (a, b)
    assert oracle.decode(oracle.encode([1e6, -1e6, 464.0, 480.0], "e4m3"), "e4m3").tolist() == \
        [448.0, -448.0, 448.0, 448.0]


def test_p9_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 50).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = oracle.encode(x.astype(np.float64), "e4m3")
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +0/-0 of tiny values may differ only in sign handling; compare values
    assert np.array_equal(oracle.decode(ours, "e4m3"), oracle.decode(ref, "e4m3"))


# ---- P10: fp16 / bf16 codecs ------------------------------------------------------------
def test_p10_f16_all_patterns():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    dec = oracle.decode(codes, "f16")
    ref = codes.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(dec[fin], ref[fin])


def test_p10_bf16_all_patterns():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    dec = oracle.decode(codes, "bf16")
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(dec[fin], ref[fin])


def test_p10_rne_encode_vs_libraries():
    rng = np.random.default_rng(10)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-8, 5, 5000),
                        [65504.0, 65519.0, 65520.0, 1e-8, 2.0 ** -24, 3 * 2.0 ** -25]]).astype(np.float32)
    ours16 = oracle.encode(x.astype(np.float64), "f16")
    assert np.array_equal(ours16, x.astype(np.float16).view(np.uint16))
    oursb = oracle.encode(x.astype(np.float64), "bf16")
    refb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oursb, refb)


# ---- P11: mask layout ----------------------------------------------------------------------
def test_p11_mask_layout_vs_packbits():
    rng = np.random.default_rng(11)
    m, n = 13, 200
    ldw = ((n + 127) // 128) * 128 // 32
    P = rng.standard_normal((m, n))
    W = oracle.mask_pass(P, ldw)
    bits = np.zeros((m, ldw * 32), np.uint8)
    bits[:, :n] = P > 0
    ref = np.packbits(bits, axis=1, bitorder="little").view("<u4")
    assert np.array_equal(W, ref)


# ---- training-side epilogues (O5..O7) ----------------------------------------
def test_gelu_deriv_matches_central_difference_of_gelu():
    """GELU' against a central difference of the oracle's own GELU (pinned
    above by its symmetry and limits): a dropped term of the product or chain
    rule shows as an O(1) gap, far above the O(h^2) of the difference."""
    h = 1e-5
    for x in np.linspace(-6.0, 6.0, 241):
        fd = (oracle.act1(x + h, "gelu_bias") - oracle.act1(x - h, "gelu_bias")) / (2 * h)
        assert abs(oracle.gelu_deriv(x) - fd) < 1e-8, x


def test_gelu_deriv_symmetry_and_limits():
    """GELU(x) - GELU(-x) = x gives GELU'(x) + GELU'(-x) = 1; GELU'(0) = 1/2;
    GELU' -> 1 as x -> +inf and -> 0 as x -> -inf."""
    for x in np.linspace(0.0, 8.0, 81):
        assert abs(oracle.gelu_deriv(x) + oracle.gelu_deriv(-x) - 1.0) < 1e-14
    assert oracle.gelu_deriv(0.0) == 0.5
    assert abs(oracle.gelu_deriv(10.0) - 1.0) < 1e-12
    assert abs(oracle.gelu_deriv(-10.0)) < 1e-12
    # GELU dips below zero for negative x, so its slope changes sign there
    assert oracle.gelu_deriv(-1.0) < 0.0 < oracle.gelu_deriv(-0.5)


def test_drelu_selects_by_mask_bits_vs_unpackbits():
    """O6 reads the O4 layout: checked against numpy's own bit unpacking of a
    random mask (little-endian bit order, 128-bit padded rows)."""
    rng = np.random.default_rng(7)
    m, n = 5, 200
    ldw = ((n + 127) // 128) * 4
    W = rng.integers(0, 2 ** 32, size=(m, ldw), dtype=np.uint64).astype(np.uint32)
    C = rng.standard_normal((m, n))
    D = oracle.drelu_pass(C, W)
    bits = np.unpackbits(W.view(np.uint8), axis=1, bitorder="little")[:, :n].astype(bool)
    assert np.array_equal(D, np.where(bits, C, 0.0))


def test_drelu_after_forward_mask_is_relu_derivative():
    """With C = 1, O6 applied to the O4 mask of P gives ReLU'(P) = (P > 0)."""
    rng = np.random.default_rng(8)
    P = rng.standard_normal((7, 130))
    P[0, :5] = 0.0   # ReLU'(0) = 0
    W = oracle.mask_pass(P, ((130 + 127) // 128) * 4)
    D = oracle.drelu_pass(np.ones_like(P), W)
    assert np.array_equal(D, (P > 0).astype(np.float64))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_dgelu_is_upstream_times_slope_of_gelu(dt):
    """O7 with P given as codes (padded rows): compared with a central
    difference of O3's GELU at the exactly decoded P, times C."""
    rng = np.random.default_rng(9)
    m, n, ld = 4, 50, 56
    Pf = (rng.standard_normal((m, ld)) * 2).astype(np.float32)
    codes = {"f32": lambda x: x, "f16": f16_codes, "bf16": bf16_codes}[dt](Pf)
    Pd = oracle.decode(np.ascontiguousarray(codes), dt)[:, :n]
    C = rng.standard_normal((m, n))
    D = oracle.dgelu_pass(C, np.ascontiguousarray(codes), dt)
    h = 1e-5
    slope = (oracle.act_pass(Pd + h, "gelu_bias") - oracle.act_pass(Pd - h, "gelu_bias")) / (2 * h)
    assert np.allclose(D, C * slope, rtol=0, atol=1e-8)


def test_bgrad_sums_along_the_other_axis():
    """O8 against numpy's sums on a non-square matrix (an axis swap changes
    the length), and exact counts for an all-ones backward result."""
    rng = np.random.default_rng(10)
    Y = rng.standard_normal((7, 12))
    assert np.allclose(oracle.bgrad_pass(Y, "row"), Y.sum(axis=1), rtol=0, atol=1e-12)
    assert np.allclose(oracle.bgrad_pass(Y, "col"), Y.sum(axis=0), rtol=0, atol=1e-12)
    ones = np.ones((5, 9))
    assert np.array_equal(oracle.bgrad_pass(ones, "row"), np.full(5, 9.0))
    assert np.array_equal(oracle.bgrad_pass(ones, "col"), np.full(9, 5.0))


def test_bgrad_of_drelu_counts_mask_bits():
    """With C = 1, the DRELU result is the mask itself, so its bias gradient
    counts the set bits of each row (row axis) or column (col axis)."""
    rng = np.random.default_rng(11)
    m, n = 6, 140
    P = rng.standard_normal((m, n))
    W = oracle.mask_pass(P, ((n + 127) // 128) * 4)
    Y = oracle.drelu_pass(np.ones((m, n)), W)
    bits = np.unpackbits(W.view(np.uint8), axis=1, bitorder="little")[:, :n]
    assert np.array_equal(oracle.bgrad_pass(Y, "row"), bits.sum(axis=1).astype(np.float64))
    assert np.array_equal(oracle.bgrad_pass(Y, "col"), bits.sum(axis=0).astype(np.float64))


def test_tanh_epilogue_properties():
    """O3 for TANH_BIAS: odd, zero at zero, bounded by 1 and saturating,
    slope 1 at 0, and equal to 2*sigmoid(2x) - 1 (a different closed form)."""
    xs = np.linspace(-9.0, 9.0, 181)
    ys = oracle.act_pass(xs, "tanh_bias")
    assert np.allclose(ys, -oracle.act_pass(-xs, "tanh_bias"), rtol=0, atol=0)
    assert oracle.act1(0.0, "tanh_bias") == 0.0
    assert np.all(np.abs(ys) <= 1.0) and abs(ys[-1] - 1.0) < 1e-7
    h = 1e-6
    assert abs((oracle.act1(h, "tanh_bias") - oracle.act1(-h, "tanh_bias")) / (2 * h) - 1.0) < 1e-9
    assert np.allclose(ys, 2.0 / (1.0 + np.exp(-2.0 * xs)) - 1.0, rtol=0, atol=1e-15)


def test_tanh_epilogue_after_zero_product_gives_tanh_of_bias():
    """A = 0: D = tanh(bias) along the bias axis (P3 for the Tanh epilogue)."""
    m, n, k = 3, 4, 5
    bias = f32([0.5, -1.0, 2.0])
    Y, P, _ = oracle.reference(f32(np.zeros((m, k))), "f32", f32(np.ones((k, n))), "f32",
                               bias, "f32", "tanh_bias", "row")
    assert np.allclose(Y, np.tanh(np.repeat(bias.astype(np.float64)[:, None], n, axis=1)), rtol=0, atol=1e-15)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_gemm_scale_factors_any_dtype(dt):
    """O1's factor sa*sb applies to every input dtype: with small integers the
    product is exact, so the scaled result is exactly sa*sb times it."""
    rng = np.random.default_rng(12)
    A = rng.integers(-4, 5, (6, 9)).astype(np.float32)
    B = rng.integers(-4, 5, (9, 7)).astype(np.float32)
    enc = {"f32": lambda x: x, "f16": f16_codes, "bf16": bf16_codes}[dt]
    C1 = oracle.gemm(np.ascontiguousarray(enc(A)), dt, np.ascontiguousarray(enc(B)), dt)
    Cs = oracle.gemm(np.ascontiguousarray(enc(A)), dt, np.ascontiguousarray(enc(B)), dt, 0, 0.5, 3.0)
    assert np.array_equal(C1, A.astype(np.float64) @ B.astype(np.float64))
    assert np.array_equal(Cs, 1.5 * C1)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_add_beta_c_exact_cases(dt):
    """O1b: beta = 0 leaves the product; A = 0 leaves beta * C exactly (small
    integers); the result is linear in beta (padded C rows)."""
    rng = np.random.default_rng(13)
    m, n, ld = 4, 6, 8
    Cin = rng.integers(-8, 9, (m, ld)).astype(np.float32)
    codes = np.ascontiguousarray({"f32": lambda x: x, "f16": f16_codes, "bf16": bf16_codes}[dt](Cin))
    P = rng.standard_normal((m, n))
    assert np.array_equal(oracle.add_beta_c(P, 0.0, codes, dt), P)
    Z = np.zeros((m, n))
    assert np.array_equal(oracle.add_beta_c(Z, 2.5, codes, dt), 2.5 * Cin[:, :n].astype(np.float64))
    d = oracle.add_beta_c(Z, 3.0, codes, dt) - oracle.add_beta_c(Z, 1.0, codes, dt)
    assert np.array_equal(d, 2.0 * Cin[:, :n].astype(np.float64))


# ---- O1x: block-scaled fp8 (one E8M0 scale per 32 K values) --------------------------
def e4m3_codes_of_ints(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e8m0_codec_from_the_format_definition():
    """E8M0 (OCP Microscaling formats): an unsigned 8-bit exponent, bias 127,
    no mantissa; 0xFF is NaN."""
    assert oracle.dec_e8m0(127) == 1.0
    assert oracle.dec_e8m0(128) == 2.0 and oracle.dec_e8m0(126) == 0.5
    assert oracle.dec_e8m0(0) == 2.0 ** -127 and oracle.dec_e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.dec_e8m0(255))


def test_mx_unit_scales_reduce_to_the_per_tensor_product():
    rng = np.random.default_rng(11)
    m, n, k = 7, 9, 100                      # a ragged last block of 4
    A = e4m3_codes_of_ints(rng.integers(-6, 7, (m, k)))
    for op_b in (0, 1):
        B = e4m3_codes_of_ints(rng.integers(-6, 7, (n, k) if op_b else (k, n)))
        ones_a = np.full((m, 4), 127, np.uint8)
        ones_b = np.full((n, 4), 127, np.uint8)
        C = oracle.gemm_mx(A, "e4m3", ones_a, B, "e4m3", ones_b, op_b, 0.5, 3.0)
        assert np.array_equal(C, oracle.gemm(A, "e4m3", B, "e4m3", op_b, 0.5, 3.0))


def test_mx_power_of_two_scales_exact_on_integer_codes_brute_force():
    """Integer codes times powers of two are exact in float64, so the whole
    sum is: compare with exact rational arithmetic on tiny shapes."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    for m, n, k in itertools.product((1, 2, 3), (1, 2, 5), (1, 31, 32, 33, 70)):
        kb = (k + 31) // 32
        Ai = rng.integers(-8, 9, (m, k))
        Bi = rng.integers(-8, 9, (k, n))
        SA = rng.integers(117, 138, (m, kb)).astype(np.uint8)
        SB = rng.integers(117, 138, (n, kb)).astype(np.uint8)
        C = oracle.gemm_mx(e4m3_codes_of_ints(Ai), "e4m3", SA, e4m3_codes_of_ints(Bi), "e4m3", SB)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(int(Ai[i, p]) * int(Bi[p, j])) *
                            Fraction(2) ** (int(SA[i, p // 32]) + int(SB[j, p // 32]) - 254) for p in range(k))
                assert C[i, j] == float(exact), (m, n, k, i, j)


def test_mx_block_index_and_layouts():
    """Raising one scale of row i, block b by one (x2) adds exactly block b's
    share of row i; B given n x k with the same SB gives the same product; a
    NaN scale (0xFF) poisons only the row it belongs to; the absolute form
    bounds the product."""
    rng = np.random.default_rng(13)
    m, n, k = 4, 6, 96
    Ai = rng.integers(-5, 6, (m, k))
    Bi = rng.integers(-5, 6, (k, n))
    A, Bn, Bt = e4m3_codes_of_ints(Ai), e4m3_codes_of_ints(Bi), e4m3_codes_of_ints(Bi.T)
    SA = rng.integers(120, 135, (m, 3)).astype(np.uint8)
    SB = rng.integers(120, 135, (n, 3)).astype(np.uint8)
    C = oracle.gemm_mx(A, "e4m3", SA, Bn, "e4m3", SB, 0)
    assert np.array_equal(C, oracle.gemm_mx(A, "e4m3", SA, Bt, "e4m3", SB, 1))
    SA2 = SA.copy()
    SA2[2, 1] += 1
    C2 = oracle.gemm_mx(A, "e4m3", SA2, Bn, "e4m3", SB, 0)
    share = np.array([sum(Ai[2, p] * Bi[p, j] * 2.0 ** (int(SA[2, 1]) + int(SB[j, 1]) - 254)
                          for p in range(32, 64)) for j in range(n)])
    assert np.array_equal(C2[2] - C[2], share)
    assert np.array_equal(np.delete(C2, 2, 0), np.delete(C, 2, 0))
    SAn = SA.copy()
    SAn[1, 0] = 0xFF
    Cn = oracle.gemm_mx(A, "e4m3", SAn, Bn, "e4m3", SB, 0)
    assert np.isnan(Cn[1]).all() and np.isfinite(np.delete(Cn, 1, 0)).all()
    G = oracle.gemm_mx_abs(A, "e4m3", SA, Bn, "e4m3", SB, 0)
    assert (np.abs(C) <= G).all()


def test_mx_entries_match_the_whole_product():
    rng = np.random.default_rng(14)
    m, n, k = 5, 7, 80
    A = e4m3_codes_of_ints(rng.integers(-6, 7, (m, k)))
    for op_b in (0, 1):
        B = e4m3_codes_of_ints(rng.integers(-6, 7, (n, k) if op_b else (k, n)))
        SA = rng.integers(118, 136, (m, 16)).astype(np.uint8)
        SB = rng.integers(118, 136, (n, 16)).astype(np.uint8)
        C = oracle.gemm_mx(A, "e4m3", SA, B, "e4m3", SB, op_b, 2.0, 0.25)
        G = oracle.gemm_mx_abs(A, "e4m3", SA, B, "e4m3", SB, op_b, 2.0, 0.25)
        rows, cols = np.array([0, 4, 2, 2, 1]), np.array([6, 0, 3, 3, 5])
        assert np.array_equal(oracle.gemm_mx_entries(A, "e4m3", SA, rows, cols, B, "e4m3", SB, op_b, 2.0, 0.25),
                              C[rows, cols])
        assert np.array_equal(oracle.gemm_mx_abs_entries(A, "e4m3", SA, rows, cols, B, "e4m3", SB, op_b, 2.0, 0.25),
                              G[rows, cols])
