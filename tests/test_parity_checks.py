"""CPU checks of the parity checkers themselves (no GPU).

A device result is simulated with an ordinary fp32 computation (torch's CPU
matmul, its own summation order, then the bias, the activation and an RNE
conversion): the per-element bound must accept it.  Then single, localised
mistakes are planted in that simulated result -- one row's bias taken from
the next row, one 32 x 32 block scaled by 1.02, a small-|Y| region of a GELU
output shifted -- and the per-element bound must reject each, including the
ones the relative Frobenius gate alone would let through.
"""
import numpy as np
import pytest
import torch

import synth
from parity import Result, check_full, check_sampled, oracle_parts, rel_fro, tolerance

TD = synth.TORCH_DTYPE


def simulate(w, inp, ldd=None):
    """An fp32 device-like result of the whole epilogue on the CPU."""
    A = inp.A.float()
    B = inp.B.float()
    Bm = B.T if w.op_b else B
    s = 1.0
    if inp.scale_a is not None:
        s = float(inp.scale_a) * float(inp.scale_b)
    C = (A @ Bm) * s
    b = inp.bias.reshape(-1).float()
    P = C + (b[:, None] if w.axis == "row" else b[None, :])
    if w.epilog in ("relu_bias", "relu_aux_bias"):
        Y = torch.relu(P)
    elif w.epilog == "gelu_bias":
        Y = torch.nn.functional.gelu(P, approximate="tanh")
    elif w.epilog == "tanh_bias":
        Y = torch.tanh(P)
    else:
        Y = P
    ldd = ldd or w.n
    D = torch.full((w.m, ldd), float("nan"), dtype=TD[w.out_dtype])
    D[:, : w.n] = Y.to(TD[w.out_dtype])
    return D, P


def result(w, inp, D):
    return Result(D=D, aux=None, A=inp.A.contiguous(), B=inp.B.contiguous(), bias=inp.bias.reshape(-1),
                  sa=inp.scale_a, sb=inp.scale_b, lda=w.k, ldb=(w.k if w.op_b else w.n), ldd=D.shape[1],
                  desc="simulated", cin=None, beta=None, ldw=None)


def wl(m, n, k, a, d, ep, axis="row", op_b=0, seed=5):
    return synth.Workload("t", "sim", m, n, k, a, d, ep, axis, op_b, seed,
                          ("normal", 1.0), ("normal", 1.0), ("normal", 1.0))


CASES = [("bf16", "bf16", "relu_bias"), ("f16", "f16", "gelu_bias"), ("bf16", "f32", "bias"),
         ("f32", "f32", "tanh_bias"), ("e4m3", "bf16", "relu_bias"), ("f16", "f32", "gelu_bias")]


@pytest.mark.parametrize("a,d,ep", CASES)
@pytest.mark.parametrize("axis", ["row", "col"])
def test_simulated_fp32_result_passes(a, d, ep, axis):
    w = wl(150, 200, 136, a, d, ep, axis)
    inp = synth.make_inputs(w)
    D, _ = simulate(w, inp)
    check_full(w, result(w, inp, D))


def test_wrong_bias_on_one_row_is_caught_by_the_bound_not_the_norm():
    # 1500 rows: one wrong row of 1500 moves the norm by less than 5e-3
    w = wl(1500, 200, 136, "bf16", "bf16", "relu_bias", "row")
    inp = synth.make_inputs(w)
    D, P = simulate(w, inp)
    b = inp.bias.reshape(-1).float()
    # a row whose neighbour's bias differs by 0.3 .. 0.6: well above the
    # output's rounding, well below what moves the norm of 1500 rows
    d = (b[1:] - b[:-1]).abs()
    i = int(torch.nonzero((d > 0.3) & (d < 0.6))[0])
    bad = torch.relu(P[i] - b[i] + b[i + 1])
    D[i, : w.n] = bad.to(torch.bfloat16)
    r = result(w, inp, D)
    o = oracle_parts(w, r)
    from parity import decode_output
    assert rel_fro(decode_output(w, r), o.Y) <= tolerance("bf16", "bf16")   # the norm alone passes
    with pytest.raises(AssertionError, match="per-element bound"):
        check_full(w, r)


def test_one_scaled_block_is_caught():
    # one 32 x 32 block of 1500 x 200 off by 3%: under the norm's 5e-3,
    # about eight times the bf16 rounding of each element
    w = wl(1500, 200, 136, "bf16", "bf16", "bias", "col")
    inp = synth.make_inputs(w)
    D, _ = simulate(w, inp)
    D[64:96, 32:64] = (D[64:96, 32:64].float() * 1.03).to(torch.bfloat16)
    r = result(w, inp, D)
    from parity import decode_output
    assert rel_fro(decode_output(w, r), oracle_parts(w, r).Y) <= tolerance("bf16", "bf16")
    with pytest.raises(AssertionError, match="per-element bound"):
        check_full(w, r)


def test_gelu_small_region_shift_is_caught():
    w = wl(150, 200, 136, "f16", "f16", "gelu_bias", "col")
    inp = synth.make_inputs(w)
    D, P = simulate(w, inp)
    region = (P.abs() < 0.5)
    Df = D[:, : w.n].float()
    Df[region] += 2e-3
    D[:, : w.n] = Df.to(torch.float16)
    r = result(w, inp, D)
    with pytest.raises(AssertionError, match="per-element bound"):
        check_full(w, r)


def test_fp8_systematic_scale_error_is_caught():
    w = wl(150, 200, 456, "e4m3", "bf16", "relu_bias", "row")
    inp = synth.make_inputs(w)
    inp.scale_a = inp.scale_a * 1.03      # a 3% scale error
    D, _ = simulate(w, inp)
    inp.scale_a = inp.scale_a / 1.03
    with pytest.raises(AssertionError):
        check_full(w, result(w, inp, D))


def test_sampled_check_accepts_simulated_and_catches_one_wrong_row():
    w = wl(600, 300, 512, "bf16", "bf16", "relu_bias", "row", seed=9)
    inp = synth.make_inputs(w)
    D, P = simulate(w, inp)
    r = result(w, inp, D)
    check_sampled(w, r, 123)
    # row m-1 is always among the full rows of the sample
    b = inp.bias.reshape(-1).float()
    D[w.m - 1, : w.n] = torch.relu(P[w.m - 1] - b[w.m - 1] + 0.5).to(torch.bfloat16)
    with pytest.raises(AssertionError):
        check_sampled(w, result(w, inp, D), 123)
