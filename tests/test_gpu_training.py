"""GPU parity of the training-side epilogues against the CPU oracle:
GELU_AUX_BIAS (GELU forward that also stores the pre-activation), DRELU and
DGELU (the backward product scaled by ReLU' from a stored mask or by GELU'
of a stored pre-activation).  Every dtype combination and B layout, every
tile shape, ragged tails, padded leading dimensions, the unfused pair, the
forward -> backward hand-over of the aux buffer, integer-exact inputs, and
the full 8192^3 shape in the launch configuration bench.py times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (check_full, check_sampled, codes, decode_output, make_aux_input, rel_fro,
                    run_library, tolerance)

pytestmark = pytest.mark.gpu

TRAIN = ["gelu_aux_bias", "drelu", "dgelu", "drelu_bgrad", "dgelu_bgrad"]
COMBOS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("bf16", "f32"), ("e4m3", "bf16")]


def wl(m, n, k, a, d, ep, axis="row", op_b=0, seed=7):
    return synth.Workload("t", "test", m, n, k, a, d, ep, axis, op_b, seed,
                          ("normal", 1.0), ("normal", 1.0), ("normal", 1.0))


@pytest.mark.parametrize("a,d", COMBOS, ids=[f"{a}->{d}" for a, d in COMBOS])
@pytest.mark.parametrize("ep", TRAIN)
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("op_b", [0, 1])
def test_training_epilogues_ragged(a, d, ep, axis, op_b):
    # 150 x 200 x 136: several 64-wide tiles with ragged tails, padded rows
    w = wl(150, 200, 136, a, d, ep, axis, op_b)
    r = run_library(w, synth.make_inputs(w), pad=1, path=1)
    check_full(w, r)


TILES = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f32"), ("e4m3", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("op_b", [0, 1])
def test_training_epilogues_every_tile(tile, a, d, op_b):
    if a == "f32" and tile > 4:
        pytest.skip("the pipelined tiles take 16-bit and fp8 inputs only")
    if a == "e4m3" and tile in (13, 14):
        pytest.skip("the pipelined 64x64 tile takes 16-bit inputs only")
    if a != "e4m3" and tile == 16:
        pytest.skip("tile 16 (64-byte fp8 K steps) takes fp8 inputs only")
    k = 456 if a == "e4m3" else 200
    cases = [(ep, "col") for ep in TRAIN] + [("drelu_bgrad", "row"), ("dgelu_bgrad", "row")]
    if tile == 14:   # the split-K tile does not take the bias-gradient epilogues
        cases = [c for c in cases if not c[0].endswith("_bgrad")]
    for ep, axis in cases:
        w = wl(300, 520, k, a, d, ep, axis, op_b, seed=tile)
        r = run_library(w, synth.make_inputs(w), pad=2, path=1, tile=tile)
        check_full(w, r)


@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("e4m3", "bf16")])
@pytest.mark.parametrize("ep", TRAIN)
def test_training_unfused_pair(a, d, ep):
    w = wl(260, 300, 96, a, d, ep, "row", 0, seed=5)
    inp = synth.make_inputs(w)
    aux_in = make_aux_input(w) if ep != "gelu_aux_bias" else None
    ru = run_library(w, inp, pad=1, unfused=1, aux_in=aux_in)
    assert "unfused=1" in ru.desc
    check_full(w, ru)
    rf = run_library(w, inp, pad=1, aux_in=aux_in)
    # the pair rounds the product to D's dtype first: two roundings apart
    assert rel_fro(decode_output(w, ru), decode_output(w, rf)) <= 2 * tolerance(a, d)


@pytest.mark.parametrize("tile", [1, 11, 13])
def test_forward_mask_and_preactivation_feed_backward(tile):
    """The aux buffer a forward epilogue writes is what the backward one
    reads: RELU_AUX_BIAS -> DRELU and GELU_AUX_BIAS -> DGELU, both on the
    device, checked against the oracle on the forward's own output bytes."""
    m, n, k = 260, 390, 160
    for fwd, bwd in (("relu_aux_bias", "drelu"), ("gelu_aux_bias", "dgelu")):
        wf = wl(m, n, k, "bf16", "bf16", fwd, "row", 0, seed=21)
        rf = run_library(wf, synth.make_inputs(wf), path=1, tile=tile)
        check_full(wf, rf)
        wb = wl(m, n, 96, "bf16", "bf16", bwd, "row", 0, seed=22)
        rb = run_library(wb, synth.make_inputs(wb), path=1, tile=tile, aux_in=rf.aux)
        check_full(wb, rb)


@pytest.mark.parametrize("tile", [1, 3, 7, 11])
@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f32", "f32")])
def test_drelu_integer_bit_exact(tile, a, d):
    """Integer inputs keep the product exact, and DRELU only selects, so D
    is the RNE encoding of the masked exact product bit for bit."""
    if a == "f32" and tile > 4:
        pytest.skip("fp32 inputs take the register-staged tiles")
    m, n, k = 384, 512, 520
    w = wl(m, n, k, a, d, "drelu", "row", 0)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4))
    r = run_library(w, inp, path=1, tile=tile)
    from parity import oracle_full
    Y, _, _ = oracle_full(w, r)
    want = Y.astype(np.float32) if d == "f32" else oracle.encode(Y, d).reshape(Y.shape)
    assert np.array_equal(codes(r.D)[:, :n], want)


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("mnk", [(0, 70, 40), (50, 0, 40), (50, 70, 0), (1, 1, 1)])
def test_bias_gradient_degenerate_shapes(axis, mnk):
    """An empty sum is zero: m = 0 (col axis) or n = 0 (row axis) still
    writes the gradient; k = 0 gives D = 0 and a zero gradient."""
    m, n, k = mnk
    w = wl(m, n, k, "bf16", "bf16", "dgelu_bgrad", axis, 0, seed=3)
    ru8 = lambda x: max(8, (x + 7) // 8 * 8)   # 16-byte rows
    r = run_library(w, synth.make_inputs(w), path=1, lda=ru8(k), ldb=ru8(n), ldd=ru8(n))
    got = oracle.decode(np.ascontiguousarray(codes(r.bias)), "bf16")
    if m and n:
        check_full(w, r)
    else:
        assert np.array_equal(got, np.zeros_like(got))


def test_dgelu_bgrad_full_size():
    """bf16 DGELU_BGRAD at 8192^3 in the planner's launch configuration: D
    sampled (4096 entries + 16 rows) and the bias gradient of 8 columns, each
    a sum over all 8192 rows, from the oracle's own GEMM of those columns."""
    w = synth.WORKLOADS["F1d"]
    inp = synth.make_inputs(w, device="cuda")
    r = run_library(w, inp, path=0, aux_in=synth.make_aux(w, device="cuda"))
    assert "tile_id=6 " in r.desc, r.desc
    check_sampled(w, r, seed=w.seed)
    cols = np.array([0, 1, 255, 256, 4095, 4096, 8190, 8191], dtype=np.int64)
    Ac = codes(r.A)[:, : w.k]
    Bsel = np.ascontiguousarray(codes(r.B)[: w.k][:, cols])
    C = oracle.gemm(np.ascontiguousarray(Ac), "bf16", Bsel, "bf16")
    Y = oracle.dgelu_pass(C, np.ascontiguousarray(codes(r.aux)[:, cols]), "bf16")
    want = oracle.bgrad_pass(Y, "col")
    got = oracle.decode(np.ascontiguousarray(codes(r.bias)[cols]), "bf16")
    assert rel_fro(got, want) <= tolerance("bf16", "bf16"), (got, want)


def test_dgelu_full_size_sampled():
    """bf16 DGELU at 8192^3 (the backward of the 8192^3 GELU workload) in
    the launch configuration the planner picks: 4096 entries + 16 rows."""
    w = synth.WORKLOADS["F1b"]
    inp = synth.make_inputs(w, device="cuda")
    r = run_library(w, inp, path=0, aux_in=synth.make_aux(w, device="cuda"))
    assert "tile_id=6 " in r.desc, r.desc
    check_sampled(w, r, seed=w.seed)


def test_gelu_aux_full_size_sampled():
    w = synth.WORKLOADS["F1a"]
    inp = synth.make_inputs(w, device="cuda")
    r = run_library(w, inp, path=0)
    assert "tile_id=6 " in r.desc, r.desc
    check_sampled(w, r, seed=w.seed)
