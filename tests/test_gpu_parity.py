"""GPU parity: the HIP library (through its C ABI) against the CPU oracle,
element by element, on seeded inputs.  Sizes span several tiles with ragged
tails; every dtype combination, epilogue, bias axis and B layout; padded
leading dimensions with NaN-poisoned padding (it must never be read, and D's
padding must never be written); the small-m path with and without split-K;
the unfused pair; integer-exact inputs (bit-exact); determinism.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_full, codes, decode_output, rel_fro, run_library, tolerance

pytestmark = pytest.mark.gpu

COMBOS = [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
          ("e4m3", "bf16"), ("e4m3", "f16"), ("e4m3", "f32")]
EPILOGS = ["none", "bias", "relu_bias", "relu_aux_bias", "gelu_bias", "tanh_bias"]


def wl(m, n, k, a, d, ep, axis="row", op_b=0, seed=7, **kw):
    base = synth.Workload("t", "test", m, n, k, a, d, ep, axis, op_b, seed,
                          ("normal", 1.0), ("normal", 1.0), ("normal", 1.0))
    return synth.scaled(base, **kw) if kw else base


def case_id(*a):
    return "-".join(str(x) for x in a)


@pytest.mark.parametrize("a,d", COMBOS, ids=[f"{a}->{d}" for a, d in COMBOS])
@pytest.mark.parametrize("ep", EPILOGS)
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("op_b", [0, 1])
def test_tile_all_combos_ragged(a, d, ep, axis, op_b):
    # 150 x 200 x 136: three 64-row tiles, four 64-column tiles, ragged tails
    w = wl(150, 200, 136, a, d, ep, axis, op_b)
    inp = synth.make_inputs(w)
    r = run_library(w, inp, pad=1, path=1)
    check_full(w, r)


@pytest.mark.parametrize("tile", [1, 2, 3, 4])
@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("e4m3", "bf16")])
@pytest.mark.parametrize("op_b", [0, 1])
def test_every_tile_shape(tile, a, d, op_b):
    # several 256-wide tiles plus tails in m, n and k
    w = wl(300, 520, 200, a, d, "relu_aux_bias", "row", op_b, seed=11)
    inp = synth.make_inputs(w)
    r = run_library(w, inp, pad=2, path=1, tile=tile)
    check_full(w, r)


PIPELINED = [5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16]
COMBOS16 = [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f16", "f32"),
            ("e4m3", "bf16"), ("e4m3", "f16"), ("e4m3", "f32")]


def skip_unsupported(tile, a):
    if tile in (13, 14) and a == "e4m3":
        pytest.skip("the pipelined 64x64 tile takes 16-bit inputs only (planner rejects fp8)")
    if tile == 16 and a != "e4m3":
        pytest.skip("tile 16 (64-byte fp8 K steps) takes fp8 inputs only")


@pytest.mark.parametrize("tile", PIPELINED)
@pytest.mark.parametrize("a,d", COMBOS16, ids=[f"{a}->{d}" for a, d in COMBOS16])
@pytest.mark.parametrize("op_b", [0, 1])
def test_pipelined_tiles_ragged(tile, a, d, op_b):
    skip_unsupported(tile, a)
    # the direct-to-LDS kernel: ragged m and n (clamped copies), k = 200 for
    # 16-bit inputs (six full 32-deep steps plus a register-loaded tail of 8)
    # and 456 for fp8 (three full 128-deep steps plus a tail of 72), padded
    # leading dimensions with NaN padding, both bias axes
    k = 456 if a == "e4m3" else 200
    for ep, axis in (("relu_aux_bias", "row"), ("gelu_bias", "col")):
        w = wl(300, 520, k, a, d, ep, axis, op_b, seed=tile * 10 + op_b)
        r = run_library(w, synth.make_inputs(w), pad=2, path=1, tile=tile)
        assert f"tile_id={tile} kernel={ {9: 3, 10: 3, 11: 4, 12: 4, 13: 4, 14: 5, 16: 6}.get(tile, 2)}" in r.desc
        check_full(w, r)


@pytest.mark.parametrize("rot", [1, 3, 7])
@pytest.mark.parametrize("tile", [5, 6, 8, 9, 11, 13, 15, 16])
@pytest.mark.parametrize("a", ["bf16", "e4m3"])
def test_pipelined_k_rotation(tile, a, rot, monkeypatch):
    """The full K steps taken in a rotated order (GE_K_STAGGER overrides the
    planner's rotation): each tile starts rot * (its row in the group + its
    column) steps in and wraps round, the ragged step last.  Ragged m, n and
    k: 16-bit k = 488 (fifteen 32-deep steps and a tail of 8; 64-deep tiles
    seven and a tail of 40), fp8 k = 1000 (seven 128-deep steps and a tail of
    104; tile 16 fifteen 64-deep ones and 40), 3 x 4 to 10 x 13 tiles."""
    skip_unsupported(tile, a)
    monkeypatch.setenv("GE_K_STAGGER", str(rot))
    k = 1000 if a == "e4m3" else 488
    for op_b in (0, 1):
        w = wl(600, 776, k, a, "bf16", "relu_aux_bias", "row", op_b, seed=rot * 100 + tile)
        r = run_library(w, synth.make_inputs(w), pad=1, path=1, tile=tile)
        assert f"tile_id={tile} " in r.desc and r.desc.endswith(f" k_stagger={rot}"), r.desc
        check_full(w, r)


@pytest.mark.parametrize("tile", [6, 8, 15, 16])
@pytest.mark.parametrize("a", ["bf16", "e4m3"])
def test_pipelined_k_rotation_integer_bit_exact(tile, a, monkeypatch):
    """Integer inputs under a rotated K order: each K step must be taken
    exactly once (a step skipped or taken twice changes the exact sum)."""
    skip_unsupported(tile, a)
    monkeypatch.setenv("GE_K_STAGGER", "5")
    m, n, k = 520, 392, 1104
    w = wl(m, n, k, a, "bf16", "relu_bias", "col", 1)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4), bias_dist=("int", -64, 64))
    if a == "e4m3":
        g = torch.Generator().manual_seed(9)
        inp.A = torch.randint(-4, 5, (m, k), generator=g).float().to(torch.float8_e4m3fn)
        inp.B = torch.randint(-4, 5, (n, k), generator=g).float().to(torch.float8_e4m3fn)
        inp.scale_a = torch.ones(1)
        inp.scale_b = torch.ones(1)
    r = run_library(w, inp, path=1, tile=tile)
    assert r.desc.endswith(" k_stagger=5"), r.desc
    from parity import oracle_full
    Y, P, _ = oracle_full(w, r)
    assert np.array_equal(codes(r.D)[:, :n], oracle.encode(Y, "bf16").reshape(Y.shape))


@pytest.mark.parametrize("k", [1, 8, 31, 32, 33, 64, 95, 96, 97, 128, 129, 256, 385, 512])
@pytest.mark.parametrize("tile", [5, 6, 8, 9, 11, 13, 14, 15, 16])
@pytest.mark.parametrize("a", ["bf16", "e4m3"])
def test_pipelined_short_and_ragged_k(k, tile, a):
    skip_unsupported(tile, a)
    # fewer K steps than pipeline stages, exact multiples and one-element tails
    for op_b in (0, 1):
        w = wl(130, 136, k, a, "bf16", "bias", "row", op_b, seed=k)
        r = run_library(w, synth.make_inputs(w), pad=1, path=1, tile=tile)
        check_full(w, r)


@pytest.mark.parametrize("tile", PIPELINED)
@pytest.mark.parametrize("op_b", [0, 1])
@pytest.mark.parametrize("a", ["bf16", "e4m3"])
def test_pipelined_integer_bit_exact(tile, op_b, a):
    """Integer inputs: every fp32 partial sum is exact, so the pipelined
    kernel must reproduce the RNE encoding of the exact result bit for bit
    (fp8: small integers are exact E4M3 codes, unit scales)."""
    skip_unsupported(tile, a)
    m, n, k = 512, 384, 1056
    w = wl(m, n, k, a, "bf16", "relu_bias", "col", op_b)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4), bias_dist=("int", -64, 64))
    if a == "e4m3":
        g = torch.Generator().manual_seed(5)
        inp.A = torch.randint(-4, 5, (m, k), generator=g).float().to(torch.float8_e4m3fn)
        inp.B = torch.randint(-4, 5, (n, k) if op_b else (k, n), generator=g).float().to(torch.float8_e4m3fn)
        inp.scale_a = torch.ones(1)
        inp.scale_b = torch.ones(1)
    r = run_library(w, inp, path=1, tile=tile)
    from parity import oracle_full
    Y, P, _ = oracle_full(w, r)
    assert np.array_equal(codes(r.D)[:, :n], oracle.encode(Y, "bf16").reshape(Y.shape))


@pytest.mark.parametrize("k", [1, 5, 37, 64, 65, 127])
@pytest.mark.parametrize("a", ["bf16", "f32", "e4m3"])
def test_ragged_k_with_poisoned_padding(k, a):
    d = "bf16" if a == "e4m3" else a
    for op_b in (0, 1):
        w = wl(70, 90, k, a, d, "gelu_bias", "col", op_b, seed=k)
        r = run_library(w, synth.make_inputs(w), pad=1, path=1)
        check_full(w, r)


def test_zero_k_gives_activated_bias():
    w = wl(40, 72, 0, "bf16", "f32", "gelu_bias", "col")
    inp = synth.make_inputs(w)
    r = run_library(w, inp, path=1, lda=8, ldb=72)
    check_full(w, r)


def test_empty_output_is_noop():
    w = wl(0, 64, 32, "bf16", "bf16", "bias", "row")
    inp = synth.make_inputs(w)
    r = run_library(w, inp, path=1)
    assert r.D.numel() == 0


@pytest.mark.parametrize("m", [1, 3, 16])
@pytest.mark.parametrize("n,k", [(48, 40), (1000, 1000), (272, 4096)])
@pytest.mark.parametrize("a,d", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("split", [0, 3])
def test_smallm_path(m, n, k, a, d, split):
    for ep in ("gelu_bias", "relu_aux_bias", "tanh_bias"):
        for axis in ("col", "row"):
            w = wl(m, n, k, a, d, ep, axis, op_b=1, seed=m * 1000 + n)
            r = run_library(w, synth.make_inputs(w), pad=1, path=2, split_k=split)
            assert "path=smallm" in r.desc
            check_full(w, r)


@pytest.mark.parametrize("m", [1, 5, 16])
@pytest.mark.parametrize("n,k", [(48, 1000), (1000, 4096), (272, 8200)])
@pytest.mark.parametrize("rg", [2, 4])
@pytest.mark.parametrize("split", [0, 3])
def test_smallm_row_groups(m, n, k, rg, split):
    """Two or four 16-row groups of W per wave sharing each x fragment: a
    workgroup covers 32 or 64 columns, groups past n are clamped (their
    outputs and mask bits never stored), with and without a K split."""
    for ep, axis in (("gelu_bias", "col"), ("relu_aux_bias", "row"), ("bias", "col")):
        w = wl(m, n, k, "bf16", "bf16", ep, axis, op_b=1, seed=m + n + rg)
        r = run_library(w, synth.make_inputs(w), pad=1, path=2, split_k=split, group_m=rg)
        assert "path=smallm" in r.desc and f"group_m={rg} " in r.desc, r.desc
        check_full(w, r)


@pytest.mark.parametrize("m,n", [(5, 8200), (16, 8192)])
def test_smallm_auto_row_groups(m, n):
    """The planner's own choice of two row groups per wave once 32-column
    blocks fill the chip (n >= 8161), ragged and whole."""
    for ep, axis in (("gelu_bias", "col"), ("relu_aux_bias", "row")):
        w = wl(m, n, 512, "f16", "f16", ep, axis, op_b=1, seed=n)
        r = run_library(w, synth.make_inputs(w), pad=1)
        assert "path=smallm" in r.desc and "group_m=2 " in r.desc, r.desc
        check_full(w, r)


@pytest.mark.parametrize("rg,split", [(2, 2), (4, 4), (4, 1)])
def test_smallm_row_groups_integer_bit_exact(rg, split):
    """Integer inputs: every partial and slice sum is exact, so each row
    group's outputs must equal the oracle's RNE encoding bit for bit."""
    m, n, k = 16, 520, 8200
    w = wl(m, n, k, "f16", "f16", "relu_aux_bias", "col", 1)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4), bias_dist=("int", -64, 64))
    r = run_library(w, inp, path=2, split_k=split, group_m=rg)
    assert f"split_k={split} " in r.desc and f"group_m={rg} " in r.desc, r.desc
    from parity import oracle_full
    Y, P, _ = oracle_full(w, r)
    assert np.array_equal(codes(r.D)[:, :n], oracle.encode(Y, "f16").reshape(Y.shape))
    check_full(w, r)


@pytest.mark.parametrize("m,n,k,split", [(16, 130, 8200, 8), (4, 128, 65560, 32), (1, 1000, 4096, 4)])
def test_smallm_auto_split_ragged(m, n, k, split):
    """The planner's own K split (few column blocks, long K, a ragged last
    slice and a ragged last step) against the oracle."""
    for ep, axis in (("gelu_bias", "col"), ("relu_aux_bias", "row")):
        w = wl(m, n, k, "bf16", "bf16", ep, axis, op_b=1, seed=n + k)
        r = run_library(w, synth.make_inputs(w), pad=1)
        assert "path=smallm" in r.desc and f"split_k={split} " in r.desc, r.desc
        check_full(w, r)


@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f32")])
def test_smallm_split_integer_bit_exact(a, d):
    """Integer inputs keep every partial and slice sum exact, so the split
    reduction must reproduce the RNE encoding of the exact result."""
    m, n, k = 16, 520, 8200
    w = wl(m, n, k, a, d, "relu_bias", "col", 1)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4), bias_dist=("int", -64, 64))
    r = run_library(w, inp)
    assert "split_k=4 " in r.desc, r.desc
    from parity import oracle_full
    Y, _, _ = oracle_full(w, r)
    got = codes(r.D)[:, :n]
    want = Y.astype(np.float32) if d == "f32" else oracle.encode(Y, d).reshape(Y.shape)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("e4m3", "bf16")])
@pytest.mark.parametrize("ep", ["bias", "relu_aux_bias", "gelu_bias"])
def test_unfused_pair_matches_oracle_and_fused(a, d, ep):
    w = wl(260, 300, 96, a, d, ep, "row", 0, seed=5)
    inp = synth.make_inputs(w)
    ru = run_library(w, inp, pad=1, unfused=1)
    check_full(w, ru)
    rf = run_library(w, inp, pad=1)
    Du, Df = decode_output(w, ru), decode_output(w, rf)
    # the unfused pair rounds the product to D's dtype before the bias add,
    # so the two paths agree to about two output roundings
    assert rel_fro(Du, Df) <= 2 * tolerance(a, d)


def test_unfused_smallm():
    w = wl(16, 512, 1024, "f16", "f16", "gelu_bias", "col", 1)
    r = run_library(w, synth.make_inputs(w), path=2, unfused=1)
    check_full(w, r)


@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f16"), ("e4m3", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("tile", [1, 3])
def test_integer_inputs_bit_exact(a, d, tile):
    """Small integers make every fp32 partial sum exact, so D must equal the
    RNE encoding of the exact result bit for bit, whatever the order."""
    m, n, k = 512, 384, 1024
    w = wl(m, n, k, a, d, "relu_bias", "row", 0)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4), bias_dist=("int", -64, 64))
    if a == "e4m3":   # keep codes exact: unit scales
        inp.A = torch.clamp(torch.randint(-4, 5, (m, k), generator=torch.Generator().manual_seed(1)).float(),
                            -4, 4).to(torch.float8_e4m3fn)
        inp.B = torch.randint(-4, 5, (k, n), generator=torch.Generator().manual_seed(2)).float().to(
            torch.float8_e4m3fn)
        inp.scale_a = torch.ones(1)
        inp.scale_b = torch.ones(1)
    r = run_library(w, inp, path=1, tile=tile)
    from parity import oracle_full
    Y, P, _ = oracle_full(w, r)
    got = codes(r.D)[:, :n]
    if d == "f32":
        want = Y.astype(np.float32)
    else:
        want = oracle.encode(Y, d).reshape(Y.shape)
    assert np.array_equal(got, want)


def test_deterministic_bitwise():
    w = wl(700, 650, 520, "bf16", "bf16", "relu_aux_bias", "row", 0, seed=3)
    inp = synth.make_inputs(w)
    r1 = run_library(w, inp)
    r2 = run_library(w, inp)
    assert torch.equal(r1.D.view(torch.int16), r2.D.view(torch.int16))
    assert torch.equal(r1.aux, r2.aux)
    w2 = wl(16, 4096, 4096, "f16", "f16", "gelu_bias", "col", 1, seed=3)
    inp2 = synth.make_inputs(w2)
    r3 = run_library(w2, inp2, split_k=4, path=2)
    r4 = run_library(w2, inp2, split_k=4, path=2)
    assert torch.equal(r3.D.view(torch.int16), r4.D.view(torch.int16))


@pytest.mark.parametrize("split", [2, 3, 5])
@pytest.mark.parametrize("a,d", [("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")])
@pytest.mark.parametrize("op_b", [0, 1])
def test_split_k_tile_ragged(split, a, d, op_b):
    """Tile 14: K slices with a ragged last slice and a ragged last step,
    every epilogue kind the tile takes, padded leading dimensions."""
    for ep, axis, k in (("relu_aux_bias", "row", 1000), ("gelu_bias", "col", 1333), ("none", "row", 200)):
        w = wl(150, 200, k, a, d, ep, axis, op_b, seed=split * 7 + k)
        r = run_library(w, synth.make_inputs(w), pad=1, path=1, tile=14, split_k=split)
        # the planner cuts K into whole 64-element steps, which may leave fewer slices
        steps = -(-k // 64)
        eff = -(-k // (-(-steps // split) * 64))
        assert "tile_id=14 kernel=5" in r.desc and f"split_k={eff} " in r.desc, r.desc
        check_full(w, r)


@pytest.mark.parametrize("split", [2, 4])
def test_split_k_tile_integer_bit_exact_and_deterministic(split):
    """Integer inputs: the slice sums are exact, so D is bit-exact; two runs
    give the same bits (the slices are summed in a fixed order)."""
    m, n, k = 320, 256, 2048
    w = wl(m, n, k, "bf16", "bf16", "relu_bias", "col", 0)
    inp = synth.make_inputs(w, a_dist=("int", -4, 4), b_dist=("int", -4, 4), bias_dist=("int", -64, 64))
    r = run_library(w, inp, path=1, tile=14, split_k=split)
    from parity import oracle_full
    Y, _, _ = oracle_full(w, r)
    assert np.array_equal(codes(r.D)[:, :n], oracle.encode(Y, "bf16").reshape(Y.shape))
    w2 = wl(m, n, k, "bf16", "bf16", "gelu_bias", "row", 0, seed=3)
    inp2 = synth.make_inputs(w2)
    r1 = run_library(w2, inp2, path=1, tile=14, split_k=split)
    r2 = run_library(w2, inp2, path=1, tile=14, split_k=split)
    assert torch.equal(r1.D.view(torch.int16), r2.D.view(torch.int16))


def test_split_k_tile_unfused_and_repeated_calls():
    """Repeated calls (each clears its counters first) and the split-K tile as
    the unfused pair's first kernel."""
    w = wl(256, 192, 4096, "f16", "f16", "bias", "row", 0, seed=12)
    inp = synth.make_inputs(w)
    for _ in range(3):
        r = run_library(w, inp, path=1, tile=14, split_k=8)
        check_full(w, r)
    r = run_library(w, inp, path=1, tile=14, split_k=8, unfused=1)
    check_full(w, r)


@pytest.mark.parametrize("m,n,k,split", [(128, 128, 65536, 16), (1000, 500, 8200, 2), (500, 500, 8192, 4),
                                         (250, 260, 4100, 4)])
def test_split_k_tile_planner_choice(m, n, k, split):
    """The planner's own split-K plans, ragged where the shape allows: up to
    256 workgroups, 16 slices on 4 tiles, the last slice shorter than the
    others (k = 8200 in 2, 4100 in 4)."""
    w = wl(m, n, k, "bf16", "bf16", "relu_aux_bias", "row", 0, seed=m + k)
    r = run_library(w, synth.make_inputs(w), pad=1)
    assert "tile_id=14 " in r.desc and f" split_k={split} " in r.desc, r.desc
    check_full(w, r)


# ---- the mask's tie rule: P == 0 gives bit 0 ---------------------------------------
def int_inputs(w, lo=-2, hi=2, blo=-8, bhi=8, seed=31):
    """Small-integer operands and bias: every fp32 partial sum and the
    pre-activation are exact in any order, so P == 0 happens often and the
    mask must equal (P > 0) everywhere, ties included."""
    inp = synth.make_inputs(w, a_dist=("int", lo, hi), b_dist=("int", lo, hi), bias_dist=("int", blo, bhi))
    if w.in_dtype == "e4m3":
        g = torch.Generator().manual_seed(seed)
        inp.A = torch.randint(lo, hi + 1, (w.m, w.k), generator=g).float().to(torch.float8_e4m3fn)
        shape = (w.n, w.k) if w.op_b else (w.k, w.n)
        inp.B = torch.randint(lo, hi + 1, shape, generator=g).float().to(torch.float8_e4m3fn)
        inp.scale_a = torch.ones(1)
        inp.scale_b = torch.ones(1)
    return inp


def assert_mask_exact_with_ties(w, r):
    from parity import oracle_full
    Y, P, M = oracle_full(w, r)
    ties = int((P == 0.0).sum())
    assert ties > 50, f"only {ties} entries with P == 0: the case does not test the tie rule"
    got = codes(r.aux)
    assert np.array_equal(got, M), (
        f"{int((np.unpackbits(got.view(np.uint8)) != np.unpackbits(M.view(np.uint8))).sum())} mask bits "
        f"differ from (P > 0) ({ties} ties): {r.desc}")
    assert np.array_equal(codes(r.D)[:, : w.n], oracle.encode(Y, "bf16").reshape(Y.shape)), r.desc


@pytest.mark.parametrize("tile,a", [(1, "bf16"), (11, "bf16"), (13, "bf16"), (15, "bf16"),
                                    (15, "e4m3"), (11, "e4m3"), (14, "bf16"), (6, "bf16"), (6, "e4m3"),
                                    (16, "e4m3")])
@pytest.mark.parametrize("op_b", [0, 1])
def test_relu_aux_tie_rule_tiles(tile, a, op_b):
    w = wl(300, 520, 200 if a == "bf16" else 456, a, "bf16", "relu_aux_bias", "row", op_b, seed=tile)
    r = run_library(w, int_inputs(w), path=1, tile=tile, split_k=3 if tile == 14 else 0)
    assert f"tile_id={tile} " in r.desc
    assert_mask_exact_with_ties(w, r)


@pytest.mark.parametrize("split", [0, 4])
def test_relu_aux_tie_rule_smallm(split):
    w = wl(16, 520, 1024, "bf16", "bf16", "relu_aux_bias", "col", 1)
    r = run_library(w, int_inputs(w, -1, 1), path=2, split_k=split)
    assert "path=smallm" in r.desc
    assert_mask_exact_with_ties(w, r)


def test_relu_aux_tie_rule_unfused():
    # the pair rounds the product to bf16 first: integers up to 256 in
    # magnitude stay exact (|C| <= 200 * 4 = 800 would not, so k is small)
    w = wl(300, 520, 16, "bf16", "bf16", "relu_aux_bias", "row", 0)
    r = run_library(w, int_inputs(w), unfused=1)
    assert "unfused=1" in r.desc
    assert_mask_exact_with_ties(w, r)
