"""GPU parity of block-scaled fp8 (MX: OCP E4M3 elements, one E8M0 scale per
32 K values of each row of A and each column of B) through
gemm_epilog_execute_mx, against the oracle's block-scaled product (O1x):
ragged shapes (a last K step holding 1 to 3 whole blocks and a partial one,
whose scale padding must be ignored), every output dtype, both B layouts,
the inference epilogues; unit scales against the per-tensor fp8 path;
integer codes with power-of-two scales bit-exact; a batch; and the H200
shape sampled in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_epilogue_02_amd import binding as B
from parity import check_full, check_sampled, codes, decode_output, rel_fro, run_library, oracle_full

pytestmark = pytest.mark.gpu


def wl(m, n, k, d, ep, axis="row", op_b=0, seed=7, a="mxf8"):
    return synth.Workload("t", "mx test", m, n, k, a, d, ep, axis, op_b, seed,
                          ("normal", 1.0), ("normal", 1.0), ("normal", 1.0))


@pytest.mark.parametrize("d", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("op_b", [0, 1])
@pytest.mark.parametrize("ep,axis", [("relu_aux_bias", "row"), ("relu_bias", "row"), ("gelu_bias", "col"),
                                     ("none", "row"), ("bias", "col")])
def test_mx_ragged(d, op_b, ep, axis):
    # 300 x 520: three 128-row tiles, five 128-column tiles, ragged; k = 456:
    # three full 128-deep steps and a tail of 72 (blocks 12, 13 whole, 14
    # partial; the row's 16th scale byte is padding)
    w = wl(300, 520, 456, d, ep, axis, op_b, seed=op_b * 10 + len(ep))
    inp = synth.make_inputs(w)
    # poison the scale padding: the kernel must not read it
    inp.mx_a[:, (w.k + 31) // 32:] = 0xFF
    inp.mx_b[:, (w.k + 31) // 32:] = 0xFF
    r = run_library(w, inp, pad=2)
    assert "tile_id=8 " in r.desc, r.desc
    check_full(w, r)


@pytest.mark.parametrize("k", [1, 31, 32, 33, 64, 127, 128, 129, 200, 1024])
@pytest.mark.parametrize("op_b", [0, 1])
def test_mx_short_and_ragged_k(k, op_b):
    w = wl(130, 136, k, "bf16", "bias", "row", op_b, seed=k)
    inp = synth.make_inputs(w)
    inp.mx_a[:, (k + 31) // 32:] = 0xFF
    inp.mx_b[:, (k + 31) // 32:] = 0xFF
    check_full(w, run_library(w, inp, pad=1))


@pytest.mark.parametrize("rot", [0, 1, 2, 5])
@pytest.mark.parametrize("op_b", [0, 1])
def test_mx_k_rotation(rot, op_b, monkeypatch):
    """The block-scaled tile with its K steps in a rotated order: each step's
    scale words must follow its data (k = 1000: seven 128-deep steps and a
    tail of 104 values, 4 x 5 tiles of 128)."""
    monkeypatch.setenv("GE_K_STAGGER", str(rot))
    w = wl(500, 520, 1000, "bf16", "gelu_bias", "col", op_b, seed=40 + rot)
    r = run_library(w, synth.make_inputs(w), pad=1)
    assert r.desc.endswith(f" k_stagger={rot}"), r.desc
    check_full(w, r)


def test_mx_unit_scales_match_the_per_tensor_path():
    """All block scales 2^0: the block-scaled kernel must compute what the
    per-tensor fp8 kernel computes on the same codes (same tile)."""
    w = wl(260, 264, 520, "f32", "bias", "row", 0, seed=3)
    inp = synth.make_inputs(w)
    inp.mx_a.fill_(127)
    inp.mx_b.fill_(127)
    r_mx = run_library(w, inp)
    w8 = wl(260, 264, 520, "f32", "bias", "row", 0, seed=3, a="e4m3")
    inp8 = synth.Inputs(inp.A, inp.B, inp.bias, None, None)
    r8 = run_library(w8, inp8, tile=8)
    assert rel_fro(decode_output(w, r_mx), decode_output(w8, r8)) <= 1e-6
    check_full(w, r_mx)


@pytest.mark.parametrize("op_b", [0, 1])
def test_mx_integer_codes_power_of_two_scales_bit_exact(op_b):
    """Integer codes |x| <= 4 and scales 2^0 .. 2^3 keep every product an
    integer and every sum below 2^24: the result is exact in any order, so D
    must be the RNE encoding of the oracle's value bit for bit."""
    m, n, k = 384, 264, 1056
    w = wl(m, n, k, "bf16", "relu_bias", "col", op_b, seed=9)
    inp = synth.make_inputs(w, bias_dist=("int", -64, 64))
    g = torch.Generator().manual_seed(19)
    inp.A = torch.randint(-4, 5, (m, k), generator=g).float().to(torch.float8_e4m3fn)
    inp.B = torch.randint(-4, 5, (n, k) if op_b else (k, n), generator=g).float().to(torch.float8_e4m3fn)
    kb = (k + 31) // 32
    inp.mx_a[:, :kb] = torch.randint(127, 131, (m, kb), generator=g).to(torch.uint8)
    inp.mx_b[:, :kb] = torch.randint(127, 131, (n, kb), generator=g).to(torch.uint8)
    r = run_library(w, inp)
    Y, _, _ = oracle_full(w, r)
    assert np.array_equal(codes(r.D)[:, :n], oracle.encode(Y, "bf16").reshape(Y.shape))


def test_mx_batched():
    """Two products in one launch: product z reads its block scales at
    z*m*ld and z*n*ld."""
    m, n, k, nb = 150, 144, 256, 2   # 16-byte rows: fp8 k, bf16 n and the column bias of each product
    w = wl(m, n, k, "bf16", "gelu_bias", "col", 0, seed=5)
    inps = [synth.make_inputs(w, seed=w.seed + 31 * z) for z in range(nb)]
    dev = "cuda"
    ld = B.mx_scale_ld(k)
    A = torch.stack([i.A for i in inps]).to(dev).contiguous()
    Bm = torch.stack([i.B for i in inps]).to(dev).contiguous()
    SA = torch.stack([i.mx_a for i in inps]).to(dev).contiguous()
    SB = torch.stack([i.mx_b for i in inps]).to(dev).contiguous()
    bias = torch.stack([i.bias.reshape(-1) for i in inps]).to(dev).contiguous()
    D = torch.full((nb, m, n), float("nan"), dtype=torch.bfloat16, device=dev)
    g = B.GemmEpilog(m, n, k, "mxf8", "bf16", 0, k, n, n, batch=nb)
    try:
        g.plan("gelu_bias", "col")
        B.gemm_epilog_execute_mx(g.h, A, Bm, SA, SB, bias, D)
        torch.cuda.synchronize()
    finally:
        g.free()
    for z in range(nb):
        Cz = oracle.gemm_mx(codes(A[z]), "e4m3", codes(SA[z]), codes(Bm[z]), "e4m3", codes(SB[z]), 0)
        Yz = oracle.act_pass(oracle.bias_pass(Cz, codes(bias[z]), "bf16", "col"), "gelu_bias")
        Dz = oracle.decode(codes(D[z]), "bf16")
        assert rel_fro(Dz, Yz) <= 5e-3, z
    assert SA.shape[-1] == ld


def test_mx_h200_shape_sampled():
    """The block-scaled benchmark workload at full size, in the planner's
    launch configuration: 4096 seeded entries and 16 full rows."""
    w = synth.WORKLOADS["F2a"]
    inp = synth.make_inputs(w, device="cuda")
    r = run_library(w, inp, poison=False)
    del inp
    errs = check_sampled(w, r, w.seed)
    print("F2a", r.desc, "rel_fro entries/rows:", errs[:2])
    del r
    torch.cuda.empty_cache()
