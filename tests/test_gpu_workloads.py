"""The pages' workloads at full size, in the launch configuration the
benchmark times (the planner's automatic choice).  Small ones are compared
whole; the large ones on 4096 seeded entries plus 16 full rows."""
import pytest
import torch

import synth
from parity import check_full, check_sampled, run_library

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", ["C1", "C2", "C3"])
def test_workload_whole(key):
    w = synth.WORKLOADS[key]
    inp = synth.make_inputs(w)
    r = run_library(w, inp, poison=False)
    err = check_full(w, r)
    print(key, r.desc, f"rel_fro={err:.3e}")


@pytest.mark.parametrize("key", ["C4", "C5a", "C5b"])
def test_workload_sampled(key):
    w = synth.WORKLOADS[key]
    inp = synth.make_inputs(w, device="cuda")
    r = run_library(w, inp, poison=False)
    del inp
    errs = check_sampled(w, r, w.seed)
    print(key, r.desc, "rel_fro entries/rows, band mismatches:", errs)
    del r
    torch.cuda.empty_cache()


def test_c4_shape_integer_bit_exact():
    """Integer-valued inputs at the 8192^3 shape: every fp32 partial sum is
    exact, so sampled outputs must equal the RNE encoding of the exact value."""
    w = synth.scaled(synth.WORKLOADS["C4"], epilog="relu_bias")
    inp = synth.make_inputs(w, device="cuda", a_dist=("int", -3, 3), b_dist=("int", -3, 3),
                            bias_dist=("int", -100, 100))
    r = run_library(w, inp, poison=False)
    del inp
    check_sampled(w, r, 77, exact=True)
    del r
    torch.cuda.empty_cache()


def test_c4_shape_relu_aux_tie_rule_integer():
    """RELU_AUX_BIAS at the 8192^3 shape with integer inputs: P is exact, so
    every sampled mask bit must equal (P > 0), the P == 0 ties included."""
    w = synth.WORKLOADS["C4"]
    inp = synth.make_inputs(w, device="cuda", a_dist=("int", -1, 1), b_dist=("int", -1, 1),
                            bias_dist=("int", -40, 40))
    r = run_library(w, inp, poison=False)
    del inp
    check_sampled(w, r, 78, exact=True)
    del r
    torch.cuda.empty_cache()
