"""The float64 oracle against facts other than itself (runs on the CPU)."""
import numpy as np
import pytest

import oracle_pins as P
from oracle import load_oracle
from cfc_recurrent_cell_amd.workloads import TINY, make_cfc_inputs


@pytest.fixture(scope="module")
def lib():
    return load_oracle()


@pytest.mark.parametrize("name", sorted(P.ALL_PINS))
def test_pin(lib, name):
    P.ALL_PINS[name](lib)


def test_finite_differences_tiny_workload(lib):
    """Every one of the 1600 parameters of the tiny workload (b = 0, h0 = 0)."""
    inp = make_cfc_inputs(TINY)
    err = P.pin_finite_differences(lib, inp, eps=1e-6, rtol=1e-6, atol=1e-8)
    assert err < 1e-7


def test_autograd_smoke_rows(lib):
    """Autograd on two rows of the smoke-shaped workload (K=64, H=128)."""
    from cfc_recurrent_cell_amd.workloads import SMOKE
    inp = make_cfc_inputs(SMOKE, B=2)
    P.pin_autograd(lib, inp)


def test_input_grad_finite_differences_tiny_workload(lib):
    """dL/dx (512 entries) and dL/dh0 (128) of the tiny workload.  The loss is
    about 67 here, so each central difference carries a rounding error of about
    2 * 67 * 2^-53 / (2 * 1e-6) = 7e-9; atol is four times that."""
    inp = make_cfc_inputs(TINY)
    P.pin_input_grad_finite_differences(lib, inp, eps=1e-6, rtol=1e-6, atol=3e-8)


def test_tau_decay_tiny_workload_finite_differences(lib):
    """Every parameter (416) and input (256 + 64) of the tau-decay tiny
    workload: the shape and dt of the pages' B=1 backward test."""
    from cfc_recurrent_cell_amd.workloads import TAU_TINY
    inp = make_cfc_inputs(TAU_TINY)
    P.pin_finite_differences(lib, inp, eps=1e-6, rtol=1e-6, atol=1e-8)
    P.pin_input_grad_finite_differences(lib, inp, eps=1e-6, rtol=1e-6, atol=1e-8)
