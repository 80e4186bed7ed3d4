"""The parity checker itself, on the CPU: a result that differs from the fp64
oracle only by the single bf16 rounding of each output passes both bars, and a
single misplaced output element, which the per-group Frobenius bar cannot see
at these sizes, fails the per-element bound."""
import numpy as np
import pytest

import synth
from oracle import qalg_oracle as O
from qalg_check import (BF16_TOL, assert_elementwise, assert_groups, forward_elementwise, rel_frob_col_groups)


def _bf16_round(a: np.ndarray) -> np.ndarray:
    return synth.f64_from_bf16_bits(synth.bf16_bits_from_f32(a.astype(np.float32)))


@pytest.fixture(scope="module")
def case():
    M, K, N, q = 32768, 128, 256, 4   # a group of 32768 x 64 outputs, as tall as the workloads
    X = synth.normal_operand(61, (M, K), 1.0, "bf16")
    W = synth.normal_operand(62, (K, N), K ** -0.5, "bf16")
    tau = (np.arange(M) % q).astype(np.int32)
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    return X, W, tau, q, Yr


def test_rounded_oracle_passes_both_bars(case):
    X, W, tau, q, Yr = case
    got = _bf16_round(Yr)
    assert_groups(rel_frob_col_groups(got, Yr, q), BF16_TOL, "Y")
    assert forward_elementwise(got, Yr, X.f64, W.f64, tau, q, "bf16", "Y") <= 1.0


@pytest.mark.parametrize("plant", ["swap_rows", "dropped_piece", "one_ulp_x4"])
def test_localized_error_is_caught_elementwise(case, plant):
    X, W, tau, q, Yr = case
    got = _bf16_round(Yr)
    if plant == "swap_rows":        # one 8-column piece of row 5 written to row 9
        got[9, 40:48] = got[5, 40:48]
    elif plant == "dropped_piece":  # one 8-column piece never written
        got[100, 96:104] = 0.0
    else:                           # one element off by 4 bf16 ulps
        got[7, 3] = got[7, 3] * (1 + 4 * 2.0 ** -7)
    # the per-group norm does not notice ...
    assert_groups(rel_frob_col_groups(got, Yr, q), BF16_TOL, "Y")
    # ... the per-element bound does
    with pytest.raises(AssertionError, match="per-element bound"):
        forward_elementwise(got, Yr, X.f64, W.f64, tau, q, "bf16", "Y")


def test_zero_reference_demands_exact_zero():
    ref = np.zeros((4, 4))
    got = ref.copy()
    assert assert_elementwise(got, ref, np.zeros_like(ref), 16, "bf16", "z") == 0.0
    got[1, 2] = 1e-30
    with pytest.raises(AssertionError):
        assert_elementwise(got, ref, np.zeros_like(ref), 16, "bf16", "z")
