"""The two error measures the parity tests report (CPU): the per-output metric
(max over (n,h) slices of max |diff| / max |ref|) and its elementwise log
with a floor of 1e-3 max |ref| per slice."""
import numpy as np

from tests import parity as P


def test_max_rel_is_per_slice():
    ref = np.array([[1.0, -4.0], [100.0, 1.0]])
    got = ref + np.array([[0.4, 0.0], [0.0, 1.0]])
    # slice 0: 0.4 / 4 = 0.1; slice 1: 1 / 100 = 0.01
    assert np.isclose(P.max_rel(got, ref, 2), 0.1)


def test_elem_rel_floor():
    ref = np.array([[1.0, 1e-9, 0.0, -2.0]])
    got = ref + np.array([[1e-3, 1e-6, 2e-6, 0.0]])
    # floor = 1e-3 * 2 = 2e-3: ratios 1e-3 / 1, 1e-6 / 2e-3, 2e-6 / 2e-3, 0
    assert np.isclose(P.elem_rel(got, ref, 1), 1e-3)
    got2 = ref + np.array([[0.0, 0.0, 4e-3, 0.0]])
    assert np.isclose(P.elem_rel(got2, ref, 1), 2.0)
    assert P.elem_rel(np.zeros((2, 0)), np.zeros((2, 0)), 2) == 0.0
