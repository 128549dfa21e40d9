"""The recentred sketch of the oracle (sketch_direct_centered) pinned outside
itself (CPU only).

  C1  centre 0 is the plain sketch
  C2  every key at the centre: closed forms n e^{<q,c>} and mean(v) for any p
  C3  brute force with np.kron powers of k - c
  C4  Lagrange bound with the shifted radius; convergence to the exact answers
  C5  moment route on k - c times e^{<q,c>}
"""

import oracle
from tests import oracle_pins as pins

TIGHT = 1e-12


def test_c1_zero_centre():
    assert pins.pin_centered_zero_centre(oracle) < TIGHT


def test_c2_identical_keys():
    assert pins.pin_centered_identical_keys(oracle) < TIGHT


def test_c3_kron():
    assert pins.pin_centered_kron(oracle) < TIGHT


def test_c4_bound_and_convergence():
    ratio, err14 = pins.pin_centered_bound(oracle)
    assert ratio <= 1.0
    assert err14 < 1e-12


def test_c5_moments():
    assert pins.pin_centered_moments(oracle) < 1e-12
