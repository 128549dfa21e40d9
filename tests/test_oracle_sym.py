"""The multiset-storage oracle (oracle.sym) pinned outside itself (CPU only).

  S1  row counts C(d + j - 1, j), C(d + p, p); lexicographic sorted tuples; the
      multinomial theorem for alpha!
  S2  stored entries and answers against pure-Python sums over all index tuples
  S3  answers == the plain definition sum_i T_p(<q, k_i>) on the five workloads
  S4  entries spread to every index tuple == np.kron-built Kronecker moments
  S5  merge(A, B) == sketch(A u B)
"""

import pytest

import oracle
from synthetic import WORKLOADS, generate
from tests import oracle_pins as pins

TIGHT = 1e-12


@pytest.mark.parametrize("d,p", [(1, 4), (2, 5), (3, 4), (4, 3), (8, 6), (16, 4), (5, 0)])
def test_s1_counts(d, p):
    assert pins.pin_sym_counts(oracle, d, p) < TIGHT


@pytest.mark.parametrize("d,p", [(2, 0), (2, 3), (3, 2), (3, 4), (1, 3)])
def test_s2_bruteforce(d, p):
    assert pins.pin_sym_bruteforce(oracle, d, p) < TIGHT


@pytest.mark.parametrize("ident,n,m,chunk", [(1, 4096, 64, 512), (2, 384, 24, 128),
                                            (3, 384, 24, 128), (4, 384, 24, 128),
                                            (5, 200, 12, 64)])
def test_s3_equals_direct(ident, n, m, chunk):
    w = WORKLOADS[ident].scaled(n=n, m=m, h=1)
    K, V, Q = generate(w)
    assert pins.pin_sym_equals_direct(oracle, K[0], V[0], Q[0], w.p, chunk) < 1e-11


@pytest.mark.parametrize("d,p", [(2, 4), (3, 3), (4, 2), (5, 2)])
def test_s4_expand_equals_kron(d, p):
    assert pins.pin_sym_expand(oracle, d, p) < TIGHT


def test_s5_merge():
    assert pins.pin_sym_merge(oracle) < TIGHT
