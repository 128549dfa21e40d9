"""The float64 oracle pinned to references outside itself (CPU only).

Pins (see tests/oracle_pins.py for the references each one uses):
  P1  brute force with explicit Kronecker powers (np.kron), incl. the state layout
  P2  moment route == direct route on small versions of the five workloads
  P3  stream of identical keys: closed forms n*T_p(q.k), n*e^(q.k), mean(v)
  P4  q = 0: Z = Zhat = n, o = ohat = mean(v)
  P5  p = 0 and p = 1 (linear attention) closed forms
  P6  merge(A, B) == sketch(A u B)
  P7  |Zhat_p - Z|/Z falls to rounding as p grows
  P8  the Lagrange truncation bound holds per query (and the ohat bound)
  P9  each level of the state is a symmetric tensor
  P10 M_{j+1} (as a d^j x d matrix) == Phi_j(K)^T K
  P11 values mapped by alpha*v + beta map outputs the same way
  P12 exact path == scipy softmax / logsumexp
  P13 sign of T_p: positive for even p; one real root for odd p (numpy.roots)
  P14 exact path == plain Python sums (math.fsum, math.exp)
  P15 empty stream
  golden: hand-worked examples in tests/golden/hand_worked.json
"""

import math

import numpy as np
import pytest

import oracle
from synthetic import WORKLOADS, generate
from tests import oracle_pins as pins

TIGHT = 1e-12


@pytest.mark.parametrize("d,p", [(2, 0), (2, 1), (2, 4), (3, 2), (3, 4), (1, 5)])
def test_p1_bruteforce(d, p):
    assert pins.pin_bruteforce(oracle, d, p) < TIGHT


@pytest.mark.parametrize("ident,n,m,chunk", [(1, 4096, 64, 512), (2, 384, 24, 128),
                                            (3, 384, 24, 128), (4, 384, 24, 128),
                                            (5, 96, 12, 16)])
def test_p2_moment_equals_direct(ident, n, m, chunk):
    w = WORKLOADS[ident].scaled(n=n, m=m, h=1)
    K, V, Q = generate(w)
    assert pins.pin_moment_equals_direct(oracle, K[0], V[0], Q[0], w.p, chunk) < 1e-11


@pytest.mark.parametrize("p", [0, 1, 2, 3, 5, 7])
def test_p3_identical_keys(p):
    assert pins.pin_identical_keys(oracle, p) < TIGHT


@pytest.mark.parametrize("p", [0, 1, 3, 6])
def test_p4_zero_query(p):
    assert pins.pin_zero_query(oracle, p) < TIGHT


def test_p5_low_orders():
    assert pins.pin_low_orders(oracle) < TIGHT


def test_p6_merge():
    assert pins.pin_merge(oracle) < TIGHT


def test_p7_convergence():
    e20, excess8, rises = pins.pin_convergence(oracle)
    assert e20 < 1e-14
    assert excess8 == 0.0
    assert rises == 0


@pytest.mark.parametrize("ident", [1, 2, 3, 4, 5])
def test_p8_truncation_bound(ident):
    w = WORKLOADS[ident].scaled(n=2048, m=48, h=1)
    K, V, Q = generate(w)
    K, V, Q = K[0], V[0], Q[0]
    rho = oracle.measured_radius(K, Q)
    od, Zd = oracle.sketch_direct(K, V, Q, w.p)
    oe, Ze = oracle.exact_attention(K, V, Q)
    zb = oracle.kde_relative_bound(w.p, rho)
    assert np.all(np.abs(Zd - Ze) / Ze <= zb)
    ob = oracle.attention_abs_bound(w.p, rho, V)
    assert np.all(np.abs(od - oe) <= ob[None, :])
    # the bound is not vacuous where the regime is high-temperature
    if ident in (1, 2, 4):
        assert zb < 0.5


@pytest.mark.parametrize("d,p", [(3, 3), (4, 2), (2, 5)])
def test_p9_level_symmetry(d, p):
    rng = np.random.default_rng(9)
    K = rng.standard_normal((25, d))
    V = rng.standard_normal((25, 2))
    sk = oracle.MomentSketch(d, 2, p).update(K, V)
    for j in range(2, p + 1):
        Mj = sk.M[j].reshape((d,) * j)
        Nj = sk.N[j].reshape((d,) * j + (2,))
        for perm in [tuple(reversed(range(j))), tuple([1, 0] + list(range(2, j)))]:
            assert np.abs(Mj - Mj.transpose(perm)).max() < 1e-12
            assert np.abs(Nj - Nj.transpose(perm + (j,))).max() < 1e-12


@pytest.mark.parametrize("d,p", [(3, 3), (4, 2), (5, 3)])
def test_p10_kfold_identity(d, p):
    rng = np.random.default_rng(10)
    K = rng.standard_normal((31, d))
    V = rng.standard_normal((31, 3))
    sk = oracle.MomentSketch(d, 3, p).update(K, V)
    for j in range(p):
        Phi_j = np.stack([pins.kron_power(k, j) for k in K])
        assert np.abs(sk.M[j + 1].reshape(d ** j, d) - Phi_j.T @ K).max() < 1e-12


def test_p11_affine_values():
    assert pins.pin_affine_values(oracle) < TIGHT


def test_p12_textbook_attention():
    assert pins.pin_textbook_attention(oracle) < TIGHT


@pytest.mark.parametrize("p", list(range(0, 10)))
def test_p13_taylor_sign(p):
    xs = np.linspace(-12.0, 4.0, 4001)
    t = oracle.taylor_exp(xs, p)
    coef = pins.taylor_coeffs(p)
    roots = np.roots(list(reversed(coef))) if p > 0 else np.array([])
    real = np.sort(roots[np.abs(roots.imag) < 1e-9].real)
    if p % 2 == 0:
        assert np.all(t > 0)
        assert len(real) == 0
    else:
        assert len(real) == 1
        r = real[0]
        assert abs(oracle.taylor_exp(np.array([r]), p)[0]) < 1e-10
        assert np.all(t[xs < r - 1e-6] < 0) and np.all(t[xs > r + 1e-6] > 0)
    if p == 1:
        assert abs(real[0] + 1.0) < 1e-12


def test_taylor_incomplete_gamma():
    assert pins.pin_taylor_gamma(oracle) < 1e-13


def test_p14_exact_python():
    assert pins.pin_exact_python(oracle) < TIGHT


def test_p15_empty_stream():
    K = np.zeros((0, 3))
    V = np.zeros((0, 2))
    Q = np.ones((2, 3))
    oe, Ze = oracle.exact_attention(K, V, Q)
    od, Zd = oracle.sketch_direct(K, V, Q, 3)
    om, Zm = oracle.MomentSketch(3, 2, 3).query(Q)
    for o, z in ((oe, Ze), (od, Zd), (om, Zm)):
        assert np.all(z == 0.0)
        assert np.all(np.isnan(o))


def test_hand_worked_golden():
    assert pins.pin_hand_worked(oracle) < TIGHT


def test_truncation_bound_values():
    """The bound function against its closed form at a few radii (hand values)."""
    # p = 2, rho = 0.5625: eps1 = 0.5625^3/6 * e^0.5625
    eps1 = 0.5625 ** 3 / 6.0 * math.exp(0.5625)
    assert abs(oracle.taylor_term_bound(2, 0.5625) - eps1) < 1e-15
    assert abs(oracle.kde_relative_bound(2, 0.5625) - eps1 * math.exp(0.5625)) < 1e-15
    # a bound must dominate the true remainder on a grid
    for p in range(0, 8):
        for rho in (0.25, 1.0, 2.5):
            xs = np.linspace(-rho, rho, 201)
            rem = np.abs(np.exp(xs) - oracle.taylor_exp(xs, p)).max()
            assert rem <= oracle.taylor_term_bound(p, rho) * (1 + 1e-12)


def test_bound_closed_form_values():
    assert pins.pin_bound_table(oracle) == 0.0


def test_term_bound_is_lagrange_tight():
    assert pins.pin_term_bound_tight(oracle) == 0.0


def test_measured_radius_hand_example():
    assert pins.pin_measured_radius(oracle) < 1e-15


def test_attention_bound_near_tight():
    assert pins.pin_attention_bound_near_tight(oracle) == 0.0
